// The forward kernel (O and LSE).
#include "bsa_device.h"

namespace bsa {
namespace {

// ---------------------------------------------------------------------------
// forward: O and LSE, Q-block outer
// ---------------------------------------------------------------------------
// The forward the backward differentiates (aclnnBlockSparseAttentionGrad page,
// 功能说明 / 计算公式: S = Mask(scale * Q K^T), P = Softmax(S), Out = P V),
// evaluated over the selected blocks only with a running maximum and sum per
// query row (the FlashSoftmax rescaling of the FlashAttentionScore page,
// 实现原理).  One workgroup per (batch, query head, Q block, 128-row part),
// 32 query rows per wave held in registers as MFMA B operands; K/V slices of
// the selected KV blocks stream through the same double-buffered LDS tiles as
// the dQ kernel.  S^T = K Q^T leaves each lane one query row's scores, so the
// running maximum needs one exchange with the partner lane (+-32), and the
// output is accumulated transposed, O^T += V^T P^T, so that each lane also
// holds its own row of O and rescales it in place.  Rows that select nothing
// (and BNSD padding rows) get O = 0 and LSE = -inf.
constexpr float kLazyRescale = 8.f;  // forward: how far (log2 units) a row maximum may pass its reference

template <class E>
__device__ __forceinline__ u16x4 pack4(const float* x) {
  u16x4 r;
#pragma unroll
  for (int t = 0; t < 4; ++t) r[t] = E::from_f32(x[t]);
  return r;
}

template <class E, int D, int W, bool AM>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(D >= 256 ? 1 : 2))) void fwd_kernel(Params p) {
  constexpr int KS = D / 16;
  constexpr int NT = D / 32;
  constexpr int NB = ring_buffers(W);
  using Ring = KVRing<D, W, NB>;
  __shared__ __align__(1024) unsigned short sK[NB][32 * D], sV[NB][32 * D];
  __shared__ int sN[NB];  // valid rows of the slice in each buffer (0 = past the end)
  __shared__ int sR[NB];  // its first key row (sequence-local)
  __shared__ int sList[kListChunk];
  // per buffer and wave: attenMask words of the slice's keys for the wave's 32
  // queries ([0, 32): word row0 / 32, [32, 64): the next word; zeros without a mask)
  __shared__ __align__(16) uint32_t sAB[NB][AM ? W : 1][64];
  constexpr int kWait = Ring::WAIT + (AM ? NB - 2 : 0);  // the ring's copies (+ one mask-word copy per stage)

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, l32 = lane & 31, g = lane >> 5;

  int wid = blockIdx.x;
  const int nsub = (p.bx + kTileRows - 1) / kTileRows;
  const int sub = wid % nsub;
  wid /= nsub;
  const int ib = wid % p.nqb;
  wid /= p.nqb;
  const int n = wid % p.N;
  const int b = wid / p.N;
  const SeqInfo si = seq_of(p, b);
  const int q0 = ib * p.bx + sub * kTileRows;
  const int part_end = min(ib * p.bx + p.bx, q0 + kTileRows);
  const int q_end = min(part_end, si.len_q);
  const int w_end = min(part_end, si.wlim_q);
  if (q0 >= w_end) return;

  const int h = n / p.G;
  const int64_t bn = static_cast<int64_t>(b) * p.N + n;
  const int my_q = q0 + 32 * w + l32;
  const bool q_ok = my_q < q_end;
  const unsigned short* qp = static_cast<const unsigned short*>(p.q) + b * p.q_sb + si.off_q * p.q_sr + n * p.q_sh;
  u16x8 qreg[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    u16x8 zq = {0, 0, 0, 0, 0, 0, 0, 0};
    if (q_ok) zq = *reinterpret_cast<const u16x8*>(qp + my_q * p.q_sr + 16 * s + 8 * g);
    qreg[s] = zq;
  }
#pragma unroll
  for (int s = 0; s < KS; ++s) settle(qreg[s]);

  f32x16 aot[NT];  // O^T[d][q]: this lane's column is query row my_q
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) aot[nt] = f32x16{};
  float m_run = -__builtin_inff(), l_run = 0.f;

  const int64_t kv_base = b * p.kv_sb + si.off_kv * p.kv_sr + h * p.kv_sh;
  const unsigned short* kp = static_cast<const unsigned short*>(p.k) + kv_base;
  const unsigned short* vp = static_cast<const unsigned short*>(p.v) + kv_base;
  const float c2 = p.scale_log2e;

  const Ring ring(p.kv_sr, w, lane);
  LdsListWalk walk{-1, p.row_cnt[bn * p.nqb + ib], 0, 0, 0, p.row_list + (bn * p.nqb + ib) * p.nkb, sList};
  walk.fill(0, tid, 64 * W);
  auto issue = [&](int slot) {
    Slice sl;
    if (!walk.next(p, si.len_kv, sl, tid, 64 * W)) sl = Slice{0, 0, 0};
    ring.issue(sK[slot], sV[slot], sl, kp, vp, p.kv_sr, p.consts);
    if constexpr (AM) {  // one copy per wave and stage, so the waits stay constants
      const int wi = (sl.row0 >> 5) + g;
      const bool ok = sl.nrows > 0 && my_q < p.sq_max && wi < p.am_wk;
      dma4(ok ? static_cast<const void*>(p.am_rows + static_cast<int64_t>(my_q) * p.am_wk + wi) : p.consts,
           lds_addr(&sAB[slot][w][0]));
    }
    if (tid == 0) {
      sN[slot] = sl.nrows;
      sR[slot] = sl.row0;
    }
  };

  auto compute = [&](const unsigned short* tk, const unsigned short* tv, int nrows, int row0, int slot) {
    f32x16 st = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      st = E::mma(frag_along_row<D>(tk, 0, 16 * ks, lane), qreg[ks], st);  // S^T[kv][q]
    float x[16];
    float mx = -__builtin_inff();
    if (nrows == 32 && !AM && rect_in_band(p, q0 + 32 * w, 32, row0, 32)) {  // uniform: no mask needed
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        x[i] = st[i] * c2;  // scaled score in log2 units
        mx = fmaxf(mx, x[i]);
      }
    } else {
      const uint32_t ex = AM ? mask_word(sAB[slot][AM ? w : 0], row0, l32) : 0u;
      const uint32_t keep = ((nrows >= 32 ? 0xffffffffu : ((1u << nrows) - 1u)) & ~ex & band_keys(p, my_q, row0)) >> (4 * g);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        x[i] = ((keep >> (8 * (i >> 2) + (i & 3))) & 1u) ? st[i] * c2 : -__builtin_inff();
        mx = fmaxf(mx, x[i]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));  // the partner lane holds the row's other 16 keys
    // Lazy rescale: the reference maximum m_run moves only once the row's
    // maximum exceeds it by more than kLazyRescale (log2 units).  P is then
    // at most 2^kLazyRescale, harmless in the fp32 sums and as a 16-bit MFMA
    // operand, and O = acc / l and LSE = m_run + log2(l) hold for any
    // reference, so the result is the same; most slices skip the O rescale.
    const bool grow = mx > m_run + kLazyRescale;  // always once m_run is -inf and a key is valid
    const float m_new = grow ? mx : m_run;
    const float m_use = m_new == -__builtin_inff() ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);  // exactly 1 where the reference stays
    float pv[16], ls = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      pv[i] = fast_exp2(x[i] - m_use);
      ls += pv[i];
    }
    l_run = l_run * alpha + ls;
    if (__any(grow)) {  // wave-uniform test
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) aot[nt] *= alpha;
    }
    m_run = m_new;
    const u16x8 pa[2] = {pack8<E>(pv), pack8<E>(pv + 8)};
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        aot[nt] = E::mma(frag_down_rows<D>(tv, 16 * hh, 32 * nt, lane), pa[hh], aot[nt]);  // O^T += V^T P^T
    }
  };

  // the dQ kernel's stage loop: NB - 1 slices in flight ahead of the compute
#pragma unroll
  for (int t = 0; t < NB - 1; ++t) issue(t);
  wait_vmcnt<kWait>();
  __syncthreads();
  int nrows = sN[0];
  for (int t = 0; nrows > 0;) {
    const int cur = t % NB;
    issue((t + NB - 1) % NB);
    compute(sK[cur], sV[cur], nrows, sR[cur], cur);
    ++t;
    wait_vmcnt<kWait>();
    __syncthreads();
    nrows = sN[t % NB];
  }
  wait_vmcnt<0>();

  float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!q_ok) l_tot = 0.f;  // padding rows: nothing selected by definition
  const float inv = (l_tot > 0.f ? 1.f / l_tot : 0.f) * p.o_scale;
  if (my_q < w_end) {
    unsigned short* op = static_cast<unsigned short*>(p.out_o) + b * p.o_sb + si.off_q * p.o_sr + n * p.o_sh +
                         static_cast<int64_t>(my_q) * p.o_sr;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        float v4[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) v4[c] = aot[nt][4 * a + c] * inv;
        *reinterpret_cast<u16x4*>(op + 32 * nt + 8 * a + 4 * g) = pack4<E>(v4);
      }
    }
    if (g == 0)
      p.out_lse[b * p.lse_sb + (si.off_q + my_q) * p.lse_sr + n * p.lse_sh] =
          l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * 0.6931471805599453f : -__builtin_inff();
  }
}

}  // namespace

int launch_fwd(const Params& p, void* stream) {
  const dim3 grid(static_cast<unsigned>(p.n_dq_units));
  BSA_DISPATCH(fwd_kernel, waves_for(p.bx), grid, static_cast<hipStream_t>(stream), p);
  return static_cast<int>(hipGetLastError());
}

}  // namespace bsa
