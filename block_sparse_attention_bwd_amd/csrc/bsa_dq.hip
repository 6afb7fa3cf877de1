// The dQ kernel (Q-block outer; it also computes softmax_grad) and the store of
// the atomic mode's dQ accumulator.
#include "bsa_device.h"

namespace bsa {
namespace {


// ---------------------------------------------------------------------------
// dQ: Q-block-outer
// ---------------------------------------------------------------------------
// One workgroup per (batch, query head, Q block, 128-row part); it walks the
// slices of the KV blocks its Q block selects, in list (ascending) order.
template <class E, int D, int W, bool AM>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(D >= 256 ? 1 : 2))) void dq_kernel(Params p) {
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

  int wid = PlanView(p).dq_order[blockIdx.x];
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
  const int64_t bn = static_cast<int64_t>(b) * p.N + n;
  const int my_q = q0 + 32 * w + l32;  // B-operand column == score column of this lane
  // this lane writes row my_q of the softmax_grad / lse2 arrays (zeros past
  // the sequence's length, as for every position below maxSq)
  const bool row_out = g == 0 && my_q < min(part_end, p.sq_max);
  if (q0 >= w_end) {  // no row of the sequence here (a TND block past its end)
    if (row_out) {
      p.delta[bn * p.sq_max + my_q] = 0.f;
      p.lse2[bn * p.sq_max + my_q] = 0.f;
    }
    return;
  }

  const int h = n / p.G;
  const bool q_ok = my_q < q_end;
  const int64_t q_base = b * p.q_sb + si.off_q * p.q_sr + n * p.q_sh;
  const unsigned short* qp = static_cast<const unsigned short*>(p.q) + q_base;
  const unsigned short* dop = static_cast<const unsigned short*>(p.dout) + q_base;

  // Invalid query lanes hold zero Q/dO rows and LSE = softmax_grad = 0, so
  // their dP is 0 and so is every dS they produce.
  u16x8 qreg[KS], oreg[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    u16x8 zq = {0, 0, 0, 0, 0, 0, 0, 0};
    u16x8 zo = zq;
    if (q_ok) {
      zq = *reinterpret_cast<const u16x8*>(qp + my_q * p.q_sr + 16 * s + 8 * g);
      zo = *reinterpret_cast<const u16x8*>(dop + my_q * p.q_sr + 16 * s + 8 * g);
    }
    qreg[s] = zq;
    oreg[s] = zo;
  }
  // softmax_grad (aclnnBlockSparseAttentionGrad page, 功能说明: softmaxGrad of
  // dOut and attentionOut, the row sums of dOut o Out).  This lane holds the
  // row's 8-element chunks 2s + g of dOut (s < KS); it sums each chunk in
  // order, folds the KS chunk sums in halves (chunk 2s with 2s + KS, then
  // with 2s + KS / 2, ...), and adds the partner lane's (+-32) result: the
  // order of the prologue's pass (chunk sums combined by lane shuffles at
  // distances D/16, D/32, ..., 1), so both give the same bits.  Written
  // negated for the dK/dV kernel, which runs after this one and seeds dP's
  // accumulator with it; lse2 = LSE * log2(e) too.
  float part = 0.f, lse = 0.f;
  if (q_ok) {
    const unsigned short* orow = static_cast<const unsigned short*>(p.o) + q_base + my_q * p.q_sr;
    u16x8 ov[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) ov[s] = *reinterpret_cast<const u16x8*>(orow + 16 * s + 8 * g);
    lse = p.lse[b * p.lse_sb + (si.off_q + my_q) * p.lse_sr + n * p.lse_sh];
    float cs[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      cs[s] = 0.f;
#pragma unroll
      for (int t = 0; t < 8; ++t) cs[s] += E::to_f32(oreg[s][t]) * E::to_f32(ov[s][t]);
    }
#pragma unroll
    for (int half = KS / 2; half >= 1; half >>= 1)
#pragma unroll
      for (int s = 0; s < half; ++s) cs[s] += cs[s + half];
    part = cs[0];
  }
  part += __shfl_xor(part, 32);
  const float dl = q_ok ? -(part * p.delta_scale) : 0.f;  // -softmax_grad
  const float l2 = q_ok ? lse * kLog2e : 0.f;
  if (row_out) {
    p.delta[bn * p.sq_max + my_q] = dl;
    p.lse2[bn * p.sq_max + my_q] = l2;
  }
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    settle(qreg[s]);
    settle(oreg[s]);
  }
  settle(l2);
  settle(dl);

  f32x16 adq[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) adq[nt] = f32x16{};

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
    // Two waves share each SIMD: the wave in an MFMA phase issues first, the
    // other one's softmax fills the gaps (measured: 2-3% faster here; the
    // forward kernel, whose online softmax is longer, ran 3-5% slower with it)
    __builtin_amdgcn_s_setprio(1);
    f32x16 st = {}, dpt = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      st = E::mma(frag_along_row<D>(tk, 0, 16 * ks, lane), qreg[ks], st);   // S^T[kv][q]
      dpt = E::mma(frag_along_row<D>(tv, 0, 16 * ks, lane), oreg[ks], dpt); // dP^T[kv][q]
    }
    __builtin_amdgcn_s_setprio(0);
    float dsv[16];
    if (nrows == 32 && !AM && rect_in_band(p, q0 + 32 * w, 32, row0, 32)) {  // uniform: no mask needed
#pragma unroll
      for (int i = 0; i < 16; ++i) dsv[i] = fast_exp2(st[i] * c2 - l2) * (dpt[i] + dl);  // dl = -softmax_grad
    } else {
      const uint32_t ex = AM ? mask_word(sAB[slot][AM ? w : 0], row0, l32) : 0u;
      // bit kv of keep: slice key kv takes part (valid, in the window, not
      // excluded); shifted as in the dK/dV kernel
      const uint32_t keys_ok = nrows >= 32 ? 0xffffffffu : ((1u << nrows) - 1u);
      const uint32_t keep = (keys_ok & ~ex & band_keys(p, my_q, row0)) >> (4 * g);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float x = ((keep >> (8 * (i >> 2) + (i & 3))) & 1u) ? fast_exp2(st[i] * c2 - l2) : 0.f;
        dsv[i] = x * (dpt[i] + dl);
      }
    }
    const u16x8 da[2] = {pack8<E>(dsv), pack8<E>(dsv + 8)};
    __builtin_amdgcn_s_setprio(1);
    // dQ^T += K^T dS^T: the fragment read down K's rows is, as an A operand,
    // K^T with the same k order as the dS^T registers (the B operand), so
    // each lane accumulates its own query row of dQ
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        adq[nt] = E::mma(frag_down_rows<D>(tk, 16 * hh, 32 * nt, lane), da[hh], adq[nt]);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // slices 0 .. NB-2 in flight, then per stage: wait for this wave's copies of
  // slice t, barrier (all copies landed; everyone is done with slice t - 1),
  // refill the freed buffer with slice t + NB - 1, compute slice t
#pragma unroll
  for (int t = 0; t < NB - 1; ++t) issue(t);
  wait_vmcnt<kWait>();
  __syncthreads();
  int nrows = sN[0];
  for (int t = 0; nrows > 0;) {  // nrows is uniform; 0 once the walk is over
    const int cur = t % NB;
    issue((t + NB - 1) % NB);
    compute(sK[cur], sV[cur], nrows, sR[cur], cur);
    ++t;
    wait_vmcnt<kWait>();
    __syncthreads();
    nrows = sN[t % NB];
  }
  wait_vmcnt<0>();  // copies of the empty slices past the end

  // lane: query row my_q; register i of column tile nt: element 32 nt + 8 (i / 4) + 4 g + i % 4
  if (my_q < w_end) {
    unsigned short* dqp = static_cast<unsigned short*>(p.dq) + b * p.dq_sb + (si.off_q + my_q) * p.dq_sr + n * p.dq_sh;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        float x[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) x[t] = adq[nt][4 * a + t] * p.dq_scale;
        store4<E>(dqp + 32 * nt + 8 * a + 4 * g, x);
      }
  }
}

// ---------------------------------------------------------------------------
// dQ by atomic adds (bsa_bwd_ex with BSA_DQ_ATOMIC)
// ---------------------------------------------------------------------------
// dq_acc = 0 before the dK/dV kernel adds into it (a fill kernel, so the call
// records no memset).
__global__ __launch_bounds__(256) void dq_acc_zero_kernel(float4* acc, int64_t n4) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n4;
       i += static_cast<int64_t>(gridDim.x) * 256)
    acc[i] = float4{0.f, 0.f, 0.f, 0.f};
}

// dQ = dq_acc * dq_scale rounded to the element type, one workgroup per 64
// positions of one (batch, query head), every row the call writes (rows past
// the sequence end hold zeros in dq_acc).
template <class E, int D>
__global__ __launch_bounds__(256) void dq_acc_store_kernel(Params p, int n_runs) {
  const int runs = (p.sq_max + 63) / 64;
  const int bn = blockIdx.x / runs;
  const int r0 = (blockIdx.x % runs) * 64;
  const int b = bn / p.N, n = bn % p.N;
  const SeqInfo si = seq_of(p, b);
  const int r1 = min(r0 + 64, si.wlim_q);
  constexpr int CH = D / 8;  // 8-element chunks per row
  unsigned short* dq = static_cast<unsigned short*>(p.dq) + b * p.dq_sb + si.off_q * p.dq_sr + n * p.dq_sh;
  const float* acc = p.dq_acc + static_cast<int64_t>(bn) * p.sq_max * D;
  for (int i = threadIdx.x; i < (r1 - r0) * CH; i += 256) {
    const int r = r0 + i / CH, c = 8 * (i % CH);
    const float4 x = *reinterpret_cast<const float4*>(acc + static_cast<int64_t>(r) * D + c);
    const float4 y = *reinterpret_cast<const float4*>(acc + static_cast<int64_t>(r) * D + c + 4);
    const float lo[4] = {x.x * p.dq_scale, x.y * p.dq_scale, x.z * p.dq_scale, x.w * p.dq_scale};
    const float hi[4] = {y.x * p.dq_scale, y.y * p.dq_scale, y.z * p.dq_scale, y.w * p.dq_scale};
    store4<E>(dq + r * p.dq_sr + c, lo);
    store4<E>(dq + r * p.dq_sr + c + 4, hi);
  }
}

}  // namespace

int launch_dq_acc_zero(const Params& p, void* stream) {
  const int64_t n4 = static_cast<int64_t>(p.B) * p.N * p.sq_max * p.D / 4;
  const int64_t blocks = std::min<int64_t>((n4 + 255) / 256, 8192);
  if (blocks == 0) return 0;
  hipLaunchKernelGGL(dq_acc_zero_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), reinterpret_cast<float4*>(p.dq_acc), n4);
  return static_cast<int>(hipGetLastError());
}

int launch_dq(const Params& p, void* stream) {
  if (p.dq_acc) {  // dQ by atomic adds: scale and store the accumulator
    const int n_runs = p.B * p.N * ((p.sq_max + 63) / 64);
    const dim3 grid(static_cast<unsigned>(n_runs));
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const bool bf = p.dtype == 2;
    if (p.D == 128) {
      if (bf) hipLaunchKernelGGL((dq_acc_store_kernel<EBf16, 128>), grid, dim3(256), 0, s, p, n_runs);
      else hipLaunchKernelGGL((dq_acc_store_kernel<EF16, 128>), grid, dim3(256), 0, s, p, n_runs);
    } else {
      if (bf) hipLaunchKernelGGL((dq_acc_store_kernel<EBf16, 64>), grid, dim3(256), 0, s, p, n_runs);
      else hipLaunchKernelGGL((dq_acc_store_kernel<EF16, 64>), grid, dim3(256), 0, s, p, n_runs);
    }
    return static_cast<int>(hipGetLastError());
  }
  if (p.n_dq_units == 0) return 0;
  const dim3 grid(static_cast<unsigned>(p.n_dq_units));
  BSA_DISPATCH(dq_kernel, waves_for(p.bx), grid, static_cast<hipStream_t>(stream), p);
  return static_cast<int>(hipGetLastError());
}

}  // namespace bsa
