// HIP kernels of the block-sparse attention backward for gfx950 (CDNA4).
//
// Stages, all enqueued on the caller's stream (aclnnBlockSparseAttentionGrad
// page, 功能说明 / 计算公式 for the equations):
//
//   stage_seq   copy the per-sequence table (offsets, lengths) into the workspace
//   (pack_amask / stage_fp8: only with an attenMask / fp8 inputs)
//   prologue    one launch, three block ranges:
//                 - per-Q-block lists of selected in-range KV blocks
//                 - per-KV-block lists of selected in-range Q blocks
//                 - softmax_grad: delta = rowsum(dOut o Out) in fp32, stored
//                   negated (it seeds dP's accumulator: dP - delta), and
//                   lse2 = softmaxLse * log2(e), both [B, N, maxSq]
//   plan        one workgroup: splits KV blocks that many Q blocks select
//               into pieces and orders the dK/dV work longest first; picks
//               the dQ workgroup order
//   dkdv        one workgroup per work item (batch, KV head, KV block
//               [, 128-row part] [, piece]); K/V rows stay in registers;
//               walks the Q blocks that select it for every query head of
//               its group:  S, P, dV += P^T dO, dP, dS, dK += dS^T Q  (four
//               MFMA GEMMs per step).  Q/dO tiles (XOR-swizzled) are
//               double-buffered in LDS, the next one copied in by DMA during
//               the current one.
//   dq          one workgroup per (batch, query head, Q block [, part]);
//               Q/dO rows in registers; streams 32-row slices of its KV blocks
//               through a ring of XOR-swizzled LDS buffers filled by DMA:
//               S, P, dP, dS, dQ += dS K (three MFMA GEMMs per slice).  Extra
//               workgroups of the same launch sum the pieces of split dK/dV
//               work items in piece order.  No atomics on outputs anywhere,
//               so every output is written in a fixed order.
//   fwd         (the forward entry point) the dq kernel's structure with an
//               online softmax: O and LSE.
// MFMA used: v_mfma_f32_32x32x16_{bf16,f16}.  Operand layout (wave64, lane l,
// g = l / 32):  A[m][k]: lane holds row m = l % 32, k = 8g .. 8g+7;
// B[k][n]: lane holds column n = l % 32, k = 8g .. 8g+7;  C[m][n] (16 fp32):
// register i holds row 8*(i/4) + 4g + (i%4), column l % 32.
// A C tile's registers 8h..8h+7 therefore hold, per lane, the rows
// 16h + {4g..4g+3, 8+4g..8+4g+3}: the same (g, t) -> index map is used for
// the K dimension of the next product, so a score tile feeds the next MFMA
// straight from registers and only the other operand is gathered from LDS in
// that order.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "bsa_internal.h"

namespace bsa {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kTileRows = 128;  // rows per workgroup part (32 per wave, at most 4 waves)

struct EBf16 {
  static __device__ __forceinline__ f32x16 mma(u16x8 a, u16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ unsigned short from_f32(float x) {
    return __builtin_bit_cast(unsigned short, static_cast<__bf16>(x));
  }
  static __device__ __forceinline__ float to_f32(unsigned short u) {
    return __uint_as_float(static_cast<unsigned>(u) << 16);
  }
};

struct EF16 {
  static __device__ __forceinline__ f32x16 mma(u16x8 a, u16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ unsigned short from_f32(float x) {
    return __builtin_bit_cast(unsigned short, static_cast<_Float16>(x));
  }
  static __device__ __forceinline__ float to_f32(unsigned short u) {
    return static_cast<float>(__builtin_bit_cast(_Float16, u));
  }
};

template <class E>
__device__ __forceinline__ u16x8 pack8(const float* x) {
  u16x8 r;
#pragma unroll
  for (int t = 0; t < 8; ++t) r[t] = E::from_f32(x[t]);
  return r;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Four consecutive outputs rounded to the element type, as one 8-byte store
// when the address allows it (outputs may have any outer strides; the row
// start is 2-byte aligned only in general), else as four 2-byte stores.
template <class E>
__device__ __forceinline__ void store4(unsigned short* dst, const float (&x)[4]) {
  unsigned short r[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) r[t] = E::from_f32(x[t]);
  if ((reinterpret_cast<uintptr_t>(dst) & 7u) == 0) {
    typedef unsigned short u16x4_t __attribute__((ext_vector_type(4)));
    *reinterpret_cast<u16x4_t*>(dst) = u16x4_t{r[0], r[1], r[2], r[3]};
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) dst[t] = r[t];
  }
}

// The sliding window (preTokens / nextTokens): key position j takes part for
// query position i only if i - pre <= j <= i + next.  Positions are below
// 2^31, so j - i fits in 32 bits; pre and next are clamped on the host.
// Every pair of rows [r0, r0 + nr) x columns [c0, c0 + nc) is in the window
// (true without one): the differences j - i fill [c0 - r0 - nr + 1, c0 + nc - 1 - r0].
__device__ __forceinline__ bool rect_in_band(const Params& p, int r0, int nr, int c0, int nc) {
  return !p.win || (c0 - (r0 + nr - 1) >= -p.win_pre && (c0 + nc - 1) - r0 <= p.win_next);
}
// Bits lo..hi (clipped to 0..31) of a 32-bit word: the contiguous run of a
// slice's 32 rows or keys that a lane's window admits (0 if none).
__device__ __forceinline__ uint32_t bit_run(int64_t lo, int64_t hi) {
  if (lo < 0) lo = 0;
  if (hi > 31) hi = 31;
  if (lo > hi) return 0u;
  return (0xffffffffu >> (31 - static_cast<int>(hi))) & (0xffffffffu << static_cast<int>(lo));
}
// The rows r of a slice whose query qs + r has key j in the window
// (i - pre <= j <= i + next, i.e. j - next <= i <= j + pre); all without one.
__device__ __forceinline__ uint32_t band_rows(const Params& p, int qs, int j) {
  if (!p.win) return 0xffffffffu;
  return bit_run(static_cast<int64_t>(j) - p.win_next - qs, static_cast<int64_t>(j) + p.win_pre - qs);
}
// The keys k of a slice starting at key row0 in the window of query i.
__device__ __forceinline__ uint32_t band_keys(const Params& p, int i, int row0) {
  if (!p.win) return 0xffffffffu;
  return bit_run(static_cast<int64_t>(i) - p.win_pre - row0, static_cast<int64_t>(i) + p.win_next - row0);
}
// attenMask bits of a 32-key slice starting at key row0, for the query of
// lane l32, from the two words staged for it (bit k: key row0 + k excluded).
__device__ __forceinline__ uint32_t mask_word(const uint32_t* staged, int row0, int l32) {
  const uint64_t two = (static_cast<uint64_t>(staged[32 + l32]) << 32) | staged[l32];
  return static_cast<uint32_t>(two >> (row0 & 31));
}
// Some pair of the rectangle is in the window: the differences j - i over it
// fill [c0 - (r0 + nr - 1), c0 + nc - 1 - r0], which must meet [-pre, next]
// (empty when pre + next < 0: such a window admits no pair at all).
__device__ __forceinline__ bool rect_meets_band(const Params& p, int r0, int nr, int c0, int nc) {
  return !p.win || (c0 - (r0 + nr - 1) <= p.win_next && (c0 + nc - 1) - r0 >= -p.win_pre &&
                    static_cast<int64_t>(p.win_pre) + p.win_next >= 0);
}

// ---------------------------------------------------------------------------
// per-sequence table
// ---------------------------------------------------------------------------
__global__ void stage_seq_kernel(SeqChunk c, SeqInfo* dst, float* consts) {
  const int t = threadIdx.x;
  if (t < c.count) dst[c.first + t] = c.s[t];
  if (c.first == 0) {
    for (int i = t; i < kConstFloats; i += blockDim.x)
      consts[i] = i == kConstPosInf ? __builtin_inff() : i == kConstNegInf ? -__builtin_inff() : 0.f;
  }
}

// ---------------------------------------------------------------------------
// fp8 inputs: decode to bf16 copies
// ---------------------------------------------------------------------------
// OCP 8-bit floats -> bf16, exactly: v_cvt_pk_f32_fp8 / _bf8 decode two
// E4M3FN / E5M2 codes (gfx950 takes the OCP encodings) to fp32, whose upper
// 16 bits are the bf16 value (an fp8 value has at most 4 significant bits).
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ unsigned pack_bf16x2(f32x2 v) {
  return (__float_as_uint(v[0]) >> 16) | (__float_as_uint(v[1]) & 0xffff0000u);
}

// One thread per 16-byte group: 16 codes in, two 16-byte stores of bf16 out.
// Groups are numbered over the tensors in order; a workgroup may straddle two.
__global__ __launch_bounds__(256) void stage_fp8_kernel(Fp8Stage st) {
  int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  int t = 0;
  while (t < st.count && gid >= st.n16[t]) gid -= st.n16[t++];
  if (t >= st.count) return;
  const bool e5 = st.fmt[t] == 1;
  const uint4 in = reinterpret_cast<const uint4*>(st.src[t])[gid];
  const unsigned w[4] = {in.x, in.y, in.z, in.w};
  unsigned o[8];  // bf16 pairs: codes 2k, 2k + 1
  if (e5) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = pack_bf16x2(__builtin_amdgcn_cvt_pk_f32_bf8(w[i], false));
      o[2 * i + 1] = pack_bf16x2(__builtin_amdgcn_cvt_pk_f32_bf8(w[i], true));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = pack_bf16x2(__builtin_amdgcn_cvt_pk_f32_fp8(w[i], false));
      o[2 * i + 1] = pack_bf16x2(__builtin_amdgcn_cvt_pk_f32_fp8(w[i], true));
    }
  }
  uint4* out = reinterpret_cast<uint4*>(st.dst[t]) + 2 * gid;
  out[0] = uint4{o[0], o[1], o[2], o[3]};
  out[1] = uint4{o[4], o[5], o[6], o[7]};
}

// ---------------------------------------------------------------------------
// attenMask: bytes -> bits
// ---------------------------------------------------------------------------
// One wave per 64 x 64 tile of the [maxSq, maxSkv] byte mask: lane l reads
// column j0 + l of each of the 64 rows (64 contiguous bytes per row); a
// ballot over the lanes gives the row's two 32-key words, and each lane
// gathers its column's two 32-query words in registers.  Bits past the
// mask's edges are 0.
__global__ __launch_bounds__(256) void pack_amask_kernel(Params p, int tiles_i, int tiles_j) {
  const int lane = threadIdx.x & 63;
  const int64_t tile = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (tile >= static_cast<int64_t>(tiles_i) * tiles_j) return;  // uniform over the wave
  const int ti = static_cast<int>(tile / tiles_j), tj = static_cast<int>(tile % tiles_j);
  const int i0 = 64 * ti, j = 64 * tj + lane;
  const int sq = p.sq_max;
  const int64_t skv = p.amask_ld;
  uint32_t col[2] = {0u, 0u};
#pragma unroll 8
  for (int r = 0; r < 64; ++r) {
    const int i = i0 + r;
    const bool x = i < sq && j < skv && p.amask[static_cast<int64_t>(i) * skv + j] != 0;
    const uint64_t row = __ballot(x);
    const int w = 2 * tj + lane;
    if (i < sq && lane < 2 && w < p.am_wk)
      p.am_rows[static_cast<int64_t>(i) * p.am_wk + w] = static_cast<uint32_t>(lane ? row >> 32 : row);
    col[r >> 5] |= static_cast<uint32_t>(x) << (r & 31);
  }
  if (p.am_cols != nullptr && j < skv) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      if (2 * ti + h < p.am_wq) p.am_cols[static_cast<int64_t>(j) * p.am_wq + 2 * ti + h] = col[h];
  }
}

// ---------------------------------------------------------------------------
// prologue: softmax_grad + lse2, block lists
// ---------------------------------------------------------------------------
// softmax_grad = row sums of dOut o Out, and lse2 = LSE * log2(e), for every
// row of the [B, N, maxSq] grid (0 past a sequence's length).  A workgroup
// takes 64 consecutive positions of one (b, n), for either layout: its loads
// are whole rows (D contiguous elements each) and its stores one contiguous
// run of the [B, N, maxSq] arrays.  LPR lanes read a row's D elements 16
// bytes each, and every pass's loads are issued together.
template <class E, int D>
__device__ void delta_part(const Params& p, int blk) {
  constexpr int LPR = D / 8;        // lanes per row, 8 elements (16 bytes) each
  constexpr int RPP = 256 / LPR;    // rows per pass of the 256-thread block
  constexpr int NP = kDeltaRowsPerBlock / RPP;
  const int tid = threadIdx.x;
  const int sub = tid % LPR, rloc = tid / LPR;
  const unsigned short* op = static_cast<const unsigned short*>(p.o);
  const unsigned short* dp = static_cast<const unsigned short*>(p.dout);
  const int per_run = (p.sq_max + kDeltaRowsPerBlock - 1) / kDeltaRowsPerBlock;
  const int outer = blk / per_run;  // b * N + n
  const int f0 = (blk % per_run) * kDeltaRowsPerBlock;
  float acc[NP], l2[NP];
  int64_t out[NP];
  bool valid[NP];
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    const int i = f0 + k * RPP + rloc;  // position within the (b, n) run
    const int b = outer / p.N;
    const int n = outer - b * p.N;
    const SeqInfo si = p.seq[b];
    out[k] = i < p.sq_max ? (static_cast<int64_t>(b) * p.N + n) * p.sq_max + i : -1;
    valid[k] = i < si.len_q;
    acc[k] = 0.f;
    l2[k] = 0.f;
    if (valid[k]) {
      const int64_t off = b * p.q_sb + (si.off_q + i) * p.q_sr + n * p.q_sh + sub * 8;
      const u16x8 ov = *reinterpret_cast<const u16x8*>(op + off);
      const u16x8 dv = *reinterpret_cast<const u16x8*>(dp + off);
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[k] += E::to_f32(dv[t]) * E::to_f32(ov[t]);
      if (sub == 0) l2[k] = p.lse[b * p.lse_sb + (si.off_q + i) * p.lse_sr + n * p.lse_sh] * kLog2e;
    }
  }
#pragma unroll
  for (int k = 0; k < NP; ++k) {
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) acc[k] += __shfl_xor(acc[k], m);
    if (sub == 0 && out[k] >= 0) {
      p.delta[out[k]] = -(acc[k] * p.delta_scale);  // stored negated
      p.lse2[out[k]] = l2[k];
    }
  }
}

// One wave per (b, n, Q block): ascending list of selected in-range KV blocks.
__device__ void row_list_part(const Params& p, int blk) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t R = static_cast<int64_t>(blk) * 4 + w;
  if (R >= static_cast<int64_t>(p.B) * p.N * p.nqb) return;  // wave-uniform
  const int ib = static_cast<int>(R % p.nqb);
  const int b = static_cast<int>(R / p.nqb / p.N);
  const SeqInfo si = p.seq[b];
  const int nq_b = (si.len_q + p.bx - 1) / p.bx;
  const int nk_b = (si.len_kv + p.by - 1) / p.by;
  int base = 0;
  if (ib < nq_b) {
    int32_t* out = p.row_list + R * p.nkb;
    const uint8_t* mrow = p.mask ? p.mask + R * p.nkb : nullptr;
    const int r0 = ib * p.bx, nr = min(p.bx, si.len_q - r0);
    // the mask bytes of kRowSteps steps of 64 blocks are loaded before any
    // list entry is stored (the int32 stores could otherwise alias the byte
    // loads, which would then wait for each other step by step)
    constexpr int kRowSteps = 8;
    for (int j00 = 0; j00 < nk_b; j00 += 64 * kRowSteps) {
      uint8_t sel[kRowSteps];
#pragma unroll
      for (int u = 0; u < kRowSteps; ++u) {
        const int j = j00 + 64 * u + lane;
        sel[u] = j < nk_b ? (mrow ? mrow[j] : 1) : 0;
      }
#pragma unroll
      for (int u = 0; u < kRowSteps; ++u) {
        const int j = j00 + 64 * u + lane;
        const bool on = sel[u] != 0 && rect_meets_band(p, r0, nr, j * p.by, min(p.by, si.len_kv - j * p.by));
        const uint64_t bal = __ballot(on);
        const int pre = __popcll(bal & ((1ull << lane) - 1ull));
        if (on) out[base + pre] = j;
        base += __popcll(bal);
      }
    }
  }
  if (lane == 0) p.row_cnt[R] = base;
}

// One workgroup per (b, n, group of 64 KV blocks): ascending lists of the
// selected in-range Q blocks of those 64 columns.  The mask is taken 64 Q-block
// rows at a time through an LDS tile (byte rows at a pitch of 68, so that a
// column read down the 64 rows hits 64 distinct banks); wave w then compacts
// columns 16w .. 16w + 15 of the tile with one ballot per column.
constexpr int kColTilePitch = 68;
__device__ void col_list_part(const Params& p, int blk) {
  __shared__ uint8_t tile[64 * kColTilePitch];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int ncw = (p.nkb + 63) / 64;
  const int cw = blk % ncw;
  const int64_t bn = blk / ncw;
  const int b = static_cast<int>(bn / p.N);
  const SeqInfo si = p.seq[b];
  const int nq_b = (si.len_q + p.bx - 1) / p.bx;
  const int nk_b = (si.len_kv + p.by - 1) / p.by;
  const int j0 = cw * 64;
  int cnt[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) cnt[k] = 0;
  for (int i0 = 0; i0 < nq_b; i0 += 64) {  // uniform over the workgroup
    __syncthreads();  // the previous tile is consumed
    {
      const int r = tid >> 2, c0 = 16 * (tid & 3);
      const int i = i0 + r;
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const int j = j0 + c0 + c;
        uint8_t v = 0;
        if (i < nq_b && j < nk_b &&
            rect_meets_band(p, i * p.bx, min(p.bx, si.len_q - i * p.bx), j * p.by, min(p.by, si.len_kv - j * p.by)))
          v = p.mask ? p.mask[(bn * p.nqb + i) * p.nkb + j] : 1;
        tile[r * kColTilePitch + c0 + c] = v;
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int c = 16 * w + k;
      const bool on = tile[lane * kColTilePitch + c] != 0;  // 0 outside the in-range rows/columns
      const uint64_t bal = __ballot(on);
      const int j = j0 + c;
      if (on) p.col_list[(bn * p.nkb + j) * p.nqb + cnt[k] + __popcll(bal & ((1ull << lane) - 1ull))] = i0 + lane;
      cnt[k] += __popcll(bal);
    }
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int j = j0 + 16 * w + k;
    if (lane == 0 && j < p.nkb) p.col_cnt[bn * p.nkb + j] = cnt[k];
  }
}

// Row lists, then column lists, then softmax_grad workgroups (the forward
// launches the row lists only).  The list workgroups are latency-bound (a
// row-list wave walks its mask row 64 blocks per dependent load); dispatched
// first, they overlap the bandwidth-bound softmax_grad pass instead of
// trailing it.
template <class E, int D>
__global__ __launch_bounds__(256) void prologue_kernel(Params p, int nb_rows, int nb_cols) {
  const int bid = blockIdx.x;
  if (bid < nb_rows) row_list_part(p, bid);
  else if (bid < nb_rows + nb_cols) col_list_part(p, bid - nb_rows);
  else delta_part<E, D>(p, bid - nb_rows - nb_cols);
}


// ---------------------------------------------------------------------------
// work split of the dK/dV kernel
// ---------------------------------------------------------------------------
// One dK/dV unit (batch, KV head, KV block, 128-row part) walks every Q block
// that selects it, for every query head of its group: T_u entries.  Units with
// far more entries than the rest (a KV block every Q block selects) would keep
// one workgroup busy long after the others finish, so a unit with
// T_u > chunk is cut into ceil(T_u / chunk) pieces of consecutive entries;
// each piece writes an fp32 partial dK/dV and the pieces are summed in order
// afterwards, so the result is the same on every run.  Pieces get slots by an
// exclusive scan over units in unit order; units that would overflow the slot
// capacity stay whole.  One workgroup of 1024 threads.
__device__ __forceinline__ int unit_entries(const Params& p, int u) {
  const int nsub = (p.by + kTileRows - 1) / kTileRows;
  int w = u / nsub;
  const int jb = w % p.nkb;
  w /= p.nkb;
  const int h = w % p.Nkv;
  const int b = w / p.Nkv;
  int t = 0;
  for (int n = h * p.G; n < (h + 1) * p.G; ++n) t += p.col_cnt[(static_cast<int64_t>(b) * p.N + n) * p.nkb + jb];
  return t;
}

// dQ workgroup order.  Hardware hands workgroup i to XCD i % 8.  With XCD
// ranges, XCD x runs the x-th of eight contiguous ranges of dQ units (range x
// starts at x * per + min(x, rem) for per = n / 8, rem = n % 8), so the Q
// blocks of a head group, which read the same K/V rows, share one L2; the plan
// kernel picks it only when the eight ranges hold nearly equal work, since one
// heavy range (a long sequence among short ones) would leave seven XCDs idle.
// Either way the units are launched longest first (see plan_kernel).
// The XCD whose range holds unit u.
__device__ __forceinline__ int xcd_of_unit(int u, int n) {
  const int per = n >> 3, rem = n & 7;
  const int big = (per + 1) * rem;  // the first rem ranges hold per + 1 units
  return u < big ? u / (per + 1) : rem + (u - big) / max(per, 1);
}
constexpr int kDqOrderPlain = 0, kDqOrderXcdRange = 1;

// The plan region, in order: [0] chunk, [1] number of work items, [2] dQ order, [3]
// the next work item to take (the persistent dK/dV kernel's counter), then per unit its piece count and first slot, per slot its unit
// (-1 = unused) and piece, the work items (unit, piece) in launch order, and
// the dQ units in launch order.
struct PlanView {
  int32_t* unit_k;
  int32_t* unit_base;
  int32_t* slot_unit;
  int32_t* slot_chunk;
  int32_t* order_unit;
  int32_t* order_piece;
  int32_t* dq_order;  // dQ workgroup k runs dQ unit dq_order[k]
  __device__ explicit PlanView(const Params& p) {
    unit_k = p.plan + 4;
    unit_base = unit_k + p.n_units;
    slot_unit = unit_base + p.n_units;
    slot_chunk = slot_unit + p.slots_cap;
    order_unit = slot_chunk + p.slots_cap;
    order_piece = order_unit + p.n_units + p.slots_cap;
    dq_order = order_piece + p.n_units + p.slots_cap;
  }
};

// Launch order of the work items: longest first, so that the last workgroups
// to start are short ones.  Costs (Q-block entries of the piece) are binned
// into kOrderBins classes, class kOrderBins-1 holding pieces of about `chunk`
// entries and class 0 the units with nothing to do (they only write zeros).
// The order inside a class depends on scheduling; the results do not, since
// every piece sums its entries in list order and pieces are reduced in order.
constexpr int kOrderBins = 64;
__device__ __forceinline__ int order_bin(int cost, int chunk) {
  if (cost <= 0) return 0;
  return min(kOrderBins - 1, 1 + static_cast<int>((static_cast<long long>(cost - 1) * (kOrderBins - 1)) / chunk));
}

constexpr int kPlanCachedUnits = 8192;  // units whose T_u the plan kernel keeps in LDS

__global__ __launch_bounds__(1024) void plan_kernel(Params p) {
  __shared__ long long s_red[1024];
  __shared__ int s_scan[1024];
  __shared__ int s_hist[kOrderBins], s_cursor[kOrderBins];
  __shared__ unsigned long long s_xcd[8];
  __shared__ int s_T[kPlanCachedUnits];
  __shared__ int s_dq[8 * kOrderBins];  // dQ cost classes per XCD range: counts, then cursors
  __shared__ int s_dqmax;
  const int tid = threadIdx.x;
  const PlanView pv(p);
  const int per = (p.n_units + 1023) / 1024;
  const int u0 = min(p.n_units, tid * per), u1 = min(p.n_units, u0 + per);
  if (tid < kOrderBins) s_hist[tid] = 0;
  if (tid < 8) s_xcd[tid] = 0;
  if (tid < 8 * kOrderBins) s_dq[tid] = 0;
  if (tid == 0) s_dqmax = 0;
  // T_u, read from the column counts once (each thread reads back only its own units)
  const bool cached = p.n_units <= kPlanCachedUnits;
  auto T = [&](int u) { return cached ? s_T[u] : unit_entries(p, u); };

  long long tot = 0;
  for (int u = u0; u < u1; ++u) {
    const int t = unit_entries(p, u);
    if (cached) s_T[u] = t;
    tot += t;
  }
  s_red[tid] = tot;
  __syncthreads();
  for (int st = 512; st > 0; st >>= 1) {
    if (tid < st) s_red[tid] += s_red[tid + st];
    __syncthreads();
  }
  const long long total = s_red[0];
  const int chunk = static_cast<int>(max(static_cast<long long>(kMinChunk),
                                         (total + kBalanceGroups - 1) / kBalanceGroups));

  int mine = 0;
  for (int u = u0; u < u1; ++u) {
    const int t = T(u);
    if (t > chunk) mine += (t + chunk - 1) / chunk;
  }
  s_scan[tid] = mine;
  for (int i = tid; i < p.slots_cap; i += 1024) pv.slot_unit[i] = -1;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive scan
    const int v = tid >= off ? s_scan[tid - off] : 0;
    __syncthreads();
    s_scan[tid] += v;
    __syncthreads();
  }
  int run = s_scan[tid] - mine;  // exclusive prefix
  int extra = 0;                 // pieces >= 1 this thread creates
  for (int u = u0; u < u1; ++u) {
    const int t = T(u);
    const int k = t > chunk ? (t + chunk - 1) / chunk : 1;
    if (k > 1 && run + k <= p.slots_cap) {
      pv.unit_k[u] = k;
      pv.unit_base[u] = run;
      for (int c = 0; c < k; ++c) {
        pv.slot_unit[run + c] = u;
        pv.slot_chunk[run + c] = c;
        atomicAdd(&s_hist[order_bin(min(chunk, t - c * chunk), chunk)], 1);
      }
      run += k;
      extra += k - 1;
    } else {
      pv.unit_k[u] = 1;
      pv.unit_base[u] = 0;
      atomicAdd(&s_hist[order_bin(t, chunk)], 1);
    }
  }
  s_scan[tid] = extra;
  __syncthreads();
  for (int st = 512; st > 0; st >>= 1) {
    if (tid < st) s_scan[tid] += s_scan[tid + st];
    __syncthreads();
  }
  // dQ order: work of each XCD range, a unit costing its selected KV blocks + 1
  {
    // strided over the units (coalesced, several loads in flight per thread);
    // a thread's units change XCD range only every nd / 8 units
    const int nd = p.n_dq_units, nsub_q = (p.bx + kTileRows - 1) / kTileRows;
    unsigned long long acc = 0;
    int cur = xcd_of_unit(min(tid, max(nd - 1, 0)), max(nd, 1));
    int mx = 0;
#pragma unroll 4
    for (int u = tid; u < nd; u += 1024) {
      const int x = xcd_of_unit(u, nd);
      const int rc = p.row_cnt[u / nsub_q];
      const unsigned c = 1u + static_cast<unsigned>(rc);
      if (x != cur) {
        atomicAdd(&s_xcd[cur], acc);
        acc = 0;
        cur = x;
      }
      acc += c;
      mx = max(mx, rc);
    }
    if (acc) atomicAdd(&s_xcd[cur], acc);
    atomicMax(&s_dqmax, mx);
  }
  __syncthreads();
  if (tid == 0) {
    unsigned long long tot = 0, mx = 0;
    for (int x = 0; x < 8; ++x) {
      tot += s_xcd[x];
      mx = max(mx, s_xcd[x]);
    }
    // contiguous ranges only if the heaviest holds at most 1/32 more than the mean
    p.plan[2] = 8 * mx * 32 <= tot * 33 ? kDqOrderXcdRange : kDqOrderPlain;
    int base = 0;  // classes in descending order
    for (int c = kOrderBins - 1; c >= 0; --c) {
      s_cursor[c] = base;
      base += s_hist[c];
    }
    p.plan[0] = chunk;
    p.plan[1] = p.n_units + s_scan[0];
    p.plan[3] = 0;  // the persistent dK/dV kernel's item counter
  }
  __syncthreads();
  for (int u = u0; u < u1; ++u) {
    const int t = T(u);
    const int k = pv.unit_k[u];
    for (int c = 0; c < k; ++c) {
      const int at = atomicAdd(&s_cursor[order_bin(k > 1 ? min(chunk, t - c * chunk) : t, chunk)], 1);
      pv.order_unit[at] = u;
      pv.order_piece[at] = c;
    }
  }
  // dQ launch order, longest first (cost classes of the selected KV-block
  // count): with XCD ranges, within each range (workgroup 8 k + x runs the
  // k-th unit of range x, as the hardware hands workgroup i to XCD i % 8);
  // otherwise over all units, dealt round-robin to the XCDs.  Results do not
  // depend on the order.
  {
    const int nd = p.n_dq_units, nsub_q = (p.bx + kTileRows - 1) / kTileRows;
    const bool ranges = p.plan[2] == kDqOrderXcdRange;
    const int mxc = max(s_dqmax, 1);
    auto cls = [&](int u) { return order_bin(p.row_cnt[u / nsub_q], mxc); };
    for (int u = tid; u < nd; u += 1024) atomicAdd(&s_dq[(ranges ? xcd_of_unit(u, nd) : 0) * kOrderBins + cls(u)], 1);
    __syncthreads();
    if (tid < (ranges ? 8 : 1)) {  // per range: cursors of the classes in descending order
      int base = 0;
      for (int c = kOrderBins - 1; c >= 0; --c) {
        const int n = s_dq[tid * kOrderBins + c];
        s_dq[tid * kOrderBins + c] = base;
        base += n;
      }
    }
    __syncthreads();
    for (int u = tid; u < nd; u += 1024) {
      const int x = ranges ? xcd_of_unit(u, nd) : 0;
      const int k = atomicAdd(&s_dq[x * kOrderBins + cls(u)], 1);
      pv.dq_order[ranges ? 8 * k + x : k] = u;
    }
  }
}

// ---------------------------------------------------------------------------
// shared pieces of the two MFMA kernels
// ---------------------------------------------------------------------------
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) unsigned short lds_u16;
typedef __attribute__((address_space(3))) void lds_void;

// LDS tiles: row-major, D elements per row, no padding; the 16-byte chunks of
// row r are XOR-permuted by swz(r) so that 16-byte reads of one chunk column
// by 16 consecutive rows and transposing reads of 4 consecutive rows spread
// over the banks (the best single layout for both patterns measured on gfx950).
// Rows of 256 B and of 512 B both start on bank 0, so D = 256 takes D = 128's
// permutation (of its first 16 chunks).
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D >= 128) return 2 * (r & 3) + ((r >> 2) & 1) + 8 * ((r >> 3) & 1);
  else return 2 * (r & 3) + ((r >> 2) & 1);
}
template <int D>
__device__ __forceinline__ int tile_off(int r, int col) {
  return r * D + ((((col >> 3) ^ swz<D>(r))) << 3) + (col & 7);
}

// ds_read_b64_tr_b16: within each 16-lane block, lanes 4t..4t+3 address four
// consecutive 16-bit elements of row t (t = 0..3); lane j of the block then
// holds column j of those four rows, one row per element.
__device__ __forceinline__ u16x4 lds_read_tr(const unsigned short* tile, int elem) {
  // C-style casts: generic -> LDS address-space conversion of a pointer into __shared__ memory
  lds_u16* base = (lds_u16*)(tile);
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + elem));
  return __builtin_bit_cast(u16x4, v);
}

// MFMA B fragment read down the rows of a tile: lane (column n = l % 32,
// g = l / 32) gets rows r0 + 4g + {0..3} and r0 + 8 + 4g + {0..3} of column
// col0 + n -- the k order of a C tile's registers 8h..8h+7 (see the layout
// note at the top of this file).
template <int D>
__device__ __forceinline__ u16x8 frag_down_rows(const unsigned short* tile, int r0, int col0, int lane) {
  const int row = r0 + 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int col = col0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const u16x4 a = lds_read_tr(tile, tile_off<D>(row, col));
  const u16x4 b = lds_read_tr(tile, tile_off<D>(row + 8, col));
  return u16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// MFMA A fragment read along a row: lane (row m = l % 32, g) gets columns
// col0 + 8g .. col0 + 8g + 7 of row r0 + m.
template <int D>
__device__ __forceinline__ u16x8 frag_along_row(const unsigned short* tile, int r0, int col0, int lane) {
  return *reinterpret_cast<const u16x8*>(tile + tile_off<D>(r0 + (lane & 31), col0 + 8 * (lane >> 5)));
}

// The work of a workgroup is a stream of 32-row slices (of Q blocks for the
// dK/dV kernel, of KV blocks for the dQ and forward kernels); every wave
// computes on every slice.  nrows == 0 marks an empty slice.
struct Slice {
  int head;   // query head (dK/dV kernel); unused by the dQ kernel
  int row0;   // first sequence-local row
  int nrows;  // valid rows, 0..32
};

// The LDS-DMA loads read m0 for their destination, and an SALU write of m0
// needs one wait state before such a load reads it (a gfx9 hazard the
// compiler observes for its own code but cannot see inside inline assembly):
// hence the s_nop between the two.
//
// Direct global -> LDS copy (global_load_lds_dwordx4): lane L's 16 bytes,
// read from a wave-uniform base (held in an SGPR pair) plus a per-lane 32-bit
// byte offset, land at LDS byte address m0 + 16 L, with no register staging
// and no per-lane 64-bit address arithmetic.  Issued from inline assembly so
// that the compiler adds no waits of its own around it: the caller waits on
// vmcnt for its own copies, then a barrier publishes the buffer to the
// workgroup.  (Compiler-issued vector loads are counted by the same vmcnt;
// loads complete in issue order, so either side's waits may only wait longer
// than needed, never shorter.)
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return static_cast<unsigned>(reinterpret_cast<uintptr_t>((lds_void*)(p)));
}
__device__ __forceinline__ void dma16s(const void* base, unsigned voff, unsigned lds) {
  // base and lds are wave-uniform by construction; readfirstlane states it to
  // the compiler, which may not prove it and then could not place base in SGPRs
  const unsigned m = __builtin_amdgcn_readfirstlane(lds);
  // (readfirstlane yields an int: each half is widened through unsigned, so
  // that the low half is zero-extended)
  const uint64_t bp = reinterpret_cast<uintptr_t>(base);
  const unsigned lo = static_cast<unsigned>(__builtin_amdgcn_readfirstlane(static_cast<unsigned>(bp)));
  const unsigned hi = static_cast<unsigned>(__builtin_amdgcn_readfirstlane(static_cast<unsigned>(bp >> 32)));
  const uint64_t sb = (static_cast<uint64_t>(hi) << 32) | lo;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sb), "s"(m)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* src, unsigned lds) {  // lane L's 4 bytes -> m0 + 4 L
  const unsigned m = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" : : "v"(src), "s"(m) : "memory", "m0");
}
// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding: vmcnt
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// A ring of NB LDS buffers, each holding one 32-row slice of K and of V in the
// swizzled tile layout, filled by DMA NB - 1 slices ahead of the compute.  One
// wave instruction fills 1 KB (512 / D rows): lane L writes physical chunk
// L % (D/8) of row L / (D/8) and so fetches the logical chunk that the swizzle
// puts there, at a per-lane byte offset from the slice's first row that is the
// same for every slice (computed once).  Lanes of rows past a slice's end read
// a chunk of its first row instead (finite data that the kernels mask to a
// zero weight); an empty slice reads a zero block.  Every stage issues the
// same number of copies, so the wait before a stage is a constant.
template <int D, int W, int NB>
struct KVRing {
  static constexpr int RPI = 512 / D;       // rows per wave instruction
  static constexpr int IPT = 32 / RPI;      // wave instructions per tensor and slice
  static constexpr int IPW = IPT / W;       // ... per wave
  static constexpr int NI = 2 * IPW;        // copies per wave and stage (K and V)
  static constexpr int WAIT = (NB - 2) * NI;  // copies of the two later stages still in flight
  static_assert(IPW >= 1 && IPW * W == IPT, "slice must split evenly over the waves");

  unsigned voff[IPW];  // byte offset of this lane's chunk from the slice's first row
  unsigned vz;         // a chunk of the first row (rows past the end)
  int lrow;            // this lane's row within an instruction's RPI rows
  int w;

  __device__ __forceinline__ KVRing(int64_t sr, int w_, int lane) : w(w_) {
    lrow = lane / (D / 8);
    vz = 16u * static_cast<unsigned>(lane % (D / 8 < 16 ? D / 8 : 16));  // inside the zero block too
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int r = (w * IPW + i) * RPI + lrow;
      const int c = (lane % (D / 8)) ^ swz<D>(r);
      voff[i] = static_cast<unsigned>(2 * (r * sr + 8 * c));
    }
  }

  __device__ __forceinline__ void issue(unsigned short* tk, unsigned short* tv, const Slice& s,
                                        const unsigned short* kp, const unsigned short* vp, int64_t sr,
                                        const void* zeros) const {
    const unsigned kb = lds_addr(tk), vb = lds_addr(tv);
    const bool any = s.nrows > 0;
    const void* kbase = any ? static_cast<const void*>(kp + static_cast<int64_t>(s.row0) * sr) : zeros;
    const void* vbase = any ? static_cast<const void*>(vp + static_cast<int64_t>(s.row0) * sr) : zeros;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int ins = w * IPW + i;
      const unsigned v = ins * RPI + lrow < s.nrows ? voff[i] : vz;
      dma16s(kbase, v, kb + 1024u * ins);
      dma16s(vbase, v, vb + 1024u * ins);
    }
  }
};
// Buffers per ring: 4 (three slices in flight) for 4-wave workgroups; with
// fewer waves a workgroup has less work per slice, and 64 KB of LDS would cap
// a CU at two of them, so they use 2 (one slice in flight, 32 KB).
__host__ __device__ constexpr int ring_buffers(int waves) { return waves >= 4 ? 4 : 2; }

// Make the compiler complete the loads of x here: a use it cannot see through.
// Called on values loaded before the first copy, so that its waits for them
// are not left inside the stage loop (where, loads completing in order, they
// would wait for every copy in flight).
template <class T>
__device__ __forceinline__ void settle(const T& x) {
  asm volatile("" : : "v"(x));
}

// The KV-slice walk of a Q block over its list of selected KV blocks, with
// the list read from an LDS copy (kListChunk entries at a time): the stage
// loop then issues no vector loads of its own.  Every thread walks the same
// list, so the refill branch is uniform over the workgroup.
constexpr int kListChunk = 1024;
struct LdsListWalk {
  int e, cnt, k, kend, base;
  const int32_t* lst;
  int* sl;  // kListChunk entries in LDS: lst[base .. base + kListChunk)

  __device__ __forceinline__ void fill(int from, int tid, int nthr) {
    __syncthreads();  // everyone is done reading the previous chunk
    base = from;
    for (int i = tid; i < kListChunk && from + i < cnt; i += nthr) sl[i] = lst[from + i];
    __syncthreads();
  }
  __device__ __forceinline__ bool next(const Params& p, int len_kv, Slice& s, int tid, int nthr) {
    while (k >= kend) {
      if (++e >= cnt) return false;
      if (e >= base + kListChunk) fill(e, tid, nthr);
      k = sl[e - base] * p.by;
      kend = min(k + p.by, len_kv);
    }
    s.head = 0;
    s.row0 = k;
    s.nrows = min(32, kend - k);
    k += 32;
    return true;
  }
};

// ---------------------------------------------------------------------------
// dK / dV: KV-block-outer
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// dK / dV: KV-block-outer
// ---------------------------------------------------------------------------
// Walk state over (query head n of the group, position e in its list of
// Q blocks selecting this KV block, first row q0 of the stage in that block).
struct QTile {
  int n, e, q0, qend;
};

// Move (t.n, t.e) to entry t.e of the group's merged list (head t.n's entries,
// then the next head's, ...), i.e. past the heads whose lists it overruns.
__device__ __forceinline__ bool dkdv_seek(const Params& p, int64_t bn0, int jb, int n_end, int len_q, QTile& t) {
  while (t.n < n_end) {
    const int64_t col = (bn0 + t.n) * p.nkb + jb;
    const int cnt = p.col_cnt[col];
    if (t.e < cnt) {
      const int ib = p.col_list[col * p.nqb + t.e];
      t.q0 = ib * p.bx;
      t.qend = min(t.q0 + p.bx, len_q);
      return true;
    }
    t.e -= cnt;
    ++t.n;
  }
  return false;
}

// What one dK/dV workgroup accumulates: both gradients (four GEMMs per step),
// or, where K, V and both accumulators would not fit in registers (D = 256),
// one of them per workgroup, each work item running twice: the dV pass needs
// S, P and dV += P^T dO, the dK pass S, dP, dS and dK += dS^T Q.
enum DkdvMode { kDkdvBoth = 0, kDkdvOnlyV = 1, kDkdvOnlyK = 2 };
// Q rows per staged tile: 32 per wave (16 at D = 256, so that two buffers of
// Q and dOut fit in LDS), and at least one 32-row slice.
template <int D, int W>
__host__ __device__ constexpr int dkdv_tile_rows() {
  return (D >= 256 ? 16 : 32) * W < 32 ? 32 : (D >= 256 ? 16 : 32) * W;
}

// attenMask words staged with a Q tile: for each of the workgroup's KV
// columns, the 32-query words covering the tile's rows (one more than H / 32,
// as the tile need not start on a word boundary).
template <int D, int W>
__host__ __device__ constexpr int dkdv_mask_words() { return dkdv_tile_rows<D, W>() / 32 + 1; }

// Epilogue of a dK/dV work item: the fp32 partial of a piece of a split unit,
// or the scaled, rounded rows of a whole unit (every row up to w_end, zeros
// where nothing contributed; rows from kv_end on are stored as zeros whatever
// their accumulators hold).
template <class E, int D, int W, int MODE>
__device__ __forceinline__ void dkdv_store(const Params& p, int u, int piece, int pieces, int kv0, int kv_end, int w_end, int b,
                                           int h, const SeqInfo& si, const f32x16 (&adv)[MODE != kDkdvOnlyK ? D / 32 : 1],
                                           const f32x16 (&adk)[MODE != kDkdvOnlyV ? D / 32 : 1]) {
  constexpr int NT = D / 32;
  constexpr bool kDoV = MODE != kDkdvOnlyK, kDoK = MODE != kDkdvOnlyV;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, l32 = lane & 31, g = lane >> 5;
  const PlanView pv(p);
  const int32_t* unit_base = pv.unit_base;
  if (pieces > 1) {  // fp32 partial of this piece; the reduction applies the output factors
    float* dst = p.partial + static_cast<int64_t>(unit_base[u] + piece) * 2 * kTileRowsMax * D;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int rl = 32 * w + 8 * (i >> 2) + 4 * g + (i & 3);
        if (kv0 + rl < w_end) {
          const bool live = kv0 + rl < kv_end;
          if constexpr (kDoK) dst[rl * D + 32 * nt + l32] = live ? adk[nt][i] : 0.f;
          if constexpr (kDoV) dst[(kTileRowsMax + rl) * D + 32 * nt + l32] = live ? adv[nt][i] : 0.f;
        }
      }
    }
    return;
  }
  unsigned short* dkp = static_cast<unsigned short*>(p.dk) + b * p.dk_sb + si.off_kv * p.dk_sr + h * p.dk_sh;
  unsigned short* dvp = static_cast<unsigned short*>(p.dv) + b * p.dv_sb + si.off_kv * p.dv_sr + h * p.dv_sh;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = kv0 + 32 * w + 8 * (i >> 2) + 4 * g + (i & 3);
      if (r < w_end) {
        const bool live = r < kv_end;
        if constexpr (kDoK) dkp[r * p.dk_sr + 32 * nt + l32] = E::from_f32(live ? adk[nt][i] * p.dk_scale : 0.f);
        if constexpr (kDoV) dvp[r * p.dv_sr + 32 * nt + l32] = E::from_f32(live ? adv[nt][i] * p.dv_scale : 0.f);
      }
    }
  }
}

// The same epilogue for transposed accumulators (dV^T / dK^T tiles: lane l
// holds key row 32 w + l % 32, register i of column tile nt holds element
// 32 nt + 8 (i / 4) + 4 g + i % 4): four consecutive elements per store.
template <class E, int D>
__device__ __forceinline__ void dkdv_store_t(const Params& p, int u, int piece, int pieces, int kv0, int kv_end,
                                             int w_end, int b, int h, const SeqInfo& si, const f32x16 (&adv)[D / 32],
                                             const f32x16 (&adk)[D / 32]) {
  constexpr int NT = D / 32;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, l32 = lane & 31, g = lane >> 5;
  const int rl = 32 * w + l32;  // this lane's key row within the part
  if (kv0 + rl >= w_end) return;
  const bool live = kv0 + rl < kv_end;
  if (pieces > 1) {  // fp32 partial of this piece; the reduction applies the output factors
    const PlanView pv(p);
    float* dst = p.partial + static_cast<int64_t>(pv.unit_base[u] + piece) * 2 * kTileRowsMax * D;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int c = 32 * nt + 8 * a + 4 * g;
        float4 vk, vv;
        vk.x = live ? adk[nt][4 * a] : 0.f, vk.y = live ? adk[nt][4 * a + 1] : 0.f;
        vk.z = live ? adk[nt][4 * a + 2] : 0.f, vk.w = live ? adk[nt][4 * a + 3] : 0.f;
        vv.x = live ? adv[nt][4 * a] : 0.f, vv.y = live ? adv[nt][4 * a + 1] : 0.f;
        vv.z = live ? adv[nt][4 * a + 2] : 0.f, vv.w = live ? adv[nt][4 * a + 3] : 0.f;
        *reinterpret_cast<float4*>(dst + rl * D + c) = vk;
        *reinterpret_cast<float4*>(dst + (kTileRowsMax + rl) * D + c) = vv;
      }
    return;
  }
  const int r = kv0 + rl;
  unsigned short* dkp = static_cast<unsigned short*>(p.dk) + b * p.dk_sb + (si.off_kv + r) * p.dk_sr + h * p.dk_sh;
  unsigned short* dvp = static_cast<unsigned short*>(p.dv) + b * p.dv_sb + (si.off_kv + r) * p.dv_sr + h * p.dv_sh;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int c = 32 * nt + 8 * a + 4 * g;
      float k4[4], v4[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        k4[t] = live ? adk[nt][4 * a + t] * p.dk_scale : 0.f;
        v4[t] = live ? adv[nt][4 * a + t] * p.dv_scale : 0.f;
      }
      store4<E>(dkp + c, k4);
      store4<E>(dvp + c, v4);
    }
}

template <class E, int D, int W, int MODE, bool AM>
__device__ __forceinline__ void dkdv_work(const Params& p, int item, unsigned short (*sQ)[dkdv_tile_rows<D, W>() * D],
                                          unsigned short (*sO)[dkdv_tile_rows<D, W>() * D],
                                          float (*sL)[dkdv_tile_rows<D, W>()], float (*sDl)[dkdv_tile_rows<D, W>()],
                                          uint32_t (*sB)[AM ? dkdv_mask_words<D, W>() : 1][32 * W]) {
  constexpr int KS = D / 16;  // K=16 steps over the head dim
  constexpr int NT = D / 32;  // 32-wide column tiles of the head dim
  constexpr int H = dkdv_tile_rows<D, W>();
  constexpr int RW = H / W;   // rows copied per wave
  constexpr bool kDoV = MODE != kDkdvOnlyK, kDoK = MODE != kDkdvOnlyV;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, l32 = lane & 31, g = lane >> 5;

  // Work item `item` of the plan's launch order: piece `piece` of unit u
  // (the whole unit unless it is split).
  const PlanView pv(p);
  if (item >= p.plan[1]) return;
  const int u = pv.order_unit[item];
  const int piece = pv.order_piece[item];
  const int32_t* unit_k = pv.unit_k;
  const int32_t* unit_base = pv.unit_base;
  const int pieces = unit_k[u];
  const int chunk = p.plan[0];

  int wid = u;
  const int nsub = (p.by + kTileRows - 1) / kTileRows;
  const int sub = wid % nsub;
  wid /= nsub;
  const int jb = wid % p.nkb;
  wid /= p.nkb;
  const int h = wid % p.Nkv;
  const int b = wid / p.Nkv;
  const SeqInfo si = p.seq[b];
  const int kv0 = jb * p.by + sub * kTileRows;
  const int part_end = min(jb * p.by + p.by, kv0 + kTileRows);
  const int kv_end = min(part_end, si.len_kv);  // rows that take part
  const int w_end = min(part_end, si.wlim_kv);  // rows this workgroup writes
  if (kv0 >= w_end) return;                     // uniform over the workgroup

  const int my_kv = kv0 + 32 * w + l32;  // B-operand column == score column of this lane
  const bool kv_ok = my_kv < kv_end;
  const int64_t kv_base = b * p.kv_sb + si.off_kv * p.kv_sr + h * p.kv_sh;
  const unsigned short* kp = static_cast<const unsigned short*>(p.k) + kv_base;
  const unsigned short* vp = static_cast<const unsigned short*>(p.v) + kv_base;

  u16x8 kreg[KS], vreg[kDoK ? KS : 1];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    u16x8 zk = {0, 0, 0, 0, 0, 0, 0, 0};
    u16x8 zv = zk;
    if (kv_ok) {
      zk = *reinterpret_cast<const u16x8*>(kp + my_kv * p.kv_sr + 16 * s + 8 * g);
      if constexpr (kDoK) zv = *reinterpret_cast<const u16x8*>(vp + my_kv * p.kv_sr + 16 * s + 8 * g);
    }
    kreg[s] = zk;
    if constexpr (kDoK) vreg[s] = zv;
  }

  f32x16 adv[kDoV ? NT : 1], adk[kDoK ? NT : 1];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if constexpr (kDoV) adv[nt] = f32x16{};
    if constexpr (kDoK) adk[nt] = f32x16{};
  }

  const float c2 = p.scale_log2e;
  const int64_t bn0 = static_cast<int64_t>(b) * p.N;
  const int n_end = (h + 1) * p.G;
  const unsigned short* qbase = static_cast<const unsigned short*>(p.q) + b * p.q_sb + si.off_q * p.q_sr;
  const unsigned short* obase = static_cast<const unsigned short*>(p.dout) + b * p.q_sb + si.off_q * p.q_sr;

  // DMA of one tile into buffer `buf`: wave w copies rows RW w .. RW w + RW - 1
  // of Q and dOut (one 1 KB wave instruction per 512 / D rows, lanes fetching
  // the swizzled chunk they land on, at a byte offset from the tile's first
  // row that is the same for every tile) and their LSE / softmax_grad values.
  // Lanes of rows past the tile's valid rows fetch a chunk of its first row
  // (finite data) and those rows get LSE = +inf and softmax_grad = 0, so their
  // P and dS are exactly 0 with no per-element test.
  constexpr int RPI = 512 / D;
  constexpr int NCP = RW / RPI;  // copies per wave and tensor
  const int lrow = lane / (D / 8);
  const unsigned vz = 16u * static_cast<unsigned>(lane % (D / 8));
  unsigned voff[NCP];
#pragma unroll
  for (int i = 0; i < NCP; ++i) {
    const int r = (w * NCP + i) * RPI + lrow;
    const int c = (lane % (D / 8)) ^ swz<D>(r);
    voff[i] = static_cast<unsigned>(2 * (r * p.q_sr + 8 * c));
  }
  auto issue = [&](const QTile& t, int buf) {
    const int rows = min(H, t.qend - t.q0);
    const int64_t first = static_cast<int64_t>(t.q0) * p.q_sr + t.n * p.q_sh;
    const unsigned short* qa = qbase + first;
    const unsigned short* oa = obase + first;
    const unsigned qb = lds_addr(sQ[buf]), ob = lds_addr(sO[buf]);
#pragma unroll
    for (int i = 0; i < NCP; ++i) {
      const int ins = w * NCP + i;
      const unsigned v = ins * RPI + lrow < rows ? voff[i] : vz;
      dma16s(qa, v, qb + 1024u * ins);
      dma16s(oa, v, ob + 1024u * ins);
    }
    if (lane < RW) {
      const int r = RW * w + lane;
      const int64_t li = (bn0 + t.n) * p.sq_max + t.q0 + r;
      dma4(r < rows ? static_cast<const void*>(p.lse2 + li) : p.consts + kConstPosInf, lds_addr(&sL[buf][RW * w]));
      dma4(r < rows ? static_cast<const void*>(p.delta + li) : p.consts, lds_addr(&sDl[buf][RW * w]));
    }
    if constexpr (AM) {  // attenMask bits of this wave's 32 KV columns over the tile's rows
      if (lane < 32) {
        const int wb = t.q0 >> 5;
#pragma unroll
        for (int m = 0; m < dkdv_mask_words<D, W>(); ++m) {
          const bool ok = my_kv < kv_end && wb + m < p.am_wq;
          dma4(ok ? static_cast<const void*>(p.am_cols + static_cast<int64_t>(my_kv) * p.am_wq + wb + m) : p.consts,
               lds_addr(&sB[buf][m][32 * w]));
        }
      }
    }
  };
#pragma unroll
  for (int s = 0; s < KS; ++s) {  // complete the K/V loads before the first copy
    settle(kreg[s]);
    if constexpr (kDoK) settle(vreg[s]);
  }

  // entries [piece * chunk, piece * chunk + chunk) of the merged list, or all of them
  int left = pieces > 1 ? chunk : 0x7fffffff;
  QTile cur{h * p.G, pieces > 1 ? piece * chunk : 0, 0, 0};
  bool have = dkdv_seek(p, bn0, jb, n_end, si.len_q, cur);
  if (have) issue(cur, 0);
  wait_vmcnt<0>();
  __syncthreads();
  for (int buf = 0; have; buf ^= 1) {
    const int rows = min(H, cur.qend - cur.q0);
    QTile nxt = cur;
    nxt.q0 += H;
    bool more = nxt.q0 < nxt.qend;
    if (!more && --left > 0) {
      ++nxt.e;
      more = dkdv_seek(p, bn0, jb, n_end, si.len_q, nxt);
    }
    if (more) issue(nxt, buf ^ 1);  // the other buffer: everyone finished with it at the last barrier
    const unsigned short* tQ = sQ[buf];
    const unsigned short* tO = sO[buf];
    const float* tL = sL[buf];
    const float* tD = sDl[buf];

    for (int c0 = 0; c0 < rows; c0 += 32) {
      f32x16 s = {}, dpv = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u16x8 aq = frag_along_row<D>(tQ, c0, 16 * ks, lane);
        s = E::mma(aq, kreg[ks], s);  // S[q][kv] (unscaled); this lane's column is my_kv
        if constexpr (kDoK) {
          const u16x8 ao = frag_along_row<D>(tO, c0, 16 * ks, lane);
          dpv = E::mma(ao, vreg[ks], dpv);  // dP[q][kv] = dOut * V^T
        }
      }
      // this lane's 16 score rows are c0 + 8a + 4g + {0..3}: four float4 reads each
      float4 l4[4], d4[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        l4[a] = *reinterpret_cast<const float4*>(tL + c0 + 8 * a + 4 * g);
        d4[a] = *reinterpret_cast<const float4*>(tD + c0 + 8 * a + 4 * g);
      }
      float pv[16], dsv[16];
      if (!AM && rect_in_band(p, cur.q0 + c0, 32, kv0 + 32 * w, 32)) {  // uniform: no mask cuts anything here
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float li = l4[i >> 2][i & 3], di = d4[i >> 2][i & 3];
          const float x = fast_exp2(s[i] * c2 - li);  // P = exp(scale*S - LSE)
          pv[i] = kv_ok ? x : 0.f;
          dsv[i] = pv[i] * (dpv[i] + di);              // dS = P o (dP - softmax_grad); di = -softmax_grad
        }
      } else {
        // attenMask bits of this lane's 32 query rows (bit r: row cur.q0 + c0 + r excluded)
        uint32_t ex = 0;
        if constexpr (AM) {
          const int qs = cur.q0 + c0, m0 = (qs >> 5) - (cur.q0 >> 5);
          const uint64_t two = (static_cast<uint64_t>(sB[buf][m0 + 1][32 * w + l32]) << 32) | sB[buf][m0][32 * w + l32];
          ex = static_cast<uint32_t>(two >> (qs & 31));
        }
        // bit r of keep: slice row r takes part (this lane's key valid, row in
        // range, in the window, not excluded); shifted so that register i
        // tests bit 8 (i / 4) + i % 4, its row minus 4g
        const int qs = cur.q0 + c0;
        const int nv = cur.qend - qs;  // >= 1
        const uint32_t rows_ok = nv >= 32 ? 0xffffffffu : ((1u << nv) - 1u);
        const uint32_t keep = (kv_ok ? rows_ok & ~ex & band_rows(p, qs, my_kv) : 0u) >> (4 * g);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float li = l4[i >> 2][i & 3], di = d4[i >> 2][i & 3];
          const float x = fast_exp2(s[i] * c2 - li);
          pv[i] = ((keep >> (8 * (i >> 2) + (i & 3))) & 1u) ? x : 0.f;  // a select: li may be -inf
          dsv[i] = pv[i] * (dpv[i] + di);
        }
      }
      const u16x8 pa[2] = {pack8<E>(pv), pack8<E>(pv + 8)};
      const u16x8 da[2] = {pack8<E>(dsv), pack8<E>(dsv + 8)};
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          if constexpr (kDoV) {
            const u16x8 bo = frag_down_rows<D>(tO, c0 + 16 * hh, 32 * nt, lane);
            adv[nt] = E::mma(pa[hh], bo, adv[nt]);  // dV += P^T * dOut
          }
          if constexpr (kDoK) {
            const u16x8 bq = frag_down_rows<D>(tQ, c0 + 16 * hh, 32 * nt, lane);
            adk[nt] = E::mma(da[hh], bq, adk[nt]);  // dK += dS^T * Q
          }
        }
      }
    }
    wait_vmcnt<0>();  // this wave's copies of the next tile
    __syncthreads();  // everyone's copies landed; everyone is done with this tile
    cur = nxt;
    have = more;
  }

  dkdv_store<E, D, W, MODE>(p, u, piece, pieces, kv0, w_end, w_end, b, h, si, adv, adk);
}

// ---------------------------------------------------------------------------
// dK / dV, scheduled build (fp16/bf16, head dim 64 or 128, no attenMask)
// ---------------------------------------------------------------------------
// The same work as dkdv_work in kDkdvBoth mode, laid out for one wave per
// SIMD so that the matrix cores stay busy.  A wave keeps issuing VALU and LDS
// instructions while its MFMAs execute, but issues in order: a VALU that waits
// for an MFMA result also holds back every MFMA behind it.  So the slices of a
// tile (NSL slices of 32 Q rows, unrolled) are software-pipelined: while the
// softmax of slice i runs on the VALU, the matrix cores compute slice i + 1's
// scores, and every VALU instruction reads results of the phase before:
//   P    S(0) = Q_0 K^T, dP(0) = dO_0 V^T - softmax_grad             16 MFMA
//   X(i) S(i+1), dP(i+1)                                              16 MFMA
//        || P = exp2(S(i) c - lse2), dS = P o dP(i), rounded pairs     VALU
//        || dO^T, Q^T fragments of slice i                             LDS
//   Y(i) dV += P^T dO_i, dK += dS^T Q_i                                16 MFMA
//        || Q, dO fragments of slice i + 2, LSE / softmax_grad rows    LDS
// dP's accumulator starts at -softmax_grad (the prologue stores it negated).
// Every LDS fragment comes from a per-lane byte address computed once per
// work item plus an immediate offset (slice, half, tensor), so the tile does
// no address arithmetic.  Rows past a tile's valid rows hold finite data with
// LSE = +inf and softmax_grad = 0: their P and dS are exactly 0, so whole
// tiles of NSL slices are computed without guards (NSL follows the block
// height).  Keys past the sequence end hold zero K/V rows; their P and dS are
// left unmasked, as they feed only that lane's own dK/dV rows, which the
// epilogue stores as zeros.  With a sliding window the pairs outside it get
// P = 0 by a bit mask (lse2 may be -inf there).
template <int D, int W, int NSL>
struct DkdvPipe {
  static constexpr int KS = D / 16, NT = D / 32;
  static constexpr int H = 32 * NSL;          // rows per tile
  static constexpr int RW = H / W;            // rows each wave copies per tile
  static constexpr unsigned TB = 2u * H * D;  // bytes of one tile tensor (Q or dO)
  static constexpr unsigned BUF = 2u * TB;    // bytes of one buffer: Q tile, then dO tile
  static_assert(D <= 128, "head dim 256 takes the two-pass build");
  static_assert(TB + 2u * (H - 16) * D <= 65535u, "immediate LDS offsets");
};
// slices per tile for a block height of bx rows with W waves: up to 4 (the
// whole 128-row part), and at most W so that 4 / W workgroups (one wave per
// SIMD) fit the CU's LDS at head dim 128
__host__ __device__ constexpr int dkdv_pipe_nsl(int bx, int W) {
  const int want = bx <= 32 ? 1 : bx <= 64 ? 2 : 4;
  return want < W ? want : W;
}

typedef __attribute__((address_space(3))) u16x8 lds_u16x8;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
__device__ __forceinline__ u16x8 lds_b128(unsigned addr) { return *(const lds_u16x8*)(static_cast<uintptr_t>(addr)); }
__device__ __forceinline__ f32x4 lds_f4(unsigned addr) { return *(const lds_f32x4*)(static_cast<uintptr_t>(addr)); }
__device__ __forceinline__ u16x4 lds_tr(unsigned addr) {
  return __builtin_bit_cast(u16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(static_cast<uintptr_t>(addr))));
}
__device__ __forceinline__ u16x8 cat8(u16x4 a, u16x4 b) { return u16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]}; }

// scheduling group masks (sched_group_barrier)
constexpr int kSgMfma = 0x008, kSgValu = 0x002, kSgDsRead = 0x100;

// Per-lane LDS byte addresses of a work item's fragments in buffer 0.
template <int D, int W, int NSL>
struct DkdvAddr {
  using T = DkdvPipe<D, W, NSL>;
  unsigned a[T::KS];      // along-row fragment ks of the Q tile (+TB: dO)
  unsigned b[T::NT][2];   // down-rows fragment nt, upper/lower 8 rows, of the Q tile (+TB: dO)
  unsigned l;             // this lane's LSE*log2e row quadruple (+4H: -softmax_grad)
};

// The fragments and row values one slice needs.
template <int D>
struct DkdvSliceIn {
  u16x8 aq[D / 16], ao[D / 16];  // Q, dO along rows (MFMA A operands of S, dP)
  f32x4 d4[4];                   // -softmax_grad of the lane's 16 rows (dP's initial accumulator)
  f32x4 l4[4];                   // LSE*log2e of the lane's 16 rows
};

template <int D, int W, int NSL>
__device__ __forceinline__ void dkdv_read_a(const DkdvAddr<D, W, NSL>& ad, int sl, DkdvSliceIn<D>& in) {
  using T = DkdvPipe<D, W, NSL>;
  const unsigned cb = 2u * 32 * sl * D;
#pragma unroll
  for (int ks = 0; ks < T::KS; ++ks) {
    in.aq[ks] = lds_b128(ad.a[ks] + cb);
    in.ao[ks] = lds_b128(ad.a[ks] + T::TB + cb);
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    in.d4[a] = lds_f4(ad.l + 4u * T::H + 128u * sl + 32u * a);
    in.l4[a] = lds_f4(ad.l + 128u * sl + 32u * a);
  }
}

template <class E, int D>
__device__ __forceinline__ void dkdv_sdp(const DkdvSliceIn<D>& in, const u16x8 (&kreg)[D / 16],
                                         const u16x8 (&vreg)[D / 16], f32x16& s, f32x16& dp) {
  s = f32x16{};
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int t = 0; t < 4; ++t) dp[4 * a + t] = in.d4[a][t];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    s = E::mma(in.aq[ks], kreg[ks], s);    // S[q][kv] (unscaled); this lane's column is its key
    dp = E::mma(in.ao[ks], vreg[ks], dp);  // dP[q][kv] - softmax_grad[q]
  }
}

template <class E, int D, int W, int NSL, bool WIN>
__device__ __forceinline__ void dkdv_pipe_tile(const DkdvAddr<D, W, NSL>& ad, const u16x8 (&kreg)[D / 16],
                                               const u16x8 (&vreg)[D / 16], f32x16 (&adv)[D / 32],
                                               f32x16 (&adk)[D / 32], float c2, const uint32_t (&keep)[NSL]) {
  using T = DkdvPipe<D, W, NSL>;
  constexpr int KS = T::KS, NT = T::NT;
  constexpr unsigned TB = T::TB;
  DkdvSliceIn<D> in[2];
  f32x16 s[2], dp[2];
  // P: slice 0's S and dP; loads slice 1's fragments
  dkdv_read_a<D, W, NSL>(ad, 0, in[0]);
  dkdv_sdp<E, D>(in[0], kreg, vreg, s[0], dp[0]);
  if constexpr (NSL > 1) {
    dkdv_read_a<D, W, NSL>(ad, 1, in[1]);
    __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2 * KS + 8, 0);  // slice 0's reads first
#pragma unroll
    for (int k = 0; k < 2 * KS; ++k) {
      __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSgDsRead, (2 * KS + 8 + 2 * KS - 1) / (2 * KS), 0);
    }
  }
#pragma unroll
  for (int sl = 0; sl < NSL; ++sl) {
    const int cur = sl & 1, nxt = cur ^ 1;
    const unsigned cb = 2u * 32 * sl * D;
    // ---- X(sl): slice sl + 1's S / dP on the matrix cores, slice sl's softmax on the VALU
    const f32x4(&l4)[4] = in[cur].l4;
    if (sl + 1 < NSL) dkdv_sdp<E, D>(in[nxt], kreg, vreg, s[nxt], dp[nxt]);
    float pv[16], dsv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float x = fast_exp2(s[cur][i] * c2 - l4[i >> 2][i & 3]);  // P = exp(scale*S - LSE)
      if constexpr (WIN)
        pv[i] = __uint_as_float(__float_as_uint(x) & (0u - ((keep[sl] >> (8 * (i >> 2) + (i & 3))) & 1u)));
      else pv[i] = x;
      dsv[i] = pv[i] * dp[cur][i];  // dS = P o (dP - softmax_grad)
    }
    const u16x8 pa[2] = {pack8<E>(pv), pack8<E>(pv + 8)};
    const u16x8 da[2] = {pack8<E>(dsv), pack8<E>(dsv + 8)};
    u16x4 bo[2][NT][2], bq[2][NT][2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          bo[hh][nt][h2] = lds_tr(ad.b[nt][h2] + TB + cb + 2u * 16 * hh * D);
          bq[hh][nt][h2] = lds_tr(ad.b[nt][h2] + cb + 2u * 16 * hh * D);
        }
    if (sl + 1 < NSL) {
#pragma unroll
      for (int k = 0; k < 2 * KS; ++k) {
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, (8 * NT + 2 * KS - 1) / (2 * KS), 0);
        __builtin_amdgcn_sched_group_barrier(kSgValu, (WIN ? 128 : 96) / (2 * KS), 0);
      }
    }
    // ---- Y(sl): dV^T += dO^T P, dK^T += Q^T dS; loads slice sl + 2's fragments.
    // The fragment read down dO's (Q's) rows is, as an A operand, dO^T with
    // the same k order as P's (dS's) registers, which serve as the B operand:
    // the accumulators hold dV^T / dK^T, one key row per lane, so the
    // epilogue stores four consecutive elements at a time.
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) adv[nt] = E::mma(cat8(bo[hh][nt][0], bo[hh][nt][1]), pa[hh], adv[nt]);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) adk[nt] = E::mma(cat8(bq[hh][nt][0], bq[hh][nt][1]), da[hh], adk[nt]);
    if (sl + 2 < NSL) dkdv_read_a<D, W, NSL>(ad, sl + 2, in[cur]);
#pragma unroll
    for (int k = 0; k < 4 * NT; ++k) {
      __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
      if (sl + 2 < NSL) __builtin_amdgcn_sched_group_barrier(kSgDsRead, (2 * KS + 8 + 4 * NT - 1) / (4 * NT), 0);
    }
  }
}

// A dK/dV work item's share of the merged list (the group's query heads in
// order, each with its ascending list of Q blocks selecting the item's KV
// block) is copied into LDS once, with every load in flight together, so that
// finding the next tile is an LDS read.  Entry j holds (query head - first head
// of the group, Q block).  Holds up to kDkdvListChunk entries at a time; longer
// items refill it between tiles.
constexpr int kDkdvListChunk = 1024;
constexpr int kDkdvMaxGroup = 256;  // heads per KV head (the counts sit in LDS too)
struct DkdvList {
  int* ib;             // [kDkdvListChunk]
  unsigned short* n;   // [kDkdvListChunk]
  int* cnt;            // [kDkdvMaxGroup] list length of each head of the group
  int first, count;    // the item's entries [first, first + count) of the merged list
  int base;            // merged-list index of ib[0]
};

// Fill the LDS list from merged-list entry `from` (relative to the item's
// first entry); every thread of the workgroup takes part.
__device__ __forceinline__ void dkdv_list_fill(const Params& p, int64_t col0, int jb, DkdvList& l, int from) {
  __syncthreads();  // everyone is done with the previous contents
  const int nf = min(kDkdvListChunk, l.count - from);
  for (int j = threadIdx.x; j < nf; j += blockDim.x) {
    int e = l.first + from + j, n = 0;
    while (e >= l.cnt[n]) e -= l.cnt[n++];
    l.ib[j] = p.col_list[((col0 + n) * p.nkb + jb) * static_cast<int64_t>(p.nqb) + e];
    l.n[j] = static_cast<unsigned short>(n);
  }
  l.base = from;
  __syncthreads();
}

// Persistent: a grid of as many workgroups as fit the GPU at once, each taking
// work items from the plan's launch order (longest first) through a counter
// in the plan region, which the plan kernel zeroes.  When an item's tiles are
// done, the workgroup first starts the next item (its list, its first tile's
// copies, its K and V rows) and only then issues the finished item's stores,
// so those loads fly while the stores are issued.  Which workgroup runs an
// item does not change the item's result.
// Epilogue of a whole unit through LDS: every lane writes its key row's dK (then
// dV) into `stage` (transposed accumulators: 4 consecutive elements per
// 8-byte write; rows of D elements with their 16-byte chunks XOR-permuted by
// the row's low bits (as many as index a row's chunks), so the rows of one
// write spread over the banks),
// then every 16-byte store of a wave covers 1 KB of consecutive rows.  STAGE
// is the stage's size in bytes: both tensors at once when they fit, else one
// after the other.  Rows from kv_end on are stored as zeros.  The caller syncs
// the workgroup before the stage is reused.  Falls back to dkdv_store_t when an
// output row is not 16-byte aligned, for a piece of a split unit, or when
// one tensor's rows do not fit the stage.
template <class E, int D, int W, unsigned STAGE>
__device__ __forceinline__ void dkdv_store_staged(const Params& p, int u, int piece, int pieces, int kv0, int kv_end,
                                                  int w_end, int b, int h, const SeqInfo& si,
                                                  const f32x16 (&adv)[D / 32], const f32x16 (&adk)[D / 32],
                                                  unsigned stage) {
  constexpr int NT = D / 32, CPR = D / 8;  // 16-byte chunks per row (a power of two)
  constexpr int RT = 32 * W;               // rows of one tensor
  static_assert((CPR & (CPR - 1)) == 0, "chunk permutation");
  constexpr unsigned TBYTES = 2u * RT * D;
  unsigned short* dkp = static_cast<unsigned short*>(p.dk) + b * p.dk_sb + si.off_kv * p.dk_sr + h * p.dk_sh;
  unsigned short* dvp = static_cast<unsigned short*>(p.dv) + b * p.dv_sb + si.off_kv * p.dv_sr + h * p.dv_sh;
  const bool aligned = ((reinterpret_cast<uintptr_t>(dkp) | reinterpret_cast<uintptr_t>(dvp)) & 15u) == 0 &&
                       ((p.dk_sr | p.dv_sr) & 7) == 0;
  if (TBYTES > STAGE || pieces > 1 || !aligned) {  // uniform
    dkdv_store_t<E, D>(p, u, piece, pieces, kv0, kv_end, w_end, b, h, si, adv, adk);
    return;
  }
  constexpr int NPASS = 2 * TBYTES <= STAGE ? 1 : 2;  // tensors per pass: 2 / NPASS
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, l32 = lane & 31, g = lane >> 5;
  const int rl = 32 * w + l32;
  const bool live = kv0 + rl < kv_end;
  const int rows = min(w_end - kv0, RT);
  typedef __attribute__((address_space(3))) u16x4 lds_u16x4;
#pragma unroll
  for (int pass = 0; pass < NPASS; ++pass) {
    if (pass) __syncthreads();  // the first tensor's rows are read out
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int chunk = (4 * nt + a) ^ (rl & (CPR - 1));
        const unsigned off = 2u * (rl * D + 8 * chunk + 4 * g);
        u16x4 kv4, vv4;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          kv4[t] = E::from_f32(live ? adk[nt][4 * a + t] * p.dk_scale : 0.f);
          vv4[t] = E::from_f32(live ? adv[nt][4 * a + t] * p.dv_scale : 0.f);
        }
        if (NPASS == 1) {
          *(lds_u16x4*)(static_cast<uintptr_t>(stage + off)) = kv4;
          *(lds_u16x4*)(static_cast<uintptr_t>(stage + TBYTES + off)) = vv4;
        } else {
          *(lds_u16x4*)(static_cast<uintptr_t>(stage + off)) = pass ? vv4 : kv4;
        }
      }
    __syncthreads();
    const int nten = 2 / NPASS;
    for (int i = tid; i < nten * rows * CPR; i += 64 * W) {  // (tensor, row, chunk), chunks fastest
      const int t = i / (rows * CPR), rem = i - t * rows * CPR;
      const int r = rem / CPR, c = rem - r * CPR;
      const u16x8 v = lds_b128(stage + t * TBYTES + 2u * (r * D + 8 * (c ^ (r & (CPR - 1)))));
      const bool is_k = NPASS == 1 ? t == 0 : pass == 0;
      unsigned short* dst = (is_k ? dkp + (kv0 + r) * p.dk_sr : dvp + (kv0 + r) * p.dv_sr) + 8 * c;
      *reinterpret_cast<u16x8*>(dst) = v;
    }
  }
}

template <class E, int D, int W, int NSL, bool WIN>
__global__ __launch_bounds__(64 * W) void dkdv_pipe_kernel(Params p) {
  using T = DkdvPipe<D, W, NSL>;
  constexpr int KS = T::KS, NT = T::NT, H = T::H, RW = T::RW;
  constexpr unsigned TB = T::TB, BUF = T::BUF;
  // Q / dO tiles of buffer b at byte 2 b TB (swizzled rows); per buffer the
  // LSE*log2e rows, then the -softmax_grad rows
  __shared__ __align__(1024) unsigned short sT[2 * 2 * H * D];
  __shared__ __align__(16) float sLD[2 * 2 * H];
  __shared__ int sListIb[kDkdvListChunk], sListCnt[kDkdvMaxGroup];
  __shared__ unsigned short sListN[kDkdvListChunk];
  __shared__ int sItem;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, l32 = lane & 31, g = lane >> 5;
  const PlanView pv(p);
  const int chunk = p.plan[0], n_items = p.plan[1];
  const int nsub = (p.by + kTileRows - 1) / kTileRows;
  const float c2 = p.scale_log2e;

  // one work item: piece `piece` of unit u (batch b, KV head h, KV rows [kv0, w_end))
  struct Item {
    int u, piece, pieces, kv0, kv_end, w_end, b, h, jb;
    SeqInfo si;
    int64_t bn0, col0;
  };
  auto grab = [&]() {  // the next item of the launch order, for the whole workgroup
    __syncthreads();   // everyone read the previous one
    if (tid == 0) sItem = atomicAdd(&p.plan[3], 1);
    __syncthreads();
    return sItem;
  };
  auto decode = [&](int item, Item& it) {  // false: the item writes nothing
    it.u = pv.order_unit[item];
    it.piece = pv.order_piece[item];
    it.pieces = pv.unit_k[it.u];
    int wid = it.u;
    const int sub = wid % nsub;
    wid /= nsub;
    it.jb = wid % p.nkb;
    wid /= p.nkb;
    it.h = wid % p.Nkv;
    it.b = wid / p.Nkv;
    it.si = p.seq[it.b];
    it.kv0 = it.jb * p.by + sub * kTileRows;
    const int part_end = min(it.jb * p.by + p.by, it.kv0 + kTileRows);
    it.kv_end = min(part_end, it.si.len_kv);
    it.w_end = min(part_end, it.si.wlim_kv);
    it.bn0 = static_cast<int64_t>(it.b) * p.N;
    it.col0 = it.bn0 + static_cast<int64_t>(it.h) * p.G;  // (b, first head of the group)
    return it.kv0 < it.w_end;
  };

  // DMA of one tile into buffer `buf` (as in dkdv_work): Q rows, dO rows and
  // their LSE*log2e / -softmax_grad values (+inf / 0 past the valid rows).
  constexpr int RPI = 512 / D;  // rows per 1 KB wave instruction
  constexpr int NCP = RW / RPI;
  static_assert(NCP >= 1 && NCP * RPI == RW, "a tile splits evenly over the waves' copies");
  const int lrow = lane / (D / 8);
  const unsigned vz = 16u * static_cast<unsigned>(lane % (D / 8));
  unsigned voff[NCP];
#pragma unroll
  for (int i = 0; i < NCP; ++i) {
    const int r = (w * NCP + i) * RPI + lrow;
    const int c = (lane % (D / 8)) ^ swz<D>(r);
    voff[i] = static_cast<unsigned>(2 * (r * p.q_sr + 8 * c));
  }
  const unsigned t0 = lds_addr(sT), l0 = lds_addr(sLD);
  auto issue = [&](const Item& it, const QTile& t, int buf) {
    const int rows = min(H, t.qend - t.q0);
    const int64_t first = (it.b * p.q_sb + it.si.off_q * p.q_sr) + static_cast<int64_t>(t.q0) * p.q_sr + t.n * p.q_sh;
    const unsigned short* qa = static_cast<const unsigned short*>(p.q) + first;
    const unsigned short* oa = static_cast<const unsigned short*>(p.dout) + first;
    const unsigned qb = t0 + BUF * buf, ob = qb + TB;
#pragma unroll
    for (int i = 0; i < NCP; ++i) {
      const int ins = w * NCP + i;
      const unsigned v = ins * RPI + lrow < rows ? voff[i] : vz;
      dma16s(qa, v, qb + 1024u * ins);
      dma16s(oa, v, ob + 1024u * ins);
    }
#pragma unroll
    for (int r0 = 0; r0 < RW; r0 += 64) {
      if (lane < RW - r0) {
        const int r = RW * w + r0 + lane;
        const int64_t li = (it.bn0 + t.n) * p.sq_max + t.q0 + r;
        const unsigned lb = l0 + 8u * H * buf + 4u * (RW * w + r0);
        dma4(r < rows ? static_cast<const void*>(p.lse2 + li) : p.consts + kConstPosInf, lb);
        dma4(r < rows ? static_cast<const void*>(p.delta + li) : p.consts, lb + 4u * H);
      }
    }
  };
  // the item's entries in LDS: counts of the group's heads, then the entries
  DkdvList lst{sListIb, sListN, sListCnt, 0, 0, 0};
  auto list_start = [&](const Item& it) {
    __syncthreads();  // everyone is done with the previous item's list
    for (int t = tid; t < p.G; t += 64 * W) lst.cnt[t] = p.col_cnt[(it.col0 + t) * p.nkb + it.jb];
    __syncthreads();
    int tot = 0;
    for (int t = 0; t < p.G; ++t) tot += lst.cnt[t];
    lst.first = it.pieces > 1 ? it.piece * chunk : 0;
    lst.count = it.pieces > 1 ? min(chunk, tot - lst.first) : tot;
    dkdv_list_fill(p, it.col0, it.jb, lst, 0);
  };
  // tile of list entry e (relative to the item), first rows of its Q block
  auto tile_of = [&](const Item& it, int e) {
    if (e - lst.base >= kDkdvListChunk) dkdv_list_fill(p, it.col0, it.jb, lst, e);  // uniform
    const int ib = lst.ib[e - lst.base];
    QTile t{it.h * p.G + lst.n[e - lst.base], e, ib * p.bx, 0};
    t.qend = min(t.q0 + p.bx, it.si.len_q);
    return t;
  };
  // K and V rows of the item (zero rows for keys past the sequence end; their
  // P and dS are not masked, as they feed only the lane's own dK/dV rows,
  // which the epilogue stores as zeros)
  u16x8 kreg[KS], vreg[KS];
  auto load_kv = [&](const Item& it) {
    const int64_t kv_base = it.b * p.kv_sb + it.si.off_kv * p.kv_sr + it.h * p.kv_sh;
    const unsigned short* kp = static_cast<const unsigned short*>(p.k) + kv_base;
    const unsigned short* vp = static_cast<const unsigned short*>(p.v) + kv_base;
    const int my_kv = it.kv0 + 32 * w + l32;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u16x8 zk = {0, 0, 0, 0, 0, 0, 0, 0};
      u16x8 zv = zk;
      if (my_kv < it.kv_end) {
        zk = *reinterpret_cast<const u16x8*>(kp + my_kv * p.kv_sr + 16 * s + 8 * g);
        zv = *reinterpret_cast<const u16x8*>(vp + my_kv * p.kv_sr + 16 * s + 8 * g);
      }
      kreg[s] = zk;
      vreg[s] = zv;
    }
  };
  // start an item: its list, its first tile's copies into buffer 0, its K/V rows
  auto start = [&](const Item& it, QTile& first) {
    list_start(it);
    if (lst.count > 0) {
      first = tile_of(it, 0);
      issue(it, first, 0);
    }
    load_kv(it);
  };

  Item cur_it{};
  int item = grab();
  while (item < n_items && !decode(item, cur_it)) item = grab();
  if (item >= n_items) return;  // uniform
  QTile cur{};
  start(cur_it, cur);
  f32x16 adv[NT], adk[NT];
  for (;;) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      adv[nt] = f32x16{};
      adk[nt] = f32x16{};
    }
    wait_vmcnt<0>();
#pragma unroll
    for (int s = 0; s < KS; ++s) {  // the K/V loads are complete: no waits for them in the tile loop
      settle(kreg[s]);
      settle(vreg[s]);
    }
    DkdvAddr<D, W, NSL> ad;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) ad.a[ks] = t0 + 2u * tile_off<D>(l32, 16 * ks + 8 * g);
    {
      const int rr = 4 * g + ((lane & 15) >> 2);
      const int col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        ad.b[nt][0] = t0 + 2u * tile_off<D>(rr, 32 * nt + col);
        ad.b[nt][1] = t0 + 2u * tile_off<D>(rr + 8, 32 * nt + col);
      }
    }
    ad.l = l0 + 16u * g;
    __syncthreads();  // the first tile landed for every wave
    const int my_kv = cur_it.kv0 + 32 * w + l32;
    bool have = lst.count > 0;
    for (int buf = 0; have; buf ^= 1) {
      QTile nxt = cur;
      nxt.q0 += H;
      bool more = nxt.q0 < nxt.qend;
      if (!more && cur.e + 1 < lst.count) {
        nxt = tile_of(cur_it, cur.e + 1);
        more = true;
      }
      if (more) issue(cur_it, nxt, buf ^ 1);  // the other buffer: everyone finished with it at the last barrier
      // with a window, bit r of keep[sl]: row r of slice sl is in it for this
      // lane's key, pre-shifted so that register i tests bit 8 (i / 4) + i % 4
      uint32_t keep[NSL];
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl) keep[sl] = WIN ? band_rows(p, cur.q0 + 32 * sl, my_kv) >> (4 * g) : 0u;
      dkdv_pipe_tile<E, D, W, NSL, WIN>(ad, kreg, vreg, adv, adk, c2, keep);
      wait_vmcnt<0>();  // this wave's copies of the next tile
      __syncthreads();  // everyone's copies landed; everyone is done with this tile
      const unsigned flip = buf ? 0u - BUF : BUF;  // the next tile sits in the other buffer
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) ad.a[ks] += flip;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        ad.b[nt][0] += flip;
        ad.b[nt][1] += flip;
      }
      ad.l += buf ? 0u - 8u * H : 8u * H;
      cur = nxt;
      have = more;
    }
    // the next item starts before this one's stores are issued
    Item nx_it{};
    int nitem = grab();
    bool next = false;
    while (nitem < n_items && !(next = decode(nitem, nx_it))) nitem = grab();
    QTile nx{};
    if (next) start(nx_it, nx);  // the next item's first tile goes to buffer 0; buffer 1 stages the stores
    dkdv_store_staged<E, D, W, BUF>(p, cur_it.u, cur_it.piece, cur_it.pieces, cur_it.kv0, cur_it.kv_end,
                                    cur_it.w_end, cur_it.b, cur_it.h, cur_it.si, adv, adk, t0 + BUF);
    if (!next) break;  // uniform
    cur_it = nx_it;
    cur = nx;
  }
}

// AM: built for calls with an attenMask (its bits staged with the Q tiles);
// the builds without one carry none of that code.
template <class E, int D, int W, bool AM>
__global__ __launch_bounds__(256) void dkdv_kernel(Params p) {
  constexpr int H = dkdv_tile_rows<D, W>();
  // Q and dOut tiles (swizzled layout) and their LSE*log2(e) / softmax_grad
  // rows, double-buffered: tile t + 1 is copied in by DMA during tile t
  __shared__ __align__(1024) unsigned short sQ[2][H * D];
  __shared__ __align__(1024) unsigned short sO[2][H * D];  // dOut rows
  __shared__ __align__(16) float sL[2][H];
  __shared__ __align__(16) float sDl[2][H];
  __shared__ __align__(16) uint32_t sB[2][AM ? dkdv_mask_words<D, W>() : 1][32 * W];  // attenMask bits
  if constexpr (dkdv_passes(D) == 1) {
    dkdv_work<E, D, W, kDkdvBoth, AM>(p, blockIdx.x, sQ, sO, sL, sDl, sB);
  } else {  // workgroups 2i and 2i + 1 run the dV and the dK pass of work item i
    if (blockIdx.x & 1) dkdv_work<E, D, W, kDkdvOnlyK, AM>(p, blockIdx.x >> 1, sQ, sO, sL, sDl, sB);
    else dkdv_work<E, D, W, kDkdvOnlyV, AM>(p, blockIdx.x >> 1, sQ, sO, sL, sDl, sB);
  }
}

// Sum the pieces of split dK/dV unit slot_unit[s] (for the slot holding its
// piece 0) in piece order, scale dK, round and store both.  Runs as extra
// workgroups of the dQ launch, which starts after the dK/dV kernel finished.
template <class E, int D>
__device__ void reduce_pieces(const Params& p, int s) {
  const PlanView pv(p);
  const int u = pv.slot_unit[s];
  if (u < 0 || pv.slot_chunk[s] != 0) return;
  const int pieces = pv.unit_k[u];
  const float* src = p.partial + static_cast<int64_t>(pv.unit_base[u]) * 2 * kTileRowsMax * D;
  int wid = u;
  const int nsub = (p.by + kTileRows - 1) / kTileRows;
  const int sub = wid % nsub;
  wid /= nsub;
  const int jb = wid % p.nkb;
  wid /= p.nkb;
  const int h = wid % p.Nkv;
  const int b = wid / p.Nkv;
  const SeqInfo si = p.seq[b];
  const int kv0 = jb * p.by + sub * kTileRows;
  const int w_end = min(min(jb * p.by + p.by, kv0 + kTileRows), si.wlim_kv);
  if (kv0 >= w_end) return;
  unsigned short* dkp = static_cast<unsigned short*>(p.dk) + b * p.dk_sb + si.off_kv * p.dk_sr + h * p.dk_sh;
  unsigned short* dvp = static_cast<unsigned short*>(p.dv) + b * p.dv_sb + si.off_kv * p.dv_sr + h * p.dv_sh;
  const int n4 = 2 * (w_end - kv0) * D / 4;  // float4 groups over [dK rows, dV rows]
  for (int q = threadIdx.x; q < n4; q += blockDim.x) {
    const int t = q / ((w_end - kv0) * D / 4);  // 0: dK, 1: dV
    const int rem = q % ((w_end - kv0) * D / 4);
    const int rl = rem / (D / 4), d = 4 * (rem % (D / 4));
    float4 acc = *reinterpret_cast<const float4*>(src + (t * kTileRowsMax + rl) * D + d);
    for (int c = 1; c < pieces; ++c) {
      const float4 x = *reinterpret_cast<const float4*>(src + (static_cast<int64_t>(c) * 2 * kTileRowsMax + t * kTileRowsMax + rl) * D + d);
      acc.x += x.x;
      acc.y += x.y;
      acc.z += x.z;
      acc.w += x.w;
    }
    const float sc = t == 0 ? p.dk_scale : p.dv_scale;
    unsigned short* dst = (t == 0 ? dkp + (kv0 + rl) * p.dk_sr : dvp + (kv0 + rl) * p.dv_sr) + d;
    dst[0] = E::from_f32(acc.x * sc);
    dst[1] = E::from_f32(acc.y * sc);
    dst[2] = E::from_f32(acc.z * sc);
    dst[3] = E::from_f32(acc.w * sc);
  }
}

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

  if (static_cast<int>(blockIdx.x) >= p.n_dq_units) {  // the workgroups after the dQ ones reduce split dK/dV units
    reduce_pieces<E, D>(p, blockIdx.x - p.n_dq_units);
    return;
  }
  int wid = PlanView(p).dq_order[blockIdx.x];
  const int nsub = (p.bx + kTileRows - 1) / kTileRows;
  const int sub = wid % nsub;
  wid /= nsub;
  const int ib = wid % p.nqb;
  wid /= p.nqb;
  const int n = wid % p.N;
  const int b = wid / p.N;
  const SeqInfo si = p.seq[b];
  const int q0 = ib * p.bx + sub * kTileRows;
  const int part_end = min(ib * p.bx + p.bx, q0 + kTileRows);
  const int q_end = min(part_end, si.len_q);
  const int w_end = min(part_end, si.wlim_q);
  if (q0 >= w_end) return;

  const int h = n / p.G;
  const int64_t bn = static_cast<int64_t>(b) * p.N + n;
  const int my_q = q0 + 32 * w + l32;  // B-operand column == score column of this lane
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
  const float l2 = q_ok ? p.lse2[bn * p.sq_max + my_q] : 0.f;
  const float dl = q_ok ? p.delta[bn * p.sq_max + my_q] : 0.f;
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
  const SeqInfo si = p.seq[b];
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

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
inline int waves_for(int rows) {
  const int r = rows < kTileRows ? rows : kTileRows;
  const int w = (r + 31) / 32;
  return w == 3 ? 4 : w;  // kernels are built for 1, 2 and 4 waves
}

}  // namespace

// ---------------------------------------------------------------------------
// scratch array of the entry point that allocates nothing
// ---------------------------------------------------------------------------
// Every device the library runs on holds its own copy of this array from the
// module's load to the end of the process.  Host code must not pass the name
// itself to a kernel (on the host it is only a stand-in for the symbol): the
// device address comes from hipGetSymbolAddress, looked up once per device with
// that device current.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

int scratch_region(void** ptr, uint64_t* bytes) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return static_cast<int>(e);
  if (dev < 0 || dev >= kMaxDevices) return static_cast<int>(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return static_cast<int>(e);
    if (a == nullptr) return static_cast<int>(hipErrorInvalidSymbol);
    addr[dev] = a;
  }
  *ptr = addr[dev];
  *bytes = kScratchBytes;
  return 0;
}

int launch_stage_fp8(const Fp8Stage& st, void* stream) {
  int64_t groups = 0;
  for (int t = 0; t < st.count; ++t) groups += st.n16[t];
  if (groups == 0) return 0;
  hipLaunchKernelGGL(stage_fp8_kernel, dim3(static_cast<unsigned>((groups + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), st);
  return static_cast<int>(hipGetLastError());
}

int launch_pack_amask(const Params& p, void* stream) {
  const int tiles_i = (p.sq_max + 63) / 64;
  const int tiles_j = static_cast<int>((p.amask_ld + 63) / 64);
  const int64_t tiles = static_cast<int64_t>(tiles_i) * tiles_j;
  hipLaunchKernelGGL(pack_amask_kernel, dim3(static_cast<unsigned>((tiles + 3) / 4)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), p, tiles_i, tiles_j);
  return static_cast<int>(hipGetLastError());
}

int launch_stage_seq(const SeqChunk& chunk, SeqInfo* dst, float* consts, void* stream) {
  hipLaunchKernelGGL(stage_seq_kernel, dim3(1), dim3(kMaxInlineSeq), 0,
                     static_cast<hipStream_t>(stream), chunk, dst, consts);
  return static_cast<int>(hipGetLastError());
}

// prologue_kernel<E, D> for the data type and head dim of p
template <class... A>
void launch_prologue_kernel(const Params& p, dim3 grid, hipStream_t s, A... a) {
  const bool bf = p.dtype == 2;
  if (p.D == 256) {
    if (bf) hipLaunchKernelGGL((prologue_kernel<EBf16, 256>), grid, dim3(256), 0, s, p, a...);
    else hipLaunchKernelGGL((prologue_kernel<EF16, 256>), grid, dim3(256), 0, s, p, a...);
  } else if (p.D == 128) {
    if (bf) hipLaunchKernelGGL((prologue_kernel<EBf16, 128>), grid, dim3(256), 0, s, p, a...);
    else hipLaunchKernelGGL((prologue_kernel<EF16, 128>), grid, dim3(256), 0, s, p, a...);
  } else {
    if (bf) hipLaunchKernelGGL((prologue_kernel<EBf16, 64>), grid, dim3(256), 0, s, p, a...);
    else hipLaunchKernelGGL((prologue_kernel<EF16, 64>), grid, dim3(256), 0, s, p, a...);
  }
}

int launch_prologue(const Params& p, void* stream) {
  const PrologueGrid pg = prologue_grid(p.B, p.N, p.sq_max, p.nqb, p.nkb, p.tnd != 0);
  launch_prologue_kernel(p, dim3(static_cast<unsigned>(pg.total())), static_cast<hipStream_t>(stream),
                         static_cast<int>(pg.rows), static_cast<int>(pg.cols));
  return static_cast<int>(hipGetLastError());
}

#define BSA_DISPATCH_AM(KERNEL, E, D, W, AM, GRID, S, P)                                    \
  do {                                                                                       \
    if ((W) == 4) hipLaunchKernelGGL((KERNEL<E, D, 4, AM>), GRID, dim3(256), 0, S, P);       \
    else if ((W) == 2) hipLaunchKernelGGL((KERNEL<E, D, 2, AM>), GRID, dim3(128), 0, S, P);  \
    else hipLaunchKernelGGL((KERNEL<E, D, 1, AM>), GRID, dim3(64), 0, S, P);                 \
  } while (0)
#define BSA_DISPATCH_W(KERNEL, E, D, W, GRID, S, P)                 \
  do {                                                             \
    if ((P).amask) BSA_DISPATCH_AM(KERNEL, E, D, W, true, GRID, S, P); \
    else BSA_DISPATCH_AM(KERNEL, E, D, W, false, GRID, S, P);          \
  } while (0)

#define BSA_DISPATCH(KERNEL, W, GRID, S, P)                                     \
  do {                                                                          \
    const bool bf_ = (P).dtype == 2;                                            \
    if ((P).D == 256) {                                                         \
      if (bf_) BSA_DISPATCH_W(KERNEL, EBf16, 256, W, GRID, S, P);               \
      else BSA_DISPATCH_W(KERNEL, EF16, 256, W, GRID, S, P);                    \
    } else if ((P).D == 128) {                                                  \
      if (bf_) BSA_DISPATCH_W(KERNEL, EBf16, 128, W, GRID, S, P);               \
      else BSA_DISPATCH_W(KERNEL, EF16, 128, W, GRID, S, P);                    \
    } else {                                                                    \
      if (bf_) BSA_DISPATCH_W(KERNEL, EBf16, 64, W, GRID, S, P);                \
      else BSA_DISPATCH_W(KERNEL, EF16, 64, W, GRID, S, P);                     \
    }                                                                           \
  } while (0)

int launch_prologue_rows(const Params& p, void* stream) {
  const PrologueGrid pg = prologue_grid(p.B, p.N, p.sq_max, p.nqb, p.nkb, p.tnd != 0);
  launch_prologue_kernel(p, dim3(static_cast<unsigned>(pg.rows)), static_cast<hipStream_t>(stream),
                         static_cast<int>(pg.rows), 0);
  return static_cast<int>(hipGetLastError());
}

int launch_fwd(const Params& p, void* stream) {
  const dim3 grid(static_cast<unsigned>(p.n_dq_units));
  BSA_DISPATCH(fwd_kernel, waves_for(p.bx), grid, static_cast<hipStream_t>(stream), p);
  return static_cast<int>(hipGetLastError());
}

int launch_plan(const Params& p, void* stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, static_cast<hipStream_t>(stream), p);
  return static_cast<int>(hipGetLastError());
}

// Compute units of the current device (looked up once per device).
int device_cus() {
  constexpr int kMaxDevices = 64;
  static int cus[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

// The scheduled dK/dV build: fp16/bf16 at head dim 64 or 128 without an
// attenMask; persistent, as many workgroups as run at once (one wave per SIMD:
// 4 / W workgroups per compute unit), or fewer if there are fewer work items.
template <class E, int D, int W, int NSL>
void launch_dkdv_pipe(const Params& p, dim3 items, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(std::min<int64_t>(items.x, static_cast<int64_t>(device_cus()) * (4 / W))));
  if (p.win) hipLaunchKernelGGL((dkdv_pipe_kernel<E, D, W, NSL, true>), grid, dim3(64 * W), 0, s, p);
  else hipLaunchKernelGGL((dkdv_pipe_kernel<E, D, W, NSL, false>), grid, dim3(64 * W), 0, s, p);
}
template <class E, int D>
void launch_dkdv_pipe_w(const Params& p, int w, dim3 grid, hipStream_t s) {
  const int nsl = dkdv_pipe_nsl(p.bx, w);
  if (w == 4) {
    if (nsl == 4) launch_dkdv_pipe<E, D, 4, 4>(p, grid, s);
    else if (nsl == 2) launch_dkdv_pipe<E, D, 4, 2>(p, grid, s);
    else launch_dkdv_pipe<E, D, 4, 1>(p, grid, s);
  } else if (w == 2) {
    if (nsl == 2) launch_dkdv_pipe<E, D, 2, 2>(p, grid, s);
    else launch_dkdv_pipe<E, D, 2, 1>(p, grid, s);
  } else {
    launch_dkdv_pipe<E, D, 1, 1>(p, grid, s);
  }
}

int launch_dkdv(const Params& p, void* stream) {
  const dim3 grid(static_cast<unsigned>(dkdv_passes(p.D) * (p.n_units + p.slots_cap)));
  if (p.amask == nullptr && p.D <= 128 && p.G <= kDkdvMaxGroup) {
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const int w = waves_for(p.by);
    const bool bf = p.dtype == 2;
    if (p.D == 128) {
      if (bf) launch_dkdv_pipe_w<EBf16, 128>(p, w, grid, s);
      else launch_dkdv_pipe_w<EF16, 128>(p, w, grid, s);
    } else {
      if (bf) launch_dkdv_pipe_w<EBf16, 64>(p, w, grid, s);
      else launch_dkdv_pipe_w<EF16, 64>(p, w, grid, s);
    }
    return static_cast<int>(hipGetLastError());
  }
  // head dim 256: the 1- and 2-wave builds spill registers, so KV blocks of
  // up to 64 rows also take the 4-wave one (its waves past the block's rows
  // compute on zero K/V rows and store nothing)
  const int w = p.D >= 256 ? 4 : waves_for(p.by);
  BSA_DISPATCH(dkdv_kernel, w, grid, static_cast<hipStream_t>(stream), p);
  return static_cast<int>(hipGetLastError());
}

int launch_dq(const Params& p, void* stream) {
  const dim3 grid(static_cast<unsigned>(p.n_dq_units + p.slots_cap));
  BSA_DISPATCH(dq_kernel, waves_for(p.bx), grid, static_cast<hipStream_t>(stream), p);
  return static_cast<int>(hipGetLastError());
}

}  // namespace bsa
