// Device code shared by the HIP kernels of the block-sparse attention
// backward (and forward) for gfx950 (CDNA4).  The kernels themselves live in
// bsa_prologue.hip (stage_seq, stage_fp8, pack_amask, prologue, plan),
// bsa_dkdv*.hip / bsa_dkdv.h (dK/dV), bsa_dq.hip (dQ) and bsa_fwd.hip (forward).
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
//               into pieces, orders the dK/dV work items longest first and
//               the dQ workgroups longest first
//   dkdv        work item = (batch, KV head, KV block [, 128-row part]
//               [, piece]); K/V rows stay in registers; it walks the Q blocks
//               that select its KV block for every query head of the group:
//               S, P, dV += P^T dO, dP, dS, dK += dS^T Q (four MFMA GEMMs per
//               step).  Q/dO tiles (XOR-swizzled) are double-buffered in LDS,
//               the next one copied in by DMA during the current one.  The
//               scheduled build (head dim <= 128, no attenMask) is persistent:
//               as many workgroups as fit the GPU take the items in order from
//               a counter; the generic build runs one workgroup per item.
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
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>

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

// The record of sequence b (offsets, lengths, rows written).
__device__ __forceinline__ SeqInfo seq_of(const Params& p, int b) { return p.seq_uniform ? p.seq0 : p.seq[b]; }

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

// The plan region, in order: [0] entries per piece, [1] number of work items, [2] dQ order,
// [3] the next work item to take (the persistent dK/dV kernel's counter), then
// per unit its piece count and first slot, per slot its unit (-1 = unused) and
// piece, the work items (unit, piece) in launch order, the dQ units in launch
// order, and per unit the count of its finished pieces.
struct PlanView {
  int32_t* unit_k;
  int32_t* unit_base;
  int32_t* slot_unit;
  int32_t* slot_chunk;
  int32_t* order_unit;
  int32_t* order_piece;
  int32_t* dq_order;  // dQ workgroup k runs dQ unit dq_order[k]
  int32_t* piece_done;  // finished pieces (and passes) of each split unit
  __device__ explicit PlanView(const Params& p) {
    unit_k = p.plan + 4;
    unit_base = unit_k + p.n_units;
    slot_unit = unit_base + p.n_units;
    slot_chunk = slot_unit + p.slots_cap;
    order_unit = slot_chunk + p.slots_cap;
    order_piece = order_unit + p.n_units + p.slots_cap;
    dq_order = order_piece + p.n_units + p.slots_cap;
    piece_done = dq_order + p.n_dq_units;
  }
};

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

// Wait states inside the copy helpers (gfx9 hazards that the compiler observes
// for its own code but cannot see inside inline assembly):
//  - the LDS-DMA loads read m0 for their destination, and an SALU write of m0
//    needs one wait state before such a load reads it;
//  - a vector memory instruction that reads an SGPR written by a VALU
//    instruction needs five wait states in between.  The wave-uniform base of
//    dma16s often comes from v_readfirstlane (a VALU write of the SGPR pair)
//    placed by the compiler right before the asm block, so the block waits
//    five states (s_nop 4) after the m0 write before the load reads the base.
//    Without them the load may address from a stale base (a copy of other
//    rows); the compiled kernels are checked for this by tests/test_isa_hazards.py.
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
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sb), "s"(m)
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
// dispatch
// ---------------------------------------------------------------------------
inline int waves_for(int rows) {
  const int r = rows < kTileRows ? rows : kTileRows;
  const int w = (r + 31) / 32;
  return w == 3 ? 4 : w;  // kernels are built for 1, 2 and 4 waves
}

}  // namespace

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
}  // namespace bsa
