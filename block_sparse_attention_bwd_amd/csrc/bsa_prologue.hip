// Prologue stages of the backward and the forward: the sequence table, fp8
// decode, attenMask packing, softmax_grad and the block lists, the dK/dV work
// plan; and the scratch array of the entry point that allocates nothing.
#include <mutex>

#include "bsa_device.h"

namespace bsa {
namespace {

// ---------------------------------------------------------------------------
// per-sequence table
// ---------------------------------------------------------------------------
__global__ void stage_seq_kernel(SeqChunk c, SeqInfo* dst) {
  const int t = threadIdx.x;
  if (t < c.count) dst[c.first + t] = c.s[t];
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
    const SeqInfo si = seq_of(p, b);
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
  const SeqInfo si = seq_of(p, b);
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
  const SeqInfo si = seq_of(p, b);
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

// Row lists, then column lists, then softmax_grad workgroups: those only
// where the dQ kernel does not compute softmax_grad itself (dQ by atomic
// adds); the forward launches the row lists only.  The list workgroups are
// latency-bound (a row-list wave walks its mask row 64 blocks per dependent
// load); dispatched first, they overlap the bandwidth-bound softmax_grad pass
// instead of trailing it.
template <class E, int D>
__global__ __launch_bounds__(256) void prologue_kernel(Params p, int nb_rows, int nb_cols) {
  const int bid = blockIdx.x;
  if (bid == 0 && threadIdx.x < kConstFloats) {  // the constant block (zeros, +inf, -inf)
    const int i = threadIdx.x;
    p.consts[i] = i == kConstPosInf ? __builtin_inff() : i == kConstNegInf ? -__builtin_inff() : 0.f;
  }
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
// T_u > chunk is cut into ceil(T_u / piece) pieces of consecutive entries,
// piece = ceil(chunk / 2): half the balanced share, so that the pieces end
// well before the kernel does and the sum that follows the last of them
// (which waits for every piece) stays off the end of the schedule.  Each
// piece writes an fp32 partial dK/dV and the pieces are summed in order, so
// the result is the same on every run.  Pieces get slots by an
// exclusive scan over units in unit order; units that would overflow the slot
// capacity stay whole.  One workgroup of 1024 threads.
__device__ __forceinline__ int unit_entries(const Params& p, int u) {
  // u = ((b Nkv + h) nkb + jb) nsub + sub, and head n = h G + i of batch b
  // has column counts at ((b Nkv + h) G + i) nkb + jb: two divisions
  const int nsub = (p.by + kTileRows - 1) / kTileRows;
  const int w = nsub == 1 ? u : u / nsub;
  const int bh = w / p.nkb;
  const int jb = w - bh * p.nkb;
  const int32_t* c = p.col_cnt + static_cast<int64_t>(bh) * p.G * p.nkb + jb;
  int t = 0;
  for (int i = 0; i < p.G; ++i) t += c[static_cast<int64_t>(i) * p.nkb];
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


// Launch order of the work items: longest first, so that the last workgroups
// to start are short ones.  Costs (Q-block entries of the piece) are binned
// into kOrderBins classes, class kOrderBins-1 holding units of about `chunk`
// entries and class 0 the units with nothing to do (they only write zeros).
// The order inside a class depends on scheduling; the results do not, since
// every piece sums its entries in list order and pieces are reduced in order.
constexpr int kOrderBins = 64;
__device__ __forceinline__ int order_bin(int cost, int chunk) {
  if (cost <= 0) return 0;
  const unsigned long long num = static_cast<unsigned long long>(cost - 1) * (kOrderBins - 1);
  const unsigned long long q = num >> 32 ? num / static_cast<unsigned>(chunk)  // (cost above 2^32 / 63)
                                         : static_cast<unsigned>(num) / static_cast<unsigned>(chunk);
  return min(static_cast<unsigned long long>(kOrderBins - 1), 1 + q);
}

constexpr int kPlanThreads = 1024, kPlanWaves = kPlanThreads / 64;
constexpr int kPlanCachedUnits = 8192;  // units whose T_u the plan kernel keeps in LDS
constexpr int kPlanCachedDq = 32768;    // dQ units whose KV-block count it keeps in LDS (16 bits)
// The dQ units are launched longest first only up to this many: with more,
// each workgroup slot runs a long queue of units, the order changes little at
// the end, and the sort's LDS atomics (one per unit, on a few class counters)
// cost more than it saves.
constexpr int kDqSortMaxUnits = 8192;

// Workgroup-wide sum, returned to every thread (s_w: one slot per wave).
__device__ __forceinline__ long long plan_sum(long long v, long long* s_w) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  __syncthreads();  // earlier readers of s_w are done
  if ((threadIdx.x & 63) == 0) s_w[threadIdx.x >> 6] = v;
  __syncthreads();
  long long t = 0;
#pragma unroll
  for (int i = 0; i < kPlanWaves; ++i) t += s_w[i];
  return t;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(v, off, 64);
    if (lane >= off) v += t;
  }
  return v;
}

// Workgroup-wide exclusive prefix sum in thread order.
__device__ __forceinline__ int plan_excl_scan(int v, long long* s_w) {
  const int incl = wave_incl_scan(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 63) s_w[threadIdx.x >> 6] = incl;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < (static_cast<int>(threadIdx.x) >> 6); ++i) before += static_cast<int>(s_w[i]);
  return before + incl - v;
}

// One wave: replace the kOrderBins counts in `bins` by the first position of
// each class when the classes are laid out in descending order (the position
// of class c is the count of every class above it).
static_assert(kOrderBins == 64, "one class per lane");
__device__ __forceinline__ void desc_class_cursors(int* bins) {
  const int c = kOrderBins - 1 - (threadIdx.x & 63);
  const int v = bins[c];
  bins[c] = wave_incl_scan(v) - v;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(Params p) {
  __shared__ long long s_w[kPlanWaves];
  __shared__ int s_hist[kOrderBins];  // counts of the cost classes, then their cursors
  __shared__ unsigned long long s_xcd[8];
  __shared__ int s_T[kPlanCachedUnits];
  __shared__ unsigned short s_rc[kPlanCachedDq];
  __shared__ int s_dq[8 * kOrderBins];  // dQ cost classes per XCD range: counts, then cursors
  __shared__ int s_dqmax;
  const int tid = threadIdx.x;
  const PlanView pv(p);
  const int per = (p.n_units + kPlanThreads - 1) / kPlanThreads;
  const int u0 = min(p.n_units, tid * per), u1 = min(p.n_units, u0 + per);
  if (tid < kOrderBins) s_hist[tid] = 0;
  if (tid < 8) s_xcd[tid] = 0;
  if (tid < 8 * kOrderBins) s_dq[tid] = 0;
  if (tid == 0) s_dqmax = 0;
  __syncthreads();
  const bool cached = p.n_units <= kPlanCachedUnits;
  auto T = [&](int u) { return cached ? s_T[u] : unit_entries(p, u); };
  const int nd = p.n_dq_units, nsub_q = (p.bx + kTileRows - 1) / kTileRows;
  const bool sort_dq = nd <= kDqSortMaxUnits;
  const bool rc_cached = sort_dq && p.nkb <= 65535;

  // T_u from the column counts, and the dQ units' KV-block counts, loaded in
  // one loop strided over the units (coalesced; both loads of an iteration,
  // and of the next, in flight together); the per-thread unit ranges below
  // read s_T after plan_sum's barriers.  Per XCD range of dQ units its work,
  // a unit costing its selected KV blocks + 1 (a thread's units change range
  // only every nd / 8 units).
  long long tot = 0;
  {
    unsigned long long acc = 0;
    int cur = xcd_of_unit(min(tid, max(nd - 1, 0)), max(nd, 1));
    int mx = 0;
    const int n_all = max(p.n_units, nd);
#pragma unroll 2
    for (int u = tid; u < n_all; u += kPlanThreads) {
      const int t = u < p.n_units ? unit_entries(p, u) : 0;
      const int rc = u < nd ? p.row_cnt[nsub_q == 1 ? u : u / nsub_q] : 0;
      if (u < p.n_units) {
        if (cached) s_T[u] = t;
        tot += t;
      }
      if (u < nd) {
        const int x = xcd_of_unit(u, nd);
        if (rc_cached) s_rc[u] = static_cast<unsigned short>(rc);
        if (x != cur) {
          atomicAdd(&s_xcd[cur], acc);
          acc = 0;
          cur = x;
        }
        acc += 1u + static_cast<unsigned>(rc);
        mx = max(mx, rc);
      }
    }
    // one LDS atomic per wave where its lanes end in the same range (the
    // common case: 64 consecutive units), else one per lane
    const int cur0 = __shfl(cur, 0, 64);
    if (__all(cur == cur0)) {
      unsigned long long w = acc;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) w += __shfl_xor(w, off, 64);
      if ((tid & 63) == 0 && w) atomicAdd(&s_xcd[cur0], w);
    } else if (acc) {
      atomicAdd(&s_xcd[cur], acc);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = max(mx, __shfl_xor(mx, off, 64));
    if ((tid & 63) == 0) atomicMax(&s_dqmax, mx);
  }
  const long long total = plan_sum(tot, s_w);
  const int chunk = static_cast<int>(max(static_cast<long long>(kMinChunk),
                                         (total + kBalanceGroups - 1) / kBalanceGroups));

  const int pc = (chunk + 1) / 2;  // entries per piece of a split unit
  int mine = 0;
  for (int u = u0; u < u1; ++u) {
    const int t = T(u);
    if (t > chunk) mine += (t + pc - 1) / pc;
  }
  for (int i = tid; i < p.slots_cap; i += kPlanThreads) pv.slot_unit[i] = -1;
  for (int i = tid; i < p.n_units; i += kPlanThreads) pv.piece_done[i] = 0;
  int run = plan_excl_scan(mine, s_w);
  const int run0 = run;  // the order loop below replays the piece counts from here
  int extra = 0;  // pieces >= 1 this thread creates
  for (int u = u0; u < u1; ++u) {
    const int t = T(u);
    const int k = t > chunk ? (t + pc - 1) / pc : 1;
    if (k > 1 && run + k <= p.slots_cap) {
      pv.unit_k[u] = k;
      pv.unit_base[u] = run;
      for (int c = 0; c < k; ++c) {
        pv.slot_unit[run + c] = u;
        pv.slot_chunk[run + c] = c;
        atomicAdd(&s_hist[order_bin(min(pc, t - c * pc), chunk)], 1);
      }
      run += k;
      extra += k - 1;
    } else {
      pv.unit_k[u] = 1;
      pv.unit_base[u] = 0;
      atomicAdd(&s_hist[order_bin(t, chunk)], 1);
    }
  }
  const long long extra_total = plan_sum(extra, s_w);  // (its barriers also complete s_hist)
  // dQ order: XCD ranges only if the heaviest holds at most 1/32 more than the mean
  unsigned long long xtot = 0, xmx = 0;
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    xtot += s_xcd[x];
    xmx = max(xmx, s_xcd[x]);
  }
  const bool ranges = 8 * xmx * 32 <= xtot * 33;
  if (tid < 64) desc_class_cursors(s_hist);
  if (tid == 0) {
    p.plan[0] = pc;
    p.plan[1] = p.n_units + static_cast<int>(extra_total);
    p.plan[2] = ranges ? kDqOrderXcdRange : kDqOrderPlain;
    p.plan[3] = 0;  // the persistent dK/dV kernel's item counter
  }
  __syncthreads();
  run = run0;
  for (int u = u0; u < u1; ++u) {
    const int t = T(u);
    int k = t > chunk ? (t + pc - 1) / pc : 1;  // as above, without reading unit_k back
    if (k > 1 && run + k <= p.slots_cap) run += k;
    else k = 1;
    for (int c = 0; c < k; ++c) {
      const int at = atomicAdd(&s_hist[order_bin(k > 1 ? min(pc, t - c * pc) : t, chunk)], 1);
      pv.order_unit[at] = u;
      pv.order_piece[at] = c;
    }
  }
  // dQ launch order: with XCD ranges, workgroup 8 k + x runs the k-th unit of
  // range x (the hardware hands workgroup i to XCD i % 8); otherwise the units
  // are dealt round-robin to the XCDs.  With few units, longest first (cost
  // classes of the selected KV-block count) within each range or overall;
  // else in unit order.  Results do not depend on the order.
  if (!sort_dq) {
    const int per_x = nd >> 3, rem_x = nd & 7;
    for (int u = tid; u < nd; u += kPlanThreads) {
      const int x = ranges ? xcd_of_unit(u, nd) : 0;
      const int k = ranges ? u - (x * per_x + min(x, rem_x)) : u;
      pv.dq_order[ranges ? 8 * k + x : k] = u;
    }
    return;
  }
  const int mxc = max(s_dqmax, 1);
  auto cls = [&](int u) { return order_bin(rc_cached ? static_cast<int>(s_rc[u]) : p.row_cnt[u / nsub_q], mxc); };
  for (int u = tid; u < nd; u += kPlanThreads)
    atomicAdd(&s_dq[(ranges ? xcd_of_unit(u, nd) : 0) * kOrderBins + cls(u)], 1);
  __syncthreads();
  if (tid < (ranges ? 8 : 1) * 64) desc_class_cursors(s_dq + (tid >> 6) * kOrderBins);
  __syncthreads();
  for (int u = tid; u < nd; u += kPlanThreads) {
    const int x = ranges ? xcd_of_unit(u, nd) : 0;
    const int k = atomicAdd(&s_dq[x * kOrderBins + cls(u)], 1);
    pv.dq_order[ranges ? 8 * k + x : k] = u;
  }
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

int launch_stage_seq(const SeqChunk& chunk, SeqInfo* dst, void* stream) {
  hipLaunchKernelGGL(stage_seq_kernel, dim3(1), dim3(kMaxInlineSeq), 0,
                     static_cast<hipStream_t>(stream), chunk, dst);
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
  const int64_t blocks = pg.rows + pg.cols + (p.fused_delta ? 0 : pg.delta);  // softmax_grad blocks last
  if (blocks == 0) return 0;
  launch_prologue_kernel(p, dim3(static_cast<unsigned>(blocks)), static_cast<hipStream_t>(stream),
                         static_cast<int>(pg.rows), static_cast<int>(pg.cols));
  return static_cast<int>(hipGetLastError());
}

int launch_prologue_rows(const Params& p, void* stream) {
  const PrologueGrid pg = prologue_grid(p.B, p.N, p.sq_max, p.nqb, p.nkb, p.tnd != 0);
  launch_prologue_kernel(p, dim3(static_cast<unsigned>(pg.rows)), static_cast<hipStream_t>(stream),
                         static_cast<int>(pg.rows), 0);
  return static_cast<int>(hipGetLastError());
}

int launch_plan(const Params& p, void* stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, static_cast<hipStream_t>(stream), p);
  return static_cast<int>(hipGetLastError());
}

}  // namespace bsa
