// The dK/dV kernels (KV-block outer): the device code and launch templates that
// the dK/dV translation units instantiate (bsa_dkdv.hip: the dispatcher and the
// builds without an attenMask; bsa_dkdv_am.hip: the attenMask builds;
// bsa_dkdv_pipe_bf16.hip / _f16.hip: the scheduled builds per element type).
#pragma once

#include "bsa_device.h"

namespace bsa {

int device_cus();  // compute units of the current device (bsa_dkdv.hip)

namespace {

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

// Sum the pieces of split unit u in piece order, scale dK, round and store
// both (every thread of the workgroup takes part).
template <class E, int D>
__device__ void reduce_unit(const Params& p, int u) {
  const PlanView pv(p);
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
  const SeqInfo si = seq_of(p, b);
  const int kv0 = jb * p.by + sub * kTileRows;
  const int w_end = min(min(jb * p.by + p.by, kv0 + kTileRows), si.wlim_kv);
  if (kv0 >= w_end) return;
  unsigned short* dkp = static_cast<unsigned short*>(p.dk) + b * p.dk_sb + si.off_kv * p.dk_sr + h * p.dk_sh;
  unsigned short* dvp = static_cast<unsigned short*>(p.dv) + b * p.dv_sb + si.off_kv * p.dv_sr + h * p.dv_sh;
  const int per_t = (w_end - kv0) * D / 4;  // float4 groups of one tensor
  const int nthr = blockDim.x;
  // GB groups per thread at a time and up to PB pieces' loads in flight
  // together, summed in piece order
  constexpr int GB = 4, PB = 4;
  constexpr int64_t PSTRIDE = 2 * kTileRowsMax * D;  // floats between pieces
  for (int q0 = threadIdx.x; q0 < 2 * per_t; q0 += GB * nthr) {
    float4 acc[GB];
    const float* at[GB];
    bool ok[GB];
#pragma unroll
    for (int i = 0; i < GB; ++i) {
      const int q = q0 + i * nthr;
      ok[i] = q < 2 * per_t;
      const int t = ok[i] ? q / per_t : 0;  // 0: dK, 1: dV
      const int rem = ok[i] ? q - t * per_t : 0;
      at[i] = src + (t * kTileRowsMax + rem / (D / 4)) * D + 4 * (rem % (D / 4));
      acc[i] = ok[i] ? *reinterpret_cast<const float4*>(at[i]) : float4{0.f, 0.f, 0.f, 0.f};
    }
    for (int c0 = 1; c0 < pieces; c0 += PB) {
      float4 x[PB][GB];
#pragma unroll
      for (int j = 0; j < PB; ++j)
#pragma unroll
        for (int i = 0; i < GB; ++i)
          x[j][i] = ok[i] && c0 + j < pieces ? *reinterpret_cast<const float4*>(at[i] + (c0 + j) * PSTRIDE)
                                              : float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < PB; ++j)
#pragma unroll
        for (int i = 0; i < GB; ++i)
          if (c0 + j < pieces) {
            acc[i].x += x[j][i].x;
            acc[i].y += x[j][i].y;
            acc[i].z += x[j][i].z;
            acc[i].w += x[j][i].w;
          }
    }
#pragma unroll
    for (int i = 0; i < GB; ++i) {
      if (!ok[i]) continue;
      const int q = q0 + i * nthr;
      const int t = q / per_t, rem = q - t * per_t;
      const int rl = rem / (D / 4), d = 4 * (rem % (D / 4));
      const float sc = t == 0 ? p.dk_scale : p.dv_scale;
      const float v[4] = {acc[i].x * sc, acc[i].y * sc, acc[i].z * sc, acc[i].w * sc};
      store4<E>((t == 0 ? dkp + (kv0 + rl) * p.dk_sr : dvp + (kv0 + rl) * p.dv_sr) + d, v);
    }
  }
}

// After a workgroup has stored its piece of split unit u: count the piece
// (each of the dkdv_passes workgroups of a piece counts once), and the
// workgroup that completes the count sums the unit (no workgroup waits for
// another).  Every wave first waits for its own partial stores to complete
// (the barrier alone waits for LDS operations only), so that after the
// barrier one thread's release fence (agent scope: it writes the XCD's L2
// back, so the stores are visible on every XCD) covers all of them before
// the count; only the last workgroup takes
// the acquire fence (it invalidates its XCD's L2, which costs every other
// workgroup there its cached tiles), again in one thread, with the barrier
// ordering the sum after it.  The sum is the same whichever workgroup does
// it.  `flag` is an LDS word.
template <class E, int D>
__device__ void piece_finished(const Params& p, int u, int* flag) {
  wait_vmcnt<0>();  // this wave's partial stores have reached its XCD's L2
  __syncthreads();  // ... for every wave, before the fence below
  if (threadIdx.x == 0) {
    const PlanView pv(p);
    const int total = pv.unit_k[u] * dkdv_passes(D);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const bool last = atomicAdd(&pv.piece_done[u], 1) == total - 1;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // the other pieces' stores, before the sum
    *flag = last;
  }
  __syncthreads();
  if (*flag) reduce_unit<E, D>(p, u);  // uniform
  __syncthreads();  // everyone read the flag before it is written again
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
                                          uint32_t (*sB)[AM ? dkdv_mask_words<D, W>() : 1][32 * W], int* sFlag) {
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
  const int pieces = pv.unit_k[u];
  const int chunk = p.plan[0];

  int wid = u;
  const int nsub = (p.by + kTileRows - 1) / kTileRows;
  const int sub = wid % nsub;
  wid /= nsub;
  const int jb = wid % p.nkb;
  wid /= p.nkb;
  const int h = wid % p.Nkv;
  const int b = wid / p.Nkv;
  const SeqInfo si = seq_of(p, b);
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
  if (pieces > 1) piece_finished<E, D>(p, u, sFlag);  // uniform
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

// dQ by atomic adds: the dS tile of one 32-row slice in LDS, [key row][query]
// with rows of kDsPitch elements (32 queries + 4, so that the rows of one
// transposing read and of one write spread over the banks).
constexpr int kDsPitch = 36;
template <int W>
__host__ __device__ constexpr unsigned ds_slice_bytes() { return 2u * kDsPitch * 32 * W; }

// DQA: also write each slice's dS (as rounded for the dK product) to the dS
// region at byte address ds_wr (this lane's key row and query quad; slice sl
// at + sl * ds_slice_bytes), zero for keys past the sequence end.
template <class E, int D, int W, int NSL, bool WIN, bool DQA>
__device__ __forceinline__ void dkdv_pipe_tile(const DkdvAddr<D, W, NSL>& ad, const u16x8 (&kreg)[D / 16],
                                               const u16x8 (&vreg)[D / 16], f32x16 (&adv)[D / 32],
                                               f32x16 (&adk)[D / 32], float c2, const uint32_t (&keep)[NSL],
                                               unsigned ds_wr, bool kv_ok) {
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
  // DV: slice NSL-2's dV products wait for X(NSL-1), which has no S / dP of
  // its own to hide slice NSL-1's softmax under (the accumulation order
  // stays slice order).  For two-slice tiles only: that softmax is a quarter
  // of their VALU work (3% off the kernel at 64-row blocks), while with four
  // slices the longer-lived operands cost more than they hide (+1.5%).
  constexpr bool DV = NSL == 2;
  u16x8 pa_d[2];
  u16x4 bo_d[2][NT][2];
#pragma unroll
  for (int sl = 0; sl < NSL; ++sl) {
    const int cur = sl & 1, nxt = cur ^ 1;
    const unsigned cb = 2u * 32 * sl * D;
    // ---- X(sl): slice sl + 1's S / dP on the matrix cores, slice sl's softmax on the VALU
    const f32x4(&l4)[4] = in[cur].l4;
    if (sl + 1 < NSL) dkdv_sdp<E, D>(in[nxt], kreg, vreg, s[nxt], dp[nxt]);
    if (DV && sl + 1 == NSL) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) adv[nt] = E::mma(cat8(bo_d[hh][nt][0], bo_d[hh][nt][1]), pa_d[hh], adv[nt]);
    }
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
    if constexpr (DQA) {
      // registers 8hh..8hh+3 hold query rows 16hh + 4g + {0..3}, the next four
      // rows 16hh + 8 + 4g + {0..3}: two 8-byte writes per half
      typedef __attribute__((address_space(3))) u16x4 lds_u16x4;
      const u16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const u16x8 v = kv_ok ? da[hh] : z;
        const unsigned a = ds_wr + sl * ds_slice_bytes<W>() + 32u * hh;
        *(lds_u16x4*)(static_cast<uintptr_t>(a)) = u16x4{v[0], v[1], v[2], v[3]};
        *(lds_u16x4*)(static_cast<uintptr_t>(a + 16u)) = u16x4{v[4], v[5], v[6], v[7]};
      }
    }
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
    } else if (DV) {
#pragma unroll
      for (int k = 0; k < 2 * NT; ++k) {
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, (8 * NT + 2 * NT - 1) / (2 * NT), 0);
        __builtin_amdgcn_sched_group_barrier(kSgValu, (WIN ? 128 : 96) / (2 * NT), 0);
      }
    }
    // ---- Y(sl): dV^T += dO^T P, dK^T += Q^T dS; loads slice sl + 2's fragments.
    // The fragment read down dO's (Q's) rows is, as an A operand, dO^T with
    // the same k order as P's (dS's) registers, which serve as the B operand:
    // the accumulators hold dV^T / dK^T, one key row per lane, so the
    // epilogue stores four consecutive elements at a time.
    if (DV && sl + 2 == NSL) {  // to X(NSL-1)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        pa_d[hh] = pa[hh];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          bo_d[hh][nt][0] = bo[hh][nt][0];
          bo_d[hh][nt][1] = bo[hh][nt][1];
        }
      }
    } else {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) adv[nt] = E::mma(cat8(bo[hh][nt][0], bo[hh][nt][1]), pa[hh], adv[nt]);
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) adk[nt] = E::mma(cat8(bq[hh][nt][0], bq[hh][nt][1]), da[hh], adk[nt]);
    if (sl + 2 < NSL) dkdv_read_a<D, W, NSL>(ad, sl + 2, in[cur]);
#pragma unroll
    for (int k = 0; k < (DV && sl + 2 == NSL ? 2 : 4) * NT; ++k) {
      __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
      if (sl + 2 < NSL) __builtin_amdgcn_sched_group_barrier(kSgDsRead, (2 * KS + 8 + 4 * NT - 1) / (4 * NT), 0);
    }
  }
}

// dQ by atomic adds, for one finished tile (its dS region written by every
// wave, the barrier after the tile passed): wave w takes the head-dim stripes
// nt = w, w + W, ... of 32 columns; per 32-row slice, dQ[q][d] = sum over the
// item's 32 W keys of dS[q][key] K[key][d], with dS from the tile's region
// and K from the item's K rows in LDS (tile layout), both read down their key
// rows in the same order; each lane then adds its 16 results into dq_acc
// (row base `row0` of (batch, query head)), a 128-byte run of one row per
// half-wave and register.  Rows from qend on are not added.
template <class E, int D, int W, int NSL>
__device__ __forceinline__ void dkdv_dq_tile(const Params& p, unsigned kt, unsigned ds, int64_t row0, int q0,
                                             int qend) {
  constexpr int NT = D / 32;
  constexpr unsigned DS_ROW = 2u * kDsPitch;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l32 = lane & 31, g = lane >> 5;
  const int rr = 4 * g + ((lane & 15) >> 2);
  const int col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
  for (int sl = 0; sl < NSL; ++sl) {
    if (q0 + 32 * sl >= qend) break;  // uniform
    const unsigned dsl = ds + sl * ds_slice_bytes<W>() + rr * DS_ROW + 2u * col;
#pragma unroll
    for (int nt = w; nt < NT; nt += W) {
      f32x16 c = {};
#pragma unroll
      for (int kk = 0; kk < 2 * W; ++kk) {
        const u16x8 a = cat8(lds_tr(dsl + 16u * kk * DS_ROW), lds_tr(dsl + (16u * kk + 8u) * DS_ROW));
        const u16x8 b = cat8(lds_tr(kt + 2u * tile_off<D>(16 * kk + rr, 32 * nt + col)),
                             lds_tr(kt + 2u * tile_off<D>(16 * kk + rr + 8, 32 * nt + col)));
        c = E::mma(a, b, c);  // dQ[q][d] (unscaled): lane's column d = 32 nt + l32
      }
      float* dst = p.dq_acc + (row0 + q0 + 32 * sl) * D + 32 * nt + l32;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int q = 8 * (i >> 2) + 4 * g + (i & 3);
        if (q0 + 32 * sl + q < qend) unsafeAtomicAdd(dst + static_cast<int64_t>(q) * D, c[i]);
      }
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
    // read-out: lane tid takes chunk c = tid % CPR of rows tid / CPR + RPP k,
    // all of a tensor's reads issued before its stores
    constexpr int RPP = 64 * W / CPR;  // rows one sweep of the workgroup covers
    constexpr int KPT = RT / RPP;      // sweeps per tensor
    static_assert(KPT * RPP == RT, "rows split evenly over the sweeps");
    const int c = tid % CPR, r0 = tid / CPR;
#pragma unroll
    for (int t = 0; t < 2 / NPASS; ++t) {
      const bool is_k = NPASS == 1 ? t == 0 : pass == 0;
      const int64_t sr = is_k ? p.dk_sr : p.dv_sr;
      unsigned short* dst = (is_k ? dkp : dvp) + (kv0 + r0) * sr + 8 * c;
      u16x8 v[KPT];
#pragma unroll
      for (int k = 0; k < KPT; ++k) {
        const int r = r0 + RPP * k;
        v[k] = lds_b128(stage + t * TBYTES + 2u * (r * D + 8 * (c ^ (r & (CPR - 1)))));
      }
#pragma unroll
      for (int k = 0; k < KPT; ++k)
        if (r0 + RPP * k < rows) *reinterpret_cast<u16x8*>(dst + RPP * k * sr) = v[k];
    }
  }
}

// Persistent: a grid of as many workgroups as fit the GPU at once, each taking
// work items from the plan's launch order (longest first) through a counter
// in the plan region, which the plan kernel zeroes.  When an item's tiles are
// done, the workgroup first starts the next item (its list, its first tile's
// copies, its K and V rows) and only then issues the finished item's stores,
// so those loads fly while the stores are issued.  Which workgroup runs an
// item does not change the item's result.
// DQA: dQ by atomic adds (Params::dq_acc); the item's K rows are copied into
// LDS too, and every finished tile's dQ is added into dq_acc (dkdv_dq_tile)
// at the start of the next tile, after that tile's copies are issued.
template <class E, int D, int W, int NSL, bool WIN, bool DQA>
__global__ __launch_bounds__(64 * W) void dkdv_pipe_kernel(Params p) {
  using T = DkdvPipe<D, W, NSL>;
  constexpr int KS = T::KS, NT = T::NT, H = T::H, RW = T::RW;
  constexpr unsigned TB = T::TB, BUF = T::BUF;
  static_assert(!DQA || NSL <= 2, "with dQ by atomics the LDS holds at most two slices per tile");
  // Q / dO tiles of buffer b at byte 2 b TB (swizzled rows); per buffer the
  // LSE*log2e rows, then the -softmax_grad rows
  __shared__ __align__(1024) unsigned short sT[2 * 2 * H * D];
  __shared__ __align__(16) float sLD[2 * 2 * H];
  __shared__ int sListIb[kDkdvListChunk], sListCnt[kDkdvMaxGroup];
  __shared__ unsigned short sListN[kDkdvListChunk];
  __shared__ int sItem, sFlag;
  // DQA: the item's K rows (tile layout), and per buffer the tile's dS slices
  __shared__ __align__(1024) unsigned short sKt[DQA ? 32 * W * D : 8];
  __shared__ __align__(16) unsigned short sDS[DQA ? 2 * NSL * 32 * W * kDsPitch : 8];

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
    it.si = seq_of(p, it.b);
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
  // DQA: the item's 32 W K rows into sKt by DMA, each wave its own 32 rows;
  // rows past the sequence end copy a chunk of the item's first row (finite;
  // their dS is written as zero)
  constexpr int NCK = 32 / RPI;  // copies per wave
  const unsigned kt0 = lds_addr(sKt), ds0 = lds_addr(sDS);
  auto load_kt = [&](const Item& it) {
    const unsigned short* kp = static_cast<const unsigned short*>(p.k) + it.b * p.kv_sb +
                               (it.si.off_kv + it.kv0) * p.kv_sr + it.h * p.kv_sh;
#pragma unroll
    for (int i = 0; i < NCK; ++i) {
      const int ins = w * NCK + i;
      const int r = ins * RPI + lrow;
      const int c = (lane % (D / 8)) ^ swz<D>(r);
      const unsigned v = static_cast<unsigned>(2 * (r * p.kv_sr + 8 * c));
      dma16s(kp, it.kv0 + r < it.kv_end ? v : vz, kt0 + 1024u * ins);
    }
  };
  // start an item: its list, its first tile's copies into buffer 0, its K/V rows
  auto start = [&](const Item& it, QTile& first) {
    list_start(it);
    if (lst.count > 0) {
      first = tile_of(it, 0);
      issue(it, first, 0);
    }
    if constexpr (DQA) load_kt(it);
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
    // DQA: this lane's dS writes (its key row, its query quad) in buffer 0's region
    const unsigned ds_wr = ds0 + (32u * w + l32) * 2u * kDsPitch + 8u * g;
    constexpr unsigned DSB = NSL * ds_slice_bytes<W>();  // one buffer's dS region
    QTile prev{};
    bool have_prev = false;
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
      if constexpr (DQA)  // the previous tile's dQ, its dS region complete since the last barrier
        if (have_prev)
          dkdv_dq_tile<E, D, W, NSL>(p, kt0, ds0 + (buf ^ 1) * DSB, (cur_it.bn0 + prev.n) * p.sq_max, prev.q0,
                                     prev.qend);
      dkdv_pipe_tile<E, D, W, NSL, WIN, DQA>(ad, kreg, vreg, adv, adk, c2, keep, ds_wr + buf * DSB,
                                             my_kv < cur_it.kv_end);
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
      prev = cur;
      have_prev = true;
      cur = nxt;
      have = more;
      if constexpr (DQA)  // the last tile's dQ (buffer buf ^ 1 after the flip below is this one's)
        if (!have) dkdv_dq_tile<E, D, W, NSL>(p, kt0, ds0 + buf * DSB, (cur_it.bn0 + prev.n) * p.sq_max, prev.q0,
                                              prev.qend);
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
    if (cur_it.pieces > 1) piece_finished<E, D>(p, cur_it.u, &sFlag);  // uniform
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
  __shared__ int sFlag;
  if constexpr (dkdv_passes(D) == 1) {
    dkdv_work<E, D, W, kDkdvBoth, AM>(p, blockIdx.x, sQ, sO, sL, sDl, sB, &sFlag);
  } else {  // workgroups 2i and 2i + 1 run the dV and the dK pass of work item i
    if (blockIdx.x & 1) dkdv_work<E, D, W, kDkdvOnlyK, AM>(p, blockIdx.x >> 1, sQ, sO, sL, sDl, sB, &sFlag);
    else dkdv_work<E, D, W, kDkdvOnlyV, AM>(p, blockIdx.x >> 1, sQ, sO, sL, sDl, sB, &sFlag);
  }
}

// The scheduled dK/dV build: fp16/bf16 at head dim 64 or 128 without an
// attenMask; persistent, as many workgroups as run at once (one wave per SIMD:
// 4 / W workgroups per compute unit, fewer where the LDS of the dQ-by-atomics
// build does not fit that many), or fewer if there are fewer work items.
template <class E, int D, int W, int NSL, bool DQA>
void launch_dkdv_pipe(const Params& p, dim3 items, hipStream_t s) {
  int per_cu = 4 / W;
  if constexpr (DQA) {
    static int fit = 0;  // workgroups of this build per compute unit (looked up once)
    if (fit == 0) {
      int n = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, dkdv_pipe_kernel<E, D, W, NSL, false, true>, 64 * W, 0) !=
              hipSuccess ||
          n <= 0) {
        (void)hipGetLastError();
        n = 1;
      }
      fit = n;
    }
    per_cu = std::min(per_cu, fit);
  }
  const dim3 grid(static_cast<unsigned>(std::min<int64_t>(items.x, static_cast<int64_t>(device_cus()) * per_cu)));
  if (p.win) hipLaunchKernelGGL((dkdv_pipe_kernel<E, D, W, NSL, true, DQA>), grid, dim3(64 * W), 0, s, p);
  else hipLaunchKernelGGL((dkdv_pipe_kernel<E, D, W, NSL, false, DQA>), grid, dim3(64 * W), 0, s, p);
}
template <class E, int D, bool DQA>
void launch_dkdv_pipe_w(const Params& p, int w, dim3 grid, hipStream_t s) {
  int nsl = dkdv_pipe_nsl(p.bx, w);
  if (DQA && nsl > 2) nsl = 2;  // the dS and K regions take the LDS of two slices
  if (w == 4) {
    if (nsl == 4) {
      if constexpr (!DQA) launch_dkdv_pipe<E, D, 4, 4, DQA>(p, grid, s);
    } else if (nsl == 2) {
      launch_dkdv_pipe<E, D, 4, 2, DQA>(p, grid, s);
    } else {
      launch_dkdv_pipe<E, D, 4, 1, DQA>(p, grid, s);
    }
  } else if (w == 2) {
    if (nsl == 2) launch_dkdv_pipe<E, D, 2, 2, DQA>(p, grid, s);
    else launch_dkdv_pipe<E, D, 2, 1, DQA>(p, grid, s);
  } else {
    launch_dkdv_pipe<E, D, 1, 1, DQA>(p, grid, s);
  }
}

// The generic dK/dV build (every head dim, with or without an attenMask).
template <bool AM>
int launch_dkdv_generic(const Params& p, int w, dim3 grid, hipStream_t s) {
  const bool bf = p.dtype == 2;
  if (p.D == 256) {
    if (bf) BSA_DISPATCH_AM(dkdv_kernel, EBf16, 256, w, AM, grid, s, p);
    else BSA_DISPATCH_AM(dkdv_kernel, EF16, 256, w, AM, grid, s, p);
  } else if (p.D == 128) {
    if (bf) BSA_DISPATCH_AM(dkdv_kernel, EBf16, 128, w, AM, grid, s, p);
    else BSA_DISPATCH_AM(dkdv_kernel, EF16, 128, w, AM, grid, s, p);
  } else {
    if (bf) BSA_DISPATCH_AM(dkdv_kernel, EBf16, 64, w, AM, grid, s, p);
    else BSA_DISPATCH_AM(dkdv_kernel, EF16, 64, w, AM, grid, s, p);
  }
  return static_cast<int>(hipGetLastError());
}

}  // namespace

// The scheduled builds, one translation unit per element type and head dim
// (bsa_dkdv_pipe.hip, compiled once for each).
int launch_dkdv_pipe_bf16_d64(const Params& p, dim3 grid, hipStream_t s);
int launch_dkdv_pipe_bf16_d128(const Params& p, dim3 grid, hipStream_t s);
int launch_dkdv_pipe_f16_d64(const Params& p, dim3 grid, hipStream_t s);
int launch_dkdv_pipe_f16_d128(const Params& p, dim3 grid, hipStream_t s);
int launch_dkdv_generic_am(const Params& p, int w, dim3 grid, hipStream_t s);

}  // namespace bsa
