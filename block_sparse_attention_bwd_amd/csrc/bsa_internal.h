// Internal plan shared by the host API (validation, planning) and the HIP
// kernels.  Plain data only; no HIP types.
#pragma once

#include <stdint.h>

namespace bsa {

// One row of the per-sequence table staged into the workspace.
struct SeqInfo {
  int64_t off_q;   // TND: first token of the sequence in Q/O/dO/LSE; BNSD: 0
  int64_t off_kv;  // TND: first token in K/V; BNSD: 0
  int32_t len_q;   // valid query rows of the sequence
  int32_t len_kv;  // valid key rows
  int32_t wlim_q;  // rows of dQ this sequence owns (BNSD: S, so padding is zeroed; TND: len_q)
  int32_t wlim_kv; // rows of dK/dV it owns
};
static_assert(sizeof(SeqInfo) == 32, "SeqInfo layout");

// Everything a launch needs.  Strides are in elements; a "row" is one
// sequence position of one head.  Row r of head n of sequence b of a
// query-side tensor lives at  b*sb + (off_q + r)*sr + n*sh.
struct Params {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  const uint8_t* mask;  // nullptr = every block selected
  void* dq;
  void* dk;
  void* dv;
  void* out_o;      // forward outputs: attention_out, softmax_lse (natural log)
  float* out_lse;

  int64_t q_sb, q_sh, q_sr;    // query, attention_out, dout (identical, contiguous)
  int64_t kv_sb, kv_sh, kv_sr; // key, value
  int64_t dq_sb, dq_sh, dq_sr;
  int64_t dk_sb, dk_sh, dk_sr;
  int64_t dv_sb, dv_sh, dv_sr;
  int64_t lse_sb, lse_sh, lse_sr;
  int64_t o_sb, o_sh, o_sr;    // forward output O (any outer strides)

  int32_t B, N, Nkv, G, D;
  int32_t bx, by;      // block shape (Q rows, KV rows)
  int32_t nqb, nkb;    // mask block grid: ceil(maxSq/bx), ceil(maxSkv/by)
  int32_t sq_max;      // row extent of the delta/lse2 arrays
  int32_t dtype;       // bsa_dtype of the data tensors
  int32_t tnd;         // 1 for the TND layout (rows of one token's heads are adjacent)
  // sliding window: key j takes part for query i only if i - win_pre <= j <= i + win_next
  // (sequence-local positions); win == 0 means no window
  int32_t win, win_pre, win_next;
  // attenMask [maxSq, maxSkv] bytes, 1 = the pair does not take part (nullptr: none)
  const uint8_t* amask;
  int64_t amask_ld;
  // the attenMask packed to bits (1 = excluded) by pack_amask_kernel:
  // am_rows[i * am_wk + w] bit b <-> (query i, key 32 w + b);
  // am_cols[j * am_wq + w] bit b <-> (query 32 w + b, key j); zero past the edges
  uint32_t* am_rows;
  uint32_t* am_cols;    // nullptr in the forward (only the row form is read there)
  int32_t am_wk, am_wq; // ceil(maxSkv / 32), ceil(maxSq / 32)
  float scale;         // scale_value rounded to fp32
  float scale_log2e;   // factor from a raw score (row dot product) to log2 units: scale * log2(e)
                       // (fp8 inputs: times query's and key's dequantisation factors)
  // Factors applied to the fp32 accumulators on the way out, and to the row
  // sums of dOut o Out; for fp16/bf16 inputs: scale, scale, 1, 1, 1.  With fp8
  // inputs the kernels run on the codes' values (factor 1) and these restore
  // the dequantised result (see the fp8 entry points).
  float dq_scale, dk_scale, dv_scale, delta_scale, o_scale;

  // the per-sequence records: seq_uniform = 1 when every sequence has the same
  // one (BNSD with all lengths equal to S), which is then seq0 and no table is
  // staged; otherwise the table `seq` (see seq_of in the kernels)
  int32_t seq_uniform;
  SeqInfo seq0;

  // workspace regions
  SeqInfo* seq;
  float* consts;        // kConstFloats floats after the sequence table: zeros, then +inf, -inf (written by
                        // the prologue kernel)
  float* delta;         // -softmax_grad (negated: it seeds the dP accumulator of the dK/dV kernel)
  float* lse2;
  int32_t* row_cnt;
  int32_t* row_list;
  int32_t* col_cnt;
  int32_t* col_list;

  // load balance of the dK/dV kernel (see plan_kernel)
  int32_t n_units;     // dK/dV work units: B * Nkv * nKB * ceil(by / 128)
  int32_t n_dq_units;  // dQ workgroups: B * N * nQB * ceil(bx / 128)
  int32_t slots_cap;   // partial-result slots for units split over several workgroups
  int32_t* plan;       // [0] entries per piece, [1] work items, [2] dQ order, [3] the persistent dK/dV
                       // kernel's item counter, unit_k[n_units], unit_base[n_units],
                       // slot_unit[slots_cap], slot_chunk[slots_cap], order_unit[n_units + slots_cap],
                       // order_piece[n_units + slots_cap], dq_order[n_dq_units],
                       // piece_done[n_units] (finished pieces of each split unit)
  float* partial;      // [slots_cap][2][kTileRowsMax][D] fp32 (dK unscaled, dV)
  // 1: the dQ kernel computes softmax_grad and lse2 (and writes them for the
  // dK/dV kernel, which then runs after it) and the prologue skips them;
  // 0 (the forward, and dQ by atomic adds): the prologue computes them
  int32_t fused_delta;
  // dQ by atomic adds (bsa_bwd_ex with BSA_DQ_ATOMIC; nullptr otherwise): fp32
  // [B][N][sq_max][D] of unscaled dS K sums, zeroed before the dK/dV kernel
  // adds into it and scaled, rounded and stored by the dQ launch
  float* dq_acc;
};

// Work-split parameters: a unit with more than `chunk` selecting Q blocks is
// split into ceil(T / piece) pieces, chunk = max(kMinChunk, ceil(total /
// kBalanceGroups)), piece = ceil(chunk / 2); at most kMaxSlots pieces exist
// in total, which that choice guarantees (pieces <= total / piece + split
// units <= 2 x kBalanceGroups + kBalanceGroups).
constexpr int kTileRowsMax = 128;

// Words (int32) of the plan region: 4 header words, then per unit its piece
// count and first slot, per slot its unit and piece, the launch order as
// two arrays (unit, piece) of n_units + slots entries, the dQ launch order
// (n_dq entries), and per unit a count of its finished pieces.
inline constexpr int64_t plan_words(int64_t n_units, int64_t slots, int64_t n_dq) {
  return 4 + 4 * (n_units + slots) + n_dq + n_units;
}
constexpr int kBalanceGroups = 256;
// Workgroups per dK/dV work item: 1, or 2 where dK and dV are accumulated by
// separate workgroups (head dim 256: K, V and both accumulators do not fit
// in one wave's registers).
inline constexpr int dkdv_passes(int D) { return D >= 256 ? 2 : 1; }
constexpr int kMinChunk = 4;
// The scheduled dK/dV build runs calls with head dim <= 128, no attenMask and
// at most kDkdvMaxGroup query heads per KV head (the group's list counts sit
// in LDS); the generic build runs the rest.
constexpr int kDkdvMaxGroup = 256;
inline constexpr bool dkdv_scheduled(int D, bool amask, int G) { return D <= 128 && !amask && G <= kDkdvMaxGroup; }
constexpr int kMaxSlots = 3 * kBalanceGroups;

// Launch-grid limits.  A dispatch counts work-items in 32 bits, so a grid of
// 256-thread workgroups holds at most kMaxGridGroups of them.
constexpr int64_t kMaxGridGroups = ((int64_t(1) << 32) - 1) / 256;

// Workgroups of the prologue launch: row lists (4 Q-block rows each), column
// lists (64 KV blocks each), softmax_grad (kDeltaRowsPerBlock consecutive
// positions of one (b, n) each).
constexpr int kDeltaRowsPerBlock = 64;
struct PrologueGrid {
  int64_t delta, rows, cols;
  int64_t total() const { return delta + rows + cols; }
};
inline PrologueGrid prologue_grid(int64_t B, int64_t N, int64_t sq_max, int64_t nqb, int64_t nkb, bool tnd) {
  PrologueGrid g;
  (void)tnd;  // the same 64-position runs of one (b, n) for both layouts
  g.delta = B * N * ((sq_max + kDeltaRowsPerBlock - 1) / kDeltaRowsPerBlock);
  g.rows = (B * N * nqb + 3) / 4;
  g.cols = B * N * ((nkb + 63) / 64);
  return g;
}

// Constant block staged with the sequence table: kZeroFloats zeros (rows past a
// slice's end are loaded from here), then +inf and -inf.
constexpr int kZeroFloats = 64;
constexpr int kConstFloats = kZeroFloats + 64;
constexpr int kConstPosInf = kZeroFloats;
constexpr int kConstNegInf = kZeroFloats + 1;

// Host-side description of the sequences (at most kMaxInlineSeq per staging launch).
constexpr int kMaxInlineSeq = 64;
struct SeqChunk {
  SeqInfo s[kMaxInlineSeq];
  int32_t first;
  int32_t count;
};

// fp8 -> bf16 staging: up to five tensors, each `n16` groups of 16 bytes,
// decoded into bf16 copies (exact: every E4M3FN and E5M2 value is a bf16
// value).  fmt: 0 = E4M3FN, 1 = E5M2.
constexpr int kMaxStaged = 5;
struct Fp8Stage {
  const uint8_t* src[kMaxStaged];
  uint16_t* dst[kMaxStaged];
  int64_t n16[kMaxStaged];
  int32_t fmt[kMaxStaged];
  int32_t count;
};

// Launch helpers (bsa_kernels.hip).  Return a hipError_t value (0 = success).
int launch_stage_fp8(const Fp8Stage& st, void* stream);
int launch_pack_amask(const Params& p, void* stream);  // attenMask -> am_rows / am_cols
int launch_stage_seq(const SeqChunk& chunk, SeqInfo* dst, void* stream);
int launch_prologue(const Params& p, void* stream);
int launch_plan(const Params& p, void* stream);
int launch_prologue_rows(const Params& p, void* stream);  // row lists only (the forward's)
int launch_fwd(const Params& p, void* stream);
int launch_dkdv(const Params& p, void* stream);
int launch_dq(const Params& p, void* stream);
int launch_dq_acc_zero(const Params& p, void* stream);  // dq_acc = 0 (atomic dQ mode)

// The library's own device scratch array, used as the workspace of the entry
// point that allocates nothing: its address on the current device (looked up
// once per device) and its size in bytes.  Returns a hipError_t value.
constexpr uint64_t kScratchBytes = uint64_t(64) << 20;  // BSA_NOALLOC_SCRATCH_BYTES
int scratch_region(void** ptr, uint64_t* bytes);

}  // namespace bsa
