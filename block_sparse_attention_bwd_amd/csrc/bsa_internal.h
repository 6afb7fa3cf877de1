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

  int64_t q_sb, q_sh, q_sr;    // query, attention_out, dout (identical, contiguous)
  int64_t kv_sb, kv_sh, kv_sr; // key, value
  int64_t dq_sb, dq_sh, dq_sr;
  int64_t dk_sb, dk_sh, dk_sr;
  int64_t dv_sb, dv_sh, dv_sr;
  int64_t lse_sb, lse_sh, lse_sr;

  int32_t B, N, Nkv, G, D;
  int32_t bx, by;      // block shape (Q rows, KV rows)
  int32_t nqb, nkb;    // mask block grid: ceil(maxSq/bx), ceil(maxSkv/by)
  int32_t sq_max;      // row extent of the delta/lse2 arrays
  int32_t dtype;       // bsa_dtype of the data tensors
  float scale;         // scale_value rounded to fp32
  float scale_log2e;   // scale * log2(e)

  // workspace regions
  SeqInfo* seq;
  const float* consts;  // kConstFloats floats after the sequence table: zeros, then +inf, -inf
  float* delta;
  float* lse2;
  int32_t* row_cnt;
  int32_t* row_list;
  int32_t* col_cnt;
  int32_t* col_list;
};

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

// Launch helpers (bsa_kernels.hip).  Return a hipError_t value (0 = success).
int launch_stage_seq(const SeqChunk& chunk, SeqInfo* dst, float* consts, void* stream);
int launch_prologue(const Params& p, void* stream);
int launch_dkdv(const Params& p, void* stream);
int launch_dq(const Params& p, void* stream);

}  // namespace bsa
