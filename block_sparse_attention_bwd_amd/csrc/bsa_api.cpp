// Host side of the C ABI declared in include/bsa_bwd.h: argument validation
// (aclnnBlockSparseAttentionGrad page, 参数说明 / 返回值 / 约束说明), the
// workspace plan, and the launch sequences of the backward and of the forward
// it differentiates, on the caller's stream.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "bsa_bwd.h"
#include "bsa_internal.h"

static_assert(bsa::kScratchBytes == BSA_NOALLOC_SCRATCH_BYTES, "scratch size in the header and the library");

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

constexpr int64_t kInt32Max = 2147483647;
constexpr int64_t kNoWindow = 2147483647;  // preTokens/nextTokens value meaning "no sliding window"
constexpr uint64_t kAlign = 256;

uint64_t align_up(uint64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Args {
  const bsa_tensor* dout;
  const bsa_tensor* query;
  const bsa_tensor* key;
  const bsa_tensor* value;
  const bsa_tensor* attention_out;
  const bsa_tensor* softmax_lse;
  const bsa_tensor* block_sparse_mask;
  const bsa_tensor* atten_mask;
  const int64_t* block_shape;
  int64_t block_shape_len;
  const int64_t* actual_seq_lengths;
  int64_t actual_seq_lengths_len;
  const int64_t* actual_seq_lengths_kv;
  int64_t actual_seq_lengths_kv_len;
  const char* q_input_layout;
  const char* kv_input_layout;
  int64_t num_key_value_heads;
  int64_t mask_type;
  double scale_value;
  int64_t pre_tokens;
  int64_t next_tokens;
  const bsa_tensor* dq;
  const bsa_tensor* dk;
  const bsa_tensor* dv;
  bool fwd;  // forward: dout/dq/dk/dv absent; attention_out and softmax_lse are outputs
  bool fp8;                // fp8 entry points: fp8 data inputs, bf16 outputs
  const double* descale;   // fp8: {dout, query, key, value, attention_out} or {query, key, value}; NULL = 1
  // partial-result slots for split dK/dV units: at most this many (fewer
  // only load-balance heavy units less well; results are the same)
  int64_t max_slots = bsa::kMaxSlots;
  int32_t dq_mode = BSA_DQ_RECOMPUTE;  // bsa_bwd_ex
};

enum Fp8Role { kRoleDout = 0, kRoleQuery, kRoleKey, kRoleValue, kRoleOut };

struct Plan {
  bsa::Params p{};
  std::vector<bsa::SeqInfo> seq;
  uint64_t off[BSA_WS_NUM] = {};
  int64_t dims[4] = {};
  bsa::Fp8Stage stage{};             // fp8: sources, formats and sizes (dst filled in at launch)
  uint64_t stage_off[bsa::kMaxStaged] = {};  // fp8: offset of each bf16 copy within BSA_WS_STAGE
  int stage_role[bsa::kMaxStaged] = {};  // which input each copy stands for (an Fp8Role)
};

bool row_major_contiguous(const bsa_tensor* t) {
  int64_t expect = 1;
  for (int d = t->ndim - 1; d >= 0; --d) {
    if (t->shape[d] != 1 && t->stride[d] != expect) return false;
    expect *= t->shape[d];
  }
  return true;
}

// No two index tuples of t map to one element: taking the dimensions of
// extent > 1 by ascending stride, each stride is at least the span of the
// dimensions before it.  (A zero stride on such a dimension fails.)  This
// accepts every layout torch makes by slicing, transposing or padding a
// contiguous tensor.
bool non_overlapping(const bsa_tensor* t) {
  int idx[4], m = 0;
  for (int d = 0; d < t->ndim; ++d)
    if (t->shape[d] > 1) idx[m++] = d;
  std::sort(idx, idx + m, [&](int x, int y) { return t->stride[x] < t->stride[y]; });
  int64_t span = 1;  // elements covered by the dimensions taken so far
  for (int i = 0; i < m; ++i) {
    const int d = idx[i];
    if (t->stride[d] < span) return false;
    span = t->stride[d] * (t->shape[d] - 1) + span;
  }
  return true;
}

const char* dtype_name(int32_t d) {
  switch (d) {
    case BSA_DTYPE_F16: return "float16";
    case BSA_DTYPE_BF16: return "bfloat16";
    case BSA_DTYPE_F32: return "float32";
    case BSA_DTYPE_BOOL: return "bool";
    case BSA_DTYPE_FP8_E4M3FN: return "float8_e4m3fn";
    case BSA_DTYPE_FP8_E5M2: return "float8_e5m2";
    default: return "unknown";
  }
}

int check_dims(const bsa_tensor* t, const char* name) {
  if (t->ndim < 1 || t->ndim > 4) return fail(BSA_ERR_PARAM_INVALID, "%s: ndim %d out of range", name, t->ndim);
  for (int d = 0; d < t->ndim; ++d) {
    if (t->shape[d] <= 0)
      return fail(BSA_ERR_PARAM_INVALID, "%s: dimension %d is %lld (empty tensors are not supported)", name, d,
                  static_cast<long long>(t->shape[d]));
    if (t->shape[d] > kInt32Max)
      return fail(BSA_ERR_PARAM_INVALID, "%s: dimension %d exceeds 2^31-1", name, d);
  }
  return BSA_OK;
}

bool same_shape(const bsa_tensor* a, const bsa_tensor* b) {
  if (a->ndim != b->ndim) return false;
  for (int d = 0; d < a->ndim; ++d)
    if (a->shape[d] != b->shape[d]) return false;
  return true;
}

int make_plan(const Args& a, Plan* plan) {
  // ---- null pointers (返回值: 161001) ------------------------------------
  struct Named {
    const bsa_tensor* t;
    const char* name;
  };
  const Named required_bwd[] = {{a.dout, "dout"},         {a.query, "query"},
                                {a.key, "key"},           {a.value, "value"},
                                {a.attention_out, "attentionOut"}, {a.softmax_lse, "softmaxLse"},
                                {a.dq, "dq"},             {a.dk, "dk"},
                                {a.dv, "dv"}};
  const Named required_fwd[] = {{a.query, "query"}, {a.key, "key"}, {a.value, "value"},
                                {a.attention_out, "attentionOut"}, {a.softmax_lse, "softmaxLse"}};
  const std::vector<Named> required = a.fwd ? std::vector<Named>(std::begin(required_fwd), std::end(required_fwd))
                                            : std::vector<Named>(std::begin(required_bwd), std::end(required_bwd));
  for (const Named& n : required) {
    if (n.t == nullptr) return fail(BSA_ERR_PARAM_NULLPTR, "%s is a null pointer", n.name);
    if (n.t->data == nullptr) return fail(BSA_ERR_PARAM_NULLPTR, "%s has a null data pointer", n.name);
  }
  if (a.block_sparse_mask != nullptr && a.block_sparse_mask->data == nullptr)
    return fail(BSA_ERR_PARAM_NULLPTR, "blockSparseMask has a null data pointer");
  if (a.q_input_layout == nullptr || a.kv_input_layout == nullptr)
    return fail(BSA_ERR_PARAM_NULLPTR, "input layout string is a null pointer");

  // ---- layouts ----------------------------------------------------------
  const bool q_tnd = std::strcmp(a.q_input_layout, "TND") == 0;
  const bool q_bnsd = std::strcmp(a.q_input_layout, "BNSD") == 0;
  const bool kv_tnd = std::strcmp(a.kv_input_layout, "TND") == 0;
  const bool kv_bnsd = std::strcmp(a.kv_input_layout, "BNSD") == 0;
  if (!(q_tnd || q_bnsd)) return fail(BSA_ERR_PARAM_INVALID, "qInputLayout '%s' is not BNSD or TND", a.q_input_layout);
  if (!(kv_tnd || kv_bnsd))
    return fail(BSA_ERR_PARAM_INVALID, "kvInputLayout '%s' is not BNSD or TND", a.kv_input_layout);
  if (q_tnd != kv_tnd) return fail(BSA_ERR_PARAM_INVALID, "qInputLayout and kvInputLayout differ");
  const bool tnd = q_tnd;
  if (tnd && a.actual_seq_lengths == nullptr)
    return fail(BSA_ERR_PARAM_NULLPTR, "TND layout needs actualSeqLengths");
  if (tnd && a.actual_seq_lengths_kv == nullptr)
    return fail(BSA_ERR_PARAM_NULLPTR, "TND layout needs actualSeqLengthsKv");

  // ---- dtypes -----------------------------------------------------------
  // (the kernels' element type: the data dtype, or bf16 for the fp8 entry
  // points, whose inputs are decoded to bf16 copies first)
  int32_t dt = a.query->dtype;
  double fac[5] = {1, 1, 1, 1, 1};  // fp8 dequantisation factors: dout, query, key, value, attentionOut
  if (a.fp8) {
    const Named fp8_in[] = {{a.fwd ? nullptr : a.dout, "dout"}, {a.query, "query"}, {a.key, "key"},
                            {a.value, "value"}, {a.fwd ? nullptr : a.attention_out, "attentionOut"}};
    for (const Named& n : fp8_in)
      if (n.t != nullptr && n.t->dtype != BSA_DTYPE_FP8_E4M3FN && n.t->dtype != BSA_DTYPE_FP8_E5M2)
        return fail(BSA_ERR_PARAM_INVALID, "%s dtype %s is not float8_e4m3fn/float8_e5m2", n.name,
                    dtype_name(n.t->dtype));
    const Named bf16_out[] = {{a.fwd ? a.attention_out : nullptr, "attentionOut"}, {a.dq, "dq"},
                              {a.dk, "dk"}, {a.dv, "dv"}};
    for (const Named& n : bf16_out)
      if (n.t != nullptr && n.t->dtype != BSA_DTYPE_BF16)
        return fail(BSA_ERR_PARAM_INVALID, "%s dtype %s is not bfloat16 (fp8 inputs give bf16 outputs)", n.name,
                    dtype_name(n.t->dtype));
    if (a.descale != nullptr) {
      const int n = a.fwd ? 3 : 5;
      for (int i = 0; i < n; ++i) {
        const double f = a.descale[i];
        if (!(std::isfinite(f) && f > 0))
          return fail(BSA_ERR_PARAM_INVALID, "descale[%d] must be finite and > 0", i);
        fac[a.fwd ? i + 1 : i] = f;
      }
    }
    dt = BSA_DTYPE_BF16;
  } else {
    if (dt != BSA_DTYPE_F16 && dt != BSA_DTYPE_BF16)
      return fail(BSA_ERR_PARAM_INVALID, "query dtype %s is not float16/bfloat16%s", dtype_name(dt),
                  dt == BSA_DTYPE_FP8_E4M3FN || dt == BSA_DTYPE_FP8_E5M2 ? " (fp8 inputs: the bsa_*_fp8 entry points)"
                                                                       : "");
    const Named same_dtype[] = {{a.dout, "dout"}, {a.key, "key"}, {a.value, "value"},
                                {a.attention_out, "attentionOut"}, {a.dq, "dq"},
                                {a.dk, "dk"}, {a.dv, "dv"}};
    for (const Named& n : same_dtype)
      if (n.t != nullptr && n.t->dtype != dt)
        return fail(BSA_ERR_PARAM_INVALID, "%s dtype %s differs from query dtype %s", n.name,
                    dtype_name(n.t->dtype), dtype_name(dt));
  }
  {  // inputs are read with 16-byte vector loads and copies
    const Named in16[] = {{a.fwd ? nullptr : a.dout, "dout"}, {a.query, "query"}, {a.key, "key"},
                          {a.value, "value"}, {a.fwd ? nullptr : a.attention_out, "attentionOut"}};
    for (const Named& n : in16)
      if (n.t != nullptr && reinterpret_cast<uintptr_t>(n.t->data) % 16 != 0)
        return fail(BSA_ERR_PARAM_INVALID, "%s data pointer is not 16-byte aligned", n.name);
  }
  if (a.softmax_lse->dtype != BSA_DTYPE_F32)
    return fail(BSA_ERR_PARAM_INVALID, "softmaxLse dtype %s is not float32", dtype_name(a.softmax_lse->dtype));
  if (a.block_sparse_mask && a.block_sparse_mask->dtype != BSA_DTYPE_BOOL)
    return fail(BSA_ERR_PARAM_INVALID, "blockSparseMask dtype %s is not bool/uint8",
                dtype_name(a.block_sparse_mask->dtype));

  // ---- reserved attributes ------------------------------------------------
  if (a.atten_mask != nullptr && a.atten_mask->data == nullptr)
    return fail(BSA_ERR_PARAM_NULLPTR, "attenMask has a null data pointer");
  if (a.atten_mask != nullptr && a.atten_mask->dtype != BSA_DTYPE_BOOL)
    return fail(BSA_ERR_PARAM_INVALID, "attenMask dtype %s is not bool/uint8", dtype_name(a.atten_mask->dtype));
  if (a.mask_type != 0) return fail(BSA_ERR_PARAM_INVALID, "maskType %lld is not supported (only 0)",
                                    static_cast<long long>(a.mask_type));

  if (!std::isfinite(a.scale_value)) return fail(BSA_ERR_PARAM_INVALID, "scaleValue is not finite");

  // ---- shapes -----------------------------------------------------------
  const Named all[] = {{a.dout, "dout"}, {a.query, "query"}, {a.key, "key"}, {a.value, "value"},
                       {a.attention_out, "attentionOut"}, {a.softmax_lse, "softmaxLse"},
                       {a.dq, "dq"}, {a.dk, "dk"}, {a.dv, "dv"}};
  for (const Named& n : all) {
    if (n.t == nullptr) continue;
    int rc = check_dims(n.t, n.name);
    if (rc) return rc;
  }
  const int want_nd = tnd ? 3 : 4;
  const Named data_t[] = {{a.dout, "dout"}, {a.query, "query"}, {a.key, "key"}, {a.value, "value"},
                          {a.attention_out, "attentionOut"}, {a.dq, "dq"}, {a.dk, "dk"}, {a.dv, "dv"}};
  for (const Named& n : data_t)
    if (n.t != nullptr && n.t->ndim != want_nd)
      return fail(BSA_ERR_PARAM_INVALID, "%s has %d dims; layout %s needs %d", n.name, n.t->ndim,
                  a.q_input_layout, want_nd);
  const Named qlike[] = {{a.dout, "dout"}, {a.attention_out, "attentionOut"}, {a.dq, "dq"}};
  for (const Named& n : qlike)
    if (n.t != nullptr && !same_shape(n.t, a.query)) return fail(BSA_ERR_PARAM_INVALID, "%s shape differs from query", n.name);
  const Named kvlike[] = {{a.value, "value"}, {a.dk, "dk"}, {a.dv, "dv"}};
  for (const Named& n : kvlike)
    if (n.t != nullptr && !same_shape(n.t, a.key)) return fail(BSA_ERR_PARAM_INVALID, "%s shape differs from key", n.name);

  const bsa_tensor* q = a.query;
  const bsa_tensor* k = a.key;
  int64_t B, N, Nkv, D, Sq = 0, Skv = 0, Tq = 0, Tkv = 0;
  if (tnd) {
    Tq = q->shape[0];
    N = q->shape[1];
    D = q->shape[2];
    Tkv = k->shape[0];
    Nkv = k->shape[1];
    if (k->shape[2] != D) return fail(BSA_ERR_PARAM_INVALID, "key head dim differs from query");
    B = a.actual_seq_lengths_len;
    if (B <= 0) return fail(BSA_ERR_PARAM_INVALID, "actualSeqLengths is empty");
    if (a.actual_seq_lengths_kv_len != B)
      return fail(BSA_ERR_PARAM_INVALID, "actualSeqLengths and actualSeqLengthsKv have different lengths");
  } else {
    B = q->shape[0];
    N = q->shape[1];
    Sq = q->shape[2];
    D = q->shape[3];
    if (k->shape[0] != B) return fail(BSA_ERR_PARAM_INVALID, "key batch differs from query");
    Nkv = k->shape[1];
    Skv = k->shape[2];
    if (k->shape[3] != D) return fail(BSA_ERR_PARAM_INVALID, "key head dim differs from query");
  }
  if (a.num_key_value_heads != Nkv)
    return fail(BSA_ERR_PARAM_INVALID, "numKeyValueHeads %lld does not match key's head count %lld",
                static_cast<long long>(a.num_key_value_heads), static_cast<long long>(Nkv));
  if (N < Nkv || N % Nkv != 0)
    return fail(BSA_ERR_PARAM_INVALID, "query heads %lld must be a multiple of KV heads %lld",
                static_cast<long long>(N), static_cast<long long>(Nkv));
  if (D != 64 && D != 128 && D != 256)
    return fail(BSA_ERR_PARAM_INVALID, "head dim %lld is not supported (64, 128 or 256)", static_cast<long long>(D));

  // ---- contiguity: inputs contiguous, outputs unit innermost stride ----------
  // (forward: attentionOut is an output with free outer strides; softmaxLse
  // is written densely, so it must be contiguous either way)
  const Named inputs[] = {{a.dout, "dout"}, {a.query, "query"}, {a.key, "key"}, {a.value, "value"},
                          {a.fwd ? nullptr : a.attention_out, "attentionOut"}, {a.softmax_lse, "softmaxLse"}};
  for (const Named& n : inputs)
    if (n.t != nullptr && !row_major_contiguous(n.t))
      return fail(BSA_ERR_PARAM_INVALID, "%s is not contiguous", n.name);
  const Named outputs[] = {{a.dq, "dq"}, {a.dk, "dk"}, {a.dv, "dv"}, {a.fwd ? a.attention_out : nullptr, "attentionOut"}};
  for (const Named& n : outputs) {
    if (n.t == nullptr) continue;
    if (n.t->stride[n.t->ndim - 1] != 1)
      return fail(BSA_ERR_PARAM_INVALID, "%s innermost stride must be 1", n.name);
    for (int d = 0; d < n.t->ndim - 1; ++d)
      if (n.t->stride[d] < 0) return fail(BSA_ERR_PARAM_INVALID, "%s has a negative stride", n.name);
    if (!non_overlapping(n.t))
      return fail(BSA_ERR_PARAM_INVALID,
                  "%s strides let two elements share an address (each output element is written once)", n.name);
  }
  if (a.fwd) {  // attention_out is stored four elements (8 bytes) at a time
    const bsa_tensor* o = a.attention_out;
    bool ok = reinterpret_cast<uintptr_t>(o->data) % 8 == 0;
    for (int d = 0; d < o->ndim - 1; ++d) ok = ok && o->stride[d] % 4 == 0;
    if (!ok)
      return fail(BSA_ERR_PARAM_INVALID,
                  "attentionOut: data pointer must be 8-byte aligned and outer strides multiples of 4 elements");
  }

  // ---- sequence lengths (参数说明: actualSeqLengths[Kv]Optional) ----------
  std::vector<int64_t> lq(B), lk(B);
  if (tnd) {
    int64_t sq = 0, sk = 0;
    for (int64_t b = 0; b < B; ++b) {
      lq[b] = a.actual_seq_lengths[b];
      lk[b] = a.actual_seq_lengths_kv[b];
      if (lq[b] < 0 || lk[b] < 0) return fail(BSA_ERR_PARAM_INVALID, "negative sequence length");
      sq += lq[b];
      sk += lk[b];
    }
    if (sq != Tq) return fail(BSA_ERR_PARAM_INVALID, "actualSeqLengths sum %lld != query tokens %lld",
                              static_cast<long long>(sq), static_cast<long long>(Tq));
    if (sk != Tkv) return fail(BSA_ERR_PARAM_INVALID, "actualSeqLengthsKv sum %lld != key tokens %lld",
                               static_cast<long long>(sk), static_cast<long long>(Tkv));
    for (int64_t b = 0; b < B; ++b) {
      Sq = lq[b] > Sq ? lq[b] : Sq;
      Skv = lk[b] > Skv ? lk[b] : Skv;
    }
  } else {
    for (int64_t b = 0; b < B; ++b) {
      lq[b] = Sq;
      lk[b] = Skv;
    }
    if (a.actual_seq_lengths != nullptr) {
      if (a.actual_seq_lengths_len != B)
        return fail(BSA_ERR_PARAM_INVALID, "actualSeqLengths has %lld entries, batch is %lld",
                    static_cast<long long>(a.actual_seq_lengths_len), static_cast<long long>(B));
      for (int64_t b = 0; b < B; ++b) {
        lq[b] = a.actual_seq_lengths[b];
        if (lq[b] < 0 || lq[b] > Sq) return fail(BSA_ERR_PARAM_INVALID, "actualSeqLengths[%lld] out of [0, S]",
                                                 static_cast<long long>(b));
      }
    }
    if (a.actual_seq_lengths_kv != nullptr) {
      if (a.actual_seq_lengths_kv_len != B)
        return fail(BSA_ERR_PARAM_INVALID, "actualSeqLengthsKv has %lld entries, batch is %lld",
                    static_cast<long long>(a.actual_seq_lengths_kv_len), static_cast<long long>(B));
      for (int64_t b = 0; b < B; ++b) {
        lk[b] = a.actual_seq_lengths_kv[b];
        if (lk[b] < 0 || lk[b] > Skv)
          return fail(BSA_ERR_PARAM_INVALID, "actualSeqLengthsKv[%lld] out of [0, S]", static_cast<long long>(b));
      }
    }
  }
  if (Sq <= 0 || Skv <= 0) return fail(BSA_ERR_PARAM_INVALID, "every sequence is empty");

  // ---- softmaxLse shape -----------------------------------------------------
  {
    const bsa_tensor* l = a.softmax_lse;
    const bool trailing1 = (l->ndim == (tnd ? 3 : 4)) && l->shape[l->ndim - 1] == 1;
    const int core = trailing1 ? l->ndim - 1 : l->ndim;
    bool ok;
    if (tnd) ok = (core == 2) && l->shape[0] == Tq && l->shape[1] == N;
    else ok = (core == 3) && l->shape[0] == B && l->shape[1] == N && l->shape[2] == Sq;
    if (!ok || (l->ndim != core && !trailing1))
      return fail(BSA_ERR_PARAM_INVALID, "softmaxLse shape must be %s", tnd ? "[T, N] or [T, N, 1]" : "[B, N, S] or [B, N, S, 1]");
  }

  // ---- block shape and mask (参数说明: blockShapeOptional, blockSparseMaskOptional) ----
  int64_t bx = 128, by = 128;
  if (a.block_sparse_mask != nullptr && a.block_shape != nullptr) {
    if (a.block_shape_len < 2) return fail(BSA_ERR_PARAM_INVALID, "blockShape needs at least two elements");
    bx = a.block_shape[0];
    by = a.block_shape[1];
    if (bx <= 0 || by <= 0) return fail(BSA_ERR_PARAM_INVALID, "blockShape elements must be > 0");
    if (bx > (int64_t(1) << 30) || by > (int64_t(1) << 30))
      return fail(BSA_ERR_PARAM_INVALID, "blockShape elements must be <= 2^30");
  }
  const int64_t nqb = ceil_div(Sq, bx), nkb = ceil_div(Skv, by);
  if (a.block_sparse_mask != nullptr) {
    const bsa_tensor* m = a.block_sparse_mask;
    int rc = check_dims(m, "blockSparseMask");
    if (rc) return rc;
    if (m->ndim != 4 || m->shape[0] != B || m->shape[1] != N || m->shape[2] != nqb || m->shape[3] != nkb)
      return fail(BSA_ERR_PARAM_INVALID,
                  "blockSparseMask shape must be [B, N, ceil(maxSq/bx), ceil(maxSkv/by)] = [%lld, %lld, %lld, %lld]",
                  static_cast<long long>(B), static_cast<long long>(N), static_cast<long long>(nqb),
                  static_cast<long long>(nkb));
    if (!row_major_contiguous(m)) return fail(BSA_ERR_PARAM_INVALID, "blockSparseMask is not contiguous");
  }
  if (a.atten_mask != nullptr) {  // [maxSq, maxSkv], sequence-local positions
    const bsa_tensor* m = a.atten_mask;
    int rc = check_dims(m, "attenMask");
    if (rc) return rc;
    if (m->ndim != 2 || m->shape[0] != Sq || m->shape[1] != Skv)
      return fail(BSA_ERR_PARAM_INVALID, "attenMask shape must be [maxSq, maxSkv] = [%lld, %lld]",
                  static_cast<long long>(Sq), static_cast<long long>(Skv));
    if (!row_major_contiguous(m)) return fail(BSA_ERR_PARAM_INVALID, "attenMask is not contiguous");
  }
  if (B * N * nqb * nkb > kInt32Max) return fail(BSA_ERR_PARAM_INVALID, "block grid too large for int32 lists");
  const int64_t nsub_q = ceil_div(bx, 128), nsub_kv = ceil_div(by, 128);
  if (B * N * nqb * nsub_q + bsa::kMaxSlots > bsa::kMaxGridGroups ||
      bsa::dkdv_passes(static_cast<int>(D)) * (B * Nkv * nkb * nsub_kv + bsa::kMaxSlots) > bsa::kMaxGridGroups ||
      bsa::prologue_grid(B, N, Sq, nqb, nkb, tnd).total() > bsa::kMaxGridGroups ||
      (tnd ? Sq * N : Sq) > kInt32Max)
    return fail(BSA_ERR_PARAM_INVALID, "launch grid too large (more than %lld workgroups)",
                static_cast<long long>(bsa::kMaxGridGroups));

  // ---- plan -----------------------------------------------------------------
  bsa::Params& p = plan->p;
  p = bsa::Params{};
  p.q = a.query->data;
  p.k = a.key->data;
  p.v = a.value->data;
  p.mask = a.block_sparse_mask ? static_cast<const uint8_t*>(a.block_sparse_mask->data) : nullptr;
  p.amask = a.atten_mask ? static_cast<const uint8_t*>(a.atten_mask->data) : nullptr;
  p.amask_ld = Skv;
  if (a.fwd) {
    p.out_o = a.attention_out->data;
    p.out_lse = static_cast<float*>(a.softmax_lse->data);
  } else {
    p.o = a.attention_out->data;
    p.dout = a.dout->data;
    p.lse = static_cast<const float*>(a.softmax_lse->data);
    p.dq = a.dq->data;
    p.dk = a.dk->data;
    p.dv = a.dv->data;
  }
  // strides of a q-like output: dq, or the forward's attention_out
  const bsa_tensor* qout = a.fwd ? a.attention_out : a.dq;
  const bsa_tensor* kout = a.fwd ? a.key : a.dk;  // dk/dv strides (unused by the forward)
  const bsa_tensor* vout = a.fwd ? a.value : a.dv;
  if (tnd) {
    p.q_sb = 0, p.q_sr = N * D, p.q_sh = D;
    p.kv_sb = 0, p.kv_sr = Nkv * D, p.kv_sh = D;
    p.dq_sb = 0, p.dq_sr = qout->stride[0], p.dq_sh = qout->stride[1];
    p.dk_sb = 0, p.dk_sr = kout->stride[0], p.dk_sh = kout->stride[1];
    p.dv_sb = 0, p.dv_sr = vout->stride[0], p.dv_sh = vout->stride[1];
    p.lse_sb = 0, p.lse_sr = N, p.lse_sh = 1;
  } else {
    p.q_sb = N * Sq * D, p.q_sh = Sq * D, p.q_sr = D;
    p.kv_sb = Nkv * Skv * D, p.kv_sh = Skv * D, p.kv_sr = D;
    p.dq_sb = qout->stride[0], p.dq_sh = qout->stride[1], p.dq_sr = qout->stride[2];
    p.dk_sb = kout->stride[0], p.dk_sh = kout->stride[1], p.dk_sr = kout->stride[2];
    p.dv_sb = vout->stride[0], p.dv_sh = vout->stride[1], p.dv_sr = vout->stride[2];
    p.lse_sb = N * Sq, p.lse_sh = Sq, p.lse_sr = 1;
  }
  p.o_sb = p.dq_sb, p.o_sh = p.dq_sh, p.o_sr = p.dq_sr;
  // the MFMA kernels address the rows of a tile (at most 128) from its first
  // row by 32-bit byte offsets
  if (2 * (128 * std::max(p.q_sr, p.kv_sr) + D) > 0xffffffffLL)
    return fail(BSA_ERR_PARAM_INVALID, "row stride of %lld elements too large for 32-bit tile offsets",
                static_cast<long long>(std::max(p.q_sr, p.kv_sr)));
  p.B = static_cast<int32_t>(B);
  p.N = static_cast<int32_t>(N);
  p.Nkv = static_cast<int32_t>(Nkv);
  p.G = static_cast<int32_t>(N / Nkv);
  p.D = static_cast<int32_t>(D);
  p.bx = static_cast<int32_t>(bx);
  p.by = static_cast<int32_t>(by);
  p.nqb = static_cast<int32_t>(nqb);
  p.nkb = static_cast<int32_t>(nkb);
  p.sq_max = static_cast<int32_t>(Sq);
  p.dtype = dt;
  p.tnd = tnd ? 1 : 0;
  // preTokens / nextTokens (参数说明): both 2147483647 = no window; otherwise the
  // window, clamped to +-(Sq + Skv + 1), which no position difference reaches
  if (a.pre_tokens != kNoWindow || a.next_tokens != kNoWindow) {
    const int64_t lim = std::min<int64_t>(Sq + Skv + 1, kInt32Max);
    p.win = 1;
    p.win_pre = static_cast<int32_t>(std::max(-lim, std::min(lim, a.pre_tokens)));
    p.win_next = static_cast<int32_t>(std::max(-lim, std::min(lim, a.next_tokens)));
  }
  p.scale = static_cast<float>(a.scale_value);
  {
    // fac: dout, query, key, value, attentionOut (all 1 without fp8 inputs)
    const double sc = a.scale_value;
    const double f[6] = {sc * fac[1] * fac[2] * 1.4426950408889634, sc * fac[0] * fac[3] * fac[2],
                         sc * fac[0] * fac[3] * fac[1], fac[0], fac[4] / fac[3], fac[3]};
    float* dst[6] = {&p.scale_log2e, &p.dq_scale, &p.dk_scale, &p.dv_scale, &p.delta_scale, &p.o_scale};
    for (int i = 0; i < 6; ++i) {
      *dst[i] = static_cast<float>(f[i]);
      if (a.fp8 && !(std::isfinite(*dst[i]) && std::fabs(*dst[i]) >= 1.1754944e-38f))
        return fail(BSA_ERR_PARAM_INVALID, "scaleValue and descale give a factor outside the fp32 normal range");
    }
    if (!a.fp8) p.o_scale = 1.f, p.delta_scale = 1.f, p.dv_scale = 1.f;  // exactly 1, not value / value
  }

  plan->seq.resize(B);
  int64_t oq = 0, ok = 0;
  for (int64_t b = 0; b < B; ++b) {
    bsa::SeqInfo& s = plan->seq[b];
    s.off_q = tnd ? oq : 0;
    s.off_kv = tnd ? ok : 0;
    s.len_q = static_cast<int32_t>(lq[b]);
    s.len_kv = static_cast<int32_t>(lk[b]);
    s.wlim_q = static_cast<int32_t>(tnd ? lq[b] : Sq);
    s.wlim_kv = static_cast<int32_t>(tnd ? lk[b] : Skv);
    oq += lq[b];
    ok += lk[b];
  }
  // one record for every sequence: no table to stage
  p.seq_uniform = !tnd && std::all_of(plan->seq.begin(), plan->seq.end(), [&](const bsa::SeqInfo& s) {
    return s.len_q == Sq && s.len_kv == Skv;
  });
  p.seq0 = bsa::SeqInfo{0, 0, static_cast<int32_t>(Sq), static_cast<int32_t>(Skv), static_cast<int32_t>(Sq),
                        static_cast<int32_t>(Skv)};

  // workspace regions (sizes from shapes, block shape and lengths only)
  uint64_t off = 0;
  auto take = [&](int region, uint64_t bytes) {
    plan->off[region] = off;
    off = align_up(off + bytes);
  };
  // (the forward needs only the sequence table and the row lists: the other
  // regions are empty)
  const uint64_t bwd = a.fwd ? 0 : 1;
  const uint64_t rows = static_cast<uint64_t>(B) * N * Sq;
  take(BSA_WS_SEQ, sizeof(bsa::SeqInfo) * static_cast<uint64_t>(B) + 4 * bsa::kConstFloats);
  take(BSA_WS_DELTA, bwd * 4 * rows);
  take(BSA_WS_LSE2, bwd * 4 * rows);
  take(BSA_WS_ROW_CNT, 4ull * B * N * nqb);
  take(BSA_WS_ROW_LIST, 4ull * B * N * nqb * nkb);
  take(BSA_WS_COL_CNT, bwd * 4ull * B * N * nkb);
  take(BSA_WS_COL_LIST, bwd * 4ull * B * N * nkb * nqb);
  const int64_t n_units = B * Nkv * nkb * nsub_kv;
  const int64_t max_pieces = n_units * (N / Nkv) * nqb;  // a piece holds at least one Q block
  const int64_t slots_lim = std::max<int64_t>(0, std::min<int64_t>(a.max_slots, bsa::kMaxSlots));
  const int64_t slots = max_pieces < slots_lim ? max_pieces : slots_lim;
  take(BSA_WS_PLAN, bwd * 4ull * bsa::plan_words(n_units, slots, B * N * nqb * nsub_q));
  take(BSA_WS_PARTIAL, bwd * 4ull * slots * 2 * bsa::kTileRowsMax * D);
  // attenMask as bits: by query row (all) and by key (the backward's dK/dV kernel)
  const bool am = a.atten_mask != nullptr;
  const uint64_t wk = static_cast<uint64_t>(ceil_div(Skv, 32)), wq = static_cast<uint64_t>(ceil_div(Sq, 32));
  take(BSA_WS_AMASK, am ? 4 * (static_cast<uint64_t>(Sq) * wk + bwd * static_cast<uint64_t>(Skv) * wq) : 0);
  if (am && (ceil_div(Sq, 64) * ceil_div(Skv, 64) + 3) / 4 > bsa::kMaxGridGroups)  // pack_amask: a 64 x 64 tile per wave
    return fail(BSA_ERR_PARAM_INVALID, "attenMask too large for one packing launch");
  p.am_wk = static_cast<int32_t>(wk);
  p.am_wq = static_cast<int32_t>(wq);
  // fp8: bf16 copies of the data inputs, each 256-byte aligned
  uint64_t stage_bytes = 0;
  if (a.fp8) {
    struct In {
      const bsa_tensor* t;
      int role;
    } ins[bsa::kMaxStaged] = {{a.fwd ? nullptr : a.dout, kRoleDout}, {a.query, kRoleQuery}, {a.key, kRoleKey},
                              {a.value, kRoleValue}, {a.fwd ? nullptr : a.attention_out, kRoleOut}};
    bsa::Fp8Stage& st = plan->stage;
    for (const In& in : ins) {
      if (in.t == nullptr) continue;
      uint64_t numel = 1;
      for (int d = 0; d < in.t->ndim; ++d) numel *= static_cast<uint64_t>(in.t->shape[d]);
      const int i = st.count++;
      st.src[i] = static_cast<const uint8_t*>(in.t->data);
      st.n16[i] = static_cast<int64_t>(numel / 16);  // numel is a multiple of D, hence of 16
      st.fmt[i] = in.t->dtype == BSA_DTYPE_FP8_E5M2 ? 1 : 0;
      plan->stage_off[i] = stage_bytes;
      plan->stage_role[i] = in.role;
      stage_bytes = align_up(stage_bytes + 2 * numel);
    }
    int64_t groups = 0;
    for (int i = 0; i < st.count; ++i) groups += st.n16[i];
    if ((groups + 255) / 256 > bsa::kMaxGridGroups)
      return fail(BSA_ERR_PARAM_INVALID, "fp8 inputs too large for one decode launch");
  }
  take(BSA_WS_STAGE, stage_bytes);
  // dQ by atomic adds: the fp32 accumulator, [B, N, maxSq, D]
  const bool dq_atomic = !a.fwd && a.dq_mode == BSA_DQ_ATOMIC;
  if (!a.fwd && a.dq_mode != BSA_DQ_RECOMPUTE && a.dq_mode != BSA_DQ_ATOMIC)
    return fail(BSA_ERR_PARAM_INVALID, "dq_mode %d is not BSA_DQ_RECOMPUTE (0) or BSA_DQ_ATOMIC (1)", a.dq_mode);
  if (dq_atomic) {
    if (a.fp8) return fail(BSA_ERR_PARAM_INVALID, "BSA_DQ_ATOMIC takes fp16/bf16 inputs");
    if (!bsa::dkdv_scheduled(static_cast<int>(D), am, static_cast<int>(N / Nkv)))
      return fail(BSA_ERR_PARAM_INVALID,
                  "BSA_DQ_ATOMIC needs head dim 64 or 128, no attenMask and at most %d query heads per KV head",
                  bsa::kDkdvMaxGroup);
    if (B * N * ceil_div(Sq, 64) + slots > bsa::kMaxGridGroups)
      return fail(BSA_ERR_PARAM_INVALID, "problem too large for the dQ store launch");
  }
  take(BSA_WS_DQ_ACC, dq_atomic ? 4ull * rows * D : 0);
  // the dQ kernel computes softmax_grad (and runs before dK/dV) unless dQ is
  // formed by atomic adds in the dK/dV kernel
  p.fused_delta = !a.fwd && !dq_atomic;
  plan->off[BSA_WS_TOTAL] = off;
  p.n_units = static_cast<int32_t>(n_units);
  p.n_dq_units = static_cast<int32_t>(B * N * nqb * nsub_q);
  p.slots_cap = static_cast<int32_t>(slots);
  plan->dims[0] = bx;
  plan->dims[1] = by;
  plan->dims[2] = nqb;
  plan->dims[3] = nkb;
  return BSA_OK;
}

// ---- plan dump (environment variable BSA_LOG=1) ---------------------------
// One block of text on stderr per validated call: what was decided from the
// arguments (sizes, block grid, work units, workspace regions, kernel shapes).
// Read on every call, so it can be switched on and off while a process runs.
bool plan_log_on() {
  const char* v = std::getenv("BSA_LOG");
  return v != nullptr && v[0] == '1';
}

void log_plan(const char* entry, const Args& a, const Plan& plan) {
  static const char* const kRegion[BSA_WS_NUM] = {"seq", "delta", "lse2", "row_cnt", "row_list", "col_cnt",
                                                  "col_list", "plan", "partial", "amask", "stage", "dq_acc",
                                                  "total"};
  const bsa::Params& p = plan.p;
  std::fprintf(stderr, "[bsa] %s: %s B=%d N=%d Nkv=%d G=%d D=%d dtype=%s maxSq=%d block=%dx%d nQB=%d nKB=%d\n",
               entry, p.tnd ? "TND" : "BNSD", p.B, p.N, p.Nkv, p.G, p.D, a.fp8 ? "fp8->bf16" : dtype_name(p.dtype),
               p.sq_max, p.bx, p.by, p.nqb, p.nkb);
  std::fprintf(stderr, "[bsa]   mask=%s attenMask=%s window=%s", p.mask ? "given" : "null (dense)",
               p.amask ? "given" : "none", p.win ? "" : "none");
  if (p.win) std::fprintf(stderr, "[-%d, +%d]", p.win_pre, p.win_next);
  std::fprintf(stderr, " scale=%.9g (scale*log2e=%.9g)\n", a.scale_value, static_cast<double>(p.scale_log2e));
  for (size_t b = 0; b < plan.seq.size() && b < 8; ++b)
    std::fprintf(stderr, "[bsa]   seq %zu: q[%lld +%d] kv[%lld +%d] writes %d / %d rows\n", b,
                 static_cast<long long>(plan.seq[b].off_q), plan.seq[b].len_q,
                 static_cast<long long>(plan.seq[b].off_kv), plan.seq[b].len_kv, plan.seq[b].wlim_q,
                 plan.seq[b].wlim_kv);
  if (plan.seq.size() > 8) std::fprintf(stderr, "[bsa]   ... %zu sequences in all\n", plan.seq.size());
  if (!a.fwd)
    std::fprintf(stderr, "[bsa]   dK/dV units=%d (+%d split slots, %d workgroup(s) per item)  dQ workgroups=%d%s\n",
                 p.n_units, p.slots_cap, bsa::dkdv_passes(p.D), p.n_dq_units,
                 a.dq_mode == BSA_DQ_ATOMIC ? " (dQ by atomic adds in the dK/dV kernel instead)" : "");
  else
    std::fprintf(stderr, "[bsa]   forward workgroups=%d\n", p.n_dq_units);
  for (int r = 0; r < BSA_WS_TOTAL; ++r) {
    const uint64_t sz = plan.off[r + 1] - plan.off[r];
    if (sz) std::fprintf(stderr, "[bsa]   ws %-8s @%-12llu %llu bytes\n", kRegion[r],
                         static_cast<unsigned long long>(plan.off[r]), static_cast<unsigned long long>(sz));
  }
  std::fprintf(stderr, "[bsa]   workspace total %llu bytes\n", static_cast<unsigned long long>(plan.off[BSA_WS_TOTAL]));
}

// ---- profiling -----------------------------------------------------------
constexpr int kStages = 4;
const char* const kStageNames[kStages] = {"prologue", "dkdv", "dq", "fwd"};
enum { kStagePrologue = 0, kStageDkdv, kStageDq, kStageFwd };
struct Profile {
  bool on = false;
  int max_calls = 0;
  std::vector<hipEvent_t> ev;  // per call: a start event, then one event after each stage run
  std::vector<int> tag;        // -1 for a call's start event, else the stage that event ends
} g_prof;

void free_profile_events() {
  for (hipEvent_t e : g_prof.ev) (void)hipEventDestroy(e);
  g_prof.ev.clear();
  g_prof.tag.clear();
}

int record_stage(hipStream_t s, int tag) {
  hipEvent_t e;
  if (hipEventCreate(&e) != hipSuccess) return fail(BSA_ERR_RUNTIME, "hipEventCreate failed");
  g_prof.ev.push_back(e);
  g_prof.tag.push_back(tag);
  if (hipEventRecord(e, s) != hipSuccess) return fail(BSA_ERR_RUNTIME, "hipEventRecord failed");
  return BSA_OK;
}

int check_device_pointer(const void* ptr, int device, const char* name) {
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, ptr);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(BSA_ERR_PARAM_INVALID, "%s is not device memory (%s)", name, hipGetErrorString(e));
  }
  if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged && attr.type != hipMemoryTypeUnified)
    return fail(BSA_ERR_PARAM_INVALID, "%s is not device memory", name);
  if (attr.type == hipMemoryTypeDevice && attr.device != device)
    return fail(BSA_ERR_PARAM_INVALID, "%s lives on device %d, the current device is %d", name, attr.device, device);
  return BSA_OK;
}

// The data tensors of a call live in device memory of the current device.
int check_tensors_on_device(const Args& a, int* device) {
  if (hipGetDevice(device) != hipSuccess) {
    (void)hipGetLastError();
    return fail(BSA_ERR_RUNTIME, "hipGetDevice failed (no usable GPU?)");
  }
  struct Ptr {
    const bsa_tensor* t;
    const char* name;
  };
  const Ptr ptrs[] = {{a.dout, "dout"}, {a.query, "query"}, {a.key, "key"},
                      {a.value, "value"}, {a.attention_out, "attentionOut"},
                      {a.softmax_lse, "softmaxLse"}, {a.block_sparse_mask, "blockSparseMask"},
                      {a.atten_mask, "attenMask"},
                      {a.dq, "dq"}, {a.dk, "dk"}, {a.dv, "dv"}};
  for (const Ptr& q : ptrs) {
    if (q.t == nullptr || q.t->data == nullptr) continue;
    int rc = check_device_pointer(q.t->data, *device, q.name);
    if (rc) return rc;
  }
  return BSA_OK;
}

int enqueue(const Args& a, Plan& plan, char* ws, void* stream, bool allow_profile);

// Validate, carve the caller's workspace and enqueue the kernels of one call.
int run(const Args& a, void* workspace, uint64_t workspace_size, void* stream) {
  Plan plan;
  int rc = make_plan(a, &plan);
  if (rc) return rc;
  if (plan_log_on()) log_plan(a.fwd ? "bsa_fwd" : "bsa_bwd", a, plan);
  const uint64_t need = plan.off[BSA_WS_TOTAL];
  if (workspace_size < need)
    return fail(BSA_ERR_PARAM_INVALID, "workspace of %llu bytes is smaller than the %llu needed",
                static_cast<unsigned long long>(workspace_size), static_cast<unsigned long long>(need));
  if (need > 0 && workspace == nullptr) return fail(BSA_ERR_PARAM_NULLPTR, "workspace is a null pointer");
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
    return fail(BSA_ERR_PARAM_INVALID, "workspace must be %llu-byte aligned", static_cast<unsigned long long>(kAlign));
  int device = -1;
  if ((rc = check_tensors_on_device(a, &device))) return rc;
  if (workspace != nullptr && (rc = check_device_pointer(workspace, device, "workspace"))) return rc;
  return enqueue(a, plan, static_cast<char*>(workspace), stream, true);
}

// The backward with the library's own scratch array as its workspace (see
// bsa_bwd_noalloc): the plan takes as many partial-result slots as fit.
int run_noalloc(const Args& a, void* stream) {
  void* base = nullptr;
  uint64_t cap = 0;
  const int herr = bsa::scratch_region(&base, &cap);
  if (herr) return fail(BSA_ERR_RUNTIME, "scratch lookup failed: %s", hipGetErrorString(static_cast<hipError_t>(herr)));
  Plan plan;
  Args b = a;
  int rc = make_plan(b, &plan);
  if (rc) return rc;
  if (plan.off[BSA_WS_TOTAL] > cap && plan.p.slots_cap > 0) {
    // the slots are the one region that may shrink: what is left after the
    // other regions, one slot at a time (each also takes 8 plan bytes)
    b.max_slots = 0;
    if ((rc = make_plan(b, &plan))) return rc;
    const uint64_t per_slot = 2ull * bsa::kTileRowsMax * static_cast<uint64_t>(plan.p.D) * 4 + 8;
    b.max_slots = plan.off[BSA_WS_TOTAL] < cap ? static_cast<int64_t>((cap - plan.off[BSA_WS_TOTAL]) / per_slot) : 0;
    for (;;) {
      if ((rc = make_plan(b, &plan))) return rc;
      if (plan.off[BSA_WS_TOTAL] <= cap || b.max_slots == 0) break;
      b.max_slots = b.max_slots > 8 ? b.max_slots - 8 : 0;  // alignment padding of the regions
    }
  }
  if (plan_log_on()) log_plan("bsa_bwd_noalloc", b, plan);
  if (plan.off[BSA_WS_TOTAL] > cap)
    return fail(BSA_ERR_PARAM_INVALID,
                "this problem needs %llu bytes of workspace; the library's scratch array holds %llu "
                "(use bsa_bwd with a caller workspace)",
                static_cast<unsigned long long>(plan.off[BSA_WS_TOTAL]), static_cast<unsigned long long>(cap));
  int device = -1;
  if ((rc = check_tensors_on_device(b, &device))) return rc;
  return enqueue(b, plan, static_cast<char*>(base), stream, false);
}

// Carve the workspace at `ws` by the plan and enqueue the stages.
int enqueue(const Args& a, Plan& plan, char* ws, void* stream, bool allow_profile) {
  int rc = BSA_OK;
  bsa::Params& p = plan.p;
  p.seq = reinterpret_cast<bsa::SeqInfo*>(ws + plan.off[BSA_WS_SEQ]);
  float* consts = reinterpret_cast<float*>(ws + plan.off[BSA_WS_SEQ] + sizeof(bsa::SeqInfo) * plan.seq.size());
  p.consts = consts;
  p.row_cnt = reinterpret_cast<int32_t*>(ws + plan.off[BSA_WS_ROW_CNT]);
  p.row_list = reinterpret_cast<int32_t*>(ws + plan.off[BSA_WS_ROW_LIST]);
  if (!a.fwd) {
    p.delta = reinterpret_cast<float*>(ws + plan.off[BSA_WS_DELTA]);
    p.lse2 = reinterpret_cast<float*>(ws + plan.off[BSA_WS_LSE2]);
    p.col_cnt = reinterpret_cast<int32_t*>(ws + plan.off[BSA_WS_COL_CNT]);
    p.col_list = reinterpret_cast<int32_t*>(ws + plan.off[BSA_WS_COL_LIST]);
    p.plan = reinterpret_cast<int32_t*>(ws + plan.off[BSA_WS_PLAN]);
    p.partial = reinterpret_cast<float*>(ws + plan.off[BSA_WS_PARTIAL]);
    p.dq_acc = a.dq_mode == BSA_DQ_ATOMIC ? reinterpret_cast<float*>(ws + plan.off[BSA_WS_DQ_ACC]) : nullptr;
  }
  if (p.amask) {
    p.am_rows = reinterpret_cast<uint32_t*>(ws + plan.off[BSA_WS_AMASK]);
    p.am_cols = a.fwd ? nullptr : p.am_rows + static_cast<uint64_t>(p.sq_max) * p.am_wk;
  }

  // Profiling: one event before the first stage and one after each stage run.
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool prof = allow_profile && g_prof.on && g_prof.max_calls > 0;
  if (prof) --g_prof.max_calls;
  auto mark = [&](int tag) { return prof ? record_stage(s, tag) : static_cast<int>(BSA_OK); };
  auto launch_failed = [&](int herr, const char* what) {
    return fail(BSA_ERR_RUNTIME, "%s launch failed: %s", what, hipGetErrorString(static_cast<hipError_t>(herr)));
  };
  if ((rc = mark(-1))) return rc;
  int herr = 0;
  if (a.fp8) {  // decode the fp8 inputs into their bf16 copies; the kernels read those
    bsa::Fp8Stage st = plan.stage;
    for (int i = 0; i < st.count; ++i) {
      st.dst[i] = reinterpret_cast<uint16_t*>(ws + plan.off[BSA_WS_STAGE] + plan.stage_off[i]);
      const void* copy = st.dst[i];
      switch (plan.stage_role[i]) {
        case kRoleDout: p.dout = copy; break;
        case kRoleQuery: p.q = copy; break;
        case kRoleKey: p.k = copy; break;
        case kRoleValue: p.v = copy; break;
        default: p.o = copy; break;
      }
    }
    if ((herr = bsa::launch_stage_fp8(st, stream))) return launch_failed(herr, "fp8 decode");
  }
  // the sequence table (not needed when every sequence has the same record)
  for (size_t first = 0; !p.seq_uniform && first < plan.seq.size() && herr == 0; first += bsa::kMaxInlineSeq) {
    bsa::SeqChunk chunk{};
    chunk.first = static_cast<int32_t>(first);
    chunk.count = static_cast<int32_t>(std::min<size_t>(bsa::kMaxInlineSeq, plan.seq.size() - first));
    for (int i = 0; i < chunk.count; ++i) chunk.s[i] = plan.seq[first + i];
    herr = bsa::launch_stage_seq(chunk, p.seq, stream);
  }
  if (herr == 0 && p.amask) herr = bsa::launch_pack_amask(p, stream);
  if (a.fwd) {
    if (herr == 0) herr = bsa::launch_prologue_rows(p, stream);
    if (herr) return launch_failed(herr, "prologue");
    if ((rc = mark(kStagePrologue))) return rc;
    if ((herr = bsa::launch_fwd(p, stream))) return launch_failed(herr, "forward");
    return mark(kStageFwd);
  }
  if (herr == 0) herr = bsa::launch_prologue(p, stream);
  if (herr == 0) herr = bsa::launch_plan(p, stream);
  if (herr == 0 && p.dq_acc) herr = bsa::launch_dq_acc_zero(p, stream);
  if (herr) return launch_failed(herr, "prologue");
  if ((rc = mark(kStagePrologue))) return rc;
  if (p.fused_delta) {  // dQ first: it writes the softmax_grad rows the dK/dV kernel reads
    if ((herr = bsa::launch_dq(p, stream))) return launch_failed(herr, "dQ");
    if ((rc = mark(kStageDq))) return rc;
    if ((herr = bsa::launch_dkdv(p, stream))) return launch_failed(herr, "dK/dV");
    return mark(kStageDkdv);
  }
  if ((herr = bsa::launch_dkdv(p, stream))) return launch_failed(herr, "dK/dV");
  if ((rc = mark(kStageDkdv))) return rc;
  if ((herr = bsa::launch_dq(p, stream))) return launch_failed(herr, "dQ");
  return mark(kStageDq);
}

}  // namespace

#define BSA_FWD_ARGS_DECL                                                                           \
  const bsa_tensor *query, const bsa_tensor *key, const bsa_tensor *value,                          \
      const bsa_tensor *block_sparse_mask, const bsa_tensor *atten_mask, const int64_t *block_shape, \
      int64_t block_shape_len, const int64_t *actual_seq_lengths, int64_t actual_seq_lengths_len,   \
      const int64_t *actual_seq_lengths_kv, int64_t actual_seq_lengths_kv_len,                      \
      const char *q_input_layout, const char *kv_input_layout, int64_t num_key_value_heads,         \
      int64_t mask_type, double scale_value, int64_t pre_tokens, int64_t next_tokens,               \
      const bsa_tensor *attention_out, const bsa_tensor *softmax_lse

#define BSA_FWD_ARGS_PACK                                                                          \
  Args {                                                                                           \
    nullptr, query, key, value, attention_out, softmax_lse, block_sparse_mask, atten_mask,         \
        block_shape, block_shape_len, actual_seq_lengths, actual_seq_lengths_len,                  \
        actual_seq_lengths_kv, actual_seq_lengths_kv_len, q_input_layout, kv_input_layout,         \
        num_key_value_heads, mask_type, scale_value, pre_tokens, next_tokens, nullptr, nullptr,    \
        nullptr, true                                                                              \
  }

#define BSA_ARGS_DECL                                                                               \
  const bsa_tensor *dout, const bsa_tensor *query, const bsa_tensor *key, const bsa_tensor *value,  \
      const bsa_tensor *attention_out, const bsa_tensor *softmax_lse,                               \
      const bsa_tensor *block_sparse_mask, const bsa_tensor *atten_mask, const int64_t *block_shape, \
      int64_t block_shape_len, const int64_t *actual_seq_lengths, int64_t actual_seq_lengths_len,   \
      const int64_t *actual_seq_lengths_kv, int64_t actual_seq_lengths_kv_len,                      \
      const char *q_input_layout, const char *kv_input_layout, int64_t num_key_value_heads,         \
      int64_t mask_type, double scale_value, int64_t pre_tokens, int64_t next_tokens,               \
      const bsa_tensor *dq, const bsa_tensor *dk, const bsa_tensor *dv

#define BSA_ARGS_PACK                                                                              \
  Args {                                                                                           \
    dout, query, key, value, attention_out, softmax_lse, block_sparse_mask, atten_mask,            \
        block_shape, block_shape_len, actual_seq_lengths, actual_seq_lengths_len,                  \
        actual_seq_lengths_kv, actual_seq_lengths_kv_len, q_input_layout, kv_input_layout,         \
        num_key_value_heads, mask_type, scale_value, pre_tokens, next_tokens, dq, dk, dv, false    \
  }

extern "C" {

int bsa_bwd_workspace_size(BSA_ARGS_DECL, uint64_t* workspace_size) {
  g_err.clear();
  if (workspace_size == nullptr) return fail(BSA_ERR_PARAM_NULLPTR, "workspaceSize is a null pointer");
  Plan plan;
  const Args a = BSA_ARGS_PACK;
  int rc = make_plan(a, &plan);
  if (rc) return rc;
  if (plan_log_on()) log_plan("bsa_bwd_workspace_size", a, plan);
  *workspace_size = plan.off[BSA_WS_TOTAL];
  return BSA_OK;
}

int bsa_bwd_workspace_layout(BSA_ARGS_DECL, uint64_t* offsets, int64_t* dims) {
  g_err.clear();
  if (offsets == nullptr) return fail(BSA_ERR_PARAM_NULLPTR, "offsets is a null pointer");
  Plan plan;
  int rc = make_plan(BSA_ARGS_PACK, &plan);
  if (rc) return rc;
  for (int i = 0; i < BSA_WS_NUM; ++i) offsets[i] = plan.off[i];
  if (dims)
    for (int i = 0; i < 4; ++i) dims[i] = plan.dims[i];
  return BSA_OK;
}

int bsa_bwd(BSA_ARGS_DECL, void* workspace, uint64_t workspace_size, void* stream) {
  g_err.clear();
  return run(BSA_ARGS_PACK, workspace, workspace_size, stream);
}

int bsa_bwd_ex_workspace_size(BSA_ARGS_DECL, int32_t dq_mode, uint64_t* workspace_size) {
  g_err.clear();
  if (workspace_size == nullptr) return fail(BSA_ERR_PARAM_NULLPTR, "workspaceSize is a null pointer");
  Plan plan;
  Args a = BSA_ARGS_PACK;
  a.dq_mode = dq_mode;
  int rc = make_plan(a, &plan);
  if (rc) return rc;
  if (plan_log_on()) log_plan("bsa_bwd_ex_workspace_size", a, plan);
  *workspace_size = plan.off[BSA_WS_TOTAL];
  return BSA_OK;
}

int bsa_bwd_ex(BSA_ARGS_DECL, int32_t dq_mode, void* workspace, uint64_t workspace_size, void* stream) {
  g_err.clear();
  Args a = BSA_ARGS_PACK;
  a.dq_mode = dq_mode;
  return run(a, workspace, workspace_size, stream);
}

int bsa_bwd_noalloc(BSA_ARGS_DECL, void* stream) {
  g_err.clear();
  return run_noalloc(BSA_ARGS_PACK, stream);
}

int bsa_fwd_workspace_size(BSA_FWD_ARGS_DECL, uint64_t* workspace_size) {
  g_err.clear();
  if (workspace_size == nullptr) return fail(BSA_ERR_PARAM_NULLPTR, "workspaceSize is a null pointer");
  Plan plan;
  const Args a = BSA_FWD_ARGS_PACK;
  int rc = make_plan(a, &plan);
  if (rc) return rc;
  if (plan_log_on()) log_plan("bsa_fwd_workspace_size", a, plan);
  *workspace_size = plan.off[BSA_WS_TOTAL];
  return BSA_OK;
}

int bsa_fwd(BSA_FWD_ARGS_DECL, void* workspace, uint64_t workspace_size, void* stream) {
  g_err.clear();
  return run(BSA_FWD_ARGS_PACK, workspace, workspace_size, stream);
}

int bsa_bwd_fp8_workspace_size(BSA_ARGS_DECL, const double* descale, uint64_t* workspace_size) {
  g_err.clear();
  if (workspace_size == nullptr) return fail(BSA_ERR_PARAM_NULLPTR, "workspaceSize is a null pointer");
  Args a = BSA_ARGS_PACK;
  a.fp8 = true;
  a.descale = descale;
  Plan plan;
  int rc = make_plan(a, &plan);
  if (rc) return rc;
  *workspace_size = plan.off[BSA_WS_TOTAL];
  return BSA_OK;
}

int bsa_bwd_fp8(BSA_ARGS_DECL, const double* descale, void* workspace, uint64_t workspace_size, void* stream) {
  g_err.clear();
  Args a = BSA_ARGS_PACK;
  a.fp8 = true;
  a.descale = descale;
  return run(a, workspace, workspace_size, stream);
}

int bsa_fwd_fp8_workspace_size(BSA_FWD_ARGS_DECL, const double* descale, uint64_t* workspace_size) {
  g_err.clear();
  if (workspace_size == nullptr) return fail(BSA_ERR_PARAM_NULLPTR, "workspaceSize is a null pointer");
  Args a = BSA_FWD_ARGS_PACK;
  a.fp8 = true;
  a.descale = descale;
  Plan plan;
  int rc = make_plan(a, &plan);
  if (rc) return rc;
  *workspace_size = plan.off[BSA_WS_TOTAL];
  return BSA_OK;
}

int bsa_fwd_fp8(BSA_FWD_ARGS_DECL, const double* descale, void* workspace, uint64_t workspace_size,
                void* stream) {
  g_err.clear();
  Args a = BSA_FWD_ARGS_PACK;
  a.fp8 = true;
  a.descale = descale;
  return run(a, workspace, workspace_size, stream);
}

const char* bsa_last_error(void) { return g_err.c_str(); }

int bsa_profile_start(int32_t max_calls) {
  g_err.clear();
  if (max_calls <= 0) return fail(BSA_ERR_PARAM_INVALID, "max_calls must be > 0");
  free_profile_events();
  g_prof.on = true;
  g_prof.max_calls = max_calls;
  g_prof.ev.reserve(static_cast<size_t>(max_calls) * (kStages + 1));
  g_prof.tag.reserve(static_cast<size_t>(max_calls) * (kStages + 1));
  return BSA_OK;
}

int bsa_profile_stop(double* stage_ms, int32_t n_stages, int32_t* n_calls) {
  g_err.clear();
  int rc = BSA_OK;
  int calls = 0;
  if (stage_ms)
    for (int i = 0; i < n_stages; ++i) stage_ms[i] = 0.0;
  if (!g_prof.ev.empty() && hipEventSynchronize(g_prof.ev.back()) != hipSuccess)
    rc = fail(BSA_ERR_RUNTIME, "hipEventSynchronize failed");
  for (size_t i = 0; i < g_prof.ev.size() && rc == BSA_OK; ++i) {
    const int st = g_prof.tag[i];
    if (st < 0) {
      ++calls;
      continue;
    }
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, g_prof.ev[i - 1], g_prof.ev[i]) != hipSuccess) {
      rc = fail(BSA_ERR_RUNTIME, "hipEventElapsedTime failed");
      break;
    }
    if (stage_ms && st < n_stages) stage_ms[st] += ms;
  }
  if (n_calls) *n_calls = calls;
  free_profile_events();
  g_prof.on = false;
  g_prof.max_calls = 0;
  return rc;
}

const char* bsa_stage_name(int32_t stage) {
  if (stage < 0 || stage >= kStages) return nullptr;
  return kStageNames[stage];
}

}  // extern "C"
