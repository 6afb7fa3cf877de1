/*
 * bsa_bwd.h -- C ABI of the block-sparse attention backward for AMD MI355X (gfx950).
 *
 * Operation (aclnnBlockSparseAttentionGrad page, 功能说明 / 计算公式): given the
 * forward S = Mask(scale * Q * K_sparse^T), P = Softmax(S), Out = P * V_sparse,
 * compute
 *     softmax_grad_i = sum_d dOut[i,d] * Out[i,d]          (row sum of dOut o Out)
 *     P              = exp(scale * Q * K^T - softmaxLse)    on selected blocks only
 *     dP             = dOut * V^T
 *     dS             = P o (dP - softmax_grad)              (element-wise)
 *     dV             = P^T * dOut
 *     dQ             = (dS * K) * scale
 *     dK             = (dS^T * Q) * scale
 * where the block mask picks, for every Q block of blockShape[0] rows, the KV
 * blocks of blockShape[1] rows that take part (and an optional sliding window
 * further restricts each row to a band of keys); everything outside is
 * excluded from the softmax and contributes nothing.  With GQA, query
 * head n reads KV head n / (N / Nkv) and dK/dV sum over the query heads of a
 * group (in ascending head order, so results are run-to-run bitwise identical).
 *
 * Two-phase use, mirroring the page's prototypes (函数原型):
 *   1. bsa_bwd_workspace_size(...)  -- host only: validates every argument and
 *      returns the device workspace size the call needs (a function of the
 *      shapes, block shape and sequence lengths only; never of the mask values).
 *   2. bsa_bwd(..., workspace, workspace_size, stream) -- re-validates, then
 *      enqueues the kernels on `stream` and returns without synchronising.
 *
 * Ownership: the caller owns every device buffer (inputs, dq/dk/dv, workspace)
 * and the stream.  The library allocates no device memory, frees nothing and
 * never synchronises the stream.  Host arrays (block_shape, actual_seq_*) and
 * strings are read only during the call.  All tensors passed to bsa_bwd must
 * live in device memory of the current HIP device, and the data pointers of the
 * input tensors (dout, query, key, value, attention_out) must be 16-byte
 * aligned (161002 otherwise).  Every element of dq/dk/dv
 * is written (zeros where nothing contributes: padded BNSD rows, query rows
 * that select no key, keys no row selects), so outputs need no pre-zeroing.
 * Calls on different streams that share a workspace race; give each in-flight
 * call its own workspace.
 *
 * Error behaviour: every entry point returns BSA_OK or one of the bsa_status
 * codes below; on a non-zero status nothing has been enqueued and
 * bsa_last_error() (thread-local) describes the first failed check.
 *
 * Diagnostics: with the environment variable BSA_LOG=1 (read on every call),
 * each call that passes validation (workspace-size queries included) writes
 * its plan to stderr: sizes, block grid, sequence table, work units and the
 * workspace regions with their offsets and sizes.
 */
#ifndef BSA_BWD_H
#define BSA_BWD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types (参数说明 table: FLOAT16/BFLOAT16 data, FLOAT LSE, BOOL mask). */
enum bsa_dtype {
  BSA_DTYPE_F16 = 1,
  BSA_DTYPE_BF16 = 2,
  BSA_DTYPE_F32 = 3,
  BSA_DTYPE_BOOL = 4, /* one byte per element, nonzero = selected (UINT8 accepted) */
  /* 8-bit floats (the page's FLOAT8_E4M3FN / FLOAT8_E5M2, OCP encodings);
   * taken only by the bsa_*_fp8 entry points */
  BSA_DTYPE_FP8_E4M3FN = 5, /* sign, 4 exponent bits (bias 7), 3 mantissa bits; no inf, NaN = 0x7f/0xff */
  BSA_DTYPE_FP8_E5M2 = 6    /* sign, 5 exponent bits (bias 15), 2 mantissa bits; IEEE inf/NaN */
};

/* Status codes (返回值 table of the page; runtime/inner codes of the same family). */
enum bsa_status {
  BSA_OK = 0,
  BSA_ERR_PARAM_NULLPTR = 161001, /* a required tensor/pointer is NULL; TND without lengths */
  BSA_ERR_PARAM_INVALID = 161002, /* dtype, layout, shape, stride, attribute or size invalid */
  BSA_ERR_RUNTIME = 361001,       /* a HIP call failed (launch, pointer query, event) */
  BSA_ERR_INNER = 561002          /* internal planning failure */
};

/* Non-owning tensor descriptor.  `data` is a device pointer; shape and stride
 * are in elements, outermost first; only the first `ndim` entries are read. */
typedef struct bsa_tensor {
  void* data;
  int32_t dtype; /* enum bsa_dtype */
  int32_t ndim;  /* 1..4 */
  int64_t shape[4];
  int64_t stride[4];
} bsa_tensor;

/*
 * Phase 1: validate and size the workspace.  Arguments in the page's order
 * (参数说明 of aclnnBlockSparseAttentionGradGetWorkspaceSize):
 *
 *  dout, query, attention_out  [B, N, Sq, D] (BNSD) or [Tq, N, D] (TND); fp16/bf16,
 *                              contiguous.  All eight data tensors share one dtype.
 *  key, value                  [B, Nkv, Skv, D] or [Tkv, Nkv, D]; contiguous.
 *  softmax_lse                 fp32 [B, N, Sq] or [B, N, Sq, 1] (BNSD),
 *                              [Tq, N] or [Tq, N, 1] (TND); natural-log
 *                              log-sum-exp of the scaled scores; contiguous.
 *  block_sparse_mask           bool/uint8 [B, N, ceil(maxSq/bx), ceil(maxSkv/by)],
 *                              contiguous; NULL = every block selected.
 *  atten_mask                  optional element mask (参数说明 attenMaskOptional, BOOL,
 *                              2 dims): bool/uint8 [maxSq, maxSkv], contiguous,
 *                              1 = the pair does not take part (the FlashAttentionScore
 *                              page's polarity); shared by every batch and head and
 *                              indexed by sequence-local positions.  NULL = none.
 *  block_shape, _len           {bx, by} (first two entries used, each > 0);
 *                              NULL = {128, 128}.  Ignored without a mask.
 *  actual_seq_lengths(_kv), _len
 *                              per-sequence token counts, length B.  Required
 *                              for TND (sums must equal Tq / Tkv); optional for
 *                              BNSD (each in [0, S]; padding past it is ignored
 *                              and its outputs are zero).
 *  q_input_layout, kv_input_layout   "BNSD" or "TND", equal.
 *  num_key_value_heads         Nkv; N >= Nkv and N % Nkv == 0 (约束说明).
 *  mask_type                   must be 0 (the only mask type the page defines).
 *  scale_value                 the scale (typically D^-0.5); finite.
 *  pre_tokens, next_tokens     sliding window (参数说明 preTokens / nextTokens: how
 *                              many earlier / later tokens a token may attend to):
 *                              key j takes part for query i only if
 *                              i - pre_tokens <= j <= i + next_tokens, positions
 *                              sequence-local from 0.  Both 2147483647 = no window;
 *                              any int64 otherwise (a window that leaves a row no
 *                              key gives that row LSE = -inf and zero outputs).
 *  dq, dk, dv                  outputs, same dtype/shape as query/key/value;
 *                              any outer strides, innermost stride 1, no two
 *                              elements at one address (zero or overlapping
 *                              strides are rejected with 161002).
 *  workspace_size              out: bytes of device workspace needed.
 *
 * Head dim D must be 64, 128 or 256 (the tile set built into this library;
 * the pages' own implementation takes 128 only, the FlashAttentionScore page
 * allows up to 512).  The kernels address the rows of a tile from its first
 * row by 32-bit byte offsets: a row stride (D for BNSD, N * D or Nkv * D for
 * TND) above (2^31 - D) / 128 elements is rejected with 161002.
 */
int bsa_bwd_workspace_size(const bsa_tensor* dout, const bsa_tensor* query, const bsa_tensor* key,
                           const bsa_tensor* value, const bsa_tensor* attention_out,
                           const bsa_tensor* softmax_lse, const bsa_tensor* block_sparse_mask,
                           const bsa_tensor* atten_mask, const int64_t* block_shape,
                           int64_t block_shape_len, const int64_t* actual_seq_lengths,
                           int64_t actual_seq_lengths_len, const int64_t* actual_seq_lengths_kv,
                           int64_t actual_seq_lengths_kv_len, const char* q_input_layout,
                           const char* kv_input_layout, int64_t num_key_value_heads,
                           int64_t mask_type, double scale_value, int64_t pre_tokens,
                           int64_t next_tokens, const bsa_tensor* dq, const bsa_tensor* dk,
                           const bsa_tensor* dv, uint64_t* workspace_size);

/*
 * Phase 2 (aclnnBlockSparseAttentionGrad): same arguments, then the device
 * workspace (at least the size phase 1 returned, 256-byte aligned; may be NULL
 * only if that size is 0) and the hipStream_t to enqueue on (NULL = the null
 * stream).  Returns after enqueueing; completion is observed through the stream.
 */
int bsa_bwd(const bsa_tensor* dout, const bsa_tensor* query, const bsa_tensor* key,
            const bsa_tensor* value, const bsa_tensor* attention_out, const bsa_tensor* softmax_lse,
            const bsa_tensor* block_sparse_mask, const bsa_tensor* atten_mask,
            const int64_t* block_shape, int64_t block_shape_len, const int64_t* actual_seq_lengths,
            int64_t actual_seq_lengths_len, const int64_t* actual_seq_lengths_kv,
            int64_t actual_seq_lengths_kv_len, const char* q_input_layout,
            const char* kv_input_layout, int64_t num_key_value_heads, int64_t mask_type,
            double scale_value, int64_t pre_tokens, int64_t next_tokens, const bsa_tensor* dq,
            const bsa_tensor* dk, const bsa_tensor* dv, void* workspace, uint64_t workspace_size,
            void* stream);

/*
 * The backward without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments and results as bsa_bwd without
 * workspace / workspace_size; the stages run on the library's own static
 * device scratch array of 64 MiB (BSA_NOALLOC_SCRATCH_BYTES), one copy per GPU,
 * held from the library's first use on that GPU until the process ends.  The
 * call allocates nothing (no hipMalloc or hipFree, no allocating library call).
 *
 * Limit: a problem whose workspace does not fit the scratch array is rejected
 * with 161002 (bsa_last_error() gives both sizes) and nothing is enqueued; the
 * partial-result slots of split dK/dV work are first reduced to what fits,
 * which changes the load balance, not the results.  The sequence table, lists,
 * softmax_grad, plan and partials are all rewritten by every call before they
 * are read, so no scratch contents carry over from one call to the next.
 * Every call on one GPU shares that GPU's array: calls that overlap in time on
 * one GPU (different streams, or different host threads) race and give wrong
 * results; serialise them.  Profiling (bsa_profile_start) does not record these
 * calls.  fp16 / bf16 inputs only (no fp8 variant).
 */
#define BSA_NOALLOC_SCRATCH_BYTES (64ull << 20)
int bsa_bwd_noalloc(const bsa_tensor* dout, const bsa_tensor* query, const bsa_tensor* key,
                    const bsa_tensor* value, const bsa_tensor* attention_out, const bsa_tensor* softmax_lse,
                    const bsa_tensor* block_sparse_mask, const bsa_tensor* atten_mask,
                    const int64_t* block_shape, int64_t block_shape_len, const int64_t* actual_seq_lengths,
                    int64_t actual_seq_lengths_len, const int64_t* actual_seq_lengths_kv,
                    int64_t actual_seq_lengths_kv_len, const char* q_input_layout,
                    const char* kv_input_layout, int64_t num_key_value_heads, int64_t mask_type,
                    double scale_value, int64_t pre_tokens, int64_t next_tokens, const bsa_tensor* dq,
                    const bsa_tensor* dk, const bsa_tensor* dv, void* stream);

/*
 * The backward with a choice of how dQ is formed (dq_mode).  Arguments and
 * results otherwise as bsa_bwd_workspace_size / bsa_bwd.
 *
 * BSA_DQ_RECOMPUTE  the dQ kernel recomputes S and dP for every selected block
 *                   and forms dQ = (dS K) scale ([BSA] page, 功能说明 / 计算公式)
 *                   with no atomics: the mode of bsa_bwd, bitwise reproducible.
 * BSA_DQ_ATOMIC     opt-in: the dK/dV kernel, which already holds dS rounded to
 *                   the input dtype, also multiplies it by its KV block's K and
 *                   adds the product into an fp32 accumulator in the workspace
 *                   with atomic adds; a last kernel applies scale, rounds and
 *                   stores dQ.  No recompute, but the order of the fp32
 *                   additions into a dQ element depends on scheduling, so dQ is
 *                   not bitwise reproducible (dK and dV still are).  Head dim 64
 *                   or 128, no attenMask, at most 256 query heads per KV head;
 *                   other calls return 161002.  The workspace grows by
 *                   4 * B * N * maxSq * D bytes (BSA_WS_DQ_ACC).
 *
 * Any other dq_mode returns 161002.
 */
#define BSA_DQ_RECOMPUTE 0
#define BSA_DQ_ATOMIC 1
int bsa_bwd_ex_workspace_size(const bsa_tensor* dout, const bsa_tensor* query, const bsa_tensor* key,
                              const bsa_tensor* value, const bsa_tensor* attention_out,
                              const bsa_tensor* softmax_lse, const bsa_tensor* block_sparse_mask,
                              const bsa_tensor* atten_mask, const int64_t* block_shape, int64_t block_shape_len,
                              const int64_t* actual_seq_lengths, int64_t actual_seq_lengths_len,
                              const int64_t* actual_seq_lengths_kv, int64_t actual_seq_lengths_kv_len,
                              const char* q_input_layout, const char* kv_input_layout,
                              int64_t num_key_value_heads, int64_t mask_type, double scale_value,
                              int64_t pre_tokens, int64_t next_tokens, const bsa_tensor* dq,
                              const bsa_tensor* dk, const bsa_tensor* dv, int32_t dq_mode,
                              uint64_t* workspace_size);
int bsa_bwd_ex(const bsa_tensor* dout, const bsa_tensor* query, const bsa_tensor* key,
               const bsa_tensor* value, const bsa_tensor* attention_out, const bsa_tensor* softmax_lse,
               const bsa_tensor* block_sparse_mask, const bsa_tensor* atten_mask,
               const int64_t* block_shape, int64_t block_shape_len, const int64_t* actual_seq_lengths,
               int64_t actual_seq_lengths_len, const int64_t* actual_seq_lengths_kv,
               int64_t actual_seq_lengths_kv_len, const char* q_input_layout,
               const char* kv_input_layout, int64_t num_key_value_heads, int64_t mask_type,
               double scale_value, int64_t pre_tokens, int64_t next_tokens, const bsa_tensor* dq,
               const bsa_tensor* dk, const bsa_tensor* dv, int32_t dq_mode, void* workspace,
               uint64_t workspace_size, void* stream);

/*
 * Forward (the operation the backward differentiates; aclnnBlockSparseAttentionGrad
 * page, 计算公式: S = Mask(scale * Q * K^T), P = Softmax(S), Out = P * V, with the
 * softmax taken over the selected blocks only, as the FlashAttentionScore page's
 * 实现原理 describes for the dense case).  Produces the attentionOut and softmaxLse
 * inputs of bsa_bwd:
 *     attention_out[i] = sum_j P_ij * V[j]
 *     softmax_lse[i]   = ln sum_j exp(scale * Q[i] . K[j])     (natural log)
 * over the selected in-range keys j of query row i.  A row that selects no key
 * (and every BNSD row past its actual length) gets attention_out = 0 and
 * softmax_lse = -inf.
 *
 * Arguments are those of bsa_bwd_workspace_size without dout, dq, dk and dv, in
 * the same order and with the same rules, except:
 *  attention_out   output, dtype of query, shape of query; outer strides
 *                  multiples of 4 elements, innermost stride 1, no two elements
 *                  at one address; data pointer 8-byte aligned (it is stored
 *                  four elements at a time; 161002 otherwise).  Every element
 *                  is written.
 *  softmax_lse     output, fp32, [B, N, S] / [B, N, S, 1] (BNSD) or
 *                  [T, N] / [T, N, 1] (TND), contiguous.  Every element is written.
 * Ownership, stream, workspace and error behaviour are as for bsa_bwd; the
 * forward's workspace (sequence table and row lists) is smaller than the
 * backward's.
 */
int bsa_fwd_workspace_size(const bsa_tensor* query, const bsa_tensor* key, const bsa_tensor* value,
                           const bsa_tensor* block_sparse_mask, const bsa_tensor* atten_mask,
                           const int64_t* block_shape, int64_t block_shape_len,
                           const int64_t* actual_seq_lengths, int64_t actual_seq_lengths_len,
                           const int64_t* actual_seq_lengths_kv, int64_t actual_seq_lengths_kv_len,
                           const char* q_input_layout, const char* kv_input_layout,
                           int64_t num_key_value_heads, int64_t mask_type, double scale_value,
                           int64_t pre_tokens, int64_t next_tokens, const bsa_tensor* attention_out,
                           const bsa_tensor* softmax_lse, uint64_t* workspace_size);

int bsa_fwd(const bsa_tensor* query, const bsa_tensor* key, const bsa_tensor* value,
            const bsa_tensor* block_sparse_mask, const bsa_tensor* atten_mask, const int64_t* block_shape,
            int64_t block_shape_len, const int64_t* actual_seq_lengths, int64_t actual_seq_lengths_len,
            const int64_t* actual_seq_lengths_kv, int64_t actual_seq_lengths_kv_len,
            const char* q_input_layout, const char* kv_input_layout, int64_t num_key_value_heads,
            int64_t mask_type, double scale_value, int64_t pre_tokens, int64_t next_tokens,
            const bsa_tensor* attention_out, const bsa_tensor* softmax_lse, void* workspace,
            uint64_t workspace_size, void* stream);

/*
 * fp8 inputs with per-tensor scaling.  The page lists FLOAT8_E4M3FN and
 * FLOAT8_E5M2 as types some products do not take (产品支持情况 note under 参数说明)
 * and fixes no scaling rule; here each fp8 input tensor carries one
 * dequantisation factor: the value of an element is its decoded code times
 * the factor, and the operation is the one above on those values.
 *
 * Arguments are those of bsa_bwd_workspace_size / bsa_bwd (resp. the
 * forward's), in the same order and with the same rules, except:
 *  dout, query, key, value, attention_out
 *                  BSA_DTYPE_FP8_E4M3FN or BSA_DTYPE_FP8_E5M2, chosen per
 *                  tensor (e.g. E5M2 for dout, E4M3FN for the others);
 *                  contiguous, 16-byte aligned.  In the forward,
 *                  attention_out is the output and must be bf16.
 *  dq, dk, dv      outputs, BSA_DTYPE_BF16 (an fp8 gradient with no output
 *                  factor would lose most of its range).
 *  descale         host array: factors of {dout, query, key, value,
 *                  attention_out} (backward) or {query, key, value}
 *                  (forward), each finite and > 0; NULL = all 1.  Read only
 *                  during the call.
 * The inputs are decoded exactly into bf16 copies in the workspace (region
 * BSA_WS_STAGE, 2 bytes per input element) and the bf16 kernels run on the
 * codes' values; the factors are applied in fp32 where the scores are formed
 * (scale * f_query * f_key), to softmax_grad (f_attention_out / f_value) and to
 * the outputs (dQ: scale * f_dout * f_value * f_key, dK: scale * f_dout *
 * f_value * f_query, dV: f_dout; forward O: f_value).  Ownership, stream,
 * workspace and error behaviour are those of bsa_bwd / bsa_fwd; the
 * fp16/bf16 entry points reject fp8 dtypes and these reject fp16/bf16 inputs.
 */
int bsa_bwd_fp8_workspace_size(const bsa_tensor* dout, const bsa_tensor* query, const bsa_tensor* key,
                               const bsa_tensor* value, const bsa_tensor* attention_out,
                               const bsa_tensor* softmax_lse, const bsa_tensor* block_sparse_mask,
                               const bsa_tensor* atten_mask, const int64_t* block_shape,
                               int64_t block_shape_len, const int64_t* actual_seq_lengths,
                               int64_t actual_seq_lengths_len, const int64_t* actual_seq_lengths_kv,
                               int64_t actual_seq_lengths_kv_len, const char* q_input_layout,
                               const char* kv_input_layout, int64_t num_key_value_heads, int64_t mask_type,
                               double scale_value, int64_t pre_tokens, int64_t next_tokens,
                               const bsa_tensor* dq, const bsa_tensor* dk, const bsa_tensor* dv,
                               const double* descale, uint64_t* workspace_size);

int bsa_bwd_fp8(const bsa_tensor* dout, const bsa_tensor* query, const bsa_tensor* key,
                const bsa_tensor* value, const bsa_tensor* attention_out, const bsa_tensor* softmax_lse,
                const bsa_tensor* block_sparse_mask, const bsa_tensor* atten_mask,
                const int64_t* block_shape, int64_t block_shape_len, const int64_t* actual_seq_lengths,
                int64_t actual_seq_lengths_len, const int64_t* actual_seq_lengths_kv,
                int64_t actual_seq_lengths_kv_len, const char* q_input_layout,
                const char* kv_input_layout, int64_t num_key_value_heads, int64_t mask_type,
                double scale_value, int64_t pre_tokens, int64_t next_tokens, const bsa_tensor* dq,
                const bsa_tensor* dk, const bsa_tensor* dv, const double* descale, void* workspace,
                uint64_t workspace_size, void* stream);

int bsa_fwd_fp8_workspace_size(const bsa_tensor* query, const bsa_tensor* key, const bsa_tensor* value,
                               const bsa_tensor* block_sparse_mask, const bsa_tensor* atten_mask,
                               const int64_t* block_shape, int64_t block_shape_len,
                               const int64_t* actual_seq_lengths, int64_t actual_seq_lengths_len,
                               const int64_t* actual_seq_lengths_kv, int64_t actual_seq_lengths_kv_len,
                               const char* q_input_layout, const char* kv_input_layout,
                               int64_t num_key_value_heads, int64_t mask_type, double scale_value,
                               int64_t pre_tokens, int64_t next_tokens, const bsa_tensor* attention_out,
                               const bsa_tensor* softmax_lse, const double* descale, uint64_t* workspace_size);

int bsa_fwd_fp8(const bsa_tensor* query, const bsa_tensor* key, const bsa_tensor* value,
                const bsa_tensor* block_sparse_mask, const bsa_tensor* atten_mask, const int64_t* block_shape,
                int64_t block_shape_len, const int64_t* actual_seq_lengths, int64_t actual_seq_lengths_len,
                const int64_t* actual_seq_lengths_kv, int64_t actual_seq_lengths_kv_len,
                const char* q_input_layout, const char* kv_input_layout, int64_t num_key_value_heads,
                int64_t mask_type, double scale_value, int64_t pre_tokens, int64_t next_tokens,
                const bsa_tensor* attention_out, const bsa_tensor* softmax_lse, const double* descale,
                void* workspace, uint64_t workspace_size, void* stream);

/* Workspace regions, as byte offsets filled in by bsa_bwd_workspace_layout. */
enum bsa_ws_region {
  BSA_WS_SEQ = 0,      /* per-sequence table {int64 q_offset, kv_offset; int32 len_q, len_kv, wlim_q, wlim_kv} x B, then 128 fp32 constants */
  BSA_WS_DELTA = 1,    /* fp32 [B, N, maxSq]: -softmax_grad (negated row sums of dOut o Out); 0 past len_q */
  BSA_WS_LSE2 = 2,     /* fp32 [B, N, maxSq]: softmaxLse * log2(e) */
  BSA_WS_ROW_CNT = 3,  /* int32 [B, N, nQB]: number of selected in-range KV blocks per Q block */
  BSA_WS_ROW_LIST = 4, /* int32 [B, N, nQB, nKB]: ascending KV-block lists, first ROW_CNT entries valid */
  BSA_WS_COL_CNT = 5,  /* int32 [B, N, nKB]: number of selected in-range Q blocks per KV block */
  BSA_WS_COL_LIST = 6, /* int32 [B, N, nKB, nQB]: ascending Q-block lists, first COL_CNT entries valid */
  BSA_WS_PLAN = 7,     /* int32: dK/dV work split (chunk size, per-unit piece counts and slots, slot table) */
  BSA_WS_PARTIAL = 8,  /* fp32 per-piece dK/dV partial sums of split units, reduced in piece order */
  BSA_WS_AMASK = 9,    /* with an attenMask (else empty): uint32 [maxSq][ceil(maxSkv/32)] bits by query row,
                          then (backward) uint32 [maxSkv][ceil(maxSq/32)] bits by key; 1 = excluded */
  BSA_WS_STAGE = 10,   /* fp8 entry points only (else empty): bf16 copies of the fp8 inputs, each 256-byte aligned */
  BSA_WS_DQ_ACC = 11,  /* BSA_DQ_ATOMIC only (else empty): fp32 [B, N, maxSq, D] dQ accumulator (unscaled) */
  BSA_WS_TOTAL = 12,   /* total bytes (== the phase-1 size) */
  BSA_WS_NUM = 13
};

/*
 * Test and tooling hook: the same validation as phase 1, then the byte offset
 * of every workspace region (offsets[BSA_WS_NUM]) and the plan's block grid
 * (dims[4] = {bx, by, nQB, nKB}; may be NULL).  After a bsa_bwd call has
 * completed, these regions hold softmax_grad and lse2 (written by the dQ
 * kernel) and the mask compaction.
 */
int bsa_bwd_workspace_layout(const bsa_tensor* dout, const bsa_tensor* query,
                             const bsa_tensor* key, const bsa_tensor* value,
                             const bsa_tensor* attention_out, const bsa_tensor* softmax_lse,
                             const bsa_tensor* block_sparse_mask, const bsa_tensor* atten_mask,
                             const int64_t* block_shape, int64_t block_shape_len,
                             const int64_t* actual_seq_lengths, int64_t actual_seq_lengths_len,
                             const int64_t* actual_seq_lengths_kv,
                             int64_t actual_seq_lengths_kv_len, const char* q_input_layout,
                             const char* kv_input_layout, int64_t num_key_value_heads,
                             int64_t mask_type, double scale_value, int64_t pre_tokens,
                             int64_t next_tokens, const bsa_tensor* dq, const bsa_tensor* dk,
                             const bsa_tensor* dv, uint64_t* offsets, int64_t* dims);

/* Message for the last non-zero status returned on this thread ("" if none). */
const char* bsa_last_error(void);

/*
 * Per-stage timing for benchmarks.  bsa_profile_start(max_calls) makes the
 * next max_calls bsa_bwd / bsa_fwd calls on this process record HIP events
 * between their kernel stages (on the call's stream).  bsa_profile_stop waits
 * for the recorded events, writes the summed milliseconds of each stage into
 * stage_ms[0..n_stages) (stage order: 0 = sequence table + mask compaction +
 * work plan (+ the attenMask packing, + the fp8 decode of the fp8 entry
 * points, + softmax_grad in the forward and with BSA_DQ_ATOMIC),
 * 1 = dK/dV, including the sums of split dK/dV units, 2 = dQ (by default it
 * runs before dK/dV and also computes softmax_grad; with BSA_DQ_ATOMIC it
 * runs after dK/dV and stores the accumulated dQ),
 * 3 = forward; a stage a call does not run adds 0), writes the number of
 * profiled calls to *n_calls, frees the events and turns recording off.
 * Not thread-safe.
 */
int bsa_profile_start(int32_t max_calls);
int bsa_profile_stop(double* stage_ms, int32_t n_stages, int32_t* n_calls);

/* Name of a profiling stage, or NULL past the last one. */
const char* bsa_stage_name(int32_t stage);

#ifdef __cplusplus
}
#endif

#endif /* BSA_BWD_H */
