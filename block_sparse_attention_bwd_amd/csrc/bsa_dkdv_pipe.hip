// The scheduled dK/dV builds of one element type and head dim, chosen by
// BSA_PIPE_BF16 (1: bf16, 0: fp16) and BSA_PIPE_D (64 or 128) at compile time;
// the library links one object for each of the four.
#include "bsa_dkdv.h"

#if !defined(BSA_PIPE_BF16) || !defined(BSA_PIPE_D)
#error "compile with -DBSA_PIPE_BF16=0|1 -DBSA_PIPE_D=64|128"
#endif

#define BSA_CAT4(a, b, c, d) a##b##c##d
#define BSA_PIPE_NAME(e, d) BSA_CAT4(launch_dkdv_pipe_, e, _d, d)
#if BSA_PIPE_BF16
#define BSA_PIPE_E EBf16
#define BSA_PIPE_FN BSA_PIPE_NAME(bf16, BSA_PIPE_D)
#else
#define BSA_PIPE_E EF16
#define BSA_PIPE_FN BSA_PIPE_NAME(f16, BSA_PIPE_D)
#endif

namespace bsa {

int BSA_PIPE_FN(const Params& p, dim3 grid, hipStream_t s) {
  if (p.dq_acc) launch_dkdv_pipe_w<BSA_PIPE_E, BSA_PIPE_D, true>(p, waves_for(p.by), grid, s);
  else launch_dkdv_pipe_w<BSA_PIPE_E, BSA_PIPE_D, false>(p, waves_for(p.by), grid, s);
  return static_cast<int>(hipGetLastError());
}

}  // namespace bsa
