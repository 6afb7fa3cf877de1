// The generic dK/dV builds for calls with an attenMask.
#include "bsa_dkdv.h"

namespace bsa {

int launch_dkdv_generic_am(const Params& p, int w, dim3 grid, hipStream_t s) {
  return launch_dkdv_generic<true>(p, w, grid, s);
}

}  // namespace bsa
