// The dK/dV dispatcher and the generic builds without an attenMask.
#include "bsa_dkdv.h"

namespace bsa {

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

int launch_dkdv(const Params& p, void* stream) {
  const dim3 grid(static_cast<unsigned>(dkdv_passes(p.D) * (p.n_units + p.slots_cap)));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (dkdv_scheduled(p.D, p.amask != nullptr, p.G)) {
    if (p.dtype == 2) return p.D == 128 ? launch_dkdv_pipe_bf16_d128(p, grid, s) : launch_dkdv_pipe_bf16_d64(p, grid, s);
    return p.D == 128 ? launch_dkdv_pipe_f16_d128(p, grid, s) : launch_dkdv_pipe_f16_d64(p, grid, s);
  }
  // head dim 256: the 1- and 2-wave builds spill registers, so KV blocks of
  // up to 64 rows also take the 4-wave one (its waves past the block's rows
  // compute on zero K/V rows and store nothing)
  const int w = p.D >= 256 ? 4 : waves_for(p.by);
  return p.amask ? launch_dkdv_generic_am(p, w, grid, s) : launch_dkdv_generic<false>(p, w, grid, s);
}

}  // namespace bsa
