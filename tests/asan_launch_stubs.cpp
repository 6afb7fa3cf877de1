// Launch helpers for the AddressSanitizer build of the host library: the host
// code (validation, planning, workspace layout, argument marshalling) is built
// and checked on its own, so the kernel launches are replaced by stubs that
// report an error.  A host test that reached a launch would see that error.
#include "bsa_internal.h"

namespace bsa {
constexpr int kNoKernels = 98;  // hipErrorInvalidDeviceFunction: no kernel in this build
int launch_stage_fp8(const Fp8Stage&, void*) { return kNoKernels; }
int launch_pack_amask(const Params&, void*) { return kNoKernels; }
int launch_stage_seq(const SeqChunk&, SeqInfo*, void*) { return kNoKernels; }
int launch_prologue(const Params&, void*) { return kNoKernels; }
int launch_plan(const Params&, void*) { return kNoKernels; }
int launch_prologue_rows(const Params&, void*) { return kNoKernels; }
int launch_fwd(const Params&, void*) { return kNoKernels; }
int launch_dkdv(const Params&, void*) { return kNoKernels; }
int launch_dq(const Params&, void*) { return kNoKernels; }
int launch_dq_acc_zero(const Params&, void*) { return kNoKernels; }
int scratch_region(void**, uint64_t*) { return kNoKernels; }
}  // namespace bsa
