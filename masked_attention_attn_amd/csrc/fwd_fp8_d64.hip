// Head dimension 64 instantiations of the E4M3-input masked forward (kernel and its
// design: fwd_bf16.cuh, FP8 = true).  Built like the bf16 D = 64 kernels, with
// VGPR-form MFMAs.
#include "fwd_bf16.cuh"

namespace mattn {
hipError_t launch_fwd_fp8_d64(const FwdArgs& a) { return fwdk::launch_fp8<64>(a); }
}  // namespace mattn
