// Head dimension 128 instantiations of the E4M3-input masked forward (kernel and its
// design: fwd_bf16.cuh, FP8 = true).
#include "fwd_bf16.cuh"

namespace mattn {
hipError_t launch_fwd_fp8_d128(const FwdArgs& a) { return fwdk::launch_fp8<128>(a); }
}  // namespace mattn
