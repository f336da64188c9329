// Head dimension 128 instantiations of the bf16 masked forward (kernel and its
// design: fwd_bf16.cuh).  The larger output accumulator lives in AGPRs here.
#include "fwd_bf16.cuh"

namespace mattn {
hipError_t launch_fwd_bf16_d128(const FwdArgs& a) { return fwdk::launch<128>(a); }
}  // namespace mattn
