// Head dimension 128 instantiations of the bf16 masked forward (kernel and its
// design: fwd_bf16.cuh).  The larger output accumulator lives in AGPRs here.
#include "fwd_bf16.cuh"

namespace mattn {
hipError_t launch_fwd_bf16_d128(const FwdArgs& a) {
    if (a.varlen)
        return a.lse ? fwdk::launch_one<128, true, true>(a) : fwdk::launch_one<128, false, true>(a);
    return a.lse ? fwdk::launch_one<128, true, false>(a) : fwdk::launch_one<128, false, false>(a);
}
}  // namespace mattn
