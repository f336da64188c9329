// Head dimension 64 instantiations of the bf16 masked forward (kernel and its
// design: fwd_bf16.cuh).  Built with VGPR-form MFMAs so the score blocks stay
// in VGPRs for the vector unit.
#include "fwd_bf16.cuh"

namespace mattn {
hipError_t launch_fwd_bf16_d64(const FwdArgs& a) { return fwdk::launch<64>(a); }
}  // namespace mattn
