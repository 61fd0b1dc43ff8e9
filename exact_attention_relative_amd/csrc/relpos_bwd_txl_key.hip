// The T-XL key-side backward pass (dK, dV and the r-window table GEMM), alone in this
// translation unit so that it can be compiled with options of its own (the build adds the
// AMDGPU scheduler's register-pressure trackers, which halve its spills) and with 64-bit
// staging addresses (see stage_addr).
#define RELPOS_STAGE_ADDR64
#include "relpos_bwd_body.h"

namespace relpos {

void launch_bwd_txl_key(const BwdArgs& a, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((bwd_kernel<uint16_t, MECH_TXL, 1, 0>), grid, dim3(256), 0, stream, a);
}

}  // namespace relpos
