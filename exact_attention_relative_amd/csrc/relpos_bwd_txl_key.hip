// The T-XL key-side backward pass (dK, dV and the r-window table GEMM), alone in this
// translation unit so that it can be compiled with options of its own (the build adds the
// AMDGPU scheduler's register-pressure trackers, which halve its spills) and with 64-bit
// staging addresses (see stage_addr).
#define RELPOS_STAGE_ADDR64
#include "relpos_bwd_body.h"

namespace relpos {

// The first launch of a folded pass stores the r partials and the later ones add to them: a
// kernel for each, so that neither carries the other's writes behind a branch (the compiler
// would then count both among the memory operations a later read waits for).
void launch_bwd_txl_key(const BwdArgs& a, dim3 grid, hipStream_t stream) {
  if (a.sub == 0)
    hipLaunchKernelGGL((bwd_kernel<uint16_t, MECH_TXL, 1, 0, 1>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((bwd_kernel<uint16_t, MECH_TXL, 1, 0, 0>), grid, dim3(256), 0, stream, a);
}

}  // namespace relpos
