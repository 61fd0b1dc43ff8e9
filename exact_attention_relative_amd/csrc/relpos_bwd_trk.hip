// Backward passes compiled with the AMDGPU scheduler's register-pressure trackers (the build
// adds -amdgpu-use-amdgpu-trackers for this translation unit): the T-XL query-side pass and the
// key-side light and general passes of Shaw and DeBERTa, which each ran faster with them
// (measured); the other passes ran as fast or slower and stay in relpos_bwd.hip.
#include "relpos_bwd_body.h"

namespace relpos {

void launch_bwd_trk(int mech, int dir, int part, const BwdArgs& a, dim3 grid, hipStream_t stream) {
  if (mech == MECH_TXL && dir == 0)
    hipLaunchKernelGGL((bwd_kernel<uint16_t, MECH_TXL, 0, 0>), grid, dim3(256), 0, stream, a);
  else if (mech == MECH_SHAW && dir == 1 && part == 1)
    hipLaunchKernelGGL((bwd_kernel<uint16_t, MECH_SHAW, 1, 1>), grid, dim3(256), 0, stream, a);
  else if (mech == MECH_SHAW && dir == 1 && part == 2)
    hipLaunchKernelGGL((bwd_kernel<uint16_t, MECH_SHAW, 1, 2>), grid, dim3(256), 0, stream, a);
  else if (mech == MECH_DEBERTA && dir == 1 && part == 1)
    hipLaunchKernelGGL((bwd_kernel<uint16_t, MECH_DEBERTA, 1, 1>), grid, dim3(256), 0, stream, a);
  else if (mech == MECH_DEBERTA && dir == 1 && part == 2)
    hipLaunchKernelGGL((bwd_kernel<uint16_t, MECH_DEBERTA, 1, 2>), grid, dim3(256), 0, stream, a);
}

}  // namespace relpos
