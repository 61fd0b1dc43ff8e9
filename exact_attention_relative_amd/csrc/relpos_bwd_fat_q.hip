// The query-side general (relation-product) backward passes of Shaw and DeBERTa, alone in this
// translation unit so that they can be compiled with options of their own: with the MFMA
// accumulators forced into VGPRs (-amdgpu-mfma-vgpr-form) the compiler moves fewer values
// between the two register files.
#include "relpos_bwd_body.h"

namespace relpos {

void launch_bwd_fat_q(int mech, const BwdArgs& a, dim3 grid, hipStream_t stream) {
  if (mech == MECH_SHAW)
    hipLaunchKernelGGL((bwd_kernel<uint16_t, MECH_SHAW, 0, 2>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((bwd_kernel<uint16_t, MECH_DEBERTA, 0, 2>), grid, dim3(256), 0, stream, a);
}

}  // namespace relpos
