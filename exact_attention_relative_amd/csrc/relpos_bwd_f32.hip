// The fp32 backward passes (two bf16 planes per operand, one workgroup per CU), one translation
// unit of their own so that they compile in parallel with the bf16 passes.
#include "relpos_bwd_body.h"

namespace relpos {

template <int MECH, int DIR, int PART>
static void go(const BwdArgs& a, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((bwd_kernel<float, MECH, DIR, PART>), grid, dim3(256), 0, stream, a);
}

template <int MECH, int DIR>
static void by_part(int part, const BwdArgs& a, dim3 grid, hipStream_t stream) {
  if constexpr (MECH == MECH_SHAW || MECH == MECH_DEBERTA) {
    if (part == 1) go<MECH, DIR, 1>(a, grid, stream);
    else go<MECH, DIR, 2>(a, grid, stream);
  } else {
    go<MECH, DIR, 0>(a, grid, stream);
  }
}

template <int MECH>
static void by_dir(int dir, int part, const BwdArgs& a, dim3 grid, hipStream_t stream) {
  if (dir == 0) by_part<MECH, 0>(part, a, grid, stream);
  else by_part<MECH, 1>(part, a, grid, stream);
}

void launch_bwd_f32(int mech, int dir, int part, const BwdArgs& a, dim3 grid, hipStream_t stream) {
  switch (mech) {
    case MECH_T5: by_dir<MECH_T5>(dir, part, a, grid, stream); break;
    case MECH_SHAW: by_dir<MECH_SHAW>(dir, part, a, grid, stream); break;
    case MECH_TXL: by_dir<MECH_TXL>(dir, part, a, grid, stream); break;
    case MECH_DEBERTA: by_dir<MECH_DEBERTA>(dir, part, a, grid, stream); break;
    case MECH_ALIBI: by_dir<MECH_ALIBI>(dir, part, a, grid, stream); break;
    default: break;
  }
}

}  // namespace relpos
