// Backward launch logic: per mechanism and direction, the pass variants of relpos_bwd_body.h.
// The T-XL key-side pass is instantiated in relpos_bwd_txl_key.hip, a translation unit of its
// own compiled with the scheduler's register-pressure trackers, which spill less there; the
// query-side general passes of Shaw and DeBERTa in relpos_bwd_fat_q.hip; the T-XL query-side
// pass and the key-side passes of Shaw and DeBERTa in relpos_bwd_trk.hip.
#include "relpos_bwd_body.h"

namespace relpos {

// relpos_bwd_txl_key.hip
void launch_bwd_txl_key(const BwdArgs& a, dim3 grid, hipStream_t stream);
// relpos_bwd_fat_q.hip: the query-side general passes of Shaw and DeBERTa
void launch_bwd_fat_q(int mech, const BwdArgs& a, dim3 grid, hipStream_t stream);
// relpos_bwd_trk.hip: passes compiled with the register-pressure trackers
void launch_bwd_trk(int mech, int dir, int part, const BwdArgs& a, dim3 grid, hipStream_t stream);
// relpos_bwd_f32.hip: every fp32 pass
void launch_bwd_f32(int mech, int dir, int part, const BwdArgs& a, dim3 grid, hipStream_t stream);

// Shaw and DeBERTa run in two parts: a light pass over the clipped steps, then the general pass.
template <int MECH>
constexpr bool split_pass() {
  return MECH == MECH_SHAW || MECH == MECH_DEBERTA;
}
template <int MECH, int DIR, int PART>
static void launch_part(const BwdArgs& a, bool fp32, dim3 grid, hipStream_t stream) {
  if (fp32)
    launch_bwd_f32(MECH, DIR, PART, a, grid, stream);
  else if constexpr (MECH == MECH_TXL && DIR == 1)
    launch_bwd_txl_key(a, grid, stream);
  else if constexpr (MECH == MECH_TXL && DIR == 0)
    launch_bwd_trk(MECH, DIR, 0, a, grid, stream);
  else if constexpr (DIR == 0 && PART == 2)
    launch_bwd_fat_q(MECH, a, grid, stream);
  else if constexpr (DIR == 1 && PART != 0)
    launch_bwd_trk(MECH, DIR, PART, a, grid, stream);
  else
    hipLaunchKernelGGL((bwd_kernel<uint16_t, MECH, DIR, PART>), grid, dim3(256), 0, stream, a);
}
template <int MECH, int DIR>
static void launch_one(const BwdArgs& a, bool fp32, dim3 grid, hipStream_t stream) {
  if constexpr (split_pass<MECH>()) {
    launch_part<MECH, DIR, 1>(a, fp32, grid, stream);
    // general pass: a.fold launches, each with one workgroup per (group of a.fold batch entries,
    // head, block) taking the group's next entry (same-stream order: each launch adds to the
    // partial slots the previous one wrote)
    const int nb = (a.sh.L + BLANE - 1) / BLANE;
    const int ng = a.fold_slices ? (a.sh.B * a.sh.H + a.fold - 1) / a.fold
                                 : (a.sh.B + a.fold - 1) / a.fold * a.sh.H;
    BwdArgs g = a;
    for (g.sub = 0; g.sub < a.fold; ++g.sub)
      launch_part<MECH, DIR, 2>(g, fp32, dim3((unsigned)(nb * ng)), stream);
  } else {
    launch_part<MECH, DIR, 0>(a, fp32, grid, stream);
  }
}

template <int DIR>
static hipError_t launch_bwd_dir(const BwdArgs& a, bool fp32, hipStream_t stream) {
  const int nb = (a.sh.L + BLANE - 1) / BLANE;
  const int nbh = a.nbh > 0 ? a.nbh : a.sh.B * a.sh.H;
  const dim3 grid((unsigned)(nb * nbh));
  switch (a.sh.mech) {
    case MECH_T5: launch_one<MECH_T5, DIR>(a, fp32, grid, stream); break;
    case MECH_SHAW: launch_one<MECH_SHAW, DIR>(a, fp32, grid, stream); break;
    case MECH_TXL: launch_one<MECH_TXL, DIR>(a, fp32, grid, stream); break;
    case MECH_DEBERTA: launch_one<MECH_DEBERTA, DIR>(a, fp32, grid, stream); break;
    case MECH_ALIBI: launch_one<MECH_ALIBI, DIR>(a, fp32, grid, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdArgs& a, bool fp32, hipStream_t stream) {
  return launch_bwd_dir<0>(a, fp32, stream);
}
hipError_t launch_bwd_dkdv(const BwdArgs& a, bool fp32, hipStream_t stream) {
  return launch_bwd_dir<1>(a, fp32, stream);
}

}  // namespace relpos
