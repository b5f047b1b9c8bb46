// Low-Rank Bypass step: instances for ranks up to 4, and the dispatch over
// the rank bound (the kernel is in lsq_lrb_impl.h).
#include "lsq_internal.h"
#include "lsq_lrb_impl.h"

namespace lsq {

hipError_t launch_lrb_step(const StepArgs& a, int bits, int dk, int policy, int rounding,
                           int delta, int diag, hipStream_t s) {
  if (a.lrb_rank <= 4) return launch_lrb_rmax<4>(a, bits, dk, policy, rounding, delta, diag, s);
  return launch_lrb_step_r8(a, bits, dk, policy, rounding, delta, diag, s);
}

}  // namespace lsq
