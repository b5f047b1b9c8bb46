// Low-Rank Bypass step: instances for ranks 5 to 8 (the kernel is in
// lsq_lrb_impl.h).
#include "lsq_internal.h"
#include "lsq_lrb_impl.h"

namespace lsq {

hipError_t launch_lrb_step_r8(const StepArgs& a, int bits, int dk, int policy, int rounding,
                              int delta, int diag, hipStream_t s) {
  return launch_lrb_rmax<8>(a, bits, dk, policy, rounding, delta, diag, s);
}

}  // namespace lsq
