// INT4 decode-step kernel instances with fp32 group scales (group sizes 32/64/128, Dk 64/128).
#include "lsq_step_impl.h"

namespace lsq {
hipError_t launch_step_q4(const StepArgs& a, int dk, int policy, int rounding, int delta, int diag,
                          hipStream_t s) {
  if (dk == 128) return dev::launch_family<4, 128, 0>(a, policy, rounding, delta, diag, s);
  if (dk == 64) return dev::launch_family<4, 64, 0>(a, policy, rounding, delta, diag, s);
  return hipErrorInvalidValue;
}
}  // namespace lsq
