// INT4 decode-step kernel instances with bfloat16 group scales (group sizes 16-128, Dk 64/128).
#include "lsq_step_impl.h"

namespace lsq {
hipError_t launch_step_q4_bf16(const StepArgs& a, int dk, int policy, int rounding, int delta,
                               int diag, hipStream_t s) {
  if (dk == 128) return dev::launch_family<4, 128, 2>(a, policy, rounding, delta, diag, s);
  if (dk == 64) return dev::launch_family<4, 64, 2>(a, policy, rounding, delta, diag, s);
  return hipErrorInvalidValue;
}
}  // namespace lsq
