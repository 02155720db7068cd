// gate.hpp -- the decay gate value, shared by the gate kernel and the fused
// decode kernel so the two compute it with the same operations.
//
// fm_kernel_ssm.h (Foundry), "Decay gate" section: g = a * softplus(alpha + dt),
// with a = -exp(A_log) precomputed by the caller; scr_state.hpp (regolith),
// log_gate: softplus passes its argument through when it exceeds 20.
#pragma once
#include <hip/hip_runtime.h>

namespace gdn {

__device__ __forceinline__ float decay_gate_value(float alpha, float dt, float a) {
  const float v = alpha + dt;
  const float sp = v > 20.0f ? v : log1pf(expf(v));
  return a * sp;
}

}  // namespace gdn
