// k_gate.hip -- decay gate g = a * softplus(alpha + dt), softplus guarded at 20.
// fm_kernel_ssm.h (Foundry), "Decay gate" section; scr_state.hpp (regolith),
// log_gate for the strict comparison.  One thread per (row, head): the op is a
// few bytes per element and launch-latency bound at decode sizes.
#include <hip/hip_runtime.h>

#include "gate.hpp"
#include "gdn.h"
#include "launch.hpp"

namespace gdn {

__global__ __launch_bounds__(256) void k_decay_gate(const float *__restrict__ alpha,
                                                    const float *__restrict__ dt,
                                                    const float *__restrict__ a,
                                                    float *__restrict__ g, int64_t n, int H) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int h = (int)(i % H);
  g[i] = decay_gate_value(alpha[i], dt[h], a[h]);
}

int launch_decay_gate(const float *alpha, const float *dt, const float *a, float *g, int rows,
                      int n_heads, hipStream_t stream) {
  const int64_t n = (int64_t)rows * n_heads;
  if (n == 0) return GDN_OK;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  return launch_kernel(k_decay_gate, dim3(blocks), dim3(256), 0, stream, alpha, dt, a, g, n,
                       n_heads);
}

}  // namespace gdn
