// k_measure.hip -- measurement aids (include/gdn_measure.h): a non-temporal
// streaming copy, the access pattern of the recurrence's state stream without
// its arithmetic.  One 16-byte load and store per thread: a sweep of 1, 2, 4
// and 8 per thread on 192 MiB gave the best rate at one.
#include <hip/hip_runtime.h>

#include "gdn.h"
#include "gdn_measure.h"
#include "launch.hpp"

namespace gdn {

typedef float f32x4m __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_stream_copy(const f32x4m *__restrict__ src,
                                                     f32x4m *__restrict__ dst, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace gdn

extern "C" int gdn_stream_copy(void *dst, const void *src, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return GDN_OK;
  if (!dst || !src) return GDN_ERR_NULL;
  const uintptr_t d = reinterpret_cast<uintptr_t>(dst), s = reinterpret_cast<uintptr_t>(src);
  if ((d & 15) || (s & 15) || (bytes & 15)) return GDN_ERR_SHAPE;
  if (d < s + bytes && s < d + bytes) return GDN_ERR_ALIAS;
  const size_t n = bytes / 16;
  const size_t blocks = (n + 255) / 256;
  if (blocks > 0x7fffffffu) return GDN_ERR_SHAPE;
  return gdn::launch_kernel(gdn::k_stream_copy, dim3((unsigned)blocks), dim3(256), 0, stream,
                            static_cast<const gdn::f32x4m *>(src), static_cast<gdn::f32x4m *>(dst),
                            n);
}
