// Host-to-device staging of one decode step's index data (block tables,
// context lengths, slot mapping, copy pairs, launch order) by a kernel that
// reads page-locked host memory directly.  A copy-engine transfer of a few KB
// costs little by itself, but on the compute stream it is bracketed by two
// cross-engine synchronisations that leave the GPU idle for 15-40 us per step;
// a kernel on the same queue needs only the ordinary dispatch gap.
//
// Host writes made before the launch are read with system-scope loads, so the
// copy is correct whether the pinned buffer is mapped coherently or not, and
// a staging buffer reused every other step never yields stale lines.
#include "device_common.hpp"
#include "launch.hpp"

namespace pa {

__global__ __launch_bounds__(256) void upload_kernel(uint32_t* __restrict__ dst, const uint32_t* src,
                                                     int64_t words) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < words; i += stride)
    dst[i] = __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

hipError_t launch_upload(void* dst, const void* src_device_view, int64_t nbytes, hipStream_t stream) {
  const int64_t words = nbytes / 4;
  if (words == 0) return hipSuccess;
  int64_t grid = (words + 255) / 256;
  if (grid > 256) grid = 256;  // one pass of up to 64 K words in flight; the rest loops
  launch_kernel(upload_kernel, dim3(static_cast<uint32_t>(grid)), dim3(256), stream,
                     static_cast<uint32_t*>(dst), static_cast<const uint32_t*>(src_device_view), words);
  return hipGetLastError();
}

}  // namespace pa
