// chunk_fwd.hip -- chunkwise forward of the gated delta rule on gfx950.
#include "gdn_device.hpp"
#include "gdn_kernels.hpp"

namespace gdn {
namespace {

__global__ void state_copy_kernel(const float* __restrict__ src, float* __restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = src ? src[i] : 0.f;
}

}  // namespace

hipError_t launch_state_copy(const float* state_in, float* state_out, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  state_copy_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(state_in, state_out, n);
  return hipGetLastError();
}

hipError_t launch_chunk_fwd(const ChunkArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace gdn
