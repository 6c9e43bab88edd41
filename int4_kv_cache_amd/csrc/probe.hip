// probe.hip -- streaming 128-bit read of a large buffer, to measure the HBM
// read bandwidth the chip actually sustains (context for the roofline).
#include "kv4_common.h"
#include "kv4_launch.h"

namespace kv4 {
namespace {

constexpr int kProbeBlocks = 256 * 8;

__global__ __launch_bounds__(256) void probe_kernel(const uint4* __restrict__ buf, int64_t n16,
                                                    uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  // four independent loads in flight per iteration
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = buf[i];
    const uint4 b = buf[i + stride];
    const uint4 c = buf[i + 2 * stride];
    const uint4 d = buf[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = buf[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] ^= red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0];
}

}  // namespace

int32_t probe_blocks() { return kProbeBlocks; }

hipError_t launch_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  hipLaunchKernelGGL(probe_kernel, dim3(kProbeBlocks), dim3(256), 0, stream,
                     static_cast<const uint4*>(buf), int64_t(bytes / 16), sink);
  return hipGetLastError();
}

}  // namespace kv4
