// probe.hip -- streaming 128-bit read of a large buffer, to measure the HBM
// read bandwidth the chip actually sustains (context for the roofline).
#include "kv4_common.h"
#include "kv4_launch.h"

namespace kv4 {
namespace {

constexpr int kProbeBlocks = 256 * 8;  // workgroups of 4 waves
constexpr int kRound = 16;              // 1-KiB wave loads in flight per wave

typedef uint32_t u32x4v_t __attribute__((ext_vector_type(4)));

// Each wave streams its own contiguous share of the buffer in rounds of
// kRound whole-KiB loads with the nontemporal hint (the pattern that sustains
// the highest read rate on gfx950); whatever is left after the equal shares
// is read by the whole grid.
__global__ __launch_bounds__(256) void probe_kernel(const u32x4v_t* __restrict__ buf, int64_t n16,
                                                    uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t nwaves = int64_t(gridDim.x) * (blockDim.x / 64);
  const int64_t w = int64_t(blockIdx.x) * (blockDim.x / 64) + threadIdx.x / 64;
  const int64_t per = (n16 / nwaves) / (64 * kRound) * (64 * kRound);
  uint32_t acc = 0;
  for (int64_t i = w * per; i < (w + 1) * per; i += 64 * kRound) {
    u32x4v_t v[kRound];
#pragma unroll
    for (int r = 0; r < kRound; ++r) v[r] = __builtin_nontemporal_load(buf + i + 64 * r + lane);
#pragma unroll
    for (int r = 0; r < kRound; ++r) acc ^= v[r].x ^ v[r].y ^ v[r].z ^ v[r].w;
  }
  for (int64_t i = nwaves * per + int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16;
       i += int64_t(gridDim.x) * blockDim.x) {
    const u32x4v_t a = buf[i];
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
                     static_cast<const u32x4v_t*>(buf), int64_t(bytes / 16), sink);
  return hipGetLastError();
}

}  // namespace kv4
