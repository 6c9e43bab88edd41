// append.hip -- kv4_append / kv8_append / kvbf16_append launches.  The
// per-(token, kv head) work (quantizer, block and side-row writes) is in
// append_body.h.
#include "append_body.h"

namespace kv4 {
namespace {

template <int FMT, int E>
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
  append_row<FMT, E>(p, int64_t(blockIdx.x) * (blockDim.x / kWave) + threadIdx.x / kWave);
}

template <int FMT>
hipError_t launch_fmt(const AppendParams& p, int head_dim, hipStream_t stream) {
  const int64_t waves = int64_t(p.total_new) * p.num_kv_heads;
  const unsigned blocks = unsigned((waves + 3) / 4);
  if (head_dim == 128)
    hipLaunchKernelGGL((append_kernel<FMT, 2>), dim3(blocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((append_kernel<FMT, 1>), dim3(blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(int fmt, const AppendParams& p, int head_dim, hipStream_t stream) {
  if (fmt == kFmtKV4) return launch_fmt<kFmtKV4>(p, head_dim, stream);
  if (fmt == kFmtKV8) return launch_fmt<kFmtKV8>(p, head_dim, stream);
  return launch_fmt<kFmtBF16>(p, head_dim, stream);
}

}  // namespace kv4
