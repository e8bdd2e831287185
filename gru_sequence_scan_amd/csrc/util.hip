// Small stream-ordered helpers: zero-fill of workspace words and copies of
// host int arrays (lengths, packed offsets) into the workspace through
// kernel arguments, so nothing has to stay alive on the host after a call.
#include "kernels.hpp"

namespace rnnk {

namespace {

__global__ void fill_zero_kernel(uint32_t* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

struct IntChunk {
  int v[kIntsPerLaunch];
};

__global__ void write_ints_kernel(int* dst, IntChunk c, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = c.v[i];
}

}  // namespace

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream) {
  const size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  const size_t want = (n + 255) / 256;
  const int blocks = (int)(want < 256 ? want : 256);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, stream, reinterpret_cast<uint32_t*>(p), n);
  return hipGetLastError();
}

hipError_t launch_write_ints(int* dst, const int* src, int n, hipStream_t stream) {
  for (int base = 0; base < n; base += kIntsPerLaunch) {
    const int m = n - base < kIntsPerLaunch ? n - base : kIntsPerLaunch;
    IntChunk c;
    for (int i = 0; i < m; ++i) c.v[i] = src[base + i];
    hipLaunchKernelGGL(write_ints_kernel, dim3(1), dim3(256), 0, stream, dst + base, c, m);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace rnnk
