// Small stream-ordered helpers: zero-fill of workspace words and copies of
// host int arrays (lengths, packed offsets) into the workspace through
// kernel arguments, so nothing has to stay alive on the host after a call;
// and a probe of the device-coherent round trip that bounds every step of
// the persistent kernels.
#include "device_common.hpp"
#include "kernels.hpp"

namespace rnnk {

namespace {

__global__ void fill_u32_kernel(uint32_t* p, size_t n, uint32_t value) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = value;
}

// Element i < n1 of the joint range goes to p1, the rest to p2.
__global__ void fill2_u32_kernel(uint32_t* p1, size_t n1, uint32_t v1, uint32_t* p2, size_t n2, uint32_t v2) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n1 + n2; i += (size_t)gridDim.x * blockDim.x) {
    if (i < n1)
      p1[i] = v1;
    else
      p2[i - n1] = v2;
  }
}

struct IntChunk {
  int v[kIntsPerLaunch];
};

__global__ void write_ints_kernel(int* dst, IntChunk c, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = c.v[i];
}

// Two workgroups (ids 0 and 1, which the dispatcher places on different
// XCDs) pass a counter back and forth through two words 256 bytes apart,
// with the same device-scope stores and loads the persistent kernels use
// for their exchange. Word 0 carries A's value, word 64 B's echo. Every
// wait is bounded by `spin` polls; a wait that runs out sets out[1].
__global__ void exchange_probe_kernel(unsigned* buf, int iters, unsigned spin, unsigned long long* out) {
  if (threadIdx.x != 0 || blockIdx.x > 1) return;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(buf, 512);
  const bool a_side = blockIdx.x == 0;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  unsigned failed = 0;
  for (int i = 1; i <= iters && !failed; ++i) {
    if (a_side) {
      coh_store4(rs, 0, (unsigned)i);
      unsigned n = 0;
      while (coh_poll4(rs, 256) != (unsigned)i)
        if (++n > spin) { failed = 1; break; }
    } else {
      unsigned n = 0;
      while (coh_poll4(rs, 0) != (unsigned)i)
        if (++n > spin) { failed = 1; break; }
      if (!failed) coh_store4(rs, 256, (unsigned)i);
    }
  }
  wait_all_mem();
  const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
  if (a_side) {
    out[0] = t1 - t0;
    out[1] = failed;
  } else {
    out[2] = failed;
  }
}

__global__ void copy_int_kernel(int* dst, const int* src) {
  if (threadIdx.x == 0) *dst = *src;
}

}  // namespace

hipError_t launch_copy_int(int* dst, const int* src, hipStream_t stream) {
  launch_kernel(copy_int_kernel, dim3(1), dim3(64), 0, stream, dst, src);
  return hipGetLastError();
}

hipError_t launch_exchange_probe(void* buf, int iters, unsigned long long* out, hipStream_t stream) {
  launch_kernel(exchange_probe_kernel, dim3(2), dim3(64), 0, stream, reinterpret_cast<unsigned*>(buf), iters,
                     2000000u, out);
  return hipGetLastError();
}

hipError_t launch_fill_u32(void* p, size_t bytes, uint32_t value, hipStream_t stream) {
  const size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  const size_t want = (n + 255) / 256;
  const int blocks = (int)(want < 256 ? want : 256);
  launch_kernel(fill_u32_kernel, dim3(blocks), dim3(256), 0, stream, reinterpret_cast<uint32_t*>(p), n, value);
  return hipGetLastError();
}

hipError_t launch_fill2_u32(void* p1, size_t bytes1, uint32_t value1, void* p2, size_t bytes2, uint32_t value2,
                            hipStream_t stream) {
  const size_t n1 = bytes1 / 4, n2 = bytes2 / 4;
  if (n1 + n2 == 0) return hipSuccess;
  const size_t want = (n1 + n2 + 255) / 256;
  const int blocks = (int)(want < 256 ? want : 256);
  launch_kernel(fill2_u32_kernel, dim3(blocks), dim3(256), 0, stream, reinterpret_cast<uint32_t*>(p1), n1, value1,
                reinterpret_cast<uint32_t*>(p2), n2, value2);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream) { return launch_fill_u32(p, bytes, 0u, stream); }

hipError_t launch_write_ints(int* dst, const int* src, int n, hipStream_t stream) {
  for (int base = 0; base < n; base += kIntsPerLaunch) {
    const int m = n - base < kIntsPerLaunch ? n - base : kIntsPerLaunch;
    IntChunk c;
    for (int i = 0; i < m; ++i) c.v[i] = src[base + i];
    launch_kernel(write_ints_kernel, dim3(1), dim3(256), 0, stream, dst + base, c, m);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace rnnk
