// Kernel 2b: the scan for recurrences whose gate rows fit one wavefront
// (gates * H <= 64: LSTM with H <= 16, GRU with H <= 21), one wavefront per
// (direction, batch row).
//
// The apache/tvm PR "[TOPI] TE implementation of LSTM using scan" measures
// exactly such a shape (T = 256, B = 1, input and hidden 16) and finds the
// time dominated by per-step overhead rather than arithmetic. Here a step is
// a few dozen instructions of one wave and nothing else:
//   * lane j owns gate row j: its W_hh row sits in registers for the launch;
//   * lane u < H owns hidden unit u: h_u (and the LSTM cell c_u) in a
//     register; the product W_hh h reads h_k from lane k with readlane;
//   * the gate values meet at the unit lanes through cross-lane permutes;
//   * no LDS, no workgroup barrier, no exchange between waves (batch rows
//     and directions are independent), so waves run at their own pace and
//     each stops at its own sequence length;
//   * Gx is read four steps ahead through a buffer resource (lanes past G
//     read out of range, which returns zero, so every lane issues the same
//     loads and the compiler's waits count only what is needed).
// Gate conventions, bias placement, variable lengths, reverse direction and
// clipping are those of the tiled scan.
#include "device_common.hpp"
#include "kernels.hpp"

namespace rnnk {

namespace {

constexpr int kWaveThreads = 256;  // four independent waves per workgroup
constexpr int kWaveMaxK = 21;      // recurrent width bound (GRU: 3 * 21 = 63 rows)

__device__ __forceinline__ float bcast(float v, int src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), src));
}
// value of v at lane src (0 <= src < 64) for every lane
__device__ __forceinline__ float from_lane(float v, int src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, v)));
}

template <typename DT>
__device__ __forceinline__ void store_out(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off, float v);
template <>
__device__ __forceinline__ void store_out<float>(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rs, (int)byte_off, 0, 0);
}
template <>
__device__ __forceinline__ void store_out<bf16>(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off, float v) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (bf16)v), rs, (int)byte_off, 0, 0);
}

template <typename DT, bool GRU>
__global__ void __launch_bounds__(kWaveThreads) scan_wave_kernel(ScanArgs a) {
  constexpr int kMaxK = GRU ? 21 : 16;  // 3 * 21 or 4 * 16 gate rows fit 64 lanes
  const int lane = threadIdx.x & 63;
  const int gw = __builtin_amdgcn_readfirstlane(blockIdx.x * (kWaveThreads / 64) + (threadIdx.x >> 6));
  if (gw >= a.D * a.B) return;
  const int d = gw / a.B, b = gw - d * a.B;
  const int H = a.H, K = a.K, G = a.G;
  const int DG = a.D * G, DK = a.D * K;
  const bool rev = d == 1;
  const int n = a.lengths ? __builtin_amdgcn_readfirstlane(a.lengths[b]) : a.T[0];

  // this lane's gate row: gate q, unit u
  const int q = lane / H, u = lane - q * H;
  const DT* whh = reinterpret_cast<const DT*>(a.w_hh[d]);
  float w[kMaxK];
#pragma unroll
  for (int k = 0; k < kMaxK; ++k) w[k] = (lane < G && k < K) ? to_f32<DT>(whh[(size_t)lane * K + k]) : 0.f;
  float bhn = 0.f;  // GRU: b_hn stays inside the reset product
  if (GRU && a.has_bias && q == 2 && lane < G) bhn = to_f32<DT>(reinterpret_cast<const DT*>(a.b_hh[d])[lane]);
  const DT* h0 = reinterpret_cast<const DT*>(a.h0[d]);
  const DT* c0 = reinterpret_cast<const DT*>(a.c0[d]);
  float h = (lane < K && h0) ? to_f32<DT>(h0[(size_t)b * K + lane]) : 0.f;
  float c = (!GRU && lane < H && c0) ? to_f32<DT>(c0[(size_t)b * H + lane]) : 0.f;
  const int l = lane < H ? lane : 0;  // unit lanes gather from l + g * H
  // The weights and initial state feed the step loop through loop-carried
  // registers; waiting for them here keeps the loop's own waits down to the
  // Gx prefetch.
  __builtin_amdgcn_s_waitcnt(0);

  // packed offsets through the scalar cache (never written by this kernel)
  const __attribute__((address_space(4))) int* offs = (const __attribute__((address_space(4))) int*)a.offsets;
  auto row_of = [&](int t) -> int { return a.packed ? offs[t] : t * a.B; };
  auto t_of = [&](int k) { return rev ? n - 1 - k : k; };
  auto gx_at = [&](int k) -> float {  // Gx of step k (clamped into the sequence)
    const int t = t_of(k < n ? k : n - 1);
    // (fp32 G_x: the host keeps G_x in fp32 for layers this kernel runs)
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(reinterpret_cast<const float*>(a.gx[0]) + ((size_t)(row_of(t) + b) * DG + d * G), (uint32_t)G * 4u);
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, lane * 4, 0, 0));
  };
  DT* y = reinterpret_cast<DT*>(a.y[0]);

  // One step. Steps past the sequence (the tail of the last group of four)
  // run the same instructions with the state kept and the store sent out of
  // range, so every path issues the same memory operations.
  auto step = [&](int k, float gx) {
    const bool on = k < n;
    const int t = t_of(on ? k : n - 1);
    // lanes >= K hold h = 0 and w[j >= K] = 0, so the padded terms add
    // exact zeros and the product has no branches
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) acc = fmaf(w[j], bcast(h, j), acc);
    if constexpr (GRU) {
      const float rz = fsigmoid(gx + acc);            // r on lanes [0, H), z on [H, 2H)
      const float rr = from_lane(rz, u);              // the unit's r, wanted on n lanes
      const float nn = ftanh(gx + rr * (acc + bhn));  // n on lanes [2H, 3H)
      const float zg = from_lane(rz, H + l);
      const float ng = from_lane(nn, 2 * H + l);
      const float hn = (1.f - zg) * ng + zg * h;
      h = lane < K ? (on ? hn : h) : 0.f;
    } else {
      const float act = q == 2 ? ftanh(gx + acc) : fsigmoid(gx + acc);
      const float fg = from_lane(act, H + l);
      const float gg = from_lane(act, 2 * H + l);
      const float og = from_lane(act, 3 * H + l);
      const float cn = clampf(fg * c + act * gg, a.c_lo, a.c_hi);  // act is i on the unit lanes
      const float hn = og * ftanh(cn);
      c = lane < H ? (on ? cn : c) : 0.f;
      h = lane < K ? (on ? hn : h) : 0.f;
    }
    const __amdgpu_buffer_rsrc_t ys =
        make_rsrc(y + ((size_t)(row_of(t) + b) * DK + d * K), (uint32_t)(K * sizeof(DT)));
    // lanes >= K fall outside the resource and store nothing
    store_out<DT>(ys, on ? lane * (uint32_t)sizeof(DT) : 0x80000000u, h);
  };

  // Steps in groups of four, each followed by the load four steps ahead.
  // The first group is peeled so that the loop is always entered with the
  // same pattern of outstanding stores and loads as on its back edge: the
  // wait before each step then counts exactly the six younger operations.
  float g0 = gx_at(0), g1 = gx_at(1), g2 = gx_at(2), g3 = gx_at(3);
  auto group = [&](int k) {
    step(k, g0);
    g0 = gx_at(k + 4);
    step(k + 1, g1);
    g1 = gx_at(k + 5);
    step(k + 2, g2);
    g2 = gx_at(k + 6);
    step(k + 3, g3);
    g3 = gx_at(k + 7);
  };
  group(0);
  for (int k = 4; k < n; k += 4) group(k);
  DT* hn = reinterpret_cast<DT*>(a.h_n[d]);
  DT* cn = reinterpret_cast<DT*>(a.c_n[d]);
  if (hn && lane < K) hn[(size_t)b * K + lane] = from_f32<DT>(h);
  if (!GRU && cn && lane < H) cn[(size_t)b * H + lane] = from_f32<DT>(c);
}

template <typename DT, bool GRU>
hipError_t launch_as(const ScanArgs& a, hipStream_t stream) {
  const int waves = a.D * a.B;
  const int grid = (waves + kWaveThreads / 64 - 1) / (kWaveThreads / 64);
  hipLaunchKernelGGL((scan_wave_kernel<DT, GRU>), dim3(grid), dim3(kWaveThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

bool scan_wave_fits(int mode, int H, int K) { return mode != kLSTMP && K == H && K <= kWaveMaxK && (mode == kGRU ? 3 : 4) * H <= 64; }

int scan_wave_grid(int D, int B) { return (D * B + kWaveThreads / 64 - 1) / (kWaveThreads / 64); }

hipError_t launch_scan_wave(const ScanArgs& a, int dtype_bf16, hipStream_t stream) {
  if (!scan_wave_fits(a.mode, a.H, a.K)) return hipErrorInvalidValue;
  if (a.mode == kGRU) return dtype_bf16 ? launch_as<bf16, true>(a, stream) : launch_as<float, true>(a, stream);
  return dtype_bf16 ? launch_as<bf16, false>(a, stream) : launch_as<float, false>(a, stream);
}

}  // namespace rnnk
