// Kernel 2b: the scan for recurrences whose gate rows fit one wavefront
// (LSTM and GRU with H <= 16), one wavefront per (direction, batch row).
//
// The apache/tvm PR "[TOPI] TE implementation of LSTM using scan" measures
// exactly such a shape (T = 256, B = 1, input and hidden 16) and finds the
// time dominated by per-step overhead rather than arithmetic. Here a step is
// a few dozen instructions of one wave and nothing else:
//   * lane 4u + q owns gate q of hidden unit u (LSTM i, f, g, o; GRU r, z,
//     n and one idle lane): its W_hh row sits in registers for the launch,
//     and the four gates of a unit meet inside their quad of lanes through
//     DPP broadcasts, at full ALU rate (no LDS round trip);
//   * every lane of a quad keeps the unit's h (and the LSTM cell c), so the
//     product W_hh h reads h_k from lane 4k with readlane;
//   * one exponential and one reciprocal per gate, with the scale of the
//     exponent folded into the lane's weights: sigmoid lanes, and tanh
//     lanes as 2 sigmoid(2y) - 1 (LSTM cell input, GRU n);
//   * no workgroup barrier and no exchange between waves (batch rows and
//     directions are independent), so waves run at their own pace and each
//     stops at its own sequence length.
// Narrow inputs (rows of at most 128 bytes in whole 16-byte chunks, the
// sequence's x within 16 KB) have their input projection inside the kernel: the wave stages its
// sequence's x in LDS once, and step k's G_x row is formed during step k - 1
// from LDS broadcasts (the input-hidden product of the same PR's three dense
// ops, here off the recurrence's dependent chain). Wider inputs read G_x
// from kernel 1, four steps ahead through a buffer resource (lanes without a
// gate row read out of range, which returns zero, so every lane issues the
// same loads and the compiler's waits count only what is needed).
// Gate conventions, bias placement, variable lengths, reverse direction and
// clipping are those of the tiled scan.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace rnnk {

namespace {

constexpr int kWaveThreads = 256;  // four independent waves per workgroup
constexpr int kWaveMaxK = 16;      // recurrent width bound (4 gates x 16 units = 64 lanes)
constexpr int kWaveXBytes = 16384; // fused input projection: x of one sequence in LDS
constexpr int kWaveRowBytes = 4096;  // and its steps' y byte offsets (n <= 1024 steps)
constexpr int kWaveLds = kWaveXBytes + kWaveRowBytes;

__device__ __forceinline__ float bcast(float v, int src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), src));
}
// value of v at lane Q of this lane's quad (DPP quad_perm [Q, Q, Q, Q])
template <int Q>
__device__ __forceinline__ float qbcast(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), Q * 0x55, 0xF, 0xF, true));
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

// CPR > 0: the input projection inside, x rows staged as CPR 16-byte chunks
// (the row's own chunks, then zeros); CPR = 0: G_x from kernel 1.
template <typename DT, bool GRU, int CPR>
__global__ void __launch_bounds__(kWaveThreads) scan_wave_kernel(ScanArgs a) {
  constexpr bool FUSED = CPR > 0;
  extern __shared__ __attribute__((aligned(16))) char lds[];  // FUSED: each wave's x
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int gw = __builtin_amdgcn_readfirstlane(blockIdx.x * (kWaveThreads / 64) + wv);
  if (a.zero_status && gw == 0 && lane == 0) *a.status = 0;
  if (gw >= a.D * a.B) return;
  const int d = gw / a.B, b = gw - d * a.B;
  const int H = a.H, K = a.K, G = a.G;
  const int DG = a.D * G, DK = a.D * K;
  const bool rev = d == 1;
  const int n = a.lengths ? __builtin_amdgcn_readfirstlane(a.lengths[b]) : a.T[0];

  // this lane's gate row r = q * H + u (valid when row_ok)
  constexpr int gates = GRU ? 3 : 4;
  const int u = lane >> 2, q = lane & 3;
  const bool row_ok = u < H && q < gates;
  const int r = q * H + u;
  const DT* whh = reinterpret_cast<const DT*>(a.w_hh[d]);
  float w[kWaveMaxK];
#pragma unroll
  for (int k = 0; k < kWaveMaxK; ++k) w[k] = (row_ok && k < K) ? to_f32<DT>(whh[(size_t)r * K + k]) : 0.f;
  float bhn = 0.f;  // GRU: b_hn stays inside the reset product
  if (GRU && a.has_bias && q == 2 && row_ok) bhn = to_f32<DT>(reinterpret_cast<const DT*>(a.b_hh[d])[r]);
  const DT* h0 = reinterpret_cast<const DT*>(a.h0[d]);
  const DT* c0 = reinterpret_cast<const DT*>(a.c0[d]);
  float h = (u < K && h0) ? to_f32<DT>(h0[(size_t)b * K + u]) : 0.f;
  float c = (!GRU && u < H && c0) ? to_f32<DT>(c0[(size_t)b * H + u]) : 0.f;

  // packed offsets through the scalar cache (never written by this kernel)
  const __attribute__((address_space(4))) int* offs = (const __attribute__((address_space(4))) int*)a.offsets;
  auto row_of = [&](int t) -> int { return a.packed ? offs[t] : t * a.B; };
  auto t_of = [&](int k) { return rev ? n - 1 - k : k; };
  DT* y = reinterpret_cast<DT*>(a.y[0]);

  // fused input projection: W_ih row and the folded biases in registers,
  // the sequence's x rows [t][in] in this wave's LDS region
  constexpr int kEpc = 16 / (int)sizeof(DT);   // elements per 16-byte chunk
  const int in_w = FUSED ? a.in_w : 0;
  const int cpr = in_w / kEpc;                  // chunks of an x row (<= CPR)
  float wi[FUSED ? CPR * kEpc : 1];
  float bias = 0.f;
  char* xl = lds + wv * kWaveLds;
  int* rowl = reinterpret_cast<int*>(xl + kWaveXBytes);
  if constexpr (FUSED) {
    const DT* wih = reinterpret_cast<const DT*>(a.w_ih[d]);
#pragma unroll
    for (int i = 0; i < CPR * kEpc; ++i) wi[i] = (row_ok && i < in_w) ? to_f32<DT>(wih[(size_t)r * in_w + i]) : 0.f;
    if (a.has_bias && row_ok) {
      bias = to_f32<DT>(reinterpret_cast<const DT*>(a.b_ih[d])[r]);
      if (!(GRU && q == 2)) bias += to_f32<DT>(reinterpret_cast<const DT*>(a.b_hh[d])[r]);
    }
    // stage each step's y byte offset (its token's row), and rows t < n as
    // CPR chunks each (zeros past the row): sixteen 16-byte loads in flight
    // per lane (one round trip for 16 KB)
    for (int t = lane; t < n; t += 64) rowl[t] = ((a.packed ? a.offsets[t] : t * a.B) + b) * DK * (int)sizeof(DT);
    const char* xs = reinterpret_cast<const char*>(a.x);
    const int total = n * CPR;
    for (int base = 0; base < total; base += 64 * 16) {
      u32x4 v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int ch = base + i * 64 + lane;
        const int t = ch / CPR, cc = ch - t * CPR;
        const bool ld = ch < total && cc < cpr;
        const int row = ld ? (a.packed ? a.offsets[t] : t * a.B) + b : 0;
        v[i] = ld ? *reinterpret_cast<const u32x4*>(xs + ((size_t)row * in_w + cc * kEpc) * sizeof(DT))
                  : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int ch = base + i * 64 + lane;
        if (ch < total) *reinterpret_cast<u32x4*>(xl + ch * 16) = v[i];
      }
    }
  }
  // Each lane's pre-activation enters exp2 scaled: sigmoid lanes by
  // -log2(e), tanh lanes (LSTM cell input, GRU n; tanh y = 2 sigmoid(2y) - 1)
  // by -2 log2(e). The scale is folded into the lane's weight rows and
  // biases, so the product's chain ends at the exponent.
  constexpr float kL2e = 1.44269504088896341f;
  const bool th = q == 2;
  const float es = th ? -2.0f * kL2e : -kL2e;
#pragma unroll
  for (int k = 0; k < kWaveMaxK; ++k) w[k] *= es;
  bhn *= es;
  if constexpr (FUSED) {
#pragma unroll
    for (int i = 0; i < CPR * kEpc; ++i) wi[i] *= es;
    bias *= es;
  }
  const float fa = th ? 2.0f : 1.0f, fb = th ? -1.0f : 0.0f;  // LSTM: act = fa * sigmoid + fb
  // The weights, initial state and staged x feed the loop through
  // loop-carried registers and LDS; waiting for them here keeps the loop's
  // own waits down to what it issues itself.
  __builtin_amdgcn_s_waitcnt(0);

  // G_x of the fused path: the x row of step k read from LDS (a broadcast:
  // every lane reads the same address), then the projection
  u32x4 xrow[FUSED ? CPR : 1];
  int xrow_at = 0;  // the y byte offset of that step's row
  auto x_read = [&](int k) __attribute__((always_inline)) {
    const int t = t_of(k < n ? k : n - 1);
    const u32x4* src = reinterpret_cast<const u32x4*>(xl + t * CPR * 16);
#pragma unroll
    for (int cc = 0; cc < (FUSED ? CPR : 0); ++cc) xrow[cc] = src[cc];
    xrow_at = rowl[t];
  };
  auto x_proj = [&]() __attribute__((always_inline)) -> float {
    float s0 = bias, s1 = 0.f;
#pragma unroll
    for (int cc = 0; cc < (FUSED ? CPR : 0); ++cc) {
#pragma unroll
      for (int e = 0; e < kEpc; ++e) {
        const uint32_t word = xrow[cc][e * (int)sizeof(DT) / 4];
        const float xv = sizeof(DT) == 4 ? __builtin_bit_cast(float, word)
                                         : __builtin_bit_cast(float, (e & 1) ? (word & 0xFFFF0000u) : (word << 16));
        if (e & 1) s1 = fmaf(wi[cc * kEpc + e], xv, s1);
        else s0 = fmaf(wi[cc * kEpc + e], xv, s0);
      }
    }
    // lanes without a gate row take zero (whatever x holds), so their
    // state stays finite and adds exact zeros to the product
    return row_ok ? s0 + s1 : 0.f;
  };
  // G_x of step k from kernel 1 (clamped into the sequence)
  auto gx_load = [&](int k) -> float {
    const int t = t_of(k < n ? k : n - 1);
    // (fp32 G_x: the host keeps G_x in fp32 for layers this kernel runs)
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(reinterpret_cast<const float*>(a.gx[0]) + ((size_t)(row_of(t) + b) * DG + d * G), (uint32_t)G * 4u);
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, row_ok ? r * 4 : 0x40000000, 0, 0)) * es;
  };

  // y through one resource from this direction's column: a row's offset is
  // below 2^31 bytes (the host checks), and the lanes that do not store get
  // an offset past the resource's end.
  const __amdgpu_buffer_rsrc_t ys = make_rsrc(y + d * K, 0x7FFFFFFFu);

  // One step; gx is the lane's scaled G_x and `row` the byte offset of step
  // k's y row. Steps past the sequence (the tail of the last group of four
  // on the G_x path) run the same instructions with the state kept and the
  // store sent out of range, so every path issues the same memory
  // operations. CLIP: clamp the cell (a second copy of the loop without it
  // keeps four dependent operations off the chain).
  const float c_lo = a.c_lo, c_hi = a.c_hi;
  auto step = [&](int k, float gx, int row, auto clip) __attribute__((always_inline)) {
    constexpr bool CLIP = decltype(clip)::value;
    const bool on = k < n;
    // h_k sits on lanes 4k .. 4k + 3; w[k >= K] = 0, so the padded terms add
    // exact zeros and the product has no branches
    // (all sixteen reads first, into distinct registers, then four
    // independent chains: one register reused for every read would
    // serialise read, wait and multiply-add sixteen times)
    float hk[kWaveMaxK];
#pragma unroll
    for (int k2 = 0; k2 < kWaveMaxK; ++k2) hk[k2] = bcast(h, 4 * k2);
    // (GRU n lanes start from b_hn: their product stays apart from G_x)
    float acc4[4] = {GRU && th ? bhn : gx, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k2 = 0; k2 < kWaveMaxK; ++k2) acc4[k2 & 3] = fmaf(w[k2], hk[k2], acc4[k2 & 3]);
    const float acc = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
    const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(acc));  // sigmoid
    if constexpr (GRU) {
      // n lanes: tanh(gx + r (W_hn h + b_hn)), scaled like the rest
      const float v = fmaf(qbcast<0>(sg), acc, gx);
      const float nn = fmaf(__builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(v)), 2.0f, -1.0f);
      const float z = qbcast<1>(sg), nq = qbcast<2>(nn);
      const float hn = fmaf(z, h - nq, nq);  // (1 - z) n + z h
      h = on ? hn : h;
    } else {
      const float act = fmaf(sg, fa, fb);  // i, f, g (tanh), o
      float cn = fmaf(qbcast<1>(act), c, qbcast<0>(act) * qbcast<2>(act));
      if constexpr (CLIP) cn = clampf(cn, c_lo, c_hi);
      const float tc = fmaf(__builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(cn * (-2.0f * kL2e))), 2.0f, -1.0f);
      const float hn = qbcast<3>(act) * tc;
      c = on ? cn : c;
      h = on ? hn : h;
    }
    // one lane per unit stores; the others fall outside the resource
    store_out<DT>(ys, (on && q == 0 && u < K) ? (uint32_t)row + u * (uint32_t)sizeof(DT) : 0x80000000u, h);
  };

  auto run = [&](auto clip) __attribute__((always_inline)) {
  if constexpr (FUSED) {
    // step k + 1's x row is read before step k's dependent chain and its
    // projection formed after it, so the LDS latency and the products
    // overlap the chain
    x_read(0);
    float gcur = x_proj();
    int rcur = xrow_at;
    for (int k = 0; k < n; ++k) {
      x_read(k + 1);
      step(k, gcur, rcur, clip);
      gcur = x_proj();
      rcur = xrow_at;
    }
  } else {
    // Steps in groups of four, each followed by the load four steps ahead.
    // The first group is peeled so that the loop is always entered with the
    // same pattern of outstanding stores and loads as on its back edge: the
    // wait before each step then counts exactly the six younger operations.
    float g0 = gx_load(0), g1 = gx_load(1), g2 = gx_load(2), g3 = gx_load(3);
    auto row_at = [&](int k) { return (row_of(t_of(k < n ? k : n - 1)) + b) * DK * (int)sizeof(DT); };
    auto group = [&](int k) {
      step(k, g0, row_at(k), clip);
      g0 = gx_load(k + 4);
      step(k + 1, g1, row_at(k + 1), clip);
      g1 = gx_load(k + 5);
      step(k + 2, g2, row_at(k + 2), clip);
      g2 = gx_load(k + 6);
      step(k + 3, g3, row_at(k + 3), clip);
      g3 = gx_load(k + 7);
    };
    group(0);
    for (int k = 4; k < n; k += 4) group(k);
  }
  };
  if (!GRU && (c_lo > -__builtin_inff() || c_hi < __builtin_inff()))
    run(std::true_type{});
  else
    run(std::false_type{});
  DT* hn = reinterpret_cast<DT*>(a.h_n[d]);
  DT* cn = reinterpret_cast<DT*>(a.c_n[d]);
  if (hn && q == 0 && u < K) hn[(size_t)b * K + u] = from_f32<DT>(h);
  if (!GRU && cn && q == 0 && u < H) cn[(size_t)b * H + u] = from_f32<DT>(c);
}

template <typename DT, bool GRU, int CPR>
hipError_t launch_as(const ScanArgs& a, hipStream_t stream) {
  const int waves = a.D * a.B;
  const int grid = (waves + kWaveThreads / 64 - 1) / (kWaveThreads / 64);
  const int lds = CPR > 0 ? (kWaveThreads / 64) * kWaveLds : 0;
  if (CPR > 0) {
    const hipError_t e = hipFuncSetAttribute((const void*)scan_wave_kernel<DT, GRU, CPR>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
  }
  launch_kernel((scan_wave_kernel<DT, GRU, CPR>), dim3(grid), dim3(kWaveThreads), lds, stream, a);
  return hipGetLastError();
}

// chunks an x row is staged as: the row's own rounded up to a power of two
int staged_chunks(int in_w, int esize) {
  const int c = in_w * esize / 16;
  return c <= 1 ? 1 : c <= 2 ? 2 : c <= 4 ? 4 : 8;
}

template <typename DT, bool GRU>
hipError_t launch_mode(const ScanArgs& a, hipStream_t stream) {
  if (!a.x) return launch_as<DT, GRU, 0>(a, stream);
  switch (staged_chunks(a.in_w, (int)sizeof(DT))) {
    case 1: return launch_as<DT, GRU, 1>(a, stream);
    case 2: return launch_as<DT, GRU, 2>(a, stream);
    case 4: return launch_as<DT, GRU, 4>(a, stream);
    default: return launch_as<DT, GRU, 8>(a, stream);
  }
}

template <typename DT>
hipError_t launch_dt(const ScanArgs& a, hipStream_t stream) {
  return a.mode == kGRU ? launch_mode<DT, true>(a, stream) : launch_mode<DT, false>(a, stream);
}

}  // namespace

bool scan_wave_fits(int mode, int H, int K) { return mode != kLSTMP && K == H && H >= 1 && H <= kWaveMaxK; }

bool scan_wave_fuses(int in_w, int esize, long long max_steps) {
  return in_w >= 1 && in_w * esize <= 128 && in_w * esize % 16 == 0 &&
         max_steps * staged_chunks(in_w, esize) * 16 <= kWaveXBytes && max_steps * 4 <= kWaveRowBytes;
}

int scan_wave_lds_bytes(int in_w, int esize, long long max_steps) {
  return scan_wave_fuses(in_w, esize, max_steps) ? (kWaveThreads / 64) * kWaveLds : 0;
}

int scan_wave_grid(int D, int B) { return (D * B + kWaveThreads / 64 - 1) / (kWaveThreads / 64); }

hipError_t launch_scan_wave(const ScanArgs& a, int dtype_bf16, hipStream_t stream) {
  if (!scan_wave_fits(a.mode, a.H, a.K)) return hipErrorInvalidValue;
  if (a.x && !scan_wave_fuses(a.in_w, dtype_bf16 ? 2 : 4, a.T[0])) return hipErrorInvalidValue;
  return dtype_bf16 ? launch_dt<bf16>(a, stream) : launch_dt<float>(a, stream);
}

}  // namespace rnnk
