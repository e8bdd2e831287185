// Small products on v_mfma_f32_4x4x1f32 for the RSSM kernels: batch rows
// (at most four) are the rows of each 4x4 block, output columns the lanes.
#pragma once

#include "device_common.hpp"

namespace rnnk {
namespace rssmk {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxRows = 4;  // batch rows per group: one 4x4 MFMA block row set

__host__ __device__ inline int r4(int x) { return (x + 3) & ~3; }
// Row stride (floats) of an LDS matrix whose rows are read one per lane in
// 16-byte chunks: an odd number of chunks keeps the 64 lanes of a read on
// distinct banks.
__host__ __device__ inline int ld_rows(int x) { return (r4(x) / 4) % 2 == 1 ? r4(x) : r4(x) + 4; }

// acc += sum over 16-byte chunks k4 in [k4a, k4b) of the 4x4x1 MFMA products
// of X chunk (lane's batch row) and W chunk (lane's output column). One
// accumulator: an MFMA whose accumulator input is exactly the previous MFMA's
// output issues back to back, so a single chain runs at full rate and needs
// no register shuffling. Four chunks per iteration keep their eight LDS reads
// in flight together. Bounds must be wave-uniform.
__device__ __forceinline__ f32x4 dot_chain(const float* xr, const float* wr, int k4a, int k4b, f32x4 acc) {
  k4a = __builtin_amdgcn_readfirstlane(k4a);
  k4b = __builtin_amdgcn_readfirstlane(k4b);
  int k4 = k4a;
  for (; k4 + 4 <= k4b; k4 += 4) {
    f32x4 x[4], y[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      x[q] = *reinterpret_cast<const f32x4*>(xr + 4 * (k4 + q));
      y[q] = *reinterpret_cast<const f32x4*>(wr + 4 * (k4 + q));
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_4x4x1f32(x[q][e], y[q][e], acc, 0, 0, 0);
  }
  for (; k4 < k4b; ++k4) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(xr + 4 * k4);
    const f32x4 y = *reinterpret_cast<const f32x4*>(wr + 4 * k4);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_4x4x1f32(x[e], y[e], acc, 0, 0, 0);
  }
  return acc;
}

// acc += the 4x4x1 products over chunks [k0, k0 + n) of X and W rows (n <=
// MAXC, wave-uniform), in groups of four chunks whose eight LDS reads are
// issued together (a short tail group included), so a chain of n chunks
// waits on LDS ceil(n / 4) times.
template <int MAXC>
__device__ __forceinline__ f32x4 dot_batch(const float* xr, const float* wr, int k0, int n, f32x4 acc) {
  n = __builtin_amdgcn_readfirstlane(n);
  k0 = __builtin_amdgcn_readfirstlane(k0);
#pragma unroll
  for (int i0 = 0; i0 < MAXC; i0 += 4) {
    if (i0 < n) {
      f32x4 x[4], y[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (i0 + j < n) {
          x[j] = *reinterpret_cast<const f32x4*>(xr + 4 * (k0 + i0 + j));
          y[j] = *reinterpret_cast<const f32x4*>(wr + 4 * (k0 + i0 + j));
        }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (i0 + j < n) {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_4x4x1f32(x[j][e], y[j][e], acc, 0, 0, 0);
        }
    }
  }
  return acc;
}

// dst[r * ldd + c] = src[r * ldsrc + c] for r < rows, c < cols: a global
// matrix staged into LDS by the whole workgroup, wave w taking rows w * RB
// onwards RB at a time (their loads in flight together), lanes taking
// columns. A loop of single load-store pairs waits out one memory latency
// per element.
template <int RB = 8>
__device__ __forceinline__ void stage_rows(float* dst, int ldd, const float* src, size_t ldsrc, int rows, int cols) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int c0 = 0; c0 < cols; c0 += 64) {
    const int c = c0 + lane;
    for (int r0 = wave * RB; r0 < rows; r0 += kWaves * RB) {
      float v[RB];
#pragma unroll
      for (int j = 0; j < RB; ++j)
        if (r0 + j < rows && c < cols) v[j] = src[(size_t)(r0 + j) * ldsrc + c];
#pragma unroll
      for (int j = 0; j < RB; ++j)
        if (r0 + j < rows && c < cols) dst[(r0 + j) * ldd + c] = v[j];
    }
  }
}

constexpr int kWholePassK4 = 16;  // K up to 64: one wave per 64-column pass

struct Plain {
  __device__ float operator()(int, int, float x) const { return x; }
};

// Fixed-order sum over the waves of the partials of (row v, column c) that
// the K-split products leave in `red` (kWaves waves x 4 rows x 64 floats).
__device__ __forceinline__ float red_sum(const float* red, int v, int c) {
  float s = red[v * 64 + c];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) s += red[(w * 4 + v) * 64 + c];
  return s;
}

// out[v * ldo + c] = epi(v, c, sum_{k < K} X[v * ldx + k] * W[c * ldw + k]) for
// all four rows v of X (rows past the group's batch rows hold zeros and are
// ignored by the callers) and c < N, on v_mfma_f32_4x4x1f32: 16 blocks of
// 4x4 per instruction, lane l of a pass owning output column 64 * pass + l.
// X and W rows are 16-byte aligned and zero-padded to a multiple of 4.
// Narrow products (N <= 64) split K over all waves; wider ones give each
// 64-column pass two waves that split K in halves, or whole passes per wave
// when there are more passes than wave pairs or K is short (a reduction
// through LDS and a barrier would cost more than the chain it shortens);
// partials meet in `red` (kWaves x 4 x 64 floats) and are summed in a fixed
// order.
template <typename Epi = Plain>
__device__ void mv4(const float* X, int ldx, const float* W, int ldw, float* out, int ldo, int N, int K,
                    float* red, Epi epi = Epi()) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int K4 = (K + 3) >> 2;
  const float* xr = X + (lane & 3) * ldx;
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  if (N > 64) {
    const int npass = (N + 63) >> 6;
    if (2 * npass > kWaves || K4 <= kWholePassK4) {
      for (int cg = __builtin_amdgcn_readfirstlane(wave); cg < npass; cg += kWaves) {
        const int c = cg * 64 + lane;
        const f32x4 acc = dot_chain(xr, W + (c < N ? c : N - 1) * ldw, 0, K4, zero4);
        if (c < N) {
#pragma unroll
          for (int v = 0; v < 4; ++v) out[v * ldo + c] = epi(v, c, acc[v]);
        }
      }
      return;
    }
    // pass wave / 2, K half wave % 2
    const int pass = wave >> 1, half = wave & 1, kh = (K4 + 1) >> 1;
    if (pass < npass) {
      const int c = pass * 64 + lane;
      const f32x4 acc = dot_chain(xr, W + (c < N ? c : N - 1) * ldw, half ? kh : 0, half ? K4 : kh, zero4);
#pragma unroll
      for (int v = 0; v < 4; ++v) red[((pass * 2 + half) * 4 + v) * 64 + lane] = acc[v];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 4 * N; i += kThreads) {
      const int v = i / N, c = i - v * N, p = c >> 6, l = c & 63;
      out[v * ldo + c] = epi(v, c, red[((p * 2) * 4 + v) * 64 + l] + red[((p * 2 + 1) * 4 + v) * 64 + l]);
    }
    return;
  }
  const int per = (K4 + kWaves - 1) / kWaves;
  const int ka = min(K4, wave * per), kb = min(K4, ka + per);
  const f32x4 acc = dot_chain(xr, W + (lane < N ? lane : N - 1) * ldw, ka, kb, zero4);
#pragma unroll
  for (int v = 0; v < 4; ++v) red[(wave * 4 + v) * 64 + lane] = acc[v];
  __syncthreads();
  for (int i = threadIdx.x; i < 4 * N; i += kThreads) {
    const int v = i / N, c = i - v * N;
    out[v * ldo + c] = epi(v, c, red_sum(red, v, c));
  }
}

}  // namespace rssmk
}  // namespace rnnk
