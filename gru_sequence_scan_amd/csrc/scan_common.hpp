// Pieces shared by the forward and backward persistent scans: LDS-resident
// products on MFMA or the vector ALUs, the coherent tile copy, and the
// weight-slice loader. Workgroups of these kernels have kScanThreads threads.
#pragma once

#include "device_common.hpp"

namespace rnnk {
namespace {

constexpr int kScanThreads = 256;

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations (the s_waitcnt immediate keeps vmcnt and expcnt at their
// maximum, lgkmcnt 0) and meets the other waves. __syncthreads also drains
// every outstanding global store, which a barrier that only orders LDS
// accesses does not need.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One 16-byte chunk per lane of each operand feeds one 16x16 MFMA step:
// bf16 16x16x32 takes 8 values of k per lane directly; fp32 16x16x4 takes
// one value per lane per instruction, so the chunk's 4 values go to 4
// instructions. Lane l supplies k-group l / 16 of every step for both
// operands, which keeps each dot product intact.
template <typename DT>
struct Chunk;
template <>
struct Chunk<bf16> {
  typedef bf16x8 T;
  static constexpr int kK = 32;  // k covered by one chunk across the 4 lane quads
  __device__ static f32x4 mfma(const T& a, const T& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Chunk<float> {
  typedef f32x4 T;
  static constexpr int kK = 16;
  __device__ static f32x4 mfma(const T& a, const T& b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
  }
};

// NT output tiles of one wave over the whole K, two chunks of loads in flight;
// each finished 16x16 accumulator goes to epi(tm, tn, c), where lane l holds
// column tn * 16 + l % 16, rows tm * 16 + 4 * (l / 16) + v.
template <typename DT, int NT, typename Epi>
__device__ __forceinline__ void mm_tiles_epi(const DT* As, int as_ld, const DT* Ws, int w_ld, const int* tm,
                                             const int* tn, int kp, Epi&& epi) {
  typedef typename Chunk<DT>::T V;
  constexpr int kEpc = 16 / sizeof(DT);
  constexpr int kK = Chunk<DT>::kK;
  const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
  const DT* ap[NT];
  const DT* bp[NT];
  f32x4 c[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    ap[j] = As + (tm[j] * 16 + lr) * as_ld + lq * kEpc;
    bp[j] = Ws + (tn[j] * 16 + lr) * w_ld + lq * kEpc;
    c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int nch = kp / kK;
  int ch = 0;
  for (; ch + 1 < nch; ch += 2) {
    V a0[NT], b0[NT], a1[NT], b1[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      a0[j] = *reinterpret_cast<const V*>(ap[j] + ch * kK);
      b0[j] = *reinterpret_cast<const V*>(bp[j] + ch * kK);
      a1[j] = *reinterpret_cast<const V*>(ap[j] + (ch + 1) * kK);
      b1[j] = *reinterpret_cast<const V*>(bp[j] + (ch + 1) * kK);
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) c[j] = Chunk<DT>::mfma(a0[j], b0[j], c[j]);
#pragma unroll
    for (int j = 0; j < NT; ++j) c[j] = Chunk<DT>::mfma(a1[j], b1[j], c[j]);
  }
  if (ch < nch) {
    V a0[NT], b0[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      a0[j] = *reinterpret_cast<const V*>(ap[j] + ch * kK);
      b0[j] = *reinterpret_cast<const V*>(bp[j] + ch * kK);
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) c[j] = Chunk<DT>::mfma(a0[j], b0[j], c[j]);
  }
#pragma unroll
  for (int j = 0; j < NT; ++j) epi(tm[j], tn[j], c[j]);
}

template <typename DT, int NT>
__device__ __forceinline__ void mm_tiles(const DT* As, int as_ld, const DT* Ws, int w_ld, float* acc, int acc_ld,
                                         const int* tm, const int* tn, int kp) {
  const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
  mm_tiles_epi<DT, NT>(As, as_ld, Ws, w_ld, tm, tn, kp, [&](int m, int n, const f32x4& c) {
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[(m * 16 + 4 * lq + v) * acc_ld + n * 16 + lr] = c[v];
  });
}

// acc[r][c] = sum_k A[r][k] * W[c][k] on 16x16 MFMA tiles (rows a multiple
// of 16), A and W in LDS. Each wave takes a contiguous run of tiles and
// computes up to four of them together.
template <typename DT>
__device__ void mm_mfma(const char* lds, int as_off, int as_ld, int w_off, int w_ld, float* acc,
                        int acc_ld, int mtiles, int ntiles, int kp) {
  const DT* As = reinterpret_cast<const DT*>(lds + as_off);
  const DT* Ws = reinterpret_cast<const DT*>(lds + w_off);
  const int wave = threadIdx.x >> 6;
  const int total = mtiles * ntiles;
  const int per = (total + 3) / 4;
  int t0 = wave * per;
  const int t1 = min(total, t0 + per);
  while (t0 < t1) {
    const int n = min(4, t1 - t0);
    int tm[4], tn[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tt = t0 + min(j, n - 1);
      tm[j] = tt / ntiles;
      tn[j] = tt - tm[j] * ntiles;
    }
    switch (n) {
      case 1: mm_tiles<DT, 1>(As, as_ld, Ws, w_ld, acc, acc_ld, tm, tn, kp); break;
      case 2: mm_tiles<DT, 2>(As, as_ld, Ws, w_ld, acc, acc_ld, tm, tn, kp); break;
      case 3: mm_tiles<DT, 3>(As, as_ld, Ws, w_ld, acc, acc_ld, tm, tn, kp); break;
      default: mm_tiles<DT, 4>(As, as_ld, Ws, w_ld, acc, acc_ld, tm, tn, kp); break;
    }
    t0 += n;
  }
}

// The same tiling with each finished accumulator handed to epi (mm_tiles_epi's
// layout) instead of written to LDS.
template <typename DT, typename Epi>
__device__ void mm_mfma_epi(const char* lds, int as_off, int as_ld, int w_off, int w_ld, int mtiles, int ntiles,
                            int kp, Epi&& epi) {
  const DT* As = reinterpret_cast<const DT*>(lds + as_off);
  const DT* Ws = reinterpret_cast<const DT*>(lds + w_off);
  const int wave = threadIdx.x >> 6;
  const int total = mtiles * ntiles;
  const int per = (total + 3) / 4;
  int t0 = wave * per;
  const int t1 = min(total, t0 + per);
  while (t0 < t1) {
    const int n = min(4, t1 - t0);
    int tm[4], tn[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tt = t0 + min(j, n - 1);
      tm[j] = tt / ntiles;
      tn[j] = tt - tm[j] * ntiles;
    }
    switch (n) {
      case 1: mm_tiles_epi<DT, 1>(As, as_ld, Ws, w_ld, tm, tn, kp, epi); break;
      case 2: mm_tiles_epi<DT, 2>(As, as_ld, Ws, w_ld, tm, tn, kp, epi); break;
      case 3: mm_tiles_epi<DT, 3>(As, as_ld, Ws, w_ld, tm, tn, kp, epi); break;
      default: mm_tiles_epi<DT, 4>(As, as_ld, Ws, w_ld, tm, tn, kp, epi); break;
    }
    t0 += n;
  }
}

// Same product on the vector ALUs for small batch blocks (bb < 16).
template <typename DT>
__device__ __forceinline__ void mm_valu(const char* lds, int as_off, int as_ld, int w_off, int w_ld, float* acc,
                                        int acc_ld, int rows, int cols, int kp) {
  lds_gemv_rows<DT, 4, 2>(reinterpret_cast<const DT*>(lds + as_off), as_ld,
                          reinterpret_cast<const DT*>(lds + w_off), w_ld, acc, acc_ld, rows, cols,
                          kp * (int)sizeof(DT) / 16);
}

// Copy `rows` rows of `width_el` elements from a coherent exchange buffer
// (row stride `src_ld` elements) into LDS (row stride `dst_ld`). Rows whose
// batch index is outside [0, B) are zero-filled.
template <typename DT>
__device__ void load_tile_coherent(__amdgpu_buffer_rsrc_t rs, uint32_t src_base_el, int src_ld, int b0,
                                   int B, int rows, int width_el, char* lds, int dst_off, int dst_ld) {
  constexpr int kEpc = 16 / sizeof(DT);
  const int cpr = width_el / kEpc;
  const int total = rows * cpr;
  DT* dst = reinterpret_cast<DT*>(lds + dst_off);
  for (int base = 0; base < total; base += kScanThreads * 8) {
    u32x4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = base + i * kScanThreads + threadIdx.x;
      const int r = idx / cpr, cc = idx - r * cpr;
      if (idx < total && b0 + r < B)
        v[i] = coh_load16(rs, (src_base_el + (uint32_t)(r * src_ld + cc * kEpc)) * sizeof(DT));
      else
        v[i] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = base + i * kScanThreads + threadIdx.x;
      if (idx < total) {
        const int r = idx / cpr, cc = idx - r * cpr;
        *reinterpret_cast<u32x4*>(dst + r * dst_ld + cc * kEpc) = v[i];
      }
    }
  }
}

// Load `nrows` weight rows into LDS as [nrows][ld], zero-padding k >= klen
// and rows for which row_of() returns -1.
template <typename DT, typename RowFn>
__device__ void load_weights(const DT* w, int klen, int kpad, int nrows, RowFn row_of, char* lds,
                             int off, int ld) {
  DT* dst = reinterpret_cast<DT*>(lds + off);
  const int total = nrows * kpad;
  for (int idx = threadIdx.x; idx < total; idx += kScanThreads) {
    const int r = idx / kpad, k = idx - r * kpad;
    const int gr = row_of(r);
    dst[r * ld + k] = (gr >= 0 && k < klen) ? w[(size_t)gr * klen + k] : (DT)0.0f;
  }
}


}  // namespace
}  // namespace rnnk
