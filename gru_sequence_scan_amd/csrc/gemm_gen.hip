// The backward's plain products and reductions, all fp32:
//   * a strided GEMM, C (+)= A B with A(m, k) and B(k, n) addressed through
//     arbitrary strides, which covers dx = dG W_ih (A row-major, B
//     row-major) and dW = dG^T X (A read transposed) without copies;
//   * a deterministic two-pass column sum (the bias gradients);
//   * the gather of each token's incoming state h_{t-1} (the right operand
//     of dW_hh).
#include <algorithm>

#include "device_common.hpp"
#include "kernels.hpp"

namespace rnnk {

namespace {

constexpr int kGemmThreads = 256;
constexpr int kBM = 128, kBN = 128;  // output tile; four waves of 64 x 64 (2 x 2 MFMA blocks of 32 x 32)
constexpr int kBK = 32;              // k per LDS stage
// Row stride (floats) of the k-major LDS tiles: an MFMA operand read has
// lanes 0..31 on row k and lanes 32..63 on row k + 1, which this stride puts
// 32 banks apart (no conflicts).
constexpr int kLd = 160;
constexpr int kTileFloats = kBK * kLd;
constexpr int kGemmLds = 2 * 2 * kTileFloats * 4;  // two stages of both operands: 80 KiB, two workgroups per CU
constexpr int kQuads = kBM * kBK / 4 / kGemmThreads;  // groups of 4 elements per thread, operand and stage
constexpr int kXcds = 8;
// K is split so that a launch has about this many workgroups (two per CU
// of a 256-CU device). A fixed figure keeps the split, and so the rounding
// of the result, the same on every device.
constexpr int kSplitTarget = 512;
constexpr int kMinSplitK = 256;

// Operand quad q of this thread in one stage: 4 consecutive elements along
// the operand's unit-stride dimension ("fast"), at `slow` in the other.
// Operand A is [m][k]: fast = m (m-fast, the transposed dG of dW) or k
// (dG of dX); operand B is [k][n] with fast = n. Out-of-range elements
// read as zero.
struct Quad {
  int fast, slow;
};
__device__ __forceinline__ Quad quad_of(int e4, int fast_extent_quads) {
  return Quad{(e4 % fast_extent_quads) * 4, e4 / fast_extent_quads};
}

template <bool A_KFAST>
__global__ void __launch_bounds__(kGemmThreads, 2) gemm_gen_kernel(GemmGenArgs a, int kchunk) {
  extern __shared__ __attribute__((aligned(16))) float lds[];  // [stage][A, B][kBK][kLd]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;

  // XCD-aware tile order: consecutive workgroup ids go to different XCDs,
  // so ids are regrouped to give each XCD a contiguous run of tiles (same
  // k chunk and row panel, neighbouring column tiles) that share operands
  // in its L2.
  const int ntn = gridDim.x, ntm = gridDim.y;
  const int total = ntn * ntm * gridDim.z;
  int id = blockIdx.x + ntn * (blockIdx.y + ntm * blockIdx.z);
  const int full = total - total % kXcds;
  if (id < full) id = (id % kXcds) * (full / kXcds) + id / kXcds;
  const int tn = id % ntn, tm = (id / ntn) % ntm, z = id / (ntn * ntm);
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int kbeg = z * kchunk, kend = min(a.K, kbeg + kchunk);

  // this thread's quads: A is m-fast ([k][128 m]: 32 quads per k row) or
  // k-fast ([m][32 k]: 8 quads per m row); B is n-fast (32 quads per k row)
  Quad qa[kQuads], qb[kQuads];
#pragma unroll
  for (int i = 0; i < kQuads; ++i) {
    qa[i] = quad_of(tid + i * kGemmThreads, A_KFAST ? kBK / 4 : kBM / 4);
    qb[i] = quad_of(tid + i * kGemmThreads, kBN / 4);
  }
  f32x4 ra[kQuads], rb[kQuads];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < kQuads; ++i) {
      // operand A: element (m, k)
      const int m_base = m0 + (A_KFAST ? qa[i].slow : qa[i].fast);
      const int k_base = k0 + (A_KFAST ? qa[i].fast : qa[i].slow);
      if (a.vec_a) {
        ra[i] = (m_base < a.M && k_base < kend) ? *reinterpret_cast<const f32x4*>(a.A + (long long)m_base * a.sam + (long long)k_base * a.sak)
                   : f32x4{0.f, 0.f, 0.f, 0.f};
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m = m_base + (A_KFAST ? 0 : q), k = k_base + (A_KFAST ? q : 0);
          ra[i][q] = (m < a.M && k < kend) ? a.A[(long long)m * a.sam + (long long)k * a.sak] : 0.f;
        }
      }
      // operand B: element (k, n)
      const int n_base = n0 + qb[i].fast, kb = k0 + qb[i].slow;
      if (a.vec_b) {
        rb[i] = (n_base < a.N && kb < kend)
                    ? *reinterpret_cast<const f32x4*>(a.B + (long long)kb * a.sbk + (long long)n_base * a.sbn)
                    : f32x4{0.f, 0.f, 0.f, 0.f};
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n_base + q;
          rb[i][q] = (n < a.N && kb < kend) ? a.B[(long long)kb * a.sbk + (long long)n * a.sbn] : 0.f;
        }
      }
    }
  };
  auto stage = [&](int st) {  // registers -> LDS stage st, both operands k-major
    float* As = lds + st * 2 * kTileFloats;
    float* Bs = As + kTileFloats;
#pragma unroll
    for (int i = 0; i < kQuads; ++i) {
      if (A_KFAST) {
#pragma unroll
        for (int q = 0; q < 4; ++q) As[(qa[i].fast + q) * kLd + qa[i].slow] = ra[i][q];
      } else {
        *reinterpret_cast<f32x4*>(As + qa[i].slow * kLd + qa[i].fast) = ra[i];
      }
      *reinterpret_cast<f32x4*>(Bs + qb[i].slow * kLd + qb[i].fast) = rb[i];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nst = kend > kbeg ? (kend - kbeg + kBK - 1) / kBK : 0;
  if (nst > 0) {
    load(kbeg);
    stage(0);
    __syncthreads();
  }
  for (int s = 0; s < nst; ++s) {
    if (s + 1 < nst) load(kbeg + (s + 1) * kBK);  // in flight during this stage's MFMAs
    const float* As = lds + (s & 1) * 2 * kTileFloats;
    const float* Bs = As + kTileFloats;
    const int ar = half * kLd + wm * 64 + l32, br = half * kLd + wn * 64 + l32;
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 2) {
      const float a0 = As[kk * kLd + ar], a1 = As[kk * kLd + ar + 32];
      const float b0 = Bs[kk * kLd + br], b1 = Bs[kk * kLd + br + 32];
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
    }
    if (s + 1 < nst) stage((s + 1) & 1);  // the other stage: its last readers finished before the previous barrier
    __syncthreads();
  }

  // 32x32 accumulator layout: lane holds column l32, rows 8*(v/4) + 4*half + (v%4)
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 64 + j * 32 + l32;
    if (n >= a.N) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
        if (m >= a.M) continue;
        if (gridDim.z > 1) {
          a.part[((long long)z * a.M + m) * a.N + n] = acc[i][j][v];
        } else {
          float* c = a.C + (long long)m * a.ldc + n;
          *c = a.accumulate ? *c + acc[i][j][v] : acc[i][j][v];
        }
      }
  }
}

// C (+)= sum over the splits of part[z], in split order
__global__ void __launch_bounds__(256) gemm_split_reduce_kernel(const float* part, int splits, int M, int N,
                                                                 float* C, long long ldc, int accumulate) {
  const long long mn = (long long)M * N;
  for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < mn; e += (long long)gridDim.x * 256) {
    const long long m = e / N, n = e - m * N;
    float* c = C + m * ldc + n;
    float v = accumulate ? *c : 0.f;
    for (int z = 0; z < splits; ++z) v += part[z * mn + e];
    *c = v;
  }
}

// partial[c][n] = sum over rows m in chunk c of A[m * lda + n], in order
__global__ void __launch_bounds__(256) colsum_partial_kernel(const float* A, long long lda, int M, int N,
                                                             float* partial, int nchunk) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int c = blockIdx.y;
  if (n >= N) return;
  const int per = (M + nchunk - 1) / nchunk;
  const int ma = c * per, mb = min(M, ma + per);
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
  int m = ma;
  for (; m + 4 <= mb; m += 4) {
    s0 += A[(long long)m * lda + n];
    s1 += A[(long long)(m + 1) * lda + n];
    s2 += A[(long long)(m + 2) * lda + n];
    s3 += A[(long long)(m + 3) * lda + n];
  }
  for (; m < mb; ++m) s0 += A[(long long)m * lda + n];
  partial[(size_t)c * N + n] = (s0 + s1) + (s2 + s3);
}

__global__ void __launch_bounds__(256) colsum_final_kernel(const float* partial, int N, int nchunk, float* out) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  float s = 0.f;
  for (int c = 0; c < nchunk; ++c) s += partial[(size_t)c * N + n];
  out[n] = s;
}

__global__ void __launch_bounds__(256) hprev_kernel(HprevArgs a) {
  const int t = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= a.B * a.H) return;
  const int b = e / a.H, j = e - b * a.H;
  const int len = a.lengths ? a.lengths[b] : a.T;
  if (a.packed && t >= len) return;  // no packed row for (t, b)
  const long long row = (long long)(a.packed ? a.offsets[t] : t * a.B) + b;
  float v = 0.f;
  if (t < len) {
    const bool has_prev = a.rev ? (t + 1 < len) : (t >= 1);
    if (has_prev) {
      const int tp = a.rev ? t + 1 : t - 1;
      const long long prow = (long long)(a.packed ? a.offsets[tp] : tp * a.B) + b;
      v = a.y[prow * a.ldy + a.col0 + j];
    } else if (a.h0) {
      v = a.h0[(size_t)b * a.H + j];
    }
  }
  a.out[row * a.H + j] = v;
}

}  // namespace

void gemm_gen_split(int M, int N, int K, int* splits, int* kchunk) {
  const long long tiles = (long long)((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  int sp = 1;
  if (tiles > 0 && tiles < kSplitTarget && K > 2 * kMinSplitK)
    sp = (int)std::min<long long>((kSplitTarget + tiles - 1) / tiles, K / kMinSplitK);
  sp = std::max(1, std::min(sp, 64));
  int kc = (K + sp - 1) / sp;
  kc = std::max(kBK, (kc + kBK - 1) / kBK * kBK);
  *kchunk = kc;
  *splits = K > 0 ? (K + kc - 1) / kc : 1;
}

size_t gemm_gen_part_floats(int M, int N, int K) {
  int sp, kc;
  gemm_gen_split(M, N, K, &sp, &kc);
  return sp > 1 ? (size_t)sp * M * N : 0;
}

hipError_t launch_gemm_gen(const GemmGenArgs& in, hipStream_t stream) {
  if (in.M <= 0 || in.N <= 0) return hipSuccess;
  GemmGenArgs a = in;
  int splits, kchunk;
  gemm_gen_split(a.M, a.N, a.K, &splits, &kchunk);
  if (splits > 1 && !a.part) return hipErrorInvalidValue;
  const bool a_kfast = a.sak == 1 && a.sam != 1;
  auto aligned = [](const void* p) { return ((uintptr_t)p & 15u) == 0; };
  // whole quads along the unit-stride dimension: a quad is then either
  // entirely inside the operand or entirely outside
  a.vec_a = a_kfast ? (a.sam % 4 == 0 && a.K % 4 == 0 && aligned(a.A))
                    : (a.sam == 1 && a.sak % 4 == 0 && a.M % 4 == 0 && aligned(a.A));
  a.vec_b = a.sbn == 1 && a.sbk % 4 == 0 && a.N % 4 == 0 && aligned(a.B);
  const void* fn = a_kfast ? (const void*)gemm_gen_kernel<true> : (const void*)gemm_gen_kernel<false>;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kGemmLds);
  if (e != hipSuccess) return e;
  dim3 grid((a.N + kBN - 1) / kBN, (a.M + kBM - 1) / kBM, splits);
  if (a_kfast)
    launch_kernel(gemm_gen_kernel<true>, grid, dim3(kGemmThreads), kGemmLds, stream, a, kchunk);
  else
    launch_kernel(gemm_gen_kernel<false>, grid, dim3(kGemmThreads), kGemmLds, stream, a, kchunk);
  if ((e = hipGetLastError()) != hipSuccess || splits == 1) return e;
  const long long mn = (long long)a.M * a.N;
  const int blocks = (int)std::min<long long>((mn + 255) / 256, 4096);
  launch_kernel(gemm_split_reduce_kernel, dim3(blocks), dim3(256), 0, stream, a.part, splits, a.M, a.N, a.C,
                     a.ldc, a.accumulate);
  return hipGetLastError();
}

hipError_t launch_colsum(const float* A, long long lda, int M, int N, float* partial, int nchunk, float* out,
                         hipStream_t stream) {
  if (N <= 0) return hipSuccess;
  dim3 g1((N + 255) / 256, nchunk);
  launch_kernel(colsum_partial_kernel, g1, dim3(256), 0, stream, A, lda, M, N, partial, nchunk);
  launch_kernel(colsum_final_kernel, dim3((N + 255) / 256), dim3(256), 0, stream, (const float*)partial, N,
                     nchunk, out);
  return hipGetLastError();
}

hipError_t launch_hprev(const HprevArgs& a, hipStream_t stream) {
  dim3 grid((a.B * a.H + 255) / 256, a.T);
  launch_kernel(hprev_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace rnnk
