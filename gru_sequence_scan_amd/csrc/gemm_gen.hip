// The backward's plain products and reductions, all fp32:
//   * a strided GEMM, C (+)= A B with A(m, k) and B(k, n) addressed through
//     arbitrary strides, which covers dx = dG W_ih (A row-major, B
//     row-major) and dW = dG^T X (A read transposed) without copies;
//   * a deterministic two-pass column sum (the bias gradients);
//   * the gather of each token's incoming state h_{t-1} (the right operand
//     of dW_hh).
#include "device_common.hpp"
#include "kernels.hpp"

namespace rnnk {

namespace {

constexpr int kGemmThreads = 256;
constexpr int kTile = 64;   // 64 x 64 output tile, four waves of 32 x 32
constexpr int kSlab = 32;   // k per LDS stage
constexpr int kPer = kTile * kSlab / kGemmThreads;  // elements per thread per operand and stage

// Each stage's operands are loaded into registers one stage ahead, so the
// global-load latency overlaps the previous stage's MFMAs; consecutive
// threads walk each operand's unit-stride dimension (coalesced).
__global__ void __launch_bounds__(kGemmThreads) gemm_gen_kernel(GemmGenArgs a) {
  // k-major tiles: As[k][m], Bs[k][n]; one column of padding per row
  __shared__ float As[kSlab][kTile + 1];
  __shared__ float Bs[kSlab][kTile + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * kTile, n0 = blockIdx.x * kTile;
  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;
  const bool a_kfast = a.sak == 1;
  const bool b_nfast = a.sbn == 1;
  int am[kPer], ak[kPer], bn[kPer], bk[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = tid + i * kGemmThreads;
    am[i] = a_kfast ? e / kSlab : e % kTile;
    ak[i] = a_kfast ? e % kSlab : e / kTile;
    bn[i] = b_nfast ? e % kTile : e / kSlab;
    bk[i] = b_nfast ? e / kTile : e % kSlab;
  }
  float ra[kPer], rb[kPer];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int gm = m0 + am[i], gk = k0 + ak[i];
      ra[i] = (gm < a.M && gk < a.K) ? a.A[gm * a.sam + gk * a.sak] : 0.f;
      const int gn = n0 + bn[i], gk2 = k0 + bk[i];
      rb[i] = (gn < a.N && gk2 < a.K) ? a.B[gk2 * a.sbk + gn * a.sbn] : 0.f;
    }
  };
  load(0);
  for (int k0 = 0; k0 < a.K; k0 += kSlab) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      As[ak[i]][am[i]] = ra[i];
      Bs[bk[i]][bn[i]] = rb[i];
    }
    __syncthreads();
    if (k0 + kSlab < a.K) load(k0 + kSlab);
#pragma unroll
    for (int kk = 0; kk < kSlab; kk += 2)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(As[kk + half][wm * 32 + l32], Bs[kk + half][wn * 32 + l32], acc,
                                                 0, 0, 0);
    __syncthreads();
  }
  // 32x32 accumulator layout: lane holds column l32, rows 8*(v/4) + 4*half + (v%4)
  const int n = n0 + wn * 32 + l32;
  if (n < a.N) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = m0 + wm * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
      if (m < a.M) {
        float* c = a.C + m * a.ldc + n;
        *c = a.accumulate ? *c + acc[v] : acc[v];
      }
    }
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

hipError_t launch_gemm_gen(const GemmGenArgs& a, hipStream_t stream) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  dim3 grid((a.N + kTile - 1) / kTile, (a.M + kTile - 1) / kTile);
  hipLaunchKernelGGL(gemm_gen_kernel, grid, dim3(kGemmThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_colsum(const float* A, long long lda, int M, int N, float* partial, int nchunk, float* out,
                         hipStream_t stream) {
  if (N <= 0) return hipSuccess;
  dim3 g1((N + 255) / 256, nchunk);
  hipLaunchKernelGGL(colsum_partial_kernel, g1, dim3(256), 0, stream, A, lda, M, N, partial, nchunk);
  hipLaunchKernelGGL(colsum_final_kernel, dim3((N + 255) / 256), dim3(256), 0, stream, (const float*)partial, N,
                     nchunk, out);
  return hipGetLastError();
}

hipError_t launch_hprev(const HprevArgs& a, hipStream_t stream) {
  dim3 grid((a.B * a.H + 255) / 256, a.T);
  hipLaunchKernelGGL(hprev_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace rnnk
