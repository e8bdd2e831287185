// Device-side building blocks shared by the gfx950 kernels: device-coherent
// exchange buffers, the per-step group barrier with its watchdog, the gate
// activations and small vector types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rnnk {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Device status word values (mirror RnnStatus).
constexpr int kStatusOk = 0;
constexpr int kStatusTimeout = -9;

// ---------------------------------------------------------------------------
// Device-coherent access. Workgroups of one persistent launch exchange the
// recurrent state through small global buffers every step. The L2 of each
// XCD is not coherent with the others, so these buffers are written and read
// with device-scope cache policy (the sc1 bit) on buffer instructions: the
// write reaches the device coherence point before its completion is counted,
// and the read is served from there. Ordinary loads and stores are used for
// everything that is read-only during the launch.
// ---------------------------------------------------------------------------
constexpr int kCohPolicy = 16;  // sc1: device scope

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 coh_load16(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(rs, (int)byte_off, 0, kCohPolicy);
}
__device__ __forceinline__ uint32_t coh_load4(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b32(rs, (int)byte_off, 0, kCohPolicy);
}
// Polling reads: the same device-scope loads behind a compiler memory
// barrier, so a load repeated in a spin loop is issued every iteration
// (without the barrier the compiler treats the buffer load as a pure read
// and hoists it out of the loop as an invariant).
__device__ __forceinline__ u32x4 coh_poll16(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off) {
  asm volatile("" ::: "memory");
  return __builtin_amdgcn_raw_buffer_load_b128(rs, (int)byte_off, 0, kCohPolicy);
}
__device__ __forceinline__ uint32_t coh_poll4(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off) {
  asm volatile("" ::: "memory");
  return __builtin_amdgcn_raw_buffer_load_b32(rs, (int)byte_off, 0, kCohPolicy);
}
__device__ __forceinline__ void coh_store16(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, rs, (int)byte_off, 0, kCohPolicy);
}
__device__ __forceinline__ void coh_store4(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, rs, (int)byte_off, 0, kCohPolicy);
}
__device__ __forceinline__ void coh_store2(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off, uint16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, rs, (int)byte_off, 0, kCohPolicy);
}

// Store one element of type T (float or bf16) to a coherent buffer.
template <typename T>
__device__ __forceinline__ void coh_store_elem(__amdgpu_buffer_rsrc_t rs, uint32_t elem, float v);
template <>
__device__ __forceinline__ void coh_store_elem<float>(__amdgpu_buffer_rsrc_t rs, uint32_t elem, float v) {
  coh_store4(rs, elem * 4u, __builtin_bit_cast(uint32_t, v));
}
template <>
__device__ __forceinline__ void coh_store_elem<bf16>(__amdgpu_buffer_rsrc_t rs, uint32_t elem, float v) {
  coh_store2(rs, elem * 2u, __builtin_bit_cast(uint16_t, (bf16)v));
}

// Fill LDS from global memory for i = 0 .. n-1: value(i) loads element i
// (or gives a constant), put(i, v) stores it. Each thread issues eight loads
// before any of their stores waits; a plain loop waits for every load in
// turn (the forward scan's W_hr slice, 32 such iterations per thread, took
// 20 us to load that way).
template <int kT, typename LoadFn, typename PutFn>
__device__ __forceinline__ void lds_fill(int n, LoadFn value, PutFn put) {
  for (int base = 0; base < n; base += 8 * kT) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + u * kT + (int)threadIdx.x;
      v[u] = i < n ? value(i) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + u * kT + (int)threadIdx.x;
      if (i < n) put(i, v[u]);
    }
  }
}

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

// Wait until every memory operation this wave issued has completed.
__device__ __forceinline__ void wait_all_mem() {
  __builtin_amdgcn_s_waitcnt(0);
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// Group barrier. A group is the set of workgroups that exchange state with
// each other (all of them serve the same batch rows and direction). Each
// member adds 1 to the group's counter once per barrier; barrier number n
// (1-based) completes when the counter reaches n * members. Counters are
// zeroed before the launch. Only thread 0 touches the counter; the
// workgroup's coherent stores are complete before it arrives.
//
// Watchdog: a waiter that sees no progress for ~2 s of the device's 100 MHz
// real-time clock, or that sees another member's error, writes
// kStatusTimeout to the status word and makes the whole workgroup return.
// Every member then leaves within the same bound, so a launch whose
// workgroups are not all resident ends instead of hanging.
// ---------------------------------------------------------------------------
constexpr uint64_t kWatchdogTicks = 200000000ull;  // 2 s at 100 MHz

// Arrive at the group barrier: wait for this wave's memory operations
// (in particular the coherent stores of the exchanged state), join the
// workgroup, then thread 0 adds 1 to the counter. Work that does not feed
// the exchange (output stores, prefetches) can be issued between
// group_arrive and group_wait so that it overlaps the wait.
__device__ __forceinline__ void group_arrive(unsigned* counter) {
  wait_all_mem();
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until the counter reaches `target` (barrier n of a group of m
// members completes at n * m). Returns false if the watchdog fired.
__device__ __forceinline__ bool group_wait(unsigned* counter, unsigned target, int* status, int* abort_flag_lds) {
  if (threadIdx.x == 0) {
    uint64_t t0 = 0;
    unsigned polls = 0;
    while (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      if ((++polls & 63u) == 0) {
        const uint64_t now = __builtin_amdgcn_s_memrealtime();
        if (t0 == 0) t0 = now;
        const int st = __hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (st != kStatusOk || now - t0 > kWatchdogTicks) {
          __hip_atomic_store(status, kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          *abort_flag_lds = 1;
          break;
        }
      }
    }
  }
  __syncthreads();
  return *abort_flag_lds == 0;
}

__device__ __forceinline__ bool group_barrier(unsigned* counter, unsigned target, int* status,
                                              int* abort_flag_lds) {
  group_arrive(counter);
  return group_wait(counter, target, status, abort_flag_lds);
}

// ---------------------------------------------------------------------------
// Activations in fp32 from the hardware exp2 / log2. Near zero, where
// exp(x) - 1 and log(1 + y) cancel, short Taylor polynomials keep the
// relative error at the fp32 rounding level.
// ---------------------------------------------------------------------------
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fexp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

// Clamp to [lo, hi] by comparisons, so NaN passes through (a min/max pair
// would replace it by a bound). Infinite bounds make it the identity.
__device__ __forceinline__ float clampf(float x, float lo, float hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Logistic function with the hardware reciprocal (about 1 ulp): exp2 of a
// large argument gives +inf and rcp(inf) = 0, so both tails are exact.
__device__ __forceinline__ float fsigmoid(float x) { return __builtin_amdgcn_rcpf(1.0f + fexp(-x)); }

// tanh(x) = sign(x) (1 - e) / (1 + e) with e = exp(-2|x|) in (0, 1]; near
// zero the absolute error stays at the fp32 rounding level of 1.
__device__ __forceinline__ float ftanh(float x) {
  const float e = fexp(-2.0f * __builtin_fabsf(x));
  const float r = (1.0f - e) * __builtin_amdgcn_rcpf(1.0f + e);
  return __builtin_copysignf(r, x);
}

__device__ __forceinline__ float fexpm1(float x) {
  if (__builtin_fabsf(x) < 0.0625f) {
    return x * (1.0f + x * (0.5f + x * (0.166666666667f + x * (0.041666666667f + x * 0.008333333333f))));
  }
  return fexp(x) - 1.0f;
}

// ELU with alpha = 1 without branches: both branches of expm1 are formed and
// selected (the exp branch overflows harmlessly for large positive x, which
// takes x itself), so a wave never runs them one after the other.
__device__ __forceinline__ float felu(float x) {
  const float p = x * (1.0f + x * (0.5f + x * (0.166666666667f + x * (0.041666666667f + x * 0.008333333333f))));
  const float q = fexp(x) - 1.0f;
  const float m = __builtin_fabsf(x) < 0.0625f ? p : q;
  return x > 0.0f ? x : m;
}

__device__ __forceinline__ float flog1p_small(float y) {  // 0 <= y <= 1
  if (y < 0.0625f) {
    return y * (1.0f + y * (-0.5f + y * (0.333333333333f + y * (-0.25f + y * (0.2f + y * (-0.166666666667f + y * 0.142857142857f))))));
  }
  return __builtin_amdgcn_logf(1.0f + y) * kLn2;
}

// softplus(x) = log(1 + exp(x)) = max(x, 0) + log1p(exp(-|x|)).
__device__ __forceinline__ float fsoftplus(float x) {
  return __builtin_fmaxf(x, 0.0f) + flog1p_small(fexp(-__builtin_fabsf(x)));
}

// ---------------------------------------------------------------------------
// Small-batch product on the vector ALUs, operands in LDS:
//   out[r * ldo + c] = sum_k X[r * ldx + k] * W[c * ldw + k],  r < rows, c < cols
// over `kchunks` 16-byte chunks of K (rows 16-byte aligned, zero-padded past
// the true K). Each lane keeps MAXR rows x CPT columns of partial sums in
// registers while it walks a strided share of the chunks, so every 16-byte
// W read feeds MAXR * CPT * (elements per chunk) FMAs and many LDS reads are
// in flight; a power-of-two team of lanes then reduces by shuffles. The
// reduction order is fixed, so results are deterministic.
// ---------------------------------------------------------------------------
template <typename DT>
__device__ __forceinline__ void chunk_to_f32(const DT* p, float* f);
template <>
__device__ __forceinline__ void chunk_to_f32<float>(const float* p, float* f) {
  const f32x4 v = *reinterpret_cast<const f32x4*>(p);
  f[0] = v[0]; f[1] = v[1]; f[2] = v[2]; f[3] = v[3];
}
template <>
__device__ __forceinline__ void chunk_to_f32<bf16>(const bf16* p, float* f) {
  const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (float)v[i];
}

template <typename DT, int MAXR, int CPT>
__device__ void lds_gemv_rows(const DT* X, int ldx, const DT* W, int ldw, float* out, int ldo, int rows,
                              int cols, int kchunks) {
  constexpr int kEpc = 16 / sizeof(DT);
  const int ngrp = (cols + CPT - 1) / CPT;
  int team = 1;
  while (team < 16 && team * 2 * ngrp <= (int)blockDim.x && team * 2 <= kchunks) team *= 2;
  const int teams = blockDim.x / team;
  const int ti = threadIdx.x / team, li = threadIdx.x - ti * team;
  for (int r0 = 0; r0 < rows; r0 += MAXR) {
    const int nr = rows - r0 < MAXR ? rows - r0 : MAXR;
    for (int g = ti; g < ngrp; g += teams) {
      float acc[MAXR][CPT];
#pragma unroll
      for (int r = 0; r < MAXR; ++r)
#pragma unroll
        for (int j = 0; j < CPT; ++j) acc[r][j] = 0.f;
      const int c0 = g * CPT;
      for (int kc = li; kc < kchunks; kc += team) {
        float wv[CPT][kEpc];
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
          if (c0 + j < cols) {
            chunk_to_f32<DT>(W + (c0 + j) * ldw + kc * kEpc, wv[j]);
          } else {
#pragma unroll
            for (int e = 0; e < kEpc; ++e) wv[j][e] = 0.f;
          }
        }
#pragma unroll
        for (int r = 0; r < MAXR; ++r) {
          if (r < nr) {
            float xv[kEpc];
            chunk_to_f32<DT>(X + (r0 + r) * ldx + kc * kEpc, xv);
#pragma unroll
            for (int j = 0; j < CPT; ++j)
#pragma unroll
              for (int e = 0; e < kEpc; ++e) acc[r][j] = __builtin_fmaf(xv[e], wv[j][e], acc[r][j]);
          }
        }
      }
      for (int off = team >> 1; off > 0; off >>= 1) {
#pragma unroll
        for (int r = 0; r < MAXR; ++r)
#pragma unroll
          for (int j = 0; j < CPT; ++j) acc[r][j] += __shfl_xor(acc[r][j], off, 64);
      }
      if (li == 0) {
#pragma unroll
        for (int r = 0; r < MAXR; ++r)
          if (r < nr)
#pragma unroll
            for (int j = 0; j < CPT; ++j)
              if (c0 + j < cols) out[(r0 + r) * ldo + c0 + j] = acc[r][j];
      }
    }
  }
}

template <typename T>
__device__ __forceinline__ float to_f32(T v);
template <>
__device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ float to_f32<bf16>(bf16 v) { return (float)v; }

template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

}  // namespace rnnk
