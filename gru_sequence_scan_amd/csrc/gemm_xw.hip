// Kernel 1: the input-hidden dense op hoisted out of the time loop.
//
//   Gx[m, n] = sum_k X[m, k] * W_dir(n)[n mod G, k] + bias(n)
//
// for every token row m at once (apache/tvm PR "[TOPI] TE implementation of
// LSTM using scan", description: the initial input-hidden dense is one of the
// three dense ops of an LSTM). Both directions of a bidirectional layer share
// one launch (N = D * G). bias(n) folds b_ih and, except for the GRU n gate
// whose b_hn sits inside the reset product, b_hh.
//
// gfx950 design: 128x128 output tile per 256-thread workgroup, 4 waves in a
// 2x2 arrangement, each wave a 64x64 block of 32x32 MFMA tiles
// (v_mfma_f32_32x32x16_bf16 for bf16 operands, v_mfma_f32_32x32x2_f32 for
// fp32). K advances 64 bytes per stage. The main form streams stages
// straight from global memory into a three-deep LDS ring (below); a simpler
// register-staged double buffer handles ragged K and unaligned rows.
// Every lane reads whole 16-byte chunks from LDS: the k index a lane supplies
// to each MFMA step is permuted identically for both operands, which leaves
// each dot product unchanged. Output tiles are dealt to XCDs in contiguous
// runs so that tiles sharing X rows share an L2.
#include <algorithm>

#include "device_common.hpp"
#include "kernels.hpp"

namespace rnnk {

namespace {

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kRowBytes = 64;        // one K stage of one row
constexpr int kLdsRow = 80;          // padded LDS row stride (bytes)
constexpr int kTileBytes = kBM * kLdsRow;

template <typename DT>
struct Mfma;

template <>
struct Mfma<bf16> {
  static constexpr int kSteps = 2;  // 16 k per step, 32 k per stage
  __device__ static void run(const char* a_row, const char* b_row, int half, f32x16& acc) {
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const bf16x8 av = *reinterpret_cast<const bf16x8*>(a_row + (2 * s + half) * 16);
      const bf16x8 bv = *reinterpret_cast<const bf16x8*>(b_row + (2 * s + half) * 16);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
    }
  }
};

template <>
struct Mfma<float> {
  static constexpr int kSteps = 8;  // 2 k per step, 16 k per stage
  __device__ static void run(const char* a_row, const char* b_row, int half, f32x16& acc) {
    const f32x4 a0 = *reinterpret_cast<const f32x4*>(a_row + (2 * half) * 16);
    const f32x4 a1 = *reinterpret_cast<const f32x4*>(a_row + (2 * half + 1) * 16);
    const f32x4 b0 = *reinterpret_cast<const f32x4*>(b_row + (2 * half) * 16);
    const f32x4 b1 = *reinterpret_cast<const f32x4*>(b_row + (2 * half + 1) * 16);
    const float av[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    const float bv[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
    for (int s = 0; s < kSteps; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[s], bv[s], acc, 0, 0, 0);
  }
};

// Load the 16-byte chunk `cc` (of four) of row `row` for the K stage at k0.
template <typename DT>
__device__ __forceinline__ u32x4 load_chunk(const DT* base, int rows, int K, int row, int k0, int cc,
                                            bool vec_ok) {
  constexpr int kEpc = 16 / sizeof(DT);
  const int k = k0 + cc * kEpc;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (row >= rows) return v;
  const DT* p = base + (size_t)row * K + k;
  if (vec_ok && k + kEpc <= K) return *reinterpret_cast<const u32x4*>(p);
  DT tmp[kEpc];
#pragma unroll
  for (int e = 0; e < kEpc; ++e) tmp[e] = (k + e < K) ? p[e] : (DT)0.0f;
  __builtin_memcpy(&v, tmp, 16);
  return v;
}

// Epilogue: bias fold and fp32 store of the 128x128 tile. The accumulators
// pass through LDS 64 rows at a time (one pass per wave row), so that each
// lane then stores whole 16-byte chunks of a C row: a wave writes two full
// 512-byte row segments per instruction instead of 2 x 128 bytes of single
// dwords. The stores are non-temporal: G_x is read back only by the
// recurrence, after the whole product. 32x32 accumulator layout: lane holds
// column l32 and rows 8 (v / 4) + 4 half + v % 4. The LDS row stride of 136
// floats puts the two lane halves (rows 4 apart) on disjoint banks.
// b_ih(n) plus, except for the GRU candidate rows, b_hh(n) (zero without biases).
template <typename DT>
__device__ __forceinline__ float fold_bias(const GemmArgs& a, int n) {
  if (!a.has_bias) return 0.0f;
  const int dir = n / a.G, nr = n - dir * a.G;
  float b = to_f32<DT>(reinterpret_cast<const DT*>(a.b_ih[dir])[nr]);
  if (nr < a.hh_fold_rows) b += to_f32<DT>(reinterpret_cast<const DT*>(a.b_hh[dir])[nr]);
  return b;
}

// K stages [kt0, kt1) of this workgroup's split (blockIdx.y), and where its
// tile goes: the output with the bias fold, or its partial buffer.
struct KRange {
  int kt0, kt1;
  void* C;
  bool with_bias;
};
__device__ __forceinline__ KRange k_range(const GemmArgs& a, int nk) {
  if (a.splits <= 1) return KRange{0, nk, a.C, true};
  const int s = blockIdx.y, per = (nk + a.splits - 1) / a.splits;
  const int kt0 = min(nk, s * per), kt1 = min(nk, kt0 + per);
  return KRange{kt0, kt1, a.part + (size_t)s * a.M * a.N, false};
}

constexpr int kEpiStride = 136;
constexpr int kEpiBytes = 64 * kEpiStride * 4;  // 34816
static_assert(kEpiBytes <= 2 * 2 * kTileBytes, "epilogue staging exceeds the operand buffers");

// Four outputs as bf16 (round to nearest even), one 8-byte store.
__device__ __forceinline__ void store4_bf16(bf16* dst, const f32x4& v, bool vec, int valid) {
  if (vec) {
    uint32_t w[2];
#pragma unroll
    for (int e = 0; e < 2; ++e)
      w[e] = (uint32_t)__builtin_bit_cast(uint16_t, (bf16)v[2 * e]) |
             (uint32_t)__builtin_bit_cast(uint16_t, (bf16)v[2 * e + 1]) << 16;
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    __builtin_nontemporal_store(u32x2{w[0], w[1]}, reinterpret_cast<u32x2*>(dst));
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (e < valid) dst[e] = (bf16)v[e];
  }
}

template <typename DT>
__device__ __forceinline__ void store_tile(const GemmArgs& a, f32x16 (&acc)[2][2], float* lds, int m0, int n0,
                                           void* Cv, bool with_bias) {
  const bool out_bf16 = with_bias && a.c_bf16;  // partial tiles stay fp32
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, half = lane >> 5, l32 = lane & 31;
  const int c4 = tid & 31, rbase = tid >> 5;  // this thread's 16-byte column chunk and first row
  const int n = n0 + 4 * c4;
  float bias[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (with_bias) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (n + e < a.N) bias[e] = fold_bias<DT>(a, n + e);
    }
  }
  const bool vec = (a.N & 3) == 0 && (reinterpret_cast<uintptr_t>(Cv) & 15) == 0 && n + 4 <= a.N;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    if (p) __syncthreads();  // the first pass's reads are done
    if (wm == p) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            lds[(i * 32 + 8 * (v >> 2) + 4 * half + (v & 3)) * kEpiStride + wn * 64 + j * 32 + l32] = acc[i][j][v];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = rbase + 8 * i;
      const int m = m0 + p * 64 + r;
      if (m >= a.M) break;
      f32x4 v = *reinterpret_cast<const f32x4*>(lds + r * kEpiStride + 4 * c4);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += bias[e];
      if (out_bf16) {
        store4_bf16(reinterpret_cast<bf16*>(Cv) + (size_t)m * a.N + n, v, vec, a.N - n);
        continue;
      }
      float* dst = reinterpret_cast<float*>(Cv) + (size_t)m * a.N + n;
      if (vec) {
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dst));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < a.N) dst[e] = v[e];
      }
    }
  }
}

template <typename DT>
__global__ void __launch_bounds__(256) gemm_xw_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[2][2][kTileBytes];
  constexpr int kBK = kRowBytes / sizeof(DT);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ntn = (a.N + kBN - 1) / kBN;
  const int ntm = (a.M + kBM - 1) / kBM;
  const int ntiles = ntn * ntm;

  // XCD-aware order: workgroup ids are dealt round-robin over the 8 XCDs;
  // give each XCD a contiguous run of tiles (row-major, N fastest).
  int bid = blockIdx.x;
  const int per_xcd = ntiles / 8;
  if (bid < per_xcd * 8) bid = (bid & 7) * per_xcd + (bid >> 3);
  const int tile_m = bid / ntn, tile_n = bid - tile_m * ntn;
  const int m0 = tile_m * kBM, n0 = tile_n * kBN;

  const DT* A = reinterpret_cast<const DT*>(a.A);
  // Rows of this thread's two chunks (A and B use the same mapping).
  const int c0 = tid, c1 = tid + 256;
  const int r0 = c0 >> 2, cc0 = c0 & 3, r1 = c1 >> 2, cc1 = c1 & 3;
  // B rows: output column n -> direction and weight row.
  auto wrow = [&](int r, const DT*& base) -> int {
    const int n = n0 + r;
    if (n >= a.N) { base = nullptr; return 0; }
    const int dir = n / a.G;
    base = reinterpret_cast<const DT*>(a.W[dir]);
    return n - dir * a.G;
  };
  const DT* wb0; const DT* wb1;
  const int wr0 = wrow(r0, wb0), wr1 = wrow(r1, wb1);

  const int nk = (a.K + kBK - 1) / kBK;
  u32x4 ra0, ra1, rb0, rb1;
  auto gload = [&](int k0) {
    ra0 = load_chunk<DT>(A, a.M, a.K, m0 + r0, k0, cc0, a.vec_ok);
    ra1 = load_chunk<DT>(A, a.M, a.K, m0 + r1, k0, cc1, a.vec_ok);
    rb0 = wb0 ? load_chunk<DT>(wb0, a.G, a.K, wr0, k0, cc0, a.vec_ok) : u32x4{0u, 0u, 0u, 0u};
    rb1 = wb1 ? load_chunk<DT>(wb1, a.G, a.K, wr1, k0, cc1, a.vec_ok) : u32x4{0u, 0u, 0u, 0u};
  };
  auto lstore = [&](int buf) {
    *reinterpret_cast<u32x4*>(&smem[buf][0][r0 * kLdsRow + cc0 * 16]) = ra0;
    *reinterpret_cast<u32x4*>(&smem[buf][0][r1 * kLdsRow + cc1 * 16]) = ra1;
    *reinterpret_cast<u32x4*>(&smem[buf][1][r0 * kLdsRow + cc0 * 16]) = rb0;
    *reinterpret_cast<u32x4*>(&smem[buf][1][r1 * kLdsRow + cc1 * 16]) = rb1;
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int wm = wave >> 1, wn = wave & 1;
  const int half = lane >> 5, l32 = lane & 31;

  const KRange kr = k_range(a, nk);
  gload(kr.kt0 * kBK);
  lstore(0);
  __syncthreads();
  for (int kt = kr.kt0; kt < kr.kt1; ++kt) {
    const int buf = (kt - kr.kt0) & 1;
    if (kt + 1 < kr.kt1) gload((kt + 1) * kBK);
    const char* As = smem[buf][0];
    const char* Bs = smem[buf][1];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const char* arow = As + (wm * 64 + i * 32 + l32) * kLdsRow;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const char* brow = Bs + (wn * 64 + j * 32 + l32) * kLdsRow;
        Mfma<DT>::run(arow, brow, half, acc[i][j]);
      }
    }
    if (kt + 1 < kr.kt1) lstore(buf ^ 1);
    __syncthreads();
  }

  store_tile<DT>(a, acc, reinterpret_cast<float*>(&smem[0][0][0]), m0, n0, kr.C, kr.with_bias);
}

// ---------------------------------------------------------------------------
// Pipelined form: operands go from global memory straight into LDS
// (global_load_lds_dwordx4: lane l of a wave writes LDS bytes 16 l .. 16 l + 15
// of the wave's 1 KiB block), kStages K stages deep, so several stages'
// loads are in flight while the MFMAs consume the oldest one. A stage is 64
// bytes of every row of the A and B tiles. Rows are stored unpadded with the
// 16-byte chunk c of row r at position c ^ ((r >> 2) & 3): the lanes of one
// MFMA operand read (16 consecutive rows, one chunk) then hit 16 distinct
// bank groups. Needs K to be a whole number of stages and 16-byte aligned
// rows; rows past M or N read a zero chunk.
// ---------------------------------------------------------------------------
constexpr int kStages = 3;  // 48 KiB: three workgroups per CU (measured 6% faster than four stages at two)
constexpr int kStageBytes = (kBM + kBN) * kRowBytes;  // 16 KiB
static_assert(kEpiBytes <= kStages * kStageBytes, "epilogue staging exceeds the LDS ring");

__device__ __forceinline__ int swz(int row, int c) { return c ^ ((row >> 2) & 3); }

template <typename DT>
struct MfmaSwz;

template <>
struct MfmaSwz<bf16> {
  // 32 k per stage: two 32x32x16 steps; lane half h supplies chunks 2s + h
  __device__ static void run(const char* A, int ar, const char* B, int br, int half, f32x16& acc) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bf16x8 av = *reinterpret_cast<const bf16x8*>(A + ar * kRowBytes + swz(ar, 2 * s + half) * 16);
      const bf16x8 bv = *reinterpret_cast<const bf16x8*>(B + br * kRowBytes + swz(br, 2 * s + half) * 16);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
    }
  }
};

template <>
struct MfmaSwz<float> {
  // 16 k per stage: eight 32x32x2 steps; lane half h supplies chunks 2h, 2h + 1
  __device__ static void run(const char* A, int ar, const char* B, int br, int half, f32x16& acc) {
    const f32x4 a0 = *reinterpret_cast<const f32x4*>(A + ar * kRowBytes + swz(ar, 2 * half) * 16);
    const f32x4 a1 = *reinterpret_cast<const f32x4*>(A + ar * kRowBytes + swz(ar, 2 * half + 1) * 16);
    const f32x4 b0 = *reinterpret_cast<const f32x4*>(B + br * kRowBytes + swz(br, 2 * half) * 16);
    const f32x4 b1 = *reinterpret_cast<const f32x4*>(B + br * kRowBytes + swz(br, 2 * half + 1) * 16);
    const float av[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    const float bv[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
    for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[s], bv[s], acc, 0, 0, 0);
  }
};

// Wait until at most n (0, 4 or 8) of this wave's vector memory operations
// are pending. s_waitcnt fields: vmcnt bits 3:0 (and 15:14), expcnt 6:4,
// lgkmcnt 11:8; the latter two are left at their maxima (no constraint).
__device__ __forceinline__ void wait_vm(int n) {
  if (n >= 8)
    __builtin_amdgcn_s_waitcnt(0x0F78);
  else if (n >= 4)
    __builtin_amdgcn_s_waitcnt(0x0F74);
  else
    __builtin_amdgcn_s_waitcnt(0x0F70);
}

template <typename DT>
__global__ void __launch_bounds__(256) gemm_xw_pipe_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[kStages][kStageBytes];
  constexpr int kEpc = 16 / sizeof(DT);
  constexpr int kBK = kRowBytes / sizeof(DT);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ntn = (a.N + kBN - 1) / kBN;
  const int ntm = (a.M + kBM - 1) / kBM;
  const int ntiles = ntn * ntm;
  int bid = blockIdx.x;
  const int per_xcd = ntiles / 8;
  if (bid < per_xcd * 8) bid = (bid & 7) * per_xcd + (bid >> 3);
  const int tile_m = bid / ntn, tile_n = bid - tile_m * ntn;
  const int m0 = tile_m * kBM, n0 = tile_n * kBN;

  // This thread's four 16-byte slots of a stage: wave w, block j covers LDS
  // rows 16 (4 w + j) .. + 15 of the stacked [A; B] tile; lane l writes row
  // 16 (4 w + j) + l / 4 at position l % 4, which holds chunk swz(row, l % 4).
  const char* src[4];
  int kofs[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 16 * (4 * wave + j) + (lane >> 2);
    const int c = swz(row & (kBM - 1), lane & 3);
    const DT* p = nullptr;
    if (row < kBM) {
      const int m = m0 + row;
      if (m < a.M) p = reinterpret_cast<const DT*>(a.A) + (size_t)m * a.K;
    } else {
      const int n = n0 + row - kBM;
      if (n < a.N) {
        const int dir = n / a.G;
        p = reinterpret_cast<const DT*>(a.W[dir]) + (size_t)(n - dir * a.G) * a.K;
      }
    }
    src[j] = p ? reinterpret_cast<const char*>(p) : reinterpret_cast<const char*>(a.zero16);
    kofs[j] = p ? c * kEpc * (int)sizeof(DT) : 0;  // byte offset of the chunk within a stage
  }
  const int nk = a.K / kBK;
  const KRange kr = k_range(a, nk);
  auto issue = [&](int kt) {
    char* dst = smem[(kt - kr.kt0) % kStages];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const char* g = src[j] == a.zero16 ? src[j] : src[j] + (size_t)kt * kRowBytes + kofs[j];
      __builtin_amdgcn_global_load_lds(g, dst + (4 * wave + j) * 1024, 16, 0, 0);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int wm = wave >> 1, wn = wave & 1;
  const int half = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s)
    if (kr.kt0 + s < kr.kt1) issue(kr.kt0 + s);
  for (int kt = kr.kt0; kt < kr.kt1; ++kt) {
    // Stage kt landed once at most the later stages' loads are pending. A
    // bare barrier then makes every wave's part of it visible (and every
    // wave is done reading the buffer that the next issue refills, since its
    // MFMAs consumed those reads); __syncthreads would also drain the
    // younger stages' loads.
    wait_vm(4 * min(kStages - 2, kr.kt1 - 1 - kt));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kt + kStages - 1 < kr.kt1) issue(kt + kStages - 1);
    const char* As = smem[(kt - kr.kt0) % kStages];
    const char* Bs = As + kBM * kRowBytes;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        MfmaSwz<DT>::run(As, wm * 64 + i * 32 + l32, Bs, wn * 64 + j * 32 + l32, half, acc[i][j]);
  }

  // Every wave is done reading the ring before the epilogue reuses it.
  __syncthreads();
  store_tile<DT>(a, acc, reinterpret_cast<float*>(&smem[0][0]), m0, n0, kr.C, kr.with_bias);
}

// C = sum over the splits, in split order, of the partial products, plus the
// bias fold: four consecutive outputs per thread (N % 4 == 0) or one. Plain
// stores: a split product is small, and the recurrence reads it next.
template <typename DT>
__global__ void __launch_bounds__(256) gemm_xw_reduce_kernel(GemmArgs a) {
  const size_t total = (size_t)a.M * a.N;
  const size_t plane = total;
  if ((a.N & 3) == 0 && (reinterpret_cast<uintptr_t>(a.C) & 15) == 0 &&
      (reinterpret_cast<uintptr_t>(a.part) & 15) == 0) {
    for (size_t i4 = (size_t)blockIdx.x * 256 + threadIdx.x; i4 * 4 < total; i4 += (size_t)gridDim.x * 256) {
      const size_t i = i4 * 4;
      f32x4 v = *reinterpret_cast<const f32x4*>(a.part + i);
      for (int s = 1; s < a.splits; ++s) v += *reinterpret_cast<const f32x4*>(a.part + s * plane + i);
      const int n = (int)(i % a.N);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += fold_bias<DT>(a, n + e);
      if (a.c_bf16)
        store4_bf16(reinterpret_cast<bf16*>(a.C) + i, v, true, 4);
      else
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.C) + i) = v;
    }
  } else {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (size_t)gridDim.x * 256) {
      float v = a.part[i];
      for (int s = 1; s < a.splits; ++s) v += a.part[s * plane + i];
      v += fold_bias<DT>(a, (int)(i % a.N));
      if (a.c_bf16)
        reinterpret_cast<bf16*>(a.C)[i] = (bf16)v;
      else
        reinterpret_cast<float*>(a.C)[i] = v;
    }
  }
}

}  // namespace

// Products with fewer than 64 output tiles leave most of the 256 CUs idle
// (the TVM benchmark's T = 80, B = 1 LSTM has 8): split K so that the launch
// has about 128 workgroups, each keeping at least four K stages.
int gemm_xw_splits(long long M, int N, int K, int dtype_bf16) {
  const long long tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  if (tiles >= 64) return 1;
  const int nk = (K + kRowBytes / (dtype_bf16 ? 2 : 4) - 1) / (kRowBytes / (dtype_bf16 ? 2 : 4));
  int s = (int)std::min<long long>(8, std::max<long long>(1, 128 / tiles));
  s = std::min(s, std::max(1, nk / 4));
  return s;
}

hipError_t launch_gemm_xw(const GemmArgs& a, int dtype_bf16, hipStream_t stream) {
  const int ntn = (a.N + kBN - 1) / kBN;
  const int ntm = (a.M + kBM - 1) / kBM;
  const dim3 grid(ntn * ntm, a.splits > 1 ? a.splits : 1), block(256);
  // fp32 operands: the streamed form (measured 10% faster at K = 1024). bf16
  // operands: the register-staged form (up to four workgroups per CU),
  // measured 0-30% faster than the streamed one.
  const bool pipe = !dtype_bf16 && a.vec_ok && a.zero16 && a.K % (kRowBytes / 4) == 0;
  if (dtype_bf16) {
    if (pipe)
      launch_kernel(gemm_xw_pipe_kernel<bf16>, grid, block, 0, stream, a);
    else
      launch_kernel(gemm_xw_kernel<bf16>, grid, block, 0, stream, a);
  } else {
    if (pipe)
      launch_kernel(gemm_xw_pipe_kernel<float>, grid, block, 0, stream, a);
    else
      launch_kernel(gemm_xw_kernel<float>, grid, block, 0, stream, a);
  }
  if (a.splits > 1) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t work = ((size_t)a.M * a.N + 3) / 4;
    const int blocks = (int)std::min<size_t>(1024, (work + 255) / 256);
    if (dtype_bf16)
      launch_kernel(gemm_xw_reduce_kernel<bf16>, dim3(blocks), block, 0, stream, a);
    else
      launch_kernel(gemm_xw_reduce_kernel<float>, dim3(blocks), block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace rnnk
