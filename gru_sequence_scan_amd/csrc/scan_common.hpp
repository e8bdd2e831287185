// Pieces shared by the forward and backward persistent scans: LDS-resident
// products on MFMA or the vector ALUs, the coherent tile copy, and the
// weight-slice loader. Workgroups of these kernels have kScanThreads threads.
#pragma once

#include "device_common.hpp"
#include "kernels.hpp"

namespace rnnk {
namespace {

constexpr int kScanThreads = 256;


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
__device__ __forceinline__ void mm_mfma(const char* lds, int as_off, int as_ld, int w_off, int w_ld, float* acc,
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
// and rows for which row_of() returns -1. Rows of whole 16-byte chunks (the
// usual case) move as 16-byte loads, eight in flight per thread before any
// LDS store waits for them; otherwise element by element.
template <typename DT, typename RowFn>
__device__ __forceinline__ void load_weights(const DT* w, int klen, int kpad, int nrows, RowFn row_of, char* lds,
                             int off, int ld) {
  DT* dst = reinterpret_cast<DT*>(lds + off);
  constexpr int kEpc = 16 / sizeof(DT);
  if (klen % kEpc == 0 && ld % kEpc == 0 && (reinterpret_cast<uintptr_t>(w) & 15u) == 0) {
    const int cpr = kpad / kEpc, total = nrows * cpr;
    for (int base = 0; base < total; base += kScanThreads * 8) {
      u32x4 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int idx = base + i * kScanThreads + threadIdx.x;
        const int r = idx / cpr, cc = idx - r * cpr;
        const int gr = idx < total ? row_of(r) : -1;
        v[i] = gr >= 0 && cc * kEpc < klen
                   ? *reinterpret_cast<const u32x4*>(w + (size_t)gr * klen + cc * kEpc)
                   : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int idx = base + i * kScanThreads + threadIdx.x;
        if (idx < total) {
          const int r = idx / cpr, cc = idx - r * cpr;
          *reinterpret_cast<u32x4*>(dst + r * ld + cc * kEpc) = v[i];
        }
      }
    }
    return;
  }
  const int total = nrows * kpad;
  for (int idx = threadIdx.x; idx < total; idx += kScanThreads) {
    const int r = idx / kpad, k = idx - r * kpad;
    const int gr = row_of(r);
    dst[r * ld + k] = (gr >= 0 && k < klen) ? w[(size_t)gr * klen + k] : (DT)0.0f;
  }
}


// ---------------------------------------------------------------------------
// Ring exchange of the forward scan. Step k's exchanged state goes to slot
// k mod kRingSlots of a ring that holds the all-ones sentinel (0xFFFF per
// bf16 element, 0xFFFFFFFF per fp32 element) until the element's owner
// stores its value; readers poll their 16-byte chunks with device-scope
// loads until no sentinel is left in them (padding columns hold zeros). A NaN
// result is stored as the canonical quiet NaN, so no value equals the
// sentinel. The store is plain when every member of the group runs on one
// XCD (it lands in that XCD's L2, where the others' device-scope loads find
// it) and device-scope otherwise.
// ---------------------------------------------------------------------------
constexpr int kRingSlots = kScanRingSlots;

template <typename DT>
__device__ __forceinline__ void ring_store(__amdgpu_buffer_rsrc_t rs, uint32_t elem, float v, bool local);
template <>
__device__ __forceinline__ void ring_store<float>(__amdgpu_buffer_rsrc_t rs, uint32_t elem, float v, bool local) {
  const uint32_t bits = v == v ? __builtin_bit_cast(uint32_t, v) : 0x7FC00000u;
  if (local)
    __builtin_amdgcn_raw_buffer_store_b32(bits, rs, (int)(elem * 4u), 0, 0);
  else
    __builtin_amdgcn_raw_buffer_store_b32(bits, rs, (int)(elem * 4u), 0, kCohPolicy);
}
template <>
__device__ __forceinline__ void ring_store<bf16>(__amdgpu_buffer_rsrc_t rs, uint32_t elem, float v, bool local) {
  const uint16_t bits = v == v ? __builtin_bit_cast(uint16_t, (bf16)v) : (uint16_t)0x7FC0u;
  if (local)
    __builtin_amdgcn_raw_buffer_store_b16(bits, rs, (int)(elem * 2u), 0, 0);
  else
    __builtin_amdgcn_raw_buffer_store_b16(bits, rs, (int)(elem * 2u), 0, kCohPolicy);
}
// Plain store of one element at a byte offset; dropped when the offset lies
// past the end of the buffer.
template <typename DT>
__device__ __forceinline__ void out_store(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off, float v) {
  if constexpr (sizeof(DT) == 4)
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rs, (int)byte_off, 0, 0);
  else
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (bf16)v), rs, (int)byte_off, 0, 0);
}

// Put an element back to the sentinel.
template <typename DT>
__device__ __forceinline__ void ring_reset(__amdgpu_buffer_rsrc_t rs, uint32_t elem, bool local) {
  if (sizeof(DT) == 4) {
    if (local)
      __builtin_amdgcn_raw_buffer_store_b32(0xFFFFFFFFu, rs, (int)(elem * 4u), 0, 0);
    else
      __builtin_amdgcn_raw_buffer_store_b32(0xFFFFFFFFu, rs, (int)(elem * 4u), 0, kCohPolicy);
  } else {
    if (local)
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)0xFFFFu, rs, (int)(elem * 2u), 0, 0);
    else
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)0xFFFFu, rs, (int)(elem * 2u), 0, kCohPolicy);
  }
}

// True when any element of a 16-byte chunk holds the sentinel.
template <typename DT>
__device__ __forceinline__ bool chunk_pending(const u32x4& v) {
  if (sizeof(DT) == 4) return v[0] == 0xFFFFFFFFu || v[1] == 0xFFFFFFFFu || v[2] == 0xFFFFFFFFu || v[3] == 0xFFFFFFFFu;
  bool s = false;
#pragma unroll
  for (int e = 0; e < 4; ++e) s = s || (v[e] & 0xFFFFu) == 0xFFFFu || v[e] >= 0xFFFF0000u;
  return s;
}

// True when any element of eight chunks holds the sentinel: the sentinel is
// the largest value of the element's unsigned integer type, so one running
// maximum (packed per 16-bit half for bf16) answers for all of them.
template <typename DT>
__device__ __forceinline__ bool batch_pending(const u32x4 (&v)[8]) {
  if (sizeof(DT) == 4) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = max(m, max(max(v[i][0], v[i][1]), max(v[i][2], v[i][3])));
    return m == 0xFFFFFFFFu;
  }
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  u16x2 m = {0, 0};
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // through a scalar: hipcc's __builtin_bit_cast of an ext-vector element
      // expression reads element 0 whatever the index
      const uint32_t x = v[i][e];
      m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, x));
    }
  return m[0] == 0xFFFFu || m[1] == 0xFFFFu;
}

// Polling a tile of `rows` rows (at most 64) of width `width` elements (a
// multiple of a chunk) into LDS (row stride dst_ld elements). Row r comes
// from the ring at element ring_el + r * ring_ld when bit r of `ring` is
// set (polled until complete), from the first h0_valid elements of
// h0 + r * h0_ld when bit r of `init` is set (a row's first step; the rest
// of the row is zero), and is zero otherwise. The ring's padding columns
// hold zeros, so whole chunks are checked and copied.
//
// Thread t handles chunks t, t + 256, ... of the tile (row-major), eight at
// a time (a batch): poll_issue loads a batch, poll_finish loads its pending
// chunks again until their values arrive and writes the batch to LDS. A
// chunk's (row, column) comes from a cursor advanced by 256 chunks with
// adds and one compare, and the cursor enters each call through an opaque
// copy: the per-chunk index math is redone every step instead of being
// hoisted out of the step loop into registers.
//
// When the watchdog fires (no progress for ~2 s, or another member's error
// in *status) the status word gets kStatusTimeout, *abort_lds is set and
// poll_finish returns false; the caller checks the flag after its next
// workgroup barrier.
struct PollGeom {
  int cpr;       // chunks per row
  int q, rem;    // 256 chunks = q rows + rem chunks
  int total;     // chunks in the tile
};

__device__ __forceinline__ PollGeom poll_geom(int rows, int width, int epc) {
  PollGeom g;
  g.cpr = width / epc;
  g.q = kScanThreads / g.cpr;
  g.rem = kScanThreads - g.q * g.cpr;
  g.total = rows * g.cpr;
  return g;
}

// Cursor (row, chunk column) of chunk threadIdx.x, packed as row << 16 | col.
__device__ __forceinline__ uint32_t poll_cursor0(const PollGeom& g) {
  const int t = threadIdx.x;
  return (uint32_t)(t / g.cpr) << 16 | (uint32_t)(t % g.cpr);
}

__device__ __forceinline__ void cursor_step(int& r, int& cc, const PollGeom& g) {
  cc += g.rem;
  r += g.q;
  if (cc >= g.cpr) {
    cc -= g.cpr;
    ++r;
  }
}

struct PollBatch {
  u32x4 v[8];
  unsigned pend;
  uint32_t cur;  // cursor of the batch's first chunk
};

// A byte offset past the end of every ring (each under 2 GiB).
constexpr uint32_t kPollOob = 0x7FFFFFF0u;

template <typename DT>
__device__ __forceinline__ void poll_issue(PollBatch& pb, uint32_t cur, int base, const PollGeom& g,
                                           __amdgpu_buffer_rsrc_t rs, uint32_t ring_el, int ring_ld, uint64_t ring) {
  constexpr int kEpc = 16 / sizeof(DT);
  asm volatile("" : "+v"(cur));
  pb.cur = cur;
  pb.pend = 0;
  int r = (int)(cur >> 16), cc = (int)(cur & 0xFFFFu);
  // Eight loads, unconditionally: a chunk that is not polled reads past the
  // end of the buffer (zero). Straight-line code lets the compiler wait for
  // exactly these loads, not for what the caller issues after them.
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bool in = base + i * kScanThreads + (int)threadIdx.x < g.total;
    const bool from_ring = in && ((ring >> r) & 1ull);
    const uint32_t off = (ring_el + (uint32_t)(r * ring_ld + cc * kEpc)) * (uint32_t)sizeof(DT);
    pb.v[i] = coh_poll16(rs, from_ring ? off : kPollOob);
    cursor_step(r, cc, g);
  }
}

template <typename DT>
__device__ __forceinline__ bool poll_finish(PollBatch& pb, int base, const PollGeom& g, __amdgpu_buffer_rsrc_t rs,
                                            uint32_t ring_el, int ring_ld, uint64_t init, const DT* h0, int h0_ld,
                                            int h0_valid, char* lds, int dst_off, int dst_ld, int* status,
                                            int* abort_lds) {
  constexpr int kEpc = 16 / sizeof(DT);
  DT* dst = reinterpret_cast<DT*>(lds + dst_off);
  bool ok = true;
  uint64_t t0 = 0;
  unsigned polls = 0;
  // First check, branch-free (chunks not polled read zero: never pending);
  // chunk by chunk only when some sentinel is left.
  pb.pend = 0;
  if (batch_pending<DT>(pb.v)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) pb.pend |= chunk_pending<DT>(pb.v[i]) ? 1u << i : 0u;
  }
  while (pb.pend) {
    if ((++polls & 63u) == 0) {
      const uint64_t now = __builtin_amdgcn_s_memrealtime();
      if (t0 == 0) t0 = now;
      const int st = __hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (st != kStatusOk || now - t0 > kWatchdogTicks) {
        __hip_atomic_store(status, kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *abort_lds = 1;
        ok = false;
        break;
      }
    }
    {
      int r = (int)(pb.cur >> 16), cc = (int)(pb.cur & 0xFFFFu);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if ((pb.pend >> i) & 1u)
          pb.v[i] = coh_poll16(rs, (ring_el + (uint32_t)(r * ring_ld + cc * kEpc)) * (uint32_t)sizeof(DT));
        cursor_step(r, cc, g);
      }
    }
    // Check every chunk, branch-free: a completed chunk stays complete, and
    // no load result is left unread on any path (a register with a load in
    // flight on some path makes the compiler wait for all memory operations
    // before the register is next written).
    pb.pend = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) pb.pend |= chunk_pending<DT>(pb.v[i]) ? 1u << i : 0u;
  }
  {
    int r = (int)(pb.cur >> 16), cc = (int)(pb.cur & 0xFFFFu);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (base + i * kScanThreads + (int)threadIdx.x < g.total)
        *reinterpret_cast<u32x4*>(dst + r * dst_ld + cc * kEpc) = pb.v[i];
      cursor_step(r, cc, g);
    }
  }
  // Rows at their first step take h0 (rare: kept out of the unrolled code).
  // The same thread wrote the chunk's zeros just above.
  if (init && h0) {
    int r = (int)(pb.cur >> 16), cc = (int)(pb.cur & 0xFFFFu);
#pragma nounroll
    for (int i = 0; i < 8; ++i) {
      if (base + i * kScanThreads + (int)threadIdx.x < g.total && ((init >> r) & 1ull)) {
#pragma nounroll
        for (int e = 0; e < kEpc && cc * kEpc + e < h0_valid; ++e)
          dst[r * dst_ld + cc * kEpc + e] = h0[(size_t)r * h0_ld + cc * kEpc + e];
      }
      cursor_step(r, cc, g);
    }
  }
  return ok;
}

// The whole tile. cur0 = poll_cursor0(g). between() runs after the first
// batch's loads are issued and before they are waited for (work whose
// memory operations should not delay the poll: the vector-memory counter
// retires in issue order).
template <typename DT, typename BetweenFn>
__device__ __forceinline__ void poll_tile(const PollGeom& g, uint32_t cur0, __amdgpu_buffer_rsrc_t rs,
                                          uint32_t ring_el, int ring_ld, uint64_t ring, uint64_t init, const DT* h0,
                                          int h0_ld, int h0_valid, char* lds, int dst_off, int dst_ld, int* status,
                                          int* abort_lds, BetweenFn between) {
  PollBatch pb;
  poll_issue<DT>(pb, cur0, 0, g, rs, ring_el, ring_ld, ring);
  between();
  bool ok = poll_finish<DT>(pb, 0, g, rs, ring_el, ring_ld, init, h0, h0_ld, h0_valid, lds, dst_off, dst_ld, status,
                            abort_lds);
  if (g.total <= 8 * kScanThreads) return;
  int r = (int)(pb.cur >> 16), cc = (int)(pb.cur & 0xFFFFu);
  for (int base = kScanThreads * 8; ok && base < g.total; base += kScanThreads * 8) {
#pragma unroll
    for (int i = 0; i < 8; ++i) cursor_step(r, cc, g);
    poll_issue<DT>(pb, (uint32_t)r << 16 | (uint32_t)cc, base, g, rs, ring_el, ring_ld, ring);
    ok = poll_finish<DT>(pb, base, g, rs, ring_el, ring_ld, init, h0, h0_ld, h0_valid, lds, dst_off, dst_ld, status,
                         abort_lds);
  }
}

// Whether every member of a group runs on one XCD. publish_xcd: each member
// stores its hardware XCC id (device-scope) into ids[member], which holds
// the sentinel before the launch. group_on_one_xcd, called by every thread:
// reads all members' ids at once, one thread each (bounded wait; one thread
// reading them in turn took ~7 us for 32 members); the answer is the same in
// every member. *ok turns false when the wait ran out (the members were not
// all resident).
__device__ __forceinline__ void publish_xcd(unsigned* ids, int members, int me) {
  if (threadIdx.x == 0) {
    unsigned hw;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(hw));
    coh_store4(make_rsrc(ids, (uint32_t)members * 4u), (uint32_t)me * 4u, hw & 0xFu);
  }
}
__device__ bool group_on_one_xcd(unsigned* ids, int members, int* ok_lds, int* flag_lds) {
  unsigned hw;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(hw));
  hw &= 0xFu;
  if (threadIdx.x == 0) {
    *flag_lds = 1;
    *ok_lds = 1;
  }
  __syncthreads();
  // thread m reads member m's id (all in flight at once)
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(ids, (uint32_t)members * 4u);
  for (int m = threadIdx.x; m < members; m += kScanThreads) {
    unsigned polls = 0, id;
    uint64_t t0 = 0;
    while ((id = coh_poll4(xr, (uint32_t)m * 4u)) == 0xFFFFFFFFu) {
      if ((++polls & 63u) == 0) {
        const uint64_t now = __builtin_amdgcn_s_memrealtime();
        if (t0 == 0) t0 = now;
        if (now - t0 > kWatchdogTicks) break;
      }
    }
    if (id == 0xFFFFFFFFu) *ok_lds = 0;
    else if (id != hw) *flag_lds = 0;
  }
  __syncthreads();
  return *flag_lds != 0;
}

}  // namespace

}  // namespace rnnk
