// Kernel 2: the persistent scan over time of one layer (all directions).
// The kernel template; scan_<dtype>_<weights>.hip instantiate it.
//
// The recurrence is a true sequential loop over t that runs inside one
// launch (apache/tvm PR "[TOPI] TE implementation of LSTM using scan",
// description: te.scan keeps the time loop sequential instead of unrolling
// it, with a symbolic length). Each step does the hidden-hidden dense op
// h_{t-1} W_hh^T, the gate math with the hoisted Gx added (gates and
// activations fused into the step, as in the same PR's benchmark notes),
// and for LSTMP the hidden-projection dense op h_t = W_hr m_t.
//
// Work split. The batch is cut into blocks of `bb` rows and the hidden units
// into slices of `hs`. A group (one direction x one batch block) is `ns`
// workgroups, one per hidden slice; each keeps its slice of W_hh (all gates
// of its units) and, for LSTMP, a slice of `ps` rows of W_hr resident in
// LDS for the whole launch. Groups never talk to each other. Inside a group
// the state h_t (for LSTMP m_t, then the projected h_t) is exchanged through
// rings of write-once slots in global memory, with no barrier across
// workgroups: step k's values go to slot k mod 4, which holds an all-ones
// sentinel until they arrive, and each member polls its tile of the slot
// until no sentinel is left. A member puts its own entries of a slot back to
// the sentinel once a poll has shown that every member has moved past it.
//
// Variable length (apache/mxnet issue "RNN Op Changes", RFC): row b is
// active at step t iff t < L_b. Inactive rows read nothing, write nothing
// and keep their state, so a reverse-direction row starts at its own
// t = L_b - 1 from h0. A group stops once none of its rows is active.
#pragma once

#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"
#include "scan_common.hpp"

namespace rnnk {

namespace {

constexpr int kThreads = kScanThreads;
constexpr int kMaxEpt = 4;  // owned gate elements per thread: bb * hs <= 1024

struct ScanLds {
  int ws, wr, as, acc, red, lens, flag, total;  // byte offsets
  int ws_ld, wr_ld, as_ld, acc_ld;    // row strides in elements
  int ncw, ncp;                       // W rows (padded to 16), acc columns
  int ncp_wr;                         // W_hr rows held in LDS (LSTMP)
};

__host__ __device__ inline int rup(int x, int m) { return (x + m - 1) / m * m; }

__host__ __device__ inline ScanLds scan_lds(const ScanArgs& a, int esize) {
  ScanLds L;
  const int gates = a.mode == kGRU ? 3 : 4;
  const int pad = 16 / esize;
  const int nc = gates * a.hs;
  L.ncw = rup(nc, 16);
  // register MFMA layouts cover 4 * rnt / rks column tiles (the last ones
  // may be zero padding), all of which the product writes
  if (a.wreg && a.rnt > 0 && 64 * a.rnt / a.rks > L.ncw) L.ncw = 64 * a.rnt / a.rks;
  int ps16 = a.mode == kLSTMP ? rup(a.ps, 16) : 0;
  if (a.mode == kLSTMP && a.pnt > 0 && 64 * a.pnt / a.pks > ps16) ps16 = 64 * a.pnt / a.pks;
  L.ncp = L.ncw > ps16 ? L.ncw : ps16;
  L.ws_ld = a.Kp + pad;
  L.wr_ld = a.Hp + pad;
  const int aw = a.mode == kLSTMP ? (a.Kp > a.Hp ? a.Kp : a.Hp) : a.Kp;
  L.as_ld = aw + pad;
  L.acc_ld = L.ncp + 1;
  const int bb16 = rup(a.bb, 16);
  int off = 0;
  L.ws = off; off += a.wreg ? 0 : rup(L.ncw * L.ws_ld * esize, 16);
  L.ncp_wr = ps16;
  L.wr = off; off += a.mode == kLSTMP ? rup(ps16 * L.wr_ld * esize, 16) : 0;
  L.as = off; off += rup(bb16 * L.as_ld * esize, 16);
  L.acc = off; off += rup(bb16 * L.acc_ld * 4, 16);
  // K-split partial sums of the register-weight and projection products
  int ks_max = a.wreg ? a.rks : 1;
  if (a.mode == kLSTMP && a.pnt > 0 && a.pks > ks_max) ks_max = a.pks;
  L.red = off; off += ks_max > 1 ? rup(ks_max * bb16 * L.acc_ld * 4, 16) : 0;
  L.lens = off; off += rup(a.bb * 4, 16);
  L.flag = off; off += 16;
  L.total = off;
  return L;
}

// ---------------------------------------------------------------------------
// W_hh slice resident in registers. Each lane keeps kScanRegChunks 16-byte
// chunks of the slice for the whole launch, so a step's product reads only
// the h tile from LDS.
// ---------------------------------------------------------------------------
// Global W_hh row of row r of the slice (gate q, owned unit u), -1 for padding.
__device__ __forceinline__ int slice_row(int r, int hs, int hs_act, int gates, int H, int j0) {
  const int q = r / hs, u = r - q * hs;
  return (q < gates && u < hs_act) ? q * H + j0 + u : -1;
}

// Chunk of global row gr of W (row length K) starting at column k0; zero
// for padding rows and columns. The register path is only planned when W is
// 16-byte aligned and K is a multiple of a chunk, so a chunk is one aligned
// 16-byte load that lies wholly inside or wholly outside the row.
template <typename DT>
__device__ __forceinline__ typename Chunk<DT>::T load_chunk(const DT* w, int gr, int K, int k0) {
  typedef typename Chunk<DT>::T V;
  V v = {};
  if (gr >= 0 && k0 < K) v = *reinterpret_cast<const V*>(w + (size_t)gr * K + k0);
  return v;
}

// MFMA layout: wave w holds column tiles (w / rks) * NTC + j, j < NTC, over
// K chunks [(w % rks) * rcpt, + rcpt); lane l holds, for each, row
// 16 * tile + l % 16 at k-group l / 16 (the B operand of Chunk<DT>::mfma).
template <typename DT, int NTC>
__device__ __forceinline__ void load_wreg_mfma(typename Chunk<DT>::T (&wr)[kScanRegChunks], const DT* w,
                                               const ScanArgs& a, int gates, int j0, int hs_act) {
  constexpr int CPT = kScanRegChunks / NTC;
  constexpr int kEpc = 16 / sizeof(DT), kK = Chunk<DT>::kK;
  const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4, wave = threadIdx.x >> 6;
  const int tg = wave / a.rks, ks = wave - tg * a.rks;
#pragma unroll
  for (int j = 0; j < NTC; ++j) {
    const int gr = slice_row((tg * NTC + j) * 16 + lr, a.hs, hs_act, gates, a.H, j0);
#pragma unroll
    for (int ch = 0; ch < CPT; ++ch)
      wr[j * CPT + ch] = load_chunk<DT>(w, ch < a.rcpt ? gr : -1, a.K, (ks * a.rcpt + ch) * kK + lq * kEpc);
  }
}

// out[r][c] (row stride out_ld) = sum_k A[r][k] W[c][k] for the wave's tiles,
// rows 16 * rtiles; with rks > 1 each K share writes its own partial block
// (16 * rtiles rows apart) for reduce_ksplit.
template <typename DT, int NTC>
__device__ __forceinline__ void mm_wreg(const typename Chunk<DT>::T (&wr)[kScanRegChunks], const DT* As, int as_ld,
                                        int rtiles, const ScanArgs& a, float* out, int out_ld) {
  typedef typename Chunk<DT>::T V;
  constexpr int CPT = kScanRegChunks / NTC;
  constexpr int kEpc = 16 / sizeof(DT), kK = Chunk<DT>::kK;
  const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4, wave = threadIdx.x >> 6;
  const int tg = wave / a.rks, ks = wave - tg * a.rks;
  float* o = out + ks * rtiles * 16 * out_ld;
  for (int rt = 0; rt < rtiles; ++rt) {
    f32x4 c[NTC];
#pragma unroll
    for (int j = 0; j < NTC; ++j) c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const DT* ap = As + (rt * 16 + lr) * as_ld + lq * kEpc + ks * a.rcpt * kK;
    // Groups of four A chunks, each loaded before the previous group's
    // MFMAs so that its LDS latency overlaps them.
    V x[2][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) x[0][q] = *reinterpret_cast<const V*>(ap + q * kK);
#pragma unroll
    for (int g = 0; g < CPT; g += 4) {
      if (g < a.rcpt) {  // rcpt is a multiple of 4
        const int cur = (g / 4) & 1;
        if (g + 4 < a.rcpt) {
#pragma unroll
          for (int q = 0; q < 4; ++q) x[cur ^ 1][q] = *reinterpret_cast<const V*>(ap + (g + 4 + q) * kK);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int j = 0; j < NTC; ++j) c[j] = Chunk<DT>::mfma(x[cur][q], wr[j * CPT + g + q], c[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < NTC; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) o[(rt * 16 + 4 * lq + v) * out_ld + (tg * NTC + j) * 16 + lr] = c[j][v];
  }
}

// The same wave layout with the B operand read from LDS (W rows of stride
// w_ld): wave w takes column tiles (w / ks) * NTC + j over K chunks
// [(w % ks) * cpt, + cpt); with ks > 1 each K share writes its own partial
// block for reduce_ksplit.
template <typename DT, int NTC>
__device__ __forceinline__ void mm_lds_split(const DT* As, int as_ld, const DT* Ws, int w_ld, int rtiles, int ks_n,
                                             int cpt, float* out, int out_ld) {
  typedef typename Chunk<DT>::T V;
  constexpr int kEpc = 16 / sizeof(DT), kK = Chunk<DT>::kK;
  const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4, wave = threadIdx.x >> 6;
  const int tg = wave / ks_n, ks = wave - tg * ks_n;
  float* o = out + ks * rtiles * 16 * out_ld;
  const DT* wp[NTC];
#pragma unroll
  for (int j = 0; j < NTC; ++j) wp[j] = Ws + ((tg * NTC + j) * 16 + lr) * w_ld + lq * kEpc + ks * cpt * kK;
  for (int rt = 0; rt < rtiles; ++rt) {
    f32x4 c[NTC];
#pragma unroll
    for (int j = 0; j < NTC; ++j) c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const DT* ap = As + (rt * 16 + lr) * as_ld + lq * kEpc + ks * cpt * kK;
    for (int g = 0; g < cpt; g += 4) {  // cpt is a multiple of 4
      V x[4], y[4][NTC];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        x[q] = *reinterpret_cast<const V*>(ap + (g + q) * kK);
#pragma unroll
        for (int j = 0; j < NTC; ++j) y[q][j] = *reinterpret_cast<const V*>(wp[j] + (g + q) * kK);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < NTC; ++j) c[j] = Chunk<DT>::mfma(x[q], y[q][j], c[j]);
    }
#pragma unroll
    for (int j = 0; j < NTC; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) o[(rt * 16 + 4 * lq + v) * out_ld + (tg * NTC + j) * 16 + lr] = c[j][v];
  }
}

// VALU layout (batch blocks below 16 rows): thread t owns column
// t % (256 / rks) of the slice over K chunks [(t / (256 / rks)) * rcpt, + rcpt).
template <typename DT>
__device__ __forceinline__ void load_wreg_valu(typename Chunk<DT>::T (&wr)[kScanRegChunks], const DT* w,
                                               const ScanArgs& a, int gates, int j0, int hs_act) {
  constexpr int kEpc = 16 / sizeof(DT);
  const int C = kThreads / a.rks;
  const int c = threadIdx.x % C, q = threadIdx.x / C;
  const int gr = slice_row(c, a.hs, hs_act, gates, a.H, j0);
#pragma unroll
  for (int s = 0; s < kScanRegChunks; ++s)
    wr[s] = load_chunk<DT>(w, s < a.rcpt ? gr : -1, a.K, (q * a.rcpt + s) * kEpc);
}

// One chunk of a VALU dot product into two accumulators. bf16 pairs go
// through the packed dot instruction, so the resident weights are never
// widened (widened copies would be hoisted out of the loop and double the
// registers they occupy).
template <typename DT>
__device__ __forceinline__ void valu_chunk(const typename Chunk<DT>::T& wv, const DT* xp, float& s0, float& s1);
template <>
__device__ __forceinline__ void valu_chunk<float>(const f32x4& wv, const float* xp, float& s0, float& s1) {
  const f32x4 x = *reinterpret_cast<const f32x4*>(xp);
  s0 = __builtin_fmaf(x[0], wv[0], s0);
  s1 = __builtin_fmaf(x[1], wv[1], s1);
  s0 = __builtin_fmaf(x[2], wv[2], s0);
  s1 = __builtin_fmaf(x[3], wv[3], s1);
}
template <>
__device__ __forceinline__ void valu_chunk<bf16>(const bf16x8& wv, const bf16* xp, float& s0, float& s1) {
  const bf16x8 x = *reinterpret_cast<const bf16x8*>(xp);
  s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 0, 1), __builtin_shufflevector(wv, wv, 0, 1),
                                       s0, false);
  s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 2, 3), __builtin_shufflevector(wv, wv, 2, 3),
                                       s1, false);
  s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 4, 5), __builtin_shufflevector(wv, wv, 4, 5),
                                       s0, false);
  s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 6, 7), __builtin_shufflevector(wv, wv, 6, 7),
                                       s1, false);
}

// out[r][c] = sum_k A[r][k] W[c][k], r < rows, for the thread's column and
// K share; with rks > 1 each share writes its own partial block (rows apart
// by `rows`) for reduce_ksplit. All lanes of a wave read the same A chunk.
template <typename DT>
__device__ __forceinline__ void mm_wreg_valu(const typename Chunk<DT>::T (&wr)[kScanRegChunks], const DT* As,
                                             int as_ld, int rows, int ncols, const ScanArgs& a, float* out,
                                             int out_ld) {
  constexpr int kEpc = 16 / sizeof(DT);
  const int C = kThreads / a.rks;
  const int c = threadIdx.x % C, q = threadIdx.x / C;
  float* o = out + q * rows * out_ld;
  for (int r = 0; r < rows; ++r) {
    const DT* xr = As + r * as_ld + q * a.rcpt * kEpc;
    float s0 = 0.f, s1 = 0.f;
    if ((a.rcpt & 3) == 0) {
#pragma unroll
      for (int g = 0; g < kScanRegChunks; g += 4) {
        if (g < a.rcpt) {
#pragma unroll
          for (int u = 0; u < 4; ++u) valu_chunk<DT>(wr[g + u], xr + (g + u) * kEpc, s0, s1);
        }
      }
    } else {
#pragma unroll
      for (int g = 0; g < kScanRegChunks; ++g)
        if (g < a.rcpt) valu_chunk<DT>(wr[g], xr + g * kEpc, s0, s1);
    }
    if (c < ncols) o[r * out_ld + c] = s0 + s1;
  }
}

// acc[r][c] = sum over the rks K shares of their partial blocks (fixed order).
__device__ __forceinline__ void reduce_ksplit(const float* red, int rks, int rows, int ncols, float* acc,
                                              int acc_ld) {
  for (int i = threadIdx.x; i < rows * ncols; i += kThreads) {
    const int r = i / ncols, c = i - r * ncols;
    float v = red[r * acc_ld + c];
    for (int k = 1; k < rks; ++k) v += red[(k * rows + r) * acc_ld + c];
    acc[r * acc_ld + c] = v;
  }
}

// EPT: gate elements (and, for LSTMP, projection outputs) owned per thread,
// 1, 2 or 4 (bb * hs <= 256 * EPT). PROJ: LSTMP (the hidden projection).
// GXB: G_x stored as bf16 (bf16 storage only). RSV: training, the gate
// values go to the reserve (fp32 only; the forward instances carry none of
// that code or its scalar state).
template <typename DT, bool WREG, int EPT, bool PROJ, bool GXB, bool RSV>
__global__ void __launch_bounds__(kThreads) scan_kernel(ScanArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const ScanLds L = scan_lds(a, (int)sizeof(DT));
  const int tid = threadIdx.x;
  const int gates = a.mode == kGRU ? 3 : 4;

  // Workgroup -> (layer slot, direction, batch block, hidden slice).
  // Workgroups are dealt to the XCDs round-robin by id, so with gpx > 0 the
  // ids xcd, xcd + nxcd, ... form the groups of one XCD and a group's
  // exchange stays between the CUs of one chiplet (placement only;
  // correctness never depends on it).
  int s, grp;
  if (a.gpx > 0) {
    const int xcd = blockIdx.x % a.nxcd, pos = blockIdx.x / a.nxcd;
    grp = xcd * a.gpx + pos / a.ns;
    s = pos % a.ns;
  } else {
    s = blockIdx.x % a.ns;
    grp = blockIdx.x / a.ns;
  }
  const int gpl = a.D * a.nbb;  // groups per layer slot
  if (grp >= a.nslot * gpl) return;  // padding slots of the XCD-aligned layout
  const int ls = grp / gpl;
  if (a.T[ls] <= 0) return;  // idle slot
  grp -= ls * gpl;
  const int nb = grp % a.nbb;
  const int d = grp / a.nbb;
  const int q = ls * a.D + d;  // index of the per-(slot, direction) tensors
  const int b0 = nb * a.bb;
  const int j0 = s * a.hs;
  const int hs_act = min(a.hs, a.H - j0);  // may be <= 0 for a trailing slice
  const int p0 = s * a.ps;
  const int ps_act = PROJ ? min(a.ps, a.P - p0) : 0;
  const bool rev = d == 1;
  const int DK = a.D * a.K;
  const int DG = a.D * a.G;
  // flags[0]: abort (a member's watchdog fired), flags[1]: the group shares
  // one XCD, flags[2]: every member published its XCD id in time
  int* flags = reinterpret_cast<int*>(lds + L.flag);
  int* abort_flag = flags;

  // Ring slots: step k's exchanged state (h_t, for LSTMP the projected h_t)
  // goes to hx slot k mod kRingSlots; LSTMP's m_t to mx slot k mod kRingSlots.
  const uint32_t hx_bytes = (uint32_t)(kRingSlots * a.D * a.B * a.Kp) * sizeof(DT);
  const __amdgpu_buffer_rsrc_t hx_rs = make_rsrc(a.hx[ls], hx_bytes);
  const uint32_t mx_bytes = PROJ ? (uint32_t)(kRingSlots * a.D * a.B * a.Hp) * sizeof(DT) : 16u;
  const __amdgpu_buffer_rsrc_t mx_rs = make_rsrc(PROJ ? a.mx[ls] : a.hx[ls], mx_bytes);
  auto hx_el = [&](int k, int b, int c) -> uint32_t {
    return (uint32_t)((((k & (kRingSlots - 1)) * a.D + d) * a.B + b) * a.Kp + c);
  };
  auto mx_el = [&](int k, int b, int j) -> uint32_t {
    return (uint32_t)((((k & (kRingSlots - 1)) * a.D + d) * a.B + b) * a.Hp + j);
  };
  // Lengths of the block's rows, staged once: reading them from global
  // memory inside the step loop would make every use wait for all of the
  // wave's outstanding memory operations.
  int* lens = reinterpret_cast<int*>(lds + L.lens);
  for (int r = tid; r < a.bb; r += kThreads)
    lens[r] = b0 + r < a.B ? (a.lengths ? a.lengths[b0 + r] : a.T[ls]) : 0;
  if (tid == 0) {
    flags[0] = 0;
    flags[1] = 1;
    flags[2] = 1;
  }
  __syncthreads();
  auto len_of = [&](int b) -> int { return lens[b - b0]; };

  // --- resident weights -----------------------------------------------------
  const DT* whh = reinterpret_cast<const DT*>(a.w_hh[q]);
  typename Chunk<DT>::T wreg[WREG ? kScanRegChunks : 1];
  if constexpr (WREG) {
    switch (a.rnt) {
      case 1: load_wreg_mfma<DT, 1>(wreg, whh, a, gates, j0, hs_act); break;
      case 2: load_wreg_mfma<DT, 2>(wreg, whh, a, gates, j0, hs_act); break;
      case 4: load_wreg_mfma<DT, 4>(wreg, whh, a, gates, j0, hs_act); break;
      default: load_wreg_valu<DT>(wreg, whh, a, gates, j0, hs_act); break;
    }
  } else {
    load_weights<DT>(whh, a.K, a.Kp, L.ncw, [&](int r) -> int {
      return slice_row(r, a.hs, hs_act, gates, a.H, j0);
    }, lds, L.ws, L.ws_ld);
  }
  if (PROJ) {
    const DT* whr = reinterpret_cast<const DT*>(a.w_hr[q]);
    load_weights<DT>(whr, a.H, a.Hp, L.ncp_wr, [&](int r) -> int {
      return r < ps_act ? p0 + r : -1;
    }, lds, L.wr, L.wr_ld);
  }

  // A group of one workgroup owns every hidden unit of its rows: h_t then
  // never leaves the workgroup and is written straight into the LDS operand
  // tile of the next step (no exchange buffer, no group barrier).
  const bool solo = a.ns == 1 && !PROJ;
  const bool use_mfma = (a.bb % 16) == 0;
  const int tile_rows = use_mfma ? rup(a.bb, 16) : a.bb;
  DT* tile = reinterpret_cast<DT*>(lds + L.as);
  // Plain stores suffice for the ring when the whole group runs on one XCD.
  bool local = true;
  if (a.ns > 1) {
    // (publishing at kernel entry instead, to overlap the members' arrival
    // with the weight loads, measured 12-16% slower steps on every shape)
    publish_xcd(a.xid[ls] + (size_t)grp * a.ns, a.ns, s);
    local = group_on_one_xcd(a.xid[ls] + (size_t)grp * a.ns, a.ns, flags + 2, flags + 1);
    if (!flags[2]) {
      if (tid == 0) __hip_atomic_store(a.status, kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
  }
  // The first member zeroes the rings' padding columns of the block's rows
  // in every slot (readers check and copy whole chunks; the sentinel stays
  // in them until these stores arrive).
  if (!solo && s == 0) {
    const int padh = a.Kp - a.K, padm = PROJ ? a.Hp - a.H : 0;
    for (int e = tid; e < kRingSlots * a.bb * (padh + padm); e += kThreads) {
      const int q = e / (a.bb * (padh + padm)), rem = e - q * (a.bb * (padh + padm));
      const int r = rem / (padh + padm), c = rem - r * (padh + padm);
      if (b0 + r >= a.B) continue;
      if (c < padh)
        ring_store<DT>(hx_rs, hx_el(q, b0 + r, a.K + c), 0.f, local);
      else
        ring_store<DT>(mx_rs, mx_el(q, b0 + r, a.H + c - padh), 0.f, local);
    }
  }
  if (solo) {
    const DT* h0s = reinterpret_cast<const DT*>(a.h0[q]);
    for (int e = tid; e < tile_rows * a.Kp; e += kThreads) {
      const int r = e / a.Kp, k = e - r * a.Kp;
      const int b = b0 + r;
      tile[r * L.as_ld + k] = (h0s && b < a.B && k < a.K) ? h0s[(size_t)b * a.K + k] : (DT)0.0f;
    }
  }

  // --- owned state: gate elements e = tid + i * 256 -> (row r, unit u) -------
  const int n_el = a.bb * a.hs;
  float hreg[EPT], creg[EPT];
  float bhn[EPT];
  const DT* h0 = reinterpret_cast<const DT*>(a.h0[q]);
  const DT* c0 = reinterpret_cast<const DT*>(a.c0[q]);
  const DT* bhh = reinterpret_cast<const DT*>(a.b_hh[q]);
  // Owned element i: row er[i] of the block, unit eu[i] of the slice, and the
  // row's length (0 when the element is not owned), computed once.
  int lenreg[EPT], er[EPT], eu[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int e = tid + i * kThreads;
    const int r = e / a.hs, u = e - r * a.hs;
    const int b = b0 + r;
    er[i] = r;
    eu[i] = u;
    hreg[i] = 0.f; creg[i] = 0.f; bhn[i] = 0.f;
    lenreg[i] = (e < n_el && u < hs_act && b < a.B) ? len_of(b) : 0;
    if (e < n_el && u < hs_act && b < a.B) {
      const int j = j0 + u;
      if (!PROJ && a.h0f[q])
        hreg[i] = a.h0f[q][(size_t)b * a.H + j];
      else if (!PROJ && h0)
        hreg[i] = to_f32<DT>(h0[(size_t)b * a.K + j]);
      if (a.mode != kGRU && a.c0f[q])
        creg[i] = a.c0f[q][(size_t)b * a.H + j];
      else if (a.mode != kGRU && c0)
        creg[i] = to_f32<DT>(c0[(size_t)b * a.H + j]);
      if (a.mode == kGRU && a.has_bias) bhn[i] = to_f32<DT>(bhh[2 * a.H + j]);
    }
  }

  // Longest sequence of this block bounds the steps it takes part in
  // (wave-uniform, so per-step indices stay in scalar registers).
  int maxlen = 0;
  for (int r = 0; r < a.bb && b0 + r < a.B; ++r) maxlen = max(maxlen, len_of(b0 + r));
  maxlen = __builtin_amdgcn_readfirstlane(maxlen);

  float* acc = reinterpret_cast<float*>(lds + L.acc);
  const int mtiles = rup(a.bb, 16) / 16;
  DT* yout = reinterpret_cast<DT*>(a.y[ls]);
  DT* hn = reinterpret_cast<DT*>(a.h_n[q]);
  DT* cn = reinterpret_cast<DT*>(a.c_n[q]);
  // The block takes part in steps t < maxlen: forward t = 0 .. maxlen-1,
  // reverse t = maxlen-1 .. 0 (earlier reverse steps have no active row).
  const int nsteps = maxlen;
  auto t_of = [&](int k) { return rev ? maxlen - 1 - k : k; };
  // The offsets are read through the constant address space: a scalar load,
  // so the step does not wait for the vector memory counter to drain, and
  // the buffer resources built from the result stay in scalar registers.
  typedef const __attribute__((address_space(4))) int const_int;
  const const_int* offs = (const const_int*)a.offsets;
  auto rowbase_of = [&](int t) { return a.packed ? offs[t] : t * a.B; };

  // Where the block's rows take h_{t-1} at loop step k, as wave-uniform bit
  // masks over the rows (lane r of every wave evaluates row r): `ring` the
  // ring slot of step k - 1, `init` h0 (the row's first active step); other
  // rows are inactive (their products are computed on zeros and not used).
  const int lane = tid & 63;
  const int lane_len = lane < a.bb ? lens[lane] : 0;
  auto row_masks = [&](int k, uint64_t& ring, uint64_t& init) __attribute__((always_inline)) {
    const int first = rev ? maxlen - lane_len : 0;
    const bool act = lane < a.bb && k >= first && (rev || k < lane_len);
    ring = __ballot(act && k > first);
    init = __ballot(act && k == first);
  };
  const PollGeom ghx = poll_geom(tile_rows, a.Kp, 16 / (int)sizeof(DT));
  const PollGeom gmx = poll_geom(tile_rows, a.Hp, 16 / (int)sizeof(DT));
  const uint32_t cur_hx = poll_cursor0(ghx), cur_mx = poll_cursor0(gmx);
  const DT* h0b = h0 ? h0 + (size_t)b0 * a.K : nullptr;

  // The memory operations issued between a step's first poll loads and the
  // wait for them (outputs of the previous step, G_x of the next) are a
  // fixed number of unconditional buffer instructions: an inactive element
  // gets an offset past the end of the buffer (its load returns zero, its
  // store is dropped). The compiler then waits for the poll loads alone.
  constexpr uint32_t kOob = 0x7FFFFFF0u;
  const uint32_t es = sizeof(DT);

  // G_x of the owned elements for loop step k1 (zero for inactive ones), as
  // raw words (GXB: 16-bit loads of bf16 G_x, else 32-bit), widened by gxf
  // where the gate math uses them: widening here would make every load
  // wait at once. For the 16-bit loads the offsets pass through an opaque
  // copy: the select with a constant arm is otherwise split into two loads
  // on divergent branches, which both issue when lanes differ and leave the
  // compiler's count of younger loads short, so the poll check would wait
  // for some G_x loads (for the 32-bit loads the split measured faster).
  typedef typename std::conditional<GXB, uint16_t, uint32_t>::type GxW;
  constexpr uint32_t gsz = sizeof(GxW);
  auto prefetch = [&](int k1, uint32_t (&g)[EPT][4]) __attribute__((always_inline)) {
    const bool in = k1 < nsteps;
    const int t1 = in ? t_of(k1) : 0;
    const __amdgpu_buffer_rsrc_t g_rs = make_rsrc(
        reinterpret_cast<const char*>(a.gx[ls]) + (size_t)rowbase_of(t1) * DG * gsz, (uint32_t)(a.B * DG) * gsz);
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const bool act = in && t1 < lenreg[i];
      const uint32_t e0 = (uint32_t)((b0 + er[i]) * DG + d * a.G + j0 + eu[i]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t off = act && q < gates ? (e0 + (uint32_t)(q * a.H)) * gsz : kOob;
        if constexpr (GXB) asm volatile("" : "+v"(off));
        if constexpr (GXB)
          g[i][q] = __builtin_amdgcn_raw_buffer_load_b16(g_rs, (int)off, 0, 0);
        else
          g[i][q] = __builtin_amdgcn_raw_buffer_load_b32(g_rs, (int)off, 0, 0);
      }
    }
  };
  auto gxf = [&](uint32_t w) __attribute__((always_inline)) { return __builtin_bit_cast(float, GXB ? w << 16 : w); };
  // Output y of loop step kp, whose h is still in hreg (for LSTMP: whose
  // projected h is still in acc). h_n and c_n are written after the loop.
  auto outputs = [&](int kp) __attribute__((always_inline)) {
    const bool in = kp >= 0;
    const int tp = in ? t_of(kp) : 0;
    const __amdgpu_buffer_rsrc_t y_rs = make_rsrc(yout + (size_t)rowbase_of(tp) * DK, (uint32_t)(a.B * DK) * es);
    if (!PROJ) {
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        const int b = b0 + er[i], j = j0 + eu[i];
        const bool act = in && tp < lenreg[i];
        out_store<DT>(y_rs, act ? (uint32_t)(b * DK + d * a.K + j) * es : kOob, hreg[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        const int e = tid + i * kThreads;
        const int r = e / a.ps, p = e - r * a.ps;
        const int b = b0 + r;
        const bool own = e < a.bb * a.ps && p < ps_act && b < a.B;
        const int lb = lens[own ? r : 0] * (own ? 1 : 0);
        const bool act = in && tp < lb;
        const float h = clampf(acc[own ? r * L.acc_ld + p : 0], a.p_lo, a.p_hi);
        out_store<DT>(y_rs, act ? (uint32_t)(b * DK + d * a.K + p0 + p) * es : kOob, h);
      }
    }
  };

  // One loop step. gc holds this step's G_x; the next step's goes to gn and
  // is moved to gc once the gate math is done (before the ring stores, so
  // the move waits for nothing issued after the loads).
  uint32_t gc[EPT][4], gn[EPT][4];
  float hlast[EPT];  // LSTMP: last projected h of each owned output (for h_n)
#pragma unroll
  for (int i = 0; i < EPT; ++i) hlast[i] = 0.f;
  auto step = [&](int k) __attribute__((always_inline)) -> bool {
    const int t = t_of(k);
    const int rowbase = rowbase_of(t);
    uint64_t mring = 0, minit = 0;
    if (!solo) row_masks(k, mring, minit);
    // h_{t-1} of the block -> LDS, then the hidden-hidden product.
    if (!solo) {
      poll_tile<DT>(ghx, cur_hx, hx_rs, hx_el(k - 1, b0, 0), a.Kp, mring, minit, h0b, a.K, a.K, lds, L.as, L.as_ld,
                    a.status, abort_flag, [&] {
                      outputs(k - 1);
                      prefetch(k + 1, gn);
                    });
      lds_barrier();
      if (*abort_flag) return false;
      // Every member has published step k - 1, after reading slot k - 2:
      // put this workgroup's entries of that slot back to the sentinel.
      if (!PROJ && k >= 2) {
        const int tp = t_of(k - 2);
#pragma unroll
        for (int i = 0; i < EPT; ++i)
          if (tp < lenreg[i]) ring_reset<DT>(hx_rs, hx_el(k - 2, b0 + er[i], j0 + eu[i]), local);
      }
    } else {
      outputs(k - 1);
      prefetch(k + 1, gn);
    }
    if constexpr (WREG) {
      const DT* As = reinterpret_cast<const DT*>(lds + L.as);
      float* part = a.rks > 1 ? reinterpret_cast<float*>(lds + L.red) : acc;
      switch (a.rnt) {
        case 1: mm_wreg<DT, 1>(wreg, As, L.as_ld, mtiles, a, part, L.acc_ld); break;
        case 2: mm_wreg<DT, 2>(wreg, As, L.as_ld, mtiles, a, part, L.acc_ld); break;
        case 4: mm_wreg<DT, 4>(wreg, As, L.as_ld, mtiles, a, part, L.acc_ld); break;
        default: mm_wreg_valu<DT>(wreg, As, L.as_ld, a.bb, L.ncw, a, part, L.acc_ld); break;
      }
      if (a.rks > 1) {
        lds_barrier();
        reduce_ksplit(part, a.rks, a.rnt ? tile_rows : a.bb, L.ncw, acc, L.acc_ld);
      }
    } else if (use_mfma) {
      mm_mfma<DT>(lds, L.as, L.as_ld, L.ws, L.ws_ld, acc, L.acc_ld, mtiles, L.ncw / 16, a.Kp);
    } else {
      mm_valu<DT>(lds, L.as, L.as_ld, L.ws, L.ws_ld, acc, L.acc_ld, a.bb, gates * a.hs, a.Kp);
    }
    lds_barrier();

    // Gate math on the owned elements.
    float gsv[EPT][5];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int r = er[i], u = eu[i];
      if (t >= lenreg[i]) continue;
      const float* ar = acc + r * L.acc_ld;
      if (a.mode == kGRU) {
        const float rg = fsigmoid(gxf(gc[i][0]) + ar[u]);
        const float zg = fsigmoid(gxf(gc[i][1]) + ar[a.hs + u]);
        const float hn_pre = ar[2 * a.hs + u] + bhn[i];
        const float ng = ftanh(gxf(gc[i][2]) + rg * hn_pre);
        gsv[i][0] = rg;
        gsv[i][1] = zg;
        gsv[i][2] = ng;
        gsv[i][3] = hn_pre;
        hreg[i] = (1.f - zg) * ng + zg * hreg[i];
      } else {
        const float ig = fsigmoid(gxf(gc[i][0]) + ar[u]);
        const float fg = fsigmoid(gxf(gc[i][1]) + ar[a.hs + u]);
        const float gg = ftanh(gxf(gc[i][2]) + ar[2 * a.hs + u]);
        const float og = fsigmoid(gxf(gc[i][3]) + ar[3 * a.hs + u]);
        const float c = clampf(fg * creg[i] + ig * gg, a.c_lo, a.c_hi);
        gsv[i][0] = ig;
        gsv[i][1] = fg;
        gsv[i][2] = gg;
        gsv[i][3] = og;
        gsv[i][4] = c;
        creg[i] = c;
        hreg[i] = og * ftanh(c);
      }
    }
#pragma unroll
    for (int i = 0; i < EPT; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) gc[i][q] = gn[i][q];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int r = er[i], u = eu[i];
      const int b = b0 + r;
      if (t >= lenreg[i]) continue;
      const int j = j0 + u;
      const float h = hreg[i];
      if (solo)
        tile[r * L.as_ld + j] = from_f32<DT>(h);
      else if (!PROJ)
        ring_store<DT>(hx_rs, hx_el(k, b, j), h, local);
      else
        ring_store<DT>(mx_rs, mx_el(k, b, j), h, local);
      if (RSV) {
        const int nsv = a.mode == kGRU ? 4 : 5;
        float* rv = a.rsv + ((size_t)(rowbase + b) * a.D + d) * (nsv * a.H) + j;
#pragma unroll
        for (int q = 0; q < 5; ++q)
          if (q < nsv) rv[q * a.H] = gsv[i][q];
      }
    }
    if (solo) lds_barrier();
    if (!PROJ) return true;

    // hidden-projection dense: h_t = m_t W_hr^T for this slice of P
    poll_tile<DT>(gmx, cur_mx, mx_rs, mx_el(k, b0, 0), a.Hp, mring | minit, 0ull, (const DT*)nullptr, 0, 0, lds,
                  L.as, L.as_ld, a.status, abort_flag, [] {});
    lds_barrier();
    if (*abort_flag) return false;
    // Every member has published m of step k: it has read h of step k - 1
    // and m of step k - 1, so this workgroup's entries of both slots go
    // back to the sentinel.
    if (k >= 1) {
      const int tp = t_of(k - 1);
#pragma unroll
      for (int i = 0; i < EPT; ++i)
        if (tp < lenreg[i]) ring_reset<DT>(mx_rs, mx_el(k - 1, b0 + er[i], j0 + eu[i]), local);
      for (int e = tid; e < a.bb * a.ps; e += kThreads) {
        const int r = e / a.ps, p = e - r * a.ps;
        const int b = b0 + r;
        if (p < ps_act && b < a.B && tp < len_of(b)) ring_reset<DT>(hx_rs, hx_el(k - 1, b, p0 + p), local);
      }
    }
    if (use_mfma && a.pnt > 0) {
      const DT* As = reinterpret_cast<const DT*>(lds + L.as);
      const DT* Wr = reinterpret_cast<const DT*>(lds + L.wr);
      float* part = a.pks > 1 ? reinterpret_cast<float*>(lds + L.red) : acc;
      switch (a.pnt) {
        case 1: mm_lds_split<DT, 1>(As, L.as_ld, Wr, L.wr_ld, mtiles, a.pks, a.pcpt, part, L.acc_ld); break;
        case 2: mm_lds_split<DT, 2>(As, L.as_ld, Wr, L.wr_ld, mtiles, a.pks, a.pcpt, part, L.acc_ld); break;
        default: mm_lds_split<DT, 4>(As, L.as_ld, Wr, L.wr_ld, mtiles, a.pks, a.pcpt, part, L.acc_ld); break;
      }
      if (a.pks > 1) {
        lds_barrier();
        reduce_ksplit(part, a.pks, tile_rows, 64 * a.pnt / a.pks, acc, L.acc_ld);
      }
    } else if (use_mfma) {
      mm_mfma<DT>(lds, L.as, L.as_ld, L.wr, L.wr_ld, acc, L.acc_ld, mtiles, rup(a.ps, 16) / 16, a.Hp);
    } else {
      mm_valu<DT>(lds, L.as, L.as_ld, L.wr, L.wr_ld, acc, L.acc_ld, a.bb, a.ps, a.Hp);
    }
    lds_barrier();
    // acc keeps the projected h_t until the next step's product: the outputs
    // are written from it at the top of the next step.
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int e = tid + i * kThreads;
      const int r = e / a.ps, p = e - r * a.ps;
      const int b = b0 + r;
      if (e >= a.bb * a.ps || p >= ps_act || b >= a.B) continue;
      if (t >= len_of(b)) continue;
      const float h = clampf(acc[r * L.acc_ld + p], a.p_lo, a.p_hi);
      hlast[i] = h;
      ring_store<DT>(hx_rs, hx_el(k, b, p0 + p), h, local);
    }
    return true;
  };

  prefetch(0, gc);
  // Nothing outstanding when the loop starts (the resident weights, G_x of
  // the first step), so no wait inside the loop has to cover them; the
  // barrier publishes the LDS weights and the solo tile.
  wait_all_mem();
  __syncthreads();
  for (int k = 0; k < nsteps; ++k)
    if (!step(k)) return;
  if (nsteps > 0) outputs(nsteps - 1);
  // Final state: every owned element's registers hold its row's last step.
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    if (lenreg[i] <= 0) continue;
    const int b = b0 + er[i], j = j0 + eu[i];
    if (!PROJ && hn) hn[(size_t)b * a.K + j] = from_f32<DT>(hreg[i]);
    if (a.mode != kGRU && cn) cn[(size_t)b * a.H + j] = from_f32<DT>(creg[i]);
    if (!PROJ && a.h_nf[q]) a.h_nf[q][(size_t)b * a.H + j] = hreg[i];
    if (a.mode != kGRU && a.c_nf[q]) a.c_nf[q][(size_t)b * a.H + j] = creg[i];
  }
  if (PROJ && hn) {
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int e = tid + i * kThreads;
      const int r = e / a.ps, p = e - r * a.ps;
      const int b = b0 + r;
      if (e < a.bb * a.ps && p < ps_act && b < a.B && lens[r] > 0) hn[(size_t)b * a.K + p0 + p] = from_f32<DT>(hlast[i]);
    }
  }
}


// Launch of one instance: EPT from the owned elements, PROJ from the mode.
template <typename DT, bool WREG, int EPT, bool PROJ, bool GXB, bool RSV>
hipError_t launch_scan_as(const ScanArgs& a, int lds, dim3 grid, hipStream_t stream) {
  hipError_t e = hipFuncSetAttribute((const void*)scan_kernel<DT, WREG, EPT, PROJ, GXB, RSV>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  launch_kernel((scan_kernel<DT, WREG, EPT, PROJ, GXB, RSV>), grid, dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

template <typename DT, bool WREG, bool PROJ, bool GXB, bool RSV>
hipError_t launch_scan_ept(const ScanArgs& a, int lds, dim3 grid, hipStream_t stream) {
  const int own = max(a.bb * a.hs, PROJ ? a.bb * a.ps : 0);
  if (own <= kThreads) return launch_scan_as<DT, WREG, 1, PROJ, GXB, RSV>(a, lds, grid, stream);
  if (own <= 2 * kThreads) return launch_scan_as<DT, WREG, 2, PROJ, GXB, RSV>(a, lds, grid, stream);
  if (own <= kMaxEpt * kThreads) return launch_scan_as<DT, WREG, kMaxEpt, PROJ, GXB, RSV>(a, lds, grid, stream);
  return hipErrorInvalidValue;
}

// bf16 G_x only with bf16 storage; RSV: the training instances (a.rsv set).
template <typename DT, bool WREG, bool GXB, bool RSV = false>
hipError_t launch_scan_proj(const ScanArgs& a, int lds, dim3 grid, hipStream_t stream) {
  if ((a.rsv != nullptr) != RSV) return hipErrorInvalidValue;
  return a.mode == kLSTMP ? launch_scan_ept<DT, WREG, true, GXB, RSV>(a, lds, grid, stream)
                          : launch_scan_ept<DT, WREG, false, GXB, RSV>(a, lds, grid, stream);
}

}  // namespace
}  // namespace rnnk
