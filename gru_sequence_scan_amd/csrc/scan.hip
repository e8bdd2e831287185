// Kernel 2: the persistent scan over time of one layer (all directions).
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
// the state h_t is exchanged through a device-coherent ping-pong buffer and
// one barrier per step (two for LSTMP: after m_t, after h_t).
//
// Variable length (apache/mxnet issue "RNN Op Changes", RFC): row b is
// active at step t iff t < L_b. Inactive rows read nothing, write nothing
// and keep their state, so a reverse-direction row starts at its own
// t = L_b - 1 from h0. A group stops once none of its rows is active.
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

template <typename DT, bool WREG>
__global__ void __launch_bounds__(kThreads) scan_kernel(ScanArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const ScanLds L = scan_lds(a, (int)sizeof(DT));
  const int tid = threadIdx.x;
  const int gates = a.mode == kGRU ? 3 : 4;

  // Workgroup -> (direction, batch block, hidden slice). Workgroups are dealt
  // to the XCDs round-robin by id, so with gpx > 0 the ids xcd, xcd + nxcd,
  // ... form the groups of one XCD and a group's exchange stays between the
  // CUs of one chiplet (placement only; correctness never depends on it).
  int s, grp;
  if (a.gpx > 0) {
    const int xcd = blockIdx.x % a.nxcd, slot = blockIdx.x / a.nxcd;
    grp = xcd * a.gpx + slot / a.ns;
    s = slot % a.ns;
  } else {
    s = blockIdx.x % a.ns;
    grp = blockIdx.x / a.ns;
  }
  if (grp >= a.D * a.nbb) return;  // padding slots of the XCD-aligned layout
  const int nb = grp % a.nbb;
  const int d = grp / a.nbb;
  const int b0 = nb * a.bb;
  const int j0 = s * a.hs;
  const int hs_act = min(a.hs, a.H - j0);  // may be <= 0 for a trailing slice
  const int p0 = s * a.ps;
  const int ps_act = a.mode == kLSTMP ? min(a.ps, a.P - p0) : 0;
  const bool rev = d == 1;
  const int DK = a.D * a.K;
  const int DG = a.D * a.G;
  unsigned* counter = a.counters + (size_t)grp * 16;
  int* abort_flag = reinterpret_cast<int*>(lds + L.flag);

  const uint32_t hx_bytes = (uint32_t)(2 * a.D * a.B * a.Kp) * sizeof(DT);
  const __amdgpu_buffer_rsrc_t hx_rs = make_rsrc(a.hx, hx_bytes);
  const uint32_t mx_bytes = a.mode == kLSTMP ? (uint32_t)(a.D * a.B * a.Hp) * sizeof(DT) : 16u;
  const __amdgpu_buffer_rsrc_t mx_rs = make_rsrc(a.mode == kLSTMP ? a.mx : a.hx, mx_bytes);
  auto hx_el = [&](int par, int b, int k) -> uint32_t {
    return (uint32_t)(((par * a.D + d) * a.B + b) * a.Kp + k);
  };
  auto mx_el = [&](int b, int j) -> uint32_t { return (uint32_t)((d * a.B + b) * a.Hp + j); };
  // Lengths of the block's rows, staged once: reading them from global
  // memory inside the step loop would make every use wait for all of the
  // wave's outstanding memory operations.
  int* lens = reinterpret_cast<int*>(lds + L.lens);
  for (int r = tid; r < a.bb; r += kThreads)
    lens[r] = b0 + r < a.B ? (a.lengths ? a.lengths[b0 + r] : a.T) : 0;
  if (tid == 0) *abort_flag = 0;
  __syncthreads();
  auto len_of = [&](int b) -> int { return lens[b - b0]; };

  // --- resident weights -----------------------------------------------------
  const DT* whh = reinterpret_cast<const DT*>(a.w_hh[d]);
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
  if (a.mode == kLSTMP) {
    const DT* whr = reinterpret_cast<const DT*>(a.w_hr[d]);
    load_weights<DT>(whr, a.H, a.Hp, L.ncp_wr, [&](int r) -> int {
      return r < ps_act ? p0 + r : -1;
    }, lds, L.wr, L.wr_ld);
  }

  // A group of one workgroup owns every hidden unit of its rows: h_t then
  // never leaves the workgroup and is written straight into the LDS operand
  // tile of the next step (no exchange buffer, no group barrier).
  const bool solo = a.ns == 1 && a.mode != kLSTMP;
  const bool use_mfma = (a.bb % 16) == 0;
  const int tile_rows = use_mfma ? rup(a.bb, 16) : a.bb;
  DT* tile = reinterpret_cast<DT*>(lds + L.as);
  if (solo) {
    const DT* h0s = reinterpret_cast<const DT*>(a.h0[d]);
    for (int e = tid; e < tile_rows * a.Kp; e += kThreads) {
      const int r = e / a.Kp, k = e - r * a.Kp;
      const int b = b0 + r;
      tile[r * L.as_ld + k] = (h0s && b < a.B && k < a.K) ? h0s[(size_t)b * a.K + k] : (DT)0.0f;
    }
  }

  // --- owned state: gate elements e = tid + i * 256 -> (row r, unit u) -------
  const int n_el = a.bb * a.hs;
  float hreg[kMaxEpt], creg[kMaxEpt];
  float bhn[kMaxEpt];
  const DT* h0 = reinterpret_cast<const DT*>(a.h0[d]);
  const DT* c0 = reinterpret_cast<const DT*>(a.c0[d]);
  const DT* bhh = reinterpret_cast<const DT*>(a.b_hh[d]);
  // Owned element i: row er[i] of the block, unit eu[i] of the slice, and the
  // row's length (0 when the element is not owned), computed once.
  int lenreg[kMaxEpt], er[kMaxEpt], eu[kMaxEpt];
#pragma unroll
  for (int i = 0; i < kMaxEpt; ++i) {
    const int e = tid + i * kThreads;
    const int r = e / a.hs, u = e - r * a.hs;
    const int b = b0 + r;
    er[i] = r;
    eu[i] = u;
    hreg[i] = 0.f; creg[i] = 0.f; bhn[i] = 0.f;
    lenreg[i] = (e < n_el && u < hs_act && b < a.B) ? len_of(b) : 0;
    if (e < n_el && u < hs_act && b < a.B) {
      const int j = j0 + u;
      if (a.mode != kLSTMP && h0) hreg[i] = to_f32<DT>(h0[(size_t)b * a.K + j]);
      if (a.mode != kGRU && c0) creg[i] = to_f32<DT>(c0[(size_t)b * a.H + j]);
      if (a.mode == kGRU && a.has_bias) bhn[i] = to_f32<DT>(bhh[2 * a.H + j]);
      if (a.mode != kLSTMP && !solo) {
        coh_store_elem<DT>(hx_rs, hx_el(0, b, j), hreg[i]);
        coh_store_elem<DT>(hx_rs, hx_el(1, b, j), hreg[i]);
      }
    }
  }
  if (a.mode == kLSTMP) {
    // projection owners publish h0 for their outputs
    for (int e = tid; e < a.bb * a.ps; e += kThreads) {
      const int r = e / a.ps, p = e - r * a.ps;
      const int b = b0 + r;
      if (p < ps_act && b < a.B) {
        const float v = h0 ? to_f32<DT>(h0[(size_t)b * a.K + p0 + p]) : 0.f;
        coh_store_elem<DT>(hx_rs, hx_el(0, b, p0 + p), v);
        coh_store_elem<DT>(hx_rs, hx_el(1, b, p0 + p), v);
      }
    }
  }
  if (s == 0 && !solo) {  // zero the padding columns of this block's exchange rows
    for (int e = tid; e < a.bb * (a.Kp - a.K); e += kThreads) {
      const int r = e / (a.Kp - a.K), k = a.K + (e - r * (a.Kp - a.K));
      if (b0 + r < a.B) {
        coh_store_elem<DT>(hx_rs, hx_el(0, b0 + r, k), 0.f);
        coh_store_elem<DT>(hx_rs, hx_el(1, b0 + r, k), 0.f);
      }
    }
    if (a.mode == kLSTMP) {
      for (int e = tid; e < a.bb * (a.Hp - a.H); e += kThreads) {
        const int r = e / (a.Hp - a.H), k = a.H + (e - r * (a.Hp - a.H));
        if (b0 + r < a.B) coh_store_elem<DT>(mx_rs, mx_el(b0 + r, k), 0.f);
      }
    }
  }

  // Longest sequence of this block bounds the steps it takes part in
  // (wave-uniform, so per-step indices stay in scalar registers).
  int maxlen = 0;
  for (int r = 0; r < a.bb && b0 + r < a.B; ++r) maxlen = max(maxlen, len_of(b0 + r));
  maxlen = __builtin_amdgcn_readfirstlane(maxlen);

  float* acc = reinterpret_cast<float*>(lds + L.acc);
  const int mtiles = rup(a.bb, 16) / 16;
  DT* yout = reinterpret_cast<DT*>(a.y);
  DT* hn = reinterpret_cast<DT*>(a.h_n[d]);
  DT* cn = reinterpret_cast<DT*>(a.c_n[d]);

  // Gx of the owned elements for step t (zero for inactive ones).
  float gxv[kMaxEpt][4];
  auto prefetch = [&](int t) {
    const int rowbase = a.packed ? a.offsets[t] : t * a.B;
#pragma unroll
    for (int i = 0; i < kMaxEpt; ++i) {
      const int b = b0 + er[i], u = eu[i];
      const bool act = t < lenreg[i];
#pragma unroll
      for (int q = 0; q < 4; ++q) gxv[i][q] = 0.f;
      if (act) {
        const float* g = a.gx + (size_t)(rowbase + b) * DG + d * a.G + j0 + u;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (q < gates) gxv[i][q] = g[q * a.H];
      }
    }
  };
  // The block takes part in steps t < maxlen: forward t = 0 .. maxlen-1,
  // reverse t = maxlen-1 .. 0 (earlier reverse steps have no active row).
  const int nsteps = maxlen;
  auto t_of = [&](int k) { return rev ? maxlen - 1 - k : k; };

  // h0 is published: arrive, prefetch the first step's Gx, then wait.
  unsigned nbar = 1;
  if (!solo) group_arrive(counter);
  if (nsteps > 0) prefetch(t_of(0));
  if (solo)
    __syncthreads();
  else if (!group_wait(counter, nbar * a.ns, a.status, abort_flag))
    return;
  int par = 0;  // exchange buffer holding h_{t-1}

  for (int k = 0; k < nsteps; ++k) {
    const int t = t_of(k);
    const int rowbase = a.packed ? a.offsets[t] : t * a.B;
    // The previous step's output stores and this step's G_x prefetch were
    // issued before the group barrier, which took longer than they do: an
    // explicit wait here is free, and it leaves no load pending on any
    // register, so the compiler need not wait for every outstanding memory
    // operation before each LDS read and MFMA of the product below.
    if (!solo) wait_all_mem();

    // h_{t-1} of the block -> LDS, then the hidden-hidden product.
    if (!solo) {
      load_tile_coherent<DT>(hx_rs, hx_el(par, b0, 0), a.Kp, b0, a.B, tile_rows, a.Kp, lds, L.as, L.as_ld);
      __syncthreads();
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
        __syncthreads();
        reduce_ksplit(part, a.rks, a.rnt ? tile_rows : a.bb, L.ncw, acc, L.acc_ld);
      }
    } else if (use_mfma) {
      mm_mfma<DT>(lds, L.as, L.as_ld, L.ws, L.ws_ld, acc, L.acc_ld, mtiles, L.ncw / 16, a.Kp);
    } else {
      mm_valu<DT>(lds, L.as, L.as_ld, L.ws, L.ws_ld, acc, L.acc_ld, a.bb, gates * a.hs, a.Kp);
    }
    __syncthreads();

    // Gate math on the owned elements: every element first, then every
    // store. The G_x values were loaded a step ahead, but the vector-memory
    // counter retires in order, so a wait for them placed after a store of
    // this step would also wait for that store to reach the coherence point.
    // Only the exchanged state is stored before the barrier arrival.
    float gsv[kMaxEpt][5];
#pragma unroll
    for (int i = 0; i < kMaxEpt; ++i) {
      const int r = er[i], u = eu[i];
      if (t >= lenreg[i]) continue;
      const float* ar = acc + r * L.acc_ld;
      if (a.mode == kGRU) {
        const float rg = fsigmoid(gxv[i][0] + ar[u]);
        const float zg = fsigmoid(gxv[i][1] + ar[a.hs + u]);
        const float hn_pre = ar[2 * a.hs + u] + bhn[i];
        const float ng = ftanh(gxv[i][2] + rg * hn_pre);
        gsv[i][0] = rg;
        gsv[i][1] = zg;
        gsv[i][2] = ng;
        gsv[i][3] = hn_pre;
        hreg[i] = (1.f - zg) * ng + zg * hreg[i];
      } else {
        const float ig = fsigmoid(gxv[i][0] + ar[u]);
        const float fg = fsigmoid(gxv[i][1] + ar[a.hs + u]);
        const float gg = ftanh(gxv[i][2] + ar[2 * a.hs + u]);
        const float og = fsigmoid(gxv[i][3] + ar[3 * a.hs + u]);
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
    for (int i = 0; i < kMaxEpt; ++i) {
      const int r = er[i], u = eu[i];
      const int b = b0 + r;
      if (t >= lenreg[i]) continue;
      const int j = j0 + u;
      const float h = hreg[i];
      if (solo)
        tile[r * L.as_ld + j] = from_f32<DT>(h);
      else if (a.mode != kLSTMP)
        coh_store_elem<DT>(hx_rs, hx_el(par ^ 1, b, j), h);
      else
        coh_store_elem<DT>(mx_rs, mx_el(b, j), h);
      if (a.rsv) {
        const int nsv = a.mode == kGRU ? 4 : 5;
        float* rv = a.rsv + ((size_t)(rowbase + b) * a.D + d) * (nsv * a.H) + j;
#pragma unroll
        for (int q = 0; q < 5; ++q)
          if (q < nsv) rv[q * a.H] = gsv[i][q];
      }
    }
    ++nbar;
    if (!solo) group_arrive(counter);
    // While the other members arrive: outputs of this step, Gx of the next.
#pragma unroll
    for (int i = 0; i < kMaxEpt; ++i) {
      const int b = b0 + er[i], u = eu[i];
      const int lb = lenreg[i];
      if (t >= lb) continue;
      const bool last = rev ? (t == 0) : (t == lb - 1);
      const int j = j0 + u;
      if (a.mode != kLSTMP) yout[(size_t)(rowbase + b) * DK + d * a.K + j] = from_f32<DT>(hreg[i]);
      if (last && hn && a.mode != kLSTMP) hn[(size_t)b * a.K + j] = from_f32<DT>(hreg[i]);
      if (last && cn && a.mode != kGRU) cn[(size_t)b * a.H + j] = from_f32<DT>(creg[i]);
    }
    if (k + 1 < nsteps) prefetch(t_of(k + 1));
    if (solo)
      __syncthreads();
    else if (!group_wait(counter, nbar * a.ns, a.status, abort_flag))
      return;

    if (a.mode == kLSTMP) {
      wait_all_mem();  // as at the top of the step
      // hidden-projection dense: h_t = m_t W_hr^T for this slice of P
      load_tile_coherent<DT>(mx_rs, mx_el(b0, 0), a.Hp, b0, a.B, use_mfma ? rup(a.bb, 16) : a.bb,
                             a.Hp, lds, L.as, L.as_ld);
      __syncthreads();
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
          __syncthreads();
          reduce_ksplit(part, a.pks, tile_rows, 64 * a.pnt / a.pks, acc, L.acc_ld);
        }
      } else if (use_mfma) {
        mm_mfma<DT>(lds, L.as, L.as_ld, L.wr, L.wr_ld, acc, L.acc_ld, mtiles, rup(a.ps, 16) / 16, a.Hp);
      } else {
        mm_valu<DT>(lds, L.as, L.as_ld, L.wr, L.wr_ld, acc, L.acc_ld, a.bb, a.ps, a.Hp);
      }
      __syncthreads();
      for (int e = tid; e < a.bb * a.ps; e += kThreads) {
        const int r = e / a.ps, p = e - r * a.ps;
        const int b = b0 + r;
        if (p >= ps_act || b >= a.B) continue;
        if (t >= len_of(b)) continue;
        coh_store_elem<DT>(hx_rs, hx_el(par ^ 1, b, p0 + p), clampf(acc[r * L.acc_ld + p], a.p_lo, a.p_hi));
      }
      ++nbar;
      group_arrive(counter);
      // acc stays untouched until the next product, so the outputs are
      // written from it while the other members arrive.
      for (int e = tid; e < a.bb * a.ps; e += kThreads) {
        const int r = e / a.ps, p = e - r * a.ps;
        const int b = b0 + r;
        if (p >= ps_act || b >= a.B) continue;
        const int lb = len_of(b);
        if (t >= lb) continue;
        const bool last = rev ? (t == 0) : (t == lb - 1);
        const DT h = from_f32<DT>(clampf(acc[r * L.acc_ld + p], a.p_lo, a.p_hi));
        yout[(size_t)(rowbase + b) * DK + d * a.K + p0 + p] = h;
        if (last && hn) hn[(size_t)b * a.K + p0 + p] = h;
      }
      if (!group_wait(counter, nbar * a.ns, a.status, abort_flag)) return;
    }
    par ^= 1;
  }
}

}  // namespace

int scan_lds_bytes(const ScanArgs& a, int esize) { return scan_lds(a, esize).total; }

template <typename DT, bool WREG>
hipError_t launch_scan_as(const ScanArgs& a, int lds, dim3 grid, hipStream_t stream) {
  hipError_t e = hipFuncSetAttribute((const void*)scan_kernel<DT, WREG>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((scan_kernel<DT, WREG>), grid, dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_scan(const ScanArgs& a, int dtype_bf16, hipStream_t stream) {
  const int esize = dtype_bf16 ? 2 : 4;
  const int lds = scan_lds(a, esize).total;
  const dim3 grid(a.gpx > 0 ? a.nxcd * a.gpx * a.ns : a.D * a.nbb * a.ns);
  if (dtype_bf16)
    return a.wreg ? launch_scan_as<bf16, true>(a, lds, grid, stream) : launch_scan_as<bf16, false>(a, lds, grid, stream);
  return a.wreg ? launch_scan_as<float, true>(a, lds, grid, stream) : launch_scan_as<float, false>(a, lds, grid, stream);
}

}  // namespace rnnk
