// Kernel 2c: the scan for a few independent sequences (small batch and
// width up to 512), one group of workgroups per (direction, batch row).
//
// With one or a few rows, a step of the recurrence is a matrix-vector
// product W_hh h_{t-1} (4H x H for LSTM, 3H x H for GRU) and a little gate
// math; the apache/tvm PR "[TOPI] TE implementation of LSTM using scan"
// benchmarks exactly this shape (T = 80, B = 1, H = 256) and finds the
// per-step overhead dominant. The tiled scan spends most of such a step in
// workgroup barriers, LDS round trips and a K-split reduction. Here:
//   * a wave owns UW hidden units: all their gate rows, spread over its four
//     16-lane DPP rows (RG rows each), every lane holding its rows' W_hh
//     over its share of K in registers (chunks li + 16 j of 4 elements);
//   * each lane reads its own chunks of h_{t-1} straight from the exchange
//     ring (no LDS, no workgroup barrier anywhere in the step loop), sums
//     over its 16-lane row with DPP rotations, and reads the row sums of
//     the four DPP rows with readlane, so every lane has the gate
//     pre-activations of the wave's units;
//   * the gate math runs once per unit (uniform values), and lane v < UW
//     publishes unit v's h_t to the ring slot t mod 4 and to y.
// The ring protocol is the tiled scan's: write-once slots holding an
// all-ones sentinel until written, NaN published as the canonical quiet NaN,
// a member resetting its own entries of slot t - 2 once it has read all of
// slot t - 1, plain stores when the group's members share one XCD (their
// device-scope loads then find the values in that XCD's L2).
// Gate conventions, the bias fold (G_x holds b_ih + b_hh except GRU's b_hn),
// variable lengths, packed rows, the reverse direction and cell clipping are
// those of the tiled scan.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"
#include "scan_common.hpp"

namespace rnnk {

namespace {

constexpr int kSmThreads = 512;  // eight waves per member
constexpr int kSmWaves = kSmThreads / 64;

// every lane of a 16-lane DPP row gets the row's sum (rotations by 8, 4, 2, 1)
__device__ __forceinline__ float row_sum16(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x122, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x121, 0xF, 0xF, false));
  return v;
}

__device__ __forceinline__ float lane_val(float v, int src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), src));
}

// UW units per wave, JC chunks of K per lane (K <= 64 JC).
template <typename DT, bool GRU, int UW, int JC>
__global__ void __launch_bounds__(kSmThreads) scan_small_kernel(ScanArgs a) {
  constexpr int gates = GRU ? 3 : 4;
  constexpr int R = gates * UW;        // gate rows of a wave
  constexpr int RG = (R + 3) / 4;      // rows per 16-lane DPP row
  __shared__ int xcd_ok, xcd_same;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 15, grp = lane >> 4;
  const int M = a.ns;                  // members per group
  // group and member: with gpx > 0 the ids xcd, xcd + nxcd, ... are one
  // XCD's workgroups, holding gpx whole groups
  int g, m;
  if (a.gpx > 0) {
    const int xcd = blockIdx.x % a.nxcd, slot_id = blockIdx.x / a.nxcd;
    g = xcd * a.gpx + slot_id / M;
    m = slot_id % M;
  } else {
    g = blockIdx.x / M;
    m = blockIdx.x % M;
  }
  if (a.zero_status && blockIdx.x == 0 && threadIdx.x == 0) *a.status = 0;
  if (g >= a.D * a.B) return;
  const int d = g / a.B, b = g - d * a.B;
  const int H = a.H, K = a.K, G = a.G;
  const int DG = a.D * G, DK = a.D * K;
  const bool rev = d == 1;
  const int n = a.lengths ? a.lengths[b] : a.T[0];

  // members on one XCD: plain ring stores (decided before the first one)
  publish_xcd(a.xid[0] + g * M, M, m);
  const bool local = group_on_one_xcd(a.xid[0] + g * M, M, &xcd_ok, &xcd_same);
  if (!xcd_ok) {
    if (threadIdx.x == 0) __hip_atomic_store(a.status, kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }

  // this wave's units and gate rows: row rho = q * UW + v (gate q of unit
  // u0 + v) sits on DPP row rho / RG, slot rho % RG
  const int u0 = (m * kSmWaves + wave) * UW;
  const DT* whh = reinterpret_cast<const DT*>(a.w_hh[d]);
  float w[RG][JC][4];
#pragma unroll
  for (int s = 0; s < RG; ++s) {
    const int rho = grp * RG + s, q = rho / UW, v = rho - q * UW;
    const bool ok = rho < R && u0 + v < H;
    const size_t row = (size_t)(q * H + u0 + v) * K;
#pragma unroll
    for (int j = 0; j < JC; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k = 4 * (li + 16 * j) + e;
        w[s][j][e] = (ok && k < K) ? to_f32<DT>(whh[row + k]) : 0.f;
      }
  }
  // per unit (uniform): GRU b_hn; the state h (and c)
  float bhn[UW], h[UW], c[UW];
  const DT* h0 = reinterpret_cast<const DT*>(a.h0[d]);
  const DT* c0 = reinterpret_cast<const DT*>(a.c0[d]);
#pragma unroll
  for (int v = 0; v < UW; ++v) {
    const int u = u0 + v;
    bhn[v] = (GRU && a.has_bias && u < H) ? to_f32<DT>(reinterpret_cast<const DT*>(a.b_hh[d])[2 * H + u]) : 0.f;
    h[v] = (u < H && h0) ? to_f32<DT>(h0[(size_t)b * K + u]) : 0.f;
    c[v] = (!GRU && u < H && c0) ? to_f32<DT>(c0[(size_t)b * H + u]) : 0.f;
  }
  // h_{t-1} chunks of this lane (valid elements: k < K), from h0 for step 0
  float hv[JC][4];
#pragma unroll
  for (int j = 0; j < JC; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k = 4 * (li + 16 * j) + e;
      hv[j][e] = (k < K && h0) ? to_f32<DT>(h0[(size_t)b * K + k]) : 0.f;
    }

  const int Kq = a.Kp;  // ring row stride (floats, >= 64 JC)
  const uint32_t slot_el = (uint32_t)(a.D * a.B) * (uint32_t)Kq;
  const __amdgpu_buffer_rsrc_t ring = make_rsrc(a.hx[0], slot_el * (uint32_t)kScanRingSlots * 4u);
  auto ring_el = [&](int k, int col) -> uint32_t {
    return (uint32_t)(k & (kScanRingSlots - 1)) * slot_el + (uint32_t)g * (uint32_t)Kq + (uint32_t)col;
  };
  const int* offs = a.offsets;
  auto row_of = [&](int t) -> int { return a.packed ? offs[t] : t * a.B; };
  auto t_of = [&](int k) { return rev ? n - 1 - k : k; };
  const float* gx = reinterpret_cast<const float*>(a.gx[0]);
  const __amdgpu_buffer_rsrc_t ys = make_rsrc(reinterpret_cast<DT*>(a.y[0]) + d * K, 0x7FFFFFFFu);
  const float c_lo = a.c_lo, c_hi = a.c_hi;
  // the weights and initial state feed the loop through registers
  wait_all_mem();

  for (int k = 0; k < n; ++k) {
    const int t = t_of(k);
    // G_x of the wave's rows (uniform loads)
    const float* gxr = gx + (size_t)(row_of(t) + b) * DG + d * G;
    float gxv[gates][UW];
#pragma unroll
    for (int q = 0; q < gates; ++q)
#pragma unroll
      for (int v = 0; v < UW; ++v) gxv[q][v] = u0 + v < H ? gxr[q * H + u0 + v] : 0.f;
    if (k > 0) {
      // h_{t-1}: this lane's chunks of ring slot k - 1, polled until no
      // valid element holds the sentinel
      // (each poll also moves its values into hv: extracting them after the
      // loop from the last poll's registers measured wrong, every element
      // of a chunk taking the first one's value)
      uint64_t t0 = 0;
      unsigned polls = 0;
      // a poll that finds a sentinel costs a whole round trip more: a short
      // wait first (~400 cycles) measured 124 -> 121 us on the B=1 scan (a
      // longer one, 130)
      __builtin_amdgcn_s_sleep(6);
      while (true) {
        u32x4 raw[JC];
#pragma unroll
        for (int j = 0; j < JC; ++j) raw[j] = coh_poll16(ring, ring_el(k - 1, 4 * (li + 16 * j)) * 4u);
        bool pend = false;
#pragma unroll
        for (int j = 0; j < JC; ++j) {
          const f32x4 rv = __builtin_bit_cast(f32x4, raw[j]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool valid = 4 * (li + 16 * j) + e < K;
            pend = pend || (valid && raw[j][e] == 0xFFFFFFFFu);
            hv[j][e] = valid ? rv[e] : 0.f;
          }
        }
        if (!__builtin_amdgcn_ballot_w64(pend)) break;
        if ((++polls & 63u) == 0) {  // watchdog: ~2 s, or another member's error
          const uint64_t now = __builtin_amdgcn_s_memrealtime();
          if (t0 == 0) t0 = now;
          const int st = __hip_atomic_load(a.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (st != kStatusOk || now - t0 > kWatchdogTicks) {
            __hip_atomic_store(a.status, kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
          }
        }
      }
      // every member has published step k - 1, so every member is done
      // with slot k - 2: put this wave's entries of it back to the sentinel
      if (k >= 2 && lane < UW && u0 + lane < H) ring_reset<float>(ring, ring_el(k - 2, u0 + lane), local);
    }
    // the wave's gate rows over this lane's share of K, summed over its
    // 16-lane row; then every lane reads the rows' sums
    float acc[RG];
#pragma unroll
    for (int s = 0; s < RG; ++s) {
      float p0 = 0.f, p1 = 0.f;
#pragma unroll
      for (int j = 0; j < JC; ++j) {
        p0 = fmaf(w[s][j][0], hv[j][0], p0);
        p1 = fmaf(w[s][j][1], hv[j][1], p1);
        p0 = fmaf(w[s][j][2], hv[j][2], p0);
        p1 = fmaf(w[s][j][3], hv[j][3], p1);
      }
      acc[s] = row_sum16(p0 + p1);
    }
    float pre[gates][UW];
#pragma unroll
    for (int q = 0; q < gates; ++q)
#pragma unroll
      for (int v = 0; v < UW; ++v) {
        const int rho = q * UW + v;
        pre[q][v] = lane_val(acc[rho % RG], 16 * (rho / RG));
      }
    // gate math per unit (uniform), then lane v publishes unit v
    float hout = 0.f;
#pragma unroll
    for (int v = 0; v < UW; ++v) {
      if constexpr (GRU) {
        const float r = fsigmoid(gxv[0][v] + pre[0][v]);
        const float z = fsigmoid(gxv[1][v] + pre[1][v]);
        const float nn = ftanh(gxv[2][v] + r * (pre[2][v] + bhn[v]));
        h[v] = (1.f - z) * nn + z * h[v];
      } else {
        const float ig = fsigmoid(gxv[0][v] + pre[0][v]);
        const float fg = fsigmoid(gxv[1][v] + pre[1][v]);
        const float gg = ftanh(gxv[2][v] + pre[2][v]);
        const float og = fsigmoid(gxv[3][v] + pre[3][v]);
        c[v] = clampf(fg * c[v] + ig * gg, c_lo, c_hi);
        h[v] = og * ftanh(c[v]);
      }
      hout = lane == v ? h[v] : hout;
    }
    if (lane < UW && u0 + lane < H) {
      ring_store<float>(ring, ring_el(k, u0 + lane), hout, local);
      out_store<DT>(ys, (uint32_t)((row_of(t) + b) * DK + u0 + lane) * (uint32_t)sizeof(DT), hout);
    }
  }
  DT* hn = reinterpret_cast<DT*>(a.h_n[d]);
  DT* cn = reinterpret_cast<DT*>(a.c_n[d]);
#pragma unroll
  for (int v = 0; v < UW; ++v) {
    if (lane == v && u0 + v < H) {
      if (hn) hn[(size_t)b * K + u0 + v] = from_f32<DT>(h[v]);
      if (!GRU && cn) cn[(size_t)b * H + u0 + v] = from_f32<DT>(c[v]);
    }
  }
}

template <typename DT, bool GRU, int UW, int JC>
hipError_t launch_small_as(const ScanArgs& a, hipStream_t stream) {
  const int groups = a.D * a.B;
  const int grid = a.gpx > 0 ? a.nxcd * a.gpx * a.ns : groups * a.ns;
  launch_kernel((scan_small_kernel<DT, GRU, UW, JC>), dim3(grid), dim3(kSmThreads), 0, stream, a);
  return hipGetLastError();
}

template <typename DT, bool GRU, int UW>
hipError_t launch_small_jc(const ScanArgs& a, hipStream_t stream) {
  switch (scan_small_chunks(a.K)) {
    case 1: return launch_small_as<DT, GRU, UW, 1>(a, stream);
    case 2: return launch_small_as<DT, GRU, UW, 2>(a, stream);
    case 4: return launch_small_as<DT, GRU, UW, 4>(a, stream);
    case 8: return launch_small_as<DT, GRU, UW, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename DT, bool GRU>
hipError_t launch_small_uw(const ScanArgs& a, hipStream_t stream) {
  switch (a.hs) {
    case 1 * kSmWaves: return launch_small_jc<DT, GRU, 1>(a, stream);
    case 2 * kSmWaves: return launch_small_jc<DT, GRU, 2>(a, stream);
    case 4 * kSmWaves: return launch_small_jc<DT, GRU, 4>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int scan_small_chunks(int K) {
  const int j = (K + 63) / 64;
  return j <= 1 ? 1 : j <= 2 ? 2 : j <= 4 ? 4 : j <= 8 ? 8 : 0;
}

int scan_small_units_per_wg(int units_per_wave) { return units_per_wave * kSmWaves; }

hipError_t launch_scan_small(const ScanArgs& a, int dtype_bf16, hipStream_t stream) {
  if (a.mode != kLSTM && a.mode != kGRU) return hipErrorInvalidValue;
  const bool gru = a.mode == kGRU;
  if (dtype_bf16) return gru ? launch_small_uw<bf16, true>(a, stream) : launch_small_uw<bf16, false>(a, stream);
  return gru ? launch_small_uw<float, true>(a, stream) : launch_small_uw<float, false>(a, stream);
}

}  // namespace rnnk
