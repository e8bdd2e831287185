// Kernel 3b: the RSSM prior unrolled over given actions, with wide members
// whose GRU weights live in registers.
//
// Same step as kernel 3 (pytorch/rl issue "[Feature Request] CUDNN version
// of RSSM", Solution: RSSMPrior.forward inside the first unroll loop):
//   e_t = ELU(W_as [s_{t-1}; a_t] + b_as);  h_t = GRUCell(e_t, h_{t-1});
//   u_t = ELU(W_1 h_t + b_1);  v_t = W_2 u_t + b_2;
//   mean = v[:S];  std = softplus(v[S:]) + scale_lb;  s_t = mean + eps_t * std.
//
// What differs from kernel 3 is the cost of the per-step exchange, which
// dominates a step:
//   * Fewer, wider members (a handful of workgroups per group instead of
//     ten or more). Every member reads the whole h_t and every member's
//     partial sums of W_1 h_t each step, so the bytes crossing between
//     compute units grow with the square of the member count; wide members
//     cut them several-fold. A member's slice of W_ih and W_hh (all three
//     gates of its units) is held in registers (the 4x4x1 MFMA B operand,
//     one output column per lane, K split over the waves); W_1's columns for
//     the slice, W_2 and W_as stay in LDS.
//   * No counter barrier. The exchange buffers are rings of write-once
//     slots: step t's values go to slot t mod 4, which holds a sentinel bit
//     pattern until its writer stores the value, and readers poll their
//     chunks until no sentinel is left. A member resets its own entries of
//     slot t - 1 once it has read every member's step-t values (by then all
//     members have finished reading slot t - 1); it writes that slot again
//     only at step t + 3, after two more exchanges whose waits retire the
//     reset stores first. A published value that is NaN is stored as the
//     canonical quiet NaN, so no result equals the sentinel.
//   * The members of a group share one XCD (workgroups are dealt to the
//     XCDs round-robin by id, so ids equal modulo the XCD count land on one
//     XCD), so plain stores, which land in that XCD's L2, are visible to the
//     other members' device-scope loads: the exchange never leaves the
//     chiplet. At start the members of a group compare their hardware XCC
//     ids through device-scope stores; a group that is split over XCDs
//     reports a device status error instead of computing.
//
// With an actor in the loop (the issue's second unroll; the actor is the
// MLP a = tanh(W_a2 ELU(W_a1 [s; h] + b_a1) + b_a2)), the action of step
// t + 1 comes from s_t and h_t at the end of step t, as in kernel 3: the
// belief part W_a1[:, S:] h_t is split over the members like W_1 and rides
// the same exchange (more partial-sum columns per row); the state part, the
// ELU, W_a2 and the tanh are small products every member does whole.
#include "device_common.hpp"
#include "kernels.hpp"
#include "rssm_common.hpp"

namespace rnnk {

namespace {

using namespace rssmk;

constexpr int kRing = 4;
constexpr uint32_t kSentinel = 0xFFFFFFFFu;
constexpr int kMaxMembers2 = 8;  // members per group (their partials are read in one batch)

__device__ __forceinline__ uint32_t publish_bits(float v) {
  return v == v ? __builtin_bit_cast(uint32_t, v) : 0x7FC00000u;
}
__device__ __forceinline__ void pub_store(__amdgpu_buffer_rsrc_t rs, uint32_t elem, uint32_t bits) {
  __builtin_amdgcn_raw_buffer_store_b32(bits, rs, (int)(elem * 4u), 0, 0);
}
__device__ __forceinline__ bool has_sentinel(const u32x4& v, int valid) {
  bool s = false;
#pragma unroll
  for (int k = 0; k < 4; ++k) s = s || (k < valid && v[k] == kSentinel);
  return s;
}

// Register layout of a GRU slice product (N = 3 * hp <= 128 output columns,
// K over 16-byte chunks): wave w takes column pass w & 1 (columns
// 64 * (w & 1) + lane) over K quarter w >> 1, chunks [q * QC, q * QC + QC)
// of the K4 chunks; lane holds row `row` of W (or zeros).
template <int NQ>
__device__ __forceinline__ void load_slice_reg(f32x4 (&wr)[NQ], const float* W, int row, int K, int k0, int n) {
  // whole 16-byte chunks when every row starts 16-byte aligned (a quarter
  // of the load instructions of element-wise reads, which are bound by the
  // cache-line requests of 64 lanes on 64 rows)
  const bool vec = (K & 3) == 0 && (reinterpret_cast<uintptr_t>(W) & 15) == 0;
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    if (vec) {
      wr[i] = (row >= 0 && i < n) ? *reinterpret_cast<const f32x4*>(W + (size_t)row * K + 4 * (k0 + i))
                                  : f32x4{0.f, 0.f, 0.f, 0.f};
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k = 4 * (k0 + i) + e;
        wr[i][e] = (row >= 0 && i < n && k < K) ? W[(size_t)row * K + k] : 0.f;
      }
    }
  }
}

// acc = sum over the wave's NQ chunks from k0 of X chunk (LDS row of the
// lane's batch row) times the resident chunks. Every chunk is multiplied,
// with no bound checks: chunks past the wave's share hold zero weights, and
// the X rows are padded with zeros far enough (row stride >= 16 NQ floats)
// that a read past the row's data stays inside its own zero padding. Two
// interleaved accumulator chains, summed at the end (a fixed order).
template <int NQ>
__device__ __forceinline__ f32x4 reg_product(const float* xr, const f32x4 (&wr)[NQ], int k0) {
  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
  const float* xp = xr + 4 * k0;
  f32x4 x[NQ];
#pragma unroll
  for (int i = 0; i < NQ; ++i) x[i] = *reinterpret_cast<const f32x4*>(xp + 4 * i);
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    a0 = __builtin_amdgcn_mfma_f32_4x4x1f32(x[i][0], wr[i][0], a0, 0, 0, 0);
    a1 = __builtin_amdgcn_mfma_f32_4x4x1f32(x[i][1], wr[i][1], a1, 0, 0, 0);
    a0 = __builtin_amdgcn_mfma_f32_4x4x1f32(x[i][2], wr[i][2], a0, 0, 0, 0);
    a1 = __builtin_amdgcn_mfma_f32_4x4x1f32(x[i][3], wr[i][3], a1, 0, 0, 0);
  }
  return a0 + a1;
}

// Register chunks per lane of a GRU slice product for K = E or Hb.
__host__ __device__ inline int rssm_reg_nq(const RssmArgs& a) {
  const int e4 = (a.E + 3) / 4, h4 = (a.Hb + 3) / 4;
  const int q = ((e4 > h4 ? e4 : h4) + 3) / 4;
  return q <= 4 ? 4 : (q <= 8 ? 8 : (q <= 13 ? 13 : (q <= 16 ? 16 : 0)));
}

// Row stride of an LDS operand read by reg_product: at least 16 NQ floats
// (the farthest chunk a wave reads), an odd number of 16-byte chunks.
__host__ __device__ inline int ld_reg_rows(int x, int nq) {
  const int m = x > 16 * nq ? x : 16 * nq;
  return ld_rows(m);
}

// Steps of noise and actions staged in LDS at a time: the step loop then
// issues no global loads besides the exchange polls (a pending load whose
// destination registers get reused makes the compiler wait for every
// outstanding memory operation, stores included).
constexpr int kStage = 32;
// With the actor only the noise is staged, for fewer steps at a time (its
// weights take the LDS).
constexpr int kStageActor = 16;

// e[v][c] = ELU(sum_k X[v][k] W[c][k] + bias[c]) for c < N (N <= 64 kWaves
// columns, one 64-column pass per wave, K <= 64): no K split, so no
// reduction or extra barrier; the column's bias is read once.
__device__ __forceinline__ void elu_pass_product(const float* X, int ldx, const float* W, int ldw, const float* bias,
                                                 float* out, int ldo, int N, int K) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int npass = (N + 63) >> 6;
  const int K4 = (K + 3) >> 2;
  for (int p = __builtin_amdgcn_readfirstlane(wave); p < npass; p += kWaves) {
    const int c = p * 64 + lane, cc = c < N ? c : N - 1;
    const float bc = bias[cc];
    const f32x4 acc = dot_batch<16>(X + (lane & 3) * ldx, W + cc * ldw, 0, K4, f32x4{0.f, 0.f, 0.f, 0.f});
    if (c < N) {
#pragma unroll
      for (int v = 0; v < 4; ++v) out[v * ldo + c] = felu(acc[v] + bc);
    }
  }
}

// out[v][c] = ELU(sum_k X[v][k] W[c][k] + add[v][c] + bias[c]), as
// elu_pass_product with a per-element term (the actor's belief part).
__device__ __forceinline__ void elu_pass_product_add(const float* X, int ldx, const float* W, int ldw,
                                                     const float* bias, const float* add, int lda, float* out,
                                                     int ldo, int N, int K) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int npass = (N + 63) >> 6;
  const int K4 = (K + 3) >> 2;
  for (int p = __builtin_amdgcn_readfirstlane(wave); p < npass; p += kWaves) {
    const int c = p * 64 + lane, cc = c < N ? c : N - 1;
    const float bc = bias[cc];
    const f32x4 acc = dot_batch<16>(X + (lane & 3) * ldx, W + cc * ldw, 0, K4, f32x4{0.f, 0.f, 0.f, 0.f});
    if (c < N) {
#pragma unroll
      for (int v = 0; v < 4; ++v) out[v * ldo + c] = felu(acc[v] + add[v * lda + c] + bc);
    }
  }
}

struct Rssm2Lds {
  // float offsets (multiples of 4)
  int was, bas, b1, b2, w2, w1s;
  int wa1s, ba1, wa2, ba2, q, qa;  // actor (empty without one)
  int sa, e, h, hs, u, gh, redg, redv, stg, flag, total;
  int ld_sa, ld_e, ld_h, ld_hs, ld_stg, ld_s, ld_q;
};

// (Ea is passed apart so that the kernel without the actor sees a constant
// zero: its offsets then fold as they would with no actor fields at all.)
__host__ __device__ inline Rssm2Lds rssm2_lds(const RssmArgs& a, int Ea) {
  Rssm2Lds L;
  const int SA = a.S + a.A;
  const int nq = rssm_reg_nq(a);
  L.ld_sa = ld_rows(SA);
  L.ld_e = ld_reg_rows(a.E, nq);
  L.ld_h = ld_reg_rows(a.Hb, nq);
  L.ld_hs = ld_rows(a.h_per);
  L.ld_s = ld_rows(a.S);
  L.ld_q = ld_rows(Ea);
  const int R = kMaxRows;
  int o = 0;
  auto take = [&](int n) { const int at = o; o += r4(n); return at; };
  L.was = take(a.E * L.ld_sa);
  L.bas = take(a.E);
  L.b1 = take(a.E);
  L.b2 = take(2 * a.S);
  L.w2 = take(2 * a.S * L.ld_e);
  L.w1s = take((a.E + Ea) * L.ld_hs);  // W_1 columns, then W_a1 belief columns
  L.wa1s = take(Ea * L.ld_s);
  L.ba1 = take(Ea);
  L.wa2 = take(Ea > 0 ? a.A * L.ld_q : 0);
  L.ba2 = take(Ea > 0 ? a.A : 0);
  L.q = take(Ea > 0 ? R * L.ld_q : 0);
  L.qa = take(Ea > 0 ? R * L.ld_q : 0);
  L.sa = take(R * L.ld_sa);
  L.e = take(R * L.ld_e);
  L.h = take(R * L.ld_h);
  L.hs = take(R * L.ld_hs);
  L.u = take(R * L.ld_e);
  L.gh = take(R * 128);
  L.redg = take(4 * 4 * 128);        // 4 K quarters x 4 rows x 128 columns
  L.redv = take(kWaves * 4 * 64);    // W_2 (and W_a2): 8 K parts x 4 rows x 64 columns
  // per (row, step): eps (S), then (no actor) the next action (A). Without
  // the actor the buffer sits 8 KiB further on and is sized for four rows:
  // that placement measured 1.8% faster steps than the packed one.
  L.ld_stg = Ea > 0 ? a.S : SA;
  if (Ea == 0) take(kWaves * 4 * 64);
  L.stg = take((Ea > 0 ? (a.rows > 0 ? a.rows : 1) : R) * (Ea > 0 ? kStageActor : kStage) * L.ld_stg);
  L.flag = take(4);
  L.total = o * 4;
  return L;
}

template <int NQ, bool ACTOR>
__global__ void __launch_bounds__(kThreads) rssm_reg_kernel(RssmArgs a) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  const Rssm2Lds L = rssm2_lds(a, ACTOR ? a.Ea : 0);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  // group and member: the ids xcd, xcd + nxcd, ... are the workgroups of one
  // XCD, which hold gpx whole groups of nw members
  const int xcd = blockIdx.x % a.nxcd, slot_id = blockIdx.x / a.nxcd;
  const int g = xcd * a.gpx + slot_id / a.nw;
  const int w = slot_id % a.nw;
  if (g >= a.ngroups) return;  // padding slots of the last XCDs
  int* abort_flag = reinterpret_cast<int*>(sm + L.flag);
  if (tid == 0) {
    *abort_flag = 0;
    if (a.nxcd > 1) {
      // Every member publishes its hardware XCC id with a device-scope store
      // and reads the others' (bounded wait): the plain-store exchange below
      // is only valid when they all match.
      unsigned hw;
      asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(hw));
      hw &= 0xFu;
      const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.xid, (uint32_t)(a.ngroups * a.nw) * 4u);
      coh_store4(xr, (uint32_t)(g * a.nw + w) * 4u, hw);
      uint64_t t0 = 0;
      for (int m = 0; m < a.nw && !*abort_flag; ++m) {
        unsigned polls = 0, id;
        while ((id = coh_poll4(xr, (uint32_t)(g * a.nw + m) * 4u)) == kSentinel) {
          if ((++polls & 63u) == 0) {
            const uint64_t now = __builtin_amdgcn_s_memrealtime();
            if (t0 == 0) t0 = now;
            if (now - t0 > kWatchdogTicks) break;
          }
        }
        if (id != hw) {
          __hip_atomic_store(a.status, kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          *abort_flag = 1;
        }
      }
    }
  }
  __syncthreads();
  if (*abort_flag) return;

  const int b0 = g * a.rows;
  const int nrows = min(a.rows, a.B - b0);
  const int S = a.S, A = a.A, E = a.E, Hb = a.Hb, SA = a.S + a.A;
  const int Ea = ACTOR ? a.Ea : 0;
  const int SH = S + Hb;   // W_a1 row length
  const int ea0 = r4(E);   // first actor column of an exchange row
  const int N1 = E + Ea;   // columns of the per-member partial product
  const int hp = a.h_per;
  const int j0 = w * hp, hn = max(0, min(hp, Hb - j0));
  const int nw = a.nw;
  const uint32_t hring = (uint32_t)a.B * a.Hbp;            // floats per h slot
  const uint32_t pring = (uint32_t)a.B * nw * a.Ep;        // floats per partial slot
  const __amdgpu_buffer_rsrc_t hx_rs = make_rsrc(a.ex_h, hring * kRing * 4u);
  const __amdgpu_buffer_rsrc_t px_rs = make_rsrc(a.ex_p, pring * kRing * 4u);
  auto hx_el = [&](int s, int b, int j) -> uint32_t { return (uint32_t)s * hring + (uint32_t)(b * a.Hbp + j); };
  auto px_el = [&](int s, int b, int m, int k) -> uint32_t {
    return (uint32_t)s * pring + (uint32_t)((b * nw + m) * a.Ep + k);
  };

  // --- LDS: zero (padding rows and columns read as zero), then resident data
  for (int i = tid; i < L.total / 4; i += kThreads) sm[i] = 0.f;
  __syncthreads();
  // (batched row copies measured 1% faster unrolls without the actor and
  // 2% slower with it, whose step loop then spills more SGPRs)
  if constexpr (!ACTOR) {
    stage_rows(sm + L.was, L.ld_sa, a.w_as, SA, E, SA);
  } else {
    for (int i = tid; i < E * SA; i += kThreads) {
      const int r = i / SA, c = i - r * SA;
      sm[L.was + r * L.ld_sa + c] = a.w_as[i];
    }
  }
  for (int i = tid; i < E; i += kThreads) {
    sm[L.bas + i] = a.b_as[i];
    sm[L.b1 + i] = a.b_1[i];
  }
  for (int i = tid; i < 2 * S; i += kThreads) sm[L.b2 + i] = a.b_2[i];
  // W_2, and W_1's columns of the slice: w1s[k][jj] = W_1[k][j0 + jj]
  if constexpr (!ACTOR) {
    stage_rows(sm + L.w2, L.ld_e, a.w_2, E, 2 * S, E);
    stage_rows(sm + L.w1s, L.ld_hs, a.w_1 + j0, Hb, E, hn);
  } else {
    for (int i = tid; i < 2 * S * E; i += kThreads) {
      const int r = i / E, c = i - r * E;
      sm[L.w2 + r * L.ld_e + c] = a.w_2[i];
    }
    for (int i = tid; i < E * hp; i += kThreads) {
      const int k = i / hp, jj = i - k * hp;
      if (jj < hn) sm[L.w1s + k * L.ld_hs + jj] = a.w_1[(size_t)k * Hb + j0 + jj];
    }
  }
  if constexpr (ACTOR) {
    // belief columns of W_a1 for the slice (rows E .. E + Ea - 1 of w1s),
    // its state columns whole, W_a2 whole, and both biases
    for (int i = tid; i < Ea * hp; i += kThreads) {
      const int k = i / hp, jj = i - k * hp;
      if (jj < hn) sm[L.w1s + (E + k) * L.ld_hs + jj] = a.w_a1[(size_t)k * SH + S + j0 + jj];
    }
    for (int i = tid; i < Ea * S; i += kThreads) {
      const int r = i / S, c = i - r * S;
      sm[L.wa1s + r * L.ld_s + c] = a.w_a1[(size_t)r * SH + c];
    }
    for (int i = tid; i < A * Ea; i += kThreads) {
      const int r = i / Ea, c = i - r * Ea;
      sm[L.wa2 + r * L.ld_q + c] = a.w_a2[i];
    }
    for (int i = tid; i < Ea; i += kThreads) sm[L.ba1 + i] = a.b_a1[i];
    for (int i = tid; i < A; i += kThreads) sm[L.ba2 + i] = a.b_a2[i];
  }

  // --- registers: the slice of W_ih and W_hh (column c = 64 * pass + lane is
  // slice row c: gate c / hp, unit c % hp); W_2 (column = lane) is read from
  // LDS over this wave's eighth of K
  const int pass = wave & 1, quarter = wave >> 1;
  const int E4 = (E + 3) / 4, H4 = (Hb + 3) / 4;
  const int qe = (E4 + 3) / 4, qh = (H4 + 3) / 4;
  const int ke0 = min(E4, quarter * qe), ne = min(E4, ke0 + qe) - ke0;
  const int kh0 = min(H4, quarter * qh), nh = min(H4, kh0 + qh) - kh0;
  const int q2 = (E4 + kWaves - 1) / kWaves;
  const int k20 = min(E4, wave * q2), n2 = min(E4, k20 + q2) - k20;
  const int col = pass * 64 + lane;
  const int gq = col / hp, gu = col - gq * hp;
  const int grow = (col < 3 * hp && gu < hn) ? gq * Hb + j0 + gu : -1;
  f32x4 wih[NQ], whh[NQ];
  load_slice_reg<NQ>(wih, a.w_ih, grow, E, ke0, ne);
  load_slice_reg<NQ>(whh, a.w_hh, grow, Hb, kh0, nh);
  // The resident registers must not count as pending loads inside the step
  // loop: otherwise the compiler waits for every outstanding memory
  // operation (output and exchange stores included) before each product.
  wait_all_mem();
  const float* w2row = sm + L.w2 + (lane < 2 * S ? lane : 2 * S - 1) * L.ld_e;

  // --- initial state: [s_0; a_0], whole h_0, the owned units' h ------------
  for (int i = tid; i < nrows * SA; i += kThreads) {
    const int r = i / SA, c = i - r * SA;
    const int b = b0 + r;
    // (the actor's a_0 is computed below)
    sm[L.sa + r * L.ld_sa + c] = c < S    ? (a.s0 ? a.s0[(size_t)b * S + c] : 0.f)
                                 : ACTOR ? 0.f
                                         : a.actions[((size_t)b * a.T + 0) * A + (c - S)];
  }
  for (int i = tid; i < nrows * Hb; i += kThreads) {
    const int r = i / Hb, c = i - r * Hb;
    sm[L.h + r * L.ld_h + c] = a.h0 ? a.h0[(size_t)(b0 + r) * Hb + c] : 0.f;
  }
  const int own_r = tid / max(hp, 1), own_j = tid - own_r * hp;
  const bool owner = tid < a.rows * hp && own_r < nrows && own_j < hn;
  float hreg = (owner && a.h0) ? a.h0[(size_t)(b0 + own_r) * Hb + j0 + own_j] : 0.f;
  float bias_r = 0.f, bias_z = 0.f, bias_nx = 0.f, bias_nh = 0.f;
  if (owner) {
    bias_r = a.b_ih[j0 + own_j] + a.b_hh[j0 + own_j];
    bias_z = a.b_ih[Hb + j0 + own_j] + a.b_hh[Hb + j0 + own_j];
    bias_nx = a.b_ih[2 * Hb + j0 + own_j];
    bias_nh = a.b_hh[2 * Hb + j0 + own_j];
  }
  const int tr = tid / S, tc = tid - tr * S;
  const bool tail_owner = tid < nrows * S;
  const int ar = tid / A, ac = tid - ar * A;
  const bool act_owner = tid < nrows * A;
  float* redg = sm + L.redg;
  float* redv = sm + L.redv;
  float* gh = sm + L.gh;
  const int ng = 3 * hp;  // slice product columns
  __syncthreads();
  if constexpr (ACTOR) {
    // a_0 = actor(s_0, h_0), once, straight from global W_a1 and from W_a2
    for (int i = tid; i < nrows * Ea; i += kThreads) {
      const int r = i / Ea, c = i - r * Ea;
      const float* wr = a.w_a1 + (size_t)c * SH;
      float acc = 0.f;
      for (int k = 0; k < S; ++k) acc += wr[k] * sm[L.sa + r * L.ld_sa + k];
      for (int k = 0; k < Hb; ++k) acc += wr[S + k] * sm[L.h + r * L.ld_h + k];
      sm[L.q + r * L.ld_q + c] = felu(acc + sm[L.ba1 + c]);
    }
    __syncthreads();
    if (act_owner) {
      float acc = 0.f;
      for (int k = 0; k < Ea; ++k) acc += sm[L.wa2 + ac * L.ld_q + k] * sm[L.q + ar * L.ld_q + k];
      const float act = ftanh(acc + sm[L.ba2 + ac]);
      sm[L.sa + ar * L.ld_sa + S + ac] = act;
      if (w == 0 && a.act_out) a.act_out[((size_t)(b0 + ar) * a.T + 0) * A + ac] = act;
    }
    __syncthreads();
  }

  // gh = W_hh h_0 on the slice; e_0 = ELU(W_as [s_0; a_0] + b_as)
  {
    const f32x4 acc = reg_product<NQ>(sm + L.h + (lane & 3) * L.ld_h, whh, kh0);
#pragma unroll
    for (int v = 0; v < 4; ++v) redg[(quarter * 4 + v) * 128 + col] = acc[v];
  }
  elu_pass_product(sm + L.sa, L.ld_sa, sm + L.was, L.ld_sa, sm + L.bas, sm + L.e, L.ld_e, E, SA);
  __syncthreads();
  for (int i = tid; i < 4 * ng; i += kThreads) {
    const int v = i / ng, c = i - v * ng;
    gh[v * 128 + c] = redg[v * 128 + c] + redg[(4 + v) * 128 + c] + redg[(8 + v) * 128 + c] + redg[(12 + v) * 128 + c];
  }
  __syncthreads();

  const int EC = a.Ep / 4, HC = a.Hbp / 4, ECU = ea0 / 4;  // chunks past ECU are the actor's
  const int npass_1 = (N1 + 63) / 64;
  float* stg = sm + L.stg;
  // staged steps and columns (noise, then without the actor the next action)
  constexpr int KS = ACTOR ? kStageActor : kStage;
  const int SC = ACTOR ? S : SA;
  // nothing loaded in the prologue may count as pending inside the loop
  wait_all_mem();
  for (int t = 0; t < a.T; ++t) {
    const int slot = t & (kRing - 1);
    if (t % KS == 0) {
      // noise of steps t .. t + KS - 1 and the actions they feed forward
      // (action t' + 1 beside noise t'), for this group's rows
      const int ns = min(KS, a.T - t);
      for (int i = tid; i < nrows * ns * SC; i += kThreads) {
        const int r = i / (ns * SC), rem = i - r * (ns * SC), k = rem / SC, c = rem - k * SC;
        const int b = b0 + r, tt = t + k;
        float v = 0.f;
        if (c < S)
          v = a.eps[((size_t)b * a.T + tt) * S + c];
        else if (tt + 1 < a.T)
          v = a.actions[((size_t)b * a.T + tt + 1) * A + (c - S)];
        stg[(r * KS + k) * L.ld_stg + c] = v;
      }
      __syncthreads();
    }
    const float* stg_t = stg + (t % KS) * L.ld_stg;
    // ---- GRU input product on the slice: gi = W_ih e_t ----
    {
      const f32x4 acc = reg_product<NQ>(sm + L.e + (lane & 3) * L.ld_e, wih, ke0);
#pragma unroll
      for (int v = 0; v < 4; ++v) redg[(quarter * 4 + v) * 128 + col] = acc[v];
    }
    __syncthreads();
    // ---- gates; publish h_t of the owned units ----
    if (owner) {
      const float* rg0 = redg + own_r * 128 + own_j;
      auto gsum = [&](int c) { return rg0[c] + rg0[512 + c] + rg0[1024 + c] + rg0[1536 + c]; };
      const float* ghr = gh + own_r * 128 + own_j;
      const float rg = fsigmoid(gsum(0) + ghr[0] + bias_r);
      const float zg = fsigmoid(gsum(hp) + ghr[hp] + bias_z);
      const float ng_ = ftanh(gsum(2 * hp) + bias_nx + rg * (ghr[2 * hp] + bias_nh));
      const float h = (1.f - zg) * ng_ + zg * hreg;
      hreg = h;
      sm[L.hs + own_r * L.ld_hs + own_j] = h;
      pub_store(hx_rs, hx_el(slot, b0 + own_r, j0 + own_j), publish_bits(h));
      a.beliefs[((size_t)(b0 + own_r) * a.T + t) * Hb + j0 + own_j] = h;
    }
    __syncthreads();
    // ---- this slice's share of W_1 h_t (and of the actor's W_a1[:, S:] h_t),
    //      stored to the ring from the MFMA lanes ----
    if (wave < npass_1) {
      const int c = wave * 64 + lane;
      const f32x4 acc = dot_batch<16>(sm + L.hs + (lane & 3) * L.ld_hs, sm + L.w1s + (c < N1 ? c : N1 - 1) * L.ld_hs,
                                      0, (hp + 3) / 4, f32x4{0.f, 0.f, 0.f, 0.f});
      if (c < N1) {
        const int col = c < E ? c : ea0 + (c - E);
#pragma unroll
        for (int v = 0; v < kMaxRows; ++v)
          if (v < nrows) pub_store(px_rs, px_el(slot, b0 + v, w, col), publish_bits(acc[v]));
      }
    }

    // ---- whole h_t and u_t = ELU(sum of every member's partials + b_1):
    //      poll the chunks of slot t until no sentinel is left. Whole waves
    //      take u chunks (every member's partials of one chunk) or h chunks,
    //      so each wave polls one buffer; load offsets are computed before
    //      the first load, so a reload never waits on an unrelated one. ----
    {
      const int nu = nrows * EC, nhc = nrows * HC;
      const int hbase = (nu + 63) & ~63;
      const bool wave_u = __builtin_amdgcn_readfirstlane(tid < hbase ? 1 : 0) != 0;  // hbase is a multiple of 64
      const int i = wave_u ? tid : tid - hbase;
      const bool act = wave_u ? i < nu : i < nhc;
      const int per = wave_u ? EC : HC;
      const int r = act ? i / per : 0, c = act ? i - r * per : 0;
      const int valid = !wave_u                ? min(4, Hb - 4 * c)
                        : (!ACTOR || c < ECU) ? min(4, E - 4 * c)
                                              : min(4, Ea - 4 * (c - ECU));
      const int nm = act ? (wave_u ? nw : 1) : 0;
      const __amdgpu_buffer_rsrc_t rs = wave_u ? px_rs : hx_rs;
      uint32_t off[kMaxMembers2];
#pragma unroll
      for (int m = 0; m < kMaxMembers2; ++m)
        off[m] = (wave_u ? px_el(slot, b0 + r, m, 4 * c) : hx_el(slot, b0 + r, 4 * c)) * 4u;
      u32x4 v[kMaxMembers2];
      unsigned pend = 0;
#pragma unroll
      for (int m = 0; m < kMaxMembers2; ++m)
        if (m < nm) {
          v[m] = coh_poll16(rs, off[m]);
          pend |= 1u << m;
        }
      uint64_t t0 = 0;
      unsigned polls = 0;
      while (true) {
#pragma unroll
        for (int m = 0; m < kMaxMembers2; ++m)
          if ((pend >> m) & 1u)
            if (!has_sentinel(v[m], valid)) pend &= ~(1u << m);
        if (!pend) break;
        if ((++polls & 63u) == 0) {  // watchdog: ~2 s without completing, or another member's error
          const uint64_t now = __builtin_amdgcn_s_memrealtime();
          if (t0 == 0) t0 = now;
          const int st = __hip_atomic_load(a.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (st != kStatusOk || now - t0 > kWatchdogTicks) {
            __hip_atomic_store(a.status, kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            *abort_flag = 1;
            break;
          }
        }
#pragma unroll
        for (int m = 0; m < kMaxMembers2; ++m)
          if ((pend >> m) & 1u) v[m] = coh_poll16(rs, off[m]);
      }
      // every load of the poll has returned (nothing younger was issued)
      wait_all_mem();
      if (act && wave_u) {
        f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < kMaxMembers2; ++m)
          if (m < nw) s4 += __builtin_bit_cast(f32x4, v[m]);
        if (!ACTOR || c < ECU) {
#pragma unroll
          for (int k = 0; k < 4; ++k) s4[k] = k < valid ? felu(s4[k] + sm[L.b1 + 4 * c + k]) : 0.f;
          *reinterpret_cast<f32x4*>(sm + L.u + r * L.ld_e + 4 * c) = s4;
        } else {
          // the actor's belief term, summed (its activation comes with s_t)
#pragma unroll
          for (int k = 0; k < 4; ++k)
            if (k >= valid) s4[k] = 0.f;
          *reinterpret_cast<f32x4*>(sm + L.qa + r * L.ld_q + 4 * (c - ECU)) = s4;
        }
      } else if (act) {
        f32x4 hf = __builtin_bit_cast(f32x4, v[0]);
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (k >= valid) hf[k] = 0.f;
        *reinterpret_cast<f32x4*>(sm + L.h + r * L.ld_h + 4 * c) = hf;
      }
    }
    __syncthreads();
    if (*abort_flag) return;
    // ---- v_t = W_2 u_t and, for the next step, W_hh h_t on the slice ----
    {
      const f32x4 cv = dot_batch<8>(sm + L.u + (lane & 3) * L.ld_e, w2row, k20, n2, f32x4{0.f, 0.f, 0.f, 0.f});
      const f32x4 ch = reg_product<NQ>(sm + L.h + (lane & 3) * L.ld_h, whh, kh0);
      // every member has published step t, so every member is done with
      // slot t - 1: reset this member's entries of it (while the products run)
      if (t > 0) {
        const int old = (t - 1) & (kRing - 1);
        if (owner) pub_store(hx_rs, hx_el(old, b0 + own_r, j0 + own_j), kSentinel);
        if (wave < npass_1) {
          const int c = wave * 64 + lane;
          if (c < N1) {
            const int col = c < E ? c : ea0 + (c - E);
#pragma unroll
            for (int v = 0; v < kMaxRows; ++v)
              if (v < nrows) pub_store(px_rs, px_el(old, b0 + v, w, col), kSentinel);
          }
        }
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        redv[(wave * 4 + v) * 64 + lane] = cv[v];
        redg[(quarter * 4 + v) * 128 + col] = ch[v];
      }
    }
    __syncthreads();
    // ---- (mean, std, s_t) from the reduction of v_t; gh for step t + 1;
    //      the next action into [s; a] ----
    if (tail_owner) {
      const float vm = red_sum(redv, tr, tc) + sm[L.b2 + tc];
      const float vs = red_sum(redv, tr, S + tc) + sm[L.b2 + S + tc];
      const float sd = fsoftplus(vs) + a.scale_lb;
      const float st = vm + stg_t[tr * KS * L.ld_stg + tc] * sd;
      sm[L.sa + tr * L.ld_sa + tc] = st;
      if (w == 0) {
        const size_t o = ((size_t)(b0 + tr) * a.T + t) * S + tc;
        a.means[o] = vm;
        a.stds[o] = sd;
        a.states[o] = st;
      }
    }
    for (int i = tid; i < 4 * ng; i += kThreads) {
      const int v = i / ng, c = i - v * ng;
      gh[v * 128 + c] =
          redg[v * 128 + c] + redg[(4 + v) * 128 + c] + redg[(8 + v) * 128 + c] + redg[(12 + v) * 128 + c];
    }
    if (!ACTOR && act_owner && t + 1 < a.T) sm[L.sa + ar * L.ld_sa + S + ac] = stg_t[ar * KS * L.ld_stg + S + ac];
    __syncthreads();
    if constexpr (ACTOR) {
      if (t + 1 < a.T) {
        // ---- a_{t+1} = tanh(W_a2 ELU(W_a1[:, :S] s_t + W_a1[:, S:] h_t + b_a1)
        //      + b_a2), written into the action slot that e_{t+1} reads ----
        elu_pass_product_add(sm + L.sa, L.ld_sa, sm + L.wa1s, L.ld_s, sm + L.ba1, sm + L.qa, L.ld_q, sm + L.q,
                             L.ld_q, Ea, S);
        __syncthreads();
        {
          const int Q4 = (Ea + 3) / 4, per = (Q4 + kWaves - 1) / kWaves;
          const int ka = min(Q4, wave * per), kn = min(Q4, ka + per) - ka;
          const f32x4 acc = dot_batch<8>(sm + L.q + (lane & 3) * L.ld_q, sm + L.wa2 + (lane < A ? lane : A - 1) * L.ld_q,
                                         ka, kn, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int v = 0; v < 4; ++v) redv[(wave * 4 + v) * 64 + lane] = acc[v];
        }
        __syncthreads();
        if (act_owner) {
          const float act = ftanh(red_sum(redv, ar, ac) + sm[L.ba2 + ac]);
          sm[L.sa + ar * L.ld_sa + S + ac] = act;
          if (w == 0 && a.act_out) a.act_out[((size_t)(b0 + ar) * a.T + t + 1) * A + ac] = act;
        }
        __syncthreads();
      }
    }
    // ---- e_{t+1} = ELU(W_as [s_t; a_{t+1}] + b_as) ----
    if (t + 1 < a.T) {
      elu_pass_product(sm + L.sa, L.ld_sa, sm + L.was, L.ld_sa, sm + L.bas, sm + L.e, L.ld_e, E, SA);
      __syncthreads();
    }
  }
}

template <int NQ, bool ACTOR>
hipError_t launch_rssm_reg_as(const RssmArgs& a, int lds, hipStream_t stream) {
  hipError_t e = hipFuncSetAttribute((const void*)rssm_reg_kernel<NQ, ACTOR>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  const int grid = a.nxcd * a.gpx * a.nw;
  launch_kernel((rssm_reg_kernel<NQ, ACTOR>), dim3(grid), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

template <bool ACTOR>
hipError_t launch_rssm_reg_nq(const RssmArgs& a, int lds, hipStream_t stream) {
  switch (rssm_reg_nq(a)) {
    case 4: return launch_rssm_reg_as<4, ACTOR>(a, lds, stream);
    case 8: return launch_rssm_reg_as<8, ACTOR>(a, lds, stream);
    case 13: return launch_rssm_reg_as<13, ACTOR>(a, lds, stream);
    default:
      // (rssm_reg_fits keeps the actor off the widest layout)
      if constexpr (ACTOR) return hipErrorInvalidValue;
      else return launch_rssm_reg_as<16, ACTOR>(a, lds, stream);
  }
}

}  // namespace

int rssm_reg_lds_bytes(const RssmArgs& a) { return rssm2_lds(a, a.Ea).total; }

bool rssm_reg_fits(const RssmArgs& a) {
  // (actor: the partial columns take at most one 64-column pass per wave,
  // W_a2's K split gives each wave at most eight chunks, one lane per action)
  // (and the widest register layout would spill with the actor's working set)
  const bool actor_ok = a.Ea == 0 || (a.Ea <= 256 && a.E + a.Ea <= 64 * kWaves && a.A <= 64 &&
                                      a.Ep == r4(a.E) + r4(a.Ea) && rssm_reg_nq(a) <= 13);
  return actor_ok && a.rows >= 1 && a.rows <= kMaxRows && a.nw >= 1 && a.nw <= kMaxMembers2 && a.h_per >= 1 &&
         3 * a.h_per <= 128 && (a.h_per + 3) / 4 <= 16 && 2 * a.S <= 64 && a.S + a.A <= 64 &&
         rssm_reg_nq(a) > 0 && a.rows * a.h_per <= kThreads &&
         ((a.rows * (a.Ep / 4) + 63) & ~63) + a.rows * (a.Hbp / 4) <= kThreads && a.rows * a.S <= kThreads &&
         a.rows * a.A <= kThreads &&
         a.E <= 256;
}

int rssm_ring_slots() { return kRing; }
int rssm_reg_max_members() { return kMaxMembers2; }

hipError_t launch_rssm_reg(const RssmArgs& a, hipStream_t stream) {
  const int lds = rssm2_lds(a, a.Ea).total;
  return a.Ea > 0 ? launch_rssm_reg_nq<true>(a, lds, stream) : launch_rssm_reg_nq<false>(a, lds, stream);
}

}  // namespace rnnk
