// Kernel 3: the RSSM prior unrolled over given actions, one launch.
//
// Step t (pytorch/rl issue "[Feature Request] CUDNN version of RSSM",
// Solution: RSSMPrior.forward inside the first unroll loop):
//   e_t   = ELU(W_as [s_{t-1}; a_t] + b_as)
//   h_t   = GRUCell(e_t, h_{t-1})                   (belief)
//   u_t   = ELU(W_1 h_t + b_1)
//   v_t   = W_2 u_t + b_2;  mean = v[:S];  std = softplus(v[S:]) + scale_lb
//   s_t   = mean + eps_t * std                      (eps injected)
// The issue explains why a fused GRU cannot serve here: every step has
// these extra ops between two GRU cells. This kernel keeps the whole unroll
// on the device instead of one host launch per op per step.
//
// Work split. Batch rows are independent, so the batch is cut into groups
// of `rows` rows that never talk to each other. Inside a group, `nw`
// workgroups each own a slice of the GRU hidden units: the W_ih and W_hh rows
// of all three gates for those units, and the matching columns of W_1, all
// resident in LDS. One exchange per step suffices:
//   * the GRU phase produces the owned slice of h_t, and from it the
//     slice's contribution W_1[:, slice] h_t[slice] to every output of the
//     projector's first layer (a K-split partial sum);
//   * after one group barrier every member reads the whole h_t (needed by
//     the next GRU phase) and all members' partials, sums the partials in a
//     fixed order (deterministic), and computes u_t, v_t, s_t and e_{t+1}
//     itself (W_2 and W_as are small enough to keep whole in every member).
//
// With an actor in the loop (the issue's second unroll, the actor being the
// synthetic MLP a = tanh(W_a2 ELU(W_a1 [s; h] + b_a1) + b_a2)), the action
// of step t + 1 is computed from s_t and h_t at the end of step t: the
// belief part W_a1[:, S:] h_t is split over the members like W_1 and rides
// the same exchange (extra partial-sum columns); the state part, the ELU,
// W_a2 and the tanh are small products every member does whole.
#include "device_common.hpp"
#include "kernels.hpp"
#include "rssm_common.hpp"

namespace rnnk {

namespace {

using namespace rssmk;

// Two independent narrow products (N1, N2 <= 64) in one K-split pass: their
// chains interleave, so the second costs little extra latency. The waves'
// partial sums are left in red1 / red2 (kWaves x 4 rows x 64 floats) for the
// caller to reduce after a barrier.
__device__ void mv4_pair(const float* X1, int ldx1, const float* W1, int ldw1, int N1, int K1, float* red1,
                         const float* X2, int ldx2, const float* W2, int ldw2, int N2, int K2, float* red2) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int A4 = (K1 + 3) >> 2, B4 = (K2 + 3) >> 2;
  const int pa = (A4 + kWaves - 1) / kWaves, pb = (B4 + kWaves - 1) / kWaves;
  const int a0 = min(A4, wave * pa), a1 = min(A4, a0 + pa);
  const int b0 = min(B4, wave * pb), b1 = min(B4, b0 + pb);
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  const float* x1 = X1 + (lane & 3) * ldx1;
  const float* x2 = X2 + (lane & 3) * ldx2;
  const float* w1 = W1 + (lane < N1 ? lane : N1 - 1) * ldw1;
  const float* w2 = W2 + (lane < N2 ? lane : N2 - 1) * ldw2;
  f32x4 c1 = zero4, c2 = zero4;
  // common part: both chains advance together, four chunks per iteration
  const int n1 = a1 - a0, n2 = b1 - b0, nc = __builtin_amdgcn_readfirstlane(min(n1, n2));
  int q = 0;
  for (; q + 4 <= nc; q += 4) {
    f32x4 xa[4], wa[4], xb[4], wb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      xa[u] = *reinterpret_cast<const f32x4*>(x1 + 4 * (a0 + q + u));
      wa[u] = *reinterpret_cast<const f32x4*>(w1 + 4 * (a0 + q + u));
      xb[u] = *reinterpret_cast<const f32x4*>(x2 + 4 * (b0 + q + u));
      wb[u] = *reinterpret_cast<const f32x4*>(w2 + 4 * (b0 + q + u));
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c1 = __builtin_amdgcn_mfma_f32_4x4x1f32(xa[u][e], wa[u][e], c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_4x4x1f32(xb[u][e], wb[u][e], c2, 0, 0, 0);
      }
  }
  c1 = dot_chain(x1, w1, a0 + q, a1, c1);
  c2 = dot_chain(x2, w2, b0 + q, b1, c2);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    red1[(wave * 4 + v) * 64 + lane] = c1[v];
    red2[(wave * 4 + v) * 64 + lane] = c2[v];
  }
}


// W_hh (owned slice) and W_2 can live in registers when both products are
// narrow (one 64-column pass) and each wave's share of K fits kRegChunks
// 16-byte chunks.
constexpr int kRegChunks = 8;
__host__ __device__ inline bool rssm_regw(const RssmArgs& a) {
  const int e4 = (a.E + 3) / 4, h4 = (a.Hb + 3) / 4;
  return 2 * a.S <= 64 && 3 * a.h_per <= 64 && e4 <= kRegChunks * kWaves && h4 <= kRegChunks * kWaves;
}

// acc += sum over this wave's chunks [k0, k0 + n) of X chunk (LDS, lane's
// batch row) times the resident W chunks wr[0 .. n) (lane's column).
__device__ __forceinline__ f32x4 dot_chain_reg(const float* xr, const f32x4 (&wr)[kRegChunks], int k0, int n,
                                               f32x4 acc) {
  n = __builtin_amdgcn_readfirstlane(n);
  f32x4 x[kRegChunks];
#pragma unroll
  for (int q = 0; q < kRegChunks; ++q)
    if (q < n) x[q] = *reinterpret_cast<const f32x4*>(xr + 4 * (k0 + q));
#pragma unroll
  for (int q = 0; q < kRegChunks; ++q)
    if (q < n) {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_4x4x1f32(x[q][e], wr[q][e], acc, 0, 0, 0);
    }
  return acc;
}

// Resident chunks of W row `row` (or zeros when row < 0) for this wave's
// share of K4 chunks: wr[q] = W[row][4 (k0 + q) .. + 3], k < K.
__device__ __forceinline__ void load_wreg(f32x4 (&wr)[kRegChunks], const float* W, int row, int K, int k0, int n) {
#pragma unroll
  for (int q = 0; q < kRegChunks; ++q) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k = 4 * (k0 + q) + e;
      wr[q][e] = (row >= 0 && q < n && k < K) ? W[(size_t)row * K + k] : 0.f;
    }
  }
}

struct RssmLds {
  // float offsets (all multiples of 4)
  int was, bas, w2, b2, wih, whh, w1s, b1;
  int wa1s, ba1, wa2, ba2, q, qa;  // actor (empty without one)
  int sa, e, h, hs, u, v, gi, gh, red, red2, flag, total;
  int ld_sa, ld_e, ld_h, ld_hs, ld_v, ld_g, ld_s, ld_q;
};

__host__ __device__ inline RssmLds rssm_lds(const RssmArgs& a) {
  RssmLds L;
  const int SA = a.S + a.A;
  L.ld_sa = ld_rows(SA);
  L.ld_e = ld_rows(a.E);
  L.ld_h = ld_rows(a.Hb);
  L.ld_hs = ld_rows(a.h_per);
  L.ld_v = r4(2 * a.S);
  L.ld_g = r4(3 * a.h_per);
  L.ld_s = ld_rows(a.S);
  L.ld_q = ld_rows(a.Ea);
  const int Ea = a.Ea;
  const int R = kMaxRows;
  int o = 0;
  auto take = [&](int n) { const int at = o; o += r4(n); return at; };
  L.was = take(a.E * L.ld_sa);
  L.bas = take(a.E);
  const bool regw = rssm_regw(a);
  L.w2 = take(regw ? 0 : 2 * a.S * L.ld_e);
  L.b2 = take(2 * a.S);
  L.wih = take(3 * a.h_per * L.ld_e);
  L.whh = take(regw ? 0 : 3 * a.h_per * L.ld_h);
  L.w1s = take((a.E + Ea) * L.ld_hs);  // W_1 columns, then W_a1 belief columns
  L.b1 = take(a.E);
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
  L.v = take(R * L.ld_v);
  L.gi = take(R * L.ld_g);
  L.gh = take(R * L.ld_g);
  L.red = take(kWaves * 4 * 64);
  L.red2 = take(kWaves * 4 * 64);
  L.flag = take(4);
  L.total = o * 4;
  return L;
}

template <bool REGW, bool ACTOR>
__global__ void __launch_bounds__(kThreads) rssm_kernel(RssmArgs a) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  const RssmLds L = rssm_lds(a);
  const int tid = threadIdx.x;
  // Group and member of this workgroup. Workgroups are dealt to the XCDs
  // round-robin by id, so with gpx > 0 the ids xcd, xcd + nxcd, ... form the
  // groups of one XCD: the members' coherent exchange then stays between
  // the CUs of one chiplet (placement only; correctness never depends on it).
  int g, w;
  if (a.gpx > 0) {
    const int xcd = blockIdx.x % a.nxcd, slot = blockIdx.x / a.nxcd;
    g = xcd * a.gpx + slot / a.nw;
    w = slot % a.nw;
  } else {
    g = blockIdx.x / a.nw;
    w = blockIdx.x % a.nw;
  }
  if (g >= a.ngroups) return;  // padding slots of the XCD-aligned layout
  const int b0 = g * a.rows;
  const int nrows = min(a.rows, a.B - b0);
  const int S = a.S, A = a.A, E = a.E, Hb = a.Hb, SA = a.S + a.A;
  const int Ea = ACTOR ? a.Ea : 0;
  const int SH = S + Hb;        // W_a1 row length
  const int ea0 = r4(E);        // first actor column of an exchange row
  const int hp = a.h_per;
  const int j0 = w * hp, hn = max(0, min(hp, Hb - j0));  // owned hidden slice
  unsigned* counter = a.counters + (size_t)g * 16;
  int* abort_flag = reinterpret_cast<int*>(sm + L.flag);
  float* red = sm + L.red;

  const __amdgpu_buffer_rsrc_t hx_rs = make_rsrc(a.ex_h, (uint32_t)(2 * a.B * a.Hbp * 4));
  const __amdgpu_buffer_rsrc_t px_rs = make_rsrc(a.ex_p, (uint32_t)(2 * a.B * a.nw * a.Ep * 4));
  auto hx_el = [&](int par, int b, int j) -> uint32_t { return (uint32_t)((par * a.B + b) * a.Hbp + j); };
  auto px_el = [&](int par, int b, int m, int k) -> uint32_t {
    return (uint32_t)(((par * a.B + b) * a.nw + m) * a.Ep + k);
  };

  // --- zero all of LDS (padding rows and columns must read as zero) --------
  for (int i = tid; i < L.total / 4; i += kThreads) sm[i] = 0.f;
  __syncthreads();
  if (tid == 0) *abort_flag = 0;

  // --- resident weights -----------------------------------------------------
  for (int i = tid; i < E * SA; i += kThreads) {
    const int r = i / SA, c = i - r * SA;
    sm[L.was + r * L.ld_sa + c] = a.w_as[i];
  }
  for (int i = tid; i < E; i += kThreads) {
    sm[L.bas + i] = a.b_as[i];
    sm[L.b1 + i] = a.b_1[i];
  }
  if (!REGW) {
    for (int i = tid; i < 2 * S * E; i += kThreads) {
      const int r = i / E, c = i - r * E;
      sm[L.w2 + r * L.ld_e + c] = a.w_2[i];
    }
  }
  for (int i = tid; i < 2 * S; i += kThreads) sm[L.b2 + i] = a.b_2[i];
  // GRU slice: local row q * hp + jj <-> global row q * Hb + j0 + jj
  for (int i = tid; i < 3 * hp * E; i += kThreads) {
    const int r = i / E, c = i - r * E;
    const int q = r / hp, jj = r - q * hp;
    if (jj < hn) sm[L.wih + r * L.ld_e + c] = a.w_ih[(size_t)(q * Hb + j0 + jj) * E + c];
  }
  if (!REGW) {
    for (int i = tid; i < 3 * hp * Hb; i += kThreads) {
      const int r = i / Hb, c = i - r * Hb;
      const int q = r / hp, jj = r - q * hp;
      if (jj < hn) sm[L.whh + r * L.ld_h + c] = a.w_hh[(size_t)(q * Hb + j0 + jj) * Hb + c];
    }
  }
  // Resident W_2 and W_hh chunks (REGW): lane c holds row c of each (W_hh:
  // slice row c = gate q, unit jj) over this wave's share of K.
  const int wave = tid >> 6, lane = tid & 63;
  const int E4 = (E + 3) / 4, H4 = (Hb + 3) / 4;
  const int per_e = (E4 + kWaves - 1) / kWaves, per_h = (H4 + kWaves - 1) / kWaves;
  const int ke0 = min(E4, wave * per_e), ne = min(E4, ke0 + per_e) - ke0;
  const int kh0 = min(H4, wave * per_h), nh = min(H4, kh0 + per_h) - kh0;
  f32x4 w2r[REGW ? kRegChunks : 1], whr[REGW ? kRegChunks : 1];
  if constexpr (REGW) {
    load_wreg(w2r, a.w_2, lane < 2 * S ? lane : -1, E, ke0, ne);
    const int q = lane / hp, jj = lane - q * hp;
    load_wreg(whr, a.w_hh, (lane < 3 * hp && jj < hn) ? q * Hb + j0 + jj : -1, Hb, kh0, nh);
  }
  // W_1 columns of the slice: w1s[k][jj] = W_1[k][j0 + jj]
  for (int i = tid; i < E * hp; i += kThreads) {
    const int k = i / hp, jj = i - k * hp;
    if (jj < hn) sm[L.w1s + k * L.ld_hs + jj] = a.w_1[(size_t)k * Hb + j0 + jj];
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

  // --- initial state: [s_0; a_0], whole h_0, own h copy ----------------------
  for (int i = tid; i < nrows * SA; i += kThreads) {
    const int r = i / SA, c = i - r * SA;
    const int b = b0 + r;
    if (c < S)
      sm[L.sa + r * L.ld_sa + c] = a.s0 ? a.s0[(size_t)b * S + c] : 0.f;
    else if (!ACTOR)
      sm[L.sa + r * L.ld_sa + c] = a.actions[((size_t)b * a.T + 0) * A + (c - S)];
  }
  for (int i = tid; i < nrows * Hb; i += kThreads) {
    const int r = i / Hb, c = i - r * Hb;
    sm[L.h + r * L.ld_h + c] = a.h0 ? a.h0[(size_t)(b0 + r) * Hb + c] : 0.f;
  }
  const int own_r = tid / hp, own_j = tid - own_r * hp;
  const bool owner = tid < a.rows * hp && own_r < nrows && own_j < hn;
  float hreg = (owner && a.h0) ? a.h0[(size_t)(b0 + own_r) * Hb + j0 + own_j] : 0.f;
  // the owner's gate biases: r and z take b_ih + b_hh, the candidate keeps
  // b_hn inside the reset product
  float bias_r = 0.f, bias_z = 0.f, bias_nx = 0.f, bias_nh = 0.f;
  if (owner) {
    const float* bi = a.b_ih;
    const float* bh = a.b_hh;
    bias_r = bi[j0 + own_j] + bh[j0 + own_j];
    bias_z = bi[Hb + j0 + own_j] + bh[Hb + j0 + own_j];
    bias_nx = bi[2 * Hb + j0 + own_j];
    bias_nh = bh[2 * Hb + j0 + own_j];
  }
  // per-thread (row, state unit) of the tail, fixed for the launch
  const int tr = tid / S, tc = tid - tr * S;
  const bool tail_owner = tid < nrows * S;
  const int ar = tid / A, ac = tid - ar * A;
  const bool act_owner = tid < nrows * A;
  __syncthreads();
  if constexpr (ACTOR) {
    // a_0 = actor(s_0, h_0), once, straight from global W_a1 (not resident)
    for (int i = tid; i < nrows * Ea; i += kThreads) {
      const int r = i / Ea, c = i - r * Ea;
      const float* wr = a.w_a1 + (size_t)c * SH;
      float acc = 0.f;
      for (int k = 0; k < S; ++k) acc += wr[k] * sm[L.sa + r * L.ld_sa + k];
      for (int k = 0; k < Hb; ++k) acc += wr[S + k] * sm[L.h + r * L.ld_h + k];
      sm[L.q + r * L.ld_q + c] = felu(acc + sm[L.ba1 + c]);
    }
    __syncthreads();
    for (int i = tid; i < nrows * A; i += kThreads) {
      const int r = i / A, c = i - r * A;
      float acc = 0.f;
      for (int k = 0; k < Ea; ++k) acc += sm[L.wa2 + c * L.ld_q + k] * sm[L.q + r * L.ld_q + k];
      const float act = ftanh(acc + sm[L.ba2 + c]);
      sm[L.sa + r * L.ld_sa + S + c] = act;
      if (w == 0 && a.act_out) a.act_out[((size_t)(b0 + r) * a.T + 0) * A + c] = act;
    }
    __syncthreads();
  }
  // e_0 = ELU(W_as [s_0; a_0] + b_as) and the hidden part of the first GRU
  // step, W_hh h_0 on the owned slice
  const float* bas = sm + L.bas;
  auto elu_bias = [bas](int, int c, float x) { return felu(x + bas[c]); };
  mv4(sm + L.sa, L.ld_sa, sm + L.was, L.ld_sa, sm + L.e, L.ld_e, E, SA, red, elu_bias);
  __syncthreads();
  if constexpr (REGW) {
    const f32x4 acc = dot_chain_reg(sm + L.h + (lane & 3) * L.ld_h, whr, kh0, nh, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int v = 0; v < 4; ++v) red[(wave * 4 + v) * 64 + lane] = acc[v];
    __syncthreads();
    for (int i = tid; i < 4 * 3 * hp; i += kThreads) {
      const int v = i / (3 * hp), c = i - v * (3 * hp);
      sm[L.gh + v * L.ld_g + c] = red_sum(red, v, c);
    }
  } else {
    mv4(sm + L.h, L.ld_h, sm + L.whh, L.ld_h, sm + L.gh, L.ld_g, 3 * hp, Hb, red);
  }
  __syncthreads();

  unsigned nbar = 0;
  for (int t = 0; t < a.T; ++t) {
    const int par = t & 1;
    // ---- GRU phase on the owned slice: W_ih e_t here, W_hh h_{t-1} was
    //      computed alongside the previous step's projector ----
    mv4(sm + L.e, L.ld_e, sm + L.wih, L.ld_e, sm + L.gi, L.ld_g, 3 * hp, E, red);
    __syncthreads();
    if (owner) {
      const float* gi = sm + L.gi + own_r * L.ld_g;
      const float* gh = sm + L.gh + own_r * L.ld_g;
      const float rg = fsigmoid(gi[own_j] + gh[own_j] + bias_r);
      const float zg = fsigmoid(gi[hp + own_j] + gh[hp + own_j] + bias_z);
      const float ng = ftanh(gi[2 * hp + own_j] + bias_nx + rg * (gh[2 * hp + own_j] + bias_nh));
      const float h = (1.f - zg) * ng + zg * hreg;
      hreg = h;
      sm[L.hs + own_r * L.ld_hs + own_j] = h;
      coh_store_elem<float>(hx_rs, hx_el(par, b0 + own_r, j0 + own_j), h);
    }
    __syncthreads();
    // ---- this slice's share of the projector's first layer, stored to the
    //      exchange straight from the MFMA lanes (lane = output column) ----
    {
      const int lane = tid & 63;
      const float* xr = sm + L.hs + (lane & 3) * L.ld_hs;
      const int N1 = E + Ea;
      for (int cg = __builtin_amdgcn_readfirstlane(tid >> 6); cg * 64 < N1; cg += kWaves) {
        const int c = cg * 64 + lane;
        const f32x4 acc = dot_chain(xr, sm + L.w1s + (c < N1 ? c : N1 - 1) * L.ld_hs, 0, (hp + 3) / 4,
                                    f32x4{0.f, 0.f, 0.f, 0.f});
        if (c < N1) {
          const int col = c < E ? c : ea0 + (c - E);
#pragma unroll
          for (int v = 0; v < kMaxRows; ++v)
            if (v < nrows) coh_store_elem<float>(px_rs, px_el(par, b0 + v, w, col), acc[v]);
        }
      }
    }
    ++nbar;
    group_arrive(counter);
    // while the other members arrive: this step's belief, next inputs
    if (owner) a.beliefs[((size_t)(b0 + own_r) * a.T + t) * Hb + j0 + own_j] = hreg;
    const float eps_v = tail_owner ? a.eps[((size_t)(b0 + tr) * a.T + t) * S + tc] : 0.f;
    const float act_v =
        (!ACTOR && act_owner && t + 1 < a.T) ? a.actions[((size_t)(b0 + ar) * a.T + t + 1) * A + ac] : 0.f;
    if (!group_wait(counter, nbar * a.nw, a.status, abort_flag)) return;

    // ---- whole h_t for the next GRU phase; u_t from the summed partials.
    //      Thread i < nrows * EC owns chunk i of h (when it exists) and of the
    //      partial sums; all its loads are issued before the first is used.
    //      Elements past Hb or E (exchange padding nobody writes) read as 0.
    {
      const int EC = (E + 3) / 4, HC = a.Hbp / 4;
      const int i = tid;
      if (i < nrows * EC || i < nrows * HC) {
        const bool has_h = i < nrows * HC, has_p = i < nrows * EC;
        const int rh = has_h ? i / HC : 0, ch = i - rh * HC;
        const int rp = has_p ? i / EC : 0, cp = i - rp * EC;
        u32x4 hv = {0u, 0u, 0u, 0u};
        if (has_h) hv = coh_load16(hx_rs, hx_el(par, b0 + rh, 4 * ch) * 4u);
        f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
        if (has_p) {
          // all members' partials in a fixed order, up to sixteen loads in
          // flight (no load past the last member: traffic at the coherence
          // point delays the other members' exchange)
          for (int m0 = 0; m0 < a.nw; m0 += 16) {
            u32x4 pv[16];
#pragma unroll
            for (int m = 0; m < 16; ++m)
              pv[m] = m0 + m < a.nw ? coh_load16(px_rs, px_el(par, b0 + rp, m0 + m, 4 * cp) * 4u)
                                    : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int m = 0; m < 16; ++m) {
              const f32x4 v = __builtin_bit_cast(f32x4, pv[m]);
              s4 += (m0 + m < a.nw) ? v : f32x4{0.f, 0.f, 0.f, 0.f};
            }
          }
          // u_t = ELU(W_1 h_t + b_1); padding columns stay 0
#pragma unroll
          for (int k = 0; k < 4; ++k) s4[k] = 4 * cp + k < E ? felu(s4[k] + sm[L.b1 + 4 * cp + k]) : 0.f;
          *reinterpret_cast<f32x4*>(sm + L.u + rp * L.ld_e + 4 * cp) = s4;
        }
        if (has_h) {
          f32x4 hf = __builtin_bit_cast(f32x4, hv);
#pragma unroll
          for (int k = 0; k < 4; ++k)
            if (4 * ch + k >= Hb) hf[k] = 0.f;
          *reinterpret_cast<f32x4*>(sm + L.h + rh * L.ld_h + 4 * ch) = hf;
        }
      }
      if constexpr (ACTOR) {
        // belief part of the actor's pre-activation for step t + 1: all
        // members' partials of W_a1[:, S:] h_t in the same fixed order, on
        // the threads after those busy above (rotated thread index)
        const int EA = (Ea + 3) / 4;
        const int busy = max(nrows * EC, nrows * HC) % kThreads;
        for (int j = (tid - busy + kThreads) % kThreads; j < nrows * EA; j += kThreads) {
          const int rq = j / EA, cq = j - rq * EA;
          f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
          for (int m0 = 0; m0 < a.nw; m0 += 16) {
            u32x4 pv[16];
#pragma unroll
            for (int m = 0; m < 16; ++m)
              pv[m] = m0 + m < a.nw ? coh_load16(px_rs, px_el(par, b0 + rq, m0 + m, ea0 + 4 * cq) * 4u)
                                    : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int m = 0; m < 16; ++m) {
              const f32x4 v = __builtin_bit_cast(f32x4, pv[m]);
              s4 += (m0 + m < a.nw) ? v : f32x4{0.f, 0.f, 0.f, 0.f};
            }
          }
#pragma unroll
          for (int k = 0; k < 4; ++k)
            if (4 * cq + k >= Ea) s4[k] = 0.f;
          *reinterpret_cast<f32x4*>(sm + L.qa + rq * L.ld_q + 4 * cq) = s4;
        }
      }
    }
    __syncthreads();
    // ---- v_t = W_2 u_t and, for the next GRU step, W_hh h_t on the owned
    //      slice, in one K-split pass ----
    const bool pair = 2 * S <= 64 && 3 * hp <= 64;
    if constexpr (REGW) {
      // both chains from resident weights, interleaved by the scheduler
      const f32x4 c1 = dot_chain_reg(sm + L.u + (lane & 3) * L.ld_e, w2r, ke0, ne, f32x4{0.f, 0.f, 0.f, 0.f});
      const f32x4 c2 = dot_chain_reg(sm + L.h + (lane & 3) * L.ld_h, whr, kh0, nh, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        red[(wave * 4 + v) * 64 + lane] = c1[v];
        sm[L.red2 + (wave * 4 + v) * 64 + lane] = c2[v];
      }
    } else if (pair) {
      mv4_pair(sm + L.u, L.ld_e, sm + L.w2, L.ld_e, 2 * S, E, red, sm + L.h, L.ld_h, sm + L.whh, L.ld_h, 3 * hp, Hb,
               sm + L.red2);
    } else {
      mv4(sm + L.u, L.ld_e, sm + L.w2, L.ld_e, sm + L.v, L.ld_v, 2 * S, E, red);
      __syncthreads();
      mv4(sm + L.h, L.ld_h, sm + L.whh, L.ld_h, sm + L.gh, L.ld_g, 3 * hp, Hb, sm + L.red2);
    }
    __syncthreads();
    // (mean, std, s_t) straight from the reduction of v_t
    if (tail_owner) {
      const float vm = pair ? red_sum(red, tr, tc) : sm[L.v + tr * L.ld_v + tc];
      const float vs = pair ? red_sum(red, tr, S + tc) : sm[L.v + tr * L.ld_v + S + tc];
      const float mean = vm + sm[L.b2 + tc];
      const float sd = fsoftplus(vs + sm[L.b2 + S + tc]) + a.scale_lb;
      const float st = mean + eps_v * sd;
      sm[L.sa + tr * L.ld_sa + tc] = st;
      if (w == 0) {
        const size_t o = ((size_t)(b0 + tr) * a.T + t) * S + tc;
        a.means[o] = mean;
        a.stds[o] = sd;
        a.states[o] = st;
      }
    }
    if (pair) {
      const float* red2 = sm + L.red2;
      for (int i = tid; i < 4 * 3 * hp; i += kThreads) {
        const int v = i / (3 * hp), c = i - v * (3 * hp);
        sm[L.gh + v * L.ld_g + c] = red_sum(red2, v, c);
      }
    }
    if (t + 1 < a.T) {
      if constexpr (ACTOR) {
        __syncthreads();
        // a_{t+1} = tanh(W_a2 ELU(W_a1[:, :S] s_t + (W_a1[:, S:] h_t) + b_a1) + b_a2),
        // written into the action slot that e_{t+1} reads
        const float* qa = sm + L.qa;
        const float* ba1 = sm + L.ba1;
        const int ldq = L.ld_q;
        mv4(sm + L.sa, L.ld_sa, sm + L.wa1s, L.ld_s, sm + L.q, L.ld_q, Ea, S, red,
            [qa, ba1, ldq](int v, int c, float x) { return felu(x + qa[v * ldq + c] + ba1[c]); });
        __syncthreads();
        const float* ba2 = sm + L.ba2;
        mv4(sm + L.q, L.ld_q, sm + L.wa2, L.ld_q, sm + L.sa + S, L.ld_sa, A, Ea, red,
            [ba2](int, int c, float x) { return ftanh(x + ba2[c]); });
        __syncthreads();
        if (w == 0 && a.act_out && act_owner)
          a.act_out[((size_t)(b0 + ar) * a.T + t + 1) * A + ac] = sm[L.sa + ar * L.ld_sa + S + ac];
      } else {
        if (act_owner) sm[L.sa + ar * L.ld_sa + S + ac] = act_v;
        __syncthreads();
      }
      // e_{t+1} = ELU(W_as [s_t; a_{t+1}] + b_as), every member, whole
      mv4(sm + L.sa, L.ld_sa, sm + L.was, L.ld_sa, sm + L.e, L.ld_e, E, SA, red, elu_bias);
    }
    __syncthreads();
  }
}

}  // namespace

int rssm_lds_bytes(const RssmArgs& a) { return rssm_lds(a).total; }
int rssm_max_rows() { return kMaxRows; }

template <bool REGW, bool ACTOR>
hipError_t launch_rssm_as(const RssmArgs& a, int lds, hipStream_t stream) {
  hipError_t e = hipFuncSetAttribute((const void*)rssm_kernel<REGW, ACTOR>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  const int grid = a.gpx > 0 ? a.nxcd * a.gpx * a.nw : a.ngroups * a.nw;
  hipLaunchKernelGGL((rssm_kernel<REGW, ACTOR>), dim3(grid), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_rssm(const RssmArgs& a, hipStream_t stream) {
  const int lds = rssm_lds(a).total;
  const bool regw = rssm_regw(a), actor = a.Ea > 0;
  if (regw) return actor ? launch_rssm_as<true, true>(a, lds, stream) : launch_rssm_as<true, false>(a, lds, stream);
  return actor ? launch_rssm_as<false, true>(a, lds, stream) : launch_rssm_as<false, false>(a, lds, stream);
}

}  // namespace rnnk
