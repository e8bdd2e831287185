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
#include "device_common.hpp"
#include "kernels.hpp"

namespace rnnk {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxRows = 4;  // batch rows per group: one 4x4 MFMA block row set

__host__ __device__ inline int r4(int x) { return (x + 3) & ~3; }

// out[v * ldo + c] = sum_{k < K} X[v * ldx + k] * W[c * ldw + k] for all four
// rows v of X (rows past the group's batch rows hold zeros and are ignored
// by the callers) and c < N, on v_mfma_f32_4x4x1f32: 16 blocks of 4x4 per
// instruction, lane l of a pass owning output column 64 * pass + l. X and W
// rows are 16-byte aligned and zero-padded to a multiple of 4. Narrow
// products (N <= 64) split K over the four waves and reduce through `red`
// (4 waves x 4 rows x 64 floats); wider ones give the waves whole 64-column
// passes.
__device__ void mv4(const float* X, int ldx, const float* W, int ldw, float* out, int ldo, int N, int K,
                    float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int K4 = (K + 3) >> 2;
  const float* xr = X + (lane & 3) * ldx;
  // One accumulator: an MFMA whose accumulator input is exactly the
  // previous MFMA's output issues back to back, so a single chain runs at
  // full rate and needs no register shuffling. Two chunks per iteration let
  // the second chunk's LDS reads overlap the first chunk's products. Bounds
  // are wave-uniform.
  auto run = [&](int c, int k4a, int k4b) -> f32x4 {
    k4a = __builtin_amdgcn_readfirstlane(k4a);
    k4b = __builtin_amdgcn_readfirstlane(k4b);
    const float* wr = W + (c < N ? c : N - 1) * ldw;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    int k4 = k4a;
    for (; k4 + 2 <= k4b; k4 += 2) {
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(xr + 4 * k4);
      const f32x4 b0 = *reinterpret_cast<const f32x4*>(wr + 4 * k4);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(xr + 4 * k4 + 4);
      const f32x4 b1 = *reinterpret_cast<const f32x4*>(wr + 4 * k4 + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_4x4x1f32(a0[e], b0[e], acc, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_4x4x1f32(a1[e], b1[e], acc, 0, 0, 0);
    }
    if (k4 < k4b) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(xr + 4 * k4);
      const f32x4 b = *reinterpret_cast<const f32x4*>(wr + 4 * k4);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_4x4x1f32(a[e], b[e], acc, 0, 0, 0);
    }
    return acc;
  };
  if (N > 64) {
    for (int cg = __builtin_amdgcn_readfirstlane(wave); cg * 64 < N; cg += 4) {
      const int c = cg * 64 + lane;
      const f32x4 acc = run(c, 0, K4);
      if (c < N) {
#pragma unroll
        for (int v = 0; v < 4; ++v) out[v * ldo + c] = acc[v];
      }
    }
    return;
  }
  const int per = (K4 + 3) >> 2;
  const int ka = min(K4, wave * per), kb = min(K4, ka + per);
  const f32x4 acc = run(lane, ka, kb);
#pragma unroll
  for (int v = 0; v < 4; ++v) red[(wave * 4 + v) * 64 + lane] = acc[v];
  __syncthreads();
  for (int i = threadIdx.x; i < 4 * N; i += kThreads) {
    const int v = i / N, c = i - v * N;
    out[v * ldo + c] = red[(0 * 4 + v) * 64 + c] + red[(1 * 4 + v) * 64 + c] + red[(2 * 4 + v) * 64 + c] +
                       red[(3 * 4 + v) * 64 + c];
  }
}

struct RssmLds {
  // float offsets (all multiples of 4)
  int was, bas, w2, b2, wih, whh, bih, bhh, w1s, b1;
  int sa, e, h, hs, u, v, gi, gh, pu, red, flag, total;
  int ld_sa, ld_e, ld_h, ld_hs, ld_v, ld_g;
};

__host__ __device__ inline RssmLds rssm_lds(const RssmArgs& a) {
  RssmLds L;
  const int SA = a.S + a.A;
  L.ld_sa = r4(SA);
  L.ld_e = r4(a.E);
  L.ld_h = r4(a.Hb);
  L.ld_hs = r4(a.h_per);
  L.ld_v = r4(2 * a.S);
  L.ld_g = r4(3 * a.h_per);
  const int R = kMaxRows;
  int o = 0;
  auto take = [&](int n) { const int at = o; o += r4(n); return at; };
  L.was = take(a.E * L.ld_sa);
  L.bas = take(a.E);
  L.w2 = take(2 * a.S * L.ld_e);
  L.b2 = take(2 * a.S);
  L.wih = take(3 * a.h_per * L.ld_e);
  L.whh = take(3 * a.h_per * L.ld_h);
  L.bih = take(3 * a.h_per);
  L.bhh = take(3 * a.h_per);
  L.w1s = take(a.E * L.ld_hs);
  L.b1 = take(a.E);
  L.sa = take(R * L.ld_sa);
  L.e = take(R * L.ld_e);
  L.h = take(R * L.ld_h);
  L.hs = take(R * L.ld_hs);
  L.u = take(R * L.ld_e);
  L.v = take(R * L.ld_v);
  L.gi = take(R * L.ld_g);
  L.gh = take(R * L.ld_g);
  L.pu = take(R * L.ld_e);
  L.red = take(4 * 4 * 64);
  L.flag = take(4);
  L.total = o * 4;
  return L;
}

__global__ void __launch_bounds__(kThreads) rssm_kernel(RssmArgs a) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  const RssmLds L = rssm_lds(a);
  const int tid = threadIdx.x;
  const int w = blockIdx.x % a.nw;
  const int g = blockIdx.x / a.nw;
  const int b0 = g * a.rows;
  const int nrows = min(a.rows, a.B - b0);
  const int S = a.S, A = a.A, E = a.E, Hb = a.Hb, SA = a.S + a.A;
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
  for (int i = tid; i < 2 * S * E; i += kThreads) {
    const int r = i / E, c = i - r * E;
    sm[L.w2 + r * L.ld_e + c] = a.w_2[i];
  }
  for (int i = tid; i < 2 * S; i += kThreads) sm[L.b2 + i] = a.b_2[i];
  // GRU slice: local row q * hp + jj <-> global row q * Hb + j0 + jj
  for (int i = tid; i < 3 * hp * E; i += kThreads) {
    const int r = i / E, c = i - r * E;
    const int q = r / hp, jj = r - q * hp;
    if (jj < hn) sm[L.wih + r * L.ld_e + c] = a.w_ih[(size_t)(q * Hb + j0 + jj) * E + c];
  }
  for (int i = tid; i < 3 * hp * Hb; i += kThreads) {
    const int r = i / Hb, c = i - r * Hb;
    const int q = r / hp, jj = r - q * hp;
    if (jj < hn) sm[L.whh + r * L.ld_h + c] = a.w_hh[(size_t)(q * Hb + j0 + jj) * Hb + c];
  }
  for (int i = tid; i < 3 * hp; i += kThreads) {
    const int q = i / hp, jj = i - q * hp;
    if (jj < hn) {
      sm[L.bih + i] = a.b_ih[q * Hb + j0 + jj];
      sm[L.bhh + i] = a.b_hh[q * Hb + j0 + jj];
    }
  }
  // W_1 columns of the slice: w1s[k][jj] = W_1[k][j0 + jj]
  for (int i = tid; i < E * hp; i += kThreads) {
    const int k = i / hp, jj = i - k * hp;
    if (jj < hn) sm[L.w1s + k * L.ld_hs + jj] = a.w_1[(size_t)k * Hb + j0 + jj];
  }

  // --- initial state: [s_0; a_0], whole h_0, own h copy ----------------------
  for (int i = tid; i < nrows * SA; i += kThreads) {
    const int r = i / SA, c = i - r * SA;
    const int b = b0 + r;
    sm[L.sa + r * L.ld_sa + c] = c < S ? (a.s0 ? a.s0[(size_t)b * S + c] : 0.f)
                                       : a.actions[((size_t)b * a.T + 0) * A + (c - S)];
  }
  for (int i = tid; i < nrows * Hb; i += kThreads) {
    const int r = i / Hb, c = i - r * Hb;
    sm[L.h + r * L.ld_h + c] = a.h0 ? a.h0[(size_t)(b0 + r) * Hb + c] : 0.f;
  }
  const int own_r = tid / hp, own_j = tid - own_r * hp;
  const bool owner = tid < a.rows * hp && own_r < nrows && own_j < hn;
  float hreg = (owner && a.h0) ? a.h0[(size_t)(b0 + own_r) * Hb + j0 + own_j] : 0.f;
  // per-thread (row, state unit) of the tail, fixed for the launch
  const int tr = tid / S, tc = tid - tr * S;
  const bool tail_owner = tid < nrows * S;
  const int ar = tid / A, ac = tid - ar * A;
  const bool act_owner = tid < nrows * A;
  __syncthreads();
  mv4(sm + L.sa, L.ld_sa, sm + L.was, L.ld_sa, sm + L.e, L.ld_e, E, SA, red);
  __syncthreads();
  for (int i = tid; i < nrows * E; i += kThreads) {
    const int r = i / E, c = i - r * E;
    sm[L.e + r * L.ld_e + c] = felu(sm[L.e + r * L.ld_e + c] + sm[L.bas + c]);
  }
  __syncthreads();

  unsigned nbar = 0;
  for (int t = 0; t < a.T; ++t) {
    const int par = t & 1;
    // ---- GRU phase on the owned slice: gi = W_ih e_t, gh = W_hh h_{t-1} ----
    mv4(sm + L.e, L.ld_e, sm + L.wih, L.ld_e, sm + L.gi, L.ld_g, 3 * hp, E, red);
    __syncthreads();
    mv4(sm + L.h, L.ld_h, sm + L.whh, L.ld_h, sm + L.gh, L.ld_g, 3 * hp, Hb, red);
    __syncthreads();
    if (owner) {
      const float* gi = sm + L.gi + own_r * L.ld_g;
      const float* gh = sm + L.gh + own_r * L.ld_g;
      const int jr = own_j, jz = hp + own_j, jn = 2 * hp + own_j;
      const float rg = fsigmoid(gi[jr] + sm[L.bih + jr] + gh[jr] + sm[L.bhh + jr]);
      const float zg = fsigmoid(gi[jz] + sm[L.bih + jz] + gh[jz] + sm[L.bhh + jz]);
      const float ng = ftanh(gi[jn] + sm[L.bih + jn] + rg * (gh[jn] + sm[L.bhh + jn]));
      const float h = (1.f - zg) * ng + zg * hreg;
      hreg = h;
      sm[L.hs + own_r * L.ld_hs + own_j] = h;
      coh_store_elem<float>(hx_rs, hx_el(par, b0 + own_r, j0 + own_j), h);
    }
    __syncthreads();
    // ---- this slice's share of the projector's first layer ----
    mv4(sm + L.hs, L.ld_hs, sm + L.w1s, L.ld_hs, sm + L.pu, L.ld_e, E, hp, red);
    __syncthreads();
    for (int i = tid; i < nrows * (L.ld_e / 4); i += kThreads) {
      const int r = i / (L.ld_e / 4), c4 = i - r * (L.ld_e / 4);
      coh_store16(px_rs, px_el(par, b0 + r, w, 4 * c4) * 4u,
                  *reinterpret_cast<const u32x4*>(sm + L.pu + r * L.ld_e + 4 * c4));
    }
    ++nbar;
    group_arrive(counter);
    // while the other members arrive: this step's belief, next inputs
    if (owner) a.beliefs[((size_t)(b0 + own_r) * a.T + t) * Hb + j0 + own_j] = hreg;
    const float eps_v = tail_owner ? a.eps[((size_t)(b0 + tr) * a.T + t) * S + tc] : 0.f;
    const float act_v = (act_owner && t + 1 < a.T) ? a.actions[((size_t)(b0 + ar) * a.T + t + 1) * A + ac] : 0.f;
    if (!group_wait(counter, nbar * a.nw, a.status, abort_flag)) return;

    // ---- whole h_t for the next GRU phase; u_t from the summed partials ----
    for (int i = tid; i < nrows * (a.Hbp / 4); i += kThreads) {
      const int r = i / (a.Hbp / 4), c4 = i - r * (a.Hbp / 4);
      *reinterpret_cast<u32x4*>(sm + L.h + r * L.ld_h + 4 * c4) = coh_load16(hx_rs, hx_el(par, b0 + r, 4 * c4) * 4u);
    }
    for (int i = tid; i < nrows * (L.ld_e / 4); i += kThreads) {
      const int r = i / (L.ld_e / 4), c4 = i - r * (L.ld_e / 4);
      // all members' partials in a fixed order, eight loads in flight
      f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
      for (int m0 = 0; m0 < a.nw; m0 += 8) {
        u32x4 pv[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) pv[m] = coh_load16(px_rs, px_el(par, b0 + r, min(m0 + m, a.nw - 1), 4 * c4) * 4u);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const f32x4 v = __builtin_bit_cast(f32x4, pv[m]);
          s4 += (m0 + m < a.nw) ? v : f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
      *reinterpret_cast<f32x4*>(sm + L.u + r * L.ld_e + 4 * c4) = s4;
    }
    __syncthreads();
    for (int i = tid; i < nrows * E; i += kThreads) {
      const int r = i / E, k = i - r * E;
      sm[L.u + r * L.ld_e + k] = felu(sm[L.u + r * L.ld_e + k] + sm[L.b1 + k]);
    }
    __syncthreads();
    // ---- v_t, (mean, std, s_t), then e_{t+1} (every member, whole) ----
    mv4(sm + L.u, L.ld_e, sm + L.w2, L.ld_e, sm + L.v, L.ld_v, 2 * S, E, red);
    __syncthreads();
    if (tail_owner) {
      const float* vr = sm + L.v + tr * L.ld_v;
      const float mean = vr[tc] + sm[L.b2 + tc];
      const float sd = fsoftplus(vr[S + tc] + sm[L.b2 + S + tc]) + a.scale_lb;
      const float st = mean + eps_v * sd;
      sm[L.sa + tr * L.ld_sa + tc] = st;
      if (w == 0) {
        const size_t o = ((size_t)(b0 + tr) * a.T + t) * S + tc;
        a.means[o] = mean;
        a.stds[o] = sd;
        a.states[o] = st;
      }
    }
    if (t + 1 < a.T) {
      if (act_owner) sm[L.sa + ar * L.ld_sa + S + ac] = act_v;
      __syncthreads();
      mv4(sm + L.sa, L.ld_sa, sm + L.was, L.ld_sa, sm + L.e, L.ld_e, E, SA, red);
      __syncthreads();
      for (int i = tid; i < nrows * E; i += kThreads) {
        const int r = i / E, c = i - r * E;
        sm[L.e + r * L.ld_e + c] = felu(sm[L.e + r * L.ld_e + c] + sm[L.bas + c]);
      }
    }
    __syncthreads();
  }
}

}  // namespace

int rssm_lds_bytes(const RssmArgs& a) { return rssm_lds(a).total; }
int rssm_max_rows() { return kMaxRows; }

hipError_t launch_rssm(const RssmArgs& a, hipStream_t stream) {
  const int lds = rssm_lds(a).total;
  hipError_t e = hipFuncSetAttribute((const void*)rssm_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(rssm_kernel, dim3(a.ngroups * a.nw), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace rnnk
