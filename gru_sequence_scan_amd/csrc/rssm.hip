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
constexpr int kMaxRows = 8;  // batch rows per group (register blocking)

__host__ __device__ inline int r4(int x) { return (x + 3) & ~3; }

// Product of up to kMaxRows batch rows with LDS-resident weights (K in
// floats, zero-padded to a multiple of 4).
template <int CPT>
__device__ __forceinline__ void mv_rows(const float* X, int ldx, const float* W, int ldw, float* out, int ldo,
                                        int rows, int cols, int K) {
  lds_gemv_rows<float, kMaxRows, CPT>(X, ldx, W, ldw, out, ldo, rows, cols, r4(K) >> 2);
}

struct RssmLds {
  // float offsets (all multiples of 4)
  int was, bas, w2, b2, wih, whh, bih, bhh, w1s, b1;
  int sa, e, h, hs, u, v, gi, gh, pu, flag, total;
  int ld_sa, ld_e, ld_h, ld_hs;
};

__host__ __device__ inline RssmLds rssm_lds(const RssmArgs& a) {
  RssmLds L;
  const int SA = a.S + a.A;
  L.ld_sa = r4(SA);
  L.ld_e = r4(a.E);
  L.ld_h = r4(a.Hb);
  L.ld_hs = r4(a.h_per);
  const int R = a.rows;
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
  L.v = take(R * 2 * a.S);
  L.gi = take(R * 3 * a.h_per);
  L.gh = take(R * 3 * a.h_per);
  L.pu = take(R * a.E);
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

  const __amdgpu_buffer_rsrc_t hx_rs = make_rsrc(a.ex_h, (uint32_t)(2 * a.B * a.Hbp * 4));
  const __amdgpu_buffer_rsrc_t px_rs = make_rsrc(a.ex_p, (uint32_t)(2 * a.B * a.nw * a.Ep * 4));
  auto hx_el = [&](int par, int b, int j) -> uint32_t { return (uint32_t)((par * a.B + b) * a.Hbp + j); };
  auto px_el = [&](int par, int b, int m, int k) -> uint32_t {
    return (uint32_t)(((par * a.B + b) * a.nw + m) * a.Ep + k);
  };

  // --- zero all of LDS (padding columns must read as zero) -------------------
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
  __syncthreads();
  mv_rows<4>(sm + L.sa, L.ld_sa, sm + L.was, L.ld_sa, sm + L.e, L.ld_e, nrows, E, SA);
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
    mv_rows<2>(sm + L.e, L.ld_e, sm + L.wih, L.ld_e, sm + L.gi, 3 * hp, nrows, 3 * hp, E);
    mv_rows<2>(sm + L.h, L.ld_h, sm + L.whh, L.ld_h, sm + L.gh, 3 * hp, nrows, 3 * hp, Hb);
    __syncthreads();
    if (owner) {
      const float* gi = sm + L.gi + own_r * 3 * hp;
      const float* gh = sm + L.gh + own_r * 3 * hp;
      const int jr = own_j, jz = hp + own_j, jn = 2 * hp + own_j;
      const float rg = fsigmoid(gi[jr] + sm[L.bih + jr] + gh[jr] + sm[L.bhh + jr]);
      const float zg = fsigmoid(gi[jz] + sm[L.bih + jz] + gh[jz] + sm[L.bhh + jz]);
      const float ng = ftanh(gi[jn] + sm[L.bih + jn] + rg * (gh[jn] + sm[L.bhh + jn]));
      const float h = (1.f - zg) * ng + zg * hreg;
      hreg = h;
      const int b = b0 + own_r;
      sm[L.hs + own_r * L.ld_hs + own_j] = h;
      coh_store_elem<float>(hx_rs, hx_el(par, b, j0 + own_j), h);
      a.beliefs[((size_t)b * a.T + t) * Hb + j0 + own_j] = h;
    }
    __syncthreads();
    // ---- this slice's share of the projector's first layer ----
    mv_rows<4>(sm + L.hs, L.ld_hs, sm + L.w1s, L.ld_hs, sm + L.pu, E, nrows, E, hp);
    __syncthreads();
    for (int i = tid; i < nrows * E; i += kThreads) {
      const int r = i / E, k = i - r * E;
      coh_store_elem<float>(px_rs, px_el(par, b0 + r, w, k), sm[L.pu + r * E + k]);
    }
    ++nbar;
    if (!group_barrier(counter, nbar * a.nw, a.status, abort_flag)) return;

    // ---- whole h_t for the next GRU phase; u_t from the summed partials ----
    for (int i = tid; i < nrows * Hb; i += kThreads) {
      const int r = i / Hb, c = i - r * Hb;
      sm[L.h + r * L.ld_h + c] = __builtin_bit_cast(float, coh_load4(hx_rs, hx_el(par, b0 + r, c) * 4u));
    }
    for (int i = tid; i < nrows * E; i += kThreads) {
      const int r = i / E, k = i - r * E;
      float p[8];
      float s = 0.f;
      for (int m0 = 0; m0 < a.nw; m0 += 8) {
#pragma unroll
        for (int m = 0; m < 8; ++m)
          p[m] = m0 + m < a.nw ? __builtin_bit_cast(float, coh_load4(px_rs, px_el(par, b0 + r, m0 + m, k) * 4u)) : 0.f;
#pragma unroll
        for (int m = 0; m < 8; ++m) s += p[m];
      }
      sm[L.u + r * L.ld_e + k] = felu(s + sm[L.b1 + k]);
    }
    __syncthreads();
    // ---- v_t, (mean, std, s_t), then e_{t+1} (every member, whole) ----
    mv_rows<2>(sm + L.u, L.ld_e, sm + L.w2, L.ld_e, sm + L.v, 2 * S, nrows, 2 * S, E);
    __syncthreads();
    for (int i = tid; i < nrows * S; i += kThreads) {
      const int r = i / S, c = i - r * S;
      const int b = b0 + r;
      const float* vr = sm + L.v + r * 2 * S;
      const float mean = vr[c] + sm[L.b2 + c];
      const float sd = fsoftplus(vr[S + c] + sm[L.b2 + S + c]) + a.scale_lb;
      const float st = mean + a.eps[((size_t)b * a.T + t) * S + c] * sd;
      sm[L.sa + r * L.ld_sa + c] = st;
      if (w == 0) {
        const size_t o = ((size_t)b * a.T + t) * S + c;
        a.means[o] = mean;
        a.stds[o] = sd;
        a.states[o] = st;
      }
    }
    if (t + 1 < a.T) {
      for (int i = tid; i < nrows * A; i += kThreads) {
        const int r = i / A, c = i - r * A;
        sm[L.sa + r * L.ld_sa + S + c] = a.actions[((size_t)(b0 + r) * a.T + t + 1) * A + c];
      }
      __syncthreads();
      mv_rows<4>(sm + L.sa, L.ld_sa, sm + L.was, L.ld_sa, sm + L.e, L.ld_e, nrows, E, SA);
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
