// Backward through time of one layer's scan (training), all directions in
// one launch. It walks the forward's steps in the opposite order with the
// chain rule through the cell equations (PyTorch conventions; the backward
// of these cells is what the pytorch/pytorch issue "Integrating CuDNN API
// for LSTMs with projections" discusses in its thread):
//   LSTM  dct = dc + dh o (1 - tanh^2 c);  d(i, f, g, o) pre-activations
//         = (dct g i(1-i), dct c_{t-1} f(1-f), dct i (1-g^2), dh tanh(c) o(1-o));
//         dc_{t-1} = dct f
//   GRU   dn = dh (1 - z), dz = dh (h_{t-1} - n), dan = dn (1 - n^2),
//         dr = dan (W_hn h + b_hn); input side (dr r(1-r), dz z(1-z), dan),
//         hidden side the same with dan r in the n slot; the direct term
//         dh z joins dh_{t-1}
//   dh_{t-1} = W_hh^T (hidden-side gradients) (+ dh z for GRU) + dy_{t-1}.
//
// Work split as in the forward: a group of ns workgroups per (direction,
// batch block), each owning hs hidden units. A member computes the gate
// gradients of its own units, multiplies them by its own W_hh rows (kept
// transposed in LDS) into partial sums over all H columns of dh_{t-1},
// and publishes them; after the group barrier every member sums its own
// columns over all members in a fixed order (deterministic). The reserve
// written by the training forward holds the gate values of every token.
#include "device_common.hpp"
#include "kernels.hpp"
#include "scan_common.hpp"

namespace rnnk {

namespace {

constexpr int kBT = kScanThreads;
constexpr int kMaxEptB = 4;  // owned elements per thread: bb * hs <= 1024
constexpr int kBwdMaxMembersDev = kScanBwdMaxMembers;

__host__ __device__ inline int rup_b(int x, int m) { return (x + m - 1) / m * m; }

struct BwdLds {
  int wt, wt_ld, as, as_ld, acc, acc_ld, lens, flag, total;  // byte offsets, lds in floats
};

__host__ __device__ inline BwdLds bwd_lds(const ScanBwdArgs& a) {
  BwdLds L;
  const int rows = rup_b(a.bb, 16);
  // odd numbers of 16-byte chunks per row keep row-parallel reads on
  // distinct banks
  L.wt_ld = a.kp + 4;
  L.as_ld = a.kp + 4;
  L.acc_ld = a.acc_cols + 4;
  int o = 0;
  L.wt = o;
  o += a.Hp * L.wt_ld * 4;  // wt[c][q * hs + u] = W_hh[q * H + j0 + u][c]
  L.as = o;
  o += rows * L.as_ld * 4;  // own hidden-side gate gradients [rows][gates * hs]
  L.acc = o;
  // one pass of this member's partial sums [rows][acc_cols] (the vector-ALU
  // product only: the MFMA product stores from its accumulators)
  if (a.bb % 16 != 0) o += rows * L.acc_ld * 4;
  L.lens = o;
  o += rup_b(a.bb, 4) * 4;
  L.flag = o;
  o += 16;
  L.total = o;
  return L;
}

__global__ void __launch_bounds__(kBT) scan_bwd_kernel(ScanBwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const BwdLds L = bwd_lds(a);
  const int tid = threadIdx.x;
  const bool gru = a.mode == kGRU;
  const int gates = gru ? 3 : 4;
  const int H = a.H, G = a.G, D = a.D;
  const int R = gru ? 4 * H : 5 * H;
  int grp, s;
  if (a.gpx > 0) {
    const int xcd = blockIdx.x % a.nxcd, slot = blockIdx.x / a.nxcd;
    grp = xcd * a.gpx + slot / a.ns;
    s = slot % a.ns;
  } else {
    grp = blockIdx.x / a.ns;
    s = blockIdx.x % a.ns;
  }
  if (grp >= D * a.nbb) return;  // padding slots of the XCD-aligned layout
  const int d = grp / a.nbb, blk = grp - d * a.nbb;
  const bool rev = d == 1;
  const int b0 = blk * a.bb;
  const int j0 = s * a.hs, hs_act = max(0, min(a.hs, H - j0));
  unsigned* counter = a.counters + (size_t)grp * 16;
  int* abort_flag = reinterpret_cast<int*>(lds + L.flag);
  int* lens = reinterpret_cast<int*>(lds + L.lens);
  float* wt = reinterpret_cast<float*>(lds + L.wt);
  float* As = reinterpret_cast<float*>(lds + L.as);
  float* acc = reinterpret_cast<float*>(lds + L.acc);
  const int tile_rows = rup_b(a.bb, 16);
  const bool use_mfma = a.bb % 16 == 0;

  if (tid == 0) *abort_flag = 0;
  for (int r = tid; r < a.bb; r += kBT) lens[r] = b0 + r < a.B ? (a.lengths ? a.lengths[b0 + r] : a.T) : 0;
  const float* W = a.w_hh[d];
  lds_fill<kBT>(a.Hp * a.kp, [&](int e) {
    const int c = e / a.kp, kk = e - c * a.kp;
    const int q = kk / a.hs, u = kk - q * a.hs;
    return (c < H && q < gates && u < hs_act) ? W[(size_t)(q * H + j0 + u) * H + c] : 0.f;
  }, [&](int e, float v) {
    const int c = e / a.kp, kk = e - c * a.kp;
    wt[c * L.wt_ld + kk] = v;
  });
  for (int e = tid; e < tile_rows * L.as_ld; e += kBT) As[e] = 0.f;
  __syncthreads();
  int maxlen = 0;
  for (int r = 0; r < a.bb; ++r) maxlen = max(maxlen, lens[r]);
  maxlen = __builtin_amdgcn_readfirstlane(maxlen);
  const int nsteps = maxlen;
  // the forward took t = 0 .. maxlen-1 (reverse: maxlen-1 .. 0); walk back
  auto t_of = [&](int k) { return rev ? k : maxlen - 1 - k; };
  const __attribute__((address_space(4))) int* offs = (const __attribute__((address_space(4))) int*)a.offsets;
  auto row_of = [&](int t) -> int { return a.packed ? offs[t] : t * a.B; };

  const uint32_t ex_bytes = (uint32_t)(2 * D * a.ns * a.B * a.Hp) * 4u;
  const __amdgpu_buffer_rsrc_t ex_rs = make_rsrc(a.ex, ex_bytes);
  auto ex_el = [&](int par, int m, int b, int c) -> uint32_t {
    return (uint32_t)((((par * D + d) * a.ns + m) * a.B + b) * a.Hp + c);
  };

  // owned elements: e = tid + i * kBT -> (row r, unit u)
  int er[kMaxEptB], eu[kMaxEptB], elen[kMaxEptB];
  float dcr[kMaxEptB], dhd[kMaxEptB];
#pragma unroll
  for (int i = 0; i < kMaxEptB; ++i) {
    const int e = tid + i * kBT;
    const int r = e / a.hs, u = e - r * a.hs;
    er[i] = r;
    eu[i] = u;
    elen[i] = (e < a.bb * a.hs && u < hs_act && b0 + r < a.B) ? lens[r] : 0;
    dcr[i] = 0.f;
    dhd[i] = 0.f;
  }

  // The loads of a step that do not depend on the exchange (reserved gate
  // values, dy, the previous state, the final-state gradients) are issued one
  // step early, between this workgroup's arrival at the group barrier and its
  // wait, so that their latency overlaps the wait.
  float pre_rv[kMaxEptB][5], pre_dy[kMaxEptB], pre_prev[kMaxEptB], pre_dhn[kMaxEptB], pre_dcn[kMaxEptB];
  auto prefetch = [&](int k) {
    const int t = k < nsteps ? t_of(k) : -1;
    const int tpk = k > 0 ? t_of(k - 1) : -1;
    const int rowbase = t >= 0 ? row_of(t) : 0;
#pragma unroll
    for (int i = 0; i < kMaxEptB; ++i) {
      const int b = b0 + er[i], j = j0 + eu[i];
      const int len = elen[i];
      const bool act = t >= 0 && t < len;
      const bool was = tpk >= 0 && tpk < len;
      const size_t row = (size_t)rowbase + b;
      const bool has_prev = act && (rev ? (t + 1 < len) : (t >= 1));
      const int tp = rev ? t + 1 : t - 1;
      const size_t prow = has_prev ? (size_t)row_of(tp) + b : 0;
#pragma unroll
      for (int q = 0; q < 5; ++q) pre_rv[i][q] = 0.f;
      pre_dy[i] = pre_prev[i] = pre_dhn[i] = pre_dcn[i] = 0.f;
      if (act) {
        const float* rv = a.rsv + (row * D + d) * R + j;
#pragma unroll
        for (int q = 0; q < 5; ++q)
          if (q < (gru ? 4 : 5)) pre_rv[i][q] = rv[q * H];
        pre_dy[i] = a.dy[row * (D * H) + d * H + j];
        if (gru)
          pre_prev[i] = has_prev ? a.y[prow * (D * H) + d * H + j] : (a.h0[d] ? a.h0[d][(size_t)b * H + j] : 0.f);
        else
          pre_prev[i] =
              has_prev ? a.rsv[(prow * D + d) * R + 4 * H + j] : (a.c0[d] ? a.c0[d][(size_t)b * H + j] : 0.f);
        if (!was) {
          pre_dhn[i] = a.dh_n[d] ? a.dh_n[d][(size_t)b * H + j] : 0.f;
          pre_dcn[i] = (!gru && a.dc_n[d]) ? a.dc_n[d][(size_t)b * H + j] : 0.f;
        }
      }
    }
  };

  prefetch(0);
  unsigned nbar = 0;
  for (int k = 0; k <= nsteps; ++k) {
    const int t = k < nsteps ? t_of(k) : -1;
    const int tpk = k > 0 ? t_of(k - 1) : -1;  // the step handled last
    const int rowbase = t >= 0 ? row_of(t) : 0;
#pragma unroll
    for (int i = 0; i < kMaxEptB; ++i) {
      const int r = er[i], u = eu[i], b = b0 + r, j = j0 + u;
      const int len = elen[i];
      const bool act = t >= 0 && t < len;
      const bool was = tpk >= 0 && tpk < len;
      const size_t row = (size_t)rowbase + b;
      float rvv[5];
#pragma unroll
      for (int q = 0; q < 5; ++q) rvv[q] = pre_rv[i][q];
      const float dyv = pre_dy[i], prevv = pre_prev[i], dhn = pre_dhn[i], dcn = pre_dcn[i];
      // recurrent gradient from the previous step's partial sums, summed
      // over the members in order (up to 64 loads in flight)
      float dh_rec = 0.f;
      if (was) {
        float pv[kBwdMaxMembersDev];
#pragma unroll
        for (int m = 0; m < kBwdMaxMembersDev; ++m)
          if (m < a.ns) pv[m] = __builtin_bit_cast(float, coh_load4(ex_rs, ex_el((k - 1) & 1, m, b, j) * 4u));
#pragma unroll
        for (int m = 0; m < kBwdMaxMembersDev; ++m)
          if (m < a.ns) dh_rec += pv[m];
        dh_rec += dhd[i];
      }
      if (was && !act) {  // this row's walk is over: gradients of the initial state
        if (a.dh0[d]) a.dh0[d][(size_t)b * H + j] = dh_rec;
        if (!gru && a.dc0[d]) a.dc0[d][(size_t)b * H + j] = dcr[i];
      }
      if (len == 0 || u >= hs_act) continue;
      if (!act) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (q < gates) As[r * L.as_ld + q * a.hs + u] = 0.f;
        continue;
      }
      const float dh = (was ? dh_rec : dhn) + dyv;
      float* gx = a.dgx + (row * D + d) * G + j;
      if (gru) {
        const float rg = rvv[0], zg = rvv[1], ng = rvv[2], ahn = rvv[3];
        const float hp = prevv;
        const float dn = dh * (1.f - zg);
        const float dz = dh * (hp - ng);
        const float dan = dn * (1.f - ng * ng);
        const float dar = dan * ahn * rg * (1.f - rg);
        const float daz = dz * zg * (1.f - zg);
        gx[0] = dar;
        gx[H] = daz;
        gx[2 * H] = dan;
        float* gh = a.dgh + (row * D + d) * G + j;
        gh[0] = dar;
        gh[H] = daz;
        gh[2 * H] = dan * rg;
        As[r * L.as_ld + u] = dar;
        As[r * L.as_ld + a.hs + u] = daz;
        As[r * L.as_ld + 2 * a.hs + u] = dan * rg;
        dhd[i] = dh * zg;
      } else {
        const float ig = rvv[0], fg = rvv[1], gg = rvv[2], og = rvv[3], c = rvv[4];
        const float dc_in = was ? dcr[i] : dcn;
        const float cp = prevv;
        const float tc = ftanh(c);
        const float dct = dc_in + dh * og * (1.f - tc * tc);
        const float dai = dct * gg * ig * (1.f - ig);
        const float daf = dct * cp * fg * (1.f - fg);
        const float dag = dct * ig * (1.f - gg * gg);
        const float dao = dh * tc * og * (1.f - og);
        dcr[i] = dct * fg;
        gx[0] = dai;
        gx[H] = daf;
        gx[2 * H] = dag;
        gx[3 * H] = dao;
        As[r * L.as_ld + u] = dai;
        As[r * L.as_ld + a.hs + u] = daf;
        As[r * L.as_ld + 2 * a.hs + u] = dag;
        As[r * L.as_ld + 3 * a.hs + u] = dao;
      }
    }
    if (k == nsteps) break;
    lds_barrier();
    // this member's share of W_hh^T (hidden-side gradients), all H columns
    if (use_mfma) {
      // Columns of the recurrent width as the MFMA rows, batch rows as its
      // columns: every lane finishes with four consecutive columns of one
      // batch row and stores them from its accumulator in one 16-byte store
      // (rows past the block or the batch go out of range and are dropped).
      const int lr = tid & 15, lq = (tid & 63) >> 4;
      mm_mfma_epi<float>(lds, L.wt, L.wt_ld, L.as, L.as_ld, a.Hp / 16, tile_rows / 16, a.kp,
                         [&](int m, int n, const f32x4& c) {
                           const int r = n * 16 + lr;
                           const uint32_t off = (r < a.bb && b0 + r < a.B)
                                                    ? ex_el(k & 1, s, b0 + r, m * 16 + 4 * lq) * 4u
                                                    : 0x80000000u;
                           coh_store16(ex_rs, off, __builtin_bit_cast(u32x4, c));
                         });
    } else {
      // in passes of acc_cols columns through the LDS accumulator
      const int cpr = a.acc_cols / 4;
      for (int c0 = 0; c0 < a.Hp; c0 += a.acc_cols) {
        mm_valu<float>(lds, L.as, L.as_ld, L.wt + c0 * L.wt_ld * 4, L.wt_ld, acc, L.acc_ld, a.bb, a.acc_cols, a.kp);
        lds_barrier();
        for (int e = tid; e < a.bb * cpr; e += kBT) {
          const int r = e / cpr, cc = e - r * cpr;
          if (b0 + r < a.B)
            coh_store16(ex_rs, ex_el(k & 1, s, b0 + r, c0 + 4 * cc) * 4u,
                        *reinterpret_cast<const u32x4*>(acc + r * L.acc_ld + 4 * cc));
        }
        if (c0 + a.acc_cols < a.Hp) lds_barrier();  // the accumulator is reused
      }
    }
    ++nbar;
    group_arrive(counter);
    prefetch(k + 1);
    if (!group_wait(counter, nbar * a.ns, a.status, abort_flag)) return;
  }
}


// ---------------------------------------------------------------------------
// LSTMP: the recurrent input is the projection h = W_hr m (width P). Per
// step, two exchanges as in the forward:
//   1. each member sums, for its own ps projection outputs, every member's
//      partial W_hh^T dG of the previous step, adds dy, and publishes dh_t;
//   2. after the first barrier every member reads the whole dh_t, forms
//      dm = W_hr^T dh_t for its own units, runs the cell backward with dm
//      in place of dh, and publishes its partial W_hh^T dG over P.
// ---------------------------------------------------------------------------
struct BwdPLds {
  int wht, wht_ld, wrt, wrt_ld, as, as_ld, dht, dht_ld, acc1, acc1_ld, acc2, acc2_ld, lens, flag, total;
};

__host__ __device__ inline BwdPLds bwdp_lds(const ScanBwdArgs& a) {
  BwdPLds L;
  const int rows = rup_b(a.bb, 16), hsp = rup_b(a.hs, 16);
  L.wht_ld = a.kp + 4;
  L.wrt_ld = a.Pp + 4;
  L.as_ld = a.kp + 4;
  L.dht_ld = a.Pp + 4;
  L.acc1_ld = a.Pp + 4;
  L.acc2_ld = hsp + 4;
  int o = 0;
  L.wht = o;
  o += a.Pp * L.wht_ld * 4;  // wht[p][q * hs + u] = W_hh[q * H + j0 + u][p]
  L.wrt = o;
  o += hsp * L.wrt_ld * 4;   // wrt[u][p] = W_hr[p][j0 + u]
  L.as = o;
  o += rows * L.as_ld * 4;   // own gate gradients
  L.dht = o;
  o += rows * L.dht_ld * 4;  // the whole dh_t of the block
  L.acc1 = o;
  o += rows * L.acc1_ld * 4;  // partial W_hh^T dG over P
  L.acc2 = o;
  o += rows * L.acc2_ld * 4;  // dm of the own units
  L.lens = o;
  o += rup_b(a.bb, 4) * 4;
  L.flag = o;
  o += 16;
  L.total = o;
  return L;
}

__global__ void __launch_bounds__(kBT) scan_bwd_proj_kernel(ScanBwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const BwdPLds L = bwdp_lds(a);
  const int tid = threadIdx.x;
  const int H = a.H, P = a.P, G = a.G, D = a.D, R = 5 * H;
  int grp, s;
  if (a.gpx > 0) {
    const int xcd = blockIdx.x % a.nxcd, slot = blockIdx.x / a.nxcd;
    grp = xcd * a.gpx + slot / a.ns;
    s = slot % a.ns;
  } else {
    grp = blockIdx.x / a.ns;
    s = blockIdx.x % a.ns;
  }
  if (grp >= D * a.nbb) return;
  const int d = grp / a.nbb, blk = grp - d * a.nbb;
  const bool rev = d == 1;
  const int b0 = blk * a.bb;
  const int j0 = s * a.hs, hs_act = max(0, min(a.hs, H - j0));
  const int p0 = s * a.ps, ps_act = max(0, min(a.ps, P - p0));
  const int hsp = rup_b(a.hs, 16);
  unsigned* counter = a.counters + (size_t)grp * 16;
  int* abort_flag = reinterpret_cast<int*>(lds + L.flag);
  int* lens = reinterpret_cast<int*>(lds + L.lens);
  float* wht = reinterpret_cast<float*>(lds + L.wht);
  float* wrt = reinterpret_cast<float*>(lds + L.wrt);
  float* As = reinterpret_cast<float*>(lds + L.as);
  float* acc1 = reinterpret_cast<float*>(lds + L.acc1);
  float* acc2 = reinterpret_cast<float*>(lds + L.acc2);
  const int tile_rows = rup_b(a.bb, 16);
  const bool use_mfma = a.bb % 16 == 0;

  if (tid == 0) *abort_flag = 0;
  for (int r = tid; r < a.bb; r += kBT) lens[r] = b0 + r < a.B ? (a.lengths ? a.lengths[b0 + r] : a.T) : 0;
  const float* Whh = a.w_hh[d];
  const float* Whr = a.w_hr[d];
  lds_fill<kBT>(a.Pp * a.kp, [&](int e) {
    const int p = e / a.kp, kk = e - p * a.kp;
    const int q = kk / a.hs, u = kk - q * a.hs;
    return (p < P && q < 4 && u < hs_act) ? Whh[(size_t)(q * H + j0 + u) * P + p] : 0.f;
  }, [&](int e, float v) {
    const int p = e / a.kp, kk = e - p * a.kp;
    wht[p * L.wht_ld + kk] = v;
  });
  lds_fill<kBT>(hsp * a.Pp, [&](int e) {
    const int u = e / a.Pp, p = e - u * a.Pp;
    return (u < hs_act && p < P) ? Whr[(size_t)p * H + j0 + u] : 0.f;
  }, [&](int e, float v) {
    const int u = e / a.Pp, p = e - u * a.Pp;
    wrt[u * L.wrt_ld + p] = v;
  });
  for (int e = tid; e < tile_rows * L.as_ld; e += kBT) As[e] = 0.f;
  const __amdgpu_buffer_rsrc_t ex2_rs = make_rsrc(a.ex2, (uint32_t)(D * a.B * a.Pp) * 4u);
  if (s == 0) {  // the padding columns of this block's dh_t rows read as zero
    for (int e = tid; e < a.bb * (a.Pp - P); e += kBT) {
      const int r = e / (a.Pp - P), p = P + (e - r * (a.Pp - P));
      if (b0 + r < a.B) coh_store4(ex2_rs, (uint32_t)((d * a.B + b0 + r) * a.Pp + p) * 4u, 0u);
    }
  }
  __syncthreads();
  int maxlen = 0;
  for (int r = 0; r < a.bb; ++r) maxlen = max(maxlen, lens[r]);
  maxlen = __builtin_amdgcn_readfirstlane(maxlen);
  const int nsteps = maxlen;
  auto t_of = [&](int k) { return rev ? k : maxlen - 1 - k; };
  const __attribute__((address_space(4))) int* offs = (const __attribute__((address_space(4))) int*)a.offsets;
  auto row_of = [&](int t) -> int { return a.packed ? offs[t] : t * a.B; };
  const __amdgpu_buffer_rsrc_t ex_rs = make_rsrc(a.ex, (uint32_t)(2 * D * a.ns * a.B * a.Pp) * 4u);
  auto ex_el = [&](int par, int m, int b, int c) -> uint32_t {
    return (uint32_t)((((par * D + d) * a.ns + m) * a.B + b) * a.Pp + c);
  };

  float dcr[kMaxEptB];
#pragma unroll
  for (int i = 0; i < kMaxEptB; ++i) dcr[i] = 0.f;

  unsigned nbar = 0;
  for (int k = 0; k <= nsteps; ++k) {
    const int t = k < nsteps ? t_of(k) : -1;
    const int tpk = k > 0 ? t_of(k - 1) : -1;
    const int rowbase = t >= 0 ? row_of(t) : 0;
    // stage 1: own projection outputs of dh_t
#pragma unroll
    for (int i = 0; i < kMaxEptB; ++i) {
      const int e = tid + i * kBT;
      const int r = e / a.ps, pp = e - r * a.ps;
      const int b = b0 + r, p = p0 + pp;
      const int len = (e < a.bb * a.ps && pp < ps_act && b < a.B) ? lens[r] : 0;
      const bool act = t >= 0 && t < len;
      const bool was = tpk >= 0 && tpk < len;
      const size_t row = (size_t)rowbase + b;
      const float dyv = act ? a.dy[row * (D * P) + d * P + p] : 0.f;
      const float dhn = (act && !was && a.dh_n[d]) ? a.dh_n[d][(size_t)b * P + p] : 0.f;
      float dh_rec = 0.f;
      if (was) {
        float pv[kBwdMaxMembersDev];
#pragma unroll
        for (int m = 0; m < kBwdMaxMembersDev; ++m)
          if (m < a.ns) pv[m] = __builtin_bit_cast(float, coh_load4(ex_rs, ex_el((k - 1) & 1, m, b, p) * 4u));
#pragma unroll
        for (int m = 0; m < kBwdMaxMembersDev; ++m)
          if (m < a.ns) dh_rec += pv[m];
      }
      if (was && !act && a.dh0[d]) a.dh0[d][(size_t)b * P + p] = dh_rec;
      if (act) {
        const float dh = (was ? dh_rec : dhn) + dyv;
        a.dh[(row * D + d) * P + p] = dh;
        coh_store4(ex2_rs, (uint32_t)((d * a.B + b) * a.Pp + p) * 4u, __builtin_bit_cast(uint32_t, dh));
      }
    }
    // rows whose walk ended: the cell-state gradient of the initial state
#pragma unroll
    for (int i = 0; i < kMaxEptB; ++i) {
      const int e = tid + i * kBT;
      const int r = e / a.hs, u = e - r * a.hs;
      const int len = (e < a.bb * a.hs && u < hs_act && b0 + r < a.B) ? lens[r] : 0;
      const bool act = t >= 0 && t < len, was = tpk >= 0 && tpk < len;
      if (was && !act && a.dc0[d]) a.dc0[d][(size_t)(b0 + r) * H + j0 + u] = dcr[i];
    }
    if (k == nsteps) break;
    ++nbar;
    if (!group_barrier(counter, nbar * a.ns, a.status, abort_flag)) return;
    // stage 2: the whole dh_t, dm = W_hr^T dh_t for the own units
    load_tile_coherent<float>(ex2_rs, (uint32_t)((d * a.B + b0) * a.Pp), a.Pp, b0, a.B, use_mfma ? tile_rows : a.bb,
                              a.Pp, lds, L.dht, L.dht_ld);
    __syncthreads();
    if (use_mfma)
      mm_mfma<float>(lds, L.dht, L.dht_ld, L.wrt, L.wrt_ld, acc2, L.acc2_ld, tile_rows / 16, hsp / 16, a.Pp);
    else
      mm_valu<float>(lds, L.dht, L.dht_ld, L.wrt, L.wrt_ld, acc2, L.acc2_ld, a.bb, hsp, a.Pp);
    __syncthreads();
    // stage 3: the cell backward of the own units with dm
#pragma unroll
    for (int i = 0; i < kMaxEptB; ++i) {
      const int e = tid + i * kBT;
      const int r = e / a.hs, u = e - r * a.hs;
      const int b = b0 + r, j = j0 + u;
      const int len = (e < a.bb * a.hs && u < hs_act && b < a.B) ? lens[r] : 0;
      if (len == 0) continue;
      const bool act = t < len, was = tpk >= 0 && tpk < len;
      if (!act) {
#pragma unroll
        for (int q = 0; q < 4; ++q) As[r * L.as_ld + q * a.hs + u] = 0.f;
        continue;
      }
      const size_t row = (size_t)rowbase + b;
      const bool has_prev = rev ? (t + 1 < len) : (t >= 1);
      const int tp = rev ? t + 1 : t - 1;
      const float* rv = a.rsv + (row * D + d) * R + j;
      const float ig = rv[0], fg = rv[H], gg = rv[2 * H], og = rv[3 * H], c = rv[4 * H];
      const float cp = has_prev ? a.rsv[(((size_t)row_of(tp) + b) * D + d) * R + 4 * H + j]
                                : (a.c0[d] ? a.c0[d][(size_t)b * H + j] : 0.f);
      const float dc_in = was ? dcr[i] : (a.dc_n[d] ? a.dc_n[d][(size_t)b * H + j] : 0.f);
      const float dm = acc2[r * L.acc2_ld + u];
      const float tc = ftanh(c);
      const float dct = dc_in + dm * og * (1.f - tc * tc);
      const float dai = dct * gg * ig * (1.f - ig);
      const float daf = dct * cp * fg * (1.f - fg);
      const float dag = dct * ig * (1.f - gg * gg);
      const float dao = dm * tc * og * (1.f - og);
      dcr[i] = dct * fg;
      float* gx = a.dgx + (row * D + d) * G + j;
      gx[0] = dai;
      gx[H] = daf;
      gx[2 * H] = dag;
      gx[3 * H] = dao;
      As[r * L.as_ld + u] = dai;
      As[r * L.as_ld + a.hs + u] = daf;
      As[r * L.as_ld + 2 * a.hs + u] = dag;
      As[r * L.as_ld + 3 * a.hs + u] = dao;
    }
    __syncthreads();
    // stage 4: this member's partial W_hh^T dG over the P columns
    if (use_mfma)
      mm_mfma<float>(lds, L.as, L.as_ld, L.wht, L.wht_ld, acc1, L.acc1_ld, tile_rows / 16, a.Pp / 16, a.kp);
    else
      mm_valu<float>(lds, L.as, L.as_ld, L.wht, L.wht_ld, acc1, L.acc1_ld, a.bb, a.Pp, a.kp);
    __syncthreads();
    const int cpr = a.Pp / 4;
    for (int e = tid; e < a.bb * cpr; e += kBT) {
      const int r = e / cpr, cc = e - r * cpr;
      if (b0 + r < a.B)
        coh_store16(ex_rs, ex_el(k & 1, s, b0 + r, 4 * cc) * 4u,
                    *reinterpret_cast<const u32x4*>(acc1 + r * L.acc1_ld + 4 * cc));
    }
    ++nbar;
    if (!group_barrier(counter, nbar * a.ns, a.status, abort_flag)) return;
  }
}

__global__ void __launch_bounds__(256) mgather_kernel(const float* rsv, int D, int d, int H, long long rows,
                                                      float* out) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= rows * H) return;
  const long long row = e / H;
  const int j = (int)(e - row * H);
  const float* rv = rsv + (row * D + d) * (5 * H) + j;
  out[e] = rv[3 * H] * tanhf(rv[4 * H]);
}

}  // namespace

int scan_bwd_lds_bytes(const ScanBwdArgs& a) { return a.mode == kLSTMP ? bwdp_lds(a).total : bwd_lds(a).total; }

hipError_t launch_mgather(const float* rsv, int D, int d, int H, long long rows, float* out, hipStream_t stream) {
  const long long n = rows * H;
  if (n <= 0) return hipSuccess;
  launch_kernel(mgather_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, rsv, D, d, H, rows, out);
  return hipGetLastError();
}

hipError_t launch_scan_bwd(const ScanBwdArgs& a, hipStream_t stream) {
  const bool proj = a.mode == kLSTMP;
  const int lds = scan_bwd_lds_bytes(a);
  const void* fn = proj ? (const void*)scan_bwd_proj_kernel : (const void*)scan_bwd_kernel;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  const int groups = a.D * a.nbb;
  const int grid = a.gpx > 0 ? a.nxcd * a.gpx * a.ns : groups * a.ns;
  if (proj)
    launch_kernel(scan_bwd_proj_kernel, dim3(grid), dim3(kBT), lds, stream, a);
  else
    launch_kernel(scan_bwd_kernel, dim3(grid), dim3(kBT), lds, stream, a);
  return hipGetLastError();
}

}  // namespace rnnk
