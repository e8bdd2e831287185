// Host side of the C ABI declared in include/rnn.h: argument validation,
// workspace layout, launch planning and the enqueue of the kernels.
//
// Everything a call needs is derived from its arguments; the only state kept
// between calls is a per-device cache of immutable facts (architecture name,
// compute-unit count), filled once under a lock.
#include <hip/hip_runtime.h>
#include <rocprofiler-sdk-roctx/roctx.h>

#include <algorithm>
#include <limits>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/rnn.h"
#include "kernels.hpp"

using namespace rnnk;

rnnk::LaunchEvents& rnnk::launch_events() {
  thread_local LaunchEvents ev;
  return ev;
}

namespace {

constexpr size_t kAlign = 256;
// 16 zero bytes inside the status block of the workspace (cleared at the
// start of every call, never written afterwards): the GEMM's stand-in for
// rows past the matrix.
constexpr size_t kZeroChunk = 128;
constexpr int kMaxLds = 160 * 1024;
constexpr int kCounterBytes = 64;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int rup(int x, int m) { return (x + m - 1) / m * m; }
int cdiv(int x, int m) { return (x + m - 1) / m; }

// ---------------------------------------------------------------------------
// Device facts
// ---------------------------------------------------------------------------
struct DeviceInfo {
  bool ok = false;
  int cus = 0;
  int xcds = 1;
};

constexpr int kMaxDevices = 64;
std::mutex g_dev_mu;
DeviceInfo g_dev[kMaxDevices];
bool g_dev_init[kMaxDevices] = {};

int current_device_info(DeviceInfo* out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return RNN_E_DEVICE;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (!g_dev_init[dev]) {
    hipDeviceProp_t p;
    DeviceInfo info;
    if (hipGetDeviceProperties(&p, dev) == hipSuccess) {
      info.ok = std::strncmp(p.gcnArchName, "gfx950", 6) == 0;
      info.cus = p.multiProcessorCount;
      int x = 0;
      if (hipDeviceGetAttribute(&x, hipDeviceAttributeNumberOfXccs, dev) == hipSuccess && x > 0) info.xcds = x;
    }
    g_dev[dev] = info;
    g_dev_init[dev] = true;
  }
  *out = g_dev[dev];
  return out->ok ? RNN_OK : RNN_E_DEVICE;
}

// ---------------------------------------------------------------------------
// Validation
// ---------------------------------------------------------------------------
bool is_rnn_mode(int m) { return m == RNN_MODE_LSTM || m == RNN_MODE_GRU || m == RNN_MODE_LSTMP; }
bool is_rssm(int m) { return m == RNN_MODE_RSSM_PRIOR || m == RNN_MODE_RSSM_ACTOR; }

int validate_desc(const RnnDesc* d) {
  if (!d) return RNN_E_NULL;
  for (int r : d->reserved)
    if (r != 0) return RNN_E_SHAPE;
  if (d->gx_dtype != RNN_GX_AS_DTYPE && d->gx_dtype != RNN_GX_F32) return RNN_E_SHAPE;
  if (d->layer_pipeline < RNN_PIPE_AUTO || d->layer_pipeline > RNN_PIPE_ON) return RNN_E_SHAPE;
  if (d->placement < 0 || d->placement > 2) return RNN_E_SHAPE;
  if (d->weights < 0 || d->weights > 2) return RNN_E_SHAPE;
  if (d->dtype != RNN_DTYPE_F32 && d->dtype != RNN_DTYPE_BF16) return RNN_E_UNSUPPORTED;
  if (d->T < 1 || d->B < 1) return RNN_E_SHAPE;
  if (d->tile_batch < 0 || d->tile_hidden < 0) return RNN_E_SHAPE;
  if (d->mode == RNN_MODE_RSSM_ACTOR ? d->actor_dim < 1 : d->actor_dim != 0) return RNN_E_SHAPE;
  if (is_rssm(d->mode)) {
    if (d->layout != RNN_LAYOUT_BATCH_MAJOR) return RNN_E_UNSUPPORTED;
    if (d->dtype != RNN_DTYPE_F32) return RNN_E_UNSUPPORTED;
    if (d->num_layers != 1 || d->bidirectional != 0 || d->proj_size != 0) return RNN_E_UNSUPPORTED;
    if (!d->has_bias) return RNN_E_UNSUPPORTED;
    if (d->state_dim < 1 || d->action_dim < 1 || d->embed_dim < 1 || d->belief_dim < 1) return RNN_E_SHAPE;
    if (!std::isfinite(d->scale_lb)) return RNN_E_SHAPE;
    if (d->clip != 0) return RNN_E_UNSUPPORTED;
    if (d->gx_dtype != RNN_GX_AS_DTYPE) return RNN_E_UNSUPPORTED;  // no hoisted G_x
    if (d->layer_pipeline != 0) return RNN_E_UNSUPPORTED;          // one layer
    const double big = (double)d->B * d->T * std::max({d->state_dim, d->belief_dim, d->action_dim});
    if (big > 2e9) return RNN_E_SHAPE;
    const double wa1 = (double)d->actor_dim * (d->state_dim + d->belief_dim);
    if (wa1 > 2e9) return RNN_E_SHAPE;
    return RNN_OK;
  }
  if (!is_rnn_mode(d->mode)) return RNN_E_UNSUPPORTED;
  if (d->clip & ~(RNN_CLIP_CELL | RNN_CLIP_PROJ)) return RNN_E_UNSUPPORTED;
  if ((d->clip & RNN_CLIP_CELL) && d->mode == RNN_MODE_GRU) return RNN_E_UNSUPPORTED;
  if ((d->clip & RNN_CLIP_PROJ) && d->mode != RNN_MODE_LSTMP) return RNN_E_UNSUPPORTED;
  if ((d->clip & RNN_CLIP_CELL) &&
      (std::isnan(d->cell_clip_lo) || std::isnan(d->cell_clip_hi) || !(d->cell_clip_lo <= d->cell_clip_hi)))
    return RNN_E_SHAPE;
  if ((d->clip & RNN_CLIP_PROJ) && !(d->proj_clip >= 0.f)) return RNN_E_SHAPE;
  if (d->layout != RNN_LAYOUT_PADDED && d->layout != RNN_LAYOUT_PACKED) return RNN_E_UNSUPPORTED;
  if ((d->mode == RNN_MODE_LSTMP) != (d->proj_size > 0)) return RNN_E_UNSUPPORTED;
  if (d->proj_size < 0) return RNN_E_SHAPE;
  if (d->num_layers < 1 || d->num_layers > RNN_MAX_LAYERS) return RNN_E_SHAPE;
  if (d->bidirectional != 0 && d->bidirectional != 1) return RNN_E_SHAPE;
  if (d->input_size < 1 || d->hidden_size < 1) return RNN_E_SHAPE;
  // sizes in double: the products of valid int fields can overflow int
  const double D = d->bidirectional ? 2 : 1;
  const double G = (d->mode == RNN_MODE_GRU ? 3.0 : 4.0) * d->hidden_size;
  const double K = d->mode == RNN_MODE_LSTMP ? d->proj_size : d->hidden_size;
  const double rows = (double)d->T * d->B;
  const double in_max = std::max((double)d->input_size, D * K);
  if (rows * D * G > 2e9 || rows * in_max > 2e9) return RNN_E_SHAPE;
  if ((double)d->hidden_size * in_max > 2e9) return RNN_E_SHAPE;
  return RNN_OK;
}

int validate_lengths(const RnnDesc* d, const int32_t* len, long long* n_tok, int* t_max) {
  if (is_rssm(d->mode)) {
    *n_tok = (long long)d->T * d->B;
    *t_max = d->T;
    return RNN_OK;
  }
  if (!len) {
    if (d->layout == RNN_LAYOUT_PACKED) return RNN_E_LENGTHS;
    *n_tok = (long long)d->T * d->B;
    *t_max = d->T;
    return RNN_OK;
  }
  long long s = 0;
  int mx = 0;
  for (int b = 0; b < d->B; ++b) {
    if (len[b] < 1 || len[b] > d->T) return RNN_E_LENGTHS;
    if (d->layout == RNN_LAYOUT_PACKED && b > 0 && len[b] > len[b - 1]) return RNN_E_LENGTHS;
    s += len[b];
    mx = std::max(mx, (int)len[b]);
  }
  *n_tok = s;
  *t_max = mx;
  return RNN_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// ---------------------------------------------------------------------------
// Workspace layout (independent of the launch plan, so rnn_workspace_bytes
// needs no device)
// ---------------------------------------------------------------------------
struct WsLayout {
  size_t status, counters, ints, gx, inter0, inter1, ex_h, ex_p, xid, ring_end, gpart, total;
  size_t counters_bytes;
  int n_ints;
  // forward scan exchange, one block per layer: XCD ids, h ring, m ring
  size_t ex, ex_layer, ex_hx, ex_mx;  // first block, block size, ring offsets in a block
  // layer pipelining (when the descriptor allows it): G_x of one time chunk
  // for each layer above the first (layer 0's is all in gx), and the state
  // carried between chunks (h in the storage dtype [B, K]; fp32 h and c
  // [B, H]), two sets [2][num_layers] by parity
  size_t gxp, gxp_layer, sth, sth_layer, sthf, stcf, stf_layer;
};

struct Dims {
  int D, G, K, Kp, Hp, gates, esize;
  long long rows;  // Gx / y rows per layer
};

Dims dims_of(const RnnDesc* d, long long n_tok) {
  Dims m{};
  m.D = d->bidirectional ? 2 : 1;
  m.gates = d->mode == RNN_MODE_GRU ? 3 : 4;
  m.G = m.gates * d->hidden_size;
  m.K = d->mode == RNN_MODE_LSTMP ? d->proj_size : d->hidden_size;
  m.Kp = rup(m.K, 32);
  m.Hp = rup(d->hidden_size, 32);
  m.esize = d->dtype == RNN_DTYPE_BF16 ? 2 : 4;
  m.rows = d->layout == RNN_LAYOUT_PACKED ? n_tok : (long long)d->T * d->B;
  return m;
}

// Columns of one member's partial-sum row in the RSSM exchange: W_1 h
// (E, padded to 4), then the actor's W_a1[:, S:] h (Ea, padded to 4).
int rssm_ex_cols(const RnnDesc* d) { return rup(d->embed_dim, 4) + rup(d->actor_dim, 4); }

bool use_wave_scan(const RnnDesc* d, const Dims& m);

// Bytes per element of the hoisted G_x: the storage dtype's unless fp32 is
// requested, or the one-wave scan runs the layer (its G_x reads are one
// word per lane per step, where bf16 saves nothing and costs the widening).
bool small_scan_shape(const RnnDesc* d, const Dims& m);

int gx_esize(const RnnDesc* d, const Dims& m) {
  return d->dtype == RNN_DTYPE_BF16 && d->gx_dtype == RNN_GX_AS_DTYPE && !use_wave_scan(d, m) &&
                 !small_scan_shape(d, m)
             ? 2
             : 4;
}

// Per-layer exchange regions of the forward scan (aligned sizes, so the
// layers' regions stay aligned).
size_t xid_layer_bytes() { return align_up((size_t)kScanMaxWorkgroups * 4, kAlign); }
size_t hx_ring_bytes(const RnnDesc* d, const Dims& m) {
  size_t b = (size_t)kScanRingSlots * m.D * d->B * m.Kp * m.esize;
  // kernel 2c's ring: fp32, rows of 64 x its K chunks per lane
  if (small_scan_shape(d, m))
    b = std::max(b, (size_t)kScanRingSlots * m.D * d->B * 64 * scan_small_chunks(m.K) * 4);
  return align_up(b, kAlign);
}
size_t mx_ring_bytes(const RnnDesc* d, const Dims& m) {
  return align_up((size_t)kScanRingSlots * m.D * d->B * m.Hp * m.esize, kAlign);
}

// Layer pipelining: a unidirectional, padded, fixed-length stack of >= 2
// LSTM / GRU / LSTMP layers (not the one-wave scan) can be scanned in time
// chunks, one launch per wave covering a chunk of every layer. The chunk
// count balances the fixed cost of a wave (~40 us measured: exchange reset,
// chunk product, scan launch) against the pipeline's fill and drain (L - 1
// chunks): (n + L - 1) (F + s T / n) is least at n = sqrt((L - 1) s T / F),
// i.e. sqrt((L - 1) T / 8) for steps of s ~ 5 us. The shape depends only on
// the descriptor, so the workspace size does too.
constexpr int kPipeMinChunk = 32;  // steps per chunk at least
struct PipeShape {
  bool on;
  int chunk, nchunks;
};
PipeShape pipe_shape(const RnnDesc* d, bool has_lengths, const Dims& m) {
  PipeShape ps{false, 0, 0};
  if (d->layer_pipeline == RNN_PIPE_OFF || d->num_layers < 2 || d->bidirectional ||
      d->layout != RNN_LAYOUT_PADDED || has_lengths || !is_rnn_mode(d->mode) || use_wave_scan(d, m))
    return ps;
  const long n0 = std::lround(std::sqrt((d->num_layers - 1) * (double)d->T / 8.0));
  const int chunk = std::max(kPipeMinChunk, cdiv(d->T, (int)std::max(2L, n0)));
  const int n = cdiv(d->T, chunk);
  if (n < 2) return ps;
  return PipeShape{true, chunk, n};
}

WsLayout layout_of(const RnnDesc* d, long long n_tok, bool has_lengths) {
  WsLayout w{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes, kAlign);
    return at;
  };
  w.status = take(kAlign);
  if (is_rssm(d->mode)) {
    w.counters_bytes = (size_t)d->B * kCounterBytes;
    w.counters = take(w.counters_bytes);
    // exchange buffers sized for either RSSM kernel: ping-pong (kernel 3)
    // or a ring of write-once slots (kernel 3b), and the members' XCC ids
    const int Hbp = rup(d->belief_dim, 4), Ep = rssm_ex_cols(d);
    const int slots = std::max(2, rssm_ring_slots());
    w.xid = take((size_t)d->B * kRssmMaxMembers * 4);
    w.ex_h = take((size_t)slots * d->B * Hbp * 4);
    w.ex_p = take((size_t)slots * d->B * kRssmMaxMembers * Ep * 4);
    w.total = o;
    return w;
  }
  const Dims m = dims_of(d, n_tok);
  w.counters_bytes = (size_t)d->num_layers * m.D * d->B * kCounterBytes;
  w.counters = take(w.counters_bytes);
  w.n_ints = has_lengths ? d->B + d->T + 1 : 0;
  w.ints = take((size_t)std::max(w.n_ints, 1) * 4);
  // (16 bytes of slack: a bf16 element is read with the aligned word that holds it)
  w.gx = take((size_t)m.rows * m.D * m.G * gx_esize(d, m) + 16);
  const size_t inter = (size_t)m.rows * m.D * m.K * m.esize;
  w.inter0 = d->num_layers > 1 ? take(inter) : 0;
  w.inter1 = d->num_layers > 2 ? take(inter) : 0;
  // the forward scan's exchange, one block per layer (the members' XCD ids,
  // the h ring and, LSTMP, the m ring), all sentinel-filled by one fill
  // before the first layer (per layer and chunk when pipelined)
  w.ex_hx = xid_layer_bytes();
  w.ex_mx = w.ex_hx + hx_ring_bytes(d, m);
  w.ex_layer = w.ex_mx + (d->mode == RNN_MODE_LSTMP ? mx_ring_bytes(d, m) : 0);
  w.ex = take(w.ex_layer * d->num_layers);
  w.ring_end = o;
  const PipeShape ps = pipe_shape(d, has_lengths, m);
  if (ps.on) {
    w.gxp_layer = align_up((size_t)ps.chunk * d->B * m.G * gx_esize(d, m) + 16, kAlign);
    w.gxp = take(w.gxp_layer * (d->num_layers - 1));  // layers 1 .. L-1 (layer 0 uses gx)
    // two sets, by chunk parity: a chunk reads one and writes the other
    w.sth_layer = align_up((size_t)d->B * m.K * m.esize, kAlign);
    w.sth = take(w.sth_layer * d->num_layers * 2);
    w.stf_layer = align_up((size_t)d->B * d->hidden_size * 4, kAlign);
    w.sthf = take(w.stf_layer * d->num_layers * 2);
    w.stcf = take(w.stf_layer * d->num_layers * 2);
  }
  // split-K partial products of the input GEMMs with few output tiles
  size_t gpart = 0;
  for (int l = 0; l < d->num_layers; ++l) {
    const int in_l = l == 0 ? d->input_size : m.D * m.K;
    const int sp = gemm_xw_splits(m.rows, m.D * m.G, in_l, d->dtype == RNN_DTYPE_BF16);
    if (sp > 1) gpart = std::max(gpart, (size_t)sp * (size_t)m.rows * m.D * m.G * 4);
  }
  w.gpart = gpart ? take(gpart) : 0;
  w.total = o;
  return w;
}

// ---------------------------------------------------------------------------
// Launch planning
// ---------------------------------------------------------------------------
// Per-step time model (microseconds) from measurements on MI355X: a group
// barrier with device-coherent exchange costs ~0.65 us plus 6-9 ns per member;
// the exchange read streams at roughly 100 GB/s per workgroup; MFMA and LDS
// rates are those of one compute unit at 2.4 GHz.
double barrier_us(int members) { return 0.65 + 0.009 * members; }
// The forward scan's step pays less per member: a sweep of its launch shapes
// measured LSTMP (B=32, H=1024, P=256) at 7.15 ms per layer with 32 members
// of 32 units against 7.80 ms with 16 of 64, while the best GRU, var-len and
// B=1 shapes stay where they were with 6 ns per member.
double scan_barrier_us(int members) { return 0.65 + 0.006 * members; }

double mm_us(bool mfma, int esize, int rows, int cols, int kp) {
  // (LDS-resident weights; the VALU form is bound by LDS latency, measured
  // at ~1 us plus ~8 MAC/clk)
  if (mfma) {
    const double tiles = (double)(rows / 16) * cdiv(cols, 16);
    double mf_cycles, lds_bytes;
    if (esize == 2) {
      mf_cycles = tiles * (kp / 32) * 16.0 / 4.0;
      lds_bytes = tiles * (kp / 32) * 2048.0;
    } else {
      mf_cycles = tiles * (kp / 4) * 32.0 / 4.0;
      lds_bytes = tiles * (kp / 16) * 2048.0;
    }
    // measured about twice this bound (LDS latency between dependent steps)
    return 2.0 * std::max(mf_cycles, lds_bytes / 128.0) / 2400.0;
  }
  return 1.0 + (double)rows * cols * kp / 8.0 / 2400.0;
}

struct ScanPlan {
  int bb, hs, ns, ps, nbb, gpx, lds;
  int wreg, rnt, rks, rcpt;  // register-resident W_hh layout (ScanArgs)
  int pnt, pks, pcpt;        // LSTMP projection product layout (ScanArgs)
};

// Grid of a plan over `groups_per_nbb` = layer slots x directions.
int scan_grid(const ScanPlan& p, int slots_x_dirs, int xcds) {
  return p.gpx > 0 ? xcds * p.gpx * p.ns : slots_x_dirs * p.nbb * p.ns;
}

// Register layout of a slice of ncw W_hh rows (padded to 16) for a batch
// block of bb rows, or false when none fits kScanRegChunks 16-byte chunks
// per lane. MFMA (bb a multiple of 16): rnt column tiles per wave, rks waves
// per tile set splitting K, rcpt chunks per tile (a multiple of 4). VALU:
// one output column per thread over one of rks K slices of rcpt chunks.
// MFMA wave layout of an ncw-row product over Kp: the four waves cover
// 4 * nt / ks column tiles (>= the ncw / 16 needed; extra ones are zero
// rows), ks waves splitting K into cpt chunks each (a multiple of 4), at most
// max_chunks chunks (nt * cpt) per lane. Fewest padded tiles first, then the
// least K split.
bool mfma_split(int ncw, int Kp, int esize, int max_chunks, int* rnt, int* rks, int* rcpt) {
  const int ct = ncw / 16, nch = Kp / (esize == 2 ? 32 : 16);
  int best_cols = 1 << 30;
  bool ok = false;
  for (int ks = 1; ks <= 4; ks *= 2) {
    for (int nt = 1; nt <= 4; nt *= 2) {
      const int cover = 4 * nt / ks;
      if (4 * nt % ks != 0 || cover < ct) continue;
      if (nch % ks != 0) continue;
      const int cpt = nch / ks;
      if (cpt % 4 != 0 || cpt * nt > max_chunks) continue;
      if (cover < best_cols) {
        best_cols = cover;
        *rnt = nt; *rks = ks; *rcpt = cpt;
        ok = true;
      }
    }
  }
  return ok;
}

bool reg_layout(int bb, int ncw, int Kp, int esize, int* rnt, int* rks, int* rcpt) {
  if (bb % 16 == 0) return mfma_split(ncw, Kp, esize, kScanRegChunks, rnt, rks, rcpt);
  // VALU: 256 / q columns, q K slices; a slice's chunks cost ~12 cycles each
  // in sequence, the K-split reduction ~300 cycles (barrier + LDS round trip)
  const int nch = Kp * esize / 16;
  double best = 1e30;
  bool ok = false;
  for (int q = 1; q <= 4; q *= 2) {
    if (256 / q < ncw || nch % q != 0 || nch / q > kScanRegChunks) continue;
    const double cyc = 12.0 * (nch / q) + (q > 1 ? 300.0 : 0.0);
    if (cyc < best) {
      best = cyc;
      *rnt = 0; *rks = q; *rcpt = nch / q;
      ok = true;
    }
  }
  return ok;
}

// The tiled scan's launch shape for `nslot` layer slots (stacked layers
// scanned in one launch) of D directions each, with its modelled time per
// step in *cost_us when non-null.
int plan_scan(const RnnDesc* d, const Dims& m, int cus, int xcds, bool allow_wreg, ScanPlan* out, int nslot = 1,
              double* cost_us = nullptr) {
  const int B = d->B, H = d->hidden_size, P = d->proj_size;
  const bool lstmp = d->mode == RNN_MODE_LSTMP;
  std::vector<int> bbs;
  if (d->tile_batch > 0) {
    bbs.push_back(d->tile_batch);
  } else if (B >= 16) {
    for (int bb = 16; bb <= std::min(64, rup(B, 16)); bb += 16) bbs.push_back(bb);
  } else {
    bbs.push_back(B);
  }
  std::vector<int> hss;
  if (d->tile_hidden > 0) {
    hss.push_back(d->tile_hidden);
  } else {
    for (int hs = 1; hs <= std::min(H, 256); hs *= 2) hss.push_back(hs);
    if (std::find(hss.begin(), hss.end(), H) == hss.end() && H <= 256) hss.push_back(H);
  }
  const int per_xcd = xcds > 1 ? cus / xcds : 0;
  double best = 1e30;
  bool found = false;
  for (int bb : bbs) {
    if (bb < 1 || bb > 64) continue;  // the scan tracks a block's rows in 64-bit masks
    const bool mfma = bb % 16 == 0;
    for (int hs : hss) {
      if (hs < 1 || bb * hs > 1024) continue;
      const int ns = cdiv(H, hs);
      const int nbb = cdiv(B, bb);
      if ((long long)m.D * nbb * ns > kScanMaxWorkgroups || (long long)nslot * m.D * nbb * ns > cus) continue;
      const int ps = lstmp ? cdiv(P, ns) : 0;
      if (bb * ps > 1024) continue;  // projection outputs: at most 4 per thread
      const int ncw = rup(m.gates * hs, 16);
      for (int wreg = allow_wreg && d->weights != 1 ? 1 : 0; wreg >= 0; --wreg) {
        ScanArgs a{};
        a.mode = d->mode == RNN_MODE_GRU ? kGRU : (lstmp ? kLSTMP : kLSTM);
        a.bb = bb; a.hs = hs; a.ps = ps; a.Kp = m.Kp; a.Hp = m.Hp;
        a.wreg = wreg;
        if (wreg && !reg_layout(bb, ncw, m.Kp, m.esize, &a.rnt, &a.rks, &a.rcpt)) continue;
        if (lstmp && mfma && !mfma_split(rup(ps, 16), m.Hp, m.esize, 1 << 20, &a.pnt, &a.pks, &a.pcpt))
          a.pnt = a.pks = a.pcpt = 0;
        const int lds = scan_lds_bytes(a, m.esize);
        if (lds > kMaxLds) continue;
        const int groups = nslot * m.D * nbb;
        const int gpx = per_xcd > 0 && d->placement != 1 ? cdiv(groups, xcds) : 0;
        const bool xcd_aligned = gpx > 0 && gpx * ns <= per_xcd;
        // a group whose members share one XCD exchanges ~15% faster (measured)
        const double xf = xcd_aligned && ns > 1 ? 0.85 : 1.0;
        // a one-member group keeps h in LDS: no exchange and no barrier
        const double ex =
            ns == 1 && !lstmp ? 0.1 : (scan_barrier_us(ns) + 0.3 + (double)bb * m.Kp * m.esize / 100e3) * xf;
        double mm;
        if (wreg && mfma) {
          // per wave: rtiles * rcpt chunks, rnt MFMA tiles each; the h tile
          // is the only LDS operand
          const double rt = bb / 16, per_chunk = m.esize == 2 ? 16.0 : 32.0;
          mm = std::max(rt * a.rcpt * a.rnt * per_chunk, rt * a.rcpt * 32.0) / 2400.0 + (a.rks > 1 ? 0.2 : 0.0);
        } else if (wreg) {
          mm = (double)bb * a.rcpt * 12.0 / 2400.0 + 0.1 + (a.rks > 1 ? 0.125 : 0.0);
        } else {
          mm = mm_us(mfma, m.esize, bb, m.gates * hs, mfma ? m.Kp : m.K);
        }
        double t = ex + mm + bb * hs / 256.0 * 0.05;
        if (lstmp) {
          double mp = mm_us(mfma, m.esize, bb, ps, mfma ? m.Hp : H);
          if (a.pnt > 0)  // K split over the waves
            mp = mp * a.pnt * a.pks / 4.0 + (a.pks > 1 ? 0.125 : 0.0);
          t += (scan_barrier_us(ns) + 0.3 + (double)bb * m.Hp * m.esize / 100e3) * xf + mp;
        }
        if (d->placement == 2 && !xcd_aligned) t += 1e3;  // requested: aligned plans first
        if (d->weights == 2 && !wreg) t += 1e3;            // requested: registers first
        if (t < best) {
          best = t;
          *out = ScanPlan{bb, hs, ns, ps, nbb, xcd_aligned ? gpx : 0, lds, wreg, a.rnt, a.rks, a.rcpt,
                          a.pnt, a.pks, a.pcpt};
          found = true;
        }
      }
    }
  }
  if (found && cost_us) *cost_us = best;
  return found ? RNN_OK : RNN_E_PLAN;
}

struct RssmPlan {
  int rows, ngroups, nw, h_per, gpx, lds;
  int reg;  // 1: kernel 3b (GRU slices in registers, ring exchange inside an XCD)
};

// Grid of an RSSM plan: with XCD-aligned groups every XCD gets gpx whole
// groups (the last XCDs may hold padding slots).
int rssm_grid(const RssmPlan& p, int xcds) { return p.gpx > 0 ? xcds * p.gpx * p.nw : p.ngroups * p.nw; }

// Kernel 3b: groups of at most rssm_reg_max_members() wide members whose
// GRU slices fit the register layout, every group on one XCD. The step
// model: the exchange costs ~1.1 us plus the bytes one member reads (every
// member's partial sums and the whole h_t of the group's rows) at ~43 GB/s
// per member, plus ~15 ns per unit of the slice (gates, partial products,
// publishing), both fitted to unrolls at B=50, T=50 over 2-4 rows and 5-8
// members; the products are the per-wave MFMA chains (the slice products
// take a fixed number of chunks per wave whatever the slice width) at ~12
// cycles each, plus six workgroup barriers (nine with the actor).
bool plan_rssm_reg(const RnnDesc* d, int cus, int xcds, RssmPlan* out) {
  // flat placement (consecutive ids form a group) rules it out: its
  // exchange is only valid when a group's members share an XCD
  if (!is_rssm(d->mode) || d->weights == 1 || d->placement == 1) return false;
  const int B = d->B, S = d->state_dim, A = d->action_dim, E = d->embed_dim, Hb = d->belief_dim;
  const int Ea = d->mode == RNN_MODE_RSSM_ACTOR ? d->actor_dim : 0;
  const int per_xcd = cus / xcds;
  double best = 1e30;
  bool found = false;
  for (int rows = 1; rows <= rssm_max_rows(); ++rows) {
    if (d->tile_batch > 0 && rows != d->tile_batch) continue;
    const int ngroups = cdiv(B, rows);
    const int gpx = cdiv(ngroups, xcds);
    for (int nw = 1; nw <= rssm_reg_max_members(); ++nw) {
      const int h_per = cdiv(Hb, nw);
      if (d->tile_hidden > 0 && h_per != d->tile_hidden) continue;
      if (nw > 1 && cdiv(Hb, nw - 1) == h_per) continue;
      if (gpx * nw > per_xcd) continue;
      RssmArgs a{};
      a.S = S; a.A = A; a.E = E; a.Hb = Hb; a.rows = rows; a.nw = nw; a.h_per = h_per; a.Ea = Ea;
      a.Ep = rssm_ex_cols(d); a.Hbp = rup(Hb, 4);
      if (!rssm_reg_fits(a)) continue;
      const int lds = rssm_reg_lds_bytes(a);
      if (lds > kMaxLds) continue;
      const double bytes = (double)rows * ((double)nw * a.Ep + a.Hbp) * 4.0;
      const int nq = cdiv(cdiv(std::max(E, Hb), 4), 4), n2 = cdiv(cdiv(E, 4), 8);
      const double actor = Ea > 0 ? cdiv(S, 4) + cdiv(cdiv(Ea, 4), 8) : 0;
      const double mfma = 4.0 * (2 * nq + std::max(nq, n2) + cdiv(h_per, 4) + cdiv(S + A, 4) + actor);
      const double t = 1.1 + bytes / 43e3 + 0.015 * h_per + (mfma * 12.0 + (Ea > 0 ? 9 : 6) * 150.0 + 400.0) / 2400.0;
      if (t < best) {
        best = t;
        *out = RssmPlan{rows, ngroups, nw, h_per, gpx, lds, 1};
        found = true;
      }
    }
  }
  return found;
}

int plan_rssm(const RnnDesc* d, int cus, int xcds, RssmPlan* out) {
  if (plan_rssm_reg(d, cus, xcds, out)) return RNN_OK;
  if (d->weights == 2) return RNN_E_PLAN;  // registers requested, no such plan
  const int B = d->B, S = d->state_dim, A = d->action_dim, E = d->embed_dim, Hb = d->belief_dim;
  const int Ea = d->actor_dim;
  const int per_xcd = xcds > 1 ? cus / xcds : 0;
  double best = 1e30;
  bool found = false;
  for (int rows = 1; rows <= rssm_max_rows(); ++rows) {
    if (d->tile_batch > 0 && rows != d->tile_batch) continue;
    const int ngroups = cdiv(B, rows);
    for (int nw = 1; nw <= kRssmMaxMembers; ++nw) {
      const int h_per = cdiv(Hb, nw);
      if (d->tile_hidden > 0 && h_per != d->tile_hidden) continue;
      if (nw > 1 && cdiv(Hb, nw - 1) == h_per) continue;  // same slices with fewer members
      if ((long long)ngroups * nw > cus) continue;
      if (rows * h_per > 256 || rows * S > 256 || rows * A > 256) continue;
      RssmArgs a{};
      a.S = S; a.A = A; a.E = E; a.Hb = Hb; a.rows = rows; a.nw = nw; a.h_per = h_per; a.Ea = Ea;
      const int lds = rssm_lds_bytes(a);
      if (lds > kMaxLds) continue;
      // XCD-aligned groups only on request: for this kernel they measured no
      // faster, and the planner would trade rows for them
      const int gpx = per_xcd > 0 && d->placement == 2 ? cdiv(ngroups, xcds) : 0;
      const bool xcd_aligned = gpx > 0 && gpx * nw <= per_xcd;
      // GRU slice + partial of W_1 + (redundant) partial sums, W_2 and W_as;
      // the 4x4 MFMA blocks cost the same for any 1..4 batch rows
      // (+ the actor: belief-column partials, their sum, state part, W_a2)
      const double macs = 4.0 * (3.0 * h_per * (E + Hb) + (double)(E + Ea) * h_per + (double)(E + Ea) * nw +
                                 2.0 * S * E + (double)E * (S + A) + (double)Ea * (S + A));
      const double bytes = (double)rows * (Hb + (double)nw * (E + Ea)) * 4.0;
      // products run on 8 waves: ~64 MAC/clk of the 4x4 MFMA chains (measured)
      double t = barrier_us(nw) + 0.3 + (Ea > 0 ? 0.6 : 0.0) + bytes / 100e3 + macs / 64.0 / 2400.0;
      if (d->placement == 2 && !xcd_aligned) t += 1e3;  // requested: aligned plans first
      if (t < best) {
        best = t;
        *out = RssmPlan{rows, ngroups, nw, h_per, xcd_aligned ? gpx : 0, lds, 0};
        found = true;
      }
    }
  }
  return found ? RNN_OK : RNN_E_PLAN;
}

// ---------------------------------------------------------------------------
// Forward paths
// ---------------------------------------------------------------------------
int hip_status(hipError_t e) { return e == hipSuccess ? RNN_OK : RNN_E_HIP; }

// Optional per-kernel event brackets (rnn_forward_profiled).
// kinds[n] = kernel kind | layer << 8 (kind 5, a pipelined scan: first
// layer | last layer << 4). The bracket's events ride on its launches
// (start with the first dispatch, stop with the last completion); a bracket
// that launched nothing records both directly.
// A named host range (roctx) around one public call, for timeline tools
// such as rocprofv3 --marker-trace; a no-op when no tool is attached.
struct Range {
  explicit Range(const char* name) { roctxRangePushA(name); }
  ~Range() { roctxRangePop(); }
  Range(const Range&) = delete;
  Range& operator=(const Range&) = delete;
};

// Per-launch brackets: the kind and layer of every kernel the call enqueues
// (kind 1 input projection, 2 tiled scan, 3 RSSM unroll, 4 one-wave scan,
// 5 pipelined scans of two layers), HIP events on the launch when the caller
// asked for timing, and a roctx range named after the launch.
struct Prof {
  void* const* events = nullptr;
  int n_events = 0;
  int* kinds = nullptr;
  int n = 0;
  int open = 0;  // roctx ranges pushed and not yet popped
  hipStream_t st = nullptr;
  int begin(int kind, int layer) {
    static const char* const names[] = {"?", "input_projection", "scan", "rssm_unroll", "scan_wave", "scan"};
    char label[48];
    const char* nm = kind >= 1 && kind <= 5 ? names[kind] : names[0];
    if (kind == 5)
      snprintf(label, sizeof label, "%s L%d+L%d", nm, layer & 15, layer >> 4);
    else
      snprintf(label, sizeof label, "%s L%d", nm, layer);
    roctxRangePushA(label);
    ++open;
    if (kinds && n < n_events / 2) kinds[n] = kind | layer << 8;
    if (events && n < n_events / 2) {
      rnnk::LaunchEvents& ev = rnnk::launch_events();
      ev.start = reinterpret_cast<hipEvent_t>(events[2 * n]);
      ev.stop = reinterpret_cast<hipEvent_t>(events[2 * n + 1]);
    }
    return RNN_OK;
  }
  int end() {
    int rc = RNN_OK;
    rnnk::LaunchEvents& ev = rnnk::launch_events();
    if (events && n < n_events / 2 && ev.start) {
      rc = hip_status(hipEventRecord(ev.start, st));
      if (rc == RNN_OK) rc = hip_status(hipEventRecord(ev.stop, st));
    }
    ev = rnnk::LaunchEvents{};
    ++n;
    if (open > 0) {
      roctxRangePop();
      --open;
    }
    return rc;
  }
  // an early return inside a bracket must not leave events armed for a
  // later call on this thread, nor a range open
  ~Prof() {
    rnnk::launch_events() = rnnk::LaunchEvents{};
    for (; open > 0; --open) roctxRangePop();
  }
};

int check_ptr(const void* p, size_t elem) {
  if (!p) return RNN_E_NULL;
  return aligned(p, elem) ? RNN_OK : RNN_E_ALIGN;
}

int check_opt(const void* p, size_t elem) { return (!p || aligned(p, elem)) ? RNN_OK : RNN_E_ALIGN; }

int forward_rssm(const RnnDesc* d, const RnnWeights* w, const RnnIO* io, char* ws, size_t ws_bytes,
                 hipStream_t st, int cus, int xcds, Prof& prof) {
  int rc;
  const bool actor = d->mode == RNN_MODE_RSSM_ACTOR;
  const void* req[] = {w->w_as, w->b_as, w->w_ih[0], w->w_hh[0], w->b_ih[0], w->b_hh[0], w->w_1, w->b_1,
                       w->w_2, w->b_2, io->noise, io->means, io->stds, io->states, io->beliefs};
  for (const void* p : req)
    if ((rc = check_ptr(p, 4)) != RNN_OK) return rc;
  if (actor) {
    for (const void* p : {w->w_a1, w->b_a1, w->w_a2, w->b_a2})
      if ((rc = check_ptr(p, 4)) != RNN_OK) return rc;
    if ((rc = check_opt(io->actions, 4)) != RNN_OK) return rc;
  } else if ((rc = check_ptr(io->x, 4)) != RNN_OK) {
    return rc;
  }
  if ((rc = check_opt(io->s0, 4)) != RNN_OK || (rc = check_opt(io->h0, 4)) != RNN_OK) return rc;
  const WsLayout L = layout_of(d, 0, false);
  if (!ws) return RNN_E_WORKSPACE;
  if (ws_bytes < L.total) return RNN_E_WORKSPACE;
  if (!aligned(ws, 16)) return RNN_E_ALIGN;
  RssmPlan p;
  if ((rc = plan_rssm(d, cus, xcds, &p)) != RNN_OK) return rc;

  RssmArgs a{};
  a.B = d->B; a.T = d->T; a.S = d->state_dim; a.A = d->action_dim; a.E = d->embed_dim; a.Hb = d->belief_dim;
  a.scale_lb = d->scale_lb;
  a.rows = p.rows; a.ngroups = p.ngroups; a.nw = p.nw; a.h_per = p.h_per;
  a.nxcd = xcds; a.gpx = p.gpx;
  a.w_as = (const float*)w->w_as; a.b_as = (const float*)w->b_as;
  a.w_ih = (const float*)w->w_ih[0]; a.w_hh = (const float*)w->w_hh[0];
  a.b_ih = (const float*)w->b_ih[0]; a.b_hh = (const float*)w->b_hh[0];
  a.w_1 = (const float*)w->w_1; a.b_1 = (const float*)w->b_1;
  a.w_2 = (const float*)w->w_2; a.b_2 = (const float*)w->b_2;
  a.actions = actor ? nullptr : (const float*)io->x; a.eps = (const float*)io->noise;
  a.Ea = actor ? d->actor_dim : 0;
  a.w_a1 = actor ? (const float*)w->w_a1 : nullptr; a.b_a1 = actor ? (const float*)w->b_a1 : nullptr;
  a.w_a2 = actor ? (const float*)w->w_a2 : nullptr; a.b_a2 = actor ? (const float*)w->b_a2 : nullptr;
  a.act_out = actor ? (float*)io->actions : nullptr;
  a.s0 = (const float*)io->s0; a.h0 = (const float*)io->h0;
  a.means = (float*)io->means; a.stds = (float*)io->stds; a.states = (float*)io->states;
  a.beliefs = (float*)io->beliefs;
  a.ex_h = (float*)(ws + L.ex_h); a.ex_p = (float*)(ws + L.ex_p);
  a.Ep = rssm_ex_cols(d); a.Hbp = rup(d->belief_dim, 4);
  a.xid = (unsigned*)(ws + L.xid);
  a.counters = (unsigned*)(ws + L.counters);
  a.status = (int*)(ws + L.status);
  // status word and counters are contiguous at the start of the workspace;
  // for kernel 3b the XCC ids and both rings start as the sentinel: ids, h
  // ring and the used front of the partial ring are consecutive (the fill
  // covers the alignment gaps between them too). One launch does both.
  const size_t zero_bytes = L.counters + L.counters_bytes;
  const size_t ring_end = L.ex_p + (size_t)rssm_ring_slots() * d->B * p.nw * a.Ep * 4;
  if ((rc = hip_status(launch_fill2_u32(ws, zero_bytes, 0u, ws + L.xid, p.reg ? ring_end - L.xid : 0, 0xFFFFFFFFu,
                                        st))) != RNN_OK)
    return rc;
  if ((rc = prof.begin(3, 0)) != RNN_OK) return rc;
  if ((rc = hip_status(p.reg ? launch_rssm_reg(a, st) : launch_rssm(a, st))) != RNN_OK) return rc;
  return prof.end();
}

// The one-wave-per-row scan runs when every gate row of the layer fits one
// wavefront and no tiling hint asks for the tiled scan (and y is addressed
// with 32-bit byte offsets).
bool use_wave_scan(const RnnDesc* d, const Dims& m) {
  if (d->tile_batch || d->tile_hidden || d->weights) return false;
  if ((double)m.rows * m.D * m.K * m.esize >= 2147483647.0) return false;
  const int mk = d->mode == RNN_MODE_GRU ? kGRU : (d->mode == RNN_MODE_LSTMP ? kLSTMP : kLSTM);
  return scan_wave_fits(mk, d->hidden_size, m.K);
}

// Training reserve: per layer, the gate values of every token and
// direction ([rows, D, R] fp32, R = 5H LSTM / 4H GRU) and, below the last
// layer, the layer's output ([rows, D * H] fp32), which is the next layer's
// input and the source of h_{t-1}.
struct ReserveLayout {
  size_t gates[RNN_MAX_LAYERS], y[RNN_MAX_LAYERS], total;
  int R;
};

ReserveLayout reserve_of(const RnnDesc* d, const Dims& m) {
  ReserveLayout r{};
  r.R = (d->mode == RNN_MODE_GRU ? 4 : 5) * d->hidden_size;
  size_t o = 0;
  for (int l = 0; l < d->num_layers; ++l) {
    r.gates[l] = o;
    o = align_up(o + (size_t)m.rows * m.D * r.R * 4, kAlign);
    r.y[l] = o;
    if (l + 1 < d->num_layers) o = align_up(o + (size_t)m.rows * m.D * m.K * 4, kAlign);
  }
  r.total = o;
  return r;
}

// Training is built for fp32 LSTM, LSTMP and GRU stacks without clipping.
int validate_train(const RnnDesc* d) {
  if (d->mode != RNN_MODE_LSTM && d->mode != RNN_MODE_GRU && d->mode != RNN_MODE_LSTMP) return RNN_E_UNSUPPORTED;
  if (d->dtype != RNN_DTYPE_F32 || d->clip != 0) return RNN_E_UNSUPPORTED;
  return RNN_OK;
}

// The G_x product of layer l (both directions) over `rows` rows of its
// input starting at row r0, into C.
GemmArgs layer_gemm(const RnnDesc* d, const RnnWeights* w, const Dims& m, int l, const void* in, long long r0,
                    int rows, void* C, int c_bf16, char* ws, const WsLayout& L, bool allow_split) {
  const size_t es = m.esize;
  const int in_l = l == 0 ? d->input_size : m.D * m.K;
  GemmArgs g{};
  g.A = (const char*)in + (size_t)r0 * in_l * es;
  g.M = rows; g.N = m.D * m.G; g.K = in_l; g.G = m.G;
  g.hh_fold_rows = d->mode == RNN_MODE_GRU ? 2 * d->hidden_size : m.G;
  g.has_bias = d->has_bias;
  g.C = C;
  g.c_bf16 = c_bf16;
  bool vec = (size_t)in_l * es % 16 == 0 && aligned(g.A, 16);
  for (int di = 0; di < m.D; ++di) {
    const int i = l * m.D + di;
    g.W[di] = w->w_ih[i];
    g.b_ih[di] = w->b_ih[i];
    g.b_hh[di] = w->b_hh[i];
    vec = vec && aligned(w->w_ih[i], 16);
  }
  g.vec_ok = vec;
  g.zero16 = ws + L.status + kZeroChunk;
  g.splits = allow_split ? gemm_xw_splits(g.M, g.N, g.K, d->dtype == RNN_DTYPE_BF16) : 1;
  g.part = g.splits > 1 ? (float*)(ws + L.gpart) : nullptr;
  return g;
}

// The scan arguments of layer l that do not depend on the time range: the
// problem, the plan, the weights, the clamps and the layer's exchange block.
ScanArgs layer_scan(const RnnDesc* d, const RnnWeights* w, const Dims& m, const ScanPlan& p, int xcds, int l,
                    char* ws, const WsLayout& L) {
  ScanArgs a{};
  a.mode = d->mode == RNN_MODE_GRU ? kGRU : (d->mode == RNN_MODE_LSTMP ? kLSTMP : kLSTM);
  a.B = d->B; a.H = d->hidden_size; a.K = m.K; a.P = d->proj_size; a.D = m.D; a.G = m.G;
  a.packed = d->layout == RNN_LAYOUT_PACKED;
  a.has_bias = d->has_bias;
  a.bb = p.bb; a.hs = p.hs; a.ns = p.ns; a.ps = p.ps; a.nbb = p.nbb; a.Kp = m.Kp; a.Hp = m.Hp;
  a.nxcd = xcds; a.gpx = p.gpx;
  a.wreg = p.wreg; a.rnt = p.rnt; a.rks = p.rks; a.rcpt = p.rcpt;
  a.pnt = p.pnt; a.pks = p.pks; a.pcpt = p.pcpt;
  const float inf = std::numeric_limits<float>::infinity();
  const bool cclip = d->clip & RNN_CLIP_CELL, pclip = d->clip & RNN_CLIP_PROJ;
  a.c_lo = cclip ? d->cell_clip_lo : -inf;
  a.c_hi = cclip ? d->cell_clip_hi : inf;
  a.p_lo = pclip ? -d->proj_clip : -inf;
  a.p_hi = pclip ? d->proj_clip : inf;
  for (int di = 0; di < m.D; ++di) {
    const int i = l * m.D + di;
    a.w_hh[di] = w->w_hh[i];
    a.w_hr[di] = d->mode == RNN_MODE_LSTMP ? w->w_hr[i] : nullptr;
    a.b_hh[di] = d->has_bias ? w->b_hh[i] : nullptr;
  }
  char* ex = ws + L.ex + l * L.ex_layer;
  a.nslot = 1;
  a.xid[0] = (unsigned*)ex;
  a.hx[0] = ex + L.ex_hx;
  a.mx[0] = d->mode == RNN_MODE_LSTMP ? ex + L.ex_mx : nullptr;
  a.counters = (unsigned*)(ws + L.counters + (size_t)l * m.D * d->B * kCounterBytes);
  a.status = (int*)(ws + L.status);
  return a;
}

// The launch plan of the forward: the one-wave scan, or the tiled scan's
// plan and whether the layers run pipelined: one launch then scans a time
// chunk of every stacked layer at once (layer l on chunk w - l at wave w),
// so it needs num_layers x the workgroups of a single layer's scan, and the
// stack takes nchunks + num_layers - 1 chunk scans instead of num_layers x
// nchunks. It is taken when the cost model expects it to be faster.
// Measured on MI355X: a scan step takes 2.3-2.9x the model's time (LSTMP
// B=32 6.97 us vs 3.05, GRU B=256 3.86 vs 1.34, var-len BiLSTM 4.67 vs 1.73,
// LSTM B=1 3.28 vs 1.21; the model ranks launch shapes, this scale makes it
// absolute); fixed costs per pipelined wave and per layer.
constexpr double kModelScale = 2.6, kPipeWaveUs = 40.0, kLayerUs = 35.0;

// Kernel 2c for a few independent sequences: LSTM or GRU of width up to 512,
// at most kScanSmallMaxGroups (direction, row) groups, no tiling or weight
// hint (those ask for the tiled scan), y rows addressed with 32-bit byte
// offsets. A descriptor-only test (it sizes the workspace and the G_x
// dtype); whether the launch fits the device is plan_small's.
bool small_scan_shape(const RnnDesc* d, const Dims& m) {
  if (d->mode != RNN_MODE_LSTM && d->mode != RNN_MODE_GRU) return false;
  if (d->tile_batch || d->tile_hidden || d->weights) return false;
  // (a stack asked to run pipelined runs the tiled scan's layer slots)
  if (d->layer_pipeline == RNN_PIPE_ON && d->num_layers > 1) return false;
  if (m.D * d->B > kScanSmallMaxGroups || scan_small_chunks(m.K) == 0) return false;
  if ((double)m.rows * m.D * m.K * m.esize >= 2147483647.0) return false;
  return !use_wave_scan(d, m);
}
struct SmallPlan {
  bool on;
  int hs, ns, gpx;  // units per workgroup, members per group, groups per XCD (0: flat)
};
SmallPlan plan_small(const RnnDesc* d, const Dims& m, int cus, int xcds) {
  SmallPlan s{};
  if (!small_scan_shape(d, m)) return s;
  // the fewest units per wave whose groups fit the device: a wave's chain
  // (its gate rows' sums, then its units' gate math) shortens with fewer
  // units, measured at T=80, B=1, H=256: 1, 2, 4 units per wave 125, 135,
  // 185 us per scan
  const int groups = m.D * d->B;
  s.hs = 0;
  for (int uw : {1, 2, 4}) {
    const int hs = scan_small_units_per_wg(uw), ns = cdiv(d->hidden_size, hs);
    if (groups * ns <= cus && groups * ns <= kScanMaxWorkgroups) {
      s.hs = hs;
      s.ns = ns;
      break;
    }
  }
  if (s.hs == 0) return s;
  // members of a group on one XCD when a whole number of groups fits each
  // (placement 1 asks for consecutive ids, 2 for aligned groups)
  const int gpx = cdiv(groups, xcds);
  const bool aligned_ok = xcds > 1 && gpx * s.ns <= cus / xcds;
  if (d->placement == 2 && !aligned_ok) return s;
  s.gpx = aligned_ok && d->placement != 1 ? gpx : 0;
  s.on = true;
  return s;
}
int small_grid(const SmallPlan& s, int groups, int xcds) { return s.gpx > 0 ? xcds * s.gpx * s.ns : groups * s.ns; }

struct ForwardPlan {
  bool wave, pipe;
  SmallPlan sp;
  PipeShape ps;
  ScanPlan p;
  double step_us;  // modelled time of one scan step of the chosen plan
};
int plan_forward(const RnnDesc* d, const Dims& m, bool has_len, int cus, int xcds, bool wreg_ok, bool training,
                 ForwardPlan* out) {
  ForwardPlan f{};
  f.step_us = 0.0;
  f.wave = !training && use_wave_scan(d, m);
  if (f.wave) {
    *out = f;
    return RNN_OK;
  }
  if (!training) {
    f.sp = plan_small(d, m, cus, xcds);
    if (f.sp.on) {
      *out = f;
      return RNN_OK;
    }
  }
  f.ps = pipe_shape(d, has_len, m);
  double one = 0.0;
  const int rc = plan_scan(d, m, cus, xcds, wreg_ok, &f.p, 1, &one);
  ScanPlan pp{};
  double piped = 0.0;
  if (f.ps.on && !training && plan_scan(d, m, cus, xcds, wreg_ok, &pp, d->num_layers, &piped) == RNN_OK) {
    // per-step costs times the steps each schedule walks in sequence, plus
    // the launches around each scan (a wave: exchange reset, one G_x
    // product per active layer, the scan; a layer: its product and scan)
    const int L = d->num_layers, waves = f.ps.nchunks + L - 1;
    const double tp = kModelScale * piped * (double)f.ps.chunk * waves + kPipeWaveUs * waves;
    const double tl = kModelScale * one * (double)d->T * L + kLayerUs * L;
    if (rc != RNN_OK || tp < tl || d->layer_pipeline == RNN_PIPE_ON) {
      f.pipe = true;
      f.p = pp;
    }
  }
  f.step_us = f.pipe ? piped : one;
  if (!f.pipe && rc != RNN_OK) return rc;
  *out = f;
  return RNN_OK;
}

// Layer pipelining on the caller's stream, in waves, after layer 0's G_x for
// all steps: wave w resets the exchange blocks of the active layers,
// computes layer l's (l > 0) G_x for its time chunk c = w - l from layer
// l - 1's output of chunk c (written by the previous wave), and scans every
// active layer's chunk in one launch.
// The state crosses chunk boundaries through the workspace: h in the
// storage dtype (the first step's operand, what the ring would hold) and
// fp32 h and c (the registers), so the results are those of the
// layer-by-layer run, bit for bit. Chunk c reads state set c % 2 and writes
// set (c + 1) % 2.
int forward_rnn_pipe(const RnnDesc* d, const RnnWeights* w, const RnnIO* io, char* ws, const WsLayout& L,
                     const Dims& m, const ForwardPlan& f, hipStream_t st, int xcds, Prof& prof) {
  int rc;
  const int nl = d->num_layers, n = f.ps.nchunks, chunk = f.ps.chunk;
  const size_t es = m.esize;
  const bool bf16 = d->dtype == RNN_DTYPE_BF16;
  const int gx_bf16 = gx_esize(d, m) == 2;
  const int B = d->B, H = d->hidden_size, K = m.K;
  const bool cell = d->mode != RNN_MODE_GRU;
  auto layer_out = [&](int l) -> char* {
    return l == nl - 1 ? (char*)io->y : ws + ((l % 2 == 0) ? L.inter0 : L.inter1);
  };
  // layer 0's G_x for every step in one product (its input x is all there)
  const size_t gxs = gx_esize(d, m);
  const GemmArgs g0 = layer_gemm(d, w, m, 0, io->x, 0, (int)m.rows, ws + L.gx, gx_bf16, ws, L, true);
  // status word, counters (and the GEMM's zero chunk beside them) and the
  // first wave's exchange (layer 0 only), before anything reads them
  if ((rc = hip_status(launch_fill2_u32(ws, L.counters + L.counters_bytes, 0u, ws + L.ex, L.ex_layer, 0xFFFFFFFFu,
                                        st))) != RNN_OK)
    return rc;
  if ((rc = prof.begin(1, 0)) != RNN_OK) return rc;
  if ((rc = hip_status(launch_gemm_xw(g0, bf16, st))) != RNN_OK) return rc;
  if ((rc = prof.end()) != RNN_OK) return rc;
  auto sth = [&](int set, int l) { return ws + L.sth + ((size_t)set * nl + l) * L.sth_layer; };
  auto sthf = [&](int set, int l) { return (float*)(ws + L.sthf + ((size_t)set * nl + l) * L.stf_layer); };
  auto stcf = [&](int set, int l) { return (float*)(ws + L.stcf + ((size_t)set * nl + l) * L.stf_layer); };
  for (int wv = 0; wv < n + nl - 1; ++wv) {
    const int l0 = std::max(0, wv - n + 1), l1 = std::min(nl - 1, wv);
    if (wv > 0 && (rc = hip_status(launch_fill_u32(ws + L.ex + l0 * L.ex_layer, (size_t)(l1 - l0 + 1) * L.ex_layer,
                                                   0xFFFFFFFFu, st))) != RNN_OK)
      return rc;
    ScanArgs a = layer_scan(d, w, m, f.p, xcds, 0, ws, L);
    a.nslot = nl;
    a.gx_bf16 = gx_bf16;
    for (int l = 0; l < nl; ++l) a.T[l] = 0;
    for (int l = l0; l <= l1; ++l) {
      const int c = wv - l, t0 = c * chunk, tc = std::min(d->T, t0 + chunk) - t0;
      const bool first = c == 0, last = c == n - 1;
      char* gxc;
      if (l == 0) {
        gxc = ws + L.gx + (size_t)t0 * B * m.G * gxs;
      } else {
        gxc = ws + L.gxp + (size_t)(l - 1) * L.gxp_layer;
        const GemmArgs g = layer_gemm(d, w, m, l, layer_out(l - 1), (long long)t0 * B, tc * B, gxc, gx_bf16, ws,
                                      L, false);
        if ((rc = prof.begin(1, l)) != RNN_OK) return rc;
        if ((rc = hip_status(launch_gemm_xw(g, bf16, st))) != RNN_OK) return rc;
        if ((rc = prof.end()) != RNN_OK) return rc;
      }
      const ScanArgs al = layer_scan(d, w, m, f.p, xcds, l, ws, L);
      a.T[l] = tc;
      a.gx[l] = gxc;
      a.y[l] = layer_out(l) + (size_t)t0 * B * K * es;
      a.hx[l] = al.hx[0];
      a.mx[l] = al.mx[0];
      a.xid[l] = al.xid[0];
      a.w_hh[l] = al.w_hh[0];
      a.w_hr[l] = al.w_hr[0];
      a.b_hh[l] = al.b_hh[0];
      const int rs = c % 2, wset = (c + 1) % 2;
      a.h0[l] = first ? (io->h0 ? (const char*)io->h0 + (size_t)l * B * K * es : nullptr) : sth(rs, l);
      a.c0[l] = first && cell && io->c0 ? (const char*)io->c0 + (size_t)l * B * H * es : nullptr;
      a.h0f[l] = first ? nullptr : sthf(rs, l);
      a.c0f[l] = first || !cell ? nullptr : stcf(rs, l);
      a.h_n[l] = last ? (io->h_n ? (char*)io->h_n + (size_t)l * B * K * es : nullptr) : sth(wset, l);
      a.c_n[l] = last && cell && io->c_n ? (char*)io->c_n + (size_t)l * B * H * es : nullptr;
      a.h_nf[l] = last ? nullptr : sthf(wset, l);
      a.c_nf[l] = last || !cell ? nullptr : stcf(wset, l);
    }
    // kind 5: one launch scanning layers l0 .. l1
    if ((rc = prof.begin(5, l0 | l1 << 4)) != RNN_OK) return rc;
    if ((rc = hip_status(launch_scan(a, bf16, st))) != RNN_OK) return rc;
    if ((rc = prof.end()) != RNN_OK) return rc;
  }
  return RNN_OK;
}

int forward_rnn(const RnnDesc* d, const RnnWeights* w, const RnnIO* io, char* ws, size_t ws_bytes,
                hipStream_t st, int cus, int xcds, Prof& prof, char* rsv = nullptr) {
  int rc;
  long long n_tok = 0;
  int t_max = 0;
  if ((rc = validate_lengths(d, io->lengths_host, &n_tok, &t_max)) != RNN_OK) return rc;
  const Dims m = dims_of(d, n_tok);
  const size_t es = m.esize;
  const int LD = d->num_layers * m.D;
  for (int i = 0; i < LD; ++i) {
    if ((rc = check_ptr(w->w_ih[i], es)) != RNN_OK || (rc = check_ptr(w->w_hh[i], es)) != RNN_OK) return rc;
    if (d->has_bias) {
      if ((rc = check_ptr(w->b_ih[i], es)) != RNN_OK || (rc = check_ptr(w->b_hh[i], es)) != RNN_OK) return rc;
    }
    if (d->mode == RNN_MODE_LSTMP && (rc = check_ptr(w->w_hr[i], es)) != RNN_OK) return rc;
  }
  if ((rc = check_ptr(io->x, es)) != RNN_OK || (rc = check_ptr(io->y, es)) != RNN_OK) return rc;
  if ((rc = check_opt(io->h0, es)) != RNN_OK || (rc = check_opt(io->h_n, es)) != RNN_OK) return rc;
  if (d->mode != RNN_MODE_GRU &&
      ((rc = check_opt(io->c0, es)) != RNN_OK || (rc = check_opt(io->c_n, es)) != RNN_OK))
    return rc;
  const bool has_len = io->lengths_host != nullptr;
  const WsLayout L = layout_of(d, n_tok, has_len);
  if (!ws || ws_bytes < L.total) return RNN_E_WORKSPACE;
  if (!aligned(ws, 16)) return RNN_E_ALIGN;
  // W_hh slices go to registers only as whole aligned 16-byte chunks
  bool wreg_ok = (size_t)m.K * es % 16 == 0;
  for (int i = 0; i < LD; ++i) wreg_ok = wreg_ok && aligned(w->w_hh[i], 16);
  ForwardPlan f{};
  if ((rc = plan_forward(d, m, has_len, cus, xcds, wreg_ok, rsv != nullptr, &f)) != RNN_OK) return rc;
  const bool wave = f.wave;
  const ScanPlan& p = f.p;
  // the scan addresses one layer's rings, and one step's rows of G_x and y,
  // with 32-bit byte offsets
  if (!wave && (std::max(hx_ring_bytes(d, m), mx_ring_bytes(d, m)) >= ((size_t)1 << 31) ||
                (size_t)d->B * m.D * m.G * 4 >= ((size_t)1 << 31) ||
                (size_t)d->B * m.D * m.K * es >= ((size_t)1 << 31)))
    return RNN_E_PLAN;
  const ReserveLayout RL = reserve_of(d, m);

  // The one-wave scan forms a narrow layer's G_x itself from x in LDS; when
  // it does so for every layer, the forward is its launches alone (the
  // first clears the status word, which nothing else here uses).
  auto wave_fuses = [&](int l, const void* in) {
    const int in_l = l == 0 ? d->input_size : m.D * m.K;
    return wave && scan_wave_fuses(in_l, (int)es, t_max) && aligned(in, 16);
  };
  bool all_fused = wave && aligned(io->x, 16);
  for (int l = 0; l < d->num_layers && all_fused; ++l) all_fused = wave_fuses(l, l == 0 ? io->x : ws);

  // ---- enqueue ----
  // the pipelined path zeroes the status word and counters with its first
  // ring fill
  if (f.pipe) return forward_rnn_pipe(d, w, io, ws, L, m, f, st, xcds, prof);
  // status word and counters (unless the one-wave scan clears the status
  // itself) and the exchange rings of the tiled scan, in one launch
  if ((rc = hip_status(launch_fill2_u32(ws, all_fused ? 0 : L.counters + L.counters_bytes, 0u, ws + L.ex,
                                        wave ? 0 : L.ring_end - L.ex, 0xFFFFFFFFu, st))) != RNN_OK)
    return rc;
  int* dev_len = nullptr;
  int* dev_off = nullptr;
  if (has_len) {
    std::vector<int> ints((size_t)d->B + d->T + 1, 0);
    for (int b = 0; b < d->B; ++b) ints[b] = io->lengths_host[b];
    if (d->layout == RNN_LAYOUT_PACKED) {
      // offsets[t] = sum_b min(L_b, t): first packed row of step t
      long long acc = 0;
      for (int t = 0; t <= d->T; ++t) {
        ints[d->B + t] = (int)acc;
        for (int b = 0; b < d->B; ++b)
          if (io->lengths_host[b] > t) ++acc;
      }
    }
    dev_len = (int*)(ws + L.ints);
    dev_off = dev_len + d->B;
    if ((rc = hip_status(launch_write_ints(dev_len, ints.data(), (int)ints.size(), st))) != RNN_OK) return rc;
  }

  const bool bf16 = d->dtype == RNN_DTYPE_BF16;
  // padded var-len: the reserved layer outputs are read at every position
  // by the backward's products, so the ones the scan never writes are zero
  if (rsv && has_len && d->layout == RNN_LAYOUT_PADDED)
    for (int l = 0; l + 1 < d->num_layers; ++l)
      if ((rc = hip_status(launch_fill_zero(rsv + RL.y[l], (size_t)m.rows * m.D * m.K * 4, st))) != RNN_OK)
        return rc;
  void* gx = ws + L.gx;
  const int gx_bf16 = !wave && gx_esize(d, m) == 2;
  const void* layer_in = io->x;
  for (int l = 0; l < d->num_layers; ++l) {
    void* layer_out = l == d->num_layers - 1 ? io->y
                      : rsv ? (void*)(rsv + RL.y[l])
                            : (void*)(ws + ((l % 2 == 0) ? L.inter0 : L.inter1));
    // Kernel 1: Gx for every row of this layer, both directions (unless the
    // one-wave scan forms it).
    const bool fused = wave_fuses(l, layer_in);
    if (!fused) {
      const GemmArgs g = layer_gemm(d, w, m, l, layer_in, 0, (int)m.rows, gx, gx_bf16, ws, L, true);
      if ((rc = prof.begin(1, l)) != RNN_OK) return rc;
      if ((rc = hip_status(launch_gemm_xw(g, bf16, st))) != RNN_OK) return rc;
      if ((rc = prof.end()) != RNN_OK) return rc;
    }

    // Kernel 2: the scan.
    ScanArgs a = wave ? ScanArgs{} : layer_scan(d, w, m, p, xcds, l, ws, L);
    if (f.sp.on) {
      a.hs = f.sp.hs; a.ns = f.sp.ns; a.gpx = f.sp.gpx; a.nxcd = xcds;
      a.Kp = 64 * scan_small_chunks(m.K);
    }
    if (wave) {
      a.mode = d->mode == RNN_MODE_GRU ? kGRU : (d->mode == RNN_MODE_LSTMP ? kLSTMP : kLSTM);
      a.B = d->B; a.H = d->hidden_size; a.K = m.K; a.P = d->proj_size; a.D = m.D; a.G = m.G;
      a.packed = d->layout == RNN_LAYOUT_PACKED;
      a.has_bias = d->has_bias;
      const float inf = std::numeric_limits<float>::infinity();
      const bool cclip = d->clip & RNN_CLIP_CELL;
      a.c_lo = cclip ? d->cell_clip_lo : -inf;
      a.c_hi = cclip ? d->cell_clip_hi : inf;
      a.p_lo = -inf;
      a.p_hi = inf;
      for (int di = 0; di < m.D; ++di) {
        const int i = l * m.D + di;
        a.w_hh[di] = w->w_hh[i];
        a.b_hh[di] = d->has_bias ? w->b_hh[i] : nullptr;
        a.w_ih[di] = w->w_ih[i];
        a.b_ih[di] = d->has_bias ? w->b_ih[i] : nullptr;
      }
      a.status = (int*)(ws + L.status);
      a.x = fused ? layer_in : nullptr;
      a.in_w = l == 0 ? d->input_size : m.D * m.K;
      a.zero_status = all_fused && l == 0;
    }
    a.nslot = 1;
    a.T[0] = t_max;
    for (int di = 0; di < m.D; ++di) {
      const int i = l * m.D + di;
      a.h0[di] = io->h0 ? (const char*)io->h0 + (size_t)i * d->B * m.K * es : nullptr;
      a.c0[di] = (d->mode != RNN_MODE_GRU && io->c0) ? (const char*)io->c0 + (size_t)i * d->B * d->hidden_size * es : nullptr;
      a.h_n[di] = io->h_n ? (char*)io->h_n + (size_t)i * d->B * m.K * es : nullptr;
      a.c_n[di] = (d->mode != RNN_MODE_GRU && io->c_n) ? (char*)io->c_n + (size_t)i * d->B * d->hidden_size * es : nullptr;
    }
    a.gx[0] = gx;
    a.gx_bf16 = gx_bf16;
    a.y[0] = layer_out;
    a.rsv = rsv ? (float*)(rsv + RL.gates[l]) : nullptr;
    a.lengths = dev_len;
    a.offsets = dev_off;
    if ((rc = prof.begin(wave ? 4 : 2, l)) != RNN_OK) return rc;
    if ((rc = hip_status(wave        ? launch_scan_wave(a, bf16, st)
                         : f.sp.on ? launch_scan_small(a, bf16, st)
                                   : launch_scan(a, bf16, st))) != RNN_OK)
      return rc;
    if ((rc = prof.end()) != RNN_OK) return rc;
    layer_in = layer_out;
  }
  return RNN_OK;
}


// ---------------------------------------------------------------------------
// Backward through time (training)
// ---------------------------------------------------------------------------
constexpr int kBwdMaxMembers = kScanBwdMaxMembers;

struct BwdPlan {
  int bb, hs, ns, nbb, kp, lds, ps, acc_cols;
};

// Same shape of search as plan_scan: every group co-resident, LDS within a
// CU, elements per thread bounded; the step model adds the partial-sum
// exchange (write a row block of all H columns, read the owned columns of
// every member).
int plan_scan_bwd(const RnnDesc* d, const Dims& m, int cus, BwdPlan* out) {
  const int H = d->hidden_size, B = d->B, Hp = m.Kp;  // partial-sum width: the recurrent width K, padded
  const bool proj = d->mode == RNN_MODE_LSTMP;
  std::vector<int> bbs, hss;
  if (d->tile_batch > 0) {
    bbs.push_back(d->tile_batch);
  } else {
    for (int bb = 1; bb < B; bb *= 2) bbs.push_back(bb);
    bbs.push_back(B);
  }
  if (d->tile_hidden > 0) {
    hss.push_back(d->tile_hidden);
  } else {
    for (int hs = 4; hs <= std::max(4, rup(H, 4)); hs *= 2) hss.push_back(hs);
  }
  double best = 1e30;
  bool found = false;
  for (int bb : bbs) {
    for (int hs : hss) {
      if (bb < 1 || hs < 1 || hs % 4 != 0 || bb * hs > 1024) continue;
      const int ns = cdiv(H, hs), nbb = cdiv(B, bb);
      if (ns > kBwdMaxMembers || (long long)m.D * nbb * ns > cus) continue;
      const int ps = proj ? cdiv(m.K, ns) : 0;
      if (bb * ps > 1024) continue;
      ScanBwdArgs a{};
      a.mode = d->mode == RNN_MODE_GRU ? kGRU : (proj ? kLSTMP : kLSTM);
      a.bb = bb; a.hs = hs; a.Hp = Hp; a.kp = rup(m.gates * hs, 16);
      a.P = m.K; a.Pp = Hp; a.ps = ps;
      // the partial product passes through LDS in as few column passes as fit
      int passes = 1, lds = 0;
      for (; passes <= 8; passes *= 2) {
        a.acc_cols = Hp / passes;
        if (proj || a.acc_cols % 16 != 0) a.acc_cols = Hp;
        lds = scan_bwd_lds_bytes(a);
        if (lds <= kMaxLds || proj || a.acc_cols % 32 != 0) break;
      }
      if (lds > kMaxLds) continue;
      const double xbytes = (double)ns * std::min(bb, B) * (proj ? ps : hs) * 4 + (double)bb * Hp * 4;
      double t = barrier_us(ns) + xbytes / 100e3 + mm_us(bb % 16 == 0, 4, bb, Hp, a.kp);
      if (proj) t += barrier_us(ns) + (double)bb * Hp * 4 / 100e3 + mm_us(bb % 16 == 0, 4, bb, rup(hs, 16), Hp);
      t += 0.1 * (Hp / a.acc_cols - 1);  // a barrier per extra pass
      // every member writes its partial sums of all columns each step: the
      // device-wide exchange grows with the member count
      t += (double)m.D * B * ns * Hp * 4 * 2 / 5e6;
      if (t < best) {
        best = t;
        *out = BwdPlan{bb, hs, ns, nbb, a.kp, lds, ps, a.acc_cols};
        found = true;
      }
    }
  }
  return found ? RNN_OK : RNN_E_PLAN;
}

struct BwdLayout {
  size_t status, counters, ints, dgx, dgh, hprev, dx0, dx1, ex, part, gpart, ex2, dh, mbuf, total;
  size_t counters_bytes;
  int n_ints;
};

BwdLayout bwd_layout_of(const RnnDesc* d, const Dims& m, bool has_lengths) {
  BwdLayout w{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes, kAlign);
    return at;
  };
  const size_t rows = (size_t)m.rows;
  w.status = take(kAlign);
  w.counters_bytes = (size_t)d->num_layers * m.D * d->B * kCounterBytes;
  w.counters = take(w.counters_bytes);
  w.n_ints = has_lengths ? d->B + d->T + 1 : 0;
  w.ints = take((size_t)std::max(w.n_ints, 1) * 4);
  w.dgx = take(rows * m.D * m.G * 4);
  w.dgh = d->mode == RNN_MODE_GRU ? take(rows * m.D * m.G * 4) : w.dgx;
  w.hprev = take(rows * m.K * 4);
  const size_t dxb = rows * m.D * m.K * 4;
  w.dx0 = d->num_layers > 1 ? take(dxb) : 0;
  w.dx1 = d->num_layers > 2 ? take(dxb) : 0;
  w.ex = take((size_t)2 * m.D * kBwdMaxMembers * d->B * m.Kp * 4);
  w.part = take((size_t)kColsumChunks * std::max(m.G, m.K) * 4);
  // split-K partial products of the largest weight-gradient or dX product
  size_t gp = 0;
  const int rows_i = (int)rows;
  for (int l = 0; l < d->num_layers; ++l) {
    const int in_l = l == 0 ? d->input_size : m.D * m.K;
    gp = std::max({gp, gemm_gen_part_floats(m.G, in_l, rows_i), gemm_gen_part_floats(m.G, m.K, rows_i),
                   gemm_gen_part_floats(rows_i, in_l, m.G)});
    if (d->mode == RNN_MODE_LSTMP) gp = std::max(gp, gemm_gen_part_floats(m.K, d->hidden_size, rows_i));
  }
  w.gpart = take(std::max<size_t>(gp, 1) * 4);
  if (d->mode == RNN_MODE_LSTMP) {
    w.ex2 = take((size_t)m.D * d->B * m.Kp * 4);
    w.dh = take(rows * m.D * m.K * 4);
    w.mbuf = take(rows * d->hidden_size * 4);
  }
  w.total = o;
  return w;
}

int backward_rnn(const RnnDesc* d, const RnnWeights* w, const RnnIO* io, const RnnGrads* gr, const char* rsv,
                 size_t rsv_bytes, char* ws, size_t ws_bytes, hipStream_t st, int cus) {
  int rc;
  long long n_tok = 0;
  int t_max = 0;
  if ((rc = validate_lengths(d, io->lengths_host, &n_tok, &t_max)) != RNN_OK) return rc;
  const Dims m = dims_of(d, n_tok);
  const int LD = d->num_layers * m.D, H = d->hidden_size, G = m.G, K = m.K;
  const bool proj = d->mode == RNN_MODE_LSTMP;
  for (int i = 0; i < LD; ++i) {
    if ((rc = check_ptr(w->w_ih[i], 4)) != RNN_OK || (rc = check_ptr(w->w_hh[i], 4)) != RNN_OK) return rc;
    if ((rc = check_ptr(gr->dw_ih[i], 4)) != RNN_OK || (rc = check_ptr(gr->dw_hh[i], 4)) != RNN_OK) return rc;
    if (proj && ((rc = check_ptr(w->w_hr[i], 4)) != RNN_OK || (rc = check_ptr(gr->dw_hr[i], 4)) != RNN_OK))
      return rc;
    if (d->has_bias &&
        ((rc = check_ptr(gr->db_ih[i], 4)) != RNN_OK || (rc = check_ptr(gr->db_hh[i], 4)) != RNN_OK))
      return rc;
  }
  if ((rc = check_ptr(io->x, 4)) != RNN_OK || (rc = check_ptr(io->y, 4)) != RNN_OK) return rc;
  if ((rc = check_ptr(gr->dy, 4)) != RNN_OK || (rc = check_ptr(gr->dx, 4)) != RNN_OK) return rc;
  for (const void* p : {io->h0, io->c0, gr->dh_n, gr->dc_n, (const void*)gr->dh0, (const void*)gr->dc0})
    if ((rc = check_opt(p, 4)) != RNN_OK) return rc;
  const ReserveLayout RL = reserve_of(d, m);
  if (!rsv || rsv_bytes < RL.total) return RNN_E_WORKSPACE;
  const bool has_len = io->lengths_host != nullptr;
  const BwdLayout L = bwd_layout_of(d, m, has_len);
  if (!ws || ws_bytes < L.total) return RNN_E_WORKSPACE;
  if (!aligned(ws, 16) || !aligned(rsv, 16)) return RNN_E_ALIGN;
  BwdPlan p;
  if ((rc = plan_scan_bwd(d, m, cus, &p)) != RNN_OK) return rc;

  // ---- enqueue ----
  if ((rc = hip_status(launch_fill_zero(ws, L.counters + L.counters_bytes, st))) != RNN_OK) return rc;
  int* dev_len = nullptr;
  int* dev_off = nullptr;
  if (has_len) {
    std::vector<int> ints((size_t)d->B + d->T + 1, 0);
    for (int b = 0; b < d->B; ++b) ints[b] = io->lengths_host[b];
    if (d->layout == RNN_LAYOUT_PACKED) {
      long long acc = 0;
      for (int t = 0; t <= d->T; ++t) {
        ints[d->B + t] = (int)acc;
        for (int b = 0; b < d->B; ++b)
          if (io->lengths_host[b] > t) ++acc;
      }
    }
    dev_len = (int*)(ws + L.ints);
    dev_off = dev_len + d->B;
    if ((rc = hip_status(launch_write_ints(dev_len, ints.data(), (int)ints.size(), st))) != RNN_OK) return rc;
  }
  float* dgx = (float*)(ws + L.dgx);
  float* dgh = (float*)(ws + L.dgh);
  const size_t gbytes = (size_t)m.rows * m.D * G * 4;
  // padded var-len: positions the scan never writes must read as zero
  if (has_len && d->layout == RNN_LAYOUT_PADDED) {
    if ((rc = hip_status(launch_fill_zero(dgx, gbytes, st))) != RNN_OK) return rc;
    if (dgh != dgx && (rc = hip_status(launch_fill_zero(dgh, gbytes, st))) != RNN_OK) return rc;
    if (proj && (rc = hip_status(launch_fill_zero(ws + L.dh, (size_t)m.rows * m.D * K * 4, st))) != RNN_OK)
      return rc;
  }
  float* hprev = (float*)(ws + L.hprev);
  float* gpart = (float*)(ws + L.gpart);
  float* part = (float*)(ws + L.part);
  const size_t sB = (size_t)d->B * H, sK = (size_t)d->B * K;
  const int rows = (int)m.rows;
  for (int l = d->num_layers - 1; l >= 0; --l) {
    const float* y_l = l == d->num_layers - 1 ? (const float*)io->y : (const float*)(rsv + RL.y[l]);
    const float* dy_l = l == d->num_layers - 1 ? (const float*)gr->dy
                                               : (const float*)(ws + ((l % 2 == 0) ? L.dx0 : L.dx1));
    ScanBwdArgs a{};
    a.mode = d->mode == RNN_MODE_GRU ? kGRU : (proj ? kLSTMP : kLSTM);
    a.T = t_max; a.B = d->B; a.H = H; a.D = m.D; a.G = G;
    a.packed = d->layout == RNN_LAYOUT_PACKED;
    a.bb = p.bb; a.hs = p.hs; a.ns = p.ns; a.nbb = p.nbb; a.nxcd = 1; a.gpx = 0;
    a.Hp = m.Kp; a.kp = p.kp; a.acc_cols = p.acc_cols;
    a.P = K; a.Pp = m.Kp; a.ps = p.ps;
    a.dh = proj ? (float*)(ws + L.dh) : nullptr;
    a.ex2 = proj ? (float*)(ws + L.ex2) : nullptr;
    a.rsv = (const float*)(rsv + RL.gates[l]);
    a.y = y_l;
    a.dy = dy_l;
    for (int di = 0; di < m.D; ++di) {
      const int i = l * m.D + di;
      a.w_hh[di] = (const float*)w->w_hh[i];
      a.w_hr[di] = proj ? (const float*)w->w_hr[i] : nullptr;
      a.h0[di] = io->h0 ? (const float*)io->h0 + i * sK : nullptr;
      a.c0[di] = (d->mode != RNN_MODE_GRU && io->c0) ? (const float*)io->c0 + i * sB : nullptr;
      a.dh_n[di] = gr->dh_n ? (const float*)gr->dh_n + i * sK : nullptr;
      a.dc_n[di] = (d->mode != RNN_MODE_GRU && gr->dc_n) ? (const float*)gr->dc_n + i * sB : nullptr;
      a.dh0[di] = gr->dh0 ? (float*)gr->dh0 + i * sK : nullptr;
      a.dc0[di] = (d->mode != RNN_MODE_GRU && gr->dc0) ? (float*)gr->dc0 + i * sB : nullptr;
    }
    a.dgx = dgx;
    a.dgh = d->mode == RNN_MODE_GRU ? dgh : nullptr;
    a.lengths = dev_len;
    a.offsets = dev_off;
    a.ex = (float*)(ws + L.ex);
    a.counters = (unsigned*)(ws + L.counters + (size_t)l * m.D * d->B * kCounterBytes);
    a.status = (int*)(ws + L.status);
    if ((rc = hip_status(launch_scan_bwd(a, st))) != RNN_OK) return rc;

    const int in_l = l == 0 ? d->input_size : m.D * K;
    const float* x_l = l == 0 ? (const float*)io->x : (const float*)(rsv + RL.y[l - 1]);
    float* dx_l = l == 0 ? (float*)gr->dx : (float*)(ws + (((l - 1) % 2 == 0) ? L.dx0 : L.dx1));
    for (int di = 0; di < m.D; ++di) {
      const int i = l * m.D + di;
      // dW_ih = dG_x^T X_l
      GemmGenArgs g{};
      g.A = dgx + di * G; g.sam = 1; g.sak = (long long)m.D * G;
      g.B = x_l; g.sbk = in_l; g.sbn = 1;
      g.C = (float*)gr->dw_ih[i]; g.ldc = in_l;
      g.M = G; g.N = in_l; g.K = rows; g.accumulate = 0;
      g.part = gpart;
      if ((rc = hip_status(launch_gemm_gen(g, st))) != RNN_OK) return rc;
      // dW_hh = dG_h^T H_prev
      HprevArgs hp{};
      hp.y = y_l; hp.ldy = m.D * K; hp.col0 = di * K;
      hp.h0 = a.h0[di];
      hp.out = hprev;
      hp.T = t_max; hp.B = d->B; hp.H = K; hp.packed = a.packed; hp.rev = di == 1;
      hp.lengths = dev_len; hp.offsets = dev_off;
      if ((rc = hip_status(launch_hprev(hp, st))) != RNN_OK) return rc;
      GemmGenArgs gh{};
      gh.A = dgh + di * G; gh.sam = 1; gh.sak = (long long)m.D * G;
      gh.B = hprev; gh.sbk = K; gh.sbn = 1;
      gh.C = (float*)gr->dw_hh[i]; gh.ldc = K;
      gh.M = G; gh.N = K; gh.K = rows; gh.accumulate = 0;
      gh.part = gpart;
      if ((rc = hip_status(launch_gemm_gen(gh, st))) != RNN_OK) return rc;
      if (proj) {  // dW_hr = dh^T m, m = o tanh(c) from the reserve
        float* mbuf = (float*)(ws + L.mbuf);
        if ((rc = hip_status(launch_mgather(a.rsv, m.D, di, H, m.rows, mbuf, st))) != RNN_OK) return rc;
        GemmGenArgs gr2{};
        gr2.A = (const float*)(ws + L.dh) + di * K; gr2.sam = 1; gr2.sak = (long long)m.D * K;
        gr2.B = mbuf; gr2.sbk = H; gr2.sbn = 1;
        gr2.C = (float*)gr->dw_hr[i]; gr2.ldc = H;
        gr2.M = K; gr2.N = H; gr2.K = rows; gr2.accumulate = 0;
        gr2.part = gpart;
      if ((rc = hip_status(launch_gemm_gen(gr2, st))) != RNN_OK) return rc;
      }
      if (d->has_bias) {
        if ((rc = hip_status(launch_colsum(dgx + di * G, (long long)m.D * G, rows, G, part, kColsumChunks,
                                           (float*)gr->db_ih[i], st))) != RNN_OK)
          return rc;
        if ((rc = hip_status(launch_colsum(dgh + di * G, (long long)m.D * G, rows, G, part, kColsumChunks,
                                           (float*)gr->db_hh[i], st))) != RNN_OK)
          return rc;
      }
      // dX_l (+)= dG_x W_ih
      GemmGenArgs gx{};
      gx.A = dgx + di * G; gx.sam = (long long)m.D * G; gx.sak = 1;
      gx.B = (const float*)w->w_ih[i]; gx.sbk = in_l; gx.sbn = 1;
      gx.C = dx_l; gx.ldc = in_l;
      gx.M = rows; gx.N = in_l; gx.K = G; gx.accumulate = di > 0;
      gx.part = gpart;
      if ((rc = hip_status(launch_gemm_gen(gx, st))) != RNN_OK) return rc;
    }
  }
  return RNN_OK;
}

// ---------------------------------------------------------------------------
// Library-owned workspace of rnn_forward_noalloc. Each device the library
// runs on holds its own copy of the array from the code object's load until
// the process ends. In host code `scratch` names a host-side stand-in, not
// device memory: only the address hipGetSymbolAddress returns for the
// current device may be handed to kernels.
// ---------------------------------------------------------------------------
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) char scratch[RNN_NOALLOC_MAX_WORKSPACE];

namespace {

// Device address of `scratch` on the current device, looked up once per
// device with that device current.
int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return RNN_E_DEVICE;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return RNN_E_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return RNN_OK;
}

}  // namespace

extern "C" {

int rnn_abi_version(void) { return RNN_ABI_VERSION; }

const char* rnn_strerror(int status) {
  switch (status) {
    case RNN_OK: return "ok";
    case RNN_E_NULL: return "a required pointer is NULL";
    case RNN_E_SHAPE: return "a size is out of range or inconsistent";
    case RNN_E_UNSUPPORTED: return "unsupported combination of mode, dtype, layout or options";
    case RNN_E_LENGTHS: return "sequence lengths out of range, missing, or not sorted non-increasing for the packed layout";
    case RNN_E_WORKSPACE: return "workspace missing or too small";
    case RNN_E_ALIGN: return "a pointer is not aligned to its element size (workspace: 16 bytes)";
    case RNN_E_DEVICE: return "no gfx950 device is current";
    case RNN_E_HIP: return "a HIP runtime call or kernel launch failed";
    case RNN_E_TIMEOUT: return "a step barrier timed out on the device (workgroups not co-resident)";
    case RNN_E_PLAN: return "the problem does not fit the persistent kernels' on-chip residency limits";
    default: return "unknown status";
  }
}

int rnn_workspace_bytes(const RnnDesc* desc, const int32_t* lengths_host, size_t* bytes) {
  int rc = validate_desc(desc);
  if (rc != RNN_OK) return rc;
  if (!bytes) return RNN_E_NULL;
  long long n_tok = 0;
  int t_max = 0;
  if ((rc = validate_lengths(desc, lengths_host, &n_tok, &t_max)) != RNN_OK) return rc;
  *bytes = layout_of(desc, n_tok, lengths_host != nullptr).total;
  return RNN_OK;
}

int rnn_plan_info(const RnnDesc* desc, const int32_t* lengths_host, int cus, int xcds, int* info, int n_info) {
  int rc = validate_desc(desc);
  if (rc != RNN_OK) return rc;
  if (!info || n_info < 9) return RNN_E_NULL;
  if (cus < 1 || xcds < 1 || cus % xcds != 0) return RNN_E_SHAPE;
  for (int i = 0; i < n_info; ++i) info[i] = 0;
  if (is_rssm(desc->mode)) {
    RssmPlan p;
    if ((rc = plan_rssm(desc, cus, xcds, &p)) != RNN_OK) return rc;
    info[0] = 3; info[1] = rssm_grid(p, xcds); info[2] = p.lds; info[3] = p.rows; info[4] = p.h_per;
    info[5] = p.nw; info[6] = 0; info[7] = p.ngroups; info[8] = p.gpx;
    if (n_info >= 13) info[9] = p.reg;
    return RNN_OK;
  }
  long long n_tok = 0;
  int t_max = 0;
  if ((rc = validate_lengths(desc, lengths_host, &n_tok, &t_max)) != RNN_OK) return rc;
  const Dims m = dims_of(desc, n_tok);
  if (use_wave_scan(desc, m)) {
    // one wave per (direction, row): no co-residency needed, no LDS
    info[0] = 4; info[1] = scan_wave_grid(m.D, desc->B);
    info[2] = scan_wave_lds_bytes(desc->input_size, m.esize, t_max);  // x staged for layer 0
    info[3] = 1; info[4] = desc->hidden_size;
    info[5] = 1; info[6] = 0; info[7] = desc->B; info[8] = 0;
    return RNN_OK;
  }
  ForwardPlan f;
  rc = plan_forward(desc, m, lengths_host != nullptr, cus, xcds, (size_t)m.K * m.esize % 16 == 0, false, &f);
  if (rc != RNN_OK) return rc;
  if (f.sp.on) {
    // kernel 2c: groups of ns workgroups, one per (direction, row)
    info[0] = 5; info[1] = small_grid(f.sp, m.D * desc->B, xcds); info[2] = 0;
    info[3] = 1; info[4] = f.sp.hs; info[5] = f.sp.ns; info[6] = 0; info[7] = m.D * desc->B; info[8] = f.sp.gpx;
    return RNN_OK;
  }
  const ScanPlan& p = f.p;
  info[0] = 2; info[1] = scan_grid(p, (f.pipe ? desc->num_layers : 1) * m.D, xcds); info[2] = p.lds;
  info[3] = p.bb; info[4] = p.hs; info[5] = p.ns; info[6] = p.ps; info[7] = p.nbb; info[8] = p.gpx;
  if (n_info >= 13) {
    info[9] = p.wreg; info[10] = p.rnt; info[11] = p.rks; info[12] = p.rcpt;
  }
  if (n_info >= 14) info[13] = f.pipe ? f.ps.chunk : 0;
  if (n_info >= 15) info[14] = (int)std::lround(f.step_us * 1000.0);
  return RNN_OK;
}


int rnn_reserve_bytes(const RnnDesc* desc, const int32_t* lengths_host, size_t* bytes) {
  int rc = validate_desc(desc);
  if (rc != RNN_OK) return rc;
  if ((rc = validate_train(desc)) != RNN_OK) return rc;
  if (!bytes) return RNN_E_NULL;
  long long n_tok = 0;
  int t_max = 0;
  if ((rc = validate_lengths(desc, lengths_host, &n_tok, &t_max)) != RNN_OK) return rc;
  *bytes = reserve_of(desc, dims_of(desc, n_tok)).total;
  return RNN_OK;
}

int rnn_backward_workspace_bytes(const RnnDesc* desc, const int32_t* lengths_host, size_t* bytes) {
  int rc = validate_desc(desc);
  if (rc != RNN_OK) return rc;
  if ((rc = validate_train(desc)) != RNN_OK) return rc;
  if (!bytes) return RNN_E_NULL;
  long long n_tok = 0;
  int t_max = 0;
  if ((rc = validate_lengths(desc, lengths_host, &n_tok, &t_max)) != RNN_OK) return rc;
  *bytes = bwd_layout_of(desc, dims_of(desc, n_tok), lengths_host != nullptr).total;
  return RNN_OK;
}

int rnn_forward_train(const RnnDesc* desc, const RnnWeights* weights, const RnnIO* io, void* reserve,
                      size_t reserve_bytes, void* workspace, size_t ws_bytes, void* stream) {
  Range range("rnn_forward_train");
  int rc = validate_desc(desc);
  if (rc != RNN_OK) return rc;
  if ((rc = validate_train(desc)) != RNN_OK) return rc;
  if (!weights || !io) return RNN_E_NULL;
  long long n_tok = 0;
  int t_max = 0;
  if ((rc = validate_lengths(desc, io->lengths_host, &n_tok, &t_max)) != RNN_OK) return rc;
  if (!reserve || reserve_bytes < reserve_of(desc, dims_of(desc, n_tok)).total) return RNN_E_WORKSPACE;
  if (!aligned(reserve, 16)) return RNN_E_ALIGN;
  DeviceInfo info;
  if ((rc = current_device_info(&info)) != RNN_OK) return rc;
  Prof prof;
  return forward_rnn(desc, weights, io, (char*)workspace, ws_bytes, reinterpret_cast<hipStream_t>(stream),
                     info.cus, info.xcds, prof, (char*)reserve);
}

int rnn_backward(const RnnDesc* desc, const RnnWeights* weights, const RnnIO* io, const RnnGrads* grads,
                 const void* reserve, size_t reserve_bytes, void* workspace, size_t ws_bytes, void* stream) {
  Range range("rnn_backward");
  int rc = validate_desc(desc);
  if (rc != RNN_OK) return rc;
  if ((rc = validate_train(desc)) != RNN_OK) return rc;
  if (!weights || !io || !grads) return RNN_E_NULL;
  DeviceInfo info;
  if ((rc = current_device_info(&info)) != RNN_OK) return rc;
  return backward_rnn(desc, weights, io, grads, (const char*)reserve, reserve_bytes, (char*)workspace, ws_bytes,
                      reinterpret_cast<hipStream_t>(stream), info.cus);
}

int rnn_device_check(void) {
  DeviceInfo info;
  return current_device_info(&info);
}

int rnn_exchange_roundtrip_ns(void* buffer, size_t bytes, int iters, void* stream, double* ns_per_round_trip) {
  if (!buffer || !ns_per_round_trip) return RNN_E_NULL;
  if (bytes < 1024 || iters < 1 || iters > 100000) return RNN_E_SHAPE;
  if (!aligned(buffer, 256)) return RNN_E_ALIGN;
  DeviceInfo info;
  int rc = current_device_info(&info);
  if (rc != RNN_OK) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* b = static_cast<char*>(buffer);
  unsigned long long* out = reinterpret_cast<unsigned long long*>(b + 512);
  if ((rc = hip_status(launch_fill_zero(b, 1024, st))) != RNN_OK) return rc;
  if ((rc = hip_status(launch_exchange_probe(b, iters, out, st))) != RNN_OK) return rc;
  if (hipStreamSynchronize(st) != hipSuccess) return RNN_E_HIP;
  unsigned long long h[3] = {0, 0, 0};
  if (hipMemcpy(h, out, sizeof h, hipMemcpyDeviceToHost) != hipSuccess) return RNN_E_HIP;
  if (h[1] || h[2]) return RNN_E_TIMEOUT;
  *ns_per_round_trip = (double)h[0] * 10.0 / iters;  // 100 MHz real-time clock
  return RNN_OK;
}

int rnn_forward_profiled(const RnnDesc* desc, const RnnWeights* weights, const RnnIO* io, void* workspace,
                         size_t ws_bytes, void* stream, void* const* events, int n_events, int* kinds,
                         int* n_kernels) {
  Range range("rnn_forward");
  int rc = validate_desc(desc);
  if (rc != RNN_OK) return rc;
  if (!weights || !io) return RNN_E_NULL;
  if (!is_rssm(desc->mode)) {
    long long n_tok = 0;
    int t_max = 0;
    if ((rc = validate_lengths(desc, io->lengths_host, &n_tok, &t_max)) != RNN_OK) return rc;
  }
  DeviceInfo info;
  if ((rc = current_device_info(&info)) != RNN_OK) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (n_events < 0) return RNN_E_SHAPE;
  if (n_events > 0 && !events) return RNN_E_NULL;
  Prof prof;
  prof.events = events;
  prof.n_events = n_events;
  prof.kinds = kinds;
  prof.st = st;
  rc = is_rssm(desc->mode)
           ? forward_rssm(desc, weights, io, (char*)workspace, ws_bytes, st, info.cus, info.xcds, prof)
           : forward_rnn(desc, weights, io, (char*)workspace, ws_bytes, st, info.cus, info.xcds, prof);
  if (n_kernels) *n_kernels = prof.n;
  return rc;
}

int rnn_forward(const RnnDesc* desc, const RnnWeights* weights, const RnnIO* io, void* workspace,
                size_t ws_bytes, void* stream) {
  return rnn_forward_profiled(desc, weights, io, workspace, ws_bytes, stream, nullptr, 0, nullptr, nullptr);
}

int rnn_forward_noalloc(const RnnDesc* desc, const RnnWeights* weights, const RnnIO* io, void* stream,
                        int32_t* device_status) {
  Range range("rnn_forward_noalloc");
  int rc = validate_desc(desc);
  if (rc != RNN_OK) return rc;
  if (!weights || !io) return RNN_E_NULL;
  long long n_tok = 0;
  int t_max = 0;
  const int32_t* lens = is_rssm(desc->mode) ? nullptr : io->lengths_host;
  if ((rc = validate_lengths(desc, lens, &n_tok, &t_max)) != RNN_OK) return rc;
  if (layout_of(desc, n_tok, lens != nullptr).total > (size_t)RNN_NOALLOC_MAX_WORKSPACE) return RNN_E_WORKSPACE;
  if (device_status && !aligned(device_status, 4)) return RNN_E_ALIGN;
  DeviceInfo info;
  if ((rc = current_device_info(&info)) != RNN_OK) return rc;
  void* ws = nullptr;
  if ((rc = scratch_on_current_device(&ws)) != RNN_OK) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  Prof prof;
  char* w = static_cast<char*>(ws);
  rc = is_rssm(desc->mode)
           ? forward_rssm(desc, weights, io, w, RNN_NOALLOC_MAX_WORKSPACE, st, info.cus, info.xcds, prof)
           : forward_rnn(desc, weights, io, w, RNN_NOALLOC_MAX_WORKSPACE, st, info.cus, info.xcds, prof);
  if (rc == RNN_OK && device_status)
    rc = hip_status(launch_copy_int(device_status, reinterpret_cast<const int*>(w), st));
  return rc;
}

int rnn_read_status(const void* workspace, void* stream, int* device_status) {
  if (!workspace || !device_status) return RNN_E_NULL;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(st) != hipSuccess) return RNN_E_HIP;
  int v = 0;
  if (hipMemcpy(&v, workspace, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess) return RNN_E_HIP;
  *device_status = v;
  return RNN_OK;
}

}  // extern "C"
