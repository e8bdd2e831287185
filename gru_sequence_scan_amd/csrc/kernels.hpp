// Launch interface between the host library and the gfx950 kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rnnk {

// Timing events for the launches of one bracket (host side, per thread; set
// only by the profiled entry point). The first launch after they are set
// records `start` when its dispatch begins; every launch records `stop` when
// it completes. The events travel with the dispatch packets, so timing adds
// no packets (and no gaps) between kernels.
struct LaunchEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
LaunchEvents& launch_events();

template <typename F, typename... Args>
inline void launch_kernel(F kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t stream, Args... args) {
  LaunchEvents& ev = launch_events();
  hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, ev.start, ev.stop, 0u, args...);
  ev.start = nullptr;
}

// Kernel 1: Gx = X W^T + folded bias, both directions in one launch.
struct GemmArgs {
  const void* A;        // [M, K] storage dtype
  const void* W[2];     // per direction [G, K]
  const void* b_ih[2];  // per direction [G] (has_bias)
  const void* b_hh[2];  // per direction [G] (has_bias)
  void* C;              // [M, N], N = D * G: fp32, or bf16 when c_bf16
  int c_bf16;           // store C (with the bias fold) as bf16
  int M, N, K, G;
  int hh_fold_rows;     // b_hh folded for gate rows < this (G, or 2H for GRU)
  int has_bias;
  int vec_ok;           // A and W rows 16-byte aligned (K * esize % 16 == 0)
  const void* zero16;   // 16 zero bytes in device memory (stand-in for rows past M or N)
  int splits;           // > 1: K split over blockIdx.y, partial tiles summed by a second kernel
  float* part;          // [splits][M][N] partial products (splits > 1)
};
// Split of K for a product with few output tiles (1 = none); the same figure
// sizes the workspace and drives the launch.
int gemm_xw_splits(long long M, int N, int K, int dtype_bf16);
hipError_t launch_gemm_xw(const GemmArgs& a, int dtype_bf16, hipStream_t stream);

// Kernel 2: persistent scan over time for one layer, all directions.
enum ScanMode { kLSTM = 0, kGRU = 1, kLSTMP = 2 };

// Layer slots of one scan launch: stacked layers whose time chunks are
// scanned together (layer pipelining, one direction).
constexpr int kScanMaxSlots = 8;

struct ScanArgs {
  int mode;          // ScanMode
  int nslot;         // layer slots (1, or up to kScanMaxSlots with D = 1);
                     // groups are numbered slot-major
  int T[kScanMaxSlots];  // time steps looped over per slot (T_max); 0: idle
  int B, H, K, P;    // K = recurrent width (H, or P for LSTMP)
  int D;             // directions
  int G;             // gate rows per direction
  int packed;        // 1: rows of step t start at offsets[t]
  int has_bias;
  // tiling
  int bb;            // batch rows per workgroup
  int hs;            // hidden units per workgroup
  int ns;            // workgroups per group (one group = one direction x batch block)
  int ps;            // projection outputs per workgroup (LSTMP)
  int nbb;           // batch blocks
  int nxcd;          // XCDs the launch is dealt over (round-robin by workgroup id)
  int gpx;           // > 0: groups per XCD, members of a group share one XCD;
                     // 0: consecutive workgroup ids form a group
  int Kp, Hp;        // padded widths of the exchange rows (multiples of 32)
  // Where each workgroup keeps its W_hh slice: wreg = 0 in LDS; wreg = 1 in
  // registers (kScanRegChunks 16-byte chunks per lane). MFMA register path
  // (rnt = 1, 2, 4): each wave holds rnt 16-column tiles over 1/rks of K,
  // rcpt chunks per tile. VALU register path (rnt = 0): thread t holds
  // output column t % (256 / rks) over K slice t / (256 / rks), rcpt chunks.
  int wreg, rnt, rks, rcpt;
  // LSTMP projection product (W_hr slice in LDS) on MFMA: pnt column tiles
  // per wave, pks waves splitting K, pcpt chunks each; pnt = 0: whole tiles
  // per wave without a K split.
  int pnt, pks, pcpt;
  // Clamp bounds of the updated cell state and of the projected output
  // (infinite when that clipping is off); NaN passes through.
  float c_lo, c_hi, p_lo, p_hi;
  // Training: per token and direction, the gate values the backward needs,
  // [rows, D, R] fp32 with R = 5H for LSTM (i, f, g, o, c_t) and 4H for GRU
  // (r, z, n, W_hn h_{t-1} + b_hn); null when not training.
  float* rsv;
  // per (slot, direction) tensors, index slot * D + d, already offset to
  // the slot's layer
  const void* w_hh[kScanMaxSlots];
  const void* w_hr[kScanMaxSlots];
  const void* b_hh[kScanMaxSlots];
  const void* h0[kScanMaxSlots];   // [B, K] or null
  const void* c0[kScanMaxSlots];   // [B, H] or null
  void* h_n[kScanMaxSlots];        // [B, K] or null
  void* c_n[kScanMaxSlots];        // [B, H] or null
  // fp32 copies of the carried state (time-chunked runs: bit-identical to an
  // unchunked one): initial h (GRU's update reads it; [B, H]) and c ([B, H])
  // and the final ones; each null when unused
  const float* h0f[kScanMaxSlots];
  const float* c0f[kScanMaxSlots];
  float* h_nf[kScanMaxSlots];
  float* c_nf[kScanMaxSlots];
  // per slot
  const void* gx[kScanMaxSlots];  // [rows, D * G] fp32, or bf16 when gx_bf16
  void* y[kScanMaxSlots];         // [rows, D * K]
  // exchange (workspace): rings of write-once slots, all-ones before the
  // launch (kRingSlots slots in scan_common.hpp)
  void* hx[kScanMaxSlots];        // [4][D][B][Kp] h_t (LSTMP: the projected h_t)
  void* mx[kScanMaxSlots];        // [4][D][B][Hp] m_t (LSTMP)
  unsigned* xid[kScanMaxSlots];   // [D * nbb * ns] members' XCD ids
  int gx_bf16;
  const int* lengths;  // device [B] or null (all T)
  const int* offsets;  // device [T + 1] (packed)
  // One-wave scan with the input projection inside: x [rows, in_w] and the
  // per-direction W_ih [G, in_w] and b_ih [G] (x null: G_x comes from gx)
  const void* x;
  int in_w;
  const void* w_ih[kScanMaxSlots];
  const void* b_ih[kScanMaxSlots];
  int zero_status;     // the launch first clears *status (it is the forward's first)
  unsigned* counters;  // unused by the forward scan
  int* status;
};
constexpr int kScanRingSlots = 4;
constexpr int kScanMaxWorkgroups = 4096;  // xid entries per layer
hipError_t launch_scan(const ScanArgs& a, int dtype_bf16, hipStream_t stream);
constexpr int kScanRegChunks = 32;

// Kernel 2c: a few independent sequences (direction x batch row groups of
// at most kScanSmallMaxGroups), each a group of `ns` workgroups of eight
// waves owning `hs` hidden units per workgroup (hs / 8 per wave), W_hh rows
// in registers, h exchanged through an fp32 ring of row stride Kp >= 64 x
// scan_small_chunks(K). LSTM and GRU, K <= 512.
constexpr int kScanSmallMaxGroups = 8;
int scan_small_chunks(int K);               // K chunks per lane: 1, 2, 4 or 8 (0: K > 512)
int scan_small_units_per_wg(int units_per_wave);  // units_per_wave: 1, 2 or 4
hipError_t launch_scan_small(const ScanArgs& a, int dtype_bf16, hipStream_t stream);

// Kernel 2b: one wave per (direction, batch row) when the gate rows of all
// units fit one wave (LSTM and GRU with H <= 16; not LSTMP). Uses the
// ScanArgs problem fields, slot 0's tensors, lengths, offsets, the clip
// bounds, and x / in_w / w_ih / b_ih when it forms G_x itself
// (scan_wave_fuses: x rows of at most 128 bytes in whole 16-byte chunks,
// the longest sequence's x within 16 KB); no tiling, exchange or counters.
bool scan_wave_fits(int mode, int H, int K);
bool scan_wave_fuses(int in_w, int esize, long long max_steps);
int scan_wave_lds_bytes(int in_w, int esize, long long max_steps);  // per workgroup (0 unless fused)
int scan_wave_grid(int D, int B);
hipError_t launch_scan_wave(const ScanArgs& a, int dtype_bf16, hipStream_t stream);

// Backward of one layer's scan (all directions), persistent like the
// forward: a group of ns workgroups per (direction, batch block), each
// owning hs hidden units. Walks the forward's steps in the opposite order.
struct ScanBwdArgs {
  int mode;            // kLSTM or kGRU
  int T, B, H, D, G;   // recurrent width K == H
  int packed;
  int bb, hs, ns, nbb, nxcd, gpx;
  int Hp;              // exchange row width (H rounded up to 32)
  int kp;              // product depth: gates * hs rounded up to 16
  int acc_cols;        // columns of the partial product per pass (divides Hp, multiple of 16)
  const float* w_hh[2];  // [G, H]
  const float* rsv;      // [rows, D, R] this layer (see ScanArgs::rsv)
  const float* y;        // [rows, D * H] this layer's forward output
  const float* dy;       // [rows, D * H] gradient w.r.t. y
  const float* h0[2];    // [B, H] or null
  const float* c0[2];
  const float* dh_n[2];  // [B, H] or null
  const float* dc_n[2];
  float* dh0[2];         // [B, H] or null
  float* dc0[2];
  float* dgx;            // [rows, D, G] input-side pre-activation gradients
  float* dgh;            // [rows, D, G] hidden side (GRU; null for LSTM: same as dgx)
  const int* lengths;    // device [B] or null
  const int* offsets;    // device [T + 1] (packed)
  float* ex;             // [2][D][ns][B][Hp] per-member partial sums of W_hh^T dG
                         // (LSTMP: [2][D][ns][B][Pp], the partials over P)
  unsigned* counters;
  int* status;
  // LSTMP (mode kLSTMP): recurrent width P, members also own ps projection
  // outputs; dy, y, h0, dh_n, dh0 have width P.
  int P, Pp, ps;
  const float* w_hr[2];  // [P, H]
  float* dh;             // [rows, D, P] the step gradients w.r.t. h_t (for dW_hr)
  float* ex2;            // [D][B][Pp] the whole dh_t of the step, coherent
};
int scan_bwd_lds_bytes(const ScanBwdArgs& a);
constexpr int kScanBwdMaxMembers = 64;  // members per group of the backward scan
hipError_t launch_scan_bwd(const ScanBwdArgs& a, hipStream_t stream);

// C[m, n] (+)= sum_k A(m, k) B(k, n), fp32, with A(m, k) = A[m * sam + k * sak]
// and B(k, n) = B[k * sbk + n * sbn]: the backward's NN and TN products.
struct GemmGenArgs {
  const float* A; long long sam, sak;
  const float* B; long long sbk, sbn;
  float* C; long long ldc;
  int M, N, K;
  int accumulate;      // 1: C += product, 0: C = product
  float* part;         // split-K partial products, gemm_gen_part_floats(M, N, K) floats (may be null when 0)
  int vec_a, vec_b;    // set by launch_gemm_gen
};
// The split of K for an M x N x K product (independent of the device).
void gemm_gen_split(int M, int N, int K, int* splits, int* kchunk);
size_t gemm_gen_part_floats(int M, int N, int K);
hipError_t launch_gemm_gen(const GemmGenArgs& a, hipStream_t stream);
// out[n] = sum over m of A[m * lda + n] for n < N (fixed order), using
// `partial` (nchunk * N floats) for a two-pass deterministic reduction.
hipError_t launch_colsum(const float* A, long long lda, int M, int N, float* partial, int nchunk, float* out,
                         hipStream_t stream);
constexpr int kColsumChunks = 64;
// hprev[row(t, b), :] = the state entering step t of direction d for rows
// active at t (y of the previous step, or h0), zero for inactive rows.
struct HprevArgs {
  const float* y; int ldy, col0;   // y[row * ldy + col0 + j]
  const float* h0;                 // [B, H] or null
  float* out;                      // [rows, H]
  int T, B, H, packed, rev;
  const int* lengths;              // device [B] or null
  const int* offsets;              // device [T + 1] (packed)
};
hipError_t launch_hprev(const HprevArgs& a, hipStream_t stream);
// out[row, j] = o * tanh(c) of direction d from an LSTM reserve ([rows, D,
// 5H]: i, f, g, o, c), i.e. the cell output m_t that LSTMP projects.
hipError_t launch_mgather(const float* rsv, int D, int d, int H, long long rows, float* out, hipStream_t stream);

// Kernel 3: persistent RSSM-prior unroll.
struct RssmArgs {
  int B, T, S, A, E, Hb;
  float scale_lb;
  // tiling
  int rows;          // batch rows per group
  int ngroups;
  int nw;            // workgroups per group
  int h_per;         // GRU hidden units per workgroup
  int nxcd;          // XCDs the launch is dealt over (round-robin by workgroup id)
  int gpx;           // > 0: groups per XCD, members of a group share one XCD;
                     // 0: consecutive workgroup ids form a group
  const float* w_as; const float* b_as;
  const float* w_ih; const float* w_hh; const float* b_ih; const float* b_hh;
  const float* w_1; const float* b_1; const float* w_2; const float* b_2;
  const float* actions; const float* eps; const float* s0; const float* h0;
  float* means; float* stds; float* states; float* beliefs;
  // Actor in the loop (Ea > 0): a_t = tanh(W_a2 ELU(W_a1 [s_{t-1}; h_{t-1}]
  // + b_a1) + b_a2) replaces the given actions; act_out [B, T, A] or null.
  int Ea;
  const float* w_a1; const float* b_a1; const float* w_a2; const float* b_a2;
  float* act_out;
  // exchange (workspace)
  float* ex_h;   // kernel 3: [2][B][Hbp] whole h_t, ping-pong on t;
                 // kernel 3b: [4][B][Hbp] ring of write-once slots
  float* ex_p;   // kernel 3: [2][B][nw][Ep] per-member partial sums of W_1 h_t
                 // (columns 0..E-1) and, with an actor, of W_a1[:, S:] h_t
                 // (from r4(E)); kernel 3b: [4][B][nw][Ep] ring
  unsigned* xid; // kernel 3b: [ngroups][nw] members' XCC ids (sentinel-filled)
  int Ep, Hbp;
  unsigned* counters;  // [ngroups], 64 bytes apart
  int* status;
};
hipError_t launch_rssm(const RssmArgs& a, hipStream_t stream);
int rssm_lds_bytes(const RssmArgs& a);
// Kernel 3b: the RSSM prior (no actor) with wide members holding their GRU
// slices in registers and a ring exchange inside one XCD (gpx > 0 groups per
// XCD). The rings and xid hold the sentinel 0xFFFFFFFF before the launch.
bool rssm_reg_fits(const RssmArgs& a);
int rssm_reg_lds_bytes(const RssmArgs& a);
int rssm_ring_slots();
int rssm_reg_max_members();
hipError_t launch_rssm_reg(const RssmArgs& a, hipStream_t stream);
int rssm_max_rows();
constexpr int kRssmMaxMembers = 64;
int scan_lds_bytes(const ScanArgs& a, int esize);

// Copy up to kIntsPerLaunch host ints into device memory through kernel
// arguments (stream-ordered, no host staging buffer to keep alive).
constexpr int kIntsPerLaunch = 480;
hipError_t launch_write_ints(int* dst, const int* src, int n, hipStream_t stream);

// Zero-fill of small workspace regions (counters, status word).
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream);
// Fill with a 32-bit pattern (bytes a multiple of 4).
hipError_t launch_fill_u32(void* p, size_t bytes, uint32_t value, hipStream_t stream);
// Two fills in one launch: bytes1 at p1 with value1, bytes2 at p2 with value2.
hipError_t launch_fill2_u32(void* p1, size_t bytes1, uint32_t value1, void* p2, size_t bytes2, uint32_t value2,
                            hipStream_t stream);
// *dst = *src (one int, stream-ordered).
hipError_t launch_copy_int(int* dst, const int* src, hipStream_t stream);
// Device-coherent round trip between two workgroups on different XCDs:
// buf >= 512 bytes zeroed, out[0] = 100 MHz ticks for `iters` round trips,
// out[1], out[2] nonzero when a bounded wait ran out.
hipError_t launch_exchange_probe(void* buf, int iters, unsigned long long* out, hipStream_t stream);

}  // namespace rnnk
