/*
 * rnn.h -- C ABI of the gfx950 (MI355X) multi-timestep recurrence library.
 *
 * One call, rnn_forward, runs the whole forward of a recurrent stack on the
 * caller's HIP stream:
 *   mode LSTM         nn.LSTM forward (pytorch/pytorch issue "Integrating
 *                     CuDNN API for LSTMs with projections", Motivation and
 *                     design discussion), PyTorch gate order [i | f | g | o].
 *   mode LSTMP        LSTM with a recurrent projection h = W_hr (o * tanh c),
 *                     fed back as the recurrent input: an LSTM cell followed
 *                     by one more matrix product (same issue, design
 *                     discussion; arXiv 1402.1128 cited in its Feature
 *                     section).
 *   mode GRU          GRU with PyTorch's r/z/n convention (pytorch/rl issue
 *                     "[Feature Request] CUDNN version of RSSM", RSSMPrior uses
 *                     nn.GRUCell); the reset gate multiplies W_hn h + b_hn.
 *   mode RSSM_PRIOR   the RSSM prior unrolled over given actions (same rl
 *                     issue, Solution: RSSMPrior.forward and the first unroll),
 *                     with the Gaussian draw injected as a noise tensor.
 * Variable-length batches (per-sequence lengths as an extra argument, the
 * pack/unpack handled inside the op) and bidirectional stacks follow apache/
 * mxnet issue "RNN Op Changes (was: Variable Length Support for cuDNN RNN)",
 * RFC. The three dense ops are those named in apache/tvm PR "[TOPI] TE
 * implementation of LSTM using scan", description: input-hidden (hoisted
 * over all timesteps), hidden-hidden and hidden-projection (inside the
 * sequential time loop, which runs on the device).
 *
 * Conventions for every entry point:
 *   - Device pointers are HIP device allocations owned by the caller; the
 *     library allocates no device memory, keeps no pointer after returning
 *     and reads host arrays (lengths) only during the call.
 *   - Tensors are dense with C-canonical strides (pytorch/rl PR "LSTM/GRU
 *     scan: canonical strides + ...", description: a tensor can pass
 *     is_contiguous() and still carry non-canonical strides; callers must
 *     re-materialise). Every device pointer must be aligned to its
 *     element size and the workspace to 16 bytes; 16-byte aligned inputs
 *     and weights with rows of a multiple of 16 bytes take vector loads.
 *   - Weight pointers are read-only and may alias one flat storage (same PR:
 *     per-layer views of a single flat parameter storage).
 *   - All validation happens once, before anything is enqueued (same PR,
 *     review: do the layout work before the loop). Nothing is enqueued when
 *     a call returns an error.
 *   - The library keeps no mutable global state and reads no environment
 *     variables (same PR: a module-global mode flag leaked across threads),
 *     so calls may be made from several host threads. Two calls that share
 *     a workspace must be stream-ordered.
 *   - Device residency. The recurrence kernels (the scan, the backward scan
 *     and the RSSM kernel) are persistent: the workgroups of one group wait
 *     for each other every step, so all of them must be resident at once.
 *     The launch is sized to the device's compute units assuming nothing
 *     else runs on it. If other kernels (another call on another stream,
 *     or any other work) occupy compute units during such a launch, a group
 *     can be left partly resident; its members then give up after a bounded
 *     wait (about 2 s) and the call reports RNN_E_TIMEOUT through
 *     rnn_read_status, with invalid outputs. Calls never hang, but they
 *     succeed only when these kernels have the device to themselves:
 *     serialise calls (one stream, or events) rather than overlapping them.
 *   - Floating-point results are deterministic: the same inputs give the
 *     same bits (no floating-point atomics).
 */
#ifndef GRU_SEQUENCE_SCAN_RNN_H
#define GRU_SEQUENCE_SCAN_RNN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RNN_ABI_VERSION 2
#define RNN_MAX_LAYERS 8
#define RNN_MAX_LD (2 * RNN_MAX_LAYERS) /* layers x directions */

typedef enum RnnMode {
  RNN_MODE_LSTM = 0,
  RNN_MODE_GRU = 1,
  RNN_MODE_LSTMP = 2,
  RNN_MODE_RSSM_PRIOR = 3,
  RNN_MODE_RSSM_ACTOR = 4  /* the RSSM prior with an actor choosing each action
                              (pytorch/rl issue "[Feature Request] CUDNN
                              version of RSSM", Solution, second unroll);
                              the pages leave the actor undefined, here it is
                              a_t = tanh(W_a2 ELU(W_a1 [s_{t-1}; h_{t-1}]
                              + b_a1) + b_a2)                                  */
} RnnMode;

/* Storage type of weights, inputs, initial states and outputs. Arithmetic
 * always accumulates in fp32; the LSTM cell state is always carried in fp32
 * inside the kernels. */
typedef enum RnnDtype { RNN_DTYPE_F32 = 0, RNN_DTYPE_BF16 = 1 } RnnDtype;

typedef enum RnnLayout {
  RNN_LAYOUT_PADDED = 0,      /* x [T, B, F], y [T, B, D*K]                    */
  RNN_LAYOUT_PACKED = 1,      /* x [N_tok, F], y [N_tok, D*K]: step-major rows
                                 of the sequences still active at each step,
                                 lengths sorted non-increasing (PackedSequence) */
  RNN_LAYOUT_BATCH_MAJOR = 2  /* RSSM only: [B, T, .] like the unroll's stack
                                 on dim 1                                      */
} RnnLayout;

typedef enum RnnStatus {
  RNN_OK = 0,
  RNN_E_NULL = -1,        /* a required pointer is NULL                        */
  RNN_E_SHAPE = -2,       /* a size is out of range or inconsistent            */
  RNN_E_UNSUPPORTED = -3, /* combination not defined: projection outside LSTMP,
                             LSTMP without projection, bidirectional or
                             multi-layer RSSM, RSSM in bf16, clipping outside
                             LSTM / LSTMP, ...                                 */
  RNN_E_LENGTHS = -4,     /* a length outside [1, T], or packed lengths not
                             sorted non-increasing                             */
  RNN_E_WORKSPACE = -5,   /* workspace NULL or smaller than required           */
  RNN_E_ALIGN = -6,       /* a device pointer is not aligned to its element
                             size, or the workspace not to 16 bytes            */
  RNN_E_DEVICE = -7,      /* no usable gfx950 device is current                */
  RNN_E_HIP = -8,         /* a HIP runtime call or launch failed               */
  RNN_E_TIMEOUT = -9,     /* device status only: a step barrier waited too long
                             (workgroups were not co-resident); outputs are
                             invalid                                           */
  RNN_E_PLAN = -10        /* the problem does not fit the device's persistent
                             residency limits (e.g. weights exceed on-chip
                             capacity of the available compute units)          */
} RnnStatus;

/* Problem description (all sizes in elements). */
typedef struct RnnDesc {
  int32_t mode;          /* RnnMode                                            */
  int32_t dtype;         /* RnnDtype                                           */
  int32_t layout;        /* RnnLayout                                          */
  int32_t T;             /* time extent: padded buffers' T; for PACKED an upper
                            bound on the lengths; RSSM: unroll length (the
                            actor unroll's horizon)                           */
  int32_t B;             /* batch size                                         */
  int32_t input_size;    /* F of layer 0                                       */
  int32_t hidden_size;   /* H                                                  */
  int32_t proj_size;     /* P (> 0 exactly for LSTMP)                          */
  int32_t num_layers;    /* 1 .. RNN_MAX_LAYERS                                */
  int32_t bidirectional; /* 0 or 1                                             */
  int32_t has_bias;      /* 0: bias pointers ignored (treated as zero)         */
  /* RSSM prior dimensions (mode RSSM_PRIOR only) */
  int32_t state_dim;     /* S: stochastic state size                          */
  int32_t action_dim;    /* A                                                  */
  int32_t embed_dim;     /* E: width of the action-state and prior projector
                            hidden layers                                      */
  int32_t belief_dim;    /* Hb: GRU hidden size                               */
  float scale_lb;        /* lower bound added to softplus(raw scale)          */
  /* Launch-shape hints (0 = choose automatically). They change only how the
   * work is tiled, never which arithmetic is done per output element. */
  int32_t tile_batch;    /* batch rows per workgroup in the scan               */
  int32_t tile_hidden;   /* hidden units per workgroup in the scan             */
  int32_t placement;     /* 0: automatic (scan: XCD-aligned groups when they
                            fit; RSSM: consecutive ids); 1: consecutive
                            workgroup ids form a group; 2: every group on one
                            XCD when it fits                                  */
  int32_t weights;       /* scan W_hh slice: 0 automatic; 1 in LDS; 2 in
                            registers when a layout fits (else LDS)           */
  /* Clipping, LSTM and LSTMP only (apache/mxnet issue "RNN Op Changes",
   * discussion: cuDNN's cell clipping and the requests for state and
   * projection clipping; the pages name these without a formula, read here
   * as clamps). Bits of `clip`:
   *   RNN_CLIP_CELL  each updated cell state c_t is clamped to
   *                  [cell_clip_lo, cell_clip_hi] before tanh(c_t); the
   *                  clamped value is carried to the next step and is what
   *                  c_n reports.
   *   RNN_CLIP_PROJ  (LSTMP) each projected output h_t = W_hr m_t is clamped
   *                  to [-proj_clip, proj_clip]; the clamped value is the
   *                  output and the next step's recurrent input.
   * NaN passes through both clamps. Requirements: cell_clip_lo <=
   * cell_clip_hi, proj_clip >= 0, none NaN (infinite bounds are allowed);
   * otherwise RNN_E_SHAPE. A bit set for a mode without the quantity is
   * RNN_E_UNSUPPORTED; the float fields are ignored when their bit is clear. */
  int32_t clip;
  float cell_clip_lo;
  float cell_clip_hi;
  float proj_clip;
  int32_t actor_dim;     /* RSSM_ACTOR: hidden width Ea of the actor MLP (>= 1);
                            must be 0 in every other mode                     */
  int32_t gx_dtype;      /* storage of the hoisted input projection G_x (LSTM,
                            GRU, LSTMP): RNN_GX_AS_DTYPE (0) in the storage
                            dtype (bf16 for bf16 storage: the product is
                            accumulated in fp32 and rounded once), RNN_GX_F32
                            (1) in fp32; must be 0 in the RSSM modes          */
  int32_t layer_pipeline; /* launch-shape hint for unidirectional, padded,
                            fixed-length stacks of >= 2 LSTM / GRU / LSTMP
                            layers and T > 32: RNN_PIPE_AUTO (0) one launch
                            scans a time chunk of every layer, layer l one
                            chunk behind layer l - 1, when every layer's
                            groups fit on the device at once and the
                            launch-shape model expects a gain; RNN_PIPE_OFF
                            (1) layer by layer; RNN_PIPE_ON (2) pipelined
                            whenever it fits. Results are identical in all
                            three. Must be 0 for RSSM                       */
  int32_t reserved[1];   /* must be zero                                       */
} RnnDesc;

#define RNN_GX_AS_DTYPE 0
#define RNN_GX_F32 1
#define RNN_PIPE_AUTO 0
#define RNN_PIPE_OFF 1
#define RNN_PIPE_ON 2

#define RNN_CLIP_CELL 1
#define RNN_CLIP_PROJ 2

/* Weights, PyTorch shapes and meaning. Index i = layer * D + direction
 * (direction 0 forward, 1 reverse). G = 4H (LSTM, LSTMP) or 3H (GRU);
 * K = P for LSTMP, else H; in_l = input_size for layer 0, else D*K.
 *   w_ih[i]  [G, in_l]   w_hh[i] [G, K]   b_ih[i] [G]   b_hh[i] [G]
 *   w_hr[i]  [P, H]      (LSTMP only; no projection bias)
 * RSSM_PRIOR (single layer, forward): GRU cell in w_ih[0] [3Hb, E],
 * w_hh[0] [3Hb, Hb], b_ih[0], b_hh[0] [3Hb]; plus
 *   w_as [E, S + A] (columns: state first, then action), b_as [E]
 *   w_1  [E, Hb], b_1 [E]   (first prior-projector layer, reads the belief)
 *   w_2  [2S, E], b_2 [2S]  (rows 0..S-1 mean, S..2S-1 raw scale)
 * RSSM_ACTOR additionally (NULL otherwise):
 *   w_a1 [Ea, S + Hb] (columns: state first, then belief), b_a1 [Ea]
 *   w_a2 [A, Ea], b_a2 [A]
 * All in the RnnDesc dtype. */
typedef struct RnnWeights {
  const void* w_ih[RNN_MAX_LD];
  const void* w_hh[RNN_MAX_LD];
  const void* b_ih[RNN_MAX_LD];
  const void* b_hh[RNN_MAX_LD];
  const void* w_hr[RNN_MAX_LD];
  const void* w_as;
  const void* b_as;
  const void* w_1;
  const void* b_1;
  const void* w_2;
  const void* b_2;
  const void* w_a1;
  const void* b_a1;
  const void* w_a2;
  const void* b_a2;
} RnnWeights;

/* Inputs and outputs (device pointers unless noted), all in the RnnDesc dtype.
 *   x             PADDED [T, B, F] | PACKED [N_tok, F] | RSSM actions [B, T, A]
 *                 (ignored by RSSM_ACTOR, which computes its actions)
 *   lengths_host  HOST int32 [B]; NULL means every sequence has length T.
 *                 1 <= L_b <= T; PACKED requires L_0 >= L_1 >= ... and
 *                 N_tok = sum L_b. Row b is active at step t iff t < L_b; the
 *                 reverse direction of row b starts at t = L_b - 1 from h0.
 *   h0 [L*D, B, K], c0 [L*D, B, H]   NULL = zeros (RSSM: h0 = belief0 [B, Hb])
 *   s0            RSSM initial state [B, S], NULL = zeros
 *   noise         RSSM eps [B, T, S] (the unroll's Gaussian draw, injected)
 *   y             PADDED [T, B, D*K] (positions t >= L_b are never written)
 *                 | PACKED [N_tok, D*K]; forward half first on the last axis
 *   h_n [L*D, B, K], c_n [L*D, B, H]  each row's final state; NULL = skip
 *   means, stds, states [B, T, S], beliefs [B, T, Hb]  RSSM outputs
 *   actions       RSSM_ACTOR output [B, T, A]: the action each step used;
 *                 NULL = skip (ignored by the other modes)
 * Outputs must not overlap inputs or the workspace. */
typedef struct RnnIO {
  const void* x;
  const int32_t* lengths_host;
  const void* h0;
  const void* c0;
  const void* s0;
  const void* noise;
  void* y;
  void* h_n;
  void* c_n;
  void* means;
  void* stds;
  void* states;
  void* beliefs;
  void* actions;
} RnnIO;

/* Gradients for rnn_backward (device pointers, fp32, C-dense, canonical
 * shapes; the shapes of the tensors they are gradients of):
 *   dy    like y (PADDED [T, B, D*K] | PACKED [N_tok, D*K]), required;
 *         positions t >= L_b are never read
 *   dh_n  [L*D, B, K], dc_n [L*D, B, H] (LSTM, LSTMP) or NULL (= zero)
 *   dx    like x, required; written whole (zero at t >= L_b in PADDED)
 *   dh0 [L*D, B, K], dc0 [L*D, B, H] or NULL (= skip)
 *   dw_ih[i] [G, in_l], dw_hh[i] [G, K], db_ih[i], db_hh[i] [G] and, for
 *   LSTMP, dw_hr[i] [P, H], for i = l*D + d (bias gradients required when
 *   has_bias); written, not accumulated. K = P for LSTMP, else H. */
typedef struct RnnGrads {
  const void* dy;
  const void* dh_n;
  const void* dc_n;
  void* dx;
  void* dh0;
  void* dc0;
  void* dw_ih[RNN_MAX_LD];
  void* dw_hh[RNN_MAX_LD];
  void* db_ih[RNN_MAX_LD];
  void* db_hh[RNN_MAX_LD];
  void* dw_hr[RNN_MAX_LD];
} RnnGrads;

/* Version of this ABI (RNN_ABI_VERSION). */
int rnn_abi_version(void);

/* Static description of a status code; never NULL. */
const char* rnn_strerror(int status);

/* Validates desc (and lengths_host when given) and writes the workspace size
 * rnn_forward needs into *bytes. Host-only, touches no device. Returns
 * RNN_OK or a negative RnnStatus. */
int rnn_workspace_bytes(const RnnDesc* desc, const int32_t* lengths_host, size_t* bytes);

/* Enqueues the whole forward on `stream` (a hipStream_t; NULL = the null
 * stream of the current device) and returns once everything is enqueued,
 * without synchronising. `workspace` is caller-owned device memory of at
 * least rnn_workspace_bytes() bytes; its prior contents do not matter.
 * Returns RNN_OK, or a negative RnnStatus with nothing enqueued (RNN_E_HIP
 * when a launch fails after validation). Device-side failures (RNN_E_TIMEOUT)
 * are reported through rnn_read_status after the stream completes. */
int rnn_forward(const RnnDesc* desc, const RnnWeights* weights, const RnnIO* io,
                void* workspace, size_t ws_bytes, void* stream);

/* Size of the device array rnn_forward_noalloc uses as its workspace. */
#define RNN_NOALLOC_MAX_WORKSPACE (32u << 20)

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation. The same
 * forward as rnn_forward (same kernels, launch plan, results and errors),
 * with the workspace taken from a device array the library owns instead of
 * from the caller: RNN_NOALLOC_MAX_WORKSPACE bytes per device, held from the
 * library's first use of that device until the process ends. The caller
 * still passes (and owns) every input and output. The call allocates
 * nothing: no hipMalloc, no hipFree, no allocating library routine.
 *   - Problems whose rnn_workspace_bytes exceeds RNN_NOALLOC_MAX_WORKSPACE
 *     return RNN_E_WORKSPACE before anything is enqueued.
 *   - Every call on one device shares that device's array, which keeps the
 *     last call's contents (what must start at zero is cleared by each
 *     call): calls on one device must be ordered (one stream, or events);
 *     calls that overlap in time race and give undefined results.
 *   - device_status: NULL, or a 4-byte aligned device int that receives the
 *     call's device status word (RNN_OK or RNN_E_TIMEOUT), in stream order
 *     after the forward's kernels.
 * Errors as rnn_forward. */
int rnn_forward_noalloc(const RnnDesc* desc, const RnnWeights* weights, const RnnIO* io, void* stream,
                        int32_t* device_status);

/* Same as rnn_forward, and additionally brackets each compute kernel it
 * enqueues with caller-created hipEvent_t handles: events[2i] is recorded on
 * `stream` right before the i-th kernel and events[2i + 1] right after it,
 * for i < n_events / 2; kinds[i] (when kinds is non-NULL, room for
 * n_events / 2 entries) receives 1 for the input-projection GEMM, 2 for a
 * layer's tiled scan, 3 for the RSSM kernel and 4 for a layer's
 * one-wave-per-row scan; *n_kernels (nullable) receives the
 * number of compute kernels enqueued. For timing the kernels inside a
 * measured region. Errors as rnn_forward. */
int rnn_forward_profiled(const RnnDesc* desc, const RnnWeights* weights, const RnnIO* io,
                         void* workspace, size_t ws_bytes, void* stream, void* const* events,
                         int n_events, int* kinds, int* n_kernels);

/* Synchronises `stream`, then reads the device status word of the last
 * rnn_forward that used `workspace` into *device_status (RNN_OK or
 * RNN_E_TIMEOUT). Returns RNN_OK or RNN_E_HIP / RNN_E_NULL. */
int rnn_read_status(const void* workspace, void* stream, int* device_status);

/* Host-only: the launch shape rnn_forward would use for this problem on a
 * device with `cus` compute units in `xcds` chiplets (XCDs; workgroups are
 * dealt to them round-robin). info[0..8] = {kernel (2 tiled scan, 3 RSSM,
 * 4 one-wave-per-row scan: LSTM or GRU with H <= 16 when no
 * tiling hint is set; its waves are independent, so it needs no
 * co-residency; 5 few-row scan: LSTM or GRU with H <= 512 and at most 8
 * direction x batch rows, no tiling or weight hint, not asked to pipeline
 * a stack: one group of workgroups per direction and row, no LDS),
 * workgroups launched, LDS bytes per workgroup (kernel 4: the x rows it
 * stages when it forms layer 0's input projection itself), batch rows per workgroup,
 * hidden units per workgroup, workgroups per group, projection outputs per
 * workgroup (LSTMP), number of groups (per direction for the scan), groups
 * per XCD when every group sits on one XCD (else 0)}; n_info >= 9. With
 * n_info >= 13, info[9..12] = {scan W_hh slice in registers (1) or LDS (0),
 * MFMA column tiles per wave (0: VALU), waves splitting K (VALU: K slices),
 * 16-byte chunks per tile per lane}; the plan assumes 16-byte aligned
 * weights. With n_info >= 14, info[13] = the time chunk of a pipelined
 * layer stack (0: layer by layer; when pipelined, "workgroups launched" is
 * that of one launch scanning every layer's chunk). With n_info >= 15,
 * info[14] = the launch-shape model's time per scan step in ns (0 for the
 * one-wave and RSSM kernels). For inspection and tests; touches no device. */
int rnn_plan_info(const RnnDesc* desc, const int32_t* lengths_host, int cus, int xcds, int* info, int n_info);

/* Training (backward through time; pytorch/pytorch issue "Integrating CuDNN
 * API for LSTMs with projections", thread: the backward of these cells).
 * Built for fp32 LSTM, LSTMP and GRU stacks without clipping, every layout,
 * length mix, layer count and direction the forward takes; other
 * combinations return RNN_E_UNSUPPORTED.
 *
 * rnn_reserve_bytes: size of the caller-owned reserve that
 * rnn_forward_train fills and rnn_backward reads (the gate values of every
 * token, and the outputs of the layers below the last). Host-only. */
int rnn_reserve_bytes(const RnnDesc* desc, const int32_t* lengths_host, size_t* bytes);

/* Workspace bytes rnn_backward needs (gate-gradient buffers, the exchange of
 * the backward scan, counters). Host-only. */
int rnn_backward_workspace_bytes(const RnnDesc* desc, const int32_t* lengths_host, size_t* bytes);

/* rnn_forward that also writes the reserve (16-byte aligned, at least
 * rnn_reserve_bytes). Same outputs, same workspace as rnn_forward.
 * Enqueued on `stream`; errors as rnn_forward plus RNN_E_WORKSPACE for a
 * missing or small reserve. */
int rnn_forward_train(const RnnDesc* desc, const RnnWeights* weights, const RnnIO* io, void* reserve,
                      size_t reserve_bytes, void* workspace, size_t ws_bytes, void* stream);

/* Gradients of a loss through the forward that rnn_forward_train ran with
 * the same desc, weights and io (x, h0, c0, lengths and the y it wrote are
 * read again) and filled `reserve`. For PADDED input, x must be finite at
 * positions t >= L_b (they enter the weight-gradient products with zero
 * weight). Enqueued on `stream`; the workspace (16-byte aligned, at least
 * rnn_backward_workspace_bytes) is independent of the forward's. Device
 * status as rnn_forward (rnn_read_status on this workspace). */
int rnn_backward(const RnnDesc* desc, const RnnWeights* weights, const RnnIO* io, const RnnGrads* grads,
                 const void* reserve, size_t reserve_bytes, void* workspace, size_t ws_bytes, void* stream);

/* RNN_OK when the current device is a gfx950 GPU; RNN_E_DEVICE otherwise. */
int rnn_device_check(void);

/* Measurement helper: the time one device-coherent round trip takes between
 * two workgroups on different XCDs of the current device, using the same
 * device-scope stores and loads the persistent kernels exchange their state
 * with every step (a step that waits on another compute unit's result pays
 * at least one such one-way trip; a counter barrier pays about a round
 * trip). `buffer` is caller-owned device memory of at least 1024 bytes,
 * 256-byte aligned, whose contents are overwritten; iters in [1, 100000].
 * Enqueues on `stream`, synchronises it and writes the mean nanoseconds per
 * round trip. Returns RNN_OK, RNN_E_NULL, RNN_E_SHAPE, RNN_E_ALIGN,
 * RNN_E_DEVICE, RNN_E_HIP, or RNN_E_TIMEOUT when a bounded wait ran out
 * (the two workgroups were not resident together). */
int rnn_exchange_roundtrip_ns(void* buffer, size_t bytes, int iters, void* stream, double* ns_per_round_trip);

#ifdef __cplusplus
}
#endif

#endif /* GRU_SEQUENCE_SCAN_RNN_H */
