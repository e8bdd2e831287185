#!/usr/bin/env python3
"""Benchmark of the recurrence forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload all|NAME|1..5]

A step is one rnn_forward of the whole hot path for the workload (every
kernel it enqueues: input-projection GEMMs, scans, or the RSSM kernel) on
seeded synthetic inputs already resident in HBM. Prints ONE JSON line with
the throughput in timestep*batch/s, the roofline of the dominant kernel
(timed with HIP events around its launches inside the timed region) and the
float64 CPU oracle timed on the host on a bounded sample of the same work.

Default (--workload all): the headline is the RSSM-prior unroll, B=50, T=50
(state 20, action 6, hidden 200, GRU hidden 200, fp32), at the top level of
the line; "configs" then holds the same record (value, ms per step, median
and minimum, dominant-kernel roofline, CPU baseline) for each of the five
configurations, each timed for the same K steps after W warm-ups.
"""

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published peaks
PEAK_HBM_GBS = 8000.0
# LDS: 128 bytes per clock per CU, 256 CUs at 2.4 GHz
PEAK_LDS_GBS = 128 * 256 * 2.4
PEAK_TFLOPS = {"bf16": 2500.0, "f32_mfma": 157.3, "f32_vector": 157.3}

# kernel kinds reported by rnn_forward_profiled (kind | layer << 8; kind 5, a
# launch scanning a time chunk of several stacked layers: first layer | last
# layer << 4)
KIND_NAMES = {1: "gemm_xw", 2: "scan", 3: "rssm", 4: "scan_wave", 5: "scan"}
METRIC = "timestep\u00b7batch/s per RNN config; % of MFMA / on-chip BW roofline"
UNIT = "timestep\u00b7batch/s"
HEADLINE = "rssm_b50_t50"

# Sources whose change invalidates a kernel's measured traffic.
CSRC = os.path.join(ROOT, "gru_sequence_scan_amd", "csrc")
KERNEL_SOURCES = {
    "gemm_xw": ["gemm_xw.hip", "device_common.hpp", "kernels.hpp", "rnn_api.cpp"],
    "scan": ["scan.hip", "scan_kernel.hpp", "scan_common.hpp", "scan_small.hip", "scan_bf16_reg.hip", "scan_bf16_lds.hip",
             "scan_bf16gx_reg.hip", "scan_bf16gx_lds.hip", "scan_f32_reg.hip", "scan_f32_lds.hip",
             "scan_f32t_reg.hip", "scan_f32t_lds.hip", "device_common.hpp", "kernels.hpp", "rnn_api.cpp"],
    "rssm": ["rssm.hip", "rssm2.hip", "rssm_common.hpp", "device_common.hpp", "kernels.hpp", "rnn_api.cpp"],
    "scan_wave": ["scan_wave.hip", "device_common.hpp", "kernels.hpp", "rnn_api.cpp"],
}

# HBM bytes per launch of a workload's dominant kernel, from two rocprofv3
# --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE), each divided by
# the ratio the same counter reads for a plain copy of known size
# (--calibrate-copy), and the same kernel's MFMA and LDS counters
# ("counters": MFMA FLOP executed, MFMA busy share of the 1024 SIMDs, LDS
# active share of the 256 CUs, bank-conflict cycles per LDS-active cycle)
# with those of the first input GEMM ("gemm_counters"). Valid only for the
# kernel sources they were taken on.
MEASURED_TRAFFIC = {
    "rssm_b50_t50": {"kernel": "rssm", "index": 0, "fetch_bytes": 10394800, "write_bytes": 4046400, "sources": "95d745d87b07bc55", "counters": {"mfma_flops": 6473318400, "mfma_busy": 0.12671, "lds_active": 0.11652, "lds_bank_conflict": 0.07353}},
    "lstm_t80_b1": {"kernel": "scan", "index": 0, "fetch_bytes": 1435372, "write_bytes": 89088, "sources": "4fee0762a840a6ce", "counters": {"mfma_flops": 0, "mfma_busy": 0.0, "lds_active": 3e-05, "lds_bank_conflict": 0.0}, "gemm_counters": {"mfma_flops": 134217728, "mfma_busy": 0.04447, "lds_active": 0.00636, "lds_bank_conflict": 0.0}, "gemm_sources": "e4088e4395184de3"},
    "gru_t256_b256": {"kernel": "scan", "index": 0, "fetch_bytes": 215456758, "write_bytes": 68427776, "sources": "4fee0762a840a6ce", "counters": {"mfma_flops": 137438953472, "mfma_busy": 0.05366, "lds_active": 0.10002, "lds_bank_conflict": 0.33587}, "gemm_counters": {"mfma_flops": 103079215104, "mfma_busy": 0.25616, "lds_active": 0.43209, "lds_bank_conflict": 0.2963}, "gemm_sources": "e4088e4395184de3"},
    "lstmp_t1000_b32": {"kernel": "scan", "index": "0-1", "fetch_bytes": 54539399, "write_bytes": 3594581, "sources": "4fee0762a840a6ce", "counters": {"mfma_flops": 16777216000, "mfma_busy": 0.01007, "lds_active": 0.04482, "lds_bank_conflict": 0.32038}, "gemm_counters": {"mfma_flops": 83886080000, "mfma_busy": 0.21653, "lds_active": 0.39409, "lds_bank_conflict": 0.27778}, "gemm_sources": "e4088e4395184de3"},
    "bilstm_varlen_b64": {"kernel": "scan", "index": 1, "fetch_bytes": 351878435, "write_bytes": 80773120, "sources": "4fee0762a840a6ce", "counters": {"mfma_flops": 95093260288, "mfma_busy": 0.26271, "lds_active": 0.09065, "lds_bank_conflict": 0.40562}, "gemm_counters": {"mfma_flops": 40802189312, "mfma_busy": 0.71499, "lds_active": 0.06179, "lds_bank_conflict": 0.0}, "gemm_sources": "e4088e4395184de3"},
    "lstm_t256_b1_small": {"kernel": "scan_wave", "index": 0, "fetch_bytes": 44363, "write_bytes": 16544, "sources": "bc88e60b733c51bf", "counters": {"mfma_flops": 0, "mfma_busy": 0.0, "lds_active": 0.00012, "lds_bank_conflict": 0.0}},
    "rssm_actor_b50_h50": {"kernel": "rssm", "index": 0, "fetch_bytes": 12972182, "write_bytes": 5386400, "sources": "95d745d87b07bc55", "counters": {"mfma_flops": 8308326400, "mfma_busy": 0.12246, "lds_active": 0.12681, "lds_bank_conflict": 0.06538}},
}

# The pages' own numbers for the same metric and workload (CPU, Ryzen 5900X,
# apache/tvm PR "[TOPI] TE implementation of LSTM using scan", benchmark
# thread): timestep*batch per second for the TE-scan and Relay-unrolled LSTM.
PAGES_CONTEXT = {
    "lstm_t80_b1": {"tvm_te_scan": 80 / 48.967991919999996e-3, "tvm_relay_unrolled": 80 / 14.4790252e-3},
    "lstm_t256_b1_small": {"tvm_te_scan": 256 / 0.14541639e-3, "tvm_relay_unrolled": 256 / 2.62690786e-3},
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="all",
                    help="'all' (default): the RSSM unroll as the headline plus a block per config; "
                         "or one workload name / 1-based index")
    ap.add_argument("--cpu-seconds", type=float, default=5.0)
    ap.add_argument("--prof-every", type=int, default=4,
                    help="timed steps i with i %% N == 0 carry HIP events on every kernel (an event on a "
                         "dispatch delays the next dispatch by ~5 us); the others run as a user would call them")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--tile-batch", type=int, default=0)
    ap.add_argument("--tile-hidden", type=int, default=0)
    ap.add_argument("--placement", type=int, default=0, help="0 auto, 1 flat, 2 XCD-aligned groups")
    ap.add_argument("--weights", type=int, default=0,
                    help="RnnDesc.weights hint: 0 auto, 1 LDS-resident, 2 register-resident")
    ap.add_argument("--layer-pipeline", default="auto", choices=["auto", "off", "on"],
                    help="multi-layer stacks: scan the layers' time chunks together (auto: where modelled faster)")
    ap.add_argument("--gx-f32", action="store_true",
                    help="store the hoisted G_x in fp32 also for bf16 workloads (default: the storage dtype)")
    ap.add_argument("--train", action="store_true",
                    help="time a training step (rnn_forward_train + rnn_backward) instead of the forward")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain device copy of known size (counter calibration)")
    return ap.parse_args()


def sources_digest(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def calibrate_copy():
    """A plain elementwise copy (negation) of 256 MiB fp32, launched 5 times:
    each launch reads and writes exactly 256 MiB of HBM."""
    import torch
    n = 64 << 20
    src = torch.randn(n, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "kernel": "neg fp32", "bytes_read": 4 * n, "bytes_written": 4 * n,
                      "launches": 5}), flush=True)


def _hip():
    """The HIP runtime already loaded in this process (torch's)."""
    path = None
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64" in line:
                path = line.split()[-1]
                break
    h = ctypes.CDLL(path or "libamdhip64.so.7")
    h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    h.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return h


def algorithmic(spec, d, gx_f32=False):
    """Algorithmic flops and HBM bytes per launch, by kernel kind and layer."""
    import synth  # noqa: F401
    out = {}
    if spec.mode in ("rssm", "rssm_actor"):
        B, T, S, A, E, Hb = d["B"], d["T"], d["state_dim"], d["action_dim"], d["embed_dim"], d["belief_dim"]
        Ea = d.get("actor_dim", 0)
        per_tok = 2 * (E * (S + A) + 3 * Hb * (E + Hb) + E * Hb + 2 * S * E + Ea * (S + Hb) + A * Ea)
        weights = 4 * (E * (S + A) + E + 6 * Hb * (E + Hb) / 2 + 6 * Hb + E * Hb + E + 2 * S * E + 2 * S
                       + (Ea * (S + Hb) + Ea + A * Ea + A if Ea else 0))
        io = 4 * B * T * (A + S + 3 * S + Hb)  # actions read (or, with the actor, written)
        out[3] = [{"flops": per_tok * B * T, "bytes": weights + io, "tokens": B * T}]
        return out
    D = 2 if spec.bidirectional else 1
    gates = 3 if spec.mode == "gru" else 4
    H = spec.hidden_size
    G = gates * H
    K = spec.proj_size if spec.mode == "lstmp" else H
    es = 2 if spec.dtype == "bf16" else 4
    gs = 4 if gx_f32 else es  # bytes per element of the hoisted G_x
    L = d["lengths"]
    tokens = int(L.sum()) if L is not None else spec.T * spec.B
    rows = tokens if spec.layout == "packed" else spec.T * spec.B
    gemms, scans = [], []
    for layer in range(spec.num_layers):
        in_l = spec.input_size if layer == 0 else D * K
        gemms.append({"flops": 2 * rows * D * G * in_l,
                      "bytes": rows * in_l * es + D * G * in_l * es + rows * D * G * gs, "tokens": tokens})
        fl = 2 * tokens * D * G * K
        if spec.mode == "lstmp":
            fl += 2 * tokens * D * spec.proj_size * H
        scans.append({"flops": fl, "bytes": tokens * D * (G * gs + K * es), "tokens": tokens})
    out[1] = gemms
    out[2] = scans
    out[4] = scans  # the one-wave-per-row scan does the same work
    return out


def prepare(name, args):
    """Inputs of a workload resident on the GPU and the C structs of one
    rnn_forward over them (built once, outside any timed region)."""
    import torch

    import gru_sequence_scan_amd as gss
    import synth

    spec = synth.spec(name)
    d = synth.make_inputs(name)
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if spec.dtype == "bf16" else torch.float32

    def T(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev).to(dt)

    keep = []
    hints = dict(tile_batch=args.tile_batch, tile_hidden=args.tile_hidden, placement=args.placement,
                 return_workspace=True, check_status=False)
    if spec.mode in ("rssm", "rssm_actor"):
        actor = spec.mode == "rssm_actor"
        w = {k: T(v) for k, v in d["weights"].items()}
        aw = {k: T(v) for k, v in d["actor"].items()} if actor else None
        acts, eps = T(d["actions"]), T(d["eps"])
        if actor:
            (out, ws) = gss.rssm_actor_unroll(eps, w, aw, **hints)
        else:
            (out, ws) = gss.rssm_prior_unroll(acts, eps, w, weights_hint=args.weights, **hints)
        B, Tn = d["B"], d["T"]
        desc = gss.RnnDesc()
        desc.mode, desc.dtype, desc.layout = gss.MODES[spec.mode], 0, 2
        desc.actor_dim = d.get("actor_dim", 0)
        desc.T, desc.B, desc.num_layers, desc.has_bias = Tn, B, 1, 1
        desc.state_dim, desc.action_dim = d["state_dim"], d["action_dim"]
        desc.embed_dim, desc.belief_dim, desc.scale_lb = d["embed_dim"], d["belief_dim"], 0.1
        desc.tile_batch, desc.tile_hidden, desc.placement = args.tile_batch, args.tile_hidden, args.placement
        desc.weights = args.weights
        desc.gx_dtype = 1 if args.gx_f32 else 0
        wt = gss.RnnWeights()
        wt.w_as, wt.b_as, wt.w_1, wt.b_1, wt.w_2, wt.b_2 = (w[k].data_ptr() for k in
                                                            ("w_as", "b_as", "w_1", "b_1", "w_2", "b_2"))
        wt.w_ih[0], wt.w_hh[0], wt.b_ih[0], wt.b_hh[0] = (w[k].data_ptr() for k in ("w_ih", "w_hh", "b_ih", "b_hh"))
        if actor:
            wt.w_a1, wt.b_a1, wt.w_a2, wt.b_a2 = (aw[k].data_ptr() for k in ("w_a1", "b_a1", "w_a2", "b_a2"))
        io = gss.RnnIO()
        io.x, io.noise = (acts.data_ptr() if acts is not None else None), eps.data_ptr()
        io.means, io.stds, io.states, io.beliefs = (o.data_ptr() for o in out[:4])
        if actor:
            io.actions = out[4].data_ptr()
        keep += [w, aw, acts, eps, out]
        tokens = B * Tn
        config = {"workload": name, "B": B, "T": Tn, "state": d["state_dim"], "action": d["action_dim"],
                  "hidden": d["embed_dim"], "gru_hidden": d["belief_dim"]}
        if actor:
            config["actor_hidden"] = d["actor_dim"]
        lengths = None
    else:
        params = [{k: T(v) for k, v in p.items() if v is not None} for p in d["params"]]
        x = T(d["x"])
        (out, ws) = gss.rnn_forward(spec.mode, x, params, lengths=d["lengths"], layout=spec.layout,
                                    num_layers=spec.num_layers, bidirectional=spec.bidirectional,
                                    proj_size=spec.proj_size, weights=args.weights,
                                    gx_dtype="f32" if args.gx_f32 else "auto",
                                    layer_pipeline=args.layer_pipeline, **hints)
        y, hn, cn = out
        desc = gss.RnnDesc()
        desc.mode = gss.MODES[spec.mode]
        desc.dtype = 1 if spec.dtype == "bf16" else 0
        desc.layout = 1 if spec.layout == "packed" else 0
        desc.T, desc.B = spec.T, spec.B
        desc.input_size, desc.hidden_size, desc.proj_size = spec.input_size, spec.hidden_size, spec.proj_size
        desc.num_layers, desc.bidirectional, desc.has_bias = spec.num_layers, int(spec.bidirectional), 1
        desc.tile_batch, desc.tile_hidden, desc.placement = args.tile_batch, args.tile_hidden, args.placement
        desc.weights = args.weights
        desc.gx_dtype = 1 if args.gx_f32 else 0
        desc.layer_pipeline = gss.PIPE_MODES[args.layer_pipeline]
        wt = gss.RnnWeights()
        for i, p in enumerate(params):
            for k, v in p.items():
                getattr(wt, k)[i] = v.data_ptr()
        io = gss.RnnIO()
        io.x, io.y, io.h_n = x.data_ptr(), y.data_ptr(), hn.data_ptr()
        io.c_n = cn.data_ptr() if cn is not None else None
        lengths = d["lengths"]
        keep_len, io.lengths_host = gss.binding._len_ptr(lengths, spec.B)
        keep += [params, x, out, keep_len]
        tokens = int(lengths.sum()) if lengths is not None else spec.T * spec.B
        config = {"workload": name, "mode": spec.mode, "T": spec.T, "B": spec.B, "input": spec.input_size,
                  "hidden": spec.hidden_size, "proj": spec.proj_size, "layers": spec.num_layers,
                  "bidirectional": spec.bidirectional, "layout": spec.layout, "tokens": tokens,
                  "gx_dtype": "f32" if (args.gx_f32 or spec.dtype == "f32") else spec.dtype,
                  "layer_pipeline": args.layer_pipeline}
    torch.cuda.synchronize()
    return {"name": name, "spec": spec, "d": d, "desc": desc, "wt": wt, "io": io, "ws": ws, "keep": keep,
            "tokens": tokens, "config": config, "lengths": lengths}


def onchip_bytes(spec, d, plan):
    """Bytes of resident weights one launch of the recurrence kernel reads
    from on-chip storage: every member reads its slice once per step (the
    RSSM's replicated small matrices once per member)."""
    if spec.mode in ("rssm", "rssm_actor"):
        S, A, E, Hb, Ea = d["state_dim"], d["action_dim"], d["embed_dim"], d["belief_dim"], d.get("actor_dim", 0)
        split = 3 * Hb * (E + Hb) + E * Hb + Ea * Hb                 # sliced over the members
        repl = E * (S + A) + 2 * S * E + Ea * S + A * Ea              # whole in every member
        per_step = plan["groups"] * (split + plan["members"] * repl) * 4
        return per_step * d["T"]
    D = 2 if spec.bidirectional else 1
    G = (3 if spec.mode == "gru" else 4) * spec.hidden_size
    K = spec.proj_size if spec.mode == "lstmp" else spec.hidden_size
    es = 2 if spec.dtype == "bf16" else 4
    P = spec.proj_size if spec.mode == "lstmp" else 0
    L = d["lengths"]
    steps = int(L.max()) if L is not None else spec.T
    blocks = max(1, plan.get("groups", 1))  # batch blocks per direction
    return steps * D * blocks * (G * K + P * spec.hidden_size) * es


def measure(name, args, rt_us, with_cpu):
    """Time K forwards of one workload after W warm-ups; per-kernel times from
    HIP events recorded on the launch stream by rnn_forward_profiled."""
    import torch

    import gru_sequence_scan_amd as gss

    pr = prepare(name, args)
    spec, d, desc, wt, io, ws = pr["spec"], pr["d"], pr["desc"], pr["wt"], pr["io"], pr["ws"]
    lengths, tokens = pr["lengths"], pr["tokens"]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev).cuda_stream
    hip = _hip()
    lib = gss.lib()
    lib.rnn_forward_profiled.restype = ctypes.c_int
    lib.rnn_forward_profiled.argtypes = [ctypes.POINTER(gss.RnnDesc), ctypes.POINTER(gss.RnnWeights),
                                         ctypes.POINTER(gss.RnnIO), ctypes.c_void_p, ctypes.c_size_t,
                                         ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p), ctypes.c_int,
                                         ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
    max_k = 256
    ws_ptr, ws_n = ws.data_ptr(), ws.numel()

    def step(evs=None, kinds=None, nk=None):
        if evs is None:
            st = lib.rnn_forward(ctypes.byref(desc), ctypes.byref(wt), ctypes.byref(io), ws_ptr, ws_n, stream)
        else:
            st = lib.rnn_forward_profiled(ctypes.byref(desc), ctypes.byref(wt), ctypes.byref(io), ws_ptr, ws_n,
                                          stream, evs, 2 * max_k, kinds, ctypes.byref(nk))
        if st != 0:
            raise gss.RnnError(st, "rnn_forward")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if gss.rnn_read_status(ws_ptr, stream) != 0:
        raise RuntimeError(f"{name}: device status error after warmup")

    K = args.steps
    every = max(1, args.prof_every)
    ev_arrays = []
    for _ in range((K + every - 1) // every):
        arr = (ctypes.c_void_p * (2 * max_k))()
        for j in range(2 * max_k):
            h = ctypes.c_void_p()
            hip.hipEventCreate(ctypes.byref(h))
            arr[j] = h.value
        ev_arrays.append(arr)
    kinds = (ctypes.c_int * max_k)()
    nk = ctypes.c_int(0)

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        if i % every == 0:
            step(ev_arrays[i // every], kinds, nk)
        else:
            step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    status = gss.rnn_read_status(ws_ptr, stream)
    if status != 0:
        raise RuntimeError(f"{name}: device status {status} after timed steps")

    n_k = nk.value
    per_kernel = [[] for _ in range(n_k)]
    step_ms = []
    for arr in ev_arrays:
        for j in range(min(n_k, max_k)):
            ms = ctypes.c_float(0)
            hip.hipEventElapsedTime(ctypes.byref(ms), arr[2 * j], arr[2 * j + 1])
            per_kernel[j].append(ms.value)
        ms = ctypes.c_float(0)
        hip.hipEventElapsedTime(ctypes.byref(ms), arr[0], arr[2 * (min(n_k, max_k) - 1) + 1])
        step_ms.append(ms.value)
    for arr in ev_arrays:
        for j in range(2 * max_k):
            hip.hipEventDestroy(arr[j])
    if n_k > max_k:
        raise RuntimeError(f"{name}: {n_k} kernels per forward, more than the {max_k} timed")
    kind_list = [kinds[j] for j in range(n_k)]
    algo = algorithmic(spec, d, getattr(args, "gx_f32", False))
    # One entry per (kernel kind, layer): a pipelined stack launches a G_x
    # product per layer and time chunk and one scan per wave over several
    # layers (kind 5, taken together as one entry); an entry's figures are
    # per launch (its algorithmic work and time over its launch count).
    groups = {}
    for j, kw in enumerate(kind_list):
        kd, lay = kw & 0xFF, kw >> 8
        groups.setdefault((2, -1) if kd == 5 else (kd, lay), []).append(j)
    kernels = []
    for (kd, lay), js in groups.items():
        if lay < 0:
            a = {"flops": sum(x["flops"] for x in algo[2]), "bytes": sum(x["bytes"] for x in algo[2])}
            index = f"0-{spec.num_layers - 1}"
        else:
            a = algo[kd][lay]
            index = lay
        tot = np.sum([np.asarray(per_kernel[j]) for j in js], axis=0) * 1e3  # us per forward
        v = tot / len(js)
        kernels.append({"kernel": KIND_NAMES[kd], "index": index, "launches": len(js),
                        "total_us": float(tot.mean()), "avg_us": float(v.mean()),
                        "median_us": float(np.median(v)), "min_us": float(v.min()),
                        "flops": a["flops"] / len(js), "bytes": a["bytes"] / len(js)})
    dom = max(kernels, key=lambda k: k["total_us"])
    achieved = dom["flops"] / (dom["avg_us"] * 1e-6) / 1e12
    if dom["kernel"] == "scan_wave" or (dom["kernel"] == "scan" and spec.B < 16):
        # the small-batch scans run their products on the vector ALUs
        bound, peak = "alu", PEAK_TFLOPS["f32_vector"]
    else:
        bound = "mfma"
        peak = PEAK_TFLOPS["bf16"] if spec.dtype == "bf16" else PEAK_TFLOPS["f32_mfma"]
    traffic = None
    meas = MEASURED_TRAFFIC.get(name)
    digest = sources_digest(dom["kernel"])
    if meas and (meas["kernel"], meas["index"]) == (dom["kernel"], dom["index"]) and meas["sources"] == digest:
        traffic = meas["fetch_bytes"] + meas["write_bytes"]
    roofline = {"bound": bound, "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
                "traffic": traffic, "kernel": f"{dom['kernel']}[{dom['index']}]", "avg_us": dom["avg_us"],
                "median_us": dom["median_us"], "min_us": dom["min_us"],
                "algorithmic_flops": dom["flops"], "algorithmic_hbm_bytes": dom["bytes"],
                "hbm_frac": dom["bytes"] / (dom["avg_us"] * 1e-6) / 1e9 / PEAK_HBM_GBS,
                "sources": digest}
    if meas and traffic is not None:
        roofline["traffic_fetch"] = meas["fetch_bytes"]
        roofline["traffic_write"] = meas["write_bytes"]
        # MFMA and LDS counters of the same kernel (rocprofv3 --pmc, same rule)
        if "counters" in meas:
            roofline["counters"] = meas["counters"]
    if meas and "gemm_counters" in meas and meas.get("gemm_sources") == sources_digest("gemm_xw"):
        roofline["gemm_counters"] = meas["gemm_counters"]

    # The recurrence kernel's steps, time per step and cross-CU exchanges per
    # step; its on-chip term; the fraction against the compute units the
    # launch occupies; and the floor that the measured device-coherent round
    # trip puts under its steps.
    if spec.mode in ("rssm", "rssm_actor"):
        n_rec, layer_dirs = d["T"], 1
    else:
        n_rec = int(lengths.max()) if lengths is not None else spec.T
        layer_dirs = spec.num_layers * (2 if spec.bidirectional else 1)
    plan = gss.rnn_plan_info(desc, lengths)
    piped = isinstance(dom["index"], str)  # one scan launch per wave of chunks
    slots = spec.num_layers if plan.get("pipe_chunk", 0) else 1
    if plan["kernel"] == 4:
        bars, occ = 0, min(256, plan["workgroups"])
    else:
        members = plan["members"]
        lstmp = spec.mode == "lstmp"
        bars = 0 if (members == 1 and not lstmp) else (2 if lstmp else 1)  # exchanges per step
        dirs = 1 if plan["kernel"] == 3 else (2 if spec.bidirectional else 1)
        occ = min(256, plan["groups"] * dirs * members * slots)  # workgroups that do work
    if dom["kernel"] == "gemm_xw":
        occ = 256
    ob = onchip_bytes(spec, d, plan) if dom["kernel"] in ("scan", "rssm", "scan_wave") else 0
    rec_us = dom["avg_us"]
    if piped:
        # the waves walk chunk-length steps in sequence, the layers side by side
        ch, L = plan["pipe_chunk"], spec.num_layers
        n = -(-spec.T // ch)
        n_rec = sum(max(min(ch, spec.T - c * ch) for c in range(max(0, w - L + 1), min(n - 1, w) + 1))
                    for w in range(n + L - 1))
        ob = ob * L / dom["launches"]
        rec_us = dom["total_us"]
    t_roof = max(dom["flops"] / (peak * 1e12), ob / (PEAK_LDS_GBS * 1e9), dom["bytes"] / (PEAK_HBM_GBS * 1e9))
    roofline.update({
        "recurrence_steps": n_rec, "us_per_step": rec_us / n_rec, "exchanges_per_step": bars,
        "onchip_bytes": ob, "t_roof_us": t_roof * 1e6, "roof_frac": t_roof * 1e6 / dom["avg_us"],
        "occupied_cus": occ, "frac_occupied_cus": achieved / (peak * occ / 256.0),
        "exchange_roundtrip_us": rt_us,
        "exchange_floor_us": n_rec * bars * rt_us if rt_us is not None else None,
    })
    if piped:
        roofline.update({"pipeline_chunk": plan["pipe_chunk"], "launches": dom["launches"]})
    ms_per_step = elapsed / K * 1e3
    value = tokens / (elapsed / K)
    # the kernels of a forward must fill most of a step and never exceed it:
    # a kernel whose events did not bracket its dispatch would break this
    span_us = sum(k["total_us"] for k in kernels)
    if not (0.5 * ms_per_step * 1e3 <= span_us <= 1.05 * ms_per_step * 1e3):
        raise RuntimeError(f"{name}: kernel events cover {span_us:.1f} us of a {ms_per_step * 1e3:.1f} us step")
    ctx = PAGES_CONTEXT.get(name)
    vs = (value / max(ctx.values())) if ctx else None
    rec = {"config": pr["config"], "value": value, "ms_per_step": ms_per_step,
           "median_kernel_span_ms": float(np.median(step_ms)), "min_kernel_span_ms": float(np.min(step_ms)),
           "dtype": spec.dtype, "vs_baseline": vs, "roofline": roofline, "kernels": kernels,
           "cell_steps_per_s": value * layer_dirs,
           "kernel_timing": f"HIP events carried by the dispatches of every kernel on timed steps 0, {every}, "
                            f"{2 * every}, ... ({len(ev_arrays)} of {K})"}
    if ctx:
        rec["pages_context"] = {k: v for k, v in ctx.items()}
    if with_cpu:
        rec["cpu_baseline"] = cpu_baseline_any(spec, d, args.cpu_seconds)
    del pr
    return rec


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the recurrence shards by batch with no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.train:
        train_main(args)
        return
    import torch

    import gru_sequence_scan_amd as gss
    import synth

    torch.cuda.set_device(torch.device("cuda:0"))
    try:
        rt_us = gss.rnn_exchange_roundtrip_ns(2000) / 1e3
    except gss.RnnError:
        rt_us = None
    wl = args.workload
    head = synth.ORDER[int(wl) - 1] if wl.isdigit() else (HEADLINE if wl == "all" else wl)
    others = [n for n in synth.ORDER if n != head] if wl == "all" else []
    print(f"bench: {head}", file=sys.stderr, flush=True)
    h = measure(head, args, rt_us, not args.no_cpu)
    rec = {
        "metric": METRIC, "value": h["value"], "unit": UNIT,
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": h["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": h["vs_baseline"],
        "dtype": h["dtype"], "data": "synthetic", "config": h["config"],
        "roofline": h["roofline"], "kernels": h["kernels"],
        "median_kernel_span_ms": h["median_kernel_span_ms"], "min_kernel_span_ms": h["min_kernel_span_ms"],
        "cell_steps_per_s": h["cell_steps_per_s"], "kernel_timing": h["kernel_timing"],
    }
    if "pages_context" in h:
        rec["pages_context"] = h["pages_context"]
    if "cpu_baseline" in h:
        rec["cpu_baseline"] = h["cpu_baseline"]
    if others:
        per = {}
        for n in synth.ORDER:
            if n == head:
                per[n] = {k: v for k, v in h.items()}
                continue
            print(f"bench: {n}", file=sys.stderr, flush=True)
            per[n] = measure(n, args, rt_us, not args.no_cpu)
            torch.cuda.empty_cache()
        rec["configs"] = per
    print(json.dumps(rec), flush=True)


def train_flops(spec, d):
    """Algorithmic flops of one training step: the forward (input GEMM and
    recurrent product per layer) and the backward (recurrent product,
    dW_ih, dW_hh and dX per layer)."""
    D = 2 if spec.bidirectional else 1
    G = (3 if spec.mode == "gru" else 4) * spec.hidden_size
    H = spec.hidden_size
    P = spec.proj_size if spec.mode == "lstmp" else 0
    K = P or H  # recurrent width
    L = d["lengths"]
    tokens = int(L.sum()) if L is not None else spec.T * spec.B
    rows = tokens if spec.layout == "packed" else spec.T * spec.B
    fl = 0
    for layer in range(spec.num_layers):
        in_l = spec.input_size if layer == 0 else D * K
        fl += 2 * rows * D * G * in_l + 2 * tokens * D * G * K            # forward
        fl += 2 * tokens * D * G * K                                      # backward recurrent product
        fl += 2 * rows * D * G * in_l * 2 + 2 * rows * D * G * K          # dW_ih, dX, dW_hh
        if P:
            fl += 2 * tokens * D * P * H * 2 + 2 * rows * D * P * H       # projection forward and back, dW_hr
    return fl, tokens


def train_main(args):
    """One training step = rnn_forward_train + rnn_backward over the
    workload, inputs and upstream gradients resident on the GPU."""
    import torch

    import gru_sequence_scan_amd as gss
    import synth

    name = synth.ORDER[int(args.workload) - 1] if args.workload.isdigit() else args.workload
    spec = synth.spec(name)
    if spec.mode not in ("lstm", "gru", "lstmp"):
        print(f"training is built for LSTM / GRU / LSTMP stacks; {name} is {spec.mode}", file=sys.stderr)
        sys.exit(2)
    d = synth.make_inputs(name)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def T(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    params = [{k: T(v) for k, v in p.items() if v is not None} for p in d["params"]]
    x = T(np.nan_to_num(d["x"]))
    D = 2 if spec.bidirectional else 1
    H = spec.hidden_size
    P = spec.proj_size if spec.mode == "lstmp" else 0
    K = P or H
    rng = np.random.default_rng(spec.seed + 1)
    yshape = (x.shape[0], D * K) if spec.layout == "packed" else (spec.T, spec.B, D * K)
    dy = T(rng.normal(size=yshape))
    kw = dict(lengths=d["lengths"], layout=spec.layout, num_layers=spec.num_layers,
              bidirectional=spec.bidirectional, proj_size=P, tile_batch=args.tile_batch,
              tile_hidden=args.tile_hidden)

    def step():
        _, ctx = gss.rnn_forward_train(spec.mode, x, params, **kw)
        return gss.rnn_backward(ctx, dy)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(K):
        step()
    e1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ev_ms = e0.elapsed_time(e1) / K
    flops, tokens = train_flops(spec, d)
    achieved = flops / (ev_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS["f32_mfma"]
    line = {
        "metric": METRIC, "value": tokens / (elapsed / K), "unit": UNIT, "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": elapsed / K * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": name, "pass": "forward+backward", "mode": spec.mode, "T": spec.T, "B": spec.B,
                   "input": spec.input_size, "hidden": H, "layers": spec.num_layers,
                   "bidirectional": spec.bidirectional, "layout": spec.layout, "tokens": tokens,
                   **({"proj": P} if P else {}),
                   # training computes in fp32; a bf16 forward workload's
                   # (bf16-representable) inputs are taken as fp32
                   **({"operands": "fp32 (the bf16 workload's values, widened)"} if spec.dtype == "bf16" else {})},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": None, "kernel": "training step (all kernels)",
                     "avg_us": ev_ms * 1e3, "algorithmic_flops": flops},
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline_train(spec, d, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def host_info():
    """The host CPU model and the BLAS library numpy uses (the oracle's
    products run on it)."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        b = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas = f"{b.get('name')} {b.get('version')}"
    except Exception:
        pass
    return {"cpu_model": model, "blas": blas}


def cpu_baseline_train(spec, d, seconds):
    """The float64 oracle's forward + BPTT on a sample of batch rows (all
    timesteps), sized from a one-row probe."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    L = d["lengths"]
    order = np.random.default_rng(0).permutation(spec.B)
    D = 2 if spec.bidirectional else 1
    P = spec.proj_size if spec.mode == "lstmp" else 0
    K = P or spec.hidden_size

    def run(rows):
        sub = np.sort(order[:rows])
        lengths = None if L is None else L[sub]
        if spec.layout == "packed":
            x = oracle.pack_sequence(np.nan_to_num(d["x_padded"][:, sub]), lengths)
            dy = np.ones((x.shape[0], D * K))
        else:
            x = d["x"][:, sub]
            dy = np.ones((spec.T, rows, D * K))
        kw = dict(lengths=lengths, num_layers=spec.num_layers, bidirectional=spec.bidirectional,
                  layout=spec.layout, proj_size=P)
        t0 = time.perf_counter()
        oracle.rnn_forward(spec.mode, x, d["params"], **kw)
        oracle.rnn_backward(spec.mode, x, d["params"], dy, **kw)
        el = time.perf_counter() - t0
        return (int(lengths.sum()) if lengths is not None else spec.T * rows), el

    _, t1 = run(1)
    rows = int(min(spec.B, max(1, seconds / max(t1, 1e-6))))
    tokens, el = run(rows)
    return {"value": tokens / el, "unit": UNIT, "cores": int(threads), "kind": "oracle",
            "sample": f"forward + backward of {rows} of {spec.B} batch rows over all timesteps, {el:.1f} s",
            **host_info()}


def cpu_baseline_any(spec, d, seconds):
    """The float64 oracle on the host, on a bounded sample of the workload:
    the RSSM unroll is repeated whole; for the recurrent stacks the sample is
    a subset of batch rows over all their timesteps (rows are independent),
    sized from a one-row probe to take about `seconds`."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    if spec.mode in ("rssm", "rssm_actor"):
        t0 = time.perf_counter()
        tokens, runs = 0, 0
        while True:
            if spec.mode == "rssm_actor":
                oracle.rssm_actor_unroll(d["eps"], d["weights"], d["actor"])
            else:
                oracle.rssm_prior_unroll(d["actions"], d["eps"], d["weights"])
            tokens += d["B"] * d["T"]
            runs += 1
            if time.perf_counter() - t0 > seconds:
                break
        el = time.perf_counter() - t0
        sample = f"whole unroll (B={d['B']}, T={d['T']}) x{runs}, {el:.1f} s"
    else:
        L = d["lengths"]
        order = np.random.default_rng(0).permutation(spec.B)

        def run(rows):
            sub = np.sort(order[:rows])
            lengths = None if L is None else L[sub]
            if spec.layout == "packed":
                x = oracle.pack_sequence(np.nan_to_num(d["x_padded"][:, sub]), lengths)
            else:
                x = d["x"][:, sub]
            t0 = time.perf_counter()
            oracle.rnn_forward(spec.mode, x, d["params"], lengths=lengths, num_layers=spec.num_layers,
                               bidirectional=spec.bidirectional, proj_size=spec.proj_size,
                               layout=spec.layout)
            el = time.perf_counter() - t0
            return (int(lengths.sum()) if lengths is not None else spec.T * rows), el

        _, t1 = run(1)
        rows = int(min(spec.B, max(1, seconds / max(t1, 1e-6))))
        tokens, el = run(rows)
        sample = f"{rows} of {spec.B} batch rows over all timesteps, {el:.1f} s"
    return {"value": tokens / el, "unit": UNIT, "cores": int(threads), "kind": "oracle",
            "sample": sample, **host_info()}


if __name__ == "__main__":
    main()
