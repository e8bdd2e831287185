"""Helpers shared by the GPU tests: run the library on synth inputs."""

import sys

import numpy as np
import torch

import gru_sequence_scan_amd as gss


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a, dtype, device="cuda:0"):
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.float32)))
    return t.to(device=device).to(dtype)


def tdtype(name):
    return torch.bfloat16 if name == "bf16" else torch.float32


def run_rnn(d, y_fill=None, **kw):
    """Run the GPU path on a synth RNN problem; returns numpy float64 outputs."""
    dt = tdtype(d["dtype"])
    params = []
    for p in d["params"]:
        params.append({k: to_dev(v, dt) for k, v in p.items() if v is not None})
    x = to_dev(d["x"], dt)
    h0 = to_dev(d["h0"], dt)
    c0 = to_dev(d.get("c0"), dt)
    D = 2 if d["bidirectional"] else 1
    K = d["proj_size"] if d["mode"] == "lstmp" else d["hidden_size"]
    y_out = None
    if y_fill is not None:
        shape = (x.shape[0], D * K) if d["layout"] == "packed" else (d["T"], d["B"], D * K)
        y_out = torch.full(shape, y_fill, dtype=dt, device=x.device)
    y, hn, cn = gss.rnn_forward(d["mode"], x, params, h0=h0, c0=c0, lengths=d["lengths"],
                                layout=d["layout"], num_layers=d["num_layers"],
                                bidirectional=d["bidirectional"], proj_size=d["proj_size"],
                                y_out=y_out, **kw)
    torch.cuda.synchronize()
    f = lambda t: None if t is None else t.float().cpu().numpy().astype(np.float64)
    return f(y), f(hn), f(cn)


def run_rssm(d, **kw):
    w = {k: to_dev(v, torch.float32) for k, v in d["weights"].items()}
    out = gss.rssm_prior_unroll(to_dev(d["actions"], torch.float32), to_dev(d["eps"], torch.float32), w,
                                to_dev(d["s0"], torch.float32), to_dev(d["h0"], torch.float32), **kw)
    torch.cuda.synchronize()
    return [t.cpu().numpy().astype(np.float64) for t in out]


def run_rssm_actor(d, **kw):
    w = {k: to_dev(v, torch.float32) for k, v in d["weights"].items()}
    aw = {k: to_dev(v, torch.float32) for k, v in d["actor"].items()}
    out = gss.rssm_actor_unroll(to_dev(d["eps"], torch.float32), w, aw, to_dev(d["s0"], torch.float32),
                                to_dev(d["h0"], torch.float32), **kw)
    torch.cuda.synchronize()
    return [t.cpu().numpy().astype(np.float64) for t in out]
