"""Backward through time on the GPU (rnn_forward_train + rnn_backward,
through the C ABI) against the float64 oracle's BPTT, on the same seeded
inputs and upstream gradients. Tolerance: tests/helpers.assert_grad_close."""

import zlib

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import log, to_dev
from helpers import assert_close, assert_grad_close

pytestmark = pytest.mark.gpu

gss = pytest.importorskip("gru_sequence_scan_amd")

BWD_GPU_CASES = [
    # name, mode, T, B, F, H, L, bidir, layout, varlen, bias, tile_batch
    ("lstm_valu", "lstm", 9, 5, 12, 24, 1, False, "padded", None, True, 0),
    ("lstm_mfma_b32", "lstm", 8, 32, 20, 64, 1, False, "padded", None, True, 0),
    ("gru_valu", "gru", 10, 6, 8, 20, 1, False, "padded", None, True, 0),
    ("gru_nobias_bidir", "gru", 7, 9, 10, 16, 1, True, "padded", None, False, 0),
    ("lstm_bidir_packed_2l", "lstm", 12, 11, 9, 32, 2, True, "packed", (1, 12), True, 0),
    ("gru_bidir_padded_varlen_2l", "gru", 11, 7, 6, 24, 2, True, "padded", "unsorted", True, 0),
    ("lstm_3layers_mfma", "lstm", 6, 16, 16, 48, 3, False, "padded", None, True, 16),
    ("gru_b33_rows", "gru", 5, 33, 12, 40, 1, True, "packed", (2, 5), True, 0),
    ("lstmp_mfma", "lstmp", 8, 16, 12, 32, 1, False, "padded", None, True, 16, 16),
    ("lstmp_bidir_packed_2l", "lstmp", 10, 9, 8, 24, 2, True, "packed", (1, 10), True, 0, 12),
    ("lstmp_padded_varlen_nobias", "lstmp", 9, 5, 6, 20, 1, False, "padded", "unsorted", False, 0, 8),
    # wide batch tiles (MFMA partial products stored from the accumulators)
    ("gru_b256_h512_wide", "gru", 3, 256, 32, 512, 1, False, "padded", None, True, 0),
    ("lstm_bidir_b128_h512_wide", "lstm", 4, 128, 16, 512, 1, True, "packed", (1, 4), True, 0),
    # a vector-ALU block of 40 rows: its partial products pass through LDS in
    # two column passes
    ("lstm_b40_valu_colpass", "lstm", 3, 40, 8, 512, 1, False, "padded", None, True, 40),
]


def _unpack(case):
    """name, mode, T, B, F, H, L, bidir, layout, varlen, bias, tile_batch, P."""
    return case if len(case) == 13 else case + (0,)


def _inputs(case):
    name, mode, T, B, F, H, L, bidir, layout, varlen, bias, tb, P = _unpack(case)
    lengths, vl = None, None
    if varlen == "unsorted":
        lengths = np.random.default_rng(9).integers(1, T + 1, size=B).astype(np.int32)
    elif varlen is not None:
        vl = varlen
    d = synth.make_rnn_inputs(mode, T, B, F, H, proj_size=P, num_layers=L, bidirectional=bidir, layout=layout,
                              lengths=lengths, varlen=vl, w_scale=1.0 / np.sqrt(H), bias=bias,
                              seed=zlib.crc32(name.encode()) % 1000, h0_std=0.3, c0_std=0.3)
    if layout == "padded":
        d["x"] = np.nan_to_num(d["x"])  # padded positions must be finite for training
    rng = np.random.default_rng(zlib.crc32(name.encode()) % 977)
    D = 2 if bidir else 1
    K = P if mode == "lstmp" else H
    rows = d["x"].shape[0] if layout == "packed" else None
    yshape = (rows, D * K) if layout == "packed" else (T, B, D * K)
    dy = rng.normal(size=yshape).astype(np.float32)
    dh_n = rng.normal(size=(L * D, B, K)).astype(np.float32)
    dc_n = rng.normal(size=(L * D, B, H)).astype(np.float32) if mode != "gru" else None
    return d, dy, dh_n, dc_n


@pytest.mark.parametrize("case", BWD_GPU_CASES, ids=[c[0] for c in BWD_GPU_CASES])
def test_backward_matches_oracle(case):
    name, mode, T, B, F, H, L, bidir, layout, varlen, bias, tb, P = _unpack(case)
    log(f"[gpu] backward case {name}")
    d, dy, dh_n, dc_n = _inputs(case)
    f = lambda a: to_dev(a, torch.float32)
    params = [{k: f(v) for k, v in p.items() if v is not None} for p in d["params"]]
    (y, hn, cn), ctx = gss.rnn_forward_train(mode, f(d["x"]), params, h0=f(d["h0"]), c0=f(d.get("c0")),
                                             lengths=d["lengths"], layout=layout, num_layers=L,
                                             bidirectional=bidir, proj_size=P, tile_batch=tb)
    dx, dh0, dc0, grads = gss.rnn_backward(ctx, f(dy), f(dh_n), f(dc_n))
    torch.cuda.synchronize()
    # the training forward's outputs are the forward's
    yr, hnr, cnr = oracle.rnn_forward(mode, d["x"], d["params"], lengths=d["lengths"], h0=d["h0"],
                                      c0=d.get("c0"), num_layers=L, bidirectional=bidir, proj_size=P,
                                      layout=layout)
    yg = y.cpu().numpy().astype(np.float64)
    if layout == "padded" and d["lengths"] is not None:
        yg = np.where(np.isnan(yr), np.nan, yg)
    assert_close(yg, yr, "f32", name + " y")
    assert_close(hn.cpu().numpy(), hnr, "f32", name + " h_n")
    ref = oracle.rnn_backward(mode, d["x"], d["params"], dy, dh_n=dh_n, dc_n=dc_n, lengths=d["lengths"],
                              h0=d["h0"], c0=d.get("c0"), num_layers=L, bidirectional=bidir, proj_size=P,
                              layout=layout)
    g = lambda t: t.cpu().numpy().astype(np.float64)
    assert_grad_close(g(dx), ref[0], name + " dx")
    assert_grad_close(g(dh0), ref[1], name + " dh0")
    if mode != "gru":
        assert_grad_close(g(dc0), ref[2], name + " dc0")
    for i, (gg, rr) in enumerate(zip(grads, ref[3])):
        for k in ("w_ih", "w_hh", "b_ih", "b_hh", "w_hr"):
            if "d" + k in gg:
                assert_grad_close(g(gg["d" + k]), rr[k], f"{name} [{i}] d{k}")


def test_backward_deterministic():
    case = BWD_GPU_CASES[4]
    d, dy, dh_n, dc_n = _inputs(case)
    f = lambda a: to_dev(a, torch.float32)
    params = [{k: f(v) for k, v in p.items() if v is not None} for p in d["params"]]
    outs = []
    for _ in range(2):
        _, ctx = gss.rnn_forward_train("lstm", f(d["x"]), params, h0=f(d["h0"]), c0=f(d["c0"]),
                                       lengths=d["lengths"], layout="packed", num_layers=2, bidirectional=True)
        dx, dh0, dc0, grads = gss.rnn_backward(ctx, f(dy), f(dh_n), f(dc_n))
        outs.append([dx.cpu(), dh0.cpu(), grads[0]["dw_hh"].cpu(), grads[3]["db_ih"].cpu()])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.timeout(600)
def test_backward_full_bilstm_varlen_b64():
    """The var-len stack's training step at full size (B = 64, packed,
    N_tok = 19,334, 498 steps, two bidirectional layers of 512) in the launch
    plan the training benchmark runs: dx and dh0 / dc0 on every row and every
    weight and bias gradient whole, against the oracle's BPTT."""
    name = "bilstm_varlen_b64"
    d = synth.make_inputs(name)
    log(f"[gpu] backward full-size {name}")
    rng = np.random.default_rng(2024)
    L, B, H = d["lengths"], d["B"], d["hidden_size"]
    dy = rng.normal(size=(d["x"].shape[0], 2 * H)).astype(np.float32)
    dh_n = rng.normal(size=(4, B, H)).astype(np.float32)
    dc_n = rng.normal(size=(4, B, H)).astype(np.float32)
    f = lambda a: to_dev(a, torch.float32)
    params = [{k: f(v) for k, v in p.items() if v is not None} for p in d["params"]]
    (y, hn, cn), ctx = gss.rnn_forward_train("lstm", f(d["x"]), params, lengths=L, layout="packed",
                                             num_layers=2, bidirectional=True)
    dx, dh0, dc0, grads = gss.rnn_backward(ctx, f(dy), f(dh_n), f(dc_n))
    torch.cuda.synchronize()
    g = lambda t: t.cpu().numpy().astype(np.float64)
    yr, hnr, cnr = oracle.rnn_forward("lstm", d["x"], d["params"], lengths=L, num_layers=2, bidirectional=True,
                                      layout="packed")
    assert_close(g(y), yr, "f32", name + " y")
    assert_close(g(hn), hnr, "f32", name + " h_n")
    assert_close(g(cn), cnr, "f32", name + " c_n")
    ref = oracle.rnn_backward("lstm", d["x"], d["params"], dy, dh_n=dh_n, dc_n=dc_n, lengths=L, num_layers=2,
                              bidirectional=True, layout="packed")
    assert_grad_close(g(dx), ref[0], name + " dx")
    assert_grad_close(g(dh0), ref[1], name + " dh0")
    assert_grad_close(g(dc0), ref[2], name + " dc0")
    for i, (gg, rr) in enumerate(zip(grads, ref[3])):
        for k in ("w_ih", "w_hh", "b_ih", "b_hh"):
            assert_grad_close(g(gg["d" + k]), rr[k], f"{name} [{i}] d{k}")
