"""Parity of the HIP path (called through the C ABI) with the float64 oracle.

Tolerances: fp32 elementwise |g - r| <= 1e-4 |r| + 1e-5 plus a 1e-4 relative
L2 bound; bf16 storage (fp32 accumulation) |g - r| <= 2e-2.
Small cases span several workgroup tiles and ragged tails; the five
workloads run at full size in the launch shape the bench times, and every
output element is compared with the oracle on the whole batch.
"""

import zlib

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import log, run_rnn, run_rssm, run_rssm_actor
from helpers import assert_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gru_sequence_scan_amd as gss
    assert gss.rnn_device_check() == 0, "current device is not gfx950"
    torch.cuda.set_device(0)


def _oracle(d, **kw):
    return oracle.rnn_forward(d["mode"], d["x"], d["params"], lengths=d["lengths"], h0=d["h0"],
                              c0=d.get("c0"), num_layers=d["num_layers"],
                              bidirectional=d["bidirectional"], proj_size=d["proj_size"],
                              layout=d["layout"], **kw)


def _compare(d, got, ref, what):
    y, hn, cn = got
    yr, hnr, cnr = ref
    assert_close(y, yr, d["dtype"], what + " y")
    assert_close(hn, hnr, d["dtype"], what + " h_n")
    if cnr is not None:
        assert_close(cn, cnr, d["dtype"], what + " c_n")


SMALL = [
    # name, mode, dtype, T, B, F, H, P, L, bidir, layout, varlen, bias, state
    ("lstm_b1_valu", "lstm", "f32", 9, 1, 13, 20, 0, 1, False, "padded", None, True, True),
    ("lstm_b5_valu", "lstm", "f32", 7, 5, 24, 40, 0, 1, False, "padded", None, True, False),
    ("lstm_b37_mfma", "lstm", "f32", 11, 37, 40, 72, 0, 1, False, "padded", None, True, True),
    ("lstm_nobias", "lstm", "f32", 6, 18, 16, 33, 0, 1, False, "padded", None, False, True),
    ("gru_f32", "gru", "f32", 10, 33, 20, 48, 0, 1, False, "padded", None, True, True),
    ("gru_bf16", "gru", "bf16", 12, 40, 64, 96, 0, 1, False, "padded", None, True, True),
    ("gru_b3", "gru", "f32", 8, 3, 10, 17, 0, 2, True, "padded", None, True, True),
    ("lstmp_f32", "lstmp", "f32", 9, 20, 24, 64, 24, 2, False, "padded", None, True, True),
    ("lstmp_bf16", "lstmp", "bf16", 10, 33, 40, 128, 40, 2, False, "padded", None, True, False),
    ("bilstm_packed", "lstm", "f32", 15, 21, 19, 40, 0, 2, True, "packed", (1, 15), True, True),
    ("bigru_packed_bf16", "gru", "bf16", 13, 34, 32, 64, 0, 2, True, "packed", (2, 13), True, False),
    ("bilstmp_packed", "lstmp", "f32", 12, 17, 16, 48, 16, 2, True, "packed", (1, 12), True, True),
    ("lstm_padded_varlen", "lstm", "f32", 14, 19, 12, 36, 0, 1, True, "padded", "unsorted", True, True),
    # input products with few output tiles split K over workgroups (ragged
    # split ranges; register-staged fp32, unaligned bf16 rows, streamed fp32,
    # and both layers of a packed bidirectional stack)
    ("lstm_splitk_f32", "lstm", "f32", 5, 7, 200, 48, 0, 1, False, "padded", None, True, True),
    ("gru_splitk_bf16", "gru", "bf16", 6, 5, 300, 40, 0, 1, False, "padded", None, True, True),
    ("lstm_splitk_pipe", "lstm", "f32", 4, 9, 256, 72, 0, 1, False, "padded", None, True, False),
    ("bilstm_splitk_packed", "lstm", "f32", 7, 6, 160, 96, 0, 2, True, "packed", (1, 7), True, True),
    # bf16 rows that are whole K stages (the two-stage prefetch form): split
    # ranges of five and four stages, and an odd stage count without a split
    ("gru_splitk_pf_bf16", "gru", "bf16", 4, 4, 448, 64, 0, 1, False, "padded", None, True, True),
    ("gru_pf_odd_stages_bf16", "gru", "bf16", 9, 40, 96, 96, 0, 1, False, "padded", None, True, True),
    # bf16 G_x rows of odd width (3H with H odd): a step's rows start at a
    # 2-byte offset; and the one-wave kernel on bf16 storage (G = 45), its
    # input (8 bf16) narrow enough for the projection inside the kernel
    ("gru_odd_bf16", "gru", "bf16", 9, 18, 24, 33, 0, 1, False, "padded", None, True, True),
    ("gru_wave_bf16", "gru", "bf16", 11, 3, 8, 15, 0, 1, False, "padded", None, True, True),
    # GRU just past the one-wave kernel's width (H = 17): the tiled scan
    ("gru_h17_tiled", "gru", "f32", 9, 3, 8, 17, 0, 1, False, "padded", None, True, True),
]


def _small_inputs(case):
    name, mode, dt, T, B, F, H, P, L, bidir, layout, varlen, bias, state = case
    lengths = None
    vl = None
    if varlen == "unsorted":
        lengths = np.random.default_rng(7).integers(1, T + 1, size=B).astype(np.int32)
        lengths[3] = T
    elif varlen is not None:
        vl = varlen
    return synth.make_rnn_inputs(mode, T, B, F, H, proj_size=P, num_layers=L, bidirectional=bidir,
                                 dtype=dt, layout=layout, lengths=lengths, varlen=vl,
                                 w_scale=1.0 / np.sqrt(H), bias=bias, seed=zlib.crc32(name.encode()) % 1000,
                                 h0_std=0.3 if state else 0.0, c0_std=0.3 if state else 0.0)


GX_F32 = ["gru_bf16", "lstmp_bf16", "bigru_packed_bf16", "gru_odd_bf16"]


@pytest.mark.parametrize("name", GX_F32)
def test_bf16_storage_with_fp32_gx(name):
    """bf16 storage with the hoisted product kept in fp32 (gx_dtype="f32")."""
    case = next(c for c in SMALL if c[0] == name)
    log(f"[gpu] small case {name}, fp32 G_x")
    d = _small_inputs(case)
    got = run_rnn(d, y_fill=float("nan"), gx_dtype="f32")
    _compare(d, got, _oracle(d), name + " (fp32 G_x)")


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_cases(case):
    name, mode, dt, T, B, F, H, P, L, bidir, layout, varlen, bias, state = case
    log(f"[gpu] small case {name}")
    lengths = None
    vl = None
    if varlen == "unsorted":
        lengths = np.random.default_rng(7).integers(1, T + 1, size=B).astype(np.int32)
        lengths[3] = T
    elif varlen is not None:
        vl = varlen
    d = synth.make_rnn_inputs(mode, T, B, F, H, proj_size=P, num_layers=L, bidirectional=bidir,
                              dtype=dt, layout=layout, lengths=lengths, varlen=vl,
                              w_scale=1.0 / np.sqrt(H), bias=bias, seed=zlib.crc32(name.encode()) % 1000,
                              h0_std=0.3 if state else 0.0, c0_std=0.3 if state else 0.0)
    got = run_rnn(d, y_fill=float("nan"))
    ref = _oracle(d)
    _compare(d, got, ref, name)


# The few-row scan (kernel 5 in the plan: at most 8 direction x batch rows,
# H <= 512): LSTM and GRU, fp32 and bf16, padded and packed variable
# lengths, both directions, stacked layers, one and two units per wave.
SMALL_SCAN = [
    # name, mode, dtype, T, B, F, H, L, bidir, layout, varlen, state
    ("few_bilstm_packed_2l", "lstm", "f32", 13, 4, 24, 72, 2, True, "packed", (1, 13), True),
    ("few_gru_bf16_varlen", "gru", "bf16", 11, 3, 40, 300, 1, False, "padded", "unsorted", True),
    ("few_lstm_h512_b8_two_units", "lstm", "f32", 5, 8, 512, 512, 1, False, "padded", None, False),
    ("few_gru_b1_wide_in", "gru", "f32", 7, 1, 512, 256, 1, False, "padded", None, True),
    ("few_lstm_bf16_in_600", "lstm", "bf16", 6, 2, 600, 64, 1, False, "padded", None, True),
]


@pytest.mark.parametrize("case", SMALL_SCAN, ids=[c[0] for c in SMALL_SCAN])
def test_small_scan_cases(case):
    import gru_sequence_scan_amd as gss
    name, mode, dt, T, B, F, H, L, bidir, layout, varlen, state = case
    log(f"[gpu] few-row scan case {name}")
    lengths = None
    vl = None
    if varlen == "unsorted":
        lengths = np.random.default_rng(11).integers(1, T + 1, size=B).astype(np.int32)
        lengths[1] = T
    elif varlen is not None:
        vl = varlen
    d = synth.make_rnn_inputs(mode, T, B, F, H, num_layers=L, bidirectional=bidir, dtype=dt, layout=layout,
                              lengths=lengths, varlen=vl, w_scale=1.0 / np.sqrt(H),
                              seed=zlib.crc32(name.encode()) % 1000, h0_std=0.3 if state else 0.0,
                              c0_std=0.3 if state else 0.0)
    desc = _desc_of(d)
    desc.bidirectional = int(bidir)
    desc.layout = 1 if layout == "packed" else 0
    assert gss.rnn_plan_info(desc, d["lengths"])["kernel"] == 5
    got = run_rnn(d, y_fill=float("nan"))
    ref = _oracle(d)
    _compare(d, got, ref, name)


# The largest hidden sizes the planner accepts on one MI355X: groups of 128 to
# 256 members (every CU in one group for the B = 1 fp32 and the bf16 H = 2048
# cases), weights resident in LDS or registers. One size beyond is rejected
# before launch (checked on the CPU in the planner tests).
MAX_CASES = [
    # name, mode, dtype, T, B, F, H
    ("lstm_f32_h1024_b1", "lstm", "f32", 3, 1, 64, 1024),
    ("lstm_f32_h1024_b16", "lstm", "f32", 3, 16, 64, 1024),
    ("gru_f32_h1024_b16", "gru", "f32", 3, 16, 64, 1024),
    ("lstm_bf16_h2048_b16", "lstm", "bf16", 3, 16, 64, 2048),
]


@pytest.mark.parametrize("case", MAX_CASES, ids=[c[0] for c in MAX_CASES])
def test_max_size_cases(case):
    name, mode, dt, T, B, F, H = case
    log(f"[gpu] maximum size case {name}")
    d = synth.make_rnn_inputs(mode, T, B, F, H, dtype=dt, w_scale=1.0 / np.sqrt(H),
                              seed=zlib.crc32(name.encode()) % 1000, h0_std=0.3, c0_std=0.3)
    got = run_rnn(d, y_fill=float("nan"))
    ref = _oracle(d)
    _compare(d, got, ref, name)


@pytest.mark.parametrize("case", __import__("layout_cases").REG_CASES, ids=lambda c: c[0])
def test_register_layouts(case):
    """Each register-resident W_hh layout (and the LDS fallback) against the
    oracle; the planner side of each case is checked on the CPU."""
    name, mode, dt, T, B, F, H, P, bb, hs, bidir, layout, varlen, expect = case
    log(f"[gpu] register layout case {name}")
    d = synth.make_rnn_inputs(mode, T, B, F, H, proj_size=P, num_layers=1, bidirectional=bidir, dtype=dt,
                              layout=layout, varlen=varlen, w_scale=1.0 / np.sqrt(H),
                              seed=zlib.crc32(name.encode()) % 1000, h0_std=0.3, c0_std=0.3)
    got = run_rnn(d, y_fill=float("nan"), tile_batch=bb, tile_hidden=hs, weights=2 if expect[0] else 1)
    _compare(d, got, _oracle(d), name)


CLIP_CASES = [
    # name, mode, dtype, T, B, F, H, P, L, bidir, layout, varlen, cell_clip, proj_clip
    ("clip_lstm_mfma", "lstm", "f32", 11, 37, 40, 72, 0, 1, False, "padded", None, (-0.3, 0.45), None),
    ("clip_lstm_valu", "lstm", "f32", 9, 5, 24, 40, 0, 2, False, "padded", None, 0.35, None),
    ("clip_lstm_solo", "lstm", "f32", 20, 1, 8, 16, 0, 1, False, "padded", None, (-0.5, 0.2), None),
    ("clip_lstmp_bf16", "lstmp", "bf16", 10, 33, 40, 128, 40, 2, False, "padded", None, 0.4, 0.1),
    ("clip_bilstmp_packed", "lstmp", "f32", 12, 17, 16, 48, 16, 2, True, "packed", (1, 12), (-0.25, 0.6), 0.15),
    ("clip_lstmp_proj_only", "lstmp", "f32", 9, 20, 24, 64, 24, 1, False, "padded", None, None, 0.12),
]


@pytest.mark.parametrize("case", CLIP_CASES, ids=[c[0] for c in CLIP_CASES])
def test_clipping(case):
    """Cell-state and projection clipping against the oracle, with weights
    large enough that the clamps bind on many elements."""
    name, mode, dt, T, B, F, H, P, L, bidir, layout, varlen, cc, pc = case
    log(f"[gpu] clipping case {name}")
    d = synth.make_rnn_inputs(mode, T, B, F, H, proj_size=P, num_layers=L, bidirectional=bidir,
                              dtype=dt, layout=layout, varlen=varlen, w_scale=2.0 / np.sqrt(H),
                              seed=zlib.crc32(name.encode()) % 1000, h0_std=0.3, c0_std=0.3)
    lohi = None if cc is None else ((-cc, cc) if isinstance(cc, float) else cc)
    ref = _oracle(d, cell_clip=lohi, proj_clip=pc)
    # the clamps must actually bind somewhere, else the case tests nothing
    if lohi is not None:
        assert np.isin(ref[2], lohi).mean() > 0.02
    if pc is not None:
        y = ref[0][~np.isnan(ref[0])]
        assert (np.abs(y) == pc).mean() > 0.02
    got = run_rnn(d, y_fill=float("nan"), cell_clip=cc, proj_clip=pc)
    _compare(d, got, ref, name)


WAVE_CASES = [
    # one wave per (direction, row): gates * H <= 64
    # name, mode, dtype, T, B, F, H, L, bidir, layout, varlen, bias, cell_clip
    ("wave_lstm_h16_b1", "lstm", "f32", 40, 1, 16, 16, 1, False, "padded", None, True, None),
    ("wave_bilstm_packed", "lstm", "f32", 17, 9, 12, 16, 2, True, "packed", (1, 17), True, None),
    ("wave_gru_h16_bf16", "gru", "bf16", 23, 6, 20, 16, 2, False, "padded", None, True, None),
    # input projection inside the kernel (x staged in LDS) and from kernel 1:
    # fp32 rows of 8 (fused), a sequence whose x passes 16 KB (kernel 1),
    # bf16 rows of 16 (fused) in both directions of a two-layer stack
    ("wave_gru_fused_f32", "gru", "f32", 30, 5, 8, 12, 1, False, "padded", None, True, None),
    ("wave_lstm_long_unfused", "lstm", "f32", 200, 2, 32, 16, 1, False, "padded", None, True, None),
    ("wave_bilstm_fused_bf16", "lstm", "bf16", 40, 7, 16, 8, 2, True, "padded", "unsorted", True, (-0.4, 0.3)),
    ("wave_gru_h1", "gru", "f32", 9, 3, 4, 1, 1, False, "padded", None, True, None),
    ("wave_lstm_h5_varlen", "lstm", "f32", 15, 7, 6, 5, 1, True, "padded", "unsorted", True, None),
    ("wave_lstm_clip", "lstm", "f32", 12, 4, 8, 12, 1, False, "padded", None, True, (-0.3, 0.25)),
    ("wave_lstm_nobias_bf16", "lstm", "bf16", 10, 5, 16, 16, 1, False, "padded", None, False, None),
    ("wave_gru_b300", "gru", "f32", 6, 300, 8, 8, 1, True, "padded", None, True, None),
]


@pytest.mark.parametrize("case", WAVE_CASES, ids=[c[0] for c in WAVE_CASES])
def test_wave_scan(case):
    name, mode, dt, T, B, F, H, L, bidir, layout, varlen, bias, cc = case
    log(f"[gpu] wave scan case {name}")
    lengths, vl = None, None
    if varlen == "unsorted":
        lengths = np.random.default_rng(8).integers(1, T + 1, size=B).astype(np.int32)
    elif varlen is not None:
        vl = varlen
    d = synth.make_rnn_inputs(mode, T, B, F, H, num_layers=L, bidirectional=bidir, dtype=dt, layout=layout,
                              lengths=lengths, varlen=vl, w_scale=1.5 / np.sqrt(H), bias=bias,
                              seed=zlib.crc32(name.encode()) % 1000, h0_std=0.3, c0_std=0.3)
    ref = _oracle(d, cell_clip=cc)
    got = run_rnn(d, y_fill=float("nan"), cell_clip=cc)
    _compare(d, got, ref, name)
    # the tiled scan (forced by a tiling hint) agrees with the oracle too,
    # where its persistent groups fit the device
    if B <= 32:
        got_tiled = run_rnn(d, y_fill=float("nan"), cell_clip=cc, tile_batch=1)
        _compare(d, got_tiled, ref, name + " tiled")


def test_padding_sentinel_untouched():
    log("[gpu] padding sentinel")
    lengths = np.array([5, 9, 2, 9, 1, 7, 3, 8], dtype=np.int32)
    d = synth.make_rnn_inputs("lstm", 9, 8, 12, 24, num_layers=2, bidirectional=True,
                              lengths=lengths, w_scale=0.2, seed=3)
    y, hn, cn = run_rnn(d, y_fill=1234.5)
    for b, lb in enumerate(lengths):
        assert np.all(y[lb:, b] == 1234.5), f"row {b}: padding overwritten"
        assert np.all(np.isfinite(y[:lb, b]))


def test_determinism_bitwise():
    log("[gpu] determinism")
    d = synth.make_rnn_inputs("gru", 16, 48, 32, 64, dtype="bf16", w_scale=0.125, seed=4, h0_std=0.1)
    a = run_rnn(d)
    b = run_rnn(d)
    for x, y in zip(a, b):
        if x is not None:
            assert np.array_equal(x, y)


# Layer-pipelined stacks (one launch scans a time chunk of every layer, layer
# l one chunk behind layer l - 1; the state crosses chunk boundaries through
# the workspace): several chunks each, with a ragged last one (1 step for
# the T = 65, 97 and 129 cases, whose chunks are 32 steps).
PIPE_CASES = [
    # name, mode, dtype, T, B, F, H, P, L, cell_clip, proj_clip, last chunk's steps
    ("pipe_lstm_f32", "lstm", "f32", 130, 20, 24, 64, 0, 2, None, None, 31),
    ("pipe_gru_bf16_3l", "gru", "bf16", 129, 33, 40, 96, 0, 3, None, None, 1),
    ("pipe_lstmp_bf16", "lstmp", "bf16", 100, 32, 40, 128, 40, 2, None, None, 4),
    ("pipe_lstmp_f32_4l", "lstmp", "f32", 97, 17, 16, 48, 16, 4, None, None, 1),
    ("pipe_lstm_b2", "lstm", "f32", 100, 2, 8, 24, 0, 2, None, None, 4),
    ("pipe_lstmp_clip_bf16", "lstmp", "bf16", 65, 33, 40, 128, 40, 2, 0.4, 0.1, 1),
]


def _desc_of(d):
    import gru_sequence_scan_amd as gss
    desc = gss.RnnDesc()
    desc.mode, desc.dtype = gss.MODES[d["mode"]], 1 if d["dtype"] == "bf16" else 0
    desc.T, desc.B, desc.input_size, desc.hidden_size = d["T"], d["B"], d["x"].shape[-1], d["hidden_size"]
    desc.proj_size, desc.num_layers, desc.has_bias = d["proj_size"], d["num_layers"], 1
    return desc


@pytest.mark.parametrize("case", PIPE_CASES, ids=[c[0] for c in PIPE_CASES])
def test_layer_pipeline(case):
    """The pipelined stack gives the layer-by-layer run's results bit for
    bit, and both match the oracle."""
    import gru_sequence_scan_amd as gss
    name, mode, dt, T, B, F, H, P, L, cc, pc, tail = case
    log(f"[gpu] layer pipeline case {name}")
    d = synth.make_rnn_inputs(mode, T, B, F, H, proj_size=P, num_layers=L, dtype=dt,
                              w_scale=(2.0 if cc else 1.0) / np.sqrt(H),
                              seed=zlib.crc32(name.encode()) % 1000, h0_std=0.3, c0_std=0.3)
    desc = _desc_of(d)
    desc.layer_pipeline = gss.PIPE_MODES["on"]
    plan = gss.rnn_plan_info(desc)
    chunk = plan["pipe_chunk"]
    assert chunk >= 32 and T > chunk and T - (T - 1) // chunk * chunk == tail
    # the layer-by-layer run in the same tiled launch shape (a small batch
    # would otherwise take the few-row scan, whose sums run in another order)
    tiles = dict(tile_batch=plan["rows"], tile_hidden=plan["hidden_per_wg"])
    piped = run_rnn(d, y_fill=float("nan"), cell_clip=cc, proj_clip=pc, layer_pipeline="on", **tiles)
    layered = run_rnn(d, y_fill=float("nan"), cell_clip=cc, proj_clip=pc, layer_pipeline="off", **tiles)
    for a, b, what in zip(piped, layered, ("y", "h_n", "c_n")):
        if b is not None:
            assert np.array_equal(a, b), f"{name}: pipelined {what} differs from the layer-by-layer run"
    lohi = None if cc is None else (-cc, cc)
    _compare(d, piped, _oracle(d, cell_clip=lohi, proj_clip=pc), name)
    if dt == "bf16":
        got = run_rnn(d, y_fill=float("nan"), cell_clip=cc, proj_clip=pc, gx_dtype="f32", layer_pipeline="on")
        _compare(d, got, _oracle(d, cell_clip=lohi, proj_clip=pc), name + " (fp32 G_x)")


@pytest.mark.parametrize("mode,P", [("lstm", 0), ("gru", 0), ("lstmp", 16)])
def test_time_chunking_matches_one_call(mode, P):
    log(f"[gpu] chunking {mode}")
    d = synth.make_rnn_inputs(mode, 12, 20, 16, 48, proj_size=P, num_layers=2, w_scale=0.15, seed=5)
    y, hn, cn = run_rnn(d)
    d1 = dict(d, x=d["x"][:5], x_padded=d["x"][:5], T=5)
    y1, hn1, cn1 = run_rnn(d1)
    d2 = dict(d, x=d["x"][5:], x_padded=d["x"][5:], T=7, h0=hn1.astype(np.float32),
              c0=None if cn1 is None else cn1.astype(np.float32))
    y2, hn2, cn2 = run_rnn(d2)
    assert_close(np.concatenate([y1, y2]), y, "f32", "chunked y")
    assert_close(hn2, hn, "f32", "chunked h_n")


def test_t1_equals_one_cell_step():
    log("[gpu] T=1")
    d = synth.make_rnn_inputs("lstm", 1, 16, 24, 32, w_scale=0.2, seed=6, h0_std=0.5, c0_std=0.5)
    y, hn, cn = run_rnn(d)
    p = d["params"][0]
    h1, c1 = oracle.lstm_cell(d["x"][0], d["h0"][0], d["c0"][0], p["w_ih"], p["w_hh"], p["b_ih"], p["b_hh"])
    assert_close(y[0], h1, "f32", "T=1 y")
    assert_close(cn[0], c1, "f32", "T=1 c")


def test_packed_equals_padded_on_gpu():
    log("[gpu] packed == padded")
    lengths = np.array([10, 9, 9, 6, 4, 4, 2, 1], dtype=np.int32)
    d = synth.make_rnn_inputs("lstm", 10, 8, 16, 40, num_layers=2, bidirectional=True,
                              layout="packed", lengths=lengths, w_scale=0.2, seed=8)
    yk, hk, ck = run_rnn(d)
    dp = dict(d, layout="padded", x=np.nan_to_num(d["x_padded"]))
    yp, hp, cp = run_rnn(dp, y_fill=float("nan"))
    np.testing.assert_array_equal(oracle.pack_sequence(yp, lengths), yk)
    np.testing.assert_array_equal(hk, hp)
    np.testing.assert_array_equal(ck, cp)


# ---------------------------------------------------------------------------
# RSSM prior
# ---------------------------------------------------------------------------

# weights hint: 0 lets the planner choose (the register kernel where the
# shape fits it), 1 the kernel with LDS-resident input weights
RSSM_KERNELS = [0, 1]


@pytest.mark.parametrize("wh", RSSM_KERNELS)
def test_rssm_small(wh):
    log(f"[gpu] rssm small (weights hint {wh})")
    d = synth.make_rssm_inputs(7, 9, state_dim=5, action_dim=3, embed_dim=24, belief_dim=20, seed=9,
                               s0_std=0.5, h0_std=0.5)
    got = run_rssm(d, weights_hint=wh)
    ref = oracle.rssm_prior_unroll(d["actions"], d["eps"], d["weights"], d["s0"], d["h0"])
    for g, r, nm in zip(got, ref, ("means", "stds", "states", "beliefs")):
        assert_close(g, r, "f32", "rssm " + nm)


RSSM_SHAPES = [
    # name, B, T, S, A, E, Hb, tile_batch, tile_hidden
    ("rssm_wide_state", 6, 5, 40, 4, 36, 30, 0, 0),      # 2S > 64: products in two passes
    ("rssm_wide_slice", 5, 6, 6, 2, 70, 75, 0, 25),      # 3 * slice > 64, E > 64
    ("rssm_rows4_odd", 10, 7, 8, 3, 33, 26, 4, 0),       # widths not multiples of 4
    ("rssm_rows1", 3, 4, 5, 2, 16, 12, 1, 0),
]


@pytest.mark.parametrize("wh", RSSM_KERNELS)
@pytest.mark.parametrize("case", RSSM_SHAPES, ids=[c[0] for c in RSSM_SHAPES])
def test_rssm_shapes(case, wh):
    name, B, T, S, A, E, Hb, tb, th = case
    log(f"[gpu] rssm shape {name} (weights hint {wh})")
    d = synth.make_rssm_inputs(B, T, state_dim=S, action_dim=A, embed_dim=E, belief_dim=Hb,
                               seed=zlib.crc32(name.encode()) % 1000, s0_std=0.5, h0_std=0.5)
    got = run_rssm(d, tile_batch=tb, tile_hidden=th, weights_hint=wh)
    ref = oracle.rssm_prior_unroll(d["actions"], d["eps"], d["weights"], d["s0"], d["h0"])
    for g, r, nm in zip(got, ref, ("means", "stds", "states", "beliefs")):
        assert_close(g, r, "f32", f"{name} {nm}")


@pytest.mark.parametrize("wh", RSSM_KERNELS)
def test_rssm_zero_weights_closed_form(wh):
    log(f"[gpu] rssm closed form (weights hint {wh})")
    d = synth.make_rssm_inputs(6, 4, seed=10, zero_weights=True)
    means, stds, states, beliefs = run_rssm(d, weights_hint=wh)
    assert np.all(beliefs == 0) and np.all(means == 0)
    k = np.log(2.0) + 0.1
    assert_close(stds, np.full_like(stds, k), "f32", "stds")
    assert_close(states, k * d["eps"].astype(np.float64), "f32", "states")


RSSM_ACTOR_SHAPES = [
    # name, B, T, S, A, E, Hb, Ea, tile_batch, tile_hidden
    ("actor_small", 7, 6, 5, 3, 24, 40, 17, 0, 0),         # widths not multiples of 4
    ("actor_wide", 6, 5, 8, 4, 36, 30, 90, 0, 0),          # actor wider than one 64-column pass
    ("actor_rows4", 9, 7, 4, 2, 20, 26, 33, 4, 0),
    ("actor_rows1_slices", 3, 5, 6, 5, 18, 50, 12, 1, 7),
    ("actor_lds_weights", 4, 4, 36, 3, 30, 24, 20, 0, 0),  # 2S > 64: weights stay in LDS
]


@pytest.mark.parametrize("case", RSSM_ACTOR_SHAPES, ids=[c[0] for c in RSSM_ACTOR_SHAPES])
def test_rssm_actor_shapes(case):
    name, B, T, S, A, E, Hb, Ea, tb, th = case
    log(f"[gpu] rssm actor shape {name}")
    d = synth.make_rssm_inputs(B, T, state_dim=S, action_dim=A, embed_dim=E, belief_dim=Hb, actor_dim=Ea,
                               seed=zlib.crc32(name.encode()) % 1000, s0_std=0.5, h0_std=0.5)
    got = run_rssm_actor(d, tile_batch=tb, tile_hidden=th)
    ref = oracle.rssm_actor_unroll(d["eps"], d["weights"], d["actor"], d["s0"], d["h0"])
    for g, r, nm in zip(got, ref, ("means", "stds", "states", "beliefs", "actions")):
        assert_close(g, r, "f32", f"{name} {nm}")


# The same unroll on kernel 3 (GRU weights resident in LDS, counter
# barrier), which the planner otherwise keeps for shapes kernel 3b cannot
# hold.
@pytest.mark.parametrize("case", [RSSM_ACTOR_SHAPES[0], RSSM_ACTOR_SHAPES[1]], ids=["actor_small", "actor_wide"])
def test_rssm_actor_shapes_lds_weights(case):
    name, B, T, S, A, E, Hb, Ea, tb, th = case
    log(f"[gpu] rssm actor shape {name}, LDS-resident weights")
    d = synth.make_rssm_inputs(B, T, state_dim=S, action_dim=A, embed_dim=E, belief_dim=Hb, actor_dim=Ea,
                               seed=zlib.crc32(name.encode()) % 1000, s0_std=0.5, h0_std=0.5)
    got = run_rssm_actor(d, tile_batch=tb, tile_hidden=th, weights_hint=1)
    ref = oracle.rssm_actor_unroll(d["eps"], d["weights"], d["actor"], d["s0"], d["h0"])
    for g, r, nm in zip(got, ref, ("means", "stds", "states", "beliefs", "actions")):
        assert_close(g, r, "f32", f"{name} {nm}")


def test_rssm_actor_zero_weights_closed_form():
    log("[gpu] rssm actor closed form")
    d = synth.make_rssm_inputs(5, 4, seed=11, zero_weights=True, actor_dim=24)
    d["actor"] = {k: np.zeros_like(v) for k, v in d["actor"].items()}
    means, stds, states, beliefs, actions = run_rssm_actor(d)
    assert np.all(beliefs == 0) and np.all(means == 0) and np.all(actions == 0)
    k = np.log(2.0) + 0.1
    assert_close(stds, np.full_like(stds, k), "f32", "stds")
    assert_close(states, k * d["eps"].astype(np.float64), "f32", "states")


# ---------------------------------------------------------------------------
# The five workloads at full size
# ---------------------------------------------------------------------------

def _full(name):
    """A workload at full size in the launch shape the bench times, every
    output element compared with the oracle on the whole batch."""
    d = synth.make_inputs(name)
    log(f"[gpu] full-size {name} (whole batch)")
    got = run_rnn(d, y_fill=float("nan"))
    _compare(d, got, _oracle(d), name)
    return d, got


def test_full_lstm_t80_b1():
    d = synth.make_inputs("lstm_t80_b1")
    log("[gpu] full-size lstm_t80_b1")
    _compare(d, run_rnn(d), _oracle(d), "lstm_t80_b1")


@pytest.mark.parametrize("wh", RSSM_KERNELS)
def test_full_rssm_b50_t50(wh):
    d = synth.make_inputs("rssm_b50_t50")
    log(f"[gpu] full-size rssm_b50_t50 (weights hint {wh})")
    got = run_rssm(d, weights_hint=wh)
    ref = oracle.rssm_prior_unroll(d["actions"], d["eps"], d["weights"])
    for g, r, nm in zip(got, ref, ("means", "stds", "states", "beliefs")):
        assert_close(g, r, "f32", "rssm_b50_t50 " + nm)


def test_rssm_register_kernel_chosen_for_the_headline_shape():
    """The planner takes the register kernel (wide members, ring exchange
    inside an XCD) for the B=50, T=50 unroll; hint 1 keeps the other one."""
    import gru_sequence_scan_amd as gss
    d = gss.RnnDesc()
    for k, v in dict(mode=3, dtype=0, layout=2, T=50, B=50, num_layers=1, has_bias=1, state_dim=20,
                     action_dim=6, embed_dim=200, belief_dim=200).items():
        setattr(d, k, v)
    d.scale_lb = 0.1
    p = gss.rnn_plan_info(d)
    assert p["wreg"] == 1 and p["members"] <= 8 and p["groups_per_xcd"] > 0
    d.weights = 1
    assert gss.rnn_plan_info(d)["wreg"] == 0


def test_full_gru_t256_b256():
    _full("gru_t256_b256")


def test_full_lstmp_t1000_b32():
    _full("lstmp_t1000_b32")


def test_full_bilstm_varlen_b64():
    _full("bilstm_varlen_b64")


def test_full_bilstm_varlen_b64_padded_sentinel():
    """The var-len stack in the padded layout (T = 500, x NaN past each
    length): y is pre-filled with a sentinel that must survive at every
    t >= L_b, and every written element matches the oracle."""
    d = synth.make_inputs("bilstm_varlen_b64")
    dp = dict(d, layout="padded", x=d["x_padded"], T=d["x_padded"].shape[0])
    log("[gpu] full-size bilstm_varlen_b64, padded layout with a sentinel")
    y, hn, cn = run_rnn(dp, y_fill=1234.5)
    L = d["lengths"]
    assert y.shape[0] == 500
    for b, lb in enumerate(L):
        assert np.all(y[lb:, b] == 1234.5), f"row {b}: a padded position was written"
    yr, hnr, cnr = _oracle(dp)
    written = ~np.isnan(yr)
    for b, lb in enumerate(L):
        assert written[:lb, b].all() and not written[lb:, b].any()
    _compare(dp, (np.where(written, y, np.nan), hn, cn), (yr, hnr, cnr), "bilstm_varlen_b64 padded")


def test_full_lstm_t256_b1_small():
    d = synth.make_inputs("lstm_t256_b1_small")
    log("[gpu] full-size lstm_t256_b1_small")
    _compare(d, run_rnn(d), _oracle(d), "lstm_t256_b1_small")


@pytest.mark.parametrize("weights_hint", [0, 1], ids=["planned", "lds_weights"])
def test_full_rssm_actor_b50_h50(weights_hint):
    d = synth.make_inputs("rssm_actor_b50_h50")
    log(f"[gpu] full-size rssm_actor_b50_h50 weights hint {weights_hint}")
    got = run_rssm_actor(d, weights_hint=weights_hint)
    ref = oracle.rssm_actor_unroll(d["eps"], d["weights"], d["actor"])
    for g, r, nm in zip(got, ref, ("means", "stds", "states", "beliefs", "actions")):
        assert_close(g, r, "f32", "rssm_actor_b50_h50 " + nm)


def test_exchange_roundtrip_probe():
    """The measurement helper returns a plausible device-coherent round trip
    (between 0.1 and 100 microseconds on an idle device)."""
    import gru_sequence_scan_amd as gss
    ns = gss.rnn_exchange_roundtrip_ns(500)
    log(f"[gpu] exchange round trip {ns:.0f} ns")
    assert 100.0 < ns < 100000.0
