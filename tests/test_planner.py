"""Launch planning on the CPU (rnn_plan_info): every workload gets a plan
whose workgroups are all co-resident (the per-step group barriers need
that), whose LDS fits a CU, whose slices cover the problem, and whose
XCD-aligned layout keeps each group on one XCD."""

import math

import pytest

import synth

gss = pytest.importorskip("gru_sequence_scan_amd")

LDS_MAX = 160 * 1024
CODE = {v: k for k, v in gss.STATUS.items()}


def desc_for(name, **hints):
    s = synth.spec(name)
    d = gss.RnnDesc()
    if s.mode in ("rssm", "rssm_actor"):
        d.mode, d.layout, d.T, d.B, d.num_layers, d.has_bias = gss.MODES[s.mode], 2, s.T, s.B, 1, 1
        d.state_dim, d.action_dim, d.embed_dim, d.belief_dim, d.scale_lb = (
            s.state_dim, s.action_dim, s.embed_dim, s.belief_dim, 0.1)
        d.actor_dim = s.actor_dim
    else:
        d.mode = gss.MODES[s.mode]
        d.dtype = 1 if s.dtype == "bf16" else 0
        d.layout = 1 if s.layout == "packed" else 0
        d.T, d.B = s.T, s.B
        d.input_size, d.hidden_size, d.proj_size = s.input_size, s.hidden_size, s.proj_size
        d.num_layers, d.bidirectional, d.has_bias = s.num_layers, int(s.bidirectional), 1
    for k, v in hints.items():
        setattr(d, k, v)
    lengths = synth.make_inputs(name)["lengths"] if s.varlen else None
    return s, d, lengths


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
@pytest.mark.parametrize("cus,xcds", [(256, 8), (256, 1), (32, 1), (80, 1)])
def test_plan_is_coresident_and_covers(name, cus, xcds):
    s, d, lengths = desc_for(name)
    try:
        p = gss.rnn_plan_info(d, lengths, cus=cus, xcds=xcds)
    except gss.RnnError as e:
        # a device too small for the persistent layout must say so, never
        # return a plan that would deadlock
        assert e.status == CODE["RNN_E_PLAN"]
        assert cus < 256
        return
    if p["kernel"] == 4:
        # one independent wave per (direction, row): any grid size works
        D = 2 if s.bidirectional else 1
        assert s.mode in ("lstm", "gru") and (3 if s.mode == "gru" else 4) * s.hidden_size <= 64
        # (LDS only for x staged by the kernel's own input projection)
        assert p["workgroups"] * 4 >= D * s.B and p["lds_bytes"] in (0, 4 * (16384 + 4096))
        return
    assert p["workgroups"] <= cus
    if p["kernel"] == 5:
        # the few-row scan: one group of `members` workgroups per
        # (direction, row), every group co-resident, no LDS
        D = 2 if s.bidirectional else 1
        assert s.mode in ("lstm", "gru") and D * s.B <= 8 and s.hidden_size <= 512
        assert p["groups"] == D * s.B and p["rows"] == 1 and p["lds_bytes"] == 0
        assert p["hidden_per_wg"] * p["members"] >= s.hidden_size
        assert p["hidden_per_wg"] * (p["members"] - 1) < s.hidden_size
        if p["groups_per_xcd"]:
            assert p["groups_per_xcd"] * xcds >= p["groups"]
            assert p["groups_per_xcd"] * p["members"] <= cus // xcds
            assert p["workgroups"] == xcds * p["groups_per_xcd"] * p["members"]
        else:
            assert p["workgroups"] == p["groups"] * p["members"]
        return
    assert 0 < p["lds_bytes"] <= LDS_MAX
    if p["kernel"] == 3:
        assert p["groups"] == math.ceil(s.B / p["rows"])
        assert p["hidden_per_wg"] * p["members"] >= s.belief_dim
        assert p["hidden_per_wg"] * (p["members"] - 1) < s.belief_dim
        assert 1 <= p["rows"] <= 4
    else:
        D = 2 if s.bidirectional else 1
        assert p["groups"] * p["rows"] >= s.B
        assert p["hidden_per_wg"] * p["members"] >= s.hidden_size
        assert p["rows"] * p["hidden_per_wg"] <= 1024
        if s.mode == "lstmp":
            assert p["proj_per_wg"] * p["members"] >= s.proj_size
        # a pipelined stack scans a chunk of every layer in one launch
        groups = D * p["groups"] * (s.num_layers if p["pipe_chunk"] else 1)
        if p["pipe_chunk"]:
            assert D == 1 and s.num_layers >= 2 and 1 <= p["pipe_chunk"] < s.T
        if p["groups_per_xcd"]:
            assert p["groups_per_xcd"] * xcds >= groups
            assert p["groups_per_xcd"] * p["members"] <= cus // xcds
            assert p["workgroups"] == xcds * p["groups_per_xcd"] * p["members"]
        else:
            assert p["workgroups"] == groups * p["members"]


@pytest.mark.parametrize("name", ["gru_t256_b256", "lstm_t80_b1", "rssm_b50_t50"])
def test_placement_hint(name):
    _, d, lengths = desc_for(name, placement=1)
    assert gss.rnn_plan_info(d, lengths)["groups_per_xcd"] == 0
    _, d, lengths = desc_for(name, placement=2)
    p = gss.rnn_plan_info(d, lengths)
    assert p["groups_per_xcd"] > 0
    assert p["groups_per_xcd"] * p["members"] <= 256 // 8


def test_single_xcd_device_never_aligns():
    _, d, lengths = desc_for("gru_t256_b256")
    assert gss.rnn_plan_info(d, lengths, cus=256, xcds=1)["groups_per_xcd"] == 0


def test_hints_are_honoured():
    _, d, lengths = desc_for("rssm_b50_t50", tile_batch=3, tile_hidden=14)
    p = gss.rnn_plan_info(d, lengths)
    assert (p["rows"], p["hidden_per_wg"], p["members"]) == (3, 14, 15)
    _, d, lengths = desc_for("gru_t256_b256", tile_batch=16, tile_hidden=32)
    p = gss.rnn_plan_info(d, lengths)
    assert (p["rows"], p["hidden_per_wg"]) == (16, 32)


def test_invalid_arguments():
    _, d, lengths = desc_for("gru_t256_b256")
    for cus, xcds in [(0, 1), (256, 0), (250, 8)]:
        with pytest.raises(gss.RnnError) as e:
            gss.rnn_plan_info(d, lengths, cus=cus, xcds=xcds)
        assert e.value.status == CODE["RNN_E_SHAPE"]
    _, d, lengths = desc_for("gru_t256_b256", placement=3)
    with pytest.raises(gss.RnnError) as e:
        gss.rnn_plan_info(d, lengths)
    assert e.value.status == CODE["RNN_E_SHAPE"]


@pytest.mark.parametrize("case", __import__("layout_cases").REG_CASES, ids=lambda c: c[0])
def test_forced_register_layouts(case):
    import numpy as np
    name, mode, dt, T, B, F, H, P, bb, hs, bidir, layout, varlen, expect = case
    d = gss.RnnDesc()
    d.mode = gss.MODES[mode]
    d.dtype = 1 if dt == "bf16" else 0
    d.layout = 1 if layout == "packed" else 0
    d.T, d.B, d.input_size, d.hidden_size, d.proj_size = T, B, F, H, P
    d.num_layers, d.bidirectional, d.has_bias = 1, int(bidir), 1
    d.tile_batch, d.tile_hidden = bb, hs
    d.weights = 2 if expect[0] else 1
    lengths = None
    if varlen:
        lengths = np.sort(np.random.default_rng(0).integers(varlen[0], varlen[1] + 1, size=B))[::-1]
        lengths = lengths.astype(np.int32)
    p = gss.rnn_plan_info(d, lengths)
    assert (p["rows"], p["hidden_per_wg"]) == (bb, hs)
    assert (p["wreg"], p["reg_tiles"], p["reg_ksplit"], p["reg_chunks"]) == expect


# one-wave scan (4) up to 16 units; above, the few-row scan (5) for up to 8
# (direction, row) groups and the tiled scan (2) for more rows or LSTMP
@pytest.mark.parametrize("mode,H,B,expect", [("lstm", 16, 5, 4), ("lstm", 17, 5, 5), ("gru", 16, 5, 4),
                                             ("gru", 17, 5, 5), ("lstm", 1, 5, 4), ("lstmp", 8, 5, 2),
                                             ("lstm", 17, 9, 2), ("gru", 512, 8, 5), ("gru", 513, 8, 2)])
def test_wave_scan_choice(mode, H, B, expect):
    d = gss.RnnDesc()
    d.mode, d.T, d.B, d.input_size, d.hidden_size, d.num_layers, d.has_bias = gss.MODES[mode], 8, B, 7, H, 1, 1
    if mode == "lstmp":
        d.proj_size = 4
    assert gss.rnn_plan_info(d)["kernel"] == expect
    if expect == 4:
        # a tiling hint asks for the tiled scan
        d.tile_batch = 1
        assert gss.rnn_plan_info(d)["kernel"] == 2


# Launch shapes that a sweep of the tiling hints measured fastest on MI355X
# (rows per group, hidden units per member): the cost model must keep
# choosing them.
MEASURED_BEST = {
    # (the few-row scan: one row per group; 8 units per member measured
    # 125 us per scan against 135 and 185 for 16 and 32)
    "lstm_t80_b1": (1, 8),
    "gru_t256_b256": (16, 32),
    "lstmp_t1000_b32": (16, 32),
    "bilstm_varlen_b64": (16, 16),
}


@pytest.mark.parametrize("name", list(MEASURED_BEST))
def test_plans_match_measured_best_shapes(name):
    _, d, lengths = desc_for(name)
    p = gss.rnn_plan_info(d, lengths)
    assert (p["rows"], p["hidden_per_wg"]) == MEASURED_BEST[name]


# The RSSM unroll's launch shapes on the register kernel, measured on MI355X
# (microseconds per unroll, one box): the shapes lie within a few percent of
# each other, so the planner's choice must be within 3% of the fastest.
RSSM_MEASURED_US = {(2, 40): 325.6, (3, 40): 329.1, (4, 40): 334.9, (2, 34): 321.6, (2, 29): 316.4,
                    (2, 25): 320.4, (4, 25): 328.7}


def test_rssm_plan_within_measured_best():
    _, d, lengths = desc_for("rssm_b50_t50")
    p = gss.rnn_plan_info(d, lengths)
    assert p["wreg"] == 1
    t = RSSM_MEASURED_US[(p["rows"], p["hidden_per_wg"])]
    assert t <= 1.03 * min(RSSM_MEASURED_US.values())


@pytest.mark.parametrize("mode,dtype,H,B,ok", [
    (0, 0, 1024, 1, True), (0, 0, 1024, 16, True), (1, 0, 1024, 16, True), (0, 1, 2048, 16, True),
    (0, 0, 1280, 1, False), (0, 0, 1280, 16, False), (1, 0, 1280, 16, False), (0, 1, 2560, 16, False),
])
def test_largest_hidden_sizes(mode, dtype, H, B, ok):
    """The largest recurrences that fit the persistent kernels on one device
    plan; one step beyond is RNN_E_PLAN before anything is launched."""
    d = gss.RnnDesc()
    d.mode, d.dtype, d.layout, d.T, d.B = mode, dtype, 0, 3, B
    d.input_size, d.hidden_size, d.proj_size = 64, H, 0
    d.num_layers, d.bidirectional, d.has_bias = 1, 0, 1
    if ok:
        p = gss.rnn_plan_info(d)
        assert p["hidden_per_wg"] * p["members"] >= H and p["workgroups"] <= 256
    else:
        with pytest.raises(gss.RnnError) as e:
            gss.rnn_plan_info(d)
        assert e.value.status == CODE["RNN_E_PLAN"]


def test_layer_pipeline_plans():
    """Which stacks the planner pipelines: the LSTMP stack (two layers of
    7 ms scans) by default; a short or one-layer stack never (one chunk);
    a bidirectional or packed stack never; "off" never; "on" whenever the
    stack qualifies and its launch fits."""
    _, d, _ = desc_for("lstmp_t1000_b32")
    p = gss.rnn_plan_info(d)
    assert p["pipe_chunk"] == 91 and p["workgroups"] == 256  # 11 chunks: sqrt(T / 8)
    d.layer_pipeline = gss.PIPE_MODES["off"]
    assert gss.rnn_plan_info(d)["pipe_chunk"] == 0
    _, d, lengths = desc_for("bilstm_varlen_b64")
    d.layer_pipeline = gss.PIPE_MODES["on"]
    assert gss.rnn_plan_info(d, lengths)["pipe_chunk"] == 0
    _, d, _ = desc_for("gru_t256_b256")
    d.layer_pipeline = gss.PIPE_MODES["on"]
    assert gss.rnn_plan_info(d)["pipe_chunk"] == 0  # one layer
    d.num_layers = 2
    p = gss.rnn_plan_info(d)
    assert p["pipe_chunk"] == 43  # 6 chunks
    assert p["workgroups"] == 2 * p["groups"] * p["members"] or p["groups_per_xcd"] > 0
    d.T = 32  # one chunk: nothing to overlap
    assert gss.rnn_plan_info(d)["pipe_chunk"] == 0
