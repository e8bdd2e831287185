"""rnn_forward_noalloc: the forward for callers that cannot allocate, whose
workspace is a device array the library owns. Called through the C ABI and
compared with rnn_forward (caller-owned workspace) on the same inputs: the
kernels and the launch plan are the same, so the outputs must agree bit for
bit. Each test makes two calls in a row, the second on a smaller problem,
so the second call runs on whatever the first left in the shared array."""

import ctypes

import numpy as np
import pytest
import torch

import synth
from gpu_util import log, run_rnn, run_rssm

pytestmark = pytest.mark.gpu

gss = pytest.importorskip("gru_sequence_scan_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert gss.rnn_device_check() == 0, "current device is not gfx950"
    torch.cuda.set_device(0)


def _same(a, b, what):
    if a is None:
        assert b is None
        return
    assert a.shape == b.shape, what
    assert np.array_equal(np.isnan(a), np.isnan(b)), what + ": NaN pattern differs"
    fin = ~np.isnan(a)
    assert np.array_equal(a[fin], b[fin]), what + ": values differ"


@pytest.mark.parametrize("mode,dt,P", [("lstm", "f32", 0), ("gru", "bf16", 0), ("lstmp", "f32", 16)])
def test_noalloc_matches_forward_two_calls(mode, dt, P):
    big = synth.make_rnn_inputs(mode, 15, 21, 19, 48, proj_size=P, num_layers=2, bidirectional=True, dtype=dt,
                                layout="packed", varlen=(1, 15), w_scale=0.2, seed=31, h0_std=0.3, c0_std=0.3)
    small = synth.make_rnn_inputs(mode, 6, 5, 19, 48, proj_size=P, num_layers=2, bidirectional=True, dtype=dt,
                                  layout="packed", varlen=(1, 6), w_scale=0.2, seed=32)
    for name, d in (("first call", big), ("second call, smaller", small)):
        log(f"[gpu] no-alloc {mode} {dt}: {name}")
        ref = run_rnn(d, y_fill=float("nan"))
        got = run_rnn(d, y_fill=float("nan"), noalloc=True)
        for g, r, nm in zip(got, ref, ("y", "h_n", "c_n")):
            _same(g, r, f"{mode} {name} {nm}")


def test_noalloc_rssm_two_calls():
    for name, d in (("first call", synth.make_inputs("rssm_b50_t50")),
                    ("second call, smaller", synth.make_rssm_inputs(6, 7, state_dim=5, action_dim=3, embed_dim=24,
                                                                    belief_dim=20, seed=33, s0_std=0.5,
                                                                    h0_std=0.5))):
        log(f"[gpu] no-alloc rssm: {name}")
        ref = run_rssm(d)
        got = run_rssm(d, noalloc=True)
        for g, r, nm in zip(got, ref, ("means", "stds", "states", "beliefs")):
            _same(g, r, f"rssm {name} {nm}")


def test_noalloc_rejects_a_workspace_beyond_the_array():
    """A problem whose workspace exceeds the array is refused before anything
    is enqueued, and the array size is what the header states."""
    d = gss.RnnDesc()
    for k, v in dict(mode=1, dtype=0, layout=0, T=256, B=256, input_size=512, hidden_size=512, num_layers=1,
                     has_bias=1).items():
        setattr(d, k, v)
    assert gss.rnn_workspace_bytes(d) > gss.binding.RNN_NOALLOC_MAX_WORKSPACE
    st = gss.lib().rnn_forward_noalloc(ctypes.byref(d), ctypes.byref(gss.RnnWeights()), ctypes.byref(gss.RnnIO()),
                                       None, None)
    assert st == -5  # RNN_E_WORKSPACE
    header = open(gss.lib_path().replace("gru_sequence_scan_amd/_lib/librnn_gfx950.so", "include/rnn.h")).read()
    assert "#define RNN_NOALLOC_MAX_WORKSPACE (32u << 20)" in header
    assert gss.binding.RNN_NOALLOC_MAX_WORKSPACE == 32 << 20
