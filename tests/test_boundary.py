"""The C ABI boundary, on the CPU: the library loads, exports what the header
declares, the ctypes mirrors match the C structs, and invalid arguments get
the documented status codes before anything touches a device."""

import ctypes
import os
import re
import subprocess
import threading

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rnn.h")

gss = pytest.importorskip("gru_sequence_scan_amd")

OK, E_NULL, E_SHAPE, E_UNSUPPORTED, E_LENGTHS, E_WORKSPACE, E_ALIGN, E_DEVICE = 0, -1, -2, -3, -4, -5, -6, -7


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gss.lib_path()):
        pytest.fail("native library not built: run python -m gru_sequence_scan_amd.build")
    return gss.lib()


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(rnn_\w+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert set(names) >= {"rnn_forward", "rnn_workspace_bytes", "rnn_strerror", "rnn_abi_version",
                          "rnn_read_status", "rnn_device_check"}
    for n in names:
        assert hasattr(lib, n), f"{n} declared in rnn.h but not exported"


def test_abi_version_and_strerror(lib):
    assert gss.rnn_abi_version() == gss.RNN_ABI_VERSION == 2
    for code in range(-10, 1):
        s = gss.rnn_strerror(code)
        assert isinstance(s, str) and s
    assert gss.rnn_strerror(-99) == "unknown status"


def test_ctypes_layout_matches_c(tmp_path):
    # Compile a tiny C program against the header and compare sizes/offsets.
    c = tmp_path / "layout.c"
    c.write_text(r'''
#include <stdio.h>
#include <stddef.h>
#include "rnn.h"
int main(void) {
  printf("%zu %zu %zu\n", sizeof(RnnDesc), sizeof(RnnWeights), sizeof(RnnIO));
  printf("%zu %zu %zu %zu\n", offsetof(RnnDesc, scale_lb), offsetof(RnnDesc, tile_batch),
         offsetof(RnnWeights, w_as), offsetof(RnnIO, beliefs));
  printf("%zu %zu %zu %d %d\n", offsetof(RnnDesc, clip), offsetof(RnnDesc, proj_clip),
         offsetof(RnnDesc, reserved), RNN_CLIP_CELL, RNN_CLIP_PROJ);
  printf("%zu %zu %zu %d\n", offsetof(RnnDesc, actor_dim), offsetof(RnnWeights, w_a1),
         offsetof(RnnIO, actions), (int)RNN_MODE_RSSM_ACTOR);
  return 0;
}
''')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(c), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()
    sizes = [int(v) for v in out]
    assert sizes[0] == ctypes.sizeof(gss.RnnDesc)
    assert sizes[1] == ctypes.sizeof(gss.RnnWeights)
    assert sizes[2] == ctypes.sizeof(gss.RnnIO)
    assert sizes[3] == gss.RnnDesc.scale_lb.offset
    assert sizes[4] == gss.RnnDesc.tile_batch.offset
    assert sizes[5] == gss.RnnWeights.w_as.offset
    assert sizes[6] == gss.RnnIO.beliefs.offset
    assert sizes[7] == gss.RnnDesc.clip.offset
    assert sizes[8] == gss.RnnDesc.proj_clip.offset
    assert sizes[9] == gss.RnnDesc.reserved.offset
    assert (sizes[10], sizes[11]) == (gss.CLIP_CELL, gss.CLIP_PROJ)
    assert sizes[12] == gss.RnnDesc.actor_dim.offset
    assert sizes[13] == gss.RnnWeights.w_a1.offset
    assert sizes[14] == gss.RnnIO.actions.offset
    assert sizes[15] == gss.MODES["rssm_actor"]


def _desc(**kw):
    d = gss.RnnDesc()
    base = dict(mode=0, dtype=0, layout=0, T=8, B=4, input_size=16, hidden_size=32, proj_size=0,
                num_layers=1, bidirectional=0, has_bias=1)
    base.update(kw)
    for k, v in base.items():
        setattr(d, k, v)
    return d


def _ws(desc, lengths=None):
    keep, lp = gss.binding._len_ptr(lengths, desc.B if desc is not None else 0)
    n = ctypes.c_size_t(0)
    return gss.lib().rnn_workspace_bytes(ctypes.byref(desc) if desc is not None else None, lp, ctypes.byref(n)), n.value


@pytest.mark.parametrize("kw,lengths,expect", [
    ({}, None, OK),
    ({"mode": 1}, None, OK),
    ({"mode": 2, "proj_size": 8}, None, OK),
    ({"mode": 1, "proj_size": 8}, None, E_UNSUPPORTED),      # projection is LSTM-only
    ({"mode": 0, "proj_size": 8}, None, E_UNSUPPORTED),
    ({"mode": 2, "proj_size": 0}, None, E_UNSUPPORTED),
    ({"mode": 7}, None, E_UNSUPPORTED),
    ({"dtype": 5}, None, E_UNSUPPORTED),
    ({"T": 0}, None, E_SHAPE),
    ({"B": 0}, None, E_SHAPE),
    ({"hidden_size": 0}, None, E_SHAPE),
    ({"num_layers": 9}, None, E_SHAPE),
    ({"bidirectional": 2}, None, E_SHAPE),
    ({"layout": 1}, None, E_LENGTHS),                       # packed needs lengths
    ({"layout": 1}, [8, 7, 7, 1], OK),
    ({"layout": 1}, [7, 8, 7, 1], E_LENGTHS),               # packed needs sorted lengths
    ({"layout": 0}, [7, 8, 7, 1], OK),                      # padded may be unsorted
    ({"layout": 0}, [0, 8, 7, 1], E_LENGTHS),
    ({"layout": 0}, [9, 8, 7, 1], E_LENGTHS),
    ({"layout": 2}, None, E_UNSUPPORTED),
    ({"mode": 3, "layout": 2, "state_dim": 20, "action_dim": 6, "embed_dim": 200, "belief_dim": 200,
      "scale_lb": 0.1}, None, OK),
    ({"mode": 3, "layout": 2, "dtype": 1, "state_dim": 20, "action_dim": 6, "embed_dim": 200,
      "belief_dim": 200}, None, E_UNSUPPORTED),
    ({"mode": 3, "layout": 2, "bidirectional": 1, "state_dim": 20, "action_dim": 6, "embed_dim": 200,
      "belief_dim": 200}, None, E_UNSUPPORTED),
    ({"mode": 3, "layout": 0, "state_dim": 20, "action_dim": 6, "embed_dim": 200, "belief_dim": 200},
     None, E_UNSUPPORTED),
])
def test_workspace_validation(lib, kw, lengths, expect):
    st, n = _ws(_desc(**kw), lengths)
    assert st == expect, gss.rnn_strerror(st)
    if st == OK:
        assert n > 0


INF, NAN = float("inf"), float("nan")


@pytest.mark.parametrize("kw,expect", [
    ({"clip": 1, "cell_clip_lo": -1.0, "cell_clip_hi": 1.0}, OK),
    ({"clip": 1, "cell_clip_lo": -INF, "cell_clip_hi": 0.5}, OK),
    ({"clip": 1, "cell_clip_lo": 0.25, "cell_clip_hi": 0.25}, OK),
    ({"mode": 2, "proj_size": 8, "clip": 3, "cell_clip_lo": -2.0, "cell_clip_hi": 2.0, "proj_clip": 0.5}, OK),
    ({"mode": 2, "proj_size": 8, "clip": 2, "proj_clip": INF}, OK),
    ({"clip": 1, "cell_clip_lo": 1.0, "cell_clip_hi": -1.0}, E_SHAPE),    # lo > hi
    ({"clip": 1, "cell_clip_lo": NAN, "cell_clip_hi": 1.0}, E_SHAPE),
    ({"mode": 2, "proj_size": 8, "clip": 2, "proj_clip": -0.5}, E_SHAPE),
    ({"mode": 2, "proj_size": 8, "clip": 2, "proj_clip": NAN}, E_SHAPE),
    ({"mode": 1, "clip": 1, "cell_clip_lo": -1.0, "cell_clip_hi": 1.0}, E_UNSUPPORTED),  # GRU has no cell
    ({"clip": 2, "proj_clip": 1.0}, E_UNSUPPORTED),                                     # LSTM has no projection
    ({"clip": 4}, E_UNSUPPORTED),
    ({"mode": 3, "layout": 2, "state_dim": 20, "action_dim": 6, "embed_dim": 200, "belief_dim": 200,
      "clip": 1, "cell_clip_lo": -1.0, "cell_clip_hi": 1.0}, E_UNSUPPORTED),
    ({"clip": 0, "cell_clip_lo": NAN, "proj_clip": NAN}, OK),                          # ignored when off
])
def test_clip_validation(lib, kw, expect):
    st, _ = _ws(_desc(**kw))
    assert st == expect, gss.rnn_strerror(st)


RSSM_KW = {"layout": 2, "state_dim": 20, "action_dim": 6, "embed_dim": 200, "belief_dim": 200}


@pytest.mark.parametrize("kw,expect", [
    ({"mode": 4, "actor_dim": 200}, OK),
    ({"mode": 4, "actor_dim": 1}, OK),
    ({"mode": 4, "actor_dim": 0}, E_SHAPE),             # the actor needs a width
    ({"mode": 4, "actor_dim": -3}, E_SHAPE),
    ({"mode": 3, "actor_dim": 16}, E_SHAPE),            # only the actor mode has one
    ({"mode": 0, "actor_dim": 16, "layout": 0}, E_SHAPE),
    ({"mode": 4, "actor_dim": 8, "bidirectional": 1}, E_UNSUPPORTED),
    ({"mode": 4, "actor_dim": 8, "dtype": 1}, E_UNSUPPORTED),
    ({"mode": 4, "actor_dim": 8, "layout": 0}, E_UNSUPPORTED),
])
def test_actor_mode_validation(lib, kw, expect):
    base = dict(RSSM_KW)
    base.update(kw)
    st, n = _ws(_desc(**base))
    assert st == expect, gss.rnn_strerror(st)


def test_actor_exchange_is_larger(lib):
    st0, n0 = _ws(_desc(mode=3, **RSSM_KW))
    st1, n1 = _ws(_desc(mode=4, actor_dim=200, **RSSM_KW))
    assert st0 == st1 == OK and n1 > n0


def test_reserved_fields_must_be_zero(lib):
    for i in range(1):
        d = _desc()
        d.reserved[i] = 1
        assert _ws(d)[0] == E_SHAPE


def test_gx_dtype_values(lib):
    """G_x storage: 0 follows the storage dtype, 1 forces fp32; anything else
    is a shape error, and the RSSM modes (no hoisted product) reject it."""
    d = _desc()
    d.gx_dtype = 2
    assert _ws(d)[0] == E_SHAPE
    d = _desc(mode=3, **RSSM_KW)
    d.gx_dtype = 1
    assert _ws(d)[0] == E_UNSUPPORTED


def test_layer_pipeline_values(lib):
    """The layer-pipelining hint takes 0 (auto), 1 (off) and 2 (on); other
    values are a shape error and the RSSM modes take only 0. Pipelining adds
    per-layer chunk buffers to the workspace of a qualifying stack (two
    layers, padded, unidirectional, T > 32) and nothing to one that does not
    qualify (bidirectional)."""
    kw = dict(mode=2, dtype=1, T=100, B=8, input_size=16, hidden_size=32, num_layers=2, proj_size=8)
    sizes = {}
    for v in (0, 1, 2):
        d = _desc(**kw)
        d.layer_pipeline = v
        st, sizes[v] = _ws(d)
        assert st == OK
    assert sizes[0] == sizes[2] > sizes[1]
    for v in (-1, 3):
        d = _desc(**kw)
        d.layer_pipeline = v
        assert _ws(d)[0] == E_SHAPE
    d = _desc(**dict(kw, bidirectional=1))
    n_auto = _ws(d)[1]
    d.layer_pipeline = 1
    assert _ws(d)[1] == n_auto
    d = _desc(mode=3, **RSSM_KW)
    d.layer_pipeline = 2
    assert _ws(d)[0] == E_UNSUPPORTED


def test_bf16_gx_halves_the_gate_buffer(lib):
    """bf16 storage keeps G_x in bf16 unless fp32 is requested: the workspace
    shrinks by half the G_x buffer (rows * D * G * 2 bytes, give or take the
    256-byte section alignment). (B = 16 runs the tiled scan; the few-row
    scan reads fp32 G_x whatever the storage dtype.)"""
    kw = dict(mode=1, dtype=1, T=20, B=16, input_size=16, hidden_size=32)
    st0, n_bf = _ws(_desc(**kw))
    d = _desc(**kw)
    d.gx_dtype = 1
    st1, n_f32 = _ws(d)
    assert st0 == st1 == OK
    half = 20 * 16 * 3 * 32 * 2
    assert abs((n_f32 - n_bf) - half) <= 256


def test_null_desc(lib):
    assert _ws(None)[0] == E_NULL


def test_workspace_covers_gate_buffer(lib):
    # padded LSTM T=8 B=4 H=32: Gx alone is 8*4*128 floats
    st, n = _ws(_desc())
    assert st == OK and n >= 8 * 4 * 128 * 4
    st2, n2 = _ws(_desc(bidirectional=1, num_layers=3))
    assert st2 == OK and n2 > 2 * n


def test_forward_without_gpu_reports_device(lib):
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    d = _desc()
    w = gss.RnnWeights()
    for i in range(1):
        w.w_ih[i] = w.w_hh[i] = w.b_ih[i] = w.b_hh[i] = 4096
    io = gss.RnnIO()
    io.x = io.y = 4096
    st = gss.rnn_forward_raw(d, w, io, 4096, 1 << 20, 0)
    assert st == E_DEVICE
    assert gss.rnn_device_check() == E_DEVICE


def test_forward_validates_before_device(lib):
    d = _desc(mode=1, proj_size=4)
    st = gss.rnn_forward_raw(d, gss.RnnWeights(), gss.RnnIO(), 0, 0, 0)
    assert st == E_UNSUPPORTED
    d = _desc(layout=1)
    io = gss.RnnIO()
    assert gss.rnn_forward_raw(d, gss.RnnWeights(), io, 0, 0, 0) == E_LENGTHS


def test_concurrent_calls_are_independent(lib):
    # No global mutable state: threads computing workspace sizes for
    # different problems never see each other's values.
    results = {}

    def work(i):
        out = []
        for _ in range(200):
            out.append(_ws(_desc(hidden_size=16 * (i + 1), T=3 + i))[1])
        results[i] = out

    ts = [threading.Thread(target=work, args=(i,)) for i in range(6)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    for i in range(6):
        assert len(set(results[i])) == 1
        assert results[i][0] == _ws(_desc(hidden_size=16 * (i + 1), T=3 + i))[1]


def test_binding_rematerialises_non_canonical_strides():
    from gru_sequence_scan_amd.binding import _c_dense, _dense
    base = torch.arange(20.0).reshape(1, 4, 5)
    odd = base.as_strided((1, 4, 5), (5, 5, 1))       # passes is_contiguous, strides off-canonical
    assert odd.is_contiguous() and _c_dense(odd) and _dense(odd) is odd
    t = torch.arange(40.0).reshape(4, 10)[:, ::2]      # really strided memory
    assert not _c_dense(t)
    r = _dense(t)
    assert _c_dense(r) and torch.equal(r, t)
    tt = torch.arange(12.0).reshape(3, 4).t()          # transposed
    assert not _c_dense(tt) and torch.equal(_dense(tt), tt)


@pytest.mark.parametrize("kw,expect", [
    ({}, OK),
    ({"mode": 1}, OK),
    ({"mode": 2, "proj_size": 8}, OK),
    ({"mode": 0, "bidirectional": 1, "num_layers": 3}, OK),
    ({"dtype": 1}, E_UNSUPPORTED),                                            # training is fp32
    ({"clip": 1, "cell_clip_lo": -1.0, "cell_clip_hi": 1.0}, E_UNSUPPORTED),  # no clipped backward
    ({"mode": 3, "layout": 2, "state_dim": 20, "action_dim": 6, "embed_dim": 200, "belief_dim": 200},
     E_UNSUPPORTED),
])
def test_training_sizes_validation(lib, kw, expect):
    d = _desc(**kw)
    for fn in ("rnn_reserve_bytes", "rnn_backward_workspace_bytes"):
        n = ctypes.c_size_t(0)
        st = getattr(lib, fn)(ctypes.byref(d), None, ctypes.byref(n))
        assert st == expect, (fn, gss.rnn_strerror(st))
        if st == OK:
            assert n.value > 0


def test_reserve_holds_gates_and_inner_layer_outputs(lib):
    # LSTM T=8 B=4 H=32 one layer: 5H fp32 gate values per token
    n1 = ctypes.c_size_t(0)
    assert lib.rnn_reserve_bytes(ctypes.byref(_desc()), None, ctypes.byref(n1)) == OK
    assert n1.value >= 8 * 4 * 5 * 32 * 4
    n2 = ctypes.c_size_t(0)
    assert lib.rnn_reserve_bytes(ctypes.byref(_desc(num_layers=2)), None, ctypes.byref(n2)) == OK
    assert n2.value >= 2 * n1.value + 8 * 4 * 32 * 4   # the lower layer's output is kept too


@pytest.mark.parametrize("n", [3, 5])
def test_lengths_count_must_match_batch(lib, n):
    """The C side reads exactly B lengths; a shorter or longer host list is
    refused before any call (a short list would be read past its end)."""
    d = _desc(B=4)
    with pytest.raises(ValueError, match="lengths"):
        gss.rnn_workspace_bytes(d, [2] * n)
    with pytest.raises(ValueError, match="lengths"):
        gss.rnn_plan_info(d, [2] * n)
    assert gss.rnn_workspace_bytes(d, [2] * 4) > 0


@pytest.mark.parametrize("n", [3, 5])
def test_lengths_count_checked_by_forward(lib, n):
    """rnn_forward refuses a length list whose size is not the batch size,
    for the padded layout too, before touching a device."""
    import torch
    x = torch.zeros(6, 4, 8)
    params = [{"w_ih": torch.zeros(64, 8), "w_hh": torch.zeros(64, 16)}]
    with pytest.raises(ValueError, match="lengths"):
        gss.rnn_forward("lstm", x, params, lengths=[2] * n)
