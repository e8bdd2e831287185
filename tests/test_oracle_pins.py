"""Pins of the float64 oracle to things other than itself.

Each check is chosen so that a plausible slip in the oracle (a swapped gate
chunk, the GRU reset gate outside or inside the wrong term, a dropped bias, a
wrong reverse start, a transposed weight) fails at least one of them:
closed forms, invariants, brute force on tiny inputs, and library special
cases (PyTorch's CPU modules in float64, which implement the gate
conventions the oracle follows).
"""

import math

import numpy as np
import pytest
import torch

import oracle
import synth

torch.set_default_dtype(torch.float64)

TIGHT = dict(rtol=1e-11, atol=1e-12)


def _rand_case(mode, T=7, B=5, F=6, H=4, P=0, L=1, bidir=False, bias=True, lengths=None,
               seed=0, h0=True):
    d = synth.make_rnn_inputs(mode, T, B, F, H, proj_size=P, num_layers=L, bidirectional=bidir,
                              lengths=lengths, w_scale=0.6, bias=bias, seed=seed,
                              h0_std=0.5 if h0 else 0.0, c0_std=0.5 if h0 else 0.0)
    return d


def _torch_rnn(mode, d):
    D = 2 if d["bidirectional"] else 1
    H = d["hidden_size"]
    bias = d["params"][0]["b_ih"] is not None
    if mode == "gru":
        m = torch.nn.GRU(d["input_size"], H, num_layers=d["num_layers"], bias=bias,
                         bidirectional=d["bidirectional"])
    else:
        m = torch.nn.LSTM(d["input_size"], H, num_layers=d["num_layers"], bias=bias,
                          bidirectional=d["bidirectional"], proj_size=d["proj_size"])
    sd = {}
    for layer in range(d["num_layers"]):
        for di in range(D):
            p = d["params"][layer * D + di]
            sfx = f"_l{layer}" + ("_reverse" if di == 1 else "")
            sd["weight_ih" + sfx] = torch.tensor(p["w_ih"], dtype=torch.float64)
            sd["weight_hh" + sfx] = torch.tensor(p["w_hh"], dtype=torch.float64)
            if bias:
                sd["bias_ih" + sfx] = torch.tensor(p["b_ih"], dtype=torch.float64)
                sd["bias_hh" + sfx] = torch.tensor(p["b_hh"], dtype=torch.float64)
            if mode == "lstmp":
                sd["weight_hr" + sfx] = torch.tensor(p["w_hr"], dtype=torch.float64)
    m.load_state_dict(sd)
    return m.double()


def _torch_run(mode, d):
    m = _torch_rnn(mode, d)
    K = d["proj_size"] if mode == "lstmp" else d["hidden_size"]
    D = 2 if d["bidirectional"] else 1
    LD = d["num_layers"] * D
    B = d["B"]
    h0 = torch.zeros(LD, B, K) if d["h0"] is None else torch.tensor(d["h0"], dtype=torch.float64)
    x = torch.tensor(np.nan_to_num(d["x_padded"]), dtype=torch.float64)
    lengths = d["lengths"]
    if lengths is not None:
        x = torch.nn.utils.rnn.pack_padded_sequence(x, torch.tensor(lengths, dtype=torch.int64),
                                                    enforce_sorted=False)
    with torch.no_grad():
        if mode == "gru":
            y, hn = m(x, h0)
            cn = None
        else:
            c0 = (torch.zeros(LD, B, d["hidden_size"]) if d["c0"] is None
                  else torch.tensor(d["c0"], dtype=torch.float64))
            y, (hn, cn) = m(x, (h0, c0))
    if lengths is not None:
        y, _ = torch.nn.utils.rnn.pad_packed_sequence(y, total_length=d["T"])
    return y.numpy(), hn.numpy(), None if cn is None else cn.numpy()


def _oracle_run(mode, d, **kw):
    return oracle.rnn_forward(mode, d["x"], d["params"], lengths=d["lengths"], h0=d["h0"],
                              c0=d["c0"], num_layers=d["num_layers"],
                              bidirectional=d["bidirectional"], proj_size=d["proj_size"],
                              layout=d["layout"], **kw)


def _compare_padded(y_or, y_t, lengths):
    """Oracle leaves unwritten positions NaN; torch's unpack writes zeros there."""
    if lengths is None:
        np.testing.assert_allclose(y_or, y_t, **TIGHT)
        return
    T = y_or.shape[0]
    for b, Lb in enumerate(lengths):
        np.testing.assert_allclose(y_or[:Lb, b], y_t[:Lb, b], **TIGHT)
        assert np.isnan(y_or[Lb:T, b]).all()


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------

def test_lstm_zero_weights_closed_form():
    # All weights and biases zero: i = f = o = 1/2 and g = 0, so c_t = 2^-t c0
    # and h_t = tanh(c_t) / 2 whatever h0 and x are.
    T, B, F, H = 6, 3, 5, 4
    d = _rand_case("lstm", T=T, B=B, F=F, H=H, seed=1)
    for p in d["params"]:
        for k in p:
            p[k] = np.zeros_like(p[k])
    y, hn, cn = _oracle_run("lstm", d)
    c0 = d["c0"][0].astype(np.float64)
    for t in range(T):
        ct = c0 * 2.0 ** -(t + 1)
        np.testing.assert_allclose(y[t], 0.5 * np.tanh(ct), **TIGHT)
    np.testing.assert_allclose(cn[0], c0 * 2.0 ** -T, **TIGHT)


def test_gru_zero_weights_closed_form():
    # r = z = 1/2 and n = tanh(0) = 0, so h_t = 2^-t h0.
    T = 9
    d = _rand_case("gru", T=T, seed=2)
    for p in d["params"]:
        for k in p:
            p[k] = np.zeros_like(p[k])
    y, hn, _ = _oracle_run("gru", d)
    h0 = d["h0"][0].astype(np.float64)
    for t in range(T):
        np.testing.assert_allclose(y[t], h0 * 2.0 ** -(t + 1), **TIGHT)


@pytest.mark.parametrize("beta", [0.375, -1.75, 2.5])
def test_gru_reset_gate_wraps_hidden_bias(beta):
    # W = 0, every bias 0 except b_hn = beta, h0 = 0: r = z = 1/2, so
    # h_1 = (1 - 1/2) tanh(r * beta) = tanh(beta / 2) / 2. Were b_hn outside
    # the reset product the value would be tanh(beta) / 2.
    H = 3
    d = _rand_case("gru", T=1, B=2, H=H, seed=3, h0=False)
    p = d["params"][0]
    for k in p:
        p[k] = np.zeros_like(p[k])
    p["b_hh"][2 * H:] = beta
    y, _, _ = _oracle_run("gru", d)
    np.testing.assert_allclose(y[0], np.full((2, H), 0.5 * math.tanh(beta / 2)), **TIGHT)


def test_lstm_scalar_brute_force():
    # H = 1, F = 1 with distinct hand-set gate weights: one step by hand.
    wi = np.array([[0.5], [-0.25], [1.5], [0.75]])
    wh = np.array([[0.1], [0.2], [-0.3], [0.4]])
    bi = np.array([0.01, 0.02, 0.03, 0.04])
    bh = np.array([-0.05, 0.06, -0.07, 0.08])
    x, h, c = 0.8, -0.6, 0.9
    pre = wi[:, 0] * x + wh[:, 0] * h + bi + bh
    s = lambda v: 1.0 / (1.0 + math.exp(-v))
    c1 = s(pre[1]) * c + s(pre[0]) * math.tanh(pre[2])
    h1 = s(pre[3]) * math.tanh(c1)
    hh, cc = oracle.lstm_cell(np.array([[x]]), np.array([[h]]), np.array([[c]]), wi, wh, bi, bh)
    assert abs(hh[0, 0] - h1) < 1e-14 and abs(cc[0, 0] - c1) < 1e-14


def test_gru_scalar_brute_force():
    wi = np.array([[0.5], [-0.25], [1.5]])
    wh = np.array([[0.1], [0.2], [-0.3]])
    bi = np.array([0.01, 0.02, 0.03])
    bh = np.array([-0.05, 0.06, -0.07])
    x, h = 0.8, -0.6
    s = lambda v: 1.0 / (1.0 + math.exp(-v))
    r = s(wi[0, 0] * x + bi[0] + wh[0, 0] * h + bh[0])
    z = s(wi[1, 0] * x + bi[1] + wh[1, 0] * h + bh[1])
    n = math.tanh(wi[2, 0] * x + bi[2] + r * (wh[2, 0] * h + bh[2]))
    h1 = (1 - z) * n + z * h
    got = oracle.gru_cell(np.array([[x]]), np.array([[h]]), wi, wh, bi, bh)
    assert abs(got[0, 0] - h1) < 1e-14


def test_activation_functions_against_library():
    x = np.linspace(-40, 40, 2001)
    tx = torch.tensor(x)
    np.testing.assert_allclose(oracle.sigmoid(x), torch.sigmoid(tx).numpy(), rtol=1e-14, atol=0)
    np.testing.assert_allclose(oracle.elu(x), torch.nn.functional.elu(tx).numpy(), rtol=1e-14, atol=1e-300)
    # PyTorch's softplus switches to the identity above 20; the exact value
    # differs there by log1p(exp(-x)) < 2.1e-9.
    np.testing.assert_allclose(oracle.softplus(x), torch.nn.functional.softplus(tx).numpy(),
                               rtol=0, atol=2.1e-9)
    np.testing.assert_allclose(oracle.softplus(x[x < 20]), np.log1p(np.exp(x[x < 20])), rtol=1e-14)


# ---------------------------------------------------------------------------
# Library special cases: PyTorch CPU modules in float64
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bias", [True, False])
def test_lstm_cell_matches_torch_lstmcell(bias):
    d = _rand_case("lstm", T=1, B=5, F=7, H=6, bias=bias, seed=4)
    p = d["params"][0]
    cell = torch.nn.LSTMCell(7, 6, bias=bias).double()
    with torch.no_grad():
        cell.weight_ih.copy_(torch.tensor(p["w_ih"]))
        cell.weight_hh.copy_(torch.tensor(p["w_hh"]))
        if bias:
            cell.bias_ih.copy_(torch.tensor(p["b_ih"]))
            cell.bias_hh.copy_(torch.tensor(p["b_hh"]))
        ht, ct = cell(torch.tensor(d["x"][0], dtype=torch.float64),
                      (torch.tensor(d["h0"][0], dtype=torch.float64),
                       torch.tensor(d["c0"][0], dtype=torch.float64)))
    h, c = oracle.lstm_cell(d["x"][0], d["h0"][0], d["c0"][0], p["w_ih"], p["w_hh"],
                            p["b_ih"], p["b_hh"])
    np.testing.assert_allclose(h, ht.numpy(), **TIGHT)
    np.testing.assert_allclose(c, ct.numpy(), **TIGHT)
    # T = 1 through the sequence entry point equals one cell call.
    y, hn, cn = _oracle_run("lstm", d)
    np.testing.assert_allclose(y[0], ht.numpy(), **TIGHT)
    np.testing.assert_allclose(cn[0], ct.numpy(), **TIGHT)


@pytest.mark.parametrize("bias", [True, False])
def test_gru_cell_matches_torch_grucell(bias):
    d = _rand_case("gru", T=1, B=5, F=7, H=6, bias=bias, seed=5)
    p = d["params"][0]
    cell = torch.nn.GRUCell(7, 6, bias=bias).double()
    with torch.no_grad():
        cell.weight_ih.copy_(torch.tensor(p["w_ih"]))
        cell.weight_hh.copy_(torch.tensor(p["w_hh"]))
        if bias:
            cell.bias_ih.copy_(torch.tensor(p["b_ih"]))
            cell.bias_hh.copy_(torch.tensor(p["b_hh"]))
        ht = cell(torch.tensor(d["x"][0], dtype=torch.float64),
                  torch.tensor(d["h0"][0], dtype=torch.float64))
    y, hn, _ = _oracle_run("gru", d)
    np.testing.assert_allclose(y[0], ht.numpy(), **TIGHT)
    np.testing.assert_allclose(hn[0], ht.numpy(), **TIGHT)


CASES = [
    # mode, L, bidir, P, bias, varlen
    ("lstm", 1, False, 0, True, False),
    ("lstm", 2, True, 0, True, False),
    ("lstm", 2, True, 0, False, True),
    ("lstm", 1, True, 0, True, True),
    ("gru", 1, False, 0, True, False),
    ("gru", 2, True, 0, True, True),
    ("gru", 1, False, 0, False, False),
    ("lstmp", 1, False, 3, True, False),
    ("lstmp", 2, False, 3, True, False),
    ("lstmp", 2, True, 2, False, True),
]


@pytest.mark.parametrize("mode,L,bidir,P,bias,varlen", CASES)
def test_sequence_matches_torch_modules(mode, L, bidir, P, bias, varlen):
    B, T = 5, 8
    lengths = np.array([8, 3, 6, 1, 5], dtype=np.int32) if varlen else None
    d = _rand_case(mode, T=T, B=B, F=6, H=4, P=P, L=L, bidir=bidir, bias=bias,
                   lengths=lengths, seed=10 + L + 3 * bidir + P)
    y_t, hn_t, cn_t = _torch_run(mode, d)
    y, hn, cn = _oracle_run(mode, d)
    _compare_padded(y, y_t, lengths)
    np.testing.assert_allclose(hn, hn_t, **TIGHT)
    if cn_t is not None:
        np.testing.assert_allclose(cn, cn_t, **TIGHT)


def test_packed_layout_matches_torch_packing():
    lengths = np.array([7, 7, 5, 2, 1], dtype=np.int32)
    d = synth.make_rnn_inputs("lstm", 7, 5, 3, 4, layout="packed", lengths=lengths, seed=6)
    packed_t = torch.nn.utils.rnn.pack_padded_sequence(
        torch.tensor(np.nan_to_num(d["x_padded"])), torch.tensor(lengths, dtype=torch.int64))
    np.testing.assert_array_equal(oracle.pack_sequence(d["x_padded"], lengths), packed_t.data.numpy())
    np.testing.assert_array_equal(d["x"], packed_t.data.numpy())
    bs, off = oracle.packed_offsets(lengths)
    np.testing.assert_array_equal(bs, packed_t.batch_sizes.numpy())
    back = oracle.unpack_sequence(d["x"], lengths, 7)
    np.testing.assert_array_equal(np.isnan(back), np.isnan(d["x_padded"]))
    np.testing.assert_array_equal(np.nan_to_num(back), np.nan_to_num(d["x_padded"]))


def test_oracle_rejects_projection_outside_lstm():
    d = _rand_case("gru", T=2, seed=7)
    with pytest.raises(ValueError):
        oracle.rnn_forward("gru", d["x"], d["params"], proj_size=3)
    with pytest.raises(ValueError):
        oracle.rnn_forward("lstmp", d["x"], d["params"], proj_size=0)


# ---------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------

def test_lstmp_identity_projection_reduces_to_lstm():
    d = _rand_case("lstmp", T=6, B=3, F=5, H=4, P=4, seed=8)
    d["params"][0]["w_hr"] = np.eye(4, dtype=np.float32)
    y_p, hn_p, cn_p = _oracle_run("lstmp", d)
    d2 = dict(d, proj_size=0)
    d2["params"] = [{k: v for k, v in d["params"][0].items() if k != "w_hr"}]
    y, hn, cn = _oracle_run("lstm", d2)
    np.testing.assert_allclose(y_p, y, **TIGHT)
    np.testing.assert_allclose(cn_p, cn, **TIGHT)


def test_lstmp_zero_projection_gives_zero_output():
    d = _rand_case("lstmp", T=5, B=3, F=5, H=4, P=2, seed=9, h0=False)
    d["params"][0]["w_hr"] = np.zeros_like(d["params"][0]["w_hr"])
    y, hn, cn = _oracle_run("lstmp", d)
    assert np.all(y == 0) and np.all(hn == 0)
    # Gates then depend on x only: c follows the zero-state recursion on x.
    p = d["params"][0]
    c = np.zeros((3, 4))
    for t in range(5):
        _, c = oracle.lstm_cell(d["x"][t], np.zeros((3, 2)), c, p["w_ih"], p["w_hh"], p["b_ih"], p["b_hh"])
    np.testing.assert_allclose(cn[0], c, **TIGHT)


@pytest.mark.parametrize("mode,P", [("lstm", 0), ("gru", 0), ("lstmp", 3)])
def test_time_chunking_equals_one_run(mode, P):
    d = _rand_case(mode, T=9, B=4, F=5, H=4, P=P, L=2, seed=11)
    y, hn, cn = _oracle_run(mode, d)
    d1 = dict(d, x=d["x"][:4], x_padded=d["x"][:4], T=4)
    y1, hn1, cn1 = _oracle_run(mode, d1)
    d2 = dict(d, x=d["x"][4:], x_padded=d["x"][4:], T=5, h0=hn1, c0=cn1)
    y2, hn2, cn2 = _oracle_run(mode, d2)
    np.testing.assert_allclose(np.concatenate([y1, y2]), y, **TIGHT)
    np.testing.assert_allclose(hn2, hn, **TIGHT)
    if cn is not None:
        np.testing.assert_allclose(cn2, cn, **TIGHT)


@pytest.mark.parametrize("mode,P", [("lstm", 0), ("gru", 0), ("lstmp", 2)])
def test_varlen_rows_equal_single_sequence_runs(mode, P):
    lengths = np.array([6, 6, 4, 2, 1], dtype=np.int32)
    d = synth.make_rnn_inputs(mode, 6, 5, 3, 4, proj_size=P, num_layers=2, bidirectional=True,
                              layout="packed", lengths=lengths, w_scale=0.6, h0_std=0.3,
                              c0_std=0.3, seed=12)
    y, hn, cn = _oracle_run(mode, d)
    y_pad = oracle.unpack_sequence(y, lengths, 6)
    for b, Lb in enumerate(lengths):
        xb = d["x_padded"][:Lb, b:b + 1]
        yb, hb, cb = oracle.rnn_forward(mode, xb, d["params"], h0=d["h0"][:, b:b + 1],
                                        c0=None if cn is None else d["c0"][:, b:b + 1],
                                        num_layers=2, bidirectional=True, proj_size=P)
        np.testing.assert_allclose(y_pad[:Lb, b], yb[:, 0], **TIGHT)
        np.testing.assert_allclose(hn[:, b], hb[:, 0], **TIGHT)
        if cn is not None:
            np.testing.assert_allclose(cn[:, b], cb[:, 0], **TIGHT)


def test_packed_equals_padded():
    lengths = np.array([9, 7, 7, 3, 1, 1], dtype=np.int32)
    d = synth.make_rnn_inputs("lstm", 9, 6, 4, 5, num_layers=2, bidirectional=True,
                              layout="packed", lengths=lengths, w_scale=0.5, seed=13)
    y_pk, hn_pk, cn_pk = _oracle_run("lstm", d)
    dp = dict(d, layout="padded", x=d["x_padded"])
    y_pd, hn_pd, cn_pd = _oracle_run("lstm", dp)
    np.testing.assert_allclose(oracle.pack_sequence(y_pd, lengths), y_pk, **TIGHT)
    np.testing.assert_allclose(hn_pk, hn_pd, **TIGHT)
    np.testing.assert_allclose(cn_pk, cn_pd, **TIGHT)


def test_bidirectional_is_forward_plus_reversed_forward():
    lengths = np.array([7, 5, 2], dtype=np.int32)
    d = synth.make_rnn_inputs("lstm", 7, 3, 4, 3, bidirectional=True, lengths=lengths,
                              w_scale=0.5, h0_std=0.4, c0_std=0.4, seed=14)
    y, hn, cn = _oracle_run("lstm", d)
    H = 3
    for b, Lb in enumerate(lengths):
        xb = d["x_padded"][:Lb, b:b + 1]
        yf, hf, cf = oracle.rnn_forward("lstm", xb, [d["params"][0]], h0=d["h0"][0:1, b:b + 1],
                                        c0=d["c0"][0:1, b:b + 1])
        yr, hr, cr = oracle.rnn_forward("lstm", xb[::-1], [d["params"][1]], h0=d["h0"][1:2, b:b + 1],
                                        c0=d["c0"][1:2, b:b + 1])
        np.testing.assert_allclose(y[:Lb, b, :H], yf[:, 0], **TIGHT)
        np.testing.assert_allclose(y[:Lb, b, H:], yr[::-1, 0], **TIGHT)
        np.testing.assert_allclose(hn[1, b], hr[0, 0], **TIGHT)
        np.testing.assert_allclose(cn[1, b], cr[0, 0], **TIGHT)


# ---------------------------------------------------------------------------
# RSSM prior
# ---------------------------------------------------------------------------

def _torch_rssm(w, actions, eps, s0=None, h0=None):
    """PyTorch modules assembled from the RSSMPrior description (float64)."""
    E, SA = w["w_as"].shape
    Hb = w["w_hh"].shape[1]
    S2 = w["w_2"].shape[0]
    lin_as = torch.nn.Linear(SA, E)
    gru = torch.nn.GRUCell(E, Hb)
    lin1 = torch.nn.Linear(Hb, w["w_1"].shape[0])
    lin2 = torch.nn.Linear(w["w_1"].shape[0], S2)
    with torch.no_grad():
        for mod, wk, bk in ((lin_as, "w_as", "b_as"), (lin1, "w_1", "b_1"), (lin2, "w_2", "b_2")):
            mod.weight.copy_(torch.tensor(w[wk]))
            mod.bias.copy_(torch.tensor(w[bk]))
        gru.weight_ih.copy_(torch.tensor(w["w_ih"]))
        gru.weight_hh.copy_(torch.tensor(w["w_hh"]))
        gru.bias_ih.copy_(torch.tensor(w["b_ih"]))
        gru.bias_hh.copy_(torch.tensor(w["b_hh"]))
        B, T = actions.shape[:2]
        S = S2 // 2
        state = torch.zeros(B, S) if s0 is None else torch.tensor(s0, dtype=torch.float64)
        belief = torch.zeros(B, Hb) if h0 is None else torch.tensor(h0, dtype=torch.float64)
        outs = [[], [], [], []]
        for t in range(T):
            a = torch.tensor(actions[:, t], dtype=torch.float64)
            e = torch.nn.functional.elu(lin_as(torch.cat([state, a], dim=-1)))
            belief = gru(e, belief)
            v = lin2(torch.nn.functional.elu(lin1(belief)))
            mean, raw = v[:, :S], v[:, S:]
            std = torch.nn.functional.softplus(raw) + 0.1
            state = mean + torch.tensor(eps[:, t], dtype=torch.float64) * std
            for lst, val in zip(outs, (mean, std, state, belief)):
                lst.append(val)
        return [torch.stack(o, 1).numpy() for o in outs]


def test_rssm_matches_torch_modules():
    d = synth.make_rssm_inputs(6, 9, state_dim=5, action_dim=3, embed_dim=7, belief_dim=8,
                               seed=15, s0_std=0.5, h0_std=0.5)
    got = oracle.rssm_prior_unroll(d["actions"], d["eps"], d["weights"], d["s0"], d["h0"])
    ref = _torch_rssm(d["weights"], d["actions"], d["eps"], d["s0"], d["h0"])
    for g, r in zip(got, ref):
        # softplus arguments here stay far below PyTorch's threshold of 20.
        np.testing.assert_allclose(g, r, rtol=1e-11, atol=1e-12)


def test_rssm_zero_weights_closed_form():
    # beliefs = 0, means = 0, stds = softplus(0) + 0.1 = ln 2 + 0.1 and
    # states = (ln 2 + 0.1) * eps at every step.
    d = synth.make_rssm_inputs(4, 5, seed=16, zero_weights=True)
    means, stds, states, beliefs = oracle.rssm_prior_unroll(d["actions"], d["eps"], d["weights"])
    k = math.log(2.0) + 0.1
    assert np.all(beliefs == 0) and np.all(means == 0)
    np.testing.assert_allclose(stds, np.full_like(stds, 0.7931471805599453), rtol=1e-15)
    assert abs(k - 0.7931471805599453) < 1e-15
    np.testing.assert_allclose(states, k * d["eps"].astype(np.float64), rtol=1e-15)


def test_rssm_time_chunking_and_single_step():
    d = synth.make_rssm_inputs(3, 8, state_dim=4, action_dim=2, embed_dim=6, belief_dim=5, seed=17)
    full = oracle.rssm_prior_unroll(d["actions"], d["eps"], d["weights"])
    a = oracle.rssm_prior_unroll(d["actions"][:, :3], d["eps"][:, :3], d["weights"])
    b = oracle.rssm_prior_unroll(d["actions"][:, 3:], d["eps"][:, 3:], d["weights"],
                                 a[2][:, -1], a[3][:, -1])
    for f, x, y in zip(full, a, b):
        np.testing.assert_allclose(np.concatenate([x, y], axis=1), f, **TIGHT)
    one = oracle.rssm_prior_step(np.zeros((3, 4)), np.zeros((3, 5)), d["actions"][:, 0],
                                 d["eps"][:, 0], d["weights"])
    for o, f in zip(one, full):
        np.testing.assert_allclose(o, f[:, 0], **TIGHT)


# ---------------------------------------------------------------------------
# RSSM prior with an actor in the loop (the issue's second unroll; the actor
# is the synthetic MLP tanh(W_a2 ELU(W_a1 [s; h] + b_a1) + b_a2))
# ---------------------------------------------------------------------------

def _torch_rssm_actor(w, aw, eps, s0=None, h0=None):
    """The second unroll written with PyTorch modules in float64."""
    E, SA = w["w_as"].shape
    Hb = w["w_hh"].shape[1]
    S2 = w["w_2"].shape[0]
    Ea, SH = aw["w_a1"].shape
    A = aw["w_a2"].shape[0]
    lin_as = torch.nn.Linear(SA, E)
    gru = torch.nn.GRUCell(E, Hb)
    lin1 = torch.nn.Linear(Hb, w["w_1"].shape[0])
    lin2 = torch.nn.Linear(w["w_1"].shape[0], S2)
    actor = torch.nn.Sequential(torch.nn.Linear(SH, Ea), torch.nn.ELU(), torch.nn.Linear(Ea, A), torch.nn.Tanh())
    with torch.no_grad():
        for mod, wk, bk in ((lin_as, "w_as", "b_as"), (lin1, "w_1", "b_1"), (lin2, "w_2", "b_2")):
            mod.weight.copy_(torch.tensor(w[wk]))
            mod.bias.copy_(torch.tensor(w[bk]))
        actor[0].weight.copy_(torch.tensor(aw["w_a1"]))
        actor[0].bias.copy_(torch.tensor(aw["b_a1"]))
        actor[2].weight.copy_(torch.tensor(aw["w_a2"]))
        actor[2].bias.copy_(torch.tensor(aw["b_a2"]))
        gru.weight_ih.copy_(torch.tensor(w["w_ih"]))
        gru.weight_hh.copy_(torch.tensor(w["w_hh"]))
        gru.bias_ih.copy_(torch.tensor(w["b_ih"]))
        gru.bias_hh.copy_(torch.tensor(w["b_hh"]))
        B, H = eps.shape[:2]
        S = S2 // 2
        state = torch.zeros(B, S) if s0 is None else torch.tensor(s0, dtype=torch.float64)
        belief = torch.zeros(B, Hb) if h0 is None else torch.tensor(h0, dtype=torch.float64)
        outs = [[], [], [], [], []]
        for t in range(H):
            action = actor(torch.cat([state, belief], dim=-1))
            e = torch.nn.functional.elu(lin_as(torch.cat([state, action], dim=-1)))
            belief = gru(e, belief)
            v = lin2(torch.nn.functional.elu(lin1(belief)))
            mean, raw = v[:, :S], v[:, S:]
            std = torch.nn.functional.softplus(raw) + 0.1
            state = mean + torch.tensor(eps[:, t], dtype=torch.float64) * std
            for lst, val in zip(outs, (mean, std, state, belief, action)):
                lst.append(val)
        return [torch.stack(o, 1).numpy() for o in outs]


def test_rssm_actor_matches_torch_modules():
    d = synth.make_rssm_inputs(5, 8, state_dim=4, action_dim=3, embed_dim=7, belief_dim=6, actor_dim=9,
                               seed=19, s0_std=0.5, h0_std=0.5)
    got = oracle.rssm_actor_unroll(d["eps"], d["weights"], d["actor"], d["s0"], d["h0"])
    ref = _torch_rssm_actor(d["weights"], d["actor"], d["eps"], d["s0"], d["h0"])
    for g, r in zip(got, ref):
        np.testing.assert_allclose(g, r, rtol=1e-11, atol=1e-12)


def test_rssm_actor_constant_policy_equals_given_actions():
    # W_a1 = W_a2 = 0 and b_a2 = atanh(c): the actor returns c every step,
    # so the unroll is the first one over constant actions c.
    d = synth.make_rssm_inputs(4, 7, state_dim=3, action_dim=2, embed_dim=5, belief_dim=6, actor_dim=4,
                               seed=20, s0_std=0.3, h0_std=0.3)
    c = np.array([0.4, -0.7])
    aw = {"w_a1": np.zeros((4, 9)), "b_a1": np.ones(4), "w_a2": np.zeros((2, 4)), "b_a2": np.arctanh(c)}
    got = oracle.rssm_actor_unroll(d["eps"], d["weights"], aw, d["s0"], d["h0"])
    acts = np.broadcast_to(c, (4, 7, 2))
    ref = oracle.rssm_prior_unroll(acts, d["eps"], d["weights"], d["s0"], d["h0"])
    for g, r in zip(got[:4], ref):
        np.testing.assert_allclose(g, r, **TIGHT)
    np.testing.assert_allclose(got[4], acts, rtol=1e-15)


def test_rssm_actor_zero_weights_closed_form():
    d = synth.make_rssm_inputs(3, 4, seed=21, zero_weights=True, actor_dim=8)
    aw = {k: np.zeros_like(v) for k, v in d["actor"].items()}
    means, stds, states, beliefs, actions = oracle.rssm_actor_unroll(d["eps"], d["weights"], aw)
    assert np.all(actions == 0) and np.all(beliefs == 0) and np.all(means == 0)
    np.testing.assert_allclose(stds, np.full_like(stds, 0.7931471805599453), rtol=1e-15)
    np.testing.assert_allclose(states, 0.7931471805599453 * d["eps"].astype(np.float64), rtol=1e-15)


def test_rssm_actor_time_chunking():
    d = synth.make_rssm_inputs(3, 9, state_dim=4, action_dim=2, embed_dim=6, belief_dim=5, actor_dim=7, seed=22)
    full = oracle.rssm_actor_unroll(d["eps"], d["weights"], d["actor"])
    a = oracle.rssm_actor_unroll(d["eps"][:, :4], d["weights"], d["actor"])
    b = oracle.rssm_actor_unroll(d["eps"][:, 4:], d["weights"], d["actor"], a[2][:, -1], a[3][:, -1])
    for f, x, y in zip(full, a, b):
        np.testing.assert_allclose(np.concatenate([x, y], axis=1), f, **TIGHT)


# ---------------------------------------------------------------------------
# bf16 rounding and the bf16 tolerance headroom
# ---------------------------------------------------------------------------

def test_bf16_rounding_three_ways_agree():
    rng = np.random.default_rng(18)
    v = np.concatenate([rng.normal(0, 1, 5000), rng.normal(0, 1e4, 500),
                        [0.0, -0.0, 1.0, 1.00390625, 1.005859375, 1.0078125, -2.5, 3.0e38]]).astype(np.float32)
    a = oracle.round_to_bf16(v)
    b = synth.bf16_round(v).astype(np.float64)
    c = torch.tensor(v).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(a, c)
    # Ties go to even: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7.
    assert oracle.round_to_bf16(np.float32(1.00390625)) == 1.0
    assert oracle.round_to_bf16(np.float32(1.005859375)) == 1.0078125


@pytest.mark.parametrize("mode,H,P,T,L", [("gru", 64, 0, 48, 1), ("lstmp", 128, 32, 64, 2)])
def test_bf16_state_rounding_stays_inside_tolerance(mode, H, P, T, L):
    # Rounding the recurrent operand (h, and LSTMP's m) and the layer output to
    # bf16 every step must stay well inside the 2e-2 absolute bound.
    d = synth.make_rnn_inputs(mode, T, 16, 48, H, proj_size=P, num_layers=L, dtype="bf16",
                              w_scale=1.0 / np.sqrt(H), h0_std=0.1 if mode == "gru" else 0.0,
                              seed=19)
    y, hn, cn = _oracle_run(mode, d)
    ye, hne, cne = _oracle_run(mode, d, emulate_bf16=True)
    assert np.max(np.abs(ye - y)) < 5e-3
    assert np.max(np.abs(hne - hn)) < 5e-3


# ---------------------------------------------------------------------------
# Cell and projection clipping (LSTM, LSTMP). The apache/mxnet issue "RNN Op
# Changes" names cuDNN's cell clipping and asks for state and projection
# clipping without defining them; the oracle reads them as clamps of the
# updated cell state (carried forward) and of the projected output.
# ---------------------------------------------------------------------------

def _gate_bias_case(mode, H, P=0, F=None, T=5, B=1, seed=40):
    F = F or H
    d = _rand_case(mode, T=T, B=B, F=F, H=H, P=P, seed=seed, h0=False)
    p = d["params"][0]
    for k in p:
        p[k] = np.zeros(np.shape(p[k]), dtype=np.float64)  # exact float64 gate values
    return d, p


def test_cell_clip_recursion_closed_form():
    # i = sigmoid(40) = 1 (to double precision), f = sigmoid(0) = 1/2,
    # g = tanh(atanh(-1/2)) = -1/2, o = 1/2, c0 = 4: the carried state obeys
    # c_t = clip(c_{t-1} / 2 - 1/2, lo, hi) and h_t = tanh(c_t) / 2. Clipping
    # only the output (not the carried state) would give c_2 = 1/4 here.
    H, T, lo, hi = 1, 6, -0.7, 1.0
    d, p = _gate_bias_case("lstm", H, T=T)
    p["b_ih"][0] = 40.0
    p["b_ih"][2] = math.atanh(-0.5)
    d["c0"] = np.full((1, 1, H), 4.0)
    y, hn, cn = _oracle_run("lstm", d, cell_clip=(lo, hi))
    c = 4.0
    for t in range(T):
        c = min(max(c / 2.0 - 0.5, lo), hi)
        np.testing.assert_allclose(y[t, 0, 0], 0.5 * math.tanh(c), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(cn[0, 0, 0], c, rtol=1e-14, atol=1e-15)
    assert c == lo  # the lower bound is reached and held


def test_cell_clip_per_unit_bounds():
    # f = 0, i = 1: c_t = g = tanh(b_g) per unit each step; clip bounds cut
    # the units above hi and below lo, the others pass through.
    gs = np.array([0.9, -0.9, 0.1, -0.2])
    H = gs.size
    d, p = _gate_bias_case("lstm", H, T=3)
    p["b_ih"][0:H] = 40.0
    p["b_ih"][H:2 * H] = -40.0
    p["b_ih"][2 * H:3 * H] = np.arctanh(gs)
    y, hn, cn = _oracle_run("lstm", d, cell_clip=(-0.5, 0.25))
    want_c = np.array([0.25, -0.5, 0.1, -0.2])
    np.testing.assert_allclose(cn[0, 0], want_c, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(y[2, 0], 0.5 * np.tanh(want_c), rtol=1e-14, atol=1e-15)


def test_projection_clip_scalar_brute_force():
    # P = H = F = 1. i = 1, f = 0, o = 1/2; W_ih(g) = 1 reads x, W_hh(g) = 1
    # reads the previous projected output, W_hr = 10. Then per step
    #   u_t = x_t + h_{t-1},  c_t = tanh(u_t),  h_t = clip(5 tanh(c_t), -p, p),
    # so a clipped output that is not fed back would change u_{t+1}.
    T, pc = 5, 1.5
    d, p = _gate_bias_case("lstmp", 1, P=1, F=1, T=T)
    p["b_ih"][0], p["b_ih"][1] = 40.0, -40.0
    p["w_ih"][2, 0] = 1.0
    p["w_hh"][2, 0] = 1.0
    p["w_hr"][0, 0] = 10.0
    xs = [0.8, -0.05, -3.0, 0.0, 0.3]
    d["x"] = np.array(xs, dtype=np.float64).reshape(T, 1, 1)
    y, hn, cn = _oracle_run("lstmp", d, proj_clip=pc)
    h, hits = 0.0, 0
    for t in range(T):
        v = 5.0 * math.tanh(math.tanh(xs[t] + h))
        hits += abs(v) > pc
        h = min(max(v, -pc), pc)
        np.testing.assert_allclose(y[t, 0, 0], h, rtol=1e-14, atol=1e-15)
    assert hits >= 2


def test_projection_clip_per_unit_closed_form():
    # W_hr = 10 I, W_hh = 0, i = 1, f = 0, o = 1/2, c = g: h = clip(5 tanh(g)).
    gs = np.array([0.9, -0.9, 0.1, -0.2])
    H = gs.size
    d, p = _gate_bias_case("lstmp", H, P=H, T=2)
    p["b_ih"][0:H] = 40.0
    p["b_ih"][H:2 * H] = -40.0
    p["b_ih"][2 * H:3 * H] = np.arctanh(gs)
    p["w_hr"] = 10.0 * np.eye(H)
    y, hn, cn = _oracle_run("lstmp", d, proj_clip=2.0)
    raw = 5.0 * np.tanh(gs)
    np.testing.assert_allclose(hn[0, 0], np.minimum(np.maximum(raw, -2.0), 2.0), rtol=1e-14, atol=1e-15)
    assert np.abs(raw).max() > 2.0 and np.abs(raw).min() < 2.0


@pytest.mark.parametrize("mode,P", [("lstm", 0), ("lstmp", 3)])
def test_infinite_clip_bounds_change_nothing(mode, P):
    d = _rand_case(mode, T=6, B=3, F=5, H=4, P=P, L=2, bidir=True, lengths=[6, 4, 2], seed=41)
    ref = _oracle_run(mode, d)
    kw = dict(cell_clip=(-np.inf, np.inf))
    if P:
        kw["proj_clip"] = np.inf
    got = _oracle_run(mode, d, **kw)
    for a, b in zip(ref, got):
        np.testing.assert_array_equal(a, b)


def test_clip_keeps_nan_like_numpy():
    rng = np.random.default_rng(42)
    a = rng.normal(size=200) * 3
    a[::17] = np.nan
    np.testing.assert_array_equal(oracle.clip(a, -1.25, 0.5), np.clip(a, -1.25, 0.5))


def test_clipping_outside_lstm_is_rejected():
    d = _rand_case("gru", T=3, B=2, F=3, H=2, seed=43)
    with pytest.raises(ValueError):
        _oracle_run("gru", d, cell_clip=(-1.0, 1.0))
    d = _rand_case("lstm", T=3, B=2, F=3, H=2, seed=43)
    with pytest.raises(ValueError):
        _oracle_run("lstm", d, proj_clip=1.0)


# ---------------------------------------------------------------------------
# Backward through time: torch autograd on the float64 modules, and central
# finite differences of the (pinned) forward oracle.
# ---------------------------------------------------------------------------

def _torch_grads(mode, d, dy, dh_n, dc_n):
    """Gradients of sum(dy * y) + sum(dh_n * h_n) + sum(dc_n * c_n) by autograd."""
    m = _torch_rnn(mode, d)
    K = d["proj_size"] if mode == "lstmp" else d["hidden_size"]
    D = 2 if d["bidirectional"] else 1
    LD, B = d["num_layers"] * D, d["B"]
    h0 = torch.tensor(d["h0"] if d["h0"] is not None else np.zeros((LD, B, K)), dtype=torch.float64,
                      requires_grad=True)
    x = torch.tensor(np.nan_to_num(d["x_padded"]), dtype=torch.float64, requires_grad=True)
    lengths = d["lengths"]
    xin = x if lengths is None else torch.nn.utils.rnn.pack_padded_sequence(
        x, torch.tensor(lengths, dtype=torch.int64), enforce_sorted=False)
    if mode == "gru":
        y, hn = m(xin, h0)
        cn, c0 = None, None
    else:
        c0 = torch.tensor(d["c0"] if d["c0"] is not None else np.zeros((LD, B, d["hidden_size"])),
                          dtype=torch.float64, requires_grad=True)
        y, (hn, cn) = m(xin, (h0, c0))
    if lengths is not None:
        y, _ = torch.nn.utils.rnn.pad_packed_sequence(y, total_length=d["T"])
    loss = (y * torch.tensor(dy)).sum() + (hn * torch.tensor(dh_n)).sum()
    if cn is not None:
        loss = loss + (cn * torch.tensor(dc_n)).sum()
    loss.backward()
    grads = []
    for layer in range(d["num_layers"]):
        for di in range(D):
            sfx = f"_l{layer}" + ("_reverse" if di == 1 else "")
            g = {"w_ih": getattr(m, "weight_ih" + sfx).grad.numpy(), "w_hh": getattr(m, "weight_hh" + sfx).grad.numpy()}
            if d["params"][0]["b_ih"] is not None:
                g["b_ih"] = getattr(m, "bias_ih" + sfx).grad.numpy()
                g["b_hh"] = getattr(m, "bias_hh" + sfx).grad.numpy()
            if mode == "lstmp":
                g["w_hr"] = getattr(m, "weight_hr" + sfx).grad.numpy()
            grads.append(g)
    return x.grad.numpy(), h0.grad.numpy(), None if c0 is None else c0.grad.numpy(), grads


def _bwd_case(mode, L, bidir, P, bias, varlen, seed):
    B, T = 5, 7
    lengths = np.array([7, 3, 6, 1, 5], dtype=np.int32) if varlen else None
    d = _rand_case(mode, T=T, B=B, F=4, H=3, P=P, L=L, bidir=bidir, bias=bias, lengths=lengths, seed=seed)
    rng = np.random.default_rng(seed + 100)
    D = 2 if bidir else 1
    K = P if mode == "lstmp" else 3
    dy = rng.normal(size=(T, B, D * K))
    if lengths is not None:
        for b, Lb in enumerate(lengths):
            dy[Lb:, b] = 0.0
    dh_n = rng.normal(size=(L * D, B, K))
    dc_n = rng.normal(size=(L * D, B, 3)) if mode != "gru" else None
    return d, dy, dh_n, dc_n


BWD_CASES = [
    # mode, L, bidir, P, bias, varlen
    ("lstm", 1, False, 0, True, False),
    ("lstm", 2, True, 0, True, True),
    ("lstm", 1, False, 0, False, True),
    ("gru", 1, False, 0, True, False),
    ("gru", 2, True, 0, True, True),
    ("gru", 1, True, 0, False, False),
    ("lstmp", 1, False, 2, True, False),
    ("lstmp", 2, True, 2, True, True),
]


@pytest.mark.parametrize("mode,L,bidir,P,bias,varlen", BWD_CASES)
def test_backward_matches_torch_autograd(mode, L, bidir, P, bias, varlen):
    d, dy, dh_n, dc_n = _bwd_case(mode, L, bidir, P, bias, varlen, seed=50 + L + 2 * bidir + P)
    ref = _torch_grads(mode, d, dy, dh_n, dc_n)
    got = oracle.rnn_backward(mode, d["x"], d["params"], dy, dh_n=dh_n, dc_n=dc_n, lengths=d["lengths"],
                              h0=d["h0"], c0=d["c0"], num_layers=L, bidirectional=bidir, proj_size=P)
    dx, dh0, dc0, grads = got
    np.testing.assert_allclose(dx, ref[0], **TIGHT)
    np.testing.assert_allclose(dh0, ref[1], **TIGHT)
    if ref[2] is not None:
        np.testing.assert_allclose(dc0, ref[2], **TIGHT)
    for g, r in zip(grads, ref[3]):
        for k, v in r.items():
            np.testing.assert_allclose(g[k], v, err_msg=k, **TIGHT)


@pytest.mark.parametrize("mode,P", [("lstm", 0), ("gru", 0), ("lstmp", 2)])
def test_backward_finite_differences(mode, P):
    # central differences of L = sum(dy * y) + sum(dh_n * h_n) + sum(dc_n * c_n)
    d, dy, dh_n, dc_n = _bwd_case(mode, 1, True, P, True, True, seed=60 + P)

    def loss(params=d["params"], x=d["x"], h0=d["h0"], c0=d["c0"]):
        y, hn, cn = oracle.rnn_forward(mode, x, params, lengths=d["lengths"], h0=h0, c0=c0,
                                       bidirectional=True, proj_size=P)
        s = float((np.nan_to_num(y) * dy).sum() + (hn * dh_n).sum())
        return s + (float((cn * dc_n).sum()) if cn is not None else 0.0)

    dx, dh0, dc0, grads = oracle.rnn_backward(mode, d["x"], d["params"], dy, dh_n=dh_n, dc_n=dc_n,
                                              lengths=d["lengths"], h0=d["h0"], c0=d["c0"],
                                              bidirectional=True, proj_size=P)
    eps = 1e-6
    rng = np.random.default_rng(7)
    for idx in (0, 1):
        for k in grads[idx]:
            arr = d["params"][idx][k]
            for flat in rng.choice(arr.size, size=min(4, arr.size), replace=False):
                pos = np.unravel_index(flat, arr.shape)
                plus = [dict(p) for p in d["params"]]
                minus = [dict(p) for p in d["params"]]
                a = np.array(arr, dtype=np.float64)
                a[pos] += eps
                plus[idx][k] = a.copy()
                a[pos] -= 2 * eps
                minus[idx][k] = a
                fd = (loss(params=plus) - loss(params=minus)) / (2 * eps)
                assert abs(fd - grads[idx][k][pos]) < 1e-6 * max(1.0, abs(fd)), (idx, k, pos)
    x = np.array(d["x"], dtype=np.float64)
    for pos in [(0, 0, 0), (2, 1, 3), (4, 4, 1)]:
        xp, xm = x.copy(), x.copy()
        xp[pos] += eps
        xm[pos] -= eps
        fd = (loss(x=xp) - loss(x=xm)) / (2 * eps)
        assert abs(fd - dx[pos]) < 1e-6 * max(1.0, abs(fd)), pos


def test_backward_packed_equals_padded():
    lengths = np.array([6, 6, 4, 2, 1], dtype=np.int32)
    dp = synth.make_rnn_inputs("lstm", 6, 5, 3, 4, num_layers=2, bidirectional=True, layout="packed",
                               lengths=lengths, seed=70, h0_std=0.5, c0_std=0.5)
    rng = np.random.default_rng(71)
    dy_p = rng.normal(size=(int(lengths.sum()), 8))
    kw = dict(lengths=lengths, h0=dp["h0"], c0=dp["c0"], num_layers=2, bidirectional=True)
    dxp, dh0p, dc0p, gp = oracle.rnn_backward("lstm", dp["x"], dp["params"], dy_p, layout="packed", **kw)
    x_pad = np.nan_to_num(oracle.unpack_sequence(dp["x"], lengths, 6))
    dy_pad = np.nan_to_num(oracle.unpack_sequence(dy_p, lengths, 6))
    dx, dh0, dc0, g = oracle.rnn_backward("lstm", x_pad, dp["params"], dy_pad, **kw)
    np.testing.assert_allclose(dxp, oracle.pack_sequence(dx, lengths), **TIGHT)
    np.testing.assert_allclose(dh0p, dh0, **TIGHT)
    np.testing.assert_allclose(dc0p, dc0, **TIGHT)
    for a, b in zip(gp, g):
        for k in a:
            np.testing.assert_allclose(a[k], b[k], **TIGHT)
