"""Float64 oracle: LSTM, LSTM with projection (LSTMP) and GRU recurrences.

TEST INFRASTRUCTURE ONLY (see the package docstring). Nothing here is tuned:
each step recomputes x_t.W_ih^T inside the step, exactly as the cell
definitions read.

Cell conventions. The pages name the cells (nn.GRUCell in the RSSM issue;
nn.LSTM and "LSTMCell plus one matmul" in the LSTM-with-projections issue)
without printing equations, so the equations and chunk orders are PyTorch's
documented ones:

  LSTM  gates a = W_ih x + b_ih + W_hh h + b_hh, chunks [i | f | g | o]
        c' = sigmoid(f) * c + sigmoid(i) * tanh(g)
        m  = sigmoid(o) * tanh(c')
        h' = m                     (plain LSTM)
        h' = W_hr m                (LSTMP; no projection bias)
  Optional clipping (LSTM, LSTMP), named but not defined by the apache/mxnet
  issue "RNN Op Changes" (cuDNN's cell clipping; the requests for state and
  projection clipping). Read as clamps that keep NaN:
        c' <- clip(c', lo, hi)     after the cell update, before tanh(c');
                                   the clipped c' is the carried state
        h' <- clip(W_hr m, -p, p)  (LSTMP, on the projected output)
  GRU   ax = W_ih x + b_ih, ah = W_hh h + b_hh, chunks [r | z | n]
        r = sigmoid(ax_r + ah_r), z = sigmoid(ax_z + ah_z)
        n = tanh(ax_n + r * ah_n)  (reset gate multiplies ah_n incl. b_hn)
        h' = (1 - z) * n + z * h
"""

import numpy as np

__all__ = [
    "sigmoid", "elu", "softplus", "clip", "lstm_cell", "gru_cell", "run_direction",
    "rnn_forward", "rnn_backward", "run_direction_backward", "pack_sequence", "unpack_sequence", "packed_offsets",
    "round_to_bf16",
]


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def sigmoid(x):
    """Logistic function 1 / (1 + exp(-x)), evaluated without overflow."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def elu(x):
    """ELU with alpha = 1 (nn.ELU default): x for x > 0, exp(x) - 1 otherwise."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0, x, np.expm1(np.minimum(x, 0.0)))


def softplus(x):
    """softplus(x) = log(1 + exp(x)) with beta = 1, computed as logaddexp(0, x)."""
    return np.logaddexp(0.0, np.asarray(x, dtype=np.float64))


def round_to_bf16(a):
    """Round float values to the nearest bfloat16 value (ties to even).

    Used only by the emulated-rounding variant of the oracle, which measures
    how far bf16 storage of the recurrent state can move the result.
    """
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)).astype(np.uint32)
    out = r.view(np.float32).astype(np.float64)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = np.nan
    return out.reshape(np.shape(a))


def clip(a, lo, hi):
    """Clamp to [lo, hi] elementwise; NaN stays NaN (np.clip semantics)."""
    a = np.asarray(a, dtype=np.float64)
    return np.where(a < lo, lo, np.where(a > hi, hi, a))


def lstm_cell(x, h, c, w_ih, w_hh, b_ih=None, b_hh=None, w_hr=None, round_m=None,
              cell_clip=None, proj_clip=None):
    """One LSTM (or LSTMP when ``w_hr`` is given) step for a batch of rows.

    x [B, F], h [B, K], c [B, H]; w_ih [4H, F], w_hh [4H, K], b_* [4H],
    w_hr [P, H]. K = H for LSTM, K = P for LSTMP. Returns (h', c').
    cell_clip (lo, hi) clamps the updated cell state; proj_clip p clamps
    the projected output to [-p, p] (LSTMP only).
    LSTMP is "LSTMCell plus one more matmul on the resulting hidden state"
    (pytorch/pytorch issue "Integrating CuDNN API for LSTMs with
    projections", design discussion).
    """
    H = np.shape(c)[-1]
    a = _f64(x) @ _f64(w_ih).T + _f64(h) @ _f64(w_hh).T
    if b_ih is not None:
        a = a + _f64(b_ih)
    if b_hh is not None:
        a = a + _f64(b_hh)
    i = sigmoid(a[:, 0:H])
    f = sigmoid(a[:, H:2 * H])
    g = np.tanh(a[:, 2 * H:3 * H])
    o = sigmoid(a[:, 3 * H:4 * H])
    c_new = f * _f64(c) + i * g
    if cell_clip is not None:
        c_new = clip(c_new, cell_clip[0], cell_clip[1])
    m = o * np.tanh(c_new)
    if w_hr is None:
        if proj_clip is not None:
            raise ValueError("projection clipping needs a projection")
        return m, c_new
    if round_m is not None:
        m = round_m(m)
    h_new = m @ _f64(w_hr).T
    if proj_clip is not None:
        h_new = clip(h_new, -proj_clip, proj_clip)
    return h_new, c_new


def gru_cell(x, h, w_ih, w_hh, b_ih=None, b_hh=None):
    """One GRU step (PyTorch r/z/n convention) for a batch of rows.

    x [B, F], h [B, H]; w_ih [3H, F], w_hh [3H, H], b_* [3H]. Returns h'.
    The reset gate multiplies the whole hidden-side n pre-activation,
    including its bias b_hn (nn.GRUCell, named by the pytorch/rl RSSM issue).
    """
    H = np.shape(h)[-1]
    ax = _f64(x) @ _f64(w_ih).T
    ah = _f64(h) @ _f64(w_hh).T
    if b_ih is not None:
        ax = ax + _f64(b_ih)
    if b_hh is not None:
        ah = ah + _f64(b_hh)
    r = sigmoid(ax[:, 0:H] + ah[:, 0:H])
    z = sigmoid(ax[:, H:2 * H] + ah[:, H:2 * H])
    n = np.tanh(ax[:, 2 * H:3 * H] + r * ah[:, 2 * H:3 * H])
    return (1.0 - z) * n + z * _f64(h)


def packed_offsets(lengths):
    """PackedSequence bookkeeping for lengths sorted non-increasing.

    Returns (batch_sizes [T_max], offsets [T_max + 1]) where batch_sizes[t]
    counts sequences with L_b > t and offsets[t] = sum_b min(L_b, t) is the
    packed row of step t's first entry (apache/mxnet issue "RNN Op Changes",
    RFC: sequences sorted by length and packed contiguously, as PyTorch's
    PackedSequence does).
    """
    L = np.asarray(lengths, dtype=np.int64)
    T = int(L.max()) if L.size else 0
    bs = np.array([int((L > t).sum()) for t in range(T)], dtype=np.int64)
    off = np.zeros(T + 1, dtype=np.int64)
    off[1:] = np.cumsum(bs)
    return bs, off


def pack_sequence(padded, lengths):
    """Padded [T, B, F] -> packed [N_tok, F]: step-major, batch order inside a step."""
    L = np.asarray(lengths, dtype=np.int64)
    if np.any(L[:-1] < L[1:]):
        raise ValueError("packed layout needs lengths sorted non-increasing")
    rows = []
    for t in range(int(L.max())):
        for b in range(L.size):
            if L[b] > t:
                rows.append(padded[t, b])
    return np.stack(rows, axis=0)


def unpack_sequence(packed, lengths, T, fill=np.nan):
    """Packed [N_tok, F] -> padded [T, B, F]; positions t >= L_b hold ``fill``."""
    L = np.asarray(lengths, dtype=np.int64)
    if np.any(L[:-1] < L[1:]):
        raise ValueError("packed layout needs lengths sorted non-increasing")
    B = L.size
    out = np.full((T, B) + tuple(packed.shape[1:]), fill, dtype=np.float64)
    k = 0
    for t in range(int(L.max())):
        for b in range(B):
            if L[b] > t:
                out[t, b] = packed[k]
                k += 1
    assert k == packed.shape[0]
    return out


def run_direction(mode, x, lengths, h0, c0, p, reverse=False, emulate_bf16=False,
                  cell_clip=None, proj_clip=None):
    """Run one layer in one direction over a padded batch.

    mode 'lstm' | 'lstmp' | 'gru'; x [T, B, F]; lengths [B] (1 <= L_b <= T);
    h0 [B, K]; c0 [B, H] (LSTM/LSTMP). Row b is active at step t iff t < L_b;
    inactive rows neither update nor write (apache/mxnet issue "RNN Op
    Changes", RFC: variable-length sequences that masking cannot fake). In
    reverse, each row starts at its own t = L_b - 1 from h0, c0 (PackedSequence
    semantics). cell_clip / proj_clip as in lstm_cell (LSTM and LSTMP only).
    Returns (out [T, B, K] with NaN where nothing is written, h_last [B, K],
    c_last [B, H] or None).
    """
    if mode == "gru" and (cell_clip is not None or proj_clip is not None):
        raise ValueError("clipping is an LSTM / LSTMP option")
    x = _f64(x)
    T, B = x.shape[0], x.shape[1]
    L = np.full(B, T, dtype=np.int64) if lengths is None else np.asarray(lengths, dtype=np.int64)
    h = _f64(h0).copy()
    c = None if c0 is None else _f64(c0).copy()
    K = h.shape[1]
    rnd = round_to_bf16 if emulate_bf16 else (lambda a: a)
    h = rnd(h)
    out = np.full((T, B, K), np.nan, dtype=np.float64)
    steps = range(T - 1, -1, -1) if reverse else range(T)
    for t in steps:
        rows = np.nonzero(L > t)[0]
        if rows.size == 0:
            continue
        xt = x[t, rows]
        if mode == "gru":
            hn = gru_cell(xt, h[rows], p["w_ih"], p["w_hh"], p.get("b_ih"), p.get("b_hh"))
        elif mode in ("lstm", "lstmp"):
            hn, cn = lstm_cell(xt, h[rows], c[rows], p["w_ih"], p["w_hh"], p.get("b_ih"),
                               p.get("b_hh"), p.get("w_hr") if mode == "lstmp" else None,
                               round_m=round_to_bf16 if emulate_bf16 else None,
                               cell_clip=cell_clip, proj_clip=proj_clip)
            c[rows] = cn
        else:
            raise ValueError(f"unknown mode {mode!r}")
        hn = rnd(hn)
        h[rows] = hn
        out[t, rows] = hn
    return out, h, c


def rnn_forward(mode, x, params, *, lengths=None, h0=None, c0=None, num_layers=1,
                bidirectional=False, proj_size=0, layout="padded", emulate_bf16=False,
                cell_clip=None, proj_clip=None):
    """Multi-layer, optionally bidirectional, optionally variable-length forward.

    params: list indexed l * D + d of dicts with 'w_ih', 'w_hh', 'b_ih', 'b_hh'
    (biases may be None) and 'w_hr' for LSTMP. Layer l + 1 reads the
    concatenation [forward output ; reverse output] of layer l. h_n and c_n
    are stacked at index l * D + d. layout 'padded': x [T, B, F], y [T, B,
    D * K] with NaN at unwritten positions; layout 'packed': x [N_tok, F],
    y [N_tok, D * K], lengths sorted non-increasing. cell_clip (lo, hi) and
    proj_clip p as in lstm_cell, applied in every layer and direction.
    Returns (y, h_n [L * D, B, K], c_n [L * D, B, H] or None).
    """
    if mode not in ("lstm", "lstmp", "gru"):
        raise ValueError(mode)
    if (mode == "lstmp") != (proj_size > 0):
        raise ValueError("projection is an LSTM-only option (lstmp needs proj_size > 0)")
    D = 2 if bidirectional else 1
    x = _f64(x)
    if layout == "packed":
        if lengths is None:
            raise ValueError("packed layout needs lengths")
        T = int(np.max(lengths))
        xp = unpack_sequence(x, lengths, T)
    else:
        xp = x
        T = xp.shape[0]
    B = xp.shape[1]
    H = params[0]["w_hh"].shape[0] // (3 if mode == "gru" else 4)
    K = proj_size if mode == "lstmp" else H
    hn = np.zeros((num_layers * D, B, K))
    cn = None if mode == "gru" else np.zeros((num_layers * D, B, H))
    inp = xp
    for layer in range(num_layers):
        outs = []
        for d in range(D):
            idx = layer * D + d
            h_init = np.zeros((B, K)) if h0 is None else _f64(h0)[idx]
            c_init = None if mode == "gru" else (np.zeros((B, H)) if c0 is None else _f64(c0)[idx])
            out, h_last, c_last = run_direction(mode, inp, lengths, h_init, c_init, params[idx],
                                                reverse=(d == 1), emulate_bf16=emulate_bf16,
                                                cell_clip=cell_clip, proj_clip=proj_clip)
            outs.append(out)
            hn[idx] = h_last
            if cn is not None:
                cn[idx] = c_last
        inp = np.concatenate(outs, axis=2)
    y = inp
    if layout == "packed":
        y = pack_sequence(y, lengths)
    return y, hn, cn


# ---------------------------------------------------------------------------
# Backward through time (training). The pages' AMP / TorchScript discussion
# (pytorch/pytorch issue "Integrating CuDNN API for LSTMs with projections",
# thread) is about the backward of these cells; its definition is the chain
# rule through the cell equations above, step by step in reverse time.
# ---------------------------------------------------------------------------

def _lstm_cell_backward(x, h, c, p, dh, dc, grads, w_hr=None):
    """One LSTM / LSTMP step backward for a batch of rows.

    Recomputes the step from its inputs (x, h_{t-1}, c_{t-1}), then takes
    dh (gradient of the loss w.r.t. the step's output h_t) and dc (w.r.t.
    c_t from later steps). Accumulates the weight gradients into `grads`;
    returns (dx, dh_prev, dc_prev).
    """
    H = c.shape[-1]
    a = x @ _f64(p["w_ih"]).T + h @ _f64(p["w_hh"]).T
    if p.get("b_ih") is not None:
        a = a + _f64(p["b_ih"])
    if p.get("b_hh") is not None:
        a = a + _f64(p["b_hh"])
    i = sigmoid(a[:, 0:H])
    f = sigmoid(a[:, H:2 * H])
    g = np.tanh(a[:, 2 * H:3 * H])
    o = sigmoid(a[:, 3 * H:4 * H])
    c_new = f * c + i * g
    tc = np.tanh(c_new)
    if w_hr is not None:
        m = o * tc
        grads["w_hr"] += dh.T @ m
        dh = dh @ _f64(w_hr)          # gradient w.r.t. m
    do = dh * tc
    dct = dc + dh * o * (1.0 - tc * tc)
    di, df, dg = dct * g, dct * c, dct * i
    da = np.concatenate([di * i * (1 - i), df * f * (1 - f), dg * (1 - g * g), do * o * (1 - o)], axis=1)
    grads["w_ih"] += da.T @ x
    grads["w_hh"] += da.T @ h
    grads["b_ih"] += da.sum(0)
    grads["b_hh"] += da.sum(0)
    return da @ _f64(p["w_ih"]), da @ _f64(p["w_hh"]), dct * f


def _gru_cell_backward(x, h, p, dh, grads):
    """One GRU step backward (PyTorch r/z/n convention); returns (dx, dh_prev)."""
    H = h.shape[-1]
    ax = x @ _f64(p["w_ih"]).T
    ah = h @ _f64(p["w_hh"]).T
    if p.get("b_ih") is not None:
        ax = ax + _f64(p["b_ih"])
    if p.get("b_hh") is not None:
        ah = ah + _f64(p["b_hh"])
    r = sigmoid(ax[:, 0:H] + ah[:, 0:H])
    z = sigmoid(ax[:, H:2 * H] + ah[:, H:2 * H])
    n = np.tanh(ax[:, 2 * H:3 * H] + r * ah[:, 2 * H:3 * H])
    dn = dh * (1 - z)
    dz = dh * (h - n)
    dan = dn * (1 - n * n)
    dr = dan * ah[:, 2 * H:3 * H]
    dar = dr * r * (1 - r)
    daz = dz * z * (1 - z)
    dax = np.concatenate([dar, daz, dan], axis=1)
    dah = np.concatenate([dar, daz, dan * r], axis=1)
    grads["w_ih"] += dax.T @ x
    grads["w_hh"] += dah.T @ h
    grads["b_ih"] += dax.sum(0)
    grads["b_hh"] += dah.sum(0)
    return dax @ _f64(p["w_ih"]), dah @ _f64(p["w_hh"]) + dh * z


def run_direction_backward(mode, x, lengths, h0, c0, p, dy, dh_n, dc_n, reverse=False):
    """Backward of run_direction for one layer and direction (padded layout).

    x [T, B, F]; dy [T, B, K] (ignored where t >= L_b); dh_n [B, K], dc_n
    [B, H] (LSTM / LSTMP) or None: gradients w.r.t. the final states.
    Replays the forward to recover each step's inputs, then walks the steps
    in the opposite order. Returns (dx [T, B, F] (zero where t >= L_b),
    dh0 [B, K], dc0 [B, H] or None, grads dict of w_ih, w_hh, b_ih, b_hh
    (and w_hr for LSTMP)).
    """
    x = _f64(x)
    T, B = x.shape[0], x.shape[1]
    L = np.full(B, T, dtype=np.int64) if lengths is None else np.asarray(lengths, dtype=np.int64)
    h = _f64(h0).copy()
    c = None if c0 is None else _f64(c0).copy()
    steps = list(range(T - 1, -1, -1)) if reverse else list(range(T))
    w_hr = p.get("w_hr") if mode == "lstmp" else None
    # forward replay: the state entering each step
    saved = []
    for t in steps:
        rows = np.nonzero(L > t)[0]
        if rows.size == 0:
            saved.append(None)
            continue
        saved.append((rows, h[rows].copy(), None if c is None else c[rows].copy()))
        if mode == "gru":
            h[rows] = gru_cell(x[t, rows], h[rows], p["w_ih"], p["w_hh"], p.get("b_ih"), p.get("b_hh"))
        else:
            hn, cn = lstm_cell(x[t, rows], h[rows], c[rows], p["w_ih"], p["w_hh"], p.get("b_ih"),
                               p.get("b_hh"), w_hr)
            h[rows], c[rows] = hn, cn
    grads = {k: np.zeros(np.shape(p[k])) for k in ("w_ih", "w_hh")}
    G = np.shape(p["w_ih"])[0]
    grads["b_ih"] = np.zeros(G)
    grads["b_hh"] = np.zeros(G)
    if w_hr is not None:
        grads["w_hr"] = np.zeros(np.shape(w_hr))
    dx = np.zeros_like(x)
    dh = _f64(dh_n).copy()
    dc = None if c is None else (np.zeros_like(c) if dc_n is None else _f64(dc_n).copy())
    dy = _f64(dy)
    for t, sv in zip(reversed(steps), reversed(saved)):
        if sv is None:
            continue
        rows, hp, cp = sv
        g_h = dh[rows] + dy[t, rows]
        if mode == "gru":
            dxt, dhp = _gru_cell_backward(x[t, rows], hp, p, g_h, grads)
        else:
            dxt, dhp, dcp = _lstm_cell_backward(x[t, rows], hp, cp, p, g_h, dc[rows], grads, w_hr)
            dc[rows] = dcp
        dx[t, rows] = dxt
        dh[rows] = dhp
    return dx, dh, dc, grads


def rnn_backward(mode, x, params, dy, *, dh_n=None, dc_n=None, lengths=None, h0=None, c0=None,
                 num_layers=1, bidirectional=False, proj_size=0, layout="padded"):
    """Gradients of a loss through rnn_forward (same arguments), given
    dy (shape of y), dh_n [L * D, B, K] and dc_n [L * D, B, H] (None = 0).

    Layer l + 1 reads [forward output ; reverse output] of layer l, so the
    gradient w.r.t. layer l's output is the matching half of layer l + 1's
    input gradient. Returns (dx like x, dh0 [L * D, B, K], dc0 [L * D, B, H]
    or None, grads: list over l * D + d of dicts w_ih, w_hh, b_ih, b_hh
    (+ w_hr)).
    """
    if mode not in ("lstm", "lstmp", "gru"):
        raise ValueError(mode)
    D = 2 if bidirectional else 1
    x = _f64(x)
    dy = _f64(dy)
    if layout == "packed":
        T = int(np.max(lengths))
        xp = unpack_sequence(x, lengths, T, fill=0.0)
        dyp = unpack_sequence(dy, lengths, T, fill=0.0)
    else:
        xp, dyp = x, np.nan_to_num(dy)
        T = xp.shape[0]
    B = xp.shape[1]
    H = params[0]["w_hh"].shape[0] // (3 if mode == "gru" else 4)
    K = proj_size if mode == "lstmp" else H
    h0 = np.zeros((num_layers * D, B, K)) if h0 is None else _f64(h0)
    c0 = None if mode == "gru" else (np.zeros((num_layers * D, B, H)) if c0 is None else _f64(c0))
    dh_n = np.zeros((num_layers * D, B, K)) if dh_n is None else _f64(dh_n)
    dc_n = None if mode == "gru" else (np.zeros((num_layers * D, B, H)) if dc_n is None else _f64(dc_n))
    # layer inputs from a forward pass (unwritten positions as zeros)
    inputs = [xp]
    for layer in range(num_layers - 1):
        outs = []
        for d in range(D):
            idx = layer * D + d
            out, _, _ = run_direction(mode, inputs[-1], lengths, h0[idx], None if c0 is None else c0[idx],
                                      params[idx], reverse=(d == 1))
            outs.append(np.nan_to_num(out))
        inputs.append(np.concatenate(outs, axis=2))
    grads = [None] * (num_layers * D)
    dh0 = np.zeros_like(h0)
    dc0 = None if c0 is None else np.zeros_like(c0)
    d_out = dyp
    for layer in range(num_layers - 1, -1, -1):
        d_in = np.zeros_like(inputs[layer])
        for d in range(D):
            idx = layer * D + d
            dx, dh, dc, g = run_direction_backward(
                mode, inputs[layer], lengths, h0[idx], None if c0 is None else c0[idx], params[idx],
                d_out[:, :, d * K:(d + 1) * K], dh_n[idx], None if dc_n is None else dc_n[idx],
                reverse=(d == 1))
            d_in += dx
            dh0[idx] = dh
            if dc0 is not None:
                dc0[idx] = dc
            grads[idx] = g
        d_out = d_in
    dx = d_out
    if layout == "packed":
        dx = pack_sequence(dx, lengths)
    return dx, dh0, dc0, grads
