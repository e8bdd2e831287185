"""Seeded synthetic inputs for the recurrence workloads.

This module holds no arithmetic of the method: it only draws weights, inputs,
initial states and lengths with NumPy's PCG64 generator, casts them to the
storage precision and lays them out. Both the CPU oracle (via the tests and
the bench's CPU leg) and the GPU path consume exactly these arrays, so the
two see identical bits.

Workloads (named by what they are):
  lstm_t80_b1      single-layer LSTM, fp32, T=80, B=1, in 512, hidden 256
                   (the TVM TE-scan vs Relay benchmark shape, apache/tvm PR
                   "[TOPI] TE implementation of LSTM using scan", thread)
  rssm_b50_t50     RSSM-prior unroll, fp32, B=50, T=50, action 6, state 20,
                   hidden 200, GRU hidden 200 (pytorch/rl issue "CUDNN
                   version of RSSM", RSSMPrior defaults)
  gru_t256_b256    single-layer GRU, bf16 storage, T=256, B=256, 512/512
  lstmp_t1000_b32  2-layer LSTMP, bf16 storage, T=1000, B=32, in 320,
                   hidden 1024, projection 256
  bilstm_varlen_b64  2-layer bidirectional LSTM on packed var-len batches,
                   fp32, B=64, L_b ~ U{50..500} sorted descending, in 256,
                   hidden 512 per direction
  lstm_t256_b1_small  the TVM thread's second shape: T=256, B=1, in 16, h 16
  rssm_actor_b50_h50  the same issue's second unroll: the RSSM prior with a
                   synthetic actor (hidden 200) choosing each action from
                   the previous state and belief, B=50, horizon 50

Draw order per workload (one ``np.random.default_rng(seed)``): lengths (var-len
only); weights in parameter order (layer-major, forward before reverse; w_ih,
w_hh, b_ih, b_hh, then w_hr); x; h0, c0; then actions and eps (RSSM).
Values are drawn in float64, cast to float32 and, for bf16 workloads, rounded
to bfloat16 (nearest, ties to even) and carried as float32 arrays whose
values are exactly representable in bf16.
"""

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = [
    "Spec", "WORKLOADS", "spec", "make_rnn_inputs", "make_rssm_inputs",
    "make_inputs", "bf16_round", "bf16_bits", "packed_layout",
]


@dataclass(frozen=True)
class Spec:
    name: str
    mode: str                 # 'lstm' | 'gru' | 'lstmp' | 'rssm'
    dtype: str                # 'f32' | 'bf16'
    T: int = 1
    B: int = 1
    input_size: int = 0
    hidden_size: int = 0
    proj_size: int = 0
    num_layers: int = 1
    bidirectional: bool = False
    layout: str = "padded"    # 'padded' | 'packed' | 'batch_major'
    varlen: Optional[tuple] = None   # (lo, hi) inclusive length range
    w_scale: float = 0.0      # U(-w_scale, w_scale) for every weight and bias
    h0_std: float = 0.0       # N(0, h0_std^2) initial state, 0 = zeros
    seed: int = 0
    # RSSM dimensions
    state_dim: int = 0
    action_dim: int = 0
    embed_dim: int = 0
    belief_dim: int = 0
    actor_dim: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def tokens(self):
        return None


WORKLOADS = {
    "lstm_t80_b1": Spec("lstm_t80_b1", "lstm", "f32", T=80, B=1, input_size=512,
                        hidden_size=256, w_scale=1.0 / 16.0, seed=1001),
    "rssm_b50_t50": Spec("rssm_b50_t50", "rssm", "f32", T=50, B=50, layout="batch_major",
                         state_dim=20, action_dim=6, embed_dim=200, belief_dim=200, seed=1002),
    "gru_t256_b256": Spec("gru_t256_b256", "gru", "bf16", T=256, B=256, input_size=512,
                          hidden_size=512, w_scale=1.0 / np.sqrt(512.0), h0_std=0.1, seed=1003),
    "lstmp_t1000_b32": Spec("lstmp_t1000_b32", "lstmp", "bf16", T=1000, B=32, input_size=320,
                            hidden_size=1024, proj_size=256, num_layers=2,
                            w_scale=1.0 / np.sqrt(1024.0), seed=1004),
    "bilstm_varlen_b64": Spec("bilstm_varlen_b64", "lstm", "f32", T=500, B=64, input_size=256,
                              hidden_size=512, num_layers=2, bidirectional=True, layout="packed",
                              varlen=(50, 500), w_scale=1.0 / np.sqrt(512.0), seed=1005),
    "lstm_t256_b1_small": Spec("lstm_t256_b1_small", "lstm", "f32", T=256, B=1, input_size=16,
                               hidden_size=16, w_scale=0.25, seed=1006),
    "rssm_actor_b50_h50": Spec("rssm_actor_b50_h50", "rssm_actor", "f32", T=50, B=50, layout="batch_major",
                               state_dim=20, action_dim=6, embed_dim=200, belief_dim=200, actor_dim=200,
                               seed=1007),
}

# The five headline workloads in their conventional order (1-based index).
ORDER = ["lstm_t80_b1", "rssm_b50_t50", "gru_t256_b256", "lstmp_t1000_b32", "bilstm_varlen_b64"]


def spec(name_or_index):
    if isinstance(name_or_index, int):
        return WORKLOADS[ORDER[name_or_index - 1]]
    return WORKLOADS[name_or_index]


def bf16_round(a):
    """float32 array -> float32 array rounded to the nearest bf16 value (RNE)."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32).reshape(f.shape)


def bf16_bits(a):
    """bf16-representable float32 array -> uint16 bit patterns (truncation is exact)."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _store(a, dtype):
    a = np.asarray(a, dtype=np.float64).astype(np.float32)
    return bf16_round(a) if dtype == "bf16" else a


def packed_layout(lengths):
    """(batch_sizes[T_max], offsets[T_max+1]) of the step-major packed layout.

    Pure indexing: the rows of step t are the sequences with L_b > t, in batch
    order, starting at offsets[t]. Lengths must be sorted non-increasing.
    """
    L = np.asarray(lengths, dtype=np.int64)
    T = int(L.max())
    counts = np.zeros(T + 1, dtype=np.int64)
    np.add.at(counts, L, 1)
    # batch_sizes[t] = #{b : L_b > t}
    bs = (L.size - np.cumsum(counts))[:T]
    off = np.zeros(T + 1, dtype=np.int64)
    off[1:] = np.cumsum(bs)
    return bs, off


def make_rnn_inputs(mode, T, B, input_size, hidden_size, *, proj_size=0, num_layers=1,
                    bidirectional=False, dtype="f32", layout="padded", lengths=None,
                    varlen=None, w_scale=None, h0_std=0.0, c0_std=0.0, bias=True, seed=0,
                    x_std=1.0):
    """Draw one LSTM / GRU / LSTMP problem.

    Returns a dict with 'params' (list over l * D + d of dicts of float32
    arrays), 'x' (padded [T, B, F] or packed [N_tok, F]), 'x_padded' (padded
    view with NaN padding, var-len only), 'lengths' (int32 [B] or None),
    'h0', 'c0' (float32 or None) and the problem description.
    """
    rng = np.random.default_rng(seed)
    D = 2 if bidirectional else 1
    G = (3 if mode == "gru" else 4) * hidden_size
    K = proj_size if mode == "lstmp" else hidden_size
    if w_scale is None:
        w_scale = 1.0 / np.sqrt(hidden_size)
    if varlen is not None and lengths is None:
        lo, hi = varlen
        lengths = np.sort(rng.integers(lo, hi + 1, size=B))[::-1].astype(np.int32)
    if lengths is not None:
        lengths = np.ascontiguousarray(np.asarray(lengths, dtype=np.int32))
    params = []
    for layer in range(num_layers):
        in_l = input_size if layer == 0 else D * K
        for _d in range(D):
            p = {
                "w_ih": _store(rng.uniform(-w_scale, w_scale, (G, in_l)), dtype),
                "w_hh": _store(rng.uniform(-w_scale, w_scale, (G, K)), dtype),
                "b_ih": _store(rng.uniform(-w_scale, w_scale, (G,)), dtype) if bias else None,
                "b_hh": _store(rng.uniform(-w_scale, w_scale, (G,)), dtype) if bias else None,
            }
            if mode == "lstmp":
                p["w_hr"] = _store(rng.uniform(-w_scale, w_scale, (proj_size, hidden_size)), dtype)
            params.append(p)
    out = {"mode": mode, "T": T, "B": B, "input_size": input_size, "hidden_size": hidden_size,
           "proj_size": proj_size, "num_layers": num_layers, "bidirectional": bidirectional,
           "dtype": dtype, "layout": layout, "lengths": lengths, "params": params}
    if layout == "packed":
        if lengths is None:
            raise ValueError("packed layout needs lengths")
        n_tok = int(np.sum(lengths))
        x = _store(rng.normal(0.0, x_std, (n_tok, input_size)), dtype)
        bs, off = packed_layout(lengths)
        xp = np.full((T, B, input_size), np.nan, dtype=np.float32)
        for t in range(bs.size):
            xp[t, :bs[t]] = x[off[t]:off[t] + bs[t]]
        out["x"] = x
        out["x_padded"] = xp
    else:
        x = _store(rng.normal(0.0, x_std, (T, B, input_size)), dtype)
        if lengths is not None:
            x = x.copy()
            for b in range(B):
                x[lengths[b]:, b] = np.nan
        out["x"] = x
        out["x_padded"] = x
    LD = num_layers * D
    out["h0"] = _store(rng.normal(0.0, h0_std, (LD, B, K)), dtype) if h0_std > 0 else None
    if mode != "gru":
        out["c0"] = _store(rng.normal(0.0, c0_std, (LD, B, hidden_size)), dtype) if c0_std > 0 else None
    else:
        out["c0"] = None
    return out


def make_rssm_inputs(B, T, *, state_dim=20, action_dim=6, embed_dim=200, belief_dim=200,
                     seed=0, s0_std=0.0, h0_std=0.0, zero_weights=False, actor_dim=0):
    """Draw one RSSM-prior unroll problem (float32).

    Every Linear and GRUCell parameter is U(-1/sqrt(fan_in), 1/sqrt(fan_in))
    as PyTorch initialises them (GRUCell uses 1/sqrt(hidden)). Order: w_as,
    b_as, w_ih, w_hh, b_ih, b_hh, w_1, b_1, w_2, b_2, then actions ~ U(-1, 1)
    [B, T, A], eps ~ N(0, 1) [B, T, S].
    actor_dim > 0: the unroll with an actor in the loop (horizon T). The
    actor's w_a1 [actor_dim, S + Hb], b_a1, w_a2 [A, actor_dim], b_a2 are
    drawn after the prior's parameters (same init rule), then eps; no
    actions are drawn ("actions" is None).
    """
    rng = np.random.default_rng(seed)
    S, A, E, Hb = state_dim, action_dim, embed_dim, belief_dim

    def u(shape, fan_in):
        k = 1.0 / np.sqrt(fan_in)
        return rng.uniform(-k, k, shape).astype(np.float32)

    w = {
        "w_as": u((E, S + A), S + A), "b_as": u((E,), S + A),
        "w_ih": u((3 * Hb, E), Hb), "w_hh": u((3 * Hb, Hb), Hb),
        "b_ih": u((3 * Hb,), Hb), "b_hh": u((3 * Hb,), Hb),
        "w_1": u((E, Hb), Hb), "b_1": u((E,), Hb),
        "w_2": u((2 * S, E), E), "b_2": u((2 * S,), E),
    }
    if zero_weights:
        w = {k: np.zeros_like(v) for k, v in w.items()}
    if actor_dim > 0:
        Ea = actor_dim
        aw = {"w_a1": u((Ea, S + Hb), S + Hb), "b_a1": u((Ea,), S + Hb),
              "w_a2": u((A, Ea), Ea), "b_a2": u((A,), Ea)}
        eps = rng.normal(0.0, 1.0, (B, T, S)).astype(np.float32)
        s0 = rng.normal(0.0, s0_std, (B, S)).astype(np.float32) if s0_std > 0 else None
        h0 = rng.normal(0.0, h0_std, (B, Hb)).astype(np.float32) if h0_std > 0 else None
        return {"mode": "rssm_actor", "B": B, "T": T, "state_dim": S, "action_dim": A, "embed_dim": E,
                "belief_dim": Hb, "actor_dim": Ea, "weights": w, "actor": aw, "actions": None,
                "eps": eps, "s0": s0, "h0": h0, "dtype": "f32"}
    actions = rng.uniform(-1.0, 1.0, (B, T, A)).astype(np.float32)
    eps = rng.normal(0.0, 1.0, (B, T, S)).astype(np.float32)
    s0 = rng.normal(0.0, s0_std, (B, S)).astype(np.float32) if s0_std > 0 else None
    h0 = rng.normal(0.0, h0_std, (B, Hb)).astype(np.float32) if h0_std > 0 else None
    return {"mode": "rssm", "B": B, "T": T, "state_dim": S, "action_dim": A, "embed_dim": E,
            "belief_dim": Hb, "weights": w, "actions": actions, "eps": eps, "s0": s0, "h0": h0,
            "dtype": "f32"}


def make_inputs(name_or_index, seed=None):
    """Inputs of a named workload (see the module docstring)."""
    s = spec(name_or_index)
    sd = s.seed if seed is None else seed
    if s.mode in ("rssm", "rssm_actor"):
        return make_rssm_inputs(s.B, s.T, state_dim=s.state_dim, action_dim=s.action_dim,
                                embed_dim=s.embed_dim, belief_dim=s.belief_dim, seed=sd,
                                actor_dim=s.actor_dim)
    return make_rnn_inputs(s.mode, s.T, s.B, s.input_size, s.hidden_size, proj_size=s.proj_size,
                           num_layers=s.num_layers, bidirectional=s.bidirectional, dtype=s.dtype,
                           layout=s.layout, varlen=s.varlen, w_scale=s.w_scale,
                           h0_std=s.h0_std, seed=sd)
