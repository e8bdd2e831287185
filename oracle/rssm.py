"""Float64 oracle: RSSM prior step, its unroll over given actions, and the
unroll with an actor in the loop.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: pytorch/rl issue "[Feature Request] CUDNN version of RSSM",
Solution: the RSSMPrior module's forward and the first unroll (actions of
shape [B, T, A] given, outputs stacked on dim 1). Readings of what the page
leaves open:
  * the action-state projector sees cat([state, action]) on the last axis,
    so W_as columns are state first, then action;
  * the first prior-projector Linear reads the belief, so its in_features is
    the GRU hidden size (the page writes hidden_dim; both are 200 there);
  * NormalParamWrapper(scale_lb=0.1) splits the 2S output into loc (first
    half) and a raw scale mapped as softplus(raw) + scale_lb;
  * ELU has alpha = 1; softplus has beta = 1;
  * randn_like(std) is replaced by an injected eps tensor [B, T, S] so both
    sides see the same draw; the loop's ``action[:, i]`` means actions[:, i];
  * missing state / belief mean zeros (the forward's None branches).

The same issue's second loop computes each action from the previous prior
state and belief with an actor model it does not define. Reading: a
deterministic two-layer MLP in the style of the prior's own projectors,
    a_t = tanh(W_a2 ELU(W_a1 [s_{t-1}; h_{t-1}] + b_a1) + b_a2),
with the inputs concatenated in the call's argument order (state, belief);
tanh bounds the action like the given actions of the first unroll.
"""

import numpy as np

from .rnn import elu, gru_cell, softplus

__all__ = ["rssm_prior_step", "rssm_prior_unroll", "actor_mlp", "rssm_actor_unroll"]


def rssm_prior_step(state, belief, action, eps, w, scale_lb=0.1):
    """One RSSMPrior.forward: returns (mean, std, next_state, belief').

    state [B, S], belief [B, Hb], action [B, A], eps [B, S]. w holds
    w_as [E, S + A], b_as [E], w_ih [3Hb, E], w_hh [3Hb, Hb], b_ih, b_hh,
    w_1 [E1, Hb], b_1 [E1], w_2 [2S, E1], b_2 [2S].
    """
    f = lambda k: None if w.get(k) is None else np.asarray(w[k], dtype=np.float64)
    state = np.asarray(state, dtype=np.float64)
    sa = np.concatenate([state, np.asarray(action, dtype=np.float64)], axis=-1)
    e = elu(sa @ f("w_as").T + f("b_as"))
    belief = gru_cell(e, belief, f("w_ih"), f("w_hh"), f("b_ih"), f("b_hh"))
    u = elu(belief @ f("w_1").T + f("b_1"))
    v = u @ f("w_2").T + f("b_2")
    S = state.shape[-1]
    mean = v[:, :S]
    std = softplus(v[:, S:2 * S]) + scale_lb
    nxt = mean + np.asarray(eps, dtype=np.float64) * std
    return mean, std, nxt, belief


def rssm_prior_unroll(actions, eps, w, state0=None, belief0=None, scale_lb=0.1):
    """Unroll the prior over actions [B, T, A] with injected eps [B, T, S].

    Returns (means, stds, states, beliefs), each stacked on dim 1:
    [B, T, S], [B, T, S], [B, T, S], [B, T, Hb].
    """
    actions = np.asarray(actions, dtype=np.float64)
    eps = np.asarray(eps, dtype=np.float64)
    B, T = actions.shape[0], actions.shape[1]
    S = eps.shape[2]
    Hb = np.asarray(w["w_hh"]).shape[1]
    state = np.zeros((B, S)) if state0 is None else np.asarray(state0, dtype=np.float64)
    belief = np.zeros((B, Hb)) if belief0 is None else np.asarray(belief0, dtype=np.float64)
    means, stds, states, beliefs = [], [], [], []
    for t in range(T):
        mean, std, state, belief = rssm_prior_step(state, belief, actions[:, t], eps[:, t], w, scale_lb)
        means.append(mean)
        stds.append(std)
        states.append(state)
        beliefs.append(belief)
    return (np.stack(means, 1), np.stack(stds, 1), np.stack(states, 1), np.stack(beliefs, 1))


def actor_mlp(state, belief, aw):
    """The synthetic actor: tanh(W_a2 ELU(W_a1 [state; belief] + b_a1) + b_a2).

    state [B, S], belief [B, Hb]; aw holds w_a1 [Ea, S + Hb], b_a1 [Ea],
    w_a2 [A, Ea], b_a2 [A]. Returns the action [B, A].
    """
    f = lambda k: np.asarray(aw[k], dtype=np.float64)
    sh = np.concatenate([np.asarray(state, dtype=np.float64), np.asarray(belief, dtype=np.float64)], axis=-1)
    q = elu(sh @ f("w_a1").T + f("b_a1"))
    return np.tanh(q @ f("w_a2").T + f("b_a2"))


def rssm_actor_unroll(eps, w, aw, state0=None, belief0=None, scale_lb=0.1):
    """Unroll the prior for H = eps.shape[1] steps, each action computed on
    the fly from the previous state and belief (pytorch/rl issue "[Feature
    Request] CUDNN version of RSSM", Solution, second unroll).

    Returns (means, stds, states, beliefs, actions), stacked on dim 1:
    [B, H, S] x 3, [B, H, Hb], [B, H, A].
    """
    eps = np.asarray(eps, dtype=np.float64)
    B, H, S = eps.shape
    Hb = np.asarray(w["w_hh"]).shape[1]
    state = np.zeros((B, S)) if state0 is None else np.asarray(state0, dtype=np.float64)
    belief = np.zeros((B, Hb)) if belief0 is None else np.asarray(belief0, dtype=np.float64)
    outs = [[] for _ in range(5)]
    for t in range(H):
        action = actor_mlp(state, belief, aw)
        mean, std, state, belief = rssm_prior_step(state, belief, action, eps[:, t], w, scale_lb)
        for o, v in zip(outs, (mean, std, state, belief, action)):
            o.append(v)
    return tuple(np.stack(o, 1) for o in outs)
