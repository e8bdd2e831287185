"""The synthetic workloads carry the shapes the pages print."""

import json
import os

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_workloads.json")


def _load():
    with open(GOLDEN) as f:
        return json.load(f)


def test_tvm_benchmark_shapes():
    g = _load()["tvm_lstm_benchmark"]["cases"]
    for case, name in zip(g, ("lstm_t80_b1", "lstm_t256_b1_small")):
        s = synth.spec(name)
        assert (s.T, s.B, s.input_size, s.hidden_size) == (
            case["seq_len"], case["batch_size"], case["in_dim"], case["hidden_dim"])
        assert s.mode == "lstm" and s.num_layers == 1 and not s.bidirectional
        # throughput the pages' timings imply (timestep*batch per second)
        assert case["seq_len"] * case["batch_size"] / (case["te_scan_mean_ms"] * 1e-3) > 1000


def test_rssm_defaults():
    g = _load()["rssm_prior_defaults"]
    s = synth.spec("rssm_b50_t50")
    assert (s.embed_dim, s.belief_dim, s.state_dim) == (g["hidden_dim"], g["rnn_hidden_dim"], g["state_dim"])
    d = synth.make_inputs("rssm_b50_t50")
    assert d["actions"].shape == (50, 50, 6) and d["eps"].shape == (50, 50, 20)
    assert d["weights"]["w_as"].shape == (g["hidden_dim"], g["state_dim"] + 6)
    assert d["weights"]["w_2"].shape == (2 * g["state_dim"], g["hidden_dim"])


def test_varlen_workload_statistics():
    d = synth.make_inputs("bilstm_varlen_b64")
    L = d["lengths"]
    assert L.shape == (64,) and L.min() >= 50 and L.max() <= 500
    assert (L[:-1] >= L[1:]).all()
    assert int(L.sum()) == d["x"].shape[0]
