"""Plain, slow, float64 CPU oracle for the multi-timestep recurrences.

TEST INFRASTRUCTURE ONLY. This package defines what the GPU library must
compute, so that parity tests can compare the two element by element. Only
the test suite (``tests/``), the smoke check in ``__graft_entry__.py`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call it. The product path
(``gru_sequence_scan_amd``) never imports it, and it imports nothing from the
product path: the two share no code. The seeded input generators in
``synth/`` hold none of the method's arithmetic and are the only module both
sides use.

Every function here is the plain definition of the cell it names, evaluated
one timestep at a time, with the input projection computed inside the step
(no hoisting, no fusion, no reordering beyond what the definition states).

Sources (web pages; cited by title and section):
  * pytorch/rl issue "[Feature Request] CUDNN version of RSSM", Solution
    (the RSSMPrior module, the first unroll loop with actions given, and the
    second with an actor computing each action on the fly).
  * pytorch/pytorch issue "Integrating CuDNN API for LSTMs with projections"
    (LSTM with projections = LSTMCell plus one matmul on the hidden output;
    projection is an LSTM-only option; with- and without-bias cases).
  * apache/mxnet issue "RNN Op Changes (was: Variable Length Support for cuDNN
    RNN)", opening RFC (per-sequence lengths, sorted packed layout,
    bidirectional runs that masking cannot fake) and the later discussion
    (cell clipping in cuDNN v7.2; requests for state and projection
    clipping).
  * apache/tvm PR "[TOPI] TE implementation of LSTM using scan", description
    (input-hidden, hidden-hidden and hidden-projection dense ops; the
    recurrence is a true sequential loop).

Readings the pages leave open (gate order and equations, GRU reset-gate
bias placement, NormalParamWrapper scale map, ELU/softplus constants,
var-len reverse start) follow PyTorch's documented nn.LSTM / nn.GRU /
nn.GRUCell conventions and are listed in the design notes.

Pins: every function is checked by the not-gpu tests against closed forms,
invariants and library special cases (torch CPU float64 modules); see
tests/test_oracle_pins.py.
"""

from .rnn import (  # noqa: F401
    sigmoid, elu, softplus, clip, lstm_cell, gru_cell, run_direction, rnn_forward, rnn_backward,
    run_direction_backward,
    pack_sequence, unpack_sequence, packed_offsets, round_to_bf16,
)
from .rssm import rssm_prior_step, rssm_prior_unroll, actor_mlp, rssm_actor_unroll  # noqa: F401
