"""MI355X (gfx950) multi-timestep LSTM / GRU / LSTMP / RSSM-prior forward.

A thin ctypes binding over the C ABI in include/rnn.h. Every step of the
computation runs in the library's HIP kernels; this module only marshals
PyTorch tensors (device memory) and the current HIP stream into the C
structs. There is no CPU fallback: if the native library is missing the
calls raise.

Low level (same names as the C ABI): rnn_abi_version, rnn_strerror,
rnn_workspace_bytes, rnn_forward_raw (= C rnn_forward), rnn_read_status,
rnn_device_check, rnn_plan_info, rnn_exchange_roundtrip_ns. High level: rnn_forward (LSTM / GRU / LSTMP, padded or
packed, multi-layer, bidirectional), rssm_prior_unroll and rssm_actor_unroll; training:
rnn_forward_train and rnn_backward (fp32 LSTM / LSTMP / GRU).
"""

from .binding import (  # noqa: F401
    RNN_ABI_VERSION, RnnDesc, RnnWeights, RnnIO, RnnError, lib, lib_path,
    rnn_abi_version, rnn_strerror, rnn_workspace_bytes, rnn_forward_raw, rnn_read_status,
    rnn_device_check, rnn_exchange_roundtrip_ns, rnn_forward, rssm_prior_unroll, rssm_actor_unroll, rnn_plan_info,
    MODES, PIPE_MODES, STATUS, CLIP_CELL, CLIP_PROJ, RnnGrads, rnn_forward_train, rnn_backward, TrainContext,
)
