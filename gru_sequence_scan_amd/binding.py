"""ctypes binding of include/rnn.h plus tensor marshalling.

Only argument marshalling happens here: shape and dtype checks, re-layout of
tensors whose memory is not C-dense (pytorch/rl PR "LSTM/GRU scan: canonical
strides + ...": a tensor can pass is_contiguous() yet carry strides that a
pointer-based kernel cannot honour), allocation of outputs and workspace
with torch, and the call on torch's current HIP stream.
"""

import ctypes
import os

import torch

RNN_ABI_VERSION = 2
RNN_MAX_LAYERS = 8
RNN_MAX_LD = 2 * RNN_MAX_LAYERS

MODES = {"lstm": 0, "gru": 1, "lstmp": 2, "rssm": 3, "rssm_actor": 4}
PIPE_MODES = {"auto": 0, "off": 1, "on": 2}  # RnnDesc.layer_pipeline
DTYPES = {torch.float32: 0, torch.bfloat16: 1}
LAYOUTS = {"padded": 0, "packed": 1, "batch_major": 2}
STATUS = {
    0: "RNN_OK", -1: "RNN_E_NULL", -2: "RNN_E_SHAPE", -3: "RNN_E_UNSUPPORTED",
    -4: "RNN_E_LENGTHS", -5: "RNN_E_WORKSPACE", -6: "RNN_E_ALIGN", -7: "RNN_E_DEVICE",
    -8: "RNN_E_HIP", -9: "RNN_E_TIMEOUT", -10: "RNN_E_PLAN",
}

CLIP_CELL, CLIP_PROJ = 1, 2

_PKG = os.path.dirname(os.path.abspath(__file__))


def lib_path():
    return os.path.join(_PKG, "_lib", "librnn_gfx950.so")


class RnnDesc(ctypes.Structure):
    _fields_ = [
        ("mode", ctypes.c_int32), ("dtype", ctypes.c_int32), ("layout", ctypes.c_int32),
        ("T", ctypes.c_int32), ("B", ctypes.c_int32), ("input_size", ctypes.c_int32),
        ("hidden_size", ctypes.c_int32), ("proj_size", ctypes.c_int32),
        ("num_layers", ctypes.c_int32), ("bidirectional", ctypes.c_int32),
        ("has_bias", ctypes.c_int32), ("state_dim", ctypes.c_int32),
        ("action_dim", ctypes.c_int32), ("embed_dim", ctypes.c_int32),
        ("belief_dim", ctypes.c_int32), ("scale_lb", ctypes.c_float),
        ("tile_batch", ctypes.c_int32), ("tile_hidden", ctypes.c_int32),
        ("placement", ctypes.c_int32), ("weights", ctypes.c_int32),
        ("clip", ctypes.c_int32), ("cell_clip_lo", ctypes.c_float), ("cell_clip_hi", ctypes.c_float),
        ("proj_clip", ctypes.c_float), ("actor_dim", ctypes.c_int32), ("gx_dtype", ctypes.c_int32),
        ("layer_pipeline", ctypes.c_int32), ("reserved", ctypes.c_int32 * 1),
    ]


_PtrArr = ctypes.c_void_p * RNN_MAX_LD


class RnnWeights(ctypes.Structure):
    _fields_ = [
        ("w_ih", _PtrArr), ("w_hh", _PtrArr), ("b_ih", _PtrArr), ("b_hh", _PtrArr),
        ("w_hr", _PtrArr), ("w_as", ctypes.c_void_p), ("b_as", ctypes.c_void_p),
        ("w_1", ctypes.c_void_p), ("b_1", ctypes.c_void_p), ("w_2", ctypes.c_void_p),
        ("b_2", ctypes.c_void_p), ("w_a1", ctypes.c_void_p), ("b_a1", ctypes.c_void_p),
        ("w_a2", ctypes.c_void_p), ("b_a2", ctypes.c_void_p),
    ]


class RnnIO(ctypes.Structure):
    _fields_ = [
        ("x", ctypes.c_void_p), ("lengths_host", ctypes.POINTER(ctypes.c_int32)),
        ("h0", ctypes.c_void_p), ("c0", ctypes.c_void_p), ("s0", ctypes.c_void_p),
        ("noise", ctypes.c_void_p), ("y", ctypes.c_void_p), ("h_n", ctypes.c_void_p),
        ("c_n", ctypes.c_void_p), ("means", ctypes.c_void_p), ("stds", ctypes.c_void_p),
        ("states", ctypes.c_void_p), ("beliefs", ctypes.c_void_p), ("actions", ctypes.c_void_p),
    ]


class RnnGrads(ctypes.Structure):
    _fields_ = [
        ("dy", ctypes.c_void_p), ("dh_n", ctypes.c_void_p), ("dc_n", ctypes.c_void_p),
        ("dx", ctypes.c_void_p), ("dh0", ctypes.c_void_p), ("dc0", ctypes.c_void_p),
        ("dw_ih", _PtrArr), ("dw_hh", _PtrArr), ("db_ih", _PtrArr), ("db_hh", _PtrArr),
        ("dw_hr", _PtrArr),
    ]


class RnnError(RuntimeError):
    def __init__(self, status, where=""):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({rnn_strerror(status)})")


_lib = None


def lib():
    """Load the native library once; raise if it has not been built."""
    global _lib
    if _lib is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"native library {path} is missing; build it with "
                               "`python -m gru_sequence_scan_amd.build`")
        L = ctypes.CDLL(path)
        L.rnn_abi_version.restype = ctypes.c_int
        L.rnn_abi_version.argtypes = []
        L.rnn_strerror.restype = ctypes.c_char_p
        L.rnn_strerror.argtypes = [ctypes.c_int]
        L.rnn_workspace_bytes.restype = ctypes.c_int
        L.rnn_workspace_bytes.argtypes = [ctypes.POINTER(RnnDesc), ctypes.POINTER(ctypes.c_int32),
                                          ctypes.POINTER(ctypes.c_size_t)]
        L.rnn_forward.restype = ctypes.c_int
        L.rnn_forward.argtypes = [ctypes.POINTER(RnnDesc), ctypes.POINTER(RnnWeights),
                                  ctypes.POINTER(RnnIO), ctypes.c_void_p, ctypes.c_size_t,
                                  ctypes.c_void_p]
        L.rnn_read_status.restype = ctypes.c_int
        L.rnn_read_status.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(ctypes.c_int)]
        L.rnn_device_check.restype = ctypes.c_int
        L.rnn_device_check.argtypes = []
        L.rnn_plan_info.restype = ctypes.c_int
        L.rnn_plan_info.argtypes = [ctypes.POINTER(RnnDesc), ctypes.POINTER(ctypes.c_int32), ctypes.c_int,
                                    ctypes.c_int, ctypes.POINTER(ctypes.c_int), ctypes.c_int]
        for nm in ("rnn_reserve_bytes", "rnn_backward_workspace_bytes"):
            getattr(L, nm).restype = ctypes.c_int
            getattr(L, nm).argtypes = [ctypes.POINTER(RnnDesc), ctypes.POINTER(ctypes.c_int32),
                                       ctypes.POINTER(ctypes.c_size_t)]
        L.rnn_forward_train.restype = ctypes.c_int
        L.rnn_forward_train.argtypes = [ctypes.POINTER(RnnDesc), ctypes.POINTER(RnnWeights), ctypes.POINTER(RnnIO),
                                        ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t,
                                        ctypes.c_void_p]
        L.rnn_backward.restype = ctypes.c_int
        L.rnn_backward.argtypes = [ctypes.POINTER(RnnDesc), ctypes.POINTER(RnnWeights), ctypes.POINTER(RnnIO),
                                   ctypes.POINTER(RnnGrads), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                   ctypes.c_size_t, ctypes.c_void_p]
        L.rnn_forward_noalloc.restype = ctypes.c_int
        L.rnn_forward_noalloc.argtypes = [ctypes.POINTER(RnnDesc), ctypes.POINTER(RnnWeights),
                                          ctypes.POINTER(RnnIO), ctypes.c_void_p, ctypes.c_void_p]
        L.rnn_exchange_roundtrip_ns.restype = ctypes.c_int
        L.rnn_exchange_roundtrip_ns.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                                ctypes.POINTER(ctypes.c_double)]
        if L.rnn_abi_version() != RNN_ABI_VERSION:
            raise RuntimeError("native library ABI version mismatch")
        _lib = L
    return _lib


# ---------------------------------------------------------------------------
# Raw C entry points
# ---------------------------------------------------------------------------

def rnn_abi_version():
    return lib().rnn_abi_version()


def rnn_strerror(status):
    return lib().rnn_strerror(int(status)).decode()


def _len_ptr(lengths, B):
    """A C int32 array of the B sequence lengths (None stays None). The C
    side reads exactly B ints, so a list of any other length is refused here
    instead of being read past its end."""
    if lengths is None:
        return None, None
    vals = [int(v) for v in lengths]
    if len(vals) != int(B):
        raise ValueError(f"lengths: {len(vals)} values for a batch of {int(B)} rows")
    arr = (ctypes.c_int32 * len(vals))(*vals)
    return arr, ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))


def rnn_workspace_bytes(desc, lengths=None):
    keep, lp = _len_ptr(lengths, desc.B)
    n = ctypes.c_size_t(0)
    st = lib().rnn_workspace_bytes(ctypes.byref(desc), lp, ctypes.byref(n))
    if st != 0:
        raise RnnError(st, "rnn_workspace_bytes")
    return n.value


def rnn_forward_raw(desc, weights, io, workspace_ptr, ws_bytes, stream_ptr):
    """Direct call of the C rnn_forward; returns the status code."""
    return lib().rnn_forward(ctypes.byref(desc), ctypes.byref(weights), ctypes.byref(io),
                             ctypes.c_void_p(workspace_ptr), ctypes.c_size_t(ws_bytes),
                             ctypes.c_void_p(stream_ptr))


PLAN_FIELDS = ("kernel", "workgroups", "lds_bytes", "rows", "hidden_per_wg", "members", "proj_per_wg",
               "groups", "groups_per_xcd", "wreg", "reg_tiles", "reg_ksplit", "reg_chunks", "pipe_chunk",
               "model_step_ns")


def rnn_plan_info(desc, lengths=None, cus=256, xcds=8):
    """The launch shape the library would choose on a device with `cus`
    compute units in `xcds` XCDs (host only), as a dict of PLAN_FIELDS."""
    keep, lp = _len_ptr(lengths, desc.B)
    info = (ctypes.c_int * len(PLAN_FIELDS))()
    st = lib().rnn_plan_info(ctypes.byref(desc), lp, int(cus), int(xcds), info, len(PLAN_FIELDS))
    if st != 0:
        raise RnnError(st, "rnn_plan_info")
    return dict(zip(PLAN_FIELDS, list(info)))


def rnn_read_status(workspace_ptr, stream_ptr):
    """Synchronise the stream and return the device status word of the last
    call that used this workspace (0, or RNN_E_TIMEOUT = -9)."""
    v = ctypes.c_int(0)
    st = lib().rnn_read_status(ctypes.c_void_p(workspace_ptr), ctypes.c_void_p(stream_ptr), ctypes.byref(v))
    if st != 0:
        raise RnnError(st, "rnn_read_status")
    return v.value


def rnn_device_check():
    return lib().rnn_device_check()


def rnn_exchange_roundtrip_ns(iters=2000, device="cuda:0"):
    """Mean nanoseconds of one device-coherent round trip between two
    workgroups on different XCDs (C rnn_exchange_roundtrip_ns)."""
    buf = torch.empty(1024, dtype=torch.uint8, device=device)
    v = ctypes.c_double(0.0)
    st = lib().rnn_exchange_roundtrip_ns(buf.data_ptr(), buf.numel(), int(iters), _stream_ptr(torch.device(device)),
                                         ctypes.byref(v))
    if st != 0:
        raise RnnError(st, "rnn_exchange_roundtrip_ns")
    return v.value


# ---------------------------------------------------------------------------
# Tensor marshalling
# ---------------------------------------------------------------------------

def _c_dense(t):
    """True when the memory of t is laid out in C order (strides of size-1
    dimensions do not matter to a pointer-based kernel)."""
    expect = 1
    for size, stride in zip(reversed(t.shape), reversed(t.stride())):
        if size != 1 and stride != expect:
            return False
        expect *= size
    return True


def _dense(t):
    if t is None:
        return None
    if _c_dense(t):
        return t
    out = torch.empty(t.shape, dtype=t.dtype, device=t.device)
    out.copy_(t)
    return out


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream_ptr(device):
    return torch.cuda.current_stream(device).cuda_stream


def _check(t, name, shape, dtype, device):
    if t is None:
        return None
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype} != {dtype}")
    if t.device != device:
        raise ValueError(f"{name}: device {t.device} != {device}")
    return _dense(t)


def check_device_status(ws, device, where):
    """Wait for the stream and raise RnnError when the kernels that used
    workspace `ws` reported a device-side failure (a step barrier's watchdog:
    RNN_E_TIMEOUT), whose outputs are invalid."""
    st = rnn_read_status(ws.data_ptr(), _stream_ptr(device))
    if st != 0:
        raise RnnError(st, where + " (device status)")


RNN_NOALLOC_MAX_WORKSPACE = 32 << 20


def _call_noalloc(desc, w, io, device, check_status):
    """C rnn_forward_noalloc: the library's own workspace, the device status
    copied into a one-int tensor."""
    status = torch.zeros(1, dtype=torch.int32, device=device)
    st = lib().rnn_forward_noalloc(ctypes.byref(desc), ctypes.byref(w), ctypes.byref(io), _stream_ptr(device),
                                   ctypes.c_void_p(status.data_ptr()))
    if st != 0:
        raise RnnError(st, "rnn_forward_noalloc")
    if check_status:
        v = int(status.item())
        if v != 0:
            raise RnnError(v, "rnn_forward_noalloc (device status)")
    return status


def _call(desc, w, io, lengths, device, keep, check_status, noalloc=False):
    if noalloc:
        return _call_noalloc(desc, w, io, device, check_status)
    ws_bytes = rnn_workspace_bytes(desc, lengths)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=device)
    keep.append(ws)
    st = rnn_forward_raw(desc, w, io, ws.data_ptr(), ws.numel(), _stream_ptr(device))
    if st != 0:
        raise RnnError(st, "rnn_forward")
    if check_status:
        check_device_status(ws, device, "rnn_forward")
    return ws


def rnn_forward(mode, x, params, *, h0=None, c0=None, lengths=None, layout="padded",
                num_layers=1, bidirectional=False, proj_size=0, hidden_size=None, y_out=None,
                tile_batch=0, tile_hidden=0, placement=0, weights=0, cell_clip=None, proj_clip=None,
                gx_dtype="auto", layer_pipeline="auto", return_workspace=False, check_status=True,
                noalloc=False, _train=False):
    """Forward of an LSTM / GRU / LSTMP stack on the current HIP stream.

    x: padded [T, B, F] or packed [N_tok, F] (float32 or bfloat16, on a GPU).
    params: list over layer * D + direction of dicts with 'w_ih' [G, in_l],
    'w_hh' [G, K], optional 'b_ih', 'b_hh' [G] and, for LSTMP, 'w_hr' [P, H].
    lengths: host sequence of B ints (required for packed; for padded it
    masks rows, which are then never written past their length).
    cell_clip: c (clamp to [-c, c]) or (lo, hi), clamps the updated LSTM cell
    state; proj_clip: p, clamps the LSTMP projected output to [-p, p].
    gx_dtype: "auto" stores the hoisted input projection in x's dtype, "f32"
    always in fp32. layer_pipeline: "auto" scans a unidirectional padded
    stack's layers concurrently, one time chunk apart, where the launch-shape
    model expects a gain; "off" runs it layer by layer; "on" pipelines it
    whenever it fits (the results are the same bit for bit).
    check_status (default True): wait for the stream after the call and
    raise RnnError if the device reported a failure (a persistent group whose
    workgroups were not all resident ends with RNN_E_TIMEOUT and leaves the
    outputs invalid). With False the call stays asynchronous and the caller
    checks rnn_read_status on the returned workspace (return_workspace=True).
    noalloc: call rnn_forward_noalloc (the library's own workspace, for
    problems up to RNN_NOALLOC_MAX_WORKSPACE bytes); the returned
    "workspace" is then the one-int device status tensor.
    Returns (y, h_n, c_n) with c_n None for GRU.
    """
    mode = mode.lower()
    if mode not in ("lstm", "gru", "lstmp"):
        raise ValueError(f"mode {mode!r}")
    if lengths is not None:
        lengths = [int(v) for v in (lengths.tolist() if hasattr(lengths, "tolist") else lengths)]
        if layout == "padded" and x.dim() == 3 and len(lengths) != x.shape[1]:
            raise ValueError(f"lengths: {len(lengths)} values for a batch of {x.shape[1]} rows")
    dtype, device = x.dtype, x.device
    if dtype not in DTYPES:
        raise ValueError(f"dtype {dtype} not supported (float32, bfloat16)")
    if device.type != "cuda":
        raise ValueError("x must be a GPU tensor")
    D = 2 if bidirectional else 1
    LD = num_layers * D
    if len(params) != LD:
        raise ValueError(f"expected {LD} parameter sets, got {len(params)}")
    gates = 3 if mode == "gru" else 4
    H = params[0]["w_hh"].shape[0] // gates if hidden_size is None else hidden_size
    K = proj_size if mode == "lstmp" else H
    F = x.shape[-1]
    if layout not in ("padded", "packed"):
        raise ValueError(f"layout {layout!r}")
    if layout == "packed":
        if lengths is None:
            raise ValueError("packed layout needs lengths")
        B = len(lengths)
        T = max(lengths)
        n_tok = sum(lengths)
        x = _check(x, "x", (n_tok, F), dtype, device)
        y_shape = (n_tok, D * K)
    else:
        if x.dim() != 3:
            raise ValueError(f"x: padded layout needs [T, B, F], got shape {tuple(x.shape)}")
        T, B = x.shape[0], x.shape[1]
        if lengths is not None and len(lengths) != B:
            raise ValueError(f"lengths: {len(lengths)} values for a batch of {B} rows")
        x = _check(x, "x", (T, B, F), dtype, device)
        y_shape = (T, B, D * K)
    has_bias = params[0].get("b_ih") is not None
    keep = [x]
    w = RnnWeights()
    for i, p in enumerate(params):
        in_l = F if i < D else D * K
        pw = {"w_ih": (gates * H, in_l), "w_hh": (gates * H, K)}
        if has_bias:
            pw.update({"b_ih": (gates * H,), "b_hh": (gates * H,)})
        if mode == "lstmp":
            pw["w_hr"] = (proj_size, H)
        for name, shp in pw.items():
            t = _check(p[name], f"params[{i}].{name}", shp, dtype, device)
            keep.append(t)
            getattr(w, name)[i] = _ptr(t)
    h0 = _check(h0, "h0", (LD, B, K), dtype, device)
    c0 = _check(c0, "c0", (LD, B, H), dtype, device) if mode != "gru" else None
    keep += [h0, c0]
    if y_out is None:
        y = torch.empty(y_shape, dtype=dtype, device=device)
    else:
        if tuple(y_out.shape) != y_shape or y_out.dtype != dtype or not _c_dense(y_out):
            raise ValueError("y_out must be a C-dense tensor of the output shape and dtype")
        y = y_out
    h_n = torch.empty((LD, B, K), dtype=dtype, device=device)
    c_n = torch.empty((LD, B, H), dtype=dtype, device=device) if mode != "gru" else None

    desc = RnnDesc()
    desc.mode = MODES[mode]
    desc.dtype = DTYPES[dtype]
    desc.layout = LAYOUTS[layout]
    desc.T, desc.B = T, B
    desc.input_size, desc.hidden_size, desc.proj_size = F, H, proj_size if mode == "lstmp" else 0
    desc.num_layers, desc.bidirectional, desc.has_bias = num_layers, int(bidirectional), int(has_bias)
    desc.tile_batch, desc.tile_hidden, desc.placement = tile_batch, tile_hidden, placement
    desc.weights = weights
    if gx_dtype not in ("auto", "f32"):
        raise ValueError("gx_dtype must be 'auto' or 'f32'")
    desc.gx_dtype = 1 if gx_dtype == "f32" else 0
    if layer_pipeline not in PIPE_MODES:
        raise ValueError("layer_pipeline must be 'auto', 'off' or 'on'")
    desc.layer_pipeline = PIPE_MODES[layer_pipeline]
    if cell_clip is not None:
        lo, hi = (-cell_clip, cell_clip) if isinstance(cell_clip, (int, float)) else cell_clip
        desc.clip |= CLIP_CELL
        desc.cell_clip_lo, desc.cell_clip_hi = float(lo), float(hi)
    if proj_clip is not None:
        desc.clip |= CLIP_PROJ
        desc.proj_clip = float(proj_clip)
    io = RnnIO()
    io.x = _ptr(x)
    keep_len, io.lengths_host = _len_ptr(lengths, B)
    io.h0, io.c0 = _ptr(h0), _ptr(c0)
    io.y, io.h_n, io.c_n = _ptr(y), _ptr(h_n), _ptr(c_n)
    out = (y, h_n, c_n)
    if _train:
        n = ctypes.c_size_t(0)
        st = lib().rnn_reserve_bytes(ctypes.byref(desc), io.lengths_host, ctypes.byref(n))
        if st != 0:
            raise RnnError(st, "rnn_reserve_bytes")
        reserve = torch.empty(max(n.value, 256), dtype=torch.uint8, device=device)
        ws_bytes = rnn_workspace_bytes(desc, lengths)
        ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=device)
        st = lib().rnn_forward_train(ctypes.byref(desc), ctypes.byref(w), ctypes.byref(io), reserve.data_ptr(),
                                     reserve.numel(), ws.data_ptr(), ws.numel(), _stream_ptr(device))
        if st != 0:
            raise RnnError(st, "rnn_forward_train")
        if check_status:
            check_device_status(ws, device, "rnn_forward_train")
        ctx = TrainContext(desc, w, io, keep + [keep_len, y, h_n, c_n], reserve, lengths, mode, params, D, H, K)
        return out, ctx
    ws = _call(desc, w, io, lengths, device, keep, check_status, noalloc)
    return (out, ws) if return_workspace else out


class TrainContext:
    """What rnn_backward needs from rnn_forward_train: the C structs of that
    call, the tensors they point to (kept alive here) and the reserve."""

    def __init__(self, desc, w, io, keep, reserve, lengths, mode, params, D, H, K):
        self.desc, self.w, self.io, self.keep, self.reserve = desc, w, io, keep, reserve
        self.lengths, self.mode, self.params, self.D, self.H, self.K = lengths, mode, params, D, H, K


def rnn_forward_train(mode, x, params, **kw):
    """rnn_forward that also keeps what the backward needs (fp32 LSTM / LSTMP / GRU).
    Returns ((y, h_n, c_n), ctx); pass ctx to rnn_backward."""
    return rnn_forward(mode, x, params, _train=True, **kw)


def rnn_backward(ctx, dy, dh_n=None, dc_n=None, check_status=True):
    """Gradients through the forward recorded in ctx, given dy (shape of y)
    and optionally dh_n, dc_n (shape of h_n, c_n). Returns (dx, dh0, dc0,
    grads) with grads a list over layer * D + direction of dicts dw_ih,
    dw_hh, db_ih, db_hh (bias entries only with biases) and dw_hr (LSTMP);
    dc0 None for GRU. check_status as for rnn_forward."""
    y = ctx.keep[-3]
    device, dtype = y.device, y.dtype
    desc, io = ctx.desc, ctx.io
    LD = desc.num_layers * ctx.D
    B, H, K = desc.B, ctx.H, ctx.K
    dy = _check(dy, "dy", tuple(y.shape), dtype, device)
    dh_n = _check(dh_n, "dh_n", (LD, B, K), dtype, device)
    dc_n = _check(dc_n, "dc_n", (LD, B, H), dtype, device) if ctx.mode != "gru" else None
    x = ctx.keep[0]
    dx = torch.empty_like(x)
    dh0 = torch.empty((LD, B, K), dtype=dtype, device=device)
    dc0 = torch.empty((LD, B, H), dtype=dtype, device=device) if ctx.mode != "gru" else None
    g = RnnGrads()
    g.dy, g.dh_n, g.dc_n = _ptr(dy), _ptr(dh_n), _ptr(dc_n)
    g.dx, g.dh0, g.dc0 = _ptr(dx), _ptr(dh0), _ptr(dc0)
    grads = []
    for i, p in enumerate(ctx.params):
        gi = {"dw_ih": torch.empty_like(p["w_ih"]), "dw_hh": torch.empty_like(p["w_hh"])}
        if desc.has_bias:
            gi["db_ih"] = torch.empty_like(p["b_ih"])
            gi["db_hh"] = torch.empty_like(p["b_hh"])
        if ctx.mode == "lstmp":
            gi["dw_hr"] = torch.empty_like(p["w_hr"])
        for k, t in gi.items():
            getattr(g, k)[i] = t.data_ptr()
        grads.append(gi)
    n = ctypes.c_size_t(0)
    st = lib().rnn_backward_workspace_bytes(ctypes.byref(desc), io.lengths_host, ctypes.byref(n))
    if st != 0:
        raise RnnError(st, "rnn_backward_workspace_bytes")
    ws = torch.empty(max(n.value, 256), dtype=torch.uint8, device=device)
    st = lib().rnn_backward(ctypes.byref(desc), ctypes.byref(ctx.w), ctypes.byref(io), ctypes.byref(g),
                            ctx.reserve.data_ptr(), ctx.reserve.numel(), ws.data_ptr(), ws.numel(),
                            _stream_ptr(device))
    if st != 0:
        raise RnnError(st, "rnn_backward")
    if check_status:
        check_device_status(ws, device, "rnn_backward")
    ctx.bwd_workspace = ws
    return dx, dh0, dc0, grads


def _rssm(mode, actions, eps, weights, actor, A, state0, belief0, scale_lb, tile_batch, tile_hidden,
          placement, check_status, noalloc=False, weights_hint=0):
    """Marshal one RSSM unroll (given actions, or an actor) into the C ABI."""
    dtype, device = eps.dtype, eps.device
    if dtype != torch.float32:
        raise ValueError("the RSSM prior runs in float32")
    B, T, S = eps.shape
    E, SA = weights["w_as"].shape
    Hb = weights["w_hh"].shape[1]
    if SA != S + A:
        raise ValueError("w_as must have S + A columns")
    shapes = {"w_as": (E, S + A), "b_as": (E,), "w_ih": (3 * Hb, E), "w_hh": (3 * Hb, Hb),
              "b_ih": (3 * Hb,), "b_hh": (3 * Hb,), "w_1": (E, Hb), "b_1": (E,),
              "w_2": (2 * S, E), "b_2": (2 * S,)}
    wt = {k: _check(weights[k], k, s, dtype, device) for k, s in shapes.items()}
    Ea = 0
    if actor is not None:
        Ea = actor["w_a1"].shape[0]
        ashapes = {"w_a1": (Ea, S + Hb), "b_a1": (Ea,), "w_a2": (A, Ea), "b_a2": (A,)}
        wt.update({k: _check(actor[k], k, s, dtype, device) for k, s in ashapes.items()})
    if actions is not None:
        actions = _check(actions, "actions", (B, T, A), dtype, device)
    eps = _check(eps, "eps", (B, T, S), dtype, device)
    state0 = _check(state0, "state0", (B, S), dtype, device)
    belief0 = _check(belief0, "belief0", (B, Hb), dtype, device)
    keep = [actions, eps, state0, belief0] + list(wt.values())
    w = RnnWeights()
    w.w_as, w.b_as = _ptr(wt["w_as"]), _ptr(wt["b_as"])
    w.w_ih[0], w.w_hh[0], w.b_ih[0], w.b_hh[0] = (_ptr(wt[k]) for k in ("w_ih", "w_hh", "b_ih", "b_hh"))
    w.w_1, w.b_1, w.w_2, w.b_2 = (_ptr(wt[k]) for k in ("w_1", "b_1", "w_2", "b_2"))
    if actor is not None:
        w.w_a1, w.b_a1, w.w_a2, w.b_a2 = (_ptr(wt[k]) for k in ("w_a1", "b_a1", "w_a2", "b_a2"))
    means = torch.empty((B, T, S), dtype=dtype, device=device)
    stds = torch.empty_like(means)
    states = torch.empty_like(means)
    beliefs = torch.empty((B, T, Hb), dtype=dtype, device=device)
    acts = torch.empty((B, T, A), dtype=dtype, device=device) if actor is not None else None
    desc = RnnDesc()
    desc.mode, desc.dtype, desc.layout = MODES[mode], 0, LAYOUTS["batch_major"]
    desc.T, desc.B = T, B
    desc.num_layers, desc.bidirectional, desc.has_bias = 1, 0, 1
    desc.state_dim, desc.action_dim, desc.embed_dim, desc.belief_dim = S, A, E, Hb
    desc.actor_dim = Ea
    desc.scale_lb = scale_lb
    desc.tile_batch, desc.tile_hidden, desc.placement = tile_batch, tile_hidden, placement
    desc.weights = weights_hint
    io = RnnIO()
    io.x, io.noise, io.s0, io.h0 = _ptr(actions), _ptr(eps), _ptr(state0), _ptr(belief0)
    io.means, io.stds, io.states, io.beliefs = _ptr(means), _ptr(stds), _ptr(states), _ptr(beliefs)
    io.actions = _ptr(acts)
    ws = _call(desc, w, io, None, device, keep, check_status, noalloc)
    out = (means, stds, states, beliefs) + ((acts,) if actor is not None else ())
    return out, ws


def rssm_prior_unroll(actions, eps, weights, state0=None, belief0=None, *, scale_lb=0.1,
                      tile_batch=0, tile_hidden=0, placement=0, return_workspace=False, check_status=True,
                      noalloc=False, weights_hint=0):
    """RSSM prior unrolled over actions [B, T, A] with injected eps [B, T, S].

    weights: dict with w_as [E, S + A], b_as, w_ih [3Hb, E], w_hh [3Hb, Hb],
    b_ih, b_hh, w_1 [E, Hb], b_1, w_2 [2S, E], b_2 (float32, on the GPU).
    check_status and noalloc as for rnn_forward. weights_hint (the
    RnnDesc.weights field): 0 chooses the kernel, 1 the kernel with the GRU
    input weights in LDS and ten-odd members per group, 2 the kernel with
    every GRU weight slice in registers and wide members (RNN_E_PLAN when
    the shape does not fit it).
    Returns (means, stds, states, beliefs) stacked on dim 1.
    """
    out, ws = _rssm("rssm", actions, eps, weights, None, actions.shape[2], state0, belief0, scale_lb,
                    tile_batch, tile_hidden, placement, check_status, noalloc, weights_hint)
    return (out, ws) if return_workspace else out


def rssm_actor_unroll(eps, weights, actor, state0=None, belief0=None, *, scale_lb=0.1,
                      tile_batch=0, tile_hidden=0, placement=0, return_workspace=False, check_status=True,
                      weights_hint=0):
    """RSSM prior unrolled for H = eps.shape[1] steps with the actor choosing
    each action from the previous state and belief.

    weights as for rssm_prior_unroll; actor: dict with w_a1 [Ea, S + Hb],
    b_a1 [Ea], w_a2 [A, Ea], b_a2 [A] (float32, on the GPU).
    check_status and weights_hint as for rssm_prior_unroll.
    Returns (means, stds, states, beliefs, actions) stacked on dim 1.
    """
    out, ws = _rssm("rssm_actor", None, eps, weights, actor, actor["w_a2"].shape[0], state0, belief0,
                    scale_lb, tile_batch, tile_hidden, placement, check_status, weights_hint=weights_hint)
    return (out, ws) if return_workspace else out
