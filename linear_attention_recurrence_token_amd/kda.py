"""Python binding of libkda (ctypes).  Argument marshalling only: every step
of the computation runs in the HIP kernels behind the C ABI in include/kda.h.

``kda_token_step`` and ``kda_sequence`` take torch tensors that already live
on the GPU, check their shapes and dtypes, and call the C entry points of the
same names on the current (or given) torch stream.  A non-OK status raises
``KdaError``; nothing computes on the CPU, and a missing ``libkda.so`` raises
at import of the library rather than falling back to anything.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import threading
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkda.so")

KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_DEVICE, KDA_ERR_LAUNCH = 0, -1, -2, -3, -4
KDA_ERR_SCRATCH_LIMIT = -5
KDA_NOALLOC_SCRATCH_BYTES = 16 << 20
KDA_F32, KDA_BF16 = 0, 1
KDA_GATE_BOUNDED, KDA_GATE_LITERAL, KDA_GATE_RAW = 0, 1, 2
KDA_PREFILL_AUTO, KDA_PREFILL_FUSED, KDA_PREFILL_SPLIT, KDA_PREFILL_CHUNK, KDA_PREFILL_SHORT = 0, 1, 2, 3, 4
KDA_PREFILL_SCAN = 5
KDA_PREFILL_CHUNK_SHORT = 6
DK = DV = 128
TAPS = 4
CH = 2 * DK + DV


class kda_config(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("head_dim_k", ctypes.c_int32),
                ("head_dim_v", ctypes.c_int32), ("conv_taps", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32), ("gate_mode", ctypes.c_int32),
                ("gate_lower_bound", ctypes.c_float), ("l2_eps", ctypes.c_float),
                ("rms_eps", ctypes.c_float), ("prefill_path", ctypes.c_int32)]


TENSOR_FIELDS = ("q", "k", "v", "f", "beta", "g", "conv_w", "A_log", "dt_bias", "gamma",
                 "state", "conv_win", "y", "o_raw")


class kda_tensors(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in TENSOR_FIELDS]


EXPORTS = ("kda_token_step", "kda_sequence", "kda_sequence_workspace_size",
           "kda_status_string", "kda_version", "kda_device_check",
           "kda_projection_workspace_size", "kda_lowrank_gates", "kda_gate_projection",
           "kda_output_projection", "kda_lowrank_gates_noalloc", "kda_lowrank_factor",
           "kda_sequence_lowrank")

KDA_PROJ_LOWRANK_GATES, KDA_PROJ_GATE, KDA_PROJ_OUTPUT, KDA_PROJ_LOWRANK_FACTOR = 0, 1, 2, 3


class KdaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (where, status_string(status), status))


_lock = threading.Lock()
_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """The loaded libkda.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError("libkda.so is not built (expected at %s); run "
                                  "__graft_entry__.build() first" % LIB_PATH)
            L = ctypes.CDLL(LIB_PATH)
            cfgp, tp = ctypes.POINTER(kda_config), ctypes.POINTER(kda_tensors)
            L.kda_token_step.restype = ctypes.c_int32
            L.kda_token_step.argtypes = [cfgp, tp, ctypes.c_int32, ctypes.c_void_p]
            L.kda_sequence.restype = ctypes.c_int32
            L.kda_sequence.argtypes = [cfgp, tp, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                       ctypes.c_void_p, ctypes.c_void_p]
            L.kda_sequence_workspace_size.restype = ctypes.c_int64
            L.kda_sequence_workspace_size.argtypes = [cfgp, ctypes.c_int32, ctypes.c_int64]
            L.kda_status_string.restype = ctypes.c_char_p
            L.kda_status_string.argtypes = [ctypes.c_int32]
            L.kda_version.restype = ctypes.c_int32
            L.kda_version.argtypes = []
            L.kda_device_check.restype = ctypes.c_int32
            L.kda_device_check.argtypes = []
            vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
            L.kda_projection_workspace_size.restype = i64
            L.kda_projection_workspace_size.argtypes = [cfgp, i32, i32, i32, i64]
            L.kda_lowrank_gates.restype = i32
            L.kda_lowrank_gates.argtypes = [cfgp, vp, vp, vp, i32, i32, i64, vp, vp, vp, i64, vp]
            L.kda_gate_projection.restype = i32
            L.kda_gate_projection.argtypes = [cfgp, vp, vp, i32, i64, vp, vp, i64, vp]
            L.kda_output_projection.restype = i32
            L.kda_output_projection.argtypes = [cfgp, vp, vp, i32, i64, vp, vp, i64, vp]
            L.kda_lowrank_factor.restype = i32
            L.kda_lowrank_factor.argtypes = [cfgp, vp, vp, i32, i32, i64, vp, vp, vp, i64, vp]
            L.kda_sequence_lowrank.restype = i32
            L.kda_sequence_lowrank.argtypes = [cfgp, tp, i32, vp, vp, vp, i64, vp, vp, i32, vp]
            L.kda_lowrank_gates_noalloc.restype = i32
            L.kda_lowrank_gates_noalloc.argtypes = [cfgp, vp, vp, vp, i32, i32, i64, vp, vp, vp]
            _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().kda_status_string(int(status)).decode()


@dataclasses.dataclass
class KdaConfig:
    num_heads: int
    act_dtype: int = KDA_F32
    gate_mode: int = KDA_GATE_BOUNDED
    gate_lower_bound: float = -5.0
    l2_eps: float = 1e-6
    rms_eps: float = 1e-6
    head_dim_k: int = DK
    head_dim_v: int = DV
    conv_taps: int = TAPS
    prefill_path: int = KDA_PREFILL_AUTO

    def to_c(self) -> kda_config:
        return kda_config(self.num_heads, self.head_dim_k, self.head_dim_v, self.conv_taps,
                          self.act_dtype, self.gate_mode, self.gate_lower_bound,
                          self.l2_eps, self.rms_eps, self.prefill_path)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check_tensors(cfg: KdaConfig, T: int, N: int, ts: dict, skip=()) -> None:
    import torch
    act = torch.bfloat16 if cfg.act_dtype == KDA_BF16 else torch.float32
    H = cfg.num_heads
    dk, dv = cfg.head_dim_k, cfg.head_dim_v
    C = 2 * dk + dv
    expect = {
        "q": ((T, H, dk), act), "k": ((T, H, dk), act), "v": ((T, H, dv), act),
        "f": ((T, H, dk), torch.float32), "beta": ((T, H), torch.float32),
        "g": ((T, H, dv), act), "conv_w": ((H, C, cfg.conv_taps), torch.float32),
        "A_log": ((H, dk), torch.float32), "dt_bias": ((H, dk), torch.float32),
        "gamma": ((dv,), torch.float32), "state": ((N, H, dk, dv), torch.float32),
        "conv_win": ((N, H, cfg.conv_taps - 1, C), torch.float32),
        "y": ((T, H, dv), act), "o_raw": ((T, H, dv), torch.float32),
    }
    dev = None
    for name, (shape, dtype) in expect.items():
        if name in skip:
            continue
        t = ts.get(name)
        if t is None:
            if name == "o_raw":
                continue
            raise ValueError("missing tensor %r" % name)
        if not t.is_cuda:
            raise ValueError("%s must be a GPU tensor" % name)
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("%s is on %s, expected %s" % (name, t.device, dev))
        if t.dtype != dtype:
            raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
        if tuple(t.shape) != shape:
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), shape))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)


def _tensors_struct(ts: dict) -> kda_tensors:
    return kda_tensors(*[_ptr(ts.get(name)) for name in TENSOR_FIELDS])


def _stream_handle(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def kda_token_step(config: KdaConfig, *, q, k, v, f, beta, g, conv_w, A_log, dt_bias, gamma,
                   state, conv_win, y, o_raw=None, stream=None, check: bool = True) -> None:
    """Decode one token for each of N = q.shape[0] sequences (C: kda_token_step)."""
    ts = dict(q=q, k=k, v=v, f=f, beta=beta, g=g, conv_w=conv_w, A_log=A_log, dt_bias=dt_bias,
              gamma=gamma, state=state, conv_win=conv_win, y=y, o_raw=o_raw)
    N = int(q.shape[0])
    if check:
        _check_tensors(config, N, N, ts)
    c = config.to_c()
    t = _tensors_struct(ts)
    st = lib().kda_token_step(ctypes.byref(c), ctypes.byref(t), N, _stream_handle(stream))
    if st != KDA_OK:
        raise KdaError(st, "kda_token_step")


def kda_sequence(config: KdaConfig, *, q, k, v, f, beta, g, conv_w, A_log, dt_bias, gamma,
                 state, conv_win, y, o_raw=None, cu_seqlens=None, cu_seqlens_host=None, seq_order=None,
                 num_seqs: Optional[int] = None, workspace="auto", stream=None, side_stream=None,
                 check: bool = True) -> None:
    """Prefill over packed sequences (C: kda_sequence).

    cu_seqlens: int32 GPU tensor [N+1] of token offsets, or None for a dense
    batch (N = state.shape[0] sequences of T / N tokens).  cu_seqlens_host:
    optional host copy of the same offsets (a CPU int32 tensor or numpy
    array; the library checks it and may plan with it).  seq_order: optional
    int32 GPU tensor [N], the scheduling order of the sequences.  workspace:
    "auto" allocates (through torch) the scratch the faster path can use, as
    kda_sequence_workspace_size reports; None passes none; or a GPU tensor.
    side_stream: optional second torch stream on the same device, on which
    the two-pass path may overlap part of its work (the call is still ordered
    on `stream` as one unit)."""
    import numpy as np
    import torch
    ts = dict(q=q, k=k, v=v, f=f, beta=beta, g=g, conv_w=conv_w, A_log=A_log, dt_bias=dt_bias,
              gamma=gamma, state=state, conv_win=conv_win, y=y, o_raw=o_raw)
    T = int(q.shape[0])
    N = int(state.shape[0]) if num_seqs is None else int(num_seqs)
    if check:
        _check_tensors(config, T, N, ts)
        for name, a, n in (("cu_seqlens", cu_seqlens, N + 1), ("seq_order", seq_order, N)):
            if a is None:
                continue
            if not a.is_cuda or a.dtype != torch.int32 or tuple(a.shape) != (n,) or not a.is_contiguous():
                raise ValueError("%s must be a contiguous int32 GPU tensor of shape (%d,)" % (name, n))
    host = None
    if cu_seqlens_host is not None:
        host = np.ascontiguousarray(np.asarray(cu_seqlens_host), dtype=np.int32)
        if host.shape != (N + 1,):
            raise ValueError("cu_seqlens_host must have shape (%d,)" % (N + 1))
    c = config.to_c()
    t = _tensors_struct(ts)
    ws_ptr, ws_bytes = None, 0
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto', None or a GPU tensor")
        need = int(lib().kda_sequence_workspace_size(ctypes.byref(c), N, T))
        if need < 0:
            raise KdaError(need, "kda_sequence_workspace_size")
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        else:
            workspace = None
    if workspace is not None:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    st = lib().kda_sequence(ctypes.byref(c), ctypes.byref(t), N, _ptr(cu_seqlens),
                            host.ctypes.data if host is not None else None, _ptr(seq_order), T,
                            ws_ptr, ws_bytes, _stream_handle(stream),
                            _stream_handle(side_stream) if side_stream is not None else None)
    if st != KDA_OK:
        raise KdaError(st, "kda_sequence")


def sequence_workspace_size(config: KdaConfig, num_seqs: int, total_tokens: int) -> int:
    c = config.to_c()
    return int(lib().kda_sequence_workspace_size(ctypes.byref(c), int(num_seqs), int(total_tokens)))


def device_check() -> int:
    return int(lib().kda_device_check())


def version() -> int:
    return int(lib().kda_version())


# --- projections on either side of the step -----------------------------------

def _gpu_tensor(name, t, shape, dtype, dev=None):
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if dev is not None and t.device != dev:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, dev))
    if t.dtype != dtype:
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def projection_workspace_size(config: KdaConfig, which: int, hidden: int, tokens: int, rank: int = 0) -> int:
    c = config.to_c()
    return int(lib().kda_projection_workspace_size(ctypes.byref(c), int(which), int(hidden), int(rank),
                                                   int(tokens)))


def _workspace(config, which, hidden, tokens, rank, workspace, device):
    import torch
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto', None or a GPU tensor")
        need = projection_workspace_size(config, which, hidden, tokens, rank)
        if need < 0:
            raise KdaError(need, "kda_projection_workspace_size")
        workspace = torch.empty(need, dtype=torch.uint8, device=device) if need > 0 else None
    if workspace is None:
        return None, 0
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def kda_lowrank_gates(config: KdaConfig, *, x, w_fa_bp, w_fb, f, beta, workspace="auto", stream=None,
                      check: bool = True) -> None:
    """f = W_fb (W_fa x) and beta = sigmoid(W_bp x) for hidden rows x [T, D]
    (C: kda_lowrank_gates).  w_fa_bp [r + H, D] fp32 stacks W_fa over W_bp;
    w_fb [H * 128, r] fp32; f [T, H, 128] and beta [T, H] fp32 out.
    workspace: "auto" allocates (through torch) what
    kda_projection_workspace_size reports, or a GPU tensor."""
    import torch
    T, D = int(x.shape[0]), int(x.shape[1])
    H = config.num_heads
    r = int(w_fb.shape[1])
    if check:
        act = torch.bfloat16 if config.act_dtype == KDA_BF16 else torch.float32
        _gpu_tensor("x", x, (T, D), act)
        for name, t, shape in (("w_fa_bp", w_fa_bp, (r + H, D)), ("w_fb", w_fb, (H * DK, r)),
                               ("f", f, (T, H, DK)), ("beta", beta, (T, H))):
            _gpu_tensor(name, t, shape, torch.float32, x.device)
    c = config.to_c()
    ws_ptr, ws_bytes = _workspace(config, KDA_PROJ_LOWRANK_GATES, D, T, r, workspace, x.device)
    st = lib().kda_lowrank_gates(ctypes.byref(c), _ptr(x), _ptr(w_fa_bp), _ptr(w_fb), D, r, T, _ptr(f),
                                 _ptr(beta), ws_ptr, ws_bytes, _stream_handle(stream))
    if st != KDA_OK:
        raise KdaError(st, "kda_lowrank_gates")


def kda_lowrank_gates_noalloc(config: KdaConfig, *, x, w_fa_bp, w_fb, f, beta, stream=None,
                              check: bool = True) -> None:
    """kda_lowrank_gates with the library's static scratch as its workspace
    (C: kda_lowrank_gates_noalloc): nothing is allocated; T * r * 4 bytes
    must fit in KDA_NOALLOC_SCRATCH_BYTES, else KdaError(KDA_ERR_SCRATCH_LIMIT).
    Calls that overlap in time on one device race on that scratch."""
    import torch
    T, D = int(x.shape[0]), int(x.shape[1])
    H = config.num_heads
    r = int(w_fb.shape[1])
    if check:
        act = torch.bfloat16 if config.act_dtype == KDA_BF16 else torch.float32
        _gpu_tensor("x", x, (T, D), act)
        for name, t, shape in (("w_fa_bp", w_fa_bp, (r + H, D)), ("w_fb", w_fb, (H * DK, r)),
                               ("f", f, (T, H, DK)), ("beta", beta, (T, H))):
            _gpu_tensor(name, t, shape, torch.float32, x.device)
    c = config.to_c()
    st = lib().kda_lowrank_gates_noalloc(ctypes.byref(c), _ptr(x), _ptr(w_fa_bp), _ptr(w_fb), D, r, T,
                                         _ptr(f), _ptr(beta), _stream_handle(stream))
    if st != KDA_OK:
        raise KdaError(st, "kda_lowrank_gates_noalloc")


def kda_lowrank_factor(config: KdaConfig, *, x, w_fa_bp, a, beta, workspace="auto", stream=None,
                       check: bool = True) -> None:
    """a = W_fa x and beta = sigmoid(W_bp x) (C: kda_lowrank_factor): the first
    low-rank product alone, for kda_sequence_lowrank.  w_fa_bp [r + H, D]
    fp32; a [T, r] and beta [T, H] fp32 out."""
    import torch
    T, D = int(x.shape[0]), int(x.shape[1])
    H = config.num_heads
    r = int(a.shape[1])
    if check:
        act = torch.bfloat16 if config.act_dtype == KDA_BF16 else torch.float32
        _gpu_tensor("x", x, (T, D), act)
        for name, t, shape in (("w_fa_bp", w_fa_bp, (r + H, D)), ("a", a, (T, r)), ("beta", beta, (T, H))):
            _gpu_tensor(name, t, shape, torch.float32, x.device)
    c = config.to_c()
    ws_ptr, ws_bytes = _workspace(config, KDA_PROJ_LOWRANK_FACTOR, D, T, r, workspace, x.device)
    st = lib().kda_lowrank_factor(ctypes.byref(c), _ptr(x), _ptr(w_fa_bp), D, r, T, _ptr(a), _ptr(beta),
                                  ws_ptr, ws_bytes, _stream_handle(stream))
    if st != KDA_OK:
        raise KdaError(st, "kda_lowrank_factor")


def kda_sequence_lowrank(config: KdaConfig, *, q, k, v, a, w_fb, beta, g, conv_w, A_log, dt_bias, gamma,
                         state, conv_win, y, o_raw=None, cu_seqlens=None, cu_seqlens_host=None,
                         seq_order=None, num_seqs: Optional[int] = None, stream=None,
                         check: bool = True) -> None:
    """Prefill with f = W_fb a formed in the step (C: kda_sequence_lowrank):
    the tensors of kda_sequence without f, plus a [T, r] and w_fb [H * 128, r]
    fp32 GPU tensors (r a multiple of 32 up to 128)."""
    import numpy as np
    import torch
    T = int(q.shape[0])
    N = int(state.shape[0]) if num_seqs is None else int(num_seqs)
    H = config.num_heads
    r = int(a.shape[1]) if a.dim() == 2 else -1
    ts = dict(q=q, k=k, v=v, f=None, beta=beta, g=g, conv_w=conv_w, A_log=A_log, dt_bias=dt_bias,
              gamma=gamma, state=state, conv_win=conv_win, y=y, o_raw=o_raw)
    if check:
        _check_tensors(config, T, N, ts, skip=("f",))
        _gpu_tensor("a", a, (T, r), torch.float32, q.device)
        _gpu_tensor("w_fb", w_fb, (H * DK, r), torch.float32, q.device)
        if cu_seqlens is not None and (not cu_seqlens.is_cuda or cu_seqlens.dtype != torch.int32
                                       or tuple(cu_seqlens.shape) != (N + 1,)):
            raise ValueError("cu_seqlens must be a contiguous int32 GPU tensor of shape (%d,)" % (N + 1))
    host = None
    if cu_seqlens_host is not None:
        host = np.ascontiguousarray(np.asarray(cu_seqlens_host), dtype=np.int32)
    c = config.to_c()
    t = _tensors_struct(ts)
    st = lib().kda_sequence_lowrank(ctypes.byref(c), ctypes.byref(t), N, _ptr(cu_seqlens),
                                    host.ctypes.data if host is not None else None, _ptr(seq_order), T,
                                    _ptr(a), _ptr(w_fb), r, _stream_handle(stream))
    if st != KDA_OK:
        raise KdaError(st, "kda_sequence_lowrank")


def kda_gate_projection(config: KdaConfig, *, x, w_g, g, workspace="auto", stream=None,
                        check: bool = True) -> None:
    """g = W_g x (C: kda_gate_projection): x [T, D], w_g [H * 128, D],
    g [T, H, 128], all in the activation dtype."""
    import torch
    T, D = int(x.shape[0]), int(x.shape[1])
    H = config.num_heads
    if check:
        act = torch.bfloat16 if config.act_dtype == KDA_BF16 else torch.float32
        _gpu_tensor("x", x, (T, D), act)
        _gpu_tensor("w_g", w_g, (H * DV, D), act, x.device)
        _gpu_tensor("g", g, (T, H, DV), act, x.device)
    c = config.to_c()
    ws_ptr, ws_bytes = _workspace(config, KDA_PROJ_GATE, D, T, 0, workspace, x.device)
    st = lib().kda_gate_projection(ctypes.byref(c), _ptr(x), _ptr(w_g), D, T, _ptr(g), ws_ptr, ws_bytes,
                                   _stream_handle(stream))
    if st != KDA_OK:
        raise KdaError(st, "kda_gate_projection")


def kda_output_projection(config: KdaConfig, *, y, w_o, out, workspace="auto", stream=None,
                          check: bool = True) -> None:
    """out = W_o y (C: kda_output_projection): y [T, H, 128], w_o [D, H * 128],
    out [T, D], all in the activation dtype."""
    import torch
    T = int(y.shape[0])
    H = config.num_heads
    D = int(w_o.shape[0])
    if check:
        act = torch.bfloat16 if config.act_dtype == KDA_BF16 else torch.float32
        _gpu_tensor("y", y, (T, H, DV), act)
        _gpu_tensor("w_o", w_o, (D, H * DV), act, y.device)
        _gpu_tensor("out", out, (T, D), act, y.device)
    c = config.to_c()
    ws_ptr, ws_bytes = _workspace(config, KDA_PROJ_OUTPUT, D, T, 0, workspace, y.device)
    st = lib().kda_output_projection(ctypes.byref(c), _ptr(y), _ptr(w_o), D, T, _ptr(out), ws_ptr, ws_bytes,
                                     _stream_handle(stream))
    if st != KDA_OK:
        raise KdaError(st, "kda_output_projection")
