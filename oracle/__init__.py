"""CPU oracle for the fused KDA token step -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does; it
shares no code with it.

``kda_reference`` runs the plain fp64 C implementation in ``kda_oracle.c``
(steps in the order of "Kimi K3 Metal Gap Analysis", §2 KDA Attention table:
Conv4 + SiLU, L2 normalize q/k, Decay compute, Recurrence, O projection);
it is the parity reference.  ``kda_reference_f32_inplace`` runs the same
loops in single precision with the state updated in place: the CPU
baseline's timed mode, pinned to the fp64 one.  The shared object is
compiled with gcc on first use if it is missing.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
# KDA_ORACLE_LIB points the tests at another build of the same source (the
# sanitizer run); it must exist, it is never built from here
_LIB = os.environ.get("KDA_ORACLE_LIB") or os.path.join(_HERE, "libkda_oracle.so")

GATE_BOUNDED, GATE_LITERAL, GATE_RAW = 0, 1, 2

_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile kda_oracle.c into libkda_oracle.so (gcc, OpenMP, -O2)."""
    if os.environ.get("KDA_ORACLE_LIB"):
        if not os.path.exists(_LIB):
            raise FileNotFoundError(_LIB)
        return _LIB
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            fp = ctypes.POINTER(ctypes.c_float)
            dp = ctypes.POINTER(ctypes.c_double)
            lib.kda_oracle_run.restype = ctypes.c_int32
            lib.kda_oracle_run.argtypes = [
                ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                ctypes.POINTER(ctypes.c_int64),
                fp, fp, fp, fp, fp, fp,
                fp, fp, fp, fp,
                ctypes.c_int32, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                dp, dp, dp, dp,
            ]
            lib.kda_oracle_run_f32.restype = ctypes.c_int32
            lib.kda_oracle_run_f32.argtypes = [
                ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                ctypes.POINTER(ctypes.c_int64),
                fp, fp, fp, fp, fp, fp,
                fp, fp, fp, fp,
                ctypes.c_int32, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                fp, fp, fp, fp,
            ]
            lib.kda_oracle_version.restype = ctypes.c_int32
            _lib = lib
    return _lib


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def kda_reference(q, k, v, f, beta, g, conv_w, A_log, dt_bias, gamma,
                  state, win, cu_seqlens, *, gate_mode=GATE_BOUNDED,
                  lower_bound=-5.0, l2_eps=1e-6, rms_eps=1e-6,
                  want_o_raw=True):
    """Run the oracle.

    Shapes: q, k [T, H, dk]; v, g [T, H, dv]; f [T, H, dk]; beta [T, H];
    conv_w [H, 2dk+dv, taps]; A_log, dt_bias [H, dk]; gamma [dv];
    state [N, H, dk, dv]; win [N, H, taps-1, 2dk+dv]; cu_seqlens [N+1].
    Per-token inputs and parameters are taken as fp32 values (bf16 data must
    already be widened); state and window are carried in fp64.

    Returns dict(y, o_raw, state, win) as float64 arrays (state and window
    are new arrays; the inputs are not modified).
    """
    lib = _load()
    q, k, v, f, g = _f32(q), _f32(k), _f32(v), _f32(f), _f32(g)
    beta = _f32(beta)
    conv_w, A_log, dt_bias, gamma = _f32(conv_w), _f32(A_log), _f32(dt_bias), _f32(gamma)
    T, H, dk = q.shape
    dv = v.shape[2]
    taps = conv_w.shape[2]
    C = 2 * dk + dv
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    N = cu.shape[0] - 1
    assert k.shape == (T, H, dk) and f.shape == (T, H, dk)
    assert v.shape == (T, H, dv) and g.shape == (T, H, dv)
    assert beta.shape == (T, H)
    assert conv_w.shape == (H, C, taps)
    assert A_log.shape == (H, dk) and dt_bias.shape == (H, dk) and gamma.shape == (dv,)
    assert cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
    S = np.array(state, dtype=np.float64, copy=True, order="C")
    W = np.array(win, dtype=np.float64, copy=True, order="C")
    assert S.shape == (N, H, dk, dv) and W.shape == (N, H, taps - 1, C)
    y = np.zeros((T, H, dv), dtype=np.float64)
    o = np.zeros((T, H, dv), dtype=np.float64) if want_o_raw else None
    rc = lib.kda_oracle_run(
        N, H, dk, dv, taps, _ptr(cu, ctypes.c_int64),
        _ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float), _ptr(v, ctypes.c_float),
        _ptr(f, ctypes.c_float), _ptr(beta, ctypes.c_float), _ptr(g, ctypes.c_float),
        _ptr(conv_w, ctypes.c_float), _ptr(A_log, ctypes.c_float),
        _ptr(dt_bias, ctypes.c_float), _ptr(gamma, ctypes.c_float),
        int(gate_mode), float(lower_bound), float(l2_eps), float(rms_eps),
        _ptr(S, ctypes.c_double), _ptr(W, ctypes.c_double), _ptr(y, ctypes.c_double),
        _ptr(o, ctypes.c_double) if o is not None else ctypes.POINTER(ctypes.c_double)(),
    )
    if rc != 0:
        raise ValueError("kda_oracle_run rejected its arguments (rc=%d)" % rc)
    return {"y": y, "o_raw": o, "state": S, "win": W}


def kda_reference_f32_inplace(q, k, v, f, beta, g, conv_w, A_log, dt_bias, gamma,
                              state, win, y, cu_seqlens, o_raw=None, *, gate_mode=GATE_BOUNDED,
                              lower_bound=-5.0, l2_eps=1e-6, rms_eps=1e-6):
    """The single-precision oracle (the CPU baseline's timed mode).

    Same shapes as kda_reference.  state [N, H, dk, dv] and win [N, H,
    taps-1, C] must be C-contiguous float32 arrays and are updated in place;
    y (and o_raw when given) [T, H, dv] float32 are written.  Every array is
    used as it is (no conversion or copy), so callers pass float32,
    C-contiguous inputs.  Nothing is returned."""
    lib = _load()
    arrs = (q, k, v, f, beta, g, conv_w, A_log, dt_bias, gamma, state, win, y)
    for a in arrs + ((o_raw,) if o_raw is not None else ()):
        if a.dtype != np.float32 or not a.flags.c_contiguous:
            raise ValueError("kda_reference_f32_inplace takes C-contiguous float32 arrays")
    T, H, dk = q.shape
    dv = v.shape[2]
    taps = conv_w.shape[2]
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    N = cu.shape[0] - 1
    assert k.shape == (T, H, dk) and f.shape == (T, H, dk) and beta.shape == (T, H)
    assert g.shape == (T, H, dv) and y.shape == (T, H, dv)
    assert state.shape == (N, H, dk, dv) and win.shape == (N, H, taps - 1, 2 * dk + dv)
    assert cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
    fp = ctypes.c_float
    rc = lib.kda_oracle_run_f32(
        N, H, dk, dv, taps, _ptr(cu, ctypes.c_int64),
        _ptr(q, fp), _ptr(k, fp), _ptr(v, fp), _ptr(f, fp), _ptr(beta, fp), _ptr(g, fp),
        _ptr(conv_w, fp), _ptr(A_log, fp), _ptr(dt_bias, fp), _ptr(gamma, fp),
        int(gate_mode), float(lower_bound), float(l2_eps), float(rms_eps),
        _ptr(state, fp), _ptr(win, fp), _ptr(y, fp),
        _ptr(o_raw, fp) if o_raw is not None else ctypes.POINTER(fp)())
    if rc != 0:
        raise ValueError("kda_oracle_run_f32 rejected its arguments (rc=%d)" % rc)


def omp_threads() -> int:
    """Threads the oracle's OpenMP loop uses (OMP_NUM_THREADS, else CPUs)."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env:
        try:
            return max(1, int(env.split(",")[0]))
        except ValueError:
            pass
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1
