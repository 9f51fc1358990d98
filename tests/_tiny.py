"""Hand-built tiny KDA problems for the oracle pins (no randomness beyond a
local generator; no arithmetic of the step itself)."""
import numpy as np


def blank(N=1, H=1, T=1, dk=4, dv=4, taps=4, lengths=None):
    """All-zero problem with identity-free defaults; callers fill what they need."""
    C = 2 * dk + dv
    if lengths is None:
        lengths = [T] * N
    lengths = np.asarray(lengths, np.int64)
    cu = np.zeros(len(lengths) + 1, np.int64)
    cu[1:] = np.cumsum(lengths)
    Tt = int(cu[-1])
    return dict(
        q=np.zeros((Tt, H, dk), np.float32), k=np.zeros((Tt, H, dk), np.float32),
        v=np.zeros((Tt, H, dv), np.float32), f=np.zeros((Tt, H, dk), np.float32),
        beta=np.zeros((Tt, H), np.float32), g=np.zeros((Tt, H, dv), np.float32),
        conv_w=np.zeros((H, C, taps), np.float32), A_log=np.zeros((H, dk), np.float32),
        dt_bias=np.zeros((H, dk), np.float32), gamma=np.ones(dv, np.float32),
        state=np.zeros((len(lengths), H, dk, dv), np.float64),
        win=np.zeros((len(lengths), H, taps - 1, C), np.float64),
        cu_seqlens=cu)


def current_tap_only(p):
    """Conv taps that pass the current raw row through unchanged."""
    p["conv_w"][...] = 0.0
    p["conv_w"][:, :, -1] = 1.0
    return p


def random_dense(rng, N=1, H=1, T=8, dk=4, dv=4, taps=4, lengths=None, state_std=0.3,
                 win_std=1.0):
    p = blank(N, H, T, dk, dv, taps, lengths)
    Tt = p["q"].shape[0]
    C = 2 * dk + dv
    p["q"][...] = rng.standard_normal((Tt, H, dk))
    p["k"][...] = rng.standard_normal((Tt, H, dk))
    p["v"][...] = rng.standard_normal((Tt, H, dv))
    p["f"][...] = rng.standard_normal((Tt, H, dk))
    p["beta"][...] = rng.uniform(0.05, 0.95, (Tt, H))
    p["g"][...] = rng.standard_normal((Tt, H, dv))
    p["conv_w"][...] = 0.5 * rng.standard_normal((H, C, taps))
    p["A_log"][...] = rng.uniform(-1, 1, (H, dk))
    p["dt_bias"][...] = rng.uniform(-0.5, 0.5, (H, dk))
    p["gamma"][...] = rng.uniform(0.5, 1.5, dv)
    n = p["state"].shape[0]
    p["state"][...] = (state_std * rng.standard_normal((n, H, dk, dv))).astype(np.float32)
    p["win"][...] = (win_std * rng.standard_normal((n, H, taps - 1, C))).astype(np.float32)
    return p
