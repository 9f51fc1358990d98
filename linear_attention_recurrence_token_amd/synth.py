"""Seeded synthetic inputs for the KDA token step.

This module only draws random numbers and lays them out; it contains none of
the step's own arithmetic.  Both the HIP path (through the bench and the GPU
tests) and the CPU oracle consume what it produces.

Recipe (one PCG64 stream family per workload, seed = workload index unless
overridden; every tensor has its own SeedSequence child, large tensors are
filled in fixed blocks with per-block children so the result does not depend
on the thread count):

  lengths -> conv_w -> A_log -> dt_bias -> gamma -> initial state -> window
  -> q, k, v, g -> beta logits -> decay d -> fresh-sequence flags

* q, k, v, g ~ N(0, 1); conv taps ~ N(0, 0.5) (0.5 is a standard deviation);
  beta = sigmoid(N(0, 1)); A_log ~ U[-1, 1]; dt_bias ~ U[-0.5, 0.5].
* The decay is specified by its value d = exp(gk) ~ U[lo, hi] per token, head
  and key channel.  The pre-activation f handed to the step is obtained by
  inverting the configured gate form in fp64 (for the bounded form,
  f = logit(ln(d) / lb) / exp(A_log) - dt_bias), then rounded to fp32.
* bf16 workloads round q, k, v, g (and the carried window, which holds raw
  rows) to bf16 with round-to-nearest-even; both sides consume the same
  rounded values.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
from typing import Optional

import numpy as np

GATE_BOUNDED, GATE_LITERAL, GATE_RAW = 0, 1, 2
_BLOCK = 1 << 22


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _fill_blocks(seed_seq: np.random.SeedSequence, out: np.ndarray, draw) -> np.ndarray:
    """Fill a flat array block by block; block b uses child b of seed_seq."""
    flat = out.reshape(-1)
    n = flat.shape[0]
    nblk = (n + _BLOCK - 1) // _BLOCK
    children = seed_seq.spawn(max(nblk, 1))

    def work(b):
        lo, hi = b * _BLOCK, min(n, (b + 1) * _BLOCK)
        rng = np.random.Generator(np.random.PCG64(children[b]))
        draw(rng, flat[lo:hi])

    if nblk <= 1:
        if n:
            work(0)
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nblk)))
    return out


def _normal(ss, shape, std=1.0):
    out = np.empty(shape, dtype=np.float32)

    def draw(rng, view):
        rng.standard_normal(out=view, dtype=np.float32)
        if std != 1.0:
            view *= np.float32(std)
    return _fill_blocks(ss, out, draw)


def _uniform(ss, shape, lo, hi):
    out = np.empty(shape, dtype=np.float32)

    def draw(rng, view):
        view[...] = (lo + (hi - lo) * rng.random(view.shape[0], dtype=np.float64)).astype(np.float32)
    return _fill_blocks(ss, out, draw)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even), returned as fp32."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000))
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Bit pattern (int16) of fp32 values that are already bf16-exact."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if np.any(b & np.uint32(0xFFFF)):
        raise ValueError("values are not bf16-exact")
    return (b >> np.uint32(16)).astype(np.uint16).view(np.int16)


def _round_inplace_bf16(a: np.ndarray) -> None:
    flat = a.reshape(-1)
    n = flat.shape[0]
    nblk = (n + _BLOCK - 1) // _BLOCK

    def work(bi):
        lo, hi = bi * _BLOCK, min(n, (bi + 1) * _BLOCK)
        flat[lo:hi] = round_to_bf16(flat[lo:hi])
    if nblk <= 1:
        if n:
            work(0)
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nblk)))


@dataclasses.dataclass
class Workload:
    """Host copy of one KDA problem (all arrays C-contiguous, fp32 unless noted)."""
    name: str
    N: int
    H: int
    dk: int
    dv: int
    taps: int
    act_dtype: str                 # "f32" or "bf16" (q, k, v, g, y)
    cu_seqlens: np.ndarray         # int64 [N+1]
    q: np.ndarray                  # [T, H, dk]
    k: np.ndarray                  # [T, H, dk]
    v: np.ndarray                  # [T, H, dv]
    f: np.ndarray                  # [T, H, dk]
    beta: np.ndarray               # [T, H]
    g: np.ndarray                  # [T, H, dv]
    conv_w: np.ndarray             # [H, 2dk+dv, taps]
    A_log: np.ndarray              # [H, dk]
    dt_bias: np.ndarray            # [H, dk]
    gamma: np.ndarray              # [dv]
    state0: np.ndarray             # [N, H, dk, dv]
    win0: np.ndarray               # [N, H, taps-1, 2dk+dv]
    gate_mode: int = GATE_BOUNDED
    lower_bound: float = -5.0
    l2_eps: float = 1e-6
    rms_eps: float = 1e-6
    decode_steps: int = 0          # >0: token rows are [steps, N] (one token per sequence per step)

    @property
    def total_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def lengths(self) -> np.ndarray:
        return np.diff(self.cu_seqlens)


def _decay_to_f(d, A_log, dt_bias, gate_mode, lower_bound):
    """Pre-activation f that makes the configured gate produce decay d (fp64)."""
    d = d.astype(np.float64)
    gk = np.log(d)
    if gate_mode == GATE_RAW:
        return gk.astype(np.float32)
    A = np.exp(A_log.astype(np.float64))
    b = dt_bias.astype(np.float64)
    if gate_mode == GATE_BOUNDED:
        s = gk / lower_bound
        z = np.log(s) - np.log1p(-s)
    else:
        z = gk / lower_bound
    return (z / A - b).astype(np.float32)


def make_workload(name: str, *, seed: int, N: int, H: int, lengths=None,
                  decode_steps: int = 0, dk: int = 128, dv: int = 128, taps: int = 4,
                  act_dtype: str = "f32", state_std: Optional[float] = None,
                  win_std: Optional[float] = None, decay=(0.9, 0.999),
                  gamma_range=None, fresh_prob: Optional[float] = None,
                  gate_mode: int = GATE_BOUNDED, lower_bound: float = -5.0) -> Workload:
    """Draw one workload.

    lengths: per-sequence token counts (prefill) -- or decode_steps > 0 for a
    decode run, whose token rows are ordered [step, sequence].
    state_std / win_std: None gives zeros.  fresh_prob: per-sequence chance
    of a zero state and zero window (a fresh sequence).
    """
    root = np.random.SeedSequence(seed)
    (ss_len, ss_conv, ss_alog, ss_dtb, ss_gamma, ss_state, ss_win,
     ss_q, ss_k, ss_v, ss_g, ss_beta, ss_decay, ss_fresh) = root.spawn(14)
    C = 2 * dk + dv
    if decode_steps:
        lens = np.full(N, decode_steps, dtype=np.int64)
        T = decode_steps * N
    else:
        if lengths is None:
            raise ValueError("lengths or decode_steps required")
        if callable(lengths):
            lens = np.asarray(lengths(np.random.Generator(np.random.PCG64(ss_len))), dtype=np.int64)
        else:
            lens = np.asarray(lengths, dtype=np.int64)
        assert lens.shape == (N,) and np.all(lens >= 0)
        T = int(lens.sum())
    cu = np.zeros(N + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lens)

    conv_w = _normal(ss_conv, (H, C, taps), 0.5)
    A_log = _uniform(ss_alog, (H, dk), -1.0, 1.0)
    dt_bias = _uniform(ss_dtb, (H, dk), -0.5, 0.5)
    if gamma_range is None:
        gamma = np.ones(dv, dtype=np.float32)
    else:
        gamma = _uniform(ss_gamma, (dv,), gamma_range[0], gamma_range[1])
    state0 = (_normal(ss_state, (N, H, dk, dv), state_std) if state_std is not None
              else np.zeros((N, H, dk, dv), np.float32))
    win0 = (_normal(ss_win, (N, H, taps - 1, C), win_std) if win_std is not None
            else np.zeros((N, H, taps - 1, C), np.float32))

    q = _normal(ss_q, (T, H, dk))
    k = _normal(ss_k, (T, H, dk))
    v = _normal(ss_v, (T, H, dv))
    g = _normal(ss_g, (T, H, dv))
    bl = _normal(ss_beta, (T, H))
    beta = (1.0 / (1.0 + np.exp(-bl.astype(np.float64)))).astype(np.float32)
    d = _uniform(ss_decay, (T, H, dk), decay[0], decay[1])
    f = np.empty_like(d)
    # invert the gate over blocks of tokens (A_log, dt_bias broadcast over tokens)
    step = max(1, (_BLOCK // 4) // max(1, H * dk))

    def inv(lo):
        hi = min(T, lo + step)
        f[lo:hi] = _decay_to_f(d[lo:hi], A_log[None], dt_bias[None], gate_mode, lower_bound)
    with _cf.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(inv, range(0, T, step)))
    del d

    if fresh_prob is not None:
        fresh = np.random.Generator(np.random.PCG64(ss_fresh)).random(N) < fresh_prob
        state0[fresh] = 0.0
        win0[fresh] = 0.0

    if act_dtype == "bf16":
        for a in (q, k, v, g, win0):
            _round_inplace_bf16(a)
    elif act_dtype != "f32":
        raise ValueError(act_dtype)

    return Workload(name=name, N=N, H=H, dk=dk, dv=dv, taps=taps, act_dtype=act_dtype,
                    cu_seqlens=cu, q=q, k=k, v=v, f=f, beta=beta, g=g, conv_w=conv_w,
                    A_log=A_log, dt_bias=dt_bias, gamma=gamma, state0=state0, win0=win0,
                    gate_mode=gate_mode, lower_bound=lower_bound, decode_steps=decode_steps)


# --- the five workloads the step is measured and checked on -----------------

def workload(index: int, *, scale: Optional[dict] = None, seed: Optional[int] = None) -> Workload:
    """Workload `index` (0..5) at full size, or shrunk by `scale` overrides
    (keys: N, H, T, steps, max_len) for tests.  0..4 are the configurations
    of the method's measurement; 5 is the short multi-token prefill (13 tokens
    per sequence over a decode-sized batch)."""
    s = dict(scale or {})
    sd = index if seed is None else seed
    if index == 0:
        return make_workload("single-seq T=64 fp32", seed=sd, N=s.get("N", 1), H=s.get("H", 1),
                             lengths=[s.get("T", 64)] * s.get("N", 1))
    if index == 1:
        N, H, steps = s.get("N", 64), s.get("H", 32), s.get("steps", 1000)
        return make_workload("decode %dx%d fp32, %d steps" % (N, H, steps), seed=sd, N=N, H=H,
                             decode_steps=steps, state_std=0.02, win_std=1.0)
    if index == 2:
        N, H, T = s.get("N", 1), s.get("H", 32), s.get("T", 8192)
        return make_workload("prefill %dx%d T=%d fp32" % (N, H, T), seed=sd, N=N, H=H,
                             lengths=[T] * N)
    if index == 3:
        N, H, T = s.get("N", 16), s.get("H", 64), s.get("T", 2048)
        return make_workload("batched prefill %dx%d T=%d bf16" % (N, H, T), seed=sd, N=N, H=H,
                             lengths=[T] * N, act_dtype="bf16", state_std=0.02, win_std=1.0,
                             decay=(0.8, 0.999))
    if index == 4:
        N, H, mx = s.get("N", 256), s.get("H", 32), s.get("max_len", 4096)
        return make_workload("ragged %d seqs U[1,%d] x%d bf16" % (N, mx, H), seed=sd, N=N, H=H,
                             lengths=lambda rng: rng.integers(1, mx + 1, size=N),
                             act_dtype="bf16", state_std=0.02, win_std=1.0,
                             gamma_range=(0.5, 1.5), fresh_prob=0.5)
    if index == 5:
        N, H, T = s.get("N", 64), s.get("H", 32), s.get("T", 13)
        return make_workload("short prefill %dx%d T=%d fp32" % (N, H, T), seed=sd, N=N, H=H,
                             lengths=[T] * N, state_std=0.02, win_std=1.0)
    raise ValueError(index)


def decode_rows_as_sequences(w: Workload, arr: np.ndarray) -> np.ndarray:
    """Reorder a decode run's token rows from [step, seq] to [seq, step]."""
    steps, N = w.decode_steps, w.N
    return np.ascontiguousarray(arr.reshape((steps, N) + arr.shape[1:]).swapaxes(0, 1)
                                .reshape((steps * N,) + arr.shape[1:]))


def sequence_rows_as_decode(w: Workload, arr: np.ndarray) -> np.ndarray:
    """Inverse of decode_rows_as_sequences."""
    steps, N = w.decode_steps, w.N
    return np.ascontiguousarray(arr.reshape((N, steps) + arr.shape[1:]).swapaxes(0, 1)
                                .reshape((steps * N,) + arr.shape[1:]))


def decode_subset(w: Workload, seqs) -> Workload:
    """The sequences `seqs` (every head) of a decode run, as a prefill-layout
    workload of len(seqs) sequences of decode_steps tokens each, without
    reordering the other sequences' rows."""
    if not w.decode_steps:
        raise ValueError("not a decode workload")
    seqs = np.asarray(seqs, dtype=np.int64)
    steps, N = w.decode_steps, w.N

    def tok(a):
        sel = a.reshape((steps, N) + a.shape[1:])[:, seqs]          # [steps, n, ...]
        return np.ascontiguousarray(sel.swapaxes(0, 1)).reshape((steps * len(seqs),) + a.shape[1:])
    cu = np.arange(len(seqs) + 1, dtype=np.int64) * steps
    return dataclasses.replace(
        w, name=w.name + " (sequences %s)" % list(map(int, seqs)), N=len(seqs), cu_seqlens=cu,
        q=tok(w.q), k=tok(w.k), v=tok(w.v), f=tok(w.f), beta=tok(w.beta), g=tok(w.g),
        state0=np.ascontiguousarray(w.state0[seqs]), win0=np.ascontiguousarray(w.win0[seqs]),
        decode_steps=0)


def subset(w: Workload, seqs, heads) -> Workload:
    """The sub-problem made of the given sequences and heads (prefill layout)."""
    if w.decode_steps:
        raise ValueError("reorder decode rows with decode_rows_as_sequences first")
    seqs = np.asarray(seqs, dtype=np.int64)
    heads = np.asarray(heads, dtype=np.int64)
    rows = np.concatenate([np.arange(w.cu_seqlens[n], w.cu_seqlens[n + 1]) for n in seqs]) \
        if len(seqs) else np.zeros(0, np.int64)
    lens = w.lengths[seqs]
    cu = np.zeros(len(seqs) + 1, np.int64)
    cu[1:] = np.cumsum(lens)

    def tok(a):
        return np.ascontiguousarray(a[rows][:, heads])
    return dataclasses.replace(
        w, name=w.name + " (subset)", N=len(seqs), H=len(heads), cu_seqlens=cu,
        q=tok(w.q), k=tok(w.k), v=tok(w.v), f=tok(w.f), beta=tok(w.beta), g=tok(w.g),
        conv_w=np.ascontiguousarray(w.conv_w[heads]), A_log=np.ascontiguousarray(w.A_log[heads]),
        dt_bias=np.ascontiguousarray(w.dt_bias[heads]),
        state0=np.ascontiguousarray(w.state0[seqs][:, heads]),
        win0=np.ascontiguousarray(w.win0[seqs][:, heads]))


def to_device(w: Workload, device="cuda:0", *, with_o_raw: bool = True, decode_step: Optional[int] = None):
    """Device tensors for a workload (torch; plumbing only).

    Returns a dict with the kda_sequence / kda_token_step keyword tensors plus
    'cu_seqlens' (int32).  bf16 workloads get bf16 q, k, v, g and y.  For a
    decode workload, decode_step=None uploads every step's rows ([steps*N, ...],
    step-major); an integer uploads that step only."""
    import torch
    act = torch.bfloat16 if w.act_dtype == "bf16" else torch.float32

    def tok(a):
        if w.decode_steps and decode_step is not None:
            a = a[decode_step * w.N:(decode_step + 1) * w.N]
        return a

    def up_act(a):
        a = tok(a)
        if w.act_dtype == "bf16":
            return torch.from_numpy(bf16_bits(a)).to(device).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)

    def up32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)

    q = up_act(w.q)
    T = q.shape[0]
    d = dict(q=q, k=up_act(w.k), v=up_act(w.v), f=up32(tok(w.f)), beta=up32(tok(w.beta)),
             g=up_act(w.g), conv_w=up32(w.conv_w), A_log=up32(w.A_log), dt_bias=up32(w.dt_bias),
             gamma=up32(w.gamma), state=up32(w.state0), conv_win=up32(w.win0),
             y=torch.empty((T, w.H, w.dv), dtype=act, device=device),
             o_raw=torch.empty((T, w.H, w.dv), dtype=torch.float32, device=device) if with_o_raw else None)
    d["cu_seqlens"] = torch.from_numpy(w.cu_seqlens.astype(np.int32)).to(device)
    return d


# --- inputs of the projections around the step -------------------------------

@dataclasses.dataclass
class ProjectionInputs:
    """Host copy of the projection problem for T token rows (fp32 arrays;
    bf16 problems hold bf16-exact values in x, y, w_g and w_o).

    Hidden width D and rank r are not fixed by the method's description: the
    measured shapes take D = H * dk (the heads' total width) and r = dk."""
    name: str
    T: int
    H: int
    D: int
    r: int
    act_dtype: str                 # x, y, w_g, w_o, g, out
    x: np.ndarray                  # [T, D] hidden rows
    w_fa: np.ndarray               # [r, D]       fp32
    w_fb: np.ndarray               # [H * 128, r] fp32
    w_bp: np.ndarray               # [H, D]       fp32
    w_g: np.ndarray                # [H * 128, D] act dtype
    y: np.ndarray                  # [T, H * 128] act dtype (stand-in for the step's output)
    w_o: np.ndarray                # [D, H * 128] act dtype


def projection_inputs(name: str, *, seed: int, T: int, H: int, D: int, r: int = 128,
                      act_dtype: str = "f32", dk: int = 128, dv: int = 128) -> ProjectionInputs:
    """x, y ~ N(0, 1); every weight ~ N(0, 1 / fan_in), so that each product
    is ~N(0, 1) per output (beta logits ~N(0, 1) as in the step's own inputs).
    bf16 problems round x, y, w_g, w_o to bf16 (ties to even)."""
    root = np.random.SeedSequence([seed, 0x5052_4F4A])
    ss_x, ss_fa, ss_fb, ss_bp, ss_g, ss_y, ss_o = root.spawn(7)
    x = _normal(ss_x, (T, D))
    w_fa = _normal(ss_fa, (r, D), D ** -0.5)
    w_fb = _normal(ss_fb, (H * dk, r), r ** -0.5)
    w_bp = _normal(ss_bp, (H, D), D ** -0.5)
    w_g = _normal(ss_g, (H * dv, D), D ** -0.5)
    y = _normal(ss_y, (T, H * dv))
    w_o = _normal(ss_o, (D, H * dv), (H * dv) ** -0.5)
    if act_dtype == "bf16":
        for a in (x, w_g, y, w_o):
            _round_inplace_bf16(a)
    elif act_dtype != "f32":
        raise ValueError(act_dtype)
    return ProjectionInputs(name=name, T=T, H=H, D=D, r=r, act_dtype=act_dtype, x=x, w_fa=w_fa,
                            w_fb=w_fb, w_bp=w_bp, w_g=w_g, y=y, w_o=w_o)


def projection_workload(index: int, *, scale: Optional[dict] = None) -> ProjectionInputs:
    """The projections for the token rows of step workload `index` (1: the
    64 x 32 decode step's 64 rows; 2: 1 x 32 x 8192 fp32; 3: 16 x 64 x 2048
    bf16), D = H * 128, r = 128; `scale` overrides T, H, D, r for tests."""
    s = dict(scale or {})
    shapes = {1: (64, 32, "f32"), 2: (8192, 32, "f32"), 3: (32768, 64, "bf16")}
    T, H, dt = shapes[index]
    T, H = s.get("T", T), s.get("H", H)
    D, r = s.get("D", H * 128), s.get("r", 128)
    return projection_inputs("projections T=%d H=%d D=%d r=%d %s" % (T, H, D, r, dt), seed=100 + index,
                             T=T, H=H, D=D, r=r, act_dtype=dt)
