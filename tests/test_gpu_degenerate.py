"""The degenerate inputs of the step through every kernel, against the oracle
(the bars of tests/test_gpu_parity.py): zero raw inputs (every activation 0,
so the L2 and RMS norms see only their epsilons), beta = 0 (the state only
decays) and beta = 1, the bounded decay at its two ends (alpha -> e^lb and
alpha -> 1), saturated output gates, and inputs scaled by 1e3 and 1e-3 (the
L2 norm removes the scale of q and k).  Each case runs every prefill path and
the decode step on a small carried-state problem."""
import dataclasses

import numpy as np
import pytest

from linear_attention_recurrence_token_amd import synth
from tests import _gpu

pytestmark = pytest.mark.gpu

PATHS = ["fused", "split", "chunk", "short", "scan", "chunk_short"]


def note(msg):
    print(msg, flush=True)


def _base(seed, N=2, H=3, T=40):
    return synth.make_workload("degenerate", seed=seed, N=N, H=H, lengths=[T] * N, state_std=0.02, win_std=1.0)


def _zero_inputs(w):
    # tokens 5..20 of every sequence and the whole window: all-zero raw rows
    # (then three tokens in, every activation of those tokens is exactly 0)
    q, k, v = w.q.copy(), w.k.copy(), w.v.copy()
    for n in range(w.N):
        lo = w.cu_seqlens[n]
        for a in (q, k, v):
            a[lo + 5:lo + 21] = 0.0
    return dataclasses.replace(w, q=q, k=k, v=v, win0=np.zeros_like(w.win0))


def _beta(value):
    def f(w):
        return dataclasses.replace(w, beta=np.full_like(w.beta, value))
    return f


def _decay_end(strong):
    # bounded gate: f far above -dt_bias gives sigma -> 1 (alpha -> e^lb), far
    # below gives sigma -> 0 (alpha -> 1)
    def f(w):
        return dataclasses.replace(w, f=np.full_like(w.f, 60.0 if strong else -60.0))
    return f


def _gates(w):
    g = np.where(np.arange(w.g.size).reshape(w.g.shape) % 2 == 0, 30.0, -30.0).astype(np.float32)
    return dataclasses.replace(w, g=g)


def _scale(s):
    def f(w):
        return dataclasses.replace(w, q=w.q * np.float32(s), k=w.k * np.float32(s), v=w.v * np.float32(s),
                                   win0=w.win0 * np.float32(s))
    return f


CASES = {"zero_inputs": _zero_inputs, "beta0": _beta(0.0), "beta1": _beta(1.0),
         "strongest_decay": _decay_end(True), "no_decay": _decay_end(False), "saturated_gates": _gates,
         "scale_1e3": _scale(1e3), "scale_1e-3": _scale(1e-3)}


@pytest.mark.parametrize("case", list(CASES))
@pytest.mark.parametrize("path", PATHS)
def test_degenerate_prefill(gpu, case, path):
    w = CASES[case](_base(seed=31))
    note("degenerate %s, prefill %s" % (case, path))
    _gpu.assert_parity(_gpu.run_sequence(w, gpu, path=path), _gpu.oracle_sequence(w), label="%s %s" % (case, path))


@pytest.mark.parametrize("case", list(CASES))
def test_degenerate_decode(gpu, case):
    w = synth.make_workload("degenerate decode", seed=32, N=4, H=3, decode_steps=24, state_std=0.02, win_std=1.0)
    # apply the case to the sequence-major layout, then back to step-major rows
    seqw, _ = _gpu.decode_as_prefill(w)
    c = CASES[case](seqw)
    w = dataclasses.replace(w, win0=c.win0, **{a: synth.sequence_rows_as_decode(w, getattr(c, a))
                                              for a in ("q", "k", "v", "f", "beta", "g")})
    note("degenerate %s, decode" % case)
    _gpu.assert_parity(_gpu.run_decode(w, gpu), _gpu.oracle_decode(w), label="%s decode" % case)
