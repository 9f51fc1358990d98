"""CPU oracle for the projections around the KDA step -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module; the product library never does.

Plain fp64 numpy: every step is one library matrix product, taken in the
order the pages write it, with no blocking or reordering.  Token rows are
independent, so a test may pass any subset of rows.

* ``lowrank_gates`` -- the decay pre-activation f = W_fb (W_fa x) of
  "Kimi K3 Metal Gap Analysis", §2 KDA Attention, row "Decay compute"
  (gk is formed from W_fb W_fa x plus dt_bias), and beta from the third
  low-rank product bp.  "Metal (Apple GPU) backend for Kimi K3", table "What
  runs where (per layer)", row "KDA low-rank (fa,fb,bp)", runs all three as
  fp32 matrix products.  Reading: beta = sigmoid(W_bp x), no bias (the pages
  name bp but do not write beta's formula; a sigmoid keeps beta in (0, 1)).
* ``gate_projection`` -- g = W_g x, and ``output_projection`` -- out = W_o y,
  the two matrix products of Gap Analysis §2, row "O projection", on either
  side of the step's RMSNorm and sigmoid gate (y is the step's output).

Shapes: x [T, D]; W_fa [r, D]; W_fb [H * dk, r]; W_bp [H, D];
f [T, H, dk]; beta [T, H]; W_g [H * dv, D]; W_o [D, H * dv].
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def lowrank_gates(x, w_fa, w_fb, w_bp):
    """f [T, H, dk] and beta [T, H] from hidden rows x [T, D] (fp64)."""
    x, w_fa, w_fb, w_bp = _f64(x), _f64(w_fa), _f64(w_fb), _f64(w_bp)
    T = x.shape[0]
    H = w_bp.shape[0]
    assert w_fa.shape[1] == x.shape[1] and w_bp.shape[1] == x.shape[1]
    assert w_fb.shape[1] == w_fa.shape[0] and w_fb.shape[0] % H == 0
    a = x @ w_fa.T                       # [T, r]: the rank-r factor W_fa x
    f = a @ w_fb.T                       # [T, H * dk]: W_fb (W_fa x)
    z = x @ w_bp.T                       # [T, H]
    beta = 1.0 / (1.0 + np.exp(-z))
    return f.reshape(T, H, w_fb.shape[0] // H), beta


def gate_projection(x, w_g):
    """g [T, H * dv] = W_g x for hidden rows x [T, D] (fp64)."""
    x, w_g = _f64(x), _f64(w_g)
    assert w_g.shape[1] == x.shape[1]
    return x @ w_g.T


def output_projection(y, w_o):
    """out [T, D] = W_o y for step outputs y [T, H * dv] (fp64)."""
    y, w_o = _f64(y).reshape(y.shape[0], -1), _f64(w_o)
    assert w_o.shape[1] == y.shape[1]
    return y @ w_o.T
