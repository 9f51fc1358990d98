"""GPU parity of the three projections on seeded random shapes: token counts
on both sides of the switch between the small (split-K) and the large tile
paths, odd head counts, hidden widths and ranks of every allowed granularity,
both activation types, with and without workspace.  Bars as in
test_gpu_projections.py (fp32 outputs 1e-4 of max|ref|; bf16 outputs 2^-8
relative plus 1e-5 of max|ref|)."""
import numpy as np
import pytest

from linear_attention_recurrence_token_amd import synth
from oracle.projections import gate_projection, lowrank_gates, output_projection
from tests.test_gpu_projections import FP32_BAR, _check_bf16, _check_fp32, _np, _run_gate, _run_lowrank, _run_out

pytestmark = pytest.mark.gpu


def _shape(seed):
    rng = np.random.default_rng(seed)
    T = int(rng.choice([1, 3, 63, 64, 65, 200, 511, 512, 513, 700, 1029]))
    H = int(rng.integers(1, 6))
    D = 32 * int(rng.integers(1, 33))
    r = 32 * int(rng.integers(1, 10))
    act = str(rng.choice(["f32", "bf16"]))
    return T, H, D, r, act, bool(rng.random() < 0.75)


@pytest.mark.parametrize("seed", range(9000, 9030))
def test_projection_random_shape(gpu, seed):
    T, H, D, r, act, ws = _shape(seed)
    print("seed %d: T=%d H=%d D=%d r=%d %s workspace=%s" % (seed, T, H, D, r, act, ws), flush=True)
    p = synth.projection_inputs("random projection", seed=seed, T=T, H=H, D=D, r=r, act_dtype=act)
    f, beta = _run_lowrank(p, gpu, "auto" if ws else "minimum")
    f_ref, beta_ref = lowrank_gates(p.x, p.w_fa, p.w_fb, p.w_bp)
    _check_fp32(f, f_ref, "f")
    assert np.max(np.abs(beta - beta_ref)) <= FP32_BAR
    check = _check_bf16 if act == "bf16" else _check_fp32
    check(_np(_run_gate(p, gpu, ws)).reshape(T, H * 128), gate_projection(p.x, p.w_g), "g")
    check(_np(_run_out(p, gpu, ws)), output_projection(p.y, p.w_o), "out")
