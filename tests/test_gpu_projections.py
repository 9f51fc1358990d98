"""GPU parity of the projections around the step (kda_lowrank_gates,
kda_gate_projection, kda_output_projection) against the fp64 oracle in
oracle/projections.py, element by element.

Bars (derived from the arithmetic; the step's own bars are 1e-4 and 2e-2):
  * fp32 outputs (f, beta; g and out of fp32 problems): every product with
    an fp32 side is three bf16 products (about 2^-16 relative error each)
    summed in fp32, so max|delta| <= 1e-4 * max|ref|;
  * bf16 outputs: the fp32 sum of exact bf16 products, rounded once to bf16
    (at most 2^-9 relative), so |delta| <= 2^-8 |ref| + 1e-5 max|ref|.
Shapes span several tiles with ragged tails on both the token and the output
side, with and without the split-K scratch; the measured shapes are checked
on sampled token rows (rows are independent, so the oracle computes just
those)."""
import numpy as np
import pytest

from linear_attention_recurrence_token_amd import kda, synth
from oracle.projections import gate_projection, lowrank_gates, output_projection

pytestmark = pytest.mark.gpu

FP32_BAR = 1e-4


def _dev(a, dev, bf16=False):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return t.to(torch.bfloat16) if bf16 else t


def _cfg(H, act):
    return kda.KdaConfig(num_heads=H, act_dtype=kda.KDA_BF16 if act == "bf16" else kda.KDA_F32)


def _np(t):
    return t.double().cpu().numpy()


def _check_fp32(got, ref, what):
    err = np.max(np.abs(got - ref))
    bar = FP32_BAR * np.max(np.abs(ref))
    assert err <= bar, "%s: max|delta| %.3g > %.3g" % (what, err, bar)


def _check_bf16(got, ref, what):
    bound = 2.0 ** -8 * np.abs(ref) + 1e-5 * np.max(np.abs(ref))
    excess = np.abs(got - ref) - bound
    assert np.all(excess <= 0), "%s: worst excess %.3g over the bf16 bound" % (what, excess.max())


def _run_lowrank(p, dev, ws_mode="auto", rows=None):
    import torch
    bf = p.act_dtype == "bf16"
    x = _dev(p.x, dev, bf)
    w_fa_bp = _dev(np.concatenate([p.w_fa, p.w_bp]), dev)
    w_fb = _dev(p.w_fb, dev)
    f = torch.full((p.T, p.H, 128), float("nan"), device=dev)
    beta = torch.full((p.T, p.H), float("nan"), device=dev)
    cfg = _cfg(p.H, p.act_dtype)
    if ws_mode == "minimum":
        need = (p.T * p.r * 4 + 255) // 256 * 256
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    else:
        ws = "auto"
    kda.kda_lowrank_gates(cfg, x=x, w_fa_bp=w_fa_bp, w_fb=w_fb, f=f, beta=beta, workspace=ws)
    torch.cuda.synchronize()
    sel = slice(None) if rows is None else torch.as_tensor(rows, device=dev)
    return _np(f[sel]), _np(beta[sel])


SMALL = [  # T, H, D, r
    (1, 2, 64, 32),
    (37, 3, 96, 64),
    (300, 2, 256, 128),
    (700, 3, 160, 96),     # the large-tile path with ragged token and output tails
    (1100, 1, 544, 128),
    (530, 2, 64, 256),     # larger ranks: K of the second product spans 8 and 9 stages
    (520, 2, 64, 288),
]


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SMALL)
@pytest.mark.parametrize("ws_mode", ["auto", "minimum"])
def test_lowrank_gates_small(gpu, act, shape, ws_mode):
    T, H, D, r = shape
    p = synth.projection_inputs("lowrank test", seed=7 + T, T=T, H=H, D=D, r=r, act_dtype=act)
    f, beta = _run_lowrank(p, gpu, ws_mode)
    f_ref, beta_ref = lowrank_gates(p.x, p.w_fa, p.w_fb, p.w_bp)
    _check_fp32(f, f_ref, "f")
    assert np.max(np.abs(beta - beta_ref)) <= FP32_BAR


def _run_gate(p, dev, use_ws=True):
    import torch
    bf = p.act_dtype == "bf16"
    x = _dev(p.x, dev, bf)
    w_g = _dev(p.w_g, dev, bf)
    g = torch.full((p.T, p.H, 128), float("nan"), device=dev,
                   dtype=torch.bfloat16 if bf else torch.float32)
    kda.kda_gate_projection(_cfg(p.H, p.act_dtype), x=x, w_g=w_g, g=g, workspace="auto" if use_ws else None)
    torch.cuda.synchronize()
    return g


def _run_out(p, dev, use_ws=True):
    import torch
    bf = p.act_dtype == "bf16"
    y = _dev(p.y.reshape(p.T, p.H, 128), dev, bf)
    w_o = _dev(p.w_o, dev, bf)
    out = torch.full((p.T, p.D), float("nan"), device=dev, dtype=torch.bfloat16 if bf else torch.float32)
    kda.kda_output_projection(_cfg(p.H, p.act_dtype), y=y, w_o=w_o, out=out, workspace="auto" if use_ws else None)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SMALL)
@pytest.mark.parametrize("use_ws", [True, False])
def test_gate_and_output_projection_small(gpu, act, shape, use_ws):
    T, H, D, r = shape
    p = synth.projection_inputs("proj test", seed=11 + T, T=T, H=H, D=D, r=r, act_dtype=act)
    check = _check_bf16 if act == "bf16" else _check_fp32
    g = _np(_run_gate(p, gpu, use_ws)).reshape(T, H * 128)
    check(g, gate_projection(p.x, p.w_g), "g")
    out = _np(_run_out(p, gpu, use_ws))
    check(out, output_projection(p.y, p.w_o), "out")


def test_output_projection_hidden_not_multiple_of_32(gpu):
    # the output side needs only a multiple of 4
    p = synth.projection_inputs("proj test", seed=5, T=70, H=2, D=68, act_dtype="f32")
    _check_fp32(_np(_run_out(p, gpu)), output_projection(p.y, p.w_o), "out")


def test_zero_tokens_is_a_noop(gpu):
    import torch
    cfg = _cfg(2, "f32")
    x = torch.zeros(0, 64, device=gpu)
    kda.kda_gate_projection(cfg, x=x, w_g=torch.zeros(256, 64, device=gpu),
                            g=torch.zeros(0, 2, 128, device=gpu))


def _sample_rows(T, n=48, seed=0):
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, T - 1], rng.integers(0, T, size=n)]))
    return rows


@pytest.mark.parametrize("index", [1, 2, 3])
def test_measured_shapes_sampled_rows(gpu, index):
    """The shapes bench.py times, in the launch configuration it uses."""
    p = synth.projection_workload(index)
    rows = _sample_rows(p.T, seed=index)
    f, beta = _run_lowrank(p, gpu, rows=rows)
    f_ref, beta_ref = lowrank_gates(p.x[rows], p.w_fa, p.w_fb, p.w_bp)
    _check_fp32(f, f_ref, "f")
    assert np.max(np.abs(beta - beta_ref)) <= FP32_BAR
    check = _check_bf16 if p.act_dtype == "bf16" else _check_fp32
    import torch
    sel = torch.as_tensor(rows, device=gpu)
    g = _np(_run_gate(p, gpu)[sel]).reshape(len(rows), -1)
    check(g, gate_projection(p.x[rows], p.w_g), "g")
    out = _np(_run_out(p, gpu)[sel])
    check(out, output_projection(p.y[rows], p.w_o), "out")


def test_lowrank_gates_feed_the_step(gpu):
    """f and beta from kda_lowrank_gates drive kda_sequence to the oracle's
    result for the same hidden rows (the projections and the step composed)."""
    import dataclasses
    import torch
    from tests import _gpu
    w = synth.workload(0, scale={"T": 40})
    p = synth.projection_inputs("compose", seed=3, T=w.total_tokens, H=w.H, D=96, r=32)
    f_ref, beta_ref = lowrank_gates(p.x, p.w_fa, p.w_fb, p.w_bp)
    ref = _gpu.oracle_sequence(dataclasses.replace(w, f=f_ref.astype(np.float32),
                                                   beta=beta_ref.astype(np.float32)))
    d = synth.to_device(w, gpu, with_o_raw=True)
    kda.kda_lowrank_gates(_cfg(w.H, "f32"), x=_dev(p.x, gpu),
                          w_fa_bp=_dev(np.concatenate([p.w_fa, p.w_bp]), gpu),
                          w_fb=_dev(p.w_fb, gpu), f=d["f"], beta=d["beta"])
    kda.kda_sequence(_gpu.cfg_of(w), **_gpu.tensors(d), cu_seqlens=d["cu_seqlens"], num_seqs=w.N)
    torch.cuda.synchronize()
    got = {"y": _np(d["y"]), "o_raw": _np(d["o_raw"]), "state": _np(d["state"]),
           "win": d["conv_win"].cpu().numpy()}
    _gpu.assert_parity(got, ref, label="low-rank gates -> step")


@pytest.mark.parametrize("T,H,D", [(4200, 32, 64), (4200, 2, 4352)])
def test_bf16_many_tiles_every_element(gpu, T, H, D):
    """More than two grid rounds of 128-token x 256-output tiles, with ragged
    tiles on the token side and (4352 outputs) on the output side; every
    element is checked."""
    p = synth.projection_inputs("many tiles", seed=T + D, T=T, H=H, D=D, r=32, act_dtype="bf16")
    if H * 128 > 1024:
        g = _np(_run_gate(p, gpu)).reshape(T, H * 128)
        _check_bf16(g, gate_projection(p.x, p.w_g), "g")
    else:
        out = _np(_run_out(p, gpu))
        _check_bf16(out, output_projection(p.y, p.w_o), "out")
