"""The step with its decay pre-activation formed inside it from the low-rank
factor (kda_lowrank_factor, then kda_sequence_lowrank) against the oracle:
f and beta from the projections' oracle (f = W_fb (W_fa x), beta =
sigmoid(W_bp x) in fp64, "Kimi K3 Metal Gap Analysis", §2, row "Decay
compute"), then the step's oracle on those values.  Bars: the step's (y, o_raw
and the state within 1e-4 of max with fp32 inputs, y within 2e-2 with bf16;
o_raw and the state at 1e-4 either way; the window bit-exact).  The in-step f
is a split-bf16 product (about 2^-16 relative per product), of the same size
as the error of the separate low-rank product, which the same bars hold."""
import dataclasses

import numpy as np
import pytest

from linear_attention_recurrence_token_amd import kda, synth
from oracle.projections import lowrank_gates
from tests import _gpu

pytestmark = pytest.mark.gpu


def note(msg):
    print(msg, flush=True)


def _run_fused(w, p, dev, with_o_raw=True, order=None):
    import torch
    bf = w.act_dtype == "bf16"
    d = synth.to_device(w, dev, with_o_raw=with_o_raw)
    x = torch.from_numpy(p.x).to(dev)
    x = x.to(torch.bfloat16) if bf else x
    cfg = _gpu.cfg_of(w)
    a = torch.full((w.total_tokens, p.r), float("nan"), device=dev)
    d["beta"].fill_(float("nan"))
    kda.kda_lowrank_factor(cfg, x=x, w_fa_bp=torch.from_numpy(np.concatenate([p.w_fa, p.w_bp])).to(dev),
                           a=a, beta=d["beta"])
    ts = _gpu.tensors(d)
    ts.pop("f")
    kda.kda_sequence_lowrank(cfg, **ts, a=a, w_fb=torch.from_numpy(p.w_fb).to(dev), cu_seqlens=d["cu_seqlens"],
                             seq_order=order, num_seqs=w.N)
    torch.cuda.synchronize()
    return d


def _oracle(w, p):
    f, beta = lowrank_gates(p.x, p.w_fa, p.w_fb, p.w_bp)
    return _gpu.oracle_sequence(dataclasses.replace(w, f=f.astype(np.float32), beta=beta.astype(np.float32)))


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("rank", [32, 96, 128])
def test_lowrank_step_small(gpu, act, rank):
    # ragged lengths across the chunk size, carried state and window
    w = synth.make_workload("lowrank step", seed=500 + rank, N=3, H=3, lengths=[300, 17, 1], act_dtype=act,
                            state_std=0.02, win_std=1.0)
    p = synth.projection_inputs("lowrank step", seed=600 + rank, T=w.total_tokens, H=w.H, D=160, r=rank,
                                act_dtype=act)
    note("low-rank step 3x3 (300, 17, 1) rank %d %s" % (rank, act))
    d = _run_fused(w, p, gpu)
    got = {"y": _gpu._np(d["y"]), "o_raw": _gpu._np(d["o_raw"]), "state": _gpu._np(d["state"]),
           "win": d["conv_win"].cpu().numpy()}
    errs = _gpu.assert_parity(got, _oracle(w, p), bf16=act == "bf16", label="low-rank step")
    note("errors %s" % errs)


def test_lowrank_step_matches_the_separate_products(gpu):
    # kda_lowrank_gates + kda_sequence (f through memory) and the fused call
    # agree to the step's tolerance (not bit for bit: f is summed differently)
    import torch
    w = synth.make_workload("lowrank vs separate", seed=42, N=2, H=4, lengths=[260, 100], act_dtype="bf16",
                            state_std=0.02, win_std=1.0)
    p = synth.projection_inputs("lowrank vs separate", seed=43, T=w.total_tokens, H=w.H, D=256, r=128,
                                act_dtype="bf16")
    note("low-rank step against kda_lowrank_gates + kda_sequence")
    fused = _run_fused(w, p, gpu)
    d = synth.to_device(w, gpu)
    x = torch.from_numpy(p.x).to(gpu).to(torch.bfloat16)
    kda.kda_lowrank_gates(_gpu.cfg_of(w), x=x, w_fa_bp=torch.from_numpy(np.concatenate([p.w_fa, p.w_bp])).to(gpu),
                          w_fb=torch.from_numpy(p.w_fb).to(gpu), f=d["f"], beta=d["beta"])
    kda.kda_sequence(_gpu.cfg_of(w, prefill_path=kda.KDA_PREFILL_CHUNK), **_gpu.tensors(d),
                     cu_seqlens=d["cu_seqlens"], num_seqs=w.N)
    torch.cuda.synchronize()
    for k in ("o_raw", "state"):
        e = _gpu.rel_err(_gpu._np(fused[k]), _gpu._np(d[k]))
        assert e <= 1e-4, (k, e)
    assert _gpu.rel_err(_gpu._np(fused["y"]), _gpu._np(d["y"])) <= 2e-2
    np.testing.assert_array_equal(fused["conv_win"].cpu().numpy(), d["conv_win"].cpu().numpy())


def test_lowrank_step_full_16x64x2048(gpu):
    # the batched prefill shape (bf16, 16 sequences x 64 heads x 2048 tokens,
    # hidden 8192, rank 128) as the layer line of the bench runs it;
    # sequences 0 and 15 at heads 3 and 60 against the oracle
    import torch
    w = synth.workload(3)
    p = synth.projection_workload(3)
    seqs, heads = [0, 15], [3, 60]
    note("low-rank step full 16x64x2048 bf16, sequences %s heads %s" % (seqs, heads))
    d = _run_fused(w, p, gpu, with_o_raw=True,
                   order=torch.as_tensor(np.arange(w.N)[::-1].astype(np.int32).copy(), device=gpu))
    rows = np.concatenate([np.arange(w.cu_seqlens[n], w.cu_seqlens[n + 1]) for n in seqs])
    rs, hs, ns = (torch.as_tensor(v, device=gpu) for v in (rows, heads, seqs))
    got = {"y": _gpu._np(d["y"].index_select(0, rs).index_select(1, hs)),
           "o_raw": _gpu._np(d["o_raw"].index_select(0, rs).index_select(1, hs)),
           "state": _gpu._np(d["state"].index_select(0, ns).index_select(1, hs)),
           "win": d["conv_win"].index_select(0, ns).index_select(1, hs).cpu().numpy()}
    del d
    torch.cuda.empty_cache()
    f, beta = lowrank_gates(p.x[rows], p.w_fa, p.w_fb, p.w_bp)
    full_f = np.zeros_like(w.f)
    full_b = np.zeros_like(w.beta)
    full_f[rows] = f
    full_b[rows] = beta
    sub = synth.subset(dataclasses.replace(w, f=full_f, beta=full_b), seqs, heads)
    errs = _gpu.assert_parity(got, _gpu.oracle_sequence(sub), bf16=True, label="low-rank step full")
    note("errors %s" % errs)
