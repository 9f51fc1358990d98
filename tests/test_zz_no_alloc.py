"""The no-allocation entry point, kda_lowrank_gates_noalloc, against the
entry point it varies, kda_lowrank_gates with a workspace, through the C ABI
(ctypes, arguments marshalled by hand): two calls in a row on one device, the
second with fewer token rows (the static scratch keeps the first call's
contents), each compared with its own workspace call; both are held to the
fp32 bar of the projections (1e-4 of max) and, since they run the same kernels
with the same plan, to bit equality.  Runs last: a failure here must not hide
the other GPU tests."""
import ctypes

import numpy as np
import pytest

from linear_attention_recurrence_token_amd import kda, synth

pytestmark = pytest.mark.gpu


def _call_pair(dev, T, H, D, r, act):
    import torch
    p = synth.projection_inputs("noalloc T=%d" % T, seed=900 + T, T=T, H=H, D=D, r=r, act_dtype=act)
    bf = act == "bf16"
    dt = torch.bfloat16 if bf else torch.float32
    x = torch.from_numpy(p.x).to(dev).to(dt)
    wab = torch.from_numpy(np.concatenate([p.w_fa, p.w_bp])).to(dev)
    wfb = torch.from_numpy(p.w_fb).to(dev)
    cfg = kda.KdaConfig(num_heads=H, act_dtype=kda.KDA_BF16 if bf else kda.KDA_F32).to_c()
    L = kda.lib()
    outs = []
    for noalloc in (False, True):
        f = torch.full((T, H, 128), float("nan"), device=dev)
        beta = torch.full((T, H), float("nan"), device=dev)
        if noalloc:
            st = L.kda_lowrank_gates_noalloc(ctypes.byref(cfg), x.data_ptr(), wab.data_ptr(), wfb.data_ptr(),
                                             D, r, T, f.data_ptr(), beta.data_ptr(), None)
        else:
            need = L.kda_projection_workspace_size(ctypes.byref(cfg), kda.KDA_PROJ_LOWRANK_GATES, D, r, T)
            assert need > 0
            ws = torch.empty(need, dtype=torch.uint8, device=dev)
            st = L.kda_lowrank_gates(ctypes.byref(cfg), x.data_ptr(), wab.data_ptr(), wfb.data_ptr(), D, r, T,
                                     f.data_ptr(), beta.data_ptr(), ws.data_ptr(), need, None)
        assert st == kda.KDA_OK, kda.status_string(st)
        torch.cuda.synchronize()
        outs.append((f.double().cpu().numpy(), beta.double().cpu().numpy()))
    return outs


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_lowrank_gates_noalloc_two_calls(gpu, act):
    # first call: 2048 rows (the weights split into bf16 parts in the scratch);
    # second: 64 rows (split-K partial sums in the scratch over what the first
    # call left there)
    for T, H, D, r in ((2048, 8, 1024, 128), (64, 32, 4096, 128)):
        print("noalloc lowrank gates T=%d H=%d D=%d r=%d %s" % (T, H, D, r, act), flush=True)
        (f_ws, b_ws), (f_na, b_na) = _call_pair(gpu, T, H, D, r, act)
        for got, ref, what in ((f_na, f_ws, "f"), (b_na, b_ws, "beta")):
            assert np.all(np.isfinite(got)), what
            assert np.max(np.abs(got - ref)) <= 1e-4 * np.max(np.abs(ref)), what
            np.testing.assert_array_equal(got, ref, err_msg=what)


def test_lowrank_gates_noalloc_rejects_sizes_beyond_the_scratch(gpu):
    import torch
    # tokens * rank * 4 > 16 MiB: refused before anything is enqueued
    T, H, D, r = 33000, 1, 32, 128
    cfg = kda.KdaConfig(num_heads=H).to_c()
    x = torch.zeros((T, D), device=gpu)
    wab = torch.zeros((r + H, D), device=gpu)
    wfb = torch.zeros((H * 128, r), device=gpu)
    f = torch.zeros((T, H, 128), device=gpu)
    beta = torch.zeros((T, H), device=gpu)
    st = kda.lib().kda_lowrank_gates_noalloc(ctypes.byref(cfg), x.data_ptr(), wab.data_ptr(), wfb.data_ptr(),
                                            D, r, T, f.data_ptr(), beta.data_ptr(), None)
    assert st == kda.KDA_ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert not f.any() and not beta.any()
