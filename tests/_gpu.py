"""Helpers for the GPU parity tests: run the HIP path through the binding,
run the oracle on the same seeded inputs, compare."""
import dataclasses

import numpy as np

import oracle
from linear_attention_recurrence_token_amd import kda, synth

FP32_TOL = 1e-4     # max|delta| <= 1e-4 * max|ref| (fp32 inputs)
BF16_TOL = 2e-2     # max|delta| <= 2e-2 * max|ref| (bf16 inputs / outputs)


def cfg_of(w, **over):
    c = kda.KdaConfig(num_heads=w.H, act_dtype=kda.KDA_BF16 if w.act_dtype == "bf16" else kda.KDA_F32,
                      gate_mode=w.gate_mode, gate_lower_bound=w.lower_bound,
                      l2_eps=w.l2_eps, rms_eps=w.rms_eps)
    for k, v in over.items():
        setattr(c, k, v)
    return c


def _np(t):
    return t.double().cpu().numpy()


def tensors(d):
    return {k: d[k] for k in kda.TENSOR_FIELDS}


PATHS = {"fused": kda.KDA_PREFILL_FUSED, "split": kda.KDA_PREFILL_SPLIT, "auto": kda.KDA_PREFILL_AUTO,
         "chunk": kda.KDA_PREFILL_CHUNK, "short": kda.KDA_PREFILL_SHORT, "scan": kda.KDA_PREFILL_SCAN,
         "chunk_short": kda.KDA_PREFILL_CHUNK_SHORT}


def run_sequence(w, dev, *, with_o_raw=True, seq_order=None, dense=False, path="auto", side_stream=False,
                 cu_host=False, workspace="auto"):
    """One kda_sequence call; side_stream: pass a second stream (the two-pass
    path may then run in segments); cu_host: pass the host copy of the
    offsets too; workspace: "auto" (the size the library asks for) or None."""
    import torch
    d = synth.to_device(w, dev, with_o_raw=with_o_raw)
    order = None if seq_order is None else torch.as_tensor(np.asarray(seq_order, np.int32), device=dev)
    side = torch.cuda.Stream(device=dev) if side_stream else None
    kda.kda_sequence(cfg_of(w, prefill_path=PATHS[path]), **tensors(d),
                     cu_seqlens=None if dense else d["cu_seqlens"],
                     cu_seqlens_host=w.cu_seqlens.astype(np.int32) if (cu_host and not dense) else None,
                     seq_order=order, num_seqs=w.N, side_stream=side, workspace=workspace)
    torch.cuda.synchronize()
    out = {"y": _np(d["y"]), "state": _np(d["state"]), "win": d["conv_win"].cpu().numpy()}
    out["o_raw"] = _np(d["o_raw"]) if with_o_raw else None
    return out


def run_decode(w, dev, *, steps=None, with_o_raw=True):
    """Chain kda_token_step over the decode steps of w (rows step-major)."""
    import torch
    steps = w.decode_steps if steps is None else steps
    d = synth.to_device(w, dev, with_o_raw=with_o_raw)
    N = w.N
    cfg = cfg_of(w)
    for s in range(steps):
        sl = slice(s * N, (s + 1) * N)
        kda.kda_token_step(cfg, q=d["q"][sl], k=d["k"][sl], v=d["v"][sl], f=d["f"][sl],
                           beta=d["beta"][sl], g=d["g"][sl], conv_w=d["conv_w"], A_log=d["A_log"],
                           dt_bias=d["dt_bias"], gamma=d["gamma"], state=d["state"],
                           conv_win=d["conv_win"], y=d["y"][sl],
                           o_raw=d["o_raw"][sl] if with_o_raw else None)
    torch.cuda.synchronize()
    T = steps * N
    out = {"y": _np(d["y"][:T]), "state": _np(d["state"]), "win": d["conv_win"].cpu().numpy()}
    out["o_raw"] = _np(d["o_raw"][:T]) if with_o_raw else None
    return out


def oracle_sequence(w):
    return oracle.kda_reference(w.q, w.k, w.v, w.f, w.beta, w.g, w.conv_w, w.A_log, w.dt_bias,
                                w.gamma, w.state0, w.win0, w.cu_seqlens, gate_mode=w.gate_mode,
                                lower_bound=w.lower_bound, l2_eps=w.l2_eps, rms_eps=w.rms_eps)


def decode_as_prefill(w, steps=None):
    """The decode workload w (first `steps` steps) laid out as sequences."""
    steps = w.decode_steps if steps is None else steps
    T = steps * w.N
    ww = dataclasses.replace(w, decode_steps=steps, q=w.q[:T], k=w.k[:T], v=w.v[:T], f=w.f[:T],
                             beta=w.beta[:T], g=w.g[:T])
    re = {k: synth.decode_rows_as_sequences(ww, getattr(ww, k)) for k in ("q", "k", "v", "f", "beta", "g")}
    cu = np.arange(w.N + 1, dtype=np.int64) * steps
    return dataclasses.replace(ww, decode_steps=0, cu_seqlens=cu, **re), ww


def oracle_decode(w, steps=None):
    seqw, ww = decode_as_prefill(w, steps)
    r = oracle_sequence(seqw)
    r["y"] = synth.sequence_rows_as_decode(ww, r["y"])
    r["o_raw"] = synth.sequence_rows_as_decode(ww, r["o_raw"])
    return r


def rel_err(got, ref):
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    if ref.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref))) / max(scale, 1e-30)


def assert_parity(got, ref, *, bf16=False, keys=("y", "o_raw", "state"), label=""):
    tol_y = BF16_TOL if bf16 else FP32_TOL
    errs = {}
    for k in keys:
        if got.get(k) is None:
            continue
        e = rel_err(got[k], ref[k])
        errs[k] = e
        # o_raw and the state are fp32 on both sides, from identical (bf16-exact)
        # inputs: hold them to the fp32 bound even for bf16 workloads
        tol = tol_y if k == "y" else FP32_TOL
        assert e <= tol, "%s %s: rel err %.3g > %.1g" % (label, k, e, tol)
    np.testing.assert_array_equal(got["win"], ref["win"].astype(np.float32), err_msg=label + " window")
    return errs
