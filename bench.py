#!/usr/bin/env python3
"""Throughput of the fused KDA token step on one MI355X.

Headline (one JSON line on stdout): decode over 64 sequences x 32 heads,
dk = dv = 128, fp32 state, one kda_token_step launch per token, K steps back
to back with every step's inputs already resident in HBM.  value = total
token.heads per second.  Alongside: the decode kernel's HBM roofline, the CPU
oracle timed on this host on a bounded sample (its only use here; parity is
checked by the GPU tests at these same sizes), a disclosed over-cache decode
run, the prefill workloads (kda_sequence): the long ones with their ALU
roofline, the short multi-token one (64 x 32 x 13 tokens) with its HBM
roofline; and the projections on either side of the step (low-rank decay and
beta, output gate, output) for the decode and the batched-prefill token rows.

  python bench.py [--gpus 1] [--steps 1000] [--warmup 10]
                  [--prefill default|all|none] [--no-cpu-baseline] [--no-overcache]
"""
import argparse
import ctypes
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA tokens·heads/sec (decode + prefill); achieved HBM GB/s vs peak"
UNIT = "token·heads/s"
HBM_PEAK_GBS = 8000.0                 # MI355X HBM3E, published
FP32_VECTOR_PEAK_TFLOPS = 157.3       # MI355X fp32 vector, published (packed FP32)
DK = DV = 128
STATE_BYTES = DK * DV * 4 * 2         # state read + write per (sequence, head) per decode token
# per decode token.head: q, k, v (3 x 512) + window in/out (2 x 3 x 384 x 4) + f 512 + beta 4 + g 512 + y 512
DECODE_OTHER_BYTES = 3 * 512 + 2 * 3 * 384 * 4 + 512 + 4 + 512 + 512
RECUR_FLOPS = 7 * DK * DV             # u, p dot products (2 FMAs), decay multiply, rank-1 FMA


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def file_sha(path):
    h = hashlib.sha256()
    with open(path, "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()[:16]


def committed_traffic(kernel_file, workload_key):
    """HBM bytes per dispatch from the committed rocprofv3 PMC summary, if it was
    taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.txt" % workload_key)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    src = os.path.join(ROOT, "linear_attention_recurrence_token_amd", "csrc", kernel_file)
    if vals.get("kernel_source_sha256_16") != file_sha(src):
        return None
    try:
        return float(vals["hbm_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None


def rocm_smi_snapshot():
    try:
        out = subprocess.run(["rocm-smi", "--showtemp", "--showpower", "--showclocks", "--json"],
                             capture_output=True, text=True, timeout=20)
        data = json.loads(out.stdout)
        card = data[sorted(data)[0]]
        keep = {}
        for k, v in card.items():
            kl = k.lower()
            if any(s in kl for s in ("temperature (sensor junction)", "power", "sclk", "mclk")):
                keep[k] = v
        return keep
    except Exception as e:  # the snapshot is informational only
        return {"error": str(e)[:80]}


class TokenStepRunner:
    """Pre-marshalled kda_token_step calls, one per decode step."""

    def __init__(self, kda, cfg, d, N, steps, stream):
        self.L = kda.lib()
        self.cfg = cfg.to_c()
        self.N = N
        self.sh = stream.cuda_stream
        self.structs = []
        H = cfg.num_heads
        for s in range(steps):
            off = s * N

            def ptr(name, per_row):
                t = d[name]
                return t.data_ptr() + off * per_row * t.element_size()
            vals = {}
            for name in ("q", "k", "v", "f", "g", "y"):
                vals[name] = ptr(name, H * DK)
            vals["beta"] = ptr("beta", H)
            for name in ("conv_w", "A_log", "dt_bias", "gamma", "state", "conv_win"):
                vals[name] = d[name].data_ptr()
            vals["o_raw"] = None
            self.structs.append(kda.kda_tensors(*[vals[n] for n in kda.TENSOR_FIELDS]))

    def run(self, s):
        st = self.L.kda_token_step(ctypes.byref(self.cfg), ctypes.byref(self.structs[s]), self.N, self.sh)
        if st != 0:
            raise RuntimeError("kda_token_step returned %d" % st)


def bench_decode(torch, kda, synth, dev, N, H, steps, warmup):
    w = synth.workload(1, scale={"N": N, "H": H, "steps": steps})
    d = synth.to_device(w, dev, with_o_raw=False)
    state0, win0 = d["state"].clone(), d["conv_win"].clone()
    cfg = kda.KdaConfig(num_heads=H)
    stream = torch.cuda.current_stream()
    runner = TokenStepRunner(kda, cfg, d, N, steps, stream)
    for s in range(warmup):
        runner.run(s % steps)
    d["state"].copy_(state0)
    d["conv_win"].copy_(win0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for s in range(steps):
        runner.run(s)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1)
    res = {"w": w, "ms_total": ms, "wall_s": wall}
    del d, state0, win0
    torch.cuda.empty_cache()
    return res


def decode_as_prefill(synth, w, steps=None):
    import dataclasses
    import numpy as np
    steps = w.decode_steps if steps is None else steps
    T = steps * w.N
    ww = dataclasses.replace(w, decode_steps=steps, q=w.q[:T], k=w.k[:T], v=w.v[:T], f=w.f[:T],
                             beta=w.beta[:T], g=w.g[:T])
    re = {k: synth.decode_rows_as_sequences(ww, getattr(ww, k)) for k in ("q", "k", "v", "f", "beta", "g")}
    cu = np.arange(w.N + 1, dtype=np.int64) * steps
    return dataclasses.replace(ww, decode_steps=0, cu_seqlens=cu, **re)


def cpu_baseline_decode(synth, w, target_s):
    """The oracle as it stands, on this host, over all (sequence, head) pairs of
    the decode workload for as many of its steps as fit in about target_s."""
    import oracle

    def run(steps):
        sw = decode_as_prefill(synth, w, steps)
        t = time.perf_counter()
        oracle.kda_reference(sw.q, sw.k, sw.v, sw.f, sw.beta, sw.g, sw.conv_w, sw.A_log,
                             sw.dt_bias, sw.gamma, sw.state0, sw.win0, sw.cu_seqlens,
                             want_o_raw=False)
        return time.perf_counter() - t
    t1 = run(2) / 2.0
    steps = int(max(1, min(w.decode_steps, target_s / max(t1, 1e-6))))
    wall = run(steps)
    passes = 1
    # when the workload's steps fit in well under the target, run the same
    # steps again (from the same initial state) until about target_s of oracle
    # work is timed
    while wall < 0.8 * target_s:
        wall += run(steps)
        passes += 1
    th = w.N * w.H * steps * passes
    return {"value": th / wall, "unit": UNIT, "cores": oracle.omp_threads(), "kind": "oracle",
            "sample": "all %d x %d (sequence, head) pairs, first %d decode steps x %d pass(es), fp64 oracle, %.1f s"
                      % (w.N, w.H, steps, passes, wall)}


def bench_prefill(torch, kda, synth, dev, idx, runs):
    import numpy as np
    w = synth.workload(idx)
    d = synth.to_device(w, dev, with_o_raw=False)
    state0, win0 = d["state"].clone(), d["conv_win"].clone()
    cfg = kda.KdaConfig(num_heads=w.H, act_dtype=kda.KDA_BF16 if w.act_dtype == "bf16" else kda.KDA_F32)
    stream = torch.cuda.current_stream()
    L = kda.lib()
    ccfg = cfg.to_c()
    t = kda.kda_tensors(*[(d[n].data_ptr() if d.get(n) is not None else None) for n in kda.TENSOR_FIELDS])
    cu = d["cu_seqlens"].data_ptr()
    lens = w.lengths
    order = torch.from_numpy(np.argsort(-lens, kind="stable").astype(np.int32)).to(dev)
    ws_bytes = kda.sequence_workspace_size(cfg, w.N, w.total_tokens)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    ws_ptr = ws.data_ptr() if ws_bytes > 0 else None

    def launch():
        st = L.kda_sequence(ctypes.byref(ccfg), ctypes.byref(t), w.N, cu, order.data_ptr(),
                            w.total_tokens, ws_ptr, ws_bytes, stream.cuda_stream)
        if st != 0:
            raise RuntimeError("kda_sequence returned %d" % st)
    times = []
    for r in range(runs + 1):
        d["state"].copy_(state0)
        d["conv_win"].copy_(win0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        launch()
        e1.record(stream)
        torch.cuda.synchronize()
        if r:
            times.append(e0.elapsed_time(e1))
    ms = float(np.median(times))
    th = int(lens.sum()) * w.H
    # the kernel the automatic choice runs (the library's rule: the short-
    # sequence kernel under 8 tokens per sequence on average; else, for the
    # bounded gate with |lower bound| <= 7.5, the two-pass chunk path for at
    # most 64 pairs averaging 128 tokens or more (given its workspace) and the
    # one-pass chunk kernel otherwise; else split / fused)
    short = w.total_tokens < 8 * w.N
    chunk = (cfg.gate_mode == kda.KDA_GATE_BOUNDED and -7.5 <= cfg.gate_lower_bound <= 0.0
             and not short)
    scan = chunk and w.N * w.H <= 64 and w.total_tokens >= 128 * w.N and ws_bytes > 0
    path = ("short" if short else ("scan" if scan else ("chunk" if chunk else
                                                        ("split" if ws_bytes > 0 else "fused"))))
    # HBM traffic from the committed rocprofv3 summary of this workload, if it
    # was taken on the current source of the kernel that runs it
    traffic = None
    keys = {2: "prefill_1x32x8192", 3: "prefill_16x64x2048", 4: "prefill_ragged_256x32", 5: "prefill_short_64x32x13"}
    if path in ("chunk", "scan") and idx in keys:
        traffic = committed_traffic("kda_prefill_%s.hip" % path, keys[idx])
    flops = th * RECUR_FLOPS
    # algorithmic HBM bytes: state in+out and window in+out per pair, and per
    # token.head q, k, v, g, y (activation dtype) with f (fp32) and beta
    act_bytes = 2 if w.act_dtype == "bf16" else 4
    per_token = 5 * 128 * act_bytes + 512 + 4
    hbm_bytes = w.N * w.H * (2 * DK * DV * 4 + 2 * 3 * 384 * 4) + th * per_token
    out = {"workload": w.name, "path": path, "token_heads": th, "ms": ms, "runs": runs,
           "value": th / (ms * 1e-3), "unit": UNIT,
           "ns_per_token_per_chain": ms * 1e6 / int(lens.max()),
           "hbm_GBps_algorithmic": hbm_bytes / (ms * 1e-3) / 1e9}
    if idx == 5:
        # a few tokens per (sequence, head): the state round trip dominates
        out["roofline"] = {"bound": "hbm", "achieved": hbm_bytes / (ms * 1e-3) / 1e9,
                           "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": hbm_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "traffic": traffic}
    else:
        out["roofline"] = {"bound": "alu", "achieved": flops / (ms * 1e-3) / 1e12,
                           "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": flops / (ms * 1e-3) / 1e12 / FP32_VECTOR_PEAK_TFLOPS,
                           "traffic": traffic}
    del d, state0, win0
    torch.cuda.empty_cache()
    return out


MFMA_BF16_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 matrix cores, published
MFMA_FP32_PEAK_TFLOPS = 157.3         # MI355X dense fp32 matrix cores, published


def bench_projections(torch, kda, synth, dev, idx, runs, only=None):
    """The matrix products on either side of the step for the token rows of
    step workload idx: kda_lowrank_gates (f and beta), kda_gate_projection
    (g) and kda_output_projection (W_o y), each timed alone (only: one of
    'lowrank', 'gate', 'output' for profiling runs)."""
    import numpy as np
    p = synth.projection_workload(idx)
    bf = p.act_dtype == "bf16"
    act = torch.bfloat16 if bf else torch.float32
    eb = 2 if bf else 4
    cfg = kda.KdaConfig(num_heads=p.H, act_dtype=kda.KDA_BF16 if bf else kda.KDA_F32)
    x = torch.from_numpy(p.x).to(dev).to(act)
    wab = torch.from_numpy(np.concatenate([p.w_fa, p.w_bp])).to(dev)
    wfb = torch.from_numpy(p.w_fb).to(dev)
    f = torch.empty(p.T, p.H, 128, device=dev)
    beta = torch.empty(p.T, p.H, device=dev)
    wg = torch.from_numpy(p.w_g).to(dev).to(act)
    g = torch.empty(p.T, p.H, 128, device=dev, dtype=act)
    y = torch.from_numpy(p.y).to(dev).to(act).view(p.T, p.H, 128)
    wo = torch.from_numpy(p.w_o).to(dev).to(act)
    out = torch.empty(p.T, p.D, device=dev, dtype=act)
    T, H, D, r, HD = p.T, p.H, p.D, p.r, p.H * 128
    stream = torch.cuda.current_stream()
    ws = {}
    for which, rank in ((kda.KDA_PROJ_LOWRANK_GATES, r), (kda.KDA_PROJ_GATE, 0), (kda.KDA_PROJ_OUTPUT, 0)):
        n = kda.projection_workspace_size(cfg, which, D, T, rank)
        ws[which] = torch.empty(max(n, 1), dtype=torch.uint8, device=dev) if n > 0 else None

    # the C entry points with their arguments marshalled once, so that the
    # events time the GPU work of each call, not the binding's host-side checks
    L = kda.lib()
    ccfg = cfg.to_c()
    sh = stream.cuda_stream

    def wsa(which):
        t = ws[which]
        return (t.data_ptr(), t.numel()) if t is not None else (None, 0)

    def c_call(fn, *args):
        def run():
            st = fn(ctypes.byref(ccfg), *args, sh)
            if st != 0:
                raise RuntimeError("%s returned %d" % (fn.__name__, st))
        return run

    def timed(fn):
        # back-to-back calls between the events, as many as make about 2 ms of
        # GPU work (one probe call sizes the batch), median over runs batches
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        calls = int(min(200, max(1, 2.0 / max(e0.elapsed_time(e1), 1e-3))))
        times = []
        for rep in range(runs + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(calls):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            if rep:
                times.append(e0.elapsed_time(e1) / calls)
        return float(np.median(times))

    res = {"workload": p.name, "tokens": T, "heads": H, "hidden": D, "rank": r, "act_dtype": p.act_dtype}
    key = "%dx%dx%d_%s" % (T, H, D, p.act_dtype)
    if only in (None, "lowrank"):
        ms = timed(c_call(L.kda_lowrank_gates, x.data_ptr(), wab.data_ptr(), wfb.data_ptr(), D, r, T,
                          f.data_ptr(), beta.data_ptr(), *wsa(kda.KDA_PROJ_LOWRANK_GATES)))
        # algorithmic bytes: x, both weights, f and beta out, the rank-r factor out and back in
        by = T * D * eb + (r + H) * D * 4 + HD * r * 4 + T * HD * 4 + T * H * 4 + 2 * T * r * 4
        fl = 2 * T * D * (r + H) + 2 * T * r * HD
        res["lowrank_gates"] = {
            "ms": ms, "tflops_fp32_equiv": fl / (ms * 1e-3) / 1e12, "bytes_per_call": by,
            "roofline": {"bound": "hbm", "achieved": by / (ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "traffic": committed_traffic("kda_proj.hip", "proj_lowrank_" + key)}}
    for name, fn, K, N in (
            ("gate_projection", c_call(L.kda_gate_projection, x.data_ptr(), wg.data_ptr(), D, T, g.data_ptr(),
                                       *wsa(kda.KDA_PROJ_GATE)), D, HD),
            ("output_projection", c_call(L.kda_output_projection, y.data_ptr(), wo.data_ptr(), D, T,
                                         out.data_ptr(), *wsa(kda.KDA_PROJ_OUTPUT)), HD, D)):
        if only is not None and not name.startswith(only):
            continue
        ms = timed(fn)
        fl = 2 * T * K * N
        by = (T * K + N * K + T * N) * eb
        tf = fl / (ms * 1e-3) / 1e12
        gbs = by / (ms * 1e-3) / 1e9
        # the bound from the arithmetic intensity against the machine balance
        # of the data type's matrix-core peak (fp32 problems run as three
        # bf16 products per product, reported against the fp32 peak)
        peak = MFMA_BF16_PEAK_TFLOPS if bf else MFMA_FP32_PEAK_TFLOPS
        traffic = committed_traffic("kda_proj.hip", "proj_%s_%s" % (name.split("_")[0], key))
        if fl / by < peak * 1e3 / HBM_PEAK_GBS:
            rl = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": gbs / HBM_PEAK_GBS, "traffic": traffic}
        else:
            rl = {"bound": "mfma", "achieved": tf, "peak": peak, "unit": "TFLOP/s", "frac": tf / peak,
                  "traffic": traffic}
            if not bf:
                rl["bf16_mfma_issued_frac"] = 3 * tf / MFMA_BF16_PEAK_TFLOPS
        res[name] = {"ms": ms, "tflops": tf, "hbm_GBps_algorithmic": gbs, "roofline": rl}
    del x, wab, wfb, f, beta, wg, g, y, wo, out, ws
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--prefill", choices=["none", "default", "all"], default="default")
    ap.add_argument("--prefill-runs", type=int, default=5)
    ap.add_argument("--projections", choices=["none", "default", "all"], default="default")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-overcache", action="store_true")
    ap.add_argument("--only", default=None,
                    help="profiling runs: 'decode', 'prefill:<workload index>' or "
                         "'proj:<workload index>[:lowrank|gate|output]' alone, no baselines")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the run, copy a buffer of this many MiB three times (torch copy "
                         "kernel of known size, to scale rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print("bench.py measures one GPU only: the KDA step has no cross-GPU part in this "
                  "library (every (sequence, head) pair is independent); run with --gpus 1",
                  file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from linear_attention_recurrence_token_amd import kda, synth

    if not os.path.exists(kda.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if kda.device_check() != 0:
        raise SystemExit("libkda: the current device is not a gfx950 part")
    smi_before = rocm_smi_snapshot()

    N, H = 64, 32
    steps, warmup = max(1, args.steps), max(0, args.warmup)

    if args.only:
        out = {"only": args.only}
        if args.only == "decode":
            dec = bench_decode(torch, kda, synth, dev, N, H, steps, warmup)
            out["us_per_step"] = dec["ms_total"] / steps * 1e3
        elif args.only.startswith("proj:"):
            parts = args.only.split(":")
            out.update(bench_projections(torch, kda, synth, dev, int(parts[1]), args.prefill_runs,
                                         parts[2] if len(parts) > 2 else None))
        elif args.only.startswith("prefill:"):
            r = bench_prefill(torch, kda, synth, dev, int(args.only.split(":")[1]), args.prefill_runs)
            out.update(r)
        else:
            raise SystemExit("unknown --only %r" % args.only)
        if args.copy_calibration_mib:
            nbytes = args.copy_calibration_mib << 20
            src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).uniform_()
            dst = torch.empty_like(src)
            torch.cuda.synchronize()
            for _ in range(3):
                dst.copy_(src)
            torch.cuda.synchronize()
            out["copy_calibration_bytes_each_way"] = nbytes
        print(json.dumps(out), flush=True)
        return
    log("decode %dx%d: generating %d steps of inputs" % (N, H, steps))
    dec = bench_decode(torch, kda, synth, dev, N, H, steps, warmup)
    ms_step = dec["ms_total"] / steps
    units = N * H
    value = units * steps / (dec["ms_total"] * 1e-3)
    bytes_launch = units * (STATE_BYTES + DECODE_OTHER_BYTES)
    achieved = bytes_launch / (ms_step * 1e-3) / 1e9
    traffic = committed_traffic("kda_decode.hip", "decode_64x32")
    log("decode: %.2f us/step, %.3g token.heads/s, %.0f GB/s algorithmic" % (ms_step * 1e3, value, achieved))

    result = {
        "metric": METRIC, "value": value, "unit": UNIT, "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic (seeded PCG64, K3-shaped KDA heads)",
        "config": {"workload": "decode: 64 sequences x 32 heads, dk=dv=128, fp32 state ~N(0,0.02), "
                               "conv window carried in, one kda_token_step launch per token",
                   "num_seqs": N, "num_heads": H, "head_dim": DK, "act_dtype": "fp32",
                   "gate": "bounded", "tokens_per_step": 1},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "state_only_GBps": units * STATE_BYTES / (ms_step * 1e-3) / 1e9,
                     "bytes_per_launch": bytes_launch},
    }

    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on this host (~%.0f s)" % args.cpu_seconds)
        result["cpu_baseline"] = cpu_baseline_decode(synth, dec["w"], args.cpu_seconds)
        log("cpu baseline: %s" % result["cpu_baseline"])
    del dec

    if not args.no_overcache:
        log("over-cache decode 512x32 (1 GiB of state), 100 steps")
        oc = bench_decode(torch, kda, synth, dev, 512, H, 100, 5)
        oms = oc["ms_total"] / 100
        result["overcache_decode"] = {
            "workload": "decode 512 x 32 heads (1 GiB state, exceeds the 256 MB Infinity Cache); disclosed, not the baseline",
            "us_per_step": oms * 1e3, "value": 512 * H * 100 / (oc["ms_total"] * 1e-3),
            "achieved_GBps": 512 * H * (STATE_BYTES + DECODE_OTHER_BYTES) / (oms * 1e-3) / 1e9}
        log("over-cache: %s" % result["overcache_decode"])
        del oc

    if args.prefill != "none":
        # every prefill workload: 1x32x8192 fp32, 16x64x2048 bf16, the ragged
        # 256x32 bf16 batch and the short 64x32x13 (all = default since the
        # ragged batch generates in seconds on the GPU host's threads)
        idxs = [2, 3, 4, 5]
        result["prefill"] = []
        for idx in idxs:
            log("prefill workload %d" % idx)
            r = bench_prefill(torch, kda, synth, dev, idx, args.prefill_runs)
            log("prefill: %s" % r)
            result["prefill"].append(r)

    if args.projections != "none":
        result["projections"] = []
        for idx in ([1, 3] if args.projections == "default" else [1, 2, 3]):
            log("projections for workload %d" % idx)
            r = bench_projections(torch, kda, synth, dev, idx, args.prefill_runs)
            log("projections: %s" % r)
            result["projections"].append(r)

    result["device"] = {"name": torch.cuda.get_device_name(dev), "rocm_smi_before": smi_before,
                        "rocm_smi_after": rocm_smi_snapshot()}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
