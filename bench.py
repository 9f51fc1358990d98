#!/usr/bin/env python3
"""Throughput of the fused KDA token step on one MI355X.

Headline (one JSON line on stdout): decode over 64 sequences x 32 heads,
dk = dv = 128, fp32 state, one kda_token_step launch per token, K steps back
to back with every step's inputs already resident in HBM.  value = total
token.heads per second; roofline.frac = state bytes (64 KiB read + 64 KiB
written per pair and step) per second over the 8 TB/s HBM peak, frac_total
counting every byte of the launch.

Alongside: the CPU leg (the only part of this file that touches the oracle):
the single-precision oracle timed on this host over the same decode workload
(cpu_baseline), and the fp64 oracle checking a sample of every timed GPU run
(parity: two sequences x all heads of the decode run, every step's y and the
final state and window; sampled pairs of every prefill run).  A run whose
sample misses the tolerance prints value null.  Then a disclosed over-cache
decode run, the prefill workloads (kda_sequence; the chunk paths against the
bf16 matrix-core peak with the flops they issue, the short multi-token one
against HBM), the non-default gate forms, and the projections on either side
of the step (low-rank decay and beta, output gate, output).

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
MFMA_BF16_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 matrix cores, published
MFMA_FP32_PEAK_TFLOPS = 157.3         # MI355X dense fp32 matrix cores, published
# fp32 vector ALU, published: 157.3 TFLOP/s.  Measured on gfx950 with the
# library's flags (packed FP32 off): two wavefronts on one SIMD complete about
# 0.41 non-packed wave64 FMAs per cycle between them (one wavefront alone about
# 0.2), 0.82 of the one per two cycles that 157.3 TFLOP/s at 2.4 GHz needs;
# so the published figure is the ceiling for this code too
FP32_VECTOR_PEAK_TFLOPS = 157.3
DK = DV = 128
STATE_BYTES = DK * DV * 4 * 2         # state read + write per (sequence, head) per decode token
# per decode token.head: q, k, v (3 x 512) + window in/out (2 x 3 x 384 x 4) + f 512 + beta 4 + g 512 + y 512
DECODE_OTHER_BYTES = 3 * 512 + 2 * 3 * 384 * 4 + 512 + 4 + 512 + 512
RECUR_FLOPS = 7 * DK * DV             # u, p dot products (2 FMAs), decay multiply, rank-1 FMA
FP32_TOL, BF16_TOL = 1e-4, 2e-2

# Matrix-core flops the chunkwise kernels issue per 16-token chunk of one
# (sequence, head) pair, every split product counted as its three bf16
# products (16x16x32 step: 16384 flops, 16x16x16 step: 8192):
#   one-pass kernel, 8 wavefronts: P and R 24 x 16x16x32, Delta, O 2 x 3, the
#   state update 8 x 3 and the partial L, M 2 x 3 16x16x16 steps each ->
#   8 x (24 x 16384 + 36 x 8192);
#   two-pass state pass, 16 wavefronts (two row halves of 8 column blocks): P, R
#   12 x 16x16x32, Delta 3 and the update 4 x 3 16x16x16 each, O 3 x 16x16x16
#   on the 8 lower halves (its L and M are formed in the operand pass).
CHUNK_MFMA_FLOPS = {"chunk": 8 * (24 * 16384 + 36 * 8192),
                    "scan": 16 * (12 * 16384 + 15 * 8192) + 8 * 3 * 8192}
CHUNK = 16

# source files each measured path compiles from, besides the ones every path
# shares; a committed traffic summary counts only if it was taken on exactly
# these sources and build flags
CSRC = os.path.join(ROOT, "linear_attention_recurrence_token_amd", "csrc")
COMMON_SOURCES = ["kda_api.hip", "kda_device.hpp", "kda_internal.hpp", "../../include/kda.h"]
PATH_SOURCES = {"decode": ["kda_decode.hip"], "short": ["kda_decode.hip"],
                "chunk": ["kda_prefill_chunk.hip"], "chunk_short": ["kda_prefill_chunk.hip"], "scan": ["kda_prefill_scan.hip", "kda_prefill_split.hip"],
                "split": ["kda_prefill_split.hip"], "fused": ["kda_prefill.hip", "kda_prefill_split.hip"],
                "proj": ["kda_proj.hip"]}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_key(path):
    """sha256 (16 hex digits) over the sources `path`'s kernels compile from
    and the device build flags."""
    from linear_attention_recurrence_token_amd import _build
    h = hashlib.sha256()
    for name in sorted(PATH_SOURCES[path]) + COMMON_SOURCES:
        h.update(os.path.basename(name).encode() + b"\0")
        with open(os.path.normpath(os.path.join(CSRC, name)), "rb") as fh:
            h.update(fh.read())
    h.update((" ".join(["--offload-arch=" + _build.ARCH] + _build.DEVICE_FLAGS)).encode())
    return h.hexdigest()[:16]


def committed_traffic(path, workload_key):
    """HBM bytes per dispatch (or per call) from the committed rocprofv3 PMC
    summary profiles/traffic_<workload_key>.txt, if it was taken on the current
    sources and flags of `path` (else None)."""
    fn = os.path.join(ROOT, "profiles", "traffic_%s.txt" % workload_key)
    if not os.path.exists(fn):
        return None
    vals = {}
    for line in open(fn):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_key_sha256_16") != source_key(path):
        return None
    try:
        return float(vals["hbm_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None


def committed_sq_busy(workload_key, kernel):
    """VALU and MFMA busy fractions of `kernel` from the committed SQ counter
    summary profiles/sq_counters_<workload_key>.txt (its 'busy:' lines)."""
    fn = os.path.join(ROOT, "profiles", "sq_counters_%s.txt" % workload_key)
    if not os.path.exists(fn):
        return None
    for line in open(fn):
        if line.startswith("busy:") and kernel in line:
            parts = dict(kv.split("=") for kv in line.split()[2:] if "=" in kv)
            try:
                return {"valu_busy": float(parts["valu"]), "mfma_busy": float(parts["mfma"]),
                        "source": "profiles/sq_counters_%s.txt" % workload_key}
            except (KeyError, ValueError):
                return None
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


def host_cpu():
    info = {}
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
        for line in out.splitlines():
            if ":" in line:
                k, v = line.split(":", 1)
                info[k.strip()] = v.strip()
    except Exception:
        pass
    return {"model": info.get("Model name"), "threads_per_core": info.get("Thread(s) per core"),
            "cpus_online": info.get("CPU(s)")}


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


def bench_decode(torch, kda, synth, dev, N, H, steps, warmup, check_seqs=()):
    """K = steps timed kda_token_step launches from the initial state, after
    `warmup` untimed ones (the state and window are restored in between).
    Returns the timing and, for check_seqs, every step's y rows and the final
    state and window of those sequences (host arrays) for the parity check."""
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
    if check_seqs:
        ns = torch.as_tensor(list(check_seqs), device=dev)
        y = d["y"].view(steps, N, H, DV).index_select(1, ns).transpose(0, 1).contiguous()
        res["got"] = {"y": y.view(-1, H, DV).double().cpu().numpy(),
                      "state": d["state"].index_select(0, ns).double().cpu().numpy(),
                      "win": d["conv_win"].index_select(0, ns).cpu().numpy()}
        res["check_seqs"] = list(check_seqs)
    del d, state0, win0
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------- the CPU leg
# (the only code here that touches oracle/: the baseline timing and the parity
# checks of the timed GPU runs)

def cpu_baseline_decode(w, target_s):
    """The single-precision oracle, as it stands, on this host: the decode
    workload's steps in order from its initial state, one call per step (every
    sequence's token, state and window updated in place), as many steps as fit
    in about target_s (all of them when they fit)."""
    import numpy as np
    import oracle
    N, H = w.N, w.H
    S = w.state0.copy()
    W = w.win0.copy()
    y = np.empty((N, H, DV), np.float32)
    cu = np.arange(N + 1, dtype=np.int64)

    def step(s):
        sl = slice(s * N, (s + 1) * N)
        oracle.kda_reference_f32_inplace(w.q[sl], w.k[sl], w.v[sl], w.f[sl], w.beta[sl], w.g[sl], w.conv_w,
                                         w.A_log, w.dt_bias, w.gamma, S, W, y, cu)
    # (no OMP_PROC_BIND: binding would pin this process's main thread to one
    # CPU for the rest of the run, the input generation of later workloads
    # included)
    threads = oracle.omp_threads()
    step(0)                                   # loads the library and starts its threads
    S[...] = w.state0
    W[...] = w.win0
    t = time.perf_counter()
    done = 0
    while done < w.decode_steps:
        step(done)
        done += 1
        if time.perf_counter() - t > target_s:
            break
    wall = time.perf_counter() - t
    cpu = host_cpu()
    return {"value": N * H * done / wall, "unit": UNIT, "cores": min(threads, N * H), "kind": "oracle",
            "sample": "decode %d x %d, the first %d of %d steps from the initial state (%s), single-precision "
                      "oracle (kda_oracle_run_f32, one call per step, OpenMP over the %d (sequence, head) "
                      "pairs), %.1f s" % (N, H, done, w.decode_steps,
                                          "all of them" if done == w.decode_steps else "bounded by time",
                                          N * H, wall),
            "host_cpu": cpu["model"], "threads_per_core": cpu["threads_per_core"], "omp_threads": threads}


def parity_errors(got, ref, bf16):
    """max|delta| / max|ref| per output (y at the bf16 bound for bf16 runs,
    the state always at the fp32 bound) and the window bit-exact."""
    import numpy as np
    out = {"pass": True}
    for k in ("y", "state"):
        if k not in got:
            continue
        scale = float(np.max(np.abs(ref[k]))) if ref[k].size else 0.0
        e = float(np.max(np.abs(got[k] - ref[k]))) / max(scale, 1e-30) if ref[k].size else 0.0
        tol = BF16_TOL if (bf16 and k == "y") else FP32_TOL
        out[k + "_rel_err"] = e
        out[k + "_tol"] = tol
        out["pass"] = out["pass"] and e <= tol
    same = bool(np.array_equal(got["win"], ref["win"].astype(np.float32)))
    out["window_bit_exact"] = same
    out["pass"] = out["pass"] and same
    return out


def decode_parity(synth, w, got, seqs):
    import oracle
    sub = synth.decode_subset(w, seqs)
    ref = oracle.kda_reference(sub.q, sub.k, sub.v, sub.f, sub.beta, sub.g, sub.conv_w, sub.A_log,
                               sub.dt_bias, sub.gamma, sub.state0, sub.win0, sub.cu_seqlens, want_o_raw=False)
    r = parity_errors(got, ref, bf16=False)
    r["sample"] = "sequences %s x all %d heads, every one of the %d timed steps' y, final state and window, " \
                  "fp64 oracle" % (seqs, w.H, w.decode_steps)
    return r


def prefill_parity(synth, w, got, seqs, heads):
    import oracle
    sub = synth.subset(w, seqs, heads)
    ref = oracle.kda_reference(sub.q, sub.k, sub.v, sub.f, sub.beta, sub.g, sub.conv_w, sub.A_log,
                               sub.dt_bias, sub.gamma, sub.state0, sub.win0, sub.cu_seqlens,
                               gate_mode=sub.gate_mode, lower_bound=sub.lower_bound, want_o_raw=False)
    r = parity_errors(got, ref, bf16=w.act_dtype == "bf16")
    r["sample"] = "sequences %s x heads %s of the last timed call, fp64 oracle" % (seqs, heads)
    return r


# ---------------------------------------------------------------- prefill

def prefill_samples(w):
    """(sequences, heads) each prefill run is checked on."""
    import numpy as np
    lens = w.lengths
    seqs = sorted({0, w.N - 1, int(np.argmax(lens)), int(np.argmin(lens))})
    heads = sorted({0, w.H - 1})
    return seqs[:4], heads


# The GPU's clock ramps up over the first ~20 ms of sustained load (16 x 64 x
# 2048 bf16 back to back: 2.40, 2.35, 2.24, 2.13, 2.06, 2.01 ms for the first
# calls, then 1.82-1.90 ms from about the tenth).  Prefill and layer calls
# therefore run untimed until WARM_MS of GPU time have passed (at least one
# call), and only then are `runs` calls timed: the steady state a serving loop
# runs in, as the 1000-step decode timing is.
WARM_MS = 60.0


def warm_up(one_call):
    """Call one_call() (which returns its GPU milliseconds) until WARM_MS have
    passed; returns the number of calls."""
    total, calls = 0.0, 0
    while calls == 0 or total < WARM_MS:
        total += one_call()
        calls += 1
    return calls


def bench_prefill(torch, kda, synth, dev, w, runs, traffic_key=None, want_check=True):
    import numpy as np
    d = synth.to_device(w, dev, with_o_raw=False)
    state0, win0 = d["state"].clone(), d["conv_win"].clone()
    cfg = kda.KdaConfig(num_heads=w.H, act_dtype=kda.KDA_BF16 if w.act_dtype == "bf16" else kda.KDA_F32,
                        gate_mode=w.gate_mode, gate_lower_bound=w.lower_bound)
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

    import numpy as np
    cu_host = np.ascontiguousarray(w.cu_seqlens, dtype=np.int32)
    side = torch.cuda.Stream(device=dev)

    def launch():
        st = L.kda_sequence(ctypes.byref(ccfg), ctypes.byref(t), w.N, cu, cu_host.ctypes.data, order.data_ptr(),
                            w.total_tokens, ws_ptr, ws_bytes, stream.cuda_stream, side.cuda_stream)
        if st != 0:
            raise RuntimeError("kda_sequence returned %d" % st)
    def one_call():
        d["state"].copy_(state0)
        d["conv_win"].copy_(win0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        launch()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)
    warm_calls = warm_up(one_call)
    times = [one_call() for _ in range(runs)]
    ms = float(np.median(times))
    th = int(lens.sum()) * w.H
    # the kernel the automatic choice runs (the library's rule: for the
    # bounded gate with |lower bound| <= 7.5, the short-sequence kernel under 4
    # tokens per sequence on average, the two-pass chunk path for at most 64
    # pairs averaging 128 tokens or more (given its workspace), the chunk
    # kernel without a pipeline up to 16 tokens on average (64 from 512
    # pairs on) and the one-pass chunk kernel otherwise; for the other gates
    # the short-sequence kernel under 8 tokens, else split / fused)
    chunk_gate = cfg.gate_mode == kda.KDA_GATE_BOUNDED and -7.5 <= cfg.gate_lower_bound <= 0.0
    short = w.total_tokens < (4 if chunk_gate else 8) * w.N
    chunk = chunk_gate and not short
    scan = chunk and w.N * w.H <= 64 and w.total_tokens >= 128 * w.N and ws_bytes > 0
    chunk_short = chunk and not scan and w.total_tokens <= (64 if w.N * w.H >= 512 else 16) * w.N
    path = ("short" if short else ("scan" if scan else ("chunk_short" if chunk_short else (
        "chunk" if chunk else ("split" if ws_bytes > 0 else "fused")))))
    traffic = committed_traffic(path, traffic_key) if traffic_key else None
    # algorithmic HBM bytes: state in+out and window in+out per pair, and per
    # token.head q, k, v, g, y (activation dtype) with f (fp32) and beta
    act_bytes = 2 if w.act_dtype == "bf16" else 4
    per_token = 5 * 128 * act_bytes + 512 + 4
    hbm_bytes = w.N * w.H * (2 * DK * DV * 4 + 2 * 3 * 384 * 4) + th * per_token
    recur_tf = th * RECUR_FLOPS / (ms * 1e-3) / 1e12
    out = {"workload": w.name, "path": path, "token_heads": th, "ms": ms, "runs": runs,
           "warmup_calls": warm_calls, "ms_each": [round(x, 4) for x in times],
           "value": th / (ms * 1e-3), "unit": UNIT,
           "ns_per_token_per_chain": ms * 1e6 / int(lens.max()),
           "hbm_GBps_algorithmic": hbm_bytes / (ms * 1e-3) / 1e9,
           "recurrent_form": {"flops_per_token_head": RECUR_FLOPS, "achieved_TFLOPs": recur_tf,
                              "frac_of_fp32_vector_peak": recur_tf / FP32_VECTOR_PEAK_TFLOPS}}
    if path in ("chunk", "scan") and not short and int(lens.max()) >= 2 * CHUNK:
        chunks = int(sum((int(n) + CHUNK - 1) // CHUNK for n in lens)) * w.H
        fl = chunks * CHUNK_MFMA_FLOPS[path]
        tf = fl / (ms * 1e-3) / 1e12
        out["roofline"] = {"bound": "mfma", "achieved": tf, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": tf / MFMA_BF16_PEAK_TFLOPS, "traffic": traffic,
                           "flops": "bf16 matrix-core flops issued: %d chunks of 16 tokens x %d per chunk "
                                    "(every split product as three bf16 products)" % (chunks, CHUNK_MFMA_FLOPS[path])}
    elif path in ("fused", "split") and int(lens.max()) >= 2 * CHUNK:
        # the recurrent kernels: 7 dk dv flops per token.head on the vector ALU
        out["roofline"] = {"bound": "alu", "achieved": recur_tf, "peak": FP32_VECTOR_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": recur_tf / FP32_VECTOR_PEAK_TFLOPS, "traffic": traffic,
                           "flops": "7 dk dv per token.head (recurrent form) against the fp32 vector peak"}
    else:
        # a few tokens per (sequence, head): the state round trip dominates
        out["roofline"] = {"bound": "hbm", "achieved": hbm_bytes / (ms * 1e-3) / 1e9,
                           "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": hbm_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "traffic": traffic}
    if traffic_key:
        busy = committed_sq_busy(traffic_key, {"chunk": "prefill_chunk_kernel", "scan": "scan_kernel",
                                               "chunk_short": "prefill_chunk_short_kernel"}.get(path, path))
        if busy:
            out["roofline"]["sq_busy"] = busy
    if want_check:
        seqs, heads = prefill_samples(w)
        ns, hs = torch.as_tensor(seqs, device=dev), torch.as_tensor(heads, device=dev)
        rows = torch.as_tensor(np.concatenate([np.arange(w.cu_seqlens[n], w.cu_seqlens[n + 1]) for n in seqs]),
                               device=dev, dtype=torch.int64)
        out["_check"] = (seqs, heads, {
            "y": d["y"].index_select(0, rows).index_select(1, hs).double().cpu().numpy(),
            "state": d["state"].index_select(0, ns).index_select(1, hs).double().cpu().numpy(),
            "win": d["conv_win"].index_select(0, ns).index_select(1, hs).cpu().numpy()})
    del d, state0, win0
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------- projections

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
                         "traffic": committed_traffic("proj", "proj_lowrank_" + key)}}
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
        traffic = committed_traffic("proj", "proj_%s_%s" % (name.split("_")[0], key))
        # the bound from the arithmetic intensity against the machine balance
        # of the unit the product runs on: bf16 matrix cores for bf16; for
        # fp32, three bf16 products per product, i.e. a third of the bf16 peak
        # in fp32-equivalent flops
        eff_peak = MFMA_BF16_PEAK_TFLOPS if bf else MFMA_BF16_PEAK_TFLOPS / 3
        if fl / by < eff_peak * 1e3 / HBM_PEAK_GBS:
            rl = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": gbs / HBM_PEAK_GBS, "traffic": traffic}
        elif bf:
            rl = {"bound": "mfma", "achieved": tf, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                  "frac": tf / MFMA_BF16_PEAK_TFLOPS, "traffic": traffic}
        else:
            rl = {"bound": "mfma", "achieved": 3 * tf, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                  "frac": 3 * tf / MFMA_BF16_PEAK_TFLOPS, "traffic": traffic,
                  "flops": "bf16 matrix-core flops issued (three bf16 products per fp32 product)",
                  "fp32_equiv_vs_fp32_mfma_peak": tf / MFMA_FP32_PEAK_TFLOPS}
        res[name] = {"ms": ms, "tflops": tf, "hbm_GBps_algorithmic": gbs, "roofline": rl}
    del x, wab, wfb, f, beta, wg, g, y, wo, out, ws
    torch.cuda.empty_cache()
    return res


def bench_layer(torch, kda, synth, dev, runs):
    """The KDA layer around the step at 16 x 64 x 2048 (bf16, hidden 8192,
    rank 128), timed end to end: the low-rank decay and beta products, the
    output-gate product W_g x, the step, and the output product W_o y.  Two
    forms: f through memory (kda_lowrank_gates, then kda_sequence) and f formed
    in the step (kda_lowrank_factor, then kda_sequence_lowrank)."""
    import numpy as np
    w = synth.workload(3)
    p = synth.projection_workload(3)
    d = synth.to_device(w, dev, with_o_raw=False)
    state0, win0 = d["state"].clone(), d["conv_win"].clone()
    T, H, D, r = p.T, p.H, p.D, p.r
    cfg = kda.KdaConfig(num_heads=H, act_dtype=kda.KDA_BF16)
    x = torch.from_numpy(p.x).to(dev).to(torch.bfloat16)
    wab = torch.from_numpy(np.concatenate([p.w_fa, p.w_bp])).to(dev)
    wfb = torch.from_numpy(p.w_fb).to(dev)
    wg = torch.from_numpy(p.w_g).to(dev).to(torch.bfloat16)
    wo = torch.from_numpy(p.w_o).to(dev).to(torch.bfloat16)
    out = torch.empty(T, D, device=dev, dtype=torch.bfloat16)
    a = torch.empty(T, r, device=dev)
    g = d["g"].view(T, H * 128)
    stream = torch.cuda.current_stream()
    L = kda.lib()
    ccfg = cfg.to_c()
    sh = stream.cuda_stream

    def ws(which, rank=0):
        n = kda.projection_workspace_size(cfg, which, D, T, rank)
        return (torch.empty(n, dtype=torch.uint8, device=dev), n) if n > 0 else (None, 0)
    ws_lr, n_lr = ws(kda.KDA_PROJ_LOWRANK_GATES, r)
    ws_fa, n_fa = ws(kda.KDA_PROJ_LOWRANK_FACTOR, r)
    ws_g, n_g = ws(kda.KDA_PROJ_GATE)
    ws_o, n_o = ws(kda.KDA_PROJ_OUTPUT)
    n_sq = kda.sequence_workspace_size(cfg, w.N, T)
    ws_sq = torch.empty(n_sq, dtype=torch.uint8, device=dev) if n_sq > 0 else None
    ptr = lambda t: t.data_ptr() if t is not None else None
    t_sep = kda.kda_tensors(*[(d[n].data_ptr() if d.get(n) is not None else None) for n in kda.TENSOR_FIELDS])
    t_lr = kda.kda_tensors(*[(d[n].data_ptr() if (d.get(n) is not None and n != "f") else None)
                             for n in kda.TENSOR_FIELDS])
    cu = d["cu_seqlens"].data_ptr()

    def chk(st, what):
        if st != 0:
            raise RuntimeError("%s returned %d" % (what, st))
    parts = {
        "lowrank_gates": lambda: chk(L.kda_lowrank_gates(ctypes.byref(ccfg), x.data_ptr(), wab.data_ptr(),
                                                         wfb.data_ptr(), D, r, T, d["f"].data_ptr(),
                                                         d["beta"].data_ptr(), ptr(ws_lr), n_lr, sh), "lowrank"),
        "lowrank_factor": lambda: chk(L.kda_lowrank_factor(ctypes.byref(ccfg), x.data_ptr(), wab.data_ptr(), D, r,
                                                           T, a.data_ptr(), d["beta"].data_ptr(), ptr(ws_fa), n_fa,
                                                           sh), "factor"),
        "gate_projection": lambda: chk(L.kda_gate_projection(ctypes.byref(ccfg), x.data_ptr(), wg.data_ptr(), D, T,
                                                             g.data_ptr(), ptr(ws_g), n_g, sh), "gate"),
        "step": lambda: chk(L.kda_sequence(ctypes.byref(ccfg), ctypes.byref(t_sep), w.N, cu, None, None, T,
                                           ptr(ws_sq), n_sq, sh, None), "sequence"),
        "step_lowrank": lambda: chk(L.kda_sequence_lowrank(ctypes.byref(ccfg), ctypes.byref(t_lr), w.N, cu, None,
                                                           None, T, a.data_ptr(), wfb.data_ptr(), r, sh),
                                    "sequence_lowrank"),
        "output_projection": lambda: chk(L.kda_output_projection(ctypes.byref(ccfg), d["y"].data_ptr(), wo.data_ptr(),
                                                                 D, T, out.data_ptr(), ptr(ws_o), n_o, sh), "out"),
    }
    forms = {"f_through_memory": ["lowrank_gates", "gate_projection", "step", "output_projection"],
             "f_in_step": ["lowrank_factor", "gate_projection", "step_lowrank", "output_projection"]}

    def timed(names):
        def one_call():
            d["state"].copy_(state0)
            d["conv_win"].copy_(win0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for n in names:
                parts[n]()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1)
        warm_up(one_call)
        return float(np.median([one_call() for _ in range(runs)]))
    res = {"workload": "KDA layer 16 x 64 x 2048 bf16, hidden 8192, rank 128 (synthetic weights)",
           "token_heads": T * H, "parts_ms": {n: timed([n]) for n in parts}}
    for form, names in forms.items():
        ms = timed(names)
        res[form] = {"ms": ms, "parts": names, "value": T * H / (ms * 1e-3), "unit": UNIT}
    res["f_round_trip_bytes_removed"] = 2 * T * H * 128 * 4
    del d, state0, win0, x, wab, wfb, wg, wo, out, a
    torch.cuda.empty_cache()
    return res


def main():
    global WARM_MS
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--prefill", choices=["none", "default", "all"], default="default")
    ap.add_argument("--prefill-runs", type=int, default=5)
    ap.add_argument("--warm-ms", type=float, default=WARM_MS,
                    help="untimed GPU milliseconds before each prefill / layer timing (0: one call)")
    ap.add_argument("--projections", choices=["none", "default", "all"], default="default")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU leg: no oracle baseline and no parity check of the timed runs")
    ap.add_argument("--cpu-seconds", type=float, default=25.0)
    ap.add_argument("--no-overcache", action="store_true")
    ap.add_argument("--only", default=None,
                    help="profiling runs: 'decode', 'prefill:<workload index>' or "
                         "'proj:<workload index>[:lowrank|gate|output]' alone, no baselines")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the run, copy a buffer of this many MiB three times (torch copy "
                         "kernel of known size, to scale rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--source-key", default=None, metavar="PATH",
                    help="print the source key of a path's kernels (decode, chunk, scan, short, split, "
                         "fused, proj), as the traffic summaries record it, and exit")
    args = ap.parse_args()
    WARM_MS = max(0.0, args.warm_ms)

    if args.source_key:
        print(source_key(args.source_key))
        return
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

    N, H = 64, 32
    steps, warmup = max(1, args.steps), max(0, args.warmup)
    prefill_keys = {2: "prefill_1x32x8192", 3: "prefill_16x64x2048", 4: "prefill_ragged_256x32",
                    5: "prefill_short_64x32x13"}

    if args.only:
        out = {"only": args.only}
        if args.only == "decode":
            dec = bench_decode(torch, kda, synth, dev, N, H, steps, warmup)
            out["us_per_step"] = dec["ms_total"] / steps * 1e3
        elif args.only.startswith("proj:"):
            parts = args.only.split(":")
            out.update(bench_projections(torch, kda, synth, dev, int(parts[1]), args.prefill_runs,
                                         parts[2] if len(parts) > 2 else None))
        elif args.only == "layer":
            out.update(bench_layer(torch, kda, synth, dev, args.prefill_runs))
        elif args.only.startswith("prefill:"):
            idx = int(args.only.split(":")[1])
            r = bench_prefill(torch, kda, synth, dev, synth.workload(idx), args.prefill_runs,
                              prefill_keys.get(idx), want_check=False)
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
    # (not in the profiling runs above: under a counter-collecting profiler
    # the rocm-smi child would start with the profiler's library preloaded)
    smi_before = rocm_smi_snapshot()
    log("decode %dx%d: generating %d steps of inputs" % (N, H, steps))
    check = not args.no_cpu_baseline
    dec = bench_decode(torch, kda, synth, dev, N, H, steps, warmup, check_seqs=(0, N - 1) if check else ())
    ms_step = dec["ms_total"] / steps
    units = N * H
    value = units * steps / (dec["ms_total"] * 1e-3)
    bytes_launch = units * (STATE_BYTES + DECODE_OTHER_BYTES)
    state_gbs = units * STATE_BYTES / (ms_step * 1e-3) / 1e9
    total_gbs = bytes_launch / (ms_step * 1e-3) / 1e9
    traffic = committed_traffic("decode", "decode_64x32")
    log("decode: %.2f us/step, %.3g token.heads/s, state %.0f GB/s, all bytes %.0f GB/s"
        % (ms_step * 1e3, value, state_gbs, total_gbs))

    result = {
        "metric": METRIC, "value": value, "unit": UNIT, "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic (seeded PCG64, K3-shaped KDA heads)",
        "config": {"workload": "decode: 64 sequences x 32 heads, dk=dv=128, fp32 state ~N(0,0.02), "
                               "conv window carried in, one kda_token_step launch per token",
                   "num_seqs": N, "num_heads": H, "head_dim": DK, "act_dtype": "fp32",
                   "gate": "bounded", "tokens_per_step": 1},
        "roofline": {"bound": "hbm", "achieved": state_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": state_gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "bytes": "state only: %d pairs x %d B (64 KiB read + 64 KiB written) per launch"
                              % (units, STATE_BYTES),
                     "achieved_total_GBps": total_gbs, "frac_total": total_gbs / HBM_PEAK_GBS,
                     "bytes_per_launch_total": bytes_launch},
    }

    if check:
        log("cpu leg: single-precision oracle on this host (up to ~%.0f s)" % args.cpu_seconds)
        result["cpu_baseline"] = cpu_baseline_decode(dec["w"], args.cpu_seconds)
        log("cpu baseline: %s" % result["cpu_baseline"])
        log("cpu leg: parity of the timed decode run (fp64 oracle)")
        result["parity"] = decode_parity(synth, dec["w"], dec["got"], dec["check_seqs"])
        log("parity: %s" % result["parity"])
    else:
        result["parity"] = {"pass": None, "sample": "not checked (--no-cpu-baseline)"}
    del dec

    if not args.no_overcache:
        log("over-cache decode 512x32 (1 GiB of state), 100 steps")
        oc = bench_decode(torch, kda, synth, dev, 512, H, 100, 5)
        oms = oc["ms_total"] / 100
        result["overcache_decode"] = {
            "workload": "decode 512 x 32 heads (1 GiB state, exceeds the 256 MB Infinity Cache); disclosed, not the baseline",
            "us_per_step": oms * 1e3, "value": 512 * H * 100 / (oc["ms_total"] * 1e-3),
            "state_GBps": 512 * H * STATE_BYTES / (oms * 1e-3) / 1e9,
            "achieved_GBps": 512 * H * (STATE_BYTES + DECODE_OTHER_BYTES) / (oms * 1e-3) / 1e9}
        log("over-cache: %s" % result["overcache_decode"])
        del oc

    prefill_fail = False
    if args.prefill != "none":
        # every prefill workload: 1x32x8192 fp32, 16x64x2048 bf16, the ragged
        # 256x32 bf16 batch and the short 64x32x13; then the 16x64x2048 shape
        # with the two other gate forms (they run the recurrent kernels)
        runs = [(idx, synth.workload(idx), prefill_keys[idx]) for idx in (2, 3, 4, 5)]
        result["prefill"] = []
        for idx, w, key in runs:
            log("prefill workload %d" % idx)
            r = bench_prefill(torch, kda, synth, dev, w, args.prefill_runs, key, want_check=check)
            if "_check" in r:
                seqs, heads, got = r.pop("_check")
                r["parity"] = prefill_parity(synth, w, got, seqs, heads)
                if not r["parity"]["pass"]:
                    prefill_fail = True
                    r["value"] = None
            log("prefill: %s" % r)
            result["prefill"].append(r)
            del w
        result["prefill_gate_forms"] = []
        for mode, name in ((kda.KDA_GATE_LITERAL, "literal"), (kda.KDA_GATE_RAW, "raw")):
            w = synth.make_workload("batched prefill 16x64 T=2048 bf16, %s gate" % name, seed=3, N=16, H=64,
                                    lengths=[2048] * 16, act_dtype="bf16", state_std=0.02, win_std=1.0,
                                    decay=(0.8, 0.999), gate_mode=mode)
            log("prefill 16x64x2048, %s gate" % name)
            r = bench_prefill(torch, kda, synth, dev, w, max(1, args.prefill_runs // 2), None, want_check=check)
            if "_check" in r:
                seqs, heads, got = r.pop("_check")
                r["parity"] = prefill_parity(synth, w, got, seqs, heads)
                if not r["parity"]["pass"]:
                    prefill_fail = True
                    r["value"] = None
            log("prefill: %s" % r)
            result["prefill_gate_forms"].append(r)
            del w

    if args.projections != "none":
        log("layer 16x64x2048: projections and step end to end")
        result["layer"] = bench_layer(torch, kda, synth, dev, args.prefill_runs)
        log("layer: %s" % result["layer"])
        result["projections"] = []
        for idx in ([1, 3] if args.projections == "default" else [1, 2, 3]):
            log("projections for workload %d" % idx)
            r = bench_projections(torch, kda, synth, dev, idx, args.prefill_runs)
            log("projections: %s" % r)
            result["projections"].append(r)

    result["device"] = {"name": torch.cuda.get_device_name(dev), "rocm_smi_before": smi_before,
                        "rocm_smi_after": rocm_smi_snapshot()}
    failed = result["parity"]["pass"] is False or prefill_fail
    if failed:
        # a timed run that misses the oracle's tolerance reports no throughput
        result["value"] = None
    print(json.dumps(result), flush=True)
    if failed:
        sys.exit(1)


if __name__ == "__main__":
    main()
