"""GPU parity: the HIP path against the CPU oracle on the same seeded inputs.

Bar: max|delta| <= 1e-4 * max|ref| for y, o_raw and the state with fp32
inputs; y within 2e-2 * max|ref| when inputs and y are bf16 (o_raw and the
state stay at 1e-4 since both sides read the same bf16-exact inputs); the
conv window bit-exact.  Sizes span several chunks and a ragged tail; the
full-size cases run the bench's launch configuration and compare sampled
(sequence, head) pairs that the oracle computes one by one.
"""
import dataclasses
import sys

import numpy as np
import pytest

from linear_attention_recurrence_token_amd import kda, synth
from tests import _gpu

pytestmark = pytest.mark.gpu


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# ---------------------------------------------------------------- small sizes

PATHS = pytest.mark.parametrize("path", ["fused", "split", "chunk", "short", "scan", "chunk_short"])
PATHS_ANY_GATE = pytest.mark.parametrize("path", ["fused", "split", "short"])


@PATHS
def test_cfg0_sequence(gpu, path):
    w = synth.workload(0)
    note("cfg0 1x1x64 fp32 via kda_sequence, %s" % path)
    _gpu.assert_parity(_gpu.run_sequence(w, gpu, path=path), _gpu.oracle_sequence(w), label="cfg0")


def test_cfg0_as_token_steps(gpu):
    w0 = synth.workload(0)
    w = dataclasses.replace(w0, decode_steps=64)     # one sequence: step-major == sequence order
    note("cfg0 as 64 chained kda_token_step calls")
    got = _gpu.run_decode(w, gpu)
    _gpu.assert_parity(got, _gpu.oracle_sequence(w0), label="cfg0 decode")


@pytest.mark.parametrize("N,H,steps", [(8, 4, 24), (3, 5, 7), (1, 32, 3)])
def test_decode_small(gpu, N, H, steps):
    w = synth.workload(1, scale={"N": N, "H": H, "steps": steps}, seed=100 + N)
    note("decode N=%d H=%d steps=%d" % (N, H, steps))
    _gpu.assert_parity(_gpu.run_decode(w, gpu), _gpu.oracle_decode(w), label="decode")


@pytest.mark.parametrize("N,H,steps,act", [
    (17, 32, 3, "f32"),     # 544 pairs on 256 workgroups: two or three pairs each
    (20, 48, 2, "f32"),     # H does not divide 256: 240 workgroups of four pairs
    (2, 300, 2, "bf16"),    # H above the compute units: 300 workgroups of two pairs
    (40, 16, 3, "bf16"),    # 640 pairs: two or three each
])
def test_decode_persistent_grid_shapes(gpu, N, H, steps, act):
    # batches of more than two pairs per compute unit run the persistent
    # decode kernel, each workgroup walking several pairs of one head
    w = synth.make_workload("decode grid", seed=700 + N + H, N=N, H=H, decode_steps=steps, act_dtype=act,
                            state_std=0.02, win_std=1.0)
    note("decode persistent grid N=%d H=%d steps=%d %s" % (N, H, steps, act))
    _gpu.assert_parity(_gpu.run_decode(w, gpu), _gpu.oracle_decode(w), bf16=act == "bf16",
                       label="decode grid %dx%d" % (N, H))


def test_decode_bf16(gpu):
    w = synth.make_workload("decode bf16", seed=7, N=6, H=3, decode_steps=9, act_dtype="bf16",
                            state_std=0.02, win_std=1.0)
    note("decode bf16 6x3x9")
    _gpu.assert_parity(_gpu.run_decode(w, gpu), _gpu.oracle_decode(w), bf16=True, label="decode bf16")


@PATHS
@pytest.mark.parametrize("T", [1, 2, 3, 7, 8, 9, 15, 16, 17, 300])
def test_prefill_fp32_lengths(gpu, T, path):
    w = synth.workload(2, scale={"H": 3, "T": T}, seed=200 + T)
    w.state0[...] = synth.make_workload("s", seed=1, N=1, H=3, lengths=[1], state_std=0.02).state0
    w.win0[...] = synth.make_workload("w", seed=2, N=1, H=3, lengths=[1], win_std=1.0).win0
    note("prefill fp32 1x3 T=%d %s" % (T, path))
    _gpu.assert_parity(_gpu.run_sequence(w, gpu, path=path), _gpu.oracle_sequence(w), label="T=%d" % T)


@PATHS
def test_prefill_cfg3_small_bf16(gpu, path):
    w = synth.workload(3, scale={"N": 2, "H": 4, "T": 300})
    note("cfg3-shaped bf16 2x4x300 %s" % path)
    _gpu.assert_parity(_gpu.run_sequence(w, gpu, path=path), _gpu.oracle_sequence(w), bf16=True,
                       label="cfg3s")


@PATHS
def test_prefill_dense_mode_matches_packed(gpu, path):
    w = synth.workload(3, scale={"N": 3, "H": 2, "T": 40})
    note("dense (cu_seqlens=NULL) vs packed %s" % path)
    a = _gpu.run_sequence(w, gpu, dense=True, path=path)
    b = _gpu.run_sequence(w, gpu, path=path)
    for k in ("y", "o_raw", "state", "win"):
        np.testing.assert_array_equal(a[k], b[k])


@PATHS
@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_ragged_edges(gpu, act, path):
    lengths = [0, 1, 2, 3, 4, 5, 17, 64, 0, 300, 1000]
    w = synth.make_workload("ragged edges", seed=41, N=len(lengths), H=4, lengths=lengths,
                            act_dtype=act, state_std=0.02, win_std=1.0, gamma_range=(0.5, 1.5),
                            fresh_prob=0.5)
    note("ragged %s lengths=%s H=4 %s" % (act, lengths, path))
    _gpu.assert_parity(_gpu.run_sequence(w, gpu, path=path), _gpu.oracle_sequence(w),
                       bf16=(act == "bf16"), label="ragged")


@pytest.mark.parametrize("path", ["auto", "fused", "split", "chunk", "short", "scan", "chunk_short"])
@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_many_short_sequences(gpu, act, path):
    # lengths 1..16 over many sequences: below, at and around one chunk, and
    # on both sides of the automatic choice's length threshold
    w = synth.make_workload("short ragged", seed=31, N=40, H=3,
                            lengths=lambda rng: rng.integers(1, 17, size=40), act_dtype=act,
                            state_std=0.02, win_std=1.0, fresh_prob=0.3)
    note("many short sequences 40x3 U[1,16] %s %s" % (act, path))
    _gpu.assert_parity(_gpu.run_sequence(w, gpu, path=path), _gpu.oracle_sequence(w),
                       bf16=act == "bf16", label="short %s" % path)


@pytest.mark.parametrize("path", ["chunk", "chunk_short"])
@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_chunk_many_pairs_short_average(gpu, act, path):
    # more (sequence, head) pairs than CUs and few tokens on average: the
    # chunk path's workgroups loop over several pairs each; lengths 0..40
    # (empty ones included) give one to three chunks per pair
    w = synth.make_workload("many pairs", seed=35, N=150, H=2,
                            lengths=lambda rng: rng.integers(0, 41, size=150), act_dtype=act,
                            state_std=0.02, win_std=1.0, fresh_prob=0.3)
    note("%s path, 150 x 2 pairs, lengths U[0,40], %s" % (path, act))
    order = np.argsort(-w.lengths, kind="stable")
    for seq_order in (None, order):
        _gpu.assert_parity(_gpu.run_sequence(w, gpu, path=path, seq_order=seq_order),
                           _gpu.oracle_sequence(w), bf16=act == "bf16", label="many pairs")


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_chunk_pair_counter(gpu, act):
    # the one-pass chunk kernel with its pair counter (the workspace the
    # library asks for: one workgroup per compute unit, each taking pairs
    # until none are left) against one pair per workgroup (no workspace):
    # 400 pairs, so most workgroups take two, with empty sequences among them
    # and, in the last order, two entries out of range (skipped, leaving
    # those sequences' state as it was); every pair's
    # arithmetic is the same either way, so the results agree bit for bit
    N, H = 100, 4
    w = synth.make_workload("pair counter", seed=37, N=N, H=H,
                            lengths=lambda rng: rng.choice([0, 1, 15, 16, 17, 40, 97], size=N), act_dtype=act,
                            state_std=0.02, win_std=1.0, fresh_prob=0.3)
    assert kda.sequence_workspace_size(_gpu.cfg_of(w, prefill_path=kda.KDA_PREFILL_CHUNK), N, w.total_tokens) == 256
    order = np.argsort(-w.lengths, kind="stable").astype(np.int32)
    bad = order.copy()
    bad[3], bad[50] = -1, N + 7
    ref = _gpu.oracle_sequence(w)
    for label, seq_order in (("natural order", None), ("longest first", order), ("two entries out of range", bad)):
        note("chunk path with and without its pair counter, 100 x 4 pairs, %s, %s" % (label, act))
        a = _gpu.run_sequence(w, gpu, path="chunk", seq_order=seq_order)
        b = _gpu.run_sequence(w, gpu, path="chunk", seq_order=seq_order, workspace=None)
        for k in ("y", "o_raw", "state", "win"):
            np.testing.assert_array_equal(a[k], b[k], err_msg="%s %s" % (label, k))
        if seq_order is bad:
            skipped = [int(order[3]), int(order[50])]
            kept = [n for n in range(N) if n not in skipped]
            np.testing.assert_array_equal(a["state"][skipped], w.state0[skipped].astype(np.float32))
            sub = synth.subset(w, kept, list(range(H)))
            got = {"state": a["state"][kept], "win": a["win"][kept]}
            _gpu.assert_parity(got, _gpu.oracle_sequence(sub), keys=("state",), label=label)
        else:
            _gpu.assert_parity(a, ref, bf16=act == "bf16", label=label)


def test_chunk_pair_counter_in_a_graph(gpu):
    # the call captured in a HIP graph: its counter is zeroed by a kernel in
    # the graph, so every replay (with eager work and synchronisations
    # between them) must give the eager call's results bit for bit
    import torch
    N, H = 70, 4
    w = synth.make_workload("graph", seed=39, N=N, H=H,
                            lengths=lambda rng: rng.choice([0, 5, 16, 33, 80], size=N), act_dtype="bf16",
                            state_std=0.02, win_std=1.0, fresh_prob=0.3)
    d = synth.to_device(w, gpu, with_o_raw=True)
    s0, w0 = d["state"].clone(), d["conv_win"].clone()
    cfg = _gpu.cfg_of(w, prefill_path=kda.KDA_PREFILL_CHUNK)
    ws = torch.empty(kda.sequence_workspace_size(cfg, N, w.total_tokens), dtype=torch.uint8, device=gpu)
    assert ws.numel() == 256
    order = torch.as_tensor(np.argsort(-w.lengths, kind="stable").astype(np.int32), device=gpu)

    def call():
        kda.kda_sequence(cfg, **_gpu.tensors(d), cu_seqlens=d["cu_seqlens"], seq_order=order, num_seqs=N,
                         workspace=ws, check=False)

    def reset():
        d["state"].copy_(s0)
        d["conv_win"].copy_(w0)
        d["y"].zero_()
        d["o_raw"].zero_()

    def snap():
        return {k: d[k].float().cpu().numpy().copy() for k in ("y", "o_raw", "state", "conv_win")}

    note("chunk path with its pair counter, eager then captured, 70 x 4 pairs")
    call()
    torch.cuda.synchronize()
    ref = snap()
    _gpu.assert_parity({"y": ref["y"].astype(np.float64), "o_raw": ref["o_raw"].astype(np.float64),
                        "state": ref["state"].astype(np.float64), "win": ref["conv_win"]},
                       _gpu.oracle_sequence(w), bf16=True, label="eager")
    reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(4):
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snap()
        for k in ref:
            np.testing.assert_array_equal(got[k], ref[k], err_msg="replay %d %s" % (rep, k))


@pytest.mark.parametrize("path", ["auto", "chunk", "short", "chunk_short"])
def test_short_average_with_long_sequences(gpu, path):
    # a batch that is short on average (the chunk path's single-buffered
    # variant) but holds a few sequences of several chunks
    lens = [2] * 30 + [100, 37]
    w = synth.make_workload("mostly short", seed=33, N=len(lens), H=2, lengths=lens,
                            state_std=0.02, win_std=1.0, fresh_prob=0.3)
    note("mostly-short batch with two long sequences, %s" % path)
    _gpu.assert_parity(_gpu.run_sequence(w, gpu, path=path), _gpu.oracle_sequence(w), label="mixed")


@PATHS_ANY_GATE
@pytest.mark.parametrize("mode", [synth.GATE_LITERAL, synth.GATE_RAW])
def test_other_gate_modes(gpu, mode, path):
    w = synth.make_workload("gate", seed=50 + mode, N=2, H=3, lengths=[33, 10], gate_mode=mode,
                            state_std=0.02, win_std=1.0)
    note("gate mode %d prefill + decode %s" % (mode, path))
    _gpu.assert_parity(_gpu.run_sequence(w, gpu, path=path), _gpu.oracle_sequence(w), label="gate %d" % mode)
    wd = synth.make_workload("gate d", seed=60 + mode, N=4, H=2, decode_steps=5, gate_mode=mode,
                             state_std=0.02, win_std=1.0)
    _gpu.assert_parity(_gpu.run_decode(wd, gpu), _gpu.oracle_decode(wd), label="gate %d dec" % mode)


@PATHS
@pytest.mark.parametrize("lb", [-1.0, -9.0])
def test_bounded_gate_other_bounds(gpu, lb, path):
    # -9 * 8 tokens < -60: outside the range of the folded prefill form, so this
    # also runs the direct form with the bounded gate
    lo = 0.4 if lb > -2 else 0.2      # decays the bound can reach: exp(lb) < d < 1
    w = synth.make_workload("lb", seed=70, N=2, H=2, lengths=[29, 12], lower_bound=lb,
                            decay=(lo, 0.999), state_std=0.02, win_std=1.0)
    assert np.all(np.isfinite(w.f))
    if path in ("chunk", "scan", "chunk_short") and lb < -7.5:
        # the chunkwise forms need |lb| <= 7.5 and say so
        with pytest.raises(kda.KdaError) as ei:
            _gpu.run_sequence(w, gpu, path=path)
        assert ei.value.status == kda.KDA_ERR_UNSUPPORTED
        return
    note("bounded gate lb=%g %s" % (lb, path))
    _gpu.assert_parity(_gpu.run_sequence(w, gpu, path=path), _gpu.oracle_sequence(w), label="lb %g" % lb)


@PATHS
def test_strong_decay_chunks(gpu, path):
    # decays down to exp(-5) every token: the folded form's per-chunk scaling
    # reaches exp(-40); results must still hold the fp32 bar
    w = synth.make_workload("strong decay", seed=71, N=1, H=4, lengths=[203], decay=(0.0068, 0.05),
                            state_std=0.02, win_std=1.0)
    note("strong decay %s" % path)
    _gpu.assert_parity(_gpu.run_sequence(w, gpu, path=path), _gpu.oracle_sequence(w), label="strong decay")


def test_decode_large_state(gpu):
    # 320 x 32 x 64 KiB = 640 MiB of state: the row order used above the cache size
    w = synth.workload(1, scale={"N": 320, "H": 32, "steps": 2})
    note("decode 320x32 (640 MiB state), 2 steps, sampled")
    full = _gpu.run_decode(w, gpu)
    sw, ww = _gpu.decode_as_prefill(w)
    seqs, heads = [0, 199, 319], [1, 30]
    ref = _gpu.oracle_sequence(synth.subset(sw, seqs, heads))
    y = full["y"].reshape(2, 320, 32, 128)[:, seqs][:, :, heads]
    got = {"y": np.ascontiguousarray(y.swapaxes(0, 1)).reshape(-1, len(heads), 128),
           "state": full["state"][seqs][:, heads], "win": full["win"][seqs][:, heads]}
    _gpu.assert_parity(got, ref, keys=("y", "state"), label="decode large")


# ---------------------------------------------------------------- invariances

@pytest.mark.parametrize("other", ["split", "chunk", "short", "scan", "chunk_short"])
def test_prefill_paths_agree(gpu, other):
    w = synth.workload(3, scale={"N": 3, "H": 5, "T": 131})
    note("%s vs fused prefill" % other)
    a = _gpu.run_sequence(w, gpu, path="fused")
    b = _gpu.run_sequence(w, gpu, path=other)
    for k in ("o_raw", "state"):
        assert _gpu.rel_err(a[k], b[k]) <= 2e-5, k
    assert _gpu.rel_err(a["y"], b["y"]) <= 1e-2
    np.testing.assert_array_equal(a["win"], b["win"])


@pytest.mark.parametrize("path", ["chunk", "scan", "chunk_short"])
def test_chunk_path_rejects_unbounded_gates(gpu, path):
    w = synth.make_workload("raw", seed=5, N=1, H=2, lengths=[20], gate_mode=synth.GATE_RAW)
    with pytest.raises(kda.KdaError) as ei:
        _gpu.run_sequence(w, gpu, path=path)
    assert ei.value.status == kda.KDA_ERR_UNSUPPORTED


def test_split_sequence_and_token_steps_agree(gpu):
    import torch
    w = synth.workload(2, scale={"H": 2, "T": 50}, seed=77)
    note("split invariance T=50 -> 13 + 37, and 50 token steps")
    whole = _gpu.run_sequence(w, gpu)
    cut = 13
    a = dataclasses.replace(w, cu_seqlens=np.array([0, cut]), q=w.q[:cut], k=w.k[:cut], v=w.v[:cut],
                            f=w.f[:cut], beta=w.beta[:cut], g=w.g[:cut])
    ra = _gpu.run_sequence(a, gpu)
    b = dataclasses.replace(w, cu_seqlens=np.array([0, 50 - cut]), q=w.q[cut:], k=w.k[cut:],
                            v=w.v[cut:], f=w.f[cut:], beta=w.beta[cut:], g=w.g[cut:],
                            state0=ra["state"].astype(np.float32), win0=ra["win"])
    rb = _gpu.run_sequence(b, gpu)
    np.testing.assert_array_equal(rb["win"], whole["win"])
    assert _gpu.rel_err(rb["state"], whole["state"]) <= 1e-5
    assert _gpu.rel_err(np.concatenate([ra["y"], rb["y"]]), whole["y"]) <= 1e-5
    steps = _gpu.run_decode(dataclasses.replace(w, decode_steps=50), gpu)
    assert _gpu.rel_err(steps["state"], whole["state"]) <= 1e-5
    assert _gpu.rel_err(steps["y"], whole["y"]) <= 1e-5


@PATHS
def test_ragged_equals_each_sequence_alone_and_order(gpu, path):
    lengths = [5, 0, 40, 9]
    w = synth.make_workload("r", seed=91, N=4, H=3, lengths=lengths, act_dtype="bf16",
                            state_std=0.02, win_std=1.0)
    note("ragged vs individual vs seq_order %s" % path)
    full = _gpu.run_sequence(w, gpu, path=path)
    ordered = _gpu.run_sequence(w, gpu, seq_order=[2, 0, 3, 1], path=path)
    for k in ("y", "o_raw", "state", "win"):
        np.testing.assert_array_equal(ordered[k], full[k])
    sub = synth.subset(w, [2], [0, 1, 2])
    alone = _gpu.run_sequence(sub, gpu, path=path)
    lo, hi = w.cu_seqlens[2], w.cu_seqlens[3]
    np.testing.assert_array_equal(alone["y"], full["y"][lo:hi])
    np.testing.assert_array_equal(alone["state"][0], full["state"][2])


@PATHS
def test_repeat_runs_bitwise_and_o_raw_optional(gpu, path):
    w = synth.workload(3, scale={"N": 2, "H": 2, "T": 70})
    note("determinism and o_raw=NULL (workspace) %s" % path)
    a = _gpu.run_sequence(w, gpu, path=path)
    b = _gpu.run_sequence(w, gpu, with_o_raw=False, path=path)
    for k in ("y", "state", "win"):
        np.testing.assert_array_equal(a[k], b[k])
    wd = synth.workload(1, scale={"N": 4, "H": 2, "steps": 3})
    c = _gpu.run_decode(wd, gpu)
    e = _gpu.run_decode(wd, gpu, with_o_raw=False)
    for k in ("y", "state", "win"):
        np.testing.assert_array_equal(c[k], e[k])


@pytest.mark.parametrize("path", ["auto", "scan"])
@pytest.mark.parametrize("N,H,T,act,dense", [(2, 3, 2100, "bf16", True),    # 132 chunks: 2 segments
                                             (1, 2, 6200, "f32", False),    # 388 chunks: 3, ragged tail
                                             (1, 1, 9000, "f32", False)])   # 563 chunks: 4
def test_scan_segments_long_sequences(gpu, N, H, T, act, dense, path):
    # few pairs and at least 128 chunks each: the two-pass path cuts the
    # chunks into segments whose operand passes run on a second stream while
    # the previous segment's state pass runs; every element against the oracle,
    # and a second call bit-identical to the first
    w = synth.make_workload("segments", seed=300 + T, N=N, H=H, lengths=[T] * N, act_dtype=act,
                            state_std=0.02, win_std=1.0)
    note("two-pass segments %dx%dx%d %s dense=%s %s" % (N, H, T, act, dense, path))
    a = _gpu.run_sequence(w, gpu, dense=dense, path=path, side_stream=True)
    _gpu.assert_parity(a, _gpu.oracle_sequence(w), bf16=act == "bf16", label="segments T=%d" % T)
    b = _gpu.run_sequence(w, gpu, dense=dense, path=path, side_stream=True)
    for k in ("y", "o_raw", "state", "win"):
        np.testing.assert_array_equal(a[k], b[k])
    # one launch per pass (no second stream): the same arithmetic
    one = _gpu.run_sequence(w, gpu, dense=dense, path=path)
    for k in ("y", "o_raw", "state", "win"):
        np.testing.assert_array_equal(one[k], a[k])
    # without o_raw the readout lives in the workspace after the chunk records,
    # where the segments' RMSNorm + gate read it
    c = _gpu.run_sequence(w, gpu, dense=dense, path=path, with_o_raw=False, side_stream=True)
    for k in ("y", "state", "win"):
        np.testing.assert_array_equal(c[k], a[k])
    if N > 1:
        # the state passes take pairs in the scheduling order, the operand
        # passes in natural order: the result does not depend on the order
        r = _gpu.run_sequence(w, gpu, dense=dense, path=path, seq_order=list(range(N))[::-1], side_stream=True)
        for k in ("y", "o_raw", "state", "win"):
            np.testing.assert_array_equal(r[k], a[k])


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_scan_segments_ragged_few_sequences(gpu, act):
    # a ragged batch of three sequences (12 pairs, the longest 194 chunks):
    # with the host copy of the offsets and a second stream the two-pass path
    # runs in segments, each segment's RMSNorm + gate one launch per sequence;
    # every element against the oracle, and equal to the unsegmented call
    w = synth.make_workload("ragged segments", seed=77, N=3, H=4, lengths=[3100, 40, 2600], act_dtype=act,
                            state_std=0.02, win_std=1.0)
    note("two-pass segments, ragged 3 sequences x 4 heads %s" % act)
    a = _gpu.run_sequence(w, gpu, side_stream=True, cu_host=True)
    _gpu.assert_parity(a, _gpu.oracle_sequence(w), bf16=act == "bf16", label="ragged segments")
    for kw in ({}, {"cu_host": True}, {"side_stream": True}):
        b = _gpu.run_sequence(w, gpu, **kw)
        for k in ("y", "o_raw", "state", "win"):
            np.testing.assert_array_equal(b[k], a[k], err_msg="%s %s" % (kw, k))


def test_scan_calls_on_two_streams(gpu):
    # two independent two-pass calls (disjoint buffers) enqueued on two
    # streams, each with a second stream of its own, running concurrently;
    # both against the oracle
    import torch
    ws = [synth.make_workload("two streams %d" % i, seed=90 + i, N=1, H=8, lengths=[2300 + 500 * i],
                              state_std=0.02, win_std=1.0) for i in range(2)]
    note("two scan-path calls on two streams")
    ds = [synth.to_device(w, gpu) for w in ws]
    streams = [torch.cuda.Stream(device=gpu) for _ in ws]
    sides = [torch.cuda.Stream(device=gpu) for _ in ws]
    torch.cuda.synchronize()
    for w, d, st, sd in zip(ws, ds, streams, sides):
        kda.kda_sequence(_gpu.cfg_of(w, prefill_path=kda.KDA_PREFILL_SCAN), **_gpu.tensors(d),
                         cu_seqlens=d["cu_seqlens"], cu_seqlens_host=w.cu_seqlens.astype(np.int32), num_seqs=w.N,
                         stream=st, side_stream=sd)
    torch.cuda.synchronize()
    for w, d in zip(ws, ds):
        got = {"y": _gpu._np(d["y"]), "o_raw": _gpu._np(d["o_raw"]), "state": _gpu._np(d["state"]),
               "win": d["conv_win"].cpu().numpy()}
        _gpu.assert_parity(got, _gpu.oracle_sequence(w), label=w.name)


def test_empty_calls_are_noops(gpu):
    import torch
    w = synth.make_workload("e", seed=3, N=2, H=2, lengths=[0, 0], state_std=0.02, win_std=1.0)
    note("all-empty sequences")
    got = _gpu.run_sequence(w, gpu)
    np.testing.assert_array_equal(got["state"], w.state0.astype(np.float64))
    np.testing.assert_array_equal(got["win"], w.win0)


# ---------------------------------------------------------------- full sizes

def _sampled(w, full, seqs, heads, bf16):
    sub = synth.subset(w, seqs, heads)
    ref = _gpu.oracle_sequence(sub)
    rows = np.concatenate([np.arange(w.cu_seqlens[n], w.cu_seqlens[n + 1]) for n in seqs])
    got = {"y": full["y"][rows][:, heads], "o_raw": full["o_raw"][rows][:, heads],
           "state": full["state"][seqs][:, heads], "win": full["win"][seqs][:, heads]}
    return _gpu.assert_parity(got, ref, bf16=bf16, label=w.name)


def test_full_decode_64x32(gpu):
    w = synth.workload(1, scale={"steps": 40})
    note("full decode 64x32, 40 steps, sampled 12 units")
    full = _gpu.run_decode(w, gpu)
    seqs, heads = [0, 17, 63], [0, 5, 31, 12]
    sw, ww = _gpu.decode_as_prefill(w)
    sub = synth.subset(sw, seqs, heads)
    ref = _gpu.oracle_sequence(sub)
    y = full["y"].reshape(40, 64, 32, 128)[:, seqs][:, :, heads]      # [step, seq, head, dv]
    o = full["o_raw"].reshape(40, 64, 32, 128)[:, seqs][:, :, heads]
    got = {"y": np.ascontiguousarray(y.swapaxes(0, 1)).reshape(-1, len(heads), 128),
           "o_raw": np.ascontiguousarray(o.swapaxes(0, 1)).reshape(-1, len(heads), 128),
           "state": full["state"][seqs][:, heads], "win": full["win"][seqs][:, heads]}
    _gpu.assert_parity(got, ref, label="decode full")


def test_decode_64x32_every_pair_repeated(gpu):
    # every (sequence, head) pair of the 64x32 decode step against the oracle
    # over 8 chained steps, then four more runs bit-identical to the first:
    # 40 launches of 2048 workgroups, enough to catch a state store that loses
    # data to a register write right behind it (such a store corrupted two
    # rows of one pair or two in about one launch of three)
    w = synth.workload(1, scale={"steps": 8})
    note("decode 64x32, 8 steps, every pair, 5 runs")
    first = _gpu.run_decode(w, gpu)
    _gpu.assert_parity(first, _gpu.oracle_decode(w), label="decode 64x32 every pair")
    for rep in range(4):
        again = _gpu.run_decode(w, gpu)
        for k in ("y", "o_raw", "state", "win"):
            np.testing.assert_array_equal(again[k], first[k])


def test_decode_64x32_1000_steps(gpu):
    # the decode workload as stated: 1000 consecutive kda_token_step launches
    # over 64 sequences x 32 heads, every step's inputs resident in HBM,
    # step-major (the layout the bench times); three sequences, every head,
    # against the oracle: every step's y and o_raw, the final state and window.
    # Slow-decay channels (alpha up to 0.999) carry state over the whole run.
    import torch
    w = synth.workload(1)
    seqs = [0, 31, 63]
    note("decode 64x32, 1000 chained steps, sequences %s x all 32 heads" % seqs)
    d = synth.to_device(w, gpu)
    N, steps = w.N, w.decode_steps
    cfg = _gpu.cfg_of(w)
    for s in range(steps):
        sl = slice(s * N, (s + 1) * N)
        kda.kda_token_step(cfg, q=d["q"][sl], k=d["k"][sl], v=d["v"][sl], f=d["f"][sl],
                           beta=d["beta"][sl], g=d["g"][sl], conv_w=d["conv_w"], A_log=d["A_log"],
                           dt_bias=d["dt_bias"], gamma=d["gamma"], state=d["state"],
                           conv_win=d["conv_win"], y=d["y"][sl], o_raw=d["o_raw"][sl])
    torch.cuda.synchronize()
    ns = torch.as_tensor(seqs, device=gpu)

    def seq_major(t):      # [steps * N, H, dv] -> the sampled sequences' rows, sequence-major
        sel = t.view(steps, N, w.H, w.dv).index_select(1, ns)
        return _gpu._np(sel.transpose(0, 1).contiguous().view(-1, w.H, w.dv))
    got = {"y": seq_major(d["y"]), "o_raw": seq_major(d["o_raw"]),
           "state": _gpu._np(d["state"].index_select(0, ns)),
           "win": d["conv_win"].index_select(0, ns).cpu().numpy()}
    del d
    torch.cuda.empty_cache()
    errs = _gpu.assert_parity(got, _gpu.oracle_sequence(synth.decode_subset(w, seqs)), label="decode 1000 steps")
    note("decode 1000 steps: relative errors %s" % errs)


@pytest.mark.parametrize("path", ["auto", "chunk"])
def test_full_prefill_1x32x8192(gpu, path):
    # auto: the two-pass chunk path (32 pairs of 8192 tokens); every head
    # against the oracle
    w = synth.workload(2)
    note("full prefill 1x32x8192 fp32, all 32 heads, %s" % path)
    full = _gpu.run_sequence(w, gpu, path=path)
    _sampled(w, full, [0], list(range(w.H)), bf16=False)


def test_full_batched_prefill_16x64x2048(gpu):
    w = synth.workload(3)
    note("full batched prefill 16x64x2048 bf16, sampled 4 units")
    full = _gpu.run_sequence(w, gpu)
    _sampled(w, full, [0, 11], [3, 60], bf16=True)


def test_full_ragged_prefill_256x32(gpu):
    # the ragged batch at full size (256 sequences of U[1, 4096] tokens, 32
    # heads, bf16, fresh and carried states mixed), launched as the bench
    # launches it (automatic path, longest sequence first); the longest, the
    # shortest, a fresh and a carried sequence at three heads against the
    # oracle, sliced on the device
    import torch
    w = synth.workload(4)
    lens = w.lengths
    fresh = [n for n in range(w.N) if not w.state0[n].any()]
    carried = [n for n in range(w.N) if w.state0[n].any()]
    seqs = sorted({int(np.argmax(lens)), int(np.argmin(lens)), fresh[len(fresh) // 2], carried[len(carried) // 2]})
    heads = [0, 13, 31]
    note("full ragged prefill 256x32 bf16 (%d tokens), sequences %s (lengths %s), heads %s"
         % (w.total_tokens, seqs, [int(lens[n]) for n in seqs], heads))
    d = synth.to_device(w, gpu)
    order = torch.as_tensor(np.argsort(-lens, kind="stable").astype(np.int32), device=gpu)
    kda.kda_sequence(_gpu.cfg_of(w), **_gpu.tensors(d), cu_seqlens=d["cu_seqlens"], seq_order=order,
                     num_seqs=w.N)
    torch.cuda.synchronize()
    rows = torch.as_tensor(np.concatenate([np.arange(w.cu_seqlens[n], w.cu_seqlens[n + 1]) for n in seqs]),
                           device=gpu)
    hs, ns = torch.as_tensor(heads, device=gpu), torch.as_tensor(seqs, device=gpu)
    got = {"y": _gpu._np(d["y"].index_select(0, rows).index_select(1, hs)),
           "o_raw": _gpu._np(d["o_raw"].index_select(0, rows).index_select(1, hs)),
           "state": _gpu._np(d["state"].index_select(0, ns).index_select(1, hs)),
           "win": d["conv_win"].index_select(0, ns).index_select(1, hs).cpu().numpy()}
    del d
    torch.cuda.empty_cache()
    _gpu.assert_parity(got, _gpu.oracle_sequence(synth.subset(w, seqs, heads)), bf16=True, label=w.name)


@pytest.mark.parametrize("path", ["auto", "fused", "chunk", "short", "chunk_short"])
def test_full_short_prefill_64x32x13(gpu, path):
    # the short multi-token case: 13 tokens per sequence over a decode-sized
    # batch, state and window carried in; the oracle covers every pair
    w = synth.workload(5)
    note("full short prefill 64x32x13 fp32, all pairs, %s" % path)
    _gpu.assert_parity(_gpu.run_sequence(w, gpu, path=path), _gpu.oracle_sequence(w), label=w.name)
