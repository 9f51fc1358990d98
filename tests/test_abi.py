"""The C ABI: the library loads, exports every function include/kda.h
declares, and rejects bad arguments with the documented status before it
touches any device (CPU only; no kernel is launched here)."""
import ctypes
import os
import re

import pytest

from linear_attention_recurrence_token_amd import kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(kda_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.LIB_PATH):
        pytest.fail("libkda.so is not built; run __graft_entry__.build()")
    return kda.lib()


def test_header_declares_the_boundary():
    fns = declared_functions()
    assert fns == sorted(kda.EXPORTS), fns


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.kda_version() == 2
    for st in (0, -1, -2, -3, -4, -5):
        s = kda.status_string(st)
        assert s and s != "unknown status"
    assert kda.status_string(12345) == "unknown status"


def test_struct_layout_matches_header():
    # 6 int32 + 3 float + 1 int32, no padding; 14 pointers
    assert ctypes.sizeof(kda.kda_config) == 40
    assert ctypes.sizeof(kda.kda_tensors) == 14 * ctypes.sizeof(ctypes.c_void_p)


def _fake_tensors(**over):
    # distinct 256-byte aligned fake addresses: validation never dereferences them
    base = 1 << 40
    vals = {name: base + i * (1 << 30) for i, name in enumerate(kda.TENSOR_FIELDS)}
    vals["o_raw"] = None
    vals.update(over)
    return kda.kda_tensors(*[vals[n] for n in kda.TENSOR_FIELDS])


def _cfg(**over):
    c = kda.KdaConfig(num_heads=4)
    for kk, vv in over.items():
        setattr(c, kk, vv)
    return c.to_c()


def _step(lib, cfg, t, n=2):
    return lib.kda_token_step(ctypes.byref(cfg), ctypes.byref(t), n, None)


def _seq(lib, cfg, t, n=2, cu=None, order=None, total=8, ws=None, ws_bytes=0, cu_host=None, stream=None,
         side=None):
    return lib.kda_sequence(ctypes.byref(cfg), ctypes.byref(t), n, cu, cu_host, order, total, ws, ws_bytes, stream,
                            side)


@pytest.mark.parametrize("over,status", [
    ({"head_dim_k": 64}, kda.KDA_ERR_UNSUPPORTED),
    ({"head_dim_v": 256}, kda.KDA_ERR_UNSUPPORTED),
    ({"conv_taps": 3}, kda.KDA_ERR_UNSUPPORTED),
    ({"num_heads": 0}, kda.KDA_ERR_INVALID_ARG),
    ({"act_dtype": 7}, kda.KDA_ERR_INVALID_ARG),
    ({"gate_mode": 3}, kda.KDA_ERR_INVALID_ARG),
    ({"gate_mode": -1}, kda.KDA_ERR_INVALID_ARG),
    ({"l2_eps": -1.0}, kda.KDA_ERR_INVALID_ARG),
    ({"rms_eps": float("nan")}, kda.KDA_ERR_INVALID_ARG),
    ({"gate_lower_bound": float("nan")}, kda.KDA_ERR_INVALID_ARG),
    ({"prefill_path": 7}, kda.KDA_ERR_INVALID_ARG),
])
def test_bad_config_rejected(lib, over, status):
    t = _fake_tensors()
    assert _step(lib, _cfg(**over), t) == status
    assert _seq(lib, _cfg(**over), t) == status


@pytest.mark.parametrize("field", [f for f in kda.TENSOR_FIELDS if f != "o_raw"])
def test_null_or_misaligned_tensor_rejected(lib, field):
    assert _step(lib, _cfg(), _fake_tensors(**{field: None})) == kda.KDA_ERR_INVALID_ARG
    mis = (1 << 40) + (2 if field == "beta" else 8)      # beta needs only 4-byte alignment
    assert _step(lib, _cfg(), _fake_tensors(**{field: mis})) == kda.KDA_ERR_INVALID_ARG
    assert _seq(lib, _cfg(), _fake_tensors(**{field: None})) == kda.KDA_ERR_INVALID_ARG


def test_empty_work_is_a_noop_without_pointers(lib):
    nulls = kda.kda_tensors()
    assert _step(lib, _cfg(), nulls, n=0) == kda.KDA_OK
    assert _seq(lib, _cfg(), nulls, n=3, total=0) == kda.KDA_OK
    assert _seq(lib, _cfg(), nulls, n=0, total=0) == kda.KDA_OK
    assert _seq(lib, _cfg(head_dim_k=64), nulls, n=3, total=0) == kda.KDA_ERR_UNSUPPORTED


def test_aliasing_rejected(lib):
    base = _fake_tensors()
    assert _step(lib, _cfg(), _fake_tensors(y=base.q)) == kda.KDA_ERR_INVALID_ARG
    assert _step(lib, _cfg(), _fake_tensors(state=base.conv_win)) == kda.KDA_ERR_INVALID_ARG
    assert _step(lib, _cfg(), _fake_tensors(o_raw=base.y)) == kda.KDA_ERR_INVALID_ARG
    assert _step(lib, _cfg(), _fake_tensors(o_raw=base.beta)) == kda.KDA_ERR_INVALID_ARG
    assert _step(lib, _cfg(), _fake_tensors(o_raw=(1 << 40) + 4)) == kda.KDA_ERR_INVALID_ARG


def test_beta_needs_only_word_alignment(lib):
    # passes validation, then stops at the device check when no GPU is present;
    # with a GPU it would go on to launch on the fake pointers, so it is skipped there
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is present")
    except ImportError:
        pass
    assert _step(lib, _cfg(), _fake_tensors(beta=(1 << 40) + 4)) == kda.KDA_ERR_DEVICE


def test_workspace_size_and_checks(lib):
    # bounded gate: AUTO takes the chunkwise kernel, which asks for its pair
    # counter (256 bytes), or for short sequences on average the chunk kernel
    # without a pipeline or the short-sequence kernel, which need none
    TICKETS = 256
    assert lib.kda_sequence_workspace_size(ctypes.byref(_cfg()), 2, 100) == TICKETS
    assert lib.kda_sequence_workspace_size(ctypes.byref(_cfg()), 2, 14) == 0
    assert lib.kda_sequence_workspace_size(ctypes.byref(_cfg()), 2, 16) == 0
    # other gates, few (sequence, head) pairs: the split path wants one fp32
    # readout row per token.head
    lit = dict(gate_mode=kda.KDA_GATE_LITERAL)
    assert lib.kda_sequence_workspace_size(ctypes.byref(_cfg(**lit)), 2, 100) == 100 * 4 * 128 * 4
    assert lib.kda_sequence_workspace_size(ctypes.byref(_cfg(prefill_path=1)), 2, 100) == 0
    assert lib.kda_sequence_workspace_size(ctypes.byref(_cfg(prefill_path=3)), 2, 100) == TICKETS
    assert lib.kda_sequence_workspace_size(ctypes.byref(_cfg(prefill_path=4)), 2, 100) == 0
    assert lib.kda_sequence_workspace_size(ctypes.byref(_cfg(prefill_path=6)), 2, 100) == 0
    # the two-pass chunk path: records (35 KiB per chunk slot and head; a
    # sequence of len tokens takes at most len // 16 + 1 slots), then the readout
    rec = lambda T, N, H: ((T // 16 + N) * H * 35840 + 255) // 256 * 256
    out = lambda T, H: T * H * 128 * 4
    assert lib.kda_sequence_workspace_size(ctypes.byref(_cfg(prefill_path=5)), 2, 100) == rec(100, 2, 4) + out(100, 4)
    # AUTO takes it for at most 64 pairs (here 8) averaging at least 128 tokens
    assert lib.kda_sequence_workspace_size(ctypes.byref(_cfg()), 2, 256) == rec(256, 2, 4) + out(256, 4)
    assert lib.kda_sequence_workspace_size(ctypes.byref(_cfg()), 2, 254) == TICKETS
    assert lib.kda_sequence_workspace_size(ctypes.byref(_cfg(num_heads=64)), 2, 8192) == TICKETS   # 128 pairs
    assert lib.kda_sequence_workspace_size(ctypes.byref(_cfg(num_heads=32)), 2, 8192) == \
        rec(8192, 2, 32) + out(8192, 32)
    assert lib.kda_sequence_workspace_size(ctypes.byref(_cfg(num_heads=64, **lit)), 16, 100) == 0
    assert lib.kda_sequence_workspace_size(ctypes.byref(_cfg(num_heads=64, prefill_path=2)), 16, 100) \
        == 100 * 64 * 128 * 4
    assert lib.kda_sequence_workspace_size(ctypes.byref(_cfg()), 2, 0) == 0
    assert lib.kda_sequence_workspace_size(ctypes.byref(_cfg()), 2, -1) == kda.KDA_ERR_INVALID_ARG
    assert lib.kda_sequence_workspace_size(ctypes.byref(_cfg(head_dim_k=64)), 2, 5) == kda.KDA_ERR_UNSUPPORTED
    t = _fake_tensors()
    assert _seq(lib, _cfg(), t, ws=(1 << 41) + 4, ws_bytes=1 << 20) == kda.KDA_ERR_INVALID_ARG
    assert _seq(lib, _cfg(), t, ws=1 << 41, ws_bytes=-1) == kda.KDA_ERR_INVALID_ARG
    # forced split without o_raw or a big enough workspace
    assert _seq(lib, _cfg(prefill_path=2), t) == kda.KDA_ERR_INVALID_ARG
    assert _seq(lib, _cfg(prefill_path=2), t, ws=1 << 41, ws_bytes=64) == kda.KDA_ERR_INVALID_ARG


def test_bad_sizes_rejected(lib):
    t = _fake_tensors()
    assert _step(lib, _cfg(), t, n=-1) == kda.KDA_ERR_INVALID_ARG
    assert _seq(lib, _cfg(), t, n=-1) == kda.KDA_ERR_INVALID_ARG
    assert _seq(lib, _cfg(), t, n=3, total=8) == kda.KDA_ERR_INVALID_ARG        # dense, 8 % 3 != 0
    assert _seq(lib, _cfg(), t, n=2, total=-5) == kda.KDA_ERR_INVALID_ARG
    assert _seq(lib, _cfg(), t, n=0, total=4) == kda.KDA_ERR_INVALID_ARG
    assert _seq(lib, _cfg(), t, n=2, cu=(1 << 40) + 2) == kda.KDA_ERR_INVALID_ARG  # misaligned cu
    assert _seq(lib, _cfg(), t, n=2, order=(1 << 40) + 1) == kda.KDA_ERR_INVALID_ARG
    assert _step(lib, _cfg(num_heads=1 << 20), t, n=1 << 12) == kda.KDA_ERR_INVALID_ARG


def test_no_device_gives_device_error(lib):
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is present")
    except ImportError:
        pass
    t = _fake_tensors()
    assert _step(lib, _cfg(), t) == kda.KDA_ERR_DEVICE
    assert _seq(lib, _cfg(), t) == kda.KDA_ERR_DEVICE
    assert lib.kda_device_check() == kda.KDA_ERR_DEVICE


def test_python_binding_rejects_host_tensors():
    import torch
    cfg = kda.KdaConfig(num_heads=1)
    z = torch.zeros(1, 1, 128)
    with pytest.raises(ValueError):
        kda.kda_token_step(cfg, q=z, k=z, v=z, f=z, beta=torch.zeros(1, 1), g=z,
                           conv_w=torch.zeros(1, 384, 4), A_log=torch.zeros(1, 128),
                           dt_bias=torch.zeros(1, 128), gamma=torch.zeros(128),
                           state=torch.zeros(1, 1, 128, 128), conv_win=torch.zeros(1, 1, 3, 384),
                           y=torch.zeros(1, 1, 128))


def test_path_support_checked_before_the_device(lib):
    # both refusals depend on the arguments only, so they come back without a GPU
    t = _fake_tensors()
    assert _seq(lib, _cfg(prefill_path=3, gate_mode=kda.KDA_GATE_RAW), t) == kda.KDA_ERR_UNSUPPORTED
    assert _seq(lib, _cfg(prefill_path=3, gate_lower_bound=-8.0), t) == kda.KDA_ERR_UNSUPPORTED
    assert _seq(lib, _cfg(prefill_path=5, gate_mode=kda.KDA_GATE_LITERAL), t) == kda.KDA_ERR_UNSUPPORTED
    assert _seq(lib, _cfg(prefill_path=6, gate_mode=kda.KDA_GATE_RAW), t) == kda.KDA_ERR_UNSUPPORTED
    assert _seq(lib, _cfg(prefill_path=6, gate_lower_bound=-8.0), t) == kda.KDA_ERR_UNSUPPORTED
    # the two-pass path without the workspace it needs
    assert _seq(lib, _cfg(prefill_path=5), t, ws=1 << 41, ws_bytes=1 << 10) == kda.KDA_ERR_INVALID_ARG
    assert _seq(lib, _cfg(prefill_path=5), t) == kda.KDA_ERR_INVALID_ARG
    # the short path addresses a batch's token rows with 32-bit offsets
    big = (1 << 32) // (4 * 128 * 4) + 2           # tokens with H = 4 past 4 GiB of fp32 rows
    assert _seq(lib, _cfg(prefill_path=4), t, n=2, total=big) == kda.KDA_ERR_UNSUPPORTED


# --- the projections ------------------------------------------------------------

def _lowrank(lib, cfg=None, x=1 << 40, w=(1 << 40) + (1 << 30), wfb=(1 << 40) + (2 << 30),
             hidden=64, rank=32, tokens=10, f=(1 << 40) + (3 << 30), beta=(1 << 40) + (4 << 30),
             ws=(1 << 40) + (5 << 30), ws_bytes=1 << 20):
    cfg = cfg or _cfg()
    return lib.kda_lowrank_gates(ctypes.byref(cfg), x, w, wfb, hidden, rank, tokens, f, beta, ws, ws_bytes, None)


def _proj(lib, fn, cfg=None, a=1 << 40, w=(1 << 40) + (1 << 30), hidden=64, tokens=10,
          out=(1 << 40) + (2 << 30), ws=None, ws_bytes=0):
    cfg = cfg or _cfg()
    return getattr(lib, fn)(ctypes.byref(cfg), a, w, hidden, tokens, out, ws, ws_bytes, None)


@pytest.mark.parametrize("over,status", [
    ({"hidden": 0}, kda.KDA_ERR_INVALID_ARG),
    ({"hidden": 48}, kda.KDA_ERR_INVALID_ARG),        # not a multiple of 32
    ({"rank": 16}, kda.KDA_ERR_INVALID_ARG),
    ({"rank": 48}, kda.KDA_ERR_INVALID_ARG),
    ({"rank": 2048}, kda.KDA_ERR_INVALID_ARG),
    ({"tokens": -1}, kda.KDA_ERR_INVALID_ARG),
    ({"x": None}, kda.KDA_ERR_INVALID_ARG),
    ({"w": (1 << 40) + (1 << 30) + 8}, kda.KDA_ERR_INVALID_ARG),
    ({"f": None}, kda.KDA_ERR_INVALID_ARG),
    ({"beta": (1 << 40) + (4 << 30) + 2}, kda.KDA_ERR_INVALID_ARG),
    ({"ws": None, "ws_bytes": 0}, kda.KDA_ERR_INVALID_ARG),   # the rank-r factor needs a home
    ({"ws_bytes": 10 * 32 * 4 - 4}, kda.KDA_ERR_INVALID_ARG),
    ({"f": (1 << 40) + 64}, kda.KDA_ERR_INVALID_ARG),          # f overlaps x
    ({"beta": (1 << 40) + (3 << 30) + 64}, kda.KDA_ERR_INVALID_ARG),   # beta inside f
    ({"ws": (1 << 40) + (3 << 30) + 4096}, kda.KDA_ERR_INVALID_ARG),   # workspace inside f
    ({"cfg": _cfg(head_dim_k=64)}, kda.KDA_ERR_UNSUPPORTED),
    ({"cfg": _cfg(act_dtype=5)}, kda.KDA_ERR_INVALID_ARG),
    ({"cfg": _cfg(num_heads=(1 << 16) + 1)}, kda.KDA_ERR_INVALID_ARG),
    ({"cfg": _cfg(num_heads=(1 << 31) - 1)}, kda.KDA_ERR_INVALID_ARG),
])
def test_lowrank_gates_rejects(lib, over, status):
    assert _lowrank(lib, **over) == status


@pytest.mark.parametrize("fn", ["kda_gate_projection", "kda_output_projection"])
@pytest.mark.parametrize("over,status", [
    ({"hidden": 0}, kda.KDA_ERR_INVALID_ARG),
    ({"hidden": 66}, kda.KDA_ERR_INVALID_ARG),
    ({"tokens": -3}, kda.KDA_ERR_INVALID_ARG),
    ({"a": None}, kda.KDA_ERR_INVALID_ARG),
    ({"w": (1 << 40) + (1 << 30) + 4}, kda.KDA_ERR_INVALID_ARG),
    ({"out": (1 << 40) + (1 << 30)}, kda.KDA_ERR_INVALID_ARG),        # out is the weight
    ({"ws": (1 << 40) + (2 << 30) + 256, "ws_bytes": 1 << 20}, kda.KDA_ERR_INVALID_ARG),  # inside out
    ({"ws": (1 << 41) + 8, "ws_bytes": 1 << 20}, kda.KDA_ERR_INVALID_ARG),
    ({"ws_bytes": -1}, kda.KDA_ERR_INVALID_ARG),
    ({"cfg": _cfg(head_dim_v=64)}, kda.KDA_ERR_UNSUPPORTED),
    ({"cfg": _cfg(num_heads=1 << 20)}, kda.KDA_ERR_INVALID_ARG),
])
def test_projections_reject(lib, fn, over, status):
    assert _proj(lib, fn, **over) == status


def test_gate_projection_hidden_multiple_of_32_output_of_4(lib):
    # K = hidden must be a multiple of 32 for the gate projection; the output
    # projection only writes hidden columns (groups of 4)
    assert _proj(lib, "kda_gate_projection", hidden=68) == kda.KDA_ERR_INVALID_ARG
    try:
        import torch
        if torch.cuda.is_available():
            return
    except ImportError:
        pass
    assert _proj(lib, "kda_output_projection", hidden=68) == kda.KDA_ERR_DEVICE


def test_projections_zero_tokens_and_no_device(lib):
    assert _lowrank(lib, tokens=0, x=None, f=None, beta=None, ws=None, ws_bytes=0) == kda.KDA_OK
    for fn in ("kda_gate_projection", "kda_output_projection"):
        assert _proj(lib, fn, tokens=0, a=None, w=None, out=None) == kda.KDA_OK
    try:
        import torch
        if torch.cuda.is_available():
            return
    except ImportError:
        pass
    assert _lowrank(lib) == kda.KDA_ERR_DEVICE
    assert _proj(lib, "kda_gate_projection") == kda.KDA_ERR_DEVICE
    assert _proj(lib, "kda_output_projection", ws=1 << 42, ws_bytes=1 << 20) == kda.KDA_ERR_DEVICE


def test_projection_workspace_size(lib):
    size = lambda which, hidden, rank, tokens, cfg=None: lib.kda_projection_workspace_size(
        ctypes.byref(cfg or _cfg()), which, hidden, rank, tokens)
    c32 = _cfg(num_heads=32)
    # low-rank gates: the rank-r factor (rounded to 256 bytes), plus split-K
    # scratch for few token rows; from 512 token rows also the bf16 parts of
    # the (r + H) x hidden weights of the first product
    assert size(kda.KDA_PROJ_LOWRANK_GATES, 4096, 128, 32768, c32) == 32768 * 128 * 4 + (128 + 32) * 4096 * 4
    assert size(kda.KDA_PROJ_LOWRANK_GATES, 4096, 128, 3, c32) > 2048
    assert size(kda.KDA_PROJ_LOWRANK_GATES, 64, 32, 3) == 512
    # gate / output: scratch only when the sum is split (few token rows, long sums)
    assert size(kda.KDA_PROJ_GATE, 4096, 0, 64, c32) > 0
    assert size(kda.KDA_PROJ_OUTPUT, 4096, 0, 64, c32) > 0
    assert size(kda.KDA_PROJ_GATE, 4096, 0, 32768, c32) == 0
    assert size(kda.KDA_PROJ_GATE, 64, 0, 64) == 0          # too short a sum to split
    assert size(kda.KDA_PROJ_GATE, 4096, 0, 0, c32) == 0
    assert size(3, 64, 0, 10) == kda.KDA_ERR_INVALID_ARG
    assert size(kda.KDA_PROJ_LOWRANK_GATES, 64, 40, 10) == kda.KDA_ERR_INVALID_ARG
    assert size(kda.KDA_PROJ_GATE, 48, 0, 10) == kda.KDA_ERR_INVALID_ARG
    assert size(kda.KDA_PROJ_OUTPUT, 68, 0, 10) == 2 * 10 * 68 * 4   # K = 4 heads x 128: two splits
    assert size(kda.KDA_PROJ_GATE, 64, 0, -1) == kda.KDA_ERR_INVALID_ARG
    assert size(kda.KDA_PROJ_GATE, 64, 0, 10, _cfg(head_dim_k=64)) == kda.KDA_ERR_UNSUPPORTED


# --- the no-allocation variant of the low-rank gates ---------------------------

def _lowrank_na(lib, cfg=None, x=1 << 40, w=(1 << 40) + (1 << 30), wfb=(1 << 40) + (2 << 30),
                hidden=64, rank=32, tokens=10, f=(1 << 40) + (3 << 30), beta=(1 << 40) + (4 << 30)):
    cfg = cfg or _cfg()
    return lib.kda_lowrank_gates_noalloc(ctypes.byref(cfg), x, w, wfb, hidden, rank, tokens, f, beta, None)


@pytest.mark.parametrize("over,status", [
    ({"hidden": 48}, kda.KDA_ERR_INVALID_ARG),
    ({"rank": 16}, kda.KDA_ERR_INVALID_ARG),
    ({"tokens": -1}, kda.KDA_ERR_INVALID_ARG),
    ({"x": None}, kda.KDA_ERR_INVALID_ARG),
    ({"f": (1 << 40) + 64}, kda.KDA_ERR_INVALID_ARG),          # f overlaps x
    ({"beta": (1 << 40) + (4 << 30) + 2}, kda.KDA_ERR_INVALID_ARG),
    ({"cfg": _cfg(head_dim_k=64)}, kda.KDA_ERR_UNSUPPORTED),
    # the rank-r factor alone is tokens * rank * 4 bytes: past 16 MiB it does not fit
    ({"tokens": 32769, "rank": 128}, kda.KDA_ERR_SCRATCH_LIMIT),
    ({"tokens": 4097, "rank": 1024}, kda.KDA_ERR_SCRATCH_LIMIT),
])
def test_lowrank_gates_noalloc_rejects(lib, over, status):
    assert _lowrank_na(lib, **over) == status


def test_lowrank_gates_noalloc_limit_and_no_device(lib):
    assert kda.KDA_NOALLOC_SCRATCH_BYTES == 16 << 20
    assert "static scratch" in kda.status_string(kda.KDA_ERR_SCRATCH_LIMIT)
    assert _lowrank_na(lib, tokens=0, x=None, f=None, beta=None) == kda.KDA_OK
    try:
        import torch
        if torch.cuda.is_available():
            return
    except ImportError:
        pass
    # exactly the scratch size is allowed: the call gets as far as the device check
    assert _lowrank_na(lib, tokens=32768, rank=128) == kda.KDA_ERR_DEVICE
    assert _lowrank_na(lib) == kda.KDA_ERR_DEVICE


# --- the host copy of the offsets and the second stream -------------------------

def _host(vals):
    a = (ctypes.c_int32 * len(vals))(*vals)
    return a, ctypes.cast(a, ctypes.c_void_p).value


@pytest.mark.parametrize("vals,status", [
    ([0, 3, 8], None),                      # valid: gets as far as the device check
    ([1, 3, 8], kda.KDA_ERR_INVALID_ARG),   # cu[0] != 0
    ([0, 5, 3], kda.KDA_ERR_INVALID_ARG),   # decreasing
    ([0, 3, 7], kda.KDA_ERR_INVALID_ARG),   # does not end at total_tokens
    ([0, 8, 8], None),                      # an empty last sequence is fine
])
def test_sequence_checks_the_host_offsets(lib, vals, status):
    keep, ptr = _host(vals)
    st = _seq(lib, _cfg(), _fake_tensors(), n=2, cu=(1 << 42), total=8, cu_host=ptr)
    if status is None:
        try:
            import torch
            if torch.cuda.is_available():
                return
        except ImportError:
            pass
        assert st == kda.KDA_ERR_DEVICE
    else:
        assert st == status


def test_sequence_host_offsets_need_the_device_array_and_streams_differ(lib):
    keep, ptr = _host([0, 4, 8])
    # a host copy without the device array (a dense batch) is refused
    assert _seq(lib, _cfg(), _fake_tensors(), n=2, cu=None, total=8, cu_host=ptr) == kda.KDA_ERR_INVALID_ARG
    # the second stream may not be the call's own stream
    assert _seq(lib, _cfg(), _fake_tensors(), n=2, total=8, stream=1 << 20, side=1 << 20) == kda.KDA_ERR_INVALID_ARG


# --- the step with the low-rank decay formed inside it, and its factor product ----

def _seq_lr(lib, cfg, t, n=2, cu=None, total=8, a=(1 << 41), wfb=(1 << 41) + (1 << 30), rank=128):
    return lib.kda_sequence_lowrank(ctypes.byref(cfg), ctypes.byref(t), n, cu, None, None, total, a, wfb, rank, None)


@pytest.mark.parametrize("over,status", [
    ({"rank": 48}, kda.KDA_ERR_INVALID_ARG),
    ({"rank": 0}, kda.KDA_ERR_INVALID_ARG),
    ({"rank": 256}, kda.KDA_ERR_UNSUPPORTED),               # above the in-step product's rank
    ({"a": None}, kda.KDA_ERR_INVALID_ARG),
    ({"a": (1 << 41) + 4}, kda.KDA_ERR_INVALID_ARG),
    ({"wfb": None}, kda.KDA_ERR_INVALID_ARG),
    ({"cfg": _cfg(gate_mode=kda.KDA_GATE_LITERAL)}, kda.KDA_ERR_UNSUPPORTED),
    ({"cfg": _cfg(gate_lower_bound=-9.0)}, kda.KDA_ERR_UNSUPPORTED),
    ({"cfg": _cfg(prefill_path=kda.KDA_PREFILL_FUSED)}, kda.KDA_ERR_UNSUPPORTED),
    ({"cfg": _cfg(head_dim_k=64)}, kda.KDA_ERR_UNSUPPORTED),
])
def test_sequence_lowrank_rejects(lib, over, status):
    t = _fake_tensors(f=None)
    assert _seq_lr(lib, over.pop("cfg", _cfg()), t, **over) == status


def test_sequence_lowrank_needs_f_null_and_no_device(lib):
    # f is formed in the step: a caller f is refused
    assert _seq_lr(lib, _cfg(), _fake_tensors()) == kda.KDA_ERR_INVALID_ARG
    # w_fb may not be an output
    t = _fake_tensors(f=None)
    assert _seq_lr(lib, _cfg(), t, wfb=t.y) == kda.KDA_ERR_INVALID_ARG
    assert _seq_lr(lib, _cfg(), _fake_tensors(f=None), total=0) == kda.KDA_OK
    try:
        import torch
        if torch.cuda.is_available():
            return
    except ImportError:
        pass
    assert _seq_lr(lib, _cfg(), _fake_tensors(f=None)) == kda.KDA_ERR_DEVICE


def _factor(lib, cfg=None, x=1 << 40, w=(1 << 40) + (1 << 30), hidden=64, rank=32, tokens=10,
            a=(1 << 40) + (3 << 30), beta=(1 << 40) + (4 << 30), ws=None, ws_bytes=0):
    cfg = cfg or _cfg()
    return lib.kda_lowrank_factor(ctypes.byref(cfg), x, w, hidden, rank, tokens, a, beta, ws, ws_bytes, None)


@pytest.mark.parametrize("over,status", [
    ({"hidden": 48}, kda.KDA_ERR_INVALID_ARG),
    ({"rank": 16}, kda.KDA_ERR_INVALID_ARG),
    ({"tokens": -1}, kda.KDA_ERR_INVALID_ARG),
    ({"x": None}, kda.KDA_ERR_INVALID_ARG),
    ({"a": None}, kda.KDA_ERR_INVALID_ARG),
    ({"a": (1 << 40) + 64}, kda.KDA_ERR_INVALID_ARG),          # a overlaps x
    ({"beta": (1 << 40) + (3 << 30) + 64}, kda.KDA_ERR_INVALID_ARG),   # beta inside a
    ({"ws": (1 << 40) + (3 << 30), "ws_bytes": 1 << 20}, kda.KDA_ERR_INVALID_ARG),   # workspace is a
    ({"cfg": _cfg(head_dim_k=64)}, kda.KDA_ERR_UNSUPPORTED),
])
def test_lowrank_factor_rejects(lib, over, status):
    assert _factor(lib, **over) == status


def test_lowrank_factor_workspace_size(lib):
    cfg = _cfg(num_heads=32)
    few = kda.projection_workspace_size(kda.KdaConfig(num_heads=32), kda.KDA_PROJ_LOWRANK_FACTOR, 4096, 64, 128)
    many = kda.projection_workspace_size(kda.KdaConfig(num_heads=32), kda.KDA_PROJ_LOWRANK_FACTOR, 4096, 8192, 128)
    assert few > 0 and many >= (128 + 32) * 4096 * 4      # split-K partials; the weights' bf16 parts
    assert _factor(lib, tokens=0, x=None, a=None, beta=None) == kda.KDA_OK
