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
    assert lib.kda_version() == 1
    for st in (0, -1, -2, -3, -4):
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


def _seq(lib, cfg, t, n=2, cu=None, order=None, total=8, ws=None, ws_bytes=0):
    return lib.kda_sequence(ctypes.byref(cfg), ctypes.byref(t), n, cu, order, total, ws, ws_bytes, None)


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
    ({"prefill_path": 5}, kda.KDA_ERR_INVALID_ARG),
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
    # passes validation, then stops at the device check (no GPU here) -- or launches nothing
    # on a GPU machine because the fake pointers never reach a kernel: skip there
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is present")
    except ImportError:
        pass
    assert _step(lib, _cfg(), _fake_tensors(beta=(1 << 40) + 4)) == kda.KDA_ERR_DEVICE


def test_workspace_size_and_checks(lib):
    # bounded gate: AUTO takes the chunkwise kernel, or the short-sequence
    # kernel when the sequences are very short on average; neither needs one
    assert lib.kda_sequence_workspace_size(ctypes.byref(_cfg()), 2, 100) == 0
    assert lib.kda_sequence_workspace_size(ctypes.byref(_cfg()), 2, 14) == 0
    assert lib.kda_sequence_workspace_size(ctypes.byref(_cfg()), 2, 16) == 0
    # other gates, few (sequence, head) pairs: the split path wants one fp32
    # readout row per token.head
    lit = dict(gate_mode=kda.KDA_GATE_LITERAL)
    assert lib.kda_sequence_workspace_size(ctypes.byref(_cfg(**lit)), 2, 100) == 100 * 4 * 128 * 4
    assert lib.kda_sequence_workspace_size(ctypes.byref(_cfg(prefill_path=1)), 2, 100) == 0
    assert lib.kda_sequence_workspace_size(ctypes.byref(_cfg(prefill_path=3)), 2, 100) == 0
    assert lib.kda_sequence_workspace_size(ctypes.byref(_cfg(prefill_path=4)), 2, 100) == 0
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
    # the short path addresses a batch's token rows with 32-bit offsets
    big = (1 << 32) // (4 * 128 * 4) + 2           # tokens with H = 4 past 4 GiB of fp32 rows
    assert _seq(lib, _cfg(prefill_path=4), t, n=2, total=big) == kda.KDA_ERR_UNSUPPORTED
