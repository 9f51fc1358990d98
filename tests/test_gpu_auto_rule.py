"""The automatic prefill choice (KDA_PREFILL_AUTO), pinned through its
results: on each shape, AUTO's outputs must be bit-identical to those of
the path the rule names.

For the chunk forms' gate (bounded, |lb| <= 7.5) the rule is:
- the short-sequence kernel below 4 tokens per sequence on average;
- the two-pass path for at most 64 (sequence, head) pairs averaging 128
  tokens or more, when the workspace is given;
- the chunk kernel without a pipeline up to 16 tokens on average, or up
  to 64 from 512 pairs on;
- the pipelined chunk kernel otherwise.

With the other gates: the short-sequence kernel below 8 tokens, else the
split kernel for few pairs.

Every path gives a different rounding, so an equality with the named path
(and the AUTO result's oracle parity) pins the choice."""
import numpy as np
import pytest

from linear_attention_recurrence_token_amd import synth
from tests import _gpu

pytestmark = pytest.mark.gpu

CASES = [
    # (N, H, T, gate, the path AUTO must take, the path on the rule's other side)
    (4, 2, 3, synth.GATE_BOUNDED, "short", "chunk_short"),
    (4, 2, 4, synth.GATE_BOUNDED, "chunk_short", "short"),
    (4, 2, 16, synth.GATE_BOUNDED, "chunk_short", "chunk"),
    (4, 2, 17, synth.GATE_BOUNDED, "chunk", "chunk_short"),
    (16, 32, 40, synth.GATE_BOUNDED, "chunk_short", "chunk"),    # 512 pairs: up to 64 tokens
    (16, 32, 65, synth.GATE_BOUNDED, "chunk", "chunk_short"),
    (2, 2, 300, synth.GATE_BOUNDED, "scan", "chunk"),
    (4, 2, 7, synth.GATE_LITERAL, "short", "split"),
    (4, 2, 8, synth.GATE_LITERAL, "split", "short"),
]


def note(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("N,H,T,gate,expect,other", CASES)
def test_auto_takes_the_named_path(gpu, N, H, T, gate, expect, other):
    w = synth.make_workload("auto rule", seed=900 + T + N, N=N, H=H, lengths=[T] * N, gate_mode=gate,
                            state_std=0.02, win_std=1.0)
    note("AUTO at %dx%dx%d gate %d: expect %s" % (N, H, T, gate, expect))
    auto = _gpu.run_sequence(w, gpu, path="auto")
    named = _gpu.run_sequence(w, gpu, path=expect)
    for k in ("y", "o_raw", "state", "win"):
        np.testing.assert_array_equal(auto[k], named[k], err_msg=k)
    # the pin distinguishes: the path across the threshold rounds differently
    alt = _gpu.run_sequence(w, gpu, path=other)
    assert any(not np.array_equal(auto[k], alt[k]) for k in ("o_raw", "state")), other
    _gpu.assert_parity(auto, _gpu.oracle_sequence(w), label="auto %dx%dx%d" % (N, H, T))
