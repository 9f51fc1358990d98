"""GPU parity on seeded random small shapes: every path, both activation
types, the three gate forms, several gate bounds, carried or zero state and
window, fresh sequences, dense and packed batches, with and without o_raw.
Each case is checked against the oracle to the same bars as the other parity
tests.  The cases are fixed by their seeds."""
import numpy as np
import pytest

from linear_attention_recurrence_token_amd import synth
from tests import _gpu

pytestmark = pytest.mark.gpu

LENGTHS = [0, 1, 2, 3, 4, 7, 8, 9, 13, 15, 16, 17, 31, 32, 33, 47, 64, 100, 255, 256, 257, 600]
DECAY_LOW = {-5.0: 0.8, -2.0: 0.4, -7.5: 0.5}    # decays each bound can reach: exp(lb) < d < 1


def _case(seed):
    rng = np.random.default_rng(seed)
    kind = rng.choice(["prefill", "prefill", "prefill", "decode"])
    act = str(rng.choice(["f32", "bf16"]))
    gate = int(rng.choice([synth.GATE_BOUNDED] * 4 + [synth.GATE_LITERAL, synth.GATE_RAW]))
    lb = float(rng.choice([-5.0, -5.0, -2.0, -7.5]))
    common = dict(seed=seed, H=int(rng.integers(1, 9)), act_dtype=act,
                  state_std=0.02 if rng.random() < 0.7 else None,
                  win_std=1.0 if rng.random() < 0.7 else None,
                  gamma_range=(0.5, 1.5) if rng.random() < 0.5 else None,
                  gate_mode=gate, lower_bound=lb, decay=(DECAY_LOW[lb], 0.999))
    if kind == "decode":
        return "decode", synth.make_workload("random decode", N=int(rng.integers(1, 40)),
                                             decode_steps=int(rng.integers(1, 6)), **common), {}
    N = int(rng.integers(1, 24))
    lengths = [int(rng.choice(LENGTHS)) if rng.random() < 0.6 else int(rng.integers(0, 700)) for _ in range(N)]
    path = str(rng.choice(["auto", "fused", "split", "chunk", "short", "scan", "chunk_short"]))
    if path in ("chunk", "scan", "chunk_short") and gate != synth.GATE_BOUNDED:
        path = "auto"          # the chunkwise forms take the bounded gate only
    fresh = 0.3 if rng.random() < 0.3 else None
    w = synth.make_workload("random prefill", N=N, lengths=lengths, fresh_prob=fresh, **common)
    opts = dict(path=path, dense=len(set(lengths)) == 1 and rng.random() < 0.5,
                with_o_raw=bool(rng.random() < 0.7))
    return "prefill", w, opts


@pytest.mark.parametrize("seed", range(7000, 7080))
def test_random_shape(gpu, seed):
    kind, w, opts = _case(seed)
    label = "seed %d %s N=%d H=%d %s %s" % (seed, kind, w.N, w.H, w.act_dtype, opts)
    print(label, flush=True)
    bf16 = w.act_dtype == "bf16"
    if kind == "decode":
        _gpu.assert_parity(_gpu.run_decode(w, gpu), _gpu.oracle_decode(w), bf16=bf16, label=label)
    else:
        _gpu.assert_parity(_gpu.run_sequence(w, gpu, **opts), _gpu.oracle_sequence(w), bf16=bf16, label=label)
