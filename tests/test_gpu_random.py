"""Seeded random configurations against the oracle: layer geometries (key
heads, value heads a key head, dk and dv), stream counts, window lengths and
tree shapes, long- and short-memory gates, zero and resumed states.  Each case
draws its configuration from its own seed, so a failure names a configuration
that can be rerun alone."""
import numpy as np
import pytest

from verify_causal_conv1d_amd import inputs as gi

import test_gpu_prefill as tp
import test_gpu_rows as tr
from gpu_util import announce

pytestmark = pytest.mark.gpu


def draw(seed: int):
    rng = np.random.default_rng(seed)
    kind = ("window", "tree", "prefill")[seed % 3]
    long_memory = bool(rng.integers(0, 2))
    if kind == "prefill":
        hk = int(rng.choice([1, 2]))
        shape = gi.Shape(hk=hk, hv=hk * int(rng.choice([1, 2, 3, 4])), dk=128, dv=128)
        lengths = [int(x) for x in rng.integers(0, 300, size=int(rng.integers(1, 7)))]
        return kind, gi.make_batch(shape, lengths, seed=seed, zero_state=bool(rng.integers(0, 2)),
                                   long_memory=long_memory)
    hk = int(rng.choice([1, 2, 4]))
    shape = gi.Shape(hk=hk, hv=hk * int(rng.choice([1, 2, 3, 4])), dk=int(rng.choice([64, 128])),
                     dv=int(rng.choice([64, 128])))
    lengths = [int(x) for x in rng.integers(0 if kind == "window" else 1, 17, size=int(rng.integers(1, 21)))]
    return kind, gi.make_batch(shape, lengths, seed=seed, tree=kind == "tree", long_memory=long_memory)


@pytest.mark.parametrize("seed", list(range(9001, 9013)))
def test_random_configuration(seed):
    kind, b = draw(seed)
    s = b.shape
    announce(f"random {kind} seed={seed} hk={s.hk} hv={s.hv} dk={s.dk} dv={s.dv} lengths={b.lengths()}")
    if kind == "prefill":
        out, tail, state = tp.run_prefill(b)
        tp.check(b, out, tail, state)
    else:
        out, ts, ss = tr.run_window(b, tree=kind == "tree")
        tr.check_against_oracle(b, out, ts, ss, tree=kind == "tree")
