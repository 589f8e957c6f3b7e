"""The fp64 oracle against facts fixed by the mathematics (CPU only)."""
import pytest

import oracle
from tests import oracle_pins

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


@pytest.fixture(scope="module")
def orc():
    oracle.build()
    return oracle.default()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_thread_count_does_not_change_bits(orc):
    import numpy as np
    rng = np.random.default_rng(20)
    B, Hq, Hkv, N, d = 1, 4, 2, 40, 8
    q, k, v, dO = (rng.standard_normal(s) for s in ((B, Hq, N, d), (B, Hkv, N, d), (B, Hkv, N, d), (B, Hq, N, d)))
    a = orc.forward(q, k, v, True, 0.3, threads=1)
    b = orc.forward(q, k, v, True, 0.3, threads=7)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    a = orc.backward(q, k, v, dO, True, 0.3, threads=1)[:3]
    b = orc.backward(q, k, v, dO, True, 0.3, threads=5)[:3]
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


def test_rejects_bad_shapes(orc):
    import numpy as np
    q = np.zeros((1, 3, 4, 2)); k = np.zeros((1, 2, 4, 2))
    with pytest.raises(ValueError):
        orc.forward(q, k, k, False, 1.0)
    with pytest.raises(RuntimeError):
        orc.forward(np.zeros((1, 2, 4, 2)), k, k, False, 1.0, rows=[0, 9])


def test_causal_row_stats_shortcut_matches_full_statistics(orc):
    # The long-sequence GPU backward check feeds the oracle row statistics for only the rows it
    # needs (sampled queries and the last keys' queries); on a small causal problem that must
    # give what the oracle's own full statistics give.
    import math
    import numpy as np
    import seedgen
    from tests import gpu_harness as H
    B, Hq, Hkv, N, d = 1, 4, 2, 300, 64
    q, k, v, dO = (H.f64(x) for x in seedgen.attention_inputs(5, B, Hq, Hkv, N, d, with_do=True))
    scale = 1 / math.sqrt(d)
    qrows = seedgen.sample_rows_all(5, B * Hq, N, 8)
    tail = np.arange(N - 16, N, dtype=np.int32)
    stat_rows = np.concatenate([qrows, np.tile(tail, (B * Hq, 1))], axis=1)
    stats = H.causal_row_stats(q, k, v, dO, scale, stat_rows)
    krows = np.tile(tail, (B * Hkv, 1))
    short = orc.backward(q, k, v, dO, True, scale, qrows=qrows, krows=krows, stats=stats)[:3]
    full = orc.backward(q, k, v, dO, True, scale, qrows=qrows, krows=krows)[:3]
    for a, b in zip(short, full):
        assert np.abs(a - b).max() <= 1e-12 * max(1.0, np.abs(b).max())
