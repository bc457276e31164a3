"""Pins for the oracle's expert-load diagnostics (load_stats): closed forms
for uniform and fully concentrated loads, scipy's entropy and numpy's
population std as independent routines, and a pure-Python walk over the
counts for random loads (including empty experts)."""
import math

import numpy as np
import pytest
from scipy import stats as sps

from oracle import moe_oracle as O


def walk(counts):
    """Each figure spelled out over a Python list."""
    E, S = len(counts), sum(counts)
    mean = S / E
    if S == 0:
        return [max(counts), min(counts), mean, 0.0, 0.0, 0.0, float(counts.count(0)), 0.0]
    ent = 0.0
    for n in counts:
        if n:
            ent -= (n / S) * math.log(n / S)
    var = sum((n - mean) ** 2 for n in counts) / E
    return [max(counts), min(counts), mean, max(counts) / mean, ent,
            ent / math.log(E) if E > 1 else 1.0, float(counts.count(0)), math.sqrt(var) / mean]


@pytest.mark.parametrize("E", [1, 2, 8, 128, 256])
def test_uniform_load_closed_form(E):
    s = O.load_stats(np.full(E, 1024, dtype=np.int32))
    assert s[0] == s[1] == s[2] == 1024 and s[3] == 1.0 and s[6] == 0 and s[7] == 0
    assert s[4] == pytest.approx(math.log(E), rel=1e-14, abs=1e-15)
    assert s[5] == pytest.approx(1.0, rel=1e-14)


@pytest.mark.parametrize("E", [2, 8, 128])
def test_all_rows_on_one_expert(E):
    c = np.zeros(E, dtype=np.int32)
    c[E // 2] = 4096
    s = O.load_stats(c)
    assert s[0] == 4096 and s[1] == 0 and s[3] == pytest.approx(E) and s[4] == 0 and s[5] == 0
    assert s[6] == E - 1
    assert s[7] == pytest.approx(math.sqrt(E - 1), rel=1e-14)  # std/mean of one spike


def test_no_rows():
    s = O.load_stats(np.zeros(16, dtype=np.int32))
    assert s[6] == 16 and (np.delete(s, 6) == 0).all()


@pytest.mark.parametrize("seed", range(5))
def test_random_loads_against_scipy_and_a_walk(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(2, 257))
    c = rng.integers(0, 50, size=E).astype(np.int32)
    c[rng.integers(0, E, size=3)] = 0
    s = O.load_stats(c)
    np.testing.assert_allclose(s, walk(c.tolist()), rtol=1e-13, atol=1e-15)
    assert s[4] == pytest.approx(sps.entropy(c.astype(np.float64)), rel=1e-13)
    assert s[7] == pytest.approx(np.std(c.astype(np.float64)) / c.mean(), rel=1e-13)


def test_from_a_dispatch_plan():
    # Counts from the oracle's own dispatch of a Zipf-like assignment.
    rng = np.random.default_rng(9)
    E, T, k = 32, 500, 4
    w = np.arange(1, E + 1) ** -1.2
    idx = np.stack([rng.choice(E, size=k, replace=False, p=w / w.sum()) for _ in range(T)]).astype(np.int32)
    counts = O.dispatch_plan(idx, E)[0]
    s = O.load_stats(counts)
    assert s[2] == T * k / E and s[0] == counts.max() and s[3] > 1.0 and 0 < s[5] < 1
