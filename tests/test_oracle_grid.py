"""Pins for the oracle's element grids and rounding (CPU only).

Each check compares the oracle with something other than itself: the level
sets printed (or implied) by the pages, an independent argmin-with-ties
rounding, exact rational arithmetic, and the closed-form shrinkage error.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.conftest import read_golden


def _levels(name):
    return [float(r[0]) for r in read_golden(name)]


def test_e2m1_levels_match_pages_and_format_definition():
    page = _levels("e2m1_levels.txt")
    # E2M1 from the bit layout: 2 exponent bits (bias 1), 1 mantissa bit.
    from_bits = []
    for e in range(4):
        for m in range(2):
            from_bits.append(m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2))
    assert page == from_bits
    assert [oracle.lib().fp4r_level(0, k) for k in range(8)] == page


def test_uniform_levels_match_pages():
    page = _levels("uniform_levels.txt")
    assert [oracle.lib().fp4r_level(1, k) for k in range(8)] == page
    assert len(set(np.diff(page))) == 1  # equal spacing


def _argmin_tie_even(m: np.ndarray, levels) -> np.ndarray:
    """Independent nearest-level rounding: argmin of |L - m|, ties to the even index."""
    L = np.asarray(levels, dtype=np.float64)
    d = np.abs(m.astype(np.float64)[:, None] - L[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # prefer the even index among the (at most two) candidates
    even = cand & (np.arange(8)[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    return pick.astype(np.uint8)


def _probe_values(top: float, levels) -> np.ndarray:
    """Every fp32 within 2048 ulps of each level and midpoint, a strided sweep
    of all fp32 bit patterns in [0, 8], and random bit patterns."""
    L = np.asarray(levels, dtype=np.float64)
    mids = (L[:-1] + L[1:]) / 2
    anchors = np.concatenate([L, mids, [8.0]]).astype(np.float32)
    off = np.arange(-2048, 2049, dtype=np.int64)
    bits = anchors.view(np.int32).astype(np.int64)[:, None] + off[None, :]
    bits = bits[(bits >= 0)].astype(np.uint32)
    top_bits = np.float32(8.0).view(np.uint32)
    sweep = np.arange(0, int(top_bits) + 1, 9973, dtype=np.uint32)
    rnd = np.random.default_rng(7).integers(0, int(top_bits) + 1, 2_000_000, dtype=np.uint32)
    allb = np.unique(np.concatenate([bits, sweep, rnd]))
    return allb.view(np.float32)


@pytest.mark.parametrize("grid,fixture", [("e2m1", "e2m1_levels.txt"),
                                          ("uniform", "uniform_levels.txt")])
def test_rtne_matches_independent_argmin(grid, fixture):
    levels = _levels(fixture)
    m = _probe_values(levels[-1], levels)
    got = oracle.round_grid(m, grid, "rtne")
    want = _argmin_tie_even(m, levels)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (m[bad[:10]], got[bad[:10]], want[bad[:10]])


def test_rtne_tie_table():
    # ties go to the even code (E2M1: .25->0, .75->1.0, 1.25->1.0, 1.75->2,
    # 2.5->2, 3.5->4, 5->4; uniform: 2.5->2, 3.5->4, 6.5->6)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
    assert list(oracle.round_grid(ties, "e2m1")) == [0, 2, 2, 4, 4, 6, 6]
    ut = np.array([0.5, 1.5, 2.5, 3.5, 4.5, 5.5, 6.5], dtype=np.float32)
    assert list(oracle.round_grid(ut, "uniform")) == [0, 2, 2, 4, 4, 6, 6]


def test_saturation_and_infinity():
    m = np.array([6.0, 6.5, 7.9, 1e30, np.inf], dtype=np.float32)
    assert list(oracle.round_grid(m, "e2m1")) == [7] * 5
    m = np.array([7.0, 7.4, 1e30, np.inf], dtype=np.float32)
    assert list(oracle.round_grid(m, "uniform")) == [7] * 4


@pytest.mark.parametrize("grid,fixture", [("e2m1", "e2m1_levels.txt"),
                                          ("uniform", "uniform_levels.txt")])
def test_sr_exhaustive_over_draws(grid, fixture):
    """For each m, the draws that round up are exactly those with
    64 * u16 + 1 <= p * 2^22, p = (m - L[k]) / (L[k+1] - L[k]) in exact
    rationals: their number is min(2^16, floor((p * 2^22 - 1) / 64) + 1), so
    E[q] is within one part in 2^16 of a bin width of m (unbiased up to the
    draw resolution: TetraJet-v2 page, 2.A)."""
    levels = _levels(fixture)
    rng = np.random.default_rng(3)
    ms = np.concatenate([rng.uniform(0, levels[-1], 40),
                         np.array(levels[:-1]) + 1e-7, np.array(levels[1:]) - 1e-6,
                         [0.0, 1e-30, levels[-1] * 0.999999]]).astype(np.float32)
    u = np.arange(65536, dtype=np.uint32)
    for mf in ms:
        k_all = oracle.round_grid(np.full(65536, mf, dtype=np.float32), grid, "sr", u)
        m = Fraction(float(mf))
        k = max(i for i in range(8) if Fraction(levels[i]) <= m)
        if k == 7:
            assert (k_all == 7).all()
            continue
        lo, hi = Fraction(levels[k]), Fraction(levels[k + 1])
        p = (m - lo) / (hi - lo)
        n_up = int(np.count_nonzero(k_all == k + 1))
        X = p * (1 << 22)
        want = 0 if X < 1 else min(65536, int((X - 1) // 64) + 1)
        assert n_up == want, (float(mf), n_up, want)
        up = np.nonzero(k_all == k + 1)[0]
        assert (64 * up.astype(np.int64) + 1 <= X).all()   # exactly the small draws
        if up.size:
            assert up.max() == up.size - 1
        assert set(np.unique(k_all)) <= {k, k + 1}
        mean = lo + (hi - lo) * Fraction(n_up, 65536)
        assert abs(mean - m) <= (hi - lo) / 65536


@pytest.mark.parametrize("grid", ["e2m1", "uniform"])
def test_shrinkage_closed_form(grid):
    """Monte Carlo through the oracle: for magnitudes uniform over [0, top],
    the mean error of the values landing in each level's bin equals the
    closed form (l - r)/2 of the shrinkage-bias page (Metodologia 1)."""
    table = [(float(r[1]), float(r[4])) for r in read_golden("shrinkage_closed_form.txt")
             if r[0] == grid]
    levels = _levels("e2m1_levels.txt" if grid == "e2m1" else "uniform_levels.txt")
    rng = np.random.default_rng(11)
    v = rng.uniform(0, levels[-1], 4_000_000).astype(np.float32)
    k = oracle.round_grid(v, grid, "rtne")
    q = np.asarray(levels)[k]
    err = q - v.astype(np.float64)
    for level, expected in table:
        sel = q == level
        n = int(sel.sum())
        assert n > 1000
        mean = err[sel].mean()
        sigma = err[sel].std() / np.sqrt(n)
        assert abs(mean - expected) < 5 * sigma + 1e-9, (grid, level, mean, expected, sigma)


def test_uniform_density_nets_zero_bias():
    """Both grids have zero net RTNE bias for a density uniform over
    [0, top]: the E2M1 shrinkage comes from where the mass sits."""
    rng = np.random.default_rng(12)
    for grid, top in (("e2m1", 6.0), ("uniform", 7.0)):
        v = rng.uniform(0, top, 4_000_000).astype(np.float32)
        lev = np.asarray(_levels("e2m1_levels.txt" if grid == "e2m1" else "uniform_levels.txt"))
        err = lev[oracle.round_grid(v, grid)] - v
        assert abs(err.mean()) < 5 * err.std() / np.sqrt(v.size)
