"""The amax passes take the largest magnitude of a 16-point FWHT from its
stage-3 values: for the last butterfly pair (u, v), the larger of
|fl(u + v)| and |fl(u - v)| is fl(|u| + |v|) in binary32 round-to-nearest
(one of the two is that sum up to sign; the other is |u| - |v| rounded,
never larger).  Checked here in numpy float32 arithmetic on random pairs
across binades, on exact ties of magnitude, and on the special values."""
import numpy as np


def _both(u, v):
    with np.errstate(over="ignore", invalid="ignore"):
        full = np.fmax(np.abs(u + v), np.abs(u - v))
        short = np.abs(u) + np.abs(v)
    return full, short


def test_random_pairs_all_binades():
    rng = np.random.default_rng(7)
    n = 2_000_000
    mant = rng.random(n, dtype=np.float32) + np.float32(1.0)
    u = (mant * np.exp2(rng.integers(-140, 128, n)).astype(np.float32)).astype(np.float32)
    v = ((rng.random(n, dtype=np.float32) + np.float32(1.0)) *
         np.exp2(rng.integers(-140, 128, n)).astype(np.float32)).astype(np.float32)
    u *= rng.choice(np.float32([-1, 1]), n)
    v *= rng.choice(np.float32([-1, 1]), n)
    full, short = _both(u, v)
    assert np.array_equal(full.view(np.uint32), short.view(np.uint32))


def test_close_magnitudes_and_specials():
    rng = np.random.default_rng(8)
    base = rng.standard_normal(200_000).astype(np.float32)
    ulp = np.spacing(base)
    u = base
    v = (base + ulp * rng.integers(-3, 4, base.size)).astype(np.float32)
    v *= rng.choice(np.float32([-1, 1]), base.size)
    full, short = _both(u, v)
    assert np.array_equal(full.view(np.uint32), short.view(np.uint32))
    sp = np.float32([0.0, -0.0, np.inf, -np.inf, 3.4028235e38, -3.4028235e38, 1e-45, -1e-45, 1.0])
    uu, vv = np.meshgrid(sp, sp)
    full, short = _both(uu.ravel(), vv.ravel())
    assert np.array_equal(full.view(np.uint32), short.view(np.uint32))
