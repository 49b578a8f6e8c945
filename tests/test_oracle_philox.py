"""Pins for the oracle's Philox4x32-10 generator and its use (CPU only).

Known answers come live from rocRAND's header implementation of the same
published generator (the ``rocrand_kat`` fixture of conftest.py: a host-only
test helper, never linked into the oracle or the HIP library).  Nothing from
it is stored.
"""
import numpy as np

import oracle


def test_philox_matches_rocrand(rocrand_kat):
    rng = np.random.default_rng(1)
    rows = [(0, 0, 0, 0, 0), (1, 0, 0, 0, 0), (0, 0, 0, 1, 0), (2**64 - 1, 2**32 - 1, 7, 0, 0)]
    for _ in range(300):
        key = int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2))
        c = [int(v) for v in rng.integers(0, 2**32, 4)]
        c[1] &= 0x3FFF  # counter.xy is driven through a 64-bit offset*4
        rows.append((key, c[0], c[1], c[2], c[3]))
    want = rocrand_kat(rows)
    for r, w in zip(rows, want):
        got = [int(v) for v in oracle.philox(r[0], r[1:])]
        assert got == w, r


def test_sr_draw_layout_follows_philox_words():
    seed = 0x1234_5678_9ABC
    for g in (0, 1, 12345, 2**33 + 5):
        words = oracle.philox(seed, [g & 0xFFFFFFFF, g >> 32, 0, 0])
        draws = oracle.sr_u16(seed, [8 * g + l for l in range(8)])
        for l in range(8):
            assert draws[l] == (int(words[l >> 1]) >> (16 * (l & 1))) & 0xFFFF


def test_rht_signs_follow_philox_word0():
    for seed in (0, 1, 99, 2**63 + 1):
        assert oracle.rht_signs(seed) == int(oracle.philox(seed, [0, 0, 1, 0])[0]) & 0xFFFF


def test_sr_draws_look_uniform():
    u = oracle.sr_u16(1, np.arange(1 << 20, dtype=np.uint64))
    counts = np.bincount((u >> 12).astype(np.int64), minlength=16)
    exp = u.size / 16
    chi2 = ((counts - exp) ** 2 / exp).sum()
    assert chi2 < 50  # 15 dof; p ~ 1e-5
    assert abs(u.mean() - 32767.5) < 200
    # different seeds give different streams
    assert (oracle.sr_u16(2, np.arange(4096, dtype=np.uint64)) != u[:4096]).mean() > 0.99
