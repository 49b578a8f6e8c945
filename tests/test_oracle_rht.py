"""Pins for the oracle's 16-point random Hadamard transform (CPU only).

References independent of the oracle: scipy's Sylvester Hadamard matrix in
float64, orthogonality (norm preservation, inverse), exactness on inputs whose
partial sums are representable, and the summation error bound of a depth-4
addition tree.
"""
import numpy as np
import pytest
from scipy.linalg import hadamard

import oracle

H16 = hadamard(16).astype(np.float64)
U = 2.0 ** -24
GAMMA4 = 4 * U / (1 - 4 * U)


def _signs_vec(seed):
    s = oracle.rht_signs(seed)
    return np.array([-1.0 if (s >> j) & 1 else 1.0 for j in range(16)])


def test_hadamard_reference_is_orthogonal():
    assert np.array_equal(H16 @ H16.T, 16 * np.eye(16))


@pytest.mark.parametrize("seed", [0, 1, 7, 2**40 + 3])
def test_unit_vectors_give_scaled_hadamard_columns(seed):
    d = _signs_vec(seed)
    for k in range(16):
        a = np.zeros(16, dtype=np.float32)
        a[k] = 1.0
        y = oracle.rht16(a, seed)
        assert np.array_equal(y.astype(np.float64), 0.25 * H16[:, k] * d[k])


@pytest.mark.parametrize("seed", [0, 5, 123456789])
def test_matches_float64_definition_within_tree_bound(seed):
    d = _signs_vec(seed)
    rng = np.random.default_rng(seed)
    for trial in range(2000):
        scale = np.exp2(rng.uniform(-30, 30, 16))
        a = (rng.standard_normal(16) * scale).astype(np.float32)
        y = oracle.rht16(a, seed).astype(np.float64)
        ref = 0.25 * H16 @ (d * a.astype(np.float64))
        bound = 0.25 * GAMMA4 * np.abs(a.astype(np.float64)).sum() + 4 * 2.0 ** -149
        assert (np.abs(y - ref) <= bound).all(), trial


def test_exact_on_small_integers():
    rng = np.random.default_rng(2)
    d = _signs_vec(3)
    for _ in range(500):
        a = rng.integers(-2**16, 2**16, 16).astype(np.float32)
        y = oracle.rht16(a, 3).astype(np.float64)
        assert np.array_equal(y, 0.25 * H16 @ (d * a.astype(np.float64)))


def test_norm_preserved_and_inverse():
    rng = np.random.default_rng(4)
    for seed in (0, 9):
        for _ in range(500):
            a = rng.standard_normal(16).astype(np.float32)
            y = oracle.rht16(a, seed)
            n_a = np.linalg.norm(a.astype(np.float64))
            assert abs(np.linalg.norm(y.astype(np.float64)) - n_a) <= 4 * GAMMA4 * n_a
            back = oracle.rht16(y, seed, inverse=True).astype(np.float64)
            bound = 2 * GAMMA4 * np.abs(a.astype(np.float64)).sum() + 1e-44
            assert (np.abs(back - a) <= bound).all()


def test_tensor_rht_applies_per_group_along_axis():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((32, 48)).astype(np.float32)
    d = _signs_vec(11)
    y_row = oracle.rht(x, "row", 11)
    ref = (0.25 * (x.reshape(32, 3, 16).astype(np.float64) * d) @ H16.T).reshape(32, 48)
    assert np.abs(y_row - ref).max() <= 1e-5 * np.abs(x).max()
    y_col = oracle.rht(x, "col", 11)
    y_col_t = oracle.rht(np.ascontiguousarray(x.T), "row", 11)
    assert np.array_equal(y_col, y_col_t.T)
    back = oracle.rht(y_row, "row", 11, inverse=True)
    assert np.abs(back - x).max() <= 1e-5 * np.abs(x).max()


def test_signs_differ_between_seeds():
    s = {oracle.rht_signs(k) for k in range(64)}
    assert len(s) > 60
