"""Pins of the oracle's calibration sums (oracle/wushkv_ref.py: calib_stats) against
what the mathematics fixes: a hand-worked rank-one case, brute-force loops, the trace
identity, symmetry and positive semi-definiteness, additivity over heads and batch rows,
and invariance under reordering the rows."""
import numpy as np
import pytest

from oracle import wushkv_ref as R


def _brute(x, group):
    B, H, T, d = x.shape
    out = [[[0.0] * d for _ in range(d)] for _ in range(H // group)]
    for g in range(H // group):
        for b in range(B):
            for h in range(g * group, (g + 1) * group):
                for t in range(T):
                    for i in range(d):
                        for j in range(d):
                            out[g][i][j] += float(x[b, h, t, i]) * float(x[b, h, t, j])
    return np.array(out)


def test_rank_one_by_hand():
    x = np.array([1.0, -2.0, 3.0, 0.5]).reshape(1, 1, 1, 4)
    want = np.array([[1.0, -2.0, 3.0, 0.5],
                     [-2.0, 4.0, -6.0, -1.0],
                     [3.0, -6.0, 9.0, 1.5],
                     [0.5, -1.0, 1.5, 0.25]])
    assert np.array_equal(R.calib_stats(x)[0], want)


@pytest.mark.parametrize("shape,group", [((2, 4, 3, 5), 2), ((1, 3, 4, 6), 1), ((3, 2, 2, 4), 2)])
def test_brute_force_loops(shape, group):
    x = np.random.default_rng(7).standard_normal(shape)
    np.testing.assert_allclose(R.calib_stats(x, group), _brute(x, group), rtol=1e-12, atol=1e-12)


def test_trace_symmetry_psd():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((3, 4, 50, 16)) * rng.uniform(0.1, 10, size=16)
    s = R.calib_stats(x, 2)
    for g in range(2):
        rows = x[:, 2 * g:2 * g + 2].reshape(-1, 16)
        assert np.isclose(np.trace(s[g]), np.sum(rows * rows), rtol=1e-12)
        assert np.array_equal(s[g], s[g].T)
        assert np.linalg.eigvalsh(s[g]).min() > -1e-9 * np.trace(s[g])


def test_additive_over_heads_and_rows():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((4, 6, 7, 8))
    per_head = R.calib_stats(x, 1)
    grouped = R.calib_stats(x, 3)
    np.testing.assert_allclose(grouped[0], per_head[0:3].sum(0), rtol=1e-12)
    np.testing.assert_allclose(grouped[1], per_head[3:6].sum(0), rtol=1e-12)
    halves = R.calib_stats(x[:2], 3) + R.calib_stats(x[2:], 3)
    np.testing.assert_allclose(grouped, halves, rtol=1e-12)


def test_row_order_does_not_matter():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((2, 2, 9, 5))
    perm = rng.permutation(9)
    np.testing.assert_allclose(R.calib_stats(x[:, :, perm], 2), R.calib_stats(x, 2), rtol=1e-12)


def test_sum_abs_bounds_the_sum():
    x = np.random.default_rng(11).standard_normal((2, 2, 6, 4))
    assert np.all(np.abs(R.calib_stats(x, 2)) <= R.calib_sum_abs(x, 2) + 1e-12)
