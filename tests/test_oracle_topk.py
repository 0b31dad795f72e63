"""Pins of the oracle's top-k selection (O2): numpy's stable argsort, closed
forms, the dense degeneration (k >= candidates keeps everything) and the
tie / signed-zero rule."""
import numpy as np
import pytest


def _ref_argsort(row, k):
    r = row.astype(np.float32) + np.float32(0.0)      # -0 -> +0
    order = np.argsort(-r, kind="stable")              # descending score, ascending index on ties
    sel = np.sort(order[:k]).astype(np.int32)
    return np.concatenate([sel, -np.ones(k - len(sel), np.int32)])


def test_matches_stable_argsort(orc):
    rng = np.random.default_rng(9)
    n, ld, k = 64, 300, 37
    s = rng.standard_normal((n, ld)).astype(np.float32)
    s[:, ::5] = np.round(s[:, ::5] * 4) / 4          # many exact ties
    s[3, :50] = -0.0
    s[4, :50] = 0.0
    pos = rng.integers(0, ld, size=n).astype(np.int32)
    pos[:3] = [0, k - 1, k]
    got = orc.topk(s, pos, k)
    for t in range(n):
        np.testing.assert_array_equal(got[t], _ref_argsort(s[t, :pos[t] + 1], k))


def test_closed_forms(orc):
    k, L = 8, 40
    pos = np.full(3, L - 1, np.int32)
    s = np.zeros((3, L), np.float32)
    s[1] = np.arange(L)                # increasing in s -> the last k
    s[2] = -np.arange(L)               # decreasing -> the first k
    got = orc.topk(s, pos, k)
    np.testing.assert_array_equal(got[0], np.arange(k))          # all equal -> lowest indices
    np.testing.assert_array_equal(got[1], np.arange(L - k, L))
    np.testing.assert_array_equal(got[2], np.arange(k))


def test_dense_degeneration(orc):
    """Fewer candidates than k: every candidate is kept, ascending, -1 padded."""
    k = 16
    s = np.random.default_rng(1).standard_normal((5, 20)).astype(np.float32)
    pos = np.int32([0, 3, 14, 15, 19])
    got = orc.topk(s, pos, k)
    for t, p in enumerate(pos):
        m = min(k, p + 1)
        if p + 1 <= k:
            np.testing.assert_array_equal(got[t, :m], np.arange(p + 1))
        assert (got[t, m:] == -1).all()
        assert (np.diff(got[t, :m]) > 0).all()


def test_signed_zero_ties(orc):
    s = np.array([[-0.0, 0.0, -0.0, 0.0, -1.0]], np.float32)
    got = orc.topk(s, np.int32([4]), 3)
    np.testing.assert_array_equal(got[0], [0, 1, 2])


def test_nan_rejected(orc):
    s = np.array([[1.0, np.nan, 2.0]], np.float32)
    with pytest.raises(ValueError):
        orc.topk(s, np.int32([2]), 1)
    # NaN past the causal boundary is never read
    orc.topk(s, np.int32([0]), 1)
