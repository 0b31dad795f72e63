"""Pins of the oracle's Lightning Indexer scores (O1).

Checked against: a hand-worked example, exact rational arithmetic on tiny
inputs, integer matrix products in the exact regime E1, closed forms (one
head, zero weights) and exact symmetries (power-of-two scaling, weight sign).
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _val(code):
    """E4M3 code -> exact Fraction (written here from the format definition)."""
    code = int(code)
    s, e, m = code >> 7, (code >> 3) & 15, code & 7
    v = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -v if s else v


def _rand_codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3C      # no NaN codes
    return c


def test_worked_example(orc):
    kv = {}
    with open(os.path.join(GOLDEN, "indexer_worked_example.txt")) as f:
        for ln in f:
            if ln.strip() and not ln.startswith("#"):
                key, *vals = ln.split()
                kv[key] = vals
    q = np.array([int(c, 16) for c in kv["q_codes"]], np.uint8).reshape(1, 2, 2)
    k = np.array([int(c, 16) for c in kv["k_codes"]], np.uint8).reshape(1, 2)
    w = np.array([float(x) for x in kv["w"]], np.float32).reshape(1, 2)
    s = orc.indexer_scores(q, np.float32([kv["q_scale"][0]]), w, k, np.float32([kv["k_scale"][0]]),
                           np.int32([0]))
    assert s[0, 0] == np.float32(kv["score"][0])


def test_exact_rational_tiny(orc):
    rng = np.random.default_rng(21)
    n, h_i, d_i = 7, 3, 5
    q = _rand_codes(rng, (n, h_i, d_i))
    k = _rand_codes(rng, (n, d_i))
    qs = (rng.random(n) + 0.1).astype(np.float32)
    ks = (rng.random(n) + 0.1).astype(np.float32)
    w = rng.standard_normal((n, h_i)).astype(np.float32)
    pos = np.arange(n, dtype=np.int32)
    got = orc.indexer_scores(q, qs, w, k, ks, pos)
    for t in range(n):
        for s in range(n):
            if s > t:
                assert np.isnan(got[t, s])           # past the causal boundary: untouched
                continue
            acc = Fraction(0)
            for j in range(h_i):
                d = sum(_val(q[t, j, i]) * _val(k[s, i]) for i in range(d_i))
                if d > 0:
                    acc += Fraction(float(w[t, j])) * d
            exact = Fraction(float(qs[t])) * Fraction(float(ks[s])) * acc
            assert got[t, s] == np.float32(float(exact)), (t, s)


def test_exact_regime_integer_matmul(orc):
    """E1: integer codes, power-of-two scales, weights in (1/16)Z: every step is
    exact, so the score equals an integer computation bit for bit."""
    L, h_i, d_i = 96, 16, 64
    q = synth.e1_codes((L, h_i, d_i), 11).numpy()
    k = synth.e1_codes((L, d_i), 12).numpy()
    qs = synth.e1_pow2_scales(L, 13).numpy()
    ks = synth.e1_pow2_scales(L, 14).numpy()
    w = synth.e1_weights((L, h_i), 15).numpy()
    got = orc.indexer_scores(q, qs, w, k, ks, np.arange(L, dtype=np.int32))
    qi = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy().astype(np.int64)
    ki = torch.from_numpy(k).view(torch.float8_e4m3fn).to(torch.float64).numpy().astype(np.int64)
    w16 = (w * 16).astype(np.int64)
    D = np.einsum("tji,si->tjs", qi, ki)                       # integer dot products
    acc16 = np.einsum("tj,tjs->ts", w16, np.maximum(D, 0))      # sum_j (16 w_j) ReLU(D_j), integer
    ref = (acc16.astype(np.float64) / 16.0) * qs[:, None].astype(np.float64) * ks[None, :].astype(np.float64)
    mask = np.tril(np.ones((L, L), bool))
    assert np.abs(acc16).max() < 2 ** 24
    np.testing.assert_array_equal(got[mask], ref.astype(np.float32)[mask])


def test_single_head_unit_weights_is_relu_dot(orc):
    rng = np.random.default_rng(2)
    L, d_i = 40, 64
    q = _rand_codes(rng, (L, 1, d_i))
    k = _rand_codes(rng, (L, d_i))
    ones = np.ones(L, np.float32)
    got = orc.indexer_scores(q, ones, np.ones((L, 1), np.float32), k, ones, np.arange(L, dtype=np.int32))
    qv = torch.from_numpy(q[:, 0]).view(torch.float8_e4m3fn).double().numpy()
    kv = torch.from_numpy(k).view(torch.float8_e4m3fn).double().numpy()
    ref = np.maximum(qv @ kv.T, 0.0).astype(np.float32)
    mask = np.tril(np.ones((L, L), bool))
    np.testing.assert_array_equal(got[mask], ref[mask])


def test_zero_weights_give_zero(orc):
    rng = np.random.default_rng(3)
    L, h_i, d_i = 20, 4, 16
    q = _rand_codes(rng, (L, h_i, d_i))
    k = _rand_codes(rng, (L, d_i))
    got = orc.indexer_scores(q, np.ones(L, np.float32), np.zeros((L, h_i), np.float32), k,
                             np.ones(L, np.float32), np.arange(L, dtype=np.int32))
    assert (got[np.tril(np.ones((L, L), bool))] == 0).all()


def test_symmetries(orc):
    rng = np.random.default_rng(4)
    L, h_i, d_i = 32, 8, 32
    q = _rand_codes(rng, (L, h_i, d_i))
    k = _rand_codes(rng, (L, d_i))
    qs = (rng.random(L) + 0.5).astype(np.float32)
    ks = (rng.random(L) + 0.5).astype(np.float32)
    w = rng.standard_normal((L, h_i)).astype(np.float32)
    pos = np.arange(L, dtype=np.int32)
    m = np.tril(np.ones((L, L), bool))
    base = orc.indexer_scores(q, qs, w, k, ks, pos)
    twice = orc.indexer_scores(q, qs * 2, w, k, ks, pos)
    np.testing.assert_array_equal(twice[m], base[m] * 2)
    neg = orc.indexer_scores(q, qs, -w, k, ks, pos)
    np.testing.assert_array_equal(neg[m], -base[m])
    # a weight vector shared by all queries (w_ld = 0) equals that vector repeated
    shared = orc.indexer_scores(q, qs, w[0], k, ks, pos, w_shared=True)
    rep = orc.indexer_scores(q, qs, np.repeat(w[:1], L, 0), k, ks, pos)
    np.testing.assert_array_equal(shared[m], rep[m])


def test_multi_sequence_layout(orc):
    """Two sequences in one key array: each row only sees its own sequence."""
    rng = np.random.default_rng(5)
    h_i, d_i = 4, 16
    la, lb = 13, 21
    k = _rand_codes(rng, (la + lb, d_i))
    ks = (rng.random(la + lb) + 0.5).astype(np.float32)
    q = _rand_codes(rng, (2, h_i, d_i))
    qs = np.float32([1.5, 0.75])
    w = rng.standard_normal((2, h_i)).astype(np.float32)
    both = orc.indexer_scores(q, qs, w, k, ks, np.int32([la - 1, lb - 1]), seq_start=np.int64([0, la]),
                              q_seq=np.int32([0, 1]), ld=lb)
    a = orc.indexer_scores(q[:1], qs[:1], w[:1], k[:la], ks[:la], np.int32([la - 1]))
    b = orc.indexer_scores(q[1:], qs[1:], w[1:], k[la:], ks[la:], np.int32([lb - 1]))
    np.testing.assert_array_equal(both[0, :la], a[0])
    np.testing.assert_array_equal(both[1, :lb], b[0])
