"""Pins for the oracle's block scorer, each independent of the oracle's own loop.

The score is sum_h w[q,h] * relu(q[q,h,:] . k[b,:]) (Strata pull #1091
'qsa_select: FP32 tiled block scores below sm_80', section What). Every pin
below would fail for a plausible slip in that loop: relu applied after the
head sum, w inside the relu, a swapped head/dim index, a wrong key row, a
missing factor.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def test_hand_example(oracle_lib):
    g = json.load(open(os.path.join(GOLDEN, "scores_hand.json")))
    q = np.zeros((g["nq"], g["heads"], g["head_dim"]), np.float32)
    k = np.zeros((g["n_blocks"], g["head_dim"]), np.float32)
    for a, h, d, v in g["q_entries"]:
        q[a, h, d] = v
    for b, d, v in g["k_entries"]:
        k[b, d] = v
    w = np.array(g["w"], np.float32)
    s = oracle_lib.block_scores(q, k, w)
    assert s.tolist() == g["scores"]


@pytest.mark.parametrize("heads", [1, 3, 8, 32])
def test_one_hot_keys_pick_a_coordinate(oracle_lib, heads):
    """k[b] = e_{d(b)}  =>  q.k = q[..., d(b)], so score = sum_h w relu(q[h, d(b)])."""
    rng = _rng(heads)
    nq, n_blocks, dim = 5, 300, 128
    q = rng.standard_normal((nq, heads, dim)).astype(np.float32)
    w = rng.uniform(-1, 1, (nq, heads)).astype(np.float32)  # negative weights too
    d_of_b = (np.arange(n_blocks) * 37 + 11) % dim
    k = np.zeros((n_blocks, dim), np.float32)
    k[np.arange(n_blocks), d_of_b] = 1.0
    s = oracle_lib.block_scores(q, k, w)
    picked = q[:, :, d_of_b].astype(np.float64)          # [nq, heads, n_blocks]
    expect = (w.astype(np.float64)[:, :, None] * np.maximum(picked, 0.0)).sum(axis=1)
    np.testing.assert_allclose(s, expect, rtol=1e-15, atol=1e-15)


def test_nonnegative_inputs_reduce_to_gemv(oracle_lib):
    """q, k >= 0 make every dot >= 0, so score[q] = (w[q] @ q[q]) @ k.T (numpy BLAS)."""
    rng = _rng(7)
    nq, heads, n_blocks = 4, 16, 500
    q = rng.random((nq, heads, 128)).astype(np.float32)
    k = rng.random((n_blocks, 128)).astype(np.float32)
    w = rng.random((nq, heads)).astype(np.float32)
    s = oracle_lib.block_scores(q, k, w)
    v = np.einsum("qh,qhd->qd", w.astype(np.float64), q.astype(np.float64))
    expect = v @ k.astype(np.float64).T
    np.testing.assert_allclose(s, expect, rtol=1e-13)


def test_all_negative_dots_give_exact_zero(oracle_lib):
    rng = _rng(3)
    q = rng.random((3, 8, 128)).astype(np.float32)
    k = -rng.random((64, 128)).astype(np.float32)
    w = rng.random((3, 8)).astype(np.float32)
    s = oracle_lib.block_scores(q, k, w)
    assert (s == 0.0).all()


def test_single_head_weight_isolates_that_head(oracle_lib):
    """w = e_h  =>  score = relu(q[h] . k[b]) for that head only."""
    rng = _rng(11)
    nq, heads, n_blocks = 2, 6, 200
    q = rng.standard_normal((nq, heads, 128)).astype(np.float32)
    k = rng.standard_normal((n_blocks, 128)).astype(np.float32)
    for h in range(heads):
        w = np.zeros((nq, heads), np.float32)
        w[:, h] = 1.0
        s = oracle_lib.block_scores(q, k, w)
        dots = np.array([[math.fsum(float(a) * float(b) for a, b in zip(q[i, h], k[j]))
                          for j in range(0, n_blocks, 17)] for i in range(nq)])
        np.testing.assert_allclose(s[:, ::17], np.maximum(dots, 0.0), rtol=1e-14, atol=1e-13)


def test_exact_rational_value(oracle_lib):
    """Against exact rational arithmetic on a small case (the double sums are ~1e-16 off)."""
    rng = _rng(5)
    nq, heads, n_blocks = 2, 3, 4
    q = rng.standard_normal((nq, heads, 128)).astype(np.float32)
    k = rng.standard_normal((n_blocks, 128)).astype(np.float32)
    w = rng.random((nq, heads)).astype(np.float32)
    s = oracle_lib.block_scores(q, k, w)
    for i in range(nq):
        for b in range(n_blocks):
            total = Fraction(0)
            scale = Fraction(0)
            for h in range(heads):
                dot = sum(Fraction(float(x)) * Fraction(float(y)) for x, y in zip(q[i, h], k[b]))
                total += Fraction(float(w[i, h])) * max(dot, Fraction(0))
                scale += abs(Fraction(float(w[i, h]))) * sum(
                    abs(Fraction(float(x)) * Fraction(float(y))) for x, y in zip(q[i, h], k[b]))
            assert abs(Fraction(s[i, b]) - total) <= scale * Fraction(1, 2 ** 50)


def test_mean_relu_matches_half_normal_closed_form(oracle_lib):
    """For k ~ N(0, I): q_h . k ~ N(0, |q_h|^2), so E relu(q_h . k) = |q_h| / sqrt(2 pi).

    Averaged over 65,536 synthetic key blocks the oracle must land within 3%
    (about 5 standard errors) of sum_h w_h |q_h| / sqrt(2 pi) for every query.
    """
    import synth
    nq, heads, n_blocks = 4, 16, 65536
    q = synth.normal("pin/mean/q", (nq, heads, 128))
    k = synth.normal("pin/mean/k", (n_blocks, 128))
    w = synth.uniform01("pin/mean/w", (nq, heads))
    s = oracle_lib.block_scores(q, k, w)
    norms = np.linalg.norm(q.astype(np.float64), axis=2)
    expect = (w.astype(np.float64) * norms).sum(axis=1) / math.sqrt(2 * math.pi)
    np.testing.assert_allclose(s.mean(axis=1), expect, rtol=0.03)


def test_scores_at_matches_full(oracle_lib):
    rng = _rng(9)
    q = rng.standard_normal((3, 5, 128)).astype(np.float32)
    k = rng.standard_normal((40, 128)).astype(np.float32)
    w = rng.random((3, 5)).astype(np.float32)
    full = oracle_lib.block_scores(q, k, w, ld=48)
    qi = np.array([0, 2, 1, 2], np.int32)
    bi = np.array([39, 0, 17, 5], np.int32)
    assert (oracle_lib.block_scores_at(q, k, w, qi, bi) == full[qi, bi]).all()
    assert (full[:, 40:] == 0).all()


def test_weights_enter_linearly(oracle_lib):
    rng = _rng(13)
    q = rng.standard_normal((2, 4, 128)).astype(np.float32)
    k = rng.standard_normal((30, 128)).astype(np.float32)
    w = rng.random((2, 4)).astype(np.float32)
    s1 = oracle_lib.block_scores(q, k, w)
    s2 = oracle_lib.block_scores(q, k, 2 * w)
    assert (s2 == 2 * s1).all()

