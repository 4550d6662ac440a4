"""Pins of the float64 decode-attention oracle (oracle.attn_decode) against
closed forms of softmax attention.

[MTPLX pull request #267, "feat(kv-cache): add q6 paged KV quantization",
 PR description: dequantized cache rows feed scaled-dot-product attention]
"""
import math

import numpy as np
import pytest

import oracle


def _h(a):
    return np.asarray(a, np.float16).view(np.uint16)


def test_equal_keys_give_the_mean_of_values():
    rng = np.random.default_rng(1)
    q = _h(rng.standard_normal(64))
    k = _h(np.tile(rng.standard_normal(64), (9, 1)))
    vf = rng.standard_normal((9, 64)).astype(np.float16)
    out = oracle.attn_decode(q, k, _h(vf), 0.125)
    assert np.allclose(out, vf.astype(np.float64).mean(axis=0), rtol=0, atol=1e-15)


def test_two_positions_logistic_weight():
    """scores s0, s1: the weight of position 1 is 1 / (1 + exp(s0 - s1))."""
    q = _h([1.0, 0.0, 0.0, 0.0])
    k = _h([[0.5, 0, 0, 0], [2.0, 0, 0, 0]])
    v = _h([[1.0, -2.0, 0, 4], [3.0, 0.5, 1, 0]])
    scale = 0.75
    w1 = 1.0 / (1.0 + math.exp(scale * (0.5 - 2.0)))
    exp = (1 - w1) * np.array([1.0, -2.0, 0, 4]) + w1 * np.array([3.0, 0.5, 1, 0])
    assert np.allclose(oracle.attn_decode(q, k, v, scale), exp, rtol=0, atol=1e-15)


def test_dominant_score_selects_its_value_row():
    q = _h([8.0] * 16)
    k = np.zeros((5, 16), np.float16)
    k[3] = 4.0                      # score 512 * scale vs 0
    v = np.random.default_rng(2).standard_normal((5, 16)).astype(np.float16)
    out = oracle.attn_decode(q, _h(k), _h(v), 1.0)
    assert np.array_equal(out, v[3].astype(np.float64))


def test_permutation_and_shift_invariance():
    rng = np.random.default_rng(3)
    T, D = 37, 32
    q = rng.standard_normal(D).astype(np.float16)
    k = rng.standard_normal((T, D)).astype(np.float16)
    v = rng.standard_normal((T, D)).astype(np.float16)
    base = oracle.attn_decode(_h(q), _h(k), _h(v), 0.2)
    perm = rng.permutation(T)
    assert np.allclose(oracle.attn_decode(_h(q), _h(k[perm]), _h(v[perm]), 0.2), base, rtol=0, atol=1e-14)
    # a component with q_d = 1 and the same k_d for every row adds one constant to every score
    q2, k2 = q.copy(), k.copy()
    q2[0], k2[:, 0] = 1.0, 3.0
    q3, k3 = q2.copy(), k2.copy()
    k3[:, 0] = -5.0
    assert np.allclose(oracle.attn_decode(_h(q2), _h(k2), _h(v), 0.2),
                       oracle.attn_decode(_h(q3), _h(k3), _h(v), 0.2), rtol=0, atol=1e-14)


def test_no_rows_gives_zero():
    assert not oracle.attn_decode(_h(np.ones(8)), np.zeros((0, 8), np.uint16), np.zeros((0, 8), np.uint16), 1.0).any()
