"""Pins for the oracle's decode attention and search top-k.

Attention is pinned by special cases with closed-form answers (one token,
equal scores, a dominant score, the grouped-query head map, empty sequence)
and by rescaling invariance; search by hand-made tie cases and a brute-force
Python ordering on tiny inputs.
"""
import numpy as np
import pytest

import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_single_token_returns_its_value():
    B, Hq, Hkv, T, d = 2, 4, 2, 3, 8
    q, K, V = _rand((B, Hq, d), 1), _rand((B, Hkv, T, d), 2), _rand((B, Hkv, T, d), 3)
    out = oracle.decode_attention(q, K, V, np.array([1, 1]), 0.3)
    for b in range(B):
        for h in range(Hq):
            assert np.allclose(out[b, h], V[b, h // 2, 0], rtol=0, atol=1e-15)


def test_equal_scores_give_mean_value():
    B, Hq, Hkv, T, d = 1, 2, 1, 7, 8
    q = _rand((B, Hq, d), 1)
    K = np.repeat(_rand((B, Hkv, 1, d), 2), T, axis=2)
    V = _rand((B, Hkv, T, d), 3)
    out = oracle.decode_attention(q, K, V, np.array([T]), 1.0)
    assert np.allclose(out[0, 0], V[0, 0].mean(axis=0), atol=1e-14)
    assert np.allclose(out[0, 1], V[0, 0].mean(axis=0), atol=1e-14)


def test_dominant_score_and_seq_len_mask():
    B, Hq, Hkv, T, d = 1, 1, 1, 6, 4
    q = np.array([[[1.0, 0, 0, 0]]])
    K = np.zeros((B, Hkv, T, d))
    K[0, 0, 2, 0] = 100.0       # score 100 * scale at t = 2
    K[0, 0, 5, 0] = 1000.0      # beyond seq_len: must be ignored
    V = _rand((B, Hkv, T, d), 4)
    out = oracle.decode_attention(q, K, V, np.array([5]), 1.0)
    assert np.allclose(out[0, 0], V[0, 0, 2], atol=1e-12)


def test_two_token_closed_form():
    # p_1 = 1 / (1 + exp(-(s_1 - s_0)))
    q = np.array([[[2.0, 0.0]]])
    K = np.array([[[[0.5, 1.0], [1.0, -3.0]]]])
    V = np.array([[[[1.0, 0.0], [0.0, 1.0]]]])
    scale = 0.7
    s0, s1 = 2 * 0.5 * scale, 2 * 1.0 * scale
    p1 = 1 / (1 + np.exp(-(s1 - s0)))
    out = oracle.decode_attention(q, K, V, np.array([2]), scale)
    assert np.allclose(out[0, 0], [1 - p1, p1], atol=1e-15)


def test_empty_sequence_gives_zero():
    out = oracle.decode_attention(_rand((1, 2, 4), 1), _rand((1, 1, 3, 4), 2), _rand((1, 1, 3, 4), 3), np.array([0]), 1.0)
    assert np.all(out == 0)


def test_shift_invariance_of_scores():
    # adding the query direction to every key shifts all scores equally: output unchanged
    B, Hq, Hkv, T, d = 1, 1, 1, 9, 6
    q, K, V = _rand((B, Hq, d), 5), _rand((B, Hkv, T, d), 6), _rand((B, Hkv, T, d), 7)
    o1 = oracle.decode_attention(q, K, V, np.array([T]), 0.5)
    o2 = oracle.decode_attention(q, K + 3.0 * q[:, :, None, :], V, np.array([T]), 0.5)
    assert np.allclose(o1, o2, atol=1e-13)


def test_topk_ties_and_bruteforce():
    s = np.array([[1.0, 3.0, 3.0, 2.0, 3.0]])
    idx, val = oracle.topk_desc(s, 3)
    assert idx.tolist() == [[1, 2, 4]] and val.tolist() == [[3.0, 3.0, 3.0]]
    rng = np.random.default_rng(3)
    s = rng.integers(0, 5, size=(6, 40)).astype(float)   # many ties
    idx, _ = oracle.topk_desc(s, 7)
    for i in range(6):
        brute = sorted(range(40), key=lambda j: (-s[i, j], j))[:7]
        assert idx[i].tolist() == brute


def test_recall():
    assert oracle.recall_at_k(np.array([[1, 2, 3], [4, 5, 6]]), np.array([[3, 2, 9], [7, 8, 9]])) == pytest.approx(2 / 6)
