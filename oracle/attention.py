"""Decode attention over a TurboQuant-compressed KV cache, in fp64.

Test infrastructure only (see the package docstring).

Page followed: ai-navigate-news Gemma 4 post, section "仕組み（技術的）": the key
cache uses Algorithm 1 (it minimises ||K - K_hat||^2, which is what the scores
Q K^T need) and the value cache uses Algorithm 2 (unbiased inner products,
which is what attn_weights . V needs).

Readings where the pages are silent: standard scaled dot-product attention for
one new query token per sequence; query head h reads KV head h // (Hq/Hkv)
(contiguous grouped-query groups); scores are <q, K~_t> * scale over
t < seq_len[b] with no other mask; softmax, then o = sum_t p_t V~_t.  K~ and
V~ are the decoded caches (Algorithm 1 and Algorithm 2 decodes).  Computed the
plain way: all scores, max, exp, normalise, weighted sum.
"""
from __future__ import annotations

import numpy as np


def decode_attention(q, k_tilde, v_tilde, seq_len, scale):
    """q [B, Hq, d]; k_tilde, v_tilde [B, Hkv, T, d]; seq_len [B] -> out [B, Hq, d] fp64."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = k_tilde.shape[1]
    group = Hq // Hkv
    out = np.zeros((B, Hq, d))
    for b in range(B):
        T = int(seq_len[b])
        if T == 0:
            continue
        for h in range(Hq):
            g = h // group
            K = np.asarray(k_tilde[b, g, :T], dtype=np.float64)
            V = np.asarray(v_tilde[b, g, :T], dtype=np.float64)
            s = (K @ q[b, h]) * scale
            p = np.exp(s - np.max(s))
            p /= np.sum(p)
            out[b, h] = p @ V
    return out
