"""Inner-product search over TurboQuant codes, in fp64.

Test infrastructure only (see the package docstring).

Pages followed: AiBoss overview, section "TurboQuantの応用事例" (vector-database
search as a replacement for product quantization) and AIgent Lab explainer,
section "視点3" (recall@k against product quantization).

Readings: a database row's score for query q is the estimate <q, x~_i> with
x~_i the Algorithm 2 decode; top-k is by descending score with ties broken
toward the lower row index; recall@k = |top-k(estimate) intersect
top-k(exact)| / k averaged over queries, exact = fp64 <q, x_i>.
"""
from __future__ import annotations

import numpy as np


def score_all(queries, x_tilde):
    return np.asarray(queries, dtype=np.float64) @ np.asarray(x_tilde, dtype=np.float64).T


def topk_desc(scores, k: int):
    """Per row: indices and values of the k largest scores, ties -> lower index."""
    scores = np.asarray(scores, dtype=np.float64)
    m, n = scores.shape
    k = min(k, n)
    order = np.lexsort((np.broadcast_to(np.arange(n), (m, n)), -scores), axis=1)[:, :k]
    return order, np.take_along_axis(scores, order, axis=1)


def recall_at_k(found, exact) -> float:
    found = np.asarray(found)
    exact = np.asarray(exact)
    k = exact.shape[1]
    hits = [len(set(found[i].tolist()) & set(exact[i].tolist())) for i in range(exact.shape[0])]
    return float(np.mean(hits)) / k
