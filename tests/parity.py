"""Comparison helpers for HIP-vs-oracle parity (test code; uses only the oracle).

Tolerances (the readings stated with the design notes):
* codes and sign bits: bit-exact, except decisions within the tie zone --
  |y_j - t_k n| <= 1e-5 sigma (sigma = n/sqrt(d)) for index bits and
  |(S r)_i| <= 1e-5 ||r|| for sign bits; every mismatch must lie in the tie
  zone and mismatches must stay below 1e-4 of all codes;
* fp16 norms: bit-exact (both sides round an fp64 norm) unless the norm lies
  within 1e-9 (relative) of an fp16 rounding midpoint;
* fp16 gammas: within one fp16 ulp, and any difference must come from a
  residual norm within 1e-5 (relative) of a midpoint;
* reconstructions and attention outputs: ||delta|| <= 2e-3 ||ref|| per vector;
* scores: |delta| <= 2e-3 ||q|| ||x~|| per pair.
"""
from __future__ import annotations

import numpy as np

import oracle

TIE = 1e-5
RTOL = 2e-3


def f16_from_bits(t) -> np.ndarray:
    return np.asarray(t, dtype=np.int16).view(np.float16)


def check_codes(idx_gpu, idx_ref, margins, what="index"):
    """Return (mismatches, ties); assert every mismatch is a tie-zone decision."""
    bad = idx_gpu != idx_ref
    ties = margins <= TIE
    n_bad = int(bad.sum())
    assert not np.any(bad & ~ties), (
        f"{what}: {int((bad & ~ties).sum())} mismatches outside the tie zone "
        f"(min margin {float(np.min(margins[bad])):.3g})")
    assert n_bad <= 1e-4 * idx_ref.size, f"{what}: {n_bad} mismatches of {idx_ref.size}"
    return n_bad, int(ties.sum())


def check_norms(nh_gpu_bits, x):
    n = np.sqrt(np.sum(np.asarray(x, dtype=np.float64) ** 2, axis=1))
    ref = oracle.fp16_rne_sat(n)
    got = f16_from_bits(nh_gpu_bits)
    bad = got != ref
    assert not np.any(bad & (oracle.fp16_midpoint_margin(n) > 1e-9)), "norm rounding mismatch"
    return int(bad.sum())


def check_gammas(g_gpu_bits, g_ref_exact):
    """g_ref_exact: fp64 residual norms from the oracle."""
    ref = oracle.fp16_rne_sat(g_ref_exact)
    got = f16_from_bits(g_gpu_bits)
    bad = got != ref
    if np.any(bad):
        ulp = np.abs(got[bad].astype(np.float64) - ref[bad].astype(np.float64))
        spacing = np.spacing(np.maximum(np.abs(ref[bad]), np.abs(got[bad])).astype(np.float16)).astype(np.float64)
        assert np.all(ulp <= spacing * 1.0001), "gamma differs by more than one fp16 ulp"
        assert np.all(oracle.fp16_midpoint_margin(g_ref_exact[bad]) <= TIE), "gamma mismatch outside tie zone"
    return int(bad.sum())


def rel_rows(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.linalg.norm(got - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    return num / np.maximum(den, 1e-300)


def residual_given_index(x, idx, nhat, pi, centroids):
    """Oracle residual r = x - n_hat Pi^T c[idx] for a given index array."""
    return np.asarray(x, dtype=np.float64) - oracle.decode_mse(idx, nhat, pi, centroids)
