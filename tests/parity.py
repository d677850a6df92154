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


def check_codes(idx_gpu, idx_ref, margins, what="index", max_frac=1e-4):
    """Return (mismatches, ties); assert every mismatch is a tie-zone decision and, for inputs drawn
    from the workloads' laws (max_frac not None), that mismatches stay below max_frac of all codes.
    Inputs built to crowd the tie zone pass max_frac=None."""
    bad = idx_gpu != idx_ref
    ties = margins <= TIE
    n_bad = int(bad.sum())
    assert not np.any(bad & ~ties), (
        f"{what}: {int((bad & ~ties).sum())} mismatches outside the tie zone "
        f"(min margin {float(np.min(margins[bad])):.3g})")
    if max_frac is not None:
        assert n_bad <= max_frac * idx_ref.size, f"{what}: {n_bad} mismatches of {idx_ref.size}"
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


def f16_bits(v) -> np.ndarray:
    """fp16 values -> their int16 bit patterns (the library's norm/gamma storage)."""
    return np.ascontiguousarray(np.asarray(v, dtype=np.float16)).view(np.int16)


def oracle_mse(x, pi, bits):
    """The oracle's Algorithm-1 encoding of x: dict with idx, n_hat (f16), record (u8), centroids, bounds."""
    d = np.asarray(x).shape[1]
    c, t = oracle.lloyd_max(d, bits)
    idx, nh = oracle.encode_mse(x, pi, c, t)
    return dict(idx=idx, n_hat=nh, record=oracle.mse_record(idx, bits), c=c, t=t)


def oracle_prod(x, pi, s, bits):
    """The oracle's Algorithm-2 encoding of x (b-1 index bits + sign plane)."""
    d = np.asarray(x).shape[1]
    c, t = oracle.lloyd_max(d, bits - 1)
    idx, nh, sb, gh = oracle.encode_prod(x, pi, s, c, t)
    return dict(idx=idx, n_hat=nh, signs=sb, gamma=gh, record=oracle.prod_record(idx, sb, bits), c=c, t=t)


def untile(tiles, T, nplanes, d):
    """Token-tiled words [ceil(T/32), P, d] (bit i of word = token 32k+i) -> row records [T, P*d/8]."""
    w = np.asarray(tiles).view(np.uint32).astype(np.uint64)
    nt = w.shape[0]
    bits = ((w[..., None] >> np.arange(32, dtype=np.uint64)) & np.uint64(1)).astype(np.uint8)  # [nt, P, d, 32]
    bits = bits.transpose(0, 3, 1, 2).reshape(nt * 32, nplanes, d)[:T]
    return np.packbits(bits, axis=2, bitorder="little").reshape(T, nplanes * d // 8)


def check_prod_signs(sb_gpu, idx_gpu, enc, x, pi, s, max_frac=1e-4):
    """Sign bits vs the oracle's, on rows whose index decisions all agree (elsewhere the residual differs)."""
    same = np.all(idx_gpu == enc["idx"], axis=1)
    margins = oracle.sign_margins(x, pi, s, enc["c"], enc["t"])
    nbad, nties = check_codes(sb_gpu[same], enc["signs"][same], margins[same], "sign", max_frac)
    return nbad, nties, same


def install_oracle_slice(cache, b, g, K, V, kbits=3, vbits=2):
    """Encode the raw rows of (batch b, kv-head g) with the oracle and write the oracle's records,
    norms, gammas and token-tiled value words into that slice of a device cache (an AttnCache).

    The attention of that slice then runs on exactly the oracle's codes, so its output can be
    held to the attention tolerance (a code decision inside the tie zone may move a heavily
    weighted token's score, which no fixed tolerance on the output covers)."""
    import torch
    d = K.shape[1]
    ke = oracle_mse(K, cache.piK, kbits)
    ve = oracle_prod(V, cache.piV, cache.sV, vbits)
    dev = cache.kcodes.device

    def put(dst, arr):
        dst.copy_(torch.from_numpy(np.ascontiguousarray(arr)).to(dev).view(dst.shape))

    put(cache.kcodes[b, g], ke["record"])
    put(cache.knorms[b, g], f16_bits(ke["n_hat"]))
    put(cache.vcodes[b, g], ve["record"])
    put(cache.vnorms[b, g], f16_bits(ve["n_hat"]))
    put(cache.vgammas[b, g], f16_bits(ve["gamma"]))
    if cache.vtiles.shape[2] > 0:  # caches read through row records carry no tiles
        put(cache.vtiles[b, g], oracle.tile_records(ve["record"], d, vbits).view(np.int32))
    return ke, ve
