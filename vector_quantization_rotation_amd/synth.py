"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module draws random numbers and nothing else: it holds none of the
quantizer's arithmetic (no codebooks, rotations applied to data, packing or
scoring).  Both the HIP path and the CPU oracle receive what it returns as
plain arrays, so the two sides never share code beyond these inputs.

Workload shapes follow the synthetic stand-ins for the pages' workloads: KV
caches with a few high-energy channels per head (the outlier problem described
in the techblog-plum explainer, section "これまでの量子化の限界"), heterogeneous
local/global layer shapes (ai-navigate-news Gemma 4 post, section
"KV形状の不均一性") and a clustered vector database for inner-product search
(AiBoss overview, section "TurboQuantの応用事例", vector-database search).
"""
from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------
# scalar format helpers (bit-level conversions only)
# --------------------------------------------------------------------------


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.ascontiguousarray(x, dtype=np.float32))
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 array whose values are exactly representable in bfloat16."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


# --------------------------------------------------------------------------
# random rotation / projection inputs (the method's random draws, passed in)
# --------------------------------------------------------------------------


def haar_rotation(d: int, seed: int) -> np.ndarray:
    """Random orthogonal d x d matrix (Haar measure), returned as float32.

    QR of a seeded Gaussian matrix with the signs of R's diagonal folded into Q.
    """
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((d, d))
    q, r = np.linalg.qr(g)
    q = q * np.sign(np.diag(r))[None, :]
    return np.ascontiguousarray(q.astype(np.float32))


def gaussian_projection(d: int, seed: int) -> np.ndarray:
    """d x d matrix of iid N(0,1) entries, float32 (the QJL projection S)."""
    rng = np.random.default_rng(seed)
    return np.ascontiguousarray(rng.standard_normal((d, d)).astype(np.float32))


# --------------------------------------------------------------------------
# data generators
# --------------------------------------------------------------------------


def unit_test_vectors(n: int, d: int, seed_dir: int, seed_norm: int) -> np.ndarray:
    """n float32 vectors: iid N(0,1) direction rescaled to a norm drawn from U[0.5, 2]."""
    g = np.random.default_rng(seed_dir).standard_normal((n, d))
    rho = np.random.default_rng(seed_norm).uniform(0.5, 2.0, size=n)
    x = g / np.linalg.norm(g, axis=1, keepdims=True) * rho[:, None]
    return np.ascontiguousarray(x.astype(np.float32))


def gaussian_queries(m: int, d: int, seed: int) -> np.ndarray:
    return np.ascontiguousarray(np.random.default_rng(seed).standard_normal((m, d)).astype(np.float32))


def outlier_channels(h: int, d: int, count: int, seed: int) -> np.ndarray:
    """[h, count] distinct channel indices per head (fixed across tokens)."""
    rng = np.random.default_rng(seed)
    return np.stack([np.sort(rng.choice(d, size=count, replace=False)) for _ in range(h)])


def kv_bf16(shape, seed: int, channels: np.ndarray | None = None, scale: float = 20.0,
            student_t_nu: float | None = None) -> np.ndarray:
    """KV tensor [B, H, T, d] of bf16 bits (uint16), iid N(0,1) except chosen channels.

    channels[h] lists the per-head outlier channels.  With student_t_nu None
    those channels are multiplied by `scale`; otherwise they are redrawn from
    a Student-t law with nu degrees of freedom (unscaled).
    """
    B, H, T, d = shape
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, H, T, d), dtype=np.float32)
    if channels is not None:
        for h in range(H):
            ch = channels[h]
            if student_t_nu is None:
                x[:, h, :, ch] *= np.float32(scale)
            else:
                x[:, h, :, ch] = rng.standard_t(student_t_nu, size=(B, T, len(ch))).astype(np.float32).transpose(0, 2, 1)
    return f32_to_bf16_bits(x).reshape(B, H, T, d)


def clustered_database(n: int, d: int, n_centers: int, sigma: float, seed_centers: int,
                       seed_assign: int, seed_noise: int, chunk: int = 65536) -> np.ndarray:
    """n float32 vectors x = center[a] + sigma*N(0,I), L2-normalised; centers iid N(0,1)."""
    centers = np.random.default_rng(seed_centers).standard_normal((n_centers, d)).astype(np.float32)
    assign = np.random.default_rng(seed_assign).integers(0, n_centers, size=n)
    rng = np.random.default_rng(seed_noise)
    out = np.empty((n, d), dtype=np.float32)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        v = centers[assign[s:e]] + np.float32(sigma) * rng.standard_normal((e - s, d), dtype=np.float32)
        v /= np.linalg.norm(v, axis=1, keepdims=True)
        out[s:e] = v
    return out


# --------------------------------------------------------------------------
# large device-side inputs (torch generator; for full-size benchmark shapes)
# --------------------------------------------------------------------------


def kv_bf16_torch(shape, seed: int, channels: np.ndarray | None, device, scale: float = 20.0,
                  student_t_nu: float | None = None):
    """Same law as kv_bf16 but drawn with torch's generator on `device` (bf16 tensor).

    Used where the host generator would take minutes (gigabyte caches); the
    oracle then checks sampled slices copied back from the device.
    """
    import torch
    B, H, T, d = shape
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.empty((B, H, T, d), dtype=torch.bfloat16, device=device)
    for b in range(B):  # one batch row at a time keeps the fp32 temporary small
        xb = torch.randn((H, T, d), generator=g, device=device, dtype=torch.float32)
        if channels is not None:
            for h in range(H):
                ch = torch.as_tensor(channels[h], device=device, dtype=torch.long)
                if student_t_nu is None:
                    xb[h][:, ch] *= scale
                else:
                    # Student-t with integer nu: z / sqrt(chi2_nu / nu), chi2_nu a sum of nu squares
                    nu = int(student_t_nu)
                    z = torch.randn((T, len(ch)), generator=g, device=device, dtype=torch.float32)
                    w = torch.randn((nu, T, len(ch)), generator=g, device=device, dtype=torch.float32)
                    v = (w * w).sum(0)
                    xb[h][:, ch] = z / torch.sqrt(v / nu)
        x[b] = xb.to(torch.bfloat16)
    return x


def clustered_database_torch(n: int, d: int, n_centers: int, sigma: float, seed_centers: int, seed_assign: int,
                             seed_noise: int, device, chunk: int = 65536):
    """Same law as clustered_database (the same centres, drawn on the host) with the assignments and
    noise drawn by torch's generator on `device`: an [n, d] fp32 tensor."""
    import torch
    centers = torch.from_numpy(np.random.default_rng(seed_centers).standard_normal((n_centers, d)).astype(np.float32))
    centers = centers.to(device)
    g = torch.Generator(device=device)
    g.manual_seed(seed_assign)
    assign = torch.randint(0, n_centers, (n,), generator=g, device=device)
    g.manual_seed(seed_noise)
    out = torch.empty((n, d), dtype=torch.float32, device=device)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        v = centers[assign[s:e]] + sigma * torch.randn((e - s, d), generator=g, device=device, dtype=torch.float32)
        out[s:e] = v / torch.linalg.vector_norm(v, dim=1, keepdim=True)
    return out
