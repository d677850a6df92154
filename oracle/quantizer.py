"""Algorithm 1 (TurboQuant_mse), Algorithm 2 (TurboQuant_prod) and bit packing, in fp64.

Test infrastructure only (see the package docstring).

Pages followed:
* ai-navigate-news Gemma 4 post, section "仕組み（技術的）": Algorithm 1 rotates,
  scalar-quantizes every coordinate with the Lloyd-Max codebook of the
  Beta-shaped coordinate law and rotates back on decode; Algorithm 2 runs
  Algorithm 1 at b-1 bits and codes the residual r as sign(S r), which keeps
  inner products unbiased.  The same section stores indices and sign bits
  packed densely into bytes together with float16 norms and residual norms
  ("gammas") instead of int64 indices and float32 signs.
* techblog-plum explainer, section "TurboQuantの仕組み": the rotation is a
  random orthogonal matrix, decoding multiplies by its transpose.
* AIgent Lab explainer, section "視点1" (QJL): every residual value is reduced
  to one sign bit and a dedicated estimator removes the bias.

Readings where the pages are silent (each is also listed with the design notes):
* the input vector x is promoted exactly to fp64 (bf16/fp32 -> fp64);
* n = ||x||_2, y = Pi x, u = y / n (u = 0 when n = 0);
  idx_j = #{k in 1..L-1 : t_k < u_j}  -- a value on a boundary goes to the lower cell;
  evaluated as  t_k * n < y_j  for n > 0;
* n_hat = fp16(n), round-to-nearest-even, saturating at 65504;
* decode: x~ = n_hat * Pi^T c[idx];
* Algorithm 2 residual r = x - n_hat * Pi^T c[idx] (against what the decoder
  rebuilds); sign bit_i = 1 iff (S r)_i >= 0 (so -0 and +0 count as +1);
  gamma_hat = fp16(||r||);  S has d rows of iid N(0,1);
* Algorithm 2 decode: x~ = n_hat Pi^T c[idx] + sqrt(pi/2)/d * gamma_hat * S^T s,
  s_i = 2 bit_i - 1.  The constant is not printed on the pages: for g ~ N(0, I)
  and a unit vector v, E[sign(<g, v>) g] = sqrt(2/pi) v, so with d rows
  E[S^T sign(S r)] = d sqrt(2/pi) r/||r|| and the constant above makes the
  residual term unbiased for r;
* packing: a record is P planes of d bits (P = b for Algorithm 1; b-1 index
  planes then one sign plane for Algorithm 2), index planes LSB first; bit j
  of a plane sits in byte j//8 at bit j%8; planes are contiguous, so a record
  is P*d/8 bytes.  Norms and gammas are separate fp16 arrays.
"""
from __future__ import annotations

import math

import numpy as np

FP16_MAX = 65504.0


def qjl_scale(d: int) -> float:
    """sqrt(pi/2)/d: the unbiasing constant of the sign estimator with d Gaussian rows."""
    return math.sqrt(math.pi / 2.0) / d


def fp16_rne_sat(v) -> np.ndarray:
    """Round fp64 values to fp16 (nearest, ties to even), saturating at +-65504."""
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        h = v.astype(np.float16)  # numpy rounds float64 -> float16 directly, ties to even
    over = np.isinf(h) & np.isfinite(v)
    h[over] = np.copysign(np.float16(FP16_MAX), v[over]).astype(np.float16)
    return h


def _as64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def _norms_and_rotated(x, pi):
    x64 = _as64(x)
    n = np.sqrt(np.sum(x64 * x64, axis=1))
    y = x64 @ _as64(pi).T  # row i: Pi @ x_i
    return x64, n, y


def _indices(y, n, bounds):
    """idx_j = #{k : t_k < u_j}, u = y/n (u = 0 for the zero vector), as t_k*n < y_j."""
    t = _as64(bounds)
    nn = np.where(n > 0, n, 1.0)
    yy = np.where(n[:, None] > 0, y, 0.0)
    idx = np.zeros(yy.shape, dtype=np.int64)
    for tk in t:  # one comparison per boundary, counted
        idx += (tk * nn)[:, None] < yy
    return idx


def encode_mse(x, pi, centroids, bounds):
    """Algorithm 1 encode: returns (idx [n, d] int64, n_hat [n] float16)."""
    _, n, y = _norms_and_rotated(x, pi)
    idx = _indices(y, n, bounds)
    return idx, fp16_rne_sat(n)


def decode_mse(idx, n_hat, pi, centroids):
    """Algorithm 1 decode: n_hat * Pi^T c[idx] for every row, fp64 [n, d]."""
    c = _as64(centroids)[np.asarray(idx)]
    return (_as64(n_hat)[:, None] * c) @ _as64(pi)


def encode_prod(x, pi, s, centroids, bounds):
    """Algorithm 2 encode with an Algorithm-1 codebook of b-1 bits.

    Returns (idx [n, d], n_hat [n] f16, sign_bits [n, d] uint8, gamma_hat [n] f16).
    """
    x64, n, y = _norms_and_rotated(x, pi)
    idx = _indices(y, n, bounds)
    n_hat = fp16_rne_sat(n)
    r = x64 - decode_mse(idx, n_hat, pi, centroids)
    proj = r @ _as64(s).T  # row i: S @ r_i
    bits = (proj >= 0).astype(np.uint8)
    gamma = fp16_rne_sat(np.sqrt(np.sum(r * r, axis=1)))
    return idx, n_hat, bits, gamma


def decode_prod(idx, n_hat, sign_bits, gamma_hat, pi, s, centroids):
    """Algorithm 2 decode, fp64 [n, d]."""
    d = np.asarray(idx).shape[1]
    sgn = 2.0 * np.asarray(sign_bits, dtype=np.float64) - 1.0
    qjl = qjl_scale(d) * _as64(gamma_hat)[:, None] * (sgn @ _as64(s))
    return decode_mse(idx, n_hat, pi, centroids) + qjl


# --------------------------------------------------------------------------
# packing
# --------------------------------------------------------------------------


def pack_planes(planes) -> np.ndarray:
    """planes: list of [n, d] 0/1 arrays -> [n, P*d/8] uint8 record bytes."""
    out = [np.packbits(np.asarray(p, dtype=np.uint8), axis=1, bitorder="little") for p in planes]
    return np.ascontiguousarray(np.concatenate(out, axis=1))


def unpack_planes(codes, d: int, nplanes: int):
    codes = np.asarray(codes, dtype=np.uint8)
    w = d // 8
    return [np.unpackbits(codes[:, p * w:(p + 1) * w], axis=1, bitorder="little") for p in range(nplanes)]


def mse_record(idx, bits: int) -> np.ndarray:
    idx = np.asarray(idx)
    return pack_planes([(idx >> p) & 1 for p in range(bits)])


def prod_record(idx, sign_bits, bits: int) -> np.ndarray:
    """bits = total bits per coordinate (b): b-1 index planes, then the sign plane."""
    idx = np.asarray(idx)
    return pack_planes([(idx >> p) & 1 for p in range(bits - 1)] + [sign_bits])


def parse_mse_record(codes, d: int, bits: int):
    planes = unpack_planes(codes, d, bits)
    idx = np.zeros(planes[0].shape, dtype=np.int64)
    for p, pl in enumerate(planes):
        idx |= pl.astype(np.int64) << p
    return idx


def parse_prod_record(codes, d: int, bits: int):
    planes = unpack_planes(codes, d, bits)
    idx = np.zeros(planes[0].shape, dtype=np.int64)
    for p, pl in enumerate(planes[:-1]):
        idx |= pl.astype(np.int64) << p
    return idx, planes[-1]


def tile_records(codes, d: int, nplanes: int) -> np.ndarray:
    """Token-tiled layout of T row records: [ceil(T/32), nplanes, d] uint32.

    Word [k][p][j] has bit i equal to bit j of plane p of record 32k + i
    (zero past the last record).  The same bits as the rows, transposed per
    32-record tile.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    T = codes.shape[0]
    nt = (T + 31) // 32
    bits = np.zeros((nt * 32, nplanes, d), dtype=np.uint64)
    for p, pl in enumerate(unpack_planes(codes, d, nplanes)):
        bits[:T, p, :] = pl
    bits = bits.reshape(nt, 32, nplanes, d)
    words = np.zeros((nt, nplanes, d), dtype=np.uint64)
    for i in range(32):
        words |= bits[:, i] << np.uint64(i)
    return words.astype(np.uint32)


# --------------------------------------------------------------------------
# inner-product estimate (plain form: <q, decode(x)>)
# --------------------------------------------------------------------------


def inner_product_estimate(q, x_tilde):
    """<q_a, x~_i> for all pairs: [m, n] fp64."""
    return _as64(q) @ _as64(x_tilde).T


# --------------------------------------------------------------------------
# distance of each decision from its threshold (for tie-zone accounting)
# --------------------------------------------------------------------------


def code_margins(x, pi, bounds):
    """Per coordinate: min_k |y_j - t_k n| / sigma with sigma = n/sqrt(d) (inf for n = 0)."""
    _, n, y = _norms_and_rotated(x, pi)
    d = y.shape[1]
    t = _as64(bounds)
    if t.size == 0:  # a one-cell codebook (Algorithm 2 at b = 1) takes no index decision
        return np.full(y.shape, np.inf)
    dist = np.min(np.abs(y[:, :, None] - t[None, None, :] * n[:, None, None]), axis=2)
    sigma = n / math.sqrt(d)
    with np.errstate(divide="ignore", invalid="ignore"):
        m = dist / sigma[:, None]
    m[n == 0] = np.inf
    return m


def sign_margins(x, pi, s, centroids, bounds):
    """Per projected coordinate: |(S r)_i| / ||r|| (inf when r = 0)."""
    x64, n, y = _norms_and_rotated(x, pi)
    idx = _indices(y, n, bounds)
    r = x64 - decode_mse(idx, fp16_rne_sat(n), pi, centroids)
    proj = r @ _as64(s).T
    rn = np.sqrt(np.sum(r * r, axis=1))
    with np.errstate(divide="ignore", invalid="ignore"):
        m = np.abs(proj) / rn[:, None]
    m[rn == 0] = np.inf
    return m


def fp16_midpoint_margin(v) -> np.ndarray:
    """Relative distance of each positive value from the nearest fp16 rounding midpoint."""
    v = _as64(v)
    out = np.full(v.shape, np.inf)
    pos = (v > 0) & (v < FP16_MAX)
    e = np.floor(np.log2(v[pos]))
    ulp = np.exp2(np.maximum(e, -14.0) - 10.0)
    frac = v[pos] / ulp - np.floor(v[pos] / ulp)
    out[pos] = np.abs(frac - 0.5) * ulp / v[pos]
    return out
