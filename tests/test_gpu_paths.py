"""HIP paths outside the headline shapes, against the CPU oracle through the C ABI (needs an MI355X).

* decode through the GEMM loader (head dims above 128), both algorithms;
* scoring through the dequantizing GEMM and the top-k kernel (4-bit Algorithm-1 records);
* encode of coordinates placed exactly on, and one or two fp32 ulps around, a codebook boundary
  (t_k * ||x||) and on zero, with an identity and a Haar rotation: every decision outside the tie zone
  (|y_j - t_k n| <= 1e-5 n / sqrt(d)) must match the oracle bit for bit;
* norms that saturate fp16 (||x|| >= 65520 rounds to the largest fp16, 65504) and norms in the fp16
  subnormal range, for both algorithms.
"""
import math

import numpy as np
import pytest

import oracle
from tests import parity
from vector_quantization_rotation_amd import synth

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def api():
    from vector_quantization_rotation_amd import api as _api
    _api.load()
    return _api


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("mode,d,bits", [("prod", 256, 3), ("prod", 512, 2), ("prod", 1536, 4), ("mse", 256, 3),
                                         ("mse", 1536, 2)])
def test_decode_gemm_path(api, mode, d, bits):
    n = 300
    x = synth.unit_test_vectors(n, d, 61, 62)
    pi, s = synth.haar_rotation(d, 63), synth.gaussian_projection(d, 64)
    prod = mode == "prod"
    print(f"decode {mode} d={d} b={bits} n={n}", flush=True)
    qz = api.Quantizer(d, bits, api.TQ_PROD if prod else api.TQ_MSE, pi, s if prod else None)
    if prod:
        e = parity.oracle_prod(x, pi, s, bits)
        ref = oracle.decode_prod(e["idx"], e["n_hat"], e["signs"], e["gamma"], pi, s, e["c"])
        gam = _dev(parity.f16_bits(e["gamma"]))
    else:
        e = parity.oracle_mse(x, pi, bits)
        ref = oracle.decode_mse(e["idx"], e["n_hat"], pi, e["c"])
        gam = None
    out = qz.decode(_dev(e["record"]), _dev(parity.f16_bits(e["n_hat"])), gam).cpu().numpy()
    err = parity.rel_rows(out, ref)
    print(f"decode {mode} d={d} b={bits}: max rel err {err.max():.2e}")
    assert np.all(err <= parity.RTOL), err.max()


@pytest.mark.parametrize("k", [0, 10])
@pytest.mark.parametrize("d", [128, 256])
def test_score_gemm_fallback_mse4(api, d, k):
    """4-bit Algorithm-1 records are scored by the dequantizing GEMM (and ranked by the top-k kernel)."""
    n, m = 3000, 21
    x = synth.unit_test_vectors(n, d, 71, 72)
    pi = synth.haar_rotation(d, 73)
    q = synth.gaussian_queries(m, d, 74)
    print(f"score mse 4-bit d={d} k={k}", flush=True)
    qz = api.Quantizer(d, 4, api.TQ_MSE, pi)
    e = parity.oracle_mse(x, pi, 4)
    xt = oracle.decode_mse(e["idx"], e["n_hat"], pi, e["c"])
    ref = oracle.inner_product_estimate(q, xt)
    res = qz.score(_dev(q), _dev(e["record"]), _dev(parity.f16_bits(e["n_hat"])), None, k=k)
    if k == 0:
        tol = parity.RTOL * np.linalg.norm(q, axis=1)[:, None] * np.linalg.norm(xt, axis=1)[None, :]
        assert np.all(np.abs(res.cpu().numpy() - ref) <= tol)
        return
    vals, idx = res[0].cpu().numpy(), res[1].cpu().numpy()
    tol = parity.RTOL * np.linalg.norm(q, axis=1) * np.max(np.linalg.norm(xt, axis=1))
    ref_idx, ref_vals = oracle.topk_desc(ref, k)
    for i in range(m):
        assert len(set(idx[i].tolist())) == k
        assert np.all(np.diff(vals[i]) <= 0)
        assert np.all(np.abs(vals[i] - ref_vals[i]) <= tol[i])
        assert np.all(np.abs(ref[i, idx[i]] - ref_vals[i]) <= 2 * tol[i])
        # no row outside the returned set beats the tenth score by more than the gate
        assert np.max(np.delete(ref[i], idx[i])) <= vals[i, -1] + 2 * tol[i]


def _boundary_rows(d, t, rng, n_rows):
    """Rotated rows y whose coordinates sit exactly on t_k * ||y||, one or two fp32 ulps to either side,
    or on zero, mixed with N(0, 1/d) filler.  The norm is fixed first (the filler is rescaled so that
    ||y|| is the chosen value in fp64), then the boundary coordinates are placed against it."""
    ys = []
    for r in range(n_rows):
        nrm = float(rng.uniform(0.5, 2.0))
        y = rng.standard_normal(d) / math.sqrt(d)
        nb = d // 4
        pos = rng.choice(d, size=nb, replace=False)
        k = rng.integers(0, len(t), size=nb)
        vals = np.asarray(t)[k] * nrm
        off = rng.integers(-2, 3, size=nb)
        vals = np.array([np.nextafter(np.float32(v), np.float32(np.inf if o > 0 else -np.inf)) if o else np.float32(v)
                         for v, o in zip(vals, off)], dtype=np.float64)
        for j in np.nonzero(off == 2)[0]:
            vals[j] = float(np.nextafter(np.float32(vals[j]), np.float32(np.inf)))
        for j in np.nonzero(off == -2)[0]:
            vals[j] = float(np.nextafter(np.float32(vals[j]), np.float32(-np.inf)))
        zero = rng.choice(np.setdiff1d(np.arange(d), pos), size=4, replace=False)
        rest = np.setdiff1d(np.arange(d), np.concatenate([pos, zero]))
        y[zero] = 0.0
        y[pos] = vals
        fill = nrm * nrm - float(np.sum(vals.astype(np.float64) ** 2))
        y[rest] *= math.sqrt(max(fill, 1e-6) / float(np.sum(y[rest] ** 2)))
        ys.append(y)
    return np.array(ys, dtype=np.float32)


@pytest.mark.parametrize("rot", ["identity", "haar"])
@pytest.mark.parametrize("mode,bits", [("mse", 3), ("mse", 2), ("mse", 4), ("prod", 3), ("prod", 4)])
def test_encode_boundary_exact_coordinates(api, rot, mode, bits):
    d, n = 128, 512
    rng = np.random.default_rng(81)
    prod = mode == "prod"
    c, t = oracle.lloyd_max(d, bits - 1 if prod else bits)
    pi = np.eye(d, dtype=np.float32) if rot == "identity" else synth.haar_rotation(d, 82)
    s = synth.gaussian_projection(d, 83)
    y = _boundary_rows(d, t, rng, n)
    # x = Pi^T y in fp32 (an identity rotation keeps y exactly; a Haar one puts y within rounding of it)
    x = y if rot == "identity" else (y.astype(np.float64) @ pi.astype(np.float64)).astype(np.float32)
    print(f"boundary encode rot={rot} {mode} b={bits}", flush=True)
    qz = api.Quantizer(d, bits, api.TQ_PROD if prod else api.TQ_MSE, pi, s if prod else None)
    codes, norms, gammas = qz.encode(_dev(x))
    codes = codes.cpu().numpy()
    margins = oracle.code_margins(x, pi, t)
    # a quarter of the coordinates sit in the tie zone by construction, so the fraction cap of the
    # workloads' inputs does not apply; every differing decision must still lie in the tie zone
    if prod:
        enc = parity.oracle_prod(x, pi, s, bits)
        idx, sb = oracle.parse_prod_record(codes, d, bits)
        nbad, nties = parity.check_codes(idx, enc["idx"], margins, max_frac=None)
        parity.check_prod_signs(sb, idx, enc, x, pi, s, max_frac=None)
    else:
        enc = parity.oracle_mse(x, pi, bits)
        idx = oracle.parse_mse_record(codes, d, bits)
        nbad, nties = parity.check_codes(idx, enc["idx"], margins, max_frac=None)
    assert parity.check_norms(norms.cpu().numpy(), x) == 0
    print(f"boundary encode rot={rot} {mode} b={bits}: {nties} tie-zone coordinates, {nbad} differ")
    if rot == "identity":
        # with an exact rotation a zero coordinate is exactly on the middle boundary: index L/2 - 1
        # (the lower cell) on both sides
        L = 1 << (bits - 1 if prod else bits)
        assert np.all(idx[x == 0] == L // 2 - 1) and np.all(enc["idx"][x == 0] == L // 2 - 1)
        assert nties >= 4 * n


@pytest.mark.parametrize("xdtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode,bits", [("mse", 3), ("prod", 3)])
def test_encode_norm_saturation_and_subnormal(api, xdtype, mode, bits):
    d = 128
    rho = np.array([65519.0, 65520.0, 70000.0, 1.0e6, 3.0e7, 6.0e-5, 1.0e-5, 3.0e-6, 1.0e-7, 5.0e-8, 2.0e-8, 1.0])
    rng = np.random.default_rng(91)
    u = rng.standard_normal((len(rho) * 8, d))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    x = (u * np.repeat(rho, 8)[:, None]).astype(np.float32)
    if xdtype == "bf16":
        x = synth.round_bf16(x)
    pi, s = synth.haar_rotation(d, 92), synth.gaussian_projection(d, 93)
    prod = mode == "prod"
    print(f"norm extremes {mode} b={bits} {xdtype}", flush=True)
    qz = api.Quantizer(d, bits, api.TQ_PROD if prod else api.TQ_MSE, pi, s if prod else None)
    xt = _dev(x) if xdtype == "f32" else _dev(x).to(torch.bfloat16)
    codes, norms, gammas = qz.encode(xt)
    codes = codes.cpu().numpy()
    nb = norms.cpu().numpy()
    assert parity.check_norms(nb, x) == 0
    nh = parity.f16_from_bits(nb)
    nx = np.linalg.norm(x.astype(np.float64), axis=1)  # the norms of the rows as given (bf16 rounding moves them)
    assert np.any(nx >= 65520) and np.all(nh[nx >= 65520] == np.float16(65504))
    assert np.any((nx > 0) & (nx < 6.1e-5)) and np.all(nh[(nx > 0) & (nx < 6.1e-5)] < np.float16(6.104e-5))
    if prod:
        enc = parity.oracle_prod(x, pi, s, bits)
        idx, sb = oracle.parse_prod_record(codes, d, bits)
        parity.check_codes(idx, enc["idx"], oracle.code_margins(x, pi, enc["t"]))
        _, _, same = parity.check_prod_signs(sb, idx, enc, x, pi, s)
        rn = np.linalg.norm(parity.residual_given_index(x, enc["idx"], enc["n_hat"], pi, enc["c"]), axis=1)
        parity.check_gammas(gammas.cpu().numpy()[same], rn[same])
    else:
        enc = parity.oracle_mse(x, pi, bits)
        idx = oracle.parse_mse_record(codes, d, bits)
        parity.check_codes(idx, enc["idx"], oracle.code_margins(x, pi, enc["t"]))
