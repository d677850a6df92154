"""HIP path vs the CPU oracle through the C ABI (unit-test sizes; needs an MI355X).

Inputs are the seeded synthetic vectors of the unit-test workload (4096 x 128
fp32, random norms in [0.5, 2], Haar Pi, Gaussian S, 64 Gaussian queries),
plus ragged and degenerate shapes.
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


def _unit_inputs(n=4096, d=128):
    x = synth.unit_test_vectors(n, d, 101, 102)
    pi = synth.haar_rotation(d, 111)
    s = synth.gaussian_projection(d, 112)
    q = synth.gaussian_queries(64, d, 103)
    return x, pi, s, q


def _dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t if dtype is None else t.to(dtype)


def _idx_of(codes, d, bits, mode_prod):
    c = codes.cpu().numpy()
    if mode_prod:
        return oracle.parse_prod_record(c, d, bits)
    return oracle.parse_mse_record(c, d, bits), None


@pytest.mark.parametrize("n,d,bits", [(4096, 128, 2), (4096, 128, 3), (1000, 64, 1), (333, 256, 4), (130, 512, 3)])
def test_encode_mse_parity(api, n, d, bits):
    x, pi, _, _ = _unit_inputs(n, d) if d == 128 else (synth.unit_test_vectors(n, d, 7, 8), synth.haar_rotation(d, 9), None, None)
    qz = api.Quantizer(d, bits, api.TQ_MSE, pi)
    codes, norms, _ = qz.encode(_dev(x))
    torch.cuda.synchronize()
    c, t = oracle.lloyd_max(d, bits)
    idx_ref, _ = oracle.encode_mse(x, pi, c, t)
    idx, _ = _idx_of(codes, d, bits, False)
    nbad, nties = parity.check_codes(idx, idx_ref, oracle.code_margins(x, pi, t))
    assert parity.check_norms(norms.cpu().numpy(), x) == 0
    # records are byte-identical wherever no tie-zone decision differs
    rec_ref = oracle.mse_record(idx_ref, bits)
    same_rows = np.all(idx == idx_ref, axis=1)
    assert np.array_equal(codes.cpu().numpy()[same_rows], rec_ref[same_rows])
    print(f"mse d={d} b={bits}: mismatches {nbad}, tie-zone coords {nties}")


@pytest.mark.parametrize("n,d,bits", [(4096, 128, 3), (4096, 128, 2), (257, 256, 4), (130, 512, 3)])
def test_encode_prod_parity(api, n, d, bits):
    if d == 128:
        x, pi, s, _ = _unit_inputs(n, d)
    else:
        x, pi, s = synth.unit_test_vectors(n, d, 17, 18), synth.haar_rotation(d, 19), synth.gaussian_projection(d, 20)
    qz = api.Quantizer(d, bits, api.TQ_PROD, pi, s)
    codes, norms, gammas = qz.encode(_dev(x))
    torch.cuda.synchronize()
    c, t = oracle.lloyd_max(d, bits - 1)
    idx_ref, nh_ref, sb_ref, g_ref = oracle.encode_prod(x, pi, s, c, t)
    idx, sb = _idx_of(codes, d, bits, True)
    parity.check_codes(idx, idx_ref, oracle.code_margins(x, pi, t))
    assert parity.check_norms(norms.cpu().numpy(), x) == 0
    # sign bits: against the oracle residual built from the GPU's own indices
    r = parity.residual_given_index(x, idx, nh_ref, pi, c)
    proj = r @ s.astype(np.float64).T
    sb_ref2 = (proj >= 0).astype(np.uint8)
    rn = np.linalg.norm(r, axis=1)
    margins = np.abs(proj) / np.maximum(rn, 1e-300)[:, None]
    nbad, nties = parity.check_codes(sb, sb_ref2, margins, "sign")
    parity.check_gammas(gammas.cpu().numpy(), rn)
    print(f"prod d={d} b={bits}: sign mismatches {nbad}, tie-zone signs {nties}")


@pytest.mark.parametrize("mode,bits", [("mse", 2), ("prod", 3), ("mse", 4), ("prod", 2)])
def test_decode_parity(api, mode, bits):
    x, pi, s, _ = _unit_inputs()
    d = 128
    prod = mode == "prod"
    qz = api.Quantizer(d, bits, api.TQ_PROD if prod else api.TQ_MSE, pi, s if prod else None)
    codes, norms, gammas = qz.encode(_dev(x))
    out = qz.decode(codes, norms, gammas).cpu().numpy()
    c, _ = oracle.lloyd_max(d, bits - 1 if prod else bits)
    nh = parity.f16_from_bits(norms.cpu().numpy())
    if prod:
        idx, sb = _idx_of(codes, d, bits, True)
        ref = oracle.decode_prod(idx, nh, sb, parity.f16_from_bits(gammas.cpu().numpy()), pi, s, c)
    else:
        idx, _ = _idx_of(codes, d, bits, False)
        ref = oracle.decode_mse(idx, nh, pi, c)
    err = parity.rel_rows(out, ref)
    assert np.all(err <= parity.RTOL), err.max()
    assert err.max() < 1e-5  # fp32 contraction: far inside the gate


@pytest.mark.parametrize("mode,bits", [("mse", 2), ("prod", 3)])
def test_score_parity_all_pairs(api, mode, bits):
    x, pi, s, q = _unit_inputs()
    d = 128
    prod = mode == "prod"
    qz = api.Quantizer(d, bits, api.TQ_PROD if prod else api.TQ_MSE, pi, s if prod else None)
    codes, norms, gammas = qz.encode(_dev(x))
    sc = qz.score(_dev(q), codes, norms, gammas).cpu().numpy()
    c, _ = oracle.lloyd_max(d, bits - 1 if prod else bits)
    nh = parity.f16_from_bits(norms.cpu().numpy())
    if prod:
        idx, sb = _idx_of(codes, d, bits, True)
        xt = oracle.decode_prod(idx, nh, sb, parity.f16_from_bits(gammas.cpu().numpy()), pi, s, c)
    else:
        idx, _ = _idx_of(codes, d, bits, False)
        xt = oracle.decode_mse(idx, nh, pi, c)
    ref = oracle.inner_product_estimate(q, xt)
    tol = parity.RTOL * np.linalg.norm(q, axis=1)[:, None] * np.linalg.norm(xt, axis=1)[None, :]
    assert np.all(np.abs(sc - ref) <= tol)
    # the estimate tracks the exact inner product (report; prod is unbiased)
    exact = q.astype(np.float64) @ x.astype(np.float64).T
    print(mode, "mean est - exact:", float(np.mean(ref - exact)), "rms:", float(np.sqrt(np.mean((ref - exact) ** 2))))


@pytest.mark.parametrize("n,k", [(4096, 10), (1000, 1), (70, 64), (5000, 17)])
def test_score_topk(api, n, k):
    d = 128
    x = synth.unit_test_vectors(n, d, 31, 32)
    pi, s = synth.haar_rotation(d, 33), synth.gaussian_projection(d, 34)
    q = synth.gaussian_queries(37, d, 35)
    qz = api.Quantizer(d, 3, api.TQ_PROD, pi, s)
    codes, norms, gammas = qz.encode(_dev(x))
    full = qz.score(_dev(q), codes, norms, gammas).cpu().numpy()
    vals, idx = qz.score(_dev(q), codes, norms, gammas, k=k)
    vals, idx = vals.cpu().numpy(), idx.cpu().numpy()
    ref_idx, ref_vals = oracle.topk_desc(full, k)  # selection over the GPU's own scores: exact
    assert np.array_equal(idx, ref_idx)
    assert np.array_equal(vals, ref_vals.astype(np.float32))


def test_score_topk_ties_to_lower_index(api):
    d = 64
    pi, s = synth.haar_rotation(d, 1), synth.gaussian_projection(d, 2)
    base = synth.unit_test_vectors(5, d, 3, 4)
    x = np.repeat(base, 40, axis=0)  # identical records -> identical scores
    qz = api.Quantizer(d, 2, api.TQ_PROD, pi, s)
    codes, norms, gammas = qz.encode(_dev(x))
    q = synth.gaussian_queries(3, d, 5)
    full = qz.score(_dev(q), codes, norms, gammas).cpu().numpy()
    _, idx = qz.score(_dev(q), codes, norms, gammas, k=50)
    ref_idx, _ = oracle.topk_desc(full, 50)
    assert np.array_equal(idx.cpu().numpy(), ref_idx)


def _attn_case(api, B, Hq, Hkv, T, d, seq, qdtype, seed=0, layout=0, kbits=3, vbits=2):
    rng = np.random.default_rng(seed)
    chans = synth.outlier_channels(Hkv, d, 4, seed + 1)
    K = synth.bf16_bits_to_f32(synth.kv_bf16((B, Hkv, T, d), seed + 2, chans))
    V = synth.bf16_bits_to_f32(synth.kv_bf16((B, Hkv, T, d), seed + 3, chans))
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    if qdtype == "bf16":
        q = synth.round_bf16(q)
    piK, piV, sV = synth.haar_rotation(d, seed + 4), synth.haar_rotation(d, seed + 5), synth.gaussian_projection(d, seed + 6)
    kq = api.Quantizer(d, kbits, api.TQ_MSE, piK)
    vq = api.Quantizer(d, vbits, api.TQ_PROD, piV, sV)
    kc, kn, _ = kq.encode(_dev(K.reshape(-1, d)))
    vc, vn, vg = vq.encode(_dev(V.reshape(-1, d)))
    qt = _dev(q) if qdtype == "f32" else _dev(q).to(torch.bfloat16)
    seq_t = torch.tensor(seq, dtype=torch.int32, device="cuda")
    vsrc = vc.view(B, Hkv, T, -1)
    if layout == api.TQ_LAYOUT_TILE32:
        vsrc = api.tile_records(vq, vc.view(B * Hkv, T, -1)).view(B, Hkv, -1, vq.planes, d)
    out = api.attn_decode(kq, vq, qt, kc.view(B, Hkv, T, -1), kn.view(B, Hkv, T), vsrc,
                          vn.view(B, Hkv, T), vg.view(B, Hkv, T), seq_t, 1.0 / math.sqrt(d), vlayout=layout).cpu().numpy()
    cK, _ = oracle.lloyd_max(d, kbits)
    cV, _ = oracle.lloyd_max(d, vbits - 1)
    kidx = oracle.parse_mse_record(kc.cpu().numpy(), d, kbits)
    vidx, vsb = oracle.parse_prod_record(vc.cpu().numpy(), d, vbits)
    Kt = oracle.decode_mse(kidx, parity.f16_from_bits(kn.cpu().numpy()), piK, cK).reshape(B, Hkv, T, d)
    Vt = oracle.decode_prod(vidx, parity.f16_from_bits(vn.cpu().numpy()), vsb, parity.f16_from_bits(vg.cpu().numpy()),
                            piV, sV, cV).reshape(B, Hkv, T, d)
    ref = oracle.decode_attention(q, Kt, Vt, np.array(seq), 1.0 / math.sqrt(d))
    return out, ref


@pytest.mark.parametrize("B,Hq,Hkv,T,seq", [(2, 8, 2, 300, [300, 137]), (1, 4, 4, 64, [1]), (3, 32, 8, 520, [520, 0, 33])])
def test_attn_decode_parity(api, B, Hq, Hkv, T, seq):
    out, ref = _attn_case(api, B, Hq, Hkv, T, 128, seq, "bf16")
    for b in range(B):
        if seq[b] == 0:
            assert np.all(out[b] == 0)
            continue
        err = parity.rel_rows(out[b], ref[b])
        assert np.all(err <= parity.RTOL), (b, err.max())


ATTN_FAST_CASES = [
    # (B, Hq, Hkv, T, seq, d, kbits, vbits)
    (2, 8, 2, 300, [300, 137], 128, 3, 2),
    (1, 4, 4, 64, [1], 128, 3, 2),
    (3, 32, 8, 520, [520, 0, 33], 128, 3, 2),
    (2, 16, 2, 1100, [1100, 700], 128, 3, 2),   # 8 heads per kv head: two head groups
    (1, 6, 2, 777, [777], 128, 3, 2),           # 3 heads per kv head: partial head group
    (2, 8, 4, 513, [513, 256], 128, 2, 3),
    (1, 4, 1, 400, [399], 128, 4, 2),
    (1, 4, 1, 333, [333], 128, 1, 2),
    (2, 32, 16, 1024, [1024, 1000], 256, 3, 2),  # local-layer shape
    (1, 8, 2, 20000, [19999], 128, 3, 2),        # long sequence: many steps per work-group
    (1, 4, 4, 64, [2], 128, 3, 2),               # the largest weight maps to the top int8 digit
    (2, 8, 8, 64, [1, 1], 128, 3, 2),            # one token: output is that token's value
]


@pytest.mark.parametrize("B,Hq,Hkv,T,seq,d,kb,vb", ATTN_FAST_CASES)
def test_attn_decode_tiled_parity(api, B, Hq, Hkv, T, seq, d, kb, vb):
    out, ref = _attn_case(api, B, Hq, Hkv, T, d, seq, "bf16", seed=5, layout=api.TQ_LAYOUT_TILE32, kbits=kb, vbits=vb)
    for b in range(B):
        if seq[b] == 0:
            assert np.all(out[b] == 0)
            continue
        err = parity.rel_rows(out[b], ref[b])
        assert np.all(err <= parity.RTOL), (b, err.max())
        print(f"tiled attention case b={b}: max rel err {err.max():.2e}")


def test_tile_records_matches_oracle(api):
    d, T = 128, 100
    x = synth.unit_test_vectors(3 * T, d, 51, 52)
    vq = api.Quantizer(d, 2, api.TQ_PROD, synth.haar_rotation(d, 53), synth.gaussian_projection(d, 54))
    codes, _, _ = vq.encode(_dev(x))
    tiles = api.tile_records(vq, codes.view(3, T, -1)).cpu().numpy().view(np.uint32)
    c = codes.cpu().numpy().reshape(3, T, -1)
    for sq in range(3):
        assert np.array_equal(tiles[sq], oracle.tile_records(c[sq], d, 2))


def test_encode_zero_and_empty(api):
    d = 128
    pi, s = synth.haar_rotation(d, 1), synth.gaussian_projection(d, 2)
    x = np.zeros((3, d), dtype=np.float32)
    qm = api.Quantizer(d, 3, api.TQ_MSE, pi)
    codes, norms, _ = qm.encode(_dev(x))
    idx, _ = _idx_of(codes, d, 3, False)
    assert np.all(idx == 3) and np.all(norms.cpu().numpy() == 0)
    qp = api.Quantizer(d, 3, api.TQ_PROD, pi, s)
    codes, norms, gammas = qp.encode(_dev(x))
    idx, sb = _idx_of(codes, d, 3, True)
    assert np.all(idx == 1) and np.all(sb == 1) and np.all(gammas.cpu().numpy() == 0)
    e = torch.empty((0, d), device="cuda")
    codes, norms, _ = qm.encode(e)
    assert codes.shape == (0, qm.code_bytes)


def test_bf16_and_f16_inputs_match_f32(api):
    d = 128
    x = synth.round_bf16(synth.unit_test_vectors(512, d, 41, 42))
    pi = synth.haar_rotation(d, 43)
    qz = api.Quantizer(d, 3, api.TQ_MSE, pi)
    c32, n32, _ = qz.encode(_dev(x))
    cbf, nbf, _ = qz.encode(_dev(x).to(torch.bfloat16))
    assert torch.equal(c32, cbf) and torch.equal(n32, nbf)
    x16 = x.astype(np.float16).astype(np.float32)
    c32, n32, _ = qz.encode(_dev(x16))
    c16, n16, _ = qz.encode(_dev(x16).to(torch.float16))
    assert torch.equal(c32, c16) and torch.equal(n32, n16)
