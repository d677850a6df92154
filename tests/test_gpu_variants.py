"""Bit-width and mode variants on the GPU against the CPU oracle (needs an MI355X).

* Algorithm 2 at b = 1, the pure sign (QJL) mode of the AiBoss overview (section
  "TurboQuantの主な機能"): encode, decode and inner-product scores;
* decode attention with Algorithm-2 keys (unbiased scores) at 1-3 bits, and with 1-bit values,
  on the row-record layout.
Inputs are the unit-test law (random directions, norms in [0.5, 2]) and the KV law with outlier
channels; the oracle encodes the raw rows for every consumer test.
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


@pytest.mark.parametrize("d,xdtype", [(128, "f32"), (256, "bf16"), (64, "f32")])
def test_one_bit_prod_encode(api, d, xdtype):
    n = 1000
    x = synth.unit_test_vectors(n, d, 401, 402)
    if xdtype == "bf16":
        x = synth.round_bf16(x)
    pi, s = synth.haar_rotation(d, 403), synth.gaussian_projection(d, 404)
    print(f"1-bit prod encode d={d} {xdtype}", flush=True)
    qz = api.Quantizer(d, 1, api.TQ_PROD, pi, s)
    assert qz.planes == 1 and qz.code_bytes == d // 8
    xt = _dev(x) if xdtype == "f32" else _dev(x).to(torch.bfloat16)
    codes, norms, gammas = qz.encode(xt)
    enc = parity.oracle_prod(x, pi, s, 1)
    idx, sb = oracle.parse_prod_record(codes.cpu().numpy(), d, 1)
    assert np.all(idx == 0)
    nbad, nties, same = parity.check_prod_signs(sb, idx, enc, x, pi, s)
    assert np.all(same)
    assert parity.check_norms(norms.cpu().numpy(), x) == 0
    parity.check_gammas(gammas.cpu().numpy(), np.linalg.norm(x.astype(np.float64), axis=1))
    rows = np.all(sb == enc["signs"], axis=1)
    assert np.array_equal(codes.cpu().numpy()[rows], enc["record"][rows])
    print(f"1-bit prod d={d}: sign mismatches {nbad}, tie-zone signs {nties}")


@pytest.mark.parametrize("d", [128, 256])
def test_one_bit_prod_decode_and_score(api, d):
    n, m = 2000, 17
    x = synth.unit_test_vectors(n, d, 411, 412)
    pi, s = synth.haar_rotation(d, 413), synth.gaussian_projection(d, 414)
    q = synth.gaussian_queries(m, d, 415)
    print(f"1-bit prod decode/score d={d}", flush=True)
    qz = api.Quantizer(d, 1, api.TQ_PROD, pi, s)
    enc = parity.oracle_prod(x, pi, s, 1)
    xt = oracle.decode_prod(enc["idx"], enc["n_hat"], enc["signs"], enc["gamma"], pi, s, enc["c"])
    codes, norms, gam = _dev(enc["record"]), _dev(parity.f16_bits(enc["n_hat"])), _dev(parity.f16_bits(enc["gamma"]))
    out = qz.decode(codes, norms, gam).cpu().numpy()
    err = parity.rel_rows(out, xt)
    assert np.all(err <= parity.RTOL), err.max()
    ref = oracle.inner_product_estimate(q, xt)
    sc = qz.score(_dev(q), codes, norms, gam).cpu().numpy()
    tol = parity.RTOL * np.linalg.norm(q, axis=1)[:, None] * np.linalg.norm(xt, axis=1)[None, :]
    assert np.all(np.abs(sc - ref) <= tol)
    vals, idx = qz.score(_dev(q), codes, norms, gam, k=10)
    vals, idx = vals.cpu().numpy(), idx.cpu().numpy()
    ref_idx, ref_vals = oracle.topk_desc(ref, 10)
    tk = parity.RTOL * np.linalg.norm(q, axis=1) * np.max(np.linalg.norm(xt, axis=1))
    for i in range(m):
        assert len(set(idx[i].tolist())) == 10
        assert np.all(np.abs(vals[i] - ref_vals[i]) <= tk[i])
        assert np.max(np.delete(ref[i], idx[i])) <= vals[i, -1] + 2 * tk[i]


ATTN_VARIANTS = [
    # (d, key mode, key bits, value bits, B, Hq, Hkv, T, seq)
    (128, "prod", 3, 2, 2, 8, 2, 700, [700, 311]),
    (128, "prod", 2, 3, 1, 8, 1, 400, [399]),
    (128, "prod", 1, 2, 2, 4, 2, 300, [300, 5]),      # pure sign keys
    (128, "mse", 3, 1, 2, 8, 2, 500, [500, 77]),      # pure sign values
    (256, "prod", 3, 1, 1, 16, 4, 260, [260]),        # both variants at head dim 256
    (64, "prod", 4, 2, 2, 6, 3, 200, [200, 0]),
]


@pytest.mark.parametrize("d,kmode,kb,vb,B,Hq,Hkv,T,seq", ATTN_VARIANTS)
def test_attn_decode_mode_variants(api, d, kmode, kb, vb, B, Hq, Hkv, T, seq):
    rng = np.random.default_rng(421)
    chans = synth.outlier_channels(Hkv, d, 4, 422)
    K = synth.bf16_bits_to_f32(synth.kv_bf16((B, Hkv, T, d), 423, chans)).reshape(-1, d)
    V = synth.bf16_bits_to_f32(synth.kv_bf16((B, Hkv, T, d), 424, chans)).reshape(-1, d)
    piK, sK = synth.haar_rotation(d, 425), synth.gaussian_projection(d, 426)
    piV, sV = synth.haar_rotation(d, 427), synth.gaussian_projection(d, 428)
    q = synth.round_bf16(rng.standard_normal((B, Hq, d)).astype(np.float32))
    kprod = kmode == "prod"
    print(f"attention variant d={d} keys {kmode} {kb}-bit, values prod {vb}-bit, B={B} Hq={Hq} Hkv={Hkv} T={T}",
          flush=True)
    kq = api.Quantizer(d, kb, api.TQ_PROD if kprod else api.TQ_MSE, piK, sK if kprod else None)
    vq = api.Quantizer(d, vb, api.TQ_PROD, piV, sV)
    if kprod:
        ke = parity.oracle_prod(K, piK, sK, kb)
        Kt = oracle.decode_prod(ke["idx"], ke["n_hat"], ke["signs"], ke["gamma"], piK, sK, ke["c"])
        kg = _dev(parity.f16_bits(ke["gamma"])).view(B, Hkv, T)
    else:
        ke = parity.oracle_mse(K, piK, kb)
        Kt = oracle.decode_mse(ke["idx"], ke["n_hat"], piK, ke["c"])
        kg = None
    ve = parity.oracle_prod(V, piV, sV, vb)
    Vt = oracle.decode_prod(ve["idx"], ve["n_hat"], ve["signs"], ve["gamma"], piV, sV, ve["c"])
    ref = oracle.decode_attention(q, Kt.reshape(B, Hkv, T, d), Vt.reshape(B, Hkv, T, d), np.array(seq),
                                  1.0 / math.sqrt(d))
    out = api.attn_decode(kq, vq, _dev(q).to(torch.bfloat16), _dev(ke["record"]).view(B, Hkv, T, -1),
                          _dev(parity.f16_bits(ke["n_hat"])).view(B, Hkv, T), _dev(ve["record"]).view(B, Hkv, T, -1),
                          _dev(parity.f16_bits(ve["n_hat"])).view(B, Hkv, T),
                          _dev(parity.f16_bits(ve["gamma"])).view(B, Hkv, T),
                          torch.tensor(seq, dtype=torch.int32, device="cuda"), 1.0 / math.sqrt(d),
                          kgammas=kg).cpu().numpy()
    for b in range(B):
        if seq[b] == 0:
            assert np.all(out[b] == 0)
            continue
        err = parity.rel_rows(out[b], ref[b])
        print(f"  b={b}: max rel err {err.max():.2e}")
        assert np.all(err <= parity.RTOL), (b, err.max())


def test_tiled_layout_rejects_unsupported_variants(api):
    """The matrix-core (token-tiled) kernels take Algorithm-1 keys and values with an index bit; other
    variants are refused with TQ_ERR_UNSUPPORTED before anything is launched."""
    from vector_quantization_rotation_amd import _lib
    d, B, Hq, Hkv, T = 128, 1, 4, 1, 64
    pi, s = synth.haar_rotation(d, 1), synth.gaussian_projection(d, 2)
    for kmode, kb, vb in [(api.TQ_PROD, 3, 2), (api.TQ_MSE, 3, 1)]:
        kq = api.Quantizer(d, kb, kmode, pi, s if kmode == api.TQ_PROD else None)
        vq = api.Quantizer(d, vb, api.TQ_PROD, pi, s)
        kc = torch.zeros((B, Hkv, T, kq.code_bytes), dtype=torch.uint8, device="cuda")
        h16 = torch.zeros((B, Hkv, T), dtype=torch.int16, device="cuda")
        vt = torch.zeros((B, Hkv, (T + 31) // 32, vq.planes, d), dtype=torch.int32, device="cuda")
        q = torch.zeros((B, Hq, d), dtype=torch.bfloat16, device="cuda")
        with pytest.raises(_lib.TQError) as e:
            api.attn_decode(kq, vq, q, kc, h16, vt, h16, h16, torch.full((B,), T, dtype=torch.int32, device="cuda"),
                            0.1, vlayout=api.TQ_LAYOUT_TILE32, kgammas=h16 if kmode == api.TQ_PROD else None)
        assert e.value.status == _lib.TQ_ERR_UNSUPPORTED
