"""Parity at the benchmark's full sizes and launch configuration, on sampled outputs.

Decode attention: batch 16, 32 query heads over 8 KV heads, head_dim 128,
131072 tokens, keys mse 3-bit, values prod 2-bit (token-tiled), the exact call
bench.py times; the oracle recomputes sampled (batch, kv-head) slices from the
GPU's own records.  Encode: one layer's K/V cache (batch 8, 8 heads, 32768
tokens); sampled rows are re-encoded by the oracle and compared with the
tie-zone rule.
"""
import math

import numpy as np
import pytest

import oracle
from tests import parity

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def cache():
    from vector_quantization_rotation_amd import workloads
    c = workloads.build_attention_cache(16, 32, 8, 131072, 128)
    yield c
    del c
    torch.cuda.empty_cache()


def test_attention_full_size_sampled(cache):
    from vector_quantization_rotation_amd import api
    B, Hq, Hkv, T, d = 16, 32, 8, 131072, 128
    seq = torch.full((B,), T, dtype=torch.int32, device="cuda")
    out = api.attn_decode(cache.kq, cache.vq, cache.q, cache.kcodes, cache.knorms, cache.vtiles, cache.vnorms,
                          cache.vgammas, seq, 1 / math.sqrt(d), vlayout=api.TQ_LAYOUT_TILE32).cpu().numpy()
    cK, _ = oracle.lloyd_max(d, 3)
    cV, _ = oracle.lloyd_max(d, 1)
    G = Hq // Hkv
    worst = 0.0
    for (b, g) in [(0, 0), (7, 3), (15, 7), (9, 5)]:
        kidx = oracle.parse_mse_record(cache.kcodes[b, g].cpu().numpy(), d, 3)
        vidx, vsb = oracle.parse_prod_record(cache.vcodes[b, g].cpu().numpy(), d, 2)
        Kt = oracle.decode_mse(kidx, parity.f16_from_bits(cache.knorms[b, g].cpu().numpy()), cache.piK, cK)
        Vt = oracle.decode_prod(vidx, parity.f16_from_bits(cache.vnorms[b, g].cpu().numpy()), vsb,
                                parity.f16_from_bits(cache.vgammas[b, g].cpu().numpy()), cache.piV, cache.sV, cV)
        ref = oracle.decode_attention(cache.q_host[b:b + 1, g * G:(g + 1) * G], Kt[None, None], Vt[None, None],
                                      np.array([T]), 1 / math.sqrt(d))[0]
        err = parity.rel_rows(out[b, g * G:(g + 1) * G], ref)
        worst = max(worst, float(err.max()))
        assert np.all(err <= parity.RTOL), (b, g, err)
    print(f"full-size attention: max rel err over sampled slices {worst:.2e}")


def test_attention_tiles_match_records_full_size(cache):
    # the tiled value cache carries exactly the bits of the records (two sampled sequences)
    for (b, g) in [(3, 1), (12, 6)]:
        rec = cache.vcodes[b, g].cpu().numpy()
        tiles = cache.vtiles[b, g].cpu().numpy().view(np.uint32)
        assert np.array_equal(tiles, oracle.tile_records(rec, 128, 2))


def test_encode_full_size_sampled():
    from vector_quantization_rotation_amd import api, synth
    d = 128
    chans = synth.outlier_channels(8, d, 4, 203)
    K = synth.kv_bf16_torch((8, 8, 32768, d), 201, chans, "cuda").view(-1, d)
    V = synth.kv_bf16_torch((8, 8, 32768, d), 202, chans, "cuda").view(-1, d)
    piK, piV, sV = synth.haar_rotation(d, 211), synth.haar_rotation(d, 212), synth.gaussian_projection(d, 213)
    kq = api.Quantizer(d, 3, api.TQ_MSE, piK)
    vq = api.Quantizer(d, 3, api.TQ_PROD, piV, sV)
    kc, kn, _ = kq.encode(K)
    vc, vn, vg = vq.encode(V)
    rows = np.sort(np.random.default_rng(9).choice(K.shape[0], size=4096, replace=False))
    ri = torch.as_tensor(rows, device="cuda")
    xk = K[ri].float().cpu().numpy()
    xv = V[ri].float().cpu().numpy()
    cK, tK = oracle.lloyd_max(d, 3)
    idx_ref, _ = oracle.encode_mse(xk, piK, cK, tK)
    idx = oracle.parse_mse_record(kc[ri].cpu().numpy(), d, 3)
    parity.check_codes(idx, idx_ref, oracle.code_margins(xk, piK, tK))
    assert parity.check_norms(kn[ri].cpu().numpy(), xk) == 0
    cV, tV = oracle.lloyd_max(d, 2)
    vidx_ref, nh_ref, _, _ = oracle.encode_prod(xv, piV, sV, cV, tV)
    vidx, vsb = oracle.parse_prod_record(vc[ri].cpu().numpy(), d, 3)
    parity.check_codes(vidx, vidx_ref, oracle.code_margins(xv, piV, tV))
    r = parity.residual_given_index(xv, vidx, nh_ref, piV, cV)
    proj = r @ sV.astype(np.float64).T
    rn = np.linalg.norm(r, axis=1)
    parity.check_codes(vsb, (proj >= 0).astype(np.uint8), np.abs(proj) / rn[:, None], "sign")
    parity.check_gammas(vg[ri].cpu().numpy(), rn)
