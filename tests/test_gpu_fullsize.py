"""Parity at the benchmark's full sizes and launch configuration, on sampled outputs.

Decode attention: batch 16, 32 query heads over 8 KV heads, head_dim 128,
131072 tokens, keys mse 3-bit, values prod 2-bit (token-tiled), the exact call
bench.py times on the cache the library itself encoded.  For sampled
(batch, kv-head) slices the oracle regenerates the same raw bf16 K/V from the
seeded generator and encodes them; its records replace the library's in those
slices, the GPU attends over the whole cache, and the sampled outputs must
agree with the oracle's attention within the gate.  The library's own codes
for other sampled slices are checked against the oracle's encode.  Encode: one layer's K/V cache (batch 8, 8 heads,
32768 tokens); sampled rows are encoded by the oracle and compared with the
tie-zone rule.
"""
import math

import numpy as np
import pytest

import oracle
from tests import parity

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

B, HQ, HKV, T, D = 16, 32, 8, 131072, 128


@pytest.fixture(scope="module")
def cache():
    from vector_quantization_rotation_amd import workloads
    c = workloads.build_attention_cache(B, HQ, HKV, T, D)
    yield c
    del c
    torch.cuda.empty_cache()


def _raw_slice(which, b, g):
    """The raw bf16 K or V rows of (batch b, kv-head g), regenerated from the workload's seeds."""
    from vector_quantization_rotation_amd import synth, workloads
    seeds = workloads.ATTN_SEEDS
    chans = synth.outlier_channels(HKV, D, 4, seeds["chan"])
    x = synth.kv_bf16_torch((1, HKV, T, D), seeds[which] * 1000 + b, chans, "cuda")
    out = x[0, g].float().cpu().numpy()
    del x
    return out


def test_attention_full_size_sampled(cache):
    # sampled slices hold the oracle's own records (all others the library's); the timed call runs
    # over the whole cache and the sampled outputs are held to the attention tolerance
    from vector_quantization_rotation_amd import api
    G = HQ // HKV
    refs = {}
    # (7, 1), (9, 4), (11, 4), (13, 1): slices where value weights far below a chunk's maximum round
    # to zero on the integer weight grid; with the value sums taken from the rounded weights the
    # error stays ~4e-5 (summing the exact weights instead left a 5.8e-4 bias there)
    for (b, g) in [(0, 0), (7, 3), (15, 7), (7, 1), (9, 4), (11, 4), (13, 1)]:
        K, V = _raw_slice("K", b, g), _raw_slice("V", b, g)
        ke, ve = parity.install_oracle_slice(cache, b, g, K, V)
        Kt = oracle.decode_mse(ke["idx"], ke["n_hat"], cache.piK, ke["c"])
        Vt = oracle.decode_prod(ve["idx"], ve["n_hat"], ve["signs"], ve["gamma"], cache.piV, cache.sV, ve["c"])
        refs[(b, g)] = oracle.decode_attention(cache.q_host[b:b + 1, g * G:(g + 1) * G], Kt[None, None],
                                               Vt[None, None], np.array([T]), 1 / math.sqrt(D))[0]
    seq = torch.full((B,), T, dtype=torch.int32, device="cuda")
    out = api.attn_decode(cache.kq, cache.vq, cache.q, cache.kcodes, cache.knorms, cache.vtiles, cache.vnorms,
                          cache.vgammas, seq, 1 / math.sqrt(D), vlayout=api.TQ_LAYOUT_TILE32).cpu().numpy()
    worst = 0.0
    for (b, g), ref in refs.items():
        err = parity.rel_rows(out[b, g * G:(g + 1) * G], ref)
        worst = max(worst, float(err.max()))
        assert np.all(err <= parity.RTOL), (b, g, err)
        assert np.all(err <= 2e-4), (b, g, err)  # the kernel's arithmetic bound, ten times inside the gate
    print(f"full-size attention: max rel err over sampled slices {worst:.2e}")


def test_attention_cache_codes_full_size(cache):
    # the cache the timed call reads: key records and token-tiled value words decode to the
    # oracle's own codes (tie-zone rule), for sampled sequences
    for (b, g) in [(3, 1), (12, 6)]:
        K, V = _raw_slice("K", b, g), _raw_slice("V", b, g)
        ke = parity.oracle_mse(K, cache.piK, 3)
        kidx = oracle.parse_mse_record(cache.kcodes[b, g].cpu().numpy(), D, 3)
        parity.check_codes(kidx, ke["idx"], oracle.code_margins(K, cache.piK, ke["t"]))
        assert parity.check_norms(cache.knorms[b, g].cpu().numpy(), K) == 0
        ve = parity.oracle_prod(V, cache.piV, cache.sV, 2)
        rec = parity.untile(cache.vtiles[b, g].cpu().numpy(), T, 2, D)
        assert np.array_equal(rec, cache.vcodes[b, g].cpu().numpy())  # tiles carry exactly the rows' bits
        vidx, vsb = oracle.parse_prod_record(rec, D, 2)
        parity.check_codes(vidx, ve["idx"], oracle.code_margins(V, cache.piV, ve["t"]))
        parity.check_prod_signs(vsb, vidx, ve, V, cache.piV, cache.sV)


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
    vidx, vsb = oracle.parse_prod_record(vc[ri].cpu().numpy(), d, 3)
    ve = parity.oracle_prod(xv, piV, sV, 3)
    parity.check_codes(vidx, ve["idx"], oracle.code_margins(xv, piV, ve["t"]))
    _, _, same = parity.check_prod_signs(vsb, vidx, ve, xv, piV, sV)
    rn = np.linalg.norm(parity.residual_given_index(xv, ve["idx"], ve["n_hat"], piV, ve["c"]), axis=1)
    parity.check_gammas(vg[ri].cpu().numpy()[same], rn[same])
