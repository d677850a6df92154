"""Chunked prefill attention (tq_attn_prefill) on the GPU against the CPU oracle (needs an MI355X).

M query tokens per sequence at positions q_pos[b] + m attend, causally, the cached tokens
0..q_pos[b] + m (the chunk's own keys and values already encoded into the cache).  The oracle encodes
the cache, and the reference for query token m is its two-pass attention over the first q_pos[b] + m + 1
decoded tokens.  With M = 1 the result must equal a decode step over q_pos + 1 tokens exactly.
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


def _cache(api, d, kmode, kb, vb, B, Hkv, T, seed):
    chans = synth.outlier_channels(Hkv, d, 4, seed)
    K = synth.bf16_bits_to_f32(synth.kv_bf16((B, Hkv, T, d), seed + 1, chans)).reshape(-1, d)
    V = synth.bf16_bits_to_f32(synth.kv_bf16((B, Hkv, T, d), seed + 2, chans)).reshape(-1, d)
    piK, sK = synth.haar_rotation(d, seed + 3), synth.gaussian_projection(d, seed + 4)
    piV, sV = synth.haar_rotation(d, seed + 5), synth.gaussian_projection(d, seed + 6)
    kprod = kmode == "prod"
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
    dev = dict(kcodes=_dev(ke["record"]).view(B, Hkv, T, -1), knorms=_dev(parity.f16_bits(ke["n_hat"])).view(B, Hkv, T),
               vcodes=_dev(ve["record"]).view(B, Hkv, T, -1), vnorms=_dev(parity.f16_bits(ve["n_hat"])).view(B, Hkv, T),
               vgammas=_dev(parity.f16_bits(ve["gamma"])).view(B, Hkv, T), kgammas=kg)
    return kq, vq, Kt.reshape(B, Hkv, T, d), Vt.reshape(B, Hkv, T, d), dev


@pytest.mark.parametrize("d,kmode,kb,vb,B,M,Hq,Hkv,T,qpos", [
    (128, "mse", 3, 2, 2, 37, 8, 2, 300, [100, 250]),
    (128, "mse", 3, 2, 1, 64, 32, 8, 200, [0]),         # the first chunk of a prompt
    (256, "prod", 3, 2, 2, 9, 16, 4, 160, [151, 17]),    # Algorithm-2 keys
    (64, "mse", 2, 1, 1, 20, 4, 4, 64, [30]),            # 1-bit values
    (128, "mse", 3, 2, 1, 128, 32, 8, 600, [400]),       # 4096 rows: the rotation back as one GEMM
])
def test_attn_prefill(api, d, kmode, kb, vb, B, M, Hq, Hkv, T, qpos):
    rng = np.random.default_rng(600 + d + M)
    kq, vq, Kt, Vt, c = _cache(api, d, kmode, kb, vb, B, Hkv, T, 610)
    q = synth.round_bf16(rng.standard_normal((B, M, Hq, d)).astype(np.float32))
    print(f"prefill d={d} keys {kmode} {kb}-bit B={B} M={M} Hq={Hq} Hkv={Hkv} T={T} q_pos={qpos}", flush=True)
    out = api.attn_prefill(kq, vq, _dev(q).to(torch.bfloat16), c["kcodes"], c["knorms"], c["vcodes"], c["vnorms"],
                           c["vgammas"], torch.tensor(qpos, dtype=torch.int32, device="cuda"), 1.0 / math.sqrt(d),
                           kgammas=c["kgammas"]).cpu().numpy()
    worst = 0.0
    for m in range(M):
        lens = np.minimum(np.array(qpos) + m + 1, T)
        ref = oracle.decode_attention(q[:, m], Kt, Vt, lens, 1.0 / math.sqrt(d))
        err = parity.rel_rows(out[:, m], ref)
        worst = max(worst, float(err.max()))
        assert np.all(err <= parity.RTOL), (m, err.max())
    print(f"prefill d={d}: max rel err {worst:.2e}")


def test_prefill_one_token_equals_decode_step(api):
    d, B, Hq, Hkv, T = 128, 2, 8, 2, 500
    kq, vq, _, _, c = _cache(api, d, "mse", 3, 2, B, Hkv, T, 620)
    q = _dev(synth.round_bf16(np.random.default_rng(621).standard_normal((B, Hq, d)).astype(np.float32))).to(torch.bfloat16)
    qpos = torch.tensor([400, 33], dtype=torch.int32, device="cuda")
    pre = api.attn_prefill(kq, vq, q.view(B, 1, Hq, d), c["kcodes"], c["knorms"], c["vcodes"], c["vnorms"],
                           c["vgammas"], qpos, 1.0 / math.sqrt(d))
    dec = api.attn_decode(kq, vq, q, c["kcodes"], c["knorms"], c["vcodes"], c["vnorms"], c["vgammas"], qpos + 1,
                          1.0 / math.sqrt(d))
    assert torch.equal(pre.view(B, Hq, d), dec)


@pytest.mark.parametrize("d,kb,vb,B,M,Hq,Hkv,T,qpos", [
    (128, 3, 2, 2, 37, 8, 2, 304, [100, 250]),     # the wave-streaming kernel (stride a multiple of 8)
    (128, 3, 2, 1, 64, 32, 8, 200, [0]),           # the first chunk of a prompt
    (128, 3, 2, 1, 160, 32, 8, 400, [200]),        # 5120 query rows of one split each: rotated back by one GEMM
    (128, 3, 2, 1, 128, 32, 1, 3200, [3000]),      # 4096 rows over several splits: merge, then the GEMM
    (128, 2, 3, 1, 20, 8, 2, 301, [270]),          # 2-bit value indices: the four-wave kernel
    (256, 3, 2, 1, 12, 16, 4, 160, [140]),         # head_dim 256
    (512, 3, 2, 2, 9, 8, 1, 200, [150, 40]),       # head_dim 512: the global-layer kernel
])
def test_attn_prefill_tiled(api, d, kb, vb, B, M, Hq, Hkv, T, qpos):
    """Token-tiled values: every query token becomes a row of the decode kernels, reading its sequence's
    cache row; checked against the oracle's attention of each token over its causal prefix."""
    rng = np.random.default_rng(700 + d + M)
    kq, vq, Kt, Vt, c = _cache(api, d, "mse", kb, vb, B, Hkv, T, 710)
    vrec = c["vcodes"].cpu().numpy().reshape(B * Hkv, T, -1)
    tiles = _dev(np.stack([oracle.tile_records(vrec[i], d, vq.planes) for i in range(B * Hkv)]).view(np.int32))
    tiles = tiles.view(B, Hkv, (T + 31) // 32, vq.planes, d)
    q = synth.round_bf16(rng.standard_normal((B, M, Hq, d)).astype(np.float32))
    print(f"tiled prefill d={d} keys {kb}-bit values {vb}-bit B={B} M={M} Hq={Hq} Hkv={Hkv} T={T} q_pos={qpos}",
          flush=True)
    out = api.attn_prefill(kq, vq, _dev(q).to(torch.bfloat16), c["kcodes"], c["knorms"], tiles, c["vnorms"],
                           c["vgammas"], torch.tensor(qpos, dtype=torch.int32, device="cuda"), 1.0 / math.sqrt(d),
                           vlayout=api.TQ_LAYOUT_TILE32).cpu().numpy()
    worst = 0.0
    for m in range(M):
        lens = np.minimum(np.array(qpos) + m + 1, T)
        ref = oracle.decode_attention(q[:, m], Kt, Vt, lens, 1.0 / math.sqrt(d))
        err = parity.rel_rows(out[:, m], ref)
        worst = max(worst, float(err.max()))
        assert np.all(err <= parity.RTOL), (m, err.max())
    print(f"tiled prefill d={d}: max rel err {worst:.2e}")


def test_prefill_tiled_one_token_equals_decode_step(api):
    """M = 1 over token-tiled values: the same kernels as the decode step over q_pos + 1 tokens."""
    d, B, Hq, Hkv, T = 128, 2, 8, 2, 512
    kq, vq, _, _, c = _cache(api, d, "mse", 3, 2, B, Hkv, T, 720)
    vrec = c["vcodes"].cpu().numpy().reshape(B * Hkv, T, -1)
    tiles = _dev(np.stack([oracle.tile_records(vrec[i], d, vq.planes) for i in range(B * Hkv)]).view(np.int32))
    tiles = tiles.view(B, Hkv, T // 32, vq.planes, d)
    q = _dev(synth.round_bf16(np.random.default_rng(721).standard_normal((B, Hq, d)).astype(np.float32))).to(torch.bfloat16)
    qpos = torch.tensor([400, 33], dtype=torch.int32, device="cuda")
    pre = api.attn_prefill(kq, vq, q.view(B, 1, Hq, d), c["kcodes"], c["knorms"], tiles, c["vnorms"], c["vgammas"],
                           qpos, 1.0 / math.sqrt(d), vlayout=api.TQ_LAYOUT_TILE32)
    dec = api.attn_decode(kq, vq, q, c["kcodes"], c["knorms"], tiles, c["vnorms"], c["vgammas"], qpos + 1,
                          1.0 / math.sqrt(d), vlayout=api.TQ_LAYOUT_TILE32)
    assert torch.equal(pre.view(B, Hq, d), dec)
