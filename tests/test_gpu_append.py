"""Decode-step append (tq_attn_decode_append) on the GPU against the CPU oracle (needs an MI355X).

A decode step encodes the new token's key and value into the cache at position seq_len[b] and attends
over the seq_len[b] + 1 tokens (the past_key_values update of the ai-navigate-news Gemma 4 post,
section "セットアップ").  Checked per case:
* the record (or the token's bit of every token-tiled word) written at seq_len[b] against the oracle's
  encoding of the new rows: bit-exact outside the tie zone, fp16 norms exact, gammas within one ulp at
  rounding midpoints;
* every other byte of the cache unchanged (positions past seq_len start as random bytes);
* the attention output against the oracle's attention over the oracle's records of tokens 0..seq_len[b].
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


CASES = [
    # (d, key mode, key bits, value bits, layout, B, Hq, Hkv, Tstride, seq, new-row dtype)
    (128, "mse", 3, 2, 1, 2, 8, 2, 304, [200, 37], "bf16"),     # wave-streaming kernel (stride % 8 == 0)
    (128, "mse", 3, 2, 1, 2, 8, 2, 300, [299, 0], "f32"),       # 4-wave kernel, the last slot, an empty cache
    (128, "mse", 2, 3, 1, 1, 8, 2, 128, [64], "bf16"),          # 2-bit value indices, a new tile word
    (256, "mse", 3, 2, 1, 2, 32, 16, 96, [95, 33], "bf16"),      # local-layer head dim
    (512, "mse", 3, 2, 1, 1, 16, 2, 80, [79], "bf16"),           # global-layer head dim
    (128, "mse", 3, 2, 0, 2, 8, 2, 300, [200, 300], "bf16"),    # row layout; a full sequence gets no token
    (128, "prod", 3, 2, 0, 2, 8, 2, 120, [100, 7], "f32"),      # Algorithm-2 keys
    (128, "prod", 1, 1, 0, 1, 4, 1, 64, [10], "f32"),           # 1-bit keys and values
]


@pytest.mark.parametrize("d,kmode,kb,vb,layout,B,Hq,Hkv,T,seq,xdt", CASES)
def test_attn_decode_append(api, d, kmode, kb, vb, layout, B, Hq, Hkv, T, seq, xdt):
    rng = np.random.default_rng(500 + d + kb)
    chans = synth.outlier_channels(Hkv, d, 4, 501)
    K = synth.bf16_bits_to_f32(synth.kv_bf16((B, Hkv, T, d), 502, chans)).reshape(-1, d)
    V = synth.bf16_bits_to_f32(synth.kv_bf16((B, Hkv, T, d), 503, chans)).reshape(-1, d)
    kn_raw = synth.bf16_bits_to_f32(synth.kv_bf16((B, Hkv, 1, d), 504, chans)).reshape(B * Hkv, d)
    vn_raw = synth.bf16_bits_to_f32(synth.kv_bf16((B, Hkv, 1, d), 505, chans)).reshape(B * Hkv, d)
    if xdt == "f32":  # fp32 rows off the bf16 grid
        kn_raw = (kn_raw * (1 + 1e-3 * rng.standard_normal(kn_raw.shape))).astype(np.float32)
        vn_raw = (vn_raw * (1 + 1e-3 * rng.standard_normal(vn_raw.shape))).astype(np.float32)
    piK, sK = synth.haar_rotation(d, 506), synth.gaussian_projection(d, 507)
    piV, sV = synth.haar_rotation(d, 508), synth.gaussian_projection(d, 509)
    q = synth.round_bf16(rng.standard_normal((B, Hq, d)).astype(np.float32))
    kprod = kmode == "prod"
    print(f"append d={d} keys {kmode} {kb}-bit values {vb}-bit layout={layout} B={B} Hq={Hq} Hkv={Hkv} T={T} "
          f"seq={seq} {xdt}", flush=True)
    kq = api.Quantizer(d, kb, api.TQ_PROD if kprod else api.TQ_MSE, piK, sK if kprod else None)
    vq = api.Quantizer(d, vb, api.TQ_PROD, piV, sV)

    def kenc(x):
        return parity.oracle_prod(x, piK, sK, kb) if kprod else parity.oracle_mse(x, piK, kb)

    ke, ve = kenc(K), parity.oracle_prod(V, piV, sV, vb)
    kne, vne = kenc(kn_raw), parity.oracle_prod(vn_raw, piV, sV, vb)
    # the cache: oracle records below seq_len[b], random bytes from there on
    krec = ke["record"].reshape(B, Hkv, T, -1).copy()
    vrec = ve["record"].reshape(B, Hkv, T, -1).copy()
    kn16 = parity.f16_bits(ke["n_hat"]).reshape(B, Hkv, T).copy()
    kg16 = parity.f16_bits(ke["gamma"]).reshape(B, Hkv, T).copy() if kprod else np.zeros((B, Hkv, T), np.int16)
    vn16 = parity.f16_bits(ve["n_hat"]).reshape(B, Hkv, T).copy()
    vg16 = parity.f16_bits(ve["gamma"]).reshape(B, Hkv, T).copy()
    for b in range(B):
        t = min(seq[b], T)
        krec[b, :, t:] = rng.integers(0, 256, size=krec[b, :, t:].shape, dtype=np.uint8)
        vrec[b, :, t:] = rng.integers(0, 256, size=vrec[b, :, t:].shape, dtype=np.uint8)
        for a16 in (kn16, kg16, vn16, vg16):
            a16[b, :, t:] = rng.integers(0, 0x3C00, size=a16[b, :, t:].shape, dtype=np.int16)
    if layout == api.TQ_LAYOUT_TILE32:
        vsrc_host = np.stack([oracle.tile_records(vrec.reshape(B * Hkv, T, -1)[i], d, vb)
                              for i in range(B * Hkv)]).view(np.int32).reshape(B, Hkv, -1, vb, d)
    else:
        vsrc_host = vrec
    kc, kn, kg = _dev(krec), _dev(kn16), _dev(kg16)
    vsrc, vn, vg = _dev(vsrc_host), _dev(vn16), _dev(vg16)
    seq_t = torch.tensor(seq, dtype=torch.int32, device="cuda")
    knew, vnew = _dev(kn_raw.reshape(B, Hkv, d)), _dev(vn_raw.reshape(B, Hkv, d))
    if xdt == "bf16":
        knew, vnew = knew.to(torch.bfloat16), vnew.to(torch.bfloat16)
    out = api.attn_decode_append(kq, vq, _dev(q).to(torch.bfloat16), knew, vnew, kc, kn, vsrc, vn, vg, seq_t,
                                 1.0 / math.sqrt(d), vlayout=layout, kgammas=kg if kprod else None)
    out = out.cpu().numpy()
    kc_h, kn_h, kg_h = kc.cpu().numpy(), kn.cpu().numpy(), kg.cpu().numpy()
    vn_h, vg_h = vn.cpu().numpy(), vg.cpu().numpy()
    vsrc_h = vsrc.cpu().numpy()
    vrec_h = (np.stack([parity.untile(vsrc_h.reshape(B * Hkv, -1, vb, d)[i], T, vb, d) for i in range(B * Hkv)])
              .reshape(B, Hkv, T, -1) if layout == api.TQ_LAYOUT_TILE32 else vsrc_h)

    # the written token against the oracle's encoding of the new rows; every other byte unchanged
    exp_k, exp_v = krec.copy(), vrec.copy()
    exp = [exp_k, kn16.copy(), kg16.copy(), exp_v, vn16.copy(), vg16.copy()]
    for b in range(B):
        t = seq[b]
        if t >= T:
            continue
        for g in range(Hkv):
            r = b * Hkv + g
            xk, xv = kn_raw[r:r + 1].astype(np.float64), vn_raw[r:r + 1].astype(np.float64)
            if kprod:
                kidx, ksb = oracle.parse_prod_record(kc_h[b, g, t][None], d, kb)
                parity.check_codes(kidx, kne["idx"][r:r + 1], oracle.code_margins(xk, piK, kne["t"]), max_frac=None)
                if np.array_equal(kidx, kne["idx"][r:r + 1]):
                    parity.check_codes(ksb, kne["signs"][r:r + 1], oracle.sign_margins(xk, piK, sK, kne["c"], kne["t"]),
                                       "sign", max_frac=None)
            else:
                kidx = oracle.parse_mse_record(kc_h[b, g, t][None], d, kb)
                parity.check_codes(kidx, kne["idx"][r:r + 1], oracle.code_margins(xk, piK, kne["t"]), max_frac=None)
            assert parity.check_norms(kn_h[b, g, t:t + 1], xk) == 0
            vidx, vsb = oracle.parse_prod_record(vrec_h[b, g, t][None], d, vb)
            parity.check_codes(vidx, vne["idx"][r:r + 1], oracle.code_margins(xv, piV, vne["t"]), max_frac=None)
            if np.array_equal(vidx, vne["idx"][r:r + 1]):
                parity.check_codes(vsb, vne["signs"][r:r + 1], oracle.sign_margins(xv, piV, sV, vne["c"], vne["t"]),
                                   "sign", max_frac=None)
                rn = np.linalg.norm(parity.residual_given_index(xv, vne["idx"][r:r + 1], vne["n_hat"][r:r + 1], piV,
                                                                vne["c"]), axis=1)
                parity.check_gammas(vg_h[b, g, t:t + 1], rn)
            assert parity.check_norms(vn_h[b, g, t:t + 1], xv) == 0
            for arr, got in zip(exp, [kc_h, kn_h, kg_h, vrec_h, vn_h, vg_h]):
                arr[b, g, t] = got[b, g, t]  # the written slot is judged above
    for arr, got in zip(exp, [kc_h, kn_h, kg_h, vrec_h, vn_h, vg_h]):
        assert np.array_equal(arr, got)
    if layout == api.TQ_LAYOUT_TILE32:
        # tile words: only bit (t % 32) of the words of token t's tile may have changed
        before = vsrc_host.reshape(B, Hkv, -1).view(np.uint32)
        after = vsrc_h.reshape(B, Hkv, -1).view(np.uint32)
        for b in range(B):
            diff = before[b] ^ after[b]
            if seq[b] >= T:
                assert not np.any(diff)
            else:
                assert np.all((diff & ~np.uint32(1 << (seq[b] % 32))) == 0)

    # attention over tokens 0..seq[b] with the oracle's records (old tokens and the new one)
    Kd = kn_raw.reshape(B, Hkv, d)
    for b in range(B):
        t = seq[b]
        n_att = min(t + 1, T)
        for g in range(Hkv):
            r = b * Hkv + g
            rows = slice(r * T, r * T + min(t, T))
            if kprod:
                Kt = oracle.decode_prod(ke["idx"][rows], ke["n_hat"][rows], ke["signs"][rows], ke["gamma"][rows], piK,
                                        sK, ke["c"])
                Kn = oracle.decode_prod(kne["idx"][r:r + 1], kne["n_hat"][r:r + 1], kne["signs"][r:r + 1],
                                        kne["gamma"][r:r + 1], piK, sK, kne["c"])
            else:
                Kt = oracle.decode_mse(ke["idx"][rows], ke["n_hat"][rows], piK, ke["c"])
                Kn = oracle.decode_mse(kne["idx"][r:r + 1], kne["n_hat"][r:r + 1], piK, kne["c"])
            Vt = oracle.decode_prod(ve["idx"][rows], ve["n_hat"][rows], ve["signs"][rows], ve["gamma"][rows], piV, sV,
                                    ve["c"])
            Vn = oracle.decode_prod(vne["idx"][r:r + 1], vne["n_hat"][r:r + 1], vne["signs"][r:r + 1],
                                    vne["gamma"][r:r + 1], piV, sV, vne["c"])
            if t < T:
                Kt, Vt = np.concatenate([Kt, Kn]), np.concatenate([Vt, Vn])
            G = Hq // Hkv
            ref = oracle.decode_attention(q[b:b + 1, g * G:(g + 1) * G], Kt[None, None], Vt[None, None],
                                          np.array([n_att]), 1.0 / math.sqrt(d))[0]
            err = parity.rel_rows(out[b, g * G:(g + 1) * G], ref)
            assert np.all(err <= parity.RTOL), (b, g, err.max())
    del Kd
