"""Parity at full size for the heterogeneous-layer and search workloads, on sampled outputs.

Heterogeneous layers (Gemma 4 post, section "KV形状の不均一性"): a local layer
(batch 4, 32 query heads over 16 KV heads, head_dim 256, 1024-token window) and
a global layer (batch 4, 32 query heads over 4 KV heads, head_dim 512, 65536
tokens), bf16 N(0,1) with 4 Student-t(3) channels per head, keys mse 3-bit and
values prod 2-bit.  The library encodes the whole cache; for sampled
(batch, kv-head) slices the oracle regenerates the raw rows from the seeded
generator, encodes them, and its records replace the library's there; the GPU
attends over the whole cache and the sampled outputs are held to the attention
gate.  The library's own codes are checked against the oracle on other slices.

Search (AiBoss overview, section "TurboQuantの応用事例"): 10^6 clustered,
L2-normalised vectors of dimension 1536, TurboQuant_prod 4-bit, 1000 queries,
top-10.  Checked on samples the oracle can compute: the codes of sampled rows;
for sampled queries, the returned rows re-scored by the oracle from its own
encoding of those rows (values within the score gate, in descending order);
and no other row of the whole database, encoded and scored by the oracle,
beats the returned tenth score by more than the gate.  recall@10 against the fp64 exact
top-10 is printed; it has no value on the pages to be checked against (parity
unpinned).
"""
import math

import numpy as np
import pytest

import oracle
from tests import parity

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.mark.parametrize("kind", ["local", "global"])
def test_heterogeneous_layer_full_size(kind):
    from vector_quantization_rotation_amd import api, workloads
    L = workloads.HET_LAYERS[kind]
    B, Hq, Hkv, T, d, seeds = L["B"], L["Hq"], L["Hkv"], L["T"], L["d"], L["seeds"]
    nu = workloads.HET_NU
    G = Hq // Hkv
    cache = workloads.het_layer_cache(kind)
    tiled = cache.vtiles.shape[2] > 0

    # the library's own codes on a slice the oracle does not overwrite
    b, g = 1, 1
    K = workloads.raw_kv_slice("K", b, g, Hkv, T, d, seeds, nu)
    V = workloads.raw_kv_slice("V", b, g, Hkv, T, d, seeds, nu)
    ke = parity.oracle_mse(K, cache.piK, 3)
    kidx = oracle.parse_mse_record(cache.kcodes[b, g].cpu().numpy(), d, 3)
    parity.check_codes(kidx, ke["idx"], oracle.code_margins(K, cache.piK, ke["t"]))
    assert parity.check_norms(cache.knorms[b, g].cpu().numpy(), K) == 0
    ve = parity.oracle_prod(V, cache.piV, cache.sV, 2)
    vrec = cache.vcodes[b, g].cpu().numpy()
    if tiled:
        assert np.array_equal(parity.untile(cache.vtiles[b, g].cpu().numpy(), T, 2, d), vrec)
    vidx, vsb = oracle.parse_prod_record(vrec, d, 2)
    parity.check_codes(vidx, ve["idx"], oracle.code_margins(V, cache.piV, ve["t"]))
    parity.check_prod_signs(vsb, vidx, ve, V, cache.piV, cache.sV)

    # sampled slices on the oracle's records, attention over the whole cache
    refs = {}
    for (b, g) in [(0, 0), (B - 1, Hkv - 1)]:
        K = workloads.raw_kv_slice("K", b, g, Hkv, T, d, seeds, nu)
        V = workloads.raw_kv_slice("V", b, g, Hkv, T, d, seeds, nu)
        ke, ve = parity.install_oracle_slice(cache, b, g, K, V)
        Kt = oracle.decode_mse(ke["idx"], ke["n_hat"], cache.piK, ke["c"])
        Vt = oracle.decode_prod(ve["idx"], ve["n_hat"], ve["signs"], ve["gamma"], cache.piV, cache.sV, ve["c"])
        refs[(b, g)] = oracle.decode_attention(cache.q_host[b:b + 1, g * G:(g + 1) * G], Kt[None, None],
                                               Vt[None, None], np.array([T]), 1 / math.sqrt(d))[0]
    seq = torch.full((B,), T, dtype=torch.int32, device="cuda")
    layout = api.TQ_LAYOUT_TILE32 if tiled else api.TQ_LAYOUT_ROWS
    vsrc = cache.vtiles if tiled else cache.vcodes
    out = api.attn_decode(cache.kq, cache.vq, cache.q, cache.kcodes, cache.knorms, vsrc, cache.vnorms,
                          cache.vgammas, seq, 1 / math.sqrt(d), vlayout=layout).cpu().numpy()
    worst = 0.0
    for (b, g), ref in refs.items():
        err = parity.rel_rows(out[b, g * G:(g + 1) * G], ref)
        worst = max(worst, float(err.max()))
        assert np.all(err <= parity.RTOL), (kind, b, g, err)
    print(f"{kind} layer (d={d}, T={T}): max rel err over sampled slices {worst:.2e}")


@pytest.mark.timeout(900)
def test_search_full_size_sampled():
    from vector_quantization_rotation_amd import api, synth, workloads
    S = workloads.SEARCH
    n, d, bits, k = S["n"], S["d"], S["bits"], S["k"]
    sd = S["seeds"]
    X = workloads.search_database()
    pi, s = synth.haar_rotation(d, sd["pi"]), synth.gaussian_projection(d, sd["s"])
    qz = api.Quantizer(d, bits, api.TQ_PROD, pi, s)
    codes, norms, gammas = qz.encode(X)
    Q = workloads.search_queries()
    vals, idx = qz.score(torch.from_numpy(Q).cuda(), codes, norms, gammas, k=k)
    vals, idx = vals.cpu().numpy().astype(np.float64), idx.cpu().numpy()
    rng = np.random.default_rng(13)

    # codes of sampled rows
    rows = np.sort(rng.choice(n, size=1024, replace=False))
    ri = torch.as_tensor(rows, device="cuda")
    x = X[ri].cpu().numpy()
    ve = parity.oracle_prod(x, pi, s, bits)
    vidx, vsb = oracle.parse_prod_record(codes[ri].cpu().numpy(), d, bits)
    parity.check_codes(vidx, ve["idx"], oracle.code_margins(x, pi, ve["t"]))
    assert parity.check_norms(norms[ri].cpu().numpy(), x) == 0
    _, _, same = parity.check_prod_signs(vsb, vidx, ve, x, pi, s)
    rn = np.linalg.norm(parity.residual_given_index(x, ve["idx"], ve["n_hat"], pi, ve["c"]), axis=1)
    parity.check_gammas(gammas[ri].cpu().numpy()[same], rn[same])

    def oracle_scores(qs, row_ids):
        xr = X[torch.as_tensor(row_ids, device="cuda")].cpu().numpy()
        e = parity.oracle_prod(xr, pi, s, bits)
        xt = oracle.decode_prod(e["idx"], e["n_hat"], e["signs"], e["gamma"], pi, s, e["c"])
        return oracle.inner_product_estimate(Q[qs], xt), np.linalg.norm(xt, axis=1)

    qs = np.sort(rng.choice(Q.shape[0], size=8, replace=False))
    # the returned rows, re-scored by the oracle from its own encoding
    cand = np.unique(idx[qs].ravel())
    est_c, xtn = oracle_scores(qs, cand)
    tol = parity.RTOL * np.linalg.norm(Q[qs], axis=1) * xtn.max()
    pos = {int(r): j for j, r in enumerate(cand)}
    for i, qi in enumerate(qs):
        assert np.all(np.diff(vals[qi]) <= 0), qi
        ref = np.array([est_c[i, pos[int(r)]] for r in idx[qi]])
        assert np.all(np.abs(vals[qi] - ref) <= tol[i]), (qi, vals[qi] - ref)
    # completeness over the whole database: the oracle encodes every row (64K rows at a time) and no row
    # outside the returned ten beats the tenth returned score by more than the gate.  The estimate is
    # taken in its rotated form, n_hat <Pi q, c[idx]> + sqrt(pi/2)/d gamma <S q, 2 bits - 1>, equal to
    # <q, decode(x)> to 1e-12 relative
    qpi = Q[qs].astype(np.float64) @ pi.astype(np.float64).T
    qs_ = Q[qs].astype(np.float64) @ s.astype(np.float64).T
    best_out = np.full(len(qs), -np.inf)
    cb, tb = oracle.lloyd_max(d, bits - 1)
    for r0 in range(0, n, 65536):
        xr = X[r0:r0 + 65536].cpu().numpy()
        eidx, enh, esb, egam = oracle.encode_prod(xr, pi, s, cb, tb)
        est = (enh.astype(np.float64)[:, None] * (cb[eidx] @ qpi.T)
               + oracle.qjl_scale(d) * egam.astype(np.float64)[:, None] * ((2.0 * esb - 1.0) @ qs_.T)).T
        for i, qi in enumerate(qs):
            mine = (idx[qi] >= r0) & (idx[qi] < r0 + est.shape[1])
            est[i, idx[qi][mine] - r0] = -np.inf
        best_out = np.maximum(best_out, est.max(axis=1))
    for i, qi in enumerate(qs):
        assert best_out[i] <= vals[qi, -1] + 2 * tol[i], (qi, best_out[i], vals[qi, -1])

    # recall@10 against the exact fp64 top-10 over all rows (reported, parity unpinned)
    exact = np.full((len(qs), n), -np.inf)
    qd = Q[qs].astype(np.float64)
    for r0 in range(0, n, 65536):
        exact[:, r0:r0 + 65536] = qd @ X[r0:r0 + 65536].cpu().numpy().astype(np.float64).T
    ex_idx, _ = oracle.topk_desc(exact, k)
    print(f"search 1e6 x {d}: recall@{k} over {len(qs)} sampled queries = {oracle.recall_at_k(idx[qs], ex_idx):.3f}")
