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


# (1024 and 1100 rows at d > 128: the GEMM path's grid with the column blocks of a row block grouped on one XCD,
# 8 row blocks, and with a row-block count that is not a multiple of 8)
@pytest.mark.parametrize("n,d,bits", [(4096, 128, 2), (4096, 128, 3), (1000, 64, 1), (333, 256, 4), (130, 512, 3),
                                      (1024, 256, 3), (1100, 512, 2), (1000, 64, 3), (777, 64, 4)])
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


@pytest.mark.parametrize("n,d,bits", [(4096, 128, 3), (4096, 128, 2), (257, 256, 4), (130, 512, 3), (1024, 512, 3), (1300, 256, 2),
                                      (1024, 128, 4), (1000, 64, 3)])
def test_encode_prod_parity(api, n, d, bits):
    if d == 128:
        x, pi, s, _ = _unit_inputs(n, d)
    else:
        x, pi, s = synth.unit_test_vectors(n, d, 17, 18), synth.haar_rotation(d, 19), synth.gaussian_projection(d, 20)
    qz = api.Quantizer(d, bits, api.TQ_PROD, pi, s)
    codes, norms, gammas = qz.encode(_dev(x))
    torch.cuda.synchronize()
    enc = parity.oracle_prod(x, pi, s, bits)
    idx, sb = _idx_of(codes, d, bits, True)
    parity.check_codes(idx, enc["idx"], oracle.code_margins(x, pi, enc["t"]))
    assert parity.check_norms(norms.cpu().numpy(), x) == 0
    nbad, nties, same = parity.check_prod_signs(sb, idx, enc, x, pi, s)
    rn = np.linalg.norm(parity.residual_given_index(x, enc["idx"], enc["n_hat"], pi, enc["c"]), axis=1)
    parity.check_gammas(gammas.cpu().numpy()[same], rn[same])
    # whole records byte-identical on rows where every decision agrees
    rows = same & np.all(sb == enc["signs"], axis=1)
    assert np.array_equal(codes.cpu().numpy()[rows], enc["record"][rows])
    print(f"prod d={d} b={bits}: sign mismatches {nbad}, tie-zone signs {nties}, rows compared {int(rows.sum())}")


def _oracle_encoded(qz_bits, prod, x, pi, s):
    """Oracle records and norms as the GPU's inputs (device tensors) plus the oracle's decode."""
    if prod:
        enc = parity.oracle_prod(x, pi, s, qz_bits)
        xt = oracle.decode_prod(enc["idx"], enc["n_hat"], enc["signs"], enc["gamma"], pi, s, enc["c"])
        gam = _dev(parity.f16_bits(enc["gamma"]))
    else:
        enc = parity.oracle_mse(x, pi, qz_bits)
        xt = oracle.decode_mse(enc["idx"], enc["n_hat"], pi, enc["c"])
        gam = None
    return _dev(enc["record"]), _dev(parity.f16_bits(enc["n_hat"])), gam, xt


# (1000 rows: a last 64-record tile of 40, whose rows the kernel stores and no row past it; head dim 64: a
# thread's 16 coordinates as 16-bit plane words; 1 and 2 index bits expand by byte permutes, 3 by a select tree)
@pytest.mark.parametrize("mode,bits,n,d", [("mse", 2, 4096, 128), ("prod", 3, 4096, 128), ("mse", 4, 4096, 128),
                                           ("prod", 2, 4096, 128), ("mse", 3, 1000, 128), ("prod", 3, 1000, 128),
                                           ("mse", 1, 1000, 128), ("mse", 2, 1000, 64), ("prod", 3, 1000, 64),
                                           ("prod", 4, 1000, 64)])
def test_decode_parity(api, mode, bits, n, d):
    x, pi, s, _ = _unit_inputs(n, d)
    prod = mode == "prod"
    qz = api.Quantizer(d, bits, api.TQ_PROD if prod else api.TQ_MSE, pi, s if prod else None)
    codes, norms, gammas, ref = _oracle_encoded(bits, prod, x, pi, s)
    # rows of d within a wider buffer (row stride d + 4) with 64 rows below: what lies outside stays as it was
    big = torch.full((n + 64, d + 4), 7.0, dtype=torch.float32, device="cuda")
    qz.decode(codes, norms, gammas, out=big[:n, :d])
    big = big.cpu().numpy()
    assert np.all(big[n:] == 7.0) and np.all(big[:n, d:] == 7.0)
    out = big[:n, :d]
    err = parity.rel_rows(out, ref)
    assert np.all(err <= parity.RTOL), err.max()
    # the kernel's own arithmetic bound, far inside the gate: each product carries the top 16 significant
    # bits of both operands (head dims up to 128: two bf16 pieces; three dropped terms of <= 2^-16 each);
    # the fp32 GEMM path of larger head dims is tighter still
    assert err.max() < 1e-4


@pytest.mark.parametrize("mode,bits", [("mse", 2), ("prod", 3)])
def test_score_parity_all_pairs(api, mode, bits):
    x, pi, s, q = _unit_inputs()
    d = 128
    prod = mode == "prod"
    qz = api.Quantizer(d, bits, api.TQ_PROD if prod else api.TQ_MSE, pi, s if prod else None)
    codes, norms, gammas, xt = _oracle_encoded(bits, prod, x, pi, s)
    sc = qz.score(_dev(q), codes, norms, gammas).cpu().numpy()
    ref = oracle.inner_product_estimate(q, xt)
    tol = parity.RTOL * np.linalg.norm(q, axis=1)[:, None] * np.linalg.norm(xt, axis=1)[None, :]
    assert np.all(np.abs(sc - ref) <= tol)
    # the estimate tracks the exact inner product (report; prod is unbiased)
    exact = q.astype(np.float64) @ x.astype(np.float64).T
    print(mode, "mean est - exact:", float(np.mean(ref - exact)), "rms:", float(np.sqrt(np.mean((ref - exact) ** 2))))


def _check_topk(vals, idx, ref_scores, k, tol):
    """GPU top-k vs the oracle's scores: the same sorted values (within tol), distinct indices whose
    oracle scores sit at their rank (within 2 tol), and identical indices wherever the oracle's ranking
    is separated by more than 2 tol."""
    ref_idx, ref_vals = oracle.topk_desc(ref_scores, k)
    for i in range(ref_scores.shape[0]):
        assert len(set(idx[i].tolist())) == k
        assert np.all(np.abs(vals[i] - ref_vals[i]) <= tol[i])
        assert np.all(np.abs(ref_scores[i, idx[i]] - ref_vals[i]) <= 2 * tol[i])
        srt = np.sort(ref_scores[i])[::-1]
        gaps = srt[:k] - srt[1:k + 1] if ref_scores.shape[1] > k else np.append(srt[:k - 1] - srt[1:k], np.inf)
        for r in range(k):
            lo_sep = r == 0 or srt[r - 1] - srt[r] > 2 * tol[i]
            if lo_sep and gaps[r] > 2 * tol[i]:
                assert idx[i, r] == ref_idx[i, r], (i, r)
    return ref_idx


@pytest.mark.parametrize("n,k", [(4096, 10), (1000, 1), (70, 64), (5000, 17)])
def test_score_topk(api, n, k):
    d = 128
    x = synth.unit_test_vectors(n, d, 31, 32)
    pi, s = synth.haar_rotation(d, 33), synth.gaussian_projection(d, 34)
    q = synth.gaussian_queries(37, d, 35)
    qz = api.Quantizer(d, 3, api.TQ_PROD, pi, s)
    codes, norms, gammas, xt = _oracle_encoded(3, True, x, pi, s)
    vals, idx = qz.score(_dev(q), codes, norms, gammas, k=k)
    ref = oracle.inner_product_estimate(q, xt)
    tol = parity.RTOL * np.linalg.norm(q, axis=1) * np.max(np.linalg.norm(xt, axis=1))
    _check_topk(vals.cpu().numpy(), idx.cpu().numpy(), ref, k, tol)


def test_score_topk_ties_to_lower_index(api):
    d = 64
    pi, s = synth.haar_rotation(d, 1), synth.gaussian_projection(d, 2)
    base = synth.unit_test_vectors(5, d, 3, 4)
    x = np.repeat(base, 40, axis=0)  # identical records -> identical scores on both sides
    qz = api.Quantizer(d, 2, api.TQ_PROD, pi, s)
    codes, norms, gammas, xt = _oracle_encoded(2, True, x, pi, s)
    q = synth.gaussian_queries(3, d, 5)
    _, idx = qz.score(_dev(q), codes, norms, gammas, k=50)
    ref_idx, _ = oracle.topk_desc(oracle.inner_product_estimate(q, xt), 50)
    assert np.array_equal(idx.cpu().numpy(), ref_idx)


def _attn_case(api, B, Hq, Hkv, T, d, seq, qdtype, seed=0, layout=0, kbits=3, vbits=2, qfn=None):
    """Oracle-encoded K/V records (rows, or token-tiled by the oracle) fed to the GPU; the oracle's
    two-pass attention over its own decoded caches is the expected value.  qfn(rng, piK) -> [B, Hq, d]
    replaces the N(0, 1) queries."""
    rng = np.random.default_rng(seed)
    chans = synth.outlier_channels(Hkv, d, 4, seed + 1)
    K = synth.bf16_bits_to_f32(synth.kv_bf16((B, Hkv, T, d), seed + 2, chans)).reshape(-1, d)
    V = synth.bf16_bits_to_f32(synth.kv_bf16((B, Hkv, T, d), seed + 3, chans)).reshape(-1, d)
    piK, piV, sV = synth.haar_rotation(d, seed + 4), synth.haar_rotation(d, seed + 5), synth.gaussian_projection(d, seed + 6)
    q = rng.standard_normal((B, Hq, d)).astype(np.float32) if qfn is None else qfn(rng, piK).astype(np.float32)
    if qdtype == "bf16":
        q = synth.round_bf16(q)
    kq = api.Quantizer(d, kbits, api.TQ_MSE, piK)
    vq = api.Quantizer(d, vbits, api.TQ_PROD, piV, sV)
    ke = parity.oracle_mse(K, piK, kbits)
    ve = parity.oracle_prod(V, piV, sV, vbits)
    Kt = oracle.decode_mse(ke["idx"], ke["n_hat"], piK, ke["c"]).reshape(B, Hkv, T, d)
    Vt = oracle.decode_prod(ve["idx"], ve["n_hat"], ve["signs"], ve["gamma"], piV, sV, ve["c"]).reshape(B, Hkv, T, d)
    ref = oracle.decode_attention(q, Kt, Vt, np.array(seq), 1.0 / math.sqrt(d))
    qt = _dev(q) if qdtype == "f32" else _dev(q).to(torch.bfloat16)
    seq_t = torch.tensor(seq, dtype=torch.int32, device="cuda")
    vrec = ve["record"].reshape(B * Hkv, T, -1)
    if layout == api.TQ_LAYOUT_TILE32:
        vsrc = _dev(np.stack([oracle.tile_records(vrec[i], d, vbits) for i in range(B * Hkv)]).view(np.int32))
        vsrc = vsrc.view(B, Hkv, -1, vbits, d)
    else:
        vsrc = _dev(vrec).view(B, Hkv, T, -1)
    out = api.attn_decode(kq, vq, qt, _dev(ke["record"]).view(B, Hkv, T, -1),
                          _dev(parity.f16_bits(ke["n_hat"])).view(B, Hkv, T), vsrc,
                          _dev(parity.f16_bits(ve["n_hat"])).view(B, Hkv, T),
                          _dev(parity.f16_bits(ve["gamma"])).view(B, Hkv, T), seq_t, 1.0 / math.sqrt(d),
                          vlayout=layout).cpu().numpy()
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
    # sequence strides that are multiples of 8 take the wave-streaming kernel (head_dim 128, 1-bit values)
    (2, 8, 2, 1000, [1000, 641], 128, 3, 2),     # ragged tails inside a 64-token step
    (1, 8, 2, 4096, [4096], 128, 2, 2),
    (1, 4, 4, 2048, [1999], 128, 1, 2),
    (1, 4, 4, 2048, [1999], 128, 3, 2),          # one head per kv head
    (1, 4, 1, 2048, [1999], 128, 1, 2),          # 1-bit keys, four heads
    (1, 4, 4, 256, [256], 128, 1, 2),
    (2, 24, 4, 520, [520, 0], 128, 3, 2),        # 6 heads per kv head: a full and a partial head group
    (1, 4, 1, 192, [130], 128, 3, 2),            # one ring turn, the last step partly valid
    (1, 4, 1, 65536, [65000], 128, 3, 2),        # more than 256 sequence splits: separate merge and rotation
    (1, 32, 8, 30000, [29999], 128, 3, 2),       # many steps per wave
    # head_dim 512 (global-layer shape): Walsh coefficients applied after the matrix cores
    (1, 8, 1, 1000, [1000], 512, 3, 2),
    (2, 16, 2, 700, [700, 333], 512, 2, 2),
    (1, 32, 4, 1100, [1099], 512, 1, 2),
    (1, 4, 4, 300, [300], 512, 3, 2),            # one head per kv head
    # head_dim 512, sequence strides that are multiples of 8: the eight-wave kernel with LDS-staged steps
    (2, 16, 2, 704, [704, 333], 512, 2, 2),      # two head groups, a ragged step
    (1, 32, 4, 1104, [1099], 512, 1, 2),         # 1-bit keys, 8 heads per kv head
    (1, 4, 4, 304, [300], 512, 3, 2),            # one head per kv head
    (1, 8, 1, 65536, [65000], 512, 3, 2),        # several ring turns per work-group
    (2, 8, 2, 128, [1, 127], 512, 3, 2),         # one token; one step short of full
    (1, 4, 1, 400, [399], 256, 3, 2),            # head_dim 256 folded at 3-bit keys
    (1, 4, 1, 400, [399], 128, 4, 3),            # 4-bit keys, 3-bit values: folded, one wave per SIMD
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


def _q_spike(rng, piK):
    """Queries whose rotated image q' = Pi_K q is one coordinate of size 40 over N(0, 1e-3) noise: the
    key operand's fixed-point query digits resolve the small coordinates only to their absolute grid."""
    d = piK.shape[0]
    qr = 1e-3 * rng.standard_normal((2, 8, d))
    qr[:, :, 5] = 40.0
    qr[:, 3:, 77] = -25.0
    return qr @ np.asarray(piK, dtype=np.float64)  # q = Pi^T q'


def _q_sharp(rng, piK):
    """N(0, 1) queries scaled by 12: scores spread over hundreds of log2 units (a near one-hot softmax
    whose runner-up tokens still carry weight in some heads)."""
    return 12.0 * rng.standard_normal((2, 8, piK.shape[0]))


@pytest.mark.parametrize("kind", ["spike", "sharp"])
@pytest.mark.parametrize("kb", [3, 1, 4])
def test_attn_query_extremes(api, kind, kb):
    """The score paths on queries far from N(0, 1): the wave kernel (head_dim 128, 2-bit values, token-tiled)
    and, at 4-bit keys, the 4-wave kernel, against the oracle's attention within the gate."""
    qfn = _q_spike if kind == "spike" else _q_sharp
    out, ref = _attn_case(api, 2, 8, 2, 3000, 128, [3000, 1777], "f32", seed=31, layout=api.TQ_LAYOUT_TILE32,
                          kbits=kb, vbits=2, qfn=qfn)
    for b in range(2):
        err = parity.rel_rows(out[b], ref[b])
        print(f"{kind} queries, {kb}-bit keys, b={b}: max rel err {err.max():.2e}")
        assert np.all(err <= parity.RTOL), (b, err.max())


@pytest.mark.parametrize("T,layout", [(30000, 1), (30000, 0), (4096, 1)])
def test_attn_peaked_softmax_long_tail(api, T, layout):
    """One dominant token and a tail of T - 1 tokens with equal keys whose softmax weight relative to
    the maximum is 3e-8, below the integer weight grid of the token-tiled kernels: the chunk holding
    the dominant token rounds its tail weights to zero, the other chunks keep them (each chunk has its
    own maximum).  Held to 2e-4, ten times inside the gate.  (The whole-sequence chunk, where the tail
    behind the dominant token is long, is test_attn_whole_sequence_chunk_tail_with_common_offset.)"""
    d, Hq, Hkv = 128, 4, 1
    rng = np.random.default_rng(77)
    xa, xb = rng.standard_normal((2, d)).astype(np.float32)
    K = np.repeat(xb[None], T, axis=0)
    K[7] = xa
    K = synth.round_bf16(K)
    V = synth.bf16_bits_to_f32(synth.kv_bf16((1, Hkv, T, d), 79)).reshape(-1, d)
    piK, piV, sV = synth.haar_rotation(d, 80), synth.haar_rotation(d, 81), synth.gaussian_projection(d, 82)
    ke = parity.oracle_mse(K, piK, 3)
    ve = parity.oracle_prod(V, piV, sV, 2)
    Kt = oracle.decode_mse(ke["idx"], ke["n_hat"], piK, ke["c"])
    Vt = oracle.decode_prod(ve["idx"], ve["n_hat"], ve["signs"], ve["gamma"], piV, sV, ve["c"])
    # score gap s_7 - s_tail = ln(1 / 3e-8) along the difference of the two decoded keys, per head a
    # small shift of the common part
    diff = Kt[7] - Kt[0]
    lam = math.log(1.0 / 3e-8) * math.sqrt(d) / float(diff @ diff)
    q = np.stack([lam * diff + 0.01 * h * rng.standard_normal(d) for h in range(Hq)])[None].astype(np.float32)
    ref = oracle.decode_attention(q, Kt.reshape(1, Hkv, T, d), Vt.reshape(1, Hkv, T, d), np.array([T]),
                                  1.0 / math.sqrt(d))
    kq = api.Quantizer(d, 3, api.TQ_MSE, piK)
    vq = api.Quantizer(d, 2, api.TQ_PROD, piV, sV)
    if layout == api.TQ_LAYOUT_TILE32:
        vsrc = _dev(oracle.tile_records(ve["record"], d, 2).view(np.int32)).view(1, Hkv, -1, 2, d)
    else:
        vsrc = _dev(ve["record"]).view(1, Hkv, T, -1)
    out = api.attn_decode(kq, vq, _dev(q), _dev(ke["record"]).view(1, Hkv, T, -1),
                          _dev(parity.f16_bits(ke["n_hat"])).view(1, Hkv, T), vsrc,
                          _dev(parity.f16_bits(ve["n_hat"])).view(1, Hkv, T),
                          _dev(parity.f16_bits(ve["gamma"])).view(1, Hkv, T),
                          torch.tensor([T], dtype=torch.int32, device="cuda"), 1.0 / math.sqrt(d),
                          vlayout=layout).cpu().numpy()
    err = parity.rel_rows(out[0], ref[0])
    print(f"peaked softmax T={T} layout={layout}: max rel err {err.max():.2e}")
    assert np.all(err <= 2e-4), err


def _broadcast_sequence(t, nseq):
    """One sequence's cache array [T, ...] repeated for nseq sequences on the device: [nseq, T, ...]."""
    return t.unsqueeze(0).expand(nseq, *t.shape).contiguous()


@pytest.mark.parametrize("kind,vbits", [("sink", 2), ("spiky", 2), ("sink", 3)])
def test_attn_whole_sequence_chunk_tail_with_common_offset(api, kind, vbits):
    """A plan with as many (batch, kv-head) units as resident work-group slots, so that one work-group
    streams the whole sequence, over values that share a common offset (V = mu + N(0, 1)), held to
    2e-4.  'sink': one dominant key and 32767 equal keys whose softmax weight is 2^-20 of it, so
    that the tail carries about 3 % of the mass on the coarse end of the integer weight grid (a
    weight grid fixed to the dominant token would bias the output along mu by about 4e-3).
    'spiky': distinct random keys and a query scaled so that scores spread over about 6 log2 units
    (held to 5e-4: the softmax mass sits in a few tokens and the tail 10-20 log2 units below them
    keeps part of its rounding; a CPU emulation of a weight grid fixed to the running maximum gives
    about 1.4e-3 in this regime).  2-bit values take the wave-streaming kernel (2048 units), 3-bit
    values the 4-wave kernel (512 units).  Every unit holds the same sequence, so the oracle attends
    one of them."""
    d, T, G = 128, 32768, 4
    Hkv = 128
    B = 16 if vbits == 2 else 4
    Hq = G * Hkv
    rng = np.random.default_rng(90)
    mu = 2.0 * rng.standard_normal(d)
    V = synth.round_bf16((mu[None] + rng.standard_normal((T, d))).astype(np.float32))
    if kind == "sink":
        xa, xb = rng.standard_normal((2, d)).astype(np.float32)
        K = np.repeat(xb[None], T, axis=0)
        K[7] = xa
    else:
        K = rng.standard_normal((T, d)).astype(np.float32)
    K = synth.round_bf16(K)
    piK, piV, sV = synth.haar_rotation(d, 91), synth.haar_rotation(d, 92), synth.gaussian_projection(d, 93)
    ke = parity.oracle_mse(K, piK, 3)
    ve = parity.oracle_prod(V, piV, sV, vbits)
    Kt = oracle.decode_mse(ke["idx"], ke["n_hat"], piK, ke["c"])
    Vt = oracle.decode_prod(ve["idx"], ve["n_hat"], ve["signs"], ve["gamma"], piV, sV, ve["c"])
    if kind == "sink":
        diff = Kt[7] - Kt[0]
        lam = 20.0 * math.log(2.0) * math.sqrt(d) / float(diff @ diff)
        qg = np.stack([lam * diff + 0.01 * h * rng.standard_normal(d) for h in range(G)])
    else:
        qg = rng.standard_normal((G, d))
        qg *= 6.0 * math.log(2.0) * math.sqrt(d) / np.std(Kt @ qg.T, axis=0)[:, None]
    qg = synth.round_bf16(qg.astype(np.float32))
    ref = oracle.decode_attention(qg[None], Kt.reshape(1, 1, T, d), Vt.reshape(1, 1, T, d), np.array([T]),
                                  1.0 / math.sqrt(d))[0]
    nseq = B * Hkv
    kq = api.Quantizer(d, 3, api.TQ_MSE, piK)
    vq = api.Quantizer(d, vbits, api.TQ_PROD, piV, sV)
    kc = _broadcast_sequence(_dev(ke["record"]), nseq).view(B, Hkv, T, -1)
    kn = _broadcast_sequence(_dev(parity.f16_bits(ke["n_hat"])), nseq).view(B, Hkv, T)
    vt = _broadcast_sequence(_dev(oracle.tile_records(ve["record"], d, vbits).view(np.int32)), nseq)
    vt = vt.view(B, Hkv, -1, vbits, d)
    vn = _broadcast_sequence(_dev(parity.f16_bits(ve["n_hat"])), nseq).view(B, Hkv, T)
    vg = _broadcast_sequence(_dev(parity.f16_bits(ve["gamma"])), nseq).view(B, Hkv, T)
    q = _dev(np.broadcast_to(qg[None, None], (B, Hkv, G, d)).reshape(B, Hq, d)).to(torch.bfloat16)
    seq = torch.full((B,), T, dtype=torch.int32, device="cuda")
    print(f"whole-sequence chunk: kind={kind} value bits={vbits} B={B} Hkv={Hkv} T={T}", flush=True)
    out = api.attn_decode(kq, vq, q, kc, kn, vt, vn, vg, seq, 1.0 / math.sqrt(d), vlayout=api.TQ_LAYOUT_TILE32)
    out = out.cpu().numpy().reshape(B * Hkv, G, d)
    del kc, kn, vt, vn, vg
    err = parity.rel_rows(out, np.broadcast_to(ref[None], out.shape))
    print(f"whole-sequence chunk: kind={kind} value bits={vbits}: max rel err {err.max():.2e}")
    assert np.all(err <= (2e-4 if kind == "sink" else 5e-4)), err.max()


def test_tile_records_matches_oracle(api):
    d, T = 128, 100
    x = synth.unit_test_vectors(3 * T, d, 51, 52)
    pi, s = synth.haar_rotation(d, 53), synth.gaussian_projection(d, 54)
    vq = api.Quantizer(d, 2, api.TQ_PROD, pi, s)
    rec = parity.oracle_prod(x, pi, s, 2)["record"].reshape(3, T, -1)
    tiles = api.tile_records(vq, _dev(rec)).cpu().numpy().view(np.uint32)
    for sq in range(3):
        assert np.array_equal(tiles[sq], oracle.tile_records(rec[sq], d, 2))
        assert np.array_equal(parity.untile(tiles[sq], T, 2, d), rec[sq])


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
    """The same values given as bf16 / fp16 rows (fp16 matrix-core operands) and as fp32 rows (exact bf16
    pieces): the norms agree exactly, the codes wherever the oracle's decision is outside the tie zone."""
    d = 128
    x = synth.round_bf16(synth.unit_test_vectors(512, d, 41, 42))
    pi = synth.haar_rotation(d, 43)
    qz = api.Quantizer(d, 3, api.TQ_MSE, pi)
    _, t = oracle.lloyd_max(d, 3)
    for xs, dt in ((x, torch.bfloat16), (x.astype(np.float16).astype(np.float32), torch.float16)):
        c32, n32, _ = qz.encode(_dev(xs))
        ch, nh, _ = qz.encode(_dev(xs).to(dt))
        assert torch.equal(n32, nh)
        i32, _ = _idx_of(c32, d, 3, False)
        ih, _ = _idx_of(ch, d, 3, False)
        bad = i32 != ih
        assert not np.any(bad & (oracle.code_margins(xs, pi, t) > parity.TIE))


def _half_rows(n, d, seed, dt):
    """Rows of the benchmark law plus rows that stress the per-row power-of-two scale: norms near 1e-30
    and 1e30 (bf16) or near the fp16 range's ends, a row with one large coordinate over tiny ones, and a
    zero row; returned as the rows' exact float64 values (what the oracle encodes)."""
    x = synth.unit_test_vectors(n, d, seed, seed + 1).astype(np.float64)
    rng = np.random.default_rng(seed + 2)
    if dt == "bf16":
        x[0] *= 1e-30
        x[1] *= 1e30
        x[2] = rng.standard_normal(d) * 1e-20
        x[2, 5] = 3.0
        x[3] = 0.0
        x = synth.round_bf16(x.astype(np.float32)).astype(np.float64)
    else:
        x[0] *= 2e-3
        x[1] *= 90000.0 / np.linalg.norm(x[1])  # coordinates in the fp16 range, the norm beyond it
        x[2] = rng.standard_normal(d) * 1e-3
        x[2, 5] = 60000.0
        x[3] = 0.0
        x = x.astype(np.float16).astype(np.float64)
    return x


@pytest.mark.parametrize("d,mode,bits,dt", [(128, "mse", 3, "bf16"), (128, "prod", 3, "f16"), (64, "prod", 2, "bf16"),
                                            (128, "prod", 4, "bf16"), (256, "mse", 4, "bf16"), (256, "prod", 3, "f16"),
                                            (512, "mse", 3, "bf16"), (512, "prod", 2, "bf16")])
def test_encode_half_rows_parity(api, d, mode, bits, dt):
    """bf16 / fp16 rows (fp16 operands: row-scaled rows, two-piece matrices) against the oracle's encoding
    of the same values in fp64: codes outside the tie zone exact, fp16 norms exact, gammas within the
    midpoint rule; rows at extreme scales included."""
    n = 1000 if d <= 256 else 300
    x = _half_rows(n, d, 800 + d + bits, dt)
    pi = synth.haar_rotation(d, 810 + d)
    prod = mode == "prod"
    s = synth.gaussian_projection(d, 811 + d) if prod else None
    qz = api.Quantizer(d, bits, api.TQ_PROD if prod else api.TQ_MSE, pi, s)
    xt = _dev(x.astype(np.float32)).to(torch.bfloat16 if dt == "bf16" else torch.float16)
    assert np.array_equal(xt.float().cpu().numpy().astype(np.float64), x)  # the rows are exact in their dtype
    codes, norms, gammas = qz.encode(xt)
    torch.cuda.synchronize()
    assert parity.check_norms(norms.cpu().numpy(), x) == 0
    if prod:
        enc = parity.oracle_prod(x, pi, s, bits)
        idx, sb = _idx_of(codes, d, bits, True)
        parity.check_codes(idx, enc["idx"], oracle.code_margins(x, pi, enc["t"]))
        _, _, same = parity.check_prod_signs(sb, idx, enc, x, pi, s)
        rn = np.linalg.norm(parity.residual_given_index(x, enc["idx"], enc["n_hat"], pi, enc["c"]), axis=1)
        parity.check_gammas(gammas.cpu().numpy()[same], rn[same])
    else:
        enc = parity.oracle_mse(x, pi, bits)
        idx, _ = _idx_of(codes, d, bits, False)
        parity.check_codes(idx, enc["idx"], oracle.code_margins(x, pi, enc["t"]))


def test_profile_select_brackets_named_kernels(api):
    """tq_profile_select: while a name is selected only the matching launches record events; "" selects
    every launch again (the attention step launches prep, the wave-streaming kernel and the finish)."""
    from vector_quantization_rotation_amd import _lib, workloads
    d, T = 128, 256
    c = workloads.build_attention_cache(1, 4, 1, T, d)
    seq = torch.full((1,), T, dtype=torch.int32, device="cuda")
    out = torch.empty((1, 4, d), dtype=torch.float32, device="cuda")
    ws = torch.empty((api.attn_decode_ws_bytes(c.kq, 1, 4, 1, T, api.TQ_LAYOUT_TILE32),), dtype=torch.uint8,
                     device="cuda")
    step = api.attn_decode_bound(c.kq, c.vq, c.q, c.kcodes, c.knorms, c.vtiles, c.vnorms, c.vgammas, seq,
                                 1 / math.sqrt(d), out, ws, vlayout=api.TQ_LAYOUT_TILE32)
    try:
        for sel, expect in (("attn_wave", {"attn_wave": 2, "attn_prep": 0, "attn_combine": 0}),
                            ("", {"attn_wave": 2, "attn_prep": 2, "attn_combine": 2})):
            _lib.profile_reset()
            _lib.profile_select(sel)
            _lib.profile_enable(True)
            step()
            step()
            torch.cuda.synchronize()
            _lib.profile_enable(False)
            for name, n in expect.items():
                ms, cnt = _lib.profile_query(name)
                assert cnt == n, (sel, name, cnt)
                assert (ms > 0) == (n > 0), (sel, name, ms)
    finally:
        _lib.profile_enable(False)
        _lib.profile_select("")
        _lib.profile_reset()
