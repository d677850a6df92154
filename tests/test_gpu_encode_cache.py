"""tq_encode_cache on the GPU: a prompt's keys or values written straight into a decode cache.

Rows of x [nseq, T, d] go to positions t0 .. t0+T-1 of every sequence of a cache of Tstride positions,
as row records or as token-tiled words (the layout the decode-attention kernels stream), by the
quantizer's algorithm (Algorithm 1 or Algorithm 2 of the ai-navigate-news Gemma 4 post, section
"仕組み（技術的）").  Checked per case:
* the written records (read back from the tiles when tiled) against the oracle's encoding of the rows:
  bit-exact outside the tie zone, fp16 norms exact, gammas within one ulp at rounding midpoints;
* the same bytes as the row encode (tq_encode_mse / tq_encode_prod) of the same rows, since both run one
  arithmetic;
* every other byte of the cache unchanged; in the tiled layout the words that hold written positions
  are rewritten whole, with zero bits past the last token.
Head dims 64 and 128 take the encode kernel's own cache epilogue (an in-register bit transpose for the
tiles); other head dims and the 1-bit sign mode stage the records and move them into place.
"""
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


CASES = [
    # (d, mode, bits, layout, nseq, T, t0, Tstride, x dtype)
    (128, "mse", 3, 1, 3, 100, 32, 256, "bf16"),   # ragged T, offset start, fused kernel (4 waves)
    (128, "prod", 2, 1, 2, 64, 0, 64, "bf16"),     # the whole cache, fused Algorithm 2 (8 waves, 16 columns)
    (128, "prod", 3, 0, 3, 70, 5, 80, "f32"),      # row layout, unaligned start
    (64, "mse", 2, 1, 2, 33, 64, 160, "f16"),      # head dim 64 (16 columns per wave), one token into a new word
    (128, "prod", 3, 1, 1, 1, 32, 96, "bf16"),     # a single token
    (128, "mse", 4, 1, 2, 130, 96, 256, "bf16"),   # 4-bit indices, three 64-row tiles per sequence
    (256, "mse", 3, 1, 2, 50, 32, 128, "bf16"),    # staged path, tiled
    (256, "prod", 2, 0, 2, 40, 3, 64, "bf16"),     # staged path, rows
    (128, "prod", 1, 1, 2, 45, 0, 64, "f32"),      # the 1-bit sign mode (staged path)
]


def _x(shape, seed, xdt):
    chans = synth.outlier_channels(shape[0], shape[-1], 4, seed + 1)
    x = synth.bf16_bits_to_f32(synth.kv_bf16((1, shape[0], shape[1], shape[2]), seed, chans)).reshape(shape)
    if xdt == "f32":  # fp32 rows off the bf16 grid
        rng = np.random.default_rng(seed + 2)
        x = (x * (1 + 1e-3 * rng.standard_normal(x.shape))).astype(np.float32)
    return x


@pytest.mark.parametrize("d,mode,bits,layout,nseq,T,t0,Ts,xdt", CASES)
def test_encode_cache(api, d, mode, bits, layout, nseq, T, t0, Ts, xdt):
    print(f"encode_cache d={d} {mode} {bits}-bit layout={layout} nseq={nseq} T={T} t0={t0} Tstride={Ts} {xdt}",
          flush=True)
    prod = mode == "prod"
    x = _x((nseq, T, d), 700 + d + bits, xdt)
    pi = synth.haar_rotation(d, 701)
    s = synth.gaussian_projection(d, 702) if prod else None
    q = api.Quantizer(d, bits, api.TQ_PROD if prod else api.TQ_MSE, pi, s)
    P, cb = q.planes, q.code_bytes
    rng = np.random.default_rng(703)
    ntile = (Ts + 31) // 32
    if layout == api.TQ_LAYOUT_TILE32:
        before = rng.integers(-2**31, 2**31 - 1, size=(nseq, ntile, P, d), dtype=np.int64).astype(np.int32)
    else:
        before = rng.integers(0, 256, size=(nseq, Ts, cb), dtype=np.uint8)
    n_before = rng.integers(0, 0x3C00, size=(nseq, Ts), dtype=np.int16)
    g_before = rng.integers(0, 0x3C00, size=(nseq, Ts), dtype=np.int16)
    codes, norms = torch.from_numpy(before.copy()).cuda(), torch.from_numpy(n_before.copy()).cuda()
    gammas = torch.from_numpy(g_before.copy()).cuda() if prod else None
    xt = torch.from_numpy(x).cuda()
    if xdt == "bf16":
        xt = xt.to(torch.bfloat16)
    elif xdt == "f16":
        xt = xt.to(torch.float16)
    api.encode_cache(q, xt, codes, norms, gammas, t0=t0, layout=layout)
    # the row encode of the same rows
    rc, rn, rg = q.encode(xt.reshape(-1, d))
    torch.cuda.synchronize()
    got, n_got = codes.cpu().numpy(), norms.cpu().numpy()
    g_got = gammas.cpu().numpy() if prod else None
    rc, rn = rc.cpu().numpy().reshape(nseq, T, cb), rn.cpu().numpy().reshape(nseq, T)
    rg = rg.cpu().numpy().reshape(nseq, T) if prod else None

    # expected cache: the row encode's bytes placed at t0.., everything else as before
    exp_n = n_before.copy()
    exp_n[:, t0:t0 + T] = rn
    assert np.array_equal(n_got, exp_n)
    if prod:
        exp_g = g_before.copy()
        exp_g[:, t0:t0 + T] = rg
        assert np.array_equal(g_got, exp_g)
    if layout == api.TQ_LAYOUT_TILE32:
        exp = before.copy().view(np.uint32)
        k0, k1 = t0 // 32, (t0 + T + 31) // 32
        for sq in range(nseq):  # (positions past the last token in its word: zero bits)
            exp[sq, k0:k1] = oracle.tile_records(rc[sq], d, P)
        assert np.array_equal(got.view(np.uint32), exp)
        recs = np.stack([parity.untile(got[sq, k0:k1], T, P, d) for sq in range(nseq)])
    else:
        exp = before.copy()
        exp[:, t0:t0 + T] = rc
        assert np.array_equal(got, exp)
        recs = got[:, t0:t0 + T]

    # the records against the oracle's encoding (tie-zone rule)
    xr = x.reshape(-1, d).astype(np.float64)
    recs = recs.reshape(nseq * T, cb)
    nh = n_got[:, t0:t0 + T].reshape(-1)
    assert parity.check_norms(nh, xr) == 0
    if prod:
        enc = parity.oracle_prod(xr, pi, s, bits)
        idx, sb = oracle.parse_prod_record(recs, d, bits)
        parity.check_codes(idx, enc["idx"], oracle.code_margins(xr, pi, enc["t"]))
        _, _, same = parity.check_prod_signs(sb, idx, enc, xr, pi, s)
        gg = g_got[:, t0:t0 + T].reshape(-1)
        rn_exact = np.linalg.norm(parity.residual_given_index(xr[same], idx[same], enc["n_hat"][same], pi, enc["c"]),
                                  axis=1)
        parity.check_gammas(gg[same], rn_exact)
    else:
        enc = parity.oracle_mse(xr, pi, bits)
        idx = oracle.parse_mse_record(recs, d, bits)
        parity.check_codes(idx, enc["idx"], oracle.code_margins(xr, pi, enc["t"]))


def test_encode_cache_rejects_bad_positions(api):
    d = 128
    q = api.Quantizer(d, 3, api.TQ_MSE, synth.haar_rotation(d, 710))
    x = torch.zeros((1, 40, d), dtype=torch.bfloat16, device="cuda")
    norms = torch.zeros((1, 64), dtype=torch.int16, device="cuda")
    tiles = torch.zeros((1, 2, q.planes, d), dtype=torch.int32, device="cuda")
    rows = torch.zeros((1, 64, q.code_bytes), dtype=torch.uint8, device="cuda")
    with pytest.raises(api.TQError, match="INVALID"):
        api.encode_cache(q, x, tiles, norms, t0=16, layout=api.TQ_LAYOUT_TILE32)  # not a multiple of 32
    with pytest.raises(api.TQError, match="INVALID"):
        api.encode_cache(q, x, rows, norms, t0=30, layout=api.TQ_LAYOUT_ROWS)  # 30 + 40 > 64
    api.encode_cache(q, x[:, :0], rows, norms, t0=64, layout=api.TQ_LAYOUT_ROWS)  # nothing to write
