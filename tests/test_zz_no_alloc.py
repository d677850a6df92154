"""tq_attn_decode_noalloc (the decode-attention entry point that allocates nothing) against
tq_attn_decode (caller workspace), through the C ABI on an MI355X.

Both run the same kernels with the same plan, so the outputs must be identical (and hence within
the attention gate of each other); checked on two calls in a row, the second on a smaller input
(the library's array keeps the first call's contents), for both value layouts.  A call whose
workspace would exceed the fixed array is rejected with TQ_ERR_WORKSPACE and launches nothing.
"""
import ctypes as C
import math

import numpy as np
import pytest

import oracle
from tests import parity
from vector_quantization_rotation_amd import synth

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _case(api, kq, vq, B, Hq, Hkv, T, seq, seed, layout):
    d = kq.d
    rng = np.random.default_rng(seed)
    chans = synth.outlier_channels(Hkv, d, 4, seed + 1)
    K = synth.bf16_bits_to_f32(synth.kv_bf16((B, Hkv, T, d), seed + 2, chans)).reshape(-1, d)
    V = synth.bf16_bits_to_f32(synth.kv_bf16((B, Hkv, T, d), seed + 3, chans)).reshape(-1, d)
    ke = parity.oracle_mse(K, kq.pi_host, kq.bits)
    ve = parity.oracle_prod(V, vq.pi_host, vq.s_host, vq.bits)
    q = _dev(synth.round_bf16(rng.standard_normal((B, Hq, d)).astype(np.float32))).to(torch.bfloat16)
    vrec = ve["record"].reshape(B * Hkv, T, -1)
    if layout == api.TQ_LAYOUT_TILE32:
        vsrc = _dev(np.stack([oracle.tile_records(vrec[i], d, vq.bits) for i in range(B * Hkv)]).view(np.int32))
        vsrc = vsrc.view(B, Hkv, -1, vq.bits, d)
    else:
        vsrc = _dev(vrec).view(B, Hkv, T, -1)
    return (q, _dev(ke["record"]).view(B, Hkv, T, -1), _dev(parity.f16_bits(ke["n_hat"])).view(B, Hkv, T), vsrc,
            _dev(parity.f16_bits(ve["n_hat"])).view(B, Hkv, T), _dev(parity.f16_bits(ve["gamma"])).view(B, Hkv, T),
            torch.tensor(seq, dtype=torch.int32, device="cuda"))


@pytest.mark.parametrize("layout", [1, 0])
def test_noalloc_matches_workspace_entry_point(layout):
    from vector_quantization_rotation_amd import api
    d = 128
    piK, piV, sV = synth.haar_rotation(d, 301), synth.haar_rotation(d, 302), synth.gaussian_projection(d, 303)
    kq = api.Quantizer(d, 3, api.TQ_MSE, piK)
    vq = api.Quantizer(d, 2, api.TQ_PROD, piV, sV)
    kq.pi_host, vq.pi_host, vq.s_host = piK, piV, sV
    for (B, Hq, Hkv, T, seq, seed) in [(2, 16, 4, 3000, [3000, 1234], 310), (1, 8, 2, 520, [333], 320)]:
        print(f"no-alloc attention layout={layout} B={B} Hq={Hq} Hkv={Hkv} T={T}", flush=True)
        args = _case(api, kq, vq, B, Hq, Hkv, T, seq, seed, layout)
        ref = api.attn_decode(kq, vq, *args, 1.0 / math.sqrt(d), vlayout=layout)
        out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
        api.attn_decode_noalloc(kq, vq, *args, 1.0 / math.sqrt(d), out, vlayout=layout)
        torch.cuda.synchronize()
        a, r = out.cpu().numpy(), ref.cpu().numpy()
        for b in range(B):
            if seq[b] == 0:
                assert np.all(a[b] == 0)
                continue
            assert np.all(parity.rel_rows(a[b], r[b]) <= parity.RTOL)
        assert np.array_equal(a, r)


def test_noalloc_rejects_oversized_workspace():
    from vector_quantization_rotation_amd import _lib, api
    d = 128
    kq = api.Quantizer(d, 3, api.TQ_MSE, synth.haar_rotation(d, 1))
    vq = api.Quantizer(d, 2, api.TQ_PROD, synth.haar_rotation(d, 2), synth.gaussian_projection(d, 3))
    lib = _lib.load()
    B, Hq, Hkv, T = 64, 256, 64, 1 << 20
    need = lib.tq_attn_decode_ws_bytes(kq.handle, B, Hq, Hkv, T, api.TQ_LAYOUT_TILE32)
    assert need > _lib.TQ_NOALLOC_SCRATCH_BYTES
    # real (small) device buffers stand in for the arguments: the size check rejects the call before
    # any argument is read or anything is launched
    buf = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    p = C.c_void_p(buf.data_ptr())
    rc = lib.tq_attn_decode_noalloc(kq.handle, vq.handle, p, api.TQ_BF16, B, Hq, Hkv, p, p, None, p, p, p,
                                    api.TQ_LAYOUT_TILE32, T, p, C.c_float(1.0), p, C.c_void_p(0))
    assert rc == _lib.TQ_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.count_nonzero(buf).item() == 0
