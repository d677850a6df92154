"""PyTorch-facing wrappers over the C ABI (same names as include/tq.h, minus the prefix).

Tensors are used for device memory only; each call passes raw pointers and the
current HIP stream to libtq.so and returns the output tensors it allocated.
"""
from __future__ import annotations

import ctypes as C

import numpy as np
import torch

from . import _lib
from ._lib import (TQ_BF16, TQ_F16, TQ_F32, TQ_LAYOUT_ROWS, TQ_LAYOUT_TILE32, TQ_MSE, TQ_PROD,  # noqa: F401
                   TQError, codebook_build, load)

_DT = {torch.float32: TQ_F32, torch.bfloat16: TQ_BF16, torch.float16: TQ_F16}


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return C.c_void_p(t.data_ptr()) if t is not None else C.c_void_p(0)


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return t


class Quantizer:
    """A TurboQuant quantizer on the current device (one per vector shape and mode)."""

    def __init__(self, d: int, bits: int, mode: int, pi: np.ndarray, s: np.ndarray | None = None):
        lib = load()
        pi = np.ascontiguousarray(pi, dtype=np.float32)
        sp = None
        if s is not None:
            s = np.ascontiguousarray(s, dtype=np.float32)
            sp = s.ctypes.data_as(C.POINTER(C.c_float))
        h = C.c_void_p()
        _lib._check("tq_quantizer_create",
                    lib.tq_quantizer_create(C.byref(h), d, bits, mode, pi.ctypes.data_as(C.POINTER(C.c_float)), sp))
        self._h = h
        dd, bb, mm, pl, cb = C.c_int(), C.c_int(), C.c_int(), C.c_int(), C.c_size_t()
        _lib._check("tq_quantizer_info", lib.tq_quantizer_info(h, C.byref(dd), C.byref(bb), C.byref(mm),
                                                                C.byref(pl), C.byref(cb)))
        self.d, self.bits, self.mode, self.planes, self.code_bytes = dd.value, bb.value, mm.value, pl.value, cb.value

    @property
    def handle(self):
        return self._h

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            load().tq_quantizer_destroy(self._h)
            self._h = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- encode ------------------------------------------------------------
    def encode(self, x: torch.Tensor, codes=None, norms=None, gammas=None):
        """Encode rows of x ([n, d] or [..., d], fp32/bf16/fp16 device tensor).

        Returns (codes uint8 [n, code_bytes], norms int16-bits [n], gammas or None).
        """
        _dev(x, "x")
        x2 = x.reshape(-1, x.shape[-1])
        if x2.stride(-1) != 1:
            x2 = x2.contiguous()
        n = x2.shape[0]
        dev = x.device
        if codes is None:
            codes = torch.empty((n, self.code_bytes), dtype=torch.uint8, device=dev)
        if norms is None:
            norms = torch.empty((n,), dtype=torch.int16, device=dev)
        lib = load()
        if self.mode == TQ_MSE:
            rc = lib.tq_encode_mse(self._h, _ptr(x2), _DT[x2.dtype], n, x2.stride(0), _ptr(codes), _ptr(norms), _stream())
            _lib._check("tq_encode_mse", rc)
            return codes, norms, None
        if gammas is None:
            gammas = torch.empty((n,), dtype=torch.int16, device=dev)
        rc = lib.tq_encode_prod(self._h, _ptr(x2), _DT[x2.dtype], n, x2.stride(0), _ptr(codes), _ptr(norms),
                                _ptr(gammas), _stream())
        _lib._check("tq_encode_prod", rc)
        return codes, norms, gammas

    def decode(self, codes: torch.Tensor, norms: torch.Tensor, gammas: torch.Tensor | None = None, out=None):
        n = codes.shape[0]
        if out is None:
            out = torch.empty((n, self.d), dtype=torch.float32, device=codes.device)
        rc = load().tq_decode(self._h, _ptr(codes), _ptr(norms), _ptr(gammas), n, _ptr(out), out.stride(0), _stream())
        _lib._check("tq_decode", rc)
        return out

    def score(self, queries: torch.Tensor, codes: torch.Tensor, norms: torch.Tensor, gammas=None, k: int = 0):
        """k == 0: [m, n] scores; k > 0: (values [m, k], indices [m, k]) of the best records per query."""
        lib = load()
        m, n = queries.shape[0], codes.shape[0]
        ws_b = lib.tq_score_ws_bytes(self._h, m, n, k)
        ws = torch.empty((max(ws_b, 1),), dtype=torch.uint8, device=queries.device)
        if k == 0:
            scores = torch.empty((m, n), dtype=torch.float32, device=queries.device)
            idx = None
        else:
            scores = torch.empty((m, k), dtype=torch.float32, device=queries.device)
            idx = torch.empty((m, k), dtype=torch.int64, device=queries.device)
        rc = lib.tq_score(self._h, _ptr(queries), m, queries.stride(0), _ptr(codes), _ptr(norms), _ptr(gammas), n, k,
                          _ptr(scores), _ptr(idx), _ptr(ws), ws_b, _stream())
        _lib._check("tq_score", rc)
        return scores if k == 0 else (scores, idx)


def tile_records(q: Quantizer, codes: torch.Tensor, out=None):
    """Row-layout records [nseq, T, code_bytes] -> TQ_LAYOUT_TILE32 words [nseq, ceil(T/32), planes, d] (int32)."""
    nseq, T = codes.shape[0], codes.shape[1]
    ntile = (T + 31) // 32
    if out is None:
        out = torch.empty((nseq, ntile, q.planes, q.d), dtype=torch.int32, device=codes.device)
    rc = load().tq_tile_records(q.handle, _ptr(codes), nseq, T, _ptr(out), _stream())
    _lib._check("tq_tile_records", rc)
    return out


def attn_decode_ws_bytes(kq: Quantizer, B: int, Hq: int, Hkv: int, Tstride: int, vlayout: int = TQ_LAYOUT_ROWS) -> int:
    return load().tq_attn_decode_ws_bytes(kq.handle, B, Hq, Hkv, Tstride, vlayout)


def attn_decode(kq: Quantizer, vq: Quantizer, q: torch.Tensor, kcodes, knorms, vcodes, vnorms, vgammas,
                seq_len: torch.Tensor, scale: float, out=None, ws=None, vlayout: int = TQ_LAYOUT_ROWS):
    """q [B, Hq, d]; key caches [B, Hkv, Tstride, ...]; value records in `vlayout`; -> out [B, Hq, d] fp32."""
    lib = load()
    B, Hq, d = q.shape
    Hkv, Tstride = kcodes.shape[1], kcodes.shape[2]
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    ws_b = lib.tq_attn_decode_ws_bytes(kq.handle, B, Hq, Hkv, Tstride, vlayout)
    if ws is None:
        ws = torch.empty((max(ws_b, 1),), dtype=torch.uint8, device=q.device)
    rc = lib.tq_attn_decode(kq.handle, vq.handle, _ptr(q), _DT[q.dtype], B, Hq, Hkv, _ptr(kcodes), _ptr(knorms),
                            _ptr(vcodes), _ptr(vnorms), _ptr(vgammas), vlayout, Tstride, _ptr(seq_len), float(scale),
                            _ptr(out), _ptr(ws), ws.numel(), _stream())
    _lib._check("tq_attn_decode", rc)
    return out


def attn_decode_bound(kq: Quantizer, vq: Quantizer, q: torch.Tensor, kcodes, knorms, vcodes, vnorms, vgammas,
                      seq_len: torch.Tensor, scale: float, out: torch.Tensor, ws: torch.Tensor,
                      vlayout: int = TQ_LAYOUT_ROWS):
    """attn_decode with every argument marshalled once: returns a no-argument callable that
    enqueues the same call on the current stream (for tight decode loops)."""
    lib = load()
    B, Hq, d = q.shape
    Hkv, Tstride = kcodes.shape[1], kcodes.shape[2]
    args = (kq.handle, vq.handle, _ptr(q), _DT[q.dtype], B, Hq, Hkv, _ptr(kcodes), _ptr(knorms), _ptr(vcodes),
            _ptr(vnorms), _ptr(vgammas), vlayout, Tstride, _ptr(seq_len), C.c_float(scale), _ptr(out), _ptr(ws),
            C.c_size_t(ws.numel()), _stream())
    fn = lib.tq_attn_decode

    def call():
        rc = fn(*args)
        if rc != 0:
            _lib._check("tq_attn_decode", rc)
    return call
