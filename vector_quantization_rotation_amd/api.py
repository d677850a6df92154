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


_HALF_BITS = (torch.int16, torch.float16, torch.uint16)  # fp16 bit patterns (norms, gammas)


def _dev(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return t


def _need(t, name: str, dtypes, shape=None, device=None, contiguous: bool = True):
    """Check a tensor handed to the C ABI: on the device, dtype, shape, dense layout.

    The library receives raw pointers and cannot check any of this itself, so a
    wrong tensor would become an out-of-bounds device access; raise instead.
    """
    _dev(t, name)
    if not isinstance(dtypes, tuple):
        dtypes = (dtypes,)
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != expected {tuple(shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t


def _need_rows(t, name: str, dtypes, n: int, width: int, device):
    """[n, >= width] rows with unit stride along a row (row stride may exceed width)."""
    _need(t, name, dtypes, device=device, contiguous=False)
    if t.dim() != 2 or t.shape[0] != n or t.shape[1] < width or (n > 0 and t.stride(1) != 1):
        raise ValueError(f"{name}: expected [{n}, >= {width}] with unit column stride, got shape "
                         f"{tuple(t.shape)} stride {t.stride()}")
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
        _need(x, "x", tuple(_DT), contiguous=False)
        if x.shape[-1] != self.d:
            raise ValueError(f"x: last dimension {x.shape[-1]} != d = {self.d}")
        x2 = x.reshape(-1, x.shape[-1])
        if x2.stride(-1) != 1 or (x2.shape[0] > 1 and (x2.stride(0) * x2.element_size()) % 16 != 0):
            x2 = x2.contiguous()
        n = x2.shape[0]
        dev = x.device
        if codes is None:
            codes = torch.empty((n, self.code_bytes), dtype=torch.uint8, device=dev)
        if norms is None:
            norms = torch.empty((n,), dtype=torch.int16, device=dev)
        _need(codes, "codes", torch.uint8, (n, self.code_bytes), dev)
        _need(norms, "norms", _HALF_BITS, (n,), dev)
        lib = load()
        if self.mode == TQ_MSE:
            rc = lib.tq_encode_mse(self._h, _ptr(x2), _DT[x2.dtype], n, x2.stride(0), _ptr(codes), _ptr(norms), _stream())
            _lib._check("tq_encode_mse", rc)
            return codes, norms, None
        if gammas is None:
            gammas = torch.empty((n,), dtype=torch.int16, device=dev)
        _need(gammas, "gammas", _HALF_BITS, (n,), dev)
        rc = lib.tq_encode_prod(self._h, _ptr(x2), _DT[x2.dtype], n, x2.stride(0), _ptr(codes), _ptr(norms),
                                _ptr(gammas), _stream())
        _lib._check("tq_encode_prod", rc)
        return codes, norms, gammas

    def decode(self, codes: torch.Tensor, norms: torch.Tensor, gammas: torch.Tensor | None = None, out=None):
        """Records [n, code_bytes] (+ fp16-bit norms, gammas [n]) -> fp32 rows [n, d]."""
        _dev(codes, "codes")
        n, dev = codes.shape[0], codes.device
        _need(codes, "codes", torch.uint8, (n, self.code_bytes), dev)
        _need(norms, "norms", _HALF_BITS, (n,), dev)
        if self.mode == TQ_PROD:
            if gammas is None:
                raise ValueError("gammas are required for an Algorithm 2 quantizer")
            _need(gammas, "gammas", _HALF_BITS, (n,), dev)
        if out is None:
            out = torch.empty((n, self.d), dtype=torch.float32, device=dev)
        _need_rows(out, "out", torch.float32, n, self.d, dev)
        rc = load().tq_decode(self._h, _ptr(codes), _ptr(norms), _ptr(gammas), n, _ptr(out), out.stride(0), _stream())
        _lib._check("tq_decode", rc)
        return out

    def score(self, queries: torch.Tensor, codes: torch.Tensor, norms: torch.Tensor, gammas=None, k: int = 0):
        """k == 0: [m, n] scores; k > 0: (values [m, k], indices [m, k]) of the best records per query."""
        lib = load()
        _dev(queries, "queries")
        _dev(codes, "codes")
        m, n, dev = queries.shape[0], codes.shape[0], queries.device
        _need_rows(queries, "queries", torch.float32, m, self.d, dev)
        _need(codes, "codes", torch.uint8, (n, self.code_bytes), dev)
        _need(norms, "norms", _HALF_BITS, (n,), dev)
        if self.mode == TQ_PROD:
            if gammas is None:
                raise ValueError("gammas are required for an Algorithm 2 quantizer")
            _need(gammas, "gammas", _HALF_BITS, (n,), dev)
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
    _dev(codes, "codes")
    if codes.dim() != 3:
        raise ValueError("codes must be [nseq, T, code_bytes]")
    nseq, T = codes.shape[0], codes.shape[1]
    _need(codes, "codes", torch.uint8, (nseq, T, q.code_bytes))
    ntile = (T + 31) // 32
    if out is None:
        out = torch.empty((nseq, ntile, q.planes, q.d), dtype=torch.int32, device=codes.device)
    _need(out, "out", (torch.int32, torch.uint32), (nseq, ntile, q.planes, q.d), codes.device)
    rc = load().tq_tile_records(q.handle, _ptr(codes), nseq, T, _ptr(out), _stream())
    _lib._check("tq_tile_records", rc)
    return out


def encode_cache(q: Quantizer, x: torch.Tensor, codes: torch.Tensor, norms: torch.Tensor, gammas=None, t0: int = 0,
                 layout: int = TQ_LAYOUT_ROWS):
    """Encode x [nseq, T, d] into positions t0 .. t0+T-1 of a cache of Tstride positions per sequence.

    layout TQ_LAYOUT_ROWS: codes uint8 [nseq, Tstride, code_bytes]; TQ_LAYOUT_TILE32: codes int32
    [nseq, ceil(Tstride/32), planes, d] (t0 a multiple of 32).  norms (and gammas for an Algorithm 2
    quantizer) are fp16-bit [nseq, Tstride].  Writes in place; returns (codes, norms, gammas).
    """
    _need(x, "x", tuple(_DT), contiguous=False)
    if x.dim() != 3 or x.shape[-1] != q.d:
        raise ValueError(f"x: expected [nseq, T, {q.d}], got {tuple(x.shape)}")
    nseq, T, dev = x.shape[0], x.shape[1], x.device
    x2 = x.reshape(-1, q.d)
    if x2.stride(-1) != 1 or (x2.shape[0] > 1 and (x2.stride(0) * x2.element_size()) % 16 != 0) or \
            x2.data_ptr() % 16 != 0:
        x2 = x2.contiguous()
    _dev(norms, "norms")
    if norms.dim() != 2 or norms.shape[0] != nseq:
        raise ValueError(f"norms: expected [{nseq}, Tstride], got {tuple(norms.shape)}")
    Tstride = norms.shape[1]
    _need(norms, "norms", _HALF_BITS, (nseq, Tstride), dev)
    if layout == TQ_LAYOUT_TILE32:
        _need(codes, "codes", (torch.int32, torch.uint32), (nseq, (Tstride + 31) // 32, q.planes, q.d), dev)
    elif layout == TQ_LAYOUT_ROWS:
        _need(codes, "codes", torch.uint8, (nseq, Tstride, q.code_bytes), dev)
    else:
        raise ValueError(f"unknown layout {layout}")
    if q.mode == TQ_PROD:
        if gammas is None:
            raise ValueError("gammas are required for an Algorithm 2 quantizer")
        _need(gammas, "gammas", _HALF_BITS, (nseq, Tstride), dev)
    else:
        gammas = None
    rc = load().tq_encode_cache(q.handle, _ptr(x2), _DT[x2.dtype], nseq, T, x2.stride(0), t0, Tstride, layout,
                                _ptr(codes), _ptr(norms), _ptr(gammas), _stream())
    _lib._check("tq_encode_cache", rc)
    return codes, norms, gammas


def attn_decode_ws_bytes(kq: Quantizer, B: int, Hq: int, Hkv: int, Tstride: int, vlayout: int = TQ_LAYOUT_ROWS) -> int:
    return load().tq_attn_decode_ws_bytes(kq.handle, B, Hq, Hkv, Tstride, vlayout)


def _attn_args(kq: Quantizer, vq: Quantizer, q, kcodes, knorms, vcodes, vnorms, vgammas, seq_len, out, vlayout,
               kgammas=None):
    """Check every tensor of a decode-attention call against the shapes the C ABI assumes."""
    _dev(q, "q")
    if q.dim() != 3:
        raise ValueError("q must be [B, Hq, d]")
    B, Hq, d = q.shape
    dev = q.device
    if d != kq.d or d != vq.d:
        raise ValueError(f"q: head dim {d} does not match the quantizers (d = {kq.d}, {vq.d})")
    _need(q, "q", tuple(_DT), device=dev)
    _dev(kcodes, "kcodes")
    if kcodes.dim() != 4:
        raise ValueError("kcodes must be [B, Hkv, Tstride, code_bytes]")
    Hkv, Tstride = kcodes.shape[1], kcodes.shape[2]
    _need(kcodes, "kcodes", torch.uint8, (B, Hkv, Tstride, kq.code_bytes), dev)
    for t, nm in ((knorms, "knorms"), (vnorms, "vnorms"), (vgammas, "vgammas")):
        _need(t, nm, _HALF_BITS, (B, Hkv, Tstride), dev)
    if kq.mode == TQ_PROD:
        if kgammas is None:
            raise ValueError("kgammas are required for Algorithm 2 keys")
        _need(kgammas, "kgammas", _HALF_BITS, (B, Hkv, Tstride), dev)
    if vlayout == TQ_LAYOUT_TILE32:
        _need(vcodes, "vcodes", (torch.int32, torch.uint32), (B, Hkv, (Tstride + 31) // 32, vq.planes, d), dev)
    elif vlayout == TQ_LAYOUT_ROWS:
        _need(vcodes, "vcodes", torch.uint8, (B, Hkv, Tstride, vq.code_bytes), dev)
    else:
        raise ValueError(f"unknown value layout {vlayout}")
    _need(seq_len, "seq_len", torch.int32, (B,), dev)
    if out is not None:
        _need(out, "out", torch.float32, (B, Hq, d), dev)
    return B, Hq, Hkv, Tstride, d, dev


def attn_decode(kq: Quantizer, vq: Quantizer, q: torch.Tensor, kcodes, knorms, vcodes, vnorms, vgammas,
                seq_len: torch.Tensor, scale: float, out=None, ws=None, vlayout: int = TQ_LAYOUT_ROWS, kgammas=None):
    """q [B, Hq, d]; key caches [B, Hkv, Tstride, ...] (kgammas for Algorithm-2 keys); value records in
    `vlayout`; -> out [B, Hq, d] fp32."""
    lib = load()
    B, Hq, Hkv, Tstride, d, dev = _attn_args(kq, vq, q, kcodes, knorms, vcodes, vnorms, vgammas, seq_len, out, vlayout,
                                             kgammas)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    ws_b = lib.tq_attn_decode_ws_bytes(kq.handle, B, Hq, Hkv, Tstride, vlayout)
    if ws is None:
        ws = torch.empty((max(ws_b, 1),), dtype=torch.uint8, device=dev)
    _need(ws, "ws", torch.uint8, device=dev)
    rc = lib.tq_attn_decode(kq.handle, vq.handle, _ptr(q), _DT[q.dtype], B, Hq, Hkv, _ptr(kcodes), _ptr(knorms),
                            _ptr(kgammas), _ptr(vcodes), _ptr(vnorms), _ptr(vgammas), vlayout, Tstride, _ptr(seq_len),
                            float(scale), _ptr(out), _ptr(ws), ws.numel(), _stream())
    _lib._check("tq_attn_decode", rc)
    return out


def attn_prefill(kq: Quantizer, vq: Quantizer, q: torch.Tensor, kcodes, knorms, vcodes, vnorms, vgammas,
                 q_pos: torch.Tensor, scale: float, out=None, ws=None, kgammas=None, vlayout: int = TQ_LAYOUT_ROWS):
    """Causal attention of M query tokens per sequence, q [B, M, Hq, d] (token m at position q_pos[b] + m),
    against the cache that already holds them (value records in `vlayout`) -> out [B, M, Hq, d] fp32."""
    lib = load()
    _dev(q, "q")
    if q.dim() != 4:
        raise ValueError("q must be [B, M, Hq, d]")
    B, M, Hq, d = q.shape
    dev = q.device
    _need(q, "q", tuple(_DT), device=dev)
    _attn_args(kq, vq, q.reshape(B, M * Hq, d), kcodes, knorms, vcodes, vnorms, vgammas, q_pos, None,
               vlayout, kgammas)
    Hkv, Tstride = kcodes.shape[1], kcodes.shape[2]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    if out is None:
        out = torch.empty((B, M, Hq, d), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, (B, M, Hq, d), dev)
    ws_b = lib.tq_attn_prefill_ws_bytes(kq.handle, B, M, Hq, Hkv, Tstride, vlayout)
    if ws is None:
        ws = torch.empty((max(ws_b, 1),), dtype=torch.uint8, device=dev)
    _need(ws, "ws", torch.uint8, device=dev)
    rc = lib.tq_attn_prefill(kq.handle, vq.handle, _ptr(q), _DT[q.dtype], B, M, Hq, Hkv, _ptr(kcodes), _ptr(knorms),
                             _ptr(kgammas), _ptr(vcodes), _ptr(vnorms), _ptr(vgammas), vlayout, Tstride,
                             _ptr(q_pos), float(scale), _ptr(out), _ptr(ws), ws.numel(), _stream())
    _lib._check("tq_attn_prefill", rc)
    return out


def attn_decode_append(kq: Quantizer, vq: Quantizer, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                       kcodes, knorms, vcodes, vnorms, vgammas, seq_len: torch.Tensor, scale: float, out=None,
                       ws=None, vlayout: int = TQ_LAYOUT_ROWS, kgammas=None):
    """One decode step with the new token appended: k_new, v_new [B, Hkv, d] are encoded into the cache at
    position seq_len[b] (the cache tensors are written in place) and the step attends over seq_len[b] + 1
    tokens.  seq_len is only read: advance it before the next step.  -> out [B, Hq, d] fp32."""
    lib = load()
    B, Hq, Hkv, Tstride, d, dev = _attn_args(kq, vq, q, kcodes, knorms, vcodes, vnorms, vgammas, seq_len, out, vlayout,
                                             kgammas)
    _need(k_new, "k_new", tuple(_DT), (B, Hkv, d), dev)
    _need(v_new, "v_new", (k_new.dtype,), (B, Hkv, d), dev)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    ws_b = lib.tq_attn_decode_ws_bytes(kq.handle, B, Hq, Hkv, Tstride, vlayout)
    if ws is None:
        ws = torch.empty((max(ws_b, 1),), dtype=torch.uint8, device=dev)
    _need(ws, "ws", torch.uint8, device=dev)
    rc = lib.tq_attn_decode_append(kq.handle, vq.handle, _ptr(q), _DT[q.dtype], B, Hq, Hkv, _ptr(k_new), _ptr(v_new),
                                   _DT[k_new.dtype], _ptr(kcodes), _ptr(knorms), _ptr(kgammas), _ptr(vcodes),
                                   _ptr(vnorms), _ptr(vgammas), vlayout, Tstride, _ptr(seq_len), float(scale),
                                   _ptr(out), _ptr(ws), ws.numel(), _stream())
    _lib._check("tq_attn_decode_append", rc)
    return out


def attn_decode_noalloc(kq: Quantizer, vq: Quantizer, q: torch.Tensor, kcodes, knorms, vcodes, vnorms, vgammas,
                        seq_len: torch.Tensor, scale: float, out: torch.Tensor, vlayout: int = TQ_LAYOUT_ROWS,
                        kgammas=None):
    """attn_decode through tq_attn_decode_noalloc: no device allocation anywhere in the call (out is
    the caller's); the workspace is the library's fixed per-GPU array of TQ_NOALLOC_SCRATCH_BYTES.
    Calls that overlap on one GPU race on that array."""
    lib = load()
    B, Hq, Hkv, Tstride, d, dev = _attn_args(kq, vq, q, kcodes, knorms, vcodes, vnorms, vgammas, seq_len, out, vlayout,
                                             kgammas)
    if out is None:
        raise ValueError("out is required (the call allocates nothing)")
    need = lib.tq_attn_decode_ws_bytes(kq.handle, B, Hq, Hkv, Tstride, vlayout)
    if need > _lib.TQ_NOALLOC_SCRATCH_BYTES:
        raise ValueError(f"this call needs {need} bytes of workspace; the no-allocation entry point holds "
                         f"{_lib.TQ_NOALLOC_SCRATCH_BYTES}")
    rc = lib.tq_attn_decode_noalloc(kq.handle, vq.handle, _ptr(q), _DT[q.dtype], B, Hq, Hkv, _ptr(kcodes),
                                    _ptr(knorms), _ptr(kgammas), _ptr(vcodes), _ptr(vnorms), _ptr(vgammas), vlayout,
                                    Tstride, _ptr(seq_len), float(scale), _ptr(out), _stream())
    _lib._check("tq_attn_decode_noalloc", rc)
    return out


def attn_decode_bound(kq: Quantizer, vq: Quantizer, q: torch.Tensor, kcodes, knorms, vcodes, vnorms, vgammas,
                      seq_len: torch.Tensor, scale: float, out: torch.Tensor, ws: torch.Tensor,
                      vlayout: int = TQ_LAYOUT_ROWS, kgammas=None):
    """attn_decode with every argument checked and marshalled once: returns a no-argument
    callable that enqueues the same call on the stream that is current when it is called
    (for tight decode loops).  The callable holds references to every tensor it reads or
    writes, so they stay alive as long as it does."""
    lib = load()
    B, Hq, Hkv, Tstride, d, dev = _attn_args(kq, vq, q, kcodes, knorms, vcodes, vnorms, vgammas, seq_len, out, vlayout,
                                             kgammas)
    if out is None:
        raise ValueError("out is required")
    _need(ws, "ws", torch.uint8, device=dev)
    need = lib.tq_attn_decode_ws_bytes(kq.handle, B, Hq, Hkv, Tstride, vlayout)
    if ws.numel() < need:
        raise ValueError(f"ws holds {ws.numel()} bytes, the call needs {need}")
    keep = (kq, vq, q, kcodes, knorms, kgammas, vcodes, vnorms, vgammas, seq_len, out, ws)
    args = (kq.handle, vq.handle, _ptr(q), _DT[q.dtype], B, Hq, Hkv, _ptr(kcodes), _ptr(knorms), _ptr(kgammas),
            _ptr(vcodes), _ptr(vnorms), _ptr(vgammas), vlayout, Tstride, _ptr(seq_len), C.c_float(scale), _ptr(out),
            _ptr(ws), C.c_size_t(ws.numel()))
    fn = lib.tq_attn_decode

    def call():
        rc = fn(*args, _stream())
        if rc != 0:
            _lib._check("tq_attn_decode", rc)
    call.tensors = keep
    return call
