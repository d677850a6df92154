"""Synthetic workloads at the benchmark shapes, built with the library itself.

The decode-attention workload is a KV cache for batch B, Hkv KV heads, T
tokens, head_dim d: bf16 K/V drawn N(0,1) with 4 fixed outlier channels per
head scaled x20 (the energy-in-few-dimensions problem the techblog-plum
explainer describes in section "これまでの量子化の限界"), encoded by the
library (keys TurboQuant_mse, values TurboQuant_prod) into packed records, with
the value records also rearranged into the token-tiled layout.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import api, synth

ATTN_SEEDS = {"K": 301, "V": 302, "chan": 303, "q": 304, "piK": 311, "piV": 312, "sV": 313}


@dataclass
class AttnCache:
    kq: api.Quantizer
    vq: api.Quantizer
    piK: np.ndarray
    piV: np.ndarray
    sV: np.ndarray
    kcodes: torch.Tensor
    knorms: torch.Tensor
    vcodes: torch.Tensor
    vnorms: torch.Tensor
    vgammas: torch.Tensor
    vtiles: torch.Tensor
    q_host: np.ndarray
    q: torch.Tensor

    def packed_bytes(self) -> int:
        return int(self.kcodes.numel() + self.knorms.numel() * 2 + self.vtiles.numel() * 4 +
                   self.vnorms.numel() * 2 + self.vgammas.numel() * 2)


def build_attention_cache(B: int, Hq: int, Hkv: int, T: int, d: int, kbits: int = 3, vbits: int = 2,
                          seeds=ATTN_SEEDS, device="cuda") -> AttnCache:
    """Encode synthetic bf16 K/V into packed caches one batch row at a time (bounded temporaries)."""
    piK = synth.haar_rotation(d, seeds["piK"])
    piV = synth.haar_rotation(d, seeds["piV"])
    sV = synth.gaussian_projection(d, seeds["sV"])
    kq = api.Quantizer(d, kbits, api.TQ_MSE, piK)
    vq = api.Quantizer(d, vbits, api.TQ_PROD, piV, sV)
    dev = torch.device(device)
    kcodes = torch.empty((B, Hkv, T, kq.code_bytes), dtype=torch.uint8, device=dev)
    vcodes = torch.empty((B, Hkv, T, vq.code_bytes), dtype=torch.uint8, device=dev)
    knorms = torch.empty((B, Hkv, T), dtype=torch.int16, device=dev)
    vnorms = torch.empty((B, Hkv, T), dtype=torch.int16, device=dev)
    vgam = torch.empty((B, Hkv, T), dtype=torch.int16, device=dev)
    vtiles = torch.empty((B, Hkv, (T + 31) // 32, vq.planes, d), dtype=torch.int32, device=dev)
    chans = synth.outlier_channels(Hkv, d, 4, seeds["chan"])
    for b in range(B):
        k = synth.kv_bf16_torch((1, Hkv, T, d), seeds["K"] * 1000 + b, chans, dev)
        kq.encode(k.view(-1, d), codes=kcodes[b].view(-1, kq.code_bytes), norms=knorms[b].view(-1))
        del k
        v = synth.kv_bf16_torch((1, Hkv, T, d), seeds["V"] * 1000 + b, chans, dev)
        vq.encode(v.view(-1, d), codes=vcodes[b].view(-1, vq.code_bytes), norms=vnorms[b].view(-1),
                  gammas=vgam[b].view(-1))
        del v
        api.tile_records(vq, vcodes[b], out=vtiles[b])
    q_host = synth.round_bf16(np.random.default_rng(seeds["q"]).standard_normal((B, Hq, d)).astype(np.float32))
    q = torch.from_numpy(q_host).to(dev).to(torch.bfloat16)
    torch.cuda.synchronize()
    return AttnCache(kq, vq, piK, piV, sV, kcodes, knorms, vcodes, vnorms, vgam, vtiles, q_host, q)
