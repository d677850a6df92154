"""Synthetic workloads at the benchmark shapes, built with the library itself.

The decode-attention workload is a KV cache for batch B, Hkv KV heads, T
tokens, head_dim d: bf16 K/V drawn N(0,1) with 4 fixed outlier channels per
head scaled x20 (the energy-in-few-dimensions problem the techblog-plum
explainer describes in section "これまでの量子化の限界"), encoded by the
library (keys TurboQuant_mse, values TurboQuant_prod) into packed records, with
the value records also rearranged into the token-tiled layout.

The heterogeneous-layer workload follows the interleaved local/global layer
shapes of the Gemma 4 post (section "KV形状の不均一性"): local layers with 16
KV heads of head_dim 256 over a 1024-token sliding window, global layers with 4
KV heads of head_dim 512 over 65536 tokens, batch 4, 32 query heads, bf16
N(0,1) with 4 heavy-tailed (Student-t, nu = 3) channels per head, per-shape
rotations and codebooks.

The search workload is the inner-product retrieval use of the AiBoss overview
(section "TurboQuantの応用事例"): 10^6 database vectors of dimension 1536 drawn
from 1024 Gaussian clusters (centres N(0,1), spread 0.3) and L2-normalised,
TurboQuant_prod 4-bit, 1000 queries from the same law.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import api, synth

ATTN_SEEDS = {"K": 301, "V": 302, "chan": 303, "q": 304, "piK": 311, "piV": 312, "sV": 313}

# heterogeneous layers: (B, Hq, Hkv, T, d) and seeds per layer kind
HET_LAYERS = {
    "local": dict(B=4, Hq=32, Hkv=16, T=1024, d=256,
                  seeds={"K": 401, "V": 402, "chan": 403, "q": 404, "piK": 405, "piV": 406, "sV": 407}),
    "global": dict(B=4, Hq=32, Hkv=4, T=65536, d=512,
                   seeds={"K": 411, "V": 412, "chan": 413, "q": 414, "piK": 415, "piV": 416, "sV": 417}),
}
HET_NU = 3.0

# search: database, queries, quantizer
SEARCH = dict(n=1_000_000, d=1536, centers=1024, sigma=0.3, queries=1000, bits=4, k=10,
              seeds={"centers": 501, "assign": 502, "noise": 503, "q_assign": 504, "q_noise": 505,
                     "pi": 511, "s": 512})


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
                          seeds=ATTN_SEEDS, device="cuda", student_t_nu: float | None = None,
                          tiles: bool = True) -> AttnCache:
    """Encode synthetic bf16 K/V into packed caches one batch row at a time (bounded temporaries).

    student_t_nu: heavy-tailed outlier channels instead of the x20 scaling; tiles: also build the
    token-tiled value words (the layout the head_dim <= 256 attention kernels read)."""
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
    vtiles = torch.empty((B, Hkv, (T + 31) // 32 if tiles else 0, vq.planes, d), dtype=torch.int32, device=dev)
    chans = synth.outlier_channels(Hkv, d, 4, seeds["chan"])
    for b in range(B):
        k = synth.kv_bf16_torch((1, Hkv, T, d), seeds["K"] * 1000 + b, chans, dev, student_t_nu=student_t_nu)
        kq.encode(k.view(-1, d), codes=kcodes[b].view(-1, kq.code_bytes), norms=knorms[b].view(-1))
        del k
        v = synth.kv_bf16_torch((1, Hkv, T, d), seeds["V"] * 1000 + b, chans, dev, student_t_nu=student_t_nu)
        vq.encode(v.view(-1, d), codes=vcodes[b].view(-1, vq.code_bytes), norms=vnorms[b].view(-1),
                  gammas=vgam[b].view(-1))
        del v
        if tiles:
            api.tile_records(vq, vcodes[b], out=vtiles[b])
    q_host = synth.round_bf16(np.random.default_rng(seeds["q"]).standard_normal((B, Hq, d)).astype(np.float32))
    q = torch.from_numpy(q_host).to(dev).to(torch.bfloat16)
    torch.cuda.synchronize()
    return AttnCache(kq, vq, piK, piV, sV, kcodes, knorms, vcodes, vnorms, vgam, vtiles, q_host, q)


def raw_kv_slice(which: str, b: int, g: int, Hkv: int, T: int, d: int, seeds=ATTN_SEEDS,
                 student_t_nu: float | None = None, device="cuda") -> np.ndarray:
    """The raw bf16 K or V rows (as fp32) of (batch b, kv-head g) that build_attention_cache encoded,
    regenerated from the same seeds."""
    chans = synth.outlier_channels(Hkv, d, 4, seeds["chan"])
    x = synth.kv_bf16_torch((1, Hkv, T, d), seeds[which] * 1000 + b, chans, device, student_t_nu=student_t_nu)
    out = x[0, g].float().cpu().numpy()
    del x
    return out


def het_layer_cache(kind: str, device="cuda") -> AttnCache:
    L = HET_LAYERS[kind]
    return build_attention_cache(L["B"], L["Hq"], L["Hkv"], L["T"], L["d"], 3, 2, seeds=L["seeds"], device=device,
                                 student_t_nu=HET_NU, tiles=True)


def search_database(device="cuda") -> torch.Tensor:
    """The search database [n, d] fp32 on the device."""
    S = SEARCH
    sd = S["seeds"]
    return synth.clustered_database_torch(S["n"], S["d"], S["centers"], S["sigma"], sd["centers"], sd["assign"],
                                          sd["noise"], device)


def search_queries() -> np.ndarray:
    """The search queries [m, d] fp32 (host): same cluster law, new assignments and noise."""
    S = SEARCH
    sd = S["seeds"]
    return synth.clustered_database(S["queries"], S["d"], S["centers"], S["sigma"], sd["centers"], sd["q_assign"],
                                    sd["q_noise"])
