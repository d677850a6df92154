"""Benchmark of the TurboQuant hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]

A timed step is one decode-attention pass over a compressed KV cache
(query rotation, the split-sequence scoring/aggregation kernel and the
combine/rotate-back kernel): batch 16, 32 query heads over 8 KV heads,
head_dim 128, 131072 cached tokens per sequence, keys TurboQuant_mse 3-bit,
values TurboQuant_prod 2-bit.  The cache is built beforehand by the library's
own encode from synthetic bf16 K/V (N(0,1), 4 fixed outlier channels per head
scaled x20) and is resident in HBM when timing starts.  `value` is packed-KV
bytes streamed per second.  In the same run the encode throughput
(vectors/s) is measured on one layer's cache (batch 8, 8 KV heads, 32768
tokens, head_dim 128; keys mse 3-bit, values prod 3-bit), and the CPU oracle
is timed on a bounded sample of the attention workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0   # dense MFMA, MI355X
INT8_PEAK_TOPS = 5000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-slices", type=int, default=64, help="(batch, kv-head) slices the oracle times")
    ap.add_argument("--cpu-encode-rows", type=int, default=524288, help="rows per kind the oracle encodes")
    ap.add_argument("--only", choices=["", "encode", "attention", "global", "global_encode", "prefill", "search"],
                    default="",
                    help="a short run of one part (for counter profiles): the one-layer encode, the timed "
                         "attention steps, the global-layer attention steps, the global-layer encode, the "
                         "chunked prefill over token-tiled values, or the search scan")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain 1 GiB device copy (the reference for HBM byte counters)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_wave_kernel_traffic.md")
ATTN_SRC = os.path.join(ROOT, "vector_quantization_rotation_amd", "csrc", "attn_fast.hip")


def measured_traffic():
    """HBM bytes per launch of the attention kernel from the committed counter summary,
    or None when the kernel source changed since the counters were taken."""
    import hashlib
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    kv = {}
    for line in text.splitlines():
        if line.startswith("- ") and ": " in line:
            k, v = line[2:].split(": ", 1)
            kv[k.strip()] = v.strip().strip("`")
    src = hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()
    if kv.get("attn_fast.hip sha256") != src or "traffic bytes per launch" not in kv:
        return None
    return int(kv["traffic bytes per launch"])


def encode_only(steps: int):
    """The one-layer encode workload (keys Algorithm 1 3-bit, values Algorithm 2 3-bit, 2 x 2^21 bf16 rows of
    d 128) run `steps` times, then the decode of the value records to fp32 rows `steps` times, for profiles of
    the encode and decode kernels; prints one JSON line."""
    import torch
    from vector_quantization_rotation_amd import api, synth
    d, eB, eH, eT = 128, 8, 8, 32768
    ch = synth.outlier_channels(eH, d, 4, 203)
    K = synth.kv_bf16_torch((eB, eH, eT, d), 201, ch, "cuda").view(-1, d)
    V = synth.kv_bf16_torch((eB, eH, eT, d), 202, ch, "cuda").view(-1, d)
    kq = api.Quantizer(d, 3, api.TQ_MSE, synth.haar_rotation(d, 211))
    vq = api.Quantizer(d, 3, api.TQ_PROD, synth.haar_rotation(d, 212), synth.gaussian_projection(d, 213))
    kc, kn, _ = kq.encode(K)
    vc, vn, vg = vq.encode(V)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        kq.encode(K, codes=kc, norms=kn)
        vq.encode(V, codes=vc, norms=vn, gammas=vg)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    del K
    dec = torch.empty((V.shape[0], d), dtype=torch.float32, device="cuda")
    del V
    vq.decode(vc, vn, vg, out=dec)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        vq.decode(vc, vn, vg, out=dec)
    torch.cuda.synchronize()
    ddt = (time.perf_counter() - t0) / steps
    print(json.dumps({"encode": {"ms": round(dt * 1e3, 4), "vectors": 2 * kc.shape[0],
                                 "value": round(2 * kc.shape[0] / dt, 1), "unit": "vectors/s"},
                      "decode": {"ms": round(ddt * 1e3, 4), "vectors": dec.shape[0],
                                 "value": round(dec.shape[0] / ddt, 1), "unit": "vectors/s"}}), flush=True)


def copy_calibration():
    """A plain streaming kernel of known size (reads 1 GiB, writes 1 GiB), run three times: its FETCH_SIZE
    and WRITE_SIZE in a counter profile calibrate the HBM byte counters."""
    import torch
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.add(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst


def global_only(steps: int, warmup: int, calib: bool = False):
    """The global-layer decode attention (batch 4, 32 query heads over 4 KV heads, head_dim 512, 65536
    tokens) run warmup + steps times, for counter profiles; prints one JSON line."""
    import torch
    from vector_quantization_rotation_amd import api, workloads
    L = workloads.HET_LAYERS["global"]
    hB, hHq, hHkv, hT, hd = L["B"], L["Hq"], L["Hkv"], L["T"], L["d"]
    hc = workloads.het_layer_cache("global")
    lay = api.TQ_LAYOUT_TILE32
    hseq = torch.full((hB,), hT, dtype=torch.int32, device="cuda")
    hout = torch.empty((hB, hHq, hd), dtype=torch.float32, device="cuda")
    hws = torch.empty((api.attn_decode_ws_bytes(hc.kq, hB, hHq, hHkv, hT, lay),), dtype=torch.uint8, device="cuda")
    step = api.attn_decode_bound(hc.kq, hc.vq, hc.q, hc.kcodes, hc.knorms, hc.vtiles, hc.vnorms, hc.vgammas, hseq,
                                 1 / math.sqrt(hd), hout, hws, vlayout=lay)
    if calib:
        copy_calibration()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    pk = hc.packed_bytes()
    print(json.dumps({"global_attention": {"ms_per_step": round(dt * 1e3, 5), "packed_bytes": pk,
                                           "gbs": round(pk / dt / 1e9, 2)}}), flush=True)


def global_encode_only(steps: int):
    """The global-layer encode (keys mse 3-bit and values prod 2-bit of batch 4 x 4 KV heads x 65536 tokens,
    head_dim 512, bf16 rows: the GEMM path) run steps times, for counter profiles; prints one JSON line."""
    import torch
    from vector_quantization_rotation_amd import api, synth, workloads
    L = workloads.HET_LAYERS["global"]
    hB, hHkv, hT, hd = L["B"], L["Hkv"], L["T"], L["d"]
    hch = synth.outlier_channels(hHkv, hd, 4, L["seeds"]["chan"])
    Kr = synth.kv_bf16_torch((hB, hHkv, hT, hd), L["seeds"]["K"], hch, "cuda", student_t_nu=workloads.HET_NU).view(-1, hd)
    Vr = synth.kv_bf16_torch((hB, hHkv, hT, hd), L["seeds"]["V"], hch, "cuda", student_t_nu=workloads.HET_NU).view(-1, hd)
    kq = api.Quantizer(hd, 3, api.TQ_MSE, synth.haar_rotation(hd, L["seeds"]["piK"]))
    vq = api.Quantizer(hd, 2, api.TQ_PROD, synth.haar_rotation(hd, L["seeds"]["piV"]),
                       synth.gaussian_projection(hd, L["seeds"]["sV"]))
    n = Kr.shape[0]
    kc = torch.empty((n, kq.code_bytes), dtype=torch.uint8, device="cuda")
    vc = torch.empty((n, vq.code_bytes), dtype=torch.uint8, device="cuda")
    kn, vn, vg = (torch.empty((n,), dtype=torch.int16, device="cuda") for _ in range(3))
    times = []
    for _ in range(steps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        kq.encode(Kr, codes=kc, norms=kn)
        vq.encode(Vr, codes=vc, norms=vn, gammas=vg)
        torch.cuda.synchronize()
        times.append(time.perf_counter() - t0)
    print(json.dumps({"global_encode": {"ms": [round(t * 1e3, 3) for t in times], "vectors": 2 * n}}), flush=True)


def prefill_only(steps: int):
    """The chunked prefill of the benchmark (512 causal query tokens x 32 heads over 8 KV heads, head_dim 128,
    against a 4096-token cache, token-tiled values) run steps times, for kernel traces; prints one JSON line."""
    import torch
    from vector_quantization_rotation_amd import _lib, api, workloads
    Hq, Hkv, d = 32, 8, 128
    pB, pM, pT = 1, 512, 4096
    pc = workloads.build_attention_cache(pB, Hq, Hkv, pT, d, tiles=True)
    pq = torch.randn((pB, pM, Hq, d), generator=torch.Generator("cuda").manual_seed(721), device="cuda").to(torch.bfloat16)
    qpos = torch.full((pB,), pT - pM, dtype=torch.int32, device="cuda")
    pout = torch.empty((pB, pM, Hq, d), dtype=torch.float32, device="cuda")
    ws = torch.empty((_lib.load().tq_attn_prefill_ws_bytes(pc.kq.handle, pB, pM, Hq, Hkv, pT, 1),), dtype=torch.uint8,
                     device="cuda")
    times = []
    for _ in range(steps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        api.attn_prefill(pc.kq, pc.vq, pq, pc.kcodes, pc.knorms, pc.vtiles, pc.vnorms, pc.vgammas, qpos,
                         1 / math.sqrt(d), out=pout, ws=ws, vlayout=api.TQ_LAYOUT_TILE32)
        torch.cuda.synchronize()
        times.append(time.perf_counter() - t0)
    print(json.dumps({"prefill": {"ms": [round(t * 1e3, 3) for t in times], "query_tokens": pB * pM}}), flush=True)


def search_only(steps: int):
    """The search workload (10^6 records of d 1536, prod 4-bit, 1000 queries, top-10): encode once, then the
    scan + top-k `steps` times, for counter profiles; prints one JSON line."""
    import torch
    from vector_quantization_rotation_amd import _lib, api, synth, workloads
    SS = workloads.SEARCH
    X = workloads.search_database()
    sq = api.Quantizer(SS["d"], SS["bits"], api.TQ_PROD, synth.haar_rotation(SS["d"], SS["seeds"]["pi"]),
                       synth.gaussian_projection(SS["d"], SS["seeds"]["s"]))
    sc, sn, sg = sq.encode(X)
    del X
    torch.cuda.empty_cache()
    Qs = torch.from_numpy(workloads.search_queries()).cuda()
    sq.score(Qs, sc, sn, sg, k=SS["k"])
    torch.cuda.synchronize()
    _lib.profile_reset()
    _lib.profile_select("score_scan")
    _lib.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(steps):
        sq.score(Qs, sc, sn, sg, k=SS["k"])
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    _lib.profile_enable(False)
    _lib.profile_select("")
    scan_ms, scan_n = _lib.profile_query("score_scan")
    print(json.dumps({"search": {"scan_topk_ms": round(dt * 1e3, 4),
                                 "scan_kernel_ms": round(scan_ms / max(scan_n, 1), 4)}}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the multi-GPU sharding of this "
              f"path is a design note, not a measured configuration.", file=sys.stderr)
        sys.exit(2)
    import torch

    from vector_quantization_rotation_amd import _lib, api, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    api.load()
    torch.cuda.set_device(0)
    if args.only == "encode":
        encode_only(args.steps)
        return
    if args.only == "global":
        global_only(args.steps, args.warmup, args.copy_calib)
        return
    if args.only == "global_encode":
        global_encode_only(args.steps)
        return
    if args.only == "prefill":
        prefill_only(args.steps)
        return
    if args.only == "search":
        search_only(args.steps)
        return

    # ---------------- decode attention (timed steps) ----------------
    from vector_quantization_rotation_amd import workloads
    B, Hq, Hkv, d, T = 16, 32, 8, 128, 131072
    log("building compressed cache ...")
    t0 = time.time()
    cache = workloads.build_attention_cache(B, Hq, Hkv, T, d)
    log(f"cache built in {time.time() - t0:.1f}s")
    kq, vq = cache.kq, cache.vq
    kc, kn, vc, vn, vg, vt = cache.kcodes, cache.knorms, cache.vcodes, cache.vnorms, cache.vgammas, cache.vtiles
    qh, q = cache.q_host, cache.q
    mats = (cache.piK, cache.piV, cache.sV)
    seq = torch.full((B,), T, dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(d)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    layout = api.TQ_LAYOUT_TILE32
    ws = torch.empty((api.attn_decode_ws_bytes(kq, B, Hq, Hkv, T, layout),), dtype=torch.uint8, device="cuda")
    packed = cache.packed_bytes()

    step = api.attn_decode_bound(kq, vq, q, kc, kn, vt, vn, vg, seq, scale, out, ws, vlayout=layout)

    if args.copy_calib:
        copy_calibration()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed region: HIP events around the dominant kernel only, on every fourth step (i % 4 == 2, spread
    # over the region so the clock's drift under sustained load is sampled evenly; every step when fewer
    # than three): an event-stamped launch stands a few microseconds apart from its neighbours, so events
    # on every step would add about 3 % to the step's wall time
    sampled = [i for i in range(args.steps) if i % 4 == 2] if args.steps >= 3 else list(range(args.steps))
    _lib.profile_reset()
    _lib.profile_select("attn_wave")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        on = i in sampled
        if on:
            _lib.profile_enable(True)
        step()
        if on:
            _lib.profile_enable(False)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    _lib.profile_enable(False)
    split_ms, split_n = _lib.profile_query("attn_wave")
    kernel_name = "attn_wave_kernel<3>"
    if split_n == 0:  # the 4-wave kernel ran (a shape the wave-streaming kernel does not take)
        kernel_name = "attn_fast_kernel<128,3,1>"
        _lib.profile_reset()
        _lib.profile_select("attn_fast")
        _lib.profile_enable(True)
        for _ in range(3):
            step()
        torch.cuda.synchronize()
        _lib.profile_enable(False)
        split_ms, split_n = _lib.profile_query("attn_fast")
    # every kernel of the step, from a short pass outside the timed region
    _lib.profile_select("")
    _lib.profile_reset()
    _lib.profile_enable(True)
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    _lib.profile_enable(False)
    all_ms, _ = _lib.profile_query("attn_")
    all_ms *= args.steps / 3
    ms_per_step = dt * 1e3 / args.steps
    value = packed / (ms_per_step * 1e-3) / 1e9
    kernel_ms = split_ms / max(split_n, 1)
    achieved = packed / (kernel_ms * 1e-3) / 1e9
    log(f"attention: {ms_per_step:.4f} ms/step, {value:.1f} GB/s; {kernel_name} {kernel_ms:.4f} ms "
        f"({achieved:.1f} GB/s); attn kernels total {all_ms / args.steps:.4f} ms/step (untimed pass)")
    out_gpu = out.cpu().numpy()
    if args.only == "attention":
        print(json.dumps({"attention": {"ms_per_step": round(ms_per_step, 5), "value": round(value, 2),
                                        "kernel": kernel_name, "kernel_ms": round(kernel_ms, 5)}}), flush=True)
        return

    # ---------------- encode throughput (one layer's cache) ----------------
    eB, eH, eT = 8, 8, 32768
    echans = synth.outlier_channels(eH, d, 4, 203)
    Ke = synth.kv_bf16_torch((eB, eH, eT, d), 201, echans, "cuda").view(-1, d)
    Ve = synth.kv_bf16_torch((eB, eH, eT, d), 202, echans, "cuda").view(-1, d)
    ekq = api.Quantizer(d, 3, api.TQ_MSE, synth.haar_rotation(d, 211))
    evq = api.Quantizer(d, 3, api.TQ_PROD, synth.haar_rotation(d, 212), synth.gaussian_projection(d, 213))
    nvec = Ke.shape[0]
    ek = (torch.empty((nvec, ekq.code_bytes), dtype=torch.uint8, device="cuda"), torch.empty((nvec,), dtype=torch.int16, device="cuda"))
    ev = (torch.empty((nvec, evq.code_bytes), dtype=torch.uint8, device="cuda"), torch.empty((nvec,), dtype=torch.int16, device="cuda"),
          torch.empty((nvec,), dtype=torch.int16, device="cuda"))

    def enc():
        ekq.encode(Ke, codes=ek[0], norms=ek[1])
        evq.encode(Ve, codes=ev[0], norms=ev[1], gammas=ev[2])

    enc()
    torch.cuda.synchronize()
    esteps = 5
    _lib.profile_reset()
    _lib.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(esteps):
        enc()
    torch.cuda.synchronize()
    edt = (time.perf_counter() - t0) / esteps
    _lib.profile_enable(False)
    enc_mse_ms, enc_mse_n = _lib.profile_query("encode_mse")
    enc_prod_ms, enc_prod_n = _lib.profile_query("encode_prod")
    enc_bytes = 2 * nvec * d * 2 + ek[0].numel() + 2 * nvec + ev[0].numel() + 4 * nvec
    enc_vps = 2 * nvec / edt
    # matrix-core work the fused kernels execute on bf16 rows: fp16 operands, 2 products per rotation
    # (the row against the two pieces of the matrix), 3 per QJL projection of the two-piece residual
    # (d x d each), 2 flop per product term
    enc_flop_exec = 2.0 * nvec * d * d * (2 + 2 + 3)
    enc_flop_useful = 2.0 * nvec * d * d * (1 + 1 + 1)  # one pass per rotation / projection
    enc_hbm_ms = enc_bytes / (HBM_PEAK_GBS * 1e9) * 1e3
    enc_mfma_ms = enc_flop_exec / (BF16_PEAK_TFLOPS * 1e12) * 1e3
    log(f"encode: {edt * 1e3:.3f} ms for {2 * nvec} vectors = {enc_vps:.3e} vectors/s, {enc_bytes / edt / 1e9:.1f} GB/s; "
        f"kernels mse {enc_mse_ms / max(enc_mse_n, 1):.4f} ms, prod {enc_prod_ms / max(enc_prod_n, 1):.4f} ms")
    # the values straight into a token-tiled cache (the layout the attention kernels stream)
    vt_cache = torch.empty((eB * eH, eT // 32, evq.planes, d), dtype=torch.int32, device="cuda")
    vt_n = torch.empty((eB * eH, eT), dtype=torch.int16, device="cuda")
    vt_g = torch.empty((eB * eH, eT), dtype=torch.int16, device="cuda")
    V3 = Ve.view(eB * eH, eT, d)
    api.encode_cache(evq, V3, vt_cache, vt_n, vt_g, t0=0, layout=api.TQ_LAYOUT_TILE32)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(esteps):
        api.encode_cache(evq, V3, vt_cache, vt_n, vt_g, t0=0, layout=api.TQ_LAYOUT_TILE32)
    torch.cuda.synchronize()
    etile_ms = (time.perf_counter() - t0) / esteps * 1e3
    log(f"encode into the tiled value cache: {etile_ms:.4f} ms for {nvec} prod 3-bit vectors (row records: "
        f"{enc_prod_ms / max(enc_prod_n, 1):.4f} ms kernel)")
    del Ke, Ve, V3, vt_cache, vt_n, vt_g

    # ---------------- decode (Algorithm 2 records of the same layer) ----------------
    dec_out = torch.empty((nvec, d), dtype=torch.float32, device="cuda")
    evq.decode(ev[0], ev[1], ev[2], out=dec_out)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(3):
        evq.decode(ev[0], ev[1], ev[2], out=dec_out)
    torch.cuda.synchronize()
    ddt = (time.perf_counter() - t0) / 3
    decode = {"value": round(nvec / ddt, 1), "unit": "vectors/s", "ms": round(ddt * 1e3, 4),
              "workload": f"{nvec} prod 3-bit records, d{d}, to fp32 rows"}
    log(f"decode: {ddt * 1e3:.3f} ms for {nvec} vectors = {nvec / ddt:.3e} vectors/s")
    del dec_out, ek, ev

    def timed(fn, reps=3):
        fn()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t) / reps

    # ---------------- heterogeneous layers (local / global), encode + decode attention ----------------
    het = {}
    for kind in ("local", "global"):
        L = workloads.HET_LAYERS[kind]
        hB, hHq, hHkv, hT, hd = L["B"], L["Hq"], L["Hkv"], L["T"], L["d"]
        hc = workloads.het_layer_cache(kind)
        hch = synth.outlier_channels(hHkv, hd, 4, L["seeds"]["chan"])
        Kr = synth.kv_bf16_torch((hB, hHkv, hT, hd), L["seeds"]["K"], hch, "cuda", student_t_nu=workloads.HET_NU).view(-1, hd)
        Vr = synth.kv_bf16_torch((hB, hHkv, hT, hd), L["seeds"]["V"], hch, "cuda", student_t_nu=workloads.HET_NU).view(-1, hd)
        hn = Kr.shape[0]
        kco, kno = torch.empty_like(hc.kcodes).view(hn, -1), torch.empty_like(hc.knorms).view(-1)
        vco, vno, vgo = torch.empty_like(hc.vcodes).view(hn, -1), torch.empty_like(hc.vnorms).view(-1), torch.empty_like(hc.vgammas).view(-1)
        het_enc = timed(lambda: (hc.kq.encode(Kr, codes=kco, norms=kno), hc.vq.encode(Vr, codes=vco, norms=vno, gammas=vgo)))
        del Kr, Vr, kco, kno, vco, vno, vgo
        tiled = hc.vtiles.shape[2] > 0
        hl = api.TQ_LAYOUT_TILE32 if tiled else api.TQ_LAYOUT_ROWS
        hseq = torch.full((hB,), hT, dtype=torch.int32, device="cuda")
        hout = torch.empty((hB, hHq, hd), dtype=torch.float32, device="cuda")
        hws = torch.empty((api.attn_decode_ws_bytes(hc.kq, hB, hHq, hHkv, hT, hl),), dtype=torch.uint8, device="cuda")
        hstep = api.attn_decode_bound(hc.kq, hc.vq, hc.q, hc.kcodes, hc.knorms, hc.vtiles if tiled else hc.vcodes,
                                      hc.vnorms, hc.vgammas, hseq, 1 / math.sqrt(hd), hout, hws, vlayout=hl)
        het_att = timed(hstep, reps=10)
        hpk = hc.packed_bytes() if tiled else int(hc.kcodes.numel() + hc.vcodes.numel() + 2 * (hc.knorms.numel() + hc.vnorms.numel() + hc.vgammas.numel()))
        het[kind] = {"shape": {"batch": hB, "q_heads": hHq, "kv_heads": hHkv, "seq_len": hT, "head_dim": hd},
                     "encode_ms": round(het_enc * 1e3, 4), "encode_vectors_per_s": round(2 * hn / het_enc, 1),
                     "attn_ms": round(het_att * 1e3, 4), "attn_packed_bytes": hpk,
                     "attn_gbs": round(hpk / het_att / 1e9, 2),
                     "attn_kernel": ("attn_wide8_kernel" if hd == 512 and hHq == 8 * hHkv else "attn_wide_kernel" if hd == 512
                                    else "attn_fast_kernel") + " (token-tiled values)"
                     if tiled else "attn_split_kernel (row records)"}
        log(f"{kind} layer: encode {het_enc * 1e3:.3f} ms ({2 * hn} vectors), attention {het_att * 1e3:.4f} ms "
            f"({hpk / het_att / 1e9:.1f} GB/s)")
        del hc, hout, hws
        torch.cuda.empty_cache()

    # ---------------- search: encode the database, scan + top-10 ----------------
    SS = workloads.SEARCH
    X = workloads.search_database()
    sq = api.Quantizer(SS["d"], SS["bits"], api.TQ_PROD, synth.haar_rotation(SS["d"], SS["seeds"]["pi"]),
                       synth.gaussian_projection(SS["d"], SS["seeds"]["s"]))
    sc = torch.empty((SS["n"], sq.code_bytes), dtype=torch.uint8, device="cuda")
    sn = torch.empty((SS["n"],), dtype=torch.int16, device="cuda")
    sg = torch.empty((SS["n"],), dtype=torch.int16, device="cuda")
    s_enc = timed(lambda: sq.encode(X, codes=sc, norms=sn, gammas=sg))
    Qh = workloads.search_queries()
    Qs = torch.from_numpy(Qh).cuda()
    # exact top-k of sampled queries by fp64 inner products over every row (for recall@k)
    rq = np.sort(np.random.default_rng(13).choice(SS["queries"], size=16, replace=False))
    exact = (Qs[torch.as_tensor(rq, device="cuda")].double() @ X.double().T)
    ex_idx = torch.topk(exact, SS["k"], dim=1).indices.cpu().numpy()
    del X, exact
    torch.cuda.empty_cache()
    s_scan = timed(lambda: sq.score(Qs, sc, sn, sg, k=SS["k"]))
    _lib.profile_reset()
    _lib.profile_select("score_scan")
    _lib.profile_enable(True)
    _, s_idx = sq.score(Qs, sc, sn, sg, k=SS["k"])
    torch.cuda.synchronize()
    _lib.profile_enable(False)
    _lib.profile_select("")
    scan_ms, scan_n = _lib.profile_query("score_scan")
    scan_ms /= max(scan_n, 1)
    got = s_idx.cpu().numpy()[rq]
    recall = float(np.mean([len(set(got[i]) & set(ex_idx[i])) / SS["k"] for i in range(len(rq))]))
    s_bytes = int(sc.numel() + 4 * SS["n"])
    # int8 matrix-core work of the scan kernel: per (32 queries x 256 records) tile and 64 coordinates,
    # 5 images x 16 MFMAs of 16x16x64 per wave (2 digit rows per query), four waves; useful work: one
    # multiply-add per (query, row, coordinate) on each of the 4 bit planes
    scan_ops_exec = (SS["queries"] / 32) * (SS["n"] / 256) * (SS["d"] / 64) * 5 * 4 * 16 * (2 * 16 * 16 * 64)
    scan_ops_useful = 2.0 * SS["queries"] * SS["n"] * SS["d"] * SS["bits"]
    scan_bound_ms = scan_ops_exec / (INT8_PEAK_TOPS * 1e12) * 1e3
    search = {"workload": f"{SS['n']} x d{SS['d']} clustered, prod {SS['bits']}-bit, {SS['queries']} queries, top-{SS['k']}",
              "encode_ms": round(s_enc * 1e3, 3), "encode_vectors_per_s": round(SS["n"] / s_enc, 1),
              "scan_topk_ms": round(s_scan * 1e3, 3), "queries_per_s": round(SS["queries"] / s_scan, 1),
              "pairs_per_s": round(SS["queries"] * SS["n"] / s_scan, 1), "packed_db_bytes": s_bytes,
              "recall_at_k": round(recall, 4), "recall_queries": len(rq),
              "scan_kernel_ms": round(scan_ms, 4),
              "scan_roofline": {"bound": "mfma", "ops_executed": scan_ops_exec, "ops_useful": scan_ops_useful,
                                "bound_ms": round(scan_bound_ms, 4), "frac": round(scan_bound_ms / scan_ms, 4),
                                "frac_useful": round(scan_ops_useful / (INT8_PEAK_TOPS * 1e12) * 1e3 / scan_ms, 4),
                                "peak": INT8_PEAK_TOPS, "unit": "TOP/s (int8 dense)"}}
    log(f"search: encode {s_enc * 1e3:.2f} ms ({SS['n'] / s_enc:.3e} vectors/s); scan+top-{SS['k']} "
        f"{s_scan * 1e3:.2f} ms for {SS['queries']} queries ({SS['queries'] * SS['n'] / s_scan:.3e} pairs/s); "
        f"scan kernel {scan_ms:.3f} ms; recall@{SS['k']} over {len(rq)} queries {recall:.3f}")
    del sc, sn, sg, Qs
    torch.cuda.empty_cache()

    # ---------------- CPU oracle on a bounded sample ----------------
    cpu = None
    parity = None
    if not args.no_cpu:
        import oracle
        try:
            from threadpoolctl import threadpool_info
            blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:
            blas_threads = os.cpu_count()
        from tests import parity as parity_helpers
        piK, piV, sV = mats
        chans = synth.outlier_channels(Hkv, d, 4, workloads.ATTN_SEEDS["chan"])
        rng = np.random.default_rng(7)
        slices = sorted({(int(rng.integers(B)), int(rng.integers(Hkv))) for _ in range(args.cpu_slices)})
        G = Hq // Hkv
        errs = []
        t_cpu = 0.0
        bytes_cpu = 0
        raw = {}
        refs = {}
        for (b, g) in slices:
            # the oracle works from the raw K/V of this slice, regenerated from the workload's seeds,
            # and encodes them itself (untimed); its records replace the library's in that slice of
            # the device cache.  The timed part is what a decode step does: packed records ->
            # decoded caches -> attention
            if b not in raw:
                raw = {b: {w: synth.kv_bf16_torch((1, Hkv, T, d), workloads.ATTN_SEEDS[w] * 1000 + b, chans, "cuda")
                           for w in ("K", "V")}}
            K = raw[b]["K"][0, g].float().cpu().numpy()
            V = raw[b]["V"][0, g].float().cpu().numpy()
            ke, ve = parity_helpers.install_oracle_slice(cache, b, g, K, V)
            krec, vrec = ke["record"], ve["record"]
            kns, vns, vgs = ke["n_hat"], ve["n_hat"], ve["gamma"]
            t1 = time.perf_counter()
            kidx = oracle.parse_mse_record(krec, d, 3)
            vidx, vsb = oracle.parse_prod_record(vrec, d, 2)
            Kt = oracle.decode_mse(kidx, kns, piK, ke["c"])[None, None]
            Vt = oracle.decode_prod(vidx, vns, vsb, vgs, piV, sV, ve["c"])[None, None]
            refs[(b, g)] = oracle.decode_attention(qh[b:b + 1, g * G:(g + 1) * G], Kt, Vt, np.array([T]), scale)[0]
            t_cpu += time.perf_counter() - t1
            bytes_cpu += T * (krec.shape[-1] + 2 + vrec.shape[-1] + 4)
        del raw
        # the sampled slices now hold the oracle's records: one more launch of the timed call
        step()
        out_gpu = out.cpu().numpy()
        for (b, g), ref in refs.items():
            got = out_gpu[b, g * G:(g + 1) * G]
            errs.append(float(np.max(np.linalg.norm(got - ref, axis=-1) / np.linalg.norm(ref, axis=-1))))
        cpu = {"value": round(bytes_cpu / t_cpu / 1e9, 4), "unit": "GB/s", "cores": int(blas_threads),
               "kind": "oracle",
               "sample": f"{len(slices)} of {B * Hkv} (batch, kv-head) slices, {T} tokens x {G} query heads each: "
                         f"fp64 decode of the oracle's own packed records + two-pass softmax attention, {t_cpu:.1f}s "
                         f"(the oracle's encode of the raw slices is not timed)",
               "host_cpus": os.cpu_count()}
        parity = {"max_rel_err": max(errs), "tolerance": 2e-3, "slices": slices}
        log(f"cpu oracle: {cpu['value']} GB/s over {t_cpu:.1f}s; parity max rel err {max(errs):.2e}")
        # the oracle's encode of a sample of the one-layer encode workload (same law and seeds)
        nenc = args.cpu_encode_rows
        Ks = synth.kv_bf16_torch((eB, eH, eT, d), 201, echans, "cuda").view(-1, d)[:nenc].float().cpu().numpy()
        Vs = synth.kv_bf16_torch((eB, eH, eT, d), 202, echans, "cuda").view(-1, d)[:nenc].float().cpu().numpy()
        piKe, piVe, sVe = synth.haar_rotation(d, 211), synth.haar_rotation(d, 212), synth.gaussian_projection(d, 213)
        cK, tK = oracle.lloyd_max(d, 3)
        cV, tV = oracle.lloyd_max(d, 2)
        t1 = time.perf_counter()
        oracle.encode_mse(Ks, piKe, cK, tK)
        oracle.encode_prod(Vs, piVe, sVe, cV, tV)
        t_enc = time.perf_counter() - t1
        cpu["encode"] = {"value": round(2 * nenc / t_enc, 1), "unit": "vectors/s", "cores": int(blas_threads),
                         "sample": f"{nenc} key rows (Algorithm 1, 3-bit) + {nenc} value rows (Algorithm 2, 3-bit) "
                                   f"of the one-layer encode workload, fp64 oracle, {t_enc:.1f}s"}
        log(f"cpu oracle encode: {2 * nenc / t_enc:.3e} vectors/s over {t_enc:.1f}s")

    # ---------------- decode step with the new token appended (same shape) ----------------
    # the token goes into the last slot of every sequence (position T - 1) and the step attends all T
    # tokens; run after the oracle's sample, since it rewrites that slot
    kn_new = synth.kv_bf16_torch((B, Hkv, 1, d), 711, synth.outlier_channels(Hkv, d, 4, 712), "cuda").view(B, Hkv, d)
    vn_new = synth.kv_bf16_torch((B, Hkv, 1, d), 713, synth.outlier_channels(Hkv, d, 4, 712), "cuda").view(B, Hkv, d)
    seq_app = torch.full((B,), T - 1, dtype=torch.int32, device="cuda")

    def app_step():
        api.attn_decode_append(kq, vq, q, kn_new, vn_new, kc, kn, vt, vn, vg, seq_app, scale, out=out, ws=ws,
                               vlayout=layout)

    # the two steps alternate in short runs, so that the clock's drift under sustained load falls on both alike
    app_step()
    step()
    torch.cuda.synchronize()
    app_t = plain_t = 0.0
    runs, per = max(1, args.steps // 4), 4
    for _ in range(runs):
        t = time.perf_counter()
        for _ in range(per):
            app_step()
        torch.cuda.synchronize()
        app_t += time.perf_counter() - t
        t = time.perf_counter()
        for _ in range(per):
            step()
        torch.cuda.synchronize()
        plain_t += time.perf_counter() - t
    app_dt, plain_dt = app_t / (runs * per), plain_t / (runs * per)
    append = {"ms_per_step": round(app_dt * 1e3, 4), "plain_step_ms": round(plain_dt * 1e3, 4),
              "overhead_ms": round((app_dt - plain_dt) * 1e3, 4),
              "workload": f"decode step that encodes one new key and value per (batch, kv head) into the cache at "
                          f"position {T - 1} and attends {T} tokens; B {B}, {Hq} query heads over {Hkv} kv heads, "
                          f"d{d}, keys mse 3-bit, values prod 2-bit (token-tiled)"}
    log(f"append step: {app_dt * 1e3:.4f} ms (plain step {plain_dt * 1e3:.4f} ms)")

    # ---------------- chunked prefill: 512 query tokens against a 4096-token cache ----------------
    pB, pM, pT = 1, 512, 4096
    pc = workloads.build_attention_cache(pB, Hq, Hkv, pT, d, tiles=True)
    pq = torch.randn((pB, pM, Hq, d), generator=torch.Generator("cuda").manual_seed(721), device="cuda").to(torch.bfloat16)
    qpos = torch.full((pB,), pT - pM, dtype=torch.int32, device="cuda")
    pout = torch.empty((pB, pM, Hq, d), dtype=torch.float32, device="cuda")
    pws = torch.empty((_lib.load().tq_attn_prefill_ws_bytes(pc.kq.handle, pB, pM, Hq, Hkv, pT, 0),), dtype=torch.uint8,
                      device="cuda")
    pre_dt = timed(lambda: api.attn_prefill(pc.kq, pc.vq, pq, pc.kcodes, pc.knorms, pc.vcodes, pc.vnorms, pc.vgammas,
                                            qpos, scale, out=pout, ws=pws), reps=5)
    # the same chunk over token-tiled values: every query token a row of the decode kernels
    ptws = torch.empty((_lib.load().tq_attn_prefill_ws_bytes(pc.kq.handle, pB, pM, Hq, Hkv, pT, 1),),
                       dtype=torch.uint8, device="cuda")
    pre_t_dt = timed(lambda: api.attn_prefill(pc.kq, pc.vq, pq, pc.kcodes, pc.knorms, pc.vtiles, pc.vnorms, pc.vgammas,
                                              qpos, scale, out=pout, ws=ptws, vlayout=api.TQ_LAYOUT_TILE32), reps=5)
    wl = (f"{pM} query tokens (causal, positions {pT - pM}..{pT - 1}) x {Hq} heads over {Hkv} kv heads, d{d}, "
          f"against a {pT}-token cache (keys mse 3-bit, values prod 2-bit)")
    prefill = {"ms": round(pre_t_dt * 1e3, 4), "query_tokens_per_s": round(pB * pM / pre_t_dt, 1),
               "workload": wl + ", token-tiled values",
               "kernel": "attn_wave_kernel (one row per query token)",
               "rows_layout": {"ms": round(pre_dt * 1e3, 4), "query_tokens_per_s": round(pB * pM / pre_dt, 1),
                               "kernel": "attn_split_kernel (row records, one wave per 16 query rows)"}}
    log(f"prefill: {pre_t_dt * 1e3:.3f} ms for {pM} query tokens over token-tiled values "
        f"({pre_dt * 1e3:.3f} ms over row records)")
    del pc, pq, pout, pws, ptws

    res = {
        "metric": "packed-KV GB/s in compressed decode attention (% HBM peak); encode vectors/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 x fp4 (keys, exact fixed-point digits) and i8 (values) matrix cores on bit planes, f32 softmax",
        "data": "synthetic",
        "config": {"workload": "decode attention over a TurboQuant-packed KV cache",
                   "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d, "seq_len": T,
                   "key_bits_mse": 3, "value_bits_prod": 2, "query_dtype": "bf16",
                   "value_layout": "token-tiled (32 tokens per word)",
                   "packed_bytes": int(packed), "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "kernel": kernel_name, "kernel_ms": round(kernel_ms, 5), "launches_timed": int(split_n)},
        "cpu_baseline": cpu,
        "encode": {"value": round(enc_vps, 1), "unit": "vectors/s", "ms": round(edt * 1e3, 4),
                   "vectors": 2 * nvec, "gbs": round(enc_bytes / edt / 1e9, 2),
                   "mse_kernel_ms": round(enc_mse_ms / max(enc_mse_n, 1), 5),
                   "prod_kernel_ms": round(enc_prod_ms / max(enc_prod_n, 1), 5),
                   "prod_into_tiled_cache_ms": round(etile_ms, 5),
                   "workload": "one layer: batch 8 x 8 kv heads x 32768 tokens x d128; K mse 3-bit + V prod 3-bit",
                   "roofline": {"hbm": {"bytes": int(enc_bytes), "bound_ms": round(enc_hbm_ms, 4),
                                        "frac": round(enc_hbm_ms / (edt * 1e3), 4), "peak": HBM_PEAK_GBS,
                                        "unit": "GB/s"},
                                "mfma": {"flop_executed": enc_flop_exec, "flop_useful": enc_flop_useful,
                                         "bound_ms": round(enc_mfma_ms, 4),
                                         "frac": round(enc_mfma_ms / (edt * 1e3), 4), "peak": BF16_PEAK_TFLOPS,
                                         "unit": "TFLOP/s (fp16 dense)"}}},
        "decode": decode,
        "heterogeneous_layers": het,
        "search": search,
        "append": append,
        "prefill": prefill,
        "parity_sample": parity,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
