#!/usr/bin/env python3
"""Benchmark of the TurboQuant hot path on one MI355X.

One step = one pass over every stage of the path on synthetic inputs:
  1. quantize one layer's KV: 8 KV heads x 32768 tokens, head_dim 128, bf16,
     TurboQuant_mse b=3 (keys -> vector layout, values -> 32-vector block
     layout), 524,288 vectors, in one tq_quantize_kv call (one launch);
  2. decode attention over a resident packed cache: batch 8, 64 query / 8 KV
     heads, head_dim 128, context 131072, keys TurboQuant_prod b=3, values
     TurboQuant_mse b=3, one query token per sequence.
The decode streams 906 MB, more than the 256 MB Infinity Cache, so each step's
quantize inputs are not cache-resident when it starts.

Printed: one JSON line. `value` is the step's algorithmic HBM bytes (quantize
in + codes + norms; decode 108 B per token and KV head) per second over the
timed steps (50 by default); per-stage means, medians and p10/p90 come from HIP
events around each stage. Components timed on their own (the prod quantize, the
bit-width / head-dim sweep, vector-search scoring) run each call after reading a
512 MB buffer, so their inputs come from HBM and not the 256 MB Infinity Cache,
and report the median. Also attached: the decode kernel's roofline, the
quantize's bf16 MFMA use as a fraction of the 2.5 PFLOP/s dense peak, and the
fp64 oracle's CPU rate on a bounded sample (all host threads, and one core).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 matrix peak
FLUSH_BYTES = 512 << 20  # read before a timed call so its inputs are not cache-resident (256 MB MALL)
METRIC = "quantize Mvec/s (d=128,b=3) + decode-attention GB/s over packed KV, % roofline"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle CPU timing")
    ap.add_argument("--traffic", type=str, default=None,
                    help="counter summary with the measured HBM bytes per decode launch (default: profiles/)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only copy 1 GiB device to device 3 times (scale reference for HBM byte counters)")
    ap.add_argument("--only", choices=["quantize", "decode", "append", "split_decode"], default=None,
                    help="profiling runs: build the headline workload, then run only this stage "
                         "warmup + steps times and print its mean time (no JSON line)")
    return ap.parse_args()


def build_workloads(tq, syn, torch, dev):
    import numpy as np
    d = 128
    # ---- layer quantize (8 heads x 32768 tokens, mse b=3) ----
    H, T2 = 8, 32768
    qk2 = [tq.Quantizer(d, 3, "mse", syn.rotation(d, syn.CFG_LAYER_QUANT, syn.T_K, h)) for h in range(H)]
    qv2 = [tq.Quantizer(d, 3, "mse", syn.rotation(d, syn.CFG_LAYER_QUANT, syn.T_V, h)) for h in range(H)]
    xk2 = syn.kv_vectors_device(H, T2, d, syn.CFG_LAYER_QUANT, syn.T_K, dev)
    xv2 = syn.kv_vectors_device(H, T2, d, syn.CFG_LAYER_QUANT, syn.T_V, dev)
    out_k2 = {"codes": torch.empty((H, T2 * 48), dtype=torch.uint8, device=dev),
              "norms": torch.empty((H, T2), dtype=torch.float32, device=dev)}
    out_v2 = {"codes": torch.empty((H, T2 * 48), dtype=torch.uint8, device=dev),
              "norms": torch.empty((H, T2), dtype=torch.float32, device=dev)}
    # ---- decode cache (B=8, 64/8 heads, ctx 131072) ----
    B, Hq, Hkv, T3 = 8, 64, 8, 131072
    kq3 = [tq.Quantizer(d, 3, "prod", syn.rotation(d, syn.CFG_DECODE_128K, syn.T_K, h),
                        syn.gaussian_matrix(d, syn.CFG_DECODE_128K, syn.T_K, h)) for h in range(Hkv)]
    vq3 = [tq.Quantizer(d, 3, "mse", syn.rotation(d, syn.CFG_DECODE_128K, syn.T_V, h)) for h in range(Hkv)]
    kcodes = torch.empty((B, Hkv, T3, 32), dtype=torch.uint8, device=dev)
    ksigns = torch.empty((B, Hkv, T3, 16), dtype=torch.uint8, device=dev)
    knorms = torch.empty((B, Hkv, T3), dtype=torch.float32, device=dev)
    krn = torch.empty((B, Hkv, T3), dtype=torch.float32, device=dev)
    vcodes = torch.empty((B, Hkv, T3 // 32, 4 * 3 * d), dtype=torch.uint8, device=dev)
    vnorms = torch.empty((B, Hkv, T3), dtype=torch.float32, device=dev)
    for b in range(B):
        xk = syn.kv_vectors_device(Hkv, T3, d, syn.CFG_DECODE_128K, syn.T_K, dev, seed_offset=b)
        tq.quantize(kq3, xk, layout="vector", out={"codes": kcodes[b].view(Hkv, -1), "signs": ksigns[b],
                                                   "norms": knorms[b], "rnorms": krn[b]})
        del xk
        xv = syn.kv_vectors_device(Hkv, T3, d, syn.CFG_DECODE_128K, syn.T_V, dev, seed_offset=b)
        tq.quantize(vq3, xv, layout="block32", out={"codes": vcodes[b].view(Hkv, -1), "norms": vnorms[b]})
        del xv
    torch.cuda.synchronize()
    kcache = tq.KVCache(kq3, knorms, kcodes, ksigns, krn)
    vcache = tq.KVCache(vq3, vnorms, vcodes)
    q = torch.from_numpy(syn.decode_queries(B, Hq, d, syn.CFG_DECODE_128K)).to(dev).to(torch.bfloat16)
    lens = torch.full((B,), T3, dtype=torch.int32, device=dev)
    ws = torch.empty(tq.decode_workspace_size(B, Hq, Hkv, d, T3, kcache, vcache), dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    # a prod quantize of the layer's keys, timed on its own (residual + QJL stage)
    qp2 = [tq.Quantizer(d, 3, "prod", syn.rotation(d, syn.CFG_LAYER_QUANT, syn.T_K, h),
                        syn.gaussian_matrix(d, syn.CFG_LAYER_QUANT, syn.T_K, h)) for h in range(H)]
    out_p2 = {"codes": torch.empty((H, T2 * 32), dtype=torch.uint8, device=dev),
              "signs": torch.empty((H, T2, 16), dtype=torch.uint8, device=dev),
              "norms": torch.empty((H, T2), dtype=torch.float32, device=dev),
              "rnorms": torch.empty((H, T2), dtype=torch.float32, device=dev)}
    return dict(d=d, H=H, T2=T2, qk2=qk2, qv2=qv2, xk2=xk2, xv2=xv2, out_k2=out_k2, out_v2=out_v2,
                B=B, Hq=Hq, Hkv=Hkv, T3=T3, kcache=kcache, vcache=vcache, q=q, lens=lens, ws=ws, out=out,
                qp2=qp2, out_p2=out_p2)


# the sources of the decode kernels (their hash keys the committed traffic counters)
DECODE_SOURCES = ("tq_decode.hip", "tq_device.h", "tq_internal.h")


def decode_traffic(path=None):
    """HBM bytes per decode main-kernel launch measured with rocprofv3 FETCH_SIZE /
    WRITE_SIZE (scaled by a 1 GiB copy), read from the committed counter summary.
    None when the decode source changed since the counters were taken."""
    import hashlib
    path = path or os.path.join(ROOT, "profiles", "decode_attention_b8_ctx128k_hbm_counters.md")
    srcs = [os.path.join(ROOT, "attention_tq_quantize_amd", "csrc", f) for f in DECODE_SOURCES]
    if not (os.path.exists(path) and all(os.path.exists(f) for f in srcs)):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.split(":", 1)[0].strip() in ("decode_bytes_per_launch", "decode_source_sha256_16"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    now = hashlib.sha256(b"".join(open(f, "rb").read() for f in srcs)).hexdigest()[:16]
    if fields.get("decode_source_sha256_16") != now or "decode_bytes_per_launch" not in fields:
        return None
    return int(fields["decode_bytes_per_launch"])


def make_flush(torch, dev):
    """A 512 MB buffer, written once; reading all of it (a max reduction) evicts
    the 256 MB Infinity Cache with clean lines, so the next call reads its inputs
    from HBM and inherits no dirty lines to write back."""
    buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    def flush():
        torch.amax(buf)
    return flush


def timed_flushed(torch, fn, flush, reps):
    """reps calls of fn, each after a cache flush, each timed alone with HIP
    events on the current stream: (median, p10, p90) in ms."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        flush()
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    return ms[reps // 2], ms[reps // 10], ms[min(reps - 1, (9 * reps) // 10)]


def quantize_mfma_flops(d, variant):
    """MFMA floating-point operations the quantize kernel executes per bf16 vector:
    the rotation as bf16 hi and lo passes (2 x 2 d^2) and, for prod, the S' = S Pi^T
    projection of the residual as three bf16 passes (hi*hi, lo*hi, hi*lo)."""
    return 4 * d * d + (6 * d * d if variant == "prod" else 0)


def c4_sweep(tq, syn, torch, dev, flush, reps=20):
    """Bit-width and head-dim sweep: b in {1, 2, 4} x {mse, prod} keys (values mse b)
    x d in {64, 256}; B = 4, 64 query / 8 KV heads, 16384 tokens per sequence, bf16
    KV with the headline's outlier channels and per-token LogNormal(0, 0.5) scale.
    Per row: layer quantize of keys and values (one tq_quantize_kv call, 2 x 524,288
    vectors: one launch for mse keys, two for prod keys)
    and decode attention over the packed caches, each timed after a 512 MB cache
    flush, median of reps calls; quantize MFMA use as executed bf16 MFMA FLOPs over
    the 2.5 PFLOP/s dense peak."""
    B, Hq, Hkv, T = 4, 64, 8, 16384
    G = B * Hkv
    rows = []
    for d in (64, 256):
        xk = syn.kv_vectors_device(G, T, d, syn.CFG_SWEEP, syn.T_K, dev, lognormal_sigma=0.5)
        xv = syn.kv_vectors_device(G, T, d, syn.CFG_SWEEP, syn.T_V, dev, lognormal_sigma=0.5)
        q = torch.from_numpy(syn.decode_queries(B, Hq, d, syn.CFG_SWEEP)).to(dev).to(torch.bfloat16)
        lens = torch.full((B,), T, dtype=torch.int32, device=dev)
        for bits in (1, 2, 4):
            for var in ("mse", "prod"):
                kq = [tq.Quantizer(d, bits, var, syn.rotation(d, syn.CFG_SWEEP, syn.T_K, 700 + h),
                                   syn.gaussian_matrix(d, syn.CFG_SWEEP, syn.T_K, 700 + h) if var == "prod" else None)
                      for h in range(Hkv)]
                vq = [tq.Quantizer(d, bits, "mse", syn.rotation(d, syn.CFG_SWEEP, syn.T_V, 700 + h)) for h in range(Hkv)]
                kp = kq[0].planes
                kcodes = torch.empty((B, Hkv, T, kq[0].code_bytes), dtype=torch.uint8, device=dev) if kp > 0 else None
                ksigns = torch.empty((B, Hkv, T, d // 8), dtype=torch.uint8, device=dev) if var == "prod" else None
                knorms = torch.empty((B, Hkv, T), dtype=torch.float32, device=dev)
                krn = torch.empty((B, Hkv, T), dtype=torch.float32, device=dev) if var == "prod" else None
                vcodes = torch.empty((B, Hkv, T // 32, 4 * bits * d), dtype=torch.uint8, device=dev)
                vnorms = torch.empty((B, Hkv, T), dtype=torch.float32, device=dev)
                kout = {"norms": knorms.view(G, T)}
                if kp > 0:
                    kout["codes"] = kcodes.view(G, -1)
                if var == "prod":
                    kout["signs"] = ksigns.view(G, T, -1)
                    kout["rnorms"] = krn.view(G, T)
                vout = {"codes": vcodes.view(G, -1), "norms": vnorms.view(G, T)}
                kq_g = [kq[g % Hkv] for g in range(G)]
                vq_g = [vq[g % Hkv] for g in range(G)]

                def quant():
                    tq.quantize_kv(kq_g, vq_g, xk, xv, kout=kout, vout=vout)
                quant()
                torch.cuda.synchronize()
                kcache = tq.KVCache(kq, knorms, kcodes, ksigns, krn)
                vcache = tq.KVCache(vq, vnorms, vcodes)
                ws = torch.empty(tq.decode_workspace_size(B, Hq, Hkv, d, T, kcache, vcache), dtype=torch.uint8,
                                 device=dev)
                out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)

                def dec():
                    tq.decode_attention(q, kcache, vcache, lens, 1 / math.sqrt(d), max_ctx=T, out=out, workspace=ws)
                dec()
                qmed, q10, q90 = timed_flushed(torch, quant, flush, reps)
                dmed, d10, d90 = timed_flushed(torch, dec, flush, reps)
                n = G * T
                krec = kq[0].code_bytes + 4 + ((d // 8 + 4) if var == "prod" else 0)
                vrec = bits * d // 8 + 4
                qbytes = n * (2 * d * 2 + krec + vrec)
                dbytes = n * (krec + vrec)
                mflops = n * (quantize_mfma_flops(d, var) + quantize_mfma_flops(d, "mse"))
                rows.append({
                    "d": d, "bits": bits, "keys": var, "values": "mse",
                    "quantize_ms": round(qmed, 4), "quantize_ms_p10_p90": [round(q10, 4), round(q90, 4)],
                    "quantize_mvec_s": round(2 * n / (qmed * 1e-3) / 1e6, 1),
                    "quantize_gb_s": round(qbytes / (qmed * 1e-3) / 1e9, 1),
                    "quantize_frac_hbm": round(qbytes / (qmed * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "quantize_frac_mfma": round(mflops / (qmed * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                    "decode_ms": round(dmed, 4), "decode_ms_p10_p90": [round(d10, 4), round(d90, 4)],
                    "decode_gb_s": round(dbytes / (dmed * 1e-3) / 1e9, 1),
                    "decode_frac_hbm": round(dbytes / (dmed * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "bytes_per_token_head": krec + vrec})
                del kcache, vcache, ws, kcodes, ksigns, knorms, krn, vcodes, vnorms, kout, vout
        del xk, xv
        torch.cuda.empty_cache()
    return {"workload": "B=4, 64/8 heads, ctx 16384; keys mse|prod b, values mse b; flushed, median of "
                        f"{reps}", "rows": rows}


def cpu_baseline(syn):
    """The fp64 oracle on a bounded sample of the same workload, host cores."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    d = 128
    nq = 1 << 20
    x = syn.kv_vectors(nq, d, syn.CFG_LAYER_QUANT, syn.T_K, 0, 0)
    Pi = syn.rotation(d, syn.CFG_LAYER_QUANT, syn.T_K, 0)
    cb = O.codebook(d, 3)
    t0 = time.perf_counter()
    r = O.quantize_mse(x, Pi, cb)
    O.pack_vector_layout(r["idx"], 3)
    tq_s = time.perf_counter() - t0
    del x, r
    # decode sample: six (batch, kv head) groups, 8 query heads each, T tokens
    T, n_groups = 131072, 6
    td_s = 0.0
    for h in range(n_groups):
        Pk = syn.rotation(d, syn.CFG_DECODE_128K, syn.T_K, h)
        Sk = syn.gaussian_matrix(d, syn.CFG_DECODE_128K, syn.T_K, h)
        Pv = syn.rotation(d, syn.CFG_DECODE_128K, syn.T_V, h)
        xk = syn.kv_vectors(T, d, syn.CFG_DECODE_128K, syn.T_K, 0, h)
        xv = syn.kv_vectors(T, d, syn.CFG_DECODE_128K, syn.T_V, 0, h)
        ck, cv = O.codebook(d, 2), O.codebook(d, 3)
        rk = O.quantize_prod(xk, Pk, Sk, ck)
        rv = O.quantize_mse(xv, Pv, cv)
        kc = {"variant": "prod", "bits": 3, "d": d, "max_ctx": T, "Pi": Pk[None], "S": Sk[None],
              "codes": O.pack_vector_layout(rk["idx"], 2)[None, None], "signs": O.pack_bits(rk["signs"])[None, None],
              "norms": rk["norms"][None, None], "rnorms": rk["rnorms"][None, None]}
        vc = {"variant": "mse", "bits": 3, "d": d, "max_ctx": T, "Pi": Pv[None],
              "codes": O.pack_block_layout(rv["idx"], 3).reshape(1, 1, T // 32, -1), "norms": rv["norms"][None, None]}
        q = syn.decode_queries(1, 64, d, syn.CFG_DECODE_128K)[:, 8 * h:8 * (h + 1)]
        t0 = time.perf_counter()
        O.decode_attention(q, kc, vc, np.array([T]), 1 / math.sqrt(d))
        td_s += time.perf_counter() - t0
        if h == 0:
            first = (q, kc, vc)
    qbytes = nq * (256 + 48 + 4)
    dbytes = n_groups * T * 108
    # the same oracle on one host core (BLAS held to one thread): a smaller sample
    single = None
    try:
        from threadpoolctl import threadpool_limits
        n1 = 1 << 17
        x1 = syn.kv_vectors(n1, d, syn.CFG_LAYER_QUANT, syn.T_K, 0, 1)
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            r1 = O.quantize_mse(x1, Pi, cb)
            O.pack_vector_layout(r1["idx"], 3)
            tq1 = time.perf_counter() - t0
            q, kc, vc = first
            t0 = time.perf_counter()
            O.decode_attention(q, kc, vc, np.array([T]), 1 / math.sqrt(d))
            td1 = time.perf_counter() - t0
        b1 = n1 * (256 + 48 + 4) + T * 108
        single = {"value": round(b1 / (tq1 + td1) / 1e9, 5), "unit": "GB/s", "cores": 1,
                  "sample": (f"quantize_mse of {n1} vectors ({tq1:.2f} s) + decode attention of one (batch, kv "
                             f"head) group over {T} tokens ({td1:.2f} s), BLAS limited to one thread"),
                  "quantize_mvec_s": round(n1 / tq1 / 1e6, 5), "decode_gb_s": round(T * 108 / td1 / 1e9, 5)}
    except ImportError:
        pass
    return {"value": round((qbytes + dbytes) / (tq_s + td_s) / 1e9, 4), "unit": "GB/s", "cores": int(cores),
            "kind": "oracle",
            "sample": (f"fp64 oracle: quantize_mse of {nq} bf16 vectors (d=128, b=3; {tq_s:.2f} s) + decode "
                       f"attention of {n_groups} (batch, kv head) groups, 8 query heads each over {T} tokens "
                       f"(prod-3 keys, mse-3 values; {td_s:.2f} s); same algorithmic-byte accounting"),
            "quantize_mvec_s": round(nq / tq_s / 1e6, 5), "decode_gb_s": round(dbytes / td_s / 1e9, 5),
            "single_core": single}


def vector_search(tq, syn, torch, dev, flush, n=100000, m=16, bits=3, reps=10):
    """Vector-search workload: index n synthetic Gaussian embeddings with
    TurboQuant_prod (b = 3) at d = 1536 and 3072, then score m queries against
    the packed database with tq_inner_products (fp32 vector units) and with
    tq_search_scores (matrix cores). Scoring calls are timed after a 512 MB cache
    flush each (the database would otherwise stay in the Infinity Cache), median
    of reps."""
    import numpy as np
    out = {}
    for d in (1536, 3072):
        qz = tq.Quantizer(d, bits, "prod", syn.rotation(d, syn.CFG_SWEEP, syn.T_K, 500 + d),
                          syn.gaussian_matrix(d, syn.CFG_SWEEP, syn.T_K, 500 + d))
        gen = torch.Generator(device=dev)
        gen.manual_seed(syn.ROOT_SEED + d)
        x = torch.randn((n, d), generator=gen, device=dev, dtype=torch.float32)
        y = torch.randn((m, d), generator=gen, device=dev, dtype=torch.float32)
        rec = tq.quantize_prod(qz, x)  # warm-up and the database
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        rec = tq.quantize_prod(qz, x)
        e1.record()
        torch.cuda.synchronize()
        index_ms = e0.elapsed_time(e1)
        del x
        args = (qz, y, rec["codes"], rec["norms"], rec["signs"], rec["rnorms"])
        for _ in range(3):
            tq.inner_products(*args)
        score_ms, _, _ = timed_flushed(torch, lambda: tq.inner_products(*args), flush, reps)
        ws = torch.empty(tq.search_workspace_size(qz, m), dtype=torch.uint8, device=dev)
        for _ in range(3):
            tq.search_scores(*args, workspace=ws)
        mfma_ms, _, _ = timed_flushed(torch, lambda: tq.search_scores(*args, workspace=ws), flush, reps)
        rec_bytes = (bits - 1) * d // 8 + d // 8 + 8
        out[f"d{d}"] = {"database": n, "queries": m, "variant": f"prod b={bits}",
                        "index_ms": round(index_ms, 3), "index_mvec_s": round(n / (index_ms * 1e-3) / 1e6, 2),
                        "score_ms": round(score_ms, 3), "pairs_per_s": round(m * n / (score_ms * 1e-3), 1),
                        "score_record_gb_s": round(m * n * rec_bytes / (score_ms * 1e-3) / 1e9, 1),
                        "mfma_score_ms": round(mfma_ms, 3), "mfma_pairs_per_s": round(m * n / (mfma_ms * 1e-3), 1),
                        "mfma_database_gb_s": round(n * rec_bytes / (mfma_ms * 1e-3) / 1e9, 1)}
        del rec, qz
    return out


def decode_1m(tq, syn, torch, dev, reps=20):
    """Decode attention at 1M context: B=1, 64/8 heads, d=128, T=1,048,576, keys
    TurboQuant_prod b=3, values TurboQuant_mse b=3, KV vectors with a per-token
    LogNormal(0, 0.5) scale; the same 905,969,664 algorithmic bytes per call as
    the 128K batch, in one sequence (split-context over 1M tokens)."""
    d, Hq, Hkv, T = 128, 64, 8, 1 << 20
    kq = [tq.Quantizer(d, 3, "prod", syn.rotation(d, syn.CFG_DECODE_1M, syn.T_K, h),
                       syn.gaussian_matrix(d, syn.CFG_DECODE_1M, syn.T_K, h)) for h in range(Hkv)]
    vq = [tq.Quantizer(d, 3, "mse", syn.rotation(d, syn.CFG_DECODE_1M, syn.T_V, h)) for h in range(Hkv)]
    kcodes = torch.empty((1, Hkv, T, 32), dtype=torch.uint8, device=dev)
    ksigns = torch.empty((1, Hkv, T, 16), dtype=torch.uint8, device=dev)
    knorms = torch.empty((1, Hkv, T), dtype=torch.float32, device=dev)
    krn = torch.empty((1, Hkv, T), dtype=torch.float32, device=dev)
    vcodes = torch.empty((1, Hkv, T // 32, 4 * 3 * d), dtype=torch.uint8, device=dev)
    vnorms = torch.empty((1, Hkv, T), dtype=torch.float32, device=dev)
    xk = syn.kv_vectors_device(Hkv, T, d, syn.CFG_DECODE_1M, syn.T_K, dev, lognormal_sigma=0.5)
    tq.quantize(kq, xk, layout="vector", out={"codes": kcodes[0].view(Hkv, -1), "signs": ksigns[0],
                                              "norms": knorms[0], "rnorms": krn[0]})
    del xk
    xv = syn.kv_vectors_device(Hkv, T, d, syn.CFG_DECODE_1M, syn.T_V, dev, lognormal_sigma=0.5)
    tq.quantize(vq, xv, layout="block32", out={"codes": vcodes[0].view(Hkv, -1), "norms": vnorms[0]})
    del xv
    kcache = tq.KVCache(kq, knorms, kcodes, ksigns, krn)
    vcache = tq.KVCache(vq, vnorms, vcodes)
    q = torch.from_numpy(syn.decode_queries(1, Hq, d, syn.CFG_DECODE_1M)).to(dev).to(torch.bfloat16)
    lens = torch.full((1,), T, dtype=torch.int32, device=dev)
    ws = torch.empty(tq.decode_workspace_size(1, Hq, Hkv, d, T, kcache, vcache), dtype=torch.uint8, device=dev)
    out = torch.empty((1, Hq, d), dtype=torch.float32, device=dev)
    run = lambda: tq.decode_attention(q, kcache, vcache, lens, 1 / math.sqrt(d), max_ctx=T, out=out, workspace=ws)
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record()
        run()
        e1.record()
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    avg = sum(ms) / reps
    nbytes = Hkv * T * 108
    return {"workload": "decode B=1, 64/8 heads, d=128, ctx 1048576, keys prod b=3, values mse b=3",
            "ms": round(avg, 4), "ms_p10_p90": [round(ms[reps // 10], 4), round(ms[(9 * reps) // 10], 4)],
            "gb_s": round(nbytes / (avg * 1e-3) / 1e9, 1), "frac_hbm": round(nbytes / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def outlier_split_decode(tq, syn, torch, dev, reps=10, bits=(3, 2)):
    """Decode attention over an outlier-split cache at the 128K batch shape (B=8,
    64/8 heads, d=128, ctx 131072): keys TurboQuant_prod with each KV head's 32
    largest-RMS channels at bits[0] and the other 96 at bits[1], values TurboQuant_mse with the
    same bit split (3 + 2 bits: 96 B per (token, KV head) against 108 B for the
    uniform 3-bit cache; 4 + 3 bits: 128 B); tq_decode_attention_split (matrix-core
    split kernels)."""
    B, Hq, Hkv, d, T = 8, 64, 8, 128, 131072
    sides = []
    for tensor, var in ((syn.T_K, "prod"), (syn.T_V, "mse")):
        qs_p = [[], []]
        # every KV head keeps its own 32 largest-RMS channels (batch-0 sample of that head)
        sample = syn.kv_vectors_device(Hkv, 4096, d, syn.CFG_DECODE_128K, tensor, dev, seed_offset=0)
        order = torch.argsort(sample.float().pow(2).mean(dim=1), dim=1, descending=True, stable=True).cpu().numpy()
        chans_p = [order[:, :32], order[:, 32:]]  # [Hkv][d_p] per part
        del sample
        for p, pbits in enumerate(bits):
            dp = chans_p[p].shape[-1]
            for g in range(Hkv):
                S = syn.gaussian_matrix(dp, syn.CFG_DECODE_128K, tensor, 300 + 10 * p + g) if var == "prod" else None
                qs_p[p].append(tq.Quantizer(dp, pbits, var, syn.rotation(dp, syn.CFG_DECODE_128K, tensor, 300 + 10 * p + g), S))
        recs = []
        for p in range(2):
            q0 = qs_p[p][0]
            r = {"norms": torch.empty((B, Hkv, T), dtype=torch.float32, device=dev),
                 "codes": torch.empty((B, Hkv, T, q0.code_bytes), dtype=torch.uint8, device=dev)}
            if var == "prod":
                r["signs"] = torch.empty((B, Hkv, T, q0.d // 8), dtype=torch.uint8, device=dev)
                r["rnorms"] = torch.empty((B, Hkv, T), dtype=torch.float32, device=dev)
            recs.append(r)
        for b in range(B):
            # one grouped call per batch row: the KV heads are the groups
            x = syn.kv_vectors_device(Hkv, T, d, syn.CFG_DECODE_128K, tensor, dev, seed_offset=b)
            got = tq.quantize_split(qs_p, chans_p, x, layout="block32" if var == "mse" else "vector")
            for p in range(2):
                for key, val in got[p].items():
                    recs[p][key][b].copy_(val.view(recs[p][key][b].shape))
            del x, got
        sides.append(tq.SplitKV([(qs_p[p], chans_p[p], recs[p]) for p in range(2)]))
    k, v = sides
    q = torch.from_numpy(syn.decode_queries(B, Hq, d, syn.CFG_DECODE_128K)).to(dev).to(torch.bfloat16)
    lens = torch.full((B,), T, dtype=torch.int32, device=dev)
    ws = torch.empty(tq.decode_split_workspace_size(B, Hq, Hkv, d, T, k, v), dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    run = lambda: tq.decode_attention_split(q, k, v, lens, 1 / math.sqrt(d), out=out, workspace=ws)
    for _ in range(2):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    # record bytes per (token, KV head): codes and norms of every part, plus signs and residual norms of the keys
    per = (sum(qs[0].code_bytes + 4 + qs[0].d // 8 + 4 for qs, _, _ in k.parts)
           + sum(qs[0].code_bytes + 4 for qs, _, _ in v.parts))
    nbytes = B * Hkv * T * per
    split = f"32 ch x {bits[0]} b + 96 ch x {bits[1]} b"
    return {"workload": f"split decode B=8, 64/8 heads, d=128, ctx 131072; K prod {split}, V mse {split}",
            "bits_per_channel": (32 * bits[0] + 96 * bits[1]) / 128,
            "bytes_per_token_head": per, "ms": round(ms, 3),
            "gb_s": round(nbytes / (ms * 1e-3) / 1e9, 1), "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def outlier_split(tq, syn, torch, dev, w, flush, bits=(3, 2)):
    """Outlier-channel mixed precision on the layer's KV (8 heads x 32768 tokens,
    d = 128): per head, the 32 channels of largest RMS at bits[0] and the other 96
    at bits[1] (3 + 2: 2.25 bits per channel; 4 + 3: 3.25), keys TurboQuant_prod,
    values TurboQuant_mse, through tq_quantize_split: one grouped call per tensor
    (the heads are the groups, each with its own channels and quantizers; both
    parts in one matrix-core launch; the values' codes written in the BLOCK32
    layout the split decode reads)."""
    H, T2, d = w["H"], w["T2"], w["d"]
    calls = []
    for t, xs, var in ((syn.T_K, w["xk2"], "prod"), (syn.T_V, w["xv2"], "mse")):
        qs, chans = [[], []], [[], []]
        for h in range(H):
            rms = xs[h].float().pow(2).mean(dim=0)
            order = torch.argsort(rms, descending=True, stable=True).cpu().numpy()
            for i, (c, pbits) in enumerate(zip((order[:32], order[32:]), bits)):
                dp = len(c)
                S = syn.gaussian_matrix(dp, syn.CFG_LAYER_QUANT, t, 100 + 2 * h + i) if var == "prod" else None
                qs[i].append(tq.Quantizer(dp, pbits, var, syn.rotation(dp, syn.CFG_LAYER_QUANT, t, 100 + 2 * h + i), S))
                chans[i].append(c)
        sq = tq.SplitQuantize(qs, chans, grouped=True, layout="block32" if var == "mse" else "vector")
        calls.append((sq, xs, sq(xs)))
    run = lambda: [sq(x, out=o) for sq, x, o in calls]
    run()
    ms, ms10, ms90 = timed_flushed(torch, run, flush, 20)
    nvec = 2 * H * T2
    per_ch = (32 * bits[0] + 96 * bits[1]) / 128
    return {"split": f"32 ch x {bits[0]} b + 96 ch x {bits[1]} b ({per_ch} bits/channel), keys prod, values mse",
            "vectors": nvec, "launches": 2,
            "ms": round(ms, 4), "ms_p10_p90": [round(ms10, 4), round(ms90, 4)], "mvec_s": round(nvec / (ms * 1e-3) / 1e6, 1),
            "input_gb_s": round(nvec * d * 2 / (ms * 1e-3) / 1e9, 1)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the path is measured on a single GPU.",
              file=sys.stderr)
        return 2
    import numpy as np
    import torch
    if args.calibrate_copy:
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": 1 << 30, "copies": 3}))
        return 0
    import attention_tq_quantize_amd as tq
    import tq_synth as syn
    tq.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.only == "split_decode":
        print(json.dumps(outlier_split_decode(tq, syn, torch, dev, reps=max(args.steps, 1))), flush=True)
        return 0
    print("building workloads", file=sys.stderr, flush=True)
    w = build_workloads(tq, syn, torch, dev)

    def quantize_layer():
        tq.quantize_kv(w["qk2"], w["qv2"], w["xk2"], w["xv2"], kout=w["out_k2"], vout=w["out_v2"])

    def decode():
        tq.decode_attention(w["q"], w["kcache"], w["vcache"], w["lens"], 1 / math.sqrt(w["d"]), max_ctx=w["T3"],
                            out=w["out"], workspace=w["ws"])

    if args.only == "append":
        knew = torch.zeros((w["B"], w["Hkv"], w["d"]), dtype=torch.bfloat16, device=dev)
        knew.normal_()
        vnew = torch.randn_like(knew)
        lens_app = torch.full((w["B"],), w["T3"] - 1, dtype=torch.int32, device=dev)

        def append_step():
            tq.decode_append_attention(w["q"], knew, vnew, w["kcache"], w["vcache"], lens_app,
                                       1 / math.sqrt(w["d"]), max_ctx=w["T3"], out=w["out"], workspace=w["ws"])
    if args.only:
        stage = quantize_layer if args.only == "quantize" else decode if args.only == "decode" else append_step
        for _ in range(args.warmup):
            stage()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            stage()
        e1.record()
        torch.cuda.synchronize()
        print(f"{args.only}: {e0.elapsed_time(e1) / max(args.steps, 1):.4f} ms per call over {args.steps} calls",
              flush=True)
        return 0

    for _ in range(args.warmup):
        quantize_layer()
        decode()
    torch.cuda.synchronize()
    K = args.steps
    # two events per step: its start and the quantize/decode boundary; a step's decode ends where
    # the next step starts (the last one at t_end), so the timed region holds 2 K + 1 records
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    t_end = torch.cuda.Event(enable_timing=True)
    # torch creates the HIP event behind an Event at its first record(): record every one once
    # here so that no event is created inside the timed region
    for e in [t_end] + [x for row in ev for x in row]:
        e.record()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for k in range(K):
        ev[k][0].record()
        quantize_layer()
        ev[k][1].record()
        decode()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = ev[0][0].elapsed_time(t_end)
    ends = [ev[k + 1][0] for k in range(K - 1)] + [t_end]
    q_ms = sorted(ev[k][0].elapsed_time(ev[k][1]) for k in range(K))
    d_ms = sorted(ev[k][1].elapsed_time(ends[k]) for k in range(K))
    q_avg = sum(q_ms) / K
    d_avg = sum(d_ms) / K
    n_vec = 2 * w["H"] * w["T2"]
    q_bytes = n_vec * (256 + 48 + 4)
    d_bytes = w["B"] * w["Hkv"] * w["T3"] * 108
    ms_per_step = total_ms / K
    value = (q_bytes + d_bytes) / (ms_per_step * 1e-3) / 1e9

    flush = make_flush(torch, dev)
    # residual + QJL stage on its own: prod quantize of the layer's keys (flushed, median)
    pq = lambda: tq.quantize(w["qp2"], w["xk2"], layout="vector", out=w["out_p2"])
    for _ in range(3):
        pq()
    p_ms, _, _ = timed_flushed(torch, pq, flush, 20)
    p_vec = w["H"] * w["T2"]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    # decode step with append: the new token's key and value are quantized into the
    # caches at position ctx - 1 of every sequence, then ctx tokens are attended
    knew = torch.from_numpy(np.stack([syn.kv_vectors(w["Hkv"], w["d"], syn.CFG_DECODE_128K, syn.T_K, b, 99)
                                      for b in range(w["B"])])).to(dev).to(torch.bfloat16)
    vnew = torch.from_numpy(np.stack([syn.kv_vectors(w["Hkv"], w["d"], syn.CFG_DECODE_128K, syn.T_V, b, 99)
                                      for b in range(w["B"])])).to(dev).to(torch.bfloat16)
    lens_app = torch.full((w["B"],), w["T3"] - 1, dtype=torch.int32, device=dev)
    ws_app = torch.empty(tq.decode_append_workspace_size(w["B"], w["Hq"], w["Hkv"], w["d"], w["T3"], w["kcache"],
                                                         w["vcache"]), dtype=torch.uint8, device=dev)

    def decode_append():
        tq.decode_append_attention(w["q"], knew, vnew, w["kcache"], w["vcache"], lens_app, 1 / math.sqrt(w["d"]),
                                   max_ctx=w["T3"], out=w["out"], workspace=ws_app)

    for _ in range(3):
        decode_append()
    # the append step and the plain decode, timed alike and interleaved (so clock drift
    # falls on both): each call after a cache flush, median of 20 each
    ev_a, ev_d = [], []
    for _ in range(20):
        for fn, lst in ((decode_append, ev_a), (decode, ev_d)):
            e_0, e_1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            flush()
            e_0.record()
            fn()
            e_1.record()
            lst.append((e_0, e_1))
    torch.cuda.synchronize()
    a_ms = sorted(x.elapsed_time(y) for x, y in ev_a)[10]
    d_flushed_ms = sorted(x.elapsed_time(y) for x, y in ev_d)[10]

    vsearch = vector_search(tq, syn, torch, dev, flush)
    c4 = c4_sweep(tq, syn, torch, dev, flush)
    split = outlier_split(tq, syn, torch, dev, w, flush)
    split_35 = outlier_split(tq, syn, torch, dev, w, flush, bits=(4, 3))
    dec1m = decode_1m(tq, syn, torch, dev)
    split_dec = outlier_split_decode(tq, syn, torch, dev)
    split_dec_35 = outlier_split_decode(tq, syn, torch, dev, bits=(4, 3))

    traffic = decode_traffic(args.traffic)
    d_gbs = d_bytes / (d_avg * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 in; bf16/f16 hi+lo MFMA operands, f32 accumulate",
        "data": "synthetic (seeded N(0,1) KV with 4 outlier channels x10 per head, bf16; Haar rotations; Gaussian S)",
        "config": {"workload": "layer KV quantize (8 heads x 32768 tokens, d=128, mse b=3) + decode attention "
                               "(B=8, 64/8 heads, d=128, ctx 131072, keys prod b=3, values mse b=3)",
                   "quantize_vectors": n_vec, "decode_tokens_x_kv_heads": w["B"] * w["Hkv"] * w["T3"]},
        "components": {
            "quantize_mvec_s": round(n_vec / (q_avg * 1e-3) / 1e6, 1),
            "quantize_gb_s": round(q_bytes / (q_avg * 1e-3) / 1e9, 1),
            "quantize_ms": round(q_avg, 4),
            "quantize_frac_hbm": round(q_bytes / (q_avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "decode_gb_s": round(d_gbs, 1),
            "decode_ms": round(d_avg, 4),
            "decode_ms_p10_p90": [round(d_ms[K // 10], 4), round(d_ms[(9 * K) // 10 - 1 if K >= 10 else -1], 4)],
            "quantize_ms_median": round(q_ms[K // 2], 4),
            "quantize_ms_p10_p90": [round(q_ms[K // 10], 4), round(q_ms[(9 * K) // 10 - 1 if K >= 10 else -1], 4)],
            "decode_ms_median": round(d_ms[K // 2], 4),
            "quantize_frac_mfma": round(n_vec * quantize_mfma_flops(w["d"], "mse") / (q_avg * 1e-3) / 1e12
                                        / BF16_MFMA_PEAK_TFLOPS, 4),
            "quantize_prod_mvec_s": round(p_vec / (p_ms * 1e-3) / 1e6, 1),
            "quantize_prod_gb_s": round(p_vec * (256 + 32 + 16 + 8) / (p_ms * 1e-3) / 1e9, 1),
            "quantize_prod_ms_median_flushed": round(p_ms, 4),
            "quantize_prod_frac_mfma": round(p_vec * quantize_mfma_flops(w["d"], "prod") / (p_ms * 1e-3) / 1e12
                                             / BF16_MFMA_PEAK_TFLOPS, 4),
            "decode_append_ms": round(a_ms, 4),
            "decode_ms_flushed": round(d_flushed_ms, 4),
            "vector_search": vsearch,
            "c4_sweep": c4,
            "outlier_split": split,
            "decode_1m": dec1m,
            "outlier_split_decode": split_dec,
            "outlier_split_32x4_96x3": split_35,
            "outlier_split_decode_32x4_96x3": split_dec_35,
            "wall_s_timed_region": round(wall, 3),
        },
        "roofline": {"bound": "hbm", "achieved": round(d_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(d_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "decode attention call (prep + split main loop + combine), "
                               f"{d_bytes} algorithmic bytes per launch"},
    }
    if not args.no_cpu_baseline:
        print("timing the oracle on the host", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(syn)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
