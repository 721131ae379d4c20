"""GPU parity of decode attention over an outlier-split cache at the full
benchmark size (batch 8, 64/8 heads, head_dim 128, context 131072; keys
TurboQuant_prod with 32 channels at 3 bits and 96 at 2, each KV head with its
own channel lists, values TurboQuant_mse with the same split, codes in the
BLOCK32 layout; [NIK]
"Experiments", KV cache), in the launch
configuration the benchmark times. Two sampled (batch, KV head) groups are
quantized and packed by the fp64 oracle from seeded vectors with per-token
LogNormal(0, 0.5) scales; every other group holds seeded random bits and
positive norms. All 8 query heads of each sampled group must match the oracle's
dequantize-then-attend within rtol 1e-3 / atol 1e-4, at the full context and at
a ragged length that ends inside a 32-token chunk."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import tq_synth as syn
from tq_testlib import allclose_report

pytestmark = pytest.mark.gpu
DEV = "cuda"
B, HQ, HKV, D, T = 8, 64, 8, 128, 131072
G = HQ // HKV
KSPEC = [(32, "prod", 3), (96, "prod", 2)]
VSPEC = [(32, "mse", 3), (96, "mse", 2)]
SAMPLED = [(0, 0), (5, 3)]
RAGGED = {5: T - 777}


def _planes(bits, var):
    return bits - 1 if var == "prod" else bits


def _side(tq, spec, tensor, chans, seed):
    """Quantizers and oracle parts per (part, KV head), and device records full of
    seeded random bits and positive norms."""
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    qs, parts, recs = [], [], []
    for p, (n, var, bits) in enumerate(spec):
        planes = _planes(bits, var)
        qg, pg = [], []
        for g in range(HKV):
            Pi = syn.rotation(n, syn.CFG_DECODE_128K, tensor, 300 + 10 * p + g)
            S = syn.gaussian_matrix(n, syn.CFG_DECODE_128K, tensor, 300 + 10 * p + g) if var == "prod" else None
            qg.append(tq.Quantizer(n, bits, var, Pi, S))
            part = {"channels": chans[p][g], "variant": var, "Pi": Pi, "centroids": O.codebook(n, planes)}
            if S is not None:
                part["S"] = S
            pg.append(part)
        qs.append(qg)
        parts.append(pg)
        r = {"norms": 4.0 + 26.0 * torch.rand((B, HKV, T), device=DEV, generator=gen),
             "codes": torch.randint(0, 256, (B, HKV, T, planes * n // 8), dtype=torch.uint8, device=DEV, generator=gen)}
        if var == "prod":
            r["signs"] = torch.randint(0, 256, (B, HKV, T, n // 8), dtype=torch.uint8, device=DEV, generator=gen)
            r["rnorms"] = 0.2 + 0.3 * torch.rand((B, HKV, T), device=DEV, generator=gen)
        recs.append(r)
    return qs, parts, recs


def _pack_group(x, spec, parts_g, recs, b, g):
    """Oracle quantize_split of one group's vectors, written into the device records."""
    res = O.quantize_split(x, parts_g)
    for p, (n, var, bits) in enumerate(spec):
        planes = _planes(bits, var)
        recs[p]["norms"][b, g] = torch.from_numpy(res[p]["norms"].astype(np.float32)).to(DEV)
        # keys VECTOR, values (mse) BLOCK32, the layouts of a split cache
        pack = O.pack_vector_layout if var == "prod" else O.pack_block_layout
        codes = pack(res[p]["idx"], planes).reshape(T, planes * n // 8)
        recs[p]["codes"][b, g] = torch.from_numpy(codes).to(DEV)
        if var == "prod":
            recs[p]["signs"][b, g] = torch.from_numpy(O.pack_bits(res[p]["signs"])).to(DEV)
            recs[p]["rnorms"][b, g] = torch.from_numpy(res[p]["rnorms"].astype(np.float32)).to(DEV)
    return res


def test_split_decode_full_size(gpu_lib):
    tq = gpu_lib
    print(f"split decode full size B={B} Hq={HQ} Hkv={HKV} d={D} T={T}", flush=True)
    # every KV head keeps its own 32 largest-RMS channels (from a sample of that head)
    order = np.stack([np.argsort(-np.sqrt(np.mean(syn.kv_vectors(4096, D, syn.CFG_DECODE_128K, syn.T_K, 0, 40 + g)
                                                  .astype(np.float64) ** 2, axis=0)), kind="stable")
                      for g in range(HKV)])
    chans = [order[:, :32], order[:, 32:]]  # per part: [HKV][d_p]
    assert any(set(chans[0][g]) != set(chans[0][0]) for g in range(1, HKV))
    kq, kparts, krecs = _side(tq, KSPEC, syn.T_K, chans, 4101)
    vq, vparts, vrecs = _side(tq, VSPEC, syn.T_V, chans, 4102)
    oracle = {}
    for b, g in SAMPLED:
        print(f"  oracle packs group (b={b}, g={g})", flush=True)
        xk = syn.kv_vectors(T, D, syn.CFG_DECODE_128K, syn.T_K, b, 40 + g, lognormal_sigma=0.5)
        rk = _pack_group(xk, KSPEC, [kparts[p][g] for p in range(2)], krecs, b, g)
        del xk
        xv = syn.kv_vectors(T, D, syn.CFG_DECODE_128K, syn.T_V, b, 40 + g, lognormal_sigma=0.5)
        rv = _pack_group(xv, VSPEC, [vparts[p][g] for p in range(2)], vrecs, b, g)
        del xv
        oracle[(b, g)] = (rk, rv)
    k = tq.SplitKV([(kq[p], chans[p], krecs[p]) for p in range(2)])
    v = tq.SplitKV([(vq[p], chans[p], vrecs[p]) for p in range(2)])
    q = syn.decode_queries(B, HQ, D, syn.CFG_DECODE_128K)
    lens = np.array([RAGGED.get(b, T) for b in range(B)], np.int32)
    scale = 1 / math.sqrt(D)
    got = tq.decode_attention_split(torch.from_numpy(q).to(DEV).to(torch.bfloat16), k, v,
                                    torch.from_numpy(lens).to(DEV), scale).cpu().numpy()
    assert np.all(np.isfinite(got))
    for b, g in SAMPLED:
        print(f"  oracle attends group (b={b}, g={g}) over {lens[b]} tokens", flush=True)
        rk, rv = oracle[(b, g)]
        want = O.decode_attention_split(q[b:b + 1, g * G:(g + 1) * G], [[(rk, [kparts[p][g] for p in range(2)])]],
                                        [[(rv, [vparts[p][g] for p in range(2)])]], lens[b:b + 1], scale, D)
        nbad, emax = allclose_report(got[b:b + 1, g * G:(g + 1) * G], want)
        assert nbad == 0, (b, g, nbad, emax)
