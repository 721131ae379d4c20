"""GPU parity of decode attention over outlier-split caches
(tq_decode_attention_split; [NIK] "Experiments", KV cache: outlier channels at
more bits) against the oracle's decode_attention_split on oracle-packed
records (keys VECTOR, values BLOCK32): outputs within rtol 1e-3 / atol 1e-4,
with NaN norms in every record past a sequence's length.
Cases: the pages' split of a
128-channel head (32 channels at 3 bits, 96 at 2; prod keys, mse values) with
GQA 8 and ragged lengths; every KV head with its own channel lists (its
largest-RMS channels); parts that drop channels, with different channel
lists for keys and values, and an empty context; GQA 1 at head_dim 64; every
plane count of key and value parts; head_dim 256; splits of several chunks."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import tq_synth as syn
from tq_testlib import allclose_report

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _order(x):
    rms = np.sqrt(np.mean(x.astype(np.float64) ** 2, axis=0))
    return np.argsort(-rms, kind="stable")


def _build_side(tq, B, Hkv, T, dim, spec, tensor, seed):
    """spec: [(n_channels, variant, bits)]; each KV head picks its own channels
    from the RMS order of its batch-0 vectors (largest first), parts in order,
    so heads whose outliers sit elsewhere get different lists."""
    chans = [np.zeros((Hkv, n), np.int64) for n, _, _ in spec]  # per part: [Hkv][n]
    for g in range(Hkv):
        order = _order(syn.kv_vectors(T, dim, syn.CFG_TEST, tensor, 0, seed + g, lognormal_sigma=0.5))
        off = 0
        for p, (n, _, _) in enumerate(spec):
            chans[p][g] = order[off:off + n]
            off += n
    parts_g, qs = [], []  # per part: list over g of oracle parts / quantizers
    for p, (n, var, bits) in enumerate(spec):
        planes = bits - 1 if var == "prod" else bits
        pg, qg = [], []
        for g in range(Hkv):
            Pi = syn.rotation(n, syn.CFG_TEST, tensor, 200 + 10 * p + g)
            S = syn.gaussian_matrix(n, syn.CFG_TEST, tensor, 200 + 10 * p + g) if var == "prod" else None
            part = {"channels": chans[p][g], "variant": var, "Pi": Pi, "centroids": O.codebook(n, planes)}
            if S is not None:
                part["S"] = S
            pg.append(part)
            qg.append(tq.Quantizer(n, bits, var, Pi, S))
        parts_g.append(pg)
        qs.append(qg)
    oracle_side = [[None] * Hkv for _ in range(B)]
    recs = []
    for p, (n, var, bits) in enumerate(spec):
        planes = bits - 1 if var == "prod" else bits
        r = {"norms": np.zeros((B, Hkv, T), np.float32)}
        if planes:
            r["codes"] = np.zeros((B, Hkv, T, planes * n // 8), np.uint8)
        if var == "prod":
            r["signs"] = np.zeros((B, Hkv, T, n // 8), np.uint8)
            r["rnorms"] = np.zeros((B, Hkv, T), np.float32)
        recs.append(r)
    for b in range(B):
        for g in range(Hkv):
            x = syn.kv_vectors(T, dim, syn.CFG_TEST, tensor, b, seed + g, lognormal_sigma=0.5)
            parts = [parts_g[p][g] for p in range(len(spec))]
            res = O.quantize_split(x, parts)
            oracle_side[b][g] = (res, parts)
            for p, (n, var, bits) in enumerate(spec):
                planes = bits - 1 if var == "prod" else bits
                recs[p]["norms"][b, g] = res[p]["norms"]
                if planes:
                    # keys VECTOR, values (mse) BLOCK32, the layouts of a split cache
                    if tensor == syn.T_K:
                        recs[p]["codes"][b, g] = O.pack_vector_layout(res[p]["idx"], planes)
                    else:
                        recs[p]["codes"][b, g] = O.pack_block_layout(res[p]["idx"], planes).reshape(T, -1)
                if var == "prod":
                    recs[p]["signs"][b, g] = O.pack_bits(res[p]["signs"])
                    recs[p]["rnorms"][b, g] = res[p]["rnorms"]
    dev = {}
    side = []
    for p in range(len(spec)):
        rd = {k: torch.from_numpy(np.ascontiguousarray(v)).to(DEV) for k, v in recs[p].items()}
        side.append((qs[p], chans[p], rd))
    return tq.SplitKV(side), oracle_side


CASES = [
    # name, B, Hq, Hkv, dim, T, lens, key spec, value spec
    ("pages_32x3_96x2_gqa8", 2, 16, 2, 128, 300, [300, 177],
     [(32, "prod", 3), (96, "prod", 2)], [(32, "mse", 3), (96, "mse", 2)]),
    ("dropped_channels_empty", 2, 8, 1, 128, 513, [513, 0],
     [(64, "prod", 3), (32, "mse", 2)], [(32, "mse", 4), (64, "mse", 2)]),
    ("gqa1_d64", 3, 4, 4, 64, 40, [40, 1, 17],
     [(32, "mse", 2), (32, "prod", 2)], [(32, "mse", 3), (32, "mse", 1)]),
    # the 3.5-bit setting: 32 channels at 4 bits and 96 at 3 (prod keys, mse values)
    ("pages_32x4_96x3_gqa8", 2, 16, 2, 128, 257, [257, 100],
     [(32, "prod", 4), (96, "prod", 3)], [(32, "mse", 4), (96, "mse", 3)]),
    # every plane count of the key parts (prod b=1 is signs only, mse b=1 is one
    # plane, prod b=4 has three planes and signs), four parts per side
    ("all_key_plane_counts", 2, 8, 2, 128, 150, [150, 61],
     [(32, "prod", 1), (32, "mse", 1), (32, "mse", 3), (32, "prod", 4)], [(64, "mse", 4), (64, "mse", 1)]),
    ("mse4_keys_gqa4", 1, 8, 2, 128, 97, [97],
     [(64, "mse", 4), (64, "prod", 2)], [(96, "mse", 2), (32, "mse", 3)]),
    # head_dim 256: value vectors longer than 128 coordinates (the wider kernel)
    ("head_dim_256", 2, 16, 2, 256, 130, [130, 33],
     [(64, "prod", 3), (192, "prod", 2)], [(64, "mse", 3), (192, "mse", 2)]),
    # 8 KV heads at batch 1: 512 context splits of 64 tokens, so every split runs
    # two chunks of 32 (the second one's records in flight during the first) and
    # the last split ends in a partial chunk
    ("multi_chunk_splits", 1, 64, 8, 128, 20000, [19999],
     [(32, "prod", 3), (96, "prod", 2)], [(32, "mse", 3), (96, "mse", 2)]),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_split_decode_parity(gpu_lib, case):
    tq = gpu_lib
    name, B, Hq, Hkv, dim, T, lens, kspec, vspec = case
    print(f"split decode {name}", flush=True)
    T = -(-T // 32) * 32  # the value blocks need a context of whole 32-token blocks
    k, ok = _build_side(tq, B, Hkv, T, dim, kspec, syn.T_K, 11)
    v, ov = _build_side(tq, B, Hkv, T, dim, vspec, syn.T_V, 21)
    q = syn.decode_queries(B, Hq, dim, syn.CFG_TEST)
    lens = np.array(lens, np.int32)
    scale = 1 / math.sqrt(dim)
    # records past each sequence's length are never used: NaN norms there must not leak
    for side in (k, v):
        for _, _, r in side.parts:
            for b in range(B):
                for key in ("norms", "rnorms"):
                    if key in r:
                        r[key][b, :, int(lens[b]):] = float("nan")
    got = tq.decode_attention_split(torch.from_numpy(q).to(DEV).to(torch.bfloat16), k, v,
                                    torch.from_numpy(lens).to(DEV), scale).cpu().numpy()
    want = O.decode_attention_split(q, ok, ov, lens, scale, dim)
    nbad, emax = allclose_report(got, want)
    assert nbad == 0, (nbad, emax)
    for b in range(B):
        if lens[b] == 0:
            assert np.all(got[b] == 0)
    G = Hq // Hkv
    for g in range(Hkv):
        kept = np.zeros(dim, bool)
        for _, c, _ in v.parts:
            kept[np.asarray(c)[g]] = True
        assert np.all(got[:, g * G:(g + 1) * G, ~kept] == 0)
    if Hkv > 1 and sum(n for n, _, _ in kspec) < dim:
        # the heads really do keep different channels in this case
        assert any(not np.array_equal(np.sort(k.parts[0][1][0]), np.sort(k.parts[0][1][g])) for g in range(1, Hkv))
