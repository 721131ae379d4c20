"""GPU parity of decode attention over a packed KV cache against the fp64 oracle.

Caches are packed by the oracle and uploaded, so both sides read identical
packed KV. Scores and outputs must agree within rtol 1e-3 / atol 1e-4.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import tq_synth as syn
from tq_testlib import allclose_report, matrices, oracle_cache_slice

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _build(tq, B, Hq, Hkv, d, T, kbits, kvar, vbits, config, lognormal=0.5):
    kq, vq = [], []
    kPi, kS, vPi = [], [], []
    for h in range(Hkv):
        Pi, S = matrices(d, config, syn.T_K, h, kvar == "prod")
        kq.append(tq.Quantizer(d, kbits, kvar, Pi, S))
        kPi.append(Pi)
        kS.append(S if S is not None else np.zeros((d, d)))
        Pv, _ = matrices(d, config, syn.T_V, h, False)
        vq.append(tq.Quantizer(d, vbits, "mse", Pv))
        vPi.append(Pv)
    kp = kbits - (1 if kvar == "prod" else 0)
    kc = {"variant": kvar, "bits": kbits, "d": d, "max_ctx": T, "Pi": np.stack(kPi), "S": np.stack(kS),
          "codes": np.zeros((B, Hkv, T, max(kp, 1) * d // 8), np.uint8),
          "signs": np.zeros((B, Hkv, T, d // 8), np.uint8),
          "norms": np.zeros((B, Hkv, T), np.float32), "rnorms": np.zeros((B, Hkv, T), np.float32)}
    vc = {"variant": "mse", "bits": vbits, "d": d, "max_ctx": T, "Pi": np.stack(vPi),
          "codes": np.zeros((B, Hkv, T // 32, 4 * vbits * d), np.uint8),
          "norms": np.zeros((B, Hkv, T), np.float32)}
    for b in range(B):
        for h in range(Hkv):
            xk = syn.kv_vectors(T, d, config, syn.T_K, b, h, lognormal_sigma=lognormal)
            xv = syn.kv_vectors(T, d, config, syn.T_V, b, h, lognormal_sigma=lognormal)
            rk = oracle_cache_slice(xk, d, kbits, kvar, kPi[h], kS[h], "vector")
            rv = oracle_cache_slice(xv, d, vbits, "mse", vPi[h], None, "block32")
            if kp > 0:
                kc["codes"][b, h] = rk["codes"]
            kc["norms"][b, h] = rk["norms"]
            if kvar == "prod":
                kc["signs"][b, h] = rk["signs"]
                kc["rnorms"][b, h] = rk["rnorms"]
            vc["codes"][b, h] = rv["codes"].reshape(T // 32, -1)
            vc["norms"][b, h] = rv["norms"]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    kcache = tq.KVCache(kq, dev(kc["norms"]), dev(kc["codes"]) if kp > 0 else None,
                        dev(kc["signs"]) if kvar == "prod" else None,
                        dev(kc["rnorms"]) if kvar == "prod" else None)
    vcache = tq.KVCache(vq, dev(vc["norms"]), dev(vc["codes"]))
    return kcache, vcache, kc, vc


CASES = [
    # B, Hq, Hkv, d, T, kbits, kvar, vbits, lens
    (2, 16, 2, 128, 96, 3, "prod", 3, [96, 37]),
    (1, 8, 1, 128, 4096, 3, "prod", 3, [3001]),
    (2, 8, 2, 64, 160, 2, "mse", 2, [160, 65]),
    (1, 32, 2, 256, 128, 2, "prod", 1, [100]),
    (1, 8, 1, 128, 256, 4, "mse", 4, [255]),
    (4, 8, 1, 128, 64, 3, "prod", 3, [0, 1, 32, 33]),
    (1, 8, 1, 128, 512, 1, "prod", 3, [512]),
    (1, 16, 2, 256, 96, 3, "prod", 3, [90]),
    (1, 8, 2, 64, 96, 4, "prod", 4, [70]),
    (1, 8, 1, 256, 64, 4, "mse", 2, [64]),
    # GQA group sizes 1 and 2, and the largest number of KV heads (64)
    (2, 4, 4, 128, 64, 3, "prod", 3, [64, 50]),
    (1, 32, 16, 128, 96, 2, "mse", 3, [77]),
    (1, 64, 64, 64, 32, 3, "prod", 2, [29]),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}Hq{c[1]}Hkv{c[2]}d{c[3]}T{c[4]}K{c[6]}{c[5]}V{c[7]}")
def test_decode_parity(gpu_lib, case):
    tq = gpu_lib
    B, Hq, Hkv, d, T, kbits, kvar, vbits, lens = case
    print(f"case {case}", flush=True)
    kcache, vcache, kc, vc = _build(tq, B, Hq, Hkv, d, T, kbits, kvar, vbits, syn.CFG_TEST)
    q = syn.decode_queries(B, Hq, d, syn.CFG_TEST)
    qd = torch.from_numpy(q).to(DEV).to(torch.bfloat16)
    lens_d = torch.tensor(lens, dtype=torch.int32, device=DEV)
    scale = 1.0 / math.sqrt(d)
    scores = torch.full((B, Hq, T), float("nan"), dtype=torch.float32, device=DEV)
    out = tq.decode_attention(qd, kcache, vcache, lens_d, scale, scores=scores)
    out2 = tq.decode_attention(qd, kcache, vcache, lens_d, scale)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.array_equal(got, out2.cpu().numpy()), "decode is not deterministic"
    want = O.decode_attention(q, kc, vc, np.array(lens), scale)
    sc = scores.cpu().numpy()
    for b in range(B):
        if lens[b] == 0:
            assert np.all(got[b] == 0)
            continue
        nbad, emax = allclose_report(got[b], want[b])
        assert nbad == 0, (b, nbad, emax)
        for hq in range(Hq):
            nb, em = allclose_report(sc[b, hq, :lens[b]], _natural_scores(q, kc, b, hq, Hq, Hkv, lens[b], scale))
            assert nb == 0, (b, hq, nb, em)


def _natural_scores(q, kc, b, hq, Hq, Hkv, T, scale):
    """scale * <q, k~_t> from the oracle's dequantized keys (the oracle's attention
    returns max-shifted logits, so recompute the unshifted ones here)."""
    d = kc["d"]
    h = hq * Hkv // Hq
    kp = kc["bits"] - (1 if kc["variant"] == "prod" else 0)
    cb = O.codebook(d, kp)
    idx = O.unpack_vector_layout(kc["codes"][b, h, :T], kp, d) if kp > 0 else np.zeros((T, d), np.int64)
    if kc["variant"] == "prod":
        z = O.unpack_bits(kc["signs"][b, h, :T], d)
        K = O.dequantize_prod(idx, z, kc["norms"][b, h, :T], kc["rnorms"][b, h, :T], kc["Pi"][h], kc["S"][h], cb)
    else:
        K = O.dequantize_mse(idx, kc["norms"][b, h, :T], kc["Pi"][h], cb)
    return scale * (K @ q[b, hq].astype(np.float64))


def test_decode_rejects_small_workspace(gpu_lib):
    tq = gpu_lib
    kcache, vcache, _, _ = _build(tq, 1, 8, 1, 128, 64, 3, "prod", 3, syn.CFG_TEST)
    q = torch.zeros((1, 8, 128), dtype=torch.bfloat16, device=DEV)
    lens = torch.tensor([64], dtype=torch.int32, device=DEV)
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(tq.TQError) as e:
        tq.decode_attention(q, kcache, vcache, lens, 0.1, workspace=ws)
    assert e.value.status == tq.TQ_ERR_WORKSPACE
