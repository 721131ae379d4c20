"""GPU parity with the randomized Walsh-Hadamard rotation (quantizers built by
tq_quantizer_create_wht) against the fp64 oracle using Pi = H diag(signs)/sqrt(d):
quantize (codes bit-exact on the kernel's own rotated coordinates, flips only in
the +-1e-5 band, norms within 2 ulp) and decode attention over a WHT-rotated
cache (outputs within rtol 1e-3 / atol 1e-4)."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import tq_synth as syn
from tq_testlib import MAX_FLIP_RATE, TIE_BAND, allclose_report, near_threshold, ulp_diff_f32

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("d,variant,bits", [(64, "mse", 3), (128, "mse", 3), (256, "mse", 2), (128, "prod", 3),
                                            (64, "prod", 2), (256, "prod", 4)])
def test_wht_quantize_parity(gpu_lib, d, variant, bits):
    tq = gpu_lib
    n = 777
    print(f"wht quantize d={d} {variant} b={bits} n={n}", flush=True)
    signs = syn.wht_signs(d, syn.CFG_TEST, syn.T_K, 4)
    S = syn.gaussian_matrix(d, syn.CFG_TEST, syn.T_K, 4) if variant == "prod" else None
    q = tq.Quantizer.wht(d, bits, variant, signs, S)
    Pi = O.wht_rotation(signs)
    x = syn.kv_vectors(n, d, syn.CFG_TEST, syn.T_K, 0, 4, lognormal_sigma=0.5)
    x[10] = 0.0
    xd = torch.from_numpy(x).to(DEV).to(torch.bfloat16)
    r = tq.quantize_prod(q, xd, rot_dbg=True, proj_dbg=True) if variant == "prod" else tq.quantize_mse(q, xd, rot_dbg=True)
    torch.cuda.synchronize()
    planes = q.planes
    cb = O.codebook(d, planes)
    ref = O.quantize_prod(x, Pi, S, cb) if variant == "prod" else O.quantize_mse(x, Pi, cb)
    valid = ref["nu"] > 0
    assert ulp_diff_f32(r["norms"].cpu().numpy(), ref["nu"].astype(np.float32)).max() <= 2
    rot = r["rot"].cpu().numpy()
    assert np.abs(rot[valid] - ref["y"][valid]).max() < 2e-5
    if planes > 0:
        codes = r["codes"].cpu().numpy()
        fed = O.nearest_index(rot.astype(np.float64), cb)
        fed[~valid] = 0
        assert np.array_equal(codes, O.pack_vector_layout(fed, planes))
        idx = O.unpack_vector_layout(codes, planes, d)
        flips = idx[valid] != ref["idx"][valid]
        assert flips.mean() < MAX_FLIP_RATE
        if flips.any():
            assert np.all(near_threshold(ref["y"][valid][flips], cb, TIE_BAND))
    if variant == "prod":
        proj = r["proj"].cpu().numpy()
        fed = proj >= 0
        fed[~valid] = False
        assert np.array_equal(r["signs"].cpu().numpy(), O.pack_bits(fed))


def test_wht_decode_parity(gpu_lib):
    tq = gpu_lib
    B, Hq, Hkv, d, T = 2, 16, 2, 128, 320
    lens = np.array([320, 203], np.int32)
    print(f"wht decode B={B} Hq={Hq} Hkv={Hkv} d={d} T={T}", flush=True)
    kq, vq, kPi, kS, vPi = [], [], [], [], []
    for h in range(Hkv):
        ks = syn.wht_signs(d, syn.CFG_TEST, syn.T_K, 10 + h)
        vs = syn.wht_signs(d, syn.CFG_TEST, syn.T_V, 10 + h)
        S = syn.gaussian_matrix(d, syn.CFG_TEST, syn.T_K, 10 + h)
        kq.append(tq.Quantizer.wht(d, 3, "prod", ks, S))
        vq.append(tq.Quantizer.wht(d, 3, "mse", vs))
        kPi.append(O.wht_rotation(ks))
        kS.append(S)
        vPi.append(O.wht_rotation(vs))
    ck, cv = O.codebook(d, 2), O.codebook(d, 3)
    kc = {"variant": "prod", "bits": 3, "d": d, "max_ctx": T, "Pi": np.stack(kPi), "S": np.stack(kS),
          "codes": np.zeros((B, Hkv, T, 32), np.uint8), "signs": np.zeros((B, Hkv, T, 16), np.uint8),
          "norms": np.zeros((B, Hkv, T), np.float32), "rnorms": np.zeros((B, Hkv, T), np.float32)}
    vc = {"variant": "mse", "bits": 3, "d": d, "max_ctx": T, "Pi": np.stack(vPi),
          "codes": np.zeros((B, Hkv, T // 32, 4 * 3 * d), np.uint8), "norms": np.zeros((B, Hkv, T), np.float32)}
    for b in range(B):
        for h in range(Hkv):
            xk = syn.kv_vectors(T, d, syn.CFG_TEST, syn.T_K, b, 10 + h)
            xv = syn.kv_vectors(T, d, syn.CFG_TEST, syn.T_V, b, 10 + h)
            rk = O.quantize_prod(xk, kPi[h], kS[h], ck)
            rv = O.quantize_mse(xv, vPi[h], cv)
            kc["codes"][b, h] = O.pack_vector_layout(rk["idx"], 2)
            kc["signs"][b, h] = O.pack_bits(rk["signs"])
            kc["norms"][b, h] = rk["norms"]
            kc["rnorms"][b, h] = rk["rnorms"]
            vc["codes"][b, h] = O.pack_block_layout(rv["idx"], 3).reshape(T // 32, -1)
            vc["norms"][b, h] = rv["norms"]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    kcache = tq.KVCache(kq, dev(kc["norms"]), dev(kc["codes"]), dev(kc["signs"]), dev(kc["rnorms"]))
    vcache = tq.KVCache(vq, dev(vc["norms"]), dev(vc["codes"]))
    qn = syn.decode_queries(B, Hq, d, syn.CFG_TEST)
    scale = 1 / math.sqrt(d)
    out = tq.decode_attention(torch.from_numpy(qn).to(DEV).to(torch.bfloat16), kcache, vcache, dev(lens), scale)
    torch.cuda.synchronize()
    want = O.decode_attention(qn, kc, vc, lens, scale)
    nbad, emax = allclose_report(out.cpu().numpy(), want)
    assert nbad == 0, (nbad, emax)
