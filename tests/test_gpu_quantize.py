"""GPU parity of quantize / dequantize / inner products against the fp64 oracle.

Bars (from the written method and the pass criteria):
  * codes, bit layout and QJL signs are bit-exact when the oracle's nearest-
    centroid rule is fed the kernel's own rotated coordinates / projections;
  * against the full fp64 path, fewer than 1e-4 of codes flip, and only within
    +-1e-5 of a threshold; norms within 2 ulp;
  * dequantize within 1e-5 * |x| given identical codes.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import tq_synth as syn
from tq_testlib import (MAX_FLIP_RATE, TIE_BAND, near_threshold, oracle_cache_slice, quantizer,
                        ulp_diff_f32)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(n, d, dtype, head):
    if dtype == "f32":
        x = syn.small_keys(n, d, config=syn.CFG_TEST)
    else:
        x = syn.kv_vectors(n, d, syn.CFG_TEST, syn.T_K, 0, head, lognormal_sigma=0.5)
    x[3] = 0.0            # zero vector
    x[n - 1] = 0.0
    return x


def _to_dev(x, dtype):
    t = torch.from_numpy(x).to(DEV)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


CASES = [(d, v, b, dt) for d in (64, 128, 256) for v in ("mse", "prod") for b in (1, 2, 3, 4)
         for dt in ("bf16", "f32")]


@pytest.mark.parametrize("d,variant,bits,dtype", CASES)
def test_quantize_parity(gpu_lib, d, variant, bits, dtype):
    tq = gpu_lib
    n = 1000  # not a multiple of the 32-vector wave tile
    print(f"case d={d} {variant} b={bits} {dtype} n={n}", flush=True)
    q, Pi, S = quantizer(tq, d, bits, variant, syn.CFG_TEST, syn.T_K, 1)
    x = _inputs(n, d, dtype, 1)
    xd = _to_dev(x, dtype)
    if variant == "prod":
        r = tq.quantize_prod(q, xd, rot_dbg=True, proj_dbg=True)
    else:
        r = tq.quantize_mse(q, xd, rot_dbg=True)
    torch.cuda.synchronize()
    planes = q.planes
    cb = O.codebook(d, planes)
    rot = r["rot"].cpu().numpy()
    norms = r["norms"].cpu().numpy()
    nu64 = np.linalg.norm(x.astype(np.float64), axis=1)
    valid = nu64 > 0
    # norms: |x|_2 rounded to float32, within 2 ulp
    assert ulp_diff_f32(norms, nu64.astype(np.float32)).max() <= 2
    # codes are exactly the nearest-centroid rule applied to the kernel's own y
    if planes > 0:
        codes = r["codes"].cpu().numpy()
        idx_fed = O.nearest_index(rot.astype(np.float64), cb)
        idx_fed[~valid] = 0
        assert np.array_equal(codes, O.pack_vector_layout(idx_fed, planes))
    # against the fp64 path
    if variant == "prod":
        ref = O.quantize_prod(x, Pi, S, cb)
    else:
        ref = O.quantize_mse(x, Pi, cb)
    yerr = np.abs(rot[valid] - ref["y"][valid]).max()
    assert yerr < 2e-5, yerr
    if planes > 0:
        idx_gpu = O.unpack_vector_layout(codes, planes, d)
        flips = idx_gpu[valid] != ref["idx"][valid]
        assert flips.mean() < MAX_FLIP_RATE, flips.mean()
        if flips.any():
            assert np.all(near_threshold(ref["y"][valid][flips], cb, TIE_BAND))
        same = valid & np.all(idx_gpu == ref["idx"], axis=1)
    else:
        same = valid
    if variant == "prod":
        proj = r["proj"].cpu().numpy()
        signs = r["signs"].cpu().numpy()
        fed = proj >= 0
        fed[~valid] = False
        assert np.array_equal(signs, O.pack_bits(fed))
        rn = r["rnorms"].cpu().numpy()
        assert np.all(rn[~valid] == 0)
        assert np.allclose(rn[same], ref["gamma"][same], rtol=2e-5, atol=2e-7)
        srow = np.linalg.norm(S, axis=1)
        perr = np.abs(proj[same] - ref["p"][same]) / srow[None, :]
        assert perr.max() < 1e-5, perr.max()
        sflip = O.unpack_bits(signs, d)[same] != ref["signs"][same]
        if sflip.any():
            assert np.all((np.abs(ref["p"][same]) / srow[None, :])[sflip] <= TIE_BAND)


@pytest.mark.parametrize("d,bits", [(64, 1), (64, 4), (128, 2), (128, 3), (256, 2), (256, 3)])
def test_quantize_block_layout_grouped(gpu_lib, d, bits):
    tq = gpu_lib
    G, n = 3, 992
    print(f"case block32 d={d} b={bits} G={G} n={n}", flush=True)
    qs, xs = [], []
    for gi in range(G):
        q, Pi, _ = quantizer(tq, d, bits, "mse", syn.CFG_TEST, syn.T_V, gi)
        qs.append(q)
        xs.append(syn.kv_vectors(n, d, syn.CFG_TEST, syn.T_V, 0, gi))
    x = np.stack(xs)
    x[1, 5] = 0.0
    xd = torch.from_numpy(x).to(DEV).to(torch.bfloat16)
    r = tq.quantize(qs, xd, layout="block32", rot_dbg=True)
    rv = tq.quantize(qs, xd, layout="vector", rot_dbg=True)
    torch.cuda.synchronize()
    cb = O.codebook(d, bits)
    codes = r["codes"].cpu().numpy().reshape(G, -1)
    rot = r["rot"].cpu().numpy()
    assert np.array_equal(rot, rv["rot"].cpu().numpy())
    assert np.array_equal(r["norms"].cpu().numpy(), rv["norms"].cpu().numpy())
    for gi in range(G):
        idx = O.nearest_index(rot[gi].astype(np.float64), cb)
        idx[np.linalg.norm(x[gi], axis=1) == 0] = 0
        assert np.array_equal(codes[gi], O.pack_block_layout(idx, bits).reshape(-1))
        assert np.array_equal(rv["codes"].cpu().numpy().reshape(G, -1)[gi],
                              O.pack_vector_layout(idx, bits).reshape(-1))


@pytest.mark.parametrize("d,variant,bits,layout", [(64, "mse", 2, "vector"), (128, "prod", 3, "vector"),
                                                   (128, "mse", 3, "block32"), (256, "prod", 1, "vector"),
                                                   (256, "mse", 4, "block32"), (128, "prod", 4, "vector")])
def test_dequantize_parity(gpu_lib, d, variant, bits, layout):
    tq = gpu_lib
    n = 320
    q, Pi, S = quantizer(tq, d, bits, variant, syn.CFG_TEST, syn.T_K, 2)
    x = syn.kv_vectors(n, d, syn.CFG_TEST, syn.T_K, 1, 2, lognormal_sigma=0.5)
    ref = oracle_cache_slice(x, d, bits, variant, Pi, S, layout)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    out = tq.dequantize(q, dev(ref["codes"]) if "codes" in ref else None, dev(ref["norms"]),
                        dev(ref["signs"]) if "signs" in ref else None,
                        dev(ref["rnorms"]) if "rnorms" in ref else None, layout=layout)
    got = out.cpu().numpy()
    nu = np.linalg.norm(x.astype(np.float64), axis=1)
    err = np.abs(got - ref["xt"]).max(axis=1) / nu
    assert err.max() < 1e-5, err.max()


@pytest.mark.parametrize("d,variant,bits", [(128, "mse", 2), (128, "prod", 3), (64, "prod", 2), (256, "mse", 1)])
def test_inner_products_parity(gpu_lib, d, variant, bits):
    tq = gpu_lib
    n, m = 777, 5
    q, Pi, S = quantizer(tq, d, bits, variant, syn.CFG_TEST, syn.T_K, 3)
    x = syn.kv_vectors(n, d, syn.CFG_TEST, syn.T_K, 2, 3)
    ref = oracle_cache_slice(x, d, bits, variant, Pi, S, "vector")
    y = syn.gaussian_queries(m, d, syn.CFG_TEST)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    out = tq.inner_products(q, dev(y), dev(ref["codes"]) if "codes" in ref else None, dev(ref["norms"]),
                            dev(ref["signs"]) if "signs" in ref else None,
                            dev(ref["rnorms"]) if "rnorms" in ref else None).cpu().numpy()
    want = O.inner_products(y, ref["xt"])
    scale = np.linalg.norm(y, axis=1)[:, None] * np.linalg.norm(x.astype(np.float64), axis=1)[None, :]
    assert (np.abs(out - want) / scale).max() < 1e-5


def test_small_keys_distortion(gpu_lib):
    """4096 fp32 keys, d=128, mse b=2: D_mse and the inner-product distortion with
    16 Gaussian queries match the oracle on the same inputs and sit near d*C(f_X,2)."""
    tq = gpu_lib
    d, bits, n = 128, 2, 4096
    q, Pi, _ = quantizer(tq, d, bits, "mse", syn.CFG_SMALL_KEYS, syn.T_K, 0)
    x = syn.small_keys(n, d)
    xd = torch.from_numpy(x).to(DEV)
    r = tq.quantize_mse(q, xd)
    xt = tq.dequantize(q, r["codes"], r["norms"]).cpu().numpy().astype(np.float64)
    y = syn.gaussian_queries(16, d, syn.CFG_SMALL_KEYS)
    ip = tq.inner_products(q, torch.from_numpy(y).to(DEV), r["codes"], r["norms"]).cpu().numpy()
    x64 = x.astype(np.float64)
    nx2 = np.sum(x64 * x64, axis=1)
    dmse = np.mean(np.sum((x64 - xt) ** 2, axis=1) / nx2)
    ref = O.quantize_mse(x, Pi, O.codebook(d, bits))
    xr = O.dequantize_mse(ref["idx"], ref["norms"], Pi, O.codebook(d, bits))
    dmse_ref = np.mean(np.sum((x64 - xr) ** 2, axis=1) / nx2)
    _, cost, _ = O.lloyd_max(d, bits)
    assert abs(dmse - dmse_ref) < 1e-5
    assert abs(dmse - d * cost) < 0.01, (dmse, d * cost)
    true_ip = y.astype(np.float64) @ x64.T
    ny2 = np.sum(y.astype(np.float64) ** 2, axis=1)
    dprod = np.mean((true_ip - ip) ** 2 * d / (ny2[:, None] * nx2[None, :]))
    dprod_ref = np.mean((true_ip - y.astype(np.float64) @ xr.T) ** 2 * d / (ny2[:, None] * nx2[None, :]))
    assert abs(dprod - dprod_ref) < 1e-4 * dprod_ref + 1e-6
    assert abs(dprod - d * cost) < 0.02, (dprod, d * cost)
