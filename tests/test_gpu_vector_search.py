"""Vector-search scoring at large head dimensions ([NIK] "Experiments":
nearest neighbours with d = 1536 and 3072), against the fp64 oracle:

* quantize at d = 320 to 4096 (mse and prod, fp32 and bf16 inputs, one and
  several groups): norms within 2 ulp, rotated coordinates within 2e-5 of
  fp64, codes and QJL signs bit-exact when the oracle's rule is fed the
  kernel's own rotated coordinates / projections, flips against the full fp64
  path only within the 1e-5 band, the QJL projection within 5e-4 |e| of fp64;
* inner products <y, x~> straight from an oracle-packed database, element
  by element within rel 1e-3 / abs 1e-4 on the scale |y| |x~| / sqrt(d);
* D_prod measured from the GPU's inner products for prod b = 3 at d = 1536:
  E (<y,x> - <y,x~>)^2 d / (|x|^2 |y|^2) = (pi/2 - 1/d) d C(f_X, 2) for y
  independent of x (within 10 %).
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import tq_synth as syn
from tq_testlib import MAX_FLIP_RATE, TIE_BAND, assert_scores_close, near_threshold, ulp_diff_f32

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _mats(d, prod, head=0):
    Pi = syn.rotation(d, syn.CFG_TEST, syn.T_K, 100 + head)
    S = syn.gaussian_matrix(d, syn.CFG_TEST, syn.T_K, 100 + head) if prod else None
    return Pi, S


# d a multiple of 128 runs the matrix-core GEMM kernels; d = 320 the fp32 kernel
@pytest.mark.parametrize("d,variant,bits,dt", [(512, "mse", 2, "f32"), (1536, "mse", 3, "f32"), (1536, "prod", 3, "f32"),
                                               (3072, "prod", 2, "f32"), (640, "mse", 4, "f32"), (768, "prod", 1, "f32"),
                                               (1536, "prod", 4, "bf16"), (1024, "mse", 1, "bf16"), (320, "prod", 2, "f32"),
                                               (4096, "prod", 3, "f32")])
def test_large_d_quantize_parity(gpu_lib, d, variant, bits, dt):
    tq = gpu_lib
    n = 300
    print(f"large-d quantize d={d} {variant} b={bits} {dt} n={n}", flush=True)
    Pi, S = _mats(d, variant == "prod")
    q = tq.Quantizer(d, bits, variant, Pi, S)
    x = syn.gaussian_queries(n, d, syn.CFG_TEST, batch=d)  # Gaussian embeddings, fp32
    x[7] = 0.0
    xd = torch.from_numpy(x).to(DEV)
    if dt == "bf16":
        xd = xd.to(torch.bfloat16)
        x = xd.float().cpu().numpy()  # the oracle sees the rounded inputs
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
        rn = r["rnorms"].cpu().numpy()
        assert rn[7] == 0
        assert not r["signs"].cpu().numpy()[7].any()
        if planes > 0:
            same = valid & np.all(O.unpack_vector_layout(r["codes"].cpu().numpy(), planes, d) == ref["idx"], axis=1)
        else:
            same = valid.copy()
        assert same.sum() > 0.9 * valid.sum()
        assert np.allclose(rn[same], ref["gamma"][same], rtol=2e-5, atol=2e-7)
        # the QJL projection S r = S Pi^T e against fp64, relative to |e|
        perr = np.abs(proj[same] - ref["p"][same]).max(axis=1)
        assert np.all(perr <= 5e-4 * ref["gamma"][same]), (perr / ref["gamma"][same]).max()


def test_large_d_grouped_quantize(gpu_lib):
    """One launch over 3 groups, each with its own quantizer (d = 768, prod b = 3, n = 300 per group)."""
    tq = gpu_lib
    d, bits, n, G = 768, 3, 300, 3
    print(f"large-d grouped quantize d={d} G={G}", flush=True)
    mats = [_mats(d, True, head=h) for h in range(G)]
    qs = [tq.Quantizer(d, bits, "prod", Pi, S) for Pi, S in mats]
    x = np.stack([syn.gaussian_queries(n, d, syn.CFG_TEST, batch=900 + h) for h in range(G)])
    r = tq.quantize(qs, torch.from_numpy(x).to(DEV), rot_dbg=True, proj_dbg=True)
    torch.cuda.synchronize()
    cb = O.codebook(d, bits - 1)
    codes = r["codes"].cpu().numpy().reshape(G, n, -1)
    rot = r["rot"].cpu().numpy().reshape(G, n, d)
    for h, (Pi, S) in enumerate(mats):
        ref = O.quantize_prod(x[h], Pi, S, cb)
        assert ulp_diff_f32(r["norms"].cpu().numpy()[h], ref["nu"].astype(np.float32)).max() <= 2
        assert np.abs(rot[h] - ref["y"]).max() < 2e-5
        assert np.array_equal(codes[h], O.pack_vector_layout(O.nearest_index(rot[h].astype(np.float64), cb), bits - 1))


def _oracle_database(d, variant, bits, n, head):
    Pi, S = _mats(d, variant == "prod", head)
    x = syn.gaussian_queries(n, d, syn.CFG_TEST, batch=1000 + head)
    planes = bits - 1 if variant == "prod" else bits
    cb = O.codebook(d, planes)
    if variant == "prod":
        r = O.quantize_prod(x, Pi, S, cb)
        xt = O.dequantize_prod(r["idx"], r["signs"], r["norms"], r["rnorms"], Pi, S, cb)
    else:
        r = O.quantize_mse(x, Pi, cb)
        xt = O.dequantize_mse(r["idx"], r["norms"], Pi, cb)
    db = {"norms": r["norms"], "codes": O.pack_vector_layout(r["idx"], planes) if planes else None}
    if variant == "prod":
        db["signs"] = O.pack_bits(r["signs"])
        db["rnorms"] = r["rnorms"]
    return Pi, S, x, xt, db


@pytest.mark.parametrize("d,variant,bits,n", [(1536, "prod", 3, 3000), (1536, "mse", 2, 3000), (3072, "prod", 2, 1200),
                                              (768, "prod", 1, 1000)])
def test_large_d_inner_products_parity(gpu_lib, d, variant, bits, n):
    tq = gpu_lib
    m = 4
    print(f"large-d inner products d={d} {variant} b={bits} n={n} m={m}", flush=True)
    Pi, S, x, xt, db = _oracle_database(d, variant, bits, n, 1)
    q = tq.Quantizer(d, bits, variant, Pi, S)
    y = syn.gaussian_queries(m, d, syn.CFG_TEST, batch=5000 + d)
    dev = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    got = tq.inner_products(q, dev(y), dev(db["codes"]), dev(db["norms"]), dev(db.get("signs")),
                            dev(db.get("rnorms"))).cpu().numpy()
    want = O.inner_products(y, xt)
    assert_scores_close(got, want, y, xt)


def test_vector_search_dprod(gpu_lib):
    tq = gpu_lib
    d, bits, n, m = 1536, 3, 4000, 8
    print(f"D_prod d={d} prod b={bits} n={n} m={m}", flush=True)
    Pi, S, x, xt, db = _oracle_database(d, "prod", bits, n, 2)
    q = tq.Quantizer(d, bits, "prod", Pi, S)
    y = syn.gaussian_queries(m, d, syn.CFG_TEST, batch=6000)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    got = tq.inner_products(q, dev(y), dev(db["codes"]), dev(db["norms"]), dev(db["signs"]), dev(db["rnorms"]))
    got = got.cpu().numpy().astype(np.float64)
    true = y.astype(np.float64) @ x.astype(np.float64).T
    nx = np.sum(x.astype(np.float64) ** 2, axis=1)
    ny = np.sum(y.astype(np.float64) ** 2, axis=1)
    dprod = np.mean((true - got) ** 2 * d / (ny[:, None] * nx[None, :]))
    _, _, cost = tq.codebook_build(d, bits - 1)
    want = (math.pi / 2 - 1 / d) * d * cost
    assert abs(dprod - want) < 0.1 * want, (dprod, want)
