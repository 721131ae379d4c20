"""Vector search at the benchmark's full sizes and launch configuration
([NIK] "Experiments": 100K embeddings at d = 1536 and 3072; TurboQuant_prod
b = 3, 16 queries), checked on sampled outputs against the fp64 oracle.

* Scoring: the database is seeded random bits and norms (any bits are a valid
  packed database), scored in full by tq_search_scores and tq_inner_products;
  256 sampled records are dequantized by the oracle, and the sampled scores
  must agree element by element within rel 1e-3 / abs 1e-4 on the scale
  |y| |x~| / sqrt(d).
* Indexing: 100,000 Gaussian embeddings quantized by the GEMM kernels in one
  call; 128 sampled rows against the oracle's quantize_prod: norms within
  2 ulp, codes equal except within 1e-5 of a decision midpoint, signs equal
  except within 1e-5 |S_j| of the hyperplane, rnorms within 2e-5 where the
  codes agree.
"""
import numpy as np
import pytest
import torch

import oracle as O
import tq_synth as syn
from tq_testlib import TIE_BAND, assert_scores_close, near_threshold, ulp_diff_f32

pytestmark = pytest.mark.gpu
DEV = "cuda"
N, M, BITS = 100000, 16, 3


def _quantizer(tq, d):
    Pi = syn.rotation(d, syn.CFG_SWEEP, syn.T_K, 500 + d)
    S = syn.gaussian_matrix(d, syn.CFG_SWEEP, syn.T_K, 500 + d)
    return Pi, S, tq.Quantizer(d, BITS, "prod", Pi, S)


@pytest.mark.parametrize("d", [1536, 3072])
def test_fullsize_scores_sampled(gpu_lib, d):
    tq = gpu_lib
    print(f"full-size scoring d={d} n={N} m={M}", flush=True)
    Pi, S, q = _quantizer(tq, d)
    planes = BITS - 1
    db = syn.random_packed_group(N, d, planes * d // 8, 4, syn.CFG_SWEEP, 0, d, lognormal_sigma=0.25,
                                 norm_base=float(np.sqrt(d)))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    codes, signs, norms, rnorms = dev(db["kcodes"]), dev(db["ksigns"]), dev(db["knorms"]), dev(db["krnorms"])
    y = syn.gaussian_queries(M, d, syn.CFG_SWEEP, batch=d)
    yd = dev(y)
    got_mfma = tq.search_scores(q, yd, codes, norms, signs, rnorms).cpu().numpy()
    got_fp32 = tq.inner_products(q, yd, codes, norms, signs, rnorms).cpu().numpy()
    pick = np.sort(np.random.default_rng(d).choice(N, 256, replace=False))
    cb = O.codebook(d, planes)
    idx = O.unpack_vector_layout(db["kcodes"][pick], planes, d)
    z = O.unpack_bits(db["ksigns"][pick], d)
    xt = O.dequantize_prod(idx, z, db["knorms"][pick], db["krnorms"][pick], Pi, S, cb)
    want = O.inner_products(y, xt)
    assert_scores_close(got_mfma[:, pick], want, y, xt)
    assert_scores_close(got_fp32[:, pick], want, y, xt)


@pytest.mark.parametrize("d", [1536, 3072])
def test_fullsize_index_sampled(gpu_lib, d):
    tq = gpu_lib
    print(f"full-size indexing d={d} n={N}", flush=True)
    Pi, S, q = _quantizer(tq, d)
    x = syn.gaussian_queries(N, d, syn.CFG_SWEEP, batch=100 + d)  # Gaussian embeddings, fp32
    r = tq.quantize_prod(q, torch.from_numpy(x).to(DEV))
    torch.cuda.synchronize()
    pick = np.sort(np.random.default_rng(7 + d).choice(N, 128, replace=False))
    planes = BITS - 1
    cb = O.codebook(d, planes)
    ref = O.quantize_prod(x[pick], Pi, S, cb)
    assert ulp_diff_f32(r["norms"].cpu().numpy()[pick], ref["nu"].astype(np.float32)).max() <= 2
    idx = O.unpack_vector_layout(r["codes"].cpu().numpy()[pick], planes, d)
    fl = idx != ref["idx"]
    assert fl.mean() < 1e-4
    if fl.any():
        assert np.all(near_threshold(ref["y"][fl], cb, TIE_BAND))
    z = O.unpack_bits(r["signs"].cpu().numpy()[pick], d)
    same = ~fl.any(axis=1)
    fz = (z != ref["signs"]) & same[:, None]
    if fz.any():
        srow = np.linalg.norm(S, axis=1)
        assert np.all((np.abs(ref["p"]) / srow[None, :])[fz] <= TIE_BAND)
    rn = r["rnorms"].cpu().numpy()[pick]
    assert np.allclose(rn[same], ref["gamma"][same], rtol=2e-5, atol=2e-7)
