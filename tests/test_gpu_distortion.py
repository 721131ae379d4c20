"""Distortion measured through the GPU path for the b x variant x d sweep
([NIK] Theorem 1 and Theorem 2; the sweep shapes d in {64, 128, 256},
b in {1, 2, 3, 4}): Gaussian vectors (x/|x| uniform on the sphere for any fixed
rotation, so one rotation draw suffices) quantized and dequantized by the
library, statistics in fp64 on the host.

* mse: mean |x - x~|^2 / |x|^2 equals d C(f_X, b) within 4 standard errors;
* prod: mean (<y,x> - <y,x~>)^2 d / (|x|^2 |y|^2) over 64 query directions equals
  (pi/2 - 1/d) d C(f_X, b - 1) within 10 %, and the error has mean 0 within 4
  standard errors (unbiased).
C(f_X, b) is the oracle's Lloyd-Max cost, pinned against closed forms and the
pages' table elsewhere."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import tq_synth as syn

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_mse_distortion_on_gpu(gpu_lib, d, bits):
    tq = gpu_lib
    n = 16384
    print(f"D_mse d={d} b={bits}", flush=True)
    Pi = syn.rotation(d, syn.CFG_SWEEP, syn.T_K, 900 + bits)
    q = tq.Quantizer(d, bits, "mse", Pi)
    x = syn.gaussian_queries(n, d, syn.CFG_SWEEP, batch=d * 10 + bits)
    xd = torch.from_numpy(x).to(DEV)
    r = tq.quantize_mse(q, xd)
    xt = tq.dequantize(q, r["codes"], r["norms"]).cpu().numpy().astype(np.float64)
    x64 = x.astype(np.float64)
    rel = np.sum((x64 - xt) ** 2, axis=1) / np.sum(x64 ** 2, axis=1)
    want = d * O.lloyd_max(d, bits)[1]
    se = rel.std() / math.sqrt(n)
    assert abs(rel.mean() - want) < 4 * se, (rel.mean(), want, se)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_prod_distortion_on_gpu(gpu_lib, d, bits):
    tq = gpu_lib
    n, m = 8192, 64
    print(f"D_prod d={d} b={bits}", flush=True)
    Pi = syn.rotation(d, syn.CFG_SWEEP, syn.T_K, 950 + bits)
    S = syn.gaussian_matrix(d, syn.CFG_SWEEP, syn.T_K, 950 + bits)
    q = tq.Quantizer(d, bits, "prod", Pi, S)
    x = syn.gaussian_queries(n, d, syn.CFG_SWEEP, batch=d * 20 + bits)
    y = syn.gaussian_queries(m, d, syn.CFG_SWEEP, batch=d * 30 + bits)
    r = tq.quantize_prod(q, torch.from_numpy(x).to(DEV))
    xt = tq.dequantize(q, r["codes"], r["norms"], r["signs"], r["rnorms"]).cpu().numpy().astype(np.float64)
    x64, y64 = x.astype(np.float64), y.astype(np.float64)
    err = y64 @ xt.T - y64 @ x64.T
    norm = np.sum(y64 ** 2, axis=1)[:, None] * np.sum(x64 ** 2, axis=1)[None, :]
    dprod = np.mean(err ** 2 * d / norm)
    want = (math.pi / 2 - 1 / d) * d * O.lloyd_max(d, bits - 1)[1] if bits > 1 else (math.pi / 2 - 1 / d)
    assert abs(dprod - want) < 0.1 * want, (dprod, want)
    z = err / np.sqrt(norm)
    assert abs(z.mean()) < 4 * z.std() / math.sqrt(z.size)
