"""GPU parity of tq_search_scores, the vector-search scoring on the matrix
cores ([NIK] "Experiments": nearest-neighbour search over quantized
embeddings), against the fp64 oracle's <y, x~> with x~ its own dequantized
database, element by element within rel 1e-3 / abs 1e-4 on the scale
|y| |x~| / sqrt(d) (tq_testlib.assert_scores_close).

Cases span one and several coordinate slices (the fragments of one slice fit
the workgroup's LDS), every MSE-stage plane count 0..4, partial query groups
(m not a multiple of 8), ragged databases (n not a multiple of 32, n = 1), a
zero query, and a zero database vector."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
import tq_synth as syn
from test_gpu_vector_search import _oracle_database
from tq_testlib import assert_scores_close

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [
    # d, variant, bits, n, m
    (128, "mse", 3, 1000, 8),
    (256, "prod", 3, 777, 5),
    (768, "prod", 1, 1000, 11),
    (1536, "prod", 3, 3000, 16),
    (1536, "mse", 4, 1200, 3),   # 3 coordinate slices
    (3072, "prod", 3, 1200, 9),  # 2 slices
    (4096, "mse", 2, 500, 8),    # 2 slices
    (512, "prod", 4, 600, 8),
    (384, "mse", 1, 31, 1),
    (640, "prod", 2, 1, 7),
]


def _dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"d{c[0]}{c[1]}b{c[2]}n{c[3]}m{c[4]}")
def test_search_scores_parity(gpu_lib, case):
    tq = gpu_lib
    d, variant, bits, n, m = case
    print(f"search scores {case}", flush=True)
    Pi, S, x, xt, db = _oracle_database(d, variant, bits, n, 3)
    if n > 5:
        # a zero database vector: norm 0, every score 0
        x[5] = 0.0
        planes = bits - 1 if variant == "prod" else bits
        cb = O.codebook(d, planes)
        r = O.quantize_prod(x[5:6], Pi, S, cb) if variant == "prod" else O.quantize_mse(x[5:6], Pi, cb)
        db["norms"][5] = r["norms"][0]
        if planes:
            db["codes"][5] = O.pack_vector_layout(r["idx"], planes)[0]
        if variant == "prod":
            db["signs"][5] = O.pack_bits(r["signs"])[0]
            db["rnorms"][5] = r["rnorms"][0]
        xt[5] = 0.0
    q = tq.Quantizer(d, bits, variant, Pi, S)
    y = syn.gaussian_queries(m, d, syn.CFG_TEST, batch=7000 + d)
    if m > 2:
        y[2] = 0.0
    got = tq.search_scores(q, _dev(y), _dev(db["codes"]), _dev(db["norms"]), _dev(db.get("signs")),
                           _dev(db.get("rnorms"))).cpu().numpy()
    want = O.inner_products(y, xt)
    assert_scores_close(got, want, y, xt)
    if m > 2:
        assert np.all(got[2] == 0)
    if n > 5:
        assert np.all(got[:, 5] == 0)


def test_search_scores_repeat_and_workspace_reuse(gpu_lib):
    """Two calls in a row on one workspace, the second with fewer queries and a
    smaller database, each against the oracle; a too-small workspace is refused."""
    tq = gpu_lib
    d, bits = 1536, 3
    Pi, S, x, xt, db = _oracle_database(d, "prod", bits, 900, 4)
    q = tq.Quantizer(d, bits, "prod", Pi, S)
    ws = torch.empty(tq.search_workspace_size(q, 24), dtype=torch.uint8, device=DEV)
    for m, n in ((24, 900), (5, 333)):
        print(f"search reuse m={m} n={n}", flush=True)
        y = syn.gaussian_queries(m, d, syn.CFG_TEST, batch=8000 + m)
        got = tq.search_scores(q, _dev(y), _dev(db["codes"][:n]), _dev(db["norms"][:n]), _dev(db["signs"][:n]),
                               _dev(db["rnorms"][:n]), workspace=ws).cpu().numpy()
        want = O.inner_products(y, xt[:n])
        assert_scores_close(got, want, y, xt[:n])
    lib = tq.load()
    y = _dev(syn.gaussian_queries(24, d, syn.CFG_TEST, batch=8100))
    out = torch.empty((24, 900), dtype=torch.float32, device=DEV)
    cd, nd, sd, rd = (_dev(db[k]) for k in ("codes", "norms", "signs", "rnorms"))
    st = lib.tq_search_scores(q.handle, y.data_ptr(), 24, cd.data_ptr(), sd.data_ptr(), nd.data_ptr(),
                              rd.data_ptr(), 900, out.data_ptr(), ws.data_ptr(), ws.numel() - 1, None)
    assert st == tq.TQ_ERR_WORKSPACE
    st = lib.tq_search_scores(q.handle, y.data_ptr(), 24, cd.data_ptr(), None, nd.data_ptr(),
                              rd.data_ptr(), 900, out.data_ptr(), ws.data_ptr(), ws.numel(), None)
    assert st == tq.TQ_ERR_INVALID_ARG


def test_search_scores_unsupported_dims(gpu_lib):
    """d must be a multiple of 128: d = 64 and 320 quantizers are refused."""
    tq = gpu_lib
    lib = tq.load()
    for d in (64, 320):
        q = tq.Quantizer(d, 3, "mse", syn.rotation(d, syn.CFG_TEST, syn.T_K, 1))
        nb = ctypes.c_size_t(0)
        assert lib.tq_search_workspace_size(q.handle, 8, ctypes.byref(nb)) == tq.TQ_ERR_UNSUPPORTED


def test_misaligned_buffers_are_refused(gpu_lib):
    """The kernels load x and y in 16-byte vectors and code / sign words in 4
    bytes: misaligned buffers are refused with TQ_ERR_INVALID_ARG."""
    tq = gpu_lib
    d = 128
    q = tq.Quantizer(d, 3, "prod", syn.rotation(d, syn.CFG_TEST, syn.T_K, 5), syn.gaussian_matrix(d, syn.CFG_TEST, syn.T_K, 5))
    flat = torch.zeros(4 * d + 1, dtype=torch.bfloat16, device=DEV)
    x = flat[1:].view(4, d)  # 2-byte offset
    with pytest.raises(tq.TQError) as e:
        tq.quantize_prod(q, x)
    assert e.value.status == tq.TQ_ERR_INVALID_ARG
    yflat = torch.zeros(8 * d + 1, dtype=torch.float32, device=DEV)
    y = yflat[1:].view(8, d)
    r = tq.quantize_prod(q, torch.zeros((4, d), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(tq.TQError) as e:
        tq.search_scores(q, y, r["codes"], r["norms"], r["signs"], r["rnorms"])
    assert e.value.status == tq.TQ_ERR_INVALID_ARG
    torch.cuda.synchronize()
