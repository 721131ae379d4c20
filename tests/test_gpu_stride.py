"""Strided inputs (tq_quantize_mse / tq_quantize_prod with x_stride): one head's
slice of a [n][heads*d] projection is quantized in place, on each kernel family
(d = 64 / 128 matrix-core kernel, d = 1536 GEMM kernel, d = 320 generic fp32
kernel), against the fp64 oracle on the same slice: norms within 2 ulp, codes
bit-exact on the kernel's own rotated coordinates (flips against fp64 only
within the 1e-5 band), QJL signs bit-exact on the kernel's projection. Also the
record sizes reported by tq_quantizer_sizes and the refusal of a stride that
is not a multiple of 16 bytes."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
import tq_synth as syn
from tq_testlib import MAX_FLIP_RATE, TIE_BAND, near_threshold, ulp_diff_f32

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [
    # d, heads, head taken, variant, bits, dtype
    (128, 8, 3, "mse", 3, "bf16"),
    (128, 4, 1, "prod", 3, "f32"),
    (64, 6, 5, "mse", 2, "bf16"),
    (1536, 2, 1, "prod", 3, "f32"),
    (320, 3, 2, "mse", 2, "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"d{c[0]}h{c[2]}of{c[1]}{c[3]}b{c[4]}{c[5]}")
def test_strided_quantize_parity(gpu_lib, case):
    tq = gpu_lib
    d, H, h, variant, bits, dt = case
    n = 333
    print(f"strided quantize {case}", flush=True)
    big = syn.kv_vectors(n, H * d, syn.CFG_TEST, syn.T_K, 0, 70 + d, lognormal_sigma=0.5)
    big[4] = 0.0
    bd = torch.from_numpy(big).to(DEV)
    if dt == "bf16":
        bd = bd.to(torch.bfloat16)
    xs = bd[:, h * d:(h + 1) * d]  # row stride H * d
    assert xs.stride(0) == H * d and not xs.is_contiguous()
    x = xs.float().cpu().numpy().astype(np.float64)
    Pi = syn.rotation(d, syn.CFG_TEST, syn.T_K, 80 + d)
    S = syn.gaussian_matrix(d, syn.CFG_TEST, syn.T_K, 80 + d) if variant == "prod" else None
    q = tq.Quantizer(d, bits, variant, Pi, S)
    r = tq.quantize_prod(q, xs, rot_dbg=True, proj_dbg=True) if variant == "prod" else tq.quantize_mse(q, xs, rot_dbg=True)
    torch.cuda.synchronize()
    cb = O.codebook(d, q.planes)
    ref = O.quantize_prod(x, Pi, S, cb) if variant == "prod" else O.quantize_mse(x, Pi, cb)
    valid = ref["nu"] > 0
    assert ulp_diff_f32(r["norms"].cpu().numpy(), ref["nu"].astype(np.float32)).max() <= 2
    rot = r["rot"].cpu().numpy()
    assert np.abs(rot[valid] - ref["y"][valid]).max() < 2e-5
    codes = r["codes"].cpu().numpy()
    fed = O.nearest_index(rot.astype(np.float64), cb)
    fed[~valid] = 0
    assert np.array_equal(codes, O.pack_vector_layout(fed, q.planes))
    idx = O.unpack_vector_layout(codes, q.planes, d)
    flips = idx[valid] != ref["idx"][valid]
    assert flips.mean() < MAX_FLIP_RATE
    if flips.any():
        assert np.all(near_threshold(ref["y"][valid][flips], cb, TIE_BAND))
    if variant == "prod":
        proj = r["proj"].cpu().numpy()
        fz = proj >= 0
        fz[~valid] = False
        assert np.array_equal(r["signs"].cpu().numpy(), O.pack_bits(fz))


def test_stride_checks_and_record_sizes(gpu_lib):
    tq = gpu_lib
    lib = tq.load()
    d = 128
    q = tq.Quantizer(d, 3, "prod", syn.rotation(d, syn.CFG_TEST, syn.T_K, 1), syn.gaussian_matrix(d, syn.CFG_TEST, syn.T_K, 1))
    cbytes, sbytes = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert lib.tq_quantizer_sizes(q.handle, ctypes.byref(cbytes), ctypes.byref(sbytes)) == tq.TQ_OK
    assert (cbytes.value, sbytes.value) == (2 * d // 8, d // 8)
    qm = tq.Quantizer(d, 4, "mse", syn.rotation(d, syn.CFG_TEST, syn.T_K, 2))
    assert lib.tq_quantizer_sizes(qm.handle, ctypes.byref(cbytes), ctypes.byref(sbytes)) == tq.TQ_OK
    assert (cbytes.value, sbytes.value) == (4 * d // 8, 0)
    x = torch.zeros((4, 136), dtype=torch.bfloat16, device=DEV)  # row stride 272 bytes
    out = {k: torch.empty(s, dtype=t, device=DEV) for k, s, t in
           (("codes", (4, 32), torch.uint8), ("signs", (4, 16), torch.uint8), ("norms", 4, torch.float32),
            ("rnorms", 4, torch.float32))}
    st = lib.tq_quantize_prod(q.handle, x.data_ptr(), tq.TQ_BF16, 4, 130, out["codes"].data_ptr(),
                              out["signs"].data_ptr(), out["norms"].data_ptr(), out["rnorms"].data_ptr(), None, None, None)
    assert st == tq.TQ_ERR_INVALID_ARG  # 260 bytes per row
    st = lib.tq_quantize_prod(q.handle, x.data_ptr(), tq.TQ_BF16, 4, 100, out["codes"].data_ptr(),
                              out["signs"].data_ptr(), out["norms"].data_ptr(), out["rnorms"].data_ptr(), None, None, None)
    assert st == tq.TQ_ERR_INVALID_ARG  # stride below d
    st = lib.tq_quantize_prod(q.handle, x.data_ptr(), tq.TQ_BF16, 4, 136, out["codes"].data_ptr(),
                              out["signs"].data_ptr(), out["norms"].data_ptr(), out["rnorms"].data_ptr(), None, None, None)
    assert st == tq.TQ_OK
    torch.cuda.synchronize()
