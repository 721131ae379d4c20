"""GPU parity of the outlier-channel split (tq_quantize_split,
tq_inner_products_split; [NIK] "Experiments", KV cache: outlier channels at
more bits than the others) against the oracle's quantize_split.

The outlier channels are picked here as the 32 channels of largest RMS over the
vectors being quantized (the pages give no rule; the library takes the lists as
input). Per part: norms within 2 ulp, rotated coordinates within 2e-5 of fp64,
codes bit-exact on the kernel's own rotated coordinates and flips against fp64
only within the 1e-5 band, QJL signs bit-exact on the kernel's projection and
the projection within 5e-4 |r| of fp64. Split inner products from
oracle-packed records within 1e-4 of the largest |<y, x~>|; the prod split's
inner-product error on Gaussian rows against the per-part closed form within
10 %.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import tq_synth as syn
from tq_testlib import MAX_FLIP_RATE, TIE_BAND, near_threshold, ulp_diff_f32

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _outlier_first(x, k):
    rms = np.sqrt(np.mean(x.astype(np.float64) ** 2, axis=0))
    order = np.argsort(-rms, kind="stable")
    return order[:k], order[k:]


def _parts(tq, specs, seed0):
    """specs: list of (channels, variant, bits) -> (oracle parts, library quantizers)."""
    parts, qs = [], []
    for i, (ch, var, bits) in enumerate(specs):
        d = len(ch)
        Pi = syn.rotation(d, syn.CFG_TEST, syn.T_K, seed0 + i)
        S = syn.gaussian_matrix(d, syn.CFG_TEST, syn.T_K, seed0 + i) if var == "prod" else None
        planes = bits - 1 if var == "prod" else bits
        p = {"channels": np.asarray(ch), "variant": var, "Pi": Pi, "centroids": O.codebook(d, planes)}
        if S is not None:
            p["S"] = S
        parts.append(p)
        qs.append(tq.Quantizer(d, bits, var, Pi, S))
    return parts, qs


CASES = [
    # name, dim, n, dtype, [(n_channels or "rest", variant, bits)], dropped channels
    ("kv_mse_32x3_96x2", 128, 700, "bf16", [(32, "mse", 3), ("rest", "mse", 2)]),
    ("kv_prod_32x3_96x2", 128, 500, "f32", [(32, "prod", 3), ("rest", "prod", 2)]),
    ("mixed_drop", 128, 300, "f32", [(32, "mse", 4), (64, "prod", 1)]),
    ("d256_96_160", 256, 260, "bf16", [(96, "prod", 4), ("rest", "mse", 3)]),
]


def _build_case(tq, dim, n, dt, spec, seed):
    x = syn.kv_vectors(n, dim, syn.CFG_TEST, syn.T_K, 0, seed, lognormal_sigma=0.5)
    x[3] = 0.0
    first, rest = _outlier_first(x, spec[0][0])
    specs, used = [], 0
    order = np.concatenate([first, rest])
    for k, var, bits in spec:
        cnt = dim - used if k == "rest" else k
        specs.append((order[used:used + cnt], var, bits))
        used += cnt
    parts, qs = _parts(tq, specs, 40 + seed)
    xd = torch.from_numpy(x).to(DEV)
    if dt == "bf16":
        xd = xd.to(torch.bfloat16)
    return x, parts, qs, xd


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_split_quantize_parity(gpu_lib, case):
    tq = gpu_lib
    name, dim, n, dt, spec = case
    print(f"split quantize {name}", flush=True)
    x, parts, qs, xd = _build_case(tq, dim, n, dt, spec, 1)
    got = tq.quantize_split(qs, [p["channels"] for p in parts], xd, rot_dbg=True, proj_dbg=True)
    torch.cuda.synchronize()
    ref = O.quantize_split(x, parts)
    for p, q, g, r in zip(parts, qs, got, ref):
        d = len(p["channels"])
        valid = r["nu"] > 0
        assert ulp_diff_f32(g["norms"].cpu().numpy(), r["nu"].astype(np.float32)).max() <= 2
        rot = g["rot"].cpu().numpy()
        assert np.abs(rot[valid] - r["y"][valid]).max() < 2e-5
        cb = p["centroids"]
        if q.planes > 0:
            codes = g["codes"].cpu().numpy()
            fed = O.nearest_index(rot.astype(np.float64), cb)
            fed[~valid] = 0
            assert np.array_equal(codes, O.pack_vector_layout(fed, q.planes))
            idx = O.unpack_vector_layout(codes, q.planes, d)
            flips = idx[valid] != r["idx"][valid]
            assert flips.mean() < MAX_FLIP_RATE
            if flips.any():
                assert np.all(near_threshold(r["y"][valid][flips], cb, TIE_BAND))
        if p["variant"] == "prod":
            proj = g["proj"].cpu().numpy()
            fz = proj >= 0
            fz[~valid] = False
            assert np.array_equal(g["signs"].cpu().numpy(), O.pack_bits(fz))
            same = valid.copy()
            if q.planes > 0:
                same &= np.all(O.unpack_vector_layout(g["codes"].cpu().numpy(), q.planes, d) == r["idx"], axis=1)
            assert same.sum() > 0.9 * valid.sum()
            rn = g["rnorms"].cpu().numpy()
            assert rn[3] == 0
            assert np.allclose(rn[same], r["gamma"][same], rtol=2e-5, atol=2e-7)
            perr = np.abs(proj[same] - r["p"][same]).max(axis=1)
            assert np.all(perr <= 5e-4 * r["gamma"][same])


def _pack(parts, qs, ref):
    recs = []
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    for p, q, r in zip(parts, qs, ref):
        rec = {"norms": dev(r["norms"])}
        if q.planes > 0:
            rec["codes"] = dev(O.pack_vector_layout(r["idx"], q.planes))
        if p["variant"] == "prod":
            rec["signs"] = dev(O.pack_bits(r["signs"]))
            rec["rnorms"] = dev(r["rnorms"])
        recs.append(rec)
    return recs


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_split_inner_products_parity(gpu_lib, case):
    tq = gpu_lib
    name, dim, n, dt, spec = case
    print(f"split inner products {name}", flush=True)
    x, parts, qs, _ = _build_case(tq, dim, n, dt, spec, 2)
    if dt == "bf16":
        x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    ref = O.quantize_split(x, parts)
    y = syn.gaussian_queries(5, dim, syn.CFG_TEST, batch=300 + dim)
    got = tq.inner_products_split(qs, [p["channels"] for p in parts], torch.from_numpy(y).to(DEV),
                                  _pack(parts, qs, ref)).cpu().numpy()
    want = O.inner_products(y, O.dequantize_split(ref, parts, dim))
    err = np.abs(got - want).max()
    assert err <= 1e-4 * np.abs(want).max(), (err, np.abs(want).max())


def test_split_prod_inner_product_error_closed_form(gpu_lib):
    """The pages' split shape for keys (32 channels at 3 bits, 96 at 2, prod):
    GPU-quantized records, GPU inner products; mean squared error against
    sum_p (pi/2 - 1/d_p) d_p C(f_{d_p}, b_p - 1) |y_p|^2 |x_p|^2 / d_p.
    Gaussian rows: x_p/|x_p| is uniform on the sphere for any fixed Pi, so the
    closed form holds for one rotation draw (outlier-dominated rows need the
    average over draws)."""
    tq = gpu_lib
    dim, n, m = 128, 4000, 64  # one S per part: the closed form needs many query directions
    x = syn.gaussian_queries(n, dim, syn.CFG_TEST, batch=4321)
    ch = np.random.default_rng(12).permutation(dim)
    parts, qs = _parts(tq, [(ch[:32], "prod", 3), (ch[32:], "prod", 2)], 60)
    xd = torch.from_numpy(x).to(DEV)
    chans = [p["channels"] for p in parts]
    recs = tq.quantize_split(qs, chans, xd)
    y = syn.gaussian_queries(m, dim, syn.CFG_TEST, batch=77)
    got = tq.inner_products_split(qs, chans, torch.from_numpy(y).to(DEV), recs).cpu().numpy().astype(np.float64)
    err = got - y.astype(np.float64) @ x.astype(np.float64).T
    want = np.zeros_like(err)
    for p, b in zip(parts, (3, 2)):
        c = p["channels"]
        dp = len(c)
        cost = O.lloyd_max(dp, b - 1)[1]
        want += (math.pi / 2 - 1 / dp) * cost * np.sum(y[:, c].astype(np.float64) ** 2, axis=1)[:, None] * \
            np.sum(x[:, c].astype(np.float64) ** 2, axis=1)[None, :]
    ratio = np.mean(err ** 2) / np.mean(want)
    assert abs(ratio - 1) < 0.1, ratio
    assert abs(err.mean()) < 4 * err.std() / math.sqrt(err.size)


def test_split_rejects_bad_channel_lists(gpu_lib):
    import ctypes
    tq = gpu_lib
    lib = tq.load()
    qa = tq.Quantizer(32, 3, "mse", syn.rotation(32, syn.CFG_TEST, syn.T_K, 90))
    qb = tq.Quantizer(32, 2, "mse", syn.rotation(32, syn.CFG_TEST, syn.T_K, 91))
    hs = tq._handles([qa, qb])
    x = torch.zeros((4, 64), dtype=torch.float32, device=DEV)
    recs = [{"norms": torch.empty(4, device=DEV), "codes": torch.empty((4, q.code_bytes), dtype=torch.uint8, device=DEV)}
            for q in (qa, qb)]
    ok = np.arange(64, dtype=np.int32)
    assert lib.tq_quantize_split(hs, 2, ok.ctypes.data, 64, x.data_ptr(), tq.TQ_F32, 4, tq._records(recs), None) == tq.TQ_OK
    rep = ok.copy()
    rep[40] = 5
    assert lib.tq_quantize_split(hs, 2, rep.ctypes.data, 64, x.data_ptr(), tq.TQ_F32, 4, tq._records(recs), None) == \
        tq.TQ_ERR_INVALID_ARG
    assert b"twice" in lib.tq_last_error_message()
    far = ok.copy()
    far[0] = 64
    assert lib.tq_quantize_split(hs, 2, far.ctypes.data, 64, x.data_ptr(), tq.TQ_F32, 4, tq._records(recs), None) == \
        tq.TQ_ERR_INVALID_ARG
    assert lib.tq_quantize_split(hs, 2, ok.ctypes.data, 48, x.data_ptr(), tq.TQ_F32, 4, tq._records(recs), None) == \
        tq.TQ_ERR_INVALID_ARG
    assert lib.tq_quantize_split(hs, 2, ok.ctypes.data, 600, x.data_ptr(), tq.TQ_F32, 4, tq._records(recs), None) == \
        tq.TQ_ERR_UNSUPPORTED
    torch.cuda.synchronize()
