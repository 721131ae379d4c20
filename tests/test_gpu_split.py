"""GPU parity of the outlier-channel split (tq_quantize_split,
tq_inner_products_split; [NIK] "Experiments", KV cache: outlier channels at
more bits than the others) against the oracle's quantize_split.

The outlier channels are picked here as the 32 channels of largest RMS over the
vectors being quantized (the pages give no rule; the library takes the lists as
input). Per part: norms within 2 ulp, rotated coordinates within 2e-5 of fp64,
codes bit-exact on the kernel's own rotated coordinates and flips against fp64
only within the 1e-5 band, QJL signs bit-exact on the kernel's projection and
the projection within 5e-4 |r| of fp64. Split inner products from
oracle-packed records element by element within rel 1e-3 / abs 1e-4 on the
scale |y| |x~| / sqrt(dim); the prod split's
inner-product error on Gaussian rows against the per-part closed form within
10 %.
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
    # name, dim, n, dtype, [(n_channels or "rest", variant, bits)]; channels not
    # listed are dropped. d = 128 rows with parts of a multiple of 32 channels run
    # on the matrix-core kernel, the others on the generic fp32 kernels.
    ("kv_mse_32x3_96x2", 128, 700, "bf16", [(32, "mse", 3), ("rest", "mse", 2)]),
    ("kv_prod_32x3_96x2", 128, 500, "f32", [(32, "prod", 3), ("rest", "prod", 2)]),
    ("kv_prod_bf16_32x4_96x3", 128, 333, "bf16", [(32, "prod", 4), ("rest", "prod", 3)]),
    # the fused two-part kernel with the wider part first, and with a 1-bit prod
    # part (no code planes) beside a 2-bit one
    ("fused_mse_96x1_32x4", 128, 300, "f32", [(96, "mse", 1), ("rest", "mse", 4)]),
    ("fused_prod_64x2_64x1", 128, 257, "bf16", [(64, "prod", 2), ("rest", "prod", 1)]),
    ("mixed_drop", 128, 300, "f32", [(32, "mse", 4), (64, "prod", 1)]),
    ("mixed_drop_bf16", 128, 290, "bf16", [(64, "mse", 1), (32, "prod", 2)]),
    ("generic_dim192", 192, 200, "bf16", [(64, "mse", 3), ("rest", "prod", 2)]),
    ("d256_96_160", 256, 260, "bf16", [(96, "prod", 4), ("rest", "mse", 3)]),
]


def _split_specs(x, spec):
    first, rest = _outlier_first(x, spec[0][0])
    specs, used = [], 0
    order = np.concatenate([first, rest])
    for k, var, bits in spec:
        cnt = x.shape[1] - used if k == "rest" else k
        specs.append((order[used:used + cnt], var, bits))
        used += cnt
    return specs, order[used:]


def _build_case(tq, dim, n, dt, spec, seed):
    x = syn.kv_vectors(n, dim, syn.CFG_TEST, syn.T_K, 0, seed, lognormal_sigma=0.5)
    x[3] = 0.0
    specs, dropped = _split_specs(x, spec)
    if len(dropped):
        # a dropped channel is never read: not even a NaN there reaches the records
        x[5, dropped[0]] = np.nan
        x[6, dropped[-1]] = np.inf
    parts, qs = _parts(tq, specs, 40 + seed)
    xd = torch.from_numpy(x).to(DEV)
    if dt == "bf16":
        xd = xd.to(torch.bfloat16)
        x = xd.float().cpu().numpy()
    return x, parts, qs, xd


def _check_part(p, q, g, r):
    """One part's device records g against the oracle's r (tolerances in the module docstring)."""
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
        assert np.all(rn[~valid] == 0)
        assert np.allclose(rn[same], r["gamma"][same], rtol=2e-5, atol=2e-7)
        perr = np.abs(proj[same] - r["p"][same]).max(axis=1)
        assert np.all(perr <= 5e-4 * r["gamma"][same])


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_split_quantize_parity(gpu_lib, case):
    tq = gpu_lib
    name, dim, n, dt, spec = case
    print(f"split quantize {name}", flush=True)
    x, parts, qs, xd = _build_case(tq, dim, n, dt, spec, 1)
    got = tq.quantize_split(qs, [p["channels"] for p in parts], xd, rot_dbg=True, proj_dbg=True)
    torch.cuda.synchronize()
    ref = O.quantize_split(x, parts)
    assert ref[0]["nu"][3] == 0
    for p, q, g, r in zip(parts, qs, got, ref):
        _check_part(p, q, g, r)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_split_quantize_grouped_parity(gpu_lib, dt):
    """Grouped split (one call over G groups, e.g. the KV heads of a layer): every
    group has its own outlier channels and quantizers; 32 + 96 channels (the
    matrix-core kernel) for keys (prod) and values (mse), and a ragged n."""
    tq = gpu_lib
    G, n, dim = 3, 333, 128
    print(f"split quantize grouped {dt}", flush=True)
    for var, bits in (("prod", (3, 2)), ("mse", (3, 2)), ("mse", (4, 1))):
        xs, parts_g, qs_g = [], [], []
        for g in range(G):
            x = syn.kv_vectors(n, dim, syn.CFG_TEST, syn.T_V, g, 7, lognormal_sigma=0.5)
            x[g] = 0.0
            specs, _ = _split_specs(x, [(32, var, bits[0]), ("rest", var, bits[1])])
            parts, qs = _parts(tq, specs, 70 + 5 * g)
            xs.append(x)
            parts_g.append(parts)
            qs_g.append(qs)
        xd = torch.from_numpy(np.stack(xs)).to(DEV)
        if dt == "bf16":
            xd = xd.to(torch.bfloat16)
        xr = xd.float().cpu().numpy()
        got = tq.quantize_split([[qs_g[g][p] for g in range(G)] for p in range(2)],
                                [[parts_g[g][p]["channels"] for g in range(G)] for p in range(2)], xd,
                                rot_dbg=True, proj_dbg=True)
        torch.cuda.synchronize()
        for g in range(G):
            ref = O.quantize_split(xr[g], parts_g[g])
            assert ref[0]["nu"][g] == 0
            for p in range(2):
                _check_part(parts_g[g][p], qs_g[g][p], {k: v[g] for k, v in got[p].items()}, ref[p])


@pytest.mark.parametrize("dim,spec", [(128, [(32, 3), ("rest", 2)]), (128, [(64, 1), ("rest", 4)]),
                                      (128, [(32, 4), (32, 2)]), (192, [(64, 4), ("rest", 1)])],
                         ids=["fused_32x3_96x2", "fused_64x1_64x4", "per_part_32x4_32x2", "generic_64x4_128x1"])
def test_split_quantize_block32(gpu_lib, dim, spec):
    """layout="block32" (the value layout of a split cache): every part's codes
    equal the oracle's BLOCK32 packing of the indices the kernel's own rotated
    coordinates give, over two groups of 96 rows; norms as in the VECTOR layout."""
    tq = gpu_lib
    G, n = 2, 96
    print(f"split quantize block32 dim={dim}", flush=True)
    xs, parts_g, qs_g = [], [], []
    for g in range(G):
        x = syn.kv_vectors(n, dim, syn.CFG_TEST, syn.T_V, g, 9, lognormal_sigma=0.5)
        x[5 + g] = 0.0
        specs, _ = _split_specs(x, [(k, "mse", b) for k, b in spec])
        parts, qs = _parts(tq, specs, 80 + 5 * g)
        xs.append(x)
        parts_g.append(parts)
        qs_g.append(qs)
    xd = torch.from_numpy(np.stack(xs)).to(DEV).to(torch.bfloat16)
    xr = xd.float().cpu().numpy()
    args = ([[qs_g[g][p] for g in range(G)] for p in range(2)], [[parts_g[g][p]["channels"] for g in range(G)]
                                                                   for p in range(2)], xd)
    vec = tq.quantize_split(*args, rot_dbg=True)
    blk = tq.quantize_split(*args, rot_dbg=True, layout="block32")
    torch.cuda.synchronize()
    for g in range(G):
        ref = O.quantize_split(xr[g], parts_g[g])
        for p in range(2):
            q = qs_g[g][p]
            assert torch.equal(blk[p]["norms"][g], vec[p]["norms"][g])
            # the matrix-core kernel forms x Pi^T for blocks and Pi x for vectors
            assert torch.allclose(blk[p]["rot"][g], vec[p]["rot"][g], rtol=0, atol=2e-6)
            rot = blk[p]["rot"][g].cpu().numpy().astype(np.float64)
            fed = O.nearest_index(rot, parts_g[g][p]["centroids"])
            fed[~(ref[p]["nu"] > 0)] = 0
            want = O.pack_block_layout(fed, q.planes).reshape(n, -1)
            assert np.array_equal(blk[p]["codes"][g].cpu().numpy(), want), (g, p)
    with pytest.raises(RuntimeError):
        tq.quantize_split(args[0], args[1], xd[:, :80], layout="block32")  # 80 rows: not whole blocks


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
    xt = O.dequantize_split(ref, parts, dim)
    assert_scores_close(got, O.inner_products(y, xt), y, xt)


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
    call = lambda h, ng, ch, dim, n=4, lay=tq.TQ_LAYOUT_VECTOR: lib.tq_quantize_split(
        h, 2, ng, ch.ctypes.data, dim, x.data_ptr(), tq.TQ_F32, n, lay, tq._records(recs), None)
    assert call(hs, 1, ok, 64) == tq.TQ_OK
    rep = ok.copy()
    rep[40] = 5
    assert call(hs, 1, rep, 64) == tq.TQ_ERR_INVALID_ARG
    assert b"twice" in lib.tq_last_error_message()
    far = ok.copy()
    far[0] = 64
    assert call(hs, 1, far, 64) == tq.TQ_ERR_INVALID_ARG
    assert call(hs, 1, ok, 48) == tq.TQ_ERR_INVALID_ARG
    assert call(hs, 1, ok, 600) == tq.TQ_ERR_UNSUPPORTED
    assert call(hs, 0, ok, 64) == tq.TQ_ERR_INVALID_ARG
    assert call(hs, 1, ok, 64, lay=7) == tq.TQ_ERR_INVALID_ARG
    assert call(hs, 1, ok, 64, lay=tq.TQ_LAYOUT_BLOCK32) == tq.TQ_ERR_INVALID_ARG  # 4 rows: not whole blocks
    qp = tq.Quantizer(32, 2, "prod", syn.rotation(32, syn.CFG_TEST, syn.T_K, 93),
                      syn.gaussian_matrix(32, syn.CFG_TEST, syn.T_K, 93))
    assert call(tq._handles([qp, qb]), 1, ok, 64, 32, tq.TQ_LAYOUT_BLOCK32) == tq.TQ_ERR_UNSUPPORTED
    assert b"mse parts" in lib.tq_last_error_message()
    # two groups of two rows: part 0's handles must agree across the groups
    qc = tq.Quantizer(32, 4, "mse", syn.rotation(32, syn.CFG_TEST, syn.T_K, 92))
    two = np.concatenate([ok[:32], ok[:32], ok[32:], ok[32:]]).astype(np.int32)
    assert call(tq._handles([qa, qa, qb, qb]), 2, two, 64, 2) == tq.TQ_OK
    assert call(tq._handles([qa, qc, qb, qb]), 2, two, 64, 2) == tq.TQ_ERR_INVALID_ARG
    assert b"differ across groups" in lib.tq_last_error_message()
    # group 1 repeats a channel of its own
    bad = two.copy()
    bad[64 + 32] = bad[32]
    assert call(tq._handles([qa, qa, qb, qb]), 2, bad, 64, 2) == tq.TQ_ERR_INVALID_ARG
    assert b"group 1" in lib.tq_last_error_message()
    torch.cuda.synchronize()
