"""GPU parity of tq_quantize_kv, a layer's keys (VECTOR layout) and values
(BLOCK32 layout) in one call, against the fp64 oracle and against the two
tq_quantize calls it stands for.

Bars: records identical (bit for bit) to those of tq_quantize on the same
inputs, which the quantize parity tests hold to the oracle's nearest-centroid
rule on the kernel's own rotated coordinates; against the full fp64 path,
fewer than 1e-4 of codes flip and only within +-1e-5 of a threshold, norms
within 2 ulp.
"""
import numpy as np
import pytest
import torch

import oracle as O
import tq_synth as syn
from tq_testlib import MAX_FLIP_RATE, TIE_BAND, near_threshold, ulp_diff_f32

pytestmark = pytest.mark.gpu
DEV = "cuda"

# (d, bits, key variant, dtype, groups, vectors per group): the one-launch form
# for mse keys (d = 64 / 128 / 256, 2 to 4 planes, bf16 and fp32), two launches
# for prod keys
CASES = [
    (128, 3, "mse", "bf16", 8, 4096),
    (128, 2, "mse", "bf16", 3, 1024),
    (64, 4, "mse", "f32", 3, 1056),
    (256, 3, "mse", "bf16", 2, 2048),
    (256, 4, "mse", "f32", 2, 544),
    (128, 3, "prod", "bf16", 4, 1024),
]


def _quantizers(tq, d, bits, variant, tensor, G):
    qs, mats = [], []
    for h in range(G):
        Pi = syn.rotation(d, syn.CFG_TEST, tensor, 300 + h)
        S = syn.gaussian_matrix(d, syn.CFG_TEST, tensor, 300 + h) if variant == "prod" else None
        qs.append(tq.Quantizer(d, bits, variant, Pi, S))
        mats.append((Pi, S))
    return qs, mats


def _vectors(G, n, d, tensor, dtype):
    x = np.stack([syn.kv_vectors(n, d, syn.CFG_TEST, tensor, 0, 300 + h, lognormal_sigma=0.5) for h in range(G)])
    if n > 5:
        x[0, 5] = 0.0  # a zero vector
    t = torch.from_numpy(x).to(DEV)
    return (t.to(torch.bfloat16) if dtype == "bf16" else t), x


@pytest.mark.parametrize("d,bits,kvar,dtype,G,n", CASES)
def test_quantize_kv_parity(gpu_lib, d, bits, kvar, dtype, G, n):
    tq = gpu_lib
    print(f"case quantize_kv d={d} b={bits} keys={kvar} {dtype} G={G} n={n}", flush=True)
    kqs, kmats = _quantizers(tq, d, bits, kvar, syn.T_K, G)
    vqs, vmats = _quantizers(tq, d, bits, "mse", syn.T_V, G)
    xk, xk_np = _vectors(G, n, d, syn.T_K, dtype)
    xv, xv_np = _vectors(G, n, d, syn.T_V, dtype)
    # poison the outputs so that any record the call leaves unwritten shows
    kout = {"norms": torch.full((G, n), float("nan"), device=DEV)}
    if kqs[0].planes > 0:
        kout["codes"] = torch.full((G, n * kqs[0].code_bytes), 0xA5, dtype=torch.uint8, device=DEV)
    if kvar == "prod":
        kout["signs"] = torch.full((G, n, d // 8), 0xA5, dtype=torch.uint8, device=DEV)
        kout["rnorms"] = torch.full((G, n), float("nan"), device=DEV)
    vout = {"codes": torch.full((G, n * vqs[0].code_bytes), 0xA5, dtype=torch.uint8, device=DEV),
            "norms": torch.full((G, n), float("nan"), device=DEV)}
    tq.quantize_kv(kqs, vqs, xk, xv, kout=kout, vout=vout)
    kref = tq.quantize(kqs, xk, layout="vector")
    vref = tq.quantize(vqs, xv, layout="block32")
    torch.cuda.synchronize()
    for name in kout:
        assert torch.equal(kout[name], kref[name]), ("keys", name)
    for name in vout:
        assert torch.equal(vout[name], vref[name]), ("values", name)
    # sampled vectors of every group against the fp64 oracle
    g = np.random.default_rng(7)
    for tensor, recs, mats, x_np, variant, layout in ((syn.T_K, kout, kmats, xk_np, kvar, "vector"),
                                                     (syn.T_V, vout, vmats, xv_np, "mse", "block32")):
        planes = bits - 1 if variant == "prod" else bits
        cb = O.codebook(d, planes)
        codes = recs["codes"].cpu().numpy() if planes > 0 else None
        norms = recs["norms"].cpu().numpy()
        n_flip = n_coord = 0
        for h in range(G):
            toks = np.unique(np.concatenate([g.integers(0, n, 64), [0, 5, 31, 32, n - 1]]))
            xs = x_np[h, toks].astype(np.float32)
            if dtype == "bf16":
                xs = torch.from_numpy(xs).to(torch.bfloat16).float().numpy()
            Pi, S = mats[h]
            ref = O.quantize_prod(xs, Pi, S, cb) if variant == "prod" else O.quantize_mse(xs, Pi, cb)
            assert ulp_diff_f32(norms[h, toks], ref["nu"].astype(np.float32)).max() <= 2, (tensor, h)
            if planes == 0:
                continue
            if layout == "vector":
                idx = O.unpack_vector_layout(codes[h].reshape(n, -1)[toks], planes, d)
            else:
                blocks = codes[h].reshape(n // 32, 4 * planes * d)
                idx = np.stack([O.unpack_block_layout(blocks[t // 32][None], planes, d)[t % 32] for t in toks])
            valid = ref["nu"] > 0
            flips = (idx != ref["idx"]) & valid[:, None]
            if flips.any():
                assert np.all(near_threshold(ref["y"][flips], cb, TIE_BAND)), (tensor, h)
            n_flip += int(flips.sum())
            n_coord += flips.size
        if n_coord:
            assert n_flip / n_coord < MAX_FLIP_RATE, (tensor, n_flip, n_coord)


def _kv_pair(tq, G, n, d, kbits, vbits, dtype="bf16"):
    kqs, _ = _quantizers(tq, d, kbits, "mse", syn.T_K, G)
    vqs, _ = _quantizers(tq, d, vbits, "mse", syn.T_V, G)
    xk, _ = _vectors(G, n, d, syn.T_K, dtype)
    xv, _ = _vectors(G, n, d, syn.T_V, dtype)
    return kqs, vqs, xk, xv


@pytest.mark.parametrize("case", ["bits_differ", "many_groups"])
def test_quantize_kv_two_launch_forms(gpu_lib, case):
    # keys and values of different bit widths, and more groups than one launch
    # takes (65), go through two tq_quantize launches: records as those calls write them
    tq = gpu_lib
    G, n, kb, vb = (3, 256, 3, 2) if case == "bits_differ" else (65, 64, 3, 3)
    print(f"case quantize_kv {case} G={G} n={n} kbits={kb} vbits={vb}", flush=True)
    kqs, vqs, xk, xv = _kv_pair(tq, G, n, 128, kb, vb)
    ko, vo = tq.quantize_kv(kqs, vqs, xk, xv)
    kr = tq.quantize(kqs, xk, layout="vector")
    vr = tq.quantize(vqs, xv, layout="block32")
    torch.cuda.synchronize()
    for name in ko:
        assert torch.equal(ko[name], kr[name]), ("keys", name)
    for name in vo:
        assert torch.equal(vo[name], vr[name]), ("values", name)


def test_quantize_kv_empty_and_errors(gpu_lib):
    tq = gpu_lib
    kqs, vqs, xk, xv = _kv_pair(tq, 2, 0, 128, 3, 3)
    ko, vo = tq.quantize_kv(kqs, vqs, xk, xv)  # no vectors: nothing to do, no error
    torch.cuda.synchronize()
    assert ko["norms"].numel() == 0 and vo["norms"].numel() == 0
    kqs, vqs, xk, xv = _kv_pair(tq, 2, 64, 128, 3, 3)
    pq = [tq.Quantizer(128, 3, "prod", syn.rotation(128, syn.CFG_TEST, syn.T_V, 9),
                       syn.gaussian_matrix(128, syn.CFG_TEST, syn.T_V, 9)) for _ in range(2)]
    with pytest.raises(tq.TQError):
        tq.quantize_kv(kqs, pq, xk, xv)  # values must be mse (block layout)
    with pytest.raises(tq.TQError):
        tq.quantize_kv(kqs, vqs, xk[:, :48].contiguous(), xv[:, :48].contiguous())  # n % 32 != 0
