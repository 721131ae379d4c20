"""GPU parity of the decode step with append (tq_decode_append_attention): the
new token's key and value are quantized into the packed caches at each
sequence's length and the query attends one more token.

Bars, for every sequence (no sequence is skipped):
  * the new records are bit-exact with the oracle's nearest-centroid rule and
    QJL sign applied to the kernel's own rotated coordinates and projection
    (its debug outputs), and they differ from the oracle's fp64 quantization
    only where the fp64 coordinate lies within 1e-5 of a decision midpoint (QJL
    signs: within 1e-5 of the hyperplane); norms within 2 ulp, residual norms
    within 2e-5;
  * every other cache byte is unchanged;
  * the output equals the oracle's decode attention over the cache the GPU
    wrote, read back, within rtol 1e-3 / atol 1e-4.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import tq_synth as syn
from test_gpu_decode import _build
from tq_testlib import TIE_BAND, allclose_report, near_threshold, ulp_diff_f32

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [
    # B, Hq, Hkv, d, T, kbits, kvar, vbits, lens, kv dtype
    (5, 16, 2, 128, 256, 3, "prod", 3, [0, 37, 255, 256, 64], "bf16"),
    (3, 8, 1, 64, 96, 2, "mse", 2, [31, 32, 95], "f32"),
    (2, 16, 2, 256, 128, 4, "prod", 4, [127, 1], "bf16"),
    (2, 8, 2, 128, 64, 1, "prod", 2, [10, 63], "bf16"),
    (2, 64, 8, 128, 2048, 3, "prod", 3, [2047, 1500], "bf16"),
]


def _readback(kcache, vcache, kc, vc):
    """The caches as the GPU left them, in the oracle's dict form."""
    k = dict(kc)
    v = dict(vc)
    for n in ("codes", "signs", "norms", "rnorms"):
        t = getattr(kcache, n)
        if t is not None:
            k[n] = t.cpu().numpy()
    v["codes"] = vcache.codes.cpu().numpy()
    v["norms"] = vcache.norms.cpu().numpy()
    return k, v


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}d{c[3]}T{c[4]}K{c[6]}{c[5]}V{c[7]}{c[9]}")
def test_decode_append_parity(gpu_lib, case):
    tq = gpu_lib
    B, Hq, Hkv, d, T, kbits, kvar, vbits, lens, dt = case
    print(f"append case {case}", flush=True)
    lens = np.array(lens, np.int32)
    kcache, vcache, kc, vc = _build(tq, B, Hq, Hkv, d, T, kbits, kvar, vbits, syn.CFG_TEST)
    kp = kbits - (1 if kvar == "prod" else 0)
    # new tokens: one vector per (b, h) from a separate stream of the same generator
    knew = np.stack([syn.kv_vectors(Hkv, d, syn.CFG_TEST, syn.T_K, b, 50, lognormal_sigma=0.5) for b in range(B)])
    vnew = np.stack([syn.kv_vectors(Hkv, d, syn.CFG_TEST, syn.T_V, b, 50, lognormal_sigma=0.5) for b in range(B)])
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    q = syn.decode_queries(B, Hq, d, syn.CFG_TEST)
    scale = 1 / math.sqrt(d)
    before = {n: getattr(kcache, n).cpu().numpy().copy() for n in ("codes", "signs", "norms", "rnorms")
              if getattr(kcache, n) is not None}
    vbefore = {n: getattr(vcache, n).cpu().numpy().copy() for n in ("codes", "norms")}
    rot = torch.full((B, Hkv, 2, d), float("nan"), dtype=torch.float32, device=DEV)
    proj = torch.full((B, Hkv, d), float("nan"), dtype=torch.float32, device=DEV)
    out = tq.decode_append_attention(torch.from_numpy(q).to(DEV).to(torch.bfloat16),
                                     torch.from_numpy(knew).to(DEV).to(tdt), torch.from_numpy(vnew).to(DEV).to(tdt),
                                     kcache, vcache, torch.from_numpy(lens).to(DEV), scale,
                                     rot_dbg=rot, proj_dbg=proj if kvar == "prod" else None)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    rot = rot.cpu().numpy().astype(np.float64)
    proj = proj.cpu().numpy().astype(np.float64)
    # the inputs exactly as the kernel read them
    kin = knew.astype(np.float32) if dt == "f32" else syn.bf16_round(knew)
    vin = vnew.astype(np.float32) if dt == "f32" else syn.bf16_round(vnew)
    ck, cv = O.codebook(d, kp), O.codebook(d, vbits)
    for b in range(B):
        t = int(lens[b])
        for h in range(Hkv):
            if t >= T:
                assert np.all(np.isnan(rot[b, h])), "a full cache must not be appended"
                continue
            if kvar == "prod":
                rk = O.quantize_prod(kin[b, h][None].astype(np.float64), kc["Pi"][h], kc["S"][h], ck)
            else:
                rk = O.quantize_mse(kin[b, h][None].astype(np.float64), kc["Pi"][h], ck)
            rv = O.quantize_mse(vin[b, h][None].astype(np.float64), vc["Pi"][h], cv)
            # ---- key record ----
            assert ulp_diff_f32(np.float32(kcache.norms[b, h, t].item()), rk["norms"][0]) <= 2
            assert np.max(np.abs(rot[b, h, 0] - rk["y"][0])) <= 2e-5
            if kp > 0:
                gidx = O.unpack_vector_layout(kcache.codes[b, h, t][None].cpu().numpy(), kp, d)[0]
                assert np.array_equal(gidx, O.nearest_index(rot[b, h, 0], ck)), (b, h, "key codes vs own y")
                fl = gidx != rk["idx"][0]
                assert np.all(near_threshold(rk["y"][0][fl], ck, TIE_BAND)), (b, h, "key code flip outside band")
            if kvar == "prod":
                gz = O.unpack_bits(kcache.signs[b, h, t][None].cpu().numpy(), d)[0]
                assert np.array_equal(gz, proj[b, h] >= 0.0), (b, h, "signs vs own projection")
                fz = gz != rk["signs"][0]
                srow = np.linalg.norm(kc["S"][h], axis=1)
                assert np.all((np.abs(rk["p"][0]) / srow)[fz] <= TIE_BAND), (b, h, "sign flip outside band")
                assert np.all(np.abs(proj[b, h] - rk["p"][0]) <= 1e-5 * srow + 1e-6)
                if kp == 0 or not np.any(gidx != rk["idx"][0]):
                    assert abs(kcache.rnorms[b, h, t].item() - rk["gamma"][0]) <= 2e-5 * rk["gamma"][0] + 2e-7
            # ---- value record: slot t % 32 of block t // 32 ----
            assert ulp_diff_f32(np.float32(vcache.norms[b, h, t].item()), rv["norms"][0]) <= 2
            assert np.max(np.abs(rot[b, h, 1] - rv["y"][0])) <= 2e-5
            gblk = O.unpack_block_layout(vcache.codes[b, h, t // 32][None].cpu().numpy(), vbits, d)
            assert np.array_equal(gblk[t % 32], O.nearest_index(rot[b, h, 1], cv)), (b, h, "value codes vs own y")
            fv = gblk[t % 32] != rv["idx"][0]
            assert np.all(near_threshold(rv["y"][0][fv], cv, TIE_BAND)), (b, h, "value code flip outside band")
    # every other cache byte is unchanged
    for n, arr in before.items():
        now = getattr(kcache, n).cpu().numpy()
        mask = np.ones(now.shape[:3], bool)
        for b in range(B):
            if lens[b] < T:
                mask[b, :, lens[b]] = False
        assert np.array_equal(now[mask], arr[mask]), n
    for n, arr in vbefore.items():
        now = getattr(vcache, n).cpu().numpy()
        if n == "norms":
            mask = np.ones(now.shape, bool)
            for b in range(B):
                if lens[b] < T:
                    mask[b, :, lens[b]] = False
            assert np.array_equal(now[mask], arr[mask])
        else:
            for b in range(B):
                for h in range(Hkv):
                    t = int(lens[b])
                    nb = O.unpack_block_layout(now[b, h], vbits, d)
                    ob = O.unpack_block_layout(arr[b, h], vbits, d)
                    keep = np.ones(nb.shape[0], bool)
                    if t < T:
                        keep[t] = False
                    assert np.array_equal(nb[keep], ob[keep]), (b, h)
    # attention over the cache exactly as the GPU wrote it, for every sequence
    k_gpu, v_gpu = _readback(kcache, vcache, kc, vc)
    want = O.decode_attention(q, k_gpu, v_gpu, np.minimum(lens + 1, T), scale)
    for b in range(B):
        nbad, emax = allclose_report(got[b], want[b])
        assert nbad == 0, (b, int(lens[b]), nbad, emax)
