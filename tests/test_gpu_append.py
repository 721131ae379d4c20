"""GPU parity of the decode step with append (tq_decode_append_attention):
the new token's key and value are quantized into the packed caches at each
sequence's length and the query attends one more token. The oracle quantizes
the same new vectors in fp64, writes them into its copy of the caches with its
own packers, and runs its decode over length + 1 tokens.

Bars: every cache byte other than the new token's records is unchanged; the new
codes equal the oracle's except where the fp64 rotated coordinate lies within
1e-5 of a decision midpoint (QJL signs: within 1e-5 of the hyperplane); norms
within 2 ulp, residual norms within 2e-5; outputs within rtol 1e-3 / atol 1e-4.
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
]


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
    out = tq.decode_append_attention(torch.from_numpy(q).to(DEV).to(torch.bfloat16),
                                     torch.from_numpy(knew).to(DEV).to(tdt), torch.from_numpy(vnew).to(DEV).to(tdt),
                                     kcache, vcache, torch.from_numpy(lens).to(DEV), scale)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    # oracle: quantize the new vectors and write them with its own packers
    ck, cv = O.codebook(d, kp), O.codebook(d, vbits)
    clean = np.ones(B, bool)
    for b in range(B):
        t = int(lens[b])
        for h in range(Hkv):
            if t >= T:
                continue
            if kvar == "prod":
                rk = O.quantize_prod(knew[b, h][None].astype(np.float64), kc["Pi"][h], kc["S"][h], ck)
            else:
                rk = O.quantize_mse(knew[b, h][None].astype(np.float64), kc["Pi"][h], ck)
            rv = O.quantize_mse(vnew[b, h][None].astype(np.float64), vc["Pi"][h], cv)
            # keys
            gk = kcache.norms[b, h, t].item()
            assert ulp_diff_f32(np.float32(gk), rk["norms"][0]) <= 2
            if kp > 0:
                gidx = O.unpack_vector_layout(kcache.codes[b, h, t][None].cpu().numpy(), kp, d)
                fl = gidx != rk["idx"]
                if fl.any():
                    assert np.all(near_threshold(rk["y"][fl], ck, TIE_BAND))
                    clean[b] = False
                kc["codes"][b, h, t] = O.pack_vector_layout(rk["idx"], kp)[0]
            if kvar == "prod":
                gz = O.unpack_bits(kcache.signs[b, h, t][None].cpu().numpy(), d)
                fz = gz != rk["signs"]
                if fz.any():
                    srow = np.linalg.norm(kc["S"][h], axis=1)
                    assert np.all((np.abs(rk["p"]) / srow[None, :])[fz] <= TIE_BAND)
                    clean[b] = False
                if clean[b]:
                    assert abs(kcache.rnorms[b, h, t].item() - rk["gamma"][0]) <= 2e-5 * rk["gamma"][0] + 2e-7
                kc["signs"][b, h, t] = O.pack_bits(rk["signs"])[0]
                kc["rnorms"][b, h, t] = rk["rnorms"][0]
            kc["norms"][b, h, t] = rk["norms"][0]
            # values: slot t % 32 of block t // 32
            assert ulp_diff_f32(np.float32(vcache.norms[b, h, t].item()), rv["norms"][0]) <= 2
            gblk = O.unpack_block_layout(vcache.codes[b, h, t // 32][None].cpu().numpy(), vbits, d)
            fv = gblk[t % 32] != rv["idx"][0]
            if fv.any():
                assert np.all(near_threshold(rv["y"][0][fv], cv, TIE_BAND))
                clean[b] = False
            blk = O.unpack_block_layout(vc["codes"][b, h, t // 32][None], vbits, d)
            blk[t % 32] = rv["idx"][0]
            vc["codes"][b, h, t // 32] = O.pack_block_layout(blk, vbits)[0]
            vc["norms"][b, h, t] = rv["norms"][0]
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
    want = O.decode_attention(q, kc, vc, np.minimum(lens + 1, T), scale)
    for b in range(B):
        if not clean[b]:
            continue
        nbad, emax = allclose_report(got[b], want[b])
        assert nbad == 0, (b, int(lens[b]), nbad, emax)
    assert clean.sum() >= B - 1
