"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times, on outputs the fp64 oracle computes one by one.

* Layer quantize: 8 heads x 32768 tokens x {K, V}, d=128, mse b=3, bf16 in,
  keys in the vector layout and values in the 32-vector block layout, one call
  per tensor over all heads. Sampled vectors are re-quantized by the oracle:
  norms within 2 ulp, codes equal except where the fp64 rotated coordinate lies
  within 1e-5 of a decision midpoint (fewer than 1e-4 of them).
* Decode at context 131072 (batch 8, 64/8 heads) and 1,048,576 (batch 1, 64/8
  heads), keys prod b=3, values mse b=3. At 131072 the sampled (batch, kv head)
  groups are packed by the oracle from seeded vectors; at 1,048,576 the sampled
  group holds seeded random bits with per-token LogNormal norms (quantizing a
  million vectors in fp64 would take minutes). Every other group holds seeded
  random bits. All query heads of a sampled group must match the oracle's
  dequantize-then-attend within rtol 1e-3 / atol 1e-4, with full and ragged
  context lengths.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import tq_synth as syn
from tq_testlib import MAX_FLIP_RATE, TIE_BAND, allclose_report, near_threshold, ulp_diff_f32

pytestmark = pytest.mark.gpu
DEV = "cuda"
D = 128


def test_layer_quantize_full_size(gpu_lib):
    tq = gpu_lib
    H, T = 8, 32768
    print(f"layer quantize H={H} T={T} d={D} mse b=3", flush=True)
    cb = O.codebook(D, 3)
    g = np.random.default_rng(20260401)
    # the benchmark's call: keys and values of the layer in one tq_quantize_kv launch
    qs_kv = {t: [tq.Quantizer(D, 3, "mse", syn.rotation(D, syn.CFG_LAYER_QUANT, t, h)) for h in range(H)]
             for t in (syn.T_K, syn.T_V)}
    xs_kv = {t: syn.kv_vectors_device(H, T, D, syn.CFG_LAYER_QUANT, t, DEV) for t in (syn.T_K, syn.T_V)}
    outs = {t: {"codes": torch.empty((H, T * 48), dtype=torch.uint8, device=DEV),
                "norms": torch.empty((H, T), dtype=torch.float32, device=DEV)} for t in (syn.T_K, syn.T_V)}
    tq.quantize_kv(qs_kv[syn.T_K], qs_kv[syn.T_V], xs_kv[syn.T_K], xs_kv[syn.T_V], kout=outs[syn.T_K],
                   vout=outs[syn.T_V])
    torch.cuda.synchronize()
    for tensor, layout in ((syn.T_K, "vector"), (syn.T_V, "block32")):
        x = xs_kv[tensor]
        out = outs[tensor]
        codes = out["codes"].cpu().numpy()
        norms = out["norms"].cpu().numpy()
        n_flip = n_coord = 0
        for h in range(H):
            toks = np.unique(np.concatenate([g.integers(0, T, 512), [0, 31, 32, T - 33, T - 1]]))
            xs = x[h, torch.from_numpy(toks).to(DEV)].float().cpu().numpy()
            ref = O.quantize_mse(xs, syn.rotation(D, syn.CFG_LAYER_QUANT, tensor, h), cb)
            assert ulp_diff_f32(norms[h, toks], ref["nu"].astype(np.float32)).max() <= 2
            if layout == "vector":
                idx = O.unpack_vector_layout(codes[h].reshape(T, 48)[toks], 3, D)
            else:
                blocks = codes[h].reshape(T // 32, 4 * 3 * D)
                idx = np.stack([O.unpack_block_layout(blocks[t // 32][None], 3, D)[t % 32] for t in toks])
            flips = idx != ref["idx"]
            if flips.any():
                assert np.all(near_threshold(ref["y"][flips], cb, TIE_BAND)), (tensor, h)
            n_flip += int(flips.sum())
            n_coord += flips.size
        assert n_flip / n_coord < MAX_FLIP_RATE, (tensor, n_flip, n_coord)
    del xs_kv, outs


def _planes(bits, variant):
    return bits - 1 if variant == "prod" else bits


def _group_cache(T, d, kbits, kvar, vbits, config, b, h, lognormal):
    """Oracle-packed keys and values of one (batch, kv head) from seeded vectors."""
    Pk = syn.rotation(d, config, syn.T_K, h)
    Sk = syn.gaussian_matrix(d, config, syn.T_K, h) if kvar == "prod" else None
    Pv = syn.rotation(d, config, syn.T_V, h)
    kp = _planes(kbits, kvar)
    xk = syn.kv_vectors(T, d, config, syn.T_K, b, h, lognormal_sigma=lognormal)
    if kvar == "prod":
        rk = O.quantize_prod(xk, Pk, Sk, O.codebook(d, kp))
    else:
        rk = O.quantize_mse(xk, Pk, O.codebook(d, kp))
    del xk
    xv = syn.kv_vectors(T, d, config, syn.T_V, b, h, lognormal_sigma=lognormal)
    rv = O.quantize_mse(xv, Pv, O.codebook(d, vbits))
    del xv
    grp = {"knorms": rk["norms"], "vcodes": O.pack_block_layout(rv["idx"], vbits).reshape(T // 32, -1),
           "vnorms": rv["norms"], "Pk": Pk, "Sk": Sk, "Pv": Pv}
    if kp > 0:
        grp["kcodes"] = O.pack_vector_layout(rk["idx"], kp)
    if kvar == "prod":
        grp["ksigns"] = O.pack_bits(rk["signs"])
        grp["krnorms"] = rk["rnorms"]
    return grp


def _random_group(T, d, kbits, kvar, vbits, config, b, h, lognormal):
    """Seeded random bits and norms for one (batch, kv head) (prod b=3 keys, mse b=3 values)."""
    assert (kbits, kvar, vbits) == (3, "prod", 3)
    grp = syn.random_packed_group(T, d, 2 * d // 8, 4 * 3 * d, config, b, h, lognormal_sigma=lognormal)
    grp.update(Pk=syn.rotation(d, config, syn.T_K, h), Sk=syn.gaussian_matrix(d, config, syn.T_K, h),
               Pv=syn.rotation(d, config, syn.T_V, h))
    return grp


def _filled_cache(B, Hkv, T, d, kbits, kvar, vbits, seed):
    """Device cache arrays holding seeded random bits and positive norms."""
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    rb = lambda *s: torch.randint(0, 256, s, dtype=torch.uint8, device=DEV, generator=gen)
    rf = lambda lo, hi: lo + (hi - lo) * torch.rand((B, Hkv, T), device=DEV, generator=gen)
    kp = _planes(kbits, kvar)
    cache = {"knorms": rf(4.0, 30.0), "vcodes": rb(B, Hkv, T // 32, 4 * vbits * d), "vnorms": rf(4.0, 30.0)}
    if kp > 0:
        cache["kcodes"] = rb(B, Hkv, T, kp * d // 8)
    if kvar == "prod":
        cache["ksigns"] = rb(B, Hkv, T, d // 8)
        cache["krnorms"] = rf(0.2, 0.5)
    return cache


def _oracle_group_outputs(grp, d, kbits, kvar, vbits, q_heads, lens, scale):
    """softmax attention of each query head over the group's dequantized cache,
    for each context length in lens: [len(lens), n_heads, d]."""
    T = max(lens)
    kp = _planes(kbits, kvar)
    ck = O.codebook(d, kp)
    idx_k = O.unpack_vector_layout(grp["kcodes"][:T], kp, d) if kp > 0 else np.zeros((T, d), np.int64)
    if kvar == "prod":
        z = O.unpack_bits(grp["ksigns"][:T], d)
        K = O.dequantize_prod(idx_k, z, grp["knorms"][:T], grp["krnorms"][:T], grp["Pk"], grp["Sk"], ck)
        del z
    else:
        K = O.dequantize_mse(idx_k, grp["knorms"][:T], grp["Pk"], ck)
    del idx_k
    idx_v = O.unpack_block_layout(grp["vcodes"][:(T + 31) // 32], vbits, d)[:T]
    V = O.dequantize_mse(idx_v, grp["vnorms"][:T], grp["Pv"], O.codebook(d, vbits))
    del idx_v
    return np.stack([np.stack([O.attention(qh, K[:n], V[:n], scale)[0] for qh in q_heads]) for n in lens])


def _decode_full(tq, B, Hq, Hkv, T, d, kbits, kvar, vbits, config, lognormal, groups, ragged,
                 make_group=_group_cache):
    print(f"decode B={B} Hq={Hq} Hkv={Hkv} d={d} T={T} K {kvar}{kbits} V mse{vbits} groups={groups}", flush=True)
    cache = _filled_cache(B, Hkv, T, d, kbits, kvar, vbits, 1000 + config)
    oracle_groups = {}
    for (b, h) in groups:
        grp = make_group(T, d, kbits, kvar, vbits, config, b, h, lognormal)
        for k in ("kcodes", "ksigns", "knorms", "krnorms", "vcodes", "vnorms"):
            if k in cache:
                cache[k][b, h].copy_(torch.from_numpy(np.ascontiguousarray(grp[k])))
        oracle_groups[(b, h)] = grp
    kq, vq = [], []
    for h in range(Hkv):
        S = syn.gaussian_matrix(d, config, syn.T_K, h) if kvar == "prod" else None
        kq.append(tq.Quantizer(d, kbits, kvar, syn.rotation(d, config, syn.T_K, h), S))
        vq.append(tq.Quantizer(d, vbits, "mse", syn.rotation(d, config, syn.T_V, h)))
    kcache = tq.KVCache(kq, cache["knorms"], cache.get("kcodes"), cache.get("ksigns"), cache.get("krnorms"))
    vcache = tq.KVCache(vq, cache["vnorms"], cache["vcodes"])
    qn = syn.decode_queries(B, Hq, d, config)
    q = torch.from_numpy(qn).to(DEV).to(torch.bfloat16)
    scale = 1.0 / math.sqrt(d)
    ws = torch.empty(tq.decode_workspace_size(B, Hq, Hkv, d, T, kcache, vcache), dtype=torch.uint8, device=DEV)
    outs = []
    for lens in (np.full(B, T, np.int32), ragged):
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=DEV)
        tq.decode_attention(q, kcache, vcache, torch.from_numpy(lens).to(DEV), scale, max_ctx=T, out=out, workspace=ws)
        outs.append((lens, out))
    torch.cuda.synchronize()
    assert all(torch.isfinite(o).all().item() for _, o in outs)
    group = Hq // Hkv
    for (b, h), grp in oracle_groups.items():
        heads = list(range(h * group, (h + 1) * group))
        lens_bh = [int(outs[0][0][b]), int(outs[1][0][b])]
        print(f"  oracle group b={b} h={h} lens={lens_bh}", flush=True)
        want = _oracle_group_outputs(grp, d, kbits, kvar, vbits, qn[b, heads], lens_bh, scale)
        for i, (lens, out) in enumerate(outs):
            got = out[b, heads].cpu().numpy()
            nbad, emax = allclose_report(got, want[i])
            assert nbad == 0, (b, h, int(lens[b]), nbad, emax)


def test_decode_full_size_ctx128k(gpu_lib):
    T = 131072
    ragged = np.array([T, T - 1, T - 31, T - 33, 1, 4096 + 17, T // 2 + 5, T - 7], np.int32)
    _decode_full(gpu_lib, 8, 64, 8, T, D, 3, "prod", 3, syn.CFG_DECODE_128K, 0.0, [(0, 0), (7, 5)], ragged)


def test_decode_full_size_ctx1m(gpu_lib):
    T = 1 << 20
    _decode_full(gpu_lib, 1, 64, 8, T, D, 3, "prod", 3, syn.CFG_DECODE_1M, 0.5, [(0, 3)],
                 np.array([T - 77], np.int32), make_group=_random_group)


SWEEP = [(d, kvar, b) for d in (64, 256) for kvar in ("mse", "prod") for b in (1, 2, 4)]


@pytest.mark.parametrize("d,kvar,bits", SWEEP, ids=lambda v: str(v))
def test_decode_sweep_full_size(gpu_lib, d, kvar, bits):
    """b x variant x d sweep at batch 4, 64/8 heads, context 16384 (values mse at the same b)."""
    T = 16384
    ragged = np.array([T, T - 3, 977, 33], np.int32)
    _decode_full(gpu_lib, 4, 64, 8, T, d, bits, kvar, bits, syn.CFG_SWEEP, 0.0, [(1, 6), (3, 2)], ragged)


@pytest.mark.parametrize("d,variant,bits", SWEEP, ids=lambda v: str(v))
def test_quantize_sweep_full_size(gpu_lib, d, variant, bits):
    """Quantize of the sweep's keys (batch 4 x 8 heads x 16384 tokens) in one call per batch
    entry, sampled vectors against the oracle (codes, signs, norms, residual norms)."""
    tq = gpu_lib
    H, T = 8, 16384
    print(f"sweep quantize d={d} {variant} b={bits} H={H} T={T}", flush=True)
    planes = _planes(bits, variant)
    cb = O.codebook(d, planes)
    g = np.random.default_rng(7 + d + bits)
    mats = []
    qs = []
    for h in range(H):
        Pi = syn.rotation(d, syn.CFG_SWEEP, syn.T_K, h)
        S = syn.gaussian_matrix(d, syn.CFG_SWEEP, syn.T_K, h) if variant == "prod" else None
        mats.append((Pi, S))
        qs.append(tq.Quantizer(d, bits, variant, Pi, S))
    n_flip = n_coord = 0
    for b in (0, 3):
        x = syn.kv_vectors_device(H, T, d, syn.CFG_SWEEP, syn.T_K, DEV, seed_offset=b)
        out = {"norms": torch.empty((H, T), dtype=torch.float32, device=DEV)}
        if planes > 0:
            out["codes"] = torch.empty((H, T * planes * d // 8), dtype=torch.uint8, device=DEV)
        if variant == "prod":
            out["signs"] = torch.empty((H, T, d // 8), dtype=torch.uint8, device=DEV)
            out["rnorms"] = torch.empty((H, T), dtype=torch.float32, device=DEV)
        tq.quantize(qs, x, layout="vector", out=out)
        torch.cuda.synchronize()
        for h in range(H):
            toks = np.unique(np.concatenate([g.integers(0, T, 256), [0, T - 1]]))
            xs = x[h, torch.from_numpy(toks).to(DEV)].float().cpu().numpy()
            Pi, S = mats[h]
            ref = O.quantize_prod(xs, Pi, S, cb) if variant == "prod" else O.quantize_mse(xs, Pi, cb)
            assert ulp_diff_f32(out["norms"][h, toks].cpu().numpy(), ref["nu"].astype(np.float32)).max() <= 2
            same = np.ones(len(toks), bool)
            if planes > 0:
                idx = O.unpack_vector_layout(out["codes"][h].view(T, -1)[torch.from_numpy(toks).to(DEV)].cpu().numpy(),
                                             planes, d)
                flips = idx != ref["idx"]
                if flips.any():
                    assert np.all(near_threshold(ref["y"][flips], cb, TIE_BAND)), (b, h)
                n_flip += int(flips.sum())
                n_coord += flips.size
                same = ~flips.any(axis=1)
            if variant == "prod":
                rn = out["rnorms"][h, toks].cpu().numpy()
                assert np.allclose(rn[same], ref["gamma"][same], rtol=2e-5, atol=2e-7)
                z = O.unpack_bits(out["signs"][h, torch.from_numpy(toks).to(DEV)].cpu().numpy(), d)
                srow = np.linalg.norm(S, axis=1)
                sflip = z[same] != ref["signs"][same]
                if sflip.any():
                    assert np.all((np.abs(ref["p"][same]) / srow[None, :])[sflip] <= TIE_BAND), (b, h)
        del x, out
    if n_coord:
        assert n_flip / n_coord < MAX_FLIP_RATE, (n_flip, n_coord)
