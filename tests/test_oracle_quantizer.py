"""Pins for the oracle's quantizers, bit layouts and attention.

Each check ties the oracle to something other than its own formulas: brute force
over every code on tiny d, a hand-made layout example, Monte-Carlo expectations
that the pages state as theorems ("Eternal mathematics of TurboQuant": Theorem 1,
the bias section, the QJL lemma, Theorem 2), torch's float64 attention, and
special cases with known answers.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
import tq_synth as syn

HERE = os.path.dirname(__file__)
PAGE = json.load(open(os.path.join(HERE, "golden", "page_tables.json")))


def _haar(d, rng):
    q, r = np.linalg.qr(rng.standard_normal((d, d)))
    return q * np.sign(np.diag(r))[None, :]


def test_rotation_is_orthogonal():
    for d in (64, 128, 256):
        P = syn.rotation(d, syn.CFG_TEST, 0, 3)
        assert np.max(np.abs(P @ P.T - np.eye(d))) <= 1e-12


def test_pack_worked_example():
    ex = json.load(open(os.path.join(HERE, "golden", "pack_example.json")))
    idx = np.array([ex["idx"]])
    packed = O.pack_vector_layout(idx, ex["bits"])
    assert packed.tolist() == [ex["bytes"]]
    assert O.unpack_vector_layout(packed, ex["bits"], ex["d"]).tolist() == [ex["idx"]]


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_layout_roundtrips_and_bit_positions(bits, d):
    g = np.random.Generator(np.random.PCG64(bits * 1000 + d))
    idx = g.integers(0, 1 << bits, size=(64, d))
    v = O.pack_vector_layout(idx, bits)
    assert v.shape == (64, bits * d // 8)
    assert np.array_equal(O.unpack_vector_layout(v, bits, d), idx)
    blk = O.pack_block_layout(idx, bits)
    assert blk.shape == (2, 4 * bits * d)
    assert np.array_equal(O.unpack_block_layout(blk, bits, d), idx)
    # direct bit lookups from the written definitions, one element at a time
    for _ in range(200):
        n, j, p = int(g.integers(64)), int(g.integers(d)), int(g.integers(bits))
        want = (idx[n, j] >> p) & 1
        assert (v[n, p * d // 8 + j // 8] >> (j % 8)) & 1 == want
        blk_i, u = divmod(n, 32)
        half, rem = divmod(u, 16)
        gg, k = divmod(rem, 4)
        w, r = divmod(j, 4)
        word_off = ((p * 4 + gg) * (d // 4) + w) * 4
        word = int.from_bytes(bytes(blk[blk_i, word_off:word_off + 4]), "little")
        assert (word >> (16 * half + 4 * r + k)) & 1 == want


@pytest.mark.parametrize("d,bits", [(3, 1), (3, 2), (3, 3), (4, 1), (4, 2), (4, 3), (8, 1), (8, 2)])
def test_brute_force_argmin_over_all_codes(d, bits):
    """Q_mse(x) must be the packed code whose reconstruction is nearest to y = Pi x/|x|,
    over every one of the 2^(b d) codes (pins argmin, separability and the layout)."""
    rng = np.random.Generator(np.random.PCG64(d * 10 + bits))
    Pi = _haar(d, rng)
    c = O.codebook(d, bits)
    nbytes = bits * ((d + 7) // 8)
    allcodes = np.arange(1 << (bits * d), dtype=np.uint64)
    # reference unpack from the definition (plane p of coordinate j is bit p*d + j of the code integer)
    idx_all = np.zeros((allcodes.size, d), dtype=np.int64)
    for p in range(bits):
        for j in range(d):
            idx_all[:, j] |= ((allcodes >> np.uint64(p * d + j)) & np.uint64(1)).astype(np.int64) << p
    recon = c[idx_all]
    x = rng.standard_normal((20, d))
    r = O.quantize_mse(x, Pi, c)
    for i in range(x.shape[0]):
        err = np.sum((recon - r["y"][i]) ** 2, axis=1)
        best = int(np.argmin(err))
        assert np.array_equal(idx_all[best], r["idx"][i])
        if d % 8 == 0:
            packed = O.pack_vector_layout(r["idx"][i:i + 1], bits)[0]
            as_int = 0
            for p in range(bits):
                for j in range(d):
                    as_int |= int((packed[p * d // 8 + j // 8] >> (j % 8)) & 1) << (p * d + j)
            assert as_int == best
    del nbytes


def test_nearest_index_ties_go_low():
    c = np.array([-1.0, 0.0, 1.0])
    assert O.nearest_index([-0.5, 0.5, 0.0, -2, 2], c).tolist() == [0, 1, 1, 0, 2]


def test_zero_vector():
    d = 64
    Pi = syn.rotation(d, syn.CFG_TEST)
    S = syn.gaussian_matrix(d, syn.CFG_TEST)
    x = np.zeros((2, d)); x[1, 3] = 2.0
    r = O.quantize_mse(x, Pi, O.codebook(d, 3))
    assert np.all(r["idx"][0] == 0) and r["norms"][0] == 0
    assert np.all(O.dequantize_mse(r["idx"], r["norms"], Pi, O.codebook(d, 3))[0] == 0)
    rp = O.quantize_prod(x, Pi, S, O.codebook(d, 2))
    assert np.all(rp["idx"][0] == 0) and not rp["signs"][0].any() and rp["rnorms"][0] == 0
    xt = O.dequantize_prod(rp["idx"], rp["signs"], rp["norms"], rp["rnorms"], Pi, S, O.codebook(d, 2))
    assert np.all(xt[0] == 0)


def test_rotated_query_identity():
    d = 128
    Pi = syn.rotation(d, syn.CFG_TEST)
    g = np.random.Generator(np.random.PCG64(3))
    q, yt = g.standard_normal(d), g.standard_normal(d)
    assert abs(q @ (yt @ Pi) - (Pi @ q) @ yt) < 1e-12


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_mse_distortion_is_data_oblivious(bits):
    """Theorem 1: E_Pi |u - u~|^2 = d * C(f_X, b) for ANY fixed unit u (here e_1 and an
    outlier-heavy vector), because Pi u is uniform on the sphere. Also the bias
    section: E <x, x~> = (1 - D) |x|^2 (2/pi in the Gaussian limit at b = 1)."""
    d, trials = 32, 3000
    c = O.codebook(d, bits)
    _, cost, _ = O.lloyd_max(d, bits)
    D = d * cost
    rng = np.random.Generator(np.random.PCG64(100 + bits))
    u1 = np.zeros(d); u1[0] = 1.0
    u2 = np.ones(d); u2[:3] = 30.0
    for u in (u1, u2 / np.linalg.norm(u2)):
        errs, dots = np.empty(trials), np.empty(trials)
        for t in range(trials):
            Pi = _haar(d, rng)
            r = O.quantize_mse(u[None, :], Pi, c)
            ut = O.dequantize_mse(r["idx"], r["norms"].astype(np.float64), Pi, c)[0]
            errs[t] = np.sum((u - ut) ** 2)
            dots[t] = u @ ut
        se = errs.std() / math.sqrt(trials)
        assert abs(errs.mean() - D) < 4 * se + 1e-12, (errs.mean(), D, se)
        se2 = dots.std() / math.sqrt(trials)
        assert abs(dots.mean() - (1 - D)) < 4 * se2 + 1e-12


@pytest.mark.parametrize("d", [64, 128])
def test_requantize_is_idempotent(d):
    """Q(Q^-1(Q(x))) = Q(x) for mse ([NIK] "Step 2": dequantize is the centroid
    lookup then Pi^T). Re-quantizing sees y' = c[idx] / |c[idx]|, each centroid
    scaled by s = 1/|c[idx]|. The symmetric codebook keeps every centroid in its
    own cell (mids[i-1], mids[i]] exactly for s in (s_lo, s_hi), computed from the
    codebook; when every observed s lies there the indices must come back
    unchanged. A transposed Pi in either direction or a wrong centroid lookup
    breaks it."""
    Pi = syn.rotation(d, syn.CFG_TEST, syn.T_K, 3)
    x = np.random.default_rng(1).standard_normal((2000, d))
    for bits in (1, 2, 3, 4):
        c = O.codebook(d, bits)
        mids = (c[:-1] + c[1:]) / 2  # cell i is (mids[i-1], mids[i]]
        pos = c > 0  # by symmetry the negative half mirrors it
        s_hi = np.min(mids[pos[:-1]] / c[:-1][pos[:-1]]) if pos[:-1].any() else np.inf
        inner = pos[1:] & (mids > 0)
        s_lo = np.max(mids[inner] / c[1:][inner]) if inner.any() else 0.0
        r = O.quantize_mse(x, Pi, c)
        scale = 1.0 / np.linalg.norm(c[r["idx"]], axis=1)
        assert scale.min() > s_lo and scale.max() < s_hi, (bits, s_lo, s_hi, scale.min(), scale.max())
        xt = O.dequantize_mse(r["idx"], r["norms"], Pi, c)
        assert np.array_equal(O.quantize_mse(xt, Pi, c)["idx"], r["idx"])
        assert not np.array_equal(O.quantize_mse(xt, Pi.T, c)["idx"], r["idx"])


def test_qjl_unbiased_and_variance():
    """QJL lemma: E <y, Q^-1(Q(x))> = <y, x>, Var = (pi/2 |y|^2 - <x,y>^2)/d <= pi/(2d) |y|^2."""
    d, trials = 32, 10000
    rng = np.random.Generator(np.random.PCG64(5))
    x = rng.standard_normal(d); x /= np.linalg.norm(x)
    y = rng.standard_normal(d)
    est = np.empty(trials)
    for t in range(trials):
        S = rng.standard_normal((d, d))
        est[t] = y @ O.qjl_inverse(O.qjl(x[None, :], S), S)[0]
    se = est.std() / math.sqrt(trials)
    assert abs(est.mean() - x @ y) < 4 * se
    var_exact = (math.pi / 2 * (y @ y) - (x @ y) ** 2) / d
    assert abs(est.var() - var_exact) < 0.06 * var_exact
    assert est.var() <= math.pi / (2 * d) * (y @ y) * 1.05


@pytest.mark.parametrize("bits", [1, 2, 3])
def test_prod_unbiased_and_distortion(bits):
    """Theorem 2: prod is unbiased for <y, x>; with y independent of x the normalized
    distortion D_prod d / |y|^2 = (pi/2 - 1/d) * D_mse(b-1) (from the conditional
    variance in the proof), within the page's table to +-15 percent."""
    d, trials = 64, 4000
    cb = O.codebook(d, bits - 1)
    _, cost_bm1, _ = O.lloyd_max(d, bits - 1) if bits > 1 else (None, 1.0 / d, 0)
    rng = np.random.Generator(np.random.PCG64(50 + bits))
    x = rng.standard_normal(d); x /= np.linalg.norm(x)
    y = rng.standard_normal(d)
    est = np.empty(trials)
    dn = np.empty(trials)
    for t in range(trials):
        Pi = _haar(d, rng)
        S = rng.standard_normal((d, d))
        r = O.quantize_prod(x[None, :], Pi, S, cb)
        xt = O.dequantize_prod(r["idx"], r["signs"], r["nu"], r["gamma"], Pi, S, cb)[0]
        est[t] = y @ xt
        yr = rng.standard_normal(d)   # a fresh direction independent of x for the distortion
        dn[t] = (yr @ x - yr @ xt) ** 2 * d / (yr @ yr)
    se = est.std() / math.sqrt(trials)
    assert abs(est.mean() - x @ y) < 4 * se
    expect = (math.pi / 2 - 1.0 / d) * d * cost_bm1
    se_d = dn.std() / math.sqrt(trials)
    assert abs(dn.mean() - expect) < 4 * se_d
    printed = PAGE["d_prod_times_d_over_y2"][str(bits)]
    assert abs(expect - printed) < 0.15 * printed


def test_prod_b1_is_pure_qjl():
    d = 64
    rng = np.random.Generator(np.random.PCG64(9))
    Pi, S = _haar(d, rng), rng.standard_normal((d, d))
    x = rng.standard_normal((5, d))
    r = O.quantize_prod(x, Pi, S, O.codebook(d, 0))
    assert np.all(r["idx"] == 0)
    assert np.allclose(r["gamma"], 1.0)
    assert np.array_equal(r["signs"], O.qjl(x / np.linalg.norm(x, axis=1, keepdims=True), S))


def test_attention_matches_torch_sdpa_float64():
    rng = np.random.Generator(np.random.PCG64(11))
    T, d = 37, 16
    q, K, V = rng.standard_normal(d), rng.standard_normal((T, d)), rng.standard_normal((T, d))
    scale = 1 / math.sqrt(d)
    o, _ = O.attention(q, K, V, scale)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[None, None, None, :], torch.tensor(K)[None, None], torch.tensor(V)[None, None],
        scale=scale)[0, 0, 0].numpy()
    assert np.allclose(o, ref, rtol=1e-13, atol=1e-14)


def test_attention_special_cases():
    rng = np.random.Generator(np.random.PCG64(12))
    d = 8
    V = rng.standard_normal((1, d))
    o, _ = O.attention(rng.standard_normal(d), rng.standard_normal((1, d)), V, 0.3)
    assert np.allclose(o, V[0], rtol=0, atol=1e-15)
    K = np.repeat(rng.standard_normal((1, d)), 5, axis=0)
    V = rng.standard_normal((5, d))
    o, _ = O.attention(rng.standard_normal(d), K, V, 0.3)
    assert np.allclose(o, V.mean(axis=0), rtol=0, atol=1e-14)


def _small_cache(B, Hkv, T, d, kbits, kvar, vbits, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    Pk = np.stack([_haar(d, rng) for _ in range(Hkv)])
    Pv = np.stack([_haar(d, rng) for _ in range(Hkv)])
    Sk = rng.standard_normal((Hkv, d, d))
    kp = kbits - (1 if kvar == "prod" else 0)
    ck, cv = O.codebook(d, kp), O.codebook(d, vbits)
    Xk = rng.standard_normal((B, Hkv, T, d))
    Xv = rng.standard_normal((B, Hkv, T, d))
    kc = {"variant": kvar, "bits": kbits, "d": d, "max_ctx": T, "Pi": Pk, "S": Sk,
          "codes": np.zeros((B, Hkv, T, max(kp, 1) * d // 8), np.uint8),
          "signs": np.zeros((B, Hkv, T, d // 8), np.uint8),
          "norms": np.zeros((B, Hkv, T), np.float32), "rnorms": np.zeros((B, Hkv, T), np.float32)}
    vc = {"variant": "mse", "bits": vbits, "d": d, "max_ctx": T, "Pi": Pv,
          "codes": np.zeros((B, Hkv, T // 32, 4 * vbits * d), np.uint8),
          "norms": np.zeros((B, Hkv, T), np.float32)}
    Kd = np.zeros((B, Hkv, T, d)); Vd = np.zeros((B, Hkv, T, d))
    for b in range(B):
        for h in range(Hkv):
            if kvar == "prod":
                r = O.quantize_prod(Xk[b, h], Pk[h], Sk[h], ck)
                kc["signs"][b, h] = O.pack_bits(r["signs"])
                kc["rnorms"][b, h] = r["rnorms"]
                Kd[b, h] = O.dequantize_prod(r["idx"], r["signs"], r["norms"], r["rnorms"], Pk[h], Sk[h], ck)
            else:
                r = O.quantize_mse(Xk[b, h], Pk[h], ck)
                Kd[b, h] = O.dequantize_mse(r["idx"], r["norms"], Pk[h], ck)
            if kp > 0:
                kc["codes"][b, h] = O.pack_vector_layout(r["idx"], kp)
            kc["norms"][b, h] = r["norms"]
            rv = O.quantize_mse(Xv[b, h], Pv[h], cv)
            vc["codes"][b, h] = O.pack_block_layout(rv["idx"], vbits).reshape(T // 32, -1)
            vc["norms"][b, h] = rv["norms"]
            Vd[b, h] = O.dequantize_mse(rv["idx"], rv["norms"], Pv[h], cv)
    return kc, vc, Kd, Vd


@pytest.mark.parametrize("kvar", ["prod", "mse"])
def test_decode_attention_is_dequantize_then_attend(kvar):
    B, Hkv, Hq, T, d = 2, 2, 4, 64, 32
    kc, vc, Kd, Vd = _small_cache(B, Hkv, T, d, 3, kvar, 2, 77)
    rng = np.random.Generator(np.random.PCG64(78))
    q = rng.standard_normal((B, Hq, d))
    lens = np.array([64, 37])
    out = O.decode_attention(q, kc, vc, lens, 0.2)
    for b in range(B):
        for hq in range(Hq):
            h = hq * Hkv // Hq
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.tensor(q[b, hq])[None, None, None, :],
                torch.tensor(Kd[b, h, :lens[b]])[None, None], torch.tensor(Vd[b, h, :lens[b]])[None, None],
                scale=0.2)[0, 0, 0].numpy()
            assert np.allclose(out[b, hq], ref, rtol=1e-12, atol=1e-13)
