"""Pins of the oracle's outlier-channel split ([NIK] "Experiments", KV cache:
outlier channels and the others quantized by separate TurboQuant instances at
different bit widths):

* one part holding every channel in a permuted order is plain TurboQuant with
  the rotation Pi P (P the permutation), which pins the direction of the
  channel indexing;
* a vector living on one part's channels leaves the other part at norm 0 and
  all-zero codes, and the first part equal to plain TurboQuant of the
  sub-vector;
* on Gaussian rows the split's mean squared error is the closed form
  sum_p E|x_p|^2 d_p C(f_{d_p}, b_p) = sum_p d_p^2 C(f_{d_p}, b_p), since each
  part is TurboQuant in d_p dimensions and |x_p| is independent of x_p/|x_p|;
  swapping the parts' bit widths changes it by far more than the error bar;
* prod parts keep inner products unbiased, with the variance the sum of the
  parts' (pi/2 - 1/d_p) d_p C(f_{d_p}, b_p - 1) |y_p|^2 |x_p|^2 / d_p.
"""
import math

import numpy as np
import pytest

import oracle as O
import tq_synth as syn


def _cost(d, b):
    return O.lloyd_max(d, b)[1]


def _part(channels, variant, bits, seed):
    d = len(channels)
    planes = bits - 1 if variant == "prod" else bits
    p = {"channels": np.asarray(channels), "variant": variant, "Pi": syn.rotation(d, syn.CFG_TEST, syn.T_K, seed),
         "centroids": O.codebook(d, planes)}
    if variant == "prod":
        p["S"] = syn.gaussian_matrix(d, syn.CFG_TEST, syn.T_K, seed)
    return p


@pytest.mark.parametrize("variant", ["mse", "prod"])
def test_single_permuted_part_is_plain_turboquant(variant):
    d, n, bits = 64, 200, 3
    perm = np.random.default_rng(3).permutation(d)
    part = _part(perm, variant, bits, 1)
    x = np.random.default_rng(4).standard_normal((n, d))
    r = O.quantize_split(x, [part])[0]
    P = np.zeros((d, d))
    P[np.arange(d), perm] = 1.0  # (P u)_j = u[perm[j]]
    Pi2 = part["Pi"] @ P
    S2 = part["S"] @ P if variant == "prod" else None  # the residual is P^T r_sub in the original channels
    ref = O.quantize_prod(x, Pi2, S2, part["centroids"]) if variant == "prod" else \
        O.quantize_mse(x, Pi2, part["centroids"])
    assert np.array_equal(r["idx"], ref["idx"])
    assert np.array_equal(r["norms"], ref["norms"])
    assert np.abs(r["y"] - ref["y"]).max() < 1e-12
    if variant == "prod":
        assert np.array_equal(r["signs"], ref["signs"])
        assert np.abs(r["gamma"] - ref["gamma"]).max() < 1e-12
    # and the transposed permutation is a different quantizer
    bad = O.quantize_mse(x, part["Pi"] @ P.T, part["centroids"])
    assert not np.array_equal(r["idx"], bad["idx"])
    xt = O.dequantize_split([r], [part], d)
    xref = O.dequantize_prod(ref["idx"], ref["signs"], ref["norms"], ref["rnorms"], Pi2, S2, part["centroids"]) \
        if variant == "prod" else O.dequantize_mse(ref["idx"], ref["norms"], Pi2, part["centroids"])
    assert np.abs(xt - xref).max() < 1e-12


def test_vector_on_one_part():
    dim = 128
    ch = np.random.default_rng(5).permutation(dim)
    parts = [_part(ch[:32], "mse", 3, 2), _part(ch[32:], "prod", 2, 3)]
    x = np.zeros((10, dim))
    x[:, ch[:32]] = np.random.default_rng(6).standard_normal((10, 32))
    ra, rb = O.quantize_split(x, parts)
    assert np.all(rb["norms"] == 0) and not rb["idx"].any() and not rb["signs"].any() and np.all(rb["rnorms"] == 0)
    ref = O.quantize_mse(x[:, ch[:32]], parts[0]["Pi"], parts[0]["centroids"])
    assert np.array_equal(ra["idx"], ref["idx"])
    xt = O.dequantize_split([ra, rb], parts, dim)
    assert np.all(xt[:, ch[32:]] == 0)


def test_split_mse_closed_form():
    """The pages' split of a 128-channel head: 32 channels at 3 bits, 96 at 2."""
    dim, n = 128, 20000
    ch = np.random.default_rng(7).permutation(dim)
    parts = [_part(ch[:32], "mse", 3, 4), _part(ch[32:], "mse", 2, 5)]
    x = np.random.default_rng(8).standard_normal((n, dim))
    xt = O.dequantize_split(O.quantize_split(x, parts), parts, dim)
    err = np.sum((x - xt) ** 2, axis=1)
    want = 32 * 32 * _cost(32, 3) + 96 * 96 * _cost(96, 2)
    se = err.std() / math.sqrt(n)
    assert abs(err.mean() - want) < 4 * se, (err.mean(), want, se)
    swapped = 32 * 32 * _cost(32, 2) + 96 * 96 * _cost(96, 3)
    assert abs(swapped - want) > 40 * se
    # bits per channel of this split: (32 * 3 + 96 * 2) / 128
    assert (32 * 3 + 96 * 2) / 128 == 2.25


def test_split_prod_unbiased_with_closed_form_variance():
    dim, n = 128, 6000
    ch = np.random.default_rng(9).permutation(dim)
    parts = [_part(ch[:32], "prod", 3, 6), _part(ch[32:], "prod", 2, 7)]
    x = np.random.default_rng(10).standard_normal((n, dim))
    y = np.random.default_rng(11).standard_normal((32, dim))  # one S per part: average over query directions
    xt = O.dequantize_split(O.quantize_split(x, parts), parts, dim)
    err = O.inner_products(y, xt) - O.inner_products(y, x)  # [32, n]
    assert abs(err.mean()) < 4 * err.std() / math.sqrt(err.size)
    want = 0.0
    for p, b in zip(parts, (3, 2)):
        c = np.asarray(p["channels"])
        dp = len(c)
        yy = np.sum(y[:, c] ** 2, axis=1)[:, None]
        xx = np.sum(x[:, c] ** 2, axis=1)[None, :]
        want = want + (math.pi / 2 - 1 / dp) * dp * _cost(dp, b - 1) * yy * xx / dp
    ratio = np.mean(err ** 2) / np.mean(want)
    assert abs(ratio - 1) < 0.06, ratio


def test_split_decode_with_one_full_part_is_plain_decode():
    """One key part and one value part holding every channel in order reduce the
    split decode to the plain decode over the same records."""
    B, Hq, Hkv, d, T = 2, 4, 2, 32, 40
    lens = np.array([40, 0])
    ch = np.arange(d)
    kc = {"variant": "prod", "bits": 3, "d": d, "max_ctx": T, "Pi": [], "S": [],
          "codes": np.zeros((B, Hkv, T, 2 * d // 8), np.uint8), "signs": np.zeros((B, Hkv, T, d // 8), np.uint8),
          "norms": np.zeros((B, Hkv, T), np.float32), "rnorms": np.zeros((B, Hkv, T), np.float32)}
    vc = {"variant": "mse", "bits": 3, "d": d, "max_ctx": T, "Pi": [],
          "codes": np.zeros((B, Hkv, T // 32 if T % 32 == 0 else 0, 4 * 3 * d), np.uint8),
          "norms": np.zeros((B, Hkv, T), np.float32)}
    keys = [[None] * Hkv for _ in range(B)]
    values = [[None] * Hkv for _ in range(B)]
    kparts = [_part(ch, "prod", 3, 30 + g) for g in range(Hkv)]
    vparts = [_part(ch, "mse", 3, 40 + g) for g in range(Hkv)]
    Tp = 64  # block layout needs whole 32-token blocks: pad the value records
    vc["codes"] = np.zeros((B, Hkv, Tp // 32, 4 * 3 * d), np.uint8)
    for b in range(B):
        for g in range(Hkv):
            x = syn.kv_vectors(Tp, d, syn.CFG_TEST, syn.T_K, b, g)
            xv = syn.kv_vectors(Tp, d, syn.CFG_TEST, syn.T_V, b, g)
            rk = O.quantize_split(x[:T], [kparts[g]])
            rv = O.quantize_split(xv, [vparts[g]])
            keys[b][g] = (rk, [kparts[g]])
            values[b][g] = ([{k: (v[:T] if hasattr(v, "__len__") else v) for k, v in rv[0].items()}], [vparts[g]])
            kc["codes"][b, g] = O.pack_vector_layout(rk[0]["idx"], 2)
            kc["signs"][b, g] = O.pack_bits(rk[0]["signs"])
            kc["norms"][b, g] = rk[0]["norms"]
            kc["rnorms"][b, g] = rk[0]["rnorms"]
            vc["codes"][b, g] = O.pack_block_layout(rv[0]["idx"], 3).reshape(Tp // 32, -1)
            vc["norms"][b, g] = rv[0]["norms"][:T]
    kc["Pi"] = np.stack([p["Pi"] for p in kparts])
    kc["S"] = np.stack([p["S"] for p in kparts])
    vc["Pi"] = np.stack([p["Pi"] for p in vparts])
    q = syn.decode_queries(B, Hq, d, syn.CFG_TEST)
    got = O.decode_attention_split(q, keys, values, lens, 0.2, d)
    want = O.decode_attention(q, kc, vc, lens, 0.2)
    assert np.abs(got - want).max() < 1e-12
    assert np.all(got[1] == 0)
