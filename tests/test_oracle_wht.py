"""Pins of the oracle's randomized Walsh-Hadamard rotation ([NIK] "What the
community did", item 3): the Sylvester-Hadamard closed form against the
textbook routine and its recursion, orthogonality, a butterfly transform, and
the MSE distortion re-measured under the structured rotation."""
import math

import numpy as np
import pytest
import scipy.linalg

import oracle as O
import tq_synth as syn

# d * C(f_X, b) at d = 128 (exact Lloyd-Max cost, pinned in test_oracle_codebook.py)
DMSE_128 = {1: 0.360889, 2: 0.116000, 3: 0.033966, 4: 0.009315}


@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 64, 128, 256])
def test_hadamard_equals_textbook_routine(d):
    assert np.array_equal(O.hadamard(d), scipy.linalg.hadamard(d).astype(np.float64))


@pytest.mark.parametrize("d", [2, 8, 64, 256])
def test_hadamard_sylvester_recursion_and_orthogonality(d):
    h = O.hadamard(d // 2)
    assert np.array_equal(O.hadamard(d), np.block([[h, h], [h, -h]]))
    H = O.hadamard(d)
    assert np.array_equal(H @ H.T, d * np.eye(d))


def test_hadamard_rejects_other_sizes():
    for d in (0, 3, 96, 100):
        with pytest.raises(ValueError):
            O.hadamard(d)


def _fwht(x):
    """Iterative butterfly transform (unnormalized), an algorithm independent of the closed form."""
    x = np.array(x, dtype=np.float64)
    n = x.shape[-1]
    h = 1
    while h < n:
        for i in range(0, n, 2 * h):
            a = x[..., i:i + h].copy()
            b = x[..., i + h:i + 2 * h].copy()
            x[..., i:i + h] = a + b
            x[..., i + h:i + 2 * h] = a - b
        h *= 2
    return x


@pytest.mark.parametrize("d", [64, 128, 256])
def test_wht_rotation_is_orthogonal_and_matches_butterflies(d):
    s = syn.wht_signs(d, syn.CFG_TEST, syn.T_K, 3)
    assert set(np.unique(s)) <= {-1.0, 1.0}
    Pi = O.wht_rotation(s)
    assert np.abs(Pi @ Pi.T - np.eye(d)).max() <= 1e-12
    u = np.random.default_rng(5).standard_normal((17, d))
    want = _fwht(u * s[None, :]) / math.sqrt(d)
    assert np.abs(u @ Pi.T - want).max() <= 1e-12


def test_wht_flat_column_distortion_closed_form():
    """e_1 maps to a flat vector (every coordinate +-1/sqrt(d)), so its MSE
    distortion is d (1/sqrt(d) - c*)^2 with c* the centroid nearest 1/sqrt(d):
    the structured rotation is not Haar on this input."""
    d = 128
    s = syn.wht_signs(d, syn.CFG_TEST, syn.T_K, 0)
    Pi = O.wht_rotation(s)
    x = np.zeros((1, d))
    x[0, 0] = 1.0
    for b in (1, 2, 3, 4):
        cb = O.codebook(d, b)
        r = O.quantize_mse(x, Pi, cb)
        xt = O.dequantize_mse(r["idx"], r["norms"], Pi, cb)
        a = 1 / math.sqrt(d)
        cstar = cb[np.argmin(np.abs(cb - a))]
        assert abs(np.sum((x - xt) ** 2) - d * (a - cstar) ** 2) < 1e-12
    # b = 2: the flat vector sits between the two positive centroids, far from both
    cb2 = O.codebook(d, 2)
    assert d * (1 / math.sqrt(d) - cb2[np.argmin(np.abs(cb2 - 1 / math.sqrt(d)))]) ** 2 > 2 * DMSE_128[2]


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_wht_mse_distortion_on_gaussian_inputs(b):
    """For x ~ N(0, I), x/|x| is uniform on the sphere and any fixed orthogonal
    Pi keeps it uniform, so the mean distortion equals the Haar value d C(f_X, b)."""
    d, n = 128, 20000
    s = syn.wht_signs(d, syn.CFG_TEST, syn.T_K, 1)
    Pi = O.wht_rotation(s)
    x = np.random.default_rng(11 + b).standard_normal((n, d))
    cb = O.codebook(d, b)
    r = O.quantize_mse(x, Pi, cb)
    u = x / np.linalg.norm(x, axis=1, keepdims=True)
    ut = O.dequantize_mse(r["idx"], np.ones(n), Pi, cb)
    err = np.sum((u - ut) ** 2, axis=1)
    se = err.std() / math.sqrt(n)
    assert abs(err.mean() - DMSE_128[b]) <= 4 * se, (err.mean(), DMSE_128[b], se)


@pytest.mark.parametrize("outliers", [0, 4])
def test_wht_mse_distortion_on_kv_vectors(outliers):
    """Re-measured on the synthetic KV vectors, averaged over 16 rotations of
    each kind (d = 128, b = 3). Without outlier channels both rotations give the
    Haar value d C(f_X, 3). With 4 outlier channels x10 per head a Haar rotation
    still averages to that value (over rotations, for any fixed input), while the
    structured rotation maps each outlier channel to a flat +-1/sqrt(d) pattern and
    lands about 10 % lower, at 0.0305, with little spread between sign draws."""
    d, n, b, draws = 128, 2048, 3, 16
    cb = O.codebook(d, b)
    res = {"haar": [], "wht": []}
    for h in range(draws):
        x = syn.kv_vectors(n, d, syn.CFG_TEST, syn.T_K, 0, h, outliers=outliers).astype(np.float64)
        u = x / np.linalg.norm(x, axis=1, keepdims=True)
        for name, Pi in (("haar", syn.rotation(d, syn.CFG_TEST, syn.T_K, h)),
                         ("wht", O.wht_rotation(syn.wht_signs(d, syn.CFG_TEST, syn.T_K, h)))):
            r = O.quantize_mse(x, Pi, cb)
            ut = O.dequantize_mse(r["idx"], np.ones(n), Pi, cb)
            res[name].append(np.mean(np.sum((u - ut) ** 2, axis=1)))
    haar, wht = np.mean(res["haar"]), np.mean(res["wht"])
    assert abs(haar - DMSE_128[b]) < 0.03 * DMSE_128[b], res
    if outliers == 0:
        assert abs(wht - DMSE_128[b]) < 0.02 * DMSE_128[b], res
    else:
        assert 0.029 < wht < 0.032, res
        assert np.std(res["wht"]) < 0.2 * np.std(res["haar"]), res
