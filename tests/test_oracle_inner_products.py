"""Pins for the oracle's inner products <y_i, x~_j> (the quantity D_prod is
defined on in "Eternal mathematics of TurboQuant", problem statement and
Theorem 2, and the score a vector search ranks by, section "Experiments").

The oracle computes the whole [m, n] matrix with one library product; these
checks tie it to values worked out by hand, to one-pair-at-a-time sums, and to
the rotated-space form of the dequantizers (the score the decode kernels use),
so that a transposed operand, a swapped query/vector order or a dropped QJL
term fails here.
"""
import math

import numpy as np

import oracle as O
import tq_synth as syn


def test_hand_worked_integer_example():
    # m = 2 queries, n = 3 vectors, d = 3; every entry worked out by hand
    y = np.array([[1.0, 2.0, -1.0], [0.0, 3.0, 4.0]])
    xt = np.array([[2.0, 0.0, 1.0], [1.0, 1.0, 1.0], [-3.0, 2.0, 5.0]])
    got = O.inner_products(y, xt)
    assert got.shape == (2, 3)
    assert got.tolist() == [[1.0, 2.0, -4.0], [4.0, 7.0, 26.0]]


def test_pairwise_sums_and_exact_inner_product_when_unquantized():
    g = np.random.Generator(np.random.PCG64(11))
    m, n, d = 5, 7, 96
    y = g.standard_normal((m, d))
    x = g.standard_normal((n, d))
    got = O.inner_products(y, x)
    assert got.shape == (m, n)
    for i in range(m):
        for j in range(n):
            want = math.fsum(float(y[i, k]) * float(x[j, k]) for k in range(d))
            assert abs(got[i, j] - want) <= 1e-12 * (1.0 + abs(want))


def test_zero_query_and_linearity_in_the_query():
    g = np.random.Generator(np.random.PCG64(12))
    y1, y2, x = g.standard_normal((3, 64)), g.standard_normal((3, 64)), g.standard_normal((4, 64))
    assert np.all(O.inner_products(np.zeros((2, 64)), x) == 0.0)
    lhs = O.inner_products(2.0 * y1 - 3.0 * y2, x)
    rhs = 2.0 * O.inner_products(y1, x) - 3.0 * O.inner_products(y2, x)
    assert np.max(np.abs(lhs - rhs)) <= 1e-12 * (1.0 + np.max(np.abs(rhs)))


def _rotated_mse_score(y, nu, Pi, c, idx):
    # <y, nu Pi^T c[idx]> = nu <Pi y, c[idx]>, one coordinate at a time
    py = [math.fsum(float(Pi[k, l]) * float(y[l]) for l in range(len(y))) for k in range(Pi.shape[0])]
    return float(nu) * math.fsum(py[k] * float(c[idx[k]]) for k in range(len(py)))


def test_matches_rotated_space_scores_of_mse_records():
    d, bits = 32, 3
    Pi = syn.rotation(d, syn.CFG_TEST, syn.T_K, 40)
    c = O.codebook(d, bits)
    g = np.random.Generator(np.random.PCG64(13))
    x = g.standard_normal((6, d)) * 3.0
    y = g.standard_normal((4, d))
    r = O.quantize_mse(x, Pi, c)
    xt = O.dequantize_mse(r["idx"], r["norms"], Pi, c)
    got = O.inner_products(y, xt)
    for i in range(4):
        for j in range(6):
            want = _rotated_mse_score(y[i], r["norms"][j], Pi, c, r["idx"][j])
            assert abs(got[i, j] - want) <= 1e-11 * (1.0 + abs(want))


def test_matches_rotated_space_scores_of_prod_records():
    # prod adds nu |r| sqrt(pi/2)/d <S y, z> with z = +-1 ("QJL: a one-bit method",
    # "TurboQuant proper"); dropping or mis-scaling that term fails this check
    d, bits = 32, 3
    Pi = syn.rotation(d, syn.CFG_TEST, syn.T_K, 41)
    S = syn.gaussian_matrix(d, syn.CFG_TEST, syn.T_K, 41)
    c = O.codebook(d, bits - 1)
    g = np.random.Generator(np.random.PCG64(14))
    x = g.standard_normal((5, d))
    y = g.standard_normal((3, d))
    r = O.quantize_prod(x, Pi, S, c)
    xt = O.dequantize_prod(r["idx"], r["signs"], r["norms"], r["rnorms"], Pi, S, c)
    got = O.inner_products(y, xt)
    kappa = math.sqrt(math.pi / 2.0) / d
    for i in range(3):
        sy = [math.fsum(float(S[k, l]) * float(y[i, l]) for l in range(d)) for k in range(d)]
        for j in range(5):
            mse = _rotated_mse_score(y[i], r["norms"][j], Pi, c, r["idx"][j])
            z = [1.0 if s else -1.0 for s in r["signs"][j]]
            qjl = float(r["norms"][j]) * float(r["rnorms"][j]) * kappa * math.fsum(sy[k] * z[k] for k in range(d))
            want = mse + qjl
            assert abs(got[i, j] - want) <= 1e-11 * (1.0 + abs(want))
