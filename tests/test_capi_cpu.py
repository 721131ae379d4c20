"""Host-side checks of libtq: it loads, exports every declared symbol, its
Lloyd-Max codebook matches the oracle's independent solver, and invalid
arguments come back as documented status codes (no GPU needed)."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import attention_tq_quantize_amd as tq
import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return tq.load()


def test_exports_every_declared_symbol(lib):
    header = open(os.path.join(ROOT, "include", "tq.h")).read()
    declared = sorted(set(re.findall(r"\b(tq_[a-z_]+)\s*\(", header)))
    assert declared, "no declarations parsed"
    for name in declared:
        assert hasattr(lib, name), f"libtq.so does not export {name}"
    assert sorted(tq.EXPORTS) == declared
    assert lib.tq_version() >= 10000


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("bits", [0, 1, 2, 3, 4])
def test_codebook_matches_oracle(lib, d, bits):
    c, t, cost = tq.codebook_build(d, bits)
    oc = O.codebook(d, bits)
    assert np.array_equal(c.astype(np.float64), oc), (c, oc)
    if bits == 0:
        assert abs(cost - 1.0 / d) < 1e-15
        return
    _, ocost, _ = O.lloyd_max(d, bits)
    assert abs(cost - ocost) <= 1e-11 * ocost
    # thresholds: the largest float32 not above the exact midpoint of neighbouring centroids
    mids = (c[:-1].astype(np.float64) + c[1:].astype(np.float64)) / 2
    assert np.all(t.astype(np.float64) <= mids)
    assert np.all(np.nextafter(t, np.float32(np.inf)).astype(np.float64) > mids)


def test_codebook_threshold_compare_equals_argmin(lib):
    # for float32 y, (y > t_i) counting must equal the oracle's argmin with ties low
    d, bits = 128, 3
    c, t, _ = tq.codebook_build(d, bits)
    g = np.random.Generator(np.random.PCG64(1))
    y = (g.standard_normal(200000) / math.sqrt(d)).astype(np.float32)
    mids = ((c[:-1].astype(np.float64) + c[1:].astype(np.float64)) / 2).astype(np.float32)
    y = np.concatenate([y, mids, t, np.nextafter(t, np.float32(1)), np.nextafter(t, np.float32(-1))])
    idx_thr = np.sum(y[:, None] > t[None, :], axis=1)
    idx_arg = O.nearest_index(y.astype(np.float64), c.astype(np.float64))
    assert np.array_equal(idx_thr, idx_arg)


def test_codebook_special_cases(lib):
    # d = 3 is the uniform law: the uniform quantizer, D = 4^-b
    for bits in (1, 2, 3):
        c, _, cost = tq.codebook_build(3, bits)
        K = 1 << bits
        assert np.allclose(c, -1 + (2 * np.arange(K) + 1) / K, atol=1e-7)
        assert abs(3 * cost - 4.0 ** -bits) < 1e-12
    # b = 1 closed form
    for d in (16, 128, 1000):
        c, _, _ = tq.codebook_build(d, 1)
        cf = math.exp(math.lgamma(d / 2) - math.lgamma((d + 1) / 2)) / math.sqrt(math.pi)
        assert abs(c[1] - cf) <= 1e-7 * cf


def _status(fn, *args):
    return fn(*args)


def test_argument_errors(lib):
    pi = np.eye(128)
    h = ctypes.c_void_p()
    assert lib.tq_quantizer_create(100, 3, tq.TQ_MSE, pi.ctypes.data, None, ctypes.byref(h)) == tq.TQ_ERR_UNSUPPORTED
    assert lib.tq_quantizer_create(128, 5, tq.TQ_MSE, pi.ctypes.data, None, ctypes.byref(h)) == tq.TQ_ERR_UNSUPPORTED
    assert lib.tq_quantizer_create(128, 0, tq.TQ_MSE, pi.ctypes.data, None, ctypes.byref(h)) == tq.TQ_ERR_UNSUPPORTED
    assert lib.tq_quantizer_create(128, 3, tq.TQ_MSE, None, None, ctypes.byref(h)) == tq.TQ_ERR_INVALID_ARG
    assert lib.tq_quantizer_create(128, 3, tq.TQ_PROD, pi.ctypes.data, None, ctypes.byref(h)) == tq.TQ_ERR_INVALID_ARG
    assert lib.tq_quantizer_create(128, 3, 7, pi.ctypes.data, None, ctypes.byref(h)) == tq.TQ_ERR_INVALID_ARG
    assert lib.tq_quantizer_create(128, 3, tq.TQ_MSE, pi.ctypes.data, None, None) == tq.TQ_ERR_INVALID_ARG
    bad = np.eye(128); bad[0, 1] = 0.5
    assert lib.tq_quantizer_create(128, 3, tq.TQ_MSE, bad.ctypes.data, None, ctypes.byref(h)) == tq.TQ_ERR_INVALID_ARG
    assert b"orthogonal" in lib.tq_last_error_message()
    nanpi = np.eye(128); nanpi[3, 3] = np.nan
    assert lib.tq_quantizer_create(128, 3, tq.TQ_MSE, nanpi.ctypes.data, None, ctypes.byref(h)) == tq.TQ_ERR_INVALID_ARG
    c = np.zeros(256, np.float32)
    assert lib.tq_codebook_build(2, 2, c.ctypes.data, None, None) == tq.TQ_ERR_INVALID_ARG
    assert lib.tq_codebook_build(128, 9, c.ctypes.data, None, None) == tq.TQ_ERR_INVALID_ARG
    assert lib.tq_codebook_build(128, 2, None, None, None) == tq.TQ_ERR_INVALID_ARG
    assert lib.tq_quantize(None, 1, 10, None, 1, 0, None, None, None, None, None, None, None) == tq.TQ_ERR_INVALID_ARG
    arr = (ctypes.c_void_p * 1)(None)
    assert lib.tq_quantize(arr, 1, 10, None, 1, 0, None, None, None, None, None, None, None) == tq.TQ_ERR_INVALID_ARG
    assert lib.tq_quantize(arr, 0, 10, None, 1, 0, None, None, None, None, None, None, None) == tq.TQ_ERR_INVALID_ARG
    assert lib.tq_quantizer_destroy(None) == tq.TQ_ERR_INVALID_ARG
    assert lib.tq_dequantize(None, 0, None, None, None, None, 1, None, None) == tq.TQ_ERR_INVALID_ARG
    assert lib.tq_inner_products(None, None, 1, None, None, None, None, 1, None, None) == tq.TQ_ERR_INVALID_ARG
    nb = ctypes.c_size_t(0)
    assert lib.tq_decode_workspace_size(None, None, None, ctypes.byref(nb)) == tq.TQ_ERR_INVALID_ARG
    shape = tq.AttnShape(1, 8, 1, 128, 100)  # max_ctx not a multiple of 32
    kv = tq.PackedKV(None, None, None, None, None)
    assert lib.tq_decode_workspace_size(ctypes.byref(shape), ctypes.byref(kv), ctypes.byref(kv),
                                        ctypes.byref(nb)) == tq.TQ_ERR_INVALID_ARG
    shape = tq.AttnShape(1, 12, 8, 128, 128)  # 12 % 8 != 0
    assert lib.tq_decode_workspace_size(ctypes.byref(shape), ctypes.byref(kv), ctypes.byref(kv),
                                        ctypes.byref(nb)) == tq.TQ_ERR_INVALID_ARG
    assert lib.tq_decode_attention(None, None, None, None, None, ctypes.c_float(1.0), None, None, None, 0,
                                   None) == tq.TQ_ERR_INVALID_ARG
    assert lib.tq_status_string(tq.TQ_ERR_WORKSPACE) == b"workspace too small"


def test_wht_argument_errors(lib):
    h = ctypes.c_void_p()
    ok = np.ones(128)
    assert lib.tq_quantizer_create_wht(128, 3, tq.TQ_MSE, None, None, ctypes.byref(h)) == tq.TQ_ERR_INVALID_ARG
    assert lib.tq_quantizer_create_wht(128, 3, tq.TQ_MSE, ok.ctypes.data, None, None) == tq.TQ_ERR_INVALID_ARG
    assert lib.tq_quantizer_create_wht(96, 3, tq.TQ_MSE, ok.ctypes.data, None, ctypes.byref(h)) == tq.TQ_ERR_UNSUPPORTED
    bad = np.ones(128)
    bad[5] = 0.5
    assert lib.tq_quantizer_create_wht(128, 3, tq.TQ_MSE, bad.ctypes.data, None, ctypes.byref(h)) == tq.TQ_ERR_INVALID_ARG
    assert b"signs[5]" in lib.tq_last_error_message()
    # the rotation it builds is checked by the dense constructor: prod without s is refused there
    assert lib.tq_quantizer_create_wht(128, 3, tq.TQ_PROD, ok.ctypes.data, None, ctypes.byref(h)) == tq.TQ_ERR_INVALID_ARG


def test_append_argument_errors(lib):
    assert lib.tq_decode_append_attention(None, None, None, None, 1, None, None, None, ctypes.c_float(1.0), None,
                                          None, None, 0, None) == tq.TQ_ERR_INVALID_ARG
    nb = ctypes.c_size_t(0)
    shape = tq.AttnShape(1, 8, 1, 128, 100)
    kv = tq.PackedKV(None, None, None, None, None)
    assert lib.tq_decode_append_workspace_size(ctypes.byref(shape), ctypes.byref(kv), ctypes.byref(kv),
                                               ctypes.byref(nb)) == tq.TQ_ERR_INVALID_ARG


def test_search_argument_errors(lib):
    nb = ctypes.c_size_t(0)
    assert lib.tq_search_workspace_size(None, 8, ctypes.byref(nb)) == tq.TQ_ERR_INVALID_ARG
    assert lib.tq_search_scores(None, None, 1, None, None, None, None, 1, None, None, 0, None) == tq.TQ_ERR_INVALID_ARG


def test_split_argument_errors(lib):
    ch = (ctypes.c_int32 * 4)(0, 1, 2, 3)
    assert lib.tq_quantize_split(None, 1, 1, ch, 4, None, 0, 1, 0, None, None) == tq.TQ_ERR_INVALID_ARG
    assert lib.tq_inner_products_split(None, 1, ch, 4, None, 1, None, 1, None, None) == tq.TQ_ERR_INVALID_ARG


def test_split_decode_argument_errors(lib):
    """Shape and cache-description checks of the split decode run before any
    device work: NULL shape, empty or oversize shapes, NULL cache descriptions."""
    nb = ctypes.c_size_t(0)
    empty = tq.SplitCache(0, None, None, None)
    ok_shape = tq.AttnShape(1, 8, 1, 128, 64)
    assert lib.tq_decode_split_workspace_size(None, ctypes.byref(empty), ctypes.byref(empty),
                                              ctypes.byref(nb)) == tq.TQ_ERR_INVALID_ARG
    assert lib.tq_decode_split_workspace_size(ctypes.byref(ok_shape), ctypes.byref(empty), ctypes.byref(empty),
                                              None) == tq.TQ_ERR_INVALID_ARG
    for shape, err in ((tq.AttnShape(0, 8, 1, 128, 64), tq.TQ_ERR_INVALID_ARG),     # empty batch
                       (tq.AttnShape(1, 18, 9, 128, 64), tq.TQ_ERR_UNSUPPORTED),    # more than 8 KV heads
                       (tq.AttnShape(1, 18, 1, 128, 64), tq.TQ_ERR_UNSUPPORTED),    # 18 query heads per KV head
                       (tq.AttnShape(1, 12, 8, 128, 64), tq.TQ_ERR_UNSUPPORTED),    # heads do not divide
                       (tq.AttnShape(1, 8, 1, 512, 64), tq.TQ_ERR_UNSUPPORTED),     # head_dim above 256
                       (tq.AttnShape(1, 8, 1, 128, 1 << 32), tq.TQ_ERR_UNSUPPORTED),
                       (tq.AttnShape(1, 8, 1, 128, 100), tq.TQ_ERR_INVALID_ARG),    # value blocks need max_ctx % 32 == 0
                       (ok_shape, tq.TQ_ERR_INVALID_ARG)):                          # NULL cache description
        assert lib.tq_decode_split_workspace_size(ctypes.byref(shape), ctypes.byref(empty), ctypes.byref(empty),
                                                  ctypes.byref(nb)) == err, (shape.n_q_heads, shape.n_kv_heads)
        assert lib.tq_decode_attention_split(ctypes.byref(shape), None, ctypes.byref(empty), ctypes.byref(empty),
                                             None, ctypes.c_float(1.0), None, None, 0, None) == err


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("bits", [3, 4])
def test_magnitude_search_rule(lib, d, bits):
    # The quantize kernels find the nearest centroid of 3- and 4-plane codebooks
    # from the magnitude (the codebook is symmetric, its middle threshold 0):
    # key(y) = 2 bits(|y|) + [y <= 0] as uint32 against TK_j = 2 bits(t_u) + [the
    # midpoint of centroids u, u + 1 is not a float32] for the upper thresholds
    # u = K/2 + j; with J the number of keys passed, idx = K/2 - 1 - J for y <= 0
    # and K/2 + J otherwise. That rule must be the argmin with ties low for every
    # float32, in particular on and next to each threshold, on both sides, and on
    # midpoints that are float32 (d = 128, b = 3 has one).
    c, t, _ = tq.codebook_build(d, bits)
    K = 1 << bits
    assert np.array_equal(c[::-1], -c) and t[K // 2 - 1] == 0.0
    up = np.arange(K // 2, K - 1)
    mids = (c[up].astype(np.float64) + c[up + 1].astype(np.float64)) / 2
    exact = mids.astype(np.float32).astype(np.float64) == mids
    tk = 2 * t[up].view(np.uint32).astype(np.uint64) + (~exact).astype(np.uint64)
    near = [t, mids.astype(np.float32)]
    above, below = t.copy(), t.copy()
    for _ in range(3):  # one to three float32 steps either side of every threshold
        above = np.nextafter(above, np.float32(np.inf))
        below = np.nextafter(below, np.float32(-np.inf))
        near += [above, below]
    g = np.random.Generator(np.random.PCG64(3))
    y = np.concatenate(near + [(g.standard_normal(100000) / math.sqrt(d)).astype(np.float32),
                               np.array([0.0, -0.0, 1e-30, -1e-30, 2.0, -2.0], np.float32)])
    y = np.concatenate([y, -y]).astype(np.float32)
    neg = y <= 0
    key = (2 * y.view(np.uint32).astype(np.uint64)) % (1 << 32) + neg
    J = np.sum(key[:, None] > tk[None, :], axis=1)
    idx = np.where(neg, K // 2 - 1 - J, K // 2 + J)
    assert np.array_equal(idx, O.nearest_index(y.astype(np.float64), c.astype(np.float64)))


def test_quantize_kv_argument_errors(lib):
    arr = (ctypes.c_void_p * 1)(None)
    assert lib.tq_quantize_kv(None, None, 1, 32, None, None, tq.TQ_BF16, None, None, None, None, None, None,
                              None) == tq.TQ_ERR_INVALID_ARG
    assert lib.tq_quantize_kv(arr, arr, 1, 32, None, None, tq.TQ_BF16, None, None, None, None, None, None,
                              None) == tq.TQ_ERR_INVALID_ARG
