"""fp64 oracle: plain definitions of every step of the quantize / decode path.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by tests,
``__graft_entry__.smoke()`` and bench.py's cpu_baseline leg, never by the
library.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
from scipy import special

__all__ = [
    "coord_density", "cell_mass", "cell_first_moment", "lloyd_max", "codebook",
    "nearest_index", "quantize_mse", "quantize_prod", "dequantize_mse", "dequantize_prod",
    "qjl", "qjl_inverse", "pack_vector_layout", "unpack_vector_layout", "pack_bits",
    "unpack_bits", "pack_block_layout", "unpack_block_layout", "attention",
    "decode_attention", "inner_products", "QJL_SCALE", "hadamard", "wht_rotation",
    "quantize_split", "dequantize_split", "decode_attention_split",
]


# ---------------------------------------------------------------------------
# Coordinate density of a uniform point on S^{d-1}
# [NIK] "Step 1: random rotation", Lemma (distribution of coordinates on the
# sphere): f_X(x) = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)) (1 - x^2)^((d-3)/2).
# ---------------------------------------------------------------------------

def _norm_const(d: int) -> float:
    return math.exp(math.lgamma(d / 2.0) - math.lgamma((d - 1) / 2.0)) / math.sqrt(math.pi)


def coord_density(d: int, x):
    x = np.asarray(x, dtype=np.float64)
    k = (d - 3) / 2.0
    inside = np.abs(x) <= 1.0
    base = np.where(inside, 1.0 - x * x, 0.0)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = _norm_const(d) * np.power(base, k)
    return np.where(inside, v, 0.0)


def cell_mass(d: int, a, b):
    """P(a < X <= b) for X ~ f_X. With x = 2t - 1, f_X is the Beta((d-1)/2, (d-1)/2)
    law of t, so the mass is a difference of regularized incomplete Beta values
    (library special function)."""
    k1 = (d - 1) / 2.0
    a = np.clip(np.asarray(a, dtype=np.float64), -1.0, 1.0)
    b = np.clip(np.asarray(b, dtype=np.float64), -1.0, 1.0)
    return special.betainc(k1, k1, (1.0 + b) / 2.0) - special.betainc(k1, k1, (1.0 + a) / 2.0)


def cell_first_moment(d: int, a, b):
    """int_a^b x f_X(x) dx in closed form:
    C_d [(1 - a^2)^(k+1) - (1 - b^2)^(k+1)] / (2 (k + 1)),  k = (d - 3) / 2."""
    k = (d - 3) / 2.0
    a = np.clip(np.asarray(a, dtype=np.float64), -1.0, 1.0)
    b = np.clip(np.asarray(b, dtype=np.float64), -1.0, 1.0)
    return _norm_const(d) * (np.power(1.0 - a * a, k + 1) - np.power(1.0 - b * b, k + 1)) / (2.0 * (k + 1))


# ---------------------------------------------------------------------------
# Lloyd-Max scalar quantizer for f_X
# [NIK] "Step 2: optimal scalar quantization (Lloyd-Max)": minimize
# C(f_X, b) = sum_i int_{cell_i} (x - c_i)^2 f_X(x) dx over 2^b ordered centroids;
# the optimum has cell boundaries at midpoints of neighbouring centroids and each
# centroid at the conditional mean of its cell; Lloyd-Max alternates the two.
# ---------------------------------------------------------------------------

def lloyd_max(d: int, bits: int, tol: float = 1e-15, max_iter: int = 200000):
    """Return (centroids float64 ascending, cost C(f_X, b), iterations)."""
    if d < 3:
        raise ValueError("d >= 3 required")
    K = 1 << bits
    if K == 1:
        return np.zeros(1), 1.0 / d, 0
    k1 = (d - 1) / 2.0
    # start at the quantiles (i + 1/2)/K of f_X
    q = (np.arange(K) + 0.5) / K
    c = 2.0 * special.betaincinv(k1, k1, q) - 1.0
    it = 0
    for it in range(1, max_iter + 1):
        t = 0.5 * (c[:-1] + c[1:])                       # thresholds = midpoints
        lo = np.concatenate(([-1.0], t))
        hi = np.concatenate((t, [1.0]))
        mass = cell_mass(d, lo, hi)
        c_new = cell_first_moment(d, lo, hi) / mass      # centroids = conditional means
        delta = np.max(np.abs(c_new - c))
        c = c_new
        if delta < tol:
            break
    t = 0.5 * (c[:-1] + c[1:])
    lo = np.concatenate(([-1.0], t))
    hi = np.concatenate((t, [1.0]))
    mass = cell_mass(d, lo, hi)
    # at the fixed point int_cell x f = c_i P_i, so sum_i int (x - c_i)^2 f = E[X^2] - sum c_i^2 P_i,
    # and E[X^2] = 1/d for a coordinate of a unit vector.
    cost = 1.0 / d - float(np.sum(c * c * mass))
    return c, cost, it


_CODEBOOK_CACHE: dict = {}


def codebook(d: int, bits: int) -> np.ndarray:
    """The stored codebook: Lloyd-Max centroids rounded to float32 (returned as float64)."""
    key = (d, bits)
    if key not in _CODEBOOK_CACHE:
        c, _, _ = lloyd_max(d, bits)
        _CODEBOOK_CACHE[key] = c.astype(np.float32).astype(np.float64)
    return _CODEBOOK_CACHE[key].copy()


def nearest_index(y, centroids) -> np.ndarray:
    """[NIK] "Step 2": for every coordinate, the index of the nearest centroid.
    Ties go to the lower index. Distances are compared exactly: where the fp64
    distances of the two best candidates are within rounding of each other,
    they are recomputed in rational arithmetic."""
    y = np.asarray(y, dtype=np.float64)
    c = np.asarray(centroids, dtype=np.float64)
    out = np.empty(y.shape, dtype=np.int64)
    flat_y = y.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 20
    for s in range(0, flat_y.size, step):
        ys = flat_y[s:s + step]
        dist = np.abs(ys[:, None] - c[None, :])
        best = np.argmin(dist, axis=1)
        flat_o[s:s + step] = best
        if c.size > 1:
            part = np.partition(dist, 1, axis=1)
            near = np.nonzero(part[:, 1] - part[:, 0] <= 1e-12 * (np.abs(ys) + np.max(np.abs(c))))[0]
            for i in near:
                yi = Fraction(float(ys[i]))
                exact = [abs(yi - Fraction(float(ci))) for ci in c]
                flat_o[s + i] = min(range(c.size), key=lambda k: (exact[k], k))
    return out


# ---------------------------------------------------------------------------
# Randomized Walsh-Hadamard rotation: [NIK] "What the community did", item 3
# (a Walsh-Hadamard transform for the MSE stage, with a random transform for
# QJL drawn independently). Pi = H D / sqrt(d), H the Sylvester-Hadamard
# matrix of order d (a power of two), D a random +-1 diagonal.
# ---------------------------------------------------------------------------

def hadamard(d: int) -> np.ndarray:
    """Sylvester-Hadamard matrix, closed form H[i, j] = (-1)^popcount(i & j)."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    i = np.arange(d)
    parity = np.zeros((d, d), dtype=np.int64)
    m = i[:, None] & i[None, :]
    while np.any(m):
        parity ^= m & 1
        m = m >> 1
    return np.where(parity == 1, -1.0, 1.0)


def wht_rotation(signs) -> np.ndarray:
    """Pi = H diag(signs) / sqrt(d): orthogonal, y = Pi u."""
    signs = np.asarray(signs, dtype=np.float64)
    d = signs.size
    return hadamard(d) * signs[None, :] / math.sqrt(d)


# ---------------------------------------------------------------------------
# TurboQuant_mse: [NIK] "Step 0: normalization", "Step 1", "Step 2"
# ---------------------------------------------------------------------------

def _normalize(x):
    x = np.asarray(x, dtype=np.float64)
    nu = np.sqrt(np.sum(x * x, axis=1))
    safe = np.where(nu > 0, nu, 1.0)
    u = x / safe[:, None]
    u[nu == 0] = 0.0
    return nu, u


def quantize_mse(x, Pi, centroids):
    """Q_mse. Returns dict(idx [n,d] int, norms float32 [n], y fp64 [n,d]).

    nu = |x|_2 stored as float32; u = x / nu; y = Pi u; idx_j = nearest centroid of y_j.
    A zero vector gets idx = 0 everywhere (all code bits zero)."""
    nu, u = _normalize(x)
    y = u @ np.asarray(Pi, dtype=np.float64).T
    idx = nearest_index(y, centroids)
    idx[nu == 0] = 0
    return {"idx": idx, "norms": nu.astype(np.float32), "y": y, "nu": nu}


def dequantize_mse(idx, norms, Pi, centroids):
    """Q_mse^{-1}: x~ = nu * Pi^T c[idx]  ([NIK] "Step 2", last paragraph)."""
    c = np.asarray(centroids, dtype=np.float64)
    yt = c[np.asarray(idx)]
    return np.asarray(norms, dtype=np.float64)[:, None] * (yt @ np.asarray(Pi, dtype=np.float64))


# ---------------------------------------------------------------------------
# QJL: [NIK] "QJL: a one-bit method":
#   Q_qjl(x) = sign(S x),  Q_qjl^{-1}(z) = sqrt(pi/2) / d * S^T z
# ---------------------------------------------------------------------------

def QJL_SCALE(d: int) -> float:
    return math.sqrt(math.pi / 2.0) / d


def qjl(x, S):
    """sign(S x) as booleans (True = +1); sign(0) = +1."""
    p = np.asarray(x, dtype=np.float64) @ np.asarray(S, dtype=np.float64).T
    return p >= 0.0


def qjl_inverse(z, S):
    d = np.asarray(S).shape[1]
    zpm = np.where(np.asarray(z), 1.0, -1.0)
    return QJL_SCALE(d) * (zpm @ np.asarray(S, dtype=np.float64))


# ---------------------------------------------------------------------------
# TurboQuant_prod: [NIK] "TurboQuant proper" and Theorem 2:
#   1) Q_mse with b-1 bits, 2) r = u - Q_mse^{-1}(Q_mse(u)),
#   3) store sign(S r) and |r|_2, 4) dequantize as the sum of both parts.
# ---------------------------------------------------------------------------

def quantize_prod(x, Pi, S, centroids_bm1):
    """Q_prod on x (normalized first). centroids_bm1 is the (b-1)-bit codebook
    ({0} when b = 1). Returns idx, signs (bool), norms, rnorms (float32), y, p."""
    nu, u = _normalize(x)
    Pi = np.asarray(Pi, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    c = np.asarray(centroids_bm1, dtype=np.float64)
    y = u @ Pi.T
    idx = nearest_index(y, c)
    idx[nu == 0] = 0
    r = u - c[idx] @ Pi
    r[nu == 0] = 0.0
    gamma = np.sqrt(np.sum(r * r, axis=1))
    p = r @ S.T
    signs = p >= 0.0
    signs[nu == 0] = False
    return {"idx": idx, "signs": signs, "norms": nu.astype(np.float32),
            "rnorms": gamma.astype(np.float32), "y": y, "p": p, "nu": nu, "gamma": gamma}


def dequantize_prod(idx, signs, norms, rnorms, Pi, S, centroids_bm1):
    """x~ = nu * (Pi^T c[idx] + |r| * sqrt(pi/2)/d * S^T z)."""
    Pi = np.asarray(Pi, dtype=np.float64)
    c = np.asarray(centroids_bm1, dtype=np.float64)
    x_mse = c[np.asarray(idx)] @ Pi
    x_qjl = np.asarray(rnorms, dtype=np.float64)[:, None] * qjl_inverse(signs, S)
    return np.asarray(norms, dtype=np.float64)[:, None] * (x_mse + x_qjl)


def inner_products(yq, x_tilde):
    """<y_i, x~_j> for every query i and vector j."""
    return np.asarray(yq, dtype=np.float64) @ np.asarray(x_tilde, dtype=np.float64).T


# ---------------------------------------------------------------------------
# Outlier-channel split: [NIK] "Experiments" (KV cache): outlier channels and
# the other channels go through separate TurboQuant instances with different
# bit widths. Part p takes the sub-vector x[:, channels_p] and is plain
# TurboQuant in d_p = len(channels_p) dimensions, with its own rotation, norm,
# codebook and (prod) QJL matrix. A part is a dict with keys "channels",
# "variant" ("mse" or "prod"), "Pi", "S" (prod) and "centroids" (the d_p-dim
# codebook of b_p bits for mse, b_p - 1 bits for prod).
# ---------------------------------------------------------------------------

def quantize_split(x, parts):
    """Per-part results of quantize_mse / quantize_prod on x[:, channels_p]."""
    x = np.asarray(x, dtype=np.float64)
    res = []
    for p in parts:
        sub = x[:, np.asarray(p["channels"], dtype=np.int64)]
        if p["variant"] == "prod":
            res.append(quantize_prod(sub, p["Pi"], p["S"], p["centroids"]))
        else:
            res.append(quantize_mse(sub, p["Pi"], p["centroids"]))
    return res


def dequantize_split(results, parts, dim: int):
    """x~ [n, dim]: each part's dequantized sub-vector at its channels, 0 at channels no part keeps."""
    n = len(results[0]["norms"])
    xt = np.zeros((n, dim))
    for r, p in zip(results, parts):
        if p["variant"] == "prod":
            sub = dequantize_prod(r["idx"], r["signs"], r["norms"], r["rnorms"], p["Pi"], p["S"], p["centroids"])
        else:
            sub = dequantize_mse(r["idx"], r["norms"], p["Pi"], p["centroids"])
        xt[:, np.asarray(p["channels"], dtype=np.int64)] = sub
    return xt


def decode_attention_split(q, keys, values, ctx_lens, scale, dim: int):
    """Decode attention over split caches: keys[b][g] and values[b][g] are
    (per-part results over the cached tokens, parts) as quantize_split returns
    them for KV head g of batch b. Every query head h of KV head g = h // (Hq/Hkv)
    attends the first ctx_lens[b] tokens of the dequantized caches (channels no
    part keeps are 0); an empty context gives 0."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, _ = q.shape
    Hkv = len(keys[0])
    G = Hq // Hkv
    out = np.zeros((B, Hq, dim))
    for b in range(B):
        n = int(ctx_lens[b])
        if n == 0:
            continue
        for g in range(Hkv):
            K = dequantize_split(*keys[b][g], dim)[:n]
            V = dequantize_split(*values[b][g], dim)[:n]
            for h in range(G):
                out[b, g * G + h] = attention(q[b, g * G + h], K, V, scale)[0]
    return out


# ---------------------------------------------------------------------------
# Bit layouts (the library's documented contract, re-implemented here).
#
# Vector layout: for each vector, `bits` planes of d bits; plane p holds bit p
# of every index; coordinate j of plane p sits at byte p*d/8 + j/8, bit j%8.
#
# Block layout (32 vectors per block, used for the value cache): for plane p,
# group g in 0..3 and word w in 0..d/4-1, a little-endian 32-bit word at byte
# offset ((p*4 + g) * d/4 + w) * 4 inside the block; bit 4r+k (r, k in 0..3)
# is plane-p bit of coordinate 4w+r of vector 4g+k of the block, and bit
# 16+4r+k the same for vector 16+4g+k. A block is 4*bits*d bytes.
# ---------------------------------------------------------------------------

def pack_vector_layout(idx, bits: int) -> np.ndarray:
    idx = np.asarray(idx, dtype=np.int64)
    n, d = idx.shape
    out = np.zeros((n, bits, d // 8), dtype=np.uint8)
    for p in range(bits):
        bitp = ((idx >> p) & 1).astype(np.uint8)
        for i in range(8):
            out[:, p, :] |= bitp[:, i::8] << i
    return out.reshape(n, bits * d // 8)


def unpack_vector_layout(codes, bits: int, d: int) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8).reshape(-1, bits, d // 8)
    n = codes.shape[0]
    idx = np.zeros((n, d), dtype=np.int64)
    for p in range(bits):
        for i in range(8):
            idx[:, i::8] |= ((codes[:, p, :] >> i) & 1).astype(np.int64) << p
    return idx


def pack_bits(flags) -> np.ndarray:
    """Boolean [n, d] -> [n, d/8] bytes, coordinate j at byte j/8 bit j%8."""
    return pack_vector_layout(np.asarray(flags).astype(np.int64), 1)


def unpack_bits(packed, d: int) -> np.ndarray:
    return unpack_vector_layout(packed, 1, d).astype(bool)


def pack_block_layout(idx, bits: int) -> np.ndarray:
    idx = np.asarray(idx, dtype=np.int64)
    n, d = idx.shape
    if n % 32 or d % 4:
        raise ValueError("block layout needs n % 32 == 0 and d % 4 == 0")
    nb = n // 32
    blk = idx.reshape(nb, 32, d)
    words = np.zeros((nb, bits, 4, d // 4), dtype=np.uint64)
    for p in range(bits):
        bitp = ((blk >> p) & 1).astype(np.uint64)
        for g in range(4):
            for r in range(4):
                for k in range(4):
                    words[:, p, g, :] |= bitp[:, 4 * g + k, r::4] << np.uint64(4 * r + k)
                    words[:, p, g, :] |= bitp[:, 16 + 4 * g + k, r::4] << np.uint64(16 + 4 * r + k)
    return words.astype("<u4").view(np.uint8).reshape(nb, 4 * bits * d)


def unpack_block_layout(codes, bits: int, d: int) -> np.ndarray:
    codes = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    nb = codes.size // (4 * bits * d)
    words = codes.reshape(-1).view("<u4").reshape(nb, bits, 4, d // 4).astype(np.uint64)
    idx = np.zeros((nb, 32, d), dtype=np.int64)
    for p in range(bits):
        for g in range(4):
            for r in range(4):
                for k in range(4):
                    b_lo = (words[:, p, g, :] >> np.uint64(4 * r + k)) & np.uint64(1)
                    b_hi = (words[:, p, g, :] >> np.uint64(16 + 4 * r + k)) & np.uint64(1)
                    idx[:, 4 * g + k, r::4] |= b_lo.astype(np.int64) << p
                    idx[:, 16 + 4 * g + k, r::4] |= b_hi.astype(np.int64) << p
    return idx.reshape(nb * 32, d)


# ---------------------------------------------------------------------------
# Attention for one decode token ([NIK] problem statement: the query is compared
# with all previous keys, values are weighted by the resulting scores; [NAH]:
# the full prod variant needs its own attention kernel over the packed cache).
# ---------------------------------------------------------------------------

def attention(q, K, V, scale: float):
    """softmax(scale * K q) V for one query vector; K, V are [T, d] (T >= 1)."""
    s = scale * (np.asarray(K, dtype=np.float64) @ np.asarray(q, dtype=np.float64))
    s = s - np.max(s)
    w = np.exp(s)
    return (w @ np.asarray(V, dtype=np.float64)) / np.sum(w), s


def decode_attention(q, kcache, vcache, ctx_lens, scale, *, return_scores=False):
    """Decode attention over a packed KV cache, computed by dequantizing every
    key and value in full and running plain softmax attention per query head.

    q: [B, Hq, d] float.  kcache / vcache: dicts with
       'variant' ('mse' | 'prod'), 'bits', 'd', 'max_ctx',
       'codes'  (K: [B, Hkv, T, planes*d/8] vector layout;
                 V: [B, Hkv, T/32, 4*bits*d] block layout),
       'signs' [B, Hkv, T, d/8] (prod keys), 'norms', 'rnorms' [B, Hkv, T],
       'Pi' [Hkv, d, d], 'S' [Hkv, d, d] (prod keys).
    GQA: query head h reads key/value head floor(h * Hkv / Hq).
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = kcache["norms"].shape[1]
    out = np.zeros((B, Hq, d))
    scores = {}
    kv_bits_k = kcache["bits"] - (1 if kcache["variant"] == "prod" else 0)
    ck = codebook(d, kv_bits_k)
    cv = codebook(d, vcache["bits"])
    for b in range(B):
        T = int(ctx_lens[b])
        if T == 0:
            continue  # no cached token: no attention mass, the output is defined as 0
        for h in range(Hkv):
            Kt = _dequant_k(kcache, b, h, T, ck)
            Vt = _dequant_v(vcache, b, h, T, cv)
            for hq in range(Hq):
                if (hq * Hkv) // Hq != h:
                    continue
                o, s = attention(q[b, hq], Kt, Vt, scale)
                out[b, hq] = o
                if return_scores:
                    scores[(b, hq)] = s + 0.0
    if return_scores:
        return out, scores
    return out


def _dequant_k(kc, b, h, T, ck):
    d = kc["d"]
    planes = kc["bits"] - (1 if kc["variant"] == "prod" else 0)
    if planes > 0:
        idx = unpack_vector_layout(kc["codes"][b, h, :T], planes, d)
    else:
        idx = np.zeros((T, d), dtype=np.int64)
    if kc["variant"] == "prod":
        z = unpack_bits(kc["signs"][b, h, :T], d)
        return dequantize_prod(idx, z, kc["norms"][b, h, :T], kc["rnorms"][b, h, :T],
                               kc["Pi"][h], kc["S"][h], ck)
    return dequantize_mse(idx, kc["norms"][b, h, :T], kc["Pi"][h], ck)


def _dequant_v(vc, b, h, T, cv):
    d = vc["d"]
    nblk = (T + 31) // 32
    idx = unpack_block_layout(vc["codes"][b, h, :nblk], vc["bits"], d)[:T]
    return dequantize_mse(idx, vc["norms"][b, h, :T], vc["Pi"][h], cv)
