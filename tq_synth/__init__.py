"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module draws random numbers and arranges them into the shapes of the
workloads; it holds none of the quantizer's or the attention's arithmetic.
Everything is numpy PCG64 keyed by a SeedSequence of
``[20260401, config, role, tensor, batch, head]`` so that any slice of a large
workload can be regenerated on its own.

Random draws that the method itself makes are produced here and passed to both
sides as plain inputs:
  * the rotation matrix Pi: a Haar-random orthogonal matrix, taken as the Q
    factor of a QR decomposition of an i.i.d. Gaussian matrix with the signs of
    R's diagonal folded into Q (the page "Eternal mathematics of TurboQuant",
    section "Step 1: random rotation");
  * the QJL matrix S: i.i.d. N(0, 1) entries, drawn from a seed stream that is
    independent of Pi's (same page, sections "QJL" and the community note on
    independent transforms).
"""
from __future__ import annotations

import numpy as np

ROOT_SEED = 20260401

# roles
ROLE_PI, ROLE_S, ROLE_DATA, ROLE_QUERY, ROLE_OUTLIER, ROLE_SCALE, ROLE_CTX, ROLE_PACKED, ROLE_WHT = (
    0, 1, 2, 3, 4, 5, 6, 7, 8)
# tensors
T_K, T_V, T_Q = 0, 1, 2

# workload identifiers (used only as seed components)
CFG_SMALL_KEYS = 1       # 4096 fp32 keys, d=128, mse b=2
CFG_LAYER_QUANT = 2      # one layer's KV: 8 heads x 32768 tokens, bf16
CFG_DECODE_128K = 3      # decode, B=8, 64/8 heads, ctx 131072
CFG_SWEEP = 4            # b / d sweep, B=4, 8 kv heads, ctx 16384
CFG_DECODE_1M = 5        # decode, B=1, 64/8 heads, ctx 1,048,576
CFG_TEST = 9             # small ad-hoc test shapes


def rng(config: int, role: int, tensor: int = 0, batch: int = 0, head: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence([ROOT_SEED, int(config), int(role), int(tensor), int(batch), int(head)])
    return np.random.Generator(np.random.PCG64(ss))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return r.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 values that are already bf16-exact -> their uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def rotation(d: int, config: int, tensor: int = 0, head: int = 0) -> np.ndarray:
    """Haar-random d x d orthogonal matrix in float64."""
    g = rng(config, ROLE_PI, tensor, 0, head).standard_normal((d, d))
    q, r = np.linalg.qr(g)
    s = np.sign(np.diag(r))
    s[s == 0] = 1.0
    return np.ascontiguousarray(q * s[None, :])


def wht_signs(d: int, config: int, tensor: int = 0, head: int = 0) -> np.ndarray:
    """Random +-1 diagonal of a randomized Walsh-Hadamard rotation (float64 [d]),
    from its own seed stream (independent of Pi and S)."""
    return rng(config, ROLE_WHT, tensor, 0, head).integers(0, 2, d).astype(np.float64) * 2.0 - 1.0


def gaussian_matrix(d: int, config: int, tensor: int = 0, head: int = 0) -> np.ndarray:
    """d x d matrix of i.i.d. N(0,1) entries in float64 (the QJL projection)."""
    return np.ascontiguousarray(rng(config, ROLE_S, tensor, 0, head).standard_normal((d, d)))


def outlier_channels(d: int, config: int, tensor: int, head: int, count: int = 4) -> np.ndarray:
    return np.sort(rng(config, ROLE_OUTLIER, tensor, 0, head).choice(d, size=count, replace=False))


def kv_vectors(n: int, d: int, config: int, tensor: int, batch: int, head: int, *,
               outliers: int = 4, outlier_scale: float = 10.0, lognormal_sigma: float = 0.0,
               start: int = 0) -> np.ndarray:
    """Synthetic key/value head vectors, bf16-exact float32 array [n, d].

    N(0,1) entries, ``outliers`` fixed channels per (tensor, head) scaled by
    ``outlier_scale``, and optionally a per-vector LogNormal(0, sigma) scale.
    ``start`` skips the first ``start`` vectors of the stream so a token range
    can be regenerated alone (draws are made in fixed 4096-vector chunks).
    """
    chunk = 4096
    out = np.empty((n, d), dtype=np.float32)
    ch = outlier_channels(d, config, tensor, head, outliers) if outliers else None
    first_chunk = start // chunk
    last_chunk = (start + n - 1) // chunk if n > 0 else first_chunk - 1
    pos = 0
    for c in range(first_chunk, last_chunk + 1):
        g = rng(config, ROLE_DATA, tensor, batch, head * 65536 + c)
        v = g.standard_normal((chunk, d), dtype=np.float32)
        if lognormal_sigma > 0:
            s = np.exp(lognormal_sigma * g.standard_normal(chunk)).astype(np.float32)
            v *= s[:, None]
        if ch is not None:
            v[:, ch] *= np.float32(outlier_scale)
        lo = max(start, c * chunk) - c * chunk
        hi = min(start + n, (c + 1) * chunk) - c * chunk
        out[pos:pos + hi - lo] = v[lo:hi]
        pos += hi - lo
    return bf16_round(out)


def small_keys(n: int = 4096, d: int = 128, config: int = CFG_SMALL_KEYS) -> np.ndarray:
    """fp32 keys x = s * g, g ~ N(0, I_d), s ~ LogNormal(0, 0.5) per vector."""
    g = rng(config, ROLE_DATA, T_K)
    x = g.standard_normal((n, d))
    s = np.exp(0.5 * rng(config, ROLE_SCALE, T_K).standard_normal(n))
    return (x * s[:, None]).astype(np.float32)


def gaussian_queries(m: int, d: int, config: int, batch: int = 0) -> np.ndarray:
    """m Gaussian query vectors, float32 (not rounded)."""
    return rng(config, ROLE_QUERY, T_Q, batch).standard_normal((m, d)).astype(np.float32)


def decode_queries(batch: int, n_q_heads: int, d: int, config: int) -> np.ndarray:
    """bf16-exact float32 queries [B, Hq, d] ~ N(0, 1)."""
    q = rng(config, ROLE_QUERY, T_Q).standard_normal((batch, n_q_heads, d), dtype=np.float32)
    return bf16_round(q)


def ragged_lengths(batch: int, max_ctx: int, config: int, minimum: int = 1) -> np.ndarray:
    """Context lengths in [minimum, max_ctx], int32, with the extremes included."""
    g = rng(config, ROLE_CTX)
    lens = g.integers(minimum, max_ctx + 1, size=batch)
    if batch >= 2:
        lens[0] = max_ctx
        lens[1] = minimum
    return lens.astype(np.int32)


def kv_vectors_device(G: int, n: int, d: int, config: int, tensor: int, device, *,
                      outliers: int = 4, outlier_scale: float = 10.0, lognormal_sigma: float = 0.0,
                      seed_offset: int = 0):
    """Bulk synthetic head vectors drawn on the GPU with torch's seeded generator,
    bf16 tensor [G, n, d]. Same distribution as ``kv_vectors`` (N(0,1), fixed
    outlier channels x10 per group, optional per-vector LogNormal scale) but a
    different random stream: used to fill large caches whose values are never
    compared element by element with the oracle."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(ROOT_SEED * 1000 + config * 100 + tensor * 10 + seed_offset)
    out = torch.empty((G, n, d), dtype=torch.bfloat16, device=device)
    for gi in range(G):
        v = torch.randn((n, d), generator=gen, device=device, dtype=torch.float32)
        if lognormal_sigma > 0:
            s = torch.exp(lognormal_sigma * torch.randn((n,), generator=gen, device=device))
            v *= s[:, None]
        if outliers:
            ch = torch.from_numpy(outlier_channels(d, config, tensor, gi, outliers)).to(device)
            v[:, ch] *= outlier_scale
        out[gi] = v.to(torch.bfloat16)
    return out


def random_packed_group(T: int, d: int, key_code_bytes: int, value_block_bytes: int, config: int,
                        batch: int, head: int, *, lognormal_sigma: float = 0.0, norm_base: float = 22.9):
    """Packed cache arrays of one (batch, kv head) made of seeded random bits:
    key codes [T, key_code_bytes], key sign bytes [T, d/8], value blocks
    [T/32, value_block_bytes] (uint8, uniform), key and value norms
    ``norm_base`` times a LogNormal(0, sigma) per token, residual norms uniform in
    [0.25, 0.45] (float32). Any bits form a valid packed cache; the norm scales
    follow the synthetic vectors (N(0,1) with 4 channels x10 has |x| ~ 22.9 at d=128)."""
    g = rng(config, ROLE_PACKED, 0, batch, head)
    out = {"kcodes": g.integers(0, 256, (T, key_code_bytes), dtype=np.uint8),
           "ksigns": g.integers(0, 256, (T, d // 8), dtype=np.uint8),
           "vcodes": g.integers(0, 256, (T // 32, value_block_bytes), dtype=np.uint8)}
    for k in ("knorms", "vnorms"):
        s = np.exp(lognormal_sigma * g.standard_normal(T)) if lognormal_sigma > 0 else np.ones(T)
        out[k] = (norm_base * s * (1.0 + 0.05 * g.standard_normal(T))).astype(np.float32)
    out["krnorms"] = g.uniform(0.25, 0.45, T).astype(np.float32)
    return out
