"""Shared helpers for the GPU parity tests: quantizers from seeded matrices,
caches packed by the oracle, and comparisons in the documented tolerances."""
import math

import numpy as np

import oracle as O
import tq_synth as syn

RTOL, ATOL = 1e-3, 1e-4          # scores and attention outputs
TIE_BAND = 1e-5                   # codes may flip only this close to a threshold
MAX_FLIP_RATE = 1e-4


def matrices(d, config, tensor, head, prod):
    Pi = syn.rotation(d, config, tensor, head)
    S = syn.gaussian_matrix(d, config, tensor, head) if prod else None
    return Pi, S


def quantizer(tq, d, bits, variant, config, tensor, head):
    Pi, S = matrices(d, config, tensor, head, variant == "prod")
    return tq.Quantizer(d, bits, variant, Pi, S), Pi, S


def oracle_cache_slice(x, d, bits, variant, Pi, S, layout):
    """Quantize float vectors x [T, d] with the oracle; return numpy arrays in the
    library's layouts plus the dequantized vectors."""
    planes = bits - 1 if variant == "prod" else bits
    cb = O.codebook(d, planes)
    if variant == "prod":
        r = O.quantize_prod(x, Pi, S, cb)
        xt = O.dequantize_prod(r["idx"], r["signs"], r["norms"], r["rnorms"], Pi, S, cb)
    else:
        r = O.quantize_mse(x, Pi, cb)
        xt = O.dequantize_mse(r["idx"], r["norms"], Pi, cb)
    out = {"norms": r["norms"], "xt": xt, "idx": r["idx"]}
    if planes > 0:
        out["codes"] = (O.pack_block_layout(r["idx"], planes) if layout == "block32"
                        else O.pack_vector_layout(r["idx"], planes))
    if variant == "prod":
        out["signs"] = O.pack_bits(r["signs"])
        out["rnorms"] = r["rnorms"]
    return out


def allclose_report(got, want, rtol=RTOL, atol=ATOL):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    err = np.abs(got - want)
    bad = err > atol + rtol * np.abs(want)
    return int(bad.sum()), float(err.max()) if err.size else 0.0


def assert_scores_close(got, want, y, xt, rtol=RTOL, atol=ATOL):
    """Inner products against the oracle, element by element:
        |got_ij - want_ij| <= atol * sigma_ij + rtol * |want_ij|,
    sigma_ij = |y_i| |xt_j| / sqrt(d), the spread of <y_i, x> over directions of
    x. The score tolerance (rel 1e-3 / abs 1e-4) is stated for attention scores,
    which the 1/sqrt(d) scaling of unit-variance vectors brings to unit spread;
    for raw inner products of any scale its absolute part is read in those units
    (fp32 rounding grows with |y| |x|, so no fixed absolute bar fits every scale)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    xt = np.asarray(xt, dtype=np.float64)
    sigma = np.linalg.norm(y, axis=1)[:, None] * np.linalg.norm(xt, axis=1)[None, :] / math.sqrt(y.shape[1])
    err = np.abs(got - want)
    bar = atol * sigma + rtol * np.abs(want)
    bad = err > bar
    worst = float(np.max(err / np.where(bar > 0, bar, 1.0))) if err.size else 0.0
    assert not bad.any(), f"{int(bad.sum())} of {err.size} scores outside the bar (worst err/bar {worst:.3g})"
    return worst


def near_threshold(y, centroids, band=TIE_BAND):
    mids = (centroids[:-1] + centroids[1:]) / 2
    if mids.size == 0:
        return np.zeros_like(y, dtype=bool)
    return np.min(np.abs(np.asarray(y)[..., None] - mids), axis=-1) <= band


def ulp_diff_f32(a, b):
    a = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(a - b)
