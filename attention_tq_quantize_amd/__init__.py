"""Python binding of libtq (TurboQuant quantize + quantized-KV decode attention, gfx950).

Argument marshalling only: every step of the path runs in the HIP library
behind include/tq.h. torch is used for device memory and streams. If the
shared library is missing, every call raises; there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq.so")

TQ_OK, TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_NO_MEMORY, TQ_ERR_DEVICE, TQ_ERR_WORKSPACE = range(6)
TQ_MSE, TQ_PROD = 0, 1
TQ_F32, TQ_BF16 = 0, 1
TQ_LAYOUT_VECTOR, TQ_LAYOUT_BLOCK32 = 0, 1

EXPORTS = [
    "tq_status_string", "tq_last_error_message", "tq_version", "tq_codebook_build",
    "tq_quantizer_create", "tq_quantizer_create_wht", "tq_quantizer_destroy", "tq_quantizer_info",
    "tq_quantizer_sizes", "tq_quantize",
    "tq_quantize_mse", "tq_quantize_prod", "tq_dequantize", "tq_inner_products",
    "tq_decode_workspace_size", "tq_decode_attention", "tq_decode_append_workspace_size",
    "tq_decode_append_attention", "tq_search_workspace_size", "tq_search_scores", "tq_quantize_split",
    "tq_inner_products_split", "tq_decode_split_workspace_size", "tq_decode_attention_split",
]


class TQError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: status {status} ({message})")
        self.status = status


class AttnShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int), ("n_q_heads", ctypes.c_int), ("n_kv_heads", ctypes.c_int),
                ("head_dim", ctypes.c_int), ("max_ctx", ctypes.c_int64)]


class PackedKV(ctypes.Structure):
    _fields_ = [("qz", ctypes.POINTER(ctypes.c_void_p)), ("codes", ctypes.c_void_p),
                ("signs", ctypes.c_void_p), ("norms", ctypes.c_void_p), ("rnorms", ctypes.c_void_p)]


class Records(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("signs", ctypes.c_void_p), ("norms", ctypes.c_void_p),
                ("rnorms", ctypes.c_void_p), ("rot_dbg", ctypes.c_void_p), ("proj_dbg", ctypes.c_void_p)]


class SplitCache(ctypes.Structure):
    _fields_ = [("n_parts", ctypes.c_int), ("qz", ctypes.POINTER(ctypes.c_void_p)),
                ("channels", ctypes.c_void_p), ("rec", ctypes.c_void_p)]


_lib = None

_VP, _I, _I64, _F, _D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_double


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libtq.so (built in-tree by __graft_entry__.build() or _build.py). Raises if missing."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libtq.so not found at {p}; build it first (python -m attention_tq_quantize_amd._build)")
    lib = ctypes.CDLL(p)
    lib.tq_status_string.restype = ctypes.c_char_p
    lib.tq_status_string.argtypes = [_I]
    lib.tq_last_error_message.restype = ctypes.c_char_p
    lib.tq_last_error_message.argtypes = []
    lib.tq_version.restype = _I
    lib.tq_codebook_build.argtypes = [_I, _I, _VP, _VP, _VP]
    lib.tq_quantizer_create.argtypes = [_I, _I, _I, _VP, _VP, ctypes.POINTER(_VP)]
    lib.tq_quantizer_create_wht.argtypes = [_I, _I, _I, _VP, _VP, ctypes.POINTER(_VP)]
    lib.tq_quantizer_destroy.argtypes = [_VP]
    lib.tq_quantizer_info.argtypes = [_VP, _VP, _VP, _VP, _VP]
    lib.tq_quantize.argtypes = [_VP, _I, _I64, _VP, _I, _I, _VP, _VP, _VP, _VP, _VP, _VP, _VP]
    lib.tq_quantize_mse.argtypes = [_VP, _VP, _I, _I64, _I64, _VP, _VP, _VP, _VP]
    lib.tq_quantize_prod.argtypes = [_VP, _VP, _I, _I64, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _VP]
    lib.tq_quantizer_sizes.argtypes = [_VP, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]
    lib.tq_dequantize.argtypes = [_VP, _I, _VP, _VP, _VP, _VP, _I64, _VP, _VP]
    lib.tq_inner_products.argtypes = [_VP, _VP, _I64, _VP, _VP, _VP, _VP, _I64, _VP, _VP]
    lib.tq_quantize_split.argtypes = [_VP, _I, _VP, _I, _VP, _I, _I64, ctypes.POINTER(Records), _VP]
    lib.tq_inner_products_split.argtypes = [_VP, _I, _VP, _I, _VP, _I64, ctypes.POINTER(Records), _I64, _VP, _VP]
    lib.tq_decode_split_workspace_size.argtypes = [ctypes.POINTER(AttnShape), ctypes.POINTER(SplitCache),
                                                   ctypes.POINTER(SplitCache), ctypes.POINTER(ctypes.c_size_t)]
    lib.tq_decode_attention_split.argtypes = [ctypes.POINTER(AttnShape), _VP, ctypes.POINTER(SplitCache),
                                              ctypes.POINTER(SplitCache), _VP, _F, _VP, _VP, ctypes.c_size_t, _VP]
    lib.tq_search_workspace_size.argtypes = [_VP, _I64, ctypes.POINTER(ctypes.c_size_t)]
    lib.tq_search_scores.argtypes = [_VP, _VP, _I64, _VP, _VP, _VP, _VP, _I64, _VP, _VP, ctypes.c_size_t, _VP]
    lib.tq_decode_workspace_size.argtypes = [ctypes.POINTER(AttnShape), ctypes.POINTER(PackedKV),
                                             ctypes.POINTER(PackedKV), ctypes.POINTER(ctypes.c_size_t)]
    lib.tq_decode_attention.argtypes = [ctypes.POINTER(AttnShape), _VP, ctypes.POINTER(PackedKV),
                                        ctypes.POINTER(PackedKV), _VP, _F, _VP, _VP, _VP, ctypes.c_size_t, _VP]
    lib.tq_decode_append_workspace_size.argtypes = [ctypes.POINTER(AttnShape), ctypes.POINTER(PackedKV),
                                                    ctypes.POINTER(PackedKV), ctypes.POINTER(ctypes.c_size_t)]
    lib.tq_decode_append_attention.argtypes = [ctypes.POINTER(AttnShape), _VP, _VP, _VP, _I,
                                               ctypes.POINTER(PackedKV), ctypes.POINTER(PackedKV), _VP, _F, _VP,
                                               _VP, ctypes.c_size_t, _VP]
    for name in EXPORTS:
        if name not in ("tq_status_string", "tq_last_error_message", "tq_version"):
            getattr(lib, name).restype = _I
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != TQ_OK:
        msg = _lib.tq_last_error_message().decode() if _lib else ""
        raise TQError(status, where, msg or _lib.tq_status_string(status).decode())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


# ----------------------------------------------------------------------------------------
def codebook_build(d: int, bits: int):
    """Lloyd-Max codebook for one rotated coordinate: (centroids, thresholds, cost C(f_X, b))."""
    lib = load()
    K = 1 << bits
    c = np.zeros(K, dtype=np.float32)
    t = np.zeros(max(K - 1, 1), dtype=np.float32)
    cost = ctypes.c_double(0.0)
    _check(lib.tq_codebook_build(d, bits, c.ctypes.data, t.ctypes.data, ctypes.byref(cost)), "tq_codebook_build")
    return c, t[:K - 1], cost.value


class Quantizer:
    """Owns one tq_quantizer handle (device tables on the current device)."""

    def __init__(self, d: int, bits: int, variant: str, pi: np.ndarray, s: Optional[np.ndarray] = None):
        lib = load()
        self.d, self.bits, self.variant = int(d), int(bits), variant
        v = TQ_PROD if variant == "prod" else TQ_MSE
        pi64 = np.ascontiguousarray(pi, dtype=np.float64)
        s64 = None if s is None else np.ascontiguousarray(s, dtype=np.float64)
        h = ctypes.c_void_p()
        _check(lib.tq_quantizer_create(d, bits, v, pi64.ctypes.data,
                                       None if s64 is None else s64.ctypes.data, ctypes.byref(h)),
               "tq_quantizer_create")
        self.handle = h
        self.planes = bits - 1 if variant == "prod" else bits

    @classmethod
    def wht(cls, d: int, bits: int, variant: str, signs: np.ndarray, s: Optional[np.ndarray] = None) -> "Quantizer":
        """Quantizer with the randomized Walsh-Hadamard rotation H diag(signs) / sqrt(d)."""
        lib = load()
        self = cls.__new__(cls)
        self.d, self.bits, self.variant = int(d), int(bits), variant
        v = TQ_PROD if variant == "prod" else TQ_MSE
        sg = np.ascontiguousarray(signs, dtype=np.float64)
        s64 = None if s is None else np.ascontiguousarray(s, dtype=np.float64)
        h = ctypes.c_void_p()
        _check(lib.tq_quantizer_create_wht(d, bits, v, sg.ctypes.data, None if s64 is None else s64.ctypes.data,
                                           ctypes.byref(h)), "tq_quantizer_create_wht")
        self.handle = h
        self.planes = bits - 1 if variant == "prod" else bits
        return self

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            _check(_lib.tq_quantizer_destroy(self.handle), "tq_quantizer_destroy")
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def code_bytes(self) -> int:
        return self.planes * self.d // 8


def _handles(qs: Sequence[Quantizer]):
    arr = (ctypes.c_void_p * len(qs))(*[q.handle.value for q in qs])
    return arr


def quantize(qs: Sequence[Quantizer], x, layout: str = "vector", rot_dbg: bool = False,
             proj_dbg: bool = False, out: Optional[dict] = None, stream=None) -> dict:
    """Grouped quantize: x is [G, n, d] (float32 or bfloat16 torch CUDA tensor), group g uses qs[g]."""
    import torch
    lib = load()
    q0 = qs[0]
    G = len(qs)
    assert x.dim() == 3 and x.shape[0] == G and x.shape[2] == q0.d, "x must be [n_groups, n, d]"
    x = x.contiguous()
    n = x.shape[1]
    dev = x.device
    lay = TQ_LAYOUT_BLOCK32 if layout == "block32" else TQ_LAYOUT_VECTOR
    dt = TQ_BF16 if x.dtype == torch.bfloat16 else TQ_F32
    if dt == TQ_F32 and x.dtype != torch.float32:
        raise TypeError("x must be float32 or bfloat16")
    o = out if out is not None else {}
    if "norms" not in o:
        o["norms"] = torch.empty((G, n), dtype=torch.float32, device=dev)
        if q0.planes > 0:
            o["codes"] = torch.empty((G, n * q0.code_bytes), dtype=torch.uint8, device=dev)
        if q0.variant == "prod":
            o["signs"] = torch.empty((G, n, q0.d // 8), dtype=torch.uint8, device=dev)
            o["rnorms"] = torch.empty((G, n), dtype=torch.float32, device=dev)
    if rot_dbg and "rot" not in o:
        o["rot"] = torch.empty((G, n, q0.d), dtype=torch.float32, device=dev)
    if proj_dbg and "proj" not in o:
        o["proj"] = torch.empty((G, n, q0.d), dtype=torch.float32, device=dev)
    hs = _handles(qs)
    _check(lib.tq_quantize(hs, G, n, _ptr(x), dt, lay, _ptr(o.get("codes")), _ptr(o.get("signs")),
                           _ptr(o["norms"]), _ptr(o.get("rnorms")), _ptr(o.get("rot")), _ptr(o.get("proj")),
                           _stream(stream)), "tq_quantize")
    return o


def _rows(x):
    """x [n, d] with unit column stride read in place (its row stride passed on), else a contiguous copy."""
    if x.dim() == 2 and x.stride(1) == 1 and x.stride(0) >= x.shape[1]:
        return x, x.stride(0)
    x = x.contiguous()
    return x, x.shape[-1]


def quantize_mse(q: Quantizer, x, rot_dbg: bool = False, stream=None) -> dict:
    import torch
    lib = load()
    n = x.shape[0]
    x, stride = _rows(x)
    dt = TQ_BF16 if x.dtype == torch.bfloat16 else TQ_F32
    o = {"codes": torch.empty((n, q.code_bytes), dtype=torch.uint8, device=x.device),
         "norms": torch.empty(n, dtype=torch.float32, device=x.device)}
    if rot_dbg:
        o["rot"] = torch.empty((n, q.d), dtype=torch.float32, device=x.device)
    _check(lib.tq_quantize_mse(q.handle, _ptr(x), dt, n, stride, _ptr(o["codes"]), _ptr(o["norms"]),
                               _ptr(o.get("rot")), _stream(stream)), "tq_quantize_mse")
    return o


def quantize_prod(q: Quantizer, x, rot_dbg: bool = False, proj_dbg: bool = False, stream=None) -> dict:
    import torch
    lib = load()
    n = x.shape[0]
    x, stride = _rows(x)
    dt = TQ_BF16 if x.dtype == torch.bfloat16 else TQ_F32
    dev = x.device
    o = {"codes": torch.empty((n, max(q.code_bytes, 1)), dtype=torch.uint8, device=dev),
         "signs": torch.empty((n, q.d // 8), dtype=torch.uint8, device=dev),
         "norms": torch.empty(n, dtype=torch.float32, device=dev),
         "rnorms": torch.empty(n, dtype=torch.float32, device=dev)}
    if rot_dbg:
        o["rot"] = torch.empty((n, q.d), dtype=torch.float32, device=dev)
    if proj_dbg:
        o["proj"] = torch.empty((n, q.d), dtype=torch.float32, device=dev)
    _check(lib.tq_quantize_prod(q.handle, _ptr(x), dt, n, stride, _ptr(o["codes"]) if q.planes else None,
                                _ptr(o["signs"]), _ptr(o["norms"]), _ptr(o["rnorms"]), _ptr(o.get("rot")),
                                _ptr(o.get("proj")), _stream(stream)), "tq_quantize_prod")
    return o


def dequantize(q: Quantizer, codes, norms, signs=None, rnorms=None, layout: str = "vector", stream=None):
    import torch
    lib = load()
    n = norms.numel()
    out = torch.empty((n, q.d), dtype=torch.float32, device=norms.device)
    lay = TQ_LAYOUT_BLOCK32 if layout == "block32" else TQ_LAYOUT_VECTOR
    _check(lib.tq_dequantize(q.handle, lay, _ptr(codes) if q.planes else None, _ptr(signs), _ptr(norms),
                             _ptr(rnorms), n, _ptr(out), _stream(stream)), "tq_dequantize")
    return out


def inner_products(q: Quantizer, y, codes, norms, signs=None, rnorms=None, stream=None):
    import torch
    lib = load()
    m, n = y.shape[0], norms.numel()
    out = torch.empty((m, n), dtype=torch.float32, device=y.device)
    _check(lib.tq_inner_products(q.handle, _ptr(y.contiguous()), m, _ptr(codes) if q.planes else None,
                                 _ptr(signs), _ptr(norms), _ptr(rnorms), n, _ptr(out), _stream(stream)),
           "tq_inner_products")
    return out


def _split_args(qs, channels):
    import numpy as np
    ch = np.ascontiguousarray(np.concatenate([np.asarray(c, dtype=np.int32).ravel() for c in channels]), dtype=np.int32)
    for q, c in zip(qs, channels):
        assert len(c) == q.d, "each part's channel list must have its quantizer's d entries"
    return ch


def _records(rs):
    arr = (Records * len(rs))()
    for i, r in enumerate(rs):
        arr[i] = Records(_ptr(r.get("codes")), _ptr(r.get("signs")), _ptr(r["norms"]), _ptr(r.get("rnorms")),
                         _ptr(r.get("rot")), _ptr(r.get("proj")))
    return arr


def quantize_split(qs: Sequence[Quantizer], channels, x, rot_dbg: bool = False, proj_dbg: bool = False,
                   stream=None) -> list:
    """Outlier-channel split (tq_quantize_split): part p quantizes x[:, channels[p]] with qs[p].
    x: [n, dim] float32 or bfloat16 CUDA tensor; returns one record dict per part."""
    import torch
    lib = load()
    x = x.contiguous()
    n, dim = x.shape
    dt = TQ_BF16 if x.dtype == torch.bfloat16 else TQ_F32
    ch = _split_args(qs, channels)
    outs = []
    for q in qs:
        o = {"norms": torch.empty(n, dtype=torch.float32, device=x.device)}
        if q.planes > 0:
            o["codes"] = torch.empty((n, q.code_bytes), dtype=torch.uint8, device=x.device)
        if q.variant == "prod":
            o["signs"] = torch.empty((n, q.d // 8), dtype=torch.uint8, device=x.device)
            o["rnorms"] = torch.empty(n, dtype=torch.float32, device=x.device)
            if proj_dbg:
                o["proj"] = torch.empty((n, q.d), dtype=torch.float32, device=x.device)
        if rot_dbg:
            o["rot"] = torch.empty((n, q.d), dtype=torch.float32, device=x.device)
        outs.append(o)
    _check(lib.tq_quantize_split(_handles(qs), len(qs), ch.ctypes.data, dim, _ptr(x), dt, n, _records(outs),
                                 _stream(stream)), "tq_quantize_split")
    return outs


def inner_products_split(qs: Sequence[Quantizer], channels, y, recs, stream=None):
    """sum over parts of <y restricted to part p, x~_p> (tq_inner_products_split); y: [m, dim] float32."""
    import torch
    lib = load()
    y = y.contiguous()
    m, dim = y.shape
    n = recs[0]["norms"].numel()
    ch = _split_args(qs, channels)
    out = torch.empty((m, n), dtype=torch.float32, device=y.device)
    _check(lib.tq_inner_products_split(_handles(qs), len(qs), ch.ctypes.data, dim, _ptr(y), m, _records(recs), n,
                                       _ptr(out), _stream(stream)), "tq_inner_products_split")
    return out


def search_workspace_size(q: Quantizer, m: int) -> int:
    lib = load()
    nb = ctypes.c_size_t(0)
    _check(lib.tq_search_workspace_size(q.handle, m, ctypes.byref(nb)), "tq_search_workspace_size")
    return nb.value


def search_scores(q: Quantizer, y, codes, norms, signs=None, rnorms=None, workspace=None, stream=None):
    """<y_i, x~_j> on the matrix cores (tq_search_scores); workspace: a uint8 device
    tensor of at least search_workspace_size(q, m) bytes (allocated when None)."""
    import torch
    lib = load()
    m, n = y.shape[0], norms.numel()
    out = torch.empty((m, n), dtype=torch.float32, device=y.device)
    if workspace is None:
        workspace = torch.empty(max(search_workspace_size(q, m), 1), dtype=torch.uint8, device=y.device)
    _check(lib.tq_search_scores(q.handle, _ptr(y.contiguous()), m, _ptr(codes) if q.planes else None,
                                _ptr(signs), _ptr(norms), _ptr(rnorms), n, _ptr(out), _ptr(workspace),
                                workspace.numel(), _stream(stream)), "tq_search_scores")
    return out


@dataclass
class KVCache:
    """Packed cache of one tensor (keys or values) for decode attention."""
    qz: Sequence[Quantizer]           # one per KV head
    norms: object                     # [B, Hkv, T] float32
    codes: object = None              # keys: [B, Hkv, T, planes*d/8]; values: [B, Hkv, T/32, 4*bits*d]
    signs: object = None              # prod keys: [B, Hkv, T, d/8]
    rnorms: object = None             # prod keys: [B, Hkv, T]

    def packed(self):
        arr = _handles(self.qz)
        kv = PackedKV(ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)), _ptr(self.codes), _ptr(self.signs),
                      _ptr(self.norms), _ptr(self.rnorms))
        return kv, arr


def decode_workspace_size(batch, n_q_heads, n_kv_heads, d, max_ctx, kcache: KVCache, vcache: KVCache) -> int:
    lib = load()
    shape = AttnShape(batch, n_q_heads, n_kv_heads, d, max_ctx)
    kp, ka = kcache.packed()
    vp, va = vcache.packed()
    nbytes = ctypes.c_size_t(0)
    _check(lib.tq_decode_workspace_size(ctypes.byref(shape), ctypes.byref(kp), ctypes.byref(vp),
                                        ctypes.byref(nbytes)), "tq_decode_workspace_size")
    return nbytes.value


def decode_attention(q, kcache: KVCache, vcache: KVCache, ctx_lens, scale: Optional[float] = None,
                     max_ctx: Optional[int] = None, out=None, scores=None, workspace=None, stream=None):
    """q: [B, Hq, d] bfloat16; ctx_lens: int32 [B] (device). Returns out [B, Hq, d] float32."""
    import torch
    lib = load()
    B, Hq, d = q.shape
    Hkv = len(kcache.qz)
    T = int(max_ctx if max_ctx is not None else kcache.norms.shape[-1])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    shape = AttnShape(B, Hq, Hkv, d, T)
    kp, ka = kcache.packed()
    vp, va = vcache.packed()
    if workspace is None:
        nbytes = decode_workspace_size(B, Hq, Hkv, d, T, kcache, vcache)
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _check(lib.tq_decode_attention(ctypes.byref(shape), _ptr(q.contiguous()), ctypes.byref(kp), ctypes.byref(vp),
                                   _ptr(ctx_lens), float(scale), _ptr(out), _ptr(scores), _ptr(workspace),
                                   workspace.numel(), _stream(stream)), "tq_decode_attention")
    return out


@dataclass
class SplitKV:
    """One side (keys or values) of a split cache: parts[p] = (quantizers per KV head,
    channel list, records dict of device tensors [B, Hkv, T, ...] / [B, Hkv, T])."""
    parts: Sequence[tuple]

    def packed(self, n_kv_heads):
        import numpy as np
        P = len(self.parts)
        qz = (ctypes.c_void_p * (P * n_kv_heads))()
        for p, (qs, _, _) in enumerate(self.parts):
            assert len(qs) == n_kv_heads
            for g, q in enumerate(qs):
                qz[p * n_kv_heads + g] = q.handle.value
        ch = np.ascontiguousarray(np.concatenate([np.asarray(c, dtype=np.int32).ravel() for _, c, _ in self.parts]),
                                  dtype=np.int32)
        recs = _records([r for _, _, r in self.parts])
        sc = SplitCache(P, qz, ch.ctypes.data, ctypes.cast(recs, ctypes.c_void_p))
        return sc, (qz, ch, recs)  # keep the arrays alive for the call


def decode_split_workspace_size(batch, n_q_heads, n_kv_heads, dim, max_ctx, k: SplitKV, v: SplitKV) -> int:
    lib = load()
    shape = AttnShape(batch, n_q_heads, n_kv_heads, dim, max_ctx)
    kc, ka = k.packed(n_kv_heads)
    vc, va = v.packed(n_kv_heads)
    nbytes = ctypes.c_size_t(0)
    _check(lib.tq_decode_split_workspace_size(ctypes.byref(shape), ctypes.byref(kc), ctypes.byref(vc),
                                              ctypes.byref(nbytes)), "tq_decode_split_workspace_size")
    return nbytes.value


def decode_attention_split(q, k: SplitKV, v: SplitKV, ctx_lens, scale: Optional[float] = None,
                           max_ctx: Optional[int] = None, out=None, workspace=None, stream=None):
    """Decode attention over outlier-split caches (tq_decode_attention_split).
    q: [B, Hq, dim] bfloat16; ctx_lens: int32 [B] (device). Returns out [B, Hq, dim] float32."""
    import torch
    lib = load()
    B, Hq, dim = q.shape
    Hkv = len(k.parts[0][0])
    T = int(max_ctx if max_ctx is not None else k.parts[0][2]["norms"].shape[-1])
    if scale is None:
        scale = 1.0 / math.sqrt(dim)
    shape = AttnShape(B, Hq, Hkv, dim, T)
    kc, ka = k.packed(Hkv)
    vc, va = v.packed(Hkv)
    if workspace is None:
        workspace = torch.empty(max(decode_split_workspace_size(B, Hq, Hkv, dim, T, k, v), 1), dtype=torch.uint8,
                                device=q.device)
    if out is None:
        out = torch.empty((B, Hq, dim), dtype=torch.float32, device=q.device)
    _check(lib.tq_decode_attention_split(ctypes.byref(shape), _ptr(q.contiguous()), ctypes.byref(kc),
                                         ctypes.byref(vc), _ptr(ctx_lens), float(scale), _ptr(out),
                                         _ptr(workspace), workspace.numel(), _stream(stream)),
           "tq_decode_attention_split")
    return out


def decode_append_workspace_size(batch, n_q_heads, n_kv_heads, d, max_ctx, kcache: KVCache,
                                 vcache: KVCache) -> int:
    lib = load()
    shape = AttnShape(batch, n_q_heads, n_kv_heads, d, max_ctx)
    kp, ka = kcache.packed()
    vp, va = vcache.packed()
    nbytes = ctypes.c_size_t(0)
    _check(lib.tq_decode_append_workspace_size(ctypes.byref(shape), ctypes.byref(kp), ctypes.byref(vp),
                                               ctypes.byref(nbytes)), "tq_decode_append_workspace_size")
    return nbytes.value


def decode_append_attention(q, k_new, v_new, kcache: KVCache, vcache: KVCache, ctx_lens,
                            scale: Optional[float] = None, max_ctx: Optional[int] = None, out=None,
                            workspace=None, stream=None):
    """Quantize k_new / v_new ([B, Hkv, d], float32 or bfloat16) into the caches at
    token ctx_lens[b], then attend ctx_lens[b] + 1 tokens. ctx_lens is not advanced."""
    import torch
    lib = load()
    B, Hq, d = q.shape
    Hkv = len(kcache.qz)
    T = int(max_ctx if max_ctx is not None else kcache.norms.shape[-1])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    assert tuple(k_new.shape) == (B, Hkv, d) and tuple(v_new.shape) == (B, Hkv, d)
    if k_new.dtype != v_new.dtype or k_new.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("k_new and v_new must share a float32 or bfloat16 dtype")
    dt = TQ_BF16 if k_new.dtype == torch.bfloat16 else TQ_F32
    shape = AttnShape(B, Hq, Hkv, d, T)
    kp, ka = kcache.packed()
    vp, va = vcache.packed()
    if workspace is None:
        nbytes = decode_append_workspace_size(B, Hq, Hkv, d, T, kcache, vcache)
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _check(lib.tq_decode_append_attention(ctypes.byref(shape), _ptr(q.contiguous()), _ptr(k_new.contiguous()),
                                          _ptr(v_new.contiguous()), dt, ctypes.byref(kp), ctypes.byref(vp),
                                          _ptr(ctx_lens), float(scale), _ptr(out), _ptr(workspace),
                                          workspace.numel(), _stream(stream)), "tq_decode_append_attention")
    return out
