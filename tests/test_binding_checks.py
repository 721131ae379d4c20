"""Argument checks of the Python binding: wrong dtypes, shapes and cache extents
are refused before anything reaches the library (no GPU needed). A float16
input read as float32, or a cache shorter than max_ctx, would otherwise make a
kernel read past its buffers."""
from types import SimpleNamespace

import pytest
import torch

import attention_tq_quantize_amd as tq


def _q(d=128, bits=3, variant="mse"):
    planes = bits - 1 if variant == "prod" else bits
    return SimpleNamespace(d=d, bits=bits, variant=variant, planes=planes, code_bytes=planes * d // 8,
                           handle=None)


def test_quantize_refuses_other_float_types():
    x16 = torch.zeros((4, 128), dtype=torch.float16)
    with pytest.raises(TypeError):
        tq.quantize_mse(_q(), x16)
    with pytest.raises(TypeError):
        tq.quantize_prod(_q(variant="prod"), x16)
    with pytest.raises(TypeError):
        tq.quantize([_q()], x16[None])
    with pytest.raises(TypeError):
        tq.quantize_split([_q(d=32), _q(d=96)], [list(range(32)), list(range(32, 128))], x16)


def test_quantize_refuses_a_wrong_head_dimension():
    with pytest.raises(ValueError):
        tq.quantize_mse(_q(d=128), torch.zeros((4, 64), dtype=torch.float32))
    with pytest.raises(ValueError):
        tq.quantize([_q(d=128)], torch.zeros((1, 4, 64), dtype=torch.float32))


def _caches(B, Hkv, d, T, short=None):
    def t(n, dt):
        return torch.zeros(n, dtype=dt)
    G = B * Hkv
    kq, vq = _q(d, 3, "prod"), _q(d, 3, "mse")
    k = tq.KVCache([kq] * Hkv, t(G * T, torch.float32), t(G * T * kq.code_bytes, torch.uint8),
                   t(G * T * d // 8, torch.uint8), t(G * T, torch.float32))
    v = tq.KVCache([vq] * Hkv, t(G * T, torch.float32), t(G * T * vq.code_bytes, torch.uint8))
    if short == "k.codes":
        k.codes = t(G * T * kq.code_bytes - 1, torch.uint8)
    if short == "v.codes":
        v.codes = t(G * (T - 32) * vq.code_bytes, torch.uint8)
    if short == "v.norms":
        v.norms = t(G * T - 1, torch.float32)
    return k, v


def test_decode_refuses_wrong_dtypes():
    B, Hq, Hkv, d, T = 2, 16, 2, 128, 64
    k, v = _caches(B, Hkv, d, T)
    lens = torch.full((B,), T, dtype=torch.int32)
    with pytest.raises(TypeError):
        tq.decode_attention(torch.zeros((B, Hq, d), dtype=torch.float32), k, v, lens)
    with pytest.raises(TypeError):
        tq.decode_attention(torch.zeros((B, Hq, d), dtype=torch.bfloat16), k, v, lens.long())
    with pytest.raises(ValueError):
        tq.decode_attention(torch.zeros((B, Hq, d), dtype=torch.bfloat16), k, v, lens[:1])


@pytest.mark.parametrize("short", ["k.codes", "v.codes", "v.norms"])
def test_decode_refuses_caches_shorter_than_max_ctx(short):
    B, Hq, Hkv, d, T = 2, 16, 2, 128, 64
    k, v = _caches(B, Hkv, d, T, short=short)
    q = torch.zeros((B, Hq, d), dtype=torch.bfloat16)
    lens = torch.full((B,), T, dtype=torch.int32)
    with pytest.raises(ValueError, match=short):
        tq.decode_attention(q, k, v, lens, max_ctx=T)


def test_decode_append_refuses_wrong_new_token_shapes_and_dtypes():
    B, Hq, Hkv, d, T = 2, 16, 2, 128, 64
    k, v = _caches(B, Hkv, d, T)
    q = torch.zeros((B, Hq, d), dtype=torch.bfloat16)
    lens = torch.zeros((B,), dtype=torch.int32)
    good = torch.zeros((B, Hkv, d), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        tq.decode_append_attention(q, good[:, :1], good, k, v, lens)
    with pytest.raises(TypeError):
        tq.decode_append_attention(q, good.half(), good.half(), k, v, lens)
