"""GPU check of tq_decode_attention_noalloc, the decode entry point that takes
its workspace from the library's static per-GPU scratch instead of the caller:
its output must equal tq_decode_attention's (same kernels and split schedule,
so the same bits) on two calls in a row, the second with a smaller input (the
scratch keeps the first call's partials), and a shape needing more scratch
than the static array holds must be refused before any launch.
"""
import math

import numpy as np
import pytest
import torch

import tq_synth as syn
from test_gpu_decode import _build
from tq_testlib import matrices

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _decode_both(tq, case):
    B, Hq, Hkv, d, T, kbits, kvar, vbits, lens = case
    print(f"noalloc case {case}", flush=True)
    kcache, vcache, _, _ = _build(tq, B, Hq, Hkv, d, T, kbits, kvar, vbits, syn.CFG_TEST)
    q = torch.from_numpy(syn.decode_queries(B, Hq, d, syn.CFG_TEST)).to(DEV).to(torch.bfloat16)
    ctx = torch.tensor(lens, dtype=torch.int32, device=DEV)
    scale = 1.0 / math.sqrt(d)
    ref = tq.decode_attention(q, kcache, vcache, ctx, scale)
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=DEV)
    got = tq.decode_attention_noalloc(q, kcache, vcache, ctx, out, scale)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    return ref.cpu().numpy(), out.cpu().numpy()


def test_noalloc_matches_workspace_entry_twice(gpu_lib):
    tq = gpu_lib
    # first a large call (many splits, long contexts), then a smaller one of another
    # shape: the second must not see anything of the first call's partials
    for case in [(4, 64, 8, 128, 4096, 3, "prod", 3, [4096, 3001, 17, 0]),
                 (2, 16, 2, 64, 256, 2, "mse", 2, [200, 33])]:
        ref, got = _decode_both(tq, case)
        assert np.all(np.isfinite(got))
        assert np.array_equal(got, ref), (case, float(np.max(np.abs(got - ref))))


def test_noalloc_refuses_shapes_beyond_the_static_scratch(gpu_lib):
    tq = gpu_lib
    B, Hq, Hkv, d, T = 128, 64, 8, 256, 32
    kq, vq = [], []
    for h in range(Hkv):
        Pi, S = matrices(d, syn.CFG_TEST, syn.T_K, h, True)
        kq.append(tq.Quantizer(d, 3, "prod", Pi, S))
        Pv, _ = matrices(d, syn.CFG_TEST, syn.T_V, h, False)
        vq.append(tq.Quantizer(d, 3, "mse", Pv))
    z = lambda *shape, dt=torch.float32: torch.zeros(shape, dtype=dt, device=DEV)
    kcache = tq.KVCache(kq, z(B, Hkv, T), z(B, Hkv, T, 2 * d // 8, dt=torch.uint8),
                        z(B, Hkv, T, d // 8, dt=torch.uint8), z(B, Hkv, T))
    vcache = tq.KVCache(vq, z(B, Hkv, T), z(B, Hkv, T // 32, 4 * 3 * d, dt=torch.uint8))
    need = tq.decode_workspace_size(B, Hq, Hkv, d, T, kcache, vcache)
    assert need > (32 << 20), need
    q = z(B, Hq, d, dt=torch.bfloat16)
    out = torch.full((B, Hq, d), 7.0, dtype=torch.float32, device=DEV)
    ctx = torch.full((B,), T, dtype=torch.int32, device=DEV)
    with pytest.raises(tq.TQError, match="static scratch"):
        tq.decode_attention_noalloc(q, kcache, vcache, ctx, out)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)  # refused before any launch
