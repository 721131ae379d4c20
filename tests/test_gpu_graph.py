"""Decode attention and the decode step with append captured in a HIP graph
(torch.cuda.CUDAGraph on ROCm): the library launches on the caller's stream and
allocates nothing, so the calls capture as plain kernel nodes. Each replay,
with eager work and synchronizations in between, must reproduce the eager
result bit for bit (both paths are deterministic for a fixed shape)."""
import math

import numpy as np
import pytest
import torch

import tq_synth as syn
from test_gpu_decode import _build

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_decode_and_append_in_graph(gpu_lib):
    tq = gpu_lib
    B, Hq, Hkv, d, T = 2, 16, 2, 128, 256
    print(f"graph capture B={B} Hq={Hq} Hkv={Hkv} d={d} T={T}", flush=True)
    kcache, vcache, _, _ = _build(tq, B, Hq, Hkv, d, T, 3, "prod", 3, syn.CFG_TEST)
    q = torch.from_numpy(syn.decode_queries(B, Hq, d, syn.CFG_TEST)).to(DEV).to(torch.bfloat16)
    lens = torch.tensor([200, 97], dtype=torch.int32, device=DEV)
    knew = torch.from_numpy(np.stack([syn.kv_vectors(Hkv, d, syn.CFG_TEST, syn.T_K, b, 77) for b in range(B)])).to(DEV)
    vnew = torch.from_numpy(np.stack([syn.kv_vectors(Hkv, d, syn.CFG_TEST, syn.T_V, b, 77) for b in range(B)])).to(DEV)
    scale = 1 / math.sqrt(d)
    ws = torch.empty(tq.decode_append_workspace_size(B, Hq, Hkv, d, T, kcache, vcache), dtype=torch.uint8,
                     device=DEV)
    out_d = torch.empty((B, Hq, d), dtype=torch.float32, device=DEV)
    out_a = torch.empty((B, Hq, d), dtype=torch.float32, device=DEV)

    def step():
        tq.decode_attention(q, kcache, vcache, lens, scale, max_ctx=T, out=out_d, workspace=ws)
        tq.decode_append_attention(q, knew, vnew, kcache, vcache, lens, scale, max_ctx=T, out=out_a, workspace=ws)

    # eager reference (the append writes the same token at the same slot every time)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    want_d, want_a = out_d.clone(), out_a.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(3):
        out_d.fill_(float("nan"))
        out_a.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_d, want_d), i
        assert torch.equal(out_a, want_a), i
        # eager work between replays
        step()
        torch.cuda.synchronize()
        assert torch.equal(out_d, want_d) and torch.equal(out_a, want_a), i
