"""swa_decode_step_noalloc, the decode step for callers that cannot allocate device memory: the
library's static scratch stands in for the workspace.  Its outputs must equal swa_decode_step's
with a caller-allocated workspace bit for bit (same kernels, same fixed merge order), on two calls
in a row whose second input is smaller, both needing the scratch (workgroup splits)."""
import numpy as np
import pytest
import torch

import sliding_window_attention_02_amd as swa
from sliding_window_attention_02_amd import binding

pytestmark = pytest.mark.gpu


def gpos(vals):
    return torch.tensor(vals, dtype=torch.int64, device="cuda")


def filled_cache(B, Hkv, d, w, s, T, seed):
    g = torch.Generator().manual_seed(seed)
    k = torch.randn(B, T, Hkv, d, generator=g).to(torch.bfloat16).cuda()
    v = torch.randn(B, T, Hkv, d, generator=g).to(torch.bfloat16).cuda()
    kc, vc = swa.alloc_cache(B, Hkv, d, w, s)
    swa.kv_append(kc, vc, k, v, gpos([0] * B), w, s)
    return kc, vc


def test_noalloc_decode_equals_workspace_decode_on_two_calls():
    shapes = [(6, 32, 8, 128, 300, 4), (2, 8, 2, 64, 200, 2)]  # the second call is smaller
    for i, (B, Hq, Hkv, d, w, s) in enumerate(shapes):
        need = swa.decode_workspace_bytes(B, Hq, Hkv, d, w, s)
        assert 0 < need <= 8 << 20
        T = w + s + 7
        kc, vc = filled_cache(B, Hkv, d, w, s, T, seed=10 + i)
        g = torch.Generator().manual_seed(20 + i)
        q = torch.randn(B, Hq, d, generator=g).to(torch.bfloat16).cuda()
        pos = gpos([T - 1 - (b % 3) for b in range(B)])  # mixed positions, all after the wrap
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        ref = swa.decode_step(q, kc, vc, pos, w, s, workspace=ws)
        got = binding.decode_step_noalloc(q, kc, vc, pos, w, s)
        torch.cuda.synchronize()
        assert torch.isfinite(got).all()
        assert torch.equal(got, ref), float((got - ref).abs().max())


def test_noalloc_decode_refuses_shapes_beyond_the_scratch():
    B, Hq, Hkv, d, w, s = 64, 32, 8, 128, 5000, 4
    assert swa.decode_workspace_bytes(B, Hq, Hkv, d, w, s) > 8 << 20
    q = torch.zeros(B, Hq, d, dtype=torch.bfloat16, device="cuda")
    kc, vc = swa.alloc_cache(B, Hkv, d, w, s)
    with pytest.raises(binding.SwaError, match="static scratch holds"):
        binding.decode_step_noalloc(q, kc, vc, gpos([0] * B), w, s)
