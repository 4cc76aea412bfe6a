"""HIP-graph capture of the decode step loop and the prefill: every replay, with eager work
and synchronisations between replays, must reproduce the eager results bit for bit."""
import pytest
import torch

import sliding_window_attention_02_amd as swa
from sliding_window_attention_02_amd import inputs

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    B, Hq, Hkv, d, w, s, T, P = 4, 32, 8, 128, 64, 4, 40, 1000
    dev = torch.device("cuda")
    kc, vc = swa.alloc_cache(B, Hkv, d, w, s, device=dev)
    ws = swa.alloc_workspace(B, Hq, Hkv, d, w, s, device=dev)
    seed_k, seed_v = inputs.kv_span(3, list(range(s)) + list(range(P - w, P)), B, Hkv, d)
    swa.kv_append(kc, vc, seed_k[:, :s].contiguous().to(dev), seed_v[:, :s].contiguous().to(dev),
                  torch.zeros(B, dtype=torch.int64, device=dev), w, s)
    swa.kv_append(kc, vc, seed_k[:, s:].contiguous().to(dev), seed_v[:, s:].contiguous().to(dev),
                  torch.full((B,), P - w, dtype=torch.int64, device=dev), w, s)
    snap = kc.clone(), vc.clone()
    gen = torch.Generator().manual_seed(5)
    dq = torch.randn(T, B, Hq, d, generator=gen).to(torch.bfloat16).to(dev)
    dk = torch.randn(T, B, 1, Hkv, d, generator=gen).to(torch.bfloat16).to(dev)
    dv = torch.randn(T, B, 1, Hkv, d, generator=gen).to(torch.bfloat16).to(dev)
    dpos = (P + torch.arange(T)).repeat_interleave(B).view(T, B).to(dev)
    out = torch.zeros(T, B, Hq, d, device=dev)
    q, k, v = [x.to(dev) for x in inputs.random_qkv(1, 700, 32, 8, 128, seed=9, sink_boost_n=4, sink_boost=4.0)]
    pout = torch.zeros(1, 700, 32, 128, device=dev)

    def work():
        for i in range(T):
            swa.kv_append(kc, vc, dk[i], dv[i], dpos[i], w, s)
            swa.decode_step(dq[i], kc, vc, dpos[i], w, s, out=out[i], workspace=ws)
        swa.prefill(q, k, v, 64, 4, out=pout)

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        work()
    stream.synchronize()
    eager, eager_p = out.clone(), pout.clone()

    kc.copy_(snap[0]); vc.copy_(snap[1])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        work()
    torch.cuda.synchronize()
    for r in range(4):
        kc.copy_(snap[0]); vc.copy_(snap[1])
        out.zero_(); pout.zero_()
        swa.prefill(q, k, v, 16, 0)  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), r
        assert torch.equal(pout, eager_p), r
