"""GPU parity of swa_prefill_chunk (chunked prefill into the bounded cache) against the fp64
oracle, through the C ABI.

A sequence fed chunk by chunk must give, row for row, the whole-sequence SWA(w,s) prefill
(max abs error <= 2e-2), from an empty cache (filled with NaN, which must never reach a
result) through sink-fill, ring-fill and wrap-around, with chunks shorter and longer than
the window; the cache afterwards must equal, bit for bit, the cache that appending every
position one by one leaves.  Far from the start (positions past 2^31) each row is checked
against the oracle's decode row over the explicit set of keys the row may see.
"""
import numpy as np
import pytest
import torch

import sliding_window_attention_02_amd as swa
from oracle import oracle as orc
from sliding_window_attention_02_amd import inputs

pytestmark = pytest.mark.gpu

TOL = 2e-2


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def say(*a):
    print(*a, flush=True)


def sequence(seed, B, L, Hq, Hkv, d, std=1.0):
    q, k, v = inputs.random_qkv(B, L, Hq, Hkv, d, seed, std=std, sink_boost_n=4, sink_boost=4.0)
    return q, k, v  # bf16 [B][L][H][d] on the CPU


def nan_cache(B, Hkv, d, w, s, conv):
    kc, vc = swa.alloc_cache(B, Hkv, d, w, s, conv)
    kc.fill_(float("nan"))
    vc.fill_(float("nan"))
    return kc, vc


CASES = [
    # B, Hq, Hkv, d, w, s, conv, chunk sizes (their sum is L)
    (2, 8, 2, 128, 16, 4, 0, [1, 3, 16, 40, 7, 100, 33]),
    (1, 4, 4, 64, 8, 0, 0, [8] * 12 + [4]),
    (3, 12, 4, 128, 20, 4, 1, [2, 2, 50, 96]),  # the first chunks end inside the sinks
    (1, 32, 8, 128, 64, 4, 0, [64] * 9 + [24]),  # Llama-shaped heads, chunks of the window
    (2, 8, 8, 128, 300, 2, 0, [100, 156]),  # window longer than the sequence: full causal
    (1, 8, 2, 64, 33, 9, 0, [5, 61, 1, 1, 90]),
    # four q-heads per kv-head, chunks starting on 32-key but not 64-key boundaries (the resident
    # form's 32-token q-tiles over cached keys)
    (1, 16, 4, 128, 64, 4, 0, [32, 96, 32, 50]),
    # windows over 64 keys: whole 64-key tiles of cached window keys, read as consecutive ring
    # slots, next to tiles whose slots wrap around the ring's end (both head sizes, both window
    # conventions, chunks longer and shorter than the window)
    (1, 8, 2, 128, 200, 4, 0, [300, 150, 200, 77]),
    (2, 16, 4, 64, 160, 8, 1, [70, 200, 130, 100]),
    (1, 16, 4, 128, 512, 4, 0, [512, 512, 300]),
    # chunks whose grids fill the chip (the 128-row forms over cached keys; the smaller chunks
    # above take the 64-row forms): the tile walk at 512-560 workgroups per chunk, the resident
    # form on padded chunks of 2,048 tokens
    (2, 32, 8, 128, 300, 4, 0, [1100, 1024, 400]),
    (1, 32, 8, 128, 64, 4, 0, [2048, 2048]),
]


@pytest.mark.parametrize("B,Hq,Hkv,d,w,s,conv,chunks", CASES)
def test_chunked_prefill_equals_prefill_rows_and_cache(B, Hq, Hkv, d, w, s, conv, chunks, parity):
    """Outputs and (every other chunk) the optional per-row log-sum-exp against the oracle."""
    L = sum(chunks)
    say("chunked", B, Hq, Hkv, d, w, s, conv, chunks)
    q, k, v = sequence(2024, B, L, Hq, Hkv, d)
    scale = 1.0 / np.sqrt(d)
    ref = orc.prefill(f64(q), f64(k), f64(v), w, s, scale, conv)
    ref_lse = orc.lse_rows(f64(q), f64(k), 0, L, w, s, scale, conv)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    kc, vc = nan_cache(B, Hkv, d, w, s, conv)
    outs, lses, p0 = [], [], 0
    for i, C in enumerate(chunks):
        sl = slice(p0, p0 + C)
        lse = torch.full((B, C, Hq), float("nan"), dtype=torch.float32, device="cuda") if i % 2 == 0 else None
        outs.append(swa.prefill_chunk(qg[:, sl].contiguous(), kg[:, sl].contiguous(), vg[:, sl].contiguous(),
                                      kc, vc, p0, w, s, scale, conv, lse=lse))
        if lse is not None:
            lses.append((p0, lse))
        p0 += C
    got = torch.cat(outs, dim=1).cpu().numpy()
    err = np.abs(got - ref)
    say(f"max {err.max():.3e}")
    parity("chunked prefill outputs", err)
    assert np.isfinite(got).all() and err.max() <= TOL
    for p0, lse in lses:
        e = np.abs(lse.cpu().numpy() - ref_lse[:, p0:p0 + lse.shape[1]])
        parity("chunked prefill log-sum-exp", e)
        assert np.isfinite(e).all() and e.max() <= TOL, float(e.max())
    # The cache equals the one that appending every position one by one leaves (bitwise,
    # NaN-filled slots included).
    kc2, vc2 = nan_cache(B, Hkv, d, w, s, conv)
    for t in range(L):
        pos = torch.full((B,), t, dtype=torch.int64, device="cuda")
        swa.kv_append(kc2, vc2, kg[:, t:t + 1].contiguous(), vg[:, t:t + 1].contiguous(), pos, w, s, conv)
    assert torch.equal(kc.view(torch.int16), kc2.view(torch.int16))
    assert torch.equal(vc.view(torch.int16), vc2.view(torch.int16))


@pytest.mark.parametrize("P", [2 ** 31 + 100, 2 ** 18])
def test_chunk_far_from_start_matches_decode_rows(P):
    """The cache holds the state after P-1 (sinks and the window before P); a chunk of 50
    tokens at P; every row against the oracle's decode row over the keys it may see."""
    B, Hq, Hkv, d, w, s, C = 2, 8, 2, 128, 24, 4, 50
    w_loc = w
    say("chunk-far", P)
    seed = 77
    gen = dict(B=B, Hkv=Hkv, d=d, std=1.0, sink_boost_n=4, sink_boost=4.0)
    prev = list(range(s)) + list(range(P - w_loc, P))
    pk, pv = inputs.kv_span(seed, prev, **gen)
    ck, cv = inputs.kv_span(seed, list(range(P, P + C)), **gen)
    cq = torch.stack([inputs.q_at(seed, P + i, B, Hq, d) for i in range(C)], dim=1)
    kc, vc = nan_cache(B, Hkv, d, w, s, 0)
    swa.kv_append(kc, vc, pk[:, :s].contiguous().cuda(), pv[:, :s].contiguous().cuda(),
                  torch.zeros(B, dtype=torch.int64, device="cuda"), w, s)
    swa.kv_append(kc, vc, pk[:, s:].contiguous().cuda(), pv[:, s:].contiguous().cuda(),
                  torch.full((B,), P - w_loc, dtype=torch.int64, device="cuda"), w, s)
    scale = 1.0 / np.sqrt(d)
    out = swa.prefill_chunk(cq.cuda(), ck.cuda(), cv.cuda(), kc, vc, P, w, s, scale).cpu().numpy()
    pos_all = np.array(prev + list(range(P, P + C)), dtype=np.int64)
    k_all = torch.cat([pk, ck], dim=1)
    v_all = torch.cat([pv, cv], dim=1)
    worst = 0.0
    for b in range(B):
        for i in range(C):
            t = P + i
            ref, kept = orc.decode_row(f64(cq[b, i]), pos_all, f64(k_all[b]), f64(v_all[b]), t, w, s, scale)
            assert kept == min(t + 1, w_loc + s)
            worst = max(worst, float(np.abs(out[b, i] - ref).max()))
    say(f"max {worst:.3e}")
    assert worst <= TOL


def test_chunk_of_one_token_equals_decode_step():
    """A one-token chunk is a decode step: same row (to the tolerance; different kernels) and
    the same cache afterwards."""
    B, Hq, Hkv, d, w, s = 2, 32, 8, 128, 64, 4
    L = 150
    q, k, v = sequence(5, B, L, Hq, Hkv, d)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    kc1, vc1 = nan_cache(B, Hkv, d, w, s, 0)
    kc2, vc2 = nan_cache(B, Hkv, d, w, s, 0)
    ws = swa.alloc_workspace(B, Hq, Hkv, d, w, s)
    worst = 0.0
    for t in range(L):
        sl = slice(t, t + 1)
        a = swa.prefill_chunk(qg[:, sl].contiguous(), kg[:, sl].contiguous(), vg[:, sl].contiguous(), kc1, vc1,
                              t, w, s)[:, 0]
        pos = torch.full((B,), t, dtype=torch.int64, device="cuda")
        b = swa.append_decode_step(qg[:, t].contiguous(), kc2, vc2, kg[:, t].contiguous(), vg[:, t].contiguous(),
                                   pos, w, s, workspace=ws)
        worst = max(worst, float((a - b).abs().max()))
    say(f"max {worst:.3e}")
    assert worst <= TOL
    assert torch.equal(kc1.view(torch.int16), kc2.view(torch.int16))
    assert torch.equal(vc1.view(torch.int16), vc2.view(torch.int16))


def _random_chunkings(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 4]))
        d = int(rng.choice([64, 128]))
        w = int(rng.integers(1, 120))
        s = int(rng.integers(0, 8))
        L = int(rng.integers(1, 300))
        chunks, left = [], L
        while left > 0:
            c = int(min(left, rng.integers(1, 2 * w + 8)))
            chunks.append(c)
            left -= c
        out.append((int(rng.integers(1, 3)), G * Hkv, Hkv, d, w, s, 0, chunks))
    return out


@pytest.mark.parametrize("B,Hq,Hkv,d,w,s,conv,chunks", _random_chunkings(6, 777))
def test_chunked_prefill_on_drawn_chunkings(B, Hq, Hkv, d, w, s, conv, chunks, parity):
    test_chunked_prefill_equals_prefill_rows_and_cache(B, Hq, Hkv, d, w, s, conv, chunks, parity)


def test_chunk_at_the_largest_cache(parity):
    """A chunk of 64 tokens against the largest cache the boundary accepts (s + w_loc = 2^23 - 1
    slots at d = 128, filled by one append, the ring wrapped): head 0 of every row aims at the
    key in the cache's last slot, head 1 at the oldest key of the row's window (the ring's
    wrap-around region), so a wrong cached-key address shows at full size; rows checked against
    the oracle over every key they may see."""
    B, Hq, Hkv, d, s, C = 1, 2, 1, 128, 4, 64
    n_slots = 2 ** 23 - 1
    w = n_slots - s
    pos0 = n_slots + 100
    say("chunk at the largest cache", n_slots, pos0)
    _, k, v = inputs.random_qkv_device(B, pos0 + C, 1, Hkv, d, seed=93, device="cuda", sink_boost_n=4,
                                       sink_boost=4.0)
    kc, vc = swa.alloc_cache(B, Hkv, d, w, s)
    swa.kv_append(kc, vc, k[:, :pos0], v[:, :pos0], torch.zeros(B, dtype=torch.int64, device="cuda"), w, s)
    last_slot_pos = w - 1  # slot s + (p mod w) = n_slots - 1, inside every row's window
    rows_t = [pos0 + r for r in range(C)]
    aims = [[last_slot_pos, t - w + 1] for t in rows_t]
    q = torch.stack([torch.stack([k[0, p_, 0].float() * 20.0 for p_ in a]) for a in aims])[None]
    q = q.to(torch.bfloat16).contiguous()
    scale = 1.0 / np.sqrt(d)
    out = swa.prefill_chunk(q, k[:, pos0:].contiguous(), v[:, pos0:].contiguous(), kc, vc, pos0, w, s,
                            scale).cpu().numpy()
    say("chunk attended")
    lo = pos0 - w + 1  # the first row's window start; later rows' windows start later
    pos = np.concatenate([np.arange(s), np.arange(lo, pos0 + C)]).astype(np.int64)
    kk = f64(torch.cat([k[0, :s], k[0, lo:pos0 + C]]))
    vv = f64(torch.cat([v[0, :s], v[0, lo:pos0 + C]]))
    qq = f64(q[0])
    del k, v, kc, vc
    torch.cuda.empty_cache()
    say("oracle inputs on the host")
    worst = 0.0
    for r in (0, 1, 17, C - 1):
        t = rows_t[r]
        ref, kept = orc.decode_row(qq[r], pos, kk, vv, t, w, s, scale)
        assert kept == n_slots
        for h, p_ in enumerate(aims[r]):  # the rows are dominated by the targeted values
            assert np.abs(ref[h] - vv[s + p_ - lo, 0]).max() < 0.1
        err = np.abs(out[0, r] - ref)
        parity("chunked prefill at the largest cache", err)
        worst = max(worst, float(err.max()))
        say("row", r, f"max {worst:.3e}")
    assert worst <= TOL
