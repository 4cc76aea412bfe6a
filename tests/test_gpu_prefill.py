"""GPU parity of swa_prefill against the fp64 oracle (called through the C ABI).

Tolerance: max |gpu - oracle| <= 2e-2 on every compared element (bf16 inputs, bf16
products with fp32 accumulation, fp32 softmax, probabilities rounded to bf16 for the value
product).  Index sets are compared bit for bit.
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


# ------------------------------------------------------------------ index sets


MASK_CASES = [
    # L, Hq, Hkv, w, s, conv
    (1, 4, 4, 1, 0, 0), (1, 4, 1, 64, 4, 0), (5, 4, 4, 2, 1, 0), (64, 4, 1, 64, 4, 0),
    (65, 4, 1, 64, 4, 0), (127, 8, 2, 5, 3, 0), (128, 4, 4, 1, 0, 0), (129, 4, 4, 65, 64, 0),
    (300, 32, 8, 64, 4, 0), (300, 12, 4, 33, 70, 0), (333, 6, 1, 100, 63, 0), (500, 16, 2, 200, 65, 0),
    (1000, 4, 4, 5000, 0, 0), (1000, 32, 8, 128, 4, 1), (1025, 4, 1, 256, 200, 1), (777, 5, 1, 96, 1, 0),
    (4096, 32, 8, 64, 4, 0), (2048, 32, 8, 512, 4, 0),
    # the resident form (four q-heads per kv-head) over many 32-token q-tiles, ragged tails,
    # windows and sinks at its limits (three window chunks, or sinks spanning a chunk)
    (1000, 32, 8, 33, 0, 0), (777, 8, 2, 20, 30, 0), (257, 4, 1, 64, 32, 0), (555, 16, 4, 1, 64, 0),
    (2000, 4, 1, 68, 4, 1), (161, 8, 2, 64, 4, 0),
    # the resident form (two q-heads per kv-head, 64-token q-tiles as one pass)
    (700, 8, 4, 30, 2, 0), (333, 2, 1, 1, 32, 0), (1025, 6, 3, 33, 0, 0),
    # the resident form over 2,000+ tokens and 8-16 kv-heads (three window chunks and no sinks,
    # the total-window convention, sinks in a chunk of their own)
    (2085, 32, 8, 96, 0, 0), (2048, 32, 8, 68, 4, 1), (2100, 64, 16, 33, 30, 0),
    # the 128-row tile walk (grids of 512 workgroups and more): two q-heads per kv-head, the
    # total-window convention; the cases above with windows past four chunks take the 64-row walk
    (4096, 32, 8, 128, 4, 1), (4100, 16, 8, 300, 7, 0),
]


def launched_form(L, Hq, Hkv, w, s, conv, d=128):
    return swa.prefill_describe(1, Hq, Hkv, L, d, w, s, conv)["form"]


def test_index_set_cases_cover_every_kernel_form():
    forms = {launched_form(L, Hq, Hkv, w, s, conv) for L, Hq, Hkv, w, s, conv in MASK_CASES}
    assert forms == {0, 1, 2, 3}
    for form in (0, 1, 2, 3):  # every form over more than twenty q-tiles, at least three times
        assert len([c for c in MASK_CASES if launched_form(*c) == form and c[0] > 640]) >= 3


@pytest.mark.parametrize("L,Hq,Hkv,w,s,conv", MASK_CASES)
def test_prefill_index_set_white_box(L, Hq, Hkv, w, s, conv):
    """The kernel's own walk, mask and slot map (swa_debug_prefill_mask) visit every key of A(t)
    exactly once for every query and nothing else: counts, not just the set."""
    form = launched_form(L, Hq, Hkv, w, s, conv)
    say("mask", L, Hq, Hkv, w, s, conv, "form", form)
    got = swa.debug_prefill_mask(L, Hq, Hkv, w, s, conv).cpu().numpy()
    ref = orc.mask(L, orc.local_window(w, s, conv), s)
    assert np.array_equal(got, ref.astype(np.uint8)), (int(got.max()), int((got != ref).sum()))


@pytest.mark.parametrize("d,L,Hq,Hkv,w,s,conv", [
    (128, 128, 4, 2, 5, 3, 0), (128, 100, 8, 2, 64, 4, 0), (64, 64, 4, 4, 7, 0, 0), (128, 128, 3, 1, 1, 0, 0),
    (128, 128, 4, 4, 128, 0, 0), (64, 64, 2, 1, 10, 70, 0), (128, 97, 32, 8, 20, 4, 1), (64, 61, 16, 2, 3, 2, 0),
    # the resident form over several q-tiles (L up to the one-hot width d)
    (128, 128, 8, 2, 33, 4, 0), (128, 121, 4, 1, 10, 32, 0), (64, 64, 16, 4, 17, 9, 1),
])
def test_prefill_index_set_black_box(d, L, Hq, Hkv, w, s, conv):
    """q = 0 and one-hot values: output row t is exactly 1/|A(t)| on A(t) and 0 elsewhere."""
    say("onehot", d, L, Hq, Hkv, w, s, conv, "form", launched_form(L, Hq, Hkv, w, s, conv, d))
    q = torch.zeros(1, L, Hq, d, dtype=torch.bfloat16)
    k = inputs.random_qkv(1, L, 1, Hkv, d, seed=3)[1]
    v = torch.zeros(1, L, Hkv, d, dtype=torch.bfloat16)
    for i in range(L):
        v[0, i, :, i] = 1.0
    out = swa.prefill(q.cuda(), k.cuda(), v.cuda(), w, s, 1.0, conv).cpu().numpy()
    ref = orc.mask(L, orc.local_window(w, s, conv), s)
    cnt = ref.sum(1).astype(np.float32)
    for h in range(Hq):
        o = out[0, :, h, :]
        assert np.array_equal(o[:, :L] != 0, ref)
        assert np.all(o[:, L:] == 0)
        np.testing.assert_allclose(o[:, :L][ref], np.repeat(1.0 / cnt, ref.sum(1)), rtol=1e-6, atol=0)


# ------------------------------------------------------------------ values


PARITY = [
    # B, L, Hq, Hkv, d, w, s, conv, std, boost_n
    (2, 300, 8, 2, 128, 64, 4, 0, 1.0, 4),
    (1, 1000, 32, 8, 128, 64, 4, 0, 0.5, 4),
    (2, 777, 32, 8, 128, 128, 4, 0, 1.0, 4),
    (1, 1000, 16, 4, 128, 256, 0, 0, 1.0, 4),
    (1, 1100, 8, 2, 128, 512, 4, 0, 1.0, 4),
    (1, 1500, 8, 2, 128, 1000, 4, 0, 1.0, 0),
    # the resident form (every q-tile within four 32-key chunks): two sink chunks, a full sink
    # chunk, the total-window convention at d = 64, w = 1 with one head per kv-head
    (1, 97, 8, 2, 128, 33, 64, 0, 1.0, 4),
    (2, 257, 4, 1, 128, 64, 32, 0, 1.0, 4),
    (1, 200, 16, 4, 64, 64, 4, 1, 1.0, 4),
    (1, 130, 2, 2, 128, 1, 0, 0, 1.0, 0),
    # windows of 1000+ keys at d = 128: long runs of middle tiles, ragged tails, G = 4, 2, 1
    (1, 2600, 8, 2, 128, 1024, 4, 0, 1.0, 4),
    (2, 1300, 6, 3, 128, 1100, 0, 1, 1.0, 0),
    (1, 1200, 2, 2, 128, 2000, 3, 0, 1.0, 4),
    (1, 200, 12, 4, 128, 33, 70, 0, 1.0, 4),
    (1, 333, 16, 2, 64, 50, 5, 1, 1.0, 4),
    (1, 129, 4, 4, 64, 1, 0, 0, 1.0, 0),
    (1, 1, 4, 1, 128, 64, 4, 0, 1.0, 4),
    (1, 64, 4, 1, 128, 1000, 0, 0, 1.0, 0),
    (3, 190, 6, 3, 64, 17, 2, 0, 2.0, 4),
    (1, 513, 5, 1, 128, 100, 1, 0, 1.0, 4),
    # the resident form (G = 4) at d = 64: a last q-tile of one token
    (3, 161, 8, 2, 64, 64, 4, 0, 1.0, 4),
    # the 128-row tile walk (512 workgroups and more; the smaller grids above take the 64-row
    # walk or a resident form): G = 4, 2 and 1, both head sizes, both conventions, ragged tails
    (8, 1100, 8, 2, 128, 512, 4, 0, 1.0, 4),
    (5, 1300, 12, 6, 64, 300, 0, 1, 1.0, 0),
    (2, 2100, 16, 16, 128, 1000, 3, 0, 1.0, 4),
    # the 64-row tile walk at d = 64 (16-token q-tiles, a window past four chunks)
    (2, 700, 8, 2, 64, 300, 4, 0, 1.0, 4),
]

# Many 32-token q-tiles per kv-head in the 128-row resident form (grids of 512 workgroups and
# more): ragged last q-tiles, both head sizes, both window conventions, sinks in a chunk of
# their own, batches.  The 64-row resident form (smaller grids) runs in most PARITY cases.
RESIDENT_LARGE = [
    # B, L, Hq, Hkv, d, w, s, conv, std, boost_n
    (1, 4113, 32, 8, 128, 64, 4, 0, 1.0, 4),
    (4, 1100, 16, 4, 64, 40, 8, 0, 1.0, 4),
    (2, 2053, 32, 8, 128, 96, 0, 0, 1.0, 0),
    (1, 2048, 32, 8, 128, 68, 4, 1, 1.0, 4),
    (2, 4096, 32, 8, 64, 33, 30, 0, 0.5, 4),
]


def check_close(got, ref, what, parity=None):
    err = np.abs(got - ref)
    say(f"{what}: max {err.max():.3e} mean {err.mean():.3e} p99.9 {np.percentile(err, 99.9):.3e}")
    if parity is not None:
        parity(what, err)
    assert np.isfinite(got).all()
    assert err.max() <= TOL, what


@pytest.mark.parametrize("B,L,Hq,Hkv,d,w,s,conv,std,boost", PARITY)
def test_prefill_matches_oracle(B, L, Hq, Hkv, d, w, s, conv, std, boost, parity):
    say("parity", B, L, Hq, Hkv, d, w, s, conv)
    q, k, v = inputs.random_qkv(B, L, Hq, Hkv, d, seed=L + 17 * w + s, std=std, sink_boost_n=boost, sink_boost=4.0)
    scale = 1.0 / np.sqrt(d)
    out = swa.prefill(q.cuda(), k.cuda(), v.cuda(), w, s, scale, conv).cpu().numpy()
    ref = orc.prefill(f64(q), f64(k), f64(v), w, s, scale, conv)
    check_close(out, ref, "prefill parity cases (all elements)", parity)


@pytest.mark.parametrize("B,L,Hq,Hkv,d,w,s,conv,std,boost", RESIDENT_LARGE)
def test_resident_form_large_matches_oracle(B, L, Hq, Hkv, d, w, s, conv, std, boost, parity):
    info = swa.prefill_describe(B, Hq, Hkv, L, d, w, s, conv)
    say("resident large", B, L, Hq, Hkv, d, w, s, conv, info)
    assert info["form"] == 1
    q, k, v = inputs.random_qkv(B, L, Hq, Hkv, d, seed=L + 31 * w + s, std=std, sink_boost_n=boost, sink_boost=4.0)
    scale = 1.0 / np.sqrt(d)
    out = swa.prefill(q.cuda(), k.cuda(), v.cuda(), w, s, scale, conv).cpu().numpy()
    ref = orc.prefill(f64(q), f64(k), f64(v), w, s, scale, conv)
    check_close(out, ref, "prefill resident form, large (all elements)", parity)


def test_tiny_workload_full_parity(parity):
    wl = inputs.prefill_workloads()["tiny_swa64_4"]
    q, k, v = inputs.prefill_inputs(wl)
    out = swa.prefill(q.cuda(), k.cuda(), v.cuda(), wl.w, wl.s, wl.scale).cpu().numpy()
    ref = orc.prefill(f64(q), f64(k), f64(v), wl.w, wl.s, wl.scale)
    check_close(out, ref, f"{wl.name} prefill (all elements)", parity)


def sample_rows(L, w_loc, s, rng, n_random=12):
    fixed = [0, 1, 2, 3, 4, 5, 31, 32, 63, 64, 65, 66, 67, 68, 127, 128, w_loc - 1, w_loc, w_loc + 1,
             w_loc + s, w_loc + s + 1, L // 2, L - 65, L - 2, L - 1]
    rows = {t for t in fixed if 0 <= t < L}
    rows |= set(int(x) for x in rng.integers(0, L, n_random))
    return sorted(rows)


def oracle_rows(q, k, v, b, rows, w, s, conv, scale):
    """Oracle rows for sampled positions, each from the sinks plus a margin below the window
    (entries outside A(t) are dropped by the oracle's own predicate)."""
    w_loc = orc.local_window(w, s, conv)
    out = {}
    for t in rows:
        cand = sorted(set(range(min(s, t + 1))) | set(range(max(0, t - w_loc - 2), t + 1)))
        out[t], used = orc.decode_row(f64(q[b, t]), cand, f64(k[b, cand]), f64(v[b, cand]), t, w, s, scale, conv)
        assert used == min(t + 1, w_loc + s)
    return out


@pytest.mark.parametrize("name", [n for n in inputs.prefill_workloads() if n != "tiny_swa64_4"])
def test_full_size_workloads_sampled_rows(name, parity):
    """Full-size workloads in the benchmark's launch configuration, checked on sampled rows."""
    wl = inputs.prefill_workloads()[name]
    say("full", name)
    q, k, v = inputs.prefill_inputs(wl)
    out = swa.prefill(q.cuda(), k.cuda(), v.cuda(), wl.w, wl.s, wl.scale, wl.conv).cpu()
    assert torch.isfinite(out).all()
    rng = np.random.default_rng(wl.seed)
    w_loc = orc.local_window(wl.w, wl.s, wl.conv)
    for b in sorted({0, wl.B - 1}):
        rows = sample_rows(wl.L, w_loc, wl.s, rng)
        ref = oracle_rows(q, k, v, b, rows, wl.w, wl.s, wl.conv, wl.scale)
        got = np.stack([out[b, t].numpy() for t in rows])
        check_close(got, np.stack([ref[t] for t in rows]), f"{name} prefill (sampled rows)", parity)


@pytest.mark.parametrize("w,s,form", [(64, 4, 1), (1000, 4, 0)])
def test_longest_sequence_sampled_rows(w, s, form, parity):
    """Two sequences, each of the most q elements the boundary accepts (L Hq d = 2^31 - 1024 at
    Hq = 8, d = 128: L = 2,097,151, a ragged last q-tile): the second sequence's q, k, v and
    output start past 2^31 elements and its output past 2^33 bytes.  The resident form and the
    tile walk, checked on sampled rows of both sequences."""
    B, Hq, Hkv, d = 2, 8, 2, 128
    L = (2 ** 31 - 1) // (Hq * d)
    assert swa.prefill_describe(B, Hq, Hkv, L, d, w, s)["form"] == form
    say("longest", B, L, Hq, Hkv, d, w, s)
    q, k, v = inputs.random_qkv_device(B, L, Hq, Hkv, d, seed=77, device="cuda", sink_boost_n=4, sink_boost=4.0)
    scale = 1.0 / np.sqrt(d)
    out = swa.prefill(q, k, v, w, s, scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    rng = np.random.default_rng(77)
    for b in range(B):
        rows = sample_rows(L, w, s, rng) + [L - 33, L - 32, L - 31]
        rows = sorted(set(rows))
        ref = oracle_rows(q, k, v, b, rows, w, s, 0, scale)
        got = out[b, rows].cpu().numpy()
        check_close(got, np.stack([ref[t] for t in rows]), "prefill at the longest sequence (sampled rows)", parity)
    del q, k, v, out
    torch.cuda.empty_cache()


def test_prefill_is_deterministic_and_keeps_guard_bands():
    B, L, Hq, Hkv, d = 1, 700, 32, 8, 128
    q, k, v = [t.cuda() for t in inputs.random_qkv(B, L, Hq, Hkv, d, seed=5, sink_boost_n=4, sink_boost=4.0)]
    n = B * L * Hq * d
    guard = 1024
    buf = torch.full((n + 2 * guard,), float("nan"), dtype=torch.float32, device="cuda")
    out = buf[guard:guard + n].view(B, L, Hq, d)
    swa.prefill(q, k, v, 64, 4, out=out)
    first = out.clone()
    swa.prefill(q, k, v, 64, 4, out=out)
    assert torch.equal(first, out)
    assert torch.isfinite(out).all()
    assert torch.isnan(buf[:guard]).all() and torch.isnan(buf[guard + n:]).all()


def test_prefill_on_a_side_stream():
    q, k, v = [t.cuda() for t in inputs.random_qkv(1, 256, 8, 2, 128, seed=8)]
    ref = swa.prefill(q, k, v, 32, 4)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out = swa.prefill(q, k, v, 32, 4)
    s.synchronize()
    assert torch.equal(out, ref)


def test_timed_prefill_matches_and_stamps_kernel_time():
    q, k, v = [t.cuda() for t in inputs.random_qkv(1, 1024, 32, 8, 128, seed=12, sink_boost_n=4, sink_boost=4.0)]
    ref = swa.prefill(q, k, v, 64, 4)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    e1.record()
    out = swa.prefill(q, k, v, 64, 4, events=(e0, e1))
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert e0.elapsed_time(e1) > 0


def _random_cases(n, seed):
    """Shapes drawn from a fixed generator: every run checks the same cases."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 3, 4, 6, 8]))
        d = int(rng.choice([64, 128]))
        L = int(rng.integers(1, 700))
        w = int(rng.integers(1, 400))
        s = int(rng.integers(0, 12))
        conv = int(rng.integers(0, 2))
        if conv == 1 and w - s < 1:
            w = s + 1 + int(rng.integers(0, 50))
        B = int(rng.integers(1, 3))
        cases.append((B, L, G * Hkv, Hkv, d, w, s, conv))
    return cases


@pytest.mark.parametrize("B,L,Hq,Hkv,d,w,s,conv", _random_cases(12, 20261203))
def test_prefill_matches_oracle_on_drawn_shapes(B, L, Hq, Hkv, d, w, s, conv, parity):
    say("drawn", B, L, Hq, Hkv, d, w, s, conv)
    q, k, v = inputs.random_qkv(B, L, Hq, Hkv, d, seed=L * 7 + w, std=1.0, sink_boost_n=4, sink_boost=4.0)
    scale = 1.0 / np.sqrt(d)
    ref = orc.prefill(f64(q), f64(k), f64(v), w, s, scale, conv)
    got = swa.prefill(q.cuda(), k.cuda(), v.cuda(), w, s, scale, conv).cpu().numpy()
    check_close(got, ref, "prefill drawn shapes (all elements)", parity)
