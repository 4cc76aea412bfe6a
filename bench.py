"""Benchmark: SWA(w,s) prefill useful TFLOP/s + decode tokens/s on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
  * prefill of the Mistral-7B-shaped workload (B=1, L=16384, Hq=32, Hkv=8, d=128, SWA(4096,4),
    bf16 N(0,1) inputs, fp32 output), one swa_prefill launch, with L2 and the Infinity Cache
    evicted first (a 512 MiB buffer overwritten) so that q, k and v come from HBM;
  * 256 decode tokens of the SWA(64,4) ring-cache workload at batch 64 (Hq=32, Hkv=8, d=128),
    each token one swa_append_decode_step (append + attend in one launch), positions
    2^18 .. 2^18+255, the steps rotating over 32 independent caches (570 MB, over twice the
    Infinity Cache, so every step reads its cache from HBM), captured once in a HIP graph.
Inputs are resident in HBM before the timed region, which is bracketed by
torch.cuda.synchronize(); inside it, the prefill kernel stamps a pair of HIP events with its own
start and end (swa_prefill_timed), and HIP events on the stream bracket every decode replay.

Printed JSON line (one):
  value            prefill useful TFLOP/s = 4*d*Hq*B*sum_t |A(t)| / mean prefill kernel time (cold)
  roofline         the prefill kernel against the bf16 dense MFMA peak (this workload does ~2050
                   useful flop per algorithmic byte, far above the 315 flop/byte ridge); traffic:
                   HBM bytes per launch from the committed counter summary of the same kernel source
  decode           tokens/s of the decode leg (graph replay) and its KV bandwidth; kernel_only: the
                   same launches made one by one, each stamped by its own dispatch
                   (swa_append_decode_step_timed); secondary figures: the cache-resident set, batch
                   1 and batch 1024
  roofline_decode  the decode kernel against HBM peak: graph step and kernel-only
  prefill.others   the other prefill workloads (Llama SWA(64,4), the window sweep), cold and warm,
                   with the fraction of their attainable roofline min(MFMA peak, AI x HBM peak)
  cpu_baseline     the fp64 oracle timed on the host cores on a bounded sample of the same
                   prefill workload (the last rows of the sequence, every head), all allowed
                   threads and one thread
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PROFILES = os.path.join(ROOT, "profiles")
PREFILL_SRC = os.path.join(ROOT, "sliding_window_attention_02_amd", "csrc", "swa_prefill.hip")
DEVICE_SRC = os.path.join(ROOT, "sliding_window_attention_02_amd", "csrc", "swa_device.h")


def kernel_source_digest() -> str:
    """Digest of the prefill kernel's code: its sources with comments and blank space removed,
    so that a profile stays matched to the code it measured across comment-only edits."""
    h = hashlib.sha256()
    for p in (PREFILL_SRC, DEVICE_SRC):
        with open(p, encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("\n".join(" ".join(line.split()) for line in text.splitlines() if line.strip()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per prefill launch from the committed rocprofv3 counter summary, or None
    when the summary is missing or was taken on a different kernel source."""
    path = os.path.join(PROFILES, f"prefill_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"kernel source digest:\s*([0-9a-f]+)", text)
    m_b = re.search(r"HBM bytes per launch \(calibrated\):\s*([0-9]+)", text)
    if not m_src or not m_b or m_src.group(1) != kernel_source_digest():
        return None
    return int(m_b.group(1))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mistral7b_w4096_s4", help="prefill workload of the step")
    ap.add_argument("--other-workloads", default="llama8b_swa64_4,sweep_w512_s4,sweep_w256_s4,sweep_w128_s4",
                    help="secondary prefill workloads, timed cold and warm outside the steps")
    ap.add_argument("--decode-batch", type=int, default=64)
    ap.add_argument("--decode-tokens", type=int, default=256)
    ap.add_argument("--decode-start", type=int, default=2 ** 18)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the measurements outside the steps (other decode batches, cold prefill)")
    ap.add_argument("--cpu-threads", type=int, default=0, help="oracle threads (0: min(16, cores))")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this size (counter calibration)")
    ap.add_argument("--prefill-only", default="", help="only time this prefill workload (profiling)")
    ap.add_argument("--cold", action="store_true", help="with --prefill-only: evict the caches before each launch")
    ap.add_argument("--decode-only", type=int, default=0, help="only time the decode graph at this batch (profiling)")
    ap.add_argument("--chunked", default="", help="only time this prefill workload fed in chunks (swa_prefill_chunk)")
    ap.add_argument("--chunk", type=int, default=4096, help="with --chunked: tokens per chunk")
    ap.add_argument("--compare-full", action="store_true", help="only time SWA against full causal attention")
    ap.add_argument("--cache-sets", type=int, default=32, help="caches the decode steps rotate over")
    ap.add_argument("--eager", action="store_true",
                    help="with --decode-only: launch the steps one by one, each stamped by its dispatch")
    ap.add_argument("--model-sweep", action="store_true",
                    help="only time decode of a 4-layer decoder (Llama-3.1-8B layer shape, batch 1) against context")
    ap.add_argument("--model-layers", type=int, default=4)
    ap.add_argument("--model-tokens", type=int, default=8, help="with --model-sweep: tokens per HIP graph")
    ap.add_argument("--model-contexts", default="128,1024,4096,16384,65536,262144")
    return ap.parse_args()


def copy_probe(mib: int):
    import torch
    n = mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_each_way": n * 4, "launches": 3}))


def host_cpu():
    """(logical CPUs the process may use, CPU model name) of this host."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return len(os.sched_getaffinity(0)), model


def cpu_baseline(wl, q, k, v, threads: int, target_s: float = 6.0, reps: int = 3):
    """The oracle as it stands on the host cores, on a bounded sample of the prefill workload:
    the last R rows of every sequence and head (rows whose window is full), R sized from a short
    calibration so that one pass takes about target_s; the median of `reps` passes; then the
    same with one thread on a smaller sample.  Useful TFLOP/s of the sample, the workload's own
    unit."""
    from oracle import oracle as orc

    w_loc = wl.w if wl.conv == 0 else wl.w - wl.s
    qd, kd, vd = (t.double().numpy() for t in (q, k, v))

    def run(rows: int, nth: int):
        t0 = time.perf_counter()
        orc.prefill_rows(qd, kd, vd, wl.L - rows, wl.L, wl.w, wl.s, wl.scale, wl.conv, nthreads=nth)
        dt = time.perf_counter() - t0
        pairs = sum(min(t + 1, w_loc + wl.s) for t in range(wl.L - rows, wl.L)) * wl.Hq * wl.B
        return 4 * wl.d * pairs / dt / 1e12, dt

    def sized(nth: int, budget: float, first: int):
        _, dt = run(first, nth)  # calibration
        rows = max(first, min(wl.L, int(first * budget / max(dt, 1e-3))))
        passes = sorted(run(rows, nth) for _ in range(reps))
        tf, dt = passes[len(passes) // 2]
        return tf, dt, rows, sorted(round(p[1], 2) for p in passes)

    tf_n, dt_n, rows_n, secs_n = sized(threads, target_s, 32)
    tf_1, dt_1, rows_1, secs_1 = sized(1, target_s / 3, 4)
    nproc, model = host_cpu()
    return {"value": round(tf_n, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"rows {wl.L - rows_n}..{wl.L - 1} of the {wl.name} prefill (B={wl.B}, every one of "
                      f"Hq={wl.Hq} heads, d={wl.d}, SWA({wl.w},{wl.s}), fp64 C oracle), median of {reps} passes "
                      f"of {dt_n:.1f} s on {threads} threads; useful flops of the sample / time",
            "pass_seconds": secs_n,
            "single_thread": {"value": round(tf_1, 6), "rows": rows_1, "seconds": round(dt_1, 2),
                              "pass_seconds": secs_1},
            "host_nproc": nproc, "cpu_model": model}


def decode_graph(swa, inputs, dw, B: int, T: int, P: int, dev, n_sets: int = 1):
    """A HIP graph of T decode steps of workload dw at batch B, each step one
    swa_append_decode_step (append the token's K/V to its slot and attend), and a function that
    restores the caches to their state after position P-1 (run it before every replay, so each
    replay decodes the same tokens).  Every input is seeded: a cache holds the sinks and
    positions max(s, P-w_loc) .. P-1.  With n_sets > 1 the steps rotate over that many independent
    caches (step i uses cache i % n_sets at position P + i // n_sets), so that consecutive steps
    never find their cache in the Infinity Cache once n_sets caches exceed it."""
    import torch

    w_loc = dw.w if dw.conv == 0 else dw.w - dw.s
    gen = dict(B=B, Hkv=dw.Hkv, d=dw.d, std=dw.std, sink_boost_n=dw.sink_boost_n, sink_boost=dw.sink_boost)
    kc, vc = swa.alloc_cache(B, dw.Hkv, dw.d, dw.w, dw.s, dw.conv, device=dev)
    ws = swa.alloc_workspace(B, dw.Hq, dw.Hkv, dw.d, dw.w, dw.s, dw.conv, device=dev)
    lo = max(dw.s, P - w_loc)  # first window position in the cache after P-1
    seed_pos = list(range(min(dw.s, P))) + list(range(lo, P))
    sk, sv = inputs.kv_span(dw.seed, seed_pos, **gen)
    n_sink = min(dw.s, P)
    if n_sink > 0:
        swa.kv_append(kc, vc, sk[:, :n_sink].contiguous().to(dev), sv[:, :n_sink].contiguous().to(dev),
                      torch.zeros(B, dtype=torch.int64, device=dev), dw.w, dw.s, dw.conv)
    if P > lo:
        swa.kv_append(kc, vc, sk[:, n_sink:].contiguous().to(dev), sv[:, n_sink:].contiguous().to(dev),
                      torch.full((B,), lo, dtype=torch.int64, device=dev), dw.w, dw.s, dw.conv)
    snap_k, snap_v = kc.clone(), vc.clone()
    caches = [(kc, vc)] + [(snap_k.clone(), snap_v.clone()) for _ in range(n_sets - 1)]
    n_pos = (T + n_sets - 1) // n_sets
    dq = torch.stack([inputs.q_at(dw.seed, P + i, B, dw.Hq, dw.d, dw.std) for i in range(n_pos)]).to(dev)
    kvs = [inputs.kv_at(dw.seed, P + i, **gen) for i in range(n_pos)]
    dk = torch.stack([x[0] for x in kvs]).to(dev)  # [n_pos][B][Hkv][d]
    dv = torch.stack([x[1] for x in kvs]).to(dev)
    dpos = (P + torch.arange(n_pos, dtype=torch.int64)).repeat_interleave(B).view(n_pos, B).to(dev)
    dout = torch.empty((T, B, dw.Hq, dw.d), dtype=torch.float32, device=dev)

    def steps():
        for i in range(T):
            ck, cv = caches[i % n_sets]
            j = i // n_sets
            swa.append_decode_step(dq[j], ck, cv, dk[j], dv[j], dpos[j], dw.w, dw.s, dw.scale, dw.conv,
                                   out=dout[i], workspace=ws)

    def restore():
        for ck, cv in caches:
            ck.copy_(snap_k)
            cv.copy_(snap_v)

    stream = torch.cuda.Stream(device=dev)
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        steps()  # eager warm-up on the capture stream
    stream.synchronize()
    restore()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        steps()
    torch.cuda.synchronize()
    return graph, restore


def decode_point(swa, inputs, acc, dw, B: int, T: int, P: int, dev, reps: int = 5, n_sets: int = 1):
    """Per-token step time of the decode graph at batch B (not part of the bench step)."""
    import torch

    graph, restore = decode_graph(swa, inputs, dw, B, T, P, dev, n_sets)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ms = []
    for _ in range(reps + 1):
        restore()
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    step_us = sum(ms[1:]) / reps * 1e3 / T
    w_loc = dw.w if dw.conv == 0 else dw.w - dw.s
    kv = acc.decode_kv_bytes(B, dw.Hkv, dw.d, acc.decode_keys(P, w_loc, dw.s))
    gbs = kv / (step_us * 1e-6) / 1e9
    # every byte the step moves: the KV reads plus q, the new token's K/V (read and written to
    # the cache) and the fp32 output
    all_gbs = (kv + acc.decode_other_bytes(B, dw.Hq, dw.Hkv, dw.d)) / (step_us * 1e-6) / 1e9
    rec = {"B": B, "us_per_token_step": round(step_us, 3), "tokens_per_s": round(B / (step_us * 1e-6), 1),
           "kv_gb_per_s": round(gbs, 2), "frac_of_hbm_peak": round(gbs / acc.PEAK_HBM_GBS, 5),
           "all_bytes_gb_per_s": round(all_gbs, 2), "all_bytes_frac_of_hbm_peak": round(all_gbs / acc.PEAK_HBM_GBS, 5)}
    if n_sets > 1:
        rec["cache_sets"] = n_sets
    return rec


def decode_kernel_only(swa, inputs, acc, dw, B: int, T: int, P: int, dev, n_sets: int = 32):
    """The decode launches of decode_graph made one by one (no graph), each stamped with its own
    kernel start and end by its dispatch (swa_append_decode_step_timed): mean kernel time and the
    KV bandwidth it implies."""
    import torch

    w_loc = dw.w if dw.conv == 0 else dw.w - dw.s
    gen = dict(B=B, Hkv=dw.Hkv, d=dw.d, std=dw.std, sink_boost_n=dw.sink_boost_n, sink_boost=dw.sink_boost)
    kc, vc = swa.alloc_cache(B, dw.Hkv, dw.d, dw.w, dw.s, dw.conv, device=dev)
    ws = swa.alloc_workspace(B, dw.Hq, dw.Hkv, dw.d, dw.w, dw.s, dw.conv, device=dev)
    lo = max(dw.s, P - w_loc)
    seed_pos = list(range(min(dw.s, P))) + list(range(lo, P))
    sk, sv = inputs.kv_span(dw.seed, seed_pos, **gen)
    n_sink = min(dw.s, P)
    swa.kv_append(kc, vc, sk[:, :n_sink].contiguous().to(dev), sv[:, :n_sink].contiguous().to(dev),
                  torch.zeros(B, dtype=torch.int64, device=dev), dw.w, dw.s, dw.conv)
    swa.kv_append(kc, vc, sk[:, n_sink:].contiguous().to(dev), sv[:, n_sink:].contiguous().to(dev),
                  torch.full((B,), lo, dtype=torch.int64, device=dev), dw.w, dw.s, dw.conv)
    caches = [(kc, vc)] + [(kc.clone(), vc.clone()) for _ in range(n_sets - 1)]
    n_pos = (T + n_sets - 1) // n_sets
    dq = torch.stack([inputs.q_at(dw.seed, P + i, B, dw.Hq, dw.d, dw.std) for i in range(n_pos)]).to(dev)
    kvs = [inputs.kv_at(dw.seed, P + i, **gen) for i in range(n_pos)]
    dk = torch.stack([x[0] for x in kvs]).to(dev)
    dv = torch.stack([x[1] for x in kvs]).to(dev)
    dpos = (P + torch.arange(n_pos, dtype=torch.int64)).repeat_interleave(B).view(n_pos, B).to(dev)
    out = torch.empty((B, dw.Hq, dw.d), dtype=torch.float32, device=dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(T)] for _ in range(2)]
    for e in evs[0] + evs[1]:
        e.record()
    torch.cuda.synchronize()
    for i in range(T):
        ck, cv = caches[i % n_sets]
        j = i // n_sets
        swa.append_decode_step(dq[j], ck, cv, dk[j], dv[j], dpos[j], dw.w, dw.s, dw.scale, dw.conv, out=out,
                               workspace=ws, events=(evs[0][i], evs[1][i]))
    torch.cuda.synchronize()
    us = sorted(evs[0][i].elapsed_time(evs[1][i]) * 1e3 for i in range(T))
    mean = sum(us) / T
    kv = acc.decode_kv_bytes(B, dw.Hkv, dw.d, acc.decode_keys(P, w_loc, dw.s))
    return {"B": B, "launches": T, "cache_sets": n_sets, "mean_kernel_us": round(mean, 3),
            "median_kernel_us": round(us[T // 2], 3), "kv_gb_per_s": round(kv / (mean * 1e-6) / 1e9, 2),
            "frac_of_hbm_peak": round(kv / (mean * 1e-6) / 1e9 / acc.PEAK_HBM_GBS, 5)}


def flush_buffer(dev, mib: int = 512):
    """A buffer whose fill evicts the 4 MB L2s and the 256 MB Infinity Cache."""
    import torch

    return torch.empty(mib * (1 << 20) // 4, dtype=torch.float32, device=dev)


def prefill_timing(swa, wl, qg, kg, vg, out, reps: int, warmup: int, flush=None):
    """Kernel-stamped launch times (ms) of `reps` prefills; with `flush`, the caches are
    evicted (the buffer is overwritten) before every launch."""
    import torch

    for _ in range(warmup):
        swa.prefill(qg, kg, vg, wl.w, wl.s, wl.scale, wl.conv, out=out)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(reps)] for _ in range(2)]
    for e in evs[0] + evs[1]:
        e.record()
    torch.cuda.synchronize()
    for i in range(reps):
        if flush is not None:
            flush.fill_(float(i))
        swa.prefill(qg, kg, vg, wl.w, wl.s, wl.scale, wl.conv, out=out, events=(evs[0][i], evs[1][i]))
    torch.cuda.synchronize()
    return [evs[0][i].elapsed_time(evs[1][i]) for i in range(reps)]


def prefill_only(args, dev):
    """--prefill-only WORKLOAD: time that prefill alone (warm, and with --cold caches evicted
    before every launch) and print one JSON line."""
    import torch

    import sliding_window_attention_02_amd as swa
    from sliding_window_attention_02_amd import accounting as acc
    from sliding_window_attention_02_amd import inputs

    wl = inputs.prefill_workloads()[args.prefill_only]
    w_loc = wl.w if wl.conv == 0 else wl.w - wl.s
    q, k, v = inputs.prefill_inputs(wl)
    qg, kg, vg = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty((wl.B, wl.L, wl.Hq, wl.d), dtype=torch.float32, device=dev)
    flush = flush_buffer(dev) if args.cold else None
    ms = prefill_timing(swa, wl, qg, kg, vg, out, args.steps, args.warmup, flush)
    mean = sum(ms) / len(ms)
    useful = acc.useful_flops(wl.B, wl.Hq, wl.L, wl.d, w_loc, wl.s)
    algo = acc.prefill_bytes(wl.B, wl.L, wl.Hq, wl.Hkv, wl.d)
    tf = useful / (mean * 1e-3) / 1e12
    gbs = algo / (mean * 1e-3) / 1e9
    print(json.dumps({"workload": wl.name, "caches": "evicted before each launch" if args.cold else "warm",
                      "launches": len(ms), "mean_launch_us": round(mean * 1e3, 3),
                      "useful_tflops": round(tf, 3), "frac_of_bf16_mfma_peak": round(tf / acc.PEAK_BF16_TFLOPS, 5),
                      "algorithmic_gb_per_s": round(gbs, 2), "frac_of_hbm_peak": round(gbs / acc.PEAK_HBM_GBS, 5)}),
          flush=True)


def chunked_only(args, dev):
    """--chunked WORKLOAD --chunk C: the workload's sequences fed to swa_prefill_chunk in chunks
    of C tokens from an empty cache (every chunk call captured in one HIP graph; the cache is
    cleared before each replay), against the whole-sequence prefill.  One JSON line."""
    import torch

    import sliding_window_attention_02_amd as swa
    from sliding_window_attention_02_amd import accounting as acc
    from sliding_window_attention_02_amd import inputs

    wl = inputs.prefill_workloads()[args.chunked]
    w_loc = wl.w if wl.conv == 0 else wl.w - wl.s
    C = args.chunk
    q, k, v = inputs.prefill_inputs(wl)
    qg, kg, vg = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty((wl.B, wl.L, wl.Hq, wl.d), dtype=torch.float32, device=dev)
    kc, vc = swa.alloc_cache(wl.B, wl.Hkv, wl.d, wl.w, wl.s, wl.conv, device=dev)
    starts = list(range(0, wl.L, C))
    pieces = [(p, min(C, wl.L - p)) for p in starts]
    qs = [qg[:, p:p + n].contiguous() for p, n in pieces]
    ks = [kg[:, p:p + n].contiguous() for p, n in pieces]
    vs = [vg[:, p:p + n].contiguous() for p, n in pieces]
    outs = [torch.empty((wl.B, n, wl.Hq, wl.d), dtype=torch.float32, device=dev) for _, n in pieces]

    def run():
        for i, (p, n) in enumerate(pieces):
            swa.prefill_chunk(qs[i], ks[i], vs[i], kc, vc, p, wl.w, wl.s, wl.scale, wl.conv, out=outs[i])

    stream = torch.cuda.Stream(device=dev)
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        run()
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ms = []
    for _ in range(args.warmup + args.steps):
        kc.zero_()
        vc.zero_()
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    chunked = sum(ms[args.warmup:]) / args.steps
    whole = sum(prefill_timing(swa, wl, qg, kg, vg, out, args.steps, args.warmup)) / args.steps
    useful = acc.useful_flops(wl.B, wl.Hq, wl.L, wl.d, w_loc, wl.s)
    print(json.dumps({"workload": wl.name, "chunk": C, "chunks": len(pieces), "chunked_ms": round(chunked, 4),
                      "chunked_useful_tflops": round(useful / (chunked * 1e-3) / 1e12, 3),
                      "whole_sequence_ms": round(whole, 4),
                      "whole_sequence_useful_tflops": round(useful / (whole * 1e-3) / 1e12, 3),
                      "chunked_over_whole": round(chunked / whole, 3)}), flush=True)


def compare_full(args, dev):
    """--compare-full: SWA against full causal attention with the same kernels (full attention
    is SWA with a window covering the whole sequence or context).  Prefill: the Mistral-shaped
    workload with w=4096 and with w >= L.  Decode at batch 1: SWA(64,4) on its 68-slot ring
    against a growing cache holding every position up to the context, at contexts 2^7 .. 2^17,
    64 append+attend steps each (one HIP graph).  One JSON line; every input is seeded."""
    import math

    import torch

    import sliding_window_attention_02_amd as swa
    from sliding_window_attention_02_amd import accounting as acc
    from sliding_window_attention_02_amd import inputs

    rec = {"prefill": {}, "decode": []}
    wl = inputs.prefill_workloads()["mistral7b_w4096_s4"]
    q, k, v = inputs.prefill_inputs(wl)
    qg, kg, vg = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty((wl.B, wl.L, wl.Hq, wl.d), dtype=torch.float32, device=dev)
    for name, w, s in (("swa_w4096_s4", wl.w, wl.s), ("full_causal", wl.L, 0)):
        cfg = type("W", (), dict(w=w, s=s, scale=wl.scale, conv=0))
        ms = prefill_timing(swa, cfg, qg, kg, vg, out, args.steps, args.warmup)
        mean = sum(ms) / len(ms)
        useful = acc.useful_flops(wl.B, wl.Hq, wl.L, wl.d, w, s)
        rec["prefill"][name] = {"ms": round(mean, 4), "useful_tflops": round(useful / (mean * 1e-3) / 1e12, 2)}
    rec["prefill"]["full_over_swa"] = round(rec["prefill"]["full_causal"]["ms"] / rec["prefill"]["swa_w4096_s4"]["ms"], 3)

    dw = inputs.decode_workloads()["decode_swa64_4_b1"]
    T = 64
    for e in range(7, 18):
        P = 2 ** e
        swa_pt = decode_point(swa, inputs, acc, dw, 1, T, P, dev, reps=3)
        # Full attention: s = 0 and a local window of P + T slots, so the cache grows with the
        # context and no position is evicted (slot p holds position p).
        full = type("D", (), dict(w=P + T, s=0, conv=0, Hq=dw.Hq, Hkv=dw.Hkv, d=dw.d, std=dw.std,
                                  sink_boost_n=dw.sink_boost_n, sink_boost=dw.sink_boost, seed=dw.seed,
                                  scale=dw.scale))
        full_pt = decode_point(swa, inputs, acc, full, 1, T, P, dev, reps=3)
        rec["decode"].append({"context": P, "swa_us_per_step": swa_pt["us_per_token_step"],
                              "full_us_per_step": full_pt["us_per_token_step"],
                              "full_kv_gb_per_s": full_pt["kv_gb_per_s"]})
    print(json.dumps(rec), flush=True)


def model_sweep(args, dev):
    """--model-sweep: decode throughput and KV state memory of a stack of decoder layers at
    batch 1 against context length, the measurement the pages report for a 4-layer Transformer
    (128 to 256K tokens of context).  Layers have the Llama-3.1-8B shape (dm 4096, 32 q-heads,
    8 kv-heads, d 128, SwiGLU 14336) with seeded random bf16 weights; attention is SWA(w,4) on a
    sink + ring cache for w in 64..512, full attention (a cache holding every position), or a
    hybrid stack (every layer SWA(64,4) but the last, which is full).  Each point is a HIP graph
    of T tokens, every token one swa_stack_decode_step through the layers; caches hold seeded random
    keys and values for the positions before the context.  One JSON line."""
    import math

    import torch

    import sliding_window_attention_02_amd as swa
    from sliding_window_attention_02_amd import inputs

    nl = args.model_layers
    dm, Hq, Hkv, d, f = 4096, 32, 8, 128, 14336
    B, T, eps, seed = 1, args.model_tokens, 1e-5, 2026
    scale = 1.0 / math.sqrt(d)
    weights = [{k: v.to(dev) for k, v in inputs.layer_weights(seed, li, dm, Hq, Hkv, d, f).items()}
               for li in range(nl)]
    weight_bytes = sum(v.numel() * 2 for w in weights for v in w.values())
    rec = {"model": {"layers": nl, "dm": dm, "Hq": Hq, "Hkv": Hkv, "d": d, "f": f, "batch": B,
                     "weight_gb": round(weight_bytes / 1e9, 4), "tokens_per_graph": T}, "points": []}

    # Streaming bandwidth of the linear kernel on the largest matrix (gate and up, 235 MB),
    # rotating over the layers so that no launch finds its weights in the Infinity Cache.
    h = torch.randn(B, dm, device=dev).to(torch.bfloat16)
    act = torch.empty(B, f, dtype=torch.bfloat16, device=dev)
    for li in range(nl):
        swa.linear(weights[li]["w_gate_up"], h, "silu_mul", out=act)
    reps = 5
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        for li in range(nl):
            swa.linear(weights[li]["w_gate_up"], h, "silu_mul", out=act)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * nl)
    gu_bytes = 2 * f * dm * 2
    rec["linear_gate_up"] = {"us_per_launch": round(us, 2), "gb_per_s": round(gu_bytes / (us * 1e-6) / 1e9, 1),
                             "frac_of_hbm_peak": round(gu_bytes / (us * 1e-6) / 8e12, 4)}

    # The fp64 layer oracle on the host, as it stands, for the same SWA(64,4) step: one layer
    # (its weights converted once, outside the timing) over a history of 68 positions, timed
    # for a few tokens and scaled to the stack.
    if not args.no_cpu_baseline:
        import numpy as np

        from oracle import layer as olayer
        wcpu = inputs.layer_weights(seed, 0, dm, Hq, Hkv, d, f)
        ow = olayer.LayerWeights(*[wcpu[k].double().numpy() for k in
                                   ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate_up", "w_down")])
        hist = [olayer.History()]
        kvg = torch.Generator().manual_seed(seed)
        for pcpu in list(range(4)) + list(range(1000 - 64, 1000)):
            hist[0].add(pcpu, torch.randn(Hkv, d, generator=kvg).double().numpy(),
                        torch.randn(Hkv, d, generator=kvg).double().numpy())
        xo = inputs.residual(seed, 0, B, dm).double().numpy()
        n_tok, t0 = 0, time.perf_counter()
        while n_tok < 3 or time.perf_counter() - t0 < 5.0:
            xo = olayer.layer_step(xo, ow, hist, [1000 + n_tok], Hq, Hkv, d, 64, 4, scale, 0, eps)
            n_tok += 1
        sec_layer = (time.perf_counter() - t0) / n_tok
        rec["cpu_baseline"] = {"value": round(1.0 / (sec_layer * nl), 3), "unit": "tokens/s", "kind": "oracle",
                               "cores": len(os.sched_getaffinity(0)),
                               "sample": f"{n_tok} single-layer fp64 oracle steps (numpy matmuls, SWA(64,4) over 68 "
                                         f"cached positions), scaled to {nl} layers"}
        del ow, wcpu

    variants = [("swa64_4", [(64, 4)] * nl), ("swa128_4", [(128, 4)] * nl), ("swa256_4", [(256, 4)] * nl),
                ("swa512_4", [(512, 4)] * nl), ("full", None), ("hybrid_swa64_4_last_full", "hybrid")]
    contexts = [int(c) for c in args.model_contexts.split(",")]
    gen = torch.Generator(device=dev)
    for P in contexts:
        for name, cfg in variants:
            if cfg is None:
                layer_cfg = [(P + T, 0)] * nl  # a window covering every position: full attention
            elif cfg == "hybrid":
                layer_cfg = [(64, 4)] * (nl - 1) + [(P + T, 0)]
            else:
                layer_cfg = cfg
            gen.manual_seed(seed + P)
            caches = []
            for (w, s) in layer_cfg:
                kc, vc = swa.alloc_cache(B, Hkv, d, w, s, device=dev)
                kc.copy_(torch.randn(kc.shape, generator=gen, device=dev))
                vc.copy_(torch.randn(vc.shape, generator=gen, device=dev))
                caches.append((kc, vc))
            state_bytes = sum(kc.numel() * 2 * 2 for kc, _ in caches)
            windows = [(w, s, 0) for w, s in layer_cfg]
            ws = torch.empty(swa.stack_workspace_bytes(windows, B, dm, Hq, Hkv, d, f), dtype=torch.uint8, device=dev)
            stack = [(weights[li], caches[li][0], caches[li][1], w, s, 0) for li, (w, s) in enumerate(layer_cfg)]
            xin = torch.stack([inputs.residual(seed, i, B, dm) for i in range(T)]).to(dev)
            x = torch.empty(B, dm, dtype=torch.float32, device=dev)
            dpos = [torch.full((B,), P + i, dtype=torch.int64, device=dev) for i in range(T)]

            def tokens():
                for i in range(T):
                    x.copy_(xin[i])
                    swa.stack_decode_step(x, stack, dpos[i], Hq, scale, eps, workspace=ws)

            stream = torch.cuda.Stream(device=dev)
            stream.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(stream):
                tokens()
            stream.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                tokens()
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            e0.record()
            for _ in range(reps):
                graph.replay()
            e1.record()
            torch.cuda.synchronize()
            ms_tok = e0.elapsed_time(e1) / (reps * T)
            assert torch.isfinite(x).all(), "non-finite residual stream"
            rec["points"].append({"attention": name, "context": P, "ms_per_token": round(ms_tok, 4),
                                  "tokens_per_s": round(1e3 / ms_tok, 1), "kv_state_mb": round(state_bytes / 2 ** 20, 3),
                                  "weight_gb_per_s": round(weight_bytes / (ms_tok * 1e-3) / 1e9, 1)})
            print(json.dumps(rec["points"][-1]), file=sys.stderr, flush=True)
            del graph, caches, ws, stack
            torch.cuda.empty_cache()
    print(json.dumps(rec), flush=True)


def decode_only(args, dev):
    """--decode-only B: time the decode graph at batch B (or, with --eager, the same launches one by
    one, each stamped by its own dispatch) and print one JSON line."""
    import sliding_window_attention_02_amd as swa
    from sliding_window_attention_02_amd import accounting as acc
    from sliding_window_attention_02_amd import inputs

    dw = inputs.decode_workloads()["decode_swa64_4_b64"]
    if args.eager:
        rec = decode_kernel_only(swa, inputs, acc, dw, args.decode_only, args.decode_tokens, args.decode_start, dev,
                                 n_sets=args.cache_sets)
    else:
        rec = decode_point(swa, inputs, acc, dw, args.decode_only, args.decode_tokens, args.decode_start, dev,
                           reps=args.steps, n_sets=args.cache_sets)
    print(json.dumps(rec), flush=True)


def decode_label(swa, dw, B: int) -> str:
    """The decode kernel launched for workload dw at batch B (swa_decode_describe)."""
    i = swa.decode_describe(B, dw.Hq, dw.Hkv, dw.d, dw.w, dw.s, dw.conv)
    nch = -(-i["slots_per_split"] // 32)
    how = (f"{i['waves_per_workgroup']} waves per workgroup, one 32-slot chunk each, merged in LDS"
           if i["waves_per_workgroup"] > 1 else f"one wave per split of {i['slots_per_split']} slots")
    merge = ", plus merge_kernel" if i["merge_launch"] else ""
    return (f"decode_kernel<{dw.d}, {1 if i['waves_per_workgroup'] > 1 else nch}, {i['waves_per_workgroup']}> "
            f"(fused append + attend; {how}; {i['workgroups']} workgroups{merge})")


def describe(swa, wl):
    """The prefill kernel launched for workload wl (swa_prefill_describe) and its label."""
    info = swa.prefill_describe(wl.B, wl.Hq, wl.Hkv, wl.L, wl.d, wl.w, wl.s, wl.conv)
    names = {0: "tile walk", 1: "resident form", 2: "resident form, 64-row workgroups",
             3: "tile walk, 64-row workgroups"}
    info["kernel"] = f"prefill_kernel<{wl.d}, {info['form']}> ({names[info['form']]}, " \
                     f"{info['tokens_per_tile']}-token q-tiles x {info['heads_per_tile']} q-heads)"
    return info


def prefill_figures(acc, wl, ms_list):
    """Mean/p10/p90 launch time and the throughput figures of one prefill workload."""
    w_loc = wl.w if wl.conv == 0 else wl.w - wl.s
    useful = acc.useful_flops(wl.B, wl.Hq, wl.L, wl.d, w_loc, wl.s)
    algo = acc.prefill_bytes(wl.B, wl.L, wl.Hq, wl.Hkv, wl.d)
    ms = sorted(ms_list)
    mean = sum(ms) / len(ms)
    tf = useful / (mean * 1e-3) / 1e12
    return {"mean_launch_us": round(mean * 1e3, 3), "p10_us": round(ms[len(ms) // 10] * 1e3, 3),
            "p90_us": round(ms[(9 * len(ms)) // 10] * 1e3, 3), "useful_tflops": round(tf, 3),
            "frac_of_bf16_mfma_peak": round(tf / acc.PEAK_BF16_TFLOPS, 5),
            "algorithmic_gb_per_s": round(algo / (mean * 1e-3) / 1e9, 2),
            "frac_of_hbm_peak": round(algo / (mean * 1e-3) / 1e9 / acc.PEAK_HBM_GBS, 5),
            "frac_of_attainable": round(tf / acc.attainable_tflops(useful, algo), 5)}


def other_prefills(swa, inputs, acc, names, dev, reps: int, flush):
    """Secondary prefill workloads, each timed cold (caches evicted before every launch) and warm."""
    import torch

    recs = []
    for name in names:
        wl = inputs.prefill_workloads()[name]
        q, k, v = inputs.prefill_inputs(wl)
        qg, kg, vg = q.to(dev), k.to(dev), v.to(dev)
        out = torch.empty((wl.B, wl.L, wl.Hq, wl.d), dtype=torch.float32, device=dev)
        cold = prefill_timing(swa, wl, qg, kg, vg, out, reps, 2, flush)
        warm = prefill_timing(swa, wl, qg, kg, vg, out, reps, 2)
        w_loc = wl.w if wl.conv == 0 else wl.w - wl.s
        useful = acc.useful_flops(wl.B, wl.Hq, wl.L, wl.d, w_loc, wl.s)
        algo = acc.prefill_bytes(wl.B, wl.L, wl.Hq, wl.Hkv, wl.d)
        recs.append({"workload": name, "kernel": describe(swa, wl)["kernel"],
                     "bound": "mfma" if acc.attainable_tflops(useful, algo) >= acc.PEAK_BF16_TFLOPS else "hbm",
                     "cold": prefill_figures(acc, wl, cold), "warm": prefill_figures(acc, wl, warm)})
        del qg, kg, vg, out
        torch.cuda.empty_cache()
    return recs


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the SWA(w,s) library runs on a single device and has "
              "no multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
        return

    import torch

    import sliding_window_attention_02_amd as swa
    from sliding_window_attention_02_amd import accounting as acc
    from sliding_window_attention_02_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    modes = [(args.prefill_only, prefill_only), (args.decode_only, decode_only), (args.chunked, chunked_only),
             (args.model_sweep, model_sweep), (args.compare_full, compare_full)]
    for flag, fn in modes:
        if flag:
            fn(args, dev)
            return

    # ---------------------------------------------------------------- prefill inputs
    wl = inputs.prefill_workloads()[args.workload]
    w_loc = wl.w if wl.conv == 0 else wl.w - wl.s
    q, k, v = inputs.prefill_inputs(wl)
    qg, kg, vg = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty((wl.B, wl.L, wl.Hq, wl.d), dtype=torch.float32, device=dev)
    useful = acc.useful_flops(wl.B, wl.Hq, wl.L, wl.d, w_loc, wl.s)
    algo_bytes = acc.prefill_bytes(wl.B, wl.L, wl.Hq, wl.Hkv, wl.d)
    info = describe(swa, wl)
    executed = 4 * wl.d * info["executed_pairs"]
    flush = flush_buffer(dev)

    # ---------------------------------------------------------------- decode inputs
    dw = inputs.decode_workloads()["decode_swa64_4_b64"]
    DB, T, P, NS = args.decode_batch, args.decode_tokens, args.decode_start, args.cache_sets
    dw_loc = dw.w if dw.conv == 0 else dw.w - dw.s
    graph, restore = decode_graph(swa, inputs, dw, DB, T, P, dev, n_sets=NS)

    def step(evs=None, i=0):
        # The decode caches back to their state after P-1, the decode graph, then the caches evicted
        # and the prefill (its dispatch stamps its own start and end).
        restore()
        if evs is not None:
            evs[2][i].record()
        graph.replay()
        if evs is not None:
            evs[3][i].record()
        flush.fill_(float(i))
        swa.prefill(qg, kg, vg, wl.w, wl.s, wl.scale, wl.conv, out=out,
                    events=None if evs is None else (evs[0][i], evs[1][i]))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(K)] for _ in range(4)]
    for e in evs[0] + evs[1]:
        e.record()  # creates the underlying HIP events, which the timed launches then stamp
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(evs, i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    pre_ms = [evs[0][i].elapsed_time(evs[1][i]) for i in range(K)]
    dec_ms = [evs[2][i].elapsed_time(evs[3][i]) for i in range(K)]
    pre = prefill_figures(acc, wl, pre_ms)
    tflops = pre["useful_tflops"]
    pre_mean_s = pre["mean_launch_us"] * 1e-6
    dec_mean = sum(dec_ms) / K
    dec_step_us = dec_mean * 1e3 / T
    dec_kv_bytes = acc.decode_kv_bytes(DB, dw.Hkv, dw.d, acc.decode_keys(P, dw_loc, dw.s))
    dec_gbs = dec_kv_bytes / (dec_step_us * 1e-6) / 1e9
    dec_all_gbs = (dec_kv_bytes + acc.decode_other_bytes(DB, dw.Hq, dw.Hkv, dw.d)) / (dec_step_us * 1e-6) / 1e9
    traffic = measured_traffic(wl.name)

    warm = kernel_only = None
    points, others = [], []
    if not args.no_extras:
        warm = prefill_figures(acc, wl, prefill_timing(swa, wl, qg, kg, vg, out, K, 3))
        kernel_only = decode_kernel_only(swa, inputs, acc, dw, DB, T, P, dev, n_sets=NS)
        for b, t, n in ((DB, T, 1), (1, 256, 1), (1024, 32, 1)):
            rec = decode_point(swa, inputs, acc, dw, b, t, P, dev, n_sets=n)
            rec["note"] = {DB: "one cache set: the working set stays in the 256 MB Infinity Cache",
                           1: "one sequence: launch-latency bound", 1024: "285 MB of KV per step, read from HBM"}[b]
            points.append(rec)
        del qg, kg, vg, out
        torch.cuda.empty_cache()
        others = other_prefills(swa, inputs, acc, [n for n in args.other_workloads.split(",") if n], dev,
                                max(10, K // 2), flush)

    base = None
    if not args.no_cpu_baseline:
        threads = args.cpu_threads or min(16, len(os.sched_getaffinity(0)))
        base = cpu_baseline(wl, q, k, v, threads)

    rec = {
        "metric": "SWA(w,s) prefill useful TFLOP/s + decode tokens/s, % of MFMA/HBM roofline",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name} prefill (caches evicted first) + decode_swa64_4_b{DB} ({T} tokens per step "
                        f"over {NS} rotating caches)",
            "prefill": {"B": wl.B, "L": wl.L, "Hq": wl.Hq, "Hkv": wl.Hkv, "d": wl.d, "w": wl.w, "s": wl.s,
                        "conv": "additive" if wl.conv == 0 else "total", "inputs": f"bf16 N(0,1)*{wl.std}",
                        "out": "fp32"},
            "decode": {"B": DB, "Hq": dw.Hq, "Hkv": dw.Hkv, "d": dw.d, "w": dw.w, "s": dw.s,
                       "positions": [P, P + (T + NS - 1) // NS - 1], "tokens_per_step": T, "cache_sets": NS,
                       "hip_graph": True},
        },
        "prefill": dict(pre, **{
            "kernel": info["kernel"],
            "caches": "evicted before every launch",
            "executed_mfma_tflops": round(executed / pre_mean_s / 1e12, 3),
            "executed_over_useful": round(executed / useful, 4),
            "useful_gflop_per_launch": round(useful / 1e9, 4),
            "algorithmic_mb_per_launch": round(algo_bytes / 1e6, 3),
            "warm": warm,
            "others": others,
        }),
        "decode": {
            "tokens_per_s": round(T * DB / (dec_mean * 1e-3), 1),
            "us_per_token_step": round(dec_step_us, 3),
            "kv_bytes_per_step": dec_kv_bytes,
            "kv_gb_per_s": round(dec_gbs, 2),
            "frac_of_hbm_peak": round(dec_gbs / acc.PEAK_HBM_GBS, 5),
            "all_bytes_frac_of_hbm_peak": round(dec_all_gbs / acc.PEAK_HBM_GBS, 5),
            "kernel_only": kernel_only,
            "other_points": points,
        },
        "roofline": {
            "kernel": info["kernel"],
            "bound": "mfma",
            "achieved": round(tflops, 3),
            "peak": acc.PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / acc.PEAK_BF16_TFLOPS, 5),
            "traffic": traffic,
        },
        # The decode half of the metric: KV bytes per step against HBM peak, over the per-step time
        # of the graph (dispatch gaps included) and over the kernel alone.
        "roofline_decode": {
            "kernel": decode_label(swa, dw, DB),
            "bound": "hbm",
            "batch": DB,
            "achieved": round(dec_gbs, 2),
            "peak": acc.PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(dec_gbs / acc.PEAK_HBM_GBS, 5),
            "kernel_only_achieved": None if kernel_only is None else kernel_only["kv_gb_per_s"],
            "kernel_only_frac": None if kernel_only is None else kernel_only["frac_of_hbm_peak"],
        },
        "cpu_baseline": base,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
