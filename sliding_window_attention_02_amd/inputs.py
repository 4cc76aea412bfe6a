"""Seeded synthetic inputs for the SWA(w,s) prefill and decode workloads.

This module draws random numbers and rounds them to bfloat16; it holds none of the
attention arithmetic, so the GPU path and the fp64 oracle can both take their inputs
from here without sharing any of the method.

Recipe (every draw on the CPU, torch.Generator, fp32 N(0,1)):
  * prefill: one generator seeded with the workload's seed draws q [B][L][Hq][d], then
    k [B][L][Hkv][d], then v; each is multiplied by the workload's std; keys at positions
    0..sink_boost_n-1 are multiplied by sink_boost (x4 is exact in binary floating point);
    then every tensor is rounded to bf16 with round-to-nearest-even.
  * decode: values are drawn per absolute position so any position up to 2^18 and beyond
    can be produced without the history before it.  The generator for (seed, stream,
    position) is seeded with splitmix64(seed, stream, position); stream 0 gives the k and
    v of a position ([B][Hkv][d] each, k first), stream 1 gives the query [B][Hq][d].
    The same std / sink boost / bf16 rounding apply.

  * decoder layers (multi-layer decode): one generator seeded with (seed, layer) draws, in
    order, the two norm weights (1 + 0.1 N(0,1)) and the weight matrices w_qkv, w_o,
    w_gate_up, w_down, each N(0,1) / sqrt(fan-in); all rounded to bf16.  The residual
    stream of a step is N(0,1) fp32 from the generator seeded with (seed, 2, step).

The workloads mirror the shapes the pages discuss: Llama-3.1-8B heads (32 q-heads, 8
kv-heads, d=128) at 4K context with windows 64..512 as in the S-NIAH study, the decode
sweep from 128 to 256K context, and Mistral-7B at 16K with window 4096.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

MASK64 = (1 << 64) - 1


def splitmix64(x: int) -> int:
    """One step of the SplitMix64 output function (Steele, Lea, Flood 2014)."""
    x = (x + 0x9E3779B97F4A7C15) & MASK64
    z = x
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def position_seed(seed: int, stream: int, position: int) -> int:
    """Counter-based 63-bit seed for one (seed, stream, position) triple."""
    h = splitmix64(seed & MASK64)
    h = splitmix64(h ^ (stream & MASK64))
    h = splitmix64(h ^ (position & MASK64))
    return h >> 1


@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    L: int
    w: int
    s: int
    std: float
    sink_boost_n: int
    sink_boost: float
    seed: int
    conv: int = 0  # 0 = additive (w recent keys plus s sinks), 1 = total window

    @property
    def scale(self) -> float:
        return 1.0 / (self.d ** 0.5)


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    w: int
    s: int
    std: float
    sink_boost_n: int
    sink_boost: float
    seed: int
    steps: int = 256
    points: tuple = field(default_factory=lambda: tuple(2 ** e for e in range(7, 19)))
    conv: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / (self.d ** 0.5)


def prefill_workloads() -> dict:
    """The prefill workloads by name."""
    w = {}
    w["tiny_swa64_4"] = PrefillWorkload("tiny_swa64_4", B=1, Hq=4, Hkv=4, d=64, L=256, w=64, s=4,
                                        std=1.0, sink_boost_n=4, sink_boost=4.0, seed=1001)
    w["llama8b_swa64_4"] = PrefillWorkload("llama8b_swa64_4", B=1, Hq=32, Hkv=8, d=128, L=4096,
                                           w=64, s=4, std=0.5, sink_boost_n=4, sink_boost=4.0,
                                           seed=1002)
    for win in (128, 256, 512):
        for s in (4, 0):
            n = f"sweep_w{win}_s{s}"
            w[n] = PrefillWorkload(n, B=4, Hq=32, Hkv=8, d=128, L=4096, w=win, s=s, std=1.0,
                                   sink_boost_n=4, sink_boost=4.0, seed=1003)
    for s in (4, 0):
        n = f"mistral7b_w4096_s{s}"
        w[n] = PrefillWorkload(n, B=1, Hq=32, Hkv=8, d=128, L=16384, w=4096, s=s, std=1.0,
                               sink_boost_n=0, sink_boost=1.0, seed=1005)
    return w


def decode_workloads() -> dict:
    w = {}
    for B in (1, 64):
        n = f"decode_swa64_4_b{B}"
        w[n] = DecodeWorkload(n, B=B, Hq=32, Hkv=8, d=128, w=64, s=4, std=1.0, sink_boost_n=4,
                              sink_boost=4.0, seed=1004)
    return w


def _round_bf16(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16)


def prefill_inputs(wl: PrefillWorkload, L: int | None = None, B: int | None = None):
    """(q, k, v) bf16 CPU tensors for a prefill workload; L / B may be cut for small tests
    (the draw order is unchanged, so a cut is not a prefix of the full draw)."""
    L = wl.L if L is None else L
    B = wl.B if B is None else B
    return random_qkv(B, L, wl.Hq, wl.Hkv, wl.d, wl.seed, wl.std, wl.sink_boost_n, wl.sink_boost)


def random_qkv(B, L, Hq, Hkv, d, seed, std=1.0, sink_boost_n=0, sink_boost=1.0):
    """Seeded bf16 q [B][L][Hq][d], k, v [B][L][Hkv][d] on the CPU."""
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, L, Hq, d, generator=g, dtype=torch.float32) * std
    k = torch.randn(B, L, Hkv, d, generator=g, dtype=torch.float32) * std
    v = torch.randn(B, L, Hkv, d, generator=g, dtype=torch.float32) * std
    if sink_boost_n > 0:
        k[:, :sink_boost_n] *= sink_boost
    return _round_bf16(q), _round_bf16(k), _round_bf16(v)


def random_qkv_device(B, L, Hq, Hkv, d, seed, device, std=1.0, sink_boost_n=0, sink_boost=1.0):
    """Seeded bf16 q [B][L][Hq][d], k, v [B][L][Hkv][d] drawn on `device` (a generator of that
    device, one sequence at a time, so inputs of many GiB need no host copy); the same recipe as
    random_qkv with another stream of random numbers."""
    g = torch.Generator(device=device).manual_seed(seed)
    out = []
    for H in (Hq, Hkv, Hkv):
        t = torch.empty(B, L, H, d, dtype=torch.bfloat16, device=device)
        for b in range(B):
            x = torch.randn(L, H, d, generator=g, dtype=torch.float32, device=device) * std
            t[b] = x.to(torch.bfloat16)  # round to nearest even
            del x
        out.append(t)
    if sink_boost_n > 0:
        out[1][:, :sink_boost_n] *= sink_boost  # x4 is exact in bf16
    return tuple(out)


def kv_at(seed: int, position: int, B: int, Hkv: int, d: int, std: float = 1.0,
          sink_boost_n: int = 0, sink_boost: float = 1.0):
    """(k, v) bf16 [B][Hkv][d] of one absolute position."""
    g = torch.Generator().manual_seed(position_seed(seed, 0, position))
    k = torch.randn(B, Hkv, d, generator=g, dtype=torch.float32) * std
    v = torch.randn(B, Hkv, d, generator=g, dtype=torch.float32) * std
    if position < sink_boost_n:
        k *= sink_boost
    return _round_bf16(k), _round_bf16(v)


def kv_span(seed: int, positions, B: int, Hkv: int, d: int, std: float = 1.0,
            sink_boost_n: int = 0, sink_boost: float = 1.0):
    """(k, v) bf16 [B][n][Hkv][d] for a list of positions (the append layout)."""
    ks, vs = [], []
    for p in positions:
        k, v = kv_at(seed, int(p), B, Hkv, d, std, sink_boost_n, sink_boost)
        ks.append(k)
        vs.append(v)
    return torch.stack(ks, dim=1), torch.stack(vs, dim=1)


def q_at(seed: int, position: int, B: int, Hq: int, d: int, std: float = 1.0):
    """Query bf16 [B][Hq][d] of the token at one absolute position."""
    g = torch.Generator().manual_seed(position_seed(seed, 1, position))
    return _round_bf16(torch.randn(B, Hq, d, generator=g, dtype=torch.float32) * std)


def layer_weights(seed: int, layer: int, dm: int, Hq: int, Hkv: int, d: int, f: int) -> dict:
    """bf16 CPU tensors of one decoder layer (names as the layer step takes them)."""
    g = torch.Generator().manual_seed(position_seed(seed, 3, layer))
    def mat(n, k):
        return _round_bf16(torch.randn(n, k, generator=g) / (k ** 0.5))
    out = {"attn_norm": _round_bf16(1 + 0.1 * torch.randn(dm, generator=g)),
           "mlp_norm": _round_bf16(1 + 0.1 * torch.randn(dm, generator=g))}
    out["w_qkv"] = mat((Hq + 2 * Hkv) * d, dm)
    out["w_o"] = mat(dm, Hq * d)
    out["w_gate_up"] = mat(2 * f, dm)
    out["w_down"] = mat(dm, f)
    return out


def residual(seed: int, step: int, B: int, dm: int) -> torch.Tensor:
    """fp32 [B][dm] N(0,1) residual-stream input of a step."""
    g = torch.Generator().manual_seed(position_seed(seed, 2, step))
    return torch.randn(B, dm, generator=g)
