"""fp64 oracle of one decoder-layer decode step around SWA(w,s) attention.

TEST INFRASTRUCTURE ONLY: the test suite and the benchmark's CPU-baseline leg are the only
callers; the GPU package never imports this module and this module imports nothing from it.

The pages time decode through a 4-layer Transformer at batch 1 (page "几亿Token白练了？微软实测：
免训练滑动窗口，让线性注意力破防" (PaperWeekly), section "小窗口也有工程优势": decode throughput
and state memory against context length).  They give no layer
dimensions or layer recipe, so this oracle takes the plainest standard pre-norm decoder layer:

    h   = bf16( rmsnorm(x) * g_attn )                 x: fp32 residual stream [dm]
    q, k, v = split( bf16( W_qkv h ) )               W_qkv: [(Hq + 2 Hkv) d][dm]
    o   = SWA(w,s) decode of q at position t over every (position, k, v) appended so far
    x  += W_o bf16(o)                                 W_o: [dm][Hq d]
    h2  = bf16( rmsnorm(x) * g_mlp )
    a   = bf16( silu(W_gate h2) * (W_up h2) )         W_gate_up: [2 f][dm], gate rows first
    x  += W_down a                                    W_down: [dm][f]

with rmsnorm(x) = x / sqrt(mean(x^2) + eps) and silu(z) = z / (1 + exp(-z)).  No positional
encoding and no output head: the pages name neither, and neither changes the bytes a decode
step moves.  bf16(.) is round-to-nearest-even to bfloat16 at the points where the layer
stores activations in bf16; everything else is fp64.  The attention step is
oracle.oracle.decode_rows over the explicit history, so it shares nothing with the GPU
path's ring layout.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import oracle as swa_oracle


def bf16_round(x) -> np.ndarray:
    """Round to the nearest bfloat16 (ties to even), returned as float64.

    The value is first rounded to float32 (as a float32 accumulator holds it), then the low
    16 bits of the float32 pattern are rounded away: add 0x7fff plus the lowest kept bit, then
    truncate.  Finite inputs only.
    """
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64)).astype(np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    rounded = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16) << 16
    return rounded.astype(np.uint32).view(np.float32).astype(np.float64)


def rmsnorm(x, g, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g over the last axis (fp64)."""
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def silu(z) -> np.ndarray:
    """z * sigmoid(z) = z / (1 + exp(-z)) (fp64; exp overflow for very negative z gives 0)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


@dataclass
class LayerWeights:
    """bf16-valued weights held as float64 arrays (exact)."""
    g_attn: np.ndarray   # [dm]
    w_qkv: np.ndarray    # [(Hq + 2 Hkv) d][dm]
    w_o: np.ndarray      # [dm][Hq d]
    g_mlp: np.ndarray    # [dm]
    w_gate_up: np.ndarray  # [2 f][dm]
    w_down: np.ndarray   # [dm][f]


@dataclass
class History:
    """Every (position, k, v) a layer has appended, per batch item: k, v are [n][Hkv][d]."""
    pos: list = field(default_factory=list)
    k: list = field(default_factory=list)
    v: list = field(default_factory=list)

    def add(self, p: int, k, v):
        self.pos.append(int(p))
        self.k.append(np.asarray(k, dtype=np.float64))
        self.v.append(np.asarray(v, dtype=np.float64))


def layer_step(x, wts: LayerWeights, hist: list, t, Hq: int, Hkv: int, d: int, w: int, s: int,
               scale: float, conv: int, eps: float) -> np.ndarray:
    """One decode step of one layer for a batch.

    x: [B][dm] residual stream (fp64 holding the fp32 state); hist: one History per batch item,
    to which the step appends (t[b], k, v); t: [B] positions.  Returns the new x [B][dm].
    """
    x = np.asarray(x, dtype=np.float64)
    B, dm = x.shape
    t = np.asarray(t, dtype=np.int64)
    f = wts.w_down.shape[1]
    h = bf16_round(rmsnorm(x, wts.g_attn, eps))
    qkv = bf16_round(h @ wts.w_qkv.T)
    q = qkv[:, :Hq * d].reshape(B, Hq, d)
    kn = qkv[:, Hq * d:(Hq + Hkv) * d].reshape(B, Hkv, d)
    vn = qkv[:, (Hq + Hkv) * d:].reshape(B, Hkv, d)
    o = np.empty((B, Hq, d))
    for b in range(B):
        hist[b].add(t[b], kn[b], vn[b])
        pos = np.array(hist[b].pos, dtype=np.int64)
        kk = np.stack(hist[b].k)[None]
        vv = np.stack(hist[b].v)[None]
        o[b] = swa_oracle.decode_rows(q[b][None], pos, kk, vv, t[b:b + 1], w, s, scale, conv, nthreads=1)[0]
    x1 = x + bf16_round(o.reshape(B, Hq * d)) @ wts.w_o.T
    h2 = bf16_round(rmsnorm(x1, wts.g_mlp, eps))
    gu = h2 @ wts.w_gate_up.T
    a = bf16_round(silu(gu[:, :f]) * gu[:, f:])
    return x1 + a @ wts.w_down.T
