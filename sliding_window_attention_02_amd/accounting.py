"""Work and traffic accounting for SWA(w,s) prefill and decode (roofline denominators).

Units of work follow the FLOP table on page "从长文档摘要说起：为什么注意力范围成了瓶颈"
(wiblog.cn), section "注意力计算量的来源：平方项藏在哪": per head, the QK product and the
V weighting each cost 2*d flops per (query, key) pair, and SWA replaces the s^2 pair
count by the pairs inside the window (section "计算与显存的节省：从平方到线性").  Softmax
work is not counted as useful flops.  KV cache size follows the same page's 2*L*s*d_q*n_kv
formula.
"""
from __future__ import annotations

# MI355X published peaks.
PEAK_HBM_GBS = 8000.0            # HBM3E, GB/s
PEAK_BF16_TFLOPS = 2516.6        # dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk), TFLOP/s
PEAK_FP32_VALU_TFLOPS = 157.3


def pairs_per_head(L: int, w_loc: int, s: int) -> int:
    """sum_t |A(t)| over t < L with |A(t)| = min(t+1, w_loc+s)."""
    m = min(L, w_loc + s)
    return m * (m + 1) // 2 + (L - m) * (w_loc + s)


def useful_flops(B: int, Hq: int, L: int, d: int, w_loc: int, s: int) -> int:
    """2*d (QK) + 2*d (PV) flops per allowed (query, key) pair and q-head."""
    return 4 * d * Hq * B * pairs_per_head(L, w_loc, s)


def prefill_bytes(B: int, L: int, Hq: int, Hkv: int, d: int) -> int:
    """Algorithmic HBM bytes: bf16 q, k, v read once, fp32 out written once."""
    return B * L * (Hq * d * 2 + 2 * Hkv * d * 2 + Hq * d * 4)


def decode_keys(t: int, w_loc: int, s: int) -> int:
    return min(t + 1, w_loc + s)


def decode_kv_bytes(B: int, Hkv: int, d: int, n_keys: int) -> int:
    """bf16 K and V bytes one decode step reads."""
    return B * Hkv * n_keys * d * 2 * 2


def decode_other_bytes(B: int, Hq: int, Hkv: int, d: int) -> int:
    """q (bf16) read, out (fp32) written, one new K/V token (bf16) read and written."""
    return B * (Hq * d * 2 + Hq * d * 4 + 2 * 2 * Hkv * d * 2)


def kv_cache_bytes(layers: int, seq: int, d_q: int, n_kv: int, bytes_per_value: int) -> int:
    """2 * layers * seq * d_q * n_kv values (K and V) times bytes per value."""
    return 2 * layers * seq * d_q * n_kv * bytes_per_value


def attainable_tflops(useful_flops_: float, algorithmic_bytes: float) -> float:
    """Roofline bound of a kernel doing useful_flops_ over algorithmic_bytes: the smaller of the
    bf16 MFMA peak and arithmetic intensity x HBM peak (TFLOP/s)."""
    return min(PEAK_BF16_TFLOPS, useful_flops_ / algorithmic_bytes * PEAK_HBM_GBS / 1e3)
