"""ctypes front end of the fp64 SWA(w,s) oracle in ``oracle/swa_oracle.c``.

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the benchmark's
CPU-baseline leg are the only callers.  Nothing here imports the GPU package, and the
GPU package never imports this module.

Every function follows the plain definition of SWA(w,s) given on the page
"滑动窗口注意力（SWA）配 sinks 比 post-training 线性注意力更划算" (papers.ananclaw.com,
arXiv 2608.28444 explainer), section 核心方法 1 (the x_t equation and the swa_mask
pseudocode), with the readings listed in the C file's header.  The pins that tie each
function to the pages and to independent mathematics are in tests/test_oracle_pins.py.

Inputs are numpy float64 arrays (callers convert the bf16-rounded tensors exactly).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "swa_oracle.c")
LIB = os.path.join(HERE, "libswa_oracle.so")

ADDITIVE = 0
TOTAL = 1

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (strict IEEE: no fast-math, no FMA contraction)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
               "-ffp-contract=off", "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB):
        build(force=True)
    lib = ctypes.CDLL(LIB)
    i64, i32, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_double
    vp = ctypes.c_void_p
    lib.swa_oracle_local_window.argtypes = [i64, i64, i32, ctypes.POINTER(i64)]
    lib.swa_oracle_local_window.restype = i32
    lib.swa_oracle_allowed.argtypes = [i64, i64, i64, i64]
    lib.swa_oracle_allowed.restype = i32
    lib.swa_oracle_mask.argtypes = [vp, i64, i64, i64]
    lib.swa_oracle_mask.restype = None
    lib.swa_oracle_row_weights.argtypes = [vp, vp, i64, i32, i64, i64, i64, dbl, vp]
    lib.swa_oracle_row_weights.restype = i64
    lib.swa_oracle_prefill.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, dbl, i32]
    lib.swa_oracle_prefill.restype = i32
    lib.swa_oracle_prefill_rows.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, dbl, i64, i64, i32]
    lib.swa_oracle_prefill_rows.restype = i32
    lib.swa_oracle_lse_rows.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, dbl, i64, i64]
    lib.swa_oracle_lse_rows.restype = i32
    lib.swa_oracle_decode_row.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, dbl, vp]
    lib.swa_oracle_decode_row.restype = i64
    lib.swa_oracle_decode_rows.argtypes = [vp, vp, vp, vp, i64, i64, vp, i64, i64, i64, i64, i64, dbl, vp, i32]
    lib.swa_oracle_decode_rows.restype = i32
    lib.swa_oracle_ring_simulate.argtypes = [i64, i64, i64, vp]
    lib.swa_oracle_ring_simulate.restype = i32
    _lib = lib
    return lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


def local_window(w: int, s: int, conv: int = ADDITIVE) -> int:
    """w_loc: w for the additive convention, w - s for the total-window convention."""
    out = ctypes.c_int64(0)
    if _load().swa_oracle_local_window(w, s, conv, ctypes.byref(out)) != 0:
        raise ValueError(f"no local window for w={w}, s={s}, conv={conv}")
    return out.value


def allowed(t: int, i: int, w_loc: int, s: int) -> bool:
    """True iff key i is in the allowed set A(t)."""
    return bool(_load().swa_oracle_allowed(t, i, w_loc, s))


def mask(L: int, w_loc: int, s: int) -> np.ndarray:
    """Dense [L][L] boolean matrix of the allowed-key predicate (row = query)."""
    m = np.zeros((L, L), dtype=np.uint8)
    _load().swa_oracle_mask(_ptr(m), L, w_loc, s)
    return m.astype(bool)


def row_weights(q_row, k_rows, t: int, w_loc: int, s: int, scale: float) -> np.ndarray:
    """Softmax weights of query t over keys 0..t (zeros outside A(t)); k_rows is [>=t+1][d]."""
    q_row = _f64(q_row)
    k_rows = _f64(k_rows)
    d = q_row.shape[0]
    assert k_rows.ndim == 2 and k_rows.shape[1] == d and k_rows.shape[0] > t
    p = np.zeros(t + 1, dtype=np.float64)
    _load().swa_oracle_row_weights(_ptr(q_row), _ptr(k_rows), d, d, t, w_loc, s, float(scale), _ptr(p))
    return p


def prefill(q, k, v, w: int, s: int, scale: float, conv: int = ADDITIVE,
            nthreads: int | None = None) -> np.ndarray:
    """SWA(w,s) attention over whole sequences.

    q: [B][L][Hq][d], k/v: [B][L][Hkv][d]; returns fp64 [B][L][Hq][d].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, L, Hq, d = q.shape
    Hkv = k.shape[2]
    assert k.shape == (B, L, Hkv, d) and v.shape == k.shape
    w_loc = local_window(w, s, conv)
    out = np.empty_like(q)
    rc = _load().swa_oracle_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, L, d,
                                    w_loc, s, float(scale), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"swa_oracle_prefill failed ({rc})")
    return out


def prefill_rows(q, k, v, t_lo: int, t_hi: int, w: int, s: int, scale: float, conv: int = ADDITIVE,
                 nthreads: int | None = None) -> np.ndarray:
    """Rows t_lo <= t < t_hi of prefill(q, k, v, ...): fp64 [B][t_hi - t_lo][Hq][d], each row
    computed exactly as prefill computes it."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, L, Hq, d = q.shape
    Hkv = k.shape[2]
    assert k.shape == (B, L, Hkv, d) and v.shape == k.shape and 0 <= t_lo < t_hi <= L
    w_loc = local_window(w, s, conv)
    out = np.empty((B, t_hi - t_lo, Hq, d), dtype=np.float64)
    rc = _load().swa_oracle_prefill_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, L, d, w_loc, s,
                                         float(scale), t_lo, t_hi, nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"swa_oracle_prefill_rows failed ({rc})")
    return out


def lse_rows(q, k, t_lo: int, t_hi: int, w: int, s: int, scale: float, conv: int = ADDITIVE) -> np.ndarray:
    """ln of the softmax denominator, sum over A(t) of exp(scale <q_t, k_i>), for rows
    t_lo <= t < t_hi: fp64 [B][t_hi - t_lo][Hq]."""
    q, k = _f64(q), _f64(k)
    B, L, Hq, d = q.shape
    Hkv = k.shape[2]
    assert k.shape == (B, L, Hkv, d) and 0 <= t_lo < t_hi <= L
    w_loc = local_window(w, s, conv)
    out = np.empty((B, t_hi - t_lo, Hq), dtype=np.float64)
    if _load().swa_oracle_lse_rows(_ptr(q), _ptr(k), _ptr(out), B, Hq, Hkv, L, d, w_loc, s, float(scale),
                                   t_lo, t_hi) != 0:
        raise RuntimeError("swa_oracle_lse_rows failed")
    return out


def decode_row(q, pos, k, v, t: int, w: int, s: int, scale: float, conv: int = ADDITIVE):
    """One decode row from explicit cached entries.

    q: [Hq][d]; pos: [n] distinct positions; k/v: [n][Hkv][d].  Entries outside A(t) are
    ignored.  Returns (out [Hq][d] fp64, number of entries used).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    pos = np.ascontiguousarray(np.asarray(pos, dtype=np.int64))
    Hq, d = q.shape
    n, Hkv, d2 = k.shape
    assert d2 == d and v.shape == k.shape and pos.shape == (n,)
    w_loc = local_window(w, s, conv)
    out = np.empty((Hq, d), dtype=np.float64)
    kept = _load().swa_oracle_decode_row(_ptr(q), _ptr(pos), _ptr(k), _ptr(v), n, t, Hq, Hkv, d,
                                         w_loc, s, float(scale), _ptr(out))
    if kept < 0:
        raise ValueError("swa_oracle_decode_row: bad arguments or duplicate positions")
    return out, int(kept)


def decode_rows(q, pos, k, v, t, w: int, s: int, scale: float, conv: int = ADDITIVE,
                nthreads: int | None = None) -> np.ndarray:
    """decode_row for every batch item: q [B][Hq][d], pos [n] shared candidate positions,
    k/v [B][n][Hkv][d], t [B] query positions -> fp64 [B][Hq][d]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    pos = np.ascontiguousarray(np.asarray(pos, dtype=np.int64))
    t = np.ascontiguousarray(np.asarray(t, dtype=np.int64))
    B, Hq, d = q.shape
    _, n, Hkv, _ = k.shape
    assert k.shape == (B, n, Hkv, d) and v.shape == k.shape and pos.shape == (n,) and t.shape == (B,)
    w_loc = local_window(w, s, conv)
    out = np.empty((B, Hq, d), dtype=np.float64)
    rc = _load().swa_oracle_decode_rows(_ptr(q), _ptr(pos), _ptr(k), _ptr(v), B, n, _ptr(t), Hq, Hkv, d,
                                        w_loc, s, float(scale), _ptr(out), nthreads or default_threads())
    if rc != 0:
        raise ValueError("swa_oracle_decode_rows: bad arguments or duplicate positions")
    return out


def ring_simulate(n_appended: int, w_loc: int, s: int) -> np.ndarray:
    """Positions held by each of the s + w_loc cache slots after appending 0..n_appended-1."""
    out = np.empty(s + w_loc, dtype=np.int64)
    if _load().swa_oracle_ring_simulate(n_appended, w_loc, s, _ptr(out)) != 0:
        raise ValueError("bad ring arguments")
    return out
