"""ctypes binding of libswa.so: argument marshalling only.

Each function checks device, dtype, contiguity and shapes of torch tensors, then passes raw
device pointers, sizes and the current HIP stream to the C ABI declared in include/swa.h.
Every step of the computation runs in the HIP kernels; there is no fallback.  If the
library has not been built the first call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

ADDITIVE = 0
TOTAL = 1

SWA_OK = 0
SWA_EINVAL = -1
SWA_EUNSUPPORTED = -2
SWA_EHIP = -3

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libswa.so")

EXPORTS = (
    "swa_prefill",
    "swa_prefill_timed",
    "swa_prefill_describe",
    "swa_cache_slots",
    "swa_kv_append",
    "swa_decode_workspace_bytes",
    "swa_decode_describe",
    "swa_decode_step",
    "swa_decode_step_noalloc",
    "swa_append_decode_step",
    "swa_append_decode_step_timed",
    "swa_prefill_chunk",
    "swa_last_error",
    "swa_debug_prefill_mask",
    "swa_debug_decode_slots",
    "swa_rmsnorm",
    "swa_linear",
    "swa_layer_workspace_bytes",
    "swa_layer_decode_step",
    "swa_stack_workspace_bytes",
    "swa_stack_decode_step",
)

LINEAR_MODES = {"store": 0, "add": 1, "silu_mul": 2}


class _PrefillInfoC(ctypes.Structure):
    _fields_ = [("form", ctypes.c_int), ("tokens_per_tile", ctypes.c_int), ("heads_per_tile", ctypes.c_int),
                ("workgroups", ctypes.c_longlong), ("executed_pairs", ctypes.c_longlong)]


class _DecodeInfoC(ctypes.Structure):
    _fields_ = [("splits", ctypes.c_int), ("waves_per_workgroup", ctypes.c_int), ("slots_per_split", ctypes.c_int),
                ("heads_per_wave", ctypes.c_int), ("workgroups", ctypes.c_longlong), ("merge_launch", ctypes.c_int),
                ("workspace_bytes", ctypes.c_size_t)]


class _LayerWeightsC(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate_up", "w_down")]

_lib = None


class SwaError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code


def lib() -> ctypes.CDLL:
    """Load libswa.so (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m sliding_window_attention_02_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i32, vp, f32, sz = ctypes.c_int, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t
    L.swa_prefill.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, i32, vp]
    L.swa_prefill.restype = i32
    L.swa_prefill_timed.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, i32, vp, vp, vp]
    L.swa_prefill_timed.restype = i32
    L.swa_prefill_describe.argtypes = [i32] * 8 + [ctypes.POINTER(_PrefillInfoC)]
    L.swa_prefill_describe.restype = i32
    L.swa_decode_describe.argtypes = [i32] * 7 + [ctypes.POINTER(_DecodeInfoC)]
    L.swa_decode_describe.restype = i32
    L.swa_cache_slots.argtypes = [i32, i32, i32]
    L.swa_cache_slots.restype = ctypes.c_longlong
    L.swa_kv_append.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp]
    L.swa_kv_append.restype = i32
    L.swa_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    L.swa_decode_workspace_bytes.restype = sz
    L.swa_decode_step.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, vp, sz, vp]
    L.swa_decode_step.restype = i32
    L.swa_decode_step_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, vp]
    L.swa_decode_step_noalloc.restype = i32
    L.swa_append_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, vp, sz,
                                         vp]
    L.swa_append_decode_step.restype = i32
    L.swa_append_decode_step_timed.argtypes = L.swa_append_decode_step.argtypes + [vp, vp]
    L.swa_append_decode_step_timed.restype = i32
    i64 = ctypes.c_int64
    L.swa_prefill_chunk.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, i32, i32, i32, f32, i32, vp]
    L.swa_prefill_chunk.restype = i32
    L.swa_last_error.argtypes = []
    L.swa_last_error.restype = ctypes.c_char_p
    L.swa_debug_prefill_mask.argtypes = [vp, i32, i32, i32, i32, i32, i32, i32, vp]
    L.swa_debug_prefill_mask.restype = i32
    L.swa_debug_decode_slots.argtypes = [vp, vp, i32, i32, i32, i32, vp]
    L.swa_debug_decode_slots.restype = i32
    L.swa_rmsnorm.argtypes = [vp, vp, vp, i32, i32, f32, vp]
    L.swa_rmsnorm.restype = i32
    L.swa_linear.argtypes = [vp, vp, i32, vp, i32, i32, i32, i32, vp]
    L.swa_linear.restype = i32
    L.swa_layer_workspace_bytes.argtypes = [i32] * 9
    L.swa_layer_workspace_bytes.restype = sz
    L.swa_layer_decode_step.argtypes = [vp, ctypes.POINTER(_LayerWeightsC), vp, vp, vp] + [i32] * 8 + [f32, i32, f32,
                                                                                             vp, sz, vp]
    L.swa_layer_decode_step.restype = i32
    ip = ctypes.POINTER(ctypes.c_int)
    L.swa_stack_workspace_bytes.argtypes = [i32, ip, ip, ip] + [i32] * 6
    L.swa_stack_workspace_bytes.restype = sz
    L.swa_stack_decode_step.argtypes = [vp, i32, ctypes.POINTER(_LayerWeightsC), ctypes.POINTER(vp),
                                        ctypes.POINTER(vp), ip, ip, ip, vp] + [i32] * 6 + [f32, f32, vp, sz, vp]
    L.swa_stack_decode_step.restype = i32
    _lib = L
    return L


def last_error() -> str:
    return lib().swa_last_error().decode()


def _check(rc: int):
    if rc != SWA_OK:
        raise SwaError(rc, last_error())


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def cache_slots(w: int, s: int, conv: int = ADDITIVE) -> int:
    """Slots per (sequence, kv-head) of the decode cache, s + w_loc (swa_cache_slots)."""
    n = lib().swa_cache_slots(w, s, conv)
    if n < 0:
        raise SwaError(SWA_EINVAL, last_error())
    return int(n)


def local_window(w: int, s: int, conv: int = ADDITIVE) -> int:
    """Local window length w_loc: w (additive convention) or w - s (total-window convention)."""
    return cache_slots(w, s, conv) - s


def prefill_describe(B: int, Hq: int, Hkv: int, L: int, d: int, w: int, s: int, conv: int = ADDITIVE) -> dict:
    """What swa_prefill launches for this shape (swa_prefill_describe): kernel form, q-tile
    geometry, grid size and the (query row, key) pairs its matrix cores compute."""
    info = _PrefillInfoC()
    _check(lib().swa_prefill_describe(B, Hq, Hkv, L, d, w, s, conv, ctypes.byref(info)))
    return {f: getattr(info, f) for f, _ in _PrefillInfoC._fields_}


def prefill(q, k, v, w: int, s: int, scale: float | None = None, conv: int = ADDITIVE, out=None,
            events=None):
    """SWA(w,s) prefill.  q bf16 [B][L][Hq][d], k/v bf16 [B][L][Hkv][d] -> fp32 [B][L][Hq][d].

    events: optional (start, stop) torch.cuda.Event pair (timing enabled, already recorded
    once so the underlying HIP events exist); the kernel dispatch stamps them with its own
    start and end (swa_prefill_timed)."""
    if q.dim() != 4:
        raise ValueError("q must be [B][L][Hq][d]")
    B, L, Hq, d = q.shape
    Hkv = k.shape[2] if k.dim() == 4 else -1
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16, (B, L, Hkv, d))
    _need(v, "v", torch.bfloat16, (B, L, Hkv, d))
    if out is None:
        out = torch.empty((B, L, Hq, d), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (B, L, Hq, d))
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if events is None:
        _check(lib().swa_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, Hq, Hkv, L, d,
                                 w, s, scale, conv, _stream(q)))
    else:
        start, stop = events
        _check(lib().swa_prefill_timed(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, Hq, Hkv, L,
                                       d, w, s, scale, conv, _stream(q), start.cuda_event, stop.cuda_event))
    return out


def decode_describe(B: int, Hq: int, Hkv: int, d: int, w: int, s: int, conv: int = ADDITIVE) -> dict:
    """How the decode step splits this shape (swa_decode_describe)."""
    info = _DecodeInfoC()
    _check(lib().swa_decode_describe(B, Hq, Hkv, d, w, s, conv, ctypes.byref(info)))
    return {f: getattr(info, f) for f, _ in _DecodeInfoC._fields_}


def alloc_cache(B: int, Hkv: int, d: int, w: int, s: int, conv: int = ADDITIVE, device="cuda"):
    """Empty (k_cache, v_cache), bf16 [B][Hkv][s + w_loc][d] each."""
    n = cache_slots(w, s, conv)
    k = torch.zeros((B, Hkv, n, d), dtype=torch.bfloat16, device=device)
    return k, torch.zeros_like(k)


def kv_append(k_cache, v_cache, k_new, v_new, pos, w: int, s: int, conv: int = ADDITIVE):
    """Write k_new/v_new bf16 [B][n_new][Hkv][d] at positions pos[b] .. pos[b]+n_new-1."""
    B, Hkv, n_slots, d = k_cache.shape
    n_new = k_new.shape[1]
    if n_slots != cache_slots(w, s, conv):
        raise ValueError("cache slot count does not match s + w_loc")
    _need(k_cache, "k_cache", torch.bfloat16)
    _need(v_cache, "v_cache", torch.bfloat16, k_cache.shape)
    _need(k_new, "k_new", torch.bfloat16, (B, n_new, Hkv, d))
    _need(v_new, "v_new", torch.bfloat16, (B, n_new, Hkv, d))
    _need(pos, "pos", torch.int64, (B,))
    _check(lib().swa_kv_append(k_cache.data_ptr(), v_cache.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                               pos.data_ptr(), B, Hkv, d, w, s, n_new, conv, _stream(k_cache)))


def decode_workspace_bytes(B: int, Hq: int, Hkv: int, d: int, w: int, s: int, conv: int = ADDITIVE) -> int:
    return int(lib().swa_decode_workspace_bytes(B, Hq, Hkv, d, w, s, conv))


def alloc_workspace(B: int, Hq: int, Hkv: int, d: int, w: int, s: int, conv: int = ADDITIVE, device="cuda"):
    n = decode_workspace_bytes(B, Hq, Hkv, d, w, s, conv)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def decode_step(q, k_cache, v_cache, pos, w: int, s: int, scale: float | None = None, conv: int = ADDITIVE,
                out=None, workspace=None):
    """One-token decode: q bf16 [B][Hq][d] at positions pos[b] (already appended) -> fp32 [B][Hq][d]."""
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    _need(q, "q", torch.bfloat16)
    _need(k_cache, "k_cache", torch.bfloat16, (B, Hkv, cache_slots(w, s, conv), d))
    _need(v_cache, "v_cache", torch.bfloat16, k_cache.shape)
    _need(pos, "pos", torch.int64, (B,))
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (B, Hq, d))
    need = decode_workspace_bytes(B, Hq, Hkv, d, w, s, conv)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr, ws_bytes = (0, 0) if workspace is None else (workspace.data_ptr(), workspace.numel() * workspace.element_size())
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _check(lib().swa_decode_step(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(),
                                 pos.data_ptr(), B, Hq, Hkv, d, w, s, scale, conv, ws_ptr or None, ws_bytes,
                                 _stream(q)))
    return out


def decode_step_noalloc(q, k_cache, v_cache, pos, w: int, s: int, scale: float | None = None,
                        conv: int = ADDITIVE, out=None):
    """decode_step with the library's static scratch in place of a workspace
    (swa_decode_step_noalloc: no device allocation by the library)."""
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    _need(q, "q", torch.bfloat16)
    _need(k_cache, "k_cache", torch.bfloat16, (B, Hkv, cache_slots(w, s, conv), d))
    _need(v_cache, "v_cache", torch.bfloat16, k_cache.shape)
    _need(pos, "pos", torch.int64, (B,))
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (B, Hq, d))
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _check(lib().swa_decode_step_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(),
                                         pos.data_ptr(), B, Hq, Hkv, d, w, s, scale, conv, _stream(q)))
    return out


def append_decode_step(q, k_cache, v_cache, k_new, v_new, pos, w: int, s: int, scale: float | None = None,
                       conv: int = ADDITIVE, out=None, workspace=None, events=None):
    """kv_append of one token per sequence (k_new/v_new bf16 [B][Hkv][d] at positions pos[b])
    and decode_step for the query at that position, in one launch -> fp32 [B][Hq][d].

    events: optional (start, stop) torch.cuda.Event pair (timing enabled, already recorded once
    so that the HIP events exist); the kernel dispatches stamp them (swa_append_decode_step_timed)."""
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    _need(q, "q", torch.bfloat16)
    _need(k_cache, "k_cache", torch.bfloat16, (B, Hkv, cache_slots(w, s, conv), d))
    _need(v_cache, "v_cache", torch.bfloat16, k_cache.shape)
    _need(k_new, "k_new", torch.bfloat16, (B, Hkv, d))
    _need(v_new, "v_new", torch.bfloat16, (B, Hkv, d))
    _need(pos, "pos", torch.int64, (B,))
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (B, Hq, d))
    need = decode_workspace_bytes(B, Hq, Hkv, d, w, s, conv)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr, ws_bytes = (0, 0) if workspace is None else (workspace.data_ptr(), workspace.numel() * workspace.element_size())
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    args = (q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), out.data_ptr(),
            pos.data_ptr(), B, Hq, Hkv, d, w, s, scale, conv, ws_ptr or None, ws_bytes, _stream(q))
    if events is None:
        _check(lib().swa_append_decode_step(*args))
    else:
        _check(lib().swa_append_decode_step_timed(*args, events[0].cuda_event, events[1].cuda_event))
    return out


def prefill_chunk(q, k, v, k_cache, v_cache, pos0: int, w: int, s: int, scale: float | None = None,
                  conv: int = ADDITIVE, out=None, lse=None):
    """Prefill of a chunk at positions pos0 .. pos0+C-1 against the cache (state after pos0-1),
    then the chunk appended.  q bf16 [B][C][Hq][d], k/v bf16 [B][C][Hkv][d] -> fp32 [B][C][Hq][d].
    lse: optional fp32 [B][C][Hq] that receives ln of each row's softmax denominator."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B][C][Hq][d] and k, v [B][C][Hkv][d]")
    B, C, Hq, d = q.shape
    Hkv = k.shape[2]
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16, (B, C, Hkv, d))
    _need(v, "v", torch.bfloat16, (B, C, Hkv, d))
    n_slots = cache_slots(w, s, conv)
    _need(k_cache, "k_cache", torch.bfloat16, (B, Hkv, n_slots, d))
    _need(v_cache, "v_cache", torch.bfloat16, (B, Hkv, n_slots, d))
    if out is None:
        out = torch.empty((B, C, Hq, d), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (B, C, Hq, d))
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, C, Hq))
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _check(lib().swa_prefill_chunk(q.data_ptr(), k.data_ptr(), v.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                   out.data_ptr(), None if lse is None else lse.data_ptr(), int(pos0), B, Hq, Hkv, C,
                                   d, w, s, scale, conv, _stream(q)))
    return out


def debug_prefill_mask(L: int, Hq: int, Hkv: int, w: int, s: int, conv: int = ADDITIVE, device="cuda", d: int = 128):
    """uint8 [L][L]: how often the prefill kernel launched for these arguments attends to each
    (query, key) pair (1 on A(t) and 0 elsewhere for a correct kernel)."""
    m = torch.empty((L, L), dtype=torch.uint8, device=device)
    _check(lib().swa_debug_prefill_mask(m.data_ptr(), L, Hq, Hkv, d, w, s, conv, _stream(m)))
    return m


def debug_decode_slots(pos, w: int, s: int, conv: int = ADDITIVE):
    """int64 [B][s + w_loc]: position the decode kernel reads from each slot, -1 if skipped."""
    _need(pos, "pos", torch.int64)
    B = pos.shape[0]
    out = torch.empty((B, cache_slots(w, s, conv)), dtype=torch.int64, device=pos.device)
    _check(lib().swa_debug_decode_slots(out.data_ptr(), pos.data_ptr(), B, w, s, conv, _stream(pos)))
    return out


# ------------------------------------------------------------------ decoder-layer pieces

def rmsnorm(x, weight, eps: float, out=None):
    """bf16 [B][n] = bf16(x / sqrt(mean(x^2) + eps) * weight); x fp32 [B][n], weight bf16 [n]."""
    B, n = x.shape
    _need(x, "x", torch.float32)
    _need(weight, "weight", torch.bfloat16, (n,))
    if out is None:
        out = torch.empty((B, n), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, (B, n))
    _check(lib().swa_rmsnorm(x.data_ptr(), weight.data_ptr(), out.data_ptr(), B, n, float(eps), _stream(x)))
    return out


def linear(W, x, mode: str = "store", out=None):
    """y = W x over x [B][K] (bf16, or fp32 rounded to bf16 on read), fp32 accumulation.

    mode "store": W bf16 [N][K] -> bf16 [B][N]; "add": W [N][K], out fp32 [B][N] += y (out
    required); "silu_mul": W [2N][K] (gate rows, then up rows) -> bf16 silu(gate) * up [B][N].
    """
    B, K = x.shape
    if x.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("x must be bf16 or fp32")
    _need(x, "x", x.dtype)
    _need(W, "W", torch.bfloat16)
    if W.dim() != 2 or W.shape[1] != K:
        raise ValueError(f"W must be [N][{K}]")
    m = LINEAR_MODES[mode]
    N = W.shape[0] // 2 if mode == "silu_mul" else W.shape[0]
    if mode == "add":
        if out is None:
            raise ValueError("mode 'add' accumulates into out, which must be given")
        _need(out, "out", torch.float32, (B, N))
    else:
        if out is None:
            out = torch.empty((B, N), dtype=torch.bfloat16, device=x.device)
        _need(out, "out", torch.bfloat16, (B, N))
    _check(lib().swa_linear(W.data_ptr(), x.data_ptr(), int(x.dtype == torch.float32), out.data_ptr(), m, B, N, K,
                            _stream(x)))
    return out


def layer_workspace_bytes(B: int, dm: int, Hq: int, Hkv: int, d: int, f: int, w: int, s: int,
                          conv: int = ADDITIVE) -> int:
    return int(lib().swa_layer_workspace_bytes(B, dm, Hq, Hkv, d, f, w, s, conv))


def layer_decode_step(x, weights: dict, k_cache, v_cache, pos, Hq: int, w: int, s: int, scale: float | None = None,
                      conv: int = ADDITIVE, eps: float = 1e-5, workspace=None):
    """One decode step of one decoder layer; x fp32 [B][dm] is updated in place.

    weights: dict of bf16 tensors attn_norm [dm], w_qkv [(Hq + 2 Hkv) d][dm], w_o [dm][Hq d],
    mlp_norm [dm], w_gate_up [2 f][dm], w_down [dm][f].  k_cache/v_cache: this layer's bf16
    [B][Hkv][s + w_loc][d]; pos int64 [B]: position of this step's token.
    """
    B, dm = x.shape
    _, Hkv, n_slots, d = k_cache.shape
    f = weights["w_down"].shape[1]
    _need(x, "x", torch.float32)
    _need(k_cache, "k_cache", torch.bfloat16, (B, Hkv, cache_slots(w, s, conv), d))
    _need(v_cache, "v_cache", torch.bfloat16, k_cache.shape)
    _need(pos, "pos", torch.int64, (B,))
    shapes = {"attn_norm": (dm,), "w_qkv": ((Hq + 2 * Hkv) * d, dm), "w_o": (dm, Hq * d), "mlp_norm": (dm,),
              "w_gate_up": (2 * f, dm), "w_down": (dm, f)}
    for name, shape in shapes.items():
        _need(weights[name], name, torch.bfloat16, shape)
    cw = _LayerWeightsC(*[weights[n].data_ptr() for n in shapes])
    need = layer_workspace_bytes(B, dm, Hq, Hkv, d, f, w, s, conv)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _check(lib().swa_layer_decode_step(x.data_ptr(), ctypes.byref(cw), k_cache.data_ptr(), v_cache.data_ptr(),
                                       pos.data_ptr(), B, dm, Hq, Hkv, d, f, w, s, scale, conv, float(eps),
                                       workspace.data_ptr(), workspace.numel(), _stream(x)))
    return x


def _ints(xs):
    return (ctypes.c_int * len(xs))(*[int(x) for x in xs])


def stack_workspace_bytes(windows, B: int, dm: int, Hq: int, Hkv: int, d: int, f: int) -> int:
    """Workspace of swa_stack_decode_step for layers with windows [(w, s, conv)]."""
    n = len(windows)
    return int(lib().swa_stack_workspace_bytes(n, _ints([w for w, _, _ in windows]), _ints([s for _, s, _ in windows]),
                                               _ints([c for _, _, c in windows]), B, dm, Hq, Hkv, d, f))


def stack_decode_step(x, layers, pos, Hq: int, scale: float | None = None, eps: float = 1e-5, workspace=None):
    """One decode step through a stack of decoder layers (swa_stack_decode_step); x fp32 [B][dm]
    is updated in place.

    layers: list of (weights, k_cache, v_cache, w, s, conv), each as for layer_decode_step; a
    global layer is a window at least as long as the context with s = 0.
    """
    B, dm = x.shape
    _need(x, "x", torch.float32)
    _need(pos, "pos", torch.int64, (B,))
    _, Hkv, _, d = layers[0][1].shape
    f = layers[0][0]["w_down"].shape[1]
    names = ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate_up", "w_down")
    shapes = {"attn_norm": (dm,), "w_qkv": ((Hq + 2 * Hkv) * d, dm), "w_o": (dm, Hq * d), "mlp_norm": (dm,),
              "w_gate_up": (2 * f, dm), "w_down": (dm, f)}
    n = len(layers)
    cws = (_LayerWeightsC * n)()
    kcs, vcs = (ctypes.c_void_p * n)(), (ctypes.c_void_p * n)()
    for i, (wts, kc, vc, w, s, conv) in enumerate(layers):
        for name in names:
            _need(wts[name], name, torch.bfloat16, shapes[name])
        _need(kc, "k_cache", torch.bfloat16, (B, Hkv, cache_slots(w, s, conv), d))
        _need(vc, "v_cache", torch.bfloat16, kc.shape)
        cws[i] = _LayerWeightsC(*[wts[m].data_ptr() for m in names])
        kcs[i], vcs[i] = kc.data_ptr(), vc.data_ptr()
    windows = [(w, s, conv) for _, _, _, w, s, conv in layers]
    if workspace is None:
        workspace = torch.empty(max(stack_workspace_bytes(windows, B, dm, Hq, Hkv, d, f), 1), dtype=torch.uint8,
                                device=x.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _check(lib().swa_stack_decode_step(x.data_ptr(), n, cws, kcs, vcs, _ints([w for w, _, _ in windows]),
                                       _ints([s for _, s, _ in windows]), _ints([c for _, _, c in windows]),
                                       pos.data_ptr(), B, dm, Hq, Hkv, d, f, scale, float(eps), workspace.data_ptr(),
                                       workspace.numel(), _stream(x)))
    return x
