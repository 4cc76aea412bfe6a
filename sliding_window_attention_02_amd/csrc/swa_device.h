// swa_device.h -- index arithmetic shared by the SWA(w,s) kernels and their debug dumps.
//
// Everything that decides WHICH keys a query sees lives here, so the hot kernels and
// the test hooks (swa_debug_prefill_mask / swa_debug_decode_slots) run the same code.
//
// Allowed set (0-based): A(t) = { i <= t : i >= t - w_loc + 1 or i < s }.  Sources:
// page "滑动窗口注意力（SWA）配 sinks 比 post-training 线性注意力更划算" (papers.ananclaw.com),
// section 核心方法 1 (x_t equation, swa_mask recipe), read causally; page
// "从长文档摘要说起" (wiblog.cn), section "SWA 的核心机制" (window of W keys ending at i).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swa {

// Element predicate of A(t).
__device__ __forceinline__ bool key_allowed(int t, int i, int w_loc, int s)
{
    return i <= t && (i > t - w_loc || i < s);
}

// ----------------------------------------------------------------------------- prefill
//
// A workgroup owns the queries of tokens [t0, t1] (t1 clamped to L-1).  Its key tiles
// of kTileN keys are the sink tiles [0, n_sink) followed by the window tiles
// [win_lo, win_hi]; no other tile holds a key of A(t) for any t in [t0, t1], so the
// L x L mask is never formed and every other tile is skipped (loads and exp alike).
struct TileWalk {
    int n_sink;  // tiles 0 .. n_sink-1 hold sinks below the window
    int win_lo;  // first window tile
    int win_hi;  // last window tile
    __device__ __forceinline__ int count() const { return n_sink + (win_hi - win_lo + 1); }
    __device__ __forceinline__ int tile(int n) const { return n < n_sink ? n : win_lo + (n - n_sink); }
};

__device__ __forceinline__ TileWalk plan_tiles(int t0, int t1, int w_loc, int s, int tile_n)
{
    TileWalk tw;
    const int lo = (t0 - w_loc + 1 > 0) ? t0 - w_loc + 1 : 0;  // first window key of token t0
    tw.win_lo = lo / tile_n;
    tw.win_hi = t1 / tile_n;
    const int sink_keys = s < t1 + 1 ? s : t1 + 1;
    const int sink_tiles = (sink_keys + tile_n - 1) / tile_n;
    tw.n_sink = sink_tiles < tw.win_lo ? sink_tiles : tw.win_lo;
    return tw;
}

// True when every (t, i) with t in [t0, t1] and i in the tile starting at j0 is allowed,
// so the tile needs no element mask.
__device__ __forceinline__ bool tile_mask_free(int j0, int tile_n, int t0, int t1, int w_loc, int s)
{
    const int j1 = j0 + tile_n - 1;
    const bool causal = j1 <= t0;
    const bool in_window = j0 > t1 - w_loc;
    const bool all_sinks = j1 < s;
    return causal && (in_window || all_sinks);
}

// ------------------------------------------------------------------------------ decode
//
// Cache of s pinned sink slots followed by a ring of w_loc slots.  Position p lives in
// slot p (p < s) or s + (p mod w_loc).  Rotation: page "从长文档摘要说起", section
// "与 KV Cache 的配合：轮转替换策略" (evict the oldest entry; circular buffer indexed
// modulo the window).

__device__ __forceinline__ int64_t append_slot(int64_t p, int s, int w_loc)
{
    return p < s ? p : s + (p % w_loc);
}

// Position held by slot j when the latest appended position is t, or -1 when the slot
// holds nothing in A(t) (a sink slot beyond t, or a ring slot whose latest position
// would be a sink or negative).
__device__ __forceinline__ int64_t slot_position(int j, int64_t t, int s, int w_loc)
{
    if (j < s)
        return (int64_t)j <= t ? (int64_t)j : -1;
    const int64_t r = j - s;
    int64_t back = (t - r) % w_loc;
    if (back < 0)
        back += w_loc;
    const int64_t p = t - back;
    return (p >= s && p >= 0) ? p : -1;
}

}  // namespace swa
