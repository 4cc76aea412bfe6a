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

// LDS pointer in the local address space, as the direct global -> LDS load takes it.  The
// cast is written inline: an implicit conversion (or a helper function) there makes the host
// pass drop the kernel's launch stub.
#define SWA_LDS_PTR(p) ((__attribute__((address_space(3))) void *)(p))
// The same pointer, opaque to the compiler: a direct load given it carries no alias information
// about its LDS destination, so the compiler does not order later LDS reads after it.  Without
// this, a read from one stage of a double buffer while loads into the other stage are in flight
// (or any such read at a loop head) gets a wait for every outstanding vector-memory operation.
// Every kernel here orders its loads and reads itself: counted waits on this wave's loads, then
// a barrier for the other waves' loads.
#define SWA_LDS_DMA_DST(p)                                                                        \
    ({                                                                                           \
        __attribute__((address_space(3))) void *lds_dma_dst_ = SWA_LDS_PTR(p);                   \
        asm volatile("" : "+s"(lds_dma_dst_));                                                   \
        lds_dma_dst_;                                                                            \
    })

namespace swa {

// The walk and index functions below run in the kernels and on the host (work accounting).
#define SWA_HD __host__ __device__ __forceinline__

// Element predicate of A(t) (bitwise on the comparisons: no branches in the kernels' masks).
SWA_HD bool key_allowed(int t, int i, int w_loc, int s)
{
    return (i <= t) & ((i > t - w_loc) | (i < s));
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
    SWA_HD int count() const { return n_sink + (win_hi - win_lo + 1); }
    SWA_HD int tile(int n) const { return n < n_sink ? n : win_lo + (n - n_sink); }
};

SWA_HD TileWalk plan_tiles(int t0, int t1, int w_loc, int s, int tile_n)
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

// The window tiles all of whose keys every token of [t0, t1] may see (each key is at most t0 and
// inside the window of t1) need neither a chunk selection nor an element mask: they are the
// middle tiles [mid_lo, mid_hi] (none when mid_lo > mid_hi).  The other tiles of the walk are
// its edge tiles, visited in walk order by edge_tile(i), i < n_edge.
struct WalkSplit {
    int mid_lo, mid_hi, n_edge;
    SWA_HD int n_mid() const { return mid_hi >= mid_lo ? mid_hi - mid_lo + 1 : 0; }
    SWA_HD int edge_tile(const TileWalk &tw, int i) const
    {
        if (i < tw.n_sink)
            return i;
        int t = tw.win_lo + (i - tw.n_sink);
        if (t >= mid_lo)
            t += n_mid();
        return t;
    }
};

SWA_HD WalkSplit split_walk(const TileWalk &tw, int t0, int t1, int w_loc, int tile_n)
{
    WalkSplit sp;
    const int lo = t1 - w_loc + 1;  // first key inside the window of t1
    const int first = lo > 0 ? (lo + tile_n - 1) / tile_n : 0;
    sp.mid_lo = first > tw.win_lo ? first : tw.win_lo;
    const int last = (t0 + 1) / tile_n - 1;  // last tile whose keys are all <= t0
    sp.mid_hi = last < tw.win_hi ? last : tw.win_hi;
    sp.n_edge = tw.count() - sp.n_mid();
    return sp;
}

// The kChunkN-key chunks (kChunkN below) holding a key of A(t) for some t in [t0, t1]: the sink
// chunks below the window's first chunk, then the window's chunks, in that order.  The chunk
// walk of the resident prefill, which keeps every chunk of a q-tile in LDS at once.
struct ChunkWalk {
    int n_sink;          // chunks 0 .. n_sink-1 (sinks below the window)
    int win_lo, win_hi;  // window chunks
    SWA_HD int count() const { return n_sink + (win_hi - win_lo + 1); }
    SWA_HD int chunk(int k) const { return k < n_sink ? k : win_lo + (k - n_sink); }
};

SWA_HD ChunkWalk plan_chunks(int t0, int t1, int w_loc, int s, int chunk_n)
{
    ChunkWalk cw;
    const int lo = (t0 - w_loc + 1 > 0) ? t0 - w_loc + 1 : 0;
    cw.win_lo = lo / chunk_n;
    cw.win_hi = t1 / chunk_n;
    const int sink_keys = s < t1 + 1 ? s : t1 + 1;
    const int sink_chunks = (sink_keys + chunk_n - 1) / chunk_n;
    cw.n_sink = sink_chunks < cw.win_lo ? sink_chunks : cw.win_lo;
    return cw;
}

// A tile is processed in chunks of kChunkN keys.  Sets [c_lo, c_hi], the smallest chunk
// range that covers every chunk holding a key of A(t) for some t in [t0, t1] (the needed
// keys of a q-tile are the sinks [0, min(s, t1+1)) and the window [max(0, t0-w_loc+1), t1]);
// chunks outside the range are skipped, loads and exp alike.
constexpr int kChunkN = 32;

SWA_HD void tile_chunks(int j0, int n_chunks, int t0, int t1, int w_loc, int s, int &c_lo, int &c_hi)
{
    const int lo = (t0 - w_loc + 1 > 0) ? t0 - w_loc + 1 : 0;
    const int sink_end = s < t1 + 1 ? s : t1 + 1;
    c_lo = n_chunks;
    c_hi = -1;
    for (int c = 0; c < n_chunks; ++c) {
        const int a = j0 + c * kChunkN, b = a + kChunkN - 1;
        const bool need = a < sink_end || (b >= lo && a <= t1);
        if (need) {
            c_lo = c < c_lo ? c : c_lo;
            c_hi = c;
        }
    }
}

// True when every (t, i) with t in [t0, t1] and i in [k_lo, k_hi] is allowed, so those
// keys need no element mask.
SWA_HD bool range_mask_free(int k_lo, int k_hi, int t0, int t1, int w_loc, int s)
{
    const bool causal = k_hi <= t0;
    const bool in_window = k_lo > t1 - w_loc;
    const bool all_sinks = k_hi < s;
    return causal && (in_window || all_sinks);
}

// Key tile of the main prefill walk: first key, needed chunk range, and whether every visited
// (query, key) pair is allowed (then no element mask is applied).
struct TileInfo {
    int j0, c_lo, c_hi;
    int mask_free;  // (an int: a bool member would leave padding that the copies carry)
    SWA_HD bool full() const { return c_lo == 0 && c_hi == 1 && mask_free; }
};

SWA_HD TileInfo tile_info(int tile, int tile_n, int t0, int t1, int w_loc, int s)
{
    TileInfo ti;
    ti.j0 = tile * tile_n;
    tile_chunks(ti.j0, tile_n / kChunkN, t0, t1, w_loc, s, ti.c_lo, ti.c_hi);
    ti.mask_free = range_mask_free(ti.j0 + ti.c_lo * kChunkN, ti.j0 + ti.c_hi * kChunkN + kChunkN - 1, t0, t1,
                                   w_loc, s);
    return ti;
}

// Resident prefill forms: chunk slot k of a workgroup whose chunk walk is cw holds the keys
// resident_slot_key0(cw, k) + r, r < kChunkN (rows past the sequence hold its last key).
SWA_HD int resident_slot_key0(const ChunkWalk &cw, int k) { return cw.chunk(k) * kChunkN; }

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

// Slot -> position map for a query at position t (the latest appended position): slot j
// holds position(j), or -1 when the slot holds nothing in A(t) (a sink slot beyond t, or a
// ring slot whose latest position would be a sink or negative).  The one modulo is taken at
// construction (32-bit unless t needs 64); position() is 32-bit arithmetic plus one 64-bit
// subtraction.
struct SlotMap {
    int64_t t;
    int s, w_loc, t_mod;
    int t_clamp;  // min(t, 2^31 - 1), or -1 for t < 0: enough to decide validity in 32 bits
    __device__ __forceinline__ SlotMap(int64_t t_, int s_, int w_loc_) : t(t_), s(s_), w_loc(w_loc_)
    {
        if (t_ < 0)
            t_mod = 0;
        else if (t_ <= 0x7fffffffLL)
            t_mod = (int)((uint32_t)t_ % (uint32_t)w_loc_);
        else
            t_mod = (int)(t_ % w_loc_);
        t_clamp = t_ < 0 ? -1 : (t_ > 0x7fffffffLL ? 0x7fffffff : (int)t_);
    }
    __device__ __forceinline__ int64_t position(int j) const
    {
        if (j < s)
            return (int64_t)j <= t ? (int64_t)j : -1;
        // ring slot r = j - s holds the latest p <= t with p = r (mod w_loc):
        // p = t - ((t - r) mod w_loc) and (t - r) mod w_loc = (t_mod - r) mod w_loc
        int back = t_mod - (j - s);
        if (back < 0)
            back += w_loc;
        const int64_t p = t - back;
        return (p >= s && p >= 0) ? p : -1;
    }
    __device__ __forceinline__ bool valid(int j) const { return position(j) >= 0; }
    // valid(j) in 32-bit arithmetic, branch-free: a sink slot j < s is valid iff j <= t; a
    // ring slot holds p = t - back with back = (t_mod - (j - s)) mod w_loc < w_loc, valid iff
    // p >= s, i.e. back <= t - s (t_clamp keeps that exact when t >= 2^31, as back < 2^31).
    __device__ __forceinline__ bool valid32(int j) const
    {
        int back = t_mod - (j - s);
        back += back < 0 ? w_loc : 0;
        return ((j < s) & (j <= t_clamp)) | ((j >= s) & (back <= t_clamp - s));
    }
    // slot of position t itself (t >= 0)
    __device__ __forceinline__ int slot_of_t() const { return t < s ? (int)t : s + t_mod; }
    // Once the ring has wrapped (t >= s + w_loc - 1) every slot holds a position of A(t).
    __device__ __forceinline__ bool wrapped() const { return t >= (int64_t)s + w_loc - 1; }
    // Whether the decode step attends to slot j of a split segment ending at seg_hi (rows past the
    // segment repeat its last slot): after the wrap every slot of the segment, before it the
    // slots that valid32 admits.  `wrap` is wrapped(), passed in so that a caller branching on
    // it gets straight-line code in each branch.
    __device__ __forceinline__ bool admits(int j, int seg_hi, bool wrap) const
    {
        return (j < seg_hi) & (wrap | valid32(j));
    }
};

}  // namespace swa
