// swa_launch.h -- host-side launchers shared between the C ABI and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace swa {

// ----------------------------------------------------------------------------- prefill
//
// A workgroup computes `rows` query rows (128; 64 for the small-grid forms): Tm
// consecutive tokens times Gw q-heads of one kv-head (GQA packing), so each K/V tile staged in
// LDS serves Gw heads at once.
struct PrefillGeometry {
    int G;          // q-heads per kv-head
    int Gw;         // q-heads per workgroup (largest divisor of G that is <= 4)
    int rows;       // query rows per workgroup
    int Tm;         // tokens per workgroup (rows / Gw)
    int n_hslices;  // G / Gw
    int n_qtiles;   // ceil(L / Tm)
};
// The geometry of kernel form `form` (0 tile walk, 1 resident; 2 resident and 3 tile walk with
// 64-row workgroups) over L query tokens.
PrefillGeometry prefill_geometry(int L, int Hq, int Hkv, int form);
// Whether q-tiles of Tm tokens starting at q_lo need at most four 32-key chunks for any q-tile:
// then the prefill keeps all of a q-tile's keys in LDS at once (the resident form).
bool prefill_resident(int Tm, int q_lo, int w_loc, int s);
// The form launched for Lq queries (per sequence, B sequences) starting at key index q_lo:
// resident where its bound holds for its q-tiles, else the tile walk; each with 64-row workgroups
// when the 128-row grid would be small.
int prefill_form(int B, int Hq, int Hkv, int Lq, int q_lo, int w_loc, int s);

// What launch_prefill launches for a whole-sequence prefill: the kernel form (0 tile walk,
// 1 resident), the geometry as launched, the grid,
// and the (query row, key) pairs whose scores and value products the matrix cores compute (rows of
// a workgroup times the keys of the tiles or chunks it visits, padding rows included).
struct PrefillPlan {
    int form;
    PrefillGeometry g;
    long long workgroups;
    long long executed_pairs;
};
PrefillPlan prefill_plan(int B, int Hq, int Hkv, int L, int w_loc, int s);

// Chunked prefill: the first n_cached of the L keys are read from a sink+ring cache
// [B][Hkv][s + w_loc][d] (key j < ns: sink slot j; key j >= ns: ring slot
// s + (ring0 + j - ns) mod w_loc), the rest from k and v, which hold L - n_cached rows; only
// the last L - n_cached keys are queries (q and out hold L - n_cached rows).
struct PrefillKeySource {
    const void *k_cache, *v_cache;
    int n_cached, ns, ring0;
};

// start/stop: optional events stamped by the kernel dispatch itself (null: plain launch).
// cached: null for a whole-sequence prefill.  lse: optional fp32 [B][L - n_cached][Hq], ln of each
// query row's softmax denominator.
hipError_t launch_prefill(const void *q, const void *k, const void *v, float *out, int B, int Hq,
                          int Hkv, int L, int d, int w_loc, int s, float scale, hipStream_t stream,
                          hipEvent_t start = nullptr, hipEvent_t stop = nullptr,
                          const PrefillKeySource *cached = nullptr, float *lse = nullptr);

hipError_t launch_debug_prefill_mask(uint8_t *mask, int L, int Hq, int Hkv, int d, int w_loc, int s,
                                     hipStream_t stream);

// ------------------------------------------------------------------------------ decode
struct DecodePlan {
    int n_slots;          // s + w_loc
    int Gb;               // q-heads per workgroup (largest divisor of G that is <= 16)
    int n_hslices;        // G / Gb
    int n_split;          // splits of the slot range of one (b, kv-head, head slice)
    int wg_waves;         // splits per workgroup (one wave each): 1, or n_split (merged in LDS)
    int slots_per_split;  // slots per split
    size_t workspace_bytes;
};
DecodePlan decode_plan(int B, int Hq, int Hkv, int d, int w_loc, int s);

// The static scratch of swa_decode_step_noalloc: its size, and its address on the current device
// (taken once per device with hipGetSymbolAddress, then cached).
size_t scratch_capacity();
hipError_t scratch_pointer(void **ptr);

// pos: device [B] first positions, or null to append every sequence at pos0.
hipError_t launch_kv_append(void *k_cache, void *v_cache, const void *k_new, const void *v_new,
                            const int64_t *pos, int B, int Hkv, int d, int w_loc, int s, int n_new,
                            hipStream_t stream, int64_t pos0 = 0);

// k_new / v_new: null for a plain decode step; otherwise the new token of each sequence
// ([B][Hkv][d]) is written to its slot and attended in the same launch.  start/stop: optional
// events stamped by the dispatches themselves (the first kernel's start, the last kernel's end).
hipError_t launch_decode(const void *q, void *k_cache, void *v_cache, const void *k_new, const void *v_new,
                         float *out, const int64_t *pos, int B, int Hq, int Hkv, int d, int w_loc, int s,
                         float scale, void *workspace, const DecodePlan &plan, hipStream_t stream,
                         hipEvent_t start = nullptr, hipEvent_t stop = nullptr);

// ----------------------------------------------------------------------- chunked prefill
//
// A chunk of C tokens at positions pos0 .. pos0 + C - 1 against a cache that holds the state
// after pos0 - 1.  Its keys, in position order, are ns cached sinks, nw cached window positions
// (pos0 - nw .. pos0 - 1) and the chunk itself: a sequence of rows = ns + nw + C keys whose
// queries are the last C, on which the SWA(w,s) predicate holds unchanged (the window rows
// hold no sink positions and run contiguously into the chunk).
struct ChunkPlan {
    int ns;     // min(s, pos0)
    int nw;     // min(w_loc - 1, pos0 - s) when pos0 > s, else 0
    int rows;   // ns + nw + C
    int ring0;  // (pos0 - nw) mod w_loc: ring slot s + ring0 holds the first window key
};
ChunkPlan chunk_plan(int64_t pos0, int C, int w_loc, int s);

// ---------------------------------------------------------------- decoder-layer pieces
//
// out bf16 [B][n] = bf16(x / sqrt(mean(x^2) + eps) * g), x fp32 [B][n], g bf16 [n]; n % 4 == 0.
hipError_t launch_rmsnorm(const float *x, const void *g, void *out, int B, int n, float eps, hipStream_t stream);

// y = W x for x [B][K] (bf16, or fp32 rounded to bf16 on read when x_f32), K % 8 == 0:
//   LIN_STORE    W [N][K]; outputs [seg[i], seg[i+1]) -> out_bf16[i] as bf16 [B][seg[i+1] - seg[i]]
//   LIN_ADD      W [N][K]; out_f32 [B][N] += y
//   LIN_SILU_MUL W [2N][K] (gate rows, then up rows); out_bf16[0] [B][N] = bf16(silu(gate) * up)
enum { LIN_STORE = 0, LIN_ADD = 1, LIN_SILU_MUL = 2 };
hipError_t launch_linear(int mode, bool x_f32, const void *W, const void *x, int B, int N, int K,
                         void *const out_bf16[3], const int seg[4], float *out_f32, hipStream_t stream);

hipError_t launch_debug_decode_slots(int64_t *slot_pos, const int64_t *pos, int B, int w_loc, int s,
                                     hipStream_t stream);

}  // namespace swa
