// swa_prefill.hip -- SWA(w,s) causal prefill for gfx950 (MI355X): bf16 MFMA, fp32 online softmax.
//
// Operation: out[b][t][h] = sum_{i in A(t)} softmax(scale <q_t, k_i>) v_i with
// A(t) = { i <= t : i > t - w_loc or i < s }  (page "滑动窗口注意力（SWA）配 sinks 比
// post-training 线性注意力更划算", section 核心方法 1: x_t equation and swa_mask recipe).
// Only key tiles meeting A(t) are visited, the tile skipping described on page
// "Hybrid Sliding Window Attention", section 三.3.  The online softmax (running maximum,
// rescaled running sum) is the published method of Milakov & Gimelshein (2018).
//
// Workgroup: 256 threads = 4 waves, 128 query rows = Tm tokens x Gw q-heads of one
// kv-head.  Wave w owns rows 32w .. 32w+31 as two 16-column MFMA blocks (64-row forms: rows
// 16w .. 16w+15, one block).
//
// Matrix layout trick.  With v_mfma_f32_16x16x32_bf16, lane l holds row (l % 16) of the
// A operand and column (l % 16) of the B operand, eight k-values each, and receives
// rows 4*(l/16) .. +3 of column (l % 16) of the result.  The kernel computes
//     S^T (keys x queries) = K (keys x d) . Q^T (d x queries)
// so each lane ends up with the scores of ONE query column for a few keys; the
// probabilities P^T then already sit in the B-operand layout of
//     O^T (d x queries) += V^T (d x keys) . P^T (keys x queries)
// and the per-query softmax statistics (max, sum) only combine the four lanes
// l % 16 + 16g that share a column.  The 16-key row blocks of S^T are assigned keys so
// that lane group g of the PV product sees the 8 consecutive keys 32*kc + 8g .. +7, which
// two transposed 8-byte LDS reads of row-major V deliver as the V^T A operand.  Any
// k-ordering the hardware uses inside the 8-value groups is the same for A and B, so the
// contraction is exact regardless.
//
// Memory: K and V tiles of 64 keys go from global memory straight into LDS (direct
// global -> LDS loads, double-buffered, one barrier per tile), both row-major with the
// 16-byte pieces of each row XOR-swizzled so that the K fragment reads hit distinct banks and
// the transposed V reads (ds_read_b64_tr_b16) spread over distinct pieces.  Q stays in registers for the
// whole key loop.  Workgroups are ordered heavy-first (last q-tile first) and mapped so
// that consecutive logical workgroups share an XCD and its L2, where neighbouring q-tiles
// re-read the same K/V tiles.  The fp32 output goes out in whole 128-byte lines with
// non-temporal stores (store_pair).
//
// Two kinds of form.  The tile walk (main form) goes through the tiles with a running softmax:
// edge tiles one per step, then the middle tiles through a software pipeline.  The resident
// form, for windows whose q-tiles need at most four 32-key chunks (SWA(64,4)), loads all of a
// q-tile's keys into LDS at once, takes the exact maximum, and stores O block by block as it
// completes: no load follows any store, so the output drains under the compute (the chip
// counts loads and stores in one in-order counter, so in the tile walk the output of a round
// of workgroups is written after its compute and overlaps nothing).  Each comes with 128-row
// workgroups and, for grids too small to fill the chip, 64-row ones (twice the workgroups).
#include "swa_device.h"
#include "swa_launch.h"

#include <hip/hip_ext.h>
#include <math.h>

#include <algorithm>
#include <type_traits>

namespace swa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kTileN = 64;     // keys per KV tile
constexpr int kThreads = 256;  // 4 waves
// 16-column MFMA blocks per wave: a workgroup holds 64 NQB query rows.  Forms: 0 the tile walk
// and 1 resident, with two blocks per wave (128 rows); 2 resident and 3 the tile walk with one
// (64 rows: twice the workgroups, each with half the serial work, for grids too small to fill
// the chip).
constexpr int nqb_of_form(int form) { return form <= 1 ? 2 : 1; }
constexpr bool resident_form(int form) { return form == 1 || form == 2; }
constexpr int rows_per_block(int form) { return 64 * nqb_of_form(form); }
// Grids of 128-row workgroups that take the 64-row forms instead: the resident form below two
// workgroups per CU, the tile walk (whose workgroups each walk many tiles) at most one.
constexpr long long kSmallResidentGrid = 512;
constexpr long long kSmallWalkGrid = 256;

struct PrefillArgs {
    const uint16_t *q;
    const uint16_t *k;
    const uint16_t *v;
    float *out;
    float *lse;  // optional [B][Lq][Hq]: ln of each row's softmax denominator (null: not written)
    int L, Hq, Hkv, G, Gw, Tm, n_qtiles, n_hslices;
    int Lq, q_lo;  // queries are key positions q_lo .. q_lo + Lq - 1 (rows 0 .. Lq-1 of q, out)
    // Keys 0 .. n_cached-1 come from a sink+ring cache [B][Hkv][s + w_loc][d] instead of k, v
    // (chunked prefill): key j < ns is sink slot j; keys ns .. w0-1 are padding that no query
    // admits (read from slot 0); key j >= w0 is ring slot s + (ring0 + j - w0) mod w_loc, with
    // ring0 < w_loc and j - w0 < w_loc.  k and v then hold keys n_cached .. L-1.  n_cached = 0
    // for a whole-sequence prefill.
    const uint16_t *kc, *vc;
    int n_cached, ns, w0, ring0;
    int w_loc, s;
    float scale_log2;
    int nblocks;
};

template <int D>
struct Lds {
    static constexpr int kPieces = D / 8;                // 16-byte pieces per row
    static constexpr int kRowBytes = D * 2;              // rows are unpadded
    static constexpr int kTileBytes = kTileN * kRowBytes;
    static constexpr int kRowsPerLoad = 1024 / kRowBytes;  // rows one 64-lane 16-byte load fills
    static constexpr int kLoadsPerTile = kTileBytes / 1024;
};

// Maximum over the four lane groups (lanes l, l^16, l^32, l^48) that hold one query column,
// with the gfx950 cross-row swaps (VALU only, no LDS round trip).  permlane32_swap on (x, x)
// hands each lane the value of lane l^32 in one of its two results and its own in the other;
// permlane16_swap does the same for lane l^16.  (This file is built assuming no NaNs: fmaxf on
// the swapped bits would otherwise first quiet them as possible signalling NaNs, one more
// instruction per operand.)
__device__ __forceinline__ float max_over_groups(float x)
{
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
    const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

// max_over_groups of two values at once, x0 and x1 (two 16-column blocks): one swap puts the
// l / l^32 pairs of x0 in lanes 0-31 and those of x1 in lanes 32-63, so one maximum and one
// 16-lane swap finish both, and a last swap hands every lane both results.  Three swaps and two
// maxima instead of four and four.
__device__ __forceinline__ void max_over_groups2(float &x0, float &x1)
{
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x0), __float_as_uint(x1), false, false);
    float z = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
    const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(z), __float_as_uint(z), false, false);
    z = fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(z), __float_as_uint(z), false, false);
    x0 = __uint_as_float(r[0]);
    x1 = __uint_as_float(r[1]);
}

// Sum over the same four lane groups, as (x_l + x_l^16) + (x_l^32 + x_l^48), with the same swaps.
__device__ __forceinline__ float sum_over_groups(float x)
{
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// XOR swizzles of the 16-byte pieces of a row in LDS (physical piece = logical piece ^ swizzle).
// K: the 16 rows one S^T fragment read touches (32*kc + 8a + 4h + b, a, b = 0..3) get 16
// distinct swizzles, so the 16-byte reads of 16 consecutive lanes hit distinct bank groups.  V:
// the transposed 8-byte reads take rows r..r+3 (r = 0 mod 4) at pieces P, P+1 (P even); swizzles
// 0, 2, 4, 6 spread them over 8 distinct pieces.  (The counters charge every transposed read two
// bank-conflict cycles whatever the layout: a swizzle that also separates the row quads of lanes
// 0-15 and 16-31 left the count unchanged and ran 1-4% slower.)
template <int D>
__device__ __forceinline__ int swz_k(int r)
{
    return D == 128 ? ((((r >> 3) & 3) << 2) | (r & 3)) : ((((r >> 3) & 1) << 2) | (r & 3));
}
__device__ __forceinline__ int swz_v(int r) { return (r & 3) << 1; }

// acc + the sum of the eight bf16 values of p, in fp32 (four v_dot2 with a pair of ones).
__device__ __forceinline__ float sum8(const bf16x8 &p, float acc)
{
    const bf16x2 one = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bf16x2 y = {p[2 * i], p[2 * i + 1]};
        acc = __builtin_amdgcn_fdot2_f32_bf16(y, one, acc, false);
    }
    return acc;
}

// s_waitcnt immediate that waits for at most n outstanding vector-memory operations and
// nothing else (gfx9 encoding: vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
constexpr int waitcnt_vm(int n) { return 0x0f70 | (n & 15) | ((n >> 4) << 14); }


// Output stores in whole 128-byte lines.  Lane (g, c) holds column c of a 16-column block of
// O^T at d = 16 db + 4 g .. +3, so one plain store would write 64 bytes of each of 16 rows.  For
// a pair of d-blocks (2m, 2m+1), instruction A writes columns 0-7 and B columns 8-15, each lane
// 16 bytes at d = 32 m + 16 (c / 8) + 4 g, so 8 lanes fill one 128-byte line of a row: lanes
// c >= 8 take block 2m+1 of lane c-8 for A, lanes c < 8 block 2m of lane c+8 for B (DPP row
// shifts within each 16-lane row).  Whole lines can bypass L2 (non-temporal) without the
// partial-line traffic that made 64-byte non-temporal stores write 1.5x the output bytes.
// The stores are buffer stores over the q-tile's output rows: a row past the sequence (or a
// padding row) gets an offset past the buffer's size and the hardware drops its store, so the
// stores need no branch (a branch would end the compiler's scheduling region at every store).
constexpr uint32_t kDropOffset = 0x80000000u;  // any offset at or past the buffer size
__device__ __forceinline__ void store_pair(__amdgpu_buffer_rsrc_t rs, uint32_t offa, uint32_t offb, f32x4 lo, f32x4 hi)
{
    f32x4 av, bv;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // One row shift each (row_shr:8 for A, row_shl:8 for B) with bound_ctrl off: a lane whose
        // source lies outside its 16-lane row keeps `old`, its own value, so no select is needed.
        av[i] = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(lo[i]), __float_as_int(hi[i]), 0x118, 0xf, 0xf, false));
        bv[i] = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(hi[i]), __float_as_int(lo[i]), 0x108, 0xf, 0xf, false));
    }
    // (aux 2: the non-temporal policy)
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, av), rs, (int)offa, 0, 2);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, bv), rs, (int)offb, 0, 2);
}

// ln of a row's softmax denominator: the probabilities were taken as exp2(score * scale * log2(e)
// - m) with m in log2 units, so sum_i exp(scale * score_i) = 2^m * l.
__device__ __forceinline__ void store_lse(const PrefillArgs &a, int b, int t, int h, float m, float l)
{
    a.lse[((size_t)b * a.Lq + (t - a.q_lo)) * a.Hq + h] = (m + log2f(l)) * 0.6931471805599453f;
}

// Maps the hardware workgroup id to (b, kv-head, head slice, q-tile).
struct BlockCoord {
    int b, hkv, hs, qt;
};

__device__ __forceinline__ BlockCoord block_coord(const PrefillArgs &a)
{
    // Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a contiguous
    // range of logical ids so the q-tiles of one head share an L2.
    const int pb = blockIdx.x;
    const int nb8 = a.nblocks & ~7;
    const int logical = pb < nb8 ? (pb & 7) * (nb8 >> 3) + (pb >> 3) : pb;
    BlockCoord c;
    c.qt = a.n_qtiles - 1 - (logical % a.n_qtiles);  // heavy (late) tiles first
    int rest = logical / a.n_qtiles;
    c.hs = rest % a.n_hslices;
    rest /= a.n_hslices;
    c.hkv = rest % a.Hkv;
    c.b = rest / a.Hkv;
    return c;
}

// FORM: 0 tile walk, 1 resident (four chunk slots), 2 resident and 3 tile walk with 64-row
// workgroups.  CACHED: the key sequence begins with a.n_cached keys held in the sink+ring cache
// (chunked prefill); the whole-sequence instantiation has no cache code at all.
template <int D, int FORM, bool CACHED>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(PrefillArgs a)
{
    constexpr bool RES = resident_form(FORM);
    constexpr int NQB = nqb_of_form(FORM);  // 16-column blocks per wave
    constexpr int kPieces = Lds<D>::kPieces;
    constexpr int kKSteps = D / 32;    // MFMA k-steps for S
    constexpr int kDBlocks = D / 16;   // 16-row blocks of O^T
    constexpr int kRowBytes = Lds<D>::kRowBytes;
    constexpr int kTileBytes = Lds<D>::kTileBytes;
    constexpr int kRowsPerLoad = Lds<D>::kRowsPerLoad;
    constexpr int kHalfLoads = Lds<D>::kLoadsPerTile / 2 / (kThreads / 64);  // per wave and 32-row half
    static_assert(kHalfLoads >= 1, "tile load split");

    // Two buffers of (K tile, V tile), both row-major with swizzled 16-byte pieces, one variable
    // each: the reads then carry alias information that tells the compiler they do not depend on
    // the loads in flight (whose LDS destinations are opaque to it).
    __shared__ __attribute__((aligned(1024))) unsigned char lds_b0[2][kTileBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char lds_b1[2][kTileBytes];
    auto ldsbuf = [&](int buf) __attribute__((always_inline)) -> unsigned char(*)[kTileBytes] {
        return buf == 0 ? lds_b0 : lds_b1;  // (buf is a constant after inlining)
    };
    constexpr int kChunkBytes = kChunkN * kRowBytes;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g16 = lane >> 4;  // lane group 0..3
    const int c16 = lane & 15;  // column inside a 16-wide MFMA block

    const BlockCoord bc = block_coord(a);
    const int t0 = a.q_lo + bc.qt * a.Tm;
    const int t1 = min(t0 + a.Tm - 1, a.L - 1);
    const float c = a.scale_log2;

    // This lane's query column in each of its 16-column blocks (the wave owns rows
    // 16 NQB wave .. +16 NQB - 1).
    // Row r of the workgroup is head slot r / Tm, token t0 + r % Tm.  Tm >= 16, so a 16-column
    // block (first row `base`, uniform) crosses at most one head boundary: with base = gh0 Tm +
    // rem (scalar arithmetic; gh0 <= 3 as base < 4 Tm), column col is head slot
    // gh0 + (rem + col >= Tm).
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const int hbase = bc.hkv * a.G + bc.hs * a.Gw;  // first q-head of the workgroup
    auto row_of = [&](int qb, int col, int &gh, int &tk) __attribute__((always_inline)) {
        const int base = wave_s * 16 * NQB + qb * 16;
        const int gh0 = (base >= a.Tm) + (base >= 2 * a.Tm) + (base >= 3 * a.Tm);
        const int x = base - gh0 * a.Tm + col;
        const bool next = x >= a.Tm;
        gh = gh0 + (next ? 1 : 0);
        tk = t0 + (next ? x - a.Tm : x);
    };
    int tok[NQB], head[NQB];
    bool valid[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        int gh;
        row_of(qb, c16, gh, tok[qb]);
        head[qb] = hbase + gh;
        valid[qb] = gh < a.Gw && tok[qb] < a.L;
    }

    // Q^T B-operand fragments: d = kk*32 + 8*g16 .. +7 of the lane's query.
    bf16x8 qf[NQB][kKSteps];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        const uint16_t *qrow = a.q + (((size_t)bc.b * a.Lq + (valid[qb] ? tok[qb] - a.q_lo : 0)) * a.Hq +
                                      (valid[qb] ? head[qb] : 0)) * D;
#pragma unroll
        for (int kk = 0; kk < kKSteps; ++kk) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (valid[qb])
                x = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(qrow + kk * 32 + g16 * 8));
            qf[qb][kk] = as_bf16x8(x);
        }
    }


    // Output buffer: the rows of tokens t0 .. t1, every head (fewer than 2^31 bytes: checked on
    // the host).  row_off: byte offset of the row of column `col` of block qb (as tok/head above)
    // plus this lane's 16 bytes of a 128-byte line for store_pair, or kDropOffset for a row that
    // does not exist.
    const __amdgpu_buffer_rsrc_t out_rs = __builtin_amdgcn_make_buffer_rsrc(
        a.out + ((size_t)bc.b * a.Lq + (t0 - a.q_lo)) * a.Hq * D, 0, (t1 - t0 + 1) * a.Hq * D * 4, 0x00020000);
    auto row_off = [&](int qb, int col) __attribute__((always_inline)) {
        int gh, tk;
        row_of(qb, col, gh, tk);
        // (24-bit products: tk - t0 < 2^8 and Hq < 2^16, and the offset is below 2^31)
        const uint32_t off = ((uint32_t)__umul24(tk - t0, a.Hq) + hbase + gh) * (D * 4u) + (16 * (c16 >> 3) + 4 * g16) * 4u;
        return (gh < a.Gw && tk < a.L) ? off : kDropOffset;
    };
    const int kv_row = a.Hkv * D;  // elements between consecutive positions
    const int L_in = a.L - (CACHED ? a.n_cached : 0);  // key rows held by k and v
    const uint16_t *kbase = a.k + ((size_t)bc.b * L_in * a.Hkv + bc.hkv) * D;
    const uint16_t *vbase = a.v + ((size_t)bc.b * L_in * a.Hkv + bc.hkv) * D;
    const size_t cache_base = ((size_t)bc.b * a.Hkv + bc.hkv) * ((size_t)a.s + a.w_loc) * D;

    // Direct global -> LDS loads of 32-row halves of a tile: load j of a half fills its LDS bytes
    // [1024 j, 1024 j + 1024), lane l the 16 bytes at 16 l: row kRowsPerLoad*j + l / kPieces of
    // the half, physical piece l % kPieces, which holds logical piece (physical ^ swizzle).  A
    // row's swizzle depends on its index mod 32 only, so both halves take the same offsets.  This
    // wave issues loads j = wave*kHalfLoads .. +kHalfLoads-1 of each half.  Rows past the end of
    // the sequence read the last row (finite values; such keys are always masked).
    // The wave index as a uniform (scalar) value: the LDS destinations (M0) are then scalar.
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    uint32_t ld_koff[kHalfLoads], ld_voff[kHalfLoads];  // byte offsets from the half's first row
#pragma unroll
    for (int i = 0; i < kHalfLoads; ++i) {
        const int row = kRowsPerLoad * (wave * kHalfLoads + i) + lane / kPieces;
        const int phys = lane % kPieces;
        ld_koff[i] = (uint32_t)(row * kv_row + (phys ^ swz_k<D>(row)) * 8) * 2u;
        ld_voff[i] = (uint32_t)(row * kv_row + (phys ^ swz_v(row)) * 8) * 2u;
    }
    // Buffer resources over this (b, kv-head)'s rows of k and v (fewer than 2^32 bytes: one
    // sequence of q holds fewer than 2^31 elements and Hkv <= Hq): a half's byte offset is a
    // scalar operand and each lane adds its 32-bit offset, so a load costs no vector address
    // arithmetic.
    const uint32_t kv_bytes = (uint32_t)(((size_t)L_in * a.Hkv - bc.hkv) * D * 2);
    const __amdgpu_buffer_rsrc_t k_rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(kbase), 0, (int)kv_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t v_rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(vbase), 0, (int)kv_bytes, 0x00020000);
    // ... and over this (b, kv-head)'s sink and ring slots of the cache (chunked prefill).
    const uint32_t cache_bytes = (uint32_t)(((size_t)a.s + a.w_loc) * D * 2);
    const __amdgpu_buffer_rsrc_t kc_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(CACHED ? a.kc + cache_base : a.k), 0, (int)cache_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t vc_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(CACHED ? a.vc + cache_base : a.v), 0, (int)cache_bytes, 0x00020000);
    // Loads the K rows (kv = 0) or the V rows (kv = 1) of keys j0 .. j0+31 into half `half` of LDS
    // buffer buf.  Every load is a buffer load (a flat-encoded global load may, as far as the
    // compiler knows, also touch LDS, after which it waits for all outstanding memory operations
    // wherever it cannot prove otherwise) into an opaque LDS destination (SWA_LDS_DMA_DST): the
    // kernel orders loads and LDS reads itself, with counted waits and barriers.
    auto issue_half = [&](int j0, int buf, int half, auto kv_c) __attribute__((always_inline)) {
        constexpr int kv = decltype(kv_c)::value;
        const int last = a.L - 1;
        const int n_cached = CACHED ? a.n_cached : 0;
        if (j0 >= n_cached && j0 + kChunkN - 1 <= last) {
            // Every row is a key of k/v inside the sequence.
            const int half_off = __builtin_amdgcn_readfirstlane((int)((uint32_t)(j0 - n_cached) * (uint32_t)kv_row * 2u));
#pragma unroll
            for (int i = 0; i < kHalfLoads; ++i) {
                const int j = wave_u * kHalfLoads + i;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(kv ? v_rs : k_rs,
                                                         SWA_LDS_DMA_DST(&ldsbuf(buf)[kv][half * kChunkBytes + 1024 * j]),
                                                         16, (int)(kv ? ld_voff[i] : ld_koff[i]), half_off, 0, 0);
            }
            return;
        }
        if (CACHED && j0 >= a.w0 && j0 + kChunkN - 1 < n_cached) {
            // Every row is a cached window key.  When their ring slots run on without wrapping,
            // the rows are consecutive cache rows: the same lane offsets with the cache's row
            // stride (d elements instead of Hkv d), the first slot as the scalar offset.
            int r0 = a.ring0 + (j0 - a.w0);
            r0 = r0 >= a.w_loc ? r0 - a.w_loc : r0;
            if (r0 + kChunkN <= a.w_loc) {
                const int slot_off = __builtin_amdgcn_readfirstlane((a.s + r0) * D * 2);
#pragma unroll
                for (int i = 0; i < kHalfLoads; ++i) {
                    const int j = wave_u * kHalfLoads + i;
                    const uint32_t row = (uint32_t)(kRowsPerLoad * j + lane / kPieces);
                    const uint32_t off = (kv ? ld_voff[i] : ld_koff[i]) - row * (uint32_t)((kv_row - D) * 2);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        kv ? vc_rs : kc_rs, SWA_LDS_DMA_DST(&ldsbuf(buf)[kv][half * kChunkBytes + 1024 * j]),
                        16, (int)off, slot_off, 0, 0);
                }
                return;
            }
        }
        // Rows past the sequence's end (they read its last row: finite values, and such keys are
        // always masked) or holding cached keys (their sink or ring slots): per-lane offsets, a
        // cached key's lanes through the cache's resource (one more load instruction when the
        // half mixes the two, which only makes the counted waits stricter).
#pragma unroll
        for (int i = 0; i < kHalfLoads; ++i) {
            const int j = wave_u * kHalfLoads + i;
            const int row = kRowsPerLoad * j + lane / kPieces;
            const int piece = (lane % kPieces) ^ (kv ? swz_v(row) : swz_k<D>(row));
            const int key = min(j0 + row, last);
            // (made opaque outside the per-lane branch, where it is still a scalar)
            auto *const dst = SWA_LDS_DMA_DST(&ldsbuf(buf)[kv][half * kChunkBytes + 1024 * j]);
            if (!CACHED || key >= n_cached) {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(kv ? v_rs : k_rs, dst, 16,
                                                         (int)((uint32_t)((key - n_cached) * kv_row + piece * 8) * 2u),
                                                         0, 0, 0);
            } else {
                int slot = key;
                if (key >= a.w0) {
                    const int r = a.ring0 + key - a.w0;
                    slot = a.s + (r >= a.w_loc ? r - a.w_loc : r);
                } else if (key >= a.ns) {
                    slot = 0;  // padding between the sinks and the window: never admitted
                }
                __builtin_amdgcn_raw_ptr_buffer_load_lds(kv ? vc_rs : kc_rs, dst, 16,
                                                         (int)((uint32_t)(slot * D + piece * 8) * 2u), 0, 0, 0);
            }
        }
    };
    // A whole 64-key tile: both halves, with one test for each common case (a tile of k/v rows
    // inside the sequence, a tile of cached window keys in consecutive ring slots), so the middle
    // tiles' path takes one branch per tile.
    auto issue = [&](int j0, int buf, auto kv_c) __attribute__((always_inline)) {
        constexpr int kv = decltype(kv_c)::value;
        const int n_cached = CACHED ? a.n_cached : 0;
        if (j0 >= n_cached && j0 + kTileN - 1 <= a.L - 1) {
            const int tile_off = __builtin_amdgcn_readfirstlane((int)((uint32_t)(j0 - n_cached) * (uint32_t)kv_row * 2u));
#pragma unroll
            for (int half = 0; half < 2; ++half)
#pragma unroll
                for (int i = 0; i < kHalfLoads; ++i) {
                    const int j = wave_u * kHalfLoads + i;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        kv ? v_rs : k_rs, SWA_LDS_DMA_DST(&ldsbuf(buf)[kv][half * kChunkBytes + 1024 * j]), 16,
                        (int)(kv ? ld_voff[i] : ld_koff[i]), tile_off + half * kChunkN * kv_row * 2, 0, 0);
                }
            return;
        }
        if (CACHED && j0 >= a.w0 && j0 + kTileN - 1 < n_cached) {
            int r0 = a.ring0 + (j0 - a.w0);
            r0 = r0 >= a.w_loc ? r0 - a.w_loc : r0;
            if (r0 + kTileN <= a.w_loc) {
                const int slot_off = __builtin_amdgcn_readfirstlane((a.s + r0) * D * 2);
#pragma unroll
                for (int half = 0; half < 2; ++half)
#pragma unroll
                    for (int i = 0; i < kHalfLoads; ++i) {
                        const int j = wave_u * kHalfLoads + i;
                        const uint32_t row = (uint32_t)(kRowsPerLoad * j + lane / kPieces);
                        const uint32_t off = (kv ? ld_voff[i] : ld_koff[i]) - row * (uint32_t)((kv_row - D) * 2);
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(
                            kv ? vc_rs : kc_rs, SWA_LDS_DMA_DST(&ldsbuf(buf)[kv][half * kChunkBytes + 1024 * j]),
                            16, (int)off, slot_off + half * kChunkN * D * 2, 0, 0);
                    }
                return;
            }
        }
        issue_half(j0, buf, 0, kv_c);
        issue_half(j0 + kChunkN, buf, 1, kv_c);
    };
    // (tags as types, passed as temporaries: named tag objects captured by the lambdas below
    // end up in private memory)
    using KRows = std::integral_constant<int, 0>;
    using VRows = std::integral_constant<int, 1>;
    // LDS read offsets (bytes, within a tile) that do not depend on the tile.
    // K fragment (kc, h, kk): row 32kc + 4h + r with r = 8(c16/4) + c16%4, logical piece
    // 4kk + g16.  Adding 32kc + 4h to r changes neither r % 4 nor (r / 8) % 4, so the row's
    // swizzle is that of r: the offset is k_lane[kk] plus the constant (32kc + 4h) * kRowBytes.
    int k_lane[kKSteps];
#pragma unroll
    for (int kk = 0; kk < kKSteps; ++kk) {
        const int r = 8 * (c16 >> 2) + (c16 & 3);
        k_lane[kk] = r * kRowBytes + 16 * ((4 * kk + g16) ^ swz_k<D>(r));
    }
    // V^T fragment (db, kc) from two transposed 8-byte reads (h = 0, 1): lane 16g + s reads
    // row 32kc + 4h + 8g + s/4 at d = 16db + 4(s%4) .. +3 (byte 8(s%2) of logical piece
    // 2db + (s/2)%2); the read hands lane s the values at d = 16db + s of the four rows
    // 32kc + 4h + 8g .. +3.  The row's swizzle is 2(s/4) whatever kc, h, and XOR with an even
    // swizzle keeps the low piece bit, so the physical piece is 2(db ^ s/4) + (s/2)%2 and the
    // offset is v_lane[db % 4] plus the constant (32kc + 4h) * kRowBytes + 32 (db - db % 4).
    int v_lane[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
        v_lane[m] = (8 * g16 + (c16 >> 2)) * kRowBytes + 32 * (m ^ (c16 >> 2)) + 16 * ((c16 >> 1) & 1) + 8 * (c16 & 1);

    if constexpr (RES) {
        // Resident form (windows whose 32-token q-tile needs at most four 32-key chunks): every
        // chunk of the workgroup is loaded at once, slot k into half k & 1 of buffer k >> 1, then
        // one barrier, after which the workgroup issues no more loads.  Each 16-column block is then done over all of its
        // chunks and stored at once: the stores of one block drain while the next computes (a
        // later wait for a load would also wait for those stores, since loads and stores share
        // one in-order counter).
        constexpr int kSlots = 4;
        const ChunkWalk cw = plan_chunks(t0, t1, a.w_loc, a.s, kChunkN);
        // Every slot is always loaded (a slot past the workgroup's chunks holds keys after t1, and
        // rows past the sequence read its last row), so any slot holds finite keys and values.
#pragma unroll
        for (int k = 0; k < kSlots; ++k) {
            issue_half(resident_slot_key0(cw, k), k >> 1, k & 1, KRows());
            issue_half(resident_slot_key0(cw, k), k >> 1, k & 1, VRows());
        }
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        __syncthreads();
        // LDS rows of chunk slot k (K or V).
        auto slot_rows = [&](int k, int kv) __attribute__((always_inline)) -> const unsigned char * {
            return &ldsbuf(k >> 1)[kv][0] + (k & 1) * kChunkBytes;
        };
        // With every key of the q-tile at hand the softmax needs no running maximum: all scores,
        // the exact column maximum, the probabilities, then O^T = V^T P^T.  Slot k holds chunk
        // cw.chunk(k) (four chunks, straight-line code: a chunk past the q-tile's last needed one
        // holds keys after its last token, which the element mask removes by causality).
        // The usual q-tile (all but the first few): slot 0 holds chunk 0, which lies below the
        // window of every query of the q-tile, and the other slots hold chunks free of sinks.  Then
        // slot 0's mask is key < s for both passes, applied through the initial value of its score
        // accumulators (0 or -inf: K Q^T + (-inf) = -inf), and another slot's is the one unsigned
        // compare t - key < w_loc (exact for keys >= s: causal and window bound at once), three
        // vector instructions per score instead of five.  Other q-tiles test the whole predicate.
        const bool usual = cw.n_sink == 1 && a.s <= kChunkN && t0 - a.w_loc + 1 >= kChunkN;
        f32x4 sink_init[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                sink_init[h][j] = 8 * g16 + 4 * h + j < a.s ? 0.f : -INFINITY;
        auto pass = [&](auto qb_c, auto usual_c) __attribute__((always_inline)) {
            constexpr int qb = decltype(qb_c)::value;
            constexpr bool USUAL = decltype(usual_c)::value;
            const int t = tok[qb];
            f32x4 sr[4][2];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const unsigned char *kt = slot_rows(k, 0);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    sr[k][h] = USUAL && k == 0 ? sink_init[h] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < kKSteps; ++kk) {
                        const bf16x8 af = *reinterpret_cast<const bf16x8 *>(kt + k_lane[kk] + 4 * h * kRowBytes);
                        sr[k][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, qf[qb][kk], sr[k][h], 0, 0, 0);
                    }
                }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int key0 = cw.chunk(k) * kChunkN + 8 * g16;  // key of (h, j) = (0, 0)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    if (!USUAL) {
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const bool ok = key_allowed(t, key0 + 4 * h + j, a.w_loc, a.s);
                            sr[k][h][j] = ok ? sr[k][h][j] : -INFINITY;
                        }
                    } else if (k > 0) {
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const bool ok = (uint32_t)(t - key0 - (4 * h + j)) < (uint32_t)a.w_loc;
                            sr[k][h][j] = ok ? sr[k][h][j] : -INFINITY;
                        }
                    }
                    mx = fmaxf(fmaxf(mx, sr[k][h][0]), sr[k][h][1]);
                    mx = fmaxf(fmaxf(mx, sr[k][h][2]), sr[k][h][3]);
                }
            }
            const float mm = max_over_groups(mx) * c;
            const float m_use = mm == -INFINITY ? 0.f : mm;
            // Probabilities, their column sums, then O^T one 16-row block at a time, each stored as
            // soon as it is complete, so the stores spread over the compute.
            bf16x8 pf[4];
            float l = 0.f;  // this lane's keys; the lane groups are added below
#pragma unroll
            for (int k = 0; k < 4; ++k) {
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        pf[k][4 * h + j] = static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(sr[k][h][j], c, -m_use)));
                l = sum8(pf[k], l);
            }
            l = sum_over_groups(l);
            const float inv = __builtin_amdgcn_rcpf(l);  // (1 ulp; the exact quotient takes ten instructions)
            if (a.lse != nullptr && g16 == 0 && valid[qb])
                store_lse(a, bc.b, tok[qb], head[qb], m_use, l);
            const uint32_t oa = row_off(qb, c16 & 7), ob = row_off(qb, (c16 & 7) + 8);
            f32x4 od_lo = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int db = 0; db < kDBlocks; ++db) {
                f32x4 od = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const unsigned char *vt = slot_rows(k, 1);
                    bf16x8 af;
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int off = v_lane[db & 3] + 4 * h * kRowBytes + 32 * (db & ~3);
                        const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) s16x4 *)(vt + off));
                        const bf16x4 y = __builtin_bit_cast(bf16x4, x);
                        af[4 * h + 0] = y[0];
                        af[4 * h + 1] = y[1];
                        af[4 * h + 2] = y[2];
                        af[4 * h + 3] = y[3];
                    }
                    od = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, pf[k], od, 0, 0, 0);
                }
                if (db & 1)
                    store_pair(out_rs, oa + 64 * (db - 1), ob + 64 * (db - 1), od_lo * inv, od * inv);
                else
                    od_lo = od;
            }
        };
        if (usual) {
            pass(std::integral_constant<int, 0>(), std::true_type());
            if constexpr (NQB > 1)
                pass(std::integral_constant<int, NQB - 1>(), std::true_type());
        } else {
            pass(std::integral_constant<int, 0>(), std::false_type());
            if constexpr (NQB > 1)
                pass(std::integral_constant<int, NQB - 1>(), std::false_type());
        }
    } else {
        const TileWalk tw = plan_tiles(t0, t1, a.w_loc, a.s, kTileN);
        const WalkSplit sp = split_walk(tw, t0, t1, a.w_loc, kTileN);
        auto tile_info = [&](int tile) __attribute__((always_inline)) {
            return swa::tile_info(tile, kTileN, t0, t1, a.w_loc, a.s);
        };

        f32x4 o[kDBlocks][NQB];
#pragma unroll
        for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb)
                o[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
        // Softmax state per query column, in log2 units: the reference maximum m_ref the
        // probabilities are taken against.  The running sum of the probabilities adds the same
        // bf16-rounded values that weight V (v_dot2 with a pair of ones, fp32 accumulation): each
        // lane sums the keys it holds and the four lane groups of a column are added at the end,
        // so the dominant weight's rounding cancels between numerator and denominator.
        // thr is m_ref + 8 in score units: a column maximum above it moves m_ref (below).
        float m_ref[NQB], thr[NQB], lsum[NQB], cmx[NQB];
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
            m_ref[qb] = -INFINITY;
            thr[qb] = -INFINITY;
            lsum[qb] = 0.f;
        }
        const float inv_c = 1.f / c;

        // S^T = K Q^T of one chunk, K rows from LDS at kt.  Row m of 16-key block h holds key
        // 8*(m/4) + 4*h + m%4 of the chunk, so lane group g later owns keys 8g .. 8g+7.
        auto scores = [&](f32x4(&sc)[2][NQB], const unsigned char *kt) __attribute__((always_inline)) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb)
                    sc[h][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < kKSteps; ++kk) {
                    const bf16x8 af = *reinterpret_cast<const bf16x8 *>(kt + k_lane[kk] + 4 * h * kRowBytes);
#pragma unroll
                    for (int qb = 0; qb < NQB; ++qb)
                        sc[h][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, qf[qb][kk], sc[h][qb], 0, 0, 0);
                }
            }
        };

        // Element mask of one chunk whose first key is key0 (when some pair in it is outside A(t)).
        auto mask_chunk = [&](f32x4(&sc)[2][NQB], int key0) __attribute__((always_inline)) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const bool ok = key_allowed(tok[qb], key0 + 8 * g16 + 4 * h + j, a.w_loc, a.s);
                        sc[h][qb][j] = ok ? sc[h][qb][j] : -INFINITY;
                    }
        };
        // Column maxima of NC chunks (into cmx) and whether any column of this lane passed its
        // threshold: the reference maximum only moves (move_ref, O and the sums rescaled) when the
        // column maximum exceeds it by more than 8 in log2 units, so the probabilities stay below
        // 256 and most steps take one compare per column.
        auto col_max = [&](const f32x4(*sc)[2][NQB], auto nc_c) __attribute__((always_inline)) {
            constexpr int NC = decltype(nc_c)::value;
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) {
                // (pairs folded into the running maximum: three-input maxima)
                float mx = -INFINITY;
#pragma unroll
                for (int kc = 0; kc < NC; ++kc)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        mx = fmaxf(fmaxf(mx, sc[kc][h][qb][0]), sc[kc][h][qb][1]);
                        mx = fmaxf(fmaxf(mx, sc[kc][h][qb][2]), sc[kc][h][qb][3]);
                    }
                cmx[qb] = mx;
            }
#pragma unroll
            for (int qb = 0; qb + 1 < NQB; qb += 2)
                max_over_groups2(cmx[qb], cmx[qb + 1]);
            if (NQB % 2 != 0)
                cmx[NQB - 1] = max_over_groups(cmx[NQB - 1]);
            bool grow_any = false;
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb)
                grow_any |= cmx[qb] > thr[qb];
            return grow_any;
        };

        // The move: each column above its threshold takes its maximum as the new m_ref, and O and
        // the sums are rescaled by alpha = 2^(old - new).  (A column with no allowed key so far
        // keeps m_ref = -inf and alpha = 1.)
        auto move_ref = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) {
                const bool grow = cmx[qb] > thr[qb];
                const float m_new = cmx[qb] * c;
                const float alpha = grow ? __builtin_amdgcn_exp2f(m_ref[qb] - m_new) : 1.f;
                m_ref[qb] = grow ? m_new : m_ref[qb];
                thr[qb] = grow ? (m_new + 8.f) * inv_c : thr[qb];
#pragma unroll
                for (int db = 0; db < kDBlocks; ++db)
                    o[db][qb] *= alpha;
                lsum[qb] *= alpha;
            }
        };

        // Probabilities of one chunk against the reference maximum, as P^T B-operand fragments.
        // `finite`: every column already has a finite m_ref (the middle tiles, which follow a
        // tile whose keys every query sees).
        auto probs = [&](const f32x4(&sc)[2][NQB], bf16x8(&pf)[NQB], auto finite_c) __attribute__((always_inline)) {
            constexpr bool finite = decltype(finite_c)::value;
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) {
                const float m_use = finite ? m_ref[qb] : (m_ref[qb] == -INFINITY ? 0.f : m_ref[qb]);
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        pf[qb][4 * h + j] = static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(sc[h][qb][j], c, -m_use)));
            }
        };

        // O^T += V^T P^T of one chunk, V rows from LDS at vt, and the probability sums.
        auto accumulate = [&](const bf16x8(&pf)[NQB], const unsigned char *vt) __attribute__((always_inline)) {
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb)
                lsum[qb] = sum8(pf[qb], lsum[qb]);
#pragma unroll
            for (int db = 0; db < kDBlocks; ++db) {
                bf16x8 af;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int off = v_lane[db & 3] + 4 * h * kRowBytes + 32 * (db & ~3);
                    const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) s16x4 *)(vt + off));
                    const bf16x4 y = __builtin_bit_cast(bf16x4, x);
                    af[4 * h + 0] = y[0];
                    af[4 * h + 1] = y[1];
                    af[4 * h + 2] = y[2];
                    af[4 * h + 3] = y[3];
                }
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb)
                    o[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, pf[qb], o[db][qb], 0, 0, 0);
            }
        };

        // The online softmax takes the chunks in any order: the edge tiles first, one per step,
        // then the middle tiles through a software pipeline.
        f32x4 sc[2][2][2][NQB];  // scores of two tiles: [parity][chunk][h][qb]
        using Even = std::integral_constant<int, 0>;
        using Odd = std::integral_constant<int, 1>;
        using One = std::integral_constant<int, 1>;
        using Two = std::integral_constant<int, 2>;

        // Edge tiles: step i computes tile i's needed chunks while K and V of tile i+1 load into
        // the other buffer.  The scores of both chunks come first, so the second chunk's matrix
        // work runs beside the first chunk's softmax.
        if (sp.n_edge > 0) {
            TileInfo cur = tile_info(sp.edge_tile(tw, 0));
            issue(cur.j0, 0, KRows());
            issue(cur.j0, 0, VRows());
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
            __syncthreads();
            auto edge_step = [&](const int i, auto buf_c) __attribute__((always_inline)) {
                constexpr int buf = decltype(buf_c)::value;  // i & 1
                TileInfo nxt = cur;
                if (i + 1 < sp.n_edge) {
                    nxt = tile_info(sp.edge_tile(tw, i + 1));
                    issue(nxt.j0, buf ^ 1, KRows());
                    issue(nxt.j0, buf ^ 1, VRows());
                }
                // Each needed chunk takes its own maximum, so the first chunk's products with V
                // run beside the second chunk's softmax.
                f32x4(&es)[2][2][NQB] = sc[0];
                const bool need0 = cur.c_lo == 0, need1 = cur.c_hi == 1;
                if (need0)
                    scores(es[0], ldsbuf(buf)[0]);
                if (need1)
                    scores(es[1], ldsbuf(buf)[0] + kChunkBytes);
                bf16x8 pf[NQB];
#pragma unroll
                for (int kc = 0; kc < 2; ++kc) {
                    if (!(kc == 0 ? need0 : need1))
                        continue;
                    if (!cur.mask_free)
                        mask_chunk(es[kc], cur.j0 + kc * kChunkN);
                    if (__any(col_max(&es[kc], One())))
                        move_ref();
                    probs(es[kc], pf, std::false_type());
                    accumulate(pf, ldsbuf(buf)[1] + kc * kChunkBytes);
                }
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the next tile has landed
                __syncthreads();
                cur = nxt;
            };
            for (int i = 0; i < sp.n_edge; i += 2) {
                edge_step(i, Even());
                if (i + 1 < sp.n_edge)
                    edge_step(i + 1, Odd());
            }
        }

        // Middle tiles m = 0 .. nm-1 (keys jm + 64m ..): full and mask-free.  Step m computes, with
        // no dependence between the two halves,
        //     matrix cores: S of tile m+1, then O += V^T P^T of tile m
        //     vector ALUs:  probabilities of tile m, then the maxima of tile m+1
        // so the exponentials of one tile run while the matrix cores work on the next.  K runs one
        // tile ahead of V: step m reads K of tile m+1 and V of tile m (LDS buffers (m+1)&1 and m&1)
        // while K of tile m+2 and V of tile m+1 load into the other two; one barrier per step.  The
        // rescale for tile m+1 (rare) closes step m, after O has taken tile m.  (A pipeline over
        // 32-key chunks, one barrier per tile, measured 6% slower at w = 4096.)
        const int nm = sp.n_mid();
        if (nm > 0) {
            const int jm = sp.mid_lo * kTileN;
            auto tile_scores = [&](f32x4(&st)[2][2][NQB], const unsigned char *kt) __attribute__((always_inline)) {
                scores(st[0], kt);
                scores(st[1], kt + kChunkBytes);
            };
            auto tile_pv = [&](const f32x4(&st)[2][2][NQB], const unsigned char *vt) __attribute__((always_inline)) {
                bf16x8 pf[2][NQB];
                probs(st[0], pf[0], std::true_type());
                probs(st[1], pf[1], std::true_type());
                accumulate(pf[0], vt);
                accumulate(pf[1], vt + kChunkBytes);
            };
            issue(jm, 0, KRows());
            issue(jm, 0, VRows());
            if (nm > 1)
                issue(jm + kTileN, 1, KRows());
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
            __syncthreads();
            tile_scores(sc[0], ldsbuf(0)[0]);
            if (__any(col_max(sc[0], Two())))
                move_ref();

            auto mid_step = [&](const int m, auto buf_c) __attribute__((always_inline)) {  // m + 1 < nm
                constexpr int buf = decltype(buf_c)::value;  // m & 1
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // this wave's loads of the last step landed
                __syncthreads();                            // ... and every wave's; K buffer buf, V buffer buf^1 free
                if (m + 2 < nm)
                    issue(jm + (m + 2) * kTileN, buf, KRows());
                issue(jm + (m + 1) * kTileN, buf ^ 1, VRows());
                tile_scores(sc[buf ^ 1], ldsbuf(buf ^ 1)[0]);
                tile_pv(sc[buf], ldsbuf(buf)[1]);
                if (__any(col_max(sc[buf ^ 1], Two())))
                    move_ref();
            };
            // The last middle tile: its probabilities and O += V^T P^T.
            auto mid_last = [&](auto buf_c) __attribute__((always_inline)) {
                constexpr int buf = decltype(buf_c)::value;
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
                __syncthreads();
                tile_pv(sc[buf], ldsbuf(buf)[1]);
            };
            int m = 0;
            for (; m + 2 < nm; m += 2) {
                mid_step(m, Even());
                mid_step(m + 1, Odd());
            }
            if (m + 1 < nm) {
                mid_step(m, Even());
                mid_last(Odd());
            } else {
                mid_last(Even());
            }
        }

        // Epilogue: finish the row sums across the four lane groups, normalise, store fp32.
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
            const float l = sum_over_groups(lsum[qb]);  // this lane's keys, then the column's
            const float inv = 1.f / l;
            if (a.lse != nullptr && g16 == 0 && valid[qb])
                store_lse(a, bc.b, tok[qb], head[qb], m_ref[qb] == -INFINITY ? 0.f : m_ref[qb], l);
            const uint32_t oa = row_off(qb, c16 & 7), ob = row_off(qb, (c16 & 7) + 8);
#pragma unroll
            for (int m = 0; m < kDBlocks / 2; ++m)
                store_pair(out_rs, oa + 128 * m, ob + 128 * m, o[2 * m][qb] * inv, o[2 * m + 1][qb] * inv);
        }
    }
}

// Debug: how often the prefill kernel of form `form` (q-tiles of Tm tokens as launched) attends
// each (query, key) pair: mask[t][key] counts the visits in which the kernel's walk and element
// mask admit the pair, recorded at the key the visited LDS row actually holds.  The walks are the
// kernel's own device functions: for the main form the edge tiles (chunk selection, mask-free
// classification, element predicate) and the middle tiles (whole, unmasked); for the resident
// form the chunk walk with the keys its slots hold.  A correct kernel gives exactly 1 on A(t) and
// 0 elsewhere.  One workgroup per q-tile, one thread per query (no two threads write one row).
__global__ void debug_prefill_mask_kernel(uint8_t *mask, int L, int Tm, int form, int w_loc, int s)
{
    const int t0 = blockIdx.x * Tm;
    const int t1 = min(t0 + Tm - 1, L - 1);
    const int t = t0 + (int)threadIdx.x;
    if (t > t1)
        return;
    uint8_t *row = mask + (size_t)t * L;
    auto visit = [&](int key, bool admitted) {  // a key as the kernel computes it; LDS holds min(key, L-1)
        if (admitted)
            ++row[min(key, L - 1)];
    };
    if (resident_form(form)) {
        const ChunkWalk cw = plan_chunks(t0, t1, w_loc, s, kChunkN);
        for (int k = 0; k < 4; ++k)
            for (int r = 0; r < kChunkN; ++r) {
                const int key = cw.chunk(k) * kChunkN + r;        // the key the element mask tests
                const int held = resident_slot_key0(cw, k) + r;  // the key slot k holds
                if (key_allowed(t, key, w_loc, s))
                    ++row[min(held, L - 1)];
            }
        return;
    }
    const TileWalk tw = plan_tiles(t0, t1, w_loc, s, kTileN);
    const WalkSplit sp = split_walk(tw, t0, t1, w_loc, kTileN);
    for (int i = 0; i < sp.n_edge; ++i) {
        const TileInfo ti = tile_info(sp.edge_tile(tw, i), kTileN, t0, t1, w_loc, s);
        for (int c = ti.c_lo; c <= ti.c_hi; ++c)
            for (int r = 0; r < kChunkN; ++r) {
                const int key = ti.j0 + c * kChunkN + r;
                visit(key, ti.mask_free || key_allowed(t, key, w_loc, s));
            }
    }
    for (int tile = sp.mid_lo; tile < sp.mid_lo + sp.n_mid(); ++tile)
        for (int r = 0; r < kTileN; ++r)
            visit(tile * kTileN + r, true);
}

__global__ void fill_zero_kernel(uint8_t *p, size_t n)
{
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

}  // namespace

bool prefill_resident(int Tm, int q_lo, int w_loc, int s)
{
    // With q-tiles starting on 32-key boundaries a q-tile needs at most Tm/32 + ceil((w_loc-1)/32)
    // window chunks; 16-token q-tiles on 16-key boundaries at most 1 + ceil((w_loc-1)/32) (a tile
    // starting mid-chunk reaches no further); and ceil(s/32) sink chunks.
    long long win;
    if (Tm % kChunkN == 0 && q_lo % kChunkN == 0)
        win = Tm / kChunkN;
    else if (Tm == kChunkN / 2 && q_lo % (kChunkN / 2) == 0)
        win = 1;
    else
        return false;
    const long long n = win + ((long long)w_loc - 1 + kChunkN - 1) / kChunkN + ((long long)s + kChunkN - 1) / kChunkN;
    return n <= 4;
}

PrefillGeometry prefill_geometry(int L, int Hq, int Hkv, int form)
{
    PrefillGeometry g;
    g.G = Hq / Hkv;
    g.Gw = 1;
    for (int c = 4; c >= 1; --c)
        if (g.G % c == 0) {
            g.Gw = c;
            break;
        }
    g.rows = rows_per_block(form);
    g.Tm = g.rows / g.Gw;
    g.n_hslices = g.G / g.Gw;
    g.n_qtiles = (L + g.Tm - 1) / g.Tm;
    return g;
}

int prefill_form(int B, int Hq, int Hkv, int Lq, int q_lo, int w_loc, int s)
{
    const PrefillGeometry g1 = prefill_geometry(Lq, Hq, Hkv, 1), g2 = prefill_geometry(Lq, Hq, Hkv, 2);
    const bool r1 = prefill_resident(g1.Tm, q_lo, w_loc, s), r2 = prefill_resident(g2.Tm, q_lo, w_loc, s);
    // The 64-row forms where the 128-row ones would leave the chip short of workgroups (both
    // 128-row forms have the same grid).
    const long long wg1 = (long long)B * Hkv * g1.n_hslices * g1.n_qtiles;
    if (r2 && (!r1 || wg1 < kSmallResidentGrid))
        return 2;
    if (r1)
        return 1;
    return wg1 <= kSmallWalkGrid ? 3 : 0;
}

PrefillPlan prefill_plan(int B, int Hq, int Hkv, int L, int w_loc, int s)
{
    PrefillPlan p;
    p.form = prefill_form(B, Hq, Hkv, L, 0, w_loc, s);
    p.g = prefill_geometry(L, Hq, Hkv, p.form);
    const long long per_tile_group = (long long)B * Hkv * p.g.n_hslices;  // workgroups per q-tile
    p.workgroups = per_tile_group * p.g.n_qtiles;
    long long keys = 0;  // summed over the q-tiles: keys whose products one row of the tile computes
    for (int qt = 0; qt < p.g.n_qtiles; ++qt) {
        const int t0 = qt * p.g.Tm, t1 = std::min(t0 + p.g.Tm - 1, L - 1);
        if (resident_form(p.form)) {
            keys += 4 * kChunkN;  // four chunk slots per pass
        } else {
            const TileWalk tw = plan_tiles(t0, t1, w_loc, s, kTileN);
            const WalkSplit sp = split_walk(tw, t0, t1, w_loc, kTileN);
            for (int i = 0; i < sp.n_edge; ++i) {
                const TileInfo ti = tile_info(sp.edge_tile(tw, i), kTileN, t0, t1, w_loc, s);
                keys += (long long)(ti.c_hi - ti.c_lo + 1) * kChunkN;
            }
            keys += (long long)sp.n_mid() * kTileN;
        }
    }
    p.executed_pairs = per_tile_group * keys * p.g.rows;
    return p;
}

hipError_t launch_prefill(const void *q, const void *k, const void *v, float *out, int B, int Hq,
                          int Hkv, int L, int d, int w_loc, int s, float scale, hipStream_t stream,
                          hipEvent_t start, hipEvent_t stop, const PrefillKeySource *cached, float *lse)
{
    int Lq = L, q_lo = 0, gap = 0;
    if (cached != nullptr) {
        Lq = L - cached->n_cached;
        q_lo = cached->n_cached;
    }
    // A chunk after the cache has filled (all s sinks and w_loc - 1 window keys cached) whose
    // queries start off a 32-key boundary: padding rows between the sinks and the window move
    // them onto one, so the resident form can take the chunk (all of a q-tile's keys in one
    // load instead of a chain of dependent tile steps), and the tile walk's q-tiles start on a
    // chunk boundary (each diagonal in one chunk, not two).  No query admits a padding row: the
    // first query's window starts right after the padding, and the padding lies past the sinks.
    if (cached != nullptr && cached->ns == s && cached->n_cached - cached->ns == w_loc - 1 &&
        q_lo % kChunkN != 0)
        gap = kChunkN - q_lo % kChunkN;
    L += gap;
    q_lo += gap;
    const int form = prefill_form(B, Hq, Hkv, Lq, q_lo, w_loc, s);
    const PrefillGeometry g = prefill_geometry(Lq, Hq, Hkv, form);
    PrefillArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.out = out;
    a.lse = lse;
    a.L = L;
    a.Lq = Lq;
    a.q_lo = q_lo;
    a.kc = cached ? static_cast<const uint16_t *>(cached->k_cache) : nullptr;
    a.vc = cached ? static_cast<const uint16_t *>(cached->v_cache) : nullptr;
    a.n_cached = cached ? cached->n_cached + gap : 0;
    a.ns = cached ? cached->ns : 0;
    a.w0 = cached ? cached->ns + gap : 0;
    a.ring0 = cached ? cached->ring0 : 0;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = g.G;
    a.Gw = g.Gw;
    a.Tm = g.Tm;
    a.n_qtiles = g.n_qtiles;
    a.n_hslices = g.n_hslices;
    a.w_loc = w_loc;
    a.s = s;
    a.scale_log2 = scale * 1.4426950408889634f;
    const long long nb = (long long)B * Hkv * g.n_hslices * g.n_qtiles;
    if (nb > 0x7fffffffLL)
        return hipErrorInvalidConfiguration;
    a.nblocks = (int)nb;
    void (*const kernels[2][2][4])(PrefillArgs) = {
        {{prefill_kernel<64, 0, false>, prefill_kernel<64, 1, false>, prefill_kernel<64, 2, false>,
          prefill_kernel<64, 3, false>},
         {prefill_kernel<128, 0, false>, prefill_kernel<128, 1, false>, prefill_kernel<128, 2, false>,
          prefill_kernel<128, 3, false>}},
        {{prefill_kernel<64, 0, true>, prefill_kernel<64, 1, true>, prefill_kernel<64, 2, true>,
          prefill_kernel<64, 3, true>},
         {prefill_kernel<128, 0, true>, prefill_kernel<128, 1, true>, prefill_kernel<128, 2, true>,
          prefill_kernel<128, 3, true>}}};
    void (*kern)(PrefillArgs) = kernels[a.n_cached > 0 ? 1 : 0][d == 128 ? 1 : 0][form];
    if (start != nullptr || stop != nullptr)
        hipExtLaunchKernelGGL(kern, dim3(a.nblocks), dim3(kThreads), 0, stream, start, stop, 0, a);
    else
        hipLaunchKernelGGL(kern, dim3(a.nblocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_debug_prefill_mask(uint8_t *mask, int L, int Hq, int Hkv, int d, int w_loc, int s,
                                     hipStream_t stream)
{
    (void)d;  // one tile geometry serves both head sizes
    // The geometry and form launch_prefill chooses for a whole-sequence prefill.
    const PrefillPlan plan = prefill_plan(1, Hq, Hkv, L, w_loc, s);
    const PrefillGeometry &g = plan.g;
    const int form = plan.form;
    const size_t n = (size_t)L * L;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(256), dim3(256), 0, stream, mask, n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(debug_prefill_mask_kernel, dim3(g.n_qtiles), dim3(g.Tm), 0, stream, mask, L, g.Tm,
                       form, w_loc, s);
    return hipGetLastError();
}

}  // namespace swa
