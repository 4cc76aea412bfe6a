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
// kv-head.  Wave w owns rows 32w .. 32w+31 as two 16-column MFMA blocks.
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
// 16-byte pieces of each row XOR-swizzled so that the K fragment reads and the transposed
// V reads (ds_read_b64_tr_b16) are free of bank conflicts.  Q stays in registers for the
// whole key loop.  Workgroups are ordered heavy-first (last q-tile first) and mapped so
// that consecutive logical workgroups share an XCD and its L2, where neighbouring q-tiles
// re-read the same K/V tiles.  The fp32 output goes out in whole 128-byte lines with
// non-temporal stores (store_pair).
//
// Three forms.  The main form walks the tiles with a running softmax: edge tiles one per step,
// then the middle tiles through a software pipeline.  The resident form, for windows whose
// 32-token q-tiles need at most four 32-key chunks (SWA(64,4)), loads all of a q-tile's keys
// into LDS at once, takes the exact maximum, and stores O block by block as it completes: no
// load follows any store, so the output drains under the compute (the chip counts loads and
// stores in one in-order counter, so in the main form the output of a round of workgroups is
// written after its compute and overlaps nothing).  The wide resident form does the same for
// 64-token q-tiles when four q-heads share a kv-head: five chunk slots (80 KiB, two
// workgroups per CU) serve both 32-token halves, and each wave takes its head's two halves in
// turn, so the keys shared by the halves are loaded once and half as many workgroups run.
#include "swa_device.h"
#include "swa_launch.h"

#include <hip/hip_ext.h>
#include <math.h>

#include <type_traits>

namespace swa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kTileN = 64;     // keys per KV tile
constexpr int kThreads = 256;  // 4 waves
constexpr int kRowsPerBlock = 128;

struct PrefillArgs {
    const uint16_t *q;
    const uint16_t *k;
    const uint16_t *v;
    float *out;
    int L, Hq, Hkv, G, Gw, Tm, n_qtiles, n_hslices;
    int Lq, q_lo;  // queries are key positions q_lo .. q_lo + Lq - 1 (rows 0 .. Lq-1 of q, out)
    // Keys 0 .. n_cached-1 come from a sink+ring cache [B][Hkv][s + w_loc][d] instead of k, v
    // (chunked prefill): key j < ns is sink slot j; key j >= ns is ring slot
    // s + (ring0 + j - ns) mod w_loc, with ring0 < w_loc and j - ns < w_loc.  k and v then hold
    // keys n_cached .. L-1.  n_cached = 0 for a whole-sequence prefill.
    const uint16_t *kc, *vc;
    int n_cached, ns, ring0;
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

// XOR swizzles of the 16-byte pieces of a row (physical piece = logical piece ^ swizzle).
// K: the 16 rows one S^T fragment read touches (32*kc + 8a + 4h + b, a, b = 0..3) get 16
// distinct swizzles, so the 16-byte reads of any 8 or 16 consecutive lanes hit distinct
// bank groups.  V: the transposed 8-byte reads take rows r..r+3 (r = 0 mod 4) at pieces
// P, P+1 (P even); swizzles 0, 2, 4, 6 spread them over 8 distinct pieces.
template <int D>
__device__ __forceinline__ int swz_k(int r)
{
    return D == 128 ? ((((r >> 3) & 3) << 2) | (r & 3)) : ((((r >> 3) & 1) << 2) | (r & 3));
}
__device__ __forceinline__ int swz_v(int r) { return (r & 3) << 1; }

// Maximum over the four lane groups (lanes l, l^16, l^32, l^48) that hold one query column,
// with the gfx950 cross-row swaps (VALU only, no LDS round trip).  permlane32_swap on (x, x)
// hands each lane the value of lane l^32 in one of its two results and its own in the other;
// permlane16_swap does the same for lane l^16.
__device__ __forceinline__ float max_over_groups(float x)
{
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
    const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// s_waitcnt immediate that waits for at most n outstanding vector-memory operations and
// nothing else (gfx9 encoding: vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
constexpr int waitcnt_vm(int n) { return 0x0f70 | (n & 15) | ((n >> 4) << 14); }

// LDS pointer in the local address space, as the direct global -> LDS load takes it.  The
// cast is written inline: an implicit conversion (or a helper function) there makes the host
// pass drop the kernel's launch stub.
#define SWA_LDS_PTR(p) ((__attribute__((address_space(3))) void *)(p))

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

// Key tile of the walk: first key, needed chunk range, and whether no element mask is needed.
struct TileInfo {
    int j0, c_lo, c_hi;
    int mask_free;  // (an int: a bool member would leave padding that the copies carry)
    __device__ __forceinline__ bool full() const { return c_lo == 0 && c_hi == 1 && mask_free; }
};

// FORM: 0 main (tile walk), 1 resident (32-token q-tiles, four chunk slots), 2 wide resident
// (64-token q-tiles taken as two 32-token halves per wave, five chunk slots).
template <int D, int FORM>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(PrefillArgs a)
{
    constexpr bool RES = FORM != 0;
    constexpr bool WIDE = FORM == 2;
    constexpr int NQB = WIDE ? 4 : 2;  // 16-column blocks per wave
    constexpr int kPieces = Lds<D>::kPieces;
    constexpr int kKSteps = D / 32;    // MFMA k-steps for S
    constexpr int kDBlocks = D / 16;   // 16-row blocks of O^T
    constexpr int kRowBytes = Lds<D>::kRowBytes;
    constexpr int kTileBytes = Lds<D>::kTileBytes;
    constexpr int kRowsPerLoad = Lds<D>::kRowsPerLoad;
    constexpr int kLoadsPerWave = Lds<D>::kLoadsPerTile / (kThreads / 64);
    static_assert(kLoadsPerWave >= 1, "tile load split");

    // Two buffers of (K tile, V tile), both row-major with swizzled 16-byte pieces.
    __shared__ __attribute__((aligned(1024))) unsigned char lds[2][2][kTileBytes];
    // The wide form's fifth chunk slot (K, V); a token array in the other forms.
    constexpr int kChunkBytes = kChunkN * kRowBytes;
    __shared__ __attribute__((aligned(1024))) unsigned char lds5[2][WIDE ? kChunkBytes : 16];

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
    int tok[NQB], head[NQB];
    bool valid[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        const int r = wave * 16 * NQB + qb * 16 + c16;
        const int gh = r / a.Tm;
        tok[qb] = t0 + r % a.Tm;
        head[qb] = bc.hkv * a.G + bc.hs * a.Gw + gh;
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
        const int r = wave * 16 * NQB + qb * 16 + col;
        const int gh = r / a.Tm;
        const int tk = t0 + r % a.Tm;
        const int hd = bc.hkv * a.G + bc.hs * a.Gw + gh;
        const uint32_t off = (uint32_t)(((tk - t0) * a.Hq + hd) * D + 16 * (c16 >> 3) + 4 * g16) * 4u;
        return (gh < a.Gw && tk < a.L) ? off : kDropOffset;
    };
    const int kv_row = a.Hkv * D;  // elements between consecutive positions
    const int L_in = a.L - a.n_cached;  // key rows held by k and v
    const uint16_t *kbase = a.k + ((size_t)bc.b * L_in * a.Hkv + bc.hkv) * D;
    const uint16_t *vbase = a.v + ((size_t)bc.b * L_in * a.Hkv + bc.hkv) * D;
    const size_t cache_base = ((size_t)bc.b * a.Hkv + bc.hkv) * ((size_t)a.s + a.w_loc) * D;

    // Direct global -> LDS loads: load j of a tile fills LDS bytes [1024 j, 1024 j + 1024),
    // lane l the 16 bytes at 16 l: row kRowsPerLoad*j + l / kPieces, physical piece
    // l % kPieces, which holds logical piece (physical ^ swizzle).  This wave issues loads
    // j = wave*kLoadsPerWave .. +kLoadsPerWave-1.  Rows past the end of the sequence read the
    // last row (finite values; such keys are always masked).
    // The wave index as a uniform (scalar) value: the LDS destinations (M0) are then scalar.
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    uint32_t ld_koff[kLoadsPerWave], ld_voff[kLoadsPerWave];  // byte offsets from the tile's first row
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i) {
        const int row = kRowsPerLoad * (wave * kLoadsPerWave + i) + lane / kPieces;
        const int phys = lane % kPieces;
        ld_koff[i] = (uint32_t)(row * kv_row + (phys ^ swz_k<D>(row)) * 8) * 2u;
        ld_voff[i] = (uint32_t)(row * kv_row + (phys ^ swz_v(row)) * 8) * 2u;
    }
    // Loads the K rows (kv = 0) or the V rows (kv = 1) of the tile at key j0 into LDS buffer buf
    // (buf 2: the wide form's fifth chunk slot, which holds tile rows 0 .. 31, so only waves 0
    // and 1 load into it).
    auto issue = [&](int j0, int buf, auto kv_c) __attribute__((always_inline)) {
        constexpr int kv = decltype(kv_c)::value;
        const uint16_t *base = kv ? vbase : kbase;
        const int last = a.L - 1;
        if (j0 >= a.n_cached && j0 + kTileN - 1 <= last) {
            // Every row of the tile is a key of k/v inside the sequence: a scalar tile base plus
            // the per-lane offsets.
            const char *tile0 = reinterpret_cast<const char *>(base + (size_t)(j0 - a.n_cached) * kv_row);
#pragma unroll
            for (int i = 0; i < kLoadsPerWave; ++i) {
                const int j = wave_u * kLoadsPerWave + i;
                // (the builtin takes a non-const global pointer; the source is only read)
                __builtin_amdgcn_global_load_lds(const_cast<char *>(tile0 + (kv ? ld_voff[i] : ld_koff[i])),
                                                 SWA_LDS_PTR(buf == 2 ? &lds5[kv][1024 * j] : &lds[buf][kv][1024 * j]),
                                                 16, 0, 0);
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < kLoadsPerWave; ++i) {
            const int j = wave_u * kLoadsPerWave + i;
            const int row = kRowsPerLoad * j + lane / kPieces;
            const int piece = (lane % kPieces) ^ (kv ? swz_v(row) : swz_k<D>(row));
            const int key = min(j0 + row, last);
            const uint16_t *src;
            if (key >= a.n_cached) {
                src = base + (key - a.n_cached) * kv_row + piece * 8;
            } else {  // a cached key: its sink or ring slot
                int slot = key;
                if (key >= a.ns) {
                    const int r = a.ring0 + key - a.ns;
                    slot = a.s + (r >= a.w_loc ? r - a.w_loc : r);
                }
                src = (kv ? a.vc : a.kc) + cache_base + (size_t)slot * D + piece * 8;
            }
            __builtin_amdgcn_global_load_lds(const_cast<uint16_t *>(src),
                                             SWA_LDS_PTR(buf == 2 ? &lds5[kv][1024 * j] : &lds[buf][kv][1024 * j]),
                                             16, 0, 0);
        }
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

    f32x4 o[kDBlocks][2];
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db)
        o[db][0] = o[db][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Softmax state per query column, in log2 units: the reference maximum m_ref the
    // probabilities are taken against.  The running sum of the probabilities is computed
    // by the matrix cores from the same bf16-rounded values that weight V: a constant
    // A fragment whose row 0 is all ones turns one extra MFMA per chunk into
    // lsum[0] += sum_k P^T[k][q] (lane group 0 holds it; the other rows are zero).  The
    // dominant weight's rounding then cancels between numerator and denominator.
    float m_ref[2] = {-INFINITY, -INFINITY};
    f32x4 lsum[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    const __bf16 one_or_zero = static_cast<__bf16>(c16 == 0 ? 1.f : 0.f);
    const bf16x8 ones_row = {one_or_zero, one_or_zero, one_or_zero, one_or_zero,
                             one_or_zero, one_or_zero, one_or_zero, one_or_zero};

    if constexpr (RES) {
        // Resident forms (windows whose 32-token q-tile needs at most four 32-key chunks): every
        // chunk of the workgroup is loaded at once, slot k into rows 32 (k & 1) .. of buffer
        // k >> 1 (waves 2 (k & 1) and 2 (k & 1) + 1 load it; buffer 2 is the wide form's fifth
        // slot), then one barrier, after which the workgroup issues no more loads (the queries of
        // both halves in the wide form were loaded before it).  Each 16-column block is then done
        // over all of its chunks and stored at once: the stores of one block drain while the next
        // computes (a later wait for a load would also wait for those stores, since loads and
        // stores share one in-order counter).
        constexpr int kSlots = WIDE ? 5 : 4;
        const ChunkWalk cw = plan_chunks(t0, t1, a.w_loc, a.s, kChunkN);
        // Every slot is always loaded (a slot past the workgroup's chunks holds keys after t1, and
        // rows past the sequence read its last row), so any slot holds finite keys and values.
#pragma unroll
        for (int k = 0; k < kSlots; ++k) {
            if ((wave_u >> 1) == (k & 1)) {
                const int j0 = cw.chunk(k) * kChunkN - (k & 1) * kChunkN;  // tile row 0 holds key j0
                issue(j0, k >> 1, KRows());
                issue(j0, k >> 1, VRows());
            }
        }
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        __syncthreads();
        // LDS rows of chunk slot k (K or V).
        auto slot_rows = [&](int k, int kv) __attribute__((always_inline)) -> const unsigned char * {
            if (WIDE && k == 4)
                return &lds5[kv][0];
            return &lds[k >> 1][kv][0] + (k & 1) * kChunkBytes;
        };
        // With every key of a 32-token half at hand the softmax needs no running maximum: all
        // scores, the exact column maximum, the probabilities, then O^T = V^T P^T.  hw is the half's
        // own chunk walk (four chunks, straight-line code: a chunk past the half's last needed one
        // holds keys after its last token, which the element mask removes by causality), and
        // slot[k] the slot holding chunk hw.chunk(k).
        auto pass = [&](auto qb_c, const ChunkWalk &hw, const int (&slot)[4]) __attribute__((always_inline)) {
            constexpr int qb = decltype(qb_c)::value;
            const int t = tok[qb];
            f32x4 sr[4][2];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const unsigned char *kt = slot_rows(slot[k], 0);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    sr[k][h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < kKSteps; ++kk) {
                        const bf16x8 af = *reinterpret_cast<const bf16x8 *>(kt + k_lane[kk] + 4 * h * kRowBytes);
                        sr[k][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, qf[qb][kk], sr[k][h], 0, 0, 0);
                    }
                }
                if constexpr (WIDE)
                    if (k & 1)
                        __builtin_amdgcn_sched_barrier(0);
            }
            float mx = -INFINITY;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int key0 = hw.chunk(k) * kChunkN + 8 * g16;  // key of (h, j) = (0, 0)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int key = key0 + 4 * h + j;
                        const bool ok = (key <= t) & ((key > t - a.w_loc) | (key < a.s));
                        sr[k][h][j] = ok ? sr[k][h][j] : -INFINITY;
                    }
                    mx = fmaxf(fmaxf(mx, sr[k][h][0]), sr[k][h][1]);
                    mx = fmaxf(fmaxf(mx, sr[k][h][2]), sr[k][h][3]);
                }
            }
            const float mm = max_over_groups(mx) * c;
            const float m_use = mm == -INFINITY ? 0.f : mm;
            // Probabilities, their column sums (the ones-row MFMA), then O^T one 16-row block at a
            // time, each stored as soon as it is complete, so the stores spread over the compute.
            bf16x8 pf[4];
            f32x4 lq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        pf[k][4 * h + j] = static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(sr[k][h][j], c, -m_use)));
                lq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones_row, pf[k], lq, 0, 0, 0);
            }
            float l = lq[0];  // non-zero in lane group 0 only
            l += __shfl_xor(l, 16);
            l += __shfl_xor(l, 32);
            const float inv = 1.f / l;
            const uint32_t oa = row_off(qb, c16 & 7), ob = row_off(qb, (c16 & 7) + 8);
            f32x4 od_lo = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int db = 0; db < kDBlocks; ++db) {
                f32x4 od = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const unsigned char *vt = slot_rows(slot[k], 1);
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
        if constexpr (!WIDE) {
            const int slot[4] = {0, 1, 2, 3};
            pass(std::integral_constant<int, 0>(), cw, slot);
            pass(std::integral_constant<int, 1>(), cw, slot);
        } else {
            // The two 32-token halves of the q-tile, each with its own chunk walk.  A chunk the half
            // needs is one the workgroup needs, so it has a slot: below cw.n_sink the sink slots,
            // else the window slot counted from cw.win_lo.  A chunk past the half's needs may have
            // none (its keys are masked whatever the slot holds): it takes the last slot.
            auto half = [&](int h0, ChunkWalk &hw, int(&slot)[4]) __attribute__((always_inline)) {
                hw = plan_chunks(h0, min(h0 + kChunkN - 1, t1), a.w_loc, a.s, kChunkN);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int ch = hw.chunk(k);
                    const int sl = ch < cw.n_sink ? ch : cw.n_sink + (ch - cw.win_lo);
                    slot[k] = min(max(sl, 0), kSlots - 1);
                }
            };
            ChunkWalk hw;
            int slot[4];
            half(t0, hw, slot);
            pass(std::integral_constant<int, 0>(), hw, slot);
            pass(std::integral_constant<int, 1>(), hw, slot);
            if (t0 + kChunkN <= t1) {
                half(t0 + kChunkN, hw, slot);
                pass(std::integral_constant<int, 2>(), hw, slot);
                pass(std::integral_constant<int, 3>(), hw, slot);
            }
        }
    } else {
        const TileWalk tw = plan_tiles(t0, t1, a.w_loc, a.s, kTileN);
        const WalkSplit sp = split_walk(tw, t0, t1, a.w_loc, kTileN);
        auto tile_info = [&](int tile) __attribute__((always_inline)) {
            TileInfo ti;
            ti.j0 = tile * kTileN;
            tile_chunks(ti.j0, 2, t0, t1, a.w_loc, a.s, ti.c_lo, ti.c_hi);
            ti.mask_free = range_mask_free(ti.j0 + ti.c_lo * kChunkN, ti.j0 + ti.c_hi * kChunkN + kChunkN - 1, t0, t1,
                                           a.w_loc, a.s);
            return ti;
        };

        // The steps below take `fast` as a compile-time flag: a fast tile has both chunks needed and
        // no element mask, so its code is straight-line; otherwise chunks outside [c_lo, c_hi] are
        // skipped (loads aside: a tile is always loaded whole) and the mask is applied.

        // S^T = K Q^T of one tile, K from LDS.  Row m of 16-key block (kc, h) holds key
        // 32*kc + 8*(m/4) + 4*h + m%4, so lane group g later owns keys 32*kc + 8g .. +7.
        // (Skipped chunks are set to zero all the same: every element of sacc is then written by
        // each call, so the compiler does not keep the previous tile's scores alive.)
        auto scores = [&](f32x4(&sacc)[2][2][2], const unsigned char *kt, const TileInfo &ti, auto fast_c) __attribute__((always_inline)) {
            constexpr bool fast = decltype(fast_c)::value;
    #pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
    #pragma unroll
                for (int h = 0; h < 2; ++h)
                    sacc[kc][h][0] = sacc[kc][h][1] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (!fast && (kc < ti.c_lo || kc > ti.c_hi))
                    continue;
    #pragma unroll
                for (int h = 0; h < 2; ++h) {
    #pragma unroll
                    for (int kk = 0; kk < kKSteps; ++kk) {
                        const bf16x8 af =
                            *reinterpret_cast<const bf16x8 *>(kt + k_lane[kk] + (kc * kChunkN + 4 * h) * kRowBytes);
    #pragma unroll
                        for (int qb = 0; qb < 2; ++qb)
                            sacc[kc][h][qb] =
                                __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, qf[qb][kk], sacc[kc][h][qb], 0, 0, 0);
                    }
                }
            }
        };

        // Element mask of one tile (when some visited pair is outside A(t)), its column maxima, and
        // the lazy move of the reference maximum: m_ref only moves (and O and the sums are rescaled
        // by alpha) when the column maximum exceeds it by more than 8 in log2 units, so the
        // probabilities stay below 256 and most tiles need no rescale.  Returns whether any column
        // of this lane moved.
        auto tile_max = [&](f32x4(&sacc)[2][2][2], const TileInfo &ti, auto fast_c, float(&alpha)[2]) __attribute__((always_inline)) {
            constexpr bool fast = decltype(fast_c)::value;
            if (!fast && !ti.mask_free) {
    #pragma unroll
                for (int kc = 0; kc < 2; ++kc) {
                    if (kc < ti.c_lo || kc > ti.c_hi)
                        continue;
    #pragma unroll
                    for (int h = 0; h < 2; ++h)
    #pragma unroll
                        for (int qb = 0; qb < 2; ++qb)
    #pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                const int key = ti.j0 + kc * kChunkN + 8 * g16 + 4 * h + j;
                                const int t = tok[qb];
                                const bool ok = (key <= t) & ((key > t - a.w_loc) | (key < a.s));
                                sacc[kc][h][qb][j] = ok ? sacc[kc][h][qb][j] : -INFINITY;
                            }
                }
            }
            bool grow_any = false;
    #pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                // (pairs folded into the running maximum: three-input maxima)
                float mx = -INFINITY;
    #pragma unroll
                for (int kc = 0; kc < 2; ++kc) {
                    if (!fast && (kc < ti.c_lo || kc > ti.c_hi))
                        continue;
    #pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        mx = fmaxf(fmaxf(mx, sacc[kc][h][qb][0]), sacc[kc][h][qb][1]);
                        mx = fmaxf(fmaxf(mx, sacc[kc][h][qb][2]), sacc[kc][h][qb][3]);
                    }
                }
                mx = max_over_groups(mx);
                const float m_tile = mx * c;
                const bool grow = m_tile > m_ref[qb] + 8.f;
                // (a column with no allowed key so far keeps m_ref = -inf and alpha = 1)
                alpha[qb] = grow ? __builtin_amdgcn_exp2f(m_ref[qb] - m_tile) : 1.f;
                m_ref[qb] = grow ? m_tile : m_ref[qb];
                grow_any |= grow;
            }
            return grow_any;
        };

        // Probabilities of one tile against the reference maximum, as P^T B-operand fragments.
        auto probs = [&](const f32x4(&sacc)[2][2][2], const TileInfo &ti, auto fast_c, bf16x8(&pf)[2][2]) __attribute__((always_inline)) {
            constexpr bool fast = decltype(fast_c)::value;
    #pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const float m_use = m_ref[qb] == -INFINITY ? 0.f : m_ref[qb];
    #pragma unroll
                for (int kc = 0; kc < 2; ++kc) {
                    if (!fast && (kc < ti.c_lo || kc > ti.c_hi))
                        continue;
    #pragma unroll
                    for (int h = 0; h < 2; ++h)
    #pragma unroll
                        for (int j = 0; j < 4; ++j)
                            pf[kc][qb][4 * h + j] =
                                static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(sacc[kc][h][qb][j], c, -m_use)));
                }
            }
        };

        // O^T += V^T P^T over the tile's needed chunks, V from LDS, and the probability sums.
        auto accumulate = [&](const bf16x8(&pf)[2][2], const unsigned char *vt, const TileInfo &ti, auto fast_c) __attribute__((always_inline)) {
            constexpr bool fast = decltype(fast_c)::value;
    #pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
                if (!fast && (kc < ti.c_lo || kc > ti.c_hi))
                    continue;
    #pragma unroll
                for (int qb = 0; qb < 2; ++qb)
                    lsum[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones_row, pf[kc][qb], lsum[qb], 0, 0, 0);
    #pragma unroll
                for (int db = 0; db < kDBlocks; ++db) {
                    bf16x8 af;
    #pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int off = v_lane[db & 3] + (kc * kChunkN + 4 * h) * kRowBytes + 32 * (db & ~3);
                        const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) s16x4 *)(vt + off));
                        const bf16x4 y = __builtin_bit_cast(bf16x4, x);
                        af[4 * h + 0] = y[0];
                        af[4 * h + 1] = y[1];
                        af[4 * h + 2] = y[2];
                        af[4 * h + 3] = y[3];
                    }
    #pragma unroll
                    for (int qb = 0; qb < 2; ++qb)
                        o[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, pf[kc][qb], o[db][qb], 0, 0, 0);
                }
            }
        };

        auto rescale = [&](const float(&alpha)[2]) __attribute__((always_inline)) {
    #pragma unroll
            for (int db = 0; db < kDBlocks; ++db) {
                o[db][0] *= alpha[0];
                o[db][1] *= alpha[1];
            }
            lsum[0] *= alpha[0];
            lsum[1] *= alpha[1];
        };

        // The online softmax takes the tiles in any order: the edge tiles first, one per step,
        // then the middle tiles through a software pipeline.
        f32x4 sacc[2][2][2][2];  // [tile parity][kc][h][qb]
        float alpha[2];
        using Generic = std::integral_constant<bool, false>;
        using Fast = std::integral_constant<bool, true>;
        using Even = std::integral_constant<int, 0>;
        using Odd = std::integral_constant<int, 1>;

        // Edge tiles: step i computes tile i while K and V of tile i+1 load into the other buffer.
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
                scores(sacc[0], lds[buf][0], cur, Generic());
                if (__any(tile_max(sacc[0], cur, Generic(), alpha)))
                    rescale(alpha);
                bf16x8 pf[2][2];
                probs(sacc[0], cur, Generic(), pf);
                accumulate(pf, lds[buf][1], cur, Generic());
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
        // rescale for tile m+1 (rare) closes step m, after O has taken tile m.
        const int nm = sp.n_mid();
        if (nm > 0) {
            const int jm = sp.mid_lo * kTileN;
            const TileInfo full = {0, 0, 1, 1};  // (the fast steps read none of it)
            issue(jm, 0, KRows());
            issue(jm, 0, VRows());
            if (nm > 1)
                issue(jm + kTileN, 1, KRows());
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
            __syncthreads();
            scores(sacc[0], lds[0][0], full, Fast());
            if (__any(tile_max(sacc[0], full, Fast(), alpha)))
                rescale(alpha);

            auto mid_step = [&](const int m, auto buf_c) __attribute__((always_inline)) {  // m + 1 < nm
                constexpr int buf = decltype(buf_c)::value;  // m & 1
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // this wave's loads of the last step landed
                __syncthreads();                            // ... and every wave's; K buffer buf, V buffer buf^1 free
                if (m + 2 < nm)
                    issue(jm + (m + 2) * kTileN, buf, KRows());
                issue(jm + (m + 1) * kTileN, buf ^ 1, VRows());
                scores(sacc[buf ^ 1], lds[buf ^ 1][0], full, Fast());
                bf16x8 pf[2][2];
                probs(sacc[buf], full, Fast(), pf);
                accumulate(pf, lds[buf][1], full, Fast());
                const bool grow = tile_max(sacc[buf ^ 1], full, Fast(), alpha);
                if (__any(grow))
                    rescale(alpha);
            };
            // The last middle tile: its probabilities and O += V^T P^T.
            auto mid_last = [&](auto buf_c) __attribute__((always_inline)) {
                constexpr int buf = decltype(buf_c)::value;
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
                __syncthreads();
                bf16x8 pf[2][2];
                probs(sacc[buf], full, Fast(), pf);
                accumulate(pf, lds[buf][1], full, Fast());
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
        for (int qb = 0; qb < 2; ++qb) {
            float l = lsum[qb][0];  // non-zero in lane group 0 only
            l += __shfl_xor(l, 16);
            l += __shfl_xor(l, 32);
            const float inv = 1.f / l;
            const uint32_t oa = row_off(qb, c16 & 7), ob = row_off(qb, (c16 & 7) + 8);
    #pragma unroll
            for (int m = 0; m < kDBlocks / 2; ++m)
                store_pair(out_rs, oa + 128 * m, ob + 128 * m, o[2 * m][qb] * inv, o[2 * m + 1][qb] * inv);
        }
    }
}

// Debug: the set of (query, key) pairs the prefill kernel admits, from the same tile walk and
// split: edge tiles through the chunk selection, mask-free classification and element
// predicate; middle tiles whole and unmasked, as the kernel takes them.  One workgroup per
// q-tile.
__global__ void debug_prefill_mask_kernel(uint8_t *mask, int L, int Tm, int resident, int w_loc, int s)
{
    const int t0 = blockIdx.x * Tm;
    const int t1 = min(t0 + Tm - 1, L - 1);
    if (resident) {  // the resident form's chunk walk, every chunk element-masked
        const ChunkWalk cw = plan_chunks(t0, t1, w_loc, s, kChunkN);
        for (int k = 0; k < cw.count(); ++k) {
            const int k_lo = cw.chunk(k) * kChunkN;
            for (int idx = threadIdx.x; idx < Tm * kChunkN; idx += blockDim.x) {
                const int t = t0 + idx / kChunkN;
                const int key = k_lo + idx % kChunkN;
                if (t <= t1 && key < L && key_allowed(t, key, w_loc, s))
                    mask[(size_t)t * L + key] = 1;
            }
        }
        return;
    }
    const TileWalk tw = plan_tiles(t0, t1, w_loc, s, kTileN);
    const WalkSplit sp = split_walk(tw, t0, t1, w_loc, kTileN);
    for (int n = 0; n < tw.count(); ++n) {
        const bool middle = n >= sp.n_edge;
        const int j0 = (middle ? sp.mid_lo + (n - sp.n_edge) : sp.edge_tile(tw, n)) * kTileN;
        int c_lo = 0, c_hi = kTileN / kChunkN - 1;
        if (!middle)
            tile_chunks(j0, kTileN / kChunkN, t0, t1, w_loc, s, c_lo, c_hi);
        const int k_lo = j0 + c_lo * kChunkN, k_hi = j0 + c_hi * kChunkN + kChunkN - 1;
        const bool mask_free = middle || range_mask_free(k_lo, k_hi, t0, t1, w_loc, s);
        const int width = k_hi - k_lo + 1;
        for (int idx = threadIdx.x; idx < Tm * width; idx += blockDim.x) {
            const int t = t0 + idx / width;
            const int key = k_lo + idx % width;
            if (t > t1 || key >= L)
                continue;
            if (mask_free || key_allowed(t, key, w_loc, s))
                mask[(size_t)t * L + key] = 1;
        }
    }
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
    // window chunks and ceil(s/32) sink chunks.
    if (Tm % kChunkN != 0 || q_lo % kChunkN != 0)
        return false;
    const long long n = Tm / kChunkN + ((long long)w_loc - 1 + kChunkN - 1) / kChunkN + ((long long)s + kChunkN - 1) / kChunkN;
    return n <= 4;
}

namespace {

// Kernel form of a launch: the wide resident form where a wave's 64 rows are one head's 64
// tokens (four q-heads per kv-head slice) and each 32-token half fits the resident bound (then
// the 64-token q-tile needs at most five chunks); else the resident form; else the main form.
int prefill_form(const PrefillGeometry &g, int q_lo, int w_loc, int s)
{
    if (g.Gw == 4 && prefill_resident(g.Tm, q_lo, w_loc, s))
        return 2;
    return prefill_resident(g.Tm, q_lo, w_loc, s) ? 1 : 0;
}

}  // namespace

PrefillGeometry prefill_geometry(int L, int Hq, int Hkv)
{
    PrefillGeometry g;
    g.G = Hq / Hkv;
    g.Gw = 1;
    for (int c = 4; c >= 1; --c)
        if (g.G % c == 0) {
            g.Gw = c;
            break;
        }
    g.Tm = kRowsPerBlock / g.Gw;
    g.n_hslices = g.G / g.Gw;
    g.n_qtiles = (L + g.Tm - 1) / g.Tm;
    return g;
}

hipError_t launch_prefill(const void *q, const void *k, const void *v, float *out, int B, int Hq,
                          int Hkv, int L, int d, int w_loc, int s, float scale, hipStream_t stream,
                          hipEvent_t start, hipEvent_t stop, const PrefillKeySource *cached)
{
    int Lq = L, q_lo = 0;
    if (cached != nullptr) {
        Lq = L - cached->n_cached;
        q_lo = cached->n_cached;
    }
    PrefillGeometry g = prefill_geometry(Lq, Hq, Hkv);
    const int form = prefill_form(g, q_lo, w_loc, s);
    if (form == 2) {  // 64-token q-tiles: twice the rows per workgroup
        g.Tm *= 2;
        g.n_qtiles = (Lq + g.Tm - 1) / g.Tm;
    }
    PrefillArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.out = out;
    a.L = L;
    a.Lq = Lq;
    a.q_lo = q_lo;
    a.kc = cached ? static_cast<const uint16_t *>(cached->k_cache) : nullptr;
    a.vc = cached ? static_cast<const uint16_t *>(cached->v_cache) : nullptr;
    a.n_cached = cached ? cached->n_cached : 0;
    a.ns = cached ? cached->ns : 0;
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
    void (*const kernels[2][3])(PrefillArgs) = {
        {prefill_kernel<64, 0>, prefill_kernel<64, 1>, prefill_kernel<64, 2>},
        {prefill_kernel<128, 0>, prefill_kernel<128, 1>, prefill_kernel<128, 2>}};
    void (*kern)(PrefillArgs) = kernels[d == 128 ? 1 : 0][form];
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
    const PrefillGeometry g = prefill_geometry(L, Hq, Hkv);
    const size_t n = (size_t)L * L;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(256), dim3(256), 0, stream, mask, n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(debug_prefill_mask_kernel, dim3(g.n_qtiles), dim3(256), 0, stream, mask, L, g.Tm,
                       prefill_resident(g.Tm, 0, w_loc, s) ? 1 : 0, w_loc, s);
    return hipGetLastError();
}

}  // namespace swa
