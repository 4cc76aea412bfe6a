// swa_decode.hip -- bounded-cache SWA(w,s) decode for gfx950: append, split-K attend, merge.
//
// Cache per (b, kv-head): s pinned sink slots then a ring of w_loc slots, bf16
// [B][Hkv][s + w_loc][d].  Position p is stored in slot p (p < s) or s + (p mod w_loc):
// the rotating cache of page "从长文档摘要说起" (wiblog.cn), section "与 KV Cache 的配合：
// 轮转替换策略", with the sinks kept as on the first page's deployment notes (64+4=68
// tokens of KV at any context length).
//
// A step reads (s + w_loc) * d * 2 * 2 bytes per (b, kv-head) and does 4*d flops per key
// and q-head: with 4 q-heads per kv-head that is 8 flops per byte, more than the fp32 vector
// units sustain at HBM speed, so the products run on bf16 MFMA (the q-heads of a kv-head
// are the MFMA columns) and the kernel stays bound by the bytes it reads.  Split-K over the
// slot range of a (b, kv-head): when the range is at most four 32-slot chunks, the waves of one workgroup take one chunk each and merge their partial
// (max, sum, weighted values) through LDS; when the range exceeds what one wave holds (96
// slots), the splits are workgroups whose partials merge in a separate kernel.  Both merges
// visit the splits in a fixed order, so results do not depend on scheduling.
#include "swa_device.h"
#include "swa_launch.h"

#include <hip/hip_ext.h>
#include <math.h>

#include <mutex>

namespace swa {

// Static scratch for callers that cannot allocate (swa_decode_step_noalloc): the split partials
// (m, l, o) live here instead of in a caller workspace.  Each GPU the library runs on holds one
// copy for the life of the process; host code reaches it only through the per-device address
// that scratch_pointer() takes from hipGetSymbolAddress (the array's name in host code is a
// host-side stand-in, not a device address).
constexpr size_t kScratchBytes = size_t(8) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// V rows in LDS: 16-byte pieces XOR-swizzled so the transposed 8-byte reads of rows
// r..r+3 (r = 0 mod 4) at pieces P, P+1 hit 8 distinct pieces.
__device__ __forceinline__ int swz_v(int r) { return (r & 3) << 1; }

constexpr int kChunk = 32;      // slots per MFMA step
constexpr int kMaxChunks = 3;   // slots per wave <= 96
constexpr int kMaxWaveSplits = 4;  // waves (one chunk each) when a workgroup splits its slots

// Sum over the four lane groups (lanes l, l^16, l^32, l^48) that hold one MFMA column, with
// the gfx950 cross-row swaps: permlane32_swap(x, x) hands each lane its own value and the
// value of lane l^32 (one in each result), permlane16_swap likewise for lane l^16.
__device__ __forceinline__ float sum_over_groups(float x)
{
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}
__device__ __forceinline__ float max_over_groups(float x)
{
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
    const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

struct DecodeArgs {
    const uint16_t *q;
    uint16_t *kc;  // written only by the fused append path
    uint16_t *vc;
    const uint16_t *kn;  // fused append: new token's K/V [B][Hkv][d], or null
    const uint16_t *vn;
    float *out;
    const int64_t *pos;
    float *ws;  // [B][Hq][n_split][d + 2] partials (m, l, o[d]) when n_split > 1
    int Hq, Hkv, G, Gb, n_hslices;
    int s, w_loc, n_slots, n_split, slots_per_split;
    float scale_log2;
};

// grid: (n_split / WAVES, Hkv * n_hslices, B); WAVES waves per workgroup, wave w owning the
// slot segment [seg_lo, seg_hi) of split blockIdx.x * WAVES + w (at most NCH chunks of 32
// slots) of one (b, kv-head, head slice).  The
// GB <= 16 q-heads of the kv-head are the 16 columns of a bf16 MFMA (unused columns are zero),
// so the per-key work runs on the matrix cores:
//     S^T (32 keys x heads) = K (32 keys x d) . Q^T (d x heads)
//     O^T (d x heads)     += V^T (d x 32 keys) . P^T (32 keys x heads)
// the prefill kernel's layout (lane l holds column l % 16 of S^T for keys 8(l/16) .. +7 of
// the chunk, which is the B-operand layout of P^T).
//
// Latency: every load of the workgroup (Q, the K fragments of all chunks into registers, the
// V rows of all chunks straight into LDS, the new token) is issued before anything waits on
// the position, so a step costs one memory round trip.  The addresses do not depend on the
// position: once the ring has wrapped (t >= s + w_loc - 1) every slot holds a position of
// A(t).  Before that, the V rows of empty slots are zeroed in LDS after they land and their
// scores are masked, so whatever bytes such a slot holds never reach the result.  The fused
// path takes the new token's K (registers) and V (written over its LDS row) from the input.
template <int D, int NCH, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void decode_kernel(DecodeArgs a)
{
    constexpr int kKSteps = D / 32;   // MFMA k-steps for S
    constexpr int kDBlocks = D / 16;  // 16-row blocks of O^T
    constexpr int kPieces = D / 8;    // 16-byte pieces per row
    constexpr int kRowBytes = D * 2;
    constexpr int kRowsPerLoad = 1024 / kRowBytes;
    constexpr int kLoads = kChunk / kRowsPerLoad;  // 1 KiB direct loads per chunk of V
    __shared__ __attribute__((aligned(1024))) unsigned char vlds_all[WAVES][NCH][kChunk * kRowBytes];
    __shared__ float red_m[WAVES][16], red_l[WAVES][16];

    const int lane = threadIdx.x & 63;
    const int g16 = lane >> 4;
    const int c16 = lane & 15;
    // The wave as a uniform value (the direct-to-LDS destinations are scalar).
    const int wave = WAVES > 1 ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : 0;
    unsigned char(&vlds)[NCH][kChunk * kRowBytes] = vlds_all[wave];
    const int split = blockIdx.x * WAVES + wave;
    const int hkv = blockIdx.y / a.n_hslices;
    const int hs = blockIdx.y % a.n_hslices;
    const int b = blockIdx.z;
    const int GB = a.Gb;                 // heads of this workgroup (<= 16)
    const int h0 = hkv * a.G + hs * GB;  // first q-head of this workgroup
    const size_t cache_base = ((size_t)b * a.Hkv + hkv) * a.n_slots * D;
    const uint16_t *kcache = a.kc + cache_base;
    const uint16_t *vcache = a.vc + cache_base;
    const int seg_lo = split * a.slots_per_split;
    const int seg_hi = min(seg_lo + a.slots_per_split, a.n_slots);
    const int nch = (seg_hi - seg_lo + kChunk - 1) / kChunk;  // <= NCH
    const bool fused = a.kn != nullptr;

    // ---- every load, none of which depends on the position.
    const int64_t t = a.pos[b];
    bf16x8 qf[kKSteps];  // Q^T B operand: column c16 = q-head h0 + c16 (zero beyond GB)
    {
        const uint16_t *qrow = a.q + ((size_t)b * a.Hq + h0 + min(c16, GB - 1)) * D + g16 * 8;
#pragma unroll
        for (int kk = 0; kk < kKSteps; ++kk) {
            const u32x4 x = *reinterpret_cast<const u32x4 *>(qrow + kk * 32);
            qf[kk] = __builtin_bit_cast(bf16x8, c16 < GB ? x : u32x4{0u, 0u, 0u, 0u});
        }
    }
    // Rows past the segment repeat its last slot (in-bounds; their scores are masked).
    const int last = seg_hi - 1;
    // K first (the scores need it first), then V, which is only needed after the softmax.
    bf16x8 kf[NCH][2][kKSteps];  // K fragment (chunk, kb, kk): row 8(c16/4) + 4kb + c16%4
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
        if (ch < nch) {
            const int c0 = seg_lo + ch * kChunk;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int slot = min(c0 + 8 * (c16 >> 2) + 4 * kb + (c16 & 3), last);
#pragma unroll
                for (int kk = 0; kk < kKSteps; ++kk)
                    kf[ch][kb][kk] = __builtin_bit_cast(
                        bf16x8, *reinterpret_cast<const u32x4 *>(kcache + (size_t)slot * D + kk * 32 + g16 * 8));
            }
        }
    }
    // The new token's K at this lane's fragment pieces (every wave of the fused step: the scores
    // need it and the position, which says which wave's chunk holds it, is not read yet).
    const uint16_t *knew = fused ? a.kn + ((size_t)b * a.Hkv + hkv) * D : nullptr;
    bf16x8 knf[kKSteps];
    if (fused) {
#pragma unroll
        for (int kk = 0; kk < kKSteps; ++kk)
            knf[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(knew + kk * 32 + g16 * 8));
    }
    // V by buffer loads (a flat-encoded global load may, as far as the compiler knows, also
    // touch LDS, after which it would wait for every outstanding load, V included, before the
    // first score) into opaque LDS destinations (this wave reads only its own rows, after the
    // explicit wait below), so the scores and the softmax run while V lands.  Every chunk slot
    // is loaded (one past the segment repeats its last chunk and is never read): the same number
    // of loads on every path keeps the compiler's count of outstanding loads exact, so its waits
    // for Q and K do not also wait for V.
    const __amdgpu_buffer_rsrc_t v_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(vcache), 0, a.n_slots * kRowBytes, 0x00020000);
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
        const int c0 = seg_lo + min(ch, nch - 1) * kChunk;
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const int r = kRowsPerLoad * i + lane / kPieces;
            const int slot = min(c0 + r, last);
            const int piece = (lane % kPieces) ^ swz_v(r);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(v_rs, SWA_LDS_DMA_DST(&vlds[ch][1024 * i]), 16,
                                                     (slot * D + piece * 8) * 2, 0, 0, 0);
        }
    }

    // The position (a scalar load issued first) decides which wave holds the new token's slot;
    // the wait for it and the slot arithmetic come after every position-independent load is in
    // flight.  Only the owning wave loads the new token's row pieces (for its LDS row and the
    // cache write, both after V has landed).
    const SlotMap sm(t, a.s, a.w_loc);
    const int slot_t = t >= 0 ? sm.slot_of_t() : -1;
    const bool wrapped = sm.wrapped();  // every slot holds a position of A(t)
    const bool owns_new = fused && slot_t >= seg_lo && slot_t < seg_hi;
    u32x4 kn_piece = {0u, 0u, 0u, 0u}, vn_piece = {0u, 0u, 0u, 0u};  // piece `lane` of the new rows
    if (owns_new) {
        const uint16_t *vnew = a.vn + ((size_t)b * a.Hkv + hkv) * D;
        const int piece = min(lane, kPieces - 1);  // lanes past the row repeat its last piece
        kn_piece = *reinterpret_cast<const u32x4 *>(knew + piece * 8);
        vn_piece = *reinterpret_cast<const u32x4 *>(vnew + piece * 8);
    }

    // ---- scores of the whole segment (at most 96 slots, all in registers at once, so the
    // softmax takes the exact maximum in one pass: no running rescale).
    f32x4 sacc[NCH][2];
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
        const int c0 = seg_lo + ch * kChunk;
        if (fused && slot_t >= c0 && slot_t < c0 + kChunk) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const bool mine = c0 + 8 * (c16 >> 2) + 4 * kb + (c16 & 3) == slot_t;
#pragma unroll
                for (int kk = 0; kk < kKSteps; ++kk)
                    kf[ch][kb][kk] = mine ? knf[kk] : kf[ch][kb][kk];
            }
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            sacc[ch][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (ch < nch) {
#pragma unroll
                for (int kk = 0; kk < kKSteps; ++kk)
                    sacc[ch][kb] =
                        __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ch][kb][kk], qf[kk], sacc[ch][kb], 0, 0, 0);
            }
        }
    }
    // Mask: before the ring wraps, the slots outside A(t) and past the segment; after, only
    // the slots past the segment (rows the loads filled with the segment's last slot).  Then
    // the column maximum over the four lane groups.
    float mx = -INFINITY;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
        const int c0 = seg_lo + ch * kChunk;
        if (!wrapped) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int sj = c0 + 8 * g16 + 4 * kb + j;
                    sacc[ch][kb][j] = sm.admits(sj, seg_hi, false) ? sacc[ch][kb][j] : -INFINITY;
                }
        } else if (c0 + kChunk > seg_hi) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    sacc[ch][kb][j] = sm.admits(c0 + 8 * g16 + 4 * kb + j, seg_hi, true) ? sacc[ch][kb][j] : -INFINITY;
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            mx = fmaxf(mx, fmaxf(fmaxf(sacc[ch][kb][0], sacc[ch][kb][1]), fmaxf(sacc[ch][kb][2], sacc[ch][kb][3])));
    }
    mx = max_over_groups(mx);
    const float m_ref = mx * a.scale_log2;  // log2 units; -inf when the column sees no key
    const float m_use = mx == -INFINITY ? 0.f : m_ref;
    // P^T (bf16, B operand of PV) and its column sums from the same rounded values: a
    // constant A fragment whose row 0 is all ones makes one MFMA per chunk add the column
    // sum into lane group 0.
    const __bf16 one_or_zero = static_cast<__bf16>(c16 == 0 ? 1.f : 0.f);
    const bf16x8 ones_row = {one_or_zero, one_or_zero, one_or_zero, one_or_zero,
                             one_or_zero, one_or_zero, one_or_zero, one_or_zero};
    bf16x8 pf[NCH];
    f32x4 lsum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                pf[ch][4 * kb + j] =
                    static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(sacc[ch][kb][j], a.scale_log2, -m_use)));
        if (ch < nch)
            lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones_row, pf[ch], lsum, 0, 0, 0);
    }

    // ---- V: wait for the rows in LDS, fix them up, O^T += V^T P^T per chunk.
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): every V row is in LDS
    // The new token's cache rows (their pieces have landed with V).
    if (owns_new && hs == 0 && lane < kPieces) {
        *reinterpret_cast<u32x4 *>(a.kc + cache_base + (size_t)slot_t * D + lane * 8) = kn_piece;
        *reinterpret_cast<u32x4 *>(a.vc + cache_base + (size_t)slot_t * D + lane * 8) = vn_piece;
    }
    // Fix-ups (LDS operations of a wave complete in order, so the transposed reads below see
    // them): before the ring wraps, zero the rows of slots outside A(t) and past the segment
    // (after it wraps, every row holds finite cache data and the masked ones get weight 0);
    // put the new token's row over its slot.
    if (!wrapped) {
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) {
            const int c0 = seg_lo + ch * kChunk;
#pragma unroll
            for (int i = 0; i < kLoads; ++i) {
                const int sj = c0 + kRowsPerLoad * i + lane / kPieces;
                if (ch < nch && !sm.admits(sj, seg_hi, false))
                    *reinterpret_cast<u32x4 *>(&vlds[ch][1024 * i + 16 * lane]) = u32x4{0u, 0u, 0u, 0u};
            }
        }
    }
    if (fused && slot_t >= seg_lo && slot_t < seg_hi && lane < kPieces) {
        const int ch = (slot_t - seg_lo) / kChunk, r = (slot_t - seg_lo) % kChunk;
        // Rows past the segment loaded the segment's last slot.  When that slot is the one this
        // step writes (with s = 0, the step that first fills the ring's last slot is the step
        // the ring wraps), they hold its bytes from before the write, which may not be finite;
        // their weight is 0, but 0 * NaN is NaN, so they take the new row as well.
        const int r_end = slot_t == seg_hi - 1 ? kChunk : r + 1;
        for (int rr = r; rr < r_end; ++rr)
            *reinterpret_cast<u32x4 *>(&vlds[0][0] + ch * kChunk * kRowBytes + rr * kRowBytes +
                                       16 * (lane ^ swz_v(rr))) = vn_piece;
    }
    const int vt_row0 = 8 * g16 + (c16 >> 2);
    const int vt_half = 8 * (c16 & 1);
    const int vt_pbit = (c16 >> 1) & 1;
    f32x4 o[kDBlocks];
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db)
        o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
        if (ch >= nch)
            break;
#pragma unroll
        for (int db = 0; db < kDBlocks; ++db) {
            bf16x8 af;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int row = 4 * h + vt_row0;
                const int off = row * kRowBytes + 16 * ((2 * db + vt_pbit) ^ swz_v(row)) + vt_half;
                const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4 *)(&vlds[ch][off]));
                const bf16x4 y = __builtin_bit_cast(bf16x4, x);
                af[4 * h + 0] = y[0];
                af[4 * h + 1] = y[1];
                af[4 * h + 2] = y[2];
                af[4 * h + 3] = y[3];
            }
            o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, pf[ch], o[db], 0, 0, 0);
        }
    }

    // ---- output (one split), the partial (m, l, o) of this split, or the fixed-order merge of
    // the WAVES splits of this workgroup through LDS.
    float ll = sum_over_groups(lsum[0]);  // non-zero in lane group 0 only
    if constexpr (WAVES > 1) {
        // Each wave leaves (m, l) and its unscaled O^T (the columns of real heads only) in its own
        // LDS rows (it alone read them, so no barrier is needed first); after one barrier, wave w
        // rescales and adds, in wave order, the d-blocks db = w, w + WAVES, ... of all waves and
        // stores them.
        f32x4 *ored = reinterpret_cast<f32x4 *>(&vlds[0][0]);
        if (g16 == 0) {
            red_m[wave][c16] = m_ref;
            red_l[wave][c16] = ll;
        }
        if (c16 < GB) {
#pragma unroll
            for (int db = 0; db < kDBlocks; ++db)
                ored[db * 64 + lane] = o[db];
        }
        __syncthreads();
        if (c16 >= GB)
            return;
        float mm = -INFINITY;
#pragma unroll
        for (int w = 0; w < WAVES; ++w)
            mm = fmaxf(mm, red_m[w][c16]);
        const float mm_use = mm == -INFINITY ? 0.f : mm;
        float sc[WAVES];
        ll = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            sc[w] = __builtin_amdgcn_exp2f(red_m[w][c16] - mm_use);  // 0 for a split with no key
            ll += red_l[w][c16] * sc[w];
        }
        const float inv = ll > 0.f ? 1.f / ll : 0.f;
        float *orow = a.out + ((size_t)b * a.Hq + h0 + c16) * D;
#pragma unroll
        for (int db = 0; db < kDBlocks; ++db) {
            if (db % WAVES != wave)
                continue;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w = 0; w < WAVES; ++w)
                acc += reinterpret_cast<const f32x4 *>(&vlds_all[w][0][0])[db * 64 + lane] * sc[w];
            *reinterpret_cast<f32x4 *>(orow + db * 16 + g16 * 4) = acc * inv;
        }
        return;
    }
    if (c16 >= GB)
        return;
    const int h = h0 + c16;
    if (a.n_split == WAVES) {
        const float inv = ll > 0.f ? 1.f / ll : 0.f;
        float *orow = a.out + ((size_t)b * a.Hq + h) * D;
#pragma unroll
        for (int db = 0; db < kDBlocks; ++db)
            *reinterpret_cast<f32x4 *>(orow + db * 16 + g16 * 4) = o[db] * inv;
    } else {
        float *part = a.ws + (((size_t)b * a.Hq + h) * a.n_split + split) * (D + 2);
#pragma unroll
        for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                part[2 + db * 16 + g16 * 4 + j] = o[db][j];
        if (g16 == 0) {
            part[0] = m_ref;
            part[1] = ll;
        }
    }
}

// Fixed-order merge of the split partials.  grid: (Hq, B), block: kMergeThreads.  Thread t
// takes element dd = t % D of the splits i = g, g + G, g + 2G, ... (g = t / D, G groups); the
// groups' sums are then added in group order, so the result does not depend on scheduling.
constexpr int kMergeThreads = 1024;

template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const float *ws, float *out, int Hq, int n_split)
{
    constexpr int G = kMergeThreads / D;
    __shared__ float red[kMergeThreads];
    __shared__ float red_l[G];
    const int h = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
    const int dd = t % D, g = t / D;
    const float *part = ws + ((size_t)b * Hq + h) * n_split * (D + 2);
    // Maximum of the split maxima.
    float mm = -INFINITY;
    for (int i = t; i < n_split; i += kMergeThreads)
        mm = fmaxf(mm, part[(size_t)i * (D + 2)]);
    red[t] = mm;
    __syncthreads();
    for (int stride = kMergeThreads / 2; stride > 0; stride >>= 1) {
        if (t < stride)
            red[t] = fmaxf(red[t], red[t + stride]);
        __syncthreads();
    }
    mm = red[0];
    __syncthreads();
    const float m_use = mm == -INFINITY ? 0.f : mm;
    float ll = 0.f, oo = 0.f;
#pragma unroll 4
    for (int i = g; i < n_split; i += G) {
        const float *pi = part + (size_t)i * (D + 2);
        const float sc = __builtin_amdgcn_exp2f(pi[0] - m_use);
        ll += pi[1] * sc;
        oo += pi[2 + dd] * sc;
    }
    red[t] = oo;
    if (dd == 0)
        red_l[g] = ll;
    __syncthreads();
    if (g == 0) {
        float o_sum = 0.f, l_sum = 0.f;
#pragma unroll
        for (int j = 0; j < G; ++j) {
            o_sum += red[j * D + dd];
            l_sum += red_l[j];
        }
        out[((size_t)b * Hq + h) * D + dd] = l_sum > 0.f ? o_sum / l_sum : 0.f;
    }
}

// One thread per (b, token, kv-head, 16-byte chunk).  Positions that a later token of the
// same call overwrites are skipped, so no slot is written twice.
template <int D>
__global__ void kv_append_kernel(uint16_t *kc, uint16_t *vc, const uint16_t *kn, const uint16_t *vn,
                                 const int64_t *pos, int64_t pos0, int B, int Hkv, int s, int w_loc, int n_new)
{
    constexpr int kChunks = D / 8;
    const size_t total = (size_t)B * n_new * Hkv * kChunks;
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total)
        return;
    const int ch = (int)(idx % kChunks);
    size_t rest = idx / kChunks;
    const int hkv = (int)(rest % Hkv);
    rest /= Hkv;
    const int j = (int)(rest % n_new);
    const int b = (int)(rest / n_new);
    const int64_t p0 = pos != nullptr ? pos[b] : pos0;  // every sequence at pos0 when pos is null
    const int64_t p = p0 + j;
    if (p < 0)
        return;
    const int64_t last = p0 + n_new - 1;
    if (p >= s && p <= last - w_loc)
        return;  // overwritten by a later token of this call
    const int64_t slot = append_slot(p, s, w_loc);
    const size_t n_slots = (size_t)s + w_loc;
    const size_t src = (((size_t)b * n_new + j) * Hkv + hkv) * D + ch * 8;
    const size_t dst = (((size_t)b * Hkv + hkv) * n_slots + slot) * D + ch * 8;
    *reinterpret_cast<u32x4 *>(kc + dst) = *reinterpret_cast<const u32x4 *>(kn + src);
    *reinterpret_cast<u32x4 *>(vc + dst) = *reinterpret_cast<const u32x4 *>(vn + src);
}

// Debug: what the decode step attends to.  For each (b, split) of the decode plan, every slot of
// the split's segment goes through the kernel's own admission (SlotMap::admits: the wrap
// shortcut, else the 32-bit validity test); slot_pos[b][j] = the position slot j holds (position
// t at the slot the fused step writes, slot_of_t) if admitted, else -1.  Inconsistencies are
// flagged instead: -2 for an admitted slot that holds no position of A(t), -3 for a slot that two
// splits cover.  One thread per (b, split).
__global__ void debug_decode_slots_kernel(int64_t *slot_pos, const int64_t *pos, int B, int s, int w_loc,
                                          int n_split, int slots_per_split)
{
    const int n_slots = s + w_loc;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < B * n_split; i += gridDim.x * blockDim.x) {
        const int b = i / n_split, split = i % n_split;
        const SlotMap sm(pos[b], s, w_loc);
        const bool wrap = sm.wrapped();
        const int slot_t = pos[b] >= 0 ? sm.slot_of_t() : -1;
        const int seg_lo = split * slots_per_split;
        const int seg_hi = min(seg_lo + slots_per_split, n_slots);
        const int nch = (seg_hi - seg_lo + kChunk - 1) / kChunk;
        int64_t *out = slot_pos + (size_t)b * n_slots;
        for (int sj = seg_lo; sj < seg_lo + nch * kChunk; ++sj) {
            if (!sm.admits(sj, seg_hi, wrap))
                continue;  // (rows past the segment are never admitted)
            const int64_t p = sj == slot_t ? pos[b] : sm.position(sj);
            out[sj] = out[sj] != -1 ? -3 : (sm.position(sj) < 0 ? -2 : p);
        }
    }
}

__global__ void fill_i64_kernel(int64_t *p, size_t n, int64_t v)
{
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = v;
}

// Launches kern; with start/stop events the dispatch itself stamps them (kernel-only timing).
template <typename K>
void launch_timed(K kern, dim3 grid, dim3 block, hipStream_t stream, hipEvent_t start, hipEvent_t stop,
                  const DecodeArgs &a)
{
    if (start != nullptr || stop != nullptr)
        hipExtLaunchKernelGGL(kern, grid, block, 0, stream, start, stop, 0, a);
    else
        hipLaunchKernelGGL(kern, grid, block, 0, stream, a);
}

template <int D>
void launch_decode_d(const DecodeArgs &a, int wg_waves, int B, hipStream_t stream, hipEvent_t start, hipEvent_t stop)
{
    const dim3 grid(a.n_split / wg_waves, a.Hkv * a.n_hslices, B);
    const int nch = (a.slots_per_split + kChunk - 1) / kChunk;
    if (wg_waves == 2)
        launch_timed(decode_kernel<D, 1, 2>, grid, dim3(128), stream, start, stop, a);
    else if (wg_waves == 3)
        launch_timed(decode_kernel<D, 1, 3>, grid, dim3(192), stream, start, stop, a);
    else if (wg_waves == 4)
        launch_timed(decode_kernel<D, 1, 4>, grid, dim3(256), stream, start, stop, a);
    else if (nch <= 1)
        launch_timed(decode_kernel<D, 1, 1>, grid, dim3(64), stream, start, stop, a);
    else if (nch == 2)
        launch_timed(decode_kernel<D, 2, 1>, grid, dim3(64), stream, start, stop, a);
    else
        launch_timed(decode_kernel<D, 3, 1>, grid, dim3(64), stream, start, stop, a);
}

}  // namespace

DecodePlan decode_plan(int B, int Hq, int Hkv, int d, int w_loc, int s)
{
    DecodePlan p;
    const int G = Hq / Hkv;
    p.n_slots = s + w_loc;
    p.Gb = 1;
    for (int c = 16; c >= 1; --c)
        if (G % c == 0) {
            p.Gb = c;
            break;
        }
    p.n_hslices = G / p.Gb;
    // At most four 32-slot chunks: one workgroup of one wave per chunk for each (b, kv-head,
    // head slice), merged in LDS (faster than one wave over every chunk at each batch size
    // measured, 1 to 2048).  Otherwise one wave per workgroup over as few splits as its
    // register and LDS budget (kMaxChunks * 32 slots) allows: a second kernel (the merge)
    // costs more than the parallelism it buys, even at batch 1.
    const int chunks = (p.n_slots + kChunk - 1) / kChunk;
    if (chunks > 1 && chunks <= kMaxWaveSplits) {
        p.slots_per_split = kChunk;
        p.n_split = chunks;
        p.wg_waves = chunks;
        p.workspace_bytes = 0;
        return p;
    }
    p.wg_waves = 1;
    const long long want = (p.n_slots + kMaxChunks * kChunk - 1) / (kMaxChunks * kChunk);
    p.slots_per_split = (int)((p.n_slots + want - 1) / want);
    p.n_split = (p.n_slots + p.slots_per_split - 1) / p.slots_per_split;
    p.workspace_bytes = p.n_split > 1 ? (size_t)B * Hq * p.n_split * (d + 2) * sizeof(float) : 0;
    return p;
}

hipError_t launch_kv_append(void *k_cache, void *v_cache, const void *k_new, const void *v_new,
                            const int64_t *pos, int B, int Hkv, int d, int w_loc, int s, int n_new,
                            hipStream_t stream, int64_t pos0)
{
    const size_t total = (size_t)B * n_new * Hkv * (d / 8);
    const size_t blocks = (total + 255) / 256;
    if (blocks > 0x7fffffffULL)
        return hipErrorInvalidConfiguration;
    uint16_t *kc = static_cast<uint16_t *>(k_cache);
    uint16_t *vc = static_cast<uint16_t *>(v_cache);
    const uint16_t *kn = static_cast<const uint16_t *>(k_new);
    const uint16_t *vn = static_cast<const uint16_t *>(v_new);
    if (d == 128)
        hipLaunchKernelGGL(kv_append_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, stream, kc, vc, kn, vn,
                           pos, pos0, B, Hkv, s, w_loc, n_new);
    else
        hipLaunchKernelGGL(kv_append_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, stream, kc, vc, kn, vn,
                           pos, pos0, B, Hkv, s, w_loc, n_new);
    return hipGetLastError();
}

hipError_t launch_decode(const void *q, void *k_cache, void *v_cache, const void *k_new, const void *v_new,
                         float *out, const int64_t *pos, int B, int Hq, int Hkv, int d, int w_loc, int s,
                         float scale, void *workspace, const DecodePlan &plan, hipStream_t stream,
                         hipEvent_t start, hipEvent_t stop)
{
    const bool merged = plan.n_split != plan.wg_waves;  // a second kernel merges the splits
    DecodeArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.kc = static_cast<uint16_t *>(k_cache);
    a.vc = static_cast<uint16_t *>(v_cache);
    a.kn = static_cast<const uint16_t *>(k_new);
    a.vn = static_cast<const uint16_t *>(v_new);
    a.out = out;
    a.pos = pos;
    a.ws = static_cast<float *>(workspace);
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.Gb = plan.Gb;
    a.n_hslices = plan.n_hslices;
    a.s = s;
    a.w_loc = w_loc;
    a.n_slots = plan.n_slots;
    a.n_split = plan.n_split;
    a.slots_per_split = plan.slots_per_split;
    a.scale_log2 = scale * 1.4426950408889634f;
    // With a merge, the decode kernel stamps the start and the merge kernel the end.
    if (d == 128)
        launch_decode_d<128>(a, plan.wg_waves, B, stream, start, merged ? nullptr : stop);
    else
        launch_decode_d<64>(a, plan.wg_waves, B, stream, start, merged ? nullptr : stop);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !merged)
        return e;
    auto merge = d == 128 ? merge_kernel<128> : merge_kernel<64>;
    if (stop != nullptr)
        hipExtLaunchKernelGGL(merge, dim3(Hq, B), dim3(kMergeThreads), 0, stream, nullptr, stop, 0,
                              (const float *)a.ws, out, Hq, plan.n_split);
    else
        hipLaunchKernelGGL(merge, dim3(Hq, B), dim3(kMergeThreads), 0, stream, (const float *)a.ws, out, Hq,
                           plan.n_split);
    return hipGetLastError();
}

size_t scratch_capacity() { return kScratchBytes; }

hipError_t scratch_pointer(void **ptr)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *ptrs[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (ptrs[dev] == nullptr) {  // once per device, with that device current
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        ptrs[dev] = p;
    }
    *ptr = ptrs[dev];
    return hipSuccess;
}

ChunkPlan chunk_plan(int64_t pos0, int C, int w_loc, int s)
{
    ChunkPlan p;
    p.ns = pos0 < s ? (int)pos0 : s;
    p.nw = pos0 > s ? (int)(pos0 - s < w_loc - 1 ? pos0 - s : w_loc - 1) : 0;
    p.rows = p.ns + p.nw + C;
    p.ring0 = (int)((pos0 - p.nw) % w_loc);
    return p;
}

hipError_t launch_debug_decode_slots(int64_t *slot_pos, const int64_t *pos, int B, int w_loc, int s,
                                     hipStream_t stream)
{
    // The split geometry depends on the slot count only (heads and d pick the head slices).
    const DecodePlan plan = decode_plan(B, 1, 1, 128, w_loc, s);
    const size_t n = (size_t)B * plan.n_slots;
    hipLaunchKernelGGL(fill_i64_kernel, dim3(64), dim3(256), 0, stream, slot_pos, n, (int64_t)-1);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(debug_decode_slots_kernel, dim3(64), dim3(256), 0, stream, slot_pos, pos, B, s, w_loc,
                       plan.n_split, plan.slots_per_split);
    return hipGetLastError();
}

}  // namespace swa
