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
// are the MFMA columns) and the kernel stays bound by the bytes it reads.  The slot range
// of a (b, kv-head) is split over workgroups (split-K) when there are too few (b, kv-head)
// pairs to fill the GPU; partial (max, sum, weighted values) merge in a separate kernel
// that visits splits in a fixed order, so results do not depend on scheduling.
#include "swa_device.h"
#include "swa_launch.h"

#include <math.h>

namespace swa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// LDS pointer in the local address space for the direct global -> LDS load (written inline:
// a helper or an implicit conversion there makes the host pass drop the launch stub).
#define SWA_LDS_PTR(p) ((__attribute__((address_space(3))) void *)(p))

// V rows in LDS: 16-byte pieces XOR-swizzled so the transposed 8-byte reads of rows
// r..r+3 (r = 0 mod 4) at pieces P, P+1 hit 8 distinct pieces.
__device__ __forceinline__ int swz_v(int r) { return (r & 3) << 1; }

constexpr int kThreads = 256;
constexpr int kWaves = 4;


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

// grid: (n_split, Hkv * n_hslices, B); 4 waves.  The GB <= 16 q-heads of a kv-head are the
// 16 columns of a bf16 MFMA (unused columns are zero), so the per-key work runs on the
// matrix cores and the kernel stays bound by the cache bytes it reads:
//     S^T (32 keys x heads) = K (32 keys x d) . Q^T (d x heads)
//     O^T (d x heads)     += V^T (d x 32 keys) . P^T (32 keys x heads)
// exactly the prefill kernel's layout (lane l holds column l % 16 of S^T for keys
// 8(l/16) .. +7 of the chunk, which is the B-operand layout of P^T).  K fragments come
// straight from global memory; V rows go to a per-wave LDS buffer and come back transposed
// through ds_read_b64_tr_b16.  Each wave walks 32-slot chunks of the workgroup's segment
// with its own online-softmax state; the four states merge through LDS at the end.
template <int D>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a)
{
    constexpr int kChunk = 32;             // slots per wave iteration
    constexpr int kKSteps = D / 32;        // MFMA k-steps for S
    constexpr int kDBlocks = D / 16;       // 16-row blocks of O^T
    constexpr int kPieces = D / 8;         // 16-byte pieces per row
    constexpr int kRowBytes = D * 2;
    constexpr int kRowsPerLoad = 1024 / kRowBytes;
    constexpr int kLoads = kChunk / kRowsPerLoad;  // 1 KiB direct loads per chunk

    // V staging (per wave), reused after the slot loop for the wave merge of O.
    static_assert(kWaves * kChunk * kRowBytes == kWaves * 16 * D * 4, "merge buffer size");
    __shared__ __attribute__((aligned(1024))) unsigned char vlds[kWaves][kChunk * kRowBytes];
    __shared__ float red_m[kWaves][16];
    __shared__ float red_l[kWaves][16];
    float(*red_o)[16][D] = reinterpret_cast<float(*)[16][D]>(&vlds[0][0]);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g16 = lane >> 4;
    const int c16 = lane & 15;
    const int split = blockIdx.x;
    const int hkv = blockIdx.y / a.n_hslices;
    const int hs = blockIdx.y % a.n_hslices;
    const int b = blockIdx.z;
    const int GB = a.Gb;                 // heads of this workgroup (<= 16)
    const int h0 = hkv * a.G + hs * GB;  // first q-head of this workgroup

    const int64_t t = a.pos[b];
    const SlotMap sm(t, a.s, a.w_loc);
    const size_t cache_base = ((size_t)b * a.Hkv + hkv) * a.n_slots * D;
    const uint16_t *kcache = a.kc + cache_base;
    const uint16_t *vcache = a.vc + cache_base;
    const int seg_lo = split * a.slots_per_split;
    const int seg_hi = min(seg_lo + a.slots_per_split, a.n_slots);

    // The slot of position t.  Fused append: that slot's K/V come from the input (never from
    // the cache) in every workgroup, and one workgroup writes them to the cache.
    const bool fused = a.kn != nullptr;
    const int slot_t = t >= 0 ? sm.slot_of_t() : -1;
    const uint16_t *knew = fused ? a.kn + ((size_t)b * a.Hkv + hkv) * D : nullptr;
    const uint16_t *vnew = fused ? a.vn + ((size_t)b * a.Hkv + hkv) * D : nullptr;
    if (fused && hs == 0 && slot_t >= seg_lo && slot_t < seg_hi && tid < kPieces) {
        *reinterpret_cast<u32x4 *>(a.kc + cache_base + (size_t)slot_t * D + tid * 8) =
            *reinterpret_cast<const u32x4 *>(knew + tid * 8);
        *reinterpret_cast<u32x4 *>(a.vc + cache_base + (size_t)slot_t * D + tid * 8) =
            *reinterpret_cast<const u32x4 *>(vnew + tid * 8);
    }
    // Row pointer for a slot; slots that hold nothing of A(t) read the row of position t
    // instead (finite data, masked out), so no lane ever touches an unwritten row.
    auto krow = [&](int slot, bool valid) -> const uint16_t * {
        const int sl = valid ? slot : slot_t;
        if (sl < 0)
            return kcache;
        return (fused && sl == slot_t) ? knew : kcache + (size_t)sl * D;
    };
    auto vrow = [&](int slot, bool valid) -> const uint16_t * {
        const int sl = valid ? slot : slot_t;
        if (sl < 0)
            return vcache;
        return (fused && sl == slot_t) ? vnew : vcache + (size_t)sl * D;
    };

    // Q^T B-operand fragments: column c16 = q-head h0 + c16 (zero beyond GB).
    bf16x8 qf[kKSteps];
#pragma unroll
    for (int kk = 0; kk < kKSteps; ++kk) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (c16 < GB)
            x = *reinterpret_cast<const u32x4 *>(a.q + ((size_t)b * a.Hq + h0 + c16) * D + kk * 32 + g16 * 8);
        qf[kk] = __builtin_bit_cast(bf16x8, x);
    }
    const __bf16 one_or_zero = static_cast<__bf16>(c16 == 0 ? 1.f : 0.f);
    const bf16x8 ones_row = {one_or_zero, one_or_zero, one_or_zero, one_or_zero,
                             one_or_zero, one_or_zero, one_or_zero, one_or_zero};

    f32x4 o[kDBlocks];
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db)
        o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 lsum = {0.f, 0.f, 0.f, 0.f};
    float m_ref = -INFINITY;  // log2 units, per column; probabilities stay below 2^8

    unsigned char *vbuf = vlds[wave];
    const int vt_row0 = 8 * g16 + (c16 >> 2);
    const int vt_half = 8 * (c16 & 1);
    const int vt_pbit = (c16 >> 1) & 1;

    for (int c0 = seg_lo + wave * kChunk; c0 < seg_hi; c0 += kWaves * kChunk) {
        // V rows of the chunk -> this wave's LDS buffer (row-major, swizzled pieces).
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const int r = kRowsPerLoad * i + lane / kPieces;
            const int slot = c0 + r;
            const bool valid = slot < seg_hi && sm.valid(slot);
            const int piece = (lane % kPieces) ^ swz_v(r);
            __builtin_amdgcn_global_load_lds(const_cast<uint16_t *>(vrow(slot, valid) + piece * 8),
                                             SWA_LDS_PTR(vbuf + 1024 * i), 16, 0, 0);
        }
        // K fragments straight from global: row 8(c16/4) + 4kb + c16%4 of the chunk.
        bf16x8 kf[2][kKSteps];
        bool kvalid[2][4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int r = 8 * (c16 >> 2) + 4 * kb + (c16 & 3);
            const int slot = c0 + r;
            const bool valid = slot < seg_hi && sm.valid(slot);
            const uint16_t *kr = krow(slot, valid);
#pragma unroll
            for (int kk = 0; kk < kKSteps; ++kk)
                kf[kb][kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(kr + kk * 32 + g16 * 8));
            // validity of the keys this lane will hold in S^T: 8*g16 + 4kb + j
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int sj = c0 + 8 * g16 + 4 * kb + j;
                kvalid[kb][j] = sj < seg_hi && sm.valid(sj);
            }
        }
        f32x4 sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < kKSteps; ++kk)
                sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kb][kk], qf[kk], sacc[kb], 0, 0, 0);
        }
        // Mask, then the online softmax of the column (lazy rescale, threshold 8 in log2).
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                sacc[kb][j] = kvalid[kb][j] ? sacc[kb][j] : -INFINITY;
                mx = fmaxf(mx, sacc[kb][j]);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_tile = mx * a.scale_log2;
        if (__any(m_tile > m_ref + 8.f)) {
            const float m_new = fmaxf(m_ref, m_tile);
            const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
#pragma unroll
            for (int db = 0; db < kDBlocks; ++db)
                o[db] *= alpha;
            lsum *= alpha;
            m_ref = m_new;
        }
        const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
        bf16x8 pf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                pf[4 * kb + j] = static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(sacc[kb][j], a.scale_log2, -m_use)));
        lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones_row, pf, lsum, 0, 0, 0);

        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's V rows are in LDS
#pragma unroll
        for (int db = 0; db < kDBlocks; ++db) {
            bf16x8 af;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int row = 4 * h + vt_row0;
                const int off = row * kRowBytes + 16 * ((2 * db + vt_pbit) ^ swz_v(row)) + vt_half;
                const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(vbuf + off));
                const bf16x4 y = __builtin_bit_cast(bf16x4, x);
                af[4 * h + 0] = y[0];
                af[4 * h + 1] = y[1];
                af[4 * h + 2] = y[2];
                af[4 * h + 3] = y[3];
            }
            o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, pf, o[db], 0, 0, 0);
        }
        // The next iteration's loads overwrite vbuf: the transposed reads above must have
        // returned (they have: the MFMAs consumed them) before the loads are issued.
    }

    // Per-wave states -> LDS, then merge the waves: thread -> (head g, element d).
    __syncthreads();  // every wave is done with its V buffer, which now holds red_o
    if (g16 == 0 && c16 < GB) {
        red_m[wave][c16] = m_ref;
        red_l[wave][c16] = lsum[0];
    }
    if (c16 < GB) {
#pragma unroll
        for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                red_o[wave][c16][db * 16 + 4 * g16 + j] = o[db][j];
    }
    __syncthreads();
    for (int idx = tid; idx < GB * D; idx += kThreads) {
        const int g = idx / D, dd = idx % D;
        float mm = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
            mm = fmaxf(mm, red_m[w][g]);
        const float m_use = mm == -INFINITY ? 0.f : mm;
        float ll = 0.f, oo = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float sc = __builtin_amdgcn_exp2f(red_m[w][g] - m_use);
            ll += red_l[w][g] * sc;
            oo += red_o[w][g][dd] * sc;
        }
        const int h = h0 + g;
        if (a.n_split == 1) {
            a.out[((size_t)b * a.Hq + h) * D + dd] = ll > 0.f ? oo / ll : 0.f;
        } else {
            float *part = a.ws + (((size_t)b * a.Hq + h) * a.n_split + split) * (D + 2);
            part[2 + dd] = oo;
            if (dd == 0) {
                part[0] = mm;
                part[1] = ll;
            }
        }
    }
}

// Fixed-order merge of the split partials.  grid: (Hq, B), block: D threads.
template <int D>
__global__ __launch_bounds__(D) void merge_kernel(const float *ws, float *out, int Hq, int n_split)
{
    const int h = blockIdx.x, b = blockIdx.y, dd = threadIdx.x;
    const float *part = ws + ((size_t)b * Hq + h) * n_split * (D + 2);
    float mm = -INFINITY;
    for (int i = 0; i < n_split; ++i)
        mm = fmaxf(mm, part[i * (D + 2)]);
    const float m_use = mm == -INFINITY ? 0.f : mm;
    float ll = 0.f, oo = 0.f;
    for (int i = 0; i < n_split; ++i) {
        const float sc = __builtin_amdgcn_exp2f(part[i * (D + 2)] - m_use);
        ll += part[i * (D + 2) + 1] * sc;
        oo += part[i * (D + 2) + 2 + dd] * sc;
    }
    out[((size_t)b * Hq + h) * D + dd] = ll > 0.f ? oo / ll : 0.f;
}

// One thread per (b, token, kv-head, 16-byte chunk).  Positions that a later token of the
// same call overwrites are skipped, so no slot is written twice.
template <int D>
__global__ void kv_append_kernel(uint16_t *kc, uint16_t *vc, const uint16_t *kn, const uint16_t *vn,
                                 const int64_t *pos, int B, int Hkv, int s, int w_loc, int n_new)
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
    const int64_t p0 = pos[b];
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

__global__ void debug_decode_slots_kernel(int64_t *slot_pos, const int64_t *pos, int B, int s, int w_loc)
{
    const int n_slots = s + w_loc;
    const size_t total = (size_t)B * n_slots;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
        const int b = (int)(i / n_slots), j = (int)(i % n_slots);
        slot_pos[i] = SlotMap(pos[b], s, w_loc).position(j);
    }
}

template <int D>
void launch_decode_d(const DecodeArgs &a, int B, hipStream_t stream)
{
    hipLaunchKernelGGL(decode_kernel<D>, dim3(a.n_split, a.Hkv * a.n_hslices, B), dim3(kThreads), 0, stream, a);
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
    // Enough workgroups to cover the 256 CUs twice, but at least 32 slots per split.
    const long long pairs = (long long)B * Hkv * p.n_hslices;
    long long want = (512 + pairs - 1) / pairs;
    const long long max_split = (p.n_slots + 31) / 32;
    if (want > max_split)
        want = max_split;
    if (want < 1)
        want = 1;
    p.slots_per_split = (int)((p.n_slots + want - 1) / want);
    p.n_split = (p.n_slots + p.slots_per_split - 1) / p.slots_per_split;
    p.workspace_bytes = p.n_split > 1 ? (size_t)B * Hq * p.n_split * (d + 2) * sizeof(float) : 0;
    return p;
}

hipError_t launch_kv_append(void *k_cache, void *v_cache, const void *k_new, const void *v_new,
                            const int64_t *pos, int B, int Hkv, int d, int w_loc, int s, int n_new,
                            hipStream_t stream)
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
                           pos, B, Hkv, s, w_loc, n_new);
    else
        hipLaunchKernelGGL(kv_append_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, stream, kc, vc, kn, vn,
                           pos, B, Hkv, s, w_loc, n_new);
    return hipGetLastError();
}

hipError_t launch_decode(const void *q, void *k_cache, void *v_cache, const void *k_new, const void *v_new,
                         float *out, const int64_t *pos, int B, int Hq, int Hkv, int d, int w_loc, int s,
                         float scale, void *workspace, const DecodePlan &plan, hipStream_t stream)
{
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
    if (d == 128)
        launch_decode_d<128>(a, B, stream);
    else
        launch_decode_d<64>(a, B, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || plan.n_split == 1)
        return e;
    if (d == 128)
        hipLaunchKernelGGL(merge_kernel<128>, dim3(Hq, B), dim3(128), 0, stream, a.ws, out, Hq, plan.n_split);
    else
        hipLaunchKernelGGL(merge_kernel<64>, dim3(Hq, B), dim3(64), 0, stream, a.ws, out, Hq, plan.n_split);
    return hipGetLastError();
}

hipError_t launch_debug_decode_slots(int64_t *slot_pos, const int64_t *pos, int B, int w_loc, int s,
                                     hipStream_t stream)
{
    hipLaunchKernelGGL(debug_decode_slots_kernel, dim3(64), dim3(256), 0, stream, slot_pos, pos, B, s, w_loc);
    return hipGetLastError();
}

}  // namespace swa
