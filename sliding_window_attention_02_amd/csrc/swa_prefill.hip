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
// and the per-query softmax statistics (max, sum) never leave the lane group.  The
// 16-key row blocks of S^T are assigned keys so that lane group g of the PV product
// sees the 8 consecutive keys 32*kc + 8g .. 32*kc + 8g + 7, which V^T in LDS serves
// with one 16-byte read.  Any k-ordering the hardware uses inside the 8-value groups
// is the same for A and B, so the contraction is exact regardless.
//
// Memory: K and V tiles of 64 keys are staged global -> registers -> LDS with double
// buffering (one barrier per tile).  K is stored row-major with a 16-byte row pad
// (conflict-free 16-byte reads of 16 rows); V is stored transposed (V^T, row = d) with
// a 16-byte pad.  Q stays in registers for the whole key loop.  Workgroups are ordered
// heavy-first (last q-tile first) and mapped so that consecutive logical workgroups share
// an XCD and its L2, where neighbouring q-tiles re-read the same K/V tiles.
#include "swa_device.h"
#include "swa_launch.h"

#include <math.h>

namespace swa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTileN = 64;     // keys per KV tile
constexpr int kThreads = 256;  // 4 waves
constexpr int kRowsPerBlock = 128;

struct PrefillArgs {
    const uint16_t *q;
    const uint16_t *k;
    const uint16_t *v;
    float *out;
    int L, Hq, Hkv, G, Gw, Tm, n_qtiles, n_hslices;
    int w_loc, s;
    float scale_log2;
    int nblocks;
};

template <int D>
struct Lds {
    static constexpr int kKStride = D + 8;       // bf16 per K row
    static constexpr int kVStride = kTileN + 8;  // bf16 per V^T row
    static constexpr int kKElems = kTileN * kKStride;
    static constexpr int kVElems = D * kVStride;
};

__device__ __forceinline__ u32x4 ld16(const uint16_t *p) { return *reinterpret_cast<const u32x4 *>(p); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

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

template <int D>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(PrefillArgs a)
{
    constexpr int kChunks = D / 8;                           // 16-byte chunks per row
    constexpr int kKSteps = D / 32;                          // MFMA k-steps for S
    constexpr int kDBlocks = D / 16;                         // 16-row blocks of O^T
    constexpr int kKUnits = kTileN * kChunks / kThreads;     // K chunks per thread
    constexpr int kVUnits = (kTileN / 2) * kChunks / kThreads;  // V key-pair chunks per thread
    constexpr int kKStride = Lds<D>::kKStride;
    constexpr int kVStride = Lds<D>::kVStride;

    __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][Lds<D>::kKElems];
    __shared__ __attribute__((aligned(16))) uint16_t lds_v[2][Lds<D>::kVElems];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g16 = lane >> 4;  // lane group 0..3
    const int c16 = lane & 15;  // column inside a 16-wide MFMA block

    const BlockCoord bc = block_coord(a);
    const int t0 = bc.qt * a.Tm;
    const int t1 = min(t0 + a.Tm - 1, a.L - 1);

    // This lane's query column in each of its two 16-column blocks.
    int tok[2], head[2];
    bool valid[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int r = wave * 32 + qb * 16 + c16;
        const int gh = r / a.Tm;
        tok[qb] = t0 + r % a.Tm;
        head[qb] = bc.hkv * a.G + bc.hs * a.Gw + gh;
        valid[qb] = gh < a.Gw && tok[qb] < a.L;
    }

    // Q^T B-operand fragments: d = kk*32 + 8*g16 .. +7 of the lane's query.
    bf16x8 qf[2][kKSteps];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const uint16_t *qrow =
            a.q + (((size_t)bc.b * a.L + (valid[qb] ? tok[qb] : 0)) * a.Hq + (valid[qb] ? head[qb] : 0)) * D;
#pragma unroll
        for (int kk = 0; kk < kKSteps; ++kk) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (valid[qb])
                x = ld16(qrow + kk * 32 + g16 * 8);
            qf[qb][kk] = as_bf16x8(x);
        }
    }

    const size_t kv_row = (size_t)a.Hkv * D;  // elements between consecutive positions
    const uint16_t *kbase = a.k + ((size_t)bc.b * a.L * a.Hkv + bc.hkv) * D;
    const uint16_t *vbase = a.v + ((size_t)bc.b * a.L * a.Hkv + bc.hkv) * D;

    const TileWalk tw = plan_tiles(t0, t1, a.w_loc, a.s, kTileN);
    const int ntiles = tw.count();

    // Global -> register staging of one tile.
    u32x4 kst[kKUnits];
    u32x4 vst[kVUnits][2];
    auto stage = [&](int jt) {
        const int j0 = jt * kTileN;
#pragma unroll
        for (int u = 0; u < kKUnits; ++u) {
            const int unit = tid + u * kThreads;
            const int row = unit / kChunks, ch = unit % kChunks;
            const int key = j0 + row;
            kst[u] = u32x4{0u, 0u, 0u, 0u};
            if (key < a.L)
                kst[u] = ld16(kbase + (size_t)key * kv_row + ch * 8);
        }
#pragma unroll
        for (int u = 0; u < kVUnits; ++u) {
            const int unit = tid + u * kThreads;
            const int kp = unit % (kTileN / 2), ch = unit / (kTileN / 2);
            const int key = j0 + 2 * kp;
            vst[u][0] = u32x4{0u, 0u, 0u, 0u};
            vst[u][1] = u32x4{0u, 0u, 0u, 0u};
            if (key < a.L)
                vst[u][0] = ld16(vbase + (size_t)key * kv_row + ch * 8);
            if (key + 1 < a.L)
                vst[u][1] = ld16(vbase + (size_t)(key + 1) * kv_row + ch * 8);
        }
    };
    // Register -> LDS: K row-major, V transposed with two keys packed per 32-bit word.
    auto commit = [&](int buf) {
#pragma unroll
        for (int u = 0; u < kKUnits; ++u) {
            const int unit = tid + u * kThreads;
            const int row = unit / kChunks, ch = unit % kChunks;
            *reinterpret_cast<u32x4 *>(&lds_k[buf][row * kKStride + ch * 8]) = kst[u];
        }
#pragma unroll
        for (int u = 0; u < kVUnits; ++u) {
            const int unit = tid + u * kThreads;
            const int kp = unit % (kTileN / 2), ch = unit / (kTileN / 2);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t lo = vst[u][0][e >> 1], hi = vst[u][1][e >> 1];
                const uint32_t packed = (e & 1) ? ((lo >> 16) | (hi & 0xffff0000u))
                                                : ((lo & 0xffffu) | (hi << 16));
                *reinterpret_cast<uint32_t *>(&lds_v[buf][(ch * 8 + e) * kVStride + 2 * kp]) = packed;
            }
        }
    };

    f32x4 o[kDBlocks][2];
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db)
        o[db][0] = o[db][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[2] = {-INFINITY, -INFINITY};
    float l_run[2] = {0.f, 0.f};

    stage(tw.tile(0));
    commit(0);
    __syncthreads();

    for (int n = 0; n < ntiles; ++n) {
        const int buf = n & 1;
        const int j0 = tw.tile(n) * kTileN;
        if (n + 1 < ntiles)
            stage(tw.tile(n + 1));

        // S^T = K Q^T.  Row m of 16-key block kb holds key 32*(kb/2) + 8*(m/4) + 4*(kb%2) + m%4.
        f32x4 sacc[4][2];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            sacc[kb][0] = sacc[kb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int krow = 32 * (kb >> 1) + 8 * (c16 >> 2) + 4 * (kb & 1) + (c16 & 3);
#pragma unroll
            for (int kk = 0; kk < kKSteps; ++kk) {
                const bf16x8 af =
                    *reinterpret_cast<const bf16x8 *>(&lds_k[buf][krow * kKStride + kk * 32 + g16 * 8]);
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
                    sacc[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, qf[qb][kk], sacc[kb][qb], 0, 0, 0);
            }
        }

        // Element mask on edge tiles only, then the online softmax update per query column.
        const bool mask_free = tile_mask_free(j0, kTileN, t0, t1, a.w_loc, a.s);
        bf16x8 pf[2][2];  // [kc][qb]: P^T B-operand fragments
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            float sv[4][4];
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float x = sacc[kb][qb][j] * a.scale_log2;
                    if (!mask_free) {
                        const int key = j0 + 32 * (kb >> 1) + 8 * g16 + 4 * (kb & 1) + j;
                        if (!key_allowed(tok[qb], key, a.w_loc, a.s))
                            x = -INFINITY;
                    }
                    sv[kb][j] = x;
                    mx = fmaxf(mx, x);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run[qb], mx);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_use);
            m_run[qb] = m_new;
            float psum = 0.f;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float p = __builtin_amdgcn_exp2f(sv[kb][j] - m_use);
                    psum += p;
                    pf[kb >> 1][qb][4 * (kb & 1) + j] = static_cast<__bf16>(p);
                }
            l_run[qb] = l_run[qb] * alpha + psum;
#pragma unroll
            for (int db = 0; db < kDBlocks; ++db)
                o[db][qb] *= alpha;
        }

        // O^T += V^T P^T.
#pragma unroll
        for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
                const bf16x8 af = *reinterpret_cast<const bf16x8 *>(
                    &lds_v[buf][(db * 16 + c16) * kVStride + 32 * kc + 8 * g16]);
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
                    o[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, pf[kc][qb], o[db][qb], 0, 0, 0);
            }

        if (n + 1 < ntiles)
            commit(buf ^ 1);
        __syncthreads();
    }

    // Epilogue: finish the row sums across the four lane groups, normalise, store fp32.
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        float l = l_run[qb];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        const float inv = 1.f / l;
        if (valid[qb]) {
            float *orow = a.out + (((size_t)bc.b * a.L + tok[qb]) * a.Hq + head[qb]) * D;
#pragma unroll
            for (int db = 0; db < kDBlocks; ++db)
                *reinterpret_cast<f32x4 *>(orow + db * 16 + g16 * 4) = o[db][qb] * inv;
        }
    }
}

// Debug: the set of (query, key) pairs the prefill kernel admits, from the same tile walk,
// tile classification and element predicate.  One workgroup per q-tile.
__global__ void debug_prefill_mask_kernel(uint8_t *mask, int L, int Tm, int w_loc, int s)
{
    const int t0 = blockIdx.x * Tm;
    const int t1 = min(t0 + Tm - 1, L - 1);
    const TileWalk tw = plan_tiles(t0, t1, w_loc, s, kTileN);
    for (int n = 0; n < tw.count(); ++n) {
        const int j0 = tw.tile(n) * kTileN;
        const bool mask_free = tile_mask_free(j0, kTileN, t0, t1, w_loc, s);
        for (int idx = threadIdx.x; idx < Tm * kTileN; idx += blockDim.x) {
            const int t = t0 + idx / kTileN;
            const int key = j0 + idx % kTileN;
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
                          int Hkv, int L, int d, int w_loc, int s, float scale, hipStream_t stream)
{
    const PrefillGeometry g = prefill_geometry(L, Hq, Hkv);
    PrefillArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.out = out;
    a.L = L;
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
    if (d == 128)
        hipLaunchKernelGGL(prefill_kernel<128>, dim3(a.nblocks), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(prefill_kernel<64>, dim3(a.nblocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_debug_prefill_mask(uint8_t *mask, int L, int Hq, int Hkv, int w_loc, int s,
                                     hipStream_t stream)
{
    const PrefillGeometry g = prefill_geometry(L, Hq, Hkv);
    const size_t n = (size_t)L * L;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(256), dim3(256), 0, stream, mask, n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(debug_prefill_mask_kernel, dim3(g.n_qtiles), dim3(256), 0, stream, mask, L, g.Tm,
                       w_loc, s);
    return hipGetLastError();
}

}  // namespace swa
