// swa_decode.hip -- bounded-cache SWA(w,s) decode for gfx950: append, split-K attend, merge.
//
// Cache per (b, kv-head): s pinned sink slots then a ring of w_loc slots, bf16
// [B][Hkv][s + w_loc][d].  Position p is stored in slot p (p < s) or s + (p mod w_loc):
// the rotating cache of page "从长文档摘要说起" (wiblog.cn), section "与 KV Cache 的配合：
// 轮转替换策略", with the sinks kept as on the first page's deployment notes (64+4=68
// tokens of KV at any context length).
//
// The step is memory-bound: each (b, kv-head) reads (s + w_loc) * d * 2 * 2 bytes and does
// 4*d flops per key and q-head.  A workgroup of 4 waves serves one (b, kv-head, head
// slice, split); lanes read 16-byte chunks so a wave instruction covers whole 256-byte
// rows (d = 128: 4 rows, d = 64: 8 rows), the Gb q-heads of the kv-head are dotted
// against each key in registers, and each row group keeps its own online-softmax state.
// States merge across row groups with cross-lane shuffles, across waves through LDS,
// and across splits in a separate merge kernel that visits splits in a fixed order (so
// results do not depend on scheduling).
#include "swa_device.h"
#include "swa_launch.h"

#include <math.h>

namespace swa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

struct DecodeArgs {
    const uint16_t *q;
    const uint16_t *kc;
    const uint16_t *vc;
    float *out;
    const int64_t *pos;
    float *ws;  // [B][Hq][n_split][d + 2] partials (m, l, o[d]) when n_split > 1
    int Hq, Hkv, G, Gb, n_hslices;
    int s, w_loc, n_slots, n_split, slots_per_split;
    float scale_log2;
};

// grid: (n_split, Hkv * n_hslices, B)
template <int D, int GB>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a)
{
    constexpr int kChunks = D / 8;             // lanes per cache row
    constexpr int kRowsPerWave = 64 / kChunks;  // rows covered by one wave instruction
    constexpr int kGroups = kWaves * kRowsPerWave;

    __shared__ float red_m[kWaves][GB];
    __shared__ float red_l[kWaves][GB];
    __shared__ float red_o[kWaves][GB][D];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int rg = lane / kChunks;  // row group inside the wave
    const int ch = lane % kChunks;  // 16-byte chunk of the row
    const int split = blockIdx.x;
    const int hkv = blockIdx.y / a.n_hslices;
    const int hs = blockIdx.y % a.n_hslices;
    const int b = blockIdx.z;

    const int64_t t = a.pos[b];
    const int h0 = hkv * a.G + hs * GB;  // first q-head of this workgroup

    // Queries of the GB heads, this lane's 8 values each, in fp32.
    float qv[GB][8];
#pragma unroll
    for (int g = 0; g < GB; ++g) {
        const u32x4 x = *reinterpret_cast<const u32x4 *>(a.q + ((size_t)b * a.Hq + h0 + g) * D + ch * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            qv[g][2 * e] = bf16_lo(x[e]);
            qv[g][2 * e + 1] = bf16_hi(x[e]);
        }
    }

    const size_t cache_base = ((size_t)b * a.Hkv + hkv) * a.n_slots * D;
    const uint16_t *kbase = a.kc + cache_base;
    const uint16_t *vbase = a.vc + cache_base;

    const int seg_lo = split * a.slots_per_split;
    const int seg_hi = min(seg_lo + a.slots_per_split, a.n_slots);

    float m[GB], l[GB], o[GB][8];
#pragma unroll
    for (int g = 0; g < GB; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            o[g][e] = 0.f;
    }

    for (int base = seg_lo; base < seg_hi; base += kGroups) {
        const int slot = base + wave * kRowsPerWave + rg;
        const bool in_seg = slot < seg_hi;
        const bool live = in_seg && slot_position(slot, t, a.s, a.w_loc) >= 0;
        u32x4 kx = {0u, 0u, 0u, 0u}, vx = {0u, 0u, 0u, 0u};
        if (live) {
            kx = *reinterpret_cast<const u32x4 *>(kbase + (size_t)slot * D + ch * 8);
            vx = *reinterpret_cast<const u32x4 *>(vbase + (size_t)slot * D + ch * 8);
        }
        float kf[8], vf[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            kf[2 * e] = bf16_lo(kx[e]);
            kf[2 * e + 1] = bf16_hi(kx[e]);
            vf[2 * e] = bf16_lo(vx[e]);
            vf[2 * e + 1] = bf16_hi(vx[e]);
        }
#pragma unroll
        for (int g = 0; g < GB; ++g) {
            float dot = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                dot = fmaf(qv[g][e], kf[e], dot);
            // Sum over the kChunks lanes of this row (they are consecutive lanes).
#pragma unroll
            for (int off = kChunks / 2; off >= 1; off >>= 1)
                dot += __shfl_xor(dot, off);
            const float x = live ? dot * a.scale_log2 : -INFINITY;
            const float m_new = fmaxf(m[g], x);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m[g] - m_use);
            const float p = __builtin_amdgcn_exp2f(x - m_use);
            m[g] = m_new;
            l[g] = l[g] * alpha + p;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                o[g][e] = fmaf(p, vf[e], o[g][e] * alpha);
        }
    }

    // Merge the row groups of the wave (lanes ch, ch + kChunks, ...).
#pragma unroll
    for (int g = 0; g < GB; ++g) {
#pragma unroll
        for (int off = kChunks; off < 64; off <<= 1) {
            const float m_o = __shfl_xor(m[g], off);
            const float l_o = __shfl_xor(l[g], off);
            const float m_new = fmaxf(m[g], m_o);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float a_s = __builtin_amdgcn_exp2f(m[g] - m_use);
            const float a_o = __builtin_amdgcn_exp2f(m_o - m_use);
            l[g] = l[g] * a_s + l_o * a_o;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float o_o = __shfl_xor(o[g][e], off);
                o[g][e] = o[g][e] * a_s + o_o * a_o;
            }
            m[g] = m_new;
        }
    }
    if (rg == 0) {
#pragma unroll
        for (int g = 0; g < GB; ++g) {
            if (ch == 0) {
                red_m[wave][g] = m[g];
                red_l[wave][g] = l[g];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e)
                red_o[wave][g][ch * 8 + e] = o[g][e];
        }
    }
    __syncthreads();

    // Merge the waves: thread -> (head g, element d).
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
        slot_pos[i] = slot_position(j, pos[b], s, w_loc);
    }
}

template <int D, int GB>
void launch_decode_t(const DecodeArgs &a, int B, hipStream_t stream)
{
    hipLaunchKernelGGL((decode_kernel<D, GB>), dim3(a.n_split, a.Hkv * a.n_hslices, B), dim3(kThreads), 0,
                       stream, a);
}

template <int D>
void launch_decode_d(const DecodeArgs &a, int B, hipStream_t stream)
{
    switch (a.Gb) {
    case 1: launch_decode_t<D, 1>(a, B, stream); break;
    case 2: launch_decode_t<D, 2>(a, B, stream); break;
    case 3: launch_decode_t<D, 3>(a, B, stream); break;
    case 4: launch_decode_t<D, 4>(a, B, stream); break;
    case 5: launch_decode_t<D, 5>(a, B, stream); break;
    case 6: launch_decode_t<D, 6>(a, B, stream); break;
    case 7: launch_decode_t<D, 7>(a, B, stream); break;
    default: launch_decode_t<D, 8>(a, B, stream); break;
    }
}

}  // namespace

DecodePlan decode_plan(int B, int Hq, int Hkv, int d, int w_loc, int s)
{
    DecodePlan p;
    const int G = Hq / Hkv;
    p.n_slots = s + w_loc;
    p.Gb = 1;
    for (int c = 8; c >= 1; --c)
        if (G % c == 0) {
            p.Gb = c;
            break;
        }
    p.n_hslices = G / p.Gb;
    // Enough workgroups to cover the 256 CUs twice, but at least 16 slots per split.
    const long long pairs = (long long)B * Hkv * p.n_hslices;
    long long want = (512 + pairs - 1) / pairs;
    const long long max_split = (p.n_slots + 15) / 16;
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

hipError_t launch_decode(const void *q, const void *k_cache, const void *v_cache, float *out,
                         const int64_t *pos, int B, int Hq, int Hkv, int d, int w_loc, int s,
                         float scale, void *workspace, const DecodePlan &plan, hipStream_t stream)
{
    DecodeArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.kc = static_cast<const uint16_t *>(k_cache);
    a.vc = static_cast<const uint16_t *>(v_cache);
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
