// swa_model.hip -- the decoder-layer pieces around SWA(w,s) decode: RMSNorm and a streaming
// bf16 matrix-vector product for small batches with fused epilogues.
//
// They exist for the multi-layer decode measurement the pages describe (page "几亿Token白练了？
// 微软实测：免训练滑动窗口，让线性注意力破防" (PaperWeekly), section "小窗口也有工程优势": decode
// throughput and state memory of a 4-layer Transformer at batch 1 from 128 to 256K tokens of
// context).  The layer recipe (pre-norm, GQA attention, SwiGLU MLP) is the standard one; the
// pages fix none of it.
//
// At batch 1 every weight byte is read once per token and used for 2 flops per batch row, so
// the layer is bound by HBM bandwidth on the weights; the products run on the vector ALUs
// (v_dot2_f32_bf16: two bf16 products and an fp32 add per instruction), not on the matrix
// cores, which would idle 15 of their 16 columns.
#include "swa_launch.h"

#include <math.h>

namespace swa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint16_t to_bf16(float x) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x)); }
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    return (uint32_t)to_bf16(lo) | ((uint32_t)to_bf16(hi) << 16);
}

// acc + sum of the eight products w[i] x[i], as four two-product dot instructions.  (The
// pairs are taken with vector shuffles: bit-casting single 32-bit elements of a vector to
// bf16 pairs here made the compiler feed the first pair to all four instructions.)
__device__ __forceinline__ float dot8(bf16x8 w, bf16x8 x, float acc)
{
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(w, w, 0, 1), __builtin_shufflevector(x, x, 0, 1), acc,
                                          false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(w, w, 2, 3), __builtin_shufflevector(x, x, 2, 3), acc,
                                          false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(w, w, 4, 5), __builtin_shufflevector(x, x, 4, 5), acc,
                                          false);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(w, w, 6, 7), __builtin_shufflevector(x, x, 6, 7),
                                           acc, false);
}

__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        x += __shfl_xor(x, m, 64);
    return x;
}

// ----------------------------------------------------------------------------- RMSNorm
//
// out[b][i] = bf16( x[b][i] / sqrt(mean_i x[b][i]^2 + eps) * g[i] ); one workgroup per row.
// Rows of at most kNormThreads * 4 * kNormHeld elements stay in registers between the sum of
// squares and the scaling (one memory round trip); longer rows are read twice.
constexpr int kNormThreads = 256;
constexpr int kNormHeld = 4;  // float4 pieces per thread held in registers

__device__ __forceinline__ void norm_store(uint16_t *orow, int i, f32x4 v, uint2 gg, float inv)
{
    const float g0 = __uint_as_float(gg.x << 16), g1 = __uint_as_float(gg.x & 0xffff0000u);
    const float g2 = __uint_as_float(gg.y << 16), g3 = __uint_as_float(gg.y & 0xffff0000u);
    uint2 o;
    o.x = pack_bf16(v.x * inv * g0, v.y * inv * g1);
    o.y = pack_bf16(v.z * inv * g2, v.w * inv * g3);
    *reinterpret_cast<uint2 *>(orow + i) = o;
}

__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(const float *x, const uint16_t *g, uint16_t *out,
                                                               int n, float eps)
{
    const int b = blockIdx.x;
    const float *xr = x + (size_t)b * n;
    uint16_t *orow = out + (size_t)b * n;
    const bool held = n <= kNormThreads * 4 * kNormHeld;
    f32x4 v[kNormHeld];
    uint2 gg[kNormHeld];
    float ss = 0.f;
    if (held) {
#pragma unroll
        for (int k = 0; k < kNormHeld; ++k) {
            const int i = (threadIdx.x + k * kNormThreads) * 4;
            v[k] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (i < n) {
                v[k] = *reinterpret_cast<const f32x4 *>(xr + i);
                gg[k] = *reinterpret_cast<const uint2 *>(g + i);
            }
            ss += v[k].x * v[k].x + v[k].y * v[k].y + v[k].z * v[k].z + v[k].w * v[k].w;
        }
    } else {
        for (int i = threadIdx.x * 4; i < n; i += kNormThreads * 4) {
            const f32x4 w = *reinterpret_cast<const f32x4 *>(xr + i);
            ss += w.x * w.x + w.y * w.y + w.z * w.z + w.w * w.w;
        }
    }
    __shared__ float part[kNormThreads / 64];
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0)
        part[threadIdx.x >> 6] = ss;
    __syncthreads();
    ss = 0.f;
#pragma unroll
    for (int w = 0; w < kNormThreads / 64; ++w)
        ss += part[w];
    const float inv = 1.f / sqrtf(ss / (float)n + eps);
    if (held) {
#pragma unroll
        for (int k = 0; k < kNormHeld; ++k) {
            const int i = (threadIdx.x + k * kNormThreads) * 4;
            if (i < n)
                norm_store(orow, i, v[k], gg[k], inv);
        }
    } else {
        for (int i = threadIdx.x * 4; i < n; i += kNormThreads * 4)
            norm_store(orow, i, *reinterpret_cast<const f32x4 *>(xr + i), *reinterpret_cast<const uint2 *>(g + i),
                       inv);
    }
}

// ------------------------------------------------------------------------------ linear
//
// y[b][n] = sum_k W[n][k] x[b][k] for a batch of at most kLinBatch rows per workgroup
// (grid.y covers more) and kLinRows outputs per workgroup.  The 256 threads stride over the
// 16-byte pieces of the rows together (each round reads 4 KiB contiguous per weight row), so
// the weight stream is coalesced whatever K is; partial sums meet in a wave reduction and an
// LDS exchange.  Weights are read once (non-temporal loads: they do not fit in the caches);
// x is tiny and stays in L2.
constexpr int kLinThreads = 256;
constexpr int kLinRows = 2;
constexpr int kLinBatch = 4;

struct LinearArgs {
    const uint16_t *W;  // [N][K], or [2N][K] (gate rows, then up rows) for LIN_SILU_MUL
    const void *x;      // [B][K] bf16, or fp32 rounded to bf16 as it is read
    int B, N, K;
    uint16_t *out_bf16[3];  // LIN_STORE: outputs [seg[i], seg[i+1]) go to out_bf16[i] ([B][seg[i+1]-seg[i]])
    int seg[4];
    float *out_f32;  // LIN_ADD: [B][N], accumulated into
};

template <int MODE, bool IN_F32>
__global__ __launch_bounds__(kLinThreads) void linear_kernel(LinearArgs a)
{
    constexpr int kWRows = MODE == LIN_SILU_MUL ? 2 * kLinRows : kLinRows;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int n0 = blockIdx.x * kLinRows;
    const int b0 = blockIdx.y * kLinBatch;
    const int nb = min(kLinBatch, a.B - b0);
    const int P = a.K / 8;  // 16-byte pieces per row

    const uint16_t *wrow[kWRows];
#pragma unroll
    for (int r = 0; r < kWRows; ++r) {
        const int n = min(n0 + r % kLinRows, a.N - 1);  // rows past N repeat the last (results dropped)
        wrow[r] = a.W + (size_t)(r >= kLinRows ? a.N + n : n) * a.K;
    }
    float acc[kLinBatch][kWRows];
#pragma unroll
    for (int bb = 0; bb < kLinBatch; ++bb)
#pragma unroll
        for (int r = 0; r < kWRows; ++r)
            acc[bb][r] = 0.f;

    // x piece p of batch row bb as four bf16 pairs.
    auto x_piece = [&](int bb, int p) {
        u32x4 v;
        if (IN_F32) {
            const float *xr = static_cast<const float *>(a.x) + (size_t)(b0 + bb) * a.K + p * 8;
            const f32x4 lo = *reinterpret_cast<const f32x4 *>(xr);
            const f32x4 hi = *reinterpret_cast<const f32x4 *>(xr + 4);
            v = u32x4{pack_bf16(lo.x, lo.y), pack_bf16(lo.z, lo.w), pack_bf16(hi.x, hi.y), pack_bf16(hi.z, hi.w)};
        } else {
            v = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(a.x) + (size_t)(b0 + bb) * a.K + p * 8);
        }
        return v;
    };
    auto fma_piece = [&](int p) {
        u32x4 wv[kWRows];
#pragma unroll
        for (int r = 0; r < kWRows; ++r)
            wv[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(wrow[r] + (size_t)p * 8));
#pragma unroll
        for (int bb = 0; bb < kLinBatch; ++bb) {
            if (bb >= nb)
                break;
            const u32x4 xv = x_piece(bb, p);
            const bf16x8 xb = __builtin_bit_cast(bf16x8, xv);
#pragma unroll
            for (int r = 0; r < kWRows; ++r)
                acc[bb][r] = dot8(__builtin_bit_cast(bf16x8, wv[r]), xb, acc[bb][r]);
        }
    };
    int p = tid;
    for (; p + kLinThreads < P; p += 2 * kLinThreads) {  // two pieces in flight per weight row
        fma_piece(p);
        fma_piece(p + kLinThreads);
    }
    if (p < P)
        fma_piece(p);

    __shared__ float red[kLinThreads / 64][kLinBatch * kWRows];
#pragma unroll
    for (int bb = 0; bb < kLinBatch; ++bb) {
        if (bb >= nb)
            break;
#pragma unroll
        for (int r = 0; r < kWRows; ++r) {
            const float v = wave_sum(acc[bb][r]);
            if (lane == 0)
                red[wave][bb * kWRows + r] = v;
        }
    }
    __syncthreads();
    if (tid >= kLinBatch * kLinRows)
        return;
    const int bb = tid / kLinRows, r = tid % kLinRows;
    const int n = n0 + r, b = b0 + bb;
    if (bb >= nb || n >= a.N)
        return;
    float y = 0.f;
#pragma unroll
    for (int w = 0; w < kLinThreads / 64; ++w)
        y += red[w][bb * kWRows + r];
    if (MODE == LIN_STORE) {
        int i = 0;
        while (i < 2 && n >= a.seg[i + 1])
            ++i;
        const int len = a.seg[i + 1] - a.seg[i];
        a.out_bf16[i][(size_t)b * len + (n - a.seg[i])] = to_bf16(y);
    } else if (MODE == LIN_ADD) {
        a.out_f32[(size_t)b * a.N + n] += y;
    } else {
        float u = 0.f;
#pragma unroll
        for (int w = 0; w < kLinThreads / 64; ++w)
            u += red[w][bb * kWRows + kLinRows + r];
        a.out_bf16[0][(size_t)b * a.N + n] = to_bf16(y / (1.f + expf(-y)) * u);
    }
}

}  // namespace

hipError_t launch_rmsnorm(const float *x, const void *g, void *out, int B, int n, float eps, hipStream_t stream)
{
    hipLaunchKernelGGL(rmsnorm_kernel, dim3(B), dim3(kNormThreads), 0, stream, x, static_cast<const uint16_t *>(g),
                       static_cast<uint16_t *>(out), n, eps);
    return hipGetLastError();
}

hipError_t launch_linear(int mode, bool x_f32, const void *W, const void *x, int B, int N, int K,
                         void *const out_bf16[3], const int seg[4], float *out_f32, hipStream_t stream)
{
    LinearArgs a;
    a.W = static_cast<const uint16_t *>(W);
    a.x = x;
    a.B = B;
    a.N = N;
    a.K = K;
    for (int i = 0; i < 3; ++i)
        a.out_bf16[i] = static_cast<uint16_t *>(out_bf16[i]);
    for (int i = 0; i < 4; ++i)
        a.seg[i] = seg[i];
    a.out_f32 = out_f32;
    const dim3 grid((N + kLinRows - 1) / kLinRows, (B + kLinBatch - 1) / kLinBatch);
    void (*kern)(LinearArgs) = nullptr;
    if (mode == LIN_STORE)
        kern = x_f32 ? linear_kernel<LIN_STORE, true> : linear_kernel<LIN_STORE, false>;
    else if (mode == LIN_ADD)
        kern = x_f32 ? linear_kernel<LIN_ADD, true> : linear_kernel<LIN_ADD, false>;
    else
        kern = x_f32 ? linear_kernel<LIN_SILU_MUL, true> : linear_kernel<LIN_SILU_MUL, false>;
    hipLaunchKernelGGL(kern, grid, dim3(kLinThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace swa
