// swa_api.cpp -- the C ABI of libswa.so (declared in include/swa.h).
//
// Every entry point validates its arguments on the host before touching HIP, resolves
// the window convention to the local window w_loc, and enqueues kernels on the caller's
// stream.  Nothing here allocates, frees or synchronises device memory.
#include "swa.h"
#include "swa_launch.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>
#include <vector>

namespace {

thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok()
{
    g_last_error.clear();
    return SWA_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define CHECK_PTR(p)                                                                   \
    do {                                                                               \
        if ((p) == nullptr)                                                            \
            return fail(SWA_EINVAL, "%s: " #p " is null", fn);                         \
        if (!aligned16(p))                                                             \
            return fail(SWA_EINVAL, "%s: " #p " is not 16-byte aligned", fn);          \
    } while (0)

// Local window from (w, s, conv): w for SWA_CONV_ADDITIVE, w - s for SWA_CONV_TOTAL.
int resolve_window(const char *fn, int w, int s, int conv, int *w_loc)
{
    if (w < 1)
        return fail(SWA_EINVAL, "%s: w must be >= 1 (got %d)", fn, w);
    if (s < 0)
        return fail(SWA_EINVAL, "%s: s must be >= 0 (got %d)", fn, s);
    if (conv == SWA_CONV_ADDITIVE)
        *w_loc = w;
    else if (conv == SWA_CONV_TOTAL)
        *w_loc = w - s;
    else
        return fail(SWA_EINVAL, "%s: unknown window convention %d", fn, conv);
    if (*w_loc < 1)
        return fail(SWA_EINVAL, "%s: the total window w=%d leaves no local window after s=%d sinks", fn, w,
                    s);
    return SWA_OK;
}

int check_heads(const char *fn, int B, int Hq, int Hkv, int d)
{
    if (B < 1 || Hq < 1 || Hkv < 1)
        return fail(SWA_EINVAL, "%s: B, Hq, Hkv must be >= 1 (got %d, %d, %d)", fn, B, Hq, Hkv);
    if (Hq % Hkv != 0)
        return fail(SWA_EINVAL, "%s: Hq=%d is not a multiple of Hkv=%d", fn, Hq, Hkv);
    if (d != 64 && d != 128)
        return fail(SWA_EUNSUPPORTED, "%s: head dimension d=%d is not supported (64 or 128)", fn, d);
    return SWA_OK;
}

int check_scale(const char *fn, float scale)
{
    if (!std::isfinite(scale) || !(scale > 0.f))
        return fail(SWA_EINVAL, "%s: scale must be finite and > 0", fn);
    return SWA_OK;
}

// A (sequence, kv-head) cache of s + w_loc rows of d bf16 values is addressed by 32-bit signed
// byte offsets in the kernels: at most 2^31 - 1 bytes.
int check_cache(const char *fn, int s, int w_loc, int d)
{
    const long long rows = (long long)s + w_loc;
    if (rows * d * 2 > 0x7fffffffLL)
        return fail(SWA_EUNSUPPORTED, "%s: a cache of s + w_loc = %lld rows of d = %d exceeds 2^31 - 1 bytes per sequence and kv-head",
                    fn, rows, d);
    return SWA_OK;
}

// The decode launches index sequences by the grid's third dimension (the merge by its second),
// which holds at most 65535 blocks.
constexpr int kMaxDecodeBatch = 65535;

int check_decode_batch(const char *fn, int B)
{
    if (B > kMaxDecodeBatch)
        return fail(SWA_EUNSUPPORTED, "%s: B=%d exceeds the decode launch's %d sequences", fn, B, kMaxDecodeBatch);
    return SWA_OK;
}

// One sequence of q (and so of k and v, Hkv <= Hq) holds fewer than 2^31 elements, and a
// q-tile's output rows span less than 2 GiB: the kernels' 32-bit offsets.
int check_prefill_sizes(const char *fn, int L, int Hq, int d)
{
    if ((long long)L * Hq * d > 0x7fffffffLL)
        return fail(SWA_EUNSUPPORTED, "%s: one sequence of q holds more than 2^31-1 elements", fn);
    if ((long long)Hq * d >= (1LL << 22))
        return fail(SWA_EUNSUPPORTED, "%s: Hq * d = %lld reaches 2^22", fn, (long long)Hq * d);
    return SWA_OK;
}

int hip_status(const char *fn, hipError_t e)
{
    if (e != hipSuccess)
        return fail(SWA_EHIP, "%s: HIP error %d (%s)", fn, (int)e, hipGetErrorString(e));
    return ok();
}

int prefill_impl(const char *fn, const void *q, const void *k, const void *v, float *out, int B, int Hq, int Hkv,
                 int L, int d, int w, int s, float scale, int conv, void *stream, void *start, void *stop)
{
    CHECK_PTR(q);
    CHECK_PTR(k);
    CHECK_PTR(v);
    CHECK_PTR(out);
    int rc = check_heads(fn, B, Hq, Hkv, d);
    if (rc)
        return rc;
    if (L < 1)
        return fail(SWA_EINVAL, "%s: L must be >= 1 (got %d)", fn, L);
    int w_loc = 0;
    if ((rc = resolve_window(fn, w, s, conv, &w_loc)))
        return rc;
    if ((rc = check_scale(fn, scale)))
        return rc;
    if ((rc = check_prefill_sizes(fn, L, Hq, d)))
        return rc;
    return hip_status(fn, swa::launch_prefill(q, k, v, out, B, Hq, Hkv, L, d, w_loc, s, scale,
                                              static_cast<hipStream_t>(stream), static_cast<hipEvent_t>(start),
                                              static_cast<hipEvent_t>(stop)));
}

int decode_impl(const char *fn, const void *q, const void *k_cache, const void *v_cache, const void *k_new,
                const void *v_new, float *out, const int64_t *pos, int B, int Hq, int Hkv, int d, int w, int s,
                float scale, int conv, void *workspace, size_t workspace_bytes, void *stream, void *start = nullptr,
                void *stop = nullptr, bool use_scratch = false)
{
    CHECK_PTR(q);
    CHECK_PTR(k_cache);
    CHECK_PTR(v_cache);
    CHECK_PTR(out);
    if (pos == nullptr)
        return fail(SWA_EINVAL, "%s: pos is null", fn);
    int rc = check_heads(fn, B, Hq, Hkv, d);
    if (rc || (rc = check_decode_batch(fn, B)))
        return rc;
    int w_loc = 0;
    if ((rc = resolve_window(fn, w, s, conv, &w_loc)))
        return rc;
    if ((rc = check_scale(fn, scale)))
        return rc;
    if ((rc = check_cache(fn, s, w_loc, d)))
        return rc;
    const swa::DecodePlan plan = swa::decode_plan(B, Hq, Hkv, d, w_loc, s);
    if (use_scratch && plan.workspace_bytes > 0) {  // the static scratch stands in for the workspace
        if (plan.workspace_bytes > swa::scratch_capacity())
            return fail(SWA_EUNSUPPORTED, "%s: needs %zu bytes of scratch, the static scratch holds %zu", fn,
                        plan.workspace_bytes, swa::scratch_capacity());
        const hipError_t e = swa::scratch_pointer(&workspace);
        if (e != hipSuccess)
            return hip_status(fn, e);
        workspace_bytes = swa::scratch_capacity();
    }
    if (plan.workspace_bytes > 0) {
        if (workspace == nullptr || workspace_bytes < plan.workspace_bytes)
            return fail(SWA_EINVAL, "%s: workspace of %zu bytes needed, %zu given", fn, plan.workspace_bytes,
                        workspace == nullptr ? (size_t)0 : workspace_bytes);
        if (!aligned16(workspace))
            return fail(SWA_EINVAL, "%s: workspace is not 16-byte aligned", fn);
    }
    return hip_status(fn, swa::launch_decode(q, const_cast<void *>(k_cache), const_cast<void *>(v_cache), k_new,
                                             v_new, out, pos, B, Hq, Hkv, d, w_loc, s, scale, workspace, plan,
                                             static_cast<hipStream_t>(stream), static_cast<hipEvent_t>(start),
                                             static_cast<hipEvent_t>(stop)));
}

int chunk_impl(const char *fn, const void *q, const void *k, const void *v, void *k_cache, void *v_cache, float *out,
               float *lse, int64_t pos0, int B, int Hq, int Hkv, int C, int d, int w, int s, float scale, int conv,
               void *stream)
{
    CHECK_PTR(q);
    CHECK_PTR(k);
    CHECK_PTR(v);
    CHECK_PTR(k_cache);
    CHECK_PTR(v_cache);
    CHECK_PTR(out);
    if (lse != nullptr && !aligned16(lse))
        return fail(SWA_EINVAL, "%s: lse is not 16-byte aligned", fn);
    int rc = check_heads(fn, B, Hq, Hkv, d);
    if (rc)
        return rc;
    if (C < 1)
        return fail(SWA_EINVAL, "%s: C must be >= 1 (got %d)", fn, C);
    if (pos0 < 0)
        return fail(SWA_EINVAL, "%s: pos0 must be >= 0 (got %lld)", fn, (long long)pos0);
    int w_loc = 0;
    if ((rc = resolve_window(fn, w, s, conv, &w_loc)))
        return rc;
    if ((rc = check_scale(fn, scale)))
        return rc;
    if ((rc = check_cache(fn, s, w_loc, d)))
        return rc;
    // (the key rows may grow by up to 31 padding rows between the sinks and the window)
    if ((long long)s + w_loc - 1 + C + 31 > 0x7fffffffLL || (long long)C * Hq * d > 0x7fffffffLL)
        return fail(SWA_EUNSUPPORTED, "%s: one sequence's keys or queries exceed 2^31-1 elements", fn);
    if ((long long)Hq * d >= (1LL << 22))  // a q-tile's output rows must span less than 2 GiB
        return fail(SWA_EUNSUPPORTED, "%s: Hq * d = %lld reaches 2^22", fn, (long long)Hq * d);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const swa::ChunkPlan plan = swa::chunk_plan(pos0, C, w_loc, s);
    const swa::PrefillKeySource cached = {k_cache, v_cache, plan.ns + plan.nw, plan.ns, plan.ring0};
    // Attend (reading the cache as it stands), then append: the chunk's slots may hold keys
    // that its first queries still need.
    hipError_t e = swa::launch_prefill(q, k, v, out, B, Hq, Hkv, plan.rows, d, w_loc, s, scale, st, nullptr,
                                       nullptr, &cached, lse);
    if (e == hipSuccess)
        e = swa::launch_kv_append(k_cache, v_cache, k, v, nullptr, B, Hkv, d, w_loc, s, C, st, pos0);
    return hip_status(fn, e);
}

// ----------------------------------------------------------------- decoder-layer step
//
// Workspace of one layer step: bf16 h [B][dm], q [B][Hq d], k_new and v_new [B][Hkv d], fp32
// attention output [B][Hq d], bf16 MLP activation [B][f], then the attention's split
// workspace; each piece starts on a 256-byte boundary.
struct LayerWorkspace {
    size_t h, q, kn, vn, o, act, dec, total;
};

LayerWorkspace layer_workspace(int B, int dm, int Hq, int Hkv, int d, int f, size_t dec_bytes)
{
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    LayerWorkspace L;
    size_t off = 0;
    L.h = off;
    off += up((size_t)B * dm * 2);
    L.q = off;
    off += up((size_t)B * Hq * d * 2);
    L.kn = off;
    off += up((size_t)B * Hkv * d * 2);
    L.vn = off;
    off += up((size_t)B * Hkv * d * 2);
    L.o = off;
    off += up((size_t)B * Hq * d * 4);
    L.act = off;
    off += up((size_t)B * f * 2);
    L.dec = off;
    off += up(dec_bytes);
    L.total = off;
    return L;
}

int check_layer_dims(const char *fn, int B, int dm, int Hq, int Hkv, int d, int f)
{
    int rc = check_heads(fn, B, Hq, Hkv, d);
    if (rc)
        return rc;
    if (dm < 8 || dm % 8 != 0 || dm > (1 << 24))
        return fail(SWA_EINVAL, "%s: dm must be a multiple of 8 in [8, 2^24] (got %d)", fn, dm);
    if (f < 8 || f % 8 != 0 || f > (1 << 24))
        return fail(SWA_EINVAL, "%s: f must be a multiple of 8 in [8, 2^24] (got %d)", fn, f);
    if ((long long)B * (dm > f ? dm : f) > 0x7fffffffLL || (long long)(Hq + 2 * Hkv) * d > (1 << 24))
        return fail(SWA_EUNSUPPORTED, "%s: sizes exceed the supported range", fn);
    return SWA_OK;
}

int check_eps(const char *fn, float eps)
{
    if (!std::isfinite(eps) || eps < 0.f)
        return fail(SWA_EINVAL, "%s: eps must be finite and >= 0", fn);
    return SWA_OK;
}

// Everything swa_layer_decode_step checks for one layer except the workspace size; on success
// *w_loc is the layer's local window and *need its workspace bytes.
int check_layer(const char *fn, const swa_layer_weights *wts, const void *k_cache, const void *v_cache, int B, int dm,
                int Hq, int Hkv, int d, int f, int w, int s, int conv, int *w_loc, size_t *need)
{
    if (wts == nullptr)
        return fail(SWA_EINVAL, "%s: wts is null", fn);
    CHECK_PTR(wts->attn_norm);
    CHECK_PTR(wts->w_qkv);
    CHECK_PTR(wts->w_o);
    CHECK_PTR(wts->mlp_norm);
    CHECK_PTR(wts->w_gate_up);
    CHECK_PTR(wts->w_down);
    CHECK_PTR(k_cache);
    CHECK_PTR(v_cache);
    int rc = check_layer_dims(fn, B, dm, Hq, Hkv, d, f);
    if (rc || (rc = check_decode_batch(fn, B)))
        return rc;
    if ((rc = resolve_window(fn, w, s, conv, w_loc)))
        return rc;
    if ((rc = check_cache(fn, s, *w_loc, d)))
        return rc;
    *need = layer_workspace(B, dm, Hq, Hkv, d, f, swa::decode_plan(B, Hq, Hkv, d, *w_loc, s).workspace_bytes).total;
    return SWA_OK;
}

// The seven launches of one checked layer step: h = norm(x); q, k_new, v_new = W_qkv h; attend
// (appending k_new, v_new); x += W_o o; h = norm(x); act = silu(W_gate h) * (W_up h);
// x += W_down act.
hipError_t run_layer(float *x, const swa_layer_weights *wts, void *k_cache, void *v_cache, const int64_t *pos, int B,
                     int dm, int Hq, int Hkv, int d, int f, int w_loc, int s, float scale, float eps, char *ws,
                     hipStream_t st)
{
    const swa::DecodePlan plan = swa::decode_plan(B, Hq, Hkv, d, w_loc, s);
    const LayerWorkspace L = layer_workspace(B, dm, Hq, Hkv, d, f, plan.workspace_bytes);
    void *h = ws + L.h, *q = ws + L.q, *kn = ws + L.kn, *vn = ws + L.vn, *act = ws + L.act;
    float *o = reinterpret_cast<float *>(ws + L.o);
    const int nq = Hq * d, nkv = Hkv * d, nqkv = nq + 2 * nkv;
    void *none[3] = {nullptr, nullptr, nullptr};
    const int seg_none[4] = {0, 0, 0, 0};
    void *qkv_out[3] = {q, kn, vn};
    const int qkv_seg[4] = {0, nq, nq + nkv, nqkv};
    void *act_out[3] = {act, act, act};
    const int act_seg[4] = {0, f, f, f};
    hipError_t e = swa::launch_rmsnorm(x, wts->attn_norm, h, B, dm, eps, st);
    if (e == hipSuccess)
        e = swa::launch_linear(swa::LIN_STORE, false, wts->w_qkv, h, B, nqkv, dm, qkv_out, qkv_seg, nullptr, st);
    if (e == hipSuccess)
        e = swa::launch_decode(q, k_cache, v_cache, kn, vn, o, pos, B, Hq, Hkv, d, w_loc, s, scale,
                               plan.workspace_bytes > 0 ? ws + L.dec : nullptr, plan, st);
    if (e == hipSuccess)
        e = swa::launch_linear(swa::LIN_ADD, true, wts->w_o, o, B, dm, nq, none, seg_none, x, st);
    if (e == hipSuccess)
        e = swa::launch_rmsnorm(x, wts->mlp_norm, h, B, dm, eps, st);
    if (e == hipSuccess)
        e = swa::launch_linear(swa::LIN_SILU_MUL, false, wts->w_gate_up, h, B, f, dm, act_out, act_seg, nullptr, st);
    if (e == hipSuccess)
        e = swa::launch_linear(swa::LIN_ADD, false, wts->w_down, act, B, dm, f, none, seg_none, x, st);
    return e;
}

}  // namespace

extern "C" {

const char *swa_last_error(void) { return g_last_error.c_str(); }

int swa_prefill_chunk(const void *q, const void *k, const void *v, void *k_cache, void *v_cache, float *out,
                      float *lse, int64_t pos0, int B, int Hq, int Hkv, int C, int d, int w, int s, float scale,
                      int conv, void *stream)
{
    return chunk_impl("swa_prefill_chunk", q, k, v, k_cache, v_cache, out, lse, pos0, B, Hq, Hkv, C, d, w, s, scale,
                      conv, stream);
}


int swa_prefill(const void *q, const void *k, const void *v, float *out, int B, int Hq, int Hkv, int L,
                int d, int w, int s, float scale, int conv, void *stream)
{
    return prefill_impl("swa_prefill", q, k, v, out, B, Hq, Hkv, L, d, w, s, scale, conv, stream, nullptr,
                        nullptr);
}

int swa_prefill_describe(int B, int Hq, int Hkv, int L, int d, int w, int s, int conv, swa_prefill_info *info)
{
    const char *fn = "swa_prefill_describe";
    if (info == nullptr)
        return fail(SWA_EINVAL, "%s: info is null", fn);
    int rc = check_heads(fn, B, Hq, Hkv, d);
    if (rc)
        return rc;
    if (L < 1)
        return fail(SWA_EINVAL, "%s: L must be >= 1 (got %d)", fn, L);
    if ((rc = check_prefill_sizes(fn, L, Hq, d)))
        return rc;
    int w_loc = 0;
    if ((rc = resolve_window(fn, w, s, conv, &w_loc)))
        return rc;
    const swa::PrefillPlan p = swa::prefill_plan(B, Hq, Hkv, L, w_loc, s);
    info->form = p.form;
    info->tokens_per_tile = p.g.Tm;
    info->heads_per_tile = p.g.Gw;
    info->workgroups = p.workgroups;
    info->executed_pairs = p.executed_pairs;
    return ok();
}

int swa_prefill_timed(const void *q, const void *k, const void *v, float *out, int B, int Hq, int Hkv, int L,
                      int d, int w, int s, float scale, int conv, void *stream, void *start_event,
                      void *stop_event)
{
    if (start_event == nullptr || stop_event == nullptr)
        return fail(SWA_EINVAL, "swa_prefill_timed: start_event and stop_event must not be null");
    return prefill_impl("swa_prefill_timed", q, k, v, out, B, Hq, Hkv, L, d, w, s, scale, conv, stream,
                        start_event, stop_event);
}

int swa_kv_append(void *k_cache, void *v_cache, const void *k_new, const void *v_new, const int64_t *pos,
                  int B, int Hkv, int d, int w, int s, int n_new, int conv, void *stream)
{
    const char *fn = "swa_kv_append";
    CHECK_PTR(k_cache);
    CHECK_PTR(v_cache);
    CHECK_PTR(k_new);
    CHECK_PTR(v_new);
    if (pos == nullptr)
        return fail(SWA_EINVAL, "%s: pos is null", fn);
    int rc = check_heads(fn, B, Hkv, Hkv, d);
    if (rc)
        return rc;
    if (n_new < 1)
        return fail(SWA_EINVAL, "%s: n_new must be >= 1 (got %d)", fn, n_new);
    int w_loc = 0;
    if ((rc = resolve_window(fn, w, s, conv, &w_loc)))
        return rc;
    if ((rc = check_cache(fn, s, w_loc, d)))
        return rc;
    return hip_status(fn, swa::launch_kv_append(k_cache, v_cache, k_new, v_new, pos, B, Hkv, d, w_loc, s,
                                                n_new, static_cast<hipStream_t>(stream)));
}

long long swa_cache_slots(int w, int s, int conv)
{
    int w_loc = 0;
    if (resolve_window("swa_cache_slots", w, s, conv, &w_loc))
        return -1;
    ok();
    return (long long)s + w_loc;
}

size_t swa_decode_workspace_bytes(int B, int Hq, int Hkv, int d, int w, int s, int conv)
{
    const char *fn = "swa_decode_workspace_bytes";
    if (check_heads(fn, B, Hq, Hkv, d) || check_decode_batch(fn, B))
        return 0;
    int w_loc = 0;
    if (resolve_window(fn, w, s, conv, &w_loc))
        return 0;
    if (check_cache(fn, s, w_loc, d))
        return 0;
    return swa::decode_plan(B, Hq, Hkv, d, w_loc, s).workspace_bytes;
}


int swa_decode_describe(int B, int Hq, int Hkv, int d, int w, int s, int conv, swa_decode_info *info)
{
    const char *fn = "swa_decode_describe";
    if (info == nullptr)
        return fail(SWA_EINVAL, "%s: info is null", fn);
    int rc = check_heads(fn, B, Hq, Hkv, d);
    if (rc || (rc = check_decode_batch(fn, B)))
        return rc;
    int w_loc = 0;
    if ((rc = resolve_window(fn, w, s, conv, &w_loc)))
        return rc;
    if ((rc = check_cache(fn, s, w_loc, d)))
        return rc;
    const swa::DecodePlan p = swa::decode_plan(B, Hq, Hkv, d, w_loc, s);
    info->splits = p.n_split;
    info->waves_per_workgroup = p.wg_waves;
    info->slots_per_split = p.slots_per_split;
    info->heads_per_wave = p.Gb;
    info->workgroups = (long long)B * Hkv * p.n_hslices * (p.n_split / p.wg_waves);
    info->merge_launch = p.n_split != p.wg_waves;
    info->workspace_bytes = p.workspace_bytes;
    return ok();
}

int swa_decode_step(const void *q, const void *k_cache, const void *v_cache, float *out, const int64_t *pos,
                    int B, int Hq, int Hkv, int d, int w, int s, float scale, int conv, void *workspace,
                    size_t workspace_bytes, void *stream)
{
    return decode_impl("swa_decode_step", q, k_cache, v_cache, nullptr, nullptr, out, pos, B, Hq, Hkv, d, w, s,
                       scale, conv, workspace, workspace_bytes, stream);
}

int swa_decode_step_noalloc(const void *q, const void *k_cache, const void *v_cache, float *out, const int64_t *pos,
                            int B, int Hq, int Hkv, int d, int w, int s, float scale, int conv, void *stream)
{
    return decode_impl("swa_decode_step_noalloc", q, k_cache, v_cache, nullptr, nullptr, out, pos, B, Hq, Hkv, d, w,
                       s, scale, conv, nullptr, 0, stream, nullptr, nullptr, true);
}

int swa_append_decode_step(const void *q, void *k_cache, void *v_cache, const void *k_new, const void *v_new,
                           float *out, const int64_t *pos, int B, int Hq, int Hkv, int d, int w, int s,
                           float scale, int conv, void *workspace, size_t workspace_bytes, void *stream)
{
    const char *fn = "swa_append_decode_step";
    CHECK_PTR(k_new);
    CHECK_PTR(v_new);
    return decode_impl(fn, q, k_cache, v_cache, k_new, v_new, out, pos, B, Hq, Hkv, d, w, s, scale, conv,
                       workspace, workspace_bytes, stream);
}

int swa_append_decode_step_timed(const void *q, void *k_cache, void *v_cache, const void *k_new, const void *v_new,
                                 float *out, const int64_t *pos, int B, int Hq, int Hkv, int d, int w, int s,
                                 float scale, int conv, void *workspace, size_t workspace_bytes, void *stream,
                                 void *start_event, void *stop_event)
{
    const char *fn = "swa_append_decode_step_timed";
    if (start_event == nullptr || stop_event == nullptr)
        return fail(SWA_EINVAL, "%s: start_event and stop_event must not be null", fn);
    CHECK_PTR(k_new);
    CHECK_PTR(v_new);
    return decode_impl(fn, q, k_cache, v_cache, k_new, v_new, out, pos, B, Hq, Hkv, d, w, s, scale, conv,
                       workspace, workspace_bytes, stream, start_event, stop_event);
}

int swa_debug_prefill_mask(uint8_t *mask, int L, int Hq, int Hkv, int d, int w, int s, int conv, void *stream)
{
    const char *fn = "swa_debug_prefill_mask";
    if (mask == nullptr)
        return fail(SWA_EINVAL, "%s: mask is null", fn);
    int rc = check_heads(fn, 1, Hq, Hkv, d);
    if (rc)
        return rc;
    if (L < 1 || L > 8192)
        return fail(SWA_EINVAL, "%s: L must be in [1, 8192] (got %d)", fn, L);
    int w_loc = 0;
    if ((rc = resolve_window(fn, w, s, conv, &w_loc)))
        return rc;
    return hip_status(fn, swa::launch_debug_prefill_mask(mask, L, Hq, Hkv, d, w_loc, s,
                                                         static_cast<hipStream_t>(stream)));
}

int swa_debug_decode_slots(int64_t *slot_pos, const int64_t *pos, int B, int w, int s, int conv, void *stream)
{
    const char *fn = "swa_debug_decode_slots";
    if (slot_pos == nullptr || pos == nullptr)
        return fail(SWA_EINVAL, "%s: null pointer", fn);
    if (B < 1)
        return fail(SWA_EINVAL, "%s: B must be >= 1", fn);
    int w_loc = 0;
    int rc = resolve_window(fn, w, s, conv, &w_loc);
    if (rc)
        return rc;
    return hip_status(fn, swa::launch_debug_decode_slots(slot_pos, pos, B, w_loc, s,
                                                         static_cast<hipStream_t>(stream)));
}

int swa_rmsnorm(const float *x, const void *weight, void *out, int B, int n, float eps, void *stream)
{
    const char *fn = "swa_rmsnorm";
    CHECK_PTR(x);
    CHECK_PTR(weight);
    CHECK_PTR(out);
    if (B < 1 || n < 4 || n % 4 != 0)
        return fail(SWA_EINVAL, "%s: need B >= 1 and n a positive multiple of 4 (got %d, %d)", fn, B, n);
    int rc = check_eps(fn, eps);
    if (rc)
        return rc;
    return hip_status(fn, swa::launch_rmsnorm(x, weight, out, B, n, eps, static_cast<hipStream_t>(stream)));
}

int swa_linear(const void *W, const void *x, int x_f32, void *out, int mode, int B, int N, int K, void *stream)
{
    const char *fn = "swa_linear";
    CHECK_PTR(W);
    CHECK_PTR(x);
    CHECK_PTR(out);
    if (mode != SWA_LINEAR_STORE && mode != SWA_LINEAR_ADD && mode != SWA_LINEAR_SILU_MUL)
        return fail(SWA_EINVAL, "%s: unknown mode %d", fn, mode);
    if (B < 1 || N < 1 || K < 8 || K % 8 != 0)
        return fail(SWA_EINVAL, "%s: need B, N >= 1 and K a positive multiple of 8 (got %d, %d, %d)", fn, B, N, K);
    if (N > (1 << 28) || K > (1 << 28) || (long long)B * (N > K ? N : K) > 0x7fffffffLL)
        return fail(SWA_EUNSUPPORTED, "%s: sizes exceed the supported range", fn);
    void *outs[3] = {out, out, out};
    const int seg[4] = {0, N, N, N};
    const int m = mode == SWA_LINEAR_STORE ? swa::LIN_STORE : mode == SWA_LINEAR_ADD ? swa::LIN_ADD : swa::LIN_SILU_MUL;
    return hip_status(fn, swa::launch_linear(m, x_f32 != 0, W, x, B, N, K, outs, seg, static_cast<float *>(out),
                                             static_cast<hipStream_t>(stream)));
}

size_t swa_layer_workspace_bytes(int B, int dm, int Hq, int Hkv, int d, int f, int w, int s, int conv)
{
    const char *fn = "swa_layer_workspace_bytes";
    if (check_layer_dims(fn, B, dm, Hq, Hkv, d, f) || check_decode_batch(fn, B))
        return 0;
    int w_loc = 0;
    if (resolve_window(fn, w, s, conv, &w_loc) || check_cache(fn, s, w_loc, d))
        return 0;
    return layer_workspace(B, dm, Hq, Hkv, d, f, swa::decode_plan(B, Hq, Hkv, d, w_loc, s).workspace_bytes).total;
}

int swa_layer_decode_step(float *x, const swa_layer_weights *wts, void *k_cache, void *v_cache, const int64_t *pos,
                          int B, int dm, int Hq, int Hkv, int d, int f, int w, int s, float scale, int conv, float eps,
                          void *workspace, size_t workspace_bytes, void *stream)
{
    const char *fn = "swa_layer_decode_step";
    CHECK_PTR(x);
    CHECK_PTR(workspace);
    if (pos == nullptr)
        return fail(SWA_EINVAL, "%s: pos is null", fn);
    int w_loc = 0, rc;
    size_t need = 0;
    if ((rc = check_layer(fn, wts, k_cache, v_cache, B, dm, Hq, Hkv, d, f, w, s, conv, &w_loc, &need)))
        return rc;
    if ((rc = check_scale(fn, scale)) || (rc = check_eps(fn, eps)))
        return rc;
    if (workspace_bytes < need)
        return fail(SWA_EINVAL, "%s: workspace of %zu bytes needed, %zu given", fn, need, workspace_bytes);
    return hip_status(fn, run_layer(x, wts, k_cache, v_cache, pos, B, dm, Hq, Hkv, d, f, w_loc, s, scale, eps,
                                    static_cast<char *>(workspace), static_cast<hipStream_t>(stream)));
}

size_t swa_stack_workspace_bytes(int n_layers, const int *w, const int *s, const int *conv, int B, int dm, int Hq,
                                 int Hkv, int d, int f)
{
    const char *fn = "swa_stack_workspace_bytes";
    if (n_layers < 1 || w == nullptr || s == nullptr || conv == nullptr) {
        fail(SWA_EINVAL, "%s: n_layers must be >= 1 and w, s, conv non-null", fn);
        return 0;
    }
    size_t most = 0;
    for (int i = 0; i < n_layers; ++i) {
        const size_t need = swa_layer_workspace_bytes(B, dm, Hq, Hkv, d, f, w[i], s[i], conv[i]);
        if (need == 0)
            return 0;
        most = need > most ? need : most;
    }
    return most;
}

int swa_stack_decode_step(float *x, int n_layers, const swa_layer_weights *wts, void *const *k_caches,
                          void *const *v_caches, const int *w, const int *s, const int *conv, const int64_t *pos,
                          int B, int dm, int Hq, int Hkv, int d, int f, float scale, float eps, void *workspace,
                          size_t workspace_bytes, void *stream)
{
    const char *fn = "swa_stack_decode_step";
    CHECK_PTR(x);
    CHECK_PTR(workspace);
    if (pos == nullptr)
        return fail(SWA_EINVAL, "%s: pos is null", fn);
    if (n_layers < 1)
        return fail(SWA_EINVAL, "%s: n_layers must be >= 1 (got %d)", fn, n_layers);
    if (wts == nullptr || k_caches == nullptr || v_caches == nullptr || w == nullptr || s == nullptr || conv == nullptr)
        return fail(SWA_EINVAL, "%s: a per-layer array is null", fn);
    int rc;
    if ((rc = check_scale(fn, scale)) || (rc = check_eps(fn, eps)))
        return rc;
    // Every layer is checked before the first launch, so an invalid layer leaves x and every
    // cache untouched.
    std::vector<int> w_loc(n_layers);
    for (int i = 0; i < n_layers; ++i) {
        size_t need = 0;
        if ((rc = check_layer(fn, &wts[i], k_caches[i], v_caches[i], B, dm, Hq, Hkv, d, f, w[i], s[i], conv[i],
                              &w_loc[i], &need)))
        {
            const std::string what = g_last_error;
            return fail(rc, "%s (layer %d)", what.c_str(), i);
        }
        if (workspace_bytes < need)
            return fail(SWA_EINVAL, "%s: workspace of %zu bytes needed (layer %d), %zu given", fn, need, i,
                        workspace_bytes);
    }
    const hipStream_t st = static_cast<hipStream_t>(stream);
    for (int i = 0; i < n_layers; ++i) {
        const hipError_t e = run_layer(x, &wts[i], k_caches[i], v_caches[i], pos, B, dm, Hq, Hkv, d, f, w_loc[i],
                                       s[i], scale, eps, static_cast<char *>(workspace), st);
        if (e != hipSuccess)
            return hip_status(fn, e);
    }
    return ok();
}

}  // extern "C"
