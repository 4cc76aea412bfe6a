/*
 * swa.h -- C ABI of libswa.so: SWA(w,s) causal softmax attention on MI355X (gfx950).
 *
 * SWA(w,s): query t attends to the keys at positions max(0, t-w_loc+1) .. t (the
 * w_loc most recent tokens, itself included) together with the first s positions
 * ("attention sinks"), restricted to positions <= t, with a softmax taken over that
 * allowed set only.  Sources: page "滑动窗口注意力（SWA）配 sinks 比 post-training
 * 线性注意力更划算" (papers.ananclaw.com explainer of arXiv 2608.28444), section
 * 核心方法 1 (the notation paragraph, the x_t equation and the swa_mask recipe);
 * page "从长文档摘要说起：为什么注意力范围成了瓶颈" (wiblog.cn), section "SWA 的核心机制"
 * (token i sees i-W+1 .. i).
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library never
 *     allocates, frees or synchronises.  Work is enqueued on `stream` (a hipStream_t;
 *     NULL means the null stream) and runs asynchronously.
 *   - bf16 means IEEE bfloat16 stored as 16-bit words; all tensors are dense,
 *     row-major (last index fastest) and 16-byte aligned.
 *   - Arguments are validated on the host before any HIP call.  A non-zero return
 *     leaves the device untouched (for SWA_EINVAL / SWA_EUNSUPPORTED) and sets a
 *     thread-local message readable with swa_last_error().
 *   - Window convention `conv`: SWA_CONV_ADDITIVE gives w_loc = w (w recent keys plus
 *     s sinks, the "64+4=68 tokens" reading of the first page's deployment notes);
 *     SWA_CONV_TOTAL gives w_loc = w - s (a total window of w that includes the sinks,
 *     as the PaperWeekly page "几亿Token白练了？" phrases SWA(64,4)).  w_loc must be >= 1.
 *   - Grouped-query attention: Hq % Hkv == 0 and q-head h reads kv-head h / (Hq/Hkv).
 *   - Supported head dimensions: d = 64 and d = 128 (others give SWA_EUNSUPPORTED).
 *   - Every call that takes a sink+ring cache (swa_kv_append, the decode steps, the chunked
 *     prefill, the layer and stack steps and their workspace queries) gives SWA_EUNSUPPORTED
 *     when one (sequence, kv-head) cache, (s + w_loc) * d * 2 bytes, exceeds 2^31 - 1 bytes
 *     (more than 8,388,607 slots at d = 128): the kernels address it with 32-bit offsets.
 */
#ifndef SWA_H
#define SWA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define SWA_OK 0
#define SWA_EINVAL (-1)        /* bad argument (null/misaligned pointer, bad size...) */
#define SWA_EUNSUPPORTED (-2)  /* valid request the library does not implement (d, sizes) */
#define SWA_EHIP (-3)          /* the HIP runtime reported an error at launch */

/* Window conventions. */
#define SWA_CONV_ADDITIVE 0
#define SWA_CONV_TOTAL 1

/*
 * swa_prefill -- SWA(w,s) attention over whole sequences.
 *
 * Operation: for every batch b, position t < L and q-head h,
 *   out[b][t][h][:] = sum_{i in A(t)} softmax_i(scale * <q[b][t][h], k[b][i][g(h)]>)
 *                     * v[b][i][g(h)][:]
 * with A(t) = { i <= t : i >= t - w_loc + 1 or i < s } and g(h) = h / (Hq/Hkv).
 * Defined by the first page's x_t equation and swa_mask recipe (section 核心方法 1),
 * with the readings stated above.  The computation visits only key tiles that meet
 * A(t) for some query of a tile, the tile skipping described on page "Hybrid Sliding
 * Window Attention" (bittide), section 三.3 (FlashAttention-2/3 window support).
 *
 *   q    bf16 [B][L][Hq][d]     (in)
 *   k    bf16 [B][L][Hkv][d]    (in)
 *   v    bf16 [B][L][Hkv][d]    (in)
 *   out  fp32 [B][L][Hq][d]     (out; every element written)
 *   scale  logit multiplier (1/sqrt(d) in the x_t equation); finite and > 0.
 * Arithmetic: bf16 products with fp32 accumulation, fp32 softmax, probabilities
 * rounded to bf16 for the value product.
 * Errors: SWA_EINVAL for null or non-16-byte-aligned pointers, B, L, Hq, Hkv < 1,
 * Hq % Hkv != 0, w < 1, s < 0, unknown conv, w_loc < 1, non-finite or non-positive
 * scale; SWA_EUNSUPPORTED for d not in {64, 128}, a sequence of more than 2^31 - 1
 * elements in q or out, or Hq * d >= 2^22; SWA_EHIP if the launch fails.
 */
int swa_prefill(const void *q, const void *k, const void *v, float *out, int B, int Hq, int Hkv,
                int L, int d, int w, int s, float scale, int conv, void *stream);

/*
 * swa_prefill_timed -- swa_prefill that also stamps two caller-created HIP events
 * (hipEvent_t, created with timing enabled) with the start and the end of the prefill
 * kernel itself (hipExtLaunchKernel), for callers that time the kernel rather than the
 * stream interval around it.  Same arguments, layout and errors as swa_prefill, plus
 * SWA_EINVAL if either event is null.
 */
int swa_prefill_timed(const void *q, const void *k, const void *v, float *out, int B, int Hq, int Hkv,
                      int L, int d, int w, int s, float scale, int conv, void *stream,
                      void *start_event, void *stop_event);

/*
 * swa_prefill_describe -- what swa_prefill launches for a shape (host only, no GPU call): the
 * kernel form, its tile geometry and the work its matrix cores do.
 *
 *   form            0: the tile walk (64-key tiles; edge tiles masked, middle tiles unmasked);
 *                   1: resident (every 32-key chunk a q-tile needs held in LDS at once, at most
 *                      four: Tm/32 + ceil((w_loc-1)/32) + ceil(s/32) <= 4 for Tm-token q-tiles);
 *                   2: resident with 64-row workgroups (Tm/32 read as 1 for 16-token q-tiles),
 *                      launched where form 1 does not apply or would start fewer than 512
 *                      workgroups;
 *                   3: the tile walk with 64-row workgroups, launched instead of 0 where form 0
 *                      would start at most 256 workgroups (one per CU)
 *   tokens_per_tile query tokens per workgroup; heads_per_tile q-heads per workgroup
 *   workgroups      grid size
 *   executed_pairs  (query row, key) pairs whose scores and value products the matrix cores
 *                   compute, padding rows and masked keys included (each costs 4 d flops)
 * Errors: as swa_prefill for the sizes, window and convention; SWA_EINVAL for a null info.
 */
typedef struct swa_prefill_info {
    int form;
    int tokens_per_tile;
    int heads_per_tile;
    long long workgroups;
    long long executed_pairs;
} swa_prefill_info;
int swa_prefill_describe(int B, int Hq, int Hkv, int L, int d, int w, int s, int conv, swa_prefill_info *info);

/*
 * swa_kv_append -- write new tokens' keys and values into the bounded decode cache.
 *
 * Cache layout (per batch b and kv-head): s pinned sink slots followed by a ring of
 * w_loc slots, i.e. k_cache / v_cache are bf16 [B][Hkv][s + w_loc][d].  Position p goes
 * to slot p when p < s, else to slot s + (p mod w_loc), replacing the oldest ring entry.
 * The rotation (evict the oldest, circular buffer addressed modulo the window) is the
 * one on page "从长文档摘要说起" (wiblog.cn), section "与 KV Cache 的配合：轮转替换策略";
 * the pinned sinks follow the first page's deployment notes (64+4=68 tokens kept).
 *
 *   k_new, v_new  bf16 [B][n_new][Hkv][d]   (in) tokens at positions pos[b] .. pos[b]+n_new-1
 *   pos           int64 [B] device          (in) absolute position of k_new[b][0]
 * When n_new > w_loc only the positions that survive the call are written (the sinks
 * and the last w_loc positions), so every slot is written at most once.  Negative
 * positions are skipped (nothing written).
 * Errors: as swa_prefill, plus SWA_EINVAL for n_new < 1 or a null pos.
 */
int swa_kv_append(void *k_cache, void *v_cache, const void *k_new, const void *v_new,
                  const int64_t *pos, int B, int Hkv, int d, int w, int s, int n_new, int conv,
                  void *stream);

/*
 * swa_cache_slots -- slots per (sequence, kv-head) of the bounded decode cache: s + w_loc, with
 * w_loc = w (SWA_CONV_ADDITIVE) or w - s (SWA_CONV_TOTAL).  Returns -1 (and sets the message)
 * for w < 1, s < 0, an unknown conv or w_loc < 1.
 */
long long swa_cache_slots(int w, int s, int conv);

/*
 * swa_decode_workspace_bytes -- device workspace that swa_decode_step needs for this
 * shape (0 when the step runs without a split).  Returns 0 for invalid arguments too.
 */
size_t swa_decode_workspace_bytes(int B, int Hq, int Hkv, int d, int w, int s, int conv);

/*
 * swa_decode_describe -- how swa_decode_step / swa_append_decode_step split a shape (host only):
 *   splits               slot segments per (sequence, kv-head, head slice)
 *   waves_per_workgroup  1, or the splits of one workgroup merged in LDS (2-4 waves, one 32-slot
 *                        chunk each, when s + w_loc spans 2-4 chunks)
 *   slots_per_split      slots of a segment (at most 96 for one wave)
 *   heads_per_wave       q-heads sharing a kv-head taken as the MFMA columns of one wave (<= 16)
 *   workgroups           grid size of the attend kernel
 *   merge_launch         1 when a second kernel merges workgroup splits through the workspace
 *   workspace_bytes      as swa_decode_workspace_bytes
 * Errors: as swa_decode_step for the sizes, window and convention; SWA_EINVAL for a null info.
 */
typedef struct swa_decode_info {
    int splits;
    int waves_per_workgroup;
    int slots_per_split;
    int heads_per_wave;
    long long workgroups;
    int merge_launch;
    size_t workspace_bytes;
} swa_decode_info;
int swa_decode_describe(int B, int Hq, int Hkv, int d, int w, int s, int conv, swa_decode_info *info);

/*
 * swa_decode_step -- one-token GQA decode over the bounded cache.
 *
 * For each batch b with query position t = pos[b] (already appended with
 * swa_kv_append), out[b][h] is the SWA(w,s) attention row t of q[b][h] over the cache:
 * the sinks 0 .. min(s, t+1)-1 and the ring slots holding positions
 * max(s, t-w_loc+1) .. t.  Slot validity is derived from t alone: a slot that holds no
 * position of A(t) (never written yet, or stale from earlier use of the cache) contributes
 * nothing, whatever bytes it holds.  The cache is read in storage order; the softmax sum
 * does not depend on order.  When s + w_loc exceeds 96 slots the slot range is split over
 * workgroups and the partial (max, sum, weighted values) are merged in a fixed order.
 *
 *   q          bf16 [B][Hq][d]   (in)
 *   k_cache,   bf16 [B][Hkv][s + w_loc][d] (in)
 *   v_cache
 *   out        fp32 [B][Hq][d]   (out)
 *   pos        int64 [B] device  (in)  must be >= 0
 *   workspace  device scratch of at least swa_decode_workspace_bytes(...) bytes, or
 *              NULL when that is 0; contents on entry are ignored.
 * Errors: as swa_prefill, plus SWA_EINVAL for a too-small workspace and SWA_EUNSUPPORTED
 * for B above 65535 (the launch grid indexes sequences by a dimension of at most 65535
 * blocks).  Concurrent calls that share a workspace must be ordered by the caller.
 */
int swa_decode_step(const void *q, const void *k_cache, const void *v_cache, float *out,
                    const int64_t *pos, int B, int Hq, int Hkv, int d, int w, int s, float scale,
                    int conv, void *workspace, size_t workspace_bytes, void *stream);

/*
 * swa_decode_step_noalloc -- swa_decode_step without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, allocation-free serving loops,
 * harnesses that forbid hipMalloc).  When the shape needs a workspace (s + w_loc > 128 slots:
 * partial (max, sum, weighted values) per split), a static device array of 8 MiB inside the
 * library serves as one; the library takes its address once per device (on the first call with
 * that device current) and never allocates or frees anything.  Every partial is written before
 * it is read within one call, so nothing needs clearing between calls.
 *
 * Same arguments, layout and results as swa_decode_step without workspace/workspace_bytes; runs
 * on the current device's copy of the scratch (the stream must belong to the current device).
 * Every call on one GPU shares that copy: calls whose work overlaps on one GPU (different
 * streams, or different threads without ordering) race and must be ordered by the caller.
 * Errors: as swa_decode_step; SWA_EUNSUPPORTED when the shape needs more scratch than 8 MiB
 * (B * Hq * splits * (d + 2) * 4 bytes, see swa_decode_describe); SWA_EHIP if the scratch
 * address cannot be obtained or the launch fails.
 */
int swa_decode_step_noalloc(const void *q, const void *k_cache, const void *v_cache, float *out,
                            const int64_t *pos, int B, int Hq, int Hkv, int d, int w, int s, float scale,
                            int conv, void *stream);

/*
 * swa_append_decode_step -- swa_kv_append of one token per sequence followed by
 * swa_decode_step, in one launch.  The new token k_new[b], v_new[b] (bf16 [B][Hkv][d], the
 * token at position pos[b]) is written to its slot and attended directly from k_new/v_new;
 * every other slot is read from the cache.  Results, and the cache contents afterwards, are
 * identical to the two-call sequence.  Same arguments and errors as swa_decode_step, plus
 * SWA_EINVAL for null or misaligned k_new / v_new.  The caches are written.
 */
int swa_append_decode_step(const void *q, void *k_cache, void *v_cache, const void *k_new,
                           const void *v_new, float *out, const int64_t *pos, int B, int Hq,
                           int Hkv, int d, int w, int s, float scale, int conv, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * swa_append_decode_step_timed -- swa_append_decode_step whose kernel dispatches also stamp two
 * caller-created HIP events (hipEvent_t, timing enabled) with the start of the step's first
 * kernel and the end of its last one (hipExtLaunchKernel), for callers that time the kernels
 * rather than the stream interval around them.  Same arguments, layout and errors as
 * swa_append_decode_step, plus SWA_EINVAL if either event is null.
 */
int swa_append_decode_step_timed(const void *q, void *k_cache, void *v_cache, const void *k_new,
                                 const void *v_new, float *out, const int64_t *pos, int B, int Hq,
                                 int Hkv, int d, int w, int s, float scale, int conv, void *workspace,
                                 size_t workspace_bytes, void *stream, void *start_event, void *stop_event);

/*
 * swa_prefill_chunk -- prefill of one prompt chunk against the bounded cache, then the chunk
 * appended to it: the long-prompt procedure of page "从长文档摘要说起" (wiblog.cn), section
 * "长 Prompt 的分块处理与工程实现" and its flow description (a long input is processed in
 * consecutive chunks, each attending within the window, with the cache rotating between chunks
 * so that only the window's keys stay cached).
 *
 * The cache holds the state after position pos0 - 1 (every sequence at the same position).
 * For each b and i < C, out[b][i][h] is the SWA(w,s) attention row pos0 + i of q[b][i][h] over
 * the sinks and window keys in the cache and the chunk's own keys pos0 .. pos0 + i: the same
 * row a whole-sequence swa_prefill gives.  Afterwards the cache holds the state after
 * pos0 + C - 1 (as swa_kv_append of the chunk would leave it).  Any C >= 1 works (the pages
 * keep chunks within the window; larger chunks are fine here).
 *
 *   q           bf16 [B][C][Hq][d]   (in)   the chunk's queries
 *   k, v        bf16 [B][C][Hkv][d]  (in)   the chunk's keys and values
 *   k_cache,    bf16 [B][Hkv][s + w_loc][d] (in/out), the layout swa_kv_append writes
 *   v_cache
 *   out         fp32 [B][C][Hq][d]   (out)
 *   lse         fp32 [B][C][Hq] (out) or NULL: ln sum_{i in A(t)} exp(scale <q_t, k_i>) of each row,
 *               the log of its softmax denominator (for callers that merge partial attention
 *               results); the probabilities are summed as they weight V (bf16), so it carries
 *               their rounding (~2^-9 relative in the sum)
 *   pos0        position of the chunk's first token, >= 0 (host value)
 * Two launches on `stream` (attend, reading the cached keys in place; then append); no
 * workspace, no synchronisation.
 * Errors: as swa_prefill, plus SWA_EINVAL for C < 1, pos0 < 0 or a non-16-byte-aligned lse;
 * SWA_EUNSUPPORTED when
 * s + w_loc + 30 + C key rows (the cached and the chunk's keys, plus up to 31 padding rows), or the
 * C query rows, of one sequence exceed 2^31-1 elements.
 */
int swa_prefill_chunk(const void *q, const void *k, const void *v, void *k_cache, void *v_cache,
                      float *out, float *lse, int64_t pos0, int B, int Hq, int Hkv, int C, int d, int w,
                      int s, float scale, int conv, void *stream);

/*
 * Decoder-layer decode step around SWA(w,s) attention, for the multi-layer decode
 * measurement of page "几亿Token白练了？微软实测：免训练滑动窗口，让线性注意力破防" (PaperWeekly)
 * (section "小窗口也有工程优势": decode throughput and state memory of a 4-layer Transformer
 * at batch 1 from 128 to 256K tokens of context).  The pages fix no layer recipe; this is the
 * standard pre-norm layer, with activations stored in bf16 where noted:
 *
 *   h = bf16(rmsnorm(x) * attn_norm);  q | k_new | v_new = bf16(w_qkv h)
 *   o = SWA(w,s) decode of q at pos[b] after appending (k_new, v_new) there (as
 *       swa_append_decode_step, on this layer's cache)
 *   x += w_o bf16(o);  h = bf16(rmsnorm(x) * mlp_norm)
 *   x += w_down bf16(silu(gate) * up),  gate | up = w_gate_up h
 *
 * with rmsnorm(x) = x / sqrt(mean(x^2) + eps), silu(z) = z / (1 + e^-z); no positional
 * encoding, no output head.  All pointers are device memory owned by the caller; every call
 * is asynchronous on `stream`; nothing is allocated.
 */
enum { SWA_LINEAR_STORE = 0, SWA_LINEAR_ADD = 1, SWA_LINEAR_SILU_MUL = 2 };

typedef struct swa_layer_weights {
    const void *attn_norm;  /* bf16 [dm] */
    const void *w_qkv;      /* bf16 [(Hq + 2 Hkv) d][dm]: q rows (head-major), then k, then v */
    const void *w_o;        /* bf16 [dm][Hq d] */
    const void *mlp_norm;   /* bf16 [dm] */
    const void *w_gate_up;  /* bf16 [2 f][dm]: gate rows, then up rows */
    const void *w_down;     /* bf16 [dm][f] */
} swa_layer_weights;

/* out bf16 [B][n] = bf16(x / sqrt(mean(x^2) + eps) * weight); x fp32 [B][n], weight bf16 [n].
 * Errors: SWA_EINVAL for null or unaligned pointers, B < 1, n not a positive multiple of 4,
 * eps negative or not finite. */
int swa_rmsnorm(const float *x, const void *weight, void *out, int B, int n, float eps, void *stream);

/* y[b][n] = sum_k W[n][k] x[b][k], fp32 accumulation, for x [B][K] bf16 (x_f32 = 0) or fp32
 * rounded to bf16 as it is read (x_f32 != 0); K % 8 == 0.
 *   SWA_LINEAR_STORE     W bf16 [N][K]; out bf16 [B][N] = bf16(y)
 *   SWA_LINEAR_ADD       W bf16 [N][K]; out fp32 [B][N] += y
 *   SWA_LINEAR_SILU_MUL  W bf16 [2N][K] (gate rows, then up rows); out bf16 [B][N] = bf16(silu(g) u)
 * Errors: SWA_EINVAL for null or unaligned pointers, an unknown mode, B or N < 1, K not a
 * positive multiple of 8; SWA_EUNSUPPORTED for N or K above 2^28. */
int swa_linear(const void *W, const void *x, int x_f32, void *out, int mode, int B, int N, int K,
               void *stream);

/* Workspace bytes swa_layer_decode_step needs (0 for invalid arguments). */
size_t swa_layer_workspace_bytes(int B, int dm, int Hq, int Hkv, int d, int f, int w, int s, int conv);

/* One decode step of one layer for B sequences:
 *   x        fp32 [B][dm] residual stream (in/out, updated in place)
 *   wts      the layer's weights (host struct of device pointers, each 16-byte aligned)
 *   k_cache, bf16 [B][Hkv][s + w_loc][d] (in/out): this layer's sink + ring cache, the layout
 *   v_cache  swa_kv_append writes; the step appends its token at pos[b]
 *   pos      int64 [B] device: position of this step's token
 * dm, f % 8 == 0; d in {64, 128}.  Seven launches on `stream`.
 * Errors: as swa_append_decode_step and swa_linear, plus SWA_EINVAL for a workspace smaller
 * than swa_layer_workspace_bytes. */
int swa_layer_decode_step(float *x, const swa_layer_weights *wts, void *k_cache, void *v_cache,
                          const int64_t *pos, int B, int dm, int Hq, int Hkv, int d, int f, int w, int s,
                          float scale, int conv, float eps, void *workspace, size_t workspace_bytes,
                          void *stream);

/*
 * Hybrid stacks: decoder layers whose attention windows differ, SWA layers interleaved with
 * global layers at a fixed ratio (page "Hybrid Sliding Window Attention (Hybrid SWA)", section
 * 一.2, the design mechanism; the same page's note on caches: a rolling cache for the SWA layers,
 * a growing one for the global layers).  A global layer is a window at least as long as the
 * context with s = 0: its ring then holds every position (swa_cache_slots gives its slots).
 *
 * swa_stack_workspace_bytes -- the workspace swa_stack_decode_step needs: the largest of the
 * layers' swa_layer_workspace_bytes (the layers run one after another on one stream and share
 * it).  w, s, conv: host int [n_layers].  0 for invalid arguments.
 *
 * swa_stack_decode_step -- one decode step through n_layers layers for B sequences: layer i is
 * swa_layer_decode_step with weights wts[i], cache k_caches[i] / v_caches[i] (bf16
 * [B][Hkv][s[i] + w_loc(i)][d] each) and window (w[i], s[i], conv[i]); x fp32 [B][dm] is the
 * residual stream in and out, pos int64 [B] device the step's positions.  wts, k_caches,
 * v_caches, w, s, conv are host arrays of n_layers entries (the cache pointers are device
 * addresses).  7 n_layers launches on `stream`.
 * Errors: SWA_EINVAL for n_layers < 1 or a null array; for a layer that swa_layer_decode_step
 * would reject, the code it would return (the message names the layer); every layer is checked
 * before the first launch, so on an error x and the caches are untouched.  SWA_EHIP if a launch
 * fails.
 */
size_t swa_stack_workspace_bytes(int n_layers, const int *w, const int *s, const int *conv, int B, int dm, int Hq,
                                 int Hkv, int d, int f);
int swa_stack_decode_step(float *x, int n_layers, const swa_layer_weights *wts, void *const *k_caches,
                          void *const *v_caches, const int *w, const int *s, const int *conv, const int64_t *pos,
                          int B, int dm, int Hq, int Hkv, int d, int f, float scale, float eps, void *workspace,
                          size_t workspace_bytes, void *stream);

/* Message for the last non-OK return on the calling thread ("" if none). */
const char *swa_last_error(void);

/*
 * Test hooks: the index sets the kernels attend to, derived by the kernels' own device
 * functions (walks, slot maps and admission tests shared with the hot kernels).
 *
 * swa_debug_prefill_mask: mask uint8 [L][L] device (out).  mask[t][i] counts how often the
 * prefill kernel that swa_prefill launches for (L, Hq, Hkv, d, w, s, conv) attends to the key
 * held at position i for query t: the same form and q-tile geometry (swa_prefill_describe), the
 * same tile or chunk walk, mask-free classification and element predicate, and (resident form)
 * the key each LDS chunk slot actually holds.  A
 * correct kernel gives 1 on A(t) and 0 elsewhere.  Requires L <= 8192.
 *
 * swa_debug_decode_slots: slot_pos int64 [B][s + w_loc] device (out).  For every split segment
 * of the decode plan, each slot goes through the decode kernel's admission test (once the ring
 * has wrapped, every slot of the segment; before, the 32-bit validity test from t alone);
 * slot_pos[b][j] = the position slot j holds for query position pos[b] if admitted (position
 * pos[b] at the slot the fused append+decode step writes), else -1.  -2 marks an admitted slot
 * holding no position of A(pos[b]), -3 a slot covered by two split segments (neither occurs in
 * a correct kernel).
 */
int swa_debug_prefill_mask(uint8_t *mask, int L, int Hq, int Hkv, int d, int w, int s, int conv,
                           void *stream);
int swa_debug_decode_slots(int64_t *slot_pos, const int64_t *pos, int B, int w, int s, int conv,
                           void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SWA_H */
