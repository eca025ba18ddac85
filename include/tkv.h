/*
 * tkv.h -- C ABI of the tiered KV-cache decode hot path (libtkv.so, gfx950).
 *
 * The method: the technical summary pages of "Not All Thoughts Need HBM"
 * (gist.science, paper 2605.09490; the French page's section names are used
 * below).  A reasoning model's KV cache is split into four tiers by a cumulative
 * attention-importance score: T0 in HBM (protected prompt, sink and recent
 * tokens plus the most important ones), T1 in host DDR at full precision and
 * brought to the GPU before each attention step, T2 on the host at 8 bits, and
 * T3 dropped (Methodologie section 1).  The score adds, every decode step, the
 * attention weight each position receives averaged over heads and layers
 * (Methodologie section 2).  Tiers are recomputed every Delta = 64 steps
 * (Methodologie section 4).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every function returns tkv_status: TKV_OK (0) or a negative code.  On a
 *   negative code nothing has been enqueued, except TKV_ERR_HIP from a failed
 *   launch or copy; tkv_last_error() then holds a message (thread-local).
 * - Arguments are validated before any HIP call.  Device-resident contents
 *   (tier maps, slot maps) cannot be validated from the host; where a kernel
 *   detects a bad state it reports it through its count outputs (documented
 *   per call) and leaves its other outputs unspecified.
 * - The caller owns every buffer.  The library allocates no caller-visible
 *   memory and keeps no pointer after it returns.  Device buffers must stay
 *   alive until the stream has passed the call.
 * - All device work is asynchronous on the caller's stream.  Per-sequence
 *   lengths arrive as HOST int32 arrays so that grids are sized without a sync.
 * - Key/value/query elements are bf16 bit patterns (uint16) when
 *   kv_dtype == TKV_BF16, or float32 when kv_dtype == TKV_F32.
 * - Layouts are row-major; "[B][L][Hkv][D]" means D is contiguous.
 *   Key and value pools, windows and staging ("[B][L][Hkv][cap][D] tiles") hold
 *   the same elements in the order the matrix-core products consume them:
 *   each (sequence, layer, KV head) block of cap slots is cut into 32-slot
 *   blocks of 32*D elements, and element (slot, d) of a block sits at
 *     keys   (K-tiles): (slot/32)*32*D + u*16*D + ((d/8)*16 + row)*8 + d%8,
 *            with r = slot%32, u = (r/4)%2, row = 4*(r/8) + r%4;
 *     values (V-tiles): (slot/32)*32*D + ((d/16)*4 + r/8)*128 + (d%16)*8 + r%8.
 *   With it every operand load of the attention kernel is one contiguous
 *   1 KB wave access.  The optional int8 T2 pool uses the same element order at
 *   one byte per element.  Capacities (cap0, cap1, cap2) must be multiples of 32.
 *   Per sequence, the T0 pool holds the T0 positions in slots [0, t0_len) and
 *   the T1 window holds the T1 positions in slots [0, t1_len), in any order:
 *   the slot -> position maps t0_pos / t1_pos [B][cap] say which position a
 *   slot holds (an appended token takes slot t0_len; tkv_compact fills the
 *   holes a reassignment leaves).  The "attended index" j of a sequence runs
 *   over T0 slots then T1 slots: j < t0_len is T0 slot j, otherwise T1 slot
 *   j - t0_len; the _t2 calls continue with the T2 slots after T1.
 * - Query head h reads KV head h / (Hq / Hkv) (contiguous grouping).
 * - Supported shapes: head_dim 64 or 128; 1 <= Hq / Hkv <= 16.
 * - Calls on one stream are ordered; calls that write the same buffers on
 *   different streams race.  The library itself holds no mutable global state
 *   apart from the optional kernel timers (tkv_timing_*), which are meant for
 *   benchmarks and are not thread-safe.
 */
#ifndef TKV_H
#define TKV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t tkv_status;
#define TKV_OK 0
#define TKV_ERR_ARG (-1)      /* null pointer, bad shape, bad fraction, bad order */
#define TKV_ERR_CAPACITY (-2) /* a length above its capacity, workspace too small */
#define TKV_ERR_STATE (-3)    /* inconsistent lengths / maps detected on the host */
#define TKV_ERR_HIP (-4)      /* a HIP runtime call failed; see tkv_last_error() */

#define TKV_BF16 0
#define TKV_F32 1

#define TKV_ABI_VERSION 4

/* Model shape.  softmax_scale <= 0 selects 1/sqrt(head_dim).
 * alpha_scratch (0 or 1): with 1 the decode calls use their alpha buffer as
 * scratch only -- it is left holding the raw base-2 logits, the normalised
 * weights are never stored -- for callers that need the weights only through the
 * importance score (Methodologie section 2 consumes them as a per-position sum
 * over heads and layers, which the fused score update still adds exactly as with
 * 0).  Each step then writes the weights once (the logits) instead of twice.
 *
 * t0_caps, t1_caps (optional host arrays over the batch of every call, or null):
 * per-sequence capacities of the T0 pool and of the device T1 window, so that a
 * batch of sequences of different lengths does not pad every sequence to the
 * longest one's budget (Importance et revendications section 1: HBM holds only
 * what the tiers need).  With t0_caps, sequence b's T0 block holds t0_caps[b]
 * slots per (layer, KV head) (a multiple of 32, at most cap0) and the blocks are
 * packed in sequence order: sequence b's block starts L * Hkv * (t0_caps[0] + ...
 * + t0_caps[b-1]) slots of D elements after the start of k_t0 / v_t0, laid out
 * [L][Hkv][t0_caps[b]][D] tiles.  t1_caps likewise for k_t1 / v_t1 (the device T1
 * window; not the host-resident T1 of tkv_compact_host_t1 / the streamed calls).
 * Null: cap0 (cap1) slots for every sequence, [B][L][Hkv][cap][D].  The calls' cap0
 * / cap1 arguments stay the strides of the slot -> position maps and of the
 * workspaces; lengths are checked against the per-sequence capacities. */
typedef struct {
  int32_t num_layers;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t kv_dtype; /* TKV_BF16 or TKV_F32 */
  float softmax_scale;
  int32_t alpha_scratch;
  const int32_t* t0_caps;
  const int32_t* t1_caps;
} tkv_model;

/* Tier policy (Methodologie sections 1 and 4).  The fractions are of the
 * current length n: N_k = floor((double)frac_tk * n) for k = 1, 2, 3 and T0
 * takes the rest.  Protected positions: [0, max(prompt_len, num_sinks)) and
 * the last recent_window positions. */
typedef struct {
  int32_t prompt_len;
  int32_t num_sinks;
  int32_t recent_window;
  float frac_t1;
  float frac_t2;
  float frac_t3;
  int32_t delta;
} tkv_policy;

int32_t tkv_abi_version(void);
/* Message of the last failure on this thread ("" if none). */
const char* tkv_last_error(void);

/*
 * tkv_append -- every generated token adds one key/value pair, which enters T0
 * (Enonce du probleme; Methodologie section 1: the recent window is in T0).
 *
 * k_new, v_new : device [B][L][Hkv][D]
 * k_t0, v_t0   : device T0 pools [B][L][Hkv][cap0][D] tiles (or per-sequence
 *                capacities, tkv_model.t0_caps); slot t0_len[b]
 *                of sequence b is written
 * t0_len       : host [B], current T0 length (the slot written); < cap0
 * t0_pos       : device [B][cap0] slot -> position map; t0_pos[b][t0_len[b]]
 *                is set to position[b]
 * position     : host [B], position of the new token (its current length n)
 * scores, tier : optional device [B][max_ctx]; if non-null, scores[b][pos] = 0
 *                and tier[b][pos] = 0 (T0).  position[b] < max_ctx.
 */
tkv_status tkv_append(const tkv_model* model, int32_t batch, const void* k_new,
                      const void* v_new, void* k_t0, void* v_t0, int32_t cap0,
                      const int32_t* t0_len, int32_t* t0_pos, const int32_t* position,
                      float* scores, uint8_t* tier, int32_t max_ctx, hipStream_t stream);

/* Bytes of device workspace tkv_decode_step needs for these capacities (split
 * records of the split-K attention and the per-row softmax statistics). */
size_t tkv_decode_workspace_bytes(const tkv_model* model, int32_t batch, int32_t n_layers,
                                  int32_t cap0, int32_t cap1);

/*
 * tkv_decode_step -- decode attention over the attended set A = T0 u T1 of
 * layers [layer_begin, layer_end), with the T1 rows already in their device
 * window (Methodologie section 1, T1 is brought to the GPU before attention;
 * section 3, it then contributes exactly as if it had stayed in HBM).  Writes
 * the output and the normalised attention weights alpha, which the importance
 * score sums (Methodologie section 2).
 *
 * q          : device [B][Lr][Hq][D], Lr = layer_end - layer_begin
 * k_t0, v_t0 : device [B][L][Hkv][cap0][D] tiles (or per-sequence capacities,
 *              tkv_model.t0_caps); t0_len host [B] (<= the sequence's capacity)
 * k_t1, v_t1 : device [B][L][Hkv][cap1][D] tiles; t1_len host [B] (<= cap1);
 *              may be null when every t1_len is 0
 * out        : device [B][Lr][Hq][D] float32
 * alpha      : device [B][Lr][Hq][alpha_stride] float32; entry j is the weight
 *              of attended index j (alpha_stride >= t0_len + t1_len); with
 *              model->alpha_scratch = 1 its contents after the call are
 *              unspecified (scratch)
 * Fused score update (optional: pass scores = null to skip): with t0_pos
 *   [B][cap0], t1_pos [B][cap1] (device slot -> position maps) and scores
 *   device [B][max_ctx] float32, adds to scores[b][pos(j)] the sum over the
 *   call's layers and heads of alpha / (num_layers * Hq), exactly what
 *   tkv_update_scores would add.
 * workspace  : device, at least tkv_decode_workspace_bytes(model, batch, Lr,
 *              cap0, cap1) bytes (scratch; no initial contents needed)
 * Numerics: bf16 data use the matrix cores with float32 accumulation (the
 * softmax weights enter P.V as a bf16 pair hi + lo, ~2^-17 relative);
 * float32 data use plain float32 FMAs.
 * A sequence with t0_len + t1_len == 0 gets out = 0 and no weights.
 */
tkv_status tkv_decode_step(const tkv_model* model, int32_t batch, int32_t layer_begin,
                           int32_t layer_end, const void* q, const void* k_t0,
                           const void* v_t0, const int32_t* t0_len, int32_t cap0,
                           const void* k_t1, const void* v_t1, const int32_t* t1_len,
                           int32_t cap1, float* out, float* alpha, int32_t alpha_stride,
                           const int32_t* t0_pos, const int32_t* t1_pos, float* scores,
                           int32_t max_ctx, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * tkv_decode_step_noalloc -- tkv_decode_step for callers that cannot allocate
 * device memory or pass a workspace (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  The workspace is a 64 MiB array
 * inside the library, one per GPU, held until the process ends; its device
 * address is looked up on the first call made with that GPU current (the only
 * global state of the library besides the benchmark timers; the lookup is
 * mutex-guarded).  The call allocates nothing.
 * Arguments, outputs, numerics and errors as for tkv_decode_step without the
 * workspace; a call whose tkv_decode_workspace_bytes(model, batch, Lr, cap0,
 * cap1) exceeds 64 MiB is rejected with TKV_ERR_CAPACITY before anything is
 * queued.  Every call on one GPU uses the same array: calls that overlap on that
 * GPU (on different streams, or from different threads) race.  The workspace
 * needs no initial contents, so nothing is cleared between calls.
 */
tkv_status tkv_decode_step_noalloc(const tkv_model* model, int32_t batch, int32_t layer_begin,
                                   int32_t layer_end, const void* q, const void* k_t0,
                                   const void* v_t0, const int32_t* t0_len, int32_t cap0,
                                   const void* k_t1, const void* v_t1, const int32_t* t1_len,
                                   int32_t cap1, float* out, float* alpha, int32_t alpha_stride,
                                   const int32_t* t0_pos, const int32_t* t1_pos, float* scores,
                                   int32_t max_ctx, hipStream_t stream);

/*
 * tkv_append_decode_step -- tkv_append followed by tkv_decode_step over all
 * layers, as one pass over the key/value rows: each generated token adds one
 * key/value pair (Enonce du probleme), which enters T0 and is attended in the
 * same step.  With bf16 data the attention kernel reads the new rows from
 * k_new/v_new, writes them into the T0 pool at slot t0_len[b] and records
 * t0_pos[b][t0_len[b]] = position[b], score 0 and tier 0 (when scores / tier are
 * given); float32 data run the two calls.
 *
 * Arguments as for tkv_append and tkv_decode_step, with t0_len the lengths
 * BEFORE the append (the call attends t0_len[b] + 1 T0 rows, so
 * t0_len[b] + 1 <= cap0); layer_begin = 0 and layer_end = num_layers.
 * The caller adds one to its t0_len after the call.
 */
tkv_status tkv_append_decode_step(const tkv_model* model, int32_t batch, const void* k_new,
                                  const void* v_new, const int32_t* position, uint8_t* tier,
                                  const void* q, void* k_t0, void* v_t0, const int32_t* t0_len,
                                  int32_t cap0, const void* k_t1, const void* v_t1,
                                  const int32_t* t1_len, int32_t cap1, float* out, float* alpha,
                                  int32_t alpha_stride, int32_t* t0_pos, const int32_t* t1_pos,
                                  float* scores, int32_t max_ctx, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/*
 * tkv_decode_step_window -- tkv_decode_step with a T1 window that holds only
 * the call's layers: t1_win is device [B][Lr][Hkv][2][cap1][D] tiles
 * (Lr = layer_end - layer_begin), window layer i holding layer layer_begin + i,
 * and each (sequence, layer, KV head) row holding its cap1 key slots followed
 * by its cap1 value slots (the layout of the streamed host copy, so one 2-D copy
 * per sequence fills a window).  q, out and alpha hold EVERY layer here
 * ([B][L][Hq][D], [B][L][Hq][D], [B][L][Hq][alpha_stride]); the call reads and
 * writes the rows of its layers.  Methodologie section 1 brings T1 from host
 * memory to the GPU before each attention step; with this call the T1 rows can
 * be streamed layer by layer into a small double-buffered device window (copy
 * layer l + 1 while layer l attends), so HBM holds T0 plus two layers of T1
 * instead of every layer.  Other arguments, outputs, numerics and errors as for
 * tkv_decode_step.
 */
tkv_status tkv_decode_step_window(const tkv_model* model, int32_t batch, int32_t layer_begin,
                                  int32_t layer_end, const void* q, const void* k_t0,
                                  const void* v_t0, const int32_t* t0_len, int32_t cap0,
                                  const void* t1_win, const int32_t* t1_len, int32_t cap1,
                                  float* out, float* alpha, int32_t alpha_stride,
                                  const int32_t* t0_pos, const int32_t* t1_pos, float* scores,
                                  int32_t max_ctx, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/*
 * tkv_decode_step_streamed -- the decode step over all layers with the T1 rows
 * streamed from pinned host memory (Methodologie section 1: T1 stays in host
 * DDR at full precision and is brought to the GPU before each attention step).
 * The layers run in chunks of chunk_layers; the host-to-device copy of chunk
 * c + 2 goes on side_stream as soon as chunk c has read its buffer of the
 * two-buffer device window, so copies overlap attention.  Only the 32-slot
 * blocks that hold live T1 rows cross the link: per chunk, one 2-D copy per
 * sequence of ceil32(t1_len[b]) slots of each of its chunk_layers * Hkv * 2 rows.
 * The score update runs once, after the last chunk, over the group sums of
 * every layer (the same summation as a single tkv_decode_step over all layers),
 * so each score takes one float32 rounding per step.
 *
 * host_t1  : pinned host [B][L][Hkv][2][cap1][D] tiles: per (sequence, layer,
 *            KV head), the keys then the values of the T1 rows in the
 *            window-slot order of t1_pos
 * win      : device [2][B][chunk_layers][Hkv][2][cap1][D] tiles (two buffers)
 * side_stream2 : optional (may be null) second copy stream: chunks then
 *                alternate between the two, so the next copy is queued when the
 *                running one ends (shorter idle gaps on the link)
 * events   : four caller-owned events (two "copied", two "read"); their
 *            previous contents are overwritten
 * link_bytes : optional host out: bytes queued host -> device by this call
 * workspace: tkv_decode_workspace_bytes(model, batch, L, cap0, cap1) bytes
 * batch    : at most 64 (TKV_ERR_CAPACITY above)
 * q, out, alpha and the rest as for tkv_decode_step over layers [0, L).
 * Every argument is checked before anything is queued.
 */
tkv_status tkv_decode_step_streamed(const tkv_model* model, int32_t batch, const void* q,
                                    const void* k_t0, const void* v_t0, const int32_t* t0_len,
                                    int32_t cap0, const void* host_t1, const int32_t* t1_len,
                                    int32_t cap1, void* win, int32_t chunk_layers, float* out,
                                    float* alpha, int32_t alpha_stride, const int32_t* t0_pos,
                                    const int32_t* t1_pos, float* scores, int32_t max_ctx,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream,
                                    hipStream_t side_stream, hipStream_t side_stream2,
                                    hipEvent_t* events, int64_t* link_bytes);

/*
 * Attended T2 pool (optional variant of the decode step).  Methodologie
 * section 1 keeps T2 tokens at reduced precision (8-bit quantisation), and the
 * accuracy the pages report for offloading to T2 ("Resultats cles") is that of
 * a model still attending them: each T2 row enters the same softmax as
 * code * scale of its 8-bit row (the format of tkv_quantize_t2), after the T1
 * rows.  The pool lives in device memory:
 *
 * k_codes, v_codes : device [B][L][Hkv][cap2][D] int8, in the K-tile / V-tile
 *                    element order of the bf16 pools (one byte per element),
 *                    16-byte aligned
 * k_scale, v_scale : device [B][L][Hkv][cap2] float32 (one scale per row),
 *                    16-byte aligned
 * t2_pos           : device [B][cap2] slot -> position map (read by the fused
 *                    score update; may be null when scores are not updated)
 * t2_len           : host [B], T2 rows in slots [0, t2_len) (<= cap2)
 * cap2             : multiple of 32
 * With a T2 pool, the attended index j runs over T0 slots, then T1 slots, then
 * T2 slots (j - t0_len - t1_len), alpha_stride must cover t0_len + t1_len +
 * t2_len, and the decode workspace is
 * tkv_decode_workspace_bytes(model, batch, Lr, cap0, cap1 + cap2).
 */
typedef struct {
  const int8_t* k_codes;
  const int8_t* v_codes;
  const float* k_scale;
  const float* v_scale;
  const int32_t* t2_pos;
  const int32_t* t2_len;
  int32_t cap2;
} tkv_t2_pool;

/*
 * tkv_decode_step_t2 / tkv_append_decode_step_t2 -- tkv_decode_step and
 * tkv_append_decode_step over the attended set T0 u T1 u T2, with the T2 rows
 * read from the 8-bit pool `t2` (non-null; see tkv_t2_pool).  Other arguments,
 * outputs and errors as for the calls without _t2.  Numerics: bf16 data widen
 * the int8 codes exactly to bf16 for the matrix-core products; the key scale
 * multiplies the row's logit and the value scale its weight in P.V (the
 * softmax sum uses the plain weight); float32 data use code * scale in
 * float32.
 */
tkv_status tkv_decode_step_t2(const tkv_model* model, int32_t batch, int32_t layer_begin,
                              int32_t layer_end, const void* q, const void* k_t0,
                              const void* v_t0, const int32_t* t0_len, int32_t cap0,
                              const void* k_t1, const void* v_t1, const int32_t* t1_len,
                              int32_t cap1, const tkv_t2_pool* t2, float* out, float* alpha,
                              int32_t alpha_stride, const int32_t* t0_pos,
                              const int32_t* t1_pos, float* scores, int32_t max_ctx,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

tkv_status tkv_append_decode_step_t2(const tkv_model* model, int32_t batch, const void* k_new,
                                     const void* v_new, const int32_t* position, uint8_t* tier,
                                     const void* q, void* k_t0, void* v_t0,
                                     const int32_t* t0_len, int32_t cap0, const void* k_t1,
                                     const void* v_t1, const int32_t* t1_len, int32_t cap1,
                                     const tkv_t2_pool* t2, float* out, float* alpha,
                                     int32_t alpha_stride, int32_t* t0_pos,
                                     const int32_t* t1_pos, float* scores, int32_t max_ctx,
                                     void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/*
 * tkv_update_scores -- the importance-score recurrence (Methodologie section 2):
 * scores[b][pos(j)] += (1/(num_layers*Hq)) * sum over layers in
 * [layer_begin, layer_end) and heads of alpha[b][l][h][j], for every attended
 * index j.  Calling it once for all layers or once per layer adds the same
 * mass (up to float32 summation order).
 *
 * alpha  : device [B][Lr][Hq][alpha_stride] float32 (normalised weights)
 * t0_pos, t1_pos : device slot -> position maps [B][cap0], [B][cap1]
 * t0_len, t1_len : host [B]
 * scores : device [B][max_ctx] float32, read-modify-write
 */
tkv_status tkv_update_scores(const tkv_model* model, int32_t batch, int32_t layer_begin,
                             int32_t layer_end, const float* alpha, int32_t alpha_stride,
                             const int32_t* t0_pos, const int32_t* t0_len, int32_t cap0,
                             const int32_t* t1_pos, const int32_t* t1_len, int32_t cap1,
                             float* scores, int32_t max_ctx, hipStream_t stream);

/*
 * tkv_assign_tiers -- rank positions [0, ctx_len[b]) of every sequence into
 * T0..T3 (Methodologie sections 1 and 4).  Keep order: higher score first,
 * equal scores keep the lower position first.  Always taking the least
 * important candidates:
 *   1. T3 is absorbing; evict clamp(N3 - |T3|, 0, |pool|) more from the
 *      non-protected positions in T0/T1/T2;
 *   2. surviving T2 positions stay T2; move clamp(N2 - |survivors|, 0, |live|)
 *      more from the remaining non-protected T0/T1 positions into T2;
 *   3. move min(N1, |live left|) of the rest into T1;
 *   4. everything else (with protected T0/T1 positions) becomes T0.
 *
 * ctx_len   : host [B], current length n of each sequence (<= max_ctx)
 * scores    : device [B][max_ctx] float32 (finite values)
 * tier_prev : device [B][max_ctx] uint8 previous tiers (0..3)
 * tier_next : device [B][max_ctx] uint8 new tiers; may equal tier_prev
 * counts    : device [B][4] int32 counts of T0..T3.  If tier_prev holds a
 *             value above 3, counts[b] is {-1,-1,-1,-1} and tier_next of that
 *             sequence is left untouched.
 * Bit-exact and deterministic: ties are broken by position only.
 */
tkv_status tkv_assign_tiers(int32_t batch, const int32_t* ctx_len, int32_t max_ctx,
                            const float* scores, const tkv_policy* policy,
                            const uint8_t* tier_prev, uint8_t* tier_next, int32_t* counts,
                            hipStream_t stream);

/* Bytes of device workspace tkv_compact needs (0 for an invalid model or a
 * negative size).  It grows with batch * (max_ctx + cap0 + cap1) words plus a
 * staging area of batch * cap1 rows of L * Hkv * 2 * D elements. */
size_t tkv_compact_workspace_bytes(const tkv_model* model, int32_t batch, int32_t max_ctx,
                                   int32_t cap0, int32_t cap1);

/*
 * tkv_compact -- after a reassignment, bring the resident T0 pool and the T1
 * window in line with the new tier map, in place, and turn the rows that
 * newly entered T2 into 8-bit rows (Methodologie section 4: tiers change every
 * Delta steps and only the tokens whose tier changed move; section 1: T2 holds
 * low-importance tokens at reduced precision).
 *
 * Slot order inside the pool and the window is not position order: the slot
 * -> position maps t0_pos / t1_pos say which position each slot holds.  A row
 * moves only if its tier changed, or if it stays but sits at or past the new
 * length of its pool; each mover fills a hole (a slot below the new length
 * whose row left or which was past the old length), the i-th mover in
 * position order taking the i-th hole in slot order.  Rows leaving for T3 are
 * dropped.  Every new T0/T1 row is already resident, because T2 and T3 never
 * return to T0/T1.  Slots at or past the new lengths keep stale rows.
 *
 * ctx_len          : host [B]
 * tier_prev/next   : device [B][max_ctx] uint8, distinct buffers
 * k/v_t0, cap0     : T0 pool [B][L][Hkv][cap0][D] (tiles), updated in place
 * t0_pos           : device [B][cap0] slot -> position, updated in place
 * t0_len           : host [B] current T0 lengths
 * k/v_t1, t1_pos, t1_len, cap1 : the T1 window, likewise
 * t2_src, t2_pos   : device [B][t2_cap]: the old slot code of each newly-T2 row
 *                    (s >= 0 T0 slot s, s < 0 T1 slot -s-1) and its position,
 *                    in ascending position order
 * t2_codes/scales  : device, as tkv_quantize_t2's codes/scales with max_rows =
 *                    t2_cap; filled for the newly-T2 rows (may be null if
 *                    t2_cap is 0)
 * new_lens         : device [B][4] int32: new T0 length, new T1 length,
 *                    newly-T2 count, row copies made (moves into T1 and T0
 *                    plus promoted rows staged).  If a capacity would be exceeded or the
 *                    maps disagree with tier_prev and the lengths (a position
 *                    without its slot, a slot pointing outside the context,
 *                    a T2/T3 position marked T0/T1 again), new_lens[b] is
 *                    {-1,-1,-1,-1} and nothing of sequence b is changed.
 * workspace        : device, tkv_compact_workspace_bytes() bytes
 * Calls that overlap on the same buffers race.
 */
tkv_status tkv_compact(const tkv_model* model, int32_t batch, const int32_t* ctx_len,
                       int32_t max_ctx, const uint8_t* tier_prev, const uint8_t* tier_next,
                       void* k_t0, void* v_t0, int32_t* t0_pos, const int32_t* t0_len,
                       int32_t cap0, void* k_t1, void* v_t1, int32_t* t1_pos,
                       const int32_t* t1_len, int32_t cap1, int32_t* t2_src, int32_t* t2_pos,
                       int32_t t2_cap, int8_t* t2_codes, float* t2_scales, int32_t* new_lens,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * tkv_t0_capacity -- a T0 pool capacity that no reassignment at a length in
 * [n_from, n_to] can exceed, Delta appended rows included (Methodologie sections
 * 1 and 4: T0 keeps the protected rows and the most important rest; the tier
 * budgets are fractions of the current length).  After a reassignment at length
 * n, T0 holds at most max(N0(n), |protected(n)|) rows, N0(n) = n - N1 - N2 - N3;
 * the result is that bound's maximum over [n_from, n_to] plus delta, rounded up
 * to a multiple of 32.  A caller can shrink its T0 pool to it after the first
 * reassignment.  Returns -1 on a bad policy or range.
 */
int32_t tkv_t0_capacity(const tkv_policy* policy, int32_t n_from, int32_t n_to);

/* Bytes of device workspace and of pinned host scratch tkv_compact_host_t1
 * needs (0 for an invalid model or a negative size).  The device workspace is
 * tkv_compact's without its row staging: the rows that cross the link are staged
 * in the host scratch. */
size_t tkv_compact_host_t1_workspace_bytes(const tkv_model* model, int32_t batch, int32_t max_ctx,
                                           int32_t cap0, int32_t cap1);
size_t tkv_compact_host_t1_scratch_bytes(const tkv_model* model, int32_t batch, int32_t max_ctx,
                                         int32_t cap1);

/*
 * tkv_compact_host_t1 -- tkv_compact for T1 rows that live in host memory
 * (Methodologie section 1: T1 in host DDR at full precision; section 4: at a
 * reassignment only the tokens whose tier changed move, and only newly
 * promoted tokens go from host memory to the GPU).  The device holds the T0
 * pool and the T1 slot -> position map; the host holds a store of full-precision
 * rows by position and the streamed T1 window in window-slot order.  Only these
 * rows cross the host link:
 *   device -> host : rows that enter T1 from T0 (into the store);
 *   host -> device : rows that leave T1 for T0 (promoted) or for T2 (to be
 *                    quantised on the device);
 * plus the tier and slot maps the host reads (2 max_ctx + 16 cap1 + 32 bytes per
 * sequence: both tier maps, the T1 slot map before and after, the list of rows
 * entering T1, the new lengths and list counts).  Rows that stay in T1 never move; the window slots whose
 * position changed are rewritten on the host from the store.  Results are those
 * of tkv_compact on the same state (same holes, same slot maps, same int8 rows).
 * The call is host-synchronous: it returns when every queued operation is done.
 *
 * Arguments as for tkv_compact, without the device T1 window, and:
 * workspace        : device, tkv_compact_host_t1_workspace_bytes() bytes
 * store_k, store_v : host [B][L][Hkv][max_ctx][D] full-precision rows by
 *                    position (read and written by host threads)
 * t1_host          : pinned host [B][L][Hkv][2][cap1][D] tiles: the window that
 *                    tkv_decode_step_streamed streams, updated in place
 * new_lens_host    : host [B][4], a copy of new_lens
 * host_scratch     : pinned, device-mapped host memory of
 *                    tkv_compact_host_t1_scratch_bytes() bytes; the device reads
 *                    and writes its row staging directly (TKV_ERR_HIP if the
 *                    memory is not device-mapped)
 * link_bytes       : optional host out: bytes that crossed the link
 * A sequence whose maps disagree with tier_prev gets new_lens {-1,-1,-1,-1} as
 * with tkv_compact; its T1 window is then left as it was.
 */
tkv_status tkv_compact_host_t1(const tkv_model* model, int32_t batch, const int32_t* ctx_len,
                               int32_t max_ctx, const uint8_t* tier_prev,
                               const uint8_t* tier_next, void* k_t0, void* v_t0,
                               int32_t* t0_pos, const int32_t* t0_len, int32_t cap0,
                               int32_t* t1_pos, const int32_t* t1_len, int32_t cap1,
                               void* store_k, void* store_v, void* t1_host, int32_t* t2_src,
                               int32_t* t2_pos, int32_t t2_cap, int8_t* t2_codes,
                               float* t2_scales, int32_t* new_lens, int32_t* new_lens_host,
                               void* workspace, size_t workspace_bytes, void* host_scratch,
                               size_t host_scratch_bytes, int64_t* link_bytes,
                               hipStream_t stream);

/*
 * tkv_quantize_t2 -- 8-bit rows of the tokens that enter T2 (Methodologie
 * section 1, T2 holds low-importance tokens at reduced precision, 8-bit
 * quantisation being the example).  Per (row, layer, KV head, K or V) row of D
 * values x: scale = absmax(x) / 127 and code = round-half-even(x / scale),
 * both IEEE float32 divisions, clamped to [-127, 127]; an all-zero row gets
 * scale 0 and codes 0.  Dequantised value: code * scale.
 *
 * k/v_t0, cap0, k/v_t1, cap1 : the pool and window the rows are read from
 * src     : device [B][max_rows]: s >= 0 is T0 slot s, s < 0 is T1 slot -s-1
 * n_rows  : device int32, element b * n_rows_stride is the row count of
 *           sequence b (tkv_compact's new_lens with stride 4, offset 2, fits)
 * max_rows: host bound on every row count (rows at or beyond it are ignored)
 * codes   : device [B][max_rows][L][Hkv][2][D] int8 (index 0 = K, 1 = V)
 * scales  : device [B][max_rows][L][Hkv][2] float32
 */
tkv_status tkv_quantize_t2(const tkv_model* model, int32_t batch, const void* k_t0,
                           const void* v_t0, int32_t cap0, const void* k_t1, const void* v_t1,
                           int32_t cap1, const int32_t* src, const int32_t* n_rows,
                           int32_t n_rows_stride, int32_t max_rows, int8_t* codes,
                           float* scales, hipStream_t stream);

/* Bytes of device workspace tkv_t2_update needs (hole and move lists). */
size_t tkv_t2_update_workspace_bytes(int32_t batch, int32_t cap2);

/*
 * tkv_t2_update -- after a reassignment, bring the attended T2 pool in line
 * with the new tier map, in place (Methodologie section 4: only the tokens
 * whose tier changed move; section 1: T2 keeps 8-bit rows).  T2 is left only
 * for T3 (those rows are dropped), and receives the rows tkv_compact has just
 * quantised.  Holes are slots below the new length whose row left or which
 * were past the old length, in slot order; movers are rows that stay but sit
 * at or past the new length (slot order), then the new rows in their list
 * order; the i-th mover fills the i-th hole.  Rows that stay below the new
 * length keep their slots.  Call it after tkv_compact on the same stream.
 *
 * ctx_len          : host [B]
 * tier_next        : device [B][max_ctx], the new tier map
 * k/v_codes, k/v_scale, t2_pos, cap2 : the pool (see tkv_t2_pool), in/out
 * t2_len           : host [B], current pool lengths
 * new_pos          : device [B][max_rows] positions of the new rows
 *                    (tkv_compact's t2_pos, max_rows = its t2_cap)
 * new_codes/scales : device [B][max_rows][L][Hkv][2][D] int8 and
 *                    [B][max_rows][L][Hkv][2] float32 (tkv_compact's output)
 * n_new            : device int32, element b * n_new_stride is the new row count
 *                    of sequence b (tkv_compact's new_lens + 2 with stride 4)
 * new_t2_len       : device [B][2] int32: the new pool length and the row moves
 *                    made.  If a slot of the old pool maps to a position >= n or
 *                    to one whose new tier is T0/T1, if the new row count is
 *                    negative or above max_rows, if the new length exceeds cap2,
 *                    or if it differs from the number of T2 positions of
 *                    tier_next, new_t2_len[b] is {-1,-1} and nothing of
 *                    sequence b is changed.
 * workspace        : device, tkv_t2_update_workspace_bytes(batch, cap2) bytes
 */
tkv_status tkv_t2_update(const tkv_model* model, int32_t batch, const int32_t* ctx_len,
                         int32_t max_ctx, const uint8_t* tier_next, int8_t* k_codes,
                         int8_t* v_codes, float* k_scale, float* v_scale, int32_t* t2_pos,
                         const int32_t* t2_len, int32_t cap2, const int32_t* new_pos,
                         const int8_t* new_codes, const float* new_scales, const int32_t* n_new,
                         int32_t n_new_stride, int32_t max_rows, int32_t* new_t2_len,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * tkv_gather_t1 -- bring one sequence's T1 rows to the GPU (Methodologie
 * section 1: T1 stays in host DDR at full precision and is brought to the GPU
 * before each attention step).  Packs the rows of the host store at the given
 * positions, in the given order, into contiguous pinned staging with host
 * threads, then queues the host-to-device copy of the staging on side_stream
 * and records `ready` there.  The attention stream must wait on `ready` before
 * reading the window.
 *
 * host_k, host_v : host [L][Hkv][max_ctx][D] full-precision store
 * positions      : host [n_t1], distinct, each < max_ctx: window slot i
 *                  receives positions[i] (pass the window's slot -> position
 *                  map); null re-sends the staging as it is (no pack)
 * staging        : pinned host [L][Hkv][2][cap1][D] tiles (n_t1 <= cap1): per
 *                  (layer, KV head) the key slots, then the value slots, in the
 *                  device window's storage order (slots past n_t1 in the last
 *                  32-slot block are zeroed)
 * dev_t1         : device window of the same layout ([L][Hkv][2][cap1][D], the
 *                  layout of tkv_decode_step_window); null packs only.  Only the
 *                  ceil32(n_t1) leading slots of each row are copied.
 * ready          : event recorded on side_stream after the copy; may be null
 * Before packing, a call with dev_t1 waits for the work already queued on
 * side_stream (an earlier copy may still be reading the staging); a pack-only
 * call (dev_t1 null) leaves that ordering to its caller.  The pack is
 * synchronous on the calling thread; only the copy is queued.
 */
tkv_status tkv_gather_t1(const tkv_model* model, const void* host_k, const void* host_v,
                         int32_t max_ctx, const int32_t* positions, int32_t n_t1, void* staging,
                         int32_t cap1, void* dev_t1, hipStream_t side_stream, hipEvent_t ready);

/*
 * tkv_read_probe -- benchmark aid: streams `bytes` of device memory (a multiple of
 * 16 KB, 16-byte aligned) with the access pattern of the decode-attention kernel
 * (`waves` waves, one per SIMD when waves = 4 x CUs, each reading one contiguous
 * range in 16 KB units of 1 KB wave loads, non-temporal) and stores one word per
 * wave into sink (device, `waves` words).  Timed by the kernel timers as
 * "read_probe": the read ceiling the attention kernel is measured against.
 */
tkv_status tkv_read_probe(const void* buf, size_t bytes, int32_t waves, uint32_t* sink,
                          hipStream_t stream);

/*
 * Kernel timers for benchmarks.  While enabled, every kernel the library
 * launches is bracketed by HIP events on its own stream; tkv_timing_read
 * synchronises those events and returns the summed milliseconds and launch
 * count of one kernel (by name, e.g. "attn_partial") since the last reset.
 * tkv_timing_select restricts the timers to a comma-separated list of kernel
 * names (NULL or "" = every kernel): each pair of events adds a few
 * microseconds between launches, so a throughput run times only the kernel
 * it reports.  Not thread-safe.
 */
tkv_status tkv_timing_enable(int32_t enable);
tkv_status tkv_timing_select(const char* kernels);
tkv_status tkv_timing_reset(void);
tkv_status tkv_timing_read(const char* kernel, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* TKV_H */
