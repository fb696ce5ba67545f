/*
 * kvc.h -- C ABI of the compressed-KV-cache hot path for AMD MI355X (gfx950).
 *
 * The path (one transformer layer per call):
 *   kvc_select      SnapKV/PyramidKV selection: the last W prompt queries score
 *                   every earlier prompt position, the scores are max-pooled and
 *                   the top-k positions per KV head are kept.
 *   kvc_quantize    KIVI/MiniKV group quantization of the kept tokens (keys per
 *                   channel, values per token, groups of g = 32 or 16, 2 or 4 bits, fp16
 *                   scale and zero-point) into a packed cache plus a bf16
 *                   residual of the most recent tokens.
 *   kvc_decode_attn one decode step: append the new token, flush a full group of
 *                   the residual into the packed history, then single-query
 *                   attention over packed history (dequantized on the fly) and
 *                   residual under one softmax.
 *   kvc_budget      host-only per-layer budgets (uniform or pyramid) and the
 *                   cache footprint; kvc_budget_weighted: budgets proportional
 *                   to per-layer weights (the variance policies).
 *   kvc_window_scores, kvc_topk
 *                   the two halves of kvc_select (scores and their variance;
 *                   pool + top-k of given scores).
 *   kvc_select_recent
 *                   position-only selection: attention sinks plus the recent
 *                   window, or the sliding window alone.
 *   kvc_prefill_attn
 *                   the prefill's causal attention that also returns the
 *                   attention each key accumulates (MiniKV's selective
 *                   flash-attention); kvc_select_h2o: heavy hitters on it.
 *
 * Conventions shared by every call
 *   Memory:   every device buffer is allocated and owned by the caller; the
 *             library allocates no device memory and keeps no global mutable
 *             state besides a thread-local last-HIP-error code (and, for
 *             kvc_decode_attn_noalloc only, its per-device scratch array and
 *             that array's address, set once per device).  Scratch space
 *             comes from a caller workspace: pass ws == NULL to have the
 *             required size written to *ws_bytes (nothing is launched).
 *   Streams:  device work is only enqueued on `stream` (a hipStream_t passed as
 *             void*, NULL = default stream); no call synchronizes.  kvc_budget
 *             runs on the host and returns when done.
 *   Errors:   every call returns a kvc_status and never aborts or throws.  All
 *             argument checks happen before any launch, so a validation error
 *             leaves caller memory untouched.  KVC_ERR_HIP means a launch
 *             failed (kvc_last_hip_error() gives the hipError_t); cache contents
 *             are then undefined.  Faults inside kernels surface at the caller's
 *             next synchronization, as with any HIP work.
 *   Dtypes:   q/k/v inputs are float32 or bfloat16 (kvc_dtype); the residual is
 *             bfloat16 (round to nearest even from float32 inputs); attention
 *             output is float32.
 *   Shapes:   1 <= D <= 256 with D % 32 == 0; Hq % Hkv == 0; Hq/Hkv <= 16.
 *
 * Cache layout (one layer; C-contiguous, capacities are the strides):
 *   k_codes [B][Hkv][q_cap][D*bits/32]  uint32: word w of token t holds
 *                                       channel (32/bits)*w+i at bits bits*i
 *   k_meta  [B][Hkv][q_cap/g][D]        uint32: group q = tokens gq..gq+g-1,
 *                                       channel c (g = the cache's group)
 *   v_codes [B][Hkv][q_cap*bits/32][D]  uint32: word row w, channel c holds
 *                                       token (32/bits)*w+i at bits bits*i
 *   v_meta  [B][Hkv][q_cap][D/g]        uint32: token t, channels gj..gj+g-1
 *   meta word = fp16 scale bits | (fp16 zero-point bits << 16)
 *   k_res [B][Hkv][r_cap][D]            uint16 bfloat16 keys, token-major
 *   v_res [B][Hkv][D][r_cap]            uint16 bfloat16 values, channel-major
 *                                       (a decode step reads 8 consecutive
 *                                       tokens of one channel per load)
 *   The residual is a ring: its i-th oldest token (i < r_len) is row
 *   (r_start + i) % r_cap of every (b, head).  A flush quantizes the g oldest
 *   and advances r_start by g, so no residual data is ever moved.
 * Codes are LSB-first (MiniKV Sec. 4.4: 16 INT2 values shifted into one INT32).
 * Dequantized value = zero + code * scale.
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVC_OK = 0,
  KVC_ERR_NULL = 1,      /* a required pointer is NULL                         */
  KVC_ERR_SHAPE = 2,     /* inconsistent or unsupported sizes                  */
  KVC_ERR_DTYPE = 3,     /* unknown kvc_dtype                                  */
  KVC_ERR_BITS = 4,      /* bits not in {2,4} (or group/meta invalid)          */
  KVC_ERR_CAPACITY = 5,  /* q_cap / r_cap too small, or cache not empty        */
  KVC_ERR_WORKSPACE = 6, /* *ws_bytes smaller than required                    */
  KVC_ERR_HIP = 7        /* a HIP launch or runtime call failed                */
} kvc_status;

typedef enum { KVC_F32 = 0, KVC_BF16 = 1 } kvc_dtype;

/* One layer's compressed cache.  Host struct of caller-owned device pointers.
 * The library updates q_len and r_len when it enqueues work, so the host view
 * is the state after the enqueued work completes (stream order). */
typedef struct {
  int32_t batch, kv_heads, head_dim; /* B, Hkv, D                              */
  int32_t bits;                      /* 2 or 4                                 */
  int32_t residual;                  /* R: recent tokens kept in bf16          */
  int32_t q_cap, q_len;              /* packed history, tokens: q_cap a multiple
                                        of 32, q_len a multiple of the group   */
  int32_t r_cap, r_len;              /* bf16 residual, tokens; r_cap >= R + g,
                                        r_cap a multiple of 8                  */
  int32_t r_start;                   /* ring row of the oldest residual token
                                        (a multiple of 8, < r_cap)             */
  int32_t group;                     /* g, the quantization group: 32 (0 also
                                        means 32) or 16 (MiniKV Sec. 5.1: keys
                                        per channel over 16 tokens, values per
                                        token over 16 channels)                */
  int32_t flush_all;                 /* residual policy.  0: a decode step
                                        flushes the oldest g tokens when the
                                        residual reaches R+g, and the prefill
                                        keeps R..R+g-1 tokens in bf16.  1:
                                        MiniKV Alg. 1 as printed: the prefill
                                        quantizes every complete group, and the
                                        residual is quantized whole when it
                                        reaches R (R a positive multiple of g) */
  uint32_t *k_codes, *k_meta, *v_codes, *v_meta;
  uint16_t *k_res, *v_res;
} kvc_cache;

/* Byte sizes of the six cache arrays for given capacities (host-only helper):
 * out[0..5] = k_codes, k_meta, v_codes, v_meta, k_res, v_res; group as in
 * kvc_cache (0, 16 or 32; else KVC_ERR_BITS).  q_cap must be a multiple of 32. */
kvc_status kvc_cache_sizes(int32_t batch, int32_t kv_heads, int32_t head_dim, int32_t bits, int32_t group,
                           int32_t q_cap, int32_t r_cap, size_t out[6]);

/* ------------------------------------------------------------------ budget
 * Per-layer selection budgets and footprint, on the host.
 * Uniform: every layer keeps avg_budget (MiniKV Sec. 4.2 "Uniform").
 * Pyramid: PyramidKV "Proposed Method" (budget allocation: top layer gets
 *   total/(beta*m), an arithmetic sequence between bottom and top) read with
 *   MiniKV Sec. 4.2's mean-preserving endpoints: top = avg/beta,
 *   bottom = 2*avg - avg/beta, linear in between, layer 0 largest; integerized
 *   exactly (floor, then +1 to the largest fractional parts, ties to the lower
 *   layer) so the budgets sum to layers*avg.  Each budget is then capped at
 *   prompt_len - window.  avg_budget < 0 means no eviction (all n-W kept).
 * The budget counts selected tokens, excluding the window.
 * Footprint (blog "The budget"; MiniKV "KV Cache compression ratio analysis"):
 *   bits_per_element = 16 if bits == 16 else bits + 2*meta_bits/group;
 *   bytes_per_prompt_token = 2*L*Hkv*D*bits_per_element/8 * kept fraction;
 *   bytes_total = 2*Hkv*D*bits_per_element/8 * sum over layers of
 *                 (kept + gen_len) tokens;
 *   bytes_layout = exact bytes of this library's packed layout right after
 *                 kvc_quantize for one sequence (codes + meta + bf16 residual).
 * layer_budget: host array [layers] (required).  fp may be NULL.
 * Errors: KVC_ERR_NULL, KVC_ERR_SHAPE (layers < 1, window or prompt invalid,
 *   beta < 1 or not finite for pyramid), KVC_ERR_BITS (bits not in {2,4,8,16},
 *   group not in {16,32}, meta_bits not in {8,16,32}). */
typedef struct {
  int32_t layers, kv_heads, head_dim, prompt_len, window, gen_len;
  int32_t avg_budget; /* selected tokens per head per layer; < 0: keep all   */
  int32_t pyramid;    /* 0 uniform, 1 arithmetic pyramid                     */
  double beta;        /* pyramid shape: top layer = avg/beta                  */
  int32_t bits, group, meta_bits, residual; /* bits == 16: unquantized      */
} kvc_budget_args;

typedef struct {
  double bits_per_element, bytes_per_prompt_token, bytes_total, bytes_layout;
} kvc_footprint;

kvc_status kvc_budget(const kvc_budget_args *args, int32_t *layer_budget, kvc_footprint *fp);

/* Budgets proportional to per-layer weights (MiniKV Sec. 4.2, the variance
 * policies: Var-prop weights a layer by the variance of its cumulated attention,
 * Var-inv by the reciprocal; see kvc_window_scores for the variance).  With
 * S = w_0 + w_1 + ... (in that order) and x_l = (L*avg * w_l) / S in IEEE
 * double, layer l gets floor(x_l), plus one for the layers with the largest
 * fractional parts (ties to the lower layer) until the sum is L*avg; then each
 * is capped at prompt_len - window.  args->pyramid and args->beta are ignored;
 * the footprint is as for kvc_budget.
 *   weights [layers] float64, every one finite and > 0.
 * Errors: KVC_ERR_NULL, KVC_ERR_SHAPE (as kvc_budget, avg_budget < 0, layers *
 *   avg_budget > INT32_MAX, a weight not finite or <= 0, an infinite sum),
 *   KVC_ERR_BITS. */
kvc_status kvc_budget_weighted(const kvc_budget_args *args, const double *weights, int32_t *layer_budget,
                               kvc_footprint *fp);

/* ------------------------------------------------------------------ select
 * Observation-window token selection for one layer (blog "Eviction": SnapKV;
 * PyramidKV "KV Cache Selection").  For KV head j and each of its G query
 * heads, window row r (absolute position p = n-W+r) attends causally to keys
 * 0..p with logits q.k/sqrt(D); the softmax probabilities are summed over the
 * W rows and the G heads for every candidate c < n-W, max-pooled with an odd
 * kernel `pool` (stride 1, edges clipped), and the k' = min(budget, n-W)
 * largest are selected (ties to the lower position), written in ascending
 * order.  The window [n-W, n) is always kept and is not part of idx.
 *   q_win  [B][Hq][W][D]   the last W prompt queries (post-RoPE), dtype
 *   k      [B][Hkv][n][D]  prompt keys (post-RoPE), dtype
 *   idx    [B][Hkv][k']    int32 output, ascending, in [0, n-W) (may be NULL if k' == 0)
 *   scores [B][Hkv][n-W]   float32 output of the pooled scores, or NULL
 *   budget < 0 keeps every candidate.  When every candidate is kept and scores
 *   is NULL, the ranking decides nothing: idx = 0, 1, ..., n-W-1 is written and
 *   no score is computed.
 * Errors: KVC_ERR_NULL, KVC_ERR_DTYPE, KVC_ERR_SHAPE (W < 1, W > n, pool even
 *   or < 1, shapes above), KVC_ERR_WORKSPACE, KVC_ERR_HIP. */
kvc_status kvc_select(const void *q_win, const void *k, kvc_dtype dtype, int32_t B, int32_t Hq,
                      int32_t Hkv, int32_t n, int32_t D, int32_t W, int32_t pool, int32_t budget,
                      int32_t *idx, float *scores, void *ws, size_t *ws_bytes, void *stream);

/* kvc_select_lse: kvc_select given each window row's softmax normalizer, as the
 * prompt's own prefill attention computes it (FlashAttention keeps every row's
 * log-sum-exp; MiniKV Sec. 4.3 fuses the selection scores into that prefill).
 * The scores are the same column sums; with the normalizers known, the window
 * scorer needs one pass over K instead of two (the first pass of kvc_select
 * exists only to find them).
 *   lse   float32, row w of query head h of batch row b at lse[(b*Hq + h) *
 *         lse_stride + w]: the natural-log log-sum-exp of that window row's
 *         causal logits q.k/sqrt(D) over keys 0..n-W+w (kvc_prefill_attn's lse
 *         output from its row n-W on, with lse_stride = n).
 *   lse_stride >= W.  Everything else as kvc_select (same workspace size).
 * Errors: as kvc_select; KVC_ERR_NULL also for lse NULL, KVC_ERR_SHAPE for
 *   lse_stride < W. */
kvc_status kvc_select_lse(const void *q_win, const void *k, const float *lse, int32_t lse_stride, kvc_dtype dtype,
                          int32_t B, int32_t Hq, int32_t Hkv, int32_t n, int32_t D, int32_t W, int32_t pool,
                          int32_t budget, int32_t *idx, float *scores, void *ws, size_t *ws_bytes, void *stream);

/* The two halves of kvc_select, for callers that look at the scores before
 * choosing budgets (the variance policies of kvc_budget_weighted):
 *
 * kvc_window_scores: the window scorer alone (blog "Eviction": SnapKV; PyramidKV
 * "KV Cache Selection"): raw [B][Hkv][n-W] float32 gets the column sums of the
 * window rows' causal softmax over the candidates, before pooling (kvc_select's
 * scores before its max-pool).  var [B][Hkv] float32 (may be NULL) gets the
 * population variance of each row of raw, accumulated in float64 (MiniKV Sec.
 * 4.2 and Fig. 7: the variance score Var(A_cumul); a layer's score is the
 * mean over b and KV heads, left to the caller; computed as
 * (sum x^2 - (sum x)^2 / N) / N with float64 sums).  Shapes and dtypes as
 * kvc_select; with n == W nothing is written.
 * Errors: KVC_ERR_NULL (raw NULL with n > W), KVC_ERR_DTYPE, KVC_ERR_SHAPE,
 *   KVC_ERR_WORKSPACE, KVC_ERR_HIP. */
kvc_status kvc_window_scores(const void *q_win, const void *k, kvc_dtype dtype, int32_t B, int32_t Hq,
                             int32_t Hkv, int32_t n, int32_t D, int32_t W, float *raw, float *var, void *ws,
                             size_t *ws_bytes, void *stream);

/* kvc_topk: kvc_select's second half on given scores: max-pool raw
 * [B][Hkv][N] float32 with the odd kernel `pool` (edges clipped), take the
 * k' = min(budget, N) largest per (b, KV head) (ties to the lower position),
 * ascending, into idx [B][Hkv][k'] int32; scores [B][Hkv][N] float32 (or NULL)
 * gets the pooled scores.  budget < 0 keeps all N.  idx may be NULL if k' == 0.
 * Errors: KVC_ERR_NULL, KVC_ERR_SHAPE (B, Hkv < 1, N < 0, pool even or < 1),
 *   KVC_ERR_WORKSPACE, KVC_ERR_HIP. */
kvc_status kvc_topk(const float *raw, int32_t B, int32_t Hkv, int32_t N, int32_t pool, int32_t budget,
                    int32_t *idx, float *scores, void *ws, size_t *ws_bytes, void *stream);

/* kvc_select_recent: position-only selection, no scores (blog "Eviction":
 * a sliding window keeps the last tokens, StreamingLLM also keeps the first
 * four "attention sink" tokens; PyramidKV "Baselines": StreamingLLM keeps the
 * first k - alpha and the last alpha tokens).  With the window [n-W, n) kept as
 * by kvc_select and k' = min(budget, n-W) (budget < 0: n-W), every (b, KV
 * head) row of idx [B][Hkv][k'] int32 gets the s = min(sinks, k') positions
 * 0..s-1 followed by the last k' - s candidates n-W-(k'-s) .. n-W-1, ascending:
 * the cache then holds the first s prompt tokens and the last k' - s + W.
 * sinks = 0 is the sliding window.  idx may be NULL if k' == 0.
 * Errors: KVC_ERR_SHAPE (B, Hkv < 1, W < 1, W > n, sinks < 0), KVC_ERR_NULL,
 *   KVC_ERR_HIP. */
kvc_status kvc_select_recent(int32_t B, int32_t Hkv, int32_t n, int32_t W, int32_t budget, int32_t sinks,
                             int32_t *idx, void *stream);

/* ------------------------------------------------------------------ prefill
 * Causal prefill attention with the attention accumulated by each key (MiniKV
 * Sec. 4.3 "Selective KV Compatible Attention Kernels", Fig. 9: FlashAttention
 * that also returns A_cumul along each key column, O(l_key) extra memory).
 * For query head h (KV head j = h / (Hq/Hkv)) and row r:
 *   out[b][h][r] = softmax over keys c <= r of q_r . k_c / sqrt(D), times V;
 *   acc[b][j][c] = sum over the Hq/Hkv heads of KV head j and the rows r >= c
 *                  of that softmax's probability of key c (the normalized
 *                  probabilities: H2O's accumulated attention, blog
 *                  "Eviction"; MiniKV's kernel omits the row normalization to
 *                  save the per-row state, kept here as the workspace);
 *   var[b][j]    = population variance of acc[b][j][0..n) (MiniKV Sec. 4.2 and
 *                  Fig. 7: Var(A_cumul)), float64 sums as kvc_window_scores.
 *   q [B][Hq][n][D], k, v [B][Hkv][n][D] in dtype (post-RoPE); out
 *   [B][Hq][n][D] float32; acc [B][Hkv][n] float32 or NULL (no column sums);
 *   var [B][Hkv] float32 or NULL (needs acc).  D in {32, 64, 128}.
 *   lse [B][Hq][n] float32 or NULL: each row's log-sum-exp, natural log, of its
 *                  causal logits q_r . k_c / sqrt(D) over c <= r (the softmax
 *                  normalizer FlashAttention keeps; kvc_select_lse takes the
 *                  last W rows of it).
 * Workspace: the per-row log-sum-exp, B*Hq*n floats (ws == NULL: size query).
 * acc is written in a fixed order (no atomics): the same inputs give the same
 * bits.
 * Errors: KVC_ERR_NULL (q, k, v or out NULL, var without acc), KVC_ERR_DTYPE,
 *   KVC_ERR_SHAPE (B, Hq, Hkv, n < 1, Hq % Hkv, D not 32/64/128),
 *   KVC_ERR_WORKSPACE, KVC_ERR_HIP. */
kvc_status kvc_prefill_attn(const void *q, const void *k, const void *v, kvc_dtype dtype, int32_t B, int32_t Hq,
                            int32_t Hkv, int32_t n, int32_t D, float *out, float *acc, float *var, float *lse,
                            void *ws, size_t *ws_bytes, void *stream);

/* kvc_select_h2o: heavy-hitter selection (blog "Eviction: keep fewer tokens":
 * H2O keeps the tokens with the largest accumulated attention plus a recent
 * window; PyramidKV "Baselines").  As kvc_select, the window [n-W, n) is always
 * kept and the k' = min(budget, n-W) largest of acc[b][j][0..n-W) are taken
 * (ties to the lower position, no pooling), ascending, into idx [B][Hkv][k']
 * int32; budget < 0 keeps all n-W.  acc [B][Hkv][n] float32 as written by
 * kvc_prefill_attn (rows n apart).  idx may be NULL if k' == 0.
 * Errors: KVC_ERR_NULL, KVC_ERR_SHAPE (B, Hkv < 1, W < 1, W > n),
 *   KVC_ERR_WORKSPACE, KVC_ERR_HIP. */
kvc_status kvc_select_h2o(const float *acc, int32_t B, int32_t Hkv, int32_t n, int32_t W, int32_t budget,
                          int32_t *idx, void *ws, size_t *ws_bytes, void *stream);

/* ------------------------------------------------------------------ quantize
 * Prompt compression into an empty cache (MiniKV Alg. 1 prefill: heavy
 * hitters, then Quant; Sec. 4.4 INT2 quantization kernel; blog
 * "Quantization": keys per channel, values per token, recent tokens in full
 * precision until a group fills).  The kept tokens of each (b, KV head) are
 * idx[b][j][0..k_sel) followed by the window n-W..n-1 (T = k_sel + W), or all n
 * prompt tokens when idx == NULL (T = n).  The oldest Q = g*floor(max(T-R,0)/g)
 * (g*floor(T/g) with flush_all)
 * are quantized: per group of g values, lo/hi -> scale = fp16((hi-lo)/(2^b-1)),
 * zero = fp16(lo), code = clamp(rint((x - zero) * (1/scale)), 0, 2^b-1) in IEEE
 * float32 (a zero or non-finite scale gives codes 0; inputs must be finite);
 * the last T-Q go to the residual as bf16.
 *   k, v [B][Hkv][n][D] dtype; idx [B][Hkv][k_sel] int32 (ascending, < n-W) or
 *   NULL; cache: batch/kv_heads/head_dim/bits/residual/capacities/pointers set,
 *   q_len == r_len == 0.  On success cache->q_len = Q, cache->r_len = T-Q,
 *   cache->r_start = 0.
 * Errors: KVC_ERR_NULL, KVC_ERR_DTYPE, KVC_ERR_BITS, KVC_ERR_SHAPE,
 *   KVC_ERR_CAPACITY (cache not empty, Q > q_cap, T-Q > r_cap or
 *   r_cap < R+g), KVC_ERR_HIP.  KVC_ERR_BITS also for a group not in {0, 16, 32}. */
kvc_status kvc_quantize(const void *k, const void *v, kvc_dtype dtype, int32_t n, const int32_t *idx,
                        int32_t k_sel, int32_t W, kvc_cache *cache, void *stream);

/* ------------------------------------------------------------------ decode
 * One decode step (MiniKV Eq. 1 and Alg. 1 decoding; blog attention hook):
 * k_new/v_new are appended to the bf16 residual; if the residual then holds
 * R+g tokens its oldest g are quantized (with flush_all: once it holds R tokens
 * all of them are, in groups of g; same arithmetic as kvc_quantize)
 * and appended to the packed history; then for every query head h (KV head
 * h / (Hq/Hkv)) out = softmax(q K^T / sqrt(D)) V over the q_len dequantized
 * history tokens and the r_len residual tokens, one softmax over both.
 *   q [B][Hq][D], k_new, v_new [B][Hkv][D] in dtype; out [B][Hq][D] float32.
 * Group-32 caches run the MFMA kernel; group-16 caches a direct kernel whose
 *   token range is split over workgroups and merged.
 * Workspace: *ws_bytes (ws == NULL query) is sized for q_len == q_cap, so one
 *   buffer serves every step of this cache.
 * Errors: KVC_ERR_NULL, KVC_ERR_DTYPE, KVC_ERR_BITS, KVC_ERR_SHAPE,
 *   KVC_ERR_CAPACITY (r_len+1 > r_cap, or a flush past q_cap),
 *   KVC_ERR_WORKSPACE, KVC_ERR_HIP. */
kvc_status kvc_decode_attn(kvc_cache *cache, const void *q, const void *k_new, const void *v_new,
                           kvc_dtype dtype, int32_t Hq, float *out, void *ws, size_t *ws_bytes,
                           void *stream);

/* The same decode step for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the scratch that kvc_decode_attn takes from `ws` comes from a
 * static device array inside the library, one per device, 16 MiB, reached
 * through hipGetSymbolAddress once per device.  No allocating call is made; the
 * caller still passes q, k_new, v_new and out.  Results and cache updates are
 * those of kvc_decode_attn.  Calls that overlap on one device share the array
 * and race (serialize them, e.g. on one stream); nothing in it needs clearing
 * between calls.
 * Errors: as kvc_decode_attn, with KVC_ERR_WORKSPACE when this call's split
 *   partials (units x splits x 4 heads x (D + 2) floats) exceed 16 MiB; the
 *   per-device address lookup failing gives KVC_ERR_HIP. */
kvc_status kvc_decode_attn_noalloc(kvc_cache *cache, const void *q, const void *k_new, const void *v_new,
                                   kvc_dtype dtype, int32_t Hq, float *out, void *stream);

/* hipError_t of the last failed HIP call on this thread (0 if none). */
int kvc_last_hip_error(void);

/* Static text for a status code. */
const char *kvc_status_string(kvc_status s);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H */
