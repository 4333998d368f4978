/*
 * h2o.h -- C ABI of the H2O budgeted-attention library for AMD MI355X (gfx950).
 *
 * H2O keeps, per attention head, a fixed budget of k cached tokens: a
 * heavy-hitter region (the tokens that have received the most attention so
 * far) plus a window of the most recent tokens.  Each generated token attends
 * over the cached entries only, every entry adds the attention it just received
 * to a running score, and once the cache is full one entry is evicted per head
 * per step and the new token's K/V overwrite its slot in place.
 *
 * Sources (page title, then section):
 *   [Report] "H2O: Heavy-Hitter Oracle for Efficient Generative Inference of
 *            Large Language Models -- 深度解读报告" (zako-mio llm-papers-knowledge-base)
 *            §3.1 budgeted generation, §3.3 eviction rule (the paper's
 *            Definition 4.3 / Algorithm 1), §3.4 system layout, prefill rule and
 *            decode rule.
 *   [Card]   "H2O: Heavy-Hitter Oracle for Efficient Generative Inference of
 *            Large Language Models" (phantomic12 inference-research paper card):
 *            accumulated-attention score per token, lowest-scoring entries evicted.
 *
 * Conventions for every entry point:
 *   - A *unit* is one (batch element, head); units are independent and laid out
 *     batch-major: unit = b * heads + h.
 *   - Positions are 0-based int32.  Step i (the i-th token overall) is the token
 *     at position i; a prompt of L tokens occupies positions 0..L-1.
 *   - "device" pointers are HBM addresses on the cache's GPU (e.g. a torch
 *     tensor's data_ptr()); "host" pointers are CPU memory.  All buffers are
 *     dense row-major, 16-byte aligned, and owned by the caller; they must stay
 *     valid until the stream has passed the call.
 *   - stream: a hipStream_t on the cache's device, or NULL for the null stream.
 *     Calls are asynchronous unless stated otherwise.  Each call makes the
 *     cache's device current for its duration and restores the caller's device
 *     on return; if the device cannot be made current the call returns
 *     H2O_ERR_HIP before any other work.
 *   - Return codes only: nothing throws across the ABI and nothing exits the
 *     process.  Argument and state checks run before any GPU work; when one
 *     fails the cache is left unchanged.  A fault inside an already-queued kernel
 *     is reported as H2O_ERR_HIP by a later call (h2o_cache_read synchronises);
 *     after it the cache contents are undefined and the cache should be
 *     destroyed.
 *   - One cache serves one stream from one host thread at a time; distinct
 *     caches are independent.  A model with several layers uses one cache per
 *     layer.
 */
#ifndef H2O_H_
#define H2O_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct h2o_cache h2o_cache; /* opaque; owns all of its device memory */

typedef enum {
  H2O_F32 = 0,  /* float32 inputs and cached K/V */
  H2O_BF16 = 1  /* bfloat16 inputs and cached K/V (fp32 arithmetic) */
} h2o_dtype;

typedef enum {
  H2O_OK = 0,
  H2O_ERR_INVALID_ARG = 1, /* bad pointer, size, alignment or parameter */
  H2O_ERR_STATE = 2,       /* call not valid in the cache's current state */
  H2O_ERR_OOM = 3,         /* device allocation failed */
  H2O_ERR_HIP = 4,         /* HIP runtime error (launch failure, async fault) */
  H2O_ERR_UNSUPPORTED = 5  /* a valid request the library does not implement */
} h2o_status;

typedef struct {
  int32_t batch;         /* B >= 1 */
  int32_t heads;         /* H >= 1 */
  int32_t head_dim;      /* d in {64, 128} */
  int32_t heavy_budget;  /* K_h >= 0: heavy-hitter entries kept per unit */
  int32_t recent_budget; /* K_r >= 0: most recent positions always kept */
  int32_t dtype;         /* h2o_dtype */
  float scale;           /* logit scale; <= 0 selects 1/sqrt(head_dim) */
  int32_t max_prompt;    /* >= 0: longest prompt h2o_prefill will accept */
  float rope_base;       /* > 0: rotary position embedding at positions inside
                            the cache, frequencies rope_base^(-2m/d); 0: none */
} h2o_params;
/* Position rolling (Report §4.4, Q1: H2O with position rolling streams 4 million
 * tokens).  With rope_base > 0 the caller passes unrotated queries and keys and
 * the cache keeps keys unrotated; the library rotates them (pairs (m, m + d/2),
 * angle p * rope_base^(-2m/d)) to positions *inside the cache*: at a decode step
 * the attended entries (the cached ones and the new token) take the positions
 * 0, 1, ... in order of their text positions, the new token the last one, so a
 * logit depends on how many entries lie between query and key rather than on
 * their distance in the text.  The prompt, attended before anything is
 * evicted, is rotated to its own positions 0..L-1: each rotated value is
 * computed in float32 (x*c - y*s, x*s + y*c from float32 cosines and sines of
 * double-precision angles) and, for bf16 caches, carried into the score
 * products as two bf16 parts hi = bf16(v), lo = bf16(v - hi) (three products
 * per pair of operands), so the prompt's scores follow the exact rotation to
 * fp32-level error.  The prompt is rotated chunk by chunk of units into a
 * scratch area of at most 512 MiB (or 8 units, if larger).  Decode rotations
 * are done in float32 without rounding.  rope_base must be finite and >= 0. */
/* The budget is k = K_h + K_r >= 1 (Report §3.1: k < n cached tokens).
 * B*H*max(k, max_prompt) must stay below 2^31, and one unit's prompt matrix,
 * max_prompt*d*sizeof(dtype), below 2^32 bytes. */

/* Device bytes that h2o_cache_create would allocate for these parameters.
 * kv_bytes (nullable): the cached K and V slots alone, 2 * B*H*k*d*sizeof(dtype).
 * total_bytes (nullable): everything, including per-slot scores, positions and
 * prefill/decode scratch.  Host-only; makes no GPU call.
 * Errors: H2O_ERR_INVALID_ARG for invalid parameters. */
h2o_status h2o_cache_bytes(const h2o_params* params, size_t* kv_bytes, size_t* total_bytes);

/* Create an empty cache on `device` (-1: the calling thread's current device).
 * Allocates all device memory up front (Report §3.4: the cache is preallocated
 * and later overwritten in place); no later call allocates.  *out receives the
 * cache, or NULL on failure.
 * Errors: H2O_ERR_INVALID_ARG (params, out == NULL), H2O_ERR_UNSUPPORTED
 * (head_dim not 64/128), H2O_ERR_OOM, H2O_ERR_HIP. */
h2o_status h2o_cache_create(const h2o_params* params, int device, h2o_cache** out);

/* Release the cache and its device memory.  Synchronises the device.  NULL is
 * accepted and ignored. */
h2o_status h2o_cache_destroy(h2o_cache* cache);

/* Prefill (Report §3.4, prefill rule).  (Re)initialises the cache from a prompt
 * of `prompt_len` tokens.
 *   q, k, v: device, [B, H, prompt_len, d] in the cache dtype.
 *   out:     device, nullable, [B, H, prompt_len, d] float32: when non-NULL it
 *            receives the prompt's own attention output o_r = sum_{j<=r} a_rj v_j
 *            (every prompt row attends fully; eviction starts after the prompt).
 *            bf16 caches round the softmax terms to bf16 before the product
 *            with V and normalise in float32 afterwards.  Asking for it leaves
 *            the cache and the statistics bit-identical to a call without it.
 * For each unit: every prompt row r attends causally (positions 0..r, itself
 * included) with a = softmax(scale * q_r . k_j); token j's score is the total
 * attention it receives, c_j = sum_{r >= j} a_rj (Report §2.3, §3.3).  If
 * prompt_len <= k all tokens are kept; otherwise the last K_r positions are kept
 * plus the K_h best-scored of positions [0, prompt_len - K_r), ranked by score,
 * equal scores ranked by position (the higher position wins).  Kept tokens'
 * K/V rows are copied into slots with their scores; the step counter is set to
 * prompt_len.  prompt_len == 0 gives an empty cache.  q/k/v/out may be NULL when
 * prompt_len == 0.
 * Errors: H2O_ERR_INVALID_ARG (NULL or misaligned pointers, prompt_len < 0 or
 * > max_prompt), H2O_ERR_HIP. */
h2o_status h2o_prefill(h2o_cache* cache, const void* q, const void* k, const void* v,
                       int32_t prompt_len, float* out, void* stream);

/* One decode step for every unit (Report §3.1, §3.3, §3.4 decode rule; Card).
 *   q, k, v: device, [B, H, d] in the cache dtype: the new token (position i,
 *            the cache's step counter) of every unit.
 *   out:     device, [B, H, d] float32: attention output over the cached entries
 *            plus the new token, normalised over those entries only.
 *   evicted: device, [B, H] int32, nullable: the position evicted this step, or
 *            -1 when the cache was not yet full.  With K_r == 0 it may be i
 *            itself (the new token is then not stored).
 * Then every cached entry adds its weight to its score (the new token's score
 * starts at its own weight).  While fewer than k entries are cached the new
 * token is added to a free slot.  Otherwise the victim is the entry with the
 * lowest score among the heavy hitters and the token leaving the recent window
 * (positions <= i - K_r), the lowest position on equal scores; the new token's
 * K/V, position and score overwrite the victim's slot.  The caller may reuse
 * q/k/v once the stream has passed the call.
 * Errors: H2O_ERR_INVALID_ARG (NULL or misaligned pointers), H2O_ERR_STATE (no
 * prefill yet, or the position counter would overflow int32), H2O_ERR_HIP. */
h2o_status h2o_decode_step(h2o_cache* cache, const void* q, const void* k, const void* v,
                           float* out, int32_t* evicted, void* stream);

/* Several decode steps whose tokens are all known in advance: a known text
 * streamed through the cache (the Report §4.4 Q1 streaming evaluation reads a
 * book token by token), or one layer of a model run chunk by chunk over such a
 * text.  Exactly `steps` h2o_decode_step calls, step t taking token t, with
 * bit-identical results.
 *   q, k, v: device, [steps, B, H, d] in the cache dtype.
 *   out:     device, float32: step t writes its [B, H, d] output at
 *            out + t * out_step (elements; a multiple of 4); out_step == 0
 *            leaves the last step's output.
 *   evicted: device, [steps, B, H] int32, nullable: each step's evicted
 *            position (as h2o_decode_step).
 * steps == 0 does nothing.  Arguments and state are checked once, before the
 * first step.
 * Errors: as h2o_decode_step; H2O_ERR_INVALID_ARG also for steps < 0 or a
 * negative or misaligned out_step; H2O_ERR_STATE when the position counter
 * would pass INT32_MAX within the steps. */
h2o_status h2o_decode_steps(h2o_cache* cache, const void* q, const void* k, const void* v, int32_t steps,
                            float* out, int64_t out_step, int32_t* evicted, void* stream);

/* Copy the cache contents to host memory; synchronises `stream` first and
 * reports any earlier asynchronous fault.  Every pointer is host and nullable.
 *   pos:     [B, H, k] int32, the position held by each slot, -1 for empty slots
 *   score:   [B, H, k] float32, the accumulated score of each slot: the
 *            device keeps it as a Kahan pair (sum s, compensation c), and the
 *            value written here is s - c rounded to float32
 *   k_slots, v_slots: [B, H, k, d] in the cache dtype
 *   meta:    int32[2] = {entries cached per unit, next position}
 * Slot order within a unit carries no meaning; compare by position.
 * Errors: H2O_ERR_INVALID_ARG, H2O_ERR_HIP. */
h2o_status h2o_cache_read(h2o_cache* cache, int32_t* pos, float* score, void* k_slots,
                          void* v_slots, int32_t* meta, void* stream);

/* Copy the last h2o_prefill's per-token statistics to host memory (synchronises
 * `stream`).  Each pointer is host, nullable, [B, H, L] float32 with L the last
 * prompt_len:
 *   row_lse: log sum_j exp(scale*q_r.k_j) over j <= r, the natural log of the
 *            normaliser of prompt row r's causal softmax
 *   col_sum: c_j, the attention token j received from the prompt rows
 * Errors: H2O_ERR_INVALID_ARG, H2O_ERR_STATE (no h2o_prefill yet, or an
 * h2o_column_scores / h2o_prefill_scored call since), H2O_ERR_HIP. */
h2o_status h2o_prefill_stats_read(h2o_cache* cache, float* row_lse, float* col_sum, void* stream);

/* ---- Global-score comparator (Report §2.3 and its Figure 2(d): the greedy
 * local score against a "global" one computed from the full attention of the
 * whole sequence).  The three calls below run the same budgeted attention and
 * the same keep/evict rule as h2o_prefill / h2o_decode_step, but rank tokens by
 * scores the caller supplies and fixes in advance; nothing accumulates.  The
 * global comparator is: h2o_column_scores over all N = L + T tokens, then
 * h2o_prefill_scored with the first L scores, then h2o_decode_step_scored with
 * score[i] at step i. */

/* Column scores of a whole sequence: c_j = sum_{r >= j} a_rj with a the causal
 * softmax of all n rows (the score H2O would give token j if every row of the
 * sequence were known in advance).  Computed with the prefill's two passes.
 *   q, k:   device, [B, H, n, d] in the cache dtype.
 *   scores: device, [B, H, n] float32, written.
 * Uses the cache's prefill scratch (n <= max_prompt) and leaves the cached
 * entries untouched; afterwards h2o_prefill_stats_read reports H2O_ERR_STATE
 * until the next h2o_prefill.  n == 0 does nothing (pointers may be NULL).
 * Errors: H2O_ERR_INVALID_ARG (NULL or misaligned pointers, n < 0 or
 * n > max_prompt), H2O_ERR_HIP. */
h2o_status h2o_column_scores(h2o_cache* cache, const void* q, const void* k, int32_t n, float* scores,
                             void* stream);

/* h2o_column_scores for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops that forbid hipMalloc): the same column
 * scores of a whole sequence, with no cache object.  Its scratch (each row's
 * softmax normaliser and the column sums, batch*heads*round32(n)*8 bytes, at
 * most 16 MiB) is a file-scope device array of the library rather than an
 * allocation; the call allocates nothing, host or device, after the first call
 * on a device (which looks the array up).
 *   params: batch, heads, head_dim, dtype and scale are used (budgets and
 *           max_prompt are ignored); rope_base must be 0.
 *   q, k:   device, [B, H, n, d] in params->dtype, on the current device.
 *   scores: device, [B, H, n] float32, written (stream-ordered).
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (on different streams or threads) race and must be serialised by the caller.
 * The array keeps the last call's contents; no call reads a value it has not
 * first written, so nothing needs clearing.  n == 0 does nothing.
 * Errors: H2O_ERR_INVALID_ARG (NULL params or pointers, misaligned pointers,
 * n < 0, or the scratch limit exceeded), H2O_ERR_UNSUPPORTED (head_dim not 64
 * or 128, rope_base != 0), H2O_ERR_HIP. */
h2o_status h2o_column_scores_noalloc(const h2o_params* params, const void* q, const void* k, int32_t n,
                                     float* scores, void* stream);

/* Prefill by given scores: (re)initialise the cache from a prompt of
 * `prompt_len` tokens exactly as h2o_prefill does (last K_r positions plus the
 * K_h best of [0, prompt_len - K_r), equal scores ranked by position), but
 * ranking by `scores` instead of the prompt's own column sums; the kept slots'
 * scores are set to them.  The prompt is the first prompt_len rows of each
 * unit's `seq_rows` rows (e.g. the whole sequence's K/V and column scores):
 *   k, v:   device, [B, H, seq_rows, d] in the cache dtype.
 *   scores: device, [B, H, seq_rows] float32, finite and >= 0 (the first
 *           prompt_len of each unit are read).
 * No attention is computed; prompt_len may exceed max_prompt.  Afterwards
 * h2o_prefill_stats_read reports H2O_ERR_STATE.  prompt_len == 0 gives an empty
 * cache (pointers may be NULL).
 * Errors: H2O_ERR_INVALID_ARG (NULL or misaligned pointers, prompt_len < 0,
 * seq_rows < prompt_len), H2O_ERR_HIP. */
h2o_status h2o_prefill_scored(h2o_cache* cache, const void* k, const void* v, int32_t prompt_len,
                              int32_t seq_rows, const float* scores, void* stream);

/* One decode step with fixed scores: attention and output exactly as
 * h2o_decode_step, but no entry's score changes; the new token's score is
 * new_score[unit * score_stride] (device float32, finite and >= 0; stride 1 for
 * a [B, H] array, n with the column scores of a [B, H, n] sequence offset to
 * this step's position), and the victim is the candidate with the lowest score
 * (lowest position on equal scores).
 * Errors: as h2o_decode_step, and H2O_ERR_INVALID_ARG for a NULL or misaligned
 * new_score or score_stride < 1. */
h2o_status h2o_decode_step_scored(h2o_cache* cache, const void* q, const void* k, const void* v,
                                  const float* new_score, int32_t score_stride, float* out, int32_t* evicted,
                                  void* stream);

/* ---- Heavy hitters added to a sparse attention pattern (Report §4.5, Table 2:
 * strided and fixed Sparse-Transformer patterns, each improved by adding H2). */
typedef enum {
  H2O_PATTERN_NONE = 0,    /* plain H2O (the default) */
  H2O_PATTERN_STRIDED = 1, /* at step i, the positions j with (i - j) mod period == 0 */
  H2O_PATTERN_FIXED = 2    /* the last `width` positions of every block of `period`:
                              j mod period >= period - width */
} h2o_pattern;

/* Keep a sparse pattern in preference to heavy hitters, for every later
 * h2o_prefill / h2o_prefill_scored / h2o_decode_step / h2o_decode_step_scored
 * call on this cache.  The budget and the recent window are unchanged; among
 * the eviction candidates (and the prefill's heavy-hitter pool, judged for the
 * first generated token i = prompt_len) the entries the pattern protects are
 * kept first and the heavy hitters fill the rest: the victim is the lowest
 * (protected, score, position), so a protected entry is evicted only when every
 * candidate is protected.  An evicted token never returns, so the pattern is
 * honoured as far as the cache still holds its positions.  width is ignored for
 * H2O_PATTERN_STRIDED; H2O_PATTERN_NONE ignores both.  Host-side, no GPU call.
 * Errors: H2O_ERR_INVALID_ARG (unknown kind, period < 1, width outside
 * [1, period] for H2O_PATTERN_FIXED). */
h2o_status h2o_cache_set_pattern(h2o_cache* cache, int32_t kind, int32_t period, int32_t width);

/* Host-side state, no GPU call: entries cached per unit, next position, and the
 * last prompt length (-1 before the first prefill).  Pointers nullable. */
h2o_status h2o_cache_info(const h2o_cache* cache, int32_t* count, int32_t* next_pos,
                          int32_t* prompt_len);

/* Static description of a status code. */
const char* h2o_status_str(h2o_status status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char* h2o_last_error(void);

/* Measurement aid, not part of the method: read `bytes` of device memory at
 * `buf` once, as a plain stream (16-byte non-temporal loads, 8 in flight per
 * lane, 16 blocks of 256 threads per compute unit, each block on contiguous
 * 32 KiB runs), on `stream`.  Timing it gives the streaming-read bandwidth the GPU sustains,
 * the practical ceiling for the decode kernel.  `sink` (device, 4 bytes) is
 * written with probability 2^-32 only (it keeps the loads alive).
 * Errors: H2O_ERR_INVALID_ARG (NULL pointers, buf or bytes not a multiple of
 * 16), H2O_ERR_HIP. */
h2o_status h2o_probe_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* Measurement aid, not part of the method: the instruction mix of a prefill
 * scoring pass from registers alone, on `stream`.  Every wave (4 blocks of 256
 * threads per compute unit, 4 waves per SIMD) runs `iters` iterations of
 * 16 MFMAs 32x32x16 bf16 (mode 0 and 1) and, per lane, 32 times one fma, one
 * exp2 and one add on values independent of the matrix results (mode 1 and 2):
 * the arithmetic of one 64 x 32 logit tile at d = 128, with no memory traffic
 * and no barriers.  Timing mode 0, 1 and 2 gives the matrix rate, the rate of
 * the mix and the vector rate this GPU sustains; a mode-0 or mode-1 launch
 * executes (compute units) * 16 waves * iters * 16 * 32768 MFMA flops.  `sink`
 * (device, 4 bytes) is written with probability 2^-32 only.
 * Errors: H2O_ERR_INVALID_ARG (mode not 0-2, iters < 1, NULL sink),
 * H2O_ERR_HIP. */
h2o_status h2o_probe_mix(int32_t mode, int32_t iters, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* H2O_H_ */
