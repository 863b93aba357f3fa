/*
 * kivi.h — C ABI of the MI355X (gfx950) KIVI-style quantized KV cache.
 *
 * Keys are quantized per channel over groups of G consecutive tokens and Values per
 * token over groups of G_v consecutive channels, each group to 2 or 4 bits with an
 * asymmetric min/max float16 scale and zero.  The most recent tokens stay in a
 * float16 residual window that is flushed into the quantized store when it is full.
 * Decode attention reads the packed cache directly.
 *
 * Sources (page titles; sections):
 *   "KV Cache Quantization (KIVI & FP4): How 2-Bit Key-Value Compression Scales LLM
 *    Contexts to 1 Million Tokens" — §3 (per-channel Keys, per-token Values, FP16
 *    residual window), §4 (four 2-bit codes per byte, dequantization fused into the
 *    attention kernel), §6 (prefill stays high precision, then a streaming pass
 *    stores low-bit codes).
 *   "09 — KV Cache Quantization" — "KIVI — the reference paper" (fp16 scale and zero
 *    per channel, int2/int4 storage, residual buffer), "Per-channel vs per-token in
 *    the actual attention kernel" (dequantize inside the attention tile loop, never
 *    into a full fp16 buffer).
 *   "KIVI: A Tuning-Free Asymmetric 2bit Quantization for KV Cache" — "The streaming
 *    complication" (complete groups quantized once and frozen).
 *   "4.4 KV Cache quantization" — §1 (M_KV = 2 L B T H_KV d b and its arguments),
 *    §3.1 (the two grouping directions, min/max asymmetric mapping inside a group),
 *    §3.2 (residual cache joins attention and is moved into the history in a batch).
 *   "KV Cache INT4 Quantization for 1M+ Token Context Windows" — §2 (unsigned codes
 *    in [0, 2^b - 1], scale from the group range, two 4-bit codes per byte).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All cache buffers, inputs and outputs are DEVICE pointers owned by the caller.
 *    The library never allocates or frees device memory and keeps no state between
 *    calls except a thread-local error message.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and the call
 *    returns without synchronizing.  Buffers must stay valid until the stream has
 *    passed the enqueued work.  Calls are reentrant; calls that write the same cache
 *    layer must be ordered by the caller (same stream or events).
 *  - Arguments are validated before anything is enqueued.  On any status other than
 *    KIVI_OK nothing was enqueued (except KIVI_ERR_DEVICE, returned when the HIP
 *    runtime rejected a launch) and kivi_last_error() describes the problem.
 *  - Device pointers must be 16-byte aligned.  Inputs must be finite.
 *  - Index arithmetic is 64-bit; a layer may hold more than 4 GiB.
 *
 * Cache layout (every buffer has a leading [layers] dimension; all row-major):
 *    k_codes  uint8   [L][B][H_kv][T_max][d*b/8]       per token, channels packed
 *    k_scale  float16 [L][B][H_kv][T_max/G][d]         per (Key group, channel)
 *    k_zero   float16 [L][B][H_kv][T_max/G][d]
 *    v_codes  uint8   [L][B][H_kv][T_max/16][d][2*b]   per channel, runs of 16 tokens
 *    v_scale  float16 [L][B][H_kv][T_max][d/G_v]       per (token, Value group)
 *    v_zero   float16 [L][B][H_kv][T_max][d/G_v]
 *    k_resid  float16 [L][B][H_kv][S + R][d]           rows [0, S): the sink tokens;
 *    v_resid  float16 [L][B][H_kv][S + R][d]           rows [S, S + R): the window ring
 *    scale_max float32 [L][B][H_kv][2]                 largest Key scale [0] and
 *             Value scale [1] in the quantized history (kept by the calls below)
 *  Packed runs are little-endian 32-bit words of n = 32/b codes: code j of a run is
 *  code e = j mod n of word j / n, which sits in byte e mod 4 of the word at bits
 *  [b*(e / 4), b*(e / 4) + b).  (Four 2-bit or two 4-bit codes per byte.)
 *
 * Quantizer (per group of float16 values x_i; float32 arithmetic, IEEE division,
 * round-half-to-even):  x_i += 0 (so -0 becomes +0);  mn = min x_i;  mx = max x_i;
 *  scale = float16_rne((mx - mn) / (2^b - 1));  zero = float16(mn) (exact);
 *  s = float(scale);  code_i = s == 0 ? 0 : clamp(rint((x_i - mn) / s), 0, 2^b - 1).
 *  Dequantized value: code * scale + zero.
 *
 * Residual window: after T tokens it holds r(T) tokens and the quantized history
 * holds T_q(T) = T - r(T).  With aging = KIVI_AGING_WINDOW (default),
 * r(T) = T == 0 ? 0 : ((T - 1) mod R) + 1: an append at r == R first quantizes all R
 * window tokens into the history.  With aging = KIVI_AGING_GROUP ("KIVI: A
 * Tuning-Free ...", "The streaming complication": a completed Key group is quantized
 * once, the newest tokens stay float16 until they age out), r(T) = T for T <= R and
 * R - G + ((T - R - 1) mod G) + 1 after: an append at r == R first quantizes only
 * the oldest G window tokens.  The window is a ring over its R rows: token T_q + i
 * (i < r) sits in window row (T_q + i) mod R, so the flushed tokens' rows are
 * reused by the newest ones; under KIVI_AGING_WINDOW T_q is a multiple of R and
 * token T_q + i is in row i.  Prefill of T tokens gives the same bytes as T appends.
 * All sequences of a batch share T.
 *
 * Value window (flags & KIVI_FLAG_VALUE_TOKEN_WINDOW; "4.4 KV Cache quantization" §3.2:
 * each new Value enters the float16 window and pushes the oldest one out, which is
 * quantized on its own): Keys keep the rule above, Values have a window of their own.
 * After T tokens it holds the min(T, R) most recent Values, and the quantized Values
 * are history tokens [0, T_qv(T)) with T_qv(T) = max(T - R, 0) <= T_q(T).  Value token
 * i (T_qv <= i < T) sits in window row i mod R, the row of Key token i, so v_resid row
 * i mod R holds Value i whether or not Key i is still in the window.  An append at
 * T >= R first quantizes Value T - R (its G_v groups, the quantizer above) into
 * history token T - R and then stores the new row.  A 16-token Value run fills token
 * by token: codes of tokens not yet quantized are 0, their scale and zero rows untouched.
 * Uniform batches in contiguous caches only (the ragged and paged calls return
 * KIVI_ERR_UNSUPPORTED).
 *
 * Grouped-query attention: query head j reads KV head j / (H_q / H_kv).
 */
#ifndef KIVI_H
#define KIVI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kivi_status {
  KIVI_OK = 0,
  KIVI_ERR_ARG = 1,          /* a bad argument (null pointer, bad layer, bad sizes) */
  KIVI_ERR_UNSUPPORTED = 2,  /* a valid configuration this build has no kernel for */
  KIVI_ERR_CAPACITY = 3,     /* the token count does not fit max_tokens */
  KIVI_ERR_ALIGN = 4,        /* a device pointer is not 16-byte aligned */
  KIVI_ERR_WORKSPACE = 5,    /* the decode workspace is null or too small */
  KIVI_ERR_DEVICE = 6        /* the HIP runtime rejected a launch */
} kivi_status;

#define KIVI_AGING_WINDOW 0   /* a full window is flushed whole */
#define KIVI_AGING_GROUP 1    /* a full window sends only its oldest Key group out */

/* kivi_dims.flags.
 * KIVI_FLAG_DETERMINISTIC: decode calls give the same output bits whenever they are
 *   repeated with the same arguments.  Every wave of a workgroup then takes a fixed
 *   round-robin share of the 64-token blocks instead of taking them from a queue as it
 *   runs (measured 0-7% slower per step whole job, the 70B shape the most).  Without it,
 *   repeated calls agree to float32 rounding.
 * KIVI_FLAG_VALUE_TOKEN_WINDOW: the per-token Value window ("4.4 KV Cache quantization"
 *   §3.2: each new Value pushes the oldest one out, quantized on its own); see "Value
 *   window" below. */
#define KIVI_FLAG_VALUE_TOKEN_WINDOW 1
#define KIVI_FLAG_DETERMINISTIC 2

/* Problem statement of one cache ("4.4 KV Cache quantization" §1 and §3: layers,
 * batch, KV heads, head_dim, bits, group size, residual length).
 *
 * Sink tokens ("09 — KV Cache Quantization", "Anti-patterns": the first tokens of a
 * sequence absorb large attention scores and must not be quantized; preserve the
 * first N): with sink = S, tokens [0, S) of every sequence stay in float16 for its
 * lifetime (residual rows [0, S)), and every rule of this header — groups, window,
 * flushes, T_q and r — applies to the tokens after them, counted from S:
 * T_q(T) and r(T) below mean T_q(T - S) and r(T - S) for T > S (0 for T <= S), and
 * history token i is token S + i of the sequence. */
typedef struct kivi_dims {
  int32_t layers;      /* L >= 1 */
  int32_t batch;       /* B >= 1 */
  int32_t kv_heads;    /* H_kv >= 1 */
  int32_t q_heads;     /* H_q, a multiple of H_kv with H_q / H_kv in {1, 2, 4, 8} */
  int32_t head_dim;    /* d; this build supports 128 */
  int32_t bits;        /* b in {2, 4} */
  int32_t group_k;     /* G: tokens per Key group, in {16, 32, 64} */
  int32_t group_v;     /* G_v: channels per Value group, divides d, in {16, 32, 64, 128} */
  int32_t residual;    /* R: residual window, a multiple of G and of 16 */
  int32_t sink;        /* S in [0, 1024]: tokens kept in float16 at the start of every
                          sequence (0: none); see "Sink tokens" above */
  int32_t aging;       /* KIVI_AGING_WINDOW or KIVI_AGING_GROUP; see "Residual window" */
  int32_t flags;       /* KIVI_FLAG_* bits below; every other bit must be 0 */
  int64_t max_tokens;  /* T_max: token capacity per sequence, a multiple of G and 16;
                        * a pair's codes (T_max * d * b / 8 bytes) must stay below 2^31
                        * bytes (the kernels' 32-bit buffer offsets), else every call
                        * taking these dims returns KIVI_ERR_UNSUPPORTED */
} kivi_dims;

/* The nine device buffers of a cache; layout above.  scale_max is bookkeeping of
 * this library: the quantize calls reset their half of a layer's entries and every
 * quantizing call raises them to the largest scale it writes; decode reads them to
 * fix its fixed-point exponents.  A cache restored from elsewhere must restore it
 * too (or hold an upper bound of the scales there). */
typedef struct kivi_cache {
  void* k_codes;
  void* k_scale;
  void* k_zero;
  void* v_codes;
  void* v_scale;
  void* v_zero;
  void* k_resid;
  void* v_resid;
  void* scale_max;
} kivi_cache;

#define KIVI_NUM_BUFFERS 9

/* Byte size of each of the nine buffers, in kivi_cache field order, for all
 * layers.  Host-only; enqueues nothing. */
kivi_status kivi_cache_sizes(const kivi_dims* dims, size_t bytes[KIVI_NUM_BUFFERS]);

/* Prefill quantization of the Keys of one layer ("4.4 KV Cache quantization" §3.1:
 * fix a channel, group consecutive tokens; "KV Cache Quantization (KIVI & FP4)" §6:
 * quantize the prompt's cache after prefill).
 *   k      float16 [B][H_kv][ld_tokens][d] device; tokens [0, T) are read.
 *   T      prompt length, 0 <= T <= T_max.
 *   ld     token stride of `k` (>= T).
 * Copies tokens [0, min(T, S)) into rows [0, S) of k_resid, quantizes the next T_q(T)
 * tokens into k_codes/k_scale/k_zero of `layer`, copies the last r(T) tokens into
 * rows [S, S + r(T)) of k_resid and sets the layer's Key entries of scale_max to the
 * largest Key scale written (0 if none). */
kivi_status kivi_quantize_k(const kivi_dims* dims, const kivi_cache* cache, int32_t layer,
                            const void* k, int64_t T, int64_t ld_tokens, void* stream);

/* Prefill quantization of the Values of one layer ("4.4 KV Cache quantization" §3.1:
 * fix a token, group along channels).  Same arguments as kivi_quantize_k, writing
 * v_codes/v_scale/v_zero, v_resid and the Value entries of scale_max. */
kivi_status kivi_quantize_v(const kivi_dims* dims, const kivi_cache* cache, int32_t layer,
                            const void* v, int64_t T, int64_t ld_tokens, void* stream);

/* Append one decode token per sequence to one layer ("KIVI: A Tuning-Free ...", "The
 * streaming complication"; "4.4 KV Cache quantization" §3.2).
 *   T_before   tokens cached before this call (0 <= T_before, T_before + 1 <= T_max).
 *   k_new, v_new  float16 [B][H_kv][d] device.
 * While T_before < S the new row goes to sink row T_before.  Otherwise, if
 * r(T_before) == R the oldest R (KIVI_AGING_WINDOW) or G (KIVI_AGING_GROUP) window
 * tokens are first quantized into the history at history token T_q(T_before) (same
 * arithmetic as the prefill calls); the new row then goes to window row
 * (T_before - S) mod R.  The cache then holds T_before + 1 tokens; a flush
 * raises scale_max to the largest scales it writes. */
kivi_status kivi_append_flush(const kivi_dims* dims, const kivi_cache* cache, int32_t layer,
                              int64_t T_before, const void* k_new, const void* v_new,
                              void* stream);

/* One decode step of a layer: append the new token, then attend over the
 * T_before + 1 cached tokens ("KIVI: A Tuning-Free Asymmetric 2bit Quantization for
 * KV Cache", "The streaming complication": new tokens enter the float16 window and
 * the query attends over history and window).  The result, and the cache it leaves,
 * equal kivi_append_flush(T_before, k_new, v_new) followed by
 * kivi_decode_attn(T = T_before + 1) (outputs to float32 rounding, as between any two
 * decode calls; bit for bit with KIVI_FLAG_DETERMINISTIC).  When r(T_before) < R this
 * is one kernel launch: the attention reads the new row from k_new / v_new and stores
 * it into the window; when the window is full it is the flush launch followed by the
 * decode launch.  With KIVI_FLAG_VALUE_TOKEN_WINDOW the decode launch also quantizes
 * the Value that leaves the window (in the new row's window row, before the row takes
 * the new token), except when that Value completes a 64-token block of the history:
 * that step, like a flush step, is the append launch followed by the decode launch.
 *   Arguments as kivi_append_flush and kivi_decode_attn; the workspace must hold
 *   kivi_decode_workspace_bytes(dims, T_before + 1).
 * Every check of both calls runs before anything is enqueued. */
kivi_status kivi_append_decode(const kivi_dims* dims, const kivi_cache* cache, int32_t layer,
                               int64_t T_before, const void* k_new, const void* v_new,
                               const void* q, float sm_scale, float* out, void* workspace,
                               size_t workspace_bytes, void* stream);

/* kivi_append_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, checks, kernels and results (outputs to float32 rounding, cache bytes
 * equal) without the workspace: the decode's scratch (per-pair arrival counters and
 * split partials) lives in a 4 MiB array of static device memory inside the library,
 * one copy per GPU, held until the process ends.  The library calls no hipMalloc,
 * hipFree or allocating routine here.
 *   The first call on a device looks up that device's copy and enqueues a kernel on
 *   `stream` that zeroes it; every later call leaves the counters at zero again.
 *   A step whose scratch would exceed 4 MiB (kivi_decode_workspace_bytes(dims,
 *   T_before + 1) > 4194304, e.g. beyond ~12,000 (sequence, KV head) pairs) returns
 *   KIVI_ERR_UNSUPPORTED before anything is enqueued.
 *   Every call on one GPU shares that GPU's scratch: calls that may overlap in time
 *   on one GPU (different streams without ordering between them) race and give wrong
 *   results; calls in one stream, or ordered by events, are safe. */
kivi_status kivi_append_decode_noalloc(const kivi_dims* dims, const kivi_cache* cache,
                                       int32_t layer, int64_t T_before, const void* k_new,
                                       const void* v_new, const void* q, float sm_scale,
                                       float* out, void* stream);

/* Paged caches ("KV Cache Quantization (KIVI & FP4)" §6: PagedAttention allocates the
 * cache in fixed pages, and under KIVI a page of the same bytes holds more tokens).
 * The quantized history of every sequence lives in pages of P tokens taken from a
 * pool; the float16 sink and window rows and scale_max stay per (sequence, KV head)
 * as in the contiguous layout.  Each history buffer holds, per layer and KV head, the
 * pool's pages in order, each page laid out like a P-token history:
 *    k_codes  uint8   [L][H_kv][pages][P][d*b/8]
 *    k_scale  float16 [L][H_kv][pages][P/G][d]        k_zero likewise
 *    v_codes  uint8   [L][H_kv][pages][P/16][d][2*b]
 *    v_scale  float16 [L][H_kv][pages][P][d/G_v]      v_zero likewise
 * History token t of sequence b (all its KV heads and layers) is token t mod P of page
 * block_table[b][t / P].  The table is read on the device; an entry outside
 * [0, pages) is clamped into it (every access stays inside the pool; the result is
 * then unspecified).  Pages may be shared by several sequences only where their
 * history is identical; each append writes the page that holds its flushed tokens. */
typedef struct kivi_paging {
  int32_t page_tokens;         /* P: a power of two in [64, 2^20] */
  int32_t pages_per_seq;       /* columns of block_table; pages_per_seq * P >= max_tokens */
  int64_t pages;               /* pages in the pool (per layer and KV head) */
  const int32_t* block_table;  /* device int32 [B][pages_per_seq] */
} kivi_paging;

/* Byte sizes of the nine buffers of a paged cache (layout above; the window buffers
 * and scale_max as in kivi_cache_sizes).  Host-only; block_table is not read. */
kivi_status kivi_paged_cache_sizes(const kivi_dims* dims, const kivi_paging* paging,
                                   size_t bytes[KIVI_NUM_BUFFERS]);

/* Ragged batches ("KV Cache Quantization (KIVI & FP4)" §6: serving engines hold
 * sequences of different lengths in one batch).  Each call below is the call of the
 * same name without _varlen, with sequence b holding its own token count:
 *   lens / T_before  device int32 [B]: tokens of sequence b (decode: 1 <= lens[b];
 *                    prefill: 0 <= lens[b]), or tokens before its append.
 *   T_hi             host upper bound of every entry: the capacity checks, the
 *                    workspace size and the launch are those of the uniform call at
 *                    T = T_hi (appends: T_before = T_hi).
 *   paging           NULL: the cache has the contiguous layout (kivi_cache_sizes);
 *                    else a paged cache (kivi_paged_cache_sizes) and its block table.
 * The arrays are read on the device: the host cannot check them, so each entry is
 * clamped into its valid range ([0, T_hi], decode [1, T_hi]) before use; every access
 * stays inside the cache, and a sequence whose entry was out of range gets an
 * unspecified result.  All heads of a sequence share its count.  The arrays must stay
 * valid until the stream has passed the call; the caller updates them (an append
 * leaves T_before + 1 tokens). */

/* kivi_quantize_k for a ragged batch: sequence b's first lens[b] tokens of k
 * ([B][H_kv][ld_tokens][d], ld_tokens >= T_hi). */
kivi_status kivi_quantize_k_varlen(const kivi_dims* dims, const kivi_cache* cache,
                                   const kivi_paging* paging, int32_t layer, const void* k,
                                   const int32_t* lens, int64_t T_hi, int64_t ld_tokens,
                                   void* stream);
/* kivi_quantize_v for a ragged batch. */
kivi_status kivi_quantize_v_varlen(const kivi_dims* dims, const kivi_cache* cache,
                                   const kivi_paging* paging, int32_t layer, const void* v,
                                   const int32_t* lens, int64_t T_hi, int64_t ld_tokens,
                                   void* stream);
/* kivi_append_flush for a ragged batch: sequence b appends at T_before[b], flushing
 * its own window when that is full.  One launch sized for a flush of every sequence. */
kivi_status kivi_append_flush_varlen(const kivi_dims* dims, const kivi_cache* cache,
                                     const kivi_paging* paging, int32_t layer,
                                     const int32_t* T_before, int64_t T_hi, const void* k_new,
                                     const void* v_new, void* stream);
/* kivi_decode_attn for a ragged batch: sequence b attends over its lens[b] tokens.
 * Workspace: kivi_decode_workspace_bytes(dims, T_hi).  The launch has the workgroups
 * of a batch of T_hi tokens; each (sequence, KV head) splits its own blocks among
 * them, so short sequences finish early. */
kivi_status kivi_decode_attn_varlen(const kivi_dims* dims, const kivi_cache* cache,
                                    const kivi_paging* paging, int32_t layer,
                                    const int32_t* lens, int64_t T_hi, const void* q,
                                    float sm_scale, float* out, void* workspace,
                                    size_t workspace_bytes, void* stream);
/* kivi_append_decode for a ragged batch: two launches (the flushes of the sequences
 * whose window is full, then decode attention that stores every new row); equal to
 * kivi_append_flush_varlen followed by kivi_decode_attn_varlen over T_before[b] + 1.
 * Workspace: kivi_decode_workspace_bytes(dims, T_hi + 1). */
kivi_status kivi_append_decode_varlen(const kivi_dims* dims, const kivi_cache* cache,
                                      const kivi_paging* paging, int32_t layer,
                                      const int32_t* T_before, int64_t T_hi, const void* k_new,
                                      const void* v_new, const void* q, float sm_scale,
                                      float* out, void* workspace, size_t workspace_bytes,
                                      void* stream);
/* kivi_append_decode_varlen, also given T_before_host: a host copy of T_before
 * (int32 [B], owned by the caller, read before the call returns).  A step in which no
 * sequence's residual window is full (most steps: one in R, or one in G with group
 * aging) runs as the decode launch alone; a step with a flush launches both, as
 * kivi_append_decode_varlen does.  The host copy must equal the device one: when it
 * does not, a flush that is due may be skipped and the cache no longer holds KIVI's
 * state, but every access stays inside the cache, since the device lengths still drive
 * the kernels.  The launches are chosen when the call is made: a call captured into a
 * HIP graph replays the launches chosen at capture, so a graph serves only the step
 * (counts) it was captured for.  Returns KIVI_ERR_ARG when T_before_host is NULL or an
 * entry lies outside [0, T_hi], and otherwise the errors of kivi_append_decode_varlen. */
kivi_status kivi_append_decode_varlen_host(const kivi_dims* dims, const kivi_cache* cache,
                                           const kivi_paging* paging, int32_t layer,
                                           const int32_t* T_before,
                                           const int32_t* T_before_host, int64_t T_hi,
                                           const void* k_new, const void* v_new, const void* q,
                                           float sm_scale, float* out, void* workspace,
                                           size_t workspace_bytes, void* stream);

/* Workspace bytes kivi_decode_attn needs for T cached tokens (host-only).  The size
 * never falls as T grows, so a workspace sized for T serves every call at T or fewer
 * tokens. */
kivi_status kivi_decode_workspace_bytes(const kivi_dims* dims, int64_t T, size_t* bytes);

/* Decode attention over the quantized cache of one layer, dequantizing inside the
 * kernel ("09 — KV Cache Quantization", "Per-channel vs per-token in the actual
 * attention kernel"; "KV Cache Quantization (KIVI & FP4)" §2 and §4):
 *   out[b][j][:] = softmax_t(sm_scale * q[b][j] . k_t) v_t over the T cached tokens of
 *   sequence b and KV head j / (H_q / H_kv); k_t, v_t are dequantized codes for the
 *   T_q(T) history tokens and the float16 rows for the sink and the last r(T).
 *   q          float16 [B][H_q][d] device.
 *   out        float32 [B][H_q][d] device.
 *   T          1 <= T <= T_max.
 *   workspace  device scratch of at least kivi_decode_workspace_bytes(dims, T) bytes,
 *              private to the library.  Zero-fill it before its first use with a
 *              given batch and kv_heads; later calls with the same batch and
 *              kv_heads (any T, split count, q_heads or bits that fit) reuse it
 *              without clearing.  Calls that may run concurrently must use
 *              distinct workspaces.
 * No floating-point atomics are used and partials are combined in a fixed order,
 * but which wave of a workgroup takes which 64-token block varies from call to call,
 * so repeated calls agree to float32 rounding, not bit for bit.
 * Value groups: this build's decode kernels require G_v == d (UNSUPPORTED otherwise). */
kivi_status kivi_decode_attn(const kivi_dims* dims, const kivi_cache* cache, int32_t layer,
                             int64_t T, const void* q, float sm_scale, float* out,
                             void* workspace, size_t workspace_bytes, void* stream);

/* As kivi_decode_attn with an explicit number of workgroups per (sequence, KV head)
 * (0 = the library's choice: one round of one workgroup per CU, or fewer when that
 * would leave waves without a 64-token block or float16 chunk to do).  The first
 * workgroup of a pair takes its float16 window and the others split the 64-token
 * blocks of its quantized history, so the count is clamped to [1, 1 + blocks].
 * Workspace size: kivi_decode_workspace_bytes_split. */
kivi_status kivi_decode_attn_split(const kivi_dims* dims, const kivi_cache* cache,
                                   int32_t layer, int64_t T, const void* q, float sm_scale,
                                   float* out, void* workspace, size_t workspace_bytes,
                                   int32_t n_split, void* stream);
kivi_status kivi_decode_workspace_bytes_split(const kivi_dims* dims, int64_t T,
                                              int32_t n_split, size_t* bytes);

/* Number of workgroups per (sequence, KV head) kivi_decode_attn uses for T tokens
 * (at least 1; host-only). */
kivi_status kivi_decode_splits(const kivi_dims* dims, int64_t T, int32_t* n_split);

/* Message for the last non-OK status returned on the calling thread ("" if none).
 * Valid until the next kivi_* call on the same thread. */
const char* kivi_last_error(void);

/* ==== FP8 KV cache ===================================================================
 * The cache stored as FP8 ("09 — KV Cache Quantization", "The lazy default: FP8 KV";
 * "4.4 KV Cache quantization" §4.1 formats, §4.2 scales): every token is coded on its
 * own, code = the E4M3 / E5M2 value (OCP 8-bit float formats) nearest to
 * float32(x) / s, ties to even, saturating at the largest finite value (448 / 57344),
 * sign kept; float32 IEEE division.  s is a float32 scale per (layer, KV head) for K
 * and one for V, set by the caller (1.0 uncalibrated; the same value for every head
 * is a per-tensor scale).  There is no float16 window: an appended token is coded at
 * once. */
typedef enum { KIVI_FP8_E4M3 = 0, KIVI_FP8_E5M2 = 1 } kivi_fp8_format;

typedef struct {
  int32_t layers, batch, kv_heads, q_heads;
  int32_t head_dim;     /* 128 */
  int32_t format;       /* kivi_fp8_format */
  int64_t max_tokens;   /* a positive multiple of 32; T_max * d code bytes per pair below
                         * 2^31, else KIVI_ERR_UNSUPPORTED */
} kivi_fp8_dims;

/* Device buffers, caller-owned, 16-byte aligned, sizes from kivi_fp8_cache_sizes:
 *   k        u8  [L][B][H_kv][T_max][d]: token t's codes in channel order.
 *   v        u8  [L][B][H_kv][T_max/32][d][32]: for each 32-token run and channel, the
 *            run's 32 codes in token order 0-3, 16-19, 4-7, 20-23, 8-11, 24-27, 12-15,
 *            28-31 (the order the decode's P.V product consumes them).
 *   k_scale, v_scale  f32 [L][H_kv]. */
typedef struct {
  void* k;
  void* v;
  void* k_scale;
  void* v_scale;
} kivi_fp8_cache;

/* Bytes of the four buffers (host-only). */
kivi_status kivi_fp8_cache_sizes(const kivi_fp8_dims* dims, size_t bytes[4]);

/* Code tokens [0, T) of float16 k, v [B][H_kv][ld_tokens][d] into `layer` (0 <= T <=
 * T_max).  Value codes of tokens T .. (end of T's 32-token run) are written as 0. */
kivi_status kivi_fp8_quantize(const kivi_fp8_dims* dims, const kivi_fp8_cache* cache,
                              int32_t layer, const void* k, const void* v, int64_t T,
                              int64_t ld_tokens, void* stream);

/* Code one new token per sequence (float16 k_new, v_new [B][H_kv][d]) at position
 * T_before (T_before + 1 <= T_max). */
kivi_status kivi_fp8_append(const kivi_fp8_dims* dims, const kivi_fp8_cache* cache, int32_t layer,
                            int64_t T_before, const void* k_new, const void* v_new, void* stream);

/* Workspace bytes of kivi_fp8_decode_attn over T tokens with n_split workgroups per
 * (sequence, KV head) (0 = the library's choice; clamped to [1, ceil(T / 32)]). */
kivi_status kivi_fp8_decode_workspace_bytes(const kivi_fp8_dims* dims, int64_t T, int32_t n_split,
                                            size_t* bytes);

/* Decode attention over the T cached FP8 tokens of `layer`: as kivi_decode_attn, with
 * k_t = value(code) * s_K and v_t = value(code) * s_V ("4.4 KV Cache quantization"
 * §4.5: the codes are widened to float16 exactly and attended in float32).  Workspace
 * contract as kivi_decode_attn's. */
kivi_status kivi_fp8_decode_attn(const kivi_fp8_dims* dims, const kivi_fp8_cache* cache,
                                 int32_t layer, int64_t T, const void* q, float sm_scale,
                                 float* out, void* workspace, size_t workspace_bytes,
                                 int32_t n_split, void* stream);

/* ---- MXFP4 codec ----------------------------------------------------------------
 * "KV Cache Quantization (KIVI & FP4)" §4, "Hardware Micro-Scaling": four-bit E2M1
 * values (1 sign, 2 exponent, 1 mantissa bit) in blocks sharing an 8-bit scale.  This
 * is the OCP MXFP4 format the page names: blocks of 32 consecutive channels of one
 * token (Keys and Values alike) share the scale X = 2^s, stored as the E8M0 code
 * s + 127, with s = floor(log2(max |x|)) - 2 (a block of zeros: s = -127); element
 * code = the E2M1 value nearest to x / X (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6),
 * ties to the even code, saturating at 6, sign kept.  Every token is coded on its own
 * (no float16 window).  Decoding: value(code) * X. */
typedef struct {
  int32_t layers, batch, kv_heads, q_heads;
  int32_t head_dim;     /* 128 */
  int32_t reserved;     /* must be 0 */
  int64_t max_tokens;   /* a positive multiple of 32; T_max * d / 2 code bytes per pair
                         * below 2^31, else KIVI_ERR_UNSUPPORTED */
} kivi_mxfp4_dims;

/* Device buffers, caller-owned, 16-byte aligned, sizes from kivi_mxfp4_cache_sizes:
 *   k        u8 [L][B][H_kv][T_max][d/2]: token t's codes, channel 2i in the low
 *            nibble of byte i, 2i+1 in the high nibble.
 *   k_scale  u8 [L][B][H_kv][T_max][d/32]: E8M0 codes of token t's blocks.
 *   v        u8 [L][B][H_kv][T_max/32][d][16]: for each 32-token run and channel, the
 *            run's 32 codes (two per byte, low nibble first) in token order 0-3,
 *            16-19, 4-7, 20-23, 8-11, 24-27, 12-15, 28-31.
 *   v_scale  u8 [L][B][H_kv][T_max/32][d/32][32]: E8M0 codes of each run's tokens per
 *            block, in the same token order. */
typedef struct {
  void* k;
  void* k_scale;
  void* v;
  void* v_scale;
} kivi_mxfp4_cache;

/* Bytes of the four buffers (host-only). */
kivi_status kivi_mxfp4_cache_sizes(const kivi_mxfp4_dims* dims, size_t bytes[4]);

/* Code tokens [0, T) of float16 k, v [B][H_kv][ld_tokens][d] into `layer` (0 <= T <=
 * T_max).  Codes and scales of tokens T .. (end of T's 32-token run) are written as 0. */
kivi_status kivi_mxfp4_quantize(const kivi_mxfp4_dims* dims, const kivi_mxfp4_cache* cache,
                                int32_t layer, const void* k, const void* v, int64_t T,
                                int64_t ld_tokens, void* stream);

/* Code one new token per sequence (float16 k_new, v_new [B][H_kv][d]) at position
 * T_before (T_before + 1 <= T_max); the run's other tokens keep their codes. */
kivi_status kivi_mxfp4_append(const kivi_mxfp4_dims* dims, const kivi_mxfp4_cache* cache,
                              int32_t layer, int64_t T_before, const void* k_new,
                              const void* v_new, void* stream);

/* Workspace bytes of kivi_mxfp4_decode_attn (as kivi_fp8_decode_workspace_bytes). */
kivi_status kivi_mxfp4_decode_workspace_bytes(const kivi_mxfp4_dims* dims, int64_t T,
                                              int32_t n_split, size_t* bytes);

/* Decode attention over the T cached MXFP4 tokens of `layer`: as kivi_decode_attn,
 * with k_t and v_t the decoded values.  The values are widened to float16 with their
 * block scale (exact while the scaled value is a float16 number: always for blocks
 * whose largest magnitude is 2^-20 or more) and attended on the float16 matrix cores
 * in float32.  Workspace contract as kivi_decode_attn's. */
kivi_status kivi_mxfp4_decode_attn(const kivi_mxfp4_dims* dims, const kivi_mxfp4_cache* cache,
                                   int32_t layer, int64_t T, const void* q, float sm_scale,
                                   float* out, void* workspace, size_t workspace_bytes,
                                   int32_t n_split, void* stream);

/* One MXFP4 decode step in one launch: code the new token (as kivi_mxfp4_append) and
 * attend over the T_before + 1 tokens (as kivi_mxfp4_decode_attn with the library's
 * split); the last workgroup of each (sequence, KV head), the only one that reads the
 * new token's run, codes it before reading.  Cache and output equal those of the two
 * calls (outputs to float32 rounding).  Workspace: kivi_mxfp4_decode_workspace_bytes(
 * dims, T_before + 1, 0). */
kivi_status kivi_mxfp4_append_decode(const kivi_mxfp4_dims* dims, const kivi_mxfp4_cache* cache,
                                     int32_t layer, int64_t T_before, const void* k_new,
                                     const void* v_new, const void* q, float sm_scale,
                                     float* out, void* workspace, size_t workspace_bytes,
                                     void* stream);

/* ==== Measurement aid ================================================================
 * kivi_time_next_decode: arms the calling thread's next decode-kernel launch (by any
 * kivi_*decode* call of any codec; an append launch that precedes it in the same call
 * is not meant) to record start_event and stop_event, two hipEvent_t created by the
 * caller on the launch's device, at the decode kernel's own start and end
 * (hipExtLaunchKernel), so that hipEventElapsedTime(start, stop) is that kernel's
 * duration without the dispatch around it.  The events belong to the caller; the
 * library keeps the two handles until that launch only.  Both null disarms; exactly
 * one null is KIVI_ERR_ARG.  Not for a stream that is being captured into a graph.
 * Host-only; launches nothing. */
kivi_status kivi_time_next_decode(void* start_event, void* stop_event);

/* ABI version of this library (bumped on any incompatible change). */
int32_t kivi_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KIVI_H */
