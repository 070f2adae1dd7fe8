/*
 * g4attn - Gemma 4 decoder attention on AMD Instinct MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels for one attention layer:
 *   g4attn_norm_rope  - QK-norm / V-norm prologue (plain-weight RMSNorm) with
 *                       full or zero-padded partial RoPE;
 *   g4attn_prefill    - causal / sliding-window GQA softmax attention over a
 *                       whole prompt, including the K=V global layer;
 *   g4attn_prefill_chunk, g4attn_prefill_chunk_tied - the same for a chunk
 *                       of new positions over caches (chunked prefill, padded
 *                       batches), the second over a K=V layer's cache;
 *   g4attn_decode     - one new query token per sequence over a KV cache
 *                       (split-KV plus a log-sum-exp combine);
 *   g4attn_decode_noalloc - the same without a workspace argument;
 *   g4attn_kv_tied_append, g4attn_decode_tied - a K=V global layer's cache
 *                       of its raw projection, and decode over it.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Tensors are bf16 (raw 16-bit patterns, uint16_t) unless stated; LSE
 *   outputs are fp32 natural logs.
 * - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *   library never allocates, frees, synchronises or prints.  Scratch memory
 *   is a caller-provided workspace whose size the *_workspace_bytes query
 *   returns.
 * - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *   is stream-ordered.  No call blocks.
 * - Every call validates all host-visible arguments BEFORE launching
 *   anything and returns a g4attn_status.  On any error nothing is launched
 *   and no memory is touched.  There is no fallback path.
 * - Activation layout is [B, S, H, D] with the D stride equal to 1; the
 *   batch, sequence and head strides are given in elements.  Base pointers
 *   and strides must keep every row 16-byte aligned.
 * - Thread-safe: the library keeps no state apart from a thread-local copy
 *   of the last HIP error code, and the per-GPU scratch array of
 *   g4attn_decode_noalloc.
 *
 * Source pages: "Gemma 4" (Keras port documentation), "gemma4-pt-claude"
 * (PyTorch port README) and the vinija.ai "Gemma 4" primer.
 */
#ifndef G4ATTN_H
#define G4ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t g4attn_bf16; /* raw bf16 bits */

typedef enum {
  G4ATTN_OK = 0,
  G4ATTN_ERR_NULL = 1,           /* a required pointer is NULL                        */
  G4ATTN_ERR_SHAPE = 2,          /* sizes inconsistent or out of range                */
  G4ATTN_ERR_LAYOUT = 3,         /* misaligned pointer/stride, or non-unit D stride   */
  G4ATTN_ERR_UNSUPPORTED = 4,    /* valid request this library does not implement     */
  G4ATTN_ERR_CACHE_OVERFLOW = 5, /* a cache write or read would pass the capacity     */
  G4ATTN_ERR_WORKSPACE = 6,      /* workspace NULL or smaller than required           */
  G4ATTN_ERR_HIP = 7             /* a HIP launch failed; see g4attn_last_hip_error()  */
} g4attn_status;

/*
 * One attention layer, after the argument table of the Keras port's
 * Gemma4Model ("Gemma 4" docs, Gemma4Model table: num_heads, num_kv_heads /
 * num_global_kv_heads, head_dim / global_head_dim, k_eq_v, sliding_window,
 * partial_rotary_factor).
 */
typedef struct {
  int32_t num_q_heads;  /* Hq; a multiple of num_kv_heads                                 */
  int32_t num_kv_heads; /* Hkv; query head h uses KV head h / (Hq / Hkv)                  */
  int32_t head_dim;     /* D: 256 (sliding layers) or 512 (global layers)                 */
  int32_t window;       /* 0 = global (key j visible from row i iff j <= i);              */
                        /* w > 0 = sliding (visible iff 0 <= i - j < w)                   */
  int32_t k_eq_v;       /* prefill: 1 = K=V global layer (see g4attn_prefill)             */
  int32_t rotary_dims;  /* rotated dims of q/k: head_dim (full), head_dim/4 (partial), 0  */
  float rope_theta;     /* RoPE base: 1e4 on sliding layers, 1e6 on global layers         */
  float rms_eps;        /* RMSNorm epsilon (1e-6)                                         */
  float scale;          /* logits = scale * q.k (1/sqrt(head_dim) in the workloads)       */
} g4attn_layer_desc;

/*
 * Prologue of one projection ("Gemma 4" docs, "What changed from Gemma 3":
 * plain-weight RMSNorm and zero-pad partial rope; gemma4-pt-claude README,
 * "Supported Models": QK-norm and V-norm on every variant; vinija.ai primer,
 * "Dual RoPE configurations", rotation matrix):
 *
 *   r      = 1 / sqrt(mean_d x[b,t,h,d]^2 + rms_eps)
 *   u_d    = x_d * r * weight_d            (weight NULL: u_d = x_d * r)
 *   p      = (pos0 ? pos0[b] : 0) + t
 *   f_j    = rope_theta^(-2j/D) for j < rotary_dims/2, else 0     (j < D/2)
 *   y_j    = u_j cos(p f_j) - u_{j+D/2} sin(p f_j)
 *   y_{j+D/2} = u_{j+D/2} cos(p f_j) + u_j sin(p f_j)
 *
 * computed in fp32 with the angle p*f_j formed and range-reduced in fp64,
 * and rounded once to bf16 (round to nearest even).
 *
 *   x          [B, S, H, D] bf16, strides x_strides = {batch, seq, head}.
 *   y          y_cache_cap == 0: [B, S, H, D] with strides y_strides;
 *              y_cache_cap  > 0: a contiguous cache [B, H, y_cache_cap, D];
 *              row p of sequence b, head h receives the result
 *              (y_strides ignored), or with y_cache_ring = 1 row
 *              p mod y_cache_cap: the rolling cache of a sliding layer,
 *              which keeps the last y_cache_cap (= window) positions
 *              (gemma4-pt-claude README, "KV Cache": window-sized caches on
 *              sliding layers).  Of the S positions of one call only the
 *              last y_cache_cap are written (the earlier ones would be
 *              overwritten by them).
 *   weight     [D] bf16 or NULL (weightless; the V-norm).
 *   head_dim   256 or 512; rotary_dims in {0, head_dim/4, head_dim}.
 *   pos0       device int32 [B] (first position of each sequence) or NULL
 *              (positions start at 0).
 *   max_pos    host-known upper bound of every p (pos0[b] + S - 1); required
 *              >= S - 1.  In (linear) cache mode max_pos >= y_cache_cap is
 *              G4ATTN_ERR_CACHE_OVERFLOW (the cache raises rather than
 *              evicting: gemma4-pt-claude README, "KV Cache").  The kernel
 *              also skips any row outside [0, y_cache_cap).
 *   y_cache_ring  0 or 1 (1 needs y_cache_cap > 0), else G4ATTN_ERR_SHAPE.
 * x and y may not overlap unless x == y with equal strides (in place).
 */
g4attn_status g4attn_norm_rope(const g4attn_bf16* x, g4attn_bf16* y, const g4attn_bf16* weight,
                               int32_t B, int32_t S, int32_t H, int32_t head_dim,
                               int32_t rotary_dims, float rope_theta, float rms_eps,
                               const int64_t x_strides[3], const int64_t y_strides[3],
                               const int32_t* pos0, int32_t max_pos, int32_t y_cache_cap,
                               int32_t y_cache_ring, void* stream);

/* Workspace (bytes) that g4attn_prefill needs for this layer and size. */
size_t g4attn_prefill_workspace_bytes(const g4attn_layer_desc* desc, int32_t B, int32_t S);

/*
 * Prefill attention (vinija.ai primer, "Sliding-window attention" and
 * "Global attention layers"; softmax of scaled dot products, "Why long
 * context is difficult"):
 *
 *   s_ij   = scale * q_i . k_j,   j visible from i (see g4attn_layer_desc)
 *   out_i  = sum_j softmax_j(s_ij) v_j,     lse_i = log sum_j exp(s_ij)
 *
 * for every batch b, query head h (KV head h / (Hq/Hkv)) and row i < S.
 *
 *   q          [B, S, Hq, D] post-prologue queries, strides q_strides.
 *   k_eq_v == 0:
 *     k, v     [B, S, Hkv, D] post-prologue keys and values, strides
 *              kv_strides (shared by k and v); w_k ignored (may be NULL).
 *   k_eq_v == 1 (global K=V layer; "Gemma 4" docs, "What changed from
 *              Gemma 3", K=V global MQA):
 *     k        [B, S, Hkv, D] the RAW tied projection X (before any norm),
 *              strides kv_strides; v must be NULL; w_k [D] the K-norm weight.
 *              Keys are RoPE(RMSNorm(X) * w_k) at positions 0..S-1 and
 *              values are RMSNorm(X) (weightless), both formed inside the
 *              call from one shared tile of X.  head_dim must be 512,
 *              rotary_dims 128, |scale| <= 2^30 (else G4ATTN_ERR_UNSUPPORTED).
 *   out        [B, S, Hq, D] bf16, strides o_strides.
 *   lse        [B, Hq, S] fp32 (contiguous) or NULL.
 *   span_lo,   NULL, or device int32 [B, S]: a bidirectional span per row
 *   span_hi    (the image blocks of multimodal prompts: "Gemma 4" docs, "What
 *              changed from Gemma 3", NaViT vision tower, and the
 *              use_bidirectional_vision argument: image tokens attend
 *              bidirectionally within their block on the sliding-window
 *              layers; gemma4-pt-claude README, "Tests": the spans survive
 *              the cached prefill path): row i of sequence b also
 *              sees keys span_lo[b,i] .. span_hi[b,i], whatever the window
 *              or causality says.  A text row takes span_lo = span_hi = i.
 *              Requirements (not checked): span_lo[b,i] <= i <= span_hi[b,i]
 *              and both non-decreasing in i (contiguous spans).  The kernel
 *              clamps span_lo below 0 to 0 and span_hi to S - 1, so no key
 *              outside the sequence is read.  Both or neither (else
 *              G4ATTN_ERR_NULL); with k_eq_v too.
 *   workspace  >= g4attn_prefill_workspace_bytes(desc, B, S) bytes, 16-byte
 *              aligned (per-wave flags; for K=V also the inverse RMS and
 *              rotated slice of each key row).
 * Requires S >= 1, B >= 1, and a K/V row stride kv_strides[1] below 2^25
 * elements (G4ATTN_ERR_UNSUPPORTED otherwise: a 32-key tile's row offsets are
 * formed in 32 bits).  Window and causality are applied exactly (integer
 * logic); rows never see keys past themselves.
 */
g4attn_status g4attn_prefill(const g4attn_layer_desc* desc, const g4attn_bf16* q,
                             const g4attn_bf16* k, const g4attn_bf16* v, const g4attn_bf16* w_k,
                             g4attn_bf16* out, float* lse, int32_t B, int32_t S,
                             const int64_t q_strides[3], const int64_t kv_strides[3],
                             const int64_t o_strides[3], const int32_t* span_lo, const int32_t* span_hi,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Chunked prefill over caches (gemma4-pt-claude README, "KV Cache": the
 * decoder attends over cached keys and values; "Tests": a batched forward
 * equals the single-sequence one; vinija.ai primer, "Sliding-window
 * attention"):
 *
 *   for b < B, t < qlen[b]:  p = pos0[b] + t
 *   s_tj   = scale * q[b,t,h] . k_cache[b,g,j],   j <= p  (and p - j < window)
 *   out[b,t,h] = sum_j softmax_j(s_tj) v_cache[b,g,j],  lse[b,h,t] = log sum_j exp(s_tj)
 *
 * A new chunk of S query rows continues sequences whose keys and values
 * (this chunk's included, e.g. written by g4attn_norm_rope in cache mode at
 * pos0) sit in linear caches.  Rows t >= qlen[b] are padding: not written.
 *
 *   q          [B, S, Hq, D] post-prologue queries, strides q_strides.
 *   k_cache,   [B, Hkv, cache_cap, D] contiguous post-prologue keys and
 *   v_cache    values (separate tensors; any window).
 *   pos0, qlen device int32 [B]: first position and valid rows of each
 *              sequence (qlen[b] <= S).
 *   max_pos    host-known bound of every pos0[b] + qlen[b] - 1; >= cache_cap
 *              is G4ATTN_ERR_CACHE_OVERFLOW.  The kernel clamps the device
 *              values to it: qlen[b] is taken as min(qlen[b], S,
 *              max_pos + 1 - pos0[b]) and a sequence with pos0[b] < 0 has no
 *              rows, so no cache row past max_pos is read; rows cut off this
 *              way are left unwritten, like padding.
 *   span_lo,   NULL, or [B, S] bidirectional spans as in g4attn_prefill, in
 *   span_hi    absolute positions (row t of the chunk is position
 *              pos0[b] + t); span_lo below 0 is taken as 0 and span_hi is
 *              clamped to pos0[b] + qlen[b] - 1.
 *   out        [B, S, Hq, D] bf16, strides o_strides; lse [B, Hq, S] or NULL.
 *   workspace  >= g4attn_prefill_workspace_bytes(desc, B, S) bytes, 16-byte
 *              aligned (only its per-wave flags are used here).
 * K=V layers (desc k_eq_v = 1) are G4ATTN_ERR_UNSUPPORTED here: their cache
 * holds the raw projection and its side data (g4attn_prefill_chunk_tied).
 */
g4attn_status g4attn_prefill_chunk(const g4attn_layer_desc* desc, const g4attn_bf16* q,
                                   const g4attn_bf16* k_cache, const g4attn_bf16* v_cache, int32_t cache_cap,
                                   const int32_t* pos0, const int32_t* qlen, int32_t max_pos,
                                   const int32_t* span_lo, const int32_t* span_hi,
                                   g4attn_bf16* out, float* lse, int32_t B, int32_t S,
                                   const int64_t q_strides[3], const int64_t o_strides[3], void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * Chunked prefill of a K=V global layer over the cache g4attn_kv_tied_append
 * writes ("Gemma 4" docs, "What changed from Gemma 3", K=V global MQA;
 * gemma4-pt-claude README, "KV Cache"): out and lse as in
 * g4attn_prefill_chunk, with the keys and values of cached row p formed
 * inside the call as in g4attn_decode_tied:
 *   K_p = r_p * (X_p * w_k on the unrotated dims | krot_p on the rotated)
 *   V_p = r_p * X_p
 * so a prompt can be continued (or a padded batch run) over the layer's own
 * cache, this chunk's rows appended to it first.
 *
 *   x_cache, r_cache, krot_cache, cache_cap  as g4attn_kv_tied_append
 *              writes them; w_k [512] the K-norm weight.
 *   q, pos0, qlen, max_pos, span_lo, span_hi, out, lse, B, S, strides,
 *   workspace  as in g4attn_prefill_chunk (clamps included).
 * desc: k_eq_v = 1, head_dim 512, rotary_dims 128, |scale| <= 2^30 (else
 * G4ATTN_ERR_UNSUPPORTED).  The logit scale multiplies the queries (the
 * cached r carries none), so the scores are formed from
 * bf16(scale * log2(e) * q) rather than from q.
 */
g4attn_status g4attn_prefill_chunk_tied(const g4attn_layer_desc* desc, const g4attn_bf16* q,
                                        const g4attn_bf16* x_cache, const float* r_cache,
                                        const g4attn_bf16* krot_cache, const g4attn_bf16* w_k, int32_t cache_cap,
                                        const int32_t* pos0, const int32_t* qlen, int32_t max_pos,
                                        const int32_t* span_lo, const int32_t* span_hi, g4attn_bf16* out,
                                        float* lse, int32_t B, int32_t S, const int64_t q_strides[3],
                                        const int64_t o_strides[3], void* workspace, size_t workspace_bytes,
                                        void* stream);

/* Workspace (bytes) that g4attn_decode needs; num_splits as passed to it
 * (a sliding layer's size depends on min(max_kv_len, window) only). */
size_t g4attn_decode_workspace_bytes(const g4attn_layer_desc* desc, int32_t B,
                                     int32_t max_kv_len, int32_t num_splits);

/*
 * Single-token decode over a KV cache (vinija.ai primer, "KV cache and
 * long-context scaling" and "Sliding-window attention"; gemma4-pt-claude
 * README, "KV Cache"):
 *
 *   out[b,h] = sum_{j < n_b} softmax_j(scale * q[b,h] . K[b,g,j]) V[b,g,j],
 *   lse[b,h] = log sum_{j < n_b} exp(scale * q[b,h] . K[b,g,j]),
 *   g = h / (Hq/Hkv),  n_b = kv_len[b] (global) or min(kv_len[b], window)
 *   (sliding: j runs over the filled slots of the ring)
 *
 *   q          [B, Hq, D] contiguous post-prologue queries (norm + RoPE at
 *              the new token's position, e.g. via g4attn_norm_rope).
 *   k_cache    [B, Hkv, cache_cap, D] contiguous post-prologue keys.
 *   v_cache    same shape; may equal k_cache (one tensor serves as both).
 *   kv_len     device int32 [B]; each value in [1, max_kv_len]: the number of
 *              positions of the sequence so far, the new token included.
 *              The kernels clamp it to [0, max_kv_len], so no row past
 *              max_kv_len is read; a sequence clamped to 0 gets zeros and
 *              lse = -inf.
 *              Global layer (window == 0): rows [0, kv_len[b]) are read,
 *              rows past them never.  Sliding layer (window > 0): k_cache and
 *              v_cache are rings of cache_cap == window slots (position p in
 *              slot p mod window, as g4attn_norm_rope's ring mode writes
 *              them), and the min(kv_len[b], window) filled slots, which hold
 *              exactly the positions the new token sees, are read (softmax
 *              does not depend on their order).
 *   max_kv_len host-known bound of kv_len; global layer: > cache_cap is
 *              G4ATTN_ERR_CACHE_OVERFLOW; sliding layer: cache_cap != window
 *              is G4ATTN_ERR_SHAPE.
 *   out        [B, Hq, D] bf16 contiguous;  lse  [B, Hq] fp32 or NULL.
 *   num_splits 0 = automatic (about one workgroup per compute unit over
 *              B * Hkv (sequence, KV head) pairs: min(32, ceil(256 / (B *
 *              Hkv))) chunks of at least 256 rows); otherwise the row range
 *              [0, rows) is cut into num_splits equal chunks (a multiple of
 *              64 rows each), with
 *              rows = max_kv_len (global) or min(max_kv_len, window)
 *              (sliding); the partial results are merged by a log-sum-exp
 *              combine (with one chunk per sequence the split kernel writes
 *              the result itself and no combine runs).
 *   workspace  >= g4attn_decode_workspace_bytes(desc, B, max_kv_len,
 *              num_splits) bytes, 16-byte aligned.
 */
g4attn_status g4attn_decode(const g4attn_layer_desc* desc, const g4attn_bf16* q,
                            const g4attn_bf16* k_cache, const g4attn_bf16* v_cache,
                            const int32_t* kv_len, int32_t B, int32_t max_kv_len,
                            int32_t cache_cap, g4attn_bf16* out, float* lse, int32_t num_splits,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * g4attn_decode for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops and hosts that forbid allocation.
 * Same arguments, semantics and errors as g4attn_decode, without the
 * workspace: the call allocates nothing (no hipMalloc, hipFree or allocating
 * library routine).  Its scratch is a 32 MiB device array inside the library,
 * one per GPU, set up on the first call on that GPU and held until the
 * process ends.
 *   num_splits 0: the automatic split count if its partial results fit the
 *              32 MiB (B * Hq * splits * (4 * head_dim + 8) bytes plus
 *              alignment), else the largest smaller count that fits;
 *              > 0: as in g4attn_decode if it fits.
 *   Sizes that do not fit even as one split (B * Hq * head_dim * 4 bytes
 *   near or above 32 MiB), or an explicit count that does not fit, return
 *   G4ATTN_ERR_WORKSPACE with nothing launched.
 * Every call on one GPU uses the same scratch array: calls that overlap on
 * one GPU (concurrent streams or host threads) race and must be serialised
 * by the caller.
 */
g4attn_status g4attn_decode_noalloc(const g4attn_layer_desc* desc, const g4attn_bf16* q,
                                    const g4attn_bf16* k_cache, const g4attn_bf16* v_cache,
                                    const int32_t* kv_len, int32_t B, int32_t max_kv_len, int32_t cache_cap,
                                    g4attn_bf16* out, float* lse, int32_t num_splits, void* stream);

/*
 * Append rows to a K=V global layer's own cache: the raw tied projection X
 * ("Gemma 4" docs, "What changed from Gemma 3", K=V global MQA: K =
 * RoPE(RMSNorm(X) w_k), V = RMSNorm(X), weightless) is cached as X itself
 * plus, per row, its inverse RMS r and the rotated part of its key before
 * r, so that the decode below forms K and V exactly (V unroped):
 *
 *   p = (pos0 ? pos0[b] : 0) + t
 *   x_cache[b,g,p,:]    = X[b,t,g,:]                              (copied)
 *   r_cache[b,g,p]      = 1 / sqrt(mean_d X[b,t,g,d]^2 + rms_eps)
 *   krot_cache[b,g,p,:] = RoPE_p(X[b,t,g,:] * w_k) on dims 0..63, 256..319
 *
 *   x          [B, S, Hkv, 512] raw projection, strides x_strides.
 *   w_k        [512] K-norm weight; rotary_dims must be 128 (0.25 of 512).
 *   x_cache    [B, Hkv, cache_cap, 512] bf16; r_cache [B, Hkv, cache_cap]
 *   r_cache,   fp32; krot_cache [B, Hkv, cache_cap, 128] bf16; all
 *   krot_cache contiguous.
 *   pos0, max_pos  as in g4attn_norm_rope (max_pos >= cache_cap is
 *              G4ATTN_ERR_CACHE_OVERFLOW).
 */
g4attn_status g4attn_kv_tied_append(const g4attn_bf16* x, const g4attn_bf16* w_k, int32_t B, int32_t S,
                                    int32_t Hkv, int32_t rotary_dims, float rope_theta, float rms_eps,
                                    const int64_t x_strides[3], const int32_t* pos0, int32_t max_pos,
                                    g4attn_bf16* x_cache, float* r_cache, g4attn_bf16* krot_cache,
                                    int32_t cache_cap, void* stream);

/*
 * Decode of a K=V global layer over the cache g4attn_kv_tied_append writes:
 * out and lse as in g4attn_decode with, for cached row p,
 *   K_p = r_p * (X_p * w_k on the unrotated dims | krot_p on the rotated)
 *   V_p = r_p * X_p
 * (the keys of the prefill's K=V path).  1284 bytes per cached row and KV
 * head are read once.  desc: k_eq_v = 1, head_dim 512, rotary_dims 128,
 * window 0 (else G4ATTN_ERR_UNSUPPORTED).  q, kv_len, max_kv_len,
 * cache_cap, out, lse, num_splits and the workspace as in g4attn_decode
 * (g4attn_decode_workspace_bytes gives its size).
 */
g4attn_status g4attn_decode_tied(const g4attn_layer_desc* desc, const g4attn_bf16* q, const g4attn_bf16* x_cache,
                                 const float* r_cache, const g4attn_bf16* krot_cache, const g4attn_bf16* w_k,
                                 const int32_t* kv_len, int32_t B, int32_t max_kv_len, int32_t cache_cap,
                                 g4attn_bf16* out, float* lse, int32_t num_splits, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* Static description of a status code (never NULL). */
const char* g4attn_status_str(g4attn_status status);

/* The hipError_t of the last G4ATTN_ERR_HIP returned on this thread (0 if none). */
int32_t g4attn_last_hip_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int32_t g4attn_version(void);

#ifdef __cplusplus
}
#endif
#endif /* G4ATTN_H */
