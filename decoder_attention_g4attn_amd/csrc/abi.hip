// C ABI of libg4attn: argument validation and dispatch to the kernels.
//
// Every entry point checks all host-visible arguments before any HIP call
// and returns a g4attn_status; on error nothing is launched.  Cache overflow
// is an error rather than an eviction, as the PyTorch port's KV cache raises
// when a write would overflow it [gemma4-pt-claude README, "KV Cache"].
#include <math.h>
#include <stdint.h>

#include "../../include/g4attn.h"
#include "g4attn_internal.h"

namespace {

thread_local int32_t t_last_hip_error = 0;

constexpr int32_t kVersion = 400;  // 0.4.0: K=V decode over the raw-projection cache

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool strides_ok(const int64_t* s) {
  if (!s) return false;
  for (int i = 0; i < 3; ++i)
    if (s[i] < 0 || (s[i] & 7) != 0) return false;  // 16-byte rows
  return true;
}

bool head_dim_ok(int32_t D) { return D == 256 || D == 512; }
bool rot_ok(int32_t D, int32_t rot) { return rot == 0 || rot == D / 4 || rot == D; }

g4attn_status desc_check(const g4attn_layer_desc* d) {
  if (!d) return G4ATTN_ERR_NULL;
  if (d->num_q_heads < 1 || d->num_kv_heads < 1 || d->num_q_heads % d->num_kv_heads != 0)
    return G4ATTN_ERR_SHAPE;
  if (d->num_kv_heads > 65535) return G4ATTN_ERR_SHAPE;
  if (!head_dim_ok(d->head_dim)) return G4ATTN_ERR_UNSUPPORTED;
  if (d->window < 0) return G4ATTN_ERR_SHAPE;
  if (d->k_eq_v != 0 && d->k_eq_v != 1) return G4ATTN_ERR_SHAPE;
  if (!rot_ok(d->head_dim, d->rotary_dims)) return G4ATTN_ERR_UNSUPPORTED;
  if (!(d->rope_theta > 0.f) || !isfinite(d->rope_theta)) return G4ATTN_ERR_SHAPE;
  if (!(d->rms_eps >= 0.f) || !isfinite(d->rms_eps)) return G4ATTN_ERR_SHAPE;
  if (!isfinite(d->scale)) return G4ATTN_ERR_SHAPE;
  return G4ATTN_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

g4attn_status hip_status(hipError_t e) {
  if (e == hipSuccess) return G4ATTN_OK;
  t_last_hip_error = (int32_t)e;
  return G4ATTN_ERR_HIP;
}

// Decode: rows per split chunk (a multiple of 64) and the split count.
int64_t decode_chunk(const g4attn_layer_desc* d, int32_t B, int32_t max_kv_len, int32_t num_splits) {
  int64_t target;
  if (num_splits > 0) {
    target = num_splits;
  } else {
    // Aim for about one workgroup per compute unit (256 on MI355X) over the
    // whole batch: the decode is bound by HBM, which fewer CUs than the chip
    // has already saturate, while every extra chunk pays its own pipeline
    // fill, merge and partial-result traffic (measured on the 31B K=V batch:
    // 256 -> 1.91 ms, 1024 -> 2.20 ms, 4096 -> 2.03 ms).
    // Small batches: at most 32 chunks per (sequence, KV head); past that the
    // per-chunk start-up and the combine of more partials cost more than the
    // extra workgroups gain (one sequence, 4 KV heads, 32K rows: 64 chunks
    // 66.7 us, 32 chunks 54.2 us; 128K rows: 122.4 vs 118.8 us).
    const int64_t groups = (int64_t)B * d->num_kv_heads;
    target = (256 + groups - 1) / groups;
    if (target > 32) target = 32;
    if (target < 1) target = 1;
  }
  int64_t c = ((int64_t)max_kv_len + target - 1) / target;
  c = (c + 63) / 64 * 64;
  if (num_splits == 0 && c < 256) c = 256;
  return c;
}

// Cache rows a decode reads at most: sliding layers keep the last `window`
// positions in a ring of that many slots, so min(kv_len, window) of them.
int32_t decode_rows(const g4attn_layer_desc* d, int32_t max_kv_len) {
  return d->window > 0 ? (max_kv_len < d->window ? max_kv_len : d->window) : max_kv_len;
}

}  // namespace

namespace g4attn {

g4attn_status decode_validate(const g4attn_layer_desc* d, const g4attn_bf16* q, const g4attn_bf16* k_cache,
                              const g4attn_bf16* v_cache, const int32_t* kv_len, int32_t B, int32_t max_kv_len,
                              int32_t cache_cap, const g4attn_bf16* out, const float* lse, int32_t num_splits) {
  g4attn_status st = desc_check(d);
  if (st != G4ATTN_OK) return st;
  if (!q || !k_cache || !v_cache || !kv_len || !out) return G4ATTN_ERR_NULL;
  if (d->num_q_heads / d->num_kv_heads > 16) return G4ATTN_ERR_UNSUPPORTED;
  if (B < 1 || B > 65535 || max_kv_len < 1 || cache_cap < 1 || num_splits < 0) return G4ATTN_ERR_SHAPE;
  // sliding layer: the cache is a ring of exactly `window` slots
  if (d->window != 0 && cache_cap != d->window) return G4ATTN_ERR_SHAPE;
  if (d->window == 0 && max_kv_len > cache_cap) return G4ATTN_ERR_CACHE_OVERFLOW;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
      (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return G4ATTN_ERR_LAYOUT;
  const int32_t rows = decode_rows(d, max_kv_len);
  const int64_t c = decode_chunk(d, B, rows, num_splits);
  if (((int64_t)rows + c - 1) / c > 65535) return G4ATTN_ERR_SHAPE;
  return G4ATTN_OK;
}

int32_t decode_fit_splits(const g4attn_layer_desc* d, int32_t B, int32_t max_kv_len, int32_t num_splits,
                          size_t max_bytes) {
  if (g4attn_decode_workspace_bytes(d, B, max_kv_len, num_splits) <= max_bytes) return num_splits;
  if (num_splits > 0) return -1;
  // the automatic count does not fit: the largest explicit count below it that does
  const int32_t rows = decode_rows(d, max_kv_len);
  const int64_t c = decode_chunk(d, B, rows, 0);
  for (int64_t ns = ((int64_t)rows + c - 1) / c - 1; ns >= 1; --ns)
    if (g4attn_decode_workspace_bytes(d, B, max_kv_len, (int32_t)ns) <= max_bytes) return (int32_t)ns;
  return -1;
}

g4attn_status decode_run(const g4attn_layer_desc* d, const g4attn_bf16* q, const g4attn_bf16* k_cache,
                         const g4attn_bf16* v_cache, const int32_t* kv_len, int32_t B, int32_t max_kv_len,
                         int32_t cache_cap, g4attn_bf16* out, float* lse, int32_t num_splits, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  const g4attn_status st =
      decode_validate(d, q, k_cache, v_cache, kv_len, B, max_kv_len, cache_cap, out, lse, num_splits);
  if (st != G4ATTN_OK) return st;
  const int32_t rows = decode_rows(d, max_kv_len);
  const int64_t c = decode_chunk(d, B, rows, num_splits);
  const int64_t ns = ((int64_t)rows + c - 1) / c;
  const size_t need = g4attn_decode_workspace_bytes(d, B, max_kv_len, num_splits);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return G4ATTN_ERR_WORKSPACE;

  const size_t ph = (size_t)B * d->num_q_heads;
  DecodeArgs a{};
  a.q = q; a.kc = k_cache; a.vc = v_cache; a.kv_len = kv_len; a.out = out; a.lse = lse;
  char* wsp = (char*)workspace;
  a.o_part = (float*)wsp;
  wsp += align256(ph * ns * d->head_dim * sizeof(float));
  a.lse_part = (float*)wsp;
  wsp += align256(ph * ns * sizeof(float));
  a.dmax = (float*)wsp;
  wsp += align256(ph * ns * sizeof(float));
  a.dflags = (int*)wsp;
  a.B = B; a.Hq = d->num_q_heads; a.Hkv = d->num_kv_heads; a.D = d->head_dim; a.cap = cache_cap;
  a.nsplit = (int)ns; a.chunk = (int)c; a.max_len = rows;  // kv_len is clamped to rows in the kernel
  a.scale_log2 = d->scale * kLog2e;
  return hip_status(launch_decode(a, stream));
}

g4attn_status status_of_hip(hipError_t e) { return hip_status(e); }

}  // namespace g4attn

extern "C" {

int32_t g4attn_version(void) { return kVersion; }

int32_t g4attn_last_hip_error(void) { return t_last_hip_error; }

const char* g4attn_status_str(g4attn_status s) {
  switch (s) {
    case G4ATTN_OK: return "ok";
    case G4ATTN_ERR_NULL: return "a required pointer is NULL";
    case G4ATTN_ERR_SHAPE: return "sizes inconsistent or out of range";
    case G4ATTN_ERR_LAYOUT: return "misaligned pointer or stride";
    case G4ATTN_ERR_UNSUPPORTED: return "configuration not implemented";
    case G4ATTN_ERR_CACHE_OVERFLOW: return "KV cache capacity exceeded";
    case G4ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case G4ATTN_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

g4attn_status g4attn_norm_rope(const g4attn_bf16* x, g4attn_bf16* y, const g4attn_bf16* weight,
                               int32_t B, int32_t S, int32_t H, int32_t head_dim,
                               int32_t rotary_dims, float rope_theta, float rms_eps,
                               const int64_t x_strides[3], const int64_t y_strides[3],
                               const int32_t* pos0, int32_t max_pos, int32_t y_cache_cap,
                               int32_t y_cache_ring, void* stream) {
  if (!x || !y || !x_strides) return G4ATTN_ERR_NULL;
  if (y_cache_cap == 0 && !y_strides) return G4ATTN_ERR_NULL;
  if (B < 1 || S < 1 || H < 1 || B > 65535 || y_cache_cap < 0) return G4ATTN_ERR_SHAPE;
  if (y_cache_ring != 0 && (y_cache_ring != 1 || y_cache_cap == 0)) return G4ATTN_ERR_SHAPE;
  if (!head_dim_ok(head_dim) || !rot_ok(head_dim, rotary_dims)) return G4ATTN_ERR_UNSUPPORTED;
  if (!(rope_theta > 0.f) || !isfinite(rope_theta) || !(rms_eps >= 0.f) || !isfinite(rms_eps))
    return G4ATTN_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(y) || (weight && !aligned16(weight))) return G4ATTN_ERR_LAYOUT;
  if (!strides_ok(x_strides) || (y_cache_cap == 0 && !strides_ok(y_strides))) return G4ATTN_ERR_LAYOUT;
  const int64_t top = pos0 ? (int64_t)max_pos : (int64_t)S - 1;
  if (pos0 && max_pos < S - 1) return G4ATTN_ERR_SHAPE;
  if (y_cache_cap > 0 && !y_cache_ring && top >= y_cache_cap) return G4ATTN_ERR_CACHE_OVERFLOW;

  g4attn::NormRopeArgs a{};
  a.x = x; a.y = y; a.w = weight;
  a.B = B; a.S = S; a.H = H; a.D = head_dim; a.rot = rotary_dims;
  a.log2_theta = log2((double)rope_theta);
  a.eps = rms_eps;
  for (int i = 0; i < 3; ++i) {
    a.xs[i] = x_strides[i];
    a.ys[i] = y_cache_cap > 0 ? 0 : y_strides[i];
  }
  a.pos0 = pos0;
  a.cache_cap = y_cache_cap;
  a.ring = y_cache_ring;
  return hip_status(g4attn::launch_norm_rope(a, (hipStream_t)stream));
}

// Prefill workspace: per-wave reference-overflow flags (all layers), then
// the K=V per-key factor and rotated slice.
struct PrefillWs {
  size_t flags, r, krot, total;
};
static PrefillWs prefill_ws(const g4attn_layer_desc* d, int32_t B, int32_t S) {
  PrefillWs w{};
  const int64_t G = d->num_q_heads / d->num_kv_heads;
  const int64_t ntiles = ((int64_t)S * G + 127) / 128;
  const size_t rows = (size_t)B * d->num_kv_heads * S;
  w.flags = 0;
  // per-wave flags: ntiles 128-row tiles x 4 waves (both prefill kernels run
  // 128-row workgroups of 4 waves), plus two tiles of slack
  w.r = align256((size_t)B * d->num_kv_heads * (ntiles + 2) * 4 * sizeof(int));
  w.krot = w.r + (d->k_eq_v ? align256(rows * sizeof(float)) : 0);
  w.total = w.krot + (d->k_eq_v ? align256(rows * 128 * sizeof(uint16_t)) : 0);
  return w;
}

size_t g4attn_prefill_workspace_bytes(const g4attn_layer_desc* d, int32_t B, int32_t S) {
  if (!d || B < 1 || S < 1 || d->num_kv_heads < 1 || d->num_q_heads < 1 ||
      d->num_q_heads % d->num_kv_heads != 0)
    return 0;
  return prefill_ws(d, B, S).total;
}

g4attn_status g4attn_prefill(const g4attn_layer_desc* d, const g4attn_bf16* q,
                             const g4attn_bf16* k, const g4attn_bf16* v, const g4attn_bf16* w_k,
                             g4attn_bf16* out, float* lse, int32_t B, int32_t S,
                             const int64_t q_strides[3], const int64_t kv_strides[3],
                             const int64_t o_strides[3], const int32_t* span_lo, const int32_t* span_hi,
                             void* workspace, size_t workspace_bytes, void* stream) {
  g4attn_status st = desc_check(d);
  if (st != G4ATTN_OK) return st;
  if (!q || !k || !out || !q_strides || !kv_strides || !o_strides) return G4ATTN_ERR_NULL;
  if (!span_lo != !span_hi) return G4ATTN_ERR_NULL;        // spans come as a pair
  if (d->k_eq_v) {
    if (!w_k) return G4ATTN_ERR_NULL;
    if (v) return G4ATTN_ERR_SHAPE;  // K=V takes one tensor
    if (d->head_dim != 512 || d->rotary_dims != 128) return G4ATTN_ERR_UNSUPPORTED;
    if (!(fabsf(d->scale) <= 0x1p30f)) return G4ATTN_ERR_UNSUPPORTED;
  } else if (!v) {
    return G4ATTN_ERR_NULL;
  }
  if (B < 1 || S < 1 || B > 65535) return G4ATTN_ERR_SHAPE;
  if ((int64_t)S * (d->num_q_heads / d->num_kv_heads) > (int64_t)INT32_MAX) return G4ATTN_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || (v && !aligned16(v)) || (w_k && !aligned16(w_k)) ||
      !aligned16(out) || (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return G4ATTN_ERR_LAYOUT;
  if (!strides_ok(q_strides) || !strides_ok(kv_strides) || !strides_ok(o_strides)) return G4ATTN_ERR_LAYOUT;
  // a K/V tile's 32 row offsets are formed in 32 bits
  if (kv_strides[1] >= ((int64_t)1 << 25)) return G4ATTN_ERR_UNSUPPORTED;
  const PrefillWs ws = prefill_ws(d, B, S);
  if (!workspace || workspace_bytes < ws.total || !aligned16(workspace)) return G4ATTN_ERR_WORKSPACE;

  g4attn::PrefillArgs a{};
  a.q = q; a.k = k; a.v = v; a.w_k = w_k; a.out = out; a.lse = lse;
  a.span_lo = span_lo; a.span_hi = span_hi;
  a.B = B; a.S = S; a.Hq = d->num_q_heads; a.Hkv = d->num_kv_heads; a.D = d->head_dim;
  a.window = d->window; a.kv_tied = d->k_eq_v;
  a.scale_log2 = d->scale * g4attn::kLog2e;
  // K=V: the logit scale rides on the per-key factor r (and is divided out of
  // the output) unless it is too small for that, when it scales the queries.
  const float c = a.scale_log2;
  const bool fold = fabsf(c) >= 0x1p-30f;
  a.qmul = fold ? 1.f : c;
  a.omul = fold ? 1.f / c : 1.f;
  // Per-key factor of the scores: K=V r * (c or 1), r > 0; else c itself,
  // with the smallest normal float standing in for 0 (the logits are then
  // below 2^-100 instead of 0, and masked slots still give -inf).
  if (!d->k_eq_v && c == 0.f) a.scale_log2 = 0x1p-126f;
  const bool neg = d->k_eq_v ? (fold && c < 0.f) : (a.scale_log2 < 0.f);
  a.mask_s = neg ? INFINITY : -INFINITY;
  for (int i = 0; i < 3; ++i) { a.qs[i] = q_strides[i]; a.ks[i] = kv_strides[i]; a.os[i] = o_strides[i]; }
  hipStream_t s = (hipStream_t)stream;
  char* wsp = (char*)workspace;
  a.flags = (int*)(wsp + ws.flags);
  if (d->k_eq_v) {
    float* r = (float*)(wsp + ws.r);
    uint16_t* krot = (uint16_t*)(wsp + ws.krot);
    g4attn::KvPrepArgs p{};
    p.x = k; p.w_k = w_k; p.r = r; p.krot = krot;
    p.B = B; p.S = S; p.Hkv = d->num_kv_heads; p.rot = d->rotary_dims;
    p.log2_theta = log2((double)d->rope_theta);
    p.eps = d->rms_eps;
    p.rscale = fold ? c : 1.f;
    for (int i = 0; i < 3; ++i) p.xs[i] = kv_strides[i];
    st = hip_status(g4attn::launch_kv_prep(p, s));
    if (st != G4ATTN_OK) return st;
    a.r = r; a.krot = krot; a.kv_rows = S;
  }
  return hip_status(g4attn::launch_prefill(a, s));
}

// Checks and arguments both chunked prefills share (queries, positions,
// spans, outputs, workspace); the caller adds its caches and scale.
static g4attn_status chunk_args(const g4attn_layer_desc* d, const g4attn_bf16* q, int32_t cache_cap,
                                const int32_t* pos0, const int32_t* qlen, int32_t max_pos, const int32_t* span_lo,
                                const int32_t* span_hi, g4attn_bf16* out, float* lse, int32_t B, int32_t S,
                                const int64_t q_strides[3], const int64_t o_strides[3], void* workspace,
                                size_t workspace_bytes, g4attn::PrefillArgs& a) {
  if (!q || !pos0 || !qlen || !out || !q_strides || !o_strides) return G4ATTN_ERR_NULL;
  if (!span_lo != !span_hi) return G4ATTN_ERR_NULL;
  if (B < 1 || S < 1 || B > 65535 || cache_cap < 1 || max_pos < 0) return G4ATTN_ERR_SHAPE;
  if ((int64_t)S * (d->num_q_heads / d->num_kv_heads) > (int64_t)INT32_MAX) return G4ATTN_ERR_SHAPE;
  if (max_pos >= cache_cap) return G4ATTN_ERR_CACHE_OVERFLOW;
  if (!aligned16(q) || !aligned16(out) || (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return G4ATTN_ERR_LAYOUT;
  if (!strides_ok(q_strides) || !strides_ok(o_strides)) return G4ATTN_ERR_LAYOUT;
  // only the flags: a chunk reads its key side data from the caches
  const size_t need = prefill_ws(d, B, S).r;
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return G4ATTN_ERR_WORKSPACE;
  a = g4attn::PrefillArgs{};
  a.q = q; a.out = out; a.lse = lse;
  a.pos0 = pos0; a.qlen = qlen; a.max_pos = max_pos;
  a.span_lo = span_lo; a.span_hi = span_hi;
  a.B = B; a.S = S; a.Hq = d->num_q_heads; a.Hkv = d->num_kv_heads; a.D = d->head_dim;
  a.window = d->window; a.kv_tied = d->k_eq_v;
  a.qmul = 1.f; a.omul = 1.f;
  // caches [B, Hkv, cap, D]: batch, key (row) and head strides in elements
  a.ks[0] = (int64_t)d->num_kv_heads * cache_cap * d->head_dim;
  a.ks[1] = d->head_dim;
  a.ks[2] = (int64_t)cache_cap * d->head_dim;
  for (int i = 0; i < 3; ++i) { a.qs[i] = q_strides[i]; a.os[i] = o_strides[i]; }
  a.flags = (int*)workspace;
  return G4ATTN_OK;
}

g4attn_status g4attn_prefill_chunk(const g4attn_layer_desc* d, const g4attn_bf16* q,
                                   const g4attn_bf16* k_cache, const g4attn_bf16* v_cache, int32_t cache_cap,
                                   const int32_t* pos0, const int32_t* qlen, int32_t max_pos,
                                   const int32_t* span_lo, const int32_t* span_hi,
                                   g4attn_bf16* out, float* lse, int32_t B, int32_t S,
                                   const int64_t q_strides[3], const int64_t o_strides[3], void* workspace,
                                   size_t workspace_bytes, void* stream) {
  g4attn_status st = desc_check(d);
  if (st != G4ATTN_OK) return st;
  if (!k_cache || !v_cache) return G4ATTN_ERR_NULL;
  if (d->k_eq_v) return G4ATTN_ERR_UNSUPPORTED;  // its cache is g4attn_prefill_chunk_tied's
  g4attn::PrefillArgs a;
  st = chunk_args(d, q, cache_cap, pos0, qlen, max_pos, span_lo, span_hi, out, lse, B, S, q_strides, o_strides,
                  workspace, workspace_bytes, a);
  if (st != G4ATTN_OK) return st;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return G4ATTN_ERR_LAYOUT;
  a.k = k_cache; a.v = v_cache;
  a.scale_log2 = d->scale * g4attn::kLog2e;
  if (a.scale_log2 == 0.f) a.scale_log2 = 0x1p-126f;
  a.mask_s = a.scale_log2 < 0.f ? INFINITY : -INFINITY;
  return hip_status(g4attn::launch_prefill(a, (hipStream_t)stream));
}

g4attn_status g4attn_prefill_chunk_tied(const g4attn_layer_desc* d, const g4attn_bf16* q,
                                        const g4attn_bf16* x_cache, const float* r_cache,
                                        const g4attn_bf16* krot_cache, const g4attn_bf16* w_k, int32_t cache_cap,
                                        const int32_t* pos0, const int32_t* qlen, int32_t max_pos,
                                        const int32_t* span_lo, const int32_t* span_hi, g4attn_bf16* out,
                                        float* lse, int32_t B, int32_t S, const int64_t q_strides[3],
                                        const int64_t o_strides[3], void* workspace, size_t workspace_bytes,
                                        void* stream) {
  g4attn_status st = desc_check(d);
  if (st != G4ATTN_OK) return st;
  if (!x_cache || !r_cache || !krot_cache || !w_k) return G4ATTN_ERR_NULL;
  if (!d->k_eq_v || d->head_dim != 512 || d->rotary_dims != 128) return G4ATTN_ERR_UNSUPPORTED;
  if (!(fabsf(d->scale) <= 0x1p30f)) return G4ATTN_ERR_UNSUPPORTED;
  g4attn::PrefillArgs a;
  st = chunk_args(d, q, cache_cap, pos0, qlen, max_pos, span_lo, span_hi, out, lse, B, S, q_strides, o_strides,
                  workspace, workspace_bytes, a);
  if (st != G4ATTN_OK) return st;
  if (!aligned16(x_cache) || !aligned16(krot_cache) || !aligned16(w_k) ||
      (reinterpret_cast<uintptr_t>(r_cache) & 3u))
    return G4ATTN_ERR_LAYOUT;
  a.k = x_cache; a.v = nullptr; a.w_k = w_k;
  a.r = r_cache; a.krot = krot_cache; a.kv_rows = cache_cap;
  // The cached r carries no logit scale, so scale * log2(e) rides on the
  // queries; the key factor r > 0 keeps -inf for masked slots.
  a.scale_log2 = d->scale * g4attn::kLog2e;
  a.qmul = a.scale_log2;
  a.mask_s = -INFINITY;
  return hip_status(g4attn::launch_prefill(a, (hipStream_t)stream));
}

size_t g4attn_decode_workspace_bytes(const g4attn_layer_desc* d, int32_t B, int32_t max_kv_len,
                                     int32_t num_splits) {
  if (!d || B < 1 || max_kv_len < 1 || num_splits < 0 || d->num_kv_heads < 1 || d->num_q_heads < 1 ||
      !head_dim_ok(d->head_dim))
    return 0;
  const int32_t rows = decode_rows(d, max_kv_len);
  const int64_t c = decode_chunk(d, B, rows, num_splits);
  const int64_t ns = ((int64_t)rows + c - 1) / c;
  const size_t ph = (size_t)B * d->num_q_heads;
  const size_t pg = (size_t)B * d->num_kv_heads;
  return align256(ph * ns * d->head_dim * sizeof(float)) + 2 * align256(ph * ns * sizeof(float)) +
         align256(pg * ns * sizeof(int));
}

g4attn_status g4attn_decode(const g4attn_layer_desc* d, const g4attn_bf16* q,
                            const g4attn_bf16* k_cache, const g4attn_bf16* v_cache,
                            const int32_t* kv_len, int32_t B, int32_t max_kv_len,
                            int32_t cache_cap, g4attn_bf16* out, float* lse, int32_t num_splits,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return g4attn::decode_run(d, q, k_cache, v_cache, kv_len, B, max_kv_len, cache_cap, out, lse, num_splits,
                            workspace, workspace_bytes, (hipStream_t)stream);
}

g4attn_status g4attn_kv_tied_append(const g4attn_bf16* x, const g4attn_bf16* w_k, int32_t B, int32_t S,
                                    int32_t Hkv, int32_t rotary_dims, float rope_theta, float rms_eps,
                                    const int64_t x_strides[3], const int32_t* pos0, int32_t max_pos,
                                    g4attn_bf16* x_cache, float* r_cache, g4attn_bf16* krot_cache,
                                    int32_t cache_cap, void* stream) {
  if (!x || !w_k || !x_strides || !x_cache || !r_cache || !krot_cache) return G4ATTN_ERR_NULL;
  if (B < 1 || S < 1 || Hkv < 1 || B > 65535 || cache_cap < 1) return G4ATTN_ERR_SHAPE;
  if (rotary_dims != 128) return G4ATTN_ERR_UNSUPPORTED;
  if (!(rope_theta > 0.f) || !isfinite(rope_theta) || !(rms_eps >= 0.f) || !isfinite(rms_eps))
    return G4ATTN_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(w_k) || !aligned16(x_cache) || !aligned16(krot_cache) ||
      (reinterpret_cast<uintptr_t>(r_cache) & 3u))
    return G4ATTN_ERR_LAYOUT;
  if (!strides_ok(x_strides)) return G4ATTN_ERR_LAYOUT;
  if (pos0 && max_pos < S - 1) return G4ATTN_ERR_SHAPE;
  const int64_t top = pos0 ? (int64_t)max_pos : (int64_t)S - 1;
  if (top >= cache_cap) return G4ATTN_ERR_CACHE_OVERFLOW;
  g4attn::KvPrepArgs p{};
  p.x = x; p.w_k = w_k; p.r = r_cache; p.krot = krot_cache; p.x_out = x_cache;
  p.pos0 = pos0; p.cap = cache_cap;
  p.B = B; p.S = S; p.Hkv = Hkv; p.rot = rotary_dims;
  p.log2_theta = log2((double)rope_theta);
  p.eps = rms_eps;
  p.rscale = 1.f;
  for (int i = 0; i < 3; ++i) p.xs[i] = x_strides[i];
  return hip_status(g4attn::launch_kv_prep(p, (hipStream_t)stream));
}

g4attn_status g4attn_decode_tied(const g4attn_layer_desc* d, const g4attn_bf16* q, const g4attn_bf16* x_cache,
                                 const float* r_cache, const g4attn_bf16* krot_cache, const g4attn_bf16* w_k,
                                 const int32_t* kv_len, int32_t B, int32_t max_kv_len, int32_t cache_cap,
                                 g4attn_bf16* out, float* lse, int32_t num_splits, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  g4attn_status st = desc_check(d);
  if (st != G4ATTN_OK) return st;
  if (!q || !x_cache || !r_cache || !krot_cache || !w_k || !kv_len || !out) return G4ATTN_ERR_NULL;
  if (!d->k_eq_v || d->head_dim != 512 || d->rotary_dims != 128 || d->window != 0) return G4ATTN_ERR_UNSUPPORTED;
  if (d->num_q_heads / d->num_kv_heads > 16) return G4ATTN_ERR_UNSUPPORTED;
  if (B < 1 || B > 65535 || max_kv_len < 1 || cache_cap < 1 || num_splits < 0) return G4ATTN_ERR_SHAPE;
  if (max_kv_len > cache_cap) return G4ATTN_ERR_CACHE_OVERFLOW;
  if (!aligned16(q) || !aligned16(x_cache) || !aligned16(krot_cache) || !aligned16(w_k) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(r_cache) & 3u) || (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return G4ATTN_ERR_LAYOUT;
  const int64_t c = decode_chunk(d, B, max_kv_len, num_splits);
  const int64_t ns = ((int64_t)max_kv_len + c - 1) / c;
  if (ns > 65535) return G4ATTN_ERR_SHAPE;
  const size_t need = g4attn_decode_workspace_bytes(d, B, max_kv_len, num_splits);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return G4ATTN_ERR_WORKSPACE;

  const size_t ph = (size_t)B * d->num_q_heads;
  g4attn::DecodeArgs a{};
  a.q = q; a.kc = x_cache; a.vc = x_cache; a.kv_len = kv_len; a.out = out; a.lse = lse;
  a.rc = r_cache; a.krc = krot_cache; a.w_k = w_k;
  char* wsp = (char*)workspace;
  a.o_part = (float*)wsp;
  wsp += align256(ph * ns * d->head_dim * sizeof(float));
  a.lse_part = (float*)wsp;
  wsp += align256(ph * ns * sizeof(float));
  a.dmax = (float*)wsp;
  wsp += align256(ph * ns * sizeof(float));
  a.dflags = (int*)wsp;
  a.B = B; a.Hq = d->num_q_heads; a.Hkv = d->num_kv_heads; a.D = d->head_dim; a.cap = cache_cap;
  a.nsplit = (int)ns; a.chunk = (int)c; a.max_len = max_kv_len;
  a.scale_log2 = d->scale * g4attn::kLog2e;
  return hip_status(g4attn::launch_decode_tied(a, (hipStream_t)stream));
}

}  // extern "C"
