// Fused QK-norm / V-norm + RoPE prologue, and the K=V pre-pass.
//
// RMSNorm uses the weight as is, with no 1 + w offset; RoPE rotates the pair
// (j, j + D/2) by the angle p * f_j, f_j = theta^(-2j/D) for the first
// rotary_dims/2 pairs and 0 for the rest ("Gemma 4" Keras docs, "What changed
// from Gemma 3"; vinija.ai Gemma 4 primer, "Dual RoPE configurations").
//
// Mapping: one wavefront per token, looping over that token's heads, so each
// lane forms the sines and cosines of its pairs once per token.  Lane l holds
// pairs j = E*l .. E*l+E-1 (E = D/128), i.e. dims [E*l, E*l+E) of the first
// half and the matching dims of the second half: every load and store of a
// wave covers contiguous bytes, and each pair stays inside one lane.
#include "g4attn_internal.h"

namespace g4attn {

namespace {

constexpr int kWaves = 4;

template <int E>
struct Vec;
template <>
struct Vec<2> {  // 2 bf16 = 4 bytes
  static __device__ __forceinline__ void load(const uint16_t* p, float* o) {
    uint32_t w = *(const uint32_t*)p;
    o[0] = bf_lo(w); o[1] = bf_hi(w);
  }
  static __device__ __forceinline__ void store(uint16_t* p, const float* v) {
    *(uint32_t*)p = pack_bf2(v[0], v[1]);
  }
};
template <>
struct Vec<4> {  // 4 bf16 = 8 bytes
  static __device__ __forceinline__ void load(const uint16_t* p, float* o) {
    u32x2 w = *(const u32x2*)p;
    o[0] = bf_lo(w[0]); o[1] = bf_hi(w[0]); o[2] = bf_lo(w[1]); o[3] = bf_hi(w[1]);
  }
  static __device__ __forceinline__ void store(uint16_t* p, const float* v) {
    u32x2 w; w[0] = pack_bf2(v[0], v[1]); w[1] = pack_bf2(v[2], v[3]);
    *(u32x2*)p = w;
  }
};

// cos/sin of p * f with the product and its reduction to [-pi, pi] in fp64.
__device__ __forceinline__ void rope_angle(double p, double f, float& c, float& s) {
  const double two_pi_hi = 6.283185307179586;
  const double two_pi_lo = 2.4492935982947064e-16;
  double a = p * f;
  double k = rint(a * 0.15915494309189535);
  double red = fma(-k, two_pi_hi, a);
  red = fma(-k, two_pi_lo, red);
  sincosf((float)red, &s, &c);
}

template <int D>
__global__ __launch_bounds__(256) void norm_rope_kernel(NormRopeArgs a) {
  constexpr int E = D / 128;
  constexpr int HALF = D / 2;
  const int lane = threadIdx.x & 63;
  const int64_t tok = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (tok >= (int64_t)a.B * a.S) return;
  const int b = (int)(tok / a.S);
  const int t = (int)(tok % a.S);
  const int p = (a.pos0 ? a.pos0[b] : 0) + t;
  const int j0 = E * lane;
  const int live = a.rot / 2;

  float c[E], s[E], wl[E], wh[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = j0 + e;
    if (j < live) {
      const double f = exp2(-2.0 * (double)j / (double)D * a.log2_theta);
      rope_angle((double)p, f, c[e], s[e]);
    } else {
      c[e] = 1.f; s[e] = 0.f;
    }
  }
  if (a.w) {
    Vec<E>::load(a.w + j0, wl);
    Vec<E>::load(a.w + HALF + j0, wh);
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) { wl[e] = 1.f; wh[e] = 1.f; }
  }
  const bool cache = a.cache_cap > 0;
  // linear cache: row p, p in [0, cap); ring: row p mod cap, and of the S
  // new positions only the last cap are kept (earlier ones would be
  // overwritten within this call).
  if (cache && (p < 0 || (a.ring ? t < a.S - a.cache_cap : p >= a.cache_cap))) return;
  const int row = cache && a.ring ? p % a.cache_cap : p;

  for (int h = 0; h < a.H; ++h) {
    const uint16_t* xr = a.x + b * a.xs[0] + t * a.xs[1] + h * a.xs[2];
    float lo[E], hi[E];
    Vec<E>::load(xr + j0, lo);
    Vec<E>::load(xr + HALF + j0, hi);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) ss += lo[e] * lo[e] + hi[e] * hi[e];
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)D + a.eps);
    float ylo[E], yhi[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float u = lo[e] * r * wl[e];
      const float v = hi[e] * r * wh[e];
      if (j0 + e < live) {
        ylo[e] = u * c[e] - v * s[e];
        yhi[e] = v * c[e] + u * s[e];
      } else {
        ylo[e] = u;
        yhi[e] = v;
      }
    }
    uint16_t* yr = cache ? a.y + (((int64_t)b * a.H + h) * a.cache_cap + row) * D
                         : a.y + b * a.ys[0] + t * a.ys[1] + h * a.ys[2];
    Vec<E>::store(yr + j0, ylo);
    Vec<E>::store(yr + HALF + j0, yhi);
  }
}

// K=V pre-pass on the raw tied projection X (D = 512, 128 rotated dims),
// for the prefill (rows t of [B, Hkv, S]) or appending to a decode cache
// (rows pos0[b] + t of [B, Hkv, cap], X copied into its cache as well):
//   r[b,g,t]      = rscale / sqrt(mean_d X^2 + eps)   (the inverse RMS, with
//                   the logit scale folded in by the caller)
//   krot[b,g,t,:] = RoPE_t(X * w_k) on dims 0..63 and 256..319 (no r)
// so that the attention kernel can form K = r * RoPE(X * w_k) and V = r * X
// from one tile of X (see prefill.hip).
__global__ __launch_bounds__(256) void kv_prep_kernel(KvPrepArgs a) {
  constexpr int D = 512, E = 4, HALF = 256;
  const int lane = threadIdx.x & 63;
  const int64_t tok = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (tok >= (int64_t)a.B * a.S) return;
  const int b = (int)(tok / a.S);
  const int t = (int)(tok % a.S);
  // prefill layout: row t of [B, Hkv, S]; cache layout: row p = pos0[b] + t
  // of [B, Hkv, cap], with the raw row copied into the X cache too
  const int p = a.cap ? (a.pos0 ? a.pos0[b] : 0) + t : t;
  if (a.cap && (p < 0 || p >= a.cap)) return;
  const int nrows = a.cap ? a.cap : a.S;
  const int j0 = E * lane;
  const int live = a.rot / 2;  // 64
  const bool rot_lane = j0 < live;
  float c[E], s[E], wl[E], wh[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (rot_lane) {
      const double f = exp2(-2.0 * (double)(j0 + e) / (double)D * a.log2_theta);
      rope_angle((double)p, f, c[e], s[e]);
    } else {
      c[e] = 1.f; s[e] = 0.f;
    }
  }
  Vec<E>::load(a.w_k + j0, wl);
  Vec<E>::load(a.w_k + HALF + j0, wh);
  for (int g = 0; g < a.Hkv; ++g) {
    const uint16_t* xr = a.x + b * a.xs[0] + t * a.xs[1] + g * a.xs[2];
    float lo[E], hi[E];
    Vec<E>::load(xr + j0, lo);
    Vec<E>::load(xr + HALF + j0, hi);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) ss += lo[e] * lo[e] + hi[e] * hi[e];
    ss = wave_sum(ss);
    const int64_t row = ((int64_t)b * a.Hkv + g) * nrows + p;
    if (lane == 0) a.r[row] = a.rscale / sqrtf(ss / (float)D + a.eps);
    if (a.x_out) {
      Vec<E>::store(a.x_out + row * D + j0, lo);    // exact: bf16 in, bf16 out
      Vec<E>::store(a.x_out + row * D + HALF + j0, hi);
    }
    if (rot_lane) {
      float ylo[E], yhi[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float u = lo[e] * wl[e];
        const float v = hi[e] * wh[e];
        ylo[e] = u * c[e] - v * s[e];
        yhi[e] = v * c[e] + u * s[e];
      }
      uint16_t* kr = a.krot + row * 128;
      Vec<E>::store(kr + j0, ylo);
      Vec<E>::store(kr + 64 + j0, yhi);
    }
  }
}

}  // namespace

hipError_t launch_norm_rope(const NormRopeArgs& a, hipStream_t st) {
  const int64_t toks = (int64_t)a.B * a.S;
  const dim3 grid((unsigned)((toks + kWaves - 1) / kWaves));
  if (a.D == 256)
    hipLaunchKernelGGL(norm_rope_kernel<256>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(norm_rope_kernel<512>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_kv_prep(const KvPrepArgs& a, hipStream_t st) {
  const int64_t toks = (int64_t)a.B * a.S;
  const dim3 grid((unsigned)((toks + kWaves - 1) / kWaves));
  hipLaunchKernelGGL(kv_prep_kernel, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace g4attn
