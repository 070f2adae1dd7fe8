// Fused QK-norm / V-norm + RoPE prologue, and the K=V pre-pass.
//
// RMSNorm uses the weight as is, with no 1 + w offset; RoPE rotates the pair
// (j, j + D/2) by the angle p * f_j, f_j = theta^(-2j/D) for the first
// rotary_dims/2 pairs and 0 for the rest ("Gemma 4" Keras docs, "What changed
// from Gemma 3"; vinija.ai Gemma 4 primer, "Dual RoPE configurations").
//
// Mapping: one wavefront per (token, group of up to 8 heads at D = 256, 4 at
// D = 512); the wave loads all its heads' rows, then forms the sines and
// cosines of its pairs once and normalises and rotates head by head.  Lane l holds
// pairs j = E*l .. E*l+E-1 (E = D/128), i.e. dims [E*l, E*l+E) of the first
// half and the matching dims of the second half: every load and store of a
// wave covers contiguous bytes, and each pair stays inside one lane.
#include "g4attn_internal.h"

namespace g4attn {

namespace {

constexpr int kWaves = 4;

// Row loads and stores of E bf16 per lane.  The activation rows are read
// once and written once, so they use the non-temporal policy (load_nt,
// store_nt); the weights, shared by every wave, use plain loads.
template <int E>
struct Vec;
template <>
struct Vec<2> {  // 2 bf16 = 4 bytes
  static __device__ __forceinline__ void unpack(uint32_t w, float* o) { o[0] = bf_lo(w); o[1] = bf_hi(w); }
  static __device__ __forceinline__ void load(const uint16_t* p, float* o) {
    unpack(*(const uint32_t*)p, o);
  }
  static __device__ __forceinline__ void load_nt(const uint16_t* p, float* o) {
    unpack(__builtin_nontemporal_load((const uint32_t*)p), o);
  }
  static __device__ __forceinline__ void store_nt(uint16_t* p, const float* v) {
    __builtin_nontemporal_store(pack_bf2(v[0], v[1]), (uint32_t*)p);
  }
};
template <>
struct Vec<4> {  // 4 bf16 = 8 bytes
  static __device__ __forceinline__ void unpack(u32x2 w, float* o) {
    o[0] = bf_lo(w[0]); o[1] = bf_hi(w[0]); o[2] = bf_lo(w[1]); o[3] = bf_hi(w[1]);
  }
  static __device__ __forceinline__ void load(const uint16_t* p, float* o) {
    unpack(*(const u32x2*)p, o);
  }
  static __device__ __forceinline__ void load_nt(const uint16_t* p, float* o) {
    unpack(__builtin_nontemporal_load((const u32x2*)p), o);
  }
  static __device__ __forceinline__ void store_nt(uint16_t* p, const float* v) {
    u32x2 w; w[0] = pack_bf2(v[0], v[1]); w[1] = pack_bf2(v[2], v[3]);
    __builtin_nontemporal_store(w, (u32x2*)p);
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

// Heads per wavefront: a wave issues the loads of all its HB heads before it
// reduces the first one, so HB rows per wave are in flight at once (one head
// per round trip left the prologues latency-bound: 5.2 TB/s on the 31B
// prefills, ~30 us for a 32-token decode step).  HB is the head count
// rounded up to a power of two, at most 8 rows (D = 256) or 4 (D = 512).
inline int heads_per_wave(int D, int H) {
  const int cap = D == 256 ? 8 : 4;
  int hb = 1;
  while (hb < H && hb < cap) hb *= 2;
  return hb;
}

template <int D, int HB>
__global__ __launch_bounds__(256) void norm_rope_kernel(NormRopeArgs a) {
  constexpr int E = D / 128;
  constexpr int HALF = D / 2;
  const int lane = threadIdx.x & 63;
  const int ngrp = (a.H + HB - 1) / HB;
  const int64_t wid = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (wid >= (int64_t)a.B * a.S * ngrp) return;
  const int64_t tok = wid / ngrp;
  const int h0 = (int)(wid - tok * ngrp) * HB;
  const int b = (int)(tok / a.S);
  const int t = (int)(tok % a.S);
  const int p = (a.pos0 ? a.pos0[b] : 0) + t;
  const int j0 = E * lane;
  const int live = a.rot / 2;

  const bool cache = a.cache_cap > 0;
  // linear cache: row p, p in [0, cap); ring: row p mod cap, and of the S
  // new positions only the last cap are kept (earlier ones would be
  // overwritten within this call).
  if (cache && (p < 0 || (a.ring ? t < a.S - a.cache_cap : p >= a.cache_cap))) return;
  const int row = cache && a.ring ? p % a.cache_cap : p;

  // The weights, then the rows (a tail group re-reads the last head instead
  // of branching; only heads below H are stored).  Loads complete in issue
  // order, so the small weight loads go first: waiting for them must not
  // wait for the rows as well.
  // Without a weight the loads read the wave's own first row instead (never
  // one another wave writes in place) and the factors are replaced by 1
  // after they arrive (a branch around the loads would wait for them inside
  // it).
  float c[E], s[E], wl[E], wh[E];
  const uint16_t* wsrc = a.w ? a.w : a.x + b * a.xs[0] + t * a.xs[1] + h0 * a.xs[2];
  Vec<E>::load(wsrc + j0, wl);
  Vec<E>::load(wsrc + HALF + j0, wh);
  float lo[HB][E], hi[HB][E];
#pragma unroll
  for (int i = 0; i < HB; ++i) {
    const int h = min(h0 + i, a.H - 1);
    const uint16_t* xr = a.x + b * a.xs[0] + t * a.xs[1] + h * a.xs[2];
    Vec<E>::load_nt(xr + j0, lo[i]);
    Vec<E>::load_nt(xr + HALF + j0, hi[i]);
  }

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

  if (!a.w) {
#pragma unroll
    for (int e = 0; e < E; ++e) { wl[e] = 1.f; wh[e] = 1.f; }
  }
#pragma unroll
  for (int i = 0; i < HB; ++i) {
    const int h = h0 + i;
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) ss += lo[i][e] * lo[i][e] + hi[i][e] * hi[i][e];
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)D + a.eps);
    float ylo[E], yhi[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float u = lo[i][e] * r * wl[e];
      const float v = hi[i][e] * r * wh[e];
      if (j0 + e < live) {
        ylo[e] = u * c[e] - v * s[e];
        yhi[e] = v * c[e] + u * s[e];
      } else {
        ylo[e] = u;
        yhi[e] = v;
      }
    }
    if (h < a.H) {
      uint16_t* yr = cache ? a.y + (((int64_t)b * a.H + h) * a.cache_cap + row) * D
                           : a.y + b * a.ys[0] + t * a.ys[1] + h * a.ys[2];
      Vec<E>::store_nt(yr + j0, ylo);
      Vec<E>::store_nt(yr + HALF + j0, yhi);
    }
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
template <int HB>
__global__ __launch_bounds__(256) void kv_prep_kernel(KvPrepArgs a) {
  constexpr int D = 512, E = 4, HALF = 256;
  const int lane = threadIdx.x & 63;
  const int ngrp = (a.Hkv + HB - 1) / HB;
  const int64_t wid = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (wid >= (int64_t)a.B * a.S * ngrp) return;
  const int64_t tok = wid / ngrp;
  const int g0 = (int)(wid - tok * ngrp) * HB;
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
  // the weights, then the rows of all the wave's heads, as in norm_rope_kernel
  float c[E], s[E], wl[E], wh[E];
  Vec<E>::load(a.w_k + j0, wl);
  Vec<E>::load(a.w_k + HALF + j0, wh);
  float lo[HB][E], hi[HB][E];
#pragma unroll
  for (int i = 0; i < HB; ++i) {
    const int g = min(g0 + i, a.Hkv - 1);
    const uint16_t* xr = a.x + b * a.xs[0] + t * a.xs[1] + g * a.xs[2];
    Vec<E>::load_nt(xr + j0, lo[i]);
    Vec<E>::load_nt(xr + HALF + j0, hi[i]);
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (rot_lane) {
      const double f = exp2(-2.0 * (double)(j0 + e) / (double)D * a.log2_theta);
      rope_angle((double)p, f, c[e], s[e]);
    } else {
      c[e] = 1.f; s[e] = 0.f;
    }
  }
#pragma unroll
  for (int i = 0; i < HB; ++i) {
    const int g = g0 + i;
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) ss += lo[i][e] * lo[i][e] + hi[i][e] * hi[i][e];
    ss = wave_sum(ss);
    if (g >= a.Hkv) continue;
    const int64_t row = ((int64_t)b * a.Hkv + g) * nrows + p;
    if (lane == 0) a.r[row] = a.rscale / sqrtf(ss / (float)D + a.eps);
    if (a.x_out) {
      Vec<E>::store_nt(a.x_out + row * D + j0, lo[i]);    // exact: bf16 in, bf16 out
      Vec<E>::store_nt(a.x_out + row * D + HALF + j0, hi[i]);
    }
    if (rot_lane) {
      float ylo[E], yhi[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float u = lo[i][e] * wl[e];
        const float v = hi[i][e] * wh[e];
        ylo[e] = u * c[e] - v * s[e];
        yhi[e] = v * c[e] + u * s[e];
      }
      uint16_t* kr = a.krot + row * 128;
      Vec<E>::store_nt(kr + j0, ylo);
      Vec<E>::store_nt(kr + 64 + j0, yhi);
    }
  }
}

}  // namespace

hipError_t launch_norm_rope(const NormRopeArgs& a, hipStream_t st) {
  const int hb = heads_per_wave(a.D, a.H);
  const int64_t waves = (int64_t)a.B * a.S * ((a.H + hb - 1) / hb);
  const dim3 grid((unsigned)((waves + kWaves - 1) / kWaves));
  const dim3 block(256);
  if (a.D == 256) {
    switch (hb) {
      case 1: hipLaunchKernelGGL((norm_rope_kernel<256, 1>), grid, block, 0, st, a); break;
      case 2: hipLaunchKernelGGL((norm_rope_kernel<256, 2>), grid, block, 0, st, a); break;
      case 4: hipLaunchKernelGGL((norm_rope_kernel<256, 4>), grid, block, 0, st, a); break;
      default: hipLaunchKernelGGL((norm_rope_kernel<256, 8>), grid, block, 0, st, a); break;
    }
  } else {
    switch (hb) {
      case 1: hipLaunchKernelGGL((norm_rope_kernel<512, 1>), grid, block, 0, st, a); break;
      case 2: hipLaunchKernelGGL((norm_rope_kernel<512, 2>), grid, block, 0, st, a); break;
      default: hipLaunchKernelGGL((norm_rope_kernel<512, 4>), grid, block, 0, st, a); break;
    }
  }
  return hipGetLastError();
}

hipError_t launch_kv_prep(const KvPrepArgs& a, hipStream_t st) {
  const int hb = heads_per_wave(512, a.Hkv);
  const int64_t waves = (int64_t)a.B * a.S * ((a.Hkv + hb - 1) / hb);
  const dim3 grid((unsigned)((waves + kWaves - 1) / kWaves));
  const dim3 block(256);
  switch (hb) {
    case 1: hipLaunchKernelGGL(kv_prep_kernel<1>, grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL(kv_prep_kernel<2>, grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL(kv_prep_kernel<4>, grid, block, 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace g4attn
