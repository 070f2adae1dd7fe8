// Split-KV single-token decode and its log-sum-exp combine (gfx950).
//
// For each sequence b with n_b visible cache rows, query head h and KV head
// g = h / (Hq/Hkv):
//   out[b,h] = sum_{j<n_b} softmax_j(scale q.K[b,g,j]) V[b,g,j]
// [vinija.ai Gemma 4 primer, "KV cache and long-context scaling";
// gemma4-pt-claude README, "KV Cache"].  The cache is read once: every
// workgroup owns one (b, g, chunk of rows) and all Hq/Hkv query heads of the
// group, so each cache row fetched from HBM serves every head that uses it;
// when the value cache is the key cache (one tensor for both), one LDS tile
// feeds both products.
//
// Per wave: 16-row tiles, double-buffered in the wave's own LDS region with
// direct global->LDS loads (no workgroup barrier in the loop).
//   S^T[16 keys x 16 heads] = K Q^T      v_mfma_f32_16x16x32_bf16
//   O^T[16 dims x 16 heads] += V^T P^T   v_mfma_f32_16x16x16_bf16, with V^T
//                                         fed by the transposing LDS read
// (columns past Hq/Hkv heads are zero padding).  The 4 waves' partial
// softmax states are merged in LDS; each chunk writes (O/l, lse) in fp32 and
// decode_combine_kernel merges the chunks:
//   lse = log sum_s exp(lse_s),  out = sum_s exp(lse_s - lse) O_s.
#include "g4attn_internal.h"

namespace g4attn {
namespace {

constexpr int kSegD = 1056;  // bytes per LDS row segment (1 KiB + 32)
constexpr int kRows = 16;    // keys per wave tile

typedef short i16x4_t __attribute__((ext_vector_type(4)));

template <int D>
__device__ __forceinline__ int d_row_off(int R) {
  return D == 512 ? R * kSegD : (R & 7) * kSegD + (R >> 3) * 512;
}
__device__ __forceinline__ int d_xor(int R) { return (R >> 3) & 1; }

template <int D, bool SAME_KV>
struct DCfg {
  static constexpr int TILE = (D == 512 ? 16 : 8) * kSegD;
  static constexpr int STAGE = TILE * (SAME_KV ? 1 : 2);
  static constexpr int WAVES = SAME_KV ? 4 : 2;
  static constexpr int NT = D / 32;  // QK^T k-steps
  static constexpr int NC = D / 16;  // PV dim blocks
};

template <int D>
__device__ __forceinline__ void load_rows(const uint16_t* base, int row0, int nrows, char* tile, int lane) {
  // rows row0 .. row0+15 of one (b, g) cache slice; rows >= nrows are
  // clamped to the last valid row (they are masked out of the softmax).
  if (D == 512) {
#pragma unroll
    for (int R = 0; R < kRows; ++R) {
      int row = row0 + R;
      row = row < nrows ? row : nrows - 1;
      const int ch = lane ^ d_xor(R);
      g2lds16(base + (int64_t)row * D + ch * 8, (G4_LDS void*)(tile + d_row_off<D>(R)));
    }
  } else {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int R = s + 8 * (lane >> 5);
      int row = row0 + R;
      row = row < nrows ? row : nrows - 1;
      const int ch = (lane & 31) ^ d_xor(R);
      g2lds16(base + (int64_t)row * D + ch * 8, (G4_LDS void*)(tile + s * kSegD));
    }
  }
}

template <int D, bool SAME_KV>
__global__ __launch_bounds__((SAME_KV ? 4 : 2) * 64) void decode_split_kernel(DecodeArgs a) {
  typedef DCfg<D, SAME_KV> C;
  __shared__ __attribute__((aligned(1024))) char smem[C::WAVES * 2 * C::STAGE];
  __shared__ float s_m[C::WAVES][16], s_l[C::WAVES][16];

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = a.Hq / a.Hkv;
  const int n = min(max(a.kv_len[b], 0), a.max_len);
  const int r0 = split * a.chunk;
  if (r0 >= n) return;  // beyond this sequence: the combine never reads it
  const int r1 = min(r0 + a.chunk, n);
  const int ntile = (r1 - r0 + kRows - 1) / kRows;

  const int64_t slice = ((int64_t)b * a.Hkv + g) * a.cap * D;
  const uint16_t* kbase = a.kc + slice;
  const uint16_t* vbase = a.vc + slice;
  char* mybuf = smem + wave * 2 * C::STAGE;

  // Q^T (B operand of the 16x16x32 MFMA): lane -> head (lane & 15), dims 32t + 8(lane >> 4) ..
  const int hcol = lane & 15, kq = lane >> 4;
  const bool hvalid = hcol < G;
  bf16x8 qf[C::NT];
  {
    const uint16_t* qrow = a.q + ((int64_t)b * a.Hq + g * G + (hvalid ? hcol : 0)) * D;
#pragma unroll
    for (int t = 0; t < C::NT; ++t) {
      u32x4 raw = hvalid ? *(const u32x4*)(qrow + 32 * t + 8 * kq) : u32x4{0, 0, 0, 0};
      qf[t] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  f32x4 oacc[C::NC];
#pragma unroll
  for (int c = 0; c < C::NC; ++c) oacc[c] = f32x4{};
  float m_run = -INFINITY, l_part = 0.f;

  const int k_rowoff = d_row_off<D>(lane & 15), k_x = d_xor(lane & 15);
  // transposing read: issuing lane feeds row 4*(lane>>4) + ((lane>>2)&3), dims 16cb + 4*(lane&3)
  const int tR = 4 * (lane >> 4) + ((lane >> 2) & 3);
  const int tq = lane & 3;
  const int tr_off = d_row_off<D>(tR) + (tq & 1) * 8;
  const int tr_j = (tq >> 1) ^ d_xor(tR);

  int it = 0;
  int tl = wave;
  if (tl < ntile) {
    load_rows<D>(kbase, r0 + tl * kRows, r1, mybuf, lane);
    if (!SAME_KV) load_rows<D>(vbase, r0 + tl * kRows, r1, mybuf + C::TILE, lane);
  }
  for (; tl < ntile; tl += C::WAVES, ++it) {
    wait_vmem_all();  // this tile has landed (only this wave's loads are in flight)
    char* cur = mybuf + (it & 1) * C::STAGE;
    const int nx = tl + C::WAVES;
    if (nx < ntile) {
      char* nxt = mybuf + ((it + 1) & 1) * C::STAGE;
      load_rows<D>(kbase, r0 + nx * kRows, r1, nxt, lane);
      if (!SAME_KV) load_rows<D>(vbase, r0 + nx * kRows, r1, nxt + C::TILE, lane);
    }

    f32x4 sacc = f32x4{};
#pragma unroll
    for (int t = 0; t < C::NT; ++t) {
      const int ch = (4 * t + kq) ^ k_x;
      const bf16x8 ka = lds_read_b128((const G4_LDS char*)(cur + k_rowoff + ch * 16));
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[t], sacc, 0, 0, 0);
    }
    // lane holds head hcol, keys 4*kq + i of this tile
    const int key0 = r0 + tl * kRows + 4 * kq;
    float s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = (key0 + i < r1) ? sacc[i] * a.scale_log2 : -INFINITY;
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    float p[4], ps = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) { p[i] = __builtin_amdgcn_exp2f(s[i] - m_use); ps += p[i]; }
    l_part = l_part * alpha + ps;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int c = 0; c < C::NC; ++c) oacc[c] *= alpha;
    }
    const u32x2 pw = {pack_bf2(p[0], p[1]), pack_bf2(p[2], p[3])};
    const i16x4_t pb = __builtin_bit_cast(i16x4_t, pw);
    const char* vt = SAME_KV ? cur : cur + C::TILE;
#pragma unroll
    for (int c = 0; c < C::NC; ++c) {
      const i16x4 va = lds_read_tr16((const G4_LDS char*)(vt + tr_off + (2 * c + tr_j) * 16));
      oacc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, oacc[c], 0, 0, 0);
    }
  }

  // ---- merge the waves' partial states
  float l_tot = l_part + __shfl_xor(l_part, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  if (lane < 16) { s_m[wave][lane] = m_run; s_l[wave][lane] = l_tot; }
  __syncthreads();  // all waves are done with their tiles; reuse LDS for O
  float* so = (float*)smem;  // [WAVES][16 heads][D]
  if (hvalid) {
#pragma unroll
    for (int c = 0; c < C::NC; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) so[(wave * 16 + hcol) * D + 16 * c + 4 * kq + i] = oacc[c][i];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += C::WAVES * 64) {
    const int hh = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < C::WAVES; ++w) M = fmaxf(M, s_m[w][hh]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < C::WAVES; ++w) {
      const float wt = s_m[w][hh] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s_m[w][hh] - M);
      L += wt * s_l[w][hh];
      O += wt * so[(w * 16 + hh) * D + d];
    }
    const int64_t ph = (int64_t)b * a.Hq + g * G + hh;
    a.o_part[(ph * a.nsplit + split) * D + d] = O / L;
    if (d == 0) a.lse_part[ph * a.nsplit + split] = (M + __log2f(L)) * kLn2;
  }
}

template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int n = min(max(a.kv_len[b], 0), a.max_len);
  const int ns = (n + a.chunk - 1) / a.chunk;
  const int64_t ph = (int64_t)b * a.Hq + h;
  if (ns == 0) {  // no visible row: zeros and lse = -inf
    for (int d = threadIdx.x; d < D; d += 256) a.out[ph * D + d] = 0;
    if (a.lse && threadIdx.x == 0) a.lse[ph] = -INFINITY;
    return;
  }
  const float* lp = a.lse_part + ph * a.nsplit;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, lp[s]);
  float L = 0.f;
  for (int s = 0; s < ns; ++s) L += __expf(lp[s] - M);
  const float lse = M + __logf(L);
  for (int d = threadIdx.x; d < D; d += 256) {
    float o = 0.f;
    for (int s = 0; s < ns; ++s) o += __expf(lp[s] - lse) * a.o_part[(ph * a.nsplit + s) * D + d];
    a.out[ph * D + d] = (uint16_t)f2bf(o);
  }
  if (a.lse && threadIdx.x == 0) a.lse[ph] = lse;
}

template <int D, bool SAME>
hipError_t launch_d(const DecodeArgs& a, hipStream_t st) {
  typedef DCfg<D, SAME> C;
  hipLaunchKernelGGL((decode_split_kernel<D, SAME>), dim3(a.nsplit, a.Hkv, a.B), dim3(C::WAVES * 64), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(a.Hq, a.B), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  const bool same = a.kc == a.vc;
  if (a.D == 512) return same ? launch_d<512, true>(a, st) : launch_d<512, false>(a, st);
  return same ? launch_d<256, true>(a, st) : launch_d<256, false>(a, st);
}

}  // namespace g4attn
