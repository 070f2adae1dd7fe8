// Flash-style prefill attention on bf16 MFMA (gfx950).
//
// Computes, per batch b, query head h and row i,
//   out_i = sum_{j visible} softmax_j(scale q_i.k_j) v_j,  lse_i = log sum exp
// with j visible iff j <= i (global layer) or 0 <= i - j < w (sliding layer)
// [vinija.ai Gemma 4 primer, "Sliding-window attention" and "Global attention
// layers"], GQA head grouping h -> h / (Hq/Hkv).
//
// Work decomposition
//   * A workgroup (4 waves) owns 128 "rows": consecutive (token, head) pairs
//     of one KV group, token-major, so the G = Hq/Hkv query heads that share
//     a KV head share every K/V tile the workgroup loads.
//   * Each wave owns 32 rows.  It computes S^T = K Q^T and O^T = V^T P^T with
//     v_mfma_f32_32x32x16_bf16: lane l holds query row l%32 in both results,
//     so the online softmax is per lane plus one partner lane (l ^ 32).
//     Q^T stays in registers (D/4 VGPRs), O^T accumulates in D/2 registers.
//   * K/V tiles of 32 keys are double-buffered in LDS with direct
//     global->LDS loads; tiles wholly outside the causal/window band are
//     never visited and only edge tiles are masked element by element.
//
// K=V global layers (D = 512): keys are RoPE(RMS(X) w_k), values RMS(X), from
// one raw tensor X.  With r_p the inverse RMS of key row p and R the rotated
// dims, q.k_p = r_p (sum_{d not in R} (q_d w_d) X_pd + sum_{d in R} q_d Krot_pd)
// with Krot = RoPE(X w_k) on R, and sum_p P_ip v_p = sum_p (P_ip r_p) X_p.  So
// one LDS tile of X (plus the 128-dim Krot slice and r) feeds both MFMAs.
//
// LDS layout of a K/V/X tile: rows padded to 1088-byte segments (D = 256:
// rows R and R+16 share a segment); 16-byte chunks XOR-ed with
// ((segment >> 2) & 3).  16 rows read at one chunk (QK^T operand) and the
// 4-row x 64-byte pattern of the transposing read (PV operand) both hit
// distinct bank groups, and the transposing-read addresses stay affine in
// the dim block.
#include "g4attn_internal.h"

namespace g4attn {
namespace {

constexpr int kWaves = 4;
constexpr int kBM = 128;   // rows per workgroup
constexpr int kBN = 32;    // keys per tile
constexpr int kSeg = 1088; // bytes per LDS row segment

template <int D, bool TIED>
struct Cfg {
  static constexpr int KT_BYTES = (D == 512 ? 32 : 16) * kSeg;  // one K, V or X tile
  static constexpr int KR_OFF = TIED ? KT_BYTES : 2 * KT_BYTES;  // Krot tile offset
  static constexpr int KR_BYTES = TIED ? 8 * kSeg : 0;
  static constexpr int R_OFF = KR_OFF + KR_BYTES;
  static constexpr int R_BYTES = TIED ? 256 : 0;
  static constexpr int STAGE = R_OFF + R_BYTES;
  static constexpr int NT = D / 16;  // QK^T k-steps
  static constexpr int NC = D / 32;  // PV dim blocks
};

template <int D>
__device__ __forceinline__ int kv_seg(int R) { return D == 512 ? R : (R & 15); }
template <int D>
__device__ __forceinline__ int kv_row_off(int R) {
  return D == 512 ? R * kSeg : (R & 15) * kSeg + (R >> 4) * 512;
}
template <int D>
__device__ __forceinline__ int kv_xor(int R) { return (kv_seg<D>(R) >> 2) & 3; }
__device__ __forceinline__ int kr_row_off(int R) { return (R & 7) * kSeg + (R >> 3) * 256; }
__device__ __forceinline__ int kr_xor(int R) { return (R >> 2) & 3; }

// Is the 16-dim k-step t one of the rotated (Krot) dims 0..63 / 256..319?
__device__ __forceinline__ constexpr bool rot_step(int t) { return t < 4 || (t >= 16 && t < 20); }
__device__ __forceinline__ constexpr int rot_chunk(int t) { return t < 4 ? 2 * t : 8 + 2 * (t - 16); }

template <int D, bool TIED>
__device__ __forceinline__ void load_tile(const PrefillArgs& a, char* stage, int kt, int b, int g,
                                          int wave, int lane) {
  typedef Cfg<D, TIED> C;
  const int key0 = kt * kBN;
  const int64_t kb = b * a.ks[0] + g * a.ks[2];
  auto key_ptr = [&](const uint16_t* base, int R) {
    int key = key0 + R;
    key = key < a.S ? key : a.S - 1;  // rows past S are masked; stay in bounds
    return base + kb + key * a.ks[1];
  };
  const int ntile = TIED ? 1 : 2;
#pragma unroll
  for (int which = 0; which < ntile; ++which) {
    const uint16_t* src = which == 0 ? a.k : a.v;
    char* tile = stage + which * C::KT_BYTES;
    if (D == 512) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int R = wave * 8 + i;
        const int ch = lane ^ kv_xor<D>(R);
        g2lds16(key_ptr(src, R) + ch * 8, (G4_LDS void*)(tile + kv_row_off<D>(R)));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = wave * 4 + i;
        const int R = s + 16 * (lane >> 5);
        const int ch = (lane & 31) ^ kv_xor<D>(R);
        g2lds16(key_ptr(src, R) + ch * 8, (G4_LDS void*)(tile + s * kSeg));
      }
    }
  }
  if (TIED) {
    const int64_t rowbase = ((int64_t)b * a.Hkv + g) * a.S;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int s = wave * 2 + i;
      const int R = s + 8 * (lane >> 4);
      int key = key0 + R;
      key = key < a.S ? key : a.S - 1;
      const int ch = (lane & 15) ^ kr_xor(R);
      g2lds16(a.krot + (rowbase + key) * 128 + ch * 8, (G4_LDS void*)(stage + C::KR_OFF + s * kSeg));
    }
    if (wave == 0) {
      int key = key0 + (lane & 31);
      key = key < a.S ? key : a.S - 1;
      __builtin_amdgcn_global_load_lds(a.r + rowbase + key, (G4_LDS void*)(stage + C::R_OFF), 4, 0, 0);
    }
  }
}

// REDO = false: main pass.  REDO = true: recompute the workgroups whose main
// pass flagged a reference overflow, with the row maxima the main pass found.
template <int D, bool TIED, bool REDO>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs a) {
  typedef Cfg<D, TIED> C;
  __shared__ __attribute__((aligned(1024))) char smem[2 * C::STAGE];

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int hh = lane >> 5;   // lane half
  const int lr = lane & 31;   // row within the wave
  const int G = a.Hq / a.Hkv;
  const int b = blockIdx.z;
  const int g = blockIdx.y;
  const int ntiles = (int)(((int64_t)a.S * G + kBM - 1) / kBM);
  const int tile = ntiles - 1 - (int)blockIdx.x;  // heaviest (latest) rows first

  const int64_t F0 = (int64_t)tile * kBM;
  const int64_t Flast = min(F0 + kBM - 1, (int64_t)a.S * G - 1);
  const int tq0 = (int)(F0 / G), tq1 = (int)(Flast / G);
  const int64_t F = F0 + wave * 32 + lr;
  const int tq = (int)(F / G);
  const int head = g * G + (int)(F % G);
  const bool valid = tq < a.S;

  const int kt_lo = a.window ? max(0, tq0 - a.window + 1) / kBN : 0;
  const int kt_hi = tq1 / kBN;
  int* wg_flags = a.flags + (((int64_t)b * a.Hkv + g) * ntiles + tile) * kWaves;
  const int64_t mrow_idx = ((int64_t)b * a.Hq + head) * a.S + tq;
  if (REDO) {
    if ((wg_flags[0] | wg_flags[1] | wg_flags[2] | wg_flags[3]) == 0) return;
  }

  // Prefetch the first tile, then load this lane's Q^T fragments.
  load_tile<D, TIED>(a, smem, kt_lo, b, g, wave, lane);

  bf16x8 qf[C::NT];
  {
    const uint16_t* qrow = a.q + b * a.qs[0] + (int64_t)(valid ? tq : 0) * a.qs[1] + head * a.qs[2];
#pragma unroll
    for (int t = 0; t < C::NT; ++t) {
      const int d0 = 16 * t + 8 * hh;
      u32x4 raw = valid ? *(const u32x4*)(qrow + d0) : u32x4{0, 0, 0, 0};
      if (TIED && !rot_step(t)) {
        const u32x4 w = *(const u32x4*)(a.w_k + d0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          raw[i] = pack_bf2(bf_lo(raw[i]) * bf_lo(w[i]), bf_hi(raw[i]) * bf_hi(w[i]));
      }
      qf[t] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  // Per-lane constant parts of the LDS addresses.
  const int k_rowoff = kv_row_off<D>(lr), k_x = kv_xor<D>(lr);
  const int kr_rowoff = kr_row_off(lr), kr_x = kr_xor(lr);
  // transposing read: issuing lane -> (row, chunk) of the 4x16 block it feeds
  const int tG = lane >> 4, te = (lane >> 2) & 3, tqd = lane & 3;
  const int tr_row0 = 4 * (tG >> 1) + te;                  // + 16 m + 8 u
  const int tr_chunk = 2 * (tG & 1) + (tqd >> 1);          // + 4 c
  const int tr_byte = (tqd & 1) * 8;

  // Softmax with a fixed per-row reference: m_ref (log2 domain) is the row's
  // maximum over its first tile with a visible key, and P = exp2(s - m_ref)
  // is accumulated without ever rescaling O.  m_true tracks the real maximum;
  // a wave whose rows end more than kHeadroom above m_ref flags its
  // workgroup, which the REDO launch recomputes with m_ref = m_true (every
  // P <= 1 then).
  constexpr float kHeadroom = 64.f;
  f32x16 oacc[C::NC];
#pragma unroll
  for (int c = 0; c < C::NC; ++c) oacc[c] = f32x16{};
  float m_ref = -INFINITY, m_true = -INFINITY, l_part = 0.f;
  if (REDO) m_ref = valid ? a.mrow[mrow_idx] : 0.f;

  {
    for (int kt = kt_lo; kt <= kt_hi; ++kt) {
      __syncthreads();  // tile kt has landed in LDS; every wave is done with tile kt-1
      char* cur = smem + ((kt - kt_lo) & 1) * C::STAGE;
      if (kt < kt_hi) load_tile<D, TIED>(a, smem + ((kt - kt_lo + 1) & 1) * C::STAGE, kt + 1, b, g, wave, lane);

      // ---- S^T = K Q^T (32 keys x 32 rows)
      f32x16 sacc = f32x16{};
#pragma unroll
      for (int t = 0; t < C::NT; ++t) {
        bf16x8 ka;
        if (TIED && rot_step(t)) {
          const int ch = (rot_chunk(t) + hh) ^ kr_x;
          ka = lds_read_b128((const G4_LDS char*)(cur + C::KR_OFF + kr_rowoff + ch * 16));
        } else {
          const int ch = (2 * t + hh) ^ k_x;
          ka = lds_read_b128((const G4_LDS char*)(cur + k_rowoff + ch * 16));
        }
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[t], sacc, 0, 0, 0);
        if ((t & 3) == 3) __builtin_amdgcn_sched_barrier(0);
      }

      // ---- scale (and K=V row factor), mask, exponentiate against m_ref
      float rk[16];
      if (TIED) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const f32x4 v = *(const G4_LDS f32x4*)(cur + C::R_OFF + (8 * gq + 4 * hh) * 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) rk[4 * gq + i] = v[i];
        }
      }
      float s[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = sacc[r] * a.scale_log2 * (TIED ? rk[r] : 1.f);
      const int key0 = kt * kBN;
      const bool full = (key0 + kBN - 1 <= tq0) && (a.window == 0 || key0 >= tq1 - a.window + 1);
      if (!full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 8 * (r >> 2) + 4 * hh + (r & 3);
          const int d = tq - key;
          const bool vis = d >= 0 && (a.window == 0 || d < a.window);
          s[r] = vis ? s[r] : -INFINITY;
        }
      }
      float mx = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
      m_true = fmaxf(m_true, mx);
      if (!REDO && __builtin_amdgcn_ballot_w64(m_ref == -INFINITY)) {  // a row meets its first visible key
        const float rowmx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        m_ref = m_ref == -INFINITY ? rowmx : m_ref;
      }
      const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = __builtin_amdgcn_exp2f(s[r] - m_use);
        l_part += p[r];
      }
      bf16x8 pb[2];
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r0 = 8 * mm + 2 * i;
          const float p0 = TIED ? p[r0] * rk[r0] : p[r0];
          const float p1 = TIED ? p[r0 + 1] * rk[r0 + 1] : p[r0 + 1];
          w[i] = pack_bf2(p0, p1);
        }
        pb[mm] = __builtin_bit_cast(bf16x8, w);
      }

      // ---- O^T += V^T P^T
      const char* vt = TIED ? cur : cur + C::KT_BYTES;
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        const int R0 = 16 * mm + tr_row0, R1 = R0 + 8;
        const char* p0 = vt + kv_row_off<D>(R0) + tr_byte;
        const char* p1 = vt + kv_row_off<D>(R1) + tr_byte;
        const int x0 = kv_xor<D>(R0), x1 = kv_xor<D>(R1);
#pragma unroll
        for (int c = 0; c < C::NC; ++c) {
          const int ch = 4 * c + tr_chunk;
          const i16x4 lo = lds_read_tr16((const G4_LDS char*)(p0 + (ch ^ x0) * 16));
          const i16x4 hi = lds_read_tr16((const G4_LDS char*)(p1 + (ch ^ x1) * 16));
          oacc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cat_tr(lo, hi), pb[mm], oacc[c], 0, 0, 0);
          if ((c & 3) == 3) __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }

  if (!REDO) {
    const float mt = fmaxf(m_true, __shfl_xor(m_true, 32, 64));
    const bool over = mt > m_ref + kHeadroom;
    if (lane == 0) wg_flags[wave] = __builtin_amdgcn_ballot_w64(over) != 0;
    if (valid && hh == 0) a.mrow[mrow_idx] = mt;
  }

  // ---- epilogue: normalise, round once to bf16, store
  const float l_tot = l_part + __shfl_xor(l_part, 32, 64);
  if (!valid) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  uint16_t* orow = a.out + b * a.os[0] + (int64_t)tq * a.os[1] + head * a.os[2];
#pragma unroll
  for (int c = 0; c < C::NC; ++c) {
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      u32x2 w;
      w[0] = pack_bf2(oacc[c][4 * gq + 0] * inv, oacc[c][4 * gq + 1] * inv);
      w[1] = pack_bf2(oacc[c][4 * gq + 2] * inv, oacc[c][4 * gq + 3] * inv);
      *(u32x2*)(orow + 32 * c + 8 * gq + 4 * hh) = w;
    }
  }
  if (a.lse && hh == 0) {
    a.lse[((int64_t)b * a.Hq + head) * a.S + tq] =
        l_tot > 0.f ? (m_ref + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  const int G = a.Hq / a.Hkv;
  const int64_t ntiles = ((int64_t)a.S * G + kBM - 1) / kBM;
  const dim3 grid((unsigned)ntiles, (unsigned)a.Hkv, (unsigned)a.B);
  for (int redo = 0; redo < 2; ++redo) {
    if (a.kv_tied)
      hipLaunchKernelGGL((redo ? prefill_kernel<512, true, true> : prefill_kernel<512, true, false>), grid,
                         dim3(256), 0, st, a);
    else if (a.D == 512)
      hipLaunchKernelGGL((redo ? prefill_kernel<512, false, true> : prefill_kernel<512, false, false>), grid,
                         dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((redo ? prefill_kernel<256, false, true> : prefill_kernel<256, false, false>), grid,
                         dim3(256), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace g4attn
