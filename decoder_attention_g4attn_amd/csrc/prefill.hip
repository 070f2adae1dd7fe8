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
#include "prefill_qk_asm.inc"

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

// Global->LDS copy of key tile kt.  The tile's base address is wave-uniform
// (scalar registers) and each lane adds an unsigned 32-bit byte offset (the
// scalar-base form of the load).  FULL: all 32 keys are < S; otherwise rows
// past S re-read row S-1 (they are masked).
template <int D, bool TIED, bool FULL>
__device__ __forceinline__ void load_tile_rows(const PrefillArgs& a, uint32_t stage, int kt, int b, int g,
                                               int wave, int lane) {
  typedef Cfg<D, TIED> C;
  const int key0 = kt * kBN;
  const int last = a.S - 1 - key0;  // last in-range row of the tile
  const int64_t rs = a.ks[1] * 2;   // key stride in bytes
  auto row_off = [&](int R) -> int64_t { return (int64_t)(FULL ? R : min(R, last)) * rs; };
  const int64_t tb = (b * a.ks[0] + g * a.ks[2] + (int64_t)key0 * a.ks[1]) * 2;
  const int ntile = TIED ? 1 : 2;
#pragma unroll
  for (int which = 0; which < ntile; ++which) {
    const char* src = (const char*)(which == 0 ? a.k : a.v) + tb;
    const uint32_t tile = stage + which * C::KT_BYTES;
    if (D == 512) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int R = wave * 8 + i;
        const uint32_t off = (uint32_t)(lane ^ kv_xor<D>(R)) * 16u;
        g2lds16s(src + row_off(R), off, tile + kv_row_off<D>(R));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // lanes 0..31 copy row s, lanes 32..63 row s + 16
        const int s = wave * 4 + i;
        const uint32_t d = (uint32_t)(row_off(s + 16) - row_off(s));
        const uint32_t off = (lane >> 5) * d + (uint32_t)((lane & 31) ^ kv_xor<D>(s)) * 16u;
        g2lds16s(src + row_off(s), off, tile + s * kSeg);
      }
    }
  }
  if (TIED) {
    const int64_t row0 = ((int64_t)b * a.Hkv + g) * a.S + key0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int s = wave * 2 + i;
      // lanes 16q .. 16q+15 copy Krot row s + 8q
      const int R = s + 8 * (lane >> 4);
      const int Re = FULL ? R : min(R, last);
      const uint32_t off = (uint32_t)Re * 256u + (uint32_t)((lane & 15) ^ kr_xor(R)) * 16u;
      g2lds16s(a.krot + row0 * 128, off, stage + C::KR_OFF + s * kSeg);
    }
    if (wave == 0) {
      const int R = lane & 31;
      const int Re = FULL ? R : min(R, last);
      g2lds4s(a.r + row0, (uint32_t)Re * 4u, stage + C::R_OFF);
    }
  }
}

template <int D, bool TIED>
__device__ __forceinline__ void load_tile(const PrefillArgs& a, uint32_t stage, int kt, int b, int g,
                                          int wave, int lane) {
  if (kt * kBN + kBN <= a.S)
    load_tile_rows<D, TIED, true>(a, stage, kt, b, g, wave, lane);
  else
    load_tile_rows<D, TIED, false>(a, stage, kt, b, g, wave, lane);
}

// Workgroup -> (batch b, KV group g, row tile) for the 8 XCDs of the chip.
// The dispatcher hands linear workgroup ids to the XCDs round-robin, and
// each XCD has its own L2.  With NG = B*Hkv groups of T tiles:
//   NG % 8 == 0          : each XCD takes NG/8 whole groups;
//   8 % NG == 0, T % (8/NG) == 0 : each group is spread over 8/NG XCDs, XCD
//                          c taking every (8/NG)-th tile in weight order;
//   otherwise            : plain order.
// so an XCD's L2 serves one group's keys instead of every group's, work
// per XCD stays balanced, and each XCD runs its heaviest (latest) tiles first.
__device__ __forceinline__ void wg_map(int T, int Hkv, int& b, int& g, int& tile) {
  constexpr int X = 8;
  const int NG = Hkv * (int)gridDim.z;
  const int L = (int)blockIdx.x + T * ((int)blockIdx.y + Hkv * (int)blockIdx.z);
  int grp, r;
  if (NG % X == 0) {
    const int xcd = L % X, k = L / X;
    grp = xcd * (NG / X) + k / T;
    r = k % T;
  } else if (X % NG == 0 && T % (X / NG) == 0) {
    const int m = X / NG, xcd = L % X, k = L / X;
    grp = xcd / m;
    r = k * m + xcd % m;
  } else {
    grp = (int)blockIdx.y + Hkv * (int)blockIdx.z;
    r = (int)blockIdx.x;
  }
  g = grp % Hkv;
  b = grp / Hkv;
  tile = T - 1 - r;  // heaviest (latest) rows first
}

// Scheduling-group masks (LLVM AMDGPU): MFMA, LDS read.
constexpr int kSgMfma = 0x008;
constexpr int kSgDsRead = 0x100;
constexpr int kLook = 3;  // PV: LDS operand reads issued ahead of their MFMA

// S^T (32 keys x 32 rows) = K Q^T of one LDS tile, as one assembly block
// (prefill_qk_asm.inc) that leaves S^T in VGPRs and ends with every LDS read
// complete and the MFMA result readable.  kb0/kb1 (kr0/kr1): LDS byte
// addresses of this lane's K (Krot) chunks for even/odd k-steps.
template <int D, bool TIED>
__device__ __forceinline__ f32x16 qk_tile(const bf16x8 (&qf)[D / 16], uint32_t kb0, uint32_t kb1,
                                          uint32_t kr0, uint32_t kr1) {
  f32x16 s;
  bf16x8 tmp[G4_QK_TEMPS];
  if constexpr (TIED) {
    asm volatile(G4_QK_ASM_512_TIED
                 : G4_QK_OUTS
                 : G4_QK_Q32, [kb0] "v"(kb0), [kb1] "v"(kb1), [kr0] "v"(kr0), [kr1] "v"(kr1)
                 : "memory");
  } else if constexpr (D == 512) {
    asm volatile(G4_QK_ASM_512 : G4_QK_OUTS : G4_QK_Q32, [kb0] "v"(kb0), [kb1] "v"(kb1) : "memory");
  } else {
    asm volatile(G4_QK_ASM_256 : G4_QK_OUTS : G4_QK_Q16, [kb0] "v"(kb0), [kb1] "v"(kb1) : "memory");
  }
  return s;
}

// REDO = false: main pass.  REDO = true: recompute the workgroups whose main
// pass flagged a reference overflow, after a first sweep that finds each
// row's true maximum.
template <int D, bool TIED, bool REDO>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs a) {
  typedef Cfg<D, TIED> C;
  __shared__ __attribute__((aligned(1024))) char smem[2 * C::STAGE];
  const uint32_t lds0 = lds_addr((G4_LDS void*)smem);  // LDS byte address of stage 0
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int hh = lane >> 5;   // lane half
  const int lr = lane & 31;   // row within the wave
  const int G = a.Hq / a.Hkv;
  const int ntiles = (int)(((int64_t)a.S * G + kBM - 1) / kBM);
  int b, g, tile;
  wg_map(ntiles, a.Hkv, b, g, tile);

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
  if (REDO) {
    if ((wg_flags[0] | wg_flags[1] | wg_flags[2] | wg_flags[3]) == 0) return;
  }

  // Prefetch the first tile, then load this lane's Q^T fragments (rows past S
  // read row S-1; their results are never stored).  K=V: the K-norm weight
  // is folded into the non-rotated dims, times qmul.
  load_tile<D, TIED>(a, lds0, kt_lo, b, g, wave, lane);

  bf16x8 qf[C::NT];
  {
    const uint16_t* qrow = a.q + b * a.qs[0] + (int64_t)min(tq, a.S - 1) * a.qs[1] + head * a.qs[2];
    const bool qscale = TIED && a.qmul != 1.f;
#pragma unroll
    for (int t = 0; t < C::NT; ++t) {
      const int d0 = 16 * t + 8 * hh;
      u32x4 raw = *(const u32x4*)(qrow + d0);
      if (TIED && !rot_step(t)) {
        const u32x4 w = *(const u32x4*)(a.w_k + d0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          raw[i] = pack_bf2(bf_lo(raw[i]) * bf_lo(w[i]) * a.qmul, bf_hi(raw[i]) * bf_hi(w[i]) * a.qmul);
      } else if (qscale) {
#pragma unroll
        for (int i = 0; i < 4; ++i) raw[i] = pack_bf2(bf_lo(raw[i]) * a.qmul, bf_hi(raw[i]) * a.qmul);
      }
      qf[t] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  // Per-lane LDS byte offsets within a stage.  QK^T operand (K row lr, dims
  // 16t + 8hh ..): chunk (2t + hh) ^ x keeps t>>1 in the high bits, so the
  // address is koff[t & 1] + 64 (t >> 1).
  const int k_x = kv_xor<D>(lr), kr_x = kr_xor(lr);
  const uint32_t koff0 = kv_row_off<D>(lr) + 16 * (hh ^ k_x);
  const uint32_t koff1 = kv_row_off<D>(lr) + 16 * ((2 + hh) ^ k_x);
  const uint32_t kroff0 = C::KR_OFF + kr_row_off(lr) + 16 * (hh ^ kr_x);
  const uint32_t kroff1 = C::KR_OFF + kr_row_off(lr) + 16 * ((2 + hh) ^ kr_x);
  // PV operand (transposing read): issuing lane feeds row 16m + 8u + r0 of
  // dim block c at 64c + toff[m][u].
  const int tG = lane >> 4, te = (lane >> 2) & 3, tqd = lane & 3;
  const int tr_row0 = 4 * (tG >> 1) + te;
  const int tr_chunk = 2 * (tG & 1) + (tqd >> 1);
  const int vbase = TIED ? 0 : C::KT_BYTES;
  int toff[2][2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int R = 16 * m + 8 * u + tr_row0;
      toff[m][u] = vbase + kv_row_off<D>(R) + (tqd & 1) * 8 + 16 * (tr_chunk ^ kv_xor<D>(R));
    }

  // Logit of key slot r in the log2 domain is s[r] * c[r]: c = the key's
  // inverse RMS times scale*log2(e) (K=V, from the tile) or scale*log2(e).
  const float cs = a.scale_log2;
  auto key_mul = [&](const G4_LDS char* cur, float (&c)[16]) {
    if (TIED) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const f32x4 v = *(const G4_LDS f32x4*)(cur + C::R_OFF + (8 * gq + 4 * hh) * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) c[4 * gq + i] = v[i];
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) c[r] = cs;
    }
  };
  // Does tile kt need element masks (some key not visible from some row)?
  auto edge_tile = [&](int kt) {
    const int key0 = kt * kBN;
    return !((key0 + kBN - 1 <= tq0) && (a.window == 0 || key0 >= tq1 - a.window + 1));
  };
  auto visible = [&](int kt, int r) {  // bitwise logic: no short-circuit branches
    const int d = tq - (kt * kBN + 8 * (r >> 2) + 4 * hh + (r & 3));
    return (d >= 0) & ((a.window == 0) | (d < a.window));
  };
  // Maximum logit of this lane's 16 slots of tile kt (-inf if none visible).
  auto tile_max = [&](const f32x16& s, const float (&c)[16], int kt) {
    const bool edge = edge_tile(kt);
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float x = s[r] * c[r];
      mx = fmaxf(mx, ((!edge) | visible(kt, r)) ? x : -INFINITY);
    }
    return mx;
  };
  auto lds_stage = [&](int kt) -> int { return ((kt - kt_lo) & 1) * C::STAGE; };

  // Softmax with a fixed per-row reference m_ref (log2 domain): the row's
  // maximum over its first tile with a visible key; P = exp2(x - m_ref) is
  // accumulated without ever rescaling O.  Every P is at most the row sum l,
  // so a row whose l stays <= 2^64 had no overflow risk; a wave with a larger
  // (or non-finite) l flags its workgroup, which the REDO launch recomputes
  // with m_ref = the true row maximum (every P <= 1 then).
  float m_ref = -INFINITY;
  if (REDO) {
    float m_run = -INFINITY;
    for (int kt = kt_lo; kt <= kt_hi; ++kt) {
      wait_vmem_all();
      __syncthreads();
      const int so = lds_stage(kt);
      const G4_LDS char* cur = (const G4_LDS char*)smem + so;
      if (kt < kt_hi) load_tile<D, TIED>(a, lds0 + (C::STAGE - so), kt + 1, b, g, wave, lane);
      const uint32_t base = lds0 + so;
      float c[16];
      key_mul(cur, c);
      const f32x16 s = qk_tile<D, TIED>(qf, base + koff0, base + koff1, base + kroff0, base + kroff1);
      m_run = fmaxf(m_run, tile_max(s, c, kt));
    }
    m_ref = max_xor32(m_run);
    __syncthreads();  // every wave is done with the last tile before stage 0 is reloaded
    load_tile<D, TIED>(a, lds0, kt_lo, b, g, wave, lane);
  }

  f32x16 oacc[C::NC];
#pragma unroll
  for (int c = 0; c < C::NC; ++c) oacc[c] = f32x16{};
  float l_part = 0.f;

  for (int kt = kt_lo; kt <= kt_hi; ++kt) {
    wait_vmem_all();  // this wave's copies of tile kt have landed
    __syncthreads();  // all of tile kt is in LDS; every wave is done with tile kt-1
    const int so = lds_stage(kt);
    const G4_LDS char* cur = (const G4_LDS char*)smem + so;
    if (kt < kt_hi) load_tile<D, TIED>(a, lds0 + (C::STAGE - so), kt + 1, b, g, wave, lane);

    // per-key factors first: their LDS reads complete under the K Q^T block
    const uint32_t base = lds0 + so;
    float c[16];
    key_mul(cur, c);
    const f32x16 s = qk_tile<D, TIED>(qf, base + koff0, base + koff1, base + kroff0, base + kroff1);
    __builtin_amdgcn_sched_barrier(0);  // keep the factor reads out of the PV read pipeline below
    if (!REDO && __builtin_amdgcn_ballot_w64(m_ref == -INFINITY)) {  // a row meets its first visible key
      const float rowmx = max_xor32(tile_max(s, c, kt));
      m_ref = m_ref == -INFINITY ? rowmx : m_ref;
    }
    const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = __builtin_fmaf(s[r], c[r], -m_use);
    if (edge_tile(kt)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = visible(kt, r) ? x[r] : -INFINITY;
    }
    bf16x8 pb[2];
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      u32x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r0 = 8 * mm + 2 * i;
        float p0 = __builtin_amdgcn_exp2f(x[r0]);
        float p1 = __builtin_amdgcn_exp2f(x[r0 + 1]);
        l_part += p0 + p1;
        if (TIED) { p0 *= c[r0]; p1 *= c[r0 + 1]; }
        w[i] = pack_bf2(p0, p1);
      }
      pb[mm] = __builtin_bit_cast(bf16x8, w);
    }

    // ---- O^T += V^T P^T, transposing reads kLook MFMAs ahead
    constexpr int NPV = 2 * C::NC;  // (mm, c) pairs
    auto vread = [&](int i) -> bf16x8 {
      const int mm = i / C::NC, c = i % C::NC;
      const i16x4 lo = lds_read_tr16(cur + toff[mm][0] + 64 * c);
      const i16x4 hi = lds_read_tr16(cur + toff[mm][1] + 64 * c);
      return cat_tr(lo, hi);
    };
    bf16x8 va[kLook + 1];
#pragma unroll
    for (int i = 0; i < kLook; ++i) va[i] = vread(i);
    __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2 * kLook, 0);
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      if (i + kLook < NPV) va[(i + kLook) % (kLook + 1)] = vread(i + kLook);
      const int mm = i / C::NC, c = i % C::NC;
      oacc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i % (kLook + 1)], pb[mm], oacc[c], 0, 0, 0);
      __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
      if (i + kLook < NPV) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2, 0);
    }
  }

  // ---- epilogue: flag, normalise, round once to bf16, store
  const float l_tot = sum_xor32(l_part);
  if (!REDO) {
    const bool over = valid && !(l_tot <= 0x1p64f);
    if (lane == 0) wg_flags[wave] = __builtin_amdgcn_ballot_w64(over) != 0;
  }
  if (!valid) return;
  // K=V: P carried the factor c = r * scale*log2(e) / qmul; omul undoes it.
  const float inv = l_tot > 0.f ? (TIED ? a.omul : 1.f) / l_tot : 0.f;
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
      hipLaunchKernelGGL((redo ? prefill_kernel<512, true, true> : prefill_kernel<512, true, false>),
                         grid, dim3(256), 0, st, a);
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
