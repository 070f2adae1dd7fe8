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
// Per wave: 16-row tiles streamed through a ring of NS stages in the wave's
// own LDS region with direct global->LDS loads, NS-1 tiles in flight (no
// workgroup barrier in the loop; the wait for the oldest tile is an exact
// vector-memory count).
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
  // 4 waves x 2 stages (K=V) measured faster than 2 x 4 or 3 x 3 at the same
  // LDS size: more independent waves keep more loads in flight.
  static constexpr int WAVES = SAME_KV ? 4 : 2;
  static constexpr int NS = 2;                              // ring stages per wave
  static constexpr int LPT = (SAME_KV ? 1 : 2) * (D == 512 ? 16 : 8);  // loads per tile
  static constexpr int NT = D / 32;  // QK^T k-steps
  static constexpr int NC = D / 16;  // PV dim blocks
};


// Direct global->LDS copies (as g2lds16 / g2lds4) with the non-temporal
// policy, for cache rows, which a decode reads exactly once: they then do
// not displace reused lines from L2 and the infinity cache (31B K=V batch,
// 11.7 GB: 6.1 -> 6.8 TB/s).
__device__ __forceinline__ void g2lds16_nt(const void* gptr, G4_LDS void* lds_base) {
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off nt\n\ts_mov_b32 m0, %0"
      : "=&s"(keep)
      : "v"(gptr), "s"(lds_addr(lds_base))
      : "memory");
}
__device__ __forceinline__ void g2lds4_nt(const void* gptr, G4_LDS void* lds_base) {
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dword %1, off nt\n\ts_mov_b32 m0, %0"
      : "=&s"(keep)
      : "v"(gptr), "s"(lds_addr(lds_base))
      : "memory");
}

template <int D>
__device__ __forceinline__ void load_rows(const uint16_t* base, int row0, int nrows, char* tile, int lane) {
  // rows row0 .. row0+15 of one (b, g) cache slice; rows >= nrows are
  // clamped to the last valid row (they are masked out of the softmax).
  // Cache rows are read once per decode: non-temporal copies.
  if (D == 512) {
#pragma unroll
    for (int R = 0; R < kRows; ++R) {
      int row = row0 + R;
      row = row < nrows ? row : nrows - 1;
      const int ch = lane ^ d_xor(R);
      g2lds16_nt(base + (int64_t)row * D + ch * 8, (G4_LDS void*)(tile + d_row_off<D>(R)));
    }
  } else {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int R = s + 8 * (lane >> 5);
      int row = row0 + R;
      row = row < nrows ? row : nrows - 1;
      const int ch = (lane & 31) ^ d_xor(R);
      g2lds16_nt(base + (int64_t)row * D + ch * 8, (G4_LDS void*)(tile + s * kSegD));
    }
  }
}

// Softmax per chunk with a fixed reference, as in the prefill kernel: each
// wave's reference for a head is that head's maximum over the wave's first
// tile; P = exp2(s - m_ref) is accumulated without rescaling O.  A chunk whose
// true maximum ends more than kHeadroom above a reference is flagged and
// recomputed by the REDO launch with the true maxima (every P <= 1 then).
constexpr float kHeadroom = 64.f;

// A chunk's normalised O and log-sum-exp.  With one chunk per (sequence,
// KV head) they are the result itself (the combine of a single partial has
// weight exp(0) = 1 and returns the same bits), so the split kernel writes
// out and lse directly and the combine launch is skipped.
template <int D>
__device__ __forceinline__ void write_chunk(const DecodeArgs& a, int64_t ph, int split, int d, float o, float lse) {
  if (a.nsplit == 1) {
    a.out[ph * D + d] = (uint16_t)f2bf(o);
    if (d == 0 && a.lse) a.lse[ph] = lse;
  } else {
    a.o_part[(ph * a.nsplit + split) * D + d] = o;
    if (d == 0) a.lse_part[ph * a.nsplit + split] = lse;
  }
}

// A sequence with no rows (kv_len clamped to 0) and one chunk: nothing else
// writes its heads, so the split kernel writes what the combine would (zeros,
// lse = -inf).
template <int D>
__device__ void write_empty(const DecodeArgs& a, int b, int g, int G, int nthreads) {
  for (int idx = threadIdx.x; idx < G * D; idx += nthreads) {
    const int64_t ph = (int64_t)b * a.Hq + g * G + idx / D;
    a.out[ph * D + idx % D] = 0;
    if (idx % D == 0 && a.lse) a.lse[ph] = -INFINITY;
  }
}

template <int D, bool SAME_KV, bool REDO>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  typedef DCfg<D, SAME_KV> C;
  __shared__ __attribute__((aligned(1024))) char smem[C::WAVES * C::NS * C::STAGE];
  __shared__ float s_m[C::WAVES][16], s_l[C::WAVES][16];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int G = a.Hq / a.Hkv;
  RedoCursor redo{(int64_t)a.nsplit * a.Hkv * a.B};
  for (;;) {
  int split, g, b;
  if (REDO) {
    // the next chunk whose main pass flagged a reference overflow (flag of
    // chunk L = split + nsplit (g + Hkv b) at dflags[L])
    const int64_t L = redo.next([&](int64_t c) { return a.dflags[c] != 0; });
    if (L < 0) return;
    split = (int)(L % a.nsplit);
    g = (int)((L / a.nsplit) % a.Hkv);
    b = (int)(L / ((int64_t)a.nsplit * a.Hkv));
  } else {
    split = blockIdx.x;
    g = blockIdx.y;
    b = blockIdx.z;
  }
  const int n = min(max(a.kv_len[b], 0), a.max_len);
  const int r0 = split * a.chunk;
  if (r0 >= n) {  // beyond this sequence: the combine never reads it
    if (!REDO && a.nsplit == 1) write_empty<D>(a, b, g, G, C::WAVES * 64);
    if (!REDO) return;
    continue;
  }
  const int r1 = min(r0 + a.chunk, n);
  const int ntile = (r1 - r0 + kRows - 1) / kRows;
  const int64_t blk = ((int64_t)b * a.Hkv + g) * a.nsplit + split;

  const int64_t slice = ((int64_t)b * a.Hkv + g) * a.cap * D;
  const uint16_t* kbase = a.kc + slice;
  const uint16_t* vbase = a.vc + slice;
  char* mybuf = smem + wave * C::NS * C::STAGE;

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
  float m_ref = -INFINITY, m_true = -INFINITY, l_part = 0.f;
  const int64_t hrow = ((int64_t)b * a.Hq + g * G + (hvalid ? hcol : 0)) * a.nsplit + split;
  if (REDO) m_ref = a.dmax[hrow];

  const int k_rowoff = d_row_off<D>(lane & 15), k_x = d_xor(lane & 15);
  // transposing read: issuing lane feeds row 4*(lane>>4) + ((lane>>2)&3), dims 16cb + 4*(lane&3)
  const int tR = 4 * (lane >> 4) + ((lane >> 2) & 3);
  const int tq = lane & 3;
  const int tr_off = d_row_off<D>(tR) + (tq & 1) * 8;
  const int tr_j = (tq >> 1) ^ d_xor(tR);

  // tiles of this wave: tl = wave + WAVES * it
  const int nmine = ntile > wave ? (ntile - wave + C::WAVES - 1) / C::WAVES : 0;
  auto issue = [&](int it) {
    const int tl = wave + C::WAVES * it;
    char* st = mybuf + (it % C::NS) * C::STAGE;
    load_rows<D>(kbase, r0 + tl * kRows, r1, st, lane);
    if (!SAME_KV) load_rows<D>(vbase, r0 + tl * kRows, r1, st + C::TILE, lane);
  };
#pragma unroll
  for (int it = 0; it < C::NS - 1; ++it)
    if (it < nmine) issue(it);
  for (int it = 0; it < nmine; ++it) {
    if constexpr (C::NS == 1) issue(it);  // no ring: other waves hide the latency
    // wait for tile it; tiles it+1 .. it+NS-2 (if any) may stay in flight
    const int newer = min(nmine - 1 - it, C::NS - 2);
    if constexpr (C::NS >= 4) {
      if (newer >= 2) wait_vmem<2 * C::LPT>();
      else if (newer == 1) wait_vmem<C::LPT>();
      else wait_vmem<0>();
    } else if constexpr (C::NS == 3) {
      if (newer >= 1) wait_vmem<C::LPT>();
      else wait_vmem<0>();
    } else {
      wait_vmem<0>();
    }
    if (C::NS > 1 && it + C::NS - 1 < nmine) issue(it + C::NS - 1);  // into the stage tile it-1 used
    const int tl = wave + C::WAVES * it;
    char* cur = mybuf + (it % C::NS) * C::STAGE;

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
    m_true = fmaxf(m_true, mx);
    if (!REDO && it == 0) {  // the wave's first tile fixes its reference
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      m_ref = fmaxf(mx, __shfl_xor(mx, 32, 64));
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) { p[i] = __builtin_amdgcn_exp2f(s[i] - m_ref); l_part += p[i]; }
    const u32x2 pw = {pack_bf2(p[0], p[1]), pack_bf2(p[2], p[3])};
    const i16x4_t pb = __builtin_bit_cast(i16x4_t, pw);
    const char* vt = SAME_KV ? cur : cur + C::TILE;
#pragma unroll
    for (int c = 0; c < C::NC; ++c) {
      const i16x4 va = lds_read_tr16((const G4_LDS char*)(vt + tr_off + (2 * c + tr_j) * 16));
      oacc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, oacc[c], 0, 0, 0);
    }
  }

  // ---- merge the waves' partial states (each relative to its own reference)
  float l_tot = l_part + __shfl_xor(l_part, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  float mt = fmaxf(m_true, __shfl_xor(m_true, 16, 64));
  mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
  __shared__ float s_t[C::WAVES][16];
  __shared__ int s_over[C::WAVES];
  if (lane < 16) { s_m[wave][lane] = m_ref; s_l[wave][lane] = l_tot; s_t[wave][lane] = mt; }
  if (lane == 0) s_over[wave] = __builtin_amdgcn_ballot_w64(hvalid && mt > m_ref + kHeadroom) != 0;
  __syncthreads();  // all waves are done with their tiles; reuse LDS for O
  float* so = (float*)smem;  // [WAVES][16 heads][D]
  if (hvalid) {
#pragma unroll
    for (int c = 0; c < C::NC; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) so[(wave * 16 + hcol) * D + 16 * c + 4 * kq + i] = oacc[c][i];
  }
  if (!REDO && threadIdx.x == 0) {
    int over = 0;
#pragma unroll
    for (int w = 0; w < C::WAVES; ++w) over |= s_over[w];
    a.dflags[blk] = over;
  }
  if (!REDO && threadIdx.x < G) {
    float t = -INFINITY;
#pragma unroll
    for (int w = 0; w < C::WAVES; ++w) t = fmaxf(t, s_t[w][threadIdx.x]);
    a.dmax[((int64_t)b * a.Hq + g * G + threadIdx.x) * a.nsplit + split] = t;
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
    write_chunk<D>(a, ph, split, d, O / L, (M + __log2f(L)) * kLn2);
  }
  if (!REDO) return;
  __syncthreads();  // every wave is done with the LDS before the next chunk reuses it
  }
}

// K=V decode over the raw tied projection (the global layer's own cache
// format): the cache holds X, the inverse RMS r of each row and the rotated
// part Krot = RoPE(X w_k) of its key on dims 0..63, 256..319.  With q's
// K-norm weight folded into its other dims, as in the K=V prefill,
//   q.k_p = r_p (sum_{d not in R} (q_d w_d) X_pd + sum_{d in R} q_d Krot_pd),
//   sum_p P_p v_p = sum_p (P_p r_p) X_p,
// so one LDS tile of X (plus 16 Krot rows and 16 factors) feeds both MFMAs.
// 1284 bytes per cached row and KV head, read once.  Three waves x two
// stages (the Krot slice does not fit a fourth wave's ring).
constexpr int kWavesT = 3;
constexpr int kTileX = kRows * kSegD;           // 16 X rows
constexpr int kKrOff = kTileX;                  // 16 Krot rows of 256 B, chunk c of row r at slot c ^ r
constexpr int kROff = kKrOff + kRows * 256;     // 64 factors (16 used)
constexpr int kStageT = kROff + 256;

__device__ __forceinline__ constexpr bool rot_step32(int t) { return t < 2 || (t >= 8 && t < 10); }

template <bool REDO>
__global__ __launch_bounds__(kWavesT * 64) void decode_tied_kernel(DecodeArgs a) {
  constexpr int D = 512, NT = D / 32, NC = D / 16, NS = 2;
  __shared__ __attribute__((aligned(1024))) char smem[kWavesT * NS * kStageT];
  __shared__ float s_m[kWavesT][16], s_l[kWavesT][16], s_t[kWavesT][16];
  __shared__ int s_over[kWavesT];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int G = a.Hq / a.Hkv;
  RedoCursor redo{(int64_t)a.nsplit * a.Hkv * a.B};
  for (;;) {
  int split, g, b;
  if (REDO) {
    // the next chunk whose main pass flagged a reference overflow (flag of
    // chunk L = split + nsplit (g + Hkv b) at dflags[L])
    const int64_t L = redo.next([&](int64_t c) { return a.dflags[c] != 0; });
    if (L < 0) return;
    split = (int)(L % a.nsplit);
    g = (int)((L / a.nsplit) % a.Hkv);
    b = (int)(L / ((int64_t)a.nsplit * a.Hkv));
  } else {
    split = blockIdx.x;
    g = blockIdx.y;
    b = blockIdx.z;
  }
  const int n = min(max(a.kv_len[b], 0), a.max_len);
  const int r0 = split * a.chunk;
  if (r0 >= n) {  // beyond this sequence: the combine never reads it
    if (!REDO && a.nsplit == 1) write_empty<D>(a, b, g, G, kWavesT * 64);
    if (!REDO) return;
    continue;
  }
  const int r1 = min(r0 + a.chunk, n);
  const int ntile = (r1 - r0 + kRows - 1) / kRows;
  const int64_t blk = ((int64_t)b * a.Hkv + g) * a.nsplit + split;

  const int64_t srow = ((int64_t)b * a.Hkv + g) * a.cap;   // first cache row of this (b, g)
  const uint16_t* xbase = a.kc + srow * D;
  const uint16_t* krbase = a.krc + srow * 128;
  const float* rbase = a.rc + srow;
  char* mybuf = smem + wave * NS * kStageT;

  // Q^T (B operand of the 16x16x32 MFMA): lane -> head (lane & 15), dims
  // 32t + 8(lane >> 4) ..; the non-rotated dims carry the K-norm weight.
  const int hcol = lane & 15, kq = lane >> 4;
  const bool hvalid = hcol < G;
  bf16x8 qf[NT];
  {
    const uint16_t* qrow = a.q + ((int64_t)b * a.Hq + g * G + (hvalid ? hcol : 0)) * D;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int d0 = 32 * t + 8 * kq;
      u32x4 raw = hvalid ? *(const u32x4*)(qrow + d0) : u32x4{0, 0, 0, 0};
      if (!rot_step32(t)) {
        const u32x4 w = *(const u32x4*)(a.w_k + d0);
#pragma unroll
        for (int i = 0; i < 4; ++i) raw[i] = pack_bf2(bf_lo(raw[i]) * bf_lo(w[i]), bf_hi(raw[i]) * bf_hi(w[i]));
      }
      qf[t] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  f32x4 oacc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) oacc[c] = f32x4{};
  float m_ref = -INFINITY, m_true = -INFINITY, l_part = 0.f;
  const int64_t hrow = ((int64_t)b * a.Hq + g * G + (hvalid ? hcol : 0)) * a.nsplit + split;
  if (REDO) m_ref = a.dmax[hrow];

  const int krow = lane & 15;
  const int k_rowoff = d_row_off<D>(krow), k_x = d_xor(krow);
  const int tR = 4 * (lane >> 4) + ((lane >> 2) & 3);
  const int tq = lane & 3;
  const int tr_off = d_row_off<D>(tR) + (tq & 1) * 8;
  const int tr_j = (tq >> 1) ^ d_xor(tR);

  // copy of tile tl: 16 X rows, 16 Krot rows (4 loads of 4 rows, each lane's
  // chunk XOR-swizzled by its row) and the rows' factors (all 64 lanes; 16 used)
  auto issue = [&](int it) {
    const int tl = wave + kWavesT * it;
    char* st = mybuf + (it % NS) * kStageT;
    const int row0 = r0 + tl * kRows;
    load_rows<D>(xbase, row0, r1, st, lane);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int R = 4 * j + (lane >> 4);
      const int row = min(row0 + R, r1 - 1);
      const int c = (lane & 15) ^ R;
      g2lds16_nt(krbase + (int64_t)row * 128 + c * 8, (G4_LDS void*)(st + kKrOff + j * 1024));
    }
    g2lds4_nt(rbase + min(row0 + lane, r1 - 1), (G4_LDS void*)(st + kROff));
  };
  const int nmine = ntile > wave ? (ntile - wave + kWavesT - 1) / kWavesT : 0;
  if (nmine > 0) issue(0);
  for (int it = 0; it < nmine; ++it) {
    wait_vmem<0>();
    if (it + 1 < nmine) issue(it + 1);  // into the stage tile it-1 used
    const int tl = wave + kWavesT * it;
    char* cur = mybuf + (it % NS) * kStageT;

    f32x4 sacc = f32x4{};
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      bf16x8 ka;
      if (rot_step32(t)) {
        const int u = t < 2 ? t : t - 6;
        ka = lds_read_b128((const G4_LDS char*)(cur + kKrOff + krow * 256 + (((4 * u + kq) ^ krow) * 16)));
      } else {
        const int ch = (4 * t + kq) ^ k_x;
        ka = lds_read_b128((const G4_LDS char*)(cur + k_rowoff + ch * 16));
      }
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[t], sacc, 0, 0, 0);
    }
    // lane holds head hcol, keys 4*kq + i of this tile; c = r * scale*log2(e)
    const f32x4 rv = *(const G4_LDS f32x4*)(cur + kROff + 16 * kq);
    const int key0 = r0 + tl * kRows + 4 * kq;
    float s[4], c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[i] = rv[i] * a.scale_log2;
      s[i] = (key0 + i < r1) ? sacc[i] * c[i] : -INFINITY;
    }
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    m_true = fmaxf(m_true, mx);
    if (!REDO && it == 0) {  // the wave's first tile fixes its reference
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      m_ref = fmaxf(mx, __shfl_xor(mx, 32, 64));
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = __builtin_amdgcn_exp2f(s[i] - m_ref);
      l_part += e;
      p[i] = e * rv[i];  // value row p is r_p X_p
    }
    const u32x2 pw = {pack_bf2(p[0], p[1]), pack_bf2(p[2], p[3])};
    const i16x4_t pb = __builtin_bit_cast(i16x4_t, pw);
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) {
      const i16x4 va = lds_read_tr16((const G4_LDS char*)(cur + tr_off + (2 * cb + tr_j) * 16));
      oacc[cb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, oacc[cb], 0, 0, 0);
    }
  }

  // ---- merge the waves' partial states (each relative to its own reference)
  float l_tot = l_part + __shfl_xor(l_part, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  float mt = fmaxf(m_true, __shfl_xor(m_true, 16, 64));
  mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
  if (lane < 16) { s_m[wave][lane] = m_ref; s_l[wave][lane] = l_tot; s_t[wave][lane] = mt; }
  if (lane == 0) s_over[wave] = __builtin_amdgcn_ballot_w64(hvalid && mt > m_ref + kHeadroom) != 0;
  __syncthreads();  // all waves are done with their tiles; reuse LDS for O
  float* so = (float*)smem;  // [kWavesT][16 heads][D]
  if (hvalid) {
#pragma unroll
    for (int cb = 0; cb < NC; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) so[(wave * 16 + hcol) * D + 16 * cb + 4 * kq + i] = oacc[cb][i];
  }
  if (!REDO && threadIdx.x == 0) {
    int over = 0;
#pragma unroll
    for (int w = 0; w < kWavesT; ++w) over |= s_over[w];
    a.dflags[blk] = over;
  }
  if (!REDO && threadIdx.x < G) {
    float t = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWavesT; ++w) t = fmaxf(t, s_t[w][threadIdx.x]);
    a.dmax[((int64_t)b * a.Hq + g * G + threadIdx.x) * a.nsplit + split] = t;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += kWavesT * 64) {
    const int hh = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWavesT; ++w) M = fmaxf(M, s_m[w][hh]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kWavesT; ++w) {
      const float wt = s_m[w][hh] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s_m[w][hh] - M);
      L += wt * s_l[w][hh];
      O += wt * so[(w * 16 + hh) * D + d];
    }
    const int64_t ph = (int64_t)b * a.Hq + g * G + hh;
    write_chunk<D>(a, ph, split, d, O / L, (M + __log2f(L)) * kLn2);
  }
  if (!REDO) return;
  __syncthreads();  // every wave is done with the LDS before the next chunk reuses it
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

// Recompute launch: persistent workgroups that test every chunk's flag.
dim3 redo_grid(const dim3& gr) {
  const int64_t n = (int64_t)gr.x * gr.y * gr.z;
  return dim3((unsigned)(n < 1024 ? n : 1024));
}

template <int D, bool SAME>
hipError_t launch_d(const DecodeArgs& a, hipStream_t st) {
  typedef DCfg<D, SAME> C;
  const dim3 grid(a.nsplit, a.Hkv, a.B);
  hipLaunchKernelGGL((decode_split_kernel<D, SAME, false>), grid, dim3(C::WAVES * 64), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_split_kernel<D, SAME, true>), redo_grid(grid), dim3(C::WAVES * 64), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;  // one chunk: the split kernel wrote the result
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(a.Hq, a.B), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_tied(const DecodeArgs& a, hipStream_t st) {
  const dim3 grid(a.nsplit, a.Hkv, a.B);
  hipLaunchKernelGGL(decode_tied_kernel<false>, grid, dim3(kWavesT * 64), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_tied_kernel<true>, redo_grid(grid), dim3(kWavesT * 64), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;  // one chunk: the split kernel wrote the result
  hipLaunchKernelGGL((decode_combine_kernel<512>), dim3(a.Hq, a.B), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  const bool same = a.kc == a.vc;
  if (a.D == 512) return same ? launch_d<512, true>(a, st) : launch_d<512, false>(a, st);
  return same ? launch_d<256, true>(a, st) : launch_d<256, false>(a, st);
}

}  // namespace g4attn
