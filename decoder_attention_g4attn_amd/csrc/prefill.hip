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
//     so the softmax is per lane plus one partner lane (l ^ 32).  Q^T stays
//     in registers (D/4 VGPRs), O^T accumulates in D/2 registers.
//   * K/V tiles of 32 keys stream through an LDS ring (three stages where
//     they fit) with direct global->LDS loads; tiles wholly outside the
//     causal/window band are never visited and only edge tiles are masked
//     element by element.
//   * prefill_kernel software-pipelines one wave per SIMD (D = 512);
//     prefill_d256_kernel runs two waves per SIMD (D = 256).  Both also take
//     chunked rows over caches and bidirectional spans (the EXT variant).
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
#include <type_traits>

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
  static constexpr int NST = 3 * STAGE <= 160 * 1024 ? 3 : 2;  // LDS stages
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

// Global->LDS copy of key tile kt, one load instruction ("piece") at a time
// so that the copies can be spread over the MFMAs of a tile step instead of
// stalling every wave in one burst.  The tile's row bases are wave-uniform
// (scalar registers) plus an unsigned 32-bit per-lane byte offset (the
// scalar-base form).  Rows past S re-read row S-1 (they are masked).
// Pieces per wave: D = 512: 8 rows of K (or X), then 8 of V; D = 256: 4
// instructions of two rows for K, then 4 for V; K=V: then 2 of the Krot
// slice and (wave 0) the 32 key factors.
template <int D, bool TIED>
struct TilePieces {
  static constexpr int KV = (D == 512 ? 8 : 4) * (TIED ? 1 : 2);
  static constexpr int N = KV + (TIED ? 3 : 0);
};

// Per-tile source addresses of the copy (wave-uniform, formed once per tile).
struct TileSrc {
  const char* k;      // K (or X) row key0 of this (b, g)
  const char* v;      // V row key0
  const char* krot;   // K=V: Krot row key0
  const float* r;     // K=V: key factors from key0
  uint32_t last_off;  // byte offset from row key0 of the row that stands in for rows past key_end-1
  int last;           // its index within the tile: min(key_end-1-key0, kBN-1)
};

// key_end: one past the last valid key of sequence b (S, or the chunk's end
// when the keys come from a cache).
template <int D, bool TIED>
__device__ __forceinline__ TileSrc tile_src(const PrefillArgs& a, int kt, int b, int g, int key_end) {
  const int key0 = kt * kBN;
  TileSrc t;
  const int64_t e = b * a.ks[0] + g * a.ks[2] + (int64_t)key0 * a.ks[1];
  t.k = (const char*)(a.k + e);
  t.v = TIED ? nullptr : (const char*)(a.v + e);
  const int64_t row0 = ((int64_t)b * a.Hkv + g) * a.kv_rows + key0;
  t.krot = TIED ? (const char*)(a.krot + row0 * 128) : nullptr;
  t.r = TIED ? a.r + row0 : nullptr;
  // Only rows 0..kBN-1 of the tile are copied, so the clamp row never needs
  // to exceed kBN-1; clamping first keeps last * stride within 32 bits.
  t.last = min(key_end - 1 - key0, kBN - 1);
  t.last_off = (uint32_t)t.last * (uint32_t)(a.ks[1] * 2);
  return t;
}

// Row offsets grow with the row, so clamping a row to S-1 is a min() of
// byte offsets; the lane's own 16-byte chunk rides in the same 32-bit
// offset (the key stride times 32 fits in 31 bits, checked on the host).
template <int D, bool TIED>
__device__ __forceinline__ void load_piece(const PrefillArgs& a, const TileSrc& ts, uint32_t stage, int wave,
                                           int lane, int piece) {
  typedef Cfg<D, TIED> C;
  constexpr int PER = D == 512 ? 8 : 4;  // pieces per K or V tile
  const uint32_t rs = (uint32_t)(a.ks[1] * 2);  // key stride in bytes
  if (piece < TilePieces<D, TIED>::KV) {
    const int which = piece / PER, i = piece % PER;
    const char* src = which == 0 ? ts.k : ts.v;
    const uint32_t tile = stage + which * C::KT_BYTES;
    if (D == 512) {
      const int R = wave * 8 + i;
      const uint32_t row = min((uint32_t)R * rs, ts.last_off);
      const uint32_t off = row + (uint32_t)(lane ^ kv_xor<D>(R)) * 16u;
      g2lds16s(src, off, tile + kv_row_off<D>(R));
    } else {
      // lanes 0..31 copy row s, lanes 32..63 row s + 16
      const int s = wave * 4 + i;
      const uint32_t r0 = min((uint32_t)s * rs, ts.last_off);
      const uint32_t r1 = min((uint32_t)(s + 16) * rs, ts.last_off);
      const uint32_t off = ((lane >> 5) ? r1 : r0) + (uint32_t)((lane & 31) ^ kv_xor<D>(s)) * 16u;
      g2lds16s(src, off, tile + s * kSeg);
    }
  } else if (TIED) {
    const int i = piece - TilePieces<D, TIED>::KV;
    if (i < 2) {
      const int s = wave * 2 + i;
      // lanes 16q .. 16q+15 copy Krot row s + 8q
      const int R = s + 8 * (lane >> 4);
      const uint32_t off = (uint32_t)min(R, ts.last) * 256u + (uint32_t)((lane & 15) ^ kr_xor(R)) * 16u;
      g2lds16s(ts.krot, off, stage + C::KR_OFF + s * kSeg);
    } else if (wave == 0) {
      g2lds4s(ts.r, (uint32_t)min(lane & 31, ts.last) * 4u, stage + C::R_OFF);
    }
  }
}

template <int D, bool TIED>
__device__ __forceinline__ void load_tile(const PrefillArgs& a, uint32_t stage, int kt, int b, int g,
                                          int key_end, int wave, int lane) {
  const TileSrc ts = tile_src<D, TIED>(a, kt, b, g, key_end);
#pragma unroll
  for (int p = 0; p < TilePieces<D, TIED>::N; ++p) load_piece<D, TIED>(a, ts, stage, wave, lane, p);
}

// Workgroup -> (batch b, KV group g, row tile) for the 8 XCDs of the chip.
// The dispatcher hands linear workgroup ids to the XCDs round-robin, and
// each XCD has its own L2.  With NG = B*Hkv groups of T tiles:
//   NG % 8 == 0          : each XCD takes NG/8 whole groups;
//   8 % NG == 0, T % (8/NG) == 0 : each group is spread over 8/NG XCDs, XCD
//                          c taking every (8/NG)-th tile in weight order;
//   otherwise            : plain order.
// so an XCD's L2 serves one group's keys instead of every group's, work
// per XCD stays balanced, and each XCD runs its heaviest (latest) tiles first
// (the longest-processing-time order for a causal layer's tail).  With
// LIGHT_FIRST the order is reversed: on a sliding layer every tile past the
// first window costs the same, and opening with the partial-window tiles at
// the start of each sequence makes the first round's workgroups end at
// different times, so the CUs fall out of step and later rounds' start-up
// loads (Q, first K/V tiles) no longer reach HBM all at once (31B sliding
// layer: 3-4% faster).
__device__ __forceinline__ void wg_map(int T, int Hkv, int& b, int& g, int& tile, bool light_first = false) {
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
  tile = light_first ? r : T - 1 - r;
}

constexpr int kLook = 3;  // LDS operand reads issued ahead of their MFMA

// O^T block += V^T P^T on the AGPR accumulator.  Written as assembly so that
// the compiler never allocates O (all AGPRs at D = 512) on the VGPR side;
// being volatile, these also keep the LDS reads around them in source order.
// `FIRST`: the first use of a P^T operand written by VALU just before (an
// MFMA needs 2 wait states after a VALU write of its source).
template <bool FIRST>
__device__ __forceinline__ void mfma_acc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  if (FIRST)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Keeps a value computed before this point (no code is emitted).
__device__ __forceinline__ void pin(float& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void pin(uint32_t& v) { asm volatile("" : "+v"(v)); }

// REDO = false: main pass.  REDO = true: recompute the workgroups whose main
// pass flagged a reference overflow, after a first sweep that finds each
// row's true maximum.
//
// Software pipeline (per wave, one wave per SIMD): iteration kt computes
// S(kt+1) = K(kt+1) Q^T with its MFMAs interleaved with the softmax VALU
// work of S(kt), then O += V(kt)^T P(kt)^T.  Tiles kt and kt+1 are resident
// in LDS while tile kt+2 is in flight (NST = 3 stages); configurations
// whose three stages do not fit (D = 512 without K=V) use two stages whose
// K and V halves are refilled half a step apart: K(kt+2) and V(kt+1) are
// copied during iteration kt.
// EXT: the extended masks and row layouts: rows that continue sequences
// over caches (pos0 / qlen) and bidirectional spans (span_lo / span_hi);
// each is off when its pointer is NULL.
template <int D, bool TIED, bool REDO, bool EXT>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs a) {
  typedef Cfg<D, TIED> C;
  constexpr int NST = C::NST;
  __shared__ __attribute__((aligned(1024))) char smem[NST * C::STAGE];
  const uint32_t lds0 = lds_addr((G4_LDS void*)smem);  // LDS byte address of stage 0
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int hh = lane >> 5;   // lane half
  const int lr = lane & 31;   // row within the wave
  const int G = a.Hq / a.Hkv;
  const int ntiles = (int)(((int64_t)a.S * G + kBM - 1) / kBM);
  // Main pass: one workgroup per row tile.  Recompute pass: a small grid of
  // persistent workgroups tests every row tile's flags in parallel and redoes
  // the flagged ones (most launches find none).
  RedoCursor redo{(int64_t)ntiles * a.Hkv * a.B};
  for (;;) {
    int b, g, tile;
    if (REDO) {
      // the next row tile whose main pass flagged a reference overflow (the
      // flags of tile L = tile + ntiles (g + Hkv b) sit at flags[L * waves])
      const int64_t L = redo.next([&](int64_t c) {
        const u32x4 f = *(const u32x4*)(a.flags + c * kWaves);
        return (f[0] | f[1] | f[2] | f[3]) != 0u;
      });
      if (L < 0) return;
      tile = (int)(L % ntiles);
      g = (int)((L / ntiles) % a.Hkv);
      b = (int)(L / ((int64_t)ntiles * a.Hkv));
    } else {
      wg_map(ntiles, a.Hkv, b, g, tile);
    }

    // Rows t < n of this sequence are positions P + t (P = 0, n = S unless
    // the keys come from a cache: chunked prefill, padded batches).
    // Device-side values are clamped: a sequence with pos0 < 0 has no rows,
    // and rows past the host's bound max_pos are not computed, so no key
    // past the cache is ever read.
    int P = 0, n = a.S;
    if (EXT && a.pos0) {
      P = a.pos0[b];
      n = a.qlen ? min(a.qlen[b], a.S) : a.S;
      n = P < 0 ? 0 : max(0, min(n, a.max_pos + 1 - P));
    }
    const int key_end = P + n;  // keys [0, key_end) exist
    const int64_t F0 = (int64_t)tile * kBM;
    const int64_t Flast = min(F0 + kBM - 1, (int64_t)a.S * G - 1);
    // first and last query positions of the workgroup's valid rows
    const int tr0 = (int)(F0 / G), tr1 = EXT ? min((int)(Flast / G), n - 1) : (int)(Flast / G);
    const int tq0 = P + tr0, tq1 = P + tr1;
    const int64_t F = F0 + wave * 32 + lr;
    const int tq = (int)(F / G);
    const int head = g * G + (int)(F % G);
    const bool valid = tq < n;
    const int pos = P + tq;  // this lane's query position

    // Bidirectional spans: row t also sees keys [span_lo, span_hi] (its own
    // image span).  The bounds grow with t, so the workgroup's first row has
    // the lowest and its last valid row the highest.
    const bool spans = EXT && a.span_lo != nullptr;
    const int64_t srow = (int64_t)b * a.S;
    const int kt_lo = max(0, min(a.window ? tq0 - a.window + 1 : 0, spans ? a.span_lo[srow + tr0] : tq0)) / kBN;
    const int kt_hi = min(max(tq1, spans ? a.span_hi[srow + tr1] : tq1), key_end - 1) / kBN;
    int* wg_flags = a.flags + (((int64_t)b * a.Hkv + g) * ntiles + tile) * kWaves;
    if (EXT && tq0 > tq1) {  // only padding rows: nothing to compute (uniform)
      if (!REDO && threadIdx.x < kWaves) wg_flags[threadIdx.x] = 0;
      if (!REDO) return;
      continue;
    }

    // Prefetch the first two tiles, then load this lane's Q^T fragments (rows
    // past S read row S-1; their results are never stored).  K=V: the K-norm
    // weight is folded into the non-rotated dims, times qmul.
    load_tile<D, TIED>(a, lds0, kt_lo, b, g, key_end, wave, lane);
    if (kt_lo < kt_hi) load_tile<D, TIED>(a, lds0 + C::STAGE, kt_lo + 1, b, g, key_end, wave, lane);

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

    auto lds_ptr = [&](int so) { return (const G4_LDS char*)smem + so; };
    // K fragment of k-step t of the tile in stage `so` (K=V: rotated k-steps
    // read the Krot slice, chunk 2u + hh with u = t (t < 4) or t - 12).
    auto kread = [&](int so, int t) -> bf16x8 {
      if (TIED && rot_step(t)) {
        const int u = t < 4 ? t : t - 12;
        return lds_read_b128(lds_ptr(so) + ((u & 1) ? kroff1 : kroff0) + 64 * (u >> 1));
      }
      return lds_read_b128(lds_ptr(so) + ((t & 1) ? koff1 : koff0) + 64 * (t >> 1));
    };

    // Logit of key slot r in the log2 domain is s[r] * c[r]: c = the key's
    // inverse RMS times scale*log2(e) (K=V, from the tile) or scale*log2(e).
    const float cs = a.scale_log2;
    auto key_mul = [&](int so, float (&c)[16]) {
      if (TIED) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const f32x4 v = *(const G4_LDS f32x4*)(lds_ptr(so) + C::R_OFF + (8 * gq + 4 * hh) * 4);
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
    // Key slot r of tile kt is visible iff 0 <= d < w_eff with d = pos - key:
    // one unsigned compare (a global layer takes w_eff = 2^31 - 1).
    const uint32_t w_eff = a.window ? (uint32_t)a.window : 0x7fffffffu;
    // this lane's span: keys [s_lo, s_hi] are visible besides the window
    const int s_lo = spans ? a.span_lo[srow + min(tq, a.S - 1)] : 0;
    const int s_hi = spans ? min(a.span_hi[srow + min(tq, a.S - 1)], key_end - 1) : -1;
    auto visible = [&](int kt, int r) -> bool {
      const uint32_t d = (uint32_t)(pos - 4 * hh - kt * kBN) - (uint32_t)(8 * (r >> 2) + (r & 3));
      if (!spans) return d < w_eff;
      const int key = pos - (int)d;
      return (d < w_eff) | ((key >= s_lo) & (key <= s_hi));
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

    // S^T(tile in stage so) = K Q^T, K reads kLook ahead of their MFMA.
    auto qk = [&](int so) -> f32x16 {
      bf16x8 ka[kLook + 1];
#pragma unroll
      for (int t = 0; t < kLook; ++t) ka[t] = kread(so, t);
      f32x16 s = f32x16{};
#pragma unroll
      for (int t = 0; t < C::NT; ++t) {
        if (t + kLook < C::NT) ka[(t + kLook) % (kLook + 1)] = kread(so, t + kLook);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[t % (kLook + 1)], qf[t], s, 0, 0, 0);
      }
      return s;
    };

    // Softmax with a fixed per-row reference m_ref (log2 domain): the row's
    // maximum over its first tile with a visible key; P = exp2(x - m_ref) is
    // accumulated without ever rescaling O.  Every P is at most the row sum l,
    // so a row whose l stays <= 2^64 had no overflow risk; a wave with a larger
    // (or non-finite) l flags its workgroup, which the REDO launch recomputes
    // with m_ref = the true row maximum (every P <= 1 then).
    float m_ref = -INFINITY;
    float l_part[4] = {0.f, 0.f, 0.f, 0.f};  // four partial row sums: no serial add chain
    // Masked slots of an edge tile: s = mask_s makes s * c = -inf.
    auto mask_edge = [&](f32x16& s, int kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = visible(kt, r) ? s[r] : a.mask_s;
    };
    auto first_visible = [&](const f32x16& s, const float (&c)[16], int kt) {
      if (!REDO && __builtin_amdgcn_ballot_w64(m_ref == -INFINITY)) {  // a row meets its first visible key
        const float rowmx = max_xor32(tile_max(s, c, kt));
        m_ref = m_ref == -INFINITY ? rowmx : m_ref;
      }
    };
    // The softmax of one score tile as a list of micro-ops, stage by stage so
    // that no op waits on the one before it: 16 FMA (x = s c - m), 16 EXP2,
    // 8 pair sums, 8 row-sum adds, (K=V) 16 multiplies by c, 8 bf16 packs.
    constexpr int kSmOps = TIED ? 72 : 56;
    struct Sm {
      float x[16], ps[8];
      uint32_t w[8];
    };
    // Each op's result is pinned (an empty asm that takes it in and out), so
    // the op stays in its slot instead of sinking towards the result's use.
    auto sm_op = [&](Sm& st, const f32x16& s, const float (&c)[16], float m_use, int j) {
      if (j < 16) {
        st.x[j] = __builtin_fmaf(s[j], c[j], -m_use);
        pin(st.x[j]);
      } else if (j < 32) {
        st.x[j - 16] = __builtin_amdgcn_exp2f(st.x[j - 16]);
        pin(st.x[j - 16]);
      } else if (j < 40) {
        st.ps[j - 32] = st.x[2 * (j - 32)] + st.x[2 * (j - 32) + 1];
        pin(st.ps[j - 32]);
      } else if (j < 48) {
        l_part[(j - 40) & 3] += st.ps[j - 40];
        pin(l_part[(j - 40) & 3]);
      } else if (TIED && j < 64) {
        st.x[j - 48] *= c[j - 48];
        pin(st.x[j - 48]);
      } else {
        const int i = j - (TIED ? 64 : 48);
        st.w[i] = pack_bf2(st.x[2 * i], st.x[2 * i + 1]);
        pin(st.w[i]);
      }
    };
    auto sm_out = [&](const Sm& st, bf16x8 (&pb)[2]) {
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        const u32x4 w = {st.w[4 * mm], st.w[4 * mm + 1], st.w[4 * mm + 2], st.w[4 * mm + 3]};
        pb[mm] = __builtin_bit_cast(bf16x8, w);
      }
    };
    // P^T operands of score tile s (K=V: P times the key factor).
    auto softmax = [&](const f32x16& s, const float (&c)[16], bf16x8 (&pb)[2]) {
      const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
      Sm st;
#pragma unroll
      for (int j = 0; j < kSmOps; ++j) sm_op(st, s, c, m_use, j);
      sm_out(st, pb);
    };
    // S^T of the tile in stage so, with the softmax of s_prev spread over its
    // MFMAs: each MFMA is followed by its share of the micro-ops, fenced so the
    // scheduler keeps this order (the ops run while the MFMA does).
    // Copy pieces 0 .. NQ-1 of the step's loads ride along, one after every
    // fourth MFMA (issue(p) issues piece p).
    // ka[0 .. kLook-1] hold the first K fragments, read by the caller.
    auto qk_softmax = [&](int so, bf16x8 (&ka)[kLook + 1], const f32x16& s_prev, const float (&c)[16],
                          bf16x8 (&pb)[2], auto issue, auto nq) -> f32x16 {
      constexpr int NQ = decltype(nq)::value;
      static_assert(NQ <= C::NT / 4, "copy slots of the score MFMAs");
      const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
      Sm st;
      f32x16 s = f32x16{};
#pragma unroll
      for (int t = 0; t < C::NT; ++t) {
        if (t + kLook < C::NT) ka[(t + kLook) % (kLook + 1)] = kread(so, t + kLook);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[t % (kLook + 1)], qf[t], s, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = kSmOps * t / C::NT; j < kSmOps * (t + 1) / C::NT; ++j) sm_op(st, s_prev, c, m_use, j);
        if ((t & 3) == 0 && (t >> 2) < NQ) issue(t >> 2);
        __builtin_amdgcn_sched_barrier(0);
      }
      sm_out(st, pb);
      return s;
    };

    f32x16 oacc[C::NC];
#pragma unroll
    for (int c = 0; c < C::NC; ++c) oacc[c] = f32x16{};
    // O^T += V^T P^T over the tile in stage so, transposing reads kLook ahead;
    // copy pieces P0 .. P0+NP-1 ride along, one after every fourth MFMA.
    auto pv = [&](int so, const bf16x8 (&pb)[2], auto issue, auto p0, auto np) {
      constexpr int P0 = decltype(p0)::value, NP = decltype(np)::value;
      constexpr int NPV = 2 * C::NC;  // (mm, c) pairs
      static_assert(NP <= NPV / 4, "copy slots of the PV MFMAs");
      auto vread = [&](int i) -> bf16x8 {
        const int mm = i / C::NC, c = i % C::NC;
        const i16x4 lo = lds_read_tr16(lds_ptr(so) + toff[mm][0] + 64 * c);
        const i16x4 hi = lds_read_tr16(lds_ptr(so) + toff[mm][1] + 64 * c);
        return cat_tr(lo, hi);
      };
      bf16x8 va[kLook + 1];
#pragma unroll
      for (int i = 0; i < kLook; ++i) va[i] = vread(i);
#pragma unroll
      for (int i = 0; i < NPV; ++i) {
        if (i + kLook < NPV) va[(i + kLook) % (kLook + 1)] = vread(i + kLook);
        const int mm = i / C::NC, c = i % C::NC;
        if (c == 0)
          mfma_acc<true>(oacc[c], va[i % (kLook + 1)], pb[mm]);
        else
          mfma_acc<false>(oacc[c], va[i % (kLook + 1)], pb[mm]);
        if ((i & 3) == 1 && (i >> 2) < NP) issue(P0 + (i >> 2));
      }
    };
    auto no_issue = [](int) {};

    if (REDO) {
      // first sweep: the true maximum of every row (stages 0 and 1 hold kt_lo
      // and kt_lo + 1 already; two-stage ring)
      float m_run = -INFINITY;
      int so = 0;
      for (int kt = kt_lo; kt <= kt_hi; ++kt) {
        wait_vmem_all();
        __syncthreads();  // tile kt (and kt + 1) landed; every wave is done with tile kt - 1
        if (kt > kt_lo && kt < kt_hi)
          load_tile<D, TIED>(a, lds0 + (C::STAGE - so), kt + 1, b, g, key_end, wave, lane);
        float c[16];
        key_mul(so, c);
        const f32x16 s = qk(so);
        m_run = fmaxf(m_run, tile_max(s, c, kt));
        so = C::STAGE - so;
      }
      m_ref = max_xor32(m_run);
      __syncthreads();  // every wave is done before the stages are reloaded
      load_tile<D, TIED>(a, lds0, kt_lo, b, g, key_end, wave, lane);
      if (kt_lo < kt_hi) load_tile<D, TIED>(a, lds0 + C::STAGE, kt_lo + 1, b, g, key_end, wave, lane);
    }

    wait_vmem_all();
    __syncthreads();
    // One pipeline step: softmax + PV of tile kt (scores s_cur) and the scores
    // of tile kt + 1 into s_nxt.  Written out twice per loop trip with the two
    // score registers swapped, so neither is ever copied.
    int so_cur = 0, so_nxt = C::STAGE, so_ld = NST == 3 ? 2 * C::STAGE : 0;
    constexpr int PER = D == 512 ? 8 : 4;  // copy pieces of a K or V half
    auto step = [&](int kt, f32x16& s_cur, f32x16& s_nxt) {
      // this wave's copies of tile kt+1 (three stages) or of K(kt+1) (two
      // stages: V(kt), issued after it, may still be in flight) have landed
      if (NST == 2)
        wait_vmem<PER>();
      else
        wait_vmem_all();
      __syncthreads();  // ... in every wave; every wave is done with tile kt-1
      // first K fragments of tile kt+1 right away: their latency hides under
      // the bookkeeping below
      bf16x8 ka[kLook + 1];
#pragma unroll
      for (int t = 0; t < kLook; ++t) ka[t] = kread(so_nxt, t);
      float c[16];
      key_mul(so_cur, c);
      first_visible(s_cur, c, kt);
      if (edge_tile(kt)) mask_edge(s_cur, kt);
      bf16x8 pb[2];
      // The step's copies, spread over both MFMA runs (neither target is read
      // in this step).  Three stages: tile kt+2 goes to the stage tile kt-1
      // left.  Two stages: K(kt+2), during the score MFMAs, goes where K(kt)
      // was (its scores were taken in the last step), and V(kt+1), during
      // PV, where V(kt-1) was; V(kt+1) is waited for only before the next
      // step's PV, so each half has about a step to land.  (The first step
      // copies V(kt+1) again and, past the end, K(kt_hi) again, into halves
      // nothing reads, which keeps the count of copies in flight fixed.)
      constexpr int NP = TilePieces<D, TIED>::N;
      constexpr int NQ = NST == 2 ? PER : (NP + 1) / 2;  // pieces issued during the score MFMAs
      const TileSrc tsk = tile_src<D, TIED>(a, min(kt + 2, kt_hi), b, g, key_end);
      const TileSrc tsv = tile_src<D, TIED>(a, NST == 2 ? kt + 1 : kt_hi, b, g, key_end);
      const uint32_t st_k = lds0 + (NST == 3 ? so_ld : so_cur), st_v = lds0 + so_nxt;
      auto issue = [&](int p) {
        if (NST == 3 || p < PER)
          load_piece<D, TIED>(a, tsk, st_k, wave, lane, p);
        else
          load_piece<D, TIED>(a, tsv, st_v, wave, lane, p);
      };
      s_nxt = qk_softmax(so_nxt, ka, s_cur, c, pb, issue, std::integral_constant<int, NQ>{});
      __builtin_amdgcn_sched_barrier(0);
      if (NST == 2) {  // V(kt), copied during the last step's PV, has landed in every wave
        wait_vmem<PER>();
        __syncthreads();
      }
      pv(so_cur, pb, issue, std::integral_constant<int, NQ>{}, std::integral_constant<int, NP - NQ>{});
      const int t = so_cur;
      so_cur = so_nxt;
      if (NST == 3) { so_nxt = so_ld; so_ld = t; } else { so_nxt = t; }
    };
    auto last = [&](f32x16& s_cur) {
      if (NST == 2) {  // two stages: V(kt_hi) was copied during the last step
        wait_vmem_all();
        __syncthreads();
      }
      float c[16];
      key_mul(so_cur, c);
      first_visible(s_cur, c, kt_hi);
      if (edge_tile(kt_hi)) mask_edge(s_cur, kt_hi);
      bf16x8 pb[2];
      softmax(s_cur, c, pb);
      pv(so_cur, pb, no_issue, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
    };
    f32x16 sa = qk(0), sb;
    int kt = kt_lo;
    for (; kt + 1 < kt_hi; kt += 2) {
      step(kt, sa, sb);
      step(kt + 1, sb, sa);
    }
    if (kt < kt_hi) {
      step(kt, sa, sb);
      sa = sb;
    }
    last(sa);
    wait_vmem_all();  // the extra copy of the last tile has landed before the wave ends
    // the last MFMA results are read below: 18 wait states cover an 8-pass XDL
    asm volatile("s_nop 15\n\ts_nop 1"
                 : "+a"(oacc[0]), "+a"(oacc[1]), "+a"(oacc[2]), "+a"(oacc[3]), "+a"(oacc[4]), "+a"(oacc[5]),
                   "+a"(oacc[6]), "+a"(oacc[7]));
    if constexpr (C::NC > 8)
      asm volatile(""
                   : "+a"(oacc[8 % C::NC]), "+a"(oacc[9 % C::NC]), "+a"(oacc[10 % C::NC]),
                     "+a"(oacc[11 % C::NC]), "+a"(oacc[12 % C::NC]), "+a"(oacc[13 % C::NC]),
                     "+a"(oacc[14 % C::NC]), "+a"(oacc[15 % C::NC]));

    // ---- epilogue: flag, normalise, round once to bf16, store
    const float l_tot = sum_xor32((l_part[0] + l_part[1]) + (l_part[2] + l_part[3]));
    if (!REDO) {
      const bool over = valid && !(l_tot <= 0x1p64f);
      if (lane == 0) wg_flags[wave] = __builtin_amdgcn_ballot_w64(over) != 0;
    }
    if (valid) {
      // K=V: P carried the factor c = r * scale*log2(e) / qmul; omul undoes it.
      const float inv = l_tot > 0.f ? (TIED ? a.omul : 1.f) / l_tot : 0.f;
      uint16_t* orow = a.out + b * a.os[0] + (int64_t)tq * a.os[1] + head * a.os[2];
      // 16-byte stores: a lane holds dims 8gq + 4hh .. +3 of its row; the two
      // lane halves trade so that each writes 8 consecutive dims (lanes
      // 0..31 the even gq, lanes 32..63 the odd one)
#pragma unroll
      for (int c = 0; c < C::NC; ++c) {
#pragma unroll
        for (int gp = 0; gp < 2; ++gp) {
          uint32_t pk[2][2];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const int gq = 2 * gp + k;
            pk[k][0] = pack_bf2(oacc[c][4 * gq + 0] * inv, oacc[c][4 * gq + 1] * inv);
            pk[k][1] = pack_bf2(oacc[c][4 * gq + 2] * inv, oacc[c][4 * gq + 3] * inv);
          }
          uint32_t x0, x1, x2, x3;
          half_swap(pk[0][0], pk[1][0], x0, x2);
          half_swap(pk[0][1], pk[1][1], x1, x3);
          *(u32x4*)(orow + 32 * c + 8 * (2 * gp + hh)) = u32x4{x0, x1, x2, x3};
        }
      }
      if (a.lse && hh == 0) {
        a.lse[((int64_t)b * a.Hq + head) * a.S + tq] =
            l_tot > 0.f ? (m_ref + __log2f(l_tot)) * kLn2 : -INFINITY;
      }
    }
    if (!REDO) return;
    __syncthreads();  // every wave is done with the LDS before the next tile reuses it
  }
}

// D = 256 without K=V, two waves per SIMD.  With 256 registers a wave has
// room for O (128, AGPRs), Q^T (64) and one score tile, but not for the
// software pipeline of prefill_kernel; instead the second wave on each SIMD
// runs its MFMAs while this one does its softmax, copies and barrier.  A
// workgroup of NW waves owns 32 NW rows; with NW = 4 two workgroups share a
// CU, so one can run while the other waits at its barrier (NW = 8, one per
// CU, copies each K/V tile for twice the rows but measured slower).  Two LDS
// stages (70 KiB); the tile loop is the plain one: copy tile kt+1, S = K Q^T,
// softmax, O += V^T P^T.  Same layouts, masks, fixed-reference softmax and
// recompute launch as prefill_kernel.
template <int NW, bool REDO, bool EXT>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_d256_kernel(PrefillArgs a) {
  constexpr int D = 256;
  typedef Cfg<D, false> C;
  constexpr int BM = 32 * NW;  // rows per workgroup
  constexpr int L2 = 2;  // LDS operand reads issued ahead of their MFMA
  __shared__ __attribute__((aligned(1024))) char smem[2 * C::STAGE];
  const uint32_t lds0 = lds_addr((G4_LDS void*)smem);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int hh = lane >> 5;
  const int lr = lane & 31;
  const int G = a.Hq / a.Hkv;
  const int ntiles = (int)(((int64_t)a.S * G + BM - 1) / BM);
  // Main pass: one workgroup per row tile.  Recompute pass: a small grid of
  // persistent workgroups tests every row tile's flags in parallel and redoes
  // the flagged ones (most launches find none).
  RedoCursor redo{(int64_t)ntiles * a.Hkv * a.B};
  for (;;) {
    int b, g, tile;
    if (REDO) {
      // the next row tile whose main pass flagged a reference overflow (the
      // flags of tile L = tile + ntiles (g + Hkv b) sit at flags[L * waves])
      const int64_t L = redo.next([&](int64_t c) {
        static_assert(NW == 4, "four wave flags per row tile");
        const u32x4 f = *(const u32x4*)(a.flags + c * NW);
        return (f[0] | f[1] | f[2] | f[3]) != 0u;
      });
      if (L < 0) return;
      tile = (int)(L % ntiles);
      g = (int)((L / ntiles) % a.Hkv);
      b = (int)(L / ((int64_t)ntiles * a.Hkv));
    } else {
      // sliding layers longer than their window: most tiles cost the same
      wg_map(ntiles, a.Hkv, b, g, tile, a.window > 0 && a.S > a.window);
    }

    // Rows t < n of this sequence are positions P + t (P = 0, n = S unless
    // the keys come from a cache: chunked prefill, padded batches).
    // Device-side values are clamped: a sequence with pos0 < 0 has no rows,
    // and rows past the host's bound max_pos are not computed, so no key
    // past the cache is ever read.
    int P = 0, n = a.S;
    if (EXT && a.pos0) {
      P = a.pos0[b];
      n = a.qlen ? min(a.qlen[b], a.S) : a.S;
      n = P < 0 ? 0 : max(0, min(n, a.max_pos + 1 - P));
    }
    const int key_end = P + n;  // keys [0, key_end) exist
    const int64_t F0 = (int64_t)tile * BM;
    const int64_t Flast = min(F0 + BM - 1, (int64_t)a.S * G - 1);
    // first and last query positions of the workgroup's valid rows
    const int tr0 = (int)(F0 / G), tr1 = EXT ? min((int)(Flast / G), n - 1) : (int)(Flast / G);
    const int tq0 = P + tr0, tq1 = P + tr1;
    const int64_t F = F0 + wave * 32 + lr;
    const int tq = (int)(F / G);
    const int head = g * G + (int)(F % G);
    const bool valid = tq < n;
    const int pos = P + tq;  // this lane's query position

    // Bidirectional spans: row t also sees keys [span_lo, span_hi] (its own
    // image span).  The bounds grow with t, so the workgroup's first row has
    // the lowest and its last valid row the highest.
    const bool spans = EXT && a.span_lo != nullptr;
    const int64_t srow = (int64_t)b * a.S;
    const int kt_lo = max(0, min(a.window ? tq0 - a.window + 1 : 0, spans ? a.span_lo[srow + tr0] : tq0)) / kBN;
    const int kt_hi = min(max(tq1, spans ? a.span_hi[srow + tr1] : tq1), key_end - 1) / kBN;
    int* wg_flags = a.flags + (((int64_t)b * a.Hkv + g) * ntiles + tile) * NW;
    if (EXT && tq0 > tq1) {  // only padding rows: nothing to compute (uniform)
      if (!REDO && threadIdx.x < NW) wg_flags[threadIdx.x] = 0;
      if (!REDO) return;
      continue;
    }

    // Copy of key tile kt: each of the NW waves copies 16/NW row pairs of K
    // and of V (lanes 0..31 row s, lanes 32..63 row s + 16); rows past S
    // re-read row S-1 (masked).
    auto load_tile_w = [&](uint32_t stage, int kt) {
      const TileSrc ts = tile_src<D, false>(a, kt, b, g, key_end);
      const uint32_t rs = (uint32_t)(a.ks[1] * 2);
#pragma unroll
      for (int which = 0; which < 2; ++which)
#pragma unroll
        for (int i = 0; i < 16 / NW; ++i) {
          const int s = wave * (16 / NW) + i;
          const uint32_t r0 = min((uint32_t)s * rs, ts.last_off);
          const uint32_t r1 = min((uint32_t)(s + 16) * rs, ts.last_off);
          const uint32_t off = ((lane >> 5) ? r1 : r0) + (uint32_t)((lane & 31) ^ kv_xor<D>(s)) * 16u;
          g2lds16s(which ? ts.v : ts.k, off, stage + which * C::KT_BYTES + s * kSeg);
        }
    };
    // Q^T first, then the first two tiles: the first tile's wait then leaves
    // the second one's copies in flight (vector-memory counts retire in order)
    bf16x8 qf[C::NT];
    {
      const uint16_t* qrow = a.q + b * a.qs[0] + (int64_t)min(tq, a.S - 1) * a.qs[1] + head * a.qs[2];
#pragma unroll
      for (int t = 0; t < C::NT; ++t) qf[t] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qrow + 16 * t + 8 * hh));
    }
    constexpr int kLoadsPerTile = 2 * (16 / NW);  // this wave's copies of one K/V tile
    load_tile_w(lds0, kt_lo);
    if (kt_lo < kt_hi) load_tile_w(lds0 + C::STAGE, kt_lo + 1);

    const int k_x = kv_xor<D>(lr);
    const uint32_t koff0 = kv_row_off<D>(lr) + 16 * (hh ^ k_x);
    const uint32_t koff1 = kv_row_off<D>(lr) + 16 * ((2 + hh) ^ k_x);
    const int tG = lane >> 4, te = (lane >> 2) & 3, tqd = lane & 3;
    const int tr_row0 = 4 * (tG >> 1) + te;
    const int tr_chunk = 2 * (tG & 1) + (tqd >> 1);
    int toff[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int R = 16 * m + 8 * u + tr_row0;
        toff[m][u] = C::KT_BYTES + kv_row_off<D>(R) + (tqd & 1) * 8 + 16 * (tr_chunk ^ kv_xor<D>(R));
      }
    auto lds_ptr = [&](int so) { return (const G4_LDS char*)smem + so; };

    const float cs = a.scale_log2;
    const uint32_t w_eff = a.window ? (uint32_t)a.window : 0x7fffffffu;
    auto edge_tile = [&](int kt) {
      const int key0 = kt * kBN;
      return !((key0 + kBN - 1 <= tq0) && (a.window == 0 || key0 >= tq1 - a.window + 1));
    };
    // this lane's span: keys [s_lo, s_hi] are visible besides the window
    const int s_lo = spans ? a.span_lo[srow + min(tq, a.S - 1)] : 0;
    const int s_hi = spans ? min(a.span_hi[srow + min(tq, a.S - 1)], key_end - 1) : -1;
    auto visible = [&](int kt, int r) -> bool {
      const uint32_t d = (uint32_t)(pos - 4 * hh - kt * kBN) - (uint32_t)(8 * (r >> 2) + (r & 3));
      if (!spans) return d < w_eff;
      const int key = pos - (int)d;
      return (d < w_eff) | ((key >= s_lo) & (key <= s_hi));
    };
    auto tile_max = [&](const f32x16& s, int kt) {
      const bool edge = edge_tile(kt);
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, ((!edge) | visible(kt, r)) ? s[r] * cs : -INFINITY);
      return mx;
    };
    auto qk = [&](int so) -> f32x16 {
      bf16x8 ka[L2 + 1];
      auto kread = [&](int t) {
        return lds_read_b128(lds_ptr(so) + ((t & 1) ? koff1 : koff0) + 64 * (t >> 1));
      };
#pragma unroll
      for (int t = 0; t < L2; ++t) ka[t] = kread(t);
      f32x16 s = f32x16{};
#pragma unroll
      for (int t = 0; t < C::NT; ++t) {
        if (t + L2 < C::NT) ka[(t + L2) % (L2 + 1)] = kread(t + L2);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[t % (L2 + 1)], qf[t], s, 0, 0, 0);
      }
      return s;
    };

    float m_ref = -INFINITY;
    float l_part[4] = {0.f, 0.f, 0.f, 0.f};
    if (REDO) {
      float m_run = -INFINITY;
      int so = 0;
      for (int kt = kt_lo; kt <= kt_hi; ++kt) {
        wait_vmem_all();
        __syncthreads();
        if (kt > kt_lo && kt < kt_hi) load_tile_w(lds0 + (C::STAGE - so), kt + 1);
        m_run = fmaxf(m_run, tile_max(qk(so), kt));
        so = C::STAGE - so;
      }
      m_ref = max_xor32(m_run);
      __syncthreads();
      load_tile_w(lds0, kt_lo);
      if (kt_lo < kt_hi) load_tile_w(lds0 + C::STAGE, kt_lo + 1);
    }

    // The workgroup walks the band of all its rows; a tile holding no key
    // that any of this wave's rows sees adds exact zeros to O and l, so the
    // wave skips its MFMAs and softmax (it still copies and meets the
    // barrier) and the other wave on its SIMD gets the matrix core.  Spans
    // widen the visible set, so with spans every tile is computed.
    const int64_t Fw0 = F0 + wave * 32;
    const int pw0 = P + (int)(Fw0 / G);
    const int pw1 = P + min((int)((Fw0 + 31) / G), n - 1);
    auto wave_sees = [&](int kt) {
      const int key0 = kt * kBN;
      return spans || (pw0 <= pw1 && key0 <= pw1 && (a.window == 0 || key0 + kBN - 1 > pw0 - a.window));
    };

    f32x16 oacc[C::NC];
#pragma unroll
    for (int c = 0; c < C::NC; ++c) oacc[c] = f32x16{};
    int so = 0;
    for (int kt = kt_lo; kt <= kt_hi; ++kt) {
      // this wave's copies of tile kt have landed (at kt_lo those of kt_lo+1 may not have)
      if (kt == kt_lo && kt_lo < kt_hi)
        wait_vmem<kLoadsPerTile>();
      else
        wait_vmem_all();
      __syncthreads();  // all of tile kt is in LDS; every wave is done with tile kt-1
      if (kt > kt_lo && kt < kt_hi) load_tile_w(lds0 + (C::STAGE - so), kt + 1);
      if (!wave_sees(kt)) {
        so = C::STAGE - so;
        continue;
      }
      f32x16 s = qk(so);
      if (!REDO && __builtin_amdgcn_ballot_w64(m_ref == -INFINITY)) {
        const float rowmx = max_xor32(tile_max(s, kt));
        m_ref = m_ref == -INFINITY ? rowmx : m_ref;
      }
      if (edge_tile(kt)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = visible(kt, r) ? s[r] : a.mask_s;
      }
      const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
      bf16x8 pb[2];
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r0 = 8 * mm + 2 * i;
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r0], cs, -m_use));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r0 + 1], cs, -m_use));
          l_part[i] += p0 + p1;
          w[i] = pack_bf2(p0, p1);
        }
        pb[mm] = __builtin_bit_cast(bf16x8, w);
      }
      constexpr int NPV = 2 * C::NC;
      auto vread = [&](int i) -> bf16x8 {
        const int mm = i / C::NC, cb = i % C::NC;
        const i16x4 lo = lds_read_tr16(lds_ptr(so) + toff[mm][0] + 64 * cb);
        const i16x4 hi = lds_read_tr16(lds_ptr(so) + toff[mm][1] + 64 * cb);
        return cat_tr(lo, hi);
      };
      bf16x8 va[L2 + 1];
#pragma unroll
      for (int i = 0; i < L2; ++i) va[i] = vread(i);
#pragma unroll
      for (int i = 0; i < NPV; ++i) {
        if (i + L2 < NPV) va[(i + L2) % (L2 + 1)] = vread(i + L2);
        const int mm = i / C::NC, cb = i % C::NC;
        if (cb == 0)
          mfma_acc<true>(oacc[cb], va[i % (L2 + 1)], pb[mm]);
        else
          mfma_acc<false>(oacc[cb], va[i % (L2 + 1)], pb[mm]);
      }
      so = C::STAGE - so;
    }
    asm volatile("s_nop 15\n\ts_nop 1"
                 : "+a"(oacc[0]), "+a"(oacc[1]), "+a"(oacc[2]), "+a"(oacc[3]), "+a"(oacc[4]), "+a"(oacc[5]),
                   "+a"(oacc[6]), "+a"(oacc[7]));

    const float l_tot = sum_xor32((l_part[0] + l_part[1]) + (l_part[2] + l_part[3]));
    if (!REDO) {
      const bool over = valid && !(l_tot <= 0x1p64f);
      if (lane == 0) wg_flags[wave] = __builtin_amdgcn_ballot_w64(over) != 0;
    }
    if (valid) {
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      uint16_t* orow = a.out + b * a.os[0] + (int64_t)tq * a.os[1] + head * a.os[2];
      // 16-byte stores: a lane holds dims 8gq + 4hh .. +3 of its row; the two
      // lane halves trade so that each writes 8 consecutive dims (lanes
      // 0..31 the even gq, lanes 32..63 the odd one)
#pragma unroll
      for (int c = 0; c < C::NC; ++c) {
#pragma unroll
        for (int gp = 0; gp < 2; ++gp) {
          uint32_t pk[2][2];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const int gq = 2 * gp + k;
            pk[k][0] = pack_bf2(oacc[c][4 * gq + 0] * inv, oacc[c][4 * gq + 1] * inv);
            pk[k][1] = pack_bf2(oacc[c][4 * gq + 2] * inv, oacc[c][4 * gq + 3] * inv);
          }
          uint32_t x0, x1, x2, x3;
          half_swap(pk[0][0], pk[1][0], x0, x2);
          half_swap(pk[0][1], pk[1][1], x1, x3);
          *(u32x4*)(orow + 32 * c + 8 * (2 * gp + hh)) = u32x4{x0, x1, x2, x3};
        }
      }
      if (a.lse && hh == 0) {
        a.lse[((int64_t)b * a.Hq + head) * a.S + tq] =
            l_tot > 0.f ? (m_ref + __log2f(l_tot)) * kLn2 : -INFINITY;
      }
    }
    if (!REDO) return;
    __syncthreads();  // every wave is done with the LDS before the next tile reuses it
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  const int G = a.Hq / a.Hkv;
  const int64_t ntiles = ((int64_t)a.S * G + kBM - 1) / kBM;
  const dim3 grid((unsigned)ntiles, (unsigned)a.Hkv, (unsigned)a.B);
  constexpr int kNW256 = 4;  // waves per workgroup of the D = 256 kernel (8: slower, one workgroup per CU)
  const dim3 grid256((unsigned)(((int64_t)a.S * G + 32 * kNW256 - 1) / (32 * kNW256)), (unsigned)a.Hkv,
                     (unsigned)a.B);
  // recompute pass: persistent workgroups over every row tile
  auto redo_grid = [&](const dim3& gr) {
    const int64_t n = (int64_t)gr.x * gr.y * gr.z;
    return dim3((unsigned)(n < 1024 ? n : 1024));
  };
  const bool chunk = a.pos0 != nullptr || a.span_lo != nullptr;  // the extended variant
  for (int redo = 0; redo < 2; ++redo) {
    if (a.kv_tied && chunk)
      hipLaunchKernelGGL((redo ? prefill_kernel<512, true, true, true> : prefill_kernel<512, true, false, true>),
                         redo ? redo_grid(grid) : grid, dim3(256), 0, st, a);
    else if (a.kv_tied)
      hipLaunchKernelGGL((redo ? prefill_kernel<512, true, true, false> : prefill_kernel<512, true, false, false>),
                         redo ? redo_grid(grid) : grid, dim3(256), 0, st, a);
    else if (a.D == 512 && chunk)
      hipLaunchKernelGGL((redo ? prefill_kernel<512, false, true, true> : prefill_kernel<512, false, false, true>),
                         redo ? redo_grid(grid) : grid, dim3(256), 0, st, a);
    else if (a.D == 512)
      hipLaunchKernelGGL(
          (redo ? prefill_kernel<512, false, true, false> : prefill_kernel<512, false, false, false>),
          redo ? redo_grid(grid) : grid, dim3(256), 0, st, a);
    else if (chunk)
      hipLaunchKernelGGL((redo ? prefill_d256_kernel<kNW256, true, true> : prefill_d256_kernel<kNW256, false, true>),
                         redo ? redo_grid(grid256) : grid256, dim3(64 * kNW256), 0, st, a);
    else
      hipLaunchKernelGGL(
          (redo ? prefill_d256_kernel<kNW256, true, false> : prefill_d256_kernel<kNW256, false, false>),
          redo ? redo_grid(grid256) : grid256, dim3(64 * kNW256), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace g4attn
