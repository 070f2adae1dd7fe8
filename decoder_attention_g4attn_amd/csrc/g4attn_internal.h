// Internal helpers shared by the g4attn HIP kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/g4attn.h"

namespace g4attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define G4_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even, NaN kept quiet: one v_cvt_pk_bf16_f32
// (gfx950) converts a pair.
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ uint32_t f2bf(float f) { return pack_bf2(f, 0.f) & 0xffffu; }
__device__ __forceinline__ float bf2f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// max / sum of a value and its copy in lane l ^ 32 (v_permlane32_swap: each
// result holds the lane's own value in one output and the partner's in the
// other, so combining both outputs needs no lane select).
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Exchange between lane halves (v_permlane32_swap): lanes 0..31 get their
// own `a` and their partner's `a`, lanes 32..63 their partner's `b` and
// their own `b`.  The results as {first, second} of each lane.
__device__ __forceinline__ void half_swap(uint32_t a, uint32_t b, uint32_t& first, uint32_t& second) {
  const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  first = r[0];
  second = r[1];
}

// Wave-wide (64 lanes) reductions.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Direct global->LDS copies: lane i's 16 (or 4) bytes land at lds_base +
// 16*i (4*i); lds_base must be wave-uniform.  They are issued as inline
// assembly on purpose: the compiler then does not know these loads write LDS
// and does not drain every one of them before each transposing LDS read.
// Callers therefore order them explicitly: `s_waitcnt vmcnt` (wait_vmem*)
// before any read of the data, and a workgroup barrier before a buffer is
// reused.  The instruction has no register results.
//
// The LDS destination travels in m0, a register the compiler reserves for
// itself, so each block saves m0 in a scratch SGPR, sets it, issues the load
// (which reads m0 when it is issued) and restores it: whatever the compiler
// keeps in m0 survives every copy.
__device__ __forceinline__ uint32_t lds_addr(const G4_LDS void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}
__device__ __forceinline__ void g2lds16(const void* gptr, G4_LDS void* lds_base) {
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(keep)
      : "v"(gptr), "s"(lds_addr(lds_base))
      : "memory");
}
__device__ __forceinline__ void g2lds4(const void* gptr, G4_LDS void* lds_base) {
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(keep)
      : "v"(gptr), "s"(lds_addr(lds_base))
      : "memory");
}

// The same copies with a wave-uniform 64-bit base in scalar registers plus
// an unsigned 32-bit per-lane byte offset (the scalar-base form); `lds` is the
// wave-uniform LDS byte address of lane 0's destination.
__device__ __forceinline__ void g2lds16s(const void* sbase, uint32_t voff, uint32_t lds) {
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\tglobal_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
      : "=&s"(keep)
      : "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds))
      : "memory");
}
__device__ __forceinline__ void g2lds4s(const void* sbase, uint32_t voff, uint32_t lds) {
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\tglobal_load_lds_dword %1, %2\n\ts_mov_b32 m0, %0"
      : "=&s"(keep)
      : "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds))
      : "memory");
}

__device__ __forceinline__ bf16x8 lds_read_b128(const G4_LDS char* p) {
  return *(const G4_LDS bf16x8*)p;
}
// Transposing LDS read: see the lane mapping in the kernels that use it.
__device__ __forceinline__ i16x4 lds_read_tr16(const G4_LDS char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((G4_LDS i16x4*)p);
}
__device__ __forceinline__ bf16x8 cat_tr(i16x4 a, i16x4 b) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 c = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, c);
}

__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// s_waitcnt vmcnt(n): n must be a compile-time constant.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Recompute launches: a small grid of persistent workgroups, workgroup w
// owning candidates L = w, w + grid, w + 2 grid, ... below `ntotal`.  The
// candidates are tested 64 at a time, one per lane (every wave of the
// workgroup tests the same 64 and gets the same ballot), so a launch that
// finds nothing to redo costs one round of flag loads.  next() returns the
// next candidate whose flagged(L) is true, or -1 when none is left; the
// result is wave-uniform and equal in every wave, so the caller may run
// workgroup barriers between calls.
struct RedoCursor {
  int64_t ntotal;
  int64_t k0 = -64;  // first candidate index of the current round
  uint64_t mk = 0;   // flagged candidates of the round not yet returned

  template <class Flagged>
  __device__ __forceinline__ int64_t next(Flagged flagged) {
    for (;;) {
      if (mk) {
        const int j = __builtin_ctzll(mk);
        mk &= mk - 1;
        return (int64_t)blockIdx.x + (k0 + j) * (int64_t)gridDim.x;
      }
      k0 += 64;
      if ((int64_t)blockIdx.x + k0 * gridDim.x >= ntotal) return -1;
      const int64_t Lt = (int64_t)blockIdx.x + (k0 + (threadIdx.x & 63)) * (int64_t)gridDim.x;
      mk = __builtin_amdgcn_ballot_w64(Lt < ntotal && flagged(Lt));
    }
  }
};

}  // namespace g4attn

// Launchers (host side), defined in the kernel files.
namespace g4attn {

struct NormRopeArgs {
  const uint16_t* x;
  uint16_t* y;
  const uint16_t* w;
  int B, S, H, D, rot;
  double log2_theta;
  float eps;
  int64_t xs[3], ys[3];
  const int32_t* pos0;
  int cache_cap;
  int ring;                 // cache mode: row p mod cache_cap instead of row p
};
hipError_t launch_norm_rope(const NormRopeArgs& a, hipStream_t st);

struct KvPrepArgs {         // K=V prefill pre-pass
  const uint16_t* x;        // [B, S, Hkv, 512] strided
  const uint16_t* w_k;      // [512]
  float* r;                 // [B, Hkv, S | cap] inverse RMS of each row times rscale
  uint16_t* krot;           // [B, Hkv, S | cap, 128]
  uint16_t* x_out;          // cache mode: [B, Hkv, cap, 512] copy of X, else NULL
  const int32_t* pos0;      // cache mode: [B] first position (NULL = 0)
  int cap;                  // 0: prefill layout; > 0: cache rows pos0[b] + t
  int B, S, Hkv, rot;
  float rscale;
  double log2_theta;
  float eps;
  int64_t xs[3];
};
hipError_t launch_kv_prep(const KvPrepArgs& a, hipStream_t st);

struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* k;        // K, or X (K=V)
  const uint16_t* v;        // V (NULL for K=V)
  const uint16_t* w_k;      // K=V only
  const float* r;           // K=V only: [B, Hkv, kv_rows] inverse RMS of each key row (times scale_log2
                            // in a whole-sequence prefill)
  const uint16_t* krot;     // K=V only: [B, Hkv, kv_rows, 128]
  int kv_rows;              // K=V only: rows per (b, g) of r and krot (S, or the cache capacity)
  int* flags;               // [B, Hkv, ntiles, 4] per-wave reference-overflow flags
  const int32_t* pos0;      // NULL, or [B] first query position of each sequence (keys from caches)
  const int32_t* qlen;      // NULL, or [B] valid query rows of each sequence (the rest is padding)
  int max_pos;              // with pos0: host bound of every key position (rows past it are not computed)
  const int32_t* span_lo;   // NULL, or [B, S] first key of each row's bidirectional span
  const int32_t* span_hi;   // [B, S] its last key (with span_lo)
  uint16_t* out;
  float* lse;
  int B, S, Hq, Hkv, D, window, kv_tied;
  float scale_log2;         // scale * log2(e), never 0 (FLT_MIN stands in for 0)
  float qmul, omul;         // K=V only: query and output multipliers (see g4attn_prefill)
  float mask_s;             // score of a masked slot: mask_s * (key factor) = -inf
  int64_t qs[3], ks[3], os[3];
};
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st);

struct DecodeArgs {
  const uint16_t* q;        // [B, Hq, D]
  const uint16_t* kc;       // [B, Hkv, cap, D]
  const uint16_t* vc;
  const int32_t* kv_len;    // [B]
  uint16_t* out;            // [B, Hq, D]
  float* lse;               // [B, Hq] or NULL
  float* o_part;            // [B, Hq, nsplit, D]
  float* lse_part;          // [B, Hq, nsplit]
  float* dmax;              // [B, Hq, nsplit] true logit maxima (log2 domain) of each chunk
  int* dflags;              // [B, Hkv, nsplit] reference-overflow flags of each chunk
  int B, Hq, Hkv, D, cap, nsplit, chunk;
  int max_len;              // host bound; kv_len values are clamped to [0, max_len]
  float scale_log2;
  // K=V decode over the raw projection (kc = X cache; vc unused):
  const float* rc;          // [B, Hkv, cap] inverse RMS of each cached row
  const uint16_t* krc;      // [B, Hkv, cap, 128] rotated part of each cached key, before r
  const uint16_t* w_k;      // [512] K-norm weight
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t st);
hipError_t launch_decode_tied(const DecodeArgs& a, hipStream_t st);

// Decode entry shared by g4attn_decode and g4attn_decode_noalloc (abi.hip):
// host validation of everything but the workspace, the split count whose
// workspace fits max_bytes (-1 if none), and validation + launch.
g4attn_status decode_validate(const g4attn_layer_desc* d, const g4attn_bf16* q, const g4attn_bf16* k_cache,
                              const g4attn_bf16* v_cache, const int32_t* kv_len, int32_t B, int32_t max_kv_len,
                              int32_t cache_cap, const g4attn_bf16* out, const float* lse, int32_t num_splits);
int32_t decode_fit_splits(const g4attn_layer_desc* d, int32_t B, int32_t max_kv_len, int32_t num_splits,
                          size_t max_bytes);
g4attn_status decode_run(const g4attn_layer_desc* d, const g4attn_bf16* q, const g4attn_bf16* k_cache,
                         const g4attn_bf16* v_cache, const int32_t* kv_len, int32_t B, int32_t max_kv_len,
                         int32_t cache_cap, g4attn_bf16* out, float* lse, int32_t num_splits, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);
g4attn_status status_of_hip(hipError_t e);

}  // namespace g4attn
