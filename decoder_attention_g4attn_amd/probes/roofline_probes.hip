// Roofline probes: a bare bf16 MFMA loop and an HBM streaming read.  They
// measure the attainable ceilings the attention kernels are priced against;
// see include/g4probe.h for the calls.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/g4probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kAcc = 8;  // independent accumulators (and operand pairs) per wave

// A value in [-1, 1) from a 32-bit integer hash (C. Wellons' published
// "lowbias32" mixer): full-width mantissas, like the normally distributed
// activations the attention kernels multiply.
__device__ __forceinline__ float hash_unit(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return (float)(x >> 8) * (2.0f / 16777216.0f) - 1.0f;
}

// Eight independent 32x32x16 products per round, each with its own operand
// pair: each accumulator's previous product finishes long before its next
// one issues, so the matrix core never waits on a dependency, and the
// operands change from one product to the next as in a real contraction.
// LOW_ACTIVITY: every odd element of every operand is zero and the others
// one of a few short constants, so the multipliers barely switch.
template <bool LOW_ACTIVITY>
__global__ __launch_bounds__(256) void mfma_loop(float* out, int64_t iters) {
  const uint32_t lane = threadIdx.x & 63;
  bf16x8 a[kAcc], b[kAcc];
#pragma unroll
  for (int k = 0; k < kAcc; ++k)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (LOW_ACTIVITY) {
        a[k][i] = (__bf16)((i & 1) ? 0.f : 0.5f * (float)(k + 1));
        b[k][i] = (__bf16)((i & 1) ? 0.f : 0.25f);
      } else {
        a[k][i] = (__bf16)hash_unit(lane * 131u + k * 17u + i * 7u + 1u);
        b[k][i] = (__bf16)hash_unit(lane * 137u + k * 19u + i * 5u + 99991u);
      }
    }
  f32x16 acc[kAcc];
#pragma unroll
  for (int k = 0; k < kAcc; ++k) acc[k] = f32x16{};
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < kAcc; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k], b[k], acc[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kAcc; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[k][e];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// Each workgroup reads one contiguous chunk; thread t of a round reads the
// 16-byte element beg + t + 256 u of that round, so a wave's loads cover
// 1 KiB of consecutive bytes.  Every index is checked against the chunk end.
__global__ __launch_bounds__(256) void stream_read(const u32x4* __restrict__ src, uint32_t* sink, int64_t n16) {
  constexpr int U = 8;
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t beg = (int64_t)blockIdx.x * per;
  const int64_t end = beg + per < n16 ? beg + per : n16;
  uint32_t acc = 0;
  for (int64_t i = beg + threadIdx.x; i < end; i += 256 * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = i + 256 * u;
      v[u] = j < end ? __builtin_nontemporal_load(src + j) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

extern "C" int g4probe_mfma_bf16(float* out, int32_t workgroups, int64_t iters, int32_t operands, void* stream) {
  if (!out || workgroups < 1 || iters < 1 || (operands != G4PROBE_RANDOM && operands != G4PROBE_LOW_ACTIVITY))
    return -1;
  if (operands == G4PROBE_LOW_ACTIVITY)
    hipLaunchKernelGGL(mfma_loop<true>, dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream, out, iters);
  else
    hipLaunchKernelGGL(mfma_loop<false>, dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream, out, iters);
  return (int)hipGetLastError();
}

extern "C" int g4probe_stream_read(const void* src, int64_t bytes, uint32_t* sink, int32_t workgroups,
                                   void* stream) {
  if (!src || !sink || workgroups < 1 || bytes < 16 || bytes % 16 != 0 || ((uintptr_t)src & 15u) != 0)
    return -1;
  hipLaunchKernelGGL(stream_read, dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4*)src, sink, bytes / 16);
  return (int)hipGetLastError();
}
