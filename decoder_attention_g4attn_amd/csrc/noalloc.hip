// g4attn_decode_noalloc: g4attn_decode for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, hosts
// that forbid allocation).  The decode's scratch (split partials, chunk
// maxima and recompute flags) lives in a file-scope device array instead of
// a caller workspace; the call allocates nothing.
//
// The array's name is a host-side stand-in, not a device address: each
// device's copy is looked up once with hipGetSymbolAddress (with that device
// current) and only that pointer is ever handed to kernels.
#include <mutex>

#include "g4attn_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;  // 32 MiB per device
constexpr int kMaxDevices = 64;

// One copy per device, held until the process ends.  Every call on a device
// shares it: calls that overlap on one device (several streams, several
// host threads) race on it.  Nothing in it needs to start at zero: every
// partial result, maximum and flag a launch reads was written by the same
// launch sequence first.
static __device__ __align__(256) char scratch[kScratchBytes];

std::once_flag g_once[kMaxDevices];
void* g_scratch[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

}  // namespace

extern "C" g4attn_status g4attn_decode_noalloc(const g4attn_layer_desc* desc, const g4attn_bf16* q,
                                               const g4attn_bf16* k_cache, const g4attn_bf16* v_cache,
                                               const int32_t* kv_len, int32_t B, int32_t max_kv_len,
                                               int32_t cache_cap, g4attn_bf16* out, float* lse,
                                               int32_t num_splits, void* stream) {
  const g4attn_status st = g4attn::decode_validate(desc, q, k_cache, v_cache, kv_len, B, max_kv_len, cache_cap,
                                                   out, lse, num_splits);
  if (st != G4ATTN_OK) return st;
  // the split count whose partial results fit the scratch array
  const int32_t ns = g4attn::decode_fit_splits(desc, B, max_kv_len, num_splits, kScratchBytes);
  if (ns < 0) return G4ATTN_ERR_WORKSPACE;

  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return g4attn::status_of_hip(e);
  if (dev < 0 || dev >= kMaxDevices) return G4ATTN_ERR_UNSUPPORTED;
  std::call_once(g_once[dev], [dev] {
    g_scratch_err[dev] = hipGetSymbolAddress(&g_scratch[dev], HIP_SYMBOL(scratch));
  });
  if (g_scratch_err[dev] != hipSuccess) return g4attn::status_of_hip(g_scratch_err[dev]);
  return g4attn::decode_run(desc, q, k_cache, v_cache, kv_len, B, max_kv_len, cache_cap, out, lse, ns,
                            g_scratch[dev], kScratchBytes, (hipStream_t)stream);
}
