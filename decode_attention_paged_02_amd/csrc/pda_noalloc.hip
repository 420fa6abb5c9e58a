// pda_noalloc.hip -- paged_decode_attn for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, hosts that
// forbid hipMalloc): the same call and kernels, with the workspace (split
// partials, the ordered work list) taken from a fixed device array that the
// library holds for the life of the process.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <mutex>

#include "pda.h"

namespace {

// Largest workspace the call can use: 64 MiB per GPU (the B=128 x 64-head
// ragged batch with 8 splits needs 32.3 MiB; B=1 at 32768 tokens with 64
// splits 1 MiB).
constexpr size_t kScratchBytes = size_t(64) << 20;

// The scratch array; every GPU the library runs on holds its own copy.  In
// host code this name only stands for the symbol: its device address comes
// from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_init;

// Device address of the current device's scratch array (looked up on the
// first call on that device, with the device current); PDA_ERR_HIP when the
// device or the lookup fails.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PDA_ERR_HIP;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_init);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PDA_ERR_HIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return PDA_OK;
}

}  // namespace

extern "C" int paged_decode_attn_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                         const int32_t* block_tables, const int32_t* context_lens,
                                         int group, float scale, int num_splits, void* out,
                                         float* lse, const pda_shape* shape, void* stream) {
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out || !shape)
    return PDA_ERR_INVALID_ARG;
  if (group <= 0 || group * shape->num_kv_heads != shape->num_q_heads) return PDA_ERR_INVALID_ARG;
  if (!(scale == scale) || num_splits < 0) return PDA_ERR_INVALID_ARG;
  pda_plan_info plan;
  int rc = pda_plan(shape, 0, num_splits, 0, &plan);
  if (rc != PDA_OK) return rc;
  if (shape->batch == 0) return PDA_OK;
  if (plan.workspace_bytes > kScratchBytes) return PDA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (plan.workspace_bytes > 0) {
    rc = scratch_address(&ws);
    if (rc != PDA_OK) return rc;
  }
  return paged_decode_attn(q, k_cache, v_cache, block_tables, context_lens, group, scale,
                           num_splits, out, lse, shape, ws, ws ? kScratchBytes : 0, stream);
}
