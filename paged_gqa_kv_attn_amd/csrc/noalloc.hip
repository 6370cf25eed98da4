// noalloc.hip — decode_attn_layer_noalloc: the layer call of decode_attn_global /
// decode_attn_sliding with its workspace (the stage-1 partials and their log-sum-exps) in a
// static device array of this library instead of a caller buffer, for callers that cannot
// allocate device memory. Declared and documented in include/decode_attn.h.

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "decode_attn.h"
#include "internal.h"

namespace decode_attn {
namespace {

static_assert(DECODE_ATTN_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");

// The workspace of every decode_attn_layer_noalloc call on a device. Each device that runs the
// library holds its own copy for the life of the process. In host code this name is only a
// stand-in for the symbol: its device address comes from hipGetSymbolAddress below.
__device__ __align__(256) unsigned char scratch[DECODE_ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch[kMaxScratchDevices];  // device address per device, null until looked up
std::mutex g_scratch_mu;

// Device address of the current device's scratch array, looked up once per device with that
// device current.
int scratch_address(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices)
    return DECODE_ATTN_ERR_HIP;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
        return DECODE_ATTN_ERR_HIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return DECODE_ATTN_OK;
}

}  // namespace
}  // namespace decode_attn

using namespace decode_attn;

extern "C" int decode_attn_layer_noalloc(const decode_attn_plan_t* plan, const void* q,
                                         const void* k_pool, const void* v_pool,
                                         const int32_t* block_table, const int32_t* ctx_lens,
                                         int32_t batch, int32_t window, float scale, float* out,
                                         float* lse_out, void* stream) {
  if (plan == nullptr) return DECODE_ATTN_ERR_NULL;
  if (plan->magic != kPlanMagic) return DECODE_ATTN_ERR_PLAN;
  if (window != plan->problem.window) return DECODE_ATTN_ERR_SHAPE;
  if (plan->layer_workspace_bytes > DECODE_ATTN_NOALLOC_SCRATCH_BYTES)
    return DECODE_ATTN_ERR_WORKSPACE;
  if (batch == 0)  // nothing to launch; attend() still checks the plan and the batch
    return attend(plan, window > 0 ? 2 : 1, q, k_pool, v_pool, block_table, ctx_lens, batch,
                  scale, out, lse_out, nullptr, 0, stream);
  void* ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc != DECODE_ATTN_OK) return rc;
  // Every partial row and lse of the plan is written by stage 1 before stage 2 reads it (an empty
  // chunk writes o = 0, lse = -inf), so the array needs no clearing between calls.
  return attend(plan, window > 0 ? 2 : 1, q, k_pool, v_pool, block_table, ctx_lens, batch, scale,
                out, lse_out, ws, DECODE_ATTN_NOALLOC_SCRATCH_BYTES, stream);
}
