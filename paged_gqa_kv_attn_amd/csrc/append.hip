// append.hip — paged KV append: the newest tokens' keys and values go into their page slots before
// attention reads them (the cache-manager write of Sparse-vLLM PR #27 "feat: support Gemma 4 and
// native multimodal inference", section "Gemma 4 文本推理"; the context length counts the
// tokens). With L new tokens per sequence, token i goes to position n - L + i.
//
// One workgroup of 64 lanes per (sequence and new token, KV head); every lane moves 16-byte chunks
// of the row. A position below 0 or outside the block-table row, or a page id outside [0, P), is
// skipped (nothing written).

#include <hip/hip_runtime.h>

#include "internal.h"

namespace decode_attn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(64) void append_kernel(const AppendArgs a) {
  const int b = blockIdx.x / a.q_len;
  const int i = blockIdx.x - b * a.q_len;  // new token i of sequence b
  const int g = blockIdx.y;
  const int t = a.ctx_lens[b] - a.q_len + i;
  if (t < 0) return;
  const int col = t / a.page_size;
  if (col >= a.max_pages_per_seq) return;
  const int page = a.block_table[(size_t)b * a.max_pages_per_seq + col];
  if ((unsigned)page >= (unsigned)a.num_pages) return;
  const size_t dst = (((size_t)page * a.num_kv_heads + g) * a.page_size + (t - col * a.page_size)) *
                     a.head_dim;
  const size_t src = ((size_t)blockIdx.x * a.num_kv_heads + g) * a.head_dim;
  for (int c = threadIdx.x; c < a.head_dim / 8; c += 64) {
    reinterpret_cast<u32x4*>(a.k_pool + dst)[c] = reinterpret_cast<const u32x4*>(a.k_new + src)[c];
    if (a.v_pool != a.k_pool)
      reinterpret_cast<u32x4*>(a.v_pool + dst)[c] = reinterpret_cast<const u32x4*>(a.v_new + src)[c];
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& args, int batch, hipStream_t stream) {
  dim3 grid(batch * args.q_len, args.num_kv_heads);
  dim3 block(64);
  void* kargs[] = {const_cast<AppendArgs*>(&args)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&append_kernel), grid, block, kargs, 0,
                         stream);
}

}  // namespace decode_attn
