// stage2.hip — split-KV stage 2: log-sum-exp merge of the stage-1 partials.
//
// The partial buffer keeps, per (sequence, query head, split), the chunk's normalised output and
// one extra value, its log-sum-exp (vLLM learning notes "模型库与算子层 — 概念", section
// "MLA 与 Sparse MLA（DSA）"). Merging is the identity
//     M = max_s lse_s,  w_s = exp(lse_s - M),  out = sum_s w_s o_s / sum_s w_s,
//     lse = M + ln(sum_s w_s)
// (an empty chunk has lse = -inf and weight 0; all empty gives out = 0, lse = -inf).
//
// One pass: one workgroup per (64-wide slice of d, query head, sequence), 256 threads = 16 split
// groups of 16 threads; a thread owns 4 consecutive d and walks splits g, g+16, ... in batches of
// B whose loads (partial rows and their lse) are all issued before any is used. B is the smallest
// power of two up to 8 with 16 B >= num_splits, so a plan with few splits issues no loads past its
// last split (clamped re-reads measured 0.4 us of a 4.4 us merge at 32 splits). Each thread keeps
// a running max, weight sum and weighted sum (rescaled when the max grows), so no separate pass
// over the lse values is needed. The 16 group states are merged in LDS in a fixed order
// (deterministic).

#include <hip/hip_runtime.h>

#include "internal.h"

namespace decode_attn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGroups = 16;                              // split groups per workgroup
constexpr int kGroupThreads = kStage2Threads / kGroups;  // 16 threads x 4 d = 64 d
#ifndef DECODE_ATTN_STAGE2_BATCH
#define DECODE_ATTN_STAGE2_BATCH 0
#endif
constexpr float kLog2e = 1.442695040888963407360f;
constexpr float kLn2f = 0.693147180559945309417f;

template <int kBatch>  // splits per thread per round of loads
__global__ __launch_bounds__(kStage2Threads) void stage2_kernel(const Stage2Args a) {
  __shared__ f32x4 acc_lds[kGroups][kGroupThreads];
  __shared__ float m_lds[kGroups];
  __shared__ float w_lds[kGroups];

  const int slice = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int g = tid / kGroupThreads;
  const int t = tid % kGroupThreads;
  const int ns = a.num_splits;
  const int D = a.head_dim;
  const size_t row = (size_t)b * a.num_q_heads + h;
  const float* lse = a.lse_part + row * ns;
  const int d = slice * 64 + 4 * t;
  const f32x4* o = reinterpret_cast<const f32x4*>(a.o_part + row * (size_t)ns * D + d);
  const size_t stride = (size_t)D / 4;  // f32x4 per partial row

  // Running state in base-2 units: max m, weight sum w, weighted sum acc (all relative to m).
  float m = -INFINITY, wsum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = g; s0 < ns; s0 += kGroups * kBatch) {
    float l[kBatch];
    f32x4 v[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int s = s0 + k * kGroups;
      const int sc = s < ns ? s : s0;  // in-bounds; out-of-range entries get weight 0 below
      l[k] = lse[sc];
      v[k] = o[(size_t)sc * stride];
    }
    float bm = m;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      l[k] = (s0 + k * kGroups < ns) ? l[k] * kLog2e : -INFINITY;
      bm = fmaxf(bm, l[k]);
    }
    if (bm != -INFINITY) {
      const float r = exp2f(m - bm);  // m == -inf gives 0
      wsum *= r;
      acc *= r;
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const float w = exp2f(l[k] - bm);  // -inf gives 0
        wsum += w;
        acc += w * v[k];
      }
      m = bm;
    }
  }
  acc_lds[g][t] = acc;
  if (t == 0) {
    m_lds[g] = m;
    w_lds[g] = wsum;
  }
  __syncthreads();

  if (g == 0) {
    float M = m_lds[0];
#pragma unroll
    for (int k = 1; k < kGroups; ++k) M = fmaxf(M, m_lds[k]);
    f32x4 tot = {0.f, 0.f, 0.f, 0.f};
    float W = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int k = 0; k < kGroups; ++k) {
        const float r = exp2f(m_lds[k] - M);
        tot += r * acc_lds[k][t];
        W += r * w_lds[k];
      }
    }
    const float inv = (M == -INFINITY) ? 0.f : 1.f / W;
    *reinterpret_cast<f32x4*>(a.out + row * D + d) = tot * inv;
    if (a.lse_out != nullptr && slice == 0 && t == 0)
      a.lse_out[row] = (M == -INFINITY) ? -INFINITY : (M + __log2f(W)) * kLn2f;
  }
}

}  // namespace

hipError_t launch_stage2(const Stage2Args& args, int batch, hipStream_t stream) {
  dim3 grid(args.head_dim / 64, args.num_q_heads, batch);
  dim3 block(kStage2Threads);
  void* kargs[] = {const_cast<Stage2Args*>(&args)};
  // DECODE_ATTN_STAGE2_BATCH (build knob, for A/B builds): 0 = by the split count, else that batch.
  const int ns = DECODE_ATTN_STAGE2_BATCH ? DECODE_ATTN_STAGE2_BATCH * kGroups : args.num_splits;
  const void* fn = ns <= kGroups       ? reinterpret_cast<const void*>(&stage2_kernel<1>)
                   : ns <= 2 * kGroups ? reinterpret_cast<const void*>(&stage2_kernel<2>)
                   : ns <= 4 * kGroups ? reinterpret_cast<const void*>(&stage2_kernel<4>)
                                       : reinterpret_cast<const void*>(&stage2_kernel<8>);
  return hipLaunchKernel(fn, grid, block, kargs, 0, stream);
}

}  // namespace decode_attn
