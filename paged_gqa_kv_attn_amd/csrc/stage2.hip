// stage2.hip — split-KV stage 2: log-sum-exp merge of the stage-1 partials.
//
// The partial buffer keeps, per (sequence, query head, split), the chunk's normalised output and
// one extra value, its log-sum-exp (vLLM learning notes "模型库与算子层 — 概念", section
// "MLA 与 Sparse MLA（DSA）"). Merging is the identity
//     M = max_s lse_s,  w_s = exp(lse_s - M),  out = sum_s w_s o_s / sum_s w_s,
//     lse = M + ln(sum_s w_s)
// (an empty chunk has lse = -inf and weight 0; all empty gives out = 0, lse = -inf).
//
// One workgroup per (64-wide slice of d, query head, sequence): lane l owns d = slice*64 + l, so
// every partial row is read with one coalesced 256-byte access per wave; the 4 waves take splits
// w, w+4, ... and are combined in LDS in a fixed order.

#include <hip/hip_runtime.h>

#include "internal.h"

namespace decode_attn {
namespace {

constexpr int kWaves2 = kStage2Threads / 64;
constexpr float kLog2e = 1.442695040888963407360f;
constexpr float kLn2f = 0.693147180559945309417f;

__global__ __launch_bounds__(kStage2Threads) void stage2_kernel(const Stage2Args a) {
  __shared__ float red_lds[kWaves2];
  __shared__ float acc_lds[kWaves2][64];
  __shared__ float wsum_lds[kWaves2];

  const int slice = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int ns = a.num_splits;
  const int D = a.head_dim;
  const size_t row = (size_t)b * a.num_q_heads + h;
  const float* lse = a.lse_part + row * ns;

  // M = max over splits.
  float m = -INFINITY;
  for (int s = threadIdx.x; s < ns; s += kStage2Threads) m = fmaxf(m, lse[s]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if (lane == 0) red_lds[wave] = m;
  __syncthreads();
  float M = red_lds[0];
#pragma unroll
  for (int w = 1; w < kWaves2; ++w) M = fmaxf(M, red_lds[w]);

  // Weighted sum over this wave's splits.
  const int d = slice * 64 + lane;
  const float* o = a.o_part + row * (size_t)ns * D + d;
  float acc = 0.f, wsum = 0.f;
  if (M != -INFINITY) {
#pragma unroll 4
    for (int s = wave; s < ns; s += kWaves2) {
      const float l = lse[s];
      const float w = (l == -INFINITY) ? 0.f : exp2f((l - M) * kLog2e);
      acc = fmaf(w, o[(size_t)s * D], acc);
      wsum += w;
    }
  }
  acc_lds[wave][lane] = acc;
  if (lane == 0) wsum_lds[wave] = wsum;
  __syncthreads();

  if (wave == 0) {
    float tot = 0.f, W = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves2; ++w) {
      tot += acc_lds[w][lane];
      W += wsum_lds[w];
    }
    a.out[row * D + d] = (M == -INFINITY) ? 0.f : tot / W;
    if (a.lse_out != nullptr && slice == 0 && lane == 0)
      a.lse_out[row] = (M == -INFINITY) ? -INFINITY : M + __log2f(W) * kLn2f;
  }
}

}  // namespace

hipError_t launch_stage2(const Stage2Args& args, int batch, hipStream_t stream) {
  dim3 grid(args.head_dim / 64, args.num_q_heads, batch);
  dim3 block(kStage2Threads);
  void* kargs[] = {const_cast<Stage2Args*>(&args)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&stage2_kernel), grid, block, kargs, 0,
                         stream);
}

}  // namespace decode_attn
