// append_rope.hip — the step just before attention, in one launch: RMSNorm of every q head and of
// every new k head (QK-norm), rotary position embedding of both at the token's position, an
// optional RMSNorm of the new v heads, and the paged append of k and v into their page slots.
// Sparse-vLLM PR #27 "feat: support Gemma 4 and native multimodal inference" lists a dedicated
// QKV-norm + RoPE operator (section "专用算子与性能优化") and gives each Gemma 4 layer kind its own
// RoPE parameters and RoPE cache (section "Gemma 4 文本推理"); vLLM learning notes "模型库与算子层 —
// 概念" fuse norm/RoPE with the paged KV-cache write so that no launch and no intermediate tensor
// sits between them (section "自定义 Inductor 融合 pass"), and fuse the q/k RMSNorm with RoPE in
// place for both pairings, NeoX halves and GPT-J interleaved pairs (section "内核框架（Helion）").
//
// Layout of the work: one wave per (new token, row), a row being a q head, a new k head or a new
// v head; four waves per workgroup, the workgroups of one token along grid.y. Each lane holds
// D / 64 consecutive elements of its row (one 16-byte load at D = 512, 8 bytes at D = 256), so a
// row is one coalesced read and one coalesced write. The RMS is a wave reduction; the NeoX pair
// partner (element d +- R/2, held by another lane) comes through a per-wave LDS row, the
// interleaved partner is in the same lane. Arithmetic is fp32 and each result is rounded once to
// bf16 (nearest even). The rotation table (cos and sin per position and pair, fp32) is built
// once per layer configuration by rope_cache_kernel in double precision.

#include <hip/hip_runtime.h>

#include "device_common.h"
#include "internal.h"

namespace decode_attn {
namespace {

constexpr int kRopeWaves = 4;

__global__ __launch_bounds__(256) void rope_cache_kernel(float* cos_sin, int64_t count,
                                                         int rotary_dim, int freq_dim,
                                                         double theta) {
  const int half = rotary_dim / 2;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < count;
       idx += (int64_t)gridDim.x * 256) {
    const int64_t t = idx / half;
    const int j = (int)(idx - t * half);
    // f_j = theta^(-2j / freq_dim), in double; the angle t * f_j keeps ~1e-11 rad at t = 2^20.
    const double f = pow(theta, -2.0 * j / freq_dim);
    double s, c;
    sincos((double)t * f, &s, &c);
    cos_sin[t * rotary_dim + j] = (float)c;
    cos_sin[t * rotary_dim + half + j] = (float)s;
  }
}

template <int E>
struct RowVec;
template <>
struct RowVec<4> {
  typedef u32x2 type;  // 4 bf16
};
template <>
struct RowVec<8> {
  typedef u32x4 type;  // 8 bf16
};

template <int D>
__global__ __launch_bounds__(256) void append_rope_kernel(const AppendRopeArgs a) {
  constexpr int E = D / 64;
  typedef typename RowVec<E>::type vec_t;
  __shared__ float rows[kRopeWaves][D];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tok = blockIdx.x;  // b * L + i
  const int b = tok / a.q_len;
  const int i = tok - b * a.q_len;
  const int t = a.ctx_lens[b] - a.q_len + i;
  if (t < 0 || t >= a.max_position) return;  // the same for the whole workgroup

  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const bool same = a.v_pool == a.k_pool;
  const int rows_per_token = Hq + Hkv * (same ? 1 : 2);
  const int r = blockIdx.y * kRopeWaves + wave;

  const uint16_t* src = nullptr;
  uint16_t* dst = nullptr;
  const float* weight = nullptr;
  bool norm = false, rotate = false;
  if (r < Hq) {
    src = a.q + ((size_t)tok * Hq + r) * D;
    dst = a.q_out + ((size_t)tok * Hq + r) * D;
    weight = a.q_weight;
    norm = a.norm_flags & 1;
    rotate = true;
  } else if (r < rows_per_token) {
    const bool is_v = r - Hq >= Hkv;
    const int g = is_v ? r - Hq - Hkv : r - Hq;
    const int col = t / a.page_size;
    const int page = col < a.max_pages_per_seq
                         ? a.block_table[(size_t)b * a.max_pages_per_seq + col]
                         : -1;
    if ((unsigned)page < (unsigned)a.num_pages) {
      const size_t slot =
          (((size_t)page * Hkv + g) * a.page_size + (t - col * a.page_size)) * D;
      dst = (is_v ? a.v_pool : a.k_pool) + slot;
      src = (is_v ? a.v_new : a.k_new) + ((size_t)tok * Hkv + g) * D;
      weight = is_v ? a.v_weight : a.k_weight;
      norm = is_v ? (a.norm_flags & 2) : (a.norm_flags & 1);
      rotate = !is_v;
    }
  }
  const bool active = dst != nullptr;  // the same for the whole wave

  float x[E];
  if (active) {
    const vec_t raw = reinterpret_cast<const vec_t*>(src)[lane];
#pragma unroll
    for (int e = 0; e < E; e += 2) {
      const uint32_t w2 = raw[e / 2];
      x[e] = __builtin_bit_cast(float, w2 << 16);
      x[e + 1] = __builtin_bit_cast(float, w2 & 0xFFFF0000u);
    }
    if (norm) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) ss += x[e] * x[e];
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) ss += __shfl_xor(ss, m);
      const float inv = 1.0f / sqrtf(ss * (1.0f / D) + a.eps);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        x[e] *= inv;
        if (weight) x[e] *= weight[lane * E + e];
      }
    }
  }

  const int R = a.rotary_dim;
  const int half = R / 2;
  const float* cs = a.cos_sin + (size_t)t * R;
  if (R > 0 && !a.interleaved) {
    // NeoX pairs (d, d + R/2): the partner sits in another lane, so the row goes through LDS.
    if (active && rotate) {
#pragma unroll
      for (int e = 0; e < E; ++e) rows[wave][lane * E + e] = x[e];
    }
    __syncthreads();
    if (active && rotate) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int d = lane * E + e;
        if (d < R) {
          const bool lo = d < half;
          const int j = lo ? d : d - half;
          const float p = rows[wave][lo ? d + half : j];
          const float c = cs[j], s = cs[half + j];
          x[e] = lo ? x[e] * c - p * s : x[e] * c + p * s;
        }
      }
    }
  } else if (R > 0 && active && rotate) {
    // GPT-J pairs (2j, 2j + 1): both elements are in this lane (E is even).
#pragma unroll
    for (int e = 0; e < E; e += 2) {
      const int d = lane * E + e;
      if (d < R) {
        const int j = d / 2;
        const float c = cs[j], s = cs[half + j];
        const float x1 = x[e], x2 = x[e + 1];
        x[e] = x1 * c - x2 * s;
        x[e + 1] = x2 * c + x1 * s;
      }
    }
  }

  if (active) {
    vec_t out;
#pragma unroll
    for (int e = 0; e < E; e += 2) out[e / 2] = pack_bf16x2(x[e], x[e + 1]);
    reinterpret_cast<vec_t*>(dst)[lane] = out;
  }
}

}  // namespace

hipError_t launch_rope_cache(float* cos_sin, int max_position, int rotary_dim, int freq_dim,
                             double theta, hipStream_t stream) {
  const int64_t count = (int64_t)max_position * (rotary_dim / 2);
  const int64_t blocks = (count + 255) / 256;
  dim3 grid((unsigned)(blocks < 65536 ? blocks : 65536));
  void* kargs[] = {&cos_sin, const_cast<int64_t*>(&count), &rotary_dim, &freq_dim, &theta};
  return hipLaunchKernel(reinterpret_cast<const void*>(&rope_cache_kernel), grid, dim3(256),
                         kargs, 0, stream);
}

hipError_t launch_append_rope(const AppendRopeArgs& args, int head_dim, int batch,
                              hipStream_t stream) {
  const int rows = args.num_q_heads + args.num_kv_heads * (args.v_pool == args.k_pool ? 1 : 2);
  dim3 grid(batch * args.q_len, (rows + kRopeWaves - 1) / kRopeWaves);
  dim3 block(64 * kRopeWaves);
  void* kargs[] = {const_cast<AppendRopeArgs*>(&args)};
  const void* fn = head_dim == 512 ? reinterpret_cast<const void*>(&append_rope_kernel<512>)
                                   : reinterpret_cast<const void*>(&append_rope_kernel<256>);
  return hipLaunchKernel(fn, grid, block, kargs, 0, stream);
}

}  // namespace decode_attn
