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
// Layout of the work: a row is a q head, a new k head or a new v head of one new token; a wave
// takes four consecutive rows (a row group) of a token, four waves per workgroup. Each lane holds D / 64 consecutive elements of a row (one 16-byte load at D = 512,
// 8 bytes at D = 256), so a row is one coalesced read and one coalesced write, and a wave keeps
// four rows' loads in flight at once. The RMS is a wave reduction; the NeoX pair partner (element
// d +- R/2, held by another lane) comes through the wave's LDS rows, the interleaved partner is in
// the same lane. Arithmetic is fp32 and each result is rounded once to
// bf16 (nearest even). The rotation table (cos and sin per position and pair, fp32) is built
// once per layer configuration by rope_cache_kernel in double precision.

#include <hip/hip_runtime.h>

#include "device_common.h"
#include "internal.h"

namespace decode_attn {
namespace {

constexpr int kRopeWaves = 4;
// Rows per wave (D = 512, D = 256), and whether rows are read and written with the non-temporal
// hint (each row is touched once); build knobs for A/B runs, defaults measured on MI355X.
#ifndef DECODE_ATTN_ROPE_RW
#define DECODE_ATTN_ROPE_RW 4
#endif
#ifndef DECODE_ATTN_ROPE_RW256
#define DECODE_ATTN_ROPE_RW256 DECODE_ATTN_ROPE_RW
#endif
#ifndef DECODE_ATTN_ROPE_NT
#define DECODE_ATTN_ROPE_NT 1
#endif
constexpr int kRopeRowsPerWave = DECODE_ATTN_ROPE_RW;      // D = 512
constexpr int kRopeRowsPerWave256 = DECODE_ATTN_ROPE_RW256;  // D = 256

template <typename T>
__device__ __forceinline__ T load_row(const T* p) {
  if constexpr (DECODE_ATTN_ROPE_NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <typename T>
__device__ __forceinline__ void store_row(T v, T* p) {
  if constexpr (DECODE_ATTN_ROPE_NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

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

// The lane's E consecutive floats of p (all 1 when p is NULL). FAST: p + lane * E is 16-byte
// aligned and the values come in as vector loads.
template <int N>
__device__ __forceinline__ void load_floats(const float* p, float* v) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int n = 0; n < N; n += 4) {
      const f32x4 w = *reinterpret_cast<const f32x4*>(p + n);
      v[n] = w[0];
      v[n + 1] = w[1];
      v[n + 2] = w[2];
      v[n + 3] = w[3];
    }
  } else {
    static_assert(N == 2, "two or a multiple of four floats");
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const f32x2 w = *reinterpret_cast<const f32x2*>(p);
    v[0] = w[0];
    v[1] = w[1];
  }
}

template <int E, bool FAST>
__device__ __forceinline__ void load_weights(const float* w, int lane, float* v) {
  if (!w) {
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = 1.f;
  } else if (FAST) {
    load_floats<E>(w + lane * E, v);
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = w[lane * E + e];
  }
}

// Where a row comes from and goes to. kind -1: past the token's rows (nothing to do). The source
// does not depend on the block table, so the row loads are issued before the page id arrives; a
// k/v row whose slot is skipped gets no destination.
struct RowRef {
  const uint16_t* src;
  uint16_t* dst;
  int kind;  // 0 = q head, 1 = new k head, 2 = new v head
};

__device__ __forceinline__ RowRef row_src(const AppendRopeArgs& a, int r, int tok,
                                          int rows_per_token, int D) {
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  RowRef ref{nullptr, nullptr, -1};
  if (r < Hq) {
    ref.src = a.q + ((size_t)tok * Hq + r) * D;
    ref.dst = a.q_out + ((size_t)tok * Hq + r) * D;
    ref.kind = 0;
  } else if (r < rows_per_token) {
    const bool is_v = r - Hq >= Hkv;
    const int g = is_v ? r - Hq - Hkv : r - Hq;
    ref.src = (is_v ? a.v_new : a.k_new) + ((size_t)tok * Hkv + g) * D;
    ref.kind = is_v ? 2 : 1;
  }
  return ref;
}

// Destination of k/v row r in page `page` (the token's slot t % S), or none for an invalid page.
__device__ __forceinline__ void row_dst(const AppendRopeArgs& a, RowRef& ref, int r, int page,
                                        int slot, int D) {
  if (ref.kind < 1 || (unsigned)page >= (unsigned)a.num_pages) return;
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const int g = ref.kind == 2 ? r - Hq - Hkv : r - Hq;
  ref.dst = (ref.kind == 2 ? a.v_pool : a.k_pool) +
            (((size_t)page * Hkv + g) * a.page_size + slot) * D;
}

// Wave w of a workgroup takes RW consecutive rows of one token. With `flat` 0 the grid is
// (token, slice of its rows); with `flat` 1 (FAST path only, used when a token's row groups do
// not fill whole workgroups) global wave gw takes row group gw % wpt of token gw / wpt, so that
// no wave slot idles. Either way workgroups of consecutive tokens are dispatched one after
// another and the launch streams through q, k_new and v_new in address order. Every global load
// of a wave (its RW rows, the norm weights, its lanes' cos and sin) is issued before any result
// is needed, so one memory latency covers the wave's work; the row loads and stores carry the
// non-temporal hint, as each row is touched once.
//
// FAST (chosen on the host when R is a multiple of 2 * D / 64 and the table and weights are
// 16-byte aligned): a lane's elements are all rotated or all not, and for NeoX all on one side of
// R/2, so the lane's weights and cos / sin come in as vector loads and the NeoX partner is the
// same element of lane +- R / (2 E), fetched with a cross-lane permute (no LDS, no barrier).
// Otherwise the general path: per-element table loads and the partner through LDS.
template <int D, int RW, int MODE>
__global__ __launch_bounds__(64 * kRopeWaves)
void append_rope_kernel(const AppendRopeArgs a, int tokens, int flat) {
  constexpr bool FAST = MODE != 0;
  constexpr int E = D / 64;
  typedef typename RowVec<E>::type vec_t;
  __shared__ float rows[FAST ? 1 : kRopeWaves][FAST ? 1 : RW][FAST ? 1 : D];

  const int lane = threadIdx.x & 63;
  // The wave index is the same in all lanes; readfirstlane lets the row bookkeeping below stay in
  // scalar registers and scalar branches.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool same = a.v_pool == a.k_pool;
  const int rows_per_token = a.num_q_heads + a.num_kv_heads * (same ? 1 : 2);
  int tok, r0;  // this wave's token (b * L + i) and first row
  if (FAST && flat) {
    // Flat: global wave gw takes row group gw % wpt of token gw / wpt (workgroups span tokens).
    const int wpt = (rows_per_token + RW - 1) / RW;
    const int64_t gw = (int64_t)blockIdx.x * kRopeWaves + wave;
    tok = (int)(gw / wpt);
    r0 = (int)(gw - (int64_t)tok * wpt) * RW;
  } else {
    tok = blockIdx.x;
    r0 = (blockIdx.y * kRopeWaves + wave) * RW;
  }
  const int b = (tok < tokens ? tok : 0) / a.q_len;
  const int i = (tok < tokens ? tok : 0) - b * a.q_len;
  const int t = load_uniform(a.ctx_lens, b) - a.q_len + i;
  // A token at a skipped position, or a wave past the last token, has nothing to do. Without
  // `flat` this is the same for the whole workgroup; the flat layout is only used by the FAST
  // path, which has no barrier.
  if (tok >= tokens || t < 0 || t >= a.max_position) return;
  const int R = a.rotary_dim;
  const int half = R / 2;
  const bool interleaved = MODE == 0 ? a.interleaved != 0 : MODE == 2;

  RowRef ref[RW];
#pragma unroll
  for (int k = 0; k < RW; ++k) ref[k] = row_src(a, r0 + k, tok, rows_per_token, D);
  // All RW loads go out back to back; a row with nothing to do reads this token's first q head
  // (always in bounds) and its result is dropped.
  const uint16_t* const spare = a.q + (size_t)tok * a.num_q_heads * D;
  vec_t raw[RW];
#pragma unroll
  for (int k = 0; k < RW; ++k)
    raw[k] = load_row(reinterpret_cast<const vec_t*>(ref[k].kind >= 0 ? ref[k].src : spare) + lane);
  bool has_q = false, has_k = false, has_v = false;  // row kinds present in this wave
#pragma unroll
  for (int k = 0; k < RW; ++k) {
    has_q |= ref[k].kind == 0;
    has_k |= ref[k].kind == 1;
    has_v |= ref[k].kind == 2;
  }
  // The token's page (one block-table entry for all its k/v rows), read while the loads fly.
  if (has_k || has_v) {
    const int col = t / a.page_size;
    const int page = col < a.max_pages_per_seq
                         ? load_uniform(a.block_table, (size_t)b * a.max_pages_per_seq + col)
                         : -1;
#pragma unroll
    for (int k = 0; k < RW; ++k) row_dst(a, ref[k], r0 + k, page, t - col * a.page_size, D);
  }

  const bool norm_qk = a.norm_flags & 1, norm_v = a.norm_flags & 2;
  float wq[E], wk[E], wv[E], cv[E], sv[E];
  load_weights<E, FAST>((norm_qk && has_q) ? a.q_weight : nullptr, lane, wq);
  load_weights<E, FAST>((norm_qk && has_k) ? a.k_weight : nullptr, lane, wk);
  load_weights<E, FAST>((norm_v && has_v) ? a.v_weight : nullptr, lane, wv);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    cv[e] = 1.f;
    sv[e] = 0.f;
  }
  const bool rotates = R > 0 && (has_q || has_k);
  const float* cs = a.cos_sin + (size_t)t * R;
  const bool rot_lane = lane * E < R;  // FAST: all of the lane's elements rotate, or none
  if (FAST && rotates) {
    // Every lane loads (a lane past the rotated dims reads pair 0, in bounds, and drops it below),
    // so no lane waits at a branch for the others' loads.
    if constexpr (MODE == 2) {
      // pairs (2j, 2j + 1): the lane's E / 2 pairs start at j = lane * E / 2; cv / sv hold
      // one value per pair.
      const int j0 = rot_lane ? lane * E / 2 : 0;
      load_floats<E / 2>(cs + j0, cv);
      load_floats<E / 2>(cs + half + j0, sv);
    } else {
      const int j0 = !rot_lane ? 0 : lane * E < half ? lane * E : lane * E - half;
      load_floats<E>(cs + j0, cv);
      load_floats<E>(cs + half + j0, sv);
    }
  } else if (rotates) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      // Lanes past the rotated dims read pair 0 and keep the identity rotation.
      const int d = lane * E + e;
      const int j = d >= R ? 0 : interleaved ? d / 2 : (d < half ? d : d - half);
      const float c = cs[j], sn = cs[half + j];
      cv[e] = d < R ? c : 1.f;
      sv[e] = d < R ? sn : 0.f;
    }
  }

  float x[RW][E];
#pragma unroll
  for (int k = 0; k < RW; ++k) {
#pragma unroll
    for (int e = 0; e < E; e += 2) {
      const uint32_t w2 = raw[k][e / 2];
      x[k][e] = __builtin_bit_cast(float, w2 << 16);
      x[k][e + 1] = __builtin_bit_cast(float, w2 & 0xFFFF0000u);
    }
  }
  // RMSNorm: the RW rows' sums of squares reduce across the wave side by side.
  float ss[RW];
#pragma unroll
  for (int k = 0; k < RW; ++k) {
    ss[k] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) ss[k] += x[k][e] * x[k][e];
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
#pragma unroll
    for (int k = 0; k < RW; ++k) ss[k] += __shfl_xor(ss[k], m);
  }
#pragma unroll
  for (int k = 0; k < RW; ++k) {
    const int kind = ref[k].kind;
    if ((kind <= 1 && kind >= 0 && norm_qk) || (kind == 2 && norm_v)) {
      const float inv = 1.0f / sqrtf(ss[k] * (1.0f / D) + a.eps);
#pragma unroll
      for (int e = 0; e < E; ++e)
        x[k][e] = x[k][e] * inv * (kind == 0 ? wq[e] : kind == 1 ? wk[e] : wv[e]);
    }
  }

  if (FAST && rotates) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      cv[e] = rot_lane ? cv[e] : 1.f;
      sv[e] = rot_lane ? sv[e] : 0.f;
    }
  }
  if (FAST && R > 0 && !interleaved) {
    // NeoX pairs (d, d + R/2): element e of lane l pairs with element e of lane l +- R / (2E).
    const int off = half / E;
    const bool lo = lane * E < half;
    const int partner = lane * E >= R ? lane : lo ? lane + off : lane - off;
    const float sign = lo ? -1.f : 1.f;
#pragma unroll
    for (int k = 0; k < RW; ++k)
      if (ref[k].kind == 0 || ref[k].kind == 1) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float p = __shfl(x[k][e], partner);
          x[k][e] = x[k][e] * cv[e] + sign * (p * sv[e]);
        }
      }
  } else if (R > 0 && !interleaved) {
    // NeoX pairs (d, d + R/2): the partner sits in another lane, so the rows go through LDS.
#pragma unroll
    for (int k = 0; k < RW; ++k)
      if (ref[k].kind == 0 || ref[k].kind == 1) {
#pragma unroll
        for (int e = 0; e < E; ++e) rows[wave][k][lane * E + e] = x[k][e];
      }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < RW; ++k)
      if (ref[k].kind == 0 || ref[k].kind == 1) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int d = lane * E + e;
          if (d < R) {
            const bool lo = d < half;
            const float p = rows[wave][k][lo ? d + half : d - half];
            x[k][e] = lo ? x[k][e] * cv[e] - p * sv[e] : x[k][e] * cv[e] + p * sv[e];
          }
        }
      }
  } else if (R > 0) {
    // GPT-J pairs (2j, 2j + 1): both elements are in this lane (E is even).
#pragma unroll
    for (int k = 0; k < RW; ++k)
      if (ref[k].kind == 0 || ref[k].kind == 1) {
#pragma unroll
        for (int e = 0; e < E; e += 2) {
          const int j = MODE == 2 ? e / 2 : e;  // where this pair's cos / sin sit
          const float x1 = x[k][e], x2 = x[k][e + 1];
          x[k][e] = x1 * cv[j] - x2 * sv[j];
          x[k][e + 1] = x2 * cv[j] + x1 * sv[j];
        }
      }
  }

#pragma unroll
  for (int k = 0; k < RW; ++k) {
    if (ref[k].kind < 0 || ref[k].dst == nullptr) continue;
    vec_t out;
#pragma unroll
    for (int e = 0; e < E; e += 2) out[e / 2] = pack_bf16x2(x[k][e], x[k][e + 1]);
    store_row(out, reinterpret_cast<vec_t*>(ref[k].dst) + lane);
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
  const auto a16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  const bool fast = args.rotary_dim % (2 * (head_dim / 64)) == 0 && a16(args.cos_sin) &&
                    a16(args.q_weight) && a16(args.k_weight) && a16(args.v_weight);
  int tokens = batch * args.q_len;
  const int rw = head_dim == 512 ? kRopeRowsPerWave : kRopeRowsPerWave256;
  const int row_waves = (rows + rw - 1) / rw;
  // When a token's row groups fill whole workgroups, the 2D grid (token, slice); otherwise the
  // FAST path deals the row groups out flat so that no wave slot idles (20 rows at D = 512: the
  // 2D grid would launch 8 waves per token for 5 row groups). Where both fit, the 2D grid
  // measured faster: dealt flat, 8 row groups per token put every token's q rows on even XCDs and
  // its k/v rows on odd ones (workgroups go to the XCDs round robin).
  int flat = fast && row_waves % kRopeWaves != 0;
  dim3 grid(tokens, (row_waves + kRopeWaves - 1) / kRopeWaves);
  if (flat) {
    const int64_t blocks = ((int64_t)tokens * row_waves + kRopeWaves - 1) / kRopeWaves;
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    grid = dim3((unsigned)blocks);
  }
  dim3 block(64 * kRopeWaves);
  void* kargs[] = {const_cast<AppendRopeArgs*>(&args), &tokens, &flat};
  constexpr int RW = kRopeRowsPerWave, RW2 = kRopeRowsPerWave256;
  // 0: general path; 1: FAST, NeoX pairs; 2: FAST, interleaved pairs.
  const int mode = fast ? (args.interleaved ? 2 : 1) : 0;
  const void* const kernels[2][3] = {
      {reinterpret_cast<const void*>(&append_rope_kernel<256, RW2, 0>),
       reinterpret_cast<const void*>(&append_rope_kernel<256, RW2, 1>),
       reinterpret_cast<const void*>(&append_rope_kernel<256, RW2, 2>)},
      {reinterpret_cast<const void*>(&append_rope_kernel<512, RW, 0>),
       reinterpret_cast<const void*>(&append_rope_kernel<512, RW, 1>),
       reinterpret_cast<const void*>(&append_rope_kernel<512, RW, 2>)}};
  const void* fn = kernels[head_dim == 512 ? 1 : 0][mode];
  return hipLaunchKernel(fn, grid, block, kargs, 0, stream);
}

}  // namespace decode_attn
