// stage1.hip — split-KV stage 1 of paged GQA decode attention for gfx950 (CDNA4).
//
// One workgroup per (split, kv head, sequence) reads the keys of its chunk once and serves every
// query head of the GQA group with them (several query heads sharing a KV head are handled by
// one program: Sparse-vLLM PR #27 "feat: support Gemma 4 and native multimodal inference",
// section "专用算子与性能优化"). It writes the chunk's softmax-normalised partial output and its
// log-sum-exp, the split-KV partial buffer of vLLM learning notes "模型库与算子层 — 概念",
// section "MLA 与 Sparse MLA（DSA）".
//
// Work decomposition inside a workgroup (4 wavefronts of 64 lanes):
//   * keys are processed in tiles of 16 (a page of 16 keys, or a 16-key slice of a larger page);
//     wave w takes tiles w, w+4, ... of the chunk and keeps its own running max / sum / output;
//   * scores: one v_mfma_f32_16x16x32_bf16 per 32 values of d, A = K tile (16 keys x 32 d, each
//     lane loads 16 contiguous bytes of one key row straight from HBM), B = q group (32 d x 16
//     heads, heads >= G zero), read from LDS where the workgroup stored it once;
//     lane l receives the scores of keys 4*(l/16)..+3 for head l%16;
//   * softmax: masked keys get -inf by select (never by multiplying a mask, so NaN in unused
//     slots cannot leak), running max and sum per head in base-2 units with hardware exp2;
//   * P.V on the vector ALUs: each V row is read with one coalesced 16-byte load per lane (lane l
//     owns 8 consecutive d), the probabilities of the tile are broadcast through LDS;
//   * at the end the 4 waves' states are merged in LDS in a fixed order (deterministic).
// Loads of the next tile are issued as soon as the registers of the current one are consumed
// (K right after the MFMAs, V right after the P.V update), so one tile half is always in flight.

#include <hip/hip_runtime.h>

#include "internal.h"

namespace decode_attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = kStage1Threads / 64;
constexpr float kLn2 = 0.693147180559945309417f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Read-only kernel inputs (block table, context lengths) are read through the constant address
// space so uniform indices become scalar loads that do not share the vector-memory counter.
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;

__device__ __forceinline__ int32_t load_uniform(const int32_t* p, size_t idx) {
  return ((const_i32_ptr)(p))[idx];
}

// Orders LDS accesses of one wavefront for the compiler; the hardware executes a wave's LDS
// instructions in issue order, so no wait is needed between lanes of the same wave.
__device__ __forceinline__ void wave_lds_order() { __asm__ volatile("" ::: "memory"); }

template <int D, int G>
struct Stage1Shape {
  static_assert(D == 256 || D == 512, "head_dim");
  static_assert(G >= 1 && G <= 16, "group size");
  static constexpr int kSteps = D / 32;                   // MFMA steps over d per tile
  static constexpr int kLanesPerRow = D / 8;              // lanes covering one V row (16 B each)
  static constexpr int kRowsPerLoad = 64 / kLanesPerRow;  // V rows per wave-wide load
  static constexpr int kVLoads = kTile / kRowsPerLoad;    // V loads per tile
  static constexpr int kHeadChunk = (D == 512) ? (G < 4 ? G : 4) : (G < 8 ? G : 8);
  // LDS: q operand + per-wave probability tiles during the key loop; merge slices afterwards.
  static constexpr int kQBytes = kSteps * 64 * 16;
  static constexpr int kPRowFloats = 16;                  // one row per key of the tile
  static constexpr int kPBytes = kWaves * (kTile + 1) * kPRowFloats * 4;  // + alpha row
  static constexpr int kMergeBytes = kWaves * kHeadChunk * D * 4;
  static constexpr int kLoopBytes = kQBytes + kPBytes;
  static constexpr int kUnionBytes = kLoopBytes > kMergeBytes ? kLoopBytes : kMergeBytes;
};

// acc[h][:] += p[h][key] * V[key][lane's 8 d] for the keys of one tile. MASKED: keys outside
// [key_lo, key_hi) have V replaced by 0 (their p is already 0; 0 * NaN would not be).
template <int D, int G, bool MASKED>
__device__ __forceinline__ void pv_update(float (&acc)[G][8],
                                          const u32x4 (&vreg)[Stage1Shape<D, G>::kVLoads],
                                          const float* p_lds, int v_row, int tok0, int key_lo,
                                          int key_hi) {
  using Sh = Stage1Shape<D, G>;
#pragma unroll
  for (int i = 0; i < Sh::kVLoads; ++i) {
    const int kr = i * Sh::kRowsPerLoad + v_row;
    float pv[G];
#pragma unroll
    for (int h = 0; h < G; ++h) pv[h] = p_lds[kr * 16 + h];
    const u32x4 w = vreg[i];
    float v[8] = {bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1]),
                  bf16_lo(w[2]), bf16_hi(w[2]), bf16_lo(w[3]), bf16_hi(w[3])};
    if (MASKED) {
      const int t = tok0 + kr;
      const bool valid = t >= key_lo && t < key_hi;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = valid ? v[e] : 0.f;
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pv[h], v[e], acc[h][e]);
    // Keep the scheduler from hoisting every row's reads and conversions at once.
    if ((i & 3) == 3) __builtin_amdgcn_sched_barrier(0);
  }
}

template <int D, int G>
__global__ __launch_bounds__(kStage1Threads) void stage1_kernel(const Stage1Args a) {
  using Sh = Stage1Shape<D, G>;
  constexpr int kSteps = Sh::kSteps;
  constexpr int kVLoads = Sh::kVLoads;
  constexpr int kRowsPerLoad = Sh::kRowsPerLoad;
  constexpr int kLanesPerRow = Sh::kLanesPerRow;
  constexpr int kHC = Sh::kHeadChunk;

  __shared__ __attribute__((aligned(16))) float ml_lds[kWaves][16][2];
  __shared__ __attribute__((aligned(16))) unsigned char smem[Sh::kUnionBytes];
  u32x4* q_lds = reinterpret_cast<u32x4*>(smem);
  float* p_lds_all = reinterpret_cast<float*>(smem + Sh::kQBytes);
  float* merge_lds = reinterpret_cast<float*>(smem);

  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int S = a.page_size;
  const int Hkv = a.num_kv_heads;
  const int ns = a.num_splits;

  // Key range of this sequence and the tiles of this split.
  const int max_keys = a.max_pages_per_seq * S;
  int n = load_uniform(a.ctx_lens, b);
  n = n < 0 ? 0 : (n > max_keys ? max_keys : n);
  const int lo = (a.window > 0 && n > a.window) ? n - a.window : 0;
  const int tile_lo = lo / kTile;
  const int tile_hi = (n + kTile - 1) / kTile;
  const int T = tile_hi > tile_lo ? tile_hi - tile_lo : 0;
  const int t_begin = tile_lo + (int)(((int64_t)split * T) / ns);
  const int t_end = tile_lo + (int)(((int64_t)(split + 1) * T) / ns);
  const int tiles_per_page = S / kTile;

  // q group -> LDS in MFMA B-operand order: entry (j, l) = q[h = l%16][j*32 + (l/16)*8 .. +8].
  const uint16_t* qg = a.q + ((size_t)b * a.num_q_heads + (size_t)kvh * G) * D;
  for (int idx = threadIdx.x; idx < kSteps * 64; idx += kStage1Threads) {
    const int j = idx >> 6, l = idx & 63, h = l & 15;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (h < G) v = *reinterpret_cast<const u32x4*>(qg + h * D + j * 32 + (l >> 4) * 8);
    q_lds[idx] = v;
  }
  __syncthreads();

  float* p_lds = p_lds_all + wave * (kTile + 1) * Sh::kPRowFloats;
  const bf16x8* q_op = reinterpret_cast<const bf16x8*>(q_lds) + lane;

  // Per-lane pointers inside a 16-key tile (element offsets from the tile base).
  const int k_lane_off = (lane & 15) * D + (lane >> 4) * 8;
  const int v_row = lane / kLanesPerRow;
  const int v_lane_off = v_row * D + (lane % kLanesPerRow) * 8;

  float m_run = -INFINITY;  // running max (base-2 units) of head lane%16
  float l_run = 0.f;        // running sum of exp2(s - m_run) of head lane%16
  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;

  bf16x8 kreg[kSteps];
  u32x4 vreg[kVLoads];

  // Tile -> (element offset of the tile in the pools, page valid).
  auto tile_base = [&](int ti, bool& ok) -> size_t {
    const int col = ti / tiles_per_page;
    int phys = load_uniform(a.block_table, (size_t)b * a.max_pages_per_seq + col);
    ok = (unsigned)phys < (unsigned)a.num_pages;
    phys = ok ? phys : 0;  // never dereference an invalid id; the tile is masked instead
    const int off = (ti - col * tiles_per_page) * kTile;
    return (((size_t)phys * Hkv + kvh) * S + off) * D;
  };

  int ti = t_begin + wave;
  bool ok = false;
  size_t base = 0;
  if (ti < t_end) {
    base = tile_base(ti, ok);
    const uint16_t* kp = a.k_pool + base + k_lane_off;
    const uint16_t* vp = a.v_pool + base + v_lane_off;
#pragma unroll
    for (int j = 0; j < kSteps; ++j) kreg[j] = *reinterpret_cast<const bf16x8*>(kp + j * 32);
#pragma unroll
    for (int i = 0; i < kVLoads; ++i)
      vreg[i] = *reinterpret_cast<const u32x4*>(vp + (size_t)i * kRowsPerLoad * D);
  }

  while (ti < t_end) {
    // Scores of the 16 keys for the 16 (padded) heads; two accumulators shorten the chain.
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kSteps; j += 2) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kreg[j], q_op[j * 64], s0, 0, 0, 0);
      if (j + 1 < kSteps)
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kreg[j + 1], q_op[(j + 1) * 64], s1, 0, 0, 0);
    }

    const int tn = ti + kWaves;
    const bool has_next = tn < t_end;
    bool ok_next = false;
    size_t base_next = 0;
    if (has_next) {
      base_next = tile_base(tn, ok_next);
      const uint16_t* kp = a.k_pool + base_next + k_lane_off;
#pragma unroll
      for (int j = 0; j < kSteps; ++j) kreg[j] = *reinterpret_cast<const bf16x8*>(kp + j * 32);
    }

    // Mask and online softmax for head lane%16.
    const int tok0 = ti * kTile;
    const int key_lo = ok ? (lo > tok0 ? lo : tok0) : tok0;
    const int key_hi = ok ? (n < tok0 + kTile ? n : tok0 + kTile) : tok0;
    const bool full = key_lo == tok0 && key_hi == tok0 + kTile;
    float sc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = tok0 + 4 * (lane >> 4) + r;
      const float raw = s0[r] + s1[r];
      sc[r] = (t >= key_lo && t < key_hi) ? raw * a.scale_log2 : -INFINITY;
    }
    float mt = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(sc[r] - m_use);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float ps = (p[0] + p[1]) + (p[2] + p[3]);
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    l_run = l_run * alpha + ps;
    m_run = m_new;

    // Broadcast the probabilities (key-major, 16 heads per row) and the rescale factors.
#pragma unroll
    for (int r = 0; r < 4; ++r) p_lds[(4 * (lane >> 4) + r) * 16 + (lane & 15)] = p[r];
    if (lane < 16) p_lds[kTile * 16 + lane] = alpha;
    wave_lds_order();

    if (__any(lane < G && alpha != 1.f)) {  // skip when no running max moved
      float al[G];
#pragma unroll
      for (int h = 0; h < G; ++h) al[h] = p_lds[kTile * 16 + h];
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= al[h];
    }

    // P.V: lane owns d = (lane % kLanesPerRow)*8 .. +8 of key row i*kRowsPerLoad + v_row.
    if (full)
      pv_update<D, G, false>(acc, vreg, p_lds, v_row, 0, 0, 0);
    else
      pv_update<D, G, true>(acc, vreg, p_lds, v_row, tok0, key_lo, key_hi);
    wave_lds_order();

    if (has_next) {
      const uint16_t* vp = a.v_pool + base_next + v_lane_off;
#pragma unroll
      for (int i = 0; i < kVLoads; ++i)
        vreg[i] = *reinterpret_cast<const u32x4*>(vp + (size_t)i * kRowsPerLoad * D);
    }
    ti = tn;
    ok = ok_next;
    base = base_next;
  }
  (void)base;

  // Lanes that covered different key rows of the same d fold their sums (same running max).
#pragma unroll
  for (int step = kLanesPerRow; step < 64; step *= 2)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] += __shfl_xor(acc[h][e], step);

  if (lane < 16) {
    ml_lds[wave][lane][0] = m_run;
    ml_lds[wave][lane][1] = l_run;
  }
  __syncthreads();  // ml visible; q/p regions free for the merge slices

  // Per head: overall max M, overall sum L, and this wave's weight exp2(m_w - M) / L.
  const size_t row0 = (size_t)b * a.num_q_heads + (size_t)kvh * G;
  float* o_dst = a.o_part;
#pragma unroll
  for (int hc = 0; hc < G; hc += kHC) {
#pragma unroll
    for (int hh = 0; hh < kHC; ++hh) {
      const int h = hc + hh;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, ml_lds[w][h][0]);
      float L = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = ml_lds[w][h][0];
        L += (mw == -INFINITY) ? 0.f : ml_lds[w][h][1] * __builtin_amdgcn_exp2f(mw - M);
      }
      const float mine = ml_lds[wave][h][0];
      const float f = (mine == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mine - M) / L;
      if (lane < kLanesPerRow) {
        float* dst = merge_lds + ((wave * kHC + hh) * D + lane * 8);
        f32x4 lo4 = {acc[h][0] * f, acc[h][1] * f, acc[h][2] * f, acc[h][3] * f};
        f32x4 hi4 = {acc[h][4] * f, acc[h][5] * f, acc[h][6] * f, acc[h][7] * f};
        *reinterpret_cast<f32x4*>(dst) = lo4;
        *reinterpret_cast<f32x4*>(dst + 4) = hi4;
      }
      if (threadIdx.x == 0) {
        const float lse = (M == -INFINITY) ? -INFINITY : (M + __log2f(L)) * kLn2;
        a.lse_part[(row0 + h) * ns + split] = lse;
      }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < kHC * D; idx += kStage1Threads) {
      const int hh = idx / D, d = idx - hh * D;
      float o = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) o += merge_lds[(w * kHC + hh) * D + d];
      o_dst[((row0 + hc + hh) * ns + split) * D + d] = o;
    }
    __syncthreads();
  }
}

template <int D, int G>
hipError_t launch(const Stage1Args& args, int batch, hipStream_t stream) {
  dim3 grid(args.num_splits, args.num_kv_heads, batch);
  dim3 block(kStage1Threads);
  void* kargs[] = {const_cast<Stage1Args*>(&args)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&stage1_kernel<D, G>), grid, block, kargs,
                         0, stream);
}

template <int D>
hipError_t launch_d(const Stage1Args& args, int group_size, int batch, hipStream_t stream) {
  switch (group_size) {
    case 1: return launch<D, 1>(args, batch, stream);
    case 2: return launch<D, 2>(args, batch, stream);
    case 4: return launch<D, 4>(args, batch, stream);
    case 8: return launch<D, 8>(args, batch, stream);
    case 16: return launch<D, 16>(args, batch, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool stage1_supported(int head_dim, int group_size) {
  const bool d_ok = head_dim == 256 || head_dim == 512;
  const bool g_ok = group_size == 1 || group_size == 2 || group_size == 4 || group_size == 8 ||
                    group_size == 16;
  return d_ok && g_ok;
}

hipError_t launch_stage1(const Stage1Args& args, int head_dim, int group_size, int batch,
                         hipStream_t stream) {
  switch (head_dim) {
    case 256: return launch_d<256>(args, group_size, batch, stream);
    case 512: return launch_d<512>(args, group_size, batch, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace decode_attn
