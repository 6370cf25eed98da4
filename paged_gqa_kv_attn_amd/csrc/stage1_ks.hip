// stage1_ks.hip — split-KV stage 1 of single-token decode for head_dim 256 with small query-head
// groups (the sliding-window layers of Sparse-vLLM PR #27 "feat: support Gemma 4 and native
// multimodal inference", sections "Gemma 4 文本推理" and "专用算子与性能优化": a smaller head dim
// than the global layers, and a grouped sliding decode kernel), used when the batch's (sequence,
// kv head) pairs alone fill the GPU and the plan has one chunk per pair. Writes the same partials
// as stage1.hip (vLLM learning notes "模型库与算子层 — 概念", section "MLA 与 Sparse MLA（DSA）").
//
// Work decomposition: one workgroup of NW wavefronts (8) per (split, kv head, sequence). The waves
// split the chunk's 16-key tiles between them (wave w takes tiles w, w + NW, ...), and each wave
// covers the whole head dim, so a tile's scores, softmax and P.V stay inside one wave: no per-tile
// score exchange and no per-tile barrier. The waves' softmax states are merged once, through LDS,
// when the chunk is done. A tile of one (page, kv head) is 16 x 256 bf16 = 8 KB contiguous; each
// wave keeps one tile of K and V in flight while it computes the previous one, so a workgroup has
// NW tiles in flight (the column-split kernel of stage1.hip has one per workgroup). As there,
// the page ids of the chunk the plan's expected length gives are fetched while the sequence's
// length is in flight, and kept when the length gives the same chunk.
//
//   * K: loaded in row order (load j brings keys 2j, 2j + 1: 1 KB, whole 128-byte lines), parked in
//     the wave's LDS slice and read back in the A layout of v_mfma_f32_16x16x32_bf16 (lane l: key
//     l % 16, dims 32k + 8(l / 16) .. + 8 for k-step k). B is the q group (dims x 16 columns, one per
//     query head, columns >= G zero), held in registers. Lane l gets the scores of keys
//     4(l / 16) .. + 3 for head l % 16.
//   * softmax: masked keys get -inf by select; running max and sum per head in base-2 units; the
//     four lanes of a head combine with row-half swaps.
//   * P.V: v_mfma_f32_16x16x16_bf16 with A = P (exactly the score layout, rounded to bf16) and
//     B = V. V is loaded so that lane l holds, for keys 4(l / 16) + i, the dims 8(l % 16) .. + 8 and
//     128 + 8(l % 16) .. + 8 (each load instruction: four keys x 256 contiguous bytes), and is
//     transposed in the lane with byte permutes. MFMA e (16 of them) produces output dims
//     8n + e % 8 + 128 (e / 8) of column n = l % 16 for the four heads 4(l / 16) .. + 3.
// A build knob (DECODE_ATTN_KS_VALU) replaces both products by VALU dot products (bf16 pair dot
// products for the scores, fp32 FMAs for P.V, half-wave DPP sums): the A/B against MFMA on these
// G <= 4 groups, where MFMA uses 2 of its 16 rows at G = 2.

#include <hip/hip_runtime.h>

#include "device_common.h"
#include "internal.h"

namespace decode_attn {
namespace {

#ifndef DECODE_ATTN_KS_VALU
#define DECODE_ATTN_KS_VALU 0
#endif
// Waves per workgroup (4, 8 or, for the VALU variant only, 16: at 16 waves a lane has 128
// registers).
#ifndef DECODE_ATTN_KS_WAVES
#define DECODE_ATTN_KS_WAVES 8
#endif

constexpr int kKsD = 256;

__device__ __forceinline__ void ks_fence() { __asm__ volatile("" ::: "memory"); }

// Tile geometry of one sequence for a decode query: keys [lo, n) as the tiles [w0, tile_hi).
struct KsRange {
  int n, lo, w0, T;
};

__device__ __forceinline__ KsRange ks_range(int n, int window) {
  KsRange r;
  r.n = n;
  r.lo = (window > 0 && n > window) ? n - window : 0;
  r.w0 = r.lo / kTile;
  const int tile_hi = (n + kTile - 1) / kTile;
  r.T = tile_hi > r.w0 ? tile_hi - r.w0 : 0;
  return r;
}

#ifndef DECODE_ATTN_KS_PAD
#define DECODE_ATTN_KS_PAD 8
#endif

// Page ids of this wave's tiles (list entries t0 + NW u for lane u) as a vector: lane u holds the
// id of the wave's u-th tile from t0 on, the last tile's id past the chunk (never used).
template <int NW>
__device__ __forceinline__ int32_t ks_page_ids(const int32_t* table_row, int w0, int t0,
                                               int t_last, int tiles_per_page, int lane) {
  int t = t0 + NW * lane;
  t = t < t_last ? t : t_last;
  return table_row[(w0 + t) / tiles_per_page];
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Sum of v over the 32 lanes of a half wave (lanes l and l ^ 1, ^ 2, ^ 4 .. ^ 16): quad
// permutes, the half-row and row mirrors, then the row-half swap (VALU only, no LDS).
[[maybe_unused]] __device__ __forceinline__ float ks_sum32(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1,
                                                             0xF, 0xF, false));  // [1,0,3,2]
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E,
                                                             0xF, 0xF, false));  // [2,3,0,1]
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141,
                                                             0xF, 0xF, false));  // half mirror
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140,
                                                             0xF, 0xF, false));  // row mirror
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// Combine a value with its copy in lane l ^ 32 (the other half wave).
[[maybe_unused]] __device__ __forceinline__ float ks_sum_halves(float v) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}
[[maybe_unused]] __device__ __forceinline__ float ks_max_halves(float v) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}

[[maybe_unused]] __device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
[[maybe_unused]] __device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __builtin_bit_cast(float, w & 0xFFFF0000u);
}

template <int G, int NW>
__global__ __launch_bounds__(64 * NW) void stage1_ks_kernel(const Stage1Args a) {
  constexpr int D = kKsD;
  constexpr int kKsWaves = NW;
  constexpr int kKsThreads = 64 * NW;
  constexpr bool kValu = DECODE_ATTN_KS_VALU != 0;
  constexpr int kKSteps = D / 32;   // score MFMAs per tile
  constexpr int kRow = D + DECODE_ATTN_KS_PAD;       // padded LDS row of a parked K tile (bf16)
  static_assert(G == 1 || G == 2 || G == 4, "group");
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[kValu ? 1 : NW][16][kRow];
  __shared__ __attribute__((aligned(16))) float o_lds[kKsWaves][G][D];
  __shared__ float m_lds[kKsWaves][G];
  __shared__ float l_lds[kKsWaves][G];

  const int ns = a.num_splits;
  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = lane >> 4;
  const int col = lane & 15;
  const int S = a.page_size;
  const int tiles_per_page = S / kTile;
  const int max_keys = a.max_pages_per_seq * S;
  const int32_t* table_row = a.block_table + (size_t)b * a.max_pages_per_seq;

  // Element offsets inside a tile. K in row order: load j brings keys 2j + lane / 32, dims
  // 8 (lane % 32). V: MFMA, load 2i + h brings key 4grp + i, dims 8col + 128h; VALU, row order
  // as K.
  const int k_off = 8 * lane;
  const int v_off = kValu ? 8 * lane : 4 * grp * D + 8 * col;
  auto v_elem = [&](int j) { return kValu ? 512 * j : (j >> 1) * D + 128 * (j & 1); };
  // Base of tile entry t (clamped to the chunk's last, t_end - 1) of the chunk whose tiles start
  // at physical tile w0, with its page id phys; ok = the id is a valid page.
  auto entry_base = [&](int w0, int t, int t_end_, int phys, bool& ok_) -> size_t {
    const int tc = t < t_end_ ? t : t_end_ - 1;
    const bool page_ok = (unsigned)phys < (unsigned)a.num_pages;
    ok_ = page_ok;
    const int pt = w0 + tc;
    const int within = pt - (pt / tiles_per_page) * tiles_per_page;
    return (((size_t)(page_ok ? phys : 0) * a.num_kv_heads + kvh) * S + within * kTile) * D;
  };
  u32x4 kr[8], vr[8];
  auto load_tile = [&](size_t base_) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      kr[j] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(a.k_pool + base_ + k_off + 512 * j));
#pragma unroll
    for (int j = 0; j < 8; ++j)
      vr[j] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(a.v_pool + base_ + v_off + v_elem(j)));
  };

  const size_t out_row0 = (size_t)b * a.num_q_heads + (size_t)kvh * G;
  // q of the group. MFMA: the B operand, column col is head kvh * G + col (zero for col >= G),
  // dims 32k + 8grp. VALU: every lane holds dims 8 (lane % 32) .. + 8 of each head, as bf16 pairs.
  bf16x8 qop[kValu ? 1 : kKSteps];
  u32x4 qv[kValu ? G : 1];
  if constexpr (kValu) {
#pragma unroll
    for (int h = 0; h < G; ++h)
      qv[h] = *reinterpret_cast<const u32x4*>(a.q + (out_row0 + h) * D + 8 * (lane & 31));
  } else {
    const uint16_t* qr = a.q + (out_row0 + (col < G ? col : 0)) * D;
#pragma unroll
    for (int k = 0; k < kKSteps; ++k) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qr + 32 * k + 8 * grp);
      const u32x4 z = {0u, 0u, 0u, 0u};
      qop[k] = __builtin_bit_cast(bf16x8, col < G ? v : z);
    }
  }
  // Speculative start: the page ids of the chunk this split would have at the plan's expected
  // length (a.spec_ctx) are fetched while ctx_lens is still in flight, and kept when the actual
  // length gives the same chunk (the first tile's fetch then leaves one memory round trip
  // earlier); otherwise they are fetched again.
  int n_ctx = load_uniform(a.ctx_lens, b);
  const int n_spec = a.spec_ctx < max_keys ? a.spec_ctx : max_keys;
  const KsRange Rs = ks_range(n_spec, a.window);
  const int ts_begin = (int)(((int64_t)split * Rs.T) / ns);
  const int ts_end = (int)(((int64_t)(split + 1) * Rs.T) / ns);
  const bool spec = n_spec > 0 && ts_begin < ts_end;
  int32_t pid_vec = 0;
  if (spec)
    pid_vec = ks_page_ids<NW>(table_row, Rs.w0, ts_begin + wave, ts_end - 1, tiles_per_page, lane);
  __asm__ volatile("; ks speculative loads issued" ::: "memory");

  n_ctx = n_ctx < 0 ? 0 : (n_ctx > max_keys ? max_keys : n_ctx);
  const KsRange R = ks_range(n_ctx, a.window);
  const int t_begin = (int)(((int64_t)split * R.T) / ns);
  const int t_end = (int)(((int64_t)(split + 1) * R.T) / ns);

  if (t_begin >= t_end) {  // empty split: o = 0, lse = -inf
    for (int idx = tid; idx < G * D; idx += kKsThreads)
      a.o_part[((out_row0 + idx / D) * ns + split) * D + idx % D] = 0.f;
    if (tid < G) a.lse_part[(out_row0 + tid) * ns + split] = -INFINITY;
    __builtin_amdgcn_s_waitcnt(0);  // the early loads land before the wave ends
    return;
  }
  const int t_last = t_end - 1;
  const int my_first = t_begin + wave;  // this wave's tiles: my_first + NW s < t_end
  const int my_count = my_first < t_end ? (t_end - my_first + kKsWaves - 1) / kKsWaves : 0;
  const bool hit = spec && Rs.w0 == R.w0 && ts_begin == t_begin && ts_end == t_end;
  if (!hit && my_count > 0)
    pid_vec = ks_page_ids<NW>(table_row, R.w0, my_first, t_last, tiles_per_page, lane);
  bool ok = false;
  size_t base = 0;
  if (my_count > 0) {
    base = entry_base(R.w0, my_first, t_end, __builtin_amdgcn_readlane(pid_vec, 0), ok);
    load_tile(base);
  }

  // MFMA: m_run / l_run of head col; acc[e][i]: head 4grp + i, dim 8col + e % 8 + 128 (e / 8).
  // VALU: mv / lv[h] of head h (the same in every lane); ov[h][e]: head h, dim 8 (lane % 32) + e,
  // over the keys of this half wave.
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc[kValu ? 1 : 16];
  float mv[G], lv[G], ov[kValu ? G : 1][8];
#pragma unroll
  for (int e = 0; e < (kValu ? 1 : 16); ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int h = 0; h < G; ++h) {
    mv[h] = -INFINITY;
    lv[h] = 0.f;
  }
#pragma unroll
  for (int h = 0; h < (kValu ? G : 1); ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) ov[h][e] = 0.f;

  if (my_count > 0) {
    auto tile_base = [&](int s, bool& ok_) -> size_t {
      return entry_base(R.w0, my_first + kKsWaves * s, t_end,
                        __builtin_amdgcn_readlane(pid_vec, s & 63), ok_);
    };
    __asm__ volatile("; ks prologue loads issued" ::: "memory");

    for (int s = 0; s < my_count; ++s) {
      const int tile = R.w0 + my_first + kKsWaves * s;  // physical 16-key tile of the sequence
      const bool ok_cur = ok;
      // Page ids of the next 64 tiles of this wave when this step uses the last of the vector.
      if ((s & 63) == 63 && s + 1 < my_count)
        pid_vec = ks_page_ids<NW>(table_row, R.w0, my_first + kKsWaves * (s + 1), t_last,
                              tiles_per_page, lane);
      const bool more = s + 1 < my_count;
      size_t base_n = base;
      bool ok_n = ok;

      if constexpr (kValu) {
        // Scores of keys 2j + lane / 32 for every head: partial dot products over this lane's 8
        // dims (bf16 pairs), summed over the half wave.
        float sc[8][G];
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int h = 0; h < G; ++h) {
            float d = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              // Element reads into plain values first: a bit cast of a vector element
              // subscript is compiled as element 0 by this compiler.
              const uint32_t kw = kr[j][w], qw = qv[h][w];
              d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kw),
                                                  __builtin_bit_cast(bf16x2, qw), d, false);
            }
            sc[j][h] = d;
          }
        __builtin_amdgcn_sched_barrier(0);
        if (more) {
          base_n = tile_base(s + 1, ok_n);
#pragma unroll
          for (int j = 0; j < 8; ++j)
            kr[j] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(a.k_pool + base_n + k_off + 512 * j));
        }
        __builtin_amdgcn_sched_barrier(0);
        const int tk = tile * kTile + (lane >> 5);  // key of j = 0; key 2j + lane / 32 in general
        float pr[8][G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float mt = -INFINITY;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int t = tk + 2 * j;
            const bool att = ok_cur & (t >= R.lo) & (t < R.n);
            const float full = ks_sum32(sc[j][h]);  // every lane of the half wave takes part
            sc[j][h] = att ? full * a.scale_log2 : -INFINITY;
            mt = fmaxf(mt, sc[j][h]);
          }
          mt = ks_max_halves(mt);
          const float m_new = fmaxf(mv[h], mt);
          const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
          const float alpha = __builtin_amdgcn_exp2f(mv[h] - m_use);
          float ps = 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            pr[j][h] = __builtin_amdgcn_exp2f(sc[j][h] - m_use);
            ps += pr[j][h];
          }
          lv[h] = lv[h] * alpha + ks_sum_halves(ps);
          mv[h] = m_new;
#pragma unroll
          for (int e = 0; e < 8; ++e) ov[h][e] *= alpha;
        }
        // P.V over this lane's 8 keys and 8 dims; keys outside [lo, n) or on an invalid page
        // contribute nothing (p is 0 and V is zeroed: 0 * NaN would not be).
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int t = tk + 2 * j;
          const bool valid = ok_cur & (t >= R.lo) & (t < R.n);
          float vf[8];
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t x = valid ? vr[j][w] : 0u;
            vf[2 * w] = bf16_lo(x);
            vf[2 * w + 1] = bf16_hi(x);
          }
#pragma unroll
          for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) ov[h][e] = fmaf(pr[j][h], vf[e], ov[h][e]);
        }
      } else {
        // Park K in row order, refill the registers with the next tile, read the A layout back.
#pragma unroll
        for (int j = 0; j < 8; ++j)
          *reinterpret_cast<u32x4*>(&k_lds[wave][2 * j + (lane >> 5)][8 * (lane & 31)]) = kr[j];
        ks_fence();
        __builtin_amdgcn_sched_barrier(0);
        if (more) {
          base_n = tile_base(s + 1, ok_n);
#pragma unroll
          for (int j = 0; j < 8; ++j)
            kr[j] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(a.k_pool + base_n + k_off + 512 * j));
        }
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 ka[kKSteps];
#pragma unroll
        for (int k = 0; k < kKSteps; ++k)
          ka[k] = *reinterpret_cast<const bf16x8*>(&k_lds[wave][col][32 * k + 8 * grp]);

        // Scores of keys 4grp + i of the tile for head col.
        f32x4 p0 = {0.f, 0.f, 0.f, 0.f}, p1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < kKSteps; k += 2) {
          p0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[k], qop[k], p0, 0, 0, 0);
          p1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[k + 1], qop[k + 1], p1, 0, 0, 0);
        }
        const f32x4 sc = p0 + p1;

        const int t0 = tile * kTile + 4 * grp;
        float s2[4];
        float mt = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = t0 + i;
          const bool att = ok_cur & (t >= R.lo) & (t < R.n);
          s2[i] = att ? sc[i] * a.scale_log2 : -INFINITY;
          mt = fmaxf(mt, s2[i]);
        }
        mt = max_xor16_32(mt);
        const float m_new = fmaxf(m_run, mt);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(s2[i] - m_use);
        l_run = l_run * alpha + sum_xor16_32((p[0] + p[1]) + (p[2] + p[3]));
        m_run = m_new;
        const u32x2 pa = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
        const i16x4 pop = __builtin_bit_cast(i16x4, pa);
        if (__any(alpha != 1.f)) {
          float al[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * grp + i);
#pragma unroll
          for (int e = 0; e < 16; ++e)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[e][i] *= al[i];
        }

        // P.V. Keys outside [lo, n) or on an invalid page: V := 0 (p is 0 there, 0 * NaN is not).
        u32x4 vv[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = t0 + i;
          const bool valid = ok_cur & (t >= R.lo) & (t < R.n);
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int d = 0; d < 4; ++d) vv[2 * i + h][d] = valid ? vr[2 * i + h][d] : 0u;
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const u32x2 be = {__builtin_amdgcn_perm(vv[2 + h][d], vv[h][d], 0x05040100u),
                              __builtin_amdgcn_perm(vv[6 + h][d], vv[4 + h][d], 0x05040100u)};
            const u32x2 bo = {__builtin_amdgcn_perm(vv[2 + h][d], vv[h][d], 0x07060302u),
                              __builtin_amdgcn_perm(vv[6 + h][d], vv[4 + h][d], 0x07060302u)};
            acc[8 * h + 2 * d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                pop, __builtin_bit_cast(i16x4, be), acc[8 * h + 2 * d], 0, 0, 0);
            acc[8 * h + 2 * d + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                pop, __builtin_bit_cast(i16x4, bo), acc[8 * h + 2 * d + 1], 0, 0, 0);
          }
      }
      // Next tile's V into the registers just consumed.
      __builtin_amdgcn_sched_barrier(0);
      if (more) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          vr[j] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4*>(a.v_pool + base_n + v_off + v_elem(j)));
      }
      ks_fence();  // this step's LDS reads stay before the next step's park
      base = base_n;
      ok = ok_n;
    }
  }

  // Merge the four waves' states.
  if constexpr (kValu) {
    // The two half waves hold the same dims for different keys.
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) ov[h][e] = ks_sum_halves(ov[h][e]);
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        m_lds[wave][h] = mv[h];
        l_lds[wave][h] = lv[h];
      }
    }
    if (lane < 32) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float* dst = &o_lds[wave][h][8 * lane];
        *reinterpret_cast<f32x4*>(dst) = f32x4{ov[h][0], ov[h][1], ov[h][2], ov[h][3]};
        *reinterpret_cast<f32x4*>(dst + 4) = f32x4{ov[h][4], ov[h][5], ov[h][6], ov[h][7]};
      }
    }
  } else {
    // Lane col (< G) of lane group 0 holds head col's m and l; lane (col, grp 0), register i
    // holds head i's dims 8col + e % 8 + 128 (e / 8).
    if (lane < G) {
      m_lds[wave][lane] = m_run;
      l_lds[wave][lane] = l_run;
    }
    if (grp == 0) {
#pragma unroll
      for (int i = 0; i < G; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float* dst = &o_lds[wave][i][8 * col + 128 * h];
          *reinterpret_cast<f32x4*>(dst) =
              f32x4{acc[8 * h][i], acc[8 * h + 1][i], acc[8 * h + 2][i], acc[8 * h + 3][i]};
          *reinterpret_cast<f32x4*>(dst + 4) =
              f32x4{acc[8 * h + 4][i], acc[8 * h + 5][i], acc[8 * h + 6][i], acc[8 * h + 7][i]};
        }
    }
  }
  __syncthreads();
  // Thread tid finishes (head, dim) pairs tid, tid + 64 NW, ... of the group.
  for (int idx = tid; idx < G * D; idx += kKsThreads) {
    const int h = idx / D, d = idx - h * D;
    float M = m_lds[0][h];
#pragma unroll
    for (int w = 1; w < kKsWaves; ++w) M = fmaxf(M, m_lds[w][h]);
    float W = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kKsWaves; ++w) {
        const float r = __builtin_amdgcn_exp2f(m_lds[w][h] - M);  // -inf - M gives 0
        W += r * l_lds[w][h];
        O += r * o_lds[w][h][d];
      }
    }
    const float inv = W > 0.f ? 1.f / W : 0.f;
    a.o_part[((out_row0 + h) * ns + split) * D + d] = O * inv;
    if (d == 0)
      a.lse_part[(out_row0 + h) * ns + split] =
          (M == -INFINITY) ? -INFINITY : (M + __log2f(W)) * kLn2;
  }
}

}  // namespace

bool stage1_keysplit_supported(int head_dim, int group_size, int q_len, int sink, bool shared) {
  return head_dim == kKsD && (group_size == 1 || group_size == 2 || group_size == 4) &&
         q_len == 1 && sink == 0 && !shared;
}

hipError_t launch_stage1_keysplit(const Stage1Args& args, int group_size, int batch,
                                  hipStream_t stream) {
  // Eight waves: with one chunk per (sequence, kv head) a workgroup walks the whole key range,
  // and eight tiles in flight per workgroup keep it fed (four measured slower). More splits run
  // on the column-split kernel, which measured as fast or faster there.
  constexpr int kNW = DECODE_ATTN_KS_WAVES;
  dim3 grid(args.num_splits, args.num_kv_heads, batch);
  dim3 block(64 * kNW);
  void* kargs[] = {const_cast<Stage1Args*>(&args)};
  const void* fn = nullptr;
  switch (group_size) {
    case 1: fn = reinterpret_cast<const void*>(&stage1_ks_kernel<1, kNW>); break;
    case 2: fn = reinterpret_cast<const void*>(&stage1_ks_kernel<2, kNW>); break;
    case 4: fn = reinterpret_cast<const void*>(&stage1_ks_kernel<4, kNW>); break;
    default: return hipErrorInvalidValue;
  }
  return hipLaunchKernel(fn, grid, block, kargs, 0, stream);
}

}  // namespace decode_attn
