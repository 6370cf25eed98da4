// stage1.hip — split-KV stage 1 of paged GQA decode attention for gfx950 (CDNA4).
//
// One workgroup per (split, query block, kv head, sequence) reads the keys of its chunk once and
// serves every query head of the GQA group with them (several query heads sharing a KV head are
// handled by one program: Sparse-vLLM PR #27 "feat: support Gemma 4 and native multimodal
// inference", section "专用算子与性能优化"). It writes the chunk's softmax-normalised partial output
// and its log-sum-exp, the split-KV partial buffer of vLLM learning notes "模型库与算子层 — 概念",
// section "MLA 与 Sparse MLA（DSA）".
//
// Work decomposition (NW = D / CW wavefronts of 64 lanes, each owning CW head-dim columns: CW = 128
// for head_dim 512 and 64 for 256 by default; the chunk is walked in steps of SUB tiles of 16 keys,
// a tile being a page of 16 keys or a 16-key slice of a larger page; all waves work on the same
// tiles):
//   * wave w owns the head-dim columns [CW*w, CW*w + CW) of K, V and the output;
//   * scores: v_mfma_f32_16x16x32_bf16 with A = K tile (16 keys x 32 columns) and B = the q block
//     (32 columns x 16 rows, one row per (query, head), unused rows zero, kept in registers). K is
//     loaded in row order, whole 128-byte lines per load, parked in the wave's LDS slice and read
//     back in the A layout (two-row-group blocks load the A layout directly). Each wave gets the
//     partial scores of its columns; the NW partials meet in LDS (one barrier per step) and are
//     summed in a fixed order, so every wave holds the same full scores: lane l has keys
//     4*(l/16)..+3 of row l%16;
//   * softmax: keys a row does not attend get -inf by select (never by multiplying a mask, so NaN
//     in unused slots cannot leak), running max and sum per row in base-2 units, hardware exp2,
//     the four lanes of a row combined with row-half swaps (v_permlane16/32_swap);
//   * P.V: v_mfma_f32_16x16x16_bf16 with A = P (16 rows x 16 keys, which is exactly the layout the
//     score MFMA left in the lanes, rounded to bf16) and B = V (16 keys x 16 columns). V is loaded
//     so that lane l holds CW/8 bytes of keys 4*(l/16)..+3 in its own column slice and is
//     transposed inside the lane with byte permutes; each wave accumulates O[rows][its columns];
//   * loads run one step ahead in registers: the K registers are refilled for the next step right
//     after the park (or the score MFMAs), the V registers right after the P.V MFMAs; the page ids
//     of the step after that are fetched as a small vector (lane u holds tile u's id) one step
//     earlier still, so no dependent block-table read sits on the critical path;
//   * start (one query token, no sinks): the page ids of the chunk the plan's expected length
//     gives are fetched while the sequence's length is still in flight, and kept when the length
//     gives the same chunk, so the length, page-id and tile reads cost two memory round trips
//     before the first step instead of three.
// The per-row softmax state is identical in all waves, so no merge is needed at the end: each
// wave writes its own columns of the partial output.

#include <hip/hip_runtime.h>

#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace decode_attn {
namespace {

// Build-time knobs (defaults are the values tuned on MI355X): 16-key tiles per loop step, and
// whether K/V that one workgroup alone reads are loaded with the non-temporal hint (streamed
// once, no reuse worth caching).
#ifndef DECODE_ATTN_STAGE1_SUB
#define DECODE_ATTN_STAGE1_SUB 1
#endif
#ifndef DECODE_ATTN_NT_LOADS
#define DECODE_ATTN_NT_LOADS 1
#endif

#ifndef DECODE_ATTN_COLS_PER_WAVE_512
#define DECODE_ATTN_COLS_PER_WAVE_512 128
#endif
#ifndef DECODE_ATTN_KV_PAD
#define DECODE_ATTN_KV_PAD 8
#endif
#ifndef DECODE_ATTN_COLS_PER_WAVE_256
#define DECODE_ATTN_COLS_PER_WAVE_256 64
#endif


// K/V tile loads. STREAM: no other workgroup reads these tiles, so they take the non-temporal
// hint. Several query blocks of one sequence re-read the same tiles instead, which the L2 serves
// only to ordinary loads (measured on a 512-token chunk of the 32K global layer: 9.9 ms with
// the hint, 6.7 ms without; single-token decode is 10% faster with it).
template <typename T, bool STREAM>
__device__ __forceinline__ T load_kv(const uint16_t* p) {
  if constexpr (STREAM && DECODE_ATTN_NT_LOADS)
    return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
  else
    return *reinterpret_cast<const T*>(p);
}


// Compiler-only ordering of memory accesses (no instruction is emitted).
__device__ __forceinline__ void compiler_fence() { __asm__ volatile("" ::: "memory"); }

// Workgroup barrier that waits for this wave's LDS accesses only (s_waitcnt lgkmcnt(0)), leaving
// outstanding global loads in flight.
__device__ __forceinline__ void lds_barrier() {
  compiler_fence();
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt = max, expcnt = max, lgkmcnt = 0
  __builtin_amdgcn_s_barrier();
  compiler_fence();
}

#ifndef DECODE_ATTN_COLS_PER_WAVE_RG2
#define DECODE_ATTN_COLS_PER_WAVE_RG2 128
#endif

// Columns per wave. Two row groups double the accumulators; 64 columns per wave (twice the
// waves) keeps two waves per SIMD, but on MI355X it measured no faster than 128 with one.
template <int D, int RG>
struct Shape {
  static_assert(D == 256 || D == 512, "head_dim");
  static constexpr int kCols =
      RG == 2 ? (D == 512 ? DECODE_ATTN_COLS_PER_WAVE_RG2 : DECODE_ATTN_COLS_PER_WAVE_256)
              : (D == 512 ? DECODE_ATTN_COLS_PER_WAVE_512 : DECODE_ATTN_COLS_PER_WAVE_256);
  static_assert(kCols == 64 || kCols == 128, "columns per wave");
  static constexpr int kWaves = D / kCols;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kKSteps = kCols / 32;  // score MFMAs per tile per wave
  static constexpr int kVE = kCols / 16;      // columns per lane in a V row (4 or 8)
  static constexpr int kVDwords = kVE / 2;
  using VRow = typename std::conditional<kVDwords == 4, u32x4, u32x2>::type;
};

// One step's worth of this wave's slice of K and V: SUB tiles of 16 keys.
template <int D, int RG, int SUB>
struct StepRegs {
  bf16x8 k[SUB][Shape<D, RG>::kKSteps];
  typename Shape<D, RG>::VRow v[SUB][4];  // tile u, keys 4*(lane/16)+i, i = 0..3
};

// SHARED: the pools are one buffer (layers whose values are their keys). Each tile is then read
// once; every wave parks its K slice in LDS (rows padded by 16 bytes against bank conflicts) and
// reads it back in both operand layouts.
// GENERAL: several query tokens per sequence and/or sink keys. Without it (one query token, no
// sinks) the row bounds are uniform and the query-block and sink arithmetic folds away.
// RG: groups of 16 MFMA rows per workgroup (2 only with GENERAL): 16 * RG rows share every tile
// read, so up to 32 / G query tokens cost one pass over the keys (a sequence with 64 rows or more
// per kv head runs on the prefill kernel instead, prefill.hip).
// STREAM: no other workgroup reads this block's tiles (one query block per sequence), so K/V
// loads carry the non-temporal hint; with several query blocks they are ordinary loads and the
// L2 serves the blocks' re-reads.
template <int D, int G, int SUB, bool SHARED, bool GENERAL, int RG, bool STREAM>
__global__ __launch_bounds__((Shape<D, RG>::kThreads)) void stage1_kernel(const Stage1Args a) {
  using Sh = Shape<D, RG>;
  constexpr int kWaves = Sh::kWaves;
  constexpr int kKSteps = Sh::kKSteps;
  constexpr int kVE = Sh::kVE;
  static_assert(RG == 1 || (RG == 2 && GENERAL), "row groups");

  __shared__ __attribute__((aligned(16))) f32x4 score_lds[2][SUB][RG][kWaves][64];
  constexpr int kKvRow = Sh::kCols + DECODE_ATTN_KV_PAD;  // padded row of a parked K slice (bf16 elements)
  // K in row order through LDS (whole 128-byte lines per load; the A-operand order reads half a
  // line per row per load, which doubles the L2 requests): always for SHARED, and for separate
  // pools with one row group. With two row groups the extra LDS round trip measured slower.
  constexpr bool KROW = SHARED || RG == 1;
  __shared__ __attribute__((aligned(16))) uint16_t kv_lds[KROW ? kWaves : 1][SUB][16][kKvRow];

  const int ns = a.num_splits;
  const int split = GENERAL ? (int)blockIdx.x % ns : (int)blockIdx.x;
  // Query block: queries qb * kQB + [0, kQB). Later queries attend more keys (causal), so the
  // blocks are numbered from the last one: the longest workgroups are dispatched first.
  const int qb = GENERAL ? a.num_qblocks - 1 - (int)blockIdx.x / ns : 0;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = lane >> 4;  // lane group 0..3
  const int col = lane & 15;  // scores: MFMA row (query, head); P.V: column block
  const int S = a.page_size;
  constexpr int kCols = Sh::kCols;
  using VRow = typename Sh::VRow;
  const int c0 = wave * kCols;  // first head-dim column of this wave
  const int L = GENERAL ? a.q_len : 1;
  const int sink = GENERAL ? a.sink : 0;

  // The 16 * RG MFMA rows: row r is query qb * kQB + r / G of the sequence, head kvh * G + r % G
  // (row group r / 16). Output row index (b, query, head) in the [B, L, Hq] order of q and of
  // the partials.
  constexpr int kQB = 16 * RG / G;
  auto row_query = [&](int r) { return qb * kQB + r / G; };
  auto row_valid = [&](int r) { return row_query(r) < L; };
  auto out_row = [&](int r) -> size_t {
    return ((size_t)b * L + row_query(r)) * a.num_q_heads + (size_t)kvh * G + r % G;
  };

  // q block, B operand of the score MFMA of row group rg: row 16 * rg + col, columns
  // c0 + 32*j + 8*grp .. +8; zero for rows past the last query. Every lane loads (a clamped row)
  // so no load sits under a divergent branch.
  bf16x8 qop[RG][kKSteps];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    const int rr = 16 * rg + col;
    const bool rv = row_valid(rr);
    const uint16_t* qr = a.q + out_row(rv ? rr : col % G) * D;  // query qb * kQB is valid
#pragma unroll
    for (int j = 0; j < kKSteps; ++j) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qr + c0 + 32 * j + 8 * grp);
      const u32x4 z = {0u, 0u, 0u, 0u};
      qop[rg][j] = __builtin_bit_cast(bf16x8, rv ? v : z);
    }
  }

  // Per-lane element offsets inside a tile: K (A operand) row = col, columns c0 + 32j + 8grp;
  // V rows 4grp + i, columns c0 + kVE*col .. + kVE.
  // KROW reads K in row order instead: load j brings rows kRPI*j + lane / kCPR, 16-byte chunk
  // lane % kCPR, so every load covers whole 128-byte lines; the A operand layout (and, for
  // SHARED, the V layout) is then read back from LDS.
  constexpr int kCPR = kCols / 8;   // 16-byte chunks in a row of this wave's columns
  constexpr int kRPI = 64 / kCPR;   // rows per load instruction
  const int k_off = KROW ? (lane / kCPR) * D + c0 + 8 * (lane % kCPR) : col * D + c0 + 8 * grp;
  const int k_step = KROW ? kRPI * D : 32;  // element offset between the kKSteps loads
  const int v_off = (4 * grp) * D + c0 + kVE * col;

  // Speculative start (one query token, no sinks): the page ids of the chunk this split would have
  // at the plan's expected length (a.spec_ctx) are fetched while ctx_lens is still in flight, and
  // kept when the actual length gives the same chunk (the first tiles' fetch then leaves one
  // memory round trip earlier); otherwise they are fetched again.
  StepRegs<D, RG, SUB> r;
  size_t base[SUB];
  bool ok[SUB];
  int32_t pid_first[SUB];  // page ids of list entries t_begin .. t_begin + SUB - 1
  int32_t pid_next = 0;
  const int tiles_per_page = S / kTile;
  const int32_t* table_row = a.block_table + (size_t)b * a.max_pages_per_seq;
  const int max_keys = a.max_pages_per_seq * S;
  int n_ctx = load_uniform(a.ctx_lens, b);
  int s_begin = 0, s_end = 0, s_shift = 0;
  bool spec = false;
  if constexpr (!GENERAL) {
    const int n_s = a.spec_ctx < max_keys ? a.spec_ctx : max_keys;
    const int lo_s = (a.window > 0 && n_s > a.window) ? n_s - a.window : 0;
    s_shift = lo_s / kTile;
    const int hi_s = (n_s + kTile - 1) / kTile;
    const int T_s = hi_s > s_shift ? hi_s - s_shift : 0;
    s_begin = (int)(((int64_t)split * T_s) / ns);
    s_end = (int)(((int64_t)(split + 1) * T_s) / ns);
    spec = n_s > 0 && s_begin < s_end;
    if (spec) {
#pragma unroll
      for (int u = 0; u < SUB; ++u) {
        const int tc = (s_begin + u < s_end ? s_begin + u : s_end - 1) + s_shift;
        pid_first[u] = load_uniform(table_row, tc / tiles_per_page);
      }
      const int tn = (s_begin + SUB + lane % SUB < s_end ? s_begin + SUB + lane % SUB : s_end - 1) +
                     s_shift;
      pid_next = table_row[tn / tiles_per_page];
    }
  }
  __asm__ volatile("; stage-1 speculative loads issued" ::: "memory");

  // Keys of this sequence: [0, sk) (sink keys not inside the window) and [lo, n). They are walked
  // as a list of T tiles, list index v: the sink tiles 0 .. st-1 first, then the window's tiles
  // from physical tile w0 = max(st, lo / 16) on, i.e. physical tile v + (v >= st ? shift : 0).
  // This split takes list entries [t_begin, t_end).
  //
  // Query i of the sequence sits at position n - L + i and attends keys t < n_i = n - L + i + 1,
  // t >= lo_i (its window), or t < sink. The workgroup walks the union over its queries: the
  // window of its first query up to n_i of its last one.
  n_ctx = n_ctx < 0 ? 0 : (n_ctx > max_keys ? max_keys : n_ctx);
  auto query_end = [&](int i) { const int e = n_ctx - L + i + 1; return e < 0 ? 0 : e; };
  auto window_lo = [&](int e) { return (a.window > 0 && e > a.window) ? e - a.window : 0; };
  const int q_last = (qb + 1) * kQB < L ? (qb + 1) * kQB - 1 : L - 1;
  const int n = query_end(q_last);
  const int lo = window_lo(query_end(qb * kQB));
  const int sk = sink < lo ? sink : lo;
  // This lane's rows (scores and softmax use row 16 * rg + col in row group rg).
  int row_n[RG], row_lo[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    const int rr = 16 * rg + col;
    row_n[rg] = GENERAL ? (row_valid(rr) ? query_end(row_query(rr)) : 0) : n;
    row_lo[rg] = GENERAL ? window_lo(row_n[rg]) : lo;
  }
  const int st = (sk + kTile - 1) / kTile;
  const int w0 = st > lo / kTile ? st : lo / kTile;
  const int tile_hi = (n + kTile - 1) / kTile;
  const int T = st + (tile_hi > w0 ? tile_hi - w0 : 0);
  const int shift = w0 - st;
  const int t_begin = (int)(((int64_t)split * T) / ns);
  const int t_end = (int)(((int64_t)(split + 1) * T) / ns);
  auto phys_tile = [&](int v) { return (!GENERAL || v >= st) ? v + shift : v; };

  if (t_begin >= t_end) {  // empty split: o = 0, lse = -inf
    for (int idx = lane; idx < 16 * RG * kCols; idx += 64) {
      const int r = idx / kCols;
      if (row_valid(r)) a.o_part[(out_row(r) * ns + split) * D + c0 + (idx - r * kCols)] = 0.f;
    }
    if (wave == 0 && lane < 16 * RG && row_valid(lane))
      a.lse_part[out_row(lane) * ns + split] = -INFINITY;
    __builtin_amdgcn_s_waitcnt(0);  // the early loads land before the wave ends
    return;
  }
  const int t_last = t_end - 1;

  // Tiles past the split re-read its last tile (an L2 hit; they are masked) so every load is
  // unconditional and the compiler can count outstanding loads exactly. Invalid page ids are
  // never dereferenced: page 0 is read instead and the tile is masked.
  auto clamp_tile = [&](int ti) { return ti < t_end ? ti : t_last; };
  auto tile_base = [&](int ti, int phys, bool& ok) -> size_t {
    const int tc = phys_tile(clamp_tile(ti));
    const bool page_ok = (unsigned)phys < (unsigned)a.num_pages;
    ok = ti < t_end && page_ok;
    const int pg = page_ok ? phys : 0;
    const int within = tc - (tc / tiles_per_page) * tiles_per_page;
    return (((size_t)pg * a.num_kv_heads + kvh) * S + within * kTile) * D;
  };
  // Page ids of list entries t .. t+SUB-1 as a vector: lane u holds entry (t + u % SUB)'s id.
  auto load_page_ids = [&](int t) -> int32_t {
    const int tc = phys_tile(clamp_tile(t + lane % SUB));
    return table_row[tc / tiles_per_page];
  };

  const bool hit = spec && shift == s_shift && t_begin == s_begin && t_end == s_end;
  if (!hit) {
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      const int tc = phys_tile(clamp_tile(t_begin + u));
      pid_first[u] = load_uniform(table_row, tc / tiles_per_page);
    }
    pid_next = load_page_ids(t_begin + SUB);
  }
#pragma unroll
  for (int u = 0; u < SUB; ++u) base[u] = tile_base(t_begin + u, pid_first[u], ok[u]);
#pragma unroll
  for (int u = 0; u < SUB; ++u)
#pragma unroll
    for (int j = 0; j < kKSteps; ++j)
      r.k[u][j] = load_kv<bf16x8, STREAM>(a.k_pool + base[u] + k_off + k_step * j);
  if constexpr (!SHARED) {
#pragma unroll
    for (int u = 0; u < SUB; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        r.v[u][i] = load_kv<VRow, STREAM>(a.v_pool + base[u] + v_off + i * D);
  }
  // A fence the loop latch does not have: otherwise the identical trailing V loads of this
  // prologue and of the loop body get merged into the loop header, which would turn the V
  // prefetch into a load at the top of every step.
  __asm__ volatile("; stage-1 prologue loads issued" ::: "memory");

  float m_run[RG];   // running max (base-2 units) of row 16 * rg + col
  float l_run[RG];   // running sum of exp2(s - m_run) of that row
  f32x4 acc[RG][kVE];  // O[row 16 * rg + 4*grp + i][column c0 + kVE*col + e] = acc[rg][e][i]
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    m_run[rg] = -INFINITY;
    l_run[rg] = 0.f;
#pragma unroll
    for (int e = 0; e < kVE; ++e) acc[rg][e] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  int buf = 0;
  for (int t0 = t_begin; t0 < t_end; t0 += SUB) {
    // Next step's K into the registers once they are consumed, then the page ids of the step
    // after. The scheduling barriers keep loads in program order, which the wait counts rely on.
    const int tn = t0 + SUB;
    bool ok_n[SUB];
    size_t base_n[SUB];
    int32_t pid_after;
    auto refill_k = [&]() {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < SUB; ++u)
        base_n[u] = tile_base(tn + u, __builtin_amdgcn_readlane(pid_next, u), ok_n[u]);
#pragma unroll
      for (int u = 0; u < SUB; ++u)
#pragma unroll
        for (int j = 0; j < kKSteps; ++j)
          r.k[u][j] = load_kv<bf16x8, STREAM>(a.k_pool + base_n[u] + k_off + k_step * j);
      pid_after = load_page_ids(tn + SUB);
      __builtin_amdgcn_sched_barrier(0);
    };

    // A operand of the scores: K rows col, columns 32j + 8grp. KROW parks the row-order K of this
    // step in LDS (where P.V also reads it as V when SHARED), refills the registers at once and
    // reads the A layout back; LDS accesses of one wave take effect in program order.
    bf16x8 ka[SUB][kKSteps];
    if constexpr (KROW) {
#pragma unroll
      for (int u = 0; u < SUB; ++u)
#pragma unroll
        for (int j = 0; j < kKSteps; ++j)
          *reinterpret_cast<bf16x8*>(
              &kv_lds[KROW ? wave : 0][u][kRPI * j + lane / kCPR][8 * (lane % kCPR)]) =
              r.k[u][j];
      compiler_fence();
      refill_k();
#pragma unroll
      for (int u = 0; u < SUB; ++u)
#pragma unroll
        for (int j = 0; j < kKSteps; ++j)
          ka[u][j] = *reinterpret_cast<const bf16x8*>(
              &kv_lds[KROW ? wave : 0][u][col][32 * j + 8 * grp]);
    } else {
#pragma unroll
      for (int u = 0; u < SUB; ++u)
#pragma unroll
        for (int j = 0; j < kKSteps; ++j) ka[u][j] = r.k[u][j];
    }

    // Partial scores of this wave's columns for the SUB tiles of the step.
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        f32x4 p0 = {0.f, 0.f, 0.f, 0.f}, p1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kKSteps; j += 2) {
          p0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[u][j], qop[rg][j], p0, 0, 0, 0);
          if (j + 1 < kKSteps)
            p1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[u][j + 1], qop[rg][j + 1], p1, 0, 0,
                                                         0);
        }
        score_lds[buf][u][rg][wave][lane] = p0 + p1;
      }
    }
    if constexpr (!KROW) refill_k();

    lds_barrier();
    f32x4 sc[SUB][RG];
#pragma unroll
    for (int u = 0; u < SUB; ++u)
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        sc[u][rg] = score_lds[buf][u][rg][0][lane];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) sc[u][rg] += score_lds[buf][u][rg][w][lane];
      }
    buf ^= 1;

    // Mask and online softmax for row 16 * rg + col over the SUB*16 keys of the step. Key t is
    // attended by the row iff its page is valid, t < row_n and (t >= row_lo or t < sink); it is
    // read at all (in_union) iff its page is valid, t < n and (t >= lo or t < sk). The per-lane
    // tests combine with & and | (no short circuit, hence no branches on the exec mask).
    // Without GENERAL every row has the same bounds, folded per tile into one uniform range
    // [klo, khi) (empty for an invalid page).
    int tok0[SUB], klo[SUB], khi[SUB];
    bool full = true;
    auto in_union = [&](int u, int t) {
      if constexpr (GENERAL) return ok[u] & (t < n) & ((t >= lo) | (t < sk));
      else return (t >= klo[u]) & (t < khi[u]);
    };
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      tok0[u] = phys_tile(t0 + u) * kTile;
      klo[u] = ok[u] ? (lo > tok0[u] ? lo : tok0[u]) : tok0[u] + kTile;
      khi[u] = n < tok0[u] + kTile ? n : tok0[u] + kTile;
      full = full && ok[u] && tok0[u] + kTile <= n && (tok0[u] >= lo || tok0[u] + kTile <= sk);
    }
    i16x4 pop[SUB][RG];
    float alpha[RG];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      float mt = -INFINITY;
      float s2[SUB][4];
#pragma unroll
      for (int u = 0; u < SUB; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = tok0[u] + 4 * grp + i;
          const bool att =
              GENERAL ? ok[u] & (t < row_n[rg]) & ((t >= row_lo[rg]) | (t < sink)) : in_union(u, t);
          s2[u][i] = att ? sc[u][rg][i] * a.scale_log2 : -INFINITY;
          mt = fmaxf(mt, s2[u][i]);
        }
      mt = max_xor16_32(mt);
      const float m_new = fmaxf(m_run[rg], mt);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      alpha[rg] = __builtin_amdgcn_exp2f(m_run[rg] - m_use);
      float ps = 0.f;
#pragma unroll
      for (int u = 0; u < SUB; ++u) {
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(s2[u][i] - m_use);
        ps += (p[0] + p[1]) + (p[2] + p[3]);
        // P as the A operand: P[row 16 * rg + col][keys 4*grp .. +3 of tile u] in bf16.
        const u32x2 pa = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
        pop[u][rg] = __builtin_bit_cast(i16x4, pa);
      }
      ps = sum_xor16_32(ps);
      l_run[rg] = l_run[rg] * alpha[rg] + ps;
      m_run[rg] = m_new;

      // Rescale the accumulator rows (16 * rg + 4*grp + i) when some running max moved.
      if (__any(alpha[rg] != 1.f)) {
        float al[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha[rg], 4 * grp + i);
#pragma unroll
        for (int e = 0; e < kVE; ++e)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[rg][e][i] *= al[i];
      }
    }

    // P.V, one tile at a time.
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      VRow vr[4];
      if constexpr (SHARED) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          vr[i] = *reinterpret_cast<const VRow*>(
              &kv_lds[KROW ? wave : 0][u][4 * grp + i][kVE * col]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) vr[i] = r.v[u][i];
      }
      if (!full) {  // masked keys: V := 0 (their p is 0, but 0 * NaN would not be)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool valid = in_union(u, tok0[u] + 4 * grp + i);
#pragma unroll
          for (int d = 0; d < Sh::kVDwords; ++d) vr[i][d] = valid ? vr[i][d] : 0u;
        }
      }
      // Transpose in the lane: B operand e = V[keys 4*grp + 0..3][column kVE*col + e].
#pragma unroll
      for (int d = 0; d < Sh::kVDwords; ++d) {
        const u32x2 be = {__builtin_amdgcn_perm(vr[1][d], vr[0][d], 0x05040100u),
                          __builtin_amdgcn_perm(vr[3][d], vr[2][d], 0x05040100u)};
        const u32x2 bo = {__builtin_amdgcn_perm(vr[1][d], vr[0][d], 0x07060302u),
                          __builtin_amdgcn_perm(vr[3][d], vr[2][d], 0x07060302u)};
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
          acc[rg][2 * d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
              pop[u][rg], __builtin_bit_cast(i16x4, be), acc[rg][2 * d], 0, 0, 0);
          acc[rg][2 * d + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
              pop[u][rg], __builtin_bit_cast(i16x4, bo), acc[rg][2 * d + 1], 0, 0, 0);
        }
      }
    }

    // Next step's V into the registers just consumed.
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!SHARED) {
#pragma unroll
      for (int u = 0; u < SUB; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          r.v[u][i] = load_kv<VRow, STREAM>(a.v_pool + base_n[u] + v_off + i * D);
    }
    if constexpr (KROW) compiler_fence();  // this step's LDS reads stay before the next writes
#pragma unroll
    for (int u = 0; u < SUB; ++u) ok[u] = ok_n[u];
    pid_next = pid_after;
  }

  // Normalise and write this wave's columns of the partial output; lane holds rows
  // 16 * rg + 4*grp + i.
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 16 * rg + 4 * grp + i;
      const float lh = __shfl(l_run[rg], 4 * grp + i);
      const float inv = lh > 0.f ? 1.f / lh : 0.f;
      if (row_valid(h)) {
        float* dst = a.o_part + (out_row(h) * ns + split) * D + c0 + kVE * col;
#pragma unroll
        for (int e4 = 0; e4 < kVE; e4 += 4) {
          const f32x4 v4 = {acc[rg][e4][i] * inv, acc[rg][e4 + 1][i] * inv,
                            acc[rg][e4 + 2][i] * inv, acc[rg][e4 + 3][i] * inv};
          *reinterpret_cast<f32x4*>(dst + e4) = v4;
        }
      }
    }
  if (wave == 0 && lane < 16) {
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      if (row_valid(16 * rg + lane)) {
        const float lse = (m_run[rg] == -INFINITY) ? -INFINITY
                                                   : (m_run[rg] + __log2f(l_run[rg])) * kLn2;
        a.lse_part[out_row(16 * rg + lane) * ns + split] = lse;
      }
    }
  }
}

template <int D, int G, bool SHARED>
const void* kernel_for(bool general, int row_groups, bool streaming) {
  constexpr int kSub = DECODE_ATTN_STAGE1_SUB;
  if (!general)
    return reinterpret_cast<const void*>(&stage1_kernel<D, G, kSub, SHARED, false, 1, true>);
  if (row_groups == 1)  // G * L <= 16: one query block, tiles streamed once
    return reinterpret_cast<const void*>(&stage1_kernel<D, G, kSub, SHARED, true, 1, true>);
  return streaming
             ? reinterpret_cast<const void*>(&stage1_kernel<D, G, kSub, SHARED, true, 2, true>)
             : reinterpret_cast<const void*>(&stage1_kernel<D, G, kSub, SHARED, true, 2, false>);
}

template <int D, int G>
hipError_t launch(const Stage1Args& args, bool shared, int batch, hipStream_t stream) {
  // Query blocks of one (sequence, kv head) are num_splits workgroups apart in dispatch order,
  // which deals workgroups round-robin to the 8 XCDs: each XCD runs several blocks of the same
  // sequence at once, and they share its L2 for the tiles they all read.
  dim3 grid(args.num_splits * args.num_qblocks, args.num_kv_heads, batch);
  void* kargs[] = {const_cast<Stage1Args*>(&args)};
  const bool general = args.q_len > 1 || args.sink > 0;
  const int rgs = stage1_row_groups(G, args.q_len);
  const bool streaming = args.num_qblocks == 1;  // no other query block re-reads the tiles
  dim3 block(rgs == 2 ? Shape<D, 2>::kThreads : Shape<D, 1>::kThreads);
  const void* fn =
      shared ? kernel_for<D, G, true>(general, rgs, streaming)
             : kernel_for<D, G, false>(general, rgs, streaming);
  return hipLaunchKernel(fn, grid, block, kargs, 0, stream);
}

template <int D>
hipError_t launch_d(const Stage1Args& args, int group_size, bool shared, int batch,
                    hipStream_t stream) {
  switch (group_size) {
    case 1: return launch<D, 1>(args, shared, batch, stream);
    case 2: return launch<D, 2>(args, shared, batch, stream);
    case 4: return launch<D, 4>(args, shared, batch, stream);
    case 8: return launch<D, 8>(args, shared, batch, stream);
    case 16: return launch<D, 16>(args, shared, batch, stream);
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
  const bool shared = args.k_pool == args.v_pool;
  switch (head_dim) {
    case 256: return launch_d<256>(args, group_size, shared, batch, stream);
    case 512: return launch_d<512>(args, group_size, shared, batch, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace decode_attn
