// prefill.hip — stage 1 for long query chunks (prefill over the paged cache).
//
// The operation is stage 1's (decode_attn_stage1 in decode_attn.h): for query token i of
// sequence b at position n - L + i, query head h, the softmax of scale * q.k over the keys the
// query attends inside this split's share of the block's tile list, written as a normalised
// partial output and its log-sum-exp. Prefill is the attention layer's other operation next to
// decode (vLLM learning notes "模型库与算子层 — 概念", section "核心操作"); the partial format and the
// merge are the split-KV ones of section "MLA 与 Sparse MLA（DSA）" of the same notes.
//
// What changes against the decode kernel is the shape of the work. Decode has 16-32 (query,
// head) rows per KV head and streams K/V once, so the decode kernel splits the head dim across
// its waves and is bound by HBM. A prefill chunk has thousands of rows per KV head, and every
// K/V tile serves all of them: the work is MFMA-bound. Here every wave owns 16 rows with the full
// head dim, all waves of a workgroup share one 32-key K/V tile staged in LDS, and no scores cross
// waves. At head_dim 512, for chunks of at least 128 rows per KV head, a workgroup has 8 waves
// (128 rows): the double-buffered tiles take 131 KB of LDS, so one workgroup fills a CU, and its
// 8 waves put two on each SIMD (256 registers each), so one wave's softmax and LDS traffic run
// under the other's MFMAs. Shorter chunks at head_dim 512 (one wave per SIMD) and all chunks at
// head_dim 256 (two workgroups per CU) take 4 waves (64 rows).
//
//   - K/V tile of the step (32 keys = two 16-key entries of the tile list, each on its own page)
//     in LDS, double-buffered, one barrier per step. In 128-row workgroups the tile goes from
//     memory straight into LDS (global_load_lds_dwordx4, one key row of 1 KB per wave
//     instruction), issued right after the barrier into the buffer that step has just released,
//     so it has a whole step to land; no registers hold it. 64-row workgroups fetch it into
//     registers and write it to the other buffer one step later (at head_dim 512 around the score
//     MFMAs, at 256 at the end of the step). K and V rows are padded by 32 bytes: gfx950 serves a
//     16-byte LDS read in passes that pair lanes i and i + 16, and with a row pitch of 32 bytes
//     mod 256 the score operand reads (16 keys, same 16-byte column) fill all 64 banks in every
//     pass (measured: no bank conflicts; a 16-byte pad cost about 4 conflict cycles per read).
//   - scores: S^T[32 keys][16 rows] per wave with v_mfma_f32_16x16x32_bf16, A = K (keys x 32
//     columns, from LDS), B = the wave's q rows (in registers for the whole kernel). In 128-row
//     workgroups and at head_dim 256 the operand reads run 4 ahead of the MFMAs (scheduling
//     barriers keep the compiler from pulling each read down to its MFMA), and in 128-row
//     workgroups both MFMA phases of a step run at raised wave priority, so the SIMD's other wave
//     yields its issue slots to them;
//   - online softmax per row in base 2 (masks by select, running max and sum, accumulator
//     rescaled only when a max moved); the maximum is taken over the raw scores and scaled once,
//     and each probability is one fma and one exp2;
//   - P.V with v_mfma_f32_16x16x32_bf16: A = P (16 rows x 32 keys) straight from the score
//     registers; the 32 keys of the MFMA's reduction run in the order the score layout leaves
//     them (keys 4g..4g+3 then 16+4g..16+4g+3 for lane group g), and B = V takes its keys in that
//     same order through LDS transpose reads (ds_read_b64_tr_b16: 16 columns of 4 keys per read),
//     MFMA e producing output columns 16e .. 16e + 15. (The earlier form read 16 contiguous bytes
//     of one key row per lane and transposed them in the lane with v_perm_b32.)
//
// Keys outside the union of the block's ranges (and entries past the split) are written to LDS as
// zeros, so 0 * NaN never reaches P.V; per-row causal, window and sink masks are applied to the
// scores.

#include <hip/hip_runtime.h>

#include "device_common.h"
#include "internal.h"

namespace decode_attn {
namespace {

constexpr int kStepKeys = 2 * kTile;  // two tile-list entries per loop step

// Build-time knobs of the step's order (defaults measured on MI355X; the alternatives serve A/B
// builds).
#ifndef DECODE_ATTN_PREFILL_KAHEAD
#define DECODE_ATTN_PREFILL_KAHEAD 8
#endif
#ifndef DECODE_ATTN_PREFILL_KAHEAD_SHARED
#define DECODE_ATTN_PREFILL_KAHEAD_SHARED 2
#endif
#ifndef DECODE_ATTN_PREFILL_SPLIT_STORE
#define DECODE_ATTN_PREFILL_SPLIT_STORE 1
#endif
constexpr bool kSplitStore = DECODE_ATTN_PREFILL_SPLIT_STORE;  // V half stored after the scores
#ifndef DECODE_ATTN_PREFILL_SPREAD_V
#define DECODE_ATTN_PREFILL_SPREAD_V 1
#endif
constexpr bool kSpreadV = DECODE_ATTN_PREFILL_SPREAD_V;  // V loads issued between P.V column groups
#ifndef DECODE_ATTN_PREFILL_SPREAD_K
#define DECODE_ATTN_PREFILL_SPREAD_K 1
#endif
constexpr bool kSpreadK = DECODE_ATTN_PREFILL_SPREAD_K;  // K loads issued between score batches
#ifndef DECODE_ATTN_PREFILL_EARLY_STORE
#define DECODE_ATTN_PREFILL_EARLY_STORE 1  // bit 0: head_dim 512, bit 1: head_dim 256
#endif
// P.V's V operand by LDS transpose reads (ds_read_b64_tr_b16) instead of row reads and byte
// permutes in the VALU.
#ifndef DECODE_ATTN_PREFILL_TR
#define DECODE_ATTN_PREFILL_TR 1
#endif
constexpr bool kTr = DECODE_ATTN_PREFILL_TR;
// head_dim 512: the tiles go from memory straight into LDS (global_load_lds_dwordx4, one key row
// per wave instruction) instead of through registers.
#ifndef DECODE_ATTN_PREFILL_DMA
#define DECODE_ATTN_PREFILL_DMA 1
#endif
constexpr bool kDma = DECODE_ATTN_PREFILL_DMA;
// Score operand reads in flight ahead of the MFMAs (128-row workgroups; 0 = the compiler's order,
// which reads each operand just before its MFMA); KPIPE_SB = 0 leaves the order unpinned.
#ifndef DECODE_ATTN_PREFILL_KPIPE
#define DECODE_ATTN_PREFILL_KPIPE 4
#endif
constexpr int kKPipe = DECODE_ATTN_PREFILL_KPIPE;
#ifndef DECODE_ATTN_PREFILL_KPIPE_256
#define DECODE_ATTN_PREFILL_KPIPE_256 4
#endif
constexpr int kKPipe256 = DECODE_ATTN_PREFILL_KPIPE_256;  // the same at head_dim 256 (64 rows)
#ifndef DECODE_ATTN_PREFILL_KPIPE_SB
#define DECODE_ATTN_PREFILL_KPIPE_SB 1
#endif
// The direct fetches' LDS addresses carry no alias information (below, dma16).
#ifndef DECODE_ATTN_PREFILL_DMA_OPAQUE
#define DECODE_ATTN_PREFILL_DMA_OPAQUE 1
#endif
#ifndef DECODE_ATTN_PREFILL_SETPRIO
#define DECODE_ATTN_PREFILL_SETPRIO 1
#endif
// MFMA phases (scores, P.V) at raised wave priority, so that a SIMD's other wave yields to them.
constexpr bool kSetPrio = DECODE_ATTN_PREFILL_SETPRIO;
// Padding of a K row in LDS (bf16 elements).
#ifndef DECODE_ATTN_PREFILL_PAD
#define DECODE_ATTN_PREFILL_PAD 16
#endif
#ifndef DECODE_ATTN_PREFILL_XCD
#define DECODE_ATTN_PREFILL_XCD 1
#endif
constexpr bool kXcdRemap = DECODE_ATTN_PREFILL_XCD;  // query blocks of a KV head on one XCD

template <int D, int ROWS>
struct PShape {
  static_assert(D == 256 || D == 512, "head_dim");
  static constexpr int kPitch = D + DECODE_ATTN_PREFILL_PAD;  // LDS row pitch, bf16
  static constexpr int kVPitch = kTr ? D + 16 : D + 8;      // V rows (own buffer), bf16
  static constexpr int kChunks = D / 8;                     // 16-byte chunks per key row
  static constexpr int kQSteps = D / 32;                    // score MFMAs per 16 keys
  static constexpr int kLaneCols = D / 16;                  // output columns per lane
  static constexpr int kVGroups = kLaneCols / 8;            // 8-column groups per lane
  static constexpr int kRows = ROWS;                        // (query, head) rows per workgroup
  static constexpr int kWaves = kRows / 16;                 // 16 rows per wave
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kLoads = kStepKeys * kChunks / kThreads;  // 16-B loads per thread per matrix
  static constexpr int kKeysPerPass = kThreads / kChunks;   // key rows one pass of loads covers
};

// Physical position of 16-byte chunk c inside a key row: chunks are XOR-swizzled inside each
// group of 4 (D = 512) or 2 (D = 256) by the index of their 64-column (128-byte) block, which
// spreads the 16 lanes reading column group n of one key row over all 64 banks.
template <int D>
__device__ __forceinline__ int swz(int c) {
  return c ^ ((c >> 4) & (D / 128 - 1));
}

// 16 bytes per lane from global memory to LDS: lane l's bytes land at l_base + 16 l (l_base
// wave-uniform), so one instruction fills 1 KB of LDS, checked lane by lane on gfx950.
__device__ __forceinline__ void dma16(const uint16_t* g, uint16_t* l_base) {
#if DECODE_ATTN_PREFILL_DMA_OPAQUE
  // The LDS address passes through an empty asm statement, so the fetch carries no alias
  // information about the tile buffers. Otherwise the compiler may find that the first score read
  // of a step can alias the fetch of the tile two steps ahead (same array, other buffer) and wait
  // for every fetch in flight before it. The kernel's own waits order the fetches: all land before
  // the edge masking and the barrier that publishes their buffer.
  uint32_t l = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)(l_base);
  asm volatile("" : "+s"(l));
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)(uintptr_t)l, 16, 0,
                                   0);
#else
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)(l_base), 16, 0, 0);
#endif
}

// ds_read_b64_tr_b16: within each 16-lane group, lane i gets element (i & 3) of the 4-element
// rows that lanes 4c + (i >> 2) address, for c = 0..3 (a 4 x 4 transpose of 16-bit elements
// across each quad of lanes), checked lane by lane on gfx950.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// SHARED: the pools are one buffer (values are the keys); the V tile is the K tile.
template <int D, int G, bool SHARED, int ROWS>
__global__ __launch_bounds__(4 * ROWS) void prefill_kernel(const Stage1Args a) {
  using Sh = PShape<D, ROWS>;
  static_assert(Sh::kThreads == 4 * ROWS, "launch bounds");
  // Tiles staged through registers (head_dim 256, or head_dim 512 built without direct fetches)
  // are written to LDS at the end of the step (the fetch gets the whole step to land) or, as an
  // A/B variant for head_dim 512, around the score MFMAs (K half before them, V half after, the
  // fetch of the tile after it spread over the step).
  constexpr bool kDmaD = kDma && D == 512 && ROWS == kPrefillWideRows;
  constexpr bool kEarlyStore =
      !kDmaD && ((DECODE_ATTN_PREFILL_EARLY_STORE >> (D == 512 ? 0 : 1)) & 1);
  // Score operand reads in flight (pinned order): 128-row workgroups, and 64-row ones whose score
  // phase stages nothing (head_dim 256).
  constexpr int kPipeK = kDmaD ? kKPipe : (!kEarlyStore && D == 256 ? kKPipe256 : 0);
  constexpr int kPipeKN = kPipeK > 0 ? kPipeK : 1;
  // Score operands read ahead of their MFMAs (fewer when one tile serves as K and V).
  constexpr int kKAhead = SHARED && kDmaD ? DECODE_ATTN_PREFILL_KAHEAD_SHARED
                                           : DECODE_ATTN_PREFILL_KAHEAD;
  static_assert(Sh::kQSteps % kKAhead == 0 && kKAhead % 2 == 0, "score read-ahead");
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][kStepKeys][Sh::kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][SHARED ? 1 : kStepKeys][Sh::kVPitch];
  auto KB = [&](int b) -> uint16_t(*)[Sh::kPitch] { return k_lds[b]; };
  auto VB = [&](int b) -> uint16_t(*)[Sh::kVPitch] { return v_lds[b]; };

  constexpr int kWaves = Sh::kWaves, kThreads = Sh::kThreads;
  constexpr int kQB = Sh::kRows / G;  // queries per block
  const int ns = a.num_splits;
  // Work item of this workgroup: (b, kvh) pair major, then query block, then split. Workgroups
  // are handed to the 8 XCDs round robin in launch order, so when the grid divides by 8 the
  // launch index is remapped so that each XCD takes a contiguous run of work items: the query
  // blocks of one (sequence, KV head), which all read the same K/V, then share the XCD's L2.
  const int nwg = (int)(gridDim.x * gridDim.y * gridDim.z);
  const int lin = (int)(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z));
  const int w = (kXcdRemap && nwg % 8 == 0) ? (lin % 8) * (nwg / 8) + lin / 8 : lin;
  const int per_pair = ns * a.num_qblocks;
  const int split = w % ns;
  // Later queries attend more keys: blocks are numbered from the last one so the longest
  // workgroups are dispatched first.
  const int qb = a.num_qblocks - 1 - (w % per_pair) / ns;
  const int kvh = (w / per_pair) % a.num_kv_heads;
  const int b = w / per_pair / a.num_kv_heads;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = lane >> 4;
  const int col = lane & 15;
  const int S = a.page_size;
  const int L = a.q_len;
  const int sink = a.sink;

  // Row r of the block (0..63) is query qb * kQB + r / G, head kvh * G + r % G. This wave owns
  // rows 16 * wave .. + 15; lane (col, grp) scores for row 16 * wave + col.
  auto row_query = [&](int r) { return qb * kQB + r / G; };
  auto row_valid = [&](int r) { return row_query(r) < L; };
  auto out_row = [&](int r) -> size_t {
    return ((size_t)b * L + row_query(r)) * a.num_q_heads + (size_t)kvh * G + r % G;
  };

  const int max_keys = a.max_pages_per_seq * S;
  int n_ctx = load_uniform(a.ctx_lens, b);
  n_ctx = n_ctx < 0 ? 0 : (n_ctx > max_keys ? max_keys : n_ctx);
  auto query_end = [&](int i) { const int e = n_ctx - L + i + 1; return e < 0 ? 0 : e; };
  auto window_lo = [&](int e) { return (a.window > 0 && e > a.window) ? e - a.window : 0; };
  const int q_last = (qb + 1) * kQB < L ? (qb + 1) * kQB - 1 : L - 1;
  const int n = query_end(q_last);             // union of the block's ranges: [lo, n) + sinks
  const int lo = window_lo(query_end(qb * kQB));
  const int sk = sink < lo ? sink : lo;
  const int my_row = 16 * wave + col;
  const int row_n = row_valid(my_row) ? query_end(row_query(my_row)) : 0;
  const int row_lo = window_lo(row_n);

  // Tile list (as in the decode kernel): sink tiles 0 .. st-1, then the window's tiles from
  // physical tile w0 on; this split takes entries [t_begin, t_end).
  const int st = (sk + kTile - 1) / kTile;
  const int w0 = st > lo / kTile ? st : lo / kTile;
  const int tile_hi = (n + kTile - 1) / kTile;
  const int T = st + (tile_hi > w0 ? tile_hi - w0 : 0);
  const int shift = w0 - st;
  const int t_begin = (int)(((int64_t)split * T) / ns);
  const int t_end = (int)(((int64_t)(split + 1) * T) / ns);
  // Tile pc lies in page pc / tpp, slot pc % tpp (tpp = S / 16 <= 64 tiles per page). The quotient
  // is a multiply-high by a reciprocal fixed per workgroup: with l = ceil(log2 tpp) and
  // m = ceil(2^(31 + l) / tpp) < 2^32, floor(pc * m / 2^(31 + l)) = floor(pc / tpp) for
  // 0 <= pc < 2^31, since the product exceeds pc / tpp by less than 2^-l <= 1 / tpp.
  const int tpp = S / kTile;
  const int tpp_l = tpp > 1 ? 32 - __builtin_clz((uint32_t)(tpp - 1)) : 0;
  const uint32_t tpp_m =
      tpp > 1 ? (uint32_t)((((uint64_t)1 << (31 + tpp_l)) + (uint32_t)tpp - 1) / (uint32_t)tpp) : 0u;
  auto page_of = [&](int pc) -> int {
    return tpp > 1 ? (int)(__umulhi((uint32_t)pc, tpp_m) >> (tpp_l - 1)) : pc;
  };
  auto phys_tile = [&](int v) { return v >= st ? v + shift : v; };
  const int32_t* table_row = a.block_table + (size_t)b * a.max_pages_per_seq;

  if (t_begin >= t_end) {  // empty split: o = 0, lse = -inf
    for (int idx = tid; idx < Sh::kRows * D; idx += kThreads) {
      const int r = idx / D;
      if (row_valid(r)) a.o_part[(out_row(r) * ns + split) * D + (idx - r * D)] = 0.f;
    }
    if (tid < Sh::kRows && row_valid(tid)) a.lse_part[out_row(tid) * ns + split] = -INFINITY;
    return;
  }
  const int t_last = t_end - 1;

  // q rows of this wave as the B operand of the score MFMA: lane (col, grp) holds row
  // 16 * wave + col, columns 32 * c + 8 * grp .. + 7 (zero past the last query).
  bf16x8 qop[Sh::kQSteps];
  {
    const bool rv = row_valid(my_row);
    const uint16_t* qr = a.q + out_row(rv ? my_row : my_row % G) * D;  // block's first query
#pragma unroll
    for (int c = 0; c < Sh::kQSteps; ++c) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qr + 32 * c + 8 * grp);
      const u32x4 z = {0u, 0u, 0u, 0u};
      qop[c] = __builtin_bit_cast(bf16x8, rv ? v : z);
    }
  }
  // Scores are scaled by sl2 = |scale * log2 e| (at least FLT_MIN, so that -inf * sl2 stays -inf;
  // a zero scale then gives scores of 0 up to 1e-38 relative); a negative scale flips the sign of q
  // instead, so that the softmax can take the maximum of the raw scores and scale it once.
  const float sl2 = fmaxf(fabsf(a.scale_log2), 1.17549435e-38f);
  if (a.scale_log2 < 0.f) {
#pragma unroll
    for (int c = 0; c < Sh::kQSteps; ++c) {
      const u32x4 f = {0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
      qop[c] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, qop[c]) ^ f);
    }
  }

  // Staging of one step's tile (list entries e, e + 1): thread tid loads chunks
  // tid + kThreads * k, i.e. key row k * kKeysPerPass + tid / kChunks, chunk tid % kChunks. The
  // first kLoads / 2 loads are entry e's, the rest entry e + 1's; a thread's byte offsets inside
  // a tile are the same every step, so each load is a uniform tile address plus a fixed offset.
  const int ld_key0 = tid / Sh::kChunks;
  const int ld_chunk = tid % Sh::kChunks;
  constexpr int kHalf = Sh::kLoads / 2;
  auto ld_key = [&](int k) { return k * Sh::kKeysPerPass + ld_key0; };
  uint32_t ld_off[Sh::kLoads];
#pragma unroll
  for (int k = 0; k < Sh::kLoads; ++k)
    ld_off[k] = (uint32_t)(((ld_key(k) % kTile) * D + 8 * ld_chunk) * 2);
  u32x4 stk[Sh::kLoads];
  u32x4 stv[SHARED ? 1 : Sh::kLoads];
  // Element offset of entry v's tile (page id pid) in a pool, and whether its page is valid.
  const uint64_t page_elems = (uint64_t)a.num_kv_heads * S * D;  // one page of all KV heads
  const uint64_t head_elems = (uint64_t)kvh * S * D;              // this KV head within a page
  auto entry_base = [&](int v, int pid, bool& page_ok) -> size_t {
    const int pc = phys_tile(v < t_end ? v : t_last);
    page_ok = (unsigned)pid < (unsigned)a.num_pages;
    const uint32_t pg = page_ok ? (uint32_t)pid : 0u;
    const int within = pc - page_of(pc) * tpp;
    return pg * page_elems + head_elems + (uint32_t)(within * kTile * D);
  };
  auto entry_pid = [&](int v) -> int32_t {
    const int pc = phys_tile(v < t_end ? v : t_last);
    return load_uniform(table_row, page_of(pc));
  };
  // Page ids of entries e, e + 1 as a vector (lane u holds entry e + (u & 1)), fetched a step
  // ahead and read back with v_readlane.
  auto pid_vector = [&](int e) -> int32_t {
    const int v = e + (lane & 1);
    const int pc = phys_tile(v < t_end ? v : t_last);
    return table_row[page_of(pc)];
  };
  // mats: bit 0 the K tile, bit 1 the V tile (no V tile when SHARED).
  auto issue_loads = [&](int e, int pid0, int pid1, bool* page_ok, int mats, int k_begin = 0,
                         int k_end = Sh::kLoads) {
    const size_t base0 = entry_base(e, pid0, page_ok[0]);
    const size_t base1 = entry_base(e + 1, pid1, page_ok[1]);
    const char* k0 = reinterpret_cast<const char*>(a.k_pool + base0);
    const char* k1 = reinterpret_cast<const char*>(a.k_pool + base1);
    const char* v0 = reinterpret_cast<const char*>(a.v_pool + base0);
    const char* v1 = reinterpret_cast<const char*>(a.v_pool + base1);
#pragma unroll
    for (int k = 0; k < Sh::kLoads; ++k) {
      if (k < k_begin || k >= k_end) continue;
      if (mats & 1) stk[k] = *reinterpret_cast<const u32x4*>((k < kHalf ? k0 : k1) + ld_off[k]);
      if constexpr (!SHARED)
        if (mats & 2) stv[k] = *reinterpret_cast<const u32x4*>((k < kHalf ? v0 : v1) + ld_off[k]);
    }
  };
  // Key t of entry v is in the union of the block's ranges (read at all) iff its page is valid,
  // v < t_end, t < n and (t >= lo or t < sk). An entry is full when all its 16 keys are. Entries
  // [0, f_a) (sink tiles of sk keys) and [f_b, f_c) (window tiles from the first one starting at
  // lo or later) are full whenever their pages are valid. The ranges are conservative (a full
  // entry outside them takes the exact per-key path) and let a step of the 64-row workgroups test
  // two integers instead of the per-entry bounds; the 128-row kernel keeps the per-entry tests, with
  // which the compiler schedules its P.V reads better (measured).
  const int f_a = min(min(st, sk / kTile), min(n / kTile, t_end));
  const int f_b = max(st, (lo + kTile - 1) / kTile - shift);
  const int f_c = min(n / kTile - shift, t_end);
  auto pair_in = [](int e, int ra, int rb, int rc) {  // entries e and e + 1 in [0, ra) or [rb, rc)
    return (e + 1 < ra) | ((e >= rb) & (e + 1 < rc));
  };
  auto entry_full = [&](int v, bool page_ok) {
    const int t0 = phys_tile(v < t_end ? v : t_last) * kTile;
    // (Bitwise: every term is cheap, and a chain of short-circuit branches costs more.)
    return (v < t_end) & page_ok & (t0 + kTile <= n) & ((t0 >= lo) | (t0 + kTile <= sk));
  };
  // Stores the staged tile; keys outside the union are then overwritten with zeros (only entries
  // at the edges of the ranges, or of invalid pages, have any). Returns whether both are full.
  auto store_tile = [&](int buf, int e, const bool* page_ok, int mats) -> bool {
    // K rows swizzled (score reads: 16 keys, one column); V rows in their own buffer, swizzled
    // for row reads or plain for transpose reads (16 keys, 16 columns).
    const int v_chunk = kTr ? ld_chunk : swz<D>(ld_chunk);
#pragma unroll
    for (int k = 0; k < Sh::kLoads; ++k) {
      if (mats & 1)
        *reinterpret_cast<u32x4*>(&KB(buf)[ld_key(k)][8 * swz<D>(ld_chunk)]) = stk[k];
      if constexpr (!SHARED)
        if (mats & 2) *reinterpret_cast<u32x4*>(&VB(buf)[ld_key(k)][8 * v_chunk]) = stv[k];
    }
    const bool full = pair_in(e, f_a, f_b, f_c) & page_ok[0] & page_ok[1];
    if (!full) {
#pragma unroll
      for (int k = 0; k < Sh::kLoads; ++k) {
        const int key = ld_key(k);
        const int v = e + (k < kHalf ? 0 : 1);
        const int t = phys_tile(v < t_end ? v : t_last) * kTile + key % kTile;
        const bool in = (v < t_end) & page_ok[k < kHalf ? 0 : 1] & (t < n) & ((t >= lo) | (t < sk));
        if (!in) {
          const u32x4 z = {0u, 0u, 0u, 0u};
          if (mats & 1) *reinterpret_cast<u32x4*>(&KB(buf)[key][8 * swz<D>(ld_chunk)]) = z;
          if constexpr (!SHARED)
            if (mats & 2) *reinterpret_cast<u32x4*>(&VB(buf)[key][8 * v_chunk]) = z;
        }
      }
    }
    return full;
  };

  // Direct staging (head_dim 512): wave w fetches key rows kRowsW w .. kRowsW (w + 1) - 1 of the
  // step's two entries (rows 0-15 entry e, 16-31 entry e + 1), K and V, one instruction per row;
  // lane l fetches the 16-byte chunk that belongs in slot l of the row (swizzled for K, in order
  // for V). A wave's rows all belong to one entry, so it needs that entry's address only.
  constexpr int kRowsW = kStepKeys / kWaves;
  static_assert(kTile % kRowsW == 0, "a wave's staging rows lie in one entry");
  auto issue_dma = [&](int b2, int e, int pid0, int pid1, bool* page_ok) {
    const int ent = (kRowsW * wave) / kTile;
    bool ok_own;
    const size_t base = entry_base(e + ent, ent ? pid1 : pid0, ok_own);
    page_ok[0] = (unsigned)pid0 < (unsigned)a.num_pages;
    page_ok[1] = (unsigned)pid1 < (unsigned)a.num_pages;
#pragma unroll
    for (int j = 0; j < kRowsW; ++j) {
      const int r = kRowsW * wave + j;
      const size_t rb = base + (size_t)(r % kTile) * D;
      dma16(a.k_pool + rb + 8 * swz<D>(lane), &KB(b2)[r][0]);
      if constexpr (!SHARED) dma16(a.v_pool + rb + 8 * lane, &VB(b2)[r][0]);
    }
  };
  // Once this thread's fetches have landed: zeros over the rows it fetched whose key is outside
  // the union (or on an invalid page). Returns whether both entries are full.
  auto dma_zero = [&](int b2, int e, const bool* page_ok) -> bool {
    const bool full = entry_full(e, page_ok[0]) & entry_full(e + 1, page_ok[1]);
    if (!full) {
#pragma unroll
      for (int j = 0; j < kRowsW; ++j) {
        const int r = kRowsW * wave + j;
        const int v = e + r / kTile;
        const int t = phys_tile(v < t_end ? v : t_last) * kTile + r % kTile;
        const bool in = (v < t_end) & page_ok[r / kTile] & (t < n) & ((t >= lo) | (t < sk));
        if (!in) {
          const u32x4 z = {0u, 0u, 0u, 0u};
          *reinterpret_cast<u32x4*>(&KB(b2)[r][8 * lane]) = z;
          if constexpr (!SHARED) *reinterpret_cast<u32x4*>(&VB(b2)[r][8 * lane]) = z;
        }
      }
    }
    return full;
  };

  // Rows of this wave that exist attend every key in [wave_lo, wave_n) (sinks aside): a step whose
  // keys all lie there, in two full entries, needs no per-row mask.
  int wave_n = row_valid(my_row) ? row_n : INT32_MAX;
  int wave_lo = row_valid(my_row) ? row_lo : 0;
#pragma unroll
  for (int x = 1; x < 16; x <<= 1) {
    wave_n = min(wave_n, __shfl_xor(wave_n, x));
    wave_lo = max(wave_lo, __shfl_xor(wave_lo, x));
  }
  wave_n = __builtin_amdgcn_readfirstlane(wave_n);
  wave_lo = __builtin_amdgcn_readfirstlane(wave_lo);
  // Entries whose keys every existing row of this wave attends, in the form of the full ranges:
  // sink tiles below sk (<= sink) and n' = min(n, wave_n), window tiles from the first one starting
  // at max(lo, wave_lo) and ending by n'. A step of two such entries on valid pages needs no mask.
  const int n_w = min(n, wave_n);
  const int i_a = min(min(st, sk / kTile), min(n_w / kTile, t_end));
  const int i_b = max(st, (max(lo, wave_lo) + kTile - 1) / kTile - shift);
  const int i_c = min(n_w / kTile - shift, t_end);

  // Prologue: tile of step 0 into LDS buffer 0, the tile of step 1 in flight.
  bool ok_cur[2], ok_next[2], ok_nxt[2];
  int32_t pid_next;
  bool full_cur;
  if constexpr (kDmaD) {
    issue_dma(0, t_begin, entry_pid(t_begin), entry_pid(t_begin + 1), ok_cur);
    pid_next = pid_vector(t_begin + 2);
    __builtin_amdgcn_s_waitcnt(0);
    full_cur = dma_zero(0, t_begin, ok_cur);
    issue_dma(1, t_begin + 2, __builtin_amdgcn_readlane(pid_next, 0),
              __builtin_amdgcn_readlane(pid_next, 1), ok_nxt);
    pid_next = pid_vector(t_begin + 4);
  } else {
    issue_loads(t_begin, entry_pid(t_begin), entry_pid(t_begin + 1), ok_next, 3);
    pid_next = pid_vector(t_begin + 2);
    full_cur = store_tile(0, t_begin, ok_next, 3);
    ok_cur[0] = ok_next[0];
    ok_cur[1] = ok_next[1];
    issue_loads(t_begin + 2, __builtin_amdgcn_readlane(pid_next, 0),
                __builtin_amdgcn_readlane(pid_next, 1), ok_next, 3);
    pid_next = pid_vector(t_begin + 4);
  }
  __syncthreads();

  float m_run = -INFINITY;  // running max (base 2) of row my_row
  float l_run = 0.f;        // running sum of exp2(s - m_run)
  f32x4 acc[Sh::kLaneCols];  // O[rows 16 * wave + 4 * grp + i][col * kLaneCols + e] = acc[e][i]
#pragma unroll
  for (int e = 0; e < Sh::kLaneCols; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};

  int buf = 0;
  for (int e0 = t_begin; e0 < t_end; e0 += 2) {
    // The K half of the next step's tile (in registers since the previous step) into the other
    // buffer, whose last readers finished before the previous step's barrier. Its registers then
    // take the fetch of the tile after it, issued between the score batches. (After the last step
    // this stages clamped re-reads of the last entry, which are never used.)
    bool full_nxt = false;
    if constexpr (kEarlyStore) {
      full_nxt = store_tile(buf ^ 1, e0 + 2, ok_next, kSplitStore ? 1 : 3);
      ok_nxt[0] = ok_next[0];
      ok_nxt[1] = ok_next[1];
    }

    // Scores S^T for the two entries: lane (col, grp) gets keys 4 * grp + i of entry e0 + g
    // for row my_row.
    // The K operands are read kKAhead at a time, all issued before the MFMAs that use them.
    f32x4 sc[2];
    if constexpr (kSetPrio) __builtin_amdgcn_s_setprio(1);
    if constexpr (kPipeK > 0) {
      // One accumulator per entry, the two entries' MFMAs alternating (MFMA i: entry i % 2,
      // columns 32 (i / 2) ..); operand i + kPipeK is read right after MFMA i issues, so kPipeK
      // reads are in flight throughout. Scheduling barriers keep that order.
      constexpr int kN = 2 * Sh::kQSteps;
      auto k_read = [&](int i) {
        return *reinterpret_cast<const bf16x8*>(
            &KB(buf)[kTile * (i & 1) + col][8 * swz<D>(4 * (i >> 1) + grp)]);
      };
      sc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
      sc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
      bf16x8 kb[kPipeKN];
#pragma unroll
      for (int i = 0; i < kPipeK; ++i) kb[i] = k_read(i);
#pragma unroll
      for (int i = 0; i < kN; ++i) {
        sc[i & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[i % kPipeKN], qop[i >> 1], sc[i & 1],
                                                            0, 0, 0);
        if (i + kPipeK < kN) kb[i % kPipeKN] = k_read(i + kPipeK);
        if (DECODE_ATTN_PREFILL_KPIPE_SB) __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      f32x4 p0 = {0.f, 0.f, 0.f, 0.f}, p1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c0 = 0; c0 < Sh::kQSteps; c0 += kKAhead) {
        bf16x8 kk[kKAhead];
#pragma unroll
        for (int c = 0; c < kKAhead; ++c)
          kk[c] = *reinterpret_cast<const bf16x8*>(
              &KB(buf)[kTile * g + col][8 * swz<D>(4 * (c0 + c) + grp)]);
        if constexpr (kEarlyStore && kSplitStore && kSpreadK) {
          // A share of the next-but-one tile's K loads behind this batch's LDS reads.
          constexpr int kBatches = 2 * Sh::kQSteps / kKAhead;
          constexpr int kPer = (Sh::kLoads + kBatches - 1) / kBatches;
          const int bi = g * (Sh::kQSteps / kKAhead) + c0 / kKAhead;
          issue_loads(e0 + 4, __builtin_amdgcn_readlane(pid_next, 0),
                      __builtin_amdgcn_readlane(pid_next, 1), ok_next, 1, bi * kPer,
                      bi * kPer + kPer);
        }
#pragma unroll
        for (int c = 0; c < kKAhead; c += 2) {
          p0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk[c], qop[c0 + c], p0, 0, 0, 0);
          p1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk[c + 1], qop[c0 + c + 1], p1, 0, 0, 0);
        }
      }
      sc[g] = p0 + p1;
    }
    }

    if constexpr (kSetPrio) __builtin_amdgcn_s_setprio(0);
    // Fetch of the tile two steps ahead; it lands during the softmax, P.V and the barrier.
    if constexpr (kEarlyStore) {
      const int pid0 = __builtin_amdgcn_readlane(pid_next, 0);
      const int pid1 = __builtin_amdgcn_readlane(pid_next, 1);
      if constexpr (kSplitStore) {
        // The V half of the next tile goes to LDS only now (P.V of the next step is its first
        // reader): the score reads above queued behind the K half's writes only, and these drain
        // during the softmax.
        if constexpr (!kSpreadK) issue_loads(e0 + 4, pid0, pid1, ok_next, 1);
        store_tile(buf ^ 1, e0 + 2, ok_nxt, 2);
        if constexpr (!kSpreadV) issue_loads(e0 + 4, pid0, pid1, ok_next, 2);
      } else {
        issue_loads(e0 + 4, pid0, pid1, ok_next, 3);
      }
      if constexpr (!(kSplitStore && kSpreadV)) pid_next = pid_vector(e0 + 6);
    }

    // Masks and online softmax of row my_row over the 32 keys.
    float s2[2][4];
    float mt = -INFINITY;
    const int ta = phys_tile(e0 < t_end ? e0 : t_last) * kTile;
    const int tb = phys_tile(e0 + 1 < t_end ? e0 + 1 : t_last) * kTile;
    const bool unmasked =
        kDmaD ? full_cur & ((ta > tb ? ta : tb) + kTile <= wave_n) &
                    ((ta >= wave_lo) | (ta + kTile <= sink)) & ((tb >= wave_lo) | (tb + kTile <= sink))
              : pair_in(e0, i_a, i_b, i_c) & ok_cur[0] & ok_cur[1];
    // s2: the raw scores, -inf where masked; sl2 > 0, so their maximum times sl2 is the maximum of
    // the scaled scores.
    if (unmasked) {
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s2[g][i] = sc[g][i];
          mt = fmaxf(mt, s2[g][i]);
        }
    } else {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int v = e0 + g;
        const int t0 = (g == 0 ? ta : tb) + 4 * grp;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = t0 + i;
          const bool att = (v < t_end) & ok_cur[g] & (t < row_n) & ((t >= row_lo) | (t < sink));
          s2[g][i] = att ? sc[g][i] : -INFINITY;
          mt = fmaxf(mt, s2[g][i]);
        }
      }
    }
    mt = max_xor16_32(mt) * sl2;
    const float m_new = fmaxf(m_run, mt);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float p[2][4];
    float ps = 0.f;
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[g][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s2[g][i], sl2, -m_use));
        ps += p[g][i];
      }
    ps = sum_xor16_32(ps);
    l_run = l_run * alpha + ps;
    m_run = m_new;
    if (__any(alpha != 1.f)) {
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * grp + i);
#pragma unroll
      for (int e = 0; e < Sh::kLaneCols; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[e][i] *= al[i];
    }
    // P as the A operand: row my_row, reduction index 8 * grp + j <-> key 4 * grp + j of entry
    // e0 (j < 4) or of entry e0 + 1 (j >= 4).
    const u32x4 pa = {pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]),
                      pack_bf16x2(p[1][0], p[1][1]), pack_bf16x2(p[1][2], p[1][3])};
    const bf16x8 pop = __builtin_bit_cast(bf16x8, pa);

    if constexpr (kSetPrio) __builtin_amdgcn_s_setprio(1);
    if constexpr (kTr) {
      // P.V by transpose reads: MFMA e covers output columns 16 e .. 16 e + 15, lane (col, grp)
      // column 16 e + col. Lane col of group grp addresses key row 4 grp + col / 4 (then
      // 16 + 4 grp + col / 4), columns 16 e + 4 (col % 4) .. + 3; the transpose hands it
      // keys 4 grp + c (then 16 + 4 grp + c), c < 4, of its own column: B's reduction slots
      // 8 grp + j in P's key order.
      const int r1 = 4 * grp + (col >> 2);
      const uint16_t* const v1 = SHARED ? &KB(buf)[r1][0] : &VB(buf)[r1][0];
      const uint16_t* const v2 = SHARED ? &KB(buf)[kTile + r1][0] : &VB(buf)[kTile + r1][0];
#pragma unroll
      for (int cg = 0; cg < Sh::kVGroups; ++cg) {
        u32x2 lo[8], hi[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const int d = 16 * (8 * cg + x) + 4 * (col & 3);
          const int off = SHARED ? 8 * swz<D>(d >> 3) + (d & 7) : d;
          lo[x] = lds_read_tr16(v1 + off);
          hi[x] = lds_read_tr16(v2 + off);
        }
        if constexpr (kEarlyStore && kSplitStore && kSpreadV) {
          constexpr int kPer = (Sh::kLoads + Sh::kVGroups - 1) / Sh::kVGroups;
          issue_loads(e0 + 4, __builtin_amdgcn_readlane(pid_next, 0),
                      __builtin_amdgcn_readlane(pid_next, 1), ok_next, 2, cg * kPer,
                      cg * kPer + kPer);
          if (cg == Sh::kVGroups - 1) pid_next = pid_vector(e0 + 6);
        }
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const u32x4 bv = {lo[x][0], lo[x][1], hi[x][0], hi[x][1]};
          const int e = 8 * cg + x;
          acc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pop, __builtin_bit_cast(bf16x8, bv),
                                                           acc[e], 0, 0, 0);
        }
      }
    } else {
      // P.V: lane (col, grp) reads, for each 8-column group cg of its columns, the 8 keys of its
      // reduction slots (key rows 4 * grp + j and 16 + 4 * grp + j, j < 4) and transposes them
      // into 8 B operands (one per column).
#pragma unroll
      for (int cg = 0; cg < Sh::kVGroups; ++cg) {
        const int chunk = swz<D>(col * Sh::kVGroups + cg);
        u32x4 vr[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int key = (j < 4 ? 0 : kTile) + 4 * grp + (j & 3);
          vr[j] = *reinterpret_cast<const u32x4*>(SHARED ? &KB(buf)[key][8 * chunk]
                                                         : &VB(buf)[key][8 * chunk]);
        }
        if constexpr (kEarlyStore && kSplitStore && kSpreadV) {
          // A share of the next-but-one tile's V loads between the P.V column groups, behind this
          // group's LDS reads.
          constexpr int kPer = (Sh::kLoads + Sh::kVGroups - 1) / Sh::kVGroups;
          issue_loads(e0 + 4, __builtin_amdgcn_readlane(pid_next, 0),
                      __builtin_amdgcn_readlane(pid_next, 1), ok_next, 2, cg * kPer,
                      cg * kPer + kPer);
          if (cg == Sh::kVGroups - 1) pid_next = pid_vector(e0 + 6);
        }
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const u32x4 be = {__builtin_amdgcn_perm(vr[1][d], vr[0][d], 0x05040100u),
                            __builtin_amdgcn_perm(vr[3][d], vr[2][d], 0x05040100u),
                            __builtin_amdgcn_perm(vr[5][d], vr[4][d], 0x05040100u),
                            __builtin_amdgcn_perm(vr[7][d], vr[6][d], 0x05040100u)};
          const u32x4 bo = {__builtin_amdgcn_perm(vr[1][d], vr[0][d], 0x07060302u),
                            __builtin_amdgcn_perm(vr[3][d], vr[2][d], 0x07060302u),
                            __builtin_amdgcn_perm(vr[5][d], vr[4][d], 0x07060302u),
                            __builtin_amdgcn_perm(vr[7][d], vr[6][d], 0x07060302u)};
          const int e = 8 * cg + 2 * d;
          acc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pop, __builtin_bit_cast(bf16x8, be),
                                                           acc[e], 0, 0, 0);
          acc[e + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              pop, __builtin_bit_cast(bf16x8, bo), acc[e + 1], 0, 0, 0);
        }
      }
    }

    if constexpr (kSetPrio) __builtin_amdgcn_s_setprio(0);
    if constexpr (kDmaD) {  // the next tile has landed in the other buffer: mask its edges
      __builtin_amdgcn_s_waitcnt(0);
      full_nxt = dma_zero(buf ^ 1, e0 + 2, ok_nxt);
    } else if constexpr (!kEarlyStore) {  // stage the next tile and fetch the one after it here
      full_nxt = store_tile(buf ^ 1, e0 + 2, ok_next, 3);
      ok_nxt[0] = ok_next[0];
      ok_nxt[1] = ok_next[1];
      issue_loads(e0 + 4, __builtin_amdgcn_readlane(pid_next, 0),
                  __builtin_amdgcn_readlane(pid_next, 1), ok_next, 3);
      pid_next = pid_vector(e0 + 6);
    }
    // One barrier publishes the other buffer and retires this step's reads of this one.
    full_cur = full_nxt;
    ok_cur[0] = ok_nxt[0];
    ok_cur[1] = ok_nxt[1];
    __syncthreads();
    if constexpr (kDmaD) {  // this buffer is free: the tile after the next one into it
      // (Past the split's last entry this re-fetches that entry's rows, in bounds and unused;
      // issuing it unconditionally keeps the compiler from waiting for it before the next
      // step's LDS reads, which it does when the fetch sits under a branch.)
      issue_dma(buf, e0 + 4, __builtin_amdgcn_readlane(pid_next, 0),
                __builtin_amdgcn_readlane(pid_next, 1), ok_nxt);
      pid_next = pid_vector(e0 + 6);
    }
    buf ^= 1;
  }
  // No fetch into LDS may still be landing when the workgroup ends and its LDS is reassigned.
  if constexpr (kDmaD) __builtin_amdgcn_s_waitcnt(0);

  // Normalise and write: lane (col, grp) holds rows 16 * wave + 4 * grp + i, columns
  // col * kLaneCols .. + kLaneCols.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * wave + 4 * grp + i;
    const float lh = __shfl(l_run, 4 * grp + i);
    const float inv = lh > 0.f ? 1.f / lh : 0.f;
    if (row_valid(r)) {
      float* const row_out = a.o_part + (out_row(r) * ns + split) * D;
      if constexpr (kTr) {
        // Column 16 e + col: the 16 lanes of a group write 64 contiguous bytes per e.
#pragma unroll
        for (int e = 0; e < Sh::kLaneCols; ++e) row_out[16 * e + col] = acc[e][i] * inv;
      } else {
        float* dst = row_out + col * Sh::kLaneCols;
#pragma unroll
        for (int e = 0; e < Sh::kLaneCols; e += 4) {
          const f32x4 v4 = {acc[e][i] * inv, acc[e + 1][i] * inv, acc[e + 2][i] * inv,
                            acc[e + 3][i] * inv};
          *reinterpret_cast<f32x4*>(dst + e) = v4;
        }
      }
    }
  }
  if (grp == 0 && row_valid(my_row)) {
    const float lse = (m_run == -INFINITY) ? -INFINITY : (m_run + __log2f(l_run)) * kLn2;
    a.lse_part[out_row(my_row) * ns + split] = lse;
  }
}

template <int D, int G, int ROWS>
hipError_t launch(const Stage1Args& args, bool shared, int batch, hipStream_t stream) {
  dim3 grid(args.num_splits * args.num_qblocks, args.num_kv_heads, batch);
  void* kargs[] = {const_cast<Stage1Args*>(&args)};
  const void* fn = shared ? reinterpret_cast<const void*>(&prefill_kernel<D, G, true, ROWS>)
                          : reinterpret_cast<const void*>(&prefill_kernel<D, G, false, ROWS>);
  return hipLaunchKernel(fn, grid, dim3(PShape<D, ROWS>::kThreads), kargs, 0, stream);
}

template <int D, int G>
hipError_t launch_rows(const Stage1Args& args, bool shared, int batch, hipStream_t stream) {
  if constexpr (D == 512)
    if (prefill_rows(D, G, args.q_len) == kPrefillWideRows)
      return launch<D, G, kPrefillWideRows>(args, shared, batch, stream);
  return launch<D, G, kPrefillRows>(args, shared, batch, stream);
}

template <int D>
hipError_t launch_d(const Stage1Args& args, int group_size, bool shared, int batch,
                    hipStream_t stream) {
  switch (group_size) {
    case 1: return launch_rows<D, 1>(args, shared, batch, stream);
    case 2: return launch_rows<D, 2>(args, shared, batch, stream);
    case 4: return launch_rows<D, 4>(args, shared, batch, stream);
    case 8: return launch_rows<D, 8>(args, shared, batch, stream);
    case 16: return launch_rows<D, 16>(args, shared, batch, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_prefill(const Stage1Args& args, int head_dim, int group_size, int batch,
                          hipStream_t stream) {
  const bool shared = args.k_pool == args.v_pool;
  switch (head_dim) {
    case 256: return launch_d<256>(args, group_size, shared, batch, stream);
    case 512: return launch_d<512>(args, group_size, shared, batch, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace decode_attn
