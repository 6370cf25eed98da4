// decode_attn.cpp — the extern "C" entry points of libdecode_attn.so: planning, host-side argument
// checks and the two kernel launches. Declared and documented in include/decode_attn.h.

#include "decode_attn.h"

#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cmath>
#include <cstdint>

#include "internal.h"

// Single-token decode at head_dim 256 with G <= 4 and separate pools runs on the key-split
// stage-1 kernel (stage1_ks.hip); 0 keeps it on the column-split kernel of stage1.hip (for A/B
// builds).
#ifndef DECODE_ATTN_KEYSPLIT
#define DECODE_ATTN_KEYSPLIT 1
#endif
// Stage-1 kernels may fetch the page ids of the chunk the plan's max_ctx_len gives while the
// sequence's length is in flight (kept when the length gives the same chunk); 0 disables it.
#ifndef DECODE_ATTN_SPEC
#define DECODE_ATTN_SPEC 1
#endif
// ... and, with several splits, when they give at most one key-split workgroup per CU.
#ifndef DECODE_ATTN_KS_SPLITS
#define DECODE_ATTN_KS_SPLITS 1
#endif

namespace decode_attn {
namespace {

// A layer the key-split stage-1 kernel serves (whole tiles per wave, one merge per workgroup).
bool keysplit_layer(int head_dim, int group_size, int q_len, int sink, bool shared) {
  return DECODE_ATTN_KEYSPLIT &&
         stage1_keysplit_supported(head_dim, group_size, q_len, sink, shared);
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];  // 0 = not queried yet

int query_num_cus(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DECODE_ATTN_ERR_HIP;
  if (dev >= 0 && dev < kMaxDevices) {
    const int cached = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cached > 0) {
      *cus = cached;
      return DECODE_ATTN_OK;
    }
  }
  int value = 0;
  if (hipDeviceGetAttribute(&value, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      value <= 0)
    return DECODE_ATTN_ERR_HIP;
  if (dev >= 0 && dev < kMaxDevices) g_cu_count[dev].store(value, std::memory_order_relaxed);
  *cus = value;
  return DECODE_ATTN_OK;
}

uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

// Query tokens per sequence of a resolved problem (0 means 1).
int q_len_of(const decode_attn_problem& p) { return p.q_len > 1 ? p.q_len : 1; }

// Query blocks per (sequence, kv head): a stage-1 workgroup serves 16 or 32 rows of G heads.
int qblocks_of(const decode_attn_problem& p, int group_size) {
  return stage1_query_blocks(group_size, q_len_of(p), p.head_dim);
}

// Workspace layout: o_part [B, L, Hq, ns, D] fp32, then (256-byte aligned) lse [B, L, Hq, ns]
// fp32.
void workspace_layout(const decode_attn_problem& p, int num_splits, uint64_t* lse_offset,
                      uint64_t* total) {
  const uint64_t rows = (uint64_t)p.batch * (uint64_t)q_len_of(p) * (uint64_t)p.num_q_heads *
                        (uint64_t)num_splits;
  *lse_offset = align_up(rows * (uint64_t)p.head_dim * 4u, 256);
  *total = align_up(*lse_offset + rows * 4u, 256);
}

// Workspace of a layer call (decode_attn_global / _sliding): the stage workspace, or with one
// split only the lse plane [B, L, Hq] (stage 1 writes out in place, and its lse into the
// workspace at offset 0 when the caller passes no lse_out).
uint64_t layer_workspace(const decode_attn_problem& p, int num_splits, uint64_t stage_total) {
  if (num_splits != 1) return stage_total;
  const uint64_t rows = (uint64_t)p.batch * (uint64_t)q_len_of(p) * (uint64_t)p.num_q_heads;
  return align_up(rows * 4u, 256);
}

bool aligned(const void* ptr, uintptr_t a) { return ((uintptr_t)ptr % a) == 0; }

// Checks a plan made by decode_attn_plan and not altered since.
int check_plan(const decode_attn_plan_t* plan) {
  if (plan == nullptr) return DECODE_ATTN_ERR_NULL;
  if (plan->magic != kPlanMagic) return DECODE_ATTN_ERR_PLAN;
  const decode_attn_problem& p = plan->problem;
  if (p.batch < 1 || p.num_q_heads < 1 || p.num_kv_heads < 1 ||
      p.num_q_heads % p.num_kv_heads != 0 || p.page_size < kTile || p.page_size % kTile != 0 ||
      p.max_pages_per_seq < 1 || p.num_pages < 1 || p.window < 0 || p.sink < 0 ||
      p.q_len < 0 || p.q_len > DECODE_ATTN_MAX_Q_LEN ||
      (p.values_are_keys != 0 && p.values_are_keys != 1))
    return DECODE_ATTN_ERR_PLAN;
  if (plan->group_size != p.num_q_heads / p.num_kv_heads) return DECODE_ATTN_ERR_PLAN;
  if (!stage1_supported(p.head_dim, plan->group_size)) return DECODE_ATTN_ERR_PLAN;
  if (plan->kind != (p.window > 0 ? 2 : 1)) return DECODE_ATTN_ERR_PLAN;
  if (plan->num_splits < 1 || plan->num_splits > DECODE_ATTN_MAX_SPLITS_LIMIT)
    return DECODE_ATTN_ERR_PLAN;
  uint64_t lse_off = 0, total = 0;
  workspace_layout(p, plan->num_splits, &lse_off, &total);
  if (plan->workspace_bytes != total || plan->partial_lse_offset != lse_off ||
      plan->layer_workspace_bytes != layer_workspace(p, plan->num_splits, total))
    return DECODE_ATTN_ERR_PLAN;
  return DECODE_ATTN_OK;
}

// needed: the workspace bytes the call requires (the stage or the layer figure of the plan).
int check_stage1_args(const decode_attn_plan_t* plan, const void* q, const void* k_pool,
                      const void* v_pool, const int32_t* block_table, const int32_t* ctx_lens,
                      int32_t batch, float scale, const void* workspace,
                      uint64_t workspace_bytes, uint64_t needed) {
  if (batch < 0 || batch > plan->problem.batch) return DECODE_ATTN_ERR_SHAPE;
  if (!std::isfinite(scale)) return DECODE_ATTN_ERR_SHAPE;
  if (batch == 0) return DECODE_ATTN_OK;
  if (!q || !k_pool || !v_pool || !block_table || !ctx_lens || !workspace)
    return DECODE_ATTN_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(workspace, 16) ||
      !aligned(block_table, 4) || !aligned(ctx_lens, 4))
    return DECODE_ATTN_ERR_ALIGN;
  if (plan->problem.values_are_keys && k_pool != v_pool) return DECODE_ATTN_ERR_SHAPE;
  if (workspace_bytes < needed) return DECODE_ATTN_ERR_WORKSPACE;
  return DECODE_ATTN_OK;
}

int check_stage2_args(const decode_attn_plan_t* plan, int32_t batch, const void* workspace,
                      uint64_t workspace_bytes, const float* out, const float* lse_out,
                      uint64_t needed) {
  if (batch < 0 || batch > plan->problem.batch) return DECODE_ATTN_ERR_SHAPE;
  if (batch == 0) return DECODE_ATTN_OK;
  if (!workspace || !out) return DECODE_ATTN_ERR_NULL;
  if (!aligned(workspace, 16) || !aligned(out, 16) || (lse_out && !aligned(lse_out, 4)))
    return DECODE_ATTN_ERR_ALIGN;
  if (workspace_bytes < needed) return DECODE_ATTN_ERR_WORKSPACE;
  return DECODE_ATTN_OK;
}

// Stage 1 writing its partials to o_part / lse_part ([B, L, Hq, num_splits, D] and
// [B, L, Hq, num_splits] fp32).
int run_stage1(const decode_attn_plan_t* plan, const void* q, const void* k_pool,
               const void* v_pool, const int32_t* block_table, const int32_t* ctx_lens,
               int32_t batch, float scale, float* o_part, float* lse_part, hipStream_t stream) {
  const decode_attn_problem& p = plan->problem;
  Stage1Args a;
  a.q = static_cast<const uint16_t*>(q);
  a.k_pool = static_cast<const uint16_t*>(k_pool);
  a.v_pool = static_cast<const uint16_t*>(v_pool);
  a.block_table = block_table;
  a.ctx_lens = ctx_lens;
  a.o_part = o_part;
  a.lse_part = lse_part;
  a.num_q_heads = p.num_q_heads;
  a.num_kv_heads = p.num_kv_heads;
  a.page_size = p.page_size;
  a.max_pages_per_seq = p.max_pages_per_seq;
  a.num_pages = p.num_pages;
  a.window = p.window;
  a.sink = p.window > 0 ? p.sink : 0;
  a.q_len = q_len_of(p);
  a.num_qblocks = qblocks_of(p, plan->group_size);
  a.num_splits = plan->num_splits;
  a.scale_log2 = scale * 1.442695040888963407360f;
  a.spec_ctx = DECODE_ATTN_SPEC ? p.max_ctx_len : 0;
  hipError_t err;
  if (stage1_use_prefill(plan->group_size, a.q_len))
    err = launch_prefill(a, p.head_dim, plan->group_size, batch, stream);
  else if ((plan->num_splits == 1 ||
            (DECODE_ATTN_KS_SPLITS && (int64_t)plan->num_splits * p.batch * p.num_kv_heads <=
                                          (p.num_cus > 0 ? p.num_cus : 256))) &&
           keysplit_layer(p.head_dim, plan->group_size, a.q_len, a.sink, k_pool == v_pool))
    err = launch_stage1_keysplit(a, plan->group_size, batch, stream);
  else
    err = launch_stage1(a, p.head_dim, plan->group_size, batch, stream);
  if (err != hipSuccess) return DECODE_ATTN_ERR_HIP;
  return DECODE_ATTN_OK;
}

int run_stage2(const decode_attn_plan_t* plan, int32_t batch, const void* workspace, float* out,
               float* lse_out, hipStream_t stream) {
  const decode_attn_problem& p = plan->problem;
  Stage2Args a;
  a.o_part = static_cast<const float*>(workspace);
  a.lse_part =
      reinterpret_cast<const float*>(static_cast<const char*>(workspace) + plan->partial_lse_offset);
  a.out = out;
  a.lse_out = lse_out;
  a.num_q_heads = p.num_q_heads;
  a.head_dim = p.head_dim;
  a.num_splits = plan->num_splits;
  if (launch_stage2(a, batch * q_len_of(p), stream) != hipSuccess) return DECODE_ATTN_ERR_HIP;
  return DECODE_ATTN_OK;
}

}  // namespace

int attend(const decode_attn_plan_t* plan, int expected_kind, const void* q, const void* k_pool,
           const void* v_pool, const int32_t* block_table, const int32_t* ctx_lens, int32_t batch,
           float scale, float* out, float* lse_out, void* workspace, uint64_t workspace_bytes,
           void* stream) {
  int rc = check_plan(plan);
  if (rc != DECODE_ATTN_OK) return rc;
  if (plan->kind != expected_kind) return DECODE_ATTN_ERR_PLAN;
  rc = check_stage1_args(plan, q, k_pool, v_pool, block_table, ctx_lens, batch, scale, workspace,
                         workspace_bytes, plan->layer_workspace_bytes);
  if (rc != DECODE_ATTN_OK) return rc;
  rc = check_stage2_args(plan, batch, workspace, workspace_bytes, out, lse_out,
                         plan->layer_workspace_bytes);
  if (rc != DECODE_ATTN_OK || batch == 0) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (plan->num_splits == 1) {
    // One chunk per row: its normalised output and log-sum-exp already are the result, and the
    // partial planes [B, L, Hq, 1, D] / [B, L, Hq, 1] have the layout of out / lse_out, so stage 1
    // writes them in place and the merge is skipped. Without lse_out the lse goes to the
    // workspace, which then holds only that plane.
    return run_stage1(plan, q, k_pool, v_pool, block_table, ctx_lens, batch, scale, out,
                      lse_out != nullptr ? lse_out : static_cast<float*>(workspace), s);
  }
  float* lse_ws = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan->partial_lse_offset);
  rc = run_stage1(plan, q, k_pool, v_pool, block_table, ctx_lens, batch, scale,
                  static_cast<float*>(workspace), lse_ws, s);
  if (rc != DECODE_ATTN_OK) return rc;
  return run_stage2(plan, batch, workspace, out, lse_out, s);
}

}  // namespace decode_attn

using namespace decode_attn;

extern "C" {

int decode_attn_plan(const decode_attn_problem* problem, decode_attn_plan_t* plan) {
  if (problem == nullptr || plan == nullptr) return DECODE_ATTN_ERR_NULL;
  decode_attn_problem p = *problem;
  if (p.batch < 1 || p.num_q_heads < 1 || p.num_kv_heads < 1 || p.head_dim < 1 ||
      p.page_size < 1 || p.max_pages_per_seq < 1 || p.num_pages < 1 || p.max_ctx_len < 0 ||
      p.window < 0 || p.num_cus < 0 || p.max_splits < 0 || p.force_splits < 0 || p.sink < 0 ||
      p.q_len < 0 || p.q_len > DECODE_ATTN_MAX_Q_LEN ||
      (p.values_are_keys != 0 && p.values_are_keys != 1))
    return DECODE_ATTN_ERR_SHAPE;
  if (p.num_q_heads % p.num_kv_heads != 0) return DECODE_ATTN_ERR_SHAPE;
  if (p.max_splits > DECODE_ATTN_MAX_SPLITS_LIMIT || p.force_splits > DECODE_ATTN_MAX_SPLITS_LIMIT)
    return DECODE_ATTN_ERR_SHAPE;
  if ((int64_t)p.max_pages_per_seq * p.page_size > INT32_MAX) return DECODE_ATTN_ERR_SHAPE;
  // Launch grids put (sequence, query token) pairs, and heads, on grid dimensions capped at 65535.
  if ((int64_t)p.batch * (p.q_len > 1 ? p.q_len : 1) > 65535) return DECODE_ATTN_ERR_SHAPE;
  if (p.num_q_heads > 65535) return DECODE_ATTN_ERR_SHAPE;
  const int G = p.num_q_heads / p.num_kv_heads;
  if (p.page_size % kTile != 0 || p.page_size > 1024) return DECODE_ATTN_ERR_UNSUPPORTED;
  if (!stage1_supported(p.head_dim, G)) return DECODE_ATTN_ERR_UNSUPPORTED;
  if (p.num_cus == 0) {
    const int rc = query_num_cus(&p.num_cus);
    if (rc != DECODE_ATTN_OK) return rc;
  }
  if (p.max_splits == 0) p.max_splits = kDefaultMaxSplits;
  if (p.q_len == 0) p.q_len = 1;

  // Longest key range one workgroup walks, in 16-key tiles (a window may straddle one more;
  // sink keys add their own tiles; the queries of a block widen a window by their count - 1).
  const int64_t max_keys = (int64_t)p.max_pages_per_seq * p.page_size;
  int64_t e = p.max_ctx_len > 0 ? (p.max_ctx_len < max_keys ? p.max_ctx_len : max_keys) : max_keys;
  const int per_block = stage1_block_queries(G, p.q_len, p.head_dim);
  const int64_t span = (int64_t)p.window + (p.q_len < per_block ? p.q_len : per_block) - 1;
  if (p.window > 0 && e > span) e = span;
  int64_t tiles = (e + kTile - 1) / kTile + (p.window > 0 ? 1 : 0);
  if (p.window > 0) tiles += ((int64_t)(p.sink < max_keys ? p.sink : max_keys) + kTile - 1) / kTile;
  const int64_t pairs = (int64_t)p.batch * p.num_kv_heads * qblocks_of(p, G);
  // Workgroups to aim for: one per CU for head_dim 512 (a workgroup streams one chunk with 4
  // waves; measured on MI355X, 1 per CU is as fast as 2 and beats 1.5 or 3), two per CU for
  // smaller heads (short per-workgroup chunks, more latency to hide).
  // A layer whose values are its keys reads half the bytes per tile and needs twice the
  // workgroups in flight to stay fed (measured: 1 per CU 88 us, 2 per CU 66 us, 4 per CU 80 us).
  // Blocks with two row groups (G * q_len > 16) do twice the MFMA and softmax work per tile and
  // likewise run best at two per CU (measured: 4 tokens on the 32K global layer 131 -> 113 us).
  const bool two_row_groups = stage1_row_groups(G, p.q_len) == 2;
  // Prefill workgroups (64 rows, or 128 for long head_dim-512 chunks; K/V tiles staged in LDS)
  // fit one per CU at head_dim 512 (131 KB of LDS) and two at 256.
  const bool one_per_cu = stage1_use_prefill(G, p.q_len)
                              ? p.head_dim >= 512
                              : (p.head_dim >= 512 && !p.values_are_keys && !two_row_groups);
  const int64_t target = (one_per_cu ? 1 : 2) * (int64_t)p.num_cus;
  int64_t splits = (target + pairs - 1) / pairs;
  // Head_dim 256 with G <= 4 and one chunk per (sequence, kv head) runs on the key-split kernel,
  // whose 8-wave workgroups keep eight tiles in flight: once the pairs alone give every CU a
  // workgroup, one split (and no merge) beats two (measured on 32 x 8000 keys, 8 KV heads,
  // window 1024: 42.5 against 47.1 us).
  const bool ks_layer = keysplit_layer(p.head_dim, G, p.q_len, p.window > 0 ? p.sink : 0,
                                       p.values_are_keys != 0);
  if (ks_layer && pairs >= p.num_cus)
    splits = 1;
  // With fewer pairs it also runs such layers, at one workgroup per CU (its 8 waves take two per
  // SIMD): measured on the long_ctx sliding layer (32 pairs) equal to the column-split kernel's
  // two per CU with the caches flushed before each call, 11% faster back to back (12.0 against
  // 13.5 us), and the same on 64 and 16 pairs.
  else if (DECODE_ATTN_KS_SPLITS && ks_layer)
    splits = p.num_cus / pairs > 1 ? p.num_cus / pairs : 1;
  int64_t cap = (tiles + kMinTilesPerSplit - 1) / kMinTilesPerSplit;
  if (cap > p.max_splits) cap = p.max_splits;
  if (cap < 1) cap = 1;
  if (splits > cap) splits = cap;
  if (splits < 1) splits = 1;
  if (p.force_splits > 0) splits = p.force_splits;

  decode_attn_plan_t out = {};
  out.problem = p;
  out.num_splits = (int32_t)splits;
  out.chunk_tokens = (int32_t)(((tiles + splits - 1) / splits) * kTile);
  out.group_size = G;
  out.kind = p.window > 0 ? 2 : 1;
  workspace_layout(p, out.num_splits, &out.partial_lse_offset, &out.workspace_bytes);
  out.layer_workspace_bytes = layer_workspace(p, out.num_splits, out.workspace_bytes);
  out.magic = kPlanMagic;
  *plan = out;
  return DECODE_ATTN_OK;
}

int decode_attn_global(const decode_attn_plan_t* plan, const void* q, const void* k_pool,
                       const void* v_pool, const int32_t* block_table, const int32_t* ctx_lens,
                       int32_t batch, float scale, float* out, float* lse_out, void* workspace,
                       uint64_t workspace_bytes, void* stream) {
  return attend(plan, 1, q, k_pool, v_pool, block_table, ctx_lens, batch, scale, out, lse_out,
                workspace, workspace_bytes, stream);
}

int decode_attn_sliding(const decode_attn_plan_t* plan, const void* q, const void* k_pool,
                        const void* v_pool, const int32_t* block_table, const int32_t* ctx_lens,
                        int32_t batch, int32_t window, float scale, float* out, float* lse_out,
                        void* workspace, uint64_t workspace_bytes, void* stream) {
  const int rc = check_plan(plan);
  if (rc != DECODE_ATTN_OK) return rc;
  if (plan->kind != 2) return DECODE_ATTN_ERR_PLAN;
  if (window != plan->problem.window) return DECODE_ATTN_ERR_SHAPE;
  return attend(plan, 2, q, k_pool, v_pool, block_table, ctx_lens, batch, scale, out, lse_out,
                workspace, workspace_bytes, stream);
}

int decode_attn_stage1(const decode_attn_plan_t* plan, const void* q, const void* k_pool,
                       const void* v_pool, const int32_t* block_table, const int32_t* ctx_lens,
                       int32_t batch, float scale, void* workspace, uint64_t workspace_bytes,
                       void* stream) {
  int rc = check_plan(plan);
  if (rc != DECODE_ATTN_OK) return rc;
  rc = check_stage1_args(plan, q, k_pool, v_pool, block_table, ctx_lens, batch, scale, workspace,
                         workspace_bytes, plan->workspace_bytes);
  if (rc != DECODE_ATTN_OK || batch == 0) return rc;
  return run_stage1(plan, q, k_pool, v_pool, block_table, ctx_lens, batch, scale,
                    static_cast<float*>(workspace),
                    reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                             plan->partial_lse_offset),
                    static_cast<hipStream_t>(stream));
}

int decode_attn_stage2(const decode_attn_plan_t* plan, int32_t batch, const void* workspace,
                       uint64_t workspace_bytes, float* out, float* lse_out, void* stream) {
  int rc = check_plan(plan);
  if (rc != DECODE_ATTN_OK) return rc;
  rc = check_stage2_args(plan, batch, workspace, workspace_bytes, out, lse_out,
                         plan->workspace_bytes);
  if (rc != DECODE_ATTN_OK || batch == 0) return rc;
  return run_stage2(plan, batch, workspace, out, lse_out, static_cast<hipStream_t>(stream));
}

int decode_attn_append_kv(const decode_attn_plan_t* plan, const void* k_new, const void* v_new,
                          void* k_pool, void* v_pool, const int32_t* block_table,
                          const int32_t* ctx_lens, int32_t batch, void* stream) {
  const int rc = check_plan(plan);
  if (rc != DECODE_ATTN_OK) return rc;
  if (batch < 0 || batch > plan->problem.batch) return DECODE_ATTN_ERR_SHAPE;
  if (batch == 0) return DECODE_ATTN_OK;
  const bool same = v_pool == k_pool;
  if (!k_new || !k_pool || !v_pool || !block_table || !ctx_lens || (!same && !v_new))
    return DECODE_ATTN_ERR_NULL;
  if (!aligned(k_new, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      (!same && !aligned(v_new, 16)) || !aligned(block_table, 4) || !aligned(ctx_lens, 4))
    return DECODE_ATTN_ERR_ALIGN;
  const decode_attn_problem& p = plan->problem;
  AppendArgs a;
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(same ? k_new : v_new);
  a.k_pool = static_cast<uint16_t*>(k_pool);
  a.v_pool = static_cast<uint16_t*>(v_pool);
  a.block_table = block_table;
  a.ctx_lens = ctx_lens;
  a.num_kv_heads = p.num_kv_heads;
  a.head_dim = p.head_dim;
  a.page_size = p.page_size;
  a.max_pages_per_seq = p.max_pages_per_seq;
  a.num_pages = p.num_pages;
  a.q_len = q_len_of(p);
  if (launch_append(a, batch, static_cast<hipStream_t>(stream)) != hipSuccess)
    return DECODE_ATTN_ERR_HIP;
  return DECODE_ATTN_OK;
}

int decode_attn_rope_cache(float* cos_sin, int32_t max_position, int32_t rotary_dim,
                           int32_t freq_dim, double theta, void* stream) {
  if (!cos_sin) return DECODE_ATTN_ERR_NULL;
  if (!aligned(cos_sin, 4)) return DECODE_ATTN_ERR_ALIGN;
  if (max_position < 1 || rotary_dim < 2 || rotary_dim % 2 != 0 || freq_dim < 0 ||
      !(theta > 0.0) || !std::isfinite(theta))
    return DECODE_ATTN_ERR_SHAPE;
  if (launch_rope_cache(cos_sin, max_position, rotary_dim, freq_dim ? freq_dim : rotary_dim, theta,
                        static_cast<hipStream_t>(stream)) != hipSuccess)
    return DECODE_ATTN_ERR_HIP;
  return DECODE_ATTN_OK;
}

int decode_attn_append_kv_rope(const decode_attn_plan_t* plan, const void* q, void* q_out,
                               const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                               const int32_t* block_table, const int32_t* ctx_lens, int32_t batch,
                               const float* cos_sin, int32_t max_position, int32_t rotary_dim,
                               int32_t interleaved, int32_t norm_flags, const float* q_norm_weight,
                               const float* k_norm_weight, const float* v_norm_weight, float eps,
                               void* stream) {
  const int rc = check_plan(plan);
  if (rc != DECODE_ATTN_OK) return rc;
  const decode_attn_problem& p = plan->problem;
  if (batch < 0 || batch > p.batch) return DECODE_ATTN_ERR_SHAPE;
  if (rotary_dim < 0 || rotary_dim > p.head_dim || rotary_dim % 2 != 0 || max_position < 1 ||
      (interleaved != 0 && interleaved != 1) ||
      (norm_flags & ~(DECODE_ATTN_NORM_QK | DECODE_ATTN_NORM_V)) != 0 ||
      (norm_flags != 0 && !(eps > 0.f && std::isfinite(eps))))
    return DECODE_ATTN_ERR_SHAPE;
  if (batch == 0) return DECODE_ATTN_OK;
  const bool same = v_pool == k_pool;
  if (!q || !q_out || !k_new || !k_pool || !v_pool || !block_table || !ctx_lens ||
      (!same && !v_new) || (rotary_dim > 0 && !cos_sin))
    return DECODE_ATTN_ERR_NULL;
  if (!aligned(q, 16) || !aligned(q_out, 16) || !aligned(k_new, 16) || !aligned(k_pool, 16) ||
      !aligned(v_pool, 16) || (!same && !aligned(v_new, 16)) || !aligned(block_table, 4) ||
      !aligned(ctx_lens, 4) || !aligned(cos_sin, 4) || !aligned(q_norm_weight, 4) ||
      !aligned(k_norm_weight, 4) || !aligned(v_norm_weight, 4))
    return DECODE_ATTN_ERR_ALIGN;
  AppendRopeArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.q_out = static_cast<uint16_t*>(q_out);
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(same ? k_new : v_new);
  a.k_pool = static_cast<uint16_t*>(k_pool);
  a.v_pool = static_cast<uint16_t*>(v_pool);
  a.block_table = block_table;
  a.ctx_lens = ctx_lens;
  a.cos_sin = cos_sin;
  a.q_weight = q_norm_weight;
  a.k_weight = k_norm_weight;
  a.v_weight = v_norm_weight;
  a.eps = eps;
  a.num_q_heads = p.num_q_heads;
  a.num_kv_heads = p.num_kv_heads;
  a.page_size = p.page_size;
  a.max_pages_per_seq = p.max_pages_per_seq;
  a.num_pages = p.num_pages;
  a.q_len = q_len_of(p);
  a.max_position = max_position;
  a.rotary_dim = rotary_dim;
  a.interleaved = interleaved;
  a.norm_flags = norm_flags;
  if (launch_append_rope(a, p.head_dim, batch, static_cast<hipStream_t>(stream)) != hipSuccess)
    return DECODE_ATTN_ERR_HIP;
  return DECODE_ATTN_OK;
}

const char* decode_attn_status_str(int status) {
  switch (status) {
    case DECODE_ATTN_OK: return "DECODE_ATTN_OK";
    case DECODE_ATTN_ERR_NULL: return "DECODE_ATTN_ERR_NULL: a required pointer is NULL";
    case DECODE_ATTN_ERR_SHAPE: return "DECODE_ATTN_ERR_SHAPE: inconsistent sizes or values";
    case DECODE_ATTN_ERR_UNSUPPORTED:
      return "DECODE_ATTN_ERR_UNSUPPORTED: no kernel for this head_dim / group / page size";
    case DECODE_ATTN_ERR_WORKSPACE: return "DECODE_ATTN_ERR_WORKSPACE: workspace too small";
    case DECODE_ATTN_ERR_PLAN: return "DECODE_ATTN_ERR_PLAN: invalid plan or wrong layer kind";
    case DECODE_ATTN_ERR_HIP: return "DECODE_ATTN_ERR_HIP: HIP runtime error";
    case DECODE_ATTN_ERR_ALIGN: return "DECODE_ATTN_ERR_ALIGN: pointer not aligned";
    default: return "unknown decode_attn status";
  }
}

int decode_attn_version(void) { return DECODE_ATTN_VERSION; }

}  // extern "C"
