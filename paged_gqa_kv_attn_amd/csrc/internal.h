// internal.h — declarations shared by the host entry points and the HIP kernels of
// libdecode_attn.so. Not part of the public ABI (that is include/decode_attn.h).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "decode_attn.h"

namespace decode_attn {

constexpr uint32_t kPlanMagic = 0x44415431u;  // "DAT1"
constexpr int kTile = 16;                     // keys per tile: the M dimension of one MFMA
constexpr int kDefaultMaxSplits = 256;
constexpr int kMinTilesPerSplit = 1;          // a chunk holds one 16-key tile at least
constexpr int kStage2Threads = 256;
constexpr int kPrefillRows = 64;              // (query, head) rows of a prefill workgroup

// Kernel arguments of stage 1 (one workgroup per (split, query block, kv head, sequence)).
struct Stage1Args {
  const uint16_t* q;            // [B, L, Hq, D] bf16
  const uint16_t* k_pool;       // [P, Hkv, S, D] bf16
  const uint16_t* v_pool;       // [P, Hkv, S, D] bf16
  const int32_t* block_table;   // [B, max_pages_per_seq]
  const int32_t* ctx_lens;      // [B]
  float* o_part;                // [B, L, Hq, num_splits, D]
  float* lse_part;              // [B, L, Hq, num_splits]
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t page_size;
  int32_t max_pages_per_seq;
  int32_t num_pages;
  int32_t window;               // 0 = all keys
  int32_t sink;                 // leading keys also attended by a sliding layer (0 = none)
  int32_t q_len;                // L >= 1 query tokens per sequence (q is [B, L, Hq, D])
  int32_t num_qblocks;          // ceil(L / (16 / G)): query blocks of one (sequence, kv head)
  int32_t num_splits;
  float scale_log2;             // scale * log2(e): scores in base-2 units
  int32_t spec_ctx;             // the plan's expected context length (0 = none): a kernel may
                                // fetch the page ids of that length's chunk before ctx_lens
};

// Kernel arguments of stage 2 (one workgroup per (64-wide slice of D, q head, sequence)).
// B' = B * L rows of Hq query heads (the query tokens of a sequence are consecutive rows).
struct Stage2Args {
  const float* o_part;          // [B', Hq, num_splits, D]
  const float* lse_part;        // [B', Hq, num_splits]
  float* out;                   // [B', Hq, D]
  float* lse_out;               // [B', Hq] or nullptr
  int32_t num_q_heads;
  int32_t head_dim;
  int32_t num_splits;
};

// Kernel arguments of the paged KV append (one workgroup per (sequence, new token, KV head)).
struct AppendArgs {
  const uint16_t* k_new;        // [B, L, Hkv, D] bf16
  const uint16_t* v_new;        // [B, L, Hkv, D] bf16 (unused when v_pool == k_pool)
  uint16_t* k_pool;             // [P, Hkv, S, D] bf16
  uint16_t* v_pool;             // [P, Hkv, S, D] bf16, may equal k_pool
  const int32_t* block_table;   // [B, max_pages_per_seq]
  const int32_t* ctx_lens;      // [B]
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t max_pages_per_seq;
  int32_t num_pages;
  int32_t q_len;                // L >= 1 new tokens per sequence
};

// Kernel arguments of the fused QK-norm + RoPE + paged append (one wave per (new token, row)).
struct AppendRopeArgs {
  const uint16_t* q;            // [B, L, Hq, D] bf16
  uint16_t* q_out;              // [B, L, Hq, D] bf16, may equal q
  const uint16_t* k_new;        // [B, L, Hkv, D] bf16
  const uint16_t* v_new;        // [B, L, Hkv, D] bf16 (unused when v_pool == k_pool)
  uint16_t* k_pool;             // [P, Hkv, S, D] bf16
  uint16_t* v_pool;             // [P, Hkv, S, D] bf16, may equal k_pool
  const int32_t* block_table;   // [B, max_pages_per_seq]
  const int32_t* ctx_lens;      // [B]
  const float* cos_sin;         // [max_position, rotary_dim] fp32: cos of pair j, then sin
  const float* q_weight;        // [D] fp32 or nullptr (unit scale)
  const float* k_weight;        // [D] fp32 or nullptr
  const float* v_weight;        // [D] fp32 or nullptr
  float eps;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t page_size;
  int32_t max_pages_per_seq;
  int32_t num_pages;
  int32_t q_len;                // L >= 1 new tokens per sequence
  int32_t max_position;         // positions at or past this are skipped
  int32_t rotary_dim;           // R, even, 0 = no rotation
  int32_t interleaved;          // 0: pairs (j, j + R/2); 1: pairs (2j, 2j + 1)
  int32_t norm_flags;           // bit 0: RMSNorm q and k; bit 1: RMSNorm v
};

// Launchers (stage1.hip / stage2.hip / append.hip). They return the launch status only. Stage 1
// picks its single-read variant when k_pool == v_pool.
hipError_t launch_stage1(const Stage1Args& args, int head_dim, int group_size, int batch,
                         hipStream_t stream);
hipError_t launch_stage2(const Stage2Args& args, int batch, hipStream_t stream);
// Stage 1 for long query chunks (prefill.hip): the same arguments and outputs, 64-row blocks.
hipError_t launch_prefill(const Stage1Args& args, int head_dim, int group_size, int batch,
                          hipStream_t stream);
hipError_t launch_append(const AppendArgs& args, int batch, hipStream_t stream);
// append_rope.hip: the rotation table, then the fused QK-norm + RoPE + append (head_dim 256 or 512).
hipError_t launch_rope_cache(float* cos_sin, int max_position, int rotary_dim, int freq_dim,
                             double theta, hipStream_t stream);
hipError_t launch_append_rope(const AppendRopeArgs& args, int head_dim, int batch,
                              hipStream_t stream);

// The layer call behind decode_attn_global (expected_kind 1) and decode_attn_sliding (2): checks
// the plan and the arguments against plan->layer_workspace_bytes, then launches stage 1 (and
// stage 2 when the plan has more than one split). decode_attn.cpp.
int attend(const decode_attn_plan_t* plan, int expected_kind, const void* q, const void* k_pool,
           const void* v_pool, const int32_t* block_table, const int32_t* ctx_lens, int32_t batch,
           float scale, float* out, float* lse_out, void* workspace, uint64_t workspace_bytes,
           void* stream);

// Stage 1 of single-token decode at head_dim 256 with G <= 4 and separate pools, the waves of a
// workgroup splitting the chunk's tiles (stage1_ks.hip).
bool stage1_keysplit_supported(int head_dim, int group_size, int q_len, int sink, bool shared);
hipError_t launch_stage1_keysplit(const Stage1Args& args, int group_size, int batch,
                                  hipStream_t stream);

// True when a stage-1 kernel is compiled for (head_dim, group_size).
bool stage1_supported(int head_dim, int group_size);

// Groups of 16 MFMA rows a stage-1 workgroup uses: two when the G * q_len rows of a sequence's
// queries do not fit in 16 (then 32 / G queries share each tile read), else one.
inline int stage1_row_groups(int group_size, int q_len) {
  return (q_len > 1 && group_size * q_len > 16) ? 2 : 1;
}

// Long query chunks (G * q_len >= 64 rows per kv head) run on the prefill kernel.
inline bool stage1_use_prefill(int group_size, int q_len) {
  return q_len > 1 && group_size * q_len >= kPrefillRows;
}

// Rows of a prefill workgroup (16 per wave). At head_dim 512, chunks of at least 128 rows per KV
// head take workgroups of 128 rows: eight waves share each staged tile, two per SIMD. Shorter
// chunks (no half-empty workgroups), and head_dim 256 (two workgroups per CU), take 64 rows.
constexpr int kPrefillWideRows = 128;
#ifndef DECODE_ATTN_PREFILL_WIDE_MIN_ROWS
#define DECODE_ATTN_PREFILL_WIDE_MIN_ROWS 128
#endif
inline int prefill_rows(int head_dim, int group_size, int q_len) {
  return head_dim == 512 && (int64_t)group_size * q_len >= DECODE_ATTN_PREFILL_WIDE_MIN_ROWS
             ? kPrefillWideRows
             : kPrefillRows;
}

// Queries one stage-1 workgroup serves, and the query blocks of one (sequence, kv head).
inline int stage1_block_queries(int group_size, int q_len, int head_dim) {
  if (stage1_use_prefill(group_size, q_len))
    return prefill_rows(head_dim, group_size, q_len) / group_size;
  return 16 * stage1_row_groups(group_size, q_len) / group_size;
}
inline int stage1_query_blocks(int group_size, int q_len, int head_dim) {
  const int per = stage1_block_queries(group_size, q_len, head_dim);
  return (q_len + per - 1) / per;
}

}  // namespace decode_attn
