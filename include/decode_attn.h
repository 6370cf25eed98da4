/*
 * decode_attn.h — C ABI of the paged GQA split-KV decode-attention library for MI355X (gfx950).
 *
 * What it computes. Decode attention (one new query token per sequence, or up to 8192 causal ones:
 * speculative verification and chunked prefill) over a paged KV cache for the two layer kinds of a Gemma-4-style model: "global" layers (every cached key attended; head_dim 512 in Gemma 4) and
 * "sliding-window" layers (only the last W keys attended; head_dim 256 in Gemma 4). The layer kinds
 * may differ in head dim, KV-head count and window (Sparse-vLLM PR #27 "feat: support Gemma 4 and
 * native multimodal inference", section "Gemma 4 文本推理" / Gemma 4 text inference). Several query
 * heads share one KV head (GQA); one launch handles a whole query-head group (same page, section
 * "专用算子与性能优化" / dedicated operators). Decode is one new query token per sequence attending
 * to all of its cached keys (vLLM learning notes "模型库与算子层 — 概念", section "核心操作").
 *
 * For sequence b, query token i < L (L = q_len, 1 for plain decode), query head h, KV head
 * g = h / G (G = Hq / Hkv, contiguous groups):
 *     n   = ctx_lens[b] - L + i + 1          (keys visible to the query: the cached keys up to
 *                                             and including its own position n - 1)
 *     lo  = 0 (global)  or  max(0, n - W) (sliding)
 *     A   = [lo, n), plus [0, min(sink, n)) for a sliding layer planned with sink > 0
 *     s_t = scale * <q[b,i,h,:], K_t>        for t in A
 *     out[b,i,h,:] = sum_t exp(s_t - m) V_t / sum_t exp(s_t - m),   m = max_t s_t
 *     lse[b,i,h]   = m + ln(sum_t exp(s_t - m))
 * where K_t / V_t live in pool page block_table[b, t / S] at slot t % S. An empty A (n <= 0)
 * gives out = 0 and lse = -inf. The sink keys give the StreamingLLM-style views the same page
 * supports (section "Gemma 4 文本推理"): a window of recent keys plus a few leading ones. L > 1
 * is causal multi-token verification (the last L cached keys are the new tokens themselves; vLLM
 * learning notes, the MLA backend notes on causal multi-token verification) or a chunk of a
 * prompt's prefill over the paged cache; L = 1 is the single-token decode. Section "核心操作" of
 * the same notes names both operations an attention layer serves: prefill and decode.
 *
 * How. Split-KV: stage 1 cuts each sequence's key range into num_splits chunks and writes, per
 * (b, i, h, split), the chunk's normalised partial output and its log-sum-exp; stage 2 merges the
 * partials of each (b, i, h) by their log-sum-exps. With one chunk (num_splits = 1, the planner's
 * pick when the query blocks alone fill the GPU, as in prefill) the partial is the result: stage 1
 * then writes out and lse_out directly and stage 2 is not launched. The partial buffer reserves one LSE value per
 * (b, i, h, split) next to the D partial outputs and is sized once, for the worst case, so that no
 * call allocates and calls can be captured in a HIP graph (vLLM learning notes, section
 * "MLA 与 Sparse MLA（DSA）", split-KV MLA decode). A plan is computed on the host from the shape
 * only; it holds no device pointer, in particular no page-table address, so reusing a plan across
 * requests with different block tables is always safe (Sparse-vLLM PR #27, section
 * "专用算子与性能优化", plan invalidation on page-table address change).
 *
 * Layouts (all row-major, contiguous, device memory):
 *     q            [B, L, Hq, D]          bf16   ([B, Hq, D] when L = 1)
 *     k_pool       [P, Hkv, S, D]         bf16   one (page, kv head) block is S*D contiguous values
 *     v_pool       [P, Hkv, S, D]         bf16   the same buffer as k_pool for layers whose values
 *                                                are their keys (K = V, Sparse-vLLM PR #27, section
 *                                                "Gemma 4 文本推理"): plan them with
 *                                                values_are_keys = 1 and pass one pool twice
 *     block_table  [B, max_pages_per_seq] int32  physical page ids; entries of pages holding no key
 *                                                of A are never read and may hold anything. A
 *                                                sparse view (a table naming only some of a
 *                                                sequence's pages, n counting the keys they hold)
 *                                                is attended like any other table
 *     ctx_lens     [B]                    int32
 *     out          [B, L, Hq, D]          fp32
 *     lse_out      [B, L, Hq]             fp32   (optional, may be NULL)
 *     workspace    stage-1 partials (see decode_attn_stage1): plan->workspace_bytes bytes for the
 *                  stage calls, plan->layer_workspace_bytes for the layer calls
 *
 * Ownership and threading. Every buffer is owned by the caller; the library never allocates or
 * frees device memory and keeps no mutable global state (a per-device CU count is cached). Calls
 * are asynchronous on the given stream (a hipStream_t passed as void*, NULL = default stream) and
 * never synchronise the host, so they can be captured in a HIP graph. Calls that share a
 * workspace must be ordered on one stream.
 *
 * Errors. Every argument is checked on the host before anything is launched; a nonzero
 * decode_attn_status is returned and nothing is written. DECODE_ATTN_ERR_HIP reports a launch
 * error. Device-side faults surface at the caller's next synchronisation. On any error the
 * contents of out / lse_out / workspace are unspecified.
 *
 * Robustness inside the kernels: ctx_lens[b] is clamped to [0, max_pages_per_seq * S]; a block
 * table entry outside [0, P) is never dereferenced and the keys of that page are skipped.
 */
#ifndef DECODE_ATTN_H
#define DECODE_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DECODE_ATTN_OK = 0,
  DECODE_ATTN_ERR_NULL = 1,        /* a required pointer is NULL */
  DECODE_ATTN_ERR_SHAPE = 2,       /* inconsistent sizes or values (Hq % Hkv != 0, batch > plan) */
  DECODE_ATTN_ERR_UNSUPPORTED = 3, /* head_dim, group size or page size with no compiled kernel */
  DECODE_ATTN_ERR_WORKSPACE = 4,   /* workspace smaller than the call needs (see the plan) */
  DECODE_ATTN_ERR_PLAN = 5,        /* plan not made by decode_attn_plan, or for the other layer kind */
  DECODE_ATTN_ERR_HIP = 6,         /* the HIP runtime reported an error (launch or device query) */
  DECODE_ATTN_ERR_ALIGN = 7        /* q, pools, out or workspace not 16-byte aligned */
} decode_attn_status;

/* Compiled kernel variants. */
#define DECODE_ATTN_MAX_SPLITS_LIMIT 1024 /* hard upper bound on num_splits */
#define DECODE_ATTN_MAX_Q_LEN 8192        /* most query tokens per sequence in one call */

/* The shape a plan covers. Values are upper bounds for the calls made with the plan. */
typedef struct {
  int32_t batch;             /* B >= 1: most sequences per call; B * max(1, q_len) <= 65535 */
  int32_t num_q_heads;       /* 1 <= Hq <= 65535 */
  int32_t num_kv_heads;      /* Hkv >= 1, Hq % Hkv == 0; G = Hq / Hkv in {1, 2, 4, 8, 16} */
  int32_t head_dim;          /* D in {256, 512} */
  int32_t page_size;         /* S: tokens per page, a multiple of 16, 16 <= S <= 1024 */
  int32_t max_pages_per_seq; /* columns (row stride) of the block table, >= 1 */
  int32_t num_pages;         /* P: pages in each pool, >= 1 */
  int32_t max_ctx_len;       /* longest context expected; sizes the split count, and single-token
                                calls fetch the first page ids of the chunk a sequence of this length
                                would have before its actual length arrives (kept when that length
                                gives the same chunk). Other lengths are still computed correctly.
                                0 = max_pages_per_seq * S for the split count, no early fetch */
  int32_t window;            /* 0: global layer; W > 0: sliding layer attending the last W keys */
  int32_t num_cus;           /* compute units to plan for; 0 = query the current HIP device */
  int32_t max_splits;        /* cap on num_splits; 0 = library default (256) */
  int32_t force_splits;      /* 0 = the planner chooses; > 0 = use exactly this many (<= 1024) */
  int32_t values_are_keys;   /* 1: the layer's values are its keys and calls pass one pool as both
                                k_pool and v_pool (each tile is then read once); 0: separate pools */
  int32_t sink;              /* sliding layers only: also attend the first `sink` keys of every
                                sequence (attention sinks of StreamingLLM-style views); 0 = none.
                                Ignored when window == 0, where every key is attended anyway */
  int32_t q_len;             /* L: new query tokens per sequence, 0 or 1 = single-token decode,
                                up to DECODE_ATTN_MAX_Q_LEN (speculative verification, chunked
                                prefill); every call with the plan passes L tokens per sequence */
} decode_attn_problem;

/* A plan: plain data, copy it freely; there is nothing to free. */
typedef struct {
  decode_attn_problem problem; /* copy of the problem, num_cus and max_splits resolved */
  int32_t num_splits;          /* chunks per (sequence, kv head) in stage 1 */
  int32_t chunk_tokens;        /* tokens per chunk at max_ctx_len (16-token tiles, informational) */
  int32_t group_size;          /* G = Hq / Hkv */
  int32_t kind;                /* 1 = global (window == 0), 2 = sliding (window > 0) */
  uint64_t workspace_bytes;    /* bytes of workspace decode_attn_stage1 / _stage2 need */
  uint64_t partial_lse_offset; /* byte offset of the LSE plane inside the workspace */
  uint32_t magic;              /* set by decode_attn_plan; checked by every entry point */
  int32_t reserved0;
  uint64_t layer_workspace_bytes; /* bytes of workspace decode_attn_global / _sliding need:
                                     workspace_bytes, or with num_splits == 1 only the
                                     256-byte-rounded [B, L, Hq] fp32 lse plane (stage 1 then
                                     writes out in place and its lse there when lse_out is NULL) */
  int32_t reserved[4];
} decode_attn_plan_t;

/*
 * decode_attn_plan — host only, no device work (a device query only when problem->num_cus == 0).
 * Checks the problem, picks the split count and computes the workspace size.
 * Split rule: with T = ceil(e / 16) (+ 1 for a sliding window, whose edge may straddle a tile,
 * + ceil(sink / 16) for its sink keys) tiles of 16 keys for the longest range one query block
 * walks, e = min(max_ctx_len, W + min(L, Q) - 1 or unlimited), with Q the queries of a block,
 * pairs = batch * Hkv * ceil(L / Q) and target = num_cus workgroups for head_dim 512 with
 * separate pools and G * L <= 16, and for head_dim 512 when G * L >= 64 (2 * num_cus for head_dim
 * 256, when values are keys, or for blocks of 32 rows),
 *     num_splits = clamp(ceil(target / pairs), 1, min(max_splits, T))
 * so every chunk holds at least one tile when the context allows it (short contexts are
 * latency-bound: more, shorter chunks finish sooner). Single-token layers at head_dim 256 with
 * G <= 4, separate pools and no sink keys instead take num_splits = clamp(floor(num_cus / pairs),
 * 1, min(max_splits, T)): one workgroup per CU, each of whose waves walks its own tiles.
 * force_splits > 0 overrides the rule.
 * Returns DECODE_ATTN_OK, DECODE_ATTN_ERR_NULL, _SHAPE, _UNSUPPORTED or _HIP (device query).
 */
int decode_attn_plan(const decode_attn_problem* problem, decode_attn_plan_t* plan);

/*
 * decode_attn_global — attention of a global layer (plan->problem.window == 0): stage 1 then
 * stage 2 on `stream` (stage 1 alone, writing out and lse_out, when plan->num_splits == 1). `batch` (0 <= batch <= plan->problem.batch) sequences are computed; batch 0
 * returns DECODE_ATTN_OK without launching. `scale` multiplies q.k (1/sqrt(D) for Gemma-style
 * layers). lse_out may be NULL. workspace must hold plan->layer_workspace_bytes. A plan made with
 * values_are_keys = 1 requires v_pool == k_pool (else DECODE_ATTN_ERR_SHAPE); the same pool passed
 * twice under a plan without it is computed correctly, with the other split count.
 */
int decode_attn_global(const decode_attn_plan_t* plan, const void* q, const void* k_pool,
                       const void* v_pool, const int32_t* block_table, const int32_t* ctx_lens,
                       int32_t batch, float scale, float* out, float* lse_out, void* workspace,
                       uint64_t workspace_bytes, void* stream);

/*
 * decode_attn_sliding — attention of a sliding-window layer: the same call as decode_attn_global
 * plus `window`, which must equal plan->problem.window (> 0). Only keys t with
 * max(0, n - window) <= t < n, and t < plan->problem.sink, are read; window and sink edges need
 * not fall on 16- or 32-key boundaries (Sparse-vLLM PR #27, section "专用算子与性能优化",
 * non-32-aligned blocks of the sliding kernel).
 */
int decode_attn_sliding(const decode_attn_plan_t* plan, const void* q, const void* k_pool,
                        const void* v_pool, const int32_t* block_table, const int32_t* ctx_lens,
                        int32_t batch, int32_t window, float scale, float* out, float* lse_out,
                        void* workspace, uint64_t workspace_bytes, void* stream);

/*
 * decode_attn_stage1 — stage 1 alone, for either layer kind (the window comes from the plan).
 * Writes the workspace, which holds two planes:
 *     o_part [B, L, Hq, num_splits, D] fp32 at byte offset 0
 *     lse    [B, L, Hq, num_splits]    fp32 at byte offset plan->partial_lse_offset
 * The queries of a sequence are taken in blocks of 16 / G, 32 / G when G * L > 16, 64 / G
 * when G * L >= 64, or 128 / G at head_dim 512 when G * L >= 128 (one block when L = 1).
 * Split s of a
 * block covers the tiles [floor(s*T/ns), floor((s+1)*T/ns)) of the block's list of T 16-key
 * tiles (ns = num_splits). With lo and n those of the block's first and last query respectively,
 * the list holds the tiles 0 .. ceil(k/16) - 1 that overlap the sink keys [0, k), k = min(sink,
 * lo), followed by the tiles overlapping [lo, n) not already listed; keys outside a query's A
 * are masked for it. o_part is that chunk's softmax-normalised output and lse its
 * log-sum-exp of s_t; a chunk with no key has o_part = 0 and lse = -inf. Together with
 * decode_attn_stage2 this lets the partials be produced and merged separately (for example by
 * different devices that each own part of the pages).
 */
int decode_attn_stage1(const decode_attn_plan_t* plan, const void* q, const void* k_pool,
                       const void* v_pool, const int32_t* block_table, const int32_t* ctx_lens,
                       int32_t batch, float scale, void* workspace, uint64_t workspace_bytes,
                       void* stream);

/*
 * decode_attn_stage2 — the log-sum-exp merge of the workspace partials written by stage 1:
 *     M = max_s lse_s,  w_s = exp(lse_s - M),  out = sum_s w_s o_s / sum_s w_s,
 *     lse_out = M + ln(sum_s w_s);   all lse_s = -inf gives out = 0 and lse_out = -inf.
 */
int decode_attn_stage2(const decode_attn_plan_t* plan, int32_t batch, const void* workspace,
                       uint64_t workspace_bytes, float* out, float* lse_out, void* stream);

/*
 * decode_attn_append_kv — write each sequence's L = plan->problem.q_len newest keys and values
 * into the paged pools before attention reads them (the cache-manager write of Sparse-vLLM PR #27,
 * section "Gemma 4 文本推理"; ctx_lens counts the new tokens). For b < batch, n = ctx_lens[b] and
 * i < L, the token at position t = n - L + i (skipped if t < 0) goes to page
 * block_table[b, t / S], slot t % S, for every KV head g:
 *     k_pool[page, g, t % S, :] = k_new[b, i, g, :]    and the same for V.
 * k_new, v_new: [B, L, Hkv, D] bf16 ([B, Hkv, D] when L = 1), 16-byte aligned. v_pool may equal
 * k_pool (layers whose values are their keys): then only k_new is written and v_new may be NULL.
 * A position outside the table row or a page id outside [0, P) is skipped (nothing written for
 * that token). Any plan of the layer with the same q_len can be used (only its shape is read).
 * Bitwise copy; asynchronous on `stream`.
 */
int decode_attn_append_kv(const decode_attn_plan_t* plan, const void* k_new, const void* v_new,
                          void* k_pool, void* v_pool, const int32_t* block_table,
                          const int32_t* ctx_lens, int32_t batch, void* stream);

/* Normalisation flags of decode_attn_append_kv_rope. */
#define DECODE_ATTN_NORM_QK 1 /* RMSNorm every q head and every new k head before the rotation */
#define DECODE_ATTN_NORM_V 2  /* RMSNorm every new v head (values are never rotated) */

/*
 * decode_attn_rope_cache — fill the rotation table that decode_attn_append_kv_rope reads, for one
 * layer configuration (Sparse-vLLM PR #27, section "Gemma 4 文本推理": each layer kind has its own
 * RoPE parameters and its own RoPE cache). With R = rotary_dim, for t < max_position and j < R/2:
 *     f_j = theta^(-2j / F)            F = freq_dim, or R when freq_dim = 0
 *     cos_sin[t, j] = cos(t * f_j),    cos_sin[t, R/2 + j] = sin(t * f_j)
 * computed on the device in double precision and rounded to fp32. cos_sin: [max_position, R] fp32
 * device memory owned by the caller, 4-byte aligned. A table of any other RoPE variant (scaled
 * positions or frequencies) has the same layout and can be written by the caller instead.
 * Errors: ERR_NULL (cos_sin NULL), ERR_ALIGN, ERR_SHAPE (max_position < 1, R odd or < 2,
 * freq_dim < 0, theta not finite and positive). Asynchronous on `stream`.
 */
int decode_attn_rope_cache(float* cos_sin, int32_t max_position, int32_t rotary_dim,
                           int32_t freq_dim, double theta, void* stream);

/*
 * decode_attn_append_kv_rope — the step just before attention as one launch: QK-norm, rotary
 * position embedding and the paged append (Sparse-vLLM PR #27, section "专用算子与性能优化": a
 * dedicated QKV-norm + RoPE operator; vLLM learning notes "模型库与算子层 — 概念", section
 * "自定义 Inductor 融合 pass": norm/RoPE fused with the paged KV-cache write, and section
 * "内核框架（Helion）": the q/k RMSNorm fused with RoPE in place, NeoX or GPT-J pairing).
 * For b < batch, new token i < L = plan->problem.q_len and its position t = ctx_lens[b] - L + i:
 *     rms(x; w)  = x / sqrt(mean_d x_d^2 + eps) * w       (w NULL: no scale)
 *     q_out[b, i, h]           = rope_t(rms(q[b, i, h]; q_norm_weight))
 *     k_pool[page, g, t % S]   = rope_t(rms(k_new[b, i, g]; k_norm_weight))
 *     v_pool[page, g, t % S]   = rms(v_new[b, i, g]; v_norm_weight)
 * with page = block_table[b, t / S]; rms is applied to q and k only with DECODE_ATTN_NORM_QK and
 * to v only with DECODE_ATTN_NORM_V (else v is copied bit for bit). rope_t turns pair j < R/2 of
 * the first R = rotary_dim dims, (x1, x2) -> (x1 c - x2 s, x2 c + x1 s) with c = cos_sin[t, j] and
 * s = cos_sin[t, R/2 + j]; the pair is (x_j, x_{j+R/2}) for interleaved = 0 (NeoX) and
 * (x_{2j}, x_{2j+1}) for interleaved = 1 (GPT-J); dims at or past R pass unchanged (R = 0: no
 * rotation, cos_sin may be NULL). Arithmetic is fp32; every output is rounded once to bf16.
 *
 * Arguments: q and q_out [B, L, Hq, D] bf16 ([B, Hq, D] when L = 1), q_out == q for in place, else
 * not overlapping; k_new, v_new [B, L, Hkv, D] bf16; pools, block_table and ctx_lens as for
 * attention; v_pool == k_pool for layers whose values are their keys (then only k is written and
 * v_new may be NULL); cos_sin [max_position, R] fp32 (decode_attn_rope_cache); the norm weights [D]
 * fp32 or NULL. bf16 buffers 16-byte aligned, the others 4-byte. Any plan of the layer with the
 * same q_len can be used (only its shape is read). Asynchronous on `stream`.
 *
 * Skips: a token with t < 0 or t >= max_position is skipped whole (its q_out row is not written,
 * nothing is appended). A page column t / S past the table row or a page id outside [0, P) skips
 * that token's k and v writes (its q_out row is still written).
 * Errors: ERR_PLAN, ERR_SHAPE (batch outside [0, plan batch], R odd or outside [0, D],
 * max_position < 1, interleaved not 0 or 1, unknown flags, eps not finite and positive while a
 * norm flag is set), ERR_NULL, ERR_ALIGN, ERR_HIP.
 */
int decode_attn_append_kv_rope(const decode_attn_plan_t* plan, const void* q, void* q_out,
                               const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                               const int32_t* block_table, const int32_t* ctx_lens, int32_t batch,
                               const float* cos_sin, int32_t max_position, int32_t rotary_dim,
                               int32_t interleaved, int32_t norm_flags, const float* q_norm_weight,
                               const float* k_norm_weight, const float* v_norm_weight, float eps,
                               void* stream);

/* Size of the device array behind decode_attn_layer_noalloc (64 MiB per device). */
#define DECODE_ATTN_NOALLOC_SCRATCH_BYTES (64ull << 20)

/*
 * decode_attn_layer_noalloc — for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the layer call of
 * decode_attn_global (window == 0) or decode_attn_sliding (window == plan->problem.window > 0)
 * with the same arguments minus the workspace. The stage-1 partials go to a static device array
 * of the library, DECODE_ATTN_NOALLOC_SCRATCH_BYTES long, that every device running the library
 * holds until the process ends; no call allocates or frees anything. Results are those of the
 * layer call with a caller workspace (the same kernels).
 * Limit: plans whose layer_workspace_bytes exceed DECODE_ATTN_NOALLOC_SCRATCH_BYTES are rejected
 * with DECODE_ATTN_ERR_WORKSPACE before anything else is touched (single-token decode needs
 * B * Hq * num_splits * (D + 1) * 4 bytes: 4.2 MB for 4 x 32K or 1 x 128K at 16 heads, D 512).
 * Sharing: all calls on one device use that device's one array, so calls that may overlap on
 * a device (other streams, other host threads) race and must be ordered by the caller; each call
 * writes every partial it reads, so nothing carries over from the previous call.
 * The first call on a device looks up the array's address there (hipGetSymbolAddress); make it
 * outside graph capture. Errors: those of decode_attn_global / _sliding.
 */
int decode_attn_layer_noalloc(const decode_attn_plan_t* plan, const void* q, const void* k_pool,
                              const void* v_pool, const int32_t* block_table,
                              const int32_t* ctx_lens, int32_t batch, int32_t window, float scale,
                              float* out, float* lse_out, void* stream);

/* Static, human-readable name of a status code (never NULL). */
const char* decode_attn_status_str(int status);

/* Library version, major * 10000 + minor * 100 + patch. The minor number changes with the layout
 * of decode_attn_problem / decode_attn_plan_t (0.2: sink and q_len fields); 0.2.1: q_len up to
 * 8192, one-split calls without stage 2; 0.2.2: decode_attn_rope_cache and
 * decode_attn_append_kv_rope; 0.3.0: layer_workspace_bytes in the plan. */
#define DECODE_ATTN_VERSION 300
int decode_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DECODE_ATTN_H */
