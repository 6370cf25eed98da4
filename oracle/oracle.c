/*
 * oracle.c — plain, slow, fp64 CPU oracle for paged GQA single-token decode attention.
 *
 * TEST INFRASTRUCTURE ONLY. It is called by the tests, by the smoke check and by the CPU-baseline
 * leg of the benchmark, never by the product path. It shares no code, header, table or helper with
 * the GPU library: it is written straight from the definition of decode attention, in the order
 * the definition gives, so it can be checked by eye.
 *
 * Definition followed (decode = one new query token per sequence attending its cached keys:
 * vLLM learning notes "模型库与算子层 — 概念", section "核心操作"; GQA query-head groups sharing a
 * KV head and the two Gemma-4 layer kinds, global and sliding-window: Sparse-vLLM PR #27
 * "feat: support Gemma 4 and native multimodal inference", sections "Gemma 4 文本推理" and
 * "专用算子与性能优化"; the split-KV partials and their log-sum-exp merge: vLLM learning notes,
 * section "MLA 与 Sparse MLA（DSA）"):
 *
 *   for sequence b, query head h, KV head g = h / G (G = Hq / Hkv):
 *     keys t in [lo, hi): page = block_table[b, t / S], slot = t % S,
 *                          K_t = k_pool[page, g, slot, :], V_t = v_pool[page, g, slot, :]
 *     s_t  = scale * sum_d q[b, h, d] * K_t[d]
 *     m    = max_t s_t,  Z = sum_t exp(s_t - m)
 *     out  = sum_t exp(s_t - m) * V_t / Z,   lse = m + ln Z
 *   with lo = 0 (global) or max(0, n - W) (sliding window W) and hi = n = ctx_lens[b].
 *   An empty key range gives out = 0 and lse = -inf.
 *
 * Precision: inputs are bf16 bit patterns; each converts to fp64 exactly; all arithmetic is fp64
 * (no fused or reordered reductions beyond what is written). Build without -ffast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_OK = 0, ORACLE_BAD_ARG = 1, ORACLE_BAD_PAGE = 2, ORACLE_NO_MEMORY = 3 };

/* bf16 is the top 16 bits of an IEEE-754 binary32 value. */
static double bf16_bits_to_double(uint16_t bits) {
  uint32_t word = ((uint32_t)bits) << 16;
  float value;
  memcpy(&value, &word, sizeof value);
  return (double)value;
}

/* Keys attended by a sequence of n cached keys: all of them (window 0) or the last `window`. */
void oracle_key_range(int32_t n, int32_t window, int32_t* lo, int32_t* hi) {
  if (n < 0) n = 0;
  *hi = n;
  *lo = (window > 0 && n > window) ? n - window : 0;
}

/*
 * Attention of query row (b, h) over an explicit, increasing list of key positions keys[0..count):
 * gather K_t / V_t of KV head g from the pages, s_t = scale * <q_h, K_t>, softmax, weighted sum of
 * V. Writes out[0..D) and *lse; returns ORACLE_BAD_PAGE if a key maps outside the table or pool.
 */
static int attend_keys(int32_t b, int32_t g, int32_t Hkv, int32_t D, int32_t S,
                       int32_t max_pages_per_seq, int32_t num_pages, const uint16_t* qh,
                       const uint16_t* k_pool, const uint16_t* v_pool, const int32_t* block_table,
                       const int32_t* keys, int32_t count, double scale, double* o, double* lse) {
  for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
  if (count <= 0) {
    *lse = -INFINITY;
    return ORACLE_OK;
  }
  double* s = (double*)malloc(sizeof(double) * (size_t)count);
  const uint16_t** vrow = (const uint16_t**)malloc(sizeof(uint16_t*) * (size_t)count);
  if (!s || !vrow) {
    free(s);
    free(vrow);
    return ORACLE_NO_MEMORY;
  }

  /* Gather and scores: s_t = scale * <q_h, K_t>. */
  double m = -INFINITY;
  for (int32_t i = 0; i < count; ++i) {
    const int32_t t = keys[i];
    const int32_t col = t / S;
    const int32_t page = col < max_pages_per_seq
                             ? block_table[(int64_t)b * max_pages_per_seq + col] : -1;
    if (page < 0 || page >= num_pages) {
      free(s);
      free(vrow);
      return ORACLE_BAD_PAGE;
    }
    const int64_t base = (((int64_t)page * Hkv + g) * S + (t % S)) * D;
    const uint16_t* krow = k_pool + base;
    double dot = 0.0;
    for (int32_t d = 0; d < D; ++d) dot += bf16_bits_to_double(qh[d]) * bf16_bits_to_double(krow[d]);
    s[i] = scale * dot;
    vrow[i] = v_pool + base;
    if (s[i] > m) m = s[i];
  }

  /* Softmax weights exp(s_t - m), their sum Z, and the weighted sum of values. */
  double Z = 0.0;
  for (int32_t i = 0; i < count; ++i) {
    const double e = exp(s[i] - m);
    Z += e;
    const uint16_t* v = vrow[i];
    for (int32_t d = 0; d < D; ++d) o[d] += e * bf16_bits_to_double(v[d]);
  }
  for (int32_t d = 0; d < D; ++d) o[d] /= Z;
  *lse = m + log(Z);
  free(s);
  free(vrow);
  return ORACLE_OK;
}

/*
 * Attention of every (b, h) over per-sequence key sets: the range [key_lo[b], key_hi[b]) plus,
 * when sink_len is given, the leading keys [0, min(sink_len[b], key_hi[b])) (each key once, in
 * increasing order). q [B, Hq, D], pools [P, Hkv, S, D] (bf16 bits), block_table
 * [B, max_pages_per_seq]; out [B, Hq, D] and lse [B, Hq] in fp64. num_threads <= 0 uses the
 * OpenMP default. Returns ORACLE_BAD_PAGE if a key maps outside the table row or the pool.
 */
static int attend_sets(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t S,
                       int32_t max_pages_per_seq, int32_t num_pages, const uint16_t* q,
                       const uint16_t* k_pool, const uint16_t* v_pool, const int32_t* block_table,
                       const int32_t* key_lo, const int32_t* key_hi, const int32_t* sink_len,
                       double scale, double* out, double* lse, int32_t num_threads) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || S <= 0 || Hq % Hkv != 0) return ORACLE_BAD_ARG;
  if (B == 0) return ORACLE_OK;
  if (!q || !k_pool || !v_pool || !block_table || !key_lo || !key_hi || !out || !lse)
    return ORACLE_BAD_ARG;
  const int32_t G = Hq / Hkv;
  int status = ORACLE_OK;

#ifdef _OPENMP
  if (num_threads > 0) omp_set_num_threads(num_threads);
#else
  (void)num_threads;
#endif

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t row = 0; row < (int64_t)B * Hq; ++row) {
    const int32_t b = (int32_t)(row / Hq);
    const int32_t h = (int32_t)(row % Hq);
    const int32_t g = h / G; /* GQA: query heads [g*G, (g+1)*G) share KV head g */
    const int32_t lo = key_lo[b] < 0 ? 0 : key_lo[b];
    const int32_t hi = key_hi[b];
    int32_t sk = sink_len ? sink_len[b] : 0;
    if (sk > hi) sk = hi;
    if (sk > lo) sk = lo; /* leading keys that the range does not already hold */
    if (sk < 0) sk = 0;
    const int32_t count = sk + (hi > lo ? hi - lo : 0);
    int32_t* keys = (int32_t*)malloc(sizeof(int32_t) * (size_t)(count > 0 ? count : 1));
    int rc = ORACLE_NO_MEMORY;
    if (keys) {
      int32_t c = 0;
      for (int32_t t = 0; t < sk; ++t) keys[c++] = t;
      for (int32_t t = lo; t < hi; ++t) keys[c++] = t;
      rc = attend_keys(b, g, Hkv, D, S, max_pages_per_seq, num_pages, q + row * D, k_pool, v_pool,
                       block_table, keys, count, scale, out + row * D, lse + row);
      free(keys);
    }
    if (rc != ORACLE_OK) {
#pragma omp critical
      status = rc;
    }
  }
  return status;
}

/* Attention of every (b, h) over explicit per-sequence key ranges [key_lo[b], key_hi[b]). */
int oracle_decode_attn_ranges(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t S,
                              int32_t max_pages_per_seq, int32_t num_pages, const uint16_t* q,
                              const uint16_t* k_pool, const uint16_t* v_pool,
                              const int32_t* block_table, const int32_t* key_lo,
                              const int32_t* key_hi, double scale, double* out, double* lse,
                              int32_t num_threads) {
  return attend_sets(B, Hq, Hkv, D, S, max_pages_per_seq, num_pages, q, k_pool, v_pool,
                     block_table, key_lo, key_hi, NULL, scale, out, lse, num_threads);
}

/*
 * The definition with the key range of each sequence taken from its context length and the
 * window (0 = global layer). See oracle_key_range.
 */
int oracle_decode_attn(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t S,
                       int32_t max_pages_per_seq, int32_t num_pages, const uint16_t* q,
                       const uint16_t* k_pool, const uint16_t* v_pool, const int32_t* block_table,
                       const int32_t* ctx_lens, int32_t window, double scale, double* out,
                       double* lse, int32_t num_threads) {
  if (B < 0 || (B > 0 && !ctx_lens)) return ORACLE_BAD_ARG;
  if (B == 0) return ORACLE_OK;
  int32_t* lo = (int32_t*)malloc(sizeof(int32_t) * (size_t)B);
  int32_t* hi = (int32_t*)malloc(sizeof(int32_t) * (size_t)B);
  if (!lo || !hi) {
    free(lo);
    free(hi);
    return ORACLE_NO_MEMORY;
  }
  for (int32_t b = 0; b < B; ++b) oracle_key_range(ctx_lens[b], window, &lo[b], &hi[b]);
  const int rc = oracle_decode_attn_ranges(B, Hq, Hkv, D, S, max_pages_per_seq, num_pages, q, k_pool,
                                           v_pool, block_table, lo, hi, scale, out, lse, num_threads);
  free(lo);
  free(hi);
  return rc;
}

/*
 * A sliding layer with attention sinks (StreamingLLM-style views: Sparse-vLLM PR #27, section
 * "Gemma 4 文本推理"): each sequence attends its last `window` keys and, in addition, its first
 * `sink` keys, i.e. t in [0, min(sink, n)) or t in [max(0, n - window), n). window 0 attends all
 * keys (sink then changes nothing).
 */
int oracle_decode_attn_sink(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t S,
                            int32_t max_pages_per_seq, int32_t num_pages, const uint16_t* q,
                            const uint16_t* k_pool, const uint16_t* v_pool,
                            const int32_t* block_table, const int32_t* ctx_lens, int32_t window,
                            int32_t sink, double scale, double* out, double* lse,
                            int32_t num_threads) {
  if (B < 0 || (B > 0 && !ctx_lens) || sink < 0) return ORACLE_BAD_ARG;
  if (B == 0) return ORACLE_OK;
  int32_t* lo = (int32_t*)malloc(sizeof(int32_t) * (size_t)B);
  int32_t* hi = (int32_t*)malloc(sizeof(int32_t) * (size_t)B);
  int32_t* sk = (int32_t*)malloc(sizeof(int32_t) * (size_t)B);
  if (!lo || !hi || !sk) {
    free(lo);
    free(hi);
    free(sk);
    return ORACLE_NO_MEMORY;
  }
  for (int32_t b = 0; b < B; ++b) {
    oracle_key_range(ctx_lens[b], window, &lo[b], &hi[b]);
    sk[b] = sink;
  }
  const int rc = attend_sets(B, Hq, Hkv, D, S, max_pages_per_seq, num_pages, q, k_pool, v_pool,
                             block_table, lo, hi, sk, scale, out, lse, num_threads);
  free(lo);
  free(hi);
  free(sk);
  return rc;
}

/*
 * Multi-token decode: L new query tokens per sequence (speculative verification or a short
 * chunk of prefill; vLLM learning notes "模型库与算子层 — 概念", section "核心操作" for prefill
 * vs decode and the MLA backend notes on causal multi-token verification). The last L of the n
 * cached keys of sequence b belong to the new tokens; query i (0 <= i < L) sits at position
 * p = n - L + i and attends causally, exactly as a single-token decode whose context ends at p:
 * keys t <= p, t >= max(0, p + 1 - W) for a sliding window W, plus t < min(sink, p + 1) for a
 * sliding layer with sinks. A query with p < 0 attends nothing (out 0, lse -inf).
 * q and out are [B, L, Hq, D], lse [B, L, Hq].
 */
int oracle_decode_attn_multi(int32_t B, int32_t L, int32_t Hq, int32_t Hkv, int32_t D, int32_t S,
                             int32_t max_pages_per_seq, int32_t num_pages, const uint16_t* q,
                             const uint16_t* k_pool, const uint16_t* v_pool,
                             const int32_t* block_table, const int32_t* ctx_lens, int32_t window,
                             int32_t sink, double scale, double* out, double* lse,
                             int32_t num_threads) {
  if (B < 0 || L < 1 || Hq <= 0 || Hkv <= 0 || D <= 0 || S <= 0 || Hq % Hkv != 0 || sink < 0)
    return ORACLE_BAD_ARG;
  if (B == 0) return ORACLE_OK;
  if (!q || !k_pool || !v_pool || !block_table || !ctx_lens || !out || !lse) return ORACLE_BAD_ARG;
  const int32_t G = Hq / Hkv;
  int status = ORACLE_OK;

#ifdef _OPENMP
  if (num_threads > 0) omp_set_num_threads(num_threads);
#else
  (void)num_threads;
#endif

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t row = 0; row < (int64_t)B * L * Hq; ++row) {
    const int32_t h = (int32_t)(row % Hq);
    const int32_t i = (int32_t)((row / Hq) % L);
    const int32_t b = (int32_t)(row / ((int64_t)Hq * L));
    const int32_t n = ctx_lens[b] < 0 ? 0 : ctx_lens[b];
    const int32_t p = n - L + i; /* position of query i */
    int32_t lo = 0, hi = 0;
    oracle_key_range(p + 1, window, &lo, &hi); /* the context of query i ends at p */
    int32_t sk = window > 0 ? sink : 0;
    if (sk > lo) sk = lo; /* leading keys the window does not already hold */
    const int32_t count = sk + (hi > lo ? hi - lo : 0);
    int32_t* keys = (int32_t*)malloc(sizeof(int32_t) * (size_t)(count > 0 ? count : 1));
    int rc = ORACLE_NO_MEMORY;
    if (keys) {
      int32_t c = 0;
      for (int32_t t = 0; t < sk; ++t) keys[c++] = t;
      for (int32_t t = lo; t < hi; ++t) keys[c++] = t;
      rc = attend_keys(b, h / G, Hkv, D, S, max_pages_per_seq, num_pages, q + row * D, k_pool,
                       v_pool, block_table, keys, count, scale, out + row * D, lse + row);
      free(keys);
    }
    if (rc != ORACLE_OK) {
#pragma omp critical
      status = rc;
    }
  }
  return status;
}

/*
 * Log-sum-exp merge of split partials. For each of `rows` rows, `splits` partial outputs
 * o_parts[row, s, :D] with log-sum-exps lses[row, s] (lse = -inf marks an empty part):
 *     M = max_s lse_s,  w_s = exp(lse_s - M),  W = sum_s w_s,
 *     out[row, :] = sum_s w_s * o_s / W,   lse_out[row] = M + ln W
 * and out = 0, lse_out = -inf when every part is empty. This is the identity
 * softmax over a union of disjoint key sets = LSE-weighted mixture of per-set softmaxes.
 */
int oracle_lse_merge(int32_t rows, int32_t splits, int32_t D, const double* o_parts,
                     const double* lses, double* out, double* lse_out) {
  if (rows < 0 || splits <= 0 || D <= 0) return ORACLE_BAD_ARG;
  for (int64_t r = 0; r < rows; ++r) {
    const double* l = lses + r * splits;
    double* o = out + r * D;
    double M = -INFINITY;
    for (int32_t s = 0; s < splits; ++s)
      if (l[s] > M) M = l[s];
    for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
    if (M == -INFINITY) {
      lse_out[r] = -INFINITY;
      continue;
    }
    double W = 0.0;
    for (int32_t s = 0; s < splits; ++s) {
      const double w = exp(l[s] - M);
      W += w;
      const double* part = o_parts + (r * splits + s) * D;
      for (int32_t d = 0; d < D; ++d) o[d] += w * part[d];
    }
    for (int32_t d = 0; d < D; ++d) o[d] /= W;
    lse_out[r] = M + log(W);
  }
  return ORACLE_OK;
}

/*
 * Paged KV append: the L newest tokens of each sequence (positions n - L .. n - 1, n = ctx_lens[b];
 * the context length counts them) are written into their slots: token i of the L goes to
 * position t = n - L + i, page block_table[b, t / S], slot t % S, for every KV head g:
 * pool[page, g, slot, :] = new[b, i, g, :] (new is [B, L, Hkv, D]). Positions below 0 are
 * skipped. When v_pool == k_pool (layers whose values are their keys) only K is written.
 * Returns ORACLE_BAD_PAGE if a slot lies outside the table row or the pool (nothing written for
 * that token).
 */
int oracle_append_kv(int32_t B, int32_t L, int32_t Hkv, int32_t D, int32_t S,
                     int32_t max_pages_per_seq, int32_t num_pages, const uint16_t* k_new,
                     const uint16_t* v_new, uint16_t* k_pool, uint16_t* v_pool,
                     const int32_t* block_table, const int32_t* ctx_lens) {
  if (B < 0 || L < 1 || Hkv <= 0 || D <= 0 || S <= 0) return ORACLE_BAD_ARG;
  int status = ORACLE_OK;
  for (int32_t b = 0; b < B; ++b) {
    for (int32_t i = 0; i < L; ++i) {
      const int32_t t = ctx_lens[b] - L + i;
      if (t < 0) continue;
      const int32_t col = t / S;
      if (col >= max_pages_per_seq) { status = ORACLE_BAD_PAGE; continue; }
      const int32_t page = block_table[(int64_t)b * max_pages_per_seq + col];
      if (page < 0 || page >= num_pages) { status = ORACLE_BAD_PAGE; continue; }
      for (int32_t g = 0; g < Hkv; ++g) {
        const int64_t dst = (((int64_t)page * Hkv + g) * S + (t % S)) * D;
        const int64_t src = (((int64_t)b * L + i) * Hkv + g) * D;
        for (int32_t d = 0; d < D; ++d) k_pool[dst + d] = k_new[src + d];
        if (v_pool != k_pool)
          for (int32_t d = 0; d < D; ++d) v_pool[dst + d] = v_new[src + d];
      }
    }
  }
  return status;
}

/* Threads the OpenMP runtime would use (reported by the CPU baseline). */
int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
