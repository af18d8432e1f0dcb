/*
 * pa_oracle.c -- plain, slow, fp64 CPU oracle for paged KV-cache attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this code.  The product library
 * (paged_kv_cache_275_amd) never links, imports or calls it, and it shares no
 * code, header or constant with the HIP kernels.
 *
 * What it computes, and where the pages define it:
 *
 *  - A KV cache split into fixed-size blocks of tokens ("e.g. 16 tokens"),
 *    page "轻量级的vLLM" (mini-vllm write-up), section 核心机制一：分页 KV Cache.
 *  - Each request owns a block table; logically contiguous tokens live in
 *    physically scattered blocks and attention finds the real K and V through
 *    the block table: page "从零实现一个 mini vLLM--开篇", section
 *    "5. 这个系列会怎么展开" (stages four and five), and page "vllm-v0 版本介绍",
 *    section 为什么需要推理框架？ (PagedAttention item).
 *  - Decode computes only the new token's key/value and appends them to the
 *    cache; the new token must still see every earlier token's K/V:
 *    page "从零实现一个 mini vLLM--开篇", section "2. LLM 推理到底在慢什么".
 *  - Chunked prefill is only named (same page, section 5, stage six); the
 *    reading used here: chunk row i of a sequence with c chunk rows and
 *    context length N sits at absolute position N - c + i and attends to
 *    positions 0..N - c + i inclusive.
 *
 * Paging changes where K/V live, not the mathematics: every function below is
 * exact softmax attention written out token by token, in fp64, resolving the
 * block table for every single token.  No blocking, no online softmax, no
 * fusion.
 *
 * Element types: 0 = IEEE fp32, 1 = bfloat16 (upper 16 bits of an fp32),
 * 2 = IEEE fp64 (for inputs that are exact only in fp64, such as a dequantized
 * fp8 cache: scale * e4m3 value).
 * Layouts (all row-major, contiguous):
 *   q, key, value      [rows, heads, head_dim]
 *   k_cache, v_cache   [num_blocks, block_size, num_kv_heads, head_dim]
 *   block_tables       [num_seqs, max_blocks_per_seq] int32
 *   slot_mapping       [num_tokens] int32, slot = block * block_size + offset,
 *                      negative = skip
 * Every function returns 0 on success and a negative code when an input
 * violates a precondition (out-of-range block id, duplicate slot, ...).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F64 = 2 };

static double elem_to_double(const void *base, int64_t idx, int dtype) {
    if (dtype == ORACLE_F32) {
        return (double)((const float *)base)[idx];
    }
    if (dtype == ORACLE_F64) {
        return ((const double *)base)[idx];
    }
    /* bfloat16: the 16 stored bits are the high half of an fp32 pattern. */
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static int elem_bytes(int dtype) { return dtype == ORACLE_F32 ? 4 : (dtype == ORACLE_F64 ? 8 : 2); }

/*
 * KV append: for each new token i whose slot is non-negative, its K row and
 * V row ([num_kv_heads, head_dim]) are copied, bit for bit, to
 * cache[slot / block_size, slot % block_size].
 */
int oracle_reshape_and_cache(const void *key, const void *value,
                             void *k_cache, void *v_cache,
                             const int32_t *slot_mapping, int64_t num_tokens,
                             int64_t num_kv_heads, int64_t head_dim,
                             int64_t block_size, int64_t num_blocks, int dtype) {
    const int64_t eb = elem_bytes(dtype);
    const int64_t n_slots = num_blocks * block_size;
    /* A slot written twice in one call has no unique result: reject it. */
    for (int64_t i = 0; i < num_tokens; ++i) {
        int64_t si = slot_mapping[i];
        if (si < 0) continue;
        if (si >= n_slots) return -1;
        for (int64_t j = 0; j < i; ++j) {
            if (slot_mapping[j] == si) return -2;
        }
    }
    for (int64_t i = 0; i < num_tokens; ++i) {
        int64_t slot = slot_mapping[i];
        if (slot < 0) continue;
        int64_t blk = slot / block_size;
        int64_t off = slot % block_size;
        for (int64_t h = 0; h < num_kv_heads; ++h) {
            for (int64_t d = 0; d < head_dim; ++d) {
                int64_t src = (i * num_kv_heads + h) * head_dim + d;
                int64_t dst = ((blk * block_size + off) * num_kv_heads + h) * head_dim + d;
                memcpy((char *)k_cache + dst * eb, (const char *)key + src * eb, (size_t)eb);
                memcpy((char *)v_cache + dst * eb, (const char *)value + src * eb, (size_t)eb);
            }
        }
    }
    return 0;
}

/*
 * One attention row: query vector qv (head_dim values, already in fp64)
 * against logical tokens 0..n_tokens-1 of one sequence, kv head kv.
 *   x_t = scale * sum_d q_d * K[t, d]
 *   w_t = exp(x_t - max_t x_t) / sum_u exp(x_u - max_t x_t)
 *   out = sum_t w_t * V[t, :]
 * Token t lives in physical block bt_row[t / block_size] at offset
 * t % block_size.  If weights is non-NULL it receives w_t (normalised).
 */
static int attend_row(double *out, const double *qv,
                      const void *k_cache, const void *v_cache,
                      const int32_t *bt_row, int64_t max_blocks,
                      int64_t n_tokens, int64_t kv, int64_t num_kv_heads,
                      int64_t head_dim, int64_t block_size, int64_t num_blocks,
                      double scale, int dtype, double *weights) {
    if (n_tokens == 0) {
        for (int64_t d = 0; d < head_dim; ++d) out[d] = 0.0;
        return 0;
    }
    if (n_tokens > max_blocks * block_size) return -3;
    double *x = (double *)malloc((size_t)n_tokens * sizeof(double));
    if (!x) return -9;
    for (int64_t t = 0; t < n_tokens; ++t) {
        int64_t blk = bt_row[t / block_size];
        int64_t off = t % block_size;
        if (blk < 0 || blk >= num_blocks) { free(x); return -4; }
        int64_t base = ((blk * block_size + off) * num_kv_heads + kv) * head_dim;
        double dot = 0.0;
        for (int64_t d = 0; d < head_dim; ++d) {
            dot += qv[d] * elem_to_double(k_cache, base + d, dtype);
        }
        x[t] = scale * dot;
    }
    double m = x[0];
    for (int64_t t = 1; t < n_tokens; ++t) {
        if (x[t] > m) m = x[t];
    }
    double z = 0.0;
    for (int64_t t = 0; t < n_tokens; ++t) {
        x[t] = exp(x[t] - m);
        z += x[t];
    }
    for (int64_t d = 0; d < head_dim; ++d) out[d] = 0.0;
    for (int64_t t = 0; t < n_tokens; ++t) {
        int64_t blk = bt_row[t / block_size];
        int64_t off = t % block_size;
        int64_t base = ((blk * block_size + off) * num_kv_heads + kv) * head_dim;
        double w = x[t] / z;
        if (weights) weights[t] = w;
        for (int64_t d = 0; d < head_dim; ++d) {
            out[d] += w * elem_to_double(v_cache, base + d, dtype);
        }
    }
    free(x);
    return 0;
}

static int check_heads(int64_t num_q_heads, int64_t num_kv_heads) {
    if (num_q_heads <= 0 || num_kv_heads <= 0) return -5;
    if (num_q_heads % num_kv_heads != 0) return -5;
    return 0;
}

/*
 * Decode: sequences s in [s_begin, s_end), every query head h.  Query head h
 * reads kv head h / (num_q_heads / num_kv_heads).  context_lens[s] counts
 * every cached token of the sequence, the one being decoded included.
 * out is fp64 [num_seqs, num_q_heads, head_dim]; only rows of the range are
 * written.
 */
int oracle_decode(double *out, const void *q,
                  const void *k_cache, const void *v_cache,
                  const int32_t *block_tables, int64_t max_blocks_per_seq,
                  const int32_t *context_lens, int64_t s_begin, int64_t s_end,
                  int64_t num_q_heads, int64_t num_kv_heads, int64_t head_dim,
                  int64_t block_size, int64_t num_blocks, double scale, int dtype) {
    int rc = check_heads(num_q_heads, num_kv_heads);
    if (rc) return rc;
    const int64_t group = num_q_heads / num_kv_heads;
    double *qv = (double *)malloc((size_t)head_dim * sizeof(double));
    if (!qv) return -9;
    for (int64_t s = s_begin; s < s_end && rc == 0; ++s) {
        int64_t n = context_lens[s];
        if (n < 0) { rc = -6; break; }
        for (int64_t h = 0; h < num_q_heads && rc == 0; ++h) {
            for (int64_t d = 0; d < head_dim; ++d) {
                qv[d] = elem_to_double(q, (s * num_q_heads + h) * head_dim + d, dtype);
            }
            rc = attend_row(out + (s * num_q_heads + h) * head_dim, qv, k_cache, v_cache,
                            block_tables + s * max_blocks_per_seq, max_blocks_per_seq, n,
                            h / group, num_kv_heads, head_dim, block_size, num_blocks,
                            scale, dtype, NULL);
        }
    }
    free(qv);
    return rc;
}

/*
 * Chunked prefill: sequence s owns query rows query_start_loc[s] ..
 * query_start_loc[s+1]-1 (c rows, the last c tokens of its context of
 * context_lens[s] tokens).  Row i of the chunk is at absolute position
 * p = context_lens[s] - c + i and attends causally to tokens 0..p inclusive.
 * out is fp64 [total_rows, num_q_heads, head_dim]; rows of sequences in
 * [s_begin, s_end) are written.
 */
int oracle_prefill(double *out, const void *q,
                   const void *k_cache, const void *v_cache,
                   const int32_t *block_tables, int64_t max_blocks_per_seq,
                   const int32_t *query_start_loc, const int32_t *context_lens,
                   int64_t s_begin, int64_t s_end,
                   int64_t num_q_heads, int64_t num_kv_heads, int64_t head_dim,
                   int64_t block_size, int64_t num_blocks, double scale, int dtype) {
    int rc = check_heads(num_q_heads, num_kv_heads);
    if (rc) return rc;
    const int64_t group = num_q_heads / num_kv_heads;
    double *qv = (double *)malloc((size_t)head_dim * sizeof(double));
    if (!qv) return -9;
    for (int64_t s = s_begin; s < s_end && rc == 0; ++s) {
        int64_t r0 = query_start_loc[s];
        int64_t c = query_start_loc[s + 1] - r0;
        int64_t n = context_lens[s];
        if (c < 0 || c > n) { rc = -7; break; }
        for (int64_t i = 0; i < c && rc == 0; ++i) {
            int64_t row = r0 + i;
            int64_t pos = n - c + i;
            for (int64_t h = 0; h < num_q_heads && rc == 0; ++h) {
                for (int64_t d = 0; d < head_dim; ++d) {
                    qv[d] = elem_to_double(q, (row * num_q_heads + h) * head_dim + d, dtype);
                }
                rc = attend_row(out + (row * num_q_heads + h) * head_dim, qv, k_cache, v_cache,
                                block_tables + s * max_blocks_per_seq, max_blocks_per_seq,
                                pos + 1, h / group, num_kv_heads, head_dim, block_size,
                                num_blocks, scale, dtype, NULL);
            }
        }
    }
    free(qv);
    return rc;
}

/*
 * The normalised softmax weights w_t of one decode row (sequence s, query
 * head h), written to weights[0..context_lens[s]-1], and that row's output.
 * Exposed so that tests can check properties of the weights themselves.
 */
int oracle_decode_row_weights(double *weights, double *out_row, const void *q,
                              const void *k_cache, const void *v_cache,
                              const int32_t *block_tables, int64_t max_blocks_per_seq,
                              const int32_t *context_lens, int64_t s, int64_t h,
                              int64_t num_q_heads, int64_t num_kv_heads, int64_t head_dim,
                              int64_t block_size, int64_t num_blocks, double scale,
                              int dtype) {
    int rc = check_heads(num_q_heads, num_kv_heads);
    if (rc) return rc;
    double *qv = (double *)malloc((size_t)head_dim * sizeof(double));
    if (!qv) return -9;
    for (int64_t d = 0; d < head_dim; ++d) {
        qv[d] = elem_to_double(q, (s * num_q_heads + h) * head_dim + d, dtype);
    }
    rc = attend_row(out_row, qv, k_cache, v_cache, block_tables + s * max_blocks_per_seq,
                    max_blocks_per_seq, context_lens[s], h / (num_q_heads / num_kv_heads),
                    num_kv_heads, head_dim, block_size, num_blocks, scale, dtype, weights);
    free(qv);
    return rc;
}
