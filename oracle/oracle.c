/*
 * oracle.c -- plain, slow, fp64 CPU reference for one paged decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library includes, links
 * or calls this file; only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load it.  It shares no code, header or constant with the
 * GPU path.
 *
 * What it computes (sources are the pages this project follows):
 *  - Attention(Q,K,V) = softmax(Q K^T / sqrt(d_head)) V, evaluated for one
 *    query row per (sequence, query head): page "x321.org/?p=939", section
 *    "First understand what the KV cache is storing".
 *  - The cache is cut into fixed-size blocks; a per-sequence table maps each
 *    logical block to a physical block anywhere in the pool, and attention
 *    follows that mapping while the logical order stays intact: same page,
 *    section "PagedAttention borrows an operating-system trick"; page
 *    "chenhuiyu.github.io/blog/llm-infra-vllm-en", sections "Why naive KV
 *    allocation wastes memory" and "Logical continuity, physical flexibility".
 *  - The cache grows by one token per decode step, appended after the old
 *    ones: page "x321.org/?p=939", section "First understand what the KV
 *    cache is storing".
 *
 * Readings where the pages leave a step open (stated once here, and in the
 * design notes):
 *  - Block layout: K and V pools are each [num_blocks][num_kv_heads]
 *    [block_size][head_dim], row-major.
 *  - A slot is physical_block * block_size + offset; a negative slot is
 *    skipped.
 *  - context_lens[i] counts every valid token of sequence i, including the
 *    token written in this step.
 *  - Query head h reads KV head h / (num_q_heads / num_kv_heads).
 *  - scale is given as an fp32 number and widened to fp64 here.
 *  - A sequence with no tokens yields an all-zero output row.
 *
 * Element storage: elem_bytes 4 = IEEE binary32, 2 = bfloat16 (the upper
 * 16 bits of a binary32).  Every stored value is widened to fp64 exactly.
 */
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_ERR_ARGS (-1)
#define ORACLE_ERR_SLOT (-2)
#define ORACLE_ERR_TABLE (-3)
#define ORACLE_ERR_LEN (-4)
#define ORACLE_ERR_NOMEM (-5)

/* Widen element idx of an array of bf16 or fp32 values to fp64 (exact). */
static double load_elem(const void *base, int64_t idx, int elem_bytes)
{
    float f;
    if (elem_bytes == 4) {
        memcpy(&f, (const char *)base + idx * 4, 4);
    } else {
        uint16_t b;
        uint32_t u;
        memcpy(&b, (const char *)base + idx * 2, 2);
        u = ((uint32_t)b) << 16;
        memcpy(&f, &u, 4);
    }
    return (double)f;
}

/*
 * Append step: token t's key and value rows go to slot slot_mapping[t],
 * i.e. physical block slot / block_size at offset slot % block_size, for
 * every KV head.  The copy is of raw bytes, so every bit pattern (NaN
 * payloads, -0.0, subnormals) arrives unchanged.
 *
 * k_new, v_new: [num_tokens][num_kv_heads][head_dim]
 * k_cache, v_cache: [num_blocks][num_kv_heads][block_size][head_dim], updated in place.
 */
int oracle_kv_write(const void *k_new, const void *v_new, const int32_t *slot_mapping,
                    int32_t num_tokens, void *k_cache, void *v_cache, int32_t num_blocks,
                    int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                    int32_t elem_bytes)
{
    int32_t t, h;
    int64_t row_bytes;
    if (num_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0 || block_size <= 0 ||
        head_dim <= 0 || (elem_bytes != 2 && elem_bytes != 4))
        return ORACLE_ERR_ARGS;
    row_bytes = (int64_t)head_dim * elem_bytes;
    for (t = 0; t < num_tokens; ++t) {
        int64_t slot = slot_mapping[t];
        int64_t blk, off;
        if (slot < 0)
            continue;
        blk = slot / block_size;
        off = slot % block_size;
        if (blk >= num_blocks)
            return ORACLE_ERR_SLOT;
        for (h = 0; h < num_kv_heads; ++h) {
            int64_t dst = ((blk * num_kv_heads + h) * block_size + off) * row_bytes;
            int64_t src = ((int64_t)t * num_kv_heads + h) * row_bytes;
            memcpy((char *)k_cache + dst, (const char *)k_new + src, (size_t)row_bytes);
            memcpy((char *)v_cache + dst, (const char *)v_new + src, (size_t)row_bytes);
        }
    }
    return ORACLE_OK;
}

/*
 * One output row: sequence i, query head h.
 *
 * 1. Rebuild the sequence's keys and values for KV head g in logical order:
 *    token j lives in physical block block_tables[i][j / block_size] at
 *    offset j % block_size.  Only the first ceil(n / block_size) table
 *    entries are touched.
 * 2. s_j = scale * sum_x q[i][h][x] * K[j][x]           (scores)
 * 3. w_j = exp(s_j - max_j s_j);  out = sum_j w_j V[j] / sum_j w_j   (softmax . V)
 */
static int attend_one(const void *q, const void *k_cache, const void *v_cache, int elem_bytes,
                      const int32_t *block_tables, int32_t max_blocks_per_seq,
                      const int32_t *context_lens, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t num_blocks, int32_t block_size, int32_t head_dim, double scale,
                      int32_t i, int32_t h, double *out_row)
{
    const int64_t D = head_dim;
    const int32_t group = num_q_heads / num_kv_heads;
    const int32_t g = h / group;
    const int64_t n = context_lens[i];
    double *kh, *vh, *s, *qv;
    double m, denom;
    int64_t j, x;

    for (x = 0; x < D; ++x)
        out_row[x] = 0.0;
    if (n == 0)
        return ORACLE_OK;
    if (n < 0 || n > (int64_t)max_blocks_per_seq * block_size)
        return ORACLE_ERR_LEN;

    kh = (double *)malloc(sizeof(double) * (size_t)(n * D));
    vh = (double *)malloc(sizeof(double) * (size_t)(n * D));
    s = (double *)malloc(sizeof(double) * (size_t)n);
    qv = (double *)malloc(sizeof(double) * (size_t)D);
    if (!kh || !vh || !s || !qv) {
        free(kh); free(vh); free(s); free(qv);
        return ORACLE_ERR_NOMEM;
    }

    /* step 1: logical K and V rows of this sequence, for KV head g */
    for (j = 0; j < n; ++j) {
        int64_t phys = block_tables[(int64_t)i * max_blocks_per_seq + j / block_size];
        int64_t off = j % block_size;
        int64_t base;
        if (phys < 0 || phys >= num_blocks) {
            free(kh); free(vh); free(s); free(qv);
            return ORACLE_ERR_TABLE;
        }
        base = ((phys * num_kv_heads + g) * block_size + off) * D;
        for (x = 0; x < D; ++x) {
            kh[j * D + x] = load_elem(k_cache, base + x, elem_bytes);
            vh[j * D + x] = load_elem(v_cache, base + x, elem_bytes);
        }
    }
    for (x = 0; x < D; ++x)
        qv[x] = load_elem(q, ((int64_t)i * num_q_heads + h) * D + x, elem_bytes);

    /* step 2: scaled scores */
    for (j = 0; j < n; ++j) {
        double acc = 0.0;
        for (x = 0; x < D; ++x)
            acc += qv[x] * kh[j * D + x];
        s[j] = scale * acc;
    }

    /* step 3: softmax over the n scores, then the weighted sum of values */
    m = s[0];
    for (j = 1; j < n; ++j)
        if (s[j] > m)
            m = s[j];
    denom = 0.0;
    for (j = 0; j < n; ++j) {
        s[j] = exp(s[j] - m);
        denom += s[j];
    }
    for (j = 0; j < n; ++j)
        for (x = 0; x < D; ++x)
            out_row[x] += s[j] * vh[j * D + x];
    for (x = 0; x < D; ++x)
        out_row[x] /= denom;

    free(kh); free(vh); free(s); free(qv);
    return ORACLE_OK;
}

/*
 * Decode attention for a batch.
 *
 * q: [num_seqs][num_q_heads][head_dim]; caches as in oracle_kv_write;
 * block_tables: [num_seqs][max_blocks_per_seq]; context_lens: [num_seqs].
 * rows == NULL: every (sequence, head), out is [num_seqs][num_q_heads][head_dim].
 * rows != NULL: num_rows pairs (sequence, head), out is [num_rows][head_dim].
 * Rows are independent; OpenMP spreads them over the host cores.
 */
int oracle_attn_decode(const void *q, const void *k_cache, const void *v_cache,
                       int32_t elem_bytes, const int32_t *block_tables,
                       int32_t max_blocks_per_seq, const int32_t *context_lens,
                       int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t num_blocks, int32_t block_size, int32_t head_dim, float scale,
                       const int32_t *rows, int32_t num_rows, double *out)
{
    int64_t r, total;
    int err = ORACLE_OK;
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
        num_q_heads % num_kv_heads != 0 || num_blocks <= 0 || block_size <= 0 ||
        head_dim <= 0 || max_blocks_per_seq <= 0 || (elem_bytes != 2 && elem_bytes != 4))
        return ORACLE_ERR_ARGS;
    total = rows ? (int64_t)num_rows : (int64_t)num_seqs * num_q_heads;

#pragma omp parallel for schedule(dynamic, 1)
    for (r = 0; r < total; ++r) {
        int32_t i = rows ? rows[2 * r] : (int32_t)(r / num_q_heads);
        int32_t h = rows ? rows[2 * r + 1] : (int32_t)(r % num_q_heads);
        int e;
        if (i < 0 || i >= num_seqs || h < 0 || h >= num_q_heads) {
            e = ORACLE_ERR_ARGS;
        } else {
            e = attend_one(q, k_cache, v_cache, elem_bytes, block_tables, max_blocks_per_seq,
                           context_lens, num_q_heads, num_kv_heads, num_blocks, block_size,
                           head_dim, (double)scale, i, h, out + r * head_dim);
        }
        if (e != ORACLE_OK) {
#pragma omp critical
            err = e;
        }
    }
    return err;
}

/* Host threads the row loop above may use (reported beside CPU timings). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Several new tokens per sequence (a chunk of a prefill split into chunks,
 * page "x321.org/?p=939", section "Continuous batching is the other half of
 * the story"; attention over the existing context during autoregressive
 * generation, section "First understand what the KV cache is storing").
 *
 * Sequence i holds n = context_lens[i] tokens, the last q_len = cu_q[i + 1] -
 * cu_q[i] of them new.  Query row j of the sequence is the token at position
 * p = n - q_len + j and attends to tokens 0 .. p of the sequence (the ones it
 * would have seen had they been generated one at a time):
 *   out[cu_q[i] + j][h] = sum_{t <= p} w_t V[t] / sum_{t <= p} w_t,
 *   w_t = exp(s_t - max_{u <= p} s_u),  s_t = scale * q[cu_q[i] + j][h] . K[t].
 *
 * q, out: [total_q][num_q_heads][head_dim] with total_q = cu_q[num_seqs];
 * other arguments as oracle_attn_decode.  ORACLE_ERR_LEN if q_len > n or
 * q_len < 0.
 */
static int attend_causal(const void *q, const void *k_cache, const void *v_cache, int elem_bytes,
                         const int32_t *block_tables, int32_t max_blocks_per_seq, int64_t n,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t num_blocks,
                         int32_t block_size, int32_t head_dim, double scale, int32_t i,
                         int64_t qrow, int64_t pos, int32_t h, double *out_row)
{
    const int64_t D = head_dim;
    const int32_t g = h / (num_q_heads / num_kv_heads);
    const int64_t visible = pos + 1;
    double *s, *qv;
    double m, denom;
    int64_t t, x;

    for (x = 0; x < D; ++x)
        out_row[x] = 0.0;
    if (n > (int64_t)max_blocks_per_seq * block_size)
        return ORACLE_ERR_LEN;
    s = (double *)malloc(sizeof(double) * (size_t)visible);
    qv = (double *)malloc(sizeof(double) * (size_t)D);
    if (!s || !qv) {
        free(s); free(qv);
        return ORACLE_ERR_NOMEM;
    }
    for (x = 0; x < D; ++x)
        qv[x] = load_elem(q, (qrow * num_q_heads + h) * D + x, elem_bytes);
    /* scores of the visible tokens, each key read through the block table */
    for (t = 0; t < visible; ++t) {
        int64_t phys = block_tables[(int64_t)i * max_blocks_per_seq + t / block_size];
        int64_t base;
        double acc = 0.0;
        if (phys < 0 || phys >= num_blocks) {
            free(s); free(qv);
            return ORACLE_ERR_TABLE;
        }
        base = ((phys * num_kv_heads + g) * block_size + t % block_size) * D;
        for (x = 0; x < D; ++x)
            acc += qv[x] * load_elem(k_cache, base + x, elem_bytes);
        s[t] = scale * acc;
    }
    m = s[0];
    for (t = 1; t < visible; ++t)
        if (s[t] > m)
            m = s[t];
    denom = 0.0;
    for (t = 0; t < visible; ++t) {
        s[t] = exp(s[t] - m);
        denom += s[t];
    }
    for (t = 0; t < visible; ++t) {
        int64_t phys = block_tables[(int64_t)i * max_blocks_per_seq + t / block_size];
        int64_t base = ((phys * num_kv_heads + g) * block_size + t % block_size) * D;
        for (x = 0; x < D; ++x)
            out_row[x] += s[t] * load_elem(v_cache, base + x, elem_bytes);
    }
    for (x = 0; x < D; ++x)
        out_row[x] /= denom;
    free(s); free(qv);
    return ORACLE_OK;
}

int oracle_attn_multi(const void *q, const void *k_cache, const void *v_cache, int32_t elem_bytes,
                      const int32_t *block_tables, int32_t max_blocks_per_seq,
                      const int32_t *context_lens, const int32_t *cu_q, int32_t num_seqs,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t num_blocks,
                      int32_t block_size, int32_t head_dim, float scale, double *out)
{
    int64_t total, r;
    int32_t i;
    int32_t *row_seq;
    int err = ORACLE_OK;
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
        num_q_heads % num_kv_heads != 0 || num_blocks <= 0 || block_size <= 0 ||
        head_dim <= 0 || max_blocks_per_seq <= 0 || (elem_bytes != 2 && elem_bytes != 4) ||
        cu_q[0] != 0)
        return ORACLE_ERR_ARGS;
    for (i = 0; i < num_seqs; ++i) {
        const int32_t ql = cu_q[i + 1] - cu_q[i];
        if (ql < 0 || ql > context_lens[i])
            return ORACLE_ERR_LEN;
    }
    total = cu_q[num_seqs];
    row_seq = (int32_t *)malloc(sizeof(int32_t) * (size_t)(total > 0 ? total : 1));
    if (!row_seq)
        return ORACLE_ERR_NOMEM;
    for (i = 0; i < num_seqs; ++i)
        for (r = cu_q[i]; r < cu_q[i + 1]; ++r)
            row_seq[r] = i;

#pragma omp parallel for schedule(dynamic, 1)
    for (r = 0; r < total * num_q_heads; ++r) {
        const int64_t qrow = r / num_q_heads;
        const int32_t h = (int32_t)(r % num_q_heads);
        const int32_t s = row_seq[qrow];
        const int64_t n = context_lens[s];
        const int64_t ql = cu_q[s + 1] - cu_q[s];
        const int64_t pos = n - ql + (qrow - cu_q[s]);
        int e = attend_causal(q, k_cache, v_cache, elem_bytes, block_tables, max_blocks_per_seq, n,
                              num_q_heads, num_kv_heads, num_blocks, block_size, head_dim,
                              (double)scale, s, qrow, pos, h, out + r * head_dim);
        if (e != ORACLE_OK) {
#pragma omp critical
            err = e;
        }
    }
    free(row_seq);
    return err;
}
