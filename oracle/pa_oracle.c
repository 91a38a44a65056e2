/*
 * Plain fp64 CPU oracle for paged decode attention, the slot-mapped cache write and the block copy.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's CPU-baseline leg load this
 * file's library. It shares no code, header or table with the HIP library and must never be used as a
 * fallback for it. It is deliberately slow and written to be checked by eye against the pages:
 *
 *  - vLLM PagedAttention, page 1 ("LLM inference framework evaluation ... PagedAttention"), section 3.2: the KV
 *    cache is split into fixed-size blocks held in one global pool laid out as
 *    [num_blocks, block_size, num_heads, head_dim]; a sequence's tokens live in non-contiguous physical blocks
 *    and a per-sequence block table maps each logical position to its physical place. Page 3 (vLLM
 *    architecture), section 2.2, gives the example "logical block 0 -> physical block 7".
 *  - page 2 ("vLLM-v0.11.0 ... how much memory does PagedAttention save"), section 4.2: a sequence of
 *    length L occupies ceil(L / block_size) blocks.
 *  - page 1 section 3.1 and page 3 section 2.1: each decode step the new token reads the K and V of all
 *    previous tokens, and after sampling the new token's K/V is appended to the cache.
 *  - page 1 section 3.2 (sharing and copy-on-write): sequences may share physical blocks; a shared block is
 *    copied before it is written.
 *
 * Paging changes where K and V live, never what is attended, so decode attention is the plain definition
 * softmax(scale * q . K^T) . V over the logically ordered keys and values, computed here in fp64 after an
 * exact decode of every stored element (bf16 bits << 16 give the fp32 value; fp32 widens exactly to fp64).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_E4M3 2 /* OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities */

/*
 * Value of an OCP FP8 E4M3 code, from the format's definition: exponent field 15 with mantissa 7 is NaN;
 * exponent field 0 is subnormal, m * 2^-9; otherwise (1 + m / 8) * 2^(e - 7). Largest finite value 448.
 */
static double e4m3_value(uint8_t c) {
    const int e = (c >> 3) & 0xF, m = c & 7;
    const double sign = (c & 0x80) ? -1.0 : 1.0;
    if (e == 15 && m == 7) {
        return NAN;
    }
    if (e == 0) {
        return sign * ldexp((double)m, -9);
    }
    return sign * ldexp(1.0 + m / 8.0, e - 7);
}

/* One stored element, decoded exactly to fp64. */
static double elem(const void *base, int64_t index, int dtype) {
    if (dtype == ORACLE_F32) {
        return (double)((const float *)base)[index];
    }
    if (dtype == ORACLE_E4M3) {
        return e4m3_value(((const uint8_t *)base)[index]);
    }
    uint32_t bits = (uint32_t)((const uint16_t *)base)[index] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/*
 * Quantisation of the FP8 cache write: y = x / scale as an fp32 division (correctly rounded), saturated to
 * [-448, 448] (infinities included), then rounded to the nearest E4M3 value, ties to an even mantissa; NaN
 * becomes code 0x7F. Exact: the scalings below are by powers of two, and nearbyint rounds ties to even in the
 * default rounding mode.
 */
static uint8_t e4m3_quantize(float x, float scale) {
    const float y = x / scale;
    if (isnan(y)) {
        return 0x7F;
    }
    const uint8_t sign = signbit(y) ? 0x80 : 0x00;
    double a = fabs((double)y);
    if (a > 448.0) {
        a = 448.0;
    }
    if (a < ldexp(1.0, -6)) { /* below the smallest normal: units of 2^-9, and 8 units is that normal */
        return sign | (uint8_t)nearbyint(ldexp(a, 9));
    }
    int e = ilogb(a); /* 2^e <= a < 2^(e+1), e in [-6, 8] */
    double q = nearbyint(ldexp(a, 3 - e)); /* in [8, 16] */
    if (q == 16.0) {
        q = 8.0;
        ++e;
    }
    return sign | (uint8_t)(((e + 7) << 3) | ((int)q - 8));
}

void oracle_e4m3_values(double *out) {
    for (int c = 0; c < 256; ++c) {
        out[c] = e4m3_value((uint8_t)c);
    }
}

/* dst[i] = quantised src[i] (src float32 or bf16 bits) for i < n. */
int oracle_quantize_e4m3(uint8_t *dst, const void *src, int src_dtype, int64_t n, float scale) {
    if (src_dtype != ORACLE_F32 && src_dtype != ORACLE_BF16) {
        return -1;
    }
    for (int64_t i = 0; i < n; ++i) {
        dst[i] = e4m3_quantize((float)elem(src, i, src_dtype), scale);
    }
    return 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * One output row: head h of query row q_row attends over the first L logical positions of the sequence whose
 * block-table row is s. K/V are reassembled in logical order through the block table (page 1 section 3.2,
 * page 3 section 2.2), then out = sum_t w_t v_t / sum_t w_t with w_t = exp(z_t - max z), z_t = scale * q.k_t.
 */
static int attend_row(double *o, const void *query, int q_dtype, int64_t q_row, const void *key_cache,
                      const void *value_cache, int kv_dtype, double k_scale, double v_scale,
                      const int32_t *block_tables, int32_t s, int32_t h, int64_t L, double scale,
                      int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t max_blocks_per_seq) {
    const int32_t G = num_q_heads / num_kv_heads;
    const int32_t g = h / G;
    for (int32_t d = 0; d < head_dim; ++d) {
        o[d] = 0.0;
    }
    if (L <= 0) {
        return 0;
    }
    double *q = malloc(sizeof(double) * head_dim);
    double *k = malloc(sizeof(double) * L * head_dim);
    double *v = malloc(sizeof(double) * L * head_dim);
    double *z = malloc(sizeof(double) * L);
    if (!q || !k || !v || !z) {
        free(q); free(k); free(v); free(z);
        return -4;
    }
    const int64_t q_base = (q_row * num_q_heads + h) * head_dim;
    for (int32_t d = 0; d < head_dim; ++d) {
        q[d] = elem(query, q_base + d, q_dtype);
    }
    /* reassemble this head's K and V in logical order through the block table */
    for (int64_t t = 0; t < L; ++t) {
        const int64_t phys = block_tables[(int64_t)s * max_blocks_per_seq + t / block_size];
        const int64_t off = t % block_size;
        const int64_t base = ((phys * block_size + off) * num_kv_heads + g) * head_dim;
        for (int32_t d = 0; d < head_dim; ++d) {
            k[t * head_dim + d] = k_scale * elem(key_cache, base + d, kv_dtype);
            v[t * head_dim + d] = v_scale * elem(value_cache, base + d, kv_dtype);
        }
    }
    double m = -INFINITY;
    for (int64_t t = 0; t < L; ++t) {
        double acc = 0.0;
        for (int32_t d = 0; d < head_dim; ++d) {
            acc += q[d] * k[t * head_dim + d];
        }
        z[t] = scale * acc;
        if (z[t] > m) {
            m = z[t];
        }
    }
    double sum = 0.0;
    for (int64_t t = 0; t < L; ++t) {
        z[t] = exp(z[t] - m); /* z now holds the unnormalised weight w_t */
        sum += z[t];
    }
    for (int64_t t = 0; t < L; ++t) {
        for (int32_t d = 0; d < head_dim; ++d) {
            o[d] += z[t] * v[t * head_dim + d];
        }
    }
    for (int32_t d = 0; d < head_dim; ++d) {
        o[d] /= sum;
    }
    free(q); free(k); free(v); free(z);
    return 0;
}

static int check_tables(const int32_t *block_tables, const int32_t *context_lens, int32_t block_size,
                        int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                        int64_t num_blocks, int32_t max_blocks_per_seq) {
    if (block_size <= 0 || num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        num_q_heads % num_kv_heads != 0 || max_blocks_per_seq <= 0) {
        return -1;
    }
    for (int32_t s = 0; s < num_seqs; ++s) {
        int64_t L = context_lens[s];
        if (L < 0 || (L + block_size - 1) / block_size > max_blocks_per_seq) {
            return -2;
        }
        for (int64_t j = 0; j < (L + block_size - 1) / block_size; ++j) {
            int32_t b = block_tables[(int64_t)s * max_blocks_per_seq + j];
            if (b < 0 || b >= num_blocks) {
                return -3;
            }
        }
    }
    return 0;
}

/*
 * Decode attention for the (sequence, query head) rows listed in `rows` (pairs s, h; distinct, since rows are
 * computed in parallel, each into its own output row), or for every row when rows == NULL. out is [num_seqs, num_q_heads, head_dim] fp64; rows not listed are left untouched.
 *
 * Stored K and V elements are multiplied by k_scale and v_scale after decoding (1 for float32 / bf16 caches;
 * the dequantisation scales of an FP8 cache).
 *
 * For each row: G = num_q_heads / num_kv_heads query heads share KV head g = h / G (consecutive grouping);
 * position t of the sequence sits in physical block block_tables[s][t / block_size] at offset
 * t % block_size; z_t = scale * sum_d q[d] k_t[d] (d ascending); m = max z; w_t = exp(z_t - m);
 * out = sum_t w_t v_t / sum_t w_t. A context of length 0 gives a zero row.
 *
 * Returns 0, or -1 on a bad shape, -2 when a length exceeds the table width, -3 when a table entry that the
 * length makes live is not a valid block id, -4 when memory runs out.
 */
int oracle_decode(double *out, const void *query, int q_dtype, const void *key_cache, const void *value_cache,
                  int kv_dtype, double k_scale, double v_scale, const int32_t *block_tables,
                  const int32_t *context_lens, double scale,
                  int32_t block_size, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                  int32_t head_dim, int64_t num_blocks, int32_t max_blocks_per_seq, const int32_t *rows,
                  int64_t num_rows) {
    int status = check_tables(block_tables, context_lens, block_size, num_seqs, num_q_heads, num_kv_heads,
                              head_dim, num_blocks, max_blocks_per_seq);
    if (status != 0) {
        return status;
    }
    const int64_t total = rows ? num_rows : (int64_t)num_seqs * num_q_heads;

#pragma omp parallel for schedule(dynamic)
    for (int64_t r = 0; r < total; ++r) {
        int32_t s, h;
        if (rows) {
            s = rows[2 * r];
            h = rows[2 * r + 1];
        } else {
            s = (int32_t)(r / num_q_heads);
            h = (int32_t)(r % num_q_heads);
        }
        double *o = out + ((int64_t)s * num_q_heads + h) * head_dim;
        const int rc = attend_row(o, query, q_dtype, s, key_cache, value_cache, kv_dtype, k_scale, v_scale,
                                  block_tables, s, h, context_lens[s], scale, block_size, num_q_heads,
                                  num_kv_heads, head_dim, max_blocks_per_seq);
        if (rc != 0) {
#pragma omp atomic write
            status = rc;
        }
    }
    return status;
}

/*
 * Several new tokens per sequence (speculative verification, page 1 section 6; a chunk of a prompt). Sequence
 * s owns query rows query_start[s] .. query_start[s + 1] - 1, its QL = query_start[s + 1] - query_start[s]
 * newest tokens: token j sits at position L - QL + j of its L = context_lens[s] positions and attends over
 * positions 0 .. L - QL + j (causal: the cache already holds all L rows, the later ones are not attended).
 * A token with no position to attend (QL > L) gets a zero row. rows lists distinct (query row, head) pairs, or is NULL
 * for all; out is [num_tokens, num_q_heads, head_dim] fp64. Returns what oracle_decode returns, or -5 when
 * query_start is not a non-decreasing run from 0 to num_tokens.
 */
int oracle_decode_multi(double *out, const void *query, int q_dtype, const void *key_cache,
                        const void *value_cache, int kv_dtype, double k_scale, double v_scale,
                        const int32_t *block_tables, const int32_t *context_lens, const int32_t *query_start,
                        double scale, int32_t block_size, int32_t num_seqs, int32_t num_tokens,
                        int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                        int32_t max_blocks_per_seq, const int32_t *rows, int64_t num_rows) {
    int status = check_tables(block_tables, context_lens, block_size, num_seqs, num_q_heads, num_kv_heads,
                              head_dim, num_blocks, max_blocks_per_seq);
    if (status != 0) {
        return status;
    }
    if (num_tokens < 0 || query_start[0] != 0 || query_start[num_seqs] != num_tokens) {
        return -5;
    }
    int32_t *seq_of = malloc(sizeof(int32_t) * (num_tokens > 0 ? num_tokens : 1));
    if (!seq_of) {
        return -4;
    }
    for (int32_t s = 0; s < num_seqs; ++s) {
        if (query_start[s + 1] < query_start[s]) {
            free(seq_of);
            return -5;
        }
        for (int32_t t = query_start[s]; t < query_start[s + 1]; ++t) {
            seq_of[t] = s;
        }
    }
    const int64_t total = rows ? num_rows : (int64_t)num_tokens * num_q_heads;

#pragma omp parallel for schedule(dynamic)
    for (int64_t r = 0; r < total; ++r) {
        int32_t t, h;
        if (rows) {
            t = rows[2 * r];
            h = rows[2 * r + 1];
        } else {
            t = (int32_t)(r / num_q_heads);
            h = (int32_t)(r % num_q_heads);
        }
        const int32_t s = seq_of[t];
        const int64_t QL = query_start[s + 1] - query_start[s];
        const int64_t j = t - query_start[s];
        const int64_t E = (int64_t)context_lens[s] - QL + j + 1; /* positions this token attends over */
        double *o = out + ((int64_t)t * num_q_heads + h) * head_dim;
        const int rc = attend_row(o, query, q_dtype, t, key_cache, value_cache, kv_dtype, k_scale, v_scale,
                                  block_tables, s, h, E, scale, block_size, num_q_heads, num_kv_heads, head_dim,
                                  max_blocks_per_seq);
        if (rc != 0) {
#pragma omp atomic write
            status = rc;
        }
    }
    free(seq_of);
    return status;
}

/*
 * The new token's K/V goes into its slot: for token n with slot = slot_mapping[n] >= 0, physical block
 * slot / block_size, offset slot % block_size receives key[n] (all KV heads, all dims), likewise value.
 * Slots < 0 are skipped. Bytes are copied unchanged. Returns 0, or -1 when a slot is beyond the pool.
 */
int oracle_reshape_and_cache(void *key_cache, void *value_cache, const void *key, const void *value,
                             const int32_t *slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int64_t num_blocks, int32_t elem_bytes) {
    const int64_t row = (int64_t)num_kv_heads * head_dim * elem_bytes;
    for (int32_t n = 0; n < num_tokens; ++n) {
        const int64_t slot = slot_mapping[n];
        if (slot < 0) {
            continue;
        }
        if (slot >= num_blocks * block_size) {
            return -1;
        }
        const int64_t block = slot / block_size;
        const int64_t off = slot % block_size;
        const int64_t dst = (block * block_size + off) * row;
        memcpy((char *)key_cache + dst, (const char *)key + n * row, (size_t)row);
        memcpy((char *)value_cache + dst, (const char *)value + n * row, (size_t)row);
    }
    return 0;
}

/*
 * Copy-on-write of shared blocks: for each pair (src, dst), the whole dst block of both pools becomes a byte
 * copy of the src block. Pairs are applied in order. Returns 0, or -1 on an id outside the pool.
 */
/*
 * Block swap between two pools of the same block shape, e.g. the device pool and a host pool (page 1 section 5:
 * swap space on the host; page 2 section 7.2: inactive blocks moved to host memory): for each (src, dst) pair,
 * block dst of the destination pools becomes a copy of block src of the source pools, for K and for V.
 * Returns -1 when a pair names a block outside its pool.
 */
int oracle_swap_blocks(void *dst_key, void *dst_value, int64_t dst_num_blocks, const void *src_key,
                       const void *src_value, int64_t src_num_blocks, const int32_t *pairs, int32_t num_pairs,
                       int64_t block_bytes) {
    for (int32_t p = 0; p < num_pairs; ++p) {
        const int64_t src = pairs[2 * p], dst = pairs[2 * p + 1];
        if (src < 0 || src >= src_num_blocks || dst < 0 || dst >= dst_num_blocks) {
            return -1;
        }
        memcpy((char *)dst_key + dst * block_bytes, (const char *)src_key + src * block_bytes, (size_t)block_bytes);
        memcpy((char *)dst_value + dst * block_bytes, (const char *)src_value + src * block_bytes,
               (size_t)block_bytes);
    }
    return 0;
}

int oracle_copy_blocks(void *key_cache, void *value_cache, const int32_t *pairs, int32_t num_pairs,
                       int64_t block_bytes, int64_t num_blocks) {
    for (int32_t p = 0; p < num_pairs; ++p) {
        const int64_t src = pairs[2 * p], dst = pairs[2 * p + 1];
        if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) {
            return -1;
        }
        memmove((char *)key_cache + dst * block_bytes, (const char *)key_cache + src * block_bytes,
                (size_t)block_bytes);
        memmove((char *)value_cache + dst * block_bytes, (const char *)value_cache + src * block_bytes,
                (size_t)block_bytes);
    }
    return 0;
}

/*
 * Logical-order gather of one pool: out[(sum of earlier lengths) + t] = cache row of position t of each
 * sequence, all KV heads, raw bytes. out has sum(context_lens) rows of num_kv_heads*head_dim*elem_bytes.
 * Returns 0, or -3 on a live table entry outside the pool.
 */
int oracle_gather(void *out, const void *cache, const int32_t *block_tables, const int32_t *context_lens,
                  int32_t num_seqs, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                  int64_t num_blocks, int32_t max_blocks_per_seq, int32_t elem_bytes) {
    const int64_t row = (int64_t)num_kv_heads * head_dim * elem_bytes;
    int64_t r = 0;
    for (int32_t s = 0; s < num_seqs; ++s) {
        for (int64_t t = 0; t < context_lens[s]; ++t) {
            const int64_t phys = block_tables[(int64_t)s * max_blocks_per_seq + t / block_size];
            if (phys < 0 || phys >= num_blocks) {
                return -3;
            }
            memcpy((char *)out + r * row, (const char *)cache + (phys * block_size + t % block_size) * row,
                   (size_t)row);
            ++r;
        }
    }
    return 0;
}

/*
 * The FP8 cache write: the new token's K/V rows (float32 or bf16) are quantised (e4m3_quantize with k_scale,
 * v_scale) into slot slot_mapping[n] of the E4M3 pools. Slots < 0 are skipped; -1 for a slot past the pool.
 */
int oracle_reshape_and_cache_e4m3(uint8_t *key_cache, uint8_t *value_cache, const void *key, const void *value,
                                  int src_dtype, const int32_t *slot_mapping, int32_t num_tokens,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                  float k_scale, float v_scale) {
    const int64_t row = (int64_t)num_kv_heads * head_dim;
    for (int32_t n = 0; n < num_tokens; ++n) {
        const int64_t slot = slot_mapping[n];
        if (slot < 0) {
            continue;
        }
        if (slot >= num_blocks * block_size) {
            return -1;
        }
        for (int64_t i = 0; i < row; ++i) {
            key_cache[slot * row + i] = e4m3_quantize((float)elem(key, n * row + i, src_dtype), k_scale);
            value_cache[slot * row + i] = e4m3_quantize((float)elem(value, n * row + i, src_dtype), v_scale);
        }
    }
    return 0;
}
