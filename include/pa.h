/*
 * pa.h -- C ABI of libpagedattn.so, the MI355X (gfx950) paged decode attention library.
 *
 * The paged KV cache (vLLM PagedAttention, page 1 "LLM inference framework evaluation ...", section 3.2):
 * keys and values live in two global block pools, each laid out as
 *     [num_blocks][block_size][num_kv_heads][head_dim]        (row-major, contiguous)
 * and each sequence owns a row of a block table that maps its logical block j (positions j*block_size ..
 * (j+1)*block_size-1) to a physical block id (page 3, section 2.2: logical block 0 may sit in physical block
 * 7). A sequence of length L uses its first ceil(L / block_size) table entries (page 2, section 4.2).
 *
 * Conventions for every call below:
 *  - Tensor arguments are DEVICE pointers into caller-owned memory (for instance PyTorch allocations),
 *    row-major and contiguous. The library allocates no device memory, keeps no per-call state and is
 *    reentrant; split-context scratch comes only from the caller's workspace.
 *  - dtype codes: PA_F32 (IEEE fp32), PA_BF16 (bfloat16) and, for caches, PA_FP8_E4M3. Attention
 *    output is always fp32.
 *  - `stream` is a hipStream_t (NULL = the null stream). Work is enqueued on it and the call returns
 *    without synchronising; results are valid once the caller synchronises that stream.
 *  - Every argument the host can check is checked before anything is launched; on failure the call
 *    returns a negative status and launches nothing. A launch failure returns PA_ERR_HIP.
 *  - Device-side contents (table entries, lengths, slots, copy pairs) are caller contracts, not checked on
 *    the host. The kernels still never touch memory outside the pools for them: a table entry outside
 *    [0, num_blocks) turns that (sequence, head) output row into NaN, a length is clamped to
 *    max_context_len, and out-of-range slots or copy pairs are skipped.
 *  - Pointers must be 16-byte aligned (PA_ERR_ALIGN otherwise).
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 2

/* dtype codes */
#define PA_F32 0
#define PA_BF16 1
#define PA_FP8_E4M3 2 /* OCP 8-bit float E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; max 448) */

/* status codes */
#define PA_OK 0
#define PA_ERR_NULL (-1)        /* a required pointer is NULL */
#define PA_ERR_SHAPE (-2)       /* a size is negative or zero where it must be positive, or sizes disagree */
#define PA_ERR_DTYPE (-3)       /* unknown dtype code or unsupported (query, cache) dtype pair */
#define PA_ERR_UNSUPPORTED (-4) /* head_dim, block_size or grid size outside what the kernels implement */
#define PA_ERR_WORKSPACE (-5)   /* the split-context path needs a larger workspace */
#define PA_ERR_HIP (-6)         /* a HIP launch or runtime call failed */
#define PA_ERR_ALIGN (-7)       /* a pointer is not 16-byte aligned */
#define PA_ERR_POINTER (-10)    /* swap_blocks: a pool or the pairs are not memory this device can access */
#define PA_ERR_SCRATCH (-11)    /* paged_attention_decode_noalloc: more scratch than PA_STATIC_SCRATCH_BYTES */

/* bytes of the static device scratch of paged_attention_decode_noalloc (one copy per GPU, 32 MiB) */
#define PA_STATIC_SCRATCH_BYTES ((size_t)32 << 20)

/* partition_size value that asks for the balanced split (see paged_attention_decode) */
#define PA_PARTITION_BALANCED 1

/* PA_ABI_VERSION of the loaded library. */
int pa_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char *pa_strerror(int status);

/*
 * Partition size (in tokens) that paged_attention_decode uses for a given `partition_size` argument (arguments
 * in the order of paged_attention_workspace_bytes: max_context_len, then block_size):
 * 0 stays 0 (single pass), a positive value is returned unchanged, -1 is replaced by the library's choice
 * for these sizes (PA_PARTITION_BALANCED when that is the balanced split). Returns a negative status for an
 * invalid request.
 */
int32_t paged_attention_partition_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t max_context_len, int32_t block_size,
                                       int32_t kv_dtype, int32_t partition_size);

/*
 * Bytes of workspace paged_attention_decode needs for these sizes (0 when the call runs single pass).
 * Arguments mean what they mean in paged_attention_decode; note the order here: max_context_len, then
 * block_size. Returns 0 as well for invalid sizes (the decode call reports them).
 * Split into partitions of P tokens: partials [num_seqs][num_q_heads][ceil(max_context_len / S)][head_dim]
 * fp32, then their (max, sum) pairs, each part 256-byte aligned, where S = P, or S = 2P when grouped heads run
 * on the matrix cores at head_dim <= 128 with 512 <= P < 1024 (one wave covers two partitions and merges them
 * itself).
 * Balanced split: partials [num_q_heads][R][2][head_dim] fp32 and their pairs, then (query rows + 1) int32
 * tile counts, for R runs. On the single-head kernel R = 1024 / ceil(ceil(num_q_heads / H) / 2) per head,
 * where a wave takes H = 2 adjacent heads if head rows are 64 or 128 bytes (E4M3 at head_dim 64 or 128, bf16
 * at 64) or bf16 rows of 256 bytes (head_dim 128), and num_q_heads == num_kv_heads, else H = 1. On the matrix-core kernel (grouped heads)
 * R = 2048 / (num_kv_heads rounded up to whole workgroups of W = min(8, largest power of two <= num_kv_heads)
 * KV heads). R is at least 1 either way.
 */
size_t paged_attention_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t max_context_len, int32_t block_size,
                                       int32_t kv_dtype, int32_t partition_size);

/*
 * Decode attention over the paged cache: for every sequence s and query head h,
 *     out[s][h][:] = softmax_t( scale * query[s][h][:] . K_t ) . V_t ,  t = 0 .. L-1,  L = context_lens[s],
 * where K_t / V_t are row (block_tables[s][t / block_size], t % block_size, h / G) of the pools and
 * G = num_q_heads / num_kv_heads query heads share one KV head (consecutive grouping). Each new token reads
 * every earlier K/V of its sequence (page 1 section 3.1); paging changes only where those rows live. A
 * length-0 context gives a zero row.
 *
 *   out            [num_seqs][num_q_heads][head_dim] fp32, written; must not alias any input
 *   query          [num_seqs][num_q_heads][head_dim] q_dtype
 *   key_cache      [num_blocks][block_size][num_kv_heads][head_dim] kv_dtype; at most 2^32 slots
 *                  (num_blocks * block_size), else PA_ERR_UNSUPPORTED (paged_gather alike)
 *   value_cache    same layout as key_cache
 *   block_tables   int32 [num_seqs][max_blocks_per_seq]; only entries j < ceil(L / block_size) are read
 *   context_lens   int32 [num_seqs]; 0 <= L <= max_context_len (longer lengths are clamped)
 *   scale          multiplies q . k before the softmax (1/sqrt(head_dim) in the usual models)
 *   block_size     tokens per block: 8, 16, 32, 64, 128 or 256 (page 1 section 5 suggests 8 for short
 *                  sequences; 8 needs head rows of at least 128 bytes, so not E4M3 at head_dim 64)
 *   head_dim       64, 80, 96, 112, 128, 192 or 256 (grouped heads with bf16 or E4M3 caches run on the matrix
 *                  cores at every head dim; one query head per KV head and fp32 caches on the vector ALUs)
 *   num_q_heads    a multiple of num_kv_heads
 *   max_context_len  upper bound of context_lens, <= max_blocks_per_seq * block_size
 *   (q_dtype, kv_dtype)  (PA_F32, PA_F32) or (PA_BF16, PA_BF16); accumulation is fp32 either way (FP8
 *                  caches: paged_attention_decode_scaled)
 *   partition_size 0 = one pass over each context; > 0 = split each context into partitions of this many
 *                  tokens (a multiple of 16) and merge the partial softmax states with a log-sum-exp
 *                  reduction; PA_PARTITION_BALANCED = the balanced split: the K/V tiles of all sequences,
 *                  in sequence order, are cut into equal runs, one per wave of a grid that fills the chip, so
 *                  every wave streams the same number of bytes; a sequence cut by run boundaries is merged
 *                  by the same log-sum-exp reduction (at most 2048 query rows and rows x max_context_len <=
 *                  2^30; grouped heads that run on the matrix cores -- bf16 or E4M3 caches -- also need
 *                  G <= 16 heads per KV head; PA_ERR_UNSUPPORTED otherwise); -1 = the library chooses
 *                  (paged_attention_partition_size): the balanced split wherever the single-head kernel would
 *                  otherwise split its contexts, and on the matrix cores wherever its partitions would launch
 *                  more than one round of 2048 resident waves; partitions otherwise
 *   workspace      device scratch of at least paged_attention_workspace_bytes(...) bytes when that is
 *                  non-zero (may be NULL otherwise); contents need no initialisation and are clobbered
 *   stream         hipStream_t
 * num_seqs == 0 is a no-op returning PA_OK.
 */
int paged_attention_decode(float *out, const void *query, const void *key_cache, const void *value_cache,
                           const int32_t *block_tables, const int32_t *context_lens, float scale,
                           int32_t block_size, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int64_t num_blocks, int32_t max_blocks_per_seq,
                           int32_t max_context_len, int32_t q_dtype, int32_t kv_dtype, int32_t partition_size,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * paged_attention_decode over caches whose stored elements are multiplied by a per-pool scale:
 *     K_t = k_scale * key_cache row,  V_t = v_scale * value_cache row,
 * the dequantisation of an FP8 KV cache (a quantised cache halves the bytes of a bandwidth-bound path;
 * page 1 section 4.1 and page 3 section 2.3 name FP8 among the quantised formats). Arguments as in
 * paged_attention_decode, plus k_scale and v_scale (finite, non-zero); the (q_dtype, kv_dtype) pairs are
 * (PA_F32, PA_F32), (PA_BF16, PA_BF16) and (PA_BF16, PA_FP8_E4M3). Every E4M3 code is exactly a bf16 value, so
 * the arithmetic after the load is that of the bf16 cache: k_scale folds into `scale` and v_scale into the
 * output. paged_attention_decode(...) is this call with k_scale = v_scale = 1.
 */
int paged_attention_decode_scaled(float *out, const void *query, const void *key_cache, const void *value_cache,
                                  const int32_t *block_tables, const int32_t *context_lens, float scale,
                                  float k_scale, float v_scale, int32_t block_size, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                                  int32_t max_blocks_per_seq, int32_t max_context_len, int32_t q_dtype,
                                  int32_t kv_dtype, int32_t partition_size, void *workspace,
                                  size_t workspace_bytes, void *stream);

/*
 * One decode step's cache write and attention in one call: the slot-mapped write of the new rows --
 * reshape_and_cache(key, value, key_cache, value_cache, slot_mapping, num_seqs, ...) for an fp32 or bf16 cache,
 * reshape_and_cache_fp8(..., src_dtype = q_dtype, k_scale, v_scale, ...) for an E4M3 cache -- followed by
 * paged_attention_decode_scaled(...) over the updated pools. Each new token is appended where it is produced
 * and attends at once (page 3 section 2.1: every decode step updates the KV cache; page 1 section 3.1: the new
 * token attends over every earlier K/V of its sequence, itself included).
 *
 *   key, value     [num_seqs][num_kv_heads][head_dim]: sequence s's new token, in kv_dtype for an fp32 or bf16
 *                  cache (written unchanged), in q_dtype for an E4M3 cache (quantised with k_scale / v_scale as
 *                  reshape_and_cache_fp8 does); written into slot slot_mapping[s] of both pools (updated in place;
 *                  slots < 0 or >= num_blocks * block_size are skipped, as in the cache writes)
 *   other arguments as in paged_attention_decode_scaled
 * Contract: for every s whose slot is written, position context_lens[s] - 1 of sequence s lies in that slot
 * through the block table (the new token is the last position of the sequence) and context_lens[s] >= 1. As in
 * paged_attention_decode, lengths beyond max_context_len are clamped: such a sequence's new token is written but
 * not attended over. The decode launch does both, whatever the plan: the last position of such a sequence is
 * taken from `key` / `value` (quantised first for E4M3) instead of the pool, and a wave of that sequence writes
 * it into the pools. Only a call with max_context_len 0 (no position attended anywhere), or an E4M3 call with
 * |k_scale| or |v_scale| outside [2^-32, 2^32] (where the decode kernels' quantiser would need a division per
 * value), launches the cache write first. Either way the pools end as the cache write leaves them, byte for byte. The output equals that of the
 * two calls bit for bit on the matrix-core kernels (grouped heads over bf16 or E4M3 caches); the single-head
 * kernels add the new token to its row's softmax after the pool rows of its tile or partition (the same values,
 * another order of floating-point additions).
 */
int paged_attention_decode_append(float *out, const void *query, const void *key, const void *value, void *key_cache,
                                  void *value_cache, const int32_t *block_tables, const int32_t *context_lens,
                                  const int32_t *slot_mapping, float scale, float k_scale, float v_scale,
                                  int32_t block_size, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int64_t num_blocks, int32_t max_blocks_per_seq,
                                  int32_t max_context_len, int32_t q_dtype, int32_t kv_dtype, int32_t partition_size,
                                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * paged_attention_decode_scaled for callers that cannot allocate device memory or pass a workspace: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. Same arguments, plan, kernels and
 * results as paged_attention_decode_scaled (bit for bit), without the workspace arguments: the split-context
 * partials go to a static device buffer of PA_STATIC_SCRATCH_BYTES inside the library, one per GPU, allocated
 * when the library's device code is loaded and held until the process ends. The call allocates nothing.
 *
 * The buffer's device address is looked up once per GPU, on the first call with that GPU current. Calls whose
 * plan needs more than PA_STATIC_SCRATCH_BYTES (paged_attention_workspace_bytes for the same sizes) return
 * PA_ERR_SCRATCH and launch nothing. Every call on one GPU shares that GPU's buffer: two calls that may run at
 * the same time on one GPU (on different streams without ordering between them) race, and must be ordered by
 * the caller. No call needs the buffer cleared: each writes the partials it reads.
 */
int paged_attention_decode_noalloc(float *out, const void *query, const void *key_cache, const void *value_cache,
                                   const int32_t *block_tables, const int32_t *context_lens, float scale,
                                   float k_scale, float v_scale, int32_t block_size, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                                   int32_t max_blocks_per_seq, int32_t max_context_len, int32_t q_dtype,
                                   int32_t kv_dtype, int32_t partition_size, void *stream);

/*
 * Attention of several new tokens per sequence over the paged cache (speculative verification, which page 1
 * section 6 lists as future work combined with paging; a chunk of a prompt). Sequence s brings the query rows
 * query_start[s] .. query_start[s + 1] - 1, its QL newest tokens, whose K/V are already in the cache: its
 * L = context_lens[s] positions end with them. Row j of QL sits at position L - QL + j and attends causally,
 *     out[r][h][:] = softmax_t( scale * query[r][h][:] . K_t ) . V_t ,  t = 0 .. L - QL + j,  r = query_start[s] + j,
 * with K_t / V_t and the scales as in paged_attention_decode_scaled. A row with no position to attend
 * (QL > L) gives a zero row. QL = 1 for every sequence is paged_attention_decode_scaled.
 *
 *   out, query     [num_query_tokens][num_q_heads][head_dim] (fp32; q_dtype), rows packed by sequence
 *   query_start    int32 [num_seqs + 1] device array: query_start[0] = 0, non-decreasing, last entry
 *                  num_query_tokens, every difference <= max_query_len (rows beyond max_query_len are left
 *                  unwritten; the contents are not checked on the host)
 *   max_query_len  the largest QL (>= 1). With bf16 or E4M3 caches the matrix cores take all of a sequence's
 *                  rows whenever grouped heads x QL give at least 2 columns, reading its K/V once per 16
 *                  (row, grouped head) columns (at most 1024 columns); other calls read a sequence's K/V once
 *                  per (row, head).
 *   partition_size as in paged_attention_decode. On the matrix cores PA_PARTITION_BALANCED needs the grouped
 *                  heads x max_query_len columns to fit one group of 16 and at most 2048 sequences
 *                  (PA_ERR_UNSUPPORTED otherwise); its tile list holds sequences, each read once for all its
 *                  rows. The library's choice (-1) there is the balanced split also where a single pass would
 *                  fill a round of 2048 waves of unequal length (several rows per sequence only).
 *   workspace      at least paged_attention_multi_workspace_bytes(...) bytes when that is non-zero; for the
 *                  balanced split on the matrix cores, as paged_attention_workspace_bytes describes with
 *                  partials [num_q_heads][R][2][max_query_len][head_dim] and (num_seqs + 1) tile counts
 * Other arguments as in paged_attention_decode_scaled. num_seqs == 0 or num_query_tokens == 0 is a no-op;
 * num_query_tokens > num_seqs * max_query_len is PA_ERR_SHAPE.
 */
int paged_attention_decode_multi(float *out, const void *query, const void *key_cache, const void *value_cache,
                                 const int32_t *block_tables, const int32_t *context_lens,
                                 const int32_t *query_start, float scale, float k_scale, float v_scale,
                                 int32_t block_size, int32_t num_seqs, int32_t num_query_tokens,
                                 int32_t max_query_len, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int64_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                                 int32_t q_dtype, int32_t kv_dtype, int32_t partition_size, void *workspace,
                                 size_t workspace_bytes, void *stream);

/* Partition size and workspace bytes of paged_attention_decode_multi, as the decode forms above. */
int32_t paged_attention_multi_partition_size(int32_t num_seqs, int32_t num_query_tokens, int32_t max_query_len,
                                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                             int32_t max_context_len, int32_t block_size, int32_t kv_dtype,
                                             int32_t partition_size);
size_t paged_attention_multi_workspace_bytes(int32_t num_seqs, int32_t num_query_tokens, int32_t max_query_len,
                                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                             int32_t max_context_len, int32_t block_size, int32_t kv_dtype,
                                             int32_t partition_size);

/*
 * Quantising cache write into PA_FP8_E4M3 pools: like reshape_and_cache, with every element of key[n]
 * (value[n]) stored as the E4M3 code of x / k_scale (x / v_scale): an fp32 division, saturated to +-448,
 * rounded to nearest with ties to an even mantissa; NaN is stored as 0x7F.
 *
 *   key, value               [num_tokens][num_kv_heads][head_dim] src_dtype (PA_F32 or PA_BF16)
 *   key_cache, value_cache   [num_blocks][block_size][num_kv_heads][head_dim] E4M3 codes, updated in place
 *   k_scale, v_scale         finite, non-zero
 */
int reshape_and_cache_fp8(const void *key, const void *value, void *key_cache, void *value_cache,
                          const int32_t *slot_mapping, int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int64_t num_blocks, int32_t src_dtype, float k_scale, float v_scale,
                          void *stream);

/*
 * Append each new token's K/V to its cache slot (page 3 section 2.1: every decode step updates the KV cache
 * after sampling; page 1 section 3.2: a slot is a (physical block, offset) pair):
 *     key_cache[slot / block_size][slot % block_size][:][:] = key[n][:][:]   (likewise value)
 * for n < num_tokens with slot = slot_mapping[n]. Bytes are copied unchanged. Slots < 0 (padding) and slots
 * >= num_blocks * block_size are skipped. Slots must be distinct (otherwise the surviving write is not
 * specified).
 *
 *   key, value               [num_tokens][num_kv_heads][head_dim] kv_dtype
 *   key_cache, value_cache   [num_blocks][block_size][num_kv_heads][head_dim] kv_dtype, updated in place
 *   slot_mapping             int32 [num_tokens]
 * num_tokens == 0 is a no-op returning PA_OK.
 */
int reshape_and_cache(const void *key, const void *value, void *key_cache, void *value_cache,
                      const int32_t *slot_mapping, int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int64_t num_blocks, int32_t kv_dtype, void *stream);

/*
 * Copy-on-write of shared blocks (page 1 section 3.2: sequences share physical blocks until one of them
 * writes; then the block is copied): for each pair p, block block_pairs[p][1] (dst) of both pools becomes a
 * byte copy of block block_pairs[p][0] (src). Destinations must be distinct and no block may be both a
 * source and a destination (pairs are then independent and run concurrently). Pairs with an id outside
 * [0, num_blocks) are skipped.
 *
 *   key_cache, value_cache   pools as above, updated in place
 *   block_pairs              int32 [num_pairs][2] = {src, dst}, device memory
 * num_pairs == 0 is a no-op returning PA_OK.
 */
int copy_blocks(void *key_cache, void *value_cache, const int32_t *block_pairs, int32_t num_pairs,
                int32_t block_size, int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks, int32_t kv_dtype,
                void *stream);

/*
 * Block swap between two pools of the same block shape, typically the device pool and a pool in pinned host
 * memory (page 1 section 5 recommends swap space on the host; page 2 section 7.2 moving inactive blocks to host
 * memory). For every pair (src, dst) of block_pairs:
 *     dst_key_cache[dst][:][:][:] = src_key_cache[src][:][:][:]      (likewise V)
 * Either side may be memory of the current device or pinned host memory (hipHostMalloc, torch's pin_memory):
 * the kernel reads and writes it directly, so a swap runs at the rate of the host link. Every pointer is looked
 * up with hipPointerGetAttributes first; pageable host memory, managed memory or another GPU's memory gives
 * PA_ERR_POINTER and nothing is launched.
 *
 *   dst_*_cache    [dst_num_blocks][block_size][num_kv_heads][head_dim] kv_dtype, written
 *   src_*_cache    [src_num_blocks][block_size][num_kv_heads][head_dim] kv_dtype, read
 *   block_pairs    int32 [num_pairs][2] = (src block, dst block), device-accessible; pairs naming a block
 *                  outside its pool are skipped; destination blocks must be distinct, and the two sides must not
 *                  overlap in memory
 * Enqueued on stream like copy_blocks: the caller owns both pools and must not reuse a swapped-out device block
 * for new writes, or read a swapped-in one, before the stream reaches the copy. num_pairs == 0 is a no-op.
 */
int swap_blocks(void *dst_key_cache, void *dst_value_cache, int64_t dst_num_blocks, const void *src_key_cache,
                const void *src_value_cache, int64_t src_num_blocks, const int32_t *block_pairs, int32_t num_pairs,
                int32_t block_size, int32_t num_kv_heads, int32_t head_dim, int32_t kv_dtype, void *stream);

/*
 * Logical-order gather through the block table, with the same device address arithmetic that
 * paged_attention_decode uses (exported so that tests can check that indexing byte for byte):
 *     out_key[s][t][:][:] = key_cache[block_tables[s][t / block_size]][t % block_size][:][:]   (likewise V)
 * for t < min(context_lens[s], max_context_len). Rows t >= L of out_key/out_value are left untouched; a row
 * whose table entry is outside [0, num_blocks) is left untouched too.
 *
 *   out_key, out_value  [num_seqs][max_context_len][num_kv_heads][head_dim] kv_dtype
 *   other arguments as in paged_attention_decode
 */
int paged_gather(void *out_key, void *out_value, const void *key_cache, const void *value_cache,
                 const int32_t *block_tables, const int32_t *context_lens, int32_t block_size, int32_t num_seqs,
                 int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks, int32_t max_blocks_per_seq,
                 int32_t max_context_len, int32_t kv_dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
