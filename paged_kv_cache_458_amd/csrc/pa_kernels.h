// Internal interface between the C ABI (pa_abi.hip) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pa.h"

namespace pa {

struct DecodeArgs {
  float* out;                  // [T][Hq][D], T query rows (T = B: one new token per sequence)
  const void* query;           // [T][Hq][D]
  const void* key_cache;       // [NB][bs][Hkv][D]
  const void* value_cache;     // [NB][bs][Hkv][D]
  const int32_t* block_tables; // [B][MB]
  const int32_t* context_lens; // [B]
  const int32_t* query_start;  // [B + 1] first query row of each sequence, or null: row s is sequence s
  float* ws_o;                 // [T][Hq][PM][D]  normalised partial outputs      (split only)
  float* ws_ml;                // [T][Hq][PM][2]  (running max in log2 units, sum) (split only)
  float scale_log2;            // scale * k_scale * log2(e): scores live in the exp2 domain
  float v_scale;               // multiplies every output row (1 unless the cache is quantised)
  int32_t num_seqs, num_q_heads, num_kv_heads, head_dim, group;
  int32_t bs_log2;
  int64_t num_blocks;
  int32_t max_blocks_per_seq, max_context_len;
  int32_t partition;           // tokens per partition (split) or >= max_context_len rounded to 16 (single)
  int32_t max_partitions;      // PM
  int32_t parts_per_wave;      // consecutive partitions one wave covers (GQA kernel; the others take 1)
  int32_t split;               // 0: every sequence is one partition, written straight to out
  int32_t num_tokens;          // T
  int32_t max_query_len;       // query rows per sequence at most (1 without query_start)
  int32_t col_groups;          // matrix-core kernel: groups of 16 (query row, head) columns per KV head
  int32_t cg_per_wave;         // matrix-core partition kernel: column groups one wave serves (1, or 2 when
                               // head_dim <= 128)
  int32_t chunks;              // balanced split: runs of tiles per query head (0: partitions as above)
  int32_t* tile_prefix;        // balanced split: tiles of the rows before each row, [T + 1] (workspace) ...
  int32_t seq_prefix;          // ... or, when 1 (matrix-core kernel), of the sequences before each, [B + 1]
  // Decode with each sequence's new token appended in the same launch: the new K/V rows [B][Hkv][D] (in the
  // cache's dtype, or bf16 for an E4M3 cache, quantised with the scales below as the cache write does), their
  // slots [B], and the pools they are written to. Null otherwise.
  const void* new_key;
  const void* new_value;
  const int32_t* slot_mapping;
  void* key_out;
  void* value_out;
  float new_k_scale, new_v_scale;
};

// The sequence that owns query row t: the last s with query_start[s] <= t (empty sequences are skipped since the
// next start equals theirs). Called by a whole wave with one t: the entries <= t form a prefix of the
// non-decreasing query_start, so each lane compares one entry of a window and a ballot counts the prefix. A
// window of up to 64 entries takes one round of loads; a longer one is first narrowed by sampling it at a
// stride (64 sequences: one round of loads where a binary search takes six dependent ones; 4096: two).
__device__ __forceinline__ int seq_of_row(const DecodeArgs& a, int t) {
  if (!a.query_start) return t;
  const int lane = __lane_id();
  int lo = 0, n = a.num_seqs;  // the owner lies in [lo, lo + n)
  while (n > 64) {
    const int stride = (n + 63) / 64;
    const int idx = lo + lane * stride;
    const bool le = lane * stride < n && a.query_start[idx] <= t;
    // at least 1 (query_start[lo] <= t); kept so even for contents that break the contract
    const int k = max(__builtin_popcountll(__builtin_amdgcn_ballot_w64(le)), 1);
    lo += (k - 1) * stride;
    n = min(stride, n - (k - 1) * stride);
  }
  const bool le = lane < n && a.query_start[lo + lane] <= t;
  const int k = __builtin_popcountll(__builtin_amdgcn_ballot_w64(le));
  return lo + max(k, 1) - 1;
}

// Query rows of sequence s as every kernel takes them: query_start[s + 1] - query_start[s], clamped to
// [0, max_query_len] (a larger difference breaks the caller's contract; its rows past max_query_len are left
// unwritten by every kernel alike).
__device__ __forceinline__ int rows_of_seq(const DecodeArgs& a, int s) {
  return min(max(a.query_start[s + 1] - a.query_start[s], 0), a.max_query_len);
}

// Positions that query row t of sequence s (length L) attends over: all L for decode; for row j of the
// sequence's QL rows (rows_of_seq), its causal prefix of L - QL + j + 1 positions (none when that is not
// positive); -1 for a row that is not among the sequence's QL rows, which no kernel computes or writes.
__device__ __forceinline__ int row_extent(const DecodeArgs& a, int s, int t, int L) {
  if (!a.query_start) return L;
  const int ql = rows_of_seq(a, s);
  const int j = t - a.query_start[s];
  if (j >= ql) return -1;
  return max(0, min(L, L - ql + j + 1));
}

// Workspace layout for a split launch: partial outputs first, then the (max, sum) pairs.
inline size_t ws_o_elems(int64_t T, int64_t Hq, int64_t PM, int64_t D) { return T * Hq * PM * D; }
inline size_t ws_ml_elems(int64_t T, int64_t Hq, int64_t PM) { return T * Hq * PM * 2; }

hipError_t launch_decode_valu(const DecodeArgs& a, int kv_dtype, hipStream_t stream);
hipError_t launch_decode_gqa_mfma(const DecodeArgs& a, int kv_dtype, hipStream_t stream);
// The matrix-core kernel takes (sequence, KV head) pairs whose group x query rows fill at least 2 of its 16
// columns, in up to kMaxColGroups column groups (each reading the K/V once).
constexpr int kMaxColGroups = 64;
bool gqa_mfma_supported(int kv_dtype, int head_dim, int group, int max_query_len);
// Column groups one wave of the matrix-core partition kernel serves: 2 (two accumulators, every K/V load and LDS
// operand read shared) where there are several and head_dim <= 128, else 1; over a bf16 cache with three or four,
// all of them (one wave per SIMD, its accumulators in AGPRs, at most 4 waves to a workgroup). Measured on MI355X,
// 70B-shaped batch with 5, 6 and 8 new tokens per sequence (40, 48 and 64 columns): bf16 261 -> 210, 268 -> 219
// and 277.5 -> 233.0 us; the E4M3 form with 8 went 173 -> 212 us, and 16 tokens per sequence (8 groups, two such
// waves) 409 -> 437 us, so only those cases take it.
inline int gqa_cg_per_wave(int col_groups, int head_dim, int kv_dtype) {
  if (head_dim > 128) return 1;
  if ((col_groups == 3 || col_groups == 4) && kv_dtype == PA_BF16) return 4;
  return col_groups >= 2 ? 2 : 1;
}
constexpr int kGqaTileTokens = 32;  // tokens per tile of the GQA kernel
hipError_t launch_lse_reduce(const DecodeArgs& a, hipStream_t stream);
// Balanced split of the single-head kernel: the tiles of all query rows, in row order, cut into `chunks`
// equal runs per head, one wave each; the grid is sized to one wave per wave slot of the chip.
constexpr int kMaxBalancedRows = 2048;  // query rows whose tile counts one workgroup scans in LDS
constexpr int kResidentWaves = 2048;    // 256 CUs x 4 SIMDs x 2 waves of the single-head kernel
// Heads per wave of the single-head balanced split: 2 where two adjacent heads' rows fill one row group
// exactly (64- or 128-byte head rows, and 256-byte bf16 rows: measured on MI355X, the mixed-length batch 613.0 ->
// 605.3 us and the 7B-shaped one unchanged; one query head per KV head), else 1.
int valu_heads_per_wave(int kv_dtype, int head_dim, int group);
int32_t balanced_chunks(int32_t num_q_heads, int32_t heads_per_wave);  // runs per head: the grid fills kResidentWaves
hipError_t launch_decode_valu_balanced(const DecodeArgs& a, int kv_dtype, hipStream_t stream);
hipError_t launch_balanced_reduce(const DecodeArgs& a, hipStream_t stream);
// Balanced split of the matrix-core kernel (one column group): the 32-token tiles of all sequences cut into
// `chunks` equal runs, one workgroup of up to 8 KV heads each; its partials take the single-head balanced
// split's layout with a further index, the query row within its sequence (max_query_len of them), and
// launch_balanced_reduce merges them.
int32_t gqa_balanced_chunks(int32_t num_kv_heads);  // runs: the grid fills kResidentWaves
hipError_t launch_decode_gqa_mfma_balanced(const DecodeArgs& a, int kv_dtype, hipStream_t stream);
// workspace of a balanced launch: partials [Hq][chunks][2][QL][D] fp32, then (m, l) [Hq][chunks][2][QL][2];
// QL = 1 but on the matrix-core kernel, where it is the most query rows of a sequence
inline size_t balanced_o_elems(int64_t Hq, int64_t chunks, int64_t D, int64_t QL = 1) { return Hq * chunks * 2 * QL * D; }
inline size_t balanced_ml_elems(int64_t Hq, int64_t chunks, int64_t QL = 1) { return Hq * chunks * 2 * QL * 2; }

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* key_cache, void* value_cache,
                                    const int32_t* slot_mapping, int32_t num_tokens, int64_t row_bytes,
                                    int32_t block_size, int64_t num_blocks, hipStream_t stream);
hipError_t launch_reshape_and_cache_fp8(const void* key, const void* value, void* key_cache, void* value_cache,
                                        const int32_t* slot_mapping, int32_t num_tokens, int64_t row_elems,
                                        int32_t block_size, int64_t num_blocks, int src_dtype, float k_scale,
                                        float v_scale, hipStream_t stream);
hipError_t launch_copy_blocks(void* key_cache, void* value_cache, const int32_t* pairs, int32_t num_pairs,
                              int64_t block_bytes, int64_t num_blocks, hipStream_t stream);
hipError_t launch_swap_blocks(void* dst_key, void* dst_value, int64_t dst_num_blocks, const void* src_key,
                              const void* src_value, int64_t src_num_blocks, const int32_t* pairs, int32_t num_pairs,
                              int64_t block_bytes, hipStream_t stream);
hipError_t launch_paged_gather(void* out_key, void* out_value, const void* key_cache, const void* value_cache,
                               const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                               int32_t bs_log2, int64_t num_blocks, int32_t max_blocks_per_seq,
                               int32_t max_context_len, int64_t row_bytes, hipStream_t stream);

}  // namespace pa
