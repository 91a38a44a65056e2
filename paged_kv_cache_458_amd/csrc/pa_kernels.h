// Internal interface between the C ABI (pa_abi.hip) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

struct DecodeArgs {
  float* out;                  // [B][Hq][D]
  const void* query;           // [B][Hq][D]
  const void* key_cache;       // [NB][bs][Hkv][D]
  const void* value_cache;     // [NB][bs][Hkv][D]
  const int32_t* block_tables; // [B][MB]
  const int32_t* context_lens; // [B]
  float* ws_o;                 // [B][Hq][PM][D]  normalised partial outputs      (split only)
  float* ws_ml;                // [B][Hq][PM][2]  (running max in log2 units, sum) (split only)
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
};

// Workspace layout for a split launch: partial outputs first, then the (max, sum) pairs.
inline size_t ws_o_elems(int64_t B, int64_t Hq, int64_t PM, int64_t D) { return B * Hq * PM * D; }
inline size_t ws_ml_elems(int64_t B, int64_t Hq, int64_t PM) { return B * Hq * PM * 2; }

hipError_t launch_decode_valu(const DecodeArgs& a, int kv_dtype, hipStream_t stream);
hipError_t launch_decode_gqa_mfma(const DecodeArgs& a, int kv_dtype, hipStream_t stream);
bool gqa_mfma_supported(int kv_dtype, int head_dim, int group);
constexpr int kGqaTileTokens = 32;  // tokens per tile of the GQA kernel
hipError_t launch_lse_reduce(const DecodeArgs& a, hipStream_t stream);

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* key_cache, void* value_cache,
                                    const int32_t* slot_mapping, int32_t num_tokens, int64_t row_bytes,
                                    int32_t block_size, int64_t num_blocks, hipStream_t stream);
hipError_t launch_reshape_and_cache_fp8(const void* key, const void* value, void* key_cache, void* value_cache,
                                        const int32_t* slot_mapping, int32_t num_tokens, int64_t row_elems,
                                        int32_t block_size, int64_t num_blocks, int src_dtype, float k_scale,
                                        float v_scale, hipStream_t stream);
hipError_t launch_copy_blocks(void* key_cache, void* value_cache, const int32_t* pairs, int32_t num_pairs,
                              int64_t block_bytes, int64_t num_blocks, hipStream_t stream);
hipError_t launch_paged_gather(void* out_key, void* out_value, const void* key_cache, const void* value_cache,
                               const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                               int32_t bs_log2, int64_t num_blocks, int32_t max_blocks_per_seq,
                               int32_t max_context_len, int64_t row_bytes, hipStream_t stream);

}  // namespace pa
