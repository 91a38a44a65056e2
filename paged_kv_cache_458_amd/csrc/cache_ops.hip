// Bandwidth kernels around the attention: the slot-mapped write of each step's new K/V, the copy-on-write
// block copy, and the logical-order gather used to check block-table indexing byte for byte.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

constexpr int kThreads = 256;

// One workgroup per new token (vLLM PagedAttention, page 3 section 2.1: after sampling, the token's K/V is
// appended). The slot indexes the flattened [num_blocks * block_size] rows of the pool, i.e. block
// slot / block_size at offset slot % block_size. Padding slots (< 0) and slots past the pool are skipped.
__global__ __launch_bounds__(kThreads) void reshape_and_cache_kernel(const U4* __restrict__ key,
                                                                     const U4* __restrict__ value,
                                                                     U4* __restrict__ key_cache,
                                                                     U4* __restrict__ value_cache,
                                                                     const int32_t* __restrict__ slot_mapping,
                                                                     int64_t row_u4, int64_t num_slots) {
  const int64_t n = blockIdx.x;
  const int32_t slot = slot_mapping[n];
  if (slot < 0 || slot >= num_slots) return;
  const U4* ks = key + n * row_u4;
  const U4* vs = value + n * row_u4;
  U4* kd = key_cache + (int64_t)slot * row_u4;
  U4* vd = value_cache + (int64_t)slot * row_u4;
  for (int64_t i = threadIdx.x; i < row_u4; i += kThreads) {
    kd[i] = ks[i];
    vd[i] = vs[i];
  }
}

// Copy-on-write (page 1 section 3.2): workgroup (pair, chunk) copies one chunk of block src to block dst in
// both pools. Pairs naming a block outside the pool are skipped.
constexpr int kCopyU4PerThread = 4;
__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(U4* __restrict__ key_cache,
                                                               U4* __restrict__ value_cache,
                                                               const int32_t* __restrict__ pairs,
                                                               int64_t block_u4, int64_t num_blocks) {
  const int32_t src = pairs[2 * blockIdx.x];
  const int32_t dst = pairs[2 * blockIdx.x + 1];
  if ((uint32_t)src >= (uint64_t)num_blocks || (uint32_t)dst >= (uint64_t)num_blocks) return;
  const int64_t chunk0 = (int64_t)blockIdx.y * kThreads * kCopyU4PerThread;
  const int64_t sbase = (int64_t)src * block_u4, dbase = (int64_t)dst * block_u4;
  U4 kv[kCopyU4PerThread], vv[kCopyU4PerThread];
#pragma unroll
  for (int j = 0; j < kCopyU4PerThread; ++j) {
    const int64_t i = chunk0 + j * kThreads + threadIdx.x;
    if (i < block_u4) {
      kv[j] = key_cache[sbase + i];
      vv[j] = value_cache[sbase + i];
    }
  }
#pragma unroll
  for (int j = 0; j < kCopyU4PerThread; ++j) {
    const int64_t i = chunk0 + j * kThreads + threadIdx.x;
    if (i < block_u4) {
      key_cache[dbase + i] = kv[j];
      value_cache[dbase + i] = vv[j];
    }
  }
}

// Logical-order gather: workgroup (tile, sequence) copies the rows of positions tile*16 .. tile*16+15 that
// are below the length, locating them with the same tile_slot_bytes() the attention kernels use.
__global__ __launch_bounds__(kThreads) void paged_gather_kernel(char* __restrict__ out_key,
                                                                char* __restrict__ out_value,
                                                                const char* __restrict__ key_cache,
                                                                const char* __restrict__ value_cache,
                                                                const int32_t* __restrict__ block_tables,
                                                                const int32_t* __restrict__ context_lens,
                                                                int32_t bs_log2, int64_t num_blocks,
                                                                int32_t max_blocks_per_seq, int32_t max_context_len,
                                                                int64_t row_bytes) {
  const int s = blockIdx.y;
  const int t = blockIdx.x * kTile;
  const int L = min(max(context_lens[s], 0), max_context_len);
  if (t >= L) return;
  bool bad = false;
  const int64_t base = tile_slot_bytes(block_tables + (int64_t)s * max_blocks_per_seq, t, bs_log2, num_blocks,
                                       row_bytes, bad);
  if (bad) return;
  const int rows = min(kTile, L - t);
  const int64_t row_u4 = row_bytes / 16;
  const int64_t obase = ((int64_t)s * max_context_len + t) * row_bytes;
  for (int64_t i = threadIdx.x; i < rows * row_u4; i += kThreads) {
    const int64_t off = i * 16;
    *reinterpret_cast<U4*>(out_key + obase + off) = *reinterpret_cast<const U4*>(key_cache + base + off);
    *reinterpret_cast<U4*>(out_value + obase + off) = *reinterpret_cast<const U4*>(value_cache + base + off);
  }
}

}  // namespace

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* key_cache, void* value_cache,
                                    const int32_t* slot_mapping, int32_t num_tokens, int64_t row_bytes,
                                    int32_t block_size, int64_t num_blocks, hipStream_t stream) {
  reshape_and_cache_kernel<<<dim3(num_tokens), dim3(kThreads), 0, stream>>>(
      static_cast<const U4*>(key), static_cast<const U4*>(value), static_cast<U4*>(key_cache),
      static_cast<U4*>(value_cache), slot_mapping, row_bytes / 16, num_blocks * block_size);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* key_cache, void* value_cache, const int32_t* pairs, int32_t num_pairs,
                              int64_t block_bytes, int64_t num_blocks, hipStream_t stream) {
  const int64_t block_u4 = block_bytes / 16;
  const int64_t per_wg = (int64_t)kThreads * kCopyU4PerThread;
  const dim3 grid(num_pairs, (unsigned)((block_u4 + per_wg - 1) / per_wg));
  copy_blocks_kernel<<<grid, dim3(kThreads), 0, stream>>>(static_cast<U4*>(key_cache), static_cast<U4*>(value_cache),
                                                          pairs, block_u4, num_blocks);
  return hipGetLastError();
}

hipError_t launch_paged_gather(void* out_key, void* out_value, const void* key_cache, const void* value_cache,
                               const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                               int32_t bs_log2, int64_t num_blocks, int32_t max_blocks_per_seq,
                               int32_t max_context_len, int64_t row_bytes, hipStream_t stream) {
  const dim3 grid((max_context_len + kTile - 1) / kTile, num_seqs);
  paged_gather_kernel<<<grid, dim3(kThreads), 0, stream>>>(
      static_cast<char*>(out_key), static_cast<char*>(out_value), static_cast<const char*>(key_cache),
      static_cast<const char*>(value_cache), block_tables, context_lens, bs_log2, num_blocks, max_blocks_per_seq,
      max_context_len, row_bytes);
  return hipGetLastError();
}

}  // namespace pa
