// Bandwidth kernels around the attention: the slot-mapped write of each step's new K/V, the copy-on-write
// block copy, and the logical-order gather used to check block-table indexing byte for byte.
#include "pa_device.h"
#include "pa_kernels.h"
#include "../../include/pa.h"

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

// 16 consecutive source elements (float32 or bf16) -> 16 E4M3 codes (e4m3_pack16 in pa_device.h).
template <int SRC>
__device__ __forceinline__ U4 e4m3_pack16_from(const char* src, const E4m3Div& dv) {
  if constexpr (SRC == PA_BF16) {
    return e4m3_pack16_bf16<true>(*reinterpret_cast<const U4*>(src), *reinterpret_cast<const U4*>(src + 16), dv);
  } else {
    float f[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const U4 v = reinterpret_cast<const U4*>(src)[i];
      f[4 * i] = __uint_as_float(v.x);
      f[4 * i + 1] = __uint_as_float(v.y);
      f[4 * i + 2] = __uint_as_float(v.z);
      f[4 * i + 3] = __uint_as_float(v.w);
    }
    return e4m3_pack16<true>(f, dv);
  }
}

// Quantising cache write: one workgroup per new token, one 16-element word per thread and step.
template <int SRC>
__global__ __launch_bounds__(kThreads) void reshape_and_cache_fp8_kernel(
    const char* __restrict__ key, const char* __restrict__ value, U4* __restrict__ key_cache,
    U4* __restrict__ value_cache, const int32_t* __restrict__ slot_mapping, int64_t row_elems, int64_t num_slots,
    float k_scale, float v_scale) {
  constexpr int kSrcEsize = SRC == PA_BF16 ? 2 : 4;
  const int64_t n = blockIdx.x;
  const int32_t slot = slot_mapping[n];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t words = row_elems / 16;
  const char* ks = key + n * row_elems * kSrcEsize;
  const char* vs = value + n * row_elems * kSrcEsize;
  U4* kd = key_cache + (int64_t)slot * words;
  U4* vd = value_cache + (int64_t)slot * words;
  const E4m3Div kdiv = e4m3_div(k_scale), vdiv = e4m3_div(v_scale);
  for (int64_t i = threadIdx.x; i < words; i += kThreads) {
    kd[i] = e4m3_pack16_from<SRC>(ks + i * 16 * kSrcEsize, kdiv);
    vd[i] = e4m3_pack16_from<SRC>(vs + i * 16 * kSrcEsize, vdiv);
  }
}

// Block copies (src, dst) from one pair of pools into another: copy-on-write inside the device pool (page 1
// section 3.2; both sides the same pools) and swaps between the device pool and a pool in pinned host memory
// (page 1 section 5, page 2 section 7.2), which the kernel reads or writes directly over the host link.
// Workgroup (pair, chunk) copies one chunk of block src to block dst in both the K and the V pools. Pairs naming
// a block outside its pool are skipped. No __restrict__: copy-on-write reads and writes one allocation.
constexpr int kCopyU4PerThread = 4;
__global__ __launch_bounds__(kThreads) void block_copy_kernel(U4* dst_key, U4* dst_value, int64_t dst_num_blocks,
                                                              const U4* src_key, const U4* src_value,
                                                              int64_t src_num_blocks,
                                                              const int32_t* __restrict__ pairs, int64_t block_u4) {
  const int32_t src = pairs[2 * blockIdx.x];
  const int32_t dst = pairs[2 * blockIdx.x + 1];
  if ((uint32_t)src >= (uint64_t)src_num_blocks || (uint32_t)dst >= (uint64_t)dst_num_blocks) return;
  const int64_t chunk0 = (int64_t)blockIdx.y * kThreads * kCopyU4PerThread;
  const int64_t sbase = (int64_t)src * block_u4, dbase = (int64_t)dst * block_u4;
  U4 kv[kCopyU4PerThread], vv[kCopyU4PerThread];
#pragma unroll
  for (int j = 0; j < kCopyU4PerThread; ++j) {
    const int64_t i = chunk0 + j * kThreads + threadIdx.x;
    if (i < block_u4) {
      kv[j] = src_key[sbase + i];
      vv[j] = src_value[sbase + i];
    }
  }
#pragma unroll
  for (int j = 0; j < kCopyU4PerThread; ++j) {
    const int64_t i = chunk0 + j * kThreads + threadIdx.x;
    if (i < block_u4) {
      dst_key[dbase + i] = kv[j];
      dst_value[dbase + i] = vv[j];
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
  // one workgroup per tile of min(16, block_size) positions: a tile never leaves its block
  const int tile = min(kTile, 1 << bs_log2);
  const int s = blockIdx.y;
  const int t = blockIdx.x * tile;
  const int L = min(max(context_lens[s], 0), max_context_len);
  if (t >= L) return;
  bool bad = false;
  const int64_t base = tile_slot_bytes(block_tables + (int64_t)s * max_blocks_per_seq, t, bs_log2, num_blocks,
                                       row_bytes, bad);
  if (bad) return;
  const int rows = min(tile, L - t);
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

hipError_t launch_reshape_and_cache_fp8(const void* key, const void* value, void* key_cache, void* value_cache,
                                        const int32_t* slot_mapping, int32_t num_tokens, int64_t row_elems,
                                        int32_t block_size, int64_t num_blocks, int src_dtype, float k_scale,
                                        float v_scale, hipStream_t stream) {
  const dim3 grid(num_tokens), block(kThreads);
  const char* k = static_cast<const char*>(key);
  const char* v = static_cast<const char*>(value);
  U4* kc = static_cast<U4*>(key_cache);
  U4* vc = static_cast<U4*>(value_cache);
  const int64_t slots = num_blocks * block_size;
  if (src_dtype == PA_BF16)
    reshape_and_cache_fp8_kernel<PA_BF16><<<grid, block, 0, stream>>>(k, v, kc, vc, slot_mapping, row_elems, slots,
                                                                      k_scale, v_scale);
  else
    reshape_and_cache_fp8_kernel<PA_F32><<<grid, block, 0, stream>>>(k, v, kc, vc, slot_mapping, row_elems, slots,
                                                                     k_scale, v_scale);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* key_cache, void* value_cache, const int32_t* pairs, int32_t num_pairs,
                              int64_t block_bytes, int64_t num_blocks, hipStream_t stream) {
  return launch_swap_blocks(key_cache, value_cache, num_blocks, key_cache, value_cache, num_blocks, pairs, num_pairs,
                            block_bytes, stream);
}

hipError_t launch_swap_blocks(void* dst_key, void* dst_value, int64_t dst_num_blocks, const void* src_key,
                              const void* src_value, int64_t src_num_blocks, const int32_t* pairs, int32_t num_pairs,
                              int64_t block_bytes, hipStream_t stream) {
  const int64_t block_u4 = block_bytes / 16;
  const int64_t per_wg = (int64_t)kThreads * kCopyU4PerThread;
  const dim3 grid(num_pairs, (unsigned)((block_u4 + per_wg - 1) / per_wg));
  block_copy_kernel<<<grid, dim3(kThreads), 0, stream>>>(
      static_cast<U4*>(dst_key), static_cast<U4*>(dst_value), dst_num_blocks, static_cast<const U4*>(src_key),
      static_cast<const U4*>(src_value), src_num_blocks, pairs, block_u4);
  return hipGetLastError();
}

hipError_t launch_paged_gather(void* out_key, void* out_value, const void* key_cache, const void* value_cache,
                               const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                               int32_t bs_log2, int64_t num_blocks, int32_t max_blocks_per_seq,
                               int32_t max_context_len, int64_t row_bytes, hipStream_t stream) {
  const int tile = min(kTile, 1 << bs_log2);
  const dim3 grid((max_context_len + tile - 1) / tile, num_seqs);
  paged_gather_kernel<<<grid, dim3(kThreads), 0, stream>>>(
      static_cast<char*>(out_key), static_cast<char*>(out_value), static_cast<const char*>(key_cache),
      static_cast<const char*>(value_cache), block_tables, context_lens, bs_log2, num_blocks, max_blocks_per_seq,
      max_context_len, row_bytes);
  return hipGetLastError();
}

}  // namespace pa
