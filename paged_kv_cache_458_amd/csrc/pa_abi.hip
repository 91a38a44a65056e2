// C ABI of libpagedattn.so: host-side argument checks, launch planning (single pass or split context,
// VALU or MFMA variant, workspace layout) and the launches themselves. Every check runs before any HIP call,
// so an invalid call returns its status without touching the device.
#include <limits.h>
#include <stdint.h>

#include <mutex>

#include "../../include/pa.h"
#include "pa_device.h"
#include "pa_kernels.h"

namespace {

constexpr int kTileTokens = 16;
// the readers of the pool address a slot by a 32-bit index (num_blocks * block_size slots at most)
constexpr int64_t kMaxPoolSlots = (int64_t)1 << 32;
constexpr int kMaxGridYZ = 65535;

int esize_of(int dtype) { return dtype == PA_F32 ? 4 : dtype == PA_BF16 ? 2 : dtype == PA_FP8_E4M3 ? 1 : 0; }
bool finite_nonzero(float x) { return x == x && x != 0.f && x - x == 0.f; }

int log2_pow2(int v) {
  if (v <= 0 || (v & (v - 1))) return -1;
  int k = 0;
  while ((1 << k) < v) ++k;
  return k;
}

bool supported_block_size(int bs) { return bs >= 8 && bs <= 256 && log2_pow2(bs) >= 0; }
bool supported_head_dim(int d) {
  return d == 64 || d == 80 || d == 96 || d == 112 || d == 128 || d == 192 || d == 256;
}
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// A pointer as a kernel on the current device must use it: this device's memory as it is, pinned host memory
// through its device-side address. Anything else -- pageable host memory HIP does not know, managed memory,
// another GPU's memory -- is not something the kernel may touch: nullptr.
void* device_view(const void* p) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (attr.type == hipMemoryTypeDevice) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess || attr.device != cur) return nullptr;
    return const_cast<void*>(p);
  }
  if (attr.type == hipMemoryTypeHost) {
    void* d = nullptr;
    if (hipHostGetDevicePointer(&d, const_cast<void*>(p), 0) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    return d;
  }
  return nullptr;
}

struct Plan {
  int status = PA_OK;
  int32_t partition = 0;       // tokens per partition as launched
  int32_t max_partitions = 1;  // partitions of the longest context
  int32_t parts_per_wave = 1;  // consecutive partitions one wave covers
  bool split = false;
  bool mfma = false;           // the matrix-core kernel runs (else the per-head one)
  int32_t col_groups = 1;      // its column groups of 16 per KV head
  int32_t cg_per_wave = 1;     // column groups one wave of its partition kernel serves
  bool balanced = false;       // balanced split (equal runs of tiles per wave) of either kernel
  int32_t chunks = 0;          // its runs (per query head for the single-head kernel)
  size_t ws_bytes = 0;
  size_t ws_ml_offset = 0;
  size_t ws_prefix_offset = 0; // balanced split: the rows' tile prefix
};

// Consecutive partitions one wave of the GQA kernel covers (1 or 2): two when the caller asks for partitions
// of 512..1023 tokens, so that a wave still streams about 1024 tokens. Needs partitions made of whole
// 32-token tiles, head_dim <= 128 and one column group per wave (the registers that park the first
// partition's state).
int32_t gqa_parts_per_wave(int32_t partition, int32_t head_dim, int32_t cg_per_wave) {
  return head_dim <= 128 && cg_per_wave == 1 && partition >= 512 && partition < 1024 &&
                 partition % pa::kGqaTileTokens == 0
             ? 2
             : 1;
}

// Library choice of partition size. A partition is the unit of work of one wave (the GQA kernel may take
// two): long enough that the partial writes and the merge stay a small fraction of the traffic and that
// per-wave start-up is amortised, short enough that the grid holds a few waves per slot of the chip so the
// load is balanced. Measured on MI355X: 512 tokens for the single-head kernel, halved while its grid would
// hold fewer than 4096 waves (two per wave slot), and 1024 for the grouped-query kernel, halved while its grid
// would hold fewer than 2048 waves (one per slot: its waves run longest when they all start together). The
// waves are counted per span a wave covers: 512-token partitions go two to a grouped-query wave, so halving
// 1024 to 512 adds no wave and the rule goes on to 256 (measured on MI355X: 64 sequences x 8 KV heads with
// 128..2048-token contexts, 88 -> 67 us).
// `rows` counts the waves per span: (sequence, KV head, column group) triples for the grouped-query kernel,
// (query row, query head) pairs for the single-head one.
// The grouped-query kernel runs single pass when its grid already holds a wave per slot without splitting
// (measured on MI355X: 13-15% faster for 7B-shaped verification batches, whose 2048 (sequence, head) waves
// fill the chip; the single-head kernel's 4096-wave rule keeps its split there, 11-13% faster than without).
int32_t pick_partition(int64_t rows, int32_t max_context_len, bool gqa, int32_t head_dim, int32_t cg_per_wave) {
  int32_t part = gqa ? 1024 : 512;
  const int64_t min_waves = gqa ? 2048 : 4096;
  if (gqa && rows >= min_waves) return 0;
  auto waves = [&](int32_t p) {
    const int64_t span = (int64_t)p * (gqa ? gqa_parts_per_wave(p, head_dim, cg_per_wave) : 1);
    return rows * ((max_context_len + span - 1) / span);
  };
  while (part > 64 && waves(part) < min_waves) part /= 2;
  return max_context_len <= part ? 0 : part;
}

// num_tokens query rows (num_seqs in decode), at most max_query_len per sequence (1 in decode).
Plan make_plan(int32_t num_seqs, int32_t num_tokens, int32_t max_query_len, int32_t num_q_heads,
               int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_context_len, int32_t kv_dtype,
               int32_t partition_size) {
  Plan p;
  if (num_seqs < 0 || num_tokens < 0 || max_query_len < 1 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0 || block_size <= 0 || max_context_len < 0 || num_q_heads % num_kv_heads != 0 ||
      (int64_t)num_tokens > (int64_t)num_seqs * max_query_len) {
    p.status = PA_ERR_SHAPE;
    return p;
  }
  if (esize_of(kv_dtype) == 0) {
    p.status = PA_ERR_DTYPE;
    return p;
  }
  // a 16-row tile is addressed through one buffer descriptor, whose size field is a signed 32-bit count
  const int64_t tile_bytes = (int64_t)kTileTokens * num_kv_heads * head_dim * esize_of(kv_dtype);
  if (!supported_head_dim(head_dim) || !supported_block_size(block_size) || num_seqs > kMaxGridYZ ||
      num_tokens > kMaxGridYZ || tile_bytes > INT32_MAX) {
    p.status = PA_ERR_UNSUPPORTED;
    return p;
  }
  // a wave-wide load covers 64 x 16 bytes of whole head rows (padded to a power of two of 16-byte chunks) and
  // must stay inside one 8-slot block: rows of at most 64 bytes (E4M3 at head_dim 64) would put 16 slots in it
  if (block_size == 8 && head_dim * esize_of(kv_dtype) <= 64) {
    p.status = PA_ERR_UNSUPPORTED;
    return p;
  }
  if (partition_size < -1 || (partition_size > PA_PARTITION_BALANCED && partition_size % kTileTokens != 0)) {
    p.status = PA_ERR_SHAPE;
    return p;
  }
  const bool gqa = pa::gqa_mfma_supported(kv_dtype, head_dim, num_q_heads / num_kv_heads, max_query_len);
  p.mfma = gqa;
  p.col_groups = gqa ? (num_q_heads / num_kv_heads * max_query_len + 15) / 16 : 1;
  p.cg_per_wave = gqa ? pa::gqa_cg_per_wave(p.col_groups, head_dim, kv_dtype) : 1;
  const int32_t slots = (p.col_groups + p.cg_per_wave - 1) / p.cg_per_wave;  // waves per (sequence, KV head)
  if ((int64_t)(num_kv_heads + 7) / 8 * p.col_groups > INT32_MAX) {
    p.status = PA_ERR_UNSUPPORTED;
    return p;
  }
  const int64_t rows = gqa ? (int64_t)num_seqs * num_kv_heads * slots : (int64_t)num_tokens * num_q_heads;
  // The balanced split needs rows (sequences, on the matrix-core kernel) one workgroup's LDS holds and tile
  // counts that fit 32 bits; on the matrix-core kernel also one column group.
  const int64_t listed = gqa ? num_seqs : num_tokens;  // items of the tile list
  const bool balanced_ok = num_tokens <= pa::kMaxBalancedRows && listed <= pa::kMaxBalancedRows &&
                           listed * (max_context_len > 0 ? max_context_len : 1) <= (int64_t)1 << 30 &&
                           (!gqa || p.col_groups == 1);
  if (partition_size == PA_PARTITION_BALANCED && !balanced_ok) {
    p.status = PA_ERR_UNSUPPORTED;
    return p;
  }
  int32_t part =
      partition_size == -1 ? pick_partition(rows, max_context_len, gqa, head_dim, p.cg_per_wave) : partition_size;
  const int64_t whole = round_up((size_t)(max_context_len > 0 ? max_context_len : 1), kTileTokens);
  // The library takes the balanced split wherever it would otherwise split the single-head kernel's contexts.
  // On the matrix cores it takes it only where the partitions would launch more than one round of resident
  // waves: measured on MI355X over grouped-query batches (bf16 and E4M3), it then gained 5-21%, while partitions
  // that all start together won by 3-8% (70B-shaped batch, 16 sequences of 8k-16k tokens) -- their fewer
  // concurrent read streams keep the memory system less congested. A shared prefix favours partitions (277
  // against 267 us for 128 sequences of 4096 tokens sharing the first 1024, with 1024-token partitions), but
  // the host cannot see sharing: a caller that knows of it asks for partitions.
  const bool split_default = partition_size == -1 && balanced_ok && part > 0 && part < whole;
  const bool more_than_a_round =
      gqa && part > 0 &&
      rows * ((max_context_len + (int64_t)part * gqa_parts_per_wave(part, head_dim, p.cg_per_wave) - 1) /
              ((int64_t)part * gqa_parts_per_wave(part, head_dim, p.cg_per_wave))) > pa::kResidentWaves;
  // Several new tokens per sequence on the matrix cores: a single pass that fills a round of resident waves
  // leaves them unequal (each reads its sequence's whole context); equal runs gained 1-8% there (7B-shaped
  // batches of 2, 4 and 8 rows per sequence, bf16 and E4M3).
  const bool uneven_pass = gqa && max_query_len > 1 && partition_size == -1 && balanced_ok &&
                           (part == 0 || part >= whole) && rows >= pa::kResidentWaves;
  if (partition_size == PA_PARTITION_BALANCED || (split_default && (!gqa || more_than_a_round)) || uneven_pass) {
    p.balanced = true;
    p.split = true;
    p.chunks = gqa ? pa::gqa_balanced_chunks(num_kv_heads)
                   : pa::balanced_chunks(num_q_heads,
                                         pa::valu_heads_per_wave(kv_dtype, head_dim, num_q_heads / num_kv_heads));
    p.partition = 0;
    p.max_partitions = 1;
    const int64_t ql = gqa ? max_query_len : 1;  // partial slots per (head, run, side)
    const size_t o_bytes = pa::balanced_o_elems(num_q_heads, p.chunks, head_dim, ql) * sizeof(float);
    p.ws_ml_offset = round_up(o_bytes, 256);
    p.ws_prefix_offset =
        round_up(p.ws_ml_offset + pa::balanced_ml_elems(num_q_heads, p.chunks, ql) * sizeof(float), 256);
    p.ws_bytes = p.ws_prefix_offset + ((size_t)listed + 1) * sizeof(int32_t);
    return p;
  }
  if (part == 0 || part >= whole) {
    p.partition = (int32_t)(whole > INT32_MAX ? INT32_MAX : whole);
    p.max_partitions = 1;
    p.split = false;
    return p;
  }
  // one partial per wave span: a grouped-query wave that covers two partitions merges their states itself
  p.parts_per_wave = gqa ? gqa_parts_per_wave(part, head_dim, p.cg_per_wave) : 1;
  const int64_t span = (int64_t)part * p.parts_per_wave;
  const int64_t pm = (max_context_len + span - 1) / span;
  if (pm > kMaxGridYZ) {
    p.status = PA_ERR_UNSUPPORTED;
    return p;
  }
  p.partition = part;
  p.max_partitions = (int32_t)pm;
  p.split = true;
  const size_t o_bytes = pa::ws_o_elems(num_tokens, num_q_heads, pm, head_dim) * sizeof(float);
  p.ws_ml_offset = round_up(o_bytes, 256);
  p.ws_bytes = p.ws_ml_offset + pa::ws_ml_elems(num_tokens, num_q_heads, pm) * sizeof(float);
  return p;
}

// Scratch of paged_attention_decode_noalloc: the split-context partials of a call that may not allocate. One copy
// per GPU the library runs on, held until the process ends. In host code `scratch` names a host-side stand-in,
// not device memory: the device address of each GPU's copy comes from hipGetSymbolAddress with that GPU
// current, and only that address is handed to kernels.
static __device__ __align__(256) char scratch[PA_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_addr[kMaxDevices] = {};

// Device address of the current GPU's scratch copy, looked up once per device (nullptr on failure).
void* scratch_of_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_addr[dev] = p;
  }
  return g_scratch_addr[dev];
}

}  // namespace

extern "C" {

int pa_abi_version(void) { return PA_ABI_VERSION; }

const char* pa_strerror(int status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE: invalid or inconsistent sizes";
    case PA_ERR_DTYPE: return "PA_ERR_DTYPE: unsupported dtype or dtype pair";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: head_dim, block_size or grid size not implemented";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing or too small";
    case PA_ERR_HIP: return "PA_ERR_HIP: a HIP launch or runtime call failed";
    case PA_ERR_ALIGN: return "PA_ERR_ALIGN: a pointer is not 16-byte aligned";
    case PA_ERR_POINTER: return "PA_ERR_POINTER: memory the device cannot access (pageable host memory, another GPU)";
    case PA_ERR_SCRATCH:
      return "PA_ERR_SCRATCH: the call needs more split-context scratch than the library's static buffer "
             "(PA_STATIC_SCRATCH_BYTES) holds; pass a workspace to paged_attention_decode_scaled instead";
    default: return "unknown status";
  }
}

int32_t paged_attention_partition_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t max_context_len, int32_t block_size,
                                       int32_t kv_dtype, int32_t partition_size) {
  const Plan p = make_plan(num_seqs, num_seqs, 1, num_q_heads, num_kv_heads, head_dim, block_size,
                           max_context_len, kv_dtype, partition_size);
  if (p.status != PA_OK) return p.status;
  return p.balanced ? PA_PARTITION_BALANCED : p.split ? p.partition : 0;
}

size_t paged_attention_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t max_context_len, int32_t block_size,
                                       int32_t kv_dtype, int32_t partition_size) {
  const Plan p = make_plan(num_seqs, num_seqs, 1, num_q_heads, num_kv_heads, head_dim, block_size,
                           max_context_len, kv_dtype, partition_size);
  return p.status == PA_OK ? p.ws_bytes : 0;
}

int32_t paged_attention_multi_partition_size(int32_t num_seqs, int32_t num_query_tokens, int32_t max_query_len,
                                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                             int32_t max_context_len, int32_t block_size, int32_t kv_dtype,
                                             int32_t partition_size) {
  const Plan p = make_plan(num_seqs, num_query_tokens, max_query_len, num_q_heads, num_kv_heads, head_dim,
                           block_size, max_context_len, kv_dtype, partition_size);
  if (p.status != PA_OK) return p.status;
  return p.balanced ? PA_PARTITION_BALANCED : p.split ? p.partition : 0;
}

size_t paged_attention_multi_workspace_bytes(int32_t num_seqs, int32_t num_query_tokens, int32_t max_query_len,
                                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                             int32_t max_context_len, int32_t block_size, int32_t kv_dtype,
                                             int32_t partition_size) {
  const Plan p = make_plan(num_seqs, num_query_tokens, max_query_len, num_q_heads, num_kv_heads, head_dim,
                           block_size, max_context_len, kv_dtype, partition_size);
  return p.status == PA_OK ? p.ws_bytes : 0;
}

int paged_attention_decode(float* out, const void* query, const void* key_cache, const void* value_cache,
                           const int32_t* block_tables, const int32_t* context_lens, float scale,
                           int32_t block_size, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int64_t num_blocks, int32_t max_blocks_per_seq,
                           int32_t max_context_len, int32_t q_dtype, int32_t kv_dtype, int32_t partition_size,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (kv_dtype == PA_FP8_E4M3) return PA_ERR_DTYPE;  // a quantised cache needs its scales
  return paged_attention_decode_scaled(out, query, key_cache, value_cache, block_tables, context_lens, scale, 1.f,
                                       1.f, block_size, num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks,
                                       max_blocks_per_seq, max_context_len, q_dtype, kv_dtype, partition_size,
                                       workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// The new tokens of paged_attention_decode_append: one K/V row per sequence and its slot, written into the pools.
struct Append {
  const void* key;
  const void* value;
  void* key_cache;
  void* value_cache;
  const int32_t* slot_mapping;
};

// Shared by the decode and multi-token entry points: query_start == nullptr means one query row per sequence.
// With static_scratch the split-context partials go to this GPU's static scratch instead of `workspace`. With
// `app`, each sequence's new token is written into the pools as part of the call (paged_attention_decode_append).
int attention(float* out, const void* query, const void* key_cache, const void* value_cache,
              const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start, float scale,
              float k_scale, float v_scale, int32_t block_size, int32_t num_seqs, int32_t num_tokens,
              int32_t max_query_len, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
              int64_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len, int32_t q_dtype,
              int32_t kv_dtype, int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream,
              bool static_scratch = false, const Append* app = nullptr) {
  const Plan plan = make_plan(num_seqs, num_tokens, max_query_len, num_q_heads, num_kv_heads, head_dim,
                              block_size, max_context_len, kv_dtype, partition_size);
  if (plan.status != PA_OK) return plan.status;
  if (static_scratch && plan.ws_bytes > PA_STATIC_SCRATCH_BYTES) return PA_ERR_SCRATCH;
  const bool pair_ok = (q_dtype == PA_F32 && kv_dtype == PA_F32) || (q_dtype == PA_BF16 && kv_dtype == PA_BF16) ||
                       (q_dtype == PA_BF16 && kv_dtype == PA_FP8_E4M3);
  if (!pair_ok) return PA_ERR_DTYPE;
  if (!finite_nonzero(k_scale) || !finite_nonzero(v_scale)) return PA_ERR_SHAPE;
  if (num_blocks <= 0 || num_blocks > INT32_MAX || max_blocks_per_seq <= 0 ||
      (int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
    return PA_ERR_SHAPE;
  if (num_blocks * block_size > kMaxPoolSlots) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0 || num_tokens == 0) return PA_OK;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens) return PA_ERR_NULL;
  if (!aligned16(out) || !aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache) ||
      !aligned4(block_tables) || !aligned4(context_lens) || !aligned4(query_start))
    return PA_ERR_ALIGN;
  if (plan.split) {
    if (static_scratch) {  // every argument is valid: the call will launch
      workspace = scratch_of_current_device();
      if (!workspace) return PA_ERR_HIP;
      workspace_bytes = PA_STATIC_SCRATCH_BYTES;
    }
    if (!workspace || workspace_bytes < plan.ws_bytes) return PA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return PA_ERR_ALIGN;
  }

  pa::DecodeArgs a;
  a.out = out;
  a.query = query;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.ws_o = plan.split ? static_cast<float*>(workspace) : nullptr;
  a.ws_ml = plan.split ? reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.ws_ml_offset) : nullptr;
  a.scale_log2 = scale * k_scale * 1.4426950408889634f;
  a.v_scale = v_scale;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.group = num_q_heads / num_kv_heads;
  a.bs_log2 = log2_pow2(block_size);
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_context_len = max_context_len;
  a.partition = plan.partition;
  a.max_partitions = plan.max_partitions;
  a.parts_per_wave = plan.parts_per_wave;
  a.split = plan.split ? 1 : 0;
  a.num_tokens = num_tokens;
  a.max_query_len = max_query_len;
  a.col_groups = plan.col_groups;
  a.cg_per_wave = plan.cg_per_wave;
  a.chunks = plan.chunks;
  a.tile_prefix =
      plan.balanced ? reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + plan.ws_prefix_offset) : nullptr;
  a.seq_prefix = plan.balanced && plan.mfma ? 1 : 0;  // the matrix-core tile list is one of sequences
  a.new_key = nullptr;
  a.new_value = nullptr;
  a.slot_mapping = nullptr;
  a.key_out = nullptr;
  a.value_out = nullptr;
  a.new_k_scale = k_scale;
  a.new_v_scale = v_scale;

  hipStream_t st = static_cast<hipStream_t>(stream);
  if (app) {
    // Every decode kernel appends the new tokens itself (for an E4M3 cache from bf16 rows, which every E4M3
    // decode has, with scales whose quotients the kernels' quantiser forms without a division: magnitudes 2^-32 ..
    // 2^32). A call with max_context_len 0 gives its sequences no tile in which a balanced run could write the
    // token, and an E4M3 scale outside that range would need the division: such calls write the tokens first,
    // as reshape_and_cache or reshape_and_cache_fp8 would, and then attend.
    const bool fused = !query_start && max_context_len > 0 &&
                       (kv_dtype != PA_FP8_E4M3 ||
                        (q_dtype == PA_BF16 && pa::e4m3_fast_scale(k_scale) && pa::e4m3_fast_scale(v_scale)));
    hipError_t e = hipSuccess;
    if (fused) {
      a.new_key = app->key;
      a.new_value = app->value;
      a.slot_mapping = app->slot_mapping;
      a.key_out = app->key_cache;
      a.value_out = app->value_cache;
    } else if (kv_dtype == PA_FP8_E4M3) {
      e = pa::launch_reshape_and_cache_fp8(app->key, app->value, app->key_cache, app->value_cache, app->slot_mapping,
                                           num_seqs, (int64_t)num_kv_heads * head_dim, block_size, num_blocks,
                                           q_dtype, k_scale, v_scale, st);
    } else {
      e = pa::launch_reshape_and_cache(app->key, app->value, app->key_cache, app->value_cache, app->slot_mapping,
                                       num_seqs, (int64_t)num_kv_heads * head_dim * esize_of(kv_dtype), block_size,
                                       num_blocks, st);
    }
    if (e != hipSuccess) return PA_ERR_HIP;
  }
  if (plan.balanced) {
    const hipError_t e = plan.mfma ? pa::launch_decode_gqa_mfma_balanced(a, kv_dtype, st)
                                   : pa::launch_decode_valu_balanced(a, kv_dtype, st);
    if (e != hipSuccess) return PA_ERR_HIP;
    return pa::launch_balanced_reduce(a, st) == hipSuccess ? PA_OK : PA_ERR_HIP;
  }
  const hipError_t err = plan.mfma ? pa::launch_decode_gqa_mfma(a, kv_dtype, st) : pa::launch_decode_valu(a, kv_dtype, st);
  if (err != hipSuccess) return PA_ERR_HIP;
  if (plan.split && pa::launch_lse_reduce(a, st) != hipSuccess) return PA_ERR_HIP;
  return PA_OK;
}

}  // namespace

extern "C" {

int paged_attention_decode_scaled(float* out, const void* query, const void* key_cache, const void* value_cache,
                                  const int32_t* block_tables, const int32_t* context_lens, float scale,
                                  float k_scale, float v_scale, int32_t block_size, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                                  int32_t max_blocks_per_seq, int32_t max_context_len, int32_t q_dtype,
                                  int32_t kv_dtype, int32_t partition_size, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return attention(out, query, key_cache, value_cache, block_tables, context_lens, nullptr, scale, k_scale, v_scale,
                   block_size, num_seqs, num_seqs, 1, num_q_heads, num_kv_heads, head_dim, num_blocks,
                   max_blocks_per_seq, max_context_len, q_dtype, kv_dtype, partition_size, workspace,
                   workspace_bytes, stream);
}

int paged_attention_decode_noalloc(float* out, const void* query, const void* key_cache, const void* value_cache,
                                   const int32_t* block_tables, const int32_t* context_lens, float scale,
                                   float k_scale, float v_scale, int32_t block_size, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                                   int32_t max_blocks_per_seq, int32_t max_context_len, int32_t q_dtype,
                                   int32_t kv_dtype, int32_t partition_size, void* stream) {
  return attention(out, query, key_cache, value_cache, block_tables, context_lens, nullptr, scale, k_scale, v_scale,
                   block_size, num_seqs, num_seqs, 1, num_q_heads, num_kv_heads, head_dim, num_blocks,
                   max_blocks_per_seq, max_context_len, q_dtype, kv_dtype, partition_size, nullptr, 0, stream,
                   /*static_scratch=*/true);
}

int paged_attention_decode_append(float* out, const void* query, const void* key, const void* value, void* key_cache,
                                  void* value_cache, const int32_t* block_tables, const int32_t* context_lens,
                                  const int32_t* slot_mapping, float scale, float k_scale, float v_scale,
                                  int32_t block_size, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int64_t num_blocks, int32_t max_blocks_per_seq,
                                  int32_t max_context_len, int32_t q_dtype, int32_t kv_dtype, int32_t partition_size,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  // the cache write's own checks first (those of reshape_and_cache, or of reshape_and_cache_fp8 with the query's
  // dtype as the source, for num_seqs new rows), then the decode's
  if (num_seqs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0) return PA_ERR_SHAPE;
  const bool quantise = kv_dtype == PA_FP8_E4M3;
  if (quantise ? q_dtype != PA_BF16 && q_dtype != PA_F32 : kv_dtype != PA_F32 && kv_dtype != PA_BF16)
    return PA_ERR_DTYPE;
  if (quantise && (!finite_nonzero(k_scale) || !finite_nonzero(v_scale))) return PA_ERR_SHAPE;
  if ((int64_t)num_kv_heads * head_dim * (quantise ? 1 : esize_of(kv_dtype)) % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (num_seqs > 0) {
    if (!key || !value || !slot_mapping) return PA_ERR_NULL;
    if (!aligned16(key) || !aligned16(value) || !aligned4(slot_mapping)) return PA_ERR_ALIGN;
  }
  const Append app{key, value, key_cache, value_cache, slot_mapping};
  return attention(out, query, key_cache, value_cache, block_tables, context_lens, nullptr, scale, k_scale, v_scale,
                   block_size, num_seqs, num_seqs, 1, num_q_heads, num_kv_heads, head_dim, num_blocks,
                   max_blocks_per_seq, max_context_len, q_dtype, kv_dtype, partition_size, workspace, workspace_bytes,
                   stream, /*static_scratch=*/false, &app);
}

int paged_attention_decode_multi(float* out, const void* query, const void* key_cache, const void* value_cache,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 const int32_t* query_start, float scale, float k_scale, float v_scale,
                                 int32_t block_size, int32_t num_seqs, int32_t num_query_tokens,
                                 int32_t max_query_len, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int64_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                                 int32_t q_dtype, int32_t kv_dtype, int32_t partition_size, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (num_seqs > 0 && num_query_tokens > 0 && !query_start) return PA_ERR_NULL;
  return attention(out, query, key_cache, value_cache, block_tables, context_lens, query_start, scale, k_scale,
                   v_scale, block_size, num_seqs, num_query_tokens, max_query_len, num_q_heads, num_kv_heads,
                   head_dim, num_blocks, max_blocks_per_seq, max_context_len, q_dtype, kv_dtype, partition_size,
                   workspace, workspace_bytes, stream);
}

int reshape_and_cache(const void* key, const void* value, void* key_cache, void* value_cache,
                      const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int64_t num_blocks, int32_t kv_dtype, void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return PA_ERR_SHAPE;
  if (esize_of(kv_dtype) == 0) return PA_ERR_DTYPE;
  const int64_t row_bytes = (int64_t)num_kv_heads * head_dim * esize_of(kv_dtype);
  if (row_bytes % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping) return PA_ERR_NULL;
  if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache) ||
      !aligned4(slot_mapping))
    return PA_ERR_ALIGN;
  if (num_tokens > INT32_MAX) return PA_ERR_UNSUPPORTED;
  return pa::launch_reshape_and_cache(key, value, key_cache, value_cache, slot_mapping, num_tokens, row_bytes,
                                      block_size, num_blocks, static_cast<hipStream_t>(stream)) == hipSuccess
             ? PA_OK
             : PA_ERR_HIP;
}

int reshape_and_cache_fp8(const void* key, const void* value, void* key_cache, void* value_cache,
                          const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int64_t num_blocks, int32_t src_dtype, float k_scale, float v_scale,
                          void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return PA_ERR_SHAPE;
  if (src_dtype != PA_F32 && src_dtype != PA_BF16) return PA_ERR_DTYPE;
  if (!finite_nonzero(k_scale) || !finite_nonzero(v_scale)) return PA_ERR_SHAPE;
  const int64_t row_elems = (int64_t)num_kv_heads * head_dim;
  if (row_elems % 16 != 0) return PA_ERR_UNSUPPORTED;  // rows are written as whole 16-byte words
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping) return PA_ERR_NULL;
  if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache) ||
      !aligned4(slot_mapping))
    return PA_ERR_ALIGN;
  return pa::launch_reshape_and_cache_fp8(key, value, key_cache, value_cache, slot_mapping, num_tokens, row_elems,
                                          block_size, num_blocks, src_dtype, k_scale, v_scale,
                                          static_cast<hipStream_t>(stream)) == hipSuccess
             ? PA_OK
             : PA_ERR_HIP;
}

int copy_blocks(void* key_cache, void* value_cache, const int32_t* block_pairs, int32_t num_pairs,
                int32_t block_size, int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks, int32_t kv_dtype,
                void* stream) {
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return PA_ERR_SHAPE;
  if (esize_of(kv_dtype) == 0) return PA_ERR_DTYPE;
  const int64_t block_bytes = (int64_t)block_size * num_kv_heads * head_dim * esize_of(kv_dtype);
  if (block_bytes % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  if (!key_cache || !value_cache || !block_pairs) return PA_ERR_NULL;
  if (!aligned16(key_cache) || !aligned16(value_cache) || !aligned4(block_pairs)) return PA_ERR_ALIGN;
  const int64_t per_wg = 256 * 4 * 16;
  if ((block_bytes + per_wg - 1) / per_wg > kMaxGridYZ) return PA_ERR_UNSUPPORTED;
  return pa::launch_copy_blocks(key_cache, value_cache, block_pairs, num_pairs, block_bytes, num_blocks,
                                static_cast<hipStream_t>(stream)) == hipSuccess
             ? PA_OK
             : PA_ERR_HIP;
}

int swap_blocks(void* dst_key_cache, void* dst_value_cache, int64_t dst_num_blocks, const void* src_key_cache,
                const void* src_value_cache, int64_t src_num_blocks, const int32_t* block_pairs, int32_t num_pairs,
                int32_t block_size, int32_t num_kv_heads, int32_t head_dim, int32_t kv_dtype, void* stream) {
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || dst_num_blocks <= 0 ||
      src_num_blocks <= 0)
    return PA_ERR_SHAPE;
  if (esize_of(kv_dtype) == 0) return PA_ERR_DTYPE;
  const int64_t block_bytes = (int64_t)block_size * num_kv_heads * head_dim * esize_of(kv_dtype);
  if (block_bytes % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  if (!dst_key_cache || !dst_value_cache || !src_key_cache || !src_value_cache || !block_pairs) return PA_ERR_NULL;
  if (!aligned16(dst_key_cache) || !aligned16(dst_value_cache) || !aligned16(src_key_cache) ||
      !aligned16(src_value_cache) || !aligned4(block_pairs))
    return PA_ERR_ALIGN;
  const int64_t per_wg = 256 * 4 * 16;
  if ((block_bytes + per_wg - 1) / per_wg > kMaxGridYZ) return PA_ERR_UNSUPPORTED;
  // the kernel reads and writes the pools directly: each must be memory this device can reach
  void* dk = device_view(dst_key_cache);
  void* dv = device_view(dst_value_cache);
  const void* sk = device_view(src_key_cache);
  const void* sv = device_view(src_value_cache);
  const int32_t* pairs = static_cast<const int32_t*>(device_view(block_pairs));
  if (!dk || !dv || !sk || !sv || !pairs) return PA_ERR_POINTER;
  return pa::launch_swap_blocks(dk, dv, dst_num_blocks, sk, sv, src_num_blocks, pairs, num_pairs, block_bytes,
                                static_cast<hipStream_t>(stream)) == hipSuccess
             ? PA_OK
             : PA_ERR_HIP;
}

int paged_gather(void* out_key, void* out_value, const void* key_cache, const void* value_cache,
                 const int32_t* block_tables, const int32_t* context_lens, int32_t block_size, int32_t num_seqs,
                 int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks, int32_t max_blocks_per_seq,
                 int32_t max_context_len, int32_t kv_dtype, void* stream) {
  if (num_seqs < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks <= 0 || num_blocks > INT32_MAX ||
      max_blocks_per_seq <= 0 || max_context_len < 0 ||
      (int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
    return PA_ERR_SHAPE;
  if (esize_of(kv_dtype) == 0) return PA_ERR_DTYPE;
  if (!supported_block_size(block_size) || num_seqs > kMaxGridYZ || num_blocks * block_size > kMaxPoolSlots)
    return PA_ERR_UNSUPPORTED;
  const int64_t row_bytes = (int64_t)num_kv_heads * head_dim * esize_of(kv_dtype);
  if (row_bytes % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0 || max_context_len == 0) return PA_OK;
  if (!out_key || !out_value || !key_cache || !value_cache || !block_tables || !context_lens) return PA_ERR_NULL;
  if (!aligned16(out_key) || !aligned16(out_value) || !aligned16(key_cache) || !aligned16(value_cache) ||
      !aligned4(block_tables) || !aligned4(context_lens))
    return PA_ERR_ALIGN;
  return pa::launch_paged_gather(out_key, out_value, key_cache, value_cache, block_tables, context_lens, num_seqs,
                                 log2_pow2(block_size), num_blocks, max_blocks_per_seq, max_context_len, row_bytes,
                                 static_cast<hipStream_t>(stream)) == hipSuccess
             ? PA_OK
             : PA_ERR_HIP;
}

}  // extern "C"
