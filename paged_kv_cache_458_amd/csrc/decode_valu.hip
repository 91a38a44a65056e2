// Paged decode attention on the vector ALUs of gfx950: one wave64 per (sequence, query head, partition).
//
// What it computes (vLLM PagedAttention, page 1 sections 3.1-3.2): the new token of each sequence attends
// over all earlier K/V of that sequence, which the block table scatters through the block pools. The
// softmax is taken in one streaming pass with a running maximum and sum (online softmax), so K and V are
// read from HBM exactly once.
//
// Lane layout. A 16-byte load covers 16 E4M3, 8 bf16 or 4 fp32 elements, so one head's row (head_dim
// elements) spans kHeadLanes lanes, padded to a power of two kRowLanes (the padding lanes read zeros through an
// out-of-range offset and store nothing), and one wave-wide load covers kRows consecutive slots of a block; a
// tile of kTileTok tokens takes kLoads (at most 4) loads for K and as many for V. Every lane consumes exactly the bytes it loaded -- there is no reuse
// to stage through LDS. Each group of kRowLanes lanes ("row group") owns the tile rows r, r + kRows, ... and
// keeps its own running (max, sum, accumulator); the groups are merged once at the end with the same
// log-sum-exp rule the split-context reduce uses. The dot product of a row is finished with DPP adds inside
// the row group, so a score never leaves its 16 lanes.
//
// Pipelining. Tile j+1 is loaded into a second register set while tile j is consumed; the block id of a
// tile comes from a scalar load of the table, so address generation stays on the scalar unit.
#include "pa_device.h"
#include "pa_kernels.h"
#include "../../include/paged_attention.h"

namespace pa {
namespace {

constexpr int next_pow2(int v) { return v <= 1 ? 1 : 2 * next_pow2((v + 1) / 2); }

template <int KV, int D>
struct Shape {
  static constexpr int kEsize = KV == PA_F32 ? 4 : KV == PA_BF16 ? 2 : 1;
  static constexpr int kEpl = 16 / kEsize;               // elements per lane per 16-byte load
  static constexpr int kHeadLanes = D / kEpl;            // lanes holding one head's row
  static constexpr int kRowLanes = next_pow2(kHeadLanes);  // lanes per row group (the rest of them idle)
  static constexpr int kRows = kWave / kRowLanes;        // slots per wave-wide load
  // tokens per tile: at most 4 loads per lane for K (and for V), at most 16 tokens
  static constexpr int kTileTok = kRows * 4 < kTile ? kRows * 4 : kTile;
  static constexpr int kLoads = kTileTok / kRows;        // loads per tile (per K and per V)
  static_assert(D % kEpl == 0 && kRowLanes <= kWave, "head_dim must fill whole 16-byte chunks");
  static constexpr int kQEsize = KV == PA_F32 ? 4 : 2;  // the query is bf16 over an E4M3 cache
  static constexpr int kQWords = kEpl * kQEsize / 16;   // 16-byte words of query per lane chunk
};

template <int N>
struct Words {
  U4 w[N];
};

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

__device__ __forceinline__ float dot2(uint32_t q, uint32_t k, float d) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q), __builtin_bit_cast(bf16x2, k), d, false);
}

template <int KV>
__device__ __forceinline__ float dot_chunk(const Words<Shape<KV, 64>::kQWords>& q, const U4& k);

template <>
__device__ __forceinline__ float dot_chunk<PA_BF16>(const Words<1>& q, const U4& k) {
  float d = dot2(q.w[0].x, k.x, 0.f);
  d = dot2(q.w[0].y, k.y, d);
  d = dot2(q.w[0].z, k.z, d);
  return dot2(q.w[0].w, k.w, d);
}

template <>
__device__ __forceinline__ float dot_chunk<PA_F32>(const Words<1>& q, const U4& k) {
  float d = __uint_as_float(q.w[0].x) * __uint_as_float(k.x);
  d = fmaf(__uint_as_float(q.w[0].y), __uint_as_float(k.y), d);
  d = fmaf(__uint_as_float(q.w[0].z), __uint_as_float(k.z), d);
  d = fmaf(__uint_as_float(q.w[0].w), __uint_as_float(k.w), d);
  return d;
}

// E4M3 keys: each word of four codes becomes two bf16 pairs, dotted with the matching bf16 query words
template <>
__device__ __forceinline__ float dot_chunk<PA_FP8_E4M3>(const Words<2>& q, const U4& k) {
  uint32_t a, b;
  float d = 0.f;
  e4m3x4_to_bf16x4(k.x, a, b);
  d = dot2(q.w[0].x, a, d);
  d = dot2(q.w[0].y, b, d);
  e4m3x4_to_bf16x4(k.y, a, b);
  d = dot2(q.w[0].z, a, d);
  d = dot2(q.w[0].w, b, d);
  e4m3x4_to_bf16x4(k.z, a, b);
  d = dot2(q.w[1].x, a, d);
  d = dot2(q.w[1].y, b, d);
  e4m3x4_to_bf16x4(k.w, a, b);
  d = dot2(q.w[1].z, a, d);
  return dot2(q.w[1].w, b, d);
}

__device__ __forceinline__ void axpy_bf16x2(float* acc, float p, uint32_t v) {
  acc[0] = fmaf(p, bf16_lo(v), acc[0]);
  acc[1] = fmaf(p, bf16_hi(v), acc[1]);
}

template <int KV>
__device__ __forceinline__ void axpy_chunk(float* acc, float p, const U4& v) {
  if constexpr (KV == PA_BF16) {
    axpy_bf16x2(acc + 0, p, v.x);
    axpy_bf16x2(acc + 2, p, v.y);
    axpy_bf16x2(acc + 4, p, v.z);
    axpy_bf16x2(acc + 6, p, v.w);
  } else if constexpr (KV == PA_FP8_E4M3) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t a, b;
      e4m3x4_to_bf16x4(w[i], a, b);
      axpy_bf16x2(acc + 4 * i, p, a);
      axpy_bf16x2(acc + 4 * i + 2, p, b);
    }
  } else {
    acc[0] = fmaf(p, __uint_as_float(v.x), acc[0]);
    acc[1] = fmaf(p, __uint_as_float(v.y), acc[1]);
    acc[2] = fmaf(p, __uint_as_float(v.z), acc[2]);
    acc[3] = fmaf(p, __uint_as_float(v.w), acc[3]);
  }
}

constexpr int kWavesPerGroup = 2;  // waves (query heads) per workgroup
constexpr int kStages = 3;         // 16-token tiles in flight per wave

template <int KV, int D>
__global__ __launch_bounds__(kWave * kWavesPerGroup) void decode_valu_kernel(const DecodeArgs a) {
  using S = Shape<KV, D>;
  constexpr int NL = S::kLoads;
  constexpr int TT = S::kTileTok;
  const int lane = threadIdx.x & (kWave - 1);
  const int h = blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6);
  const int part = blockIdx.y;
  const int row = blockIdx.z;  // query row: the sequence itself unless sequences bring several new tokens
  if (h >= a.num_q_heads) return;
  const int s = seq_of_row(a, row);

  // partitions cover the sequence's L positions; this row attends over the first E of them (E = L in decode)
  const int L = min(max(a.context_lens[s], 0), a.max_context_len);
  const int t0 = part * a.partition;
  if (part > 0 && t0 >= L) return;  // this sequence has fewer partitions
  const int E = row_extent(a, s, row, L);
  const int t1 = max(t0, min(min(L, t0 + a.partition), E));
  const int g = h / a.group;
  const int r = lane / S::kRowLanes;  // row group
  const int c = lane % S::kRowLanes;  // 16-byte chunk of the head's row
  const bool lane_ok = c < S::kHeadLanes;  // false for the padding lanes of a row group

  const int64_t row_bytes = (int64_t)a.num_kv_heads * D * S::kEsize;
  // padding lanes load at an offset above every descriptor's size (at most 16 rows < 2^30 bytes), so they read
  // zeros without touching memory
  constexpr uint32_t kNowhere = 0x80000000u;
  uint32_t lane_off[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i)
    lane_off[i] = lane_ok ? (uint32_t)((i * S::kRows + r) * row_bytes + (int64_t)g * D * S::kEsize + c * 16)
                          : kNowhere;

  const char* __restrict__ kbase = static_cast<const char*>(a.key_cache);
  const char* __restrict__ vbase = static_cast<const char*>(a.value_cache);
  const int32_t* __restrict__ table = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  Words<S::kQWords> q;
  {
    const char* qp = static_cast<const char*>(a.query) + ((int64_t)row * a.num_q_heads + h) * D * S::kQEsize +
                     (lane_ok ? c : 0) * 16 * S::kQWords;
#pragma unroll
    for (int i = 0; i < S::kQWords; ++i) {
      const U4 v = reinterpret_cast<const U4*>(qp)[i];
      q.w[i] = lane_ok ? v : U4{0u, 0u, 0u, 0u};
    }
  }

  float m = -INFINITY, l = 0.f;
  float acc[S::kEpl];
#pragma unroll
  for (int e = 0; e < S::kEpl; ++e) acc[e] = 0.f;
  bool bad = false;
  const int ntiles = (t1 - t0 + TT - 1) / TT;

  U4 kb[kStages][NL], vb[kStages][NL];
  // The loads stay unconditional, so the wait counters of the two register sets never merge across a branch:
  // a 16-token tile has a descriptor per 8-row half that covers only its rows below the partition end, and
  // rows past it (a tile index past the end: all of them) read as zero without touching memory. The halves lie
  // in one block unless blocks hold 8 slots; a wave-wide load of at most 8 rows never straddles them. Shapes
  // with 16 rows per load (E4M3 at head_dim 64) take the whole tile through the first descriptor: the host
  // refuses 8-slot blocks for them. Tiles of at most 8 tokens always lie in one block.
  constexpr bool kHalves = TT == kTile && S::kRows <= kTile / 2;
  const int last8 = (t1 - 1) & ~(kTile / 2 - 1);  // start of the last live 8-row group
  auto issue = [&](U4* kq, U4* vq, int tile) {
    const int t = t0 + min(tile, ntiles - 1) * TT;
    const int64_t base0 = tile_slot_bytes(table, t, a.bs_log2, a.num_blocks, row_bytes, bad);
    const int64_t base1 = !kHalves ? base0
                          : a.bs_log2 == 3
                              ? tile_slot_bytes(table, min(t + kTile / 2, last8), a.bs_log2, a.num_blocks,
                                                row_bytes, bad)
                              : base0 + (kTile / 2) * row_bytes;
    const int rows = tile < ntiles ? min(TT, t1 - t) : 0;
    const uint32_t live0 = (uint32_t)(kHalves ? min(rows, kTile / 2) : rows) * (uint32_t)row_bytes;
    const uint32_t live1 = (uint32_t)max(rows - kTile / 2, 0) * (uint32_t)row_bytes;
    const __amdgpu_buffer_rsrc_t kr0 = make_rsrc(kbase + base0, live0), kr1 = make_rsrc(kbase + base1, live1);
    const __amdgpu_buffer_rsrc_t vr0 = make_rsrc(vbase + base0, live0), vr1 = make_rsrc(vbase + base1, live1);
    const uint32_t half_off = (uint32_t)((kTile / 2) * row_bytes);
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      if (!kHalves || i * S::kRows < kTile / 2) {
        kq[i] = load16<kPolStream>(kr0, lane_off[i]);
        vq[i] = load16<kPolStream>(vr0, lane_off[i]);
      } else {
        kq[i] = load16<kPolStream>(kr1, lane_off[i] - half_off);
        vq[i] = load16<kPolStream>(vr1, lane_off[i] - half_off);
      }
    }
  };
  auto consume = [&](const U4* kq, const U4* vq, int tile) {
    const int t = t0 + tile * TT;
    const bool full = t + TT <= t1;
    float sc[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      sc[i] = group_sum<S::kRowLanes>(dot_chunk<KV>(q, kq[i])) * a.scale_log2;
      if (!full && t + i * S::kRows + r >= t1) sc[i] = -INFINITY;
    }
    float mt = sc[0];
#pragma unroll
    for (int i = 1; i < NL; ++i) mt = fmaxf(mt, sc[i]);
    const float mn = fmaxf(m, mt);
    const float mref = mn == -INFINITY ? 0.f : mn;
    const float alpha = fast_exp2(m - mref);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < S::kEpl; ++e) acc[e] *= alpha;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const float p = fast_exp2(sc[i] - mref);
      l += p;
      U4 v = vq[i];
      if (!full && t + i * S::kRows + r >= t1) v = U4{0u, 0u, 0u, 0u};  // a past-the-end slot may hold NaN
      axpy_chunk<KV>(acc, p, v);
    }
    m = mn;
  };

  // kStages register sets in a ring: tile j + kStages - 1 is in flight while tile j is consumed
  if (ntiles > 0) {
#pragma unroll
    for (int i = 0; i < kStages - 1; ++i) issue(kb[i], vb[i], i);
    int j = 0;
    for (; j + kStages <= ntiles; j += kStages) {
#pragma unroll
      for (int i = 0; i < kStages; ++i) {
        issue(kb[(i + kStages - 1) % kStages], vb[(i + kStages - 1) % kStages], j + i + kStages - 1);
        consume(kb[i], vb[i], j + i);
      }
    }
#pragma unroll
    for (int i = 0; i < kStages - 1; ++i)
      if (j + i < ntiles) consume(kb[i], vb[i], j + i);
  }

  // merge the row groups: lanes l, l ^ kRowLanes, ... hold the same dims of different token subsets
#pragma unroll
  for (int off = S::kRowLanes; off < kWave; off <<= 1) {
    const float mo = __shfl_xor(m, off);
    const float lo = __shfl_xor(l, off);
    const float M = fmaxf(m, mo);
    const float Mr = M == -INFINITY ? 0.f : M;
    const float fa = fast_exp2(m - Mr), fb = fast_exp2(mo - Mr);
    l = l * fa + lo * fb;
#pragma unroll
    for (int e = 0; e < S::kEpl; ++e) acc[e] = acc[e] * fa + __shfl_xor(acc[e], off) * fb;
    m = M;
  }

  if (r == 0 && lane_ok) {
    const float inv = l > 0.f ? a.v_scale / l : 0.f;
    const float poison = __uint_as_float(0x7fc00000u);
    float res[S::kEpl];
#pragma unroll
    for (int e = 0; e < S::kEpl; ++e) res[e] = bad ? poison : acc[e] * inv;
    float* dst;
    if (!a.split || L <= a.partition) {
      dst = a.out + ((int64_t)row * a.num_q_heads + h) * D + c * S::kEpl;
    } else {
      const int64_t wrow = ((int64_t)row * a.num_q_heads + h) * a.max_partitions + part;
      dst = a.ws_o + wrow * D + c * S::kEpl;
      if (c == 0) {
        a.ws_ml[2 * wrow] = bad ? poison : m;
        a.ws_ml[2 * wrow + 1] = l;
      }
    }
#pragma unroll
    for (int e = 0; e < S::kEpl; e += 4)
      *reinterpret_cast<float4*>(dst + e) = make_float4(res[e], res[e + 1], res[e + 2], res[e + 3]);
  }
}

// Merge of split-context partials: with partition p giving running max m_p (log2 units), sum l_p and
// normalised output o_p, out = sum_p w_p o_p / sum_p w_p with w_p = l_p * 2^(m_p - max_p m_p). One wave per
// (sequence, head): lane p owns partition p's weight, and every lane accumulates its own head_dim / 64 dims.
// The kernel is latency-bound, so the (max, sum) pairs and the first kSpec partitions' outputs are loaded
// before the context length is known (slots past the row's partition count hold stale values and are never
// combined: the loops below stop at the count).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

constexpr int kSpec = 16;  // partitions whose outputs are loaded up front

template <int D>
__global__ __launch_bounds__(kWave) void lse_reduce_kernel(const DecodeArgs a) {
  constexpr int kDpl = (D + kWave - 1) / kWave;  // dims per lane
  constexpr int kActive = D / kDpl;              // lanes holding dims (all of them when 64 divides D)
  static_assert(D % kDpl == 0, "whole dims per lane");
  const int lane = threadIdx.x;
  const bool lane_ok = lane < kActive;  // the other lanes read lane 0's dims and store nothing
  const int h = blockIdx.x;
  const int row = blockIdx.y;  // query row
  const int s = seq_of_row(a, row);
  const int pm = a.max_partitions;
  const int64_t row0 = ((int64_t)row * a.num_q_heads + h) * pm;
  const float2* __restrict__ ml = reinterpret_cast<const float2*>(a.ws_ml) + row0;
  const float* __restrict__ o = a.ws_o + row0 * D + (lane_ok ? lane : 0) * kDpl;

  // indexes clamped to the row's last slot keep every speculative load inside the workspace without a branch
  const float2 v0 = ml[min(lane, pm - 1)];
  float ov[kSpec][kDpl];
#pragma unroll
  for (int k = 0; k < kSpec; ++k)
#pragma unroll
    for (int e = 0; e < kDpl; ++e) ov[k][e] = o[(int64_t)min(k, pm - 1) * D + e];

  // a row with a single partition was written by the partition kernel: it is merged as one partition here
  // (no early exit, which would let the compiler sink the loads above behind the length) and not stored
  const int L = min(max(a.context_lens[s], 0), a.max_context_len);
  const bool merge = L > a.partition;
  const int np = merge ? (L + a.partition - 1) / a.partition : 1;

  float M = lane < np ? v0.x : -INFINITY;
  for (int p = lane + kWave; p < np; p += kWave) M = fmaxf(M, ml[p].x);
  M = wave_max(M);
  // a row that attends over nothing (a new token with no earlier position) has only empty partials
  const float Mr = M == -INFINITY ? 0.f : M;
  float acc[kDpl];
#pragma unroll
  for (int e = 0; e < kDpl; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  for (int p0 = 0; p0 < np; p0 += kWave) {
    float w = 0.f;
    if (p0 + lane < np) {
      const float2 v = p0 == 0 ? v0 : ml[p0 + lane];
      w = v.y * fast_exp2(v.x - Mr);
    }
    wsum += w;
    const int n = min(kWave, np - p0);
    int k0 = 0;
    if (p0 == 0) {
#pragma unroll
      for (int k = 0; k < kSpec; ++k) {
        if (k < n) {
          const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), k));
#pragma unroll
          for (int e = 0; e < kDpl; ++e) acc[e] = fmaf(wk, ov[k][e], acc[e]);
        }
      }
      k0 = kSpec;
    }
    const float* __restrict__ op = o + (int64_t)p0 * D;
    for (; k0 < n; k0 += 8) {  // eight partitions' loads in flight at a time
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int k = k0 + kk;
        if (k < n) {
          const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), k));
#pragma unroll
          for (int e = 0; e < kDpl; ++e) acc[e] = fmaf(wk, op[(int64_t)k * D + e], acc[e]);
        }
      }
    }
  }
  const float wtot = wave_sum(wsum);
  const float inv = wtot > 0.f ? 1.0f / wtot : 0.f;
  if (!merge || !lane_ok) return;
  float* dst = a.out + ((int64_t)row * a.num_q_heads + h) * D + lane * kDpl;
#pragma unroll
  for (int e = 0; e < kDpl; ++e) dst[e] = acc[e] * inv;
}

}  // namespace

template <int KV>
hipError_t launch_kv(const DecodeArgs& a, dim3 grid, dim3 block, hipStream_t stream) {
  switch (a.head_dim) {
    case 64: decode_valu_kernel<KV, 64><<<grid, block, 0, stream>>>(a); break;
    case 80: decode_valu_kernel<KV, 80><<<grid, block, 0, stream>>>(a); break;
    case 96: decode_valu_kernel<KV, 96><<<grid, block, 0, stream>>>(a); break;
    case 112: decode_valu_kernel<KV, 112><<<grid, block, 0, stream>>>(a); break;
    case 128: decode_valu_kernel<KV, 128><<<grid, block, 0, stream>>>(a); break;
    case 192: decode_valu_kernel<KV, 192><<<grid, block, 0, stream>>>(a); break;
    case 256: decode_valu_kernel<KV, 256><<<grid, block, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_valu(const DecodeArgs& a, int kv_dtype, hipStream_t stream) {
  const dim3 grid((a.num_q_heads + kWavesPerGroup - 1) / kWavesPerGroup, a.split ? a.max_partitions : 1,
                  a.num_tokens);
  const dim3 block(kWave * kWavesPerGroup);
  if (kv_dtype == PA_BF16) return launch_kv<PA_BF16>(a, grid, block, stream);
  if (kv_dtype == PA_F32) return launch_kv<PA_F32>(a, grid, block, stream);
  if (kv_dtype == PA_FP8_E4M3) return launch_kv<PA_FP8_E4M3>(a, grid, block, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_lse_reduce(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.num_q_heads, a.num_tokens);
  const dim3 block(kWave);
  switch (a.head_dim) {
    case 64: lse_reduce_kernel<64><<<grid, block, 0, stream>>>(a); break;
    case 80: lse_reduce_kernel<80><<<grid, block, 0, stream>>>(a); break;
    case 96: lse_reduce_kernel<96><<<grid, block, 0, stream>>>(a); break;
    case 112: lse_reduce_kernel<112><<<grid, block, 0, stream>>>(a); break;
    case 128: lse_reduce_kernel<128><<<grid, block, 0, stream>>>(a); break;
    case 192: lse_reduce_kernel<192><<<grid, block, 0, stream>>>(a); break;
    case 256: lse_reduce_kernel<256><<<grid, block, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
