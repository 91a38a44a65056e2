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
#include "../../include/pa.h"

namespace pa {
namespace {

constexpr int next_pow2(int v) { return v <= 1 ? 1 : 2 * next_pow2((v + 1) / 2); }

// HPW heads per wave: 1, or 2 adjacent heads whose rows are exactly one row group (64- or 128-byte head rows
// without grouping), so that every wave-wide load covers pieces of two heads' rows at once.
template <int KV, int D, int HPW = 1>
struct Shape {
  static constexpr int kEsize = KV == PA_F32 ? 4 : KV == PA_BF16 ? 2 : 1;
  static constexpr int kEpl = 16 / kEsize;               // elements per lane per 16-byte load
  static constexpr int kHeadLanes = D / kEpl;            // lanes holding one head's row
  static constexpr int kRowLanes = next_pow2(kHeadLanes * HPW);  // lanes per row group (the rest of them idle)
  static_assert(HPW == 1 || (HPW == 2 && kHeadLanes * HPW == kRowLanes), "two heads fill a row group exactly");
  static constexpr int kSumLanes = HPW == 1 ? kRowLanes : kHeadLanes;  // lanes one dot product is summed over
  static constexpr int kRows = kWave / kRowLanes;        // slots per wave-wide load
  // tokens per tile: at most 4 loads per lane for K (and for V), 2 with two heads per wave (the same bytes in
  // flight per wave as one head; 4 where two heads' rows take 512 bytes, two rows per load), at most 16 tokens
  static constexpr int kMaxLoads = HPW == 1 || kRows == 2 ? 4 : 2;
  static constexpr int kTileTok = kRows * kMaxLoads < kTile ? kRows * kMaxLoads : kTile;
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
    // codes widened straight to fp32: one conversion per two values (through bf16 pairs it took three)
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float f[4];
      e4m3x4_to_f32x4(w[i], f);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[4 * i + e] = fmaf(p, f[e], acc[4 * i + e]);
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
// The balanced split's ring: two tiles. Measured on MI355X against three: 7B-shaped batch 191.1 -> 189.5 us, its
// E4M3 form 105.4 -> 102.1, the mixed-length batch 614.8 -> 613.9 -- fewer concurrent reads per wave, as in the
// grouped-query kernels, congest the memory system less.
constexpr int kBalStages = 2;

// kAppend: decode with each sequence's new token appended in this launch (one query row per sequence). The wave
// whose partition holds the token's position reads one position less from the pool and adds the token from the
// new rows after its tiles; the first partition's wave of the first query head of each KV head writes it into
// the pools.
template <int KV, int D, bool kAppend>
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
  if (E < 0) return;  // not one of the sequence's query rows: left unwritten
  int t1 = max(t0, min(min(L, t0 + a.partition), E));
  const int g = h / a.group;
  const int r = lane / S::kRowLanes;  // row group
  const int c = lane % S::kRowLanes;  // 16-byte chunk of the head's row
  const bool lane_ok = c < S::kHeadLanes;  // false for the padding lanes of a row group

  // appended decode: this lane's chunk of head g's new K/V row (16 bytes as given, or 32 bytes of bf16 for 16
  // E4M3 codes), loaded unconditionally and first read after the tiles
  constexpr int kNewPieces = S::kEsize == 1 ? 2 : 1;
  U4 nk[kNewPieces], nv[kNewPieces];
  bool attend_new = false, store_new = false;
  int64_t new_slot = 0;
  if constexpr (kAppend) {
    const int64_t src = (((int64_t)s * a.num_kv_heads + g) * D * (kNewPieces == 2 ? 2 : S::kEsize)) / 16 +
                        (lane_ok ? c : 0) * kNewPieces;
#pragma unroll
    for (int e = 0; e < kNewPieces; ++e) {
      nk[e] = static_cast<const U4*>(a.new_key)[src + e];
      nv[e] = static_cast<const U4*>(a.new_value)[src + e];
    }
    const int Lraw = a.context_lens[s];
    new_slot = a.slot_mapping[s];
    if (Lraw >= 1 && new_slot >= 0 && new_slot < (a.num_blocks << a.bs_log2)) {
      store_new = part == 0 && h % a.group == 0;
      attend_new = Lraw <= a.max_context_len && Lraw - 1 >= t0 && Lraw - 1 < t1;  // then Lraw - 1 == t1 - 1
      if (attend_new) --t1;
    }
  }

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

  // appended decode: the new token (exactly as the pool would hold it: quantised for E4M3, by the waves that
  // attend over it or store it), one more position of row group 0
  U4 nkc{}, nvc{};
  if constexpr (kAppend) {
    if constexpr (kNewPieces == 2) {
      if (attend_new || store_new) {
        nkc = e4m3_pack16_bf16<false>(nk[0], nk[1], e4m3_div(a.new_k_scale));
        nvc = e4m3_pack16_bf16<false>(nv[0], nv[1], e4m3_div(a.new_v_scale));
      }
    } else {
      nkc = nk[0];
      nvc = nv[0];
    }
    if (attend_new) {
      float sn = group_sum<S::kRowLanes>(dot_chunk<KV>(q, nkc)) * a.scale_log2;
      if (r != 0) sn = -INFINITY;
      const float m2 = fmaxf(m, sn);
      const float mref2 = m2 == -INFINITY ? 0.f : m2;
      const float alpha2 = fast_exp2(m - mref2);
      const float pn = fast_exp2(sn - mref2);
      l = l * alpha2 + pn;
#pragma unroll
      for (int e = 0; e < S::kEpl; ++e) acc[e] *= alpha2;
      axpy_chunk<KV>(acc, pn, nvc);
      m = m2;
    }
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
  if constexpr (kAppend) {
    if (store_new && r == 0 && lane_ok) {  // the new token into its slot of both pools
      const int64_t dst = new_slot * row_bytes + (int64_t)g * D * S::kEsize + c * 16;
      *reinterpret_cast<U4*>(static_cast<char*>(a.key_out) + dst) = nkc;
      *reinterpret_cast<U4*>(static_cast<char*>(a.value_out) + dst) = nvc;
    }
  }
}

// Merge of split-context partials: with partition p giving running max m_p (log2 units), sum l_p and
// normalised output o_p, out = sum_p w_p o_p / sum_p w_p with w_p = l_p * 2^(m_p - max_p m_p). One wave per
// (query row, head), four heads' waves to a workgroup (both merge kernels: a quarter of the workgroups to launch,
// 7B-shaped balanced merge 4.9 -> 4.3 us): lane p owns partition p's weight, and every lane accumulates its own
// head_dim / 64 dims.
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

// kSpec is the smallest of 4, 8 and 16 that covers the longest row's partitions (16 past that): with the clamped
// indexes a larger kSpec would only repeat the last slot's loads, which for short grids of many rows (several
// new tokens per sequence, a few partitions each) was the bulk of the merge's time.
template <int D, int kSpec>
__global__ __launch_bounds__(kWave * 4) void lse_reduce_kernel(const DecodeArgs a) {
  constexpr int kDpl = (D + kWave - 1) / kWave;  // dims per lane
  constexpr int kActive = D / kDpl;              // lanes holding dims (all of them when 64 divides D)
  static_assert(D % kDpl == 0, "whole dims per lane");
  const int lane = threadIdx.x & (kWave - 1);
  const bool lane_ok = lane < kActive;  // the other lanes read lane 0's dims and store nothing
  const int h = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  if (h >= a.num_q_heads) return;
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
  const int span = a.partition * a.parts_per_wave;  // positions behind one partial: a wave's span
  // a row that is not one of its sequence's query rows was not computed and is not written
  const bool merge = L > span && (!a.query_start || row - a.query_start[s] < rows_of_seq(a, s));
  const int np = merge ? (L + span - 1) / span : 1;

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

// ---------------------------------------------------------------------------------------------------------
// Balanced split. The partition kernel gives each wave one partition of one row, so a batch of unequal
// lengths leaves waves of unequal length: once the short ones finish, part of the chip idles while the
// longest drain. Here the tiles of all query rows, taken in row order, form one list cut into `chunks` equal
// runs of consecutive tiles, one run per (head, wave); the host sizes the grid to one wave per wave slot of
// the chip, so every wave streams the same number of tiles from start to end. A run crosses row boundaries:
// a row lying wholly inside one run is finished there and written to `out`; a row cut by run boundaries leaves
// one partial (max, sum, normalised output) per run it touches, merged by balanced_reduce_kernel with the
// rule of the partition merge. Partial slots: [head][run][2], slot 0 for the row a run starts inside, slot 1
// for the row it ends inside. Loads keep a ring of tiles like the partition kernel's; a row's query
// rides in the ring with the row's first tile of the run.
//
// Every workgroup first derives the rows' extents and the exclusive prefix of their tile counts in LDS
// (rows of one sequence in several-token batches: row j of QL attends over L - QL + j + 1 positions); the
// first workgroup also publishes the prefix for the merge.
// At least two waves per SIMD, which the grid's size assumes (without the bound the E4M3 kernels at head_dim 192
// and 256 would take 256 VGPRs plus 12 AGPRs and one wave per SIMD).
template <int KV, int D, bool kMulti, int HPW, bool kAppend>
__global__ __launch_bounds__(kWave * kWavesPerGroup, 2) void decode_valu_balanced_kernel(const DecodeArgs a) {
  using S = Shape<KV, D, HPW>;
  constexpr int NL = S::kLoads;
  constexpr int TT = S::kTileTok;
  constexpr int NT = kWave * kWavesPerGroup;
  extern __shared__ int32_t lds_rows[];
  __shared__ int32_t wave_total[kWavesPerGroup];
  const int T = a.num_tokens;
  int32_t* __restrict__ P = lds_rows;           // P[r]: tiles of the rows before r; P[T]: all tiles
  int32_t* __restrict__ Ex = lds_rows + T + 1;  // positions row r attends over
  int32_t* __restrict__ Sq = Ex + T;            // sequence of row r (several-token batches only)
  // appended decode (one row per sequence, so Sq is free): Sq[r] = the slot to write row r's new token into, -1
  // for none; Sa[r] = 1 when that token is also the row's last position attended over
  int32_t* __restrict__ Sa = Sq + T;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // extents and tile counts; P[r + 1] holds row r's count until the scan. Rows no sequence claims stay empty.
  for (int r = tid; r < T; r += NT) {
    P[r + 1] = 0;
    Ex[r] = 0;
    if constexpr (kMulti) Sq[r] = 0;
  }
  __syncthreads();
  for (int s = tid; s < a.num_seqs; s += NT) {
    const int L = min(max(a.context_lens[s], 0), a.max_context_len);
    int64_t q0 = s, ql = 1;
    if constexpr (kMulti) {
      q0 = a.query_start[s];
      ql = rows_of_seq(a, s);
    }
    const int64_t jb = q0 < 0 ? -q0 : 0, je = min(ql, (int64_t)T - q0);  // rows inside [0, T) only
    for (int64_t j = jb; j < je; ++j) {
      const int E = (int)max((int64_t)0, min((int64_t)L, L - ql + j + 1));
      Ex[q0 + j] = E;
      P[q0 + j + 1] = (E + TT - 1) / TT;
      if constexpr (kMulti) Sq[q0 + j] = s;
    }
    if constexpr (kAppend) {
      const int raw = a.context_lens[s];
      const int slot = a.slot_mapping[s];
      const bool ok = raw >= 1 && slot >= 0 && (int64_t)slot < (a.num_blocks << a.bs_log2);
      Sq[s] = ok ? slot : -1;
      Sa[s] = ok && raw <= a.max_context_len ? 1 : 0;
    }
  }
  __syncthreads();
  block_exclusive_scan<NT>(P, T, wave_total);
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int r = tid; r <= T; r += NT) a.tile_prefix[r] = P[r];

  const int h0 = (blockIdx.x * kWavesPerGroup + wave) * HPW;  // the wave's first head
  if (h0 >= a.num_q_heads) return;
  const int chunk = blockIdx.y;
  const int total = __builtin_amdgcn_readfirstlane(P[T]);
  const int C = (total + a.chunks - 1) / a.chunks;  // tiles per run
  const int g0 = chunk * C;                          // this wave's run: tiles [g0, g1) of the list
  const int g1 = min(g0 + C, total);
  if (g0 >= g1) return;
  const int n = g1 - g0;

  const int r = lane / S::kRowLanes;
  const int c = lane % S::kRowLanes;
  const int hw = HPW == 1 ? 0 : c / S::kHeadLanes;  // the lane's head within the wave
  const int cc = HPW == 1 ? c : c % S::kHeadLanes;  // its 16-byte chunk of that head's row
  const int h = h0 + hw;
  const bool lane_ok = HPW == 1 ? c < S::kHeadLanes : h < a.num_q_heads;
  const int g = h / a.group;
  const int64_t row_bytes = (int64_t)a.num_kv_heads * D * S::kEsize;
  constexpr uint32_t kNowhere = 0x80000000u;
  uint32_t lane_off[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i)
    lane_off[i] = lane_ok ? (uint32_t)((i * S::kRows + r) * row_bytes + (int64_t)g * D * S::kEsize + cc * 16)
                          : kNowhere;
  constexpr uint32_t kQBytes = D * S::kQEsize;
  uint32_t q_off[S::kQWords];
#pragma unroll
  for (int i = 0; i < S::kQWords; ++i)
    q_off[i] = lane_ok ? (uint32_t)(hw * kQBytes + (cc * S::kQWords + i) * 16) : kNowhere;
  const char* __restrict__ kbase = static_cast<const char*>(a.key_cache);
  const char* __restrict__ vbase = static_cast<const char*>(a.value_cache);
  const char* __restrict__ qbase = static_cast<const char*>(a.query) + (int64_t)h0 * kQBytes;
  const int64_t q_row_bytes = (int64_t)a.num_q_heads * kQBytes;

  // the run's first row: the first r with P[r + 1] > g0
  int lo = 0, hi = T - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (__builtin_amdgcn_readfirstlane(P[mid + 1]) <= g0) lo = mid + 1;
    else hi = mid;
  }
  // the next row holding tiles after `row` (one exists while tiles of the run remain)
  auto next_row = [&](int row) {
    int x = row + 1;
    while (__builtin_amdgcn_readfirstlane(P[x + 1]) == __builtin_amdgcn_readfirstlane(P[x])) ++x;
    return x;
  };
  // What the consumer of a tile needs, packed at issue into one scalar per ring slot: live rows of the tile,
  // whether it opens (takes the row's query) or closes its row segment, whether that segment is the whole row
  // (written to out) or a partial and in which slot, a block id outside the pool, and the query row.
  constexpr uint32_t kRowsMask = 31u, kFirst = 1u << 5, kLast = 1u << 6, kWhole = 1u << 7, kSlot1 = 1u << 8,
                     kBad = 1u << 9, kNew = 1u << 10, kNewAttend = 1u << 11;
  constexpr int kRowShift = 12;
  auto table_of = [&](int row) {
    const int s = kMulti ? __builtin_amdgcn_readfirstlane(Sq[row]) : row;
    return as_constant(a.block_tables) + (int64_t)s * a.max_blocks_per_seq;
  };

  // Appended decode: sequence s's new token is its last position L - 1. It is not read from the pool (the same
  // launch writes it there) but from the new rows, once, after the row's last tile, and the wave that reaches that
  // tile writes it into the pools at its slot. A slot outside the pool is skipped, as the cache write skips it
  // (the pool is then read as it was); a length beyond max_context_len clamps the positions attended over, so
  // the token is written but not attended to, as the two separate calls would do. The returned value is the
  // slot to write (-1: none); `attend` says whether the token is also the row's last position. Both come from
  // the prologue's LDS arrays (global loads at every row switch would stall the next tile's issue).
  auto new_slot_of = [&](int row, bool& attend) {
    if constexpr (!kAppend) {
      attend = false;
      return -1;
    } else {
      attend = __builtin_amdgcn_readfirstlane(Sa[row]) != 0;
      return __builtin_amdgcn_readfirstlane(Sq[row]);
    }
  };

  // issue cursor: row, tile within the row, the row's first tile in the list and tile count, extent, table
  int i_row = lo;
  int i_p0 = __builtin_amdgcn_readfirstlane(P[i_row]);
  int i_nt = __builtin_amdgcn_readfirstlane(P[i_row + 1]) - i_p0;
  int i_ext = __builtin_amdgcn_readfirstlane(Ex[i_row]);
  int i_tile = g0 - i_p0;
  const ConstI32* i_table = table_of(i_row);
  bool i_attend;
  int i_slot = new_slot_of(i_row, i_attend);

  Words<S::kQWords> q;
  float m = -INFINITY, l = 0.f;
  float acc[S::kEpl];
#pragma unroll
  for (int e = 0; e < S::kEpl; ++e) acc[e] = 0.f;
  bool seg_bad = false;

  U4 kb[kBalStages][NL], vb[kBalStages][NL];
  Words<S::kQWords> qb[kBalStages];
  uint32_t info[kBalStages];
  // appended decode: the new token's K/V chunk, as given (row group 0's lanes) or, for an E4M3 cache, as the 32
  // bytes of bf16 that its 16 codes are quantised from, the first half in row group 0's lanes and the second in
  // row group 1's (one 16-byte load per lane, as for the other dtypes)
  constexpr bool kQuantNew = S::kEsize == 1;
  static_assert(!kQuantNew || S::kRows >= 2, "an E4M3 row's new token takes two row groups");
  U4 kn[kBalStages], vn[kBalStages];
  int nslot[kBalStages];
  const char* __restrict__ nkbase = static_cast<const char*>(a.new_key);
  const char* __restrict__ nvbase = static_cast<const char*>(a.new_value);
  constexpr bool kHalves = TT == kTile && S::kRows <= kTile / 2;
  auto issue = [&](U4* kq, U4* vq, Words<S::kQWords>& qq, uint32_t& tinfo, U4& kq_new, U4& vq_new, int& slot_new,
                   int jj) {
    const bool live = jj < n;
    const int t = i_tile * TT;
    bool bad = false;
    const int last8 = (i_ext - 1) & ~(kTile / 2 - 1);
    const int64_t base0 = tile_slot_bytes(i_table, t, a.bs_log2, a.num_blocks, row_bytes, bad);
    const int64_t base1 = !kHalves ? base0
                          : a.bs_log2 == 3
                              ? tile_slot_bytes(i_table, min(t + kTile / 2, last8), a.bs_log2, a.num_blocks,
                                                row_bytes, bad)
                              : base0 + (kTile / 2) * row_bytes;
    // appended decode: the row's last tile loads the new token from the new rows (row group 0's lanes, and for
    // an E4M3 cache row group 1's, one 16-byte chunk each; the others read nothing) and, when the token is that
    // tile's last position, reads one row less from the pool
    const bool newtok = kAppend && live && i_tile == i_nt - 1 && i_slot >= 0;
    const bool attend_new = newtok && i_attend;
    // (taken through a scalar register: the descriptors below must stay wave-uniform)
    const int rows = __builtin_amdgcn_readfirstlane(live ? min(TT, i_ext - t) - (attend_new ? 1 : 0) : 0);
    if constexpr (kAppend) {
      // issued for every tile (an empty descriptor reads nothing), so that the loads in flight are the same on
      // every path and the waits for a tile's K/V stay as tight as without the append
      // (bf16 rows of an E4M3 cache take twice the bytes of the pool's rows, at twice the offsets)
      constexpr int kW = kQuantNew ? 2 : 1;
      const uint32_t noff = !lane_ok || r >= kW ? kNowhere : (lane_off[0] - (uint32_t)(r * row_bytes)) * kW + 16 * r;
      const uint32_t nbytes = newtok ? (uint32_t)(row_bytes * kW) : 0u;
      kq_new = load16<0>(make_rsrc(nkbase + (int64_t)i_row * row_bytes * kW, nbytes), noff);
      vq_new = load16<0>(make_rsrc(nvbase + (int64_t)i_row * row_bytes * kW, nbytes), noff);
      slot_new = i_slot;
    }
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
    // the row's query, with its first tile of the run (an empty descriptor otherwise: zeros, no access)
    const bool first = i_tile == 0 || jj == 0;
    const __amdgpu_buffer_rsrc_t qr =
        make_rsrc(qbase + (int64_t)i_row * q_row_bytes, live && first ? kQBytes * HPW : 0u);
#pragma unroll
    for (int i = 0; i < S::kQWords; ++i) qq.w[i] = load16<0>(qr, q_off[i]);
    tinfo = (uint32_t)rows | (first ? kFirst : 0u) | (i_tile == i_nt - 1 || jj == n - 1 ? kLast : 0u) |
            (i_p0 >= g0 && i_p0 + i_nt <= g1 ? kWhole : 0u) | (i_p0 > g0 ? kSlot1 : 0u) | (bad ? kBad : 0u) |
            (newtok ? kNew : 0u) | (attend_new ? kNewAttend : 0u) | ((uint32_t)i_row << kRowShift);
    if (live && jj + 1 < n && ++i_tile == i_nt) {
      i_row = next_row(i_row);
      i_p0 = __builtin_amdgcn_readfirstlane(P[i_row]);
      i_nt = __builtin_amdgcn_readfirstlane(P[i_row + 1]) - i_p0;
      i_ext = __builtin_amdgcn_readfirstlane(Ex[i_row]);
      i_table = table_of(i_row);
      i_slot = new_slot_of(i_row, i_attend);
      i_tile = 0;
    }
  };

  // finish the current row segment: merge the row groups, write the row or its partial, reset the state
  auto flush = [&](uint32_t tinfo) {
#pragma unroll
    for (int off = S::kRowLanes; off < kWave; off <<= 1) {
      const float mo = __shfl_xor(m, off);
      const float lo2 = __shfl_xor(l, off);
      const float M = fmaxf(m, mo);
      const float Mr = M == -INFINITY ? 0.f : M;
      const float fa = fast_exp2(m - Mr), fb = fast_exp2(mo - Mr);
      l = l * fa + lo2 * fb;
#pragma unroll
      for (int e = 0; e < S::kEpl; ++e) acc[e] = acc[e] * fa + __shfl_xor(acc[e], off) * fb;
      m = M;
    }
    if (r == 0 && lane_ok) {
      const float inv = l > 0.f ? a.v_scale / l : 0.f;
      const float poison = __uint_as_float(0x7fc00000u);
      float* dst;
      if (tinfo & kWhole) {
        dst = a.out + ((int64_t)(tinfo >> kRowShift) * a.num_q_heads + h) * D + cc * S::kEpl;
      } else {
        const int64_t wrow = ((int64_t)h * a.chunks + chunk) * 2 + (tinfo & kSlot1 ? 1 : 0);
        dst = a.ws_o + wrow * D + cc * S::kEpl;
        if (cc == 0) {
          a.ws_ml[2 * wrow] = seg_bad ? poison : m;
          a.ws_ml[2 * wrow + 1] = l;
        }
      }
#pragma unroll
      for (int e = 0; e < S::kEpl; e += 4)
        *reinterpret_cast<float4*>(dst + e) =
            seg_bad ? make_float4(poison, poison, poison, poison)
                    : make_float4(acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv);
    }
    m = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int e = 0; e < S::kEpl; ++e) acc[e] = 0.f;
    seg_bad = false;
  };

  // the new token's 16 bytes as the pool holds them, in row group 0's lanes (E4M3: quantised exactly as the
  // quantising cache write does, from the two halves; called by the whole wave)
  auto new_piece = [&](const U4& mine, float scale) __attribute__((always_inline)) {
    if constexpr (kQuantNew) {
      const U4 hi{(uint32_t)__shfl_down((int)mine.x, S::kRowLanes), (uint32_t)__shfl_down((int)mine.y, S::kRowLanes),
                  (uint32_t)__shfl_down((int)mine.z, S::kRowLanes), (uint32_t)__shfl_down((int)mine.w, S::kRowLanes)};
      return e4m3_pack16_bf16<false>(mine, hi, e4m3_div(scale));
    } else {
      return mine;
    }
  };
  auto consume = [&](const U4* kq, const U4* vq, const Words<S::kQWords>& qq, uint32_t tinfo, const U4& kq_new,
                     const U4& vq_new, int slot_new) {
    tinfo = __builtin_amdgcn_readfirstlane(tinfo);
    if (tinfo & kFirst) q = qq;
    seg_bad |= (tinfo & kBad) != 0;
    const int rows = (int)(tinfo & kRowsMask);
    const bool full = rows == TT;
    float sc[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      sc[i] = group_sum<S::kSumLanes>(dot_chunk<KV>(q, kq[i])) * a.scale_log2;
      if (!full && i * S::kRows + r >= rows) sc[i] = -INFINITY;
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
      if (!full && i * S::kRows + r >= rows) v = U4{0u, 0u, 0u, 0u};
      axpy_chunk<KV>(acc, p, v);
    }
    m = mn;
    if constexpr (kAppend) {
      if (tinfo & kNew) {
        // (a token attended over is always one that is written: its pieces are formed once, for both)
        const U4 kp = new_piece(kq_new, a.new_k_scale), vp = new_piece(vq_new, a.new_v_scale);
        if (tinfo & kNewAttend) {
          // the new token, one more position of row group 0 (the other groups' state does not move)
          float sn = group_sum<S::kSumLanes>(dot_chunk<KV>(q, kp)) * a.scale_log2;
          if (r != 0) sn = -INFINITY;
          const float m2 = fmaxf(m, sn);
          const float mref2 = m2 == -INFINITY ? 0.f : m2;
          const float alpha2 = fast_exp2(m - mref2);
          const float pn = fast_exp2(sn - mref2);
          l = l * alpha2 + pn;
#pragma unroll
          for (int e = 0; e < S::kEpl; ++e) acc[e] *= alpha2;
          axpy_chunk<KV>(acc, pn, vp);
          m = m2;
        }
        // its rows into the pools, by one wave per KV head
        if (r == 0 && lane_ok && h % a.group == 0) {
          const int64_t dst = (int64_t)slot_new * row_bytes + lane_off[0];
          *reinterpret_cast<U4*>(static_cast<char*>(a.key_out) + dst) = kp;
          *reinterpret_cast<U4*>(static_cast<char*>(a.value_out) + dst) = vp;
        }
      }
    }
    if (tinfo & kLast) flush(tinfo);
  };

#pragma unroll
  for (int i = 0; i < kBalStages - 1; ++i) issue(kb[i], vb[i], qb[i], info[i], kn[i], vn[i], nslot[i], i);
  int j = 0;
  for (; j + kBalStages <= n; j += kBalStages) {
#pragma unroll
    for (int i = 0; i < kBalStages; ++i) {
      const int w = (i + kBalStages - 1) % kBalStages;
      issue(kb[w], vb[w], qb[w], info[w], kn[w], vn[w], nslot[w], j + i + kBalStages - 1);
      consume(kb[i], vb[i], qb[i], info[i], kn[i], vn[i], nslot[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < kBalStages - 1; ++i)
    if (j + i < n) consume(kb[i], vb[i], qb[i], info[i], kn[i], vn[i], nslot[i]);
}

// Merge of the balanced split's partials: one wave per (query row, head). The tile list holds query rows, or
// sequences on the matrix-core kernel (seq_prefix), whose partials then carry the row's index qi within its
// sequence. A row whose list item lies in one run was written by the decode kernel; an item with no tile
// attends over nothing and its rows get a zero row here; an item spanning runs c0 .. c1 has the partial of run
// c0 on side 1 (side 0 when it starts exactly at c0's first tile) and those of runs c0 + 1 .. c1 on side 0.
template <int D>
__global__ __launch_bounds__(kWave * 4) void balanced_reduce_kernel(const DecodeArgs a) {
  constexpr int kDpl = (D + kWave - 1) / kWave;
  constexpr int kActive = D / kDpl;
  const int lane = threadIdx.x & (kWave - 1);
  const bool lane_ok = lane < kActive;
  const int h = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  if (h >= a.num_q_heads) return;
  const int row = blockIdx.y;
  // sizes taken as values (a select between two fields of the argument block went through scratch memory)
  const bool by_seq = a.seq_prefix != 0;
  const int items = __builtin_amdgcn_readfirstlane(by_seq ? a.num_seqs : a.num_tokens);
  const int ql = by_seq ? __builtin_amdgcn_readfirstlane(a.max_query_len) : 1;
  int item = row, qi = 0;
  if (a.query_start) {
    const int s = seq_of_row(a, row);
    const int q0 = a.query_start[s];
    if (row - q0 >= rows_of_seq(a, s)) return;  // not one of the sequence's query rows: left unwritten
    if (by_seq) {
      item = s;
      qi = row - q0;
    }
  }
  const int p0 = a.tile_prefix[item], p1 = a.tile_prefix[item + 1], total = a.tile_prefix[items];
  float* dst = a.out + ((int64_t)row * a.num_q_heads + h) * D + (lane_ok ? lane : 0) * kDpl;
  if (p1 <= p0) {
    if (lane_ok)
#pragma unroll
      for (int e = 0; e < kDpl; ++e) dst[e] = 0.f;
    return;
  }
  const int C = (total + a.chunks - 1) / a.chunks;
  const int c0 = p0 / C, c1 = (p1 - 1) / C;
  if (c0 == c1) return;
  const int np = c1 - c0 + 1;
  const int64_t base = ((int64_t)h * a.chunks + c0) * 2;
  const int64_t first = base + (p0 != c0 * C ? 1 : 0);
  const float2* __restrict__ ml = reinterpret_cast<const float2*>(a.ws_ml);
  const float* __restrict__ o = a.ws_o + (lane_ok ? lane : 0) * kDpl;
  auto slot = [&](int k) { return (k == 0 ? first : base + 2 * (int64_t)k) * ql + qi; };

  float M = -INFINITY;
  for (int k = lane; k < np; k += kWave) M = fmaxf(M, ml[slot(k)].x);
  M = wave_max(M);
  const float Mr = M == -INFINITY ? 0.f : M;
  float acc[kDpl];
#pragma unroll
  for (int e = 0; e < kDpl; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  for (int k0 = 0; k0 < np; k0 += kWave) {
    float w = 0.f;
    if (k0 + lane < np) {
      const float2 v = ml[slot(k0 + lane)];
      w = v.y * fast_exp2(v.x - Mr);
    }
    wsum += w;
    const int cnt = min(kWave, np - k0);
    for (int k = 0; k < cnt; ++k) {
      const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), k));
      const float* __restrict__ op = o + slot(k0 + k) * D;
#pragma unroll
      for (int e = 0; e < kDpl; ++e) acc[e] = fmaf(wk, op[e], acc[e]);
    }
  }
  const float wtot = wave_sum(wsum);
  const float inv = wtot > 0.f ? 1.0f / wtot : 0.f;
  if (!lane_ok) return;
#pragma unroll
  for (int e = 0; e < kDpl; ++e) dst[e] = acc[e] * inv;
}

}  // namespace

template <int KV, bool kAppend>
hipError_t launch_kv_append(const DecodeArgs& a, dim3 grid, dim3 block, hipStream_t stream) {
  switch (a.head_dim) {
    case 64: decode_valu_kernel<KV, 64, kAppend><<<grid, block, 0, stream>>>(a); break;
    case 80: decode_valu_kernel<KV, 80, kAppend><<<grid, block, 0, stream>>>(a); break;
    case 96: decode_valu_kernel<KV, 96, kAppend><<<grid, block, 0, stream>>>(a); break;
    case 112: decode_valu_kernel<KV, 112, kAppend><<<grid, block, 0, stream>>>(a); break;
    case 128: decode_valu_kernel<KV, 128, kAppend><<<grid, block, 0, stream>>>(a); break;
    case 192: decode_valu_kernel<KV, 192, kAppend><<<grid, block, 0, stream>>>(a); break;
    case 256: decode_valu_kernel<KV, 256, kAppend><<<grid, block, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int KV>
hipError_t launch_kv(const DecodeArgs& a, dim3 grid, dim3 block, hipStream_t stream) {
  if (!a.new_key) return launch_kv_append<KV, false>(a, grid, block, stream);
  if (a.query_start) return hipErrorInvalidValue;  // appended decode: one new token (query row) per sequence
  return launch_kv_append<KV, true>(a, grid, block, stream);
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

template <int KV, bool kMulti, bool kAppend>
hipError_t launch_balanced_kv(const DecodeArgs& a, int hpw, dim3 grid, dim3 block, size_t lds, hipStream_t stream) {
  switch (a.head_dim) {
    case 64:
      if constexpr (KV != PA_F32)
        if (hpw == 2) {
          decode_valu_balanced_kernel<KV, 64, kMulti, 2, kAppend><<<grid, block, lds, stream>>>(a);
          break;
        }
      decode_valu_balanced_kernel<KV, 64, kMulti, 1, kAppend><<<grid, block, lds, stream>>>(a);
      break;
    case 80: decode_valu_balanced_kernel<KV, 80, kMulti, 1, kAppend><<<grid, block, lds, stream>>>(a); break;
    case 96: decode_valu_balanced_kernel<KV, 96, kMulti, 1, kAppend><<<grid, block, lds, stream>>>(a); break;
    case 112: decode_valu_balanced_kernel<KV, 112, kMulti, 1, kAppend><<<grid, block, lds, stream>>>(a); break;
    case 128:
      if constexpr (KV != PA_F32)
        if (hpw == 2) {
          decode_valu_balanced_kernel<KV, 128, kMulti, 2, kAppend><<<grid, block, lds, stream>>>(a);
          break;
        }
      decode_valu_balanced_kernel<KV, 128, kMulti, 1, kAppend><<<grid, block, lds, stream>>>(a);
      break;
    case 192: decode_valu_balanced_kernel<KV, 192, kMulti, 1, kAppend><<<grid, block, lds, stream>>>(a); break;
    case 256: decode_valu_balanced_kernel<KV, 256, kMulti, 1, kAppend><<<grid, block, lds, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int KV>
hipError_t launch_balanced_dtype(const DecodeArgs& a, int hpw, dim3 grid, dim3 block, hipStream_t stream) {
  const bool multi = a.query_start != nullptr;
  const size_t lds = (size_t)((multi ? 3 : a.new_key ? 4 : 2) * (int64_t)a.num_tokens + 1) * sizeof(int32_t);
  if (a.new_key) {  // appended decode: one new token per sequence (rows in the cache's dtype, bf16 for E4M3)
    if (multi) return hipErrorInvalidValue;
    return launch_balanced_kv<KV, false, true>(a, hpw, grid, block, lds, stream);
  }
  return multi ? launch_balanced_kv<KV, true, false>(a, hpw, grid, block, lds, stream)
               : launch_balanced_kv<KV, false, false>(a, hpw, grid, block, lds, stream);
}

int valu_heads_per_wave(int kv_dtype, int head_dim, int group) {
  const int row_bytes = head_dim * (kv_dtype == PA_F32 ? 4 : kv_dtype == PA_BF16 ? 2 : 1);
  return group == 1 && (row_bytes == 64 || row_bytes == 128 || (row_bytes == 256 && kv_dtype == PA_BF16)) ? 2 : 1;
}

int32_t balanced_chunks(int32_t num_q_heads, int32_t heads_per_wave) {
  const int32_t waves = (num_q_heads + heads_per_wave - 1) / heads_per_wave;
  const int32_t groups = (waves + kWavesPerGroup - 1) / kWavesPerGroup;
  return groups >= kResidentWaves / kWavesPerGroup ? 1 : kResidentWaves / kWavesPerGroup / groups;
}

hipError_t launch_decode_valu_balanced(const DecodeArgs& a, int kv_dtype, hipStream_t stream) {
  if (a.num_tokens > kMaxBalancedRows || a.chunks <= 0 || !a.tile_prefix) return hipErrorInvalidValue;
  const int hpw = valu_heads_per_wave(kv_dtype, a.head_dim, a.group);
  const int waves = (a.num_q_heads + hpw - 1) / hpw;
  const dim3 grid((waves + kWavesPerGroup - 1) / kWavesPerGroup, a.chunks, 1);
  const dim3 block(kWave * kWavesPerGroup);
  if (kv_dtype == PA_BF16) return launch_balanced_dtype<PA_BF16>(a, hpw, grid, block, stream);
  if (kv_dtype == PA_F32) return launch_balanced_dtype<PA_F32>(a, hpw, grid, block, stream);
  if (kv_dtype == PA_FP8_E4M3) return launch_balanced_dtype<PA_FP8_E4M3>(a, hpw, grid, block, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_balanced_reduce(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid((a.num_q_heads + 3) / 4, a.num_tokens);
  const dim3 block(kWave * 4);
  switch (a.head_dim) {
    case 64: balanced_reduce_kernel<64><<<grid, block, 0, stream>>>(a); break;
    case 80: balanced_reduce_kernel<80><<<grid, block, 0, stream>>>(a); break;
    case 96: balanced_reduce_kernel<96><<<grid, block, 0, stream>>>(a); break;
    case 112: balanced_reduce_kernel<112><<<grid, block, 0, stream>>>(a); break;
    case 128: balanced_reduce_kernel<128><<<grid, block, 0, stream>>>(a); break;
    case 192: balanced_reduce_kernel<192><<<grid, block, 0, stream>>>(a); break;
    case 256: balanced_reduce_kernel<256><<<grid, block, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int kSpec>
hipError_t launch_lse_reduce_spec(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid((a.num_q_heads + 3) / 4, a.num_tokens);
  const dim3 block(kWave * 4);
  switch (a.head_dim) {
    case 64: lse_reduce_kernel<64, kSpec><<<grid, block, 0, stream>>>(a); break;
    case 80: lse_reduce_kernel<80, kSpec><<<grid, block, 0, stream>>>(a); break;
    case 96: lse_reduce_kernel<96, kSpec><<<grid, block, 0, stream>>>(a); break;
    case 112: lse_reduce_kernel<112, kSpec><<<grid, block, 0, stream>>>(a); break;
    case 128: lse_reduce_kernel<128, kSpec><<<grid, block, 0, stream>>>(a); break;
    case 192: lse_reduce_kernel<192, kSpec><<<grid, block, 0, stream>>>(a); break;
    case 256: lse_reduce_kernel<256, kSpec><<<grid, block, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_lse_reduce(const DecodeArgs& a, hipStream_t stream) {
  if (a.max_partitions <= 4) return launch_lse_reduce_spec<4>(a, stream);
  if (a.max_partitions <= 8) return launch_lse_reduce_spec<8>(a, stream);
  return launch_lse_reduce_spec<16>(a, stream);
}

}  // namespace pa
