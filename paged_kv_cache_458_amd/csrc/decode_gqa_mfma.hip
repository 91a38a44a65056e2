// Grouped-query paged decode on the MFMA units of gfx950: one wave64 per (sequence, KV head, partition).
//
// When G = num_q_heads / num_kv_heads query heads share one KV head, every K/V row read from HBM serves G
// dot products and G axpys; at G = 8 that would keep the vector ALUs busier than the memory system, so the
// two products run as small dense contractions on v_mfma_f32_16x16x32_bf16 (bf16 inputs, fp32 accumulate):
//
//   S^T[32 tokens x 16]  = K_tile[32 x D] . Q^T[D x 16]      (the G heads padded to 16 columns)
//   O^T[D x 16]         += V_tile^T[D x 32] . (P_hi + P_lo)^T[32 x 16]
//
// The probabilities enter as two bf16 operands, P_hi = bf16(P) and P_lo = bf16(P - P_hi), so the second
// product keeps about 16 significant bits of every weight (V is exact in bf16); the extra MFMAs are free in a
// kernel bound by its loads.
//
// The same columns serve sequences that bring several new tokens (speculative verification, a prompt chunk):
// G heads x QL rows, each column with its own causal limit, so K/V are still read once per (sequence, KV
// head) however many of its tokens attend. Without grouping (G = 1) the columns are the QL rows alone. More
// than 16 columns run as column groups of 16 in waves of their own, each reading the K/V again.
//
// Loads. K and V rows are read from the pool with every wave-wide load covering kRows whole head rows (256
// bytes of bf16 at D = 128: full cache lines, non-temporal, each row is read once per call); both go through a
// per-wave LDS slice (rows padded by 16 bytes). Loading K straight into the MFMA operand layout instead (16 rows x 64 bytes per
// load, each line split across two loads) costs about 12% of bandwidth with non-temporal loads.
//
// Operand layouts. K rows are the A operand of the first product: lane (n, j) = (lane % 16, lane / 16) reads
// row n, elements 32c + 8j .. 32c + 8j + 7 of each 16-row half from LDS. The result leaves lane (n, j) with the scores of head n
// for tokens 4j..4j+3 of both halves; those eight probabilities are exactly that lane's B operands of the
// second product once the contraction index k = 8j + e is mapped to token (e < 4 ? 4j + e : 16 + 4j + e - 4)
// -- no data moves between lanes. V^T needs eight tokens of one dim per lane, the transpose of the pool's
// layout: gfx950's transposing LDS reads give it with two 8-byte reads per 16-dim column tile. The
// accumulator of the second product leaves lane (n, j) with head n, the same head as its softmax state, so
// the online-softmax rescale is a per-lane multiply, skipped for the whole wave once no maximum moves. A
// head's tile maximum spans the wave's four 16-lane rows and is taken with gfx950's row swaps, in registers;
// positions past the range are masked only in a tile that holds some; weights become bf16 pairs through
// packed conversions.
//
// A tile's loads land in one register set and are staged into LDS; the next tile's loads are then issued into the
// same registers while the staged tile goes through the products. Block ids come from scalar loads of the block table (one per 16-token half, one per 8-token quarter with 8-slot blocks). Scores use the exp2 domain (scale * log2 e folded in).
//
// An FP8 (OCP E4M3) cache is read at one byte per element and staged into LDS as it is; its operands are
// widened to bf16 after the LDS reads (every E4M3 value is exactly a bf16 value): K through 8-byte reads, V^T
// through gfx950's 8-bit transposing read, one per 16-dim column tile. Staging the widened values instead
// (32 bytes per lane and load) stepped the lanes of each LDS write 32 bytes apart, with bank conflicts on every
// write. The cache's scales enter as k_scale folded into the score scale and v_scale into the final
// normalisation.
#include "pa_device.h"
#include "pa_kernels.h"
#include "../../include/pa.h"

namespace pa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kTileTok = 32;   // tokens per tile: two 16-row halves

__device__ __forceinline__ f32x4 mfma(const U4& a, const U4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 8-byte transposing LDS read (gfx950 ds_read_b64_tr_b16).
__device__ __forceinline__ u32x2 lds_read_tr16(const char* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

typedef int i32x2 __attribute__((ext_vector_type(2)));

// 8-byte transposing LDS read of 8-bit elements (gfx950 ds_read_b64_tr_b8). Within each 16-lane group, lane l
// receives element l % 8 of the 8-byte rows addressed by lanes (l % 16) / 8 + 2e, e = 0..7, in order of e
// (checked on the device with an in-bounds probe).
__device__ __forceinline__ u32x2 lds_read_tr8(const char* p) {
  typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
  const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Maximum over lanes n, n + 16, n + 32 and n + 48, in registers (no LDS round trip). gfx950's row swaps with
// both operands holding x: the 16-lane swap returns (rows 0, 0, 2, 2) and (rows 1, 1, 3, 3) of x, the 32-lane
// swap (low half twice) and (high half twice) (checked on the device with an in-bounds probe).
__device__ __forceinline__ float max_over_rows(float x) {
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

// 8 E4M3 codes (first in the lowest byte) -> 8 bf16 values, exactly
__device__ __forceinline__ U4 widen8(const u32x2& c) {
  U4 r;
  e4m3x4_to_bf16x4(c.x, r.x, r.y);
  e4m3x4_to_bf16x4(c.y, r.z, r.w);
  return r;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to bf16 (nearest even) in one word, the first in the low half: one packed conversion.
__device__ __forceinline__ uint32_t bf16x2_bits(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// A lane's eight probabilities exp2(sv[e] - mref) as the B operands of the P.V product, each weight split into
// a bf16 pair p = hi + lo (lo rounds the exact fp32 remainder), so the two products together carry about 16
// significant bits of every weight. With one bf16 rounding alone (8 bits), a context of a few tokens, where
// one or two weights dominate, moves outputs by up to a few 1e-3. `psum` adds the fp32 weights.
__device__ __forceinline__ void prob_operands(const float* sv, float mref, U4& hi, U4& lo, float& psum) {
  uint32_t h[4], r[4];
  psum = 0.f;
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const float x0 = fast_exp2(sv[e] - mref), x1 = fast_exp2(sv[e + 1] - mref);
    const uint32_t hw = bf16x2_bits(x0, x1);
    psum += x0 + x1;
    h[e / 2] = hw;
    r[e / 2] = bf16x2_bits(x0 - __uint_as_float(hw << 16), x1 - __uint_as_float(hw & 0xffff0000u));
  }
  hi = U4{h[0], h[1], h[2], h[3]};
  lo = U4{r[0], r[1], r[2], r[3]};
}

constexpr int pow2_ceil(int v) { return v <= 1 ? 1 : 2 * pow2_ceil((v + 1) / 2); }

// Geometry of the K/V tiles of both grouped-query kernels (bf16 or E4M3 cache, head_dim D: 64, 80, 96, 112, 128,
// 192 or 256).
template <int KV, int D>
struct GqaShape {
  static constexpr int kEsize = KV == PA_BF16 ? 2 : 1;  // bytes per cached element
  static constexpr int kDP = (D + 31) / 32 * 32;        // dims of the QK product, zero-padded to 32-dim k-chunks
  static constexpr int kChunks = kDP / 32;              // 32-dim k-chunks of the QK product
  static constexpr int kNt = D / 16;                    // 16-dim column tiles of the PV product
  // E4M3 codes are staged as they are and widened to bf16 after the LDS reads
  static constexpr bool kRaw = KV != PA_BF16;
  static constexpr int kPitch = kDP * (kRaw ? 1 : 2) + 16;  // LDS bytes per K or V row, padded by 16
  static constexpr int kSlice = kTileTok * kPitch;          // one 32-row tile of K or of V
  static constexpr int kHeadLanes = D * kEsize / 16;        // 16-byte pieces of one head row
  // lanes per head row with 16-byte loads, a power of two; the lanes past the row's pieces load nothing, and those
  // inside the padded dims store the zeros they read there
  static constexpr int kRowLanes = pow2_ceil(kHeadLanes);
  static constexpr int kStageLanes = kDP * (kRaw ? 1 : 2) / 16;  // lanes whose 16 bytes lie in the staged row
  static constexpr int kRows = kWave / kRowLanes;               // rows per wave-wide load
  static constexpr int kLoads = kTile / kRows;                  // loads per 16-row half, for K and for V
  // bf16 head rows over 256 bytes: K and V take turns through one register set and one LDS slice (two slices of
  // 32 rows of such rows would not fit 8 waves in a CU's LDS, nor two register sets in the register file)
  static constexpr bool kPhased = !kRaw && D > 128;
  static constexpr int kSlices = kPhased ? 1 : 2;
  // a wave may cover two consecutive partitions only at head_dim <= 128 (registers for the parked state)
  static constexpr bool kTwoParts = D <= 128;
  // a load of at most 8 rows stays inside one 8-row quarter; 16-row loads (E4M3 at head_dim 64) take a whole
  // half through the even quarter's descriptor (the host refuses 8-slot blocks for them)
  static constexpr int kQuarterRows = kRows <= kTile / 2 ? kTile / 2 : kTile;
  static_assert(kLoads * kRows == kTile, "whole rows per load");

  // Where lane (n, j) = (lane % 16, lane / 16) reads its operands in a tile's LDS slices. K, the A operand of
  // S^T = K Q^T: row n, elements 32c + 8j .. 32c + 8j + 7 (plus c * 64 bytes of bf16 or c * 32 of codes).
  static __device__ __forceinline__ const char* k_read(const char* kslice, int n, int j) {
    return kslice + n * kPitch + j * (kRaw ? 8 : 16);
  }
  // V^T, the A operand of O^T += V^T P^T, for contraction index k = 8j + e -> token (e < 4 ? 4j + e : 16 + 4j +
  // e - 4). bf16: two 16-bit transposing reads per 16-dim column tile; within each 16-lane group, lane l
  // receives element l % 4 of the 8-byte rows addressed by lanes (l % 16) / 4 + 4e, e = 0..3, so lane
  // (q, r) = (n / 4, n % 4) addresses token row 4j + q at dims 16nt + 4r .. + 3 and ends up with its own dim
  // 16nt + n of the four token rows. E4M3: one 8-bit transposing read; lane n addresses token e = n / 2 at dims
  // 16nt + 8 (n % 2) .. + 7 and receives dim 16nt + n of the eight tokens in order.
  static __device__ __forceinline__ const char* v_read(const char* vslice, int n, int j) {
    if constexpr (kRaw) {
      const int e = n >> 1;
      return vslice + (e < 4 ? 4 * j + e : kTile + 4 * j + e - 4) * kPitch + 8 * (n & 1);
    } else {
      return vslice + (4 * j + (n >> 2)) * kPitch + 8 * (n & 3);
    }
  }
};

// Loads of one 32-token tile's K (LK) and/or V (LV) into register sets. `t` is the tile's first position, clamped to the last live
// tile (table entries are read at live positions only); `t_live` is the unclamped one. Each 8-row quarter goes
// through a descriptor covering only its rows below `u1`: the rest read as zero without touching memory.
// Quarters of one 16-row half share a block unless blocks hold 8 slots. `last8` is the start of the last live
// 8-row group.
template <int KV, int D, bool LK, bool LV, int NL, typename TablePtr>
__device__ __forceinline__ void gqa_issue(U4 (*kb)[NL], U4 (*vb)[NL], TablePtr table, int t, int t_live, int u1,
                                          int last8, const DecodeArgs& a, int64_t row_bytes, const char* kbase,
                                          const char* vbase, const uint32_t* off, bool& bad) {
  using S = GqaShape<KV, D>;
  static_assert(NL == S::kLoads, "register sets of the tile's shape");
  // each half's first slot; with blocks of 32 slots or more the tile lies in one block, and the second half is
  // an offset from the first (one table read per tile: 70B-shaped E4M3 batch 72.9-73.1 -> 71.5-71.7 us)
  int64_t half_base[2];
  half_base[0] = tile_slot_bytes(table, min(t, last8), a.bs_log2, a.num_blocks, row_bytes, bad);
  half_base[1] = a.bs_log2 >= 5 ? half_base[0] + kTile * row_bytes
                                : tile_slot_bytes(table, min(t + kTile, last8), a.bs_log2, a.num_blocks, row_bytes, bad);
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const int h2 = q4 >> 1;
    const int64_t base = (q4 & 1) == 0 ? half_base[h2]
                         : a.bs_log2 == 3 ? tile_slot_bytes(table, min(t + q4 * (kTile / 2), last8), a.bs_log2,
                                                            a.num_blocks, row_bytes, bad)
                                          : half_base[h2] + (kTile / 2) * row_bytes;
    const int rows = min(S::kQuarterRows, u1 - (t_live + q4 * (kTile / 2)));
    const uint32_t live = rows > 0 ? (uint32_t)rows * (uint32_t)row_bytes : 0u;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kbase + base, live);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vbase + base, live);
    const uint32_t qoff = (uint32_t)((q4 & 1) * (kTile / 2) * row_bytes);
#pragma unroll
    for (int i = 0; i < S::kLoads; ++i) {
      if ((S::kRows * i < kTile / 2) == ((q4 & 1) == 0)) {
        if constexpr (LK) kb[h2][i] = load16<kPolStream>(kr, off[i] - qoff);
        if constexpr (LV) vb[h2][i] = load16<kPolStream>(vr, off[i] - qoff);
      }
    }
  }
}

// Stage one tile of K or V from the load registers into an LDS slice (rows past the range end were loaded as
// zeros); this is where the wave waits for those loads. Lanes past the padded row store nothing. The caller
// orders it against the slice's reads (wave_lds_sync before and after).
template <int KV, int D, int NL>
__device__ __forceinline__ void gqa_stage(const U4 (*rb)[NL], char* slice, int wofs, bool stage_lane) {
  using S = GqaShape<KV, D>;
  static_assert(NL == S::kLoads, "register sets of the tile's shape");
  if (S::kStageLanes == S::kRowLanes || stage_lane) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int i = 0; i < S::kLoads; ++i)
        *reinterpret_cast<U4*>(slice + (h2 * kTile + S::kRows * i) * S::kPitch + wofs) = rb[h2][i];
  }
}

// The scores of one staged K tile through the matrix cores (E4M3 widened to bf16 after the LDS reads), for NCG
// groups of 16 columns that share each K operand read: S^T = K Q^T, then each group's online-softmax update of
// (m, l) in the exp2 domain with positions >= `lim` masked unless the whole tile is `full`, the rescale of its
// accumulator, and its tile weights as the bf16 pair (pb, pl).
template <int KV, int D, int NCG>
__device__ __forceinline__ void gqa_scores(const char* kread, const U4 (*qb)[GqaShape<KV, D>::kChunks],
                                           float scale_log2, int t, bool full, const int* lim, int j, float* m,
                                           float* l, f32x4 (*o)[GqaShape<KV, D>::kNt], U4* pb, U4* pl) {
  using S = GqaShape<KV, D>;
  f32x4 sc[NCG][2];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
    for (int k = 0; k < NCG; ++k) sc[k][h2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < S::kChunks; ++c) {
      const U4 kop = S::kRaw ? widen8(*reinterpret_cast<const u32x2*>(kread + h2 * kTile * S::kPitch + c * 32))
                             : *reinterpret_cast<const U4*>(kread + h2 * kTile * S::kPitch + c * 64);
#pragma unroll
      for (int k = 0; k < NCG; ++k) sc[k][h2] = mfma(kop, qb[k][c], sc[k][h2]);
    }
  }
#pragma unroll
  for (int k = 0; k < NCG; ++k) {
    float sv[8];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[h2 * 4 + i] = sc[k][h2][i] * scale_log2;
    if (!full) {
      // this lane's score (h2, i) is position t + h2 * kTile + 4j + i: masked from offset `rel` on
      const int rel = lim[k] - t - 4 * j;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (h2 * kTile + i >= rel) sv[h2 * 4 + i] = -INFINITY;
    }
    float mt = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) mt = fmaxf(mt, sv[e]);
    mt = max_over_rows(mt);
    const float mn = fmaxf(m[k], mt);
    const float mref = mn == -INFINITY ? 0.f : mn;
    const float alpha = fast_exp2(m[k] - mref);
    m[k] = mn;
    float psum;
    prob_operands(sv, mref, pb[k], pl[k], psum);
    l[k] = l[k] * alpha + psum;
    // Once the running maxima settle, alpha = exp2(0) is exactly 1 in every lane and the rescale would change
    // nothing: it is skipped for the whole wave then.
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int nt = 0; nt < S::kNt; ++nt) {
        o[k][nt][0] *= alpha;
        o[k][nt][1] *= alpha;
        o[k][nt][2] *= alpha;
        o[k][nt][3] *= alpha;
      }
    }
  }
}

// O^T += V^T (P_hi + P_lo)^T over one staged V tile, for NCG groups of columns sharing each V^T operand read.
template <int KV, int D, int NCG>
__device__ __forceinline__ void gqa_pv(const char* rbase, const U4* pb, const U4* pl,
                                       f32x4 (*o)[GqaShape<KV, D>::kNt]) {
  using S = GqaShape<KV, D>;
#pragma unroll
  for (int nt = 0; nt < S::kNt; ++nt) {
    // A operand: V^T rows = dims 16nt + n, contraction index k = 8j + e -> token (e < 4 ? 4j + e : 16 + 4j + e - 4);
    // this lane gets dim 16nt + n of tokens 4j..4j+3 and 16+4j..16+4j+3
    U4 vt;
    if constexpr (S::kRaw) {
      vt = widen8(lds_read_tr8(rbase + nt * 16));
    } else {
      const u32x2 lo = lds_read_tr16(rbase + nt * 32);
      const u32x2 hi = lds_read_tr16(rbase + kTile * S::kPitch + nt * 32);
      vt = U4{lo.x, lo.y, hi.x, hi.y};
    }
#pragma unroll
    for (int k = 0; k < NCG; ++k) o[k][nt] = mfma(vt, pl[k], mfma(vt, pb[k], o[k][nt]));
  }
}

// Both products of one tile staged whole (K and V in their own slices).
template <int KV, int D, int NCG>
__device__ __forceinline__ void gqa_compute(const char* kread, const char* rbase,
                                            const U4 (*qb)[GqaShape<KV, D>::kChunks], float scale_log2, int t,
                                            bool full, const int* lim, int j, float* m, float* l,
                                            f32x4 (*o)[GqaShape<KV, D>::kNt]) {
  U4 pb[NCG], pl[NCG];
  gqa_scores<KV, D, NCG>(kread, qb, scale_log2, t, full, lim, j, m, l, o, pb, pl);
  gqa_pv<KV, D, NCG>(rbase, pb, pl, o);
}

// Q^T, the B operand of S^T = K Q^T, for a column whose query row starts at element `qe` of the bf16 query:
// lane (n, j) holds dims 32c + 8j .. 32c + 8j + 7; dims past D (the zero padding of the last k-chunk) and columns
// that hold no query row (`ok` false) are 0. Every load stays inside the column's row (or row 0, head 0).
template <int D>
__device__ __forceinline__ void load_query_operand(const void* query, bool ok, int64_t qe, int j, U4* qb) {
  constexpr int kChunks = (D + 31) / 32;
  const char* qptr = static_cast<const char*>(query) + (ok ? qe * 2 : 0);
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const bool in = 32 * c + 8 * j < D;
    const U4 v = *reinterpret_cast<const U4*>(qptr + (in ? c * 64 + j * 16 : 0));
    qb[c] = ok && in ? v : U4{0u, 0u, 0u, 0u};
  }
}

// Per-lane byte offsets of a wave-wide load inside a 16-row half tile: lane (rr, rc) takes the 16-byte piece rc
// of row rr + kRows i. Lanes past the head row's pieces load at an offset above every descriptor's size (at most
// 8 rows, under 2^30 bytes), so they read zeros without touching memory.
template <int KV, int D>
__device__ __forceinline__ void gqa_offsets(int rr, int rc, int64_t row_bytes, int64_t head_off, uint32_t* off) {
  using S = GqaShape<KV, D>;
  constexpr uint32_t kNowhere = 0x80000000u;
#pragma unroll
  for (int i = 0; i < S::kLoads; ++i)
    off[i] = rc < S::kHeadLanes ? (uint32_t)((rr + S::kRows * i) * row_bytes + head_off + rc * 16) : kNowhere;
}

// W waves (KV heads of one sequence) per workgroup: they stream the same slots of the pool side by side. At
// least two waves per SIMD: with smaller workgroups the compiler would otherwise spend the register budget of
// one (measured on MI355X with 4, 2 and 1 KV heads: 3-8% slower). A wave serves NCG consecutive groups of 16
// columns (1, or 2 at head_dim <= 128 where the registers hold two accumulators): they share every K/V load and
// every LDS operand read.
template <int KV, int D, int W, int NCG, bool kAppend>
__global__ __launch_bounds__(kWave * W, NCG >= 4 ? 1 : 2) void decode_gqa_mfma_kernel(const DecodeArgs a) {
  using S = GqaShape<KV, D>;
  constexpr int kEsize = S::kEsize, kChunks = S::kChunks, kNt = S::kNt, kPitch = S::kPitch, kSlice = S::kSlice;
  constexpr int kRowLanes = S::kRowLanes, kLoads = S::kLoads;
  // a wave may cover two partitions (parking the first one's state) only with one column group
  constexpr bool kPark = S::kTwoParts && NCG == 1;
  __shared__ __attribute__((aligned(16))) char lds[W * S::kSlices * kSlice];

  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x >> 6;
  // Work item (KV-head group, partition group, sequence) and the wave's column-group slot cg (columns
  // 16 NCG cg .. 16 NCG (cg + 1) - 1). With one slot the grid indexes the item directly. With several, the slots
  // of one item read the same K/V, so they are given workgroup ids 8 apart -- ids are dispatched in order and
  // round-robin over the 8 XCDs, so those run back to back on one XCD and the later ones find the K/V in its L2.
  const int nslots = (a.col_groups + NCG - 1) / NCG;
  int bx = blockIdx.x, by = blockIdx.y, bz = blockIdx.z, cg = 0;
  const int64_t n_all = (int64_t)gridDim.x * gridDim.y * gridDim.z;
  if (nslots == 1 && n_all * W <= kResidentWaves) {
    // One round of workgroups: the XCD with the most bytes sets the kernel's time. Workgroup ids are dispatched
    // in order, round-robin over the 8 XCDs, which gives an XCD the same span of every eighth item -- with
    // unequal contexts, the full first spans to some XCDs and the short last ones to others. The ids are remapped
    // (a bijection) so that each XCD takes a contiguous block of (KV-head group, span, sequence) items: whole
    // sequences. Measured on MI355X: 70B-shaped batch 135.8 -> 131.6 us, its E4M3 form 80.4 -> 74.3, 16
    // sequences of 8k-16k tokens 147.1 -> 132.4. Grids of several rounds keep the dispatch order: there the
    // sequences' first spans run together on two XCDs, whose L2 then serves a prefix they share (128 sequences
    // sharing 1024 tokens, 1024-token partitions: 267.4 us, against 322.9 remapped).
    const int64_t lin = blockIdx.x + (int64_t)gridDim.x * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
    const int64_t x = lin % 8, k = lin / 8;
    const int64_t item = x * (n_all / 8) + min<int64_t>(x, n_all % 8) + k;
    bx = (int)(item % gridDim.x);
    by = (int)(item / gridDim.x % gridDim.y);
    bz = (int)(item / ((int64_t)gridDim.x * gridDim.y));
  } else if (nslots > 1) {
    const int nkvg = gridDim.x / nslots;
    const int64_t lin = blockIdx.x + (int64_t)gridDim.x * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
    const int64_t items = n_all / nslots;
    const int64_t base = lin / (8 * nslots) * 8;         // first item of this run of 8 x nslots workgroups
    const int64_t width = min<int64_t>(8, items - base);  // items in the run (fewer in the last one)
    const int64_t r = lin - base * nslots;
    cg = (int)(r / width);
    const int64_t u = base + r % width;
    bx = (int)(u % nkvg);
    by = (int)(u / nkvg % gridDim.y);
    bz = (int)(u / ((int64_t)nkvg * gridDim.y));
  }
  const int g = bx * W + w;
  const int s = bz;
  if (g >= a.num_kv_heads) return;  // no workgroup barriers below: each wave owns its LDS slice

  // The wave covers parts_per_wave (1 or 2) consecutive partitions, [u0, u1), in one load pipeline. Its online
  // softmax restarts at the partition boundary; the two partitions' states are merged by the log-sum-exp rule
  // at the end, and the wave leaves one partial result for its span (partition boundaries fall on 32-token
  // tiles whenever parts_per_wave is 2).
  const int L = min(max(a.context_lens[s], 0), a.max_context_len);
  const int span = a.partition * a.parts_per_wave;
  const int u0 = by * span;
  if (by > 0 && u0 >= L) return;
  const int u1 = min(L, u0 + span);
  const int G = a.group;
  const int n = lane & 15;  // MFMA column
  const int j = lane >> 4;  // 0..3
  // Column c = qi * G + hh is head g * G + hh of the sequence's query row qi: in decode the sequence has one
  // row (qi = 0, c < G). With several new tokens per sequence, row qi of its QL rows attends causally over the
  // first L - QL + qi + 1 positions, and the columns hold G heads of the rows in groups of 16.
  int q0 = s, ql = 1;
  if (a.query_start) {
    q0 = a.query_start[s];
    ql = rows_of_seq(a, s);
  }
  int qrow[NCG], hh[NCG], lim[NCG];
  bool head_ok[NCG];
#pragma unroll
  for (int k = 0; k < NCG; ++k) {
    const int col = (cg * NCG + k) * 16 + n;
    const int qi = col / G;
    hh[k] = col - qi * G;
    qrow[k] = q0 + qi;  // the column's query row
    head_ok[k] = qi < ql && qrow[k] < a.num_tokens;
    lim[k] = head_ok[k] ? min(u1, L - ql + qi + 1) : u0;  // the column attends over positions < lim
  }
  const int ufull = min(u1, L - ql + 1);  // every column attends over positions < ufull
  const int rr = lane / kRowLanes;  // loads: row within a wave-wide load
  const int rc = lane % kRowLanes;  //        16-byte chunk within the row
  const int64_t row_bytes = (int64_t)a.num_kv_heads * D * kEsize;
  const int64_t head_off = (int64_t)g * D * kEsize;
  char* const kslice = lds + w * S::kSlices * kSlice;
  char* const vslice = S::kPhased ? kslice : kslice + kSlice;  // phased: V takes K's slice after the scores

  // Q^T (B operand of S^T = K Q^T): lane (n, j) holds dims 32c + 8j .. 32c + 8j + 7 of its column's query row
  U4 qb[NCG][kChunks];
#pragma unroll
  for (int k = 0; k < NCG; ++k)
    load_query_operand<D>(a.query, head_ok[k], ((int64_t)qrow[k] * a.num_q_heads + (int64_t)g * G + hh[k]) * D, j,
                          qb[k]);

  // per-lane byte offsets inside a 16-row half tile: each wave-wide load covers kRows whole head rows (full
  // cache lines: 256 bytes of bf16 or 128 of E4M3 at D = 128), for K as for V
  uint32_t off[kLoads];
  gqa_offsets<KV, D>(rr, rc, row_bytes, head_off, off);
  const bool stage_lane = rc < S::kStageLanes;

  // Decode with the sequence's new token appended in this launch (the cache write of page 3 section 2.1 and the
  // attention over it in one pass). Every lane of a head row's lane group loads its piece of head g's new K/V
  // row: 16 bytes as given, or 32 bytes of bf16 that become 16 E4M3 codes, quantised exactly as the quantising
  // cache write does. The loads are unconditional, and their registers are first read once the first tile's
  // loads are in flight, so no wait for them holds back those loads. The waves whose span holds the new
  // position stage the row over the tile's pool row, which may or may not have been written yet, and the one of
  // them in the first column-group slot stores it into its slot of both pools, after its loop (a position past
  // max_context_len is not attended over, and the first span's wave stores it). Only these waves form the row
  // as the pool holds it. A token whose slot the cache write would skip (slot < 0 or past the pool) is neither
  // written nor substituted.
  constexpr int kNewPieces = S::kRaw ? 2 : 1;
  int tj_new = -1, r_new = 0;
  bool lane_new = false, lane_store = false, need_new = false;
  int64_t store_at = 0;
  U4 nk[kNewPieces], nv[kNewPieces];
  U4 nkc{}, nvc{};  // the pieces as the pool holds them
  if constexpr (kAppend) {
    const bool piece = rc < S::kHeadLanes;
    // this lane's piece of the input row (the first piece for lanes past the row), in 16-byte units
    const int64_t src = (((int64_t)s * a.num_kv_heads + g) * D * (S::kRaw ? 2 : kEsize)) / 16 +
                        (piece ? rc : 0) * kNewPieces;
#pragma unroll
    for (int e = 0; e < kNewPieces; ++e) {
      nk[e] = static_cast<const U4*>(a.new_key)[src + e];
      nv[e] = static_cast<const U4*>(a.new_value)[src + e];
    }
    const int Lraw = a.context_lens[s];
    const int64_t slot = a.slot_mapping[s];
    if (slot >= 0 && slot < (a.num_blocks << a.bs_log2) && Lraw >= 1) {
      const int p = Lraw - 1;
      const bool attended = Lraw <= a.max_context_len;
      const bool here = attended && p >= u0 && p < u1;
      const bool stores = cg == 0 && (attended ? here : by == 0);
      need_new = here || stores;
      lane_store = stores && rr == 0 && piece;
      store_at = slot * row_bytes + head_off + rc * 16;
      if (here) {
        tj_new = (p - u0) / kTileTok;
        r_new = (p - u0) % kTileTok;
        lane_new = piece && rr == (r_new % kTile) % S::kRows;
      }
    }
  }
  // the lane's 16 bytes of the new K or V row as the pool holds them
  auto new_piece = [&](const U4* raw, float scale) __attribute__((always_inline)) {
    if constexpr (S::kRaw)
      return e4m3_pack16_bf16<false>(raw[0], raw[1], e4m3_div(scale));
    else
      return raw[0];
  };

  const char* __restrict__ kbase = static_cast<const char*>(a.key_cache);
  const char* __restrict__ vbase = static_cast<const char*>(a.value_cache);
  // with the pool stores of an appended decode, the table is read through the constant address space: only
  // there do its loads stay scalar, and the tile descriptors wave-uniform
  const auto* __restrict__ table = [&] {
    if constexpr (kAppend)
      return as_constant(a.block_tables);
    else
      return a.block_tables;
  }() + (int64_t)s * a.max_blocks_per_seq;

  float m[NCG], l[NCG];
  f32x4 o[NCG][kNt];
#pragma unroll
  for (int k = 0; k < NCG; ++k) {
    m[k] = -INFINITY;
    l[k] = 0.f;
#pragma unroll
    for (int nt = 0; nt < kNt; ++nt) o[k][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  bool bad = false;
  const int ntiles = (u1 - u0 + kTileTok - 1) / kTileTok;
  const int last8 = ntiles > 0 ? ((u1 - 1) & ~(kTile / 2 - 1)) : u0;  // start of the last live 8-token group
  // One register set: a tile's loads land in it, are staged into LDS, and the next tile's loads are issued into
  // it before the staged tile's products are computed -- about one tile of loads in flight per wave at all times.
  // (Two register sets, two tiles in flight, were measured slower: more concurrent reads congest the memory
  // system rather than feed it.) Phased shapes hold K or V of a tile at a time.
  U4 kR[2][kLoads], vR[2][S::kPhased ? 1 : kLoads];
  auto issue_kv = [&](int tile) {
    gqa_issue<KV, D, true, !S::kPhased>(kR, (U4(*)[kLoads])vR, table, u0 + min(tile, ntiles - 1) * kTileTok,
                                        u0 + tile * kTileTok, u1, last8, a, row_bytes, kbase, vbase, off, bad);
  };
  auto issue_v = [&](int tile) {  // phased: V of a tile into the register set K has left
    bool unused = false;  // the same table entries as the tile's K loads
    gqa_issue<KV, D, false, true>(kR, kR, table, u0 + min(tile, ntiles - 1) * kTileTok, u0 + tile * kTileTok, u1,
                                  last8, a, row_bytes, kbase, vbase, off, unused);
  };

  // LDS: row r of the tile at slice + r * kPitch, K and V each in their own slice (bf16, or E4M3 codes as
  // loaded). This lane writes its 16 loaded bytes of rows rr + kRows*i (+16 for the second half) at byte
  // rc * 16 of both slices; it reads its MFMA operands back as S::k_read and S::v_read describe.
  const int wofs = rr * kPitch + rc * 16;
  const char* const kread = S::k_read(kslice, n, j);
  const char* const rbase = S::v_read(vslice, n, j);

  // A wave covers at most two partitions. Finishing the first one mid-range only parks its state in
  // registers: any store inside the load loop would leave the compiler unable to count outstanding memory
  // operations, and it would then drain the load pipeline on every tile.
  const int cut = min(u0 + a.partition, u1);  // end of the wave's first partition (u1 unless kPark)
  float m_first = -INFINITY, l_first = 0.f;
  constexpr int kNtFirst = kPark ? kNt : 1;
  f32x4 o_first[kNtFirst];
#pragma unroll
  for (int nt = 0; nt < kNtFirst; ++nt) o_first[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto park_first = [&]() {
    if constexpr (!kPark) return;
    m_first = m[0];
    l_first = l[0];
#pragma unroll
    for (int nt = 0; nt < kNtFirst; ++nt) o_first[nt] = o[0][nt];
    m[0] = -INFINITY;
    l[0] = 0.f;
#pragma unroll
    for (int nt = 0; nt < kNt; ++nt) o[0][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  // Normalise the span's rows of column group k and write them: the output itself when the sequence fits one
  // span, else partial p of the split workspace.
  const float poison = __uint_as_float(0x7fc00000u);
  auto write_rows = [&](int k, int p, float mp, float lp, const f32x4* op) {
    // each lane summed the probabilities of its own token group j; the max is already shared
    float lt = lp + __shfl_xor(lp, 16);
    lt += __shfl_xor(lt, 32);
    if (!head_ok[k]) return;
    const int h = g * G + hh[k];
    const float inv = lt > 0.f ? a.v_scale / lt : 0.f;
    float* dst;
    if (!a.split || L <= span) {
      dst = a.out + ((int64_t)qrow[k] * a.num_q_heads + h) * D;
    } else {
      const int64_t wrow = ((int64_t)qrow[k] * a.num_q_heads + h) * a.max_partitions + p;
      dst = a.ws_o + wrow * D;
      if (j == 0) {
        a.ws_ml[2 * wrow] = bad ? poison : mp;
        a.ws_ml[2 * wrow + 1] = lt;
      }
    }
#pragma unroll
    for (int nt = 0; nt < kNt; ++nt) {
      const f32x4 v = op[nt];
      *reinterpret_cast<float4*>(dst + nt * 16 + 4 * j) =
          bad ? make_float4(poison, poison, poison, poison)
              : make_float4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    }
  };

  // the appended row over the staged pool row: the same lane staged that piece, so its write lands after
  auto substitute = [&](int tj, char* slice, const U4& piece) __attribute__((always_inline)) {
    if constexpr (kAppend)
      if (tj == tj_new && lane_new) *reinterpret_cast<U4*>(slice + r_new * kPitch + rc * 16) = piece;
  };
  auto tile_step = [&](int tj) {
    const int t = u0 + tj * kTileTok;
    const bool full = t + kTileTok <= ufull;  // no column masks a position of a tile below ufull
    wave_lds_sync();  // the previous tile's reads come first
    gqa_stage<KV, D>(kR, kslice, wofs, stage_lane);
    substitute(tj, kslice, nkc);
    if constexpr (S::kPhased) {
      wave_lds_sync();
      issue_v(tj);
      U4 pb[NCG], pl[NCG];
      gqa_scores<KV, D, NCG>(kread, qb, a.scale_log2, t, full, lim, j, m, l, o, pb, pl);
      wave_lds_sync();
      gqa_stage<KV, D>(kR, vslice, wofs, stage_lane);
      substitute(tj, vslice, nvc);
      wave_lds_sync();
      issue_kv(tj + 1);  // past the last tile every row is beyond the range: nothing is read
      gqa_pv<KV, D, NCG>(rbase, pb, pl, o);
    } else {
      gqa_stage<KV, D>((U4(*)[kLoads])vR, vslice, wofs, stage_lane);
      substitute(tj, vslice, nvc);
      wave_lds_sync();
      issue_kv(tj + 1);  // past the last tile every row is beyond the range: nothing is read
      gqa_compute<KV, D, NCG>(kread, rbase, qb, a.scale_log2, t, full, lim, j, m, l, o);
    }
  };
  if (ntiles > 0) {
    issue_kv(0);
    if constexpr (kAppend) {
      // after every load of the first tile is out (computed inside the tile loop, it would be hoisted before
      // them, and without the barrier the scheduler would wait for the new row between them)
      __builtin_amdgcn_sched_barrier(0);
      if (need_new) {
        nkc = new_piece(nk, a.new_k_scale);
        nvc = new_piece(nv, a.new_v_scale);
      }
    }
    // The tiles of the first partition, the park, then the rest: two loops around one pipeline. (A park taken
    // conditionally inside a single loop made the compiler copy every accumulator and parked register on each
    // tile, about 100 moves per tile.)
    const int ncut = kPark && cut < u1 ? (cut - u0) / kTileTok : ntiles;
    int tj = 0;
    for (; tj < ncut; ++tj) tile_step(tj);
    if (kPark && cut < u1) park_first();  // the tile before ends the first of two partitions
    for (; tj < ntiles; ++tj) tile_step(tj);
  }
  if (kPark && cut < u1) {
    // merge the first partition's state into the second's: one partial per wave
    const float M = fmaxf(m_first, m[0]);
    const float Mr = M == -INFINITY ? 0.f : M;
    const float fa = fast_exp2(m_first - Mr), fb = fast_exp2(m[0] - Mr);
    l[0] = l_first * fa + l[0] * fb;
#pragma unroll
    for (int nt = 0; nt < kNtFirst; ++nt)
#pragma unroll
      for (int e = 0; e < 4; ++e) o[0][nt][e] = o_first[nt][e] * fa + o[0][nt][e] * fb;
    m[0] = M;
  }
  // an empty context writes a zero row (l = 0)
#pragma unroll
  for (int k = 0; k < NCG; ++k) write_rows(k, by, m[k], l[k], o[k]);
  if constexpr (kAppend) {
    if (lane_store) {
      if (ntiles <= 0) {  // (no tile loop: not formed above)
        nkc = new_piece(nk, a.new_k_scale);
        nvc = new_piece(nv, a.new_v_scale);
      }
      *reinterpret_cast<U4*>(static_cast<char*>(a.key_out) + store_at) = nkc;
      *reinterpret_cast<U4*>(static_cast<char*>(a.value_out) + store_at) = nvc;
    }
  }
}

// Balanced split (one column group: the G heads of a KV head times at most 16 / G query rows per sequence). With
// one wave per (sequence, KV head, partition), unequal contexts leave waves of unequal length, and a grid of whole
// workgroups of 8 KV heads leaves some CUs without one and some XCDs with more bytes than others. Here the
// 32-token tiles of all sequences, in sequence order, form one list cut into `chunks` equal runs; workgroup
// (x, r) takes run r for KV heads Wx .. Wx + W - 1, and the host sizes the grid to one wave per wave slot of the
// chip, so every wave streams the same number of tiles and every XCD the same bytes. A run crosses sequence
// boundaries: the load pipeline runs straight through them (the first tile of the next sequence is in flight while
// the last one of the current sequence goes through the products, and its query rows come in with it), so a wave
// never drains its loads between sequences. When a sequence's last tile of the run is done, its rows are written:
// a sequence lying wholly inside the run goes to `out`; one cut by run boundaries leaves, for each of its query
// rows qi, a partial in slot [head][run][2][qi] -- side 0 for the sequence the run starts inside, side 1 for the
// one it ends inside -- and balanced_reduce_kernel merges them. A sequence without query rows contributes no tiles.
//
// Every workgroup first derives the prefix of the sequences' tile counts in LDS; the first one also
// publishes it for the merge.
//
// Decode with each sequence's new token appended in this launch (kAppend; one query row per sequence): as in the
// partition kernel, every lane loads its piece of head g's new row, for each sequence when its query comes in,
// and the wave whose run holds the sequence's last tile stages that row over the pool's and stores it into the
// sequence's slot once the segment is done.
template <int KV, int D, int W, bool kAppend>
__global__ __launch_bounds__(kWave * W, 2) void decode_gqa_mfma_balanced_kernel(const DecodeArgs a) {
  using S = GqaShape<KV, D>;
  constexpr int kEsize = S::kEsize, kChunks = S::kChunks, kNt = S::kNt, kPitch = S::kPitch, kSlice = S::kSlice;
  constexpr int kRowLanes = S::kRowLanes, kLoads = S::kLoads;
  constexpr int NT = kWave * W;
  __shared__ __attribute__((aligned(16))) char lds[W * S::kSlices * kSlice];
  __shared__ int32_t wave_total[W];
  extern __shared__ int32_t P[];  // [num_seqs + 1]: tiles of the sequences before each one

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = a.num_seqs;
  const ConstI32* __restrict__ lens = as_constant(a.context_lens);
  for (int s = tid; s < T; s += NT) {
    const int L = min(max(lens[s], 0), a.max_context_len);
    const int ql = a.query_start ? rows_of_seq(a, s) : 1;
    P[s + 1] = ql > 0 ? (L + kTileTok - 1) / kTileTok : 0;
  }
  __syncthreads();
  block_exclusive_scan<NT>(P, T, wave_total);
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int r = tid; r <= T; r += NT) a.tile_prefix[r] = P[r];

  const int g = blockIdx.x * W + w;
  if (g >= a.num_kv_heads) return;  // no workgroup barriers below: each wave owns its LDS slice
  const int chunk = blockIdx.y;
  const int total = __builtin_amdgcn_readfirstlane(P[T]);
  const int C = (total + a.chunks - 1) / a.chunks;  // tiles per run
  const int g0 = chunk * C;                          // this run: tiles [g0, g1) of the list
  const int g1 = min(g0 + C, total);
  if (g0 >= g1) return;

  const int G = a.group;
  const int n = lane & 15;  // MFMA column n = qi * G + hh: head g * G + hh of the sequence's query row qi
  const int j = lane >> 4;
  const int qi = n / G;
  const int hh = n - qi * G;
  const int rr = lane / kRowLanes;
  const int rc = lane % kRowLanes;
  const int64_t row_bytes = (int64_t)a.num_kv_heads * D * kEsize;
  const int64_t head_off = (int64_t)g * D * kEsize;
  char* const kslice = lds + w * S::kSlices * kSlice;
  char* const vslice = S::kPhased ? kslice : kslice + kSlice;  // phased: V takes K's slice after the scores
  uint32_t off[kLoads];
  gqa_offsets<KV, D>(rr, rc, row_bytes, head_off, off);
  const bool stage_lane = rc < S::kStageLanes;
  const int wofs = rr * kPitch + rc * 16;
  const char* const kread = S::k_read(kslice, n, j);
  const char* const rbase = S::v_read(vslice, n, j);
  const char* __restrict__ kbase = static_cast<const char*>(a.key_cache);
  const char* __restrict__ vbase = static_cast<const char*>(a.value_cache);
  const float poison = __uint_as_float(0x7fc00000u);

  // appended decode: sequence s's new K/V piece of this lane (16 bytes as given, or 32 bytes of bf16 for 16 E4M3
  // codes), loaded unconditionally (lanes past the head row take the first piece)
  constexpr int kNewPieces = S::kRaw ? 2 : 1;
  const bool piece = rc < S::kHeadLanes;
  auto load_new = [&](int s, U4* k, U4* v) __attribute__((always_inline)) {
    if constexpr (kAppend) {
      const int64_t src = (((int64_t)s * a.num_kv_heads + g) * D * (S::kRaw ? 2 : kEsize)) / 16 +
                          (piece ? rc : 0) * kNewPieces;
#pragma unroll
      for (int e = 0; e < kNewPieces; ++e) {
        k[e] = static_cast<const U4*>(a.new_key)[src + e];
        v[e] = static_cast<const U4*>(a.new_value)[src + e];
      }
    }
  };
  // the piece as the pool holds it (E4M3: quantised exactly as the quantising cache write does)
  auto new_piece = [&](const U4* raw, float scale) __attribute__((always_inline)) {
    if constexpr (S::kRaw)
      return e4m3_pack16_bf16<false>(raw[0], raw[1], e4m3_div(scale));
    else
      return raw[0];
  };

  // the run's first sequence: the first s with P[s + 1] > g0
  int lo = 0, hi = T - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (__builtin_amdgcn_readfirstlane(P[mid + 1]) <= g0) lo = mid + 1;
    else hi = mid;
  }

  // A sequence segment of the run: the sequence's tiles in [g0, g1), positions [u0, u1).
  struct Seg {
    int s, p0, p1, L, u1, last8;
    const ConstI32* table;
  };
  auto segment = [&](int s) {
    Seg q;
    q.s = s;
    q.p0 = __builtin_amdgcn_readfirstlane(P[s]);
    q.p1 = __builtin_amdgcn_readfirstlane(P[s + 1]);
    q.L = min(max(lens[s], 0), a.max_context_len);
    q.u1 = min(q.L, (min(q.p1, g1) - q.p0) * kTileTok);
    q.last8 = (q.u1 - 1) & ~(kTile / 2 - 1);  // start of the last live 8-token group
    q.table = as_constant(a.block_tables) + (int64_t)s * a.max_blocks_per_seq;
    return q;
  };
  // the next sequence holding tiles after s (one exists while tiles of the run remain)
  auto next_seq = [&](int s) {
    ++s;
    while (__builtin_amdgcn_readfirstlane(P[s + 1]) == __builtin_amdgcn_readfirstlane(P[s])) ++s;
    return s;
  };
  // the query operand of sequence s's columns (Q^T, B operand of S^T = K Q^T): lane (n, j) holds dims 32c + 8j ..
  // 32c + 8j + 7 of its column's query row; columns past the sequence's rows are 0 (and read row 0, head 0)
  auto load_query = [&](int s, U4* qv) {
    int q0 = s, ql = 1;
    if (a.query_start) {
      q0 = __builtin_amdgcn_readfirstlane(a.query_start[s]);
      ql = rows_of_seq(a, s);
    }
    const bool ok = qi < ql && q0 + qi < a.num_tokens;
    load_query_operand<D>(a.query, ok, ((int64_t)(q0 + qi) * a.num_q_heads + (int64_t)g * G + hh) * D, j, qv);
  };

  // issue cursor: the segment of the next tile to load; compute cursor: the segment of the staged tile
  Seg is = segment(lo);
  Seg cs = is;
  U4 qb[kChunks], qn[kChunks];
  load_query(cs.s, qb);
  // appended decode: the issue cursor's sequence's new pieces as loaded, the compute cursor's as the pool holds
  // them (converted once the next tile's loads are in flight, so that no wait for them holds those back)
  U4 nkn[kNewPieces], nvn[kNewPieces];
  U4 nkc{}, nvc{};
  load_new(cs.s, nkn, nvn);
  // one register set (phased shapes: K or V of a tile at a time), as in the partition kernel
  U4 kR[2][kLoads], vR[2][S::kPhased ? 1 : kLoads];
  bool bad_staged = false, bad_issued = false;
  auto issue_kv = [&](int gi) {  // tile gi of the list, inside the issue segment
    const int t = (gi - is.p0) * kTileTok;
    gqa_issue<KV, D, true, !S::kPhased>(kR, (U4(*)[kLoads])vR, is.table, t, t, is.u1, is.last8, a, row_bytes,
                                        kbase, vbase, off, bad_issued);
  };
  auto issue_v = [&](int gi) {  // phased: V of tile gi (still in the issue segment) into the set K has left
    const int t = (gi - is.p0) * kTileTok;
    bool unused = false;  // the same table entries as the tile's K loads
    gqa_issue<KV, D, false, true>(kR, kR, is.table, t, t, is.u1, is.last8, a, row_bytes, kbase, vbase, off,
                                  unused);
  };

  // per-segment state of the compute cursor
  int q0, ql, qrow, lim0, ufull;
  bool head_ok;
  // appended decode: whether this run holds the sequence's last tile and writes its new token (slot), whether the
  // token is attended over (the lane then stages its piece as row r_new of that tile)
  bool seg_store = false, lane_new = false;
  int64_t seg_slot = 0;
  int r_new = 0;
  auto begin_segment = [&]() {
    if constexpr (kAppend) {
      const int Lraw = lens[cs.s];
      const int64_t slot = as_constant(a.slot_mapping)[cs.s];
      seg_store = cs.p1 <= g1 && Lraw >= 1 && slot >= 0 && slot < (a.num_blocks << a.bs_log2);
      seg_slot = slot;
      r_new = (Lraw - 1) % kTileTok;
      lane_new = seg_store && Lraw <= a.max_context_len && piece && rr == (r_new % kTile) % S::kRows;
    }
    q0 = cs.s;
    ql = 1;
    if (a.query_start) {
      q0 = __builtin_amdgcn_readfirstlane(a.query_start[cs.s]);
      ql = rows_of_seq(a, cs.s);
    }
    qrow = q0 + qi;
    head_ok = qi < ql && qrow < a.num_tokens;
    // row qi attends causally over its first L - ql + qi + 1 positions, every column over those below ufull
    lim0 = head_ok ? min(cs.u1, cs.L - ql + qi + 1) : 0;
    ufull = min(cs.u1, cs.L - ql + 1);
  };
  begin_segment();
  float m = -INFINITY, l = 0.f;
  f32x4 o[kNt];
#pragma unroll
  for (int nt = 0; nt < kNt; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  bool bad = false;

  auto issue_next = [&](int gi) {  // the tile after gi, if the run holds one
    if (gi + 1 < g1) {
      if (gi + 1 >= is.p1) {  // the next tile opens the next sequence: its query rows come in with it
        is = segment(next_seq(is.s));
        load_query(is.s, qn);
        load_new(is.s, nkn, nvn);
      }
      issue_kv(gi + 1);
    }
  };

  issue_kv(g0);
  if constexpr (kAppend) {  // only a segment that holds its sequence's last tile stages or stores the row
    __builtin_amdgcn_sched_barrier(0);  // after the first tile's loads, as in the partition kernel
    if (seg_store) {
      nkc = new_piece(nkn, a.new_k_scale);
      nvc = new_piece(nvn, a.new_v_scale);
    }
  }
  // the appended row over the staged pool row of the sequence's last tile (the lane staged that piece)
  auto substitute = [&](int gi, char* slice, const U4& pc) __attribute__((always_inline)) {
    if constexpr (kAppend)
      if (gi == cs.p1 - 1 && lane_new) *reinterpret_cast<U4*>(slice + r_new * kPitch + rc * 16) = pc;
  };
  // Segments in an outer loop, their tiles in an inner one. (Closing a segment conditionally inside one tile loop
  // made the compiler copy every accumulator on each tile, as in the partition kernel.)
  int gi = g0;
  while (true) {
    const int gend = min(cs.p1, g1);  // the segment's tiles in this run end here
    for (; gi < gend; ++gi) {
      const int cu0 = (max(g0, cs.p0) - cs.p0) * kTileTok;  // the segment's first position
      const int t = (gi - cs.p0) * kTileTok;
      const int lim = head_ok ? lim0 : cu0;
      const bool full = t + kTileTok <= ufull;
      wave_lds_sync();  // the previous tile's reads come first
      gqa_stage<KV, D>(kR, kslice, wofs, stage_lane);
      substitute(gi, kslice, nkc);
      bad_staged = bad_issued;
      bad_issued = false;
      if constexpr (S::kPhased) {
        wave_lds_sync();
        issue_v(gi);
        U4 pb, pl;
        gqa_scores<KV, D, 1>(kread, (const U4(*)[kChunks])qb, a.scale_log2, t, full, &lim, j, &m, &l,
                             (f32x4(*)[kNt])o, &pb, &pl);
        wave_lds_sync();
        gqa_stage<KV, D>(kR, vslice, wofs, stage_lane);
        substitute(gi, vslice, nvc);
        wave_lds_sync();
        issue_next(gi);
        gqa_pv<KV, D, 1>(rbase, &pb, &pl, (f32x4(*)[kNt])o);
      } else {
        gqa_stage<KV, D>((U4(*)[kLoads])vR, vslice, wofs, stage_lane);
        substitute(gi, vslice, nvc);
        wave_lds_sync();
        issue_next(gi);
        gqa_compute<KV, D, 1>(kread, rbase, (const U4(*)[kChunks])qb, a.scale_log2, t, full, &lim, j, &m, &l,
                              (f32x4(*)[kNt])o);
      }
      bad |= bad_staged;
    }

    // the segment's last tile is done: its rows, whole in this run -> out; else the run's partial for row qi in
    // slot 0 (the run starts inside the sequence) or slot 1 (it ends inside it)
    float lt = l + __shfl_xor(l, 16);
    lt += __shfl_xor(lt, 32);
    if (head_ok) {
      const int h = g * G + hh;
      const float inv = lt > 0.f ? a.v_scale / lt : 0.f;
      float* dst;
      if (cs.p0 >= g0 && cs.p1 <= g1) {
        dst = a.out + ((int64_t)qrow * a.num_q_heads + h) * D;
      } else {
        const int64_t wrow = (((int64_t)h * a.chunks + chunk) * 2 + (cs.p0 > g0 ? 1 : 0)) * a.max_query_len + qi;
        dst = a.ws_o + wrow * D;
        if (j == 0) {
          a.ws_ml[2 * wrow] = bad ? poison : m;
          a.ws_ml[2 * wrow + 1] = lt;
        }
      }
#pragma unroll
      for (int nt = 0; nt < kNt; ++nt) {
        const f32x4 v = o[nt];
        *reinterpret_cast<float4*>(dst + nt * 16 + 4 * j) =
            bad ? make_float4(poison, poison, poison, poison)
                : make_float4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
      }
    }
    if constexpr (kAppend) {
      if (seg_store && rr == 0 && piece) {  // the sequence's new token into its slot of both pools
        const int64_t dst = seg_slot * row_bytes + head_off + rc * 16;
        *reinterpret_cast<U4*>(static_cast<char*>(a.key_out) + dst) = nkc;
        *reinterpret_cast<U4*>(static_cast<char*>(a.value_out) + dst) = nvc;
      }
    }
    if (gi >= g1) break;
    // the next segment: the one the issue cursor opened
    cs = is;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) qb[c] = qn[c];
    begin_segment();
    if constexpr (kAppend) {
      if (seg_store) {
        nkc = new_piece(nkn, a.new_k_scale);
        nvc = new_piece(nvn, a.new_v_scale);
      }
    }
    m = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int nt = 0; nt < kNt; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    bad = false;
  }
}

}  // namespace

bool gqa_mfma_supported(int kv_dtype, int head_dim, int group, int max_query_len) {
  const int64_t columns = (int64_t)group * max_query_len;
  const bool dim_ok = head_dim == 64 || head_dim == 80 || head_dim == 96 || head_dim == 112 || head_dim == 128 ||
                      head_dim == 192 || head_dim == 256;
  return (kv_dtype == PA_BF16 || kv_dtype == PA_FP8_E4M3) && dim_ok &&
         columns >= 2 && columns <= 16 * kMaxColGroups;
}

template <int KV, int D, int W, int NCG>
hipError_t launch_wc(const DecodeArgs& a, hipStream_t stream) {
  if (a.parts_per_wave > (GqaShape<KV, D>::kTwoParts && NCG == 1 ? 2 : 1)) return hipErrorInvalidValue;
  const int groups = a.split ? a.max_partitions : 1;  // one partial slot per wave span
  // the waves' column-group slots share the x dimension with the KV-head groups (the kernel unpacks them)
  const int nslots = (a.col_groups + NCG - 1) / NCG;
  const dim3 grid((a.num_kv_heads + W - 1) / W * nslots, groups, a.num_seqs);
  if (a.new_key) {  // appended decode: one new token (query row) per sequence
    if (a.query_start) return hipErrorInvalidValue;
    decode_gqa_mfma_kernel<KV, D, W, NCG, true><<<grid, dim3(kWave * W), 0, stream>>>(a);
  } else {
    decode_gqa_mfma_kernel<KV, D, W, NCG, false><<<grid, dim3(kWave * W), 0, stream>>>(a);
  }
  return hipGetLastError();
}

template <int KV, int D, int W>
hipError_t launch_w(const DecodeArgs& a, hipStream_t stream) {
  if constexpr (D <= 128)
    if (a.cg_per_wave == 2) return launch_wc<KV, D, W, 2>(a, stream);
  if constexpr (D <= 128 && W <= 4 && KV == PA_BF16)
    if (a.cg_per_wave == 4) return launch_wc<KV, D, W, 4>(a, stream);
  if (a.cg_per_wave != 1) return hipErrorInvalidValue;
  return launch_wc<KV, D, W, 1>(a, stream);
}

// KV heads per workgroup of either grouped-query kernel: up to 8 KV heads of a sequence; the LDS slices of 8
// waves fit one CU (8 x 17 KB at D 128)
int waves_per_group(int32_t num_kv_heads) {
  return num_kv_heads >= 8 ? 8 : num_kv_heads >= 4 ? 4 : num_kv_heads >= 2 ? 2 : 1;
}

template <int KV, int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t stream) {
  // four column groups per wave take one wave per SIMD: at most 4 waves to a workgroup
  switch (a.cg_per_wave == 4 ? min(4, waves_per_group(a.num_kv_heads)) : waves_per_group(a.num_kv_heads)) {
    case 8: return launch_w<KV, D, 8>(a, stream);
    case 4: return launch_w<KV, D, 4>(a, stream);
    case 2: return launch_w<KV, D, 2>(a, stream);
    default: return launch_w<KV, D, 1>(a, stream);
  }
}

struct Launch {
  template <int KV, int D>
  static hipError_t run(const DecodeArgs& a, hipStream_t stream) { return launch_d<KV, D>(a, stream); }
};

// the head dims the grouped-query kernels serve
template <int KV, typename L>
hipError_t dispatch_dim(const DecodeArgs& a, hipStream_t stream) {
  switch (a.head_dim) {
    case 64: return L::template run<KV, 64>(a, stream);
    case 80: return L::template run<KV, 80>(a, stream);
    case 96: return L::template run<KV, 96>(a, stream);
    case 112: return L::template run<KV, 112>(a, stream);
    case 128: return L::template run<KV, 128>(a, stream);
    case 192: return L::template run<KV, 192>(a, stream);
    case 256: return L::template run<KV, 256>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_gqa_mfma(const DecodeArgs& a, int kv_dtype, hipStream_t stream) {
  if (kv_dtype == PA_BF16) return dispatch_dim<PA_BF16, Launch>(a, stream);
  if (kv_dtype == PA_FP8_E4M3) return dispatch_dim<PA_FP8_E4M3, Launch>(a, stream);
  return hipErrorInvalidValue;
}

namespace {

template <int KV, int D, int W>
hipError_t launch_balanced_w(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid((a.num_kv_heads + W - 1) / W, a.chunks, 1);
  const size_t lds = ((size_t)a.num_seqs + 1) * sizeof(int32_t);
  if (a.new_key) {  // appended decode: one new token (query row) per sequence
    if (a.query_start) return hipErrorInvalidValue;
    decode_gqa_mfma_balanced_kernel<KV, D, W, true><<<grid, dim3(kWave * W), lds, stream>>>(a);
  } else {
    decode_gqa_mfma_balanced_kernel<KV, D, W, false><<<grid, dim3(kWave * W), lds, stream>>>(a);
  }
  return hipGetLastError();
}

template <int KV, int D>
hipError_t launch_balanced_d(const DecodeArgs& a, hipStream_t stream) {
  switch (waves_per_group(a.num_kv_heads)) {
    case 8: return launch_balanced_w<KV, D, 8>(a, stream);
    case 4: return launch_balanced_w<KV, D, 4>(a, stream);
    case 2: return launch_balanced_w<KV, D, 2>(a, stream);
    default: return launch_balanced_w<KV, D, 1>(a, stream);
  }
}

struct LaunchBalanced {
  template <int KV, int D>
  static hipError_t run(const DecodeArgs& a, hipStream_t stream) { return launch_balanced_d<KV, D>(a, stream); }
};

}  // namespace

int32_t gqa_balanced_chunks(int32_t num_kv_heads) {
  const int32_t w = waves_per_group(num_kv_heads);
  const int32_t waves = (num_kv_heads + w - 1) / w * w;  // waves of one run across the KV heads
  return waves >= kResidentWaves ? 1 : kResidentWaves / waves;
}

hipError_t launch_decode_gqa_mfma_balanced(const DecodeArgs& a, int kv_dtype, hipStream_t stream) {
  if (a.num_seqs > kMaxBalancedRows || a.chunks <= 0 || !a.tile_prefix || a.col_groups != 1 ||
      a.group * a.max_query_len > 16 || !a.seq_prefix)
    return hipErrorInvalidValue;
  if (kv_dtype == PA_BF16) return dispatch_dim<PA_BF16, LaunchBalanced>(a, stream);
  if (kv_dtype == PA_FP8_E4M3) return dispatch_dim<PA_FP8_E4M3, LaunchBalanced>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
