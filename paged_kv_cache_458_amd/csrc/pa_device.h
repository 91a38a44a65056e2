// Device helpers shared by the gfx950 kernels of libpagedattn: block-table address arithmetic, bf16 decode,
// wave64 cross-lane reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kWave = 64;
constexpr int kTile = 16;  // tokens per tile; tiles start on multiples of 16 (with 8-slot blocks, a tile has two 8-row halves)

struct alignas(16) U4 {
  uint32_t x, y, z, w;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Cache-policy bits of a vector memory instruction on gfx950 (the `aux` operand of the buffer builtins).
constexpr int kPolSc0 = 1;  // sc0
constexpr int kPolNt = 2;   // nt: non-temporal, the line is not kept for reuse
constexpr int kPolSc1 = 16; // sc1

// Policy of the K/V loads: within one call every row is read by one wave, so the loads are non-temporal.
// Measured on MI355X: plain streaming reads reach about 6.3 TB/s, non-temporal ones about 7.1 TB/s; rows
// that several sequences share (a common prefix) still see most of their reuse served from cache.
constexpr int kPolStream = kPolNt;

// Buffer resource over `bytes` bytes at a wave-uniform base (gfx9 raw buffer: stride 0, 32-bit dwords).
// Loads beyond `bytes` return zero instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const char* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, (int)bytes, 0x00020000);
}

// 16-byte load at byte `off` of a buffer resource with cache policy POL.
template <int POL>
__device__ __forceinline__ U4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, POL);
  return U4{v.x, v.y, v.z, v.w};
}

// 16-byte non-temporal load through a flat pointer (diagnostic streaming kernels).
__device__ __forceinline__ U4 load_stream(const char* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return U4{v.x, v.y, v.z, v.w};
}

// Four OCP E4M3 codes (a word, first code in the lowest byte) -> two words of two bf16 each, exactly: every
// E4M3 value is a bf16 value (gfx950 v_cvt_scalef32_pk_bf16_fp8 with scale 1).
__device__ __forceinline__ void e4m3x4_to_bf16x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false));
  hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true));
}

// Four OCP E4M3 codes (first code in the lowest byte) -> four floats in order, exactly (gfx950
// v_cvt_scalef32_pk_f32_fp8 with scale 1: each converts the codes of one half-word).
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void e4m3x4_to_f32x4(uint32_t w, float* f) {
  const f32x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)w, 1.0f, false);
  const f32x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)w, 1.0f, true);
  f[0] = lo.x;
  f[1] = lo.y;
  f[2] = hi.x;
  f[3] = hi.y;
}

// bf16 -> fp32 is exact: the bf16 bits are the high half of the fp32 word.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// OCP E4M3 quantisation, shared by the quantising cache write and the decode kernels that append a new row
// themselves, so both store the same codes. The code of x / scale: the quotient rounded to nearest fp32 (as an
// IEEE division), saturated to +-448, rounded to nearest with ties to even by the hardware conversion (which
// would turn |y| >= 480 into NaN, hence the clamp); NaN is stored as 0x7F. Four values packed into one word,
// first value in the lowest byte.
//
// The quotient without a division per value: with inv = RN(1 / scale) and q = RN(x * inv), the residual
// x - q * scale is exact in one fma, and q + residual * inv rounded once is the correctly rounded quotient
// whenever it is a normal number (Markstein's correction step for division with a fused multiply-add). For
// |scale| in [2^-32, 2^32] every quotient that decides a code (|x / scale| in [2^-11, 512)) is normal, and so
// is every x that gives one; a smaller quotient gives a zero code of its sign, a larger one saturates, either
// way. Exact quotients and signed zeros keep q (zero residual), and so do infinite or NaN q. Other scales take
// the division; kAnyScale = false leaves that path out (callers that only see scales in the range: the decode
// kernels, which the host gives no other scale).
struct E4m3Div {
  float scale, inv;
  bool fast;
};
__host__ __device__ __forceinline__ bool e4m3_fast_scale(float scale) {
  const float a = scale < 0.f ? -scale : scale;
  return a >= 0x1p-32f && a <= 0x1p32f;
}
__device__ __forceinline__ E4m3Div e4m3_div(float scale) { return E4m3Div{scale, 1.0f / scale, e4m3_fast_scale(scale)}; }
template <bool kAnyScale>
__device__ __forceinline__ float e4m3_quotient(float x, const E4m3Div& d) {
  if (kAnyScale && !d.fast) return x / d.scale;
  const float q = x * d.inv;
  const float r = __builtin_fmaf(-q, d.scale, x);
  const float y = __builtin_fmaf(r, d.inv, q);
  return r == 0.f || !__builtin_isfinite(q) ? q : y;
}
template <bool kAnyScale>
__device__ __forceinline__ float e4m3_prepare(float x, const E4m3Div& d) {
  const float y = e4m3_quotient<kAnyScale>(x, d);
  return y != y ? y : fminf(fmaxf(y, -448.f), 448.f);
}
__device__ __forceinline__ uint32_t nan_to_7f(uint32_t word, float a, float b, float c, float d) {
  if (a != a) word = (word & 0xffffff00u) | 0x7fu;
  if (b != b) word = (word & 0xffff00ffu) | 0x7f00u;
  if (c != c) word = (word & 0xff00ffffu) | 0x7f0000u;
  if (d != d) word = (word & 0x00ffffffu) | 0x7f000000u;
  return word;
}
template <bool kAnyScale>
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d, const E4m3Div& dv) {
  a = e4m3_prepare<kAnyScale>(a, dv);
  b = e4m3_prepare<kAnyScale>(b, dv);
  c = e4m3_prepare<kAnyScale>(c, dv);
  d = e4m3_prepare<kAnyScale>(d, dv);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return nan_to_7f((uint32_t)w, a, b, c, d);
}
// 16 values -> 16 codes
template <bool kAnyScale>
__device__ __forceinline__ U4 e4m3_pack16(const float* f, const E4m3Div& dv) {
  return U4{e4m3_pack4<kAnyScale>(f[0], f[1], f[2], f[3], dv), e4m3_pack4<kAnyScale>(f[4], f[5], f[6], f[7], dv),
            e4m3_pack4<kAnyScale>(f[8], f[9], f[10], f[11], dv),
            e4m3_pack4<kAnyScale>(f[12], f[13], f[14], f[15], dv)};
}
// 16 consecutive bf16 values, as two 16-byte pieces -> 16 codes
template <bool kAnyScale>
__device__ __forceinline__ U4 e4m3_pack16_bf16(U4 a, U4 b, const E4m3Div& dv) {
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  float f[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    f[2 * i] = bf16_lo(w[i]);
    f[2 * i + 1] = bf16_hi(w[i]);
  }
  return e4m3_pack16<kAnyScale>(f, dv);
}

// ---------------------------------------------------------------------------------------------------------
// Paged addressing (vLLM PagedAttention, page 1 section 3.2; page 3 section 2.2). Pools are
// [num_blocks][block_size][num_kv_heads][head_dim]; one "row" is a slot: all KV heads of one position,
// row_bytes = num_kv_heads * head_dim * element size. Position t of a sequence sits in slot
// block_table_row[t >> bs_log2] * block_size + (t & (block_size - 1)).
//
// Byte offset of the slot holding position t (t a multiple of kTile, so the kTile positions t .. t+15 are
// consecutive slots of one block). A table entry outside [0, num_blocks) is replaced by block 0 -- always a
// valid address -- and reported through `bad` so the caller can poison its result instead of faulting.
template <typename TablePtr>
__device__ __forceinline__ int64_t tile_slot_bytes(TablePtr table_row, int t, int bs_log2, int64_t num_blocks,
                                                   int64_t row_bytes, bool& bad) {
  const int32_t phys = table_row[t >> bs_log2];
  const bool ok = (uint32_t)phys < (uint64_t)num_blocks;
  bad |= !ok;
  // the slot index fits 32 bits (the host refuses pools of more than 2^32 slots): a 32 x 32-bit product
  const uint32_t slot = ((ok ? (uint32_t)phys : 0u) << bs_log2) + (uint32_t)(t & ((1 << bs_log2) - 1));
  return (int64_t)((uint64_t)slot * (uint32_t)row_bytes);
}

// Block tables are not written while a kernel runs. Read through the constant address space, a wave-uniform
// load of them stays a scalar load even in a kernel that also stores inside its main loop (where the compiler
// could not otherwise rule out that a store changes the table, and would load it per lane and wait for every
// load in flight before using it).
typedef const __attribute__((address_space(4))) int32_t ConstI32;
__device__ __forceinline__ const ConstI32* as_constant(const int32_t* p) { return (const ConstI32*)p; }

// ---------------------------------------------------------------------------------------------------------
// Sum over aligned groups of N lanes (N = 4 .. 64), result in every lane of the group, via DPP
// (quad_perm swaps, then half-row and row mirrors: each step adds the partner's partial sum).
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group size");
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xf, 0xf, false));  // lane ^ 1
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xf, 0xf, false));  // lane ^ 2
  if constexpr (N >= 8)
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xf, 0xf, false));  // 8-mirror
  if constexpr (N >= 16)
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xf, 0xf, false));  // 16-mirror
  if constexpr (N >= 32) v += __shfl_xor(v, 16);
  if constexpr (N == 64) v += __shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Exclusive prefix sum in LDS over the counts of T items: on entry P[r + 1] holds item r's count, on exit P[r]
// holds the sum of the counts of items 0 .. r-1 and P[T] the total. Called by all NT threads of the workgroup
// (NT / kWave waves; `wave_total` holds one int per wave); each thread sums a run of items, a wave scan and
// the waves' totals give its offset. Ends with a barrier.
template <int NT>
__device__ __forceinline__ void block_exclusive_scan(int32_t* P, int T, int32_t* wave_total) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int per = (T + NT - 1) / NT;
  const int rb = tid * per;
  int sum = 0;
  for (int k = 0; k < per; ++k)
    if (rb + k < T) sum += P[rb + k + 1];
  int inc = sum;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int v = __shfl_up(inc, off);
    if (lane >= off) inc += v;
  }
  if (lane == kWave - 1) wave_total[wave] = inc;
  __syncthreads();
  for (int w = 0; w < wave; ++w) inc += wave_total[w];
  int run = inc - sum;
  for (int k = 0; k < per; ++k)
    if (rb + k < T) {
      run += P[rb + k + 1];
      P[rb + k + 1] = run;
    }
  if (tid == 0) P[0] = 0;
  __syncthreads();
}

// Orders one wave's LDS accesses when lanes exchange data through LDS: everything before it (in every lane) is
// visible to everything after it. Without it the compiler may move a lane's read of another lane's data
// above that lane's own earlier write, since a single lane sees no dependence between the two.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace pa
