// Device helpers shared by the gfx950 kernels of libflamia.
//
// Matrix instruction: v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 operands (format selectors 0).
// Lane layout (64 lanes; lane l = n + 32 h, n in [0,32), h in {0,1}):
//   operand bytes: lane (n, h) holds 32 K-values of row/column n; byte k (0..31) of group h is
//     K index kidx(h, k) = 32 * (k / 16) + 8 * ((k % 16) / 4) + 4 * h + (k % 4)
//     (any fixed permutation of K is valid as long as both operands use it; this one is the
//     order in which the accumulator layout below hands out rows, so a score tile can be fed
//     back as an operand without moving data between lanes);
//   scale blocks: the scale byte of lane (n, 0) applies to K indices 0..31 of row n (bytes 0..15
//     of both lane groups) and that of lane (n, 1) to K indices 32..63 (bytes 16..31);
//   accumulator: lane (n, h) register i holds row 8 * (i / 4) + 4 * h + (i % 4), column n.
// These were established by probes on the hardware (see the design notes).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flamia {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v2i* lds_v2i_ptr;

constexpr int BLK = 32;        // tokens per scale block
constexpr int KV_TILE = 128;   // keys per tile (running-max and dQ-partial granularity)
constexpr int ITEM_Q = 256;    // queries per forward work item
constexpr int P_SHIFT = 8;     // forward probability operand: E4M3(2^8 p), scale 2^-8
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ v16f mfma_scaled(const v8i& a, const v8i& b, const v16f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}
// The same instruction on E2M1 operands (format 4): each lane supplies 16 bytes (registers 0..3;
// the upper four are not read), lane (n, h) holding K indices 32 h .. 32 h + 31 of row n, two per
// byte with the lower index in the low nibble, and its scale byte applies to exactly those
// (established by a probe on the hardware).
__device__ __forceinline__ v16f mfma_scaled_fp4(const v4i& a, const v4i& b, const v16f& c, int sa, int sb) {
  const v8i a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0}, b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, 0, sa, 0, sb);
}

// End of an accumulation chain whose result is read next.  The scaled FP8 instruction writes
// its last accumulator registers late; the compiler's padding before the first read has been
// seen to fall one wait state short when scalar instructions fill the gap.  This no-op block is
// tied to the accumulator, so it sits between the last instruction of the chain and every read
// of the result and adds a fixed margin to whatever padding the compiler places.
// mfma_drain: the result is read by vector instructions, so it is kept in (arch) VGPRs;
// mfma_drain_acc: a long-lived accumulator kept in the matrix-core registers (AGPRs).
__device__ __forceinline__ void mfma_drain(v16f& acc) { asm volatile("s_nop 3" : "+v"(acc)); }
__device__ __forceinline__ void mfma_drain_acc(v16f& acc) { asm volatile("s_nop 3" : "+a"(acc)); }

// Workgroup barrier for LDS hand-offs.  The fences cover LDS only, so global loads still in
// flight (prefetches, waited for where their registers are used) and global stores (results no
// wave of this workgroup reads back) do not hold the barrier up; __syncthreads() would wait for
// every outstanding global access at each barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Dynamic assignment of a persistent grid's units ([J] §3.4 "Work scheduling"): each of the
// `first` workgroups that share a counter runs one of units 0 .. first - 1 first, then takes the
// next unit from the atomic counter (counted from `first`) when it has finished the current one,
// so no unit is reserved while its taker is still busy.  Every thread of the workgroup calls
// this; the value is passed through LDS.
__device__ __forceinline__ int next_unit(int32_t* counter, int* slot, int first) {
  if (threadIdx.x == 0) *slot = atomicAdd(counter, 1) + first;
  lds_barrier();
  const int u = *slot;
  lds_barrier();  // every thread has read it before the next write
  return u;
}

// The unit partition of the backward's persistent grids.  Workgroups are dispatched to the
// eight XCDs round robin (workgroup w on XCD w mod 8), and each XCD has an L2 of its own.  With
// KV heads a multiple of 8 (and a grid of whole rounds), XCD x takes the units of the KV heads
// g with g mod 8 = x, in list order, from a counter of its own: units of one head, which share
// its K/V and Q/dO tiles, then meet in one L2.  Otherwise one counter serves the whole grid.
struct UnitPartition {
  int part;    // this workgroup's counter (its XCD, or 0)
  int first;   // workgroups sharing the counter: the first unit index taken from it
  int rank;    // this workgroup's first unit
  int kv_per;  // KV heads per counter
  bool by_xcd;
};
__device__ __forceinline__ UnitPartition unit_partition(int Hkv) {
  const int G = gridDim.x, w = blockIdx.x;
  UnitPartition u;
  u.by_xcd = (Hkv & 7) == 0 && (G & 7) == 0;
  u.part = u.by_xcd ? (w & 7) : 0;
  u.first = u.by_xcd ? (G >> 3) : G;
  u.rank = u.by_xcd ? (w >> 3) : w;
  u.kv_per = u.by_xcd ? (Hkv >> 3) : Hkv;
  return u;
}
// KV head of local index j (0 .. kv_per - 1) of partition `part`.
__device__ __forceinline__ int partition_kv(const UnitPartition& u, int j) {
  return u.by_xcd ? u.part + 8 * j : j;
}

// Accumulator row held by register i of lane group h.
__device__ __forceinline__ int acc_row(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

// ---------------------------------------------------------------------------------------------
// LDS tiles: [rows][COLS] bytes, COLS in {64, 128}, with the 16-byte chunks of each row permuted
// by an XOR with a function of the row.  Taking the LDS as 64 banks of 4 bytes (256 bytes per
// cycle), the permutation keeps both access patterns free of bank conflicts:
//   row-major operand reads: 16 consecutive lanes read the same 16-byte chunk of 16 consecutive
//     rows, which land in 16 distinct 16-byte bank groups;
//   transpose reads: 32 lanes read rows {b..b+3, b+8..b+11} (b = 0 or 4 mod 16) at two adjacent
//     chunks, again 16 distinct bank groups.
// COLS = 128 (two rows per 256 bytes): chunk ^ g(m), m = (row >> 1) & 7, g a permutation of 0..7
//   with g(m) >> 1 distinct over m in {0, 1, 4, 5} and over m in {2, 3, 6, 7};
// COLS = 64 (four rows per 256 bytes): chunk ^ ((row >> 2) & 3).
// COLS = 32 (eight rows per 256 bytes; the 4-bit K tile at d = 64, row-major reads only):
//   chunk ^ ((row >> 3) & 1), so rows r and r + 8 of a 16-row group fill the odd and even groups.
template <int COLS>
__device__ __forceinline__ int lds_swizzle(int row) {
  if constexpr (COLS == 32) {  // eight rows per 256 bytes: rows 8 apart take the other chunk
    return (row >> 3) & 1;
  } else if constexpr (COLS == 128) {
    const int m = (row >> 1) & 7;
    return 2 * ((m & 1) | (((m >> 2) & 1) << 1)) + ((m >> 1) & 1);
  } else {
    return (row >> 2) & 3;
  }
}
template <int COLS>
__device__ __forceinline__ int lds_off(int row, int col) {
  return row * COLS + ((((col >> 4) ^ lds_swizzle<COLS>(row)) << 4) | (col & 15));
}

// Row-major operand: lane reads 32 contiguous bytes of `row` starting at `col` (multiple of 32).
template <int COLS>
__device__ __forceinline__ v8i lds_read_row32(const uint8_t* tile, int row, int col) {
  v4i lo = *reinterpret_cast<const v4i*>(tile + lds_off<COLS>(row, col));
  v4i hi = *reinterpret_cast<const v4i*>(tile + lds_off<COLS>(row, col + 16));
  v8i r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// Row-major 4-bit operand: lane reads 16 contiguous bytes (32 E2M1 values) of `row` at `col`
// (multiple of 16).
template <int COLS>
__device__ __forceinline__ v4i lds_read_row16(const uint8_t* tile, int row, int col) {
  return *reinterpret_cast<const v4i*>(tile + lds_off<COLS>(row, col));
}

// Transposed operand: the K dimension runs along the tile's rows.  For the 64-row K chunk that
// starts at `row0` and the 32 columns that start at `col0` (the operand's M or N index), lane
// (n, h) receives the 32 bytes tile[row0 + kidx(h, k)][col0 + n], k = 0..31, assembled with
// ds_read_b64_tr_b8: in each 16-lane group, source lane s supplies the 8-byte piece of row
// K_(s/2) at column chunk (s & 1), and output lane i receives column i of rows K_0..K_7.
template <int COLS>
__device__ __forceinline__ v8i lds_read_tr32(const uint8_t* tile, int row0, int col0, int lane) {
  const int i = lane & 15;              // position in the 16-lane group
  const int grp = lane >> 4;            // 16-lane group
  const int h = grp >> 1;               // lane group of the operand layout
  const int colbase = col0 + 16 * (grp & 1);
  const int j = i >> 1, e = i & 1;
  v8i r;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = row0 + 32 * (q >> 1) + 16 * (q & 1) + 8 * (j >> 2) + 4 * h + (j & 3);
    const uint8_t* p = tile + lds_off<COLS>(row, colbase + 8 * e);
    v2i t = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_ptr)(p));
    r[2 * q] = t[0];
    r[2 * q + 1] = t[1];
  }
  return r;
}

// ---------------------------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void* lds_void_ptr;

// Direct global -> LDS loads (lane l writes bytes 16 l .. 16 l + 15, or 4 l .. 4 l + 3, of the
// block at the LDS address), issued as inline assembly, out of the compiler's sight: it cannot tell
// that they write other buffers than the ones being read, and would otherwise wait for them
// (for the whole global-memory round trip) before every LDS read that follows.  The kernels
// wait for them explicitly (s_waitcnt) before the barrier that publishes the buffer.  M0 holds
// the LDS address of the wave's block; one wait state separates its write from the load.  M0 is
// a reserved register, so the compiler does not honour its clobber here: these kernels must not
// use M0 for anything else, which a host-side check of their assembly verifies.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)(uintptr_t)(lds_void_ptr)p);
}
__device__ __forceinline__ void dma_load16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(g) : "memory", "m0");
}
// The same with a wave-uniform base address and a 32-bit per-lane byte offset (no per-lane
// 64-bit address arithmetic).
__device__ __forceinline__ void dma_load16_sv(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(base)
               : "memory", "m0");
}
__device__ __forceinline__ void dma_load4(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(lds), "v"(g) : "memory", "m0");
}

// ---------------------------------------------------------------------------------------------
// E8M0 / E4M3 helpers.

// Smallest s with amax <= 448 * 2^s, clamped to >= -127 (amax = 0 or subnormal gives -127);
// 128 for NaN / infinity.  Integer arithmetic on the float's fields: for amax = 1.f * 2^E,
// s = E - 8 + (f > 0.75).
__device__ __forceinline__ int e8m0_roundup(float amax) {
  const uint32_t b = __float_as_uint(amax) & 0x7FFFFFFFu;
  if (b >= 0x7F800000u) return 128;  // infinity or NaN
  // 448 = 1.75 * 2^8: adding 2^21 - 1 carries into the exponent field exactly when the mantissa
  // exceeds 0.75, which is when amax / 2^(E - 127 - 8) exceeds 448; zero and subnormal amax
  // land below -127 and clamp there
  const int s = (int)((b + 0x1FFFFFu) >> 23) - 135;
  return s < -127 ? -127 : s;
}
// The same exponent as its E8M0 byte s + 127 (255 for NaN / infinity), for amax >= +0 (sign bit
// clear), in fewer steps: max((b + 2^21 - 1) >> 23, 8) - 8 is the clamped s + 127.
__device__ __forceinline__ uint32_t e8m0_byte_nonneg(float amax) {
  const uint32_t b = __float_as_uint(amax);
  if (b >= 0x7F800000u) return 255;  // infinity or NaN
  return max((b + 0x1FFFFFu) >> 23, 8u) - 8u;
}
// The same for a wave-uniform maximum, in scalar instructions, with the scale 2^(byte - 127) as a
// float beside the byte (the scaled conversions take it from a scalar register).
__device__ __forceinline__ uint32_t e8m0_byte_uniform(float amax, float& scale) {
  const uint32_t b = (uint32_t)__builtin_amdgcn_readfirstlane((int)__float_as_uint(amax));
  const uint32_t e = (b + 0x1FFFFFu) >> 23;
  uint32_t r = e > 8u ? e - 8u : 0u;
  r = b >= 0x7F800000u ? 255u : r;  // infinity or NaN
  r = (uint32_t)__builtin_amdgcn_readfirstlane((int)r);
  scale = __uint_as_float((uint32_t)__builtin_amdgcn_readfirstlane((int)(r << 23)));
  return r;
}
// 2^-s as a float, for s in [-127, 127].
__device__ __forceinline__ float exp2i_neg(int s) { return __uint_as_float((uint32_t)(127 - s) << 23); }
__device__ __forceinline__ float exp2i(int s) { return __uint_as_float((uint32_t)(127 + s) << 23); }

// E4M3 conversion: round to nearest even, hardware instruction.
// Four floats -> one dword of E4M3 bytes (a0 lowest).
// The first conversion's upper half is overwritten by the second, so its starting value is left
// undefined (no instruction clears the register first).
__device__ __forceinline__ int pack4_fp8(float a0, float a1, float a2, float a3) {
  int u;
  asm volatile("" : "=v"(u));  // an undefined register, formed by no instruction
  const int r = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, u, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, r, true);
}

// Four floats -> one dword of E4M3 codes of x * 2^-s (round to nearest even), s in [-127, 127].
// The scaled conversion instruction divides by the power of two whose float exponent field is
// s + 127 (the field alone is used, so +0.0 stands for 2^-127); on gfx950 it gives exactly the
// codes of the multiply-then-convert sequence, ties, subnormal and saturating results included
// (checked on the hardware for every exponent).
// The scale is given as its E8M0 byte s + 127.
typedef short v2s __attribute__((ext_vector_type(2)));
__device__ __forceinline__ int pack4_fp8_scalef(float a0, float a1, float a2, float a3, float scale) {
  const v2s lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(__builtin_bit_cast(v2s, a0), a0, a1, scale, false);
  const v2s r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, a2, a3, scale, true);
  return __builtin_bit_cast(int, r);
}
__device__ __forceinline__ int pack4_fp8_scaled(float a0, float a1, float a2, float a3, uint32_t sbyte) {
  const float scale = __uint_as_float(sbyte << 23);
  // the first conversion's upper half is overwritten by the second: any value will do there
  const v2s lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(__builtin_bit_cast(v2s, a0), a0, a1, scale, false);
  const v2s r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, a2, a3, scale, true);
  return __builtin_bit_cast(int, r);
}

// ---------------------------------------------------------------------------------------------
// Wave reductions (64 lanes): DPP within rows of 16, then permlane swaps across rows.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));    // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp<0x4E>(x));    // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp<0x124>(x));   // row_ror:4
  x = fmaxf(x, dpp<0x128>(x));   // row_ror:8
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  x = fmaxf(__int_as_float((int)a[0]), __int_as_float((int)a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float((int)b[0]), __int_as_float((int)b[1]));
}
// Maxima over the wave of two non-negative floats a and b at once (unsigned maxima of the bit
// patterns, the same order for non-negative floats).  One permlane32 swap pairs each value's upper
// half of the wave with its lower half, so after one maximum lanes 0-31 carry a's partial maxima
// and lanes 32-63 b's; four DPP steps finish each row of 16 and one permlane16 swap joins the two
// rows of each half.  Lane 0 then holds a's maximum and lane 32 b's (returned wave-uniform): one
// chain of cross-lane steps instead of one per value.
__device__ __forceinline__ void wave_max2_nonneg(float a, float b, float& ma, float& mb) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_int(a), __float_as_int(b), false, false);
  uint32_t u = max((uint32_t)s[0], (uint32_t)s[1]);
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x124, 0xF, 0xF, false));  // row_ror:4
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x128, 0xF, 0xF, false));  // row_ror:8
  const auto t = __builtin_amdgcn_permlane16_swap((int)u, (int)u, false, false);
  u = max((uint32_t)t[0], (uint32_t)t[1]);
  ma = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)u, 0));
  mb = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)u, 32));
}
// Combine the two lane groups (l and l ^ 32).
__device__ __forceinline__ float halves_max(float x) {
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float((int)b[0]), __int_as_float((int)b[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float((int)b[0]) + __int_as_float((int)b[1]);
}
// Max within each row of 16 lanes.
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x124>(x));
  x = fmaxf(x, dpp<0x128>(x));
  return x;
}
__device__ __forceinline__ float row16_sum(float x) {
  x = x + dpp<0xB1>(x);
  x = x + dpp<0x4E>(x);
  x = x + dpp<0x124>(x);
  x = x + dpp<0x128>(x);
  return x;
}

// bf16 helpers: conversions round to nearest even.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
// Rounding in integer arithmetic: the same results as pack_bf16 below (NaN stays NaN, its
// payload may differ).  Used where the packed instruction changes the register allocation of a
// whole kernel (the key-tile pass's dQ for one-tile documents: with it the compiler spills 83
// registers); the branches it compiles to cost little there.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16_int(float a, float b) { return f32_to_bf16(a) | (f32_to_bf16(b) << 16); }
// Two floats to BF16 (a in the low half) with one packed conversion instruction, rounding to
// nearest even; NaN stays NaN.  Branch-free: epilogues that convert a whole tile run it once
// per two values.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{a, b}, b2));
}

// f(k, L) for the documents k of [k0, k1) in order, with L = cu[k + 1] - cu[k]: the bounds are
// loaded 32 documents at a time, every load of a batch issued before the first is used (one
// round trip per batch instead of one per document).
template <typename F>
__device__ __forceinline__ void for_docs(const int32_t* __restrict__ cu, int k0, int k1, F&& f) {
  constexpr int B = 32;
  for (int kb = k0; kb < k1; kb += B) {
    int c[B + 1];
#pragma unroll
    for (int x = 0; x <= B; ++x) c[x] = kb + x <= k1 ? cu[kb + x] : 0;
#pragma unroll
    for (int x = 0; x < B; ++x)
      if (kb + x < k1) f(kb + x, c[x + 1] - c[x]);
  }
}

// Document containing token t: the k with cu[k] <= t < cu[k+1], or -1.
__device__ __forceinline__ int find_doc(const int32_t* __restrict__ cu, int n_docs, int t) {
  if (n_docs <= 0 || t < cu[0] || t >= cu[n_docs]) return -1;
  int lo = 0, hi = n_docs;  // invariant: cu[lo] <= t < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

}  // namespace flamia
