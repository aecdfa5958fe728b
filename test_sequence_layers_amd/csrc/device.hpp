// Device primitives for the gfx950 (CDNA4) TTT kernels: bf16 helpers, 16x16 MFMA wrappers and
// the lane layout they imply. Everything here is independent of the TTT method.
//
// MFMA 16x16 tiles on a 64-wide wavefront. With l = lane id, r = l & 15 and g = l >> 4:
//   A operand (16 rows x K): lane l holds row r, k slots of group g;
//   B operand (K x 16 cols): lane l holds column r, k slots of group g;
//   C/D (16 x 16, fp32):     lane l holds column r, rows 4g .. 4g+3 (element j -> row 4g + j).
// For a given product, slot i of group g in A multiplies slot i of group g in B, so any map
// (g, i) -> k used consistently by both operands gives the same sum. Two maps are used:
//   contiguous:  k = 8g + i                         (one 16-byte row read per lane)
//   c-layout:    k = 4g + i (i < 4), 16 + 4g + i - 4 (one 32-row block as two 16-row tiles)
// The c-layout map lets the C/D tile of one product feed the next product as its B operand
// (contraction over the C/D rows) without leaving registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttt {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// D = A(16x32) B(32x16) + C, bf16 operands, fp32 accumulate.
__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D = A(16x16) B(16x16) + C, bf16 operands (4 k slots per lane, k = 4g + i), fp32 accumulate.
__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                   __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}

// Round-to-nearest-even fp32 -> bf16 (gfx950 converts in hardware, two values per instruction).
// Each half is converted as a 2-vector and the halves are joined as 32-bit words: converted
// element by element into a 4-vector, a fragment that ends up as a 16x16x16 MFMA operand (a
// 16-bit integer vector) was compiled as four single conversions and two byte permutes.
__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 x) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const bf16x2 lo = __builtin_convertvector(f32x2{x[0], x[1]}, bf16x2);
  const bf16x2 hi = __builtin_convertvector(f32x2{x[2], x[3]}, bf16x2);
  return __builtin_bit_cast(bf16x4, make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)));
}

__device__ __forceinline__ bf16x4 to_bf16x4_scaled(f32x4 x, float s) { return to_bf16x4(x * s); }

__device__ __forceinline__ bf16x8 cat8(bf16x4 lo, bf16x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ f32x4 add4(f32x4 a, f32x4 b) { return a + b; }

// Loads of bf16 vectors from LDS or global memory (caller guarantees alignment).
__device__ __forceinline__ bf16x8 ld8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ bf16x4 ld4(const bf16* p) { return *reinterpret_cast<const bf16x4*>(p); }

// Identity tile as an MFMA B operand: lane (r, g) holds I[4g + i][r].
__device__ __forceinline__ bf16x4 identity_b(int r, int g) {
  bf16x4 x;
  for (int i = 0; i < 4; ++i) x[i] = (bf16)(4 * g + i == r ? 1.f : 0.f);
  return x;
}

// A 16 x 16 bf16 tile T (T[t][c] = base[t * pitch + c]) in accumulator layout: lane (r, g) holds
// T[4g + i][r], i.e. the A operand of T^T and the B operand of T. It is formed on the matrix cores
// as T * I from row-contiguous LDS reads (exact), instead of four 2-byte column reads.
__device__ __forceinline__ bf16x4 tile_columns(const bf16* base, int pitch, bf16x4 ident, int r,
                                               int g) {
  return to_bf16x4(mma16(ld4(base + r * pitch + 4 * g), ident, zero4()));
}

// A 16 x 16 bf16 tile T (T[t][c] = base[t * pitch + c], base in LDS) in accumulator layout, by
// gfx950's LDS transpose read (ds_read_b64_tr_b16): lane (r, g) gets T[4g + j][r]. Within each
// 16-lane group that instruction gives lane t, as its element j, element t & 3 of the 8 bytes
// addressed by lane 4j + (t >> 2); so lane 4j + q of group g addresses T[4g + j][4q .. 4q + 3].
// base and pitch must keep those 8-byte reads aligned.
__device__ __forceinline__ bf16x4 tile_tr(const bf16* base, int pitch, int l) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const int u = l & 15;
  const bf16* p = base + (4 * (l >> 4) + (u >> 2)) * pitch + 4 * (u & 3);
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p));
}

// Four bf16 read down a column (stride in elements), e.g. a transposed operand from a row-major tile.
__device__ __forceinline__ bf16x4 ld4_col(const bf16* p, int stride) {
  bf16x4 r;
  r[0] = p[0];
  r[1] = p[stride];
  r[2] = p[2 * stride];
  r[3] = p[3 * stride];
  return r;
}

// 16-byte copy helper for staging (uint4 keeps the access a single dwordx4).
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

// A 16-byte store of a streamed output that the kernel does not read back, with the nontemporal
// hint: it leaves the caches to the inputs and to the small records a later launch reads. Used where
// a wave writes whole 128-byte rows (the full-batch read-out); for 8-byte pieces, and for the
// chunked scans' O tiles, the hint measured slower.
typedef unsigned u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void st16_out(void* p, uint4 v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4_nt, v), reinterpret_cast<u32x4_nt*>(p));
}
// A 16-byte load with the nontemporal hint, for input read once.
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p)));
}

}  // namespace ttt
