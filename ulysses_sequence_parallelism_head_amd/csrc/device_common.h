// device_common.h -- vector types and small device helpers shared by the
// gfx950 kernels of this library (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ulysses {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Round two floats to bfloat16 (nearest, ties to even) and pack them
// little-endian into one 32-bit word: `lo` in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  bf16x2 b = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

// Widen the bfloat16 halves of a packed word to float (exact).
__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 32x32x16 bf16 matrix-core product, fp32 accumulate:  C += A * B.
// Lane l holds row (l % 32) of A and column (l % 32) of B, 8 contraction
// elements each (the same 8 contraction slots for A and B); C's lane l holds
// column (l % 32) and rows (i/4)*8 + 4*(l/32) + i%4 for i = 0..15.
__device__ __forceinline__ f32x16 mfma32x32x16(const u32x4 a, const u32x4 b, const f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Exchange a value with the lane 32 positions away (the other half-wave).
__device__ __forceinline__ float swap_halves(float x) {
  return __shfl_xor(x, 32, 64);
}

// Round-up division by an invariant 32-bit divisor (Granlund & Montgomery,
// "Division by Invariant Integers using Multiplication", PLDI 1994):
// q = (mulhi(n, m) + n) >> s, exact for every 32-bit n.
struct FastDiv {
  uint32_t d, m, s;
};

__host__ inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t s = 0;
  while ((uint64_t(1) << s) < d) ++s;              // s = ceil(log2 d)
  f.s = s;
  f.m = uint32_t(((uint64_t(1) << 32) * ((uint64_t(1) << s) - d)) / d + 1);
  return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
  uint64_t t = __umulhi(n, f.m);
  return uint32_t((t + n) >> f.s);
}

// ---- transposed operand tiles in LDS
//
// A lane holds its 32-slot share of scores (or probabilities / dS) for keys
// (or query rows) (i/4)*8 + 4*(l/32) + i%4, i = 0..15 (the MFMA accumulator
// row order).  To use them directly as an MFMA operand, the matching
// transposed tile (V^T, K^T, Q^T or dO^T) stores element x of a 32-slice at
// slot tslot(x): bits 2 and 3 swapped, so a lane's 8 values for a 16-wide
// contraction slice sit in 8 consecutive slots.
__device__ __forceinline__ int tslot(int x32) {
  return (x32 & ~12) | ((x32 & 4) << 1) | ((x32 & 8) >> 1);
}

// Byte offset of 16-byte chunk `chunk` (0..7) of row r in a transposed tile
// with 64 slots (128 B) per row.  Chunks are XOR-swizzled by row so that the
// MFMA operand reads (8 consecutive rows, same chunk) and the transposing
// staging writes (rows 8 apart) both spread over all banks.
__device__ __forceinline__ int t64_off(int r, int chunk) {
  const int swz = (r & 7) ^ ((r >> 3) & 7);
  return r * 128 + ((chunk ^ swz) << 4);
}

// Same for a tile with 32 slots (64 B) per row, chunks 0..3.
__device__ __forceinline__ int t32_off(int r, int chunk) {
  const int swz = ((r >> 1) ^ (r >> 3)) & 3;
  return r * 64 + ((chunk ^ swz) << 4);
}

// Transpose a 4-row x 8-column block of bf16 (rows[e] = 8 columns of row e)
// into 8 column words of 4 rows each: out[c] = {row0[c] | row1[c] << 16,
// row2[c] | row3[c] << 16}.
__device__ __forceinline__ u32x2 transpose_col(const u32x4* rows, int c) {
  const int w = c >> 1;
  uint32_t x0, x1, x2, x3;
  if (c & 1) {
    x0 = rows[0][w] >> 16; x1 = rows[1][w] >> 16; x2 = rows[2][w] >> 16; x3 = rows[3][w] >> 16;
  } else {
    x0 = rows[0][w] & 0xffffu; x1 = rows[1][w] & 0xffffu; x2 = rows[2][w] & 0xffffu; x3 = rows[3][w] & 0xffffu;
  }
  return u32x2{x0 | (x1 << 16), x2 | (x3 << 16)};
}

// ---- row-major tiles with XOR-swizzled 16-byte chunks
//
// A tile row holds D bf16 (D/8 chunks of 16 bytes).  Chunk c of row r is
// stored at physical chunk c ^ rm_swz(r) (low three bits only), where
// rm_swz takes all 8 values on any 8 consecutive rows and the 4 values of one
// parity on any 4 aligned rows.  Then
//  * 16-byte row reads by 8 lanes on 8 consecutive rows (an MFMA operand whose
//    rows are on the lanes) hit 8 distinct bank groups, and
//  * transposing reads (ds_read_b64_tr_b16), where 16 lanes cover 4 aligned
//    rows x 32 bytes, hit 8 distinct bank groups too.
__device__ __forceinline__ int rm_swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

__device__ __forceinline__ int rm_off(int r, int chunk, int row_bytes) {
  return r * row_bytes + ((chunk ^ rm_swz(r)) << 4);
}

// gfx950 transposing LDS read.  Within each group of 16 lanes, lane i returns
// element (i % 4) of the 8-byte chunks supplied by lanes 4e + i/4, e = 0..3:
// the 16 lanes together read 4 rows x 16 columns and each lane receives one
// column (4 rows).
__device__ __forceinline__ u32x2 ds_read_tr16_b64(const uint8_t* lds) {
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(const_cast<uint8_t*>(lds)));
  return __builtin_bit_cast(u32x2, r);
}

// MFMA A operand (row m = l%32 of a 32-row block, 8 contraction slots) taken
// transposed from a row-major swizzled tile T[rows][D]: lane l gets
// T[r][col] for col = col0 + l%32 and the 8 rows
//   r0 + 4*(l/32) + {0,1,2,3}  and  r0 + 8 + 4*(l/32) + {0,1,2,3},
// i.e. exactly the row order in which a lane holds its share of an MFMA
// accumulator column (rows (i/4)*8 + 4*(l/32) + i%4, i = 8k .. 8k+7).
// r0 must be a multiple of 16 and col0 a multiple of 32.
__device__ __forceinline__ u32x4 tr_operand(const uint8_t* tile, int row_bytes, int r0, int col0, int lane) {
  const int hh = lane >> 5;
  const int r = r0 + 4 * hh + ((lane & 15) >> 2);
  const int col = col0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int sub = (col & 7) * 2;                    // byte offset inside the 16-byte chunk (0 or 8)
  const u32x2 a = ds_read_tr16_b64(tile + rm_off(r, col >> 3, row_bytes) + sub);
  const u32x2 b = ds_read_tr16_b64(tile + rm_off(r + 8, col >> 3, row_bytes) + sub);
  return u32x4{a[0], a[1], b[0], b[1]};
}

}  // namespace ulysses
