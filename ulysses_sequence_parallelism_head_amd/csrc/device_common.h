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

// acc + (low bf16 of w) + (high bf16 of w), one v_dot2 with ones
__device__ __forceinline__ float sum_bf16x2(uint32_t w, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, 0x3f803f80u), acc,
                                         false);
}

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

// Combine a value with the one held by the lane 32 positions away (the other
// half-wave), without going through LDS: v_permlane32_swap returns the two
// halves exchanged, so each lane sees {x[l], x[l ^ 32]} in its two results.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Lower bound of the keys row t may see in a packed sequence of documents:
// the first position of t's document, clamped to [0, t] so that no value of
// the array can move an index out of its range.
__device__ __forceinline__ int doc_lower(const int32_t* row_starts, int t) {
  return min(max(row_starts[t], 0), t);
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

// ---- row-major tiles with XOR-swizzled 16-byte chunks
//
// A tile row holds D bf16 (D/8 chunks of 16 bytes).  Chunk c of row r is
// stored at physical chunk c ^ rm_swz(r).  gfx950's LDS has 64 banks (256
// bytes per pass); a 16-byte read is serviced 16 lanes per pass and an
// 8-byte read 32 lanes per pass.  The swizzle makes every access pattern of
// the kernels hit 64 distinct banks per pass:
//  * 16-byte row reads, 16 lanes on 16 consecutive rows, same logical chunk
//    (an MFMA operand whose rows are on the lanes);
//  * transposing reads (ds_read_b64_tr_b16), 32 lanes on 4 aligned rows x 64
//    bytes;
//  * the staging writes, 16 lanes on consecutive chunks.
// D = 128: rows are 256 bytes (one pass), all 4 chunk-index bits are
// swizzled; D = 64: two 128-byte rows share a pass.
template <int ROW_BYTES>
__device__ __forceinline__ int rm_swz(int r) {
  if (ROW_BYTES >= 256) return ((r & 3) << 2) | ((r >> 2) & 3);
  return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

template <int ROW_BYTES>
__device__ __forceinline__ int rm_off(int r, int chunk) {
  return r * ROW_BYTES + ((chunk ^ rm_swz<ROW_BYTES>(r)) << 4);
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
template <int ROW_BYTES>
__device__ __forceinline__ u32x4 tr_operand(const uint8_t* tile, int r0, int col0, int lane) {
  const int hh = lane >> 5;
  // the swizzle depends on the low four row bits only, so the 16-row-aligned
  // r0 is a plain byte offset (an immediate when r0 is a constant)
  const int rr = 4 * hh + ((lane & 15) >> 2);
  const int col = col0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int sub = (col & 7) * 2;                    // byte offset inside the 16-byte chunk (0 or 8)
  const uint8_t* t = tile + r0 * ROW_BYTES + sub;
  const u32x2 a = ds_read_tr16_b64(t + rm_off<ROW_BYTES>(rr, col >> 3));
  const u32x2 b = ds_read_tr16_b64(t + rm_off<ROW_BYTES>(rr + 8, col >> 3));
  return u32x4{a[0], a[1], b[0], b[1]};
}

// The same operand with r0 inside the swizzled row index.  Identical
// addresses; for kernels at the edge of their register budget this form
// lets the compiler recompute addresses instead of keeping one per 16-row
// block live across the loop (in dkdv the folded form parks them in
// accumulator registers and costs more moves than it saves adds).
template <int ROW_BYTES>
__device__ __forceinline__ u32x4 tr_operand_rows(const uint8_t* tile, int r0, int col0, int lane) {
  const int hh = lane >> 5;
  const int r = r0 + 4 * hh + ((lane & 15) >> 2);
  const int col = col0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int sub = (col & 7) * 2;
  const u32x2 a = ds_read_tr16_b64(tile + rm_off<ROW_BYTES>(r, col >> 3) + sub);
  const u32x2 b = ds_read_tr16_b64(tile + rm_off<ROW_BYTES>(r + 8, col >> 3) + sub);
  return u32x4{a[0], a[1], b[0], b[1]};
}

// ---- instruction scheduling hints
//
// Order the LDS reads and MFMAs of the enclosing basic block as a software
// pipeline: AHEAD reads first, then alternating pairs of MFMAs and pairs of
// reads, then the remaining MFMAs (N reads feeding N MFMAs in total).  The
// compiler's latency model treats LDS reads as short and otherwise issues
// them only two ahead of their use.
template <int AHEAD, int N>
__device__ __forceinline__ void pipeline_reads_mfma() {
  constexpr int kMaskMfma = 0x008, kMaskDsRead = 0x100;
  __builtin_amdgcn_sched_group_barrier(kMaskDsRead, AHEAD, 0);
#pragma unroll
  for (int i = 0; i < (N - AHEAD) / 2; ++i) {
    __builtin_amdgcn_sched_group_barrier(kMaskMfma, 2, 0);
    __builtin_amdgcn_sched_group_barrier(kMaskDsRead, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kMaskMfma, AHEAD, 0);
}

// The same for LDS reads that each feed two MFMAs (an operand shared by two
// accumulators): AHEAD reads first, then two MFMAs and one read at a time,
// then the last 2 * AHEAD MFMAs (N reads, 2N MFMAs).
template <int AHEAD, int N>
__device__ __forceinline__ void pipeline_reads_mfma2() {
  constexpr int kMaskMfma = 0x008, kMaskDsRead = 0x100;
  __builtin_amdgcn_sched_group_barrier(kMaskDsRead, AHEAD, 0);
#pragma unroll
  for (int i = 0; i < N - AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(kMaskMfma, 2, 0);
    __builtin_amdgcn_sched_group_barrier(kMaskDsRead, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kMaskMfma, 2 * AHEAD, 0);
}

// Transposed operands (two LDS reads each) that each feed two MFMAs: reads
// for AHEAD operands first, then two MFMAs and one operand's two reads at a
// time, then the last 2 * AHEAD MFMAs (2N reads, 2N MFMAs).
template <int AHEAD, int N>
__device__ __forceinline__ void pipeline_tr_reads_mfma2() {
  constexpr int kMaskMfma = 0x008, kMaskDsRead = 0x100;
  __builtin_amdgcn_sched_group_barrier(kMaskDsRead, 2 * AHEAD, 0);
#pragma unroll
  for (int i = 0; i < N - AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(kMaskMfma, 2, 0);
    __builtin_amdgcn_sched_group_barrier(kMaskDsRead, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kMaskMfma, 2 * AHEAD, 0);
}

// The same for MFMAs whose A operand takes two LDS reads (the transposing
// reads): reads for AHEAD MFMAs first, then one MFMA and its two reads at a
// time, then the last AHEAD MFMAs (2N reads, N MFMAs).
template <int AHEAD, int N>
__device__ __forceinline__ void pipeline_tr_reads_mfma() {
  constexpr int kMaskMfma = 0x008, kMaskDsRead = 0x100;
  __builtin_amdgcn_sched_group_barrier(kMaskDsRead, 2 * AHEAD, 0);
#pragma unroll
  for (int i = 0; i < N - AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(kMaskMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kMaskDsRead, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kMaskMfma, AHEAD, 0);
}

// ---- direct global -> LDS staging (buffer loads with the LDS destination)
//
// One buffer_load ... lds instruction moves 16 (or 4) bytes per lane from
// global memory straight into LDS, lane l landing at (wave-uniform LDS base
// in M0) + 16*l (4*l), without passing through registers.  Offsets at or
// beyond the buffer resource's byte size read as zero, which pads sequence
// tails for free.
//
// The instructions are issued from inline assembly, out of the compiler's
// sight: it would otherwise make every later LDS read it cannot prove
// disjoint (transposing reads carry no alias information) wait for all
// outstanding DMA, including the prefetch into the other staging buffer.
// Callers therefore synchronise by hand: wait_vmem() and a workgroup barrier
// before the staged data is read, and a barrier before a buffer is refilled.
// M0 is saved and restored around each instruction, and one wait state
// separates the M0 write from the load that reads it.
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t* lds_u8_ptr;

// Buffer resource for a raw byte range [base, base + bytes) (gfx9 layout:
// 48-bit base, stride 0, byte size, default format word).
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = int(uint32_t(a));
  r[1] = int(uint32_t(a >> 32) & 0xffffu);
  r[2] = int(bytes);
  r[3] = 0x00020000;
  return r;
}

// The resource and the LDS base are wave-uniform by construction; reading
// them through the first lane puts them in scalar registers as the
// instruction requires.
__device__ __forceinline__ i32x4 uniform_rsrc(const i32x4 r) {
  i32x4 u;
  u[0] = __builtin_amdgcn_readfirstlane(r[0]);
  u[1] = __builtin_amdgcn_readfirstlane(r[1]);
  u[2] = __builtin_amdgcn_readfirstlane(r[2]);
  u[3] = __builtin_amdgcn_readfirstlane(r[3]);
  return u;
}

__device__ __forceinline__ uint32_t lds_addr(uint8_t* lds) {
  // the low 32 bits of a flat address in the LDS aperture are the LDS offset
  // (an address-space cast would add a null check to every call)
  return __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>(lds)));
}

// 4 bytes per lane: global rsrc + voffset -> LDS lds + 4 * lane
__device__ __forceinline__ void dma4(const i32x4 rsrc, uint8_t* lds, int voffset) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr(lds)), "v"(voffset), "s"(uniform_rsrc(rsrc))
      : "memory");
}

// Wait until this wave's outstanding global loads (including the LDS DMA)
// have landed: s_waitcnt vmcnt(0), expcnt and lgkmcnt left at their maxima
// (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).  The
// builtin, unlike an asm statement, tells the compiler's wait-count tracking
// that every earlier load is complete, so it inserts no vmcnt wait of its
// own in the loop that follows (one that would also stall on the prefetch).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// One 16-byte-per-lane load: rsrc + vo[0] into LDS m0[0] + 16 * lane.
__device__ __forceinline__ void dma16x1(const i32x4 rsrc, const uint32_t (&m0)[1], const int (&vo)[1]) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0[0]), "v"(vo[0]), "s"(uniform_rsrc(rsrc))
      : "memory");
}

// Two or four 16-byte-per-lane loads in one asm statement (one M0 save and
// restore): load u reads rsrc + vo[u] into LDS m0[u] + 16 * lane.
__device__ __forceinline__ void dma16x2(const i32x4 rsrc, const uint32_t (&m0)[2], const int (&vo)[2]) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %3, %5, 0 offen lds\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %4, %5, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0[0]), "s"(m0[1]), "v"(vo[0]), "v"(vo[1]), "s"(uniform_rsrc(rsrc))
      : "memory");
}

__device__ __forceinline__ void dma16x4(const i32x4 rsrc, const uint32_t (&m0)[4], const int (&vo)[4]) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %5, %9, 0 offen lds\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %6, %9, 0 offen lds\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %7, %9, 0 offen lds\n\t"
      "s_mov_b32 m0, %4\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %8, %9, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0[0]), "s"(m0[1]), "s"(m0[2]), "s"(m0[3]), "v"(vo[0]), "v"(vo[1]), "v"(vo[2]), "v"(vo[3]),
        "s"(uniform_rsrc(rsrc))
      : "memory");
}

// DMA a ROWS x D bf16 tile, rows row0.. of a row-major tensor whose rows are
// row_stride_bytes apart, into the swizzled LDS layout of rm_off.  `rows_ok`
// rows hold data; the rest of the tile is zero-filled.  Every wave of the
// workgroup calls this with its wave index; together they cover the tile.
// Load u of this wave writes the tile's 1 KB block u * NWAVES + wave, 16
// bytes per lane, at the row and (swizzled) chunk that block position holds.
template <int D, int ROWS, int NWAVES>
__device__ __forceinline__ void dma_tile(uint8_t* lds_tile, const uint16_t* row0, int row_stride_bytes, int rows_ok,
                                         int wave, int lane) {
  constexpr int NC = D / 8;                      // 16-byte chunks per row
  constexpr int ROW_BYTES = 2 * D;
  constexpr int PER_WAVE = ROWS * NC / (64 * NWAVES);
  static_assert(ROWS * NC % (64 * NWAVES) == 0, "tile must split evenly across the waves");
  static_assert(PER_WAVE == 1 || PER_WAVE == 2 || PER_WAVE == 4, "one, two or four loads per wave");
  const i32x4 rsrc = buffer_rsrc(row0, uint32_t(rows_ok > 0 ? rows_ok : 0) * uint32_t(row_stride_bytes));
  const uint32_t base = lds_addr(lds_tile);
  uint32_t m0[PER_WAVE];
  int vo[PER_WAVE];
#pragma unroll
  for (int u = 0; u < PER_WAVE; ++u) {
    const int blk = u * NWAVES + wave;
    const int pos = blk * 64 + lane;             // physical chunk position
    const int r = pos / NC;
    const int c = (pos % NC) ^ rm_swz<ROW_BYTES>(r);
    m0[u] = base + uint32_t(blk) * 1024u;
    vo[u] = r * row_stride_bytes + c * 16;
  }
  if constexpr (PER_WAVE == 4) dma16x4(rsrc, m0, vo);
  else if constexpr (PER_WAVE == 2) dma16x2(rsrc, m0, vo);
  else dma16x1(rsrc, m0, vo);
}

}  // namespace ulysses
