// proj.hip -- the projections on either side of the exchanges, each fused
// with its exchange: the QKV projection writes straight into the
// head-sharded layout of the first all-to-all, and the output projection
// reads the attention output straight from the head-sharded layout of the
// second.
//
// Source: [ALST] "Paralelismul de Secvență Ulysses: Antrenarea modelelor AI
// cu contexte de un milion de token-uri", section "Mecanismul de funcționare
// Ulysses", steps 2-3 (each rank projects Q, K, V for its own sequence
// shard, then the first exchange) and 5-6 (the second exchange, then each
// rank's output projection of its shard); [HFSUM] "Ulysses 序列平行化的原理".
// A projection is x @ W^T with W laid out [out features][in features]; the
// fused QKV weight stacks the Hq query heads, the Hkv key heads and the Hkv
// value heads (D features each); a token's attention output is its Hq heads
// concatenated in head order.
//
// Design (bf16 inputs, fp32 accumulation, one rounding to bf16): a workgroup
// of 8 waves computes a 256-feature x 256-token tile of the transposed
// product C^T = W X^T on the 32x32x16 bf16 matrix cores, so that each lane
// owns one token and 16 of its features per accumulator (4 runs of 4
// consecutive features, 8 contiguous output bytes each).  Each wave holds a
// 128-feature x 64-token block (4 x 2 accumulators: 6 operand reads per 8
// matrix instructions), and scheduling hints keep two contraction steps of
// operand reads ahead of the matrix instructions.  The 64-wide contraction slabs of W and of the token rows
// are DMA'd into swizzled row-major LDS tiles (the attention kernels'
// layout) and double-buffered, one barrier per slab.  A token tile never
// crosses a shard boundary, so its rows are equally spaced in memory in
// both layouts: in the head-sharded attention output a token's Hq*D
// features are P runs of (Hq/P)*D, and a 64-wide slab always lies inside
// one run.  Each XCD takes a contiguous range of tiles (workgroups are
// dealt to the 8 XCDs in turn), walked in groups of 8 token tiles with the
// token tile fastest: the 32 workgroups resident on an XCD then cover about
// 8 token tiles x 4 feature tiles and, moving through the contraction
// together, share each slab of them through the XCD's L2 (weights and
// tokens both re-read about 4-8 times less from memory than with one of
// them varying fastest).
#include "device_common.h"
#include "internal.h"

namespace ulysses {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTileF = 256;          // features per workgroup
constexpr int kTileT = 256;          // tokens per workgroup
constexpr int kXcds = 8;
constexpr int kGroupT = 8;           // token tiles per group of the tile order
constexpr int kSlab = 64;            // contraction elements per stage
constexpr int kRowBytes = 2 * kSlab;
constexpr int kTileBytes = kTileF * kRowBytes;       // 32 KB (the token tile is the same size)
constexpr int kStage = 2 * kTileBytes;

struct ProjParams {
  const uint16_t* w;   // [N][K]
  const uint16_t* a;   // token rows: x [P][B][nl][K] (QKV) or o [P][B][n][Hq/P][D] (output)
  uint16_t* out0;      // QKV: q [P][B][n][Hq/P][D]; output: y [P][B][nl][N]
  uint16_t* out1;      // QKV: k [P][B][n][Hkv/P][D]
  uint16_t* out2;      // QKV: v
  int32_t P, B, nl, K, N;
  int32_t Hq, Hkv, D;
  int32_t seg;         // output projection: (Hq/P) * D, the run of one head shard in a token row
  int32_t t_tiles;     // ceil(nl / kTileT)
  int32_t f_tiles;     // ceil(N / kTileF)
};

// Scheduling hints for one slab (24 operand reads, 32 matrix instructions):
// 12 reads (two contraction steps) issued ahead, then 4 instructions per 2
// reads, then the last instructions.
__device__ __forceinline__ void proj_pipeline() {
  constexpr int kMaskMfma = 0x008, kMaskDsRead = 0x100;
  __builtin_amdgcn_sched_group_barrier(kMaskDsRead, 12, 0);
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    __builtin_amdgcn_sched_group_barrier(kMaskMfma, 4, 0);
    __builtin_amdgcn_sched_group_barrier(kMaskDsRead, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kMaskMfma, 8, 0);
}

// DMA contraction slab k0 .. k0+63 of the weight tile and of the token tile.
template <int MODE>
__device__ __forceinline__ void proj_issue(uint8_t* stage, const ProjParams& p, int f0, int rows_f, int i, int b,
                                           int s0, int rows_t, int k0, int wave, int lane) {
  dma_tile<kSlab, kTileF, kWaves>(stage, p.w + int64_t(f0) * p.K + k0, p.K * 2, rows_f, wave, lane);
  const uint16_t* row0;
  int stride;
  if (MODE == 0) {
    row0 = p.a + ((int64_t(i) * p.B + b) * p.nl + s0) * p.K + k0;
    stride = p.K * 2;
  } else {
    const int j = k0 / p.seg;                    // head shard holding these features
    const int64_t n = int64_t(p.P) * p.nl;
    row0 = p.a + ((int64_t(j) * p.B + b) * n + int64_t(i) * p.nl + s0) * p.seg + (k0 - j * p.seg);
    stride = p.seg * 2;
  }
  dma_tile<kSlab, kTileT, kWaves>(stage + kTileBytes, row0, stride, rows_t, wave, lane);
}

template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void proj_kernel(const ProjParams p) {
  __shared__ __attribute__((aligned(128))) uint8_t smem[2 * kStage];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // workgroup w runs on XCD w % 8: give each XCD a contiguous range of tiles
  const int nblk = int(gridDim.x);
  const int per_xcd = (nblk + kXcds - 1) / kXcds;
  const int xcd = int(blockIdx.x) % kXcds;
  const int full = nblk - (per_xcd - 1) * kXcds;     // XCDs that get per_xcd tiles (the rest per_xcd - 1)
  const int pos = int(blockIdx.x) / kXcds;
  const int tile = xcd < full ? xcd * per_xcd + pos : full * per_xcd + (xcd - full) * (per_xcd - 1) + pos;
  // groups of kGroupT token tiles (the last one may be smaller), token tile fastest
  const int tt_all = p.t_tiles * p.B * p.P;
  const int group = tile / (kGroupT * p.f_tiles);
  const int gt = min(kGroupT, tt_all - group * kGroupT);
  const int in_group = tile - group * kGroupT * p.f_tiles;
  const int ft = in_group / gt;
  const int tt = group * kGroupT + in_group % gt;      // token tile = (i, b, st)
  const int st = tt % p.t_tiles;
  const int ib = tt / p.t_tiles;
  const int b = ib % p.B;
  const int i = ib / p.B;
  const int f0 = ft * kTileF;
  const int s0 = st * kTileT;
  const int rows_f = min(kTileF, p.N - f0);
  const int rows_t = min(kTileT, p.nl - s0);
  const int fw = (wave & 1) * 128;               // this wave's features and tokens in the tile
  const int tw = (wave >> 1) * 64;

  f32x16 acc[4][2];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 2; ++c) acc[r][c] = f32x16{};

  const int nslab = p.K / kSlab;
  proj_issue<MODE>(smem, p, f0, rows_f, i, b, s0, rows_t, 0, wave, lane);
  wait_vmem();
  __syncthreads();

  auto slab = [&](int it, uint8_t* cur, uint8_t* nxt) {
    if (it + 1 < nslab) proj_issue<MODE>(nxt, p, f0, rows_f, i, b, s0, rows_t, (it + 1) * kSlab, wave, lane);
    const uint8_t* ws = cur;
    const uint8_t* xs = cur + kTileBytes;
#pragma unroll
    for (int kk = 0; kk < kSlab / 16; ++kk) {
      u32x4 a[4], x[2];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        a[r] = *reinterpret_cast<const u32x4*>(ws + rm_off<kRowBytes>(fw + 32 * r + l32, 2 * kk + hh));
#pragma unroll
      for (int c = 0; c < 2; ++c)
        x[c] = *reinterpret_cast<const u32x4*>(xs + rm_off<kRowBytes>(tw + 32 * c + l32, 2 * kk + hh));
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 2; ++c) acc[r][c] = mfma32x32x16(a[r], x[c], acc[r][c]);
    }
    proj_pipeline();
    wait_vmem();
    __syncthreads();
  };
  int it = 0;
  for (; it + 1 < nslab; it += 2) {
    slab(it, smem, smem + kStage);
    slab(it + 1, smem + kStage, smem);
  }
  if (it < nslab) slab(it, smem, smem + kStage);

  // ---- epilogue: lane = token, 4 runs of 4 consecutive features per accumulator
  const int64_t n = int64_t(p.P) * p.nl;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int s = s0 + tw + 32 * c + l32;
    if (s >= p.nl) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int f = f0 + fw + 32 * r + 8 * i4 + 4 * hh;
        if (f >= p.N) continue;
        const u32x2 val{pack_bf16x2(acc[r][c][4 * i4], acc[r][c][4 * i4 + 1]),
                        pack_bf16x2(acc[r][c][4 * i4 + 2], acc[r][c][4 * i4 + 3])};
        uint16_t* dst;
        if (MODE == 0) {
          // feature -> (tensor, head, dim) -> head-sharded position of token (i, b, s)
          int h = f / p.D;
          const int dim = f - h * p.D;
          int H = p.Hq;
          uint16_t* base = p.out0;
          if (h >= p.Hq + p.Hkv) {
            h -= p.Hq + p.Hkv;
            H = p.Hkv;
            base = p.out2;
          } else if (h >= p.Hq) {
            h -= p.Hq;
            H = p.Hkv;
            base = p.out1;
          }
          const int hp = H / p.P;
          const int j = h / hp;
          dst = base + (((int64_t(j) * p.B + b) * n + int64_t(i) * p.nl + s) * hp + (h - j * hp)) * p.D + dim;
        } else {
          dst = p.out0 + ((int64_t(i) * p.B + b) * p.nl + s) * p.N + f;
        }
        *reinterpret_cast<u32x2*>(dst) = val;
      }
    }
  }
}

hipError_t launch(const ProjParams& p, int mode, hipStream_t stream) {
  const int64_t blocks = int64_t(p.f_tiles) * p.t_tiles * p.B * p.P;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (mode == 0) hipLaunchKernelGGL(proj_kernel<0>, dim3(blocks), dim3(kThreads), 0, stream, p);
  else hipLaunchKernelGGL(proj_kernel<1>, dim3(blocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qkv_proj_seq2head(const void* x, const void* w, void* q, void* k, void* v, int32_t P, int32_t B,
                                    int32_t n_local, int32_t hidden, int32_t Hq, int32_t Hkv, int32_t D,
                                    hipStream_t stream) {
  ProjParams p{};
  p.w = static_cast<const uint16_t*>(w);
  p.a = static_cast<const uint16_t*>(x);
  p.out0 = static_cast<uint16_t*>(q);
  p.out1 = static_cast<uint16_t*>(k);
  p.out2 = static_cast<uint16_t*>(v);
  p.P = P; p.B = B; p.nl = n_local; p.K = hidden; p.N = (Hq + 2 * Hkv) * D;
  p.Hq = Hq; p.Hkv = Hkv; p.D = D;
  p.seg = 0;
  p.t_tiles = (n_local + kTileT - 1) / kTileT;
  p.f_tiles = (p.N + kTileF - 1) / kTileF;
  return launch(p, 0, stream);
}

hipError_t launch_head2seq_out_proj(const void* o, const void* w_o, void* y, int32_t P, int32_t B, int32_t n_local,
                                    int32_t Hq, int32_t D, int32_t hidden, hipStream_t stream) {
  ProjParams p{};
  p.w = static_cast<const uint16_t*>(w_o);
  p.a = static_cast<const uint16_t*>(o);
  p.out0 = static_cast<uint16_t*>(y);
  p.P = P; p.B = B; p.nl = n_local; p.K = Hq * D; p.N = hidden;
  p.Hq = Hq; p.Hkv = 0; p.D = D;
  p.seg = (Hq / P) * D;
  p.t_tiles = (n_local + kTileT - 1) / kTileT;
  p.f_tiles = (p.N + kTileF - 1) / kTileF;
  return launch(p, 1, stream);
}

}  // namespace ulysses
