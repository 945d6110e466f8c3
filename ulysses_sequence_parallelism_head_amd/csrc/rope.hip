// rope.hip -- the first all-to-all fused with the rotary position embedding
// of Q or K at global positions (one HBM pass instead of two).
//
// Source: the ms-swift page ("ms-swift性能优化：Ulysses并行技术降低长文本显存",
// section "6. 使用建议与避坑指南", troubleshooting table) traces repeated
// tokens to a rotary encoding that ignores the shard's offset in the
// sequence; with contiguous shards ([ALST] "Paralelismul de Secvență Ulysses:
// Antrenarea modelelor AI cu contexte de un milion de token-uri", section
// "Mecanismul de funcționare Ulysses", step 1) rank i's token s is at global
// position i * n_local + s.  The rotation pairs dimension d with d + D/2:
//   theta_d = (pos / scale) * base^(-2d/D)
//   out[d] = x[d] cos - x[d+D/2] sin,  out[d+D/2] = x[d+D/2] cos + x[d] sin
// and the exchange is that of repack.hip (seq2head).
//
// Design: one wave per token.  All H heads of a token share the D/2 angles:
// lane a < D/2 computes angle a once (frequency in double precision, angle
// reduced to [-pi, pi] in double, then a double sine/cosine), and the lanes
// fetch the values they need with cross-lane reads.  The token's H*D
// elements are read in 16-byte chunks, 64 lanes (one contiguous 1 KB span)
// per step; a chunk of the first half of a head and its partner in the
// second half sit cph/2 lanes apart (cph = chunks per head), so the pair is
// exchanged with one lane-xor shuffle per 32-bit word.  Results are rounded
// once to the output type and written to the head-sharded layout (runs of
// H/P heads stay contiguous).  Streaming, non-temporal loads and stores.
#include <math.h>

#include "device_common.h"
#include "internal.h"

namespace ulysses {

namespace {

constexpr int kRopeWaves = 4;                 // tokens per workgroup (one per wave)

struct RopeParams {
  const void* src;
  void* dst;
  int64_t tokens;        // P * B * n_local
  int32_t P, B, n_local, H, D;
  double base;           // rotary base
  double scale;          // linear position scaling factor
};

// ES = element size (2: bf16, 4: fp32)
template <int ES, int D>
__global__ __launch_bounds__(64 * kRopeWaves) void seq2head_rope_kernel(const RopeParams p) {
  constexpr int EPC = 16 / ES;               // elements per 16-byte chunk
  constexpr int CPH = D * ES / 16;           // chunks per head (divides 64)
  constexpr int HALF = D / 2;
  static_assert(64 % CPH == 0 && CPH % 2 == 0, "chunk layout");
  const int lane = threadIdx.x & 63;
  const int64_t tok = int64_t(blockIdx.x) * kRopeWaves + (threadIdx.x >> 6);
  if (tok >= p.tokens) return;               // whole wave; no workgroup barrier below

  // token -> (shard i, batch b, local position s); global position i*nl + s
  const int s = int(tok % p.n_local);
  const int64_t ib = tok / p.n_local;
  const int b = int(ib % p.B);
  const int i = int(ib / p.B);
  const int64_t pos = int64_t(i) * p.n_local + s;

  // this lane's angle a = lane % (D/2)
  float cs, sn;
  {
    const int a = lane % HALF;
    const double inv_freq = exp2(-(2.0 * a / D) * log2(p.base));
    const double theta = (double(pos) / p.scale) * inv_freq;
    // reduce to [-pi, pi]: 2*pi split in two doubles so k*2pi is exact enough
    constexpr double kTwoPiHi = 6.283185307179586;
    constexpr double kTwoPiLo = 2.4492935982947064e-16;
    const double k = rint(theta * (1.0 / kTwoPiHi));
    double r = fma(-k, kTwoPiHi, theta);
    r = fma(-k, kTwoPiLo, r);
    double sd, cd;
    sincos(r, &sd, &cd);
    cs = float(cd);
    sn = float(sd);
  }
  // chunk c of a head (c = lane % CPH for every step) covers dims c*EPC ..
  const int c = lane % CPH;
  const bool first_half = c < CPH / 2;
  const int a0 = (c * EPC) % HALF;
  float cv[EPC], sv[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) {
    cv[e] = __shfl(cs, a0 + e, 64);
    sv[e] = __shfl(sn, a0 + e, 64);
  }

  const int hp = p.H / p.P;
  const int64_t n = int64_t(p.P) * p.n_local;
  const int chunks = p.H * CPH;
  const u32x4* src = static_cast<const u32x4*>(p.src) + tok * chunks;
  for (int g0 = 0; g0 < chunks; g0 += 64) {
    const int gc = g0 + lane;
    const bool live = gc < chunks;           // a head's chunks are all live or all not
    u32x4 x = live ? __builtin_nontemporal_load(src + gc) : u32x4{0, 0, 0, 0};
    u32x4 y;
#pragma unroll
    for (int w = 0; w < 4; ++w) y[w] = __shfl_xor(x[w], CPH / 2, 64);
    float xf[EPC], yf[EPC];
    if (ES == 2) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        xf[2 * w] = bf16lo_to_f32(x[w]);
        xf[2 * w + 1] = bf16hi_to_f32(x[w]);
        yf[2 * w] = bf16lo_to_f32(y[w]);
        yf[2 * w + 1] = bf16hi_to_f32(y[w]);
      }
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        xf[w] = __uint_as_float(x[w]);
        yf[w] = __uint_as_float(y[w]);
      }
    }
    // first half: x cos - y sin (y = second-half partner); second half: x cos + y sin
    float o[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) o[e] = fmaf(first_half ? -yf[e] : yf[e], sv[e], xf[e] * cv[e]);
    u32x4 out;
    if (ES == 2) {
#pragma unroll
      for (int w = 0; w < 4; ++w) out[w] = pack_bf16x2(o[2 * w], o[2 * w + 1]);
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) out[w] = __float_as_uint(o[w]);
    }
    if (live) {
      const int h = gc / CPH;
      const int j = h / hp;
      const int hl = h - j * hp;
      // dst[j][b][i*nl + s][hl][chunk c]
      const int64_t row = (int64_t(j) * p.B + b) * n + int64_t(i) * p.n_local + s;
      u32x4* dst = static_cast<u32x4*>(p.dst) + (row * hp + hl) * CPH + c;
      __builtin_nontemporal_store(out, dst);
    }
  }
}

template <int ES>
hipError_t launch_es(const RopeParams& p, hipStream_t stream) {
  const int64_t blocks = (p.tokens + kRopeWaves - 1) / kRopeWaves;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (p.D == 128)
    hipLaunchKernelGGL((seq2head_rope_kernel<ES, 128>), dim3(blocks), dim3(64 * kRopeWaves), 0, stream, p);
  else
    hipLaunchKernelGGL((seq2head_rope_kernel<ES, 64>), dim3(blocks), dim3(64 * kRopeWaves), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_seq2head_rope(const void* src, void* dst, int32_t P, int32_t B, int32_t n_local, int32_t H,
                                int32_t D, int elem_bytes, double base, double scale, hipStream_t stream) {
  RopeParams p;
  p.src = src;
  p.dst = dst;
  p.tokens = int64_t(P) * B * n_local;
  p.P = P;
  p.B = B;
  p.n_local = n_local;
  p.H = H;
  p.D = D;
  p.base = base;
  p.scale = scale;
  return elem_bytes == 2 ? launch_es<2>(p, stream) : launch_es<4>(p, stream);
}

}  // namespace ulysses
