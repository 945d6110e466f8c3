// attn_fwd_f32.hip -- exact softmax attention forward with logsumexp in
// float32 throughout (float32 inputs and output).
//
// Operation: [ALST] "Paralelismul de Secvență Ulysses: Antrenarea modelelor
// AI cu contexte de un milion de token-uri", section "Mecanismul de
// funcționare Ulysses", step 4.
//
// This is the full-precision path: no matrix cores (there is no fp32 input
// rounding to hide), plain VALU FMAs.  Two lanes (the two half-waves) share
// one query row, each holding half of the head dimension; a workgroup of two
// waves owns 64 rows of one query head and streams 32-key K/V tiles through
// LDS.  The online softmax works per tile: scores for 32 keys, one max, one
// rescale, then the weighted V accumulation.  With packed documents (a
// per-row lower bound on the keys) the tile loop starts at the tile holding
// the first row's bound.
#include "device_common.h"
#include "internal.h"

namespace ulysses {

namespace {

constexpr int kF32Threads = 128;
constexpr int kF32Rows = 64;      // rows per workgroup
constexpr int kF32Keys = 32;      // keys per tile

struct F32Params {
  const float* q;
  const float* k;
  const float* v;
  const uint8_t* valid;
  const int32_t* doc_start;   // [B][n] first position of each row's document, or null
  float* o;
  float* lse;
  int32_t B, n, Hq, Hkv, g;
  int32_t n_rblocks;
  float scale;
  int32_t causal;
};

template <int D, bool HAS_MASK, bool DOCS>
__global__ __launch_bounds__(kF32Threads) void attn_fwd_f32_kernel(const F32Params p) {
  constexpr int DH = D / 2;
  __shared__ float ks[kF32Keys][D + 1];
  __shared__ float vs[kF32Keys][D + 1];
  __shared__ uint8_t okey[kF32Keys];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int hh = lane >> 5;

  const int per_blk = p.Hq * p.B;
  const int rb = p.n_rblocks - 1 - int(blockIdx.x) / per_blk;   // longest-first
  const int rem = int(blockIdx.x) % per_blk;
  const int b = rem / p.Hq;
  const int head = rem % p.Hq;
  const int kvh = head / p.g;
  const int t = rb * kF32Rows + wave * 32 + (lane & 31);
  const int wg_last = min(rb * kF32Rows + kF32Rows, p.n) - 1;
  const int kend = p.causal ? wg_last + 1 : p.n;
  int kbeg = 0, lo_row = 0;
  if (DOCS) {
    const int32_t* rs = p.doc_start + int64_t(b) * p.n;
    kbeg = doc_lower(rs, rb * kF32Rows) / kF32Keys * kF32Keys;
    lo_row = t < p.n ? doc_lower(rs, t) : 0;
  }

  float qv[DH], acc[DH];
  {
    const bool ok = t < p.n;
    const float* qp = p.q + ((int64_t(b) * p.n + (ok ? t : 0)) * p.Hq + head) * D + hh * DH;
#pragma unroll
    for (int c = 0; c < DH; ++c) {
      qv[c] = ok ? qp[c] * p.scale : 0.f;
      acc[c] = 0.f;
    }
  }
  float m = -INFINITY, lsum = 0.f;

  for (int k0 = kbeg; k0 < kend; k0 += kF32Keys) {
    __syncthreads();
    for (int e = tid; e < kF32Keys * D; e += kF32Threads) {
      const int r = e / D, c = e % D;
      const int key = k0 + r;
      float kx = 0.f, vx = 0.f;
      if (key < p.n) {
        const int64_t off = ((int64_t(b) * p.n + key) * p.Hkv + kvh) * D + c;
        kx = p.k[off];
        vx = p.v[off];
      }
      ks[r][c] = kx;
      vs[r][c] = vx;
    }
    if (tid < kF32Keys) {
      const int key = k0 + tid;
      okey[tid] = (key < p.n) && (!HAS_MASK || p.valid[int64_t(b) * p.n + key] != 0);
    }
    __syncthreads();

    float s[kF32Keys];
#pragma unroll
    for (int j = 0; j < kF32Keys; ++j) {
      float part = 0.f;
#pragma unroll
      for (int c = 0; c < DH; ++c) part = fmaf(qv[c], ks[j][hh * DH + c], part);
      s[j] = halves_sum(part);
    }
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < kF32Keys; ++j) {
      const int key = k0 + j;
      const bool ok = okey[j] && !(p.causal && key > t) && !(DOCS && key < lo_row);
      s[j] = ok ? s[j] : -INFINITY;
      mt = fmaxf(mt, s[j]);
    }
    const float m_new = fmaxf(m, mt);
    if (m_new == -INFINITY) continue;        // nothing visible yet for this row
    const float alpha = expf(m - m_new);     // m = -inf gives 0
    lsum *= alpha;
#pragma unroll
    for (int c = 0; c < DH; ++c) acc[c] *= alpha;
#pragma unroll
    for (int j = 0; j < kF32Keys; ++j) {
      const float pj = expf(s[j] - m_new);
      lsum += pj;
#pragma unroll
      for (int c = 0; c < DH; ++c) acc[c] = fmaf(pj, vs[j][hh * DH + c], acc[c]);
    }
    m = m_new;
  }

  if (t < p.n) {
    const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
    float* op = p.o + ((int64_t(b) * p.n + t) * p.Hq + head) * D + hh * DH;
#pragma unroll
    for (int c = 0; c < DH; ++c) op[c] = acc[c] * inv;
    if (hh == 0) p.lse[(int64_t(b) * p.Hq + head) * p.n + t] = lsum > 0.f ? m + logf(lsum) : -INFINITY;
  }
}

}  // namespace

hipError_t launch_attn_fwd_f32(const float* q, const float* k, const float* v, const uint8_t* valid,
                               const int32_t* doc_start, float* o, float* lse, const AttnShape& s,
                               hipStream_t stream) {
  F32Params p;
  p.q = q; p.k = k; p.v = v; p.valid = valid; p.doc_start = doc_start; p.o = o; p.lse = lse;
  p.B = s.B; p.n = int32_t(s.n); p.Hq = s.Hq; p.Hkv = s.Hkv; p.g = s.Hq / s.Hkv;
  p.n_rblocks = int32_t((s.n + kF32Rows - 1) / kF32Rows);
  p.scale = s.scale;
  p.causal = s.causal;
  const int64_t blocks = int64_t(p.n_rblocks) * p.Hq * p.B;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const bool m = valid != nullptr;
  const bool docs = doc_start != nullptr;
  if (s.D == 128) {
    if (docs) {
      if (m) hipLaunchKernelGGL((attn_fwd_f32_kernel<128, true, true>), dim3(blocks), dim3(kF32Threads), 0, stream, p);
      else hipLaunchKernelGGL((attn_fwd_f32_kernel<128, false, true>), dim3(blocks), dim3(kF32Threads), 0, stream, p);
    } else {
      if (m) hipLaunchKernelGGL((attn_fwd_f32_kernel<128, true, false>), dim3(blocks), dim3(kF32Threads), 0, stream, p);
      else hipLaunchKernelGGL((attn_fwd_f32_kernel<128, false, false>), dim3(blocks), dim3(kF32Threads), 0, stream, p);
    }
  } else {
    if (docs) {
      if (m) hipLaunchKernelGGL((attn_fwd_f32_kernel<64, true, true>), dim3(blocks), dim3(kF32Threads), 0, stream, p);
      else hipLaunchKernelGGL((attn_fwd_f32_kernel<64, false, true>), dim3(blocks), dim3(kF32Threads), 0, stream, p);
    } else {
      if (m) hipLaunchKernelGGL((attn_fwd_f32_kernel<64, true, false>), dim3(blocks), dim3(kF32Threads), 0, stream, p);
      else hipLaunchKernelGGL((attn_fwd_f32_kernel<64, false, false>), dim3(blocks), dim3(kF32Threads), 0, stream, p);
    }
  }
  return hipGetLastError();
}

}  // namespace ulysses
