// loss.hip -- the loss aggregated over sequence shards, weighted by each
// shard's number of valid tokens.
//
// Source: [ALST] "Paralelismul de Secvență Ulysses: Antrenarea modelelor AI
// cu contexte de un milion de token-uri", section "Integrarea cu Accelerate"
// (each rank's loss covers its part of the sequence; the ranks' losses are
// combined weighted by their valid tokens, padding and masked prompt tokens
// excluded).  Per rank r: sum_r over its valid tokens' losses and count_r;
// the loss is (sum over r of sum_r) / (sum over r of count_r), NaN when no
// token is valid.
//
// Two launches.  The first has one workgroup per rank: every thread sums a
// strided slice of the rank's tokens in double precision, then a fixed
// tree in LDS adds the 1024 partial sums (same order on every call, so the
// result is deterministic).  The second, one wave, adds the P rank sums and
// counts in rank order and divides.  The token losses are a few bytes per
// token; this is latency-bound at any realistic size.
#include "device_common.h"
#include "internal.h"

namespace ulysses {

namespace {

constexpr int kLossThreads = 1024;

__global__ __launch_bounds__(kLossThreads) void rank_sums_kernel(const float* __restrict__ token_loss,
                                                                 const uint8_t* __restrict__ valid,
                                                                 int64_t per_rank, double* rank_sum,
                                                                 int64_t* rank_count) {
  __shared__ double ssum[kLossThreads];
  __shared__ int64_t scnt[kLossThreads];
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const float* tl = token_loss + int64_t(r) * per_rank;
  const uint8_t* va = valid ? valid + int64_t(r) * per_rank : nullptr;
  double acc = 0.0;
  int64_t cnt = 0;
  for (int64_t t = tid; t < per_rank; t += kLossThreads) {
    if (va == nullptr || va[t] != 0) {
      acc += double(tl[t]);
      ++cnt;
    }
  }
  ssum[tid] = acc;
  scnt[tid] = cnt;
  __syncthreads();
  for (int w = kLossThreads / 2; w > 0; w >>= 1) {
    if (tid < w) {
      ssum[tid] += ssum[tid + w];
      scnt[tid] += scnt[tid + w];
    }
    __syncthreads();
  }
  if (tid == 0) {
    rank_sum[r] = ssum[0];
    rank_count[r] = scnt[0];
  }
}

__global__ __launch_bounds__(64) void combine_kernel(const double* rank_sum, const int64_t* rank_count, int32_t P,
                                                     float* loss) {
  if (threadIdx.x != 0) return;
  double s = 0.0;
  int64_t c = 0;
  for (int r = 0; r < P; ++r) {
    s += rank_sum[r];
    c += rank_count[r];
  }
  loss[0] = c > 0 ? float(s / double(c)) : __builtin_nanf("");
}

}  // namespace

hipError_t launch_loss_aggregate(const float* token_loss, const uint8_t* valid, int32_t P, int64_t per_rank,
                                 double* rank_sum, int64_t* rank_count, float* loss, hipStream_t stream) {
  hipLaunchKernelGGL(rank_sums_kernel, dim3(P), dim3(kLossThreads), 0, stream, token_loss, valid, per_rank, rank_sum,
                     rank_count);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(combine_kernel, dim3(1), dim3(64), 0, stream, rank_sum, rank_count, P, loss);
  return hipGetLastError();
}

}  // namespace ulysses
