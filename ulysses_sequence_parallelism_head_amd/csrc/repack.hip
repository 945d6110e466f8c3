// repack.hip -- the two Ulysses all-to-all exchanges, emulated on one GPU as
// layout permutations (pure bit copies, HBM-bound).
//
// Source: [ALST] "Paralelismul de Secvență Ulysses: Antrenarea modelelor AI
// cu contexte de un milion de token-uri", section "Mecanismul de funcționare
// Ulysses", steps 1, 3 and 5.
//
// Both directions are a transpose of two axes of runs of R contiguous bytes,
// R = (H/P) * D * element size:
//   seq2head:  dst[j][b][i][s][r] = src[i][b][s][j][r]
//   head2seq:  dst[i][b][s][j][r] = src[j][b][i][s][r]
// (i = sequence shard, j = head block, s = token within the shard).
// The grid walks the sequence-sharded side linearly (the source of seq2head,
// the destination of head2seq) in vectors of 16 bytes when the run size and
// both pointers allow it.  That side is then one contiguous stream and the
// head-sharded side is P sequential streams (one per head block), each
// advancing one run at a time: both sides stay DRAM-page friendly.
// Streaming loads/stores are marked non-temporal: nothing is reused.
#include "device_common.h"
#include "internal.h"

namespace ulysses {

namespace {

constexpr int kRepackThreads = 64;     // measured best for both directions at 512 MiB
constexpr int kRepackUnroll = 4;     // vectors in flight per thread

template <typename V>
__global__ __launch_bounds__(kRepackThreads) void repack_kernel(const V* __restrict__ src, V* __restrict__ dst,
                                                               uint32_t total_vecs, FastDiv fd_rv, FastDiv fd_nl,
                                                               FastDiv fd_P, FastDiv fd_B, int seq2head) {
  // total_vecs < 2^32 and every run index < 2^32 are checked on the host.
  // Linear index o walks the sequence-sharded layout [i][b][s][j][r]; its run
  // ((i*B + b)*nl + s)*P + j maps to the head-sharded run ((j*B + b)*P + i)*nl + s.
  const uint32_t Rv = fd_rv.d, nl = fd_nl.d, P = fd_P.d, B = fd_B.d;
  const uint64_t base = uint64_t(blockIdx.x) * (kRepackThreads * kRepackUnroll) + threadIdx.x;
  V val[kRepackUnroll];
  uint64_t hidx[kRepackUnroll];
#pragma unroll
  for (int u = 0; u < kRepackUnroll; ++u) {
    const uint64_t o64 = base + uint64_t(u) * kRepackThreads;
    hidx[u] = 0;
    if (o64 < total_vecs) {
      const uint32_t o = uint32_t(o64);
      const uint32_t run = fdiv(o, fd_rv);
      const uint32_t e = o - run * Rv;
      const uint32_t q1 = fdiv(run, fd_P);
      const uint32_t j = run - q1 * P;
      const uint32_t q2 = fdiv(q1, fd_nl);
      const uint32_t s = q1 - q2 * nl;
      const uint32_t i = fdiv(q2, fd_B);
      const uint32_t b = q2 - i * B;
      hidx[u] = uint64_t(((j * B + b) * P + i) * nl + s) * Rv + e;
      val[u] = __builtin_nontemporal_load(src + (seq2head ? o64 : hidx[u]));
    }
  }
#pragma unroll
  for (int u = 0; u < kRepackUnroll; ++u) {
    const uint64_t o64 = base + uint64_t(u) * kRepackThreads;
    if (o64 < total_vecs) __builtin_nontemporal_store(val[u], dst + (seq2head ? hidx[u] : o64));
  }
}

template <typename V>
hipError_t launch_repack_t(const void* src, void* dst, uint64_t total_bytes, uint32_t run_bytes, uint32_t P,
                           uint32_t B, uint32_t nl, int seq2head, hipStream_t stream) {
  const uint32_t Rv = run_bytes / sizeof(V);
  const uint64_t total_vecs = total_bytes / sizeof(V);
  const uint64_t per_block = uint64_t(kRepackThreads) * kRepackUnroll;
  const uint64_t blocks = (total_vecs + per_block - 1) / per_block;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(repack_kernel<V>, dim3(uint32_t(blocks)), dim3(kRepackThreads), 0, stream,
                     static_cast<const V*>(src), static_cast<V*>(dst), uint32_t(total_vecs), make_fastdiv(Rv),
                     make_fastdiv(nl), make_fastdiv(P), make_fastdiv(B), seq2head);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_repack(const void* src, void* dst, uint32_t P, uint32_t B, uint32_t n_local,
                         uint32_t run_bytes, uint32_t vec_bytes, int seq2head, hipStream_t stream) {
  const uint64_t total_bytes = uint64_t(P) * B * n_local * P * run_bytes;
  switch (vec_bytes) {
    case 16: return launch_repack_t<u32x4>(src, dst, total_bytes, run_bytes, P, B, n_local, seq2head, stream);
    case 8:  return launch_repack_t<u32x2>(src, dst, total_bytes, run_bytes, P, B, n_local, seq2head, stream);
    case 4:  return launch_repack_t<uint32_t>(src, dst, total_bytes, run_bytes, P, B, n_local, seq2head, stream);
    default: return launch_repack_t<uint16_t>(src, dst, total_bytes, run_bytes, P, B, n_local, seq2head, stream);
  }
}

}  // namespace ulysses
