// Host-side check of the C ABI's argument validation under AddressSanitizer
// and UndefinedBehaviorSanitizer (built by tests/test_abi_sanitizers.py).
//
// The ABI layer (abi.hip) and the workspace sizing (workspace.hip) are
// linked against the stub launchers below instead of the kernels: a
// validation path that lets an invalid call through reaches a stub, which
// counts it, and the driver fails.  Every call here uses pointers that are
// never dereferenced (validation only reads their values), so the
// sanitizers watch the validation arithmetic itself: size products,
// overlap tests, alignment masks, the status strings.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ulysses.h"
#include "../../ulysses_sequence_parallelism_head_amd/csrc/internal.h"

static int g_launches = 0;

namespace ulysses {
hipError_t launch_repack(const void*, void*, uint32_t, uint32_t, uint32_t, uint32_t, uint32_t, int, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_attn_fwd_bf16(const void*, const void*, const void*, const uint8_t*, const int32_t*, void*, float*,
                                const AttnShape&, int, hipStream_t, const KeyBlock*) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_attn_fwd_f32(const float*, const float*, const float*, const uint8_t*, const int32_t*, float*,
                               float*, const AttnShape&, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_attn_bwd_bf16(const void*, const void*, const void*, const uint8_t*, const int32_t*, const void*,
                                const float*, const void*, float*, float*, float*, float*, const AttnShape&, int, int,
                                hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_seq2head_rope(const void*, void*, int32_t, int32_t, int32_t, int32_t, int32_t, int, double, double,
                                hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_qkv_proj_seq2head(const void*, const void*, void*, void*, void*, int32_t, int32_t, int32_t, int32_t,
                                    int32_t, int32_t, int32_t, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_head2seq_out_proj(const void*, const void*, void*, int32_t, int32_t, int32_t, int32_t, int32_t,
                                    int32_t, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_clock_probe(uint64_t*, int32_t, uint32_t, int32_t*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_loss_aggregate(const float*, const uint8_t*, int32_t, int64_t, double*, int64_t*, float*,
                                 hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
}  // namespace ulysses

static int g_fail = 0;
#define EXPECT(call, want)                                                                          \
  do {                                                                                              \
    const int got_ = int(call);                                                                     \
    if (got_ != int(want)) {                                                                        \
      fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, got_, int(want)); \
      ++g_fail;                                                                                     \
    }                                                                                               \
  } while (0)

static void* P(uint64_t a) { return reinterpret_cast<void*>(a); }
static const uint64_t G = uint64_t(1) << 36;   // fake buffers 64 GiB apart never overlap

int main() {
  const ulysses_status_t OK = ULYSSES_OK, INV = ULYSSES_ERR_INVALID_ARG, UNS = ULYSSES_ERR_UNSUPPORTED;
  const ulysses_dtype_t BF = ULYSSES_DTYPE_BF16, F32 = ULYSSES_DTYPE_F32;
  for (int s = 0; s < 8; ++s)
    if (ulysses_status_string(ulysses_status_t(s)) == nullptr || strlen(ulysses_status_string(ulysses_status_t(s))) == 0)
      ++g_fail;
  EXPECT(ulysses_abi_version(), 1);

  // repacks: constraints on heads and shards, dtypes, null, alignment, overlap, extreme sizes
  for (int dir = 0; dir < 2; ++dir) {
    auto rp = [&](const void* src, void* dst, int32_t P_, int32_t B, int64_t nl, int32_t H, int32_t D,
                  ulysses_dtype_t t) {
      return dir ? ulysses_repack_head2seq(src, dst, P_, B, nl, H, D, t, nullptr)
                 : ulysses_repack_seq2head(src, dst, P_, B, nl, H, D, t, nullptr);
    };
    EXPECT(rp(P(G), P(2 * G), 4, 1, 16, 2, 128, BF), INV);            // H < P
    EXPECT(rp(P(G), P(2 * G), 4, 1, 16, 6, 128, BF), INV);            // H % P
    EXPECT(rp(P(G), P(2 * G), 0, 1, 16, 4, 128, BF), INV);            // P < 1
    EXPECT(rp(P(G), P(2 * G), 2, -1, 16, 4, 128, BF), INV);           // B < 0
    EXPECT(rp(P(G), P(2 * G), 2, 1, -3, 4, 128, BF), INV);            // n_local < 0
    EXPECT(rp(P(G), P(2 * G), 2, 1, 16, 4, 8, ulysses_dtype_t(7)), INV);
    EXPECT(rp(nullptr, P(2 * G), 2, 1, 16, 4, 8, BF), INV);
    EXPECT(rp(P(G + 1), P(2 * G), 2, 1, 16, 4, 8, BF), INV);          // misaligned
    EXPECT(rp(P(G), P(G + 64), 2, 1, 16, 4, 8, BF), INV);             // overlap
    EXPECT(rp(nullptr, nullptr, 2, 0, 16, 4, 8, BF), OK);             // empty
    EXPECT(rp(P(G), P(2 * G), 2, 1, int64_t(1) << 40, 4, 8, BF), UNS);   // too many runs
    EXPECT(rp(P(G), P(2 * G), 2, 0x7fffffff, 0x7fffffff, 4, 8, BF), UNS);
  }

  // forward
  auto fwd = [&](int64_t n, int32_t Hq, int32_t Hkv, int32_t D, float sc, int32_t causal, ulysses_dtype_t it,
                 ulysses_dtype_t ot, uint64_t o = 4 * G) {
    return ulysses_attn_fwd(P(G), P(2 * G), P(3 * G), nullptr, P(o), reinterpret_cast<float*>(5 * G), 1, n, Hq, Hkv,
                            D, sc, causal, it, ot, nullptr);
  };
  EXPECT(fwd(64, 8, 2, 96, 0.1f, 1, BF, BF), UNS);
  EXPECT(fwd(64, 8, 2, 128, 0.1f, 1, F32, BF), UNS);
  EXPECT(fwd(64, 6, 4, 128, 0.1f, 1, BF, BF), INV);
  EXPECT(fwd(64, 8, 0, 128, 0.1f, 1, BF, BF), INV);
  EXPECT(fwd(-1, 8, 2, 128, 0.1f, 1, BF, BF), INV);
  EXPECT(fwd(64, 8, 2, 128, 0.f, 1, BF, BF), INV);
  EXPECT(fwd(64, 8, 2, 128, -1.f / 0.f, 1, BF, BF), INV);
  EXPECT(fwd(64, 8, 2, 128, 0.1f, 2, BF, BF), INV);
  EXPECT(fwd(64, 8, 2, 128, 0.1f, 1, BF, BF, 2 * G + 256), INV);     // o overlaps k
  EXPECT(fwd(int64_t(1) << 31, 8, 2, 128, 0.1f, 1, BF, BF), UNS);
  EXPECT(fwd(int64_t(1) << 30, 0x40000, 0x40000, 128, 0.1f, 1, BF, BF), UNS);   // element count >= 2^40
  EXPECT(ulysses_attn_fwd_docs(P(G), P(2 * G), P(3 * G), nullptr, nullptr, P(4 * G), reinterpret_cast<float*>(5 * G),
                               1, 64, 8, 2, 128, 0.1f, BF, BF, nullptr),
         INV);                                                         // documents required
  EXPECT(ulysses_attn_fwd_block(P(G), P(2 * G), P(3 * G), nullptr, reinterpret_cast<float*>(4 * G),
                                reinterpret_cast<float*>(5 * G), 1, 64, 0, 8, 2, 128, 0.1f, 5, 1, 0, BF, nullptr),
         INV);                                                         // nk = 0

  // backward, its workspace, the no-allocation variant
  const size_t need = ulysses_attn_bwd_workspace_bytes(1, 64, 8, 2, 128);
  if (need == 0 || need % 256 != 0) ++g_fail;
  EXPECT(ulysses_attn_bwd_workspace_bytes(0, 64, 8, 2, 128), 0);
  EXPECT(ulysses_attn_bwd_workspace_bytes(0x7fffffff, int64_t(1) << 40, 0x7fffffff, 1, 128) > 0, 1);
  auto bwd = [&](size_t wsb, uint64_t ws, int64_t n, ulysses_dtype_t it, uint64_t dq = 6 * G) {
    return ulysses_attn_bwd(P(G), P(2 * G), P(3 * G), nullptr, P(4 * G), reinterpret_cast<float*>(5 * G),
                            P(10 * G), reinterpret_cast<float*>(dq), reinterpret_cast<float*>(7 * G),
                            reinterpret_cast<float*>(8 * G), P(ws), wsb, 1, n, 8, 2, 128, 0.1f, 1, it, BF, nullptr);
  };
  EXPECT(bwd(need - 1, 9 * G, 64, BF), INV);
  EXPECT(bwd(need, 0, 64, BF), INV);
  EXPECT(bwd(need, 9 * G + 16, 64, BF), INV);
  EXPECT(bwd(need, 9 * G, 64, BF, 10 * G + 64), INV);                 // dq overlaps dout
  EXPECT(bwd(need, 9 * G, 64, F32), UNS);
  EXPECT(bwd(need, 0, 0, BF), OK);                                    // empty
  auto bna = [&](int64_t n, int32_t Hq, uint64_t dq = 6 * G) {
    return ulysses_attn_bwd_noalloc(P(G), P(2 * G), P(3 * G), nullptr, P(4 * G), reinterpret_cast<float*>(5 * G),
                                    P(10 * G), reinterpret_cast<float*>(dq), reinterpret_cast<float*>(7 * G),
                                    reinterpret_cast<float*>(8 * G), 1, n, Hq, 2, 128, 0.1f, 1, BF, BF, nullptr);
  };
  EXPECT(bna((int64_t(1) << 21) / 8 + 1, 8), ULYSSES_ERR_SCRATCH_LIMIT);
  EXPECT(bna(64, 7), INV);
  EXPECT(bna(64, 8, 0), INV);
  EXPECT(bna(0, 8), OK);

  // the other calls
  EXPECT(ulysses_repack_seq2head_rope(P(G), P(2 * G), 4, 1, 16, 32, 128, 0.0, 1.0, BF, nullptr), INV);
  EXPECT(ulysses_repack_seq2head_rope(P(G), P(2 * G), 4, 1, 16, 32, 128, 1e6, -1.0, BF, nullptr), INV);
  EXPECT(ulysses_qkv_proj_seq2head(P(G), P(2 * G), P(3 * G), P(4 * G), P(5 * G), 4, 1, 16, 4000, 32, 8, 128, nullptr),
         UNS);
  EXPECT(ulysses_head2seq_out_proj(P(G), P(2 * G), P(3 * G), 4, 1, 16, 30, 128, 4096, nullptr), INV);
  EXPECT(ulysses_loss_aggregate(nullptr, nullptr, 2, 10, reinterpret_cast<double*>(G), reinterpret_cast<int64_t*>(2 * G),
                                reinterpret_cast<float*>(3 * G), nullptr),
         INV);
  int32_t khz = 0;
  EXPECT(ulysses_clock_probe(nullptr, 4, 10, &khz, nullptr), INV);
  EXPECT(ulysses_clock_probe(reinterpret_cast<uint64_t*>(G), 0, 10, &khz, nullptr), INV);

  if (g_launches != 0) {
    fprintf(stderr, "%d invalid or empty call(s) reached a launcher\n", g_launches);
    ++g_fail;
  }

  // valid calls do reach the launchers (the validation is not a blanket refusal)
  EXPECT(fwd(64, 8, 2, 128, 0.1f, 1, BF, BF), OK);
  EXPECT(bwd(need, 9 * G, 64, BF), OK);
  EXPECT(ulysses_repack_seq2head(P(G), P(2 * G), 2, 1, 16, 4, 8, BF, nullptr), OK);
  if (g_launches != 3) {
    fprintf(stderr, "valid calls reached %d launchers, expected 3\n", g_launches);
    ++g_fail;
  }
  printf("abi validation under sanitizers: %s\n", g_fail ? "FAILED" : "ok");
  return g_fail ? 1 : 0;
}
