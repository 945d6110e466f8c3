// abi.hip -- the exported C entry points of libulysses: host-side argument
// validation, then dispatch to the kernels' launchers.  Declarations and the
// contract of every call are in include/ulysses.h.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/ulysses.h"
#include "internal.h"

namespace {

using ulysses::AttnShape;

constexpr int32_t kAbiVersion = 1;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Half-open byte ranges [a, a+na) and [b, b+nb) intersect.
bool overlap(const void* a, uint64_t na, const void* b, uint64_t nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

uint32_t elem_size(ulysses_dtype_t t) { return t == ULYSSES_DTYPE_BF16 ? 2u : 4u; }
bool known_dtype(ulysses_dtype_t t) { return t == ULYSSES_DTYPE_F32 || t == ULYSSES_DTYPE_BF16; }

ulysses_status_t from_hip(hipError_t e) { return e == hipSuccess ? ULYSSES_OK : ULYSSES_ERR_HIP; }

ulysses_status_t repack(const void* src, void* dst, int32_t P, int32_t B, int64_t n_local, int32_t H, int32_t D,
                        ulysses_dtype_t dtype, void* stream, int seq2head) {
  if (P < 1 || B < 0 || n_local < 0 || H < 1 || D < 1) return ULYSSES_ERR_INVALID_ARG;
  if (H < P || H % P != 0) return ULYSSES_ERR_INVALID_ARG;
  if (!known_dtype(dtype)) return ULYSSES_ERR_INVALID_ARG;
  if (B == 0 || n_local == 0) return ULYSSES_OK;
  if (src == nullptr || dst == nullptr) return ULYSSES_ERR_INVALID_ARG;
  const uint32_t es = elem_size(dtype);
  if (!aligned(src, es) || !aligned(dst, es)) return ULYSSES_ERR_INVALID_ARG;
  const uint64_t run_bytes = uint64_t(H / P) * uint64_t(D) * es;
  const uint64_t runs = uint64_t(P) * uint64_t(B) * uint64_t(n_local) * uint64_t(P);
  if (run_bytes >= (uint64_t(1) << 32) || runs >= (uint64_t(1) << 32)) return ULYSSES_ERR_UNSUPPORTED;
  const uint64_t total = runs * run_bytes;
  if (overlap(src, total, dst, total)) return ULYSSES_ERR_INVALID_ARG;
  uint32_t vec = 16;
  while (vec > es && (run_bytes % vec != 0 || !aligned(src, vec) || !aligned(dst, vec))) vec >>= 1;
  if (total / vec >= (uint64_t(1) << 32)) return ULYSSES_ERR_UNSUPPORTED;
  return from_hip(ulysses::launch_repack(src, dst, uint32_t(P), uint32_t(B), uint32_t(n_local), uint32_t(run_bytes),
                                         vec, seq2head, static_cast<hipStream_t>(stream)));
}

// Shared checks of the attention calls.  Returns OK, or the error status;
// sets *empty for zero-sized problems.
ulysses_status_t check_attn_shape(int32_t B, int64_t n, int32_t Hq, int32_t Hkv, int32_t D, float scale,
                                  int32_t causal, ulysses_dtype_t in_dtype, ulysses_dtype_t o_dtype, bool* empty) {
  *empty = false;
  if (B < 0 || n < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ULYSSES_ERR_INVALID_ARG;
  if (!isfinite(scale) || !(scale > 0.f)) return ULYSSES_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return ULYSSES_ERR_INVALID_ARG;
  if (!known_dtype(in_dtype) || !known_dtype(o_dtype)) return ULYSSES_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return ULYSSES_ERR_UNSUPPORTED;
  if (n >= (int64_t(1) << 31) - 256) return ULYSSES_ERR_UNSUPPORTED;
  const int64_t Hmax = Hq > Hkv ? Hq : Hkv;
  if (int64_t(B) * n * Hmax * D >= (int64_t(1) << 40)) return ULYSSES_ERR_UNSUPPORTED;
  if (B == 0 || n == 0) *empty = true;
  return ULYSSES_OK;
}

// Forward with an optional per-row document bound (doc_start, causal only).
ulysses_status_t attn_fwd(const void* q, const void* k, const void* v, const uint8_t* key_valid,
                          const int32_t* doc_start, void* o, float* lse, int32_t B, int64_t n, int32_t Hq,
                          int32_t Hkv, int32_t D, float softmax_scale, int32_t causal, ulysses_dtype_t in_dtype,
                          ulysses_dtype_t o_dtype, void* stream) {
  bool empty = false;
  ulysses_status_t st = check_attn_shape(B, n, Hq, Hkv, D, softmax_scale, causal, in_dtype, o_dtype, &empty);
  if (st != ULYSSES_OK || empty) return st;
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || lse == nullptr) return ULYSSES_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
      !aligned(doc_start, 4))
    return ULYSSES_ERR_INVALID_ARG;
  const bool bf16_in = in_dtype == ULYSSES_DTYPE_BF16;
  if (!bf16_in && o_dtype != ULYSSES_DTYPE_F32) return ULYSSES_ERR_UNSUPPORTED;
  const uint64_t ei = elem_size(in_dtype), eo = elem_size(o_dtype);
  const uint64_t nq = uint64_t(B) * n * Hq * D, nkv = uint64_t(B) * n * Hkv * D;
  const uint64_t bo = nq * eo, bl = uint64_t(B) * Hq * n * 4;
  const void* ins[5] = {q, k, v, key_valid, doc_start};
  const uint64_t inb[5] = {nq * ei, nkv * ei, nkv * ei, key_valid ? uint64_t(B) * n : 0,
                           doc_start ? uint64_t(B) * n * 4 : 0};
  for (int i = 0; i < 5; ++i)
    if (overlap(o, bo, ins[i], inb[i]) || overlap(lse, bl, ins[i], inb[i])) return ULYSSES_ERR_INVALID_ARG;
  if (overlap(o, bo, lse, bl)) return ULYSSES_ERR_INVALID_ARG;
  AttnShape s{B, n, Hq, Hkv, D, softmax_scale, causal};
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (bf16_in)
    return from_hip(
        ulysses::launch_attn_fwd_bf16(q, k, v, key_valid, doc_start, o, lse, s, o_dtype == ULYSSES_DTYPE_F32, hs));
  return from_hip(ulysses::launch_attn_fwd_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                                               static_cast<const float*>(v), key_valid, doc_start,
                                               static_cast<float*>(o), lse, s, hs));
}

// Checks of the backward's arguments.  With workspace == nullptr the caller
// supplies none (the no-allocation call, whose scratch is the library's own):
// only the other buffers are checked.  Sets *empty for zero-sized problems.
ulysses_status_t check_bwd(const void* q, const void* k, const void* v, const uint8_t* key_valid,
                           const int32_t* doc_start, const void* o, const float* lse, const void* dout,
                           const float* dq, const float* dk, const float* dv, const void* workspace,
                           size_t workspace_bytes, bool own_workspace, int32_t B, int64_t n, int32_t Hq,
                           int32_t Hkv, int32_t D, float softmax_scale, int32_t causal, ulysses_dtype_t in_dtype,
                           ulysses_dtype_t o_dtype, bool* empty) {
  ulysses_status_t st = check_attn_shape(B, n, Hq, Hkv, D, softmax_scale, causal, in_dtype, o_dtype, empty);
  if (st != ULYSSES_OK || *empty) return st;
  if (in_dtype != ULYSSES_DTYPE_BF16) return ULYSSES_ERR_UNSUPPORTED;
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || lse == nullptr || dout == nullptr ||
      dq == nullptr || dk == nullptr || dv == nullptr || (own_workspace && workspace == nullptr))
    return ULYSSES_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
      !aligned(lse, 4) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(workspace, 256) ||
      !aligned(doc_start, 4))
    return ULYSSES_ERR_INVALID_ARG;
  const size_t need =
      ulysses::attn_bwd_workspace_bytes(B, n, Hq, Hkv, D, own_workspace ? ulysses::attn_bwd_nsplit_max(B, n, Hkv) : 1);
  if (own_workspace && workspace_bytes < need) return ULYSSES_ERR_INVALID_ARG;
  const uint64_t nq = uint64_t(B) * n * Hq * D, nkv = uint64_t(B) * n * Hkv * D;
  const void* ins[8] = {q, k, v, key_valid, o, lse, dout, doc_start};
  const uint64_t inb[8] = {nq * 2, nkv * 2, nkv * 2, key_valid ? uint64_t(B) * n : 0,
                           nq * elem_size(o_dtype), uint64_t(B) * Hq * n * 4, nq * 2,
                           doc_start ? uint64_t(B) * n * 4 : 0};
  const void* outs[4] = {dq, dk, dv, own_workspace ? workspace : nullptr};
  const uint64_t outb[4] = {nq * 4, nkv * 4, nkv * 4, need};
  for (int a = 0; a < 4; ++a) {
    for (int i = 0; i < 8; ++i)
      if (overlap(outs[a], outb[a], ins[i], inb[i])) return ULYSSES_ERR_INVALID_ARG;
    for (int c = a + 1; c < 4; ++c)
      if (overlap(outs[a], outb[a], outs[c], outb[c])) return ULYSSES_ERR_INVALID_ARG;
  }
  return ULYSSES_OK;
}

// Backward with an optional per-row document bound (doc_start, causal only).
ulysses_status_t attn_bwd(const void* q, const void* k, const void* v, const uint8_t* key_valid,
                          const int32_t* doc_start, const void* o, const float* lse, const void* dout, float* dq,
                          float* dk, float* dv, void* workspace, size_t workspace_bytes, int32_t B, int64_t n,
                          int32_t Hq, int32_t Hkv, int32_t D, float softmax_scale, int32_t causal,
                          ulysses_dtype_t in_dtype, ulysses_dtype_t o_dtype, void* stream) {
  bool empty = false;
  ulysses_status_t st = check_bwd(q, k, v, key_valid, doc_start, o, lse, dout, dq, dk, dv, workspace,
                                  workspace_bytes, true, B, n, Hq, Hkv, D, softmax_scale, causal, in_dtype, o_dtype,
                                  &empty);
  if (st != ULYSSES_OK || empty) return st;
  AttnShape s{B, n, Hq, Hkv, D, softmax_scale, causal};
  const ulysses::BwdKind kind = doc_start != nullptr ? ulysses::BwdKind::kDocs
                                : causal             ? ulysses::BwdKind::kCausal
                                                     : ulysses::BwdKind::kFull;
  return from_hip(ulysses::launch_attn_bwd_bf16(q, k, v, key_valid, doc_start, o, lse, dout, dq, dk, dv,
                                                static_cast<float*>(workspace), s, o_dtype == ULYSSES_DTYPE_F32,
                                                ulysses::attn_bwd_nsplit(B, n, Hkv, kind), static_cast<hipStream_t>(stream)));
}

// ---- the no-allocation backward
//
// Its scratch (the two float32 [B][Hq][n] row arrays of the backward) is a
// file-scope device array: the code object holds one copy on every GPU the
// library runs on, until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory, so host code never passes it to a
// kernel: the device address comes from hipGetSymbolAddress, taken once per
// device (with that device current) and kept below.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this GPU's `scratch`, or null with *err set.
void* scratch_on_current_device(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    *err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int32_t ulysses_abi_version(void) { return kAbiVersion; }

const char* ulysses_status_string(ulysses_status_t status) {
  switch (status) {
    case ULYSSES_OK: return "ok";
    case ULYSSES_ERR_INVALID_ARG: return "invalid argument";
    case ULYSSES_ERR_UNSUPPORTED: return "unsupported configuration";
    case ULYSSES_ERR_HIP: return "HIP launch failed";
    case ULYSSES_ERR_SCRATCH_LIMIT:
      return "problem exceeds the fixed scratch of the no-allocation call (2 * B * Hq * n * 4 bytes > 16 MiB)";
    default: return "unknown status";
  }
}

ulysses_status_t ulysses_repack_seq2head(const void* src, void* dst, int32_t P, int32_t B, int64_t n_local,
                                         int32_t H, int32_t D, ulysses_dtype_t dtype, void* stream) {
  return repack(src, dst, P, B, n_local, H, D, dtype, stream, 1);
}

ulysses_status_t ulysses_repack_head2seq(const void* src, void* dst, int32_t P, int32_t B, int64_t n_local,
                                         int32_t H, int32_t D, ulysses_dtype_t dtype, void* stream) {
  return repack(src, dst, P, B, n_local, H, D, dtype, stream, 0);
}

ulysses_status_t ulysses_attn_fwd(const void* q, const void* k, const void* v, const uint8_t* key_valid, void* o,
                                  float* lse, int32_t B, int64_t n, int32_t Hq, int32_t Hkv, int32_t D,
                                  float softmax_scale, int32_t causal, ulysses_dtype_t in_dtype,
                                  ulysses_dtype_t o_dtype, void* stream) {
  return attn_fwd(q, k, v, key_valid, nullptr, o, lse, B, n, Hq, Hkv, D, softmax_scale, causal, in_dtype, o_dtype,
                  stream);
}

ulysses_status_t ulysses_attn_fwd_docs(const void* q, const void* k, const void* v, const uint8_t* key_valid,
                                       const int32_t* doc_start, void* o, float* lse, int32_t B, int64_t n,
                                       int32_t Hq, int32_t Hkv, int32_t D, float softmax_scale,
                                       ulysses_dtype_t in_dtype, ulysses_dtype_t o_dtype, void* stream) {
  if (doc_start == nullptr && B > 0 && n > 0) return ULYSSES_ERR_INVALID_ARG;
  return attn_fwd(q, k, v, key_valid, doc_start, o, lse, B, n, Hq, Hkv, D, softmax_scale, 1, in_dtype, o_dtype,
                  stream);
}

size_t ulysses_attn_bwd_workspace_bytes(int32_t B, int64_t n, int32_t Hq, int32_t Hkv, int32_t D) {
  if (B <= 0 || n <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0) return 0;
  return ulysses::attn_bwd_workspace_bytes(B, n, Hq, Hkv, D, ulysses::attn_bwd_nsplit_max(B, n, Hkv));
}

ulysses_status_t ulysses_attn_bwd(const void* q, const void* k, const void* v, const uint8_t* key_valid,
                                  const void* o, const float* lse, const void* dout, float* dq, float* dk, float* dv,
                                  void* workspace, size_t workspace_bytes, int32_t B, int64_t n, int32_t Hq,
                                  int32_t Hkv, int32_t D, float softmax_scale, int32_t causal,
                                  ulysses_dtype_t in_dtype, ulysses_dtype_t o_dtype, void* stream) {
  return attn_bwd(q, k, v, key_valid, nullptr, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, n, Hq, Hkv,
                  D, softmax_scale, causal, in_dtype, o_dtype, stream);
}

ulysses_status_t ulysses_attn_bwd_noalloc(const void* q, const void* k, const void* v, const uint8_t* key_valid,
                                          const void* o, const float* lse, const void* dout, float* dq, float* dk,
                                          float* dv, int32_t B, int64_t n, int32_t Hq, int32_t Hkv, int32_t D,
                                          float softmax_scale, int32_t causal, ulysses_dtype_t in_dtype,
                                          ulysses_dtype_t o_dtype, void* stream) {
  bool empty = false;
  ulysses_status_t st = check_bwd(q, k, v, key_valid, nullptr, o, lse, dout, dq, dk, dv, nullptr, 0, false, B, n,
                                  Hq, Hkv, D, softmax_scale, causal, in_dtype, o_dtype, &empty);
  if (st != ULYSSES_OK || empty) return st;
  if (ulysses::attn_bwd_workspace_bytes(B, n, Hq, Hkv, D, 1) > kNoAllocScratchBytes) return ULYSSES_ERR_SCRATCH_LIMIT;
  hipError_t e = hipSuccess;
  void* ws = scratch_on_current_device(&e);
  if (ws == nullptr) return ULYSSES_ERR_HIP;
  AttnShape s{B, n, Hq, Hkv, D, softmax_scale, causal};
  return from_hip(ulysses::launch_attn_bwd_bf16(q, k, v, key_valid, nullptr, o, lse, dout, dq, dk, dv,
                                                static_cast<float*>(ws), s, o_dtype == ULYSSES_DTYPE_F32, 1,
                                                static_cast<hipStream_t>(stream)));
}

ulysses_status_t ulysses_attn_bwd_docs(const void* q, const void* k, const void* v, const uint8_t* key_valid,
                                       const int32_t* doc_start, const void* o, const float* lse, const void* dout,
                                       float* dq, float* dk, float* dv, void* workspace, size_t workspace_bytes,
                                       int32_t B, int64_t n, int32_t Hq, int32_t Hkv, int32_t D,
                                       float softmax_scale, ulysses_dtype_t in_dtype, ulysses_dtype_t o_dtype,
                                       void* stream) {
  if (doc_start == nullptr && B > 0 && n > 0) return ULYSSES_ERR_INVALID_ARG;
  return attn_bwd(q, k, v, key_valid, doc_start, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, n, Hq, Hkv,
                  D, softmax_scale, 1, in_dtype, o_dtype, stream);
}

ulysses_status_t ulysses_attn_fwd_block(const void* q, const void* k, const void* v, const uint8_t* key_valid,
                                        float* o, float* lse, int32_t B, int64_t nq, int64_t nk, int32_t Hq,
                                        int32_t Hkv, int32_t D, float softmax_scale, int64_t causal_offset,
                                        int32_t causal, int32_t accumulate, ulysses_dtype_t in_dtype,
                                        void* stream) {
  bool empty = false;
  ulysses_status_t st =
      check_attn_shape(B, nq, Hq, Hkv, D, softmax_scale, causal, in_dtype, ULYSSES_DTYPE_F32, &empty);
  if (st != ULYSSES_OK) return st;
  if (nk < 1 || (accumulate != 0 && accumulate != 1)) return ULYSSES_ERR_INVALID_ARG;
  if (in_dtype != ULYSSES_DTYPE_BF16) return ULYSSES_ERR_UNSUPPORTED;
  if (nk >= (int64_t(1) << 31) - 256 || nq + nk >= (int64_t(1) << 31) - 256) return ULYSSES_ERR_UNSUPPORTED;
  if (int64_t(B) * nk * Hkv * D >= (int64_t(1) << 40)) return ULYSSES_ERR_UNSUPPORTED;
  if (empty) return ULYSSES_OK;
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || lse == nullptr) return ULYSSES_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return ULYSSES_ERR_INVALID_ARG;
  const uint64_t nqe = uint64_t(B) * nq * Hq * D, nke = uint64_t(B) * nk * Hkv * D;
  const uint64_t bo = nqe * 4, bl = uint64_t(B) * Hq * nq * 4;
  const void* ins[4] = {q, k, v, key_valid};
  const uint64_t inb[4] = {nqe * 2, nke * 2, nke * 2, key_valid ? uint64_t(B) * nk : 0};
  for (int i = 0; i < 4; ++i)
    if (overlap(o, bo, ins[i], inb[i]) || overlap(lse, bl, ins[i], inb[i])) return ULYSSES_ERR_INVALID_ARG;
  if (overlap(o, bo, lse, bl)) return ULYSSES_ERR_INVALID_ARG;
  // offsets past the block's extent change nothing: clamp to [-nq, nk]
  const int64_t delta = causal_offset < -nq ? -nq : (causal_offset > nk ? nk : causal_offset);
  ulysses::KeyBlock kb{nk, causal ? delta : nk, accumulate};
  AttnShape s{B, nq, Hq, Hkv, D, softmax_scale, causal};
  return from_hip(ulysses::launch_attn_fwd_bf16(q, k, v, key_valid, nullptr, o, lse, s, 1,
                                                static_cast<hipStream_t>(stream), &kb));
}

ulysses_status_t ulysses_repack_seq2head_rope(const void* src, void* dst, int32_t P, int32_t B, int64_t n_local,
                                              int32_t H, int32_t D, double rope_base, double rope_scale,
                                              ulysses_dtype_t dtype, void* stream) {
  if (P < 1 || B < 0 || n_local < 0 || H < 1 || D < 1) return ULYSSES_ERR_INVALID_ARG;
  if (H < P || H % P != 0) return ULYSSES_ERR_INVALID_ARG;
  if (!known_dtype(dtype)) return ULYSSES_ERR_INVALID_ARG;
  if (!isfinite(rope_base) || !(rope_base > 0.0) || !isfinite(rope_scale) || !(rope_scale > 0.0))
    return ULYSSES_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return ULYSSES_ERR_UNSUPPORTED;
  if (B == 0 || n_local == 0) return ULYSSES_OK;
  if (src == nullptr || dst == nullptr) return ULYSSES_ERR_INVALID_ARG;
  if (!aligned(src, 16) || !aligned(dst, 16)) return ULYSSES_ERR_INVALID_ARG;
  if (n_local >= (int64_t(1) << 31) || int64_t(P) * B * n_local >= (int64_t(1) << 37)) return ULYSSES_ERR_UNSUPPORTED;
  const uint64_t total = uint64_t(P) * uint64_t(B) * uint64_t(n_local) * uint64_t(H) * uint64_t(D) * elem_size(dtype);
  if (overlap(src, total, dst, total)) return ULYSSES_ERR_INVALID_ARG;
  return from_hip(ulysses::launch_seq2head_rope(src, dst, P, B, int32_t(n_local), H, D, int(elem_size(dtype)),
                                                rope_base, rope_scale, static_cast<hipStream_t>(stream)));
}

ulysses_status_t ulysses_qkv_proj_seq2head(const void* x, const void* w, void* q, void* k, void* v, int32_t P,
                                           int32_t B, int64_t n_local, int32_t hidden, int32_t Hq, int32_t Hkv,
                                           int32_t D, void* stream) {
  if (P < 1 || B < 0 || n_local < 0 || hidden < 1 || Hq < 1 || Hkv < 1 || D < 1) return ULYSSES_ERR_INVALID_ARG;
  if (Hq % P != 0 || Hkv % P != 0) return ULYSSES_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return ULYSSES_ERR_UNSUPPORTED;
  if (hidden % 64 != 0) return ULYSSES_ERR_UNSUPPORTED;
  if (n_local >= (int64_t(1) << 31) / P) return ULYSSES_ERR_UNSUPPORTED;
  const uint64_t tokens = uint64_t(P) * uint64_t(B) * uint64_t(n_local);
  const uint64_t N = uint64_t(Hq + 2 * Hkv) * D;
  if (tokens * (uint64_t(hidden) + N) >= (uint64_t(1) << 40) || N >= (uint64_t(1) << 31)) return ULYSSES_ERR_UNSUPPORTED;
  if (B == 0 || n_local == 0) return ULYSSES_OK;
  if (x == nullptr || w == nullptr || q == nullptr || k == nullptr || v == nullptr) return ULYSSES_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16))
    return ULYSSES_ERR_INVALID_ARG;
  const void* ins[2] = {x, w};
  const uint64_t inb[2] = {tokens * hidden * 2, N * hidden * 2};
  void* outs[3] = {q, k, v};
  const uint64_t outb[3] = {tokens * Hq * D * 2, tokens * Hkv * D * 2, tokens * Hkv * D * 2};
  for (int a = 0; a < 3; ++a) {
    for (int i = 0; i < 2; ++i)
      if (overlap(outs[a], outb[a], ins[i], inb[i])) return ULYSSES_ERR_INVALID_ARG;
    for (int c = a + 1; c < 3; ++c)
      if (overlap(outs[a], outb[a], outs[c], outb[c])) return ULYSSES_ERR_INVALID_ARG;
  }
  return from_hip(ulysses::launch_qkv_proj_seq2head(x, w, q, k, v, P, B, int32_t(n_local), hidden, Hq, Hkv, D,
                                                    static_cast<hipStream_t>(stream)));
}

ulysses_status_t ulysses_head2seq_out_proj(const void* o, const void* w_o, void* y, int32_t P, int32_t B,
                                           int64_t n_local, int32_t Hq, int32_t D, int32_t hidden, void* stream) {
  if (P < 1 || B < 0 || n_local < 0 || hidden < 1 || Hq < 1 || D < 1) return ULYSSES_ERR_INVALID_ARG;
  if (Hq % P != 0) return ULYSSES_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return ULYSSES_ERR_UNSUPPORTED;
  if (((Hq / P) * D) % 64 != 0 || hidden % 4 != 0) return ULYSSES_ERR_UNSUPPORTED;
  if (n_local >= (int64_t(1) << 31) / P) return ULYSSES_ERR_UNSUPPORTED;
  const uint64_t tokens = uint64_t(P) * uint64_t(B) * uint64_t(n_local);
  const uint64_t K = uint64_t(Hq) * D;
  if (tokens * (K + uint64_t(hidden)) >= (uint64_t(1) << 40) || K >= (uint64_t(1) << 31)) return ULYSSES_ERR_UNSUPPORTED;
  if (B == 0 || n_local == 0) return ULYSSES_OK;
  if (o == nullptr || w_o == nullptr || y == nullptr) return ULYSSES_ERR_INVALID_ARG;
  if (!aligned(o, 16) || !aligned(w_o, 16) || !aligned(y, 16)) return ULYSSES_ERR_INVALID_ARG;
  const uint64_t yb = tokens * hidden * 2;
  if (overlap(y, yb, o, tokens * K * 2) || overlap(y, yb, w_o, uint64_t(hidden) * K * 2)) return ULYSSES_ERR_INVALID_ARG;
  return from_hip(ulysses::launch_head2seq_out_proj(o, w_o, y, P, B, int32_t(n_local), Hq, D, hidden,
                                                    static_cast<hipStream_t>(stream)));
}

ulysses_status_t ulysses_clock_probe(uint64_t* out, int32_t samples, int32_t interval_us, int32_t* wall_khz,
                                     void* stream) {
  if (out == nullptr || wall_khz == nullptr || samples < 1 || samples > 65536 || interval_us < 1 ||
      interval_us > 1000000)
    return ULYSSES_ERR_INVALID_ARG;
  if (!aligned(out, 8)) return ULYSSES_ERR_INVALID_ARG;
  return from_hip(ulysses::launch_clock_probe(out, samples, uint32_t(interval_us), wall_khz,
                                              static_cast<hipStream_t>(stream)));
}

ulysses_status_t ulysses_loss_aggregate(const float* token_loss, const uint8_t* valid, int32_t P, int64_t per_rank,
                                        double* rank_sum, int64_t* rank_count, float* loss, void* stream) {
  if (P < 1 || P > 65535 || per_rank < 0) return ULYSSES_ERR_INVALID_ARG;
  if (rank_sum == nullptr || rank_count == nullptr || loss == nullptr) return ULYSSES_ERR_INVALID_ARG;
  if (per_rank > 0 && token_loss == nullptr) return ULYSSES_ERR_INVALID_ARG;
  if (!aligned(token_loss, 4) || !aligned(rank_sum, 8) || !aligned(rank_count, 8) || !aligned(loss, 4))
    return ULYSSES_ERR_INVALID_ARG;
  const uint64_t nt = uint64_t(P) * uint64_t(per_rank);
  const void* ins[2] = {token_loss, per_rank > 0 ? valid : nullptr};
  const uint64_t inb[2] = {nt * 4, valid ? nt : 0};
  const void* outs[3] = {rank_sum, rank_count, loss};
  const uint64_t outb[3] = {uint64_t(P) * 8, uint64_t(P) * 8, 4};
  for (int a = 0; a < 3; ++a) {
    for (int i = 0; i < 2; ++i)
      if (overlap(outs[a], outb[a], ins[i], inb[i])) return ULYSSES_ERR_INVALID_ARG;
    for (int c = a + 1; c < 3; ++c)
      if (overlap(outs[a], outb[a], outs[c], outb[c])) return ULYSSES_ERR_INVALID_ARG;
  }
  return from_hip(ulysses::launch_loss_aggregate(token_loss, per_rank > 0 ? valid : nullptr, P, per_rank, rank_sum,
                                                 rank_count, loss, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
