// internal.h -- launchers behind the C ABI (not exported).  Arguments are
// already validated by abi.hip; these only pick kernel variants and launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ulysses {

// The exchange permutations.  run_bytes = (H/P)*D*elem; vec_bytes divides
// run_bytes and both pointers' alignment.
hipError_t launch_repack(const void* src, void* dst, uint32_t P, uint32_t B, uint32_t n_local,
                         uint32_t run_bytes, uint32_t vec_bytes, int seq2head, hipStream_t stream);

struct AttnShape {
  int32_t B;
  int64_t n;
  int32_t Hq, Hkv, D;
  float scale;
  int32_t causal;
};

// doc_start: NULL, or int32 [B][n] per-row lower bound of the visible keys
// (the first position of the row's document) on top of the causal mask;
// callers pass it only with s.causal == 1.

// A separate key block for the forward: nk keys, key u visible to row t iff
// u <= t + delta (causal); accumulate merges into the float32 (O, LSE)
// already in the outputs.  Callers keep nk >= 1, -n <= delta <= nk.
struct KeyBlock {
  int64_t nk;
  int64_t delta;
  int32_t accumulate;
};

// bf16 inputs, matrix cores; o_f32 selects a float32 (else bf16) output;
// kb = nullptr: the keys are the rows' own sequence (nk = n, delta = 0).
hipError_t launch_attn_fwd_bf16(const void* q, const void* k, const void* v, const uint8_t* valid,
                                const int32_t* doc_start, void* o, float* lse, const AttnShape& s, int o_f32,
                                hipStream_t stream, const KeyBlock* kb = nullptr);

// float32 inputs and output, fp32 arithmetic throughout.
hipError_t launch_attn_fwd_f32(const float* q, const float* k, const float* v, const uint8_t* valid,
                               const int32_t* doc_start, float* o, float* lse, const AttnShape& s,
                               hipStream_t stream);

// bf16 inputs; o is bf16 or float32 (o_f32); gradients are float32.
// workspace holds the per-row dO.O values and the base-2 logsumexp, and with
// nsplit > 1 the splits' partial dK/dV (attn_bwd_workspace_bytes(..., nsplit)).
hipError_t launch_attn_bwd_bf16(const void* q, const void* k, const void* v, const uint8_t* valid,
                                const int32_t* doc_start, const void* o, const float* lse, const void* dout,
                                float* dq, float* dk, float* dv, float* workspace, const AttnShape& s, int o_f32,
                                int nsplit, hipStream_t stream);

// workgroups per work item of the dK/dV pass for this shape and kind of
// call, and the largest over the kinds (what the workspace is sized for)
enum class BwdKind { kCausal, kFull, kDocs };
int attn_bwd_nsplit(int32_t B, int64_t n, int32_t Hkv, BwdKind kind);
int attn_bwd_nsplit_max(int32_t B, int64_t n, int32_t Hkv);
// where each array of the backward's workspace lives (offsets in floats)
struct BwdWorkspace {
  size_t rowdot, lse2, dk_part, dv_part;
  size_t bytes;   // total
};
BwdWorkspace attn_bwd_workspace(int32_t B, int64_t n, int32_t Hq, int32_t Hkv, int32_t D, int nsplit);
size_t attn_bwd_workspace_bytes(int32_t B, int64_t n, int32_t Hq, int32_t Hkv, int32_t D, int nsplit);

// seq2head fused with the rotary embedding at global positions; elem_bytes
// 2 (bf16) or 4 (fp32), D 64 or 128, H % P == 0.
hipError_t launch_seq2head_rope(const void* src, void* dst, int32_t P, int32_t B, int32_t n_local, int32_t H,
                                int32_t D, int elem_bytes, double base, double scale, hipStream_t stream);

// the projections fused with their exchanges (bf16; hidden and Hq*D multiples
// of 64, (Hq/P)*D a multiple of 64, D 64 or 128)
hipError_t launch_qkv_proj_seq2head(const void* x, const void* w, void* q, void* k, void* v, int32_t P, int32_t B,
                                    int32_t n_local, int32_t hidden, int32_t Hq, int32_t Hkv, int32_t D,
                                    hipStream_t stream);
hipError_t launch_head2seq_out_proj(const void* o, const void* w_o, void* y, int32_t P, int32_t B, int32_t n_local,
                                    int32_t Hq, int32_t D, int32_t hidden, hipStream_t stream);

// one wave sampling (real-time stamp, shader cycles) pairs every interval_us;
// *wall_khz receives the real-time counter's rate
hipError_t launch_clock_probe(uint64_t* out, int32_t samples, uint32_t interval_us, int32_t* wall_khz,
                              hipStream_t stream);

// per-rank sums and counts of the valid tokens' losses, and their ratio
hipError_t launch_loss_aggregate(const float* token_loss, const uint8_t* valid, int32_t P, int64_t per_rank,
                                 double* rank_sum, int64_t* rank_count, float* loss, hipStream_t stream);

}  // namespace ulysses
