/*
 * ulysses.h -- C ABI of the single-GPU Ulysses sequence-parallel hot path
 * (MI355X / gfx950).
 *
 * The hot path is one GPU's share of an attention layer under Ulysses
 * sequence parallelism:
 *   1. the first all-to-all, sequence shard -> head shard, emulated on one
 *      device as a layout permutation          (ulysses_repack_seq2head)
 *   2. exact softmax attention over the full sequence for the heads this
 *      GPU holds, forward with logsumexp        (ulysses_attn_fwd)
 *      and backward for dQ, dK, dV              (ulysses_attn_bwd)
 *   3. the second all-to-all, head shard -> sequence shard
 *                                               (ulysses_repack_head2seq)
 * and, for packed sequences of variable-length documents, the attention
 * calls with a document mask (ulysses_attn_fwd_docs, ulysses_attn_bwd_docs).
 * For the ring-attention alternative the pages compare against, the
 * forward over one separate key block with an exact merge of partial
 * results (ulysses_attn_fwd_block).
 * Around the path, the projections fused with their exchanges
 * (ulysses_qkv_proj_seq2head, ulysses_head2seq_out_proj).
 * Beside the path: the first exchange fused with the rotary position
 * embedding at global positions (ulysses_repack_seq2head_rope), and the
 * loss aggregated over shards by valid tokens (ulysses_loss_aggregate).
 *
 * Sources (web pages, cited by title and section):
 *   [ALST]  "Paralelismul de Secvență Ulysses: Antrenarea modelelor AI cu
 *           contexte de un milion de token-uri" (world.tibi.club)
 *   [HFSUM] "Ulysses 序列平行化：突破百萬標記長上下文的訓練瓶頸"
 *           (agents-report.net)
 *   [SWIFT] "ms-swift性能优化：Ulysses并行技术降低长文本显存" (hotelren.com)
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every pointer is caller-owned device memory (global memory of the
 *    current HIP device).  The library never allocates or frees device
 *    memory, keeps no pointer after returning, and fully overwrites every
 *    output it is given.  Inputs are never written.
 *  - `stream` is a hipStream_t passed as void*; NULL means the default
 *    stream.  Calls enqueue work and return without synchronising.
 *  - Arguments are validated on the host before anything is launched; on
 *    any error status nothing is launched and no output is touched.
 *  - Element types: ULYSSES_DTYPE_BF16 buffers hold IEEE bfloat16 bit
 *    patterns (uint16), ULYSSES_DTYPE_F32 buffers hold IEEE float32.
 *  - Multi-dimensional buffers are dense and row-major (C order) in the
 *    bracketed shape given for each argument, last index fastest.
 *  - Zero-sized problems (B == 0, or zero tokens) are valid no-ops; pointer
 *    arguments may then be NULL.
 *  - Kernel faults, if any, surface at the caller's next synchronisation of
 *    `stream` as HIP errors; ULYSSES_ERR_HIP reports a failed launch.
 *  - The library holds no mutable global state apart from a per-device
 *    cache of one device address (ulysses_attn_bwd_noalloc's scratch,
 *    filled under a lock): calls are thread-safe and may be issued
 *    concurrently on different streams, except ulysses_attn_bwd_noalloc
 *    calls that overlap on one GPU (they share its scratch).
 */
#ifndef ULYSSES_H_
#define ULYSSES_H_

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define ULYSSES_API __attribute__((visibility("default")))
#else
#define ULYSSES_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ULYSSES_OK = 0,
  ULYSSES_ERR_INVALID_ARG = 1,  /* a null pointer, a bad size, a violated constraint, misalignment, aliasing */
  ULYSSES_ERR_UNSUPPORTED = 2,  /* valid in principle, not built: head dim, dtype combination, size limits */
  ULYSSES_ERR_HIP = 3,          /* a HIP launch failed */
  ULYSSES_ERR_SCRATCH_LIMIT = 4, /* too large for ulysses_attn_bwd_noalloc's fixed scratch */
  ULYSSES_STATUS_MAX_ENUM = 0x7fffffff
} ulysses_status_t;

/* The *_MAX_ENUM values are not codes: they keep each type 32 bits wide, so
   that any non-negative int a C caller passes is a value of the type (the
   library then rejects unknown ones as INVALID_ARG). */
typedef enum {
  ULYSSES_DTYPE_F32 = 0,
  ULYSSES_DTYPE_BF16 = 1,
  ULYSSES_DTYPE_MAX_ENUM = 0x7fffffff
} ulysses_dtype_t;

/* Version of this ABI (incremented on any incompatible change). */
ULYSSES_API int32_t ulysses_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
ULYSSES_API const char* ulysses_status_string(ulysses_status_t status);

/*
 * ulysses_repack_seq2head -- the first all-to-all of Ulysses SP, emulated.
 *
 * Source: [ALST] section "Mecanismul de funcționare Ulysses", step 1 (rank i
 * holds tokens [i*n/P, (i+1)*n/P)) and step 3 (after the exchange every rank
 * holds all positions for a subset of the heads); [HFSUM] section
 * "Ulysses 序列平行化的原理".  Rank j's subset is the contiguous head block
 * [j*H/P, (j+1)*H/P), and received chunks are concatenated in source-rank
 * order, which is global token order.
 *
 *   src  [P][B][n_local][H][D]    the P sequence shards, rank-major
 *   dst  [P][B][P*n_local][H/P][D]  the P head shards, rank-major
 *   dst[j][b][i*n_local + s][h][c] = src[i][b][s][j*H/P + h][c]
 *
 * A pure bit copy: no arithmetic, every bit pattern (NaN payloads included)
 * is preserved.  `dtype` only fixes the element size (2 or 4 bytes).
 * Errors: INVALID_ARG for null src/dst (non-empty problem), P < 1, B < 0,
 * n_local < 0, H < P or H % P != 0 (the head count may not be smaller than
 * the shard count: [HFSUM] section "與 Ring Attention 的比較"), D < 1,
 * an unknown dtype, pointers not aligned to the element size, or
 * overlapping src and dst (no in-place).  UNSUPPORTED if a dimension
 * product exceeds the 32-bit index range of the kernel (2^32 runs).
 */
ULYSSES_API ulysses_status_t ulysses_repack_seq2head(const void* src, void* dst,
                                         int32_t P, int32_t B, int64_t n_local,
                                         int32_t H, int32_t D,
                                         ulysses_dtype_t dtype, void* stream);

/*
 * ulysses_repack_head2seq -- the second all-to-all, emulated: the exact
 * inverse of ulysses_repack_seq2head with the same parameters.
 *
 * Source: [ALST] section "Mecanismul de funcționare Ulysses", step 5 (the
 * second exchange restores the sequence-sharded layout).
 *
 *   src  [P][B][P*n_local][H/P][D]  the P head shards
 *   dst  [P][B][n_local][H][D]      the P sequence shards
 *   dst[i][b][s][j*H/P + h][c] = src[j][b][i*n_local + s][h][c]
 *
 * In the backward pass this same call carries dQ, dK and dV back to the
 * sequence layout (the adjoint of a permutation is its inverse), and
 * ulysses_repack_seq2head carries dO forward.  Errors as for seq2head.
 */
ULYSSES_API ulysses_status_t ulysses_repack_head2seq(const void* src, void* dst,
                                         int32_t P, int32_t B, int64_t n_local,
                                         int32_t H, int32_t D,
                                         ulysses_dtype_t dtype, void* stream);

/*
 * ulysses_attn_fwd -- exact softmax attention over the full sequence for
 * the heads resident on this GPU, with logsumexp.
 *
 * Source: [ALST] section "Mecanismul de funcționare Ulysses", step 4 (each
 * rank runs ordinary scaled-dot-product attention for its heads) and its
 * closing paragraph (heads are independent); [ALST] section "Provocarea
 * antrenării cu secvențe lungi" (tiling keeps memory linear in n while the
 * work stays quadratic); padding keys take no part ([ALST] section
 * "Integrarea cu Accelerate").
 *
 * For batch b, query head h (KV head h / (Hq/Hkv)), query row t:
 *   allowed keys u: (u <= t if causal) and (key_valid == NULL or key_valid[b][u] != 0)
 *   s_u = softmax_scale * <q[b][t][h], k[b][u][kvh]>
 *   o[b][t][h]   = sum_u softmax(s)_u v[b][u][kvh]
 *   lse[b][h][t] = ln sum_u exp(s_u)          (natural log)
 * A row with no allowed key gets o = 0 and lse = -inf.
 *
 *   q          [B][n][Hq][D]   in_dtype
 *   k, v       [B][n][Hkv][D]  in_dtype
 *   key_valid  [B][n] uint8 (nonzero = valid key) or NULL (all valid).
 *              A padding key takes no part in any softmax, but its K and V
 *              rows still enter the matrix products (with weight zero), so
 *              they must hold finite values (0 * Inf is NaN): zeros, or any
 *              finite data, are fine.
 *   o          [B][n][Hq][D]   o_dtype             (output)
 *   lse        [B][Hq][n]      float32             (output)
 *
 * Built combinations: in_dtype BF16 with o_dtype BF16 or F32 (bf16 matrix
 * cores, fp32 accumulation and softmax); in_dtype F32 with o_dtype F32
 * (fp32 throughout).  D must be 64 or 128.
 * Errors: INVALID_ARG for null pointers (non-empty problem), B < 0, n < 0,
 * Hq < 1, Hkv < 1, Hq % Hkv != 0, a scale that is not finite and positive,
 * causal not 0/1,
 * q/k/v/o not 16-byte aligned, lse not 4-byte aligned, or an output
 * overlapping any input or the other output.  UNSUPPORTED for other D or
 * dtype combinations, or n*max(Hq,Hkv)*D >= 2^40 elements.
 */
ULYSSES_API ulysses_status_t ulysses_attn_fwd(const void* q, const void* k, const void* v,
                                  const uint8_t* key_valid,
                                  void* o, float* lse,
                                  int32_t B, int64_t n, int32_t Hq, int32_t Hkv, int32_t D,
                                  float softmax_scale, int32_t causal,
                                  ulysses_dtype_t in_dtype, ulysses_dtype_t o_dtype,
                                  void* stream);

/*
 * Bytes of device workspace ulysses_attn_bwd needs for this problem: two
 * float32 [B][Hq][n] arrays (the per-row dot products dO.O, and the
 * logsumexp in base 2), each rounded up to 256 B, and on short sequences
 * the partial dK and dV of the workgroups that share a key block
 * (2 * S * B * n * Hkv * D float32, S <= 8 chosen from B, n and Hkv: the
 * largest count any kind of backward call takes for the shape).
 */
ULYSSES_API size_t ulysses_attn_bwd_workspace_bytes(int32_t B, int64_t n, int32_t Hq, int32_t Hkv, int32_t D);

/*
 * ulysses_attn_bwd -- gradients of sum(o * dout) with respect to q, k, v.
 *
 * Source: the operation is the backward of ulysses_attn_fwd; the pages do
 * not spell it out (they train with it: [HFSUM] section "最佳實踐與效能結果").
 * The probabilities are recomputed from q, k and lse (memory linear in n,
 * [ALST] section "Provocarea antrenării cu secvențe lungi"):
 *   P = exp(s - lse), dV = P^T dO, dP = dO V^T, Dl = rowsum(dO * O),
 *   dS = P * (dP - Dl), dQ = scale * dS K, dK = scale * dS^T Q,
 * with dK and dV summed over the query heads sharing a KV head.  A padding
 * key (key_valid 0) gets dK = dV = 0 exactly, whatever its K and V rows hold.
 *
 *   q, k, v, key_valid   as for ulysses_attn_fwd (in_dtype)
 *   o          [B][n][Hq][D]   o_dtype   the forward output
 *   lse        [B][Hq][n]      float32   the forward logsumexp
 *   dout       [B][n][Hq][D]   in_dtype  gradient of the output
 *   dq         [B][n][Hq][D]   float32   (output, overwritten)
 *   dk, dv     [B][n][Hkv][D]  float32   (outputs, overwritten)
 *   workspace  device scratch of at least
 *              ulysses_attn_bwd_workspace_bytes(...) bytes, 256-byte
 *              aligned; contents on entry are ignored, on exit undefined.
 *
 * On short sequences (fewer than 1024 work items of the dK/dV pass: pairs
 * of 128-key blocks over B and Hkv when causal, single blocks otherwise)
 * each key block's query rows may be spread over up to 8 workgroups, as many
 * as minimise the pass's length on 256 CUs; they write partial dK/dV into
 * the workspace and a second pass adds them in a fixed order, so the result
 * is the same on every run.  The count depends on the shape and the kind of
 * call (causal, non-causal, documents) only.
 *
 * Built combinations: in_dtype BF16 with o_dtype BF16 or F32; D 64 or 128.
 * Errors: as ulysses_attn_fwd, plus INVALID_ARG for a null or too small
 * workspace, misaligned dq/dk/dv (16 B) or workspace (256 B), and any
 * output (dq, dk, dv, workspace) overlapping an input or another output.
 */
ULYSSES_API ulysses_status_t ulysses_attn_bwd(const void* q, const void* k, const void* v,
                                  const uint8_t* key_valid,
                                  const void* o, const float* lse, const void* dout,
                                  float* dq, float* dk, float* dv,
                                  void* workspace, size_t workspace_bytes,
                                  int32_t B, int64_t n, int32_t Hq, int32_t Hkv, int32_t D,
                                  float softmax_scale, int32_t causal,
                                  ulysses_dtype_t in_dtype, ulysses_dtype_t o_dtype,
                                  void* stream);

/*
 * ulysses_attn_bwd_noalloc -- ulysses_attn_bwd for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving or
 * training loops, harnesses that forbid hipMalloc): the same computation
 * and kernels, with the workspace taken from a fixed scratch array that
 * the library's code object holds on each GPU it runs on (16 MiB, kept
 * until the process ends).  The call itself allocates nothing and frees
 * nothing; the caller passes every input and output as for
 * ulysses_attn_bwd.
 *
 * Limit: 2 * B * Hq * n * 4 bytes <= 16 MiB, i.e. B * Hq * n <= 2^21 rows
 * (the 64K workload's 8 query heads use 2^19).  Larger problems return
 * ULYSSES_ERR_SCRATCH_LIMIT before anything is launched.  The scratch holds
 * only the two row arrays: this call never spreads a key block's query
 * rows over several workgroups (ulysses_attn_bwd does on short sequences,
 * adding partial sums from its workspace), so on short sequences its dK
 * and dV may differ from ulysses_attn_bwd's in float32 rounding; dQ is
 * identical.
 * Every call on a GPU uses that GPU's one scratch array, and nothing in it
 * needs to start at zero (each call writes every value before reading
 * it): calls that overlap in time on one GPU -- on different streams, or
 * from different threads -- race on it and must be serialised by the
 * caller.  The first call on a device looks the array's address up
 * (hipGetSymbolAddress) and keeps it; ULYSSES_ERR_HIP if that fails.
 * Arguments, built combinations and other errors: as ulysses_attn_bwd.
 */
ULYSSES_API ulysses_status_t ulysses_attn_bwd_noalloc(const void* q, const void* k, const void* v,
                                          const uint8_t* key_valid,
                                          const void* o, const float* lse, const void* dout,
                                          float* dq, float* dk, float* dv,
                                          int32_t B, int64_t n, int32_t Hq, int32_t Hkv, int32_t D,
                                          float softmax_scale, int32_t causal,
                                          ulysses_dtype_t in_dtype, ulysses_dtype_t o_dtype,
                                          void* stream);

/*
 * ulysses_attn_fwd_docs -- ulysses_attn_fwd over a packed sequence of
 * documents: causal attention in which a token sees only the tokens of its
 * own document.
 *
 * Source: the trainers' switch for variable sequence lengths ([ALST]
 * section "Integrarea cu Transformers Trainer și TRL SFTTrainer") packs
 * several documents into one sequence; the page names the switch, and the
 * mask here is its plain reading: no token attends across a document
 * boundary.  Padding keys are excluded as in ulysses_attn_fwd ([ALST]
 * section "Integrarea cu Accelerate").
 *
 * For batch b, query head h, query row t, the allowed keys are
 *   doc_start[b][t] <= u <= t  and  (key_valid == NULL or key_valid[b][u] != 0)
 * and everything else is as in ulysses_attn_fwd (o, natural-log lse, a row
 * with no allowed key gets o = 0 and lse = -inf).  Whole tiles of keys
 * outside every row's document are never read.
 *
 *   doc_start  [B][n] int32, device: the position of the first token of
 *              token t's document (pad tokens belong to the document they
 *              follow).  Required: 0 <= doc_start[b][t] <= t and
 *              doc_start[b][t] non-decreasing in t (documents are
 *              contiguous).  Any array meeting these two conditions is
 *              computed exactly (a sliding window, max(0, t - W + 1), is
 *              one).  An array that violates them is not checked (it lives
 *              on the device): no access then leaves the buffers, but the
 *              results are unspecified.
 *   other arguments as for ulysses_attn_fwd; the mask is always causal.
 *
 * Built combinations and errors: as ulysses_attn_fwd, plus INVALID_ARG for
 * a null or not 4-byte aligned doc_start (non-empty problem) and for an
 * output overlapping doc_start.
 */
ULYSSES_API ulysses_status_t ulysses_attn_fwd_docs(const void* q, const void* k, const void* v,
                                       const uint8_t* key_valid, const int32_t* doc_start,
                                       void* o, float* lse,
                                       int32_t B, int64_t n, int32_t Hq, int32_t Hkv, int32_t D,
                                       float softmax_scale,
                                       ulysses_dtype_t in_dtype, ulysses_dtype_t o_dtype,
                                       void* stream);

/*
 * ulysses_attn_bwd_docs -- gradients of ulysses_attn_fwd_docs: the
 * backward of ulysses_attn_bwd restricted to the same document mask
 * (doc_start as for ulysses_attn_fwd_docs; o and lse from that call).
 * The workspace size is ulysses_attn_bwd_workspace_bytes(...).  Each key's
 * dK/dV gather only the query rows of its own document, and the tiles of
 * rows past the end of that document are never read.
 *
 * Built combinations and errors: as ulysses_attn_bwd, plus INVALID_ARG for
 * a null or not 4-byte aligned doc_start (non-empty problem) and for an
 * output overlapping doc_start.
 */
ULYSSES_API ulysses_status_t ulysses_attn_bwd_docs(const void* q, const void* k, const void* v,
                                       const uint8_t* key_valid, const int32_t* doc_start,
                                       const void* o, const float* lse, const void* dout,
                                       float* dq, float* dk, float* dv,
                                       void* workspace, size_t workspace_bytes,
                                       int32_t B, int64_t n, int32_t Hq, int32_t Hkv, int32_t D,
                                       float softmax_scale,
                                       ulysses_dtype_t in_dtype, ulysses_dtype_t o_dtype,
                                       void* stream);

/*
 * ulysses_attn_fwd_block -- the forward of ulysses_attn_fwd over one
 * separate block of keys, optionally merged into a running result: the
 * step a rank of Ring Attention takes at each hop.
 *
 * Source: Ring Attention keeps each rank's query shard and passes the
 * key/value shards around a ring in P - 1 point-to-point hops ([HFSUM]
 * section "與 Ring Attention 的比較"; [ALST] sections "Complexitatea
 * comunicațională" and "Comparând Ulysses cu Ring Attention").  The pages
 * do not say how the hops' results combine; the exact combination of
 * softmax attentions over disjoint key sets is used:
 *   L = ln(e^L_old + e^L_blk),  O = e^(L_old - L) O_old + e^(L_blk - L) O_blk
 *
 * For batch b, query head h (KV head h / (Hq/Hkv)), block row t:
 *   allowed keys u of the block: (u <= t + causal_offset if causal) and
 *   (key_valid == NULL or key_valid[b][u] != 0)
 * and O_blk, L_blk are the attention and logsumexp over those keys (a row
 * with none gets O_blk = 0, L_blk = -inf).  For query rows at global
 * positions q0.. and keys at k0.., causal_offset = q0 - k0.
 *
 *   q          [B][nq][Hq][D]   bf16
 *   k, v       [B][nk][Hkv][D]  bf16
 *   key_valid  [B][nk] uint8 or NULL
 *   o          [B][nq][Hq][D]   float32  accumulate = 0: overwritten with O_blk;
 *                                        accumulate = 1: holds O_old, replaced by O
 *   lse        [B][Hq][nq]      float32  likewise L_blk, or L_old -> L (natural log)
 *   causal_offset  any value; values past [-nq, nk] act as the nearest end
 *   causal     1: the mask above; 0: every key of the block is visible
 *
 * Built: bf16 inputs, D 64 or 128 (the bf16 forward's kernels).
 * Errors: as ulysses_attn_fwd (with nq as n), plus INVALID_ARG for nk < 1
 * or accumulate not 0/1; UNSUPPORTED for float32 inputs or nq + nk >= 2^31.
 */
ULYSSES_API ulysses_status_t ulysses_attn_fwd_block(const void* q, const void* k, const void* v,
                                        const uint8_t* key_valid, float* o, float* lse,
                                        int32_t B, int64_t nq, int64_t nk, int32_t Hq, int32_t Hkv,
                                        int32_t D, float softmax_scale, int64_t causal_offset,
                                        int32_t causal, int32_t accumulate,
                                        ulysses_dtype_t in_dtype, void* stream);

/*
 * ulysses_repack_seq2head_rope -- ulysses_repack_seq2head with the rotary
 * position embedding applied on the way, at each token's global position.
 *
 * Source: the rotary encoding must follow a shard's offset in the sequence
 * ([SWIFT] section "6. 使用建议与避坑指南", troubleshooting table: repeated
 * tokens when it does not; linear position scaling named as a workaround);
 * shards are contiguous ([ALST] "Mecanismul de funcționare Ulysses", step
 * 1), so rank i's local token s has global position pos = i*n_local + s.
 * The rotation (not on the pages; the form of the pages' Qwen models) pairs
 * dimension d with d + D/2, for d in [0, D/2):
 *   theta = (pos / rope_scale) * rope_base^(-2d/D)
 *   out[d]       = x[d] cos(theta) - x[d+D/2] sin(theta)
 *   out[d+D/2]   = x[d+D/2] cos(theta) + x[d] sin(theta)
 * then out lands where ulysses_repack_seq2head would put x:
 *   dst[j][b][i*n_local + s][h][c] = out(src[i][b][s][j*H/P + h])[c]
 *
 *   src, dst   as for ulysses_repack_seq2head (Q or K; V takes the plain call)
 *   rope_base  rotary base (> 0, finite; 1e6 for the workloads' Qwen heads)
 *   rope_scale linear position scaling factor (> 0, finite; 1 = none)
 *
 * Arithmetic: angles in double precision (reduced to [-pi, pi] before the
 * sine and cosine), the rotation in float32, one rounding to dtype.
 * Built: dtype BF16 or F32, D 64 or 128.
 * Errors: as ulysses_repack_seq2head, plus INVALID_ARG for a base or scale
 * that is not finite and positive and for src/dst not 16-byte aligned;
 * UNSUPPORTED for other D, n_local >= 2^31 or P*B*n_local >= 2^37.
 */
ULYSSES_API ulysses_status_t ulysses_repack_seq2head_rope(const void* src, void* dst,
                                              int32_t P, int32_t B, int64_t n_local,
                                              int32_t H, int32_t D,
                                              double rope_base, double rope_scale,
                                              ulysses_dtype_t dtype, void* stream);

/*
 * ulysses_qkv_proj_seq2head -- the QKV projection of every sequence shard
 * fused with the first exchange: the projected heads are written straight
 * into the head-sharded layout.
 *
 * Source: [ALST] "Mecanismul de funcționare Ulysses", steps 2-3 (each rank
 * projects query, key and value for its own shard, then the first
 * all-to-all); [HFSUM] "Ulysses 序列平行化的原理".  The weight layout is a
 * reading: W is [out features][in features] and stacks the Hq query heads,
 * the Hkv key heads and the Hkv value heads, D features each.
 *
 *   x   [P][B][n_local][hidden]   bf16, the sequence shards
 *   w   [(Hq + 2 Hkv) * D][hidden] bf16
 *   q   [P][B][P*n_local][Hq/P][D]  bf16 (output)   q[j][b][i*n_local + s][h][c] =
 *       sum_e x[i][b][s][e] * w[(j*Hq/P + h)*D + c][e]
 *   k, v [P][B][P*n_local][Hkv/P][D] bf16 (outputs), rows (Hq + head)*D + c and
 *       (Hq + Hkv + head)*D + c of w likewise
 *
 * Arithmetic: bf16 products on the matrix cores, float32 accumulation, one
 * rounding to bf16.  Errors: INVALID_ARG for P < 1, B < 0, n_local < 0,
 * sizes < 1, Hq or Hkv not divisible by P, null or not 16-byte aligned
 * pointers (non-empty problem), any output overlapping an input or another
 * output; UNSUPPORTED for D other than 64 and 128, hidden not a multiple
 * of 64, or sizes past the kernel's index range.
 */
ULYSSES_API ulysses_status_t ulysses_qkv_proj_seq2head(const void* x, const void* w,
                                           void* q, void* k, void* v,
                                           int32_t P, int32_t B, int64_t n_local, int32_t hidden,
                                           int32_t Hq, int32_t Hkv, int32_t D, void* stream);

/*
 * ulysses_head2seq_out_proj -- the second exchange fused with each shard's
 * output projection: the attention output is read straight from the
 * head-sharded layout.
 *
 * Source: [ALST] "Mecanismul de funcționare Ulysses", steps 5-6 (the second
 * all-to-all restores the sequence sharding, then each rank's output
 * projection of its shard).  Reading: a token's attention output is its Hq
 * heads concatenated in head order; W_o is [hidden][Hq * D].
 *
 *   o    [P][B][P*n_local][Hq/P][D]  bf16, the attention output, head-sharded
 *   w_o  [hidden][Hq * D]            bf16
 *   y    [P][B][n_local][hidden]     bf16 (output)
 *        y[i][b][s][f] = sum_{h,c} o[h / (Hq/P)][b][i*n_local + s][h % (Hq/P)][c] * w_o[f][h*D + c]
 *
 * Arithmetic as ulysses_qkv_proj_seq2head.  Errors: INVALID_ARG as there
 * (with Hq % P), y overlapping o or w_o; UNSUPPORTED for D other than 64 and
 * 128, (Hq/P)*D not a multiple of 64, hidden not a multiple of 4, or sizes
 * past the kernel's index range.
 */
ULYSSES_API ulysses_status_t ulysses_head2seq_out_proj(const void* o, const void* w_o, void* y,
                                           int32_t P, int32_t B, int64_t n_local,
                                           int32_t Hq, int32_t D, int32_t hidden, void* stream);

/*
 * ulysses_loss_aggregate -- the loss of a sequence split over P ranks,
 * weighted by each rank's valid tokens.
 *
 * Source: [ALST] section "Integrarea cu Accelerate" (each rank's loss covers
 * its part of the sequence; the losses are combined weighted by the number
 * of valid tokens per rank, padding and masked prompt tokens excluded) and
 * section "Cele mai bune practici și recomandări", item 6.
 *
 *   token_loss [P][per_rank] float32   per-token losses of each rank's shard
 *                                      (per_rank = B * n_local)
 *   valid      [P][per_rank] uint8     nonzero = counted, or NULL (all counted)
 *   rank_sum   [P] float64  (output)   sum of rank r's counted losses
 *   rank_count [P] int64    (output)   number of rank r's counted tokens
 *   loss       [1] float32  (output)   sum of rank_sum / sum of rank_count,
 *                                      NaN when nothing is counted
 *
 * Sums are accumulated in double precision in a fixed order (deterministic).
 * Errors: INVALID_ARG for P < 1 or P > 65535, per_rank < 0, a null output,
 * a null token_loss with per_rank > 0, misalignment (token_loss and loss 4
 * bytes, rank_sum and rank_count 8), or an output overlapping an input or
 * another output.
 */
ULYSSES_API ulysses_status_t ulysses_loss_aggregate(const float* token_loss, const uint8_t* valid,
                                        int32_t P, int64_t per_rank,
                                        double* rank_sum, int64_t* rank_count, float* loss,
                                        void* stream);

/*
 * ulysses_clock_probe -- a measurement aid, not a step of the path: samples
 * the engine (shader) clock while another kernel runs.
 *
 * The matrix-core peak scales with the engine clock, which under sustained
 * matrix work runs below its maximum; a rate measured against the nominal
 * peak is also reported against the peak at the clock actually sustained.
 * One wave, launched on `stream` (a second stream beside the measured
 * kernel's), records every interval_us microseconds the pair
 *   out[2s]     real-time counter stamp (constant rate, *wall_khz kHz)
 *   out[2s + 1] shader cycles elapsed since the previous sample
 * for s = 0 .. samples-1, so the clock over sample s is
 *   out[2s+1] / ((out[2s] - out[2s-2]) / (*wall_khz * 1e3))   Hz.
 * The wave needs a few registers and no LDS, so it runs beside the attention
 * kernels' waves.  It ends after samples * interval_us microseconds (each
 * wait is also bounded by a fixed number of polls).
 *
 *   out       [2 * samples] uint64, device, 8-byte aligned (output)
 *   wall_khz  host int32 (output): the real-time counter's rate, kHz
 * Errors: INVALID_ARG for a null or misaligned out, a null wall_khz,
 * samples outside [1, 65536] or interval_us outside [1, 10^6].
 */
ULYSSES_API ulysses_status_t ulysses_clock_probe(uint64_t* out, int32_t samples, int32_t interval_us,
                                     int32_t* wall_khz, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ULYSSES_H_ */
