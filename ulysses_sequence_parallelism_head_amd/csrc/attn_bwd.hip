// attn_bwd.hip -- backward of exact causal grouped-query softmax attention,
// bf16 inputs on gfx950 matrix cores, float32 gradients.
//
// The operation is the gradient of sum(O * dO) of the forward in
// attn_fwd.hip ([ALST] "Paralelismul de Secvență Ulysses: Antrenarea
// modelelor AI cu contexte de un milion de token-uri", section "Mecanismul
// de funcționare Ulysses", step 4); the probabilities are recomputed from
// the saved logsumexp so memory stays linear in n (same page, section
// "Provocarea antrenării cu secvențe lungi").
//
//   P = exp(S - lse)      dV = P^T dO        dP = dO V^T
//   Dl = rowsum(dO * O)   dS = P * (dP - Dl) dQ = scale dS K   dK = scale dS^T Q
//
// Two kernels (and a reduction of partial dK/dV when a key block's work is
// split over several workgroups), dq first:
//  1. dq (Q-stationary, laid out like the forward): each wave first forms
//     Dl = dO . O and the base-2 logsumexp of its rows and stores them in the
//     workspace for dkdv; then it recomputes S^T = K Q^T and dP^T = V dO^T
//     with the query on the lane and accumulates dQ^T += K^T dS^T, the K^T
//     operand read transposed from the row-major K tile.  Keeping dQ in its
//     own pass avoids float32 atomics (whose traffic would grow as n^2 /
//     block) and makes every gradient deterministic.
//  2. dkdv (KV-stationary): a workgroup of 8 waves owns 128 keys of one KV
//     head (4 groups of 32 keys, two waves per group) and streams the 64-row
//     query tiles of every query head of the group that can see them (for
//     causal attention, two key blocks in turn, ordered so that resident
//     workgroups read the same tiles at the same time).  In each group one
//     wave holds the K rows and computes S = Q K^T, P and dV^T += dO^T P, the
//     other holds the V rows and computes dP = dO V^T, dS and dK^T += Q^T dS,
//     receiving P through LDS; the key is on the lane, so P and dS come out
//     as MFMA B operands.  Q and dO are staged once, row-major with swizzled
//     chunks; the Q^T and dO^T operands come from transposing LDS reads
//     (ds_read_b64_tr_b16).  Splitting a group's work over two waves halves
//     each wave's registers, so two waves share a SIMD and one's
//     exponentials and waits overlap the other's matrix work.
// Masks run only on the tiles that need them, chosen per run of tiles
// outside the loops: dkdv applies the causal compare on the two query tiles
// at a key block's diagonal and no per-key mask at all (a padding key's P
// and dS reach only its own dK/dV column, written as zero); dq applies the
// causal and tail compares on the diagonal and tail tiles.
// Rows below kSplitRows use a hi/lo bf16 split of P and dS (two MFMAs) for
// accuracy where few keys carry large weights.
// Packed documents (a per-row lower bound on the visible keys, the first
// position of the row's document): dq starts at the tile holding its first
// row's bound, as the forward does; a dkdv workgroup finds the end of the
// last document its keys belong to (a 64-lane search over the bounds) and
// visits only the query tiles up to it, sweeping down from there so that the
// workgroups of one document read the same tiles at the same time.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace ulysses {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kSplitRows = 512;   // a multiple of both query tile heights (64)
constexpr int kDqSplitBlocks = 512;   // dq grids up to this size take the key split
constexpr int kDqWideBlocks = 512;    // 8-wave dq grids from this size on share each K/V tile
constexpr float kLog2e = 1.4426950408889634f;

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint8_t* valid;
  const int32_t* doc_start;   // [B][n] first position of each row's document, or null
  const void* o;
  const float* lse;
  const uint16_t* dout;
  float* dq;
  float* dk;
  float* dv;
  float* rowdot;      // [B][Hq][n] -(dO . O) (workspace)
  float* lse2;        // [B][Hq][n] lse * log2(e), +inf for empty rows (workspace)
  float* dk_part;     // [nsplit][B][n][Hkv][D] partial dK of each split (workspace; nsplit > 1)
  float* dv_part;     // [nsplit][B][n][Hkv][D] partial dV
  int32_t nsplit;     // workgroups sharing one key block's query units (a power of two)
  int32_t lsplit;     // log2(nsplit)
  int32_t B, n, Hq, Hkv, g;
  float scale;
  float c;            // scale * log2(e)
  int32_t causal;
  int32_t o_f32;       // O is float32 (else bf16)
  // dq grid (same as the forward)
  int32_t gh, pw, n_pblocks, n_hsub;
  // dkdv grid
  int32_t n_kblocks;
};

// ------------------------------------------------------------------- dkdv
// Pack 8 floats (x[0..7]) as the bf16 B operand of one MFMA, and optionally
// the bf16 residual x - bf16(x) as a second operand.
__device__ __forceinline__ u32x4 pack8(const float* x) {
  return u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
}

__device__ __forceinline__ u32x4 pack8_residual(const float* x, const u32x4 hi) {
  float r[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[2 * e] = x[2 * e] - bf16lo_to_f32(hi[e]);
    r[2 * e + 1] = x[2 * e + 1] - bf16hi_to_f32(hi[e]);
  }
  return pack8(r);
}

// End (exclusive) of the rows that can see key `klast`: the first row t >
// klast whose bound exceeds klast, or n.  The bounds never decrease along a
// batch row, so the answer is found by a search over positions: each round
// the 64 lanes probe 64 evenly spaced rows of the remaining range and the
// first probe above klast narrows it to one gap (three rounds for 2^18
// rows).  Every probe is in [klast+1, n), whatever the array holds.
__device__ __forceinline__ int doc_rows_end(const int32_t* rs, int klast, int n, int lane) {
  int lo = klast + 1, hi = n;           // the answer lies in [lo, hi]
  while (lo < hi) {
    const int step = (hi - lo + 63) / 64;
    const int pos = lo + lane * step;
    const bool above = pos < hi && rs[pos] > klast;
    const uint64_t m = __ballot(above);
    if (m == 0) {
      // every probe below hi is at or under klast: the answer is past the last one
      const int last = min(63, (hi - 1 - lo) / step);
      lo = lo + last * step + 1;
    } else {
      const int j = __builtin_ctzll(m);
      hi = lo + j * step;
      if (j > 0) lo = lo + (j - 1) * step + 1;
    }
  }
  return lo;
}

// Run of key block kb (128 keys; last key klast): the blocks whose last key
// lies between the bound of kb's last key and the end of the rows that see
// it, [r0, r1) = [bound / 128, rend / 128) (r1 = nkb when rend = n).  For
// documents these are the blocks whose last keys share a document.  The
// partner r0 + r1 - 1 - kb is used only if it computes the same run, so the
// pairing is an involution whatever the bounds hold; otherwise kb is done
// alone.  Both indices always stay in [0, nkb).
__device__ __forceinline__ int docs_run_end(const int32_t* rs, int kb, int n, int nkb, int lane, int* r0) {
  const int klast = min(kb * 128 + 127, n - 1);
  const int rend = doc_rows_end(rs, klast, n, lane);
  *r0 = doc_lower(rs, klast) / 128;
  return rend >= n ? nkb : rend / 128;
}

__device__ __forceinline__ int docs_partner(const int32_t* rs, int kb, int n, int nkb, int lane) {
  int r0, q0;
  const int r1 = docs_run_end(rs, kb, n, nkb, lane, &r0);
  const int partner = r0 + r1 - 1 - kb;
  if (partner == kb) return kb;
  const int q1 = docs_run_end(rs, partner, n, nkb, lane, &q0);
  return (q0 == r0 && q1 == r1) ? partner : kb;
}

// Sum of the splits' partial dK and dV in split order: out[i] = sum_s part[s][i]
// (a fixed order, so the result does not depend on scheduling); the first
// `blocks` workgroups take dK, the rest dV.
__global__ __launch_bounds__(256) void dkdv_reduce_kernel(const float* part_k, float* out_k, const float* part_v,
                                                          float* out_v, int64_t count, int32_t nsplit, int32_t blocks) {
  const bool is_v = int32_t(blockIdx.x) >= blocks;
  const float* part = is_v ? part_v : part_k;
  float* out = is_v ? out_v : out_k;
  const int64_t i = (int64_t(blockIdx.x) - (is_v ? blocks : 0)) * 1024 + int64_t(threadIdx.x) * 4;
  if (i >= count) return;
  f32x4 acc = *reinterpret_cast<const f32x4*>(part + i);
  for (int32_t sp = 1; sp < nsplit; ++sp) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(part + sp * count + i);
    acc = f32x4{acc[0] + x[0], acc[1] + x[1], acc[2] + x[2], acc[3] + x[3]};
  }
  *reinterpret_cast<f32x4*>(out + i) = acc;
}

// dkdv (KV-stationary): a workgroup of 8 waves owns 128 keys of one KV head
// as 4 groups of 32, two waves per group on one SIMD.  The P wave holds the
// group's K rows and computes S = Q K^T, P and dV^T += dO^T P; the dS wave
// holds the V rows and computes dP = dO V^T, dS = P (dP - Dl) and
// dK^T += Q^T dS.  Both have the key on the lane, so P and dS come out as
// MFMA B operands, and P passes from one wave to the other through LDS, lane
// to the same lane, in float32.  Each wave keeps one accumulator set and one
// operand set, so two waves fit on a SIMD (256 registers each), and one
// wave's exponentials, operand reads and waits overlap the other wave's
// matrix work.  Q and dO are staged once per unit, row-major with swizzled
// chunks; the Q^T and dO^T operands come from transposing LDS reads.
constexpr int kPairWaves = 8;
constexpr int kPairThreads = kPairWaves * 64;
constexpr int kRowAhead = 6;  // row-major operands read ahead of their MFMAs
constexpr int kTrAhead = 3;   // transposed operands read ahead of their MFMAs

template <int D, bool DOCS>
struct DkdvPairLayout {
  static constexpr int kRows = 64;                         // query rows per unit
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kTile = kRows * kRowBytes;          // one bf16 row-major tile
  // a stage: Q, dO, the base-2 logsumexp, Dl and (documents) the rows' bounds
  static constexpr int kSQ = 0;
  static constexpr int kSDO = kTile;
  static constexpr int kSLSE = 2 * kTile;
  static constexpr int kSDL = kSLSE + kRows * 4;
  static constexpr int kSLO = kSDL + kRows * 4;
  static constexpr int kStage = (kSLO + (DOCS ? kRows * 4 : 0) + 127) / 128 * 128;
  // two stages, then P of the 4 key groups: 64 lanes x 32 floats (two 32-row blocks) each
  static constexpr int kOffX = 2 * kStage;
  static constexpr int kXGroup = 64 * 32 * 4;
  static constexpr int kBytes = kOffX + 4 * kXGroup;
};

// DMA unit tile t0 .. t0+63 of query head `head` for the two-wave kernel: Q,
// dO, the base-2 logsumexp, Dl (and the rows' bounds) into stage `st` (rows
// past n read as zero), by NWI waves (`wave` counts among them).
template <int D, bool DOCS, int NWI = kPairWaves>
__device__ __forceinline__ void dkdv_pair_issue(uint8_t* st, const BwdParams& p, int b, int head, int t0, int wave,
                                                int lane) {
  using X = DkdvPairLayout<D, DOCS>;
  const int rows_ok = min(X::kRows, p.n - t0);
  const int64_t off = ((int64_t(b) * p.n + t0) * p.Hq + head) * D;
  const int stride = p.Hq * D * 2;
  // NWI issuing waves (8 or 4): each covers the shares of 8 / NWI waves of
  // the 8-wave layout, one batch at a time
#pragma unroll
  for (int h = 0; h < kPairWaves / NWI; ++h) {
    dma_tile<D, X::kRows, kPairWaves>(st + X::kSQ, p.q + off, stride, rows_ok, wave + h * NWI, lane);
    dma_tile<D, X::kRows, kPairWaves>(st + X::kSDO, p.dout + off, stride, rows_ok, wave + h * NWI, lane);
  }
  const int64_t roff = (int64_t(b) * p.Hq + head) * p.n + t0;
  if (wave == 0) dma4(buffer_rsrc(p.lse2 + roff, uint32_t(rows_ok) * 4u), st + X::kSLSE, lane * 4);
  if (wave == 1) dma4(buffer_rsrc(p.rowdot + roff, uint32_t(rows_ok) * 4u), st + X::kSDL, lane * 4);
  if (DOCS && wave == 2)
    dma4(buffer_rsrc(p.doc_start + int64_t(b) * p.n + t0, uint32_t(rows_ok) * 4u), st + X::kSLO, lane * 4);
}

// Software pipeline of N matrix-core steps that each take one A operand
// from LDS: the operands of the first AH steps are read first, then step t
// issues its MFMAs together with the read for step t + AH, and a scheduling
// fence after every step keeps that order (the compiler's latency model
// takes LDS reads as short and would otherwise read each operand just
// before its MFMA).  `before` runs between the first reads and the first
// step.
template <int AH, int N, typename Load, typename Before, typename Step>
__device__ __forceinline__ void lds_pipeline(Load&& load, Before&& before, Step&& step) {
  static_assert(AH >= 1 && AH <= N, "read-ahead within the steps");
  u32x4 win[AH];
#pragma unroll
  for (int t = 0; t < AH; ++t) win[t] = load(t);
  __builtin_amdgcn_sched_barrier(0);
  before();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < N; ++t) {
    const u32x4 a = win[t % AH];
    if (t + AH < N) win[t % AH] = load(t + AH);
    step(t, a);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The lane index from an instruction the compiler cannot merge or move:
// values derived from it are computed where they are used, not hoisted
// above branches and loops where they would hold registers throughout.
__device__ __forceinline__ int opaque_lane_id() {
  int lane;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
  return lane;
}

// P of one 32-row block of the staged tile (rows rb*32 + (i/4)*8 + 4hh + i%4,
// key u on the lane) from the scores s.  DIAG applies the causal mask (only
// tiles that reach above the block's last key need it), LOWER the rows'
// document bounds (key u is visible to row t only if u >= bound).  Invisible
// keys, and rows with no visible key (base-2 LSE = +inf), get exponent -inf:
// exp2(-inf) = 0 exactly.  A key that is padding or past n is not masked
// here: its P and dS reach only its own column of dV^T and dK^T (the lane's
// key), which the epilogue writes as zero.
template <bool CAUSAL, bool DIAG, bool LOWER>
__device__ __forceinline__ void dkdv_probs(const float* lses, const int32_t* los, const f32x16& s, int rb, int t0,
                                           int u, int hh, float c, float (&pr)[16]) {
  const int lim = (CAUSAL && DIAG) ? u - t0 - 4 * hh : -0x7fffffff;
#pragma unroll
  for (int g4 = 0; g4 < 4; ++g4) {
    const int rr = rb * 32 + g4 * 8 + hh * 4;
    const f32x4 l4 = *reinterpret_cast<const f32x4*>(lses + rr);
    i32x4 b4 = i32x4{0, 0, 0, 0};
    if (LOWER) b4 = *reinterpret_cast<const i32x4*>(los + rr);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = g4 * 4 + e;
      const int ci = rb * 32 + g4 * 8 + e;
      const bool ok = (!(CAUSAL && DIAG) || ci >= lim) && (!LOWER || b4[e] <= u);
      const float x = ok ? fmaf(s[i], c, -l4[e]) : -INFINITY;
      pr[i] = __builtin_amdgcn_exp2f(x);
    }
  }
}

// Work items and tile order.  A work item is one key block (non-causal) or,
// for causal attention, the pair of key blocks (nkb-1-w, w): the first one
// sweeps the query tiles from the last down to its diagonal, the second from
// its diagonal up to the last, so every pair does the same number of tiles.
// Query heads of the group are the innermost loop.  With this order every
// resident workgroup reads, at unit U, either tile ntq-1-U/g (first phase) or
// tile U/g + 2nkb-2-ntq (second phase) of query head U%g: the workgroups of
// one XCD share two tiles at a time, which the XCD's L2 keeps.
// With documents the same pairing is made inside each run of key blocks
// whose last keys lie in one document (they share the end of their rows):
// block r0 + t goes with block r1 - 1 - t, the later one swept down from the
// document's last tile, then the earlier one up to it, so the pairs of a
// run do equal work and read the same tile at the same time.  The workgroup
// of the earlier block does the pair; the later block's exits at once.
// Which blocks form a run is read from the bounds (see docs_partner below).
template <int D, bool HAS_MASK, bool CAUSAL, bool DOCS>
__global__ __launch_bounds__(kPairThreads, 1) void dkdv_pair_kernel(const BwdParams p) {
  static_assert(CAUSAL || !DOCS, "documents are causal");
  using X = DkdvPairLayout<D, DOCS>;
  constexpr int KK = D / 16;
  constexpr int DJ = D / 32;
  constexpr int kKeys = 128;                      // keys per workgroup (4 groups x 32)
  __shared__ __attribute__((aligned(128))) uint8_t smem[X::kBytes];

  const int tid = threadIdx.x;
  // scalar wave index: every branch around a matrix-core instruction is wave-uniform
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw = wave & 3;                        // key group; waves kw and kw + 4 share it
  const int lane0 = tid & 63;
  float* xp = reinterpret_cast<float*>(smem + X::kOffX + kw * X::kXGroup);

  // block -> (split, work item, kv head, batch); split fastest, then kv head
  const int sp = int(blockIdx.x) & (p.nsplit - 1);
  const int bid = int(blockIdx.x) >> p.lsplit;
  const int per_w = p.Hkv * p.B;
  const int w = bid / per_w;
  const int rem = bid % per_w;
  const int b = rem / p.Hkv;
  const int kvh = rem % p.Hkv;
  const int ntq = (p.n + X::kRows - 1) / X::kRows;
  int nph = (CAUSAL && p.n_kblocks - 1 - w != w) ? 2 : 1;
  int kb_first = p.n_kblocks - 1 - w;
  if (DOCS) {
    kb_first = docs_partner(p.doc_start + int64_t(b) * p.n, w, p.n, p.n_kblocks, lane0);
    if (kb_first < w) return;           // uniform across the workgroup: no barrier passed yet
    nph = kb_first == w ? 1 : 2;
  }

  // the whole sweep of one role; the two roles run the same units and meet
  // at the same barriers
  auto go = [&](auto role_tag) __attribute__((always_inline)) {
    constexpr bool PW = decltype(role_tag)::value;   // P wave (else dS wave)
    // (per role: derived values are not kept live through the other role's loops)
    const int lane = opaque_lane_id();
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    for (int ph = 0; ph < nph; ++ph) {
      const bool down = CAUSAL && ph == 0;
      const int kb = down ? kb_first : w;
      const int k0w = kb * kKeys + kw * 32;
      const int u = k0w + l32;
      const bool wave_live = k0w < p.n;

      // K rows (P wave) or V rows (dS wave) of this lane's key as B operands
      u32x4 kv[KK];
      bool key_ok = u < p.n;
      {
        const uint16_t* src = PW ? p.k : p.v;
        const int lk = opaque_lane_id();   // (the row address is formed here, not kept across phases)
        const int uk = k0w + (lk & 31);
        const int64_t off = ((int64_t(b) * p.n + (key_ok ? uk : 0)) * p.Hkv + kvh) * D + 8 * (lk >> 5);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          kv[kk] = key_ok ? *reinterpret_cast<const u32x4*>(src + off + 16 * kk) : u32x4{0, 0, 0, 0};
        if (HAS_MASK && key_ok) key_ok = p.valid[int64_t(b) * p.n + u] != 0;
      }
      f32x16 acc[DJ];                    // dV^T (P wave) or dK^T (dS wave)
#pragma unroll
      for (int j = 0; j < DJ; ++j) acc[j] = f32x16{};

      const int tfirst = CAUSAL ? (kb * kKeys) / X::kRows : 0;
      int tend = ntq;
      int split_end = kSplitRows;
      bool lower = false;
      if (DOCS) {
        const int32_t* rs = p.doc_start + int64_t(b) * p.n;
        const int kfirst = kb * kKeys;
        const int klast = min(kfirst + kKeys, p.n) - 1;
        const int rend = doc_rows_end(rs, klast, p.n, lane);
        tend = (rend + X::kRows - 1) / X::kRows;
        split_end = doc_lower(rs, rend - 1) + kSplitRows;
        lower = doc_lower(rs, min(tend * X::kRows, p.n) - 1) > kfirst;
      }
      const int niter = (tend - tfirst) * p.g;
      auto tile_of = [&](int it) { return down ? tend - 1 - it / p.g : tfirst + it / p.g; };
      const int u0 = __builtin_amdgcn_readfirstlane((niter * sp) >> p.lsplit);
      const int u1 = __builtin_amdgcn_readfirstlane((niter * (sp + 1)) >> p.lsplit);

      // unit it's stage: it % 2.  The byte offset passes through an opaque
      // scalar: the compiler then forms each address where it is used (base
      // + lane offset + immediate) instead of precomputing one register per
      // stage and operand ahead of the loops.
      auto sbuf = [&](int it) {
        int off = (it & 1) * X::kStage;
        asm volatile("" : "+s"(off));
        return smem + off;
      };
      if (u0 < u1) dkdv_pair_issue<D, DOCS>(sbuf(u0), p, b, kvh * p.g + u0 % p.g, tile_of(u0) * X::kRows, wave, lane);
      wait_vmem();
      __syncthreads();

      // Unit it, in two halves separated by a barrier:
      //   P wave:  S = Q K^T, P, store P | dV^T += dO^T P
      //   dS wave: dP = dO V^T           | load P, dS, dK^T += Q^T dS
      // then a barrier before the other stage is refilled and the P slot
      // rewritten.
      auto run = [&](int it0, int it1, auto split_tag, auto diag_tag, auto lower_tag) __attribute__((always_inline)) {
        constexpr bool SPLIT = decltype(split_tag)::value;
        constexpr bool DIAG = decltype(diag_tag)::value;
        constexpr bool LOWER = decltype(lower_tag)::value;
        // P (P wave) or dS (dS wave) as bf16 B operands: hi, and the
        // residual lo with SPLIT
        u32x4 bh[2][2], bl[2][2];
        // the products with transposed A operands from tile `ts` for 32-row
        // blocks RB0 .. RB0+NRB-1, step t = (rb, f, j) = (RB0 + t / 2DJ,
        // t / DJ % 2, t % DJ)
        auto tr_products = [&](const uint8_t* ts, auto rb0_tag, auto nrb_tag) __attribute__((always_inline)) {
          constexpr int RB0 = decltype(rb0_tag)::value;
          constexpr int NRB = decltype(nrb_tag)::value;
          lds_pipeline<SPLIT ? kTrAhead - 1 : kTrAhead, NRB * 2 * DJ>(
              [&](int t) {
                return tr_operand<X::kRowBytes>(ts, (RB0 + t / (2 * DJ)) * 32 + 16 * (t / DJ % 2), 32 * (t % DJ),
                                                lane);
              },
              [] {},
              [&](int t, const u32x4 a) {
                acc[t % DJ] = mfma32x32x16(a, bh[RB0 + t / (2 * DJ)][t / DJ % 2], acc[t % DJ]);
                if (SPLIT) acc[t % DJ] = mfma32x32x16(a, bl[RB0 + t / (2 * DJ)][t / DJ % 2], acc[t % DJ]);
              });
        };
        // unit it's tile, and the next unit's tile and head, advanced by
        // additions (wave-uniform scalars)
        int tile = tile_of(it0);
        int ntile = tile_of(it0 + 1), nhead = (it0 + 1) % p.g;
        const int tstep = down ? -1 : 1;
        for (int it = it0; it < it1; ++it) {
          // the dS waves alone stage the next unit: the P waves, which the SIMD
          // issues first, go straight to the score products on the critical
          // chain (1-3 % on most shapes)
          if constexpr (!PW) {
            if (it + 1 < u1)
              dkdv_pair_issue<D, DOCS, 4>(sbuf(it + 1), p, b, kvh * p.g + nhead, ntile * X::kRows, wave - 4, lane);
          }
          const int t0 = tile * X::kRows;
          const uint8_t* st = sbuf(it);
          const uint8_t* qs = st + X::kSQ;
          const uint8_t* dos = st + X::kSDO;
          f32x16 sc[2];                  // S (P wave) or dP (dS wave)
          if (wave_live) {
            // S = Q K^T (P wave) or dP = dO V^T (dS wave); step t = (kk, rb) =
            // (t / 2, t % 2), A operand row-major from the tile
            const uint8_t* as = PW ? qs : dos;
            if constexpr (PW) {
#pragma unroll
              for (int rb = 0; rb < 2; ++rb) sc[rb] = f32x16{};
            } else {
              // dP accumulators start from -Dl of their rows: the products
              // then leave dP - Dl, the factor of dS
              const float* ndl = reinterpret_cast<const float*>(st + X::kSDL);
#pragma unroll
              for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int c4 = 0; c4 < 4; ++c4) {
                  const f32x4 d4 = *reinterpret_cast<const f32x4*>(ndl + rb * 32 + c4 * 8 + hh * 4);
#pragma unroll
                  for (int e = 0; e < 4; ++e) sc[rb][4 * c4 + e] = d4[e];
                }
            }
            lds_pipeline<DOCS ? kRowAhead - 2 : kRowAhead, 2 * KK>(   // (documents: registers)
                [&](int t) {
                  return *reinterpret_cast<const u32x4*>(as + rm_off<X::kRowBytes>((t % 2) * 32 + l32, t + hh - t % 2));
                },
                [] {},
                [&](int t, const u32x4 a) { sc[t % 2] = mfma32x32x16(a, kv[t / 2], sc[t % 2]); });
            if constexpr (PW) {
              const float* lses = reinterpret_cast<const float*>(st + X::kSLSE);
              const int32_t* los = reinterpret_cast<const int32_t*>(st + X::kSLO);
#pragma unroll
              for (int rb = 0; rb < 2; ++rb) {
                float pr[16];
                dkdv_probs<CAUSAL, DIAG, LOWER>(lses, los, sc[rb], rb, t0, u, hh, p.c, pr);
                // P to the dS wave: float4 c of block rb at xp[(rb*4 + c)*64 + lane]
#pragma unroll
                for (int c4 = 0; c4 < 4; ++c4)
                  *reinterpret_cast<f32x4*>(xp + ((rb * 4 + c4) * 64 + lane) * 4) =
                      f32x4{pr[4 * c4], pr[4 * c4 + 1], pr[4 * c4 + 2], pr[4 * c4 + 3]};
#pragma unroll
                for (int f = 0; f < 2; ++f) {
                  bh[rb][f] = pack8(pr + 8 * f);
                  if (SPLIT) bl[rb][f] = pack8_residual(pr + 8 * f, bh[rb][f]);
                }
              }
            }
          }
          __syncthreads();               // P is in LDS
          if (wave_live) {
            if constexpr (PW) {
              tr_products(dos, std::integral_constant<int, 0>{}, std::integral_constant<int, 2>{});   // dV^T += dO^T P
            } else {
              // each block's dS = P (dP - Dl) just before its products dK^T += Q^T dS
              auto block = [&](auto rb_tag) __attribute__((always_inline)) {
                constexpr int rb = decltype(rb_tag)::value;
                float ds[16];
#pragma unroll
                for (int c4 = 0; c4 < 4; ++c4) {
                  const f32x4 p4 = *reinterpret_cast<const f32x4*>(xp + ((rb * 4 + c4) * 64 + lane) * 4);
#pragma unroll
                  for (int e = 0; e < 4; ++e) ds[4 * c4 + e] = p4[e] * sc[rb][4 * c4 + e];
                }
#pragma unroll
                for (int f = 0; f < 2; ++f) {
                  bh[rb][f] = pack8(ds + 8 * f);
                  if (SPLIT) bl[rb][f] = pack8_residual(ds + 8 * f, bh[rb][f]);
                }
                __builtin_amdgcn_sched_barrier(0);
                tr_products(qs, rb_tag, std::integral_constant<int, 1>{});
              };
              // the dS wave's products lead the unit's critical chain here (the
              // P wave's dV has slack until the end barrier): its issue goes
              // first on the SIMD
              __builtin_amdgcn_s_setprio(1);
              block(std::integral_constant<int, 0>{});
              block(std::integral_constant<int, 1>{});
              __builtin_amdgcn_s_setprio(0);
            }
          }
          wait_vmem();
          __syncthreads();               // the stage and the P slot are free again
          tile = ntile;
          if (++nhead == p.g) {          // unit it+2 starts the next tile
            nhead = 0;
            ntile += tstep;
          }
        }
      };
      const int nsplit_u = max(0, min((split_end + X::kRows - 1) / X::kRows, tend) - tfirst) * p.g;
      const int ndiag = CAUSAL ? min(kKeys / X::kRows, tend - tfirst) * p.g : 0;
      auto sweep = [&](auto lower_tag) __attribute__((always_inline)) {
        using T = std::true_type;
        using F = std::false_type;
        const int n1 = min(nsplit_u, ndiag), n2 = max(nsplit_u, ndiag);
        auto seg = [&](int a, int z, auto split_tag, auto diag_tag) __attribute__((always_inline)) {
          const int x0 = max(down ? niter - z : a, u0);
          const int x1 = min(down ? niter - a : z, u1);
          if (x0 >= x1) return;
          run(x0, x1, split_tag, diag_tag, lower_tag);
        };
        if (down) {
          seg(n2, niter, F{}, F{});
          if (nsplit_u > ndiag) seg(n1, n2, T{}, F{});
          else seg(n1, n2, F{}, T{});
          seg(0, n1, T{}, T{});
        } else {
          seg(0, n1, T{}, T{});
          if (nsplit_u > ndiag) seg(n1, n2, T{}, F{});
          else seg(n1, n2, F{}, T{});
          seg(n2, niter, F{}, F{});
        }
      };
      if constexpr (DOCS) {
        if (lower) sweep(std::true_type{});
        else sweep(std::false_type{});
      } else {
        (void)lower;
        sweep(std::false_type{});
      }

      // dV (P wave) or dK = scale * dK^T^T (dS wave); lane = key u, dims
      // 32j + 8*(i/4) + 4hh + i%4; a padding key's gradients are zero
      float* out = PW ? p.dv : p.dk;
      if (p.nsplit > 1) out = (PW ? p.dv_part : p.dk_part) + sp * (int64_t(p.B) * p.n * p.Hkv * D);
      const int le = opaque_lane_id();   // (not hoisted out of the phase loop)
      const int ue = k0w + (le & 31);
      if (ue < p.n) {
        const int64_t base = ((int64_t(b) * p.n + ue) * p.Hkv + kvh) * D;
#pragma unroll
        for (int j = 0; j < DJ; ++j)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int d0 = j * 32 + i4 * 8 + (le >> 5) * 4;
            f32x4 o4;
            if constexpr (PW)
              o4 = f32x4{acc[j][i4 * 4], acc[j][i4 * 4 + 1], acc[j][i4 * 4 + 2], acc[j][i4 * 4 + 3]};
            else
              o4 = f32x4{acc[j][i4 * 4] * p.scale, acc[j][i4 * 4 + 1] * p.scale, acc[j][i4 * 4 + 2] * p.scale,
                         acc[j][i4 * 4 + 3] * p.scale};
            if (!key_ok) o4 = f32x4{0.f, 0.f, 0.f, 0.f};
            *reinterpret_cast<f32x4*>(out + base + d0) = o4;
          }
      }
    }
  };
  if (wave < 4) go(std::true_type{});
  else go(std::false_type{});
}

// --------------------------------------------------------------------- dq
template <int D>
struct DqLayout {
  static constexpr int kBN = 64;                          // keys per tile
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kChunks = D / 8;
  static constexpr int kBytesRM = kBN * kRowBytes;
  static constexpr int kOffK = 0;
  static constexpr int kOffV = kOffK + kBytesRM;
  static constexpr int kOffValid = kOffV + kBytesRM;
  static constexpr int kStage = kOffValid + kBN * 4;     // per-key score bias: 0 (valid) or -inf
  static constexpr int kStageAligned = (kStage + 127) / 128 * 128;
};

template <int D, bool HAS_MASK, int NW>
__device__ __forceinline__ void dq_issue(uint8_t* stage, uint32_t& vbyte, const BwdParams& p, int b, int kvh,
                                         int tile, int wave, int lane, int tid) {
  // (wave, tid: indices among the NW waves that stage this tile)
  using L = DqLayout<D>;
  const int key0 = tile * L::kBN;
  const int rows_ok = min(L::kBN, p.n - key0);
  const int64_t off = ((int64_t(b) * p.n + key0) * p.Hkv + kvh) * D;
  const int stride = p.Hkv * D * 2;
  dma_tile<D, L::kBN, NW>(stage + L::kOffK, p.k + off, stride, rows_ok, wave, lane);
  dma_tile<D, L::kBN, NW>(stage + L::kOffV, p.v + off, stride, rows_ok, wave, lane);
  // the key-valid byte as loaded (keys past n read key n-1's: the tail
  // compare masks them); nothing is computed on it before the tile's end, so
  // the wave does not wait here for this load and the tile's DMA with it
  if (HAS_MASK && tid < L::kBN) vbyte = p.valid[int64_t(b) * p.n + min(key0 + tid, p.n - 1)];
}

// One 32-key half of a staged K/V tile against this wave's 32 query rows:
// S^T and dP^T, dS^T, then dQ^T += K^T dS^T.  With MASKED, key row C of the
// half is visible iff C <= lim, and with documents iff also C >= lo;
// without it every key is (the tile lies wholly below the diagonal and
// inside n).  With HAS_MASK the score accumulators start from the keys'
// bias staged at vb (0, or -inf for a padding key), so the product applies
// the key mask itself.  SPLIT adds the bf16 residual of dS as second MFMAs.
template <int D, bool HAS_MASK, bool SPLIT, bool DOCS, bool MASKED, bool DLPASS>
__device__ __forceinline__ void dq_half(const uint8_t* ks, const uint8_t* vs, const uint8_t* vb, int half, int lim,
                                        int lo, const u32x4 (&qf)[D / 16], const u32x4 (&df)[D / 16], float lse2,
                                        float dl, float c, int l32, int hh, int lane, f32x16 (&dqa)[D / 32],
                                        float& dlacc) {
  using L = DqLayout<D>;
  constexpr int KK = D / 16;
  constexpr int DJ = D / 32;
  // S^T[key][q] and dP^T[key][q]: lane = query row, rows key = (i/4)*8 + 4hh + i%4
  f32x16 s = f32x16{}, dp = f32x16{};
  if (HAS_MASK) {
    const float* bias = reinterpret_cast<const float*>(vb) + half * 32 + hh * 4;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x4 b4 = *reinterpret_cast<const f32x4*>(bias + g4 * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) s[g4 * 4 + e] = b4[e];
    }
  }
  // (matrix blocks at raised wave priority, as in the forward)
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const int off = rm_off<L::kRowBytes>(half * 32 + l32, 2 * kk + hh);
    s = mfma32x32x16(*reinterpret_cast<const u32x4*>(ks + off), qf[kk], s);
    dp = mfma32x32x16(*reinterpret_cast<const u32x4*>(vs + off), df[kk], dp);
  }
  pipeline_reads_mfma<6, 2 * KK>();   // three k-steps of K/V rows in flight
  __builtin_amdgcn_s_setprio(0);
  if constexpr (DLPASS) {
    // Dl = sum over the visible keys of P dP, in float32 from the scores
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = g4 * 4 + e;
        const int ci = g4 * 8 + e;
        const bool ok = !MASKED || (ci <= lim && (!DOCS || ci >= lo));
        const float x = ok ? fmaf(s[i], c, -lse2) : -INFINITY;
        dlacc = fmaf(__builtin_amdgcn_exp2f(x), dp[i], dlacc);
      }
    }
    return;
  }
  float ds[16];
  // element i is key row C_i = (i/4)*8 + i%4 of the half (plus 4hh)
#pragma unroll
  for (int g4 = 0; g4 < 4; ++g4) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = g4 * 4 + e;
      const int ci = g4 * 8 + e;
      const bool ok = !MASKED || (ci <= lim && (!DOCS || ci >= lo));
      // invisible keys (and rows with no visible key: lse2 = +inf) get exponent -inf
      const float x = ok ? fmaf(s[i], c, -lse2) : -INFINITY;
      ds[i] = __builtin_amdgcn_exp2f(x) * (dp[i] - dl);
    }
  }
  u32x4 dh[2], dlo[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    dh[f] = pack8(ds + 8 * f);
    if (SPLIT) dlo[f] = pack8_residual(ds + 8 * f, dh[f]);
  }
  // dQ^T += K^T dS^T  (K^T read transposed from the row-major K tile)
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int f = 0; f < 2; ++f) {
#pragma unroll
    for (int j = 0; j < DJ; ++j) {
      const u32x4 a = tr_operand<L::kRowBytes>(ks, half * 32 + 16 * f, 32 * j, lane);
      dqa[j] = mfma32x32x16(a, dh[f], dqa[j]);
      if (SPLIT) dqa[j] = mfma32x32x16(a, dlo[f], dqa[j]);
    }
  }
  if (!SPLIT) pipeline_tr_reads_mfma<3, 2 * DJ>();
  __builtin_amdgcn_s_setprio(0);
}

// KS (key split, 8 waves, plain causal): two groups of 4 waves take the same
// rows, the first group the first half of their key tiles (rounded up) and
// the second the rest, each with its own staging buffers; at the end the
// second group hands its dQ^T accumulators to the first through LDS, which
// adds them and writes dQ.  On short grids, where every workgroup is
// resident at once and the longest block (the last rows, which see every
// key) sets the kernel's time, each block then lasts about half as long.
// Blocks whose rows see fewer than kSplitRows keys (the hi/lo split and the
// exact-Dl sweep) stay whole in the first group: they are short anyway.
// WIDE (8 waves, long plain causal grids): one group of 8 waves whose rows
// (64 positions of the KV head's query heads) share every staged K/V tile,
// half the staging per flop of two 4-wave workgroups, as in the forward.
template <int D, bool HAS_MASK, bool CAUSAL, bool DOCS, bool KS = false, bool WIDE = false>
__global__ __launch_bounds__((KS || WIDE) ? 2 * kThreads : kThreads, (KS || WIDE) ? 1 : 2) void dq_kernel(
    const BwdParams p) {
  static_assert(CAUSAL || !DOCS, "documents are causal");
  static_assert(!KS || (CAUSAL && !DOCS), "the key split is for plain causal attention");
  static_assert(!(KS && WIDE), "one 8-wave form at a time");
  constexpr int GW = WIDE ? 2 * kWaves : kWaves;  // waves that share one staged tile
  using L = DqLayout<D>;
  constexpr int KK = D / 16;
  constexpr int DJ = D / 32;
  constexpr int NG = KS ? 2 : 1;                  // wave groups
  __shared__ __attribute__((aligned(128))) uint8_t smem[NG * 2 * L::kStageAligned];

  // wave index as a scalar: every branch that guards a matrix-core instruction
  // must be wave-uniform to the compiler (MFMA does not honour EXEC)
  const int wave_all = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
  const int grp = KS ? wave_all / kWaves : 0;      // wave group
  const int wave = wave_all - grp * kWaves;       // wave within its group (all 8 with WIDE)
  const int tid = int(threadIdx.x) - grp * kThreads;
  uint8_t* const gsmem = smem + grp * 2 * L::kStageAligned;   // the group's staging buffers
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const int per_pos = p.n_hsub * p.Hkv * p.B;
  const int pb = p.n_pblocks - 1 - int(blockIdx.x) / per_pos;
  int rem = int(blockIdx.x) % per_pos;
  const int b = rem / (p.n_hsub * p.Hkv);
  rem = rem % (p.n_hsub * p.Hkv);
  const int kvh = rem / p.n_hsub;
  const int hs = rem % p.n_hsub;
  const int head = kvh * p.g + hs * p.gh + (wave % p.gh);
  const int p0 = pb * p.pw + (wave / p.gh) * 32;
  const int t = p0 + l32;
  const int wave_last = min(p0 + 31, p.n - 1);
  const int wg_last = min(pb * p.pw + p.pw, p.n) - 1;
  const int kend = CAUSAL ? wg_last + 1 : p.n;
  const int ntiles = (kend + L::kBN - 1) / L::kBN;
  const bool wave_live = p0 < p.n;

  // packed documents: first tile, the last row's bound (tiles below it take
  // the lower mask), the wave's first row's bound (tiles below it are
  // skipped) and this lane's row's bound
  int it_first = 0, lo_last = 0, lo_wave = 0, lo_row = 0;
  if (DOCS) {
    const int32_t* rs = p.doc_start + int64_t(b) * p.n;
    it_first = doc_lower(rs, pb * p.pw) / L::kBN;
    lo_last = doc_lower(rs, wg_last);
    lo_wave = wave_live ? doc_lower(rs, p0) : 0;
    lo_row = t < p.n ? doc_lower(rs, t) : 0;
  }

  u32x4 qf[KK], df[KK];
  float lse2 = INFINITY, dl = 0.f;
  {
    const bool ok = t < p.n;
    const int64_t off = ((int64_t(b) * p.n + (ok ? t : 0)) * p.Hq + head) * D + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      qf[kk] = ok ? *reinterpret_cast<const u32x4*>(p.q + off + 16 * kk) : u32x4{0, 0, 0, 0};
      df[kk] = ok ? *reinterpret_cast<const u32x4*>(p.dout + off + 16 * kk) : u32x4{0, 0, 0, 0};
    }
    // Dl = dO . O of the lane's row: this half-wave's dims 16kk + 8hh .. +7,
    // then the other half's; with the base-2 logsumexp (+inf for a row with
    // no visible key, so that every exponent is -inf) it goes to the
    // workspace for the dK/dV pass, which runs after this kernel
    float part = 0.f;
    if (ok) {
      if (p.o_f32) {
        const float* op = static_cast<const float*>(p.o) + off;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const f32x4 o0 = *reinterpret_cast<const f32x4*>(op + 16 * kk);
          const f32x4 o1 = *reinterpret_cast<const f32x4*>(op + 16 * kk + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float olo = e < 2 ? o0[2 * e] : o1[2 * e - 4];
            const float ohi = e < 2 ? o0[2 * e + 1] : o1[2 * e - 3];
            part = fmaf(bf16lo_to_f32(df[kk][e]), olo, part);
            part = fmaf(bf16hi_to_f32(df[kk][e]), ohi, part);
          }
        }
      } else {
        const uint16_t* op = static_cast<const uint16_t*>(p.o) + off;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const u32x4 ov = *reinterpret_cast<const u32x4*>(op + 16 * kk);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            part = fmaf(bf16lo_to_f32(df[kk][e]), bf16lo_to_f32(ov[e]), part);
            part = fmaf(bf16hi_to_f32(df[kk][e]), bf16hi_to_f32(ov[e]), part);
          }
        }
      }
      const float l = p.lse[(int64_t(b) * p.Hq + head) * p.n + t];
      lse2 = (l == -INFINITY) ? INFINITY : l * kLog2e;
    }
    dl = halves_sum(part);
    if (ok && hh == 0 && grp == 0) {
      const int64_t idx = (int64_t(b) * p.Hq + head) * p.n + t;
      p.rowdot[idx] = -dl;   // stored negated: the dK/dV pass starts its dP accumulators from it
      p.lse2[idx] = lse2;
    }
  }

  // Rows with fewer than kSplitRows visible keys take the hi/lo path; the
  // choice is made once per workgroup so the common path carries no
  // residuals.  Every row sees at least (first row) - (last row's bound)
  // keys.  Those rows also get their Dl recomputed from the scores, in a
  // first sweep over the same tiles: Dl = sum_u P dP = dO . (sum_u P v_u) is
  // dO . O with O exact, where the O handed in may carry bf16 storage
  // rounding, which on rows with few keys (|O| near the size of a V row)
  // moves dQ and dK by up to ~1e-2.  The value is written back to the
  // workspace for the dK/dV pass, which runs after this kernel.
  auto run = [&](auto split_tag) {
    constexpr bool SPLIT = decltype(split_tag)::value;
    f32x16 dqa[DJ];
#pragma unroll
    for (int j = 0; j < DJ; ++j) dqa[j] = f32x16{};

    // Tiles that need the index masks: the causal diagonal (tiles reaching
    // past the workgroup's first row) and the tail past n, the last ones.
    // The steps split into a run without and a run with them, decided
    // outside the loop.  With documents every tile takes the masks (measured:
    // the split gained nothing there).
    const int nsteps_all = ntiles - it_first;
    const int first_row = pb * p.pw;
    int mask_from = CAUSAL ? max(first_row - L::kBN + 1, 0) : p.n - L::kBN + 1;   // first key0 of a masked tile
    mask_from = min(mask_from, p.n - L::kBN + 1);
    // tiles it_first .. ntiles-1 from mask_tile on take the masks
    const int mask_tile = (mask_from + L::kBN - 1) / L::kBN;
    // this group's tiles g_first .. g_first+g_steps-1; both groups run
    // `nsteps` loop steps (the same barriers), the second group one fewer
    // real step when the count is odd, or none on the split workgroups
    int g_first = it_first, g_steps = nsteps_all, nsteps = nsteps_all;
    if (KS) {
      const int h = SPLIT ? nsteps_all : (nsteps_all + 1) / 2;
      g_first = it_first + (grp == 1 ? h : 0);
      g_steps = grp == 0 ? h : nsteps_all - h;
      nsteps = h;
    }
    const int j_hi = DOCS ? 0 : min(max(mask_tile - g_first, 0), nsteps);   // steps >= j_hi masked

    // one sweep over the tiles: the dQ products, or (DLPASS) only the row sums of P dP
    auto sweep = [&](auto dlpass_tag) __attribute__((always_inline)) {
      constexpr bool DLPASS = decltype(dlpass_tag)::value;
      float dlacc = 0.f;
      // step j works on tile it_first + j, staged in buffer j & 1 (the LDS
      // addresses depend on the step counter only)
      uint32_t vbyte = 0;
      if (g_steps > 0) {
        dq_issue<D, HAS_MASK, GW>(gsmem, vbyte, p, b, kvh, g_first, wave, lane, tid);
        if (HAS_MASK && tid < L::kBN) reinterpret_cast<float*>(gsmem + L::kOffValid)[tid] = vbyte ? 0.f : -INFINITY;
      }
      wait_vmem();
      __syncthreads();
      auto steps = [&](int j0, int j1, auto masked_tag) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        for (int j = j0; j < j1; ++j) {
          const int it = g_first + j;
          // prefetch tile it+1 into the other buffer while computing on this one
          uint8_t* cur = gsmem + (j & 1) * L::kStageAligned;
          uint8_t* nxt = gsmem + ((j + 1) & 1) * L::kStageAligned;
          if (j + 1 < g_steps) {
            if constexpr (WIDE) {
              // waves 4-7 alone stage the tiles after the first: the SIMD issues
              // waves 0-3 first, and they go straight to their products
              if (wave >= kWaves)
                dq_issue<D, HAS_MASK, kWaves>(nxt, vbyte, p, b, kvh, it + 1, wave - kWaves, lane, tid - kThreads);
            } else {
              dq_issue<D, HAS_MASK, GW>(nxt, vbyte, p, b, kvh, it + 1, wave, lane, tid);
            }
          }
          const int tile0 = it * L::kBN;
          if ((!KS || j < g_steps) && wave_live && !(CAUSAL && tile0 > wave_last) &&
              !(DOCS && tile0 + L::kBN <= lo_wave)) {
            const uint8_t* ks = cur + L::kOffK;
            const uint8_t* vs = cur + L::kOffV;
            const uint8_t* vb = cur + L::kOffValid;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
              const int key0 = tile0 + half * 32;
              if (CAUSAL && key0 > wave_last) break;
              // visible iff key < n, and key <= t if causal
              int lim = p.n - 1 - key0 - 4 * hh;
              if (CAUSAL) lim = min(lim, t - key0 - 4 * hh);
              // documents: key >= the row's bound (no-op above the last row's bound)
              const int lo = (DOCS && tile0 < lo_last) ? lo_row - key0 - 4 * hh : -0x7fffffff;
              dq_half<D, HAS_MASK, SPLIT, DOCS, MASKED, DLPASS>(ks, vs, vb, half, lim, lo, qf, df, lse2, dl, p.c, l32,
                                                                hh, lane, dqa, dlacc);
            }
          }
          if constexpr (WIDE) {
            if (HAS_MASK && j + 1 < g_steps && wave >= kWaves && tid - kThreads < L::kBN)
              reinterpret_cast<float*>(nxt + L::kOffValid)[tid - kThreads] = vbyte ? 0.f : -INFINITY;
          } else if (HAS_MASK && j + 1 < g_steps && tid < L::kBN) {
            reinterpret_cast<float*>(nxt + L::kOffValid)[tid] = vbyte ? 0.f : -INFINITY;
          }
          wait_vmem();
          __syncthreads();
        }
      };
      if (!DOCS) steps(0, j_hi, std::false_type{});
      steps(j_hi, nsteps, std::true_type{});
      return dlacc;
    };

    if constexpr (SPLIT) {
      // the two half-waves hold complementary keys of the same row (with the
      // key split, the first group holds all of them)
      dl = halves_sum(sweep(std::true_type{}));
      if (t < p.n && hh == 0 && grp == 0) p.rowdot[(int64_t(b) * p.Hq + head) * p.n + t] = -dl;
    }
    sweep(std::false_type{});

    if constexpr (KS) {
      // the second group's dQ^T to the first, through the second group's
      // staging buffers (free: both groups are past their last barrier):
      // float4 (j, i4) of wave w at xch[((w * DJ + j) * 4 + i4) * 64 + lane]
      f32x4* xch = reinterpret_cast<f32x4*>(smem + 2 * L::kStageAligned);
      if (grp == 1)
#pragma unroll
        for (int j = 0; j < DJ; ++j)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4)
            xch[((wave * DJ + j) * 4 + i4) * 64 + lane] =
                f32x4{dqa[j][i4 * 4], dqa[j][i4 * 4 + 1], dqa[j][i4 * 4 + 2], dqa[j][i4 * 4 + 3]};
      __syncthreads();
      if (grp == 1) return;
#pragma unroll
      for (int j = 0; j < DJ; ++j)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const f32x4 x = xch[((wave * DJ + j) * 4 + i4) * 64 + lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) dqa[j][i4 * 4 + e] += x[e];
        }
    }

    if (t < p.n) {
      const int64_t base = ((int64_t(b) * p.n + t) * p.Hq + head) * D;
#pragma unroll
      for (int j = 0; j < DJ; ++j)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d0 = j * 32 + i4 * 8 + hh * 4;
          *reinterpret_cast<f32x4*>(p.dq + base + d0) =
              f32x4{dqa[j][i4 * 4] * p.scale, dqa[j][i4 * 4 + 1] * p.scale, dqa[j][i4 * 4 + 2] * p.scale,
                    dqa[j][i4 * 4 + 3] * p.scale};
        }
    }
  };
  // non-causal rows see all n positions
  const bool few_keys = CAUSAL ? (pb * p.pw - lo_last < kSplitRows) : (p.n < kSplitRows);
  if (few_keys) run(std::true_type{});
  else run(std::false_type{});
}

// dq grid shape for NW waves per workgroup: query heads per workgroup (the
// largest divisor of g that divides NW) and positions per workgroup
void dq_shape(BwdParams& p, int nw) {
  int gh = 1;
  for (int c = nw; c >= 1; --c)
    if (p.g % c == 0 && nw % c == 0) { gh = c; break; }
  p.gh = gh;
  p.pw = 32 * (nw / gh);
  p.n_pblocks = int32_t((int64_t(p.n) + p.pw - 1) / p.pw);
  p.n_hsub = p.g / gh;
}

template <int D, bool HAS_MASK, bool CAUSAL, bool DOCS>
hipError_t launch_grads(const BwdParams& p, int64_t kv_blocks, int64_t q_blocks, hipStream_t stream) {
  // dq first: it rewrites Dl of the rows with few visible keys, which dkdv reads
  // short plain causal grids (every 4-wave block resident at once, two per
  // CU) take the key split: one 8-wave workgroup per block
  // long ones take the 8-wave form whose waves share each K/V tile
  if constexpr (CAUSAL && !DOCS) {
    BwdParams p8 = p;
    dq_shape(p8, 2 * kWaves);
    const int64_t q_blocks8 = int64_t(p8.n_pblocks) * p8.n_hsub * p8.Hkv * p8.B;
    if (q_blocks <= kDqSplitBlocks)
      hipLaunchKernelGGL((dq_kernel<D, HAS_MASK, true, false, true>), dim3(q_blocks), dim3(2 * kThreads), 0, stream, p);
    else if (q_blocks8 >= kDqWideBlocks)
      hipLaunchKernelGGL((dq_kernel<D, HAS_MASK, true, false, false, true>), dim3(q_blocks8), dim3(2 * kThreads), 0,
                         stream, p8);
    else
      hipLaunchKernelGGL((dq_kernel<D, HAS_MASK, true, false>), dim3(q_blocks), dim3(kThreads), 0, stream, p);
  } else {
    hipLaunchKernelGGL((dq_kernel<D, HAS_MASK, CAUSAL, DOCS>), dim3(q_blocks), dim3(kThreads), 0, stream, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((dkdv_pair_kernel<D, HAS_MASK, CAUSAL, DOCS>), dim3(kv_blocks), dim3(kPairThreads), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess || p.nsplit == 1) return e;
  const int64_t count = int64_t(p.B) * p.n * p.Hkv * D;   // a multiple of 4 (D is)
  const int64_t rblocks = (count / 4 + 255) / 256;
  if (2 * rblocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(dkdv_reduce_kernel, dim3(2 * rblocks), dim3(256), 0, stream, p.dk_part, p.dk, p.dv_part, p.dv,
                     count, p.nsplit, int32_t(rblocks));
  return hipGetLastError();
}

template <int D, bool HAS_MASK>
hipError_t dispatch_grads(const BwdParams& p, int64_t kv_blocks, int64_t q_blocks, hipStream_t stream) {
  if (p.doc_start != nullptr) return launch_grads<D, HAS_MASK, true, true>(p, kv_blocks, q_blocks, stream);
  if (p.causal) return launch_grads<D, HAS_MASK, true, false>(p, kv_blocks, q_blocks, stream);
  return launch_grads<D, HAS_MASK, false, false>(p, kv_blocks, q_blocks, stream);
}

template <int D>
hipError_t launch_bwd_d(const BwdParams& p, bool has_mask, hipStream_t stream) {
  // causal: one workgroup per pair of key blocks (nkb-1-w, w); documents:
  // one per key block
  const int64_t kv_work = (p.causal && p.doc_start == nullptr) ? (int64_t(p.n_kblocks) + 1) / 2 : p.n_kblocks;
  const int64_t kv_blocks = kv_work * p.Hkv * p.B * p.nsplit;
  const int64_t q_blocks = int64_t(p.n_pblocks) * p.n_hsub * p.Hkv * p.B;
  if (kv_blocks > 0x7fffffff || q_blocks > 0x7fffffff) return hipErrorInvalidValue;
  return has_mask ? dispatch_grads<D, true>(p, kv_blocks, q_blocks, stream)
                  : dispatch_grads<D, false>(p, kv_blocks, q_blocks, stream);
}

}  // namespace

hipError_t launch_attn_bwd_bf16(const void* q, const void* k, const void* v, const uint8_t* valid,
                                const int32_t* doc_start, const void* o, const float* lse, const void* dout,
                                float* dq, float* dk, float* dv, float* workspace, const AttnShape& s, int o_f32,
                                int nsplit, hipStream_t stream) {
  BwdParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.valid = valid;
  p.doc_start = doc_start;
  p.o = o;
  p.lse = lse;
  p.dout = static_cast<const uint16_t*>(dout);
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.nsplit = nsplit < 1 ? 1 : nsplit;
  p.lsplit = 0;
  while ((1 << p.lsplit) < p.nsplit) ++p.lsplit;
  const BwdWorkspace ws = attn_bwd_workspace(s.B, s.n, s.Hq, s.Hkv, s.D, p.nsplit);
  p.rowdot = workspace + ws.rowdot;
  p.lse2 = workspace + ws.lse2;
  p.dk_part = workspace + ws.dk_part;
  p.dv_part = workspace + ws.dv_part;
  p.B = s.B;
  p.n = int32_t(s.n);
  p.Hq = s.Hq;
  p.Hkv = s.Hkv;
  p.g = s.Hq / s.Hkv;
  p.scale = s.scale;
  p.c = s.scale * kLog2e;
  p.causal = s.causal;
  p.o_f32 = o_f32 != 0;
  dq_shape(p, kWaves);
  p.n_kblocks = int32_t((s.n + 127) / 128);
  if (int64_t(p.B) * p.n == 0) return hipSuccess;
  if (s.D == 128) return launch_bwd_d<128>(p, valid != nullptr, stream);
  return launch_bwd_d<64>(p, valid != nullptr, stream);
}

}  // namespace ulysses
