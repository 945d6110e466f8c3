// attn_fwd.hip -- exact causal grouped-query softmax attention, forward with
// logsumexp, bf16 inputs on gfx950 matrix cores.
//
// Operation: [ALST] "Paralelismul de Secvență Ulysses: Antrenarea modelelor
// AI cu contexte de un milion de token-uri", section "Mecanismul de
// funcționare Ulysses", step 4 (local attention over all positions for the
// heads this rank holds); the tiled, never-materialised score matrix follows
// the same page's section "Provocarea antrenării cu secvențe lungi".
//
// Design (gfx950, wave64):
//  * A workgroup of 4 waves owns one KV head and a block of query rows; every
//    32-row group is (32 consecutive positions, one query head).  With a GQA
//    group of g >= 4 query heads per KV head the 4 waves take the same 32
//    positions of 4 different query heads, so each K/V tile staged in LDS
//    feeds 128 query rows with identical causal extents.
//  * Scores are computed transposed, S^T = K Q^T (32 keys x 32 queries per
//    32x32x16 bf16 MFMA), so each lane owns one query row: row max, row sum
//    and the rescale of O stay in-lane (one half-wave exchange for the
//    max).  O is accumulated transposed too, O^T += V^T P^T, with P^T used
//    straight from the score registers as the B operand.
//  * K and V tiles are stored row-major in LDS with XOR-swizzled 16-byte
//    chunks.  K rows feed S^T = K Q^T directly; the V^T operand of the PV
//    product is read with the gfx950 transposing LDS read (ds_read_b64_tr_b16),
//    in the key order of the score registers, so nothing is transposed in
//    registers and both read patterns are free of bank conflicts.
//  * Tile i+1 is copied global->LDS by buffer-load DMA (no registers, keys
//    past n read as zero) while the MFMA work runs on tile i (double-buffered
//    LDS, one barrier per tile).
//  * The loop body has no branch between matrix instructions: the hi/lo split
//    is chosen per workgroup outside the loop, and on a causal diagonal tile
//    both 32-key halves are computed (a half with no visible key adds zeros).
//  * Online softmax in base 2: the row max is taken on raw scores and each
//    probability is one FMA (score * scale*log2(e) - max) and one v_exp_f32.
//    The running max is only raised when a tile's max exceeds it by more than
//    8 (log2 units): O and the row sum then carry factors up to 2^8, harmless
//    in fp32, and the rescale of O is skipped on almost every tile.
//  * Rows below kSplitRows use a hi/lo split of P (two bf16 MFMAs) to keep
//    the error of the few-key rows, whose weights are large, far below 1e-2.
//  * The grid is launched longest-first (last query blocks first) so the
//    causal triangle's long blocks do not trail at the end.
//  * Packed documents (a per-row lower bound on the visible keys, the first
//    position of the row's document): the workgroup starts at the tile that
//    holds its first row's bound, so whole tiles of earlier documents are
//    never loaded, and only tiles below its last row's bound take the
//    per-row lower mask.
//  * Key blocks (ring attention's hops): the keys may be a separate block of
//    nk positions whose causal relation to the rows is an offset delta (key
//    u of the block is visible to row t iff u <= t + delta); the epilogue can
//    merge this block's (O, LSE) into a running float32 result already in
//    the output, by the exact logsumexp combination for disjoint key sets.
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace ulysses {

namespace {

constexpr int kBN = 64;                 // keys per tile
constexpr int kSplitRows = 512;         // rows using the hi/lo split of P
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;   // log2 units
constexpr int kWide8Blocks = 512;       // 8-wave workgroups from this grid size on (plain causal, D = 128)
constexpr int kWide8OtherBlocks = 2048; // the same with documents or without the causal mask

template <int D>
struct FwdLayout {
  static constexpr int kRowBytes = 2 * D;                // one K or V row (bf16) in LDS
  static constexpr int kChunks = D / 8;                  // 16-byte chunks per row
  static constexpr int kBytesK = kBN * kRowBytes;
  static constexpr int kBytesV = kBN * kRowBytes;
  static constexpr int kBytesValid = kBN * 4;            // per-key score bias: 0 (valid) or -inf
  static constexpr int kStage = kBytesK + kBytesV + kBytesValid;
  static constexpr int kStageAligned = (kStage + 127) / 128 * 128;
};

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint8_t* valid;
  const int32_t* doc_start;   // [B][n] first position of each row's document, or null
  void* o;
  float* lse;
  int32_t B, n, Hq, Hkv;
  int32_t nk;         // keys (n, or the length of a separate key block)
  int32_t delta;      // causal offset: key u visible to row t iff u <= t + delta (0 for one sequence)
  int32_t accumulate; // merge into the float32 (O, LSE) already in the output
  int32_t g;          // query heads per KV head
  int32_t gh;         // query heads per workgroup
  int32_t pw;         // positions per workgroup
  int32_t n_pblocks;  // ceil(n / pw)
  int32_t n_hsub;     // g / gh
  float c;            // softmax scale * log2(e)
  int32_t causal;
};

// DMA the K and V rows of 64-key tile `tile` into the swizzled row-major
// tiles of `stage` (keys past n read as zero), and load the tile's key-valid
// bytes into a register of the first 64 threads (keys past nk read key
// nk-1's byte: the tail compare masks them).  The caller turns them into the
// tile's score bias once the buffer is free; nothing is computed on the byte
// here, since a use would make the wave wait for this load, and with it for
// the whole tile's DMA, at the start of its tile.
template <int NW, int D, bool HAS_MASK>
__device__ __forceinline__ void fwd_issue(uint8_t* stage, uint32_t& vbyte, const FwdParams& p, int b, int kvh,
                                          int tile, int wave, int lane, int tid) {
  // (wave, tid: indices within the NW waves that stage this tile)
  using L = FwdLayout<D>;
  const int key0 = tile * kBN;
  const int rows_ok = min(kBN, p.nk - key0);
  const int64_t off = ((int64_t(b) * p.nk + key0) * p.Hkv + kvh) * D;
  const int stride = p.Hkv * D * 2;
  dma_tile<D, kBN, NW>(stage, p.k + off, stride, rows_ok, wave, lane);
  dma_tile<D, kBN, NW>(stage + L::kBytesK, p.v + off, stride, rows_ok, wave, lane);
  if (HAS_MASK && tid < kBN) vbyte = p.valid[int64_t(b) * p.nk + min(key0 + tid, p.nk - 1)];
}

// KS (key split, 8 waves): two groups of 4 waves take the same rows, the
// first group the first half of their key tiles and the second the rest,
// each with its own staging buffers and online softmax; at the end the
// second group hands its (O, max, row sum) to the first through LDS, which
// merges them exactly (the same combination as for disjoint key blocks) and
// writes the output.  Every workgroup then lasts about half as long as its
// block's keys, which evens out the causal triangle on short grids, where
// all blocks are resident at once and the longest one sets the time.
template <int NW, int D, bool HAS_MASK, bool O_F32, bool CAUSAL, bool DOCS, bool KS>
__global__ __launch_bounds__(NW * 64, 8 / NW) void attn_fwd_bf16_kernel(const FwdParams p) {
  static_assert(CAUSAL || !DOCS, "documents are causal");
  static_assert(!KS || (NW == 8 && !DOCS), "the key split pairs two 4-wave groups");
  using L = FwdLayout<D>;
  constexpr int KK = D / 16;     // contraction slices of the score product
  constexpr int DJ = D / 32;     // 32-row blocks of O^T
  constexpr int NG = KS ? 2 : 1;         // wave groups
  constexpr int GW = NW / NG;            // waves per group
  __shared__ __attribute__((aligned(128))) uint8_t smem[NG * 2 * L::kStageAligned];

  const int tid_all = threadIdx.x;
  // wave index as a scalar: every branch that guards a matrix-core instruction
  // must be wave-uniform to the compiler (MFMA does not honour EXEC)
  const int wave_all = __builtin_amdgcn_readfirstlane(tid_all >> 6);
  const int grp = KS ? wave_all / GW : 0;
  const int wave = wave_all % GW;        // wave within its group
  const int tid = tid_all % (GW * 64);   // thread within its group
  uint8_t* const gsmem = smem + grp * 2 * L::kStageAligned;   // the group's two staging buffers
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // ---- block coordinates (longest-first over position blocks)
  const int per_pos = p.n_hsub * p.Hkv * p.B;
  const int L_id = blockIdx.x;
  const int pb = p.n_pblocks - 1 - L_id / per_pos;
  int rem = L_id % per_pos;
  const int b = rem / (p.n_hsub * p.Hkv);
  rem = rem % (p.n_hsub * p.Hkv);
  const int kvh = rem / p.n_hsub;
  const int hs = rem % p.n_hsub;

  const int head = kvh * p.g + hs * p.gh + (wave % p.gh);
  const int p0 = pb * p.pw + (wave / p.gh) * 32;      // first position of this wave's rows
  const int t = p0 + l32;                               // this lane's query row
  const int wave_last = min(p0 + 31, p.n - 1);
  const int wg_last = min(pb * p.pw + p.pw, p.n) - 1;
  const int kend = CAUSAL ? min(wg_last + 1 + p.delta, p.nk) : p.nk;
  const int ntiles = (kend + kBN - 1) / kBN;
  const bool wave_live = p0 < p.n;

  // ---- packed documents: first tile, and the bounds of the lower mask
  int it_first = 0;   // first tile holding a key any row of the workgroup sees
  int lo_last = 0;    // bound of the last row: tiles below it need the lower mask
  int lo_wave = 0;    // bound of the wave's first row: tiles below it are skipped
  int lo_row = 0;     // bound of this lane's row
  if (DOCS) {
    const int32_t* rs = p.doc_start + int64_t(b) * p.n;
    it_first = doc_lower(rs, pb * p.pw) / kBN;
    lo_last = doc_lower(rs, wg_last);
    lo_wave = wave_live ? doc_lower(rs, p0) : 0;
    lo_row = t < p.n ? doc_lower(rs, t) : 0;
  }

  // ---- Q fragment (B operand of S^T = K Q^T): lane holds row t, dims 16kk + 8hh .. +7
  u32x4 qf[KK];
  {
    const bool ok = t < p.n;
    const int64_t off = ((int64_t(b) * p.n + (ok ? t : 0)) * p.Hq + head) * D + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qf[kk] = ok ? *reinterpret_cast<const u32x4*>(p.q + off + 16 * kk) : u32x4{0, 0, 0, 0};
  }

  // Rows with fewer than kSplitRows visible keys take the hi/lo path; the
  // choice is made once per workgroup, outside the tile loop, so the loop
  // body has no branch between its matrix instructions.  Every row t of the
  // workgroup sees at least (first row) - (last row's bound) keys.
  auto run = [&](auto split_tag) {
    constexpr bool SPLIT = decltype(split_tag)::value;
    f32x16 oacc[DJ];
#pragma unroll
    for (int j = 0; j < DJ; ++j) oacc[j] = f32x16{};
    float m_ref = -INFINITY;   // running reference max (log2 units), identical in both half-waves
    float lsum = 0.f;          // this half-wave's share of the row sum

    // this group's tiles [it_beg, it_end), in nsteps steps of one barrier each
    // (with the key split the first group takes the first half, rounded up)
    const int nsteps = KS ? (max(ntiles - it_first, 0) + 1) / 2 : 0;
    const int it_beg = KS ? it_first + (grp == 1 ? nsteps : 0) : it_first;
    const int it_end = KS && grp == 0 ? it_first + nsteps : ntiles;

    // With 8 waves on one K/V tile, waves 4-7 alone stage the tiles after the
    // first.  The SIMD issues the older wave of its pair first: waves 0-3
    // end their tile's work about 700 cycles before waves 4-7 and wait at
    // the barrier.  Staging by waves 4-7 measured 2-3 % faster on long runs
    // than by all 8 waves or by waves 0-3.
    constexpr bool kUpperDma = NW == 8 && !KS;
    const bool dma_wave = !kUpperDma || wave >= 4;
    const int dwave = kUpperDma ? wave - 4 : wave;   // index among the staging waves
    const int dtid = kUpperDma ? tid - 256 : tid;

    uint32_t vbyte = 0;
    if (!KS || it_beg < it_end) fwd_issue<GW, D, HAS_MASK>(gsmem, vbyte, p, b, kvh, it_beg, wave, lane, tid);
    if (HAS_MASK && tid < kBN) reinterpret_cast<float*>(gsmem + L::kBytesK + L::kBytesV)[tid] = vbyte ? 0.f : -INFINITY;
    wait_vmem();
    __syncthreads();

    // one tile: prefetch tile it+1 into `nxt` while computing on `cur`.  The
    // loop below is unrolled by two so each copy names its buffers
    // statically and every LDS address folds the buffer into the
    // instruction's immediate offset.
    auto tile = [&](int it, uint8_t* cur, uint8_t* nxt) {
      if (it + 1 < it_end && dma_wave)
        fwd_issue<kUpperDma ? 4 : GW, D, HAS_MASK>(nxt, vbyte, p, b, kvh, it + 1, dwave, lane, dtid);

      const int tile0 = it * kBN;
      // (with the key split the second group may have one step fewer than the first)
      if ((!KS || it < it_end) && wave_live && !(CAUSAL && tile0 > wave_last + p.delta) &&
          !(DOCS && tile0 + kBN <= lo_wave)) {
        const uint8_t* ks = cur;
        const uint8_t* vs = cur + L::kBytesK;

        // ---- S^T for the two 32-key halves.  On a causal diagonal tile the
        // second half may hold no visible key; it is computed anyway (its
        // scores are masked to -inf below, so it adds exact zeros to O).
        // With padding the accumulators start from the keys' bias (0, or
        // -inf for a padding key): the product applies the key mask itself
        // (element i holds key 32*half + 8*(i/4) + 4hh + i%4).
        f32x16 s0 = f32x16{}, s1 = f32x16{};
        if (HAS_MASK) {
          const float* vb = reinterpret_cast<const float*>(cur + L::kBytesK + L::kBytesV);
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4 b0 = *reinterpret_cast<const f32x4*>(vb + g4 * 8 + hh * 4);
            const f32x4 b1 = *reinterpret_cast<const f32x4*>(vb + 32 + g4 * 8 + hh * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              s0[g4 * 4 + e] = b0[e];
              s1[g4 * 4 + e] = b1[e];
            }
          }
        }
        // (the matrix blocks issue at raised wave priority: of the SIMD's two
        // waves, the one with MFMAs to issue goes first and the other's
        // softmax fills the gaps; measured 3-5 % on the masked kernels)
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const u32x4 a0 = *reinterpret_cast<const u32x4*>(ks + rm_off<L::kRowBytes>(l32, 2 * kk + hh));
          const u32x4 a1 = *reinterpret_cast<const u32x4*>(ks + rm_off<L::kRowBytes>(32 + l32, 2 * kk + hh));
          s0 = mfma32x32x16(a0, qf[kk], s0);
          s1 = mfma32x32x16(a1, qf[kk], s1);
        }
        pipeline_reads_mfma<6, 2 * KK>();   // three k-steps of K rows in flight
        __builtin_amdgcn_s_setprio(0);

        // ---- raw scores and masks (masked keys -> -inf)
        float x[32];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          x[i] = s0[i];
          x[16 + i] = s1[i];
        }
        const bool diag = CAUSAL && (tile0 + kBN - 1 > p0 + p.delta);
        const bool tail = tile0 + kBN > p.nk;
        const bool lower = DOCS && tile0 < lo_last;
        if (diag || tail || lower) {
          // element i holds key tile0 + 4hh + C_i with C_i a compile-time constant;
          // it is visible iff lo <= C_i <= lim.  Causal: key <= t + delta; always
          // key < nk.  Documents: key >= the row's bound.
          const int lim = (CAUSAL ? min(t + p.delta, p.nk - 1) : p.nk - 1) - tile0 - 4 * hh;
          const int lo = DOCS ? lo_row - tile0 - 4 * hh : -0x7fffffff;
#pragma unroll
          for (int i = 0; i < 32; ++i) {
            const int ci = (i >> 4) * 32 + ((i & 15) >> 2) * 8 + (i & 3);
            x[i] = (ci > lim || ci < lo) ? -INFINITY : x[i];
          }
        }

        // ---- online softmax (lazy rescale); scale > 0, so max(s * c) = max(s) * c
        float mr = x[0];
#pragma unroll
        for (int i = 1; i < 32; ++i) mr = fmaxf(mr, x[i]);
        mr = halves_max(mr);
        const float mx = mr * p.c;
        const bool raise = mx > m_ref + kRescaleSlack;
        if (__any(raise)) {
          const float alpha = raise ? __builtin_amdgcn_exp2f(m_ref - mx) : 1.0f;
          if (raise) m_ref = mx;
          lsum *= alpha;
#pragma unroll
          for (int j = 0; j < DJ; ++j)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[j][i] *= alpha;
        }
        const float neg_m = (m_ref == -INFINITY) ? 0.f : -m_ref;
        float pr[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) pr[i] = __builtin_amdgcn_exp2f(fmaf(x[i], p.c, neg_m));

        // ---- P^T as B operand: per half-tile and 16-key slice f, the lane's 8 scores
        u32x4 phi[4], plo[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const float* pp = pr + f * 8;
          phi[f] = u32x4{pack_bf16x2(pp[0], pp[1]), pack_bf16x2(pp[2], pp[3]), pack_bf16x2(pp[4], pp[5]),
                         pack_bf16x2(pp[6], pp[7])};
          if (SPLIT) {
            float r[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              r[2 * e] = pp[2 * e] - bf16lo_to_f32(phi[f][e]);
              r[2 * e + 1] = pp[2 * e + 1] - bf16hi_to_f32(phi[f][e]);
            }
            plo[f] = u32x4{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]), pack_bf16x2(r[4], r[5]),
                           pack_bf16x2(r[6], r[7])};
          }
          // row sum of exactly the rounded weights the PV product uses (so O is
          // a normalised combination of V rows): two bf16 per dot2 instruction
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            lsum = sum_bf16x2(phi[f][e], lsum);
            if (SPLIT) lsum = sum_bf16x2(plo[f][e], lsum);
          }
        }

        // ---- O^T += V^T P^T
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int f = 0; f < 4; ++f) {
#pragma unroll
          for (int j = 0; j < DJ; ++j) {
            // V^T rows d = 32j + l%32, keys in the order of phi[f] (tile rows 16f + ...)
            const u32x4 a = tr_operand<L::kRowBytes>(vs, 16 * f, 32 * j, lane);
            oacc[j] = mfma32x32x16(a, phi[f], oacc[j]);
            if (SPLIT) oacc[j] = mfma32x32x16(a, plo[f], oacc[j]);
          }
        }
        if (!SPLIT) pipeline_tr_reads_mfma<4, 4 * DJ>();
        __builtin_amdgcn_s_setprio(0);
      }

      if (HAS_MASK && it + 1 < it_end && dma_wave && dtid < kBN)
        reinterpret_cast<float*>(nxt + L::kBytesK + L::kBytesV)[dtid] = vbyte ? 0.f : -INFINITY;
      wait_vmem();
      __syncthreads();
    };
    if constexpr (KS) {
      int st = 0;
      for (; st + 1 < nsteps; st += 2) {
        tile(it_beg + st, gsmem, gsmem + L::kStageAligned);
        tile(it_beg + st + 1, gsmem + L::kStageAligned, gsmem);
      }
      if (st < nsteps) tile(it_beg + st, gsmem, gsmem + L::kStageAligned);
    } else {
      int it = it_first;
      for (; it + 1 < ntiles; it += 2) {
        tile(it, smem, smem + L::kStageAligned);
        tile(it + 1, smem + L::kStageAligned, smem);
      }
      if (it < ntiles) tile(it, smem, smem + L::kStageAligned);
    }

    if constexpr (KS) {
      // the second group's (row max, row-sum share, O accumulators) to LDS,
      // lane-contiguous per value; the first group merges them into its own.
      // Every tile read is behind the last step's barrier, so the staging
      // buffers are free.
      constexpr int NV = 2 + 16 * DJ;
      float* xch = reinterpret_cast<float*>(smem) + wave * NV * 64 + lane;
      if (grp == 1) {
        xch[0] = m_ref;
        xch[64] = lsum;
#pragma unroll
        for (int j = 0; j < DJ; ++j)
#pragma unroll
          for (int i = 0; i < 16; ++i) xch[(2 + 16 * j + i) * 64] = oacc[j][i];
      }
      __syncthreads();
      if (grp == 1) return;
      // weights 2^(m_g - m) of each group's terms (0 for a group that saw no key)
      const float m_b = xch[0];
      const float m = fmaxf(m_ref, m_b);
      const float wa = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - m);
      const float wb = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_b - m);
      lsum = lsum * wa + xch[64] * wb;
#pragma unroll
      for (int j = 0; j < DJ; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[j][i] = oacc[j][i] * wa + xch[(2 + 16 * j + i) * 64] * wb;
      m_ref = m;
    }

    // ---- epilogue: normalise, write O (row t, dims 32j + 8*(i/4) + 4hh + i%4) and LSE
    if (t < p.n) {
      const float ltot = halves_sum(lsum);
      const int64_t obase = ((int64_t(b) * p.n + t) * p.Hq + head) * D;
      const int64_t lidx = (int64_t(b) * p.Hq + head) * p.n + t;
      float lse_out = ltot > 0.f ? (m_ref + __log2f(ltot)) * kLn2 : -INFINITY;
      float w_new = ltot > 0.f ? 1.0f / ltot : 0.f;   // scales the accumulator to this block's O
      float w_old = 0.f;                              // weight of the O already in the output
      if (O_F32 && p.accumulate) {
        // L = ln(e^L_old + e^L_new), O = e^(L_old - L) O_old + e^(L_new - L) O_new
        const float l_old = p.lse[lidx];
        const float m = fmaxf(l_old, lse_out);
        if (m == -INFINITY) {
          w_new = 0.f;
        } else {
          const float a = expf(l_old - m), c = expf(lse_out - m);
          const float sum = a + c;
          w_old = a / sum;
          w_new *= c / sum;
          lse_out = m + logf(sum);
        }
      }
#pragma unroll
      for (int j = 0; j < DJ; ++j) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d0 = j * 32 + i4 * 8 + hh * 4;
          float v0 = oacc[j][i4 * 4 + 0] * w_new, v1 = oacc[j][i4 * 4 + 1] * w_new;
          float v2 = oacc[j][i4 * 4 + 2] * w_new, v3 = oacc[j][i4 * 4 + 3] * w_new;
          if (O_F32) {
            f32x4* op = reinterpret_cast<f32x4*>(static_cast<float*>(p.o) + obase + d0);
            if (p.accumulate) {
              const f32x4 prev = *op;
              v0 = fmaf(w_old, prev[0], v0);
              v1 = fmaf(w_old, prev[1], v1);
              v2 = fmaf(w_old, prev[2], v2);
              v3 = fmaf(w_old, prev[3], v3);
            }
            *op = f32x4{v0, v1, v2, v3};
          } else {
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.o) + obase + d0) =
                u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
          }
        }
      }
      // both half-waves have read the old LSE above; only one writes it
      if (hh == 0) p.lse[lidx] = lse_out;
    }
  };
  // fewest keys of any row: min(first row + delta, nk - 1) + 1 - (last row's bound)
  if (min(pb * p.pw + p.delta, p.nk - 1) - lo_last < kSplitRows) run(std::true_type{});
  else run(std::false_type{});
}

template <int NW, int D, bool HAS_MASK, bool O_F32, bool CAUSAL, bool DOCS, bool KS = false>
hipError_t launch_fwd_t(const FwdParams& p, int blocks, hipStream_t stream) {
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<NW, D, HAS_MASK, O_F32, CAUSAL, DOCS, KS>), dim3(blocks), dim3(NW * 64), 0,
                     stream, p);
  return hipGetLastError();
}

// Long plain causal runs use 8-wave workgroups (one per CU, two waves per
// SIMD as with two 4-wave workgroups): each staged K/V tile then feeds 8
// waves, which halves the DMA writes into LDS and the L2 reads per flop
// (measured 4 % faster at n = 64K, 10 % on 128K single-head runs, identical
// output).  Short plain causal grids, where every block is resident at once
// and the longest sets the time, use the key split: 8-wave workgroups over
// the 4-wave blocks, each block's keys halved between two groups.
template <int D, bool HAS_MASK, bool O_F32>
hipError_t dispatch_causal(const FwdParams& p4, const FwdParams& p8, int blocks4, int blocks8, hipStream_t stream) {
  if constexpr (D == 128) {
    // with documents, or without the causal mask, the 8-wave form pays only
    // on long grids (measured 4-5 % faster on the 96K documents workload and
    // a 64K non-causal run, 2-4 % slower at 16K-32K)
    if (p4.doc_start != nullptr && blocks8 >= kWide8OtherBlocks)
      return launch_fwd_t<8, D, HAS_MASK, O_F32, true, true>(p8, blocks8, stream);
    if (!p4.causal && blocks8 >= kWide8OtherBlocks)
      return launch_fwd_t<8, D, HAS_MASK, O_F32, false, false>(p8, blocks8, stream);
  }
  if (p4.doc_start != nullptr) return launch_fwd_t<4, D, HAS_MASK, O_F32, true, true>(p4, blocks4, stream);
  if (!p4.causal) return launch_fwd_t<4, D, HAS_MASK, O_F32, false, false>(p4, blocks4, stream);
  if constexpr (D == 128) {
    if (blocks8 >= kWide8Blocks) return launch_fwd_t<8, D, HAS_MASK, O_F32, true, false>(p8, blocks8, stream);
    return launch_fwd_t<8, D, HAS_MASK, O_F32, true, false, true>(p4, blocks4, stream);
  }
  return launch_fwd_t<4, D, HAS_MASK, O_F32, true, false>(p4, blocks4, stream);
}

template <int D>
hipError_t dispatch_fwd(const FwdParams& p4, const FwdParams& p8, int blocks4, int blocks8, bool has_mask, bool o_f32,
                        hipStream_t stream) {
  if (has_mask)
    return o_f32 ? dispatch_causal<D, true, true>(p4, p8, blocks4, blocks8, stream)
                 : dispatch_causal<D, true, false>(p4, p8, blocks4, blocks8, stream);
  return o_f32 ? dispatch_causal<D, false, true>(p4, p8, blocks4, blocks8, stream)
               : dispatch_causal<D, false, false>(p4, p8, blocks4, blocks8, stream);
}

// workgroup shape for NW waves: query heads per workgroup (the largest
// divisor of g that divides NW) and positions per workgroup
void set_shape(FwdParams& p, int nw, int64_t n) {
  int gh = 1;
  for (int c = nw; c >= 1; --c)
    if (p.g % c == 0 && nw % c == 0) { gh = c; break; }
  p.gh = gh;
  p.pw = 32 * (nw / gh);
  p.n_pblocks = int32_t((n + p.pw - 1) / p.pw);
  p.n_hsub = p.g / gh;
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const void* q, const void* k, const void* v, const uint8_t* valid,
                                const int32_t* doc_start, void* o, float* lse, const AttnShape& s, int o_f32,
                                hipStream_t stream, const KeyBlock* kb) {
  FwdParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.valid = valid;
  p.doc_start = doc_start;
  p.o = o;
  p.lse = lse;
  p.B = s.B;
  p.n = int32_t(s.n);
  p.nk = kb ? int32_t(kb->nk) : int32_t(s.n);
  p.delta = kb ? int32_t(kb->delta) : 0;
  p.accumulate = kb ? kb->accumulate : 0;
  p.Hq = s.Hq;
  p.Hkv = s.Hkv;
  p.g = s.Hq / s.Hkv;
  p.c = s.scale * kLog2e;
  p.causal = s.causal;
  FwdParams p8 = p;
  set_shape(p, 4, s.n);
  set_shape(p8, 8, s.n);
  const int64_t blocks = int64_t(p.n_pblocks) * p.n_hsub * p.Hkv * p.B;
  const int64_t blocks8 = int64_t(p8.n_pblocks) * p8.n_hsub * p8.Hkv * p8.B;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const bool has_mask = valid != nullptr;
  if (s.D == 128) return dispatch_fwd<128>(p, p8, int(blocks), int(blocks8), has_mask, o_f32 != 0, stream);
  return dispatch_fwd<64>(p, p8, int(blocks), int(blocks8), has_mask, o_f32 != 0, stream);
}

}  // namespace ulysses
