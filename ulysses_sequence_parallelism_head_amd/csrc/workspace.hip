// workspace.hip -- host-side sizing of the backward's workspace (no device
// code): how many workgroups share a key block in the dK/dV pass, and where
// each array lives in the caller's workspace.  Shared by the ABI layer (the
// size query and its validation) and the backward's launcher (the layout).
#include <algorithm>

#include "internal.h"

namespace ulysses {

namespace {
// one float32 [B][Hq][n] array, rounded up to 256 bytes
size_t row_array_bytes(int32_t B, int64_t n, int32_t Hq) {
  const size_t bytes = size_t(B) * size_t(n) * size_t(Hq) * sizeof(float);
  return (bytes + 255) / 256 * 256;
}
}  // namespace

// Workgroups per work item of the dK/dV pass (a pair of key blocks for
// causal attention, one key block otherwise), a power of two up to 8.  The
// pass runs one 8-wave workgroup per CU (registers and LDS), so its grid
// takes ceil(W s / kSlots) rounds of 1/s of an item each: the choice is the
// smallest s that minimises that makespan.  With documents the items have
// unequal lengths and more, smaller pieces balance them: there s grows until
// about 1.5 workgroups per slot.  A function of the shape only, so the
// result of a call does not depend on the device or the workspace handed in.
int attn_bwd_nsplit(int32_t B, int64_t n, int32_t Hkv, BwdKind kind) {
  constexpr int64_t kSlots = 256;   // resident workgroups of the pass on MI355X (256 CUs)
  // (factors clamped so that no product below overflows, whatever the shape)
  const int64_t nkb = std::min<int64_t>(n / 128 + (n % 128 != 0), int64_t(1) << 30);
  const int64_t heads = std::min<int64_t>(int64_t(Hkv) * B, int64_t(1) << 30);
  const int64_t items = (kind == BwdKind::kFull ? nkb : (nkb + 1) / 2) * heads;
  // four or more rounds unsplit: a split would only trim the last round
  if (items >= 4 * kSlots) return 1;
  int s = 1;
  if (kind == BwdKind::kDocs) {
    while (s < 8 && items * s < 3 * kSlots / 2) s *= 2;
    return s;
  }
  // compare ceil(items t / kSlots) / t across t = 1, 2, 4, 8 (as fractions over 8)
  int64_t best = (items + kSlots - 1) / kSlots * 8;
  for (int t = 2; t <= 8; t *= 2) {
    const int64_t cost = (items * t + kSlots - 1) / kSlots * (8 / t);
    if (cost < best) {
      best = cost;
      s = t;
    }
  }
  return s;
}

// The most any kind of call takes: what the workspace is sized for.
int attn_bwd_nsplit_max(int32_t B, int64_t n, int32_t Hkv) {
  return std::max({attn_bwd_nsplit(B, n, Hkv, BwdKind::kCausal), attn_bwd_nsplit(B, n, Hkv, BwdKind::kFull),
                   attn_bwd_nsplit(B, n, Hkv, BwdKind::kDocs)});
}

// Layout (offsets in floats): -Dl = -(dO . O), then the base-2 logsumexp, then
// with several splits their partial dK and dV, [nsplit][B][n][Hkv][D] each.
BwdWorkspace attn_bwd_workspace(int32_t B, int64_t n, int32_t Hq, int32_t Hkv, int32_t D, int nsplit) {
  BwdWorkspace w;
  const size_t rows = row_array_bytes(B, n, Hq) / sizeof(float);
  const size_t part = nsplit > 1 ? size_t(nsplit) * size_t(B) * size_t(n) * size_t(Hkv) * size_t(D) : 0;
  w.rowdot = 0;
  w.lse2 = rows;
  w.dk_part = 2 * rows;
  w.dv_part = 2 * rows + part;
  w.bytes = (2 * rows + 2 * part) * sizeof(float);
  return w;
}

size_t attn_bwd_workspace_bytes(int32_t B, int64_t n, int32_t Hq, int32_t Hkv, int32_t D, int nsplit) {
  return attn_bwd_workspace(B, n, Hq, Hkv, D, nsplit).bytes;
}

}  // namespace ulysses
