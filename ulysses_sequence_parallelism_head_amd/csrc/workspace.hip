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

// Workgroups per key-block pair of the dK/dV pass: enough that short
// sequences still give the 256 CUs about two workgroups each (one resident
// per CU).  A function of the shape only, so the result of a call does not
// depend on the device or the workspace handed in.
int attn_bwd_nsplit(int32_t B, int64_t n, int32_t Hkv) {
  const int64_t pairs = ((n + 127) / 128 + 1) / 2 * int64_t(Hkv) * B;
  int s = 1;
  while (s < 8 && pairs * s < 384) s *= 2;   // a power of two, at most 8
  return s;
}

// Layout (offsets in floats): Dl = dO . O, then the base-2 logsumexp, then
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
