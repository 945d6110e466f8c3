"""Oracle for the ring-attention alternative, emulated on one device.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Pinned by
``tests/test_oracle_ring.py``.

What the pages fix: Ring Attention keeps each rank's sequence shard of the
queries and passes the key/value shards around a ring, P - 1
point-to-point hops, with no limit on the head count ([HFSUM] "與 Ring
Attention 的比較"; [ALST] "Complexitatea comunicațională" and "Comparând
Ulysses cu Ring Attention").  The pages do not say how a rank combines the
attention over the blocks it receives.  The reading taken is the exact
combination of softmax attentions over disjoint key sets:

  for one row, block b gives O_b (softmax over b's visible keys) and L_b
  (logsumexp over the same keys); over the union of the blocks
      L = ln sum_b exp(L_b),      O = sum_b exp(L_b - L) O_b
  (a block with no visible key has L_b = -inf and weight 0).

Rank i holds queries at global positions [i*nl, (i+1)*nl) and, at hop h,
the key/value shard j = (i - h) mod P at positions [j*nl, (j+1)*nl);
causal masking is on global positions.  All heads stay on every rank
(grouped-query heads map as in ``attention``).  Float64 throughout.
"""
from __future__ import annotations

import numpy as np

from .attention import kv_head_of


def block_attn(q, k, v, scale: float, q_off: int, k_off: int, causal: bool = True, key_valid=None):
    """Attention of ``q`` ``[B][nq][Hq][D]`` (global rows q_off..) against the
    key block ``k``, ``v`` ``[B][nk][Hkv][D]`` (global keys k_off..) alone.
    Returns ``(O [B][nq][Hq][D], L [B][Hq][nq])``; rows with no visible key in
    the block get O = 0 and L = -inf."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, nq, Hq, D = q.shape
    nk, Hkv = k.shape[1], k.shape[2]
    rows = q_off + np.arange(nq)
    keys = k_off + np.arange(nk)
    O = np.zeros((B, nq, Hq, D))
    L = np.full((B, Hq, nq), -np.inf)
    for b in range(B):
        allow = np.ones((nq, nk), dtype=bool)
        if causal:
            allow &= keys[None, :] <= rows[:, None]
        if key_valid is not None:
            allow &= (np.asarray(key_valid[b]) != 0)[None, :]
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            S = scale * (q[b, :, h, :] @ k[b, :, g, :].T)
            Sm = np.where(allow, S, -np.inf)
            m = Sm.max(axis=1)
            ms = np.where(np.isfinite(m), m, 0.0)
            w = np.where(allow, np.exp(Sm - ms[:, None]), 0.0)
            tot = w.sum(axis=1)
            with np.errstate(divide="ignore", invalid="ignore"):
                O[b, :, h, :] = np.where(tot[:, None] > 0, (w @ v[b, :, g, :]) / tot[:, None], 0.0)
                L[b, h, :] = np.where(tot > 0, m + np.log(tot), -np.inf)
    return O, L


def merge(O1, L1, O2, L2):
    """Combine two partial results over disjoint key sets (formula above)."""
    L1 = np.asarray(L1, dtype=np.float64)
    L2 = np.asarray(L2, dtype=np.float64)
    m = np.maximum(L1, L2)
    ms = np.where(np.isfinite(m), m, 0.0)
    w1 = np.where(np.isfinite(L1), np.exp(L1 - ms), 0.0)
    w2 = np.where(np.isfinite(L2), np.exp(L2 - ms), 0.0)
    s = w1 + w2
    with np.errstate(divide="ignore", invalid="ignore"):
        L = np.where(s > 0, ms + np.log(s), -np.inf)
        # weights per row, moved to the [B][n][H] layout of O
        a1 = np.where(s > 0, w1 / s, 0.0).transpose(0, 2, 1)[..., None]
        a2 = np.where(s > 0, w2 / s, 0.0).transpose(0, 2, 1)[..., None]
    return a1 * O1 + a2 * O2, L


def ring_fwd(q_seq, k_seq, v_seq, scale: float, causal: bool = True, key_valid_seq=None):
    """Sequence-sharded ``[P][B][nl][H][D]`` inputs (all heads on every rank)
    -> ``(O_seq [P][B][nl][Hq][D], L [P][B][Hq][nl])``.  Rank i starts with
    its own shard and merges the blocks it receives at hops 1..P-1; blocks
    entirely in the causal future of its rows contribute nothing."""
    P, B, nl = q_seq.shape[:3]
    Os, Ls = [], []
    for i in range(P):
        O = L = None
        for h in range(P):
            j = (i - h) % P
            kv = None if key_valid_seq is None else key_valid_seq[j]
            Ob, Lb = block_attn(q_seq[i], k_seq[j], v_seq[j], scale, i * nl, j * nl, causal, kv)
            if O is None:
                O, L = Ob, Lb
            else:
                O, L = merge(O, L, Ob, Lb)
        Os.append(O)
        Ls.append(L)
    return np.stack(Os), np.stack(Ls)
