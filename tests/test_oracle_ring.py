"""Pins for the oracle's ring-attention emulation (CPU only): block
attention and the logsumexp merge over the hops.

Checked against things other than themselves:
  * a hand-derived two-block example (tests/golden/worked_ring_merge.txt);
  * equality with unsharded attention (``oracle.attention``, itself pinned
    against brute force, torch SDPA and worked examples) for causal and
    full attention, grouped-query heads, padding, P = 1..4;
  * merge algebra: commutative, associative, an empty block is neutral;
  * blocks wholly in the causal future give L = -inf and O = 0;
  * planted mistakes (swapped weights, log-sum replaced by a max, causal mask
    on local instead of global positions) each break one of the above.
"""
import numpy as np
import pytest

import oracle
from oracle.ring import block_attn, merge, ring_fwd


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def test_worked_merge(golden):
    g = golden("worked_ring_merge.txt")
    q = np.array(g["q"]).reshape(1, 1, 1, 1)
    k = np.array(g["k"]).reshape(1, 2, 1, 1)
    v = np.array(g["v"]).reshape(1, 2, 1, 1)
    O1, L1 = block_attn(q, k[:, :1], v[:, :1], 1.0, 1, 0)
    O2, L2 = block_attn(q, k[:, 1:], v[:, 1:], 1.0, 1, 1)
    assert O1.ravel()[0] == g["o1"] and L1.ravel()[0] == g["l1"]
    np.testing.assert_allclose([O2.ravel()[0], L2.ravel()[0]], [g["o2"], g["l2"]], rtol=0, atol=1e-15)
    O, L = merge(O1, L1, O2, L2)
    np.testing.assert_allclose([O.ravel()[0], L.ravel()[0]], [g["o"], g["lse"]], rtol=0, atol=1e-15)


@pytest.mark.parametrize("P,nl,Hq,Hkv,D,causal,masked", [
    (1, 9, 2, 1, 3, True, False), (2, 5, 4, 2, 4, True, True), (4, 6, 4, 4, 2, True, False),
    (3, 4, 2, 1, 5, False, True), (4, 8, 8, 2, 3, True, True),
])
def test_ring_equals_unsharded(P, nl, Hq, Hkv, D, causal, masked):
    B = 2
    qs, ks, vs = rnd(1, P, B, nl, Hq, D), rnd(2, P, B, nl, Hkv, D), rnd(3, P, B, nl, Hkv, D)
    valid = None
    if masked:
        valid = (np.random.default_rng(4).random((P, B, nl)) > 0.3).astype(np.uint8)
        valid[0, :, 0] = 1
    O, L = ring_fwd(qs, ks, vs, 0.45, causal, valid)
    full_valid = None if valid is None else oracle.unshard(valid[..., None, None])[..., 0, 0]
    Of, Lf = oracle.attn_fwd(oracle.unshard(qs), oracle.unshard(ks), oracle.unshard(vs), 0.45, causal, full_valid)
    np.testing.assert_allclose(oracle.unshard(O), Of, rtol=0, atol=1e-12)
    Lr = np.concatenate([L[i] for i in range(P)], axis=-1)            # [B][Hq][n]
    np.testing.assert_array_equal(np.isneginf(Lr), np.isneginf(Lf))
    np.testing.assert_allclose(Lr[np.isfinite(Lf)], Lf[np.isfinite(Lf)], rtol=0, atol=1e-12)


def test_merge_algebra():
    parts = []
    for s in range(3):
        q, k, v = rnd(10 + s, 1, 7, 2, 4), rnd(20 + s, 1, 5, 1, 4), rnd(30 + s, 1, 5, 1, 4)
        parts.append(block_attn(q, k, v, 0.7, 0, 0, causal=False))
    (a, la), (b, lb), (c, lc) = parts
    O1, L1 = merge(a, la, b, lb)
    O2, L2 = merge(b, lb, a, la)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
    O3, L3 = merge(*merge(a, la, b, lb), c, lc)
    O4, L4 = merge(a, la, *merge(b, lb, c, lc))
    np.testing.assert_allclose(O3, O4, rtol=0, atol=1e-14)
    np.testing.assert_allclose(L3, L4, rtol=0, atol=1e-14)
    empty_O, empty_L = np.zeros_like(a), np.full_like(la, -np.inf)
    O5, L5 = merge(a, la, empty_O, empty_L)
    assert np.array_equal(O5, a) and np.array_equal(L5, la)


def test_future_block_is_empty():
    q, k, v = rnd(5, 1, 6, 2, 3), rnd(6, 1, 6, 1, 3), rnd(7, 1, 6, 1, 3)
    O, L = block_attn(q, k, v, 1.0, 0, 6)
    assert np.all(O == 0) and np.all(np.isneginf(L))


def _merge_swapped(O1, L1, O2, L2):
    return _orig_merge(O1, L2, O2, L1)


def _merge_max(O1, L1, O2, L2):
    O, L = _orig_merge(O1, L1, O2, L2)
    return O, np.maximum(L1, L2)


def _block_local(q, k, v, scale, q_off, k_off, causal=True, key_valid=None):
    return _orig_block(q, k, v, scale, 0, 0, causal, key_valid)


_orig_merge = oracle.ring.merge
_orig_block = oracle.ring.block_attn


@pytest.mark.parametrize("attr,fn", [("merge", _merge_swapped), ("merge", _merge_max), ("block_attn", _block_local)])
def test_ring_mutation_is_caught(attr, fn, monkeypatch):
    monkeypatch.setattr(oracle.ring, attr, fn)
    with pytest.raises(AssertionError):
        test_ring_equals_unsharded(2, 5, 4, 2, 4, True, True)
