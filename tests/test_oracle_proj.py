"""Pins for the oracle's projections around the exchanges (CPU only).

Checked against things other than themselves:
  * brute force: every output element as a math.fsum over the input row and
    the weight row, placed by hand at its head-sharded (or sequence-sharded)
    position;
  * closed forms: identity weights make the QKV projection the plain first
    exchange of x (bitwise, against ``exchange.seq2head``, itself pinned),
    and the output projection with identity weights the plain second
    exchange; a weight with a single 1 picks one input feature;
  * linearity in x and in W;
  * planted mistakes (K and V weight blocks swapped, heads concatenated in
    the wrong order) each break one of the above.
"""
import math

import numpy as np
import pytest

import oracle
from oracle.proj import qkv_proj_seq2head, head2seq_out_proj


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def test_qkv_brute_force():
    P, B, nl, hidden, Hq, Hkv, D = 2, 1, 3, 5, 4, 2, 2
    x, w = rnd(1, P, B, nl, hidden), rnd(2, (Hq + 2 * Hkv) * D, hidden)
    q, k, v = qkv_proj_seq2head(x, w, Hq, Hkv, D)
    outs = {"q": (q, 0, Hq), "k": (k, Hq, Hkv), "v": (v, Hq + Hkv, Hkv)}
    for name, (arr, h0, H) in outs.items():
        hp = H // P
        for i in range(P):
            for b in range(B):
                for s in range(nl):
                    for h in range(H):
                        for c in range(D):
                            f = (h0 + h) * D + c
                            val = math.fsum(x[i, b, s, e] * w[f, e] for e in range(hidden))
                            j, hl = h // hp, h % hp
                            assert abs(arr[j, b, i * nl + s, hl, c] - val) <= 1e-13, (name, i, s, h, c)


def test_out_proj_brute_force():
    P, B, nl, Hq, D, hidden = 2, 2, 3, 4, 2, 3
    o_h = rnd(3, P, B, P * nl, Hq // P, D)
    w_o = rnd(4, hidden, Hq * D)
    y = head2seq_out_proj(o_h, w_o)
    hp = Hq // P
    for i in range(P):
        for b in range(B):
            for s in range(nl):
                row = [o_h[h // hp, b, i * nl + s, h % hp, c] for h in range(Hq) for c in range(D)]
                for f in range(hidden):
                    val = math.fsum(r * w_o[f, e] for e, r in enumerate(row))
                    assert abs(y[i, b, s, f] - val) <= 1e-13


def test_identity_weights_are_the_exchanges():
    P, B, nl, Hq, Hkv, D = 4, 2, 5, 8, 4, 3
    hidden = Hq * D
    x = rnd(5, P, B, nl, hidden)
    w = np.zeros(((Hq + 2 * Hkv) * D, hidden))
    w[:Hq * D] = np.eye(hidden)
    w[Hq * D:(Hq + Hkv) * D, :Hkv * D] = np.eye(Hkv * D)          # K = the first Hkv heads of x
    w[(Hq + Hkv) * D:, hidden - Hkv * D:] = np.eye(Hkv * D)        # V = the last Hkv heads of x
    q, k, v = qkv_proj_seq2head(x, w, Hq, Hkv, D)
    xs = x.reshape(P, B, nl, Hq, D)
    assert np.array_equal(q, oracle.seq2head(xs))
    assert np.array_equal(k, oracle.seq2head(xs[..., :Hkv, :]))
    assert np.array_equal(v, oracle.seq2head(xs[..., Hq - Hkv:, :]))
    y = head2seq_out_proj(q, np.eye(hidden))
    assert np.array_equal(y, x)


def test_linearity():
    P, B, nl, hidden, Hq, Hkv, D = 2, 1, 4, 6, 2, 2, 3
    x1, x2 = rnd(6, P, B, nl, hidden), rnd(7, P, B, nl, hidden)
    w1, w2 = rnd(8, (Hq + 2 * Hkv) * D, hidden), rnd(9, (Hq + 2 * Hkv) * D, hidden)
    a = qkv_proj_seq2head(2 * x1 + x2, w1, Hq, Hkv, D)
    b1, b2 = qkv_proj_seq2head(x1, w1, Hq, Hkv, D), qkv_proj_seq2head(x2, w1, Hq, Hkv, D)
    for t, u, z in zip(a, b1, b2):
        np.testing.assert_allclose(t, 2 * u + z, rtol=0, atol=1e-12)
    c = qkv_proj_seq2head(x1, w1 - 3 * w2, Hq, Hkv, D)
    d1, d2 = qkv_proj_seq2head(x1, w1, Hq, Hkv, D), qkv_proj_seq2head(x1, w2, Hq, Hkv, D)
    for t, u, z in zip(c, d1, d2):
        np.testing.assert_allclose(t, u - 3 * z, rtol=0, atol=1e-12)


def _kv_swapped(x_seq, w, Hq, Hkv, D):
    q, k, v = _orig_qkv(x_seq, w, Hq, Hkv, D)
    return q, v, k


def _heads_reversed(o_heads, w_o):
    o = oracle.head2seq(np.asarray(o_heads, dtype=np.float64))[..., ::-1, :]
    P, B, nl, Hq, D = o.shape
    return o.reshape(P, B, nl, Hq * D) @ np.asarray(w_o).T


_orig_qkv = oracle.proj.qkv_proj_seq2head


@pytest.mark.parametrize("name,fn,pin", [("kv_swapped", _kv_swapped, "test_qkv_brute_force"),
                                         ("heads_reversed", _heads_reversed, "test_out_proj_brute_force")])
def test_proj_mutation_is_caught(name, fn, pin, monkeypatch):
    attr = "qkv_proj_seq2head" if name == "kv_swapped" else "head2seq_out_proj"
    monkeypatch.setitem(globals(), attr, fn)
    with pytest.raises(AssertionError):
        globals()[pin]()
