"""Pins for the oracle's rotary embedding at global positions and its
loss aggregation (CPU only).

Rotary embedding, checked against things other than itself:
  * a hand-derived example at a global position, with and without linear
    position scaling (tests/golden/worked_rope_loss.txt), exact;
  * the complex-number form: each pair (x[d], x[d + D/2]) as z = a + ib is
    multiplied by exp(i theta_d) (NumPy complex arithmetic);
  * closed forms and invariants: position 0 is the identity, each rotated
    pair keeps its norm, the score <rope(q, m), rope(k, n)> depends only on
    m - n, rotating back by the negative position restores x, scaling by f
    equals the position divided by f;
  * the exchange: rotating each shard at its global positions and then
    exchanging equals exchanging and then rotating at the head-sharded
    layout's positions 0..n-1 (bitwise), and rotating at local positions
    (the pitfall) does not.
Loss aggregation: the hand-derived example; the mean over every valid token
of the unsharded sequence; resharding invariance; equal to the mean of the
per-rank means only when the counts are equal; NaN without valid tokens.
"""
import math

import numpy as np
import pytest

import oracle
from oracle.rope import rope, seq2head_rope, global_positions
from oracle.loss import aggregate


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def complex_rope(x, pos, base, scale=1.0):
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    h = D // 2
    z = x[..., :h] + 1j * x[..., h:]
    inv = np.power(float(base), -np.arange(0, D, 2) / D)              # [h]
    theta = (np.asarray(pos, dtype=np.float64) / scale)[..., None, None] * inv
    w = z * np.exp(1j * theta)
    return np.concatenate([w.real, w.imag], axis=-1)


# ------------------------------------------------------------------- rope
def test_rope_worked_example(golden):
    g = golden("worked_rope_loss.txt")
    pos = global_positions(g["rope_P"], g["rope_n_local"])[g["rope_rank"], g["rope_local"]]
    assert pos == 2
    x = np.array(g["rope_x"]).reshape(1, 1, 4)
    out = rope(x, np.array([pos]), g["rope_base"])
    np.testing.assert_allclose(out.ravel(), g["rope_out"], rtol=0, atol=1e-15)
    out2 = rope(x, np.array([pos]), g["rope_base"], scale=2.0)
    np.testing.assert_allclose(out2.ravel(), g["rope_out_scale2"], rtol=0, atol=1e-15)


@pytest.mark.parametrize("D,base,scale", [(128, 1e6, 1.0), (64, 1e4, 1.0), (128, 1e4, 4.0), (2, 10.0, 1.0)])
def test_rope_complex_form(D, base, scale):
    x = rnd(1, 37, 3, D)
    pos = np.random.default_rng(2).integers(0, 100000, 37)
    # the two forms round the frequency and the angle differently: angles up
    # to 1e5 rad carry an absolute error of a few ulp of 1e5 (~1e-11)
    tol = 8 * 2.0 ** -52 * float(pos.max()) * float(np.abs(x).max())
    np.testing.assert_allclose(rope(x, pos, base, scale), complex_rope(x, pos, base, scale), rtol=0, atol=tol)


def test_rope_closed_forms():
    x = rnd(3, 5, 4, 64)
    assert np.array_equal(rope(x, np.zeros(5), 1e4), x)                      # position 0
    pos = np.array([1, 17, 1000, 65535, 98303])
    y = rope(x, pos, 1e4)
    np.testing.assert_allclose(x[..., :32] ** 2 + x[..., 32:] ** 2, y[..., :32] ** 2 + y[..., 32:] ** 2,
                               rtol=1e-13)                                     # pair norms
    np.testing.assert_allclose(rope(y, -pos, 1e4), x, rtol=0, atol=1e-12)     # inverse rotation
    np.testing.assert_array_equal(rope(x, pos * 4, 1e4, scale=4.0), rope(x, pos, 1e4))


def test_rope_relative_positions():
    q, k = rnd(4, 1, 2, 128), rnd(5, 1, 2, 128)
    def score(m, n):
        return np.sum(rope(q, np.array([m]), 1e6) * rope(k, np.array([n]), 1e6), axis=-1)
    for m, n, shift in ((10, 3, 7), (5000, 4990, 60000), (0, 0, 12345)):
        np.testing.assert_allclose(score(m, n), score(m + shift, n + shift), rtol=0, atol=1e-9)


@pytest.mark.parametrize("P,nl,H,D", [(2, 3, 4, 4), (4, 8, 8, 64)])
def test_rope_before_exchange_uses_global_positions(P, nl, H, D):
    x = rnd(6, P, 2, nl, H, D)
    got = seq2head_rope(x, 1e4)
    n = P * nl
    after = oracle.seq2head(x)                                   # [P][B][n][H/P][D]
    ref = rope(after, np.broadcast_to(np.arange(n), (P, 2, n)), 1e4)
    assert np.array_equal(got, ref)
    local = oracle.seq2head(rope(x, np.broadcast_to(np.arange(nl), (P, 2, nl)), 1e4))
    assert not np.allclose(local, ref)


# ------------------------------------------------------------------- loss
def test_loss_worked_example(golden):
    g = golden("worked_rope_loss.txt")
    tl = np.array(g["loss_tokens"]).reshape(2, 1, 3)
    va = np.array(g["loss_valid"], dtype=np.uint8).reshape(2, 1, 3)
    sums, counts, loss = aggregate(tl, va)
    assert list(sums) == g["loss_rank_sum"] and list(counts) == g["loss_rank_count"]
    assert loss == g["loss_value"]
    assert np.mean(sums / counts) == 3.0 and loss != 3.0


def test_loss_is_the_mean_over_valid_tokens():
    P, B, nl = 4, 2, 257
    tl = np.abs(rnd(7, P, B, nl)) * 3.0
    va = (np.random.default_rng(8).random((P, B, nl)) > 0.3).astype(np.uint8)
    _, counts, loss = aggregate(tl, va)
    flat = tl[va != 0]
    np.testing.assert_allclose(loss, flat.mean(), rtol=1e-14)
    assert counts.sum() == flat.size
    # resharding the same tokens over 2 ranks leaves the loss unchanged
    _, _, loss2 = aggregate(tl.reshape(2, 2 * B, nl), va.reshape(2, 2 * B, nl))
    np.testing.assert_allclose(loss2, loss, rtol=1e-15)


def test_loss_equal_counts_and_empty():
    tl = np.abs(rnd(9, 3, 1, 10))
    sums, counts, loss = aggregate(tl, None)
    np.testing.assert_allclose(loss, np.mean(sums / counts), rtol=1e-15)
    s, c, l = aggregate(tl, np.zeros((3, 1, 10), np.uint8))
    assert np.all(s == 0) and np.all(c == 0) and math.isnan(l)


# ------------------------------------------------------------- planted mistakes
def _interleaved(x, positions, base, scale=1.0):
    """Wrong pairing: adjacent dims (2d, 2d+1) instead of the two halves."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    out = np.empty_like(x)
    pos = np.asarray(positions, dtype=np.float64) / scale
    for d in range(D // 2):
        th = pos * base ** (-2.0 * d / D)
        c, s = np.cos(th)[..., None], np.sin(th)[..., None]
        a, b = x[..., 2 * d], x[..., 2 * d + 1]
        out[..., 2 * d], out[..., 2 * d + 1] = a * c - b * s, b * c + a * s
    return out


def _sign_flipped(x, positions, base, scale=1.0):
    return _orig_rope(x, -np.asarray(positions, dtype=np.float64), base, scale)


def _half_frequency(x, positions, base, scale=1.0):
    return _orig_rope(x, np.asarray(positions, dtype=np.float64), base ** 0.5, scale)


def _local_positions(x_seq, base, scale=1.0):
    x = np.asarray(x_seq, dtype=np.float64)
    P, B, nl = x.shape[:3]
    return oracle.seq2head(_orig_rope(x, np.broadcast_to(np.arange(nl), (P, B, nl)), base, scale))


_orig_rope = oracle.rope.rope


def _rope_pins_fail(golden):
    try:
        test_rope_worked_example(golden)
        test_rope_complex_form(128, 1e6, 1.0)
        test_rope_before_exchange_uses_global_positions(2, 3, 4, 4)
    except AssertionError:
        return True
    return False


@pytest.mark.parametrize("name,attr,fn", [("interleaved", "rope", _interleaved), ("sign", "rope", _sign_flipped),
                                          ("frequency", "rope", _half_frequency),
                                          ("local_positions", "seq2head_rope", _local_positions)])
def test_rope_mutation_is_caught(name, attr, fn, golden, monkeypatch):
    assert not _rope_pins_fail(golden)
    monkeypatch.setattr(oracle.rope, attr, fn)
    monkeypatch.setitem(globals(), attr, fn)
    assert _rope_pins_fail(golden), f"planted mistake {name!r} went unnoticed"
