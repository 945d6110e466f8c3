"""Pins for the oracle's emulated all-to-all exchanges (CPU only).

Each check is independent of the oracle's own loops: a hand-written index
fixture, an independent reshape/transpose derivation, round trips, the
P = 1 and H = P special cases, survival of every bfloat16 bit pattern, and
the constraints the pages state (heads >= shards; n divisible by shards).
"""
import numpy as np
import pytest

import oracle
from synth import random_bits, streams


def test_golden_index_example(golden):
    g = golden("seq2head_P2_n4_H4_D1.txt")
    xs = np.zeros((2, 1, 2, 4, 1), dtype=np.int64)
    xs[0, 0, :, :, 0] = np.array(g["src_rank0"])
    xs[1, 0, :, :, 0] = np.array(g["src_rank1"])
    y = oracle.seq2head(xs)
    assert y.shape == (2, 1, 4, 2, 1)
    assert np.array_equal(y[0, 0, :, :, 0], np.array(g["dst_rank0"]))
    assert np.array_equal(y[1, 0, :, :, 0], np.array(g["dst_rank1"]))
    assert np.array_equal(oracle.head2seq(y), xs)


@pytest.mark.parametrize("P,B,nl,H,D", [(1, 1, 5, 3, 4), (2, 1, 3, 4, 2), (4, 2, 3, 8, 3), (8, 1, 2, 8, 1), (3, 2, 4, 6, 5)])
def test_index_formula_on_iota(P, B, nl, H, D):
    """dst[j][b][i*nl+s][h'][c] == src[i][b][s][j*H/P+h'][c] for every index."""
    xs = np.arange(P * B * nl * H * D, dtype=np.int64).reshape(P, B, nl, H, D)
    y = oracle.seq2head(xs)
    hp = H // P
    for j in range(P):
        for b in range(B):
            for i in range(P):
                for s in range(nl):
                    for hh in range(hp):
                        for c in range(D):
                            assert y[j, b, i * nl + s, hh, c] == xs[i, b, s, j * hp + hh, c]


@pytest.mark.parametrize("P,nl,H,D", [(2, 3, 4, 2), (4, 5, 8, 3), (4, 2, 32, 4)])
def test_matches_reshape_transpose_derivation(P, nl, H, D):
    """Independent derivation: [P_src][nl][P_dst][H/P*D] -> [P_dst][P_src][nl][H/P*D]."""
    xs = np.arange(P * nl * H * D, dtype=np.int64).reshape(P, 1, nl, H, D)
    a = xs.reshape(P, nl, P, (H // P) * D).transpose(2, 0, 1, 3)
    expect = a.reshape(P, 1, P * nl, H // P, D)
    assert np.array_equal(oracle.seq2head(xs), expect)
    # and the inverse derivation for head2seq: [P_dst][P_src][nl][r] -> [P_src][nl][P_dst][r]
    back = expect.reshape(P, P, nl, (H // P) * D).transpose(1, 2, 0, 3).reshape(P, 1, nl, H, D)
    assert np.array_equal(oracle.head2seq(expect), back)


def test_round_trip_bitwise_random_bits():
    g = streams(11)[5]
    xs = random_bits(g, (4, 2, 7, 8, 16))
    y = oracle.seq2head(xs)
    assert np.array_equal(oracle.head2seq(y).view(np.uint16), xs.view(np.uint16))
    assert np.array_equal(oracle.seq2head(oracle.head2seq(y)), y)


def test_all_bf16_bit_patterns_survive():
    pats = np.arange(1 << 16, dtype=np.uint16)          # includes NaN payloads, Inf, subnormals
    xs = pats.reshape(4, 1, 64, 8, 32)
    y = oracle.seq2head(xs)
    assert np.array_equal(np.sort(y.ravel()), pats)
    assert np.array_equal(oracle.head2seq(y), xs)


def test_P1_is_identity():
    xs = np.arange(2 * 6 * 3 * 4, dtype=np.int32).reshape(1, 2, 6, 3, 4)
    assert np.array_equal(oracle.seq2head(xs), xs)
    assert np.array_equal(oracle.head2seq(xs), xs)


def test_one_head_per_rank():
    P, nl, D = 4, 3, 2
    x = np.arange(P * nl * P * D, dtype=np.int64).reshape(1, P * nl, P, D)   # global [B][n][H=P][D]
    y = oracle.seq2head(oracle.shard(x, P))
    for j in range(P):
        assert np.array_equal(y[j][:, :, 0, :], x[:, :, j, :])


def test_shard_unshard():
    x = np.arange(2 * 12 * 4 * 3).reshape(2, 12, 4, 3)
    xs = oracle.shard(x, 4)
    for i in range(4):
        assert np.array_equal(xs[i], x[:, 3 * i:3 * i + 3])
    assert np.array_equal(oracle.unshard(xs), x)


@pytest.mark.parametrize("P,n,H", [(4, 8, 2), (4, 8, 6), (3, 10, 6), (0, 4, 4)])
def test_constraints_rejected(P, n, H):
    with pytest.raises(ValueError):
        oracle.check_constraints(P, n, H)


def test_constraint_in_exchange():
    with pytest.raises(ValueError):
        oracle.seq2head(np.zeros((4, 1, 2, 2, 1)))          # H=2 < P=4
    with pytest.raises(ValueError):
        oracle.shard(np.zeros((1, 10, 4, 1)), 4)            # n=10 not divisible by 4
