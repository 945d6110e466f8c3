"""Oracle for the two emulated all-to-all exchanges of Ulysses SP.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Pinned by
``tests/test_oracle_exchange.py``.

What the pages fix ([ALST] section "Mecanismul de funcționare Ulysses",
steps 1, 3 and 5; [HFSUM] section "Ulysses 序列平行化的原理"):
  * the sequence of n tokens is cut into P contiguous shards, rank i holding
    tokens [i*n/P, (i+1)*n/P);
  * the first all-to-all leaves every rank with all n positions but only a
    subset of the heads;
  * the second all-to-all undoes the first.
Readings taken where the pages are silent:
  * rank j's head subset is the contiguous block [j*H/P, (j+1)*H/P);
  * the receive buffer of rank j is the chunks from ranks 0..P-1 concatenated
    in source-rank order along the sequence, i.e. ``[B][n][H/P][D]``, which
    (shards being contiguous) is plain global token order.
The constraints come from [HFSUM] section "與 Ring Attention 的比較" (the head
count may not be smaller than the number of shards) and [ALST] section
"Cele mai bune practici și recomandări", item 1 (the sequence length must be
divisible by the number of shards).

Arrays are moved, never computed on: any dtype works, and bit patterns
(uint16 views of bfloat16, NaN payloads included) survive unchanged.
"""
from __future__ import annotations

import numpy as np


def check_constraints(P: int, n: int, H: int) -> None:
    """Raise ValueError unless P >= 1, H >= P, H % P == 0 and n % P == 0."""
    if P < 1:
        raise ValueError(f"P={P}: need at least one shard")
    if H < P:
        raise ValueError(f"H={H} < P={P}: every rank needs at least one head")
    if H % P != 0:
        raise ValueError(f"H={H} is not divisible by P={P}")
    if n % P != 0:
        raise ValueError(f"n={n} is not divisible by P={P}")


def shard(x: np.ndarray, P: int) -> np.ndarray:
    """Sequence sharding: ``x[B][n][H][D]`` -> ``xs[P][B][n/P][H][D]``,
    rank i taking tokens [i*n/P, (i+1)*n/P)."""
    B, n, H, D = x.shape
    check_constraints(P, n, H)
    nl = n // P
    xs = np.empty((P, B, nl, H, D), dtype=x.dtype)
    for i in range(P):
        xs[i] = x[:, i * nl:(i + 1) * nl]
    return xs


def unshard(xs: np.ndarray) -> np.ndarray:
    """Inverse of :func:`shard`: concatenate the rank shards along the sequence."""
    P, B, nl, H, D = xs.shape
    x = np.empty((B, P * nl, H, D), dtype=xs.dtype)
    for i in range(P):
        x[:, i * nl:(i + 1) * nl] = xs[i]
    return x


def seq2head(xs: np.ndarray) -> np.ndarray:
    """First all-to-all, emulated: ``xs[P][B][n_l][H][D]`` -> ``y[P][B][n][H/P][D]``.

    Written as the exchange itself: every source rank i sends to every
    destination rank j the slice of its shard holding j's heads, and rank j
    stores what it receives from i at i's token range.
    """
    P, B, nl, H, D = xs.shape
    check_constraints(P, P * nl, H)
    hp = H // P
    y = np.empty((P, B, P * nl, hp, D), dtype=xs.dtype)
    for i in range(P):                      # source rank (sequence shard i)
        for j in range(P):                  # destination rank (head block j)
            sent = xs[i][:, :, j * hp:(j + 1) * hp, :]
            y[j][:, i * nl:(i + 1) * nl, :, :] = sent
    return y


def head2seq(y: np.ndarray) -> np.ndarray:
    """Second all-to-all, emulated: ``y[P][B][n][H/P][D]`` -> ``xs[P][B][n/P][H][D]``.

    Every source rank j (holding head block j for all tokens) sends to every
    destination rank i the token range of i's shard; rank i stores it at
    head block j.
    """
    P, B, n, hp, D = y.shape
    H = hp * P
    check_constraints(P, n, H)
    nl = n // P
    xs = np.empty((P, B, nl, H, D), dtype=y.dtype)
    for j in range(P):                      # source rank (head block j)
        for i in range(P):                  # destination rank (sequence shard i)
            sent = y[j][:, i * nl:(i + 1) * nl, :, :]
            xs[i][:, :, j * hp:(j + 1) * hp, :] = sent
    return xs
