"""Oracle for rotary position embedding at global positions, applied before
the first exchange.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Pinned by
``tests/test_oracle_rope_loss.py``.

What the pages fix: the ms-swift page ([SWIFT] "ms-swift性能优化：Ulysses并行
技术降低长文本显存", section "6. 使用建议与避坑指南", its troubleshooting
table) traces repeated tokens to a rotary position encoding that ignores the
offset of the sequence after sharding, and names linear position scaling as
a workaround.  With contiguous shards ([ALST] "Mecanismul de funcționare
Ulysses", step 1) rank i's local token s sits at global position
i * n/P + s, and that is the position its rotation must use.

The rotation itself is not on the pages.  The reading taken is the rotary
embedding as the pages' models (Qwen) use it, with the two halves of the head
dimension paired: for d in [0, D/2)

  theta_d(pos) = (pos / scale) * base ** (-2 d / D)
  out[d]       = x[d] cos(theta) - x[d + D/2] sin(theta)
  out[d + D/2] = x[d + D/2] cos(theta) + x[d] sin(theta)

``scale`` is the linear position scaling factor (1 = none); ``base`` the
rotary base.  Evaluated in float64 with NumPy's cos/sin.
"""
from __future__ import annotations

import numpy as np


def global_positions(P: int, n_local: int) -> np.ndarray:
    """[P][n_local] global position of local token s on rank i."""
    return (np.arange(P, dtype=np.int64)[:, None] * n_local + np.arange(n_local, dtype=np.int64)[None, :])


def rope(x, positions, base: float, scale: float = 1.0) -> np.ndarray:
    """Rotate ``x`` ``[..., n][H][D]`` (float64) at ``positions`` ``[..., n]``."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    if D % 2 != 0:
        raise ValueError("the head dimension must be even")
    half = D // 2
    pos = np.asarray(positions, dtype=np.float64) / float(scale)
    out = np.empty_like(x)
    for d in range(half):
        theta = pos * float(base) ** (-2.0 * d / D)          # [..., n]
        c = np.cos(theta)[..., None]                          # broadcast over heads
        s = np.sin(theta)[..., None]
        a, b = x[..., d], x[..., d + half]
        out[..., d] = a * c - b * s
        out[..., d + half] = b * c + a * s
    return out


def seq2head_rope(x_seq, base: float, scale: float = 1.0) -> np.ndarray:
    """Sequence shards ``[P][B][n/P][H][D]``: rotate each shard at its global
    positions, then run the first exchange.  Returns ``[P][B][n][H/P][D]``
    float64."""
    from .exchange import seq2head
    x = np.asarray(x_seq, dtype=np.float64)
    P, B, nl = x.shape[:3]
    pos = global_positions(P, nl)[:, None, :]                 # [P][1][nl]
    pos = np.broadcast_to(pos, (P, B, nl))
    return seq2head(rope(x, pos, base, scale))
