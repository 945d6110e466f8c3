"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module holds none of the method's arithmetic: it draws random numbers,
rounds them to bfloat16 storage, and builds the key-validity vector and the
per-token document starts of a packed sequence of variable-length
documents.  Both the HIP path and the
CPU oracle receive exactly these arrays, so the two sides never share any
step of the computation itself.

Recipe (one ``numpy.random.SeedSequence`` per workload number ``c``):
``SeedSequence(c).spawn(7)`` gives, in order, the child streams for
Q, K, V, dO, the document lengths, the repack bit patterns and the row
sampler.  Each child drives a ``numpy.random.Generator(PCG64(child))``.
Activations are ``standard_normal(float32)`` in C order of the stated
shape, then rounded to bfloat16 with round-to-nearest-even (the fp32
workload keeps the fp32 values).

The pages describe the inputs only as the per-rank query/key/value
projections of a training sequence (page "Paralelismul de Secvență
Ulysses...", section "Mecanismul de funcționare Ulysses", steps 1-2);
N(0,1) activations of the stated shapes stand in for the projections of
the real models and datasets the pages train on.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

STREAM_Q, STREAM_K, STREAM_V, STREAM_DO, STREAM_DOCS, STREAM_BITS, STREAM_ROWS = range(7)


def streams(c: int) -> list[np.random.Generator]:
    """The seven independent generators of workload ``c`` (order fixed above)."""
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(c).spawn(7)]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16 (round to nearest, ties to even).

    Returns the uint16 bit patterns.  Only finite inputs are expected here
    (normal draws); NaN/Inf bit patterns are produced directly as raw uint16
    by :func:`random_bits` when a test wants them.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float64."""
    return bf16_bits_to_f32(b).astype(np.float64)


def normal_bf16(gen: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) float32 draws in C order, rounded to bfloat16 bits."""
    return f32_to_bf16_bits(gen.standard_normal(size=shape, dtype=np.float32))


def random_bits(gen: np.random.Generator, shape) -> np.ndarray:
    """Uniform 16-bit patterns (every encoding, NaN/Inf/subnormal included)."""
    return gen.integers(0, 1 << 16, size=shape, dtype=np.uint16)


def documents(gen: np.random.Generator, n: int, pad_multiple: int, max_len: int):
    """A packed sequence of variable-length documents.

    Document lengths L ~ U{1..max_len}; each document is followed by
    ``(-L) mod pad_multiple`` pad tokens (padding to a multiple of the
    number of shards).  Packing stops at the first document that no longer
    fits; it is truncated to fill the sequence exactly, with no pad after it.
    Returns ``(valid, doc_start, lengths)``: ``valid`` (uint8, 1 = real
    token), ``doc_start`` (int32, the position of the first token of each
    token's document; a document's pad tokens belong to it) and the list of
    document lengths as packed.
    """
    valid = np.zeros(n, dtype=np.uint8)
    doc_start = np.zeros(n, dtype=np.int32)
    pos = 0
    lengths: list[int] = []
    while pos < n:
        L = int(gen.integers(1, max_len + 1))
        pad = (-L) % pad_multiple
        if pos + L + pad > n:
            L = n - pos
            pad = 0
        valid[pos:pos + L] = 1
        doc_start[pos:pos + L + pad] = pos
        lengths.append(L)
        pos += L + pad
    return valid, doc_start, lengths


def document_valid(gen: np.random.Generator, n: int, pad_multiple: int, max_len: int) -> tuple[np.ndarray, list[int]]:
    """Key-validity vector and document lengths of :func:`documents` (same draws)."""
    valid, _, lengths = documents(gen, n, pad_multiple, max_len)
    return valid, lengths


def sample_rows(gen: np.random.Generator, n: int, count: int, extra=()) -> np.ndarray:
    """Sorted, unique seeded row indices in [0, n) plus the given extra rows."""
    picks = gen.choice(n, size=min(count, n), replace=False)
    rows = np.unique(np.concatenate([picks, np.asarray(list(extra), dtype=np.int64)]).astype(np.int64))
    return rows[(rows >= 0) & (rows < n)]


def stratified_rows(gen: np.random.Generator, n: int, count: int, valid: np.ndarray | None = None) -> np.ndarray:
    """Rows that stress tiling and masking: first/last, tile edges +-1, the
    first 512 positions (coarsely), rows next to pad tokens, plus seeded picks."""
    extra = {0, 1, 2, n - 2, n - 1}
    for t in (32, 64, 128, 256, 512, 1024):
        for m in (t - 1, t, t + 1):
            if 0 <= m < n:
                extra.add(m)
    extra.update(range(0, min(n, 512), 37))
    if valid is not None:
        edges = np.nonzero(np.diff(valid.astype(np.int8)))[0]
        for e in edges[:16]:
            extra.update((int(e), int(e) + 1))
    return sample_rows(gen, n, count, extra)


# --------------------------------------------------------------------------
# the five workloads


@dataclass
class Workload:
    """Shapes of one workload.  ``P`` is the number of emulated shards; the
    attention shapes are one GPU's share after the sequence->head exchange."""
    number: int
    name: str
    n: int
    P: int
    Hq_global: int
    Hkv_global: int
    D: int
    dtype: str           # "f32" or "bf16"
    scale: float
    causal: bool = True
    docs: bool = False   # key-padding mask from packed documents
    backward: bool = False
    notes: dict = field(default_factory=dict)

    @property
    def hq(self) -> int:
        return self.Hq_global // self.P

    @property
    def hkv(self) -> int:
        return self.Hkv_global // self.P

    @property
    def n_local(self) -> int:
        return self.n // self.P


WORKLOADS = {
    1: Workload(1, "tiny-fp32-n256-P2-4q4kv-d64", 256, 2, 4, 4, 64, "f32", 1.0 / 8.0),
    2: Workload(2, "gqa-n8192-8q2kv-d128-bf16-fwd", 8192, 4, 32, 8, 128, "bf16", 1.0 / np.sqrt(128.0)),
    3: Workload(3, "gqa-n65536-8q2kv-d128-bf16-fwd+repack", 65536, 4, 32, 8, 128, "bf16", 1.0 / np.sqrt(128.0)),
    4: Workload(4, "gqa-n98304-8q2kv-d128-bf16-docs-fwd+bwd", 98304, 4, 32, 8, 128, "bf16", 1.0 / np.sqrt(128.0),
                docs=True, backward=True),
    5: Workload(5, "mha-n1048576-1q1kv-d128-bf16-fwd", 1048576, 32, 32, 32, 128, "bf16", 1.0 / np.sqrt(128.0)),
}

# mean document length ~28.7K tokens: lengths uniform on 1..57344
DOC_MAX_LEN = 57344


def local_attention_inputs(c: int, n: int | None = None, with_grad: bool = False):
    """One GPU's attention inputs for workload ``c`` (optionally at a smaller n).

    Returns a dict with ``q``, ``k``, ``v`` (and ``do``) as bfloat16 bit
    patterns (uint16) or float32 values, shaped ``[1][n][h][D]``, plus
    ``valid`` (uint8 ``[1][n]`` or None) and the workload record.
    Drawn directly at the local shape: the local share after the exchange is
    a permutation of the global tensor, and the permutation itself is
    exercised separately on the global tensors.
    """
    w = WORKLOADS[c]
    n = w.n if n is None else n
    g = streams(c)
    shp_q = (1, n, w.hq, w.D)
    shp_kv = (1, n, w.hkv, w.D)
    if w.dtype == "bf16":
        draw = normal_bf16
    else:
        def draw(gen, shape):
            return gen.standard_normal(size=shape, dtype=np.float32)
    out = {
        "q": draw(g[STREAM_Q], shp_q),
        "k": draw(g[STREAM_K], shp_kv),
        "v": draw(g[STREAM_V], shp_kv),
        "valid": None,
        "workload": w,
        "n": n,
    }
    if with_grad or w.backward:
        out["do"] = draw(g[STREAM_DO], shp_q)
    if w.docs:
        valid, doc_start, lengths = documents(g[STREAM_DOCS], n, w.P, min(DOC_MAX_LEN, n))
        out["valid"] = valid.reshape(1, n)
        out["doc_start"] = doc_start.reshape(1, n)
        out["doc_lengths"] = lengths
    out["row_gen"] = g[STREAM_ROWS]
    return out


def global_sharded_inputs(c: int, n: int | None = None):
    """Sequence-sharded global Q/K/V for workload ``c``: ``[P][1][n/P][H][D]``.

    Rank i holds global tokens [i*n/P, (i+1)*n/P) (page "Paralelismul de
    Secvență Ulysses...", section "Mecanismul de funcționare Ulysses", step 1).
    """
    w = WORKLOADS[c]
    n = w.n if n is None else n
    g = streams(c)
    nl = n // w.P
    if w.dtype == "bf16":
        draw = normal_bf16
    else:
        def draw(gen, shape):
            return gen.standard_normal(size=shape, dtype=np.float32)
    return {
        "q": draw(g[STREAM_Q], (w.P, 1, nl, w.Hq_global, w.D)),
        "k": draw(g[STREAM_K], (w.P, 1, nl, w.Hkv_global, w.D)),
        "v": draw(g[STREAM_V], (w.P, 1, nl, w.Hkv_global, w.D)),
        "workload": w,
        "n": n,
    }


def repack_bits(c: int, shape) -> np.ndarray:
    """Random 16-bit patterns of the given shape for the bitwise repack checks."""
    return random_bits(streams(c)[STREAM_BITS], shape)
