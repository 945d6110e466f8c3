"""Checks of the seeded input generators (CPU only)."""
import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    x = synth.streams(0)[0].standard_normal(100000, dtype=np.float32) * 3.0
    x = np.concatenate([x, np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0], np.float32)])
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_streams_are_deterministic_and_distinct():
    a = synth.streams(3)
    b = synth.streams(3)
    assert np.array_equal(a[0].standard_normal(5), b[0].standard_normal(5))
    c = synth.streams(3)
    assert not np.array_equal(c[0].standard_normal(5), c[1].standard_normal(5))


def test_document_mask_properties():
    n, P = 98304, 4
    valid, lengths = synth.document_valid(synth.streams(4)[synth.STREAM_DOCS], n, P, synth.DOC_MAX_LEN)
    assert valid.shape == (n,) and valid[0] == 1
    assert sum(lengths) == int(valid.sum())
    # every document but the last is padded to a multiple of P
    pos = 0
    for L in lengths[:-1]:
        assert np.all(valid[pos:pos + L] == 1)
        pad = (-L) % P
        assert np.all(valid[pos + L:pos + L + pad] == 0)
        pos += L + pad
    assert pos + lengths[-1] == n and np.all(valid[pos:] == 1)


def test_local_inputs_shapes():
    d = synth.local_attention_inputs(2, n=256)
    assert d["q"].shape == (1, 256, 8, 128) and d["q"].dtype == np.uint16
    assert d["k"].shape == (1, 256, 2, 128)
    d4 = synth.local_attention_inputs(4, n=1024)
    assert d4["valid"].shape == (1, 1024) and "do" in d4
    d1 = synth.local_attention_inputs(1)
    assert d1["q"].dtype == np.float32 and d1["q"].shape == (1, 256, 2, 64)


def test_document_starts_follow_the_packing():
    n, P = 98304, 4
    valid, doc_start, lengths = synth.documents(synth.streams(4)[synth.STREAM_DOCS], n, P, synth.DOC_MAX_LEN)
    v2, l2 = synth.document_valid(synth.streams(4)[synth.STREAM_DOCS], n, P, synth.DOC_MAX_LEN)
    assert np.array_equal(valid, v2) and lengths == l2
    assert doc_start.dtype == np.int32 and doc_start.shape == (n,)
    t = np.arange(n)
    assert np.all(doc_start <= t) and np.all(np.diff(doc_start) >= 0)
    # each document (with its pad) is one run whose start is its first position
    pos = 0
    for L in lengths:
        span = L + ((-L) % P if pos + L < n else 0)
        assert np.all(doc_start[pos:pos + span] == pos)
        pos += span
    assert pos == n
