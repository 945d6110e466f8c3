"""GPU parity of the exchange permutations: bit-exact against the oracle.

Random 16-bit patterns (every bfloat16 encoding, NaN payloads included) and
float32 values are pushed through ulysses_repack_seq2head / head2seq via the
C ABI and compared bitwise with the oracle's explicit per-rank loops, from
tiny ragged shapes up to the 64K workload's [4][1][16384][32][128] bf16
tensor (512 MiB) in both directions.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import ulysses_sequence_parallelism_head_amd as U
from tests.gpu_helpers import say, device_bits

pytestmark = pytest.mark.gpu


def _bits_dev(a):
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda:0")


@pytest.mark.parametrize("P,B,nl,H,D", [
    (1, 1, 5, 3, 7), (2, 1, 3, 4, 5), (2, 2, 37, 4, 64), (4, 1, 16, 32, 128), (4, 2, 9, 8, 3),
    (8, 1, 13, 8, 128), (4, 1, 1, 4, 1), (3, 2, 11, 6, 10),
])
def test_repack_bf16_bits(P, B, nl, H, D):
    say(f"repack bf16 P={P} B={B} nl={nl} H={H} D={D}")
    g = synth.streams(100 + P * 10 + D)[synth.STREAM_BITS]
    xs = synth.random_bits(g, (P, B, nl, H, D))
    y = U.ulysses_repack_seq2head(_bits_dev(xs))
    torch.cuda.synchronize()
    assert np.array_equal(device_bits(y), oracle.seq2head(xs))
    back = U.ulysses_repack_head2seq(y)
    torch.cuda.synchronize()
    assert np.array_equal(device_bits(back), xs)


@pytest.mark.parametrize("P,B,nl,H,D", [(2, 1, 128, 4, 64), (4, 3, 7, 8, 5)])
def test_repack_f32(P, B, nl, H, D):
    say(f"repack f32 P={P} B={B} nl={nl} H={H} D={D}")
    g = synth.streams(7)[synth.STREAM_BITS]
    xs = g.integers(0, 2 ** 32, size=(P, B, nl, H, D), dtype=np.uint32)   # any bit pattern
    t = torch.from_numpy(xs.view(np.int32)).view(torch.float32).to("cuda:0")
    y = U.ulysses_repack_seq2head(t)
    got = y.view(torch.int32).cpu().numpy().view(np.uint32)
    assert np.array_equal(got, oracle.seq2head(xs))
    back = U.ulysses_repack_head2seq(y).view(torch.int32).cpu().numpy().view(np.uint32)
    assert np.array_equal(back, xs)


def test_repack_all_bf16_patterns():
    say("repack: all 65536 bf16 patterns")
    xs = np.arange(1 << 16, dtype=np.uint16).reshape(4, 1, 64, 8, 32)
    y = U.ulysses_repack_seq2head(_bits_dev(xs))
    assert np.array_equal(device_bits(y), oracle.seq2head(xs))


def test_repack_unaligned_view():
    """A source that is only element-aligned takes the narrow-vector path."""
    say("repack: 2-byte aligned source")
    g = synth.streams(9)[synth.STREAM_BITS]
    flat = synth.random_bits(g, (1 + 2 * 1 * 6 * 4 * 8,))
    base = _bits_dev(flat)
    src = base[1:].view(2, 1, 6, 4, 8)           # offset by one element: 2-byte alignment only
    assert src.data_ptr() % 16 != 0
    y = U.ulysses_repack_seq2head(src)
    assert np.array_equal(device_bits(y), oracle.seq2head(flat[1:].reshape(2, 1, 6, 4, 8)))


def test_repack_64k_workload_bitwise():
    """The 64K workload's global [4][1][16384][32][128] bf16 tensor, both directions."""
    say("repack: 64K workload, 512 MiB, both directions")
    shape = (4, 1, 16384, 32, 128)
    xs = synth.repack_bits(3, shape)
    src = _bits_dev(xs)
    y = U.ulysses_repack_seq2head(src)
    torch.cuda.synchronize()
    ref = oracle.seq2head(xs)
    assert np.array_equal(device_bits(y), ref)
    del ref
    back = U.ulysses_repack_head2seq(y)
    torch.cuda.synchronize()
    assert np.array_equal(device_bits(back), xs)


def test_repack_empty_is_noop():
    say("repack: empty")
    src = torch.empty((2, 1, 0, 4, 8), dtype=torch.bfloat16, device="cuda:0")
    y = U.ulysses_repack_seq2head(src)
    assert y.shape == (2, 1, 0, 2, 8)
