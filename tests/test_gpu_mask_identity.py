"""A key mask of all ones changes nothing: the forward and the backward called
with it equal the calls without a mask, bit for bit.

The masked kernels stage each key tile's validity bytes and start the score
accumulators from a bias of 0 (valid) or -inf (padding); keys past n take the
byte of key n-1 and are removed by the tail compare.  With every key valid the
bias is 0 everywhere and 0 + s = s exactly, so both paths must agree on every
bit.  The cases reach each workgroup form of the forward and of dq (4-wave,
key split, 8-wave), ragged n, D = 64 and 128, non-causal attention and packed
documents.  The outputs are compared with each other, not with the oracle:
their agreement with it is checked by the parity tests of each path."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
import ulysses_sequence_parallelism_head_amd as U
from gpu_helpers import bits_to_device, device_bits, say

pytestmark = pytest.mark.gpu


def _inputs(seed, n, Hq, Hkv, D):
    g = synth.streams(seed)
    q = bits_to_device(synth.normal_bf16(g[0], (1, n, Hq, D)))
    k = bits_to_device(synth.normal_bf16(g[1], (1, n, Hkv, D)))
    v = bits_to_device(synth.normal_bf16(g[2], (1, n, Hkv, D)))
    do = bits_to_device(synth.normal_bf16(g[3], (1, n, Hq, D)))
    return q, k, v, do


def _same_f32(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def _step(q, k, v, do, valid, scale, causal, docs):
    """Forward with a bf16 O (as the timed step stores it), then the backward."""
    if docs is None:
        o, lse = U.ulysses_attn_fwd(q, k, v, valid, scale, causal, o_dtype=torch.bfloat16)
        dq, dk, dv = U.ulysses_attn_bwd(q, k, v, o, lse, do, valid, scale, causal)
    else:
        o, lse = U.ulysses_attn_fwd_docs(q, k, v, docs, valid, scale, o_dtype=torch.bfloat16)
        dq, dk, dv = U.ulysses_attn_bwd_docs(q, k, v, o, lse, do, docs, valid, scale)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


@pytest.mark.parametrize("n,Hq,Hkv,D,causal,docs", [
    (300, 8, 2, 128, True, False),      # key-split forward and dq
    (1000, 4, 4, 64, True, False),      # D = 64, 4-wave workgroups
    (8200, 8, 2, 128, True, False),     # key split, ragged tail tile
    (16390, 8, 2, 128, True, False),    # 8-wave forward and dq, ragged
    (2100, 8, 2, 128, False, False),    # non-causal
    (3000, 8, 2, 128, True, True),      # packed documents
])
def test_all_valid_mask_is_bitwise_no_mask(n, Hq, Hkv, D, causal, docs):
    say(f"all-valid mask vs none: n={n} Hq={Hq} Hkv={Hkv} D={D} causal={causal} docs={docs}")
    q, k, v, do = _inputs(71, n, Hq, Hkv, D)
    ds = None
    if docs:
        _, d, _ = synth.documents(synth.streams(72)[4], n, 4, n // 3)
        ds = torch.from_numpy(d.reshape(1, n)).to("cuda:0")
    ones = torch.ones((1, n), dtype=torch.uint8, device="cuda:0")
    scale = D ** -0.5
    o0, l0, dq0, dk0, dv0 = _step(q, k, v, do, None, scale, causal, ds)
    o1, l1, dq1, dk1, dv1 = _step(q, k, v, do, ones, scale, causal, ds)
    assert np.array_equal(device_bits(o0), device_bits(o1)), "O"
    assert _same_f32(l0, l1), "LSE"
    assert _same_f32(dq0, dq1), "dQ"
    assert _same_f32(dk0, dk1), "dK"
    assert _same_f32(dv0, dv1), "dV"
