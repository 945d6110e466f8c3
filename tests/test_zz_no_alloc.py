"""The no-allocation backward, ulysses_attn_bwd_noalloc, through the C ABI:
its gradients must match ulysses_attn_bwd's (same kernels, the workspace
taken from the library's fixed per-GPU scratch) on calls in a row whose
sizes shrink (nothing left in the shared scratch by one call may leak into
the next) and at the scratch limit, and it must refuse a problem one
row-block beyond the limit.  The call itself allocates nothing: torch's
allocator counts no allocation across it.

dQ must be bit-identical.  dK and dV too where the workspace call runs its
key blocks unsplit (long sequences); on short sequences the workspace call
spreads each key block's query units over several workgroups and adds
their partial sums (its workspace holds them), which the no-allocation
call, whose scratch holds only the row arrays, does not: there the two
agree to float32 summation order (relative 1e-5), and both meet the
oracle's 1e-2."""
import numpy as np
import pytest
import torch

import oracle
import synth
import ulysses_sequence_parallelism_head_amd as U
from tests.gpu_helpers import say, bits_to_device, to_f64, to_host_f64, assert_close

pytestmark = pytest.mark.gpu

LIMIT_ROWS = 1 << 21          # B * Hq * n at 16 MiB of scratch (two float32 row arrays)


def _inputs(seed, n, Hq, Hkv, D, masked):
    g = synth.streams(seed)
    q = synth.normal_bf16(g[0], (1, n, Hq, D))
    k = synth.normal_bf16(g[1], (1, n, Hkv, D))
    v = synth.normal_bf16(g[2], (1, n, Hkv, D))
    do = synth.normal_bf16(g[3], (1, n, Hq, D))
    valid = synth.document_valid(g[4], n, 4, max(1, n // 3))[0].reshape(1, n) if masked else None
    return q, k, v, do, valid


def _both(q, k, v, do, valid, scale, causal, o_dtype):
    """Gradients from the workspace call and from the no-allocation call."""
    tq, tk, tv, tdo = (bits_to_device(x) for x in (q, k, v, do))
    tval = None if valid is None else torch.from_numpy(valid).to("cuda:0")
    o, lse = U.ulysses_attn_fwd(tq, tk, tv, tval, scale, causal, o_dtype=o_dtype)
    ref = U.ulysses_attn_bwd(tq, tk, tv, o, lse, tdo, tval, scale, causal)
    outs = [torch.full_like(r, float("nan")) for r in ref]        # every element must be written
    torch.cuda.synchronize()
    before = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
    got = U.ulysses_attn_bwd_noalloc(tq, tk, tv, o, lse, tdo, *outs, key_valid=tval, softmax_scale=scale,
                                     causal=causal)
    after = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
    torch.cuda.synchronize()
    assert after == before, "the no-allocation call allocated through torch"
    assert all(g is x for g, x in zip(got, outs))
    return [to_host_f64(r) for r in ref], [to_host_f64(g) for g in got]


def _same(ref, got, split):
    for name, r, g in zip(("dq", "dk", "dv"), ref, got):
        assert not np.any(np.isnan(g)), f"{name}: element not written"
        if name == "dq" or not split:
            assert np.array_equal(r, g), f"{name}: differs from the workspace call"
        else:
            tol = 1e-5 * max(1.0, float(np.abs(r).max()))
            assert float(np.abs(r - g).max()) <= tol, f"{name}: differs from the workspace call beyond {tol}"


def _splits(n, Hq, Hkv, D):
    """Whether the workspace call splits its key blocks: its workspace then
    holds more than the two row arrays."""
    return U.ulysses_attn_bwd_workspace_bytes(1, n, Hq, Hkv, D) > 2 * n * Hq * 4 + 512


def test_noalloc_equals_workspace_call_shrinking_sizes():
    """Two calls in a row, the second smaller (and of another head dim and O
    type), each bitwise equal to the workspace call and within 1e-2 of the
    oracle."""
    cases = [(3000, 8, 2, 128, True, True, torch.bfloat16), (700, 4, 1, 64, False, True, torch.float32),
             (300, 2, 2, 128, True, False, torch.bfloat16)]
    for i, (n, Hq, Hkv, D, masked, causal, o_dtype) in enumerate(cases):
        say(f"noalloc call {i}: n={n} Hq={Hq} Hkv={Hkv} D={D} masked={masked} causal={causal} o={o_dtype}")
        q, k, v, do, valid = _inputs(4040 + i, n, Hq, Hkv, D, masked)
        scale = D ** -0.5
        ref, got = _both(q, k, v, do, valid, scale, causal, o_dtype)
        _same(ref, got, _splits(n, Hq, Hkv, D))
        dQ, dK, dV, _, _ = oracle.attn_bwd(to_f64(q), to_f64(k), to_f64(v), to_f64(do), scale, causal, valid)
        assert_close("dQ", got[0], dQ, 1e-2)
        assert_close("dK", got[1], dK, 1e-2)
        assert_close("dV", got[2], dV, 1e-2)


def test_noalloc_at_the_limit_and_beyond():
    """B * Hq * n exactly at the scratch limit runs and matches; one more
    query head's rows is refused before any launch."""
    n, Hq, Hkv, D = 16384, 128, 32, 128
    assert n * Hq == LIMIT_ROWS
    say(f"noalloc at the limit: n={n} Hq={Hq} Hkv={Hkv}")
    q, k, v, do, _ = _inputs(4050, n, Hq, Hkv, D, False)
    ref, got = _both(q, k, v, do, None, D ** -0.5, True, torch.bfloat16)
    assert not _splits(n, Hq, Hkv, D)
    _same(ref, got, False)
    del ref, got
    say("noalloc beyond the limit")
    n2 = n + 64
    t = lambda *shape, dt=torch.bfloat16: torch.zeros(*shape, dtype=dt, device="cuda:0")
    args = (t(1, n2, Hq, D), t(1, n2, Hkv, D), t(1, n2, Hkv, D), t(1, n2, Hq, D), t(1, Hq, n2, dt=torch.float32),
            t(1, n2, Hq, D), t(1, n2, Hq, D, dt=torch.float32), t(1, n2, Hkv, D, dt=torch.float32),
            t(1, n2, Hkv, D, dt=torch.float32))
    with pytest.raises(ValueError, match="scratch"):
        U.ulysses_attn_bwd_noalloc(*args)
    torch.cuda.synchronize()
