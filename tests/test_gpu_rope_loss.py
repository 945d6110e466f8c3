"""GPU parity of the first exchange fused with the rotary embedding at
global positions, and of the valid-token-weighted loss aggregation, against
the fp64 oracle.

Rotary tolerance (derived from the kernel's arithmetic): angles are exact to
double precision, their sine and cosine are rounded to float32, the rotation
x cos -/+ y sin is one float32 product and one fused multiply-add, and the
result is rounded once to the output type.  So
  |got - ref| <= u_out |ref| + 2^-21 (|x| + |y|)
with u_out the unit roundoff of the output type (2^-8 for bfloat16's 8-bit
significand, 2^-24 for float32), x and y the pair of inputs combined.  Loss: sums accumulate in double precision
(|error| <= per_rank 2^-53 sum|l|), counts exact, the loss one float32
rounding of the double quotient.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
import ulysses_sequence_parallelism_head_amd as U
from tests.gpu_helpers import say, bits_to_device, f32_to_device, to_f64, to_host_f64

pytestmark = pytest.mark.gpu


def _partner_mag(x):
    """|x| + |partner| per element (the pair the rotation combines)."""
    h = x.shape[-1] // 2
    a = np.abs(x)
    return a + np.concatenate([a[..., h:], a[..., :h]], axis=-1)


def _check_rope(got, ref, x_pair, dtype):
    u = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -24
    bound = u * np.abs(ref) + 2.0 ** -21 * x_pair + 1e-30
    err = np.abs(got - ref)
    worst = float(np.max(err / bound)) if err.size else 0.0
    say(f"  rope: max_abs_err={float(err.max()):.3e}, worst err/bound={worst:.3f}")
    assert not np.any(np.isnan(got))
    assert np.all(err <= bound), f"error/bound {worst}"


CASES = [
    # P, B, n_local, H, D, dtype, base, scale
    (1, 1, 1, 1, 64, "bf16", 1e4, 1.0),
    (2, 1, 3, 4, 64, "bf16", 1e4, 1.0),
    (4, 2, 37, 8, 128, "bf16", 1e6, 1.0),
    (4, 1, 100, 32, 128, "bf16", 1e6, 4.0),
    (2, 1, 64, 2, 128, "bf16", 1e4, 1.0),      # H/P = 1
    (4, 1, 50, 4, 64, "f32", 1e4, 1.0),        # H/P = 1, fp32
    (2, 2, 33, 8, 128, "f32", 1e6, 2.0),
]


@pytest.mark.parametrize("P,B,nl,H,D,dtype,base,scale", CASES)
def test_seq2head_rope(P, B, nl, H, D, dtype, base, scale):
    say(f"rope P={P} B={B} nl={nl} H={H} D={D} {dtype} base={base} scale={scale}")
    g = synth.streams(100 + nl)
    shape = (P, B, nl, H, D)
    if dtype == "bf16":
        x = synth.normal_bf16(g[0], shape)
        tx = bits_to_device(x)
    else:
        x = g[0].standard_normal(shape, dtype=np.float32)
        tx = f32_to_device(x)
    out = U.ulysses_repack_seq2head_rope(tx, base, scale)
    torch.cuda.synchronize()
    xf = to_f64(x)
    ref = oracle.rope.seq2head_rope(xf, base, scale)
    pair = oracle.seq2head(_partner_mag(xf))
    _check_rope(to_host_f64(out), ref, pair, dtype)


def test_seq2head_rope_64k_sampled():
    """The 64K workload's global Q ([4][1][16384][32][128] bf16), rotated at
    positions up to 65535 with base 1e6: every output element of sampled
    tokens (shard edges and the last position included)."""
    say("rope 64K Q, sampled tokens")
    w = synth.WORKLOADS[3]
    P, nl = w.P, w.n_local
    g = synth.streams(w.number)
    x = synth.normal_bf16(g[synth.STREAM_Q], (P, 1, nl, w.Hq_global, w.D))
    out = U.ulysses_repack_seq2head_rope(bits_to_device(x), 1e6, 1.0)
    torch.cuda.synchronize()
    got = to_host_f64(out)                                   # [P][1][n][H/P][D]
    rows = synth.sample_rows(g[synth.STREAM_ROWS], w.n, 48, extra=(0, 1, nl - 1, nl, 2 * nl, w.n - 1))
    i, s = rows // nl, rows % nl
    xs = to_f64(x[i, 0, s])                                  # [R][H][D]
    ref = oracle.rope.rope(xs, rows, 1e6)                    # rotated at global positions
    hp = w.Hq_global // P
    ref_h = ref.reshape(len(rows), P, hp, w.D).transpose(1, 0, 2, 3)      # [P][R][H/P][D]
    pair = _partner_mag(xs).reshape(len(rows), P, hp, w.D).transpose(1, 0, 2, 3)
    _check_rope(got[:, 0, rows], ref_h, pair, "bf16")


@pytest.mark.parametrize("P,per_rank,masked", [(1, 1, False), (4, 24576, True), (3, 1000, True), (8, 7, False)])
def test_loss_aggregate(P, per_rank, masked):
    say(f"loss P={P} per_rank={per_rank} masked={masked}")
    g = synth.streams(200 + per_rank)
    tl = np.abs(g[0].standard_normal((P, per_rank), dtype=np.float32)) * 3.0
    va = None
    if masked:
        va = (g[1].random((P, per_rank)) > 0.25).astype(np.uint8)
        va[0, :] = 0                                     # an empty rank
    sums, counts, loss = U.ulysses_loss_aggregate(f32_to_device(tl), None if va is None else
                                                  torch.from_numpy(va).to("cuda:0"))
    torch.cuda.synchronize()
    rs, rc, rl = oracle.loss.aggregate(tl.astype(np.float64), va)
    gs, gc, gl = sums.cpu().numpy(), counts.cpu().numpy(), float(loss.cpu().numpy()[0])
    assert np.array_equal(gc, rc)
    bound = per_rank * 2.0 ** -52 * np.sum(np.abs(tl), axis=1) + 1e-300
    assert np.all(np.abs(gs - rs) <= bound), (gs, rs)
    if math.isnan(rl):
        assert math.isnan(gl)
    else:
        assert abs(gl - rl) <= 2.0 ** -24 * abs(rl) + 1e-12 * abs(rl)
    say(f"  loss={gl!r} oracle={rl!r}")


def test_loss_nothing_valid():
    tl = torch.ones((2, 5), dtype=torch.float32, device="cuda:0")
    va = torch.zeros((2, 5), dtype=torch.uint8, device="cuda:0")
    s, c, l = U.ulysses_loss_aggregate(tl, va)
    torch.cuda.synchronize()
    assert np.all(s.cpu().numpy() == 0) and np.all(c.cpu().numpy() == 0) and math.isnan(float(l.cpu()[0]))
