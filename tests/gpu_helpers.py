"""Helpers shared by the GPU parity tests: device transfer of seeded inputs
and the tolerance checks.  Everything here is host-side marshalling and
comparison; no step of the computation under test lives here."""
from __future__ import annotations

import sys

import numpy as np
import torch

import synth


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bits_to_device(bits: np.ndarray) -> torch.Tensor:
    """uint16 bfloat16 bit patterns -> torch.bfloat16 tensor on cuda:0."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to("cuda:0")


def f32_to_device(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda:0")


def to_f64(bits_or_f32: np.ndarray) -> np.ndarray:
    if bits_or_f32.dtype == np.uint16:
        return synth.bf16_bits_to_f64(bits_or_f32)
    return bits_or_f32.astype(np.float64)


def device_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def to_host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def max_abs(a: np.ndarray, b: np.ndarray) -> float:
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    d = np.where(both_inf, 0.0, np.abs(a - b))
    return float(np.nanmax(d)) if d.size else 0.0


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half a bfloat16 ulp at |x| (8 significant bits): the largest error of
    rounding x to bfloat16 storage (normal range)."""
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - 8.0), 0.0)


def assert_close(name: str, got: np.ndarray, ref: np.ndarray, tol: float, bf16_out: bool = False):
    """max |got - ref| <= tol.

    ``bf16_out``: ``got`` was stored in bfloat16.  Below |ref| = 4 the
    storage rounding is at most 2^-7, inside the 1e-2 bound, and the bound
    stays tol.  At |ref| >= 4 the half-ulp of storage alone exceeds it; such
    elements get their own half-ulp plus the same compute margin
    (tol - 2^-7)."""
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert not np.any(np.isnan(got)), f"{name}: NaN in output"
    both_inf = np.isinf(got) & np.isinf(ref) & (np.sign(got) == np.sign(ref))
    with np.errstate(invalid="ignore"):
        err = np.where(both_inf, 0.0, np.abs(got - ref))
    fin = np.where(np.isfinite(ref), ref, 0.0)
    bound = np.maximum(tol, bf16_half_ulp(fin) + (tol - 2.0 ** -7)) if bf16_out else tol
    worst = float(err.max()) if err.size else 0.0
    bad = err > bound
    maxref = float(np.abs(fin).max()) if ref.size else 0.0
    wide = int(np.count_nonzero(np.abs(fin) >= 4.0)) if bf16_out else 0
    say(f"  {name}: max_abs_err={worst:.3e} (tol {tol:g}{', bf16 output' if bf16_out else ''}"
        f"{f', {wide} elements with |ref| >= 4' if wide else ''}), max|ref|={maxref:.3f}")
    if np.any(bad):
        idx = np.unravel_index(int(np.argmax(np.where(bad, err, -1))), err.shape)
        lim = bound[idx] if np.ndim(bound) else bound
        raise AssertionError(f"{name}: error {float(err[idx]):.4e} > {float(lim):.4e} at {idx}: "
                             f"got {got[idx]!r} ref {ref[idx]!r}")
    return worst


def load_sampled_golden(stem: str, d: dict) -> dict:
    """Expected values at sampled rows of a full-size workload, written by
    ``tests/golden/make_sampled_goldens.py`` from the oracle alone; checks
    that ``d`` (the regenerated inputs) are the inputs they were made from."""
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", f"bwd_{stem}_sampled.npz")
    with np.load(path, allow_pickle=False) as z:
        g = {k: z[k] for k in z.files}
    check = np.stack([d[x].reshape(-1)[:8].astype(np.uint16) for x in ("q", "k", "v", "do")])
    assert np.array_equal(check, g["seed_check"]), "inputs differ from the ones the golden file was made from"
    for k in ("O", "LSE", "dQ", "dK", "dV"):
        g[k] = g[k].astype(np.float64)
    return g
