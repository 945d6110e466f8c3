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


def assert_close(name: str, got: np.ndarray, ref: np.ndarray, tol: float, rel_bf16_storage: bool = False):
    """max |got - ref| <= tol (+ half an ulp of bfloat16 storage when asked)."""
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert not np.any(np.isnan(got)), f"{name}: NaN in output"
    both_inf = np.isinf(got) & np.isinf(ref) & (np.sign(got) == np.sign(ref))
    err = np.where(both_inf, 0.0, np.abs(got - ref))
    bound = tol + (2.0 ** -8) * np.abs(np.where(both_inf, 0.0, ref)) if rel_bf16_storage else tol
    worst = float(err.max()) if err.size else 0.0
    bad = err > bound
    tol_txt = f"{tol:g}" if np.ndim(tol) == 0 else f"1e-2 + bound (max {float(np.max(tol)):.3g})"
    say(f"  {name}: max_abs_err={worst:.3e} (tol {tol_txt}{' + bf16 ulp' if rel_bf16_storage else ''}), "
        f"max|ref|={float(np.abs(np.where(np.isfinite(ref), ref, 0)).max()) if ref.size else 0:.3f}")
    if np.any(bad):
        idx = np.unravel_index(int(np.argmax(np.where(bad, err, -1))), err.shape)
        lim = bound[idx] if np.ndim(bound) else bound
        raise AssertionError(f"{name}: error {float(err[idx]):.4e} > {float(lim):.4e} at {idx}: "
                             f"got {got[idx]!r} ref {ref[idx]!r}")
    return worst
