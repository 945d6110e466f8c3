"""Shared pytest set-up: the ``gpu`` marker, the repo root on sys.path, and a
loader for the hand-derived fixtures under ``tests/golden/``."""
import math
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def load_golden(name):
    """Parse ``name = expression`` lines (only the math module is visible)."""
    env = {"math": math, "__builtins__": {}}
    out = {}
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, expr = line.split("=", 1)
            out[key.strip()] = eval(expr, env)  # noqa: S307 - fixed local fixture, math only
    return out


@pytest.fixture
def golden():
    return load_golden
