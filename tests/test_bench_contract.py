"""Host-side checks of bench.py's command-line contract (no GPU needed).

The measurement runs on one GPU: asking for more exits with a message and
a non-zero status before anything touches a device, and the multi-GB
measured-traffic table only reports bytes for the kernel sources it was
taken on.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          cwd=ROOT, env=env, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2")
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="4", RANK="0", LOCAL_RANK="0")
    r = _bench(env=env)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_measured_traffic_tracks_sources():
    """An entry is reported only while its hash matches the current kernel
    sources, and a changed source turns it into null."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    for (call, workload), m in b.MEASURED_TRAFFIC.items():
        same = b.sources_sha256(m["sources"]) == m["sha256"]
        assert b.measured_traffic(call, workload) == (m["bytes"] if same else None), (call, workload)
    real = b.sources_sha256
    try:
        b.sources_sha256 = lambda names: "0" * 64
        for call, workload in b.MEASURED_TRAFFIC:
            assert b.measured_traffic(call, workload) is None
    finally:
        b.sources_sha256 = real
