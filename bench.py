"""Benchmark of the single-GPU Ulysses sequence-parallel hot path on MI355X.

One step = one pass of the whole hot path over one batch of synthetic input,
at the 64K workload (global Q [4][1][16384][32][128], K/V [4][1][16384][8][128]
bf16; one GPU's P=4 share = 8 query heads and 2 KV heads over n = 65536):

  seq2head(Q, K, V)          the first all-to-all, emulated (full 4-shard tensors)
  attn_fwd  (rank 0 share)   O (bf16), LSE
  seq2head(dO)               the backward's first exchange
  attn_bwd  (rank 0 share)   dQ, dK, dV (fp32)
  head2seq(O)                the second all-to-all (bf16)
  head2seq(dQ, dK, dV)       the backward's second exchange (fp32)

Inputs are resident in HBM before timing starts.  ``value`` is the step's
algorithmic attention work (4*D flops per visible (query, key) pair per query
head for the forward, 10*D for the backward) divided by the measured step
time.  Per-call durations come from HIP events recorded on the stream the
library launches on (torch's current stream).

With ``--workload 4`` the step runs the 96K documents workload (n = 98304,
padding keys masked); adding ``--docs`` also applies the document mask (a
token sees only earlier tokens of its own document, the ``*_docs`` calls),
so the work is the tokens' own documents' pairs.  The flop count is always
that of the visible (query, key) pairs, counted exactly from the masks.
``--rope-loss`` runs the step as a model would around the path: Q and K go
through the first exchange fused with the rotary embedding at global
positions (base 1e6), V through the plain one, and the step ends with the
valid-token-weighted loss aggregation over the P shards' token losses.
``--ring`` times the ring-attention alternative instead (forward only): each
of the P emulated ranks keeps all heads of its query shard and merges the
key/value shards of its hops with ``ulysses_attn_fwd_block``; the same
attention is timed the Ulysses way (P head-shard forwards over the whole
sequence) beside it.
``--proj`` times the projections fused with the exchanges (QKV projection
writing the head-sharded layout, output projection reading it) at the
workload's model width (hidden = Hq * D), beside the same work done unfused
with torch's library GEMM followed by the plain exchange.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload C] [--docs] [--no-cpu-baseline]
Prints ONE JSON line on stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2516.6     # 256 CU x 4096 flop/clk x 2.4 GHz (dense)
HBM_PEAK_GBS = 8000.0

# HBM bytes per launch of each attention call at this workload, from rocprofv3
# FETCH_SIZE and WRITE_SIZE passes (scaled by a 512 MiB copy calibration; the
# summary is under profiles/), valid only for the kernel sources they were
# measured on: the roofline reports null traffic once those sources change.
CSRC = os.path.join(ROOT, "ulysses_sequence_parallelism_head_amd", "csrc")
MEASURED_TRAFFIC = {      # keyed by (call, workload as named in the config)
    ("attn_bwd", "gqa-n65536-8q2kv-d128-bf16-fwd+repack"): {
        "bytes": 5.231e+09, "sources": ("attn_bwd.hip", "device_common.h", "internal.h", "workspace.hip"),
        "sha256": "70924eedd331bdd8f91830bbfba059251ff8082b6b038c7dc1f852a84d33928e"},
    ("attn_fwd", "gqa-n65536-8q2kv-d128-bf16-fwd+repack"): {
        "bytes": 1.798e+09, "sources": ("attn_fwd.hip", "device_common.h", "internal.h"),
        "sha256": "36183a88ad6bfe6cbdc7db29facb30f2667362b40fc06870e057e6f7c34e14ef"},
    ("attn_bwd", "gqa-n98304-8q2kv-d128-bf16-docs-fwd+bwd+document-mask"): {
        "bytes": 6.934e+09, "sources": ("attn_bwd.hip", "device_common.h", "internal.h", "workspace.hip"),
        "sha256": "70924eedd331bdd8f91830bbfba059251ff8082b6b038c7dc1f852a84d33928e"},
    ("attn_fwd", "gqa-n98304-8q2kv-d128-bf16-docs-fwd+bwd+document-mask"): {
        "bytes": 1.562e+09, "sources": ("attn_fwd.hip", "device_common.h", "internal.h"),
        "sha256": "36183a88ad6bfe6cbdc7db29facb30f2667362b40fc06870e057e6f7c34e14ef"},
}


def sources_sha256(names) -> str:
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(call: str, workload: str):
    m = MEASURED_TRAFFIC.get((call, workload))
    if m is None or sources_sha256(m["sources"]) != m["sha256"]:
        return None
    return m["bytes"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def visible_keys(n: int, valid=None, doc_start=None) -> np.ndarray:
    """Per query row, the number of keys it sees: u <= t, valid[u], and
    u >= doc_start[t] when documents are given."""
    cv = np.zeros(n + 1, dtype=np.int64)
    cv[1:] = np.cumsum(np.ones(n, np.int64) if valid is None else (np.asarray(valid).reshape(n) != 0))
    lo = np.zeros(n, np.int64) if doc_start is None else np.asarray(doc_start, np.int64).reshape(n)
    return cv[1:] - cv[lo]


def cpu_baseline(workload, docs: bool, budget_s: float = 12.0):
    """The oracle (as it stands) on a bounded sample of the same workload:
    full causal forward rows at seeded positions, timed on the host cores."""
    import oracle
    import synth
    d = synth.local_attention_inputs(workload)
    w = d["workload"]
    q = synth.bf16_bits_to_f64(d["q"])
    k = synth.bf16_bits_to_f64(d["k"])
    v = synth.bf16_bits_to_f64(d["v"])
    valid = d["valid"]
    ds = d.get("doc_start") if docs else None
    seen = visible_keys(w.n, None if valid is None else valid[0], None if ds is None else ds[0])
    gen = np.random.Generator(np.random.PCG64(12345))
    workers = host_cores()
    done_rows, flops, spent = 0, 0.0, 0.0
    batch = 64
    while spent < budget_s:
        rows = np.sort(gen.choice(w.n, size=batch, replace=False))
        t0 = time.perf_counter()
        oracle.attn_fwd(q, k, v, w.scale, True, valid, rows=rows, block=16, workers=workers, doc_start=ds)
        spent += time.perf_counter() - t0
        flops += float(4 * w.D * w.hq * np.sum(seen[rows]))
        done_rows += batch
    kind = "document-masked causal" if docs else "causal"
    return {"value": flops / spent / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{done_rows} seeded query rows x {w.hq} heads of the n={w.n} {kind} forward "
                      f"(fp64 NumPy, {workers} worker threads with one BLAS thread each, {spent:.1f} s)"}


def host_cores() -> int:
    """Cores this process may run on (its affinity set)."""
    try:
        return len(os.sched_getaffinity(0))
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def measure_sclk(U, torch, fn, call_ms: float, window_ms: float = 40.0):
    """Median engine clock (MHz) while `fn` (one launch of a kernel) runs back
    to back for about window_ms, sampled by the library's clock probe on a
    second stream (default priority).  None if the probe reads nothing."""
    reps = max(2, int(np.ceil((window_ms + 10.0) / max(call_ms, 1e-3))))
    samples, interval_us = 20, int(window_ms * 1000 / 20)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        out, khz = U.ulysses_clock_probe(samples, interval_us, stream=side)
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    mhz = U.clock_probe_mhz(out, khz)[2:]        # the first intervals may precede the kernels
    return float(np.median(mhz)) if mhz else None


def bench_ring(args, w):
    """Ring attention (forward) on P emulated ranks against Ulysses' forward
    of the same attention; one JSON line."""
    import torch
    import synth
    import ulysses_sequence_parallelism_head_amd as U
    dev = torch.device("cuda:0")
    P, nl, n, D = w.P, w.n_local, w.n, w.D
    g = synth.streams(w.number)

    def dev_bits(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    log(f"[bench] ring emulation, workload {w.name}")
    q_seq = dev_bits(synth.normal_bf16(g[synth.STREAM_Q], (P, 1, nl, w.Hq_global, D)))
    k_seq = dev_bits(synth.normal_bf16(g[synth.STREAM_K], (P, 1, nl, w.Hkv_global, D)))
    v_seq = dev_bits(synth.normal_bf16(g[synth.STREAM_V], (P, 1, nl, w.Hkv_global, D)))
    o_ring = torch.empty((P, 1, nl, w.Hq_global, D), dtype=torch.float32, device=dev)
    l_ring = torch.empty((P, 1, w.Hq_global, nl), dtype=torch.float32, device=dev)
    q_h = U.ulysses_repack_seq2head(q_seq)
    k_h = U.ulysses_repack_seq2head(k_seq)
    v_h = U.ulysses_repack_seq2head(v_seq)
    o_uly = torch.empty((P, 1, n, w.hq, D), dtype=torch.float32, device=dev)
    l_uly = torch.empty((P, 1, w.hq, n), dtype=torch.float32, device=dev)
    hops = [(i, j) for i in range(P) for j in ((i - h) % P for h in range(P)) if j <= i]

    def ring():
        for i, j in hops:
            U.ulysses_attn_fwd_block(q_seq[i], k_seq[j], v_seq[j], o_ring[i], l_ring[i], (i - j) * nl, None,
                                     w.scale, True, accumulate=j != i)

    def ulysses():
        for j in range(P):
            U.ulysses_attn_fwd(q_h[j], k_h[j], v_h[j], None, w.scale, True, o_dtype=torch.float32,
                               out=o_uly[j], lse=l_uly[j])

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        t0 = time.perf_counter()
        e[0].record()
        for s_ in range(args.steps):
            fn()
            e[s_ + 1].record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / args.steps
        return wall * 1e3, [e[s_].elapsed_time(e[s_ + 1]) for s_ in range(args.steps)]

    ms_ring, per_ring = timed(ring)
    ms_uly, _ = timed(ulysses)
    flops = 4.0 * D * w.Hq_global * float(visible_keys(n).sum())
    ring_tf = flops / (np.mean(per_ring) * 1e-3) / 1e12
    result = {
        "metric": f"ring-attention emulation: causal attn fwd TFLOP/s @{n // 1024}K, {w.Hq_global}q/{w.Hkv_global}kv "
                  f"heads d{D} bf16 on P={P} ranks",
        "value": round(flops / (ms_ring * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_ring, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name + "+ring", "n": n, "P": P, "q_heads": w.Hq_global, "kv_heads": w.Hkv_global,
                   "head_dim": D, "hops_launched": len(hops), "causal": True},
        "ring_fwd_ms": round(ms_ring, 3),
        "ulysses_fwd_all_ranks_ms": round(ms_uly, 3),
        "ring_over_ulysses_time": round(ms_ring / ms_uly, 4),
        "roofline": {"bound": "mfma", "kernel": "attn_fwd_block (all hops of all ranks)", "achieved": round(ring_tf, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(ring_tf / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None},
    }
    print(json.dumps(result), flush=True)


def bench_proj(args, w):
    """QKV projection + first exchange and second exchange + output
    projection, fused, against library GEMM + plain exchange; one JSON line."""
    import torch
    import synth
    import ulysses_sequence_parallelism_head_amd as U
    dev = torch.device("cuda:0")
    P, nl, n, D = w.P, w.n_local, w.n, w.D
    Hq, Hkv = w.Hq_global, w.Hkv_global
    hidden = Hq * D
    g = synth.streams(w.number)

    def dev_bits(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    def weights(gen, rows, cols):
        return dev_bits(synth.f32_to_bf16_bits(gen.standard_normal((rows, cols), dtype=np.float32)
                                               / np.float32(np.sqrt(cols))))

    log(f"[bench] projections, workload {w.name}, hidden {hidden}")
    x = dev_bits(synth.normal_bf16(g[synth.STREAM_Q], (P, 1, nl, hidden)))
    w_qkv = weights(g[synth.STREAM_K], (Hq + 2 * Hkv) * D, hidden)
    w_o = weights(g[synth.STREAM_V], hidden, Hq * D)
    q_h = torch.empty((P, 1, n, Hq // P, D), dtype=torch.bfloat16, device=dev)
    k_h = torch.empty((P, 1, n, Hkv // P, D), dtype=torch.bfloat16, device=dev)
    v_h = torch.empty_like(k_h)
    y = torch.empty((P, 1, nl, hidden), dtype=torch.bfloat16, device=dev)
    # unfused reference path: library GEMM, then the plain exchange
    o_seq = torch.empty((P, 1, nl, Hq, D), dtype=torch.bfloat16, device=dev)

    def fused_qkv():
        U.ulysses_qkv_proj_seq2head(x, w_qkv, Hq, Hkv, D, q_h, k_h, v_h)

    def fused_out():
        U.ulysses_head2seq_out_proj(q_h, w_o, y)

    yq = torch.empty((P, 1, nl, Hq, D), dtype=torch.bfloat16, device=dev)
    yk = torch.empty((P, 1, nl, Hkv, D), dtype=torch.bfloat16, device=dev)
    yv = torch.empty_like(yk)

    def unfused_qkv():
        # library GEMMs into separate Q, K, V buffers, then the plain exchange of each
        xf = x.view(-1, hidden)
        torch.matmul(xf, w_qkv[:Hq * D].t(), out=yq.view(-1, Hq * D))
        torch.matmul(xf, w_qkv[Hq * D:(Hq + Hkv) * D].t(), out=yk.view(-1, Hkv * D))
        torch.matmul(xf, w_qkv[(Hq + Hkv) * D:].t(), out=yv.view(-1, Hkv * D))
        U.ulysses_repack_seq2head(yq, q_h)
        U.ulysses_repack_seq2head(yk, k_h)
        U.ulysses_repack_seq2head(yv, v_h)

    def unfused_out():
        U.ulysses_repack_head2seq(q_h, o_seq)
        torch.matmul(o_seq.view(-1, Hq * D), w_o.t(), out=y.view(-1, hidden))

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms_qkv, ms_out = timed(fused_qkv), timed(fused_out)
    ms_uq, ms_uo = timed(unfused_qkv), timed(unfused_out)
    tokens = P * nl
    f_qkv = 2.0 * tokens * hidden * (Hq + 2 * Hkv) * D
    f_out = 2.0 * tokens * Hq * D * hidden
    tf_qkv = f_qkv / (ms_qkv * 1e-3) / 1e12
    tf_out = f_out / (ms_out * 1e-3) / 1e12
    result = {
        "metric": f"projections fused with the exchanges TFLOP/s @{n // 1024}K, hidden {hidden}, {Hq}q/{Hkv}kv heads "
                  f"d{D} bf16, P={P}",
        "value": round((f_qkv + f_out) / ((ms_qkv + ms_out) * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_qkv + ms_out, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name + "+projections", "n": n, "P": P, "hidden": hidden, "q_heads": Hq,
                   "kv_heads": Hkv, "head_dim": D},
        "qkv_proj_seq2head_ms": round(ms_qkv, 4),
        "qkv_proj_seq2head_tflops": round(tf_qkv, 2),
        "head2seq_out_proj_ms": round(ms_out, 4),
        "head2seq_out_proj_tflops": round(tf_out, 2),
        "unfused_library_gemm_then_exchange_ms": {"qkv": round(ms_uq, 4), "out": round(ms_uo, 4)},
        "roofline": {"bound": "mfma", "kernel": "proj_kernel (QKV)", "achieved": round(tf_qkv, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tf_qkv / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None},
    }
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--rope-loss", action="store_true",
                    help="fuse the rotary embedding into Q/K's first exchange and aggregate the loss")
    ap.add_argument("--ring", action="store_true", help="time the ring-attention emulation (forward)")
    ap.add_argument("--proj", action="store_true", help="time the projections fused with the exchanges")
    ap.add_argument("--docs", action="store_true",
                    help="document-masked attention (workloads with packed documents only)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time only a plain 512 MiB device-to-device copy (torch copy_), the reference kernel "
                         "for scaling the FETCH_SIZE / WRITE_SIZE hardware counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the Ulysses hot path; the all-to-all is emulated on a "
              "single device, so only --gpus 1 is supported.", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import ulysses_sequence_parallelism_head_amd as U

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    U.load_library()
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.int16, device=dev).fill_(1)     # 512 MiB
        dst = torch.empty_like(src)
        for _ in range(args.warmup):
            dst.copy_(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / args.steps
        print(json.dumps({"copy_bytes_read": src.numel() * 2, "copy_bytes_written": src.numel() * 2,
                          "ms": dt * 1e3, "GBs": 2 * src.numel() * 2 / dt / 1e9}), flush=True)
        return
    w = synth.WORKLOADS[args.workload]
    P, nl, n, D = w.P, w.n_local, w.n, w.D
    hq, hkv = w.hq, w.hkv
    if args.docs and not w.docs:
        print(f"--docs needs a workload with packed documents (workload {w.number} has none)", file=sys.stderr)
        sys.exit(2)

    if args.ring:
        bench_ring(args, w)
        return
    if args.proj:
        bench_proj(args, w)
        return
    log(f"[bench] generating workload {w.name}")
    g = synth.streams(w.number)

    def dev_bits(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    big = P * nl * w.Hq_global * D > (1 << 30)
    if big:
        # tensors of several GB (the 1M-token workload's 32 shards): drawn on the device from a
        # seeded generator (same shapes and N(0,1) bf16 values; host generation would take minutes)
        gen = torch.Generator(device=dev)
        gen.manual_seed(w.number)

        def draw(shape):
            return torch.randn(shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)

        q_seq = draw((P, 1, nl, w.Hq_global, D))
        k_seq = draw((P, 1, nl, w.Hkv_global, D))
        v_seq = draw((P, 1, nl, w.Hkv_global, D))
        do_seq = draw((P, 1, nl, w.Hq_global, D))
    else:
        q_seq = dev_bits(synth.normal_bf16(g[synth.STREAM_Q], (P, 1, nl, w.Hq_global, D)))
        k_seq = dev_bits(synth.normal_bf16(g[synth.STREAM_K], (P, 1, nl, w.Hkv_global, D)))
        v_seq = dev_bits(synth.normal_bf16(g[synth.STREAM_V], (P, 1, nl, w.Hkv_global, D)))
        do_seq = dev_bits(synth.normal_bf16(g[synth.STREAM_DO], (P, 1, nl, w.Hq_global, D)))
    # packed documents (global positions, the same on every rank after the exchange)
    valid_np = ds_np = valid_t = ds_t = None
    if w.docs:
        valid_np, ds_np, _ = synth.documents(g[synth.STREAM_DOCS], n, P, min(synth.DOC_MAX_LEN, n))
        valid_t = torch.from_numpy(valid_np.reshape(1, n)).to(dev)
        if args.docs:
            ds_t = torch.from_numpy(ds_np.reshape(1, n)).to(dev)

    # buffers (allocated once; the library allocates nothing)
    bf, f32 = torch.bfloat16, torch.float32
    q_h = torch.empty((P, 1, n, hq, D), dtype=bf, device=dev)
    k_h = torch.empty((P, 1, n, hkv, D), dtype=bf, device=dev)
    v_h = torch.empty((P, 1, n, hkv, D), dtype=bf, device=dev)
    do_h = torch.empty((P, 1, n, hq, D), dtype=bf, device=dev)
    o_h = torch.zeros((P, 1, n, hq, D), dtype=bf, device=dev)       # rank 0's slot written by attn_fwd
    lse = torch.empty((1, hq, n), dtype=f32, device=dev)
    dq_h = torch.zeros((P, 1, n, hq, D), dtype=f32, device=dev)
    dk_h = torch.zeros((P, 1, n, hkv, D), dtype=f32, device=dev)
    dv_h = torch.zeros((P, 1, n, hkv, D), dtype=f32, device=dev)
    o_seq = torch.empty((P, 1, nl, w.Hq_global, D), dtype=bf, device=dev)
    dq_seq = torch.empty((P, 1, nl, w.Hq_global, D), dtype=f32, device=dev)
    dk_seq = torch.empty((P, 1, nl, w.Hkv_global, D), dtype=f32, device=dev)
    dv_seq = torch.empty((P, 1, nl, w.Hkv_global, D), dtype=f32, device=dev)
    ws = torch.empty(max(256, U.ulysses_attn_bwd_workspace_bytes(1, n, hq, hkv, D)), dtype=torch.uint8, device=dev)
    rope_base = 1e6
    if args.rope_loss:
        # per-token losses of each rank's shard; counted where the key is valid
        tok_loss = torch.from_numpy(np.abs(g[synth.STREAM_BITS].standard_normal((P, nl), dtype=np.float32))).to(dev)
        tok_valid = None if valid_np is None else torch.from_numpy(valid_np.reshape(P, nl)).to(dev)
        l_sum = torch.empty(P, dtype=torch.float64, device=dev)
        l_cnt = torch.empty(P, dtype=torch.int64, device=dev)
        l_val = torch.empty(1, dtype=torch.float32, device=dev)

    names = ["seq2head_qkv", "attn_fwd", "seq2head_do", "attn_bwd", "head2seq_o", "head2seq_dqkv"]
    if args.rope_loss:
        names.append("loss_aggregate")
    Ev = torch.cuda.Event

    def step(events=None):
        def mark(i):
            if events is not None:
                events[i].record()
        mark(0)
        if args.rope_loss:
            U.ulysses_repack_seq2head_rope(q_seq, rope_base, out=q_h)
            U.ulysses_repack_seq2head_rope(k_seq, rope_base, out=k_h)
        else:
            U.ulysses_repack_seq2head(q_seq, q_h)
            U.ulysses_repack_seq2head(k_seq, k_h)
        U.ulysses_repack_seq2head(v_seq, v_h)
        mark(1)
        if ds_t is None:
            U.ulysses_attn_fwd(q_h[0], k_h[0], v_h[0], valid_t, w.scale, True, out=o_h[0], lse=lse)
        else:
            U.ulysses_attn_fwd_docs(q_h[0], k_h[0], v_h[0], ds_t, valid_t, w.scale, out=o_h[0], lse=lse)
        mark(2)
        U.ulysses_repack_seq2head(do_seq, do_h)
        mark(3)
        if ds_t is None:
            U.ulysses_attn_bwd(q_h[0], k_h[0], v_h[0], o_h[0], lse, do_h[0], valid_t, w.scale, True,
                               dq=dq_h[0], dk=dk_h[0], dv=dv_h[0], workspace=ws)
        else:
            U.ulysses_attn_bwd_docs(q_h[0], k_h[0], v_h[0], o_h[0], lse, do_h[0], ds_t, valid_t, w.scale,
                                    dq=dq_h[0], dk=dk_h[0], dv=dv_h[0], workspace=ws)
        mark(4)
        U.ulysses_repack_head2seq(o_h, o_seq)
        mark(5)
        U.ulysses_repack_head2seq(dq_h, dq_seq)
        U.ulysses_repack_head2seq(dk_h, dk_seq)
        U.ulysses_repack_head2seq(dv_h, dv_seq)
        mark(6)
        if args.rope_loss:
            U.ulysses_loss_aggregate(tok_loss, tok_valid, l_sum, l_cnt, l_val)
            mark(7)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    log(f"[bench] timing {args.steps} steps")
    per = {k: [] for k in names}
    nev = len(names) + 1
    evs = [[Ev(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = []
    for s in range(args.steps):
        e = evs[s]
        for i, k in enumerate(names):
            per[k].append(e[i].elapsed_time(e[i + 1]))
        step_ms.append(e[0].elapsed_time(e[nev - 1]))
    ms_step = wall * 1e3 / args.steps
    avg = {k: float(np.mean(v)) for k, v in per.items()}
    med = {k: float(np.median(v)) for k, v in per.items()}
    mins = {k: float(np.min(v)) for k, v in per.items()}

    # engine clock under each attention call (outside the timed steps)
    log("[bench] engine clock under the attention calls")

    def fwd_call():
        if ds_t is None:
            U.ulysses_attn_fwd(q_h[0], k_h[0], v_h[0], valid_t, w.scale, True, out=o_h[0], lse=lse)
        else:
            U.ulysses_attn_fwd_docs(q_h[0], k_h[0], v_h[0], ds_t, valid_t, w.scale, out=o_h[0], lse=lse)

    def bwd_call():
        if ds_t is None:
            U.ulysses_attn_bwd(q_h[0], k_h[0], v_h[0], o_h[0], lse, do_h[0], valid_t, w.scale, True,
                               dq=dq_h[0], dk=dk_h[0], dv=dv_h[0], workspace=ws)
        else:
            U.ulysses_attn_bwd_docs(q_h[0], k_h[0], v_h[0], o_h[0], lse, do_h[0], ds_t, valid_t, w.scale,
                                    dq=dq_h[0], dk=dk_h[0], dv=dv_h[0], workspace=ws)

    sclk = {"attn_fwd": measure_sclk(U, torch, fwd_call, avg["attn_fwd"]),
            "attn_bwd": measure_sclk(U, torch, bwd_call, avg["attn_bwd"])}

    # reference for the repacks, outside the timed steps: a plain 512 MiB device-to-device
    # copy on the same stream (HIP events, median of 5)
    csrc = torch.empty(1 << 28, dtype=torch.int16, device=dev).fill_(1)
    cdst = torch.empty_like(csrc)
    cdst.copy_(csrc)
    cms = []
    for _ in range(5):
        c0, c1 = Ev(enable_timing=True), Ev(enable_timing=True)
        c0.record()
        cdst.copy_(csrc)
        c1.record()
        torch.cuda.synchronize()
        cms.append(c0.elapsed_time(c1))
    copy_gbs = 2 * csrc.numel() * 2 / (float(np.median(cms)) * 1e-3) / 1e9
    del csrc, cdst

    pairs = int(visible_keys(n, valid_np, ds_np if args.docs else None).sum())
    fwd_flops = 4.0 * D * hq * pairs
    bwd_flops = 10.0 * D * hq * pairs
    bf2, f4 = 2, 4
    bytes_qkv = 2 * bf2 * P * nl * (w.Hq_global + 2 * w.Hkv_global) * D       # read + write
    bytes_do = 2 * bf2 * P * nl * w.Hq_global * D
    bytes_o = bytes_do
    bytes_dqkv = 2 * f4 * P * nl * (w.Hq_global + 2 * w.Hkv_global) * D
    fwd_tf = fwd_flops / (avg["attn_fwd"] * 1e-3) / 1e12
    bwd_tf = bwd_flops / (avg["attn_bwd"] * 1e-3) / 1e12
    rep = {
        "seq2head_qkv_GBs": bytes_qkv / (avg["seq2head_qkv"] * 1e-3) / 1e9,
        "seq2head_do_GBs": bytes_do / (avg["seq2head_do"] * 1e-3) / 1e9,
        "head2seq_o_GBs": bytes_o / (avg["head2seq_o"] * 1e-3) / 1e9,
        "head2seq_dqkv_GBs": bytes_dqkv / (avg["head2seq_dqkv"] * 1e-3) / 1e9,
    }
    value = (fwd_flops + bwd_flops) / (ms_step * 1e-3) / 1e12

    # roofline of each attention call: algorithmic flops over the average
    # launch duration; also against the peak at the engine clock measured
    # under that call (the peak scales with the clock; 2.4 GHz is its maximum)
    def roof(call, flops):
        achieved = flops / (avg[call] * 1e-3) / 1e12
        r = {"bound": "mfma", "kernel": call, "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
             "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
             "traffic": measured_traffic(call, w.name + ("+document-mask" if args.docs else ""))}
        if sclk[call]:
            peak_at = MFMA_BF16_PEAK_TFLOPS * sclk[call] / 2400.0
            r["sclk_MHz"] = round(sclk[call], 1)
            r["peak_at_sclk"] = round(peak_at, 1)
            r["frac_at_sclk"] = round(achieved / peak_at, 4)
        return r

    # dominant launch: the call with the largest share of the step
    dom = max(("attn_fwd", "attn_bwd"), key=lambda k: avg[k])
    roofline = roof(dom, fwd_flops if dom == "attn_fwd" else bwd_flops)
    other = "attn_bwd" if dom == "attn_fwd" else "attn_fwd"
    roofline_other = roof(other, bwd_flops if other == "attn_bwd" else fwd_flops)

    metric = "causal attn TFLOP/s @64K, 8q/2kv heads d128 bf16; % MFMA peak; repack GB/s"
    if args.docs:
        metric = f"document-masked causal attn TFLOP/s @{n // 1024}K, {hq}q/{hkv}kv heads d{D} bf16"
    if args.rope_loss:
        metric += " (rotary embedding fused into the first exchange, loss aggregation)"
    elif w.number != 3:
        metric = f"causal attn TFLOP/s @{n // 1024}K, {hq}q/{hkv}kv heads d{D} bf16"
    result = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic" + (" (drawn on the device, seeded)" if big else ""),
        "config": {"workload": w.name + ("+document-mask" if args.docs else ""), "n": n, "P": P, "q_heads": hq,
                   "kv_heads": hkv, "head_dim": D, "global_q_shape": [P, 1, nl, w.Hq_global, D], "causal": True,
                   "padding_mask": valid_np is not None, "document_mask": bool(args.docs),
                   "rope_fused": bool(args.rope_loss), "loss_aggregation": bool(args.rope_loss),
                   "visible_pairs_per_head": pairs,
                   "step": "seq2head(q,k,v) > attn_fwd > seq2head(dO) > attn_bwd > head2seq(o) > head2seq(dq,dk,dv)"},
        "breakdown_ms": {k: round(v, 4) for k, v in avg.items()},
        "per_call_ms": {k: {"mean": round(avg[k], 4), "median": round(med[k], 4), "min": round(mins[k], 4)}
                        for k in names},
        "attn_fwd_tflops_median": round(fwd_flops / (med["attn_fwd"] * 1e-3) / 1e12, 2),
        "attn_bwd_tflops_median": round(bwd_flops / (med["attn_bwd"] * 1e-3) / 1e12, 2),
        "attn_fwd_tflops": round(fwd_tf, 2),
        "attn_fwd_frac_mfma_peak": round(fwd_tf / MFMA_BF16_PEAK_TFLOPS, 4),
        "attn_bwd_tflops": round(bwd_tf, 2),
        "attn_bwd_frac_mfma_peak": round(bwd_tf / MFMA_BF16_PEAK_TFLOPS, 4),
        "repack_GBs": {k: round(v, 1) for k, v in rep.items()},
        "repack_frac_hbm_peak": {k: round(v / HBM_PEAK_GBS, 4) for k, v in rep.items()},
        "device_copy_512MiB_GBs": round(copy_gbs, 1),
        "repack_frac_device_copy": {k: round(v / copy_gbs, 4) for k, v in rep.items()},
        "roofline": roofline,
        f"roofline_{other}": roofline_other,
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle sample)")
        result["cpu_baseline"] = cpu_baseline(args.workload, args.docs)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
