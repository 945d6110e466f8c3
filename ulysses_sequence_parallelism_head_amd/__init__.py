"""Python binding of libulysses, the C-ABI HIP library of the single-GPU
Ulysses sequence-parallel hot path (MI355X / gfx950).

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream; outputs not passed
in are allocated here with ``torch.empty``.  The functions carry the C
names and follow ``include/ulysses.h``; status codes become exceptions:
INVALID_ARG and SCRATCH_LIMIT -> ValueError, UNSUPPORTED ->
NotImplementedError, HIP -> RuntimeError.

There is no fallback: if ``libulysses.so`` is missing, importing the library
raises ``ImportError`` (build it with ``python -m
ulysses_sequence_parallelism_head_amd.build``).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libulysses.so")

DTYPE_F32 = 0
DTYPE_BF16 = 1

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP, ERR_SCRATCH_LIMIT = 0, 1, 2, 3, 4

_lib = None

_SIGS = {
    "ulysses_abi_version": (ctypes.c_int32, []),
    "ulysses_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "ulysses_repack_seq2head": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                               ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int,
                                               ctypes.c_void_p]),
    "ulysses_repack_head2seq": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                               ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int,
                                               ctypes.c_void_p]),
    "ulysses_attn_fwd": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float,
                                        ctypes.c_int32, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]),
    "ulysses_attn_fwd_docs": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                             ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]),
    "ulysses_attn_bwd_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                                           ctypes.c_int32, ctypes.c_int32]),
    "ulysses_attn_bwd": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_size_t,
                                        ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_float, ctypes.c_int32, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_void_p]),
    "ulysses_attn_bwd_noalloc": (ctypes.c_int, [ctypes.c_void_p] * 10 + [ctypes.c_int32, ctypes.c_int64,
                                                                          ctypes.c_int32, ctypes.c_int32,
                                                                          ctypes.c_int32, ctypes.c_float,
                                                                          ctypes.c_int32, ctypes.c_int, ctypes.c_int,
                                                                          ctypes.c_void_p]),
    "ulysses_attn_bwd_docs": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_size_t,
                                             ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_void_p]),
    "ulysses_attn_fwd_block": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                              ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_float, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_int, ctypes.c_void_p]),
    "ulysses_qkv_proj_seq2head": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_int32, ctypes.c_int32,
                                                                          ctypes.c_int64] + [ctypes.c_int32] * 4
                                  + [ctypes.c_void_p]),
    "ulysses_head2seq_out_proj": (ctypes.c_int, [ctypes.c_void_p] * 3 + [ctypes.c_int32, ctypes.c_int32,
                                                                          ctypes.c_int64] + [ctypes.c_int32] * 3
                                  + [ctypes.c_void_p]),
    "ulysses_repack_seq2head_rope": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                                    ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_double,
                                                    ctypes.c_double, ctypes.c_int, ctypes.c_void_p]),
    "ulysses_clock_probe": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.POINTER(ctypes.c_int32), ctypes.c_void_p]),
    "ulysses_loss_aggregate": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
}

EXPORTED = tuple(_SIGS)


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libulysses.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} not found: build it with `python -m ulysses_sequence_parallelism_head_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int, what: str) -> None:
    if status == OK:
        return
    msg = f"{what}: {load_library().ulysses_status_string(status).decode()}"
    if status in (ERR_INVALID_ARG, ERR_SCRATCH_LIMIT):
        raise ValueError(msg)
    if status == ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise RuntimeError(msg)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need_contig_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous and on the GPU")


def _expect(t, name: str, shape, dtypes, device) -> None:
    """The library derives every extent from the leading tensor's shape and
    receives raw pointers, so a smaller or differently typed buffer would be
    read or written out of bounds: check shape, dtype and device here, before
    any call."""
    if t is None:
        return
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(int(x) for x in shape)}, got {tuple(t.shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must have dtype {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


_F32 = (torch.float32,)
_BF16 = (torch.bfloat16,)
_FLOAT = (torch.bfloat16, torch.float32)


def ulysses_abi_version() -> int:
    return int(load_library().ulysses_abi_version())


def ulysses_repack_seq2head(src: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """src ``[P][B][n_local][H][D]`` -> ``[P][B][P*n_local][H/P][D]`` (first exchange)."""
    lib = load_library()
    _need_contig_cuda(src, out)
    P, B, nl, H, D = src.shape
    if H % P != 0 or H < P:
        _check(ERR_INVALID_ARG, "ulysses_repack_seq2head")
    _expect(out, "out", (P, B, P * nl, H // P, D), (src.dtype,), src.device)
    if out is None:
        out = torch.empty((P, B, P * nl, H // P, D), dtype=src.dtype, device=src.device)
    _check(lib.ulysses_repack_seq2head(_ptr(src), _ptr(out), P, B, nl, H, D, _dtype_code(src), _stream(src.device)),
           "ulysses_repack_seq2head")
    return out


def ulysses_repack_head2seq(src: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """src ``[P][B][n][H/P][D]`` -> ``[P][B][n/P][H][D]`` (second exchange)."""
    lib = load_library()
    _need_contig_cuda(src, out)
    P, B, n, hp, D = src.shape
    if n % P != 0:
        _check(ERR_INVALID_ARG, "ulysses_repack_head2seq")
    nl, H = n // P, hp * P
    _expect(out, "out", (P, B, nl, H, D), (src.dtype,), src.device)
    if out is None:
        out = torch.empty((P, B, nl, H, D), dtype=src.dtype, device=src.device)
    _check(lib.ulysses_repack_head2seq(_ptr(src), _ptr(out), P, B, nl, H, D, _dtype_code(src), _stream(src.device)),
           "ulysses_repack_head2seq")
    return out


def ulysses_attn_fwd_block(q, k, v, o, lse, causal_offset: int, key_valid=None, softmax_scale=None,
                           causal: bool = True, accumulate: bool = False):
    """Forward of the bf16 rows ``q`` ``[B][nq][Hq][D]`` over the key block
    ``k``/``v`` ``[B][nk][Hkv][D]`` (key u visible to row t iff
    u <= t + causal_offset when causal).  ``o`` (float32 ``[B][nq][Hq][D]``)
    and ``lse`` (float32 ``[B][Hq][nq]``) are overwritten, or merged into
    when ``accumulate``.  Returns ``(o, lse)``."""
    lib = load_library()
    _need_contig_cuda(q, k, v, o, lse, key_valid)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [B][n][H][D]")
    B, nq, Hq, D = q.shape
    nk, Hkv = k.shape[1], k.shape[2]
    dev = q.device
    _expect(k, "k", (B, nk, Hkv, D), (q.dtype,), dev)
    _expect(v, "v", (B, nk, Hkv, D), (q.dtype,), dev)
    _expect(key_valid, "key_valid", (B, nk), (torch.uint8,), dev)
    _expect(o, "o", (B, nq, Hq, D), _F32, dev)
    _expect(lse, "lse", (B, Hq, nq), _F32, dev)
    scale = D ** -0.5 if softmax_scale is None else float(softmax_scale)
    _check(lib.ulysses_attn_fwd_block(_ptr(q), _ptr(k), _ptr(v), _ptr(key_valid), _ptr(o), _ptr(lse), B, nq, nk,
                                      Hq, Hkv, D, scale, int(causal_offset), int(bool(causal)),
                                      int(bool(accumulate)), _dtype_code(q), _stream(q.device)),
           "ulysses_attn_fwd_block")
    return o, lse


def ulysses_qkv_proj_seq2head(x: torch.Tensor, w: torch.Tensor, Hq: int, Hkv: int, D: int, q=None, k=None, v=None):
    """x bf16 ``[P][B][n_local][hidden]``, w bf16 ``[(Hq + 2 Hkv) D][hidden]`` ->
    head-sharded ``(q [P][B][P n_local][Hq/P][D], k, v [P][B][P n_local][Hkv/P][D])``."""
    lib = load_library()
    _need_contig_cuda(x, w, q, k, v)
    P, B, nl, hidden = x.shape
    if tuple(w.shape) != ((Hq + 2 * Hkv) * D, hidden) or x.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
        raise ValueError("x and w must be bf16 with w [(Hq + 2 Hkv) D][hidden]")
    if Hq % P or Hkv % P:
        _check(ERR_INVALID_ARG, "ulysses_qkv_proj_seq2head")
    dev = x.device
    _expect(w, "w", w.shape, _BF16, dev)
    _expect(q, "q", (P, B, P * nl, Hq // P, D), _BF16, dev)
    _expect(k, "k", (P, B, P * nl, Hkv // P, D), _BF16, dev)
    _expect(v, "v", (P, B, P * nl, Hkv // P, D), _BF16, dev)
    q = torch.empty((P, B, P * nl, Hq // P, D), dtype=torch.bfloat16, device=dev) if q is None else q
    k = torch.empty((P, B, P * nl, Hkv // P, D), dtype=torch.bfloat16, device=dev) if k is None else k
    v = torch.empty((P, B, P * nl, Hkv // P, D), dtype=torch.bfloat16, device=dev) if v is None else v
    _check(lib.ulysses_qkv_proj_seq2head(_ptr(x), _ptr(w), _ptr(q), _ptr(k), _ptr(v), P, B, nl, hidden, Hq, Hkv, D,
                                         _stream(dev)),
           "ulysses_qkv_proj_seq2head")
    return q, k, v


def ulysses_head2seq_out_proj(o: torch.Tensor, w_o: torch.Tensor, y=None):
    """o bf16 ``[P][B][P n_local][Hq/P][D]`` (head-sharded attention output),
    w_o bf16 ``[hidden][Hq D]`` -> y bf16 ``[P][B][n_local][hidden]``."""
    lib = load_library()
    _need_contig_cuda(o, w_o, y)
    P, B, n, hp, D = o.shape
    Hq = hp * P
    hidden = w_o.shape[0]
    if tuple(w_o.shape) != (hidden, Hq * D) or o.dtype != torch.bfloat16 or w_o.dtype != torch.bfloat16 or n % P:
        raise ValueError("o and w_o must be bf16 with w_o [hidden][Hq D] and n divisible by P")
    _expect(w_o, "w_o", w_o.shape, _BF16, o.device)
    _expect(y, "y", (P, B, n // P, hidden), _BF16, o.device)
    y = torch.empty((P, B, n // P, hidden), dtype=torch.bfloat16, device=o.device) if y is None else y
    _check(lib.ulysses_head2seq_out_proj(_ptr(o), _ptr(w_o), _ptr(y), P, B, n // P, Hq, D, hidden, _stream(o.device)),
           "ulysses_head2seq_out_proj")
    return y


def ulysses_repack_seq2head_rope(src: torch.Tensor, rope_base: float, rope_scale: float = 1.0,
                                 out: torch.Tensor | None = None) -> torch.Tensor:
    """Like :func:`ulysses_repack_seq2head`, rotating each head vector at its
    token's global position on the way (Q and K before the first exchange)."""
    lib = load_library()
    _need_contig_cuda(src, out)
    P, B, nl, H, D = src.shape
    if H % P != 0 or H < P:
        _check(ERR_INVALID_ARG, "ulysses_repack_seq2head_rope")
    _expect(out, "out", (P, B, P * nl, H // P, D), (src.dtype,), src.device)
    if out is None:
        out = torch.empty((P, B, P * nl, H // P, D), dtype=src.dtype, device=src.device)
    _check(lib.ulysses_repack_seq2head_rope(_ptr(src), _ptr(out), P, B, nl, H, D, float(rope_base), float(rope_scale),
                                            _dtype_code(src), _stream(src.device)),
           "ulysses_repack_seq2head_rope")
    return out


def ulysses_loss_aggregate(token_loss: torch.Tensor, valid: torch.Tensor | None = None, rank_sum=None,
                           rank_count=None, loss=None):
    """token_loss float32 ``[P][...]`` (one row of per-token losses per rank),
    valid uint8 of the same shape or None.  Returns ``(rank_sum float64 [P],
    rank_count int64 [P], loss float32 [1])``."""
    lib = load_library()
    _need_contig_cuda(token_loss, valid, rank_sum, rank_count, loss)
    if token_loss.dtype != torch.float32:
        raise ValueError("token_loss must be float32")
    if valid is not None and (valid.dtype != torch.uint8 or valid.shape != token_loss.shape):
        raise ValueError("valid must be uint8 with token_loss's shape")
    P = token_loss.shape[0]
    per_rank = token_loss.numel() // P if P else 0
    dev = token_loss.device
    _expect(rank_sum, "rank_sum", (P,), (torch.float64,), dev)
    _expect(rank_count, "rank_count", (P,), (torch.int64,), dev)
    _expect(loss, "loss", (1,), _F32, dev)
    rank_sum = torch.empty(P, dtype=torch.float64, device=dev) if rank_sum is None else rank_sum
    rank_count = torch.empty(P, dtype=torch.int64, device=dev) if rank_count is None else rank_count
    loss = torch.empty(1, dtype=torch.float32, device=dev) if loss is None else loss
    _check(lib.ulysses_loss_aggregate(_ptr(token_loss), _ptr(valid), P, per_rank, _ptr(rank_sum), _ptr(rank_count),
                                      _ptr(loss), _stream(dev)),
           "ulysses_loss_aggregate")
    return rank_sum, rank_count, loss


def ulysses_clock_probe(samples: int, interval_us: int, stream=None):
    """Launch the clock sampler on ``stream`` (a torch.cuda.Stream; the
    current stream if None).  Returns ``(out, wall_khz)``: ``out`` is the
    uint64 device buffer of (stamp, cycles) pairs as an int64 tensor
    ``[samples][2]`` (valid once the stream has finished), ``wall_khz`` the
    real-time counter's rate."""
    lib = load_library()
    dev = torch.device("cuda", torch.cuda.current_device())
    out = torch.zeros((samples, 2), dtype=torch.int64, device=dev)
    khz = ctypes.c_int32(0)
    st = ctypes.c_void_p((stream if stream is not None else torch.cuda.current_stream(dev)).cuda_stream)
    _check(lib.ulysses_clock_probe(_ptr(out), int(samples), int(interval_us), ctypes.byref(khz), st),
           "ulysses_clock_probe")
    return out, int(khz.value)


def clock_probe_mhz(out: torch.Tensor, wall_khz: int):
    """Engine clock (MHz) over each interval of a finished probe."""
    o = out.cpu().numpy()
    ticks = o[1:, 0] - o[:-1, 0]
    return [float(c) / (float(t) / (wall_khz * 1e3)) / 1e6 for c, t in zip(o[1:, 1], ticks) if t > 0]


def _check_docs(doc_start, B, n):
    if doc_start is not None and (doc_start.dtype != torch.int32 or tuple(doc_start.shape) != (B, n)):
        raise ValueError("doc_start must be int32 [B][n]")


def ulysses_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, key_valid: torch.Tensor | None = None,
                     softmax_scale: float | None = None, causal: bool = True, o_dtype: torch.dtype | None = None,
                     out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """Attention forward.  q ``[B][n][Hq][D]``, k/v ``[B][n][Hkv][D]``,
    key_valid ``[B][n]`` uint8 or None.  Returns ``(o, lse)``; lse is
    float32 ``[B][Hq][n]`` in natural log."""
    return _attn_fwd(q, k, v, key_valid, None, softmax_scale, causal, o_dtype, out, lse)


def ulysses_attn_fwd_docs(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, doc_start: torch.Tensor,
                          key_valid: torch.Tensor | None = None, softmax_scale: float | None = None,
                          o_dtype: torch.dtype | None = None, out: torch.Tensor | None = None,
                          lse: torch.Tensor | None = None):
    """Document-masked causal forward: ``doc_start`` int32 ``[B][n]`` is the
    first position of each token's document.  Returns ``(o, lse)``."""
    return _attn_fwd(q, k, v, key_valid, doc_start, softmax_scale, True, o_dtype, out, lse)


def _attn_fwd(q, k, v, key_valid, doc_start, softmax_scale, causal, o_dtype, out, lse):
    lib = load_library()
    _need_contig_cuda(q, k, v, key_valid, doc_start, out, lse)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [B][n][H][D]")
    B, n, Hq, D = q.shape
    Hkv = k.shape[2]
    dev = q.device
    _expect(q, "q", q.shape, _FLOAT, dev)
    _expect(k, "k", (B, n, Hkv, D), (q.dtype,), dev)
    _expect(v, "v", (B, n, Hkv, D), (q.dtype,), dev)
    _expect(key_valid, "key_valid", (B, n), (torch.uint8,), dev)
    _check_docs(doc_start, B, n)
    _expect(doc_start, "doc_start", (B, n), (torch.int32,), dev)
    scale = D ** -0.5 if softmax_scale is None else float(softmax_scale)
    if o_dtype is None:
        o_dtype = q.dtype if out is None else out.dtype
    _expect(out, "out", (B, n, Hq, D), (o_dtype,), dev)
    _expect(lse, "lse", (B, Hq, n), _F32, dev)
    if out is None:
        out = torch.empty((B, n, Hq, D), dtype=o_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, n), dtype=torch.float32, device=q.device)
    if doc_start is None:
        _check(lib.ulysses_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(key_valid), _ptr(out), _ptr(lse), B, n, Hq, Hkv,
                                    D, scale, int(bool(causal)), _dtype_code(q), _dtype_code(out), _stream(q.device)),
               "ulysses_attn_fwd")
    else:
        _check(lib.ulysses_attn_fwd_docs(_ptr(q), _ptr(k), _ptr(v), _ptr(key_valid), _ptr(doc_start), _ptr(out),
                                         _ptr(lse), B, n, Hq, Hkv, D, scale, _dtype_code(q), _dtype_code(out),
                                         _stream(q.device)),
               "ulysses_attn_fwd_docs")
    return out, lse


def ulysses_attn_bwd_workspace_bytes(B: int, n: int, Hq: int, Hkv: int, D: int) -> int:
    return int(load_library().ulysses_attn_bwd_workspace_bytes(B, n, Hq, Hkv, D))


def ulysses_attn_bwd(q, k, v, o, lse, dout, key_valid=None, softmax_scale=None, causal=True,
                     dq=None, dk=None, dv=None, workspace=None):
    """Attention backward.  Returns float32 ``(dq, dk, dv)``."""
    return _attn_bwd(q, k, v, o, lse, dout, key_valid, None, softmax_scale, causal, dq, dk, dv, workspace)


def ulysses_attn_bwd_docs(q, k, v, o, lse, dout, doc_start, key_valid=None, softmax_scale=None,
                          dq=None, dk=None, dv=None, workspace=None):
    """Backward of :func:`ulysses_attn_fwd_docs`.  Returns float32 ``(dq, dk, dv)``."""
    return _attn_bwd(q, k, v, o, lse, dout, key_valid, doc_start, softmax_scale, True, dq, dk, dv, workspace)


def ulysses_attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, key_valid=None, softmax_scale=None, causal=True):
    """:func:`ulysses_attn_bwd` without a workspace and without any
    allocation: the caller passes the float32 outputs ``dq``, ``dk``, ``dv``;
    the library uses its fixed per-GPU scratch (B * Hq * n <= 2^21).  Calls
    that overlap on one GPU race on that scratch."""
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t is None:
            raise ValueError(f"{name} is required: this call allocates nothing")
    return _attn_bwd(q, k, v, o, lse, dout, key_valid, None, softmax_scale, causal, dq, dk, dv, None, noalloc=True)


def _attn_bwd(q, k, v, o, lse, dout, key_valid, doc_start, softmax_scale, causal, dq, dk, dv, workspace,
              noalloc=False):
    lib = load_library()
    _need_contig_cuda(q, k, v, o, lse, dout, key_valid, doc_start, dq, dk, dv, workspace)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [B][n][H][D]")
    B, n, Hq, D = q.shape
    _check_docs(doc_start, B, n)
    Hkv = k.shape[2]
    scale = D ** -0.5 if softmax_scale is None else float(softmax_scale)
    dev = q.device
    _expect(q, "q", q.shape, _FLOAT, dev)
    _expect(k, "k", (B, n, Hkv, D), (q.dtype,), dev)
    _expect(v, "v", (B, n, Hkv, D), (q.dtype,), dev)
    _expect(o, "o", (B, n, Hq, D), _FLOAT, dev)
    _expect(lse, "lse", (B, Hq, n), _F32, dev)
    _expect(dout, "dout", (B, n, Hq, D), (q.dtype,), dev)
    _expect(key_valid, "key_valid", (B, n), (torch.uint8,), dev)
    _expect(doc_start, "doc_start", (B, n), (torch.int32,), dev)
    _expect(dq, "dq", (B, n, Hq, D), _F32, dev)
    _expect(dk, "dk", (B, n, Hkv, D), _F32, dev)
    _expect(dv, "dv", (B, n, Hkv, D), _F32, dev)
    if workspace is not None and workspace.device != dev:
        raise ValueError(f"workspace is on {workspace.device}, expected {dev}")
    if noalloc:
        _check(lib.ulysses_attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(key_valid), _ptr(o), _ptr(lse),
                                            _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), B, n, Hq, Hkv, D, scale,
                                            int(bool(causal)), _dtype_code(q), _dtype_code(o), _stream(dev)),
               "ulysses_attn_bwd_noalloc")
        return dq, dk, dv
    dq = torch.empty((B, n, Hq, D), dtype=torch.float32, device=dev) if dq is None else dq
    dk = torch.empty((B, n, Hkv, D), dtype=torch.float32, device=dev) if dk is None else dk
    dv = torch.empty((B, n, Hkv, D), dtype=torch.float32, device=dev) if dv is None else dv
    wsb = ulysses_attn_bwd_workspace_bytes(B, n, Hq, Hkv, D)
    if workspace is None:
        workspace = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    wbytes = workspace.numel() * workspace.element_size()
    if doc_start is None:
        _check(lib.ulysses_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(key_valid), _ptr(o), _ptr(lse), _ptr(dout),
                                    _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), wbytes,
                                    B, n, Hq, Hkv, D, scale, int(bool(causal)), _dtype_code(q), _dtype_code(o),
                                    _stream(dev)),
               "ulysses_attn_bwd")
    else:
        _check(lib.ulysses_attn_bwd_docs(_ptr(q), _ptr(k), _ptr(v), _ptr(key_valid), _ptr(doc_start), _ptr(o),
                                         _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), wbytes,
                                         B, n, Hq, Hkv, D, scale, _dtype_code(q), _dtype_code(o), _stream(dev)),
               "ulysses_attn_bwd_docs")
    return dq, dk, dv


__all__ = [
    "load_library", "EXPORTED", "LIB_PATH", "ulysses_abi_version", "ulysses_repack_seq2head",
    "ulysses_repack_head2seq", "ulysses_attn_fwd", "ulysses_attn_bwd", "ulysses_attn_bwd_workspace_bytes",
    "ulysses_attn_fwd_docs", "ulysses_attn_bwd_docs", "ulysses_attn_bwd_noalloc", "ulysses_repack_seq2head_rope", "ulysses_loss_aggregate",
    "ulysses_attn_fwd_block", "ulysses_qkv_proj_seq2head", "ulysses_head2seq_out_proj", "ulysses_clock_probe",
    "clock_probe_mhz",
]
