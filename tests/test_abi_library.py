"""The C-ABI library on the host (no GPU needed): it loads, exports every
symbol include/ulysses.h declares (and nothing else), and its host-side
argument validation returns the documented status before any launch."""
import ctypes
import os
import re
import subprocess

import pytest

import ulysses_sequence_parallelism_head_amd as U

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ulysses.h")

OK, INVALID, UNSUPPORTED = 0, 1, 2
BF16, F32 = 1, 0


def declared_symbols():
    text = open(HEADER, encoding="utf-8").read()
    return sorted(set(re.findall(r"ULYSSES_API\s+[\w\s\*]+?\b(ulysses_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return U.load_library()


def test_header_declares_the_boundary():
    syms = declared_symbols()
    for name in ("ulysses_repack_seq2head", "ulysses_repack_head2seq", "ulysses_attn_fwd", "ulysses_attn_bwd"):
        assert name in syms
    assert set(syms) == set(U.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", U.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = sorted(l.split()[-1] for l in out.splitlines() if " T " in l and "ulysses_" in l)
    assert exported == declared_symbols()
    for name in declared_symbols():
        assert hasattr(lib, name)


def test_version_and_status_strings(lib):
    assert lib.ulysses_abi_version() == 1
    for s in range(4):
        assert lib.ulysses_status_string(s)
    assert lib.ulysses_status_string(99) == b"unknown status"


# --- validation paths: every call below is rejected before any launch
FAKE = ctypes.c_void_p(0x10000)        # never dereferenced: the calls fail validation first
FAKE2 = ctypes.c_void_p(0x20000000)


@pytest.mark.parametrize("P,B,nl,H,D,dt,expect", [
    (4, 1, 16, 2, 128, BF16, INVALID),   # H < P
    (4, 1, 16, 6, 128, BF16, INVALID),   # H % P != 0
    (0, 1, 16, 4, 128, BF16, INVALID),   # P < 1
    (2, -1, 16, 4, 128, BF16, INVALID),  # B < 0
    (2, 1, -3, 4, 128, BF16, INVALID),   # n_local < 0
    (2, 1, 16, 4, 0, BF16, INVALID),     # D < 1
    (2, 1, 16, 4, 8, 7, INVALID),        # unknown dtype
    (2, 0, 16, 4, 8, BF16, OK),          # empty: no-op
    (2, 1, 0, 4, 8, BF16, OK),           # empty: no-op
])
def test_repack_validation(lib, P, B, nl, H, D, dt, expect):
    for fn in (lib.ulysses_repack_seq2head, lib.ulysses_repack_head2seq):
        assert fn(FAKE, FAKE2, P, B, nl, H, D, dt, None) == expect


def test_repack_null_and_overlap(lib):
    assert lib.ulysses_repack_seq2head(None, FAKE2, 2, 1, 4, 4, 8, BF16, None) == INVALID
    assert lib.ulysses_repack_seq2head(FAKE, None, 2, 1, 4, 4, 8, BF16, None) == INVALID
    # src and dst ranges overlap (in-place not allowed)
    assert lib.ulysses_repack_seq2head(FAKE, ctypes.c_void_p(0x10000 + 64), 2, 1, 4, 4, 8, BF16, None) == INVALID
    # misaligned for the element size
    assert lib.ulysses_repack_seq2head(ctypes.c_void_p(0x10001), FAKE2, 2, 1, 4, 4, 8, BF16, None) == INVALID


def _fwd(lib, q=FAKE, k=ctypes.c_void_p(0x1000000), v=ctypes.c_void_p(0x2000000), valid=None,
         o=ctypes.c_void_p(0x3000000), lse=ctypes.c_void_p(0x4000000), B=1, n=64, Hq=8, Hkv=2, D=128,
         scale=0.1, causal=1, it=BF16, ot=BF16):
    return lib.ulysses_attn_fwd(q, k, v, valid, o, lse, B, n, Hq, Hkv, D, scale, causal, it, ot, None)


def test_fwd_validation(lib):
    assert _fwd(lib, D=96) == UNSUPPORTED
    assert _fwd(lib, it=F32, ot=BF16) == UNSUPPORTED
    assert _fwd(lib, Hq=6, Hkv=4) == INVALID
    assert _fwd(lib, Hkv=0) == INVALID
    assert _fwd(lib, n=-1) == INVALID
    assert _fwd(lib, scale=float("nan")) == INVALID
    assert _fwd(lib, scale=float("inf")) == INVALID
    assert _fwd(lib, scale=0.0) == INVALID
    assert _fwd(lib, scale=-0.5) == INVALID
    assert _fwd(lib, causal=2) == INVALID
    assert _fwd(lib, q=None) == INVALID
    assert _fwd(lib, lse=None) == INVALID
    assert _fwd(lib, q=ctypes.c_void_p(0x10008)) == INVALID               # not 16-byte aligned
    assert _fwd(lib, o=ctypes.c_void_p(0x1000000 + 256)) == INVALID       # o overlaps k
    assert _fwd(lib, lse=ctypes.c_void_p(0x3000000 + 64)) == INVALID      # lse overlaps o
    assert _fwd(lib, B=0) == OK                                           # empty
    assert _fwd(lib, n=0, q=None, k=None, v=None, o=None, lse=None) == OK


def _bwd(lib, ws=ctypes.c_void_p(0x9000000), wsb=1 << 21, dq=ctypes.c_void_p(0x6000000), it=BF16, D=128, n=64):
    return lib.ulysses_attn_bwd(FAKE, ctypes.c_void_p(0x1000000), ctypes.c_void_p(0x2000000), None,
                                ctypes.c_void_p(0x3000000), ctypes.c_void_p(0x4000000), ctypes.c_void_p(0x5000000),
                                dq, ctypes.c_void_p(0x7000000), ctypes.c_void_p(0x8000000), ws, wsb,
                                1, n, 8, 2, D, 0.1, 1, it, BF16, None)


def test_bwd_validation(lib):
    need = lib.ulysses_attn_bwd_workspace_bytes(1, 64, 8, 2, 128)
    # two float32 row arrays, plus (short sequences) 8 splits' partial dK and dV
    assert need == 2 * 64 * 8 * 4 + 2 * 8 * 64 * 2 * 128 * 4 and need % 256 == 0
    assert lib.ulysses_attn_bwd_workspace_bytes(0, 64, 8, 2, 128) == 0
    # long sequences: no splits, the row arrays only (n = 65536, 2 KV heads: 512 key-block pairs)
    assert lib.ulysses_attn_bwd_workspace_bytes(1, 65536, 8, 2, 128) == 2 * 65536 * 8 * 4
    # 8192 tokens, 2 KV heads: 64 pairs -> 8 splits
    assert lib.ulysses_attn_bwd_workspace_bytes(1, 8192, 8, 2, 128) == 2 * 8192 * 8 * 4 + 2 * 8 * 8192 * 2 * 128 * 4
    assert _bwd(lib, wsb=need - 1) == INVALID
    assert _bwd(lib, ws=None) == INVALID
    assert _bwd(lib, ws=ctypes.c_void_p(0x9000000 + 16)) == INVALID        # workspace not 256-byte aligned
    assert _bwd(lib, dq=ctypes.c_void_p(0x5000000 + 64)) == INVALID        # dq overlaps dout
    assert _bwd(lib, it=F32) == UNSUPPORTED
    assert _bwd(lib, D=80) == UNSUPPORTED


DOCS = ctypes.c_void_p(0xA000000)


def _fwd_docs(lib, docs=DOCS, o=ctypes.c_void_p(0x3000000), B=1, n=64, it=BF16, ot=BF16):
    return lib.ulysses_attn_fwd_docs(FAKE, ctypes.c_void_p(0x1000000), ctypes.c_void_p(0x2000000), None, docs, o,
                                     ctypes.c_void_p(0x4000000), B, n, 8, 2, 128, 0.1, it, ot, None)


def _bwd_docs(lib, docs=DOCS, dq=ctypes.c_void_p(0x6000000), n=64):
    return lib.ulysses_attn_bwd_docs(FAKE, ctypes.c_void_p(0x1000000), ctypes.c_void_p(0x2000000), None, docs,
                                     ctypes.c_void_p(0x3000000), ctypes.c_void_p(0x4000000),
                                     ctypes.c_void_p(0x5000000), dq, ctypes.c_void_p(0x7000000),
                                     ctypes.c_void_p(0x8000000), ctypes.c_void_p(0x9000000), 1 << 20,
                                     1, n, 8, 2, 128, 0.1, BF16, BF16, None)


def test_docs_validation(lib):
    assert _fwd_docs(lib, docs=None) == INVALID                              # the documents are required
    assert _fwd_docs(lib, docs=ctypes.c_void_p(0xA000002)) == INVALID        # not 4-byte aligned
    assert _fwd_docs(lib, o=ctypes.c_void_p(0xA000000 - 1024)) == INVALID    # o overlaps doc_start
    assert _fwd_docs(lib, it=F32, ot=BF16) == UNSUPPORTED
    assert _fwd_docs(lib, B=0, docs=None) == OK                              # empty
    assert _bwd_docs(lib, docs=None) == INVALID
    assert _bwd_docs(lib, dq=ctypes.c_void_p(0xA000000 - 4096)) == INVALID   # dq overlaps doc_start
    assert _bwd_docs(lib, n=0, docs=None) == OK


def test_rope_validation(lib):
    f = lib.ulysses_repack_seq2head_rope
    assert f(FAKE, FAKE2, 4, 1, 16, 6, 128, 1e6, 1.0, BF16, None) == INVALID          # H % P != 0
    assert f(FAKE, FAKE2, 4, 1, 16, 32, 96, 1e6, 1.0, BF16, None) == UNSUPPORTED      # D
    assert f(FAKE, FAKE2, 4, 1, 16, 32, 128, 0.0, 1.0, BF16, None) == INVALID         # base
    assert f(FAKE, FAKE2, 4, 1, 16, 32, 128, float("nan"), 1.0, BF16, None) == INVALID
    assert f(FAKE, FAKE2, 4, 1, 16, 32, 128, 1e6, -2.0, BF16, None) == INVALID        # scale
    assert f(FAKE, FAKE2, 4, 1, 16, 32, 128, 1e6, 1.0, 7, None) == INVALID            # dtype
    assert f(FAKE, ctypes.c_void_p(0x10000 + 64), 4, 1, 16, 32, 128, 1e6, 1.0, BF16, None) == INVALID   # overlap
    assert f(ctypes.c_void_p(0x10008), FAKE2, 4, 1, 16, 32, 128, 1e6, 1.0, BF16, None) == INVALID       # alignment
    assert f(None, None, 4, 0, 16, 32, 128, 1e6, 1.0, BF16, None) == OK               # empty


def test_loss_validation(lib):
    f = lib.ulysses_loss_aggregate
    S, C, L = ctypes.c_void_p(0x5000000), ctypes.c_void_p(0x6000000), ctypes.c_void_p(0x7000000)
    assert f(FAKE, None, 0, 10, S, C, L, None) == INVALID                     # P < 1
    assert f(FAKE, None, 2, -1, S, C, L, None) == INVALID                     # per_rank < 0
    assert f(None, None, 2, 10, S, C, L, None) == INVALID                     # token_loss required
    assert f(FAKE, None, 2, 10, None, C, L, None) == INVALID                  # outputs required
    assert f(FAKE, None, 2, 10, ctypes.c_void_p(0x5000004), C, L, None) == INVALID   # rank_sum alignment
    assert f(FAKE, None, 2, 10, S, ctypes.c_void_p(0x5000008), L, None) == INVALID   # overlapping outputs
    assert f(FAKE, None, 2, 10, ctypes.c_void_p(0x10000 + 8), C, L, None) == INVALID  # output overlaps input


def test_block_validation(lib):
    f = lib.ulysses_attn_fwd_block
    O, LS = ctypes.c_void_p(0x3000000), ctypes.c_void_p(0x4000000)
    def call(nk=64, acc=0, it=BF16, causal=1, o=O, D=128, nq=64):
        return f(FAKE, ctypes.c_void_p(0x1000000), ctypes.c_void_p(0x2000000), None, o, LS, 1, nq, nk, 8, 2, D, 0.1,
                 5, causal, acc, it, None)
    assert call(nk=0) == INVALID
    assert call(acc=2) == INVALID
    assert call(causal=3) == INVALID
    assert call(it=F32) == UNSUPPORTED
    assert call(D=96) == UNSUPPORTED
    assert call(nk=(1 << 31) - 100) == UNSUPPORTED
    assert call(o=ctypes.c_void_p(0x1000000 + 256)) == INVALID     # o overlaps k
    assert call(nq=0) == OK                                        # empty


def test_proj_validation(lib):
    f = lib.ulysses_qkv_proj_seq2head
    Q, K, V = ctypes.c_void_p(0x3000000), ctypes.c_void_p(0x4000000), ctypes.c_void_p(0x5000000)
    W = ctypes.c_void_p(0x1000000)
    assert f(FAKE, W, Q, K, V, 4, 1, 16, 4096, 30, 8, 128, None) == INVALID       # Hq % P
    assert f(FAKE, W, Q, K, V, 4, 1, 16, 4096, 32, 8, 96, None) == UNSUPPORTED    # D
    assert f(FAKE, W, Q, K, V, 4, 1, 16, 4000, 32, 8, 128, None) == UNSUPPORTED   # hidden % 64
    assert f(FAKE, W, ctypes.c_void_p(0x1000000 + 64), K, V, 4, 1, 16, 4096, 32, 8, 128, None) == INVALID   # q overlaps w
    assert f(FAKE, W, Q, K, ctypes.c_void_p(0x3000010), 4, 1, 16, 4096, 32, 8, 128, None) == INVALID  # v overlaps q
    assert f(None, None, None, None, None, 4, 0, 16, 4096, 32, 8, 128, None) == OK                    # empty
    g = lib.ulysses_head2seq_out_proj
    Y = ctypes.c_void_p(0x6000000)
    assert g(FAKE, W, Y, 4, 1, 16, 30, 128, 4096, None) == INVALID                # Hq % P
    assert g(FAKE, W, Y, 4, 1, 16, 32, 128, 4098, None) == UNSUPPORTED           # hidden % 4
    assert g(FAKE, W, ctypes.c_void_p(0x10000 + 16), 4, 1, 16, 32, 128, 4096, None) == INVALID   # y overlaps o


def _bwd_noalloc(lib, B=1, n=64, Hq=8, dq=None, it=BF16, D=128):
    # buffers 2^36 bytes apart, so that even the largest sizes below do not overlap
    a = [ctypes.c_void_p((i + 1) << 36) for i in range(10)]
    if dq is not None:
        a[7] = dq
    return lib.ulysses_attn_bwd_noalloc(a[0], a[1], a[2], None, a[4], a[5], a[6], a[7], a[8], a[9],
                                        B, n, Hq, 2, D, 0.1, 1, it, BF16, None)


def test_bwd_noalloc_validation(lib):
    """The no-allocation backward: its size limit (2 * B * Hq * n * 4 bytes
    <= 16 MiB) is checked before anything touches a device, after the
    ordinary argument checks."""
    SCRATCH_LIMIT = 4
    assert b"scratch" in lib.ulysses_status_string(SCRATCH_LIMIT)
    assert _bwd_noalloc(lib, n=(1 << 21) // 8 + 1) == SCRATCH_LIMIT      # B*Hq*n just above 2^21
    assert _bwd_noalloc(lib, B=2, n=1 << 20, Hq=2) == SCRATCH_LIMIT
    assert _bwd_noalloc(lib, Hq=7) == INVALID                             # Hq % Hkv
    assert _bwd_noalloc(lib, D=80) == UNSUPPORTED
    assert _bwd_noalloc(lib, n=-1) == INVALID
    assert _bwd_noalloc(lib, B=0) == OK                                   # empty: nothing to do, no device use
    assert _bwd_noalloc(lib, dq=ctypes.c_void_p(0)) == INVALID             # null dq
    assert _bwd_noalloc(lib, dq=ctypes.c_void_p((7 << 36) + 64)) == INVALID  # dq overlaps dout
    assert _bwd_noalloc(lib, it=F32) == UNSUPPORTED
