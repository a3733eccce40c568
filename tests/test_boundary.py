"""The C ABI without a GPU: exported symbols and argument checking (CPU only).

The validators are the same checks fa2_fwd / fa2_bwd run before any HIP
call, so every error path is exercised here with fake (never dereferenced)
device addresses.
"""
import ctypes
import os
import re
import subprocess

import pytest

from exact_io_aware_26_amd import fa2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa2.h")

OK, INVALID, UNSUPPORTED, HIPERR = 0, 1, 2, 3
MB = 1 << 20


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa2.LIB_PATH):
        pytest.skip("libfa2.so not built")
    return fa2.load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"\b(fa2_[a-z_0-9]+)\s*\(", src))


def test_header_declares_the_binding_exports():
    assert declared_functions() == set(fa2.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", fa2.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (fa2_\w+)", out))
    missing = declared_functions() - exported
    assert not missing, f"declared but not exported: {missing}"
    for name in declared_functions():
        assert hasattr(lib, name)


def test_status_strings(lib):
    assert lib.fa2_status_string(OK) == b"FA2_OK"
    assert lib.fa2_status_string(INVALID) == b"FA2_ERR_INVALID_ARGUMENT"
    assert lib.fa2_status_string(UNSUPPORTED) == b"FA2_ERR_UNSUPPORTED"
    assert lib.fa2_status_string(HIPERR) == b"FA2_ERR_HIP"
    assert lib.fa2_status_string(99) == b"unknown status"


# Fake, 256-byte aligned, non-overlapping device addresses (never dereferenced).
BASE = 1 << 40
def addr(i):
    return BASE + i * (1 << 36)


def vfwd(lib, B=2, Hq=4, Hkv=2, N=100, d=128, causal=1, scale=0.125, ptrs=None):
    p = ptrs or [addr(i) for i in range(5)]
    return lib.fa2_validate_fwd(*p, B, Hq, Hkv, N, d, causal, scale)


def ws_bytes(lib, B=2, Hq=4, Hkv=2, N=100, d=128):
    return lib.fa2_bwd_workspace_bytes(B, Hq, Hkv, N, d)


def vbwd(lib, B=2, Hq=4, Hkv=2, N=100, d=128, causal=1, scale=0.125, ptrs=None, ws=None):
    p = ptrs or [addr(i) for i in range(10)]
    if ws is None:
        ws = ws_bytes(lib, B, Hq, Hkv, N, d)
    return lib.fa2_validate_bwd(*p, ws, B, Hq, Hkv, N, d, causal, scale)


def test_valid_calls_pass(lib):
    for d in (64, 128, 256):
        for causal in (0, 1):
            assert vfwd(lib, d=d, causal=causal) == OK
            assert vbwd(lib, d=d, causal=causal) == OK
    assert vfwd(lib, Hq=8, Hkv=1) == OK
    assert vbwd(lib, Hq=8, Hkv=1) == OK


@pytest.mark.parametrize("kw", [dict(B=-1), dict(Hq=-4), dict(Hkv=-2), dict(N=-5), dict(d=-64)])
def test_negative_sizes(lib, kw):
    assert vfwd(lib, **kw) == INVALID
    assert vbwd(lib, **kw) == INVALID
    assert b"negative" in lib.fa2_last_error()


@pytest.mark.parametrize("kw", [dict(B=0), dict(Hq=0, Hkv=0), dict(N=0)])
def test_empty_problems_are_ok_with_null_pointers(lib, kw):
    assert vfwd(lib, ptrs=[None] * 5, **kw) == OK
    assert vbwd(lib, ptrs=[None] * 10, ws=0, **kw) == OK
    assert lib.fa2_bwd_workspace_bytes(kw.get("B", 2), kw.get("Hq", 4), kw.get("Hkv", 2),
                                       kw.get("N", 100), 128) == 0


def test_head_grouping(lib):
    assert vfwd(lib, Hq=6, Hkv=4) == INVALID
    assert vbwd(lib, Hq=6, Hkv=4) == INVALID
    assert vfwd(lib, Hq=4, Hkv=0) == INVALID
    assert lib.fa2_bwd_workspace_bytes(2, 6, 4, 100, 128) == 0


@pytest.mark.parametrize("d", [0, 1, 32, 96, 100, 160, 192, 512])
def test_unsupported_head_dims(lib, d):
    assert vfwd(lib, d=d) == UNSUPPORTED
    assert vbwd(lib, d=d) == UNSUPPORTED


@pytest.mark.parametrize("scale", [0.0, -0.1, float("inf"), float("nan"), float("-inf")])
def test_bad_scale(lib, scale):
    assert vfwd(lib, scale=scale) == INVALID
    assert vbwd(lib, scale=scale) == INVALID


@pytest.mark.parametrize("i", range(5))
def test_fwd_null_and_misaligned_pointers(lib, i):
    p = [addr(j) for j in range(5)]
    p[i] = None
    assert vfwd(lib, ptrs=p) == INVALID
    p[i] = addr(i) + 8
    assert vfwd(lib, ptrs=p) == INVALID


@pytest.mark.parametrize("i", range(10))
def test_bwd_null_and_misaligned_pointers(lib, i):
    p = [addr(j) for j in range(10)]
    p[i] = None
    assert vbwd(lib, ptrs=p) == INVALID
    p[i] = addr(i) + (16 if i == 9 else 2)   # workspace needs 256-byte alignment
    assert vbwd(lib, ptrs=p) == INVALID


def test_workspace_size(lib):
    B, Hq, Hkv, N, d = 2, 4, 2, 100, 128
    need = ws_bytes(lib)
    rows = B * Hq * N
    rows_pad = B * Hq * ((N + 63) // 64 * 64)   # per-row arrays padded to 64 rows per head
    def up(x):
        return (x + 255) // 256 * 256
    # The default backward needs the two per-row arrays only.
    assert need == 2 * up(rows_pad * 4)
    assert vbwd(lib, ws=need - 1) == INVALID
    assert b"workspace" in lib.fa2_last_error()
    assert vbwd(lib, ws=need + 12345) == OK
    # The atomic-dQ mode also needs the fp32 dQ accumulator, and is checked against it.
    stages_ws = lib.fa2_bwd_stages_workspace_bytes
    for mask in (1, 2, 4, 7):
        assert stages_ws(mask, B, Hq, Hkv, N, d) == need
    atomic = stages_ws(7 | 8, B, Hq, Hkv, N, d)
    assert atomic == need + up(rows * d * 4)
    assert stages_ws(2 | 8, B, Hq, Hkv, N, d) == atomic
    for bad in (0, 8, 16):
        assert stages_ws(bad, B, Hq, Hkv, N, d) == 0
    p = [addr(i) for i in range(10)]
    st = lib.fa2_bwd_stages(7 | 8, *p, atomic - 1, B, Hq, Hkv, N, 96, 1, 0.125, None)
    assert st == UNSUPPORTED                       # the head dim is checked before the workspace
    st = lib.fa2_bwd_stages(7 | 8, *p, atomic - 1, B, Hq, 3, N, d, 1, 0.125, None)
    assert st == INVALID                           # Hq % Hkv, before any launch


def test_aliasing_is_rejected(lib):
    p = [addr(j) for j in range(5)]
    p[3] = p[0]                    # O = Q
    assert vfwd(lib, ptrs=p) == INVALID
    p = [addr(j) for j in range(5)]
    p[4] = p[2] + 64               # L inside V
    assert vfwd(lib, ptrs=p) == INVALID
    p = [addr(j) for j in range(5)]
    p[4] = p[3] + 256              # L inside O
    assert vfwd(lib, ptrs=p) == INVALID
    for out_i in (6, 7, 8, 9):
        for in_i in range(6):
            p = [addr(j) for j in range(10)]
            p[out_i] = p[in_i]
            assert vbwd(lib, ptrs=p) == INVALID, (out_i, in_i)
    p = [addr(j) for j in range(10)]
    p[7] = p[6]                    # dK = dQ
    assert vbwd(lib, ptrs=p) == INVALID


def test_size_overflow_and_limits(lib):
    big = 2 ** 31 - 1
    assert vfwd(lib, B=big, Hq=big, Hkv=1, N=big, d=256) in (INVALID, UNSUPPORTED)
    assert vfwd(lib, B=1, Hq=1, Hkv=1, N=(1 << 30) + 1, d=64) == UNSUPPORTED
    assert lib.fa2_bwd_workspace_bytes(big, big, 1, big, 256) == 0


def test_full_entry_points_reject_before_any_hip_call(lib):
    # The same checks run first in the real entry points, so these return
    # without touching the (absent) GPU.
    st = lib.fa2_fwd(addr(0), addr(1), addr(2), addr(3), addr(4), 2, 6, 4, 100, 128, 1, 0.1, None)
    assert st == INVALID
    st = lib.fa2_fwd(None, None, None, None, None, 0, 4, 2, 100, 128, 1, 0.1, None)
    assert st == OK
    st = lib.fa2_bwd(*[addr(i) for i in range(10)], 10, 2, 4, 2, 100, 96, 1, 0.1, None)
    assert st == UNSUPPORTED


def test_bwd_stage_mask(lib):
    p = [addr(i) for i in range(10)]
    ws = ws_bytes(lib)
    for bad in (0, 8, 16, 17, 0xFFFFFFFF):
        assert lib.fa2_bwd_stages(bad, *p, ws, 2, 4, 2, 100, 128, 1, 0.125, None) == INVALID
    # valid masks go on to the argument checks (here: an unsupported head dim)
    for good in (1, 2, 3, 4, 5, 6, 7, 9, 10, 15):
        assert lib.fa2_bwd_stages(good, *p, ws, 2, 4, 2, 100, 96, 1, 0.125, None) == UNSUPPORTED


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        fa2.load(str(tmp_path / "nope.so"))


def test_block_sparse_entry_points_check_the_mask_before_any_hip_call(lib):
    q, k, v, o, L = (addr(i) for i in range(5))
    mask = addr(5)
    fwd = lib.fa2_fwd_block_sparse
    # NULL mask with work; an empty problem needs none.
    assert fwd(q, k, v, o, L, None, 2, 4, 2, 300, 128, 1, 0.1, None) == INVALID
    assert fwd(None, None, None, None, None, None, 2, 4, 2, 0, 128, 1, 0.1, None) == OK
    # Sizes the block-sparse kernels do not cover (every head dim is covered; a NULL
    # mask is refused at d = 256 too).
    assert fwd(q, k, v, o, L, None, 2, 4, 2, 300, 256, 1, 0.1, None) == INVALID
    assert fwd(q, k, v, o, L, mask, 2, 4, 2, 300, 96, 1, 0.1, None) == UNSUPPORTED
    assert fwd(q, k, v, o, L, mask, 1, 1, 1, fa2.SPARSE_MAX_N + 1, 64, 1, 0.1, None) == UNSUPPORTED
    assert lib.fa2_fwd_block_sparse_f16(q, k, v, o, L, None, 2, 4, 2, 300, 128, 1, 0.1, None) == INVALID
    # An output overlapping the mask (mask inside O, and inside L).
    assert fwd(q, k, v, o, L, o + 64, 2, 4, 2, 300, 128, 1, 0.1, None) == INVALID
    assert fwd(q, k, v, o, L, L + 8, 2, 4, 2, 300, 128, 0, 0.1, None) == INVALID
    # The dense checks still come first.
    assert fwd(q, k, v, o, L, mask, 2, 6, 4, 300, 128, 1, 0.1, None) == INVALID
    p = [addr(i) for i in range(9)]
    ws = addr(9)
    nbytes = ws_bytes(lib, 2, 4, 2, 300, 128)
    bwd = lib.fa2_bwd_block_sparse
    assert bwd(*p, None, ws, nbytes, 2, 4, 2, 300, 128, 1, 0.1, None) == INVALID
    assert "block_mask" in lib.fa2_last_error().decode()
    nbytes256 = ws_bytes(lib, 2, 4, 2, 300, 256)
    assert bwd(*p, None, ws, nbytes256, 2, 4, 2, 300, 256, 1, 0.1, None) == INVALID
    assert lib.fa2_bwd_block_sparse_f16(*p, addr(10), ws, nbytes256 - 1, 2, 4, 2, 300, 256, 1, 0.1,
                                        None) == INVALID
    assert bwd(*p, p[6] + 16, ws, nbytes, 2, 4, 2, 300, 128, 1, 0.1, None) == INVALID   # inside dQ
    assert bwd(*p, ws + 512, ws, nbytes, 2, 4, 2, 300, 128, 1, 0.1, None) == INVALID    # inside the workspace
    assert bwd(*p, addr(10), ws, nbytes - 1, 2, 4, 2, 300, 128, 1, 0.1, None) == INVALID


def test_noalloc_backward_checks_before_any_hip_call(lib):
    """fa2_bwd_noalloc: the same argument checks as fa2_bwd (no workspace), and problems
    whose per-row scratch exceeds the static array are refused, all before any HIP call."""
    p = [addr(i) for i in range(9)]
    noalloc = lib.fa2_bwd_noalloc
    assert noalloc(*p, 0, 4, 2, 100, 128, 1, 0.125, None) == OK            # empty problem
    assert noalloc(*p, 2, 6, 4, 100, 128, 1, 0.125, None) == INVALID       # Hq % Hkv
    assert noalloc(*p, 2, 4, 2, 100, 96, 1, 0.125, None) == UNSUPPORTED    # head dim
    q = list(p)
    q[6] = q[0]                                                            # dQ = Q
    assert noalloc(*q, 2, 4, 2, 100, 128, 1, 0.125, None) == INVALID
    q = list(p)
    q[2] = None
    assert noalloc(*q, 2, 4, 2, 100, 128, 1, 0.125, None) == INVALID
    # 8 bytes per padded row: 2^21 rows fit 16 MiB, one more 64-row head does not.
    max_rows = fa2.NOALLOC_SCRATCH_BYTES // 8
    assert noalloc(*p, 1, 1, 1, max_rows + 64, 64, 1, 0.125, None) == UNSUPPORTED
    assert b"scratch" in lib.fa2_last_error()
    assert noalloc(*p, 1, 33, 1, 65536, 64, 1, 0.125, None) == UNSUPPORTED


def test_split_o_entry_points_check_before_any_hip_call(lib):
    """fa2_fwd_olo / fa2_bwd_olo / fa2_bwd_stages_olo: the dense checks, then O_lo's own
    (present, 16-byte aligned, overlapping no input; in the forward not O or L, in the
    backward no output and not the workspace), all before any HIP call."""
    q, k, v, o, L, olo = (addr(i) for i in range(6))
    fwd = lib.fa2_fwd_olo
    assert fwd(None, None, None, None, None, None, 0, 4, 2, 100, 128, 1, 0.1, None) == OK   # empty
    assert fwd(q, k, v, o, None, L, 2, 4, 2, 100, 128, 1, 0.1, None) == INVALID
    assert b"O_lo" in lib.fa2_last_error()
    assert fwd(q, k, v, o, olo + 8, L, 2, 4, 2, 100, 128, 1, 0.1, None) == INVALID        # misaligned
    assert fwd(q, k, v, o, q + 1024, L, 2, 4, 2, 100, 128, 1, 0.1, None) == INVALID       # inside Q
    assert fwd(q, k, v, o, v, L, 2, 4, 2, 100, 128, 1, 0.1, None) == INVALID              # = V
    assert fwd(q, k, v, o, o + 4096, L, 2, 4, 2, 100, 128, 1, 0.1, None) == INVALID       # inside O
    assert fwd(q, k, v, o, L - 64, L, 2, 4, 2, 100, 128, 1, 0.1, None) == INVALID         # reaches into L
    assert fwd(q, k, v, o, olo, L, 2, 6, 4, 100, 128, 1, 0.1, None) == INVALID            # Hq % Hkv first
    assert fwd(q, k, v, o, olo, L, 2, 4, 2, 100, 96, 1, 0.1, None) == UNSUPPORTED
    p = [addr(i) for i in range(10)]        # Q K V O L dO dQ dK dV ws
    olo = addr(11)
    nbytes = ws_bytes(lib)

    def bwd(o_lo, ws=p[9], n=nbytes, d=128, Hq=4, stages=None):
        args = (*p[:4], o_lo, *p[4:9], ws, n, 2, Hq, 2, 100, d, 1, 0.125, None)
        if stages is None:
            return lib.fa2_bwd_olo(*args)
        return lib.fa2_bwd_stages_olo(stages, *args)

    assert bwd(None) == INVALID
    assert bwd(olo + 2) == INVALID                       # misaligned
    assert bwd(p[0]) == INVALID                          # = Q
    assert bwd(p[6] + 256) == INVALID                    # inside dQ
    assert bwd(p[8]) == INVALID                          # = dV
    assert bwd(p[9] + 256) == INVALID                    # inside the workspace
    assert bwd(olo, n=nbytes - 1) == INVALID             # workspace too small
    assert bwd(olo, d=96) == UNSUPPORTED
    assert bwd(olo, Hq=6) == INVALID
    for bad in (0, 16, 0xFFFFFFFF):
        assert bwd(olo, stages=bad) == INVALID
    assert bwd(olo, d=96, stages=1) == UNSUPPORTED
