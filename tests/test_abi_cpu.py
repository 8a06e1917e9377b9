"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every entry point declared in include/pisa.h, its geometry helpers agree with
the oracle's independent ones, and invalid arguments are rejected on the host
with the documented status before anything is launched."""
import ctypes
import os
import re

import pytest

import oracle
from hierarchical_block_sparse_mean_amd import pisa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "pisa.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(pisa_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pisa.LIB_PATH):
        from hierarchical_block_sparse_mean_amd.build import build_library
        build_library()
    return pisa.load()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert len(names) >= 14
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(pisa.EXPORTS)
    assert lib.pisa_version().decode().startswith("pisa-mi355x")


@pytest.mark.parametrize("n,C", [(1, 64), (64, 64), (65, 64), (1000, 64), (1024, 64), (131072, 64), (262144, 128),
                                 (131073, 64), (7, 3), (330, 64)])
def test_geometry_matches_oracle(lib, n, C):
    L = lib.pisa_levels(n, C)
    assert L == oracle.levels(n, C)
    off = 0
    for l in range(1, L + 1):
        assert lib.pisa_level_rows(n, C, l) == oracle.level_rows(n, C, l)
        assert lib.pisa_level_offset(n, C, l) == off
        off += lib.pisa_level_rows(n, C, l)
    assert lib.pisa_level_offset(n, C, L + 1) == -1


def test_level_rows_far_above_the_top(lib):
    """Blocks of C 2^(l-1) tokens beyond 64 bits: one row, no overflow."""
    assert lib.pisa_level_rows(1000, 128, 62) == 1
    assert lib.pisa_level_rows(1000, 2 ** 31 - 1, 40) == 1
    assert lib.pisa_level_rows(2 ** 62, 1, 62) == 2
    assert lib.pisa_level_rows(2 ** 62 + 1, 1, 62) == 3
    assert lib.pisa_level_rows(1000, 64, 63) == 0  # beyond the documented range


def _p(**kw):
    base = dict(B=1, N=1024, Hq=4, Hkv=1, D=64, C=64, K=4, causal=False, dtype="f32")
    base.update(kw)
    return pisa.Problem(**base)


FAKE = 4096  # a non-NULL address; validation must reject before using it


@pytest.mark.parametrize("kw,status", [
    (dict(Hq=6, Hkv=4), pisa.PISA_ERR_INVALID_ARG),
    (dict(N=0), pisa.PISA_ERR_INVALID_ARG),
    (dict(K=0), pisa.PISA_ERR_INVALID_ARG),
    (dict(C=0), pisa.PISA_ERR_INVALID_ARG),
    (dict(g=3), pisa.PISA_ERR_UNSUPPORTED),
    (dict(D=96), pisa.PISA_ERR_UNSUPPORTED),
    (dict(Hq=12, Hkv=4), pisa.PISA_ERR_UNSUPPORTED),
    (dict(K=33), pisa.PISA_ERR_UNSUPPORTED),
    (dict(C=256), pisa.PISA_ERR_UNSUPPORTED),
    (dict(N=1 << 26, K=1), pisa.PISA_ERR_UNSUPPORTED),
    # a head's summary rows x D must stay below 2^31 (32-bit offsets in a head)
    (dict(N=1 << 25, C=1, K=1), pisa.PISA_ERR_UNSUPPORTED),
    (dict(cap=(1 << 31) - 1), pisa.PISA_ERR_UNSUPPORTED),
    # B*Hkv*N*K far beyond 64 bits (a plain int64 product would wrap negative)
    (dict(B=2 ** 31 - 1, Hq=2 ** 30, Hkv=2 ** 30, N=2 ** 25, K=32), pisa.PISA_ERR_UNSUPPORTED),
    # k/v beyond 2^46 elements through cap, with B*Hkv*N*K within 2^31
    (dict(B=2 ** 16, Hq=2 ** 10, Hkv=2 ** 10, N=1, K=1, C=128, cap=2 ** 30), pisa.PISA_ERR_UNSUPPORTED),
    (dict(cap=100), pisa.PISA_ERR_INVALID_ARG),
    (dict(q_tile=3), pisa.PISA_ERR_UNSUPPORTED),
    (dict(q_tile=8), pisa.PISA_ERR_UNSUPPORTED),  # two tiles per read: bf16 only
    (dict(q_tile=8, dtype="bf16", C=48), pisa.PISA_ERR_UNSUPPORTED),  # and whole 16-key blocks per leaf
    (dict(select_algo=7), pisa.PISA_ERR_INVALID_ARG),
    (dict(attn_algo=-1), pisa.PISA_ERR_INVALID_ARG),
    (dict(scale=-1.0), pisa.PISA_ERR_INVALID_ARG),
])
def test_invalid_problem_rejected(lib, kw, status):
    p = _p(**kw).c()
    rc = lib.pisa_build_pyramid(ctypes.byref(p), FAKE, FAKE, None)
    assert rc == status, lib.pisa_last_error()
    assert lib.pisa_last_error()
    assert lib.pisa_select(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None) == status
    assert lib.pisa_pyramid_bytes(ctypes.byref(p)) == 0


def test_summary_offset_bound_boundary(lib):
    """Shapes whose per-head summary elements reach 2^31 are rejected, and
    the largest accepted cap at C = 64, D = 64 sits just below that."""
    def rows(cap, C):
        return sum(oracle.level_rows(cap, C, l) for l in range(1, oracle.levels(cap, C) + 1))
    ok_cap = (1 << 30)  # rows = 2^25 - 1, x 64 = 2^31 - 64
    assert rows(ok_cap, 64) * 64 < 2 ** 31
    p = _p(cap=ok_cap).c()
    assert lib.pisa_pyramid_bytes(ctypes.byref(p)) > 0, lib.pisa_last_error()
    bad_cap = ok_cap + 64 * 2 ** 6  # 64 more leaves: 146 more rows, past the bound
    assert rows(bad_cap, 64) * 64 >= 2 ** 31
    p = _p(cap=bad_cap).c()
    assert lib.pisa_pyramid_bytes(ctypes.byref(p)) == 0
    assert "2^31" in lib.pisa_last_error().decode()


@pytest.mark.parametrize("kw", [dict(q_tile=4), dict(q_tile=8, dtype="bf16"), dict(q_tile=0, dtype="bf16"),
                                dict(q_tile=2, Hq=8, Hkv=1, dtype="bf16", C=128)])
def test_q_tile_schedules_accepted(lib, kw):
    p = _p(**kw).c()
    assert lib.pisa_select_workspace_bytes(ctypes.byref(p)) > 0, lib.pisa_last_error()


def test_null_pointers_and_small_workspace(lib):
    p = _p().c()
    assert lib.pisa_build_pyramid(ctypes.byref(p), None, FAKE, None) == pisa.PISA_ERR_INVALID_ARG
    assert lib.pisa_select(ctypes.byref(p), FAKE, None, FAKE, FAKE, None, FAKE, 1 << 40, None) == pisa.PISA_ERR_INVALID_ARG
    need = lib.pisa_select_workspace_bytes(ctypes.byref(p))
    assert need > 0
    assert lib.pisa_select(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, FAKE, need - 1, None) == pisa.PISA_ERR_WORKSPACE
    assert "workspace" in lib.pisa_last_error().decode()
    assert lib.pisa_sparse_attn(ctypes.byref(p), FAKE, FAKE, None, FAKE, FAKE, None, FAKE, 256, None) == \
        pisa.PISA_ERR_INVALID_ARG
    need_a = lib.pisa_attn_workspace_bytes(ctypes.byref(p))
    assert need_a > 256
    assert lib.pisa_sparse_attn(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, need_a - 1, None) == \
        pisa.PISA_ERR_WORKSPACE
    assert lib.pisa_flat_select(ctypes.byref(p), None, FAKE, FAKE, None, FAKE, 256, None) == pisa.PISA_ERR_INVALID_ARG
    assert lib.pisa_build_pyramid(None, FAKE, FAKE, None) == pisa.PISA_ERR_INVALID_ARG


def test_noalloc_select_host_checks(lib):
    """pisa_select_noalloc validates like pisa_select and refuses, before any
    device work, a problem whose workspace exceeds the library's scratch."""
    small = _p().c()
    assert lib.pisa_select_noalloc(ctypes.byref(small), FAKE, None, FAKE, FAKE, None, None) == \
        pisa.PISA_ERR_INVALID_ARG
    assert lib.pisa_select_noalloc(None, FAKE, FAKE, FAKE, FAKE, None, None) == pisa.PISA_ERR_INVALID_ARG
    big = pisa.Problem(B=1, N=131072, Hq=32, Hkv=8, D=128, C=64, K=16, causal=True, dtype="bf16")
    assert pisa.select_workspace_bytes(big) > pisa.NOALLOC_SCRATCH_BYTES
    assert lib.pisa_select_noalloc(ctypes.byref(big.c()), FAKE, FAKE, FAKE, FAKE, None, None) == \
        pisa.PISA_ERR_WORKSPACE
    assert b"scratch" in lib.pisa_last_error()
    fits = pisa.Problem(B=1, N=32768, Hq=32, Hkv=8, D=128, C=64, K=16, causal=True, dtype="bf16")
    assert pisa.select_workspace_bytes(fits) <= pisa.NOALLOC_SCRATCH_BYTES
    with open(os.path.join(ROOT, "include", "pisa.h")) as f:
        assert "#define PISA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)" in f.read()
    assert pisa.NOALLOC_SCRATCH_BYTES == 128 << 20


def test_backward_shape_limit(lib):
    """fp32 rows of d = 128 with C > 64 are rejected by the backward before
    any pointer is used; the forward and the other shapes are accepted."""
    big = _p(D=128, C=128).c()
    assert lib.pisa_attn_backward_workspace_bytes(ctypes.byref(big)) == 0
    args = [FAKE] * 10 + [FAKE, 1 << 40, None]
    assert lib.pisa_sparse_attn_backward(ctypes.byref(big), *args) == pisa.PISA_ERR_UNSUPPORTED
    assert "C <= 64" in lib.pisa_last_error().decode()
    assert lib.pisa_attn_workspace_bytes(ctypes.byref(big)) > 0
    for kw in (dict(D=128, C=64), dict(D=64, C=128), dict(D=128, C=128, dtype="bf16")):
        assert lib.pisa_attn_backward_workspace_bytes(ctypes.byref(_p(**kw).c())) > 0, kw


def test_decode_validation(lib):
    d = pisa.DecodeProblem(S=2, cap=100, Hq=4, Hkv=1, D=64, C=64, K=4, dtype="f32")
    args = [FAKE] * 7
    assert lib.pisa_decode_step(None, *args, FAKE, None, None, None, None) == pisa.PISA_ERR_INVALID_ARG
    bad = pisa.DecodeProblem(S=2, cap=100, Hq=4, Hkv=1, D=64, C=64, K=64, dtype="f32").c()
    assert lib.pisa_decode_step(ctypes.byref(bad), *args, FAKE, None, None, None, None) == pisa.PISA_ERR_UNSUPPORTED
    bad = pisa.DecodeProblem(S=2, cap=100, Hq=4, Hkv=1, D=64, C=64, K=4, dtype="f32").c()
    assert lib.pisa_decode_step(ctypes.byref(bad), FAKE, None, *([FAKE] * 5), FAKE, None, None, None, None) == \
        pisa.PISA_ERR_INVALID_ARG
    # caches beyond 2^46 elements (S*Hkv*cap*D, a product past 64 bits)
    big = pisa.DecodeProblem(S=2 ** 31 - 1, cap=2 ** 31 - 1, Hq=2 ** 30, Hkv=2 ** 30, D=128, C=64, K=4,
                             dtype="bf16").c()
    assert lib.pisa_decode_step(ctypes.byref(big), *args, FAKE, None, None, None, None) == pisa.PISA_ERR_UNSUPPORTED
    assert "2^46" in lib.pisa_last_error().decode()


def test_pyramid_bytes(lib):
    p = _p(N=1000, cap=1100)
    rows = sum(oracle.level_rows(1100, 64, l) for l in range(1, oracle.levels(1100, 64) + 1))
    assert lib.pisa_pyramid_bytes(ctypes.byref(p.c())) == rows * (64 * 6 + 4)


def test_product_has_no_oracle_dependency():
    pkg = os.path.join(ROOT, "hierarchical_block_sparse_mean_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp", ".c")):
                with open(os.path.join(dirpath, fn)) as f:
                    text = f.read()
                assert "import oracle" not in text and "from oracle" not in text, fn
                assert "pisa_oracle" not in text and "libpisa_oracle" not in text, fn


def test_probe_stream_host_checks(lib):
    """The streaming probe rejects, before any launch, a missing source, a size
    that is not a positive multiple of 16, an unknown mode, a missing
    destination (copy) or sink (read), a bad grid and misaligned pointers."""
    ok_ptr = ctypes.c_void_p(1 << 20)
    bad = [
        (None, ok_ptr, 1 << 20, 0, 4, ok_ptr),
        (ok_ptr, ok_ptr, 0, 0, 4, ok_ptr),
        (ok_ptr, ok_ptr, 1000, 0, 4, ok_ptr),
        (ok_ptr, ok_ptr, 1 << 20, 2, 4, ok_ptr),
        (ok_ptr, None, 1 << 20, 1, 4, None),
        (ok_ptr, None, 1 << 20, 0, 4, None),
        (ok_ptr, ok_ptr, 1 << 20, 0, 0, ok_ptr),
        (ctypes.c_void_p((1 << 20) + 8), ok_ptr, 1 << 20, 1, 4, None),
    ]
    for src, dst, nbytes, mode, wgs, sink in bad:
        assert lib.pisa_probe_stream(src, dst, nbytes, mode, wgs, sink, None) == pisa.PISA_ERR_INVALID_ARG
