"""The C ABI without a GPU: the library loads, exports every symbol the
header declares, and rejects invalid arguments with the documented status
codes before touching the HIP runtime."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _ensure_built():
    lib_path = os.path.join(ROOT, "io_aware_exact_14_amd", "libfa.so")
    if not os.path.exists(lib_path):
        import importlib.util

        spec = importlib.util.spec_from_file_location("_fa_build", os.path.join(ROOT, "io_aware_exact_14_amd",
                                                                               "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()


@pytest.fixture(scope="module")
def lib():
    _ensure_built()
    from io_aware_exact_14_amd import _lib

    return _lib.load()


@pytest.fixture(scope="module")
def L():
    _ensure_built()
    from io_aware_exact_14_amd import _lib

    return _lib


def _params(L, **kw):
    p = L.FaParams()
    p.B, p.H, p.N, p.d = 2, 3, 100, 64
    p.in_dtype = L.FA_BF16
    p.grad_dtype = L.FA_F32
    p.scale = 0.125
    p.causal = 0
    p.dropout_p = 0.0
    p.seed = 0
    p.block_mask = None
    p.mask_block = 128
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def test_header_declarations_are_exported(lib, L):
    header = open(os.path.join(ROOT, "include", "fa.h")).read()
    declared = set(re.findall(r"^\w[\w\s\*]*?\b(fa_\w+)\s*\(", header, re.M))
    assert declared == set(L.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_abi_version_and_struct_layout(lib, L):
    assert lib.fa_abi_version() == 2
    header = open(os.path.join(ROOT, "include", "fa.h")).read()
    assert "#define FA_ABI_VERSION 2" in header
    # natural C layout of fa_params on x86-64
    assert ctypes.sizeof(L.FaParams) == 80
    assert L.FaParams.dropout_p.offset == 48 and L.FaParams.block_mask.offset == 64


def test_status_strings(lib, L):
    for code in L.STATUS_NAMES:
        s = lib.fa_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.fa_status_string(999).decode() == "unknown status"


def test_header_status_codes_match_binding(L):
    header = open(os.path.join(ROOT, "include", "fa.h")).read()
    for code, name in L.STATUS_NAMES.items():
        assert re.search(rf"\b{name}\s*=\s*{code}\b", header), name


CASES = [
    (dict(d=96), "FA_ERR_HEADDIM"),
    (dict(d=32), "FA_ERR_HEADDIM"),
    (dict(N=-1), "FA_ERR_SHAPE"),
    (dict(B=-2), "FA_ERR_SHAPE"),
    (dict(N=2**31 // 64 + 1), "FA_ERR_SHAPE"),
    (dict(N=2**31 // 256 + 1), "FA_ERR_SHAPE"),        # N*d*4 bytes of a per-head fp32 tensor >= 2^31
    (dict(N=2**31 // 512 + 1, d=128), "FA_ERR_SHAPE"),
    (dict(in_dtype=7), "FA_ERR_DTYPE"),
    (dict(in_dtype=1, grad_dtype=2), "FA_ERR_DTYPE"),
    (dict(scale=0.0), "FA_ERR_SCALE"),
    (dict(scale=-1.0), "FA_ERR_SCALE"),
    (dict(scale=float("inf")), "FA_ERR_SCALE"),
    (dict(scale=float("nan")), "FA_ERR_SCALE"),
    (dict(dropout_p=1.0), "FA_ERR_DROPOUT"),
    (dict(dropout_p=-0.01), "FA_ERR_DROPOUT"),
    (dict(dropout_p=float("nan")), "FA_ERR_DROPOUT"),
    (dict(block_mask=16, mask_block=64), "FA_ERR_MASK"),
    (dict(block_mask=16, mask_block=0), "FA_ERR_MASK"),
]


@pytest.mark.parametrize("kw,status", CASES)
def test_invalid_params_rejected(lib, L, kw, status):
    p = _params(L, **kw)
    assert lib.fa_check_params(ctypes.byref(p)) == L.STATUS[status]
    # the same code from the compute entry points, nothing enqueued
    dummy = 4096
    assert lib.fa_fwd(ctypes.byref(p), dummy, dummy, dummy, dummy, dummy, None) == L.STATUS[status]
    assert lib.fa_bwd(ctypes.byref(p), *([dummy] * 9), dummy, 1 << 30, None) == L.STATUS[status]
    assert lib.fa_bwd_dq(ctypes.byref(p), *([dummy] * 7), dummy, 1 << 30, None) == L.STATUS[status]
    assert lib.fa_bwd_dkdv(ctypes.byref(p), *([dummy] * 7), dummy, 1 << 30, None) == L.STATUS[status]
    assert lib.fa_bwd_noalloc(ctypes.byref(p), *([dummy] * 9), None) == L.STATUS[status]
    assert lib.fa_bwd_workspace_bytes(ctypes.byref(p)) == 0


def test_valid_params_accepted(lib, L):
    for kw in (dict(), dict(d=128), dict(in_dtype=0), dict(in_dtype=1, grad_dtype=1), dict(causal=1),
               dict(N=2**31 // 512 - 1, d=128),
               dict(dropout_p=0.1, seed=2**64 - 1), dict(block_mask=16, mask_block=256), dict(N=0), dict(B=0)):
        assert lib.fa_check_params(ctypes.byref(_params(L, **kw))) == 0, kw


def test_null_and_alignment_rejected(lib, L):
    p = _params(L)
    assert lib.fa_check_params(None) == L.STATUS["FA_ERR_NULL"]
    assert lib.fa_fwd(None, 16, 16, 16, 16, 16, None) == L.STATUS["FA_ERR_NULL"]
    assert lib.fa_fwd(ctypes.byref(p), 16, None, 16, 16, 16, None) == L.STATUS["FA_ERR_NULL"]
    assert lib.fa_fwd(ctypes.byref(p), 16, 24, 16, 16, 16, None) == L.STATUS["FA_ERR_ALIGN"]
    assert lib.fa_bwd(ctypes.byref(p), 16, 16, 16, 16, 16, 16, 16, 16, None, 16, 1 << 20, None) == \
        L.STATUS["FA_ERR_NULL"]
    assert lib.fa_bwd(ctypes.byref(p), *([16] * 8), 8, 16, 1 << 20, None) == L.STATUS["FA_ERR_ALIGN"]


def test_backward_stage_pointer_checks(lib, L):
    p = _params(L)
    ok = [16] * 7
    NULL = L.STATUS["FA_ERR_NULL"]
    for i in range(7):  # Q, K, V, O, LSE, dO, dQ all required by the dQ stage
        args = list(ok)
        args[i] = None
        assert lib.fa_bwd_dq(ctypes.byref(p), *args, 16, 1 << 20, None) == NULL, i
    for i in range(7):  # Q, K, V, LSE, dO, dK, dV all required by the dK/dV stage
        args = list(ok)
        args[i] = None
        assert lib.fa_bwd_dkdv(ctypes.byref(p), *args, 16, 1 << 20, None) == NULL, i
    assert lib.fa_bwd_dq(ctypes.byref(p), *ok, None, 1 << 20, None) == L.STATUS["FA_ERR_WORKSPACE"]
    assert lib.fa_bwd_dkdv(ctypes.byref(p), *ok, 16, 4, None) == L.STATUS["FA_ERR_WORKSPACE"]
    assert lib.fa_bwd_dkdv(ctypes.byref(p), 16, 16, 16, 16, 16, 16, 40, 16, 1 << 20, None) == \
        L.STATUS["FA_ERR_ALIGN"]


def test_workspace_size_and_check(lib, L):
    p = _params(L)
    need = lib.fa_bwd_workspace_bytes(ctypes.byref(p))
    assert need >= 2 * 3 * 100 * 4 and need % 256 == 0
    assert lib.fa_bwd(ctypes.byref(p), *([16] * 9), None, need, None) == L.STATUS["FA_ERR_WORKSPACE"]
    assert lib.fa_bwd(ctypes.byref(p), *([16] * 9), 16, need - 1, None) == L.STATUS["FA_ERR_WORKSPACE"]


def test_dropout_mask_window_checks(lib, L):
    p = _params(L, dropout_p=0.1)
    ok_buf = 4096
    bad = [(2, 0, 0, 1, 0, 1), (0, 3, 0, 1, 0, 1), (0, 0, 99, 2, 0, 1), (0, 0, 0, 1, 100, 1), (0, 0, -1, 1, 0, 1)]
    for b, h, i0, r, j0, c in bad:
        assert lib.fa_dropout_mask(ctypes.byref(p), b, h, i0, r, j0, c, ok_buf, None) == L.STATUS["FA_ERR_RANGE"]
    assert lib.fa_dropout_mask(ctypes.byref(p), 0, 0, 0, 1, 0, 1, None, None) == L.STATUS["FA_ERR_NULL"]
    # empty windows are a no-op
    assert lib.fa_dropout_mask(ctypes.byref(p), 1, 2, 5, 0, 0, 7, ok_buf, None) == 0


def test_empty_problem_is_a_no_op(lib, L):
    p = _params(L, N=0)
    assert lib.fa_fwd(ctypes.byref(p), 16, 16, 16, 16, 16, None) == 0
    assert lib.fa_bwd(ctypes.byref(p), *([16] * 9), None, 0, None) == 0


def test_noalloc_entry_point_host_checks(lib, L):
    # fa_bwd_noalloc rejects, before any HIP call: missing pointers, and
    # B*H*N beyond its fixed scratch (FA_BWD_NOALLOC_MAX_ROWS fp32 rows)
    header = open(os.path.join(ROOT, "include", "fa.h")).read()
    assert "#define FA_BWD_NOALLOC_MAX_ROWS (1 << 22)" in header
    assert L.BWD_NOALLOC_MAX_ROWS == 1 << 22
    p = _params(L)
    for i in range(9):  # Q, K, V, O, LSE, dO, dQ, dK, dV
        args = [16] * 9
        args[i] = None
        assert lib.fa_bwd_noalloc(ctypes.byref(p), *args, None) == L.STATUS["FA_ERR_NULL"], i
    assert lib.fa_bwd_noalloc(None, *([16] * 9), None) == L.STATUS["FA_ERR_NULL"]
    big = _params(L, B=1, H=64, N=65537)  # 4194368 rows > 2^22
    assert lib.fa_check_params(ctypes.byref(big)) == 0
    assert lib.fa_bwd_noalloc(ctypes.byref(big), *([16] * 9), None) == L.STATUS["FA_ERR_SCRATCH"]
    big2 = _params(L, B=4, H=16, N=65537, d=128)
    assert lib.fa_bwd_noalloc(ctypes.byref(big2), *([16] * 9), None) == L.STATUS["FA_ERR_SCRATCH"]
    # an empty problem is a no-op (no scratch lookup, nothing enqueued)
    assert lib.fa_bwd_noalloc(ctypes.byref(_params(L, N=0)), *([16] * 9), None) == 0
