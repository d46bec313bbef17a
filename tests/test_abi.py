"""C-ABI checks that need no GPU: the library loads, exports every function
include/h2o.h declares, sizes workspaces, and rejects bad arguments on the
host before enqueuing anything (no kernel is launched by these tests)."""
import ctypes
import os
import re

import pytest

from h2o_kv_cache_amd import _lib
from h2o_kv_cache_amd._lib import H2OShape

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "h2o.h")


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


# The argument-rejection tests pass made-up device addresses and rely on the
# host-side checks returning before any launch; where a GPU is visible a
# regressed check could launch a kernel on them, so they run only where no
# GPU is present (the CPU suite).
pytestmark = pytest.mark.skipif(_gpu_visible(), reason="fake device addresses: CPU-only suite")


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s+\**\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = _declared_functions()
    assert set(names) == set(_lib.EXPORTED), names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def _shape(**kw):
    d = dict(batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128, cache_len=16384,
             chunk_len=1024, n_valid=16384, scale=0.0)
    d.update(kw)
    return H2OShape(**d)


def test_status_strings(lib):
    for st in range(5):
        assert lib.h2o_status_string(st)
    assert lib.h2o_status_string(99) == b"unknown status"


def test_workspace_size_depends_on_shape_not_fill(lib):
    a = lib.h2o_workspace_size(ctypes.byref(_shape(n_valid=0)))
    b = lib.h2o_workspace_size(ctypes.byref(_shape(n_valid=16384)))
    c = lib.h2o_workspace_size(ctypes.byref(_shape(n_valid=777)))
    assert a == b == c > 0
    assert a % 256 == 0


@pytest.mark.parametrize("bad", [
    dict(batch=0), dict(n_q_heads=0), dict(n_kv_heads=0), dict(n_q_heads=12, n_kv_heads=8),
    dict(cache_len=0), dict(chunk_len=0), dict(chunk_len=20000), dict(n_valid=-1),
    dict(n_valid=16385), dict(scale=float("nan"))])
def test_invalid_shapes_rejected(lib, bad):
    sh = _shape(**bad)
    assert lib.h2o_workspace_size(ctypes.byref(sh)) == 0
    P = ctypes.c_void_p(256)
    st = lib.h2o_attn_chunk(ctypes.byref(sh), P, P, P, P, P, P, P, P, P, 1 << 40, None)
    assert st == _lib.H2O_ERR_INVALID_ARG
    assert lib.h2o_score_accumulate(ctypes.byref(sh), P, P, P, None) == _lib.H2O_ERR_INVALID_ARG
    assert lib.h2o_evict_select(ctypes.byref(sh), P, P, None) == _lib.H2O_ERR_INVALID_ARG
    assert lib.kv_scatter(ctypes.byref(sh), P, P, P, P, P, P, P, P, 0, None) == _lib.H2O_ERR_INVALID_ARG


@pytest.mark.parametrize("bad", [dict(head_dim=96), dict(cache_len=(1 << 20) + 1, n_valid=0)])
def test_unsupported_shapes(lib, bad):
    sh = _shape(**bad)
    assert lib.h2o_workspace_size(ctypes.byref(sh)) == 0
    P = ctypes.c_void_p(256)
    assert lib.h2o_evict_select(ctypes.byref(sh), P, P, None) == _lib.H2O_ERR_UNSUPPORTED


def test_null_shape(lib):
    P = ctypes.c_void_p(256)
    assert lib.h2o_workspace_size(None) == 0
    assert lib.h2o_evict_select(None, P, P, None) == _lib.H2O_ERR_INVALID_ARG


def test_null_and_misaligned_pointers(lib):
    sh = _shape()
    A = ctypes.c_void_p(4096)
    M = ctypes.c_void_p(4098)          # not 16-byte aligned
    N = ctypes.c_void_p(None)
    ws = lib.h2o_workspace_size(ctypes.byref(sh))
    # attention: each required pointer null / misaligned in turn
    for k in range(8):
        for bad in (N, M):
            if k == 6 and bad is N:
                continue  # lse may be NULL
            args = [A] * 8
            args[k] = bad
            st = lib.h2o_attn_chunk(ctypes.byref(sh), *args, A, ws, None)
            assert st == _lib.H2O_ERR_INVALID_ARG, (k, bad)
    assert lib.h2o_score_accumulate(ctypes.byref(sh), A, N, A, None) == _lib.H2O_ERR_INVALID_ARG
    assert lib.h2o_score_accumulate(ctypes.byref(sh), A, A, M, None) == _lib.H2O_ERR_INVALID_ARG
    assert lib.h2o_evict_select(ctypes.byref(sh), N, A, None) == _lib.H2O_ERR_INVALID_ARG
    assert lib.h2o_evict_select(ctypes.byref(sh), A, M, None) == _lib.H2O_ERR_INVALID_ARG
    for k in range(8):
        for bad in (N, M):
            if k == 3 and bad is N:
                continue  # pos may be NULL
            args = [A] * 8
            args[k] = bad
            assert lib.kv_scatter(ctypes.byref(sh), *args, 0, None) == _lib.H2O_ERR_INVALID_ARG
    assert lib.kv_scatter(ctypes.byref(sh), *([A] * 8), -1, None) == _lib.H2O_ERR_INVALID_ARG


def test_workspace_checks(lib):
    sh = _shape()
    A = ctypes.c_void_p(4096)
    need = lib.h2o_workspace_size(ctypes.byref(sh))
    assert lib.h2o_attn_chunk(ctypes.byref(sh), *([A] * 8), None, need, None) == _lib.H2O_ERR_WORKSPACE
    assert lib.h2o_attn_chunk(ctypes.byref(sh), *([A] * 8), A, need - 1, None) == _lib.H2O_ERR_WORKSPACE
    assert lib.h2o_attn_chunk(ctypes.byref(sh), *([A] * 8), ctypes.c_void_p(4096 + 16), need,
                              None) == _lib.H2O_ERR_WORKSPACE


def test_backward_argument_checks(lib):
    sh = _shape()
    A = ctypes.c_void_p(4096)
    M = ctypes.c_void_p(4098)
    N = ctypes.c_void_p(None)
    need = lib.h2o_attn_bwd_workspace_size(ctypes.byref(sh))
    assert need > 0 and need % 256 == 0
    assert need == lib.h2o_attn_bwd_workspace_size(ctypes.byref(_shape(n_valid=0)))
    # every tensor pointer is required and must be 16-byte aligned
    for k in range(13):
        for bad in (N, M):
            args = [A] * 13
            args[k] = bad
            st = lib.h2o_attn_chunk_bwd(ctypes.byref(sh), *args, A, need, None)
            assert st == _lib.H2O_ERR_INVALID_ARG, (k, bad)
    assert lib.h2o_attn_chunk_bwd(ctypes.byref(sh), *([A] * 13), None, need,
                                  None) == _lib.H2O_ERR_WORKSPACE
    assert lib.h2o_attn_chunk_bwd(ctypes.byref(sh), *([A] * 13), A, need - 1,
                                  None) == _lib.H2O_ERR_WORKSPACE
    bad = _shape(head_dim=96)
    assert lib.h2o_attn_bwd_workspace_size(ctypes.byref(bad)) == 0
    assert lib.h2o_attn_chunk_bwd(ctypes.byref(bad), *([A] * 13), A, need,
                                  None) == _lib.H2O_ERR_UNSUPPORTED
    assert lib.h2o_attn_chunk_bwd(ctypes.byref(_shape(n_q_heads=12)), *([A] * 13), A, need,
                                  None) == _lib.H2O_ERR_INVALID_ARG


def test_snapkv_argument_checks(lib):
    sh = _shape(cache_len=8192, n_valid=8000, chunk_len=1024)
    D, C, S, BH = 128, 8192, 1024, 8
    A = ctypes.c_void_p(1 << 32)                       # input caches / chunk
    O = ctypes.c_void_p((1 << 32) + (1 << 30))         # output cache, disjoint
    O2 = ctypes.c_void_p((1 << 32) + (1 << 31))
    M = ctypes.c_void_p((1 << 32) + 2)
    N = ctypes.c_void_p(None)
    I = _lib.H2O_ERR_INVALID_ARG
    sel = lambda budget, w=A, k=A: lib.h2o_snapkv_select(ctypes.byref(sh), w, budget, k, None)
    for budget in (-1, 8001):
        assert sel(budget) == I
    assert sel(10, w=N) == I and sel(10, w=M) == I
    assert sel(10, k=N) == I and sel(10, k=M) == I
    # budget 0 needs no keep list; a bad shape is rejected before anything else
    assert lib.h2o_snapkv_select(ctypes.byref(_shape(head_dim=96)), A, 0, N,
                                 None) == _lib.H2O_ERR_UNSUPPORTED

    def comp(budget=4000, out_len=5024, k_out=O, v_out=O2, pos=A, pos_out=A, p0=8000,
             ins=None):
        ins = ins or [A] * 7   # k_cache, v_cache, pos, k_new, v_new, wsum, keep_idx
        ins = list(ins)
        ins[2] = pos
        return lib.h2o_snapkv_compact(ctypes.byref(sh), *ins, budget, out_len, p0, k_out, v_out,
                                      pos_out, N, None)
    assert comp(out_len=5023) == I          # budget + S > out_len
    assert comp(budget=8001) == I
    assert comp(p0=-1) == I
    assert comp(pos=N, pos_out=A) == I      # positions out need positions in
    for k in (0, 1, 3, 4, 5, 6):
        for bad in (N, M):
            ins = [A] * 7
            ins[k] = bad
            assert comp(ins=ins) == I, (k, bad)
    assert comp(k_out=N) == I and comp(v_out=M) == I
    # the output cache may not overlap an input (k_out placed on the chunk rows)
    assert comp(k_out=A) == I
    assert comp(k_out=O, v_out=ctypes.c_void_p((1 << 32) + (1 << 30) + 4096)) == I


def test_binding_argument_counts_match_the_header(lib):
    # every ctypes declaration takes as many arguments as include/h2o.h says
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    for name in _declared_functions():
        m = re.search(rf"\b{name}\s*\(([^)]*)\)\s*;", text, flags=re.S)
        assert m, name
        params = [p for p in m.group(1).split(",") if p.strip() and p.strip() != "void"]
        argtypes = getattr(lib, name).argtypes
        assert argtypes is not None and len(argtypes) == len(params), (name, len(params))


def test_static_scratch_entry_point_checks(lib):
    # argument and size checks of the no-workspace attention happen on the
    # host before the device scratch is looked up or anything is enqueued
    A = ctypes.c_void_p(4096)
    M = ctypes.c_void_p(4098)
    N = ctypes.c_void_p(None)
    sh = _shape()
    assert lib.h2o_workspace_size(ctypes.byref(sh)) <= _lib.STATIC_SCRATCH_BYTES
    for k in range(8):
        for bad in (N, M):
            if k == 6 and bad is N:
                continue  # lse may be NULL
            args = [A] * 8
            args[k] = bad
            st = lib.h2o_attn_chunk_static(ctypes.byref(sh), *args, None)
            assert st == _lib.H2O_ERR_INVALID_ARG, (k, bad)
    for bad in (dict(batch=0), dict(n_valid=16385), dict(n_q_heads=12)):
        assert lib.h2o_attn_chunk_static(ctypes.byref(_shape(**bad)), *([A] * 8),
                                         None) == _lib.H2O_ERR_INVALID_ARG
    assert lib.h2o_attn_chunk_static(ctypes.byref(_shape(head_dim=96)), *([A] * 8),
                                     None) == _lib.H2O_ERR_UNSUPPORTED
    # a shape whose workspace exceeds the static scratch (a 130048-slot cache
    # with a 1024-token window) is refused
    big = _shape(cache_len=130048, n_valid=130048)
    assert lib.h2o_workspace_size(ctypes.byref(big)) > _lib.STATIC_SCRATCH_BYTES
    assert lib.h2o_attn_chunk_static(ctypes.byref(big), *([A] * 8),
                                     None) == _lib.H2O_ERR_WORKSPACE


def test_static_scratch_size_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define H2O_STATIC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.STATIC_SCRATCH_BYTES
