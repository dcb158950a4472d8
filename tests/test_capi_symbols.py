"""The C-ABI library loads and exports every function include/nestspec.h declares (CPU only).

No compute call is made. Only host-side argument checks run: they return an
error status before any HIP call.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nestspec.h")
LIB = os.path.join(ROOT, "nested_quantized_weights_amd", "libnestspec.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.skip("libnestspec.so not built (run __graft_entry__.build())")
    return ctypes.CDLL(LIB)


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("nest_pack", "nest_act_quant", "draft_gemv", "verify_gemm", "verify_accept",
                     "kv_nest_pack", "kv_nest_attend", "nest_last_error",
                     "draft_gemv_workspace_size", "verify_accept_workspace_size",
                     "verify_gemm_workspace_size", "kv_nest_attend_workspace_size"):
        assert required in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_binding_covers_every_symbol():
    from nested_quantized_weights_amd import nestspec

    assert sorted(nestspec.SYMBOLS) == declared_functions()


def test_host_validation_reports_errors_without_a_gpu(lib):
    lib.nest_last_error.restype = ctypes.c_char_p
    f = lib.nest_pack
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    assert f(None, 4, 8, 4, None, None, None, None) == 1  # NEST_EINVAL: null pointer
    assert b"null" in lib.nest_last_error()
    dummy = ctypes.c_void_p(16)
    assert f(dummy, 4, 10, 4, dummy, dummy, dummy, None) == 3  # NEST_ESHAPE: 4 does not divide 10
    g = lib.draft_gemv
    g.restype = ctypes.c_int
    g.argtypes = [ctypes.c_void_p] * 2 + [ctypes.c_int64] * 2 + [ctypes.c_void_p] * 2 + \
        [ctypes.c_int64] * 2 + [ctypes.c_void_p] * 4 + [ctypes.c_size_t, ctypes.c_void_p]
    assert g(dummy, dummy, 1, 256, dummy, dummy, 16, 64, dummy, None, None, None, 0, None) == 5
    assert g(dummy, dummy, 1, 200, dummy, dummy, 16, 128, dummy, None, None, None, 0, None) == 3
    assert g(ctypes.c_void_p(17), dummy, 1, 256, dummy, dummy, 16, 128, dummy, None, None, None, 0,
             None) == 2  # NEST_EALIGN
    assert g(dummy, dummy, 1, 256, dummy, dummy, 16, 128, None, dummy, None, None, 0, None) == 4
    ws = lib.verify_accept_workspace_size
    ws.restype = ctypes.c_size_t
    ws.argtypes = [ctypes.c_int64] * 3
    assert ws(1, 8, 152064) > 0
    # more than 16 rows go through the batched kernel, which writes y: a
    # call without y is refused before anything runs; the accept workspace
    # holds one argmax key per row
    p = ctypes.c_void_p(256)
    assert g(p, p, 17, 256, p, p, 16, 128, None, p, None, p, 1 << 20, None) == 1  # NEST_EINVAL
    assert b"need y" in lib.nest_last_error()
    va = lib.verify_accept
    va.restype = ctypes.c_int
    va.argtypes = [ctypes.c_void_p] * 2 + [ctypes.c_int64] * 3 + [ctypes.c_void_p] * 3 + \
        [ctypes.c_int64] * 2 + [ctypes.c_void_p] * 7 + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    assert va(p, p, 2, 8, 256, p, p, p, 1000, 128, p, p, p, p, None, None, None, p, 1 << 20, None) == 1
    assert b"need y" in lib.nest_last_error()
    # over 16 rows: the row argmax's chunk keys (8 chunks of each of the 144 rows of
    # 152064 logits; one chunk of 1000) and the row indices after the counter zone
    assert ws(16, 8, 152064) >= 4352 + 144 * 8 * 8 + 144 * 4 and ws(16, 8, 1000) >= 4352 + 144 * (8 + 4)


class _KV(ctypes.Structure):
    _fields_ = [("k_base", ctypes.c_void_p), ("k_refine", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
                ("v_base", ctypes.c_void_p), ("v_refine", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("n_kv_heads", ctypes.c_int64), ("head_dim", ctypes.c_int64), ("capacity", ctypes.c_int64),
                ("block", ctypes.c_int64)]


def test_attend_host_validation_without_a_gpu(lib):
    # kv_nest_attend checks its arguments (including a 16-byte aligned
    # query: the kernels read it in 16-byte pieces) before any HIP call
    lib.nest_last_error.restype = ctypes.c_char_p
    f = lib.kv_nest_attend
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.POINTER(_KV), ctypes.c_void_p,
                  ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    p = ctypes.c_void_p(256)
    kv = _KV(256, 256, 256, 256, 256, 256, 8, 128, 32768, 128)
    ws = 1 << 24
    assert f(ctypes.c_void_p(258), 1, 32, ctypes.byref(kv), None, 4096, 0, p, p, ws, None) == 2  # NEST_EALIGN
    assert b"q must be 16-byte aligned" in lib.nest_last_error()
    assert f(p, 1, 30, ctypes.byref(kv), None, 4096, 0, p, p, ws, None) == 3  # NEST_ESHAPE: 8 does not divide 30
    assert f(p, 1, 32, ctypes.byref(kv), None, 4096, 2, p, p, ws, None) == 1  # NEST_EINVAL: view
    assert f(p, 1, 32, ctypes.byref(kv), None, 40000, 0, p, p, ws, None) == 1  # ctx_len > capacity
    # more query rows than one launch holds are taken in chunks of queries,
    # but one query's GQA group must fit a launch (64 rows)
    assert f(p, 1, 8 * 65, ctypes.byref(kv), None, 4096, 1, p, p, ws, None) == 5  # NEST_EUNSUPPORTED
    assert f(p, 1, 32, ctypes.byref(kv), None, 4096, 0, p, p, 16, None) == 4  # NEST_EWORKSPACE
    # with the length on the device the host value is an offset, and the
    # workspace must cover the whole capacity
    sz = lib.kv_nest_attend_workspace_size
    sz.restype = ctypes.c_size_t
    sz.argtypes = [ctypes.c_int64] * 5
    small, full = sz(1, 32, 8, 128, 4096), sz(1, 32, 8, 128, 32768)
    assert 0 < small < full
    assert f(p, 1, 32, ctypes.byref(kv), p, 0, 0, p, p, small, None) == 4
    assert f(p, 1, 32, ctypes.byref(kv), p, -1, 0, p, p, full, None) == 1  # negative offset
    # the exact entry's workspace adds one rebuilt open block (32 KB) and
    # two scales per (query, kv head) to the partials of the one-query split
    ex = lib.kv_nest_attend_exact_workspace_size
    ex.restype = ctypes.c_size_t
    ex.argtypes = [ctypes.c_int64] * 5
    assert ex(1, 32, 8, 128, 32768) == full
    assert ex(5, 32, 8, 128, 32768) >= 5 * full + 5 * 8 * (32768 + 8)
    assert ex(129, 32, 8, 128, 32768) == 0 and ex(5, 30, 8, 128, 32768) == 0


def test_workspaces_are_checked_without_a_gpu(lib):
    # the fp32-activation GEMVs need the caller's workspace (block counter,
    # argmax keys, quantize-first codes), 256-byte aligned; nothing runs
    # before these checks
    lib.nest_last_error.restype = ctypes.c_char_p
    sz = lib.nest_gemv_x_workspace_size
    sz.restype = ctypes.c_size_t
    sz.argtypes = [ctypes.c_int64] * 3
    need = sz(5, 3584, 37888)
    assert need >= 256 + 5 * 3584 and sz(0, 1, 1) == 0
    g = lib.verify_gemm_x
    g.restype = ctypes.c_int
    g.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64] + [ctypes.c_void_p] * 3 + \
        [ctypes.c_int64] * 2 + [ctypes.c_void_p] * 2 + [ctypes.c_size_t, ctypes.c_void_p]
    p = ctypes.c_void_p(256)
    assert g(p, 5, 3584, p, p, p, 37888, 128, p, None, 0, None) == 4  # NEST_EWORKSPACE
    assert b"workspace needs" in lib.nest_last_error()
    assert g(p, 5, 3584, p, p, p, 37888, 128, p, ctypes.c_void_p(272), need, None) == 2  # not 256-aligned
    # the batched verify splits the groups of few, long weight rows over
    # several blocks and needs a workspace for their sums (counters + one
    # 64 x 144 fp32 slot per block); other shapes need none
    vs = lib.verify_gemm_workspace_size
    vs.restype = ctypes.c_size_t
    vs.argtypes = [ctypes.c_int64] * 3
    down = vs(144, 14336, 4096)
    assert down >= 64 * 2 * 64 * 144 * 4
    assert vs(5, 14336, 4096) == 0 and vs(144, 4096, 14336) == 0 and vs(144, 4096, 4096) == 0
    assert vs(300, 14336, 4096) == down  # launches of up to 144 rows share it
    assert sz(144, 14336, 4096) >= down + 144 * 14336  # the fp32 path: codes + the same workspace
    v = lib.verify_gemm
    v.restype = ctypes.c_int
    v.argtypes = [ctypes.c_void_p] * 2 + [ctypes.c_int64] * 2 + [ctypes.c_void_p] * 3 + \
        [ctypes.c_int64] * 2 + [ctypes.c_void_p] * 3 + [ctypes.c_size_t, ctypes.c_void_p]
    assert v(p, p, 144, 14336, p, p, p, 4096, 128, p, None, None, 0, None) == 4  # NEST_EWORKSPACE
    assert b"workspace needs" in lib.nest_last_error()
    assert v(p, p, 144, 14336, p, p, p, 4096, 128, p, None, p, down - 1, None) == 4
    assert v(p, p, 144, 14336, p, p, p, 4096, 128, p, None, ctypes.c_void_p(272), down, None) == 2
    # layout: the 4352-byte counter zone every GEMV workspace starts with
    # (256 B for the argmax counter, 1024 row-block counters), then one slot
    # of 4 tiles x 9 column tiles x 64 lanes x 16 B per (row block, slice):
    # 64 row blocks x 4 slices on a 256-CU device (the count without a GPU)
    assert down == 4352 + 64 * 4 * (4 * 9 * 64 * 16)
    a = lib.kv_nest_append
    a.restype = ctypes.c_int
    a.argtypes = [ctypes.POINTER(_KV)] + [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 2 + [ctypes.c_void_p]
    kv = _KV(256, 256, 256, 256, 256, 256, 8, 128, 32768, 128)
    assert a(ctypes.byref(kv), p, p, p, p, None, 32700, 129, None) == 1  # n > block
    assert a(ctypes.byref(kv), p, p, p, p, None, 32700, 100, None) == 1  # past capacity
