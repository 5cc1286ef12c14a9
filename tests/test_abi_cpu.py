"""The C ABI library loads on a CPU-only host, exports every symbol that
include/w12.h declares, and rejects bad arguments before launching anything.
No compute call is made here."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w12.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?(?:w12_status|char|int|int64_t)\s*\*?\s*(\w+)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    import w12_weight_streaming_amd as w
    if not os.path.exists(w.LIB_PATH):
        from w12_weight_streaming_amd import build
        build.build()
    return w.lib()


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("w12_pack", "w12_decode", "w12_gemm", "w12_head_argmax", "tree_accept",
                 "w12_pack_plan", "w12_check", "w12_gemm_workspace"):
        assert must in names


def test_every_declared_symbol_is_exported(L):
    import w12_weight_streaming_amd as w
    for name in declared_functions():
        assert hasattr(L, name), name
    assert set(declared_functions()) <= set(w.exported_symbols())
    assert L.w12_abi_version() == 1
    assert b"EINVAL" in L.w12_strerror(-1)
    assert b"ECORRUPT" in L.w12_strerror(-4) and w.W12_ECORRUPT == -4


def test_num_blocks_and_shape_rules(L):
    assert L.w12_num_blocks(1024, 1024) == 1024
    assert L.w12_num_blocks(32, 256) == 8
    for n, k in ((0, 256), (31, 256), (32, 255), (32, 0), (64, 1 << 21), (1 << 22, 4096)):
        assert L.w12_num_blocks(n, k) == -1


def test_invalid_arguments_rejected_before_launch(L):
    import w12_weight_streaming_amd as w
    EINVAL = w.W12_EINVAL
    null = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    assert L.w12_pack_plan(null, 64, 256, fake, fake, null) == EINVAL
    assert L.w12_pack_plan(fake, 48, 256, fake, fake, null) == EINVAL
    assert L.w12_pack(fake, 64, 256, fake, fake, fake, null, 10, null) == EINVAL
    assert L.w12_pack(fake, 64, 256, fake, fake, fake, fake, -1, null) == EINVAL
    bad = w.W12Matrix(64, 300, 0x1000, 0x1000, 0x1000, 0x1000)
    good_null = w.W12Matrix(64, 256, 0, 0x1000, 0x1000, 0x1000)
    for d in (bad, good_null):
        assert L.w12_decode(ctypes.byref(d), fake, null) == EINVAL
        assert L.w12_check(ctypes.byref(d), fake, fake, null) == EINVAL
        assert L.w12_gemm(ctypes.byref(d), fake, 4, fake, 0, fake, 1 << 20, null) == EINVAL
        assert L.w12_head_argmax(ctypes.byref(d), fake, 4, fake, null, fake, 1 << 20, null) == EINVAL
    ok = w.W12Matrix(64, 256, 0x1000, 0x1000, 0x1000, 0x1000)
    for m in (0, 513, -3):
        assert L.w12_gemm(ctypes.byref(ok), fake, m, fake, 0, fake, 1 << 20, null) == EINVAL
    assert L.w12_gemm(ctypes.byref(ok), fake, 4, fake, 7, fake, 1 << 20, null) == EINVAL
    assert L.w12_gemm(ctypes.byref(ok), null, 4, fake, 0, fake, 1 << 20, null) == EINVAL
    sz = ctypes.c_size_t(0)
    assert L.w12_gemm_workspace(64, 257, 4, ctypes.byref(sz)) == EINVAL
    assert L.w12_gemm_workspace(64, 256, 513, ctypes.byref(sz)) == EINVAL
    assert L.tree_accept(-1, fake, 0, fake, fake, fake, fake, fake, fake, null) == EINVAL
    assert L.tree_accept(2, null, 4, fake, fake, fake, fake, fake, fake, null) == EINVAL
    assert L.tree_accept(0, null, 0, null, null, null, null, null, null, null) == w.W12_OK


def test_tree_build_limits_rejected_before_launch(L):
    import w12_weight_streaming_amd as w
    EINVAL, ENOSPC = w.W12_EINVAL, w.W12_ENOSPC
    null = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    sz = ctypes.c_size_t(0)
    assert L.w12_tree_build_workspace(24, 192, ctypes.byref(sz)) == w.W12_OK and sz.value >= 24 * 168 * 16
    for R, budget in ((0, 8), (129, 200), (4, 3), (1, 1 + 1024), (16, 16 + 600)):
        assert L.w12_tree_build_workspace(R, budget, ctypes.byref(sz)) == EINVAL, (R, budget)

    def call(R=24, D=16, K=16, budget=192, ws=fake, wsb=1 << 20, lp=fake):
        return L.w12_tree_build(R, D, K, lp, fake, fake, fake, budget, ws, wsb, fake, fake, fake, null, null, null)
    assert call(D=0) == EINVAL and call(D=17) == EINVAL
    assert call(K=0) == EINVAL and call(K=17) == EINVAL
    assert call(budget=23) == EINVAL
    assert call(lp=null) == EINVAL
    assert call(ws=ctypes.c_void_p(0x1008)) == EINVAL  # workspace not 16-byte aligned
    assert call(wsb=100) == ENOSPC


def test_binding_refuses_cpu_tensors():
    import torch
    import w12_weight_streaming_amd as w
    with pytest.raises(ValueError):
        w.w12_pack(torch.zeros(32, 256, dtype=torch.bfloat16))
