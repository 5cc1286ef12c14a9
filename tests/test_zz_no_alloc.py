"""w12_gemm_noalloc (the entry point for callers that cannot allocate device
memory) against w12_gemm, called through the C ABI.

Both run the same kernels; the no-allocation call takes its workspace from
the library's static scratch array, which keeps the previous call's contents.
So each case runs two calls in a row on the same array, the second with a
smaller input, and both must equal w12_gemm bit for bit (a stricter bar than
the GEMM tolerance); every result is also checked against the oracle.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

import synth
from oracle import verify as V

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def w12():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import w12_weight_streaming_amd as w
    w.lib()
    return w


def noalloc(w12, pw, x, ytype=0):
    m = x.shape[0]
    out = torch.empty(m, pw.n, dtype=torch.float32 if ytype == 0 else torch.bfloat16, device=DEV)
    d = pw.desc()
    st = w12.lib().w12_gemm_noalloc(ctypes.byref(d), ctypes.c_void_p(x.data_ptr()), m,
                                    ctypes.c_void_p(out.data_ptr()), ytype,
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, w12.lib().w12_strerror(st)
    return out


# (n, k, first m, second m): the MFMA path (4-strip and 2-strip tiles), the
# large-m path and the VALU path, each followed by a smaller call
CASES = [(1024, 1024, 32, 17), (320, 1792, 64, 5), (5120, 6144, 32, 1), (512, 2048, 192, 100),
         (640, 1536, 384, 257), (96, 768, 12, 2)]


@pytest.mark.parametrize("n,k,m1,m2", CASES)
def test_noalloc_equals_gemm_on_two_calls(w12, n, k, m1, m2):
    say("noalloc", n, k, m1, m2)
    bits = synth.bits_u16(synth.weights_bf16(n, k, 7000 + n, p_zero=0.03, p_outlier=0.02))
    pw = w12.w12_pack(synth.from_bits(bits, DEV))
    for m, yt in ((m1, 0), (m2, 1)):
        x = synth.activations_bf16(m, k, 7100 + m, device=DEV)
        got = noalloc(w12, pw, x, yt)
        ref = w12.w12_gemm(pw, x, out_dtype=got.dtype)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), (n, k, m)
        if yt == 0:
            y_ref, bound = V.gemm_ref(synth.bits_u16(x), bits)
            assert V.within_tolerance(got.cpu().numpy(), y_ref, bound).all()


def test_noalloc_scratch_fits_the_workloads_and_refuses_beyond(w12):
    """Every shape of the verify pass, the LM head and the batched case fits
    the scratch; a shape whose workspace does not (5 <= m <= 64 needs 128 k
    bytes of x fragments: k = 2^20) is refused with W12_ENOSPC. The refused
    call is made only after the library's own size query has said that the
    shape exceeds the scratch, so it cannot reach a launch."""
    for n, k in ((8192, 5120), (5120, 6144), (34816, 5120), (5120, 17408), (152064, 5120), (17408, 5120)):
        for m in (1, 16, 32, 64, 192, 512):
            assert w12.gemm_workspace_bytes(n, k, m) <= w12.NOALLOC_SCRATCH_BYTES, (n, k, m)
    n, k, m = 2048, 1 << 20, 64
    assert w12.gemm_workspace_bytes(n, k, m) > w12.NOALLOC_SCRATCH_BYTES
    buf = torch.zeros(1 << 20, dtype=torch.uint8, device=DEV)  # never read: the size check comes first
    p = buf.data_ptr()
    d = w12.W12Matrix(n, k, p, p, p, p)
    st = w12.lib().w12_gemm_noalloc(ctypes.byref(d), ctypes.c_void_p(p), m, ctypes.c_void_p(p), 0,
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == w12.W12_ENOSPC
