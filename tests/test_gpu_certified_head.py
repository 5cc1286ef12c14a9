"""Certified INT8 LM head on the GPU against the oracle (through the C ABI).

Bars: the INT8 copy (codes and block scale codes) bit-exact against
oracle.certified_head, its per-row bound constants within one binary32 ulp
of the oracle's (both rounded up); the certified argmax equal to the exact
head argmax of the oracle (verify.head_argmax) away from near-ties and in
the near-tie candidate set otherwise -- the same bar as the W12 head --
with the rescored row count far below the vocabulary.
"""
import sys

import numpy as np
import pytest
import torch

import synth
from oracle import certified_head as C
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


def host(t):
    return t.cpu().numpy()


def build(w12, bits):
    t = synth.from_bits(bits, DEV)
    pw = w12.w12_pack(t)
    return pw, w12.w12_cert8_pack(t, pw)


def check_argmax(idx, ref_idx, cands):
    near = 0
    for r in range(len(ref_idx)):
        if len(cands[r]) == 1:
            assert idx[r] == ref_idx[r], f"row {r}: {idx[r]} != {ref_idx[r]}"
        else:
            near += 1
            assert idx[r] in set(cands[r].tolist()), f"row {r}: {idx[r]} not in near-tie set"
    return near


@pytest.mark.parametrize("shape,kw", [((1024, 1024), dict()), ((96, 768), dict(p_zero=0.3, p_outlier=0.02)),
                                      ((640, 256), dict(p_zero=0.01, p_outlier=0.01))])
def test_cert_pack_bitexact(w12, shape, kw):
    n, k = shape
    say("cert pack", shape, kw)
    bits = synth.bits_u16(synth.weights_bf16(n, k, 2000 + n, **kw))
    pw, cert = build(w12, bits)
    ref = C.int8_copy(bits)
    rec, codes = C.record_layout(ref["q"], ref["code"])
    assert np.array_equal(host(cert.q).view(np.uint8), rec)
    assert np.array_equal(host(cert.qexp), codes)
    cb = host(cert.cbound)
    lo = np.nextafter(ref["cbound"], np.float32(-np.inf))
    hi = np.nextafter(ref["cbound"], np.float32(np.inf))
    assert np.all((cb >= lo) & (cb <= hi))
    assert np.all(cb.astype(np.float64) >= ref["c"] * (1 - 1e-12))


@pytest.mark.parametrize("m", [1, 5, 16, 17, 32, 33, 48, 64])
def test_certified_argmax_matches_exact(w12, m):
    n, k = 8192, 1024
    bits = synth.bits_u16(synth.weights_bf16(n, k, 2100))
    pw, cert = build(w12, bits)
    x = synth.activations_bf16(m, k, 2101 + m)
    say("certified head m", m)
    idx, mx, cnt = w12.w12_head_argmax_certified(pw, cert, x.to(DEV))
    ref_idx, _, cands = V.head_argmax(synth.bits_u16(x), bits)
    near = check_argmax(host(idx), ref_idx, cands)
    cnt = host(cnt)
    assert np.all(cnt >= 4) and np.all(cnt < n // 20), cnt
    # the winning logit is the exact rescoring of that row: within the GEMM bound
    y_ref, bound = V.gemm_ref(synth.bits_u16(x), bits[host(idx)])
    assert V.within_tolerance(host(mx), np.diag(y_ref), np.diag(bound)).all()
    # the oracle's certified argmax agrees (its survivors include the winner)
    o_idx, surv, _ = C.certified_argmax(synth.bits_u16(x), bits)
    assert np.array_equal(o_idx, ref_idx)
    say("  near-ties", near, "rescored median", int(np.median(cnt)), "oracle survivors median",
        int(np.median([len(s) for s in surv])))


def test_certified_argmax_dense_escapes_and_repeat(w12):
    """30% zeros and 2% outliers (escape-heavy blocks), called three times
    on one workspace: the same result every time (keys and counters return
    to zero)."""
    n, k, m = 2048, 1024, 32
    bits = synth.bits_u16(synth.weights_bf16(n, k, 2200, p_zero=0.3, p_outlier=0.02))
    pw, cert = build(w12, bits)
    x = synth.activations_bf16(m, k, 2201).to(DEV)
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=DEV)
    first = [t.clone() for t in w12.w12_head_argmax_certified(pw, cert, x, ws=ws)]
    ref_idx, _, cands = V.head_argmax(synth.bits_u16(x.cpu()), bits)
    check_argmax(host(first[0]), ref_idx, cands)
    for _ in range(2):
        again = w12.w12_head_argmax_certified(pw, cert, x, ws=ws)
        for a, b in zip(first, again):
            assert torch.equal(a, b)


def test_certified_workspace_shared_across_shapes(w12):
    """One workspace for certified calls of different shapes and rows,
    interleaved: the counters sit at the same offsets for every shape."""
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=DEV)
    mats = []
    for i, (n, k) in enumerate(((4096, 512), (2048, 1024), (1024, 256))):
        bits = synth.bits_u16(synth.weights_bf16(n, k, 2300 + i))
        mats.append((build(w12, bits), bits))
    for (pw, cert), bits in mats * 2:
        for m in (7, 40):
            x = synth.activations_bf16(m, pw.k, 2310 + m)
            idx, _, _ = w12.w12_head_argmax_certified(pw, cert, x.to(DEV), ws=ws)
            ref_idx, _, cands = V.head_argmax(synth.bits_u16(x), bits)
            check_argmax(host(idx), ref_idx, cands)


def test_certified_argmax_exact_ties(w12):
    """Integer data with duplicated winning rows: exact ties, lowest id."""
    n, k, m = 4096, 512, 32
    rng = np.random.default_rng(7)
    xi = rng.integers(-2, 3, (m, k)).astype(np.float32)
    wi = rng.integers(-2, 3, (n, k)).astype(np.float32)
    for r in range(m):
        win = 2 * np.sign(xi[r])
        a, b = rng.choice(n, 2, replace=False)
        wi[a] = win
        wi[b] = win
    xb = (xi.view(np.uint32) >> 16).astype(np.uint16)
    wb = (wi.view(np.uint32) >> 16).astype(np.uint16)
    pw, cert = build(w12, wb)
    idx, _, _ = w12.w12_head_argmax_certified(pw, cert, synth.from_bits(xb, DEV))
    L = xi.astype(np.int64) @ wi.astype(np.int64).T
    expect = np.array([np.nonzero(L[r] == L[r].max())[0][0] for r in range(m)])
    assert np.array_equal(host(idx), expect)


@pytest.mark.timeout(400)
def test_full_size_certified_head(w12):
    """The 152064x5120 head at 32 rows: every row's certified argmax equals
    the exact head argmax (oracle), and the W12 head's own argmax agrees."""
    n, k, m = 152064, 5120, 32
    w = synth.weights_bf16(n, k, 4242, device=DEV)
    pw = w12.w12_pack(w)
    cert = w12.w12_cert8_pack(w, pw)
    x = synth.activations_bf16(m, k, 4243, device=DEV)
    idx, mx, cnt = w12.w12_head_argmax_certified(pw, cert, x)
    idx_w12, _ = w12.w12_head_argmax(pw, x)
    wb = synth.bits_u16(w)
    del w
    say("full certified head: oracle argmax over 32 rows")
    ref_idx, _, cands = V.head_argmax(synth.bits_u16(x), wb, chunk=16384)
    near = check_argmax(host(idx), ref_idx, cands)
    if near == 0:
        assert torch.equal(idx, idx_w12)
    cnt = host(cnt)
    say("full certified head: near-ties", near, "rescored per row median", int(np.median(cnt)), "max",
        int(cnt.max()))
    assert np.all(cnt < n // 100)
