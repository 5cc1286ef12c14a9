"""Pins for the certified INT8 head oracle (oracle/certified_head.py).

What pins it, besides itself:
  * the INT8 copy against the closed-form properties of a power-of-two
    block scale: |q| <= 127, every kept weight within half a step, the
    scale the smallest that fits (one step smaller overflows), exact bf16
    weights, escapes exact (W12's own decode of the same weights);
  * the bound against a brute-force sum of squared errors per row, and the
    Cauchy-Schwarz inequality on random inputs;
  * certification: on random heads the result equals the exact fp64 head
    argmax away from near-ties, and the true argmax survives on every row;
    planted ties and near-ties survive together;
  * the byte layout against W12's 8-bit-view plane positions.
"""
import numpy as np
import pytest

import synth
from oracle import certified_head as C
from oracle import verify as V
from oracle import w12_format as F


def head(v, k, seed, **kw):
    return synth.bits_u16(synth.weights_bf16(v, k, seed, **kw))


@pytest.fixture(scope="module")
def small():
    bits = head(512, 512, 1301, p_zero=0.02, p_outlier=0.01)
    return bits, C.int8_copy(bits)


def test_copy_quantisation_closed_form(small):
    bits, cp = small
    w = V.bf16_to_f64(bits)
    esc = C.escaped_mask(bits)
    q = cp["q"].astype(np.int64)
    code = cp["code"].astype(np.int64)
    v_count, k = bits.shape
    for v in range(0, v_count, 7):
        for j in range(k // 32):
            sl = slice(32 * j, 32 * j + 32)
            keep = ~esc[v, sl]
            if not keep.any():
                assert code[v, j] == 0 and not q[v, sl].any()
                continue
            s = int(code[v, j]) - 133
            amax = max(abs(float(a)) for a in w[v, sl][keep])
            assert amax <= 127 * 2.0 ** s < 2 * amax + 1e-300       # smallest fitting power of two
            assert not amax <= 127 * 2.0 ** (s - 1)
            for kk in range(32):
                wv, qv = float(w[v, 32 * j + kk]), int(q[v, 32 * j + kk])
                if keep[kk]:
                    assert abs(qv) <= 127
                    assert abs(wv - qv * 2.0 ** s) <= 2.0 ** (s - 1)
                else:
                    assert qv == 0


def test_copy_weights_are_bf16_and_escapes_exact(small):
    bits, cp = small
    wq = cp["wq"]
    as_bf16 = (wq.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    back = V.bf16_to_f64(as_bf16)
    assert np.array_equal(back, wq)                       # every copy weight is a bf16 value
    # escaped weights keep W12's exact restore of the same matrix
    dec = V.bf16_to_f64(F.decode(F.pack(bits), *bits.shape))
    esc = C.escaped_mask(bits)
    assert esc.any()
    assert np.array_equal(wq[esc], dec[esc])


def test_bound_constant_against_brute_force(small):
    bits, cp = small
    w = V.bf16_to_f64(bits)
    k = bits.shape[1]
    for v in (0, 5, 99, 511):
        se = sum((float(a) - float(b)) ** 2 for a, b in zip(w[v], cp["wq"][v]))
        sw = sum(float(b) ** 2 for b in cp["wq"][v])
        c = se ** 0.5 + 2 * k * 2.0 ** -24 * sw ** 0.5
        assert cp["cbound"][v] >= c and cp["cbound"][v] <= c * (1 + 2.0 ** -22)
    rng = np.random.default_rng(4)
    x = rng.standard_normal((64, k))
    diff = np.abs(x @ w.T - x @ cp["wq"].T)
    assert np.all(diff <= np.linalg.norm(x, axis=1)[:, None] * cp["c"][None, :] + 1e-12)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_certified_equals_exact_argmax(seed):
    v_count, k, m = 4096, 1024, 16
    bits = head(v_count, k, 1400 + seed)
    xb = synth.bits_u16(synth.activations_bf16(m, k, 1500 + seed))
    idx, surv, lb = C.certified_argmax(xb, bits)
    ref, _, cands = V.head_argmax(xb, bits)
    L = V.bf16_to_f64(xb) @ V.bf16_to_f64(bits).T
    for r in range(m):
        assert int(np.argmax(L[r])) in set(surv[r].tolist())
        assert idx[r] == ref[r]
        assert 1 <= len(surv[r]) < v_count // 20          # the bound prunes


def test_planted_ties_and_near_ties_survive():
    v_count, k = 1024, 512
    bits = head(v_count, k, 1600)
    rng = np.random.default_rng(5)
    xb = synth.bits_u16(synth.activations_bf16(3, k, 1601))
    x = V.bf16_to_f64(xb)
    # row 0: an exact tie between two planted rows (ids 900 < 901 -> 900)
    plant = (np.sign(x[0]) * 0.03).astype(np.float32)
    pb = (plant.view(np.uint32) >> 16).astype(np.uint16)
    bits[900] = pb
    bits[901] = pb
    # row 1: a near tie, one weight of 301 a bf16 ulp larger in the row's favour
    plant1 = (np.sign(x[1]) * 0.03).astype(np.float32)
    p1 = (plant1.view(np.uint32) >> 16).astype(np.uint16)
    bits[300] = p1
    bits[301] = p1
    kk = int(np.argmax(np.abs(x[1])))
    bits[301, kk] = p1[kk] + 1                          # |w| one ulp up, same sign as x
    idx, surv, _ = C.certified_argmax(xb, bits)
    assert idx[0] == 900 and {900, 901} <= set(surv[0].tolist())
    assert idx[1] == 301 and {300, 301} <= set(surv[1].tolist())
    ref, _, _ = V.head_argmax(xb, bits)
    assert np.array_equal(idx, ref)


def test_exactly_representable_head_keeps_only_ties():
    """Weights exact in the copy (small integers times 2^-6): e = 0, so the
    bound is the fp32 allowance alone, and only rows within it survive."""
    rng = np.random.default_rng(6)
    v_count, k = 256, 256
    wi = rng.integers(-100, 101, (v_count, k)).astype(np.float32) * np.float32(2.0 ** -6)
    wi[wi == 0] = np.float32(2.0 ** -6)
    bits = (wi.view(np.uint32) >> 16).astype(np.uint16)
    cp = C.int8_copy(bits)
    assert np.array_equal(cp["wq"], wi.astype(np.float64))
    xi = rng.integers(-3, 4, (4, k)).astype(np.float32)
    xb = (xi.view(np.uint32) >> 16).astype(np.uint16)
    idx, surv, _ = C.certified_argmax(xb, bits, cp)
    L = xi.astype(np.float64) @ wi.astype(np.float64).T
    for r in range(4):
        assert idx[r] == int(np.argmax(L[r]))
        tol = 2 * (np.linalg.norm(xi[r]) * cp["cbound"].max() + 1e-6)
        assert set(surv[r].tolist()) <= set(np.nonzero(L[r] >= L[r].max() - tol)[0].tolist())


def test_record_layout_matches_the_eight_bit_view_plane():
    v_count, k = 64, 512
    bits = head(v_count, k, 1700, p_zero=0.02)
    cp = C.int8_copy(bits)
    rec, codes = C.record_layout(cp["q"], cp["code"])
    hi_off = F.positions(v_count, k)[0]                     # byte of (n, k) in 12 KB W12 records
    rec_w12, within = hi_off // F.REC_BYTES, hi_off % F.REC_BYTES
    assert within.max() < 8192
    pos8 = rec_w12 * 8192 + within
    assert np.array_equal(np.sort(pos8.ravel()), np.arange(v_count * k))
    assert np.array_equal(rec[pos8].view(np.int8), cp["q"])
    # codes: one byte per (channel, 32-k block), each position once
    rk = k // 256
    for n in (0, 33, 63):
        for j in range(k // 32):
            assert codes[((n // 32 * rk + j // 8) * 8 + j % 8) * 32 + n % 32] == cp["code"][n, j]
