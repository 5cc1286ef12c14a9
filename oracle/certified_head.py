"""Certified INT8 LM head: oracle (test infrastructure only).

What the pages fix ([S1] 4.1, the LM-head paragraph; [S2] W12 paragraph):
the head keeps an INT8 copy; a per-row Cauchy-Schwarz error bound proves
which vocabulary rows cannot be the argmax; those are discarded and only
the survivors are rescored exactly, so the argmax never changes.

Readings taken where the pages are open (R21-R23):
  R21 the INT8 copy: per vocabulary row v and block j of 32 consecutive k,
      the weights W12 keeps in its window are stored as q = RNE(w / 2^s),
      with s the smallest integer such that every such |w| <= 127 * 2^s
      (so |q| <= 127 and q * 2^s is exact in bf16); the weights W12 escapes
      (zeros, denormals, Inf/NaN, out of window) are q = 0 and take their
      exact value from W12's escape list. A block with no window weight has
      code 0. One power-of-two scale per row, or per row with the escapes
      left in, prunes almost nothing on this weight recipe (its x64
      outliers set the scale); per 32-weight blocks with the escapes exact
      prune all but a handful of rows.
  R22 the bound: for input row x and vocabulary row v, with w' the INT8
      copy's weights (escapes exact) and e = w - w' (zero on escapes),
      |x.w - x.w'| <= ||x|| ||e|| (Cauchy-Schwarz); the device computes
      x.w' in fp32, which adds at most 2 K 2^-24 sum|x w'| <= 2 K 2^-24
      ||x|| ||w'|| (the same allowance as the near-tie width). So
      B(x, v) = ||x|| * c_v + 1e-6 with c_v = ||e_v|| + 2 K 2^-24 ||w'_v||,
      c_v stored as binary32 rounded up.
  R23 pruning and rescoring: A = x.w'; LB = max_v (A_v - B_v); the
      survivors are {v : A_v + B_v >= LB}; the result is the lowest id
      attaining the maximum of the exact logits x.w over the survivors.
      The true argmax v* always survives (A_v* + B_v* >= x.w_v* >= x.w_lb
      >= A_lb - B_lb = LB), so the result is the exact head argmax.

This module shares no code with the HIP path.
"""
from __future__ import annotations

import numpy as np

from . import w12_format as F
from .verify import bf16_to_f64

BLOCK = 32          # k per scale block
CODE_BIAS = 133     # stored code = s + 133 (s in [-132, 122]); 0 = no window weight
QMAX = 127


def escaped_mask(bits: np.ndarray) -> np.ndarray:
    """True where W12 escapes the weight: outside its channel's window
    [E_n - 15, E_n] or not encodable ([S1] 4.1; readings R1, R3)."""
    s, e, m = F.fields(bits)
    tops = F.window_tops(bits).astype(np.int64)[:, None]
    inwin = F.encodable(e) & (e.astype(np.int64) >= tops - 15) & (e.astype(np.int64) <= tops)
    return ~inwin


def int8_copy(bits: np.ndarray):
    """The INT8 copy of a head (R21). Returns dict with
    q     int8 [V, K]   (0 on escaped weights),
    code  uint8 [V, K/32] (s + 133, 0 for a block without window weights),
    wq    fp64 [V, K]   the copy's weights w' (q * 2^s, escapes exact),
    c     fp64 [V]      ||e_v|| + 2 K 2^-24 ||w'_v|| (before rounding),
    cbound fp32 [V]     c rounded up to binary32."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    v_count, k = bits.shape
    assert k % BLOCK == 0
    w = bf16_to_f64(bits)
    esc = escaped_mask(bits)
    w3 = w.reshape(v_count, k // BLOCK, BLOCK)
    keep3 = ~esc.reshape(v_count, k // BLOCK, BLOCK)
    amax = np.where(keep3, np.abs(w3), 0.0).max(axis=2)          # [V, K/32]
    has = amax > 0
    # smallest integer s with amax <= 127 * 2^s: start below it, step up
    s = np.where(has, np.floor(np.log2(np.where(has, amax, 1.0) / QMAX)) - 2, 0.0)
    while True:
        up = has & (amax > QMAX * np.exp2(s))
        if not up.any():
            break
        s = s + up
    scale = np.exp2(s)[:, :, None]
    qq = np.where(keep3, np.round(w3 / scale), 0.0)             # exact dyadic quotients, RNE
    assert np.abs(qq).max(initial=0) <= QMAX
    q = qq.reshape(v_count, k).astype(np.int8)
    code = np.where(has, s + CODE_BIAS, 0).astype(np.uint8)
    wq = np.where(keep3, qq * scale, w3).reshape(v_count, k)
    e = w - wq
    c = np.sqrt((e * e).sum(axis=1)) + 2.0 * k * 2.0 ** -24 * np.sqrt((wq * wq).sum(axis=1))
    cb = c.astype(np.float32)
    cb = np.where(cb.astype(np.float64) < c, np.nextafter(cb, np.float32(np.inf)), cb).astype(np.float32)
    return dict(q=q, code=code, wq=wq, c=c, cbound=cb)


def certified_argmax(x_bits: np.ndarray, bits: np.ndarray, copy: dict | None = None):
    """Certified head argmax (R22, R23), all in fp64.

    Returns (idx int64 [M], survivors list of int arrays [M], LB fp64 [M]).
    The survivors use the stored bound cbound (binary32, rounded up)."""
    if copy is None:
        copy = int8_copy(bits)
    x = bf16_to_f64(x_bits)
    xn = np.sqrt((x * x).sum(axis=1))
    A = x @ copy["wq"].T
    B = xn[:, None] * copy["cbound"].astype(np.float64)[None, :] + 1e-6
    LB = (A - B).max(axis=1)
    w = bf16_to_f64(bits)
    idx = np.zeros(x.shape[0], dtype=np.int64)
    survivors = []
    for m in range(x.shape[0]):
        surv = np.nonzero(A[m] + B[m] >= LB[m])[0]
        L = w[surv] @ x[m]
        best = L.max()
        idx[m] = surv[np.nonzero(L == best)[0][0]]   # lowest id among equal maxima
        survivors.append(surv)
    return idx, survivors, LB


def record_layout(q: np.ndarray, code: np.ndarray):
    """Byte placement of the copy on the device: q in 8 KB records laid out
    as W12's 8-bit-view plane (record (s, r) at (s * K/256 + r) * 8192, byte
    t*1024 + lane*16 + j for weight (c, k'), lane = c + 32 (k'%32)/16,
    j = k'%16), codes at ((s * K/256 + r) * 8 + t) * 32 + c."""
    v_count, k = q.shape
    F.check_shape(v_count, k)
    rk = k // F.RECK
    n_idx = np.arange(v_count)[:, None]
    k_idx = np.arange(k)[None, :]
    s, c = n_idx // F.STRIP, n_idx % F.STRIP
    r, kp = k_idx // F.RECK, k_idx % F.RECK
    t, h, j = kp // F.SUBK, (kp % F.SUBK) // 16, kp % 16
    lane = c + 32 * h
    pos = (s * rk + r) * 8192 + t * 1024 + lane * 16 + j
    rec = np.zeros(v_count * k, dtype=np.uint8)
    rec[pos.ravel()] = q.view(np.uint8).ravel()
    jb = np.arange(k // BLOCK)[None, :]
    cpos = ((s * rk + jb // 8) * 8 + jb % 8) * 32 + c
    codes = np.zeros(v_count * k // BLOCK, dtype=np.uint8)
    codes[cpos.ravel()] = code.ravel()
    return rec, codes
