"""W12 packed-BF16 format: oracle pack and decode (test infrastructure only).

What the pages fix ([S1] section 4.1, [S2] W12 paragraph):
  * per output channel n, a window of 16 binades [E_n - 15, E_n];
  * an in-window weight is kept in 12 bits: sign, 4-bit exponent offset and
    all 7 mantissa bits;
  * weights outside the window, zeros and denormals go to a per-channel
    sparse escape list and are restored exactly;
  * a record is 12 KB: the first 8 KB is the 8-bit view, the last 4 KB the
    low mantissa bits; restored tensors equal the source bit-for-bit.

Readings taken where the pages are open:
  R1  E_n maximises the number of in-window weights; the smallest such E_n
      wins a tie; E_n in [16, 254] so the window holds normal exponents only.
  R2  8-bit view byte hi8 = s<<7 | o<<3 | m>>4 (sign, offset, top three
      mantissa bits); low nibble lo4 = m & 15; o = e - (E_n - 15).
  R3  Inf and NaN (exponent 255) are escaped like zeros and denormals.
  R4  an escaped weight's 12-bit slot holds 0 (hi8 = 0, lo4 = 0).
  R5  escape entry = u32 (bf16 bits << 16 | c << 5 | kk); entries grouped in
      blocks of 32 channels x 32 k, block-major, (c, kk) ascending inside a
      block, so each channel's entries appear in ascending k.
  R6  record = 32 channels x 256 k (8192 weights = 12 KB, the pages' record
      size), byte placement given by `positions` below.
  R17 the Q pass ([S1] 4.3) reads the 8-bit view with the dropped bits at
      their midpoint and still restores escaped weights from the list.

This module shares no code with the HIP path.
"""
from __future__ import annotations

import numpy as np

STRIP = 32          # channels per record
RECK = 256          # k per record
SUBK = 32           # k per subtile (and per escape block)
REC_BYTES = 12288   # 8192 weights * 12 bits
HI_BYTES = 8192     # the 8-bit view: first 2/3 of a record
E_MIN_TOP = 16      # smallest window top keeping E_n - 15 >= 1
E_MAX_TOP = 254     # largest finite exponent


def fields(bits: np.ndarray):
    """Split bf16 bit patterns into (sign, biased exponent, 7-bit mantissa)."""
    b = np.asarray(bits).astype(np.uint32)
    return b >> 15, (b >> 7) & 0xFF, b & 0x7F


def encodable(e: np.ndarray) -> np.ndarray:
    """Normal, finite, non-zero exponents are the only ones a window can hold
    ([S1] 4.1: zeros and denormals always escape; R3: Inf/NaN too)."""
    return (e >= 1) & (e <= 254)


def window_tops(bits: np.ndarray) -> np.ndarray:
    """E_n per channel (reading R1 of [S1] 4.1 "covering most").

    cov_n(E) = #{k : encodable and E-15 <= e <= E}; E_n is the smallest E in
    [16, 254] with maximal cov_n(E).
    """
    bits = np.asarray(bits)
    n, k = bits.shape
    _, e, _ = fields(bits)
    enc = encodable(e)
    rows = np.broadcast_to(np.arange(n, dtype=np.int64)[:, None], (n, k))
    hist = np.bincount((rows[enc] * 256 + e[enc]).ravel(),
                       minlength=n * 256).reshape(n, 256)
    cov = np.stack([hist[:, E - 15:E + 1].sum(axis=1)
                    for E in range(E_MIN_TOP, E_MAX_TOP + 1)], axis=1)
    return (E_MIN_TOP + np.argmax(cov, axis=1)).astype(np.uint8)


def check_shape(n: int, k: int) -> None:
    if n <= 0 or k <= 0 or n % STRIP or k % RECK:
        raise ValueError(f"W12 needs N % {STRIP} == 0 and K % {RECK} == 0, got {n}x{k}")


def num_blocks(n: int, k: int) -> int:
    """Escape blocks: one per (strip, record, subtile) = 32 channels x 32 k."""
    return (n // STRIP) * (k // RECK) * (RECK // SUBK)


def positions(n: int, k: int):
    """Byte placement of every weight (reading R6), as [n, k] index arrays.

    For weight (n, k): strip s = n // 32, channel c = n % 32, record r =
    k // 256, subtile t = (k % 256) // 32, half h = (k % 32) // 16, position
    j = k % 16 and lane = c + 32 h. The record (s, r) starts at
    (s * (K/256) + r) * 12288.
      hi8: record + t*1024 + lane*16 + j                 (8-bit view plane)
      lo4: record + 8192 + t*512 + lane*8 + 4*(j//8) + j%4; in the high
           nibble when j % 8 < 4, else the low nibble   (low-bit plane)
    Returns (hi_off, lo_off, lo_shift, block, c, kk).
    """
    check_shape(n, k)
    rk = k // RECK
    nn = np.arange(n, dtype=np.int64)[:, None]
    kk_ = np.arange(k, dtype=np.int64)[None, :]
    s, c = nn // STRIP, nn % STRIP
    r, t = kk_ // RECK, (kk_ % RECK) // SUBK
    h, j = (kk_ % SUBK) // 16, kk_ % 16
    lane = c + 32 * h
    rec = (s * rk + r) * REC_BYTES
    hi_off = rec + t * 1024 + lane * 16 + j
    lo_off = rec + HI_BYTES + t * 512 + lane * 8 + 4 * (j // 8) + (j % 4)
    lo_shift = np.where((j % 8) < 4, 4, 0)
    block = (s * rk + r) * 8 + t
    kk = kk_ % SUBK
    bshape = (n, k)
    return (np.broadcast_to(hi_off, bshape), np.broadcast_to(lo_off, bshape),
            np.broadcast_to(lo_shift, bshape), np.broadcast_to(block, bshape),
            np.broadcast_to(c, bshape), np.broadcast_to(kk, bshape))


def pack(bits: np.ndarray) -> dict:
    """Pack bf16 weights [N, K] (uint16 bit patterns) into W12 buffers.

    Returns dict(records uint8[1.5NK], e_top uint8[N], esc_off uint32[NB+1],
    esc uint32[n_esc]) -- the exact bytes of all four buffers.
    """
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    n, k = bits.shape
    check_shape(n, k)
    e_top = window_tops(bits)
    s, e, m = fields(bits)
    low = e_top.astype(np.int64)[:, None] - 15
    inwin = encodable(e) & (e >= low) & (e <= e_top[:, None])
    o = np.where(inwin, e.astype(np.int64) - low, 0).astype(np.uint32)
    hi8 = np.where(inwin, (s << 7) | (o << 3) | (m >> 4), 0).astype(np.uint8)
    lo4 = np.where(inwin, m & 15, 0).astype(np.uint8)

    hi_off, lo_off, lo_shift, block, c, kk = positions(n, k)
    records = np.zeros(n * k * 3 // 2, dtype=np.uint8)
    records[hi_off.ravel()] = hi8.ravel()
    for sh in (4, 0):  # each nibble position is written exactly once
        sel = (lo_shift == sh)
        records[lo_off[sel]] |= (lo4[sel] << sh).astype(np.uint8)

    esc_mask = ~inwin
    eb, ec, ekk = block[esc_mask], c[esc_mask], kk[esc_mask]
    ebits = bits[esc_mask].astype(np.uint32)
    order = np.lexsort((ekk, ec, eb))
    esc = ((ebits[order] << 16) | (ec[order].astype(np.uint32) << 5)
           | ekk[order].astype(np.uint32)).astype(np.uint32)
    counts = np.bincount(eb, minlength=num_blocks(n, k))
    esc_off = np.zeros(num_blocks(n, k) + 1, dtype=np.uint32)
    esc_off[1:] = np.cumsum(counts)
    return dict(records=records, e_top=e_top, esc_off=esc_off, esc=esc)


def decode(packed: dict, n: int, k: int) -> np.ndarray:
    """Restore bf16 bits [N, K] from W12 buffers ([S1] 4.1; R2, R4, R5)."""
    check_shape(n, k)
    rec = packed["records"]
    e_top = packed["e_top"].astype(np.uint32)
    hi_off, lo_off, lo_shift, _, _, _ = positions(n, k)
    hi8 = rec[hi_off].astype(np.uint32)
    lo4 = (rec[lo_off].astype(np.uint32) >> lo_shift) & 15
    s = hi8 >> 7
    o = (hi8 >> 3) & 15
    m = ((hi8 & 7) << 4) | lo4
    out = ((s << 15) | ((o + e_top[:, None] - 15) << 7) | m).astype(np.uint16)

    return apply_escapes(out, packed, n, k)


def apply_escapes(out: np.ndarray, packed: dict, n: int, k: int) -> np.ndarray:
    """Write every escape entry's exact bf16 bits over its slot (R5)."""
    esc_off = packed["esc_off"].astype(np.int64)
    esc = packed["esc"].astype(np.uint32)
    nb = num_blocks(n, k)
    blk = np.repeat(np.arange(nb, dtype=np.int64), np.diff(esc_off))
    rk = k // RECK
    strip, rec_i, t = blk // (rk * 8), (blk // 8) % rk, blk % 8
    cc = (esc >> 5) & 31
    kk = esc & 31
    out[strip * STRIP + cc, rec_i * RECK + t * SUBK + kk] = (esc >> 16).astype(np.uint16)
    return out


def eight_bit_view(packed: dict, n: int, k: int) -> np.ndarray:
    """bf16 values read from the 8-bit view alone, with the four dropped low
    mantissa bits set to their midpoint 0b1000 ([S1] 4.3: the Q pass reads
    only the first 2/3 of each record). Escaped slots come out as their zero
    code; this is a view, not a restore."""
    rec = packed["records"]
    e_top = packed["e_top"].astype(np.uint32)
    hi_off = positions(n, k)[0]
    hi8 = rec[hi_off].astype(np.uint32)
    s, o = hi8 >> 7, (hi8 >> 3) & 15
    m = ((hi8 & 7) << 4) | 8
    return ((s << 15) | ((o + e_top[:, None] - 15) << 7) | m).astype(np.uint16)


def qpass_weights(packed: dict, n: int, k: int) -> np.ndarray:
    """The weights a Q pass multiplies with ([S1] 4.3; reading R17): every
    in-window weight from the 8-bit view alone, its four dropped low mantissa
    bits at their midpoint 0b1000; escaped weights restored exactly from the
    escape list, as the format restores them ([S1] 4.1)."""
    check_shape(n, k)
    return apply_escapes(eight_bit_view(packed, n, k), packed, n, k)


def qpass_bytes(n: int, k: int, n_esc: int) -> int:
    """Bytes a Q pass reads of a matrix: the 8-bit view (first 2/3 of every
    record) + e_top + esc_off + escape entries."""
    return n * k + n + 4 * (num_blocks(n, k) + 1) + 4 * n_esc


def packed_bytes(n: int, k: int, n_esc: int) -> int:
    """Total W12 bytes: records + e_top + esc_off + escape entries."""
    return n * k * 3 // 2 + n + 4 * (num_blocks(n, k) + 1) + 4 * n_esc


def bits_per_weight(n: int, k: int, n_esc: int) -> float:
    return 8.0 * packed_bytes(n, k, n_esc) / (n * k)
