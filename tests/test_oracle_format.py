"""Pins for the oracle's W12 pack / decode (CPU only).

Each test checks the oracle against something other than its own code:
IEEE binary32 value semantics, brute-force window search, hand-derived field
values (tests/golden/w12_fields.json), layout properties the pages fix (12 KB
record = 8 KB 8-bit view + 4 KB low bits), and the exact round trip.
"""
import json
import os

import numpy as np
import pytest

from oracle import w12_format as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32_of_bf16(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def rand_bits(rng, n, k, lo_e=100, hi_e=130):
    s = rng.integers(0, 2, (n, k), dtype=np.uint32)
    e = rng.integers(lo_e, hi_e, (n, k), dtype=np.uint32)
    m = rng.integers(0, 128, (n, k), dtype=np.uint32)
    return ((s << 15) | (e << 7) | m).astype(np.uint16)


# --------------------------------------------------------------------------- golden fields

def test_golden_fields():
    """Hand-derived codes from the pages' field definition ([S1] 4.1, [S2])."""
    with open(os.path.join(GOLDEN, "w12_fields.json")) as f:
        g = json.load(f)
    chans = g["channels"]
    w = np.zeros((32, 256), dtype=np.uint16)
    for i, ch in enumerate(chans):
        w[i, :8] = [int(h, 16) for h in ch["weights_hex"]]
    p = F.pack(w)
    hi_off, lo_off, lo_shift, block, c, kk = F.positions(32, 256)
    esc_set = set()
    for b in range(len(p["esc_off"]) - 1):
        for e in p["esc"][p["esc_off"][b]:p["esc_off"][b + 1]]:
            strip, rec, t = b // 8, 0, b % 8
            esc_set.add((int(strip * 32 + ((e >> 5) & 31)), int(t * 32 + (e & 31)), int(e >> 16)))
    for i, ch in enumerate(chans):
        assert int(p["e_top"][i]) == ch["e_top"], ch["comment"]
        for j, code in enumerate(ch["codes"]):
            bits = int(ch["weights_hex"][j], 16)
            if code["escaped"]:
                assert (i, j, bits) in esc_set, (ch["comment"], j)
                assert p["records"][hi_off[i, j]] == 0
                assert (p["records"][lo_off[i, j]] >> lo_shift[i, j]) & 15 == 0
            else:
                assert (i, j, bits) not in esc_set
                assert p["records"][hi_off[i, j]] == int(code["hi8"], 16), (ch["comment"], j)
                assert (p["records"][lo_off[i, j]] >> lo_shift[i, j]) & 15 == int(code["lo4"], 16)
    assert np.array_equal(F.decode(p, 32, 256), w)


# --------------------------------------------------------------------------- window rule

def brute_window(row_bits):
    """Literal search: count, for every candidate top, the weights inside."""
    best_e, best_cov = None, -1
    for E in range(16, 255):
        cov = 0
        for b in row_bits:
            e = (int(b) >> 7) & 0xFF
            if 1 <= e <= 254 and E - 15 <= e <= E:
                cov += 1
        if cov > best_cov:
            best_e, best_cov = E, cov
    return best_e


@pytest.mark.parametrize("seed", range(6))
def test_window_vs_brute_force(seed):
    rng = np.random.default_rng(seed)
    w = np.zeros((4, 256), dtype=np.uint16)
    for r in range(4):
        spread = int(rng.integers(1, 40))
        base = int(rng.integers(1, 255 - spread))
        w[r] = rand_bits(rng, 1, 256, base, base + spread)[0]
        # sprinkle zeros, denormals, Inf/NaN
        w[r, rng.integers(0, 256, 20)] = 0
        w[r, rng.integers(0, 256, 5)] = 0x0003
        w[r, rng.integers(0, 256, 3)] = 0x7F80
        w[r, rng.integers(0, 256, 3)] = 0xFFC1
    got = F.window_tops(w)
    for r in range(4):
        assert got[r] == brute_window(w[r])


def test_window_special_cases():
    w = np.zeros((5, 256), dtype=np.uint16)
    w[0] = rand_bits(np.random.default_rng(1), 1, 256, 100, 110)[0]   # 10 binades
    w[2, :] = 0x7F7F                                                    # all at 254
    w[3, :] = 0x0001                                                    # all denormal
    w[4, :] = 0x0080                                                    # all at exponent 1
    e = F.window_tops(w)
    top = int(((w[0].astype(np.uint32) >> 7) & 0xFF).max())
    assert e[0] == top          # fits whole: top of window at the channel max
    assert e[1] == 16           # all-zero channel: nothing to cover
    assert e[2] == 254
    assert e[3] == 16
    assert e[4] == 16


# --------------------------------------------------------------------------- exhaustive codes

@pytest.mark.parametrize("e_group", [range(16, 76), range(76, 136), range(136, 196), range(196, 255)])
def test_exhaustive_bf16_x_window(e_group):
    """Every bf16 pattern under every window top: in-window patterns are coded
    (value check via binary32 semantics), others escape, and all restore."""
    tops = list(e_group)
    n = ((len(tops) + 31) // 32) * 32
    k = 65536 + 256
    w = np.zeros((n, k), dtype=np.uint16)
    allbits = np.arange(65536, dtype=np.uint32)
    for i in range(n):
        E = tops[min(i, len(tops) - 1)]
        w[i, :65536] = allbits
        # anchors: 128 weights at the window top and 128 at its bottom force E_n = E
        w[i, 65536:65536 + 128] = np.uint16(E << 7)
        w[i, 65536 + 128:] = np.uint16((E - 15) << 7)
    p = F.pack(w)
    assert np.array_equal(p["e_top"], np.array([tops[min(i, len(tops) - 1)] for i in range(n)], np.uint8))
    d = F.decode(p, n, k)
    assert np.array_equal(d, w)

    hi_off, lo_off, lo_shift, _, _, _ = F.positions(n, k)
    hi8 = p["records"][hi_off[:, :65536]].astype(np.int64)
    lo4 = (p["records"][lo_off[:, :65536]].astype(np.int64) >> lo_shift[:, :65536]) & 15
    s = hi8 >> 7
    o = (hi8 >> 3) & 15
    m = ((hi8 & 7) << 4) | lo4
    E = p["e_top"].astype(np.int64)[:, None]
    value = np.where(s == 1, -1.0, 1.0) * np.ldexp(1.0 + m / 128.0, (o + E - 15 - 127).astype(np.int32))
    exps = (allbits >> 7) & 0xFF
    inwin = (exps[None, :] >= 1) & (exps[None, :] <= 254) & (exps[None, :] >= E - 15) & (exps[None, :] <= E)
    with np.errstate(invalid="ignore"):
        truth = f32_of_bf16(allbits).astype(np.float64)[None, :]
    assert np.all(value[inwin] == np.broadcast_to(truth, inwin.shape)[inwin])
    # escaped slots hold the zero code (R4)
    assert np.all(hi8[~inwin] == 0) and np.all(lo4[~inwin] == 0)
    # the escape count equals the out-of-window count
    assert int(p["esc_off"][-1]) == int((~inwin).sum())


# --------------------------------------------------------------------------- layout

def test_layout_is_a_bijection_with_8k_4k_split():
    n, k = 64, 512
    hi_off, lo_off, lo_shift, block, c, kk = F.positions(n, k)
    total = n * k * 3 // 2
    rec_pos_hi = hi_off % F.REC_BYTES
    rec_pos_lo = lo_off % F.REC_BYTES
    assert rec_pos_hi.max() < 8192 and rec_pos_lo.min() >= 8192      # first 8 KB / last 4 KB
    assert len(np.unique(hi_off)) == n * k                           # one hi byte per weight
    nib = lo_off * 2 + (lo_shift // 4)
    assert len(np.unique(nib)) == n * k                              # one nibble per weight
    hi_all = np.zeros(total, bool)
    hi_all[hi_off.ravel()] = True
    lo_all = np.zeros(total * 2, bool)
    lo_all[nib.ravel()] = True
    for rec in range(total // F.REC_BYTES):
        base = rec * F.REC_BYTES
        assert hi_all[base:base + 8192].all() and not hi_all[base + 8192:base + F.REC_BYTES].any()
        assert lo_all[2 * (base + 8192):2 * (base + F.REC_BYTES)].all()
    # a record is one 32-channel x 256-k tile
    rec_id = hi_off // F.REC_BYTES
    strip = np.arange(n)[:, None] // 32
    r = np.arange(k)[None, :] // 256
    assert np.array_equal(rec_id, strip * (k // 256) + r)


def test_lane_view_contract():
    """Kernel-facing view: in subtile t of a record, the 16-byte group of lane
    l holds 16 consecutive k of one channel, in order."""
    n, k = 32, 256
    hi_off = F.positions(n, k)[0]
    owner = {}
    for nn in range(n):
        for kk in range(k):
            owner[int(hi_off[nn, kk])] = (nn, kk)
    for t in range(8):
        for lane in range(64):
            cells = [owner[t * 1024 + lane * 16 + j] for j in range(16)]
            chans = {cc for cc, _ in cells}
            ks = [kk for _, kk in cells]
            assert len(chans) == 1
            assert ks == list(range(ks[0], ks[0] + 16))
            # MFMA operand contract: lane l carries channel l % 32, k-half l // 32
            assert chans == {lane % 32}
            assert ks[0] == t * 32 + 16 * (lane // 32)


def test_low_plane_nibble_contract():
    """Kernel-facing placement of the low-bit plane (reading R6): for lane l of
    subtile t, byte b (0..3) of its first 4-byte group holds lo4 of position b
    in the high nibble and of position b + 4 in the low nibble; the second
    group does the same for positions 8..15."""
    n, k = 32, 256
    w = np.zeros((n, k), dtype=np.uint16)
    # channel 5, subtile 2, half 1 -> lane 37; mantissa low nibble = position j
    for j in range(16):
        w[5, 2 * 32 + 16 + j] = np.uint16((120 << 7) | j)
    w[:, 255] = np.uint16(120 << 7)  # keep every channel's window at 120
    p = F.pack(w)
    grp = p["records"][8192 + 2 * 512 + 37 * 8: 8192 + 2 * 512 + 37 * 8 + 8]
    expect = [(b << 4) | (b + 4) for b in range(4)] + [((8 + b) << 4) | (12 + b) for b in range(4)]
    assert list(grp) == expect


def test_escape_order_and_blocks():
    rng = np.random.default_rng(7)
    n, k = 64, 512
    w = rand_bits(rng, n, k, 110, 126)
    w[rng.random((n, k)) < 0.05] = 0
    w[rng.random((n, k)) < 0.01] = 0x8001
    p = F.pack(w)
    off, esc = p["esc_off"].astype(np.int64), p["esc"]
    assert off[0] == 0 and np.all(np.diff(off) >= 0) and off[-1] == len(esc)
    assert np.all((esc & 0xFC00) == 0)                 # reserved bits are zero
    for b in range(len(off) - 1):
        key = ((esc[off[b]:off[b + 1]] >> 5) & 31) * 32 + (esc[off[b]:off[b + 1]] & 31)
        assert np.all(np.diff(key.astype(np.int64)) > 0)  # (c, kk) strictly ascending
    assert np.array_equal(F.decode(p, n, k), w)
    assert F.packed_bytes(n, k, len(esc)) == (len(p["records"]) + len(p["e_top"])
                                              + 4 * len(p["esc_off"]) + 4 * len(esc))


def test_signed_zero_and_nan_payload_restored():
    w = np.zeros((32, 256), dtype=np.uint16)
    w[:, :] = 0x3F80
    w[0, 3] = 0x8000
    w[1, 5] = 0x7FC3
    w[2, 7] = 0xFF81
    w[3, 9] = 0x807F
    p = F.pack(w)
    assert np.array_equal(F.decode(p, 32, 256), w)
    assert int(p["esc_off"][-1]) == 4


def test_corruption_is_detected():
    """Flipping any stored bit changes the restore (the load-time check
    therefore catches it): a sampled set of byte flips in every buffer."""
    rng = np.random.default_rng(3)
    w = rand_bits(rng, 32, 256, 112, 127)
    w[0, 0] = 0
    p = F.pack(w)
    for name in ("records", "e_top"):
        for pos in rng.integers(0, len(p[name]), 20):
            q = {kk: v.copy() for kk, v in p.items()}
            q[name][pos] ^= np.uint8(1 << int(rng.integers(0, 8)))
            assert not np.array_equal(F.decode(q, 32, 256), w)
    q = {kk: v.copy() for kk, v in p.items()}
    q["esc"][0] ^= np.uint32(1 << 20)
    assert not np.array_equal(F.decode(q, 32, 256), w)


def test_eight_bit_view_is_within_midpoint_error():
    rng = np.random.default_rng(11)
    w = rand_bits(rng, 32, 512, 115, 127)
    p = F.pack(w)
    v8 = f32_of_bf16(F.eight_bit_view(p, 32, 512)).astype(np.float64)
    v = f32_of_bf16(w).astype(np.float64)
    e = ((w.astype(np.int64) >> 7) & 0xFF)
    assert np.all(np.abs(v8 - v) <= np.ldexp(8.0 / 128.0, (e - 127).astype(np.int32)))


def test_qpass_weights_equal_decode_with_midpoint_nibbles():
    """Independent route to the Q-pass weights: overwrite the low-nibble
    plane of the records with 0b1000 and run the exact decoder."""
    rng = np.random.default_rng(12)
    n, k = 64, 768
    w = rand_bits(rng, n, k, 110, 125)
    w[rng.random((n, k)) < 0.03] = 0                      # escapes
    w[rng.random((n, k)) < 0.01] = 0x7F00 | (w[0, 0] & 0x7F)  # far outliers
    p = F.pack(w)
    q = {kk: v.copy() for kk, v in p.items()}
    rec = q["records"].reshape(-1, F.REC_BYTES)
    rec[:, F.HI_BYTES:] = 0x88
    assert np.array_equal(F.qpass_weights(p, n, k), F.decode(q, n, k))


def test_qpass_weights_escapes_exact_rest_within_midpoint_error():
    rng = np.random.default_rng(13)
    n, k = 32, 512
    w = rand_bits(rng, n, k, 112, 126)
    w[rng.random((n, k)) < 0.05] = 0
    w[rng.random((n, k)) < 0.02] = 0x0005                  # denormals escape
    p = F.pack(w)
    wq = F.qpass_weights(p, n, k)
    e = (w.astype(np.int64) >> 7) & 0xFF
    top = p["e_top"].astype(np.int64)[:, None]
    in_window = (e >= 1) & (e <= 254) & (e >= top - 15) & (e <= top)
    assert np.array_equal(wq[~in_window], w[~in_window])
    v, vq = f32_of_bf16(w).astype(np.float64), f32_of_bf16(wq).astype(np.float64)
    bound = np.ldexp(8.0 / 128.0, (e - 127).astype(np.int32))
    assert np.all(np.abs(vq - v)[in_window] <= bound[in_window])
    # a weight whose low nibble is already the midpoint comes back exactly
    mid = in_window & ((w & 15) == 8)
    assert mid.any() and np.array_equal(wq[mid], w[mid])


def test_qpass_bytes_are_two_thirds_of_the_records():
    n, k, n_esc = 1024, 1024, 11000
    full = F.packed_bytes(n, k, n_esc)
    q = F.qpass_bytes(n, k, n_esc)
    assert full - q == n * k // 2


def test_synthetic_escape_rate_and_density():
    """Sanity against the pages ([S1] 4.1): Gaussian weights under per-channel
    windows escape rarely (the pages report 7.33e-5 on a real checkpoint) and
    cost about 12 bits per weight."""
    import torch
    import synth
    w = synth.bits_u16(synth.weights_bf16(256, 4096, seed=5, p_zero=0.0, p_outlier=0.0))
    p = F.pack(w)
    rate = int(p["esc_off"][-1]) / w.size
    assert rate < 5e-4
    bpw = F.bits_per_weight(256, 4096, int(p["esc_off"][-1]))
    assert 12.0 < bpw < 12.06
    del torch
