"""HIP path vs the CPU oracle, through the C ABI (needs an MI355X).

Bars: packing, decode, argmax indices (away from near-ties) and accepted
paths bit-exact; GEMM outputs within |y - y_ref| <= 2e-3 sum|x w| + 1e-6.
Sizes span several records/tiles, odd strip counts and ragged stream-K
slices; the full-size shapes are checked on sampled outputs.
"""
import sys

import numpy as np
import pytest
import torch

import synth
from oracle import verify as V
from oracle import w12_format as F

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="session")
def w12():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import w12_weight_streaming_amd as w
    w.lib()
    return w


DEV = "cuda:0"


def gen(n, k, seed, **kw):
    return synth.weights_bf16(n, k, seed, **kw)


def special_matrix(n=64, k=512, seed=9):
    """Zeros, -0, denormals, Inf/NaN payloads, window edges, empty channels."""
    rng = np.random.default_rng(seed)
    s = rng.integers(0, 2, (n, k), dtype=np.uint32)
    e = rng.integers(100, 125, (n, k), dtype=np.uint32)
    m = rng.integers(0, 128, (n, k), dtype=np.uint32)
    w = ((s << 15) | (e << 7) | m).astype(np.uint16)
    w[rng.random((n, k)) < 0.05] = 0
    w[rng.random((n, k)) < 0.02] = 0x8000
    w[rng.random((n, k)) < 0.02] = 0x0013
    w[rng.random((n, k)) < 0.01] = 0x7F80
    w[rng.random((n, k)) < 0.01] = 0xFFC3
    w[3, :] = 0                        # all-zero channel
    w[4, :] = 0x0080                   # exponent 1 only
    w[5, :] = 0x7F7F                   # exponent 254 only
    w[6, ::2] = (140 << 7) | 5         # two clusters 40 binades apart
    w[6, 1::2] = (100 << 7) | 3
    w[7, :300] = 0x0001                # a block with > 64 escapes
    return w


def pack_gpu(w12, bits):
    t = synth.from_bits(bits, DEV)
    return w12.w12_pack(t), t


def host(t):
    return t.cpu().numpy()


def assert_pack_equal(pw, ref):
    assert np.array_equal(host(pw.records), ref["records"])
    assert np.array_equal(host(pw.e_top), ref["e_top"])
    assert np.array_equal(host(pw.esc_off).view(np.uint32), ref["esc_off"])
    assert pw.n_esc == len(ref["esc"])
    assert np.array_equal(host(pw.esc)[:pw.n_esc].view(np.uint32), ref["esc"])


# ----------------------------------------------------------------------------- pack / decode

@pytest.mark.parametrize("shape,kw", [
    ((1024, 1024), dict(p_zero=0.01, p_outlier=0.001)),          # config-1 parity case
    ((32, 256), dict(p_zero=0.01, p_outlier=0.001)),
    ((96, 768), dict(p_zero=0.03, p_outlier=0.02)),              # odd strip count
    ((160, 1280), dict(p_zero=0.0, p_outlier=0.0)),
])
def test_pack_bitexact(w12, shape, kw):
    n, k = shape
    say("pack", shape, kw)
    bits = synth.bits_u16(gen(n, k, 101 + n, **kw))
    pw, t = pack_gpu(w12, bits)
    assert_pack_equal(pw, F.pack(bits))
    assert w12.w12_check(pw, t) == 0
    assert np.array_equal(synth.bits_u16(w12.w12_decode(pw)), bits)


def test_pack_special_values(w12):
    bits = special_matrix()
    pw, t = pack_gpu(w12, bits)
    assert_pack_equal(pw, F.pack(bits))
    assert np.array_equal(synth.bits_u16(w12.w12_decode(pw)), bits)
    assert w12.w12_check(pw, t) == 0


def upload_packed(w12, ref, n, k):
    d = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a).view(dt)).to(DEV)
    esc = ref["esc"] if len(ref["esc"]) else np.zeros(1, np.uint32)
    return w12.PackedW12(n, k, d(ref["records"], np.uint8), d(ref["e_top"], np.uint8),
                         d(ref["esc_off"], np.int32), d(esc, np.int32), len(ref["esc"]))


def test_decode_of_oracle_packed_buffers(w12):
    for (n, k, seed) in ((64, 512, 3), (1024, 1024, 4)):
        bits = synth.bits_u16(gen(n, k, seed, p_zero=0.02, p_outlier=0.01))
        pw = upload_packed(w12, F.pack(bits), n, k)
        assert np.array_equal(synth.bits_u16(w12.w12_decode(pw)), bits)
    bits = special_matrix()
    pw = upload_packed(w12, F.pack(bits), 64, 512)
    assert np.array_equal(synth.bits_u16(w12.w12_decode(pw)), bits)


def test_check_detects_corruption(w12):
    bits = synth.bits_u16(gen(64, 512, 5))
    pw, t = pack_gpu(w12, bits)
    rec = pw.records.clone()
    pw.records[777] ^= 0x10
    assert w12.w12_check(pw, t) >= 1
    pw.records.copy_(rec)
    pw.e_top[3] += 1
    assert w12.w12_check(pw, t) >= 1
    with pytest.raises(w12.W12Error) as e:
        w12.w12_require_exact(pw, t)
    assert e.value.status == w12.W12_ECORRUPT
    pw.e_top[3] -= 1
    assert w12.w12_check(pw, t) == 0
    w12.w12_require_exact(pw, t)
    # corrupt escape offsets (the last one, the escape count, stays): a block
    # whose offsets jump past the count or run backwards is counted as 1024
    # mismatches, and no entry is read outside the list
    off = pw.esc_off.clone()
    nb = pw.esc_off.numel() - 1
    pw.esc_off[5] = 0x7FFFFFF0                      # blocks 4 and 5 inconsistent
    assert w12.w12_check(pw, t) >= 2 * 1024
    pw.esc_off.copy_(off)
    pw.esc_off[nb // 2] = 0                         # offsets decrease into it
    assert w12.w12_check(pw, t) >= 1
    pw.esc_off.copy_(off)
    assert w12.w12_check(pw, t) == 0


# ----------------------------------------------------------------------------- GEMM

# (640, 256): one record per strip, so every unit ends a tile
GEMM_SHAPES = [(1024, 1024), (96, 768), (320, 1792), (640, 256)]
ROWS = [1, 2, 3, 5, 8, 9, 12, 13, 15, 16, 17, 32, 33, 64, 100, 130, 192, 256, 300, 384, 450, 512]


@pytest.fixture(scope="module")
def gemm_mats(w12):
    mats = {}
    for (n, k) in GEMM_SHAPES:
        bits = synth.bits_u16(gen(n, k, 7 * n + k, p_zero=0.03, p_outlier=0.02))
        pw, _ = pack_gpu(w12, bits)
        mats[(n, k)] = (pw, bits)
    return mats


@pytest.mark.parametrize("m", ROWS)
@pytest.mark.parametrize("shape", GEMM_SHAPES)
def test_gemm_within_tolerance(w12, gemm_mats, shape, m):
    pw, bits = gemm_mats[shape]
    say("gemm", shape, "m", m)
    x = synth.activations_bf16(m, shape[1], 11 + m)
    y = w12.w12_gemm(pw, x.to(DEV))
    y_ref, bound = V.gemm_ref(synth.bits_u16(x), bits)
    ok = V.within_tolerance(host(y), y_ref, bound)
    assert ok.all(), f"{(~ok).sum()} outputs out of tolerance"
    yb = w12.w12_gemm(pw, x.to(DEV), out_dtype=torch.bfloat16)
    assert torch.equal(yb.cpu(), y.cpu().to(torch.bfloat16))


@pytest.fixture(scope="module")
def wide_mat(w12):
    n, k = 32800, 512
    bits = synth.bits_u16(gen(n, k, 4321, p_zero=0.03, p_outlier=0.02))
    pw, _ = pack_gpu(w12, bits)
    return pw, bits


@pytest.mark.parametrize("m", [1, 3, 8, 32, 40])
def test_gemm_slices_spanning_tiles(w12, wide_mat, m):
    """32800 x 512 (1025 strips, 2 records each): on a 256-CU device the
    slices hold ~4 units, so most start inside a tile (a split first tile whose
    partial is kept until the walk ends), cross a whole tile and end inside a
    third. Every output against the oracle, the GEMM and head argmax each
    repeated bit for bit on one workspace."""
    pw, bits = wide_mat
    say("slices spanning tiles m", m)
    x = synth.activations_bf16(m, 512, 4400 + m)
    xd = x.to(DEV)
    ws = torch.zeros(w12.gemm_workspace_bytes(pw.n, pw.k, m), dtype=torch.uint8, device=DEV)
    y = w12.w12_gemm(pw, xd, ws=ws).clone()
    y_ref, bound = V.gemm_ref(synth.bits_u16(x), bits)
    ok = V.within_tolerance(host(y), y_ref, bound)
    assert ok.all(), f"{(~ok).sum()} outputs out of tolerance"
    for _ in range(3):
        assert torch.equal(w12.w12_gemm(pw, xd, ws=ws), y)
    idx, mx = w12.w12_head_argmax(pw, xd, ws=ws)
    ref_idx, _, cands = V.head_argmax(synth.bits_u16(x), bits)
    check_argmax(host(idx), ref_idx, cands)
    assert np.array_equal(host(mx), host(y)[np.arange(m), host(idx)])
    i2, m2 = w12.w12_head_argmax(pw, xd, ws=ws)
    assert torch.equal(i2, idx) and torch.equal(m2, mx)


@pytest.mark.parametrize("m", [1, 8, 32, 64])
def test_gemm_exact_pins(w12, m):
    """One-hot rows give weight columns exactly; small integers are exact."""
    n, k = 320, 1024
    bits = synth.bits_u16(gen(n, k, 21, p_zero=0.05, p_outlier=0.02))
    pw, _ = pack_gpu(w12, bits)
    x = np.zeros((m, k), np.uint16)
    cols = np.random.default_rng(m).choice(k, m, replace=False)
    x[np.arange(m), cols] = 0x3F80
    y = host(w12.w12_gemm(pw, synth.from_bits(x, DEV)))
    wf = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(y, wf[:, cols].T)
    rng = np.random.default_rng(m + 1)
    xi = rng.integers(-8, 9, (m, k)).astype(np.float32)
    wi = rng.integers(-8, 9, (n, k)).astype(np.float32)
    wi[rng.random((n, k)) < 0.05] = 0.0          # zeros travel as escapes
    wb = (wi.view(np.uint32) >> 16).astype(np.uint16)
    xb = (xi.view(np.uint32) >> 16).astype(np.uint16)
    pw2, _ = pack_gpu(w12, wb)
    y2 = host(w12.w12_gemm(pw2, synth.from_bits(xb, DEV)))
    assert np.array_equal(y2, xi @ wi.T)


@pytest.mark.parametrize("m", [1, 16, 32, 64, 100, 192, 256, 384, 512])
def test_gemm_dense_escapes(w12, m):
    """30% exact zeros: ~300 escapes per 1024-weight block, beyond what the
    load ring carries per lane (64 on the small-m path, 128 on the large-m
    path), so every block takes the rest of its entries in a second pass."""
    n, k = 320, 1024
    bits = synth.bits_u16(gen(n, k, 51, p_zero=0.3, p_outlier=0.02))
    pw, _ = pack_gpu(w12, bits)
    assert pw.n_esc > 0.25 * n * k
    say("dense escapes m", m)
    x = synth.activations_bf16(m, k, 52 + m)
    y = w12.w12_gemm(pw, x.to(DEV))
    y_ref, bound = V.gemm_ref(synth.bits_u16(x), bits)
    ok = V.within_tolerance(host(y), y_ref, bound)
    assert ok.all(), f"{(~ok).sum()} outputs out of tolerance"


@pytest.mark.parametrize("m", [1, 32])
def test_gemm_deterministic_and_workspace_reuse(w12, m):
    """Bitwise repeatable (fixed-order stream-K), and a reused workspace gives
    the same bits as a fresh zero-filled one (its counters return to zero)."""
    n, k = 5120, 6144
    w = gen(n, k, 31, device=DEV)
    pw = w12.w12_pack(w)
    x = synth.activations_bf16(m, k, 32, device=DEV)
    y1 = w12.w12_gemm(pw, x).clone()
    for _ in range(3):
        y2 = w12.w12_gemm(pw, x).clone()
        assert torch.equal(y1, y2)
    fresh = torch.zeros(w12.gemm_workspace_bytes(n, k, m), dtype=torch.uint8, device=DEV)
    assert torch.equal(y1, w12.w12_gemm(pw, x, ws=fresh))
    idx1, mx1 = w12.w12_head_argmax(pw, x)
    idx1, mx1 = idx1.clone(), mx1.clone()
    for _ in range(3):
        idx2, mx2 = w12.w12_head_argmax(pw, x)
        assert torch.equal(idx1, idx2) and torch.equal(mx1, mx2)
    assert torch.equal(mx1, y1[torch.arange(m, device=DEV), idx1.long()])


def test_workspace_shared_across_shapes(w12):
    """One workspace, calls of different shapes interleaved (the partial sums
    of one shape must never sit where another keeps its counters)."""
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=DEV)
    shapes = [(64, 512), (2048, 1024), (96, 768), (4096, 512)]
    mats = []
    for i, (n, k) in enumerate(shapes):
        bits = synth.bits_u16(gen(n, k, 300 + i, p_zero=0.02, p_outlier=0.01))
        mats.append((w12.w12_pack(synth.from_bits(bits, DEV)), bits))
    for rep in range(2):
        for (pw, bits), m in zip(mats * 2, (1, 33, 7, 64, 16, 2, 48, 1)):
            x = synth.activations_bf16(m, pw.k, 400 + m)
            y = host(w12.w12_gemm(pw, x.to(DEV), ws=ws))
            y_ref, bound = V.gemm_ref(synth.bits_u16(x), bits)
            assert V.within_tolerance(y, y_ref, bound).all(), (pw.n, pw.k, m)


def test_gemm_rejects_small_workspace(w12):
    n, k = 256, 512
    pw = w12.w12_pack(gen(n, k, 1, device=DEV))
    x = synth.activations_bf16(32, k, 2, device=DEV)
    small = torch.zeros(64, dtype=torch.uint8, device=DEV)
    with pytest.raises(w12.W12Error) as e:
        w12.w12_gemm(pw, x, ws=small)
    assert e.value.status == w12.W12_ENOSPC


# ----------------------------------------------------------------------------- head argmax

def check_argmax(idx, ref_idx, cands):
    near = 0
    for r in range(len(ref_idx)):
        if len(cands[r]) == 1:
            assert idx[r] == ref_idx[r], f"row {r}: {idx[r]} != {ref_idx[r]}"
        else:
            near += 1
            assert idx[r] in set(cands[r].tolist()), f"row {r}: {idx[r]} not in near-tie set"
    return near


@pytest.mark.parametrize("m", [1, 5, 12, 15, 16, 32, 48, 100, 192, 256, 384, 512])
def test_head_argmax(w12, m):
    n, k = 8192, 1024
    bits = synth.bits_u16(gen(n, k, 41, p_zero=0.01, p_outlier=0.001))
    pw, _ = pack_gpu(w12, bits)
    x = synth.activations_bf16(m, k, 42 + m)
    idx, mx = w12.w12_head_argmax(pw, x.to(DEV))
    ref_idx, ref_max, cands = V.head_argmax(synth.bits_u16(x), bits)
    near = check_argmax(host(idx), ref_idx, cands)
    say("head m", m, "near-ties", near)
    y = host(w12.w12_gemm(pw, x.to(DEV)))
    assert np.array_equal(host(mx), y[np.arange(m), host(idx)])


@pytest.mark.parametrize("m", [32, 160])
def test_head_argmax_exact_ties(w12, m):
    """Integer data: duplicated winning rows tie exactly; lowest id wins."""
    n, k = 4096, 512
    rng = np.random.default_rng(5)
    xi = rng.integers(-2, 3, (m, k)).astype(np.float32)
    wi = rng.integers(-2, 3, (n, k)).astype(np.float32)
    for r in range(m):
        win = 2 * np.sign(xi[r])
        a, b = rng.choice(n, 2, replace=False)
        wi[a] = win
        wi[b] = win
    xb = (xi.view(np.uint32) >> 16).astype(np.uint16)
    wb = (wi.view(np.uint32) >> 16).astype(np.uint16)
    pw, _ = pack_gpu(w12, wb)
    idx, _ = w12.w12_head_argmax(pw, synth.from_bits(xb, DEV))
    L = xi.astype(np.int64) @ wi.astype(np.int64).T
    expect = np.array([np.nonzero(L[r] == L[r].max())[0][0] for r in range(m)])
    assert np.array_equal(host(idx), expect)


# ----------------------------------------------------------------------------- Q pass (8-bit view)

@pytest.fixture(scope="module")
def qpass_mat(w12):
    n, k = 320, 1792
    bits = synth.bits_u16(gen(n, k, 61, p_zero=0.03, p_outlier=0.02))
    pw, _ = pack_gpu(w12, bits)
    wq = F.qpass_weights(F.pack(bits), n, k)
    return pw, bits, wq


@pytest.mark.parametrize("m", [1, 5, 16, 32, 64, 100, 192])
def test_qpass_gemm_within_tolerance(w12, qpass_mat, m):
    """w12_gemm_qpass against the oracle GEMM on the Q-pass weights."""
    pw, bits, wq = qpass_mat
    say("qpass gemm m", m)
    x = synth.activations_bf16(m, pw.k, 62 + m)
    y = w12.w12_gemm(pw, x.to(DEV), qpass=True)
    y_ref, bound = V.gemm_ref(synth.bits_u16(x), wq)
    ok = V.within_tolerance(host(y), y_ref, bound)
    assert ok.all(), f"{(~ok).sum()} outputs out of tolerance"


def test_qpass_is_not_the_exact_pass(w12, qpass_mat):
    """The Q pass changes results (the low nibbles matter), and no more than
    the midpoint error allows: |y_q - y| <= sum_k |x| * 2^(e-127) / 16."""
    pw, bits, wq = qpass_mat
    m = 32
    x = synth.activations_bf16(m, pw.k, 70)
    yq = host(w12.w12_gemm(pw, x.to(DEV), qpass=True)).astype(np.float64)
    ye = host(w12.w12_gemm(pw, x.to(DEV))).astype(np.float64)
    assert (yq != ye).mean() > 0.9
    e = ((bits.astype(np.int64) >> 7) & 0xFF).astype(np.int32)
    unit = np.where(e > 0, np.ldexp(1.0 / 16.0, e - 127), 0.0)
    xa = np.abs(V.bf16_to_f64(synth.bits_u16(x)))
    lim = xa @ unit.T
    yref, bound = V.gemm_ref(synth.bits_u16(x), bits)
    assert np.all(np.abs(yq - ye) <= lim + 2 * V.gemm_tolerance(bound))


@pytest.mark.parametrize("m", [1, 32, 100])
def test_qpass_head_argmax(w12, m):
    n, k = 8192, 1024
    bits = synth.bits_u16(gen(n, k, 71, p_zero=0.01, p_outlier=0.001))
    pw, _ = pack_gpu(w12, bits)
    wq = F.qpass_weights(F.pack(bits), n, k)
    x = synth.activations_bf16(m, k, 72 + m)
    idx, mx = w12.w12_head_argmax(pw, x.to(DEV), qpass=True)
    ref_idx, ref_max, cands = V.head_argmax(synth.bits_u16(x), wq)
    near = check_argmax(host(idx), ref_idx, cands)
    say("qpass head m", m, "near-ties", near)
    y = host(w12.w12_gemm(pw, x.to(DEV), qpass=True))
    assert np.array_equal(host(mx), y[np.arange(m), host(idx)])


# ----------------------------------------------------------------------------- tree acceptance

def run_tree(w12, node_off, parent, token, argmax):
    t = lambda a: torch.tensor(np.asarray(a, np.int32), device=DEV)
    acc, path, bonus = w12.tree_accept(t(node_off), t(parent), t(token), t(argmax))
    return host(acc), host(path), host(bonus)


def test_tree_accept_random_forests(w12):
    rng = np.random.default_rng(0)
    for trees, nodes in ((1, 32), (24, 8), (7, 100), (3, 300)):
        node_off, parent, token, argmax = [0], [], [], []
        for ti in range(trees):
            am = rng.integers(0, 50, nodes)
            p, tk = synth.random_tree(nodes, 16, am, None, 0.7, seed=int(rng.integers(1 << 30)), vocab=50)
            parent += list(p)
            token += list(tk)
            argmax += list(am)
            node_off.append(node_off[-1] + nodes)
        got = run_tree(w12, node_off, parent, token, argmax)
        ref = V.tree_accept(node_off, parent, token, argmax)
        for g, r in zip(got, ref):
            assert np.array_equal(g, r)


def test_tree_accept_exhaustive_and_invalid(w12):
    import itertools
    node_off, parent, token, argmax = [0], [], [], []
    rng = np.random.default_rng(1)
    for n in range(1, 6):
        for par in itertools.product(*[range(i) for i in range(1, n)]):
            par = [-1] + list(par)
            for mask in range(1 << (n - 1)):
                am = list(rng.integers(0, 3, n))
                tk = [0] + [am[par[i]] if (mask >> (i - 1)) & 1 else (am[par[i]] + 1) % 3
                            for i in range(1, n)]
                parent += par
                token += tk
                argmax += am
                node_off.append(node_off[-1] + n)
    # invalid: root parent 0, self parent, forward parent, empty tree
    for bad in ([0, 0], [-1, 1], [-1, 2, 0]):
        parent += bad
        token += [0] * len(bad)
        argmax += [0] * len(bad)
        node_off.append(node_off[-1] + len(bad))
    node_off.append(node_off[-1])
    got = run_tree(w12, node_off, parent, token, argmax)
    ref = V.tree_accept(node_off, parent, token, argmax)
    for g, r in zip(got, ref):
        assert np.array_equal(g, r)
    assert (got[0][-4:] == -1).all()


def test_tree_accept_spec_example(w12):
    import json, os
    with open(os.path.join(os.path.dirname(__file__), "golden", "spec_example_tree.json")) as f:
        g = json.load(f)
    for case in ("chain", "tree"):
        c = g[case]
        n = len(c["parent"])
        acc, path, bonus = run_tree(w12, [0, n], c["parent"], c["token"], c["argmax"])
        assert acc[0] == c["accept_len"] and bonus[0] == c["bonus"] and list(path) == c["path"]


# ----------------------------------------------------------------------------- full-size shapes

BLOCK = [("Wq", 6144, 5120), ("Wk", 1024, 5120), ("Wo", 5120, 6144),
         ("Wup", 17408, 5120), ("Wdown", 5120, 17408)]


@pytest.mark.parametrize("name,n,k", BLOCK)
def test_full_size_block_matrices(w12, name, n, k):
    say("full", name, n, k)
    w = gen(n, k, 1000 + n + k, device=DEV)
    pw = w12.w12_pack(w)                      # includes the full bit-exact check
    rng = np.random.default_rng(n)
    for s in rng.choice(n // 32, 2, replace=False):
        bits = synth.bits_u16(w[32 * s:32 * s + 32])
        ref = F.pack(bits)
        rec = host(pw.records).reshape(n // 32, -1)[s]
        assert np.array_equal(rec, ref["records"])
        assert np.array_equal(host(pw.e_top)[32 * s:32 * s + 32], ref["e_top"])
        nb = k // 256 * 8
        off = host(pw.esc_off).view(np.uint32)[s * nb:(s + 1) * nb + 1].astype(np.int64)
        assert np.array_equal(off - off[0], ref["esc_off"].astype(np.int64))
        assert np.array_equal(host(pw.esc)[off[0]:off[-1]].view(np.uint32), ref["esc"])
    for m in (1, 16, 32, 64):
        x = synth.activations_bf16(m, k, 7 + m, device=DEV)
        y = host(w12.w12_gemm(pw, x))
        cols = rng.choice(n, 64, replace=False)
        xb = synth.bits_u16(x)
        wb = synth.bits_u16(w[torch.as_tensor(cols, device=DEV)])
        y_ref, bound = V.gemm_ref(xb, wb)
        assert V.within_tolerance(y[:, cols], y_ref, bound).all(), (name, m)


@pytest.fixture(scope="module")
def plan_mats(w12):
    """At 5-32 rows on a 256-CU device the plan takes, with the y epilogue,
    4-strip tiles and x from the pre-pass for Wgate|Wup 34816x5120 (21 units
    per slice), 4-strip tiles and x read row-major for Wq|Wk|Wv 8192x5120 (5),
    and 2-strip tiles with x from the pre-pass for 20480x5120 (12.5 units at
    4 strips, 25 at 2)."""
    mats = {}

    def get(n, k):
        if (n, k) not in mats:
            w = gen(n, k, n + 3 * k, device=DEV)
            mats[(n, k)] = (w12.w12_pack(w), w)
        return mats[(n, k)]
    return get


@pytest.mark.parametrize("m", [5, 16, 32])
@pytest.mark.parametrize("n,k", [(34816, 5120), (8192, 5120), (20480, 5120)])
def test_full_size_plan_paths(w12, plan_mats, n, k, m):
    """Every channel of three 128-channel tiles (the first, one inside, the
    last) and 64 more against the oracle; repeats bit for bit on one
    workspace; bf16 output is the fp32 output rounded; the Q pass on two whole
    strips against the oracle's Q-pass weights."""
    pw, w = plan_mats(n, k)
    say("full plan paths", n, k, "m", m)
    x = synth.activations_bf16(m, k, 300 + m, device=DEV)
    ws = torch.zeros(w12.gemm_workspace_bytes(n, k, m), dtype=torch.uint8, device=DEV)
    y = w12.w12_gemm(pw, x, ws=ws).clone()
    rng = np.random.default_rng(m)
    tiles = [0, int(rng.integers(1, n // 128 - 1)), n // 128 - 1]
    cols = np.unique(np.concatenate([np.arange(128 * t, 128 * t + 128) for t in tiles]
                                    + [rng.choice(n, 64, replace=False)]))
    xb = synth.bits_u16(x)
    wb = synth.bits_u16(w[torch.as_tensor(cols, device=DEV)])
    y_ref, bound = V.gemm_ref(xb, wb)
    ok = V.within_tolerance(host(y)[:, cols], y_ref, bound)
    assert ok.all(), f"{(~ok).sum()} outputs out of tolerance"
    for _ in range(2):
        assert torch.equal(w12.w12_gemm(pw, x, ws=ws), y)
    yb = w12.w12_gemm(pw, x, ws=ws, out_dtype=torch.bfloat16)
    assert torch.equal(yb.cpu(), y.cpu().to(torch.bfloat16))
    yq = host(w12.w12_gemm(pw, x, ws=ws, qpass=True))
    for s in (int(rng.integers(0, n // 32 - 1)), n // 32 - 1):
        sb = synth.bits_u16(w[32 * s:32 * s + 32])
        yr, bd = V.gemm_ref(xb, F.qpass_weights(F.pack(sb), 32, k))
        assert V.within_tolerance(yq[:, 32 * s:32 * s + 32], yr, bd).all(), ("qpass strip", s)


@pytest.mark.parametrize("name,n,k,seed", [("Wdown", 5120, 17408, 77), ("Wup", 17408, 5120, 79)])
def test_full_size_batched_m192(w12, name, n, k, seed):
    """The batched verify shapes at 192 rows with 3% zeros and 2% x64
    outliers (~3.2% escapes), on sampled columns."""
    say("batched m=192", name, n, k)
    w = gen(n, k, seed, p_zero=0.03, p_outlier=0.02, device=DEV)
    pw = w12.w12_pack(w)
    assert pw.n_esc > 0.03 * n * k
    x = synth.activations_bf16(192, k, seed + 1, device=DEV)
    y = host(w12.w12_gemm(pw, x))
    rng = np.random.default_rng(seed)
    cols = np.concatenate([rng.choice(n - 32, 48, replace=False), np.arange(n - 32, n)])
    y_ref, bound = V.gemm_ref(synth.bits_u16(x), synth.bits_u16(w[torch.as_tensor(cols, device=DEV)]))
    assert V.within_tolerance(y[:, cols], y_ref, bound).all()


@pytest.mark.timeout(400)
def test_full_size_head_argmax_and_config4_tree(w12):
    """LM head 152064x5120 at 32 rows: every row's fused argmax against the
    oracle (exact away from near-ties), then a 32-node tree whose
    mismatching tokens come from the parent row's oracle top-16 candidates
    ([S1] 4.2), accepted on the GPU's argmax and compared with the oracle's
    acceptance on the same argmax and, when no row is a near-tie, on the
    oracle's own argmax."""
    n, k, m = 152064, 5120, 32
    w = gen(n, k, 4242, device=DEV)
    pw = w12.w12_pack(w)
    x = synth.activations_bf16(m, k, 4243, device=DEV)
    idx, _ = w12.w12_head_argmax(pw, x)
    idx = host(idx)
    wb = synth.bits_u16(w)
    del w
    xb = synth.bits_u16(x)
    say("full head: oracle argmax over 32 rows")
    ref_idx, _, cands = V.head_argmax(xb, wb, chunk=16384)
    near = check_argmax(idx, ref_idx, cands)
    say("full head: near-tie rows", near, "; oracle top-16")
    top16 = V.head_topk(xb, wb, topk=16, chunk=16384)
    assert np.array_equal(top16[:, 0], ref_idx)
    for seed in range(4):
        parent, token = synth.random_tree(m, 16, idx, top16, 0.7, seed=4_000_000 + seed, vocab=n)
        drawn = [token[i] for i in range(1, m) if token[i] != idx[parent[i]]]
        assert all(t in set(top16[parent[i]].tolist()) for i, t in
                   ((i, token[i]) for i in range(1, m)) if t != idx[parent[i]])
        got = run_tree(w12, [0, m], parent, token, idx)
        ref = V.tree_accept([0, m], parent, token, idx)
        for g, r in zip(got, ref):
            assert np.array_equal(g, r)
        if near == 0:
            ref2 = V.tree_accept([0, m], parent, token, ref_idx)
            for g, r in zip(got, ref2):
                assert np.array_equal(g, r)
        say("config-4 tree", seed, "accept_len", got[0][0], "mismatching drafts", len(drawn))


def test_full_size_head_shape_four_strip_tiles(w12):
    """At the LM-head shape (152064x5120) up to 32 rows run 4-strip tiles:
    the GEMM (exact and Q pass) on sampled columns against the oracle, and
    the fused argmax (exact and Q pass) against the argmax of those logits."""
    n, k = 152064, 5120
    w = gen(n, k, 4300, device=DEV)
    pw = w12.w12_pack(w)
    rng = np.random.default_rng(4301)
    cols = np.sort(rng.choice(n, 64, replace=False))
    wb_cols = synth.bits_u16(w[torch.as_tensor(cols, device=DEV)])
    strips = rng.choice(n // 32, 2, replace=False)
    qcols = np.concatenate([np.arange(32 * s, 32 * s + 32) for s in strips])
    wq = F.qpass_weights(F.pack(synth.bits_u16(w[torch.as_tensor(qcols, device=DEV)])), len(qcols), k)
    del w
    for m in (17, 32):
        say("head shape, 4-strip tiles, m", m)
        x = synth.activations_bf16(m, k, 4302 + m, device=DEV)
        xb = synth.bits_u16(x)
        y = host(w12.w12_gemm(pw, x))
        y_ref, bound = V.gemm_ref(xb, wb_cols)
        assert V.within_tolerance(y[:, cols], y_ref, bound).all(), m
        idx, mx = w12.w12_head_argmax(pw, x)
        idx = host(idx)
        # the fused argmax is the argmax of the same logits (lowest id on ties)
        assert np.array_equal(idx, np.argmax(y, axis=1)), m
        assert np.array_equal(host(mx), y[np.arange(m), idx]), m
    m = 32
    x = synth.activations_bf16(m, k, 4340, device=DEV)
    yq = host(w12.w12_gemm(pw, x, qpass=True))
    yq_ref, bound = V.gemm_ref(synth.bits_u16(x), wq)
    assert V.within_tolerance(yq[:, qcols], yq_ref, bound).all()
    iq, mq = w12.w12_head_argmax(pw, x, qpass=True)
    assert np.array_equal(host(iq), np.argmax(yq, axis=1))
    assert np.array_equal(host(mq), yq[np.arange(m), host(iq)])


def test_four_strip_tiles_with_a_partial_last_tile(w12):
    """2461 strips x 20 records: 4-strip tiles on a 256-CU device (12320
    units), the last tile holding one strip. Sampled columns include that
    strip; the fused argmax must equal the argmax of the logits."""
    n, k, m = 2461 * 32, 5120, 32
    w = gen(n, k, 4400, device=DEV)
    pw = w12.w12_pack(w)
    rng = np.random.default_rng(4401)
    cols = np.sort(np.concatenate([rng.choice(n - 32, 48, replace=False), np.arange(n - 32, n)]))
    wb = synth.bits_u16(w[torch.as_tensor(cols, device=DEV)])
    del w
    x = synth.activations_bf16(m, k, 4402, device=DEV)
    y = host(w12.w12_gemm(pw, x))
    y_ref, bound = V.gemm_ref(synth.bits_u16(x), wb)
    assert V.within_tolerance(y[:, cols], y_ref, bound).all()
    idx, mx = w12.w12_head_argmax(pw, x)
    idx = host(idx)
    assert idx.max() < n
    assert np.array_equal(idx, np.argmax(y, axis=1))
    assert np.array_equal(host(mx), y[np.arange(m), idx])


# ----------------------------------------------------------------------------- determinism of the hand-off

@pytest.mark.parametrize("n,k,m", [(1024, 1024, 1), (1024, 1024, 12), (5120, 6144, 32), (96, 768, 64),
                                   (320, 1792, 192), (640, 256, 33), (17408, 5120, 100), (640, 256, 384),
                                   (5120, 6144, 512)])
def test_split_tile_hand_off_is_bitwise_repeatable(w12, n, k, m):
    """Every GEMM path, shapes whose tiles are split between many workgroups
    (and one record per strip), 20 calls in a row on one workspace: each
    result equals the first bit for bit (the fixed-order stream-K hand-off),
    and the head argmax likewise."""
    say("repeat", n, k, m)
    w = gen(n, k, 9100 + n + m, p_zero=0.02, p_outlier=0.01, device=DEV)
    pw = w12.w12_pack(w)
    x = synth.activations_bf16(m, k, 9200 + m, device=DEV)
    ws = torch.zeros(w12.gemm_workspace_bytes(n, k, m), dtype=torch.uint8, device=DEV)
    y0 = w12.w12_gemm(pw, x, ws=ws).clone()
    i0, v0 = (t.clone() for t in w12.w12_head_argmax(pw, x, ws=ws))
    for rep in range(20):
        y = w12.w12_gemm(pw, x, ws=ws)
        assert torch.equal(y, y0), f"GEMM call {rep} differs"
        i, v = w12.w12_head_argmax(pw, x, ws=ws)
        assert torch.equal(i, i0) and torch.equal(v, v0), f"argmax call {rep} differs"
