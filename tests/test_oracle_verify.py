"""Pins for the oracle's GEMM reference, head argmax and tree acceptance."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import verify as V

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bits_of(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


# --------------------------------------------------------------------------- GEMM

def test_gemm_one_hot_rows_give_weight_columns():
    rng = np.random.default_rng(0)
    w = bits_of(rng.standard_normal((40, 24)).astype(np.float32)
                * np.float32(2.0) ** rng.integers(-20, 20, (40, 24)))
    w = (w & 0xFFFF)
    x = np.zeros((24, 24), dtype=np.uint16)
    for i in range(24):
        x[i, i] = 0x3F80  # 1.0
    y, b = V.gemm_ref(x, w)
    wf = (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert y.shape == (24, 40)
    assert np.array_equal(y, wf.T)
    assert np.array_equal(b, np.abs(wf.T))


def test_gemm_small_integers_are_exact():
    rng = np.random.default_rng(1)
    xi = rng.integers(-8, 9, (7, 300))
    wi = rng.integers(-8, 9, (13, 300))
    y, b = V.gemm_ref(bits_of(xi.astype(np.float32)), bits_of(wi.astype(np.float32)))
    assert np.array_equal(y, (xi @ wi.T).astype(np.float64))
    assert np.array_equal(b, (np.abs(xi) @ np.abs(wi).T).astype(np.float64))


def test_gemm_tolerance_rule():
    y_ref = np.array([[1.0, -2.0]])
    bound = np.array([[10.0, 1000.0]])
    assert V.within_tolerance(np.array([[1.0 + 0.019, -2.0 - 1.99]]), y_ref, bound).all()
    assert not V.within_tolerance(np.array([[1.0 + 0.0211, -2.0]]), y_ref, bound).all()


# --------------------------------------------------------------------------- head argmax

@pytest.mark.parametrize("chunk", [5, 64, 8192])
def test_head_argmax_lowest_index_on_exact_ties(chunk):
    rng = np.random.default_rng(2)
    xi = rng.integers(-3, 4, (6, 64))
    wi = rng.integers(-3, 4, (200, 64))
    wi[17] = 3 * np.sign(xi[0]) + (xi[0] == 0)  # row 0's clear maximum ...
    wi[150] = wi[17]                       # ... duplicated in a later chunk: exact tie
    xb, wb = bits_of(xi.astype(np.float32)), bits_of(wi.astype(np.float32))
    idx, mx, cands = V.head_argmax(xb, wb, chunk=chunk)
    L = xi @ wi.T                          # integer logits, exact
    for r in range(6):
        best = L[r].max()
        assert idx[r] == int(np.nonzero(L[r] == best)[0][0])
        assert mx[r] == best
        # integer logits: the near-tie set is exactly the tied maxima
        assert set(cands[r].tolist()) == set(np.nonzero(L[r] == best)[0].tolist())
    assert idx[0] == 17


def test_head_argmax_planted_winner_and_near_tie():
    rng = np.random.default_rng(4)
    k = 256
    x = rng.standard_normal((3, k)).astype(np.float32)
    w = rng.standard_normal((500, k)).astype(np.float32) * 0.01
    xb = bits_of(x)
    xf = (xb.astype(np.uint32) << 16).view(np.float32)
    w[321] = xf[0] * 0.5                   # row 0: clear winner 321
    w[77] = xf[1] * 0.5                    # row 1: 77 and 400 almost tie
    w[400] = xf[1] * 0.5
    wb = bits_of(w)
    wb[400, 5] ^= 1                        # last-bit difference in one weight
    idx, _, cands = V.head_argmax(xb, wb, chunk=128)
    assert idx[0] == 321 and list(cands[0]) == [321]
    assert set(cands[1].tolist()) >= {77, 400}


# --------------------------------------------------------------------------- tree acceptance

def chain_closed_form(drafts, argmax):
    """[S1] 1.1 / [S3]: accept the longest draft prefix equal to the target's
    argmax at each position, then append the target's token (tau in [1, m+1])."""
    j = 0
    while j < len(drafts) and drafts[j] == argmax[j]:
        j += 1
    return j, argmax[j]


@pytest.mark.parametrize("seed", range(20))
def test_chain_matches_longest_prefix_plus_bonus(seed):
    rng = np.random.default_rng(seed)
    m = int(rng.integers(0, 12))
    argmax = rng.integers(0, 4, m + 1)
    drafts = np.where(rng.random(m) < 0.7, argmax[:m], rng.integers(0, 4, m))
    parent = np.arange(-1, m)
    token = np.concatenate([[0], drafts])
    acc, path, bonus = V.tree_accept([0, m + 1], parent, token, argmax)
    j, b = chain_closed_form(list(drafts), list(argmax))
    assert acc[0] == j and bonus[0] == b
    assert 1 <= acc[0] + 1 <= m + 1
    assert list(path[:j + 1]) == list(range(j + 1)) and np.all(path[j + 1:] == -1)


def top_down(parent, token, argmax):
    """Independent formulation: grow the accepted set from the root, visiting
    children of accepted nodes only; best = deepest, lowest index."""
    n = len(parent)
    children = [[] for _ in range(n)]
    for i in range(1, n):
        children[parent[i]].append(i)
    depth = {0: 0}
    stack = [0]
    while stack:
        u = stack.pop()
        for v in children[u]:
            if token[v] == argmax[u]:
                depth[v] = depth[u] + 1
                stack.append(v)
    best = min(depth, key=lambda v: (-depth[v], v))
    return depth[best], best


def all_trees(n):
    for parents in itertools.product(*[range(i) for i in range(1, n)]):
        yield [-1] + list(parents)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6])
def test_exhaustive_small_trees(n):
    rng = np.random.default_rng(n)
    count = 0
    for parent in all_trees(n):
        for mask in range(1 << (n - 1)):
            argmax = rng.integers(0, 3, n)
            token = np.zeros(n, dtype=np.int64)
            for i in range(1, n):
                match = (mask >> (i - 1)) & 1
                token[i] = argmax[parent[i]] if match else (argmax[parent[i]] + 1) % 3
            acc, path, bonus = V.tree_accept([0, n], parent, token, argmax)
            d, best = top_down(parent, token, argmax)
            assert acc[0] == d and bonus[0] == argmax[best]
            p = path[:d + 1]
            assert p[0] == 0 and p[-1] == best
            for a, b in zip(p[:-1], p[1:]):
                assert parent[b] == a and token[b] == argmax[a]
            count += 1
            if count > 4000:
                return


def test_spec_worked_example():
    with open(os.path.join(GOLDEN, "spec_example_tree.json")) as f:
        g = json.load(f)
    for case in ("chain", "tree"):
        c = g[case]
        n = len(c["parent"])
        acc, path, bonus = V.tree_accept([0, n], c["parent"], c["token"], c["argmax"])
        assert acc[0] == c["accept_len"] and bonus[0] == c["bonus"]
        assert list(path) == c["path"] and acc[0] + 1 == c["tau"]


def test_multiple_trees_and_invalid():
    parent = [-1, 0, 0, 1,   -1, 0,   0, 0,   -1, 1]
    token = [0, 5, 5, 6,     0, 1,    0, 0,    0, 0]
    argmax = [5, 6, 9, 9,    2, 3,    1, 1,    4, 4]
    node_off = [0, 4, 6, 8, 10, 10]
    acc, path, bonus = V.tree_accept(node_off, parent, token, argmax)
    # tree 0: nodes 1 and 2 both match (duplicate siblings); 3 under 1 matches -> depth 2
    assert acc[0] == 2 and list(path[0:4]) == [0, 1, 3, -1] and bonus[0] == 9
    # tree 1: node 1 token 1 != argmax[0] = 2 -> only the root, tau = 1
    assert acc[1] == 0 and list(path[4:6]) == [0, -1] and bonus[1] == 2
    # tree 2: root parent is 0, not -1 -> invalid
    assert acc[2] == -1 and bonus[2] == -1 and list(path[6:8]) == [-1, -1]
    # tree 3: node 1's parent is itself -> invalid
    assert acc[3] == -1
    # tree 4: empty -> invalid
    assert acc[4] == -1 and bonus[4] == -1


# --------------------------------------------------------------------------- top-k candidates

@pytest.mark.parametrize("chunk", [3, 16, 50, 8192])
def test_head_topk_against_brute_force_with_ties(chunk):
    """The k strongest ids of a row: brute force over exact integer logits,
    ordered by (logit descending, id ascending), so ties at the cut keep the
    lowest ids. Integer data makes every logit exact and ties common; chunks
    smaller than k and not dividing the vocabulary cross the merge path."""
    rng = np.random.default_rng(11)
    xi = rng.integers(-2, 3, (5, 40))
    wi = rng.integers(-2, 3, (203, 40))
    xb, wb = bits_of(xi.astype(np.float32)), bits_of(wi.astype(np.float32))
    for topk in (1, 4, 16):
        got = V.head_topk(xb, wb, topk=topk, chunk=chunk)
        assert got.shape == (5, topk)
        for r in range(5):
            L = [int(sum(int(a) * int(b) for a, b in zip(xi[r], wi[v]))) for v in range(203)]
            want = sorted(range(203), key=lambda v: (-L[v], v))[:topk]
            assert set(got[r].tolist()) == set(want)
            assert len(set(got[r].tolist())) == topk


def test_head_topk_first_is_the_argmax_and_real_valued_rows():
    """On real-valued data the top-1 is the head argmax, and every returned
    logit is >= every logit left out (checked on fp64 logits formed one
    product at a time)."""
    rng = np.random.default_rng(12)
    x = bits_of(rng.standard_normal((3, 64)).astype(np.float32))
    w = bits_of((rng.standard_normal((300, 64)) * 0.05).astype(np.float32))
    top = V.head_topk(x, w, topk=16, chunk=37)
    idx, _, _ = V.head_argmax(x, w, chunk=37)
    xf, wf = V.bf16_to_f64(x), V.bf16_to_f64(w)
    for r in range(3):
        L = np.array([sum(float(a) * float(b) for a, b in zip(xf[r], wf[v])) for v in range(300)])
        kept = set(top[r].tolist())
        assert idx[r] in kept
        assert min(L[list(kept)]) >= max(L[[v for v in range(300) if v not in kept]])


# --------------------------------------------------------------------------- timed CPU baseline

def test_cpu_baseline_gemm_within_tolerance_of_the_reference():
    """The timed baseline (oracle decode + fp32 matmul) must give the GEMM the
    pages define, within the same bound the GPU is held to."""
    import synth
    from oracle import baseline, w12_format as F
    n, k, m = 96, 768, 5
    bits = synth.bits_u16(synth.weights_bf16(n, k, 901, p_zero=0.05, p_outlier=0.02))
    xb = synth.bits_u16(synth.activations_bf16(m, k, 902))
    y = baseline.cpu_verify_gemm(F.pack(bits), n, k, xb)
    y_ref, bound = V.gemm_ref(xb, bits)
    assert y.dtype == np.float32 and y.shape == (m, n)
    assert V.within_tolerance(y, y_ref, bound).all()
    # the decoded weights are the source: one-hot rows pick exact columns
    eye = np.zeros((4, k), np.uint16)
    eye[np.arange(4), [0, 255, 256, 767]] = 0x3F80
    y1 = baseline.cpu_verify_gemm(F.pack(bits), n, k, eye)
    wf = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(y1, wf[:, [0, 255, 256, 767]].T)


def test_cpu_baseline_reports_the_threads_it_ran_with():
    import synth
    from oracle import baseline, w12_format as F
    n, k = 64, 512
    bits = synth.bits_u16(synth.weights_bf16(n, k, 903))
    xb = synth.bits_u16(synth.activations_bf16(4, k, 904))
    one = baseline.time_cpu_verify_gemm(F.pack(bits), n, k, xb, threads=1)
    assert one["threads"] == 1 and one["seconds"] > 0
    allc = baseline.time_cpu_verify_gemm(F.pack(bits), n, k, xb)
    assert allc["threads"] >= 1
