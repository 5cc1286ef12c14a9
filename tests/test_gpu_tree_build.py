"""GPU parity of the best-first tree builder (w12_tree_build, through the C
ABI) against the oracle: node order, parents, tokens, depths and binary32
path scores must match exactly."""
import numpy as np
import pytest

import synth
from oracle import tree_build as TB

pytestmark = pytest.mark.gpu


def say(*a):
    print("[tree_build]", *a, flush=True)


@pytest.fixture(scope="module")
def w12():
    import torch
    import w12_weight_streaming_amd as w
    assert torch.cuda.is_available()
    return w


def run_both(w12, R, D, K, budget, seed, **kw):
    import torch
    say("case", R, D, K, budget, seed, kw)
    lp, tok, depths, roots = synth.draft_lattice(R, D, K, seed, **kw)
    dev = torch.device("cuda:0")
    out = w12.w12_tree_build(torch.from_numpy(lp).to(dev), torch.from_numpy(tok).to(dev),
                             torch.from_numpy(depths).to(dev), torch.from_numpy(roots).to(dev), budget)
    got = [t.cpu().numpy() for t in out]
    ref = TB.shared_budget(lp, tok, depths, roots, budget)
    names = ("node_off", "parent", "token", "depth", "score")
    for g, r, nm in zip(got, ref, names):
        if nm == "score":
            assert np.array_equal(g.view(np.uint32), r.view(np.uint32)), nm
        else:
            assert np.array_equal(g, r), (nm, g[:20], r[:20])
    return got


def test_single_request_32_node_tree(w12):
    # one request, 16 positions x top-16, 32 rows: the tree size of [S1] 4.2
    for seed in range(3):
        run_both(w12, 1, 16, 16, 32, 10 + seed, depths=[16])


def test_shared_budget_24_requests_192_rows(w12):
    # 24 requests drafting 16, 12 or 8 positions share 192 rows ([S1] 4.4)
    for seed in range(3):
        off, parent, token, depth, score = run_both(w12, 24, 16, 16, 192, 20 + seed)
        assert off[-1] == 192


@pytest.mark.parametrize("quantum", [0.5, 1.0])
def test_ties(w12, quantum):
    run_both(w12, 8, 6, 8, 8 + 100, 30, quantum=quantum)
    run_both(w12, 3, 4, 4, 3 + 60, 31, quantum=quantum, depths=[4, 4, 4])


def test_edge_cases(w12):
    run_both(w12, 5, 8, 4, 5, 40)                                   # roots only
    run_both(w12, 3, 16, 1, 3 + 40, 41, depths=[16, 16, 16])       # chains
    run_both(w12, 2, 3, 2, 2 + 100, 42, depths=[3, 3])             # lattices run out of nodes
    run_both(w12, 4, 6, 5, 4 + 30, 43, depths=[0, 6, 0, 2])        # requests drafting nothing
    run_both(w12, 1, 1, 16, 1 + 16, 44, depths=[1])                # one position


def test_size_limits(w12):
    run_both(w12, 128, 4, 8, 128 + 64, 50)                          # most requests
    run_both(w12, 8, 16, 16, 8 + 1023, 51, depths=[16] * 8)        # longest lists


def test_trees_feed_tree_accept(w12):
    import torch
    dev = torch.device("cuda:0")
    lp, tok, depths, roots = synth.draft_lattice(24, 16, 16, 60)
    off, parent, token, depth, score = w12.w12_tree_build(
        torch.from_numpy(lp).to(dev), torch.from_numpy(tok).to(dev), torch.from_numpy(depths).to(dev),
        torch.from_numpy(roots).to(dev), 192)
    # target argmax per row: the row's own best child token when it has one
    # (drafts always match), else an unrelated id
    par = parent.cpu().numpy()
    tk = token.cpu().numpy()
    o = off.cpu().numpy()
    am = np.full(len(par), 7, np.int32)
    for r in range(24):
        for i in range(o[r] + 1, o[r + 1]):
            p = o[r] + par[i]
            if am[p] == 7:
                am[p] = tk[i]
    acc, path, bonus = w12.tree_accept(off, parent, token, torch.from_numpy(am).to(dev))
    acc = acc.cpu().numpy()
    for r in range(24):
        # siblings carry distinct tokens, so exactly the chain of first
        # children is accepted, to its end
        i, d = 0, 0
        while True:
            kids = [j for j in range(1, o[r + 1] - o[r]) if par[o[r] + j] == i]
            if not kids:
                break
            i, d = min(kids), d + 1
        assert acc[r] == d, (r, acc[r], d)
