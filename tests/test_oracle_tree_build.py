"""Pins of the best-first tree oracle (oracle/tree_build.py) against brute
force and a hand-derived example; no GPU."""
import json
import os

import numpy as np
import pytest

import synth
from oracle import tree_build as TB


def brute_top(lp, depth, n, req=0):
    nodes = TB.enumerate_nodes(lp, depth)
    nodes.sort(key=lambda t: (-float(t[0]), t[1], req, t[2]))
    return nodes[:n]


@pytest.mark.parametrize("seed", range(12))
def test_best_first_equals_brute_force(seed):
    rng = np.random.default_rng(seed)
    D, K = int(rng.integers(1, 5)), int(rng.integers(1, 5))
    quantum = [None, 0.5, 1.0][seed % 3]  # quantised logits: many exact ties
    lp, tok, depths, roots = synth.draft_lattice(1, D, K, 100 + seed, depths=[D], quantum=quantum)
    total = sum(K ** d for d in range(1, D + 1))
    for n in sorted({1, 2, min(5, total), total // 2 or 1, total, total + 3}):
        got = TB.best_first(lp[0], D, n)
        ref = brute_top(lp[0], D, n)
        assert len(got) == len(ref) == min(n, total)
        for g, r in zip(got, ref):
            assert g["score"] == r[0] and g["depth"] == r[1] and g["ranks"] == r[2]
            # the slot path of the node: the parent's slots + its own slot
            assert g["slot"] == r[3][-1]
        # prefix-closed, topological: every parent comes earlier
        for i, g in enumerate(got):
            assert g["parent"] <= i
            if g["parent"] > 0:
                p = got[g["parent"] - 1]
                assert g["ranks"][:-1] == p["ranks"] and g["depth"] == p["depth"] + 1


def test_best_first_hand_example():
    with open(os.path.join(os.path.dirname(__file__), "golden", "tree_build_example.json")) as f:
        g = json.load(f)
    pr = g["lattice_probs"]
    lp = np.zeros((2, 2, 2), np.float32)
    lp[0][0] = np.log(pr["position_1_from_root"])
    lp[1][0] = np.log(pr["position_2_from_candidate_0"])
    lp[1][1] = np.log(pr["position_2_from_candidate_1"])
    got = TB.best_first(lp, 2, 6)
    for name, nd in zip(g["order"], got):
        ref = g["nodes_by_name"][name]
        assert (nd["depth"], nd["parent"], nd["slot"]) == (ref["depth"], ref["parent"], ref["slot"]), name
    probs = [g["path_probabilities"][k] for k in g["path_probabilities"]]
    assert np.allclose(np.exp([float(nd["score"]) for nd in got]), sorted(probs, reverse=True), rtol=1e-6)
    # N = 4 keeps A, B, C and the first of the tied pair
    assert [(nd["depth"], nd["slot"]) for nd in TB.best_first(lp, 2, 4)] == [(1, 0), (2, 0), (1, 1), (2, 0)]


def test_best_first_chain_when_one_candidate():
    lp, tok, depths, roots = synth.draft_lattice(1, 6, 1, 5, depths=[6])
    got = TB.best_first(lp[0], 6, 10)
    assert [g["depth"] for g in got] == [1, 2, 3, 4, 5, 6]
    assert [g["parent"] for g in got] == [0, 1, 2, 3, 4, 5]
    assert all(float(g["score"]) == 0.0 for g in got)  # log-softmax of one candidate


def test_best_first_respects_request_depth():
    lp, tok, depths, roots = synth.draft_lattice(1, 5, 3, 6, depths=[2])
    got = TB.best_first(lp[0], 2, 100)
    assert len(got) == 3 + 9 and max(g["depth"] for g in got) == 2


@pytest.mark.parametrize("seed", range(6))
def test_shared_budget_equals_brute_force(seed):
    rng = np.random.default_rng(50 + seed)
    R, D, K = int(rng.integers(1, 5)), int(rng.integers(1, 4)), int(rng.integers(1, 4))
    lp, tok, depths, roots = synth.draft_lattice(R, D, K, 200 + seed,
                                                 depths=rng.integers(1, D + 1, R),
                                                 quantum=0.5 if seed % 2 else None)
    total = sum(sum(K ** d for d in range(1, int(depths[r]) + 1)) for r in range(R))
    for budget in sorted({R, R + 1, R + 3, R + total // 2, R + total, R + total + 2}):
        off, parent, token, dep, score = TB.shared_budget(lp, tok, depths, roots, budget)
        # brute force over the union of all requests' nodes
        cand = []
        for r in range(R):
            for s, d, ranks, slots in TB.enumerate_nodes(lp[r], int(depths[r])):
                cand.append(((-float(s), d, r, ranks), r, s, d, slots))
        cand.sort(key=lambda t: t[0])
        chosen = cand[:budget - R]
        assert off[-1] == R + len(chosen)
        for r in range(R):
            mine = [c for c in chosen if c[1] == r]
            rows = slice(off[r], off[r + 1])
            assert off[r + 1] - off[r] == 1 + len(mine)
            assert parent[off[r]] == -1 and token[off[r]] == roots[r] and dep[off[r]] == 0
            assert list(score[rows][1:]) == [c[2] for c in mine]
            assert list(dep[rows][1:]) == [c[3] for c in mine]
            assert list(token[rows][1:]) == [int(tok[r][c[3] - 1][c[4][-1]]) for c in mine]
            # topological, prefix-closed: each parent precedes its node and is one level up
            loc = parent[rows]
            for i in range(1, len(loc)):
                assert 0 <= loc[i] < i and dep[rows][loc[i]] == dep[rows][i] - 1


def test_shared_budget_gives_more_to_confident_requests():
    # request 0: one candidate dominates every position; request 1: flat
    D, K = 4, 4
    lp = np.zeros((2, D, K, K), np.float32)
    lp[0] = np.log(np.array([0.97, 0.01, 0.01, 0.01], np.float32))
    lp[1] = np.log(np.full(K, 0.25, np.float32))
    tok = np.arange(2 * D * K, dtype=np.int32).reshape(2, D, K)
    off, parent, token, dep, score = TB.shared_budget(lp, tok, np.array([D, D]), np.array([7, 9]), 2 + 6)
    assert off[1] - off[0] == 1 + D  # the confident chain takes its whole depth first
    assert list(dep[1:off[1]]) == [1, 2, 3, 4]
