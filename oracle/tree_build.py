"""Best-first draft tree and shared node budget (oracle).

Test infrastructure only (see the package docstring for who may call it).

[S1] 4.2: every edge of the drafter's candidate lattice is scored by the
log-softmax of the child given its parent, and the tree keeps the N nodes with
the highest path score, the sum of the edge scores from the root.
[S1] 4.4 ("Shared node budget"): one node budget is filled across all requests of
a step from the highest path score down; a best-first tree is prefix-closed,
so each request's share is itself a tree.

Lattice of one request (reading R18): D positions x K candidates. Candidate j
of position d has token tok[d][j]. The edge from candidate i of position d - 1
(the root for d = 0, which uses row i = 0 only) to candidate j of position d
scores lp[d][i][j], a log-softmax over j (so <= 0). A request drafting fewer
positions (depth[r] < D) has no nodes deeper than depth[r].

Order (reading R19):
- A node is the path of child ranks (r_1 .. r_d). r_t is the rank of the
  chosen child among its parent's K children, sorted by edge score, highest
  first, equal scores by candidate index.
- Its score is the binary32 sum of its edge scores, accumulated from the root
  in path order (score(child) = fl32(score(parent) + edge)).
- Nodes are ordered by score (highest first), then depth (shallowest first),
  then rank path (lexicographic). Across requests the order is score, depth,
  request index, rank path.
- Edge scores are <= 0, so a node never precedes its parent. The first N
  nodes in this order therefore form a prefix-closed tree, and a prefix of
  one request's order is a tree too.

Rows (reading R20): each request's tree starts with its root row (the
committed token). A budget of B rows for R requests shares B - R draft nodes.
The output has the layout tree acceptance reads: node_off [R + 1], then per
request the root followed by its draft nodes in best-first order, with parent
indices local to the request (-1 for the root).

Every function here is pinned in tests/test_oracle_tree_build.py:
- the best-first search is checked against brute-force enumeration of small
  lattices, and against a hand-derived example;
- the shared budget is checked against brute force over the union of the
  requests' nodes.
"""
from __future__ import annotations

import heapq

import numpy as np

F32 = np.float32


def child_ranks(lp_row: np.ndarray) -> np.ndarray:
    """Candidate indices of one parent's children in rank order: edge score
    descending, equal scores by candidate index."""
    lp_row = np.asarray(lp_row, dtype=np.float32)
    return np.array(sorted(range(len(lp_row)), key=lambda j: (-float(lp_row[j]), j)), dtype=np.int64)


def _key(score: np.float32, depth: int, ranks: tuple, req: int = 0):
    """Sort key of a node: smaller is better."""
    return (-float(score), depth, req, ranks)


def enumerate_nodes(lp: np.ndarray, depth: int):
    """Every node of the lattice up to `depth` (brute force; K^depth nodes):
    list of (score, depth, ranks, slots). Only for small lattices."""
    lp = np.asarray(lp, dtype=np.float32)
    K = lp.shape[2]
    out = []

    def walk(score, slots, ranks):
        d = len(slots)
        if d == depth:
            return
        i = slots[-1] if slots else 0
        order = child_ranks(lp[d][i])
        for r, j in enumerate(order):
            s = F32(score + lp[d][i][j])
            out.append((s, d + 1, ranks + (r,), slots + (int(j),)))
            walk(s, slots + (int(j),), ranks + (r,))

    walk(F32(0.0), (), ())
    return out


def best_first(lp: np.ndarray, depth: int, n: int):
    """The first n draft nodes of one request in best-first order ([S1] 4.2),
    by a priority-queue search: a popped node's best child and its next
    sibling enter the queue. Returns a list of dicts with score, depth,
    parent (index into the list, 0 = root, nodes counted from 1), slot, ranks."""
    lp = np.asarray(lp, dtype=np.float32)
    K = lp.shape[2]
    nodes = [dict(score=F32(0.0), depth=0, parent=-1, slot=0, ranks=())]
    heap = []

    def push(parent_idx, rank):
        p = nodes[parent_idx]
        d = p["depth"]
        if d >= depth or rank >= K:
            return
        order = child_ranks(lp[d][p["slot"]])
        j = int(order[rank])
        s = F32(p["score"] + lp[d][p["slot"]][j])
        ranks = p["ranks"] + (rank,)
        heapq.heappush(heap, (_key(s, d + 1, ranks), parent_idx, rank, j, s))

    push(0, 0)
    while heap and len(nodes) <= n:
        key, parent_idx, rank, j, s = heapq.heappop(heap)
        nodes.append(dict(score=s, depth=nodes[parent_idx]["depth"] + 1, parent=parent_idx, slot=j,
                          ranks=key[3]))
        push(len(nodes) - 1, 0)       # its best child
        push(parent_idx, rank + 1)    # its next sibling
    return nodes[1:]


def shared_budget(lps, tokens, depths, roots, budget: int):
    """Shared node budget ([S1] 4.4): R requests, `budget` rows including the R
    roots. Returns node_off [R+1], parent, token, depth, score (int32/float32
    arrays over the rows)."""
    R = len(lps)
    assert budget >= R
    share = budget - R
    lists = [best_first(lps[r], int(depths[r]), share) for r in range(R)]
    cand = []
    for r in range(R):
        for i, nd in enumerate(lists[r]):
            cand.append((_key(nd["score"], nd["depth"], nd["ranks"], r), r, i))
    cand.sort()
    count = [0] * R
    for _, r, i in cand[:share]:
        count[r] = max(count[r], i + 1)
    # the chosen set of each request is a prefix of its own order
    assert sum(count) == min(share, len(cand))
    node_off = [0]
    parent, token, dep, score = [], [], [], []
    for r in range(R):
        parent.append(-1)
        token.append(int(roots[r]))
        dep.append(0)
        score.append(F32(0.0))
        for nd in lists[r][:count[r]]:
            parent.append(nd["parent"])
            token.append(int(tokens[r][nd["depth"] - 1][nd["slot"]]))
            dep.append(nd["depth"])
            score.append(nd["score"])
        node_off.append(len(parent))
    return (np.array(node_off, np.int32), np.array(parent, np.int32), np.array(token, np.int32),
            np.array(dep, np.int32), np.array(score, np.float32))
