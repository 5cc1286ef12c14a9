"""Verify-pass oracle: GEMM reference, LM-head argmax, tree acceptance.

Test infrastructure only (see the package docstring for who may call it).

GEMM ([S1] 4.1: the W12 GEMM multiplies restored weights against the verify
rows): y[m, n] = sum_k x[m, k] * w[n, k]. Every bf16 x bf16 product is exact
in binary64, so an fp64 accumulation is near exact. The pass bound is
|y - y_ref| <= 2e-3 * sum_k |x w| + 1e-6.

Head argmax ([S1] 1.1 and 4.1: the target's greedy token is the argmax of the
LM-head logits, and must never change): idx[m] = the lowest vocabulary id
attaining max_v logits[m, v]. Near-ties ([S1] 1.2: floating-point order may
flip nearly tied logits): with tt(v) = 2 K 2^-24 sum_k |x w_v| + 1e-6, the
candidate set C = {v : L[v] + tt(v) >= L[v*] - tt(v*)}; a row is exact when
|C| = 1 and a near-tie otherwise (then any member of C is acceptable).

Tree acceptance ([S1] 1.1, 4.3; [S3] "What a round guarantees"): node i of a
tree (node 0 = root, the committed token) is accepted when every edge on its
root path has token[child] == argmax[parent row]; the pass keeps the deepest
accepted node (lowest index on equal depth), returns its root path, its depth
as accept_len (accepted drafts) and argmax[best] as the bonus token, so
tau = accept_len + 1.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Value of bf16 bit patterns (the upper half of a binary32)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def gemm_ref(x_bits: np.ndarray, w_bits: np.ndarray):
    """(y_ref, bound) in fp64 for x [M, K] and w [N, K] (bf16 bit patterns):
    y_ref = x w^T and bound = |x| |w|^T."""
    x = bf16_to_f64(x_bits)
    w = bf16_to_f64(w_bits)
    return x @ w.T, np.abs(x) @ np.abs(w).T


def gemm_tolerance(bound: np.ndarray) -> np.ndarray:
    """Allowed |y - y_ref| for the W12 GEMM: 2e-3 * sum|x w| + 1e-6."""
    return 2e-3 * bound + 1e-6


def within_tolerance(y: np.ndarray, y_ref: np.ndarray, bound: np.ndarray) -> np.ndarray:
    return np.abs(np.asarray(y, dtype=np.float64) - y_ref) <= gemm_tolerance(bound)


def near_tie_width(bound: np.ndarray, k: int) -> np.ndarray:
    """Per-logit rounding allowance tt = 2 K 2^-24 sum|x w| + 1e-6 (the
    binary32 summation bound gamma_K with 2x slack for blocked order)."""
    return 2.0 * k * 2.0 ** -24 * bound + 1e-6


def head_argmax(x_bits: np.ndarray, w_bits: np.ndarray, chunk: int = 8192):
    """Exact argmax over the vocabulary of logits = x w^T, with near-tie sets.

    Returns (idx int64 [M], max fp64 [M], cand list of int arrays [M]).
    Processed in vocabulary chunks so the fp64 logits of a 152064-row head
    need not be held at once; the lowest-id rule is applied across chunks.
    """
    x = bf16_to_f64(x_bits)
    m, k = x.shape
    v_total = w_bits.shape[0]
    best = np.full(m, -np.inf)
    best_idx = np.zeros(m, dtype=np.int64)
    best_tt = np.zeros(m)
    # first pass: exact max and its lowest index
    logit_chunks = []
    for v0 in range(0, v_total, chunk):
        w = bf16_to_f64(w_bits[v0:v0 + chunk])
        L = x @ w.T
        B = np.abs(x) @ np.abs(w).T
        cmax = L.max(axis=1)
        carg = L.argmax(axis=1)  # first (lowest) index of the chunk max
        better = cmax > best      # strictly greater: earlier chunks win ties
        best_idx = np.where(better, v0 + carg, best_idx)
        best_tt = np.where(better, near_tie_width(B[np.arange(m), carg], k), best_tt)
        best = np.where(better, cmax, best)
        logit_chunks.append((v0, L, near_tie_width(B, k)))
    cands = [[] for _ in range(m)]
    floor = best - best_tt
    for v0, L, tt in logit_chunks:
        hit = (L + tt) >= floor[:, None]
        for row in range(m):
            ids = np.nonzero(hit[row])[0]
            if ids.size:
                cands[row].append(v0 + ids)
    cands = [np.concatenate(c) for c in cands]
    return best_idx, best, cands


def head_topk(x_bits: np.ndarray, w_bits: np.ndarray, topk: int = 16, chunk: int = 8192):
    """The k strongest vocabulary ids of each row: the first k ids in the
    order (fp64 logit descending, id ascending), so ties at the cut keep the
    lowest ids; returned in that order. The tests draw the mismatching draft
    tokens of synthetic trees from these ([S1] 4.2: a 32-node tree branches
    over each position's top-16 candidates)."""
    x = bf16_to_f64(x_bits)
    m = x.shape[0]
    cur_val = np.full((m, 0), -np.inf)
    cur_idx = np.zeros((m, 0), dtype=np.int64)
    for v0 in range(0, w_bits.shape[0], chunk):
        L = x @ bf16_to_f64(w_bits[v0:v0 + chunk]).T
        vals = np.concatenate([cur_val, L], axis=1)
        idxs = np.concatenate([cur_idx, np.broadcast_to(
            np.arange(v0, v0 + L.shape[1])[None, :], L.shape)], axis=1)
        keep = np.argsort(-vals, axis=1, kind="stable")[:, :topk]
        cur_val = np.take_along_axis(vals, keep, axis=1)
        cur_idx = np.take_along_axis(idxs, keep, axis=1)
    return cur_idx


def tree_accept(node_off, parent, token, argmax):
    """Brute-force greedy tree acceptance.

    node_off [T+1] int; parent/token/argmax [sum n] int, parent indices local
    to each tree (root parent -1, 0 <= parent[i] < i otherwise). argmax[i] is
    the target's greedy token for row i (the row that holds node i).
    Returns (accept_len [T], path [sum n], bonus [T]) as int32; path holds,
    per tree, the accepted root path (root first) then -1. An invalid tree
    (no nodes, root parent != -1, or a parent outside [0, i)) gives
    accept_len = bonus = -1 and an all -1 path.
    """
    node_off = np.asarray(node_off, dtype=np.int64)
    parent = np.asarray(parent, dtype=np.int64)
    token = np.asarray(token, dtype=np.int64)
    argmax = np.asarray(argmax, dtype=np.int64)
    t_count = len(node_off) - 1
    accept_len = np.full(t_count, -1, dtype=np.int32)
    bonus = np.full(t_count, -1, dtype=np.int32)
    path = np.full(len(parent), -1, dtype=np.int32)
    for t in range(t_count):
        base, n = int(node_off[t]), int(node_off[t + 1] - node_off[t])
        par = parent[base:base + n]
        tok = token[base:base + n]
        arg = argmax[base:base + n]
        valid = n >= 1 and par[0] == -1 and all(0 <= par[i] < i for i in range(1, n))
        if not valid:
            continue
        best, best_depth = 0, 0
        for i in range(n):
            ok, depth, j = True, 0, i
            while j != 0:
                p = int(par[j])
                if tok[j] != arg[p]:
                    ok = False
                depth += 1
                j = p
            if ok and depth > best_depth:  # strict: lowest index keeps ties
                best, best_depth = i, depth
        chain = []
        j = best
        while True:
            chain.append(j)
            if j == 0:
                break
            j = int(par[j])
        chain.reverse()
        path[base:base + len(chain)] = chain
        accept_len[t] = best_depth
        bonus[t] = arg[best]
    return accept_len, path, bonus
