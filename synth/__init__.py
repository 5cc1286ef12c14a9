"""Seeded synthetic inputs for the W12 verify path.

This module is the only code shared by the CPU oracle and the HIP path. It
draws random numbers and rounds them to bfloat16; it holds none of the W12
format's arithmetic (no exponent windows, codes, escapes, products or
acceptance rules).

Weight recipe (one matrix, N output channels x K inputs):
  * per-channel scale s_n = exp(scale_sigma * z_n), z_n ~ N(0, 1)
    (lognormal(0, 0.5) by default), one scale per output channel;
  * w = bf16_rne(std * g * s_n), g ~ N(0, 1), std = 0.02;
  * u ~ U[0, 1) per element: u < p_zero -> +0.0 ;
    p_zero <= u < p_zero + p_outlier -> w * 64 (exact in bf16).
Activations: x = bf16_rne(N(0, 1)), shape [M, K].

Everything is seeded through torch.Generator on the requested device. CPU and
GPU generators give different streams for the same seed; consumers that need
the same bytes on both sides generate once and copy.
"""
from __future__ import annotations

import numpy as np
import torch

DEFAULT_STD = 0.02
DEFAULT_SCALE_SIGMA = 0.5
OUTLIER_SCALE = 64.0


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def weights_bf16(n: int, k: int, seed: int, *, p_zero: float = 0.01,
                 p_outlier: float = 0.001, std: float = DEFAULT_STD,
                 scale_sigma: float = DEFAULT_SCALE_SIGMA,
                 device="cpu") -> torch.Tensor:
    """[n, k] bfloat16 weights drawn by the recipe in the module docstring."""
    dev = torch.device(device)
    g = _gen(seed, dev)
    scale = torch.exp(scale_sigma * torch.randn(n, 1, generator=g, device=dev))
    out = torch.empty(n, k, dtype=torch.bfloat16, device=dev)
    # Row blocks keep the fp32 temporaries bounded for very large matrices.
    rows = max(1, (1 << 26) // max(k, 1))
    for r0 in range(0, n, rows):
        r1 = min(n, r0 + rows)
        w = (std * torch.randn(r1 - r0, k, generator=g, device=dev)
             * scale[r0:r1]).to(torch.bfloat16)
        u = torch.rand(r1 - r0, k, generator=g, device=dev)
        w = torch.where(u < p_zero, torch.zeros((), dtype=w.dtype, device=dev), w)
        hit = (u >= p_zero) & (u < p_zero + p_outlier)
        w = torch.where(hit, w * OUTLIER_SCALE, w)
        out[r0:r1] = w
    return out


def activations_bf16(m: int, k: int, seed: int, device="cpu") -> torch.Tensor:
    """[m, k] bfloat16 activations, N(0, 1) rounded to nearest even."""
    dev = torch.device(device)
    g = _gen(seed, dev)
    return torch.randn(m, k, generator=g, device=dev).to(torch.bfloat16)


def bits_u16(t: torch.Tensor) -> np.ndarray:
    """Raw bfloat16 bit patterns of a tensor as a host uint16 array."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def from_bits(bits: np.ndarray, device="cpu") -> torch.Tensor:
    """bfloat16 tensor holding the given uint16 bit patterns."""
    a = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(device)


def random_tree(num_nodes: int, max_depth: int, row_argmax: np.ndarray,
                row_candidates: np.ndarray | None, p_match: float,
                seed: int, vocab: int):
    """One draft tree in topological order (parent < child).

    Node 0 is the root (parent -1). Node i >= 1 picks its parent uniformly
    among earlier nodes whose depth is below ``max_depth``. Its token equals
    the parent row's argmax with probability ``p_match``; otherwise it is a
    different id: drawn uniformly from the parent row's other candidates
    when ``row_candidates`` (shape [rows, C], any order) is given, else
    uniformly from the vocabulary minus the argmax.

    ``row_argmax`` are the argmax ids of this tree's rows (length num_nodes);
    they are inputs here, produced by whichever side supplies them.
    Returns (parent, token) int32 arrays.
    """
    rng = np.random.default_rng(seed)
    parent = np.full(num_nodes, -1, dtype=np.int32)
    token = np.zeros(num_nodes, dtype=np.int32)
    depth = np.zeros(num_nodes, dtype=np.int64)
    for i in range(1, num_nodes):
        eligible = np.nonzero(depth[:i] < max_depth)[0]
        p = int(rng.choice(eligible))
        parent[i] = p
        depth[i] = depth[p] + 1
        target = int(row_argmax[p])
        if rng.random() < p_match:
            token[i] = target
        elif row_candidates is not None:
            others = [int(c) for c in row_candidates[p] if int(c) != target]
            token[i] = int(rng.choice(others))
        else:
            t = int(rng.integers(0, vocab - 1))
            token[i] = t + 1 if t >= target else t
    return parent, token


def draft_lattice(num_req: int, positions: int, k: int, seed: int, *, vocab: int = 152064,
                  temperature: float = 2.0, depths=None, quantum: float | None = None):
    """Candidate lattices of a step, one per request (the drafter's output).

    Per request r, position d, parent candidate i: edge logits
    z ~ N(0, temperature^2) over the K child candidates, turned into a
    log-softmax in float64 and stored as float32 (lp [R, D, K, K]). With
    ``quantum`` the logits are rounded to multiples of it first, which makes
    equal edge scores (and equal path scores) common. Candidate tokens are K
    distinct vocabulary ids per position (tok [R, D, K]); root tokens are
    uniform ids (roots [R]). ``depths`` (positions drafted per request)
    defaults to a uniform choice among 16, 12 and 8, capped at ``positions``.
    Returns (lp, tok, depths, roots).
    """
    rng = np.random.default_rng(seed)
    z = rng.normal(0.0, temperature, (num_req, positions, k, k))
    if quantum:
        z = np.round(z / quantum) * quantum
    z = z - z.max(axis=-1, keepdims=True)
    lp = (z - np.log(np.exp(z).sum(axis=-1, keepdims=True))).astype(np.float32)
    lp = np.minimum(lp, np.float32(0.0))
    tok = np.stack([np.stack([rng.choice(vocab, k, replace=False) for _ in range(positions)])
                    for _ in range(num_req)]).astype(np.int32)
    if depths is None:
        depths = np.minimum(rng.choice([16, 12, 8], num_req), positions)
    depths = np.asarray(depths, dtype=np.int32)
    roots = rng.integers(0, vocab, num_req).astype(np.int32)
    return lp, tok, depths, roots
