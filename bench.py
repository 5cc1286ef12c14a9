#!/usr/bin/env python3
"""Benchmark: one W12 verify pass of a 27B-class transformer block at M=32
tree-node rows, on one MI355X.

A step is one pass of the whole verify hot path over resident inputs:
  QKV   [Wq;Wk;Wv]   8192 x 5120   (Wq 6144x5120, Wk/Wv 1024x5120, fused:
                                    they share their input rows)
  O     Wo           5120 x 6144
  UP    [Wgate;Wup] 34816 x 5120   (fused, shared input)
  DOWN  Wdown        5120 x 17408
  HEAD  LM head    152064 x 5120 + fused argmax per row
  TREE  greedy acceptance of one 32-node draft tree
Weights are seeded synthetic bf16 (N(0, 0.02) x per-channel lognormal(0, 0.5)
scale, 1% zeros, 0.1% x64 outliers), packed to W12 and checked bit-for-bit
before timing; activations are seeded N(0, 1) bf16 rows.

value = algorithmic bytes of a step / step time. Algorithmic bytes of a
W12 GEMM = records 1.5NK + e_top N + esc_off 4(NK/1024+1) + escapes
4 n_esc + x 2MK + y 2MN (bf16 out); the head writes 4M bytes of ids instead
of y; the tree kernel reads/writes its int32 arrays.

Prints ONE JSON line (rank 0). Only N=1 is supported.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
M_ROWS = 32
HIDDEN, Q_OUT, KV_OUT, FFN, VOCAB = 5120, 6144, 1024, 17408, 152064
METRIC = "W12 verify-GEMM effective HBM GB/s at M=32 rows; % of MI355X HBM peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "w12_weight_streaming_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def gemm_bytes(pw, m: int, out_bytes_per_elem: int) -> int:
    return pw.nbytes() + 2 * m * pw.k + out_bytes_per_elem * m * pw.n


def build_block(w12, synth, torch, dev):
    """Pack the block and head; returns dict name -> (PackedW12, x)."""
    specs = [
        ("QKV", [(Q_OUT, HIDDEN, 1), (KV_OUT, HIDDEN, 2), (KV_OUT, HIDDEN, 3)]),
        ("O", [(HIDDEN, Q_OUT, 4)]),
        ("UP", [(FFN, HIDDEN, 5), (FFN, HIDDEN, 6)]),
        ("DOWN", [(HIDDEN, FFN, 7)]),
        ("HEAD", [(VOCAB, HIDDEN, 8)]),
    ]
    mats, pack_s, pack_in = {}, 0.0, 0
    for name, parts in specs:
        # seed = 1,000,000 * config + 1000 * layer + matrix (config 2, layer 0;
        # the head is config 4)
        cfg = 4 if name == "HEAD" else 2
        w = torch.cat([synth.weights_bf16(n, k, seed=1_000_000 * cfg + idx, device=dev)
                       for (n, k, idx) in parts], dim=0)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        pw = w12.w12_pack(w, check=True)       # raises unless bit-exact
        torch.cuda.synchronize()
        pack_s += time.perf_counter() - t0
        pack_in += w.numel() * 2
        k = parts[0][1]
        x = synth.activations_bf16(M_ROWS, k, seed=1_000_000 * cfg + parts[0][2] + 500, device=dev)
        mats[name] = (pw, x)
        del w
        log(f"packed {name}: {pw.n}x{pw.k}, {pw.n_esc} escapes "
            f"({pw.n_esc / (pw.n * pw.k):.4%}), {8 * pw.nbytes() / (pw.n * pw.k):.4f} bits/weight")
    return mats, pack_in / pack_s / 1e9


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true", help="replay the step as a HIP graph")
    ap.add_argument("--copy-gib", type=float, default=1.0,
                    help="size of the calibration copy launched after timing (0 = none)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the verify path is single-GPU here, see DESIGN.md for how it would shard.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import w12_weight_streaming_amd as w12

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w12.lib()

    mats, pack_gbps = build_block(w12, synth, torch, dev)
    order = ["QKV", "O", "UP", "DOWN"]
    outs = {n: torch.empty(M_ROWS, mats[n][0].n, dtype=torch.bfloat16, device=dev) for n in order}
    head_pw, head_x = mats["HEAD"]
    ws = w12.workspace(max(w12.gemm_workspace_bytes(mats[n][0].n, mats[n][0].k, M_ROWS)
                           for n in order + ["HEAD"]), dev)

    # tree inputs: one 32-node tree over the verify rows (config 4 shape:
    # depth <= 16, a node's token equals its parent row's argmax w.p. 0.7)
    idx0, _ = w12.w12_head_argmax(head_pw, head_x, ws=ws, with_max=False)
    am = idx0.cpu().numpy().astype(np.int32)
    parent, token = synth.random_tree(M_ROWS, 16, am, None, 0.7, seed=4_000_000 + 9, vocab=VOCAB)
    t_off = torch.tensor([0, M_ROWS], dtype=torch.int32, device=dev)
    t_par = torch.tensor(parent, dtype=torch.int32, device=dev)
    t_tok = torch.tensor(token, dtype=torch.int32, device=dev)

    def launch(name):
        if name == "HEAD":
            return w12.w12_head_argmax(head_pw, head_x, ws=ws, with_max=False)[0]
        if name == "TREE":
            return w12.tree_accept(t_off, t_par, t_tok, head_idx[0])
        pw, x = mats[name]
        return w12.w12_gemm(pw, x, out=outs[name], ws=ws)

    head_idx = [idx0]

    def step():
        for n in order:
            launch(n)
        head_idx[0] = launch("HEAD")
        launch("TREE")

    names = order + ["HEAD", "TREE"]
    step_bytes = {n: gemm_bytes(mats[n][0], M_ROWS, 2) for n in order}
    step_bytes["HEAD"] = head_pw.nbytes() + 2 * M_ROWS * HIDDEN + 4 * M_ROWS
    step_bytes["TREE"] = 4 * (2 + 3 * M_ROWS) + 4 * (2 + M_ROWS)
    total_bytes = sum(step_bytes.values())

    graph = None
    if args.graph:
        step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()

    run = graph.replay if graph is not None else step
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        run()
    end.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps

    # correctness of what was timed: the accepted path is a valid greedy path
    acc, path, bonus = w12.tree_accept(t_off, t_par, t_tok, head_idx[0])
    torch.cuda.synchronize()

    # per-kernel durations, measured with events on the launch stream inside
    # full passes (so every launch streams its weights from HBM)
    reps = max(5, min(args.steps, 20))
    ev = {n: [] for n in names}
    for _ in range(reps):
        for n in names:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            r = launch(n)
            if n == "HEAD":
                head_idx[0] = r
            b.record()
            ev[n].append((a, b))
    torch.cuda.synchronize()
    kern_us = {n: 1000.0 * sum(a.elapsed_time(b) for a, b in ev[n]) / reps for n in names}

    if args.copy_gib > 0:  # plain copy of known size, the HBM-counter calibration reference
        nb = int(args.copy_gib * (1 << 30))
        src = torch.empty(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    block_us = sum(kern_us[n] for n in order)
    block_bytes = sum(step_bytes[n] for n in order)
    value = total_bytes / (ms_per_step * 1e-3) / 1e9
    block_gbps = block_bytes / (block_us * 1e-6) / 1e9
    head_gbps = step_bytes["HEAD"] / (kern_us["HEAD"] * 1e-6) / 1e9

    # roofline of the dominant kernel (most time per step)
    dominant = "HEAD" if kern_us["HEAD"] >= block_us else "BLOCK"
    if dominant == "HEAD":
        ach, kname = head_gbps, ("gemm_mfma_kernel<1,1>: LM head 152064x5120 + fused argmax, M=32 "
                                 "(event time of the w12_head_argmax call, x pre-pass included)")
        per_launch = step_bytes["HEAD"]
    else:
        ach, kname = block_gbps, ("gemm_mfma_kernel<1,0>: block GEMMs at M=32 "
                                  "(event time of the w12_gemm calls, x pre-pass included)")
        per_launch = block_bytes / len(order)
    traffic = None
    tfile = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if os.path.exists(tfile):
        with open(tfile) as f:
            t = json.load(f)
        if t.get("kernel_source_hash") == kernel_source_hash():
            traffic = t.get("per_launch_bytes", {}).get(dominant)
    roofline = {"bound": "hbm", "kernel": kname, "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "algorithmic_bytes_per_launch": int(per_launch)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(mats, synth, torch)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "config": {
            "workload": "verify pass of one 27B-class block (Wq|Wk|Wv 8192x5120, Wo 5120x6144, "
                        "Wgate|Wup 34816x5120, Wdown 5120x17408) + 152064x5120 LM-head argmax "
                        "+ 32-node tree acceptance, all weights W12",
            "rows": M_ROWS,
            "bytes_per_step": int(total_bytes),
            "graph": bool(args.graph),
        },
        "breakdown_us": {n: round(v, 2) for n, v in kern_us.items()},
        "block_gemm_GBps": round(block_gbps, 1),
        "head_GBps": round(head_gbps, 1),
        "pack_GBps_bf16_in": round(pack_gbps, 1),
        "accepted": {"accept_len": int(acc[0]), "bonus": int(bonus[0])},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(mats, synth, torch):
    """The oracle (decode + fp32 matmul) on a bounded sample: the Wo matrix
    (5120 x 6144) at M=32, timed on this host's cores."""
    import numpy as np

    from oracle import baseline, w12_format  # noqa: F401  (test infrastructure)
    pw, x = mats["O"]
    packed = {"records": pw.records.cpu().numpy(), "e_top": pw.e_top.cpu().numpy(),
              "esc_off": pw.esc_off.cpu().numpy().view(np.uint32),
              "esc": pw.esc.cpu().numpy()[:pw.n_esc].view(np.uint32)}
    xb = synth.bits_u16(x)
    first = baseline.time_cpu_verify_gemm(packed, pw.n, pw.k, xb, reps=1)
    # about 10 s of CPU work in all: repeat the same GEMM
    reps = max(1, min(60, int(10.0 / max(first["seconds"], 1e-3))))
    r = baseline.time_cpu_verify_gemm(packed, pw.n, pw.k, xb, reps=reps)
    nbytes = gemm_bytes(pw, M_ROWS, 4)
    return {"value": round(nbytes / r["seconds"] / 1e9, 3), "unit": "GB/s",
            "cores": r["threads"], "kind": "oracle",
            "sample": f"Wo 5120x6144 W12 verify GEMM at M=32 (oracle decode + fp32 matmul), "
                      f"{reps + 1} runs, {r['seconds'] * reps + first['seconds']:.1f} s of CPU time"}


if __name__ == "__main__":
    main()
