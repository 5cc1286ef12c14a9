#!/usr/bin/env python3
"""Benchmark: one W12 verify pass of a 64-layer 27B-class stack at M=32
tree-node rows, then the LM-head argmax and tree acceptance, on one MI355X.

A step is one pass of the whole verify hot path over resident inputs:
  64 layers, each
    QKV   [Wq;Wk;Wv]   8192 x 5120   (Wq 6144x5120, Wk/Wv 1024x5120, fused:
                                      they share their input rows)
    O     Wo           5120 x 6144
    UP    [Wgate;Wup] 34816 x 5120   (fused, shared input)
    DOWN  Wdown        5120 x 17408
  HEAD  LM head    152064 x 5120 + fused argmax per row
  TREE  greedy acceptance of one 32-node draft tree
Every layer has its own seeded synthetic weights (N(0, 0.02) x per-channel
lognormal(0, 0.5) scale, 1% zeros, 0.1% x64 outliers), packed to W12 and
checked bit-for-bit before timing (about 34 GB of W12 resident in HBM), and
its own seeded N(0, 1) bf16 input rows, so nothing is served from the caches
between layers.

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
LAYERS = 64
HIDDEN, Q_OUT, KV_OUT, FFN, VOCAB = 5120, 6144, 1024, 17408, 152064
METRIC = "W12 verify-GEMM effective HBM GB/s at M=32 rows; % of MI355X HBM peak"
# (name, out channels, in channels) of one layer's four W12 GEMMs
LAYER_SHAPES = (("QKV", Q_OUT + 2 * KV_OUT, HIDDEN), ("O", HIDDEN, Q_OUT),
                ("UP", 2 * FFN, HIDDEN), ("DOWN", HIDDEN, FFN))
# kernel each call type runs at M=32 on 256 compute units (the plan picks
# 2-strip tiles for Wo, 4-strip tiles for the others)
KERNEL_OF = {"QKV": "gemm_mfma_kernel<1, 0, false, 4, 0>", "O": "gemm_mfma_kernel<1, 0, false, 2, 0>",
             "UP": "gemm_mfma_kernel<1, 0, false, 4, 0>", "DOWN": "gemm_mfma_kernel<1, 0, false, 4, 0>",
             "HEAD": "gemm_mfma_kernel<1, 1, false, 4, 0>", "TREE": "tree_accept_kernel"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# The sources the verify GEMM kernels are built from: the counter traffic
# stored with the profiles holds only while these are unchanged.
GEMM_SOURCES = ("w12_gemm.hip", "w12_device.h", "w12_internal.h")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "w12_weight_streaming_amd", "csrc")
    for f in GEMM_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def gemm_bytes(pw, m: int, out_bytes_per_elem: int) -> int:
    return pw.nbytes() + 2 * m * pw.k + out_bytes_per_elem * m * pw.n


def head_bytes(pw, m: int) -> int:
    return pw.nbytes() + 2 * m * pw.k + 4 * m


def tree_bytes(m: int) -> int:
    return 4 * (2 + 3 * m) + 4 * (2 + m)


def traffic_for(name: str):
    """Counter-measured HBM bytes per launch of a call type, if the stored
    counters were taken on the current kernel sources."""
    tfile = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(tfile):
        return None
    with open(tfile) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("per_launch_bytes", {}).get(name)


def pack_layers(w12, synth, torch, dev, layers, keep_dense=False):
    """W12-pack `layers` layers of the 27B-class shape (seed 3,000,000 +
    1000 * layer + matrix) with the load-time check; each GEMM gets its own
    input rows (seed + 500). Returns ([{name: (PackedW12, x)}], dense or
    None, pack GB/s of bf16 input)."""
    mats, dense = [], ([] if keep_dense else None)
    pack_s, pack_in = 0.0, 0
    for li in range(layers):
        row, drow = {}, {}
        for j, (name, n, k) in enumerate(LAYER_SHAPES):
            seed = 1_000_000 * 3 + 1000 * li + j + 1
            w = synth.weights_bf16(n, k, seed=seed, device=dev)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            pw = w12.w12_pack(w, check=True)       # raises W12_ECORRUPT unless bit-exact
            torch.cuda.synchronize()
            pack_s += time.perf_counter() - t0
            pack_in += w.numel() * 2
            x = synth.activations_bf16(M_ROWS, k, seed=seed + 500, device=dev)
            row[name] = (pw, x)
            if keep_dense:
                drow[name] = w
            del w
        mats.append(row)
        if keep_dense:
            dense.append(drow)
        if li % 16 == 15 or li == layers - 1:
            log(f"packed {li + 1} layers")
    return mats, dense, pack_in / max(pack_s, 1e-9) / 1e9


def pack_head(w12, synth, torch, dev, keep_dense=False):
    """The 152064x5120 LM head (seed 4,000,008), its 32 input rows, and the
    top-16 candidate ids of every row (drawn with torch from the bf16
    source weights: synthetic input for the draft tree, outside any timed
    region)."""
    w = synth.weights_bf16(VOCAB, HIDDEN, seed=1_000_000 * 4 + 8, device=dev)
    pw = w12.w12_pack(w, check=True)
    x = synth.activations_bf16(M_ROWS, HIDDEN, seed=1_000_000 * 4 + 508, device=dev)
    logits = torch.cat([x.float() @ w[v0:v0 + 16384].float().t() for v0 in range(0, VOCAB, 16384)], dim=1)
    top16 = torch.topk(logits, 16, dim=1).indices.cpu().numpy()
    del logits
    log(f"packed HEAD: {pw.n}x{pw.k}, {pw.n_esc} escapes ({pw.n_esc / (pw.n * pw.k):.4%}), "
        f"{8 * pw.nbytes() / (pw.n * pw.k):.4f} bits/weight")
    return pw, x, top16, (w if keep_dense else None)


def run_pass(args, w12, synth, torch, dev):
    """The headline: 64 layers + LM head argmax + tree acceptance at M=32."""
    import numpy as np

    layers = args.layers
    keep_dense = not args.no_dense
    mats, dense, pack_gbps = pack_layers(w12, synth, torch, dev, layers, keep_dense)
    head_pw, head_x, top16, head_dense = pack_head(w12, synth, torch, dev, keep_dense)
    outs = {name: torch.empty(M_ROWS, n, dtype=torch.bfloat16, device=dev) for name, n, _ in LAYER_SHAPES}
    ws = w12.workspace(max([w12.gemm_workspace_bytes(n, k, M_ROWS) for _, n, k in LAYER_SHAPES] +
                           [w12.gemm_workspace_bytes(head_pw.n, head_pw.k, M_ROWS)]), dev)

    # tree inputs: one 32-node tree over the head's rows (depth <= 16; a
    # node's token equals its parent row's argmax w.p. 0.7, else another of
    # that row's top-16 candidates)
    idx0, _ = w12.w12_head_argmax(head_pw, head_x, ws=ws, with_max=False)
    am = idx0.cpu().numpy().astype(np.int32)
    parent, token = synth.random_tree(M_ROWS, 16, am, top16, 0.7, seed=4_000_000 + 9, vocab=VOCAB)
    t_off = torch.tensor([0, M_ROWS], dtype=torch.int32, device=dev)
    t_par = torch.tensor(parent, dtype=torch.int32, device=dev)
    t_tok = torch.tensor(token, dtype=torch.int32, device=dev)
    head_idx = [idx0]

    def launch(name, li=0):
        if name == "HEAD":
            head_idx[0] = w12.w12_head_argmax(head_pw, head_x, ws=ws, with_max=False)[0]
            return
        if name == "TREE":
            return w12.tree_accept(t_off, t_par, t_tok, head_idx[0])
        pw, x = mats[li][name]
        w12.w12_gemm(pw, x, out=outs[name], ws=ws)

    order = [name for name, _, _ in LAYER_SHAPES]

    def step():
        for li in range(layers):
            for name in order:
                launch(name, li)
        launch("HEAD")
        launch("TREE")

    step_bytes = {name: sum(gemm_bytes(row[name][0], M_ROWS, 2) for row in mats) for name in order}
    step_bytes["HEAD"] = head_bytes(head_pw, M_ROWS)
    step_bytes["TREE"] = tree_bytes(M_ROWS)
    total_bytes = sum(step_bytes.values())
    calls = {name: layers for name in order}
    calls.update({"HEAD": 1, "TREE": 1})

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

    # the accepted path of what was timed
    acc, path, bonus = w12.tree_accept(t_off, t_par, t_tok, head_idx[0])
    torch.cuda.synchronize()

    # per-call durations: for each call type, all of its calls of a pass
    # launched back to back (every layer its own weights, so each launch
    # still streams from HBM), one pair of events on the launch stream
    # around the run; the mean per call is what the kernels of one call take
    # in a stream of such calls, launch gaps included
    reps = max(2, min(args.steps, 5))
    call_us = {}
    for name in order + ["HEAD", "TREE"]:
        n_calls = layers if name in order else 1
        seq = max(1, 16 // n_calls) if name not in order else 1  # >= 16 calls per timed run
        for li in range(n_calls):  # warm the launch path of this type
            launch(name, li)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            for _ in range(seq):
                for li in range(n_calls):
                    launch(name, li)
        b.record()
        torch.cuda.synchronize()
        call_us[name] = 1000.0 * a.elapsed_time(b) / (reps * seq * n_calls)

    if args.copy_gib > 0:  # plain copy of known size, the HBM-counter calibration reference
        nb = int(args.copy_gib * (1 << 30))
        src = torch.empty(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    value = total_bytes / (ms_per_step * 1e-3) / 1e9
    per_step_us = {n: call_us[n] * calls[n] for n in call_us}
    block_us = sum(per_step_us[n] for n in order)
    block_bytes = sum(step_bytes[n] for n in order)
    gbps_of = {n: step_bytes[n] / calls[n] / (call_us[n] * 1e-6) / 1e9 for n in call_us}

    # roofline of the dominant kernel: the call type with the most time per step
    dominant = max(order + ["HEAD"], key=lambda n: per_step_us[n])
    per_launch = step_bytes[dominant] // calls[dominant]
    roofline = {"bound": "hbm",
                "kernel": f"{KERNEL_OF[dominant]}: {dominant} at M=32, {calls[dominant]} launches per step "
                          "(mean time per call from events on the launch stream around the pass's calls of "
                          "this type run back to back; every kernel of the call included)",
                "achieved": round(gbps_of[dominant], 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(gbps_of[dominant] / HBM_PEAK_GBPS, 4), "traffic": traffic_for(dominant),
                "algorithmic_bytes_per_launch": int(per_launch),
                "avg_launch_us": round(call_us[dominant], 2)}

    dense_ctx = None
    if keep_dense:
        dense_ctx = dense_context(args, torch, dev, mats, dense, head_x, head_dense, layers, ms_per_step,
                                  head_idx[0])
        del dense, head_dense
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(mats[0], synth, torch)

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
            "workload": f"verify pass of a {layers}-layer 27B-class stack (per layer Wq|Wk|Wv 8192x5120, "
                        "Wo 5120x6144, Wgate|Wup 34816x5120, Wdown 5120x17408) + 152064x5120 LM-head "
                        "argmax + 32-node tree acceptance, all weights W12, each layer its own weights "
                        "and input rows",
            "rows": M_ROWS, "layers": layers,
            "bytes_per_step": int(total_bytes),
            "graph": bool(args.graph),
        },
        "us_per_pass": round(1000.0 * ms_per_step, 1),
        "us_per_layer": round(block_us / layers, 2),
        "block_gemm_GBps": round(block_bytes / (block_us * 1e-6) / 1e9, 1),
        "head_GBps": round(gbps_of["HEAD"], 1),
        "call_us": {n: round(v, 2) for n, v in call_us.items()},
        "call_GBps": {n: round(v, 1) for n, v in gbps_of.items() if n != "TREE"},
        "sum_of_call_us_per_step": round(sum(per_step_us.values()), 1),
        "pack_GBps_bf16_in": round(pack_gbps, 1),
        "accepted": {"accept_len": int(acc[0]), "bonus": int(bonus[0])},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "dense_bf16_context": dense_ctx,
    }
    print(json.dumps(line), flush=True)


def run_cert(args, w12, synth, torch, dev):
    """The certified INT8 head next to the W12 head: 152064x5120 at M=32,
    both timed on the launch stream with events over back-to-back calls."""
    import numpy as np

    w = synth.weights_bf16(VOCAB, HIDDEN, seed=1_000_000 * 4 + 8, device=dev)
    pw = w12.w12_pack(w, check=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    cert = w12.w12_cert8_pack(w, pw)
    torch.cuda.synchronize()
    cert_pack_s = time.perf_counter() - t0
    del w
    x = synth.activations_bf16(M_ROWS, HIDDEN, seed=1_000_000 * 4 + 508, device=dev)
    ws = w12.workspace(64 << 20, dev, "bench")
    wsc = w12.workspace(256 << 20, dev, "bench-cert")
    head = lambda i: w12.w12_head_argmax(pw, x, ws=ws, with_max=False)
    certified = lambda i: w12.w12_head_argmax_certified(pw, cert, x, ws=wsc, with_max=False)
    for _ in range(args.warmup):
        head(0)
        certified(0)
    torch.cuda.synchronize()
    reps = max(10, args.steps)
    t_head = min(time_events(head, reps) for _ in range(3))
    t_cert = min(time_events(certified, reps) for _ in range(3))
    idx_w, _ = w12.w12_head_argmax(pw, x, ws=ws, with_max=False)
    idx_c, _, cnt = w12.w12_head_argmax_certified(pw, cert, x, ws=wsc, with_max=False)
    cnt = cnt.cpu().numpy()
    head_b = head_bytes(pw, M_ROWS)
    # the INT8 pass reads the copy, W12's escape lists and x; the rescoring
    # reads about 7.5 KB of records per rescored row
    pass_b = cert.nbytes() + 4 * (pw.esc_off.numel() + pw.n_esc) + 2 * M_ROWS * HIDDEN
    line = {
        "metric": "LM-head argmax time at M=32 (152064x5120): certified INT8 head vs W12 head",
        "value": round(t_cert, 2), "unit": "us", "n_gpus": 1, "steps": reps, "warmup": args.warmup,
        "ms_per_step": round(t_cert / 1000.0, 4), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "LM head 152064x5120 + argmax at M=32: INT8 copy pass (32-weight power-of-two "
                               "block scales, W12 escapes exact), per-row Cauchy-Schwarz pruning, exact W12 "
                               "rescoring of the survivors", "rows": M_ROWS},
        "w12_head_us": round(t_head, 2),
        "speedup_vs_w12_head": round(t_head / t_cert, 3),
        "argmax_agrees_with_w12_head": float((idx_w == idx_c).float().mean()),
        "rescored_per_row": {"median": int(np.median(cnt)), "max": int(cnt.max()), "of": VOCAB},
        "bytes": {"w12_head": int(head_b), "int8_pass": int(pass_b), "int8_copy": int(cert.nbytes())},
        "int8_pass_GBps": round(pass_b / (t_cert * 1e-6) / 1e9, 1),
        "cert_pack_s": round(cert_pack_s, 4),
    }
    print(json.dumps(line), flush=True)


def dense_context(args, torch, dev, mats, dense, head_x, head_dense, layers, ms_w12, idx_w12):
    """Context only: the same pass on the dense bf16 source weights through
    torch.matmul (hipBLASLt) and torch.argmax, timed the same way."""
    F = torch.nn.functional
    order = [name for name, _, _ in LAYER_SHAPES]
    ys = {name: torch.empty(M_ROWS, n, dtype=torch.bfloat16, device=dev) for name, n, _ in LAYER_SHAPES}

    def dense_step():
        for li in range(layers):
            for name in order:
                torch.matmul(mats[li][name][1], dense[li][name].t(), out=ys[name])
        return torch.argmax(F.linear(head_x, head_dense).float(), dim=1)

    for _ in range(max(1, args.warmup)):
        dense_step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        d_idx = dense_step()
    b.record()
    torch.cuda.synchronize()
    d_ms = a.elapsed_time(b) / args.steps
    d_bytes = sum(2 * dense[li][n].numel() + 2 * M_ROWS * dense[li][n].shape[1] + 2 * M_ROWS * dense[li][n].shape[0]
                  for li in range(layers) for n in order) + 2 * head_dense.numel() + 2 * M_ROWS * HIDDEN
    return {"what": "the pass's GEMMs and the head argmax on the bf16 source weights via torch.matmul "
                    "and torch.argmax (no tree acceptance); context, not a baseline",
            "ms_per_step": round(d_ms, 4), "bytes_per_step": int(d_bytes),
            "GBps": round(d_bytes / (d_ms * 1e-3) / 1e9, 1),
            "w12_step_speedup": round(d_ms / ms_w12, 3),
            "head_argmax_agrees": float((d_idx == idx_w12).float().mean())}


def run_block(args, w12, synth, torch, dev):
    """One 27B-class block + the LM head + tree at M=32: the pass with one
    layer (a quick line for development; the weights then fit in the
    last-level cache between steps, so it flatters the block GEMMs)."""
    args.layers = 1
    return run_pass(args, w12, synth, torch, dev)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--layers", type=int, default=LAYERS, help="layers of the pass workload (default 64)")
    ap.add_argument("--rows", type=int, default=192,
                    help="verify rows of the batched workload (default 192 = 24 trees x 8 nodes; at most 512)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the dense bf16 context timing of the same pass")
    ap.add_argument("--graph", action="store_true", help="replay the step as a HIP graph")
    ap.add_argument("--copy-gib", type=float, default=1.0,
                    help="size of the calibration copy launched after timing (0 = none)")
    ap.add_argument("--workload", choices=("pass", "block", "batched", "sweep", "qpass", "tree", "cert"),
                    default="pass",
                    help="pass: 64 layers + LM head argmax + tree acceptance at M=32 (the headline line); "
                         "block: the same with one layer; "
                         "batched: Wup 17408x5120 and Wdown 5120x17408 at M=192 (--rows) with 3%% zeros "
                         "and 2%% outliers; "
                         "sweep: Wgate|Wup 34816x5120 over M = 1 ... 512; "
                         "qpass: one block + head through the Q pass (8-bit view only) next to the exact pass; "
                         "tree: best-first draft trees, 24 requests sharing 192 rows and one 32-row tree; "
                         "cert: the certified INT8 LM head next to the W12 head at M=32")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the verify path runs on one GPU here; across GPUs the weights would shard by "
              "32-channel strips (column-parallel layers, the LM head) or 256-column records (row-parallel ones).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    import w12_weight_streaming_amd as w12

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w12.lib()
    fn = {"pass": run_pass, "block": run_block, "batched": run_batched, "sweep": run_sweep,
          "qpass": run_qpass, "tree": run_tree, "cert": run_cert}[args.workload]
    return fn(args, w12, synth, torch, dev)


def clone_packed(w12, pw):
    """A distinct device copy of every buffer of a packed matrix."""
    return w12.PackedW12(pw.n, pw.k, pw.records.clone(), pw.e_top.clone(), pw.esc_off.clone(),
                         pw.esc.clone(), pw.n_esc)


def time_events(fn, reps):
    """Mean microseconds of fn() over reps launches, timed with events on the
    current stream."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(reps):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return 1000.0 * a.elapsed_time(b) / reps


def run_batched(args, w12, synth, torch, dev):
    """Batched verify (24 trees x 8 nodes = 192 rows): Wup 17408x5120 then
    Wdown 5120x17408, 3% zeros and 2% x64 outliers, bf16 out; --rows sets
    another row count (every count up to 512 is one launch per matrix). Each
    matrix is held in enough distinct packed copies (>= 1 GiB in all) that
    every call streams its weights from HBM, not from the 256 MB last-level
    cache."""
    m = args.rows
    assert 1 <= m <= 512, "--rows must be in [1, 512]"
    mats = []
    for name, n, k, idx in (("UP", FFN, HIDDEN, 1), ("DOWN", HIDDEN, FFN, 2)):
        seed = 1_000_000 * 5 + idx
        w = synth.weights_bf16(n, k, seed=seed, p_zero=0.03, p_outlier=0.02, device=dev)
        pw = w12.w12_pack(w, check=True)
        del w
        x = synth.activations_bf16(m, k, seed=seed + 500, device=dev)
        ncopy = max(2, -(-(1 << 30) // pw.nbytes()))
        copies = [pw] + [clone_packed(w12, pw) for _ in range(ncopy - 1)]
        y = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
        mats.append((name, copies, x, y))
        log(f"packed {name}: {n}x{k}, {pw.n_esc} escapes ({pw.n_esc / (n * k):.4%}), {ncopy} copies")
    ws = w12.workspace(max(w12.gemm_workspace_bytes(c[0].n, c[0].k, m) for _, c, _, _ in mats), dev)

    def step(i):
        for _, copies, x, y in mats:
            w12.w12_gemm(copies[i % len(copies)], x, out=y, ws=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    us = time_events(step, args.steps)
    per = {}
    for name, copies, x, y in mats:
        per[name] = time_events(lambda i, c=copies, x=x, y=y: w12.w12_gemm(c[i % len(c)], x, out=y, ws=ws),
                                max(8, args.steps))
    nbytes = sum(gemm_bytes(c[0], m, 2) for _, c, _, _ in mats)
    flops = sum(2.0 * m * c[0].n * c[0].k for _, c, _, _ in mats)
    gbps = nbytes / (us * 1e-6) / 1e9
    tflops = flops / (us * 1e-6) / 1e12
    line = {
        "metric": f"W12 batched verify GEMM effective HBM GB/s at M={m} rows",
        "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(us / 1000.0, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"batched verify: Wup 17408x5120 + Wdown 5120x17408, M={m} rows, "
                               "3% zeros + 2% x64 outliers, bf16 out, >= 1 GiB of rotated copies",
                   "rows": m, "bytes_per_step": int(nbytes), "flops_per_step": flops},
        "breakdown_us": {n: round(v, 2) for n, v in per.items()},
        "roofline": {"hbm": {"achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                             "frac": round(gbps / HBM_PEAK_GBPS, 4)},
                     "mfma_bf16": {"achieved": round(tflops, 1), "peak": BF16_MFMA_PEAK_TFLOPS,
                                   "unit": "TFLOP/s", "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4)}},
    }
    print(json.dumps(line), flush=True)


def run_tree(args, w12, synth, torch, dev):
    """Best-first draft trees on 16-position x top-16 lattices: 24 requests
    (drafting 16, 12 or 8 positions) sharing 192 rows, and one request with a
    32-row tree; device time per build, with the oracle's time beside it."""
    import time
    cases = {"shared_24x192": (24, 192, 1_000_000 * 6), "single_32": (1, 32, 1_000_000 * 6 + 1)}
    res = {}
    for name, (R, budget, seed) in cases.items():
        lp, tok, depths, roots = synth.draft_lattice(R, 16, 16, seed, depths=None if R > 1 else [16])
        import ctypes
        lp_d, tok_d, dep_d, root_d = [torch.from_numpy(a).to(dev) for a in (lp, tok, depths, roots)]
        ws = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
        outs = [torch.empty(n, dtype=torch.int32, device=dev) for n in (R + 1, budget, budget, budget)]
        score = torch.empty(budget, dtype=torch.float32, device=dev)
        L = w12.lib()
        stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        P = lambda t: ctypes.c_void_p(t.data_ptr())

        def build(i):
            st = L.w12_tree_build(R, 16, 16, P(lp_d), P(tok_d), P(dep_d), P(root_d), budget, P(ws), ws.numel(),
                                  P(outs[0]), P(outs[1]), P(outs[2]), P(outs[3]), P(score), stream)
            assert st == 0, st
        for _ in range(args.warmup):
            build(0)
        torch.cuda.synchronize()
        us = min(time_events(build, args.steps) for _ in range(3))
        t0 = time.perf_counter()
        from oracle import tree_build as TB
        TB.shared_budget(lp, tok, depths, roots, budget)
        res[name] = {"requests": R, "rows": budget, "us": round(us, 2),
                     "oracle_cpu_us": round((time.perf_counter() - t0) * 1e6, 1)}
    line = {
        "metric": "best-first draft tree build time (16 positions x top-16 lattice)", "value": res["shared_24x192"]["us"],
        "unit": "us", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(res["shared_24x192"]["us"] / 1000.0, 4), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "24 requests sharing 192 rows (value) and one 32-row tree, 16 x 16 lattices"},
        "cases": res,
    }
    print(json.dumps(line), flush=True)


def run_sweep(args, w12, synth, torch, dev):
    """Time flatness in rows: Wgate|Wup 34816x5120 (block weight recipe) at
    M = 1 ... 512, over >= 1 GiB of distinct packed copies, bf16 out. Above
    192 rows a call runs as launches of at most 192 rows."""
    rows = (1, 2, 4, 5, 8, 12, 16, 32, 48, 64, 96, 128, 192, 256, 384, 512)
    w = torch.cat([synth.weights_bf16(FFN, HIDDEN, seed=1_000_000 * 2 + j, device=dev) for j in (5, 6)], dim=0)
    pw = w12.w12_pack(w, check=True)
    del w
    ncopy = max(2, -(-(1 << 30) // pw.nbytes()))
    copies = [pw] + [clone_packed(w12, pw) for _ in range(ncopy - 1)]
    ws = w12.workspace(max(w12.gemm_workspace_bytes(pw.n, pw.k, m) for m in rows), dev)
    by_rows = {}
    for m in rows:
        x = synth.activations_bf16(m, HIDDEN, seed=1_000_000 * 2 + 505, device=dev)
        y = torch.empty(m, pw.n, dtype=torch.bfloat16, device=dev)
        call = lambda i, x=x, y=y: w12.w12_gemm(copies[i % ncopy], x, out=y, ws=ws)
        for i in range(max(args.warmup, ncopy)):
            call(i)
        torch.cuda.synchronize()
        us = min(time_events(call, max(32, args.steps)) for _ in range(5))
        nbytes = gemm_bytes(pw, m, 2)
        by_rows[m] = {"us": round(us, 2), "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                      "TFLOPs": round(2.0 * m * pw.n * pw.k / (us * 1e-6) / 1e12, 1)}
        log(f"m={m}: {by_rows[m]}")
    v = by_rows[M_ROWS]["GBps"]
    line = {
        "metric": "W12 verify GEMM effective HBM GB/s vs rows (Wgate|Wup 34816x5120)",
        "value": v, "unit": "GB/s", "n_gpus": 1, "steps": max(32, args.steps), "warmup": args.warmup,
        "ms_per_step": round(by_rows[M_ROWS]["us"] / 1000.0, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "Wgate|Wup 34816x5120 (1.07% escapes), bf16 out, >= 1 GiB of rotated copies; "
                               "value is the M=32 point", "rows": list(rows)},
        "by_rows": {str(m): r for m, r in by_rows.items()},
        "pct_of_hbm_peak": round(100.0 * v / HBM_PEAK_GBPS, 2),
    }
    print(json.dumps(line), flush=True)


def qpass_bytes(pw, m: int, out_bytes_per_elem: int) -> int:
    """What a Q pass reads and writes: the 8-bit view (2/3 of the records) +
    e_top + esc_off + escape entries + x + y."""
    return pw.nbytes() - pw.n * pw.k // 2 + 2 * m * pw.k + out_bytes_per_elem * m * pw.n


def run_qpass(args, w12, synth, torch, dev):
    """The block step at M=32 through the Q pass (QKV, O, UP, DOWN GEMMs and
    the LM-head argmax, reading only the 8-bit view of every record), next to
    the exact pass, with the head's top-1 agreement between the two."""
    layers, _, _ = pack_layers(w12, synth, torch, dev, 1)
    mats = layers[0]
    head_pw, head_x, _, _ = pack_head(w12, synth, torch, dev)
    order = ["QKV", "O", "UP", "DOWN"]
    outs = {n: torch.empty(M_ROWS, mats[n][0].n, dtype=torch.bfloat16, device=dev) for n in order}
    ws = w12.workspace(max([w12.gemm_workspace_bytes(mats[n][0].n, mats[n][0].k, M_ROWS) for n in order] +
                           [w12.gemm_workspace_bytes(head_pw.n, head_pw.k, M_ROWS)]), dev)

    def step(qp):
        for n in order:
            w12.w12_gemm(mats[n][0], mats[n][1], out=outs[n], ws=ws, qpass=qp)
        return w12.w12_head_argmax(head_pw, head_x, ws=ws, with_max=False, qpass=qp)[0]

    res = {}
    for qp in (False, True):
        for _ in range(args.warmup):
            step(qp)
        torch.cuda.synchronize()
        res[qp] = min(time_events(lambda i, qp=qp: step(qp), args.steps) for _ in range(3))
    idx_q = step(True).cpu()
    idx_e = step(False).cpu()
    agree = float((idx_q == idx_e).float().mean())
    # top-1 agreement over more rows: 256 fresh activation rows on the head
    xs = synth.activations_bf16(256, HIDDEN, seed=1_000_000 * 4 + 900, device=dev)
    a1 = w12.w12_head_argmax(head_pw, xs, with_max=False, qpass=True)[0]
    a2 = w12.w12_head_argmax(head_pw, xs, with_max=False)[0]
    agree_256 = float((a1 == a2).float().mean())
    qbytes = sum(qpass_bytes(mats[n][0], M_ROWS, 2) for n in order) + \
        qpass_bytes(head_pw, M_ROWS, 0) + 4 * M_ROWS
    ebytes = sum(gemm_bytes(mats[n][0], M_ROWS, 2) for n in order) + \
        head_pw.nbytes() + 2 * M_ROWS * HIDDEN + 4 * M_ROWS
    gbps = qbytes / (res[True] * 1e-6) / 1e9
    line = {
        "metric": "W12 Q-pass (8-bit view) verify step effective HBM GB/s at M=32 rows",
        "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(res[True] / 1000.0, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "Q pass of one 27B-class block (QKV, O, UP, DOWN) + LM-head argmax at M=32",
                   "rows": M_ROWS, "bytes_per_step": int(qbytes)},
        "exact_ms_per_step": round(res[False] / 1000.0, 4),
        "exact_GBps": round(ebytes / (res[False] * 1e-6) / 1e9, 1),
        "speedup_vs_exact": round(res[False] / res[True], 3),
        "head_top1_agreement_32_rows": agree, "head_top1_agreement_256_rows": agree_256,
        "pct_of_hbm_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(layer, synth, torch):
    """The oracle (decode + fp32 matmul) on a bounded sample of the pass:
    the four GEMMs of one layer at M=32, timed on this host's cores, once
    with every BLAS thread and once with one."""
    import numpy as np

    from oracle import baseline  # test infrastructure: the timed CPU baseline
    items = []
    for name, _, _ in LAYER_SHAPES:
        pw, x = layer[name]
        packed = {"records": pw.records.cpu().numpy(), "e_top": pw.e_top.cpu().numpy(),
                  "esc_off": pw.esc_off.cpu().numpy().view(np.uint32),
                  "esc": pw.esc.cpu().numpy()[:pw.n_esc].view(np.uint32)}
        items.append((packed, pw.n, pw.k, synth.bits_u16(x), gemm_bytes(pw, M_ROWS, 4)))
    nbytes = sum(it[4] for it in items)

    def leg(threads):
        secs, used = 0.0, 0
        for packed, n, k, xb, _ in items:
            r = baseline.time_cpu_verify_gemm(packed, n, k, xb, reps=1, threads=threads)
            secs += r["seconds"]
            used = max(used, r["threads"])
        return secs, used

    s_all, t_all = leg(None)
    s_one, t_one = leg(1)
    return {"value": round(nbytes / s_all / 1e9, 3), "unit": "GB/s", "cores": t_all, "kind": "oracle",
            "sample": f"one layer of the pass (QKV 8192x5120, O 5120x6144, UP 34816x5120, DOWN 5120x17408) "
                      f"at M=32: oracle decode + fp32 matmul, {s_all:.1f} s with {t_all} BLAS threads "
                      f"(the decode is single-threaded numpy)",
            "one_thread": {"value": round(nbytes / s_one / 1e9, 3), "seconds": round(s_one, 2),
                           "cores": t_one}}


if __name__ == "__main__":
    main()
