"""CPU oracle for the W12 verify path -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct numpy implementation of what the HIP path
computes. Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg
may import or call anything here; the product path (the package
w12_weight_streaming_amd) never does, and shares no code with this package.

Sources (the pages these functions follow):
  [S1] "SpecPilot: Autonomous Algorithm Discovery and Systems Optimization for
       Speculative Decoding" -- long-form summary (jaehun.me):
       section 1.1 (greedy acceptance, tau range), 1.2 (lossless / exact pass,
       near-ties from floating-point order), 2.4 (discarded-candidate example),
       4.1 (W12 format, record, stream-K determinism, LM head argmax),
       4.2 (best-first tree: parent-conditioned edge scores, the N nodes
       with the highest path score), 4.3 (tree verification accepts the
       longest matching path + bonus; 8-bit view read by the Q pass),
       4.4 (shared node budget across the requests of a step).
  [S2] the same paper's digest page (agihunt.info), W12 paragraph: sign +
       4-bit exponent offset + all 7 mantissa bits; load-time check.
  [S3] "Speculative decoding" (poot-llm docs), section "What a round
       guarantees": greedy rows keep drafts equal to the target argmax, then
       the target's own next token.

Modules:
  w12_format -- pack / decode / layout / sizes           (parity pinned)
  verify     -- FP64 GEMM reference + bound, head argmax with near-tie
                classification, the top-k candidate ids of a row (which the
                tests draw mismatching draft tokens from), brute-force tree
                acceptance (parity pinned)
  tree_build -- best-first draft trees under a shared row budget (pinned)
  certified_head -- the certified INT8 LM head: INT8 copy with power-of-two
                block scales, per-row Cauchy-Schwarz bounds, pruning and
                exact rescoring (pinned)
  baseline   -- the timed CPU baseline (oracle decode + FP32 matmul), pinned
                to the fp64 GEMM reference within the GEMM bound

Every function here is pinned by a `-m "not gpu"` test against something
other than itself (closed forms, IEEE value semantics, brute force over
exact integer data, the pages' worked example); none is "parity unpinned".
"""
from . import w12_format, verify, baseline, certified_head  # noqa: F401
