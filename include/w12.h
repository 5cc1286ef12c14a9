/*
 * w12.h -- C ABI of libw12: lossless 12-bit (W12) weight streaming for the
 * verification pass of greedy speculative decoding, on AMD Instinct MI355X
 * (gfx950).
 *
 * Sources for what each call computes:
 *   [S1] "SpecPilot: Autonomous Algorithm Discovery and Systems Optimization
 *        for Speculative Decoding", long-form summary (jaehun.me):
 *        section 1.1 (greedy acceptance), 1.2 (lossless = exact-pass argmax),
 *        4.1 (W12 format, 12 KB records, deterministic stream-K GEMM, LM
 *        head argmax), 4.3 (tree verification: longest matching path + bonus).
 *   [S2] the same paper's digest page (agihunt.info), W12 paragraph (sign +
 *        4-bit exponent offset + all 7 mantissa bits, load-time check).
 *   [S3] "Speculative decoding" (poot-llm docs), "What a round guarantees"
 *        (greedy rows keep drafts equal to the argmax, then one more token)
 *        and "What is refused" (typed refusal before anything runs).
 *
 * Conventions (all calls):
 *   - Every pointer argument is DEVICE memory owned by the caller, except
 *     `const w12_matrix *` descriptors and `size_t *` / `int64_t` outputs of
 *     the *_workspace queries, which live in host memory.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream) and return as soon as the kernels are enqueued.
 *   - Argument errors return W12_EINVAL before anything is launched (null
 *     pointers, shapes the format cannot hold, m outside [1, 512], bf16
 *     matrices / records / x / y not 16-byte aligned, e_top and u32 arrays
 *     not 4-byte aligned); a
 *     workspace smaller than its query returns W12_ENOSPC; a failed launch
 *     returns W12_EHIP.  Errors found on the device (a corrupt packed
 *     weight, an invalid tree) are reported through outputs, as each call
 *     states.  The library never allocates memory.
 *   - Workspaces ("ws") must be zero-filled before their first use. A
 *     workspace holds arrival counters, which every completed call returns
 *     to zero, and partial sums, which a call writes before it reads them;
 *     so one allocation serves any number of calls.  Calls that overlap in
 *     time must not share a workspace.
 *
 * W12 layout (readings of [S1] 4.1 and [S2] for gfx950):
 *   N output channels x K inputs, N % 32 == 0, K % 256 == 0, K <= 2^20.
 *   e_top[n]   window top E_n (biased bf16 exponent) in [16, 254]; the
 *              window [E_n - 15, E_n] is the one holding the most normal
 *              weights of channel n (smallest E_n on ties).
 *   records    N*K*3/2 bytes; record (s, r) = channels [32s, 32s+32) x
 *              k [256r, 256r+256) at byte (s*(K/256) + r) * 12288.  Bytes
 *              [0, 8192) hold the 8-bit view hi8 = s<<7 | o<<3 | m>>4
 *              (o = e - (E_n - 15)), bytes [8192, 12288) the low mantissa
 *              nibbles.  Weight (c, k') of a record, subtile t = k'/32,
 *              half h = (k'%32)/16, j = k'%16, lane = c + 32h:
 *                hi8 at t*1024 + lane*16 + j,
 *                lo4 at 8192 + t*512 + lane*8 + 4*(j/8) + j%4, high nibble
 *                when j%8 < 4, low nibble otherwise.
 *              Escaped weights (zero, denormal, Inf/NaN, out of window) hold
 *              code 0 and are listed in `esc`.
 *   esc_off    [N*K/1024 + 1] u32 offsets into esc, one per escape block
 *              (strip s, record r, subtile t), block id (s*(K/256)+r)*8 + t.
 *   esc        [max(1, esc_off[last])] u32 entries (the array always holds
 *              at least one element) bits<<16 | c<<5 | kk, c the
 *              channel in the strip, kk = k % 32; (c, kk) ascending within a
 *              block, so each channel's list runs in ascending k.
 */
#ifndef W12_H
#define W12_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  W12_OK = 0,
  W12_EINVAL = -1,  /* bad argument; nothing launched                    */
  W12_ENOSPC = -2,  /* workspace smaller than the matching query         */
  W12_EHIP = -3,    /* a HIP runtime call or kernel launch failed        */
  W12_ECORRUPT = -4 /* the load-time check found weights that do not
                       restore bit-for-bit: the weights are refused
                       ([S1] 4.1, [S2]; [S3] "What is refused"). No call
                       of the library returns it: w12_check reports a
                       count through device memory, and the caller that
                       reads a non-zero count refuses the weights with
                       this status (the Python binding raises it).     */
} w12_status;

typedef enum { W12_Y_F32 = 0, W12_Y_BF16 = 1 } w12_ydtype;

/* Device-resident W12 matrix (the five buffers above). */
typedef struct w12_matrix {
  int64_t n, k;
  const uint8_t *records;
  const uint8_t *e_top;
  const uint32_t *esc_off;
  const uint32_t *esc;
} w12_matrix;

/* Human-readable name of a w12_status (static string). */
const char *w12_strerror(int status);

/* ABI version, bumped on any layout or signature change. */
int w12_abi_version(void);

/* Number of escape blocks N*K/1024; esc_off holds one more entry. */
int64_t w12_num_blocks(int64_t n, int64_t k);

/*
 * w12_pack_plan -- first half of packing ([S1] 4.1: the weights are
 * converted once, at load; per output channel the 16-binade exponent window
 * holding the most weights, everything outside it on the escape list;
 * [S2] W12 paragraph).
 *   w        [n, k] bf16 bit patterns, row-major (read only).
 *   e_top    [n] out: window tops E_n.
 *   esc_off  [w12_num_blocks(n,k) + 1] out: escape offsets; esc_off[last]
 *            is the escape count the caller reads to size `esc`.
 */
w12_status w12_pack_plan(const uint16_t *w, int64_t n, int64_t k,
                         uint8_t *e_top, uint32_t *esc_off, hipStream_t stream);

/*
 * w12_pack -- second half of packing ([S1] 4.1; [S2]): writes the 12 KB
 * records (8-bit view plane, then low-nibble plane) and the escape entries
 * (exact bf16 bits of every weight outside its channel's window).
 *   e_top, esc_off  from w12_pack_plan on the same w.
 *   records         [n*k*3/2] out.
 *   esc             [esc_capacity] out; entries past esc_capacity are
 *                   dropped (the load-time check then fails), so pass
 *                   esc_capacity >= esc_off[last].
 */
w12_status w12_pack(const uint16_t *w, int64_t n, int64_t k,
                    const uint8_t *e_top, const uint32_t *esc_off,
                    uint8_t *records, uint32_t *esc, int64_t esc_capacity,
                    hipStream_t stream);

/* w12_decode -- restore the bf16 weights [n, k] (row-major) exactly
 * ([S1] 4.1: escapes restored exactly; the same in-register decode the GEMM
 * uses). */
w12_status w12_decode(const w12_matrix *w, uint16_t *out, hipStream_t stream);

/* w12_check -- load-time bit-for-bit check ([S1] 4.1, [S2]): decodes every
 * weight and ADDS the number that differ from ref [n, k] to *mismatches
 * (device u64; the caller zeroes it). Non-zero means refuse the weights
 * (W12_ECORRUPT). An escape block whose offsets are inconsistent
 * (esc_off[b+1] < esc_off[b], esc_off[b+1] > esc_off[last], or more than
 * the block's 1024 weights) counts all of its 1024 weights as mismatches and
 * reads no entry. Reads of esc stay below esc_off[last], which the caller
 * vouches for as the length of esc. w12_decode applies the same bounds; its
 * output for such a block is the records' codes without escapes. */
w12_status w12_check(const w12_matrix *w, const uint16_t *ref,
                     unsigned long long *mismatches, hipStream_t stream);

/* Workspace bytes w12_gemm needs for this shape (host output). The
 * workspace holds what the deterministic split of the k reduction needs
 * ([S1] 4.1: stream-K with a fixed summation order): one arrival counter per
 * output tile, the partial sums of the tiles split between workgroups, the
 * argmax keys of the head, and x rearranged into matrix-core fragments. The
 * size depends on the device's compute-unit count, which the library reads
 * once per device id and keeps for the life of the process (the only state
 * the library holds besides the no-allocation entry point's scratch). */
w12_status w12_gemm_workspace(int64_t n, int64_t k, int64_t m, size_t *bytes);

/*
 * w12_gemm -- verify GEMM ([S1] 4.1): y[i, c] = sum_k x[i, k] * W[c, k] for
 * the m verify rows, streaming every W12 record from HBM once, restoring it
 * in registers, fp32 accumulation. Rows m <= 4 use a VALU dot-product path,
 * m >= 5 bf16 MFMA (more than 192 rows run as several launches of at most
 * 192 rows, each streaming W again). The reduction over k is split across workgroups in a
 * fixed order (stream-K), so results are bitwise reproducible.
 *   x   [m, k] bf16 row-major, 1 <= m <= 512.
 *   y   [m, n] row-major, fp32 (W12_Y_F32) or bf16 (W12_Y_BF16, the
 *       round-to-nearest-even of the same fp32 result).
 *   ws  zero-filled workspace of >= w12_gemm_workspace bytes.
 */
w12_status w12_gemm(const w12_matrix *w, const uint16_t *x, int64_t m,
                    void *y, int ytype, void *ws, size_t ws_bytes,
                    hipStream_t stream);

/*
 * w12_gemm_noalloc -- w12_gemm for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same kernels and results, bit for bit, with the
 * workspace taken from a static device array of the library
 * (W12_NOALLOC_SCRATCH_BYTES per device, reserved when the library is
 * loaded and held until the process ends). The call allocates nothing.
 *   Arguments and layouts as w12_gemm, without ws / ws_bytes.
 *   Returns W12_ENOSPC, before launching anything, when w12_gemm_workspace
 *   for the shape exceeds W12_NOALLOC_SCRATCH_BYTES. At 256 compute units
 *   every m <= 512 fits for k <= 400000 (192-row launches need 51.6 MB;
 *   5 <= m <= 64 adds 128 * k bytes of x fragments).
 *   The first call on a device looks up the array's device address and
 *   enqueues one kernel on `stream` that zero-fills it; every completed call
 *   leaves its counters at zero again.
 *   All calls on one device share that device's array: calls that overlap in
 *   time on one device (other streams, other threads) race and give wrong
 *   results. Serialise them.
 */
#define W12_NOALLOC_SCRATCH_BYTES (64u << 20)
w12_status w12_gemm_noalloc(const w12_matrix *w, const uint16_t *x, int64_t m,
                            void *y, int ytype, hipStream_t stream);

/* Workspace bytes w12_head_argmax needs (host output). */
w12_status w12_head_argmax_workspace(int64_t n, int64_t k, int64_t m, size_t *bytes);

/*
 * w12_head_argmax -- LM head + greedy token ([S1] 1.1, 4.1): for each verify
 * row i, idx[i] = the lowest vocabulary id v attaining max_v logits[i, v],
 * logits = x W^T computed as in w12_gemm (never written to memory).
 *   idx     [m] int32 out; maxval [m] fp32 out (may be NULL).
 */
w12_status w12_head_argmax(const w12_matrix *head, const uint16_t *x, int64_t m,
                           int32_t *idx, float *maxval, void *ws, size_t ws_bytes,
                           hipStream_t stream);

/*
 * Certified INT8 LM head ([S1] 4.1, the LM-head paragraph: an INT8 copy of
 * the head, a per-row Cauchy-Schwarz error bound that proves which tokens
 * cannot be the argmax, exact rescoring of the survivors only; the argmax
 * does not change).
 *
 * The INT8 copy of an n x k head (device memory, caller-owned):
 *   q       [n*k] int8: per vocabulary row and block of 32 consecutive k,
 *           every weight the W12 pack keeps in its window is
 *           q = RNE(w / 2^s), s the smallest integer with all of the
 *           block's window weights |w| <= 127 * 2^s; weights W12 escapes
 *           are 0 (they come back exactly from the W12 head's escape
 *           list). Layout: 8 KB records, record (strip, r) at
 *           (strip*(k/256) + r) * 8192, weight (c, k') at the byte W12's
 *           8-bit view uses: t*1024 + (c + 32h)*16 + j.
 *   qexp    [n*k/32] u8 block codes s + 133 (0: no window weight in the
 *           block) at ((strip*(k/256) + r)*8 + t)*32 + c.
 *   cbound  [n] fp32 per-row constant ||e|| + 2 k 2^-24 ||w'||, rounded up
 *           (w' = the copy's weights with the escapes exact, e = w - w').
 */
typedef struct w12_cert8 {
  int64_t n, k;
  const int8_t *q;
  const uint8_t *qexp;
  const float *cbound;
} w12_cert8;

/* w12_cert8_pack -- build the INT8 copy from the bf16 head w [n, k] and the
 * window tops e_top [n] that w12_pack_plan gave for the same w (load time).
 * q, qexp, cbound as above (q 16-byte aligned, cbound 4-byte aligned). */
w12_status w12_cert8_pack(const uint16_t *w, int64_t n, int64_t k, const uint8_t *e_top,
                          int8_t *q, uint8_t *qexp, float *cbound, hipStream_t stream);

/* Workspace bytes w12_head_argmax_certified needs (host output). */
w12_status w12_head_argmax_certified_workspace(int64_t n, int64_t k, int64_t m, size_t *bytes);

/*
 * w12_head_argmax_certified -- the certified head argmax for 1 <= m <= 64
 * rows: an MFMA pass over the INT8 copy gives A = x.w' (fp32) per row and
 * vocabulary row, with bounds A +- B, B = ||x|| cbound + 1e-6 (rounded
 * outward); LB = the row's largest lower bound; every group of 4 vocabulary
 * rows whose upper bound reaches LB is rescored exactly from the W12 head
 * (its records and escapes, fp32 accumulation). idx[i] = the lowest id
 * attaining the largest rescored logit, which is the exact head argmax
 * (within the same floating-point allowance as w12_head_argmax).
 *   head    the W12 head of the same weights; cert its INT8 copy (same n, k).
 *   idx     [m] int32 out; maxval [m] fp32 out or NULL (the winning logit);
 *   rescored [m] int32 out or NULL: vocabulary rows rescored per row.
 *   ws      zero-filled workspace of >= w12_head_argmax_certified_workspace
 *           bytes; every completed call leaves its counters and keys at
 *           zero again, so one workspace serves certified calls of any
 *           shape (but not w12_gemm / w12_head_argmax calls: their
 *           counters sit at other offsets).
 * Errors: W12_EINVAL also when one workgroup's share of the head spans more
 * than 4096 vocabulary rows (n above about 900000 at 256 compute units).
 */
w12_status w12_head_argmax_certified(const w12_matrix *head, const w12_cert8 *cert, const uint16_t *x,
                                     int64_t m, int32_t *idx, float *maxval, int32_t *rescored,
                                     void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * w12_gemm_qpass, w12_head_argmax_qpass -- the Q pass ([S1] 4.3): the same
 * products read from the 8-bit view alone (the first 2/3 of every record),
 * every dropped low mantissa nibble taken at its midpoint 0b1000; escaped
 * weights are restored from the escape list as in the exact pass. Arguments,
 * layouts, workspace (w12_gemm_workspace) and errors as w12_gemm and
 * w12_head_argmax; results are bitwise reproducible but are not those of the
 * exact pass.
 */
w12_status w12_gemm_qpass(const w12_matrix *w, const uint16_t *x, int64_t m,
                          void *y, int ytype, void *ws, size_t ws_bytes,
                          hipStream_t stream);
w12_status w12_head_argmax_qpass(const w12_matrix *head, const uint16_t *x, int64_t m,
                                 int32_t *idx, float *maxval, void *ws, size_t ws_bytes,
                                 hipStream_t stream);

/*
 * w12_tree_build -- best-first draft trees under one shared row budget
 * ([S1] 4.2: every edge scored by the log-softmax of the child given its
 * parent, the nodes of highest path score kept; [S1] 4.4: one node budget
 * shared by all requests of a step, filled from the highest path score down,
 * each request's share a prefix-closed tree).
 *   num_req R in [1, 128]; positions D in [1, 16]; k K in [1, 16].
 *   lp    [R][D][K][K] fp32: lp[r][d][i][j] = edge score from candidate i of
 *         position d - 1 (the root for d = 0, row i = 0) to candidate j of
 *         position d; expected <= 0 (a log-softmax over j), finite.
 *   tok   [R][D][K] int32 candidate tokens; depth [R] int32 positions drafted
 *         per request (values outside [0, D] are clamped); root [R] int32
 *         committed token of each request.
 *   budget rows in all, roots included: R <= budget, budget - R <= 1023 and
 *         R * (budget - R) <= 8192.
 * Order: path score (the binary32 sum of edge scores, accumulated from the
 * root in path order) highest first, then depth, then request index, then the
 * path of child ranks (a parent's children ranked by edge score, equal scores
 * by candidate index).
 * Output (device memory, caller-owned, the layout tree_accept reads):
 *   node_off [R+1]; then per request its root row (parent -1, token root[r],
 *   depth 0, score 0) followed by its draft nodes in that order, parent local
 *   to the request; parent, token, node_depth, score hold node_off[R] rows
 *   (at most budget; fewer when the lattices run out of nodes). node_depth and
 *   score may be NULL.
 * Workspace: w12_tree_build_workspace bytes, 16-byte aligned, content ignored.
 * Errors: W12_EINVAL for shapes or pointers outside the above, W12_ENOSPC for
 * a small workspace, W12_EHIP for a launch error.
 */
w12_status w12_tree_build_workspace(int32_t num_req, int32_t budget, size_t *bytes);
w12_status w12_tree_build(int32_t num_req, int32_t positions, int32_t k, const float *lp,
                          const int32_t *tok, const int32_t *depth, const int32_t *root,
                          int32_t budget, void *ws, size_t ws_bytes, int32_t *node_off,
                          int32_t *parent, int32_t *token, int32_t *node_depth, float *score,
                          hipStream_t stream);

/*
 * tree_accept -- greedy tree verification ([S1] 1.1, 4.3; [S3]).
 * Trees are concatenated: tree t owns nodes [node_off[t], node_off[t+1]),
 * node_off[0] = 0, node_off[num_trees] = total_nodes; node i of a tree is
 * verify row node_off[t] + i, with tree-local parent[i] (-1 for the root,
 * else in [0, i)), draft token token[i] and the target's argmax[i] for that
 * row. A node is accepted when every edge on its root path satisfies
 * token[child] == argmax[parent]. Per tree:
 *   accept_len[t] = depth of the deepest accepted node (lowest index on
 *                   ties) = number of accepted drafts (tau = accept_len+1);
 *   path[node_off[t] + j] = tree-local node at depth j of that path for
 *                   j <= accept_len, -1 after it;
 *   bonus[t]      = argmax of the deepest accepted node's row.
 * A tree with no nodes, a root parent other than -1, a parent outside
 * [0, i), or offsets outside [0, total_nodes] gets accept_len = bonus = -1
 * and an all -1 path (device-detected; the call itself returns W12_OK).
 * total_nodes (the length of parent, token, argmax and path) is what the
 * kernel checks device-side offsets against, so that a corrupt node_off
 * never reads or writes past those arrays.
 */
w12_status tree_accept(int32_t num_trees, const int32_t *node_off,
                       int32_t total_nodes, const int32_t *parent,
                       const int32_t *token, const int32_t *argmax,
                       int32_t *accept_len, int32_t *path, int32_t *bonus,
                       hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* W12_H */
