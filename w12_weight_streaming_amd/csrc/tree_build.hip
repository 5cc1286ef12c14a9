// Best-first draft trees and the shared node budget ("SpecPilot ..." summary,
// sections 4.2 and 4.4: edges scored by the log-softmax of the child given
// its parent, the N nodes of highest path score kept; one node budget shared
// by all requests of a step, filled from the highest path score down).
//
// Order of nodes: path score (binary32, accumulated from the root in path
// order) highest first, then depth, then the path of child ranks (a parent's
// children ranked by edge score, equal scores by candidate index); across
// requests: score, depth, request, rank path. Edge scores are <= 0, so every
// node follows its parent and any prefix of the order is a tree.
//
// Two launches:
//  * tree_search_kernel, one wave per request: lazy best-first expansion.
//    The frontier holds, for every node taken so far, its best child not yet
//    taken (its first child, or after that child was taken, the next
//    sibling); the best frontier entry is always the next node. The request's
//    first `cap` nodes in its own order go to the workspace.
//  * tree_select_kernel, one workgroup: every listed node gets a unique 64-bit
//    key (score, depth, request, position in its list); a radix select finds
//    the key of the (budget - R)-th node; each request keeps the prefix of its
//    list at or below it. The rows are written in the layout tree acceptance
//    reads.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w12_internal.h"

namespace w12 {
namespace {

constexpr int kMaxK = 16;
constexpr int kMaxD = 16;

struct ListEntry {
  float score;
  uint32_t meta;    // parent (bits 0..11, 0 = root) | slot (12..15) | depth (16..20)
  uint64_t ranks;   // rank path, level t (1..16) in bits 4 (16 - t) .. +3
};

__device__ __forceinline__ uint32_t order_key(float f) {
  // larger float -> larger key (total order on non-NaN values)
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// 64-bit maximum over the wave: every lane of a 16-lane DPP row gets the
// row maximum from exchanges with lane ^ 1, lane ^ 2, the mirrored half-row
// and the mirrored row; the four row maxima are then read from lanes 0, 16,
// 32 and 48.
template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = umax64(v, dpp64<0xB1>(v));   // quad_perm [1, 0, 3, 2]
  v = umax64(v, dpp64<0x4E>(v));   // quad_perm [2, 3, 0, 1]
  v = umax64(v, dpp64<0x141>(v));  // row_half_mirror
  v = umax64(v, dpp64<0x140>(v));  // row_mirror
  uint64_t m = 0;
#pragma unroll
  for (int row = 0; row < 4; ++row) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 16 * row);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 16 * row);
    m = umax64(m, ((uint64_t)hi << 32) | lo);
  }
  return m;
}

// 32-bit maximum over the wave (same exchanges as above).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp32<0xB1>(v));
  v = max(v, dpp32<0x4E>(v));
  v = max(v, dpp32<0x141>(v));
  v = max(v, dpp32<0x140>(v));
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32), d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(a, b), max(c, d));
}

// Primary key of a frontier entry, larger = earlier: score, then depth
// (smaller first), then the first 27 bits of the rank path (smaller first).
// Entries with equal primary keys are ordered by their whole rank paths.
__device__ __forceinline__ uint64_t primary_key(float score, uint32_t d, uint64_t ranks) {
  return ((uint64_t)order_key(score) << 32) | ((uint64_t)(31u - d) << 27) | ((~ranks >> 37) & 0x7FFFFFFull);
}

// Frontier entry fields (structure of arrays in LDS). meta: parent index
// (bits 0..11, 0 = root) | rank (12..15) | depth (16..20) | parent slot
// (21..24) | candidate slot (25..28).
constexpr int kMaxFrontier = 1024 + 1;

__global__ __launch_bounds__(64) void tree_search_kernel(const float* __restrict__ lp, const int32_t* __restrict__ depth,
                                                         int D, int K, int cap, ListEntry* __restrict__ lists,
                                                         int32_t* __restrict__ counts) {
  __shared__ float s_lp[kMaxD * kMaxK * kMaxK];        // edge scores of (position, parent slot) by rank
  __shared__ uint8_t s_slot[kMaxD * kMaxK * kMaxK];    // candidate of each rank
  __shared__ uint64_t f_pk[kMaxFrontier], f_rk[kMaxFrontier];
  __shared__ float f_sc[kMaxFrontier], f_ps[kMaxFrontier];
  __shared__ uint32_t f_meta[kMaxFrontier];

  const int r = blockIdx.x, lane = threadIdx.x;
  const int Dr = min(max(depth[r], 0), D);
  const float* L = lp + (size_t)r * D * K * K;

  // rank the K children of every (position, parent slot): count the children
  // ahead of each one (higher score, or equal score and lower index)
  // (a lane's rows are loaded before any is ranked, so their loads overlap)
  constexpr int kRowsPerLane = kMaxD * kMaxK / 64;
  float xr[kRowsPerLane][kMaxK];
#pragma unroll
  for (int t = 0; t < kRowsPerLane; ++t) {
    const int row = lane + 64 * t;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) xr[t][j] = (row < D * K && j < K) ? L[(size_t)row * K + j] : 0.f;
  }
#pragma unroll
  for (int t = 0; t < kRowsPerLane; ++t) {
    const int row = lane + 64 * t;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (row < D * K && j < K) {
        int rank = 0;
#pragma unroll
        for (int q = 0; q < kMaxK; ++q)
          rank += (q < K && (xr[t][q] > xr[t][j] || (xr[t][q] == xr[t][j] && q < j))) ? 1 : 0;
        s_lp[row * kMaxK + rank] = xr[t][j];
        s_slot[row * kMaxK + rank] = (uint8_t)j;
      }
    }
  }
  __syncthreads();

  // the root's best child (position 0 uses parent row 0)
  const bool any = Dr >= 1 && cap >= 1;
  if (lane == 0 && any) {
    const float sc = 0.f + s_lp[0];
    f_pk[0] = primary_key(sc, 1u, 0ull);
    f_rk[0] = 0ull;
    f_sc[0] = sc;
    f_ps[0] = 0.f;
    f_meta[0] = (1u << 16) | ((uint32_t)s_slot[0] << 25);
  }
  int F = any ? 1 : 0;
  __syncthreads();

  int n = 0;
  ListEntry* out = lists + (size_t)r * cap;
  while (n < cap && F > 0) {
    // best frontier entry: each lane scans its share (full order), the wave
    // takes the maximum primary key, and lanes tied on it compare rank paths
    uint64_t bpk = 0, brk = 0;  // primary keys of real entries are > 0
    int bi = -1;
    for (int e = lane; e < F; e += 64) {
      const uint64_t pk = f_pk[e], rk = f_rk[e];
      if (pk > bpk || (pk == bpk && rk < brk)) {
        bpk = pk;
        brk = rk;
        bi = e;
      }
    }
    // score part first (32 bits); lanes tied on it go on to the rest of the
    // primary key, lanes tied on the whole key to the rank paths
    const uint32_t hi = (uint32_t)(bpk >> 32);
    const uint32_t top_hi = wave_max_u32(hi);
    uint64_t tied = __ballot(hi == top_hi);
    if (__popcll(tied) > 1) {
      const uint32_t lo = hi == top_hi ? (uint32_t)bpk : 0u;
      const uint32_t top_lo = wave_max_u32(lo);
      tied = __ballot(hi == top_hi && lo == top_lo);
      if (__popcll(tied) > 1) {
        const uint64_t inv = (hi == top_hi && lo == top_lo) ? ~brk : 0ull;
        const uint64_t best = wave_max_u64(inv);
        tied = __ballot(hi == top_hi && lo == top_lo && inv == best);
      }
    }
    const int wl = __ffsll((long long)tied) - 1;
    bi = __builtin_amdgcn_readlane(bi, wl);
    ++n;
    const float fsc = f_sc[bi], fps = f_ps[bi];
    const uint32_t meta = f_meta[bi];
    const uint64_t frk = f_rk[bi];
    const uint32_t p = meta & 0xFFFu, rank = (meta >> 12) & 15u, d = (meta >> 16) & 31u;
    const uint32_t pslot = (meta >> 21) & 15u, slot = (meta >> 25) & 15u;
    const bool sib = (int)rank + 1 < K;
    const bool child = (int)d < Dr;
    if (lane == 0) {
      out[n - 1] = ListEntry{fsc, p | (slot << 12) | (d << 16), frk};
      const int row = (int)(d - 1) * K + (int)pslot;  // (position d - 1, parent slot)
      // the taken node's next sibling replaces it, or the last entry does
      if (sib) {
        const uint32_t rk = rank + 1;
        const float sc = fps + s_lp[row * kMaxK + rk];
        const uint64_t rr = frk + ((uint64_t)1 << (4 * (16 - d)));
        f_pk[bi] = primary_key(sc, d, rr);
        f_rk[bi] = rr;
        f_sc[bi] = sc;
        f_meta[bi] = p | (rk << 12) | (d << 16) | (pslot << 21) | ((uint32_t)s_slot[row * kMaxK + rk] << 25);
      } else if (bi != F - 1) {
        f_pk[bi] = f_pk[F - 1];
        f_rk[bi] = f_rk[F - 1];
        f_sc[bi] = f_sc[F - 1];
        f_ps[bi] = f_ps[F - 1];
        f_meta[bi] = f_meta[F - 1];
      }
      // the taken node's best child
      if (child) {
        const int crow = (int)d * K + (int)slot;
        const int at = sib ? F : F - 1;
        const float sc = fsc + s_lp[crow * kMaxK];
        f_pk[at] = primary_key(sc, d + 1, frk);
        f_rk[at] = frk;
        f_sc[at] = sc;
        f_ps[at] = fsc;
        f_meta[at] = (uint32_t)n | ((d + 1) << 16) | (slot << 21) | ((uint32_t)s_slot[crow * kMaxK] << 25);
      }
    }
    if (!sib) --F;
    if (child) ++F;
    // one wave: its LDS accesses complete in issue order, so lane 0's writes
    // are seen by the next scan; only the compiler must keep the order
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  if (lane == 0) counts[r] = n;
}

// 64-bit key of list entry (request r, position i): smaller = earlier.
__device__ __forceinline__ uint64_t global_key(float score, uint32_t depth, int r, int i) {
  return ((uint64_t)(~order_key(score)) << 22) | ((uint64_t)depth << 17) | ((uint64_t)r << 10) | (uint64_t)i;
}

constexpr int kSelThreads = 512;
constexpr int kSelMaxKeys = 8192;
constexpr int kSelPerThread = kSelMaxKeys / kSelThreads;  // list entries per thread

__global__ __launch_bounds__(kSelThreads) void tree_select_kernel(
    const ListEntry* __restrict__ lists, const int32_t* __restrict__ counts, int R, int cap,
    const int32_t* __restrict__ tok, const int32_t* __restrict__ roots, int D, int K, int share,
    int32_t* __restrict__ node_off, int32_t* __restrict__ parent, int32_t* __restrict__ token,
    int32_t* __restrict__ node_depth, float* __restrict__ score) {
  __shared__ uint64_t s_key[kSelMaxKeys];
  __shared__ uint32_t s_hist[256];
  __shared__ uint32_t s_sel;
  __shared__ int s_kk;
  __shared__ int s_total;
  __shared__ int s_cnt[128];
  __shared__ int s_take[128];
  __shared__ int s_off[129];

  const int tid = threadIdx.x;
  const int n = R * cap;  // cap = 0: roots only, no lists
  int np = 1;             // keys held: a power of two >= n
  while (np < n) np <<= 1;
  if (tid < 128) s_take[tid] = 0;
  if (tid == 0) s_total = 0;
  if (tid < R) s_cnt[tid] = cap > 0 ? min(counts[tid], cap) : 0;
  __syncthreads();
  if (tid < R && cap > 0) atomicAdd(&s_total, s_cnt[tid]);
  // this thread's list entries e = tid + j * kSelThreads, all loads issued
  // before any is used (entries past a list's count are read but not used)
  ListEntry le[kSelPerThread];
#pragma unroll
  for (int j = 0; j < kSelPerThread; ++j) {
    const int e = tid + j * kSelThreads;
    le[j] = e < n ? lists[e] : ListEntry{0.f, 0u, 0ull};
  }
#pragma unroll
  for (int j = 0; j < kSelPerThread; ++j) {
    const int e = tid + j * kSelThreads;
    if (e < np) {
      uint64_t key = ~0ull;  // past a list's end, and padding: sorts last
      if (e < n) {
        const int r = e / cap, i = e - r * cap;
        if (i < s_cnt[r]) key = global_key(le[j].score, (le[j].meta >> 16) & 31u, r, i);
      }
      s_key[e] = key;
    }
  }
  __syncthreads();
  const int k = min(share, s_total);  // nodes kept
  // The k smallest keys are the kept nodes (keys are unique, and every list
  // is ascending in them: a request's order is score, depth, position). A
  // radix select finds the k-th smallest, 8 bits a pass from the top; each
  // request then keeps the entries of its list at or below it.
  uint64_t thr = ~0ull - 1;  // with every listed node kept
  if (k > 0 && k < s_total) {
    uint64_t prefix = 0, mask = 0;
    int kk = k;  // rank still to find among the keys matching the prefix
    for (int pass = 7; pass >= 0; --pass) {
      if (tid < 256) s_hist[tid] = 0;
      __syncthreads();
      for (int e0 = 0; e0 < np; e0 += kSelThreads) {
        const int e = e0 + tid;
        const uint64_t key = e < np ? s_key[e] : ~0ull;
        const bool in = key != ~0ull && (key & mask) == prefix;
        const uint32_t bin = (uint32_t)(key >> (8 * pass)) & 255u;
        // a wave whose matching keys share one bin adds them with one atomic
        const uint64_t inm = __ballot(in);
        const int first = inm ? __ffsll((long long)inm) - 1 : 0;
        const uint32_t lead = (uint32_t)__builtin_amdgcn_readlane((int)bin, first);
        const uint64_t same = __ballot(in && bin == lead);
        if (inm != 0 && same == inm) {
          if ((tid & 63) == first) atomicAdd(&s_hist[lead], (uint32_t)__popcll(inm));
        } else if (in) {
          atomicAdd(&s_hist[bin], 1u);
        }
      }
      __syncthreads();
      // the bin holding rank kk: one wave scans the 256 counts, 4 per lane
      if (tid < 64) {
        uint32_t c[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) c[q] = s_hist[4 * tid + q];
        const uint32_t sum = c[0] + c[1] + c[2] + c[3];
        uint32_t incl = sum;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const uint32_t o = (uint32_t)__shfl_up((int)incl, d, 64);
          if (tid >= d) incl += o;
        }
        const uint32_t excl = incl - sum;
        // lane whose range [excl, incl) holds rank kk - 1
        const bool here = excl < (uint32_t)kk && (uint32_t)kk <= incl;
        if (here) {
          uint32_t before = excl;
          int q = 0;
          while (q < 3 && before + c[q] < (uint32_t)kk) before += c[q++];
          s_sel = (uint32_t)(4 * tid + q);
          s_kk = kk - (int)before;
        }
      }
      __syncthreads();
      const uint32_t bsel = s_sel;
      kk = s_kk;
      prefix |= (uint64_t)bsel << (8 * pass);
      mask |= (uint64_t)255 << (8 * pass);
      __syncthreads();  // s_sel and s_hist are reused by the next pass
    }
    thr = prefix;
  }
  if (k > 0) {
    for (int e = tid; e < np; e += kSelThreads) {
      const uint64_t key = s_key[e];
      if (key != ~0ull && key <= thr) atomicMax(&s_take[(int)(key >> 10) & 127], (int)(key & 1023u) + 1);
    }
  }
  __syncthreads();
  // row offsets: exclusive prefix sum of 1 + take over the requests (R <= 128),
  // two requests per lane of the first wave
  if (tid < 64) {
    const int r0 = 2 * tid, r1 = 2 * tid + 1;
    const int c0 = r0 < R ? 1 + s_take[r0] : 0, c1 = r1 < R ? 1 + s_take[r1] : 0;
    int incl = c0 + c1;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d, 64);
      if (tid >= d) incl += o;
    }
    const int excl = incl - c0 - c1;
    if (r0 < R) s_off[r0] = excl;
    if (r1 < R) s_off[r1] = excl + c0;
    if (tid == 63) s_off[R] = incl;  // lane 63 holds the total
  }
  __syncthreads();
  for (int r = tid; r <= R; r += kSelThreads) node_off[r] = s_off[r];
  for (int r = tid; r < R; r += kSelThreads) {
    const int row = s_off[r];
    parent[row] = -1;
    token[row] = roots[r];
    if (node_depth) node_depth[row] = 0;
    if (score) score[row] = 0.f;
  }
  int32_t tk[kSelPerThread];
#pragma unroll
  for (int j = 0; j < kSelPerThread; ++j) {  // token loads first, all in flight together
    const int e = tid + j * kSelThreads;
    tk[j] = 0;
    if (e < n) {
      const int r = e / cap, i = e - r * cap;
      if (i < s_take[r]) {
        const uint32_t d = (le[j].meta >> 16) & 31u, slot = (le[j].meta >> 12) & 15u;
        tk[j] = tok[((size_t)r * D + (d - 1)) * K + slot];
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kSelPerThread; ++j) {
    const int e = tid + j * kSelThreads;
    if (e < n) {
      const int r = e / cap, i = e - r * cap;
      if (i < s_take[r]) {
        const int row = s_off[r] + 1 + i;
        parent[row] = (int32_t)(le[j].meta & 0xFFFu);
        token[row] = tk[j];
        if (node_depth) node_depth[row] = (int32_t)((le[j].meta >> 16) & 31u);
        if (score) score[row] = le[j].score;
      }
    }
  }
}

}  // namespace

size_t tree_build_ws_bytes(int32_t num_req, int32_t budget) {
  const size_t cap = (size_t)(budget - num_req);
  return (size_t)num_req * cap * sizeof(ListEntry) + (size_t)num_req * 4 + 256;
}

hipError_t launch_tree_build(int32_t R, int32_t D, int32_t K, const float* lp, const int32_t* tok,
                             const int32_t* depth, const int32_t* roots, int32_t budget, void* ws,
                             int32_t* node_off, int32_t* parent, int32_t* token, int32_t* node_depth,
                             float* score, hipStream_t s) {
  const int cap = budget - R;
  ListEntry* lists = static_cast<ListEntry*>(ws);
  int32_t* counts = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + (size_t)R * cap * sizeof(ListEntry));
  if (cap > 0) {
    hipLaunchKernelGGL(tree_search_kernel, dim3(R), dim3(64), 0, s, lp, depth, D, K, cap, lists, counts);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(tree_select_kernel, dim3(1), dim3(kSelThreads), 0, s, lists, counts, R, cap, tok, roots, D, K,
                     cap, node_off, parent, token, node_depth, score);
  return hipGetLastError();
}

}  // namespace w12
