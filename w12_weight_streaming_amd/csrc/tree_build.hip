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

// a precedes b: higher score, then smaller depth, then smaller rank path
__device__ __forceinline__ bool precedes(float sa, uint32_t da, uint64_t ra, float sb, uint32_t db, uint64_t rb) {
  const uint32_t ka = order_key(sa), kb = order_key(sb);
  if (ka != kb) return ka > kb;
  if (da != db) return da < db;
  return ra < rb;
}

__device__ __forceinline__ uint64_t shfl64(uint64_t v, int src) {
  const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)v, src, 64);
  const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(v >> 32), src, 64);
  return ((uint64_t)hi << 32) | lo;
}

struct Frontier {
  float score;       // path score of the candidate node
  float pscore;      // path score of its parent
  uint32_t meta;     // parent index (0..11) | rank (12..15) | depth (16..20) | parent slot (21..24)
  uint32_t pad;
  uint64_t ranks;    // rank path of the candidate node
};

__global__ __launch_bounds__(64) void tree_search_kernel(const float* __restrict__ lp, const int32_t* __restrict__ depth,
                                                         int D, int K, int cap, ListEntry* __restrict__ lists,
                                                         int32_t* __restrict__ counts) {
  __shared__ float s_lp[kMaxD * kMaxK * kMaxK];        // edge scores of (position, parent slot) by rank
  __shared__ uint8_t s_slot[kMaxD * kMaxK * kMaxK];    // candidate of each rank
  __shared__ Frontier s_f[1024 + 1];

  const int r = blockIdx.x, lane = threadIdx.x;
  const int Dr = min(max(depth[r], 0), D);
  const float* L = lp + (size_t)r * D * K * K;

  // rank the K children of every (position, parent slot): count the children
  // ahead of each one (higher score, or equal score and lower index)
  for (int row = lane; row < D * K; row += 64) {
    const float* v = L + (size_t)row * K;
    float x[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) x[j] = j < K ? v[j] : 0.f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j >= K) break;
      int rank = 0;
#pragma unroll
      for (int q = 0; q < kMaxK; ++q)
        rank += (q < K && (x[q] > x[j] || (x[q] == x[j] && q < j))) ? 1 : 0;
      s_lp[row * kMaxK + rank] = x[j];
      s_slot[row * kMaxK + rank] = (uint8_t)j;
    }
  }
  __syncthreads();

  int F = 0;
  if (lane == 0) {
    if (Dr >= 1 && cap >= 1) {
      s_f[0] = Frontier{0.f + s_lp[0], 0.f, (0u) | (0u << 12) | (1u << 16) | (0u << 21), 0u, 0ull};
    }
  }
  if (Dr >= 1 && cap >= 1) F = 1;
  __syncthreads();

  int n = 0;
  ListEntry* out = lists + (size_t)r * cap;
  while (n < cap && F > 0) {
    // best frontier entry: each lane scans its share, then a wave reduction
    float bs = 0.f;
    uint32_t bd = 0xFFFFFFFFu;
    uint64_t br = ~0ull;
    int bi = -1;
    for (int e = lane; e < F; e += 64) {
      const Frontier f = s_f[e];
      const uint32_t d = (f.meta >> 16) & 31u;
      if (bi < 0 || precedes(f.score, d, f.ranks, bs, bd, br)) {
        bs = f.score;
        bd = d;
        br = f.ranks;
        bi = e;
      }
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const float os = __shfl_xor(bs, m, 64);
      const uint32_t od = (uint32_t)__shfl_xor((int)bd, m, 64);
      const uint64_t orr = shfl64(br, lane ^ m);
      const int oi = __shfl_xor(bi, m, 64);
      const bool take = oi >= 0 && (bi < 0 || precedes(os, od, orr, bs, bd, br));
      if (take) {
        bs = os;
        bd = od;
        br = orr;
        bi = oi;
      }
    }
    bi = __builtin_amdgcn_readfirstlane(bi);
    ++n;
    if (lane == 0) {
      const Frontier f = s_f[bi];
      const uint32_t p = f.meta & 0xFFFu, rank = (f.meta >> 12) & 15u, d = (f.meta >> 16) & 31u;
      const uint32_t pslot = (f.meta >> 21) & 15u;
      const int row = (int)(d - 1) * K + (int)pslot;          // (position d - 1, parent slot)
      const uint32_t slot = s_slot[row * kMaxK + rank];
      out[n - 1] = ListEntry{f.score, p | (slot << 12) | (d << 16), f.ranks};
      // next sibling of the taken node replaces it, or the last entry does
      if ((int)rank + 1 < K) {
        const uint32_t rk = rank + 1;
        s_f[bi] = Frontier{f.pscore + s_lp[row * kMaxK + rk], f.pscore,
                           p | (rk << 12) | (d << 16) | (pslot << 21), 0u,
                           f.ranks + ((uint64_t)1 << (4 * (16 - d)))};
      } else {
        s_f[bi] = s_f[F - 1];
      }
      // best child of the taken node
      if ((int)d < Dr) {
        const int crow = (int)d * K + (int)slot;
        const int at = ((int)rank + 1 < K) ? F : F - 1;
        s_f[at] = Frontier{f.score + s_lp[crow * kMaxK], f.score,
                           (uint32_t)n | (0u << 12) | ((d + 1) << 16) | (slot << 21), 0u, f.ranks};
      }
    }
    // frontier size after lane 0's update (every lane holds the taken
    // entry's depth and rank path; its rank is the path's level-d digit)
    {
      const int d = (int)bd;
      const int rank = (int)((br >> (4 * (16 - d))) & 15u);
      if (rank + 1 >= K) --F;
      if (d < Dr) ++F;
    }
    __syncthreads();
  }
  if (lane == 0) counts[r] = n;
}

// 64-bit key of list entry (request r, position i): smaller = earlier.
__device__ __forceinline__ uint64_t global_key(float score, uint32_t depth, int r, int i) {
  return ((uint64_t)(~order_key(score)) << 22) | ((uint64_t)depth << 17) | ((uint64_t)r << 10) | (uint64_t)i;
}

constexpr int kSelThreads = 512;
constexpr int kSelMaxKeys = 8192;

__global__ __launch_bounds__(kSelThreads) void tree_select_kernel(
    const ListEntry* __restrict__ lists, const int32_t* __restrict__ counts, int R, int cap,
    const int32_t* __restrict__ tok, const int32_t* __restrict__ roots, int D, int K, int share,
    int32_t* __restrict__ node_off, int32_t* __restrict__ parent, int32_t* __restrict__ token,
    int32_t* __restrict__ node_depth, float* __restrict__ score) {
  __shared__ uint64_t s_key[kSelMaxKeys];
  __shared__ uint32_t s_hist[256];
  __shared__ uint64_t s_prefix, s_mask;
  __shared__ int s_k, s_total;
  __shared__ int s_take[128];
  __shared__ int s_off[129];

  const int tid = threadIdx.x;
  const int n = R * cap;  // cap = 0: roots only, no lists
  for (int e = tid; e < n; e += kSelThreads) {
    const int r = e / cap, i = e - r * cap;
    s_key[e] = ~0ull;
    if (i < counts[r]) {
      const ListEntry le = lists[e];
      s_key[e] = global_key(le.score, (le.meta >> 16) & 31u, r, i);
    }
  }
  if (tid < 128) s_take[tid] = 0;
  if (tid == 0) {
    int t = 0;
    for (int r = 0; r < R && cap > 0; ++r) t += min(counts[r], cap);
    s_total = t;
    s_prefix = 0;
    s_mask = 0;
    s_k = min(share, t);  // the k-th smallest key is the last one kept
  }
  __syncthreads();
  const int k = s_k;
  uint64_t thr = 0;
  if (k > 0 && k < s_total) {
    // radix select, 8 bits at a time from the top
    for (int pass = 7; pass >= 0; --pass) {
      for (int b = tid; b < 256; b += kSelThreads) s_hist[b] = 0;
      __syncthreads();
      const uint64_t prefix = s_prefix, mask = s_mask;
      for (int e = tid; e < n; e += kSelThreads) {
        const uint64_t key = s_key[e];
        if (key != ~0ull && (key & mask) == prefix) atomicAdd(&s_hist[(key >> (8 * pass)) & 255u], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        int kk = s_k, b = 0;
        while (b < 255 && (int)s_hist[b] < kk) {
          kk -= (int)s_hist[b];
          ++b;
        }
        s_k = kk;
        s_prefix = prefix | ((uint64_t)b << (8 * pass));
        s_mask = mask | ((uint64_t)255 << (8 * pass));
      }
      __syncthreads();
    }
    thr = s_prefix;
  } else if (k > 0) {
    thr = ~0ull - 1;  // every listed node is kept
  }
  // each request keeps the prefix of its list at or below the threshold
  if (k > 0) {
    for (int e = tid; e < n; e += kSelThreads) {
      const uint64_t key = s_key[e];
      if (key != ~0ull && key <= thr) {
        const int r = e / cap, i = e - r * cap;
        atomicMax(&s_take[r], i + 1);
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    int o = 0;
    for (int r = 0; r < R; ++r) {
      s_off[r] = o;
      o += 1 + s_take[r];
    }
    s_off[R] = o;
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
  for (int e = tid; e < n; e += kSelThreads) {
    const int r = e / cap, i = e - r * cap;
    if (i < s_take[r]) {
      const ListEntry le = lists[e];
      const int row = s_off[r] + 1 + i;
      const uint32_t d = (le.meta >> 16) & 31u, slot = (le.meta >> 12) & 15u;
      parent[row] = (int32_t)(le.meta & 0xFFFu);
      token[row] = tok[((size_t)r * D + (d - 1)) * K + slot];
      if (node_depth) node_depth[row] = (int32_t)d;
      if (score) score[row] = le.score;
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
