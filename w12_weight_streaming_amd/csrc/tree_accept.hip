// Greedy tree acceptance (gfx950).
//
// "SpecPilot ..." summary, sections 1.1 and 4.3: greedy verification accepts
// the longest draft path whose every token equals the target's argmax at its
// parent, then appends that argmax as a bonus token (tau in [1, m+1] for a
// chain of m drafts); with a tree, the longest accepted root path wins.
// poot-llm docs, "What a round guarantees": greedy rows keep the drafts equal
// to the argmax, then the target's own next token.
//
// One wavefront per tree. Each lane walks its nodes' root paths (parent <
// child, so every walk ends), the wave reduces (depth, -index) to the
// deepest accepted node with the lowest index, and one lane writes the path.
#include "w12_device.h"
#include "w12_internal.h"

namespace w12 {
namespace {

__device__ __forceinline__ unsigned long long wave_max(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, o, 64);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, 64);
    const unsigned long long w = ((unsigned long long)hi << 32) | lo;
    v = w > v ? w : v;
  }
  return v;
}

__global__ __launch_bounds__(64) void tree_accept_kernel(
    int32_t num_trees, const int32_t* __restrict__ node_off, int32_t total,
    const int32_t* __restrict__ parent, const int32_t* __restrict__ token,
    const int32_t* __restrict__ argmax, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ path, int32_t* __restrict__ bonus) {
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  if (t >= num_trees) return;
  const int32_t b0 = node_off[t], b1 = node_off[t + 1];
  const bool range_ok = b0 >= 0 && b1 <= total && b0 <= b1;
  const int32_t base = b0;
  const int32_t n = range_ok ? b1 - b0 : 0;

  // validity: root parent -1, every other parent in [0, i)
  int bad = (!range_ok || n < 1) ? 1 : 0;
  for (int32_t i = lane; i < n; i += 64) {
    const int32_t p = parent[base + i];
    if (i == 0 ? (p != -1) : (p < 0 || p >= i)) bad = 1;
  }
  bad = __any(bad);
  if (bad) {
    if (range_ok)
      for (int32_t i = lane; i < n; i += 64) path[base + i] = -1;
    if (lane == 0) {
      accept_len[t] = -1;
      bonus[t] = -1;
    }
    return;
  }

  // deepest accepted node, lowest index on ties: max of (depth, ~index)
  unsigned long long best = 0;
  for (int32_t i = lane; i < n; i += 64) {
    bool ok = true;
    uint32_t depth = 0;
    int32_t j = i;
    while (j != 0) {
      const int32_t p = parent[base + j];
      if (token[base + j] != argmax[base + p]) ok = false;
      ++depth;
      j = p;
    }
    if (ok) {
      const unsigned long long key =
          ((unsigned long long)depth << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)i);
      best = key > best ? key : best;
    }
  }
  best = wave_max(best);  // the root is always accepted, so best != 0
  const int32_t node = (int32_t)(0xFFFFFFFFu - (uint32_t)best);
  const int32_t depth = (int32_t)(best >> 32);

  for (int32_t i = depth + 1 + lane; i < n; i += 64) path[base + i] = -1;
  if (lane == 0) {
    int32_t j = node;
    for (int32_t d = depth; d >= 0; --d) {
      path[base + d] = j;
      j = parent[base + j];
    }
    accept_len[t] = depth;
    bonus[t] = argmax[base + node];
  }
}

}  // namespace

hipError_t launch_tree_accept(int32_t num_trees, const int32_t* node_off, int32_t total,
                              const int32_t* parent, const int32_t* token, const int32_t* argmax,
                              int32_t* accept_len, int32_t* path, int32_t* bonus, hipStream_t s) {
  if (num_trees == 0) return hipSuccess;
  hipLaunchKernelGGL(tree_accept_kernel, dim3(num_trees), dim3(64), 0, s, num_trees, node_off,
                     total, parent, token, argmax, accept_len, path, bonus);
  return hipGetLastError();
}

}  // namespace w12
