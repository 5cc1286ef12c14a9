// W12 verify GEMM and fused LM-head argmax (gfx950).
//
// What is computed ("SpecPilot ..." summary, section 4.1): the verify pass
// multiplies every target linear layer, restored from W12 records in
// registers, against the handful of draft-tree rows in one weight read; the
// k reduction is split across workgroups in a fixed order, so the GEMM is
// deterministic. The LM-head variant keeps the logits in registers and emits
// only the greedy token (section 1.1: the target's argmax).
//
// gfx950 design for m <= 64 (HBM-bound; the layout for more rows is described
// at the large-m kernel below):
//  * Tile = 64 output channels (a pair of 32-channel strips). Unit = one
//    256-k record of a tile (2 x 12 KB). Units run tile-major; workgroup g
//    owns the contiguous slice [g*U/G, (g+1)*U/G) (stream-K). A tile split
//    between slices is finished by the last contributor to arrive, which sums
//    the slices' partials in slice order.
//  * 8 waves per workgroup; wave w restores subtile w (32 k) of both strips of
//    every unit: per lane one 16-byte load of the 8-bit view and one 8-byte
//    load of the low nibbles per strip, nontemporal, through raw buffer
//    resources (loads past a slice's end use an empty resource: no traffic).
//  * Loads run D units ahead of the arithmetic and are always issued
//    unconditionally; the loop has no barrier that waits on vector memory,
//    so the next units' loads stay in flight across every barrier.
//  * 5 <= m <= 64: bf16 MFMA 32x32x16, weights = A, x = B (one or two 32-row
//    x tiles, rows past m zero). The B fragments come from a copy of x
//    rearranged once per call so that every fragment load is one contiguous
//    1 KB per wave (xfrag_kernel); where slices are only a few units long,
//    the kernel reads them from row-major x instead and the call has no
//    pre-pass.
//  * m <= 4: lanes own channels, fdot2 against x rows (up to 2 rows read
//    from memory by every lane of a half-wave; 3-4 rows ride in the load
//    ring and are broadcast through a per-wave LDS buffer).
//  * Escapes (~1% of weights here): restored pairs go through a per-wave LDS
//    buffer, the lanes holding the block's escape entries overwrite their
//    slots, and the pairs are read back -- all synchronised within the wave.
//  * Escape-block offsets and window tops are read with vector loads in the
//    same in-order streams as the records (every lane reads the block's two
//    offsets; each lane reads the dword holding its channel's window top), so
//    one wait count covers a unit's loads.
//  * Argmax keys: one copy per XCD and one cache line per row; the last
//    workgroup of the grid merges the copies.
#include <atomic>
#include <type_traits>
#include <utility>

#include "w12_device.h"
#include "w12_internal.h"

namespace w12 {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kNW = 8;                          // waves per workgroup (= subtiles per record)
constexpr int kNT = kNW * 64;
constexpr int kRedStride = 68;                  // floats per 64-channel row (+4 pad)
constexpr int kSlotFloats = 32 * kRedStride;    // one 32-row x 64-channel reduction slot
constexpr int kLdsFloats = 4 * kSlotFloats;     // 34816 B >= 8 waves x 4 KB of patch buffers
constexpr int kRawBufferWord3 = 0x00020000;     // gfx9-family raw buffer descriptor word 3
constexpr int kNonTemporal = 2;                 // load cache policy: streaming

#ifndef W12_PIPE_DEPTH
#define W12_PIPE_DEPTH 2
#endif
constexpr int kDepth = W12_PIPE_DEPTH;          // units of weight loads in flight per wave

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1 with constant i, so
// arrays of load slots indexed by i stay in registers.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Buffer resource from wave-uniform base and size. The fields pass through
// readfirstlane so the descriptor is built in scalar registers even where the
// compiler would otherwise materialise a uniform select in vector registers
// (a descriptor in vector registers turns every load into a waterfall loop).
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  void* ub = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                           kRawBufferWord3);
}
// Wave-uniform metadata (escape-block offsets, window tops) is read through
// the scalar data cache: the loads leave the vector memory path to the weight
// stream. The buffers are read-only for the whole launch.
typedef __attribute__((address_space(4))) const uint32_t* cu32p;
__device__ __forceinline__ cu32p scalar_view(const void* p) { return (cu32p)p; }

// (E_n - 15) << 7 in both 16-bit halves for the lane's channel of strip sq:
// the strip's 32 window tops come in as 8 scalar dwords; the lane takes dword
// (lane & 31) / 4 and its byte lane & 3.
__device__ __forceinline__ uint32_t strip_bias2(const uint8_t* e_top, int sq, bool ok, int lane) {
  const cu32p c = scalar_view(e_top) + (ok ? sq : 0) * (kStrip / 4);
  uint32_t d[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) d[i] = c[i];
  const int j = (lane >> 2) & 7;
  const uint32_t d01 = (j & 1) ? d[1] : d[0], d23 = (j & 1) ? d[3] : d[2];
  const uint32_t d45 = (j & 1) ? d[5] : d[4], d67 = (j & 1) ? d[7] : d[6];
  const uint32_t d03 = (j & 2) ? d23 : d01, d47 = (j & 2) ? d67 : d45;
  const uint32_t dw = (j & 4) ? d47 : d03;
  const uint32_t e = __builtin_amdgcn_ubfe(dw, 8u * (uint32_t)(lane & 3), 8);
  return ok ? e * 0x00800080u - 0x07800780u : 0u;
}

template <int AUX = 0>
__device__ __forceinline__ u32x4 bload4(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, AUX));
}
template <int AUX = 0>
__device__ __forceinline__ u32x2 bload2(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, AUX));
}
__device__ __forceinline__ uint32_t bload1(rsrc_t r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}

// Workgroup barrier that orders LDS only: it waits for this wave's LDS
// operations, never for outstanding global loads.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
// Ordering point between LDS writes of one lane and reads of another lane of
// the same wave: a wave's LDS operations execute in issue order, so only the
// compiler has to be kept from reordering them.
__device__ __forceinline__ void wave_lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

__device__ __forceinline__ float4 f4add(float4 a, float4 b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

// Dispatch sends workgroup b to XCD b % 8. Renumber so that each XCD runs a
// contiguous run of slices: neighbours that share a split tile then share an
// L2 as well.
__device__ __forceinline__ int logical_wg(int b, int G) {
  const int x = b & 7, q = G >> 3, rem = G & 7;
  return x * q + min(x, rem) + (b >> 3);
}
__device__ __forceinline__ int chunk_begin(int g, int U, int G) {
  return (int)((int64_t)g * U / G);
}
__device__ __forceinline__ int owner_of(int u, int U, int G) {
  return (int)(((int64_t)(u + 1) * G + U - 1) / U) - 1;
}

__device__ __forceinline__ unsigned long long row16_max(unsigned long long v);

// Argmax key of row m over channels n .. n+3 -- (value key, ~index), so the
// maximum is the largest logit, lowest id on ties -- maximised over the 16
// threads of the DPP row (which hold the row's 64 channels of a tile); 0 when
// no channel is valid.
__device__ __forceinline__ unsigned long long row_key4(const GemmParams& a, int m, int n, float4 v) {
  unsigned long long best = 0;
  if (m < a.M && n < a.N) {
    const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const unsigned long long key = ((unsigned long long)float_key(vv[i]) << 32) |
                                     (uint32_t)(0xFFFFFFFFu - (uint32_t)(n + i));
      best = key > best ? key : best;
    }
  }
  return row16_max(best);
}
__device__ __forceinline__ unsigned long long kmax(unsigned long long x, unsigned long long y) { return x > y ? x : y; }
// Argmax keys: one copy per XCD (workgroup b runs on XCD b % 8) and one
// 128-byte line per row, so the grid's per-row atomics spread over 8 x M
// lines instead of queueing on the two lines 32 packed keys would share. The
// last workgroup takes the maximum of the 8 copies (max is order-free, so the
// result does not depend on which XCD ran what).
// (kKeyCopies, kKeyRows, kKeyStride: w12_internal.h, shared with the
// certified head's rescoring)
static_assert(kKeyRows >= kRowsPerLaunch, "a key row for every row of a launch");
__device__ __forceinline__ unsigned long long* key_slot(const GemmParams& a, int m) {
  return a.keys + ((int)(blockIdx.x % kKeyCopies) * kKeyRows + m) * kKeyStride;
}
__device__ __forceinline__ unsigned long long shfl_xor64(unsigned long long v, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m, 64);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m, 64);
  return ((unsigned long long)hi << 32) | lo;
}
// Final value of 4 consecutive channels (n .. n+3) of row m. For the argmax
// epilogue, 16 consecutive threads of a wave hold one row's 64 channels.
//
// Whole tiles of the argmax epilogue do not come here: their keys are kept per
// thread across the slice and published once at its end (publish_keys). On
// this family a wave's stores and atomics count in the same in-order counter
// as its loads, so a device-scope atomic at every tile end would hold up the
// weight loads issued after it until the atomic completed.
template <int EPI>
__device__ __forceinline__ void emit4(const GemmParams& a, int tid, int m, int n, float4 v) {
  const bool valid = m < a.M && n < a.N;
  if constexpr (EPI == kEpiY) {
    if (!valid) return;
    if (a.ytype == 0) {
      *reinterpret_cast<float4*>(static_cast<float*>(a.y) + (int64_t)m * a.N + n) = v;
    } else {
      const uint32_t lo = f32_to_bf16_rne(v.x) | ((uint32_t)f32_to_bf16_rne(v.y) << 16);
      const uint32_t hi = f32_to_bf16_rne(v.z) | ((uint32_t)f32_to_bf16_rne(v.w) << 16);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.y) + (int64_t)m * a.N + n) =
          make_uint2(lo, hi);
    }
  } else {
    const unsigned long long best = row_key4(a, m, n, v);
    if ((tid & 15) == 0 && best) atomicMax(key_slot(a, m), best);
  }
}

// Cross-workgroup hand-off without a device-scope fence. A device-scope
// fence on gfx950 writes back and invalidates the whole L2 of the XCD, which
// every workgroup sharing that L2 then pays for (the x fragments and escape
// metadata are L2-resident). Instead, partial sums are stored write-through
// at device scope (sc1), each thread waits until its own stores are
// acknowledged, the workgroup synchronises, and only then one thread bumps
// the device-coherent arrival counter. The last contributor reads the partials
// with device-scope loads that bypass its L2, so it cannot see stale lines.
constexpr int kDeviceScope = 16;  // sc1 cache-policy bit: coherent across XCDs

// Partial sums: slot (2g or 2g+1: the workgroup's first or last tile) x row
// x TC channels of the tile.
template <int TC>
__device__ __forceinline__ uint32_t partial_off(const GemmParams& a, int slot, int m, int c4) {
  return (uint32_t)(((slot * a.M + m) * TC + c4) * 4);
}
template <int TC>
__device__ __forceinline__ rsrc_t partial_rsrc(const GemmParams& a) {
  return make_rsrc(a.part, (uint32_t)(2 * a.G) * (uint32_t)a.M * (uint32_t)(TC * 4));
}
template <int TC>
__device__ __forceinline__ void store_partial(const GemmParams& a, int slot, int m, int c4, float4 v) {
  const u32x4 d = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)};
  __builtin_amdgcn_raw_buffer_store_b128(d, partial_rsrc<TC>(a), partial_off<TC>(a, slot, m, c4), 0, kDeviceScope);
}
template <int TC>
__device__ __forceinline__ float4 load_partial(const GemmParams& a, int slot, int m, int c4) {
  const u32x4 d = bload4<kDeviceScope>(partial_rsrc<TC>(a), partial_off<TC>(a, slot, m, c4), 0);
  return make_float4(__uint_as_float(d.x), __uint_as_float(d.y), __uint_as_float(d.z), __uint_as_float(d.w));
}
// Every thread's earlier global writes and atomics are acknowledged, then
// the workgroup synchronises.
__device__ __forceinline__ void writes_done_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
}

// A tile is split when the slice [u0, u1) does not hold all of its units.
__device__ __forceinline__ bool tile_is_split(int p, int u0, int u1, int RK) {
  return !(p * RK >= u0 && (p + 1) * RK <= u1);
}
// Partial-sum slot of workgroup g for tile p: its first tile or its last.
__device__ __forceinline__ int partial_slot(int g, int p, int U, int G, int RK) {
  return (p == chunk_begin(g, U, G) / RK) ? 2 * g : 2 * g + 1;
}

// Certified head (INT8 pass): B = ||x|| c + 1e-6 for a row norm xn and a
// channel's bound constant c, rounded up; then the group of 4 channels
// n .. n+3 of row m gets its upper bound max (A + B) stored (rounded up) and
// yields its lower bound max (A - B) (rounded down) as a key (value key, all
// ones), maximised over the 16 threads of the DPP row; 0 when not valid.
__device__ __forceinline__ float cert_bound(float xn, float c) {
  const float p = xn * c;
  return fmaf(p, 0x1p-22f, p) + 1.0001e-6f;
}
__device__ __forceinline__ unsigned long long cert_emit4(const GemmParams& a, int m, int n, float4 v, float4 cb,
                                                         float xn) {
  unsigned long long best = 0;
  if (m < a.M && n < a.N) {
    const float vv[4] = {v.x, v.y, v.z, v.w}, cc[4] = {cb.x, cb.y, cb.z, cb.w};
    float up = -__builtin_huge_valf(), lo = -__builtin_huge_valf();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float B = cert_bound(xn, cc[i]), slack = (fabsf(vv[i]) + B) * 0x1p-22f;
      up = fmaxf(up, (vv[i] + B) + slack);
      lo = fmaxf(lo, (vv[i] - B) - slack);
    }
    a.u4[(size_t)(n >> 2) * kCertMaxRows + m] = up;
    best = ((unsigned long long)float_key(lo) << 32) | 0xFFFFFFFFull;
  }
  return row16_max(best);
}

// Last contributor of a split tile sums the partials in slice order. Called
// after writes_done_barrier(), once per split tile of the slice. NT threads,
// TC channels per tile, CH float4 per thread per round; 16 consecutive
// threads share a row (TC >= 64). The partials of 4 contributors x CH float4
// are requested before any is added (missing contributors read through an
// empty resource as zero), so a round costs one memory latency, not one per
// load.
template <int EPI, int NT, int TC, int CH>
__device__ __forceinline__ void finish_split_tile(const GemmParams& a, int p, int tid, int* s_last) {
  constexpr int Q = TC / 4;  // float4 per tile row
  constexpr int kC = 4;      // contributors per round
  const int gf = owner_of(p * a.RK, a.U, a.G);
  const int gl = owner_of((p + 1) * a.RK - 1, a.U, a.G);
  if (tid == 0) {
    const uint32_t old = atomicAdd(&a.tile_cnt[p], 1u);
    *s_last = (old == (uint32_t)(gl - gf)) ? 1 : 0;
  }
  __syncthreads();
  if (*s_last) {
    const rsrc_t rp = partial_rsrc<TC>(a), r0 = make_rsrc(a.part, 0u);
    const int total = ((a.M + 31) & ~31) * Q;
    for (int e0 = 0; e0 < total; e0 += NT * CH) {
      uint32_t off[CH];
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        const int e = e0 + j * NT + tid;
        off[j] = partial_off<TC>(a, 0, min(e / Q, a.M - 1), (e % Q) * 4);
      }
      float4 v[CH];
#pragma unroll
      for (int j = 0; j < CH; ++j) v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int gg = gf; gg <= gl; gg += kC) {
        u32x4 d[kC][CH];
#pragma unroll
        for (int c = 0; c < kC; ++c) {
          const bool ok = gg + c <= gl;
          const uint32_t so = ok ? partial_off<TC>(a, partial_slot(gg + c, p, a.U, a.G, a.RK), 0, 0) : 0u;
          const rsrc_t r = ok ? rp : r0;
#pragma unroll
          for (int j = 0; j < CH; ++j) d[c][j] = bload4<kDeviceScope>(r, off[j], so);
        }
#pragma unroll
        for (int c = 0; c < kC; ++c)
#pragma unroll
          for (int j = 0; j < CH; ++j)
            v[j] = f4add(v[j], make_float4(__uint_as_float(d[c][j].x), __uint_as_float(d[c][j].y),
                                           __uint_as_float(d[c][j].z), __uint_as_float(d[c][j].w)));
      }
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        const int e = e0 + j * NT + tid;
        if constexpr (EPI == kEpiArgmax || EPI == kEpiCert) {
          // Q consecutive threads hold one row: maximise over all of them
          // (Q <= 64, one wave) before the one atomic of the row
          unsigned long long key;
          if constexpr (EPI == kEpiCert) {
            const int m = e / Q, n = p * TC + (e % Q) * 4;
            const float4 cb = n < a.N ? *reinterpret_cast<const float4*>(a.cbound + n) : make_float4(0.f, 0.f, 0.f, 0.f);
            key = cert_emit4(a, m, n, v[j], cb, m < a.M ? a.xnorm[m] : 0.f);
          } else {
            key = row_key4(a, e / Q, p * TC + (e % Q) * 4, v[j]);
          }
          if constexpr (Q >= 32) key = kmax(key, shfl_xor64(key, 16));
          if constexpr (Q >= 64) key = kmax(key, shfl_xor64(key, 32));
          if ((e % Q) == 0 && key) atomicMax(key_slot(a, e / Q), key);
        } else {
          emit4<EPI>(a, tid, e / Q, p * TC + (e % Q) * 4, v[j]);
        }
      }
    }
    if (tid == 0) atomicExch(&a.tile_cnt[p], 0u);
  }
  __syncthreads();
}

// After the whole grid is done, the last workgroup turns keys into ids and
// returns the keys and the done counter to zero (keys are read and cleared
// with device-coherent atomics).
template <int EPI, int NT>
__device__ __forceinline__ void finish_grid(const GemmParams& a, int tid, int* s_last) {
  if constexpr (EPI == kEpiArgmax) {
    writes_done_barrier();
    if (tid == 0) *s_last = (atomicAdd(a.done, 1u) == (uint32_t)(a.G - 1)) ? 1 : 0;
    __syncthreads();
    if (*s_last) {
      for (int m = tid; m < a.M; m += NT) {
        unsigned long long c[kKeyCopies];
#pragma unroll
        for (int x = 0; x < kKeyCopies; ++x) c[x] = atomicExch(a.keys + (x * kKeyRows + m) * kKeyStride, 0ull);
        unsigned long long k = c[0];
#pragma unroll
        for (int x = 1; x < kKeyCopies; ++x) k = kmax(k, c[x]);
        a.idx[m] = (int32_t)(0xFFFFFFFFu - (uint32_t)k);
        if (a.maxval) a.maxval[m] = key_float((uint32_t)(k >> 32));
      }
      if (tid == 0) atomicExch(a.done, 0u);
    }
  }
}

// End of a workgroup's slice. The partial sums of the (at most two) tiles it
// shares with its neighbours were stored when those tiles ended; the hand-off
// waits until now, so no memory round trip stalled the stream. Then, for the
// argmax epilogue, the grid-wide key-to-id step.
template <int EPI, int NT, int TC, int CH>
__device__ __forceinline__ void finish_slice(const GemmParams& a, int tid, int u0, int u1, int* s_last) {
  const int RK = a.RK, p0 = u0 / RK, p1 = (u1 - 1) / RK;
  const bool s0 = u0 < u1 && tile_is_split(p0, u0, u1, RK);
  const bool s1 = u0 < u1 && p1 != p0 && tile_is_split(p1, u0, u1, RK);
  if (s0 || s1 || EPI == kEpiArgmax) writes_done_barrier();
  if (s0) finish_split_tile<EPI, NT, TC, CH>(a, p0, tid, s_last);
  if (s1) finish_split_tile<EPI, NT, TC, CH>(a, p1, tid, s_last);
  finish_grid<EPI, NT>(a, tid, s_last);
}

// Per-wave patch buffer of one strip: 2 KB of restored weights laid out as
// halfword k4 * 512 + k3 * 256 + c * 8 + (kk & 7) for weight (channel c,
// subtile column kk = 16 k4 + 8 k3 + (kk & 7)). Lane c + 32 h writes its pairs
// 0..3 at byte h * 1024 + c * 16 and 4..7 at 512 bytes further on, so each
// half-wave of a 16-byte access covers 512 consecutive bytes.
__device__ __forceinline__ uint32_t patch_lane_off(int lane) {
  return (uint32_t)(lane & 31) * 16u + (uint32_t)(lane >> 5) * 1024u;
}
__device__ __forceinline__ void patch_store(char* buf, uint32_t lo, const uint32_t (&p)[8]) {
  *reinterpret_cast<uint4*>(buf + lo) = make_uint4(p[0], p[1], p[2], p[3]);
  *reinterpret_cast<uint4*>(buf + lo + 512) = make_uint4(p[4], p[5], p[6], p[7]);
}
__device__ __forceinline__ void patch_load(const char* buf, uint32_t lo, uint32_t (&p)[8]) {
  const uint4 r0 = *reinterpret_cast<const uint4*>(buf + lo);
  const uint4 r1 = *reinterpret_cast<const uint4*>(buf + lo + 512);
  p[0] = r0.x; p[1] = r0.y; p[2] = r0.z; p[3] = r0.w;
  p[4] = r1.x; p[5] = r1.y; p[6] = r1.z; p[7] = r1.w;
}
// Overwrite one restored weight with an escape entry (bits << 16 | c << 5 | kk):
// its byte in the layout above, straight from the entry's low bits.
__device__ __forceinline__ void patch_put(char* buf, uint32_t e) {
  const uint32_t at = ((e << 6) & 0x600u) | ((e >> 1) & 0x1F0u) | ((e << 1) & 0xEu);
  *reinterpret_cast<uint16_t*>(buf + at) = esc_bits(e);
}

// The certified head's INT8 copy: the lane's 16 codes q (one 16-byte load,
// the same place a W12 record keeps the 8-bit view) and its block's scale
// code (s + 133; 0 when the block has no window weight, then every q is 0)
// give the bf16 pairs q * 2^s, exact: |q| <= 127 has at most 7 significant
// bits, so the binary32 value q * 2^s keeps its low 16 bits zero.
__device__ __forceinline__ void cert_decode16(const uint4 hi, uint32_t code, uint32_t (&p)[8]) {
  const int sig = code ? (int)code - 133 : 0;
  const uint32_t d[4] = {hi.x, hi.y, hi.z, hi.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t word = d[i >> 1];
    const int sh = 16 * (i & 1);
    const float f0 = __builtin_amdgcn_ldexpf((float)(int)(int8_t)(word >> sh), sig);
    const float f1 = __builtin_amdgcn_ldexpf((float)(int)(int8_t)(word >> (sh + 8)), sig);
    p[i] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
  }
}

// Restore the lane's NQ x 16 weights of a unit (one subtile of each strip of
// the tile) and apply the escape blocks' entries: the restored pairs go to the
// wave's LDS patch buffer (2 KB per strip), the lanes holding entries overwrite
// their slots, the pairs are read back. Only the wave itself touches its buffer.
// For the INT8 copy, bias[q] is the lane's block scale code instead.
template <int NQ, int FMT = kFmtW12, typename SlotT>
__device__ __forceinline__ void restore_unit(const SlotT& s, const uint32_t (&bias)[NQ], char* patch,
                                             uint32_t plo, int lane, rsrc_t r_esc, uint32_t (&P)[NQ][8]) {
  int cq[NQ];
  int any = 0;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    // a block holds at most 1024 weights: corrupt offsets cannot make the
    // patch loop run longer (entries are read through a resource that ends
    // at the escape count, so reads stay in bounds either way)
    const u32x2 oq = s.off_of(q);
    cq[q] = min(max((int)(oq.y - oq.x), 0), 1024);
    any |= cq[q];
  }
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    if constexpr (FMT == kFmtCert8) {
      cert_decode16(uint4{s.hi[q].x, s.hi[q].y, s.hi[q].z, s.hi[q].w}, bias[q], P[q]);
    } else {
      decode16(uint4{s.hi[q].x, s.hi[q].y, s.hi[q].z, s.hi[q].w}, uint2{s.lo[q].x, s.lo[q].y}, bias[q], P[q]);
    }
  }
  if (any > 0) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) patch_store(patch + q * 2048, plo, P[q]);
    wave_lds_order();
    if constexpr (NQ % 2 == 0) {
      // one entry load per pair of strips: lane l holds entry l % 32 of
      // strip 2 i + l / 32 in e[i]
      const int ql = lane >> 5;
#pragma unroll
      for (int i = 0; i < NQ / 2; ++i)
        if ((lane & 31) < (ql ? cq[2 * i + 1] : cq[2 * i])) patch_put(patch + (2 * i + ql) * 2048, s.e[i]);
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        if (cq[q] > 32) {  // more than 32 entries: rare, read the rest here
          const uint32_t o = s.off_of(q).x;
          for (int j = 32 + lane; j < cq[q]; j += 64) patch_put(patch + q * 2048, bload1(r_esc, (o + j) * 4u, 0));
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        if (lane < cq[q]) patch_put(patch + q * 2048, s.e[q]);
        if (cq[q] > 64) {  // more than one entry per lane: rare, read the rest here
          const uint32_t o = s.off_of(q).x;
          for (int j = 64 + lane; j < cq[q]; j += 64) patch_put(patch + q * 2048, bload1(r_esc, (o + j) * 4u, 0));
        }
      }
    }
    wave_lds_order();
#pragma unroll
    for (int q = 0; q < NQ; ++q) patch_load(patch + q * 2048, plo, P[q]);
  }
}

// Row maximum of (value key, ~index) over the 16 lanes of a DPP row: after
// exchanges with lane ^ 1, lane ^ 2, the mirrored half-row and the mirrored
// row, every lane of the row holds the maximum.
template <int CTRL>
__device__ __forceinline__ unsigned long long max_dpp(unsigned long long v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  const unsigned long long w = ((unsigned long long)hi << 32) | lo;
  return w > v ? w : v;
}
__device__ __forceinline__ unsigned long long row16_max(unsigned long long v) {
  v = max_dpp<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v = max_dpp<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v = max_dpp<0x141>(v);  // row_half_mirror
  return max_dpp<0x140>(v);  // row_mirror
}

// Wave-uniform position of a load stream in the workgroup's slice: the unit
// it loads next, the units left before its next event (tile or slice
// boundary) and that unit's tile.
struct StreamPos {
  int u, left, p;
};

// One unit's loads for one wave (subtile t = wave of each of the NQ strips of a tile).
template <int XQ, int NQ>
struct Slot {
  u32x2 off[NQ];       // off[0], lane q < NQ: esc_off of strip q's escape block and of the next one
  __device__ __forceinline__ u32x2 off_of(int q) const {
    return u32x2{(uint32_t)__builtin_amdgcn_readlane((int)off[0].x, q), (uint32_t)__builtin_amdgcn_readlane((int)off[0].y, q)};
  }
  u32x4 hi[NQ];        // 8-bit view: 16 weights of channel lane%32, k half lane/32
  u32x2 lo[NQ];        // their low nibbles
  uint32_t et[NQ];     // et[0]: dword lane % 8 of strip (lane / 8) % NQ's window tops (INT8 copy: of
                       // the record's block scale codes); the lanes' own come by lane permute
  uint32_t e[NQ];      // escape entry number `lane` of the block (if any)
  u32x4 xv[XQ][2];     // x operands that ride with the unit
};

// Load ordering: vector loads of a wave return in issue order, so a wait for
// one load is a wait for every older one. Per unit there are three groups:
//   O  escape-block offsets                 issued D + 1 units ahead
//   W  records, window tops, x              issued D units ahead
//   E  escape entries (address <- O)        issued D units ahead, after the
//                                           arithmetic of the current unit
// E(u + D) needs O(u + D), which went out before W(u + D - 1); the only older
// loads are those of unit u, which the arithmetic of unit u has just waited
// for. So D units of weight loads stay in flight during that arithmetic. The
// ring holds D + 2 slots: O runs one slot ahead of W/E, and one slot is being
// computed.
template <int XQ, int NQ, int D>
struct Ring {
  static constexpr int NS = D + 2;
  Slot<XQ, NQ> s[NS];
};

// The Q pass (QP) reads only the 8-bit view of each record; the low nibbles
// it does not load are taken at their midpoint 0b1000.
constexpr uint32_t kMidNibbles = 0x88888888u;

// The per-unit loads shared by both small-m kernels, as two wave-uniform
// streams. Everything that changes only at a tile (the tile's record resource,
// window-top and escape-offset positions) is set up at the tile's first unit;
// per unit the streams only advance scalar offsets.
//  * W stream (records, window tops, x). The record resource covers the
//    tile's strips that exist, so a missing strip (the strip count is not a
//    multiple of NQ) reads zeros; past the slice the resources are empty and
//    the loads move no data. A missing strip's channels are never stored.
//  * O stream (escape-block offsets, one load per unit: lane q % NQ reads the
//    pair of strip q % NQ through a resource that covers esc_off exactly). A
//    missing strip, or a tile past the last, reads 1 GiB further on, out of
//    range: offsets 0, 0, no escapes.
//  * E (escape entries): one load per pair of strips, lane l reads entry
//    l % 32 of strip l / 32 of the pair's blocks, through a
//    resource that covers the n_esc entries; lanes past the block's count
//    are not used.
constexpr uint32_t kOutOfRange = 1u << 30;

// FMT = kFmtCert8 streams the certified head's INT8 copy instead: 8 KB
// records (the 8-bit-view plane layout, no low nibbles) and, in place of
// the window tops, the dword of block scale codes around the lane's channel
// (code (strip, record, subtile, channel) at byte ((strip * RK + record) * 8
// + subtile) * 32 + channel). Escapes come from the W12 head's lists.
template <int XQ, bool QP, int NQ, int FMT = kFmtW12>
struct UnitLoads {
  static constexpr bool kCert = FMT == kFmtCert8;
  static constexpr uint32_t kStep = kCert ? (uint32_t)kCertRecBytes : (uint32_t)kRecBytes;
  const GemmParams& a;
  int wave, RK, S, u1;
  uint32_t strip_bytes, v_hi, v_lo, v_l4, v_c4, v_et, sb_strip;
  rsrc_t r_esc, r_off, r_et;
  const void* x_base;
  uint32_t x_bytes, x_tile, x_step;
  // W stream
  StreamPos w;
  rsrc_t rt, rx;
  uint32_t so, sx, sb;
  // O stream
  StreamPos o;
  uint32_t oo, v_om;
  int lane_q;
  bool lane_q2;

  __device__ __forceinline__ UnitLoads(const GemmParams& a_, int wave_, int lane, int u0, int u1_,
                                       const void* xb, uint32_t xbytes, uint32_t xtile, uint32_t xstep)
      : a(a_), wave(wave_), RK(a_.RK), S(a_.S), u1(u1_), x_base(xb), x_bytes(xbytes), x_tile(xtile),
        x_step(xstep) {
    strip_bytes = (uint32_t)RK * kStep;
    sb_strip = kCert ? (uint32_t)RK * 256u : (uint32_t)kStrip;
    v_hi = (uint32_t)(wave * 1024 + lane * 16);
    v_lo = (uint32_t)(kHiBytes + wave * 512 + lane * 8);
    v_l4 = (uint32_t)lane * 4u;
    v_c4 = (uint32_t)(lane & 28);
    v_et = (uint32_t)((lane >> 3) % NQ) * sb_strip + (uint32_t)(lane & 7) * 4u;
    lane_q = lane % NQ;
    lane_q2 = lane >= 32;
    // escape count = esc_off[nb]; entries past it read as zero
    const uint32_t n_esc = scalar_view(a.w.esc_off)[a.w.nb];
    r_esc = make_rsrc(a.w.esc, n_esc < (1u << 30) ? n_esc * 4u : 0xFFFFFFFCu);
    r_off = make_rsrc(a.w.esc_off, (uint32_t)(a.w.nb + 1) * 4u);
    if constexpr (kCert) {
      r_et = make_rsrc(a.cexp, (uint32_t)(a.w.n * a.w.k / 32));
    } else {
      r_et = make_rsrc(a.w.e_top, (uint32_t)a.w.n);
    }
    const int p = u0 / RK, r = u0 - p * RK;
    w = StreamPos{u0, min(RK - r, u1 - u0), p};
    w_tile(r);
    o = StreamPos{u0, RK - r, p};
    o_tile(r);
  }

  // The W stream enters tile w.p at record r.
  __device__ __forceinline__ void w_tile(int r) {
    const int sq = NQ * w.p;
    const int ns = min(NQ, S - sq);
    rt = make_rsrc(rec_base() + (int64_t)sq * strip_bytes, (uint32_t)ns * strip_bytes);
    rx = make_rsrc(x_base, x_bytes);
    so = (uint32_t)r * kStep;
    sx = x_tile + (uint32_t)r * x_step;
    sb = kCert ? (uint32_t)(((sq * RK + r) * 8 + wave) * 32) : (uint32_t)sq * kStrip;
  }
  __device__ __forceinline__ const uint8_t* rec_base() const {
    if constexpr (kCert) {
      return reinterpret_cast<const uint8_t*>(a.cq);
    } else {
      return a.w.rec;
    }
  }
  __device__ __forceinline__ void w_next() {
    ++w.u;
    so += kStep;
    sx += x_step;
    if constexpr (kCert) sb += 256u;  // the next record's codes
    if (--w.left == 0) {
      if (w.u >= u1) {  // past the slice
        rt = make_rsrc(rec_base(), 0u);
        rx = rt;
        w.left = 1 << 30;
      } else {
        ++w.p;
        w_tile(0);
        w.left = min(RK, u1 - w.u);
      }
    }
  }
  // The O stream enters tile o.p at record r: escape block (strip, r, wave).
  __device__ __forceinline__ void o_tile(int r) {
    const int sq = NQ * o.p;
    v_om = (uint32_t)(lane_q * RK) * 32u + (sq + lane_q < S ? 0u : kOutOfRange);
    oo = (uint32_t)((((sq < S ? sq : 0) * RK + r) * 8 + wave) * 4);
  }
  __device__ __forceinline__ void o_next() {
    ++o.u;
    oo += 8 * 4;
    if (--o.left == 0) {
      ++o.p;
      o_tile(0);
      o.left = RK;
    }
  }

  __device__ __forceinline__ void issue_off(Slot<XQ, NQ>& s) const {
    // one load for all strips: lane q (< NQ) reads strip q's pair (the other
    // lanes repeat it); the strips' pairs come back by readlane
    s.off[0] = bload2(r_off, v_om, oo);
  }
  __device__ __forceinline__ void issue_w(Slot<XQ, NQ>& s) const {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const uint32_t sq = so + (uint32_t)q * strip_bytes;
      s.hi[q] = bload4<kNonTemporal>(rt, v_hi, sq);
      if constexpr (QP || kCert) {
        s.lo[q] = u32x2{kMidNibbles, kMidNibbles};
      } else {
        s.lo[q] = bload2<kNonTemporal>(rt, v_lo, sq);
      }
      // a whole dword: a byte load's result would be widened where the ring
      // wraps round, which makes the compiler wait for the load right there
      if (q == 0) {
        // one load for all NQ strips: lane l holds dword l % 8 of strip
        // (l / 8) % NQ (the tile's window tops; for the INT8 copy, the
        // record's block scale codes); each lane fetches its strips' dwords
        // with a lane permute at the unit's arithmetic (LM head, 4-strip
        // tiles: 207.7 -> 199.8 us against a load per strip)
        s.et[0] = bload1(r_et, v_et, sb);
      }
    }
  }
  __device__ __forceinline__ void issue_e(Slot<XQ, NQ>& s) const {
    if constexpr (NQ % 2 == 0) {
      // one load per pair of strips: lane l reads entry l % 32 of strip
      // 2 i + l / 32 (a block with more than 32 entries reads the rest at
      // its patch)
#pragma unroll
      for (int i = 0; i < NQ / 2; ++i) {
        const uint32_t o0 = s.off_of(2 * i).x, o1 = s.off_of(2 * i + 1).x;
        s.e[i] = bload1(r_esc, (lane_q2 ? o1 : o0) * 4u + (v_l4 & 124u), 0);
      }
    } else {
#pragma unroll
      for (int q = 0; q < NQ; ++q) s.e[q] = bload1(r_esc, s.off_of(q).x * 4u + v_l4, 0);
    }
  }
};

// The slice walk: prologue, steady state without conditional steps (a skipped
// step inside the unrolled body would make the compiler's load-wait counts
// assume fewer loads in flight and wait for the next units' loads as well),
// and a guarded tail of fewer than NS units.
template <int XQ, int NQ, int D, typename LoadsT, typename XF, typename StepF>
__device__ __forceinline__ void walk_slice(LoadsT& L, int u0, int u1, XF&& issue_x, StepF&& step) {
  Ring<XQ, NQ, D> ring;
  constexpr int NS = Ring<XQ, NQ, D>::NS;
  static_for<D + 1>([&](auto jc) {
    L.issue_off(ring.s[decltype(jc)::value]);
    L.o_next();
  });
  static_for<D>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    L.issue_w(ring.s[j]);
    issue_x(ring.s[j]);
    L.w_next();
  });
  static_for<D>([&](auto jc) { L.issue_e(ring.s[decltype(jc)::value]); });
  auto iteration = [&](auto kc) __attribute__((always_inline)) {
    constexpr int k = decltype(kc)::value;
    // a wave whose unit has arrived issues the next loads ahead of the other
    // waves' arithmetic, keeping the memory pipeline full
    __builtin_amdgcn_s_setprio(2);
    L.issue_off(ring.s[(k + D + 1) % NS]);
    L.o_next();
    L.issue_w(ring.s[(k + D) % NS]);
    issue_x(ring.s[(k + D) % NS]);
    L.w_next();
    __builtin_amdgcn_s_setprio(0);
    step(ring.s[k]);
    L.issue_e(ring.s[(k + D) % NS]);
  };
  int base = u0;
  for (; base + NS <= u1; base += NS) static_for<NS>(iteration);
  static_for<NS>([&](auto kc) {
    if (base + decltype(kc)::value < u1) iteration(kc);
  });
}

// Compute-side position: the tile whose units are being accumulated and the
// units left in it. flush(p) runs when the tile ends.
struct TileCursor {
  int p, left, u;
};

// (E_n - 15) << 7 in both 16-bit halves, from the dword of window tops that
// holds E_n in byte lane % 4.
__device__ __forceinline__ uint32_t bias2_of_top(uint32_t et4, int lane) {
  return __builtin_amdgcn_ubfe(et4, 8u * (uint32_t)(lane & 3), 8) * 0x00800080u - 0x07800780u;
}

// ============================================================================ MFMA path (5 <= m <= 64)

template <int MT, int EPI, bool QP, int NQ, int FMT = kFmtW12>
__global__ __launch_bounds__(kNT) void gemm_mfma_kernel(GemmParams a) {
  static_assert((FMT == kFmtCert8) == (EPI == kEpiCert), "the INT8 copy runs the bound epilogue");
  // x fragments of the MT tiles of 32 rows ride in the load ring.
  static_assert(MT >= 1 && MT <= 2, "small-m kernel: at most 64 rows");
  constexpr int XQ = MT;
  // NQ strips per tile (each x load serves NQ strips). With 4 strips the ring
  // is one unit deep to stay within the register file; the plan picks 4-strip
  // tiles (up to 32 rows) only where slices hold many units.
  constexpr int D = NQ == 4 ? 1 : 2;
  constexpr int TC = NQ * kStrip;       // channels per tile
  constexpr int RS = TC + 4;            // reduction slot row stride (floats)
  constexpr int SF = 32 * RS;           // reduction slot (one wave, one M-tile)
  __shared__ __align__(16) float lds[kNW * SF];  // reduction slots; patch buffers alias them
  __shared__ int s_last;
  // INT8 pass: the bound constants of the channels of the slice's tiles
  __shared__ __align__(16) float cbl[FMT == kFmtCert8 ? kCertCbFloats : 4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = logical_wg(blockIdx.x, a.G);
  const int U = a.U, RK = a.RK;
  const int u0 = chunk_begin(g, U, a.G), u1 = chunk_begin(g + 1, U, a.G);
  char* patch = reinterpret_cast<char*>(lds) + wave * (NQ * 2048);
  static_assert(kNW * NQ * 2048 <= kNW * SF * 4, "patch buffers fit in the reduction slots");

  f32x16 acc[NQ][MT];
  unsigned long long run[MT];  // argmax: best key of row mt * 32 + tid / 16 over the slice's whole tiles
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) run[mt] = 0;
#pragma unroll
  for (int q = 0; q < NQ; ++q)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[q][mt][i] = 0.f;

  // x fragment (record r, subtile t, tile mt, half h): lane l holds x[mt * 32
  // + l % 32][32 (8 r + t) + 16 (l / 32) + 8 h ..]. From the pre-pass's
  // fragment buffer it is 16 bytes at ((r * 8 + t) * MT + mt) * 2048 + h * 1024
  // + 16 l; where the plan skips the pre-pass (slices of a few units, whose
  // call the separate launch would dominate), the lane reads those 16 bytes
  // of row-major x itself, and rows >= M lie outside the resource and read as
  // zero.
  const bool xd = FMT == kFmtW12 && a.xdirect;
  const uint32_t row_bytes = 2u * (uint32_t)a.K;
  UnitLoads<XQ, QP, NQ, FMT> L(a, wave, lane, u0, u1, xd ? static_cast<const void*>(a.x) : static_cast<const void*>(a.xf),
                               xd ? (uint32_t)a.M * row_bytes : (uint32_t)(MT * 32) * row_bytes,
                               xd ? (uint32_t)(wave * 64) : (uint32_t)(wave * MT * 2048),
                               xd ? 512u : (uint32_t)(MT * 8 * 2048));
  const uint32_t plo = patch_lane_off(lane);
  const uint32_t v_x = xd ? (uint32_t)(lane & 31) * row_bytes + 32u * (uint32_t)(lane >> 5) : (uint32_t)lane * 16u;
  const uint32_t x_mt = xd ? 32u * row_bytes : 2048u, x_h = xd ? 16u : 1024u;

  // INT8 pass: the thread's row norms, and the slice's channel constants in
  // LDS (the host checks that they fit; the first tile end's barrier orders
  // these writes before any read)
  float xn[MT];
  int ch0 = 0;
  if constexpr (FMT == kFmtCert8) {
    ch0 = (u0 / RK) * TC;
    const int ch1 = u0 < u1 ? min(((u1 - 1) / RK + 1) * TC, a.N) : ch0;
    for (int i = tid; i < ch1 - ch0; i += kNT) cbl[i] = a.cbound[ch0 + i];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 32 + (tid >> 4);
      xn[mt] = m < a.M ? a.xnorm[m] : 0.f;
    }
  }

  auto issue_x = [&](Slot<XQ, NQ>& s) __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < XQ; ++mt) {
      s.xv[mt][0] = bload4(L.rx, v_x + (uint32_t)mt * x_mt, L.sx);
      s.xv[mt][1] = bload4(L.rx, v_x + (uint32_t)mt * x_mt + x_h, L.sx);
    }
  };

  // ---- tile end: reduce the 8 waves' accumulators, write or hand off. Every
  // wave writes its 32 x 64 partial to a slot of its own, then each thread
  // sums one row quad over the 8 slots in a fixed order.
  // The partial of a split tile that ends inside the slice (only the first
  // tile can) is stored after the walk, not when the tile ends: a store
  // issued between record loads holds back the completion count of every
  // later load until it is acknowledged, and a write-through store at device
  // scope is acknowledged slowly under the record stream (measured: 3.5 us per
  // Wgate|Wup launch at 32 rows, 9 us on the LM head). Until then each thread
  // keeps its own quads in LDS, or in registers for the INT8 pass's 4-strip
  // tiles, whose LDS is full.
  constexpr bool kStageInRegs = FMT == kFmtCert8 && NQ == 4;
  constexpr int kStageQ = MT * (NQ / 2);  // float4 per thread
  __shared__ __align__(16) float4 stage[kStageInRegs ? 1 : kStageQ * kNT];
  float4 stage_r[kStageInRegs ? kStageQ : 1];
  const int p_last = (u1 - 1) / RK;
  auto flush = [&](int p) __attribute__((always_inline)) {
    const bool whole = !tile_is_split(p, u0, u1, RK);
    const int slot = partial_slot(g, p, U, a.G, RK);
    static_for<MT>([&](auto mtc) {
      constexpr int mt = decltype(mtc)::value;
      lds_barrier();  // the slots (and patch buffers) are free
      {
        float* dst = lds + wave * SF;
        const int ml = lane & 31, hf = lane >> 5;
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
          for (int rb = 0; rb < 4; ++rb)
            *reinterpret_cast<float4*>(dst + ml * RS + 32 * q + 8 * rb + 4 * hf) =
                make_float4(acc[q][mt][4 * rb], acc[q][mt][4 * rb + 1], acc[q][mt][4 * rb + 2],
                            acc[q][mt][4 * rb + 3]);
      }
      lds_barrier();
      // 32 rows x 16 channel quads per pass: 16 consecutive threads hold 64
      // channels of one row
#pragma unroll
      for (int h = 0; h < NQ / 2; ++h) {
        const int ml = tid >> 4, c4 = h * 64 + (tid & 15) * 4;
        const float* b = lds + ml * RS + c4;
        float4 sw[kNW];
#pragma unroll
        for (int w = 0; w < kNW; ++w) sw[w] = *reinterpret_cast<const float4*>(b + w * SF);
        const float4 v = f4add(f4add(f4add(sw[0], sw[4]), f4add(sw[1], sw[5])),
                               f4add(f4add(sw[2], sw[6]), f4add(sw[3], sw[7])));
        const int m = mt * 32 + ml;
        if (whole) {
          if constexpr (EPI == kEpiArgmax) {
            run[mt] = kmax(run[mt], row_key4(a, m, p * TC + c4, v));
          } else if constexpr (EPI == kEpiCert) {
            const float4 cb = *reinterpret_cast<const float4*>(cbl + (p * TC + c4 - ch0));
            run[mt] = kmax(run[mt], cert_emit4(a, m, p * TC + c4, v, cb, xn[mt]));
          } else {
            emit4<EPI>(a, tid, m, p * TC + c4, v);
          }
        } else if (p == p_last) {
          if (m < a.M) store_partial<TC>(a, slot, m, c4, v);
        } else if constexpr (kStageInRegs) {
          stage_r[mt * (NQ / 2) + h] = v;
        } else {
          stage[(mt * (NQ / 2) + h) * kNT + tid] = v;
        }
      }
    });
    lds_barrier();
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[q][mt][i] = 0.f;
  };

  // ---- arithmetic of one unit
  TileCursor cur{u0 / RK, min(RK - (u0 - (u0 / RK) * RK), u1 - u0), u0};
  auto step = [&](const Slot<XQ, NQ>& s) __attribute__((always_inline)) {
    if (cur.left == 0) {
      flush(cur.p);
      ++cur.p;
      cur.left = min(RK, u1 - cur.u);
    }
    --cur.left;
    ++cur.u;
    uint32_t bias[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      if constexpr (FMT == kFmtCert8) {
        bias[q] = __builtin_amdgcn_ubfe((uint32_t)__builtin_amdgcn_ds_bpermute((q * 8 + ((lane & 31) >> 2)) * 4, (int)s.et[0]),
                                        8u * (uint32_t)(lane & 3), 8);  // block scale code
      } else {
        bias[q] = bias2_of_top((uint32_t)__builtin_amdgcn_ds_bpermute((q * 8 + ((lane & 31) >> 2)) * 4, (int)s.et[0]), lane);
      }
    }
    uint32_t P[NQ][8];
    restore_unit<NQ, FMT>(s, bias, patch, plo, lane, L.r_esc, P);
    const u32x4 (&xl)[MT][2] = s.xv;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const bf16x8 a0 = __builtin_bit_cast(bf16x8, u32x4{P[q][0], P[q][1], P[q][2], P[q][3]});
      const bf16x8 a1 = __builtin_bit_cast(bf16x8, u32x4{P[q][4], P[q][5], P[q][6], P[q][7]});
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        acc[q][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, __builtin_bit_cast(bf16x8, xl[mt][0]), acc[q][mt], 0, 0, 0);
        acc[q][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, __builtin_bit_cast(bf16x8, xl[mt][1]), acc[q][mt], 0, 0, 0);
      }
    }
  };

  if (u0 < u1) {
    walk_slice<XQ, NQ, D>(L, u0, u1, issue_x, step);
    if (const int p0 = u0 / RK; p0 != p_last && tile_is_split(p0, u0, u1, RK)) {
      const int slot0 = partial_slot(g, p0, U, a.G, RK);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int h = 0; h < NQ / 2; ++h) {
          const int m = mt * 32 + (tid >> 4), c4 = h * 64 + (tid & 15) * 4;
          const float4 v = kStageInRegs ? stage_r[mt * (NQ / 2) + h] : stage[(mt * (NQ / 2) + h) * kNT + tid];
          if (m < a.M) store_partial<TC>(a, slot0, m, c4, v);
        }
    }
    flush(cur.p);
  }
  if constexpr (EPI == kEpiArgmax || EPI == kEpiCert) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      if ((tid & 15) == 0 && run[mt]) atomicMax(key_slot(a, mt * 32 + (tid >> 4)), run[mt]);
  }
  finish_slice<EPI, kNT, TC, 2>(a, tid, u0, u1, &s_last);
}

// ============================================================================ VALU path (m <= 4)

template <int MV, int EPI, bool QP>
__global__ __launch_bounds__(kNT) void gemm_valu_kernel(GemmParams a) {
  // x of the wave's subtile rides in the load ring: the wave's block of x (up
  // to 16 rows x 64 bytes) as one 16-byte piece per lane, through a private
  // 1 KB LDS buffer from which the half-waves read their rows as broadcasts.
  // (Measured against each lane loading the 32 bytes of every row itself:
  // Wgate|Wup 34816x5120 52.8 -> 50.8 us at 1 row, 57.7 -> 51.1 us at 2; the
  // 152064x5120 head 205 -> 194 and 227 -> 195 us; bit-identical.)
  constexpr int XQ = 1;
  constexpr int kValuDepth = kDepth;
  __shared__ __align__(16) float lds[kLdsFloats];
  __shared__ __align__(16) char xlds[kNW * 1024];
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = logical_wg(blockIdx.x, a.G);
  const int U = a.U, RK = a.RK;
  const int u0 = chunk_begin(g, U, a.G), u1 = chunk_begin(g + 1, U, a.G);
  char* patch = reinterpret_cast<char*>(lds) + wave * 4096;

  float acc[2][MV];
  unsigned long long run = 0;  // argmax: best key of row tid / 16 over the slice's whole tiles
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int m = 0; m < MV; ++m) acc[q][m] = 0.f;

  // x rows >= M read 0 (voffset past the range); a record's x starts 512 bytes on.
  UnitLoads<XQ, QP, 2> L(a, wave, lane, u0, u1, a.x, (uint32_t)a.M * (uint32_t)a.K * 2u, 0u, 512u);
  const uint32_t plo = patch_lane_off(lane);
  const uint32_t row_bytes = (uint32_t)a.K * 2u;

  // block piece of this lane: row lane / 4, bytes 16 (lane % 4) of the
  // subtile's 64 (rows >= m read 0)
  const uint32_t v_xp = (uint32_t)(lane >> 2) * row_bytes + (uint32_t)(wave * kSubK) * 2u + (uint32_t)(lane & 3) * 16u;
  char* xw = xlds + wave * 1024;
  auto issue_x = [&](Slot<XQ, 2>& s) __attribute__((always_inline)) { s.xv[0][0] = bload4(L.rx, v_xp, L.sx); };

  // ---- tile end: fold the two k halves, reduce the 8 waves, write or hand off.
  // As in the matrix-core path, a split tile that ends inside the slice has
  // its partial stored after the walk (held in a register until then).
  const int p_last = (u1 - 1) / RK;
  float4 stage = make_float4(0.f, 0.f, 0.f, 0.f);
  static_assert(MV * 16 <= kNT, "one row quad per thread at a tile end");
  auto flush = [&](int p) __attribute__((always_inline)) {
    const bool whole = !tile_is_split(p, u0, u1, RK);
    const int slot = partial_slot(g, p, U, a.G, RK);
    lds_barrier();
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int m = 0; m < MV; ++m) {
        const float v = acc[q][m] + __shfl_xor(acc[q][m], 32, 64);
        if (lane < 32) lds[((wave * 2 + q) * MV + m) * 32 + lane] = v;
      }
    lds_barrier();
    for (int e = tid; e < MV * 16; e += kNT) {
      const int m = e >> 4, c4 = (e & 15) * 4, q = c4 >> 5, c = c4 & 31;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int w = 0; w < kNW; ++w)
        v = f4add(v, *reinterpret_cast<const float4*>(lds + ((w * 2 + q) * MV + m) * 32 + c));
      if (whole) {
        if constexpr (EPI == kEpiArgmax) {
          run = kmax(run, row_key4(a, m, p * 64 + c4, v));
        } else {
          emit4<EPI>(a, tid, m, p * 64 + c4, v);
        }
      } else if (p != p_last) {
        stage = v;  // at most one quad per thread: MV * 16 <= the workgroup's threads
      } else if (m < a.M) {
        store_partial<64>(a, slot, m, c4, v);
      }
    }
    lds_barrier();
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int m = 0; m < MV; ++m) acc[q][m] = 0.f;
  };

  auto dot16 = [&](const uint32_t (&P)[8], u32x4 x0, u32x4 x1, float sum) __attribute__((always_inline)) {
    const uint32_t xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i)
      sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, P[i]),
                                            __builtin_bit_cast(bf16x2, xs[i]), sum, false);
    return sum;
  };

  TileCursor cur{u0 / RK, min(RK - (u0 - (u0 / RK) * RK), u1 - u0), u0};
  auto step = [&](const Slot<XQ, 2>& s) __attribute__((always_inline)) {
    if (cur.left == 0) {
      flush(cur.p);
      ++cur.p;
      cur.left = min(RK, u1 - cur.u);
    }
    --cur.left;
    ++cur.u;
    const uint32_t bias[2] = {bias2_of_top((uint32_t)__builtin_amdgcn_ds_bpermute(((lane & 31) >> 2) * 4, (int)s.et[0]), lane),
                              bias2_of_top((uint32_t)__builtin_amdgcn_ds_bpermute((8 + ((lane & 31) >> 2)) * 4, (int)s.et[0]), lane)};
    uint32_t P[2][8];
    restore_unit<2>(s, bias, patch, plo, lane, L.r_esc, P);
    wave_lds_order();  // the previous unit's reads of the buffer come first
    *reinterpret_cast<u32x4*>(xw + lane * 16) = s.xv[0][0];
    wave_lds_order();
    const char* xr = xw + 32 * (lane >> 5);
#pragma unroll
    for (int m = 0; m < MV; ++m) {
      const u32x4 x0 = *reinterpret_cast<const u32x4*>(xr + m * 64);
      const u32x4 x1 = *reinterpret_cast<const u32x4*>(xr + m * 64 + 16);
      acc[0][m] = dot16(P[0], x0, x1, acc[0][m]);
      acc[1][m] = dot16(P[1], x0, x1, acc[1][m]);
    }
  };

  if (u0 < u1) {
    walk_slice<XQ, 2, kValuDepth>(L, u0, u1, issue_x, step);
    if (const int p0 = u0 / RK; p0 != p_last && tile_is_split(p0, u0, u1, RK) && tid < MV * 16 && (tid >> 4) < a.M)
      store_partial<64>(a, partial_slot(g, p0, U, a.G, RK), tid >> 4, (tid & 15) * 4, stage);
    flush(cur.p);
  }
  if constexpr (EPI == kEpiArgmax) {
    if ((tid & 15) == 0 && tid < MV * 16 && run) atomicMax(key_slot(a, tid >> 4), run);
  }
  finish_slice<EPI, kNT, 64, 2>(a, tid, u0, u1, &s_last);
}

// ============================================================================ large-m path (m > 64)
//
// At a few hundred rows the MFMA work per weight byte is no longer small, and
// x per record (m x 512 B) outweighs the record itself. Layout for that case:
//  * Tile = 4 strips (128 channels); unit = one record of a tile; stream-K
//    slices and the fixed-order hand-off as above. A unit is walked in 4
//    stages of 64 k.
//  * 8 waves, two per SIMD: wave (s, kg) restores subtile 2h + kg of strip s
//    in stage h (the per-wave restore and escape patch of the small-m kernel)
//    and holds one strip x all M-tiles of accumulators.
//  * x of a stage (all rows x 64 k) is read from row-major x once per
//    workgroup -- every wave instruction reads 8 whole 128-byte row pieces --
//    and written to LDS rows of 144 bytes, double-buffered: the 16-byte pad
//    keeps both the stores and the B-fragment reads free of bank conflicts.
//    Rows >= m fall outside the x resource and read as zero.
//  * At a tile end the two k halves of each strip are summed through LDS.

constexpr int kBigTC = 4 * kStrip;         // channels per tile
constexpr int kStageK = 64;                // k per stage
constexpr int kStages = kRecK / kStageK;   // stages per record
constexpr int kXRow = 2 * kStageK + 16;    // LDS bytes per x row of a stage

// Position in a slice: unit (tile, record) and stage.
struct StageIt {
  int u, p, r, h;
  __device__ __forceinline__ void init(int u0, int RK) {
    u = u0;
    p = u0 / RK;
    r = u0 - p * RK;
    h = 0;
  }
  __device__ __forceinline__ void next(int RK) {
    if (++h == kStages) {
      h = 0;
      ++u;
      if (++r == RK) {
        r = 0;
        ++p;
      }
    }
  }
};

// Weight loads run 2 stages ahead of the arithmetic and escape offsets 3;
// the ring has one slot per stage of a unit, so one trip of the unit loop has
// compile-time slots and a tile can only end between trips.
constexpr int kBigDepth = kStages - 2;

constexpr int kB8NW = 8;
constexpr int kB8NT = kB8NW * 64;

template <int MT>
struct Big8Lds {
  static constexpr int kRounds = (MT + 1) / 2;        // x pieces per thread per stage
  static constexpr int kX = kRounds * 64 * kXRow;    // one stage buffer (64 rows per round)
  static constexpr int kPatch = kB8NW * 2 * 2048;    // per wave: strip buffer + drop buffer
  static constexpr int kRedMT = (MT + 1) / 2;        // M-tiles per reduction round
  static constexpr int kRed = 4 * kRedMT * 4 * 1024; // 4 waves x kRedMT x 4 float4 x 64 lanes
  static constexpr int kBytes = 2 * kX + kPatch + kRed;
};

struct Big8Slot {
  uint32_t off[2];  // esc_off of the escape block and of the next one
  u32x4 hi;         // 8-bit view: 16 weights of channel lane%32, k half lane/32
  u32x2 lo;         // their low nibbles
  uint32_t e[2];    // escape entries number lane and lane + 64 of the block
};

// Per-stage loads of wave (s, kg): subtile 2h + kg of strip 4p + s.
template <bool QP>
struct Big8Loads {
  const GemmParams& a;
  int u0, u1, s, kg, RK, S;
  uint32_t strip_bytes, v_hi, v_lo;
  rsrc_t r_esc;

  __device__ __forceinline__ void issue_off(Big8Slot& sl, const StageIt& it) const {
    const int sq = 4 * it.p + s;
    const bool ok = it.u < u1 && sq < S;
    const uint32_t b = ok ? ((uint32_t)sq * RK + it.r) * 8 + 2 * it.h + kg : 0u;
    const cu32p c = scalar_view(a.w.esc_off);
    const uint32_t o0 = c[b], o1 = c[b + 1];
    sl.off[0] = ok ? o0 : 0u;
    sl.off[1] = ok ? o1 : 0u;
  }
  __device__ __forceinline__ void issue_w(Big8Slot& sl, const StageIt& it) const {
    const int sq = 4 * it.p + s;
    const bool ok = it.u < u1 && sq < S;
    const uint32_t t = 2 * it.h + kg, so = (uint32_t)it.r * kRecBytes;
    const rsrc_t r = make_rsrc(a.w.rec + (int64_t)(ok ? sq : 0) * strip_bytes, ok ? strip_bytes : 0u);
    sl.hi = bload4<kNonTemporal>(r, v_hi, so + t * 1024);
    if constexpr (QP) {
      sl.lo = u32x2{kMidNibbles, kMidNibbles};
    } else {
      sl.lo = bload2<kNonTemporal>(r, v_lo, so + t * 512);
    }
  }
  __device__ __forceinline__ void issue_e(Big8Slot& sl, int lane) const {
    const uint32_t o = sl.off[0];
    const int c = (int)(sl.off[1] - o);
#pragma unroll
    for (int h = 0; h < 2; ++h)
      sl.e[h] = bload1(r_esc, (c > 0 ? o + (uint32_t)min(lane + 64 * h, c - 1) : 0u) * 4u, 0);
  }
};

// Restore of one strip's 16 weights of the lane and the escape patch (first
// 128 entries branch-free, as in restore_big; the rest in a second pass).
__device__ __forceinline__ void restore_big8(const Big8Slot& sl, uint32_t bias, int cnt, char* patch, uint32_t plo,
                                             int lane, rsrc_t r_esc, uint32_t (&P)[8]) {
  decode16(uint4{sl.hi.x, sl.hi.y, sl.hi.z, sl.hi.w}, uint2{sl.lo.x, sl.lo.y}, bias, P);
  patch_store(patch, plo, P);
  wave_lds_order();
  const uint32_t base = cnt > 0 ? 0u : 2048u;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t e = sl.e[h];
    const uint32_t at = base + (((e << 6) & 0x600u) | ((e >> 1) & 0x1F0u) | ((e << 1) & 0xEu));
    *reinterpret_cast<uint16_t*>(patch + at) = esc_bits(e);
  }
  wave_lds_order();
  patch_load(patch, plo, P);
  if (cnt > 128) {  // rare: the rest of the entries in a second pass
    wave_lds_order();
    patch_store(patch, plo, P);
    wave_lds_order();
    const uint32_t o = sl.off[0];
    for (int j = 128 + lane; j < cnt; j += 64) patch_put(patch, bload1(r_esc, (o + j) * 4u, 0));
    wave_lds_order();
    patch_load(patch, plo, P);
  }
}

// Stage walk of the 8-wave layout. x runs two stages ahead in two register
// sets (x of stage s + 2 is loaded at the start of stage s, stored at the end
// of stage s + 1): loads complete in issue order, so the store's wait covers
// the weight loads issued before it, and a second stage of lead time keeps
// that wait from pacing the stages.
template <int MT, typename LoadsT, typename XL, typename XS, typename TF, typename StepF>
__device__ __forceinline__ void walk_big8(const LoadsT& L, int lane, int u0, int u1, int RK, XL&& xload,
                                          XS&& xstore, TF&& tile_end, StepF&& step) {
  constexpr int XR = Big8Lds<MT>::kRounds;
  Big8Slot ring[kStages];
  StageIt itO, itW, itX;
  itO.init(u0, RK);
  itW.init(u0, RK);
  itX.init(u0, RK);
  u32x4 xr[2][XR];
  xload(xr[0], itX);
  itX.next(RK);
  xload(xr[1], itX);
  itX.next(RK);
  L.issue_off(ring[0], itO);
  itO.next(RK);
  static_for<kBigDepth>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    L.issue_off(ring[j + 1], itO);
    itO.next(RK);
    L.issue_w(ring[j], itW);
    L.issue_e(ring[j], lane);
    itW.next(RK);
  });
  xstore(xr[0], 0);
  lds_barrier();
  auto iteration = [&](auto kc) __attribute__((always_inline)) {
    constexpr int k = decltype(kc)::value;
    xload(xr[k & 1], itX);  // x of stage k + 2
    itX.next(RK);
    L.issue_off(ring[(k + kBigDepth + 1) % kStages], itO);
    itO.next(RK);
    L.issue_w(ring[(k + kBigDepth) % kStages], itW);
    L.issue_e(ring[(k + kBigDepth) % kStages], lane);
    itW.next(RK);
    step(ring[k], k & 1);
    xstore(xr[(k + 1) & 1], (k + 1) & 1);  // x of stage k + 1
    lds_barrier();
  };
  for (int u = u0; u < u1;) {
    const int p = u / RK, ue = min(u1, (p + 1) * RK);
    for (; u < ue; ++u) static_for<kStages>(iteration);
    tile_end(p);
  }
}

template <int MT, int EPI, bool QP>
__global__ __launch_bounds__(kB8NT) void gemm_big8_kernel(GemmParams a) {
  using Lds = Big8Lds<MT>;
  constexpr int XR = Lds::kRounds;
  __shared__ __align__(16) char lds[Lds::kBytes];
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sw = wave & 3, kg = wave >> 2;
  const int g = logical_wg(blockIdx.x, a.G);
  const int U = a.U, RK = a.RK, S = a.S;
  const int u0 = chunk_begin(g, U, a.G), u1 = chunk_begin(g + 1, U, a.G);
  char* patch = lds + 2 * Lds::kX + wave * 4096;
  float* red = reinterpret_cast<float*>(lds + 2 * Lds::kX + Lds::kPatch);

  f32x16 acc[MT];
  // argmax: lanes < 32 of the kg = 0 waves keep the best key of row
  // mt * 32 + lane over their strip of the slice's whole tiles
  unsigned long long run[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) run[mt] = 0;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mt][i] = 0.f;

  // escape entries read through a resource that ends at the escape count
  const uint32_t n_esc = scalar_view(a.w.esc_off)[a.w.nb];
  const Big8Loads<QP> L{a, u0, u1, sw, kg, RK, S, (uint32_t)RK * kRecBytes, (uint32_t)(lane * 16),
                    (uint32_t)(kHiBytes + lane * 8), make_rsrc(a.w.esc, n_esc < (1u << 30) ? n_esc * 4u : 0xFFFFFFFCu)};
  const uint32_t plo = patch_lane_off(lane);

  // x staging: thread piece j = tid & 7 (16 B) of row 64 i + (tid >> 3)
  const uint32_t x_bytes = (uint32_t)a.M * (uint32_t)a.K * 2u;
  const uint32_t row64 = 128u * (uint32_t)a.K;  // bytes of 64 rows
  const uint32_t v_x = (uint32_t)(tid >> 3) * 2u * (uint32_t)a.K + (uint32_t)(tid & 7) * 16u;
  const uint32_t x_w = (uint32_t)(tid >> 3) * kXRow + (uint32_t)(tid & 7) * 16u;
  auto xload = [&](u32x4 (&xr)[XR], const StageIt& it) __attribute__((always_inline)) {
    const rsrc_t rx = make_rsrc(a.x, it.u < u1 ? x_bytes : 0u);
    const uint32_t so = ((uint32_t)it.r * kRecK + (uint32_t)it.h * kStageK) * 2u;
#pragma unroll
    for (int i = 0; i < XR; ++i) xr[i] = bload4(rx, v_x + i * row64, so);
  };
  auto xstore = [&](const u32x4 (&xr)[XR], int buf) __attribute__((always_inline)) {
    char* b = lds + buf * Lds::kX + x_w;
#pragma unroll
    for (int i = 0; i < XR; ++i) *reinterpret_cast<u32x4*>(b + i * 64 * kXRow) = xr[i];
  };
  // B fragment of (mt, i2): x[mt*32 + lane%32][32 kg + 16 (lane/32) + 8 i2 ..]
  const uint32_t x_r = (uint32_t)(lane & 31) * kXRow + 64u * kg + 32u * (uint32_t)(lane >> 5);

  // ---- tile end: sum the two k halves of each strip, write or hand off
  auto flush = [&](int p) __attribute__((always_inline)) {
    const bool whole = !tile_is_split(p, u0, u1, RK);
    const int slot = partial_slot(g, p, U, a.G, RK);
    const int c0 = sw * kStrip + 4 * (lane >> 5);  // channel within the tile
    const bool cvalid = p * kBigTC + c0 < a.N;
    unsigned long long best[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) best[mt] = 0;
    static_for<(MT + Lds::kRedMT - 1) / Lds::kRedMT>([&](auto rc) {
      constexpr int m0 = decltype(rc)::value * Lds::kRedMT;
      constexpr int m1 = m0 + Lds::kRedMT < MT ? m0 + Lds::kRedMT : MT;
      if (m0 > 0) lds_barrier();
      if (kg == 1) {
#pragma unroll
        for (int mt = m0; mt < m1; ++mt)
#pragma unroll
          for (int rb = 0; rb < 4; ++rb)
            *reinterpret_cast<float4*>(red + (((sw * Lds::kRedMT + mt - m0) * 4 + rb) * 64 + lane) * 4) =
                make_float4(acc[mt][4 * rb], acc[mt][4 * rb + 1], acc[mt][4 * rb + 2], acc[mt][4 * rb + 3]);
      }
      lds_barrier();
      if (kg == 0) {
#pragma unroll
        for (int mt = m0; mt < m1; ++mt) {
          const int m = mt * 32 + (lane & 31);
#pragma unroll
          for (int rb = 0; rb < 4; ++rb) {
            const float4 o =
                *reinterpret_cast<const float4*>(red + (((sw * Lds::kRedMT + mt - m0) * 4 + rb) * 64 + lane) * 4);
            const float4 v = make_float4(acc[mt][4 * rb] + o.x, acc[mt][4 * rb + 1] + o.y,
                                         acc[mt][4 * rb + 2] + o.z, acc[mt][4 * rb + 3] + o.w);
            const int c = c0 + 8 * rb, n = p * kBigTC + c;
            if (!whole) {
              if (m < a.M && cvalid) store_partial<kBigTC>(a, slot, m, c, v);
            } else if constexpr (EPI == kEpiY) {
              if (m < a.M && cvalid) {
                if (a.ytype == 0) {
                  *reinterpret_cast<float4*>(static_cast<float*>(a.y) + (int64_t)m * a.N + n) = v;
                } else {
                  const uint32_t lo = f32_to_bf16_rne(v.x) | ((uint32_t)f32_to_bf16_rne(v.y) << 16);
                  const uint32_t hi = f32_to_bf16_rne(v.z) | ((uint32_t)f32_to_bf16_rne(v.w) << 16);
                  *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.y) + (int64_t)m * a.N + n) =
                      make_uint2(lo, hi);
                }
              }
            } else {
              if (cvalid) {
                const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const unsigned long long key = ((unsigned long long)float_key(vv[i]) << 32) |
                                                 (uint32_t)(0xFFFFFFFFu - (uint32_t)(n + i));
                  best[mt] = key > best[mt] ? key : best[mt];
                }
              }
            }
          }
        }
      }
    });
    if constexpr (EPI == kEpiArgmax) {
      if (whole && kg == 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int m = mt * 32 + (lane & 31);
          const uint32_t lo = (uint32_t)best[mt], hi = (uint32_t)(best[mt] >> 32);
          const unsigned long long o = ((unsigned long long)(uint32_t)__shfl_xor((int)hi, 32, 64) << 32) |
                                       (uint32_t)__shfl_xor((int)lo, 32, 64);
          if (lane < 32 && m < a.M) run[mt] = kmax(run[mt], kmax(o, best[mt]));
        }
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mt][i] = 0.f;
  };

  StageIt cur;
  cur.init(u0, RK);
  uint32_t bias = 0u;
  auto step = [&](const Big8Slot& sl, int buf) __attribute__((always_inline)) {
    const int sq = 4 * cur.p + sw;
    if (cur.h == 0 && (cur.r == 0 || cur.u == u0)) bias = strip_bias2(a.w.e_top, sq, sq < S, lane);
    const int cnt = min(__builtin_amdgcn_readfirstlane((int)(sl.off[1] - sl.off[0])), 1024);
    const char* xb = lds + buf * Lds::kX + x_r;
    bf16x8 bq[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) bq[mt] = *reinterpret_cast<const bf16x8*>(xb + mt * 32 * kXRow);
    uint32_t P[8];
    restore_big8(sl, bias, cnt, patch, plo, lane, L.r_esc, P);
    static_for<2>([&](auto ic) {
      constexpr int i2 = decltype(ic)::value;
      const bf16x8 a0 = __builtin_bit_cast(bf16x8, u32x4{P[4 * i2], P[4 * i2 + 1], P[4 * i2 + 2], P[4 * i2 + 3]});
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if constexpr (i2 == 1) bq[mt] = *reinterpret_cast<const bf16x8*>(xb + mt * 32 * kXRow + 16);
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bq[mt], acc[mt], 0, 0, 0);
      }
    });
    cur.next(RK);
  };

  if (u0 < u1) walk_big8<MT>(L, lane, u0, u1, RK, xload, xstore, flush, step);
  if constexpr (EPI == kEpiArgmax) {
    // the 4 strip waves' keys of each row are maximised through LDS first:
    // one device-scope atomic per row and workgroup
    static_assert(Lds::kBytes >= MT * 4 * 32 * 8, "key buffer fits");
    unsigned long long* kb = reinterpret_cast<unsigned long long*>(lds);
    __syncthreads();
    if (kg == 0 && lane < 32) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) kb[(mt * 4 + sw) * 32 + lane] = run[mt];
    }
    __syncthreads();
    for (int r = tid; r < MT * 32; r += kB8NT) {
      unsigned long long b = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) b = kmax(b, kb[((r >> 5) * 4 + q) * 32 + (r & 31)]);
      if (b) atomicMax(key_slot(a, r), b);
    }
  }
  finish_slice<EPI, kB8NT, kBigTC, 4>(a, tid, u0, u1, &s_last);
}

// ============================================================================ x rearrangement

// x [M, K] bf16 row-major -> MFMA B fragments. Chunk (b, mt, i, l) of 16 bytes
// holds x[mt*32 + l%32][32 b + 16 (l/32) + 8 i .. +7] at byte
// ((b * MT + mt) * 2 + i) * 1024 + l * 16; rows >= M are zero.
__global__ __launch_bounds__(256) void xfrag_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                    int MT, uint4* __restrict__ xf) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int total = (K / 32) * MT * 128;
  if (c >= total) return;
  const int l = c & 63, i = (c >> 6) & 1, bm = c >> 7;
  const int mt = bm % MT, b = bm / MT;
  const int m = mt * 32 + (l & 31);
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (m < M) v = *reinterpret_cast<const uint4*>(x + (int64_t)m * K + b * 32 + 16 * (l >> 5) + 8 * i);
  xf[c] = v;
}

// Certified head: x fragments as xfrag_kernel (blocks [0, fb)), and in the
// blocks after them one wavefront per row m < M computing ||x_m|| -- the
// squares summed in fp64 (exact for bf16) in a fixed order, the root rounded
// up to binary32.
__global__ __launch_bounds__(256) void cert_prep_kernel(const uint16_t* __restrict__ x, int M, int K, int MT,
                                                        uint4* __restrict__ xf, int fb, float* __restrict__ xnorm) {
  if ((int)blockIdx.x < fb) {
    const int c = blockIdx.x * 256 + threadIdx.x;
    const int total = (K / 32) * MT * 128;
    if (c >= total) return;
    const int l = c & 63, i = (c >> 6) & 1, bm = c >> 7;
    const int mt = bm % MT, b = bm / MT;
    const int m = mt * 32 + (l & 31);
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (m < M) v = *reinterpret_cast<const uint4*>(x + (int64_t)m * K + b * 32 + 16 * (l >> 5) + 8 * i);
    xf[c] = v;
    return;
  }
  // one workgroup per row: every thread sums its 16-byte pieces, then a
  // fixed-order reduction over the workgroup
  __shared__ double part[256];
  const int m = (int)blockIdx.x - fb, tid = threadIdx.x;
  if (m >= M) return;
  const uint4* row = reinterpret_cast<const uint4*>(x + (int64_t)m * K);
  double acc = 0.0;
  for (int i = tid; i < K / 8; i += 256) {
    const uint4 v = row[i];
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double lo = (double)__uint_as_float(d[j] << 16), hi = (double)__uint_as_float(d[j] & 0xFFFF0000u);
      acc += lo * lo + hi * hi;
    }
  }
  part[tid] = acc;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) part[tid] += part[tid + o];
    __syncthreads();
  }
  if (tid == 0) {
    const double r = sqrt(part[0]) * (1.0 + 0x1p-40);
    float f = (float)r;
    if ((double)f < r) f = __uint_as_float(__float_as_uint(f) + 1u);
    xnorm[m] = f;
  }
}

// ============================================================================ dispatch

struct KernelSel {
  const void* fn;
  int mt;       // 32-row tiles of x fragments to prepare (0: none)
  int threads;  // workgroup size
};

// Units per slice (at 4 strips per tile) from which m <= 32 uses 4-strip
// tiles. Measured at 32 rows, per call with the x pre-pass, against 2-strip
// tiles: the 152064x5120 LM head (93 units per slice) 3% faster; Wgate|Wup
// 34816x5120 (21 units) 56.1-57.8 against 58.1-61.1 us; Wdown 5120x17408
// (10.6) 38.2 against 37.5 us and Wo 5120x6144 (3.75) 23.7 against 21.1 us
// slower with the pre-pass: their slices are shorter than a tile, so fewer,
// coarser units balance worse (short slices that read x row-major are the
// exception below).
constexpr int kNq4MinUnits = 16;

// Units per slice below which the one-tile (5-32 row) MFMA kernel reads x
// row-major instead of from the pre-pass's fragments (a row-major load
// touches 32 rows, so the longer the slice, the more that costs against the
// pre-pass's separate launch). Measured per call at 32 rows, bit-identical
// results, against the pre-pass: Wo 5120x6144 (7.5 units) 20.1-20.4 against
// 21.0-22.8 us; Wdown 5120x17408 on 4-strip tiles (10.6 units) 36.5 against
// 37.1 us (means of six trials); slower with longer slices: Wq|Wk|Wv
// 8192x5120 on 2-strip tiles (10 units) 20.2-20.5 against 19.8-20.2, Wgate|Wup
// (21 units) 59.4 against 56.8 and the LM head 214 against 195 us.
constexpr int kXDirectMaxUnits = 12;

// Short slices (at least this many units at 4 strips, fewer than
// kXDirectMaxUnits) also take 4-strip tiles: with x read row-major, each x
// load then serves four strips. Measured at 32 rows, per call, against 2-strip
// tiles: Wq|Wk|Wv 8192x5120 (5 units) 18.6-19.1 us against 19.9-20.2 with the
// x pre-pass; Wdown (10.6 units) as above; Wo 5120x6144 (3.75 units)
// 22.0-22.5 against 20.1-20.8, which stays on 2-strip tiles.
constexpr int kNq4ShortMinUnits = 4;

template <int EPI, bool QP>
KernelSel select_kernel(int M, int nq) {
  if (M > kSmallMaxRows) {
    switch ((M + 31) / 32) {
#define W12_BIG(MT) \
  case MT:          \
    return {reinterpret_cast<const void*>(&gemm_big8_kernel<MT, EPI, QP>), 0, kB8NT};
      W12_BIG(3) W12_BIG(4) W12_BIG(5) W12_BIG(6)
#undef W12_BIG
      default:
        return {nullptr, 0, 0};
    }
  }
  if (M >= kMfmaMinRows) {
    if (M <= 32)
      return nq == 4 ? KernelSel{reinterpret_cast<const void*>(&gemm_mfma_kernel<1, EPI, QP, 4>), 1, kNT}
                     : KernelSel{reinterpret_cast<const void*>(&gemm_mfma_kernel<1, EPI, QP, 2>), 1, kNT};
    return {reinterpret_cast<const void*>(&gemm_mfma_kernel<2, EPI, QP, 2>), 2, kNT};
  }
  static_assert(kMfmaMinRows <= 5, "the VALU path is instantiated for up to 4 rows");
  const int mv = M <= 1 ? 1 : M <= 2 ? 2 : 4;
  switch (mv) {
#define W12_VALU(MV) \
  case MV:           \
    return {reinterpret_cast<const void*>(&gemm_valu_kernel<MV, EPI, QP>), 0, kNT};
    W12_VALU(1) W12_VALU(2) W12_VALU(4)
#undef W12_VALU
    default:
      return {nullptr, 0, 0};
  }
}

}  // namespace

constexpr size_t kCounterBytes = size_t(4) << 18;              // u32 per tile, P <= 2^18
constexpr size_t kKeyBytes = kKeyRegionBytes;  // argmax keys
constexpr size_t kStateBytes = kCounterBytes + kKeyBytes + 256;                 // + done counter

GemmPlan plan_gemm(int64_t n, int64_t k, int64_t m, int num_cu, int max_nq) {
  GemmPlan pl{};
  const bool big = m > kSmallMaxRows;
  const int64_t S = n / kStrip, RK = k / kRecK;
  // Up to 32 rows, tiles of 4 strips when the slices stay long (each x
  // fragment then serves 4 strips, and tiles end half as often) or are short
  // enough for x to be read row-major; slices in between keep 2-strip tiles,
  // whose finer units balance the slices better.
  int nq = 2;
  if (!big && m >= kMfmaMinRows && m <= 32 && max_nq >= 4) {
    const int64_t U4 = ((S + 3) / 4) * RK;
    const int64_t G4 = U4 < num_cu ? U4 : num_cu;
    if (U4 >= (int64_t)kNq4MinUnits * G4 ||
        (U4 >= (int64_t)kNq4ShortMinUnits * G4 && U4 < (int64_t)kXDirectMaxUnits * G4))
      nq = 4;
  }
  const int64_t tc = big ? kBigTC : nq * kStrip;  // channels per tile of the kernel select_kernel picks
  const int64_t sp = tc / kStrip, P = (S + sp - 1) / sp;
  const int64_t mt = (!big && m >= kMfmaMinRows) ? (m + 31) / 32 : 0;
  const int64_t U = P * RK;
  // one workgroup per compute unit, every slice resident at once
  int64_t G = num_cu;
  if (G > U) G = U;
  if (G < 1) G = 1;
  pl.G = (int)G;
  pl.U = (int)U;
  pl.P = (int)P;
  pl.nq = nq;
  pl.xdirect = (!big && mt == 1 && U < (int64_t)kXDirectMaxUnits * G) ? 1 : 0;
  // The counter region has the same place and size for every shape (any
  // shape's tile counters, the argmax keys and the done counter), so a
  // workspace shared by calls of different shapes never holds old partial
  // sums where a later call expects zeroed counters.
  pl.off_cnt = 0;
  pl.off_keys = kCounterBytes;
  pl.off_done = kCounterBytes + kKeyBytes;
  pl.off_part = kStateBytes;
  const size_t part_bytes = (size_t)2 * G * m * tc * 4;
  pl.off_xf = (pl.off_part + part_bytes + 255) & ~size_t(255);
  pl.ws_bytes = pl.off_xf + (size_t)mt * 32 * k * 2;
  return pl;
}

int64_t plan_slice_channels(const GemmPlan& pl, int64_t k) {
  const int64_t RK = k / kRecK, per = ((int64_t)pl.U + pl.G - 1) / pl.G;
  const int64_t tiles = 1 + (per + RK - 2) / RK;  // a slice of `per` units starting at any record
  return tiles * pl.nq * kStrip;
}

hipError_t launch_cert_pass(const GemmParams& p, hipStream_t s) {
  const int mt = (p.M + 31) / 32;
  const int64_t chunks = (int64_t)(p.K / 32) * mt * 128;
  const int fb = (int)((chunks + 255) / 256);
  hipLaunchKernelGGL(cert_prep_kernel, dim3(fb + p.M), dim3(256), 0, s, p.x, p.M, p.K, mt, p.xf, fb,
                     const_cast<float*>(p.xnorm));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const void* fn = nullptr;
  if (mt == 1) {
    fn = p.nq == 4 ? reinterpret_cast<const void*>(&gemm_mfma_kernel<1, kEpiCert, false, 4, kFmtCert8>)
                   : reinterpret_cast<const void*>(&gemm_mfma_kernel<1, kEpiCert, false, 2, kFmtCert8>);
  } else if (mt == 2 && p.nq == 2) {
    fn = reinterpret_cast<const void*>(&gemm_mfma_kernel<2, kEpiCert, false, 2, kFmtCert8>);
  }
  if (!fn) return hipErrorInvalidValue;
  void* args[] = {const_cast<GemmParams*>(&p)};
  return hipLaunchKernel(fn, dim3(p.G), dim3(kNT), args, 0, s);
}

hipError_t launch_gemm(const GemmParams& p, int epi, bool qpass, hipStream_t s) {
  const KernelSel k = qpass ? (epi == kEpiY ? select_kernel<kEpiY, true>(p.M, p.nq) : select_kernel<kEpiArgmax, true>(p.M, p.nq))
                            : (epi == kEpiY ? select_kernel<kEpiY, false>(p.M, p.nq) : select_kernel<kEpiArgmax, false>(p.M, p.nq));
  if (!k.fn) return hipErrorInvalidValue;
  if (k.mt > 0 && !p.xdirect) {
    const int64_t chunks = (int64_t)(p.K / 32) * k.mt * 128;
    const int blocks = (int)((chunks + 255) / 256);
    hipLaunchKernelGGL(xfrag_kernel, dim3(blocks), dim3(256), 0, s, p.x, p.M, p.K, k.mt, p.xf);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  void* args[] = {const_cast<GemmParams*>(&p)};
  return hipLaunchKernel(k.fn, dim3(p.G), dim3(k.threads), args, 0, s);
}

}  // namespace w12
