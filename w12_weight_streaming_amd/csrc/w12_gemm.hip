// W12 verify GEMM and fused LM-head argmax (gfx950).
//
// What is computed ("SpecPilot ..." summary, section 4.1): the verify pass
// multiplies every target linear layer, restored from W12 records in
// registers, against the handful of draft-tree rows in one weight read; the
// split of the k reduction across workgroups runs in a fixed order, so the
// GEMM is deterministic. The LM head variant keeps the logits in registers
// and emits only the greedy token (section 1.1: the target's argmax).
//
// gfx950 design:
//  * A work unit is one record (256 k) of a 64-channel tile (a pair of
//    32-channel strips). Units run tile-major; workgroup g owns a contiguous
//    slice of them (stream-K). A tile that straddles slices is finished by
//    whichever contributor arrives last, summing the slices' partials in
//    slice order.
//  * Inside a workgroup, wave w handles subtiles t = w, w + NW, ... (32 k each)
//    of every unit, so the eight 1.5 KB pieces of a 12 KB record are read by
//    different waves with one 16-byte + one 8-byte load per lane.
//  * Each lane restores its 16 weights in registers (decode16), escapes are
//    patched through a per-wave LDS buffer, then:
//      m >= 16: bf16 MFMA 32x32x16; the lane's 16 weights are two A
//               fragments, x is the B operand (m = lane % 32);
//      m <  16: lanes own channels, fdot2 against x broadcast to the wave.
//  * Loads run two units ahead of the arithmetic (three register stages).
#include <utility>
#include <type_traits>

#include "w12_device.h"
#include "w12_internal.h"

namespace w12 {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1 with constant i, so
// register arrays indexed by i stay in registers even across barriers.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

constexpr int kRedStride = 68;                  // floats per 64-channel row (+4 pad)
constexpr int kSlotFloats = 32 * kRedStride;    // one 32-row x 64-channel slot
constexpr int kLdsFloats = 4 * kSlotFloats;     // 34816 B >= 8 waves x 4 KB patch

// Dispatch sends workgroup b to XCD b % 8. Renumber so that each XCD gets a
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
__device__ __forceinline__ int partial_slot(int g, int p, int U, int G, int RK) {
  return (p == chunk_begin(g, U, G) / RK) ? 2 * g : 2 * g + 1;
}

template <typename T>
__device__ __forceinline__ T stream_load(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
}

__device__ __forceinline__ float4 f4add(float4 a, float4 b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

// Final value of 4 consecutive channels (n .. n+3) of row m.
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
    // (value key, ~index): the max is the largest logit, lowest id on ties.
    unsigned long long best = 0;
    if (valid) {
      const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const unsigned long long key = ((unsigned long long)float_key(vv[i]) << 32) |
                                       (uint32_t)(0xFFFFFFFFu - (uint32_t)(n + i));
        best = key > best ? key : best;
      }
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) {
      const uint32_t lo = __shfl_xor((uint32_t)best, o, 64);
      const uint32_t hi = __shfl_xor((uint32_t)(best >> 32), o, 64);
      const unsigned long long w = ((unsigned long long)hi << 32) | lo;
      best = w > best ? w : best;
    }
    if ((tid & 15) == 0 && valid && best) atomicMax(&a.keys[m], best);
  }
}

// Last contributor of a split tile sums the partials in slice order.
template <int EPI>
__device__ __forceinline__ void finish_split_tile(const GemmParams& a, int p, int tid, int nthreads,
                                                  int* s_last) {
  __threadfence();
  __syncthreads();
  const int gf = owner_of(p * a.RK, a.U, a.G);
  const int gl = owner_of((p + 1) * a.RK - 1, a.U, a.G);
  if (tid == 0) {
    const uint32_t old = atomicAdd(&a.tile_cnt[p], 1u);
    *s_last = (old == (uint32_t)(gl - gf)) ? 1 : 0;
  }
  __syncthreads();
  if (*s_last) {
    __threadfence();
    for (int e = tid; e < a.M * 16; e += nthreads) {
      const int m = e >> 4, c4 = (e & 15) * 4;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int gg = gf; gg <= gl; ++gg) {
        const int sl = partial_slot(gg, p, a.U, a.G, a.RK);
        v = f4add(v, *reinterpret_cast<const float4*>(a.part + ((int64_t)sl * a.M + m) * 64 + c4));
      }
      emit4<EPI>(a, tid, m, p * 64 + c4, v);
    }
    if (tid == 0) atomicExch(&a.tile_cnt[p], 0u);
  }
  __syncthreads();
}

// After the whole grid is done, the last workgroup turns keys into ids.
template <int EPI>
__device__ __forceinline__ void finish_grid(const GemmParams& a, int tid, int nthreads, int* s_last) {
  if constexpr (EPI == kEpiArgmax) {
    __threadfence();
    __syncthreads();
    if (tid == 0) *s_last = (atomicAdd(a.done, 1u) == (uint32_t)(a.G - 1)) ? 1 : 0;
    __syncthreads();
    if (*s_last) {
      __threadfence();
      for (int m = tid; m < a.M; m += nthreads) {
        const unsigned long long k = atomicExch(&a.keys[m], 0ull);
        a.idx[m] = (int32_t)(0xFFFFFFFFu - (uint32_t)k);
        if (a.maxval) a.maxval[m] = key_float((uint32_t)(k >> 32));
      }
      if (tid == 0) atomicExch(a.done, 0u);
    }
  }
}

// Escape offsets of the units [wbase, wbase + 64) held one unit per lane.
template <int TPW, int NW>
__device__ __forceinline__ void load_offsets(const GemmParams& a, int wbase, int u1, int wave,
                                             int lane, uint32_t (&off)[TPW][4]) {
  const int u = wbase + lane;
#pragma unroll
  for (int i = 0; i < TPW; ++i) off[i][0] = off[i][1] = off[i][2] = off[i][3] = 0;
  if (u < u1) {
    const int p = u / a.RK, r = u - p * a.RK;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = wave + NW * i;
      const int64_t b0 = ((int64_t)(2 * p) * a.RK + r) * 8 + t;
      off[i][0] = a.w.esc_off[b0];
      off[i][1] = a.w.esc_off[b0 + 1];
      if (2 * p + 1 < a.S) {
        const int64_t b1 = b0 + (int64_t)a.RK * 8;
        off[i][2] = a.w.esc_off[b1];
        off[i][3] = a.w.esc_off[b1 + 1];
      }
    }
  }
}

__device__ __forceinline__ void patch_entry(uint32_t* buf, uint32_t e, int owner_base) {
  const uint32_t kk = esc_kk(e);
  reinterpret_cast<uint16_t*>(buf + (owner_base + esc_c(e) + ((kk >> 4) << 5)) * 8)[kk & 15u] =
      esc_bits(e);
}

// ============================================================================ MFMA path (m >= 16)

template <int TPW, int XS>
struct StageM {
  u32x4 hi[TPW][2];
  u32x2 lo[TPW][2];
  uint32_t e[TPW][2];
  int cnt[TPW][2];
  uint32_t eb[TPW][2];
  uint32_t bias[2];
  u32x4 xv[TPW][XS > 0 ? XS : 1][2];
};

template <int MT, int NW, int EPI>
__global__ __launch_bounds__(NW * 64) void gemm_mfma_kernel(GemmParams a) {
  constexpr int TPW = 8 / NW;
  constexpr int XS = MT <= 2 ? MT : 0;
  constexpr int NT = NW * 64;
  __shared__ __align__(16) float lds[kLdsFloats];
  __shared__ int s_last;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = logical_wg(blockIdx.x, a.G);
  const int u0 = chunk_begin(g, a.U, a.G), u1 = chunk_begin(g + 1, a.U, a.G);
  const int RK = a.RK;
  uint32_t* patch = reinterpret_cast<uint32_t*>(lds) + wave * (TPW * 1024);

  f32x16 acc[2][MT];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[q][mt][i] = 0.f;

  uint32_t off[TPW][4];
  int wbase = u0;
  load_offsets<TPW, NW>(a, wbase, u1, wave, lane, off);

  // ---- loads for one unit
  int nl = u0, lp = u0 / RK, lr = u0 - (u0 / RK) * RK;
  auto load_next = [&](StageM<TPW, XS>& st) __attribute__((always_inline)) {
    if (nl < u1) {
      if (nl - wbase >= 64) {
        wbase = nl;
        load_offsets<TPW, NW>(a, wbase, u1, wave, lane, off);
      }
      const int li = nl - wbase;
      const bool has1 = 2 * lp + 1 < a.S;
      const uint8_t* rb0 = a.w.rec + ((int64_t)(2 * lp) * RK + lr) * kRecBytes;
      const uint8_t* rb1 = rb0 + (int64_t)RK * kRecBytes;
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int t = wave + NW * i;
        st.hi[i][0] = stream_load<u32x4>(rb0 + t * 1024 + lane * 16);
        st.lo[i][0] = stream_load<u32x2>(rb0 + kHiBytes + t * 512 + lane * 8);
        if (has1) {
          st.hi[i][1] = stream_load<u32x4>(rb1 + t * 1024 + lane * 16);
          st.lo[i][1] = stream_load<u32x2>(rb1 + kHiBytes + t * 512 + lane * 8);
        } else {
          st.hi[i][1] = u32x4{0, 0, 0, 0};
          st.lo[i][1] = u32x2{0, 0};
        }
        const uint32_t o0 = __builtin_amdgcn_readlane(off[i][0], li);
        const uint32_t e0 = __builtin_amdgcn_readlane(off[i][1], li);
        const uint32_t o1 = __builtin_amdgcn_readlane(off[i][2], li);
        const uint32_t e1 = __builtin_amdgcn_readlane(off[i][3], li);
        st.cnt[i][0] = (int)(e0 - o0);
        st.cnt[i][1] = (int)(e1 - o1);
        st.eb[i][0] = o0;
        st.eb[i][1] = o1;
        st.e[i][0] = lane < (int)(e0 - o0) ? a.w.esc[o0 + lane] : 0u;
        st.e[i][1] = lane < (int)(e1 - o1) ? a.w.esc[o1 + lane] : 0u;
        if constexpr (XS > 0) {
          const int k0 = lr * kRecK + t * kSubK + 16 * (lane >> 5);
#pragma unroll
          for (int mt = 0; mt < XS; ++mt) {
            const int m = mt * 32 + (lane & 31);
            if (m < a.M) {
              const u32x4* xp = reinterpret_cast<const u32x4*>(a.x + (int64_t)m * a.K + k0);
              st.xv[i][mt][0] = xp[0];
              st.xv[i][mt][1] = xp[1];
            } else {
              st.xv[i][mt][0] = u32x4{0, 0, 0, 0};
              st.xv[i][mt][1] = u32x4{0, 0, 0, 0};
            }
          }
        }
      }
      const int n = lp * 64 + (lane & 31);
      st.bias[0] = bias2_of(a.w.e_top[n]);
      st.bias[1] = has1 ? bias2_of(a.w.e_top[n + 32]) : 0u;
    }
    ++nl;
    if (++lr == RK) { lr = 0; ++lp; }
  };

  // ---- tile flush: reduce the waves' accumulators, write or hand off
  auto flush = [&](int p) __attribute__((always_inline)) {
    const bool whole = p * RK >= u0 && (p + 1) * RK <= u1;
    const int slot = partial_slot(g, p, a.U, a.G, RK);
    static_for<MT>([&](auto mtc) {
      constexpr int mt = decltype(mtc)::value;
      auto put = [&](float* dst, bool add) __attribute__((always_inline)) {
        const int ml = lane & 31, hf = lane >> 5;
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int rb = 0; rb < 4; ++rb) {
            float4* d = reinterpret_cast<float4*>(dst + ml * kRedStride + 32 * q + 8 * rb + 4 * hf);
            float4 v = make_float4(acc[q][mt][4 * rb], acc[q][mt][4 * rb + 1],
                                   acc[q][mt][4 * rb + 2], acc[q][mt][4 * rb + 3]);
            if (add) v = f4add(*d, v);
            *d = v;
          }
      };
      __syncthreads();
      if constexpr (NW == 8) {
        if (wave >= 4) put(lds + (wave - 4) * kSlotFloats, false);
        __syncthreads();
        if (wave < 4) put(lds + wave * kSlotFloats, true);
      } else {
        put(lds + wave * kSlotFloats, false);
      }
      __syncthreads();
      for (int e = tid; e < 32 * 16; e += NT) {
        const int ml = e >> 4, c4 = (e & 15) * 4;
        const float* b = lds + ml * kRedStride + c4;
        const float4 v = f4add(f4add(*reinterpret_cast<const float4*>(b),
                                     *reinterpret_cast<const float4*>(b + kSlotFloats)),
                               f4add(*reinterpret_cast<const float4*>(b + 2 * kSlotFloats),
                                     *reinterpret_cast<const float4*>(b + 3 * kSlotFloats)));
        const int m = mt * 32 + ml;
        if (whole) {
          emit4<EPI>(a, tid, m, p * 64 + c4, v);
        } else if (m < a.M) {
          *reinterpret_cast<float4*>(a.part + ((int64_t)slot * a.M + m) * 64 + c4) = v;
        }
      }
    });
    __syncthreads();
    if (!whole) finish_split_tile<EPI>(a, p, tid, NT, &s_last);
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[q][mt][i] = 0.f;
  };

  // ---- arithmetic for one unit
  int cp = u0 / RK, cr = u0 - (u0 / RK) * RK, tile = cp;
  auto step = [&](const StageM<TPW, XS>& st) __attribute__((always_inline)) {
    if (cp != tile) {
      flush(tile);
      tile = cp;
    }
    const bool has1 = 2 * cp + 1 < a.S;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      uint32_t P[2][8];
      decode16(uint4{st.hi[i][0].x, st.hi[i][0].y, st.hi[i][0].z, st.hi[i][0].w},
               uint2{st.lo[i][0].x, st.lo[i][0].y}, st.bias[0], P[0]);
      decode16(uint4{st.hi[i][1].x, st.hi[i][1].y, st.hi[i][1].z, st.hi[i][1].w},
               uint2{st.lo[i][1].x, st.lo[i][1].y}, st.bias[1], P[1]);
      if (st.cnt[i][0] + st.cnt[i][1] > 0) {
        uint32_t* wb = patch + i * 1024;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          *reinterpret_cast<uint4*>(wb + q * 512 + lane * 8) = make_uint4(P[q][0], P[q][1], P[q][2], P[q][3]);
          *reinterpret_cast<uint4*>(wb + q * 512 + lane * 8 + 4) = make_uint4(P[q][4], P[q][5], P[q][6], P[q][7]);
        }
        wave_lds_sync();
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          if (lane < st.cnt[i][q]) patch_entry(wb, st.e[i][q], q * 64);
          for (int j = 64 + lane; j < st.cnt[i][q]; j += 64)
            patch_entry(wb, a.w.esc[st.eb[i][q] + j], q * 64);
        }
        wave_lds_sync();
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const uint4 r0 = *reinterpret_cast<const uint4*>(wb + q * 512 + lane * 8);
          const uint4 r1 = *reinterpret_cast<const uint4*>(wb + q * 512 + lane * 8 + 4);
          P[q][0] = r0.x; P[q][1] = r0.y; P[q][2] = r0.z; P[q][3] = r0.w;
          P[q][4] = r1.x; P[q][5] = r1.y; P[q][6] = r1.z; P[q][7] = r1.w;
        }
      }
      const int t = wave + NW * i;
      const int k0 = cr * kRecK + t * kSubK + 16 * (lane >> 5);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        u32x4 x0, x1;
        if constexpr (XS > 0) {
          x0 = st.xv[i][mt < XS ? mt : 0][0];
          x1 = st.xv[i][mt < XS ? mt : 0][1];
        } else {
          const int m = mt * 32 + (lane & 31);
          if (m < a.M) {
            const u32x4* xp = reinterpret_cast<const u32x4*>(a.x + (int64_t)m * a.K + k0);
            x0 = xp[0];
            x1 = xp[1];
          } else {
            x0 = u32x4{0, 0, 0, 0};
            x1 = u32x4{0, 0, 0, 0};
          }
        }
        const bf16x8 b0 = __builtin_bit_cast(bf16x8, x0);
        const bf16x8 b1 = __builtin_bit_cast(bf16x8, x1);
        const bf16x8 a00 = __builtin_bit_cast(bf16x8, u32x4{P[0][0], P[0][1], P[0][2], P[0][3]});
        const bf16x8 a01 = __builtin_bit_cast(bf16x8, u32x4{P[0][4], P[0][5], P[0][6], P[0][7]});
        acc[0][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a00, b0, acc[0][mt], 0, 0, 0);
        acc[0][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a01, b1, acc[0][mt], 0, 0, 0);
        if (has1) {
          const bf16x8 a10 = __builtin_bit_cast(bf16x8, u32x4{P[1][0], P[1][1], P[1][2], P[1][3]});
          const bf16x8 a11 = __builtin_bit_cast(bf16x8, u32x4{P[1][4], P[1][5], P[1][6], P[1][7]});
          acc[1][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a10, b0, acc[1][mt], 0, 0, 0);
          acc[1][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a11, b1, acc[1][mt], 0, 0, 0);
        }
      }
    }
    if (++cr == RK) { cr = 0; ++cp; }
  };

  if (u0 < u1) {
    StageM<TPW, XS> sA, sB, sC;
    load_next(sA);
    load_next(sB);
    for (int u = u0; u < u1; u += 3) {
      load_next(sC);
      step(sA);
      if (u + 1 >= u1) break;
      load_next(sA);
      step(sB);
      if (u + 2 >= u1) break;
      load_next(sB);
      step(sC);
    }
    flush(tile);
  }
  finish_grid<EPI>(a, tid, NT, &s_last);
}

// ============================================================================ VALU path (m < 16)

template <int XV>
struct StageV {
  u32x4 hi[2];       // [h]: k-half of the subtile; lane = channel of the tile
  u32x2 lo[2];
  uint32_t e[2];     // [q]: strip of the pair
  int cnt[2];
  uint32_t eb[2];
  uint32_t bias;
  u32x4 xv[2][XV > 0 ? XV : 1][2];
};

template <int MV, int EPI>
__global__ __launch_bounds__(512) void gemm_valu_kernel(GemmParams a) {
  constexpr int NW = 8, NT = 512;
  constexpr int XV = MV <= 2 ? MV : 0;
  __shared__ __align__(16) float lds[kLdsFloats];
  __shared__ int s_last;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, t = wave;
  const int q = lane >> 5, c = lane & 31;
  const int g = logical_wg(blockIdx.x, a.G);
  const int u0 = chunk_begin(g, a.U, a.G), u1 = chunk_begin(g + 1, a.U, a.G);
  const int RK = a.RK;
  uint32_t* patch = reinterpret_cast<uint32_t*>(lds) + wave * 1024;

  float acc[MV];
#pragma unroll
  for (int m = 0; m < MV; ++m) acc[m] = 0.f;

  uint32_t off[1][4];
  int wbase = u0;
  load_offsets<1, NW>(a, wbase, u1, wave, lane, off);

  int nl = u0, lp = u0 / RK, lr = u0 - (u0 / RK) * RK;
  auto load_next = [&](StageV<XV>& st) __attribute__((always_inline)) {
    if (nl < u1) {
      if (nl - wbase >= 64) {
        wbase = nl;
        load_offsets<1, NW>(a, wbase, u1, wave, lane, off);
      }
      const int li = nl - wbase;
      const bool mine = 2 * lp + q < a.S;
      const uint8_t* rb = a.w.rec + ((int64_t)(2 * lp + q) * RK + lr) * kRecBytes;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (mine) {
          st.hi[h] = stream_load<u32x4>(rb + t * 1024 + (c + 32 * h) * 16);
          st.lo[h] = stream_load<u32x2>(rb + kHiBytes + t * 512 + (c + 32 * h) * 8);
        } else {
          st.hi[h] = u32x4{0, 0, 0, 0};
          st.lo[h] = u32x2{0, 0};
        }
      }
      const uint32_t o0 = __builtin_amdgcn_readlane(off[0][0], li);
      const uint32_t e0 = __builtin_amdgcn_readlane(off[0][1], li);
      const uint32_t o1 = __builtin_amdgcn_readlane(off[0][2], li);
      const uint32_t e1 = __builtin_amdgcn_readlane(off[0][3], li);
      st.cnt[0] = (int)(e0 - o0);
      st.cnt[1] = (int)(e1 - o1);
      st.eb[0] = o0;
      st.eb[1] = o1;
      st.e[0] = lane < (int)(e0 - o0) ? a.w.esc[o0 + lane] : 0u;
      st.e[1] = lane < (int)(e1 - o1) ? a.w.esc[o1 + lane] : 0u;
      st.bias = mine ? bias2_of(a.w.e_top[lp * 64 + lane]) : 0u;
      if constexpr (XV > 0) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int m = 0; m < XV; ++m) {
            const u32x4* xp = reinterpret_cast<const u32x4*>(
                a.x + (int64_t)m * a.K + lr * kRecK + t * kSubK + 16 * h);
            st.xv[h][m][0] = xp[0];
            st.xv[h][m][1] = xp[1];
          }
      }
    }
    ++nl;
    if (++lr == RK) { lr = 0; ++lp; }
  };

  auto flush = [&](int p) __attribute__((always_inline)) {
    const bool whole = p * RK >= u0 && (p + 1) * RK <= u1;
    const int slot = partial_slot(g, p, a.U, a.G, RK);
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MV; ++m) lds[(wave * MV + m) * 64 + lane] = acc[m];
    __syncthreads();
    for (int e = tid; e < MV * 16; e += NT) {
      const int m = e >> 4, c4 = (e & 15) * 4;
      float4 v = *reinterpret_cast<const float4*>(lds + m * 64 + c4);
#pragma unroll
      for (int w = 1; w < NW; ++w)
        v = f4add(v, *reinterpret_cast<const float4*>(lds + (w * MV + m) * 64 + c4));
      if (whole) {
        emit4<EPI>(a, tid, m, p * 64 + c4, v);
      } else {
        *reinterpret_cast<float4*>(a.part + ((int64_t)slot * a.M + m) * 64 + c4) = v;
      }
    }
    __syncthreads();
    if (!whole) finish_split_tile<EPI>(a, p, tid, NT, &s_last);
#pragma unroll
    for (int m = 0; m < MV; ++m) acc[m] = 0.f;
  };

  int cp = u0 / RK, cr = u0 - (u0 / RK) * RK, tile = cp;
  auto step = [&](const StageV<XV>& st) __attribute__((always_inline)) {
    if (cp != tile) {
      flush(tile);
      tile = cp;
    }
    uint32_t P[2][8];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      decode16(uint4{st.hi[h].x, st.hi[h].y, st.hi[h].z, st.hi[h].w},
               uint2{st.lo[h].x, st.lo[h].y}, st.bias, P[h]);
    if (st.cnt[0] + st.cnt[1] > 0) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        *reinterpret_cast<uint4*>(patch + h * 512 + lane * 8) = make_uint4(P[h][0], P[h][1], P[h][2], P[h][3]);
        *reinterpret_cast<uint4*>(patch + h * 512 + lane * 8 + 4) = make_uint4(P[h][4], P[h][5], P[h][6], P[h][7]);
      }
      wave_lds_sync();
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        auto put = [&](uint32_t e) __attribute__((always_inline)) {
          const uint32_t kk = esc_kk(e);
          reinterpret_cast<uint16_t*>(patch + (kk >> 4) * 512 + (32 * qq + esc_c(e)) * 8)[kk & 15u] =
              esc_bits(e);
        };
        if (lane < st.cnt[qq]) put(st.e[qq]);
        for (int j = 64 + lane; j < st.cnt[qq]; j += 64) put(a.w.esc[st.eb[qq] + j]);
      }
      wave_lds_sync();
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint4 r0 = *reinterpret_cast<const uint4*>(patch + h * 512 + lane * 8);
        const uint4 r1 = *reinterpret_cast<const uint4*>(patch + h * 512 + lane * 8 + 4);
        P[h][0] = r0.x; P[h][1] = r0.y; P[h][2] = r0.z; P[h][3] = r0.w;
        P[h][4] = r1.x; P[h][5] = r1.y; P[h][6] = r1.z; P[h][7] = r1.w;
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int m = 0; m < MV; ++m) {
        u32x4 x0, x1;
        if constexpr (XV > 0) {
          x0 = st.xv[h][m < XV ? m : 0][0];
          x1 = st.xv[h][m < XV ? m : 0][1];
        } else {
          const u32x4* xp = reinterpret_cast<const u32x4*>(
              a.x + (int64_t)m * a.K + cr * kRecK + t * kSubK + 16 * h);
          x0 = xp[0];
          x1 = xp[1];
        }
        const uint32_t xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        float s = acc[m];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, P[h][i]),
                                              __builtin_bit_cast(bf16x2, xs[i]), s, false);
        acc[m] = s;
      }
    }
    if (++cr == RK) { cr = 0; ++cp; }
  };

  if (u0 < u1) {
    StageV<XV> sA, sB, sC;
    load_next(sA);
    load_next(sB);
    for (int u = u0; u < u1; u += 3) {
      load_next(sC);
      step(sA);
      if (u + 1 >= u1) break;
      load_next(sA);
      step(sB);
      if (u + 2 >= u1) break;
      load_next(sB);
      step(sC);
    }
    flush(tile);
  }
  finish_grid<EPI>(a, tid, NT, &s_last);
}

// ============================================================================ dispatch

template <int EPI>
hipError_t launch_mfma(const GemmParams& p, hipStream_t s) {
  const int mt = (p.M + 31) / 32;
  dim3 grid(p.G);
#define W12_MFMA(MT, NW)                                                                     \
  case MT:                                                                                   \
    hipLaunchKernelGGL((gemm_mfma_kernel<MT, NW, EPI>), grid, dim3(NW * 64), 0, s, p); \
    break;
  switch (mt) {
    W12_MFMA(1, 8)
    W12_MFMA(2, 8)
    W12_MFMA(3, 8)
    W12_MFMA(4, 8)
    W12_MFMA(5, 4)
    W12_MFMA(6, 4)
    W12_MFMA(7, 4)
    W12_MFMA(8, 4)
    default:
      return hipErrorInvalidValue;
  }
#undef W12_MFMA
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_valu(const GemmParams& p, hipStream_t s) {
  dim3 grid(p.G);
#define W12_VALU(MV) \
  case MV:           \
    hipLaunchKernelGGL((gemm_valu_kernel<MV, EPI>), grid, dim3(512), 0, s, p); \
    break;
  switch (p.M) {
    W12_VALU(1) W12_VALU(2) W12_VALU(3) W12_VALU(4) W12_VALU(5)
    W12_VALU(6) W12_VALU(7) W12_VALU(8) W12_VALU(9) W12_VALU(10)
    W12_VALU(11) W12_VALU(12) W12_VALU(13) W12_VALU(14) W12_VALU(15)
    default:
      return hipErrorInvalidValue;
  }
#undef W12_VALU
  return hipGetLastError();
}

}  // namespace

constexpr int kMfmaMinRows = 16;
constexpr size_t kCounterBytes = size_t(4) << 18;            // u32 per tile, P <= 2^18
constexpr size_t kStateBytes = kCounterBytes + 256 * 8 + 256;  // + keys + done, aligned

GemmPlan plan_gemm(int64_t n, int64_t k, int64_t m, int num_cu) {
  GemmPlan pl{};
  const int64_t S = n / kStrip, P = (S + 1) / 2, RK = k / kRecK, U = P * RK;
  const int per_cu = 2;
  int64_t G = (int64_t)num_cu * per_cu;
  if (G > U) G = U;
  if (G < 1) G = 1;
  pl.G = (int)G;
  // The counter region has the same place and size for every shape: any
  // shape's tile counters (P <= 2^18 because N*K < 2^32 and K >= 256), the
  // argmax keys (m <= 256) and the done counter. Partial sums always start
  // after it, so a workspace shared by calls of different shapes never has
  // old partial sums where a later call expects zeroed counters.
  (void)P;
  pl.off_cnt = 0;
  pl.off_keys = kCounterBytes;
  pl.off_done = kCounterBytes + 256 * 8;
  pl.off_part = kStateBytes;
  pl.ws_bytes = kStateBytes + (size_t)2 * G * m * 64 * 4;
  return pl;
}

hipError_t launch_gemm(const GemmParams& p, int epi, hipStream_t s) {
  if (p.M >= kMfmaMinRows)
    return epi == kEpiY ? launch_mfma<kEpiY>(p, s) : launch_mfma<kEpiArgmax>(p, s);
  return epi == kEpiY ? launch_valu<kEpiY>(p, s) : launch_valu<kEpiArgmax>(p, s);
}

}  // namespace w12
