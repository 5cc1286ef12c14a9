// Certified INT8 LM head (gfx950): the INT8 copy, and the exact rescoring of
// the vocabulary rows the bound cannot rule out.
//
// "SpecPilot ..." summary, section 4.1 (LM-head paragraph): the head keeps
// an INT8 copy; a per-row Cauchy-Schwarz error bound proves which tokens
// cannot be the argmax; only the survivors are rescored exactly, so the
// argmax never changes. Readings taken where the pages leave it open:
//  * copy: per vocabulary row and 32-k block, the weights W12 keeps in its
//    window become q = RNE(w / 2^s), s the smallest integer with every such
//    |w| <= 127 * 2^s (q * 2^s is exact in bf16); W12's escapes are q = 0
//    and come back exactly from W12's escape list;
//  * bound constant per row: c = ||e|| + 2 K 2^-24 ||w'|| (e = w - w', w'
//    the copy's weights), summed in fp64 in a fixed order and rounded up to
//    binary32;
//  * the INT8 pass (w12_gemm.hip) gives A = x.w' in fp32, per-row lower
//    bounds LB = max (A - B) and per 4-row group upper bounds U = A + B
//    (B = ||x|| c + 1e-6, both rounded outward); the rescoring below takes
//    every group with U >= LB for some row and computes those rows' exact
//    logits from the W12 records, fp32 accumulation, lowest id on ties.
#include "w12_device.h"
#include "w12_internal.h"

namespace w12 {
namespace {

constexpr int kCertBlock = 32;
constexpr int kCodeBias = 133;  // stored code = s + 133; 0: block without window weights

__device__ __forceinline__ uint32_t in_window_bits(uint32_t b, uint32_t top) {
  const uint32_t e = (b >> 7) & 0xFFu;
  return (uint32_t)(e >= 1u) & (uint32_t)(e <= 254u) & (uint32_t)(e + 15u >= top) & (uint32_t)(e <= top);
}

// q = RNE(|w| / 2^s) for a window weight of block code `code` (s = code -
// 133): |w| = (128 + m) 2^(e - 134), so |w| / 2^s = (128 + m) 2^-(code + 1 - e).
__device__ __forceinline__ int quantise(uint32_t b, uint32_t code) {
  const uint32_t e = (b >> 7) & 0xFFu, mant = 128u + (b & 0x7Fu);
  const uint32_t sh = code + 1u - e;  // >= 1 for every window weight of the block
  uint32_t q = 0;
  if (sh < 9u) {
    const uint32_t half = 1u << (sh - 1u);
    const uint32_t rest = mant & ((1u << sh) - 1u);
    q = mant >> sh;
    if (rest > half || (rest == half && (q & 1u))) ++q;
  }
  return (b & 0x8000u) ? -(int)q : (int)q;
}

__device__ __forceinline__ double bf16_value(uint32_t b) { return (double)__uint_as_float(b << 16); }

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// One wavefront per vocabulary row v. Lane L takes the row's 32-k blocks
// j = L, L + 64, ...: builds the block code and the 32 codes q, writes them
// where the record layout puts them, and sums e^2 and w'^2 in fp64.
__global__ __launch_bounds__(256) void cert_pack_kernel(const uint16_t* __restrict__ w, int64_t N, int64_t K,
                                                        const uint8_t* __restrict__ e_top,
                                                        int8_t* __restrict__ q_out, uint8_t* __restrict__ code_out,
                                                        float* __restrict__ cbound) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t v = (int64_t)blockIdx.x * 4 + wave;
  if (v >= N) return;
  const int64_t RK = K / kRecK, s = v / kStrip;
  const int c = (int)(v % kStrip);
  const uint32_t top = e_top[v];
  double se = 0.0, sw = 0.0;
  for (int64_t j = lane; j < K / kCertBlock; j += 64) {
    const uint4* src = reinterpret_cast<const uint4*>(w + v * K + j * kCertBlock);
    uint32_t b[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 d = src[i];
      const uint32_t dd[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        b[8 * i + 2 * h] = dd[h] & 0xFFFFu;
        b[8 * i + 2 * h + 1] = dd[h] >> 16;
      }
    }
    // largest magnitude among the window weights (finite and normal, so the
    // bit patterns order like the values)
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t mag = in_window_bits(b[i], top) ? (b[i] & 0x7FFFu) : 0u;
      amax = mag > amax ? mag : amax;
    }
    // smallest s with amax <= 127 * 2^s: code = s + 133 is the exponent
    // field of amax, plus one when its 8-bit significand is 255
    const uint32_t code = amax ? ((amax >> 7) + ((amax & 0x7Fu) == 0x7Fu ? 1u : 0u)) : 0u;
    uint32_t qb[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const double wv = bf16_value(b[i]);
      double wq = wv;
      if (in_window_bits(b[i], top)) {
        const int q = quantise(b[i], code);
        qb[i >> 2] |= ((uint32_t)q & 0xFFu) << (8 * (i & 3));
        wq = ldexp((double)q, (int)code - kCodeBias);
      }
      const double e = wv - wq;
      se += e * e;
      sw += wq * wq;
    }
    const int64_t r = j / 8, t = j % 8;
    int8_t* rec = q_out + (s * RK + r) * 8192 + t * 1024;
    *reinterpret_cast<uint4*>(rec + c * 16) = make_uint4(qb[0], qb[1], qb[2], qb[3]);
    *reinterpret_cast<uint4*>(rec + (c + 32) * 16) = make_uint4(qb[4], qb[5], qb[6], qb[7]);
    code_out[((s * RK + r) * 8 + t) * 32 + c] = (uint8_t)code;
  }
  se = wave_sum_f64(se);
  sw = wave_sum_f64(sw);
  if (lane == 0) {
    const double cv = sqrt(se) + 2.0 * (double)K * 0x1p-24 * sqrt(sw);
    float f = (float)cv;
    if ((double)f < cv) f = __uint_as_float(__float_as_uint(f) + 1u);  // positive: next float up
    cbound[v] = f;
  }
}

// Argmax keys in the GEMM kernels' layout (kKeyCopies x kKeyRows x
// kKeyStride u64, copy blockIdx.x % kKeyCopies).
constexpr int kGroupsPerWave = 16;
constexpr int kRecUnroll = 5;  // records a lane has in flight in the rescoring

template <int CTRL>
__device__ __forceinline__ float add_dpp(float v) {
  const int o = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false);
  return v + __int_as_float(o);
}
// Sum over the 16 lanes of a DPP row, in one fixed order; every lane of the
// row ends with the same value.
__device__ __forceinline__ float row16_sum(float v) {
  v = add_dpp<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v = add_dpp<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v = add_dpp<0x141>(v);  // row_half_mirror
  return add_dpp<0x140>(v);  // row_mirror
}
__device__ __forceinline__ unsigned long long umax64(unsigned long long a, unsigned long long b) { return a > b ? a : b; }

// Selection. Wave w of workgroup b looks at the 16 consecutive groups of 4
// vocabulary rows from group (4 b + w) * 16. Lane m < M holds row m's lower
// bound LB_m (the maximum over the 8 key copies of the INT8 pass). Every
// (group, row m) whose upper bound U[group][m] reaches LB_m goes to the list.
__global__ __launch_bounds__(256) void cert_select_kernel(CertRescoreArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ngroups = (int)(a.w.n / 4);
  float lb = __builtin_huge_valf();  // rows >= M never survive
  if (lane < a.M) {
    unsigned long long k = 0;
#pragma unroll
    for (int x = 0; x < kKeyCopies; ++x) k = umax64(k, a.lb_keys[(x * kKeyRows + lane) * kKeyStride]);
    lb = k ? key_float((uint32_t)(k >> 32)) : -__builtin_huge_valf();
  }
  const int g0 = (blockIdx.x * 4 + wave) * kGroupsPerWave;
  float u[kGroupsPerWave];
#pragma unroll
  for (int i = 0; i < kGroupsPerWave; ++i)
    u[i] = (lane < a.M && g0 + i < ngroups) ? a.u4[(size_t)(g0 + i) * kCertMaxRows + lane] : -__builtin_huge_valf();
#pragma unroll
  for (int i = 0; i < kGroupsPerWave; ++i) {
    if (u[i] >= lb) {
      const uint32_t slot = atomicAdd(a.list_count, 1u);
      a.list[slot] = make_uint2((uint32_t)(g0 + i), (uint32_t)lane);
    }
  }
}

// The exact rescoring of the listed (group, row) pairs. Workgroup b takes
// entries b, b + grid, ...; wave c takes vocabulary row 4 g + c of the
// entry's group; lane L = 16 rq + 2 t + h restores the 16 weights (subtile
// t, half h) of records rq, rq + 4, ... with the GEMM's restore and escape
// patch (5 records in flight), dots them with the input row in fp32, and the
// wave sums its 64 lanes in a fixed order. The key (value key, ~id) goes to
// an atomic maximum per row; the last workgroup turns the keys into ids and
// clears every key, count and counter.
__global__ __launch_bounds__(256) void cert_rescore_kernel(CertRescoreArgs a) {
  __shared__ __align__(16) uint32_t pbuf[256 * kRecUnroll * 8];
  __shared__ int s_last;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int rq = lane >> 4, t = (lane >> 1) & 7, h = lane & 1;
  const int RK = a.K / kRecK;
  const uint32_t n_esc = a.w.esc_off[a.w.nb];
  const uint32_t count = *a.list_count;
  uint32_t* my = pbuf + tid * kRecUnroll * 8;

  for (uint32_t i = blockIdx.x; i < count; i += gridDim.x) {
    const uint2 ent = a.list[i];
    const int g = (int)ent.x, m = (int)ent.y;
    const int v0 = 4 * g, s = v0 / kStrip, ch = v0 % kStrip + wave, v = v0 + wave;
    const uint32_t bias = bias2_of(a.w.e_top[v]);
    {
      float acc = 0.f;
      for (int r0 = 0; r0 < RK; r0 += 4 * kRecUnroll) {
        uint4 hi[kRecUnroll], x0[kRecUnroll], x1[kRecUnroll];
        uint2 lo[kRecUnroll];
        uint32_t o[kRecUnroll], cnt[kRecUnroll];
#pragma unroll
        for (int u = 0; u < kRecUnroll; ++u) {
          const int r = r0 + rq + 4 * u;
          hi[u] = make_uint4(0u, 0u, 0u, 0u);
          lo[u] = make_uint2(0u, 0u);
          x0[u] = x1[u] = make_uint4(0u, 0u, 0u, 0u);
          o[u] = 0u;
          cnt[u] = 0u;
          if (r < RK) {
            const uint8_t* rec = a.w.rec + ((int64_t)s * RK + r) * kRecBytes;
            hi[u] = *reinterpret_cast<const uint4*>(rec + t * 1024 + (ch + 32 * h) * 16);
            lo[u] = *reinterpret_cast<const uint2*>(rec + kHiBytes + t * 512 + (ch + 32 * h) * 8);
            const uint16_t* xr = a.x + (int64_t)m * a.K + (int64_t)r * kRecK + t * 32 + h * 16;
            x0[u] = *reinterpret_cast<const uint4*>(xr);
            x1[u] = *reinterpret_cast<const uint4*>(xr + 8);
            const int64_t b = ((int64_t)s * RK + r) * 8 + t;
            const uint32_t ob = a.w.esc_off[b], ob1 = a.w.esc_off[b + 1];
            o[u] = ob;
            cnt[u] = (ob <= ob1 && ob1 <= n_esc) ? min(ob1 - ob, 1024u) : 0u;
          }
        }
#pragma unroll
        for (int u = 0; u < kRecUnroll; ++u) {
          uint32_t P[8];
          decode16(hi[u], lo[u], bias, P);
          if (cnt[u]) {
            // only this thread touches its 32 bytes: no cross-lane ordering
            uint32_t* mu = my + u * 8;
            *reinterpret_cast<uint4*>(mu) = make_uint4(P[0], P[1], P[2], P[3]);
            *reinterpret_cast<uint4*>(mu + 4) = make_uint4(P[4], P[5], P[6], P[7]);
            for (uint32_t j0 = 0; j0 < cnt[u]; j0 += 8) {
              uint32_t e[8];
#pragma unroll
              for (int j = 0; j < 8; ++j) e[j] = (j0 + j < cnt[u]) ? a.w.esc[o[u] + j0 + j] : 0u;
#pragma unroll
              for (int j = 0; j < 8; ++j)
                if (j0 + j < cnt[u] && esc_c(e[j]) == (uint32_t)ch && (esc_kk(e[j]) >> 4) == (uint32_t)h)
                  reinterpret_cast<uint16_t*>(mu)[esc_kk(e[j]) & 15u] = esc_bits(e[j]);
            }
            const uint4 q0 = *reinterpret_cast<const uint4*>(mu), q1 = *reinterpret_cast<const uint4*>(mu + 4);
            P[0] = q0.x; P[1] = q0.y; P[2] = q0.z; P[3] = q0.w;
            P[4] = q1.x; P[5] = q1.y; P[6] = q1.z; P[7] = q1.w;
          }
          const uint32_t xs[8] = {x0[u].x, x0[u].y, x0[u].z, x0[u].w, x1[u].x, x1[u].y, x1[u].z, x1[u].w};
#pragma unroll
          for (int q = 0; q < 8; ++q)
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, P[q]), __builtin_bit_cast(bf16x2, xs[q]),
                                                  acc, false);
        }
      }
      // the wave's 64 lanes in one fixed order: rows of 16, then the 4 rows
      const float rs = row16_sum(acc);
      const float val = ((__shfl(rs, 0, 64) + __shfl(rs, 16, 64)) + __shfl(rs, 32, 64)) + __shfl(rs, 48, 64);
      if (lane == 0) {
        const unsigned long long key =
            ((unsigned long long)float_key(val) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)v);
        atomicMax(a.keys + ((int)(blockIdx.x % kKeyCopies) * kKeyRows + m) * kKeyStride, key);
        atomicAdd(a.counts + m, 1u);
      }
    }
  }

  // every atomic of this workgroup is done before it counts itself
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (tid == 0) s_last = (atomicAdd(a.done, 1u) == gridDim.x - 1) ? 1 : 0;
  __syncthreads();
  if (s_last) {
    for (int m = tid; m < a.M; m += 256) {
      unsigned long long k = 0;
#pragma unroll
      for (int x = 0; x < kKeyCopies; ++x) {
        k = umax64(k, atomicExch(a.keys + (x * kKeyRows + m) * kKeyStride, 0ull));
        atomicExch(a.lb_keys + (x * kKeyRows + m) * kKeyStride, 0ull);
      }
      a.idx[m] = (int32_t)(0xFFFFFFFFu - (uint32_t)k);
      if (a.maxval) a.maxval[m] = key_float((uint32_t)(k >> 32));
      const uint32_t cn = atomicExch(a.counts + m, 0u);
      if (a.rescored) a.rescored[m] = (int32_t)cn;
    }
    if (tid == 0) {
      atomicExch(a.list_count, 0u);
      atomicExch(a.done, 0u);
    }
  }
}

}  // namespace

hipError_t launch_cert_rescore(const CertRescoreArgs& a, int rescore_grid, hipStream_t s) {
  const int groups = (int)(a.w.n / 4);
  const int select_grid = (groups + 4 * kGroupsPerWave - 1) / (4 * kGroupsPerWave);
  hipLaunchKernelGGL(cert_select_kernel, dim3((unsigned)select_grid), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(cert_rescore_kernel, dim3((unsigned)rescore_grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_cert_pack(const uint16_t* w, int64_t n, int64_t k, const uint8_t* e_top, int8_t* q,
                            uint8_t* code, float* cbound, hipStream_t s) {
  hipLaunchKernelGGL(cert_pack_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, s, w, n, k, e_top, q, code,
                     cbound);
  return hipGetLastError();
}

}  // namespace w12
