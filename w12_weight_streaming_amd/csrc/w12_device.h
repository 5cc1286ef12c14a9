// Device helpers shared by the libw12 kernels (gfx950 only).
//
// The W12 code of a weight ("SpecPilot ..." summary, section 4.1; digest page,
// W12 paragraph) is sign + 4-bit exponent offset + 7 mantissa bits. The record
// stores an 8-bit view byte hi8 = s<<7 | o<<3 | m>>4 and a low nibble m & 15;
// restoring bf16 bits is  s<<15 | (o + E_n - 15)<<7 | m.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w12 {

constexpr int kStrip = 32;       // channels per record
constexpr int kRecK = 256;       // k per record
constexpr int kSubK = 32;        // k per subtile / escape block
constexpr int kRecBytes = 12288; // one record
constexpr int kHiBytes = 8192;   // the 8-bit view plane of a record

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// (E_n - 15) << 7 in both 16-bit halves: added to two 11-bit codes at once.
__device__ __forceinline__ uint32_t bias2_of(uint32_t e_top) {
  const uint32_t b = (e_top - 15u) << 7;
  return b | (b << 16);
}

// One bf16 pair from a 4-byte group of the 8-bit view (H) and a 4-byte group
// of low nibbles (L): the byte permute places hi8 above a byte whose high
// nibble is that weight's lo4, so each 16-bit half reads hi8<<8 | lo4<<4 | x.
// Shifting right by 4 and masking 11 bits leaves o<<7 | m; the bias add turns
// o into the exponent (no carry: o + E_n - 15 <= 254) and the sign comes back
// from bit 15 of the permuted word.
__device__ __forceinline__ uint32_t pair_of(uint32_t H, uint32_t L, uint32_t sel,
                                            uint32_t bias2) {
  const uint32_t y = __builtin_amdgcn_perm(H, L, sel);
  const uint32_t v = ((y >> 4) & 0x07FF07FFu) + bias2;
  return (y & 0x80008000u) | v;
}

// Restore the 16 consecutive-k weights a lane holds (16 hi8 bytes, 8 lo bytes)
// into 8 bf16 pairs p[i] = w[2i] | w[2i+1] << 16. Escaped slots come out as
// (E_n - 15) << 7 and are overwritten by the escape patch.
__device__ __forceinline__ void decode16(const uint4 hi, const uint2 lo, uint32_t bias2,
                                         uint32_t (&p)[8]) {
  constexpr uint32_t kSelLo = 0x05010400u;  // bytes [L.b0, H.b0, L.b1, H.b1]
  constexpr uint32_t kSelHi = 0x07030602u;  // bytes [L.b2, H.b2, L.b3, H.b3]
  const uint32_t l0s = lo.x << 4, l1s = lo.y << 4;  // low nibbles -> high nibbles
  p[0] = pair_of(hi.x, lo.x, kSelLo, bias2);
  p[1] = pair_of(hi.x, lo.x, kSelHi, bias2);
  p[2] = pair_of(hi.y, l0s, kSelLo, bias2);
  p[3] = pair_of(hi.y, l0s, kSelHi, bias2);
  p[4] = pair_of(hi.z, lo.y, kSelLo, bias2);
  p[5] = pair_of(hi.z, lo.y, kSelHi, bias2);
  p[6] = pair_of(hi.w, l1s, kSelLo, bias2);
  p[7] = pair_of(hi.w, l1s, kSelHi, bias2);
}

// Ordering point between LDS writes of one lane and reads of another lane of
// the same wavefront: DS operations of a wavefront execute in issue order, so
// only the compiler has to be kept from reordering or forwarding.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Escape entry fields: bits << 16 | c << 5 | kk.
__device__ __forceinline__ uint32_t esc_c(uint32_t e) { return (e >> 5) & 31u; }
__device__ __forceinline__ uint32_t esc_kk(uint32_t e) { return e & 31u; }
__device__ __forceinline__ uint16_t esc_bits(uint32_t e) { return (uint16_t)(e >> 16); }

// Monotone u32 key of a float (larger float -> larger key; -0 folded to +0).
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

}  // namespace w12
