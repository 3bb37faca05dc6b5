// formats.h -- device encoders for the block formats (gfx950).
//
// E2M1 (FP4): magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}, sign in bit 3
//   ("Microscaling FP4 Attention" blog, section "NVFP4, not MXFP4"; "MXAttention",
//   section 2, the E2M1 grid).  Rounding is to nearest with ties to the even code
//   and saturation at 6 ("MXAttention", section 3: nearest rounding followed by
//   saturation to the finite range).
// E4M3 (OCP FP8): bias 7, 3 mantissa bits, subnormals, max 448, no infinity
//   (blog, section "The probability squeeze").
// E8M0: a power of two 2^e stored as e + 127 ("MXAttention", section 2).
//
// All encoders work on the IEEE bits of float inputs with integer operations, so
// their decisions are exact; none of them depends on the hardware converts.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxattn {

__device__ __forceinline__ uint32_t f2u(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float u2f(uint32_t x) { return __builtin_bit_cast(float, x); }

// E2M1 magnitude code of y >= 0 (y finite or +inf): each comparison adds one
// step of the grid; a tie goes up exactly when the upper neighbour's code is even
// (0.75 -> 1, 1.75 -> 2, 3.5 -> 4) and stays down otherwise (0.25, 1.25, 2.5, 5).
__device__ __forceinline__ uint32_t e2m1_mag(float y) {
  return (uint32_t)(y > 0.25f) + (uint32_t)(y >= 0.75f) + (uint32_t)(y > 1.25f) +
         (uint32_t)(y >= 1.75f) + (uint32_t)(y > 2.5f) + (uint32_t)(y >= 3.5f) + (uint32_t)(y > 5.0f);
}

// E4M3 magnitude byte (0x00..0x7E) of a >= 0, nearest with ties to even, values at
// or above 448 give 448 (0x7E).
__device__ __forceinline__ uint32_t e4m3_mag(float a) {
  if (!(a < 448.0f)) return 0x7E;
  if (a < 0.015625f) {  // below 2^-6: subnormal steps of 2^-9
    return (uint32_t)__builtin_rintf(a * 512.0f);  // exact scaling, rint is ties-to-even
  }
  uint32_t b = f2u(a);
  uint32_t e = (b >> 23) - 127 + 7;  // E4M3 biased exponent, 1..15
  uint32_t m = b & 0x7FFFFF;
  uint32_t r = m >> 20, rem = m & 0xFFFFF;
  uint32_t up = (rem > 0x80000u) || (rem == 0x80000u && (r & 1u));
  return ((e << 3) | r) + up;  // a carry out of the mantissa bumps the exponent
}

// value of an E4M3 byte (finite codes only)
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  uint32_t e = (c >> 3) & 15, m = c & 7;
  float v = e == 0 ? (float)m * 0.001953125f : u2f(((e + 120) << 23) | (m << 20));
  return (c & 0x80) ? -v : v;
}

// Exponent rule of an E8M0 scale, as two integers prepared on the host:
//   e = be(M) - qe + (mantissa(M) > qm), with be/mantissa the IEEE fields of M.
// For qmax = 1.f_q * 2^(qe - 127) this is the smallest e with M <= qmax * 2^e
// (the ceiling rule); with qe = 127 + emax and qm = 0x7FFFFF (never exceeded) it
// is floor(log2 M) - emax (the OCP rule).  M = 0 gives 0; e is clamped to
// [-127, 127].
struct E8m0Rule {
  int32_t qe;
  uint32_t qm;
};

__device__ __forceinline__ int e8m0_exp(float M, E8m0Rule r) {
  uint32_t b = f2u(M);
  if (b == 0) return 0;
  int e = (int)(b >> 23) - r.qe + (int)((b & 0x7FFFFF) > r.qm);
  e = e < -127 ? -127 : e;
  return e > 127 ? 127 : e;
}

// 2^-e as a float for e in [-126, 127]; 2^127 for e = -127 is finite too.
__device__ __forceinline__ float exp2i_neg(int e) {
  // 2^-e = 2^(127-e-127); for e = -127 this is 2^127 (biased 254), for e = 127 it is 2^-127,
  // a subnormal, built by a shift of the mantissa bit.
  int be = 127 - e;
  return be >= 1 ? u2f((uint32_t)be << 23) : u2f(0x400000u);
}

}  // namespace mxattn
