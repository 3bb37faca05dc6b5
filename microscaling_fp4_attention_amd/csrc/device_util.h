// device_util.h -- small device helpers shared by the attention kernels (gfx950):
// vector types, MFMA wrappers, lane-half reductions, E2M1 packing and the key
// permutation that makes each lane's 16 scores 16 consecutive keys.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "formats.h"
#include "kernels.h"

namespace mxattn {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u4 mk4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u4 r = {a, b, c, d};
  return r;
}
__device__ __forceinline__ u2 mk2(uint32_t a, uint32_t b) {
  u2 r = {a, b};
  return r;
}

constexpr float NEG_INF = -__builtin_inff();

__device__ __forceinline__ v16f zero16() {
  v16f z;
#pragma unroll
  for (int i = 0; i < 16; i++) z[i] = 0.0f;
  return z;
}

// 16 consecutive floats from LDS (a lane's score bias of one 32-key block: its 16
// scores belong to 16 consecutive keys)
__device__ __forceinline__ v16f bias16(const uint8_t* p) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 16),
               c = *reinterpret_cast<const float4*>(p + 32), d = *reinterpret_cast<const float4*>(p + 48);
  v16f r = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w, c.x, c.y, c.z, c.w, d.x, d.y, d.z, d.w};
  return r;
}

__device__ __forceinline__ v8i v8_from4(u4 t) {
  v8i r = {(int)t.x, (int)t.y, (int)t.z, (int)t.w, 0, 0, 0, 0};
  return r;
}

__device__ __forceinline__ v16f mfma_fp4(v8i a, v8i b, v16f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 0, sa, 0, sb);
}
__device__ __forceinline__ v16f mfma_fp8(v8i a, v8i b, v16f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}
__device__ __forceinline__ v16f mfma_bf16(v8bf a, v8bf b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v16f mfma_f16(v8h a, v8h b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// A wave-uniform float held in a VGPR.  On gfx950 a VALU instruction with an SGPR
// operand issues at about 4.5 cycles per wave64 instruction, one with VGPR operands
// only at about 2.8 (an FMA; measured with independent chains), so a constant read
// once per score element (the exponent scale lambda) is copied to a VGPR once.  The
// copy is opaque to the compiler, which would otherwise keep the value in an SGPR.
__device__ __forceinline__ float to_vgpr(float x) {
  float y;
  asm volatile("v_mov_b32 %0, %1" : "=v"(y) : "v"(x));
  return y;
}

// 2^(lambda (x - msub)) formed from the difference x - msub, so that it is exactly 1
// at x = msub: block scales and the two-level pre-scale are chosen from this value,
// and at the row's maximum P~ must be the exactly represented 1 ("MXAttention",
// section 4.2; for the OCP rule 1 sits on a scale boundary, Table 1).  msub is the
// running maximum, or 0 while that is -inf (then every x is -inf and the result 0).
__device__ __forceinline__ float exp2_diff(float x, float msub, float lam) { return exp2_hw((x - msub) * lam); }

// Bit-level exponential ("FLAMIA" section 3.7 and appendix C): y = 2^23 (t + 127) in a
// float; the float whose bits are the integer part of y is Mitchell's line
// 2^floor(t) (1 + frac t) (a subnormal below t = -126).  The max clamps negative y,
// -inf and NaN to 0 (a float-to-unsigned conversion of those is undefined); y stays
// below 2^31 for the t < 129 this serves.  v_max_f32 + v_cvt_u32_f32.  (The convert
// alone saturates the same way, but written as inline assembly it split the
// scheduling regions of the exponential loop and made the kernel spill.)
__device__ __forceinline__ float exp2_bits(float y) {
  return __builtin_bit_cast(float, (uint32_t)__builtin_fmaxf(y, 0.0f));
}

// the other lane half's value (lanes q and q+32 hold the two halves of a row)
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32); }

// max that propagates NaN (v_maximum3_f32 on gfx950): unlike fmaxf it needs no
// quieting of its operands first, and scores are never NaN for finite inputs
__device__ __forceinline__ float fmaxn(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// max / sum of the two lane halves of a row, in registers: v_permlane32_swap with
// both operands x leaves x of lanes 0-31 in every lane of the first result and x of
// lanes 32-63 in every lane of the second
__device__ __forceinline__ float halves_max(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
  return fmaxn(u2f(p[0]), u2f(p[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
  return u2f(p[0]) + u2f(p[1]);
}

// two floats whose values have at most 8 significant bits -> packed bf16 (exact)
__device__ __forceinline__ uint32_t pack_bf16_exact(float lo, float hi) {
  return (f2u(lo) >> 16) | (f2u(hi) & 0xFFFF0000u);
}

// float -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  uint32_t u = f2u(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// E2M1 codes of 2 floats, y = x / 2^k with the power of two given as a float
// (the gfx950 convert uses the exponent of `scale`; it rounds to nearest even and
// saturates at 6), into byte `sel` of `old`.
#define CVT_FP4(old, x0, x1, scale, sel) __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, x0, x1, scale, sel)

// 8 floats -> 8 E2M1 codes in one dword (element 2k in the low nibble of byte k)
// `old` is any dword: the four converts overwrite every byte of it (passing a dead
// register saves the instruction that would clear one)
__device__ __forceinline__ uint32_t pack8_fp4(const float* x, float scale, uint32_t old = 0) {
  uint32_t w = old;
  w = CVT_FP4(w, x[0], x[1], scale, 0);
  w = CVT_FP4(w, x[2], x[3], scale, 1);
  w = CVT_FP4(w, x[4], x[5], scale, 2);
  w = CVT_FP4(w, x[6], x[7], scale, 3);
  return w;
}

// the 2 E2M1 values of byte `sel` of w as floats (exact)
__device__ __forceinline__ v2f fp4_pair(uint32_t w, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  }
}

// 8 E2M1 codes (one dword) times a scale -> 8 bf16 (4 dwords), exact
__device__ __forceinline__ u4 dq8_bf16(uint32_t w, float s) {
  v2f p0 = fp4_pair(w, 0), p1 = fp4_pair(w, 1), p2 = fp4_pair(w, 2), p3 = fp4_pair(w, 3);
  return mk4(pack_bf16_exact(p0[0] * s, p0[1] * s), pack_bf16_exact(p1[0] * s, p1[1] * s),
                    pack_bf16_exact(p2[0] * s, p2[1] * s), pack_bf16_exact(p3[0] * s, p3[1] * s));
}

// 8 E2M1 codes (one dword, low nibble first) times a power of two `sc` (the convert
// uses the exponent of its scale operand) -> 8 f16 (4 dwords)
__device__ __forceinline__ u4 dq8_f16_pow2(uint32_t w, float sc) {
  return mk4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 0)),
             __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 1)),
             __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 2)),
             __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 3)));
}

// 8 E2M1 codes times an E4M3 value s2 (both halves) -> 8 f16, exact: an E2M1 value
// times an E4M3 value has at most 6 significant bits and lies in [2^-10, 2688]
__device__ __forceinline__ v8h dq8_f16(uint32_t w, v2h s2) {
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  return v8h{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// fl32(x / 6), the input of an E4M3 block scale, by Markstein's division: the quotient
// from the correctly rounded reciprocal of 6 by one residual step, equal to the IEEE
// quotient for every float whose quotient is normal (6 is an E4M3 value; the host test
// of the quantizer's division checks every float of one binade under each of them);
// smaller quotients encode to the zero scale either way
__device__ __forceinline__ float div6(float x) {
  const float r = 0x1.555556p-3f;  // fl32(1/6)
  const float q = x * r;
  return __builtin_fmaf(__builtin_fmaf(-q, 6.0f, x), r, q);
}

__device__ __forceinline__ float scale_value(uint32_t byte, int kind) {
  return kind == SCALE_E8M0 ? (byte == 0 ? u2f(0x400000u) : u2f(byte << 23)) : e4m3_value(byte);
}

// Key permutation of a tile.  Output register j of sub-tile b in lane half h is
// MFMA row 8(j/4) + 4h + j%4; the key placed on that row is
//   key(b, h, j) = 64(b/2) + 32h + 16(b%2) + j            (FP4 and bf16 PV)
//   key(b, h, j) = 64(b/2) + 32(b%2) + 16h + j            (FP8 PV)
// The FP4 form gives each lane half one whole 32-key block per 64-key chunk, the
// unit one lane's E8M0 scale covers in the FP4 MFMA.  In the FP8 MFMA the scale of
// operand element n comes from lane half n/16 (each lane holds 16 elements of both
// 32-element scale groups), so there a lane half holds keys 16h + [0, 16) of both
// 32-key blocks of the chunk.
template <bool SPLIT16>
__device__ __forceinline__ int key_of(int b, int h, int j) {
  return SPLIT16 ? 64 * (b >> 1) + 32 * (b & 1) + 16 * h + j : 64 * (b >> 1) + 32 * h + 16 * (b & 1) + j;
}
// LDS row of key r (0..127) of a tile: sub-tile b, MFMA row rr (inverse of key_of)
template <bool SPLIT16>
__device__ __forceinline__ int kpos(int r) {
  int b = SPLIT16 ? 2 * (r >> 6) + ((r >> 5) & 1) : 2 * (r >> 6) + ((r >> 4) & 1);
  int hh = SPLIT16 ? (r >> 4) & 1 : (r >> 5) & 1;
  int t = r & 15;
  return 32 * b + 8 * (t >> 2) + 4 * hh + (t & 3);
}

}  // namespace mxattn
