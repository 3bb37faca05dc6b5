// quantize.hip -- block quantization of bf16 Q, K and V (gfx950).
//
// One memory-bound pass per tensor, as the pages fuse it ahead of the attention
// kernel (SageAttention3 notes, Q3: the V transpose is fused into quantization;
// "FLAMIA", section 3.5: one fused quantization launch):
//   role QK: per token, blocks of 16 or 32 consecutive channels.  Each lane loads
//            8 channels (one 16-byte load), block maxima are reduced across the 2
//            or 4 lanes of a block with lane shuffles, and each lane stores its 8
//            codes as one dword.
//   role V : per channel, blocks of consecutive tokens inside one document,
//            written transposed.  A workgroup stages 128 padded key slots x 128
//            channels in LDS with coalesced row loads, then each lane quantizes
//            64 keys of one channel and stores them contiguously.
// Scale rules ("MXAttention", section 2 and Table 1; blog "NVFP4, not MXFP4"):
//   E8M0: exponent from the block maximum by the OCP or ceiling rule, element
//         x * 2^-e (exact); E4M3: s = E4M3(fp32(M / 6)), element fp32(x / s).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_util.h"
#include "formats.h"
#include "kernels.h"

namespace mxattn {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return u2f(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return u2f(w & 0xFFFF0000u); }

// code of one element for a block whose scale is given either as 2^-e (E8M0,
// inv) or as the E4M3 value s (div)
template <int ELEM, int SCALE>
__device__ __forceinline__ uint32_t encode_elem(float x, float inv, float s) {
  uint32_t sign = f2u(x) >> 31;
  float a = __builtin_fabsf(x);
  if constexpr (ELEM == ELEM_E2M1) {
    float y;
    if constexpr (SCALE == SCALE_E8M0) y = a * inv;
    else y = (s == 0.0f) ? 0.0f : a / s;
    return e2m1_mag(y) | (sign << 3);
  } else {
    float y = a * inv;  // E4M3 elements only come with E8M0 scales
    return e4m3_mag(y) | (sign << 7);
  }
}

template <int SCALE>
__device__ __forceinline__ uint32_t block_scale(float M, E8m0Rule rule, float* inv, float* s) {
  if constexpr (SCALE == SCALE_E8M0) {
    int e = e8m0_exp(M, rule);
    *inv = exp2i_neg(e);
    *s = 0.0f;
    return (uint32_t)(e + 127);
  } else {
    uint32_t c = e4m3_mag(M / 6.0f);
    *s = e4m3_value(c);
    *inv = 0.0f;
    return c;
  }
}

// ---------------------------------------------------------------------------
// role QK: x [B][H][N][128] (strided), codes [B][H][N][64], scales [B][H][N][128/BLOCK]
// ---------------------------------------------------------------------------
template <int SCALE, int BLOCK>
__global__ __launch_bounds__(256) void quant_qk_kernel(const uint16_t* __restrict__ x, int64_t sB, int64_t sH,
                                                       int64_t sN, int64_t H, int64_t N, int64_t rows,
                                                       int64_t nslot, E8m0Rule rule, uint32_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales) {
  // 16 lanes per token row (8 elements each); a thread quantizes the rows slot + u nslot,
  // u < QK_ROWS, with all their loads issued first (a wave's load of one u covers 4
  // consecutive rows); rows past the end load the last row and store nothing
  constexpr int QK_ROWS = 4;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t slot = gid >> 4;
  const int chunk = (int)(gid & 15);
  uint4 v[QK_ROWS];
#pragma unroll
  for (int u = 0; u < QK_ROWS; u++) {
    const int64_t row = slot + u * nslot;
    // row = (b H + h) N + n; 32-bit division (the host keeps rows below 2^31)
    const uint32_t r = (uint32_t)(row < rows ? row : rows - 1);
    const uint32_t n = r % (uint32_t)N, bh = r / (uint32_t)N;
    const uint32_t h = bh % (uint32_t)H, b = bh / (uint32_t)H;
    v[u] = *reinterpret_cast<const uint4*>(x + (int64_t)b * sB + (int64_t)h * sH + (int64_t)n * sN + chunk * 8);
  }
#pragma unroll
  for (int u = 0; u < QK_ROWS; u++) {
    const int64_t row = slot + u * nslot;
    float f[8] = {bf16_lo(v[u].x), bf16_hi(v[u].x), bf16_lo(v[u].y), bf16_hi(v[u].y),
                  bf16_lo(v[u].z), bf16_hi(v[u].z), bf16_lo(v[u].w), bf16_hi(v[u].w)};
    float M = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; j++) M = __builtin_fmaxf(M, __builtin_fabsf(f[j]));
    // lanes of one block are adjacent: 2 (BLOCK 16) or 4 (BLOCK 32)
    M = __builtin_fmaxf(M, __shfl_xor(M, 1));
    if constexpr (BLOCK == 32) M = __builtin_fmaxf(M, __shfl_xor(M, 2));
    float inv, s;
    uint32_t sb = block_scale<SCALE>(M, rule, &inv, &s);
    uint32_t w = 0;
    // power-of-two scales: the scaled FP4 convert rounds to nearest even with
    // saturation and keeps the sign, as the element encoder does; blocks whose scale
    // lies near the ends of the E8M0 range (where subnormal or non-finite inputs can
    // occur) take the integer encoder
    const int e = (int)sb - 127;
    if (SCALE == SCALE_E8M0 && e >= -124 && e < 127) {
      w = pack8_fp4(f, u2f((uint32_t)(e + 127) << 23));
    } else if (SCALE == SCALE_E4M3 && M < __builtin_inff()) {
      // E4M3 scale: the quotient x / s correctly rounded from the block's correctly
      // rounded reciprocal r by one residual step (q = x r, e = x - s q exactly by
      // FMA, q + e r rounded once: Markstein's division), then the scaled FP4 convert
      // at scale 1.  The quotient takes x's sign (a zero one included, as the element
      // encoder keeps it); a zero scale gives zero quotients.
      const float r = s > 0.0f ? 1.0f / s : 0.0f;
      float y[8];
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const float q = f[j] * r;
        const float t = __builtin_fmaf(__builtin_fmaf(-q, s, f[j]), r, q);
        y[j] = __builtin_copysignf(s > 0.0f ? t : 0.0f, f[j]);
      }
      w = pack8_fp4(y, 1.0f);
    } else {
#pragma unroll
      for (int j = 0; j < 8; j++) w |= encode_elem<ELEM_E2M1, SCALE>(f[j], inv, s) << (4 * j);
    }
    if (row < rows) {
      codes[row * 16 + chunk] = w;
      if ((chunk & (BLOCK / 8 - 1)) == 0) scales[row * (128 / BLOCK) + chunk / (BLOCK / 8)] = (uint8_t)sb;
    }
  }
}

// ---------------------------------------------------------------------------
// role V: x [B][H][N][128] (strided) -> codes [B][H][128][np * bits/8],
// scales [B][H][128][np / BLOCK].  One workgroup per (b, h) and run of kt <= VQ_KT
// tiles of 128 key slots, walked in order with the next tile's loads in flight while
// the current one is encoded.  A tile gives each channel row only 128 / BLOCK scale
// bytes; they are collected in LDS and each row's bytes of the whole run are written
// at the end as one contiguous piece (per-tile byte writes to 128 rows cost a full
// write granule for every 4 useful bytes).
// cu: device document offsets (ndocs + 1) or null for one document [0, N).
// ---------------------------------------------------------------------------
constexpr int VQ_ROW = 128 * 2 + 16;  // bytes per staged token row (bf16, padded)
constexpr int VQ_MAXDOC = 1024;       // document offsets staged in LDS (more: read from memory)

// Token of padded V slot p, or -1 for padding.  Without documents slot p is token p
// (p < N).  With documents each one's slots start at a multiple of BLOCK after the
// previous document's (its blocks are document-local) and its last block is padded.
template <int BLOCK>
__device__ __forceinline__ int32_t slot_token(int64_t p, int64_t N, const int32_t* cu, int ndocs) {
  if (cu == nullptr) return p < N ? (int32_t)p : -1;
  int64_t voff = 0;
  for (int k = 0; k < ndocs; k++) {
    const int64_t L = cu[k + 1] - cu[k];
    const int64_t span = (L + BLOCK - 1) / BLOCK * BLOCK;
    if (p < voff + span) return p - voff < L ? (int32_t)(cu[k] + (p - voff)) : -1;
    voff += span;
  }
  return -1;
}

// the document offsets a V quantizer reads: staged in LDS (cu_s, VQ_MAXDOC + 1 entries)
// when they fit, else the device array
__device__ __forceinline__ const int32_t* stage_offsets(const int32_t* cu, int ndocs, int32_t* cu_s) {
  if (cu == nullptr || ndocs > VQ_MAXDOC) return cu;
  for (int i = threadIdx.x; i <= ndocs; i += blockDim.x) cu_s[i] = cu[i];
  return cu_s;  // visible after the caller's next barrier
}
constexpr int VQ_KT = 8;              // most key tiles of 128 slots per workgroup

// TILED (role VT, MXFP4 or an FP8 V, E8M0 per 32): the same bytes tile-major, key
// tile t of channel c at [t][c] (64 or 128 code bytes, 4 scale bytes).
template <int ELEM, int SCALE, int BLOCK, bool TILED = false>
__global__ __launch_bounds__(256) void quant_v_kernel(const uint16_t* __restrict__ x, int64_t sB, int64_t sH,
                                                      int64_t sN, int64_t H, int64_t N, int64_t np,
                                                      const int32_t* __restrict__ cu, int ndocs, E8m0Rule rule,
                                                      uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                      int kt) {
  constexpr int SPT = 128 / BLOCK;      // scale bytes per channel row and tile
  constexpr int SCW = VQ_KT * SPT;      // ... and per run
  __shared__ int32_t tok[2][128];
  __shared__ int32_t cu_s[VQ_MAXDOC + 1];
  __shared__ __attribute__((aligned(16))) uint8_t tile[128 * VQ_ROW];
  __shared__ __attribute__((aligned(16))) uint8_t sc[128 * SCW];
  const int tid = threadIdx.x;
  const int64_t ntiles = np / 128, nruns = (ntiles + kt - 1) / kt;
  const int64_t bh = blockIdx.x / nruns;
  const int64_t tile0 = (blockIdx.x % nruns) * kt;
  const int nt = (int)(ntiles - tile0 < kt ? ntiles - tile0 : kt);
  const int64_t b = bh / H, h = bh % H;
  const uint16_t* xb = x + b * sB + h * sH;

  // padded key slot -> token (or -1 for padding) of tile tt, by threads < 128
  const int32_t* offs = stage_offsets(cu, ndocs, cu_s);
  auto slot_tokens = [&](int tt) __attribute__((always_inline)) {
    tok[tt & 1][tid] = slot_token<BLOCK>((tile0 + tt) * 128 + tid, N, offs, ndocs);
  };
  // 128 token rows x 256 bytes: 2048 chunks of 16 bytes, 8 per thread
  uint4 ld[8];
  auto load_rows = [&](int tt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int c = tid + 256 * i, row = c >> 4, part = c & 15;
      const int32_t t = tok[tt & 1][row];
      ld[i] = make_uint4(0, 0, 0, 0);
      if (t >= 0) ld[i] = *reinterpret_cast<const uint4*>(xb + (int64_t)t * sN + part * 8);
    }
  };

  __syncthreads();  // the staged document offsets
  if (tid < 128) slot_tokens(0);
  __syncthreads();
  load_rows(0);
  for (int tt = 0; tt < nt; tt++) {
    __syncthreads();  // the previous tile's encoding is done with the staged rows
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int c = tid + 256 * i, row = c >> 4, part = c & 15;
      *reinterpret_cast<uint4*>(tile + row * VQ_ROW + part * 16) = ld[i];
    }
    if (tt + 1 < nt && tid < 128) slot_tokens(tt + 1);
    __syncthreads();
    if (tt + 1 < nt) load_rows(tt + 1);  // in flight during this tile's encoding
    const int64_t t0 = (tile0 + tt) * 128;
    if constexpr (ELEM == ELEM_E2M1 && SCALE == SCALE_E8M0 && BLOCK == 32) {
      // MXFP4: lane -> (channels 2 cp and 2 cp + 1, the 32 keys 32 kq + [0, 32)), one
      // block per channel; dword reads of the staged rows (64 lanes cover a row)
      const int cp = tid & 63, kq = tid >> 6;
      float f[2][32];
      float M[2] = {0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < 32; j++) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(tile + (32 * kq + j) * VQ_ROW + cp * 4);
        f[0][j] = bf16_lo(w);
        f[1][j] = bf16_hi(w);
        M[0] = __builtin_fmaxf(M[0], __builtin_fabsf(f[0][j]));
        M[1] = __builtin_fmaxf(M[1], __builtin_fabsf(f[1][j]));
      }
#pragma unroll
      for (int c = 0; c < 2; c++) {
        float inv, sdum;
        const uint32_t sb = block_scale<SCALE_E8M0>(M[c], rule, &inv, &sdum);
        const int e = (int)sb - 127;
        uint32_t w[4];
        if (e >= -124 && e < 127) {  // the scaled FP4 convert, as in the Q/K quantizer
          const float scv = u2f((uint32_t)(e + 127) << 23);
#pragma unroll
          for (int i = 0; i < 4; i++) w[i] = pack8_fp4(&f[c][8 * i], scv);
        } else {
#pragma unroll
          for (int i = 0; i < 4; i++) {
            w[i] = 0;
#pragma unroll
            for (int j = 0; j < 8; j++) w[i] |= encode_elem<ELEM_E2M1, SCALE_E8M0>(f[c][8 * i + j], inv, 0.0f) << (4 * j);
          }
        }
        const int64_t crow = bh * 128 + 2 * cp + c;
        uint8_t* cdst = TILED ? codes + ((bh * ntiles + t0 / 128) * 128 + 2 * cp + c) * 64 + 16 * kq
                              : codes + crow * (np / 2) + (t0 + 32 * kq) / 2;
        *reinterpret_cast<uint4*>(cdst) = make_uint4(w[0], w[1], w[2], w[3]);
        sc[(2 * cp + c) * SCW + tt * SPT + kq] = (uint8_t)sb;
      }
    } else {
      // lane -> (channel, 64 keys)
      const int ch = tid & 127, sub = tid >> 7;
      const int64_t crow = bh * 128 + ch;
      constexpr int NB = 64 / BLOCK;
      constexpr int BPE = ELEM == ELEM_E2M1 ? 4 : 8;  // bits per element
      uint32_t out[64 * BPE / 32];
#pragma unroll
      for (int i = 0; i < 64 * BPE / 32; i++) out[i] = 0;
      uint32_t sbytes = 0;
#pragma unroll
      for (int blk = 0; blk < NB; blk++) {
        float f[BLOCK];
        float M = 0.0f;
#pragma unroll
        for (int j = 0; j < BLOCK; j++) {
          int key = sub * 64 + blk * BLOCK + j;
          uint32_t hbits = *reinterpret_cast<const uint16_t*>(tile + key * VQ_ROW + ch * 2);
          f[j] = u2f(hbits << 16);
          M = __builtin_fmaxf(M, __builtin_fabsf(f[j]));
        }
        float inv, sv;
        uint32_t sb = block_scale<SCALE>(M, rule, &inv, &sv);
        sbytes |= sb << (8 * blk);
#pragma unroll
        for (int j = 0; j < BLOCK; j++) {
          int e = blk * BLOCK + j;  // element index within this lane's 64 keys
          uint32_t c = encode_elem<ELEM, SCALE>(f[j], inv, sv);
          out[(e * BPE) / 32] |= c << ((e * BPE) % 32);
        }
      }
      uint8_t* cdst = TILED ? codes + ((bh * ntiles + t0 / 128) * 128 + ch) * (128 * BPE / 8) + sub * 64 * BPE / 8
                            : codes + crow * (np * BPE / 8) + (t0 + sub * 64) * BPE / 8;
#pragma unroll
      for (int i = 0; i < 64 * BPE / 128; i++)
        reinterpret_cast<uint4*>(cdst)[i] = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
      uint8_t* sdst = sc + ch * SCW + tt * SPT + sub * NB;
      if constexpr (NB == 2) *reinterpret_cast<uint16_t*>(sdst) = (uint16_t)sbytes;
      else *reinterpret_cast<uint32_t*>(sdst) = sbytes;
    }
  }
  __syncthreads();
  // each channel row's nt * SPT scale bytes (a multiple of 4), one dword per thread step
  const int dpr = nt * SPT / 4;
  for (int i = tid; i < 128 * dpr; i += 256) {
    const int r = i / dpr, w = i - r * dpr;
    uint8_t* sdst = TILED ? scales + ((bh * ntiles + tile0 + w) * 128 + r) * 4  // SPT = 4: one dword per tile
                          : scales + (bh * 128 + r) * (np / BLOCK) + tile0 * SPT + 4 * w;
    *reinterpret_cast<uint32_t*>(sdst) = *reinterpret_cast<const uint32_t*>(sc + r * SCW + 4 * w);
  }
}

// ---------------------------------------------------------------------------
// role VKEY: the per-key form of a 4-bit V for causally safe diagonal tiles ("FLAMIA",
// section 3.2): per key slot one E8M0 scale over its 128 channels, E2M1 codes of
// x / 2^e written transposed as for role V.  x [B][H][N][128] -> codes
// [B][H][128][np / 2], scales [B][H][np].  The slot layout (documents starting at
// BLOCK boundaries) is role V's, so a key has the same slot in both forms.
// ---------------------------------------------------------------------------
template <int BLOCK>
__global__ __launch_bounds__(256) void quant_vkey_kernel(const uint16_t* __restrict__ x, int64_t sB, int64_t sH,
                                                         int64_t sN, int64_t H, int64_t N, int64_t np,
                                                         const int32_t* __restrict__ cu, int ndocs, E8m0Rule rule,
                                                         uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  __shared__ int32_t tok[128];
  __shared__ int32_t cu_s[VQ_MAXDOC + 1];
  __shared__ float inv_s[128];
  __shared__ __attribute__((aligned(16))) uint8_t tile[128 * VQ_ROW];
  const int tid = threadIdx.x;
  const int64_t ntiles = np / 128;
  const int64_t bh = blockIdx.x / ntiles;
  const int64_t t0 = (blockIdx.x % ntiles) * 128;
  const int64_t b = bh / H, h = bh % H;
  const int32_t* offs = stage_offsets(cu, ndocs, cu_s);
  __syncthreads();
  if (tid < 128) tok[tid] = slot_token<BLOCK>(t0 + tid, N, offs, ndocs);
  __syncthreads();
  const uint16_t* xb = x + b * sB + h * sH;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    int c = tid + 256 * i;
    int row = c >> 4, part = c & 15;
    int32_t t = tok[row];
    uint4 v = make_uint4(0, 0, 0, 0);
    if (t >= 0) v = *reinterpret_cast<const uint4*>(xb + (int64_t)t * sN + part * 8);
    *reinterpret_cast<uint4*>(tile + row * VQ_ROW + part * 16) = v;
  }
  __syncthreads();
  // per slot: maximum over its 128 channels (two threads of 64 channels each)
  {
    const int slot = tid >> 1, half = tid & 1;
    float M = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const uint4 v = *reinterpret_cast<const uint4*>(tile + slot * VQ_ROW + half * 128 + i * 16);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int u = 0; u < 4; u++)
        M = __builtin_fmaxf(M, __builtin_fmaxf(__builtin_fabsf(u2f(w[u] << 16)), __builtin_fabsf(u2f(w[u] & 0xFFFF0000u))));
    }
    M = __builtin_fmaxf(M, __shfl_xor(M, 1));
    const int e = e8m0_exp(M, rule);
    if (half == 0) {
      inv_s[slot] = exp2i_neg(e);
      scales[bh * np + t0 + slot] = (uint8_t)(e + 127);
    }
  }
  __syncthreads();
  // lane -> (channel, 64 keys), codes stored contiguously per channel row
  const int ch = tid & 127, sub = tid >> 7;
  uint32_t out[8];
#pragma unroll
  for (int i = 0; i < 8; i++) out[i] = 0;
#pragma unroll
  for (int j = 0; j < 64; j++) {
    const int key = sub * 64 + j;
    const uint32_t hbits = *reinterpret_cast<const uint16_t*>(tile + key * VQ_ROW + ch * 2);
    const float f = u2f(hbits << 16);
    const uint32_t c = e2m1_mag(__builtin_fabsf(f) * inv_s[key]) | ((f2u(f) >> 31) << 3);
    out[j >> 3] |= c << (4 * (j & 7));
  }
  uint8_t* cdst = codes + (bh * 128 + ch) * (np / 2) + (t0 + sub * 64) / 2;
#pragma unroll
  for (int i = 0; i < 2; i++)
    reinterpret_cast<uint4*>(cdst)[i] = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
}

hipError_t launch_quant_vkey(const QuantArgs& a, hipStream_t st) {
  dim3 grid((unsigned)(a.B * a.H * (a.np / 128)));
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  uint8_t* c = static_cast<uint8_t*>(a.codes);
  uint8_t* s = static_cast<uint8_t*>(a.scales);
  if (a.elem != ELEM_E2M1 || a.scale != SCALE_E8M0) return hipErrorInvalidValue;
  if (a.block == 32)
    quant_vkey_kernel<32><<<grid, 256, 0, st>>>(x, a.sB, a.sH, a.sN, a.H, a.N, a.np, a.cu, a.ndocs, a.rule, c, s);
  else if (a.block == 16)
    quant_vkey_kernel<16><<<grid, 256, 0, st>>>(x, a.sB, a.sH, a.sN, a.H, a.N, a.np, a.cu, a.ndocs, a.rule, c, s);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// unquantized route: a dense copy of a strided bf16 tensor, 16 bytes per thread
// (16 threads per 128-channel row)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void copy_bf16_kernel(const uint16_t* __restrict__ x, int64_t sB, int64_t sH,
                                                        int64_t sN, int64_t H, int64_t N, int64_t rows,
                                                        uint16_t* __restrict__ dst) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = t >> 4;
  if (row >= rows) return;
  const int part = (int)(t & 15);
  const int64_t n = row % N, bh = row / N, h = bh % H, b = bh / H;
  const u4 v = *reinterpret_cast<const u4*>(x + b * sB + h * sH + n * sN + 8 * part);
  *reinterpret_cast<u4*>(dst + row * 128 + 8 * part) = v;
}

hipError_t launch_copy_bf16(const void* x, int64_t sB, int64_t sH, int64_t sN, int64_t B, int64_t H, int64_t N,
                            void* dst, hipStream_t st) {
  const int64_t rows = B * H * N;
  if (rows >= (int64_t(1) << 27)) return hipErrorNotSupported;  // 32-bit thread ids
  copy_bf16_kernel<<<dim3((unsigned)((rows * 16 + 255) / 256)), 256, 0, st>>>(
      static_cast<const uint16_t*>(x), sB, sH, sN, H, N, rows, static_cast<uint16_t*>(dst));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_quant_qk(const QuantArgs& a, hipStream_t st) {
  const int64_t rows = a.B * a.H * a.N;
  if (rows >= (int64_t(1) << 31)) return hipErrorInvalidValue;  // 32-bit row indices
  const int64_t nslot = (rows + 3) / 4;  // each thread quantizes 4 rows, nslot apart
  const int64_t threads = nslot * 16;
  dim3 grid((unsigned)((threads + 255) / 256));
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  uint32_t* c = static_cast<uint32_t*>(a.codes);
  uint8_t* s = static_cast<uint8_t*>(a.scales);
  if (a.scale == SCALE_E8M0 && a.block == 32)
    quant_qk_kernel<SCALE_E8M0, 32><<<grid, 256, 0, st>>>(x, a.sB, a.sH, a.sN, a.H, a.N, rows, nslot, a.rule, c, s);
  else if (a.scale == SCALE_E8M0 && a.block == 16)
    quant_qk_kernel<SCALE_E8M0, 16><<<grid, 256, 0, st>>>(x, a.sB, a.sH, a.sN, a.H, a.N, rows, nslot, a.rule, c, s);
  else if (a.scale == SCALE_E4M3 && a.block == 16)
    quant_qk_kernel<SCALE_E4M3, 16><<<grid, 256, 0, st>>>(x, a.sB, a.sH, a.sN, a.H, a.N, rows, nslot, a.rule, c, s);
  else if (a.scale == SCALE_E4M3 && a.block == 32)
    quant_qk_kernel<SCALE_E4M3, 32><<<grid, 256, 0, st>>>(x, a.sB, a.sH, a.sN, a.H, a.N, rows, nslot, a.rule, c, s);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_quant_v(const QuantArgs& a, hipStream_t st) {
  // the longest run (8, 4, 2 or 1 tiles) whose grid fills the CUs' 768 resident
  // workgroups (3 per CU) to at least 85% over its rounds: longer runs write longer
  // scale pieces, but a last round left mostly empty idles the CUs
  const int64_t ntiles = a.np / 128;
  int kt = VQ_KT;
  for (; kt > 1; kt /= 2) {
    const int64_t nwg = a.B * a.H * ((ntiles + kt - 1) / kt), rounds = (nwg + 767) / 768;
    if (nwg * 100 >= rounds * 768 * 85) break;
  }
  dim3 grid((unsigned)(a.B * a.H * ((ntiles + kt - 1) / kt)));
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  uint8_t* c = static_cast<uint8_t*>(a.codes);
  uint8_t* s = static_cast<uint8_t*>(a.scales);
#define MXQV(E, S, BL)                                                                                   \
  quant_v_kernel<E, S, BL><<<grid, 256, 0, st>>>(x, a.sB, a.sH, a.sN, a.H, a.N, a.np, a.cu, a.ndocs, a.rule, \
                                                 c, s, kt)
  if (a.tiled) {  // role VT: MXFP4 or an FP8 V with E8M0 per 32 (checked by the host)
    if (a.scale != SCALE_E8M0 || a.block != 32) return hipErrorInvalidValue;
    if (a.elem == ELEM_E2M1)
      quant_v_kernel<ELEM_E2M1, SCALE_E8M0, 32, true><<<grid, 256, 0, st>>>(x, a.sB, a.sH, a.sN, a.H, a.N, a.np,
                                                                           a.cu, a.ndocs, a.rule, c, s, kt);
    else if (a.elem == ELEM_E4M3)
      quant_v_kernel<ELEM_E4M3, SCALE_E8M0, 32, true><<<grid, 256, 0, st>>>(x, a.sB, a.sH, a.sN, a.H, a.N, a.np,
                                                                           a.cu, a.ndocs, a.rule, c, s, kt);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  }
  if (a.elem == ELEM_E2M1 && a.scale == SCALE_E8M0 && a.block == 32) MXQV(ELEM_E2M1, SCALE_E8M0, 32);
  else if (a.elem == ELEM_E2M1 && a.scale == SCALE_E8M0 && a.block == 16) MXQV(ELEM_E2M1, SCALE_E8M0, 16);
  else if (a.elem == ELEM_E2M1 && a.scale == SCALE_E4M3 && a.block == 16) MXQV(ELEM_E2M1, SCALE_E4M3, 16);
  else if (a.elem == ELEM_E2M1 && a.scale == SCALE_E4M3 && a.block == 32) MXQV(ELEM_E2M1, SCALE_E4M3, 32);
  else if (a.elem == ELEM_E4M3 && a.scale == SCALE_E8M0 && a.block == 32) MXQV(ELEM_E4M3, SCALE_E8M0, 32);
  else if (a.elem == ELEM_E4M3 && a.scale == SCALE_E8M0 && a.block == 16) MXQV(ELEM_E4M3, SCALE_E8M0, 16);
  else return hipErrorInvalidValue;
#undef MXQV
  return hipGetLastError();
}

}  // namespace mxattn
