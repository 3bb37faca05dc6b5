// preproc.hip -- outlier pre-processing of Q and K ahead of quantization (gfx950).
//
//   channel means   per (batch, head, document) and channel, over the document's
//                   tokens ("MpFA", section 4.2, Eq. 7; blog "Microscaling FP4
//                   Attention ...", "Smooth-K is the smaller lever"): the sum is taken
//                   in double, then divided by the length in double and rounded once.
//   centered / rotated quantization
//                   y = fl32(((x - mu) H) c) per token, then the usual Q/K block
//                   quantization: H is the Sylvester Hadamard matrix of order 128 and
//                   c = fl64(1 / fl64(sqrt(128))) with the rotation ("FLAMIA", section
//                   3.4 and appendix A.2: a normalized Hadamard transform of the head
//                   channels before quantization), 1 without it.  x - mu and the
//                   +-1 butterflies run in double, where they are exact for bf16 x and
//                   float mu of realistic spans, so the butterfly order does not matter.
//   compensation    delta[j] = fl32(qmean . (K[j] - kmean)) per query head ("MpFA",
//                   section 4.3, Eq. 9), products and sums in double.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_util.h"
#include "formats.h"
#include "kernels.h"

namespace mxattn {

__device__ __forceinline__ float bf16_lo_f(uint32_t w) { return u2f(w << 16); }
__device__ __forceinline__ float bf16_hi_f(uint32_t w) { return u2f(w & 0xFFFF0000u); }

// document of token t: the last k with cu[k] <= t (cu: ndocs + 1 offsets, in device
// memory or staged in LDS)
__device__ __forceinline__ int doc_of_token(const int32_t* __restrict__ cu, int ndocs, int64_t t) {
  if (cu == nullptr || ndocs <= 1) return 0;
  int lo = 0, hi = ndocs - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// the document offsets a workgroup searches: copied to LDS when they fit (the whole
// workgroup must call this), else the device array
constexpr int DOCS_LDS = 1024;
__device__ __forceinline__ const int32_t* stage_docs(const int32_t* __restrict__ cu, int ndocs, int32_t* scu) {
  if (cu == nullptr || ndocs <= 1 || ndocs >= DOCS_LDS) return cu;
  for (int i = threadIdx.x; i <= ndocs; i += blockDim.x) scu[i] = cu[i];
  __syncthreads();
  return scu;
}

// ---------------------------------------------------------------------------
// channel means: 8 workgroups of 512 threads per (b, h, document) unit, one per group
// of 16 channels.  The 8 workgroups of a unit get ids of one residue mod 8, which the
// dispatcher deals to one XCD, so each 256-byte token row is fetched into one L2.
// Thread i sums channels 16 g + 8 (i % 2) + [0, 8) over the tokens t0 + 256 k + i / 2
// in double, 8 reads in flight; the 256 partial sums of a channel are then added in a
// fixed order.
// mean: [B][H][nd][128]; units = B H nd, the grid covers round_up(units, 8) * 8 ids.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(512) void channel_mean_kernel(const uint16_t* __restrict__ x, int64_t sB, int64_t sH,
                                                           int64_t sN, int64_t H, int64_t N,
                                                           const int32_t* __restrict__ cu, int nd, int64_t units,
                                                           float* __restrict__ mean) {
  __shared__ double part[256][17];
  const int64_t id = blockIdx.x;
  const int64_t unit = (id / 64) * 8 + id % 8;
  const int cg = (int)((id / 8) % 8);
  if (unit >= units) return;  // whole workgroup
  const int tid = threadIdx.x, half = tid & 1, slot = tid >> 1;
  // units are numbered document-major, u = doc * (B H) + (b H + h): the heads of one
  // document then have consecutive numbers and spread over the XCDs, where numbering
  // by head first would send every head of a document to the XCD of its residue
  const int64_t BH = units / nd;
  const int64_t doc = unit / BH, bh = unit % BH, b = bh / H, h = bh % H;
  const int64_t t0 = cu ? cu[doc] : 0, t1 = cu ? cu[doc + 1] : N;
  const uint16_t* base = x + b * sB + h * sH + cg * 16 + half * 8;
  double s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  // rounds of 8 tokens per thread, every read of a round issued before any is added;
  // a token past the document adds nothing (not even +0, which would turn a -0 sum
  // positive), so each thread adds its tokens t0 + slot + 256 k in increasing k
  for (int64_t t = t0 + slot; t < t1; t += 8 * 256) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; u++)
      v[u] = t + 256 * u < t1 ? *reinterpret_cast<const uint4*>(base + (t + 256 * u) * sN) : uint4{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < 8; u++) {
      if (t + 256 * u < t1) {
        s[0] += (double)bf16_lo_f(v[u].x); s[1] += (double)bf16_hi_f(v[u].x);
        s[2] += (double)bf16_lo_f(v[u].y); s[3] += (double)bf16_hi_f(v[u].y);
        s[4] += (double)bf16_lo_f(v[u].z); s[5] += (double)bf16_hi_f(v[u].z);
        s[6] += (double)bf16_lo_f(v[u].w); s[7] += (double)bf16_hi_f(v[u].w);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 8; j++) part[slot][half * 8 + j] = s[j];
  __syncthreads();
  // the 256 partial sums of a channel: 16 threads per channel add 16 each, then one
  // thread adds those 16 (a fixed order; the sums are exact in double anyway)
  __shared__ double part2[16][17];
  if (tid < 256) {
    const int c = tid & 15, g = tid >> 4;
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < 16; k++) acc += part[16 * g + k][c];
    part2[g][c] = acc;
  }
  __syncthreads();
  if (tid < 16) {
    double acc = 0.0;
#pragma unroll
    for (int g = 0; g < 16; g++) acc += part2[g][tid];
    const int64_t L = t1 - t0;
    mean[(bh * nd + doc) * 128 + cg * 16 + tid] = L > 0 ? (float)(acc / (double)L) : 0.0f;
  }
}

// ---------------------------------------------------------------------------
// role QK with pre-processing.  Lane = 8 channels of one token (16 lanes a token), as
// in the plain Q/K quantizer; the rotation's butterflies with channel strides 1, 2, 4
// stay in the lane, strides 8 .. 64 pair lanes 1, 2, 4, 8 apart.
// ---------------------------------------------------------------------------
constexpr double HADAMARD_C128 = 0x1.6a09e667f3bccp-4;  // fl64(1 / fl64(sqrt(128)))

template <int SCALE>
__device__ __forceinline__ uint32_t pre_block_scale(float M, E8m0Rule rule, float* inv, float* s) {
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

template <int SCALE, int BLOCK>
__global__ __launch_bounds__(256) void quant_qk_pre_kernel(const uint16_t* __restrict__ x, int64_t sB, int64_t sH,
                                                           int64_t sN, int64_t H, int64_t N, int64_t rows,
                                                           E8m0Rule rule, const float* __restrict__ mean,
                                                           const int32_t* __restrict__ cu, int ndocs, int hadamard,
                                                           uint32_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  __shared__ int32_t scu[DOCS_LDS];
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid >> 4;
  const int chunk = (int)(gid & 15);
  const bool live = row < rows;
  // row = (b H + h) N + n; 32-bit division (the launcher keeps rows below 2^31)
  const uint32_t r = (uint32_t)(live ? row : rows - 1);
  const int64_t n = r % (uint32_t)N, bh = r / (uint32_t)N;
  const int64_t h = (uint32_t)bh % (uint32_t)H, b = (uint32_t)bh / (uint32_t)H;
  const uint4 v = *reinterpret_cast<const uint4*>(x + b * sB + h * sH + n * sN + chunk * 8);
  const float f[8] = {bf16_lo_f(v.x), bf16_hi_f(v.x), bf16_lo_f(v.y), bf16_hi_f(v.y),
                      bf16_lo_f(v.z), bf16_hi_f(v.z), bf16_lo_f(v.w), bf16_hi_f(v.w)};
  if (mean != nullptr) cu = stage_docs(cu, ndocs, scu);  // uniform condition
  float mm[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (mean != nullptr) {
    const int nd = ndocs > 1 ? ndocs : 1;
    const float* mu = mean + ((bh * nd) + doc_of_token(cu, ndocs, n)) * 128 + chunk * 8;
    const float4 m0 = *reinterpret_cast<const float4*>(mu), m1 = *reinterpret_cast<const float4*>(mu + 4);
    mm[0] = m0.x; mm[1] = m0.y; mm[2] = m0.z; mm[3] = m0.w;
    mm[4] = m1.x; mm[5] = m1.y; mm[6] = m1.z; mm[7] = m1.w;
  }
  float z[8];
  if (hadamard) {
    double y[8];  // x - mu and the butterflies in double (exact for bf16 x, float mu)
#pragma unroll
    for (int j = 0; j < 8; j++) y[j] = (double)f[j] - (double)mm[j];
    // channel c = 8 chunk + j; a butterfly of stride s maps (y[c], y[c+s]) to
    // (y[c] + y[c+s], y[c] - y[c+s]) for c with bit s clear
#pragma unroll
    for (int s = 1; s < 8; s <<= 1)
#pragma unroll
      for (int j = 0; j < 8; j++)
        if ((j & s) == 0) {
          const double a0 = y[j], a1 = y[j + s];
          y[j] = a0 + a1;
          y[j + s] = a0 - a1;
        }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) {
      const bool upper = (chunk & m) != 0;
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const double o = __shfl_xor(y[j], m);
        y[j] = upper ? o - y[j] : y[j] + o;
      }
    }
#pragma unroll
    for (int j = 0; j < 8; j++) z[j] = (float)(y[j] * HADAMARD_C128);
  } else {
    // fl32(x - mu): one correctly rounded float subtraction
#pragma unroll
    for (int j = 0; j < 8; j++) z[j] = f[j] - mm[j];
  }
  float M = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; j++) M = __builtin_fmaxf(M, __builtin_fabsf(z[j]));
  M = __builtin_fmaxf(M, __shfl_xor(M, 1));
  if constexpr (BLOCK == 32) M = __builtin_fmaxf(M, __shfl_xor(M, 2));
  float inv, s;
  const uint32_t sb = pre_block_scale<SCALE>(M, rule, &inv, &s);
  uint32_t w = 0;
  const int e = (int)sb - 127;
  if (SCALE == SCALE_E8M0 && e >= -124 && e < 127) {
    // power-of-two scale away from the ends of the E8M0 range: the scaled FP4 convert
    // (z 2^-e is exact wherever it can round to a nonzero code; round to nearest even,
    // saturation at 6, sign kept, as the encoder below)
    w = pack8_fp4(z, u2f((uint32_t)(e + 127) << 23));
  } else if (SCALE == SCALE_E4M3 && M < __builtin_inff()) {
    // E4M3 scale: fl32(z / s) from the block's correctly rounded reciprocal r by one
    // residual step (q = z r, e = z - s q exactly by FMA, q + e r rounded once:
    // Markstein's division, equal to the IEEE quotient for every float z of every
    // binade whose quotients stay normal), then the scaled FP4 convert at scale 1,
    // with z's sign; a zero scale gives zero quotients
    const float r = s > 0.0f ? 1.0f / s : 0.0f;
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const float q = z[j] * r;
      const float t = __builtin_fmaf(__builtin_fmaf(-q, s, z[j]), r, q);
      y[j] = __builtin_copysignf(s > 0.0f ? t : 0.0f, z[j]);
    }
    w = pack8_fp4(y, 1.0f);
  } else {
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const uint32_t sign = f2u(z[j]) >> 31;
      const float a = __builtin_fabsf(z[j]);
      float q;
      if constexpr (SCALE == SCALE_E8M0) q = a * inv;
      else q = (s == 0.0f) ? 0.0f : a / s;
      w |= (e2m1_mag(q) | (sign << 3)) << (4 * j);
    }
  }
  if (live) {
    codes[row * 16 + chunk] = w;
    if ((chunk & (BLOCK / 8 - 1)) == 0) scales[row * (128 / BLOCK) + chunk / (BLOCK / 8)] = (uint8_t)sb;
  }
}

// ---------------------------------------------------------------------------
// compensation: 16 lanes per key token of KV head (b, hk); for each of the gsz query
// heads of the group, lane partial sums over its 8 channels are combined across the
// 16 lanes in a fixed butterfly order.  delta: [B][Hq][N]
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void center_comp_kernel(const float* __restrict__ qmean,
                                                          const uint16_t* __restrict__ k, int64_t sB, int64_t sH,
                                                          int64_t sN, const float* __restrict__ kmean, int64_t Hq,
                                                          int64_t Hkv, int64_t N, int64_t rows,
                                                          const int32_t* __restrict__ cu, int ndocs,
                                                          float* __restrict__ delta) {
  __shared__ int32_t scu[DOCS_LDS];
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid >> 4;  // (b, hk, token); the 16 lanes of a row are all live or all not
  const int chunk = (int)(gid & 15);
  const bool live = row < rows;
  // row = (b Hkv + hk) N + n; 32-bit division (the launcher keeps rows below 2^31)
  const uint32_t r = (uint32_t)(live ? row : rows - 1);
  const int64_t n = r % (uint32_t)N, bhk = r / (uint32_t)N;
  const int64_t hk = (uint32_t)bhk % (uint32_t)Hkv, b = (uint32_t)bhk / (uint32_t)Hkv;
  const int nd = ndocs > 1 ? ndocs : 1;
  const int doc = doc_of_token(stage_docs(cu, ndocs, scu), ndocs, n);
  const uint4 v = *reinterpret_cast<const uint4*>(k + b * sB + hk * sH + n * sN + chunk * 8);
  const float f[8] = {bf16_lo_f(v.x), bf16_hi_f(v.x), bf16_lo_f(v.y), bf16_hi_f(v.y),
                      bf16_lo_f(v.z), bf16_hi_f(v.z), bf16_lo_f(v.w), bf16_hi_f(v.w)};
  const float* km = kmean + ((bhk * nd) + doc) * 128 + chunk * 8;
  const float4 k0 = *reinterpret_cast<const float4*>(km), k1 = *reinterpret_cast<const float4*>(km + 4);
  const float kk[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
  double kc[8];
#pragma unroll
  for (int j = 0; j < 8; j++) kc[j] = (double)f[j] - (double)kk[j];
  const int64_t gsz = Hq / Hkv;
  for (int64_t g = 0; g < gsz; g++) {
    const int64_t hq = hk * gsz + g;
    const float* qm = qmean + (((b * Hq + hq) * nd) + doc) * 128 + chunk * 8;
    const float4 q0 = *reinterpret_cast<const float4*>(qm), q1 = *reinterpret_cast<const float4*>(qm + 4);
    const float qq[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
    double acc = 0.0;
#pragma unroll
    for (int j = 0; j < 8; j++) acc += (double)qq[j] * kc[j];
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) acc += __shfl_xor(acc, m);
    if (live && chunk == 0) delta[(b * Hq + hq) * N + n] = (float)acc;
  }
}

hipError_t launch_channel_mean(const QuantArgs& a, float* mean, hipStream_t st) {
  const int nd = a.ndocs > 1 ? a.ndocs : 1;
  const int64_t units = a.B * a.H * nd;
  const int64_t wgs = (units + 7) / 8 * 64;
  channel_mean_kernel<<<dim3((unsigned)wgs), 512, 0, st>>>(static_cast<const uint16_t*>(a.x), a.sB, a.sH, a.sN,
                                                           a.H, a.N, a.ndocs > 1 ? a.cu : nullptr, nd, units, mean);
  return hipGetLastError();
}

hipError_t launch_quant_qk_pre(const QuantArgs& a, const float* mean, int hadamard, hipStream_t st) {
  const int64_t rows = a.B * a.H * a.N;
  if (rows >= (int64_t(1) << 31)) return hipErrorInvalidValue;  // 32-bit row indices
  dim3 grid((unsigned)((rows * 16 + 255) / 256));
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  uint32_t* c = static_cast<uint32_t*>(a.codes);
  uint8_t* s = static_cast<uint8_t*>(a.scales);
  const int32_t* cu = a.ndocs > 1 ? a.cu : nullptr;
#define MXQP(S_, B_)                                                                                             \
  quant_qk_pre_kernel<S_, B_><<<grid, 256, 0, st>>>(x, a.sB, a.sH, a.sN, a.H, a.N, rows, a.rule, mean, cu, a.ndocs, \
                                                    hadamard, c, s)
  if (a.scale == SCALE_E8M0 && a.block == 32) MXQP(SCALE_E8M0, 32);
  else if (a.scale == SCALE_E8M0 && a.block == 16) MXQP(SCALE_E8M0, 16);
  else if (a.scale == SCALE_E4M3 && a.block == 16) MXQP(SCALE_E4M3, 16);
  else if (a.scale == SCALE_E4M3 && a.block == 32) MXQP(SCALE_E4M3, 32);
  else return hipErrorInvalidValue;
#undef MXQP
  return hipGetLastError();
}

hipError_t launch_center_comp(const CompArgs& a, hipStream_t st) {
  const int64_t rows = a.B * a.Hkv * a.N;
  if (rows >= (int64_t(1) << 31)) return hipErrorInvalidValue;  // 32-bit row indices
  center_comp_kernel<<<dim3((unsigned)((rows * 16 + 255) / 256)), 256, 0, st>>>(
      a.qmean, static_cast<const uint16_t*>(a.k), a.sB, a.sH, a.sN, a.kmean, a.Hq, a.Hkv, a.N, rows,
      a.ndocs > 1 ? a.cu : nullptr, a.ndocs, a.delta);
  return hipGetLastError();
}

}  // namespace mxattn
