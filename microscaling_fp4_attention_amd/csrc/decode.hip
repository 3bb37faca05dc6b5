// decode.hip -- split-key decode forward on MXFP4 operands (gfx950).
//
// Decode is bound by reading the key/value history, not by the matrix cores, so the
// work is spread over the history ("MpFA", section 5.3: grouped query heads packed
// into the matrix rows, the history cut into fixed partitions with local (m, l, O)
// states, merged by their log-sum-exp):
//   * the partitions are splits of 256 keys, each an online softmax over its two
//     128-key tiles (P quantized per tile as in the prefill kernels);
//   * one workgroup of 4 waves per (request, KV head, 512-key chunk); wave w owns the
//     tile of keys [512 chunk + 128 w, +128), so a split's two tiles run side by side:
//     the wave of the second tile takes the first tile's maximum (through LDS) as its
//     running maximum before its own tile, which quantizes its P exactly as the
//     split's sequential online softmax does, and the two tile states then combine by
//     their log-sum-exp (the same arithmetic as the sequential rescale, up to FP32
//     rounding).  One tile per wave keeps a wave's live registers low, so two
//     workgroups share a CU and more of the history is in flight;
//   * the query heads of the KV head's group and the R newest tokens share the query
//     columns of the MFMA (column c = head (c / R), row (c % R)): up to 16 columns on
//     the 16x16x128 MFMA (whole-row operand reads, below), up to 32 on the 32x32x64;
//   * each wave reads its K and V operands straight from HBM in the MFMA operand
//     layout (no LDS: the waves share no tile); K rows are read in the key order that
//     makes each lane's 16 scores 16 consecutive keys (key_of), so the P codes built in
//     registers are the B operand of the PV product;
//   * the 4 tile states of a chunk are merged by their log-sum-exp in LDS, and a
//     second kernel merges the chunk states of each row the same way.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "device_util.h"
#include "formats.h"
#include "kernels.h"

namespace mxattn {

constexpr int DEC_SPLIT = 256;  // keys per split (the partition of the merge)
constexpr int DEC_CHUNK = 512;  // keys per workgroup: two splits, one tile per wave

// the 4 tile states of a chunk (normalized outputs in `so` as [tile][column][channel],
// rows padded to 129, and log-sum-exps in `slse`), merged by their log-sum-exp into the
// chunk's state in the workspace; thread -> (column tid / 8, 16 channels from 16 (tid % 8))
__device__ __forceinline__ void merge_chunk(const DecArgs& a, const float* so, const float (*slse)[32], int ncol,
                                            int64_t b, int64_t hk, int gsz, int64_t chunk) {
  const int tid = threadIdx.x;
  auto sidx = [&](int w, int c, int ch) { return (w * ncol + c) * 129 + ch; };
  const int cc = tid >> 3, c0 = 16 * (tid & 7);
  if (cc >= ncol) return;
  const int gg = cc / (int)a.R, rr = cc % (int)a.R;
  const int64_t orow = ((b * a.Hq + hk * gsz + gg) * a.R + rr) * a.nsplit + chunk;
  float M = NEG_INF;
#pragma unroll
  for (int w = 0; w < 4; w++) M = fmaxn(M, slse[w][cc]);
  float wt[4], wsum = 0.0f;
#pragma unroll
  for (int w = 0; w < 4; w++) {
    wt[w] = (M == NEG_INF || slse[w][cc] == NEG_INF) ? 0.0f : __expf(slse[w][cc] - M);
    wsum += wt[w];
  }
  const float winv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  float* op = a.ws_o + orow * 128 + c0;
#pragma unroll
  for (int c = 0; c < 16; c += 4) {
    float4 t;
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; u++)
      v[u] = (wt[0] * so[sidx(0, cc, c0 + c + u)] + wt[1] * so[sidx(1, cc, c0 + c + u)] +
              wt[2] * so[sidx(2, cc, c0 + c + u)] + wt[3] * so[sidx(3, cc, c0 + c + u)]) * winv;
    t.x = v[0];
    t.y = v[1];
    t.z = v[2];
    t.w = v[3];
    *reinterpret_cast<float4*>(op + c) = t;
  }
  if ((tid & 7) == 0) a.ws_lse[orow] = wsum > 0.0f ? M + __logf(wsum) : NEG_INF;
}

// VT: V is role VT (tile-major: key tile t of channel c at [t][c], 64 code bytes and 4
// scale bytes), so a tile's V^T is one contiguous run
template <int PMODE, bool VT>
__global__ __launch_bounds__(256, 2) void decode_kernel(DecArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, ql = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t nchunk = (a.N + DEC_CHUNK - 1) / DEC_CHUNK;
  const int64_t chunk = blockIdx.x % nchunk, bhk = blockIdx.x / nchunk;
  const int64_t b = bhk / a.Hkv, hk = bhk % a.Hkv;
  const int gsz = (int)(a.Hq / a.Hkv);
  const int ncol = gsz * (int)a.R;
  const bool cvalid = ql < ncol;
  const int g = cvalid ? ql / (int)a.R : 0, r = cvalid ? ql % (int)a.R : 0;
  const int64_t hq = hk * gsz + g;
  // this wave's tile; a tile at or past the history's end stays empty
  const int kt0 = (int)chunk * DEC_CHUNK + 128 * wave;
  const float lam = a.lambda;
  static_assert(DEC_CHUNK == 4 * 128 && DEC_SPLIT == 2 * 128, "a split is the tiles of waves 2i and 2i + 1");

  // Q operand (B operand of S^T = K Q^T); an absent column reads column 0's row (its
  // scores are masked), so no read waits on a condition
  v8i qop[2];
  uint32_t qsc;
  {
    const int64_t qrow = (b * a.Hq + hq) * a.R + r;
    const uint8_t* qp = a.q + qrow * 64;
    qop[0] = v8_from4(*reinterpret_cast<const u4*>(qp + 16 * hh));
    qop[1] = v8_from4(*reinterpret_cast<const u4*>(qp + 32 + 16 * hh));
    qsc = *reinterpret_cast<const uint32_t*>(a.qs + qrow * 4) >> (8 * hh);
  }
  const uint8_t* kc = a.k + (b * a.Hkv + hk) * a.N * 64;
  const uint8_t* kscl = a.ks + (b * a.Hkv + hk) * a.N * 4;
  const int64_t vrow0 = (b * a.Hkv + hk) * 128;
  const uint32_t np = (uint32_t)a.np;

  // ---- operands of the tile, all requested before any is used (the kernel is bound by
  // these reads, so none of them waits on the history length): MFMA row ql of sub-tile
  // bb reads key kt0 + key_of(bb, (ql>>2)&1, 4(ql>>3) + (ql&3)), keys past N reading row
  // N - 1 (masked); V^T rows are channels 32 db + ql.  The padded key axis of V is a
  // multiple of 128, so a tile's codes and its 4 scale bytes lie inside the row and the
  // scale dword is aligned.
  u4 k0[4], k1[4], v0[4], v1[4];
  uint32_t ks[4], vs[4];
  v16f S[4];
  float bm16[4], tmax = NEG_INF;
  if (kt0 < (int)a.N) {
#pragma unroll
    for (int bb = 0; bb < 4; bb++) {
      int key = kt0 + key_of<false>(bb, (ql >> 2) & 1, 4 * (ql >> 3) + (ql & 3));
      key = key < (int)a.N ? key : (int)a.N - 1;
      const uint8_t* kp = kc + (int64_t)key * 64;
      k0[bb] = *reinterpret_cast<const u4*>(kp + 16 * hh);
      k1[bb] = *reinterpret_cast<const u4*>(kp + 32 + 16 * hh);
      ks[bb] = *reinterpret_cast<const uint32_t*>(kscl + (int64_t)key * 4);
    }
#pragma unroll
    for (int db = 0; db < 4; db++) {
      const int64_t vrow = vrow0 + 32 * db + ql;
      // slot of (tile, channel) in the tile-major form; kt0 < N <= np keeps both forms
      // inside the head's V
      const int64_t tslot = (int64_t)(kt0 / 128) * 128 + 32 * db + ql;
      const uint8_t* vp = VT ? a.v + vrow0 * (np / 2) + tslot * 64 : a.v + vrow * (np / 2) + kt0 / 2;
      v0[db] = *reinterpret_cast<const u4*>(vp + 16 * hh);
      v1[db] = *reinterpret_cast<const u4*>(vp + 32 + 16 * hh);
      vs[db] = *reinterpret_cast<const uint32_t*>(VT ? a.vs + vrow0 * (np / 32) + tslot * 4
                                                     : a.vs + vrow * (np / 32) + kt0 / 32);
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // every read is in flight before the MFMAs
  const int L = a.kv_len != nullptr ? a.kv_len[b] : (int)a.N;
  const int pos = L - (int)a.R + r;  // position of this column's query: keys <= pos are visible
  const bool live = kt0 < L;
  if (live) {
    // ---- S^T = K Q^T, then the mask (absent columns, keys past the history, keys
    // after the query) and the maxima
#pragma unroll
    for (int bb = 0; bb < 4; bb++) {
      const uint32_t ks4 = ks[bb] >> (8 * hh);
      v16f acc = zero16();
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(v8_from4(k0[bb]), qop[0], acc, 4, 4, 0, (int)ks4, 0,
                                                            (int)qsc);
      S[bb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(v8_from4(k1[bb]), qop[1], acc, 4, 4, 2, (int)ks4, 2,
                                                              (int)qsc);
    }
#pragma unroll
    for (int bb = 0; bb < 4; bb++)
#pragma unroll
      for (int j = 0; j < 16; j++) {
        const int key = kt0 + key_of<false>(bb, hh, j);
        S[bb][j] = (cvalid && key <= pos) ? S[bb][j] : NEG_INF;  // pos < L
      }
#pragma unroll
    for (int bb = 0; bb < 4; bb++) {
      float x = S[bb][0];
#pragma unroll
      for (int j = 1; j < 16; j++) x = fmaxn(x, S[bb][j]);
      bm16[bb] = x;
    }
    tmax = halves_max(fmaxn(fmaxn(bm16[0], bm16[1]), fmaxn(bm16[2], bm16[3])));
  }

  // ---- the running maximum before this tile: the split's first tile starts from
  // -inf, its second from the first tile's maximum
  __shared__ float smax[4][32];
  if (hh == 0) smax[wave][ql] = tmax;
  __syncthreads();
  const float m0 = (wave & 1) ? smax[wave - 1][ql] : NEG_INF;

  float m = m0, l = 0.0f, s1 = 1.0f;
  v16f O[4];
#pragma unroll
  for (int i = 0; i < 4; i++) O[i] = zero16();
  if (live) {
    // ---- online softmax step and P quantization (E2M1 with E8M0 per 32 keys); the
    // tile's state starts empty, so nothing carried needs the rescale
    const float mnew = fmaxn(m0, tmax);
    const float ms = mnew == NEG_INF ? 0.0f : mnew * lam;
    const float msub = mnew == NEG_INF ? 0.0f : mnew;
    m = mnew;
    float k1s = 1.0f;
    if constexpr (PMODE == PM_TWO_LEVEL) {
      const float rr = exp2_diff(tmax, msub, lam);
      if (rr >= 0x1p-64f) {
        s1 = rr / 2688.0f;
        k1s = 1.0f / s1;
      } else {
        k1s = 0.0f;  // a tile whose P~ stays below 2^-64 of the running maximum adds nothing
      }
    }
    int e[2];
#pragma unroll
    for (int p = 0; p < 2; p++) {
      const float bm = fmaxn(bm16[2 * p], bm16[2 * p + 1]);
      const int x = e8m0_exp(exp2_diff(bm, msub, lam) * k1s, a.prule);
      e[p] = x < -126 ? -126 : x;
    }
    const uint32_t pscw = (uint32_t)(e[0] + 127) | ((uint32_t)(e[1] + 127) << 8);
    float lsum = 0.0f;
    uint32_t w[8];
#pragma unroll
    for (int bb = 0; bb < 4; bb++) {
      const float sc = u2f((uint32_t)(e[bb >> 1] + 127) << 23);
      float y[16];
#pragma unroll
      for (int j = 0; j < 16; j++) {
        float pt = exp2_hw(__builtin_fmaf(S[bb][j], lam, -ms));
        if constexpr (PMODE != PM_PNQ) lsum += pt;
        if constexpr (PMODE == PM_TWO_LEVEL) pt *= k1s;
        y[j] = pt;
      }
      w[2 * bb] = pack8_fp4(y, sc);
      w[2 * bb + 1] = pack8_fp4(y + 8, sc);
    }
    const v8i bp0 = v8_from4(mk4(w[0], w[1], w[2], w[3]));
    const v8i bp1 = v8_from4(mk4(w[4], w[5], w[6], w[7]));

    // ---- O^T = V^T P^T: channel rows 32 db + ql, keys kt0 + [0, 128) in order
#pragma unroll
    for (int db = 0; db < 4; db++) {
      const uint32_t vs4 = vs[db] >> (8 * hh);
      O[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(v8_from4(v0[db]), bp0, O[db], 4, 4, 0, (int)vs4, 0,
                                                              (int)pscw);
      O[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(v8_from4(v1[db]), bp1, O[db], 4, 4, 2, (int)vs4, 1,
                                                              (int)pscw);
    }
    if constexpr (PMODE == PM_PNQ) {  // row sum of the dequantized P: a block of ones times P^T
      const v8i ones = {0x22222222, 0x22222222, 0x22222222, 0x22222222, 0, 0, 0, 0};
      v16f Lacc = zero16();
      Lacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, bp0, Lacc, 4, 4, 0, 127, 0, (int)pscw);
      Lacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, bp1, Lacc, 4, 4, 0, 127, 1, (int)pscw);
      l = Lacc[0];
    } else {
      l = halves_sum(lsum);
    }
  }

  // ---- the tile's normalized output and log-sum-exp, then the merge of the 4 tile
  // states of this chunk by their log-sum-exp (in LDS) into one state per chunk
  float inv = l > 0.0f ? 1.0f / l : 0.0f;
  if constexpr (PMODE == PM_TWO_LEVEL) inv *= s1;
  // so: [tile][column < ncol][channel] (rows padded to 129), sized by the launch
  extern __shared__ float so[];
  __shared__ float slse[4][32];
  if (cvalid)
#pragma unroll
    for (int db = 0; db < 4; db++)
#pragma unroll
      for (int j = 0; j < 16; j++)
        so[(wave * ncol + ql) * 129 + 32 * db + 8 * (j >> 2) + 4 * hh + (j & 3)] = O[db][j] * inv;
  if (hh == 0) slse[wave][ql] = l > 0.0f ? __logf(l) + m * a.sm_scale : NEG_INF;
  __syncthreads();
  merge_chunk(a, so, slse, ncol, b, hk, gsz, chunk);
}

// The QK4PV8 route ("MpFA", sections 4.1 and 5.3: NVFP4 Q and K, FP8 P and V): the
// same split-key decode, 32 query columns at most, with
//   * S^T = K Q^T on the f16 MFMA after exact dequantization (an E2M1 value times an
//     E4M3 block scale has at most 6 significant bits and lies in [2^-10, 2688]: exact
//     in f16, formed by the FP4-to-f16 convert and one packed multiply per pair); the
//     contraction slot j of lane half h in step s holds channel 64 h + 8 s + j, so a
//     lane reads one contiguous half of each K row (32 code bytes) and its 4 block
//     scales (one dword), and Q the same half (MXFP4 Q and K take the scaled FP4 MFMA
//     instead);
//   * P = E4M3(448 P~) (the oracle's FP8_FIXED), O^T = V^T P^T on the scaled FP8 MFMA
//     with V's E8M0 scale per 32 keys and P's unit scale, the row sum from P~, and O
//     divided by 448 with it; K rows are read in the FP8 operand's key order
//     (key_of<true>), so the P codes built in registers are the PV B operand;
//   * V in role V (channel rows) or VT (tile-major: a tile's 128 channels x 128 bytes
//     one contiguous run).
template <int QK, bool VT>
__global__ __launch_bounds__(256, 2) void decode_q4p8_kernel(DecArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, ql = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t nchunk = (a.N + DEC_CHUNK - 1) / DEC_CHUNK;
  const int64_t chunk = blockIdx.x % nchunk, bhk = blockIdx.x / nchunk;
  const int64_t b = bhk / a.Hkv, hk = bhk % a.Hkv;
  const int gsz = (int)(a.Hq / a.Hkv);
  const int ncol = gsz * (int)a.R;
  const bool cvalid = ql < ncol;
  const int g = cvalid ? ql / (int)a.R : 0, r = cvalid ? ql % (int)a.R : 0;
  const int64_t hq = hk * gsz + g;
  const int kt0 = (int)chunk * DEC_CHUNK + 128 * wave;
  const float lam = a.lambda;
  constexpr int KSB = QK == QK_FP4 ? 4 : 8;  // scale bytes per Q/K row

  // Q operand (B operand of S^T = K Q^T); an absent column reads column 0's row
  v8i qop[2];
  uint32_t qsc = 0;
  v8h qh[8];
  {
    const int64_t qrow = (b * a.Hq + hq) * a.R + r;
    const uint8_t* qp = a.q + qrow * 64;
    if constexpr (QK == QK_FP4) {
      qop[0] = v8_from4(*reinterpret_cast<const u4*>(qp + 16 * hh));
      qop[1] = v8_from4(*reinterpret_cast<const u4*>(qp + 32 + 16 * hh));
      qsc = *reinterpret_cast<const uint32_t*>(a.qs + qrow * 4) >> (8 * hh);
    } else {
      const u4 c0 = *reinterpret_cast<const u4*>(qp + 32 * hh), c1 = *reinterpret_cast<const u4*>(qp + 32 * hh + 16);
      const uint32_t sw = *reinterpret_cast<const uint32_t*>(a.qs + qrow * 8 + 4 * hh);
      const uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
      for (int s = 0; s < 8; s++) {
        const _Float16 sh = (_Float16)e4m3_value((sw >> (8 * (s >> 1))) & 0xFFu);  // exact in f16
        qh[s] = dq8_f16(cw[s], v2h{sh, sh});
      }
    }
  }
  const uint8_t* kc = a.k + (b * a.Hkv + hk) * a.N * 64;
  const uint8_t* kscl = a.ks + (b * a.Hkv + hk) * a.N * KSB;
  const int64_t vrow0 = (b * a.Hkv + hk) * 128;
  const uint32_t np = (uint32_t)a.np;

  // ---- the tile's operands, all requested before any is used: MFMA row ql of
  // sub-tile bb reads key kt0 + key_of<true>(bb, (ql>>2)&1, 4(ql>>3) + (ql&3)), keys
  // past N reading row N - 1 (masked); V^T rows are channels 32 db + ql, one byte per
  // key (np, a multiple of 128, keeps a tile's bytes and its 4 scale bytes in the row)
  u4 k0[4], k1[4], vlo[4][2], vhi[4][2];
  uint32_t ks[4], vs[4];
  v16f S[4];
  float bm16[4], tmax = NEG_INF;
  if (kt0 < (int)a.N) {
#pragma unroll
    for (int bb = 0; bb < 4; bb++) {
      int key = kt0 + key_of<true>(bb, (ql >> 2) & 1, 4 * (ql >> 3) + (ql & 3));
      key = key < (int)a.N ? key : (int)a.N - 1;
      const uint8_t* kp = kc + (int64_t)key * 64;
      if constexpr (QK == QK_FP4) {
        k0[bb] = *reinterpret_cast<const u4*>(kp + 16 * hh);
        k1[bb] = *reinterpret_cast<const u4*>(kp + 32 + 16 * hh);
        ks[bb] = *reinterpret_cast<const uint32_t*>(kscl + (int64_t)key * 4);
      } else {
        k0[bb] = *reinterpret_cast<const u4*>(kp + 32 * hh);
        k1[bb] = *reinterpret_cast<const u4*>(kp + 32 * hh + 16);
        ks[bb] = *reinterpret_cast<const uint32_t*>(kscl + (int64_t)key * 8 + 4 * hh);
      }
    }
#pragma unroll
    for (int db = 0; db < 4; db++) {
      const int64_t vrow = vrow0 + 32 * db + ql;
      // slot of (tile, channel) in the tile-major form (role VT: 128 code bytes each)
      const int64_t tslot = (int64_t)(kt0 / 128) * 128 + 32 * db + ql;
      const uint8_t* vp = VT ? a.v + vrow0 * np + tslot * 128 : a.v + vrow * np + kt0;
#pragma unroll
      for (int kcn = 0; kcn < 2; kcn++) {  // operand element n: key 64 kc + 32 (n / 16) + 16 h + n % 16
        vlo[db][kcn] = *reinterpret_cast<const u4*>(vp + 64 * kcn + 16 * hh);
        vhi[db][kcn] = *reinterpret_cast<const u4*>(vp + 64 * kcn + 32 + 16 * hh);
      }
      vs[db] = *reinterpret_cast<const uint32_t*>(VT ? a.vs + vrow0 * (np / 32) + tslot * 4
                                                     : a.vs + vrow * (np / 32) + kt0 / 32);
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // every read is in flight before the MFMAs
  const int L = a.kv_len != nullptr ? a.kv_len[b] : (int)a.N;
  const int pos = L - (int)a.R + r;  // keys <= pos are visible to this column
  const bool live = kt0 < L;
  if (live) {
#pragma unroll
    for (int bb = 0; bb < 4; bb++) {
      v16f acc = zero16();
      if constexpr (QK == QK_FP4) {
        const uint32_t ks4 = ks[bb] >> (8 * hh);
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(v8_from4(k0[bb]), qop[0], acc, 4, 4, 0, (int)ks4, 0,
                                                              (int)qsc);
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(v8_from4(k1[bb]), qop[1], acc, 4, 4, 2, (int)ks4, 2,
                                                              (int)qsc);
      } else {
        const uint32_t kw[8] = {k0[bb].x, k0[bb].y, k0[bb].z, k0[bb].w, k1[bb].x, k1[bb].y, k1[bb].z, k1[bb].w};
#pragma unroll
        for (int s = 0; s < 8; s++) {
          const _Float16 sk = (_Float16)e4m3_value((ks[bb] >> (8 * (s >> 1))) & 0xFFu);
          acc = mfma_f16(dq8_f16(kw[s], v2h{sk, sk}), qh[s], acc);
        }
      }
      S[bb] = acc;
    }
#pragma unroll
    for (int bb = 0; bb < 4; bb++)
#pragma unroll
      for (int j = 0; j < 16; j++) {
        const int key = kt0 + key_of<true>(bb, hh, j);
        S[bb][j] = (cvalid && key <= pos) ? S[bb][j] : NEG_INF;  // pos < L
      }
#pragma unroll
    for (int bb = 0; bb < 4; bb++) {
      float x = S[bb][0];
#pragma unroll
      for (int j = 1; j < 16; j++) x = fmaxn(x, S[bb][j]);
      bm16[bb] = x;
    }
    tmax = halves_max(fmaxn(fmaxn(bm16[0], bm16[1]), fmaxn(bm16[2], bm16[3])));
  }

  // ---- the running maximum before this tile (the split's second tile starts from
  // the first tile's maximum)
  __shared__ float smax[4][32];
  if (hh == 0) smax[wave][ql] = tmax;
  __syncthreads();
  const float m0 = (wave & 1) ? smax[wave - 1][ql] : NEG_INF;

  float m = m0, l = 0.0f;
  v16f O[4];
#pragma unroll
  for (int i = 0; i < 4; i++) O[i] = zero16();
  if (live) {
    const float mnew = fmaxn(m0, tmax);
    const float ms = mnew == NEG_INF ? 0.0f : mnew * lam;
    m = mnew;
    float lsum = 0.0f;
    v8i bp[2];
#pragma unroll
    for (int bb = 0; bb < 4; bb++)
#pragma unroll
      for (int dw = 0; dw < 4; dw++) {  // c = E4M3(448 P~), four codes per dword
        float y[4];
#pragma unroll
        for (int u = 0; u < 4; u++) {
          y[u] = exp2_hw(__builtin_fmaf(S[bb][4 * dw + u], lam, -ms));
          lsum += y[u];
        }
        int x = __builtin_amdgcn_cvt_pk_fp8_f32(448.0f * y[0], 448.0f * y[1], 0, false);
        x = __builtin_amdgcn_cvt_pk_fp8_f32(448.0f * y[2], 448.0f * y[3], x, true);
        bp[bb >> 1][4 * (bb & 1) + dw] = x;
      }
#pragma unroll
    for (int db = 0; db < 4; db++) {
      const uint32_t vs4 = vs[db] >> (8 * hh);
#pragma unroll
      for (int kcn = 0; kcn < 2; kcn++) {
        const u4 lo = vlo[db][kcn], hi = vhi[db][kcn];
        const v8i av = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        if (kcn == 0)
          O[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bp[0], O[db], 0, 0, 0, (int)vs4, 0, 127);
        else
          O[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bp[1], O[db], 0, 0, 2, (int)vs4, 0, 127);
      }
    }
    l = halves_sum(lsum);
  }

  // ---- the tile's normalized output (O / 448 / l) and log-sum-exp, merged per chunk
  const float inv = l > 0.0f ? 1.0f / l / 448.0f : 0.0f;
  extern __shared__ float so[];
  __shared__ float slse[4][32];
  if (cvalid)
#pragma unroll
    for (int db = 0; db < 4; db++)
#pragma unroll
      for (int j = 0; j < 16; j++)
        so[(wave * ncol + ql) * 129 + 32 * db + 8 * (j >> 2) + 4 * hh + (j & 3)] = O[db][j] * inv;
  if (hh == 0) slse[wave][ql] = l > 0.0f ? __logf(l) + m * a.sm_scale : NEG_INF;
  __syncthreads();
  merge_chunk(a, so, slse, ncol, b, hk, gsz, chunk);
}

typedef float v4f __attribute__((ext_vector_type(4)));

// The same decode for up to 16 query columns on the 16x16x128 block-scaled MFMA.  A
// 16-row operand holds each row's 128 contraction elements in four 16-byte blocks, one
// per quarter of the wave (lane l: row l % 16, block l / 16), so one 16-byte load per
// lane covers 16 whole 64-byte rows: the K rows of a sub-tile and the V^T channel rows
// are read as whole rows, where the 32-column form reads half of each of 32 rows.
//   * S^T = K Q^T per 16-key sub-tile st (8 per tile): MFMA row r reads key
//     32 (r / 4) + 4 st + r % 4 of the tile, so the lane of (column c, row group g)
//     holds the scores of the 32 consecutive keys [32 g, 32 g + 32) over the 8
//     sub-tiles (element 4 st + i is key 32 g + 4 st + i): one 32-key P block per lane,
//     whose maximum needs no other lane, and whose codes are the lane's B operand of
//     O^T = V^T P^T (block g of column c);
//   * K rows of a sub-tile come in four runs of 4 consecutive keys (256 contiguous
//     bytes each), V^T channel rows in one 1 KB run (tile-major) or 16 runs of 64 B.
template <int PMODE, bool VT>
__global__ __launch_bounds__(256, 2) void decode16_kernel(DecArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, qc = lane & 15, kb = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t nchunk = (a.N + DEC_CHUNK - 1) / DEC_CHUNK;
  const int64_t chunk = blockIdx.x % nchunk, bhk = blockIdx.x / nchunk;
  const int64_t b = bhk / a.Hkv, hk = bhk % a.Hkv;
  const int gsz = (int)(a.Hq / a.Hkv);
  const int ncol = gsz * (int)a.R;  // <= 16
  const bool cvalid = qc < ncol;
  const int g = cvalid ? qc / (int)a.R : 0, r = cvalid ? qc % (int)a.R : 0;
  const int64_t hq = hk * gsz + g;
  const int kt0 = (int)chunk * DEC_CHUNK + 128 * wave;
  const float lam = a.lambda;

  // Q operand (B of S^T = K Q^T): column qc, channel block kb; an absent column reads
  // column 0's row (its scores are masked)
  v8i qop;
  uint32_t qsc;
  {
    const int64_t qrow = (b * a.Hq + hq) * a.R + r;
    qop = v8_from4(*reinterpret_cast<const u4*>(a.q + qrow * 64 + 16 * kb));
    qsc = *reinterpret_cast<const uint32_t*>(a.qs + qrow * 4) >> (8 * kb);
  }
  const uint8_t* kc = a.k + (b * a.Hkv + hk) * a.N * 64;
  const uint8_t* kscl = a.ks + (b * a.Hkv + hk) * a.N * 4;
  const int64_t vrow0 = (b * a.Hkv + hk) * 128;
  const uint32_t np = (uint32_t)a.np;

  // ---- every operand of the tile requested before any is used; keys past N read row
  // N - 1 (masked).  The padded key axis of V is a multiple of 128, so a tile's V codes
  // and its 4 scale bytes lie inside the row and the scale dword is aligned.
  u4 kq[8], vq[8];
  uint32_t ks[8], vs[8];
  if (kt0 < (int)a.N) {
#pragma unroll
    for (int st = 0; st < 8; st++) {
      int key = kt0 + 32 * (qc >> 2) + 4 * st + (qc & 3);
      key = key < (int)a.N ? key : (int)a.N - 1;
      kq[st] = *reinterpret_cast<const u4*>(kc + (int64_t)key * 64 + 16 * kb);
      ks[st] = *reinterpret_cast<const uint32_t*>(kscl + (int64_t)key * 4);
    }
#pragma unroll
    for (int db = 0; db < 8; db++) {
      const int64_t vrow = vrow0 + 16 * db + qc;
      // slot of (tile, channel) in the tile-major form; kt0 < N <= np keeps both forms
      // inside the head's V
      const int64_t tslot = (int64_t)(kt0 / 128) * 128 + 16 * db + qc;
      const uint8_t* vp = VT ? a.v + vrow0 * (np / 2) + tslot * 64 : a.v + vrow * (np / 2) + kt0 / 2;
      vq[db] = *reinterpret_cast<const u4*>(vp + 16 * kb);
      vs[db] = *reinterpret_cast<const uint32_t*>(VT ? a.vs + vrow0 * (np / 32) + tslot * 4
                                                     : a.vs + vrow * (np / 32) + kt0 / 32);
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // every read is in flight before the MFMAs
  const int L = a.kv_len != nullptr ? a.kv_len[b] : (int)a.N;
  const int pos = L - (int)a.R + r;  // keys <= pos are visible to this column's query
  const bool live = kt0 < L;
  float y[32];  // the lane's 32 scores, key kt0 + 32 kb + j
  float bmax = NEG_INF, tmax = NEG_INF;
  if (live) {
#pragma unroll
    for (int st = 0; st < 8; st++) {
      v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(v8_from4(kq[st]), qop, acc, 4, 4, 0,
                                                             (int)(ks[st] >> (8 * kb)), 0, (int)qsc);
#pragma unroll
      for (int i = 0; i < 4; i++) y[4 * st + i] = acc[i];
    }
#pragma unroll
    for (int j = 0; j < 32; j++) {
      const int key = kt0 + 32 * kb + j;
      y[j] = (cvalid && key <= pos) ? y[j] : NEG_INF;  // pos < L
      bmax = fmaxn(bmax, y[j]);
    }
    tmax = fmaxn(bmax, __shfl_xor(bmax, 16));
    tmax = fmaxn(tmax, __shfl_xor(tmax, 32));
  }

  // ---- the running maximum before this tile: the split's first tile starts from
  // -inf, its second from the first tile's maximum
  __shared__ float smax[4][32];
  if (kb == 0) smax[wave][qc] = tmax;
  __syncthreads();
  const float m0 = (wave & 1) ? smax[wave - 1][qc] : NEG_INF;

  float m = m0, l = 0.0f, s1 = 1.0f;
  v4f O[8];
#pragma unroll
  for (int i = 0; i < 8; i++) O[i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  if (live) {
    // ---- online softmax step and P quantization (E2M1, one E8M0 scale per lane's
    // 32-key block); the tile's state starts empty, so nothing needs the rescale
    const float mnew = fmaxn(m0, tmax);
    const float ms = mnew == NEG_INF ? 0.0f : mnew * lam;
    const float msub = mnew == NEG_INF ? 0.0f : mnew;
    m = mnew;
    float k1s = 1.0f;
    if constexpr (PMODE == PM_TWO_LEVEL) {
      const float rr = exp2_diff(tmax, msub, lam);
      if (rr >= 0x1p-64f) {
        s1 = rr / 2688.0f;
        k1s = 1.0f / s1;
      } else {
        k1s = 0.0f;  // a tile whose P~ stays below 2^-64 of the running maximum adds nothing
      }
    }
    int e = e8m0_exp(exp2_diff(bmax, msub, lam) * k1s, a.prule);
    e = e < -126 ? -126 : e;
    const float sc = u2f((uint32_t)(e + 127) << 23);
    float lsum = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; j++) {
      float pt = exp2_hw(__builtin_fmaf(y[j], lam, -ms));
      if constexpr (PMODE != PM_PNQ) lsum += pt;
      if constexpr (PMODE == PM_TWO_LEVEL) pt *= k1s;
      y[j] = pt;
    }
    const v8i bp = v8_from4(mk4(pack8_fp4(y, sc), pack8_fp4(y + 8, sc), pack8_fp4(y + 16, sc), pack8_fp4(y + 24, sc)));
    const int psc = e + 127;

    // ---- O^T = V^T P^T: channel rows 16 db + qc, keys kt0 + [0, 128) in order
#pragma unroll
    for (int db = 0; db < 8; db++)
      O[db] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(v8_from4(vq[db]), bp, O[db], 4, 4, 0,
                                                               (int)(vs[db] >> (8 * kb)), 0, psc);
    if constexpr (PMODE == PM_PNQ) {  // row sum of the dequantized P: a block of ones times P^T
      const v8i ones = {0x22222222, 0x22222222, 0x22222222, 0x22222222, 0, 0, 0, 0};
      v4f Lacc = {0.0f, 0.0f, 0.0f, 0.0f};
      Lacc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, bp, Lacc, 4, 4, 0, 127, 0, psc);
      l = Lacc[0];
    } else {
      lsum += __shfl_xor(lsum, 16);
      l = lsum + __shfl_xor(lsum, 32);
    }
  }

  // ---- the tile's normalized output and log-sum-exp, then the chunk merge
  float inv = l > 0.0f ? 1.0f / l : 0.0f;
  if constexpr (PMODE == PM_TWO_LEVEL) inv *= s1;
  extern __shared__ float so[];  // [tile][column < ncol][channel], rows padded to 129
  __shared__ float slse[4][32];
  if (cvalid)
#pragma unroll
    for (int db = 0; db < 8; db++)
#pragma unroll
      for (int i = 0; i < 4; i++) so[(wave * ncol + qc) * 129 + 16 * db + 4 * kb + i] = O[db][i] * inv;
  if (kb == 0) slse[wave][qc] = l > 0.0f ? __logf(l) + m * a.sm_scale : NEG_INF;
  __syncthreads();
  merge_chunk(a, so, slse, ncol, b, hk, gsz, chunk);
}

// The QK4PV8 decode ("MpFA", sections 4.1 and 5.3) for up to 16 query columns, in the
// lane layout of decode16_kernel (lane l: column or operand row l % 16, contraction
// block l / 16), which halves the score and output accumulators of the 32-column form,
// so more waves (and more of the history) are in flight:
//   * an 8-bit operand of the 16x16x128 MFMA gives the lane of block g (lane / 16)
//     elements n = 0..31 at contraction index 64 (n / 16) + 16 g + n % 16, and the E8M0
//     scale of block g covers indices [32 g, 32 g + 32).  With the key as the index, a
//     lane's V^T row holds keys 16 g + [0, 16) and 64 + 16 g + [0, 16) (two 16-byte
//     reads) and the scale of V's block g is the lane's own;
//   * S^T = K Q^T per 16-key sub-tile st (8 per tile), MFMA row r reading key
//     64 (st / 4) + 16 (r / 4) + 4 (st % 4) + r % 4, so the lane of (column c, block g)
//     holds, as element n = 4 st + i, the score of key 64 (n / 16) + 16 g + n % 16: the
//     keys of its own P operand elements, whose codes need no other lane.  NVFP4 Q and
//     K run on the f16 16x16x32 MFMA after exact dequantization: in step s the 8
//     contraction slots of block g hold channels 32 g + 8 s + [0, 8), so a lane reads 16
//     contiguous code bytes of its K row and the two E4M3 scales that cover them; MXFP4
//     Q and K take the scaled FP4 16x16x128 MFMA;
//   * O^T = V^T P^T on the scaled FP8 MFMA with P = E4M3(448 P~) and P's unit scale.
template <int QK, bool VT>
__global__ __launch_bounds__(256, 2) void decode16_q4p8_kernel(DecArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, qc = lane & 15, kb = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t nchunk = (a.N + DEC_CHUNK - 1) / DEC_CHUNK;
  const int64_t chunk = blockIdx.x % nchunk, bhk = blockIdx.x / nchunk;
  const int64_t b = bhk / a.Hkv, hk = bhk % a.Hkv;
  const int gsz = (int)(a.Hq / a.Hkv);
  const int ncol = gsz * (int)a.R;  // <= 16
  const bool cvalid = qc < ncol;
  const int g = cvalid ? qc / (int)a.R : 0, r = cvalid ? qc % (int)a.R : 0;
  const int64_t hq = hk * gsz + g;
  const int kt0 = (int)chunk * DEC_CHUNK + 128 * wave;
  const float lam = a.lambda;
  constexpr int KSB = QK == QK_FP4 ? 4 : 8;  // scale bytes per Q/K row

  // Q operand (B of S^T = K Q^T): column qc, channels [32 kb, 32 kb + 32); an absent
  // column reads column 0's row (its scores are masked)
  v8i qop = {0, 0, 0, 0, 0, 0, 0, 0};
  uint32_t qsc = 0;
  v8h qh[4];
  {
    const int64_t qrow = (b * a.Hq + hq) * a.R + r;
    const u4 c = *reinterpret_cast<const u4*>(a.q + qrow * 64 + 16 * kb);
    if constexpr (QK == QK_FP4) {
      qop = v8_from4(c);
      qsc = *reinterpret_cast<const uint32_t*>(a.qs + qrow * 4) >> (8 * kb);
    } else {
      const uint32_t sw = *reinterpret_cast<const uint32_t*>(a.qs + qrow * 8 + 4 * (kb >> 1)) >> (16 * (kb & 1));
      const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
      for (int s = 0; s < 4; s++) {
        const _Float16 sh = (_Float16)e4m3_value((sw >> (8 * (s >> 1))) & 0xFFu);  // exact in f16
        qh[s] = dq8_f16(cw[s], v2h{sh, sh});
      }
    }
  }
  const uint8_t* kc = a.k + (b * a.Hkv + hk) * a.N * 64;
  const uint8_t* kscl = a.ks + (b * a.Hkv + hk) * a.N * KSB;
  const int64_t vrow0 = (b * a.Hkv + hk) * 128;
  const uint32_t np = (uint32_t)a.np;

  // ---- every operand of the tile requested before any is used; keys past N read row
  // N - 1 (masked).  V has one byte per key and np is a multiple of 128, so a tile's
  // bytes and its 4 scale bytes lie inside the row and the scale dword is aligned.
  u4 kq[8], vlo[8], vhi[8];
  uint32_t ks[8], vs[8];
  if (kt0 < (int)a.N) {
#pragma unroll
    for (int st = 0; st < 8; st++) {
      int key = kt0 + 64 * (st >> 2) + 16 * (qc >> 2) + 4 * (st & 3) + (qc & 3);
      key = key < (int)a.N ? key : (int)a.N - 1;
      kq[st] = *reinterpret_cast<const u4*>(kc + (int64_t)key * 64 + 16 * kb);
      if constexpr (QK == QK_FP4) ks[st] = *reinterpret_cast<const uint32_t*>(kscl + (int64_t)key * 4) >> (8 * kb);
      else ks[st] = *reinterpret_cast<const uint32_t*>(kscl + (int64_t)key * 8 + 4 * (kb >> 1)) >> (16 * (kb & 1));
    }
#pragma unroll
    for (int db = 0; db < 8; db++) {
      const int64_t vrow = vrow0 + 16 * db + qc;
      // slot of (tile, channel) in the tile-major form (role VT: 128 code bytes each)
      const int64_t tslot = (int64_t)(kt0 / 128) * 128 + 16 * db + qc;
      const uint8_t* vp = (VT ? a.v + vrow0 * np + tslot * 128 : a.v + vrow * np + kt0) + 16 * kb;
      vlo[db] = *reinterpret_cast<const u4*>(vp);
      vhi[db] = *reinterpret_cast<const u4*>(vp + 64);
      vs[db] = *reinterpret_cast<const uint32_t*>(VT ? a.vs + vrow0 * (np / 32) + tslot * 4
                                                     : a.vs + vrow * (np / 32) + kt0 / 32) >> (8 * kb);
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // every read is in flight before the MFMAs
  const int L = a.kv_len != nullptr ? a.kv_len[b] : (int)a.N;
  const int pos = L - (int)a.R + r;  // keys <= pos are visible to this column's query
  const bool live = kt0 < L;
  float y[32];  // the lane's 32 scores, key kt0 + 64 (j / 16) + 16 kb + j % 16
  float tmax = NEG_INF;
  if (live) {
#pragma unroll
    for (int st = 0; st < 8; st++) {
      v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (QK == QK_FP4) {
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(v8_from4(kq[st]), qop, acc, 4, 4, 0, (int)ks[st], 0,
                                                               (int)qsc);
      } else {
        const uint32_t kw[4] = {kq[st].x, kq[st].y, kq[st].z, kq[st].w};
#pragma unroll
        for (int s = 0; s < 4; s++) {
          const _Float16 sk = (_Float16)e4m3_value((ks[st] >> (8 * (s >> 1))) & 0xFFu);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(dq8_f16(kw[s], v2h{sk, sk}), qh[s], acc, 0, 0, 0);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; i++) y[4 * st + i] = acc[i];
    }
    float bmax = NEG_INF;
#pragma unroll
    for (int j = 0; j < 32; j++) {
      const int key = kt0 + 64 * (j >> 4) + 16 * kb + (j & 15);
      y[j] = (cvalid && key <= pos) ? y[j] : NEG_INF;  // pos < L
      bmax = fmaxn(bmax, y[j]);
    }
    tmax = fmaxn(bmax, __shfl_xor(bmax, 16));
    tmax = fmaxn(tmax, __shfl_xor(tmax, 32));
  }

  // ---- the running maximum before this tile: the split's first tile starts from
  // -inf, its second from the first tile's maximum
  __shared__ float smax[4][32];
  if (kb == 0) smax[wave][qc] = tmax;
  __syncthreads();
  const float m0 = (wave & 1) ? smax[wave - 1][qc] : NEG_INF;

  float m = m0, l = 0.0f;
  v4f O[8];
#pragma unroll
  for (int i = 0; i < 8; i++) O[i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  if (live) {
    // ---- P = E4M3(448 P~), element n (byte n % 4 of dword n / 4) for score n; the row
    // sum from P~
    const float mnew = fmaxn(m0, tmax);
    const float ms = mnew == NEG_INF ? 0.0f : mnew * lam;
    m = mnew;
    float lsum = 0.0f;
    v8i bp;
#pragma unroll
    for (int dw = 0; dw < 8; dw++) {
      float p4[4];
#pragma unroll
      for (int u = 0; u < 4; u++) {
        p4[u] = exp2_hw(__builtin_fmaf(y[4 * dw + u], lam, -ms));
        lsum += p4[u];
      }
      int x = __builtin_amdgcn_cvt_pk_fp8_f32(448.0f * p4[0], 448.0f * p4[1], 0, false);
      x = __builtin_amdgcn_cvt_pk_fp8_f32(448.0f * p4[2], 448.0f * p4[3], x, true);
      bp[dw] = x;
    }

    // ---- O^T = V^T P^T: channel rows 16 db + qc, keys kt0 + [0, 128)
#pragma unroll
    for (int db = 0; db < 8; db++) {
      const v8i av = {(int)vlo[db].x, (int)vlo[db].y, (int)vlo[db].z, (int)vlo[db].w,
                      (int)vhi[db].x, (int)vhi[db].y, (int)vhi[db].z, (int)vhi[db].w};
      O[db] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bp, O[db], 0, 0, 0, (int)vs[db], 0, 127);
    }
    lsum += __shfl_xor(lsum, 16);
    l = lsum + __shfl_xor(lsum, 32);
  }

  // ---- the tile's normalized output (O / 448 / l) and log-sum-exp, merged per chunk
  const float inv = l > 0.0f ? 1.0f / l / 448.0f : 0.0f;
  extern __shared__ float so[];  // [tile][column < ncol][channel], rows padded to 129
  __shared__ float slse[4][32];
  if (cvalid)
#pragma unroll
    for (int db = 0; db < 8; db++)
#pragma unroll
      for (int i = 0; i < 4; i++) so[(wave * ncol + qc) * 129 + 16 * db + 4 * kb + i] = O[db][i] * inv;
  if (kb == 0) slse[wave][qc] = l > 0.0f ? __logf(l) + m * a.sm_scale : NEG_INF;
  __syncthreads();
  merge_chunk(a, so, slse, ncol, b, hk, gsz, chunk);
}

// merge of the chunk states of one (request, query head, row) by their log-sum-exp.
// Workgroup = (row, quarter of the 128 channels); its 8 groups of 32 threads (thread =
// channel) take every 8th chunk in one pass, 8 chunk states in flight, keeping a running
// maximum (the weights of earlier chunks rescaled when it grows); the groups' states
// are then combined in a fixed order in LDS (deterministic).
constexpr int MERGE_GROUPS = 8;
constexpr int MERGE_BATCH = 8;  // chunk states in flight per thread
__global__ __launch_bounds__(256) void decode_merge_kernel(DecArgs a) {
  const int64_t row = blockIdx.x >> 2;  // (b, hq, r)
  const int cq = blockIdx.x & 3;
  const int64_t r = row % a.R, bh = row / a.R, hq = bh % a.Hq, b = bh / a.Hq;
  const int c = 32 * cq + (threadIdx.x & 31), grp = threadIdx.x >> 5;
  const int L = a.kv_len != nullptr ? a.kv_len[b] : (int)a.N;
  // chunks holding keys of this request (a length beyond N reads no state past the N keys)
  int64_t ns = ((int64_t)L + DEC_CHUNK - 1) / DEC_CHUNK;
  ns = ns < a.nsplit ? ns : a.nsplit;
  const float* lses = a.ws_lse + row * a.nsplit;
  const float* outs = a.ws_o + row * a.nsplit * 128 + c;
  __shared__ float red[MERGE_GROUPS][32];
  __shared__ float gmax[MERGE_GROUPS], gsum[MERGE_GROUPS];
  float M = NEG_INF, acc = 0.0f, wsum = 0.0f;
  for (int64_t s0 = grp; s0 < ns; s0 += MERGE_GROUPS * MERGE_BATCH) {
    float ls[MERGE_BATCH], ov[MERGE_BATCH];
#pragma unroll
    for (int u = 0; u < MERGE_BATCH; u++) {  // every read issued before any is used
      const int64_t s = s0 + MERGE_GROUPS * u;
      const bool in = s < ns;
      ls[u] = in ? lses[s] : NEG_INF;
      ov[u] = in ? outs[s * 128] : 0.0f;
    }
    float Mn = M;
#pragma unroll
    for (int u = 0; u < MERGE_BATCH; u++) Mn = fmaxn(Mn, ls[u]);
    if (Mn != NEG_INF) {
      const float k = M == NEG_INF ? 0.0f : __expf(M - Mn);
      acc *= k;
      wsum *= k;
#pragma unroll
      for (int u = 0; u < MERGE_BATCH; u++) {
        const float w = ls[u] == NEG_INF ? 0.0f : __expf(ls[u] - Mn);
        wsum += w;
        acc += w * ov[u];
      }
      M = Mn;
    }
  }
  red[grp][threadIdx.x & 31] = acc;
  if ((threadIdx.x & 31) == 0) {
    gmax[grp] = M;
    gsum[grp] = wsum;
  }
  __syncthreads();
  if (grp != 0) return;
  float Mall = NEG_INF;
#pragma unroll
  for (int g = 0; g < MERGE_GROUPS; g++) Mall = fmaxn(Mall, gmax[g]);
  float ws_all = 0.0f, o = 0.0f;
  if (Mall != NEG_INF) {
#pragma unroll
    for (int g = 0; g < MERGE_GROUPS; g++) {  // fixed order: deterministic
      const float k = gmax[g] == NEG_INF ? 0.0f : __expf(gmax[g] - Mall);
      ws_all += k * gsum[g];
      o += k * red[g][threadIdx.x & 31];
    }
  }
  o = ws_all > 0.0f ? o / ws_all : 0.0f;
  if (a.out_fp32) {
    static_cast<float*>(a.out)[b * a.oB + hq * a.oH + r * a.oN + c] = o;
  } else {
    static_cast<uint16_t*>(a.out)[b * a.oB + hq * a.oH + r * a.oN + c] = (uint16_t)bf16_rne(o);
  }
  if (a.lse != nullptr && cq == 0 && threadIdx.x == 0) a.lse[row] = ws_all > 0.0f ? Mall + __logf(ws_all) : NEG_INF;
}

hipError_t launch_decode(int pmode, const DecArgs& a, hipStream_t st) {
  const int64_t nchunk = (a.N + DEC_CHUNK - 1) / DEC_CHUNK;
  const dim3 grid((unsigned)(a.B * a.Hkv * nchunk));
  // the merge buffer holds the 4 tile outputs of the packed columns only
  const size_t shm = (size_t)4 * (size_t)((a.Hq / a.Hkv) * a.R) * 129 * sizeof(float);
  auto run = [&](auto kern) -> hipError_t {
    if (shm > 65536) {  // 32 columns need 66 KB of the 160 KB of LDS
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
      if (e != hipSuccess) return e;
    }
    kern<<<grid, 256, shm, st>>>(a);
    return hipSuccess;
  };
  // up to 16 query columns: the 16-column form, which reads whole K and V rows
  auto pick = [&](auto k32, auto k16) { return (a.Hq / a.Hkv) * a.R <= 16 ? run(k16) : run(k32); };
  hipError_t e0;
  const bool vt = a.vtiled != 0;
  if (pmode == PM_FP8_FIXED) {  // QK4PV8: an FP8 V, 32 columns at most
    if (vt)
      e0 = a.qk_fp4 ? pick(decode_q4p8_kernel<QK_FP4, true>, decode16_q4p8_kernel<QK_FP4, true>)
                    : pick(decode_q4p8_kernel<QK_BF16, true>, decode16_q4p8_kernel<QK_BF16, true>);
    else
      e0 = a.qk_fp4 ? pick(decode_q4p8_kernel<QK_FP4, false>, decode16_q4p8_kernel<QK_FP4, false>)
                    : pick(decode_q4p8_kernel<QK_BF16, false>, decode16_q4p8_kernel<QK_BF16, false>);
  } else if (pmode == PM_DIRECT)
    e0 = vt ? pick(decode_kernel<PM_DIRECT, true>, decode16_kernel<PM_DIRECT, true>)
            : pick(decode_kernel<PM_DIRECT, false>, decode16_kernel<PM_DIRECT, false>);
  else if (pmode == PM_PNQ)
    e0 = vt ? pick(decode_kernel<PM_PNQ, true>, decode16_kernel<PM_PNQ, true>)
            : pick(decode_kernel<PM_PNQ, false>, decode16_kernel<PM_PNQ, false>);
  else if (pmode == PM_TWO_LEVEL)
    e0 = vt ? pick(decode_kernel<PM_TWO_LEVEL, true>, decode16_kernel<PM_TWO_LEVEL, true>)
            : pick(decode_kernel<PM_TWO_LEVEL, false>, decode16_kernel<PM_TWO_LEVEL, false>);
  else return hipErrorNotSupported;
  if (e0 != hipSuccess) return e0;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  decode_merge_kernel<<<dim3((unsigned)(a.B * a.Hq * a.R * 4)), 256, 0, st>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free decode (mxattn_decode_noalloc): the split states of a
// call live in this file-scope array instead of a caller workspace.  Each GPU holds
// its own copy until the process ends, at its own address; on the host the array's
// name is not a device address, so host code uses only what hipGetSymbolAddress
// returns for the current device.  Every call on one GPU shares the array: calls that
// overlap (other streams, other threads) race.  The decode writes every split state
// before the merge reads it, so nothing needs clearing between calls.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[DECODE_SCRATCH_BYTES];

hipError_t decode_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace mxattn
