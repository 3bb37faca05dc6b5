// decode.hip -- split-key decode forward on MXFP4 operands (gfx950).
//
// Decode is bound by reading the key/value history, not by the matrix cores, so the
// work is spread over the history ("MpFA", section 5.3: grouped query heads packed
// into the matrix rows, the history cut into fixed partitions with local (m, l, O)
// states, merged by their log-sum-exp):
//   * one workgroup of 4 waves per (request, KV head, 1024-key chunk); wave w owns the
//     split of keys [256 (4 chunk + w), +256) and runs the online softmax over its two
//     128-key tiles with its own running maximum (P quantized per tile as in the
//     prefill kernels);
//   * the query heads of the KV head's group and the R newest tokens share the 32
//     query columns of the MFMA (column c = head (c / R), row (c % R));
//   * each wave reads its K and V operands straight from HBM in the MFMA operand
//     layout (no LDS: the waves share no tile); K rows are read in the key order that
//     makes each lane's 16 scores 16 consecutive keys (key_of), so the P codes built in
//     registers are the B operand of the PV product;
//   * the 4 split states of a chunk are merged by their log-sum-exp in LDS, and a
//     second kernel merges the chunk states of each row the same way.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_util.h"
#include "formats.h"
#include "kernels.h"

namespace mxattn {

constexpr int DEC_SPLIT = 256;  // keys per split (per wave)

template <int PMODE>
__global__ __launch_bounds__(256) void decode_kernel(DecArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, ql = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t nchunk = (a.N + 1023) / 1024;
  const int64_t chunk = blockIdx.x % nchunk, bhk = blockIdx.x / nchunk;
  const int64_t b = bhk / a.Hkv, hk = bhk % a.Hkv;
  const int64_t s = chunk * 4 + wave;  // split of this wave
  const int L = a.kv_len != nullptr ? a.kv_len[b] : (int)a.N;
  const int gsz = (int)(a.Hq / a.Hkv);
  const int ncol = gsz * (int)a.R;
  const bool cvalid = ql < ncol;
  const int g = cvalid ? ql / (int)a.R : 0, r = cvalid ? ql % (int)a.R : 0;
  const int64_t hq = hk * gsz + g;
  const int pos = L - (int)a.R + r;  // position of this column's query: keys <= pos are visible
  const int64_t wrow = ((b * a.Hq + hq) * a.R + r) * a.nsplit + chunk;  // this chunk's state
  const int k0 = (int)s * DEC_SPLIT;  // a split at or past the history's end stays empty
  const float lam = a.lambda;

  // Q operand (B operand of S^T = K Q^T); absent columns are zero codes
  v8i qop[2];
  uint32_t qsc = 0x7F7F7F7Fu;
  {
    const int64_t qrow = (b * a.Hq + hq) * a.R + r;
    const uint8_t* qp = a.q + qrow * 64;
    u4 z = {0, 0, 0, 0};
    qop[0] = v8_from4(cvalid ? *reinterpret_cast<const u4*>(qp + 16 * hh) : z);
    qop[1] = v8_from4(cvalid ? *reinterpret_cast<const u4*>(qp + 32 + 16 * hh) : z);
    if (cvalid) qsc = *reinterpret_cast<const uint32_t*>(a.qs + qrow * 4) >> (8 * hh);
  }
  const uint8_t* kc = a.k + (b * a.Hkv + hk) * a.N * 64;
  const uint8_t* kscl = a.ks + (b * a.Hkv + hk) * a.N * 4;
  const int64_t vrow0 = (b * a.Hkv + hk) * 128;
  const uint32_t np = (uint32_t)a.np;

  float m = NEG_INF, lpart = 0.0f, s1prev = 1.0f;
  v16f O[4], Lacc, S[4];
#pragma unroll
  for (int i = 0; i < 4; i++) O[i] = zero16();
  Lacc = zero16();
  v8i bp[2];
  uint32_t pscw = 0x7F7F;

  // operands of one 128-key tile, in registers
  struct Ops {
    u4 k0[4], k1[4], v0[4], v1[4];
    uint32_t ks[4], vs[4];
  };
  // request tile kt0's K and V operands (all before any is used: the kernel is bound by
  // these reads): MFMA row ql of sub-tile bb reads key kt0 + key_of(bb, (ql>>2)&1,
  // 4(ql>>3) + (ql&3)); V^T rows are channels 32 db + ql
  auto load_ops = [&](Ops& o, int kt0) __attribute__((always_inline)) {
#pragma unroll
    for (int bb = 0; bb < 4; bb++) {
      int key = kt0 + key_of<false>(bb, (ql >> 2) & 1, 4 * (ql >> 3) + (ql & 3));
      key = key < L ? key : L - 1;
      const uint8_t* kp = kc + (int64_t)key * 64;
      o.k0[bb] = *reinterpret_cast<const u4*>(kp + 16 * hh);
      o.k1[bb] = *reinterpret_cast<const u4*>(kp + 32 + 16 * hh);
      o.ks[bb] = *reinterpret_cast<const uint32_t*>(kscl + (int64_t)key * 4);
    }
#pragma unroll
    for (int db = 0; db < 4; db++) {
      const int64_t vrow = vrow0 + 32 * db + ql;
      const uint8_t* vp = a.v + vrow * (np / 2) + kt0 / 2;
      o.v0[db] = *reinterpret_cast<const u4*>(vp + 16 * hh);
      o.v1[db] = *reinterpret_cast<const u4*>(vp + 32 + 16 * hh);
      o.vs[db] = *reinterpret_cast<const uint32_t*>(a.vs + vrow * (np / 32) + kt0 / 32);
    }
  };
  // S^T = K Q^T of a tile
  auto scores = [&](const Ops& o) __attribute__((always_inline)) {
#pragma unroll
    for (int bb = 0; bb < 4; bb++) {
      const uint32_t ks4 = o.ks[bb] >> (8 * hh);
      v16f acc = zero16();
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(v8_from4(o.k0[bb]), qop[0], acc, 4, 4, 0, (int)ks4, 0,
                                                            (int)qsc);
      S[bb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(v8_from4(o.k1[bb]), qop[1], acc, 4, 4, 2, (int)ks4, 2,
                                                              (int)qsc);
    }
  };
  // mask, online softmax, P quantization and PV of tile kt0 (its scores in S)
  auto softmax_pv = [&](const Ops& o, int kt0) __attribute__((always_inline)) {
    // ---- mask: absent columns, keys past the history, keys after the query
#pragma unroll
    for (int bb = 0; bb < 4; bb++)
#pragma unroll
      for (int j = 0; j < 16; j++) {
        const int key = kt0 + key_of<false>(bb, hh, j);
        S[bb][j] = (cvalid && key <= pos) ? S[bb][j] : NEG_INF;  // pos < L
      }
    float bm16[4];
#pragma unroll
    for (int bb = 0; bb < 4; bb++) {
      float x = S[bb][0];
#pragma unroll
      for (int j = 1; j < 16; j++) x = fmaxn(x, S[bb][j]);
      bm16[bb] = x;
    }
    const float tmax = halves_max(fmaxn(fmaxn(bm16[0], bm16[1]), fmaxn(bm16[2], bm16[3])));

    // ---- online softmax and P quantization (E2M1 with E8M0 per 32 keys)
    const float mnew = fmaxn(m, tmax);
    const float ms = mnew == NEG_INF ? 0.0f : mnew * lam;
    const float alpha = m == mnew ? 1.0f : exp2_hw(__builtin_fmaf(m, lam, -ms));
    m = mnew;
    float k1 = 1.0f, scale_o = alpha;
    if constexpr (PMODE == PM_TWO_LEVEL) {
      const float rr = exp2_hw(__builtin_fmaf(tmax, lam, -ms));
      if (rr >= 0x1p-64f) {
        const float s1 = rr / 2688.0f;
        k1 = 1.0f / s1;
        scale_o = alpha * (s1prev / s1);
        s1prev = s1;
      } else {
        k1 = 0.0f;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 16; j++) O[i][j] *= scale_o;
    Lacc[0] *= alpha;
    int e[2];
#pragma unroll
    for (int p = 0; p < 2; p++) {
      const float bm = fmaxn(bm16[2 * p], bm16[2 * p + 1]);
      const int x = e8m0_exp(exp2_hw(__builtin_fmaf(bm, lam, -ms)) * k1, a.prule);
      e[p] = x < -126 ? -126 : x;
    }
    pscw = (uint32_t)(e[0] + 127) | ((uint32_t)(e[1] + 127) << 8);
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
        if constexpr (PMODE == PM_TWO_LEVEL) pt *= k1;
        y[j] = pt;
      }
      w[2 * bb] = pack8_fp4(y, sc);
      w[2 * bb + 1] = pack8_fp4(y + 8, sc);
    }
    if constexpr (PMODE != PM_PNQ) lpart = alpha * lpart + lsum;
    bp[0] = v8_from4(mk4(w[0], w[1], w[2], w[3]));
    bp[1] = v8_from4(mk4(w[4], w[5], w[6], w[7]));

    // ---- O^T += V^T P^T: channel rows 32 db + ql, keys kt0 + [0, 128) in order
#pragma unroll
    for (int db = 0; db < 4; db++) {
      const uint32_t vs4 = o.vs[db] >> (8 * hh);
      O[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(v8_from4(o.v0[db]), bp[0], O[db], 4, 4, 0, (int)vs4, 0,
                                                              (int)pscw);
      O[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(v8_from4(o.v1[db]), bp[1], O[db], 4, 4, 2, (int)vs4, 1,
                                                              (int)pscw);
    }
    if constexpr (PMODE == PM_PNQ) {
      const v8i ones = {0x22222222, 0x22222222, 0x22222222, 0x22222222, 0, 0, 0, 0};
      Lacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, bp[0], Lacc, 4, 4, 0, 127, 0, (int)pscw);
      Lacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, bp[1], Lacc, 4, 4, 0, 127, 1, (int)pscw);
    }
  };

  // the split's tiles in order; each tile requests all its reads before it computes
#pragma unroll 1
  for (int it = 0; it < DEC_SPLIT / 128; it++) {
    const int kt0 = k0 + 128 * it;
    if (kt0 >= L) break;
    Ops o;
    load_ops(o, kt0);
    scores(o);
    softmax_pv(o, kt0);
  }

  // ---- the split's normalized output and log-sum-exp, then the merge of the 4 splits
  // of this chunk by their log-sum-exp (in LDS) into one state per chunk
  float l;
  if constexpr (PMODE == PM_PNQ) l = Lacc[0];
  else l = halves_sum(lpart);
  float inv = l > 0.0f ? 1.0f / l : 0.0f;
  if constexpr (PMODE == PM_TWO_LEVEL) inv *= s1prev;
  __shared__ float so[4][32][129];  // [split][column][channel] (padded)
  __shared__ float slse[4][32];
#pragma unroll
  for (int db = 0; db < 4; db++)
#pragma unroll
    for (int j = 0; j < 16; j++) so[wave][ql][32 * db + 8 * (j >> 2) + 4 * hh + (j & 3)] = O[db][j] * inv;
  if (hh == 0) slse[wave][ql] = l > 0.0f ? __logf(l) + m * a.sm_scale : NEG_INF;
  __syncthreads();
  // thread -> (column cc = tid / 8, 16 channels from 16 (tid % 8))
  const int cc = tid >> 3, c0 = 16 * (tid & 7);
  if (cc < ncol) {
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
      t.x = (wt[0] * so[0][cc][c0 + c] + wt[1] * so[1][cc][c0 + c] + wt[2] * so[2][cc][c0 + c] + wt[3] * so[3][cc][c0 + c]) * winv;
      t.y = (wt[0] * so[0][cc][c0 + c + 1] + wt[1] * so[1][cc][c0 + c + 1] + wt[2] * so[2][cc][c0 + c + 1] +
             wt[3] * so[3][cc][c0 + c + 1]) * winv;
      t.z = (wt[0] * so[0][cc][c0 + c + 2] + wt[1] * so[1][cc][c0 + c + 2] + wt[2] * so[2][cc][c0 + c + 2] +
             wt[3] * so[3][cc][c0 + c + 2]) * winv;
      t.w = (wt[0] * so[0][cc][c0 + c + 3] + wt[1] * so[1][cc][c0 + c + 3] + wt[2] * so[2][cc][c0 + c + 3] +
             wt[3] * so[3][cc][c0 + c + 3]) * winv;
      *reinterpret_cast<float4*>(op + c) = t;
    }
    if ((tid & 7) == 0) a.ws_lse[orow] = wsum > 0.0f ? M + __logf(wsum) : NEG_INF;
  }
}

// merge of the chunk states of one (request, query head, row) by their log-sum-exp:
// 4 groups of 128 threads (thread = channel) take every 4th chunk, then add up in LDS
__global__ __launch_bounds__(512) void decode_merge_kernel(DecArgs a) {
  const int64_t row = blockIdx.x;  // (b, hq, r)
  const int64_t r = row % a.R, bh = row / a.R, hq = bh % a.Hq, b = bh / a.Hq;
  const int c = threadIdx.x & 127, grp = threadIdx.x >> 7;
  const int L = a.kv_len != nullptr ? a.kv_len[b] : (int)a.N;
  const int64_t ns = ((int64_t)L + 1023) / 1024;  // chunks holding keys of this request
  const float* lses = a.ws_lse + row * a.nsplit;
  __shared__ float red[4][128];
  __shared__ float rmax[4];
  float M = NEG_INF;
  for (int64_t s = grp; s < ns; s += 4) M = fmaxn(M, lses[s]);
  if (c == 0) rmax[grp] = M;
  __syncthreads();
  M = fmaxn(fmaxn(rmax[0], rmax[1]), fmaxn(rmax[2], rmax[3]));
  float acc = 0.0f, wsum = 0.0f;
  if (M != NEG_INF) {
    int64_t s = grp;
    for (; s + 12 < ns; s += 16) {  // four chunks in flight
      float ls[4], ov[4];
#pragma unroll
      for (int u = 0; u < 4; u++) {
        ls[u] = lses[s + 4 * u];
        ov[u] = a.ws_o[(row * a.nsplit + s + 4 * u) * 128 + c];
      }
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const float wgt = ls[u] == NEG_INF ? 0.0f : __expf(ls[u] - M);
        wsum += wgt;
        acc += wgt * ov[u];
      }
    }
    for (; s < ns; s += 4) {
      const float ls = lses[s];
      const float wgt = ls == NEG_INF ? 0.0f : __expf(ls - M);
      wsum += wgt;
      acc += wgt * a.ws_o[(row * a.nsplit + s) * 128 + c];
    }
  }
  __shared__ float wsums[4];
  red[grp][c] = acc;
  if (c == 0) wsums[grp] = wsum;
  __syncthreads();
  if (grp != 0) return;
  const float ws_all = wsums[0] + wsums[1] + wsums[2] + wsums[3];
  const float o = ws_all > 0.0f ? (red[0][c] + red[1][c] + red[2][c] + red[3][c]) / ws_all : 0.0f;
  if (a.out_fp32) {
    static_cast<float*>(a.out)[b * a.oB + hq * a.oH + r * a.oN + c] = o;
  } else {
    static_cast<uint16_t*>(a.out)[b * a.oB + hq * a.oH + r * a.oN + c] = (uint16_t)bf16_rne(o);
  }
  if (a.lse != nullptr && c == 0) a.lse[row] = ws_all > 0.0f ? M + __logf(ws_all) : NEG_INF;
}

hipError_t launch_decode(int pmode, const DecArgs& a, hipStream_t st) {
  const int64_t nchunk = (a.N + 1023) / 1024;
  const dim3 grid((unsigned)(a.B * a.Hkv * nchunk));
  if (pmode == PM_DIRECT) decode_kernel<PM_DIRECT><<<grid, 256, 0, st>>>(a);
  else if (pmode == PM_PNQ) decode_kernel<PM_PNQ><<<grid, 256, 0, st>>>(a);
  else if (pmode == PM_TWO_LEVEL) decode_kernel<PM_TWO_LEVEL><<<grid, 256, 0, st>>>(a);
  else return hipErrorNotSupported;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  decode_merge_kernel<<<dim3((unsigned)(a.B * a.Hq * a.R)), 512, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace mxattn
