// fwd.hip -- microscaling-FP4 attention forward for gfx950.
//
// One workgroup of 4 waves owns 128 query rows (32 per wave) of one (batch, head)
// or one (document, query tile) work item and walks key tiles of 128 in
// ascending order: the FlashAttention-2 form of the online softmax
// ("MXAttention", section 2 and Algorithm 1; "MpFA", Eqs. 3-6), with the softmax
// operand quantized inside the loop by the chosen P mode (blog "Microscaling FP4
// Attention", section "Two-level scaling"; SageAttention3 notes, Q2 Eq. 5;
// "MXAttention", section 4.2 and Algorithm 1; "MpFA", section 4.1).
//
// Operand layout on the matrix cores.  Scores are computed transposed,
// S^T = K Q^T, on 32x32 MFMA tiles, so that each lane holds the scores of ONE
// query: lane (q, h) (q = lane % 32, h = lane / 32) holds, for sub-tile b = 0..3,
// keys 64(b/2) + 32h + 16(b%2) + j, j = 0..15.  The K rows of the tile are stored
// in LDS in the permuted order that produces this, which gives every lane two
// complete 32-key blocks (blocks h and 2+h of the tile).  The output is then
// computed transposed too, O^T = V^T P^T: P enters as the B operand directly from
// the registers that hold it, one 32-key block per MFMA half, and the row
// statistics (max, alpha, sum) stay lane-local.  Each lane pairs its 32 operand
// elements with the same positions of the other operand, and its E8M0 scale
// covers exactly those 32 elements, so P blocks map one-to-one onto MFMA scale
// groups (the block-preserving permutation the SageAttention3 notes, Q3, describe
// for fusing the K permutation into quantization).
//
// Scales that do not fit the MFMA's E8M0-per-32 format (E4M3 block scales) are
// handled by dequantizing exactly to bf16 (an E2M1 value times an E4M3 scale has at
// most 6 significant bits) and using the bf16 MFMA; scales constant along the
// contraction (the two-level s1, 1/448 of FP8 P, sm_scale) are applied outside it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "formats.h"
#include "kernels.h"

namespace mxattn {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
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

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// the other lane half's value (lanes q and q+32 hold the two halves of a row)
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32); }

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
__device__ __forceinline__ uint32_t pack8_fp4(const float* x, float scale) {
  uint32_t w = 0;
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

template <int QK, int PV>
struct Lds {
  static constexpr int KROW = QK == QK_FP4 ? 80 : 256;
  static constexpr int VROW = PV == PV_FP4 ? 80 : PV == PV_BF16 ? 256 : 144;
  static constexpr int BYTES = 128 * (KROW + VROW);
};

template <int QK, int PV, int PMODE, int PSC, int VSC>
__global__ __launch_bounds__(256, 2) void fwd_kernel(FwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  using L = Lds<QK, PV>;
  uint8_t* Ks = smem;
  uint8_t* Vs = smem + 128 * L::KROW;
  constexpr int VB = VSC == SCALE_E8M0 ? 32 : 16;  // V block along keys
  constexpr bool SPLIT16 = PV == PV_FP8;            // key permutation of the FP8 MFMA

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, ql = lane & 31, hh = lane >> 5;

  // ---------------- work item ----------------
  int64_t b, hq, qt, qstart, qlen, klen, vstart;
  if (a.plan != nullptr) {
    const PlanHeader* ph = a.plan;
    const DocEntry* docs = reinterpret_cast<const DocEntry*>(ph + 1);
    const WorkItem* items = reinterpret_cast<const WorkItem*>(docs + ph->ndocs);
    int64_t item = blockIdx.x / a.Hq;
    hq = blockIdx.x % a.Hq;
    b = 0;
    if (item >= ph->n_items) return;
    WorkItem wi = items[item];
    DocEntry de = docs[wi.doc];
    qt = wi.qtile;
    qstart = de.start;
    qlen = de.len;
    klen = de.len;
    vstart = VB == 32 ? de.voff32 : de.voff16;
  } else {
    int64_t nqt = (a.N + 127) / 128, BH = a.B * a.Hq, G = a.grid;
    int64_t id = blockIdx.x, bh;
    if (a.causal) {  // longest first: the last query tiles see the most keys
      qt = nqt - 1 - id / BH;
      bh = id % BH;
    } else {  // the dispatcher deals workgroup ids round-robin to the 8 XCDs; give
              // each XCD a contiguous range so that one head's tiles share an L2
      if (G % 8 == 0) id = (id % 8) * (G / 8) + id / 8;
      bh = id / nqt;
      qt = id % nqt;
    }
    b = bh / a.Hq;
    hq = bh % a.Hq;
    qstart = 0;
    qlen = a.N;
    klen = a.N;
    vstart = 0;
  }
  const int64_t hk = hq * a.Hkv / a.Hq;
  const int64_t qloc = qt * 128 + 32 * wave + ql;  // this lane's query within its sequence
  const int64_t qrow = (b * a.Hq + hq) * a.N + qstart + (qloc < qlen ? qloc : qlen - 1);
  const int64_t kbase = (b * a.Hkv + hk) * a.N + qstart;  // K row of the sequence's first key
  const int64_t vrow0 = (b * a.Hkv + hk) * 128;           // first V^T row of the head
  int64_t nkt = (klen + 127) / 128;
  if (a.causal && nkt > qt + 1) nkt = qt + 1;
  const float lam = a.lambda;

  // ---------------- Q operand (B operand of S^T = K Q^T), held for the whole loop ----------------
  v8i qop[2];
  int qsc[2];
  v8bf qbf[8];
  if constexpr (QK == QK_FP4) {
    const uint8_t* qp = a.q + qrow * 64;
    uint32_t s4 = *reinterpret_cast<const uint32_t*>(a.qs + qrow * 4);
#pragma unroll
    for (int c = 0; c < 2; c++) {
      qop[c] = v8_from4(*reinterpret_cast<const u4*>(qp + 32 * c + 16 * hh));
      qsc[c] = (int)((s4 >> (8 * (2 * c + hh))) & 0xFF);
    }
  } else {
    const uint8_t* qp = a.q + qrow * 64;
    u2 s8 = *reinterpret_cast<const u2*>(a.qs + qrow * 8);
#pragma unroll
    for (int s = 0; s < 8; s++) {
      uint32_t w = *reinterpret_cast<const uint32_t*>(qp + 8 * s + 4 * hh);
      uint32_t sb = ((s < 4 ? s8.x : s8.y) >> (8 * (s & 3))) & 0xFF;
      u4 t = dq8_bf16(w, e4m3_value(sb));
      qbf[s] = __builtin_bit_cast(v8bf, t);
    }
  }

  // ---------------- online-softmax state ----------------
  float m = NEG_INF;  // running max of the raw scores of this lane's query
  float lpart = 0.0f; // this half's share of the row sum (modes with l from P~)
  v16f O[4], Lacc;
#pragma unroll
  for (int i = 0; i < 4; i++) O[i] = zero16();
  Lacc = zero16();

  // ---------------- staging registers (next tile) ----------------
  constexpr int NKC = 2;                              // K code chunks of 16 B per thread
  constexpr int NVC = (PV == PV_FP8 || VB == 16) ? 4 : 2;  // V code chunks per thread
  u4 kreg[NKC];
  uint32_t kscr[NKC];  // QK_FP4: row scales (thread < 128); QK_BF16: 2 scale bytes per chunk
  u4 vreg[NVC];     // VB == 16 and E2M1: only .x,.y used (8-byte chunks)
  uint32_t vscr[NVC];  // scales: PV_FP4/PV_FP8 thread >= 128 holds a channel's 4 bytes in [0];
                       // PV_BF16: the chunk's block scale byte

  auto load_tile = [&](int64_t kt) __attribute__((always_inline)) {
    // K rows: 512 chunks of 16 bytes
#pragma unroll
    for (int i = 0; i < NKC; i++) {
      int c = tid + 256 * i, row = c >> 2, part = c & 3;
      int64_t key = kt * 128 + row;
      if (key >= klen) key = klen - 1;
      kreg[i] = *reinterpret_cast<const u4*>(a.k + (kbase + key) * 64 + part * 16);
      if constexpr (QK == QK_BF16)
        kscr[i] = *reinterpret_cast<const uint16_t*>(a.ks + (kbase + key) * 8 + 2 * part);
    }
    if constexpr (QK == QK_FP4) {  // every thread loads (row tid % 128); threads < 128 store
      int64_t key = kt * 128 + (tid & 127);
      if (key >= klen) key = klen - 1;
      kscr[0] = *reinterpret_cast<const uint32_t*>(a.ks + (kbase + key) * 4);
    }
    // V^T rows (channels)
    const int64_t nvb = a.np / VB;  // scale blocks per channel row
#pragma unroll
    for (int i = 0; i < NVC; i++) {
      int c = tid + 256 * i;
      if constexpr (PV == PV_FP8) {  // 8 chunks of 16 keys per channel
        int ch = c >> 3, part = c & 7;
        int64_t key = vstart + kt * 128 + 16 * part;
        if (key > a.np - 16) key = a.np - 16;
        vreg[i] = *reinterpret_cast<const u4*>(a.v + (vrow0 + ch) * a.np + key);
      } else if constexpr (VB == 16) {  // E2M1, 8 chunks of 16 keys (8 bytes) per channel
        int ch = c >> 3, part = c & 7;
        int64_t key = vstart + kt * 128 + 16 * part;
        if (key > a.np - 16) key = a.np - 16;
        u2 t = *reinterpret_cast<const u2*>(a.v + (vrow0 + ch) * (a.np / 2) + key / 2);
        vreg[i] = mk4(t.x, t.y, 0, 0);
        vscr[i] = a.vs[(vrow0 + ch) * nvb + key / 16];
      } else {  // E2M1, 4 chunks of 32 keys (16 bytes) per channel
        int ch = c >> 2, part = c & 3;
        int64_t key = vstart + kt * 128 + 32 * part;
        if (key > a.np - 32) key = a.np - 32;
        vreg[i] = *reinterpret_cast<const u4*>(a.v + (vrow0 + ch) * (a.np / 2) + key / 2);
        if constexpr (PV == PV_BF16) vscr[i] = a.vs[(vrow0 + ch) * nvb + key / 32];
      }
    }
    if constexpr (PV != PV_BF16) {  // every thread loads (channel tid % 128); threads >= 128 store
      int ch = tid & 127;
      uint32_t w = 0;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        int64_t blk = (vstart + kt * 128) / 32 + j;
        if (blk > nvb - 1) blk = nvb - 1;
        w |= (uint32_t)a.vs[(vrow0 + ch) * nvb + blk] << (8 * j);
      }
      vscr[0] = w;
    }
  };

  auto store_tile = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NKC; i++) {
      int c = tid + 256 * i, row = c >> 2, part = c & 3;
      int pos = kpos<SPLIT16>(row);
      if constexpr (QK == QK_FP4) {
        *reinterpret_cast<u4*>(Ks + pos * 80 + part * 16) = kreg[i];
      } else {
        // 32 channels d = 32 part + [0, 32), E4M3 blocks 2 part, 2 part + 1
        float s0 = e4m3_value(kscr[i] & 0xFF), s1 = e4m3_value((kscr[i] >> 8) & 0xFF);
        uint32_t w4[4] = {kreg[i].x, kreg[i].y, kreg[i].z, kreg[i].w};
#pragma unroll
        for (int u = 0; u < 4; u++) {
          int chunk = (4 * part + u) ^ (pos & 15);
          *reinterpret_cast<u4*>(Ks + pos * 256 + chunk * 16) = dq8_bf16(w4[u], u < 2 ? s0 : s1);
        }
      }
    }
    if constexpr (QK == QK_FP4) {
      if (tid < 128) *reinterpret_cast<uint32_t*>(Ks + kpos<SPLIT16>(tid) * 80 + 64) = kscr[0];
    }
#pragma unroll
    for (int i = 0; i < NVC; i++) {
      int c = tid + 256 * i;
      if constexpr (PV == PV_FP8) {
        int ch = c >> 3, part = c & 7;
        *reinterpret_cast<u4*>(Vs + ch * 144 + part * 16) = vreg[i];
      } else if constexpr (PV == PV_FP4) {
        int ch = c >> 2, part = c & 3;
        *reinterpret_cast<u4*>(Vs + ch * 80 + part * 16) = vreg[i];
      } else if constexpr (VB == 16) {  // bf16 row of 128 keys: chunk = key / 8
        int ch = c >> 3, part = c & 7;
        float s = scale_value(vscr[i], VSC);
        *reinterpret_cast<u4*>(Vs + ch * 256 + (((2 * part) ^ (ch & 15)) * 16)) = dq8_bf16(vreg[i].x, s);
        *reinterpret_cast<u4*>(Vs + ch * 256 + (((2 * part + 1) ^ (ch & 15)) * 16)) = dq8_bf16(vreg[i].y, s);
      } else {
        int ch = c >> 2, part = c & 3;
        float s = scale_value(vscr[i], VSC);
        uint32_t w4[4] = {vreg[i].x, vreg[i].y, vreg[i].z, vreg[i].w};
#pragma unroll
        for (int u = 0; u < 4; u++)
          *reinterpret_cast<u4*>(Vs + ch * 256 + (((4 * part + u) ^ (ch & 15)) * 16)) = dq8_bf16(w4[u], s);
      }
    }
    if constexpr (PV == PV_FP4) {
      if (tid >= 128) *reinterpret_cast<uint32_t*>(Vs + (tid - 128) * 80 + 64) = vscr[0];
    } else if constexpr (PV == PV_FP8) {
      if (tid >= 128) *reinterpret_cast<uint32_t*>(Vs + (tid - 128) * 144 + 128) = vscr[0];
    }
  };

  if (nkt > 0) load_tile(0);

  for (int64_t kt = 0; kt < nkt; kt++) {
    __syncthreads();  // the previous tile's LDS reads are done
    store_tile();
    __syncthreads();
    // next tile in flight during this tile's math (the last iteration reloads its own
    // tile: an unconditional load keeps the staging registers out of scratch memory)
    load_tile(kt + 1 < nkt ? kt + 1 : kt);

    // ---------------- S^T = K Q^T ----------------
    v16f S[4];
#pragma unroll
    for (int bb = 0; bb < 4; bb++) {
      S[bb] = zero16();
      if constexpr (QK == QK_FP4) {
        const uint8_t* rp = Ks + (32 * bb + ql) * 80;
        uint32_t ks4 = *reinterpret_cast<const uint32_t*>(rp + 64);
#pragma unroll
        for (int c = 0; c < 2; c++) {
          v8i av = v8_from4(*reinterpret_cast<const u4*>(rp + 32 * c + 16 * hh));
          int sa = (int)((ks4 >> (8 * (2 * c + hh))) & 0xFF);
          S[bb] = mfma_fp4(av, qop[c], S[bb], sa, qsc[c]);
        }
      } else {
        const uint8_t* rp = Ks + (32 * bb + ql) * 256;
#pragma unroll
        for (int s = 0; s < 8; s++) {
          int chunk = (2 * s + hh) ^ (ql & 15);
          v8bf av = *reinterpret_cast<const v8bf*>(rp + chunk * 16);
          S[bb] = mfma_bf16(av, qbf[s], S[bb]);
        }
      }
    }

    // ---------------- mask (tail keys, causal diagonal) ----------------
    const int64_t k0 = kt * 128;
    const bool need_mask = (k0 + 128 > klen) || (a.causal && k0 + 127 > qt * 128 + 32 * wave);
    if (need_mask) {
#pragma unroll
      for (int bb = 0; bb < 4; bb++)
#pragma unroll
        for (int j = 0; j < 16; j++) {
          int64_t key = k0 + key_of<SPLIT16>(bb, hh, j);
          bool vis = key < klen && (!a.causal || key <= qloc);
          S[bb][j] = vis ? S[bb][j] : NEG_INF;
        }
    }

    // ---------------- row max: 16-key block maxima, 32-key block maxima, tile max ----------------
    float bm16[4];
#pragma unroll
    for (int bb = 0; bb < 4; bb++) {
      float x = S[bb][0];
#pragma unroll
      for (int j = 1; j < 16; j++) x = __builtin_fmaxf(x, S[bb][j]);
      bm16[bb] = x;
    }
    float bm[2] = {__builtin_fmaxf(bm16[0], bm16[1]), __builtin_fmaxf(bm16[2], bm16[3])};
    float tmax = __builtin_fmaxf(bm[0], bm[1]);
    tmax = __builtin_fmaxf(tmax, swap_halves(tmax));
    const float mnew = __builtin_fmaxf(m, tmax);
    const float ms = mnew == NEG_INF ? 0.0f : mnew * lam;  // exponent offset of this tile
    // exactly 1 when the max did not move (keeps the rescale skip exact), 0 while m = -inf
    const float alpha = m == mnew ? 1.0f : exp2_hw(__builtin_fmaf(m, lam, -ms));
    m = mnew;

    // ---------------- P~ = 2^(lambda (S - m)) ----------------
#pragma unroll
    for (int bb = 0; bb < 4; bb++)
#pragma unroll
      for (int j = 0; j < 16; j++) S[bb][j] = exp2_hw(__builtin_fmaf(S[bb][j], lam, -ms));

    // the maxima of P~ are the exponentials of the maxima of S (same operations, monotone)
    float pm16[4];
#pragma unroll
    for (int bb = 0; bb < 4; bb++) pm16[bb] = exp2_hw(__builtin_fmaf(bm16[bb], lam, -ms));

    // row sum from the unquantized P~
    if constexpr (PMODE != PM_PNQ) {
      float acc = 0.0f;
#pragma unroll
      for (int bb = 0; bb < 4; bb++)
#pragma unroll
        for (int j = 0; j < 16; j++) acc += S[bb][j];
      lpart = alpha * lpart + acc;
    }

    // two-level pre-scale s1 = rowmax_tile(P~) / (448 * 6)
    float s1 = 1.0f, k1 = 1.0f;
    if constexpr (PMODE == PM_TWO_LEVEL) {
      float r = exp2_hw(__builtin_fmaf(tmax, lam, -ms));
      s1 = r / 2688.0f;
      k1 = r > 0.0f ? 1.0f / s1 : 0.0f;  // a row with nothing visible in this tile adds nothing
      if (r == 0.0f) s1 = 0.0f;
#pragma unroll
      for (int bb = 0; bb < 4; bb++) {
#pragma unroll
        for (int j = 0; j < 16; j++) S[bb][j] = S[bb][j] * k1;
        pm16[bb] = pm16[bb] * k1;
      }
    }

    // ---------------- rescale the accumulators by alpha (skipped when the max did not move) ----------------
    const bool any_rescale = __builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0;
    if constexpr (PMODE != PM_TWO_LEVEL) {
      if (any_rescale) {
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
          for (int j = 0; j < 16; j++) O[i][j] *= alpha;
        Lacc[0] *= alpha;
      }
    }

    // ---------------- quantize P and run PV ----------------
    v16f D[4];
    if constexpr (PMODE == PM_TWO_LEVEL) {
#pragma unroll
      for (int i = 0; i < 4; i++) D[i] = zero16();
    }
    v16f* acc = (PMODE == PM_TWO_LEVEL) ? D : O;
    float lq = 0.0f;  // PNQ with bf16 PV: sum of the dequantized P of this half

    if constexpr (PV == PV_FP4) {
      // E2M1 codes with an E8M0 scale per 32-key block, the block being the MFMA's scale group
      v8i bp[2];
      int psc[2];
#pragma unroll
      for (int p = 0; p < 2; p++) {
        float M = __builtin_fmaxf(pm16[2 * p], pm16[2 * p + 1]);
        int e = e8m0_exp(M, a.prule);
        e = e < -126 ? -126 : e;
        float sc = u2f((uint32_t)(e + 127) << 23);
        uint32_t w[4];
#pragma unroll
        for (int dw = 0; dw < 4; dw++) {
          float y[8];
#pragma unroll
          for (int j = 0; j < 8; j++) y[j] = S[2 * p + (dw >> 1)][8 * (dw & 1) + j];
          w[dw] = pack8_fp4(y, sc);
        }
        bp[p] = v8_from4(mk4(w[0], w[1], w[2], w[3]));
        psc[p] = e + 127;
      }
#pragma unroll
      for (int db = 0; db < 4; db++) {
        const uint8_t* rp = Vs + (32 * db + ql) * 80;
        uint32_t vs4 = *reinterpret_cast<const uint32_t*>(rp + 64);
#pragma unroll
        for (int kc = 0; kc < 2; kc++) {
          v8i av = v8_from4(*reinterpret_cast<const u4*>(rp + 32 * kc + 16 * hh));
          int sa = (int)((vs4 >> (8 * (2 * kc + hh))) & 0xFF);
          acc[db] = mfma_fp4(av, bp[kc], acc[db], sa, psc[kc]);
        }
      }
      if constexpr (PMODE == PM_PNQ) {
        // row sum of the dequantized P on the matrix core: a block of ones times P^T
        const v8i ones = {0x22222222, 0x22222222, 0x22222222, 0x22222222, 0, 0, 0, 0};
        Lacc = mfma_fp4(ones, bp[0], Lacc, 127, psc[0]);
        Lacc = mfma_fp4(ones, bp[1], Lacc, 127, psc[1]);
      }
    } else if constexpr (PV == PV_BF16) {
      // P^ dequantized exactly to bf16; 16-key groups g = bb (one S sub-tile each)
      uint32_t pw[4][8];  // [bb][dword]: 16 bf16 of sub-tile bb
#pragma unroll
      for (int bb = 0; bb < 4; bb++) {
        float sc, kinv, sval;  // cvt scale (power of two), element multiplier, dequant factor
        if constexpr (PSC == SCALE_E8M0) {
          float M = __builtin_fmaxf(pm16[bb & 2], pm16[(bb & 2) + 1]);
          int e = e8m0_exp(M, a.prule);
          e = e < -126 ? -126 : e;
          sc = u2f((uint32_t)(e + 127) << 23);
          kinv = 1.0f;
          sval = sc;
        } else {
          uint32_t cb = e4m3_mag(pm16[bb] / 6.0f);
          sval = e4m3_value(cb);
          sc = 1.0f;
          kinv = sval > 0.0f ? 1.0f / sval : 0.0f;
        }
        float y[16];
#pragma unroll
        for (int j = 0; j < 16; j++) y[j] = PSC == SCALE_E8M0 ? S[bb][j] : S[bb][j] * kinv;
        uint32_t ww[2] = {pack8_fp4(y, sc), pack8_fp4(y + 8, sc)};
#pragma unroll
        for (int u = 0; u < 2; u++)
#pragma unroll
          for (int t = 0; t < 4; t++) {
            v2f pr = fp4_pair(ww[u], t);
            float x0 = pr[0] * sval, x1 = pr[1] * sval;
            if constexpr (PMODE == PM_PNQ) lq += x0 + x1;
            pw[bb][4 * u + t] = pack_bf16_exact(x0, x1);
          }
      }
#pragma unroll
      for (int db = 0; db < 4; db++) {
        const uint8_t* rp = Vs + (32 * db + ql) * 256;
#pragma unroll
        for (int s = 0; s < 8; s++) {
          // keys 64(s/4) + 32h + 8(s%4) + [0, 8) = sub-tile 2(s/4) + (s%4)/2, entries 8((s%4)%2) + [0, 8)
          int chunk = (8 * (s >> 2) + 4 * hh + (s & 3)) ^ (ql & 15);
          v8bf av = *reinterpret_cast<const v8bf*>(rp + chunk * 16);
          const int bb = 2 * (s >> 2) + ((s & 3) >> 1), o = 4 * ((s & 3) & 1);
          u4 t = mk4(pw[bb][o], pw[bb][o + 1], pw[bb][o + 2], pw[bb][o + 3]);
          acc[db] = mfma_bf16(av, __builtin_bit_cast(v8bf, t), acc[db]);
        }
      }
    } else {  // PV_FP8: c = E4M3(448 P~), unit scale; V in E4M3 with E8M0 per 32 keys
      v8i bp[2];
#pragma unroll
      for (int kc = 0; kc < 2; kc++) {
#pragma unroll
        for (int dw = 0; dw < 8; dw++) {
          const v16f& src = S[2 * kc + (dw >> 2)];
          int j0 = 4 * (dw & 3);
          int x = __builtin_amdgcn_cvt_pk_fp8_f32(448.0f * src[j0], 448.0f * src[j0 + 1], 0, false);
          x = __builtin_amdgcn_cvt_pk_fp8_f32(448.0f * src[j0 + 2], 448.0f * src[j0 + 3], x, true);
          bp[kc][dw] = x;
        }
      }
#pragma unroll
      for (int db = 0; db < 4; db++) {
        const uint8_t* rp = Vs + (32 * db + ql) * 144;
        uint32_t vs4 = *reinterpret_cast<const uint32_t*>(rp + 128);
#pragma unroll
        for (int kc = 0; kc < 2; kc++) {
          // operand element n holds key 64kc + 32(n/16) + 16h + n%16 (see key_of)
          u4 lo = *reinterpret_cast<const u4*>(rp + 64 * kc + 16 * hh);
          u4 hi = *reinterpret_cast<const u4*>(rp + 64 * kc + 32 + 16 * hh);
          v8i av = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          int sa = (int)((vs4 >> (8 * (2 * kc + hh))) & 0xFF);
          acc[db] = mfma_fp8(av, bp[kc], acc[db], sa, 127);
        }
      }
    }

    if constexpr (PMODE == PM_PNQ && PV != PV_FP4) lpart = alpha * lpart + lq;

    if constexpr (PMODE == PM_TWO_LEVEL) {
      // O = alpha O + s1 (P^2 V)
      if (any_rescale) {
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
          for (int j = 0; j < 16; j++) O[i][j] = __builtin_fmaf(s1, D[i][j], alpha * O[i][j]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
          for (int j = 0; j < 16; j++) O[i][j] = __builtin_fmaf(s1, D[i][j], O[i][j]);
      }
    }
  }

  // ---------------- epilogue: O = O~ / l, log-sum-exp ----------------
  float l;
  if constexpr (PMODE == PM_PNQ && PV == PV_FP4) {
    l = Lacc[0];
  } else {
    l = lpart + swap_halves(lpart);
  }
  float inv = l > 0.0f ? 1.0f / l : 0.0f;
  if constexpr (PV == PV_FP8) inv = inv / 448.0f;
  if (qloc < qlen) {
    const int64_t orow = qstart + qloc;
    if (a.out_fp32) {
      float* op = static_cast<float*>(a.out) + b * a.oB + hq * a.oH + orow * a.oN;
#pragma unroll
      for (int db = 0; db < 4; db++)
#pragma unroll
        for (int g = 0; g < 4; g++) {
          float4 t = make_float4(O[db][4 * g] * inv, O[db][4 * g + 1] * inv, O[db][4 * g + 2] * inv,
                                 O[db][4 * g + 3] * inv);
          *reinterpret_cast<float4*>(op + 32 * db + 8 * g + 4 * hh) = t;
        }
    } else {
      uint16_t* op = static_cast<uint16_t*>(a.out) + b * a.oB + hq * a.oH + orow * a.oN;
#pragma unroll
      for (int db = 0; db < 4; db++)
#pragma unroll
        for (int g = 0; g < 4; g++) {
          u2 t = mk2(bf16_rne(O[db][4 * g] * inv) | (bf16_rne(O[db][4 * g + 1] * inv) << 16),
                               bf16_rne(O[db][4 * g + 2] * inv) | (bf16_rne(O[db][4 * g + 3] * inv) << 16));
          *reinterpret_cast<u2*>(op + 32 * db + 8 * g + 4 * hh) = t;
        }
    }
    if (a.lse != nullptr && hh == 0) {
      float v = l > 0.0f ? __logf(l) + m * a.sm_scale : NEG_INF;
      a.lse[(b * a.Hq + hq) * a.N + orow] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
template <int QK, int PV, int PMODE, int PSC, int VSC>
static hipError_t launch_one(const FwdArgs& a, hipStream_t st) {
  constexpr int bytes = Lds<QK, PV>::BYTES;
  auto kern = fwd_kernel<QK, PV, PMODE, PSC, VSC>;
  if (bytes > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
  }
  kern<<<dim3((unsigned)a.grid), dim3(256), bytes, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_fwd(int qk, int pv, int pmode, int psc, int vsc, const FwdArgs& a, hipStream_t st) {
#define MXF(QK_, PV_, PM_, PS_, VS_) \
  if (qk == QK_ && pv == PV_ && pmode == PM_ && psc == PS_ && vsc == VS_) return launch_one<QK_, PV_, PM_, PS_, VS_>(a, st)
  // MXFP4 Q/K/V, E8M0/32 P: all on the scaled FP4 MFMA
  MXF(QK_FP4, PV_FP4, PM_DIRECT, SCALE_E8M0, SCALE_E8M0);
  MXF(QK_FP4, PV_FP4, PM_PNQ, SCALE_E8M0, SCALE_E8M0);
  MXF(QK_FP4, PV_FP4, PM_TWO_LEVEL, SCALE_E8M0, SCALE_E8M0);
  // MXFP4 Q/K/V, E4M3/16 P: bf16 PV
  MXF(QK_FP4, PV_BF16, PM_DIRECT, SCALE_E4M3, SCALE_E8M0);
  MXF(QK_FP4, PV_BF16, PM_PNQ, SCALE_E4M3, SCALE_E8M0);
  MXF(QK_FP4, PV_BF16, PM_TWO_LEVEL, SCALE_E4M3, SCALE_E8M0);
  // NVFP4 Q/K/V
  MXF(QK_BF16, PV_BF16, PM_DIRECT, SCALE_E4M3, SCALE_E4M3);
  MXF(QK_BF16, PV_BF16, PM_PNQ, SCALE_E4M3, SCALE_E4M3);
  MXF(QK_BF16, PV_BF16, PM_TWO_LEVEL, SCALE_E4M3, SCALE_E4M3);
  MXF(QK_BF16, PV_BF16, PM_DIRECT, SCALE_E8M0, SCALE_E4M3);
  MXF(QK_BF16, PV_BF16, PM_TWO_LEVEL, SCALE_E8M0, SCALE_E4M3);
  // NVFP4 Q/K with MXFP4 P/V
  MXF(QK_BF16, PV_FP4, PM_DIRECT, SCALE_E8M0, SCALE_E8M0);
  MXF(QK_BF16, PV_FP4, PM_PNQ, SCALE_E8M0, SCALE_E8M0);
  MXF(QK_BF16, PV_FP4, PM_TWO_LEVEL, SCALE_E8M0, SCALE_E8M0);
  // QK4PV8: FP8 P with the fixed scale 448 and FP8 V
  MXF(QK_BF16, PV_FP8, PM_FP8_FIXED, SCALE_E8M0, SCALE_E8M0);
  MXF(QK_FP4, PV_FP8, PM_FP8_FIXED, SCALE_E8M0, SCALE_E8M0);
#undef MXF
  return hipErrorNotSupported;  // no kernel instantiated for this route
}

}  // namespace mxattn
