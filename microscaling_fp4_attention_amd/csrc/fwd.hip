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
#include "device_util.h"
#include "kernels.h"

namespace mxattn {

template <int QK, int PV, bool BIAS = false>
struct Lds {
  static constexpr int KROW = QK == QK_FP4 ? 80 : 256;  // bytes per staged key row
  static constexpr int VROW = PV == PV_FP4 ? 80 : (PV == PV_BF16 || PV == PV_RAW) ? 256 : 144;  // per V^T row
  static constexpr int BOFF = 128 * (KROW + VROW);       // then the score bias of the 128 keys
  static constexpr int STAGE = BOFF + (BIAS ? 512 : 0);  // one key tile
  // Buffers of key tiles: 3 let tile kt be read while tile kt+2 is stored into a third
  // (one barrier per tile); 2 need a second barrier; 1 (large bf16 tiles) falls back
  // to compute-after-store.  Two workgroups share a CU's 160 KB.
  static constexpr int NB = 3 * STAGE <= 80 * 1024 ? 3 : 2 * STAGE <= 80 * 1024 ? 2 : 1;
  static constexpr int BYTES = NB * STAGE;
};

// Waves per SIMD the kernel is compiled for (256 registers each).
template <int QK, int PV>
constexpr int waves_per_simd() { return 2; }

// ---------------------------------------------------------------------------
// Plans of packed documents.  A plan is used only when its header matches the call:
// magic, document count, token count, causal flag and list sizes.  Otherwise every
// workgroup fills its rows of O and LSE with NaN, the mark of a mismatched workspace.
// Each entry is bounds-checked before it steers a read: a damaged entry is skipped.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool plan_header_ok(const FwdArgs& a) {
  const PlanHeader* ph = a.plan;
  const int64_t cap128 = (a.N + 127) / 128 + a.ndocs, cap256 = (a.N + 255) / 256 + a.ndocs;
  return ph->magic == PLAN_MAGIC && ph->ndocs == a.ndocs && (int64_t)ph->n_tokens == a.N &&
         ph->causal == (a.causal ? 1 : 0) && (int64_t)ph->cap128 == cap128 && ph->n_items >= 0 &&
         (int64_t)ph->n_items <= cap128 && ph->n_items256 >= 0 && (int64_t)ph->n_items256 <= cap256;
}

// a work item's document lies inside [0, N), its query tile inside the document and its
// V segment (vblock-aligned start, length rounded up to vblock) inside the padded keys
__device__ __forceinline__ bool plan_item_ok(const FwdArgs& a, const DocEntry& de, const WorkItem& wi, int rows,
                                             int64_t voff, int vblock) {
  return de.start >= 0 && de.len >= 0 && (int64_t)de.start <= a.N - de.len && wi.qtile >= 0 &&
         (int64_t)wi.qtile * rows < de.len && voff >= 0 &&
         voff + ((int64_t)de.len + vblock - 1) / vblock * vblock <= a.np;
}

// rows [r0, r0 + nrows) of query head hq (batch 0) of O and LSE set to NaN
__device__ void fill_nan_rows(const FwdArgs& a, int64_t hq, int64_t r0, int nrows) {
  for (int idx = threadIdx.x; idx < 2 * nrows; idx += blockDim.x) {
    const int64_t row = r0 + idx / 2;
    if (row >= a.N) continue;
    const int c0 = 64 * (idx & 1);
    if (a.out_fp32) {
      float* op = static_cast<float*>(a.out) + hq * a.oH + row * a.oN + c0;
      const float nan = __builtin_nanf("");
      for (int c = 0; c < 64; c += 4) *reinterpret_cast<float4*>(op + c) = make_float4(nan, nan, nan, nan);
    } else {
      uint16_t* op = static_cast<uint16_t*>(a.out) + hq * a.oH + row * a.oN + c0;
      for (int c = 0; c < 64; c += 8) *reinterpret_cast<u4*>(op + c) = mk4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
    }
    if (a.lse != nullptr && (idx & 1) == 0) a.lse[hq * a.N + row] = __builtin_nanf("");
  }
}

template <int QK, int PV, int PMODE, int PSC, int VSC, bool BIAS>
__global__ __launch_bounds__(256, (waves_per_simd<QK, PV>())) void fwd_kernel(FwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  using L = Lds<QK, PV, BIAS>;
  constexpr int NB = L::NB;
  constexpr int VB = VSC == SCALE_E8M0 ? 32 : 16;  // V block along keys
  constexpr bool SPLIT16 = PV == PV_FP8;            // key permutation of the FP8 MFMA

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, ql = lane & 31, hh = lane >> 5;

  // ---------------- work item ----------------
  int64_t b, hq, qt, qstart, qlen, klen, vstart;
  if (a.plan != nullptr) {
    const PlanHeader* ph = a.plan;
    const DocEntry* docs = reinterpret_cast<const DocEntry*>(ph + 1);
    const WorkItem* items = reinterpret_cast<const WorkItem*>(docs + a.ndocs);
    int64_t item = blockIdx.x / a.Hq;
    hq = blockIdx.x % a.Hq;
    b = 0;
    if (!plan_header_ok(a)) {
      fill_nan_rows(a, hq, item * 128, 128);
      return;
    }
    if (item >= ph->n_items) return;
    WorkItem wi = items[item];
    if ((uint32_t)wi.doc >= (uint32_t)a.ndocs) return;
    DocEntry de = docs[wi.doc];
    // a bf16 V keeps the token layout: its rows start at the document's first token
    const int64_t voff = PV == PV_RAW ? de.start : VB == 32 ? de.voff32 : de.voff16;
    if (!plan_item_ok(a, de, wi, 128, voff, PV == PV_RAW ? 1 : VB)) return;
    qt = wi.qtile;
    qstart = de.start;
    qlen = de.len;
    klen = de.len;
    vstart = voff;
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
  const int qloc = (int)(qt * 128) + 32 * wave + ql;  // this lane's query within its sequence
  const int64_t qrow = (b * a.Hq + hq) * a.N + qstart + (qloc < qlen ? qloc : qlen - 1);
  const int64_t kbase = (b * a.Hkv + hk) * a.N + qstart;  // K row of the sequence's first key
  const int64_t vrow0 = (b * a.Hkv + hk) * 128;           // first V^T row of the head
  int nkt = (int)((klen + 127) / 128);
  if (a.causal && nkt > qt + 1) nkt = (int)qt + 1;
  const int klen32 = (int)klen;
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
  } else if constexpr (QK == QK_RAW) {  // bf16 row of 128 channels: step s takes 16 s + 8 h + [0, 8)
    const uint8_t* qp = a.q + qrow * 256;
#pragma unroll
    for (int s = 0; s < 8; s++) qbf[s] = *reinterpret_cast<const v8bf*>(qp + 32 * s + 16 * hh);
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

  // ---------------- staging registers (a tile in flight) ----------------
  // K code chunks of 16 B per thread (a bf16 K row is 16 of them); V code chunks per
  // thread (a bf16 V: 8 rows of an 8-key x 8-channel block, transposed when stored)
  constexpr int NKC = QK == QK_RAW ? 8 : 2;
  constexpr int NVC = PV == PV_RAW ? 8 : (PV == PV_FP8 || VB == 16) ? 4 : 2;
  u4 kreg[NKC];
  uint32_t kscr[NKC];  // QK_FP4: row scales in [0]; QK_BF16: 2 scale bytes per chunk
  u4 vreg[NVC];        // VB == 16 with E2M1: only .x, .y used (8-byte chunks)
  uint32_t vscr[NVC];  // PV_FP4/PV_FP8: a channel's 4 block scales in [0]; PV_BF16: the chunk's scale

  // score bias of this query head (threads < 128 stage one key each)
  const float* hbias = BIAS ? a.bias + (b * a.Hq + hq) * a.N + qstart : nullptr;
  float rbias = 0.0f;
  auto load_tile = [&](int kt) __attribute__((always_inline)) {
    if constexpr (BIAS) {
      if (tid < 128) {
        int key = kt * 128 + tid;
        if (key >= klen32) key = klen32 - 1;
        rbias = hbias[key];
      }
    }
    // K rows: 512 chunks of 16 bytes
#pragma unroll
    for (int i = 0; i < NKC; i++) {
      if constexpr (QK == QK_RAW) {  // 16 chunks of 8 channels per key row
        int c = tid + 256 * i, row = c >> 4, part = c & 15;
        int key = kt * 128 + row;
        if (key >= klen32) key = klen32 - 1;
        kreg[i] = *reinterpret_cast<const u4*>(a.k + (kbase + key) * 256 + part * 16);
      } else {
        int c = tid + 256 * i, row = c >> 2, part = c & 3;
        int key = kt * 128 + row;
        if (key >= klen32) key = klen32 - 1;
        kreg[i] = *reinterpret_cast<const u4*>(a.k + (kbase + key) * 64 + part * 16);
        if constexpr (QK == QK_BF16)
          kscr[i] = *reinterpret_cast<const uint16_t*>(a.ks + (kbase + key) * 8 + 2 * part);
      }
    }
    if constexpr (QK == QK_FP4) {  // every thread loads (row tid % 128); threads < 128 store
      int key = kt * 128 + (tid & 127);
      if (key >= klen32) key = klen32 - 1;
      kscr[0] = *reinterpret_cast<const uint32_t*>(a.ks + (kbase + key) * 4);
    }
    // V^T rows (channels)
    const int64_t nvb = a.np / VB;  // scale blocks per channel row
#pragma unroll
    for (int i = 0; i < NVC; i++) {
      int c = tid + 256 * i;
      if constexpr (PV == PV_RAW) {  // keys 8 (tid / 16) + i, channels 8 (tid % 16) + [0, 8)
        int key = kt * 128 + 8 * (tid >> 4) + i;
        if (key >= klen32) key = klen32 - 1;
        vreg[i] = *reinterpret_cast<const u4*>(a.v + ((b * a.Hkv + hk) * a.N + vstart + key) * 256 + 16 * (tid & 15));
      } else if constexpr (PV == PV_FP8) {  // 8 chunks of 16 keys per channel
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
    if constexpr (PV == PV_FP4 || PV == PV_FP8) {  // every thread loads (channel tid % 128); threads >= 128 store
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

  auto store_tile = [&](int buf) __attribute__((always_inline)) {
    uint8_t* Ks = smem + buf * L::STAGE;
    uint8_t* Vs = Ks + 128 * L::KROW;
    if constexpr (BIAS) {
      if (tid < 128) *reinterpret_cast<float*>(Ks + L::BOFF + 4 * tid) = rbias;
    }
#pragma unroll
    for (int i = 0; i < NKC; i++) {
      if constexpr (QK == QK_RAW) {  // chunk = 8 channels, swizzled by the row position
        int c = tid + 256 * i, row = c >> 4, part = c & 15;
        int pos = kpos<SPLIT16>(row);
        *reinterpret_cast<u4*>(Ks + pos * 256 + ((part ^ (pos & 15)) * 16)) = kreg[i];
        continue;
      }
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
    if constexpr (PV == PV_RAW) {
      // the 8 x 8 block (rows: keys 8 kb + r, dword j: channels 2j, 2j + 1) transposed:
      // channel 8 cb + c gets its 8 keys as one 16-byte chunk kb of its bf16 row
      const int kb = tid >> 4, cb = tid & 15;
      const uint32_t R[8][4] = {{vreg[0].x, vreg[0].y, vreg[0].z, vreg[0].w}, {vreg[1].x, vreg[1].y, vreg[1].z, vreg[1].w},
                                {vreg[2].x, vreg[2].y, vreg[2].z, vreg[2].w}, {vreg[3].x, vreg[3].y, vreg[3].z, vreg[3].w},
                                {vreg[4].x, vreg[4].y, vreg[4].z, vreg[4].w}, {vreg[5].x, vreg[5].y, vreg[5].z, vreg[5].w},
                                {vreg[6].x, vreg[6].y, vreg[6].z, vreg[6].w}, {vreg[7].x, vreg[7].y, vreg[7].z, vreg[7].w}};
#pragma unroll
      for (int c = 0; c < 8; c++) {
        const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;  // high or low halves of keys 2m, 2m+1
        uint32_t w[4];
#pragma unroll
        for (int m = 0; m < 4; m++) w[m] = __builtin_amdgcn_perm(R[2 * m + 1][c >> 1], R[2 * m][c >> 1], sel);
        const int ch = 8 * cb + c;
        *reinterpret_cast<u4*>(Vs + ch * 256 + ((kb ^ (ch & 15)) * 16)) = mk4(w[0], w[1], w[2], w[3]);
      }
    }
#pragma unroll
    for (int i = 0; i < (PV == PV_RAW ? 0 : NVC); i++) {
      int c = tid + 256 * i;
      if constexpr (PV == PV_RAW) {
      } else if constexpr (PV == PV_FP8) {
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

  // ---------------- S^T = K Q^T of the tile in buffer `buf`, sub-tile bb (32 keys) ----------------
  auto scores_sub = [&](int buf, int bb) __attribute__((always_inline)) -> v16f {
    // the LDS offset passes through an empty asm, which keeps the compiler from hoisting
    // these loads and MFMAs (pure operations) above the stores and barrier before them
    uint32_t boff = (uint32_t)(buf * L::STAGE);
    asm volatile("" : "+v"(boff));
    const uint8_t* Ks = smem + boff;
    v16f acc = BIAS ? bias16(Ks + L::BOFF + 4 * key_of<SPLIT16>(bb, hh, 0)) : zero16();
    if constexpr (QK == QK_FP4) {
      const uint8_t* rp = Ks + (32 * bb + ql) * 80;
      uint32_t ks4 = *reinterpret_cast<const uint32_t*>(rp + 64);
#pragma unroll
      for (int c = 0; c < 2; c++) {
        v8i av = v8_from4(*reinterpret_cast<const u4*>(rp + 32 * c + 16 * hh));
        int sa = (int)((ks4 >> (8 * (2 * c + hh))) & 0xFF);
        acc = mfma_fp4(av, qop[c], acc, sa, qsc[c]);
      }
    } else {
      const uint8_t* rp = Ks + (32 * bb + ql) * 256;
#pragma unroll
      for (int s = 0; s < 8; s++) {
        int chunk = (2 * s + hh) ^ (ql & 15);
        v8bf av = *reinterpret_cast<const v8bf*>(rp + chunk * 16);
        acc = mfma_bf16(av, qbf[s], acc);
      }
    }
    return acc;
  };
  auto scores = [&](int buf, v16f* S) __attribute__((always_inline)) {
#pragma unroll
    for (int bb = 0; bb < 4; bb++) S[bb] = scores_sub(buf, bb);
  };

  // ---------------- softmax, P quantization and PV of one tile ----------------
  // S: this tile's scores (consumed)
  auto softmax_pv = [&](int kt, int buf, v16f* S) __attribute__((always_inline)) {
    const uint8_t* Vs = smem + buf * L::STAGE + 128 * L::KROW;
    // mask (tail keys, causal diagonal): wave-uniform test, per-element select
    const int k0 = kt * 128;
    const bool need_mask = (k0 + 128 > klen32) || (a.causal && k0 + 127 > (int)qt * 128 + 32 * wave);
    if (need_mask) {
      // keys below lim are visible; a lane's 16 keys of sub-tile bb are consecutive
      const int lim = a.causal && qloc + 1 < klen32 ? qloc + 1 : klen32;
#pragma unroll
      for (int bb = 0; bb < 4; bb++) {
        const int n = lim - (k0 + key_of<SPLIT16>(bb, hh, 0));
#pragma unroll
        for (int j = 0; j < 16; j++) S[bb][j] = j < n ? S[bb][j] : NEG_INF;
      }
    }

    // row max: 16-key block maxima, tile max
    float bm16[4];
#pragma unroll
    for (int bb = 0; bb < 4; bb++) {
      float x = S[bb][0];
#pragma unroll
      for (int j = 1; j < 16; j++) x = __builtin_fmaxf(x, S[bb][j]);
      bm16[bb] = x;
    }
    float tmax = __builtin_fmaxf(__builtin_fmaxf(bm16[0], bm16[1]), __builtin_fmaxf(bm16[2], bm16[3]));
    tmax = __builtin_fmaxf(tmax, swap_halves(tmax));
    const float mnew = __builtin_fmaxf(m, tmax);
    const float ms = mnew == NEG_INF ? 0.0f : mnew * lam;  // exponent offset of this tile
    const float msub = mnew == NEG_INF ? 0.0f : mnew;
    // exactly 1 when the max did not move (keeps the rescale skip exact), 0 while m = -inf
    const float alpha = m == mnew ? 1.0f : exp2_diff(m, mnew, lam);
    m = mnew;

    // the maxima of P~ are the exponentials of the maxima of S (monotone), formed from
    // the difference to the running maximum so that the row's maximum gives exactly 1
    float pm16[4];
#pragma unroll
    for (int bb = 0; bb < 4; bb++) pm16[bb] = exp2_diff(bm16[bb], msub, lam);

    // two-level pre-scale s1 = rowmax_tile(P~) / (448 * 6)
    float s1 = 1.0f, k1 = 1.0f;
    if constexpr (PMODE == PM_TWO_LEVEL) {
      float r = exp2_diff(tmax, msub, lam);
      s1 = r / 2688.0f;
      k1 = r > 0.0f ? 1.0f / s1 : 0.0f;  // a row with nothing visible in this tile adds nothing
      if (r == 0.0f) s1 = 0.0f;
#pragma unroll
      for (int bb = 0; bb < 4; bb++) pm16[bb] = pm16[bb] * k1;
    }

    // block scales of P, known before any element is touched
    float sc16[4], sv16[4], ki16[4];  // per 16-key group: convert scale, dequant factor, multiplier
    int psc[2];                       // E8M0 byte of each 32-key block (FP4 MFMA operand)
    if constexpr (PV == PV_FP4 || (PV == PV_BF16 && PSC == SCALE_E8M0)) {
#pragma unroll
      for (int p = 0; p < 2; p++) {
        int e = e8m0_exp(__builtin_fmaxf(pm16[2 * p], pm16[2 * p + 1]), a.prule);
        e = e < -126 ? -126 : e;
        float sc = u2f((uint32_t)(e + 127) << 23);
        psc[p] = e + 127;
        sc16[2 * p] = sc16[2 * p + 1] = sc;
        sv16[2 * p] = sv16[2 * p + 1] = sc;
        ki16[2 * p] = ki16[2 * p + 1] = 1.0f;
      }
    } else if constexpr (PV == PV_BF16) {  // E4M3 scale per 16 keys
#pragma unroll
      for (int bb = 0; bb < 4; bb++) {
        float sv = e4m3_value(e4m3_mag(pm16[bb] / 6.0f));
        sc16[bb] = 1.0f;
        sv16[bb] = sv;
        ki16[bb] = sv > 0.0f ? 1.0f / sv : 0.0f;
      }
    }

    // per sub-tile: P~ = 2^(lambda (S - m)), row sum, quantized operand
    float lsum = 0.0f;       // row sum of P~ (or of the dequantized P for PNQ on bf16)
    uint32_t pc[4][4];       // FP4 codes [sub-tile][dword 0..1] / FP8 codes [sub-tile][dword 0..3]
    uint32_t pw[4][8];       // bf16 P [sub-tile][dword]
#pragma unroll
    for (int bb = 0; bb < 4; bb++) {
      float y[16];
#pragma unroll
      for (int j = 0; j < 16; j++) {
        float pt = exp2_hw(__builtin_fmaf(S[bb][j], lam, -ms));
        if constexpr (PMODE != PM_PNQ) lsum += pt;
        if constexpr (PMODE == PM_TWO_LEVEL) pt *= k1;
        y[j] = pt;
      }
      if constexpr (PV == PV_FP4) {
        pc[bb][0] = pack8_fp4(y, sc16[bb]);
        pc[bb][1] = pack8_fp4(y + 8, sc16[bb]);
      } else if constexpr (PV == PV_RAW) {  // P~ rounded to bf16 (nearest even)
#pragma unroll
        for (int t = 0; t < 8; t++) pw[bb][t] = bf16_rne(y[2 * t]) | (bf16_rne(y[2 * t + 1]) << 16);
      } else if constexpr (PV == PV_BF16) {
        float z[16];
#pragma unroll
        for (int j = 0; j < 16; j++) z[j] = PSC == SCALE_E8M0 ? y[j] : y[j] * ki16[bb];
        uint32_t ww[2] = {pack8_fp4(z, sc16[bb]), pack8_fp4(z + 8, sc16[bb])};
#pragma unroll
        for (int u = 0; u < 2; u++)
#pragma unroll
          for (int t = 0; t < 4; t++) {
            v2f pr = fp4_pair(ww[u], t);
            float x0 = pr[0] * sv16[bb], x1 = pr[1] * sv16[bb];
            if constexpr (PMODE == PM_PNQ) lsum += x0 + x1;
            pw[bb][4 * u + t] = pack_bf16_exact(x0, x1);
          }
      } else {  // FP8: c = E4M3(448 P~)
#pragma unroll
        for (int dw = 0; dw < 4; dw++) {
          int x = __builtin_amdgcn_cvt_pk_fp8_f32(448.0f * y[4 * dw], 448.0f * y[4 * dw + 1], 0, false);
          pc[bb][dw] = __builtin_amdgcn_cvt_pk_fp8_f32(448.0f * y[4 * dw + 2], 448.0f * y[4 * dw + 3], x, true);
        }
      }
    }
    if constexpr (PMODE != PM_PNQ || PV != PV_FP4) lpart = alpha * lpart + lsum;

    // rescale the accumulators by alpha (skipped when no row's max moved)
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

    // PV
    v16f D[4];
    if constexpr (PMODE == PM_TWO_LEVEL) {
#pragma unroll
      for (int i = 0; i < 4; i++) D[i] = zero16();
    }
    if constexpr (PV == PV_FP4) {
      // operand of 32-key block p: sub-tiles 2p (keys +0..15) and 2p+1 (keys +16..31)
      v8i bp[2];
#pragma unroll
      for (int p = 0; p < 2; p++) bp[p] = v8_from4(mk4(pc[2 * p][0], pc[2 * p][1], pc[2 * p + 1][0], pc[2 * p + 1][1]));
#pragma unroll
      for (int db = 0; db < 4; db++) {
        const uint8_t* rp = Vs + (32 * db + ql) * 80;
        uint32_t vs4 = *reinterpret_cast<const uint32_t*>(rp + 64);
#pragma unroll
        for (int kc = 0; kc < 2; kc++) {
          v8i av = v8_from4(*reinterpret_cast<const u4*>(rp + 32 * kc + 16 * hh));
          int sa = (int)((vs4 >> (8 * (2 * kc + hh))) & 0xFF);
          if constexpr (PMODE == PM_TWO_LEVEL) D[db] = mfma_fp4(av, bp[kc], D[db], sa, psc[kc]);
          else O[db] = mfma_fp4(av, bp[kc], O[db], sa, psc[kc]);
        }
      }
      if constexpr (PMODE == PM_PNQ) {
        // row sum of the dequantized P on the matrix core: a block of ones times P^T
        const v8i ones = {0x22222222, 0x22222222, 0x22222222, 0x22222222, 0, 0, 0, 0};
        Lacc = mfma_fp4(ones, bp[0], Lacc, 127, psc[0]);
        Lacc = mfma_fp4(ones, bp[1], Lacc, 127, psc[1]);
      }
    } else if constexpr (PV == PV_BF16 || PV == PV_RAW) {
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
          if constexpr (PMODE == PM_TWO_LEVEL) D[db] = mfma_bf16(av, __builtin_bit_cast(v8bf, t), D[db]);
          else O[db] = mfma_bf16(av, __builtin_bit_cast(v8bf, t), O[db]);
        }
      }
    } else {  // PV_FP8: unit P scale; V in E4M3 with E8M0 per 32 keys
      v8i bp[2];
#pragma unroll
      for (int kc = 0; kc < 2; kc++) {
#pragma unroll
        for (int dw = 0; dw < 8; dw++) bp[kc][dw] = (int)pc[2 * kc + (dw >> 2)][dw & 3];
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
          O[db] = mfma_fp8(av, bp[kc], O[db], sa, 127);
        }
      }
    }

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
  };

  // ---------------- the key-tile loop ----------------
  if (nkt > 0) {
    v16f S[4];
    if constexpr (NB == 1) {
      // one buffer: store, then compute on it (two barriers per tile).  The unquantized
      // route's staging registers (a bf16 tile is 4 times the codes) are not held across
      // the math: it loads each tile right before storing it.
      if constexpr (QK != QK_RAW) load_tile(0);
      for (int kt = 0; kt < nkt; kt++) {
        __syncthreads();  // the previous tile's LDS reads are done
        if constexpr (QK == QK_RAW) load_tile(kt);
        store_tile(0);
        __syncthreads();
        // next tile in flight during this tile's math (the last iteration reloads its own
        // tile: an unconditional load keeps the staging registers out of scratch memory)
        if constexpr (QK != QK_RAW) load_tile(kt + 1 < nkt ? kt + 1 : kt);
        scores(0, S);
        softmax_pv(kt, 0, S);
      }
    } else {
      // tiles kt+1 and kt+2 are staged while tile kt is computed
      load_tile(0);
      store_tile(0);
      load_tile(nkt > 1 ? 1 : 0);
      store_tile(1 % NB);
      __syncthreads();
      load_tile(nkt > 2 ? 2 : nkt - 1);
      for (int kt = 0; kt < nkt; kt++) {
        scores(kt % NB, S);
        softmax_pv(kt, kt % NB, S);
        if constexpr (NB == 2) __syncthreads();  // buffer kt % 2 is free once every PV read it
        store_tile((kt + 2) % NB);               // tile kt+2 (a repeat of the last tile past the end)
        load_tile(kt + 3 < nkt ? kt + 3 : nkt - 1);
        __syncthreads();
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

// ===========================================================================
// Ping-pong form: 8 waves own 256 query rows.  Each SIMD holds one wave of group A
// (waves 0-3) and one of group B (waves 4-7).  Per key tile t a wave runs an MFMA
// phase M(t) = {PV of tile t-1, S^T of tile t and its row maxima} and a VALU phase
// V(t) = {exponentials, P quantization, staging of a later tile}; group B runs one
// phase behind group A and a workgroup barrier ends every phase, so on every SIMD
// one wave's matrix-core work overlaps the other wave's vector work.  Key tiles sit
// in 3 LDS buffers; each group stages half of every tile (64 key rows and 64 V^T
// rows) during its VALU phases, two phases after loading it.
// Routes: QK_FP4 / QK_BF16 x PV_FP4 / PV_FP8 / PV_BF16 (V with E8M0 per 32 keys).
// ===========================================================================
template <int QK, int PV, bool BIAS, bool SAFE>
struct PpLds {
  static constexpr int KROW = QK == QK_FP4 ? 80 : 256;
  static constexpr int VROW = PV == PV_FP4 ? 80 : PV == PV_FP8 ? 144 : 256;
  static constexpr int KV = 128 * KROW;             // V^T rows follow the 128 key rows of a stage
  static constexpr int BOFF = 128 * (KROW + VROW);  // then the score bias of the 128 keys
  // then the E8M0 scale dwords of the K rows and of the V^T rows, each as two arrays of
  // 128 dwords [lane half][row]: half h holds the row's dword shifted right by 8 h, so
  // its low bytes are the scales of the blocks that half's operand elements cover, and
  // the 32 lanes of a half read 32 consecutive dwords (no bank conflict)
  static constexpr int KSC = BOFF + (BIAS ? 512 : 0);
  static constexpr int VSC = KSC + (QK == QK_FP4 ? 1024 : 0);
  static constexpr int STAGE = VSC + (PV == PV_BF16 ? 0 : 1024);
  // after the 3 stages, with causally safe V scales: the per-key E8M0 bytes of the
  // workgroup's two diagonal key tiles, 128 per tile in key order (their E2M1 codes
  // come through the stages)
  static constexpr int KEYX = 3 * STAGE;
  // then, with causally safe V, the Q operand rows (80-byte rows, 256 query rows)
  static constexpr int QOFF = KEYX + 256;
  static constexpr int BYTES = KEYX + (SAFE ? 256 + (QK == QK_FP4 ? 256 * 80 : 0) : 0);
};

template <int QK, int PV, int PMODE, int PSC, bool BIAS, bool SAFE, bool EXPB>
__global__ __launch_bounds__(512, 1) void fwd_pp_kernel(FwdArgs a) {
  static_assert(!SAFE || PV == PV_FP4 || PV == PV_BF16, "the per-key form serves a 4-bit V");
  using L = PpLds<QK, PV, BIAS, SAFE>;
  // static LDS: its base is the constant 0, so stage offsets fold into the instructions
  __shared__ __attribute__((aligned(16))) uint8_t smem[L::BYTES];
  constexpr int STAGE = L::STAGE, KV = L::KV;
  constexpr bool SPLIT16 = PV == PV_FP8;
  // E4M3-scaled P with MXFP4 V: the PV product in f16 (a tile staged from the per-key
  // form of V takes bf16 products on the same accumulator)
  constexpr bool H16 = PV == PV_BF16;
  const int tid = threadIdx.x, lane = tid & 63, ql = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int grp = wave >> 2;  // 0: group A, 1: group B
  const int gt = tid & 255;   // thread within the group

  // ---------------- work item: 256 query rows ----------------
  int64_t b, hq, qt, qstart, vstart;
  int klen;
  if (a.plan != nullptr) {
    const PlanHeader* ph = a.plan;
    const DocEntry* docs = reinterpret_cast<const DocEntry*>(ph + 1);
    const WorkItem* items = reinterpret_cast<const WorkItem*>(docs + a.ndocs) + ((a.N + 127) / 128 + a.ndocs);
    const int64_t item = blockIdx.x / a.Hq;
    hq = blockIdx.x % a.Hq;
    b = 0;
    if (!plan_header_ok(a)) {
      fill_nan_rows(a, hq, item * 256, 256);
      return;
    }
    if (item >= ph->n_items256) return;
    const WorkItem wi = items[item];
    if ((uint32_t)wi.doc >= (uint32_t)a.ndocs) return;
    const DocEntry de = docs[wi.doc];
    if (!plan_item_ok(a, de, wi, 256, de.voff32, 32)) return;
    qt = wi.qtile;
    qstart = de.start;
    klen = de.len;
    vstart = de.voff32;
  } else {
    const int64_t nqt = (a.N + 255) / 256, BH = a.B * a.Hq, G = a.grid;
    const int64_t groups = a.B * a.Hkv, gsz = a.Hq / a.Hkv;  // KV heads, query heads per KV head
    int64_t id = blockIdx.x, bh;
    if (a.causal && groups % 8 == 0) {
      // Workgroup ids are dealt round-robin to the 8 XCDs: XCD id % 8 gets whole KV-head
      // groups (their K/V stay in its L2), and runs its items longest first.
      const int64_t ng = groups / 8, slot = id / 8;
      qt = nqt - 1 - slot / (ng * gsz);
      const int64_t rem = slot % (ng * gsz), grp_id = (id % 8) * ng + rem / gsz;
      bh = (grp_id / a.Hkv) * a.Hq + (grp_id % a.Hkv) * gsz + rem % gsz;
    } else if (a.causal) {  // longest first
      qt = nqt - 1 - id / BH;
      bh = id % BH;
    } else {  // one head's tiles on one XCD (workgroup ids are dealt round-robin to 8 XCDs)
      if (G % 8 == 0) id = (id % 8) * (G / 8) + id / 8;
      bh = id / nqt;
      qt = id % nqt;
    }
    b = bh / a.Hq;
    hq = bh % a.Hq;
    qstart = 0;
    klen = (int)a.N;
    vstart = 0;
  }
  const int64_t hk = hq * a.Hkv / a.Hq;
  const int qloc = (int)qt * 256 + 32 * wave + ql;  // query within its sequence
  const int64_t qrow = (b * a.Hq + hq) * a.N + qstart + (qloc < klen ? qloc : klen - 1);
  const int64_t kbase = (b * a.Hkv + hk) * a.N + qstart;  // K row of the sequence's first key
  const int64_t vrow0 = (b * a.Hkv + hk) * 128;
  int nkt = (klen + 127) / 128;
  if (a.causal && nkt > 2 * (int)qt + 2) nkt = 2 * (int)qt + 2;
  const float lam = a.lambda;
  // two-level P: lambda in a VGPR for the per-element FMA (2.8% faster at N = 32K; the
  // other modes measured 0.5-1.5% slower with it)
  const float lamv = PMODE == PM_TWO_LEVEL ? to_vgpr(lam) : lam;
  // P~ of a score s given the row's exponent offset ms = m lambda and, for the bit-level
  // exponential, cm = exp_bias - ms 2^23: one FMA and the hardware exponential, or one
  // FMA (2^23 (s lambda - ms - delta + 127), its rounding keeps 16 fraction bits of t),
  // a clamp and a convert.  Both are monotone in s, so the value at a block's largest
  // score is the block's largest P~.
  const float lamb = lam * 0x1p23f;
  auto pexp = [&](float sc, float ms, float cm) __attribute__((always_inline)) -> float {
    if constexpr (EXPB) return exp2_bits(__builtin_fmaf(sc, lamb, cm));
    else return exp2_hw(__builtin_fmaf(sc, lamv, -ms));
  };
  auto pexp_c = [&](float ms) __attribute__((always_inline)) -> float {
    return EXPB ? __builtin_fmaf(-ms, 0x1p23f, a.exp_bias) : 0.0f;
  };
  // P~ at a block's or a tile's largest score, the input of a block-scale or pre-scale
  // decision: the exact exponential is formed from the difference to the running
  // maximum (msub), which makes it exactly 1 at the row's maximum; the bit-level line
  // uses its own form (monotone, so the block's largest P~ either way)
  auto pmax = [&](float sc, float ms, float cm, float msub) __attribute__((always_inline)) -> float {
    if constexpr (EXPB) return exp2_bits(__builtin_fmaf(sc, lamb, cm));
    else return exp2_diff(sc, msub, lam);
  };

  // ---------------- Q operand ----------------
  v8i qop[2];
  uint32_t qsc = 0;
  v8h qh16[8];
  if constexpr (QK == QK_FP4) {
    const uint8_t* qp = a.q + qrow * 64;
    qsc = *reinterpret_cast<const uint32_t*>(a.qs + qrow * 4) >> (8 * hh);
    qop[0] = v8_from4(*reinterpret_cast<const u4*>(qp + 16 * hh));
    qop[1] = v8_from4(*reinterpret_cast<const u4*>(qp + 32 + 16 * hh));
    if constexpr (SAFE) {  // kept in LDS instead (the registers go to the per-key steps)
      *reinterpret_cast<u4*>(smem + L::QOFF + (32 * wave + ql) * 80 + 16 * hh) = mk4(qop[0][0], qop[0][1], qop[0][2], qop[0][3]);
      *reinterpret_cast<u4*>(smem + L::QOFF + (32 * wave + ql) * 80 + 32 + 16 * hh) = mk4(qop[1][0], qop[1][1], qop[1][2], qop[1][3]);
    }
  } else {  // NVFP4: each element dequantized exactly to f16 (an E2M1 value times an
             // E4M3 scale has at most 6 significant bits in [2^-10, 2688]); the scale
             // byte by the hardware E4M3 convert
    const uint8_t* qp = a.q + qrow * 64;
    u2 s8 = *reinterpret_cast<const u2*>(a.qs + qrow * 8);
#pragma unroll
    for (int s = 0; s < 8; s++) {
      uint32_t w = *reinterpret_cast<const uint32_t*>(qp + 8 * s + 4 * hh);
      const _Float16 sh = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)((s < 4 ? s8.x : s8.y) >> (8 * (s & 3))), 0);
      qh16[s] = dq8_f16(w, v2h{sh, sh});
    }
  }

  // ---------------- staging: this thread's share of a tile ----------------
  // K: key row kr = 64 grp + gt/4, 16-byte code chunk gt%4 (32 channels); V^T: channel
  // vc = kr, chunk gt%4 of 32 keys (FP8: two chunks of 16 keys); scales: row / channel
  // sr = 64 grp + gt%64 (K scales by gt < 64, V scales by 64 <= gt < 128).
  const int kr = 64 * grp + (gt >> 2), part = gt & 3, sr = 64 * grp + (gt & 63);
  const int kpos_r = kpos<SPLIT16>(kr), kpos_s = kpos<SPLIT16>(sr);
  // scalar (wave-uniform) bases of this head, 32-bit per-lane offsets (N and np are at
  // most 2^24).  The V scale bytes of a tile start at block vstart/32 + 4t, a multiple
  // of 4 unless a document starts inside a group of 4 blocks: two aligned dwords are
  // loaded and joined when stored (joining them at load time would wait for the loads).
  const uint8_t* hk_codes = a.k + kbase * 64;
  const uint8_t* hk_scales = a.ks + kbase * (QK == QK_FP4 ? 4 : 8);
  const uint32_t np = (uint32_t)a.np, vrow_bytes = PV == PV_FP8 ? np : np / 2;
  const uint32_t nvb = np / 32;  // V scale blocks per channel row
  const uint8_t* hv_codes = a.v + vrow0 * vrow_bytes;
  // causally safe V: the workgroup's two diagonal key tiles, 2 qt and 2 qt + 1, are
  // staged from the per-key form (E2M1 codes in the same channel-row layout, unit
  // block scales); its per-key exponents go into P in the V phase
  const uint8_t* hvk_codes = SAFE ? a.vk + vrow0 * vrow_bytes : nullptr;
  const uint8_t* hv_sbase = a.vs + vrow0 * nvb;
  const uint32_t vblk0 = (uint32_t)(vstart >> 5) & ~3u, vsh = (uint32_t)(vstart >> 5) & 3u;
  const uint32_t o_v = (uint32_t)kr * vrow_bytes, o_vs = (uint32_t)sr * nvb + vblk0;
  // score bias of this query head: wave 2 of each group stages its half's 64 keys
  const float* hbias = BIAS ? a.bias + (b * a.Hq + hq) * a.N + qstart : nullptr;
  const int bkey = 64 * grp + (gt & 63);
  u4 rk, rv0, rv1;
  uint32_t rks = 0, rvs = 0, rvs_hi = 0;
  bool rpk = false;  // the staged tile comes from the per-key form
  float rb = 0.0f;
  // f16 PV: each channel row c of V is staged as V 2^vshift_c, which places the largest
  // E8M0 exponent among the row's blocks this workgroup reads at 13 (6 2^13 < 65504).
  // Every block within 36 binades of it is then exact in f16 (its values are multiples
  // of 2^-24).  Row c of O^T = V^T P^T is the same channel, so the epilogue scales each
  // channel back by 2^-vshift_c.  The staging thread of channel row c (tid / 4) scans
  // that row's scale bytes with the three other threads of its quad, over the blocks
  // that hold keys of this workgroup's range; blocks staged past it (the tail tile's
  // next document or padding) meet only masked keys and are clamped to 2^13.  An
  // all-zero block carries the byte of 2^0: when that byte is the row's largest and a
  // block lies more than 36 binades below it, the zero blocks are told apart by their
  // codes and left out.
  int vshift = 0;
  // causally safe V on the f16 route: the per-key tiles' P operand carries 2^sigma and
  // their V 2^(vshift - sigma) in bf16, sigma = max(0, largest vshift - 125), so every
  // staged value stays below 2^128 (a bf16 E2M1 value with 2 significant bits is exact
  // down to 2^-133; vshift - sigma >= -127 for bf16 inputs, whose E8M0 block exponents
  // stay at or below 125) and P^' 2^sigma <= 2688 2^15
  int psig = 0;
  float psig_f = 1.0f, pks = 1.0f;
  __shared__ int vshift_lds[H16 ? 128 : 1];
  __shared__ int vsh_wmax[H16 && SAFE ? 8 : 1];
  if constexpr (H16) {
    const uint32_t b0 = (uint32_t)(vstart >> 5);
    const uint32_t bk = (uint32_t)((vstart + klen + 31) >> 5);       // past the range's keys
    const uint32_t bt = b0 + 4u * (uint32_t)nkt;                      // past the tiles read
    const uint32_t b1 = bk < bt ? bk : bt;                            // blocks [b0, b1)
    const uint32_t row = (uint32_t)(tid >> 2);
    const uint8_t* rp = hv_sbase + row * nvb;
    uint32_t mx = 0, mn = 255;
    auto bmax4 = [](uint32_t w) {
      return __builtin_elementwise_max(__builtin_elementwise_max(w & 0xFFu, (w >> 8) & 0xFFu),
                                       __builtin_elementwise_max((w >> 16) & 0xFFu, w >> 24));
    };
    auto bmin4 = [](uint32_t w) {
      return __builtin_elementwise_min(__builtin_elementwise_min(w & 0xFFu, (w >> 8) & 0xFFu),
                                       __builtin_elementwise_min((w >> 16) & 0xFFu, w >> 24));
    };
    // aligned dwords (nvb is a multiple of 4); bytes outside [b0, b1) are kept out
    for (uint32_t i = (b0 & ~3u) + 4u * (uint32_t)(tid & 3); i < b1; i += 16u) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(rp + i);
      uint32_t keep = 0xFFFFFFFFu;
      if (i < b0) keep &= 0xFFFFFFFFu << (8u * (b0 - i));
      if (i + 4u > b1) keep &= 0xFFFFFFFFu >> (8u * (i + 4u - b1));
      mx = __builtin_elementwise_max(mx, bmax4(w & keep));
      mn = __builtin_elementwise_min(mn, bmin4(w | ~keep));
    }
    mx = __builtin_elementwise_max(mx, (uint32_t)__shfl_xor((int)mx, 1));
    mx = __builtin_elementwise_max(mx, (uint32_t)__shfl_xor((int)mx, 2));
    mn = __builtin_elementwise_min(mn, (uint32_t)__shfl_xor((int)mn, 1));
    mn = __builtin_elementwise_min(mn, (uint32_t)__shfl_xor((int)mn, 2));
    if (mx == 127u && mn + 36u < 127u) {
      // the largest byte is 2^0, possibly of all-zero blocks: take the largest over the
      // blocks that are not 2^0 or have a nonzero code (codes: 16 bytes per block)
      const uint8_t* cp = hv_codes + row * vrow_bytes;
      uint32_t m2 = 0;
      for (uint32_t bl = b0 + (uint32_t)(tid & 3); bl < b1; bl += 4u) {
        const uint32_t byte = rp[bl];
        bool real = byte != 127u;
        if (!real) {
          const u4 c = *reinterpret_cast<const u4*>(cp + 16u * bl);
          real = (c.x | c.y | c.z | c.w) != 0u;
        }
        if (real) m2 = __builtin_elementwise_max(m2, byte);
      }
      m2 = __builtin_elementwise_max(m2, (uint32_t)__shfl_xor((int)m2, 1));
      mx = __builtin_elementwise_max(m2, (uint32_t)__shfl_xor((int)m2, 2));
    }
    vshift = 140 - (int)mx;  // biased byte mx -> exponent 13
    if ((tid & 3) == 0) vshift_lds[row] = vshift;
    if constexpr (SAFE) {
      int w = vshift;  // the same in the 4 lanes of a row
      w = __builtin_elementwise_max(w, __shfl_xor(w, 4));
      w = __builtin_elementwise_max(w, __shfl_xor(w, 8));
      w = __builtin_elementwise_max(w, __shfl_xor(w, 16));
      w = __builtin_elementwise_max(w, __shfl_xor(w, 32));
      if (lane == 0) vsh_wmax[wave] = w;
      __syncthreads();
      int mxs = vsh_wmax[0];
#pragma unroll
      for (int i = 1; i < 8; i++) mxs = __builtin_elementwise_max(mxs, vsh_wmax[i]);
      psig = mxs > 125 ? mxs - 125 : 0;
      psig_f = __builtin_ldexpf(1.0f, psig);
      pks = __builtin_ldexpf(1.0f, vshift - psig);
    }
  }
  auto load_half = [&](int t) __attribute__((always_inline)) {
    if constexpr (BIAS) {
      if (gt >= 128 && gt < 192) {  // wave-uniform
        const int k = t * 128 + bkey < klen ? t * 128 + bkey : klen - 1;
        rb = hbias[k];
      }
    }
    const int key = t * 128 + kr < klen ? t * 128 + kr : klen - 1;
    rk = *reinterpret_cast<const u4*>(hk_codes + ((uint32_t)key * 64 + part * 16));
    if constexpr (QK == QK_FP4) {
      if (gt < 64) {  // wave-uniform
        const int skey = t * 128 + sr < klen ? t * 128 + sr : klen - 1;
        rks = *reinterpret_cast<const uint32_t*>(hk_scales + (uint32_t)skey * 4);
      }
    } else {
      rks = *reinterpret_cast<const uint16_t*>(hk_scales + ((uint32_t)key * 8 + 2 * part));
    }
    const uint32_t key0 = (uint32_t)vstart + (uint32_t)t * 128;  // first padded key slot (< np)
    const bool pk = SAFE && (t >> 1) == (int)qt;                  // per-key form (wave-uniform)
    if constexpr (SAFE) rpk = pk;
    if constexpr (PV == PV_FP8) {  // two chunks of 16 keys: parts gt%4 and gt%4 + 4
      const uint32_t k1 = __builtin_elementwise_min(key0 + 16 * part, np - 16);
      const uint32_t k2 = __builtin_elementwise_min(key0 + 16 * (part + 4), np - 16);
      rv0 = *reinterpret_cast<const u4*>(hv_codes + (o_v + k1));
      rv1 = *reinterpret_cast<const u4*>(hv_codes + (o_v + k2));
    } else {
      const uint32_t k1 = __builtin_elementwise_min(key0 + 32 * part, np - 32);
      rv0 = *reinterpret_cast<const u4*>((pk ? hvk_codes : hv_codes) + (o_v + k1 / 2));
    }
    if constexpr (PV == PV_BF16) {  // the chunk's own block scale
      const uint32_t blk = __builtin_elementwise_min((key0 + 32 * part) / 32, nvb - 1);
      rvs = pk ? 127u : (uint32_t)hv_sbase[(uint32_t)kr * nvb + blk];
    } else if (gt >= 64 && gt < 128) {  // a channel's 4 block scales (wave-uniform)
      // the group of 4 after the tile's first one lies past the row only when the
      // tile's keys do (vblk0 + 4t <= nvb - 4 since key0 < np and nvb % 4 == 0)
      const uint32_t lo = o_vs + 4 * (uint32_t)t;
      const uint32_t hi = vblk0 + 4 * (uint32_t)t + 4 < nvb ? lo + 4 : lo;
      rvs = *reinterpret_cast<const uint32_t*>(hv_sbase + lo);
      rvs_hi = *reinterpret_cast<const uint32_t*>(hv_sbase + hi);
      if constexpr (SAFE) {  // unit scales on the per-key tiles
        rvs = pk ? 0x7F7F7F7Fu : rvs;
        rvs_hi = pk ? 0x7F7F7F7Fu : rvs_hi;
      }
    }
  };
  auto store_half = [&](uint32_t so) __attribute__((always_inline)) {
    uint8_t* base = smem + so;
    if constexpr (BIAS) {
      if (gt >= 128 && gt < 192) *reinterpret_cast<float*>(base + L::BOFF + 4 * bkey) = rb;
    }
    if constexpr (QK == QK_FP4) {
      *reinterpret_cast<u4*>(base + kpos_r * 80 + part * 16) = rk;
      if (gt < 64) {
        *reinterpret_cast<uint32_t*>(base + L::KSC + 4 * kpos_s) = rks;
        *reinterpret_cast<uint32_t*>(base + L::KSC + 512 + 4 * kpos_s) = rks >> 8;
      }
    } else {  // NVFP4 as exact f16: channels 32 part + [0, 32), E4M3 blocks 2 part, 2 part + 1
      const _Float16 s0 = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)rks, 0);
      const _Float16 s1 = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)rks, 1);
      const uint32_t w4[4] = {rk.x, rk.y, rk.z, rk.w};
#pragma unroll
      for (int u = 0; u < 4; u++)
        *reinterpret_cast<v8h*>(base + kpos_r * 256 + (((4 * part + u) ^ (kpos_r & 15)) * 16)) =
            dq8_f16(w4[u], u < 2 ? v2h{s0, s0} : v2h{s1, s1});
    }
    uint8_t* vb = base + KV;
    if constexpr (PV == PV_FP4) {
      *reinterpret_cast<u4*>(vb + kr * 80 + part * 16) = rv0;
      if (gt >= 64 && gt < 128) {
        const uint32_t w = __builtin_amdgcn_alignbyte(rvs_hi, rvs, vsh);
        *reinterpret_cast<uint32_t*>(base + L::VSC + 4 * sr) = w;
        *reinterpret_cast<uint32_t*>(base + L::VSC + 512 + 4 * sr) = w >> 8;
      }
    } else if constexpr (PV == PV_FP8) {
      *reinterpret_cast<u4*>(vb + kr * 144 + part * 16) = rv0;
      *reinterpret_cast<u4*>(vb + kr * 144 + (part + 4) * 16) = rv1;
      if (gt >= 64 && gt < 128) {
        const uint32_t w = __builtin_amdgcn_alignbyte(rvs_hi, rvs, vsh);
        *reinterpret_cast<uint32_t*>(base + L::VSC + 4 * sr) = w;
        *reinterpret_cast<uint32_t*>(base + L::VSC + 512 + 4 * sr) = w >> 8;
      }
    } else {  // a row of 128 keys of 2-byte values, chunk = key / 8, swizzled by the channel
      const uint32_t w4[4] = {rv0.x, rv0.y, rv0.z, rv0.w};
      if (SAFE && rpk) {  // per-key form: bf16 Vk 2^(vshift - sigma), exact
#pragma unroll
        for (int u = 0; u < 4; u++)
          *reinterpret_cast<u4*>(vb + kr * 256 + (((4 * part + u) ^ (kr & 15)) * 16)) = dq8_bf16(w4[u], pks);
      } else {  // f16 V 2^vshift
        // scale 2^(e + vshift) as the convert's operand: biased exponent byte + vshift
        // (140 at most inside the scanned blocks, clamped there outside them); blocks
        // more than 139 binades below the largest become 0
        const int be = __builtin_elementwise_min((int)rvs + vshift, 140);
        const float sc = u2f((uint32_t)(be > 1 ? be : 1) << 23);
#pragma unroll
        for (int u = 0; u < 4; u++)
          *reinterpret_cast<u4*>(vb + kr * 256 + (((4 * part + u) ^ (kr & 15)) * 16)) = dq8_f16_pow2(w4[u], sc);
      }
    }
  };

  // ---------------- state ----------------
  float m = NEG_INF, lpart = 0.0f, s1prev = 1.0f;
  float lfix = 0.0f;  // PNQ with causally safe V: this lane's share of the folded tiles' row sum
  v16f O[4], Lacc, S[4];
#pragma unroll
  for (int i = 0; i < 4; i++) O[i] = zero16();
  Lacc = zero16();
  float bm16[4], tmax;          // 16-key block maxima and the tile max of the scores in S
  v8i bp[2];                    // P operand: FP4 codes (4 dwords each) or FP8 codes (8 dwords)
  uint32_t pscw = 0x7F7F;       // FP4 P: E8M0 bytes of the two 32-key blocks (byte kc)
  uint32_t pc[8];               // bf16 P route: E2M1 codes [sub-tile][2 dwords] ...
  float pdq[4];                 // ... and the dequantization factor of each 16-key group
  // a staged scale dword is followed by a copy shifted right by 8 bits: lane half hh
  // reads the copy whose low bytes are its blocks' scales
  const uint32_t koffk = (uint32_t)(ql * L::KROW + 16 * hh);
  const uint32_t soff = (uint32_t)(512 * hh + 4 * ql);  // this lane's scale dword of a 32-row group
  bp[0] = bp[1] = v8i{0, 0, 0, 0, 0, 0, 0, 0};

  // The multiplier of the P quantization -- the two-level 1/s1, an E4M3 group scale's
  // 1/s, FP8 P's 448 -- enters the exact exponential as an offset of its argument
  // instead of a product per element: P~/s1 = 2^(lambda (S - tmax) + log2 2688), since
  // s1 is the tile's largest P~ over 2688, 1/s as -log2 s (the hardware logarithm,
  // within 2^-20 of log2 s for every E4M3 value), 448 P~ = 2^(lambda S - ms + log2 448).  One FMA per element instead of an FMA and a
  // product (two-level E8M0 at N = 32K 8%, packed documents 6% faster).
  constexpr bool PFOLD = PV == PV_BF16 && PSC != SCALE_E8M0;
  constexpr bool LOGOFF = !EXPB && (PMODE == PM_TWO_LEVEL || PFOLD || PV == PV_FP8);
  constexpr float LOG2_2688 = 0x1.6c8ddep+3f;  // log2(448 * 6) rounded to FP32
  constexpr float LOG2_448 = 0x1.19d5dap+3f;   // log2(448): FP8 P = E4M3(448 P~)

  // P of sub-tile bb (16 keys per lane) from its scores in S[bb]: the exponentials, this
  // lane's share of the row sum (returned), and the quantized operand written in place
  // (ms, cm: the row's exponent offset; k1: two-level pre-scale; sc, sv, ki: the 16-key
  // group's convert scale, dequantization factor and multiplier)
  // With LOGOFF the group's multiplier is already in ms (the argument's offset) and the
  // returned row-sum share is that of P~ times the multiplier.
  auto p_sub = [&](int bb, float ms, float cm, float k1, float sc, float sv, float ki)
      __attribute__((always_inline)) -> float {
    float lsum = 0.0f;
    float y[16];
    // an E4M3 group scale's multiplier is applied with the two-level pre-scale in one
    // product (k1 ki rounded once per group instead of each element rounded twice)
    const float kel = PFOLD ? (PMODE == PM_TWO_LEVEL ? k1 * ki : ki) : k1;
#pragma unroll
    for (int j = 0; j < 16; j++) {
      float pt = pexp(S[bb][j], ms, cm);
      if constexpr (PMODE != PM_PNQ) lsum += pt;
      if constexpr (!LOGOFF && (PMODE == PM_TWO_LEVEL || PFOLD)) pt *= kel;
      y[j] = pt;
    }
    if constexpr (PV == PV_FP4) {  // into the registers of the previous tile's P
      const int e0 = 2 * (bb & 1);
      bp[bb >> 1][e0] = (int)pack8_fp4(y, sc, (uint32_t)bp[bb >> 1][e0]);
      bp[bb >> 1][e0 + 1] = (int)pack8_fp4(y + 8, sc, (uint32_t)bp[bb >> 1][e0 + 1]);
    } else if constexpr (PV == PV_FP8) {  // c = E4M3(448 P~): 4 dwords per sub-tile
#pragma unroll
      for (int dw = 0; dw < 4; dw++) {
        constexpr float F = LOGOFF ? 1.0f : 448.0f;  // LOGOFF: y is 448 P~ already
        int x = __builtin_amdgcn_cvt_pk_fp8_f32(F * y[4 * dw], F * y[4 * dw + 1], 0, false);
        x = __builtin_amdgcn_cvt_pk_fp8_f32(F * y[4 * dw + 2], F * y[4 * dw + 3], x, true);
        bp[bb >> 1][4 * (bb & 1) + dw] = x;
      }
    } else {
      pc[2 * bb] = pack8_fp4(y, sc);  // y already carries the group's multiplier
      pc[2 * bb + 1] = pack8_fp4(y + 8, sc);
      pdq[bb] = sv;
      if constexpr (PMODE == PM_PNQ) {  // row sum of the dequantized P
#pragma unroll
        for (int u = 0; u < 2; u++)
#pragma unroll
          for (int q = 0; q < 4; q++) {
            v2f pr = fp4_pair(pc[2 * bb + u], q);
            lsum += (pr[0] + pr[1]) * sv;
          }
      }
    }
    return lsum;
  };

  // V-phase state (phase_v_pre): the exponent offset, the rescale, the two-level
  // pre-scale and the block scales of P.  With E8M0 P scales it is prepared at the end
  // of the M phase, which waits at its barrier for the co-resident wave's V phase, so
  // this short dependent chain runs in that slack instead of at the head of the V
  // phase (video-DiT 32K PNQ 1%, two-level E8M0 5.5% faster); the E4M3 scales of the
  // f16 route (a division, a rounding with branches and a reciprocal per 16 keys)
  // measured 20% slower there and stay in the V phase.
  constexpr bool PRE_IN_M = PV != PV_BF16;
  float vp_ms = 0.0f, vp_cm = 0.0f, vp_k1 = 1.0f, vp_alpha = 1.0f;
  float vp_sc[4] = {1.0f, 1.0f, 1.0f, 1.0f}, vp_sv[4] = {1.0f, 1.0f, 1.0f, 1.0f}, vp_ki[4] = {1.0f, 1.0f, 1.0f, 1.0f};
  // LOGOFF: each group's argument offset and the factor from its row-sum share to P~'s
  float vp_cg[4] = {0.0f, 0.0f, 0.0f, 0.0f}, vp_lk[4] = {1.0f, 1.0f, 1.0f, 1.0f};
  auto phase_v_pre = [&]() __attribute__((always_inline)) {
    const float mnew = fmaxn(m, tmax);
    const float ms = mnew == NEG_INF ? 0.0f : mnew * lam;
    const float msub = mnew == NEG_INF ? 0.0f : mnew;
    const float cm = pexp_c(ms);
    // exactly 1 when the max did not move (keeps the rescale skip exact), 0 while m = -inf;
    // the rescale is exact in both exponential modes
    const float alpha = m == mnew ? 1.0f : exp2_diff(m, mnew, lam);
    m = mnew;

    // two-level: s1 = rowmax_tile(P~)/2688; the accumulator holds O / s1 and is carried
    // to the new s1 by beta = alpha s1_prev / s1 (a tile whose P~ stays below 2^-64 of
    // the running maximum adds nothing and keeps s1)
    float k1 = 1.0f, scale_o = alpha;
    float c1 = ms;  // LOGOFF: the argument offset with the two-level pre-scale in it
    if constexpr (PMODE == PM_TWO_LEVEL) {
      float r = pmax(tmax, ms, cm, msub);
      if (r >= 0x1p-64f) {
        float s1 = r / 2688.0f;
        k1 = __builtin_amdgcn_rcpf(s1);  // within an ulp: the P values' products carry it
        scale_o = alpha * (s1prev * k1);
        s1prev = s1;
        if constexpr (LOGOFF) c1 = __builtin_fmaf(tmax, lam, -LOG2_2688);
      } else {
        k1 = 0.0f;
        if constexpr (LOGOFF) c1 = __builtin_inff();  // every P~ s1 of the tile is 0
      }
    }
    const bool any_rescale = __builtin_amdgcn_ballot_w64(scale_o != 1.0f) != 0;
    if (any_rescale) {
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 16; j++) O[i][j] *= scale_o;
      Lacc[0] *= alpha;
      if constexpr (SAFE) lfix *= alpha;
    }

    // block scales of P from the block maxima of P~ (exponentials of the score maxima)
    float sc16[4] = {1.0f, 1.0f, 1.0f, 1.0f}, sv16[4] = {1.0f, 1.0f, 1.0f, 1.0f},
          ki16[4] = {1.0f, 1.0f, 1.0f, 1.0f};  // per 16 keys: convert scale, dequant factor, multiplier
    int e[2] = {0, 0};
    if constexpr (PV == PV_FP4 || (PV == PV_BF16 && PSC == SCALE_E8M0)) {
#pragma unroll
      for (int p = 0; p < 2; p++) {
        const float bm = fmaxn(bm16[2 * p], bm16[2 * p + 1]);
        // LOGOFF: the block's largest element by the elements' own arithmetic
        int x = e8m0_exp(LOGOFF ? pexp(bm, c1, cm) : pmax(bm, ms, cm, msub) * k1, a.prule);
        e[p] = x < -126 ? -126 : x;
        const float sc = u2f((uint32_t)(e[p] + 127) << 23);
        sc16[2 * p] = sc16[2 * p + 1] = sv16[2 * p] = sv16[2 * p + 1] = sc;
        ki16[2 * p] = ki16[2 * p + 1] = 1.0f;
      }
      pscw = (uint32_t)(e[0] + 127) | ((uint32_t)(e[1] + 127) << 8);
    } else if constexpr (PV == PV_BF16) {  // E4M3 scale per 16 keys
#pragma unroll
      for (int bb = 0; bb < 4; bb++) {
        const float pm = PMODE == PM_TWO_LEVEL && LOGOFF ? pexp(bm16[bb], c1, cm) : pmax(bm16[bb], ms, cm, msub) * k1;
        // E4M3_rne_sat(fl32(M / 6)) by the hardware FP8 convert and back: the same code
        // as the integer encoder for every float below 464 (checked on all of them), and
        // M / 6 <= 2688 (1 + 2^-20) / 6 stays below it
        const float q6 = div6(pm);
        const float sv = __builtin_amdgcn_cvt_f32_fp8(__builtin_amdgcn_cvt_pk_fp8_f32(q6, q6, 0, false), 0);
        sc16[bb] = 1.0f;
        sv16[bb] = sv;
        ki16[bb] = sv > 0.0f ? __builtin_amdgcn_rcpf(sv) : 0.0f;
        if constexpr (LOGOFF) {
          // a zero scale dequantizes every code of its group to 0: the elements then
          // keep the offset without it (finite) and the row sum takes them as they are
          vp_cg[bb] = sv > 0.0f ? c1 + __builtin_amdgcn_logf(sv) : c1;
          vp_lk[bb] = (PMODE == PM_TWO_LEVEL ? s1prev : 1.0f) * (sv > 0.0f ? sv : 1.0f);
        }
      }
    }
    if constexpr (LOGOFF && PV == PV_FP8) {  // 448 P~ = 2^(lambda S - ms + log2 448)
#pragma unroll
      for (int bb = 0; bb < 4; bb++) {
        vp_cg[bb] = ms - LOG2_448;
        vp_lk[bb] = 1.0f / 448.0f;
      }
    } else if constexpr (LOGOFF && !PFOLD) {
#pragma unroll
      for (int bb = 0; bb < 4; bb++) {
        vp_cg[bb] = c1;
        vp_lk[bb] = s1prev;
      }
    }

    vp_ms = ms;
    vp_cm = cm;
    vp_k1 = k1;
    vp_alpha = alpha;
#pragma unroll
    for (int bb = 0; bb < 4; bb++) {
      vp_sc[bb] = sc16[bb];
      vp_sv[bb] = sv16[bb];
      vp_ki[bb] = ki16[bb];
    }
  };
  // M(t): PV of tile t-1 (stage offset sv), then S^T of tile t (stage offset sk) with
  // its mask and maxima
  // mfold: tile t-1 is a diagonal tile under causally safe V, staged in the per-key form
  // of V (unit block scales); vfold: the V phase that follows folds (no set-up here)
  auto phase_m = [&](int t, uint32_t sk, uint32_t sv, bool mfold, bool vfold) __attribute__((always_inline)) {
    if (t >= 1) {
      const bool fold = SAFE && mfold;
      const uint8_t* Vs = smem + sv + KV;
      if constexpr (PV == PV_FP4) {
#pragma unroll
        for (int db = 0; db < 4; db++) {
          const uint8_t* rp = Vs + (32 * db + ql) * 80;
          const uint32_t vs4 = *reinterpret_cast<const uint32_t*>(smem + sv + L::VSC + 128 * db + soff);
          v8i a0 = v8_from4(*reinterpret_cast<const u4*>(rp + 16 * hh));
          v8i a1 = v8_from4(*reinterpret_cast<const u4*>(rp + 32 + 16 * hh));
          O[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, bp[0], O[db], 4, 4, 0, (int)vs4, 0, (int)pscw);
          O[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, bp[1], O[db], 4, 4, 2, (int)vs4, 1, (int)pscw);
        }
        if constexpr (PMODE == PM_PNQ) {
          if (!fold) {  // the folded tile's row sum is formed in its V phase
            const v8i ones = {0x22222222, 0x22222222, 0x22222222, 0x22222222, 0, 0, 0, 0};
            Lacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, bp[0], Lacc, 4, 4, 0, 127, 0, (int)pscw);
            Lacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, bp[1], Lacc, 4, 4, 0, 127, 1, (int)pscw);
          }
        }
      } else if constexpr (PV == PV_FP8) {
#pragma unroll
        for (int db = 0; db < 4; db++) {
          const uint8_t* rp = Vs + (32 * db + ql) * 144;
          const uint32_t vs4 = *reinterpret_cast<const uint32_t*>(smem + sv + L::VSC + 128 * db + soff);
#pragma unroll
          for (int kc = 0; kc < 2; kc++) {
            // operand element n holds key 64kc + 32(n/16) + 16h + n%16 (see key_of)
            u4 lo = *reinterpret_cast<const u4*>(rp + 64 * kc + 16 * hh);
            u4 hi = *reinterpret_cast<const u4*>(rp + 64 * kc + 32 + 16 * hh);
            v8i av = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            if (kc == 0) O[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bp[0], O[db], 0, 0, 0, (int)vs4, 0, 127);
            else O[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bp[1], O[db], 0, 0, 2, (int)vs4, 0, 127);
          }
        }
      } else if (!(SAFE && fold)) {
        // P^ of step s (keys 64(s/4) + 32h + 8(s%4) + [0, 8) = sub-tile 2(s/4) + (s%4)/2,
        // entries 8((s%4)%2) + [0, 8)) dequantized exactly to f16 from its codes
        v8h pb[8];
#pragma unroll
        for (int s = 0; s < 8; s++) {
          const int bb = 2 * (s >> 2) + ((s & 3) >> 1);
          const _Float16 sh = (_Float16)pdq[bb];  // an E4M3 value: exact in f16
          pb[s] = dq8_f16(pc[2 * bb + ((s & 3) & 1)], v2h{sh, sh});
        }
#pragma unroll
        for (int db = 0; db < 4; db++) {
          const uint8_t* rp = Vs + (32 * db + ql) * 256;
#pragma unroll
          for (int s = 0; s < 8; s++) {
            const int chunk = (8 * (s >> 2) + 4 * hh + (s & 3)) ^ (ql & 15);
            v8h av = *reinterpret_cast<const v8h*>(rp + chunk * 16);
            O[db] = mfma_f16(av, pb[s], O[db]);
          }
        }
      } else {
        // a tile staged from the per-key form: bf16 P^' 2^sigma against bf16
        // Vk 2^(vshift - sigma), the same product scaled by 2^vshift, both exact
        v8bf pb[8];
#pragma unroll
        for (int s = 0; s < 8; s++) {
          const int bb = 2 * (s >> 2) + ((s & 3) >> 1);
          pb[s] = __builtin_bit_cast(v8bf, dq8_bf16(pc[2 * bb + ((s & 3) & 1)], pdq[bb] * psig_f));
        }
#pragma unroll
        for (int db = 0; db < 4; db++) {
          const uint8_t* rp = Vs + (32 * db + ql) * 256;
#pragma unroll
          for (int s = 0; s < 8; s++) {
            const int chunk = (8 * (s >> 2) + 4 * hh + (s & 3)) ^ (ql & 15);
            v8bf av = *reinterpret_cast<const v8bf*>(rp + chunk * 16);
            O[db] = mfma_bf16(av, pb[s], O[db]);
          }
        }
      }
    }
    if (t < nkt) {
      const uint8_t* Ks = smem + sk;
      // the Q operand: held in registers, or with causally safe V read from LDS here
      v8i qo0 = qop[0], qo1 = qop[1];
      if constexpr (SAFE && QK == QK_FP4) {
        qo0 = v8_from4(*reinterpret_cast<const u4*>(smem + L::QOFF + (32 * wave + ql) * 80 + 16 * hh));
        qo1 = v8_from4(*reinterpret_cast<const u4*>(smem + L::QOFF + (32 * wave + ql) * 80 + 32 + 16 * hh));
      }
#pragma unroll
      for (int bb = 0; bb < 4; bb++) {
        if constexpr (QK == QK_FP4) {
          const uint8_t* rp = Ks + bb * 32 * 80;
          const uint32_t ks4 = *reinterpret_cast<const uint32_t*>(Ks + L::KSC + 128 * bb + soff);
          v8i a0 = v8_from4(*reinterpret_cast<const u4*>(rp + koffk));
          v8i a1 = v8_from4(*reinterpret_cast<const u4*>(rp + koffk + 32));
          v16f acc = BIAS ? bias16(Ks + L::BOFF + 4 * key_of<SPLIT16>(bb, hh, 0)) : zero16();
          acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, qo0, acc, 4, 4, 0, (int)ks4, 0, (int)qsc);
          S[bb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, qo1, acc, 4, 4, 2, (int)ks4, 2, (int)qsc);
        } else {
          const uint8_t* rp = Ks + (32 * bb + ql) * 256;
          v16f acc = BIAS ? bias16(Ks + L::BOFF + 4 * key_of<SPLIT16>(bb, hh, 0)) : zero16();
#pragma unroll
          for (int s = 0; s < 8; s++) {
            const int chunk = (2 * s + hh) ^ (ql & 15);
            acc = mfma_f16(*reinterpret_cast<const v8h*>(rp + chunk * 16), qh16[s], acc);
          }
          S[bb] = acc;
        }
      }
      // mask (tail keys, causal diagonal) and the maxima, while the other group's wave
      // on this SIMD runs its exponentials
      const int k0 = t * 128;
      if ((k0 + 128 > klen) || (a.causal && k0 + 127 > (int)qt * 256 + 32 * wave)) {
        // keys below lim are visible (the tail, and under the causal mask the row's own
        // position); a lane's 16 keys of sub-tile bb are consecutive, so on the f16 P route
        // one count each and a compare per element (packed documents 2.5% faster).  The
        // FP4 and FP8 P routes keep the per-key test: there the count form measured
        // slower (video-DiT 32K 1.4%, GQA causal 32K 5%, neither of which masks most of
        // its tiles), the main loop's schedule shifting with it.
        const int lim = a.causal && qloc + 1 < klen ? qloc + 1 : klen;
#pragma unroll
        for (int bb = 0; bb < 4; bb++) {
          const int n = lim - (k0 + key_of<SPLIT16>(bb, hh, 0));
#pragma unroll
          for (int j = 0; j < 16; j++) {
            const bool vis = PV != PV_BF16 ? k0 + key_of<SPLIT16>(bb, hh, j) < klen &&
                                                 (!a.causal || k0 + key_of<SPLIT16>(bb, hh, j) <= qloc)
                                           : j < n;
            S[bb][j] = vis ? S[bb][j] : NEG_INF;
          }
        }
      }
#pragma unroll
      for (int bb = 0; bb < 4; bb++) {
        float x0 = fmaxn(fmaxn(S[bb][0], S[bb][1]), S[bb][2]);
        float x1 = fmaxn(fmaxn(S[bb][3], S[bb][4]), S[bb][5]);
        float x2 = fmaxn(fmaxn(S[bb][6], S[bb][7]), S[bb][8]);
        float x3 = fmaxn(fmaxn(S[bb][9], S[bb][10]), S[bb][11]);
        float x4 = fmaxn(fmaxn(S[bb][12], S[bb][13]), S[bb][14]);
        float y0 = fmaxn(fmaxn(x0, x1), x2);
        float y1 = fmaxn(fmaxn(x3, x4), S[bb][15]);
        bm16[bb] = fmaxn(y0, y1);
      }
      tmax = halves_max(fmaxn(fmaxn(bm16[0], bm16[1]), fmaxn(bm16[2], bm16[3])));
      if (PRE_IN_M && !(SAFE && vfold)) phase_v_pre();
    }
  };

  // V(t): exponentials and P quantization of tile t with the state from phase_v_pre
  auto phase_v = [&](int t) __attribute__((always_inline)) {
    if constexpr (!PRE_IN_M) phase_v_pre();
    float lsum = 0.0f;
#pragma unroll
    for (int bb = 0; bb < 4; bb++) {
      if constexpr (LOGOFF) {
        const float ls = p_sub(bb, vp_cg[bb], vp_cm, vp_k1, vp_sc[bb], vp_sv[bb], vp_ki[bb]);
        lsum += PMODE == PM_PNQ ? ls : ls * vp_lk[bb];
      } else {
        lsum += p_sub(bb, vp_ms, vp_cm, vp_k1, vp_sc[bb], vp_sv[bb], vp_ki[bb]);
      }
    }
    if constexpr (PMODE != PM_PNQ || PV != PV_FP4) lpart = vp_alpha * lpart + lsum;
  };

  // V phase of a diagonal tile with causally safe V scales ("FLAMIA" section 3.2): the
  // causal boundary of the 256-row query tile qt runs through key tiles 2 qt and
  // 2 qt + 1, which are staged in the per-key form of V.  P'_j = P~_j 2^e_j with the
  // key's per-key exponent (exact ldexp), quantized as P is; block maxima and the
  // two-level row maximum come from the P' values.  The row sum takes P~ (DIRECT,
  // TWO_LEVEL) or deq(P^'_j) 2^-e_j (PNQ).  (Group A's rows see no key of tile
  // 2 qt + 1: there every P' is 0.)
  auto phase_v_fold = [&](int t) __attribute__((always_inline)) {
    const float mnew = fmaxn(m, tmax);
    const float ms = mnew == NEG_INF ? 0.0f : mnew * lam;
    const float msub = mnew == NEG_INF ? 0.0f : mnew;
    const float cm = pexp_c(ms);
    const float alpha = m == mnew ? 1.0f : exp2_diff(m, mnew, lam);
    m = mnew;
    const uint8_t* kx = smem + L::KEYX + 128 * (t - 2 * (int)qt);  // per-key bytes, key order
    // exponent of the lane's key j of sub-tile bb (re-read where needed, not held)
    auto kexp = [&](int bb, int j) __attribute__((always_inline)) -> int {
      return (int)kx[key_of<false>(bb, hh, 0) + j] - 127;
    };
    float lsum = 0.0f, pm16[4];
#pragma unroll
    for (int bb = 0; bb < 4; bb++) {
      const u4 eb = *reinterpret_cast<const u4*>(kx + key_of<false>(bb, hh, 0));
      const uint32_t ew[4] = {eb.x, eb.y, eb.z, eb.w};
      float mx = 0.0f;
#pragma unroll
      for (int j = 0; j < 16; j++) {
        // on this one tile per row every P~ takes the difference form, so the one at
        // the row's maximum is exactly 1 and the block maxima of P' are exact there
        const float pt = pmax(S[bb][j], ms, cm, msub);
        if constexpr (PMODE != PM_PNQ) lsum += pt;
        const float pp = __builtin_ldexpf(pt, (int)((ew[j >> 2] >> (8 * (j & 3))) & 0xFFu) - 127);
        S[bb][j] = pp;
        mx = fmaxn(mx, pp);
      }
      pm16[bb] = mx;
    }
    float k1 = 1.0f, scale_o = alpha;
    if constexpr (PMODE == PM_TWO_LEVEL) {
      // s1 from the largest P' of the row; a tile whose P' stays below 2^-100 adds
      // nothing and keeps s1 (keeps 1/s1 and the carried O/s1 finite)
      const float r = halves_max(fmaxn(fmaxn(pm16[0], pm16[1]), fmaxn(pm16[2], pm16[3])));
      if (r >= 0x1p-100f) {
        const float s1 = r / 2688.0f;
        k1 = 1.0f / s1;
        scale_o = alpha * (s1prev / s1);
        s1prev = s1;
      } else {
        k1 = 0.0f;
      }
    }
    if (__builtin_amdgcn_ballot_w64(scale_o != 1.0f) != 0) {
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 16; j++) O[i][j] *= scale_o;
      Lacc[0] *= alpha;
      lfix *= alpha;
    }
    float lq = 0.0f;  // PNQ: deq(P^') 2^-e of this lane's keys
    if constexpr (PV == PV_FP4) {
      int e[2];
#pragma unroll
      for (int p = 0; p < 2; p++) {
        const int x = e8m0_exp(fmaxn(pm16[2 * p], pm16[2 * p + 1]) * k1, a.prule);
        e[p] = x < -126 ? -126 : x;
      }
      pscw = (uint32_t)(e[0] + 127) | ((uint32_t)(e[1] + 127) << 8);
      uint32_t w[8];
#pragma unroll
      for (int bb = 0; bb < 4; bb++) {
        const float sc = u2f((uint32_t)(e[bb >> 1] + 127) << 23);
        float y[16];
#pragma unroll
        for (int j = 0; j < 16; j++) y[j] = PMODE == PM_TWO_LEVEL ? S[bb][j] * k1 : S[bb][j];
        w[2 * bb] = pack8_fp4(y, sc);
        w[2 * bb + 1] = pack8_fp4(y + 8, sc);
        if constexpr (PMODE == PM_PNQ) {
#pragma unroll
          for (int u = 0; u < 2; u++)
#pragma unroll
            for (int q = 0; q < 4; q++) {
              const v2f pr = fp4_pair(w[2 * bb + u], q);
              lq += __builtin_ldexpf(pr[0] * sc, -kexp(bb, 8 * u + 2 * q)) +
                    __builtin_ldexpf(pr[1] * sc, -kexp(bb, 8 * u + 2 * q + 1));
            }
        }
      }
      bp[0] = v8_from4(mk4(w[0], w[1], w[2], w[3]));
      bp[1] = v8_from4(mk4(w[4], w[5], w[6], w[7]));
    } else {  // PV_BF16: E4M3 scale per 16 keys
#pragma unroll
      for (int bb = 0; bb < 4; bb++) {
        const float q6 = div6(pm16[bb] * k1);  // E4M3_rne_sat(fl32(M / 6)) as in phase_v_pre
        const float sv = __builtin_amdgcn_cvt_f32_fp8(__builtin_amdgcn_cvt_pk_fp8_f32(q6, q6, 0, false), 0);
        const float ki = sv > 0.0f ? __builtin_amdgcn_rcpf(sv) : 0.0f;
        float z[16];
#pragma unroll
        for (int j = 0; j < 16; j++) z[j] = (PMODE == PM_TWO_LEVEL ? S[bb][j] * k1 : S[bb][j]) * ki;
        pc[2 * bb] = pack8_fp4(z, 1.0f);
        pc[2 * bb + 1] = pack8_fp4(z + 8, 1.0f);
        pdq[bb] = sv;
        if constexpr (PMODE == PM_PNQ) {
#pragma unroll
          for (int u = 0; u < 2; u++)
#pragma unroll
            for (int q = 0; q < 4; q++) {
              const v2f pr = fp4_pair(pc[2 * bb + u], q);
              lq += __builtin_ldexpf(pr[0] * sv, -kexp(bb, 8 * u + 2 * q)) +
                    __builtin_ldexpf(pr[1] * sv, -kexp(bb, 8 * u + 2 * q + 1));
            }
        }
      }
    }
    if constexpr (PMODE == PM_PNQ && PV == PV_FP4) lfix += lq;
    else if constexpr (PMODE == PM_PNQ) lpart = alpha * lpart + lq;
    else lpart = alpha * lpart + lsum;
  };

  // ---------------- phases ----------------
  // Every wave runs M(0) V(0) M(1) V(1) ... M(nkt) with a workgroup barrier after each
  // phase.  Group B passes one extra barrier before M(0) and group A one after the
  // last phase, so B runs one phase behind A (the barrier counts still match).  In
  // V(t) a group stores its half of tile t+1+grp (loaded two phases earlier) and
  // loads its half of tile t+2+grp; tiles past the end repeat the last one into a
  // buffer that is no longer read.
  // Stage offsets rotate through 0, STAGE, 2 STAGE as scalars: sk holds tile t, sv
  // tile t-1, ss the tile this group stores next (t+1+grp).
  if constexpr (SAFE) {
    // the per-key exponents of key tiles 2 qt and 2 qt + 1, 256 bytes in key order
    // (dwords past the padded row repeat its last one: those keys are masked)
    if (tid < 64) {
      const uint8_t* hvks = a.vks + (b * a.Hkv + hk) * (int64_t)np;
      const uint32_t s0 = __builtin_elementwise_min((uint32_t)vstart + 256u * (uint32_t)qt + 4u * tid, np - 4);
      *reinterpret_cast<uint32_t*>(smem + L::KEYX + 4 * tid) = *reinterpret_cast<const uint32_t*>(hvks + s0);
    }
  }
  load_half(0);
  store_half(0);
  if (grp == 1) {
    load_half(nkt > 1 ? 1 : 0);
    store_half(STAGE);
  }
  load_half(nkt > 1 + grp ? 1 + grp : nkt - 1);
  __syncthreads();
  if (grp == 1) __syncthreads();
  auto rot = [](uint32_t o) { return o == 2 * STAGE ? 0u : o + STAGE; };
  uint32_t sk = 0, sv = 2 * STAGE, ss = grp == 0 ? STAGE : 2 * STAGE;
  // one M phase and one V phase; mfold and vfold (constants at each call) select the
  // forms of the diagonal tiles 2 qt and 2 qt + 1 under causally safe V: their V phases
  // fold the per-key exponents into P, and the M phases that follow take their PV from
  // the per-key form
  // Issue priority: the SIMD issues the older wave first, so a phase of the younger
  // group waits behind the co-resident wave's stream.  Where one phase's stream is the
  // one that holds up the pair, it runs at raised priority (s_setprio): the M phase
  // on the FP4 PV route (its MFMAs need an issue slot every 32 cycles, and its scale
  // chain ends the phase: video-DiT 32K 5.88 -> 5.60 ms, two-level E8M0 1.3% faster),
  // the V phase on the f16 PV route (two-level E4M3 32K 11.20 -> 10.90 ms, packed
  // documents 2-3% faster); the FP8 PV route measured best without.
  constexpr int MPRIO = QK == QK_FP4 && PV == PV_FP4 ? 1 : 0;
  constexpr int VPRIO = QK == QK_FP4 && PV == PV_BF16 ? 1 : 0;
  auto step = [&](int t, bool mfold, bool vfold) __attribute__((always_inline)) {
    if constexpr (MPRIO) __builtin_amdgcn_s_setprio(MPRIO);
    phase_m(t, sk, sv, mfold, vfold);
    __builtin_amdgcn_sched_barrier(0);  // keep the phase's MFMAs on this side of the barrier
    if constexpr (MPRIO) __builtin_amdgcn_s_setprio(0);
    __syncthreads();
    if (t < nkt) {
      // the f16 route stages the next tiles before its exponentials, in that order
      // (packed documents 3.5% faster; the other routes measured the same either way)
      constexpr bool STAGE_FIRST = PV == PV_BF16;
      const int nt = t + 2 + grp;
      if constexpr (VPRIO) __builtin_amdgcn_s_setprio(VPRIO);
      if constexpr (STAGE_FIRST) {
        store_half(ss);
        load_half(nt < nkt ? nt : nkt - 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (SAFE && vfold) phase_v_fold(t);
      else phase_v(t);
      if constexpr (VPRIO) __builtin_amdgcn_s_setprio(0);
      if constexpr (!STAGE_FIRST) {
        store_half(ss);
        load_half(nt < nkt ? nt : nkt - 1);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    sv = sk;
    sk = __builtin_amdgcn_readfirstlane(rot(sk));
    ss = __builtin_amdgcn_readfirstlane(rot(ss));
  };
  // tiles before 2 qt need no fold; step 2 qt folds in its V phase only, the steps
  // after it in both phases (each copy of the step holds one form of each phase, which
  // keeps the register allocation of the main loop)
  const int tsplit = SAFE ? (2 * (int)qt < nkt + 1 ? 2 * (int)qt : nkt + 1) : nkt + 1;
  for (int t = 0; t < tsplit; t++) step(t, false, false);
  if constexpr (SAFE) {
    if (tsplit <= nkt) step(tsplit, false, true);
    for (int t = tsplit + 1; t <= nkt; t++) step(t, true, true);
  }
  if (grp == 0) __syncthreads();

  // ---------------- epilogue ----------------
  float l;
  if constexpr (PMODE == PM_PNQ && PV == PV_FP4) l = SAFE ? Lacc[0] + halves_sum(lfix) : Lacc[0];
  else l = halves_sum(lpart);
  float inv = l > 0.0f ? 1.0f / l : 0.0f;
  if constexpr (PMODE == PM_TWO_LEVEL) inv *= s1prev;
  if constexpr (PV == PV_FP8) inv = inv / 448.0f;
  if constexpr (H16) {  // undo each channel's 2^vshift (exact); register j of block db
                         // holds channel 32 db + 8 (j / 4) + 4 hh + j % 4
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 16; j++)
        O[i][j] = __builtin_ldexpf(O[i][j] * inv, -vshift_lds[32 * i + 8 * (j >> 2) + 4 * hh + (j & 3)]);
    inv = 1.0f;
  }
  if (qloc < klen) {
    const int64_t orow = qstart + qloc;
    if (a.out_fp32) {
      float* op = static_cast<float*>(a.out) + b * a.oB + hq * a.oH + orow * a.oN;
#pragma unroll
      for (int db = 0; db < 4; db++)
#pragma unroll
        for (int g = 0; g < 4; g++) {
          float4 t4 = make_float4(O[db][4 * g] * inv, O[db][4 * g + 1] * inv, O[db][4 * g + 2] * inv,
                                  O[db][4 * g + 3] * inv);
          *reinterpret_cast<float4*>(op + 32 * db + 8 * g + 4 * hh) = t4;
        }
    } else {
      uint16_t* op = static_cast<uint16_t*>(a.out) + b * a.oB + hq * a.oH + orow * a.oN;
#pragma unroll
      for (int db = 0; db < 4; db++)
#pragma unroll
        for (int g = 0; g < 4; g++) {
          u2 t2 = mk2(bf16_rne(O[db][4 * g] * inv) | (bf16_rne(O[db][4 * g + 1] * inv) << 16),
                      bf16_rne(O[db][4 * g + 2] * inv) | (bf16_rne(O[db][4 * g + 3] * inv) << 16));
          *reinterpret_cast<u2*>(op + 32 * db + 8 * g + 4 * hh) = t2;
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
template <int QK, int PV, int PMODE, int PSC, int VSC, bool BIAS>
static hipError_t launch_one_b(const FwdArgs& a, hipStream_t st) {
  constexpr int bytes = Lds<QK, PV, BIAS>::BYTES;
  auto kern = fwd_kernel<QK, PV, PMODE, PSC, VSC, BIAS>;
  if (bytes > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
  }
  kern<<<dim3((unsigned)a.grid), dim3(256), bytes, st>>>(a);
  return hipGetLastError();
}

template <int QK, int PV, int PMODE, int PSC, int VSC>
static hipError_t launch_one(const FwdArgs& a, hipStream_t st) {
  if (a.bias != nullptr) return launch_one_b<QK, PV, PMODE, PSC, VSC, true>(a, st);
  return launch_one_b<QK, PV, PMODE, PSC, VSC, false>(a, st);
}

template <int QK, int PV, int PMODE, int PSC, bool BIAS, bool SAFE>
static hipError_t launch_pp_k(const FwdArgs& a, hipStream_t st) {
  if (a.exp_bits)
    fwd_pp_kernel<QK, PV, PMODE, PSC, BIAS, SAFE, true><<<dim3((unsigned)a.grid), dim3(512), 0, st>>>(a);
  else
    fwd_pp_kernel<QK, PV, PMODE, PSC, BIAS, SAFE, false><<<dim3((unsigned)a.grid), dim3(512), 0, st>>>(a);
  return hipGetLastError();
}

template <int QK, int PV, int PMODE, int PSC>
static hipError_t launch_pp(FwdArgs a, hipStream_t st) {
  if (a.plan == nullptr) a.grid = a.B * a.Hq * ((a.N + 255) / 256);
  const bool bias = a.bias != nullptr;
  if constexpr (PV == PV_FP4 || PV == PV_BF16) {
    if (a.vk != nullptr)
      return bias ? launch_pp_k<QK, PV, PMODE, PSC, true, true>(a, st)
                  : launch_pp_k<QK, PV, PMODE, PSC, false, true>(a, st);
  } else if (a.vk != nullptr) {
    return hipErrorNotSupported;
  }
  return bias ? launch_pp_k<QK, PV, PMODE, PSC, true, false>(a, st)
              : launch_pp_k<QK, PV, PMODE, PSC, false, false>(a, st);
}

hipError_t launch_fwd(int qk, int pv, int pmode, int psc, int vsc, const FwdArgs& a, hipStream_t st) {
  // ping-pong kernel: every route whose three key-tile buffers fit in LDS (V with E8M0
  // scales per 32 keys; not bf16 on both products)
#define MXP(QK_, PV_, PM_, PS_) \
  if (qk == QK_ && pv == PV_ && pmode == PM_ && psc == PS_ && vsc == SCALE_E8M0) return launch_pp<QK_, PV_, PM_, PS_>(a, st)
  MXP(QK_FP4, PV_FP4, PM_DIRECT, SCALE_E8M0);
  MXP(QK_FP4, PV_FP4, PM_PNQ, SCALE_E8M0);
  MXP(QK_FP4, PV_FP4, PM_TWO_LEVEL, SCALE_E8M0);
  MXP(QK_FP4, PV_BF16, PM_DIRECT, SCALE_E4M3);
  MXP(QK_FP4, PV_BF16, PM_PNQ, SCALE_E4M3);
  MXP(QK_FP4, PV_BF16, PM_TWO_LEVEL, SCALE_E4M3);
  MXP(QK_BF16, PV_FP8, PM_FP8_FIXED, SCALE_E8M0);
  MXP(QK_FP4, PV_FP8, PM_FP8_FIXED, SCALE_E8M0);
#undef MXP
  // the 4-wave kernel has no per-key V form and only the exact exponential: causally
  // safe V scales and bit-level exponentials are refused there
  if (a.vk != nullptr || a.exp_bits) return hipErrorNotSupported;
#define MXF(QK_, PV_, PM_, PS_, VS_) \
  if (qk == QK_ && pv == PV_ && pmode == PM_ && psc == PS_ && vsc == VS_) return launch_one<QK_, PV_, PM_, PS_, VS_>(a, st)
  // the rest (V with E4M3 scales per 16 keys; bf16 scores with FP4 PV): single-buffer kernel
  MXF(QK_BF16, PV_FP4, PM_DIRECT, SCALE_E8M0, SCALE_E8M0);
  MXF(QK_BF16, PV_FP4, PM_PNQ, SCALE_E8M0, SCALE_E8M0);
  MXF(QK_BF16, PV_FP4, PM_TWO_LEVEL, SCALE_E8M0, SCALE_E8M0);
  MXF(QK_BF16, PV_BF16, PM_DIRECT, SCALE_E4M3, SCALE_E4M3);
  MXF(QK_BF16, PV_BF16, PM_PNQ, SCALE_E4M3, SCALE_E4M3);
  MXF(QK_BF16, PV_BF16, PM_TWO_LEVEL, SCALE_E4M3, SCALE_E4M3);
  MXF(QK_BF16, PV_BF16, PM_DIRECT, SCALE_E8M0, SCALE_E4M3);
  MXF(QK_BF16, PV_BF16, PM_TWO_LEVEL, SCALE_E8M0, SCALE_E4M3);
  MXF(QK_FP4, PV_BF16, PM_DIRECT, SCALE_E4M3, SCALE_E4M3);
  MXF(QK_FP4, PV_BF16, PM_TWO_LEVEL, SCALE_E4M3, SCALE_E4M3);
  MXF(QK_FP4, PV_BF16, PM_PNQ, SCALE_E4M3, SCALE_E4M3);
  MXF(QK_RAW, PV_RAW, PM_NONE, SCALE_E8M0, SCALE_E8M0);  // unquantized route
#undef MXF
  return hipErrorNotSupported;  // no kernel instantiated for this route
}

}  // namespace mxattn
