// kernels.h -- launch arguments shared by the host library and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "formats.h"

namespace mxattn {

// element / scale / P-mode values (the mxattn.h enums)
enum { ELEM_E2M1 = 0, ELEM_E4M3 = 1 };
enum { SCALE_E8M0 = 0, SCALE_E4M3 = 1 };
enum { PM_NONE = 0, PM_DIRECT = 1, PM_TWO_LEVEL = 2, PM_PNQ = 3, PM_FP8_FIXED = 4 };

struct QuantArgs {
  const void* x;
  int64_t sB, sH, sN;  // element strides of x (the channel stride is 1)
  int64_t B, H, N;
  int64_t np;  // role V: padded key count (multiple of 128)
  int elem, scale, block;
  E8m0Rule rule;
  const int32_t* cu;  // role V: device document offsets, or null
  int ndocs;
  void* codes;
  void* scales;
  int tiled;  // role VT: V written tile-major ([tile][channel][64 B] codes, [tile][channel][4 B] scales)
};

hipError_t launch_quant_qk(const QuantArgs& a, hipStream_t st);
hipError_t launch_quant_v(const QuantArgs& a, hipStream_t st);
// role VKEY: per-key E8M0 scale over the 128 channels, codes transposed as role V
hipError_t launch_quant_vkey(const QuantArgs& a, hipStream_t st);
// unquantized (bf16) tensors: x with element strides (sB, sH, sN, 1) copied densely to
// dst [B][H][N][128]
hipError_t launch_copy_bf16(const void* x, int64_t sB, int64_t sH, int64_t sN, int64_t B, int64_t H, int64_t N,
                            void* dst, hipStream_t st);

// outlier pre-processing (preproc.hip)
// mean: [B][H][nd][128] float, nd = max(ndocs, 1); a.cu/a.ndocs give the documents
hipError_t launch_channel_mean(const QuantArgs& a, float* mean, hipStream_t st);
// role QK quantization of fl32(((x - mean) H) c); mean may be null, hadamard 0/1
hipError_t launch_quant_qk_pre(const QuantArgs& a, const float* mean, int hadamard, hipStream_t st);

struct CompArgs {
  const float* qmean;  // [B][Hq][nd][128]
  const void* k;       // bf16 [B][Hkv][N][128], element strides sB, sH, sN
  int64_t sB, sH, sN;
  const float* kmean;  // [B][Hkv][nd][128]
  int64_t B, Hq, Hkv, N;
  const int32_t* cu;   // device document offsets, or null
  int ndocs;
  float* delta;        // [B][Hq][N]
};
hipError_t launch_center_comp(const CompArgs& a, hipStream_t st);

// Operand routes of the forward kernel.
//   QK_FP4 : Q and K in E2M1 with E8M0/32 scales, scaled FP4 MFMA.
//   QK_BF16: Q and K in E2M1 with E4M3/16 scales, dequantized (exactly) to bf16,
//            bf16 MFMA.
//   PV_FP4 : P in E2M1 with E8M0/32 scales, V in E2M1 with E8M0/32, scaled FP4 MFMA.
//   PV_BF16: P and V in E2M1 with E8M0/32 or E4M3/16 scales, dequantized to bf16.
//   PV_FP8 : P as E4M3(448 P~) with unit scale, V in E4M3 with E8M0/32, scaled FP8 MFMA.
//   QK_RAW, PV_RAW: the unquantized route: Q, K, V in bf16 ([B][H][N][128], V not
//            transposed; V^T tiles are formed while staging), P~ rounded to bf16.
enum { QK_FP4 = 0, QK_BF16 = 1, QK_RAW = 2 };
enum { PV_FP4 = 0, PV_BF16 = 1, PV_FP8 = 2, PV_RAW = 3 };

// Document entry of a forward plan (workspace): first token, length, and the first
// padded key slot of the document in a V layout with blocks of 32 and of 16.
struct DocEntry {
  int32_t start, len, voff32, voff16;
};
// Work item of a forward plan: document and query tile (from the document's first
// token).
struct WorkItem {
  int32_t doc, qtile;
};
// Workspace header of a plan.  After it: DocEntry[ndocs], then the work list of
// 128-row query tiles (cap128 entries, n_items used), then the work list of 256-row
// query tiles (n_items256 used); each list longest first.
struct PlanHeader {
  int32_t n_items, ndocs, causal, magic;
  int32_t n_items256, cap128, n_tokens, pad1;  // n_tokens: N the plan was built for
};
constexpr int32_t PLAN_MAGIC = 0x4D585031;  // "MXP1"

struct FwdArgs {
  // Q codes [B][Hq][N][64 B], scales [B][Hq][N][4 or 8 B]
  const uint8_t* q;
  const uint8_t* qs;
  const uint8_t* k;
  const uint8_t* ks;
  // V^T codes [B][Hkv][128][np * bits / 8], scales [B][Hkv][128][np / vblock]
  const uint8_t* v;
  const uint8_t* vs;
  int64_t B, Hq, Hkv, N, np;
  float lambda;    // sm_scale * log2(e)
  float sm_scale;  // for the log-sum-exp
  int causal;
  E8m0Rule prule;  // E8M0 rule of P (PV_FP4 and PV_BF16 with E8M0 P)
  void* out;
  int64_t oB, oH, oN;  // element strides of out
  int out_fp32;
  float* lse;
  const PlanHeader* plan;  // packed documents, or null
  int ndocs;               // documents of the plan (checked against its header)
  int64_t grid;            // workgroups launched
  const float* bias;       // per-key score bias [B][Hq][N] (centering compensation), or null
  // per-key form of V for causally safe diagonal tiles (null: grouped V scales only):
  // codes [B][Hkv][128][np / 2] (E2M1), one E8M0 byte per key slot [B][Hkv][np]
  const uint8_t* vk;
  const uint8_t* vks;
  // exponential of P~: 0 exact (v_exp_f32); 1 bit-level, P~ = exp2_bits(s lambda 2^23 +
  // exp_bias - m lambda 2^23) with exp_bias = 2^23 (127 - delta) of the chosen offset
  int exp_bits;
  float exp_bias;
};

// split-key decode (decode.hip)
struct DecArgs {
  const uint8_t* q;   // Q codes [B][Hq][R][64 B], scales [B][Hq][R][4]
  const uint8_t* qs;
  const uint8_t* k;   // K codes [B][Hkv][N][64 B], scales [B][Hkv][N][4]
  const uint8_t* ks;
  const uint8_t* v;   // V^T codes [B][Hkv][128][np / 2], scales [B][Hkv][128][np / 32] (vtiled: tile-major,
                      // [B][Hkv][np / 128][128][64 B] and [B][Hkv][np / 128][128][4 B])
  const uint8_t* vs;
  int64_t B, Hq, Hkv, R, N, np;
  const int32_t* kv_len;  // device [B] keys of each request, or null (N each)
  int vtiled;             // V is role VT (tile-major)
  int qk_fp4;             // FP8 V route: Q/K MXFP4 (1) or NVFP4 (0, scales [..][8], E4M3 per 16)
  float lambda, sm_scale;
  E8m0Rule prule;
  int64_t nsplit;  // 512-key chunks of the longest history: ceil(N / 512)
  float* ws_o;     // [B][Hq][R][nsplit][128] normalized chunk outputs (4 tiles merged)
  float* ws_lse;   // [B][Hq][R][nsplit]
  void* out;       // [B][Hq][R][128] with element strides oB, oH, oN
  int64_t oB, oH, oN;
  int out_fp32;
  float* lse;      // [B][Hq][R] or null
};
hipError_t launch_decode(int pmode, const DecArgs& a, hipStream_t st);

// Allocation-free decode: the split states live in a file-scope device array of
// DECODE_SCRATCH_BYTES (decode.hip), one copy per GPU.  decode_scratch() returns its
// address on the current device (looked up once per device with hipGetSymbolAddress).
constexpr size_t DECODE_SCRATCH_BYTES = size_t(32) << 20;
hipError_t decode_scratch(void** ptr);

// psc: P block scale (SCALE_E8M0 -> blocks of 32, SCALE_E4M3 -> blocks of 16);
// vsc: V block scale (same meaning).
hipError_t launch_fwd(int qk, int pv, int pmode, int psc, int vsc, const FwdArgs& a, hipStream_t st);

}  // namespace mxattn
