/*
 * oracle.h -- plain, slow CPU reference for microscaling-FP4 attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library.  It shares no code, header, table or
 * constant with the GPU library; the GPU path never calls it.
 *
 * Every routine states the passage it follows.  Sources, by title:
 *   [MXF4]  "Microscaling FP4 Attention: Why the Softmax Operand Needs Two Scale
 *           Factors" (blog post on SageAttention3's two-level scaling)
 *   [MXA]   "MXAttention: Data-Free Optimal Scaling and Pre-Normalization
 *           Quantization for MXFP4 Attention"
 *   [SA3]   "SageAttention3 -- L2 Deep Analysis"
 *   [FLAMIA]"FLAMIA: FLAsh MIcroscaling Attention for Fast and Causally Safe
 *           Training on Blackwell"
 *   [MPFA]  "MpFA: Hardware-Efficient Train-Free QK4V8 FlashAttention Kernels on
 *           Blackwell GPUs"
 *
 * Arithmetic conventions (where the pages say FP32 the oracle uses single IEEE
 * operations in program order; compiled with -ffp-contract=off, no fast-math):
 *   - dot products: exact products of dequantized values summed in double, then
 *     rounded once to float;
 *   - exponentials: exp() in double of sm_scale*(s - m) formed in double from
 *     float operands, rounded once to float (the bit-level modes take the exact
 *     piecewise-linear value of the same argument instead);
 *   - divisions x/scale, M/6, P/s1, 448*P: single float operations.
 *
 * Parity status of every function is recorded next to it ("pinned by ..." names
 * the test file that fixes it against the pages or mathematics).
 */
#ifndef MXATTN_ORACLE_H
#define MXATTN_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element formats */
enum { ORC_ELEM_E2M1 = 0, ORC_ELEM_E4M3 = 1 };
/* block scale formats */
enum { ORC_SCALE_E8M0 = 0, ORC_SCALE_E4M3 = 1 };
/* E8M0 exponent rules ([MXA] section 2 and Table 1) */
enum { ORC_RULE_OCP = 0, ORC_RULE_CEIL = 1 };
/* how the softmax operand P is quantized inside the loop */
enum {
  ORC_P_NONE = 0,      /* unquantized P (textbook online softmax)            */
  ORC_P_DIRECT = 1,    /* phi(P~), row sum from unquantized P~ ([MXA] 5.2)   */
  ORC_P_TWO_LEVEL = 2, /* [MXF4] "Two-level scaling", [SA3] Eq. 5            */
  ORC_P_PNQ = 3,       /* [MXA] section 4.2 and Algorithm 1                  */
  ORC_P_FP8_FIXED = 4  /* [MPFA] section 4.1: cast_e4m3(448 P~)/448          */
};

typedef struct {
  int elem;    /* ORC_ELEM_*                                  */
  int scale;   /* ORC_SCALE_*                                 */
  int block;   /* elements sharing one scale (16 or 32)       */
  int rule;    /* ORC_RULE_* (E8M0 scales only)               */
  float qmax;  /* CEIL rule boundary: 6, 7.25, 448, ...       */
} orc_fmt;

/* the exponential that turns scores into P~ ([FLAMIA] section 3.7, appendix C) */
enum {
  ORC_EXP_EXACT = 0,      /* exp() in double, rounded to float                 */
  ORC_EXP_MITCHELL = 1,   /* Mitchell's line, error centred (Mitchell-P)       */
  ORC_EXP_SCHRAUDOLPH = 2 /* the same line, ratio to exp averaging one         */
};

typedef struct {
  int pmode;      /* ORC_P_*                                       */
  orc_fmt pfmt;   /* block format of P (DIRECT, TWO_LEVEL, PNQ)     */
  int causal;     /* key j visible to query i iff j <= i            */
  float sm_scale; /* 1/sqrt(d)                                      */
  int kv_tile;    /* keys per online-softmax step                   */
  int exp_mode;   /* ORC_EXP_*: the exponential of P~ (the rescale  */
                  /* factor between tiles stays exact)              */
  int score_rounds; /* flip budget only: FP32 roundings in the score   */
                  /* sums of the implementation under test (0: 2)   */
  int q_tile;     /* query rows per tile, from the sequence or      */
                  /* document start (0: kv_tile); with the per-key  */
                  /* V form it fixes a row's diagonal tiles         */
} orc_attn_params;

/* ---- bit-level exponentials ([FLAMIA] section 3.7, appendix C) ----
 * orc_exp2_bits(t): the value whose float bits are 2^23 (t + 127) read as an
 * integer -- Mitchell's piecewise-linear 2^t = 2^floor(t) (1 + t - floor(t)) for
 * t >= -126, continued by the subnormal line (t + 127) 2^-126 down to 0 at t = -127,
 * and 0 below (the clamp) and for NaN.  Exact real arithmetic in double.
 * orc_exp_offset(mode): delta subtracted from t before the line (0 for EXACT):
 * Mitchell-P centres log2 of the line's ratio to 2^t, Schraudolph's form makes
 * that ratio average one over an octave.  Pinned by tests/test_oracle_bitexp.py. */
double orc_exp2_bits(double t);
double orc_exp_offset(int exp_mode);

/* ---- formats ---- */
double orc_e2m1_value(int code);            /* code: sign<<3 | magnitude index     */
int orc_e2m1_encode(float x);               /* nearest grid value, ties to even    */
double orc_e4m3_value(int byte);            /* OCP E4M3 (no inf; S.1111.111 = NaN) */
int orc_e4m3_encode(float x);               /* nearest finite value, ties to even  */
int orc_e8m0_exponent(float amax, int rule, float qmax, int elem);
double orc_scale_value(const orc_fmt* f, int sbyte);

/* Quantize n values that share one scale.  Writes n codes (one per byte) and the
 * scale byte; returns the scale as a float. */
float orc_quant_block(const float* x, int n, const orc_fmt* f, uint8_t* codes, uint8_t* sbyte);

/* Q and K role: blocks of f->block consecutive elements along d, per row.
 * x: [rows][d] (bf16 values widened to float); codes: [rows][d]; scales: [rows][d/block] */
void orc_quantize_rows(const float* x, int64_t rows, int d, const orc_fmt* f,
                       uint8_t* codes, uint8_t* scales);
void orc_dequant_rows(const uint8_t* codes, const uint8_t* scales, int64_t rows, int d,
                      const orc_fmt* f, float* out);

/* V role: blocks of f->block consecutive tokens per channel, document-local.
 * x: [N][d]; doc_off: ndocs+1 offsets (NULL -> one document [0,N));
 * codes: [d][N]; scales: [d][nblk], blocks listed document by document,
 * nblk = sum over documents of ceil(L/block). */
int64_t orc_v_nblocks(int N, const int* doc_off, int ndocs, int block);
void orc_quantize_cols(const float* x, int N, int d, const int* doc_off, int ndocs,
                       const orc_fmt* f, uint8_t* codes, uint8_t* scales);
void orc_dequant_cols(const uint8_t* codes, const uint8_t* scales, int N, int d,
                      const int* doc_off, int ndocs, const orc_fmt* f, float* out /*[N][d]*/);

/* One query row.  K, V: [nk][d] dequantized keys/values of the row's key range
 * (a document, or the whole sequence); tiles are aligned to key 0 of that range.
 * vis: number of visible keys (keys 0..vis-1).  Outputs o[d], *lse and the row's
 * flip budget *fb: a bound on |dO| from the rounding decisions (element codes,
 * block scales) whose input lies within its window of a threshold, the window
 * being a bound on how far an FP32 implementation's value of that input can be
 * from this oracle's (p_window in oracle.c states it term by term).  Returns 0. */
int orc_attn_row(const float* q, const float* K, const float* V, int nk, int vis, int d,
                 const orc_attn_params* p, float* o, float* lse, double* fb);

/* Multi-head driver.  Q: [B][Hq][N][d], K,V: [B][Hkv][N][d] dequantized.
 * doc_off/ndocs: packed documents (requires B == 1), or NULL/0.
 * rows: flat row ids ((b*Hq + h)*N + i), or NULL for all B*Hq*N rows.
 * O: [nrows][d]; lse, fb: [nrows] (may be NULL). */
int orc_attention(const float* Q, const float* K, const float* V, int B, int Hq, int Hkv, int N,
                  int d, const int* doc_off, int ndocs, const orc_attn_params* p,
                  const int64_t* rows, int64_t nrows, float* O, float* lse, double* fb);

/* As orc_attention, plus an optional per-key score bias: bias [B][Hq][N] (NULL for
 * none) is added to every score of its key before masking and before the running
 * maximum, s = fl32(exact dot + bias) ([MPFA] section 4.3, Eq. 10). */
int orc_attention_bias(const float* Q, const float* K, const float* V, const float* bias, int B,
                       int Hq, int Hkv, int N, int d, const int* doc_off, int ndocs,
                       const orc_attn_params* p, const int64_t* rows, int64_t nrows, float* O,
                       float* lse, double* fb);

/* As orc_attention_bias, plus the causally safe form of a 4-bit V ([FLAMIA] section
 * 3.2): Vk [B][Hkv][N][d] holds the E2M1 values of V's per-key form (unit scale)
 * and ek [B][Hkv][N] its per-key exponents (orc_quantize_keys).  Queries are taken
 * in tiles of q_tile rows from the start of their sequence or document; the causal
 * boundary of a query tile runs through the key tiles that start inside its rows'
 * span, [q_tile floor((i - start) / q_tile), + q_tile) -- the row's diagonal tiles.
 * On them P~_j is multiplied by 2^ek[j] before it is quantized and multiplies Vk;
 * every other tile uses V.  Requires a causal mask (returns -3 otherwise) and a
 * q_tile that is a multiple of kv_tile (returns -5); Vk/ek NULL: as
 * orc_attention_bias. */
int orc_attention_ex(const float* Q, const float* K, const float* V, const float* bias, const float* Vk,
                     const int* ek, int B, int Hq, int Hkv, int N, int d, const int* doc_off, int ndocs,
                     const orc_attn_params* p, const int64_t* rows, int64_t nrows, float* O, float* lse,
                     double* fb);

/* Per-key form of V: per token j, one E8M0 scale 2^ek[j] for its d channels by f's
 * rule and the element codes of V[j][c] / 2^ek[j].  x, codes: [N][d]; ek: [N]. */
void orc_quantize_keys(const float* x, int N, int d, const orc_fmt* f, uint8_t* codes, int* ek);

/* Decode with a split key range ([MPFA] section 5.3: the history is cut into fixed
 * partitions, each keeps its own (m, l, O) state, and the states are merged by their
 * log-sum-exp).  Q: [B][Hq][R][d] -- the R newest tokens of each request, row r at
 * position kv_len[b] - R + r, attending causally to the kv_len[b] keys of K, V:
 * [B][Hkv][N][d] (dequantized; N >= every kv_len).  The keys are cut into splits of
 * `split` keys from key 0; each split runs orc_attn_row over its own keys (tiles of
 * kv_tile from the split start, P quantized per tile against the split's running
 * maximum), giving o_s and lse_s (a split that sees no key has lse_s = -inf).  The
 * merge, in double: M = max lse_s, w_s = exp(lse_s - M), O = sum w_s o_s / sum w_s,
 * lse = M + log(sum w_s).  fb: the merged flip budget sum w_s fb_s / sum w_s.
 * O: [B][Hq][R][d]; lse, fb: [B][Hq][R] (may be NULL). */
int orc_decode(const float* Q, const float* K, const float* V, int B, int Hq, int Hkv, int R, int N,
               int d, const int* kv_len, int split, const orc_attn_params* p, float* O, float* lse,
               double* fb);

/* ---- outlier pre-processing of Q and K (before quantization) ---- */

/* Per-channel mean over the tokens of each document of one head ([MPFA] section
 * 4.2, Eq. 7; [MXF4] "Smooth-K is the smaller lever": K.mean over tokens).
 * x: [N][d]; doc_off/ndocs as above (NULL/0: one document [0, N)).
 * mean: [max(ndocs,1)][d], mean = fl32(sum / L) with the sum over the document's
 * tokens taken in double in token order (exact for bf16 inputs whose magnitudes
 * span less than 2^38) and the division in double; an empty document gets 0.
 * Pinned by tests/test_oracle_preproc.py. */
void orc_channel_mean(const float* x, int N, int d, const int* doc_off, int ndocs, float* mean);

/* Pre-processed rows y = fl32(((x - mu) H) c) of one head: mu is the channel mean of
 * the token's document (mean may be NULL: mu = 0), H the d x d Sylvester Hadamard
 * matrix H[i][j] = (-1)^popcount(i & j) when hadamard != 0 (else the identity) and
 * c = fl64(1/sqrt(d)) with the rotation, 1 without it.  The normalized rotation is
 * orthogonal, so it keeps every Q.K dot product ([FLAMIA] section 3.4 and appendix
 * A.2); centering follows [MPFA] section 4.2.  x - mu and the +-1 sum are formed
 * exactly in double (bf16 x, float mu), then multiplied by c in double and rounded
 * once to float.  out: [N][d].  Pinned by tests/test_oracle_preproc.py. */
void orc_preprocess_rows(const float* x, int N, int d, const float* mean, const int* doc_off,
                         int ndocs, int hadamard, float* out);

/* Centering compensation of one query head ([MPFA] section 4.3, Eq. 9):
 * delta[j] = fl32(sum_c qmean[doc(j)][c] * (K[j][c] - kmean[doc(j)][c])), the
 * products and the sum in double in channel order.  K: [N][d] of the query head's
 * KV head; qmean, kmean: [max(ndocs,1)][d]; delta: [N].
 * Pinned by tests/test_oracle_preproc.py. */
void orc_center_comp(const float* qmean, const float* K, const float* kmean, int N, int d,
                     const int* doc_off, int ndocs, float* delta);

#ifdef __cplusplus
}
#endif
#endif
