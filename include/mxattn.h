/*
 * mxattn.h -- C ABI of the microscaling-FP4 attention forward for AMD MI355X (gfx950).
 *
 * The library computes S = Q K^T, P = OnlineSoftmax(S), O = P V (the attention
 * statement of "SageAttention3 -- L2 Deep Analysis", Q1, and of "MXAttention",
 * section 2) on block-quantized operands:
 *   - Q, K and V are quantized once, outside the attention loop, by
 *     mxattn_quantize() to E2M1 codes with a shared scale per block
 *     (MXFP4: 1x32 blocks with an E8M0 scale; NVFP4-style: 1x16 blocks with an
 *     E4M3 scale), or V to E4M3 codes with an E8M0 scale per 32 keys
 *     ("MpFA", section 4.1 (FP8 V); "FLAMIA", section 3.2 (power-of-two token
 *     block scales)).
 *   - mxattn_fwd() runs the tiled FlashAttention-2 recurrence and quantizes the
 *     softmax operand P inside the loop: directly, with the two-level scheme
 *     ("Microscaling FP4 Attention" blog, section "Two-level scaling";
 *     SageAttention3 notes, Q2 Eq. 5), with pre-normalization quantization
 *     ("MXAttention", section 4.2 and Algorithm 1) or with the fixed FP8 scale
 *     448 ("MpFA", section 4.1).  PV accumulates in FP32.
 *
 * Conventions shared by every entry point:
 *   - Pointers are DEVICE pointers unless the parameter name ends in _host.
 *   - The caller allocates and owns every buffer.  The library never allocates,
 *     frees or synchronizes; it enqueues work on the caller's HIP stream
 *     (`stream`, a hipStream_t passed as void*, NULL = default stream) and returns.
 *     Buffers must stay alive until that work has completed.
 *   - Every entry point validates its arguments on the host first.  On failure
 *     it returns a negative mxattn_status and enqueues nothing.  A failed kernel
 *     launch returns MXATTN_E_HIP; mxattn_last_error() then holds the text.
 *   - No C++ exception crosses this interface.  Outputs are bitwise
 *     deterministic for identical inputs and parameters.
 */
#ifndef MXATTN_H
#define MXATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MXATTN_ABI_VERSION 8

typedef enum {
  MXATTN_OK = 0,
  MXATTN_E_INVALID = -1,     /* bad pointer, shape, enum or stride              */
  MXATTN_E_UNSUPPORTED = -2, /* valid but not implemented (e.g. d != 128)       */
  MXATTN_E_ALIGN = -3,       /* a pointer or row is not 16-byte aligned          */
  MXATTN_E_WORKSPACE = -4,   /* workspace missing or smaller than required       */
  MXATTN_E_HIP = -5          /* a HIP call failed; see mxattn_last_error()       */
} mxattn_status;

/* element format of the codes */
typedef enum {
  MXATTN_ELEM_E2M1 = 0, /* FP4: magnitudes {0,.5,1,1.5,2,3,4,6}, sign bit 3, 2 codes per
                           byte with the even element in the low nibble            */
  MXATTN_ELEM_E4M3 = 1, /* OCP FP8 E4M3: one code per byte, max 448, no infinity   */
  MXATTN_ELEM_BF16 = 2  /* unquantized: the bf16 values themselves, with scale NONE
                           ("MXAttention" section 2, "MpFA" section 3 Eq. 2: the
                           attention the quantized routes approximate); every role
                           keeps the [B][H][N][d] layout (V is not transposed)     */
} mxattn_elem;

/* format of the shared block scale */
typedef enum {
  MXATTN_SCALE_E8M0 = 0, /* power of two 2^e, byte e + 127 (0xFF never written)  */
  MXATTN_SCALE_E4M3 = 1, /* OCP E4M3 value s = E4M3(amax / 6)                      */
  MXATTN_SCALE_NONE = 2  /* no scale: bf16 elements only                             */
} mxattn_scale;

/* how an E8M0 exponent is chosen from the block maximum M ("MXAttention",
 * section 2 and Table 1) */
typedef enum {
  MXATTN_RULE_OCP = 0, /* e = floor(log2 M) - emax(elem); emax = 2 (E2M1), 8 (E4M3) */
  MXATTN_RULE_CEIL = 1 /* e = smallest integer with M <= qmax * 2^e
                          (qmax 7.25: UOS; 6: truncation-free; 448: FP8 V)        */
} mxattn_e8m0_rule;

/* which axis the blocks run along */
typedef enum {
  MXATTN_ROLE_QK = 0, /* blocks along the head dimension d, one row per token     */
  MXATTN_ROLE_V = 1,  /* blocks along the tokens (the PV contraction axis), stored
                         transposed: one row per channel                           */
  MXATTN_ROLE_VKEY = 2, /* the per-key form of a 4-bit V for causally safe diagonal
                          tiles ("FLAMIA" section 3.2): one E8M0 scale per key over
                          its d channels (fmt's rule), E2M1 codes stored transposed
                          in role V's slot layout (fmt->block fixes that layout);
                          scales are [B][H][n_padded], one byte per key slot      */
  MXATTN_ROLE_VT = 3   /* role V's blocks and codes stored tile-major for the split-
                          key decode (mxattn_decode): each 128-key tile of V^T is
                          one contiguous run, so the decode reads the history tile
                          by tile instead of 128 pieces one channel row apart.  No
                          documents; E2M1 or E4M3 with E8M0 scales per 32 keys     */
} mxattn_role;

/* how the softmax operand P is quantized inside the attention loop */
typedef enum {
  MXATTN_P_NONE = 0,      /* unquantized route (Q, K, V in bf16): l = sum P~ in FP32;
                             O += P V with P~ rounded to bf16 (nearest even) as the
                             bf16 matrix-core operand                               */
  MXATTN_P_DIRECT = 1,    /* P^ = phi(P~); row sum l from the unquantized P~         */
  MXATTN_P_TWO_LEVEL = 2, /* s1 = rowmax_tile(P~)/(448*6) in FP32, P^ = phi(P~/s1),
                             O += s1 * P^ V; l from P~                              */
  MXATTN_P_PNQ = 3,       /* P^ = phi(P~) feeds both l and O                         */
  MXATTN_P_FP8_FIXED = 4  /* c = E4M3(448 P~), O += c V / 448; l from P~             */
} mxattn_pmode;

/* the exponential that turns scores into P~ ("FLAMIA" section 3.7 and appendix C).
 * The bit-level modes write t = sm_scale (s - m) / ln 2 - delta in fixed point into
 * the exponent and mantissa fields of a float, which is Mitchell's piecewise-linear
 * 2^floor(t) (1 + frac t); below t = -127 the result is 0.  The rescale of the
 * running sums when the row maximum moves stays exact.  They serve inference: the
 * result is an approximation of softmax by a few per cent per weight. */
typedef enum {
  MXATTN_EXP_EXACT = 0,      /* hardware exponential (v_exp_f32)                       */
  MXATTN_EXP_MITCHELL = 1,   /* Mitchell-P: delta = E/2 centres log2 of the line's ratio
                                to 2^t, E = log2(1/ln 2) - 1/ln 2 + 1 (ratio within
                                about +-3 %); meant for 4-bit P                          */
  MXATTN_EXP_SCHRAUDOLPH = 2 /* Schraudolph's form: delta = log2(1 / (2 ln^2 2)) makes the
                                ratio average one over an octave (no mean bias in the
                                row sum); meant for FP8 P                                */
} mxattn_exp_mode;

/* a block format */
typedef struct {
  int32_t elem;  /* mxattn_elem                                   */
  int32_t scale; /* mxattn_scale                                  */
  int32_t block; /* elements per scale: 16 or 32                  */
  int32_t rule;  /* mxattn_e8m0_rule (E8M0 scales only)           */
  float qmax;    /* boundary of the CEIL rule (ignored for OCP)   */
} mxattn_qfmt;

/*
 * A quantized tensor.  The library fills it in mxattn_quantize(); the caller
 * provides `codes` and `scales` (sized by mxattn_qtensor_bytes()).  Layouts are
 * dense and row-major:
 *   role QK: codes  [B][H][N][d * bits / 8]        scales [B][H][N][d / block]
 *   role V : codes  [B][H][d][n_padded * bits / 8] scales [B][H][d][n_padded / block]
 *   BF16 (either role): codes [B][H][N][d] bf16, no scales, n_padded = N
 *   role VT: codes  [B][H][n_padded / 128][d][128 * bits / 8]  scales [B][H][n_padded / 128][d][4]
 *            (role V's bytes of key tile t and channel c moved to [t][c])
 * bits = 4 (E2M1) or 8 (E4M3).  For role V the key axis is padded: each document
 * (the whole sequence when there are no documents) occupies ceil(L / block) whole
 * blocks starting at a block boundary, in document order; n_padded is
 * N + ndocs * (block - 1) for more than one document, else N, rounded up to a multiple
 * of 128, as mxattn_qtensor_bytes() reports it.  Slots after the last document
 * and inside a document's last block hold code 0; blocks made only of padding
 * hold the scale of an all-zero block (E8M0 byte 127, E4M3 byte 0).
 */
typedef struct {
  void* codes;
  void* scales;
  mxattn_qfmt fmt;
  int32_t role;
  int32_t ndocs;    /* documents the V key axis was laid out for (1 = none) */
  int64_t B, H, N, d;
  int64_t n_padded; /* role V: padded key count; role QK: N                  */
} mxattn_qtensor;

/* forward parameters */
typedef struct {
  int32_t pmode;    /* mxattn_pmode                                                  */
  mxattn_qfmt pfmt; /* block format of P (DIRECT, TWO_LEVEL, PNQ; ignored for FP8)    */
  int32_t causal;   /* 1: key j is visible to query i iff j <= i (within a document)  */
  float sm_scale;   /* softmax scale applied to the scores, normally 1/sqrt(d)        */
  int32_t kv_tile;  /* keys per online-softmax step; must be 128                      */
  int32_t out_fp32; /* 1: O is float32, 0: O is bfloat16 (round to nearest even)      */
  const float* score_bias; /* DEVICE [B][Hq][N] float32 added to the scores of each key
                              before the mask and the running maximum (the centering
                              compensation of mxattn_center_comp()), or NULL; 16-byte
                              aligned                                                  */
  const mxattn_qtensor* vkey; /* causally safe V scales ("FLAMIA" section 3.2), or NULL: a
                        mxattn_qtensor of role VKEY quantized from the same V with the
                        same documents.  Queries go in tiles of 256 rows from the start
                        of their sequence or document; on the key tiles that start
                        inside a row's query tile (the 256 keys from 256 floor(i / 256),
                        the tiles its causal boundary runs through) the row uses this
                        per-key form and multiplies P~_j by the key's scale 2^e_j before
                        quantizing P; every other tile uses v.  Needs a causal mask and
                        a V in E2M1 with E8M0 scales per 32 keys (an FP8 V with round-up
                        exponents needs no per-key form).                              */
  int32_t exp_mode; /* mxattn_exp_mode.  The bit-level modes need a V with E8M0 scales
                       per 32 keys (E2M1 or E4M3) and are refused by mxattn_decode() */
} mxattn_fwd_params;

/* ABI version (MXATTN_ABI_VERSION of the built library). */
int mxattn_abi_version(void);

/* Static text of a status code. */
const char* mxattn_status_str(int status);

/* Text of the last MXATTN_E_HIP failure on the calling thread, or of the last
 * MXATTN_E_WORKSPACE of mxattn_decode_noalloc() ("" if none).  Thread-local; the
 * pointer stays valid until the thread's next failing call.  mxattn_last_hip_error()
 * is the same function under the name of the HIP failure it reports. */
const char* mxattn_last_error(void);
const char* mxattn_last_hip_error(void);

/*
 * Test hook of the error path: the next `count` device submissions made by library
 * calls on the calling thread are not made; each such call returns MXATTN_E_HIP with
 * hipErrorLaunchFailure in mxattn_last_error(), after its host checks passed.
 * count <= 0 turns the hook off.  Returns the count that was pending.
 */
int mxattn_debug_fail_launches(int count);

/*
 * Bytes of the codes and scales buffers of a quantized tensor.
 *   fmt, role  : format and role as passed to mxattn_quantize()
 *   B, H, N, d : shape of the bf16 tensor ([B][H][N][d])
 *   ndocs      : number of packed documents (0 or 1: one sequence)
 * Writes *code_bytes, *scale_bytes and, if not NULL, *n_padded: role V pads the
 * key axis to n_padded = round_up(N + ndocs * (block - 1), 128) slots (with
 * ndocs <= 1: round_up(N, 128)), role VT to round_up(N, 128) (it takes no
 * documents: ndocs > 1 is MXATTN_E_INVALID), role QK has n_padded = N.
 * Errors: MXATTN_E_INVALID, MXATTN_E_UNSUPPORTED.
 */
int mxattn_qtensor_bytes(const mxattn_qfmt* fmt, int role, int64_t B, int64_t H, int64_t N, int64_t d,
                         int ndocs, size_t* code_bytes, size_t* scale_bytes, int64_t* n_padded);

/*
 * Quantize one bf16 tensor x [B][H][N][d] (element strides x_strides[0..3],
 * x_strides[3] must be 1; the base and every row must be 16-byte aligned).
 *   role QK: per token, blocks of fmt->block consecutive channels.
 *   role V : per channel, blocks of fmt->block consecutive tokens inside one
 *            document, written transposed (see mxattn_qtensor).
 *   role VT: as role V without documents, written tile-major (see mxattn_qtensor);
 *            E2M1 or E4M3 elements with E8M0 scales per 32 keys only.
 * Per block with maximum magnitude M ("MXAttention" section 2; blog "NVFP4, not
 * MXFP4"):
 *   E8M0 scale: exponent by fmt->rule, clamped to [-127, 127]; M = 0 gives 2^0.
 *   E4M3 scale: s = E4M3_rne_sat(fp32(M / 6)).
 *   element   : code = RNE_sat(fp32(x / scale)) in the element format, sign kept
 *               (a negative value that rounds to zero encodes as -0); a zero scale
 *               gives zero magnitudes.
 * cu_seqlens: DEVICE array of ndocs+1 document offsets (role V with documents;
 *   requires B == 1), or NULL.  Offsets must start at 0, end at N and never
 *   decrease; the kernel reads them, the host does not check them.
 * out: caller-owned descriptor whose codes/scales point to buffers of at least
 *   the sizes from mxattn_qtensor_bytes(); the library fills the other fields.
 * Errors: MXATTN_E_INVALID (also role VT with documents), MXATTN_E_UNSUPPORTED
 *   (d != 128, block not 16/32, E4M3 elements with an E4M3 scale, role VT in any
 *   format but E2M1 or E4M3 with E8M0 per 32, role QK with B*H*N >= 2^30), MXATTN_E_ALIGN,
 *   MXATTN_E_HIP.
 */
int mxattn_quantize(const void* x_bf16, const int64_t x_strides[4], int64_t B, int64_t H, int64_t N,
                    int64_t d, int role, const mxattn_qfmt* fmt, const int32_t* cu_seqlens, int ndocs,
                    mxattn_qtensor* out, void* stream);

/*
 * Outlier pre-processing of Q and K ("MpFA" section 4.2, Eq. 7: sequence
 * centering; blog "Microscaling FP4 Attention ...", "Smooth-K is the smaller
 * lever": subtract K's per-channel mean; "FLAMIA" section 3.4 and appendix A.2:
 * a normalized Hadamard rotation of the head channels before quantization).
 *
 * mxattn_channel_mean: per-channel means of a bf16 tensor x [B][H][N][d] (strides
 *   as for mxattn_quantize) over the tokens of each document:
 *   mean[b][h][k][c] = fl32(sum / L_k), the sum over document k's tokens taken in
 *   double (exact for realistic bf16 spans, so the result does not depend on the
 *   summation order) and divided in double; an empty document gives 0.
 *   mean: DEVICE float32 [B][H][max(ndocs,1)][d], 16-byte aligned.
 *   cu_seqlens/ndocs: DEVICE document offsets as for mxattn_quantize (ndocs <= 1
 *   or cu_seqlens NULL: one document [0, N)).
 *   Errors: MXATTN_E_INVALID, MXATTN_E_UNSUPPORTED (d != 128), MXATTN_E_ALIGN,
 *   MXATTN_E_HIP.
 */
int mxattn_channel_mean(const void* x_bf16, const int64_t x_strides[4], int64_t B, int64_t H, int64_t N,
                        int64_t d, const int32_t* cu_seqlens, int ndocs, float* mean, void* stream);

/* Pre-processing applied by mxattn_quantize_pre() before the block quantization. */
typedef struct {
  const float* mean; /* DEVICE [B][H][max(ndocs,1)][d] channel means to subtract (from
                        mxattn_channel_mean), or NULL                                  */
  int32_t hadamard;  /* 1: rotate each token by H / sqrt(d), H the Sylvester Hadamard
                        matrix H[i][j] = (-1)^popcount(i & j); 0: no rotation          */
} mxattn_preproc;

/*
 * Quantize Q or K (role QK only) after pre-processing: each token becomes
 * y = fl32(((x - mean[doc]) H) c), c = fl64(1 / fl64(sqrt(128))) with the rotation
 * and 1 without it, the difference and the +-1 sums exact in double, then y is
 * quantized exactly as mxattn_quantize() quantizes x.  Rotating Q and K alike
 * keeps Q.K; subtracting K's mean alone changes each softmax row by a constant
 * (smooth-K); subtracting both means needs the compensation of
 * mxattn_center_comp() as the forward's score_bias.
 *   pre: NULL (plain quantization) or the pre-processing to apply.
 *   cu_seqlens/ndocs: DEVICE document offsets selecting each token's mean row
 *   (the qtensor is laid out as without documents: role QK has no padding).
 * Errors: as mxattn_quantize(), plus MXATTN_E_INVALID for role V and
 *   MXATTN_E_UNSUPPORTED for B*H*N >= 2^28.
 */
int mxattn_quantize_pre(const void* x_bf16, const int64_t x_strides[4], int64_t B, int64_t H, int64_t N,
                        int64_t d, int role, const mxattn_qfmt* fmt, const mxattn_preproc* pre,
                        const int32_t* cu_seqlens, int ndocs, mxattn_qtensor* out, void* stream);

/*
 * Centering compensation ("MpFA" section 4.3, Eqs. 8-9): with Q and K both
 * centered, S = Q_c K_c^T + 1 (qmean K_c^T) + (Q kmean^T) 1^T; the last term is
 * constant along each softmax row and cancels, the middle one is restored as
 *   delta[b][hq][j] = fl32(sum_c qmean[b][hq][doc(j)][c] * (k[b][hk][j][c] - kmean[b][hk][doc(j)][c]))
 * with hk = hq * Hkv / Hq, products and sums in double (within one float ulp of
 * the exactly rounded value).  Pass delta as mxattn_fwd_params.score_bias.
 *   qmean: DEVICE [B][Hq][max(ndocs,1)][d]; kmean: DEVICE [B][Hkv][max(ndocs,1)][d]
 *   k: bf16 [B][Hkv][N][d] with element strides k_strides (the unquantized K);
 *   delta: DEVICE float32 [B][Hq][N].
 * Errors: MXATTN_E_INVALID, MXATTN_E_UNSUPPORTED (d != 128, B*Hkv*N >= 2^28),
 *   MXATTN_E_ALIGN, MXATTN_E_HIP.
 */
int mxattn_center_comp(const float* qmean, const void* k_bf16, const int64_t k_strides[4], const float* kmean,
                       int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, const int32_t* cu_seqlens,
                       int ndocs, float* delta, void* stream);

/*
 * Bytes of workspace a forward over packed documents needs (a document table
 * and a work list of query tiles): N = total tokens, ndocs = documents.
 * Returns 0 when ndocs <= 0 (no documents: no workspace is used).
 */
size_t mxattn_fwd_workspace_bytes(int64_t N, int ndocs);

/*
 * Plan a forward over packed documents ("FLAMIA", section 3.6: documents are
 * packed without padding, attention stays inside each document, and work is
 * ordered longest first).  From HOST offsets cu_seqlens_host[0..ndocs]
 * (0 = first, N = last, non-decreasing) it builds, on the host, the document
 * table and the list of (document, query tile) items in decreasing order of
 * cost (key tiles visited; ties keep document order), and copies them into
 * `workspace` on `stream`.  The copy is from pageable host memory, so the call
 * may block until it is staged; the host array may be reused on return.  A plan
 * stays valid for every mxattn_fwd() with the same offsets and causal flag.
 * Errors: MXATTN_E_INVALID, MXATTN_E_WORKSPACE, MXATTN_E_HIP.
 */
int mxattn_fwd_plan(const int32_t* cu_seqlens_host, int ndocs, int64_t N, int causal, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * Attention forward on quantized operands.
 *   q: role QK, [B][Hq][N][d];  k: role QK, [B][Hkv][N][d];  v: role V, [B][Hkv][d][.]
 *   Hq must be a multiple of Hkv; query head h reads key/value head h*Hkv/Hq.
 *   params: P mode and format, causal flag, sm_scale, kv_tile (128), output type.
 *   ndocs: 0 for one sequence per batch entry; otherwise the number of packed
 *     documents (B == 1), `v` must have been quantized with the same documents
 *     and `workspace` must hold a plan from mxattn_fwd_plan().  Attention never
 *     crosses a document, and key tiles start at each document's first token.
 *     The kernels check the plan's header against the call (document count, N,
 *     causal flag, list sizes): a workspace that holds no plan, or one built
 *     for other arguments, makes every row of `out` and `lse` NaN; the entries
 *     of a plan are bounds-checked, so none is read past N.  A plan for other
 *     offsets with the same counts cannot be told apart.
 *   out: [B][Hq][N][d] with element strides out_strides (out_strides[3] == 1,
 *     16-byte aligned rows), float32 or bfloat16 per params->out_fp32.
 *   lse: optional float32 [B][Hq][N] log-sum-exp (natural log) of each row, or
 *     NULL.  Rows that see no key get O = 0 and lse = -inf.
 * The online softmax walks key tiles of 128 in ascending order; P blocks are
 * consecutive keys aligned to the tile start.  Quantized-P results depend on
 * this order, which is part of the contract.
 * Supported operand routes (others return MXATTN_E_UNSUPPORTED):
 *   Q/K: MXFP4 (E2M1, E8M0/32) or NVFP4 (E2M1, E4M3/16), the same for both.
 *   P/V: DIRECT, PNQ or TWO_LEVEL with P in E2M1 (E8M0/32 or E4M3/16) and V in
 *        E2M1 (E8M0/32 or E4M3/16); FP8_FIXED with V in E4M3 with E8M0/32.
 *   Unquantized: Q, K and V all BF16 with pmode NONE (softmax(Q K^T sm_scale) V:
 *        scores from exact products summed in FP32, P~ in FP32, P rounded to bf16
 *        for the PV product); score_bias allowed, no per-key V form, exact
 *        exponential only.
 * Sizes: N and the padded key count of `v` at most 2^24 (MXATTN_E_UNSUPPORTED
 *   beyond).
 * Errors: MXATTN_E_INVALID, MXATTN_E_UNSUPPORTED, MXATTN_E_ALIGN,
 *   MXATTN_E_WORKSPACE, MXATTN_E_HIP.
 */
int mxattn_fwd(const mxattn_qtensor* q, const mxattn_qtensor* k, const mxattn_qtensor* v,
               const mxattn_fwd_params* params, int ndocs, void* out, const int64_t out_strides[4],
               float* lse, const void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode ("MpFA" section 5.3): the R newest tokens of each request attend to its
 * key/value history.  The history of each (request, KV head) is cut into splits of
 * 256 keys from key 0; each split runs the online softmax on its own (tiles of 128
 * from the split start, P quantized per tile against the split's running maximum)
 * and the splits of each query row are merged by their log-sum-exp.  The query
 * heads of a KV head's group and the R rows share one matrix tile: (Hq/Hkv)*R <= 32.
 *   q: role QK [B][Hq][R][d]; row r sits at position kv_len[b] - R + r and sees
 *      keys 0..that position (params->causal must be 1).
 *   k: role QK [B][Hkv][N][d]; v: role V [B][Hkv][d][n_padded] without documents,
 *      or role VT (the same values tile-major: the faster layout for decode).
 *   Formats: MXFP4 Q/K/V (E2M1 with E8M0 per 32, any E8M0 rule) with P modes
 *   DIRECT, PNQ and TWO_LEVEL and P in E2M1 with E8M0 per 32; or the QK4PV8 route
 *   ("MpFA" sections 4.1 and 5.3): NVFP4 (or MXFP4) Q/K, V in E4M3 with E8M0 per 32
 *   keys (role V or VT), P mode FP8_FIXED (P = E4M3(448 P~), the row sum from P~).
 *   v->n_padded must be role V's padded length for N.  score_bias and vkey must be
 *   NULL.
 *   kv_len: DEVICE int32 [B] with R <= kv_len[b] <= N, or NULL (every history has N
 *   keys); the host does not read it.
 *   out: [B][Hq][R][d] with element strides out_strides (out_strides[3] == 1),
 *   float32 or bfloat16 per params->out_fp32; lse: optional float32 [B][Hq][R].
 *   workspace: DEVICE, at least mxattn_decode_workspace_bytes(B, Hq, R, N) bytes,
 *   16-byte aligned (split outputs and log-sum-exps; contents need no clearing).
 * Errors: MXATTN_E_INVALID, MXATTN_E_UNSUPPORTED, MXATTN_E_ALIGN,
 *   MXATTN_E_WORKSPACE, MXATTN_E_HIP.
 */
size_t mxattn_decode_workspace_bytes(int64_t B, int64_t Hq, int64_t R, int64_t N);
int mxattn_decode(const mxattn_qtensor* q, const mxattn_qtensor* k, const mxattn_qtensor* v,
                  const mxattn_fwd_params* params, const int32_t* kv_len, void* out,
                  const int64_t out_strides[4], float* lse, void* workspace, size_t workspace_bytes,
                  void* stream);

/*
 * mxattn_decode() without a workspace and without any allocation, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The split states live in a static device array
 * of the library, 32 MiB per GPU (MXATTN_DECODE_SCRATCH_BYTES), held from the first
 * call on a GPU until the process ends.  Arguments, layouts and results are those of
 * mxattn_decode(), bit for bit.
 *   Limit: mxattn_decode_workspace_bytes(B, Hq, R, N) must not exceed
 *   MXATTN_DECODE_SCRATCH_BYTES (B * Hq * R * ceil(N / 512) <= 65027 split rows, e.g. 4
 *   requests x 32 query heads x 1 row over 254K keys); larger calls return
 *   MXATTN_E_WORKSPACE with the sizes in mxattn_last_error().
 *   Every call on one GPU uses the same array: calls that overlap on one GPU (other
 *   streams or threads) race, so serialize them.  Nothing needs clearing between calls.
 * Errors: as mxattn_decode().
 */
#define MXATTN_DECODE_SCRATCH_BYTES (32u << 20)
int mxattn_decode_noalloc(const mxattn_qtensor* q, const mxattn_qtensor* k, const mxattn_qtensor* v,
                          const mxattn_fwd_params* params, const int32_t* kv_len, void* out,
                          const int64_t out_strides[4], float* lse, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MXATTN_H */
