/*
 * oracle.c -- plain, slow CPU reference for microscaling-FP4 attention forward.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg; never by the GPU library.  Source titles are
 * abbreviated as in oracle.h.  Build: gcc -O2 -ffp-contract=off -fno-fast-math.
 *
 * Parity status: every function below is pinned by tests/test_oracle_pins.py
 * (formats, scale rules, quantizers, two-level stretch, PNQ normalisation) and
 * tests/test_oracle_attention.py (online softmax against brute force, masks,
 * GQA, packed documents).  The flip budget is pinned by
 * tests/test_oracle_flip_budget.py on constructed rows whose fragile decisions
 * and their effect on O are known in closed form (an element on an E2M1
 * midpoint, a block maximum on an E8M0 boundary, a row with none), and its
 * two-level pre-scale by the per-tile invariance it implies.
 */
#include "oracle.h"

#include <limits.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* E2M1: magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}, sign bit 3 ([MXF4] "NVFP4,  */
/* not MXFP4"; [MXA] section 2, the E2M1 grid).                               */
/* ------------------------------------------------------------------------ */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_e2m1_value(int code) {
  double m = E2M1_MAG[code & 7];
  return (code & 8) ? -m : m;
}

/* Round to the nearest grid magnitude; on a tie take the even magnitude index
 * (IEEE round-half-even, the OCP MX convention); magnitudes beyond 6 take 6,
 * the nearest finite value ([MXA] section 3 describes conversion as nearest
 * rounding with saturation to the finite range).  The sign is kept, so a negative value
 * that rounds to zero gives 0x8.  NaN is outside the domain and maps to 0. */
int orc_e2m1_encode(float x) {
  int sign = signbit(x) ? 8 : 0;
  double a = fabs((double)x);
  int best = 0;
  if (isnan(x)) return 0;
  /* beyond the largest magnitude the nearest finite value is 6; testing it
   * first also keeps huge inputs, whose double distances all tie, exact */
  if (a >= 6.0) return sign | 7;
  double bd = a;
  for (int k = 1; k < 8; k++) {
    double dist = fabs(a - E2M1_MAG[k]);
    if (dist < bd || (dist == bd && (k % 2) == 0)) {
      best = k;
      bd = dist;
    }
  }
  return sign | best;
}

/* ------------------------------------------------------------------------ */
/* E4M3 (OCP FP8): bias 7, 3 mantissa bits, subnormals, no infinity,         */
/* S.1111.111 is NaN, largest finite 448 ([MXF4] "The probability squeeze").  */
/* ------------------------------------------------------------------------ */
double orc_e4m3_value(int b) {
  int e = (b >> 3) & 15, m = b & 7;
  double v;
  if ((b & 0x7f) == 0x7f) return NAN;
  v = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
  return (b & 0x80) ? -v : v;
}

/* Nearest of the 127 finite non-negative magnitudes (codes 0x00..0x7E, which
 * increase with the code), ties to the even code, beyond 448 -> 448. */
int orc_e4m3_encode(float x) {
  int sign = signbit(x) ? 0x80 : 0;
  double a = fabs((double)x);
  int lo, hi;
  if (isnan(x)) return 0x7f;
  if (a >= 448.0) return sign | 0x7e;
  /* largest code whose magnitude is <= a */
  lo = 0;
  hi = 0x7e;
  while (lo < hi) {
    int mid = (lo + hi + 1) / 2;
    if (orc_e4m3_value(mid) <= a) lo = mid; else hi = mid - 1;
  }
  {
    double below = orc_e4m3_value(lo), above = orc_e4m3_value(lo + 1);
    double db = a - below, da = above - a;
    int code = lo;
    if (da < db || (da == db && ((lo + 1) % 2) == 0)) code = lo + 1;
    return sign | code;
  }
}

/* ------------------------------------------------------------------------ */
/* E8M0 shared exponent ([MXA] section 2, section 4.1 and Table 1).           */
/*   OCP : e = floor(log2 amax) - emax_elem   (emax 2 for E2M1, 8 for E4M3)  */
/*   CEIL: e = ceil(log2(amax / qmax)), the smallest e with amax <= qmax 2^e  */
/* amax = 0 gives e = 0: an all-zero block uses sigma = 1 ([MXA] section 2).  */
/* e is clamped to [-127, 127]; the byte is e + 127 (0xFF, NaN, never used).  */
/* ------------------------------------------------------------------------ */
static int elem_emax(int elem) { return elem == ORC_ELEM_E2M1 ? 2 : 8; }
static double elem_max(int elem) { return elem == ORC_ELEM_E2M1 ? 6.0 : 448.0; }

int orc_e8m0_exponent(float amax, int rule, float qmax, int elem) {
  int e;
  if (amax == 0.0f) return 0;
  if (rule == ORC_RULE_OCP) {
    e = ilogb(amax) - elem_emax(elem);
  } else {
    /* qmax*2^e < amax holds at this start, so the search ends at the smallest e */
    e = ilogb(amax) - ilogb(qmax) - 1;
    while ((double)amax > ldexp((double)qmax, e)) e++;
  }
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return e;
}

double orc_scale_value(const orc_fmt* f, int sbyte) {
  if (f->scale == ORC_SCALE_E8M0) return ldexp(1.0, sbyte - 127);
  return orc_e4m3_value(sbyte);
}

static int encode_elem(int elem, float y) {
  return elem == ORC_ELEM_E2M1 ? orc_e2m1_encode(y) : orc_e4m3_encode(y);
}
static double elem_value(int elem, int code) {
  return elem == ORC_ELEM_E2M1 ? orc_e2m1_value(code) : orc_e4m3_value(code);
}

/* scale byte for a block maximum */
static int scale_byte_for(float amax, const orc_fmt* f) {
  if (f->scale == ORC_SCALE_E8M0)
    return orc_e8m0_exponent(amax, f->rule, f->qmax, f->elem) + 127;
  /* NVFP4-style: s = E4M3(amax / 6) with amax/6 a single float division
   * ([MXF4] "NVFP4, not MXFP4": s = max|X_block|/6; [MPFA] Eq. 1) */
  return orc_e4m3_encode(amax / (float)elem_max(f->elem));
}

/* One block: x_hat = round(x / s) with x/s a single float division; a zero
 * scale (E4M3 underflow) gives zero magnitudes with the sign kept. */
float orc_quant_block(const float* x, int n, const orc_fmt* f, uint8_t* codes, uint8_t* sbyte) {
  float amax = 0.0f, s;
  int sb, i;
  for (i = 0; i < n; i++) {
    float a = fabsf(x[i]);
    if (a > amax) amax = a;
  }
  sb = scale_byte_for(amax, f);
  s = (float)orc_scale_value(f, sb);
  for (i = 0; i < n; i++) {
    if (s == 0.0f)
      codes[i] = (uint8_t)(signbit(x[i]) ? (f->elem == ORC_ELEM_E2M1 ? 0x8 : 0x80) : 0);
    else
      codes[i] = (uint8_t)encode_elem(f->elem, x[i] / s);
  }
  *sbyte = (uint8_t)sb;
  return s;
}

void orc_quantize_rows(const float* x, int64_t rows, int d, const orc_fmt* f, uint8_t* codes,
                       uint8_t* scales) {
  int nb = d / f->block;
  for (int64_t r = 0; r < rows; r++)
    for (int b = 0; b < nb; b++)
      orc_quant_block(x + r * d + (int64_t)b * f->block, f->block, f,
                      codes + r * d + (int64_t)b * f->block, scales + r * nb + b);
}

void orc_dequant_rows(const uint8_t* codes, const uint8_t* scales, int64_t rows, int d,
                      const orc_fmt* f, float* out) {
  int nb = d / f->block;
  for (int64_t r = 0; r < rows; r++)
    for (int c = 0; c < d; c++) {
      double s = orc_scale_value(f, scales[r * nb + c / f->block]);
      out[r * d + c] = (float)(elem_value(f->elem, codes[r * d + c]) * s);
    }
}

/* V role ([SA3] and [MXF4]: V is blocked along the PV contraction axis, the
 * keys; [FLAMIA] 3.6.1: token blocks stay inside document boundaries). */
int64_t orc_v_nblocks(int N, const int* doc_off, int ndocs, int block) {
  int64_t nblk = 0;
  if (!doc_off || ndocs <= 0) return (N + block - 1) / block;
  for (int k = 0; k < ndocs; k++) nblk += (doc_off[k + 1] - doc_off[k] + block - 1) / block;
  return nblk;
}

void orc_quantize_cols(const float* x, int N, int d, const int* doc_off, int ndocs,
                       const orc_fmt* f, uint8_t* codes, uint8_t* scales) {
  int one[2] = {0, N};
  int64_t nblk = orc_v_nblocks(N, doc_off, ndocs, f->block);
  float* col = (float*)malloc(sizeof(float) * (size_t)f->block);
  uint8_t* cc = (uint8_t*)malloc((size_t)f->block);
  if (!doc_off || ndocs <= 0) {
    doc_off = one;
    ndocs = 1;
  }
  for (int c = 0; c < d; c++) {
    int64_t bi = 0;
    for (int k = 0; k < ndocs; k++) {
      for (int t0 = doc_off[k]; t0 < doc_off[k + 1]; t0 += f->block) {
        int n = doc_off[k + 1] - t0 < f->block ? doc_off[k + 1] - t0 : f->block;
        for (int j = 0; j < n; j++) col[j] = x[(int64_t)(t0 + j) * d + c];
        orc_quant_block(col, n, f, cc, scales + (int64_t)c * nblk + bi);
        for (int j = 0; j < n; j++) codes[(int64_t)c * N + t0 + j] = cc[j];
        bi++;
      }
    }
  }
  free(col);
  free(cc);
}

void orc_dequant_cols(const uint8_t* codes, const uint8_t* scales, int N, int d,
                      const int* doc_off, int ndocs, const orc_fmt* f, float* out) {
  int one[2] = {0, N};
  int64_t nblk = orc_v_nblocks(N, doc_off, ndocs, f->block);
  if (!doc_off || ndocs <= 0) {
    doc_off = one;
    ndocs = 1;
  }
  for (int c = 0; c < d; c++) {
    int64_t bi = 0;
    for (int k = 0; k < ndocs; k++)
      for (int t0 = doc_off[k]; t0 < doc_off[k + 1]; t0 += f->block, bi++) {
        double s = orc_scale_value(f, scales[(int64_t)c * nblk + bi]);
        int n = doc_off[k + 1] - t0 < f->block ? doc_off[k + 1] - t0 : f->block;
        for (int j = 0; j < n; j++)
          out[(int64_t)(t0 + j) * d + c] = (float)(elem_value(f->elem, codes[(int64_t)c * N + t0 + j]) * s);
      }
  }
}

/* ------------------------------------------------------------------------ */
/* Flip budget.  An implementation under test computes every value that     */
/* feeds a rounding decision (an element code, a block scale) with its own  */
/* FP32 arithmetic, so its value differs from this one by a bounded         */
/* relative amount w (the decision's window, see decision_window below).  A  */
/* decision whose value lies within w of a threshold may be taken the other  */
/* way; for each such decision the budget adds the largest change of the    */
/* dequantized values it can make.                                          */
/* ------------------------------------------------------------------------ */

/* alternative code of an element decision whose value y carries a relative
 * window w, or -1 */
static int elem_alt(int elem, float y, int code, double w) {
  double a = fabs((double)y);
  int mag = elem == ORC_ELEM_E2M1 ? (code & 7) : (code & 0x7f);
  int top = elem == ORC_ELEM_E2M1 ? 7 : 0x7e;
  int sign = elem == ORC_ELEM_E2M1 ? (code & 8) : (code & 0x80);
  for (int nb = -1; nb <= 1; nb += 2) {
    int other = mag + nb;
    double mid;
    if (other < 0 || other > top) continue;
    mid = 0.5 * (fabs(elem_value(elem, mag)) + fabs(elem_value(elem, other)));
    if (fabs(a - mid) <= w * a) return sign | other;
  }
  return -1;
}

/* alternative scale byte of a block decision whose maximum lies in [lo, hi]
 * on the implementation under test, or -1 */
static int scale_alt(double lo, double hi, const orc_fmt* f, int sb) {
  int a, b;
  if (hi <= 0.0) return -1;
  a = scale_byte_for((float)lo, f);
  b = scale_byte_for((float)hi, f);
  if (a != sb) return a;
  if (b != sb) return b;
  return -1;
}

/* Quantize-dequantize one P block of n values (n <= 64) and report, per
 * element, the largest change of its dequantized value that a fragile
 * decision could make (delta[]).  w[j]: relative window of x[j] for its
 * element decision; ws[j]: relative window of x[j] as an input of the
 * block's scale decision (0 where the implementation reproduces x[j]
 * exactly).  deq[] receives code*scale. */
static void p_block(const float* x, const double* w, const double* ws, int n, const orc_fmt* f,
                    double* deq, double* delta) {
  uint8_t codes[64], sb;
  float s = orc_quant_block(x, n, f, codes, &sb);
  int alt_sb;
  double lo = 0.0, hi = 0.0;
  for (int j = 0; j < n; j++) {
    int alt;
    deq[j] = elem_value(f->elem, codes[j]) * (double)s;
    delta[j] = 0.0;
    if (s != 0.0f) {
      alt = elem_alt(f->elem, x[j] / s, codes[j], w[j]);
      if (alt >= 0) delta[j] = fabs(elem_value(f->elem, alt) - elem_value(f->elem, codes[j])) * (double)s;
    }
    {
      double a = fabs((double)x[j]);
      if (a * (1.0 - ws[j]) > lo) lo = a * (1.0 - ws[j]);
      if (a * (1.0 + ws[j]) > hi) hi = a * (1.0 + ws[j]);
    }
  }
  alt_sb = scale_alt(lo, hi, f, sb);
  if (alt_sb >= 0) {
    float s2 = (float)orc_scale_value(f, alt_sb);
    for (int j = 0; j < n; j++) {
      double v2 = 0.0;
      if (s2 != 0.0f) v2 = elem_value(f->elem, encode_elem(f->elem, x[j] / s2)) * (double)s2;
      if (fabs(v2 - deq[j]) > delta[j]) delta[j] = fabs(v2 - deq[j]);
    }
  }
}

/* log2 of the largest power of two that divides a nonzero float (its last set
 * bit): the grain of the value; a product of two floats has the sum of their
 * grains as its grain */
static int grain_exp(float v) {
  uint32_t b;
  int e;
  memcpy(&b, &v, 4);
  e = (int)((b >> 23) & 0xFF);
  b &= 0x7FFFFFu;
  if (e == 0) return -149 + __builtin_ctz(b); /* subnormal (v != 0) */
  return e - 150 + __builtin_ctz(b | 0x800000u);
}

/* Relative window of an exponential P~_j = 2^(a_j), a_j = lambda (s_j - m) with
 * lambda = sm_scale / ln 2, as an implementation in FP32 computes it.  The bound,
 * term by term (u = 2^-24, the unit roundoff of FP32):
 *   - scores: the implementation sums the exact products of the dequantized
 *     operands in FP32 with score_rounds roundings, each of relative size u of a
 *     partial sum no larger than A = sum_c |q_c k_c| (+ |bias|), so
 *     |S - s| <= es = score_rounds u A (es = 0 when every partial sum is exact:
 *     A below 2^24 times the smallest power of two dividing all the terms), and
 *     the running maximum moves by at most es as well: the argument moves by at
 *     most 2 lambda es;
 *   - lambda rounded to FP32: u |a_j|;
 *   - the row offset fl(lambda m): u lambda |m|;
 *   - the rounding of the argument itself: u |a_j|;
 *   - the exponential: 1 ulp of its result on the implementation, 0.5 ulp here
 *     (3 u), plus the products of the P quantization (a reciprocal 1/s, its
 *     product with the two-level pre-scale and the element's product with it,
 *     against this oracle's single division: 4 u): 2^-20 covers both.
 *   - fold: with the exact exponential an implementation may apply the multiplier
 *     of the P quantization (the two-level 1/s1, an E4M3 block scale's 1/s, FP8's
 *     448) as an offset of the argument instead of a product: P~/s1 =
 *     2^(lambda (s - t) + L) with t the tile's largest score and L = log2(448 * 6),
 *     1/s as -log2 s, and 448 P~ = 2^(lambda (s - m) + log2 448).
 *     Its offsets are rounded to FP32 once or twice more and log2 s comes from a
 *     hardware logarithm within 2^-20 for every E4M3 value (measured); attn_row_bias
 *     passes these terms, an absolute change of the argument, as fold.
 * A change d of the argument changes 2^a by a factor 2^d, |2^d - 1| <= ln2 |d|
 * (1 + ln2 |d|).  The bit-level modes add 2^-15 (the line keeps 16 fraction bits
 * of its argument in an FP32 FMA). */
static double p_window(const orc_attn_params* p, double lam, double es, double a, double m,
                       double fold) {
  const double u = 0x1p-24;
  double darg = 2.0 * lam * es + 2.0 * u * fabs(a) + u * lam * fabs(m) + fold;
  const double ln2 = 0.69314718055994530942;
  double w = ln2 * darg * (1.0 + ln2 * darg) + 0x1p-20;
  if (p->exp_mode != ORC_EXP_EXACT) w += 0x1p-15;
  return w;
}

/* ------------------------------------------------------------------------ */
/* Bit-level exponentials ([FLAMIA] section 3.7 and appendix C, after       */
/* Mitchell 1962 and Schraudolph 1999).  A positive float read as an        */
/* integer is 2^23 (e + 127) + mantissa, so the integer 2^23 (t + 127)      */
/* puts floor(t) in the exponent field and the fraction of t in the         */
/* mantissa: the float it spells is 2^floor(t) (1 + frac t).  With the      */
/* exponent field at zero (t < -126) the same bits spell the subnormal      */
/* (t + 127) 2^-126; a negative pattern is clamped to +0.                   */
/* ------------------------------------------------------------------------ */
double orc_exp2_bits(double t) {
  double n;
  if (!(t >= -127.0)) return 0.0; /* the clamp; NaN and -inf too */
  if (t < -126.0) return ldexp(t + 127.0, -126);
  n = floor(t);
  return ldexp(1.0 + (t - n), (int)n);
}

/* Over one octave the line's ratio to 2^t is r(f) = (1 + f) 2^-f, f = frac t.
 * log2 r(f) = log2(1 + f) - f is 0 at both ends and largest at f = 1/ln2 - 1,
 * where it is E = log2(1/ln2) - 1/ln2 + 1 (about 0.0861).
 *   Mitchell-P: the offset centres the error, delta = E/2, so log2 of the ratio
 *   lies in [-E/2, E/2].
 *   Schraudolph: the offset makes the ratio average one over f in [0, 1); the
 *   integral of (1 + f) 2^-f over [0, 1] is 1/(2 ln^2 2), so delta = log2 of it. */
double orc_exp_offset(int exp_mode) {
  const double ln2 = log(2.0);
  if (exp_mode == ORC_EXP_MITCHELL) return 0.5 * (log2(1.0 / ln2) - 1.0 / ln2 + 1.0);
  if (exp_mode == ORC_EXP_SCHRAUDOLPH) return log2(1.0 / (2.0 * ln2 * ln2));
  return 0.0;
}

/* P~ of a score at x = sm_scale (s - m) nats below the running maximum */
static float p_exp(const orc_attn_params* p, double x) {
  if (p->exp_mode == ORC_EXP_EXACT) return (float)exp(x);
  return (float)orc_exp2_bits(x / log(2.0) - orc_exp_offset(p->exp_mode));
}

/* ------------------------------------------------------------------------ */
/* Attention for one query row: FlashAttention-2 form of the online softmax */
/* ([MXA] section 2 and Algorithm 1; [MPFA] Eqs. 3-6), with the P          */
/* quantization of the chosen mode applied to each tile's unnormalised     */
/* exponentials:                                                            */
/*   DIRECT    P^ = phi(P~), l from P~             ([MXA] 5.2, OCP baseline)*/
/*   TWO_LEVEL s1 = rowmax(P~)/(448*6) in FP32, P^ = phi(P~/s1), O += s1 P^V */
/*             ([MXF4] "Two-level scaling"; [SA3] Eq. 5); l from P~        */
/*   PNQ       P^ = phi(P~) feeds both l and O     ([MXA] 4.2, Algorithm 1) */
/*   FP8_FIXED c = cast_e4m3(448 P~), O += (c V)/448, l from P~ ([MPFA] 4.1)*/
/* Tiles of kv_tile keys are aligned to key 0 of the range and walked in   */
/* ascending order; P blocks are consecutive keys aligned to the tile.     */
/* ------------------------------------------------------------------------ */
static int attn_row_bias(const float* q, const float* K, const float* V, const float* sbias,
                         const float* Vk, const int* ek, int diag_lo, int nk, int vis, int d,
                         const orc_attn_params* p, float* o, float* lse, double* fb);

int orc_attn_row(const float* q, const float* K, const float* V, int nk, int vis, int d,
                 const orc_attn_params* p, float* o, float* lse, double* fb) {
  return attn_row_bias(q, K, V, NULL, NULL, NULL, -1, nk, vis, d, p, o, lse, fb);
}

/* sbias: NULL, or the score bias of keys 0..nk-1 of this range ([MPFA] Eq. 10: added
 * to the exact dot product before the mask and the running maximum).
 * Vk, ek, diag_lo: causally safe V scales ([FLAMIA] section 3.2): on the tiles that
 * start at keys diag_lo .. diag_lo + q_tile - 1 (the row's diagonal tiles) the row
 * uses the per-key form of V -- E2M1 values Vk[j][c] with unit scale and a
 * power-of-two scale 2^ek[j] per key -- and folds that scale into P,
 * P'_j = P~_j * 2^ek[j] (exact float ldexp), which is then quantized as P normally
 * is; O takes P^' Vk, and the PNQ row sum takes deq(P^'_j) 2^-ek[j].
 * Vk == NULL: no tile uses the per-key form. */
static int attn_row_bias(const float* q, const float* K, const float* V, const float* sbias,
                         const float* Vk, const int* ek, int diag_lo, int nk, int vis, int d,
                         const orc_attn_params* p, float* o, float* lse, double* fb) {
  int T = p->kv_tile;
  const int QT = p->q_tile > 0 ? p->q_tile : T;
  float m = -INFINITY, l = 0.0f;
  float* acc = (float*)calloc((size_t)d, sizeof(float));
  float* s = (float*)malloc(sizeof(float) * (size_t)T);
  float* pt = (float*)malloc(sizeof(float) * (size_t)T);
  float* x2 = (float*)malloc(sizeof(float) * (size_t)T);
  double* ph = (double*)malloc(sizeof(double) * (size_t)T);
  double* dl = (double*)malloc(sizeof(double) * (size_t)T);
  double* col = (double*)malloc(sizeof(double) * (size_t)d);
  double* we = (double*)malloc(sizeof(double) * (size_t)T); /* element windows   */
  double* ws = (double*)malloc(sizeof(double) * (size_t)T); /* scale-input windows */
  double fb1 = 0.0, fb2 = 0.0; /* flip budget: O part, l part (PNQ) */
  /* flip-budget bookkeeping: the largest error bound of a visible score so far,
   * and the two largest visible scores (is the running maximum unique?) */
  const double lam = (double)p->sm_scale / 0.69314718055994530942;
  const int rounds = p->score_rounds > 0 ? p->score_rounds : 2;
  double es_max = 0.0, m1 = -INFINITY, m2 = -INFINITY;

  int* qg = (int*)malloc(sizeof(int) * (size_t)d); /* grains of the query's entries */
  for (int c = 0; c < d; c++) qg[c] = q[c] != 0.0f ? grain_exp(q[c]) : 0;
  if (vis > nk) vis = nk;
  for (int t0 = 0; t0 < vis; t0 += T) {
    int tl = nk - t0 < T ? nk - t0 : T; /* keys in this tile */
    float mt = -INFINITY, mnew, alpha, mult = 1.0f;
    double wsum = 0.0, dsum1 = 0.0, dsum2 = 0.0;
    /* S = Q K^T: exact products of dequantized values summed in double */
    for (int j = 0; j < tl; j++) {
      if (t0 + j < vis) {
        double acc_d = 0.0, abs_d = 0.0;
        int gmin = INT_MAX;
        for (int c = 0; c < d; c++) {
          const float kv = K[(int64_t)(t0 + j) * d + c];
          double pr = (double)q[c] * (double)kv;
          acc_d += pr;
          abs_d += fabs(pr);
          if (pr != 0.0 && qg[c] + grain_exp(kv) < gmin) gmin = qg[c] + grain_exp(kv);
        }
        if (sbias) {
          acc_d += (double)sbias[t0 + j];
          abs_d += fabs((double)sbias[t0 + j]);
          if (sbias[t0 + j] != 0.0f && grain_exp(sbias[t0 + j]) < gmin) gmin = grain_exp(sbias[t0 + j]);
        }
        const double grain = gmin == INT_MAX ? INFINITY : ldexp(1.0, gmin);
        s[j] = (float)acc_d;
        /* every partial sum of these terms, in any order, is a multiple of the grain
         * no larger than abs_d: below 2^24 grains all of them are exact in FP32 and
         * the implementation's score equals this one; otherwise each of its
         * score_rounds roundings is at most 2^-24 abs_d */
        if (!(abs_d < 0x1p24 * grain) && rounds * 0x1p-24 * abs_d > es_max) es_max = rounds * 0x1p-24 * abs_d;
        if (s[j] > mt) mt = s[j];
        /* the two largest visible scores so far (a tie gives m1 == m2) */
        if ((double)s[j] > m1) {
          m2 = m1;
          m1 = s[j];
        } else if ((double)s[j] > m2) {
          m2 = s[j];
        }
      } else {
        s[j] = -INFINITY;
      }
    }
    mnew = m > mt ? m : mt;
    alpha = (m == -INFINITY) ? 0.0f : (float)exp((double)p->sm_scale * ((double)m - (double)mnew));
    for (int j = 0; j < tl; j++)
      pt[j] = (s[j] == -INFINITY) ? 0.0f : p_exp(p, (double)p->sm_scale * ((double)s[j] - (double)mnew));
    /* windows of this tile's exponentials (p_window); the element at the maximum
     * is exactly 1 on both sides when no other score lies within the score error
     * of it (the implementation forms block maxima as 2^(lambda (max - m))) */
    {
      const double es = es_max;
      const int unique = es == 0.0 || (double)mnew - m2 > 2.0 * es;
      /* the multiplier applied as an offset of the argument (p_window): the two-level
       * offset fl(lambda t - L) and L's own rounding, an E4M3 scale's offset added to it
       * (or to fl(lambda m)) and its logarithm, and the larger argument */
      double fold = 0.0;
      if (p->exp_mode == ORC_EXP_EXACT && p->pmode == ORC_P_FP8_FIXED && mt != -INFINITY) {
        /* 448 P~ as 2^(lambda s - fl(lambda m) + log2 448): the offset's rounding, the
         * rounding of log2 448 and the larger argument */
        const double u = 0x1p-24, L8 = log2(448.0);
        fold = u * (lam * fabs((double)mnew) + 2.5 * L8);
      } else if (p->exp_mode == ORC_EXP_EXACT && mt != -INFINITY) {
        const double u = 0x1p-24, L = log2(448.0 * 6.0);
        const double c1 = p->pmode == ORC_P_TWO_LEVEL ? fabs(lam * (double)mt - L) : lam * fabs((double)mnew);
        if (p->pmode == ORC_P_TWO_LEVEL) fold = u * (c1 + 1.5 * L);
        if (p->pfmt.scale == ORC_SCALE_E4M3) fold += u * (c1 + 20.0) + 0x1p-20;
      }
      for (int j = 0; j < tl; j++) {
        double a = s[j] == -INFINITY ? 0.0 : lam * ((double)s[j] - (double)mnew);
        we[j] = p_window(p, lam, es, a, mnew, fold);
        ws[j] = (p->exp_mode == ORC_EXP_EXACT && s[j] == mnew && unique) ? 0.0 : we[j];
      }
    }
    /* per-key fold of the diagonal tile: the quantizer sees P' = P~ 2^ek */
    const int fold = Vk != NULL && t0 >= diag_lo && t0 < diag_lo + QT;
    float* pq = pt;
    if (fold) {
      for (int j = 0; j < tl; j++) x2[j] = ldexpf(pt[j], ek[t0 + j]);
      pq = x2;
    }

    /* P quantization of this tile */
    for (int j = 0; j < tl; j++) {
      ph[j] = pq[j];
      dl[j] = 0.0;
    }
    if (p->pmode == ORC_P_TWO_LEVEL) {
      float r = 0.0f, s1;
      double rlo = 0.0, rhi = 0.0, wr;
      for (int j = 0; j < tl; j++) {
        if (pq[j] > r) r = pq[j];
        if ((double)pq[j] * (1.0 - ws[j]) > rlo) rlo = (double)pq[j] * (1.0 - ws[j]);
        if ((double)pq[j] * (1.0 + ws[j]) > rhi) rhi = (double)pq[j] * (1.0 + ws[j]);
      }
      if (r == 0.0f) { /* nothing visible in this tile */
        m = mnew;
        continue;
      }
      /* the pre-scale's window: where the implementation's tile maximum can lie */
      wr = ((double)r - rlo) / (double)r;
      if ((rhi - (double)r) / (double)r > wr) wr = (rhi - (double)r) / (double)r;
      s1 = r / (448.0f * 6.0f);
      for (int j = 0; j < tl; j++) {
        x2[j] = pq[j] / s1; /* in place when folded */
        we[j] += wr;
        ws[j] += wr;
      }
      for (int b0 = 0; b0 < tl; b0 += p->pfmt.block) {
        int n = tl - b0 < p->pfmt.block ? tl - b0 : p->pfmt.block;
        p_block(x2 + b0, we + b0, ws + b0, n, &p->pfmt, ph + b0, dl + b0);
      }
      mult = s1;
    } else if (p->pmode == ORC_P_DIRECT || p->pmode == ORC_P_PNQ) {
      for (int b0 = 0; b0 < tl; b0 += p->pfmt.block) {
        int n = tl - b0 < p->pfmt.block ? tl - b0 : p->pfmt.block;
        p_block(pq + b0, we + b0, ws + b0, n, &p->pfmt, ph + b0, dl + b0);
      }
    } else if (p->pmode == ORC_P_FP8_FIXED) {
      for (int j = 0; j < tl; j++) {
        float y = 448.0f * pt[j];
        int c = orc_e4m3_encode(y), alt = elem_alt(ORC_ELEM_E4M3, y, c, we[j]);
        ph[j] = orc_e4m3_value(c);
        if (alt >= 0) dl[j] = fabs(orc_e4m3_value(alt) - ph[j]);
      }
      mult = 1.0f / 448.0f; /* only scales the flip budget; O divides by 448 */
    }

    /* l = alpha l + rowsum(w): w = P^ for PNQ, P~ otherwise */
    for (int j = 0; j < tl; j++)
      wsum += (p->pmode == ORC_P_PNQ) ? (fold ? ldexp(ph[j], -ek[t0 + j]) : ph[j]) : (double)pt[j];
    l = alpha * l + (float)wsum;

    /* O~ = alpha O~ + P^ V (times s1 or 1/448); the folded tile takes the per-key V */
    const float* Vt = fold ? Vk : V;
    for (int c = 0; c < d; c++) col[c] = 0.0;
    for (int j = 0; j < tl; j++) {
      if (ph[j] == 0.0) continue;
      for (int c = 0; c < d; c++) col[c] += ph[j] * (double)Vt[(int64_t)(t0 + j) * d + c];
    }
    for (int c = 0; c < d; c++) {
      float t = (float)col[c];
      if (p->pmode == ORC_P_TWO_LEVEL) t = mult * t;
      else if (p->pmode == ORC_P_FP8_FIXED) t = t / 448.0f;
      acc[c] = alpha * acc[c] + t;
    }

    /* flip budget of this tile, carried with the same alpha as O~ */
    for (int j = 0; j < tl; j++) {
      if (dl[j] == 0.0) continue;
      double vmax = 0.0;
      for (int c = 0; c < d; c++) {
        double a = fabs((double)Vt[(int64_t)(t0 + j) * d + c]);
        if (a > vmax) vmax = a;
      }
      dsum1 += dl[j] * (double)mult * vmax;
      dsum2 += dl[j] * (double)mult * (fold ? ldexp(1.0, -ek[t0 + j]) : 1.0);
    }
    fb1 = (double)alpha * fb1 + dsum1;
    fb2 = (double)alpha * fb2 + dsum2;
    m = mnew;
  }

  if (l == 0.0f) {
    for (int c = 0; c < d; c++) o[c] = 0.0f;
    if (lse) *lse = -INFINITY;
    if (fb) *fb = 0.0;
  } else {
    double omax = 0.0;
    for (int c = 0; c < d; c++) {
      o[c] = acc[c] / l;
      if (fabs((double)o[c]) > omax) omax = fabs((double)o[c]);
    }
    if (lse) *lse = (float)(log((double)l) + (double)p->sm_scale * (double)m);
    if (fb) *fb = (fb1 + (p->pmode == ORC_P_PNQ ? fb2 * omax : 0.0)) / (double)l;
  }
  free(acc);
  free(s);
  free(pt);
  free(x2);
  free(ph);
  free(dl);
  free(col);
  free(we);
  free(ws);
  free(qg);
  return 0;
}

int orc_attention(const float* Q, const float* K, const float* V, int B, int Hq, int Hkv, int N,
                  int d, const int* doc_off, int ndocs, const orc_attn_params* p,
                  const int64_t* rows, int64_t nrows, float* O, float* lse, double* fb) {
  return orc_attention_bias(Q, K, V, NULL, B, Hq, Hkv, N, d, doc_off, ndocs, p, rows, nrows, O, lse, fb);
}

int orc_attention_bias(const float* Q, const float* K, const float* V, const float* bias, int B,
                       int Hq, int Hkv, int N, int d, const int* doc_off, int ndocs,
                       const orc_attn_params* p, const int64_t* rows, int64_t nrows, float* O,
                       float* lse, double* fb) {
  return orc_attention_ex(Q, K, V, bias, NULL, NULL, B, Hq, Hkv, N, d, doc_off, ndocs, p, rows, nrows, O,
                          lse, fb);
}

int orc_attention_ex(const float* Q, const float* K, const float* V, const float* bias, const float* Vk,
                     const int* ek, int B, int Hq, int Hkv, int N, int d, const int* doc_off, int ndocs,
                     const orc_attn_params* p, const int64_t* rows, int64_t nrows, float* O, float* lse,
                     double* fb) {
  int64_t total = (int64_t)B * Hq * N;
  const int QT = p->q_tile > 0 ? p->q_tile : p->kv_tile;
  if (Vk && !p->causal) return -3; /* the per-key form serves causal diagonal tiles */
  if (Vk && QT % p->kv_tile != 0) return -5;
  if (p->exp_mode < ORC_EXP_EXACT || p->exp_mode > ORC_EXP_SCHRAUDOLPH) return -4;
  if (!rows) nrows = total;
  if (doc_off && ndocs > 0 && B != 1) return -1;
  for (int64_t idx = 0; idx < nrows; idx++) {
    int64_t r = rows ? rows[idx] : idx;
    int64_t b = r / ((int64_t)Hq * N);
    int h = (int)((r / N) % Hq);
    int i = (int)(r % N);
    int hk = h * Hkv / Hq; /* grouped-query attention: Hq/Hkv query heads per KV head */
    int ks = 0, ke = N, nk, vis;
    const float* kb = K + ((b * Hkv + hk) * (int64_t)N) * d;
    const float* vb = V + ((b * Hkv + hk) * (int64_t)N) * d;
    if (r < 0 || r >= total) return -2;
    if (doc_off && ndocs > 0) {
      for (int k = 0; k < ndocs; k++)
        if (doc_off[k] <= i && i < doc_off[k + 1]) {
          ks = doc_off[k];
          ke = doc_off[k + 1];
        }
    }
    nk = ke - ks;
    vis = p->causal ? (i - ks + 1) : nk;
    const float* vkb = Vk ? Vk + ((b * Hkv + hk) * (int64_t)N + ks) * d : NULL;
    const int* ekb = ek ? ek + (b * Hkv + hk) * (int64_t)N + ks : NULL;
    /* the row's diagonal tiles: those starting in its query tile's rows,
     * [QT floor((i - ks) / QT), + QT) */
    int diag = Vk ? ((i - ks) / QT) * QT : -1;
    attn_row_bias(Q + r * d, kb + (int64_t)ks * d, vb + (int64_t)ks * d,
                  bias ? bias + (b * Hq + h) * (int64_t)N + ks : NULL, vkb, ekb, diag, nk, vis, d, p,
                  O + idx * d, lse ? lse + idx : NULL, fb ? fb + idx : NULL);
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Outlier pre-processing ([MPFA] section 4.2-4.3, [FLAMIA] section 3.4 and   */
/* appendix A.2, [MXF4] "Smooth-K is the smaller lever").                     */
/* ------------------------------------------------------------------------ */
static int doc_of(int t, const int* doc_off, int ndocs) {
  if (!doc_off || ndocs <= 0) return 0;
  for (int k = 0; k < ndocs; k++)
    if (doc_off[k] <= t && t < doc_off[k + 1]) return k;
  return ndocs - 1;
}

void orc_channel_mean(const float* x, int N, int d, const int* doc_off, int ndocs, float* mean) {
  int nd = (doc_off && ndocs > 0) ? ndocs : 1;
  for (int k = 0; k < nd; k++) {
    int t0 = (doc_off && ndocs > 0) ? doc_off[k] : 0;
    int t1 = (doc_off && ndocs > 0) ? doc_off[k + 1] : N;
    for (int c = 0; c < d; c++) {
      double sum = 0.0;
      for (int t = t0; t < t1; t++) sum += (double)x[(int64_t)t * d + c];
      mean[(int64_t)k * d + c] = (t1 > t0) ? (float)(sum / (double)(t1 - t0)) : 0.0f;
    }
  }
}

static int hadamard_sign(int i, int j) { return __builtin_popcount((unsigned)(i & j)) & 1 ? -1 : 1; }

void orc_preprocess_rows(const float* x, int N, int d, const float* mean, const int* doc_off,
                         int ndocs, int hadamard, float* out) {
  double* y = (double*)malloc(sizeof(double) * (size_t)d);
  const double c = 1.0 / sqrt((double)d);
  for (int t = 0; t < N; t++) {
    const float* mu = mean ? mean + (int64_t)doc_of(t, doc_off, ndocs) * d : NULL;
    for (int i = 0; i < d; i++) y[i] = (double)x[(int64_t)t * d + i] - (mu ? (double)mu[i] : 0.0);
    for (int j = 0; j < d; j++) {
      double z;
      if (hadamard) {
        z = 0.0;
        for (int i = 0; i < d; i++) z += hadamard_sign(i, j) > 0 ? y[i] : -y[i];
        z = z * c;
      } else {
        z = y[j];
      }
      out[(int64_t)t * d + j] = (float)z;
    }
  }
  free(y);
}

void orc_center_comp(const float* qmean, const float* K, const float* kmean, int N, int d,
                     const int* doc_off, int ndocs, float* delta) {
  for (int j = 0; j < N; j++) {
    int k = doc_of(j, doc_off, ndocs);
    double acc = 0.0;
    for (int c = 0; c < d; c++)
      acc += (double)qmean[(int64_t)k * d + c] *
             ((double)K[(int64_t)j * d + c] - (double)kmean[(int64_t)k * d + c]);
    delta[j] = (float)acc;
  }
}

/* Per-key form of V ([FLAMIA] section 3.2: a per-key power-of-two scale for a 4-bit
 * V on diagonal tiles): for each token j the block is its d channels, the E8M0
 * exponent ek[j] follows f's rule from the block maximum, and the codes are the
 * element codes of V[j][c] / 2^ek[j].  x: [N][d]; codes: [N][d]; ek: [N].
 * E8M0 formats only.  Pinned by tests/test_oracle_causal_safe.py. */
void orc_quantize_keys(const float* x, int N, int d, const orc_fmt* f, uint8_t* codes, int* ek) {
  orc_fmt fk = *f;
  fk.block = d;
  for (int j = 0; j < N; j++) {
    uint8_t sb;
    orc_quant_block(x + (int64_t)j * d, d, &fk, codes + (int64_t)j * d, &sb);
    ek[j] = (int)sb - 127;
  }
}

/* ------------------------------------------------------------------------ */
/* Decode with split keys and a log-sum-exp merge ([MPFA] section 5.3).      */
/* ------------------------------------------------------------------------ */
int orc_decode(const float* Q, const float* K, const float* V, int B, int Hq, int Hkv, int R, int N,
               int d, const int* kv_len, int split, const orc_attn_params* p, float* O, float* lse,
               double* fb) {
  if (split <= 0 || split % p->kv_tile != 0 || !p->causal) return -1;
  if (p->exp_mode < ORC_EXP_EXACT || p->exp_mode > ORC_EXP_SCHRAUDOLPH) return -4;
  float* os = (float*)malloc(sizeof(float) * (size_t)d);
  double* acc = (double*)malloc(sizeof(double) * (size_t)d);
  for (int b = 0; b < B; b++) {
    const int L = kv_len[b];
    if (L < R || L > N) {
      free(os);
      free(acc);
      return -2;
    }
    const int nsplit = (L + split - 1) / split;
    for (int h = 0; h < Hq; h++) {
      const int hk = h * Hkv / Hq;
      const float* kb = K + ((int64_t)(b * Hkv + hk) * N) * d;
      const float* vb = V + ((int64_t)(b * Hkv + hk) * N) * d;
      for (int r = 0; r < R; r++) {
        const int pos = L - R + r; /* keys 0..pos are visible */
        const float* q = Q + ((int64_t)((b * Hq + h) * R + r)) * d;
        double M = -INFINITY, wsum = 0.0, fbs = 0.0;
        float ls;
        double f1;
        /* first pass: the maximum lse of the splits */
        double* lses = (double*)malloc(sizeof(double) * (size_t)(nsplit > 0 ? nsplit : 1));
        for (int s = 0; s < nsplit; s++) {
          const int k0 = s * split, nk = (L - k0 < split) ? L - k0 : split;
          const int vis = pos - k0 + 1 < 0 ? 0 : (pos - k0 + 1 < nk ? pos - k0 + 1 : nk);
          orc_attn_row(q, kb + (int64_t)k0 * d, vb + (int64_t)k0 * d, nk, vis, d, p, os, &ls, &f1);
          lses[s] = (vis > 0) ? (double)ls : -INFINITY;
          if (lses[s] > M) M = lses[s];
        }
        for (int c = 0; c < d; c++) acc[c] = 0.0;
        for (int s = 0; s < nsplit; s++) {
          const int k0 = s * split, nk = (L - k0 < split) ? L - k0 : split;
          const int vis = pos - k0 + 1 < 0 ? 0 : (pos - k0 + 1 < nk ? pos - k0 + 1 : nk);
          if (vis <= 0 || lses[s] == -INFINITY) continue;
          orc_attn_row(q, kb + (int64_t)k0 * d, vb + (int64_t)k0 * d, nk, vis, d, p, os, &ls, &f1);
          const double w = exp(lses[s] - M);
          wsum += w;
          fbs += w * f1;
          for (int c = 0; c < d; c++) acc[c] += w * (double)os[c];
        }
        float* o = O + ((int64_t)((b * Hq + h) * R + r)) * d;
        for (int c = 0; c < d; c++) o[c] = wsum > 0.0 ? (float)(acc[c] / wsum) : 0.0f;
        if (lse) lse[(b * Hq + h) * R + r] = wsum > 0.0 ? (float)(M + log(wsum)) : -INFINITY;
        if (fb) fb[(b * Hq + h) * R + r] = wsum > 0.0 ? fbs / wsum : 0.0;
        free(lses);
      }
    }
  }
  free(os);
  free(acc);
  return 0;
}
