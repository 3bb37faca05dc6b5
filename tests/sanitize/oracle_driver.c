/* Sanitizer harness of the oracle: every entry point of oracle/oracle.h on small
 * inputs (several formats and P modes, causal and packed documents, bias, the per-key
 * V form, split decode, pre-processing), built with -fsanitize=address,undefined by
 * tests/test_sanitizers.py.  It checks memory and undefined-behaviour safety only;
 * parity lives in the other tests.  Inputs come from a small local generator. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static uint64_t st = 0x9E3779B97F4A7C15ull;
static float rnd(void) { /* uniform in [-2, 2) */
  st = st * 6364136223846793005ull + 1442695040888963407ull;
  return (float)((double)(st >> 11) * 0x1p-53 * 4.0 - 2.0);
}

#define D 128

static void fill(float* x, int64_t n, float scale) {
  for (int64_t i = 0; i < n; i++) x[i] = scale * rnd();
}

int main(void) {
  const int B = 1, Hq = 2, Hkv = 1, N = 161;
  const int doc_off[] = {0, 1, 40, 41, 130, 161};
  const int ndocs = 5;
  const orc_fmt fmts[] = {
      {ORC_ELEM_E2M1, ORC_SCALE_E8M0, 32, ORC_RULE_OCP, 0.0f},
      {ORC_ELEM_E2M1, ORC_SCALE_E8M0, 32, ORC_RULE_CEIL, 7.25f},
      {ORC_ELEM_E2M1, ORC_SCALE_E4M3, 16, ORC_RULE_OCP, 0.0f},
      {ORC_ELEM_E4M3, ORC_SCALE_E8M0, 32, ORC_RULE_CEIL, 448.0f},
  };
  float* q = malloc(sizeof(float) * (size_t)B * Hq * N * D);
  float* k = malloc(sizeof(float) * (size_t)B * Hkv * N * D);
  float* v = malloc(sizeof(float) * (size_t)B * Hkv * N * D);
  float* qd = malloc(sizeof(float) * (size_t)B * Hq * N * D);
  float* kd = malloc(sizeof(float) * (size_t)B * Hkv * N * D);
  float* vd = malloc(sizeof(float) * (size_t)B * Hkv * N * D);
  float* vk = malloc(sizeof(float) * (size_t)B * Hkv * N * D);
  int* ek = malloc(sizeof(int) * (size_t)B * Hkv * N);
  float* bias = malloc(sizeof(float) * (size_t)B * Hq * N);
  float* O = malloc(sizeof(float) * (size_t)B * Hq * N * D);
  float* lse = malloc(sizeof(float) * (size_t)B * Hq * N);
  double* fb = malloc(sizeof(double) * (size_t)B * Hq * N);
  uint8_t* codes = malloc((size_t)B * Hq * N * D);
  uint8_t* scales = malloc((size_t)B * Hq * N * D);
  double sum = 0.0;
  fill(q, (int64_t)B * Hq * N * D, 1.0f);
  fill(k, (int64_t)B * Hkv * N * D, 1.0f);
  fill(v, (int64_t)B * Hkv * N * D, 1.0f);
  fill(bias, (int64_t)B * Hq * N, 0.5f);
  k[5] = 0.0f;
  k[6] = -0.0f;
  k[7] = 1e-30f;
  v[9] = 3e4f;

  for (int fi = 0; fi < 4; fi++) {
    const orc_fmt* f = &fmts[fi];
    const orc_fmt* fqk = f->elem == ORC_ELEM_E4M3 ? &fmts[0] : f;
    orc_quantize_rows(q, (int64_t)B * Hq * N, D, fqk, codes, scales);
    orc_dequant_rows(codes, scales, (int64_t)B * Hq * N, D, fqk, qd);
    orc_quantize_rows(k, (int64_t)B * Hkv * N, D, fqk, codes, scales);
    orc_dequant_rows(codes, scales, (int64_t)B * Hkv * N, D, fqk, kd);
    for (int h = 0; h < B * Hkv; h++) {
      const int* dof = (fi & 1) ? doc_off : NULL;
      const int nd = (fi & 1) ? ndocs : 0;
      const int64_t nblk = orc_v_nblocks(N, dof, nd, f->block);
      if (nblk * D > (int64_t)B * Hq * N * D) return 3;
      orc_quantize_cols(v + (int64_t)h * N * D, N, D, dof, nd, f, codes, scales);
      orc_dequant_cols(codes, scales, N, D, dof, nd, f, vd + (int64_t)h * N * D);
      if (f->elem == ORC_ELEM_E2M1 && f->scale == ORC_SCALE_E8M0)
        orc_quantize_keys(v + (int64_t)h * N * D, N, D, f, codes, ek + (int64_t)h * N);
    }
    for (int64_t i = 0; i < (int64_t)B * Hkv * N * D; i++) vk[i] = (float)orc_e2m1_value(codes[i % ((int64_t)N * D)] & 15);
    for (int pm = ORC_P_NONE; pm <= ORC_P_FP8_FIXED; pm++) {
      orc_attn_params p;
      memset(&p, 0, sizeof p);
      p.pmode = pm;
      p.pfmt = pm == ORC_P_TWO_LEVEL ? fmts[2] : fmts[fi == 3 ? 0 : fi];
      p.sm_scale = 1.0f / sqrtf((float)D);
      p.kv_tile = 128;
      p.score_rounds = 2;
      for (int causal = 0; causal < 2; causal++) {
        p.causal = causal;
        for (int em = 0; em < (fi == 0 ? 3 : 1); em++) {
          p.exp_mode = em;
          orc_attention(qd, kd, vd, B, Hq, Hkv, N, D, NULL, 0, &p, NULL, 0, O, lse, fb);
          sum += O[7] + lse[3] + fb[1];
          orc_attention_bias(qd, kd, vd, bias, B, Hq, Hkv, N, D, doc_off, ndocs, &p, NULL, 0, O, lse, fb);
          sum += O[11];
          if (causal)
            orc_attention_ex(qd, kd, vd, bias, vk, ek, B, Hq, Hkv, N, D, doc_off, ndocs, &p, NULL, 0, O, lse, fb);
        }
      }
      {
        const int kv_len[1] = {N - 5};
        p.causal = 1;
        p.exp_mode = 0;
        orc_decode(qd, kd, vd, B, Hq, Hkv, 3, N, D, kv_len, 64, &p, O, lse, fb);
        sum += O[0];
      }
    }
  }
  /* element and scale encoders at their edges */
  for (int c = 0; c < 16; c++) sum += orc_e2m1_value(c);
  for (int c = 0; c < 256; c++) sum += isnan(orc_e4m3_value(c)) ? 0.0 : orc_e4m3_value(c);
  {
    const float xs[] = {0.0f, -0.0f, 1e-45f, 0.25f, 0.75f, 5.0f, 6.0f, 448.0f, 464.0f, 1e30f, INFINITY, -INFINITY};
    for (int i = 0; i < 12; i++) sum += orc_e2m1_encode(xs[i]) + orc_e4m3_encode(xs[i]);
    for (int i = 0; i < 12; i++)
      for (int r = 0; r < 2; r++) sum += orc_e8m0_exponent(fabsf(xs[i]), r, r ? 7.25f : 0.0f, ORC_ELEM_E2M1);
  }
  for (double t = -140.0; t < 130.0; t += 0.37) sum += orc_exp2_bits(t);
  sum += orc_exp_offset(0) + orc_exp_offset(1) + orc_exp_offset(2);
  /* pre-processing */
  {
    float* mean = malloc(sizeof(float) * (ndocs + 1) * D);
    float* kmean = malloc(sizeof(float) * (ndocs + 1) * D);
    float* delta = malloc(sizeof(float) * N);
    orc_channel_mean(q, N, D, doc_off, ndocs, mean);
    orc_channel_mean(k, N, D, doc_off, ndocs, kmean);
    orc_preprocess_rows(q, N, D, mean, doc_off, ndocs, 1, qd);
    orc_preprocess_rows(k, N, D, NULL, NULL, 0, 0, kd);
    orc_center_comp(mean, k, kmean, N, D, doc_off, ndocs, delta);
    sum += delta[N - 1] + qd[5] + kd[6];
    free(mean);
    free(kmean);
    free(delta);
  }
  printf("oracle sanitizer harness done (%g)\n", sum);
  free(q); free(k); free(v); free(qd); free(kd); free(vd); free(vk); free(ek); free(bias);
  free(O); free(lse); free(fb); free(codes); free(scales);
  return 0;
}
