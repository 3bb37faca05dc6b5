// host.cpp -- the C ABI of libmxattn (include/mxattn.h): argument validation,
// layout arithmetic, forward plans and kernel launches.  No allocation, no
// synchronization, no global state apart from a thread-local error text.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "kernels.h"
#include "mxattn.h"

using namespace mxattn;

namespace {

thread_local char g_err[256] = "";

// test hook: the next g_fail_launches device submissions on this thread are not made
// and report hipErrorLaunchFailure (mxattn_debug_fail_launches)
thread_local int g_fail_launches = 0;

hipError_t forced_failure() {
  if (g_fail_launches <= 0) return hipSuccess;
  g_fail_launches--;
  return hipErrorLaunchFailure;
}

int hip_fail(hipError_t e, const char* what) {
  snprintf(g_err, sizeof g_err, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
  return MXATTN_E_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// format checks shared by sizing and quantization
int check_fmt(const mxattn_qfmt* f, int role) {
  if (f == nullptr) return MXATTN_E_INVALID;
  if (f->elem == MXATTN_ELEM_BF16) {  // the unquantized route: plain bf16 values
    if (f->scale != MXATTN_SCALE_NONE) return MXATTN_E_INVALID;
    if (role != MXATTN_ROLE_QK && role != MXATTN_ROLE_V) return MXATTN_E_UNSUPPORTED;
    return MXATTN_OK;
  }
  if (f->elem != MXATTN_ELEM_E2M1 && f->elem != MXATTN_ELEM_E4M3) return MXATTN_E_INVALID;
  if (f->scale != MXATTN_SCALE_E8M0 && f->scale != MXATTN_SCALE_E4M3) return MXATTN_E_INVALID;
  if (f->block != 16 && f->block != 32) return MXATTN_E_UNSUPPORTED;
  if (role != MXATTN_ROLE_QK && role != MXATTN_ROLE_V && role != MXATTN_ROLE_VKEY && role != MXATTN_ROLE_VT)
    return MXATTN_E_INVALID;
  if (role == MXATTN_ROLE_VKEY && (f->elem != MXATTN_ELEM_E2M1 || f->scale != MXATTN_SCALE_E8M0))
    return MXATTN_E_UNSUPPORTED;
  if (role == MXATTN_ROLE_VT && (f->scale != MXATTN_SCALE_E8M0 || f->block != 32))  // MXFP4 or FP8 V
    return MXATTN_E_UNSUPPORTED;
  if (f->scale == MXATTN_SCALE_E8M0) {
    if (f->rule != MXATTN_RULE_OCP && f->rule != MXATTN_RULE_CEIL) return MXATTN_E_INVALID;
    if (f->rule == MXATTN_RULE_CEIL && !(f->qmax >= 1.0f && f->qmax <= 448.0f)) return MXATTN_E_INVALID;
  }
  if (f->elem == MXATTN_ELEM_E4M3 && (f->scale != MXATTN_SCALE_E8M0 || (role != MXATTN_ROLE_V && role != MXATTN_ROLE_VT)))
    return MXATTN_E_UNSUPPORTED;
  return MXATTN_OK;
}

// E8M0 exponent rule as the two integers the kernels use (formats.h)
E8m0Rule make_rule(const mxattn_qfmt* f) {
  E8m0Rule r;
  if (f->rule == MXATTN_RULE_OCP) {
    r.qe = 127 + (f->elem == MXATTN_ELEM_E2M1 ? 2 : 8);
    r.qm = 0x7FFFFFu;
  } else {
    uint32_t b;
    memcpy(&b, &f->qmax, 4);
    r.qe = (int32_t)(b >> 23);
    r.qm = b & 0x7FFFFFu;
  }
  return r;
}

int64_t v_padded(int64_t N, int ndocs, int block) {
  int64_t n = ndocs > 1 ? N + (int64_t)ndocs * (block - 1) : N;
  return (n + 127) / 128 * 128;
}

int bits_of(int elem) { return elem == MXATTN_ELEM_E2M1 ? 4 : elem == MXATTN_ELEM_BF16 ? 16 : 8; }

bool is_bf16(const mxattn_qfmt& f) { return f.elem == MXATTN_ELEM_BF16 && f.scale == MXATTN_SCALE_NONE; }

bool same_fmt(const mxattn_qfmt& a, const mxattn_qfmt& b) {
  if (a.elem != b.elem || a.scale != b.scale || a.block != b.block) return false;
  if (a.scale == MXATTN_SCALE_E8M0 && (a.rule != b.rule || (a.rule == MXATTN_RULE_CEIL && a.qmax != b.qmax)))
    return false;
  return true;
}

bool is_mxfp4(const mxattn_qfmt& f) {
  return f.elem == MXATTN_ELEM_E2M1 && f.scale == MXATTN_SCALE_E8M0 && f.block == 32;
}
bool is_nvfp4(const mxattn_qfmt& f) {
  return f.elem == MXATTN_ELEM_E2M1 && f.scale == MXATTN_SCALE_E4M3 && f.block == 16;
}
bool is_fp8v(const mxattn_qfmt& f) {
  return f.elem == MXATTN_ELEM_E4M3 && f.scale == MXATTN_SCALE_E8M0 && f.block == 32;
}

int64_t plan_cap(int64_t N, int ndocs, int rows) { return (N + rows - 1) / rows + ndocs; }

size_t plan_bytes(int64_t N, int ndocs) {
  if (ndocs <= 0) return 0;
  int64_t items = plan_cap(N, ndocs, 128) + plan_cap(N, ndocs, 256);
  return sizeof(PlanHeader) + sizeof(DocEntry) * (size_t)ndocs + sizeof(WorkItem) * (size_t)items;
}

}  // namespace

extern "C" {

int mxattn_abi_version(void) { return MXATTN_ABI_VERSION; }

const char* mxattn_status_str(int s) {
  switch (s) {
    case MXATTN_OK: return "ok";
    case MXATTN_E_INVALID: return "invalid argument";
    case MXATTN_E_UNSUPPORTED: return "unsupported combination";
    case MXATTN_E_ALIGN: return "misaligned pointer or stride";
    case MXATTN_E_WORKSPACE: return "workspace missing or too small";
    case MXATTN_E_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* mxattn_last_error(void) { return g_err; }
const char* mxattn_last_hip_error(void) { return g_err; }

int mxattn_debug_fail_launches(int count) {
  const int prev = g_fail_launches;
  g_fail_launches = count > 0 ? count : 0;
  return prev;
}

int mxattn_qtensor_bytes(const mxattn_qfmt* fmt, int role, int64_t B, int64_t H, int64_t N, int64_t d, int ndocs,
                         size_t* code_bytes, size_t* scale_bytes, int64_t* n_padded) {
  int rc = check_fmt(fmt, role);
  if (rc != MXATTN_OK) return rc;
  if (code_bytes == nullptr || scale_bytes == nullptr) return MXATTN_E_INVALID;
  if (B < 0 || H < 0 || N < 0 || d <= 0 || ndocs < 0) return MXATTN_E_INVALID;
  if (d != 128) return MXATTN_E_UNSUPPORTED;
  if (ndocs > 1 && B != 1) return MXATTN_E_INVALID;
  int bits = bits_of(fmt->elem);
  if (fmt->elem == MXATTN_ELEM_BF16) {  // every role: the values as [B][H][N][d]
    *code_bytes = (size_t)(B * H * N * d * 2);
    *scale_bytes = 0;
    if (n_padded) *n_padded = N;
  } else if (role == MXATTN_ROLE_QK) {
    *code_bytes = (size_t)(B * H * N * d * bits / 8);
    *scale_bytes = (size_t)(B * H * N * (d / fmt->block));
    if (n_padded) *n_padded = N;
  } else if (role == MXATTN_ROLE_V || role == MXATTN_ROLE_VT) {
    if (role == MXATTN_ROLE_VT && ndocs > 1) return MXATTN_E_INVALID;  // tile-major V takes no documents
    int64_t np = v_padded(N, ndocs, fmt->block);
    *code_bytes = (size_t)(B * H * d * np * bits / 8);
    *scale_bytes = (size_t)(B * H * d * (np / fmt->block));
    if (n_padded) *n_padded = np;
  } else {  // VKEY: role V's codes, one scale byte per key slot
    int64_t np = v_padded(N, ndocs, fmt->block);
    *code_bytes = (size_t)(B * H * d * np * bits / 8);
    *scale_bytes = (size_t)(B * H * np);
    if (n_padded) *n_padded = np;
  }
  return MXATTN_OK;
}

int mxattn_quantize(const void* x_bf16, const int64_t x_strides[4], int64_t B, int64_t H, int64_t N, int64_t d,
                    int role, const mxattn_qfmt* fmt, const int32_t* cu_seqlens, int ndocs, mxattn_qtensor* out,
                    void* stream) {
  size_t cb, sb;
  int64_t np;
  int rc = mxattn_qtensor_bytes(fmt, role, B, H, N, d, ndocs, &cb, &sb, &np);
  if (rc != MXATTN_OK) return rc;
  if (out == nullptr || x_strides == nullptr) return MXATTN_E_INVALID;
  if (ndocs > 1 && (cu_seqlens == nullptr || role == MXATTN_ROLE_QK)) return MXATTN_E_INVALID;
  if (x_strides[3] != 1 || x_strides[0] < 0 || x_strides[1] < 0 || x_strides[2] < 0) return MXATTN_E_INVALID;
  const int64_t nel = B * H * N;
  const bool raw = fmt->elem == MXATTN_ELEM_BF16;
  if (nel > 0) {
    if (x_bf16 == nullptr || out->codes == nullptr || (!raw && out->scales == nullptr)) return MXATTN_E_INVALID;
    if (!aligned16(x_bf16) || !aligned16(out->codes) || (!raw && !aligned16(out->scales))) return MXATTN_E_ALIGN;
    if ((x_strides[0] % 8) || (x_strides[1] % 8) || (x_strides[2] % 8)) return MXATTN_E_ALIGN;
  }
  out->fmt = *fmt;
  out->role = role;
  out->ndocs = ndocs > 1 ? ndocs : 1;
  out->B = B;
  out->H = H;
  out->N = N;
  out->d = d;
  out->n_padded = np;
  if (raw) {  // the unquantized route: a dense copy, [B][H][N][d]
    if (nel == 0) return MXATTN_OK;
    if (nel >= (int64_t(1) << 27)) return MXATTN_E_UNSUPPORTED;  // 16 threads per row, 32-bit ids
    hipError_t e = forced_failure();
    if (e == hipSuccess)
      e = launch_copy_bf16(x_bf16, x_strides[0], x_strides[1], x_strides[2], B, H, N, out->codes,
                           static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "mxattn_quantize launch");
    return MXATTN_OK;
  }
  if (nel == 0 && !(role != MXATTN_ROLE_QK && B * H > 0 && np > 0)) return MXATTN_OK;
  // role QK: 4 rows per thread and 16 threads per 4 rows, 32-bit row indices
  if (role == MXATTN_ROLE_QK && nel >= (int64_t(1) << 30)) return MXATTN_E_UNSUPPORTED;

  QuantArgs a;
  a.x = x_bf16;
  a.sB = x_strides[0];
  a.sH = x_strides[1];
  a.sN = x_strides[2];
  a.B = B;
  a.H = H;
  a.N = N;
  a.np = np;
  a.elem = fmt->elem;
  a.scale = fmt->scale;
  a.block = fmt->block;
  a.rule = make_rule(fmt);
  a.cu = ndocs > 1 ? cu_seqlens : nullptr;
  a.ndocs = ndocs > 1 ? ndocs : 1;
  a.codes = out->codes;
  a.scales = out->scales;
  a.tiled = role == MXATTN_ROLE_VT ? 1 : 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = forced_failure();
  if (e == hipSuccess)
    e = role == MXATTN_ROLE_QK                               ? launch_quant_qk(a, st)
        : role == MXATTN_ROLE_V || role == MXATTN_ROLE_VT ? launch_quant_v(a, st)
                                                          : launch_quant_vkey(a, st);
  if (e != hipSuccess) return hip_fail(e, "mxattn_quantize launch");
  return MXATTN_OK;
}

int mxattn_channel_mean(const void* x_bf16, const int64_t x_strides[4], int64_t B, int64_t H, int64_t N, int64_t d,
                        const int32_t* cu_seqlens, int ndocs, float* mean, void* stream) {
  if (x_strides == nullptr || B < 0 || H < 0 || N < 0 || ndocs < 0) return MXATTN_E_INVALID;
  if (d != 128) return MXATTN_E_UNSUPPORTED;
  if (ndocs > 1 && cu_seqlens == nullptr) return MXATTN_E_INVALID;
  if (x_strides[3] != 1 || x_strides[0] < 0 || x_strides[1] < 0 || x_strides[2] < 0) return MXATTN_E_INVALID;
  if (B * H == 0) return MXATTN_OK;
  if (mean == nullptr || (N > 0 && x_bf16 == nullptr)) return MXATTN_E_INVALID;
  if (!aligned16(mean) || (N > 0 && !aligned16(x_bf16))) return MXATTN_E_ALIGN;
  if ((x_strides[0] % 8) || (x_strides[1] % 8) || (x_strides[2] % 8)) return MXATTN_E_ALIGN;
  QuantArgs a{};
  a.x = x_bf16;
  a.sB = x_strides[0];
  a.sH = x_strides[1];
  a.sN = x_strides[2];
  a.B = B;
  a.H = H;
  a.N = N;
  a.cu = ndocs > 1 ? cu_seqlens : nullptr;
  a.ndocs = ndocs > 1 ? ndocs : 1;
  hipError_t e = forced_failure();
  if (e == hipSuccess) e = launch_channel_mean(a, mean, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "mxattn_channel_mean launch");
  return MXATTN_OK;
}

int mxattn_quantize_pre(const void* x_bf16, const int64_t x_strides[4], int64_t B, int64_t H, int64_t N, int64_t d,
                        int role, const mxattn_qfmt* fmt, const mxattn_preproc* pre, const int32_t* cu_seqlens,
                        int ndocs, mxattn_qtensor* out, void* stream) {
  if (role != MXATTN_ROLE_QK) return MXATTN_E_INVALID;
  if (pre == nullptr) return mxattn_quantize(x_bf16, x_strides, B, H, N, d, role, fmt, nullptr, 0, out, stream);
  if (pre->hadamard != 0 && pre->hadamard != 1) return MXATTN_E_INVALID;
  if (ndocs < 0 || (ndocs > 1 && cu_seqlens == nullptr)) return MXATTN_E_INVALID;
  size_t cb, sb;
  int64_t np;
  int rc = mxattn_qtensor_bytes(fmt, role, B, H, N, d, 0, &cb, &sb, &np);
  if (rc != MXATTN_OK) return rc;
  if (out == nullptr || x_strides == nullptr) return MXATTN_E_INVALID;
  if (x_strides[3] != 1 || x_strides[0] < 0 || x_strides[1] < 0 || x_strides[2] < 0) return MXATTN_E_INVALID;
  const int64_t nel = B * H * N;
  if (nel > 0) {
    if (x_bf16 == nullptr || out->codes == nullptr || out->scales == nullptr) return MXATTN_E_INVALID;
    if (!aligned16(x_bf16) || !aligned16(out->codes) || !aligned16(out->scales)) return MXATTN_E_ALIGN;
    if ((x_strides[0] % 8) || (x_strides[1] % 8) || (x_strides[2] % 8)) return MXATTN_E_ALIGN;
    if (pre->mean != nullptr && !aligned16(pre->mean)) return MXATTN_E_ALIGN;
  }
  out->fmt = *fmt;
  out->role = role;
  out->ndocs = 1;
  out->B = B;
  out->H = H;
  out->N = N;
  out->d = d;
  out->n_padded = np;
  if (nel == 0) return MXATTN_OK;
  if (nel >= (int64_t(1) << 28)) return MXATTN_E_UNSUPPORTED;  // 16 threads per row, 32-bit thread ids
  QuantArgs a{};
  a.x = x_bf16;
  a.sB = x_strides[0];
  a.sH = x_strides[1];
  a.sN = x_strides[2];
  a.B = B;
  a.H = H;
  a.N = N;
  a.np = np;
  a.elem = fmt->elem;
  a.scale = fmt->scale;
  a.block = fmt->block;
  a.rule = make_rule(fmt);
  a.cu = ndocs > 1 ? cu_seqlens : nullptr;
  a.ndocs = ndocs > 1 ? ndocs : 1;
  a.codes = out->codes;
  a.scales = out->scales;
  hipError_t e = forced_failure();
  if (e == hipSuccess) e = launch_quant_qk_pre(a, pre->mean, pre->hadamard, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "mxattn_quantize_pre launch");
  return MXATTN_OK;
}

int mxattn_center_comp(const float* qmean, const void* k_bf16, const int64_t k_strides[4], const float* kmean,
                       int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, const int32_t* cu_seqlens,
                       int ndocs, float* delta, void* stream) {
  if (k_strides == nullptr || B < 0 || N < 0 || ndocs < 0) return MXATTN_E_INVALID;
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return MXATTN_E_INVALID;
  if (d != 128) return MXATTN_E_UNSUPPORTED;
  if (ndocs > 1 && cu_seqlens == nullptr) return MXATTN_E_INVALID;
  if (k_strides[3] != 1 || k_strides[0] < 0 || k_strides[1] < 0 || k_strides[2] < 0) return MXATTN_E_INVALID;
  if (B * N == 0) return MXATTN_OK;
  if (B * Hkv * N >= (int64_t(1) << 28)) return MXATTN_E_UNSUPPORTED;  // 16 threads per key row
  if (qmean == nullptr || kmean == nullptr || k_bf16 == nullptr || delta == nullptr) return MXATTN_E_INVALID;
  if (!aligned16(qmean) || !aligned16(kmean) || !aligned16(k_bf16) || !aligned16(delta)) return MXATTN_E_ALIGN;
  if ((k_strides[0] % 8) || (k_strides[1] % 8) || (k_strides[2] % 8)) return MXATTN_E_ALIGN;
  CompArgs a{};
  a.qmean = qmean;
  a.k = k_bf16;
  a.sB = k_strides[0];
  a.sH = k_strides[1];
  a.sN = k_strides[2];
  a.kmean = kmean;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.N = N;
  a.cu = ndocs > 1 ? cu_seqlens : nullptr;
  a.ndocs = ndocs > 1 ? ndocs : 1;
  a.delta = delta;
  hipError_t e = forced_failure();
  if (e == hipSuccess) e = launch_center_comp(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "mxattn_center_comp launch");
  return MXATTN_OK;
}

size_t mxattn_fwd_workspace_bytes(int64_t N, int ndocs) { return plan_bytes(N, ndocs); }

size_t mxattn_decode_workspace_bytes(int64_t B, int64_t Hq, int64_t R, int64_t N) {
  if (B <= 0 || Hq <= 0 || R <= 0 || N <= 0) return 0;
  const int64_t rows = B * Hq * R * ((N + 511) / 512);  // one state per 512-key chunk
  return (size_t)(rows * 128 * 4 + (rows * 4 + 15) / 16 * 16);
}

}  // extern "C"

// mxattn_decode and its allocation-free variant: workspace == nullptr with
// use_scratch takes the split states from the library's static scratch
static int decode_impl(const mxattn_qtensor* q, const mxattn_qtensor* k, const mxattn_qtensor* v,
                       const mxattn_fwd_params* p, const int32_t* kv_len, void* out, const int64_t os[4], float* lse,
                       void* workspace, size_t ws_bytes, void* stream, bool use_scratch) {
  if (!q || !k || !v || !p || !os) return MXATTN_E_INVALID;
  if (q->role != MXATTN_ROLE_QK || k->role != MXATTN_ROLE_QK ||
      (v->role != MXATTN_ROLE_V && v->role != MXATTN_ROLE_VT))
    return MXATTN_E_INVALID;
  if (q->d != 128 || k->d != 128 || v->d != 128) return MXATTN_E_UNSUPPORTED;
  if (q->B != k->B || q->B != v->B || k->N != v->N || k->H != v->H || v->ndocs != 1) return MXATTN_E_INVALID;
  if (q->H <= 0 || k->H <= 0 || q->H % k->H != 0) return MXATTN_E_INVALID;
  if (v->n_padded != v_padded(v->N, 1, v->fmt.block)) return MXATTN_E_INVALID;  // the kernels read by it
  if (!p->causal || p->kv_tile != 128 || p->score_bias != nullptr || p->vkey != nullptr) return MXATTN_E_INVALID;
  if (!(p->sm_scale > 0.0f) || !isfinite(p->sm_scale)) return MXATTN_E_INVALID;
  if (p->exp_mode != MXATTN_EXP_EXACT) return p->exp_mode == MXATTN_EXP_MITCHELL || p->exp_mode == MXATTN_EXP_SCHRAUDOLPH
                                                 ? MXATTN_E_UNSUPPORTED : MXATTN_E_INVALID;
  const int64_t B = q->B, Hq = q->H, Hkv = k->H, R = q->N, N = k->N;
  if (R <= 0 || R > N || (Hq / Hkv) * R > 32) return MXATTN_E_UNSUPPORTED;
  const bool q4p8 = p->pmode == MXATTN_P_FP8_FIXED;
  if (!same_fmt(q->fmt, k->fmt)) return MXATTN_E_UNSUPPORTED;
  if (q4p8) {
    // QK4PV8: NVFP4 (or MXFP4) Q/K, an FP8 V (role V or VT), P = E4M3(448 P~)
    if (!(is_nvfp4(q->fmt) || is_mxfp4(q->fmt)) || !is_fp8v(v->fmt)) return MXATTN_E_UNSUPPORTED;
  } else {
    if (!is_mxfp4(q->fmt) || !is_mxfp4(v->fmt)) return MXATTN_E_UNSUPPORTED;
    if (p->pmode != MXATTN_P_DIRECT && p->pmode != MXATTN_P_PNQ && p->pmode != MXATTN_P_TWO_LEVEL)
      return p->pmode == MXATTN_P_NONE ? MXATTN_E_UNSUPPORTED : MXATTN_E_INVALID;
    int prc = check_fmt(&p->pfmt, MXATTN_ROLE_V);
    if (prc != MXATTN_OK) return prc;
    if (!is_mxfp4(p->pfmt)) return MXATTN_E_UNSUPPORTED;
  }
  if (N > (int64_t(1) << 24)) return MXATTN_E_UNSUPPORTED;
  if (B == 0) return MXATTN_OK;
  if (!q->codes || !q->scales || !k->codes || !k->scales || !v->codes || !v->scales || !out) return MXATTN_E_INVALID;
  if (!aligned16(q->codes) || !aligned16(k->codes) || !aligned16(v->codes) || !aligned16(q->scales) ||
      !aligned16(k->scales) || !aligned16(v->scales) || !aligned16(out))
    return MXATTN_E_ALIGN;
  if (os[3] != 1 || os[0] < 0 || os[1] < 0 || os[2] < 0) return MXATTN_E_INVALID;
  const size_t need = mxattn_decode_workspace_bytes(B, Hq, R, N);
  if (use_scratch) {
    if (need > DECODE_SCRATCH_BYTES) {
      snprintf(g_err, sizeof g_err, "mxattn_decode_noalloc: the split states need %zu bytes, the static scratch "
               "holds %zu", need, DECODE_SCRATCH_BYTES);
      return MXATTN_E_WORKSPACE;
    }
    hipError_t es = decode_scratch(&workspace);
    if (es != hipSuccess) return hip_fail(es, "mxattn_decode_noalloc scratch address");
    ws_bytes = DECODE_SCRATCH_BYTES;
  }
  if (workspace == nullptr || ws_bytes < need) return MXATTN_E_WORKSPACE;
  if (!aligned16(workspace)) return MXATTN_E_ALIGN;
  // grids: one workgroup per (request, KV head, 512-key chunk); four per merged row
  if (B * Hkv * ((N + 511) / 512) > 0x7FFFFFFF || B * Hq * R * 4 > 0x7FFFFFFF) return MXATTN_E_UNSUPPORTED;
  DecArgs a{};
  a.q = static_cast<const uint8_t*>(q->codes);
  a.qs = static_cast<const uint8_t*>(q->scales);
  a.k = static_cast<const uint8_t*>(k->codes);
  a.ks = static_cast<const uint8_t*>(k->scales);
  a.v = static_cast<const uint8_t*>(v->codes);
  a.vs = static_cast<const uint8_t*>(v->scales);
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.R = R;
  a.N = N;
  a.np = v->n_padded;
  a.kv_len = kv_len;
  a.vtiled = v->role == MXATTN_ROLE_VT ? 1 : 0;
  a.qk_fp4 = is_mxfp4(q->fmt) ? 1 : 0;
  a.lambda = (float)((double)p->sm_scale * 1.4426950408889634);
  a.sm_scale = p->sm_scale;
  a.prule = make_rule(&p->pfmt);
  a.nsplit = (N + 511) / 512;
  a.ws_o = static_cast<float*>(workspace);
  a.ws_lse = a.ws_o + B * Hq * R * a.nsplit * 128;
  a.out = out;
  a.oB = os[0];
  a.oH = os[1];
  a.oN = os[2];
  a.out_fp32 = p->out_fp32 ? 1 : 0;
  a.lse = lse;
  hipError_t e = forced_failure();
  if (e == hipSuccess) e = launch_decode(p->pmode, a, static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return MXATTN_E_UNSUPPORTED;
  if (e != hipSuccess) return hip_fail(e, use_scratch ? "mxattn_decode_noalloc launch" : "mxattn_decode launch");
  return MXATTN_OK;
}

extern "C" {

int mxattn_decode(const mxattn_qtensor* q, const mxattn_qtensor* k, const mxattn_qtensor* v,
                  const mxattn_fwd_params* p, const int32_t* kv_len, void* out, const int64_t os[4], float* lse,
                  void* workspace, size_t ws_bytes, void* stream) {
  return decode_impl(q, k, v, p, kv_len, out, os, lse, workspace, ws_bytes, stream, false);
}

int mxattn_decode_noalloc(const mxattn_qtensor* q, const mxattn_qtensor* k, const mxattn_qtensor* v,
                          const mxattn_fwd_params* p, const int32_t* kv_len, void* out, const int64_t os[4],
                          float* lse, void* stream) {
  return decode_impl(q, k, v, p, kv_len, out, os, lse, nullptr, 0, stream, true);
}

int mxattn_fwd_plan(const int32_t* cu_host, int ndocs, int64_t N, int causal, void* workspace, size_t ws_bytes,
                    void* stream) {
  if (cu_host == nullptr || ndocs <= 0 || N < 0) return MXATTN_E_INVALID;
  if (cu_host[0] != 0 || cu_host[ndocs] != N) return MXATTN_E_INVALID;
  for (int k = 0; k < ndocs; k++)
    if (cu_host[k + 1] < cu_host[k]) return MXATTN_E_INVALID;
  size_t need = plan_bytes(N, ndocs);
  if (workspace == nullptr || ws_bytes < need) return MXATTN_E_WORKSPACE;
  if (!aligned16(workspace)) return MXATTN_E_ALIGN;

  std::vector<uint8_t> buf(need, 0);
  PlanHeader* ph = reinterpret_cast<PlanHeader*>(buf.data());
  DocEntry* docs = reinterpret_cast<DocEntry*>(ph + 1);
  WorkItem* items = reinterpret_cast<WorkItem*>(docs + ndocs);
  const int64_t cap128 = plan_cap(N, ndocs, 128);
  WorkItem* items256 = items + cap128;
  int64_t v32 = 0, v16 = 0;
  struct Cand {
    int64_t cost;
    int32_t doc, qtile;
  };
  std::vector<Cand> cand, cand256;
  for (int k = 0; k < ndocs; k++) {
    int64_t L = cu_host[k + 1] - cu_host[k];
    docs[k].start = cu_host[k];
    docs[k].len = (int32_t)L;
    docs[k].voff32 = (int32_t)v32;
    docs[k].voff16 = (int32_t)v16;
    v32 += (L + 31) / 32 * 32;
    v16 += (L + 15) / 16 * 16;
    // cost = key tiles of 128 the query tile visits
    int64_t nkt = (L + 127) / 128;
    for (int64_t t = 0; t < nkt; t++) cand.push_back({causal ? t + 1 : nkt, k, (int32_t)t});
    int64_t nt2 = (L + 255) / 256;
    for (int64_t t = 0; t < nt2; t++) {
      int64_t c = causal ? std::min<int64_t>(nkt, 2 * t + 2) : nkt;
      cand256.push_back({c, k, (int32_t)t});
    }
  }
  // longest first (the key tiles an item visits); ties keep document order
  auto by_cost = [](const Cand& x, const Cand& y) { return x.cost > y.cost; };
  std::stable_sort(cand.begin(), cand.end(), by_cost);
  std::stable_sort(cand256.begin(), cand256.end(), by_cost);
  for (size_t i = 0; i < cand.size(); i++) items[i] = {cand[i].doc, cand[i].qtile};
  for (size_t i = 0; i < cand256.size(); i++) items256[i] = {cand256[i].doc, cand256[i].qtile};
  ph->n_items = (int32_t)cand.size();
  ph->ndocs = ndocs;
  ph->causal = causal ? 1 : 0;
  ph->magic = PLAN_MAGIC;
  ph->n_items256 = (int32_t)cand256.size();
  ph->cap128 = (int32_t)cap128;
  ph->n_tokens = (int32_t)N;
  hipError_t e = forced_failure();
  if (e == hipSuccess)
    e = hipMemcpyAsync(workspace, buf.data(), need, hipMemcpyHostToDevice, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "mxattn_fwd_plan copy");
  return MXATTN_OK;
}

int mxattn_fwd(const mxattn_qtensor* q, const mxattn_qtensor* k, const mxattn_qtensor* v,
               const mxattn_fwd_params* p, int ndocs, void* out, const int64_t os[4], float* lse,
               const void* workspace, size_t ws_bytes, void* stream) {
  if (!q || !k || !v || !p || !os) return MXATTN_E_INVALID;
  if (q->role != MXATTN_ROLE_QK || k->role != MXATTN_ROLE_QK || v->role != MXATTN_ROLE_V) return MXATTN_E_INVALID;
  if (q->d != 128 || k->d != 128 || v->d != 128) return MXATTN_E_UNSUPPORTED;
  if (q->B != k->B || q->B != v->B || q->N != k->N || q->N != v->N || k->H != v->H) return MXATTN_E_INVALID;
  if (q->H <= 0 || k->H <= 0 || q->H % k->H != 0) return MXATTN_E_INVALID;
  if (p->kv_tile != 128) return MXATTN_E_UNSUPPORTED;
  if (!(p->sm_scale > 0.0f) || !isfinite(p->sm_scale)) return MXATTN_E_INVALID;
  if (ndocs < 0) return MXATTN_E_INVALID;
  const bool docs = ndocs > 1 || (ndocs == 1 && workspace != nullptr);
  if (docs && q->B != 1) return MXATTN_E_INVALID;
  if ((docs ? ndocs : 1) != v->ndocs) return MXATTN_E_INVALID;
  if (!same_fmt(q->fmt, k->fmt)) return MXATTN_E_UNSUPPORTED;
  if (os[3] != 1 || os[0] < 0 || os[1] < 0 || os[2] < 0) return MXATTN_E_INVALID;

  // operand routes
  int qk, pv, psc = SCALE_E8M0, vsc = SCALE_E8M0;
  const int pm = p->pmode;
  const bool raw = is_bf16(q->fmt);
  if (raw != is_bf16(v->fmt) || raw != (pm == MXATTN_P_NONE)) {
    // the unquantized route takes Q, K, V in bf16 with P unquantized, nothing else
    if (pm != MXATTN_P_NONE && (pm < MXATTN_P_DIRECT || pm > MXATTN_P_FP8_FIXED)) return MXATTN_E_INVALID;
    return MXATTN_E_UNSUPPORTED;
  }
  if (raw) qk = QK_RAW;
  else if (is_mxfp4(q->fmt)) qk = QK_FP4;
  else if (is_nvfp4(q->fmt)) qk = QK_BF16;
  else return MXATTN_E_UNSUPPORTED;
  if (raw) {
    if (p->vkey != nullptr || p->exp_mode != MXATTN_EXP_EXACT) return MXATTN_E_UNSUPPORTED;
    pv = PV_RAW;
  } else if (pm == MXATTN_P_FP8_FIXED) {
    if (!is_fp8v(v->fmt)) return MXATTN_E_UNSUPPORTED;
    pv = PV_FP8;
    vsc = SCALE_E8M0;
  } else if (pm == MXATTN_P_DIRECT || pm == MXATTN_P_TWO_LEVEL || pm == MXATTN_P_PNQ) {
    int prc = check_fmt(&p->pfmt, MXATTN_ROLE_V);
    if (prc != MXATTN_OK) return prc;
    if (is_mxfp4(p->pfmt)) psc = SCALE_E8M0;
    else if (is_nvfp4(p->pfmt)) psc = SCALE_E4M3;
    else return MXATTN_E_UNSUPPORTED;
    if (is_mxfp4(v->fmt)) vsc = SCALE_E8M0;
    else if (is_nvfp4(v->fmt)) vsc = SCALE_E4M3;
    else return MXATTN_E_UNSUPPORTED;
    pv = (psc == SCALE_E8M0 && vsc == SCALE_E8M0) ? PV_FP4 : PV_BF16;
  } else {
    return MXATTN_E_INVALID;
  }
  // bit-level exponentials: the ping-pong kernel's routes (MXFP4 Q/K with an E8M0 V, or FP8 P)
  float exp_bias = 0.0f;
  if (p->exp_mode != MXATTN_EXP_EXACT) {
    const double ln2 = 0.69314718055994531;
    double delta;
    if (p->exp_mode == MXATTN_EXP_MITCHELL) delta = 0.5 * (log2(1.0 / ln2) - 1.0 / ln2 + 1.0);
    else if (p->exp_mode == MXATTN_EXP_SCHRAUDOLPH) delta = log2(1.0 / (2.0 * ln2 * ln2));
    else return MXATTN_E_INVALID;
    if (vsc != SCALE_E8M0 || (qk != QK_FP4 && pv != PV_FP8)) return MXATTN_E_UNSUPPORTED;
    exp_bias = (float)ldexp(127.0 - delta, 23);
  }

  const int64_t B = q->B, Hq = q->H, Hkv = k->H, N = q->N;
  if (B == 0 || N == 0) return MXATTN_OK;
  // the kernels address one head's K and V with 32-bit offsets
  if (N > (int64_t(1) << 24) || v->n_padded > (int64_t(1) << 24)) return MXATTN_E_UNSUPPORTED;
  if (!q->codes || !k->codes || !v->codes || !out) return MXATTN_E_INVALID;
  if (!raw && (!q->scales || !k->scales || !v->scales)) return MXATTN_E_INVALID;
  if (!aligned16(q->codes) || !aligned16(k->codes) || !aligned16(v->codes) || !aligned16(out))
    return MXATTN_E_ALIGN;
  if (!raw && (!aligned16(q->scales) || !aligned16(k->scales) || !aligned16(v->scales))) return MXATTN_E_ALIGN;
  const int esz = p->out_fp32 ? 4 : 2;
  if ((os[0] * esz) % 16 || (os[1] * esz) % 16 || (os[2] * esz) % 16) return MXATTN_E_ALIGN;
  if (docs) {
    if (workspace == nullptr || ws_bytes < plan_bytes(N, ndocs)) return MXATTN_E_WORKSPACE;
    if (!aligned16(workspace)) return MXATTN_E_ALIGN;
  }

  FwdArgs a;
  a.q = static_cast<const uint8_t*>(q->codes);
  a.qs = static_cast<const uint8_t*>(q->scales);
  a.k = static_cast<const uint8_t*>(k->codes);
  a.ks = static_cast<const uint8_t*>(k->scales);
  a.v = static_cast<const uint8_t*>(v->codes);
  a.vs = static_cast<const uint8_t*>(v->scales);
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.N = N;
  a.np = v->n_padded;
  a.lambda = (float)((double)p->sm_scale * 1.4426950408889634);
  a.sm_scale = p->sm_scale;
  a.causal = p->causal ? 1 : 0;
  a.prule = make_rule(&p->pfmt);
  a.out = out;
  a.oB = os[0];
  a.oH = os[1];
  a.oN = os[2];
  a.out_fp32 = p->out_fp32 ? 1 : 0;
  a.lse = lse;
  a.plan = docs ? static_cast<const PlanHeader*>(workspace) : nullptr;
  a.ndocs = docs ? ndocs : 0;
  a.bias = p->score_bias;
  if (a.bias != nullptr && !aligned16(a.bias)) return MXATTN_E_ALIGN;
  a.vk = nullptr;
  a.vks = nullptr;
  if (p->vkey != nullptr) {  // causally safe V scales: the per-key form of the same V
    const mxattn_qtensor* vk = p->vkey;
    if (!p->causal || vk->role != MXATTN_ROLE_VKEY) return MXATTN_E_INVALID;
    if (vk->B != v->B || vk->H != v->H || vk->N != v->N || vk->d != v->d || vk->n_padded != v->n_padded ||
        vk->ndocs != v->ndocs || vk->fmt.block != v->fmt.block)
      return MXATTN_E_INVALID;
    if (pv == PV_FP8 || vsc != SCALE_E8M0) return MXATTN_E_UNSUPPORTED;  // 4-bit V with E8M0/32 only
    if (!vk->codes || !vk->scales) return MXATTN_E_INVALID;
    if (!aligned16(vk->codes) || !aligned16(vk->scales)) return MXATTN_E_ALIGN;
    a.vk = static_cast<const uint8_t*>(vk->codes);
    a.vks = static_cast<const uint8_t*>(vk->scales);
  }
  a.exp_bits = p->exp_mode != MXATTN_EXP_EXACT ? 1 : 0;
  a.exp_bias = exp_bias;
  const int64_t nqt = (N + 127) / 128;
  a.grid = docs ? Hq * (nqt + ndocs) : B * Hq * nqt;
  if (a.grid > 0x7FFFFFFF) return MXATTN_E_UNSUPPORTED;
  hipError_t e = forced_failure();
  if (e == hipSuccess) e = launch_fwd(qk, pv, pm, psc, vsc, a, static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return MXATTN_E_UNSUPPORTED;
  if (e != hipSuccess) return hip_fail(e, "mxattn_fwd launch");
  return MXATTN_OK;
}

}  // extern "C"
