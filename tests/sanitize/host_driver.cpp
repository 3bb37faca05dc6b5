// Sanitizer harness of the host code of libmxattn (host.cpp) on the CPU: every entry
// point of include/mxattn.h with well-formed and malformed arguments, the plan
// builder over many documents, the forced launch failures and the status texts.  The
// device side is replaced by tests/sanitize/host_stubs.cpp; device pointers are fake
// and never dereferenced by the host code.  Built by tests/test_sanitizers.py with
// -fsanitize=address,undefined; a sanitizer report or a failed check exits non-zero.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "mxattn.h"

extern int g_launches;
static int fails = 0;
#define CHECK(c)                                          \
  do {                                                    \
    if (!(c)) {                                           \
      fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      fails++;                                            \
    }                                                     \
  } while (0)

static void* fake(uint64_t off) { return reinterpret_cast<void*>(uintptr_t(0x7F0000000000ull + off)); }

static mxattn_qfmt fmt(int elem, int scale, int block, int rule, float qmax) {
  mxattn_qfmt f;
  f.elem = elem;
  f.scale = scale;
  f.block = block;
  f.rule = rule;
  f.qmax = qmax;
  return f;
}

int main() {
  const mxattn_qfmt mx = fmt(MXATTN_ELEM_E2M1, MXATTN_SCALE_E8M0, 32, MXATTN_RULE_OCP, 0.0f);
  const mxattn_qfmt uos = fmt(MXATTN_ELEM_E2M1, MXATTN_SCALE_E8M0, 32, MXATTN_RULE_CEIL, 7.25f);
  const mxattn_qfmt nv = fmt(MXATTN_ELEM_E2M1, MXATTN_SCALE_E4M3, 16, MXATTN_RULE_OCP, 0.0f);
  const mxattn_qfmt f8 = fmt(MXATTN_ELEM_E4M3, MXATTN_SCALE_E8M0, 32, MXATTN_RULE_CEIL, 448.0f);
  const mxattn_qfmt bf = fmt(MXATTN_ELEM_BF16, MXATTN_SCALE_NONE, 0, MXATTN_RULE_OCP, 0.0f);
  const mxattn_qfmt* fmts[] = {&mx, &uos, &nv, &f8, &bf};
  for (int s = -7; s <= 1; s++) CHECK(mxattn_status_str(s) != nullptr);
  CHECK(mxattn_abi_version() == MXATTN_ABI_VERSION);

  // sizes and quantization, every role and format, with and without documents
  const int64_t B = 1, H = 2, N = 1000;
  const int64_t xs[4] = {H * N * 128, N * 128, 128, 1};
  for (const mxattn_qfmt* f : fmts) {
    for (int role = MXATTN_ROLE_QK; role <= MXATTN_ROLE_VT; role++) {
      for (int nd : {0, 1, 7}) {
        size_t cb = 0, sb = 0;
        int64_t np = 0;
        int rc = mxattn_qtensor_bytes(f, role, B, H, N, 128, nd, &cb, &sb, &np);
        if (rc != MXATTN_OK) continue;
        mxattn_qtensor t;
        memset(&t, 0, sizeof t);
        t.codes = fake(0x1000000);
        t.scales = fake(0x2000000);
        rc = mxattn_quantize(fake(0), xs, B, H, N, 128, role, f, nd > 1 ? static_cast<const int32_t*>(fake(0x3000000)) : nullptr,
                             nd, &t, nullptr);
        CHECK(rc == MXATTN_OK || rc == MXATTN_E_INVALID || rc == MXATTN_E_UNSUPPORTED);
        if (rc == MXATTN_OK) CHECK(t.n_padded == np && t.B == B && t.N == N);
      }
    }
  }
  // malformed quantize calls
  {
    mxattn_qtensor t;
    memset(&t, 0, sizeof t);
    t.codes = fake(0x1000000);
    t.scales = fake(0x2000000);
    const int64_t bad[4] = {1, 1, 1, 2};
    CHECK(mxattn_quantize(fake(0), bad, B, H, N, 128, MXATTN_ROLE_QK, &mx, nullptr, 0, &t, nullptr) == MXATTN_E_INVALID);
    CHECK(mxattn_quantize(fake(2), xs, B, H, N, 128, MXATTN_ROLE_QK, &mx, nullptr, 0, &t, nullptr) == MXATTN_E_ALIGN);
    CHECK(mxattn_quantize(fake(0), xs, B, H, N, 64, MXATTN_ROLE_QK, &mx, nullptr, 0, &t, nullptr) == MXATTN_E_UNSUPPORTED);
    CHECK(mxattn_quantize(fake(0), xs, B, H, N, 128, MXATTN_ROLE_QK, &mx, nullptr, 0, nullptr, nullptr) == MXATTN_E_INVALID);
    CHECK(mxattn_quantize(fake(0), xs, 1 << 20, 8, 128, 128, MXATTN_ROLE_QK, &mx, nullptr, 0, &t, nullptr) ==
          MXATTN_E_UNSUPPORTED);
  }
  // pre-processing calls
  {
    mxattn_qtensor t;
    memset(&t, 0, sizeof t);
    t.codes = fake(0x1000000);
    t.scales = fake(0x2000000);
    mxattn_preproc pre;
    pre.mean = static_cast<const float*>(fake(0x4000000));
    pre.hadamard = 1;
    CHECK(mxattn_channel_mean(fake(0), xs, B, H, N, 128, nullptr, 0, static_cast<float*>(fake(0x4000000)), nullptr) == MXATTN_OK);
    CHECK(mxattn_quantize_pre(fake(0), xs, B, H, N, 128, MXATTN_ROLE_QK, &mx, &pre, nullptr, 0, &t, nullptr) == MXATTN_OK);
    pre.hadamard = 2;
    CHECK(mxattn_quantize_pre(fake(0), xs, B, H, N, 128, MXATTN_ROLE_QK, &mx, &pre, nullptr, 0, &t, nullptr) == MXATTN_E_INVALID);
    CHECK(mxattn_center_comp(static_cast<const float*>(fake(0x4000000)), fake(0), xs, static_cast<const float*>(fake(0x5000000)), B, 4, 2, N, 128,
                             nullptr, 0, static_cast<float*>(fake(0x6000000)), nullptr) == MXATTN_OK);
  }

  // plans over many documents (lengths 0..1200), built into a host buffer by the
  // stand-in copy, then forwards that read them
  std::vector<int32_t> cu(1, 0);
  uint32_t r = 12345;
  while (cu.size() < 301) {
    r = r * 1103515245u + 12345u;
    cu.push_back(cu.back() + (int32_t)((r >> 8) % 1201));
  }
  const int nd = 300;
  const int64_t Nd = cu.back();
  for (int causal = 0; causal < 2; causal++) {
    const size_t wb = mxattn_fwd_workspace_bytes(Nd, nd);
    std::vector<unsigned char> ws(wb + 16);
    void* w = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(ws.data()) + 15) & ~uintptr_t(15));
    CHECK(mxattn_fwd_plan(cu.data(), nd, Nd, causal, w, wb, nullptr) == MXATTN_OK);
    CHECK(mxattn_fwd_plan(cu.data(), nd, Nd, causal, w, wb - 1, nullptr) == MXATTN_E_WORKSPACE);
    CHECK(mxattn_fwd_plan(cu.data(), nd, Nd + 1, causal, w, wb, nullptr) == MXATTN_E_INVALID);
    mxattn_qtensor q, k, v;
    memset(&q, 0, sizeof q);
    q.codes = fake(0x1000000);
    q.scales = fake(0x2000000);
    q.fmt = uos;
    q.role = MXATTN_ROLE_QK;
    q.ndocs = 1;
    q.B = 1;
    q.H = 4;
    q.N = Nd;
    q.d = 128;
    q.n_padded = Nd;
    k = q;
    k.H = 2;
    v = k;
    v.role = MXATTN_ROLE_V;
    v.ndocs = nd;
    v.n_padded = (Nd + (int64_t)nd * 31 + 127) / 128 * 128;
    mxattn_fwd_params p;
    memset(&p, 0, sizeof p);
    p.pmode = MXATTN_P_PNQ;
    p.pfmt = uos;
    p.causal = causal;
    p.sm_scale = 0.08838834764f;
    p.kv_tile = 128;
    p.out_fp32 = 1;
    const int64_t os[4] = {4 * Nd * 128, Nd * 128, 128, 1};
    const int before = g_launches;
    CHECK(mxattn_fwd(&q, &k, &v, &p, nd, fake(0x7000000), os, nullptr, w, wb, nullptr) == MXATTN_OK);
    CHECK(g_launches == before + 1);
    CHECK(mxattn_fwd(&q, &k, &v, &p, nd, fake(0x7000000), os, nullptr, w, wb - 1, nullptr) == MXATTN_E_WORKSPACE);
    // every P mode and format against every V format
    for (int pm = MXATTN_P_NONE; pm <= MXATTN_P_FP8_FIXED + 1; pm++)
      for (const mxattn_qfmt* pf : fmts)
        for (const mxattn_qfmt* vf : fmts) {
          p.pmode = pm;
          p.pfmt = *pf;
          v.fmt = *vf;
          const int rc = mxattn_fwd(&q, &k, &v, &p, nd, fake(0x7000000), os, nullptr, w, wb, nullptr);
          CHECK(rc == MXATTN_OK || rc == MXATTN_E_INVALID || rc == MXATTN_E_UNSUPPORTED);
        }
    // a forced launch failure reports the call
    p.pmode = MXATTN_P_PNQ;
    p.pfmt = uos;
    v.fmt = uos;
    mxattn_debug_fail_launches(1);
    CHECK(mxattn_fwd(&q, &k, &v, &p, nd, fake(0x7000000), os, nullptr, w, wb, nullptr) == MXATTN_E_HIP);
    CHECK(strstr(mxattn_last_error(), "mxattn_fwd launch") != nullptr);
  }

  // decode, with a workspace and allocation-free
  {
    mxattn_qtensor q, k, v;
    memset(&q, 0, sizeof q);
    q.codes = fake(0x1000000);
    q.scales = fake(0x2000000);
    q.fmt = mx;
    q.role = MXATTN_ROLE_QK;
    q.ndocs = 1;
    q.B = 4;
    q.H = 32;
    q.N = 1;
    q.d = 128;
    q.n_padded = 1;
    k = q;
    k.H = 8;
    k.N = 40000;
    k.n_padded = 40000;
    v = k;
    v.role = MXATTN_ROLE_VT;
    v.n_padded = (40000 + 127) / 128 * 128;
    mxattn_fwd_params p;
    memset(&p, 0, sizeof p);
    p.pmode = MXATTN_P_TWO_LEVEL;
    p.pfmt = mx;
    p.causal = 1;
    p.sm_scale = 0.08838834764f;
    p.kv_tile = 128;
    p.out_fp32 = 1;
    const int64_t os[4] = {32 * 128, 128, 128, 1};
    const size_t wb = mxattn_decode_workspace_bytes(4, 32, 1, 40000);
    CHECK(mxattn_decode(&q, &k, &v, &p, nullptr, fake(0x7000000), os, nullptr, fake(0x8000000), wb, nullptr) == MXATTN_OK);
    CHECK(mxattn_decode(&q, &k, &v, &p, nullptr, fake(0x7000000), os, nullptr, fake(0x8000000), wb - 1, nullptr) ==
          MXATTN_E_WORKSPACE);
    CHECK(mxattn_decode_noalloc(&q, &k, &v, &p, nullptr, fake(0x7000000), os, nullptr, nullptr) == MXATTN_OK);
    k.N = v.N = 512 * 509;
    v.n_padded = k.N;
    CHECK(mxattn_decode_noalloc(&q, &k, &v, &p, nullptr, fake(0x7000000), os, nullptr, nullptr) == MXATTN_E_WORKSPACE);
    CHECK(strstr(mxattn_last_error(), "static scratch") != nullptr);
  }
  if (fails) {
    fprintf(stderr, "%d checks failed\n", fails);
    return 1;
  }
  printf("host sanitizer harness done (%d launches)\n", g_launches);
  return 0;
}
