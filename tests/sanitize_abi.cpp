// Host-side argument validation of every libpa entry point, meant to be built
// with AddressSanitizer and UndefinedBehaviorSanitizer on the host code and
// run on a machine without a GPU (tests/test_host_sanitize.py does both).
//
// Device pointers here are stand-ins that are never dereferenced: every call
// either fails validation on the host or, when no GPU is visible, at its
// first HIP call.  Calls whose arguments are all valid are made only when no
// GPU is present.  Exit status: 0 when every expectation holds.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../include/pa.h"

static int g_failures = 0;
static bool g_gpu = false;

static void expect(const char* what, int got, int want) {
  const char* msg = pa_last_error();
  if (!msg || strlen(msg) == 0) {
    printf("FAIL %s: empty error message\n", what);
    ++g_failures;
  }
  if (got != want) {
    printf("FAIL %s: status %d, expected %d (%s)\n", what, got, want, msg ? msg : "");
    ++g_failures;
  }
}
// A call with valid arguments: without a GPU it must fail at the HIP layer.
static void expect_valid(const char* what, int got) {
  if (got != PA_ERR_HIP && got != PA_OK) {
    printf("FAIL %s: valid arguments refused with %d (%s)\n", what, got, pa_last_error());
    ++g_failures;
  }
}

alignas(256) static char g_fake[1 << 12];  // stands in for device buffers; never read
#define P(off) (static_cast<void*>(g_fake + (off)))

int main() {
  int n = 0;
  g_gpu = hipGetDeviceCount(&n) == hipSuccess && n > 0;
  const void* q = P(0);
  void* out = P(256);
  const void* kc = P(512);
  const void* vc = P(768);
  const int32_t* bt = static_cast<const int32_t*>(P(1024));
  const int32_t* cl = static_cast<const int32_t*>(P(1280));
  const int32_t* qs = static_cast<const int32_t*>(P(1536));
  const float* ks = static_cast<const float*>(P(1792));
  const float* vs = static_cast<const float*>(P(2048));
  const int64_t* sm = static_cast<const int64_t*>(P(2304));
  void* ws = P(2560);

  // ---- sizes and defaults (pure host functions) --------------------------
  if (pa_version() < 100) { printf("FAIL version\n"); ++g_failures; }
  if (pa_default_split_tokens(1, 16, 8, 128, PA_BF16) != 512) { printf("FAIL split\n"); ++g_failures; }
  if (pa_workspace_size(-1, 1, 16, 8, 128, 512, PA_BF16, 0) != 0) { printf("FAIL ws neg\n"); ++g_failures; }
  if (pa_workspace_size(64, 1, 16, 8, 128, 513, PA_BF16, 0) == 0) { printf("FAIL ws >0\n"); ++g_failures; }
  if (pa_workspace_size(INT_MAX, 1, 16, 8, 128, INT_MAX, PA_BF16, 16) != 0) {
    printf("FAIL ws overflow accepted\n");
    ++g_failures;
  }
  if (pa_plan_size(INT_MAX, 1, 16, 8, 128, 512, PA_BF16, 0) != 0) { printf("FAIL plan size\n"); ++g_failures; }
  if (pa_prefill_plan_size(INT_MAX, INT_MAX, 16, 8) != 0) { printf("FAIL prefill plan size\n"); ++g_failures; }
  if (pa_prefill_plan_size(4, 100, 16, 8) == 0) { printf("FAIL prefill plan size 0\n"); ++g_failures; }
  unsigned flags = 123;
  expect("check status (release)", pa_device_check_status(&flags, 1), PA_ERR_UNSUPPORTED);
  if (flags != 0) { printf("FAIL flags not cleared\n"); ++g_failures; }
  expect("check status null", pa_device_check_status(nullptr, 0), PA_ERR_INVALID_ARG);

  // ---- cache writes ------------------------------------------------------
  expect("cache: null", pa_reshape_and_cache(nullptr, kc, P(0), P(0), sm, 4, 8, 128, 64, 16, PA_BF16, nullptr), PA_ERR_INVALID_ARG);
  expect("cache: head_dim", pa_reshape_and_cache(q, kc, P(0), P(0), sm, 4, 8, 96, 64, 16, PA_BF16, nullptr), PA_ERR_UNSUPPORTED);
  expect("cache: block", pa_reshape_and_cache(q, kc, P(0), P(0), sm, 4, 8, 128, 64, 32, PA_BF16, nullptr), PA_ERR_UNSUPPORTED);
  expect("cache: dtype", pa_reshape_and_cache(q, kc, P(0), P(0), sm, 4, 8, 128, 64, 16, 7, nullptr), PA_ERR_INVALID_ARG);
  expect("cache: misaligned", pa_reshape_and_cache(P(1), kc, P(0), P(0), sm, 4, 8, 128, 64, 16, PA_BF16, nullptr), PA_ERR_INVALID_ARG);
  expect("cache: neg tokens", pa_reshape_and_cache(q, kc, P(0), P(0), sm, -1, 8, 128, 64, 16, PA_BF16, nullptr), PA_ERR_INVALID_ARG);
  expect("cache: huge", pa_reshape_and_cache(q, kc, P(0), P(0), sm, INT_MAX, INT_MAX, 128, 64, 16, PA_F32, nullptr), PA_ERR_UNSUPPORTED);
  expect("quant: in dtype", pa_reshape_and_cache_quant(q, kc, (int8_t*)P(0), (int8_t*)P(0), (float*)P(0), (float*)P(0), sm, 4, 8, 128, 64, 16, PA_INT8, nullptr), PA_ERR_INVALID_ARG);
  expect("quant: pool", pa_reshape_and_cache_quant(q, kc, (int8_t*)P(0), (int8_t*)P(0), (float*)P(0), (float*)P(0), sm, 4, 8, 128, INT_MAX, 16, PA_BF16, nullptr), PA_ERR_UNSUPPORTED);
  expect("quant: null", pa_reshape_and_cache_quant(q, kc, nullptr, (int8_t*)P(0), (float*)P(0), (float*)P(0), sm, 4, 8, 128, 64, 16, PA_BF16, nullptr), PA_ERR_INVALID_ARG);

  // ---- decode ------------------------------------------------------------
  auto dec = [&](const void* o, int N, int hq, int hkv, int D, int bs, int nb, int mb, int mcl,
                 float sc, int qd, int kd, int st, void* w, size_t wb, const float* k_s) {
    return pa_decode(const_cast<void*>(o), q, kc, vc, k_s, vs, bt, cl, N, hq, hkv, D, bs, nb, mb,
                     mcl, sc, qd, kd, st, w, wb, nullptr);
  };
  expect("decode: group", dec(out, 4, 12, 8, 128, 16, 64, 32, 512, 0.1f, PA_BF16, PA_BF16, 0, ws, 1 << 20, ks), PA_ERR_INVALID_ARG);
  expect("decode: head_dim", dec(out, 4, 16, 8, 80, 16, 64, 32, 512, 0.1f, PA_BF16, PA_BF16, 0, ws, 1 << 20, ks), PA_ERR_UNSUPPORTED);
  expect("decode: block", dec(out, 4, 16, 8, 128, 8, 64, 32, 512, 0.1f, PA_BF16, PA_BF16, 0, ws, 1 << 20, ks), PA_ERR_UNSUPPORTED);
  expect("decode: triple", dec(out, 4, 16, 8, 128, 16, 64, 32, 512, 0.1f, PA_F32, PA_BF16, 0, ws, 1 << 20, ks), PA_ERR_UNSUPPORTED);
  expect("decode: q int8", dec(out, 4, 16, 8, 128, 16, 64, 32, 512, 0.1f, PA_INT8, PA_INT8, 0, ws, 1 << 20, ks), PA_ERR_INVALID_ARG);
  expect("decode: scale nan", dec(out, 4, 16, 8, 128, 16, 64, 32, 512, NAN, PA_BF16, PA_BF16, 0, ws, 1 << 20, ks), PA_ERR_INVALID_ARG);
  expect("decode: scale inf", dec(out, 4, 16, 8, 128, 16, 64, 32, 512, INFINITY, PA_BF16, PA_BF16, 0, ws, 1 << 20, ks), PA_ERR_INVALID_ARG);
  expect("decode: split", dec(out, 4, 16, 8, 128, 16, 64, 32, 512, 0.1f, PA_BF16, PA_BF16, 24, ws, 1 << 20, ks), PA_ERR_INVALID_ARG);
  expect("decode: split big", dec(out, 4, 16, 8, 128, 16, 64, 32, 512, 0.1f, PA_BF16, PA_BF16, 8192, ws, 1 << 20, ks), PA_ERR_INVALID_ARG);
  expect("decode: len > table", dec(out, 4, 16, 8, 128, 16, 64, 32, 513, 0.1f, PA_BF16, PA_BF16, 0, ws, 1 << 20, ks), PA_ERR_INVALID_ARG);
  expect("decode: null out", dec(nullptr, 4, 16, 8, 128, 16, 64, 32, 512, 0.1f, PA_BF16, PA_BF16, 0, ws, 1 << 20, ks), PA_ERR_INVALID_ARG);
  expect("decode: misaligned out", dec(P(2), 4, 16, 8, 128, 16, 64, 32, 512, 0.1f, PA_BF16, PA_BF16, 0, ws, 1 << 20, ks), PA_ERR_INVALID_ARG);
  expect("decode: int8 no scales", dec(out, 4, 12, 2, 128, 16, 64, 32, 512, 0.1f, PA_BF16, PA_INT8, 0, ws, 1 << 20, nullptr), PA_ERR_INVALID_ARG);
  expect("decode: workspace", dec(out, 4, 16, 8, 128, 16, 64, 32, 512, 0.1f, PA_BF16, PA_BF16, 64, nullptr, 0, ks), PA_ERR_WORKSPACE);
  expect("decode: workspace small", dec(out, 4, 16, 8, 128, 16, 64, 32, 512, 0.1f, PA_BF16, PA_BF16, 64, ws, 16, ks), PA_ERR_WORKSPACE);
  expect("decode: workspace misaligned", dec(out, 4, 16, 8, 128, 16, 64, 32, 512, 0.1f, PA_BF16, PA_BF16, 64, P(2564), 1 << 20, ks), PA_ERR_WORKSPACE);
  expect("decode: grid", dec(out, INT_MAX, 16, 8, 128, 16, 64, 1 << 20, 1 << 24, 0.1f, PA_BF16, PA_BF16, 16, ws, 1 << 20, ks), PA_ERR_UNSUPPORTED);
  expect("decode: neg seqs", dec(out, -3, 16, 8, 128, 16, 64, 32, 512, 0.1f, PA_BF16, PA_BF16, 0, ws, 1 << 20, ks), PA_ERR_INVALID_ARG);
  expect("decode: zero kv heads", dec(out, 4, 16, 0, 128, 16, 64, 32, 512, 0.1f, PA_BF16, PA_BF16, 0, ws, 1 << 20, ks), PA_ERR_INVALID_ARG);
  expect("decode: group 9", dec(out, 4, 18, 2, 128, 16, 64, 32, 512, 0.1f, PA_BF16, PA_BF16, 0, ws, 1 << 20, ks), PA_ERR_UNSUPPORTED);
  expect("noalloc: oversize",
         pa_decode_noalloc(out, q, kc, vc, ks, vs, bt, cl, 64, 16, 8, 64, 16, 64, 2048, 32768, 0.1f,
                           PA_F32, PA_F32, 128, nullptr),
         PA_ERR_WORKSPACE);
  expect("append: int8",
         pa_decode_append(out, q, q, q, P(0), P(0), sm, bt, cl, 4, 12, 2, 128, 16, 64, 32, 512, 0.1f,
                          PA_BF16, PA_INT8, 0, ws, 1 << 20, nullptr),
         PA_ERR_UNSUPPORTED);
  expect("append: null key",
         pa_decode_append(out, q, nullptr, q, P(0), P(0), sm, bt, cl, 4, 16, 8, 128, 16, 64, 32, 512, 0.1f,
                          PA_BF16, PA_BF16, 0, ws, 1 << 20, nullptr),
         PA_ERR_INVALID_ARG);

  // ---- verify, varlen, prefill -------------------------------------------
  expect("verify: head_dim",
         pa_verify(out, q, kc, vc, ks, vs, bt, cl, 4, 5, 16, 8, 96, 16, 64, 32, 512, 0.1f, PA_BF16,
                   PA_BF16, 0, ws, 1 << 20, nullptr),
         PA_ERR_UNSUPPORTED);
  expect("verify: fp32",
         pa_verify(out, q, kc, vc, ks, vs, bt, cl, 4, 5, 16, 8, 128, 16, 64, 32, 512, 0.1f, PA_F32,
                   PA_F32, 0, ws, 1 << 20, nullptr),
         PA_ERR_UNSUPPORTED);
  expect("verify: zero tokens",
         pa_verify(out, q, kc, vc, ks, vs, bt, cl, 4, 0, 16, 8, 128, 16, 64, 32, 512, 0.1f, PA_BF16,
                   PA_BF16, 0, ws, 1 << 20, nullptr),
         PA_ERR_INVALID_ARG);
  expect("verify: huge rows",
         pa_verify(out, q, kc, vc, ks, vs, bt, cl, 1 << 20, 1 << 20, 16, 8, 128, 16, 64, 32, 512, 0.1f,
                   PA_BF16, PA_BF16, 0, ws, 1 << 20, nullptr),
         PA_ERR_UNSUPPORTED);
  expect("varlen: total",
         pa_verify_varlen(out, q, kc, vc, ks, vs, bt, cl, qs, 4, 21, 5, 16, 8, 128, 16, 64, 32, 512,
                          0.1f, PA_BF16, PA_BF16, 0, ws, 1 << 20, nullptr),
         PA_ERR_INVALID_ARG);
  expect("varlen: null offsets",
         pa_verify_varlen(out, q, kc, vc, ks, vs, bt, cl, nullptr, 4, 20, 5, 16, 8, 128, 16, 64, 32,
                          512, 0.1f, PA_BF16, PA_BF16, 0, ws, 1 << 20, nullptr),
         PA_ERR_INVALID_ARG);
  expect("prefill: dtype",
         pa_prefill(out, q, kc, vc, ks, vs, bt, cl, qs, 4, 100, 40, 16, 8, 128, 16, 64, 32, 512, 0.1f,
                    PA_F32, PA_F32, nullptr),
         PA_ERR_UNSUPPORTED);
  expect("prefill: total",
         pa_prefill(out, q, kc, vc, ks, vs, bt, cl, qs, 4, 161, 40, 16, 8, 128, 16, 64, 32, 512, 0.1f,
                    PA_BF16, PA_BF16, nullptr),
         PA_ERR_INVALID_ARG);
  expect("prefill: huge",
         pa_prefill(out, q, kc, vc, ks, vs, bt, cl, qs, INT_MAX, 0, INT_MAX, 16, 8, 128, 16, 64, 32,
                    512, 0.1f, PA_BF16, PA_BF16, nullptr),
         PA_ERR_UNSUPPORTED);

  // ---- plans -------------------------------------------------------------
  expect("plan: null buffer",
         pa_plan(bt, cl, 4, 1, 16, 8, 128, 32, 512, PA_BF16, 0, nullptr, 0, nullptr), PA_ERR_INVALID_ARG);
  expect("plan: small buffer",
         pa_plan(bt, cl, 4, 1, 16, 8, 128, 32, 512, PA_BF16, 0, ws, 8, nullptr), PA_ERR_INVALID_ARG);
  expect("planned: null plan",
         pa_decode_planned(out, q, kc, vc, ks, vs, bt, cl, 4, 16, 8, 128, 16, 64, 32, 512, 0.1f,
                           PA_BF16, PA_BF16, 0, ws, 1 << 20, nullptr, 0, nullptr),
         PA_ERR_INVALID_ARG);
  expect("planned: small plan",
         pa_verify_planned(out, q, kc, vc, ks, vs, bt, cl, 4, 5, 16, 8, 128, 16, 64, 32, 512, 0.1f,
                           PA_BF16, PA_BF16, 0, ws, 1 << 20, ws, 4, nullptr),
         PA_ERR_INVALID_ARG);
  expect("prefill plan: sizes",
         pa_prefill_plan(cl, qs, 4, 100, 40, 16, 7, 32, ws, 1 << 12, nullptr), PA_ERR_INVALID_ARG);
  expect("prefill planned: null",
         pa_prefill_planned(out, q, kc, vc, ks, vs, bt, cl, qs, 4, 100, 40, 16, 8, 128, 16, 64, 32, 512,
                            0.1f, PA_BF16, PA_BF16, nullptr, 0, nullptr),
         PA_ERR_INVALID_ARG);

  // ---- valid arguments (no GPU: fail at the HIP layer) -------------------
  if (!g_gpu) {
    expect_valid("valid decode", dec(out, 4, 16, 8, 128, 16, 64, 32, 512, 0.1f, PA_BF16, PA_BF16, 0, ws, 1 << 20, ks));
    expect_valid("valid verify", pa_verify(out, q, kc, vc, ks, vs, bt, cl, 4, 5, 12, 2, 128, 16, 64, 32, 512, 0.1f, PA_BF16, PA_INT8, 0, ws, 1 << 20, nullptr));
    expect_valid("valid verify on prefill", pa_verify(out, q, kc, vc, ks, vs, bt, cl, 4, 9, 12, 2, 128, 16, 64, 32, 512, 0.1f, PA_BF16, PA_BF16, 0, ws, 1 << 20, nullptr));
    expect_valid("valid noalloc", pa_decode_noalloc(out, q, kc, vc, ks, vs, bt, cl, 4, 16, 8, 128, 16, 64, 32, 512, 0.1f, PA_BF16, PA_BF16, 64, nullptr));
    expect_valid("valid cache", pa_reshape_and_cache(q, kc, P(0), P(0), sm, 4, 8, 128, 64, 16, PA_BF16, nullptr));
    expect_valid("valid plan", pa_plan(bt, cl, 4, 1, 16, 8, 128, 32, 512, PA_BF16, 0, ws, 1 << 12, nullptr));
    expect_valid("valid prefill", pa_prefill(out, q, kc, vc, ks, vs, bt, cl, qs, 4, 100, 40, 16, 8, 128, 16, 64, 32, 512, 0.1f, PA_BF16, PA_BF16, nullptr));
  }
  printf("%s: %d failure(s)%s\n", g_failures ? "FAILED" : "OK", g_failures,
         g_gpu ? " (valid-argument calls skipped: a GPU is visible)" : "");
  return g_failures ? 1 : 0;
}
