// Host-only driver of the C-ABI validation layer (fa2_api.cpp), built with
// AddressSanitizer and UndefinedBehaviorSanitizer.  The kernel launchers are
// stubs that record the call: valid arguments must reach exactly one
// launcher, invalid ones must be rejected with their code before any launch.
// Exit status 0 when every check holds.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>

#include "fa2.h"
#include "fa2_internal.h"

namespace {
int g_launches = 0;
hipError_t g_result = hipSuccess;
alignas(256) float g_scratch[64];
int g_cur_device = 0;         // what hipGetDevice reports
int g_stream_device = 0;      // what hipStreamGetDevice reports for any stream
hipError_t g_query = hipSuccess;
}  // namespace

hipError_t hipGetDevice(int *device) {
  *device = g_cur_device;
  return g_query;
}
hipError_t hipStreamGetDevice(hipStream_t, hipDevice_t *device) {
  *device = g_stream_device;
  return g_query;
}

namespace fa2 {
FwdArgs g_last_fwd;  // what the last bf16 forward launch was given
hipError_t launch_fwd_bf16(const FwdArgs &a, bool, hipStream_t) {
  ++g_launches;
  g_last_fwd = a;
  if (a.n_splits > 1 && (!a.o_part || !a.lse_part)) return hipErrorInvalidValue;
  return g_result;
}
hipError_t launch_bwd_bf16(const BwdArgs &, bool, hipStream_t) { ++g_launches; return g_result; }
hipError_t launch_fwd_fp32(const FwdArgs &, hipStream_t) { ++g_launches; return g_result; }
hipError_t launch_quantize_fp8(const QuantArgs &, hipStream_t) { ++g_launches; return g_result; }
hipError_t launch_fwd_fp8(const Fp8Args &, bool, hipStream_t) { ++g_launches; return g_result; }
hipError_t fwd_scratch(float **ptr) { *ptr = g_scratch; return hipSuccess; }
}  // namespace fa2

static int g_fail = 0;
#define EXPECT(expr, want)                                                    \
  do {                                                                        \
    const int before_ = g_launches;                                           \
    const int got_ = (expr);                                                  \
    const int launched_ = g_launches - before_;                               \
    if (got_ != (want) || launched_ != ((want) == FA2_OK ? 1 : 0)) {          \
      std::printf("FAIL line %d: %s -> %d (want %d), launches %d\n", __LINE__, \
                  #expr, got_, (want), launched_);                            \
      ++g_fail;                                                               \
    }                                                                         \
  } while (0)

// fake, never dereferenced device addresses, 64 MiB apart
static void *P(int i) { return reinterpret_cast<void *>(uintptr_t(0x10000000) + uintptr_t(i) * (64u << 20)); }
// the same, 16 GiB apart (calls whose tensors exceed 64 MiB)
static void *FAR(int i) { return reinterpret_cast<void *>((uintptr_t(1) << 40) + uintptr_t(i) * (uintptr_t(1) << 34)); }
static float *F(int i) { return static_cast<float *>(P(i)); }
static void *off(void *p, int bytes) { return static_cast<char *>(p) + bytes; }

int main() {
  const float nan = std::numeric_limits<float>::quiet_NaN();
  const float inf = std::numeric_limits<float>::infinity();
  // forward entry points with the plain signature
  typedef int (*fwd_fn)(const void *, const void *, const void *, void *, float *, int, int,
                        int, int, float, int, void *);
  fwd_fn fwds[2] = {fa2_fwd, reinterpret_cast<fwd_fn>(fa2_fwd_o32)};
  for (fwd_fn f : fwds) {
    EXPECT(f(P(0), P(1), P(2), P(3), F(4), 1, 2, 64, 64, 0.125f, 0, nullptr), FA2_OK);
    EXPECT(f(P(0), P(1), P(2), P(3), nullptr, 2, 3, 1000, 128, 0.1f, 1, nullptr), FA2_OK);
    EXPECT(f(nullptr, P(1), P(2), P(3), F(4), 1, 2, 64, 64, 0.125f, 0, nullptr), FA2_ERR_NULL);
    EXPECT(f(P(0), P(1), P(2), nullptr, F(4), 1, 2, 64, 64, 0.125f, 0, nullptr), FA2_ERR_NULL);
    EXPECT(f(P(0), P(1), P(2), P(3), F(4), 0, 2, 64, 64, 0.125f, 0, nullptr), FA2_ERR_SHAPE);
    EXPECT(f(P(0), P(1), P(2), P(3), F(4), 1, -2, 64, 64, 0.125f, 0, nullptr), FA2_ERR_SHAPE);
    EXPECT(f(P(0), P(1), P(2), P(3), F(4), 1, 2, 1 << 30, 128, 0.125f, 0, nullptr), FA2_ERR_SHAPE);
    EXPECT(f(P(0), P(1), P(2), P(3), F(4), 1 << 16, 1 << 16, 1, 64, 0.125f, 0, nullptr), FA2_ERR_SHAPE);
    EXPECT(f(P(0), P(1), P(2), P(3), F(4), INT32_MAX, INT32_MAX, INT32_MAX, 128, 0.1f, 0, nullptr),
           FA2_ERR_SHAPE);
    EXPECT(f(P(0), P(1), P(2), P(3), F(4), 1, 2, 64, 96, 0.125f, 0, nullptr), FA2_ERR_HEADDIM);
    EXPECT(f(P(0), P(1), P(2), P(3), F(4), 1, 2, 64, 64, nan, 0, nullptr), FA2_ERR_SCALE);
    EXPECT(f(P(0), P(1), P(2), P(3), F(4), 1, 2, 64, 64, -inf, 0, nullptr), FA2_ERR_SCALE);
    EXPECT(f(off(P(0), 8), P(1), P(2), P(3), F(4), 1, 2, 64, 64, 0.1f, 0, nullptr), FA2_ERR_ALIGN);
    EXPECT(f(P(0), P(1), P(2), P(3), static_cast<float *>(off(F(4), 4)), 1, 2, 64, 64, 0.1f, 0,
             nullptr), FA2_ERR_ALIGN);
    EXPECT(f(P(0), P(1), P(2), P(0), F(4), 1, 2, 64, 64, 0.1f, 0, nullptr), FA2_ERR_ALIAS);
    EXPECT(f(P(0), P(1), P(2), off(P(2), 4096), F(4), 1, 2, 64, 64, 0.1f, 0, nullptr), FA2_ERR_ALIAS);
    EXPECT(f(P(0), P(1), P(2), P(3), static_cast<float *>(off(P(3), 16)), 1, 2, 64, 64, 0.1f, 0,
           nullptr), FA2_ERR_ALIAS);
  }
  // fp32 entry point (element size 4)
  EXPECT(fa2_fwd_fp32(F(0), F(1), F(2), F(3), F(4), 1, 1, 128, 64, 0.125f, 0, nullptr), FA2_OK);
  EXPECT(fa2_fwd_fp32(F(0), F(1), F(2), static_cast<float *>(off(F(0), 16)), F(4), 1, 1, 128, 64,
                      0.125f, 0, nullptr), FA2_ERR_ALIAS);
  // grouped K/V heads
  EXPECT(fa2_fwd_gqa(P(0), P(1), P(2), P(3), F(4), 2, 8, 2, 300, 128, 0.1f, 1, nullptr), FA2_OK);
  EXPECT(fa2_fwd_gqa(P(0), P(1), P(2), P(3), F(4), 2, 8, 3, 300, 128, 0.1f, 1, nullptr), FA2_ERR_SHAPE);
  EXPECT(fa2_fwd_gqa(P(0), P(1), P(2), P(3), F(4), 2, 8, 0, 300, 128, 0.1f, 1, nullptr), FA2_ERR_SHAPE);
  // grouped short query blocks: the query heads of one K/V head are launched
  // as one block of (H / H_kv) * Nq unmasked rows when every row sees the
  // same keys and the packed head fits the per-head bound
  struct Pack { int B, H, Hkv, Nq, Nk, d, causal; bool packed; };
  const Pack packs[] = {
      {8, 32, 8, 1, 16384, 128, 1, true},      // decoding: one query sees every key
      {8, 32, 8, 1, 16384, 128, 0, true},
      {2, 8, 2, 40, 300, 64, 0, true},         // short blocks, no mask
      {2, 8, 2, 4, 300, 128, 1, false},        // causal with several queries: per-row mask
      {2, 8, 2, 128, 300, 128, 0, false},      // full blocks
      {2, 8, 8, 1, 300, 128, 0, false},        // no shared K/V heads
      {1, 66048, 1, 127, 300, 128, 0, true},   // packed head exactly at the per-head bound
      {1, 66052, 1, 127, 300, 128, 0, false},  // one that would pass it
  };
  for (const Pack &c : packs) {
    EXPECT(fa2_fwd_splitkv(FAR(0), FAR(1), FAR(2), FAR(3), static_cast<float *>(FAR(4)), c.B, c.H,
                           c.Hkv, c.Nq, c.Nk, c.d, 0.1f, c.causal, 1, nullptr, nullptr, nullptr),
           FA2_OK);
    const fa2::FwdArgs &a = fa2::g_last_fwd;
    const int g = c.H / c.Hkv;
    const bool ok = c.packed ? (a.bh == c.B * c.Hkv && a.h == c.Hkv && a.group == 1 &&
                                a.nq == c.Nq * g && a.nk == c.Nk && !a.causal)
                             : (a.bh == c.B * c.H && a.h == c.H && a.group == g &&
                                a.nq == c.Nq && a.nk == c.Nk && a.causal == (c.causal != 0));
    if (!ok) {
      std::printf("FAIL packing B=%d H=%d H_kv=%d Nq=%d causal=%d: bh=%d h=%d group=%d nq=%d "
                  "causal=%d\n", c.B, c.H, c.Hkv, c.Nq, c.causal, a.bh, a.h, a.group, a.nq,
                  int(a.causal));
      ++g_fail;
    }
  }
  // the grouped forward packs the same way (N < 128, no mask)
  EXPECT(fa2_fwd_gqa(P(0), P(1), P(2), P(3), F(4), 2, 8, 2, 100, 128, 0.1f, 0, nullptr), FA2_OK);
  const fa2::FwdArgs &gq = fa2::g_last_fwd;
  if (!(gq.bh == 4 && gq.nq == 400 && gq.nk == 100 &&
        gq.group == 1)) {
    std::printf("FAIL fa2_fwd_gqa packing: bh=%d nq=%d nk=%d group=%d\n", gq.bh,
                gq.nq, gq.nk, gq.group);
    ++g_fail;
  }
  // split key ranges, caller workspaces
  EXPECT(fa2_fwd_splitkv(P(0), P(1), P(2), P(3), F(4), 1, 4, 2, 16, 1000, 128, 0.1f, 1, 4, F(5),
                         F(6), nullptr), FA2_OK);
  EXPECT(fa2_fwd_splitkv(P(0), P(1), P(2), P(3), F(4), 1, 4, 2, 16, 1000, 128, 0.1f, 1, 1, nullptr,
                         nullptr, nullptr), FA2_OK);
  EXPECT(fa2_fwd_splitkv(P(0), P(1), P(2), P(3), F(4), 1, 4, 2, 16, 1000, 128, 0.1f, 1, 4, nullptr,
                         F(6), nullptr), FA2_ERR_NULL);
  EXPECT(fa2_fwd_splitkv(P(0), P(1), P(2), P(3), F(4), 1, 4, 2, 16, 1000, 128, 0.1f, 1, 0, F(5),
                         F(6), nullptr), FA2_ERR_SHAPE);
  EXPECT(fa2_fwd_splitkv(P(0), P(1), P(2), P(3), F(4), 1, 4, 2, 16, 1000, 128, 0.1f, 1,
                         FA2_MAX_SPLITS + 1, F(5), F(6), nullptr), FA2_ERR_SHAPE);
  EXPECT(fa2_fwd_splitkv(P(0), P(1), P(2), P(3), F(4), 1, 4, 2, 16, 1000, 128, 0.1f, 1, 4, F(5),
                         static_cast<float *>(off(F(5), 64)), nullptr), FA2_ERR_ALIAS);
  EXPECT(fa2_fwd_splitkv_o32(F(0), F(1), F(2), F(3), F(4), 1, 4, 2, 16, 1000, 128, 0.1f, 1, 4,
                             F(5), static_cast<float *>(off(F(6), 4)), nullptr), FA2_ERR_ALIGN);
  // the allocation-free variant: static workspace, size limit
  EXPECT(fa2_fwd_splitkv_noalloc(P(0), P(1), P(2), P(3), F(4), 1, 4, 2, 16, 1000, 128, 0.1f, 1, 4,
                                 nullptr), FA2_OK);
  EXPECT(fa2_fwd_splitkv_noalloc(P(0), P(1), P(2), P(3), F(4), 1, 1, 1, 1 << 16, 1 << 16, 128,
                                 0.1f, 0, 2, nullptr), FA2_ERR_WORKSPACE);
  EXPECT(fa2_fwd_splitkv_noalloc(P(0), P(1), P(2), nullptr, F(4), 1, 4, 2, 16, 1000, 128, 0.1f, 1,
                                 4, nullptr), FA2_ERR_NULL);
  EXPECT(fa2_fwd_splitkv_noalloc(P(0), P(1), P(2), P(3), F(4), INT32_MAX, INT32_MAX, 1, INT32_MAX,
                                 INT32_MAX, 128, 0.1f, 1, 1024, nullptr), FA2_ERR_SHAPE);
  EXPECT(fa2_bwd(P(0), P(1), P(2), P(3), P(4), F(5), F(6), P(7), P(8), P(9), INT32_MAX, INT32_MAX,
                 INT32_MAX, 128, 0.1f, 1, nullptr), FA2_ERR_SHAPE);
  // FP8 path
  int *E0 = static_cast<int *>(P(5));
  EXPECT(fa2_quantize_fp8(P(0), P(1), E0, 1, 2, 100, 128, 64, F(6), nullptr), FA2_OK);
  EXPECT(fa2_quantize_fp8(P(0), P(1), E0, 1, 2, 100, 128, 32, F(6), nullptr), FA2_ERR_SHAPE);
  EXPECT(fa2_quantize_fp8(P(0), P(1), E0, INT32_MAX, INT32_MAX, INT32_MAX, 128, 64, F(6), nullptr),
         FA2_ERR_SHAPE);
  EXPECT(fa2_quantize_fp8(P(0), off(P(0), 64), E0, 1, 2, 100, 128, 64, F(6), nullptr), FA2_ERR_ALIAS);
  EXPECT(fa2_fwd_fp8(P(0), static_cast<int *>(P(1)), P(2), static_cast<int *>(P(3)), P(4),
                     static_cast<int *>(P(5)), P(6), F(7), 1, 2, 100, 128, 0.1f, 1, 1, nullptr), FA2_OK);
  EXPECT(fa2_fwd_fp8(P(0), nullptr, P(2), static_cast<int *>(P(3)), P(4),
                     static_cast<int *>(P(5)), P(6), F(7), 1, 2, 100, 128, 0.1f, 1, 1, nullptr),
         FA2_ERR_NULL);
  EXPECT(fa2_fwd_fp8(P(0), static_cast<int *>(P(1)), P(2), static_cast<int *>(P(3)), P(4),
                     static_cast<int *>(P(5)), P(1), F(7), 1, 2, 100, 128, 0.1f, 1, 1, nullptr),
         FA2_ERR_ALIAS);
  // backward
  EXPECT(fa2_bwd(P(0), P(1), P(2), P(3), P(4), F(5), F(6), P(7), P(8), P(9), 1, 2, 200, 128, 0.1f,
                 1, nullptr), FA2_OK);
  EXPECT(fa2_bwd(P(0), P(1), P(2), P(3), P(4), nullptr, F(6), P(7), P(8), P(9), 1, 2, 200, 128,
                 0.1f, 1, nullptr), FA2_ERR_NULL);
  EXPECT(fa2_bwd(P(0), P(1), P(2), P(3), P(4), F(5), F(6), P(7), P(8), P(0), 1, 2, 200, 128, 0.1f,
                 1, nullptr), FA2_ERR_ALIAS);
  EXPECT(fa2_bwd(P(0), P(1), P(2), P(3), P(4), F(5), F(6), P(7), P(7), P(9), 1, 2, 200, 128, 0.1f,
                 1, nullptr), FA2_ERR_ALIAS);
  EXPECT(fa2_bwd_o32(P(0), P(1), P(2), P(3), P(4), F(5), F(6), F(7), F(8), F(9), 1, 2, 200, 64,
                     0.1f, 0, nullptr), FA2_OK);
  EXPECT(fa2_bwd_gqa(P(0), P(1), P(2), P(3), P(4), F(5), F(6), P(7), P(8), P(9), 2, 8, 2, 300, 128,
                     0.1f, 1, 4, F(10), nullptr), FA2_OK);
  EXPECT(fa2_bwd_gqa(P(0), P(1), P(2), P(3), P(4), F(5), F(6), P(7), P(8), P(9), 2, 8, 2, 300, 128,
                     0.1f, 1, 5, F(10), nullptr), FA2_ERR_SHAPE);
  EXPECT(fa2_bwd_gqa(P(0), P(1), P(2), P(3), P(4), F(5), F(6), P(7), P(8), P(9), 2, 8, 2, 300, 128,
                     0.1f, 1, 4, nullptr, nullptr), FA2_ERR_NULL);
  // a stream must belong to the current device; the null stream always does
  {
    hipStream_t st = reinterpret_cast<hipStream_t>(P(20));
    EXPECT(fa2_fwd(P(0), P(1), P(2), P(3), F(4), 1, 2, 64, 64, 0.125f, 0, st), FA2_OK);
    g_stream_device = 1;
    EXPECT(fa2_fwd(P(0), P(1), P(2), P(3), F(4), 1, 2, 64, 64, 0.125f, 0, st), FA2_ERR_DEVICE);
    EXPECT(fa2_fwd(P(0), P(1), P(2), P(3), F(4), 1, 2, 64, 64, 0.125f, 0, nullptr), FA2_OK);
    EXPECT(fa2_fwd(P(0), P(1), P(2), P(3), F(4), 1, 2, 64, 64, 0.125f, 0, hipStreamPerThread),
           FA2_OK);
    EXPECT(fa2_fwd(P(0), P(1), P(2), P(3), F(4), 1, 2, 64, 64, 0.125f, 0, hipStreamLegacy), FA2_OK);
    EXPECT(fa2_fwd_gqa(P(0), P(1), P(2), P(3), F(4), 2, 8, 2, 300, 128, 0.1f, 1, st),
           FA2_ERR_DEVICE);
    EXPECT(fa2_fwd_splitkv(P(0), P(1), P(2), P(3), F(4), 1, 4, 2, 16, 1000, 128, 0.1f, 1, 4, F(5),
                           F(6), st), FA2_ERR_DEVICE);
    EXPECT(fa2_fwd_splitkv_noalloc(P(0), P(1), P(2), P(3), F(4), 1, 4, 2, 16, 1000, 128, 0.1f, 1,
                                   4, st), FA2_ERR_DEVICE);
    EXPECT(fa2_fwd_fp32(F(0), F(1), F(2), F(3), F(4), 1, 1, 128, 64, 0.125f, 0, st),
           FA2_ERR_DEVICE);
    EXPECT(fa2_quantize_fp8(P(0), P(1), static_cast<int *>(P(2)), 1, 2, 100, 128, 64, F(6), st),
           FA2_ERR_DEVICE);
    EXPECT(fa2_fwd_fp8(P(0), static_cast<int *>(P(1)), P(2), static_cast<int *>(P(3)), P(4),
                       static_cast<int *>(P(5)), P(6), F(7), 1, 2, 100, 128, 0.1f, 1, 1, st),
           FA2_ERR_DEVICE);
    EXPECT(fa2_bwd(P(0), P(1), P(2), P(3), P(4), F(5), F(6), P(7), P(8), P(9), 1, 2, 200, 128,
                   0.1f, 1, st), FA2_ERR_DEVICE);
    // argument errors come first
    EXPECT(fa2_fwd(nullptr, P(1), P(2), P(3), F(4), 1, 2, 64, 64, 0.125f, 0, st), FA2_ERR_NULL);
    g_stream_device = 0;
    g_query = hipErrorInvalidValue;  // a failing query is a HIP error
    EXPECT(fa2_fwd(P(0), P(1), P(2), P(3), F(4), 1, 2, 64, 64, 0.125f, 0, st), FA2_ERR_HIP);
    g_query = hipSuccess;
  }
  // a failing launch is reported as FA2_ERR_HIP
  g_result = hipErrorLaunchFailure;
  {
    const int before = g_launches;
    const int rc = fa2_fwd(P(0), P(1), P(2), P(3), F(4), 1, 2, 64, 64, 0.125f, 0, nullptr);
    if (rc != FA2_ERR_HIP || g_launches != before + 1) {
      std::printf("FAIL: launch failure -> %d\n", rc);
      ++g_fail;
    }
  }
  g_result = hipSuccess;
  // every code has its own message; unknown codes too
  const int codes[] = {FA2_OK, FA2_ERR_NULL, FA2_ERR_SHAPE, FA2_ERR_HEADDIM, FA2_ERR_SCALE,
                       FA2_ERR_ALIGN, FA2_ERR_ALIAS, FA2_ERR_HIP, FA2_ERR_WORKSPACE,
                       FA2_ERR_DEVICE, 12345, -99};
  for (int c : codes) {
    const char *m = fa2_strerror(c);
    if (!m || !std::strlen(m)) {
      std::printf("FAIL: strerror(%d)\n", c);
      ++g_fail;
    }
  }
  if (fa2_version() != 8) {
    std::printf("FAIL: version %d\n", fa2_version());
    ++g_fail;
  }
  std::printf("%s: %d failures, %d launches\n", g_fail ? "FAILED" : "ok", g_fail, g_launches);
  return g_fail ? 1 : 0;
}
