// Sanitizer harness for the decode library's host-side argument checks (test
// infrastructure): tests/test_sanitizers.py compiles the library's C entry
// points (csrc/api.hip) for the host with AddressSanitizer and
// UndefinedBehaviorSanitizer and links them with this file, whose kernel
// launchers abort if reached.  Every call below must be rejected on the host
// with the documented status before any launch, or is a host-only query; a
// sanitizer report, a launch, or a wrong status fails the run.  No GPU is
// needed.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/mla_decode.h"
#include "../../mla_decode_attention_split_amd/csrc/mla_internal.hpp"

namespace mla {
hipError_t launch_sched(const int32_t*, int, int, int, int32_t*, int32_t*, hipStream_t) {
  std::fprintf(stderr, "unexpected scheduler launch\n");
  std::abort();
}
hipError_t launch_decode(const DecodeArgs&, int, hipStream_t) {
  std::fprintf(stderr, "unexpected decode launch\n");
  std::abort();
}
hipError_t launch_combine(CombineArgs, int, hipStream_t) {
  std::fprintf(stderr, "unexpected combine launch\n");
  std::abort();
}
}  // namespace mla

static int failures = 0;
#define EXPECT_EQ(a, b)                                                                 \
  do {                                                                                  \
    long long va = (long long)(a), vb = (long long)(b);                                 \
    if (va != vb) {                                                                     \
      std::fprintf(stderr, "%s:%d: %s = %lld, expected %lld (%s)\n", __FILE__, __LINE__, \
                   #a, va, vb, mla_last_error());                                       \
      ++failures;                                                                       \
    }                                                                                   \
  } while (0)

// A 16-byte aligned non-null address that is never dereferenced.
static void* const F = reinterpret_cast<void*>(uintptr_t(1) << 20);
static int32_t* const FI = static_cast<int32_t*>(F);

struct Dec {
  const void *q = F, *k = F;
  const int32_t *bt = FI, *sl = FI;
  int batch = 2, s_q = 1, h_q = 16, h_kv = 1, d = 576, dv = 512, dtype = 0, num_pages = 8,
      page = 64, max_blocks = 4;
  const int32_t* meta = FI;
  int num_parts = 8;
  const int32_t* splits = FI;
  int causal = 0;
  float scale = 0.0416f;
  void* out = F;
  float* lse = static_cast<float*>(F);
  void* ws = F;
  size_t ws_bytes = size_t(1) << 30;
  int run() const {
    return mla_decode(q, k, bt, sl, batch, s_q, h_q, h_kv, d, dv, dtype, num_pages, page,
                      max_blocks, meta, num_parts, splits, causal, scale, out, lse, ws, ws_bytes,
                      nullptr);
  }
  int run_split() const {
    return mla_decode_splitkv(q, k, bt, sl, batch, s_q, h_q, h_kv, d, dv, dtype, num_pages, page,
                              max_blocks, meta, num_parts, splits, causal, scale, out, lse, ws,
                              ws_bytes, nullptr);
  }
};

int main() {
  // host-only queries
  int tr = 0, mt = 0, fc = 0;
  EXPECT_EQ(mla_tile_shape(256, 1, &tr, &mt, &fc), MLA_OK);
  EXPECT_EQ(tr, 128);
  EXPECT_EQ(mt, 2);
  EXPECT_EQ(mla_tile_shape(0, 1, &tr, &mt, &fc), MLA_ERR_UNSUPPORTED);
  EXPECT_EQ(mla_tile_shape(16, 0, nullptr, nullptr, nullptr), MLA_ERR_INVALID_ARG);
  EXPECT_EQ(mla_workspace_bytes(32, 16, 1, 256, 512),
            (32 + 256) * 16 * 1024 + ((32 + 256) * 16 * 4 + 255) / 256 * 256);
  EXPECT_EQ(mla_workspace_bytes(MLA_MAX_BATCH, MLA_MAX_ROWS, 1, MLA_MAX_PARTS, 512) > 0, 1);
  EXPECT_EQ(mla_workspace_bytes(0, 16, 1, 256, 512), 0);
  EXPECT_EQ(mla_workspace_bytes(4, 16, 1, 256, 511), 0);
  EXPECT_EQ(std::strcmp(mla_status_string(MLA_OK), "ok"), 0);
  EXPECT_EQ(std::strcmp(mla_status_string(-99), "unknown status"), 0);
  EXPECT_EQ(mla_metadata_shape(0, 16, 1, nullptr, nullptr), MLA_ERR_INVALID_ARG);
  EXPECT_EQ(mla_metadata_shape(4, 5000, 1, nullptr, nullptr), MLA_ERR_UNSUPPORTED);

  // metadata call rejections
  EXPECT_EQ(mla_get_metadata(FI, 0, 16, 1, FI, FI, nullptr), MLA_ERR_INVALID_ARG);
  EXPECT_EQ(mla_get_metadata(FI, MLA_MAX_BATCH + 1, 16, 1, FI, FI, nullptr), MLA_ERR_INVALID_ARG);
  EXPECT_EQ(mla_get_metadata(nullptr, 4, 16, 1, FI, FI, nullptr), MLA_ERR_INVALID_ARG);
  EXPECT_EQ(mla_get_metadata(FI, 4, 16, 1, FI + 1, FI, nullptr), MLA_ERR_INVALID_ARG);
  EXPECT_EQ(mla_get_metadata(FI, 4, 0, 1, FI, FI, nullptr), MLA_ERR_UNSUPPORTED);
  EXPECT_EQ(mla_get_metadata_ex(FI, 4, 16, 1, FI, FI, nullptr, -3, 0), MLA_ERR_INVALID_ARG);
  EXPECT_EQ(mla_get_metadata_ex(FI, 4, 16, 1, FI, FI, nullptr, 8, -1), MLA_ERR_INVALID_ARG);

  // decode rejections, one bad argument at a time
  struct Case {
    const char* what;
    void (*edit)(Dec&);
    int status;
  } cases[] = {
      {"d", [](Dec& a) { a.d = 575; }, MLA_ERR_UNSUPPORTED},
      {"dv", [](Dec& a) { a.dv = 256; }, MLA_ERR_UNSUPPORTED},
      {"page", [](Dec& a) { a.page = 32; }, MLA_ERR_UNSUPPORTED},
      {"dtype", [](Dec& a) { a.dtype = 7; }, MLA_ERR_UNSUPPORTED},
      {"batch", [](Dec& a) { a.batch = 0; }, MLA_ERR_INVALID_ARG},
      {"h_kv", [](Dec& a) { a.h_kv = 3; }, MLA_ERR_INVALID_ARG},
      {"rows", [](Dec& a) { a.s_q = 64; a.h_q = 128; }, MLA_ERR_UNSUPPORTED},
      {"huge s_q", [](Dec& a) { a.s_q = 1 << 30; }, MLA_ERR_UNSUPPORTED},
      {"q", [](Dec& a) { a.q = nullptr; }, MLA_ERR_INVALID_ARG},
      {"ws", [](Dec& a) { a.ws = nullptr; }, MLA_ERR_INVALID_ARG},
      {"align", [](Dec& a) { a.out = static_cast<char*>(F) + 8; }, MLA_ERR_INVALID_ARG},
      {"parts", [](Dec& a) { a.num_parts = 0; }, MLA_ERR_INVALID_ARG},
      {"scale nan", [](Dec& a) { a.scale = __builtin_nanf(""); }, MLA_ERR_INVALID_ARG},
      {"scale 0", [](Dec& a) { a.scale = 0.f; }, MLA_ERR_INVALID_ARG},
      {"scale <0", [](Dec& a) { a.scale = -1.f; }, MLA_ERR_INVALID_ARG},
      {"ws size", [](Dec& a) { a.ws_bytes = 100; }, MLA_ERR_WORKSPACE},
      {"pages", [](Dec& a) { a.num_pages = 0; }, MLA_ERR_INVALID_ARG},
  };
  for (const Case& c : cases) {
    Dec a;
    c.edit(a);
    EXPECT_EQ(a.run(), c.status);
    EXPECT_EQ(a.run_split(), c.status);
  }
  EXPECT_EQ(mla_decode_combine(FI, 0, 1, 16, 1, 8, 0, F, static_cast<float*>(F), F, 1 << 30, nullptr),
            MLA_ERR_INVALID_ARG);
  EXPECT_EQ(mla_decode_combine(FI, 2, 1, 16, 1, 8, 0, F, static_cast<float*>(F), F, 100, nullptr),
            MLA_ERR_WORKSPACE);
  EXPECT_EQ(mla_decode_combine(FI, 2, 1, 16, 1, 8, 5, F, static_cast<float*>(F), F, 1 << 30, nullptr),
            MLA_ERR_UNSUPPORTED);
  std::printf("abi sanitizer harness: %d failures\n", failures);
  return failures ? 1 : 0;
}
