// Host-side checks of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer together with the library's host code (the
// sources compiled for the host only, no GPU code) and run on a machine
// without a GPU.  Every call below is answered by the library's argument
// checks or size arithmetic alone, so none reaches the HIP runtime; a call
// that would launch work is never made.  The sanitizers report any
// out-of-bounds access, use of freed memory, signed overflow or other
// undefined behaviour on these paths; the expectations pin the status codes.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "../../include/lsh_attn.h"

static int failures = 0;

#define EXPECT(cond)                                                     \
  do {                                                                   \
    if (!(cond)) {                                                       \
      std::fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, \
                   __LINE__, #cond);                                     \
      ++failures;                                                        \
    }                                                                    \
  } while (0)

// a non-null address the library must never dereference on these paths
static void* const kFake = reinterpret_cast<void*>(0x1000);
static uint16_t* const kFake16 = reinterpret_cast<uint16_t*>(0x1000);
static float* const kFakeF = reinterpret_cast<float*>(0x1000);

static void status_strings() {
  for (int s = -3; s <= 8; ++s) {
    const char* t = lsh_status_string(s);
    EXPECT(t != nullptr);
  }
  EXPECT(lsh_kernel_count() > 0);
  for (int k = -2; k <= lsh_kernel_count() + 2; ++k) {
    const char* n = lsh_kernel_name(k);
    EXPECT((k >= 0 && k < lsh_kernel_count()) == (n != nullptr));
  }
}

static void strides() {
  const int Ns[] = {INT_MIN, -1, 0, 1, 255, 256, 257, 8191, 8192, 8193, 1 << 20, INT_MAX};
  for (int N : Ns)
    for (int K = -2; K <= 17; ++K) {
      const int s = lsh_default_stride(N, K);
      const bool ok = N >= 1 && K >= 0 && K <= 15;
      EXPECT(ok == (s != 0));
      if (ok) EXPECT(s >= 256 && s <= 8192 && (s & (s - 1)) == 0);
    }
  const int Ss[] = {INT_MIN, -256, 0, 1, 255, 256, 3000, 8192, 16384, INT_MAX};
  for (int N : Ns)
    for (int S : Ss) {
      const int c = lsh_num_chunks(N, S);
      if (N < 1 || S < 1) EXPECT(c == 0);
      else EXPECT(c == static_cast<int>((static_cast<long long>(N) + S - 1) / S));
    }
}

static void workspace_sizes() {
  // extreme sizes: rejected (0) without overflow
  const int big[] = {INT_MIN, -1, 0, 1, 2, 64, 65536, INT_MAX};
  for (int B : big)
    for (int H : big)
      for (int N : big) {
        const size_t b = lsh_build_workspace_size(B, H, N, 128, 10, 150, 8192, LSH_BF16);
        const size_t d = lsh_decode_workspace_size(B, 4 * (H > 0 && H < INT_MAX / 4 ? H : 1), H, N, 128, 10, 150,
                                                   8192);
        if (B < 1 || H < 1 || N < 1) {
          EXPECT(b == 0);
          EXPECT(d == 0);
        }
      }
  // invalid parameters give 0
  EXPECT(lsh_build_workspace_size(1, 1, 4096, 64, 8, 32, 4096, LSH_BF16) == 0);   // d
  EXPECT(lsh_build_workspace_size(1, 1, 4096, 128, 16, 32, 4096, LSH_BF16) == 0); // K
  EXPECT(lsh_build_workspace_size(1, 1, 4096, 128, 8, 256, 4096, LSH_BF16) == 0); // L
  EXPECT(lsh_build_workspace_size(1, 1, 4096, 128, 8, 32, 3000, LSH_BF16) == 0);  // stride
  EXPECT(lsh_build_workspace_size(1, 1, 4096, 128, 8, 32, 4096, 7) == 0);         // dtype
  EXPECT(lsh_decode_workspace_size(1, 17, 1, 4096, 128, 8, 32, 4096) == 0);      // G > 16
  EXPECT(lsh_decode_workspace_size(1, 6, 4, 4096, 128, 8, 32, 4096) == 0);       // Hq % Hkv
  // the workloads' sizes: positive, and the decode's never decreases with N
  EXPECT(lsh_build_workspace_size(64, 8, 32768, 128, 10, 150, 8192, LSH_BF16) > 0);
  size_t prev = 0;
  for (int N = 1; N <= 140000; N += 977) {
    const int s = lsh_default_stride(140000, 10);
    const size_t d = lsh_decode_workspace_size(1, 32, 4, N, 128, 10, 150, s);
    EXPECT(d > 0);
    EXPECT(d >= prev);
    prev = d;
  }
  // the limit on units * L * N (2^40) and units * L (2^31)
  EXPECT(lsh_build_workspace_size(1 << 16, 1 << 10, 1 << 20, 128, 8, 255, 8192, LSH_BF16) == 0);
  EXPECT(lsh_build_workspace_size(INT_MAX, INT_MAX, INT_MAX, 128, 8, 255, 8192, LSH_BF16) == 0);
}

static void build_rejects() {
  const size_t ws = lsh_build_workspace_size(1, 1, 4096, 128, 8, 32, 4096, LSH_BF16);
  EXPECT(ws > 0);
  auto build = [&](const void* keys, const void* W, int B, int N, int K, int L, int stride, int dtype,
                   uint16_t* off, uint16_t* idx, void* wsp, size_t wsb) {
    return lsh_build_tables(keys, W, B, 1, N, 128, K, L, stride, dtype, off, idx, nullptr, wsp, wsb, nullptr);
  };
  EXPECT(build(nullptr, kFake, 1, 4096, 8, 32, 4096, LSH_BF16, kFake16, kFake16, kFake, ws) == LSH_ERR_INVALID_ARG);
  EXPECT(build(kFake, nullptr, 1, 4096, 8, 32, 4096, LSH_BF16, kFake16, kFake16, kFake, ws) == LSH_ERR_INVALID_ARG);
  EXPECT(build(kFake, kFake, 1, 4096, 8, 32, 4096, LSH_BF16, nullptr, kFake16, kFake, ws) == LSH_ERR_INVALID_ARG);
  EXPECT(build(kFake, kFake, 1, 4096, 8, 32, 4096, LSH_BF16, kFake16, nullptr, kFake, ws) == LSH_ERR_INVALID_ARG);
  EXPECT(build(kFake, kFake, 1, 4096, 8, 32, 4096, LSH_BF16, kFake16, kFake16, nullptr, ws) == LSH_ERR_INVALID_ARG);
  EXPECT(build(kFake, kFake, 0, 4096, 8, 32, 4096, LSH_BF16, kFake16, kFake16, kFake, ws) == LSH_ERR_INVALID_ARG);
  EXPECT(build(kFake, kFake, 1, 4096, 8, 32, 128, LSH_BF16, kFake16, kFake16, kFake, ws) == LSH_ERR_UNSUPPORTED);
  EXPECT(build(kFake, kFake, 1, 4096, 8, 32, 4096, LSH_BF16, kFake16, kFake16, kFake, ws - 1) ==
         LSH_ERR_WORKSPACE);
  EXPECT(build(kFake, kFake, 1, 4096, 8, 32, 4096, LSH_BF16, kFake16, kFake16, kFake, 0) == LSH_ERR_WORKSPACE);
  // an update that appends nothing launches nothing and succeeds
  EXPECT(lsh_update_tables(kFake, kFake, 1, 1, 100, 100, 4096, nullptr, nullptr, 128, 8, 32, 1024, LSH_BF16, 0,
                           kFake16, kFake16, nullptr, kFake, ws, nullptr) == LSH_OK);
  EXPECT(lsh_update_tables(kFake, kFake, 1, 1, 200, 100, 4096, nullptr, nullptr, 128, 8, 32, 1024, LSH_BF16, 0,
                           kFake16, kFake16, nullptr, kFake, ws, nullptr) == LSH_ERR_INVALID_ARG);
  EXPECT(lsh_update_tables(kFake, kFake, 1, 1, 0, 5000, 4096, nullptr, nullptr, 128, 8, 32, 1024, LSH_BF16, 0,
                           kFake16, kFake16, nullptr, kFake, ws, nullptr) == LSH_ERR_INVALID_ARG);
  EXPECT(lsh_update_tables(kFake, kFake, 1, 1, 0, 100, 4096, nullptr, nullptr, 128, 8, 32, 1024, LSH_BF16, 2,
                           kFake16, kFake16, nullptr, kFake, ws, nullptr) == LSH_ERR_INVALID_ARG);
}

static void decode_rejects() {
  const size_t ws = lsh_decode_workspace_size(1, 4, 1, 4096, 128, 8, 32, 4096);
  EXPECT(ws > 0);
  auto dec = [&](const void* q, int Hq, int Hkv, int T, float scale, int n_sink, int n_window, float* out,
                 void* wsp, size_t wsb) {
    return lsh_decode_attention_hybrid(q, kFake, kFake, kFake, kFake16, kFake16, 1, Hq, Hkv, 4096, 128, 8, 32, T,
                                       4096, scale, LSH_BF16, n_sink, n_window, out, nullptr, nullptr, nullptr,
                                       nullptr, wsp, wsb, nullptr);
  };
  EXPECT(dec(nullptr, 4, 1, 2, 0.08f, 0, 0, kFakeF, kFake, ws) == LSH_ERR_INVALID_ARG);
  EXPECT(dec(kFake, 4, 1, 2, 0.08f, 0, 0, nullptr, kFake, ws) == LSH_ERR_INVALID_ARG);
  EXPECT(dec(kFake, 4, 1, 2, 0.08f, 0, 0, kFakeF, nullptr, ws) == LSH_ERR_INVALID_ARG);
  EXPECT(dec(kFake, 6, 4, 2, 0.08f, 0, 0, kFakeF, kFake, ws) == LSH_ERR_INVALID_ARG);
  EXPECT(dec(kFake, 17, 1, 2, 0.08f, 0, 0, kFakeF, kFake, ws) == LSH_ERR_UNSUPPORTED);
  EXPECT(dec(kFake, 4, 1, 0, 0.08f, 0, 0, kFakeF, kFake, ws) == LSH_ERR_INVALID_ARG);
  EXPECT(dec(kFake, 4, 1, 33, 0.08f, 0, 0, kFakeF, kFake, ws) == LSH_ERR_INVALID_ARG);
  EXPECT(dec(kFake, 4, 1, 2, __builtin_nanf(""), 0, 0, kFakeF, kFake, ws) == LSH_ERR_INVALID_ARG);
  EXPECT(dec(kFake, 4, 1, 2, __builtin_inff(), 0, 0, kFakeF, kFake, ws) == LSH_ERR_INVALID_ARG);
  EXPECT(dec(kFake, 4, 1, 2, 0.08f, -1, 0, kFakeF, kFake, ws) == LSH_ERR_INVALID_ARG);
  EXPECT(dec(kFake, 4, 1, 2, 0.08f, 0, -1, kFakeF, kFake, ws) == LSH_ERR_INVALID_ARG);
  EXPECT(dec(kFake, 4, 1, 2, 0.08f, 0, 0, kFakeF, kFake, ws - 1) == LSH_ERR_WORKSPACE);
  // the cached decode: n_cap below N, a bad per-head flag
  EXPECT(lsh_decode_attention_cached(kFake, kFake, kFake, kFake, kFake16, kFake16, 1, 4, 1, 4096, 4000, nullptr,
                                     128, 8, 32, 2, 4096, 0.08f, LSH_BF16, 0, 0, 0, kFakeF, nullptr, nullptr,
                                     nullptr, nullptr, kFake, ws, nullptr) == LSH_ERR_INVALID_ARG);
  EXPECT(lsh_decode_attention_cached(kFake, kFake, kFake, kFake, kFake16, kFake16, 1, 4, 1, 4096, 4096, nullptr,
                                     128, 8, 32, 2, 4096, 0.08f, LSH_BF16, 3, 0, 0, kFakeF, nullptr, nullptr,
                                     nullptr, nullptr, kFake, ws, nullptr) == LSH_ERR_INVALID_ARG);
  // the no-alloc decode: its checks and its scratch limit come before any HIP call
  EXPECT(lsh_decode_attention_noalloc(nullptr, kFake, kFake, kFake, kFake16, kFake16, 1, 4, 1, 4096, 4096, nullptr,
                                      128, 8, 32, 2, 4096, 0.08f, LSH_BF16, 0, 0, 0, kFakeF, nullptr, nullptr,
                                      nullptr, nullptr, nullptr) == LSH_ERR_INVALID_ARG);
  // 8192 query heads over 64K keys: their bitmask words alone are 64 MiB
  EXPECT(lsh_decode_workspace_size(512, 16, 1, 65536, 128, 8, 32, 8192) > LSH_NOALLOC_SCRATCH_BYTES);
  EXPECT(lsh_decode_attention_noalloc(kFake, kFake, kFake, kFake, kFake16, kFake16, 512, 16, 1, 65536, 65536,
                                      nullptr, 128, 8, 32, 2, 8192, 0.08f, LSH_BF16, 0, 0, 0, kFakeF, nullptr,
                                      nullptr, nullptr, nullptr, nullptr) == LSH_ERR_WORKSPACE);
}

static void timing_window() {
  double ms[16];
  int32_t n[16];
  EXPECT(lsh_timing_end(ms, n) == LSH_ERR_INVALID_ARG);   // not open
  EXPECT(lsh_timing_begin() == LSH_OK);
  EXPECT(lsh_timing_begin() == LSH_ERR_INVALID_ARG);      // already open
  EXPECT(lsh_timing_end(ms, n) == LSH_OK);                 // nothing launched
  for (int k = 0; k < lsh_kernel_count(); ++k) EXPECT(ms[k] == 0.0 && n[k] == 0);
}

int main() {
  status_strings();
  strides();
  workspace_sizes();
  build_rejects();
  decode_rejects();
  timing_window();
  if (failures) {
    std::fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  std::printf("host checks passed\n");
  return 0;
}
