// Internal launch interface between the C-ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lsh {

// Arrays over keys have a row pitch P >= N (the capacity of a growing
// cache); offsets have nJP >= nJ chunk slots per table.  The build covers the
// keys of chunks j0 .. nJ - 1 (keys j0 * stride .. N - 1): j0 = 0 is a full
// build, a larger j0 rebuilds only the chunks that new keys fall into.
// Sequences may hold different numbers of keys: old_lens / new_lens (device,
// optional) give sequence b's range, clamped into [j0 * stride, N].
struct BuildArgs {
  const void* keys;      // [U][P][128]
  const void* W;         // [w_heads][128][L*K]
  void* wt;              // workspace: [w_heads][proj_wt_rows(K, L)][128]
  uint16_t* codes;       // [U][L][P] (caller's key_codes or workspace)
  uint16_t* offsets;     // [U][L][nJP][2^K] bucket starts inside each chunk
  uint16_t* indices;     // [U][L][P] chunk-major, key - chunk start
  const int32_t* old_lens;   // optional [B]: keys each sequence's tables hold
  const int32_t* new_lens;   // optional [B]: keys they hold afterwards
  int U, Hkv, N, K, L;
  int P, nJP, j0;
  int stride_log2, nJ;
  int w_heads;           // 1: one W for every head; Hkv: W per kv head
  int dtype;             // 0 = f32, 1 = bf16
};

struct DecodeArgs {
  const void* q;         // [B][Hq][128]
  const void* keys;      // [U][P][128], keys 0 .. len_b - 1 valid
  const void* values;    // [U][P][128]
  const void* W;         // [w_heads][128][L*K]
  const uint16_t* indices;   // [U][L][P] chunk-major
  const uint16_t* offsets;   // [U][L][nJP][2^K]
  const int32_t* seq_lens;   // optional [B]: keys of sequence b (clamped to [0, N]); N when null
  uint16_t* qcodes;      // [B*Hq][L]
  uint32_t* bitmask;     // [B*Hq][Nw]
  int32_t* chunk_nsel;   // [B*Hq][nJ]
  float* lnu_table;      // [kLnuTable + 1]
  float* partials;       // [B*Hq][nsplit + nexact][130]
  float* out;            // [B*Hq][128]
  float* lse;            // optional [B*Hq]
  int32_t* nsel;         // optional [B*Hq]
  uint8_t* counts;       // optional [B*Hq][N]
  int B, Hq, Hkv, N, K, L, T;
  int P, nJP;                // row pitch of keys / values / indices, chunk slots of offsets
  int stride_log2, nJ;
  int split_len, nsplit;
  float scale;
  int w_heads;
  int dtype;
  // exact set of sequence b (length n): keys [0, eh) and [n - et, n) with
  // eh = min(n_sink, n), et = min(n_window, n - eh)
  int n_sink, n_window;
  int exact_len, nexact;       // the exact set in nexact pieces of exact_len keys, one workgroup each
};

// Keys of sequence b: the given length clamped into [0, N], or N.
__host__ __device__ inline int seq_len_of(const int32_t* lens, int b, int N) {
  if (!lens) return N;
  const int v = lens[b];
  return v < 0 ? 0 : (v > N ? N : v);
}

// The exact set of a sequence of n keys: its first eh and its last et keys.
__host__ __device__ inline void exact_range(int n_sink, int n_window, int n, int& eh, int& et) {
  eh = n_sink < n ? n_sink : n;
  et = n_window < n - eh ? n_window : n - eh;
}

constexpr int kLnuTable = 1024;   // ln-u correction table intervals over theta in [0, pi]
constexpr int kPartialStride = 130;
constexpr int kMaxExactSplits = 16;   // partial slots per head reserved for the exact set

// Kernel kinds, in launch order; names for the timing interface.
enum KernelId {
  kKTransposeW = 0,
  kKProject,
  kKChunkSort,
  kKQhash,
  kKCountSelect,
  kKAttend,
  kKMerge,
  kKNumKernels
};
const char* kernel_name(int id);

// Start/stop events for one launch of kernel `id` while timing is on; both
// null otherwise.
void timing_events(int id, hipEvent_t* start, hipEvent_t* stop);

// Every kernel goes through here: with timing on, the dispatch packet itself
// carries the start and stop timestamps (no extra packets on the stream).
template <typename F, typename... Args>
inline hipError_t launch(int id, F kernel, dim3 grid, dim3 block, unsigned lds, hipStream_t stream,
                         Args... args) {
  hipEvent_t a = nullptr, b = nullptr;
  timing_events(id, &a, &b);
  hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, a, b, 0u, args...);
  return hipGetLastError();
}

// Raises a kernel's dynamic-LDS limit to at least `bytes` on the current
// device.  The attribute is set at most once per (kernel, device, size), so
// launches after the first make no runtime call besides the launch itself
// (which keeps them capturable into a graph).
hipError_t ensure_lds_limit(const void* kernel, size_t bytes);

// Rows of the transposed, permuted projection matrix the build keeps in its
// workspace ([rows][128] of the input dtype).
int proj_wt_rows(int K, int L);

hipError_t launch_build(const BuildArgs& a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
// The bf16 weighted-attention kernel (MFMA for q.k and P.V).
hipError_t launch_attend_bf16(const DecodeArgs& a, hipStream_t stream);

}  // namespace lsh
