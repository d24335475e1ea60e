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
  int n_old;             // the bound n_old of lsh_update_tables
  int mode;              // kUpdateSort, kUpdateInsert or both (chosen per sequence, seq_update)
};
constexpr int kUpdateSort = 1, kUpdateInsert = 2;

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
  double* lnu_samples;   // [kLnuSamples] the ln-u correction g at theta_t = t pi / (2 kLnuTable)
  float* partials;       // [B*Hq][nsplit][kPartialStride]
  int32_t* sync;         // the decode launch's counters (zeroed by the query-hash launch)
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
  bool timed;                  // false: the launches never take timing events (no allocation)
};

// Keys of sequence b: the given length clamped into [0, N], or N.
__host__ __device__ inline int seq_len_of(const int32_t* lens, int b, int N) {
  if (!lens) return N;
  const int v = lens[b];
  return v < 0 ? 0 : (v > N ? N : v);
}

// A table update appends at most this many keys per sequence by insertion.
constexpr int kInsertMax = 256;

// Sequence b's part of a table update from n_old .. n_new (= N) keys: the
// keys its tables hold before (old) and after (hi), both clamped into
// [n_old, N], and whether its new keys are inserted into the built chunks
// (at most kInsertMax keys onto tables that hold some) rather than re-sorted
// with the chunks that hold them.
struct SeqUpdate {
  int old, hi;
  bool insert;
};
__host__ __device__ inline SeqUpdate seq_update(const int32_t* old_lens, const int32_t* new_lens, int b, int n_old,
                                                int N) {
  SeqUpdate s;
  const int h = seq_len_of(new_lens, b, N);
  s.hi = h < n_old ? n_old : h;
  const int o = old_lens ? seq_len_of(old_lens, b, s.hi) : n_old;
  s.old = o < n_old ? n_old : o;
  s.insert = s.old > 0 && s.hi - s.old <= kInsertMax;
  return s;
}

// The exact set of a sequence of n keys: its first eh and its last et keys.
__host__ __device__ inline void exact_range(int n_sink, int n_window, int n, int& eh, int& et) {
  eh = n_sink < n ? n_sink : n;
  et = n_window < n - eh ? n_window : n - eh;
}

// The ln-u correction g(theta) is kept as one quadratic per interval of
// width pi / kLnuTable, g(theta_j + f h) ~ x + f (y + f z) for f in [0, 1],
// through fp64 samples at the interval's start, middle and end; the
// coefficients are formed in fp64 and rounded once, so the small y and z
// keep their relative precision.
constexpr int kLnuTable = 1024;
constexpr int kLnuSamples = 2 * kLnuTable + 1;
// A partial state (acc[128], max, sum) padded to five 128-byte lines, so no
// cache line holds two workgroups' partials.
constexpr int kResidentWG = 512;   // decode workgroups resident at once: about two per CU on 256 CUs
constexpr int kPartialStride = 160;

// Kernel kinds, in launch order; names for the timing interface.
enum KernelId {
  kKTransposeW = 0,
  kKProject,
  kKChunkSort,
  kKChunkInsert,
  kKQhash,
  kKDecode,
  kKNumKernels
};
const char* kernel_name(int id);

// Checked builds (LSH_CHECKED defined): kernels test their index arithmetic
// against the bounds the arguments promise and OR a bit into a device word
// on a violation (the access itself stays clamped as in every build).  The
// word is set with lsh_check_set; unchecked builds compile the tests out.
enum CheckBit : uint32_t {
  kChkQueryCode = 1u,      // a query code >= 2^K
  kChkSegment = 2u,        // a probed bucket's bounds outside its chunk
  kChkEntry = 4u,          // a bucket entry >= the chunk's length
  kChkSlot = 8u,           // an attention workgroup's unit or slot out of range
  kChkSortCode = 16u,      // a key code >= 2^K in the sort
  kChkInsert = 32u,        // an insert: a code >= 2^K or a bucket end outside the chunk's entries
};
#ifdef LSH_CHECKED
extern uint32_t* g_check;   // device word of the checked build (null: no checks)
#define LSH_CHECK(ptr, cond, bit) \
  do { if (!(cond) && (ptr) != nullptr) atomicOr((ptr), static_cast<unsigned>(bit)); } while (0)
#else
#define LSH_CHECK(ptr, cond, bit) do { } while (0)
#endif

// A launch id ORed with kUntimed never takes timing events.
constexpr int kUntimed = 1 << 8;

// Start/stop events for one launch of kernel `id` while timing is on; both
// null otherwise, and always for an untimed launch.
void timing_events(int id, hipEvent_t* start, hipEvent_t* stop);

// LSH_DEBUG_LAUNCH set (and not "0") in the environment when the library
// first launches: every launch prints its kernel, grid, block and LDS bytes
// to stderr (a debugging aid; the check itself is one load of a flag).
bool debug_launch();
void print_launch(int id, dim3 grid, dim3 block, unsigned lds, hipStream_t stream);

// Every kernel goes through here: with timing on, the dispatch packet itself
// carries the start and stop timestamps (no extra packets on the stream).
template <typename F, typename... Args>
inline hipError_t launch(int id, F kernel, dim3 grid, dim3 block, unsigned lds, hipStream_t stream,
                         Args... args) {
  if (debug_launch()) print_launch(id, grid, block, lds, stream);
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
// The one-launch decode over bf16 K/V (MFMA for q.k and P.V).
struct FusedParams;
hipError_t launch_decode_bf16(const FusedParams& p, int kid, hipStream_t stream);

}  // namespace lsh
