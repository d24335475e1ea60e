// C ABI of the LSH-sampled decode-attention library: argument checks,
// workspace layout and launch order.  Declarations and the definitions of
// every operation are in include/lsh_attn.h.
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <vector>

#include "../../include/lsh_attn.h"
#include "lsh_kernels.h"

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxStrideLog2 = 13;     // a chunk is sorted in one workgroup's LDS
constexpr int kMinStrideLog2 = 8;

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

int ilog2_exact(int x) {
  if (x <= 0 || (x & (x - 1))) return -1;
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

struct Geometry {
  int stride_log2 = 0, nJ = 0, LKpad = 0;
};

// Checks shared by build and decode.  Returns LSH_OK and fills `g`.
lsh_status check_common(int B, int Hkv, int N, int d, int K, int L, int stride, int dtype, Geometry* g) {
  if (B < 1 || Hkv < 1 || N < 1 || d < 1 || L < 1 || L > 255 || K < 0 || K > 15)
    return LSH_ERR_INVALID_ARG;
  if (dtype != LSH_F32 && dtype != LSH_BF16) return LSH_ERR_INVALID_ARG;
  const int sl = ilog2_exact(stride);
  if (sl < 0) return LSH_ERR_INVALID_ARG;
  if (d != 128) return LSH_ERR_UNSUPPORTED;
  if (sl < kMinStrideLog2 || sl > kMaxStrideLog2) return LSH_ERR_UNSUPPORTED;
  // keys per sequence: up to 2^30, so that index arithmetic on N in int
  // (rounding up to words, chunks or splits) cannot overflow
  if (N > (1 << 30)) return LSH_ERR_UNSUPPORTED;
  // each product is formed only once the one before it is known to be small
  const long long units = static_cast<long long>(B) * Hkv;
  if (units >= (1ll << 31) || units * L >= (1ll << 31) || units * L * static_cast<long long>(N) >= (1ll << 40))
    return LSH_ERR_UNSUPPORTED;
  g->stride_log2 = sl;
  g->nJ = lsh_num_chunks(N, stride);
  g->LKpad = lsh::proj_wt_rows(K, L);
  return LSH_OK;
}

int elem_bytes(int dtype) { return dtype == LSH_BF16 ? 2 : 4; }

struct BuildLayout {
  size_t wt = 0, codes = 0, total = 0;
};

BuildLayout build_layout(int B, int Hkv, int N, int L, int dtype, const Geometry& g, bool need_codes) {
  BuildLayout w;
  size_t off = 0;
  // WT for every kv head (one W per kv head is the larger case)
  w.wt = off;
  off = align_up(off + static_cast<size_t>(Hkv) * g.LKpad * 128 * elem_bytes(dtype));
  w.codes = off;
  if (need_codes) off = align_up(off + static_cast<size_t>(B) * Hkv * L * N * sizeof(uint16_t));
  w.total = off;
  return w;
}

struct DecodeLayout {
  size_t qcodes = 0, bitmask = 0, chunk_nsel = 0, lnu = 0, partials = 0, sync = 0, total = 0;
  int split_len = 0, nsplit = 0;
};

DecodeLayout decode_layout(int B, int Hq, int Hkv, int N, int L, const Geometry& g) {
  DecodeLayout w;
  // context split: about two resident workgroups per CU (kResidentWG over
  // the 256 CUs) over the (sequence, kv head) units, each split a multiple
  // of 256 keys
  const long long units = static_cast<long long>(B) * Hkv;
  long long per = (units * N + lsh::kResidentWG - 1) / lsh::kResidentWG;
  per = (per + 255) / 256 * 256;
  if (per < 256) per = 256;
  if (per > N) per = (static_cast<long long>(N) + 255) / 256 * 256;
  w.split_len = static_cast<int>(per);
  w.nsplit = static_cast<int>((N + per - 1) / per);
  const size_t BH = static_cast<size_t>(B) * Hq;
  size_t off = 0;
  w.qcodes = off;     off = align_up(off + BH * L * sizeof(uint16_t));
  w.bitmask = off;    off = align_up(off + BH * ((static_cast<size_t>(N) + 31) / 32) * sizeof(uint32_t));
  w.chunk_nsel = off; off = align_up(off + BH * g.nJ * sizeof(int32_t));
  w.lnu = off;        off = align_up(off + lsh::kLnuSamples * sizeof(double));
  // partial slots: nsplit <= min(ceil(N / 256), ceil(kResidentWG / units)), a bound
  // that grows with N, so the workspace size at a cache's capacity covers
  // every shorter length
  const long long slots = std::max<long long>(
      w.nsplit, std::min((static_cast<long long>(N) + 255) / 256, (lsh::kResidentWG - 1 + units) / units));
  w.partials = off;
  off = align_up(off + BH * static_cast<size_t>(slots) * lsh::kPartialStride * sizeof(float));
  // counters of the decode launch: per (unit, chunk) and per unit
  w.sync = off;
  off = align_up(off + static_cast<size_t>(units * g.nJ + units) * sizeof(int32_t));
  w.total = off;
  return w;
}

lsh_status hip_status(hipError_t e) { return e == hipSuccess ? LSH_OK : LSH_ERR_HIP; }

// Device address of each device's copy of `scratch` (below), taken once per
// device with that device current; a fixed table, so the no-alloc entry point
// allocates nothing, not even host memory.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Kernel timing.  While a timing window is open every launch takes a pair of
// events from this pool (grown on demand, reused across windows); closing the
// window waits for them and sums the elapsed times per kernel kind.
struct TimingRecord {
  int id;
  hipEvent_t start, stop;
};
std::mutex g_timing_mu;
bool g_timing_on = false;
std::vector<TimingRecord> g_timing_pool;
size_t g_timing_used = 0;

}  // namespace

// The workspace of lsh_decode_attention_noalloc: every device the library
// runs on holds its own copy until the process ends.  In host code this name
// is a host-side stand-in, never a device address: kernels receive the
// address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[LSH_NOALLOC_SCRATCH_BYTES];

namespace {

lsh_status scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LSH_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LSH_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LSH_OK;
}

}  // namespace

namespace lsh {

#ifdef LSH_CHECKED
uint32_t* g_check = nullptr;
#endif

const char* kernel_name(int id) {
  static const char* const names[kKNumKernels] = {
      "transpose_w", "project_codes", "chunk_sort", "chunk_insert", "qhash", "decode"};
  return (id >= 0 && id < kKNumKernels) ? names[id] : nullptr;
}

hipError_t ensure_lds_limit(const void* kernel, size_t bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, size_t> done;
  std::lock_guard<std::mutex> lk(mu);
  size_t& cur = done[{kernel, dev}];
  if (cur >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
  if (e == hipSuccess) cur = bytes;
  return e;
}

bool debug_launch() {
  static const bool on = [] {
    const char* e = std::getenv("LSH_DEBUG_LAUNCH");
    return e != nullptr && e[0] != '\0' && std::strcmp(e, "0") != 0;
  }();
  return on;
}

void print_launch(int id, dim3 grid, dim3 block, unsigned lds, hipStream_t stream) {
  const char* name = kernel_name(id & (kUntimed - 1));
  std::fprintf(stderr, "[lsh] launch %s%s grid (%u, %u, %u) block (%u, %u, %u) dynamic lds %u stream %p\n",
               name ? name : "?", (id & kUntimed) ? " (untimed)" : "", grid.x, grid.y, grid.z, block.x, block.y,
               block.z, lds, static_cast<void*>(stream));
}

void timing_events(int id, hipEvent_t* start, hipEvent_t* stop) {
  *start = *stop = nullptr;
  if (id & kUntimed) return;
  std::lock_guard<std::mutex> lk(g_timing_mu);
  if (!g_timing_on) return;
  if (g_timing_used == g_timing_pool.size()) {
    TimingRecord r{id, nullptr, nullptr};
    if (hipEventCreate(&r.start) != hipSuccess) return;
    if (hipEventCreate(&r.stop) != hipSuccess) {
      (void)hipEventDestroy(r.start);
      return;
    }
    g_timing_pool.push_back(r);
  }
  TimingRecord& r = g_timing_pool[g_timing_used++];
  r.id = id;
  *start = r.start;
  *stop = r.stop;
}

}  // namespace lsh

extern "C" {

#ifdef LSH_CHECKED
// checked builds: the device word (uint32, caller-owned) that the next
// launches OR their violation bits into; NULL turns the checks off
void lsh_check_set(void* word) { lsh::g_check = static_cast<uint32_t*>(word); }
#endif

const char* lsh_status_string(int status) {
  switch (status) {
    case LSH_OK: return "LSH_OK";
    case LSH_ERR_INVALID_ARG: return "LSH_ERR_INVALID_ARG: invalid argument";
    case LSH_ERR_UNSUPPORTED: return "LSH_ERR_UNSUPPORTED: valid but unsupported shape or parameter";
    case LSH_ERR_WORKSPACE:
      return "LSH_ERR_WORKSPACE: workspace smaller than the size query (lsh_decode_attention_noalloc: the call "
             "needs more than the library's static scratch holds)";
    case LSH_ERR_HIP: return "LSH_ERR_HIP: HIP runtime or launch error";
    default: return "unknown lsh_status";
  }
}

int lsh_kernel_count(void) { return lsh::kKNumKernels; }

const char* lsh_kernel_name(int id) { return lsh::kernel_name(id); }

lsh_status lsh_timing_begin(void) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  if (g_timing_on) return LSH_ERR_INVALID_ARG;
  g_timing_on = true;
  g_timing_used = 0;
  return LSH_OK;
}

lsh_status lsh_timing_end(double* total_ms, int32_t* launches) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  if (!g_timing_on) return LSH_ERR_INVALID_ARG;
  g_timing_on = false;
  if (total_ms)
    for (int k = 0; k < lsh::kKNumKernels; ++k) total_ms[k] = 0.0;
  if (launches)
    for (int k = 0; k < lsh::kKNumKernels; ++k) launches[k] = 0;
  lsh_status st = LSH_OK;
  for (size_t i = 0; i < g_timing_used; ++i) {
    const TimingRecord& r = g_timing_pool[i];
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) {
      st = LSH_ERR_HIP;
      continue;
    }
    if (total_ms) total_ms[r.id] += ms;
    if (launches) launches[r.id] += 1;
  }
  g_timing_used = 0;
  return st;
}

int lsh_num_chunks(int N, int stride) {
  if (N < 1 || stride < 1) return 0;
  return static_cast<int>((static_cast<long long>(N) + stride - 1) / stride);
}

int lsh_default_stride(int N, int K) {
  if (N < 1 || K < 0 || K > 15) return 0;
  int stride = 1 << kMinStrideLog2;
  while (stride < (1 << kMaxStrideLog2) && stride < N) stride *= 2;
  return stride;
}

size_t lsh_build_workspace_size(int B, int Hkv, int N, int d, int K, int L, int stride, int dtype) {
  Geometry g;
  if (check_common(B, Hkv, N, d, K, L, stride, dtype, &g) != LSH_OK) return 0;
  return build_layout(B, Hkv, N, L, dtype, g, true).total;
}

lsh_status lsh_update_tables(const void* keys, const void* W, int B, int Hkv, int n_old, int n_new, int n_cap,
                             const int32_t* old_lens, const int32_t* new_lens, int d, int K, int L, int stride,
                             int dtype, int w_per_head, uint16_t* offsets, uint16_t* indices, uint16_t* key_codes,
                             void* workspace, size_t workspace_bytes, void* stream) {
  Geometry g;   // at capacity: the pitch of every per-key array and the offsets' chunk slots
  lsh_status st = check_common(B, Hkv, n_cap, d, K, L, stride, dtype, &g);
  if (st != LSH_OK) return st;
  if (n_old < 0 || n_old > n_new || n_new > n_cap) return LSH_ERR_INVALID_ARG;
  if (w_per_head != 0 && w_per_head != 1) return LSH_ERR_INVALID_ARG;
  if (!keys || !offsets || !indices || !workspace || (K > 0 && !W)) return LSH_ERR_INVALID_ARG;
  const BuildLayout w = build_layout(B, Hkv, n_cap, L, dtype, g, key_codes == nullptr);
  if (workspace_bytes < w.total) return LSH_ERR_WORKSPACE;
  if (n_old == n_new) return LSH_OK;
  char* ws = static_cast<char*>(workspace);
  lsh::BuildArgs a;
  a.keys = keys;
  a.W = W;
  a.wt = ws + w.wt;
  a.codes = key_codes ? key_codes : reinterpret_cast<uint16_t*>(ws + w.codes);
  a.offsets = offsets;
  a.indices = indices;
  a.old_lens = old_lens;
  a.new_lens = new_lens;
  a.U = B * Hkv;
  a.Hkv = Hkv;
  a.w_heads = w_per_head ? Hkv : 1;
  a.N = n_new;
  a.K = K;
  a.L = L;
  a.P = n_cap;
  a.nJP = g.nJ;
  // the chunk that key n_old falls into and every later one are rebuilt
  // from their keys; earlier chunks are complete and left as they are
  a.j0 = n_old >> g.stride_log2;
  a.stride_log2 = g.stride_log2;
  a.nJ = lsh_num_chunks(n_new, stride);
  a.dtype = dtype;
  // a few keys appended to built tables are inserted into their chunks, the
  // rest re-sorted with their chunks; each sequence's kernels take the same
  // choice from its lengths, so only when the bounds settle it for every
  // sequence is one of the two launches left out
  a.n_old = n_old;
  if (n_old > 0 && n_new - n_old <= lsh::kInsertMax) a.mode = lsh::kUpdateInsert;
  else if (!old_lens && !new_lens) a.mode = lsh::kUpdateSort;
  else a.mode = lsh::kUpdateSort | lsh::kUpdateInsert;
  return hip_status(lsh::launch_build(a, static_cast<hipStream_t>(stream)));
}

lsh_status lsh_build_tables(const void* keys, const void* W, int B, int Hkv, int N, int d, int K, int L,
                            int stride, int dtype, uint16_t* offsets, uint16_t* indices, uint16_t* key_codes,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return lsh_update_tables(keys, W, B, Hkv, 0, N, N, nullptr, nullptr, d, K, L, stride, dtype, 0, offsets, indices,
                           key_codes, workspace, workspace_bytes, stream);
}

size_t lsh_decode_workspace_size(int B, int Hq, int Hkv, int N, int d, int K, int L, int stride) {
  Geometry g;
  if (check_common(B, Hkv, N, d, K, L, stride, LSH_BF16, &g) != LSH_OK) return 0;
  if (Hq < 1 || Hq % Hkv != 0 || Hq / Hkv > 16) return 0;
  return decode_layout(B, Hq, Hkv, N, L, g).total;
}

static lsh_status decode_cached(const void* q, const void* keys, const void* values, const void* W,
                                const uint16_t* indices, const uint16_t* offsets, int B, int Hq, int Hkv, int N,
                                int n_cap, const int32_t* seq_lens, int d, int K, int L, int T, int stride,
                                float sm_scale, int dtype, int w_per_head, int n_sink, int n_window, float* out,
                                float* lse, int32_t* nsel, uint16_t* q_codes, uint8_t* counts, void* workspace,
                                size_t workspace_bytes, void* stream, bool noalloc) {
  Geometry g, gcap;
  lsh_status st = check_common(B, Hkv, N, d, K, L, stride, dtype, &g);
  if (st != LSH_OK) return st;
  if (n_cap < N) return LSH_ERR_INVALID_ARG;
  st = check_common(B, Hkv, n_cap, d, K, L, stride, dtype, &gcap);
  if (st != LSH_OK) return st;
  if (Hq < 1 || Hq % Hkv != 0 || T < 1 || T > L || !std::isfinite(sm_scale)) return LSH_ERR_INVALID_ARG;
  if (n_sink < 0 || n_window < 0) return LSH_ERR_INVALID_ARG;
  if (w_per_head != 0 && w_per_head != 1) return LSH_ERR_INVALID_ARG;
  if (Hq / Hkv > 16) return LSH_ERR_UNSUPPORTED;
  if (!q || !keys || !values || !indices || !offsets || !out || (!noalloc && !workspace) || (K > 0 && !W))
    return LSH_ERR_INVALID_ARG;
  const DecodeLayout w = decode_layout(B, Hq, Hkv, N, L, g);
  if (workspace_bytes < w.total) return LSH_ERR_WORKSPACE;
  if (noalloc) {
    // every argument checked: only now the device's scratch address
    st = scratch_address(&workspace);
    if (st != LSH_OK) return st;
  }
  char* ws = static_cast<char*>(workspace);
  lsh::DecodeArgs a;
  a.q = q;
  a.keys = keys;
  a.values = values;
  a.W = W;
  a.indices = indices;
  a.offsets = offsets;
  a.qcodes = q_codes ? q_codes : reinterpret_cast<uint16_t*>(ws + w.qcodes);
  a.bitmask = reinterpret_cast<uint32_t*>(ws + w.bitmask);
  a.chunk_nsel = reinterpret_cast<int32_t*>(ws + w.chunk_nsel);
  a.lnu_samples = reinterpret_cast<double*>(ws + w.lnu);
  a.partials = reinterpret_cast<float*>(ws + w.partials);
  a.sync = reinterpret_cast<int32_t*>(ws + w.sync);
  a.out = out;
  a.lse = lse;
  a.nsel = nsel;
  a.counts = counts;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.N = N;
  a.K = K;
  a.L = L;
  a.T = T;
  a.P = n_cap;
  a.nJP = gcap.nJ;
  a.stride_log2 = g.stride_log2;
  a.nJ = g.nJ;
  a.split_len = w.split_len;
  a.nsplit = w.nsplit;
  a.scale = sm_scale;
  a.dtype = dtype;
  a.seq_lens = seq_lens;
  a.w_heads = w_per_head ? Hkv : 1;
  a.n_sink = n_sink;
  a.n_window = n_window;
  // the no-alloc path takes no timing events: the pool of events grows while
  // a timing window is open
  a.timed = !noalloc;
  // (the context splits take the exact set's keys themselves: every head of
  // the group, ln u = 0)
  return hip_status(lsh::launch_decode(a, static_cast<hipStream_t>(stream)));
}

lsh_status lsh_decode_attention_cached(const void* q, const void* keys, const void* values, const void* W,
                                       const uint16_t* indices, const uint16_t* offsets, int B, int Hq, int Hkv,
                                       int N, int n_cap, const int32_t* seq_lens, int d, int K, int L, int T,
                                       int stride, float sm_scale, int dtype, int w_per_head, int n_sink,
                                       int n_window, float* out, float* lse, int32_t* nsel, uint16_t* q_codes,
                                       uint8_t* counts, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_cached(q, keys, values, W, indices, offsets, B, Hq, Hkv, N, n_cap, seq_lens, d, K, L, T, stride,
                       sm_scale, dtype, w_per_head, n_sink, n_window, out, lse, nsel, q_codes, counts, workspace,
                       workspace_bytes, stream, false);
}

lsh_status lsh_decode_attention_noalloc(const void* q, const void* keys, const void* values, const void* W,
                                        const uint16_t* indices, const uint16_t* offsets, int B, int Hq, int Hkv,
                                        int N, int n_cap, const int32_t* seq_lens, int d, int K, int L, int T,
                                        int stride, float sm_scale, int dtype, int w_per_head, int n_sink,
                                        int n_window, float* out, float* lse, int32_t* nsel, uint16_t* q_codes,
                                        uint8_t* counts, void* stream) {
  // the scratch takes the workspace's part: a call that needs more than it
  // holds is refused (LSH_ERR_WORKSPACE) before anything is launched
  return decode_cached(q, keys, values, W, indices, offsets, B, Hq, Hkv, N, n_cap, seq_lens, d, K, L, T, stride,
                       sm_scale, dtype, w_per_head, n_sink, n_window, out, lse, nsel, q_codes, counts, nullptr,
                       LSH_NOALLOC_SCRATCH_BYTES, stream, true);
}

lsh_status lsh_decode_attention_hybrid(const void* q, const void* keys, const void* values, const void* W,
                                       const uint16_t* indices, const uint16_t* offsets, int B, int Hq, int Hkv,
                                       int N, int d, int K, int L, int T, int stride, float sm_scale, int dtype,
                                       int n_sink, int n_window, float* out, float* lse, int32_t* nsel,
                                       uint16_t* q_codes, uint8_t* counts, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  return lsh_decode_attention_cached(q, keys, values, W, indices, offsets, B, Hq, Hkv, N, N, nullptr, d, K, L, T,
                                     stride, sm_scale, dtype, 0, n_sink, n_window, out, lse, nsel, q_codes, counts,
                                     workspace, workspace_bytes, stream);
}

lsh_status lsh_decode_attention(const void* q, const void* keys, const void* values, const void* W,
                                const uint16_t* indices, const uint16_t* offsets, int B, int Hq, int Hkv, int N,
                                int d, int K, int L, int T, int stride, float sm_scale, int dtype, float* out,
                                float* lse, int32_t* nsel, uint16_t* q_codes, uint8_t* counts, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return lsh_decode_attention_hybrid(q, keys, values, W, indices, offsets, B, Hq, Hkv, N, d, K, L, T, stride,
                                     sm_scale, dtype, 0, 0, out, lse, nsel, q_codes, counts, workspace,
                                     workspace_bytes, stream);
}

}  // extern "C"
