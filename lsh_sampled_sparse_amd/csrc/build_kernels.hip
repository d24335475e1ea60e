// Table-build kernels (prefill side) for gfx950.
//
// MagicPIG builds per-table hash buckets of the keys at prefill and names an
// optimised hash-table construction (MagicPIG project summary on sourcepulse,
// "Highlighted Details").  Here the build is:
//   transpose_w     W [d, L*K] -> WT [LKpad, d] (zero-padded columns), so that
//                   a projection column is one contiguous row
//   project_codes   SimHash codes of every key: a dense bf16 (or fp32) MFMA
//                   contraction keys x W with fp32 accumulation, sign bits
//                   packed with wave ballots, codes written table-major
//   chunk_sort      per (table, key chunk): a stable counting sort of the
//                   chunk's keys by code into the chunk's own region of the
//                   index array, with the chunk's bucket offsets
#include "lsh_device.h"
#include "lsh_kernels.h"

namespace lsh {

// ---------------------------------------------------------------------------
// Projection layout.
//
// The projection is D = W^T K on MFMA 16x16 tiles whose rows are projection
// columns and whose columns are keys.  In such a tile lane (g, n) (g = lane /
// 16) holds rows 4 g .. 4 g + 3 for key n.  A slab is NCT tiles of rows, so
// every lane group g owns P = 4 NCT rows of the slab, and the rows are
// assigned so that those P rows are the K columns of TPG whole tables: each
// lane then packs the codes of its key from its own accumulators, with no
// data exchanged between lanes.  NCT (at most 8) is chosen per K to waste as
// few rows as possible; the transposed, permuted W (WT, zero rows for the
// unused positions) lives in the build workspace.
// ---------------------------------------------------------------------------
struct ProjShape {
  int nct, tpg;
};
__host__ __device__ constexpr ProjShape proj_shape(int K) {
  switch (K) {
    case 1: return {1, 4};
    case 2: return {1, 2};
    case 3: return {3, 4};
    case 4: return {1, 1};
    case 5: return {5, 4};
    case 6: return {3, 2};
    case 7: return {7, 4};
    case 8: return {2, 1};
    case 9: return {7, 3};
    case 10: return {5, 2};
    case 11: return {3, 1};
    case 12: return {3, 1};
    case 13: return {7, 2};
    case 14: return {7, 2};
    case 15: return {4, 1};
    default: return {1, 1};
  }
}

int proj_wt_rows(int K, int L) {
  if (K <= 0) return 0;
  const ProjShape ps = proj_shape(K);
  const int tps = 4 * ps.tpg;
  return (L + tps - 1) / tps * ps.nct * 16;
}

// WT[R][d] for row R = (slab, tile ct, row r = 4 g + i).  The kernel below
// shifts the signs of a lane group's positions j = 4 ct + i into a word in
// increasing j, so position j lands on bit P - 1 - j; that bit is bit b of
// table tt of the group when P - 1 - j = tt K + b, i.e. table
// slab * 4 TPG + g * TPG + tt.
template <typename T>
__global__ void transpose_w_kernel(const typename T::storage* __restrict__ W,
                                   typename T::storage* __restrict__ WT, int K, int L, int nct, int tpg,
                                   int rows) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * kHeadDim) return;
  const int R = idx / kHeadDim, d = idx % kHeadDim;
  const int slab = R / (nct * 16), p = R % (nct * 16);
  const int ct = p / 16, r = p % 16;
  const int g = r / 4, j = ct * 4 + r % 4;
  const int jr = 4 * nct - 1 - j;
  const int tt = jr / K, b = jr % K;
  const int t = slab * 4 * tpg + g * tpg + tt;
  const bool valid = tt < tpg && t < L;
  WT[idx] = valid ? W[static_cast<size_t>(d) * L * K + t * K + b] : typename T::storage(0);
}

constexpr int kProjThreads = 256;              // 4 waves
constexpr int kProjKeys = 256;                 // 64 keys per wave = 4 tiles of 16

// codes[u][l][n] for this workgroup's 256 keys.
template <typename T, int KB>
__global__ __launch_bounds__(kProjThreads) void project_codes_kernel(
    const typename T::storage* __restrict__ keys,   // [U][N][128]
    const typename T::storage* __restrict__ WT,     // [nslab * NCT * 16][128], permuted
    uint16_t* __restrict__ codes,                   // [U][L][N]
    int N, int L, int nslab) {
  using S = typename T::storage;
  constexpr ProjShape PS = proj_shape(KB);
  constexpr int NCT = PS.nct, TPG = PS.tpg, TPS = 4 * TPG;
  constexpr int kRows = NCT * 16;                                  // WT rows per slab
  constexpr int kRow = kHeadDim + 16 / T::bytes;                   // padded LDS row
  constexpr int kChunksPerRow = kHeadDim * T::bytes / 16;
  constexpr int kCPT = kRows * kChunksPerRow / kProjThreads;       // 16-byte pieces per thread
  constexpr uint32_t kMask = (1u << KB) - 1u;
  __shared__ __attribute__((aligned(16))) S wt[2][kRows * kRow];

  const int u = blockIdx.y;
  const int n0 = blockIdx.x * kProjKeys;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4;
  const S* kb = keys + static_cast<size_t>(u) * N * kHeadDim;
  uint16_t* cb = codes + static_cast<size_t>(u) * L * N;

  // key fragments (MFMA B operand): lane holds key lane & 15 of tile a, dims
  // [32 g, 32 g + 32)
  Frag<T> A[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int key = n0 + wave * 64 + a * 16 + (lane & 15);
    const bool valid = key < N;
    A[a].load(kb + static_cast<size_t>(valid ? key : 0) * kHeadDim + g * 32, valid);
  }

  u32x4_t pre[kCPT];
  auto fetch = [&](int slab) {
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(WT + static_cast<size_t>(slab) * kRows * kHeadDim);
#pragma unroll
    for (int k = 0; k < kCPT; ++k) pre[k] = src[tid + k * kProjThreads];
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int k = 0; k < kCPT; ++k) {
      const int chunk = tid + k * kProjThreads;
      *reinterpret_cast<u32x4_t*>(&wt[buf][(chunk / kChunksPerRow) * kRow +
                                          (chunk % kChunksPerRow) * (16 / T::bytes)]) = pre[k];
    }
  };
  fetch(0);
  stash(0);
  __syncthreads();

  for (int s = 0; s < nslab; ++s) {
    const int buf = s & 1;
    if (s + 1 < nslab) fetch(s + 1);
    // sign bits of the P rows of lane group g, for this lane's key in each
    // tile, shifted in row order (s = 2 s + [x > 0]).  The column-tile loop is
    // kept rolled: four accumulators are live at a time, which leaves room for
    // several waves per SIMD to overlap one wave's MFMAs with another's signs.
    uint32_t sg[4] = {0u, 0u, 0u, 0u};
#pragma unroll 1
    for (int ct = 0; ct < NCT; ++ct) {
      Frag<T> Wf;
      Wf.load(&wt[buf][(ct * 16 + (lane & 15)) * kRow + g * 32], true);
      floatx4_t acc[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        acc[a] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        acc[a] = Wf.mma(A[a], acc[a]);   // acc[a][i]: row 4 g + i, key lane & 15 of tile a
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) sg[a] = sg[a] * 2u + (acc[a][i] > 0.f ? 1u : 0u);
    }
    if (s + 1 < nslab) stash(buf ^ 1);
    // codes of tables s * TPS + g * TPG + tt
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int key = n0 + wave * 64 + a * 16 + (lane & 15);
      if (key < N) {
#pragma unroll
        for (int tt = 0; tt < TPG; ++tt) {
          const int t = s * TPS + g * TPG + tt;
          if (t < L) cb[static_cast<size_t>(t) * N + key] = static_cast<uint16_t>((sg[a] >> (tt * KB)) & kMask);
        }
      }
    }
    __syncthreads();
  }
}

// K = 0: every code is 0.
__global__ void zero_codes_kernel(uint16_t* __restrict__ codes, size_t n) {
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) codes[i] = 0;
}

// ---------------------------------------------------------------------------
// Bucketing: a stable counting sort of every (table, key chunk) by code.
//
// Output format (chunk-major two-level CSR): chunk j of table l covers keys
// [j stride, (j + 1) stride) and owns positions [j stride, (j + 1) stride)
// of the table's index array; there its keys are sorted by code, ascending
// key inside a code, each stored as (key - j stride).  offsets[j][c] is the
// start of bucket c inside the chunk's region, so bucket c of chunk j is
// positions offsets[j][c] .. offsets[j][c + 1] (the chunk's length for the
// last bucket).  No scan crosses chunks, so every (table, chunk) is sorted by
// one workgroup, and its region is written contiguously.
// ---------------------------------------------------------------------------
constexpr int kSortThreads = 512;
constexpr int kSortWaves = kSortThreads / 64;
constexpr int kSortBatches = 16;        // 64-key batches per wave: chunks of <= 8192 keys
constexpr int kMatchLo = 8;             // code bits matched through the LDS lane-mask table

// Mask of the valid lanes of this wave whose code equals this lane's, in two
// steps: a per-wave LDS table of 64-bit lane masks indexed by the low 8 code
// bits (every lane ORs its bit into its entry and reads the entry back; LDS
// operations of one wave are performed in issue order; the entry is cleared
// afterwards), then one ballot per remaining code bit.
__device__ __forceinline__ uint64_t match_lanes(int code, bool valid, int K, uint64_t* mt, int lane) {
  volatile uint64_t* vt = mt;
  const int lo = code & ((1 << kMatchLo) - 1);
  if (valid) atomicOr(reinterpret_cast<unsigned long long*>(&mt[lo]), 1ull << lane);
  __builtin_amdgcn_wave_barrier();
  uint64_t m = valid ? vt[lo] : 0ull;
  __builtin_amdgcn_wave_barrier();
  if (valid) vt[lo] = 0ull;
  for (int b = kMatchLo; b < K; ++b) {
    const bool bit = (code >> b) & 1;
    const uint64_t B = ballot(bit);
    m &= bit ? B : ~B;
  }
  return m;
}

// One workgroup (8 waves) per (table, chunk); K <= 12 so the per-wave
// histograms fit.  Each wave owns a contiguous eighth of the chunk and walks
// it in batches of 64 keys held in registers.  A lane's rank is the number of
// lanes below it with its code, so buckets keep the key order.
//   phase 1  per-wave histograms (the first lane of each code adds the count)
//   phase 2  scan: bucket starts in the chunk (the offsets output) and each
//            wave's cursor in each bucket
//   phase 3  placement into the chunk's sorted list in LDS
//   phase 4  the list is written to the chunk's region, lane i to position i
__global__ __launch_bounds__(kSortThreads) void chunk_sort_kernel(
    const uint16_t* __restrict__ codes,   // [U][L][N]
    int N, int K, int stride_log2, int nJ,
    uint16_t* __restrict__ offsets,       // [U][L][nJ][2^K]
    uint16_t* __restrict__ indices) {     // [U][L][N]
  extern __shared__ __attribute__((aligned(16))) uint64_t smem64[];
  const int nb = 1 << K;
  constexpr int kMt = 1 << kMatchLo;
  uint64_t* mt = smem64;                                               // [kSortWaves][256] lane masks
  uint16_t* buf = reinterpret_cast<uint16_t*>(mt + kSortWaves * kMt);  // [chunk] key - chunk start
  uint16_t* wh = buf + (1 << stride_log2);                             // [kSortWaves][nb] counts, cursors
  __shared__ int32_t wave_tot[kSortWaves];

  const int j = blockIdx.x;
  const size_t table = blockIdx.y;      // u * L + l
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cbeg = j << stride_log2;
  const int clen = min(1 << stride_log2, N - cbeg);
  const uint16_t* cd = codes + table * N + cbeg;

  for (int i = tid; i < kSortWaves * kMt; i += kSortThreads) mt[i] = 0ull;
  for (int i = tid; i < kSortWaves * nb; i += kSortThreads) wh[i] = 0;
  // this wave's keys: batch k = chunk keys wbeg + 64 k + lane, below wend
  const int per = (1 << stride_log2) / kSortWaves;
  const int wbeg = wave * per;
  const int wend = min(clen, wbeg + per);
  int cr[kSortBatches];
#pragma unroll
  for (int k = 0; k < kSortBatches; ++k) {
    const int n = wbeg + 64 * k + lane;
    cr[k] = (64 * k < per && n < wend) ? static_cast<int>(cd[n]) : -1;
  }
  __syncthreads();

  uint64_t* my_mt = mt + wave * kMt;
  volatile uint16_t* vwh = wh + wave * nb;
  int rs[kSortBatches];                 // rank | count << 8 of this lane's key in its batch
#pragma unroll
  for (int k = 0; k < kSortBatches; ++k) {
    rs[k] = 0;
    if (64 * k >= per) continue;        // wave-uniform: chunks shorter than 8192 keys
    const bool valid = cr[k] >= 0;
    const int code = valid ? cr[k] : 0;
    const uint64_t m = match_lanes(code, valid, K, my_mt, lane);
    const int rank = mbcnt(m), cnt = __builtin_popcountll(m);
    rs[k] = rank | (cnt << 8);
    if (valid && rank == 0) vwh[code] = static_cast<uint16_t>(vwh[code] + cnt);
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();

  // phase 2
  uint16_t* off = offsets + (table * nJ + j) * nb;
  const int bpt = (nb + kSortThreads - 1) / kSortThreads;
  const int c0 = tid * bpt, c1 = min(nb, c0 + bpt);
  int local = 0;
  for (int c = c0; c < c1; ++c)
    for (int w = 0; w < kSortWaves; ++w) local += wh[w * nb + c];
  int incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int run = incl - local;
  for (int w = 0; w < wave; ++w) run += wave_tot[w];
  for (int c = c0; c < c1; ++c) {
    off[c] = static_cast<uint16_t>(run);
    for (int w = 0; w < kSortWaves; ++w) {
      const int x = wh[w * nb + c];
      wh[w * nb + c] = static_cast<uint16_t>(run);
      run += x;
    }
  }
  __syncthreads();

  // phase 3
#pragma unroll
  for (int k = 0; k < kSortBatches; ++k) {
    if (64 * k >= per) continue;
    const bool valid = cr[k] >= 0;
    const int code = valid ? cr[k] : 0;
    const int rank = rs[k] & 0xff, cnt = rs[k] >> 8;
    const int p = valid ? static_cast<int>(vwh[code]) : 0;
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      buf[p + rank] = static_cast<uint16_t>(wbeg + 64 * k + lane);
      if (rank == 0) vwh[code] = static_cast<uint16_t>(p + cnt);
    }
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();

  // phase 4: two entries per lane, 4-byte stores when the region allows it
  uint16_t* out = indices + table * N + cbeg;
  if ((N & 1) == 0) {
    const uint32_t* b2 = reinterpret_cast<const uint32_t*>(buf);
    uint32_t* o2 = reinterpret_cast<uint32_t*>(out);
    for (int e = tid; e < (clen >> 1); e += kSortThreads) o2[e] = b2[e];
    if ((clen & 1) && tid == 0) out[clen - 1] = buf[clen - 1];
  } else {
    for (int e = tid; e < clen; e += kSortThreads) out[e] = buf[e];
  }
}

size_t chunk_sort_lds_bytes(int K, int stride_log2) {
  const size_t nb = size_t(1) << K;
  return kSortWaves * (size_t(1) << kMatchLo) * 8 + (size_t(2) << stride_log2) + kSortWaves * nb * 2;
}

// Any K (up to 15): one wave per (table, chunk) walks the chunk twice from
// global memory: histogram, scan, then placement with the same rank rule.
constexpr int kSortOneThreads = 64;

__global__ __launch_bounds__(kSortOneThreads) void chunk_sort_one_kernel(
    const uint16_t* __restrict__ codes, int N, int K, int stride_log2, int nJ,
    uint16_t* __restrict__ offsets, uint16_t* __restrict__ indices) {
  extern __shared__ __attribute__((aligned(16))) uint64_t smem64[];
  const int nb = 1 << K;
  constexpr int kMt = 1 << kMatchLo;
  uint64_t* mt = smem64;                                      // [256]
  uint16_t* buf = reinterpret_cast<uint16_t*>(mt + kMt);      // [chunk]
  uint16_t* cur = buf + (1 << stride_log2);                   // [nb]
  const int j = blockIdx.x;
  const size_t table = blockIdx.y;
  const int lane = threadIdx.x;
  const int cbeg = j << stride_log2;
  const int clen = min(1 << stride_log2, N - cbeg);
  const uint16_t* cd = codes + table * N + cbeg;
  volatile uint16_t* vcur = cur;

  for (int i = lane; i < kMt; i += 64) mt[i] = 0ull;
  for (int i = lane; i < nb; i += 64) cur[i] = 0;
  __syncthreads();
  for (int b = 0; b < clen; b += 64) {
    const int n = b + lane;
    const bool valid = n < clen;
    const int code = valid ? static_cast<int>(cd[n]) : 0;
    const uint64_t m = match_lanes(code, valid, K, mt, lane);
    if (valid && mbcnt(m) == 0) vcur[code] = static_cast<uint16_t>(vcur[code] + __builtin_popcountll(m));
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  uint16_t* off = offsets + (table * nJ + j) * nb;
  int base = 0;
  for (int c0 = 0; c0 < nb; c0 += 64) {
    const int c = c0 + lane;
    const int x = c < nb ? static_cast<int>(cur[c]) : 0;
    int incl = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    if (c < nb) {
      off[c] = static_cast<uint16_t>(base + incl - x);
      cur[c] = static_cast<uint16_t>(base + incl - x);
    }
    base += __shfl(incl, 63);
  }
  __syncthreads();
  for (int b = 0; b < clen; b += 64) {
    const int n = b + lane;
    const bool valid = n < clen;
    const int code = valid ? static_cast<int>(cd[n]) : 0;
    const uint64_t m = match_lanes(code, valid, K, mt, lane);
    const int rank = mbcnt(m);
    const int p = valid ? static_cast<int>(vcur[code]) : 0;
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      buf[p + rank] = static_cast<uint16_t>(n);
      if (rank == 0) vcur[code] = static_cast<uint16_t>(p + __builtin_popcountll(m));
    }
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  uint16_t* out = indices + table * N + cbeg;
  for (int e = lane; e < clen; e += 64) out[e] = buf[e];
}

size_t chunk_sort_one_lds_bytes(int K, int stride_log2) {
  return (size_t(1) << kMatchLo) * 8 + (size_t(2) << stride_log2) + (size_t(2) << K);
}

// ---------------------------------------------------------------------------
// Host-side launchers
// ---------------------------------------------------------------------------
template <typename T, int KB>
static hipError_t launch_project_k(const void* keys, const void* WT, uint16_t* codes, int U, int N, int L,
                                   int nslab, hipStream_t stream) {
  using S = typename T::storage;
  return launch(kKProject, project_codes_kernel<T, KB>, dim3((N + kProjKeys - 1) / kProjKeys, U),
                dim3(kProjThreads), 0, stream, static_cast<const S*>(keys), static_cast<const S*>(WT), codes, N,
                L, nslab);
}

template <typename T>
static hipError_t launch_project(const void* keys, const void* W, void* WT, uint16_t* codes,
                                 int U, int N, int K, int L, hipStream_t stream) {
  using S = typename T::storage;
  if (K == 0) {
    const size_t n = static_cast<size_t>(U) * L * N;
    return launch(kKProject, zero_codes_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream,
                  codes, n);
  }
  const ProjShape ps = proj_shape(K);
  const int rows = proj_wt_rows(K, L);
  const int nslab = rows / (ps.nct * 16);
  hipError_t e = launch(kKTransposeW, transpose_w_kernel<T>, dim3((rows * kHeadDim + 255) / 256), dim3(256), 0,
                        stream, static_cast<const S*>(W), static_cast<S*>(WT), K, L, ps.nct, ps.tpg, rows);
  if (e != hipSuccess) return e;
  switch (K) {
    case 1: return launch_project_k<T, 1>(keys, WT, codes, U, N, L, nslab, stream);
    case 2: return launch_project_k<T, 2>(keys, WT, codes, U, N, L, nslab, stream);
    case 3: return launch_project_k<T, 3>(keys, WT, codes, U, N, L, nslab, stream);
    case 4: return launch_project_k<T, 4>(keys, WT, codes, U, N, L, nslab, stream);
    case 5: return launch_project_k<T, 5>(keys, WT, codes, U, N, L, nslab, stream);
    case 6: return launch_project_k<T, 6>(keys, WT, codes, U, N, L, nslab, stream);
    case 7: return launch_project_k<T, 7>(keys, WT, codes, U, N, L, nslab, stream);
    case 8: return launch_project_k<T, 8>(keys, WT, codes, U, N, L, nslab, stream);
    case 9: return launch_project_k<T, 9>(keys, WT, codes, U, N, L, nslab, stream);
    case 10: return launch_project_k<T, 10>(keys, WT, codes, U, N, L, nslab, stream);
    case 11: return launch_project_k<T, 11>(keys, WT, codes, U, N, L, nslab, stream);
    case 12: return launch_project_k<T, 12>(keys, WT, codes, U, N, L, nslab, stream);
    case 13: return launch_project_k<T, 13>(keys, WT, codes, U, N, L, nslab, stream);
    case 14: return launch_project_k<T, 14>(keys, WT, codes, U, N, L, nslab, stream);
    case 15: return launch_project_k<T, 15>(keys, WT, codes, U, N, L, nslab, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_build(const BuildArgs& a, hipStream_t stream) {
  hipError_t e = (a.dtype == 1)
      ? launch_project<BF16>(a.keys, a.W, a.wt, a.codes, a.U, a.N, a.K, a.L, stream)
      : launch_project<F32>(a.keys, a.W, a.wt, a.codes, a.U, a.N, a.K, a.L, stream);
  if (e != hipSuccess) return e;
  const dim3 grid(a.nJ, a.U * a.L);
  if (a.K <= 12) {
    const size_t lds = chunk_sort_lds_bytes(a.K, a.stride_log2);
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(chunk_sort_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    return launch(kKChunkSort, chunk_sort_kernel, grid, dim3(kSortThreads), static_cast<unsigned>(lds), stream,
                  static_cast<const uint16_t*>(a.codes), a.N, a.K, a.stride_log2, a.nJ, a.offsets, a.indices);
  }
  const size_t lds = chunk_sort_one_lds_bytes(a.K, a.stride_log2);
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(chunk_sort_one_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  return launch(kKChunkSort, chunk_sort_one_kernel, grid, dim3(kSortOneThreads), static_cast<unsigned>(lds), stream,
                static_cast<const uint16_t*>(a.codes), a.N, a.K, a.stride_log2, a.nJ, a.offsets, a.indices);
}

}  // namespace lsh
