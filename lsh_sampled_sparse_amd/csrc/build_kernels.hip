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
//   bucket_tables   per (unit, table): sub-chunk histograms, a scan that
//                   yields the CSR offsets and the chunk bounds, and a stable
//                   scatter of key indices (ascending inside each bucket)
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
// Per-table stable bucketing: a counting sort of key indices by code.
//
// Output format: bucket c of table l occupies positions offsets[c] ..
// offsets[c + 1] of the table's index array, split by key chunk (chunk j =
// keys [j stride, (j + 1) stride)) at bounds[c][j]; inside a bucket the keys
// ascend, and each entry stores the key's index relative to its chunk start,
// which fits 16 bits because stride <= 65536.
//
// Fast path (K <= 10), two kernels over tiles of at most 8192 keys that nest
// in the chunks:
//   bucket_count    one workgroup per table: per-tile histograms in LDS, one
//                   scan over (bucket, tile) that writes the offsets, the chunk
//                   bounds and every tile's start position in every bucket
//   bucket_scatter  one workgroup per tile: a stable counting sort of the
//                   tile in LDS (per-wave histograms for the order across
//                   waves, an LDS match table for the order inside a wave),
//                   then every bucket's run of the tile is written with
//                   consecutive lanes on consecutive addresses.
// General path (any K up to 15): bucket_tables, one workgroup per table that
// scatters straight to global memory.
// ---------------------------------------------------------------------------
constexpr int kPrefetch = 8;            // 64-key batches whose codes are loaded ahead

// -------- fast path: histogram + scan
constexpr int kCountTThreads = 512;

__global__ __launch_bounds__(kCountTThreads) void bucket_count_kernel(
    const uint16_t* __restrict__ codes,   // [U][L][N]
    int N, int K, int L, int tile_log2, int ntiles, int nJ, int tpc_log2,
    int32_t* __restrict__ offsets,        // [U][L][2^K + 1]
    int32_t* __restrict__ bounds,         // [U][L][2^K][nJ + 1]
    int32_t* __restrict__ tstart) {       // [U][L][ntiles][2^K]
  extern __shared__ __attribute__((aligned(16))) int32_t hist[];   // [ntiles][nb]
  __shared__ int32_t wave_tot[kCountTThreads / 64];
  const int nb = 1 << K;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l = blockIdx.x, u = blockIdx.y;
  const size_t tbl = static_cast<size_t>(u) * L + l;
  const uint16_t* cd = codes + tbl * N;

  for (int i = tid; i < ntiles * nb; i += kCountTThreads) hist[i] = 0;
  __syncthreads();
  if ((N & 7) == 0) {
    // 16-byte loads: 8 codes of one tile per lane (tiles hold >= 256 keys)
    const u32x4_t* cv = reinterpret_cast<const u32x4_t*>(cd);
    const int nv = N >> 3;
    for (int v0 = tid; v0 < nv; v0 += kCountTThreads * 4) {
      u32x4_t pf[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int v = v0 + k * kCountTThreads;
        pf[k] = v < nv ? cv[v] : u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int v = v0 + k * kCountTThreads;
        if (v < nv) {
          int32_t* h = hist + ((v << 3) >> tile_log2) * nb;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            atomicAdd(&h[pf[k][j] & 0xffffu], 1);
            atomicAdd(&h[pf[k][j] >> 16], 1);
          }
        }
      }
    }
  } else {
    for (int n0 = tid; n0 < N; n0 += kCountTThreads * kPrefetch) {
      int pf[kPrefetch];
#pragma unroll
      for (int k = 0; k < kPrefetch; ++k) {
        const int n = n0 + k * kCountTThreads;
        pf[k] = n < N ? static_cast<int>(cd[n]) : -1;
      }
#pragma unroll
      for (int k = 0; k < kPrefetch; ++k) {
        const int n = n0 + k * kCountTThreads;
        if (pf[k] >= 0) atomicAdd(&hist[(n >> tile_log2) * nb + pf[k]], 1);
      }
    }
  }
  __syncthreads();

  const int bpt = (nb + kCountTThreads - 1) / kCountTThreads;   // buckets per thread
  const int c0 = tid * bpt, c1 = min(nb, c0 + bpt);
  int local = 0;
  for (int c = c0; c < c1; ++c)
    for (int t = 0; t < ntiles; ++t) local += hist[t * nb + c];
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
  int32_t* off = offsets + tbl * (nb + 1);
  int32_t* ts = tstart + tbl * ntiles * nb;
  for (int c = c0; c < c1; ++c) {
    off[c] = run;
    int32_t* bnd = bounds + (tbl * nb + c) * (nJ + 1);
    for (int t = 0; t < ntiles; ++t) {
      if ((t & ((1 << tpc_log2) - 1)) == 0) bnd[t >> tpc_log2] = run;
      ts[t * nb + c] = run;
      run += hist[t * nb + c];
    }
    bnd[nJ] = run;
  }
  if (tid == 0) off[nb] = N;
}

// -------- fast path: per-tile stable scatter
constexpr int kScatThreads = 512;
constexpr int kScatWaves = kScatThreads / 64;
constexpr int kScatBatches = 16;        // 64-key batches per wave: tiles of <= 8192 keys
constexpr int kMaxTileLog2 = 13;
constexpr int kMatchLo = 8;             // code bits matched through the LDS lane-mask table

// One workgroup per tile.  Each wave owns a contiguous eighth of the tile and
// walks it in batches of 64 keys.  The lanes of a batch holding the same code
// are found in two steps: a per-wave LDS table of 64-bit lane masks indexed by
// the low 8 code bits (every lane ORs its bit into its entry and reads the
// entry back; LDS operations of one wave are performed in issue order; the
// entry is cleared afterwards), then one ballot per remaining code bit.  A
// lane's rank is the number of matching lanes below it, so the order inside a
// bucket is the key order.
//   phase 1  per-wave histograms (the first lane of each code adds the count)
//   phase 2  scan: tile-local start of each bucket, per-wave cursors, and the
//            shift from tile-local to table position of each bucket
//   phase 3  placement into the tile's local CSR in LDS (key and code packed)
//   phase 4  the runs are written with consecutive lanes on consecutive
//            addresses of the table's index array
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

__global__ __launch_bounds__(kScatThreads) void bucket_scatter_kernel(
    const uint16_t* __restrict__ codes,   // [U][L][N]
    const int32_t* __restrict__ tstart,   // [U][L][ntiles][2^K]
    int N, int K, int L, int tile_log2, int ntiles, int stride_log2, int tables,
    uint16_t* __restrict__ indices) {     // [U][L][N]
  extern __shared__ __attribute__((aligned(16))) uint64_t smem64[];
  const int nb = 1 << K;
  const int T = 1 << tile_log2;
  constexpr int kMt = 1 << kMatchLo;
  uint64_t* mt = smem64;                                               // [kScatWaves][256] lane masks
  int32_t* delta = reinterpret_cast<int32_t*>(mt + kScatWaves * kMt);   // [nb]
  uint32_t* buf = reinterpret_cast<uint32_t*>(delta + nb);             // [T] key | code << 16
  uint16_t* wh = reinterpret_cast<uint16_t*>(buf + T);                // [kScatWaves][nb] counts, cursors
  __shared__ int32_t wave_tot[kScatWaves];

  // tiles of 8 consecutive tables go to one XCD (workgroups are dealt to the
  // eight XCDs in turn), so the runs that neighbouring tiles write to the same
  // cache lines meet in that XCD's L2
  const int bid = blockIdx.x;
  const int grp = bid / (8 * ntiles), rem = bid % (8 * ntiles);
  const int t = rem / 8;
  const int tb = grp * 8 + (rem % 8);     // table index u * L + l
  if (tb >= tables) return;
  const size_t table = static_cast<size_t>(tb);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tbeg = t << tile_log2;
  const int tlen = min(T, N - tbeg);
  const int cbase = (tbeg >> stride_log2) << stride_log2;
  const uint16_t* cd = codes + table * N;

  for (int i = tid; i < kScatWaves * kMt; i += kScatThreads) mt[i] = 0ull;
  for (int i = tid; i < kScatWaves * nb; i += kScatThreads) wh[i] = 0;
  // this wave's keys: batch k = keys wbeg + 64 k + lane, up to wend
  const int per = T / kScatWaves;
  const int wbeg = tbeg + wave * per;
  const int wend = min(tbeg + tlen, wbeg + per);
  int cr[kScatBatches];
#pragma unroll
  for (int k = 0; k < kScatBatches; ++k) {
    const int n = wbeg + 64 * k + lane;
    cr[k] = (64 * k < per && n < wend) ? static_cast<int>(cd[n]) : -1;
  }
  __syncthreads();

  uint64_t* my_mt = mt + wave * kMt;
  uint16_t* my_wh = wh + wave * nb;
  volatile uint16_t* vwh = my_wh;
  int rs[kScatBatches];                 // rank | count << 8 of this lane's key in its batch
#pragma unroll
  for (int k = 0; k < kScatBatches; ++k) {
    rs[k] = 0;
    if (64 * k >= per) continue;        // wave-uniform: tiles shorter than 8192 keys
    const bool valid = cr[k] >= 0;
    const int code = valid ? cr[k] : 0;
    const uint64_t m = match_lanes(code, valid, K, my_mt, lane);
    const int rank = mbcnt(m), cnt = __builtin_popcountll(m);
    rs[k] = rank | (cnt << 8);
    if (valid && rank == 0) vwh[code] = static_cast<uint16_t>(vwh[code] + cnt);
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();

  // phase 2: bucket c's tile-local start, per-wave cursors, table shift
  const int32_t* ts = tstart + (table * ntiles + t) * nb;
  const int bpt = (nb + kScatThreads - 1) / kScatThreads;
  const int c0 = tid * bpt, c1 = min(nb, c0 + bpt);
  int local = 0;
  for (int c = c0; c < c1; ++c)
    for (int w = 0; w < kScatWaves; ++w) local += wh[w * nb + c];
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
    delta[c] = ts[c] - run;
    for (int w = 0; w < kScatWaves; ++w) {
      const int x = wh[w * nb + c];
      wh[w * nb + c] = static_cast<uint16_t>(run);
      run += x;
    }
  }
  __syncthreads();

  // phase 3: placement into the local CSR
#pragma unroll
  for (int k = 0; k < kScatBatches; ++k) {
    if (64 * k >= per) continue;
    const bool valid = cr[k] >= 0;
    const int code = valid ? cr[k] : 0;
    const int rank = rs[k] & 0xff, cnt = rs[k] >> 8;
    const int p = valid ? static_cast<int>(vwh[code]) : 0;
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      buf[p + rank] = static_cast<uint32_t>(wbeg + 64 * k + lane - cbase) | (static_cast<uint32_t>(code) << 16);
      if (rank == 0) vwh[code] = static_cast<uint16_t>(p + cnt);
    }
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();

  // phase 4: entry e of the local CSR goes to table position delta[code] + e
  uint16_t* out = indices + table * N;
#pragma unroll 4
  for (int e = tid; e < tlen; e += kScatThreads) {
    const uint32_t v = buf[e];
    out[delta[v >> 16] + e] = static_cast<uint16_t>(v & 0xffffu);
  }
}

size_t scatter_lds_bytes(int K, int tile_log2) {
  const size_t nb = size_t(1) << K;
  return kScatWaves * (size_t(1) << kMatchLo) * 8 + nb * 4 + (size_t(4) << tile_log2) + kScatWaves * nb * 2;
}

// -------- general path (any K): one workgroup per table
//
// Key indices are split into sub-chunks of 2^sub_log2 keys, each owned by
// one wave that walks it in order in batches of 64:
//   pass 1  per-sub-chunk histograms with LDS atomic adds
//   pass 2  one scan over (bucket, sub-chunk) gives the offsets, the chunk
//           bounds and every sub-chunk's start position in every bucket
//   pass 3  scatter: the lanes of a batch holding the same code are found
//           with one ballot per code bit; a lane's rank among them is the
//           number of such lanes below it.
constexpr int kBucketThreads = 1024;
constexpr int kBucketWaves = kBucketThreads / 64;

// Mask of the valid lanes whose code equals this lane's: the AND over the K
// code bits of the ballot of the bit where this lane's bit is 1, or of its
// complement where it is 0.
__device__ __forceinline__ uint64_t match_code(int code, bool valid, int K) {
  uint64_t m = ballot(valid);
  for (int b = 0; b < K; ++b) {
    const bool bit = (code >> b) & 1;
    const uint64_t B = ballot(bit);
    m &= bit ? B : ~B;
  }
  return m;
}

__global__ __launch_bounds__(kBucketThreads) void bucket_tables_kernel(
    const uint16_t* __restrict__ codes,   // [U][L][N]
    int N, int K, int L, int nJ, int spc_log2, int sub_log2, int stride_log2,
    int32_t* __restrict__ offsets,        // [U][L][2^K + 1]
    uint16_t* __restrict__ indices,       // [U][L][N]
    int32_t* __restrict__ bounds) {       // [U][L][2^K][nJ + 1]
  extern __shared__ __attribute__((aligned(16))) int32_t pos[];   // [nSub][nb]
  __shared__ int32_t wave_tot[kBucketWaves];
  const int nb = 1 << K;
  const int nSub = nJ << spc_log2;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l = blockIdx.x, u = blockIdx.y;
  const size_t tbl = static_cast<size_t>(u) * L + l;
  const uint16_t* cd = codes + tbl * N;

  for (int i = tid; i < nSub * nb; i += kBucketThreads) pos[i] = 0;
  __syncthreads();

  for (int s = wave; s < nSub; s += kBucketWaves) {
    const int beg = s << sub_log2, end = min(N, beg + (1 << sub_log2));
    int32_t* ps = pos + static_cast<size_t>(s) * nb;
    for (int b0 = beg; b0 < end; b0 += 64 * kPrefetch) {
      int pf[kPrefetch];
#pragma unroll
      for (int k = 0; k < kPrefetch; ++k) {
        const int n = b0 + 64 * k + lane;
        pf[k] = n < end ? static_cast<int>(cd[n]) : -1;
      }
#pragma unroll
      for (int k = 0; k < kPrefetch; ++k)
        if (pf[k] >= 0) atomicAdd(&ps[pf[k]], 1);
    }
  }
  __syncthreads();

  {
    const int bpt = (nb + kBucketThreads - 1) / kBucketThreads;
    const int c0 = tid * bpt, c1 = min(nb, c0 + bpt);
    int local = 0;
    for (int c = c0; c < c1; ++c)
      for (int s = 0; s < nSub; ++s) local += pos[static_cast<size_t>(s) * nb + c];
    int incl = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int wbase = 0;
    for (int w = 0; w < wave; ++w) wbase += wave_tot[w];
    int run = wbase + incl - local;
    int32_t* off = offsets + tbl * (nb + 1);
    for (int c = c0; c < c1; ++c) {
      off[c] = run;
      int32_t* bnd = bounds + (tbl * nb + c) * (nJ + 1);
      for (int s = 0; s < nSub; ++s) {
        if ((s & ((1 << spc_log2) - 1)) == 0) bnd[s >> spc_log2] = run;
        const int t = pos[static_cast<size_t>(s) * nb + c];
        pos[static_cast<size_t>(s) * nb + c] = run;
        run += t;
      }
      bnd[nJ] = run;
    }
    if (tid == 0) off[nb] = N;
  }
  __syncthreads();

  uint16_t* out = indices + tbl * N;
  for (int s = wave; s < nSub; s += kBucketWaves) {
    const int beg = s << sub_log2, end = min(N, beg + (1 << sub_log2));
    const int cbase = (beg >> stride_log2) << stride_log2;
    int32_t* ps = pos + static_cast<size_t>(s) * nb;
    for (int b0 = beg; b0 < end; b0 += 64 * kPrefetch) {
      int pf[kPrefetch];
#pragma unroll
      for (int k = 0; k < kPrefetch; ++k) {
        const int n = b0 + 64 * k + lane;
        pf[k] = n < end ? static_cast<int>(cd[n]) : -1;
      }
#pragma unroll
      for (int k = 0; k < kPrefetch; ++k) {
        if (b0 + 64 * k >= end) break;
        const int n = b0 + 64 * k + lane;
        const bool valid = pf[k] >= 0;
        const int code = valid ? pf[k] : 0;
        const uint64_t m = match_code(code, valid, K);
        const int rank = mbcnt(m);
        const int p = valid ? ps[code] : 0;
        __builtin_amdgcn_wave_barrier();
        if (valid) out[p + rank] = static_cast<uint16_t>(n - cbase);
        if (valid && rank == 0) ps[code] = p + __builtin_popcountll(m);
        __builtin_amdgcn_wave_barrier();
      }
    }
  }
}

size_t bucket_lds_bytes(int nJ, int spc_log2, int K) {
  return static_cast<size_t>(nJ << spc_log2) * (size_t(1) << K) * 4;
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

bool bucket_fast_path(int N, int K, int stride_log2, int* tile_log2, int* ntiles) {
  const int tl = stride_log2 < kMaxTileLog2 ? stride_log2 : kMaxTileLog2;
  const long long nt = (static_cast<long long>(N) + (1ll << tl) - 1) >> tl;
  if (tile_log2) *tile_log2 = tl;
  if (ntiles) *ntiles = static_cast<int>(nt);
  return K <= 10 && (nt << K) <= 32768;
}

hipError_t launch_build(const BuildArgs& a, hipStream_t stream) {
  hipError_t e = (a.dtype == 1)
      ? launch_project<BF16>(a.keys, a.W, a.wt, a.codes, a.U, a.N, a.K, a.L, stream)
      : launch_project<F32>(a.keys, a.W, a.wt, a.codes, a.U, a.N, a.K, a.L, stream);
  if (e != hipSuccess) return e;
  int tile_log2 = 0, ntiles = 0;
  if (a.tstart && bucket_fast_path(a.N, a.K, a.stride_log2, &tile_log2, &ntiles)) {
    const size_t lds1 = static_cast<size_t>(ntiles) << a.K << 2;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(bucket_count_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds1));
    if (e != hipSuccess) return e;
    e = launch(kKBucketCount, bucket_count_kernel, dim3(a.L, a.U), dim3(kCountTThreads),
               static_cast<unsigned>(lds1), stream, static_cast<const uint16_t*>(a.codes), a.N, a.K, a.L,
               tile_log2, ntiles, a.nJ, a.stride_log2 - tile_log2, a.offsets, a.bounds, a.tstart);
    if (e != hipSuccess) return e;
    const size_t lds2 = scatter_lds_bytes(a.K, tile_log2);
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(bucket_scatter_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds2));
    if (e != hipSuccess) return e;
    const int tables = a.U * a.L;
    const int ngroups = (tables + 7) / 8;
    return launch(kKBucketScatter, bucket_scatter_kernel, dim3(ngroups * 8 * ntiles), dim3(kScatThreads),
                  static_cast<unsigned>(lds2), stream, static_cast<const uint16_t*>(a.codes),
                  static_cast<const int32_t*>(a.tstart), a.N, a.K, a.L, tile_log2, ntiles, a.stride_log2,
                  tables, a.indices);
  }
  const size_t lds = bucket_lds_bytes(a.nJ, a.spc_log2, a.K);
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(bucket_tables_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  return launch(kKBucket, bucket_tables_kernel, dim3(a.L, a.U), dim3(kBucketThreads),
                static_cast<unsigned>(lds), stream, static_cast<const uint16_t*>(a.codes), a.N, a.K, a.L,
                a.nJ, a.spc_log2, a.stride_log2 - a.spc_log2, a.stride_log2, a.offsets, a.indices, a.bounds);
}

}  // namespace lsh
