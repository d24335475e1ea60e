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
// W transpose
// ---------------------------------------------------------------------------
template <typename T>
__global__ void transpose_w_kernel(const typename T::storage* __restrict__ W,
                                   typename T::storage* __restrict__ WT, int LK, int LKpad) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= LKpad * kHeadDim) return;
  const int c = idx / kHeadDim, i = idx % kHeadDim;
  WT[idx] = (c < LK) ? W[static_cast<size_t>(i) * LK + c] : typename T::storage(0);
}

constexpr int kProjThreads = 256;              // 4 waves
constexpr int kProjKeys = 256;                 // 64 keys per wave = 4 tiles of 16
constexpr int kSlabCols = 64;                  // projection columns per LDS slab
template <typename T>
struct ProjLds {
  // slab row stride padded by 16 bytes so 16 rows read at one offset hit
  // different LDS banks
  static constexpr int kRow = kHeadDim + 16 / T::bytes;
  static constexpr int kSlabElems = kSlabCols * kRow;
  static constexpr int kChunksPerThread = kSlabCols * kHeadDim * T::bytes / 16 / kProjThreads;
};

// codes[u][l][n] for n in this workgroup's 256 keys.
template <typename T>
__global__ __launch_bounds__(kProjThreads) void project_codes_kernel(
    const typename T::storage* __restrict__ keys,   // [U][N][128]
    const typename T::storage* __restrict__ WT,     // [LKpad][128]
    uint16_t* __restrict__ codes,                   // [U][L][N]
    int N, int K, int L, int nslab) {
  using S = typename T::storage;
  using PL = ProjLds<T>;
  __shared__ __attribute__((aligned(16))) S wt[2][PL::kSlabElems];
  // sign masks of one slab: [slab & 1][col tile][key tile][i]; bit (16 q + c) of
  // mask i is the sign of proj[key 4 q + i][col c] within the 16 x 16 tile
  __shared__ uint64_t ring[2][4][16][4];

  const int u = blockIdx.y;
  const int n0 = blockIdx.x * kProjKeys;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const S* kb = keys + static_cast<size_t>(u) * N * kHeadDim;
  uint16_t* cb = codes + static_cast<size_t>(u) * L * N;
  const int n = n0 + tid;

  if (K == 0) {
    if (n < N)
      for (int l = 0; l < L; ++l) cb[static_cast<size_t>(l) * N + n] = 0;
    return;
  }

  Frag<T> A[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int key = n0 + wave * 64 + a * 16 + (lane & 15);
    const bool valid = key < N;
    A[a].load(kb + static_cast<size_t>(valid ? key : 0) * kHeadDim + (lane >> 4) * 32, valid);
  }

  // slab s of WT is the contiguous block WT[64 s : 64 s + 64][:]; each thread
  // moves kChunksPerThread 16-byte pieces of it into the padded LDS rows
  constexpr int kCPT = PL::kChunksPerThread;
  constexpr int kChunksPerRow = kHeadDim * T::bytes / 16;
  u32x4_t pre[kCPT];
  {
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(WT);
#pragma unroll
    for (int k = 0; k < kCPT; ++k) pre[k] = src[tid + k * kProjThreads];
#pragma unroll
    for (int k = 0; k < kCPT; ++k) {
      const int chunk = tid + k * kProjThreads;
      *reinterpret_cast<u32x4_t*>(&wt[0][(chunk / kChunksPerRow) * PL::kRow +
                                       (chunk % kChunksPerRow) * (16 / T::bytes)]) = pre[k];
    }
  }
  __syncthreads();

  const int key_tile = tid >> 4, key_row = tid & 15;

  for (int s = 0; s < nslab; ++s) {
    const int buf = s & 1;
    if (s + 1 < nslab) {
      const u32x4_t* src = reinterpret_cast<const u32x4_t*>(WT + static_cast<size_t>(s + 1) * kSlabCols * kHeadDim);
#pragma unroll
      for (int k = 0; k < kCPT; ++k) pre[k] = src[tid + k * kProjThreads];
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      Frag<T> Bf;
      Bf.load(&wt[buf][(ct * 16 + (lane & 15)) * PL::kRow + (lane >> 4) * 32], true);
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
        acc = A[a].mma(Bf, acc);
        const uint64_t m0 = ballot(acc[0] > 0.f);
        const uint64_t m1 = ballot(acc[1] > 0.f);
        const uint64_t m2 = ballot(acc[2] > 0.f);
        const uint64_t m3 = ballot(acc[3] > 0.f);
        if (lane == 0) {
          uint64_t* dst = ring[buf][ct][wave * 4 + a];
          dst[0] = m0; dst[1] = m1; dst[2] = m2; dst[3] = m3;
        }
      }
    }
    if (s + 1 < nslab) {
#pragma unroll
      for (int k = 0; k < kCPT; ++k) {
        const int chunk = tid + k * kProjThreads;
        *reinterpret_cast<u32x4_t*>(&wt[buf ^ 1][(chunk / kChunksPerRow) * PL::kRow +
                                               (chunk % kChunksPerRow) * (16 / T::bytes)]) = pre[k];
      }
    }
    __syncthreads();
    // tables whose last bit lies in this slab
    const int lb = min(L, (kSlabCols * s) / K);
    const int le = min(L, (kSlabCols * (s + 1)) / K);
    if (n < N) {
      for (int l = lb; l < le; ++l) {
        const int col0 = l * K, ct0 = col0 >> 4, sh = col0 & 15;
        // 16 sign bits of this thread's key in column tiles ct0 and ct0 + 1
        const uint64_t m0 = ring[(ct0 >> 2) & 1][ct0 & 3][key_tile][key_row & 3];
        uint32_t w = static_cast<uint32_t>(m0 >> (16 * (key_row >> 2))) & 0xffffu;
        if (sh + K > 16) {
          const int ct1 = ct0 + 1;
          const uint64_t m1 = ring[(ct1 >> 2) & 1][ct1 & 3][key_tile][key_row & 3];
          w |= (static_cast<uint32_t>(m1 >> (16 * (key_row >> 2))) & 0xffffu) << 16;
        }
        cb[static_cast<size_t>(l) * N + n] = static_cast<uint16_t>((w >> sh) & ((1u << K) - 1u));
      }
    }
    __syncthreads();
  }
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
template <typename T>
static hipError_t launch_project(const void* keys, const void* W, void* WT, uint16_t* codes,
                                 int U, int N, int K, int L, hipStream_t stream) {
  using S = typename T::storage;
  const int LK = L * K;
  const int nslab = (LK + kSlabCols - 1) / kSlabCols;
  const int LKpad = nslab * kSlabCols;
  if (LK > 0) {
    const int total = LKpad * kHeadDim;
    hipError_t e = launch(kKTransposeW, transpose_w_kernel<T>, dim3((total + 255) / 256), dim3(256), 0,
                          stream, static_cast<const S*>(W), static_cast<S*>(WT), LK, LKpad);
    if (e != hipSuccess) return e;
  }
  return launch(kKProject, project_codes_kernel<T>, dim3((N + kProjKeys - 1) / kProjKeys, U),
                dim3(kProjThreads), 0, stream, static_cast<const S*>(keys), static_cast<const S*>(WT),
                codes, N, K, L, nslab);
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
