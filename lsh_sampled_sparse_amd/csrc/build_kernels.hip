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
// Per-table stable bucketing.
//
// Key indices of a table are split into sub-chunks of 2^sub_log2 keys; each
// sub-chunk is owned by one wave, which walks it in order in batches of 64.
// Inside a batch, lanes with equal codes are grouped: every lane writes its
// lane id to a per-wave LDS slot addressed by its code; lanes that read back
// another id belong to a group of size >= 2, and those groups are peeled one
// code at a time with a ballot.  A lane's rank is the number of lower lanes
// of its group, so the order inside a bucket is the key order.
// ---------------------------------------------------------------------------
constexpr int kBucketThreads = 1024;
constexpr int kBucketWaves = kBucketThreads / 64;
constexpr int kSlotsPerWave = 1024;

__device__ __forceinline__ void group_lanes(int code, bool valid, uint8_t* slots, int lane,
                                            int& rank, int& size) {
  // volatile: the read must observe the other lanes' writes, not this lane's
  volatile uint8_t* vs = slots;
  const int slot = code & (kSlotsPerWave - 1);
  if (valid) vs[slot] = static_cast<uint8_t>(lane);
  __builtin_amdgcn_wave_barrier();
  const int winner = valid ? vs[slot] : lane;
  uint64_t losers = ballot(valid && winner != lane);
  rank = 0;
  size = 1;
  while (losers) {
    const int f = __builtin_ctzll(losers);
    const int c = __builtin_amdgcn_readlane(code, f);
    const bool mine = valid && code == c;
    const uint64_t m = ballot(mine);
    if (mine) {
      rank = mbcnt(m);
      size = __builtin_popcountll(m);
    }
    losers &= ~m;
  }
  __builtin_amdgcn_wave_barrier();
}

__global__ __launch_bounds__(kBucketThreads) void bucket_tables_kernel(
    const uint16_t* __restrict__ codes,   // [U][L][N]
    int N, int K, int L, int nJ, int spc_log2, int sub_log2,
    int32_t* __restrict__ offsets,        // [U][L][2^K + 1]
    int32_t* __restrict__ indices,        // [U][L][N]
    int32_t* __restrict__ bounds) {       // [U][L][2^K][nJ + 1]
  extern __shared__ __attribute__((aligned(16))) int32_t smem[];
  __shared__ int32_t wave_tot[kBucketWaves];
  const int nb = 1 << K;
  const int nSub = nJ << spc_log2;
  int32_t* pos = smem;                                                   // [nSub][nb]
  uint8_t* slots = reinterpret_cast<uint8_t*>(smem + static_cast<size_t>(nSub) * nb);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l = blockIdx.x, u = blockIdx.y;
  const size_t tbl = static_cast<size_t>(u) * L + l;
  const uint16_t* cd = codes + tbl * N;
  uint8_t* my_slots = slots + wave * kSlotsPerWave;

  for (int i = tid; i < nSub * nb; i += kBucketThreads) pos[i] = 0;
  __syncthreads();

  // pass 1: per-sub-chunk histograms
  for (int s = wave; s < nSub; s += kBucketWaves) {
    const int beg = s << sub_log2, end = min(N, beg + (1 << sub_log2));
    int32_t* ps = pos + static_cast<size_t>(s) * nb;
    for (int b = beg; b < end; b += 64) {
      const int n = b + lane;
      const bool valid = n < end;
      const int code = valid ? cd[n] : 0;
      int rank, size;
      group_lanes(code, valid, my_slots, lane, rank, size);
      if (valid && rank == 0) ps[code] += size;
      __builtin_amdgcn_wave_barrier();
    }
  }
  __syncthreads();

  // pass 2: offsets (scan over buckets) and per-sub-chunk start positions
  {
    const int bpt = (nb + kBucketThreads - 1) / kBucketThreads;   // buckets per thread
    const int c0 = tid * bpt, c1 = min(nb, c0 + bpt);
    int local = 0;
    for (int c = c0; c < c1; ++c)
      for (int s = 0; s < nSub; ++s) local += pos[static_cast<size_t>(s) * nb + c];
    // block exclusive scan of `local`
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

  // pass 3: stable scatter
  int32_t* out = indices + tbl * N;
  for (int s = wave; s < nSub; s += kBucketWaves) {
    const int beg = s << sub_log2, end = min(N, beg + (1 << sub_log2));
    int32_t* ps = pos + static_cast<size_t>(s) * nb;
    for (int b = beg; b < end; b += 64) {
      const int n = b + lane;
      const bool valid = n < end;
      const int code = valid ? cd[n] : 0;
      int rank, size;
      group_lanes(code, valid, my_slots, lane, rank, size);
      const int p = valid ? ps[code] : 0;
      __builtin_amdgcn_wave_barrier();
      if (valid) out[p + rank] = n;
      if (valid && rank == 0) ps[code] = p + size;
      __builtin_amdgcn_wave_barrier();
    }
  }
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

hipError_t launch_build(const BuildArgs& a, hipStream_t stream) {
  hipError_t e = (a.dtype == 1)
      ? launch_project<BF16>(a.keys, a.W, a.wt, a.codes, a.U, a.N, a.K, a.L, stream)
      : launch_project<F32>(a.keys, a.W, a.wt, a.codes, a.U, a.N, a.K, a.L, stream);
  if (e != hipSuccess) return e;
  const size_t lds = bucket_lds_bytes(a.nJ, a.spc_log2, a.K);
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(bucket_tables_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  return launch(kKBucket, bucket_tables_kernel, dim3(a.L, a.U), dim3(kBucketThreads),
                static_cast<unsigned>(lds), stream, static_cast<const uint16_t*>(a.codes), a.N, a.K, a.L,
                a.nJ, a.spc_log2, a.stride_log2 - a.spc_log2, a.offsets, a.indices, a.bounds);
}

size_t bucket_lds_bytes(int nJ, int spc_log2, int K) {
  return static_cast<size_t>(nJ << spc_log2) * (size_t(1) << K) * 4 +
         static_cast<size_t>(kBucketWaves) * kSlotsPerWave;
}

}  // namespace lsh
