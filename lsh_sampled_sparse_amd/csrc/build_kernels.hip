// Table-build kernels (prefill side) for gfx950.
//
// MagicPIG builds per-table hash buckets of the keys at prefill and names an
// optimised hash-table construction (MagicPIG project summary on sourcepulse,
// "Highlighted Details").  Here the build is:
//   transpose_w     W [d, L*K] -> -WT [LKpad, d] (negated, rows permuted,
//                   zero rows for padding), so that a projection column is
//                   one contiguous row
//   project_codes   SimHash codes of every key: a dense bf16 (or fp32) MFMA
//                   contraction keys x W with fp32 accumulation, each lane
//                   packing its own key's code bits from its accumulators (one
//                   funnel shift per bit), codes written table-major
//   chunk_sort      per (table, key chunk): a stable LSD radix sort of the
//                   chunk's keys by code into the chunk's own region of the
//                   index array, with the chunk's bucket offsets
#include <algorithm>

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

// WT[R][d] = -W[d][column] for row R = (slab, tile ct, row r = 4 g + i).  The
// kernel below shifts the signs of a lane group's positions j = 4 ct + i into
// a word in increasing j, so position j lands on bit P - 1 - j; that bit is
// bit b of table tt of the group when P - 1 - j = tt K + b, i.e. table
// slab * 4 TPG + g * TPG + tt.  W is negated so that the code bit [k.w > 0]
// is the sign bit of the MFMA result k.(-w) (see push_code_bit).
template <typename T>
__global__ void transpose_w_kernel(const typename T::storage* __restrict__ W,
                                   typename T::storage* __restrict__ WT, int K, int L, int nct, int tpg,
                                   int rows, int w_heads) {   // one W (and WT) per kv head when w_heads > 1
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= w_heads * rows * kHeadDim) return;
  const int hw = idx / (rows * kHeadDim), rem = idx % (rows * kHeadDim);
  const int R = rem / kHeadDim, d = rem % kHeadDim;
  const int slab = R / (nct * 16), p = R % (nct * 16);
  const int ct = p / 16, r = p % 16;
  const int g = r / 4, j = ct * 4 + r % 4;
  const int jr = 4 * nct - 1 - j;
  const int tt = jr / K, b = jr % K;
  const int t = slab * 4 * tpg + g * tpg + tt;
  const bool valid = tt < tpg && t < L;
  WT[idx] = valid ? negate(W[(static_cast<size_t>(hw) * kHeadDim + d) * L * K + t * K + b]) : typename T::storage(0);
}

// (s << 1) | [k.w > 0] from y = k.(-w), the MFMA result against the negated
// W: one funnel shift appends the sign bit of y.  y < 0 exactly when k.w > 0.
// A sum that is exactly zero comes out as +0: the accumulator starts at +0.0
// and an IEEE sum holding a +0 term is +0 unless it rounds from a nonzero
// value, so exact zeros give bit 0, as [k.w > 0] requires; a tiny sum that
// underflows keeps its sign.
__device__ __forceinline__ uint32_t push_code_bit(uint32_t s, float y) {
  return __builtin_amdgcn_alignbit(s, __float_as_uint(y), 31u);
}

// Sign bits of one slab (NCT column tiles of 16 projection columns) for this
// lane's key in each of the KT key tiles: sg[a] collects the P = 4 NCT rows
// of lane group g in row order (s = 2 s + [x > 0]).  `wrow` points at this
// lane's W row (tile 0, row lane % 16, dims [32 g, 32 g + 32)) in LDS; rows
// are `row` elements apart.  Software pipelined over column tiles: each of the
// 16 MFMAs of tile ct is paired with one sign update of tile ct - 1 (two
// accumulator sets, two W fragments), and the pairs are fenced so that the
// VALU work issues while the matrix pipe runs; the W fragment of tile ct + 1
// is read during tile ct.
template <typename T, int NCT, int KT>
__device__ __forceinline__ void slab_signs(const typename T::storage* wrow, int row, const Frag<T> (&A)[KT],
                                           uint32_t (&sg)[KT]) {
#pragma unroll
  for (int a = 0; a < KT; ++a) sg[a] = 0u;
  floatx4_t accA[KT], accB[KT];
  Frag<T> Wa, Wb;
  auto wtile = [&](int ct) { return wrow + min(ct, NCT - 1) * 16 * row; };
  // MFMAs of one tile (W -> acc), paired with the signs of the previous one
  auto half = [&](const Frag<T>& W, floatx4_t (&acc)[KT], const floatx4_t (&prev)[KT], bool signs) {
#pragma unroll
    for (int a = 0; a < KT; ++a) acc[a] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 4 * KT; ++q) {
      W.mma_step(q / KT, A[q % KT], acc[q % KT]);     // k-step q / KT of key tile q % KT
      if (signs) sg[q >> 2] = push_code_bit(sg[q >> 2], prev[q >> 2][q & 3]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto signs_of = [&](const floatx4_t (&acc)[KT]) {
#pragma unroll
    for (int a = 0; a < KT; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) sg[a] = push_code_bit(sg[a], acc[a][i]);
  };
  Wa.load(wtile(0), true);
  Wb.load(wtile(1), true);
  half(Wa, accA, accB, false);                        // tile 0
  int ct = 1;
#pragma unroll 1
  for (; ct + 1 < NCT; ct += 2) {
    Wa.load(wtile(ct + 1), true);
    half(Wb, accB, accA, true);                       // tile ct, signs of ct - 1
    Wb.load(wtile(ct + 2), true);
    half(Wa, accA, accB, true);                       // tile ct + 1, signs of ct
  }
  if (NCT % 2 == 0) {
    half(Wb, accB, accA, true);                       // tile NCT - 1
    signs_of(accB);
  } else {
    signs_of(accA);
  }
}

constexpr int kProjThreads = 256;              // 4 waves
constexpr int kProjKT = 4;                     // key tiles of 16 per wave
constexpr int kProjKeys = 64 * kProjKT;        // keys per workgroup

// codes[u][l][n] for this workgroup's kProjKeys keys.
template <typename T, int KB>
__global__ __launch_bounds__(kProjThreads, T::bytes == 2 ? 3 : 1) void project_codes_kernel(
    const typename T::storage* __restrict__ keys,   // [U][P][128]
    const typename T::storage* __restrict__ WT,     // [nslab * NCT * 16][128], permuted
    uint16_t* __restrict__ codes,                   // [U][L][P]
    int N, int P, int n_first, int L, int nslab,    // keys n_first .. N - 1
    int n_old,                                      // the update's bound on the old lengths
    int spz,                                        // slabs per blockIdx.z
    int Hkv, size_t wt_head_stride,                 // WT of kv head g at g * wt_head_stride
    const int32_t* __restrict__ old_lens,           // optional per-sequence ranges
    const int32_t* __restrict__ new_lens, int stride_log2) {
  using S = typename T::storage;
  constexpr ProjShape PS = proj_shape(KB);
  constexpr int NCT = PS.nct, TPG = PS.tpg, TPS = 4 * TPG;
  constexpr int kRows = NCT * 16;                                  // WT rows per slab
  constexpr int kRow = kHeadDim + 16 / T::bytes;                   // padded LDS row
  constexpr int kChunksPerRow = kHeadDim * T::bytes / 16;
  constexpr int kCPT = kRows * kChunksPerRow / kProjThreads;       // 16-byte pieces per thread
  constexpr uint32_t kMask = (1u << KB) - 1u;
  constexpr int kStgRow = kProjKeys + 8;                           // padded staging row (uint16)
  __shared__ __attribute__((aligned(16))) S wt[2][kRows * kRow];
  // codes of one slab, [table in slab][key in block], double-buffered so that
  // the write-out after a slab's barrier never races the next slab's writes
  __shared__ __attribute__((aligned(16))) uint16_t stg[2][TPS * kStgRow];

  const int u = blockIdx.y;
  const int n0 = n_first + blockIdx.x * kProjKeys;
  // this sequence's keys to (re)code: every key from the start of the chunk
  // that holds its first new key (none when its keys are inserted: the
  // insert kernel codes them)
  const SeqUpdate su = seq_update(old_lens, new_lens, u / Hkv, n_old, N);
  const int hi = su.hi;
  const int lo = su.insert ? hi : (su.old >> stride_log2) << stride_log2;
  if (n0 >= hi || n0 + kProjKeys <= lo || lo >= hi) return;
  WT += static_cast<size_t>(u % Hkv) * wt_head_stride;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4;
  const S* kb = keys + static_cast<size_t>(u) * P * kHeadDim;
  uint16_t* cb = codes + static_cast<size_t>(u) * L * P;

  // key fragments (MFMA B operand): lane holds key lane & 15 of tile a, dims
  // [32 g, 32 g + 32)
  Frag<T> A[kProjKT];
#pragma unroll
  for (int a = 0; a < kProjKT; ++a) {
    const int key = n0 + wave * 16 * kProjKT + a * 16 + (lane & 15);
    const bool valid = key >= lo && key < hi;
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
  // this workgroup's slabs: zb .. zb + ns - 1 (all of them unless a short
  // key range is spread over more workgroups by slab).  Workgroups walk
  // their slabs from different starting points, so that the CUs sharing an
  // L2 do not all read the same slab of WT at once
  const int zb = static_cast<int>(blockIdx.z) * spz;
  const int ns = min(spz, nslab - zb);
  const int s0 = static_cast<int>((blockIdx.x + 5u * blockIdx.y) % static_cast<unsigned>(ns));
  auto slab_of = [&](int s) { return zb + (s0 + s < ns ? s0 + s : s0 + s - ns); };
  fetch(slab_of(0));
  stash(0);
  __syncthreads();

  for (int s = 0; s < ns; ++s) {
    const int buf = s & 1;
    if (s + 1 < ns) fetch(slab_of(s + 1));
    uint32_t sg[kProjKT];
    slab_signs<T, NCT, kProjKT>(&wt[buf][(lane & 15) * kRow + (lane >> 4) * 32], kRow, A, sg);
    // codes of tables slab_of(s) * TPS + g * TPG + tt, staged per table row
    uint16_t* sb = stg[s & 1];
#pragma unroll
    for (int a = 0; a < kProjKT; ++a)
#pragma unroll
      for (int tt = 0; tt < TPG; ++tt)
        sb[(g * TPG + tt) * kStgRow + wave * 16 * kProjKT + a * 16 + (lane & 15)] =
            static_cast<uint16_t>((sg[a] >> (tt * KB)) & kMask);
    if (s + 1 < ns) stash(buf ^ 1);
    __syncthreads();
    // write-out: 8 consecutive keys of one table per 16-byte piece
    for (int c = tid; c < TPS * (kProjKeys / 8); c += kProjThreads) {
      const int r = c / (kProjKeys / 8), k8 = (c % (kProjKeys / 8)) * 8;
      const int t = slab_of(s) * TPS + r, key = n0 + k8;
      if (t < L && key >= lo) {                       // lo is a chunk start: a multiple of 8
        const uint16_t* src = sb + r * kStgRow + k8;
        uint16_t* dst = cb + static_cast<size_t>(t) * P + key;
        if (key + 8 <= hi && (P & 7) == 0) {
          *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
        } else {
          for (int e = 0; e < 8; ++e)
            if (key + e < hi) dst[e] = src[e];
        }
      }
    }
  }
}

// K = 0: every code is 0 (keys n_first .. N - 1 of every [U][L] row of
// pitch P, within each sequence's own range as in project_codes_kernel).
__global__ void zero_codes_kernel(uint16_t* __restrict__ codes, size_t rows, int n_first, int N, int P, int L,
                                  int n_old, int Hkv, const int32_t* __restrict__ old_lens,
                                  const int32_t* __restrict__ new_lens, int stride_log2) {
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const size_t w = static_cast<size_t>(N - n_first);
  if (i >= rows * w) return;
  const size_t row = i / w;
  const int key = n_first + static_cast<int>(i % w);
  const SeqUpdate su = seq_update(old_lens, new_lens, static_cast<int>(row / L) / Hkv, n_old, N);
  const int lo = su.insert ? su.hi : (su.old >> stride_log2) << stride_log2;
  if (key >= lo && key < su.hi) codes[row * P + key] = 0;
}

// ---------------------------------------------------------------------------
// Bucketing: a stable sort of every (table, key chunk) by code.
//
// Output format (chunk-major two-level CSR): chunk j of table l covers keys
// [j stride, (j + 1) stride) and owns positions [j stride, (j + 1) stride)
// of the table's index array; there its keys are sorted by code, ascending
// key inside a code, each stored as (key - j stride).  offsets[j][c] is the
// start of bucket c inside the chunk's region, so bucket c of chunk j is
// positions offsets[j][c] .. offsets[j][c + 1] (the chunk's length for the
// last bucket).  No scan crosses chunks, so every (table, chunk) is sorted by
// one workgroup, and its region is written contiguously.
//
// The sort is a least-significant-digit radix sort held in LDS, on digits of
// up to 5 code bits (K <= 15: at most three passes).  Elements are packed as
// code << 16 | key.  In every pass thread t owns the E consecutive positions
// E t .. E t + E - 1 of the current order, so a key's stable rank is
//   (elements of smaller digit) + (elements of its digit owned by threads
//   below t) + (elements of its digit earlier in thread t).
// Each thread counts its digits in 32 private 16-bit counters, two to a
// 32-bit word; word w of thread t sits in row w of cnt[16][nthr], at column
// swz(t), so the lanes of a wave touch distinct banks whatever their digits.
// Digit d lives in word d & 15, half d >> 4.  One exclusive scan over the
// word array in (w, t) order then gives every low half its start; a high
// half also needs the count of all low-half digits, which the block total
// carries in its low 16 bits.  Counters step by 4, so a rank comes out as the
// byte offset bfe(start + count before it, half) of the element's position:
// low halves never exceed 4 x 8192, so no carry reaches the high half.
//
// The buffer has E * nthr slots; slots at or past the chunk's length hold
// code 0xffff, whose every digit is the largest, so they stay behind all keys
// in every pass and the loops need no validity tests.
// ---------------------------------------------------------------------------
constexpr int kSortE = 32;              // elements per thread
constexpr int kDigitBits = 5;
constexpr int kCntWords = 16;           // 32 digit counters of 16 bits per thread

// LDS bank swizzle of a counter word index: bits 5-6 are folded into bits
// 2-3.  A 4-word quad stays contiguous, so a lane reading 16 consecutive
// words as four 16-byte loads spreads every 8 lanes over all 32 banks, while
// 32 consecutive indices (one per lane) still hit 32 distinct banks.
__device__ __forceinline__ int swz(int x) { return x ^ ((x >> 3) & 12); }

// Element buffer slot of position p: four padding words after every 32, for
// the same reason (a lane's run of 16 is four quads; 8 lanes cover 32 banks).
__device__ __forceinline__ int slot(int p) { return p + ((p >> 5) << 2); }

__device__ __forceinline__ void load_run(const uint32_t* buf, int p, uint32_t (&e)[kSortE]) {
#pragma unroll
  for (int q = 0; q < kSortE / 4; ++q) {
    const uint4 v = *reinterpret_cast<const uint4*>(buf + slot(p + 4 * q));
    e[4 * q] = v.x;
    e[4 * q + 1] = v.y;
    e[4 * q + 2] = v.z;
    e[4 * q + 3] = v.w;
  }
}

// Exclusive scan of the packed counter words, in place.  Thread s scans the
// 16 consecutive words 16 s .. 16 s + 15 of the (w, t) order; word (w, t) is
// stored at w * NTHR + swz(t).
template <int NTHR>
__device__ __forceinline__ void scan_counters(uint32_t* cnt, uint32_t* wave_tot) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int addr[kCntWords / 4];
  uint32_t x[kCntWords];
#pragma unroll
  for (int q = 0; q < kCntWords / 4; ++q) {
    const int f = kCntWords * tid + 4 * q;
    const int w = f / NTHR, t = f % NTHR;
    addr[q] = w * NTHR + swz(t);
    const uint4 v = *reinterpret_cast<const uint4*>(cnt + addr[q]);
    x[4 * q] = v.x;
    x[4 * q + 1] = v.y;
    x[4 * q + 2] = v.z;
    x[4 * q + 3] = v.w;
  }
  uint32_t run = 0;
#pragma unroll
  for (int q = 0; q < kCntWords; ++q) {
    const uint32_t v = x[q];
    x[q] = run;
    run += v;
  }
  uint32_t incl = run;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  uint32_t base = incl - run, total = 0;
#pragma unroll
  for (int w = 0; w < NTHR / 64; ++w) {
    const uint32_t t = wave_tot[w];
    base += w < wave ? t : 0u;
    total += t;
  }
  base += (total & 0xffffu) << 16;      // high halves start after every low-half digit
#pragma unroll
  for (int q = 0; q < kCntWords / 4; ++q)
    *reinterpret_cast<uint4*>(cnt + addr[q]) =
        make_uint4(base + x[4 * q], base + x[4 * q + 1], base + x[4 * q + 2], base + x[4 * q + 3]);
}

// One workgroup of NTHR = max(64, chunk / E) threads per (table, chunk);
// LDS: counters [16][NTHR] and the padded element buffer, 32-bit, in the same
// region, reused at the end for the bucket starts [2^K] (16-bit).
template <int NTHR>
__global__ __launch_bounds__(NTHR, NTHR >= 256 ? 4 : 1) void chunk_sort_kernel(
    const uint16_t* __restrict__ codes,   // [U][L][P]
    int N, int P, int K, int stride_log2, int nJP, int j0,   // chunks j0 + blockIdx.x
    uint16_t* __restrict__ offsets,       // [U][L][nJP][2^K]
    uint16_t* __restrict__ indices,       // [U][L][P]
    int L, int Hkv, int n_old, const int32_t* __restrict__ old_lens, const int32_t* __restrict__ new_lens
#ifdef LSH_CHECKED
    , uint32_t* check
#endif
    ) {
  constexpr int E = kSortE;
  extern __shared__ __attribute__((aligned(16))) uint32_t smem32[];
  __shared__ uint32_t wave_tot[NTHR / 64];
  constexpr int nthr = NTHR;
  // the counters and the element buffer share LDS: the elements are in
  // registers from the run load to the scatter, and the counters are dead
  // once every thread has read its ranks (barriers on both sides)
  uint32_t* cnt = smem32;                       // [16][NTHR]
  uint32_t* buf = smem32;                       // slot(position): code << 16 | key
  const int j = j0 + blockIdx.x;
  const size_t table = blockIdx.y;              // u * L + l
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nb = 1 << K;
  const int cbeg = j << stride_log2;
  // this sequence's chunks to rebuild (the same ranges as the projection;
  // none when its new keys are inserted instead)
  const SeqUpdate su = seq_update(old_lens, new_lens, static_cast<int>(table / L) / Hkv, n_old, N);
  const int hi = su.hi;
  if (su.insert || j < (su.old >> stride_log2) || cbeg >= hi) return;
  const int clen = min(1 << stride_log2, hi - cbeg);
  const int p0 = tid * E;
  const bool full = p0 + E <= clen;
  const bool vec = ((table * P) & 7) == 0;      // the chunk's codes are 16-byte aligned

  // this thread's E positions, straight from the codes
  uint32_t e[E];
  {
    const uint16_t* cd = codes + table * P + cbeg + p0;
    if (full && vec) {
      const uint4* c4 = reinterpret_cast<const uint4*>(cd);
#pragma unroll
      for (int q = 0; q < E / 8; ++q) {
        const uint4 v = c4[q];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t p = static_cast<uint32_t>(p0 + 8 * q + 2 * k);
          e[8 * q + 2 * k] = (w[k] << 16) | p;
          e[8 * q + 2 * k + 1] = (w[k] & 0xffff0000u) | (p + 1);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const uint32_t c = (p0 + i < clen) ? static_cast<uint32_t>(cd[i]) : 0xffffu;
        e[i] = (c << 16) | static_cast<uint32_t>(p0 + i);
      }
    }
  }

  uint32_t* ccol = cnt + swz(tid);              // this thread's counter column
  const int passes = (K + kDigitBits - 1) / kDigitBits;
  for (int r = 0; r < passes; ++r) {
    const int sh = 16 + r * kDigitBits;
    if (r > 0) __syncthreads();                 // every run load of buf is done
#pragma unroll
    for (int w = 0; w < kCntWords; ++w) ccol[w * NTHR] = 0u;
    // own column only: no barrier needed before counting
    // the counter word of an element's digit (recomputed where needed, to
    // keep registers for occupancy)
    auto cword = [&](uint32_t x) { return ccol + __builtin_amdgcn_ubfe(x, sh, 4) * NTHR; };
    uint32_t old[E];
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const uint32_t hb = __builtin_amdgcn_ubfe(e[i], sh + 4, 1);
      old[i] = atomicAdd(cword(e[i]), hb * 0x3fffcu + 4u);    // 4 in the digit's half
    }
    __syncthreads();
    scan_counters<NTHR>(cnt, wave_tot);
    __syncthreads();
    // the ranks' counter words, eight reads in flight at a time: the empty
    // asm makes the addresses be recomputed per group rather than kept live
    // (registers for occupancy), and it orders the groups, so one per
    // element would make every read wait for the one before
    static_assert(E % 8 == 0, "rank reads in groups of 8");
#pragma unroll
    for (int i0 = 0; i0 < E; i0 += 8) {
#pragma unroll
      for (int i = i0; i < i0 + 8; ++i) asm volatile("" : "+v"(e[i]));
      uint32_t rk[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) rk[i] = *cword(e[i0 + i]);
#pragma unroll
      for (int i = 0; i < 8; ++i) old[i0 + i] += rk[i];
    }
    __syncthreads();                            // every rank is read: buf may overwrite the counters
    // old: byte offset of the element's position in the unpadded order; the
    // padded slot adds 16 bytes per 128
    char* bbuf = reinterpret_cast<char*>(buf);
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const uint32_t hs = e[i] >> (sh + 4 - 4) & 16u;     // the digit's half: 0 or 16
      const uint32_t pos4 = __builtin_amdgcn_ubfe(old[i], hs, 16);
      *reinterpret_cast<uint32_t*>(bbuf + pos4 + ((pos4 >> 7) << 4)) = e[i];
    }
    __syncthreads();
    load_run(buf, p0, e);                       // two barriers pass before buf is written again
  }

  // the sorted region.  After a radix pass the chunk sits in LDS in position
  // order, so 8 consecutive entries go to each lane and a wave writes 1 KB
  // of contiguous index array per store, as streaming stores: the tables are
  // read by a later decode, not by anything that runs while they would still
  // be in the cache.  (K = 0 sorts nothing: thread t writes its own run.)
  uint16_t* out = indices + table * P + cbeg;
  if (passes > 0) {
    for (int c = tid; c * 8 < clen; c += NTHR) {
      const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(buf + slot(8 * c));
      const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(buf + slot(8 * c) + 4);
      if (vec && 8 * c + 8 <= clen) {
        const u32x4_t v = {__builtin_amdgcn_perm(lo[1], lo[0], 0x05040100u), __builtin_amdgcn_perm(lo[3], lo[2], 0x05040100u),
                           __builtin_amdgcn_perm(hi[1], hi[0], 0x05040100u), __builtin_amdgcn_perm(hi[3], hi[2], 0x05040100u)};
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(out + 8 * c));
      } else {
        const uint32_t w[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        for (int k = 0; k < 8 && 8 * c + k < clen; ++k) out[8 * c + k] = static_cast<uint16_t>(w[k]);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < E; ++i)
      if (p0 + i < clen) out[p0 + i] = static_cast<uint16_t>(e[i]);
  }

  // bucket starts: st[c] = first position of code c (clen when c is empty),
  // then offsets[c] = min over c' >= c of st[c'] (a suffix minimum).  The
  // code before this thread's run is the last one of the previous thread.
  int prev = __shfl_up(static_cast<int>(e[E - 1] >> 16), 1);
  if (lane == 63) wave_tot[wave] = e[E - 1] >> 16;
  __syncthreads();
  if (lane == 0) prev = wave > 0 ? static_cast<int>(wave_tot[wave - 1]) : -1;
  uint16_t* st = reinterpret_cast<uint16_t*>(smem32);
  for (int c = tid; c < nb; c += nthr) st[c] = static_cast<uint16_t>(clen);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < E; ++i) {
    LSH_CHECK(check, p0 + i >= clen || static_cast<int>(e[i] >> 16) < nb, kChkSortCode);
    const int c = min(static_cast<int>(e[i] >> 16), nb - 1);   // codes are < 2^K
    if (p0 + i < clen && c != prev) st[c] = static_cast<uint16_t>(p0 + i);
    prev = c;
  }
  __syncthreads();
  uint16_t* off = offsets + (table * nJP + j) * nb;
  // thread t owns buckets [t bpt, (t + 1) bpt); suffix minimum across threads
  // through the wave (reversed lane order) and the wave totals
  const int bpt = (nb + nthr - 1) / nthr;
  const int c0 = tid * bpt, c1 = min(nb, c0 + bpt);
  int mine = clen;
  for (int c = c1 - 1; c >= c0; --c) mine = min(mine, static_cast<int>(st[c]));
  int suf = mine;                                   // min over lanes >= lane of this wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_down(suf, o);
    if (lane + o < 64) suf = min(suf, v);
  }
  __syncthreads();                                  // wave_tot is reused
  if (lane == 0) wave_tot[wave] = static_cast<uint32_t>(suf);
  __syncthreads();
  int after = __shfl_down(suf, 1);                  // min over lanes > lane
  if (lane == 63) after = clen;
  const int nw = nthr >> 6;
  for (int w = wave + 1; w < nw; ++w) after = min(after, static_cast<int>(wave_tot[w]));
  for (int c = c1 - 1; c >= c0; --c) {
    after = min(after, static_cast<int>(st[c]));
    off[c] = static_cast<uint16_t>(after);
  }
}

// ---------------------------------------------------------------------------
// Insertion of a few appended keys into built chunks (table updates).
//
// A sequence that gains m <= kInsertMax keys onto built tables has them
// coded and inserted by one workgroup per table, with no projection of the
// rest of the chunk and no sort:
//   - codes: the table's K columns of W go through the same MFMA k-steps as
//     in project_codes, each column in the operand row and each key in the
//     column it takes there, so the codes are bit for bit the build's;
//   - a chunk holding c_old keys gains keys k0 .. k1 - 1 (all larger than its
//     old keys).  In the rebuilt chunk every bucket keeps its old entries in
//     order and appends its new keys after them, so with the new keys ranked
//     by (code, key):
//       new key r lands at ins_r + r, ins_r being the end of its bucket's old
//         segment (its insertion point among the old entries);
//       old entry i moves up by the number of new keys with ins_r <= i;
//       the start of bucket c grows by the number of new codes below c.
//     This is the layout chunk_sort writes from all the chunk's codes.
// The chunk's entries and bucket starts are staged in LDS in the same round
// of loads as the keys and W, before anything is written back, so the shift
// works in place; every write stays inside the chunk's region whatever the
// offsets hold.
// ---------------------------------------------------------------------------
constexpr int kInsertThreads = 256;
static_assert(kInsertMax <= kInsertThreads, "one thread per inserted key");

// The W operand of one projection tile for this lane's row: -W[d][bit]
// over the lane's 32 dims when the row is bit `bit` of the table, else zero
// (the rows of other tables do not touch this table's outputs).  `col` points
// at the lane's 32 dims of the table's column `bit` (any column when the row
// is not the table's): four or eight 16-byte LDS reads, the sign flipped as
// negate() flips it, the row masked afterwards, with no branch.
__device__ __forceinline__ void wfrag_of(Frag<BF16>& f, const uint16_t* col, bool valid) {
  const u32x4_t* q = reinterpret_cast<const u32x4_t*>(col);
  const uint32_t m = valid ? 0xffffffffu : 0u;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const u32x4_t x = q[k];
    const u32x4_t y = {(x[0] ^ 0x80008000u) & m, (x[1] ^ 0x80008000u) & m, (x[2] ^ 0x80008000u) & m,
                       (x[3] ^ 0x80008000u) & m};
    f.v[k] = __builtin_bit_cast(bf16x8_t, y);
  }
}
__device__ __forceinline__ void wfrag_of(Frag<F32>& f, const float* col, bool valid) {
  const u32x4_t* q = reinterpret_cast<const u32x4_t*>(col);
  const uint32_t m = valid ? 0xffffffffu : 0u;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const u32x4_t x = q[k];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) f.v[4 * k + e2] = __uint_as_float((x[e2] ^ 0x80000000u) & m);
  }
}

// A key fragment from the raw 16-byte pieces Frag<T>::load would read (zero
// when the key is not valid).
__device__ __forceinline__ void frag_from_raw(Frag<BF16>& f, const u32x4_t (&r)[4], bool valid) {
  const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int k = 0; k < 4; ++k) f.v[k] = __builtin_bit_cast(bf16x8_t, valid ? r[k] : zero);
}
__device__ __forceinline__ void frag_from_raw(Frag<F32>& f, const u32x4_t (&r)[8], bool valid) {
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int e = 0; e < 4; ++e) f.v[4 * k + e] = valid ? __uint_as_float(r[k][e]) : 0.f;
}

// Dynamic LDS: a chunk's old entries [2^stride_log2], then its bucket
// starts [2^K].
size_t chunk_insert_lds_bytes(int stride_log2, int K) {
  return ((static_cast<size_t>(1) << stride_log2) + (static_cast<size_t>(1) << K)) * 2;
}

template <typename T>
__global__ __launch_bounds__(kInsertThreads) void chunk_insert_kernel(
    const typename T::storage* __restrict__ keys,   // [U][P][128]
    const typename T::storage* __restrict__ W,      // [w_heads][128][L*K]
    uint16_t* __restrict__ codes,         // [U][L][P]: the new keys' codes are written
    int N, int P, int K, int L, int stride_log2, int nJP,
    uint16_t* __restrict__ offsets,       // [U][L][nJP][2^K]
    uint16_t* __restrict__ indices,       // [U][L][P]
    int Hkv, int w_heads, int n_old, const int32_t* __restrict__ old_lens, const int32_t* __restrict__ new_lens
#ifdef LSH_CHECKED
    , uint32_t* check
#endif
    ) {
  using S = typename T::storage;
  extern __shared__ __attribute__((aligned(16))) uint16_t s_dyn[];
  constexpr int kWRow = kHeadDim + 16 / T::bytes;  // padded LDS row (16-byte aligned)
  __shared__ __attribute__((aligned(16))) S s_w[16][kWRow];   // the table's columns of W: [bit][dim]
  __shared__ uint16_t s_new[kInsertMax];           // codes of the sequence's new keys, in key order
  // a chunk's new keys in (code, key) order: code, key, position in the new chunk
  __shared__ uint16_t s_code[kInsertMax], s_key[kInsertMax], s_pos[kInsertMax];
  uint16_t* s_old = s_dyn;                         // a chunk's old entries
  uint16_t* s_off = s_dyn + (1 << stride_log2);    // its bucket starts
  const size_t table = blockIdx.x;                 // u * L + l
  const int u = static_cast<int>(table / L), l = static_cast<int>(table % L);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nb = 1 << K;
  const SeqUpdate su = seq_update(old_lens, new_lens, u / Hkv, n_old, N);
  if (!su.insert || su.old >= su.hi) return;
  const int old = su.old, hi = su.hi;

  // ---- one round of loads: the table's W columns, this wave's first key
  // tile, the first chunk's entries and bucket starts
  const S* Wu = W + (w_heads > 1 ? static_cast<size_t>(u % Hkv) * kHeadDim * L * K : size_t(0));
  S wv[8];                                         // 128 K <= 1920 values
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int i = tid + q * kInsertThreads;
    wv[q] = i < kHeadDim * K ? Wu[static_cast<size_t>(i / K) * L * K + l * K + i % K] : S(0);
  }
  const S* ku = keys + static_cast<size_t>(u) * P * kHeadDim;
  const int tb0 = old >> 4, ntile = ((hi - 1) >> 4) - tb0 + 1;   // 16-key tiles holding new keys
  const int g = lane >> 4, col = lane & 15;
  // key n in column n % 16, as in project_codes: the lane's 32 dims as raw
  // 16-byte pieces, masked only when the fragment is formed, so that the
  // loads stay in flight with the others until the barrier
  constexpr int kKeyQ = 2 * T::bytes;              // 16-byte pieces per lane
  u32x4_t kraw[kKeyQ];
  auto key_of = [&](int kt) { return (tb0 + kt) * 16 + col; };
  auto load_keys = [&](int kt) {
    const int n = key_of(kt);
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(
        ku + static_cast<size_t>(n >= old && n < hi ? n : old) * kHeadDim + g * 32);
#pragma unroll
    for (int k = 0; k < kKeyQ; ++k) kraw[k] = src[k];
  };
  if (K > 0 && wave < ntile) load_keys(wave);
  // a chunk's old entries and bucket starts go to LDS in 16-byte pieces
  // where aligned: the first four pieces per thread of each (all entries of
  // a chunk, the bucket starts up to K = 13) are loaded straight-line, with
  // no loop whose head would wait for the loads before it
  const int j1 = old >> stride_log2;
  auto chunk_old = [&](int j) { return max(0, min(old, (j + 1) << stride_log2) - (j << stride_log2)); };
  auto ib_of = [&](int j) { return indices + table * P + (j << stride_log2); };
  auto ob_of = [&](int j) { return offsets + (table * nJP + j) * static_cast<size_t>(nb); };
  auto pieces = [&](const uint16_t* p, int n) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0 ? n >> 3 : 0; };
  u32x4_t ev[4], ov[4];
  auto stage_issue = [&](int j) {
    const int c_old = chunk_old(j);
    const int ne8 = pieces(ib_of(j), c_old), no8 = c_old > 0 ? pieces(ob_of(j), nb) : 0;
    const u32x4_t* e4 = reinterpret_cast<const u32x4_t*>(ib_of(j));
    const u32x4_t* o4 = reinterpret_cast<const u32x4_t*>(ob_of(j));
    const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = tid + q * kInsertThreads;
      ev[q] = i < ne8 ? e4[i] : zero;
      ov[q] = i < no8 ? o4[i] : zero;
    }
  };
  auto stage_commit = [&](int j) {
    const int c_old = chunk_old(j);
    const uint16_t* ib = ib_of(j);
    const uint16_t* ob = ob_of(j);
    const int ne8 = pieces(ib, c_old), no8 = c_old > 0 ? pieces(ob, nb) : 0;
    u32x4_t* so4 = reinterpret_cast<u32x4_t*>(s_old);
    u32x4_t* sf4 = reinterpret_cast<u32x4_t*>(s_off);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = tid + q * kInsertThreads;
      if (i < ne8) so4[i] = ev[q];
      if (i < no8) sf4[i] = ov[q];
    }
    // the rest: bucket starts past the first pieces (K >= 14), the last
    // entries or starts short of a piece, unaligned regions
    for (int i = 4 * kInsertThreads + tid; i < no8; i += kInsertThreads)
      sf4[i] = reinterpret_cast<const u32x4_t*>(ob)[i];
    for (int i = 8 * ne8 + tid; i < c_old; i += kInsertThreads) s_old[i] = ib[i];
    if (c_old > 0)
      for (int i = 8 * no8 + tid; i < nb; i += kInsertThreads) s_off[i] = ob[i];
  };
  stage_issue(j1);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int i = tid + q * kInsertThreads;
    if (i < kHeadDim * K) s_w[i % K][i / K] = wv[q];
  }
  stage_commit(j1);
  __syncthreads();

  // ---- codes of the new keys.  Table l is table tt of lane group gl of its
  // slab; its bit b is row position jr = P - 1 - j = tt K + b of that group
  // (j = 4 ct + i: tile ct, row 4 gl + i), as laid out by transpose_w_kernel
  if (K > 0) {
    const ProjShape ps = proj_shape(K);
    const int P4 = 4 * ps.nct;
    const int tt = l % ps.tpg, gl = (l / ps.tpg) % 4;
    const int jlo = P4 - tt * K - K;                 // the table's bits: positions jlo .. jlo + K - 1
    // this lane's operand row in tile ct: bit of the table, or -1
    auto row_bit = [&](int ct) {
      const int r = col, jr = P4 - 1 - (4 * ct + (r & 3));
      return ((r >> 2) == gl && jr >= tt * K && jr < tt * K + K) ? jr - tt * K : -1;
    };
    static_assert(kWRow * T::bytes % 16 == 0, "16-byte LDS rows");
    for (int kt = wave; kt < ntile; kt += kInsertThreads / 64) {
      if (kt != wave) load_keys(kt);
      const bool kvalid = key_of(kt) >= old && key_of(kt) < hi;
      Frag<T> Kf;
      frag_from_raw(Kf, kraw, kvalid);
      uint32_t code = 0;
      for (int ct = jlo >> 2; ct <= (jlo + K - 1) >> 2; ++ct) {
        Frag<T> Wf;
        const int bit = row_bit(ct);
        wfrag_of(Wf, &s_w[bit < 0 ? 0 : bit][32 * g], bit >= 0);
        floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < 4; ++k) Wf.mma_step(k, Kf, acc);
        // lane (g, col) holds rows 4 g + i: bit jr - tt K of the code
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int jr = P4 - 1 - (4 * ct + i);
          if (g == gl && jr >= tt * K && jr < tt * K + K)
            code |= (__float_as_uint(acc[i]) >> 31) << (jr - tt * K);
        }
      }
      const int n = (tb0 + kt) * 16 + col;
      if (g == gl && n >= old && n < hi) {
        s_new[n - old] = static_cast<uint16_t>(code);
        codes[table * P + n] = static_cast<uint16_t>(code);
      }
    }
  } else {
    for (int n = old + tid; n < hi; n += kInsertThreads) {
      s_new[n - old] = 0;
      codes[table * P + n] = 0;
    }
  }
  __syncthreads();

  // ---- insertion, chunk by chunk (one or two chunks)
  for (int j = j1; j <= (hi - 1) >> stride_log2; ++j) {
    const int cbeg = j << stride_log2, cend = cbeg + (1 << stride_log2);
    const int k0 = max(old, cbeg), k1 = min(hi, cend);
    const int m = min(k1 - k0, kInsertMax);          // >= 1
    const int c_old = max(0, min(old, cend) - cbeg);   // old entries of the chunk
    uint16_t* ob = offsets + (table * nJP + j) * static_cast<size_t>(nb);
    uint16_t* ib = indices + table * P + cbeg;
    if (j != j1) {
      stage_issue(j);
      stage_commit(j);
      __syncthreads();
    }
    if (tid < m) {
      const int c = s_new[k0 - old + tid];
      LSH_CHECK(check, c < nb, kChkInsert);
      int r = 0;                                     // rank by (code, key)
      for (int s = 0; s < m; ++s) {
        const int cs = s_new[k0 - old + s];
        r += (cs < c || (cs == c && s < tid)) ? 1 : 0;
      }
      // insertion point: the end of bucket c's old segment
      const int end = c_old == 0 ? 0 : (c + 1 < nb ? static_cast<int>(s_off[c + 1]) : c_old);
      LSH_CHECK(check, end <= c_old, kChkInsert);
      s_code[r] = static_cast<uint16_t>(c);
      s_key[r] = static_cast<uint16_t>(k0 + tid - cbeg);
      s_pos[r] = static_cast<uint16_t>(min(end, c_old) + r);
    }
    __syncthreads();
    // the rewritten span [a0, c_old + m), a0 = the first insertion point
    // rounded down to 8 entries, in 16-byte pieces: a thread forms each of
    // its pieces in registers, walking the new keys' positions (old entry
    // i moves up by the new keys placed before it), and stores it at once
    const int a0 = s_pos[0] & ~7, e1 = c_old + m;
    const bool vec = (reinterpret_cast<uintptr_t>(ib) & 15) == 0;
    for (int o0 = a0 + 8 * tid; o0 < e1; o0 += 8 * kInsertThreads) {
      int lo = 0, hi2 = m;                           // new keys placed before o0
      while (lo < hi2) {
        const int mid = (lo + hi2) >> 1;
        if (static_cast<int>(s_pos[mid]) < o0) lo = mid + 1;
        else hi2 = mid;
      }
      int nx = lo, npos = nx < m ? static_cast<int>(s_pos[nx]) : INT_MAX;
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int o = o0 + q;
        uint32_t v;
        if (o == npos) {
          v = s_key[nx];
          ++nx;
          npos = nx < m ? static_cast<int>(s_pos[nx]) : INT_MAX;
        } else {
          v = s_old[min(max(o - nx, 0), max(c_old - 1, 0))];
        }
        if (q & 1) w[q >> 1] |= v << 16;
        else w[q >> 1] = v;
      }
      if (vec && o0 + 8 <= e1) {
        *reinterpret_cast<u32x4_t*>(ib + o0) = u32x4_t{w[0], w[1], w[2], w[3]};
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (o0 + q < e1) ib[o0 + q] = static_cast<uint16_t>(w[q >> 1] >> (16 * (q & 1)));
      }
    }
    // bucket starts: + the new codes below c (a chunk without old keys is
    // written whole; otherwise pieces past the smallest new code's), eight
    // per 16-byte piece
    const int cs = c_old == 0 ? 0 : (s_code[0] + 1) & ~7;
    const bool ovec = nb >= 8 && (reinterpret_cast<uintptr_t>(ob) & 15) == 0;
    for (int c0 = cs + 8 * tid; c0 < nb; c0 += 8 * kInsertThreads) {
      int lt = 0, hi2 = m;                           // new codes below c0
      while (lt < hi2) {
        const int mid = (lt + hi2) >> 1;
        if (static_cast<int>(s_code[mid]) < c0) lt = mid + 1;
        else hi2 = mid;
      }
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int c = c0 + q;
        while (lt < m && static_cast<int>(s_code[lt]) < c) ++lt;
        const uint32_t v = static_cast<uint32_t>((c_old == 0 || c >= nb ? 0 : static_cast<int>(s_off[c])) + lt) & 0xffffu;
        if (q & 1) w[q >> 1] |= v << 16;
        else w[q >> 1] = v;
      }
      if (ovec) {
        *reinterpret_cast<u32x4_t*>(ob + c0) = u32x4_t{w[0], w[1], w[2], w[3]};
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (c0 + q < nb) ob[c0 + q] = static_cast<uint16_t>(w[q >> 1] >> (16 * (q & 1)));
      }
    }
    __syncthreads();                                 // LDS reused by the next chunk
  }
}

// Block size for a chunk of 2^stride_log2 keys, and the LDS it needs.
static int sort_threads(int stride_log2) { return max(64, (1 << stride_log2) / kSortE); }

size_t chunk_sort_lds_bytes(int stride_log2, int K) {
  const size_t nthr = static_cast<size_t>(sort_threads(stride_log2));
  const size_t elems = nthr * kSortE;
  return max(max(kCntWords * nthr, elems + (elems >> 3)) * 4, size_t(2) << K);
}

template <int NTHR>
static hipError_t launch_chunk_sort(const BuildArgs& a, hipStream_t stream) {
  const size_t lds = chunk_sort_lds_bytes(a.stride_log2, a.K);
  hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(chunk_sort_kernel<NTHR>), lds);
  if (e != hipSuccess) return e;
  return launch(kKChunkSort, chunk_sort_kernel<NTHR>, dim3(a.nJ - a.j0, a.U * a.L), dim3(NTHR),
                static_cast<unsigned>(lds), stream, static_cast<const uint16_t*>(a.codes), a.N, a.P, a.K,
                a.stride_log2, a.nJP, a.j0, a.offsets, a.indices, a.L, a.Hkv, a.n_old, a.old_lens, a.new_lens
#ifdef LSH_CHECKED
                , g_check
#endif
                );
}

// ---------------------------------------------------------------------------
// Host-side launchers
// ---------------------------------------------------------------------------

template <typename T, int KB>
static hipError_t launch_project_k(const BuildArgs& a, int nslab, hipStream_t stream) {
  using S = typename T::storage;
  const int n_first = a.j0 << a.stride_log2;
  const int gx = (a.N - n_first + kProjKeys - 1) / kProjKeys;
  // a short key range (a table update) has too few key blocks to fill the
  // chip: its slabs are then dealt over up to ~1024 workgroups in all
  const long long gxy = static_cast<long long>(gx) * a.U;
  const int zwant = static_cast<int>(std::min<long long>(nslab, std::max<long long>(1, (1023 + gxy) / gxy)));
  const int spz = (nslab + zwant - 1) / zwant;
  const int gz = (nslab + spz - 1) / spz;
  return launch(kKProject, project_codes_kernel<T, KB>, dim3(gx, a.U, gz), dim3(kProjThreads), 0, stream,
                static_cast<const S*>(a.keys), static_cast<const S*>(a.wt), a.codes, a.N, a.P, n_first, a.L,
                nslab, a.n_old, spz, a.Hkv,
                a.w_heads > 1 ? static_cast<size_t>(nslab) * proj_shape(KB).nct * 16 * kHeadDim : size_t(0),
                a.old_lens, a.new_lens, a.stride_log2);
}

template <typename T>
static hipError_t launch_project(const BuildArgs& a, hipStream_t stream) {
  using S = typename T::storage;
  const int K = a.K, L = a.L;
  if (K == 0) {
    const int n_first = a.j0 << a.stride_log2;
    const size_t rows = static_cast<size_t>(a.U) * L;
    const size_t n = rows * static_cast<size_t>(a.N - n_first);
    return launch(kKProject, zero_codes_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream,
                  a.codes, rows, n_first, a.N, a.P, L, a.n_old, a.Hkv, a.old_lens, a.new_lens, a.stride_log2);
  }
  const ProjShape ps = proj_shape(K);
  const int rows = proj_wt_rows(K, L);
  const int nslab = rows / (ps.nct * 16);
  hipError_t e = launch(kKTransposeW, transpose_w_kernel<T>, dim3((a.w_heads * rows * kHeadDim + 255) / 256),
                        dim3(256), 0, stream, static_cast<const S*>(a.W), static_cast<S*>(a.wt), K, L, ps.nct,
                        ps.tpg, rows, a.w_heads);
  if (e != hipSuccess) return e;
  switch (K) {
    case 1: return launch_project_k<T, 1>(a, nslab, stream);
    case 2: return launch_project_k<T, 2>(a, nslab, stream);
    case 3: return launch_project_k<T, 3>(a, nslab, stream);
    case 4: return launch_project_k<T, 4>(a, nslab, stream);
    case 5: return launch_project_k<T, 5>(a, nslab, stream);
    case 6: return launch_project_k<T, 6>(a, nslab, stream);
    case 7: return launch_project_k<T, 7>(a, nslab, stream);
    case 8: return launch_project_k<T, 8>(a, nslab, stream);
    case 9: return launch_project_k<T, 9>(a, nslab, stream);
    case 10: return launch_project_k<T, 10>(a, nslab, stream);
    case 11: return launch_project_k<T, 11>(a, nslab, stream);
    case 12: return launch_project_k<T, 12>(a, nslab, stream);
    case 13: return launch_project_k<T, 13>(a, nslab, stream);
    case 14: return launch_project_k<T, 14>(a, nslab, stream);
    case 15: return launch_project_k<T, 15>(a, nslab, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
static hipError_t launch_insert(const BuildArgs& a, hipStream_t stream) {
  using S = typename T::storage;
  if (a.stride_log2 > 13) return hipErrorInvalidValue;
  const size_t lds = chunk_insert_lds_bytes(a.stride_log2, a.K);
  hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(chunk_insert_kernel<T>), lds);
  if (e != hipSuccess) return e;
  return launch(kKChunkInsert, chunk_insert_kernel<T>, dim3(static_cast<unsigned>(a.U * a.L)),
                dim3(kInsertThreads), static_cast<unsigned>(lds), stream, static_cast<const S*>(a.keys),
                static_cast<const S*>(a.W), a.codes, a.N, a.P, a.K, a.L, a.stride_log2, a.nJP, a.offsets, a.indices,
                a.Hkv, a.w_heads, a.n_old, a.old_lens, a.new_lens
#ifdef LSH_CHECKED
                , g_check
#endif
                );
}

// A build, or an update: sequences whose new keys are inserted go through
// chunk_insert alone; the others through the projection and chunk_sort.
hipError_t launch_build(const BuildArgs& a, hipStream_t stream) {
  hipError_t e = hipSuccess;
  if (a.mode & kUpdateInsert) {
    e = (a.dtype == 1) ? launch_insert<BF16>(a, stream) : launch_insert<F32>(a, stream);
    if (e != hipSuccess || !(a.mode & kUpdateSort)) return e;
  }
  e = (a.dtype == 1) ? launch_project<BF16>(a, stream) : launch_project<F32>(a, stream);
  if (e != hipSuccess) return e;
  switch (sort_threads(a.stride_log2)) {
    case 64: return launch_chunk_sort<64>(a, stream);
    case 128: return launch_chunk_sort<128>(a, stream);
    case 256: return launch_chunk_sort<256>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lsh
