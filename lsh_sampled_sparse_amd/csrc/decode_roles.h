// Workgroup roles of the one-launch decode (gfx950): the per-(query head,
// key chunk) collision count and selection, and the log-sum-exp merges; the
// attention role itself lives with its dtype's kernel.
//
// One grid holds, in this order of workgroup id,
//   count    workgroups: one per (key chunk, query head), the selection bitmask
//   attend   workgroups: one per (context split, sequence, kv head)
// An attend workgroup waits, by polling a counter in the workspace, for the
// count workgroups of its split's chunks, all of LOWER id.  Workgroups of a
// launch are dispatched in id order (on each XCD in the order of the ids it
// receives), so every producer has been dispatched before any workgroup that
// waits for it, and producers never wait: the waits always end.  A bounded
// poll count turns a wait that does not end into a NaN output instead of a
// hang.
//
// Cross-workgroup data (bitmask words, chunk counts, partial states, the
// counters) is written with agent-scope atomic stores, which write through
// to memory and so stay coherent across the eight XCDs (whose L2s are not
// coherent with each other for plain accesses).  A producer waits for its
// stores to complete (s_waitcnt vmcnt(0)) before it bumps the counter a
// consumer polls.  Consumers read small data (bitmask words) with
// agent-scope atomic loads; the finishers, which read a unit's partial
// states in bulk, issue one agent-scope acquire fence and then plain loads.
// Fences in every workgroup are avoided: an L2 write-back or invalidate per
// workgroup costs far more than these few coherent accesses.
//
// The merge: each attend workgroup writes one partial state (acc,
// max, sum) per query head of its group; the last workgroups of a (sequence,
// kv head) to finish fold them into the outputs (finish_slot).  Folds run in
// slot order, whoever runs them, so the result is deterministic.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "lsh_device.h"
#include "lsh_kernels.h"

namespace lsh {

constexpr int kFusedThreads = 256;         // every role runs 4 waves
// An attention role's ring entry: the key index, with this bit set for a key
// of the hybrid decode's exact set (every head of the group, ln u = 0)
constexpr int kExactKey = static_cast<int>(0x80000000u);
constexpr int kSpinLimit = 1 << 18;        // polls before a wait gives up (a fraction of a second)

// --------------------------------------------------------------------------
// coherent accesses
// --------------------------------------------------------------------------
__device__ __forceinline__ void st_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(float* p, float v) {
  st_agent(reinterpret_cast<uint32_t*>(p), __float_as_uint(v));
}
__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_agent(const int32_t* p) {
  return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __uint_as_float(ld_agent(reinterpret_cast<const uint32_t*>(p)));
}
__device__ __forceinline__ uint64_t ld_agent(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// every vector memory access of this wave has completed (gfx9: vmcnt counts stores too)
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Thread 0 polls *ctr until it reaches `target`; the workgroup then
// proceeds.  Returns false (in every thread) when the poll limit ran out.
__device__ __forceinline__ bool wait_counter(const int32_t* ctr, int target, int* flag_lds) {
  if (threadIdx.x == 0) {
    int ok = 1, it = 0;
    while (ld_agent(ctr) < target) {
      __builtin_amdgcn_s_sleep(2);
      if (++it >= kSpinLimit) {
        ok = 0;
        break;
      }
    }
    *flag_lds = ok;
  }
  __syncthreads();
  const bool ok = *flag_lds != 0;
  __syncthreads();
  return ok;
}

// Every thread polls its share of ctr[0 .. n) until each reaches `target`.
// Returns false (in every thread) when a poll limit ran out.
__device__ __forceinline__ bool wait_counters(const int32_t* ctr, int n, int target, int* flag_lds) {
  if (threadIdx.x == 0) *flag_lds = 1;
  __syncthreads();
  int ok = 1;
  for (int j = threadIdx.x; j < n; j += blockDim.x) {
    int it = 0;
    while (ld_agent(ctr + j) < target) {
      __builtin_amdgcn_s_sleep(2);
      if (++it >= kSpinLimit) {
        ok = 0;
        break;
      }
    }
  }
  if (!ok) *flag_lds = 0;
  __syncthreads();
  const bool all = *flag_lds != 0;
  __syncthreads();
  return all;
}

// This workgroup's stores are complete; thread 0 then adds 1 to *ctr and
// returns the previous value (the same in every thread).
__device__ __forceinline__ int arrive(int32_t* ctr, int* val_lds) {
  wait_vmem();
  __syncthreads();
  if (threadIdx.x == 0) *val_lds = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int v = *val_lds;
  __syncthreads();
  return v;
}

// This workgroup's stores are complete; thread 0 then adds 1 to *ctr
// without waiting for the add to return (a workgroup that only signals).
__device__ __forceinline__ void signal(int32_t* ctr, int add = 1) {
  wait_vmem();
  __syncthreads();
  if (threadIdx.x == 0) (void)__hip_atomic_fetch_add(ctr, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// --------------------------------------------------------------------------
// Parameters of the one-launch decode
// --------------------------------------------------------------------------
struct FusedParams {
  const void* q;               // [B][Hq][128]
  const void* keys;            // [U][P][128]
  const void* values;          // [U][P][128]
  const uint16_t* indices;     // [U][L][P] chunk-major
  const uint16_t* offsets;     // [U][L][nJP][2^K]
  const int32_t* seq_lens;     // optional [B]
  const uint16_t* qcodes;      // [BH][L] (written by the query-hash launch)
  uint32_t* bitmask;           // [BH][Nw]
  int32_t* chunk_nsel;         // [BH][nJ]
  const double* lnu_samples;   // [kLnuSamples] g at theta_t = t pi / (2 kLnuTable) (query-hash launch)
  float* partials;             // [BH][npart][kPartialStride]
  int32_t* ready;              // [U][nJ] count workgroups done per (unit, chunk)
  int32_t* arrive_unit;        // [U] partial slots written per unit
  float* out;                  // [BH][128]
  float* lse;                  // optional [BH]
  int32_t* nsel;               // optional [BH]
  uint8_t* counts;             // optional [BH][N]
  int B, Hq, Hkv, G, N, P, K, L, T;
  int stride_log2, nJ, nJP;
  int split_len, nsplit, n_sink, n_window;
  int npart;
  int n_count_wg, n_attend_wg;
  int unit_group;              // units whose splits are dispatched interleaved (decode_role)
  int count_heads;             // query heads of one unit per count workgroup (divides G)
  float scale;
#ifdef LSH_TRACE
  unsigned long long* trace;   // [grid][16] phase timestamps (trace builds only)
#endif
#ifdef LSH_CHECKED
  uint32_t* check;             // violation bits (checked builds only)
#endif
};
#ifdef LSH_CHECKED
#define LSH_PCHECK(p, cond, bit) LSH_CHECK((p).check, cond, bit)
#else
#define LSH_PCHECK(p, cond, bit) do { } while (0)
#endif

// Phase timestamps of a workgroup (s_memrealtime, 100 MHz), recorded only in
// builds with LSH_TRACE defined; a profiling aid, compiled out otherwise.
#ifdef LSH_TRACE
#define LSH_STAMP(p, k) \
  do { if (threadIdx.x == 0 && (p).trace) (p).trace[blockIdx.x * 16 + (k)] = __builtin_amdgcn_s_memrealtime(); } while (0)
#else
#define LSH_STAMP(p, k) do { } while (0)
#endif

// Sync words the query-hash launch zeroes before the decode launch.
__host__ __device__ inline int fused_sync_words(int U, int nJ) { return U * nJ + U; }

// What workgroup `wid` of the decode launch does.  The grid holds every
// count workgroup first (chunk by chunk, one per count_heads query heads of
// a unit), then the
// attention workgroups of the units, a group of R units at a time
// (R = unit_group): within a group, the context splits of its units, split
// 0 of every unit of the group, then split 1, and so on.  Attention
// workgroups that take the later slots of a CU stream more slowly while the
// earlier ones run, so this gives every unit of a group its share of early
// and late slots and the units end together, instead of the last-dispatched
// unit ending last.
// Progress: count workgroups come before every attention workgroup and never
// wait; a unit's finishers wait only for workgroups of their own unit, and
// only the R units of the group being dispatched can still have workgroups
// waiting for a slot, so at most R * F finishers (F per unit, R * F <= 64)
// wait while the rest of the resident workgroups run and leave.
// (Placing each unit's count workgroups just before its attention
// workgroups, so that later units count while earlier ones stream, measured
// slower at every size tried, from 4 units of 128K keys to 512 units of 32K:
// attention workgroups held their slots while they waited, and the count
// workgroups of later units got slots late.)
struct DecodeRole {
  bool count;
  int u;
  int J, bh;       // count: key chunk and query head
  int slot;        // attention: context split
};

__device__ inline DecodeRole decode_role(const FusedParams& p, int wid) {
  DecodeRole r;
  const int U = p.B * p.Hkv;
  r.count = wid < p.n_count_wg;
  if (r.count) {
    // (unit, chunk) pairs in chunk-major order, pair = J * U + u, each with
    // Gh = G / count_heads workgroups; pairs in blocks of 8 so that workgroup
    // w of a block runs on XCD w mod 8 with all Gh workgroups of its pair
    // (the heads of a unit often probe the same bucket, whose entries the
    // XCD's L2 then serves after the first read), the last P mod 8 pairs
    // one after another
    const int Gh = p.G / p.count_heads;
    const int P8 = (U * p.nJ) & ~7;
    int pair, s;
    if (wid < P8 * Gh) {
      const int y = wid >> 3;
      pair = (y / Gh) * 8 + (wid & 7);
      s = y % Gh;
    } else {
      const int k = wid - P8 * Gh;
      pair = P8 + k / Gh;
      s = k % Gh;
    }
    r.J = pair / U;
    r.u = pair - r.J * U;
    r.bh = r.u * p.G + s * p.count_heads;                    // the first of its count_heads heads
    r.slot = 0;
    return r;
  }
  r.J = 0;
  r.bh = 0;
  const int k = wid - p.n_count_wg;
  const int grp = k / (p.unit_group * p.nsplit);            // group of units
  const int u0 = grp * p.unit_group;
  const int R = min(p.unit_group, U - u0);                   // units in this group
  const int i = k - u0 * p.nsplit;                           // position in the group
  r.u = u0 + i % R;                                          // splits, split by split
  r.slot = i / R;
  return r;
}

// --------------------------------------------------------------------------
// The ln-u correction g(theta), sampled by the query-hash launch
// --------------------------------------------------------------------------
__device__ __forceinline__ double wave_max_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// g(theta) = ln sum_{i=T}^{L} C(L,i) P^(i-T) (1-P)^(L-i), P = (1 - theta/pi)^K,
// by one wave: lane handles the terms i = T + lane + 64 k, whose log binomial
// coefficients are lc[i] = ln C(L, i); a log-sum-exp over the wave.
__device__ inline double lnu_correction_wave(double theta, int K, int L, int T, const double* lc, int lane) {
  // the exponents are sums of large terms, so they are formed in fp64; the
  // exponentials of their differences from the maximum lie in (0, 1] and a
  // float keeps their relative precision, so those run in fp32
  const double lp = log1p(-theta / 3.14159265358979323846);   // ln p
  const double lP = (K == 0) ? 0.0 : K * lp;                      // ln P
  const double lQ = (K == 0) ? -INFINITY : log(-expm1(lP));      // ln(1 - P)
  double t[4];
  double m = -INFINITY;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = T + lane + 64 * k;
    double x = -INFINITY;
    if (i <= L) {
      x = lc[i];
      if (i > T) x += (i - T) * lP;   // the zero power is 1: skip 0 * ln 0
      if (L > i) x += (L - i) * lQ;
    }
    t[k] = x;
    m = fmax(m, x);
  }
  m = wave_max_f64(m);
  float sum = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (t[k] != -INFINITY) sum += __expf(static_cast<float>(t[k] - m));
  sum = wave_sum(sum);
  return m + static_cast<double>(__logf(sum));
}

// The ln-u interval quadratics for the attention role, from the fp64
// samples the query-hash launch wrote (plain loads: that launch has
// completed).  lnu_fetch issues this thread's loads (four intervals, three
// samples each) so they can be in flight while the workgroup waits for its
// selection; lnu_store forms the quadratics in LDS (zeros when no ln u is
// needed).
struct LnuFetch {
  double g[kLnuTable / kFusedThreads][3];
};
__device__ __forceinline__ void lnu_fetch(const FusedParams& p, bool nolnu, LnuFetch& r) {
  if (nolnu) return;
#pragma unroll
  for (int q = 0; q < kLnuTable / kFusedThreads; ++q) {
    const int j = threadIdx.x + q * kFusedThreads;
#pragma unroll
    for (int t = 0; t < 3; ++t) r.g[q][t] = p.lnu_samples[2 * j + t];
  }
}
__device__ __forceinline__ void lnu_store(const LnuFetch& r, bool nolnu, float4* tab) {
#pragma unroll
  for (int q = 0; q < kLnuTable / kFusedThreads; ++q) {
    const int j = threadIdx.x + q * kFusedThreads;
    float4 e = make_float4(0.f, 0.f, 0.f, 0.f);
    if (!nolnu) {
      const double g0 = r.g[q][0], gm = r.g[q][1], g1 = r.g[q][2];
      e = make_float4(static_cast<float>(g0), static_cast<float>(-3.0 * g0 + 4.0 * gm - g1),
                      static_cast<float>(2.0 * g0 - 4.0 * gm + 2.0 * g1), 0.f);
    }
    tab[j] = e;
  }
}

// --------------------------------------------------------------------------
// Count role: one workgroup per (key chunk J, query head bh).  For every table
// the segment of the probed bucket inside chunk J is read in aligned 16-byte
// blocks of 8 entries (entries outside the segment are skipped), and each
// entry adds 1 to its key's byte counter in LDS.  Keys with count >= T, not in
// the exact set and within the sequence, form the selection bitmask.
//
// The blocks of all tables are concatenated (a scan of the per-table block
// counts) and every wave walks a contiguous range of them, 16 blocks in
// flight per lane; each block's segment comes from a map of the segments'
// first blocks (a bitmap, its per-row prefix counts and the list of
// non-empty tables), or for very long walks from a binary search over the
// scan.  Reading whole aligned blocks may read up to 14 bytes past a segment,
// inside the 16-byte block that holds its first or last entry (never past the
// 16-byte granule of the indices array's last entry).
// --------------------------------------------------------------------------
constexpr int kCountInflight = 16;

constexpr int kSegMapRows = 512;   // walks of up to 512 x 64 blocks use the segment map

// A count workgroup walks the segments of count_heads (hc) query heads of one
// unit: segment hh * L + l is head hh's bucket in table l.
constexpr int kCountSegs = 1024;                 // hc * L <= kCountSegs
constexpr int kCountCounterBytes = 32 << 10;     // byte counters: hc << stride_log2 <= this
constexpr int kSegsPerThread = kCountSegs / kFusedThreads;
constexpr int kCountRankShift = 21;              // scan word: blocks (low 21 bits), non-empty rank (high 11)

// A segment as the walk reads it, one 16-byte LDS read per block: its first
// block (low 56 bits; its head, 0 .. hc - 1, in the top 8), the exclusive
// scan of the block counts at it, and its entries [lo, hi) counted from the
// first block's first entry.
struct __attribute__((aligned(16))) SegInfo {
  long long fb;
  int v;
  short lo, hi;
};
constexpr long long kSegBlockMask = (1ll << 56) - 1;

struct CountLds {                  // laid out after the byte counters (a multiple of 256 bytes)
  SegInfo seg[kCountSegs + 1];     // the segments; seg[S].v = the total block count
  uint64_t starts[kSegMapRows];    // segment map: bit v & 63 of row v >> 6 marks a segment's first block
  int pre[kSegMapRows + 1];        // segment map: set bits in the rows before each row
  uint16_t seglist[kCountSegs];    // segment map: the non-empty segments, in order
  uint32_t spare[64];              // trace builds: keeps the traced loads alive
  uint32_t wtot[kSegsPerThread][kFusedThreads / 64];   // scan: per row of segments and wave
  int hsel[16][kFusedThreads / 64];   // selected keys per head and wave
  int flag;
};

// The bits of a bitmask word whose keys may be selected, for the word whose
// first key is k0: keys below kend (the sequence's keys in the chunk), at or
// above exact_head and below tail_start (outside the exact set).  The same
// for every head, so it is formed once per word.
__device__ __forceinline__ uint32_t bits_below(int x) { return x <= 0 ? 0u : (x >= 32 ? ~0u : (1u << x) - 1u); }
__device__ __forceinline__ uint32_t selectable_bits(int k0, int kend, int exact_head, int tail_start) {
  return bits_below(kend - k0) & ~bits_below(exact_head - k0) & bits_below(tail_start - k0);
}
// Bit k set when byte k of c4 (a key's collision count) is at least T.
__device__ __forceinline__ uint32_t counts_at_least(uint32_t c4, int T) {
  uint32_t r = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) r |= static_cast<int>((c4 >> (8 * k)) & 0xffu) >= T ? (1u << k) : 0u;
  return r;
}

// One query head per workgroup: thread l takes table l (L <= 255).
__device__ inline void count_role(const FusedParams& p, int J, int bh, unsigned char* smem) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = bh / p.Hq, h = bh % p.Hq;
  const int u = b * p.Hkv + h / p.G;
  const int nb = 1 << p.K;
  const int sl = p.stride_log2;
  const int cbeg = J << sl;
  uint32_t* cnt = reinterpret_cast<uint32_t*>(smem);                     // one byte per key of the chunk
  CountLds& s = *reinterpret_cast<CountLds*>(smem + (1 << sl));
  const int Nb = seq_len_of(p.seq_lens, b, p.N);
  const int cfull = min(1 << sl, p.N - cbeg);
  const int clen = max(0, min(1 << sl, Nb - cbeg));
  const int cwords = (cfull + 3) >> 2;
  int exact_head, exact_tail;
  exact_range(p.n_sink, p.n_window, Nb, exact_head, exact_tail);

  LSH_STAMP(p, 0);
  for (int i = tid; i < cwords; i += kFusedThreads) cnt[i] = 0;

  // segment of bucket qcode_l inside this chunk, in blocks, for table l = tid
  int nblk = 0;
  if (tid < p.L && clen > 0) {
    // (the query hash writes codes below 2^K; the mask keeps any other value
    // inside the chunk's bucket starts, and the checked build reports it)
    const int qraw = p.qcodes[static_cast<size_t>(bh) * p.L + tid];
    LSH_PCHECK(p, qraw < nb, kChkQueryCode);
    const int qc = qraw & (nb - 1);
    const size_t row = static_cast<size_t>(u) * p.L + tid;
    const uint16_t* op = p.offsets + (row * p.nJP + J) * nb + qc;
    LSH_PCHECK(p, static_cast<int>(op[0]) <= (qc + 1 < nb ? static_cast<int>(op[1]) : clen) &&
                      (qc + 1 < nb ? static_cast<int>(op[1]) : static_cast<int>(op[0])) <= clen,
               kChkSegment);
    // clamped into the chunk: tables of another stride cannot send the walk out of it
    const int s0 = min(static_cast<int>(op[0]), clen);
    const int e0 = qc + 1 < nb ? min(static_cast<int>(op[1]), clen) : clen;
    const size_t first = row * p.P + cbeg + s0;      // element index of the segment's first entry
    const int lo = static_cast<int>(first & 7);
    const int len = max(e0 - s0, 0);
    nblk = len > 0 ? (lo + len + 7) >> 3 : 0;
    s.seg[tid].fb = static_cast<long long>(first >> 3);
    s.seg[tid].lo = static_cast<short>(lo);
    s.seg[tid].hi = static_cast<short>(lo + len);
  }
  // one scan gives the block offsets (low 24 bits) and the rank of each
  // non-empty segment among them (high 8 bits)
  const uint32_t own = static_cast<uint32_t>(nblk) + (nblk > 0 ? (1u << 24) : 0u);
  uint32_t incl = own;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  if (lane == 63) s.wtot[0][wave] = incl;
  __syncthreads();
  {
    uint32_t wbase = 0;
    for (int w = 0; w < wave; ++w) wbase += s.wtot[0][w];
    incl += wbase;
    s.seg[tid + 1].v = static_cast<int>(incl & 0xffffffu);
    if (tid == 0) s.seg[0].v = 0;
    if (nblk > 0) s.seglist[(incl - own) >> 24] = static_cast<uint8_t>(tid);
  }
  __syncthreads();
  LSH_STAMP(p, 1);

  // the walk's bounds are wave-uniform (scalar), so the steps below need no
  // per-lane branches
  const int total = __builtin_amdgcn_readfirstlane(s.seg[p.L].v);
  // segment map (walks of at most kSegMapRows rows of 64 blocks): the
  // segment of block v is seglist[(set bits of starts before v) - 1]
  const int nrows = (total + 63) >> 6;
  const bool mapped = nrows <= kSegMapRows;
  if (mapped) {
    for (int r = tid; r < nrows; r += kFusedThreads) s.starts[r] = 0ull;
    __syncthreads();
    if (nblk > 0) {
      const int v = s.seg[tid].v;
      atomicOr(reinterpret_cast<unsigned long long*>(&s.starts[v >> 6]), 1ull << (v & 63));
    }
    __syncthreads();
    // exclusive scan of the rows' bit counts (two rows per thread)
    const int r0 = 2 * tid;
    const int c0 = r0 < nrows ? __popcll(s.starts[r0]) : 0;
    const int c1 = r0 + 1 < nrows ? __popcll(s.starts[r0 + 1]) : 0;
    int x = c0 + c1;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(x, o);
      if (lane >= o) x += v;
    }
    if (lane == 63) s.wtot[0][wave] = static_cast<uint32_t>(x);
    __syncthreads();
    int wb = 0;
    for (int w = 0; w < wave; ++w) wb += static_cast<int>(s.wtot[0][w]);
    x += wb;
    if (r0 < nrows) s.pre[r0] = x - c0 - c1;
    if (r0 + 1 < nrows) s.pre[r0 + 1] = x - c1;
    __syncthreads();
  }
  constexpr int kW = kFusedThreads / 64;
  const int per = ((total + kW - 1) / kW + 63) & ~63;
  const int wstart = __builtin_amdgcn_readfirstlane(wave) * per, wend = min(total, wstart + per);
  const u32x4_t* ib = reinterpret_cast<const u32x4_t*>(p.indices);
  LSH_STAMP(p, 4);
  for (int w0 = wstart; w0 < wend; w0 += 64 * kCountInflight) {
    const int v0 = w0 + lane;
    // rows of 64 blocks this wave still has (wave-uniform).  The segment
    // lookups and the loads run for every row, straight-line, so that they
    // issue back to back (a step behind a branch waits for the loads before
    // it); only the counting skips the rows past nk
    const int nk = min(kCountInflight, (wend - w0 + 63) >> 6);
    u32x4_t blk[kCountInflight];
    int lo[kCountInflight], hi[kCountInflight];
    // the segment of each block (past the wave's range: of its last block):
    // from the segment map, or else by binary searches over the scan
    int sg[kCountInflight];
    if (mapped) {
#pragma unroll
      for (int k = 0; k < kCountInflight; ++k) {
        const int v = min(v0 + 64 * k, wend - 1);
        const uint64_t below = s.starts[v >> 6] & ((2ull << (v & 63)) - 1ull);
        sg[k] = s.seglist[s.pre[v >> 6] + __popcll(below) - 1];
      }
    } else {
#pragma unroll
      for (int k = 0; k < kCountInflight; ++k) sg[k] = 0;
#pragma unroll
      for (int step = 128; step > 0; step >>= 1) {
        int sv[kCountInflight];
#pragma unroll
        for (int k = 0; k < kCountInflight; ++k)
          sv[k] = s.seg[min(sg[k] + step, 256)].v;
#pragma unroll
        for (int k = 0; k < kCountInflight; ++k) {
          const int c = sg[k] + step;
          sg[k] = (c < p.L && sv[k] <= min(v0 + 64 * k, wend - 1)) ? c : sg[k];
        }
      }
    }
    if (w0 == wstart) LSH_STAMP(p, 5);
    // blocks past the wave's range load its last block again and take no entry
#pragma unroll
    for (int k = 0; k < kCountInflight; ++k) {
      const int v = v0 + 64 * k;
      const bool in = v < wend;
      const SegInfo si = s.seg[sg[k]];
      const int i = min(v, wend - 1) - si.v;
      blk[k] = ib[si.fb + i];
      lo[k] = in ? si.lo - 8 * i : 8;
      hi[k] = in ? si.hi - 8 * i : 0;
    }
#ifdef LSH_TRACE
    if (w0 == wstart) {   // trace builds: the first row's blocks have arrived
      uint32_t z = 0;
#pragma unroll
      for (int k = 0; k < kCountInflight; ++k)
        if (k < nk) z ^= blk[k][0];
      if (z == 0x9e3779b9u) s.spare[lane] = z;
      LSH_STAMP(p, 6);
    }
#endif
    // one LDS add per entry, without branches.  A key is masked into the
    // chunk's range (the counter array holds one byte per position of a full
    // chunk), so no access can leave the array whatever the table holds; an
    // entry outside its segment adds 0.  Keys past the chunk's length (in a
    // table of another layout) count positions the selection never reads.
    const uint32_t kmask = (1u << sl) - 1u;
#pragma unroll
    for (int k = 0; k < kCountInflight; ++k) {
      if (k < nk) {
        const uint32_t inseg = (0xffu << max(lo[k], 0)) & (0xffu >> (8 - min(max(hi[k], 0), 8)));
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          LSH_PCHECK(p, !((inseg >> e) & 1u) || ((blk[k][e >> 1] >> (16 * (e & 1))) & 0xffffu) <
                            static_cast<uint32_t>(clen), kChkEntry);
          const uint32_t key = (blk[k][e >> 1] >> (16 * (e & 1))) & kmask;
          const uint32_t inc = ((inseg >> e) & 1u) << ((key & 3u) * 8u);
          __hip_atomic_fetch_add(&cnt[key >> 2], inc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
      }
    }
  }
  LSH_STAMP(p, 7);
  __syncthreads();
  LSH_STAMP(p, 2);

  const int Nw = (p.N + 31) >> 5;
  const int nwords = (cfull + 31) >> 5;
  int mysel = 0;
  for (int w = tid; w < nwords; w += kFusedThreads) {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int wi = w * 8 + j;
      m |= counts_at_least(wi < cwords ? cnt[wi] : 0u, p.T) << (4 * j);
    }
    m &= selectable_bits(cbeg + 32 * w, cbeg + clen, exact_head, Nb - exact_tail);
    st_agent(p.bitmask + static_cast<size_t>(bh) * Nw + (cbeg >> 5) + w, m);
    mysel += __builtin_popcount(m);
  }
  if (p.counts) {
    const uint8_t* c8 = reinterpret_cast<const uint8_t*>(cnt);
    uint8_t* dst = p.counts + static_cast<size_t>(bh) * p.N + cbeg;
    for (int i = tid; i < cfull; i += kFusedThreads) dst[i] = c8[i];
  }
  mysel = wave_sum_int(mysel);
  if (lane == 0) s.wtot[0][wave] = mysel;
  __syncthreads();
  if (tid == 0) {
    int t = 0;
    for (int w = 0; w < kW; ++w) t += s.wtot[0][w];
    st_agent(p.chunk_nsel + static_cast<size_t>(bh) * p.nJ + J, t);
  }
  LSH_STAMP(p, 3);
  signal(p.ready + u * p.nJ + J);
}

// Several query heads of one unit per workgroup (count_heads > 1): segment
// hh * L + l, of up to kCountSegs, is head hh's bucket in table l; the heads
// keep their own byte counters and bitmask words.
__device__ inline void count_role_heads(const FusedParams& p, int J, int bh0, unsigned char* smem) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hc = p.count_heads;
  const int S = hc * p.L;                                                // segments
  const int b = bh0 / p.Hq, h0 = bh0 % p.Hq;
  const int u = b * p.Hkv + h0 / p.G;
  const int nb = 1 << p.K;
  const int sl = p.stride_log2;
  const int cbeg = J << sl;
  const int cwp = 1 << (sl - 2);                                         // counter words per head
  uint32_t* cnt = reinterpret_cast<uint32_t*>(smem);                     // [hc][cwp]: one byte per key of the chunk
  CountLds& s = *reinterpret_cast<CountLds*>(smem + (static_cast<size_t>(hc) << sl));
  const int Nb = seq_len_of(p.seq_lens, b, p.N);
  const int cfull = min(1 << sl, p.N - cbeg);
  const int clen = max(0, min(1 << sl, Nb - cbeg));
  const int cwords = (cfull + 3) >> 2;
  int exact_head, exact_tail;
  exact_range(p.n_sink, p.n_window, Nb, exact_head, exact_tail);

  LSH_STAMP(p, 0);
  for (int i = tid; i < hc * cwp; i += kFusedThreads) cnt[i] = 0;

  // the segment of head hh's bucket in table l inside this chunk, in blocks:
  // thread t takes segment t of each row of 256 (with one head, thread l
  // takes table l); the query codes, then the bucket bounds, each set of
  // loads in flight together
  // (every load below is issued, from a clamped address where the segment
  // does not exist, so that each set is in flight at once: a load behind a
  // branch waits for the ones before it)
  int qraw[kSegsPerThread];
#pragma unroll
  for (int k = 0; k < kSegsPerThread; ++k) {
    const int sg = min(tid + k * kFusedThreads, S - 1);
    qraw[k] = p.qcodes[static_cast<size_t>(bh0 + sg / p.L) * p.L + sg % p.L];
  }
  int ob0[kSegsPerThread], ob1[kSegsPerThread];   // the bucket's first entry, and the next bucket's
#pragma unroll
  for (int k = 0; k < kSegsPerThread; ++k) {
    const int sg = min(tid + k * kFusedThreads, S - 1);
    // (the query hash writes codes below 2^K; the mask keeps any other value
    // inside the chunk's bucket starts, and the checked build reports it)
    const int qc = qraw[k] & (nb - 1);
    const size_t row = static_cast<size_t>(u) * p.L + sg % p.L;
    const uint16_t* op = p.offsets + (row * p.nJP + J) * nb + qc;
    ob0[k] = op[0];
    ob1[k] = op[qc + 1 < nb ? 1 : 0];
  }
  uint32_t own[kSegsPerThread];
#pragma unroll
  for (int k = 0; k < kSegsPerThread; ++k) {
    const int sg = tid + k * kFusedThreads;
    int nblk = 0;
    if (sg < S && clen > 0) {
      const int l = sg % p.L;
      LSH_PCHECK(p, qraw[k] < nb, kChkQueryCode);
      const int qc = qraw[k] & (nb - 1);
      const size_t row = static_cast<size_t>(u) * p.L + l;
      LSH_PCHECK(p, ob0[k] <= (qc + 1 < nb ? ob1[k] : clen) && (qc + 1 < nb ? ob1[k] : ob0[k]) <= clen,
                 kChkSegment);
      // clamped into the chunk: tables of another stride cannot send the walk out of it
      const int s0 = min(ob0[k], clen);
      const int e0 = qc + 1 < nb ? min(ob1[k], clen) : clen;
      const size_t first = row * p.P + cbeg + s0;      // element index of the segment's first entry
      const int lo = static_cast<int>(first & 7);
      const int len = max(e0 - s0, 0);
      nblk = len > 0 ? (lo + len + 7) >> 3 : 0;
      s.seg[sg].fb = static_cast<long long>(first >> 3) | (static_cast<long long>(sg / p.L) << 56);
      s.seg[sg].lo = static_cast<short>(lo);
      s.seg[sg].hi = static_cast<short>(lo + len);
    }
    // scan word: the block count, and 1 in the rank field when non-empty
    own[k] = static_cast<uint32_t>(nblk) + (nblk > 0 ? (1u << kCountRankShift) : 0u);
  }
  // one scan per row of 256 segments gives the block offsets and the rank of
  // each non-empty segment among them; the rows follow each other
  const int rows = (S + kFusedThreads - 1) / kFusedThreads;   // rows holding segments (one with one head)
  uint32_t incl[kSegsPerThread];
#pragma unroll
  for (int k = 0; k < kSegsPerThread; ++k) incl[k] = own[k];
#pragma unroll
  for (int k = 0; k < kSegsPerThread; ++k) {
    if (k < rows) {
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t v = __shfl_up(incl[k], o);
        if (lane >= o) incl[k] += v;
      }
      if (lane == 63) s.wtot[k][wave] = incl[k];
    }
  }
  __syncthreads();
  {
    constexpr uint32_t kBlocks = (1u << kCountRankShift) - 1u;
    uint32_t row_base = 0;                           // segments of the rows before
#pragma unroll
    for (int k = 0; k < kSegsPerThread; ++k) {
      if (k >= rows) break;
      uint32_t before = 0, row_tot = 0;
      for (int w = 0; w < kFusedThreads / 64; ++w) {
        if (w < wave) before += s.wtot[k][w];
        row_tot += s.wtot[k][w];
      }
      const int sg = tid + k * kFusedThreads;
      const uint32_t x = row_base + before + incl[k] - own[k];   // exclusive, at segment sg
      if (sg < S) s.seg[sg].v = static_cast<int>(x & kBlocks);
      if (sg < S && (own[k] & kBlocks) > 0) s.seglist[x >> kCountRankShift] = static_cast<uint16_t>(sg);
      row_base += row_tot;
    }
    if (tid == 0) s.seg[S].v = static_cast<int>(row_base & kBlocks);
  }
  __syncthreads();
  LSH_STAMP(p, 1);

  // the walk's bounds are wave-uniform (scalar), so the steps below need no
  // per-lane branches
  const int total = __builtin_amdgcn_readfirstlane(s.seg[S].v);
  // segment map (walks of at most kSegMapRows rows of 64 blocks): the
  // segment of block v is seglist[(set bits of starts before v) - 1]
  const int nrows = (total + 63) >> 6;
  const bool mapped = nrows <= kSegMapRows;
  if (mapped) {
    for (int r = tid; r < nrows; r += kFusedThreads) s.starts[r] = 0ull;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kSegsPerThread; ++k) {
      const int sg = tid + k * kFusedThreads;
      if (sg < S && (own[k] & ((1u << kCountRankShift) - 1u)) > 0) {
        const int v = s.seg[sg].v;
        atomicOr(reinterpret_cast<unsigned long long*>(&s.starts[v >> 6]), 1ull << (v & 63));
      }
    }
    __syncthreads();
    // exclusive scan of the rows' bit counts (two rows per thread)
    const int r0 = 2 * tid;
    const int c0 = r0 < nrows ? __popcll(s.starts[r0]) : 0;
    const int c1 = r0 + 1 < nrows ? __popcll(s.starts[r0 + 1]) : 0;
    int x = c0 + c1;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(x, o);
      if (lane >= o) x += v;
    }
    if (lane == 63) s.wtot[0][wave] = static_cast<uint32_t>(x);
    __syncthreads();
    int wb = 0;
    for (int w = 0; w < wave; ++w) wb += static_cast<int>(s.wtot[0][w]);
    x += wb;
    if (r0 < nrows) s.pre[r0] = x - c0 - c1;
    if (r0 + 1 < nrows) s.pre[r0 + 1] = x - c1;
    __syncthreads();
  }
  constexpr int kW = kFusedThreads / 64;
  const int per = ((total + kW - 1) / kW + 63) & ~63;
  const int wstart = __builtin_amdgcn_readfirstlane(wave) * per, wend = min(total, wstart + per);
  const u32x4_t* ib = reinterpret_cast<const u32x4_t*>(p.indices);
  LSH_STAMP(p, 4);
  for (int w0 = wstart; w0 < wend; w0 += 64 * kCountInflight) {
    const int v0 = w0 + lane;
    // rows of 64 blocks this wave still has (wave-uniform).  The segment
    // lookups and the loads run for every row, straight-line, so that they
    // issue back to back (a step behind a branch waits for the loads before
    // it); only the counting skips the rows past nk
    const int nk = min(kCountInflight, (wend - w0 + 63) >> 6);
    u32x4_t blk[kCountInflight];
    int lo[kCountInflight], hi[kCountInflight], cb[kCountInflight];
    // the segment of each block (past the wave's range: of its last block):
    // from the segment map, or else by binary searches over the scan
    int sg[kCountInflight];
    if (mapped) {
#pragma unroll
      for (int k = 0; k < kCountInflight; ++k) {
        const int v = min(v0 + 64 * k, wend - 1);
        const uint64_t below = s.starts[v >> 6] & ((2ull << (v & 63)) - 1ull);
        sg[k] = s.seglist[s.pre[v >> 6] + __popcll(below) - 1];
      }
    } else {
#pragma unroll
      for (int k = 0; k < kCountInflight; ++k) sg[k] = 0;
#pragma unroll
      for (int step = kCountSegs / 2; step > 0; step >>= 1) {
        int sv[kCountInflight];
#pragma unroll
        for (int k = 0; k < kCountInflight; ++k)
          sv[k] = s.seg[min(sg[k] + step, S)].v;
#pragma unroll
        for (int k = 0; k < kCountInflight; ++k) {
          const int c = sg[k] + step;
          sg[k] = (c < S && sv[k] <= min(v0 + 64 * k, wend - 1)) ? c : sg[k];
        }
      }
    }
    if (w0 == wstart) LSH_STAMP(p, 5);
    // blocks past the wave's range load its last block again and take no entry
#pragma unroll
    for (int k = 0; k < kCountInflight; ++k) {
      const int v = v0 + 64 * k;
      const bool in = v < wend;
      const SegInfo si = s.seg[sg[k]];
      const int i = min(v, wend - 1) - si.v;
      blk[k] = ib[(si.fb & kSegBlockMask) + i];
      lo[k] = in ? si.lo - 8 * i : 8;
      hi[k] = in ? si.hi - 8 * i : 0;
      cb[k] = static_cast<int>(si.fb >> 56) * cwp;   // the segment's head's counters
    }
#ifdef LSH_TRACE
    if (w0 == wstart) {   // trace builds: the first row's blocks have arrived
      uint32_t z = 0;
#pragma unroll
      for (int k = 0; k < kCountInflight; ++k)
        if (k < nk) z ^= blk[k][0];
      if (z == 0x9e3779b9u) s.spare[lane] = z;
      LSH_STAMP(p, 6);
    }
#endif
    // one LDS add per entry, without branches.  A key is masked into the
    // chunk's range (the counter array holds one byte per position of a full
    // chunk), so no access can leave the array whatever the table holds; an
    // entry outside its segment adds 0.  Keys past the chunk's length (in a
    // table of another layout) count positions the selection never reads.
    const uint32_t kmask = (1u << sl) - 1u;
#pragma unroll
    for (int k = 0; k < kCountInflight; ++k) {
      if (k < nk) {
        const uint32_t inseg = (0xffu << max(lo[k], 0)) & (0xffu >> (8 - min(max(hi[k], 0), 8)));
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          LSH_PCHECK(p, !((inseg >> e) & 1u) || ((blk[k][e >> 1] >> (16 * (e & 1))) & 0xffffu) <
                            static_cast<uint32_t>(clen), kChkEntry);
          const uint32_t key = (blk[k][e >> 1] >> (16 * (e & 1))) & kmask;
          const uint32_t inc = ((inseg >> e) & 1u) << ((key & 3u) * 8u);
          __hip_atomic_fetch_add(&cnt[cb[k] + (key >> 2)], inc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
      }
    }
  }
  LSH_STAMP(p, 7);
  __syncthreads();
  LSH_STAMP(p, 2);

  const int Nw = (p.N + 31) >> 5;
  const int nwords = (cfull + 31) >> 5;
  for (int hh = 0; hh < hc; ++hh) {
    const uint32_t* ch = cnt + hh * cwp;
    const int bh = bh0 + hh;
    int mysel = 0;
    for (int w = tid; w < nwords; w += kFusedThreads) {
      uint32_t m = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int wi = w * 8 + j;
        m |= counts_at_least(wi < cwords ? ch[wi] : 0u, p.T) << (4 * j);
      }
      m &= selectable_bits(cbeg + 32 * w, cbeg + clen, exact_head, Nb - exact_tail);
      st_agent(p.bitmask + static_cast<size_t>(bh) * Nw + (cbeg >> 5) + w, m);
      mysel += __builtin_popcount(m);
    }
    if (p.counts) {
      const uint8_t* c8 = reinterpret_cast<const uint8_t*>(ch);
      uint8_t* dst = p.counts + static_cast<size_t>(bh) * p.N + cbeg;
      for (int i = tid; i < cfull; i += kFusedThreads) dst[i] = c8[i];
    }
    mysel = wave_sum_int(mysel);
    if (lane == 0) s.hsel[hh][wave] = mysel;
  }
  __syncthreads();
  if (tid < hc) {
    int t = 0;
    for (int w = 0; w < kW; ++w) t += s.hsel[tid][w];
    st_agent(p.chunk_nsel + static_cast<size_t>(bh0 + tid) * p.nJ + J, t);
  }
  LSH_STAMP(p, 3);
  signal(p.ready + u * p.nJ + J, hc);
}

// --------------------------------------------------------------------------
// Merge
//
// Every attend workgroup of unit u writes its partial slot and then
// arrives at the unit's counter.  The last F = min(G, npart) arrivals are
// the finishers: finisher f waits until all npart slots have arrived and
// folds the slots of heads f, f + F, ... into out / lse / nsel.  Attend
// workgroups are dispatched unit by unit (see the grids), so a finisher waits
// only for workgroups that are running or will get a slot: every workgroup of
// a lower unit has been dispatched, and none of a higher unit holds a slot
// while one of its unit's is still waiting for dispatch.
// --------------------------------------------------------------------------
constexpr int kFoldRows = 16;        // float4 slot rows a thread keeps in flight in a fold
constexpr int kMergeMaxPairs = 2048; // (head, slot) pairs of a fold, in LDS

struct MergeLds {
  float m[kMergeMaxPairs];           // max, then the slot's weight exp(m - M)
  float l[kMergeMaxPairs];
  float M[16], Lm[16];
  float4 red[kFusedThreads];         // column sums of the thread groups sharing a column
  int nsel[16];
  int flag;
};

// Fold all npart slots of heads f, f + F, ... of unit u (bh0 = its first
// head) into the outputs.  The nh * 32 float4 columns (head, 4 dims) are
// spread over the threads, R threads per column (R = 256 / columns when that
// is at least 2), each R-th slot per thread.  The first batch of slot values
// (kFoldRows rows per thread: all 128 slots of a head at R = 8) goes out
// together with the heads' max / sum and chunk-count loads, so a fold of up to
// R * kFoldRows slots costs one round trip to memory.
__device__ inline void fold_heads(const FusedParams& p, int bh0, int f, int F, unsigned char* smem) {
  MergeLds& s = *reinterpret_cast<MergeLds*>(smem);
  const int tid = threadIdx.x;
  const int np = p.npart;
  constexpr int kQ = kHeadDim / 4;                              // float4 columns of a head
  constexpr int kRowQ = kPartialStride / 4;                     // float4 pitch of the slots
  const int nh = (p.G - f + F - 1) / F;                         // heads of this finisher
  const int C = nh * kQ;
  const int R = C >= kFusedThreads ? 1 : kFusedThreads / C;
  const int cpt = (C + kFusedThreads - 1) / kFusedThreads;     // column blocks (R == 1 only)
  if (tid < nh) s.nsel[tid] = 0;
  // every slot has arrived (the finisher waited for the unit's counter), and
  // each was written through to memory before its arrival; one acquire fence
  // drops any stale copy from this XCD's caches, so the fold reads the slots
  // with plain loads (a coherent load per value would be far slower in bulk)
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  __syncthreads();
  LSH_STAMP(p, 8);
  // the max / sum of every (head, slot) pair (nh * np <= kMergeMaxPairs = 8
  // per thread) and the first batch of the heads' chunk selection counts go
  // out first, loaded by the threads that hold them; then column block 0's
  // first batch of slot values.  The max / sum and counts are then waited for
  // alone (loads complete in order), and the slot values stay in flight
  // through the barrier and the weights below, until the sums need them
  static_assert(kMergeMaxPairs <= 8 * kFusedThreads, "one batch of max / sum loads");
  float2 ml[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int i = tid + q * kFusedThreads;
    const float* ps = p.partials + (static_cast<size_t>(bh0 + f + F * (i / np)) * np + i % np) * kPartialStride;
    ml[q] = i < nh * np ? *reinterpret_cast<const float2*>(ps + kHeadDim) : make_float2(0.f, 0.f);
  }
  int cv[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int i = tid + q * kFusedThreads;
    cv[q] = i < nh * p.nJ ? p.chunk_nsel[static_cast<size_t>(bh0 + f + F * (i / p.nJ)) * p.nJ + i % p.nJ] : 0;
  }
  const int c0 = R > 1 ? tid % C : tid;
  const int r0 = R > 1 ? tid / C : 0;
  const bool live0 = c0 < C && r0 < R;
  const int hi0 = live0 ? c0 / kQ : 0;
  const float4* base0 =
      reinterpret_cast<const float4*>(p.partials + static_cast<size_t>(bh0 + f + F * hi0) * np * kPartialStride) +
      c0 % kQ;
  float4 x[kFoldRows];
#pragma unroll
  for (int i = 0; i < kFoldRows; ++i) x[i] = base0[static_cast<size_t>(min(r0 + i * R, np - 1)) * kRowQ];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int i = tid + q * kFusedThreads;
    if (i < nh * np) {
      s.m[i] = ml[q].x;
      s.l[i] = ml[q].y;
    }
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int i = tid + q * kFusedThreads;
    if (i < nh * p.nJ) atomicAdd(&s.nsel[i / p.nJ], cv[q]);
  }
  // the rest of the counts (more than 2048 (head, chunk) pairs)
  for (int i0 = 8 * kFusedThreads; i0 < nh * p.nJ; i0 += 8 * kFusedThreads) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int i = min(i0 + tid + q * kFusedThreads, nh * p.nJ - 1);
      cv[q] = p.chunk_nsel[static_cast<size_t>(bh0 + f + F * (i / p.nJ)) * p.nJ + i % p.nJ];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int i = i0 + tid + q * kFusedThreads;
      if (i < nh * p.nJ) atomicAdd(&s.nsel[i / p.nJ], cv[q]);
    }
  }
  __syncthreads();
  LSH_STAMP(p, 9);
  // per head: the max over its slots, then each slot's weight exp(m - M)
  // and the weighted sum of the slot sums; wave w takes heads w, w + 4, ...,
  // its lanes the slots (reductions across the wave)
  {
    const int lane = tid & 63, wave = tid >> 6;
    for (int hi = wave; hi < nh; hi += kFusedThreads / 64) {
      float M = -INFINITY;
      for (int k = lane; k < np; k += 64) M = fmaxf(M, s.m[hi * np + k]);
      M = wave_max(M);
      float Lm = 0.f;
      for (int k = lane; k < np; k += 64) {
        const float mk = s.m[hi * np + k];
        const float w = (M == -INFINITY || mk == -INFINITY) ? 0.f : __expf(mk - M);
        Lm = fmaf(s.l[hi * np + k], w, Lm);
        s.m[hi * np + k] = w;
      }
      Lm = wave_sum(Lm);
      if (lane == 0) {
        s.M[hi] = M;
        s.Lm[hi] = Lm;
      }
    }
  }
  __syncthreads();
  LSH_STAMP(p, 10);
  for (int cb = 0; cb < cpt; ++cb) {
    const int c = cb * kFusedThreads + (R > 1 ? tid % C : tid);
    const int r = R > 1 ? tid / C : 0;
    const bool live = c < C && r < R;
    const int hi = live ? c / kQ : 0, cq = c % kQ;
    const float4* base =
        reinterpret_cast<const float4*>(p.partials + static_cast<size_t>(bh0 + f + F * hi) * np * kPartialStride) +
        cq;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k0 = r; k0 < np; k0 += R * kFoldRows) {
      if (cb != 0 || k0 != r) {   // the first batch of block 0 is already in x
#pragma unroll
        for (int i = 0; i < kFoldRows; ++i) {
          const int k = min(k0 + i * R, np - 1);   // clamped: every load issues, the extra ones add nothing
          x[i] = base[static_cast<size_t>(k) * kRowQ];
        }
      }
      // the weights: clamped reads; past the last slot (and in dead columns)
      // the weight is 0
#pragma unroll
      for (int i = 0; i < kFoldRows; ++i) {
        const int k = k0 + i * R;
        const float w = s.m[hi * np + min(k, np - 1)];
        const float wk = (live && k < np) ? w : 0.f;
        acc.x = fmaf(x[i].x, wk, acc.x);
        acc.y = fmaf(x[i].y, wk, acc.y);
        acc.z = fmaf(x[i].z, wk, acc.z);
        acc.w = fmaf(x[i].w, wk, acc.w);
      }
    }
    // the R partial sums of each column
    s.red[tid] = acc;
    __syncthreads();
    if (live && r == 0) {
      for (int q = 1; q < R; ++q) {
        const float4 o = s.red[tid + q * C];
        acc.x += o.x;
        acc.y += o.y;
        acc.z += o.z;
        acc.w += o.w;
      }
      const int bh = bh0 + f + F * hi;
      const float M = s.M[hi], Lm = s.Lm[hi];
      const bool empty = (M == -INFINITY);
      const float4 o = empty ? make_float4(0.f, 0.f, 0.f, 0.f)
                             : make_float4(acc.x / Lm, acc.y / Lm, acc.z / Lm, acc.w / Lm);
      reinterpret_cast<float4*>(p.out + static_cast<size_t>(bh) * kHeadDim)[cq] = o;
      if (cq == 0) {
        if (p.lse) p.lse[bh] = empty ? -INFINITY : M + logf(Lm);
        if (p.nsel) p.nsel[bh] = s.nsel[hi];
      }
    }
    __syncthreads();
  }
}

// After writing partial slot `slot` of unit u: arrive; the last F arrivals
// fold the unit's heads.
__device__ inline void finish_slot(const FusedParams& p, int u, int slot, unsigned char* smem) {
  MergeLds& s = *reinterpret_cast<MergeLds*>(smem);
  const int b = u / p.Hkv, g = u % p.Hkv;
  const int bh0 = b * p.Hq + g * p.G;
  const int F = min(p.G, p.npart);
  const int c = arrive(p.arrive_unit + u, &s.flag);
  if (c < p.npart - F) return;
  LSH_STAMP(p, 5);
  const int f = c - (p.npart - F);
  // every slot of the unit has arrived, and the selection counts of every
  // chunk of it are complete (chunks past a short sequence's end are waited
  // for by no attend workgroup): thread 0 polls the first, the others the
  // chunk counters, side by side
  if (threadIdx.x == 0) s.flag = 1;
  __syncthreads();
  int ok = 1;
  for (int j = static_cast<int>(threadIdx.x) - 1; j < p.nJ; j += kFusedThreads) {
    const int32_t* ctr = j < 0 ? p.arrive_unit + u : p.ready + u * p.nJ + j;
    const int target = j < 0 ? p.npart : p.G;
    int it = 0;
    while (ld_agent(ctr) < target) {
      __builtin_amdgcn_s_sleep(2);
      if (++it >= kSpinLimit) {
        ok = 0;
        break;
      }
    }
  }
  if (!ok) s.flag = 0;
  __syncthreads();
  const bool all = s.flag != 0;
  __syncthreads();
  LSH_STAMP(p, 6);
  fold_heads(p, bh0, f, F, smem);
  if (!all && threadIdx.x == 0) p.out[static_cast<size_t>(bh0 + f) * kHeadDim] = __builtin_nanf("");
  LSH_STAMP(p, 7);
}

constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }
// LDS the count and merge roles use (the attention roles add theirs)
constexpr size_t kRolesLdsBytes = cmax(static_cast<size_t>(kCountCounterBytes) + sizeof(CountLds), sizeof(MergeLds));

}  // namespace lsh
