// Decode-side kernels for gfx950.
//
// One decode step of MagicPIG's LSH sampling ("MagicPIG: LSH Sampling for
// Efficient LLM Generation", GrooveSquid summary; MagicPIG project summary on
// sourcepulse, "How It Works") runs as four launches on one stream:
//   qhash          SimHash codes of every query head (same W and sign rule as
//                  the keys); extra workgroups fill the ln-u correction table
//   count_select   per (query head, key chunk): probe the head's L buckets,
//                  restricted to the chunk through the chunk's bucket offsets,
//                  count collisions in LDS byte counters, and emit the
//                  selection bitmask (count >= T)
//   attend         per (sequence, kv head, context split): union of the
//                  group's selections, ballot compaction, gathered K/V rows,
//                  q.k on MFMA, 1/u weights, online softmax in fp32 and P.V
//                  (MFMA with P in bf16 high + low parts for bf16 K/V, FMAs
//                  for fp32), partial state (m, l, acc) per query head; with
//                  an exact set, extra workgroups attend it with unit weights
//   merge          log-sum-exp merge of the partials (the stable merge
//                  MAC-Attention also uses, "MAC-Attention" README,
//                  "How It Works")
#include <math.h>

#include "lsh_device.h"
#include "lsh_kernels.h"

namespace lsh {

constexpr float kPi = 3.14159265358979323846f;
constexpr float kLnUFloor = -69.07755278982137f;   // ln(1e-30)

// ---------------------------------------------------------------------------
// ln u correction table.
//
// u(theta) = P[Binomial(L, P) >= T] with P = (1 - theta/pi)^K.  Writing
// ln u = T ln P + g(P),  g(P) = ln sum_{i>=T} C(L,i) P^(i-T) (1-P)^(L-i),
// g is smooth on [0, 1] (g(0) = ln C(L,T), g(1) = 0), so it is sampled in
// fp64 at theta_t = t pi / (2 kLnuTable) and interpolated by one quadratic per
// interval of width pi / kLnuTable (through its start, middle and end); T ln P
// = T K ln p is evaluated from p itself.
// ---------------------------------------------------------------------------
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

// g(theta) for one table entry, computed by one wave: lane handles the terms
// i = T + lane + 64 k of the sum, whose log binomial coefficients are in
// lc[i] = ln C(L, i); the terms are combined by a log-sum-exp over the wave.
__device__ double lnu_correction_wave(double theta, int K, int L, int T, const double* lc, int lane) {
  const double p = 1.0 - theta / 3.14159265358979323846;
  const double P = (K == 0) ? 1.0 : pow(p, static_cast<double>(K));
  const double lP = log(P), lQ = log1p(-P);
  double t[4];
  double m = -INFINITY;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = T + lane + 64 * k;
    double x = -INFINITY;
    if (i <= L) {
      x = lc[i];
      if (i > T) x += (i - T) * lP;   // 0 * ln 0 is 1 here: skip the zero power
      if (L > i) x += (L - i) * lQ;
    }
    t[k] = x;
    m = fmax(m, x);
  }
  m = wave_max_f64(m);
  double sum = 0.0;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (t[k] != -INFINITY) sum += exp(t[k] - m);
  sum = wave_sum_f64(sum);
  return m + log(sum);
}

// ln u at cosine cosv (fp32 K/V path).  r = acos(|c|); theta = r for c >= 0
// and pi - r for c < 0, where p = 1 - theta / pi = r / pi is taken from r
// directly so that it keeps r's relative accuracy as theta -> pi.
__device__ __forceinline__ float log_inclusion(float cosv, const float4* tab, float TK) {
  const float c = fminf(1.f, fmaxf(-1.f, cosv));
  const float r = acosf(fabsf(c));
  const bool neg = c < 0.f;
  const float th = neg ? kPi - r : r;
  const float x = th * (static_cast<float>(kLnuTable) / kPi);
  const int j = min(static_cast<int>(x), kLnuTable - 1);
  const float fr = x - static_cast<float>(j);
  const float4 e = tab[j];
  const float g = fmaf(fr, fmaf(fr, e.z, e.y), e.x);
  const float rp = r * (1.0f / kPi);
  const float lnp = neg ? logf(rp) : log1pf(-rp);
  return fmaxf(fmaf(TK, lnp, g), kLnUFloor);
}

// ---------------------------------------------------------------------------
// qhash: SimHash codes of 16 query heads x a block of whole tables (at most
// 64 projection columns) per workgroup.  Lane c of every wave owns column c of
// the block and wave w sums dims [32 w, 32 w + 32), so each lane issues its 32
// W loads at once; the four partial sums meet in LDS.  Workgroups with
// blockIdx.y >= head_blocks fill the ln-u table instead, one entry per wave.
// ---------------------------------------------------------------------------
constexpr int kQHeads = 16;

template <typename T>
__global__ __launch_bounds__(256) void qhash_kernel(const typename T::storage* __restrict__ q,
                                                    const typename T::storage* __restrict__ W,
                                                    uint16_t* __restrict__ qcodes, double* __restrict__ lnu_samples,
                                                    int BH, int K, int L, int Tth, int head_blocks,
                                                    int G, int Hkv, size_t w_head_stride) {
  __shared__ __attribute__((aligned(16))) float qs[kQHeads][kHeadDim];
  __shared__ float part[4][kQHeads][64];
  __shared__ uint8_t sgn[kQHeads][64];
  __shared__ double lc[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (static_cast<int>(blockIdx.y) >= head_blocks) {
    if (K == 0) return;
    if (tid <= L)
      lc[tid] = lgamma(static_cast<double>(L) + 1.0) - lgamma(static_cast<double>(tid) + 1.0) -
                lgamma(static_cast<double>(L - tid) + 1.0);
    __syncthreads();
    const int j = ((blockIdx.y - head_blocks) * gridDim.x + blockIdx.x) * 4 + wave;
    const double g = lnu_correction_wave(j * (3.14159265358979323846 / (2 * kLnuTable)), K, L, Tth, lc, lane);
    if (j < kLnuSamples && lane == 0) lnu_samples[j] = g;
    return;
  }
  // a workgroup hashes hpb heads: 16 with one shared W, or the G heads of
  // one (sequence, kv head) with a W per kv head
  const int hpb = w_head_stride ? G : kQHeads;
  const int h0 = blockIdx.y * hpb;
  if (K == 0) {
    for (int e = blockIdx.x * 256 + tid; e < hpb * L; e += gridDim.x * 256) {
      const int h = h0 + e / L;
      if (h < BH) qcodes[static_cast<size_t>(h) * L + e % L] = 0;
    }
    return;
  }
  W += static_cast<size_t>((h0 / G) % Hkv) * w_head_stride;
  const int tpw = 64 / K;               // whole tables per workgroup
  const int l0 = blockIdx.x * tpw;
  for (int e = tid; e < kQHeads * kHeadDim; e += 256) {
    const int h = h0 + e / kHeadDim;
    float v = 0.f;
    if (e / kHeadDim < hpb && h < BH) {
      if constexpr (sizeof(typename T::storage) == 2)
        v = bf16_to_f32(q[static_cast<size_t>(h) * kHeadDim + e % kHeadDim]);
      else
        v = q[static_cast<size_t>(h) * kHeadDim + e % kHeadDim];
    }
    qs[e / kHeadDim][e % kHeadDim] = v;
  }
  __syncthreads();
  const int LK = L * K;
  const int col = l0 * K + lane;
  const bool colv = lane < tpw * K && col < LK;
  float w[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const size_t at = static_cast<size_t>(32 * wave + i) * LK + (colv ? col : 0);
    if constexpr (sizeof(typename T::storage) == 2)
      w[i] = bf16_to_f32(W[at]);
    else
      w[i] = W[at];
  }
#pragma unroll
  for (int hh = 0; hh < kQHeads; ++hh) {
    const floatx4_t* qv = reinterpret_cast<const floatx4_t*>(&qs[hh][32 * wave]);
    float acc = 0.f;
#pragma unroll
    for (int i4 = 0; i4 < 8; ++i4) {
      const floatx4_t x = qv[i4];
      acc = fmaf(x[0], w[4 * i4 + 0], acc);
      acc = fmaf(x[1], w[4 * i4 + 1], acc);
      acc = fmaf(x[2], w[4 * i4 + 2], acc);
      acc = fmaf(x[3], w[4 * i4 + 3], acc);
    }
    part[wave][hh][lane] = acc;
  }
  __syncthreads();
  for (int e = tid; e < kQHeads * 64; e += 256) {
    const int hh = e >> 6, c = e & 63;
    const float x = part[0][hh][c] + part[1][hh][c] + part[2][hh][c] + part[3][hh][c];
    sgn[hh][c] = x > 0.f ? 1 : 0;
  }
  __syncthreads();
  for (int e = tid; e < kQHeads * tpw; e += 256) {
    const int hh = e / tpw, t = e % tpw;
    const int l = l0 + t, h = h0 + hh;
    if (hh < hpb && h < BH && l < L) {
      uint32_t code = 0;
      for (int b = 0; b < K; ++b) code |= static_cast<uint32_t>(sgn[hh][t * K + b]) << b;
      qcodes[static_cast<size_t>(h) * L + l] = static_cast<uint16_t>(code);
    }
  }
}

// ---------------------------------------------------------------------------
// count_select: one workgroup of NT threads per (query head, key chunk).
// Every workgroup runs the same chain of dependent loads (query codes, bucket
// starts, bucket entries), so when there are many (head, chunk) pairs smaller
// workgroups let more of them be resident at once; with few pairs, large
// workgroups spread each walk over more lanes.
// ---------------------------------------------------------------------------
constexpr int kCountUnroll = 8;   // index loads each thread keeps in flight

template <int NT>
__global__ __launch_bounds__(NT) void count_select_kernel(
    const uint16_t* __restrict__ qcodes,   // [BH][L]
    const uint16_t* __restrict__ indices,  // [U][L][P] chunk-major, chunk-relative key indices
    const uint16_t* __restrict__ offsets,  // [U][L][nJP][2^K] bucket starts inside each chunk
    int Hq, int Hkv, int N, int P, int K, int L, int T, int stride_log2, int nJ, int nJP,
    uint32_t* __restrict__ bitmask,        // [BH][Nw]
    int32_t* __restrict__ chunk_nsel,      // [BH][nJ]
    uint8_t* __restrict__ counts,          // optional [BH][N]
    int n_sink, int n_window,              // the exact set, attended exactly, never sampled
    const int32_t* __restrict__ seq_lens) {  // optional [B] keys per sequence
  extern __shared__ __attribute__((aligned(16))) uint32_t cnt[];   // one byte per key of the chunk
  __shared__ int seg_start[256];
  __shared__ int seg_v[257];
  constexpr int kCountThreads = NT;
  static_assert(NT >= 256, "the first four waves hold one table per thread");
  __shared__ int wave_tot[kCountThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int J = blockIdx.x, bh = blockIdx.y;
  const int b = bh / Hq, h = bh % Hq, G = Hq / Hkv;
  const int u = b * Hkv + h / G;
  const int nb = 1 << K;
  const int cbeg = J << stride_log2;
  // cfull: the chunk's positions in the bitmask and counts; clen: the keys
  // of this sequence among them (none when the sequence ends before it)
  const int Nb = seq_len_of(seq_lens, b, N);
  const int cfull = min(1 << stride_log2, N - cbeg);
  const int clen = max(0, min(1 << stride_log2, Nb - cbeg));
  const int cwords = (cfull + 3) >> 2;
  int exact_head, exact_tail;
  exact_range(n_sink, n_window, Nb, exact_head, exact_tail);

  for (int i = tid; i < cwords; i += kCountThreads) cnt[i] = 0;

  // segment of bucket qcode_l restricted to this chunk, for every table l
  // (L <= 255, so the first four waves hold one table per thread)
  int len = 0;
  if (tid < L && clen > 0) {
    const int qc = qcodes[static_cast<size_t>(bh) * L + tid];
    const uint16_t* op = offsets + ((static_cast<size_t>(u) * L + tid) * nJP + J) * nb + qc;
    // clamped into the chunk: tables that do not match the stride cannot
    // send the walk outside the chunk's region
    const int s0 = min(static_cast<int>(op[0]), clen);
    const int e0 = qc + 1 < nb ? min(static_cast<int>(op[1]), clen) : clen;
    len = max(e0 - s0, 0);
    seg_start[tid] = cbeg + s0;
  }
  int incl = len;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  if (lane == 63 && wave < 4) wave_tot[wave] = incl;
  __syncthreads();
  if (tid < 256) {
    int wbase = 0;
    for (int w = 0; w < wave; ++w) wbase += wave_tot[w];
    seg_v[tid + 1] = wbase + incl;
    if (tid == 0) seg_v[0] = 0;
  }
  __syncthreads();

  // walk the concatenated segments: entry v of segment l is
  // indices[u][l][seg_start[l] + v - seg_v[l]], the key's offset in this chunk.
  // Every wave takes a contiguous range of entries, so its 64 lanes read 64
  // consecutive entries and cross at most one segment boundary per step.
  const int total = seg_v[L];
  constexpr int kWaves = kCountThreads / 64;
  const int per = ((total + kWaves - 1) / kWaves + 63) & ~63;
  const int wstart = wave * per, wend = min(total, wstart + per);
  const uint16_t* ib = indices + static_cast<size_t>(u) * L * P;
  int l = 0;                                      // last segment starting at or before wstart
  {
    int lo = 0, hi = L - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (seg_v[mid] <= wstart) lo = mid; else hi = mid - 1;
    }
    l = lo;
  }
  for (int v0 = wstart + lane; v0 < wend; v0 += 64 * kCountUnroll) {
    int loc[kCountUnroll];
#pragma unroll
    for (int k = 0; k < kCountUnroll; ++k) {
      const int v = v0 + 64 * k;
      loc[k] = -1;
      if (v < wend) {
        while (v >= seg_v[l + 1]) ++l;
        loc[k] = ib[static_cast<size_t>(l) * P + seg_start[l] + (v - seg_v[l])];
      }
    }
#pragma unroll
    for (int k = 0; k < kCountUnroll; ++k)
      if (loc[k] >= 0 && loc[k] < clen) atomicAdd(&cnt[loc[k] >> 2], 1u << ((loc[k] & 3) * 8));
  }
  __syncthreads();

  const int Nw = (N + 31) >> 5;
  const int nwords = (cfull + 31) >> 5;
  int mysel = 0;
  for (int w = tid; w < nwords; w += kCountThreads) {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int wi = w * 8 + j;
      const uint32_t c4 = wi < cwords ? cnt[wi] : 0u;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int key = w * 32 + j * 4 + k;
        const int n = cbeg + key;
        const bool exact = n < exact_head || n >= Nb - exact_tail;
        if (key < clen && !exact && static_cast<int>((c4 >> (8 * k)) & 0xffu) >= T) m |= 1u << (j * 4 + k);
      }
    }
    bitmask[static_cast<size_t>(bh) * Nw + (cbeg >> 5) + w] = m;
    mysel += __builtin_popcount(m);
  }
  if (counts) {
    const uint8_t* c8 = reinterpret_cast<const uint8_t*>(cnt);
    uint8_t* dst = counts + static_cast<size_t>(bh) * N + cbeg;
    for (int i = tid; i < cfull; i += kCountThreads) dst[i] = c8[i];
  }
  mysel = wave_sum_int(mysel);
  __syncthreads();
  if (lane == 0) wave_tot[wave] = mysel;
  __syncthreads();
  if (tid == 0) {
    int t = 0;
    for (int w = 0; w < kCountThreads / 64; ++w) t += wave_tot[w];
    chunk_nsel[static_cast<size_t>(bh) * nJ + J] = t;
  }
}

// ---------------------------------------------------------------------------
// attend (fp32 K/V): one workgroup (4 waves) per (sequence, kv head, context
// split); tiles of 16 selected keys, q.k on fp32 MFMA, P.V with FMAs.  The bf16
// path has its own kernel (attend_bf16.hip).
// ---------------------------------------------------------------------------
constexpr int kAttThreads = 256;
constexpr int kRing = 128;              // per-wave ring of selected keys

template <typename T>
struct VRow;
template <>
struct VRow<BF16> {   // 8 consecutive dims of one value row
  u32x4_t w;
  __device__ __forceinline__ void load(const uint16_t* p) { w = *reinterpret_cast<const u32x4_t*>(p); }
  __device__ __forceinline__ float get(int k) const {
    const uint32_t x = w[k >> 1];
    return (k & 1) ? bf16_hi(x) : bf16_lo(x);
  }
};
template <>
struct VRow<F32> {
  floatx4_t a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = reinterpret_cast<const floatx4_t*>(p)[0];
    b = reinterpret_cast<const floatx4_t*>(p)[1];
  }
  __device__ __forceinline__ float get(int k) const { return k < 4 ? a[k & 3] : b[k & 3]; }
};

template <typename T>
__device__ __forceinline__ float frag_sumsq(const Frag<T>& f);
template <>
__device__ __forceinline__ float frag_sumsq<BF16>(const Frag<BF16>& f) {
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = static_cast<float>(f.v[k][j]);
      s = fmaf(x, x, s);
    }
  return s;
}
template <>
__device__ __forceinline__ float frag_sumsq<F32>(const Frag<F32>& f) {
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 32; ++k) s = fmaf(f.v[k], f.v[k], s);
  return s;
}

__device__ __forceinline__ void wave_lds_fence() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

template <typename T, int GM>
__global__ __launch_bounds__(kAttThreads) void attend_kernel(
    const typename T::storage* __restrict__ q,       // [B][Hq][128]
    const typename T::storage* __restrict__ keys,    // [U][N][128]
    const typename T::storage* __restrict__ values,  // [U][N][128]
    const uint32_t* __restrict__ bitmask,            // [BH][Nw]
    const double* __restrict__ lnu_samples,          // [kLnuSamples]
    int Hq, int Hkv, int N, int P, int K, int Tth, float scale, int split_len, int nsplit,
    int n_sink, int n_window, int exact_len, int nexact, const int32_t* __restrict__ seq_lens,
    float* __restrict__ partials) {                  // [BH][nsplit + nexact][130]
  using S = typename T::storage;
  __shared__ float4 tab[kLnuTable];
  __shared__ float qn[16];
  __shared__ int sidx[4][kRing];
  __shared__ uint16_t shm[4][kRing];
  __shared__ float pbuf[4][16][16];     // [wave][key slot][head]
  __shared__ float abuf[4][16];         // [wave][head]
  __shared__ float wm[4][16], wl[4][16];
  __shared__ float wacc[4][GM][kHeadDim];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s = blockIdx.x, u = blockIdx.y;
  const int G = Hq / Hkv;
  const int b = u / Hkv, g = u % Hkv;
  const int bh0 = b * Hq + g * G;
  const int Nw = (N + 31) >> 5;
  const S* kb = keys + static_cast<size_t>(u) * P * kHeadDim;
  const S* vb = values + static_cast<size_t>(u) * P * kHeadDim;
  const bool k0 = (K == 0);
  const bool exact = s >= nsplit;     // a piece of the exact set (all heads, u = 1)
  const bool nolnu = k0 || exact;
  // this sequence's keys and exact set
  const int Nb = seq_len_of(seq_lens, b, N);
  int exact_head, exact_tail;
  exact_range(n_sink, n_window, Nb, exact_head, exact_tail);
  const int ne = exact_head + exact_tail;
  const int npart = nsplit + nexact;
  const float TK = static_cast<float>(Tth * K);

  for (int i = tid; i < kLnuTable; i += kAttThreads)
    tab[i] = nolnu ? make_float4(0.f, 0.f, 0.f, 0.f) : lnu_interval(lnu_samples, i);
  // query fragments: lane holds head (lane & 15), dims [32 (lane >> 4), +32)
  const int qh = lane & 15;
  Frag<T> Qf;
  Qf.load(q + static_cast<size_t>(bh0 + (qh < G ? qh : 0)) * kHeadDim + (lane >> 4) * 32, qh < G);
  if (wave == 0) {
    float ss = frag_sumsq<T>(Qf);
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    if (lane < 16) qn[lane] = sqrtf(ss);
  }
  __syncthreads();

  const int plen = exact ? exact_len : split_len;
  const int sb = exact ? (s - nsplit) * exact_len : s * split_len;
  const int se = min(exact ? ne : Nb, sb + plen);
  const int wq = plen / 4;
  const int wb = min(se, sb + wave * wq), we = min(se, sb + (wave + 1) * wq);

  const int grp = lane >> 4, slot = lane & 15;
  float m_run[4], l_run[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { m_run[i] = -INFINITY; l_run[i] = 0.f; }
  float acc[GM][8];
#pragma unroll
  for (int hh = 0; hh < GM; ++hh)
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[hh][d] = 0.f;

  int head = 0, cnt = 0;    // ring state (wave-uniform)

  auto process_tile = [&](int ntile) {
    const bool has = slot < ntile;
    const int e = (head + (has ? slot : 0)) & (kRing - 1);
    const int idx = sidx[wave][e];
    const int hmk = has ? static_cast<int>(shm[wave][e]) : 0;
    Frag<T> Kf;
    Kf.load(kb + static_cast<size_t>(idx) * kHeadDim + grp * 32, true);
    VRow<T> vr[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int vidx = __shfl(idx, grp + 4 * t);
      vr[t].load(vb + static_cast<size_t>(vidx) * kHeadDim + slot * 8);
    }
    floatx4_t sc = {0.f, 0.f, 0.f, 0.f};
    sc = Qf.mma(Kf, sc);     // sc[i] = q[head 4 grp + i] . k[slot]
    float kss = frag_sumsq<T>(Kf);
    kss += __shfl_xor(kss, 16);
    kss += __shfl_xor(kss, 32);
    const float kn = sqrtf(kss);
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = 4 * grp + i;
      const bool valid = hh < G && ((hmk >> hh) & 1);
      float logit = -INFINITY;
      if (valid) {
        const float x = sc[i];
        const float nn = qn[hh] * kn;
        const float cs = nn > 0.f ? x / nn : 0.f;
        logit = scale * x - (nolnu ? 0.f : log_inclusion(cs, tab, TK));
      }
      const float mt = row16_max(logit);
      const float mnew = fmaxf(m_run[i], mt);
      const float alpha = (mnew == -INFINITY) ? 1.f : __expf(m_run[i] - mnew);
      p[i] = (logit == -INFINITY) ? 0.f : __expf(logit - mnew);
      l_run[i] = l_run[i] * alpha + row16_sum(p[i]);
      m_run[i] = mnew;
      if (slot == 0) abuf[wave][hh] = alpha;
      pbuf[wave][slot][hh] = p[i];
    }
    wave_lds_fence();
#pragma unroll
    for (int hh = 0; hh < GM; ++hh) {
      if (hh < G) {
        const float a = abuf[wave][hh];
        if (a != 1.f) {
#pragma unroll
          for (int d = 0; d < 8; ++d) acc[hh][d] *= a;
        }
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int j = grp + 4 * t;
#pragma unroll
      for (int hh = 0; hh < GM; ++hh) {
        const float pj = pbuf[wave][j][hh];
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[hh][d] = fmaf(pj, vr[t].get(d), acc[hh][d]);
      }
    }
    wave_lds_fence();
  };

  for (int blk = wb; blk < we; blk += 64) {
    const int i = blk + lane;           // key, or position in the exact set
    int n = i, hm = 0;
    if (exact) {
      n = i < exact_head ? i : i + (Nb - ne);
      hm = (1 << G) - 1;
    } else {
      const int w0 = blk >> 5;
      for (int hh = 0; hh < G; ++hh) {
        const uint32_t* bm = bitmask + static_cast<size_t>(bh0 + hh) * Nw;
        const uint32_t lo = bm[w0];
        const uint32_t hi = (w0 + 1 < Nw) ? bm[w0 + 1] : 0u;
        const uint32_t word = lane < 32 ? lo : hi;
        hm |= static_cast<int>((word >> (lane & 31)) & 1u) << hh;
      }
    }
    const bool any = (i < we) && hm != 0;
    const uint64_t bal = ballot(any);
    if (any) {
      const int e = (head + cnt + mbcnt(bal)) & (kRing - 1);
      sidx[wave][e] = n;
      shm[wave][e] = static_cast<uint16_t>(hm);
    }
    cnt += __builtin_popcountll(bal);
    wave_lds_fence();
    while (cnt >= 16) {
      process_tile(16);
      head = (head + 16) & (kRing - 1);
      cnt -= 16;
    }
  }
  if (cnt > 0) {
    process_tile(cnt);
    head = (head + cnt) & (kRing - 1);
    cnt = 0;
  }

  // combine the four lane groups (each summed a quarter of every tile's keys)
#pragma unroll
  for (int hh = 0; hh < GM; ++hh)
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      acc[hh][d] += __shfl_xor(acc[hh][d], 16);
      acc[hh][d] += __shfl_xor(acc[hh][d], 32);
    }
  if (slot == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      wm[wave][4 * grp + i] = m_run[i];
      wl[wave][4 * grp + i] = l_run[i];
    }
  }
  if (grp == 0) {
#pragma unroll
    for (int hh = 0; hh < GM; ++hh)
#pragma unroll
      for (int d = 0; d < 8; ++d) wacc[wave][hh][slot * 8 + d] = acc[hh][d];
  }
  __syncthreads();
  for (int e = tid; e < G * kHeadDim; e += kAttThreads) {
    const int hh = e / kHeadDim, d = e % kHeadDim;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w][hh]);
    float A = 0.f, Lm = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if (wm[w][hh] == -INFINITY) continue;
        const float f = __expf(wm[w][hh] - M);
        A = fmaf(wacc[w][hh][d], f, A);
        Lm = fmaf(wl[w][hh], f, Lm);
      }
    }
    float* dst = partials + (static_cast<size_t>(bh0 + hh) * npart + s) * kPartialStride;
    dst[d] = A;
    if (d == 0) {
      dst[kHeadDim] = M;
      dst[kHeadDim + 1] = Lm;
    }
  }
}

// ---------------------------------------------------------------------------
// merge: one workgroup (4 waves) per query head.  Wave w folds the partials
// s = w, w + 4, ... (the context splits, then the pieces of the exact set of
// the hybrid decode) into a running (max, sum, acc) with each lane owning two
// dims; the four wave states are combined through LDS.
// ---------------------------------------------------------------------------
constexpr int kMergeThreads = 256;

__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const float* __restrict__ partials,
                                                              const int32_t* __restrict__ chunk_nsel,
                                                              int npart, int nJ, float* __restrict__ out,
                                                              float* __restrict__ lse, int32_t* __restrict__ nsel) {
  __shared__ float wm[4], wl[4];
  __shared__ float wacc[4][kHeadDim];
  __shared__ int wn[4];
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* P = partials + static_cast<size_t>(bh) * npart * kPartialStride;
  // the overall max first, so that every partial's weight exp(m_s - M) is
  // known without a running rescale and the loads of all of them can be in flight
  float mx = -INFINITY;
  for (int s = tid; s < npart; s += kMergeThreads) mx = fmaxf(mx, P[static_cast<size_t>(s) * kPartialStride + kHeadDim]);
  mx = wave_max(mx);
  if (lane == 0) wm[wave] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
  __syncthreads();
  float l = 0.f, a0 = 0.f, a1 = 0.f;
  if (M != -INFINITY) {
#pragma unroll 4
    for (int s = wave; s < npart; s += 4) {
      const float* ps = P + static_cast<size_t>(s) * kPartialStride;
      const float ms = ps[kHeadDim];
      const float f = (ms == -INFINITY) ? 0.f : __expf(ms - M);
      l = fmaf(ps[kHeadDim + 1], f, l);
      a0 = fmaf(ps[2 * lane], f, a0);
      a1 = fmaf(ps[2 * lane + 1], f, a1);
    }
  }
  int cnt = 0;
  for (int j = tid; j < nJ; j += kMergeThreads) cnt += chunk_nsel[static_cast<size_t>(bh) * nJ + j];
  cnt = wave_sum_int(cnt);
  if (lane == 0) {
    wl[wave] = l;
    wn[wave] = cnt;
  }
  wacc[wave][2 * lane] = a0;
  wacc[wave][2 * lane + 1] = a1;
  __syncthreads();
  if (tid < kHeadDim) {
    const float A = wacc[0][tid] + wacc[1][tid] + wacc[2][tid] + wacc[3][tid];
    const float Lm = wl[0] + wl[1] + wl[2] + wl[3];
    out[static_cast<size_t>(bh) * kHeadDim + tid] = (M == -INFINITY) ? 0.f : A / Lm;
    if (tid == 0) {
      if (lse) lse[bh] = (M == -INFINITY) ? -INFINITY : M + logf(Lm);
      if (nsel) nsel[bh] = wn[0] + wn[1] + wn[2] + wn[3];
    }
  }
}

// ---------------------------------------------------------------------------
// Host-side launcher
// ---------------------------------------------------------------------------
template <typename T, int GM>
static hipError_t launch_attend(const DecodeArgs& a, hipStream_t stream) {
  using S = typename T::storage;
  return launch(kKAttend, attend_kernel<T, GM>, dim3(a.nsplit + a.nexact, a.B * a.Hkv), dim3(kAttThreads), 0, stream,
                static_cast<const S*>(a.q), static_cast<const S*>(a.keys), static_cast<const S*>(a.values),
                static_cast<const uint32_t*>(a.bitmask), static_cast<const double*>(a.lnu_samples), a.Hq, a.Hkv,
                a.N, a.P, a.K, a.T, a.scale, a.split_len, a.nsplit, a.n_sink, a.n_window, a.exact_len, a.nexact, a.seq_lens,
                a.partials);
}

template <typename T>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  using S = typename T::storage;
  const int BH = a.B * a.Hq;
  const int G = a.Hq / a.Hkv;
  const int hpb = a.w_heads > 1 ? G : kQHeads;          // heads per qhash workgroup
  const int head_blocks = (BH + hpb - 1) / hpb;
  const size_t w_head_stride = a.w_heads > 1 ? static_cast<size_t>(kHeadDim) * a.L * a.K : 0;
  const int tpw = a.K > 0 ? 64 / a.K : 256;
  const int xblocks = (a.L + tpw - 1) / tpw;
  const int tab_blocks = (kLnuSamples + xblocks * 4 - 1) / (xblocks * 4);   // 4 samples per workgroup
  hipError_t e = launch(kKQhash, qhash_kernel<T>, dim3(xblocks, head_blocks + tab_blocks), dim3(256), 0,
                        stream, static_cast<const S*>(a.q), static_cast<const S*>(a.W), a.qcodes,
                        a.lnu_samples, BH, a.K, a.L, a.T, head_blocks, G, a.Hkv, w_head_stride);
  if (e != hipSuccess) return e;
  const size_t lds = ((static_cast<size_t>(1) << a.stride_log2) + 3) & ~static_cast<size_t>(3);
  // 1024-thread workgroups while the (head, chunk) pairs fit in about two
  // per CU, 256-thread ones beyond that
  const bool small_wg = static_cast<long long>(a.nJ) * BH > 1024;
  const void* cs = small_wg ? reinterpret_cast<const void*>(count_select_kernel<256>)
                            : reinterpret_cast<const void*>(count_select_kernel<1024>);
  e = ensure_lds_limit(cs, lds);
  if (e != hipSuccess) return e;
  if (small_wg)
    e = launch(kKCountSelect, count_select_kernel<256>, dim3(a.nJ, BH), dim3(256), static_cast<unsigned>(lds),
               stream, static_cast<const uint16_t*>(a.qcodes), a.indices, a.offsets, a.Hq, a.Hkv, a.N, a.P, a.K,
               a.L, a.T, a.stride_log2, a.nJ, a.nJP, a.bitmask, a.chunk_nsel, a.counts, a.n_sink, a.n_window,
               a.seq_lens);
  else
    e = launch(kKCountSelect, count_select_kernel<1024>, dim3(a.nJ, BH), dim3(1024), static_cast<unsigned>(lds),
               stream, static_cast<const uint16_t*>(a.qcodes), a.indices, a.offsets, a.Hq, a.Hkv, a.N, a.P, a.K,
               a.L, a.T, a.stride_log2, a.nJ, a.nJP, a.bitmask, a.chunk_nsel, a.counts, a.n_sink, a.n_window,
               a.seq_lens);
  if (e != hipSuccess) return e;
  if constexpr (sizeof(S) == 2)
    e = launch_attend_bf16(a, stream);
  else if (G <= 4)
    e = launch_attend<T, 4>(a, stream);
  else if (G <= 8)
    e = launch_attend<T, 8>(a, stream);
  else
    e = launch_attend<T, 16>(a, stream);
  if (e != hipSuccess) return e;
  return launch(kKMerge, merge_kernel, dim3(BH), dim3(kMergeThreads), 0, stream,
                static_cast<const float*>(a.partials), static_cast<const int32_t*>(a.chunk_nsel),
                a.nsplit + a.nexact, a.nJ, a.out, a.lse, a.nsel);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  return a.dtype == 1 ? launch_decode_t<BF16>(a, stream) : launch_decode_t<F32>(a, stream);
}

}  // namespace lsh
