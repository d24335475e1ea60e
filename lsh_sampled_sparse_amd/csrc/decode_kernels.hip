// Decode-side kernels for gfx950.
//
// One decode step of MagicPIG's LSH sampling ("MagicPIG: LSH Sampling for
// Efficient LLM Generation", GrooveSquid summary; MagicPIG project summary on
// sourcepulse, "How It Works") runs as two launches on one stream:
//   qhash   SimHash codes of every query head (same W and sign rule as the
//           keys); one extra row of workgroups zeroes the decode launch's
//           counters
//   decode  one grid whose workgroups take four roles (decode_roles.h):
//           the ln-u correction table; per (key chunk, query head) the probe
//           of the head's L buckets inside the chunk, the collision counts in
//           LDS byte counters and the selection bitmask (count >= T); per
//           (context split, sequence, kv head) the union of the group's
//           selections, ballot compaction, gathered K/V rows, q.k, 1/u
//           weights, online softmax in fp32 and P.V (the hybrid decode's
//           exact keys with every head and unit weights), written as one
//           partial state per query head; the log-sum-exp merges of those
//           partials (the stable merge MAC-Attention also uses,
//           "MAC-Attention" README, "How It Works") run in the last
//           workgroups to finish.  The bf16 grid is in attend_bf16.hip, the
//           fp32 one below.
#include <math.h>

#include "decode_roles.h"
#include "lsh_device.h"
#include "lsh_kernels.h"

namespace lsh {

constexpr float kPi = 3.14159265358979323846f;
constexpr float kLnUFloor = -69.07755278982137f;   // ln(1e-30)

// ---------------------------------------------------------------------------
// ln u.  u(theta) = P[Binomial(L, P) >= T] with P = (1 - theta/pi)^K.
// Writing ln u = T ln P + g(P),  g(P) = ln sum_{i>=T} C(L,i) P^(i-T) (1-P)^(L-i),
// g is smooth on [0, 1] (g(0) = ln C(L,T), g(1) = 0): the decode's table
// workgroups sample it in fp64 at theta_t = t pi / (2 kLnuTable) and store
// one quadratic per interval of width pi / kLnuTable (through its start,
// middle and end); T ln P = T K ln p is evaluated from p itself.
// ---------------------------------------------------------------------------
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
// W loads at once; the four partial sums meet in LDS.  The workgroups with
// blockIdx.y == head_blocks zero the decode launch's counters instead, and
// those past it sample the ln-u correction (one angle per wave, in fp64).
// ---------------------------------------------------------------------------
constexpr int kQHeads = 16;

template <typename T>
__global__ __launch_bounds__(256) void qhash_kernel(const typename T::storage* __restrict__ q,
                                                    const typename T::storage* __restrict__ W,
                                                    uint16_t* __restrict__ qcodes, int32_t* __restrict__ sync,
                                                    int nsync, double* __restrict__ lnu_samples, int BH, int K,
                                                    int L, int Tth, int head_blocks, int G, int Hkv,
                                                    size_t w_head_stride) {
  __shared__ __attribute__((aligned(16))) float qs[kQHeads][kHeadDim];
  __shared__ float part[4][kQHeads][64];
  __shared__ uint8_t sgn[kQHeads][64];
  __shared__ double lc[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (static_cast<int>(blockIdx.y) == head_blocks) {
    for (int i = blockIdx.x * 256 + tid; i < nsync; i += gridDim.x * 256) sync[i] = 0;
    return;
  }
  if (static_cast<int>(blockIdx.y) > head_blocks) {
    // the ln-u correction g(theta) at one sample angle per wave
    const int j = ((blockIdx.y - head_blocks - 1) * gridDim.x + blockIdx.x) * 4 + wave;
    if (K == 0 || j - wave >= kLnuSamples) return;   // (workgroup-uniform)
    // ln C(L, i) = ln L! - ln i! - ln (L - i)!: one lgamma per thread
    __shared__ double lf[256];
    if (tid <= L) lf[tid] = lgamma(static_cast<double>(tid) + 1.0);
    __syncthreads();
    if (tid <= L) lc[tid] = lf[L] - lf[tid] - lf[L - tid];
    __syncthreads();
    if (j >= kLnuSamples) return;
    const double g = lnu_correction_wave(j * (3.14159265358979323846 / (2 * kLnuTable)), K, L, Tth, lc, lane);
    if (lane == 0) lnu_samples[j] = g;
    return;
  }
  // a workgroup hashes up to 16 heads: 16 consecutive ones with one shared
  // W; with a W per kv head, the G heads of kv head g in each of 16 / G
  // consecutive sequences (they all hash with W[g]).  head_of(hh) is the
  // head of slot hh, or -1
  int Hq = 0, Bq = 0, spb = 0, gw = 0, b0 = 0;         // per-head W: the workgroup's kv head and sequences
  if (w_head_stride) {
    Hq = G * Hkv;
    Bq = BH / Hq;
    spb = kQHeads / G;
    const int nbb = (Bq + spb - 1) / spb;
    gw = static_cast<int>(blockIdx.y) / nbb;
    b0 = (static_cast<int>(blockIdx.y) % nbb) * spb;
  }
  auto head_of = [&](int hh) {
    if (!w_head_stride) {
      const int h = static_cast<int>(blockIdx.y) * kQHeads + hh;
      return hh < kQHeads && h < BH ? h : -1;
    }
    const int b = b0 + hh / G;
    return hh < spb * G && b < Bq ? b * Hq + gw * G + hh % G : -1;
  };
  if (K == 0) {
    for (int e = blockIdx.x * 256 + tid; e < kQHeads * L; e += gridDim.x * 256) {
      const int h = head_of(e / L);
      if (h >= 0) qcodes[static_cast<size_t>(h) * L + e % L] = 0;
    }
    return;
  }
  W += static_cast<size_t>(gw) * w_head_stride;
  const int tpw = 64 / K;               // whole tables per workgroup
  const int l0 = blockIdx.x * tpw;
  // this lane's column of W over the wave's 32 dims, loaded first: the loads
  // do not depend on q, so they are in flight with q's
  const int LK = L * K;
  const int col = l0 * K + lane;
  const bool colv = lane < tpw * K && col < LK;
  float w[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const size_t at = static_cast<size_t>(32 * wave + i) * LK + (colv ? col : 0);
    if constexpr (sizeof(typename T::storage) == 2)
      w[i] = bf16_to_f32(W[at]);   // (converted once the loads arrive)
    else
      w[i] = W[at];
  }
  {
    // 16 heads x 128 dims: thread t takes 8 consecutive dims of head t / 16
    // in one (bf16) or two (fp32) 16-byte loads
    const int hh = tid >> 4, c8 = (tid & 15) * 8;
    const int hq = head_of(hh);
    const bool okh = hq >= 0;
    const typename T::storage* src = q + static_cast<size_t>(okh ? hq : 0) * kHeadDim + c8;
    float v[8];
    if constexpr (sizeof(typename T::storage) == 2) {
      const u32x4_t w4 = *reinterpret_cast<const u32x4_t*>(src);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[2 * k] = bf16_lo(w4[k]);
        v[2 * k + 1] = bf16_hi(w4[k]);
      }
    } else {
      const floatx4_t a = reinterpret_cast<const floatx4_t*>(src)[0], c = reinterpret_cast<const floatx4_t*>(src)[1];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[k] = a[k];
        v[4 + k] = c[k];
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) qs[hh][c8 + k] = okh ? v[k] : 0.f;
  }
  __syncthreads();
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
    const int l = l0 + t, h = head_of(hh);
    if (h >= 0 && l < L) {
      uint32_t code = 0;
      for (int b = 0; b < K; ++b) code |= static_cast<uint32_t>(sgn[hh][t * K + b]) << b;
      qcodes[static_cast<size_t>(h) * L + l] = static_cast<uint16_t>(code);
    }
  }
}

// ---------------------------------------------------------------------------
// attend (fp32 K/V) role: partial slot s of unit u, tiles of 16 selected
// keys, q.k on fp32 MFMA, P.V with FMAs.  The bf16 path has its own role and
// grid (attend_bf16.hip).
// ---------------------------------------------------------------------------
constexpr int kRing = 128;              // per-wave ring of selected keys

struct VRowF32 {   // 8 consecutive dims of one fp32 value row
  floatx4_t a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = reinterpret_cast<const floatx4_t*>(p)[0];
    b = reinterpret_cast<const floatx4_t*>(p)[1];
  }
  __device__ __forceinline__ float get(int k) const { return k < 4 ? a[k & 3] : b[k & 3]; }
};

__device__ __forceinline__ float frag_sumsq(const Frag<F32>& f) {
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 32; ++k) s = fmaf(f.v[k], f.v[k], s);
  return s;
}

__device__ __forceinline__ void wave_lds_fence() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

template <int GM>
struct AttendF32Lds {
  float4 tab[kLnuTable];
  float qn[16];
  int sidx[4][kRing];
  uint16_t shm[4][kRing];
  float pbuf[4][16][16];     // [wave][key slot][head]
  float abuf[4][16];         // [wave][head]
  float wm[4][16], wl[4][16];
  float wacc[4][GM][kHeadDim];
  int flag;
};

template <int GM>
__device__ __forceinline__ void attend_f32_role(const FusedParams& p, int s, int u, unsigned char* smem) {
  LSH_PCHECK(p, u < p.B * p.Hkv && s < p.nsplit, kChkSlot);
  AttendF32Lds<GM>& A = *reinterpret_cast<AttendF32Lds<GM>*>(smem);
  const float* __restrict__ q = static_cast<const float*>(p.q);
  const float* __restrict__ keys = static_cast<const float*>(p.keys);
  const float* __restrict__ values = static_cast<const float*>(p.values);
  const int Hq = p.Hq, N = p.N, K = p.K;
  const float scale = p.scale;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = p.G;
  const int b = u / p.Hkv, g = u % p.Hkv;
  const int bh0 = b * Hq + g * G;
  const int Nw = (N + 31) >> 5;
  const float* kb = keys + static_cast<size_t>(u) * p.P * kHeadDim;
  const float* vb = values + static_cast<size_t>(u) * p.P * kHeadDim;
  const bool k0 = (K == 0);
  const bool nolnu = k0;
  const int Nb = seq_len_of(p.seq_lens, b, N);
  int exact_head, exact_tail;
  exact_range(p.n_sink, p.n_window, Nb, exact_head, exact_tail);
  const float TK = static_cast<float>(p.T * K);

  const int sb = s * p.split_len;
  const int se = min(Nb, sb + p.split_len);
  const int wq = p.split_len / 4;
  const int wb = min(se, sb + wave * wq), we = min(se, sb + (wave + 1) * wq);

  // query fragments: lane holds head (lane & 15), dims [32 (lane >> 4), +32)
  const int qh = lane & 15;
  Frag<F32> Qf;
  Qf.load(q + static_cast<size_t>(bh0 + (qh < G ? qh : 0)) * kHeadDim + (lane >> 4) * 32, qh < G);

  // the ln-u table's samples, in flight during the wait for the selection
  LnuFetch lf;
  lnu_fetch(p, nolnu, lf);
  // the split's selection must be complete
  bool ok = true;
  if (sb < se) {
    const int j0 = sb >> p.stride_log2, j1 = (se - 1) >> p.stride_log2;
    ok = wait_counters(p.ready + u * p.nJ + j0, j1 - j0 + 1, G, &A.flag);
  }
  lnu_store(lf, nolnu, A.tab);
  if (wave == 0) {
    float ss = frag_sumsq(Qf);
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    if (lane < 16) A.qn[lane] = sqrtf(ss);
  }
  __syncthreads();

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
    const int rix = A.sidx[wave][e];
    const int idx = rix & ~kExactKey;
    const bool exk = rix < 0;          // a key of the exact set: ln u = 0
    const int hmk = has ? static_cast<int>(A.shm[wave][e]) : 0;
    Frag<F32> Kf;
    Kf.load(kb + static_cast<size_t>(idx) * kHeadDim + grp * 32, true);
    VRowF32 vr[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int vidx = __shfl(idx, grp + 4 * t);
      vr[t].load(vb + static_cast<size_t>(vidx) * kHeadDim + slot * 8);
    }
    floatx4_t sc = {0.f, 0.f, 0.f, 0.f};
    sc = Qf.mma(Kf, sc);     // sc[i] = q[head 4 grp + i] . k[slot]
    float kss = frag_sumsq(Kf);
    kss += __shfl_xor(kss, 16);
    kss += __shfl_xor(kss, 32);
    const float kn = sqrtf(kss);
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = 4 * grp + i;
      const bool valid = hh < G && ((hmk >> hh) & 1);
      float logit = -INFINITY;
      if (valid) {
        const float x = sc[i];
        const float nn = A.qn[hh] * kn;
        const float cs = nn > 0.f ? x / nn : 0.f;
        logit = scale * x - (nolnu || exk ? 0.f : log_inclusion(cs, A.tab, TK));
      }
      const float mt = row16_max(logit);
      const float mnew = fmaxf(m_run[i], mt);
      const float alpha = (mnew == -INFINITY) ? 1.f : __expf(m_run[i] - mnew);
      pr[i] = (logit == -INFINITY) ? 0.f : __expf(logit - mnew);
      l_run[i] = l_run[i] * alpha + row16_sum(pr[i]);
      m_run[i] = mnew;
      if (slot == 0) A.abuf[wave][hh] = alpha;
      A.pbuf[wave][slot][hh] = pr[i];
    }
    wave_lds_fence();
#pragma unroll
    for (int hh = 0; hh < GM; ++hh) {
      if (hh < G) {
        const float a = A.abuf[wave][hh];
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
        const float pj = A.pbuf[wave][j][hh];
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[hh][d] = fmaf(pj, vr[t].get(d), acc[hh][d]);
      }
    }
    wave_lds_fence();
  };

  for (int blk = wb; blk < we; blk += 64) {
    const int n = blk + lane;
    int hm = 0;
    const int w0 = blk >> 5;
    for (int hh = 0; hh < G; ++hh) {
      const uint32_t* bm = p.bitmask + static_cast<size_t>(bh0 + hh) * Nw;
      const uint32_t lo = ld_agent(bm + w0);
      const uint32_t hi = (w0 + 1 < Nw) ? ld_agent(bm + w0 + 1) : 0u;
      const uint32_t word = lane < 32 ? lo : hi;
      hm |= static_cast<int>((word >> (lane & 31)) & 1u) << hh;
    }
    // a key of the exact set (never in the bitmask): every head, ln u = 0,
    // marked in bit 31 of its ring entry
    const bool ex = n < exact_head || n >= Nb - exact_tail;
    hm = ex ? (1 << G) - 1 : hm;
    const bool any = (n < we) && hm != 0;
    const uint64_t bal = ballot(any);
    if (any) {
      const int e = (head + cnt + mbcnt(bal)) & (kRing - 1);
      A.sidx[wave][e] = ex ? (n | kExactKey) : n;
      A.shm[wave][e] = static_cast<uint16_t>(hm);
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
      A.wm[wave][4 * grp + i] = m_run[i];
      A.wl[wave][4 * grp + i] = l_run[i];
    }
  }
  if (grp == 0) {
#pragma unroll
    for (int hh = 0; hh < GM; ++hh)
#pragma unroll
      for (int d = 0; d < 8; ++d) A.wacc[wave][hh][slot * 8 + d] = acc[hh][d];
  }
  __syncthreads();
  for (int e = tid; e < G * kHeadDim; e += kFusedThreads) {
    const int hh = e / kHeadDim, d = e % kHeadDim;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, A.wm[w][hh]);
    float Acc = 0.f, Lm = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if (A.wm[w][hh] == -INFINITY) continue;
        const float f = __expf(A.wm[w][hh] - M);
        Acc = fmaf(A.wacc[w][hh][d], f, Acc);
        Lm = fmaf(A.wl[w][hh], f, Lm);
      }
    }
    if (!ok) {   // a wait gave up: poison this partial
      Acc = __builtin_nanf("");
      M = 0.f;
      Lm = 1.f;
    }
    float* dst = p.partials + (static_cast<size_t>(bh0 + hh) * p.npart + s) * kPartialStride;
    st_agent(dst + d, Acc);
    if (d == 0) {
      st_agent(dst + kHeadDim, M);
      st_agent(dst + kHeadDim + 1, Lm);
    }
  }
}

// The one-launch decode for fp32 K/V (roles and their order: decode_roles.h).
template <int GM>
__global__ __launch_bounds__(kFusedThreads) void decode_f32_kernel(FusedParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[cmax(sizeof(AttendF32Lds<GM>), kRolesLdsBytes)];
  const DecodeRole r = decode_role(p, blockIdx.x);
  if (r.count) {
    if (p.count_heads > 1) count_role_heads(p, r.J, r.bh, smem);
    else count_role(p, r.J, r.bh, smem);
    return;
  }
  attend_f32_role<GM>(p, r.slot, r.u, smem);
  __syncthreads();
  finish_slot(p, r.u, r.slot, smem);
}

// ---------------------------------------------------------------------------
// Host-side launcher
// ---------------------------------------------------------------------------
template <typename T>
static hipError_t launch_qhash(const DecodeArgs& a, int nsync, int kid, hipStream_t stream) {
  using S = typename T::storage;
  const int BH = a.B * a.Hq;
  const int G = a.Hq / a.Hkv;
  // workgroups of heads: 16 consecutive heads each with one W; with a W per
  // kv head, one per (kv head, 16 / G consecutive sequences)
  const int spb = kQHeads / G;
  const int head_blocks = a.w_heads > 1 ? a.Hkv * ((a.B + spb - 1) / spb) : (BH + kQHeads - 1) / kQHeads;
  const size_t w_head_stride = a.w_heads > 1 ? static_cast<size_t>(kHeadDim) * a.L * a.K : 0;
  const int tpw = a.K > 0 ? 64 / a.K : 256;
  const int xblocks = (a.L + tpw - 1) / tpw;
  const int tab_rows = a.K > 0 ? (kLnuSamples + 4 * xblocks - 1) / (4 * xblocks) : 0;   // 4 samples per workgroup
  return launch(kid, qhash_kernel<T>, dim3(xblocks, head_blocks + 1 + tab_rows), dim3(256), 0, stream,
                static_cast<const S*>(a.q), static_cast<const S*>(a.W), a.qcodes, a.sync, nsync, a.lnu_samples,
                BH, a.K, a.L, a.T, head_blocks, G, a.Hkv, w_head_stride);
}

#ifdef LSH_TRACE
// trace builds: the buffer of per-workgroup phase stamps of the next decodes
static unsigned long long* g_trace = nullptr;
extern "C" void lsh_trace_set(void* buffer) { g_trace = static_cast<unsigned long long*>(buffer); }
#endif

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  const int U = a.B * a.Hkv;
  const int BH = a.B * a.Hq;
  FusedParams p{};
#ifdef LSH_TRACE
  p.trace = g_trace;
#endif
#ifdef LSH_CHECKED
  p.check = g_check;
#endif
  p.q = a.q;
  p.keys = a.keys;
  p.values = a.values;
  p.indices = a.indices;
  p.offsets = a.offsets;
  p.seq_lens = a.seq_lens;
  p.qcodes = a.qcodes;
  p.bitmask = a.bitmask;
  p.chunk_nsel = a.chunk_nsel;
  p.lnu_samples = a.lnu_samples;
  p.partials = a.partials;
  p.out = a.out;
  p.lse = a.lse;
  p.nsel = a.nsel;
  p.counts = a.counts;
  p.B = a.B;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.G = a.Hq / a.Hkv;
  p.N = a.N;
  p.P = a.P;
  p.K = a.K;
  p.L = a.L;
  p.T = a.T;
  p.stride_log2 = a.stride_log2;
  p.nJ = a.nJ;
  p.nJP = a.nJP;
  p.split_len = a.split_len;
  p.nsplit = a.nsplit;
  p.n_sink = a.n_sink;
  p.n_window = a.n_window;
  p.npart = a.nsplit;
  p.scale = a.scale;
  // counters: ready [U][nJ], arrive_unit [U]
  p.ready = a.sync;
  p.arrive_unit = p.ready + U * a.nJ;
  // count workgroups cover count_heads query heads of one unit (a divisor
  // of G): the fewest that fit one round of resident workgroups, within the
  // LDS for the heads' byte counters and segments
  int hc = 1;
  while (BH / hc * a.nJ > kResidentWG) {
    int nx = hc + 1;
    while (nx <= p.G && p.G % nx != 0) ++nx;
    if (nx > p.G || nx * a.L > kCountSegs || (nx << a.stride_log2) > kCountCounterBytes) break;
    hc = nx;
  }
  if (a.L > kCountSegs || (1 << a.stride_log2) > kCountCounterBytes) return hipErrorInvalidValue;
  p.count_heads = hc;
  p.n_count_wg = BH / hc * a.nJ;
  p.n_attend_wg = U * a.nsplit;
  // a fold keeps the (head, slot) pairs of its heads in LDS
  const int F = p.G < p.npart ? p.G : p.npart;
  // splits of up to 64 / F units at a time are dispatched interleaved: at
  // most 64 finishers can then wait for workgroups that have no slot yet
  p.unit_group = F > 0 && 64 / F > 1 ? 64 / F : 1;
  if ((p.G + F - 1) / F * p.npart > kMergeMaxPairs || p.G > 16 || a.L > 255) return hipErrorInvalidValue;
  const int nsync = fused_sync_words(U, a.nJ);
  const int untimed = a.timed ? 0 : kUntimed;
  const int kq = kKQhash | untimed, kd = kKDecode | untimed;
  hipError_t e = (a.dtype == 1) ? launch_qhash<BF16>(a, nsync, kq, stream) : launch_qhash<F32>(a, nsync, kq, stream);
  if (e != hipSuccess) return e;
  if (a.dtype == 1) return launch_decode_bf16(p, kd, stream);
  const dim3 grid(p.n_count_wg + p.n_attend_wg);
  if (p.G <= 4) return launch(kd, decode_f32_kernel<4>, grid, dim3(kFusedThreads), 0, stream, p);
  if (p.G <= 8) return launch(kd, decode_f32_kernel<8>, grid, dim3(kFusedThreads), 0, stream, p);
  return launch(kd, decode_f32_kernel<16>, grid, dim3(kFusedThreads), 0, stream, p);
}

}  // namespace lsh
