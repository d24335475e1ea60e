// Weighted partial attention over the selected keys, bf16 K/V, gfx950.
//
// One workgroup (4 waves) per (sequence, kv head, context split); each wave
// owns a quarter of the split.  The selected keys of the group (the union of
// its query heads' selections) are compacted with ballots into a per-wave LDS
// ring and processed in tiles of 32:
//   * the tile's K rows are loaded straight into MFMA fragments and its V
//     rows into registers; the next tile's loads are issued before the current
//     tile's softmax and P.V, so each wave keeps a tile of K/V in flight;
//   * S = q.k on MFMA 16x16x32 (fp32 accumulate), logits s q.k - ln u with the
//     1/u importance weight, online softmax per head;
//   * P.V on MFMA: V goes through LDS row-major and comes back as the B operand
//     with transposing LDS reads (ds_read_b64_tr_b16: within each 16-lane group
//     lane j receives element j & 3 of source lanes (j >> 2) + 4 i, i = 0..3);
//     P is split into bf16 high and low parts (two MFMAs) so the weights keep
//     about 16 mantissa bits.
// The 1/u weight needs arccos of the q-k cosine: a polynomial (Abramowitz &
// Stegun 4.4.46) and the hardware log2 keep it to ~35 instructions per pair.
// The four waves' (max, sum, acc) states are merged through LDS into one
// partial per query head and split, for the log-sum-exp merge that follows.
// The hybrid decode's exact set (for a sequence of n keys, keys
// [0, exact_head) and [n - exact_tail, n)) is taken by the context splits
// that hold it: such a key goes to every head of the group with weight 1
// (ln u = 0), so the split's softmax covers its sampled keys and its exact
// keys together, which equals the log-sum-exp merge of the two parts (the
// count role leaves exact keys out of the bitmask).
#include <math.h>

#include "decode_roles.h"
#include "lsh_device.h"
#include "lsh_kernels.h"

namespace lsh {

namespace {

constexpr int kWaves = 4;
constexpr int kTile = 32;         // keys per tile (the K extent of one MFMA 16x16x32)
constexpr int kRingN = 128;       // per-wave ring of compacted keys
constexpr int kVRow = 136;        // LDS row of one V row: 128 dims + 8 pad (272 B)
constexpr int kBlock = 512;       // keys whose mask words are fetched together
constexpr float kPiF = 3.14159265358979323846f;
constexpr float kLnUFloorF = -69.07755278982137f;   // ln(1e-30)

typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// 8 bytes from LDS, transposed across each 16-lane group (see above).
__device__ __forceinline__ s16x4_t ds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p));
}

__device__ __forceinline__ bf16x8_t join8(s16x4_t a, s16x4_t b) {
  struct P2 {
    s16x4_t a, b;
  } x{a, b};
  return __builtin_bit_cast(bf16x8_t, x);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
struct Bf16Pairs {
  bf16x2_t p[4];
};

// arccos of |c| in [0, 1] from the approximation of Abramowitz & Stegun
// 4.4.46 (Hastings): acos(x) = sqrt(1 - x) * sum_{i<8} a_i x^i with
// |error| <= 2e-8 in exact arithmetic (about 3e-7 rad in fp32).  The angle
// itself is theta = r for c >= 0 and pi - r for c < 0.
__device__ __forceinline__ float acos_abs_as(float c) {
  const float x = fabsf(c);
  float p = -0.0012624911f;
  p = fmaf(p, x, 0.0066700901f);
  p = fmaf(p, x, -0.0170881256f);
  p = fmaf(p, x, 0.0308918810f);
  p = fmaf(p, x, -0.0501743046f);
  p = fmaf(p, x, 0.0889789874f);
  p = fmaf(p, x, -0.2145988016f);
  p = fmaf(p, x, 1.5707963050f);
  return __builtin_amdgcn_sqrtf(1.f - x) * p;
}

// ln u of a key at cosine c with the query: T K ln p + g(theta) with
// p = 1 - theta / pi, g from the interval quadratics (lnu_interval); clamped
// at ln(1e-30).  For c < 0, p = r / pi straight from r = acos(|c|), so the
// keys nearly opposite the query (theta -> pi, the largest 1/u) keep the
// relative accuracy of r instead of the cancellation in 1 - theta / pi.
__device__ __forceinline__ float lnu_of_cos(float c, const float4* tab4, float TKln2) {
  const float cc = fminf(1.f, fmaxf(-1.f, c));
  const float r = acos_abs_as(cc);
  const bool neg = cc < 0.f;
  const float th = neg ? kPiF - r : r;
  const float x = th * (static_cast<float>(kLnuTable) / kPiF);
  const int j = min(static_cast<int>(x), kLnuTable - 1);
  const float4 e = tab4[j];
  const float f = x - static_cast<float>(j);
  const float g = fmaf(f, fmaf(f, e.z, e.y), e.x);
  // log2 p with the hardware log (absolute error ~1e-7)
  const float rp = r * (1.0f / kPiF);
  const float l2p = __builtin_amdgcn_logf(neg ? rp : 1.f - rp);
  return fmaxf(fmaf(TKln2, l2p, g), kLnUFloorF);
}

// sum of squares of a lane's 32 bf16 values with packed bf16 dot products
__device__ __forceinline__ float sumsq(const Frag<BF16>& f) {
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const Bf16Pairs pr = __builtin_bit_cast(Bf16Pairs, f.v[k]);
#pragma unroll
    for (int j = 0; j < 4; ++j) s = __builtin_amdgcn_fdot2_f32_bf16(pr.p[j], pr.p[j], s, false);
  }
  return s;
}

// DPP lane permutations inside rows of 16 lanes
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// max / sum over the 16 lanes of a row: pairs, quads, half-row mirror, row
// mirror; every lane ends with the same value (each step adds disjoint sets)
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp<0xB1>(v));    // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp<0x4E>(v));    // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp<0x141>(v));   // row_half_mirror
  return fmaxf(v, dpp<0x140>(v));  // row_mirror
}
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  return v + dpp<0x140>(v);
}

}  // namespace

// LDS of the attention role (the other roles of the launch reuse the same bytes).
struct AttendLds {
  float4 tab4[kLnuTable];                                    // interval quadratics of g
  int ring_idx[kWaves][kRingN];
  uint16_t ring_hm[kWaves][kRingN];
  __attribute__((aligned(16))) uint16_t vt[kWaves][kTile * kVRow];
  __attribute__((aligned(16))) uint16_t pt[kWaves][2][kTile * 16];
  float ep_m[kWaves][16], ep_l[kWaves][16];
  int flag;
};
constexpr size_t kFusedLdsBytes = cmax(sizeof(AttendLds), kRolesLdsBytes);

// The attention role: partial slot s (a context split) of unit u.  GW = number of 64-lane mask words per
// head and 512-key block that a lane holds: the G heads' 16 words per block
// are spread over GW loads.
template <int GW>
__device__ __forceinline__ void attend_bf16_role(const FusedParams& p, int s, int u, unsigned char* smem) {
  LSH_PCHECK(p, u < p.B * p.Hkv && s < p.nsplit, kChkSlot);
  AttendLds& A = *reinterpret_cast<AttendLds*>(smem);
  LSH_STAMP(p, 0);
  const uint16_t* __restrict__ q = static_cast<const uint16_t*>(p.q);
  const uint16_t* __restrict__ keys = static_cast<const uint16_t*>(p.keys);
  const uint16_t* __restrict__ values = static_cast<const uint16_t*>(p.values);
  const uint32_t* bitmask = p.bitmask;
  const int Hq = p.Hq, Hkv = p.Hkv, N = p.N, P = p.P, K = p.K, Tth = p.T;
  const float scale = p.scale;
  const int split_len = p.split_len;
  const int npart = p.npart;
  float4* tab4 = A.tab4;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, sl = lane & 15;
  const int G = p.G;
  const int b = u / Hkv, g = u % Hkv;
  const int bh0 = b * Hq + g * G;
  const int Nw = (N + 31) >> 5;
  const uint16_t* kb = keys + static_cast<size_t>(u) * P * kHeadDim;
  const uint16_t* vb = values + static_cast<size_t>(u) * P * kHeadDim;
  const bool k0 = (K == 0);
  const bool nolnu = k0;
  // this sequence's keys and exact set
  const int Nb = seq_len_of(p.seq_lens, b, N);
  int exact_head, exact_tail;
  exact_range(p.n_sink, p.n_window, Nb, exact_head, exact_tail);
  const uint16_t gmask = static_cast<uint16_t>((1u << G) - 1u);
  const float TKln2 = static_cast<float>(Tth * K) * 0.69314718055994531f;

  // q fragments (MFMA A operand): lane holds head sl, dims 32 k + 8 g4 + [0, 8)
  // of k-step k (the K fragments use the same order)
  Frag<BF16> Qf;
  Qf.load_interleaved(q + static_cast<size_t>(bh0 + (sl < G ? sl : 0)) * kHeadDim + g4 * 8, sl < G);
  float qss = sumsq(Qf);
  qss += __shfl_xor(qss, 16);
  qss += __shfl_xor(qss, 32);
  // reciprocal norms of this lane's output heads 4 g4 + i (lane h < 16 holds
  // head h); a zero norm gives 0, so the cosine is 0
  float rq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float x = __shfl(qss, 4 * g4 + i);
    rq[i] = x > 0.f ? __builtin_amdgcn_rsqf(x) : 0.f;
  }

  // the ln-u table's samples, in flight during the wait for the selection
  LnuFetch lf;
  lnu_fetch(p, nolnu, lf);

  // this wave's range: its quarter of the context split's keys
  const int sb = s * split_len;
  const int se = min(Nb, sb + split_len);
  const int wq = split_len / kWaves;
  const int wb = min(se, sb + wave * wq), we = min(se, sb + (wave + 1) * wq);

  int* ridx = A.ring_idx[wave];
  uint16_t* rhm = A.ring_hm[wave];
  uint16_t* V = A.vt[wave];
  uint16_t* Phi = A.pt[wave][0];
  uint16_t* Plo = A.pt[wave][1];

  // the selection of the split's key chunks must be complete (count
  // workgroups of every query head of the group); a wait that does not end
  // leaves a NaN partial
  bool ok = true;
  if (sb < se) {
    const int j0 = sb >> p.stride_log2, j1 = (se - 1) >> p.stride_log2;
    ok = wait_counters(p.ready + u * p.nJ + j0, j1 - j0 + 1, G, &A.flag);
  }

  LSH_STAMP(p, 1);
  // ---- selection masks: the 16 words (512 keys) of every head of the group
  // for one block; word w of head h sits in lane (h % 4) * 16 + w of load h / 4
  uint32_t mw[GW] = {}, mw_next[GW] = {};
  auto load_block = [&](int blk0, uint32_t (&dst)[GW]) {
#pragma unroll
    for (int k = 0; k < GW; ++k) {
      const int hh = 4 * k + g4;
      const int wi = (blk0 >> 5) + sl;
      dst[k] = (hh < G && blk0 < we && wi < Nw) ? ld_agent(bitmask + static_cast<size_t>(bh0 + hh) * Nw + wi) : 0u;
    }
  };
  int blk = wb;                        // next window to compact
  int blk_loaded = wb;                 // block start of mw
  load_block(wb, mw);
  load_block(wb + kBlock, mw_next);

  int rhead = 0, rcnt = 0;
  // compact windows of 64 keys until a full tile is queued or the range ends
  auto fill = [&]() {
    while (rcnt < kTile && blk < we) {
      if (blk >= blk_loaded + kBlock) {
        blk_loaded += kBlock;
#pragma unroll
        for (int k = 0; k < GW; ++k) mw[k] = mw_next[k];
        load_block(blk_loaded + kBlock, mw_next);
      }
      const int wsel = ((blk - blk_loaded) >> 5) + (lane >> 5);   // word of this lane's key in the block
      int hm = 0;
#pragma unroll
      for (int k = 0; k < GW; ++k)
#pragma unroll
        for (int hq = 0; hq < 4; ++hq) {
          const uint32_t w = __shfl(mw[k], hq * 16 + wsel);
          hm |= static_cast<int>((w >> (lane & 31)) & 1u) << (4 * k + hq);
        }
      const int n = blk + lane;
      // a key of the exact set (never in the bitmask): every head, ln u = 0,
      // marked in bit 31 of its ring entry
      const bool ex = n < exact_head || n >= Nb - exact_tail;
      hm = ex ? static_cast<int>(gmask) : hm;
      const bool any = n < we && hm != 0;
      const uint64_t bal = ballot(any);
      if (any) {
        const int e = (rhead + rcnt + mbcnt(bal)) & (kRingN - 1);
        ridx[e] = ex ? (n | kExactKey) : n;
        rhm[e] = static_cast<uint16_t>(hm);
      }
      rcnt += __builtin_popcountll(bal);
      blk += 64;
    }
    __builtin_amdgcn_wave_barrier();
  };

  // ---- tile loads: K rows as two 16-key MFMA B fragments (lane = key sl of
  // the group, dims 32 k + 8 g4 + [0, 8) for k-step k); V rows as 16-byte pieces (lane = piece sl of
  // rows g4 + 4 j)
  Frag<BF16> Kf[2];
  u32x4_t vr[8];
  int hmk[2];
  bool exk[2];
  auto issue = [&](int nt) {
#pragma unroll
    for (int gp = 0; gp < 2; ++gp) {
      const int slot = 16 * gp + sl;
      const int e = (rhead + (slot < nt ? slot : 0)) & (kRingN - 1);
      const int r = ridx[e];
      hmk[gp] = slot < nt ? static_cast<int>(rhm[e]) : 0;
      exk[gp] = r < 0;                               // kExactKey: an exact-set key
      Kf[gp].load_interleaved_nt(kb + static_cast<size_t>(r & ~kExactKey) * kHeadDim + g4 * 8);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = g4 + 4 * j;
      const int e = (rhead + (row < nt ? row : 0)) & (kRingN - 1);
      vr[j] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(vb + static_cast<size_t>(ridx[e] & ~kExactKey) * kHeadDim + sl * 8));
    }
  };

  float m_run[4], l_run[4];
  floatx4_t O[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m_run[i] = -INFINITY;
    l_run[i] = 0.f;
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) O[t] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  // the first tile's loads go out before waiting for the ln u table
  fill();
  int nt = min(kTile, rcnt);
  if (nt > 0) issue(nt);
  lnu_store(lf, nolnu, tab4);
  __syncthreads();   // ln u table in LDS
  LSH_STAMP(p, 2);
  while (nt > 0) {
    // V of this tile into LDS (row-major, padded rows)
#pragma unroll
    for (int j = 0; j < 8; ++j) *reinterpret_cast<u32x4_t*>(&V[(g4 + 4 * j) * kVRow + sl * 8]) = vr[j];
    // S = q.k for keys sl (group 0) and 16 + sl (group 1); rows = heads 4 g4 + i
    floatx4_t S0 = {0.f, 0.f, 0.f, 0.f}, S1 = {0.f, 0.f, 0.f, 0.f};
    S0 = Qf.mma(Kf[0], S0);
    S1 = Qf.mma(Kf[1], S1);
    float ks0 = sumsq(Kf[0]), ks1 = sumsq(Kf[1]);
    ks0 += __shfl_xor(ks0, 16);
    ks0 += __shfl_xor(ks0, 32);
    ks1 += __shfl_xor(ks1, 16);
    ks1 += __shfl_xor(ks1, 32);
    const float rk0 = ks0 > 0.f ? __builtin_amdgcn_rsqf(ks0) : 0.f;
    const float rk1 = ks1 > 0.f ? __builtin_amdgcn_rsqf(ks1) : 0.f;
    const int hm0 = hmk[0], hm1 = hmk[1];
    const bool ex0 = exk[0], ex1 = exk[1];

    // retire the tile from the ring, queue the next one and start its loads
    rhead = (rhead + nt) & (kRingN - 1);
    rcnt -= nt;
    fill();
    const int nnext = min(kTile, rcnt);
    if (nnext > 0) issue(nnext);

    // logits s q.k - ln u for this lane's 8 (head, key) pairs, computed
    // without branches so the eight independent chains interleave; pairs whose
    // key the head did not select are masked to -inf afterwards
    float lg[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x0 = S0[i], x1 = S1[i];
      const float u0 = nolnu || ex0 ? 0.f : lnu_of_cos(x0 * rq[i] * rk0, tab4, TKln2);
      const float u1 = nolnu || ex1 ? 0.f : lnu_of_cos(x1 * rq[i] * rk1, tab4, TKln2);
      const int hh = 4 * g4 + i;
      const bool ok = hh < G;
      lg[0][i] = (ok && ((hm0 >> hh) & 1)) ? fmaf(scale, x0, -u0) : -INFINITY;
      lg[1][i] = (ok && ((hm1 >> hh) & 1)) ? fmaf(scale, x1, -u1) : -INFINITY;
    }
    // online softmax per head, P = exp(logit - m) as bf16 hi + lo
    bf16x2_t phi[2][2], plo[2][2];
    bool rescale = false;
    float alpha[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lg0 = lg[0][i], lg1 = lg[1][i];
      const float mt = row_max16(fmaxf(lg0, lg1));
      const float mnew = fmaxf(m_run[i], mt);
      alpha[i] = (mnew == -INFINITY) ? 1.f : __expf(m_run[i] - mnew);
      rescale |= alpha[i] != 1.f;
      const float p0 = (lg0 == -INFINITY) ? 0.f : __expf(lg0 - mnew);
      const float p1 = (lg1 == -INFINITY) ? 0.f : __expf(lg1 - mnew);
      l_run[i] = fmaf(l_run[i], alpha[i], row_sum16(p0 + p1));
      m_run[i] = mnew;
      const __bf16 h0 = static_cast<__bf16>(p0), h1 = static_cast<__bf16>(p1);
      phi[0][i >> 1][i & 1] = h0;
      phi[1][i >> 1][i & 1] = h1;
      plo[0][i >> 1][i & 1] = static_cast<__bf16>(p0 - static_cast<float>(h0));
      plo[1][i >> 1][i & 1] = static_cast<__bf16>(p1 - static_cast<float>(h1));
    }
    if (ballot(rescale)) {
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) O[t][i] *= alpha[i];
    }
    // P tiles in LDS as [key][16 heads]: this lane's 4 heads of keys sl, 16 + sl
#pragma unroll
    for (int gp = 0; gp < 2; ++gp) {
      const int key = 16 * gp + sl;
      *reinterpret_cast<uint2*>(&Phi[key * 16 + 4 * g4]) =
          make_uint2(__builtin_bit_cast(uint32_t, phi[gp][0]), __builtin_bit_cast(uint32_t, phi[gp][1]));
      *reinterpret_cast<uint2*>(&Plo[key * 16 + 4 * g4]) =
          make_uint2(__builtin_bit_cast(uint32_t, plo[gp][0]), __builtin_bit_cast(uint32_t, plo[gp][1]));
    }
    __builtin_amdgcn_wave_barrier();
    // O[head][dim] += P[head][key] V[key][dim]: A = P (keys 8 g4 .. 8 g4 + 7 of
    // head sl), B = V (same keys, dim 16 t + sl)
    const int r0 = 8 * g4 + (sl >> 2), c0 = 4 * (sl & 3);
    const bf16x8_t Ahi = join8(ds_read_tr16(&Phi[r0 * 16 + c0]), ds_read_tr16(&Phi[(r0 + 4) * 16 + c0]));
    const bf16x8_t Alo = join8(ds_read_tr16(&Plo[r0 * 16 + c0]), ds_read_tr16(&Plo[(r0 + 4) * 16 + c0]));
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const bf16x8_t Bv = join8(ds_read_tr16(&V[r0 * kVRow + 16 * t + c0]),
                                ds_read_tr16(&V[(r0 + 4) * kVRow + 16 * t + c0]));
      O[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ahi, Bv, O[t], 0, 0, 0);
      O[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Alo, Bv, O[t], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
    nt = nnext;
  }

  LSH_STAMP(p, 3);
  // ---- merge the four waves' states per head; O[t][i] is head 4 g4 + i, dim 16 t + sl
  __syncthreads();
  float* wacc = reinterpret_cast<float*>(&A.vt[0][0]);   // [kWaves][16][128]
  if (sl == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      A.ep_m[wave][4 * g4 + i] = m_run[i];
      A.ep_l[wave][4 * g4 + i] = l_run[i];
    }
  }
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) wacc[(wave * 16 + 4 * g4 + i) * kHeadDim + 16 * t + sl] = O[t][i];
  __syncthreads();
  // G <= 4 GW heads: at most 2 GW elements of the G x 128 states per thread.
  // Without branches, so that every LDS read is in flight at once: a wave
  // that took no key of a head has max -inf and weight 0 (its state is 0)
#pragma unroll
  for (int k = 0; k < 2 * GW; ++k) {
    const int e = tid + 256 * k;
    const bool live = e < G * kHeadDim;
    const int hh = live ? e / kHeadDim : 0, d = e % kHeadDim;
    float mw[kWaves];
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      mw[w] = A.ep_m[w][hh];
      M = fmaxf(M, mw[w]);
    }
    float Acc = 0.f, Lm = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = mw[w] == -INFINITY ? 0.f : __expf(mw[w] - M);   // all -inf when M is
      Acc = fmaf(wacc[(w * 16 + hh) * kHeadDim + d], f, Acc);
      Lm = fmaf(A.ep_l[w][hh], f, Lm);
    }
    if (!ok) {   // a wait gave up: poison this partial
      Acc = __builtin_nanf("");
      M = 0.f;
      Lm = 1.f;
    }
    if (live) {
      float* dst = p.partials + (static_cast<size_t>(bh0 + hh) * npart + s) * kPartialStride;
      st_agent(dst + d, Acc);
      if (d == 0) {
        st_agent(dst + kHeadDim, M);
        st_agent(dst + kHeadDim + 1, Lm);
      }
    }
  }
}

// The one-launch decode for bf16 K/V: count and attend workgroups, unit by
// unit (decode_role).
template <int GW>
__global__ __launch_bounds__(kFusedThreads, 2) void decode_bf16_kernel(FusedParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kFusedLdsBytes];
  const DecodeRole r = decode_role(p, blockIdx.x);
  if (r.count) {
    if (p.count_heads > 1) count_role_heads(p, r.J, r.bh, smem);
    else count_role(p, r.J, r.bh, smem);
    return;
  }
  attend_bf16_role<GW>(p, r.slot, r.u, smem);
  __syncthreads();
  LSH_STAMP(p, 4);
  finish_slot(p, r.u, r.slot, smem);
}

hipError_t launch_decode_bf16(const FusedParams& p, int kid, hipStream_t stream) {
  const dim3 grid(p.n_count_wg + p.n_attend_wg);
  if (p.G <= 4) return launch(kid, decode_bf16_kernel<1>, grid, dim3(kFusedThreads), 0, stream, p);
  if (p.G <= 8) return launch(kid, decode_bf16_kernel<2>, grid, dim3(kFusedThreads), 0, stream, p);
  return launch(kid, decode_bf16_kernel<4>, grid, dim3(kFusedThreads), 0, stream, p);
}

}  // namespace lsh
