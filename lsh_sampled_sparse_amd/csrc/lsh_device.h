// Device-side helpers shared by the HIP kernels of the LSH attention library.
// gfx950 only: wave64, MFMA, 160 KB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lsh {

constexpr int kWave = 64;
constexpr int kHeadDim = 128;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float floatx4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

// Storage tags: bf16 is kept as raw uint16 bits.
struct BF16 {
  using storage = uint16_t;
  static constexpr int bytes = 2;
};
struct F32 {
  using storage = float;
  static constexpr int bytes = 4;
};

// -x of a stored element (bf16: flip the sign bit).
__device__ __forceinline__ uint16_t negate(uint16_t h) { return static_cast<uint16_t>(h ^ 0x8000u); }
__device__ __forceinline__ float negate(float x) { return -x; }

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ int mbcnt(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Reductions over the 16 lanes that share (lane / 16).
__device__ __forceinline__ float row16_max(float v) {
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// ---------------------------------------------------------------------------
// MFMA fragments (16x16 tiles).  Every lane covers the 32 consecutive
// dims [32 * (lane / 16), +32) of one row (a key for the A operand, a
// projection column or a query head for the other operand); both operands use
// the same dim <-> k-slot map, so the MFMA sums over the 128 dims of the rows.
// ---------------------------------------------------------------------------
template <typename T>
struct Frag;

template <>
struct Frag<BF16> {
  bf16x8_t v[4];
  __device__ __forceinline__ void load(const uint16_t* p, bool valid) {
    const u32x4_t* q = reinterpret_cast<const u32x4_t*>(p);
    const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = __builtin_bit_cast(bf16x8_t, valid ? q[k] : zero);
  }
  // the four 16-byte pieces at p, p + 32, p + 64 and p + 96 (elements).  With
  // p = row + 8 * (lane >> 4) for both operands, k-step k sums dims
  // [32 k, 32 k + 32), and the four lanes that share a row read 64
  // contiguous bytes of it per step (half the cache lines of load()'s order)
  __device__ __forceinline__ void load_interleaved(const uint16_t* p, bool valid) {
    const u32x4_t* q = reinterpret_cast<const u32x4_t*>(p);
    const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = __builtin_bit_cast(bf16x8_t, valid ? q[4 * k] : zero);
  }
  // load_interleaved's pieces through non-temporal loads, for rows read once
  __device__ __forceinline__ void load_interleaved_nt(const uint16_t* p) {
    const u32x4_t* q = reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = __builtin_bit_cast(bf16x8_t, __builtin_nontemporal_load(q + 4 * k));
  }
  __device__ __forceinline__ floatx4_t mma(const Frag& b, floatx4_t acc) const {
#pragma unroll
    for (int k = 0; k < 4; ++k) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v[k], b.v[k], acc, 0, 0, 0);
    return acc;
  }
  // one of the four k-steps of mma()
  __device__ __forceinline__ void mma_step(int k, const Frag& b, floatx4_t& acc) const {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v[k], b.v[k], acc, 0, 0, 0);
  }
};

template <>
struct Frag<F32> {
  float v[32];
  __device__ __forceinline__ void load(const float* p, bool valid) {
    const floatx4_t* q = reinterpret_cast<const floatx4_t*>(p);
    const floatx4_t zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const floatx4_t x = valid ? q[k] : zero;
      v[4 * k + 0] = x[0]; v[4 * k + 1] = x[1]; v[4 * k + 2] = x[2]; v[4 * k + 3] = x[3];
    }
  }
  __device__ __forceinline__ floatx4_t mma(const Frag& b, floatx4_t acc) const {
#pragma unroll
    for (int k = 0; k < 32; ++k) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(v[k], b.v[k], acc, 0, 0, 0);
    return acc;
  }
  // one quarter (8 of the 32 k-steps) of mma()
  __device__ __forceinline__ void mma_step(int k, const Frag& b, floatx4_t& acc) const {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(v[8 * k + j], b.v[8 * k + j], acc, 0, 0, 0);
  }
};

}  // namespace lsh
