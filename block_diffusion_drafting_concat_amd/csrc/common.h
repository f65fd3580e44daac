// Shared device helpers for the DFlash gfx950 kernels: storage types, bf16 rounding, MFMA
// fragments and wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dflash {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_bits;  // storage of one bfloat16 value

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(uint32_t(h) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// Storage-type traits: T is float (fp32 drafters) or uint16_t (bf16 drafters).
template <typename T> struct Storage;
template <> struct Storage<float> {
  static constexpr int kPerVec = 4;  // elements per 16-byte vector
  __device__ static float load(const float *p, size_t i) { return p[i]; }
  __device__ static void store(float *p, size_t i, float v) { p[i] = v; }
  __device__ static float round(float v) { return v; }
};
template <> struct Storage<uint16_t> {
  static constexpr int kPerVec = 8;
  __device__ static float load(const uint16_t *p, size_t i) { return bf16_to_f32(p[i]); }
  __device__ static void store(uint16_t *p, size_t i, float v) { p[i] = f32_to_bf16(v); }
  __device__ static float round(float v) { return bf16_to_f32(f32_to_bf16(v)); }
};

// 16 bytes of a row, as loaded by one lane for one MFMA K-step.
struct Vec16 {
  uint4 u;
};

__device__ __forceinline__ Vec16 load_vec16(const void *p) {
  Vec16 v;
  v.u = *reinterpret_cast<const uint4 *>(p);
  return v;
}
__device__ __forceinline__ Vec16 zero_vec16() {
  Vec16 v;
  v.u = make_uint4(0, 0, 0, 0);
  return v;
}

// acc += A * B for one 16x16 output tile, with each lane supplying 16 bytes of A (row
// lane%16) and B (column lane%16) covering the K values of lane group lane/16.
//  bf16: one v_mfma_f32_16x16x32_bf16 (8 K values per lane).
//  fp32: four v_mfma_f32_16x16x4f32 (4 K values per lane, one per instruction).
// Any assignment of K indices to (lane group, element) is valid as long as A and B agree.
template <typename T> __device__ __forceinline__ void mma16(f32x4_t &acc, const Vec16 &a, const Vec16 &b);

template <> __device__ __forceinline__ void mma16<uint16_t>(f32x4_t &acc, const Vec16 &a, const Vec16 &b) {
  bf16x8_t av, bv;
  __builtin_memcpy(&av, &a.u, 16);
  __builtin_memcpy(&bv, &b.u, 16);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
}
template <> __device__ __forceinline__ void mma16<float>(f32x4_t &acc, const Vec16 &a, const Vec16 &b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.u.x), __uint_as_float(b.u.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.u.y), __uint_as_float(b.u.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.u.z), __uint_as_float(b.u.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.u.w), __uint_as_float(b.u.w), acc, 0, 0, 0);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Sum over a block of blockDim.x threads (a multiple of 64, at most 1024).
__device__ __forceinline__ float block_sum(float v, float *scratch /* >= 16 floats */) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) scratch[wave] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += scratch[i];
  return t;
}

// (value, index) argmax step: larger value wins, the lower index wins ties.
__device__ __forceinline__ void argmax_merge(float &v, int &i, float ov, int oi) {
  if (ov > v || (ov == v && oi < i)) {
    v = ov;
    i = oi;
  }
}

}  // namespace dflash
