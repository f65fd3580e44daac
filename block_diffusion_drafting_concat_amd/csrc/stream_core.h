// Device pieces of a weight-streaming kernel that stages a block's activation rows in LDS and
// feeds v_mfma_f32_16x16x32_bf16 straight from 16-byte weight loads (the persistent layer-stack
// kernel): device-scope accesses for data handed between work-groups, the weight register
// buffers and their loads, the MFMA step of one job, LDS hand-offs between the waves of a
// work-group, and the in-order sum of split-K partial tiles.
#pragma once

#include "common.h"

namespace dflash {
namespace wave {

constexpr int kTN = 128;  // output columns of a tile
constexpr unsigned long long kWaitTicks = 100000000ull;  // 1 s of the 100 MHz real-time clock

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) const u32x4_t global_u32x4_t;

// ---- agent-coherent accesses (relaxed atomics at agent scope)
__device__ __forceinline__ uint64_t ldc64(const void *p) {
  return __hip_atomic_load(reinterpret_cast<const uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stc64(void *p, uint64_t v) {
  __hip_atomic_store(reinterpret_cast<uint64_t *>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint4 ldc128(const void *p) {
  const uint64_t a = ldc64(p), b = ldc64(static_cast<const char *>(p) + 8);
  return make_uint4((uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32));
}
__device__ __forceinline__ void stc128(void *p, uint4 v) {
  stc64(p, v.x | ((uint64_t)v.y << 32));
  stc64(static_cast<char *>(p) + 8, v.z | ((uint64_t)v.w << 32));
}
__device__ __forceinline__ float ldcf(const float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stcf(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned ldcu(const unsigned *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stcu(unsigned *p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Workspace data handed between work-groups goes through a buffer resource over the workspace:
// 128-bit loads and stores with the same cache policy (sc1) as the agent-scope accesses above, a
// 32-bit offset per access instead of a 64-bit address.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
constexpr int kSC1 = 16;  // buffer cache-policy bits: sc1
struct Ws {
  __amdgpu_buffer_rsrc_t r;
  const char *base;
  __device__ int off(const void *p) const { return (int)(static_cast<const char *>(p) - base); }
};
__device__ __forceinline__ uint4 wld128(const Ws &ws, const void *p) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(ws.r, ws.off(p), 0, kSC1);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// the same with the offset split into a per-lane part (VGPR) and a wave-uniform part (SGPR)
__device__ __forceinline__ uint4 wld128s(const Ws &ws, int voff, int soff) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(ws.r, voff, __builtin_amdgcn_readfirstlane(soff), kSC1);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint64_t wld64(const Ws &ws, const void *p) {
  const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(ws.r, ws.off(p), 0, kSC1);
  return (uint64_t)v.x | ((uint64_t)v.y << 32);
}
__device__ __forceinline__ float wldf(const Ws &ws, const float *p) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ws.r, ws.off(p), 0, kSC1));
}
__device__ __forceinline__ void wst128(const Ws &ws, void *p, uint4 v) {
  const u32x4_t t = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(t, ws.r, ws.off(p), 0, kSC1);
}
__device__ __forceinline__ void wst64(const Ws &ws, void *p, uint64_t v) {
  const u32x2_t t = {(unsigned)v, (unsigned)(v >> 32)};
  __builtin_amdgcn_raw_buffer_store_b64(t, ws.r, ws.off(p), 0, kSC1);
}
__device__ __forceinline__ void wstf(const Ws &ws, float *p, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), ws.r, ws.off(p), 0, kSC1);
}

__device__ __forceinline__ float f2(uint64_t v, int i) { return __uint_as_float((uint32_t)(v >> (32 * i))); }
__device__ __forceinline__ uint64_t pack2(float a, float b) {
  return (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
}

// ---- LDS hand-offs between the waves of a work-group (workgroup-scope release / acquire)
typedef __attribute__((address_space(3))) volatile int lds_vint;
__device__ __forceinline__ int lds_load(const int *p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// One increment per wave (lane 0), ordered after the wave's earlier LDS accesses.
__device__ __forceinline__ void lds_add(int *p, int v) {
  if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_add(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_set(int *p, int v) {
  if ((threadIdx.x & 63) == 0) __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

struct WBuf {
  Vec16 v[16];  // [column tile ct][K step]
};

// 16 bytes of global memory. The weight pointers come from the job list in LDS, which hides
// their address space from the compiler; a generic (flat) load would also count on the LDS
// counter, so every LDS wait would wait for the weight loads in flight as well. A pointer made
// from the integer address is a global one (a cast of the generic pointer stays generic).
__device__ __forceinline__ Vec16 load_global16(const void *p) {
  const u32x4_t t = *(global_u32x4_t *)(uintptr_t)p;
  Vec16 v;
  __builtin_memcpy(&v.u, &t, 16);
  return v;
}

// Every GEMM job is eight K steps of 32 columns: one matrix with a 256-column chunk, or gate and
// up with a 128-column chunk each (steps 0-3 gate, 4-7 up). Steps 0-3 accumulate into acc[0],
// steps 4-7 into acc[1], whatever the job: no branch picks registers, and for one matrix the two
// halves are added at the flush.
//
// Weight loads of one GEMM job for compute wave cw into b (16 loads of 16 B per lane): the
// 128 weight rows of the output tile start at w0 (gate|up: w0 gate, w1 up), each K long, and
// the job's chunk is K columns [kc * kr, kc * kr + kr).
__device__ __forceinline__ void issue_w(const uint16_t *w0, const uint16_t *w1, int K, int kc, int kr, bool dual,
                                        WBuf &b, int cw, int lane) {
  const int k0 = kc * kr;
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const size_t row = (size_t)(cw * 32 + ct * 16 + (lane & 15)) * K + k0 + (lane >> 4) * 8;
#pragma unroll
    for (int sp = 0; sp < 8; ++sp) {
      const bool up = dual && sp >= 4;
      const int step = dual ? (sp & 3) : sp;
      b.v[ct * 8 + sp] = load_global16((up ? w1 : w0) + row + step * 32);
    }
  }
}

// MFMAs of one GEMM job: activations from the LDS slot `sa` (16 rows of arow bytes, 32 bytes
// [8 bf16 hi][8 bf16 lo] per 8 columns), weights from b
__device__ __forceinline__ void mma_job(bool dual, int arow, const WBuf &b, const unsigned char *sa,
                                        f32x4_t (&acc)[2][2], int lane) {
#pragma unroll
  for (int sp = 0; sp < 8; ++sp) {
    const int step = dual ? (sp & 3) : sp;
    const unsigned char *pa = sa + (lane & 15) * arow + (step * 4 + (lane >> 4)) * 32;
    Vec16 hi, lo;
    hi.u = *reinterpret_cast<const uint4 *>(pa);
    lo.u = *reinterpret_cast<const uint4 *>(pa + 16);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      mma16<uint16_t>(acc[sp >> 2][ct], hi, b.v[ct * 8 + sp]);
      mma16<uint16_t>(acc[sp >> 2][ct], lo, b.v[ct * 8 + sp]);
    }
  }
}

// Sum of the count partial tiles at part, in contributor order, into out (LDS): NB contributors
// per round trip; lane + 64 e is the lane's e-th float4 of the tile.
template <int NACC>
__device__ __forceinline__ void reduce_partials(const Ws &ws, const float *part, int count, float *out, int lane) {
  constexpr int E = 8 * NACC, NB = 24 / E > 0 ? 24 / E : 1;
  const int voff = ws.off(part) + lane * 16;  // bytes
  for (int q0 = 0; q0 < count; q0 += NB) {
    uint4 v[NB][E];
#pragma unroll
    for (int qq = 0; qq < NB; ++qq)
#pragma unroll
      for (int e = 0; e < E; ++e)
        v[qq][e] = wld128s(ws, voff, (min(q0 + qq, count - 1) * NACC * 16 * kTN + e * 64 * 4) * 4);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float4 *o = reinterpret_cast<float4 *>(out + (e * 64 + lane) * 4);
      float4 sum = q0 == 0 ? make_float4(0.f, 0.f, 0.f, 0.f) : *o;
#pragma unroll
      for (int qq = 0; qq < NB; ++qq) {
        if (q0 + qq < count) {
          sum.x += __uint_as_float(v[qq][e].x);
          sum.y += __uint_as_float(v[qq][e].y);
          sum.z += __uint_as_float(v[qq][e].z);
          sum.w += __uint_as_float(v[qq][e].w);
        }
      }
      *o = sum;
    }
  }
}


}  // namespace wave
}  // namespace dflash
