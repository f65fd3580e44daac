// Weight-streaming MFMA GEMM for the drafter's projections and the LM head.
//
// Every projection of the drafter is C = A W^T with a short activation A (the block's
// rows: 16 at batch 1) and a long weight W [N, K] read once from HBM. The kernel is
// organised around streaming W: each wave owns 16 output columns (16 rows of W) and walks
// its K slice in 16-byte-per-lane loads that feed v_mfma_f32_16x16x32_bf16 directly (B
// operand = 16 W rows x 64 contiguous bytes per instruction). Up to 64 activation rows are
// held as MT accumulator tiles; larger M is covered by grid.z blocks of 64 rows. The K
// range can be split over grid.y so that even narrow projections (N = 4096) put enough
// waves on the 256 CUs to keep HBM busy; the split partials are summed in fixed order by
// the consumer kernel (no float atomics, so results are deterministic).
#include "common.h"
#include "kernels.h"

namespace dflash {
namespace {

constexpr int kWaves = 4;   // waves per work-group; each owns 16 output columns
constexpr int kUnroll = 4;  // 16-byte K steps in flight per lane per iteration

template <typename T, int MT, bool kArgmax, bool kMultiA>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  constexpr int KPV = Storage<T>::kPerVec;  // K elements per lane per 16-byte load
  constexpr int CH = 4 * KPV;               // K elements per wave step
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = (blockIdx.x * kWaves + wave) * 16;
  const int m_base = blockIdx.z * (16 * MT);
  const int ks = (g.K / g.splits + CH - 1) / CH * CH;  // K per split, a multiple of CH
  const int kb = blockIdx.y * ks;
  const int ke = min(g.K, kb + ks);
  const bool active = n0 < g.N;

  f32x4_t acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (active) {
    // this wave's 16 W rows
    int seg = 0, nbase = 0;
    while (seg < g.b_nseg - 1 && n0 >= g.b_end[seg]) nbase = g.b_end[seg++];
    const T *brow = reinterpret_cast<const T *>(g.b[seg]) + (size_t)(n0 - nbase + (lane & 15)) * g.K;
    const int kg = (lane >> 4) * KPV;
    const int a_seglen = g.K / g.a_nseg;
    bool mvalid[MT];
    size_t aoff[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int m = m_base + t * 16 + (lane & 15);
      mvalid[t] = m < g.M;
      aoff[t] = (size_t)(mvalid[t] ? m : 0) * g.lda;
    }
    auto a_ptr = [&](int k) -> const T * {
      if (kMultiA) {
        const int s = k / a_seglen;
        return reinterpret_cast<const T *>(g.a[s]) + (k - s * a_seglen);
      }
      return reinterpret_cast<const T *>(g.a[0]) + k;
    };

    int k = kb;
    for (; k + CH * kUnroll <= ke; k += CH * kUnroll) {
      Vec16 bf[kUnroll];
      Vec16 af[MT][kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) bf[u] = load_vec16(brow + k + u * CH + kg);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const T *ap = a_ptr(k + u * CH + kg);
#pragma unroll
        for (int t = 0; t < MT; ++t) af[t][u] = mvalid[t] ? load_vec16(ap + aoff[t]) : zero_vec16();
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int t = 0; t < MT; ++t) mma16<T>(acc[t], af[t][u], bf[u]);
    }
    for (; k < ke; k += CH) {
      const Vec16 bfv = load_vec16(brow + k + kg);
      const T *ap = a_ptr(k + kg);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const Vec16 afv = mvalid[t] ? load_vec16(ap + aoff[t]) : zero_vec16();
        mma16<T>(acc[t], afv, bfv);
      }
    }
  }

  // Output tile layout: lane holds rows (lane/16)*4 + i, column lane%16.
  const int col = n0 + (lane & 15);
  if (!kArgmax) {
    if (!active) return;
    float *out = g.part + (size_t)blockIdx.y * g.M * g.N;
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m_base + t * 16 + (lane >> 4) * 4 + i;
        if (m < g.M) out[(size_t)m * g.N + col] = acc[t][i];
      }
    return;
  }

  // Argmax over this work-group's 64 columns for each of its rows.
  __shared__ float sv[kWaves][16 * MT];
  __shared__ int si[kWaves][16 * MT];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = active ? acc[t][i] : -INFINITY;
      int idx = active ? col : 0x7fffffff;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const float ov = __shfl_xor(v, o, 64);
        const int oi = __shfl_xor(idx, o, 64);
        argmax_merge(v, idx, ov, oi);
      }
      if ((lane & 15) == 0) {
        sv[wave][t * 16 + (lane >> 4) * 4 + i] = v;
        si[wave][t * 16 + (lane >> 4) * 4 + i] = idx;
      }
    }
  __syncthreads();
  if (threadIdx.x < 16 * MT) {
    const int r = threadIdx.x;
    float v = sv[0][r];
    int idx = si[0][r];
    for (int w = 1; w < kWaves; ++w) argmax_merge(v, idx, sv[w][r], si[w][r]);
    const int m = m_base + r;
    if (m < g.M) {
      g.amax_val[(size_t)blockIdx.x * g.M + m] = v;
      g.amax_idx[(size_t)blockIdx.x * g.M + m] = idx;
    }
  }
}

template <typename T, bool kArgmax, bool kMultiA>
hipError_t launch_t(const GemmArgs &g, hipStream_t s) {
  const int mt = g.M >= 64 ? 4 : (g.M + 15) / 16;
  dim3 grid((g.N + 16 * kWaves - 1) / (16 * kWaves), g.splits, (g.M + 63) / 64);
  if (g.M < 64) grid.z = 1;
  switch (mt) {
    case 1: gemm_kernel<T, 1, kArgmax, kMultiA><<<grid, 256, 0, s>>>(g); break;
    case 2: gemm_kernel<T, 2, kArgmax, kMultiA><<<grid, 256, 0, s>>>(g); break;
    case 3: gemm_kernel<T, 3, kArgmax, kMultiA><<<grid, 256, 0, s>>>(g); break;
    default: gemm_kernel<T, 4, kArgmax, kMultiA><<<grid, 256, 0, s>>>(g); break;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dt(const GemmArgs &g, GemmEpi epi, hipStream_t s) {
  const bool multi = g.a_nseg > 1;
  if (epi == GemmEpi::kArgmax) return multi ? launch_t<T, true, true>(g, s) : launch_t<T, true, false>(g, s);
  return multi ? launch_t<T, false, true>(g, s) : launch_t<T, false, false>(g, s);
}

}  // namespace

int gemm_plan_splits(int M, int N, int K, bool bf16) {
  const int ch = bf16 ? 32 : 16;
  const long waves = (long)((N + 15) / 16) * ((M + 63) / 64);
  int s = 1;
  // Aim for >= 2048 streaming waves (8 per CU) while keeping >= 512 K per split.
  while (waves * s < 2048 && K / (2 * s) >= 512 && (K / (2 * s)) % ch == 0 && s < 64) s *= 2;
  return s;
}

hipError_t launch_gemm(const GemmArgs &g, bool bf16, GemmEpi epi, hipStream_t s) {
  ProfScope prof(g.tag ? g.tag : "gemm", s);
  return bf16 ? launch_dt<uint16_t>(g, epi, s) : launch_dt<float>(g, epi, s);
}

}  // namespace dflash
