// Weight-streaming MFMA GEMM for the drafter's projections and the LM head.
//
// Every projection of the drafter is C = A W^T with a short activation A (the block's rows:
// 16 at batch 1) and a long weight W [N, K] that must be read once from HBM. The kernel is
// organised around streaming W at full HBM rate:
//  * a work-group owns 16*CW output columns and one K slice of the split-K grid (grid.y);
//    its CW*KW waves are CW column tiles x KW sub-slices of K;
//  * each wave streams its 16 W rows in 16-byte-per-lane loads that feed
//    v_mfma_f32_16x16x32_bf16 directly (B operand = 16 W rows x 64 contiguous bytes), double
//    buffered in registers; its first loads are issued before the activation staging so the
//    HBM stream starts at once;
//  * the activation slice is staged in LDS (in passes of at most kPassBytes), so A fragments
//    come from LDS and the vector-memory path carries only weights;
//  * the KW sub-slice tiles are summed through LDS in a fixed order. With one split the
//    epilogue is applied in place (fp32 store, residual add, fp32 SwiGLU, or the LM head's
//    (max, lowest index) per work-group); with several, fp32 partials [split][M][N] go to
//    the workspace and the consumer kernel sums them in split order. There are no float
//    atomics, so results are deterministic.
// Up to 64 activation rows are held as MT accumulator tiles; more rows use grid.z blocks.
#include "common.h"
#include "kernels.h"

namespace dflash {
namespace {

constexpr int kPassBytes = 60 << 10;  // LDS budget of one staged A pass (+ padding < 64 KiB)
constexpr int kGroup = 4;             // 16-byte K steps per register buffer

template <typename T>
__host__ __device__ constexpr int ch_of() {
  return 4 * Storage<T>::kPerVec;  // K elements per wave MFMA step
}

// kAF32: the activation A is fp32 while W is bf16. A is staged in LDS as two bf16 planes,
// hi = bf16(a) and lo = bf16(a - hi), and every K step issues two MFMAs (hi*W + lo*W), so
// the product sees A to ~16 significant bits instead of bf16's 8.
template <typename T, int MT, int CW, int KW, GemmEpi E, bool kMultiA, bool kAF32>
__global__ __launch_bounds__(CW *KW * 64) void gemm_kernel(GemmArgs g) {
  constexpr int NW = CW * KW;
  constexpr int KPV = Storage<T>::kPerVec;
  constexpr int CH = ch_of<T>();
  constexpr bool kDual = E == GemmEpi::kSwiGLU;
  constexpr int NACC = kDual ? 2 : 1;
  constexpr int U = kGroup;
  constexpr int NPL = kAF32 ? 2 : 1;  // A planes in LDS
  static_assert(!kAF32 || (KPV == 8 && !kMultiA), "fp32 activations pair with bf16 weights");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T *sa = reinterpret_cast<T *>(smem);
  float *red = reinterpret_cast<float *>(smem);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cw = wave % CW, kw = wave / CW;
  const int n0 = blockIdx.x * 16 * CW;
  const int ncol = n0 + cw * 16;
  const int m0 = blockIdx.z * 16 * MT;
  const int kb = blockIdx.y * g.kt;
  const int ke = min(g.K, kb + g.kt);
  const int kp = g.kp;      // K per staged pass (multiple of KW * CH)
  const int as = kp + KPV;  // LDS row stride of the A pass (16-byte pad)
  const int kq = kp / KW;   // K per wave per pass
  const bool active = ncol < g.N;
  const int kg = (lane >> 4) * KPV;
  const int a_seglen = g.K / g.a_nseg;

  const T *brow[NACC];
  {
    int seg = 0, nbase = 0;
    if (!kDual)
      while (seg < g.b_nseg - 1 && ncol >= g.b_end[seg]) nbase = g.b_end[seg++];
    const int r = active ? ncol - nbase + (lane & 15) : 0;
    brow[0] = reinterpret_cast<const T *>(g.b[seg]) + (size_t)r * g.K + kg;
    if (kDual) brow[NACC - 1] = reinterpret_cast<const T *>(g.b[1]) + (size_t)r * g.K + kg;
  }

  f32x4_t acc[NACC][MT];
#pragma unroll
  for (int a = 0; a < NACC; ++a)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[a][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // The loads below are issued unconditionally (addresses clamped into the operand) so that
  // the compiler can count outstanding loads exactly: weight loads stay in flight across the
  // A staging and across each MFMA group (register double buffering).
  const int vrow = kp / KPV;  // 16-byte vectors per staged A row (per plane)
  constexpr int NA = (kPassBytes / (16 * NPL) + NW * 64 - 1) / (NW * 64);  // A vectors per thread, max
  T *sa_lo = sa + 16 * MT * as;  // lo plane (kAF32)
  for (int p0 = kb; p0 < ke; p0 += kp) {
    const int plen = min(kp, ke - p0);  // a multiple of CH
    const int q0 = kw * kq;
    const int q1 = min(plen, q0 + kq);
    const int nsteps = active && q1 > q0 ? (q1 - q0) / CH : 0;
    const int nfull = nsteps / U;
    const int total = 16 * MT * vrow;  // A vectors of this pass
    auto kclamp = [&](int st) { return p0 + min(q0 + st * CH, plen - CH); };
    auto load_group = [&](Vec16 (&b)[NACC][U], int gi) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int a = 0; a < NACC; ++a) b[a][u] = load_vec16(brow[a] + kclamp(gi * U + u));
    };
    auto compute = [&](const Vec16 (&b)[NACC][U], int st0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = q0 + (st0 + u) * CH;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const int ao = (t * 16 + (lane & 15)) * as + k + kg;
          Vec16 af;
          af.u = *reinterpret_cast<const uint4 *>(sa + ao);
#pragma unroll
          for (int a = 0; a < NACC; ++a) mma16<T>(acc[a][t], af, b[a][u]);
          if constexpr (kAF32) {
            af.u = *reinterpret_cast<const uint4 *>(sa_lo + ao);
#pragma unroll
            for (int a = 0; a < NACC; ++a) mma16<T>(acc[a][t], af, b[a][u]);
          }
        }
      }
    };

    // ---- A rows [m0, m0 + 16*MT) x K [p0, p0 + plen): loads first, then weights group 0
    Vec16 areg[NA][NPL];
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const int v = min((int)threadIdx.x + j * NW * 64, total - 1);
      const int r = v / vrow, cv = v % vrow;
      const int m = min(m0 + r, g.M - 1);
      const int k = p0 + min(cv * KPV, plen - KPV);
      if constexpr (kAF32) {  // 8 fp32 values = two 16-byte loads
        const float *ap = reinterpret_cast<const float *>(g.a[0]) + (size_t)m * g.lda + k;
        areg[j][0] = load_vec16(ap);
        areg[j][NPL - 1] = load_vec16(ap + 4);
      } else {
        const T *ap;
        if (kMultiA) {
          const int s = k / a_seglen;
          ap = reinterpret_cast<const T *>(g.a[s]) + (k - s * a_seglen);
        } else {
          ap = reinterpret_cast<const T *>(g.a[0]) + k;
        }
        areg[j][0] = load_vec16(ap + (size_t)m * g.lda);
      }
    }
    Vec16 b0[NACC][U], b1[NACC][U];
    load_group(b0, 0);
    __syncthreads();  // the previous pass has finished reading LDS
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const int v = (int)threadIdx.x + j * NW * 64;
      if (v < total) {
        const int r = v / vrow, cv = v % vrow;
        const bool ok = m0 + r < g.M && cv * KPV < plen;
        if constexpr (kAF32) {
          float f[8];
          __builtin_memcpy(f, &areg[j][0].u, 16);
          __builtin_memcpy(f + 4, &areg[j][NPL - 1].u, 16);
          uint16_t hi[8], lo[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = ok ? f[e] : 0.f;
            hi[e] = f32_to_bf16(x);
            lo[e] = f32_to_bf16(x - bf16_to_f32(hi[e]));
          }
          __builtin_memcpy(sa + r * as + cv * KPV, hi, 16);
          __builtin_memcpy(sa_lo + r * as + cv * KPV, lo, 16);
        } else {
          *reinterpret_cast<uint4 *>(sa + r * as + cv * KPV) = ok ? areg[j][0].u : make_uint4(0, 0, 0, 0);
        }
      }
    }
    __syncthreads();

    // ---- stream this wave's K range of the pass: ping-pong register buffers, so one group
    //      of weight loads is always in flight while the previous group feeds the MFMAs
    int gi = 0;
    for (; gi + 2 < nfull; gi += 2) {
      load_group(b1, gi + 1);
      compute(b0, gi * U);
      load_group(b0, gi + 2);
      compute(b1, (gi + 1) * U);
    }
    if (gi + 1 < nfull) {
      load_group(b1, gi + 1);
      compute(b0, gi * U);
      compute(b1, (gi + 1) * U);
    } else if (gi < nfull) {
      compute(b0, gi * U);
    }
    for (int st = nfull * U; st < nsteps; ++st) {
      const int k = q0 + st * CH;
      Vec16 bf[NACC];
#pragma unroll
      for (int a = 0; a < NACC; ++a) bf[a] = load_vec16(brow[a] + p0 + k);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int ao = (t * 16 + (lane & 15)) * as + k + kg;
        Vec16 af;
        af.u = *reinterpret_cast<const uint4 *>(sa + ao);
#pragma unroll
        for (int a = 0; a < NACC; ++a) mma16<T>(acc[a][t], af, bf[a]);
        if constexpr (kAF32) {
          af.u = *reinterpret_cast<const uint4 *>(sa_lo + ao);
#pragma unroll
          for (int a = 0; a < NACC; ++a) mma16<T>(acc[a][t], af, bf[a]);
        }
      }
    }
  }

  // ---- sum the KW sub-slice tiles in a fixed order, one row tile at a time. Tile layout:
  //      lane holds rows (lane/16)*4 + i, column lane%16, stored at [lane*4 + i].
  const bool direct = gridDim.y == 1;
  float *fin = red + NW * NACC * 256;  // argmax: final logits [MT][CW][256]
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    __syncthreads();
#pragma unroll
    for (int a = 0; a < NACC; ++a) *reinterpret_cast<f32x4_t *>(&red[(wave * NACC + a) * 256 + lane * 4]) = acc[a][t];
    __syncthreads();
    for (int e = threadIdx.x; e < CW * 256; e += NW * 64) {
      const int c = e / 256, li = e % 256;
      const int l = li >> 2, i = li & 3;
      const int m = m0 + t * 16 + (l >> 4) * 4 + i;
      const int col = n0 + c * 16 + (l & 15);
      float v[NACC];
#pragma unroll
      for (int a = 0; a < NACC; ++a) {
        float sum = 0.f;
#pragma unroll
        for (int q = 0; q < KW; ++q) sum += red[((q * CW + c) * NACC + a) * 256 + li];
        v[a] = sum;
      }
      if constexpr (E == GemmEpi::kArgmax) {
        fin[(t * CW + c) * 256 + li] = (m < g.M && col < g.N) ? v[0] : -INFINITY;
        continue;
      }
      if (m >= g.M || col >= g.N) continue;
      const size_t o = (size_t)m * g.N + col;
      if (!direct) {
        float *part = g.part + (size_t)blockIdx.y * g.M * g.N * NACC;
        if (kDual) {
          part[(size_t)m * 2 * g.N + col] = v[0];
          part[(size_t)m * 2 * g.N + g.N + col] = v[NACC - 1];
        } else {
          part[o] = v[0];
        }
      } else if constexpr (E == GemmEpi::kStore) {
        g.out[o] = v[0];
      } else if constexpr (E == GemmEpi::kResidAdd) {
        g.out[o] += v[0];
      } else if constexpr (E == GemmEpi::kSwiGLU) {
        const float silu = v[0] / (1.f + expf(-v[0]));
        g.act[o] = silu * v[NACC - 1];
      }
    }
  }
  if constexpr (E == GemmEpi::kArgmax) {
    // TPR threads per row scan the row's 16*CW columns, then a shuffle reduction
    constexpr int TPR0 = NW * 64 / (16 * MT);
    constexpr int TPR = TPR0 >= 32 ? 32 : TPR0 >= 16 ? 16 : TPR0 >= 8 ? 8 : TPR0 >= 4 ? 4 : TPR0 >= 2 ? 2 : 1;
    __syncthreads();
    if (threadIdx.x < 16 * MT * TPR) {
      const int r = threadIdx.x / TPR, sub = threadIdx.x % TPR;
      const int t = r / 16, rr = r % 16;
      float best = -INFINITY;
      int bi = 0x7fffffff;
      for (int j = sub; j < 16 * CW; j += TPR) {
        const int c = j / 16, jj = j % 16;
        argmax_merge(best, bi, fin[(t * CW + c) * 256 + ((rr / 4) * 16 + jj) * 4 + rr % 4], n0 + j);
      }
#pragma unroll
      for (int o = TPR / 2; o > 0; o >>= 1) {
        const float ov = __shfl_xor(best, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        argmax_merge(best, bi, ov, oi);
      }
      const int m = m0 + r;
      if (sub == 0 && m < g.M) {
        g.amax_val[(size_t)m * gridDim.x + blockIdx.x] = best;
        g.amax_idx[(size_t)m * gridDim.x + blockIdx.x] = bi;
      }
    }
  }
}

// Work-group shape (CW column tiles x KW K sub-slices) for a problem.
struct Shape {
  int cw, kw;
};
Shape pick_shape(int M, GemmEpi epi) {
  if (gemm_mt(M) > 1) return {2, 2};
  if (epi == GemmEpi::kArgmax) return {8, 1};
  return {4, 2};
}

template <typename T, int MT, int CW, int KW, GemmEpi E, bool kAF32>
size_t lds_bytes(const GemmArgs &g) {
  constexpr int KPV = Storage<T>::kPerVec;
  const size_t a = (size_t)16 * MT * (g.kp + KPV) * sizeof(T) * (kAF32 ? 2 : 1);
  const int nacc = E == GemmEpi::kSwiGLU ? 2 : 1;
  size_t r = (size_t)CW * KW * nacc * 256 * sizeof(float);
  if (E == GemmEpi::kArgmax) r += (size_t)CW * MT * 256 * sizeof(float);
  return a > r ? a : r;
}

template <typename T, int MT, int CW, int KW, GemmEpi E, bool kMultiA, bool kAF32>
hipError_t launch_k(const GemmArgs &g, int splits, hipStream_t s) {
  dim3 grid((g.N + 16 * CW - 1) / (16 * CW), splits, (g.M + 16 * MT - 1) / (16 * MT));
  gemm_kernel<T, MT, CW, KW, E, kMultiA, kAF32>
      <<<grid, CW * KW * 64, lds_bytes<T, MT, CW, KW, E, kAF32>(g), s>>>(g);
  return hipGetLastError();
}

template <typename T, GemmEpi E, bool kMultiA, bool kAF32>
hipError_t launch_t(const GemmArgs &g, int splits, hipStream_t s) {
  switch (gemm_mt(g.M)) {
    case 1:
      if constexpr (E == GemmEpi::kArgmax) return launch_k<T, 1, 8, 1, E, kMultiA, kAF32>(g, splits, s);
      else return launch_k<T, 1, 4, 2, E, kMultiA, kAF32>(g, splits, s);
    case 2: return launch_k<T, 2, 2, 2, E, kMultiA, kAF32>(g, splits, s);
    case 3: return launch_k<T, 3, 2, 2, E, kMultiA, kAF32>(g, splits, s);
    default: return launch_k<T, 4, 2, 2, E, kMultiA, kAF32>(g, splits, s);
  }
}

// fp32 drafters: A and W are fp32. bf16 drafters: W is bf16 and A is either bf16 (the
// auxiliary states of injection, possibly in several segments) or fp32 (every activation).
template <typename T, bool kAF32>
hipError_t launch_dt(const GemmArgs &g, GemmEpi epi, int splits, hipStream_t s) {
  switch (epi) {
    case GemmEpi::kStore:
      if (g.a_nseg > 1) return launch_t<T, GemmEpi::kStore, true, false>(g, splits, s);
      return launch_t<T, GemmEpi::kStore, false, kAF32>(g, splits, s);
    case GemmEpi::kResidAdd: return launch_t<T, GemmEpi::kResidAdd, false, kAF32>(g, splits, s);
    case GemmEpi::kSwiGLU: return launch_t<T, GemmEpi::kSwiGLU, false, kAF32>(g, splits, s);
    default: return launch_t<T, GemmEpi::kArgmax, false, kAF32>(g, splits, s);
  }
}

int kstep(int M, GemmEpi epi, bool bf16) {
  return pick_shape(M, epi).kw * (bf16 ? ch_of<uint16_t>() : ch_of<float>());
}

}  // namespace

int gemm_mt(int M) { return M <= 16 ? 1 : M <= 32 ? 2 : M <= 48 ? 3 : 4; }

int gemm_col_groups(int M, int N, GemmEpi epi) {
  const int cols = 16 * pick_shape(M, epi).cw;
  return (N + cols - 1) / cols;
}

int gemm_plan_splits(int M, int N, int K, bool bf16, GemmEpi epi) {
  if (epi == GemmEpi::kArgmax) return 1;
  const int step = kstep(M, epi, bf16);
  const long wgs = (long)gemm_col_groups(M, N, epi) * ((M + 16 * gemm_mt(M) - 1) / (16 * gemm_mt(M)));
  int s = 1;
  // Up to ~1024 work-groups (4 per CU) while each split keeps >= 256 K and divides K.
  while (wgs * s * 2 <= 1024 && K % (2 * s * step) == 0 && K / (2 * s) >= 256 && s < 64) s *= 2;
  return s;
}

hipError_t launch_gemm(const GemmArgs &g0, bool bf16, GemmEpi epi, int splits, hipStream_t s) {
  ProfScope prof(g0.tag ? g0.tag : "gemm", s);
  const int step = kstep(g0.M, epi, bf16);
  if ((epi != GemmEpi::kStore && g0.a_nseg > 1) || g0.N % 16 || g0.K % step || splits < 1 || g0.K % splits ||
      (g0.K / splits) % step || (epi == GemmEpi::kArgmax && splits != 1) ||
      (g0.a_nseg > 1 && (g0.K / g0.a_nseg) % (bf16 ? 8 : 4)))
    return hipErrorInvalidValue;
  GemmArgs g = g0;
  g.kt = g.K / splits;
  // K per staged pass: the split cut into equal passes that fit the LDS budget
  const int mt = gemm_mt(g.M);
  const bool af32 = bf16 && g.a_f32 && g.a_nseg == 1;
  const int esz = (bf16 && !af32) ? 2 : 4;  // LDS bytes per staged A element
  const int kp_max = kPassBytes / (16 * mt * esz) / step * step;
  const int npass = (g.kt + kp_max - 1) / kp_max;
  g.kp = ((g.kt + npass - 1) / npass + step - 1) / step * step;
  if (!bf16) return launch_dt<float, false>(g, epi, splits, s);
  return af32 ? launch_dt<uint16_t, true>(g, epi, splits, s) : launch_dt<uint16_t, false>(g, epi, splits, s);
}

}  // namespace dflash
