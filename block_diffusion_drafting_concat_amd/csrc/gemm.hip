// Weight-streaming MFMA GEMM with fused epilogues: every projection of the drafter.
//
// Every projection of the drafter is C = A W^T with a short activation A (the block's rows:
// 16 at batch 1) and a long weight W [N, K] that must be read once from HBM. The kernel is
// built around streaming W at full HBM rate:
//  * a work-group owns 16*CW output columns (a column group) and one K slice of the split-K
//    grid (grid.y); its CW*KW waves are CW column tiles x KW sub-slices of K;
//  * each wave streams its 16 W rows in 16-byte-per-lane loads that feed
//    v_mfma_f32_16x16x32_bf16 directly (B operand = 16 W rows x 64 contiguous bytes), in
//    ping-pong register buffers so a group of loads is always in flight;
//  * the activation slice is staged in LDS (in passes of at most kPassBytes), so the
//    vector-memory path carries only weights. fp32 activations are staged as an exact pair
//    of bf16 planes (hi, lo) and cost two MFMAs per step. RMSNorm can be applied while
//    staging ("norm on load"): row scales come from per-column-group sums of squares
//    written by the producer of the rows, the norm weight from its vector;
//  * the KW sub-slice tiles are summed through LDS in a fixed order into the work-group's
//    tile. With several K splits every split writes its tile to the workspace with
//    device-scope stores and the last work-group of the output tile to arrive (a device-scope
//    counter) sums all splits in split order. There are no float atomics, so results are
//    deterministic;
//  * the epilogue runs on the final tile: fp32 store, residual add, SwiGLU, the LM head's
//    per-group (max, lowest index), per-head q/k RMSNorm + RoPE of the block, or the
//    context K/V epilogue of injection (k_norm + RoPE + paged scatter). The last three
//    need a column group to be exactly one head.
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

// Per-head RMSNorm + rotate-half RoPE of one head vector held by one wave: lane i < D/2 owns
// the pair (i, i + D/2).
__device__ __forceinline__ void head_norm_rope(float &x1, float &x2, bool own, int D, float w1, float w2, float eps,
                                               float cs, float sn) {
  const float ss = wave_sum(own ? x1 * x1 + x2 * x2 : 0.f);
  const float inv = rsqrtf(ss / (float)D + eps);
  const float a = x1 * inv * w1, b = x2 * inv * w2;
  x1 = a * cs - b * sn;
  x2 = b * cs + a * sn;
}

template <typename T, int MT, int CW, int KW, GemmEpi E, bool kMultiA, bool kAF32>
__global__ __launch_bounds__(CW *KW * 64) void gemm_kernel(GemmArgs g) {
  constexpr int NW = CW * KW;
  constexpr int KPV = Storage<T>::kPerVec;
  constexpr int CH = ch_of<T>();
  constexpr bool kDual = E == GemmEpi::kSwiGLU;
  constexpr int NACC = kDual ? 2 : 1;
  constexpr int U = kGroup;
  constexpr int NPL = kAF32 ? 2 : 1;                               // A planes in LDS
  constexpr bool kF32Src = kAF32 || sizeof(T) == 4;                // A source is fp32
  constexpr int NSRC = kAF32 ? 2 : 1;                              // 16-byte source loads per vector
  constexpr int TR = 16 * MT, TC = 16 * CW;                        // final tile rows, columns
  static_assert(!kAF32 || (KPV == 8 && !kMultiA), "fp32 activations pair with bf16 weights");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T *sa = reinterpret_cast<T *>(smem);
  // after streaming the A region is reused: [red: NW*NACC*256][fin: NACC*TR*TC]
  float *red = reinterpret_cast<float *>(smem);
  float *fin = red + NW * NACC * 256;
  __shared__ float s_inv[TR];  // norm on load: per-row 1/rms
  __shared__ unsigned s_flag;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cw = wave % CW, kw = wave / CW;
  const int n0 = blockIdx.x * TC;
  const int ncol = n0 + cw * 16;
  const int m0 = blockIdx.z * TR;
  const int kb = blockIdx.y * g.kt;
  const int ke = min(g.K, kb + g.kt);
  const int kp = g.kp;      // K per staged pass (multiple of KW * CH)
  const int as = kp + KPV;  // LDS row stride of the A pass (16-byte pad)
  const int kq = kp / KW;   // K per wave per pass
  const bool active = ncol < g.N;
  const int kg = (lane >> 4) * KPV;
  const int a_seglen = g.K / g.a_nseg;
  const bool norm = g.norm_w != nullptr;

  // source row of A for tile row r (the LM head reads the kept rows of the block)
  auto src_row = [&](int m) {
    return g.keep_bs > 0 ? (m / (g.keep_bs - 1)) * g.keep_bs + m % (g.keep_bs - 1) + 1 : m;
  };
  if (norm) {
    // TPR threads per row sum the row's per-column-group sums of squares (fixed order)
    constexpr int TPR0 = NW * 64 / TR;
    constexpr int TPR = TPR0 >= 64 ? 64 : TPR0 >= 32 ? 32 : TPR0 >= 16 ? 16 : TPR0 >= 8 ? 8 : TPR0 >= 4 ? 4 : 2;
    static_assert(TR * TPR <= NW * 64, "row-scale threads");
    const int row = threadIdx.x / TPR, sub = threadIdx.x % TPR;
    float ss = 0.f;
    if (row < TR) {
      const int sr = src_row(min(m0 + row, g.M - 1));
      for (int q = sub; q < g.ss_groups; q += TPR) ss += g.ss[(size_t)q * g.ss_rows + sr];
    }
#pragma unroll
    for (int o = TPR / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
    if (row < TR && sub == 0) s_inv[row] = rsqrtf(ss / (float)g.K + g.eps);
    __syncthreads();
  }

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

  // Loads are issued unconditionally (addresses clamped into the operand) so that the
  // compiler counts outstanding loads exactly: weight loads stay in flight across the A
  // staging and across each MFMA group.
  const int vrow = kp / KPV;  // 16-byte vectors per staged A row (per plane)
  constexpr int NA = (kPassBytes / (16 * NPL) + NW * 64 - 1) / (NW * 64);  // A vectors per thread, max
  T *sa_lo = sa + TR * as;                                                 // lo plane (kAF32)
  for (int p0 = kb; p0 < ke; p0 += kp) {
    const int plen = min(kp, ke - p0);  // a multiple of CH
    const int q0 = kw * kq;
    const int q1 = min(plen, q0 + kq);
    const int nsteps = active && q1 > q0 ? (q1 - q0) / CH : 0;
    const int nfull = nsteps / U;
    const int total = TR * vrow;  // A vectors of this pass
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

    // ---- A rows [m0, m0 + TR) x K [p0, p0 + plen): loads first, then weights group 0
    Vec16 areg[NA][NSRC], wreg[NA];
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const int v = min((int)threadIdx.x + j * NW * 64, total - 1);
      const int r = v / vrow, cv = v % vrow;
      const int m = src_row(min(m0 + r, g.M - 1));
      const int k = p0 + min(cv * KPV, plen - KPV);
      // segment of the concatenated A that holds column k
      const int seg = kMultiA ? k / a_seglen : 0;
      const size_t aoff = (size_t)m * g.lda + (k - seg * a_seglen);
      if constexpr (kF32Src) {
        const float *ap = reinterpret_cast<const float *>(g.a[seg]) + aoff;
        areg[j][0] = load_vec16(ap);
        if constexpr (NSRC == 2) areg[j][NSRC - 1] = load_vec16(ap + 4);
      } else {
        areg[j][0] = load_vec16(reinterpret_cast<const T *>(g.a[seg]) + aoff);
      }
      if (norm) wreg[j] = load_vec16(reinterpret_cast<const T *>(g.norm_w) + k);
    }
    Vec16 b0[NACC][U], b1[NACC][U];
    load_group(b0, 0);
    __syncthreads();  // the previous pass (or the row scales) are done with LDS
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const int v = (int)threadIdx.x + j * NW * 64;
      if (v < total) {
        const int r = v / vrow, cv = v % vrow;
        const bool ok = m0 + r < g.M && cv * KPV < plen;
        if constexpr (kF32Src) {
          constexpr int NE = kAF32 ? 8 : KPV;  // fp32 values of this vector
          float f[NE];
          __builtin_memcpy(f, &areg[j][0].u, 16);
          if constexpr (NSRC == 2) __builtin_memcpy(f + 4, &areg[j][NSRC - 1].u, 16);
          if (norm) {
            T wv[NE];
            __builtin_memcpy(wv, &wreg[j].u, 16);
#pragma unroll
            for (int e = 0; e < NE; ++e) f[e] = f[e] * s_inv[r] * Storage<T>::load(wv, e);
          }
#pragma unroll
          for (int e = 0; e < NE; ++e) f[e] = ok ? f[e] : 0.f;
          if (g.a_out && blockIdx.x == 0 && ok)
#pragma unroll
            for (int e = 0; e < NE; ++e) g.a_out[(size_t)(m0 + r) * g.K + p0 + cv * KPV + e] = f[e];
          if constexpr (kAF32) {
            uint16_t hi[8], lo[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              hi[e] = f32_to_bf16(f[e]);
              lo[e] = f32_to_bf16(f[e] - bf16_to_f32(hi[e]));
            }
            __builtin_memcpy(sa + r * as + cv * KPV, hi, 16);
            __builtin_memcpy(sa_lo + r * as + cv * KPV, lo, 16);
          } else {
            __builtin_memcpy(sa + r * as + cv * KPV, f, 16);
          }
        } else {
          *reinterpret_cast<uint4 *>(sa + r * as + cv * KPV) = ok ? areg[j][0].u : make_uint4(0, 0, 0, 0);
        }
      }
    }
    __syncthreads();

    // ---- stream this wave's K range of the pass (ping-pong register buffers)
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

  // ---- KW sub-slice tiles -> the work-group's tile fin[a][row][col], summed in fixed order.
  //      MFMA tile layout: lane holds rows (lane/16)*4 + i, column lane%16 at [lane*4 + i].
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    __syncthreads();
#pragma unroll
    for (int a = 0; a < NACC; ++a) *reinterpret_cast<f32x4_t *>(&red[(wave * NACC + a) * 256 + lane * 4]) = acc[a][t];
    __syncthreads();
    for (int e = threadIdx.x; e < NACC * CW * 256; e += NW * 64) {
      const int a = e / (CW * 256), c = (e / 256) % CW, li = e % 256;
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < KW; ++q) s += red[((q * CW + c) * NACC + a) * 256 + li];
      const int row = t * 16 + (li >> 6) * 4 + (li & 3), col = c * 16 + ((li >> 2) & 15);
      fin[(a * TR + row) * TC + col] = s;
    }
  }
  __syncthreads();

  // ---- split-K: the last work-group of the output tile to arrive sums every split, in split
  //      order. The partials are written and read with device-scope (relaxed atomic) accesses,
  //      which are coherent across the XCDs' L2 caches by themselves; the work-group's stores
  //      are complete (s_waitcnt) before its arrival is counted, and the reducing work-group
  //      reads only after it has seen every arrival. No cache-wide write-back or invalidate is
  //      needed (the release/acquire fences that would emit them cost ~100 us per launch).
  const int S = gridDim.y;
  if (S > 1) {
    const size_t pstride = (size_t)g.M * g.N * NACC;
    float *mine = g.part + (size_t)blockIdx.y * pstride;
    for (int e = threadIdx.x; e < NACC * TR * TC; e += NW * 64) {
      const int a = e / (TR * TC), row = (e / TC) % TR, col = e % TC;
      const int m = m0 + row, n = n0 + col;
      if (m < g.M && n < g.N)
        __hip_atomic_store(&mine[((size_t)m * NACC + a) * g.N + n], fin[e], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores are acknowledged
    __syncthreads();
    unsigned *ctr = g.counters + (size_t)blockIdx.z * gridDim.x + blockIdx.x;
    if (threadIdx.x == 0) s_flag = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (s_flag != (unsigned)(S - 1)) return;
    for (int e = threadIdx.x; e < NACC * TR * TC; e += NW * 64) {
      const int a = e / (TR * TC), row = (e / TC) % TR, col = e % TC;
      const int m = m0 + row, n = n0 + col;
      float s = 0.f;
      if (m < g.M && n < g.N) {
        const float *src = g.part + ((size_t)m * NACC + a) * g.N + n;
        // loads in groups of 8 in flight, summed in split order
        for (int q0 = 0; q0 < S; q0 += 8) {
          float v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u)
            v[u] = q0 + u < S ? __hip_atomic_load(src + (size_t)(q0 + u) * pstride, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT)
                              : 0.f;
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (q0 + u < S) s += v[u];
        }
      }
      fin[e] = s;
    }
    if (threadIdx.x == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
  }

  // ---- epilogues on the final tile
  if constexpr (E == GemmEpi::kStore || E == GemmEpi::kResidAdd) {
    for (int e = threadIdx.x; e < TR * TC; e += NW * 64) {
      const int row = e / TC, col = e % TC;
      const int m = m0 + row, n = n0 + col;
      float v = fin[e];
      if (m < g.M && n < g.N) {
        const size_t o = (size_t)m * g.N + n;
        if (E == GemmEpi::kResidAdd) v += g.out[o];
        g.out[o] = v;
      } else {
        v = 0.f;
      }
      fin[e] = v * v;
    }
    if (g.ss_out) {  // per-row sum of squares over this column group, for norm on load
      __syncthreads();
      for (int row = threadIdx.x; row < TR; row += NW * 64) {
        float s = 0.f;
        for (int c = 0; c < TC; ++c) s += fin[row * TC + c];
        if (m0 + row < g.M) g.ss_out[(size_t)blockIdx.x * g.M + m0 + row] = s;
      }
    }
  } else if constexpr (E == GemmEpi::kSwiGLU) {
    for (int e = threadIdx.x; e < TR * TC; e += NW * 64) {
      const int row = e / TC, col = e % TC;
      const int m = m0 + row, n = n0 + col;
      if (m < g.M && n < g.N) {
        const float gt = fin[e], up = fin[TR * TC + e];
        g.out[(size_t)m * g.N + n] = gt / (1.f + expf(-gt)) * up;
      }
    }
  } else if constexpr (E == GemmEpi::kArgmax) {
    // TPR threads per row scan the row's columns, then a shuffle reduction
    constexpr int TPR0 = NW * 64 / TR;
    constexpr int TPR = TPR0 >= 32 ? 32 : TPR0 >= 16 ? 16 : TPR0 >= 8 ? 8 : TPR0 >= 4 ? 4 : TPR0 >= 2 ? 2 : 1;
    if (threadIdx.x < TR * TPR) {
      const int row = threadIdx.x / TPR, sub = threadIdx.x % TPR;
      float best = -INFINITY;
      int bi = 0x7fffffff;
      for (int c = sub; c < TC; c += TPR)
        if (n0 + c < g.N) argmax_merge(best, bi, fin[row * TC + c], n0 + c);
#pragma unroll
      for (int o = TPR / 2; o > 0; o >>= 1) {
        const float ov = __shfl_xor(best, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        argmax_merge(best, bi, ov, oi);
      }
      const int m = m0 + row;
      if (sub == 0 && m < g.M) {
        g.amax_val[(size_t)m * gridDim.x + blockIdx.x] = best;
        g.amax_idx[(size_t)m * gridDim.x + blockIdx.x] = bi;
      }
    }
  } else if constexpr (E == GemmEpi::kHeadNormRope || E == GemmEpi::kKvScatter) {
    // one head per column group; one wave per row; lane i < D/2 owns the pair (i, i + D/2)
    const int D = TC, half = TC / 2;
    const bool own = lane < half;
    const int i1 = own ? lane : 0, i2 = i1 + half;
    const int h = blockIdx.x;
    for (int row = wave; row < TR; row += NW) {
      const int m = m0 + row;
      if (m >= g.M) break;
      float x1 = fin[row * TC + i1], x2 = fin[row * TC + i2];
      if constexpr (E == GemmEpi::kHeadNormRope) {
        const int QH = g.n_q_heads, KVH = g.n_kv_heads;
        T *dst;
        if (h < QH + KVH) {
          const T *w = reinterpret_cast<const T *>(h < QH ? g.q_norm : g.k_norm);
          const int b = m / g.block_size, j = m % g.block_size;
          const int pos = min(min(max(g.seq_lens[b], 0), g.max_ctx) + j, g.rope_max_pos - 1);
          head_norm_rope(x1, x2, own, D, Storage<T>::load(w, i1), Storage<T>::load(w, i2), g.eps,
                         g.rope_cos[(size_t)pos * half + i1], g.rope_sin[(size_t)pos * half + i1]);
          dst = h < QH ? reinterpret_cast<T *>(g.q) + ((size_t)m * QH + h) * D
                       : reinterpret_cast<T *>(g.k) + ((size_t)m * KVH + h - QH) * D;
        } else {
          dst = reinterpret_cast<T *>(g.v) + ((size_t)m * KVH + h - QH - KVH) * D;
        }
        if (own) {
          Storage<T>::store(dst, i1, x1);
          Storage<T>::store(dst, i2, x2);
        }
      } else {
        const int KVH = g.n_kv_heads;
        const int l = h / (2 * KVH), j = h % (2 * KVH);
        const bool is_v = j >= KVH;
        const int gh = is_v ? j - KVH : j;
        const int64_t slot = g.slot_mapping[m];
        if (slot < 0 || slot >= g.num_slots) continue;  // padding row / out of range: skipped
        if (!is_v) {
          const T *w = reinterpret_cast<const T *>(g.layer_k_norm[l]);
          const int pos = min(max(g.positions[m], 0), g.rope_max_pos - 1);
          head_norm_rope(x1, x2, own, D, Storage<T>::load(w, i1), Storage<T>::load(w, i2), g.eps,
                         g.rope_cos[(size_t)pos * half + i1], g.rope_sin[(size_t)pos * half + i1]);
        }
        T *dst = reinterpret_cast<T *>(is_v ? g.v_cache[l] : g.k_cache[l]) + ((size_t)slot * KVH + gh) * D;
        if (own) {
          Storage<T>::store(dst, i1, x1);
          Storage<T>::store(dst, i2, x2);
        }
      }
    }
  }
}

// Work-group shape (CW column tiles x KW K sub-slices) for a problem.
struct Shape {
  int cw, kw;
};
Shape pick_shape(int M, int head_dim, GemmEpi epi) {
  if (epi == GemmEpi::kHeadNormRope || epi == GemmEpi::kKvScatter) return {head_dim / 16, 128 / head_dim};
  if (gemm_mt(M) > 1) return {2, 2};
  if (epi == GemmEpi::kArgmax) return {8, 1};
  return {4, 2};
}

template <typename T, int MT, int CW, int KW, GemmEpi E, bool kAF32>
size_t lds_bytes(const GemmArgs &g) {
  constexpr int KPV = Storage<T>::kPerVec;
  const size_t a = (size_t)16 * MT * (g.kp + KPV) * sizeof(T) * (kAF32 ? 2 : 1);
  const int nacc = E == GemmEpi::kSwiGLU ? 2 : 1;
  const size_t r = ((size_t)CW * KW * nacc * 256 + (size_t)nacc * 16 * MT * 16 * CW) * sizeof(float);
  return a > r ? a : r;
}

template <typename T, int MT, int CW, int KW, GemmEpi E, bool kMultiA, bool kAF32>
hipError_t launch_k(const GemmArgs &g, int splits, hipStream_t s) {
  dim3 grid((g.N + 16 * CW - 1) / (16 * CW), splits, (g.M + 16 * MT - 1) / (16 * MT));
  gemm_kernel<T, MT, CW, KW, E, kMultiA, kAF32>
      <<<grid, CW * KW * 64, lds_bytes<T, MT, CW, KW, E, kAF32>(g), s>>>(g);
  return hipGetLastError();
}

template <typename T, GemmEpi E, bool kMultiA, bool kAF32, int CW, int KW>
hipError_t launch_mt(const GemmArgs &g, int splits, hipStream_t s) {
  switch (gemm_mt(g.M)) {
    case 1: return launch_k<T, 1, CW, KW, E, kMultiA, kAF32>(g, splits, s);
    case 2: return launch_k<T, 2, CW, KW, E, kMultiA, kAF32>(g, splits, s);
    case 3: return launch_k<T, 3, CW, KW, E, kMultiA, kAF32>(g, splits, s);
    default: return launch_k<T, 4, CW, KW, E, kMultiA, kAF32>(g, splits, s);
  }
}

template <typename T, GemmEpi E, bool kMultiA, bool kAF32>
hipError_t launch_t(const GemmArgs &g, int splits, hipStream_t s) {
  if constexpr (E == GemmEpi::kHeadNormRope || E == GemmEpi::kKvScatter) {
    return g.head_dim == 128 ? launch_mt<T, E, kMultiA, kAF32, 8, 1>(g, splits, s)
                             : launch_mt<T, E, kMultiA, kAF32, 4, 2>(g, splits, s);
  } else if (gemm_mt(g.M) > 1) {
    return launch_mt<T, E, kMultiA, kAF32, 2, 2>(g, splits, s);
  } else if constexpr (E == GemmEpi::kArgmax) {
    return launch_k<T, 1, 8, 1, E, kMultiA, kAF32>(g, splits, s);
  } else {
    return launch_k<T, 1, 4, 2, E, kMultiA, kAF32>(g, splits, s);
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
    case GemmEpi::kArgmax: return launch_t<T, GemmEpi::kArgmax, false, kAF32>(g, splits, s);
    case GemmEpi::kHeadNormRope: return launch_t<T, GemmEpi::kHeadNormRope, false, kAF32>(g, splits, s);
    default: return launch_t<T, GemmEpi::kKvScatter, false, kAF32>(g, splits, s);
  }
}

int kstep(int M, int head_dim, GemmEpi epi, bool bf16) {
  return pick_shape(M, head_dim, epi).kw * (bf16 ? ch_of<uint16_t>() : ch_of<float>());
}

}  // namespace

int gemm_mt(int M) { return M <= 16 ? 1 : M <= 32 ? 2 : M <= 48 ? 3 : 4; }

int gemm_col_groups(int M, int N, int head_dim, GemmEpi epi) {
  const int cols = 16 * pick_shape(M, head_dim, epi).cw;
  return (N + cols - 1) / cols;
}

int gemm_row_blocks(int M) { return (M + 16 * gemm_mt(M) - 1) / (16 * gemm_mt(M)); }

int gemm_plan_splits(int M, int N, int K, int head_dim, bool bf16, GemmEpi epi) {
  if (epi == GemmEpi::kArgmax) return 1;
  const int step = kstep(M, head_dim, epi, bf16);
  const long wgs = (long)gemm_col_groups(M, N, head_dim, epi) * gemm_row_blocks(M);
  int s = 1;
  // Up to ~1024 work-groups (4 per CU) while each split keeps >= 256 K and divides K.
  while (wgs * s * 2 <= 1024 && K % (2 * s * step) == 0 && K / (2 * s) >= 256 && s < 64) s *= 2;
  return s;
}

hipError_t launch_gemm(const GemmArgs &g0, bool bf16, GemmEpi epi, int splits, hipStream_t s) {
  ProfScope prof(g0.tag ? g0.tag : "gemm", s);
  const int step = kstep(g0.M, g0.head_dim, epi, bf16);
  const bool head = epi == GemmEpi::kHeadNormRope || epi == GemmEpi::kKvScatter;
  if ((epi != GemmEpi::kStore && g0.a_nseg > 1) || g0.N % 16 || g0.K % step || splits < 1 || g0.K % splits ||
      (g0.K / splits) % step || (epi == GemmEpi::kArgmax && splits != 1) ||
      (g0.a_nseg > 1 && (g0.K / g0.a_nseg) % (bf16 ? 8 : 4)) || (splits > 1 && (!g0.part || !g0.counters)) ||
      (head && (g0.head_dim != 64 && g0.head_dim != 128)) ||
      ((g0.norm_w || g0.a_out) && (g0.a_nseg > 1 || (bf16 && !g0.a_f32) || !g0.ss)) ||
      (g0.keep_bs == 1))
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
