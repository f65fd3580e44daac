// Weight-streaming MFMA GEMM with fused epilogues: every projection of the drafter.
//
// Every projection of the drafter is C = A W^T with a short activation A (the block's rows:
// 16 at batch 1) and a long weight W [N, K] that must be read once from HBM. The kernel is
// built around streaming W at full HBM rate:
//  * a work-group owns 16*CW*CT output columns (a column group) and one K slice of the
//    split-K grid (grid.y); its CW*KW waves each own CT column tiles of 16 W rows and one of
//    KW sub-slices of K;
//  * each wave streams its W rows in 16-byte-per-lane loads that feed
//    v_mfma_f32_16x16x32_bf16 directly (B operand = 16 W rows x 64 contiguous bytes), in
//    ping-pong register buffers so that two groups of loads are in flight; one A fragment
//    read from LDS serves all CT tiles;
//  * the activation slice is staged in LDS in passes (up to ~132 KiB when the work-group
//    has the CU to itself), so the MFMA loop reads only weights from memory. fp32
//    activations (one row tile) are moved by LDS DMA: every wave issues global->LDS loads
//    of 1 KiB segments that need no registers, so a whole pass is in flight at once while
//    the first weight groups load; the pass is then converted in place to a pair of bf16
//    values per element, hi = bf16(f) and lo = bf16(f - hi), which costs two MFMAs per step.
//    hi + lo keeps 17 significant bits of f (relative error at most 2^-17, about 7.6e-6). RMSNorm can be
//    applied while converting ("norm on load"): row scales come from per-column-group sums
//    of squares written by the producer of the rows, the norm weight slice arrives by DMA
//    with the pass;
//  * a work-group may own several column groups (up to NCG): K passes are then the outer
//    loop, so each staged pass serves all of them and the accumulators stay in registers;
//  * the KW sub-slice tiles are summed through LDS in a fixed order into the work-group's
//    tile. With several K splits every split writes its tile to the workspace with
//    device-scope stores and the last work-group of the output tile to arrive (a device-scope
//    counter) sums all splits in split order, with the loads of all its elements in flight
//    together. There are no float atomics, so results are deterministic;
//  * the epilogue runs on the final tile: fp32 store, residual add, SwiGLU, the LM head's
//    per-group (max, lowest index), per-head q/k RMSNorm + RoPE of the block, or the
//    context K/V epilogue of injection (k_norm + RoPE + paged scatter). The last three
//    need a column group to be exactly one head.
// Up to 64 activation rows are held as MT accumulator tiles (more rows would use grid.z
// blocks). gemm_plan sends more than 64 rows of a bf16 drafter to the LDS-tiled kernels further
// down: gemm_tiled_kernel (64 x 256 or 128 x 128 tiles) and gemm_wide_kernel (256 x 256 tiles,
// one work-group per CU).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dflash {
namespace {

constexpr int kDefaultPassBytes = 60 << 10;  // LDS for one staged A pass unless the plan says more
constexpr int kMaxLds = 160 << 10;           // LDS of one CU
constexpr int kStageVecs = 2;                // A vectors staged per thread per round
constexpr int kMaxGroupsPerWg = 8;           // column groups of one persistent work-group, max

// LDS of one staged pass of fp32 activations (DMA staging): rows of whole 1 KiB DMA
// segments plus 16 bytes of padding (the 16 rows of an MFMA fragment read then fall on
// distinct banks), followed by the pass's slice of the norm weight.
__host__ __device__ constexpr int dma_row_bytes(int kp) { return (kp * 4 + 1023) / 1024 * 1024 + 16; }
__host__ __device__ constexpr int dma_w_bytes(int kp) { return (kp * 2 + 1023) / 1024 * 1024; }

// 16 bytes per lane from global memory straight into LDS at lds + 16 * lane (lds must be
// uniform across the wave).
__device__ __forceinline__ void dma16(const void *src, void *lds) {
  __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
}

template <typename T>
__host__ __device__ constexpr int ch_of() {
  return 4 * Storage<T>::kPerVec;  // K elements per wave MFMA step
}

// K steps per register buffer: about 8 16-byte weight loads per lane in each of the two
// buffers, 4 when the work-group splits K among its waves (those run several work-groups to
// a CU). Loads in flight beyond what covers the memory latency only lengthen the queues: every
// dependent access of the kernel (activation staging, the split-K hand-off) then waits longer.
__host__ __device__ constexpr int group_steps(int ct, int nacc, int kw) {
  return ct * nacc >= (kw > 1 ? 4 : 8) ? 1 : (kw > 1 ? 4 : 8) / (ct * nacc);
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

// The head epilogues on head h of output row m, one head vector per wave: lane i < D/2 owns
// the pair (x1, x2) = (i, i + D/2); every lane of the wave takes part (the norm is a wave sum).
//  kHeadNormRope: h indexes q | k | v heads of the block; q and k heads are RMS-normalised
//                 (q_norm / k_norm) and rotated at position min(seq_len, max_ctx) + j of
//                 block slot j; all are rounded to the storage type into q, k or v.
//  kKvScatter:    h indexes layer-major (k heads, v heads) of the fused context projection;
//                 keys take the layer's k_norm and RoPE at positions[m]; both are rounded and
//                 written to slot slot_mapping[m] of the layer's cache (a slot outside
//                 [0, num_slots) is skipped).
template <typename T, GemmEpi E>
__device__ __forceinline__ void head_epilogue(const GemmArgs &g, int h, int m, float x1, float x2, bool own, int i1,
                                              int D) {
  const int half = D / 2, i2 = i1 + half;
  T *dst;
  if constexpr (E == GemmEpi::kHeadNormRope) {
    const int QH = g.n_q_heads, KVH = g.n_kv_heads;
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
  } else {
    const int KVH = g.n_kv_heads;
    const int l = h / (2 * KVH), j = h % (2 * KVH);
    const bool is_v = j >= KVH;
    const int gh = is_v ? j - KVH : j;
    const int64_t slot = g.slot_mapping[m];
    if (slot < 0 || slot >= g.num_slots) return;  // padding row / out of range: skipped (uniform per wave)
    if (!is_v) {
      const T *w = reinterpret_cast<const T *>(g.layer_k_norm[l]);
      const int pos = min(max(g.positions[m], 0), g.rope_max_pos - 1);
      head_norm_rope(x1, x2, own, D, Storage<T>::load(w, i1), Storage<T>::load(w, i2), g.eps,
                     g.rope_cos[(size_t)pos * half + i1], g.rope_sin[(size_t)pos * half + i1]);
    }
    dst = reinterpret_cast<T *>(is_v ? g.v_cache[l] : g.k_cache[l]) + ((size_t)slot * KVH + gh) * D;
  }
  if (own) {
    Storage<T>::store(dst, i1, x1);
    Storage<T>::store(dst, i2, x2);
  }
}

// Occupancy at one row tile: 4-wave work-groups run four to a CU, 8-wave ones two (at most
// 128 VGPRs); a work-group that owns several column groups keeps their accumulators and has
// the CU alone.
template <typename T, int MT, int CW, int CT, int KW, int NCG, GemmEpi E, bool kMultiA, bool kAF32>
__global__ __launch_bounds__(CW *KW * 64, MT > 1 ? 1 : CW * KW == 4 ? 4 : (NCG == 1 ? 2 : 1)) void gemm_kernel(GemmArgs g) {
  constexpr int NW = CW * KW, NT = NW * 64;
  constexpr int KPV = Storage<T>::kPerVec;
  constexpr int CH = ch_of<T>();
  constexpr bool kDual = E == GemmEpi::kSwiGLU;
  constexpr int NACC = kDual ? 2 : 1;
  constexpr int U = group_steps(CT, NACC, KW);
  constexpr int NPL = kAF32 ? 2 : 1;                 // A planes in LDS
  constexpr bool kF32Src = kAF32 || sizeof(T) == 4;  // A source is fp32
  constexpr int NSRC = kAF32 ? 2 : 1;                // 16-byte source loads per staged vector
  constexpr int TR = 16 * MT, TC = 16 * CW * CT;     // final tile rows, columns
  constexpr bool kDma = kAF32 && MT == 1;  // fp32 activations of one row tile: LDS DMA staging
  static_assert(!kAF32 || (KPV == 8 && !kMultiA), "fp32 activations pair with bf16 weights");
  // LDS: [A pass][red: NW*NACC*CT*256][fin: NACC*TR*TC]. The A pass is NPL planes of
  // TR x (kp + KPV) elements, or with DMA staging TR rows of dma_row_bytes(kp) then the norm
  // weight slice: each row is first the raw fp32 values, then converted in place to 32-byte
  // chunks [8 bf16 hi][8 bf16 lo] of 8 consecutive columns.
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T *sa = reinterpret_cast<T *>(smem);
  const int rs = dma_row_bytes(g.kp);  // DMA staging: LDS bytes per A row
  unsigned char *sw = smem + (size_t)TR * rs;
  float *red = reinterpret_cast<float *>(
      smem + (kDma ? (size_t)TR * rs + dma_w_bytes(g.kp) : (size_t)NPL * TR * (g.kp + KPV) * sizeof(T)));
  float *fin = red + NW * NACC * CT * 256;
  __shared__ float s_inv[TR];  // norm on load: per-row 1/rms
  __shared__ unsigned s_flag;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cw = wave % CW, kw = wave / CW;
  const int ncg = (g.N + TC - 1) / TC;  // column groups; this work-group takes blockIdx.x + i*gridDim.x
  const int m0 = blockIdx.z * TR;
  const int kb = blockIdx.y * g.kt;
  const int ke = min(g.K, kb + g.kt);
  const int kp = g.kp;      // K per staged pass (multiple of KW * CH)
  const int as = kp + KPV;  // LDS row stride of the A pass (16-byte pad)
  const int kq = kp / KW;   // K per wave per pass
  const int kg = (lane >> 4) * KPV;
  const int a_seglen = g.K / g.a_nseg;
  const bool norm = g.norm_w != nullptr;
  const int S = gridDim.y;

  // source row of A for tile row r (the LM head reads the kept rows of the block)
  auto src_row = [&](int m) {
    return g.keep_bs > 0 ? (m / (g.keep_bs - 1)) * g.keep_bs + m % (g.keep_bs - 1) + 1 : m;
  };
  // DMA staging: every wave issues global->LDS loads of 1 KiB segments (a lane moves 16
  // bytes; the LDS address is uniform per instruction), so the whole pass is in flight at
  // once without registers. Columns past the pass read a clamped valid address; they are
  // never used.
  auto issue_dma = [&](int p0, int plen) {
    const int segs = (plen * 4 + 1023) / 1024;
    const float *a0 = reinterpret_cast<const float *>(g.a[0]);
    for (int q = wave; q < TR * segs; q += NW) {
      const int r = q / segs, sg = q % segs;
      const int m = src_row(min(m0 + r, g.M - 1));
      const int c = min(sg * 256 + lane * 4, plen - 4);
      dma16(a0 + (size_t)m * g.lda + p0 + c, smem + (size_t)r * rs + sg * 1024);
    }
    if (norm) {
      const T *w0 = reinterpret_cast<const T *>(g.norm_w);
      for (int q = wave; q * 512 < plen; q += NW)
        dma16(w0 + p0 + min(q * 512 + lane * 8, plen - 8), sw + q * 1024);
    }
  };
  // W row of this lane in each of the wave's column tiles of column group cg (a column past N
  // reads a valid row of the first segment; its results are never stored)
  auto set_rows = [&](const T *(&brow)[NACC][CT], int cg) {
    const int nw0 = cg * TC + cw * CT * 16;
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const int ncol = nw0 + c * 16;
      int seg = 0, nbase = 0;
      if (!kDual)
        while (seg < g.b_nseg - 1 && ncol >= g.b_end[seg]) nbase = g.b_end[seg++];
      const bool act = ncol < g.N;
      const int r = (act ? ncol - nbase : 0) + (lane & 15);
      brow[0][c] = reinterpret_cast<const T *>(g.b[act ? seg : 0]) + (size_t)r * g.K + kg;
      if (kDual) brow[NACC - 1][c] = reinterpret_cast<const T *>(g.b[1]) + (size_t)r * g.K + kg;
    }
  };

  // The first pass's activations (DMA) and first weight group go out before anything waits:
  // the row scales' loads then overlap them.
  if constexpr (kDma) issue_dma(kb, min(g.kp, ke - kb));
  Vec16 b0[NACC][CT][U], b1[NACC][CT][U];
  {
    const int plen = min(kp, ke - kb), q0 = kw * kq;
    const T *brow[NACC][CT];
    set_rows(brow, blockIdx.x);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int a = 0; a < NACC; ++a) b0[a][c][u] = load_vec16(brow[a][c] + kb + min(q0 + u * CH, plen - CH));
  }
  if (norm) {
    // TPR threads per row sum the row's per-column-group sums of squares (fixed order)
    constexpr int TPR0 = NT / TR;
    constexpr int TPR = TPR0 >= 64 ? 64 : TPR0 >= 32 ? 32 : TPR0 >= 16 ? 16 : TPR0 >= 8 ? 8 : TPR0 >= 4 ? 4 : 2;
    static_assert(TR * TPR <= NT, "row-scale threads");
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

  const int vrow = kp / KPV;  // 16-byte vectors per staged A row (per plane)
  T *sa_lo = sa + TR * as;    // lo plane (kAF32)
  Vec16 areg[kStageVecs][NSRC], wreg[kStageVecs];
  // ---- A rows [m0, m0 + TR) x K [p0, p0 + plen) into LDS, in rounds of kStageVecs vectors
  //      per thread (the normalised rows also go to a_out from the first column group)
  auto stage_load = [&](int p0, int plen, int base) {
    const int total = TR * vrow;
#pragma unroll
    for (int j = 0; j < kStageVecs; ++j) {
      const int v = min(base + (int)threadIdx.x + j * NT, total - 1);
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
  };
  auto stage_store = [&](int p0, int plen, int base, bool write_out) {
    const int total = TR * vrow;
#pragma unroll
    for (int j = 0; j < kStageVecs; ++j) {
      const int v = base + (int)threadIdx.x + j * NT;
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
          if (write_out && ok)
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
  };

  // DMA staging: wait for the pass, then convert it in place (norm on load, rows past M
  // zeroed, hi/lo split); the normalised rows also go to a_out from the first column group.
  auto convert_dma = [&](int p0, int plen, bool write_out) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's DMA has landed
    __syncthreads();
    const int nch = plen / 8;
    for (int v = threadIdx.x; v < TR * nch; v += NT) {
      const int r = v / nch, c = v % nch;
      unsigned char *pc = smem + (size_t)r * rs + c * 32;
      float f[8];
      __builtin_memcpy(f, pc, 32);
      if (norm) {
        T wv[8];
        __builtin_memcpy(wv, sw + c * 16, 16);
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = f[e] * s_inv[r] * Storage<T>::load(wv, e);
      }
      const bool ok = m0 + r < g.M;
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = ok ? f[e] : 0.f;
      if (write_out && ok)
#pragma unroll
        for (int e = 0; e < 8; ++e) g.a_out[(size_t)(m0 + r) * g.K + p0 + c * 8 + e] = f[e];
      uint16_t hl[16];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        hl[e] = f32_to_bf16(f[e]);
        hl[8 + e] = f32_to_bf16(f[e] - bf16_to_f32(hl[e]));
      }
      __builtin_memcpy(pc, hl, 32);
    }
    __syncthreads();
  };

  // The work-group's column groups: cg_i = blockIdx.x + i * gridDim.x for i < NCG (cg_i < ncg),
  // one accumulator set each. K passes are the outer loop, so each pass of A is staged once
  // and serves every column group of the work-group.
  f32x4_t acc[NCG][NACC][CT][MT];
#pragma unroll
  for (int i = 0; i < NCG; ++i)
#pragma unroll
    for (int a = 0; a < NACC; ++a)
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[i][a][c][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int p0 = kb; p0 < ke; p0 += kp) {
    const int plen = min(kp, ke - p0);  // a multiple of CH
    const int q0 = kw * kq;
    const int q1 = min(plen, q0 + kq);
    auto kclamp = [&](int st) { return p0 + min(q0 + st * CH, plen - CH); };

#pragma unroll
    for (int i = 0; i < NCG; ++i) {
      const int cg = blockIdx.x + i * gridDim.x;
      if (cg >= ncg) break;
      const bool wave_active = cg * TC + cw * CT * 16 < g.N;
      const int nsteps = wave_active && q1 > q0 ? (q1 - q0) / CH : 0;
      const int nfull = nsteps / U;
      const T *brow[NACC][CT];
      set_rows(brow, cg);
      auto load_group = [&](Vec16(&b)[NACC][CT][U], int gi) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int a = 0; a < NACC; ++a) b[a][c][u] = load_vec16(brow[a][c] + kclamp(gi * U + u));
      };
      auto mma_step = [&](const Vec16(&bf)[NACC][CT], int k) {
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const int ao = (t * 16 + (lane & 15)) * as + k + kg;
          const unsigned char *pd = smem + (size_t)(t * 16 + (lane & 15)) * rs + ((k + kg) >> 3) * 32;
          Vec16 af;
          af.u = kDma ? *reinterpret_cast<const uint4 *>(pd) : *reinterpret_cast<const uint4 *>(sa + ao);
#pragma unroll
          for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int a = 0; a < NACC; ++a) mma16<T>(acc[i][a][c][t], af, bf[a][c]);
          if constexpr (kAF32) {
            af.u = kDma ? *reinterpret_cast<const uint4 *>(pd + 16) : *reinterpret_cast<const uint4 *>(sa_lo + ao);
#pragma unroll
            for (int c = 0; c < CT; ++c)
#pragma unroll
              for (int a = 0; a < NACC; ++a) mma16<T>(acc[i][a][c][t], af, bf[a][c]);
          }
        }
      };
      auto compute = [&](const Vec16(&b)[NACC][CT][U], int st0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          Vec16 bf[NACC][CT];
#pragma unroll
          for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int a = 0; a < NACC; ++a) bf[a][c] = b[a][c][u];
          mma_step(bf, q0 + (st0 + u) * CH);
        }
      };

      // Loads are issued unconditionally (addresses clamped into the operand) so that the
      // compiler counts outstanding loads exactly: weight loads stay in flight across the A
      // staging and across each MFMA group.
      if (p0 != kb || i != 0) load_group(b0, 0);  // the first one was issued at the start
      if (kDma && i == 0) {
        // ---- A rows [m0, m0 + TR) x K [p0, p0 + plen) into LDS by DMA (the first pass was
        //      issued at the start; a later one once every wave is done with the previous)
        if (p0 != kb) {
          __syncthreads();
          issue_dma(p0, plen);
        }
        convert_dma(p0, plen, g.a_out != nullptr && blockIdx.x == 0);
      } else if (i == 0) {
        // ---- A rows [m0, m0 + TR) x K [p0, p0 + plen) into LDS; the first round's loads
        //      and the first weight group are in flight together
        const int total = TR * vrow;
        const bool write_out = g.a_out != nullptr && blockIdx.x == 0;
        stage_load(p0, plen, 0);
        __syncthreads();  // the previous pass (or the row scales) are done with LDS
        stage_store(p0, plen, 0, write_out);
        for (int base = kStageVecs * NT; base < total; base += kStageVecs * NT) {
          stage_load(p0, plen, base);
          stage_store(p0, plen, base, write_out);
        }
        __syncthreads();
      }

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
        Vec16 bf[NACC][CT];
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
          for (int a = 0; a < NACC; ++a) bf[a][c] = load_vec16(brow[a][c] + p0 + q0 + st * CH);
        mma_step(bf, q0 + st * CH);
      }
    }
  }

#pragma unroll
  for (int i = 0; i < NCG; ++i) {
    const int cg = blockIdx.x + i * gridDim.x;
    if (cg >= ncg) break;
    const int n0 = cg * TC;
    // residual-add: the tile's residual values load now, so the hand-off below hides them
    constexpr int NRES = E == GemmEpi::kResidAdd ? (TR * TC + NT - 1) / NT : 1;
    float res[NRES];
#pragma unroll
    for (int j = 0; j < NRES; ++j) {
      const int e = threadIdx.x + j * NT;
      const int m = m0 + e / TC, n = n0 + e % TC;
      res[j] = E == GemmEpi::kResidAdd && e < TR * TC && m < g.M && n < g.N ? g.out[(size_t)m * g.N + n] : 0.f;
    }

    // ---- KW sub-slice tiles -> the work-group's tile fin[a][row][col], summed in fixed order.
    //      MFMA tile layout: lane holds rows (lane/16)*4 + i, column lane%16 at [lane*4 + i].
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      __syncthreads();  // red and fin are free (previous tile / column group done)
#pragma unroll
      for (int a = 0; a < NACC; ++a)
#pragma unroll
        for (int c = 0; c < CT; ++c)
          *reinterpret_cast<f32x4_t *>(&red[((wave * NACC + a) * CT + c) * 256 + lane * 4]) = acc[i][a][c][t];
      __syncthreads();
      for (int e = threadIdx.x; e < NACC * CW * CT * 256; e += NT) {
        const int a = e / (CW * CT * 256), cc = (e / 256) % (CW * CT), li = e % 256;
        const int wc = cc / CT, c = cc % CT;  // owning wave column and its tile
        float s = 0.f;
#pragma unroll
        for (int q = 0; q < KW; ++q) s += red[(((q * CW + wc) * NACC + a) * CT + c) * 256 + li];
        const int row = t * 16 + (li >> 6) * 4 + (li & 3), col = cc * 16 + ((li >> 2) & 15);
        fin[(a * TR + row) * TC + col] = s;
      }
    }
    __syncthreads();

    // ---- split-K: the last work-group of the output tile to arrive sums every split, in
    //      split order. The partials are written and read with device-scope (relaxed atomic)
    //      accesses, which are coherent across the XCDs' L2 caches by themselves; the
    //      work-group's stores are complete (s_waitcnt) before its arrival is counted, and the
    //      reducing work-group reads only after it has seen every arrival. No cache-wide
    //      write-back or invalidate is needed (fences that emit them cost ~100 us per launch).
    if (S > 1) {
      const size_t pstride = (size_t)g.M * g.N * NACC;
      float *mine = g.part + (size_t)blockIdx.y * pstride;
      for (int e = threadIdx.x; e < NACC * TR * TC; e += NT) {
        const int a = e / (TR * TC), row = (e / TC) % TR, col = e % TC;
        const int m = m0 + row, n = n0 + col;
        if (m < g.M && n < g.N)
          __hip_atomic_store(&mine[((size_t)m * NACC + a) * g.N + n], fin[e], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
      __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores are acknowledged
      __syncthreads();
      unsigned *ctr = g.counters + (size_t)blockIdx.z * ncg + cg;
      if (threadIdx.x == 0) s_flag = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      if (s_flag != (unsigned)(S - 1)) continue;  // another split finishes this tile
      // the loads of all this thread's elements, 8 splits each, in flight together (one round
      // trip for up to 8 splits, not one per element); every load is issued (past the last
      // split, or for an element outside the output, a valid address whose value is dropped),
      // and each element is summed in split order
      constexpr int JR = (NACC * TR * TC + NT - 1) / NT;
      float sum[JR];
      const float *src[JR];
      bool keep[JR];
#pragma unroll
      for (int j = 0; j < JR; ++j) {
        const int e = threadIdx.x + j * NT;
        const int a = e / (TR * TC), row = (e / TC) % TR, col = e % TC;
        const int m = m0 + row, n = n0 + col;
        keep[j] = e < NACC * TR * TC && m < g.M && n < g.N;
        src[j] = keep[j] ? g.part + ((size_t)m * NACC + a) * g.N + n : g.part;
        sum[j] = 0.f;
      }
      for (int q0 = 0; q0 < S; q0 += 8) {
        float v[JR][8];
#pragma unroll
        for (int j = 0; j < JR; ++j)
#pragma unroll
          for (int u = 0; u < 8; ++u)
            v[j][u] = __hip_atomic_load(src[j] + (size_t)min(q0 + u, S - 1) * pstride, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int j = 0; j < JR; ++j)
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (keep[j] && q0 + u < S) sum[j] += v[j][u];
      }
#pragma unroll
      for (int j = 0; j < JR; ++j) {
        const int e = threadIdx.x + j * NT;
        if (e < NACC * TR * TC) fin[e] = sum[j];
      }
      if (threadIdx.x == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
    }

    // ---- epilogues on the final tile
    if constexpr (E == GemmEpi::kStore || E == GemmEpi::kResidAdd) {
#pragma unroll
      for (int j = 0; j < (TR * TC + NT - 1) / NT; ++j) {
        const int e = threadIdx.x + j * NT;
        if (e >= TR * TC) break;
        const int row = e / TC, col = e % TC;
        const int m = m0 + row, n = n0 + col;
        float v = fin[e];
        if (m < g.M && n < g.N) {
          if constexpr (E == GemmEpi::kResidAdd) v += res[j];
          g.out[(size_t)m * g.N + n] = v;
        } else {
          v = 0.f;
        }
        fin[e] = v * v;
      }
      if (g.ss_out) {  // per-row sum of squares over this column group, for norm on load
        constexpr int TPR0 = NT / TR;
        constexpr int TPR = TPR0 >= 64 ? 64 : TPR0 >= 32 ? 32 : TPR0 >= 16 ? 16 : TPR0 >= 8 ? 8 : TPR0 >= 4 ? 4 : 2;
        __syncthreads();
        const int row = threadIdx.x / TPR, sub = threadIdx.x % TPR;
        float s = 0.f;
        if (row < TR)
          for (int c = sub; c < TC; c += TPR) s += fin[row * TC + c];
  #pragma unroll
        for (int o = TPR / 2; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
        if (row < TR && sub == 0 && m0 + row < g.M) g.ss_out[(size_t)cg * g.M + m0 + row] = s;
      }
    } else if constexpr (E == GemmEpi::kSwiGLU) {
      for (int e = threadIdx.x; e < TR * TC; e += NT) {
        const int row = e / TC, col = e % TC;
        const int m = m0 + row, n = n0 + col;
        if (m < g.M && n < g.N) {
          const float gt = fin[e], up = fin[TR * TC + e];
          g.out[(size_t)m * g.N + n] = gt / (1.f + expf(-gt)) * up;
        }
      }
    } else if constexpr (E == GemmEpi::kArgmax) {
      // TPR threads per row scan the row's columns, then a shuffle reduction
      constexpr int TPR0 = NT / TR;
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
          g.amax_val[(size_t)m * ncg + cg] = best;
          g.amax_idx[(size_t)m * ncg + cg] = bi;
        }
      }
    } else if constexpr (E == GemmEpi::kHeadNormRope || E == GemmEpi::kKvScatter) {
      // one head per column group; one wave per row; lane i < D/2 owns the pair (i, i + D/2)
      const int half = TC / 2;
      const bool own = lane < half;
      const int i1 = own ? lane : 0;
      for (int row = wave; row < TR; row += NW) {
        const int m = m0 + row;
        if (m >= g.M) break;
        head_epilogue<T, E>(g, cg, m, fin[row * TC + i1], fin[row * TC + i1 + half], own, i1, TC);
      }
    }
  }  // column groups of this work-group
}


// ---- Many rows (M > 64): LDS-tiled MFMA GEMM. A work-group computes a BM x BN tile of
//      C = A W^T (128 x 128 with 64 x 64 per wave, or 64 x 256 with 32 x 128 per wave; 2 x 2
//      waves) and walks K in steps of 32. A first pass (split_rows_kernel) normalises the
//      fp32 activation rows (norm on load) and splits them into a (hi, lo) pair of bf16
//      planes (17 significant bits of each value) once, not once per column tile (the LM
//      head takes the hi plane alone, see gemm_plan); the weight and activation tiles then go
//      through registers into LDS, the loads of two steps in flight while a step's MFMAs run.
//      The LDS tiles are [rows][32] bf16 with the 16-byte chunks of a row XOR-swizzled by
//      (row / 4) % 4, so the 16 rows of a fragment read fall on distinct banks. The tile then
//      goes through LDS to the epilogue in two halves (fp32 store / residual add with per-tile
//      row sums of squares, SwiGLU, per-tile argmax, the head epilogues), which keeps a
//      work-group at 48 KiB of LDS: three fit on a CU. With fewer tiles than CUs, or to keep a
//      wide weight tile within one XCD's L2, K is split over work-groups and the last split of
//      a tile reduces. Work-group order puts every row tile (and split) of a column tile on one
//      XCD, back to back, so the weight tile is read from HBM once per column tile.
constexpr int kTileK = 32;
// LDS of a BM x BN tile (128 x 128, or 64 x 256): two A buffers (hi and lo planes), two W
// buffers, and the epilogue's half tile (BM / 2 rows of BN + 4 floats) over them
template <int BM, int BN> struct TileLds {
  static constexpr int kABytes = 2 * BM * kTileK * 2;  // A hi + A lo of one step
  static constexpr int kWBytes = BN * kTileK * 2;      // W of one step
  static constexpr int kW = 2 * kABytes;               // W slots follow the two A buffers
  static constexpr int kFinStride = BN + 4;            // floats per row of the epilogue tile
  static constexpr size_t bytes() {
    return (size_t)kW + 2 * kWBytes > (size_t)BM / 2 * kFinStride * 4 ? (size_t)kW + 2 * kWBytes
                                                                       : (size_t)BM / 2 * kFinStride * 4;
  }
};

// a SwiGLU output element o = m * N + n: fp32, or its (hi, lo) bf16 planes for a consumer that
// takes the pair (the down projection with many rows), exactly as split_rows_kernel splits
__device__ __forceinline__ void store_swiglu(const GemmArgs &g, size_t o, float v) {
  if (g.out_planes) {
    const uint16_t h = f32_to_bf16(v);
    g.out_planes[o] = h;
    g.out_planes[(size_t)g.M * g.N + o] = f32_to_bf16(v - bf16_to_f32(h));
  } else {
    g.out[o] = v;
  }
}

// two adjacent SwiGLU output elements o, o + 1 (o even, N even: 4- or 8-byte aligned) in one
// store per plane; the pairs convert with v_cvt_pk_bf16_f32, whose round to nearest even gives
// the same bits as f32_to_bf16 (NaN aside)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store_swiglu2(const GemmArgs &g, size_t o, float v0, float v1) {
  if (g.out_planes) {
    const bf16x2_t h = __builtin_convertvector(f32x2_t{v0, v1}, bf16x2_t);
    const float h0 = (float)h[0], h1 = (float)h[1];
    const bf16x2_t l = __builtin_convertvector(f32x2_t{v0 - h0, v1 - h1}, bf16x2_t);
    __builtin_memcpy(g.out_planes + o, &h, 4);
    __builtin_memcpy(g.out_planes + (size_t)g.M * g.N + o, &l, 4);
  } else {
    *reinterpret_cast<float2 *>(g.out + o) = make_float2(v0, v1);
  }
}

__device__ __forceinline__ int tile_swz(int row, int c) { return row * 64 + ((c ^ ((row >> 2) & 3)) << 4); }

// The activations of the tiled GEMM, once per launch: row m of A (the kept rows of the block
// for the LM head), normalised when the GEMM norms on load (also written to a_out), split into
// two bf16 planes hi [M][K] = bf16(f) and lo [M][K] = bf16(f - hi): hi + lo is the fp32
// value f to 17 significant bits (relative error at most 2^-17). lo == nullptr: the hi plane
// alone (a GEMM that takes bf16(f)).
__global__ __launch_bounds__(256) void split_rows_kernel(GemmArgs g, uint16_t *__restrict__ hi,
                                                         uint16_t *__restrict__ lo) {
  __shared__ float red[16];
  const int m = blockIdx.x, K = g.K;
  const int sr = g.keep_bs > 0 ? (m / (g.keep_bs - 1)) * g.keep_bs + m % (g.keep_bs - 1) + 1 : m;
  const bool norm = g.norm_w != nullptr;
  float inv = 1.f;
  if (norm) {
    float ss = 0.f;
    for (int q = threadIdx.x; q < g.ss_groups; q += blockDim.x) ss += g.ss[(size_t)q * g.ss_rows + sr];
    inv = rsqrtf(block_sum(ss, red) / (float)K + g.eps);
  }
  const float *a = reinterpret_cast<const float *>(g.a[0]) + (size_t)sr * g.lda;
  for (int k = threadIdx.x * 8; k < K; k += blockDim.x * 8) {
    float f[8];
    const Vec16 v0 = load_vec16(a + k), v1 = load_vec16(a + k + 4);
    __builtin_memcpy(f, &v0.u, 16);
    __builtin_memcpy(f + 4, &v1.u, 16);
    if (norm) {
      const Vec16 wv = load_vec16(reinterpret_cast<const uint16_t *>(g.norm_w) + k);
      uint16_t w[8];
      __builtin_memcpy(w, &wv.u, 16);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = f[e] * inv * bf16_to_f32(w[e]);
    }
    if (g.a_out)
#pragma unroll
      for (int e = 0; e < 8; ++e) g.a_out[(size_t)m * K + k + e] = f[e];
    uint16_t h[8], l[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      h[e] = f32_to_bf16(f[e]);
      l[e] = f32_to_bf16(f[e] - bf16_to_f32(h[e]));
    }
    __builtin_memcpy(hi + (size_t)m * K + k, h, 16);
    if (lo) __builtin_memcpy(lo + (size_t)m * K + k, l, 16);
  }
}

// kLo: A = the (hi, lo) planes from split_rows_kernel (g.a[0], g.a[1], row stride K), two
// MFMAs per step. Otherwise A is bf16 as given (the auxiliary target states): g.a_nseg equal
// K segments g.a[s] with row stride g.lda, each a multiple of the K step, one MFMA per step.
template <GemmEpi E, bool kLo, int BM, int BN>
__global__ __launch_bounds__(256, 3) void gemm_tiled_kernel(GemmArgs g, int mtiles, int ntiles, int splits) {
  constexpr int BK = kTileK, NT = 256;
  constexpr int WM = BM / 2, WN = BN / 2;    // wave tile (2 x 2 waves)
  constexpr int TF = WM / 16, UN = WN / 16;  // MFMA row and column tiles per wave
  constexpr int JA = BM / 64, JW = BN / 64;  // 16-byte A (per plane) and W chunks per thread and K step
  constexpr int FS = TileLds<BM, BN>::kFinStride, kTileABytes = TileLds<BM, BN>::kABytes;
  constexpr int kTileW = TileLds<BM, BN>::kW, kTileWBytes = TileLds<BM, BN>::kWBytes;
  constexpr bool kDual = E == GemmEpi::kSwiGLU;
  constexpr int OC = kDual ? BN / 2 : BN;  // output columns of a tile (SwiGLU: BN/2 gate + BN/2 up rows)
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ unsigned s_flag;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  // work-group -> (column tile, row tile, K split): consecutive work-groups of one XCD (ids
  // congruent mod 8) walk the row tiles and splits of one column tile
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int nt = (slot / (mtiles * splits)) * 8 + xcd, mt = slot % mtiles, sp = (slot / mtiles) % splits;
  if (nt >= ntiles) return;
  const int m0 = mt * BM, n0 = nt * OC;
  const int K = g.K;
  constexpr int NLD = (kLo ? 2 : 1) * JA + JW;  // 16-byte loads per thread and K step
  const int kseg = K / g.a_nseg;                // bf16 A: K columns per segment
  // Loads of one K step, per thread: JA 16-byte chunks of activation rows (hi and lo each)
  // and JW of weight rows; chunk slot j of wave w is tile row (4 j + w) * 16 + lane / 4. Tile
  // row r's chunk c is stored at tile_swz(r, c); thread slot (row, stored chunk lane % 4)
  // holds source chunk (lane % 4) ^ swz(row).
  const uint16_t *brow[JW], *ahi[JA], *alo[JA];
  size_t aoff[JA];
  int bsrc[JW], asrc[JA];
#pragma unroll
  for (int j = 0; j < JW; ++j) {
    const int r = (j * 4 + wave) * 16 + (lane >> 2);
    // weight row of tile row r (a row past N reads a valid row; its results are never stored)
    const int n = min(n0 + (kDual ? (r & (OC - 1)) : r), g.N - 1);
    int seg = 0, nbase = 0;
    if (!kDual)
      while (seg < g.b_nseg - 1 && n >= g.b_end[seg]) nbase = g.b_end[seg++];
    brow[j] = reinterpret_cast<const uint16_t *>(kDual ? g.b[r < OC ? 0 : 1] : g.b[seg]) + (size_t)(n - nbase) * K;
    bsrc[j] = ((lane & 3) ^ ((r >> 2) & 3)) * 8;
  }
#pragma unroll
  for (int j = 0; j < JA; ++j) {
    const int r = (j * 4 + wave) * 16 + (lane >> 2);
    asrc[j] = ((lane & 3) ^ ((r >> 2) & 3)) * 8;
    const int am = min(m0 + r, g.M - 1);  // rows past M: a valid row, never stored
    aoff[j] = (size_t)am * (kLo ? (size_t)K : (size_t)g.lda);
    ahi[j] = reinterpret_cast<const uint16_t *>(g.a[0]) + aoff[j];
    alo[j] = reinterpret_cast<const uint16_t *>(g.a[kLo ? 1 : 0]) + aoff[j];
  }
  // Two steps ahead: step s + 2 loads into register set s % 2 while step s computes; the LDS
  // tiles are double buffered. Every iteration issues the same six loads (the K offset clamped
  // past the end), so a fixed count of loads stays in flight. (No LDS DMA here: after one the
  // compiler must assume every LDS read depends on it and waits for all loads in flight.)
  Vec16 aregs[2][2][JA], wregs[2][JW];  // [set][hi, lo][j], [set][j]
  auto load = [&](int set, int k0) {
    if constexpr (!kLo) {  // the segment of the concatenated A holding columns [k0, k0 + BK)
      const int seg = k0 / kseg;
      const uint16_t *a0 = reinterpret_cast<const uint16_t *>(g.a[seg]) + (k0 - seg * kseg);
#pragma unroll
      for (int j = 0; j < JA; ++j) aregs[set][0][j] = load_vec16(a0 + aoff[j] + asrc[j]);
    } else {
#pragma unroll
      for (int j = 0; j < JA; ++j) {
        aregs[set][0][j] = load_vec16(ahi[j] + k0 + asrc[j]);
        aregs[set][1][j] = load_vec16(alo[j] + k0 + asrc[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < JW; ++j) wregs[set][j] = load_vec16(brow[j] + k0 + bsrc[j]);
  };
  auto store = [&](int set, int buf) {
#pragma unroll
    for (int j = 0; j < JA; ++j) {
      const int o = (j * 4 + wave) * 1024 + lane * 16;
      *reinterpret_cast<uint4 *>(smem + buf * kTileABytes + o) = aregs[set][0][j].u;
      if constexpr (kLo) *reinterpret_cast<uint4 *>(smem + buf * kTileABytes + BM * BK * 2 + o) = aregs[set][1][j].u;
    }
#pragma unroll
    for (int j = 0; j < JW; ++j)
      *reinterpret_cast<uint4 *>(smem + kTileW + buf * kTileWBytes + (j * 4 + wave) * 1024 + lane * 16) = wregs[set][j].u;
  };
  // vmcnt(NLD): the newest step's loads may stay in flight
  static_assert(NLD <= 15, "vmcnt field");
  constexpr unsigned kWaitOlder = 0x0F70u | (unsigned)NLD;

  f32x4_t acc[TF][UN];
#pragma unroll
  for (int t = 0; t < TF; ++t)
#pragma unroll
    for (int u = 0; u < UN; ++u) acc[t][u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // this split's K steps [ks0, ks0 + nk) of the K / BK (splits of near-equal length)
  const int ks0 = (int)((long)sp * (K / BK) / splits), nk = (int)((long)(sp + 1) * (K / BK) / splits) - ks0;
  auto kof = [&](int step) { return (ks0 + min(step, nk - 1)) * BK; };
  load(0, kof(0));
  load(1, kof(1));
  __builtin_amdgcn_s_waitcnt(kWaitOlder);  // step 0 has landed, step 1 in flight
  store(0, 0);
  __syncthreads();
  // one K step; the register set is a compile-time constant (the loop is unrolled by two), so
  // the loads stay in flight across the MFMAs instead of being waited for to index registers
  auto step = [&](auto set_c, int ks) {
    constexpr int set = decltype(set_c)::value;
    load(set, kof(ks + 2));  // set ks % 2 held step ks, already in LDS
    const unsigned char *sa = smem + set * kTileABytes;
    const unsigned char *sw = smem + kTileW + set * kTileWBytes;
    Vec16 bf[UN];
#pragma unroll
    for (int u = 0; u < UN; ++u) bf[u].u = *reinterpret_cast<const uint4 *>(sw + tile_swz(wn * WN + u * 16 + (lane & 15), lane >> 4));
#pragma unroll
    for (int t = 0; t < TF; ++t) {
      const int o = tile_swz(wm * WM + t * 16 + (lane & 15), lane >> 4);
      Vec16 ah, al;
      ah.u = *reinterpret_cast<const uint4 *>(sa + o);
      if constexpr (kLo) al.u = *reinterpret_cast<const uint4 *>(sa + BM * BK * 2 + o);
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        mma16<uint16_t>(acc[t][u], ah, bf[u]);
        if constexpr (kLo) mma16<uint16_t>(acc[t][u], al, bf[u]);
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitOlder);  // step ks + 1's register set has landed
    if (ks + 1 < nk) store(set ^ 1, set ^ 1);
    __syncthreads();
  };
  int ks = 0;
  for (; ks + 1 < nk; ks += 2) {
    step(std::integral_constant<int, 0>{}, ks);
    step(std::integral_constant<int, 1>{}, ks + 1);
  }
  if (ks < nk) step(std::integral_constant<int, 0>{}, ks);
  __builtin_amdgcn_s_waitcnt(0);  // the clamped loads past the end

  // ---- the tile through LDS in two halves of 64 rows (the waves with wm == h own half h),
  //      so the epilogue needs half the LDS of the tile and three work-groups fit on a CU.
  //      MFMA layout: lane holds rows (lane / 16) * 4 + i, column lane % 16.
  constexpr int HM = BM / 2;
  constexpr int TPR = NT / HM;  // threads per row of a half tile in the row-wise epilogues
  float *fin = reinterpret_cast<float *>(smem);
  auto acc_to_fin = [&](int h) {
    if (wm == h)
#pragma unroll
      for (int t = 0; t < TF; ++t)
#pragma unroll
        for (int u = 0; u < UN; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            fin[(t * 16 + (lane >> 4) * 4 + i) * FS + wn * WN + u * 16 + (lane & 15)] = acc[t][u][i];
  };
  // ---- split-K: every split stores its tile ([split][row tile][column tile] blocks of
  //      BM x BN in the workspace) and the last to arrive sums all splits in split order, with
  //      the device-scope relaxed atomic accesses and store-complete-before-arrival protocol of
  //      the streaming kernel.
  const size_t tstride = (size_t)mtiles * ntiles * BM * BN;
  const size_t tbase = ((size_t)mt * ntiles + nt) * BM * BN;
  if (splits > 1) {
    float *mine = g.part + (size_t)sp * tstride + tbase;
    for (int h = 0; h < 2; ++h) {
      __syncthreads();
      acc_to_fin(h);
      __syncthreads();
      for (int e = threadIdx.x; e < HM * BN; e += NT)
        __hip_atomic_store(mine + h * HM * BN + e, fin[(e / BN) * FS + e % BN], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores are acknowledged
    __syncthreads();
    unsigned *ctr = g.counters + (size_t)mt * ntiles + nt;
    if (threadIdx.x == 0) s_flag = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (s_flag != (unsigned)(splits - 1)) return;  // another split finishes this tile
    if (threadIdx.x == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // the piece's sums of every split into fin (last split to arrive), or the work-group's own
  // accumulators; then the epilogue. Two loops, so that the accumulators are dead while the
  // reduce has its loads in flight.
  auto reduce_to_fin = [&](int h) {
    // 8 elements x 8 splits of loads in flight per round trip (every load issued: past the
    // last split the address is the last split's, its value dropped), summed in split order
    constexpr int EPT = HM * BN / NT;  // elements of the piece per thread
    static_assert(EPT * NT == HM * BN && EPT % 8 == 0, "reduce chunks");
    for (int j0 = 0; j0 < EPT; j0 += 8) {
      float sum[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) sum[jj] = 0.f;
      for (int q0 = 0; q0 < splits; q0 += 8) {
        float v[8][8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
#pragma unroll
          for (int u = 0; u < 8; ++u)
            v[jj][u] = __hip_atomic_load(g.part + tbase + h * HM * BN + threadIdx.x + (j0 + jj) * NT +
                                             (size_t)min(q0 + u, splits - 1) * tstride,
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (q0 + u < splits) sum[jj] += v[jj][u];
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int e = threadIdx.x + (j0 + jj) * NT;
        fin[(e / BN) * FS + e % BN] = sum[jj];
      }
    }
  };
  auto epilogue = [&](int h) {
    const int mh = m0 + h * HM;  // first output row of this piece
    if constexpr (E == GemmEpi::kStore || E == GemmEpi::kResidAdd) {
      for (int e = threadIdx.x; e < HM * BN; e += NT) {
        const int row = e / BN, col = e % BN;
        const int m = mh + row, n = n0 + col;
        float v = fin[row * FS + col];
        if (m < g.M && n < g.N) {
          const size_t o = (size_t)m * g.N + n;
          if (E == GemmEpi::kResidAdd) v += g.out[o];
          g.out[o] = v;
        } else {
          v = 0.f;
        }
        fin[row * FS + col] = v * v;
      }
      if (g.ss_out) {  // per-row sum of squares over this column tile, for norm on load
        __syncthreads();
        const int row = threadIdx.x / TPR, sub = threadIdx.x % TPR;
        float sq = 0.f;
        for (int c = sub; c < BN; c += TPR) sq += fin[row * FS + c];
  #pragma unroll
        for (int o = 1; o < TPR; o <<= 1) sq += __shfl_xor(sq, o, 64);
        if (sub == 0 && mh + row < g.M) g.ss_out[(size_t)nt * g.M + mh + row] = sq;
      }
    } else if constexpr (E == GemmEpi::kSwiGLU) {
      static_assert(OC % 2 == 0, "column pairs");
      for (int e = threadIdx.x * 2; e < HM * OC; e += NT * 2) {  // two adjacent columns a thread
        const int row = e / OC, col = e % OC;
        const int m = mh + row, n = n0 + col;
        if (m < g.M && n < g.N) {
          const float g0 = fin[row * FS + col], u0 = fin[row * FS + OC + col];
          const float v0 = g0 / (1.f + expf(-g0)) * u0;
          if (n + 1 < g.N && (g.N & 1) == 0) {
            const float g1 = fin[row * FS + col + 1], u1 = fin[row * FS + OC + col + 1];
            store_swiglu2(g, (size_t)m * g.N + n, v0, g1 / (1.f + expf(-g1)) * u1);
          } else {
            store_swiglu(g, (size_t)m * g.N + n, v0);
            if (n + 1 < g.N) {
              const float g1 = fin[row * FS + col + 1], u1 = fin[row * FS + OC + col + 1];
              store_swiglu(g, (size_t)m * g.N + n + 1, g1 / (1.f + expf(-g1)) * u1);
            }
          }
        }
      }
    } else if constexpr (E == GemmEpi::kArgmax) {
      const int row = threadIdx.x / TPR, sub = threadIdx.x % TPR;
      float best = -INFINITY;
      int bi = 0x7fffffff;
      for (int c = sub; c < BN; c += TPR)
        if (n0 + c < g.N) argmax_merge(best, bi, fin[row * FS + c], n0 + c);
  #pragma unroll
      for (int o = 1; o < TPR; o <<= 1) {
        const float ov = __shfl_xor(best, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        argmax_merge(best, bi, ov, oi);
      }
      if (sub == 0 && mh + row < g.M) {
        g.amax_val[(size_t)(mh + row) * ntiles + nt] = best;
        g.amax_idx[(size_t)(mh + row) * ntiles + nt] = bi;
      }
    } else {  // head epilogues: BN / D heads per tile row, one (row, head) per wave at a time
      const int D = g.head_dim, half = D / 2, hpt = BN / D;
      const bool own = lane < half;
      const int i1 = own ? lane : 0;
      for (int q = wave; q < HM * hpt; q += NT / 64) {
        const int row = q / hpt, hh = q % hpt, m = mh + row;
        if (m >= g.M) break;
        if (n0 + hh * D >= g.N) continue;
        head_epilogue<uint16_t, E>(g, n0 / D + hh, m, fin[row * FS + hh * D + i1],
                                   fin[row * FS + hh * D + i1 + half], own, i1, D);
      }
    }
  };
  if (splits > 1) {
    for (int h = 0; h < 2; ++h) {
      __syncthreads();  // the previous piece's epilogue is done with the LDS tile
      reduce_to_fin(h);
      __syncthreads();
      if (m0 + h * HM >= g.M) break;  // rows past M: nothing to store (uniform)
      epilogue(h);
    }
  } else {
    for (int h = 0; h < 2; ++h) {
      __syncthreads();
      acc_to_fin(h);
      __syncthreads();
      if (m0 + h * HM >= g.M) break;
      epilogue(h);
    }
  }
}

// ---- Wide tiles, one work-group per CU: a 256 x 256 output tile. Eight waves (4 x 2) of
//      64 x 128 with v_mfma_f32_32x32x16_bf16 (128 accumulators per lane), two waves per SIMD;
//      K in steps of 32 with three steps in flight (register sets and LDS buffers, XOR-swizzled
//      row-major tiles as above). A work-group loads 2.5 times fewer bytes per flop than a
//      64 x 256 tile, which is what bounds the smaller tile: its loads at full MFMA rate would
//      exceed what a CU's vector-memory path delivers. A is the bf16 plane of fp32 rows (the LM
//      head and gate|up with many rows; never K-split), bf16 rows read in place in K segments
//      (fc over the auxiliary target states), or the (hi, lo) pair of fp32 rows (the down
//      projection at batch 128: two MFMAs per fragment, two K steps in flight). With fewer
//      tiles than CUs, K is split over work-groups and the last split of a tile reduces, as in
//      the tiled kernel. The tile then goes through LDS in four pieces of 64 rows to the SwiGLU,
//      per-tile argmax, or store / residual add (with per-tile row sums of squares) epilogue.
typedef float f32x16_t __attribute__((ext_vector_type(16)));
constexpr int kWideM = 256, kWideN = 256, kWideWaves = 8, kWidePiece = 64;
constexpr int kWideStages = 3;
constexpr size_t kWideLds = (size_t)kWideStages * (kWideM + kWideN) * kTileK * 2;
constexpr size_t kWideLdsPair = (size_t)2 * (2 * kWideM + kWideN) * kTileK * 2;

template <GemmEpi E, bool kSeg, bool kLo>
__global__ __launch_bounds__(kWideWaves * 64, 1) void gemm_wide_kernel(GemmArgs g, int mtiles, int ntiles, int nsplit) {
  static_assert(kSeg ? E == GemmEpi::kStore
                     : kLo ? E == GemmEpi::kResidAdd : (E == GemmEpi::kSwiGLU || E == GemmEpi::kArgmax),
                "wide tile epilogues");
  constexpr int BM = kWideM, BN = kWideN, BK = kTileK, NS = kLo ? 2 : kWideStages, HM = kWidePiece;
  constexpr int NT = kWideWaves * 64, NW = kWideWaves, WR = 4, WC = 2;
  constexpr int WM = BM / WR, WN = BN / WC, TF = WM / 32, UN = WN / 32;  // 32 x 32 MFMA tiles per wave
  constexpr int JA = BM * 4 / NT, JW = BN * 4 / NT;                  // 16-byte loads per thread, plane and step
  constexpr int NLD = (kLo ? 2 : 1) * JA + JW;
  static_assert(JA * NT == BM * 4 && JW * NT == BN * 4 && HM == WM, "one epilogue piece per wave row");
  constexpr size_t kPlane = (size_t)BM * BK * 2, kAB = (kLo ? 2 : 1) * kPlane, kWB = (size_t)BN * BK * 2;
  static_assert((size_t)HM * (BN + 4) * 4 <= kWideLds, "epilogue piece fits the K-loop buffers");
  constexpr bool kDual = E == GemmEpi::kSwiGLU;
  constexpr int OC = kDual ? BN / 2 : BN;  // output columns of a tile (SwiGLU: BN/2 gate + BN/2 up rows)
  constexpr int FS = BN + 4, TPR = NT / HM;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ unsigned s_flag;
  const int splits = kSeg || kLo ? nsplit : 1;  // the bf16-plane tiles are never split
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave / WC, wn = wave % WC;
  // work-group -> (column tile, row tile, K split): the row tiles and splits of a column tile run
  // back to back on one XCD (ids congruent mod 8), sharing the weight tile through its L2
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int nt = (slot / (mtiles * splits)) * 8 + xcd, mt = slot % mtiles, sp = (slot / mtiles) % splits;
  if (nt >= ntiles) return;
  const int m0 = mt * BM, n0 = nt * OC, K = g.K;
  // load slot j of wave w: tile row (NW j + w) * 16 + lane / 4, stored chunk lane % 4, which
  // holds source chunk (lane % 4) ^ swz(row)
  size_t aoff[JA];
  const uint16_t *brow[JW];
#pragma unroll
  for (int j = 0; j < JA; ++j) {
    const int r = (j * NW + wave) * 16 + (lane >> 2);
    // rows past M: a valid row, never stored
    aoff[j] = (size_t)min(m0 + r, g.M - 1) * (kSeg ? (size_t)g.lda : (size_t)K) + ((lane & 3) ^ ((r >> 2) & 3)) * 8;
  }
#pragma unroll
  for (int j = 0; j < JW; ++j) {
    const int r = (j * NW + wave) * 16 + (lane >> 2);
    const int n = min(n0 + (kDual ? (r & (OC - 1)) : r), g.N - 1);  // rows past N: a valid row, never stored
    brow[j] = reinterpret_cast<const uint16_t *>(g.b[kDual && r >= OC ? 1 : 0]) + (size_t)n * K +
              ((lane & 3) ^ ((r >> 2) & 3)) * 8;
  }
  const uint16_t *ahi = reinterpret_cast<const uint16_t *>(g.a[0]);
  const uint16_t *alo = reinterpret_cast<const uint16_t *>(g.a[kLo ? 1 : 0]);
  Vec16 areg[NS][JA], lreg[NS][kLo ? JA : 1], wreg[NS][JW];
  const int kseg = K / g.a_nseg;  // bf16 A in segments: K columns per segment
  auto load = [&](int set, int k0) {
    if constexpr (kSeg) {  // the segment of the concatenated A holding columns [k0, k0 + BK)
      const int seg = k0 / kseg;
      const uint16_t *a0 = reinterpret_cast<const uint16_t *>(g.a[seg]) + (k0 - seg * kseg);
#pragma unroll
      for (int j = 0; j < JA; ++j) areg[set][j] = load_vec16(a0 + aoff[j]);
    } else {
#pragma unroll
      for (int j = 0; j < JA; ++j) {
        areg[set][j] = load_vec16(ahi + aoff[j] + k0);
        if constexpr (kLo) lreg[set][j] = load_vec16(alo + aoff[j] + k0);
      }
    }
#pragma unroll
    for (int j = 0; j < JW; ++j) wreg[set][j] = load_vec16(brow[j] + k0);
  };
  auto store = [&](int set) {
    unsigned char *sa = smem + set * kAB, *sw = smem + NS * kAB + set * kWB;
#pragma unroll
    for (int j = 0; j < JA; ++j) {
      *reinterpret_cast<uint4 *>(sa + (j * NW + wave) * 1024 + lane * 16) = areg[set][j].u;
      if constexpr (kLo) *reinterpret_cast<uint4 *>(sa + kPlane + (j * NW + wave) * 1024 + lane * 16) = lreg[set][j].u;
    }
#pragma unroll
    for (int j = 0; j < JW; ++j) *reinterpret_cast<uint4 *>(sw + (j * NW + wave) * 1024 + lane * 16) = wreg[set][j].u;
  };
  // vmcnt((NS - 1) NLD): the newest NS - 1 steps' loads may stay in flight
  constexpr unsigned kWaitOlder = 0x0F70u | (unsigned)((NS - 1) * NLD);
  static_assert((NS - 1) * NLD <= 15, "vmcnt field");
  f32x16_t acc[TF][UN];
#pragma unroll
  for (int t = 0; t < TF; ++t)
#pragma unroll
    for (int u = 0; u < UN; ++u) acc[t][u] = f32x16_t{};
  // this split's K steps [ks0, ks0 + nk) of the K / BK (splits of near-equal length)
  const int ks0 = (int)((long)sp * (K / BK) / splits), nk = (int)((long)(sp + 1) * (K / BK) / splits) - ks0;
  auto kof = [&](int step) { return (ks0 + min(step, nk - 1)) * BK; };  // past the end: the last step again
#pragma unroll
  for (int q = 0; q < NS; ++q) load(q, kof(q));
  __builtin_amdgcn_s_waitcnt(kWaitOlder);  // step 0 has landed, the next NS - 1 in flight
  store(0);
  __syncthreads();
  // step ks: register set and LDS buffer ks % NS, a compile-time constant (the loop is
  // unrolled by NS), so the loads stay in flight across the MFMAs
  auto step = [&](auto set_c, int ks) {
    constexpr int set = decltype(set_c)::value, nxt = (set + 1) % NS;
    load(set, kof(ks + NS));  // set ks % NS held step ks, already in LDS
    const unsigned char *sa = smem + set * kAB, *sw = smem + NS * kAB + set * kWB;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {  // 16 K values each: chunk 2 sub + lane / 32
      const int ch = sub * 2 + (lane >> 5);
      Vec16 bf[UN];
#pragma unroll
      for (int u = 0; u < UN; ++u) bf[u].u = *reinterpret_cast<const uint4 *>(sw + tile_swz(wn * WN + u * 32 + (lane & 31), ch));
#pragma unroll
      for (int t = 0; t < TF; ++t) {
        const int o = tile_swz(wm * WM + t * 32 + (lane & 31), ch);
        Vec16 ah, al;
        ah.u = *reinterpret_cast<const uint4 *>(sa + o);
        if constexpr (kLo) al.u = *reinterpret_cast<const uint4 *>(sa + kPlane + o);
        bf16x8_t av, lv;
        __builtin_memcpy(&av, &ah.u, 16);
        if constexpr (kLo) __builtin_memcpy(&lv, &al.u, 16);
#pragma unroll
        for (int u = 0; u < UN; ++u) {
          bf16x8_t bv;
          __builtin_memcpy(&bv, &bf[u].u, 16);
          acc[t][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[t][u], 0, 0, 0);
          if constexpr (kLo) acc[t][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lv, bv, acc[t][u], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitOlder);  // step ks + 1 has landed
    if (ks + 1 < nk) store(nxt);
    __syncthreads();
  };
  int ks = 0;
  for (; ks + NS - 1 < nk; ks += NS) {  // unrolled by NS (two or three)
    step(std::integral_constant<int, 0>{}, ks);
    step(std::integral_constant<int, 1>{}, ks + 1);
    if constexpr (NS > 2) step(std::integral_constant<int, 2 % NS>{}, ks + 2);
  }
  if (ks < nk) step(std::integral_constant<int, 0>{}, ks);
  if (NS > 2 && ks + 1 < nk) step(std::integral_constant<int, 1>{}, ks + 1);
  __builtin_amdgcn_s_waitcnt(0);  // the clamped loads past the end

  // ---- the tile through LDS, one piece of 64 rows at a time: piece h is held by the waves
  //      with wm == h. 32 x 32 MFMA layout: lane holds column lane % 32, rows
  //      8 (i / 4) + 4 (lane / 32) + i % 4.
  float *fin = reinterpret_cast<float *>(smem);
  auto acc_to_fin = [&](int h) {
    if (wm == h)
#pragma unroll
      for (int t = 0; t < TF; ++t)
#pragma unroll
        for (int u = 0; u < UN; ++u)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            fin[(t * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3)) * FS + wn * WN + u * 32 + (lane & 31)] = acc[t][u][i];
  };
  // ---- split-K: every split stores its tile ([split][row tile][column tile] blocks of
  //      BM x BN in the workspace) and the last to arrive sums all splits in split order, with
  //      the device-scope relaxed atomic accesses and store-complete-before-arrival protocol of
  //      the streaming kernel.
  const size_t tstride = (size_t)mtiles * ntiles * BM * BN;
  const size_t tbase = ((size_t)mt * ntiles + nt) * BM * BN;
  if (splits > 1) {
    float *mine = g.part + (size_t)sp * tstride + tbase;
    for (int h = 0; h < BM / HM; ++h) {
      __syncthreads();
      acc_to_fin(h);
      __syncthreads();
      for (int e = threadIdx.x; e < HM * BN; e += NT)
        __hip_atomic_store(mine + h * HM * BN + e, fin[(e / BN) * FS + e % BN], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores are acknowledged
    __syncthreads();
    unsigned *ctr = g.counters + (size_t)mt * ntiles + nt;
    if (threadIdx.x == 0) s_flag = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (s_flag != (unsigned)(splits - 1)) return;  // another split finishes this tile
    if (threadIdx.x == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // the piece's sums of every split into fin (last split to arrive), or the work-group's own
  // accumulators; then the epilogue. Two loops, so that the accumulators are dead while the
  // reduce has its loads in flight.
  auto reduce_to_fin = [&](int h) {
    // 8 elements x 8 splits of loads in flight per round trip (every load issued: past the
    // last split the address is the last split's, its value dropped), summed in split order
    constexpr int EPT = HM * BN / NT;  // elements of the piece per thread
    static_assert(EPT * NT == HM * BN && EPT % 8 == 0, "reduce chunks");
    for (int j0 = 0; j0 < EPT; j0 += 8) {
      float sum[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) sum[jj] = 0.f;
      for (int q0 = 0; q0 < splits; q0 += 8) {
        float v[8][8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
#pragma unroll
          for (int u = 0; u < 8; ++u)
            v[jj][u] = __hip_atomic_load(g.part + tbase + h * HM * BN + threadIdx.x + (j0 + jj) * NT +
                                             (size_t)min(q0 + u, splits - 1) * tstride,
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (q0 + u < splits) sum[jj] += v[jj][u];
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int e = threadIdx.x + (j0 + jj) * NT;
        fin[(e / BN) * FS + e % BN] = sum[jj];
      }
    }
  };
  auto epilogue = [&](int h) {
    const int mh = m0 + h * HM;  // first output row of this piece
    if constexpr (E == GemmEpi::kStore || E == GemmEpi::kResidAdd) {
      for (int e = threadIdx.x; e < HM * BN; e += NT) {
        const int row = e / BN, col = e % BN, m = mh + row, n = n0 + col;
        float v = fin[row * FS + col];
        if (m < g.M && n < g.N) {
          const size_t o = (size_t)m * g.N + n;
          if (E == GemmEpi::kResidAdd) v += g.out[o];
          g.out[o] = v;
        } else {
          v = 0.f;
        }
        fin[row * FS + col] = v * v;
      }
      if (g.ss_out) {  // per-row sum of squares over this column tile, for norm on load
        __syncthreads();
        const int row = threadIdx.x / TPR, sub = threadIdx.x % TPR;
        float sq = 0.f;
        for (int c = sub; c < BN; c += TPR) sq += fin[row * FS + c];
  #pragma unroll
        for (int o = 1; o < TPR; o <<= 1) sq += __shfl_xor(sq, o, 64);
        if (sub == 0 && mh + row < g.M) g.ss_out[(size_t)nt * g.M + mh + row] = sq;
      }
    } else if constexpr (E == GemmEpi::kSwiGLU) {
      for (int e = threadIdx.x * 2; e < HM * OC; e += NT * 2) {  // two adjacent columns a thread
        const int row = e / OC, col = e % OC, m = mh + row, n = n0 + col;
        if (m < g.M && n < g.N) {
          const float g0 = fin[row * FS + col], u0 = fin[row * FS + OC + col];
          const float v0 = g0 / (1.f + expf(-g0)) * u0;
          if (n + 1 < g.N && (g.N & 1) == 0) {
            const float g1 = fin[row * FS + col + 1], u1 = fin[row * FS + OC + col + 1];
            store_swiglu2(g, (size_t)m * g.N + n, v0, g1 / (1.f + expf(-g1)) * u1);
          } else {
            store_swiglu(g, (size_t)m * g.N + n, v0);
            if (n + 1 < g.N) {
              const float g1 = fin[row * FS + col + 1], u1 = fin[row * FS + OC + col + 1];
              store_swiglu(g, (size_t)m * g.N + n + 1, g1 / (1.f + expf(-g1)) * u1);
            }
          }
        }
      }
    } else {
      const int row = threadIdx.x / TPR, sub = threadIdx.x % TPR;
      float best = -INFINITY;
      int bi = 0x7fffffff;
      for (int c = sub; c < BN; c += TPR)
        if (n0 + c < g.N) argmax_merge(best, bi, fin[row * FS + c], n0 + c);
  #pragma unroll
      for (int o = 1; o < TPR; o <<= 1) {
        const float ov = __shfl_xor(best, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        argmax_merge(best, bi, ov, oi);
      }
      if (sub == 0 && mh + row < g.M) {
        g.amax_val[(size_t)(mh + row) * ntiles + nt] = best;
        g.amax_idx[(size_t)(mh + row) * ntiles + nt] = bi;
      }
    }
  };
  if (splits > 1) {
    for (int h = 0; h < BM / HM; ++h) {
      __syncthreads();  // the previous piece's epilogue is done with the LDS tile
      reduce_to_fin(h);
      __syncthreads();
      if (m0 + h * HM >= g.M) break;  // rows past M: nothing to store (uniform)
      epilogue(h);
    }
  } else {
    for (int h = 0; h < BM / HM; ++h) {
      __syncthreads();
      acc_to_fin(h);
      __syncthreads();
      if (m0 + h * HM >= g.M) break;
      epilogue(h);
    }
  }
}

// bf16 A in segments (fc over the auxiliary target states), read in place
hipError_t launch_wide_seg(const GemmArgs &g, const GemmPlan &p, hipStream_t s) {
  auto kern = gemm_wide_kernel<GemmEpi::kStore, true, false>;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kWideLds);
  if (attr != hipSuccess) return attr;
  const int ntiles = p.col_groups, mtiles = p.row_blocks;
  kern<<<(ntiles + 7) / 8 * 8 * mtiles * p.splits, kWideWaves * 64, kWideLds, s>>>(g, mtiles, ntiles, p.splits);
  return hipGetLastError();
}

// the fp32 rows as their (hi, lo) pair, then the wide-tile kernel with the residual add
hipError_t launch_wide_pair(const GemmArgs &g, const GemmPlan &p, hipStream_t s) {
  auto kern = gemm_wide_kernel<GemmEpi::kResidAdd, false, true>;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kWideLdsPair);
  if (attr != hipSuccess) return attr;
  const uint16_t *hi = g.a_split, *lo = g.a_split + (size_t)g.M * g.K;
  if (g.a_planes) {  // split by the producer
    hi = g.a_planes;
    lo = g.a_planes + (size_t)g.M * g.K;
  } else {
    split_rows_kernel<<<g.M, 256, 0, s>>>(g, g.a_split, g.a_split + (size_t)g.M * g.K);
  }
  GemmArgs t = g;
  t.a[0] = hi;
  t.a[1] = lo;
  t.a_nseg = 1;
  t.lda = g.K;
  const int ntiles = p.col_groups, mtiles = p.row_blocks;
  kern<<<(ntiles + 7) / 8 * 8 * mtiles * p.splits, kWideWaves * 64, kWideLdsPair, s>>>(t, mtiles, ntiles, p.splits);
  return hipGetLastError();
}

// the fp32 rows as their bf16 plane (norm on load), then the wide-tile kernel
template <GemmEpi E>
hipError_t launch_wide(const GemmArgs &g, const GemmPlan &p, hipStream_t s) {
  if constexpr (E != GemmEpi::kSwiGLU && E != GemmEpi::kArgmax) {
    return hipErrorInvalidValue;
  } else {
    auto kern = gemm_wide_kernel<E, false, false>;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kWideLds);
    if (attr != hipSuccess) return attr;
    uint16_t *hi = g.a_split;
    split_rows_kernel<<<g.M, 256, 0, s>>>(g, hi, nullptr);
    GemmArgs t = g;
    t.a[0] = hi;
    t.a_nseg = 1;
    t.lda = g.K;
    const int ntiles = p.col_groups, mtiles = p.row_blocks;
    kern<<<(ntiles + 7) / 8 * 8 * mtiles, kWideWaves * 64, kWideLds, s>>>(t, mtiles, ntiles, 1);
    return hipGetLastError();
  }
}

template <GemmEpi E, bool kLo, int BM, int BN>
hipError_t launch_tiled_shape(const GemmArgs &g, const GemmPlan &p, hipStream_t s) {
  auto kern = gemm_tiled_kernel<E, kLo, BM, BN>;
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                          kMaxLds - 1024);
  if (attr != hipSuccess) return attr;
  const int ntiles = p.col_groups, mtiles = p.row_blocks;
  GemmArgs t = g;
  if constexpr (kLo) {
    const uint16_t *hi = g.a_split, *lo = g.a_split + (size_t)g.M * g.K;
    if (g.a_planes && !p.hi_only) {  // split by the producer
      hi = g.a_planes;
      lo = g.a_planes + (size_t)g.M * g.K;
    } else {
      split_rows_kernel<<<g.M, 256, 0, s>>>(g, g.a_split, p.hi_only ? nullptr : g.a_split + (size_t)g.M * g.K);
    }
    t.a[0] = hi;
    t.a[1] = lo;
    t.a_nseg = 1;
    if (p.hi_only) {
      // the bf16 plane alone, as a single-segment bf16 A
      t.lda = g.K;
      auto kern1 = gemm_tiled_kernel<E, false, BM, BN>;
      static const hipError_t attr1 = hipFuncSetAttribute(
          reinterpret_cast<const void *>(kern1), hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds - 1024);
      if (attr1 != hipSuccess) return attr1;
      kern1<<<(ntiles + 7) / 8 * 8 * mtiles * p.splits, 256, TileLds<BM, BN>::bytes(), s>>>(t, mtiles, ntiles,
                                                                                            p.splits);
      return hipGetLastError();
    }
  }
  kern<<<(ntiles + 7) / 8 * 8 * mtiles * p.splits, 256, TileLds<BM, BN>::bytes(), s>>>(t, mtiles, ntiles,
                                                                                         p.splits);
  return hipGetLastError();
}

template <GemmEpi E, bool kLo>
hipError_t launch_tiled(const GemmArgs &g, const GemmPlan &p, hipStream_t s) {
  if (p.tile_m == kWideM) {  // bf16 plane (SwiGLU, argmax), fc's bf16 segments, or the pair (residual add)
    if constexpr (E == GemmEpi::kStore && !kLo)
      return launch_wide_seg(g, p, s);
    else if constexpr (E == GemmEpi::kResidAdd)
      return launch_wide_pair(g, p, s);
    else
      return launch_wide<E>(g, p, s);
  }
  return p.tile_n == 256 ? launch_tiled_shape<E, kLo, 64, 256>(g, p, s) : launch_tiled_shape<E, kLo, 128, 128>(g, p, s);
}

template <typename T, int MT, int CW, int CT, int KW, GemmEpi E, bool kAF32>
size_t lds_bytes(const GemmArgs &g) {
  constexpr int KPV = Storage<T>::kPerVec;
  const size_t a = kAF32 && MT == 1 ? (size_t)16 * dma_row_bytes(g.kp) + dma_w_bytes(g.kp)
                                        : (size_t)16 * MT * (g.kp + KPV) * sizeof(T) * (kAF32 ? 2 : 1);
  const int nacc = E == GemmEpi::kSwiGLU ? 2 : 1;
  const size_t r = ((size_t)CW * KW * nacc * CT * 256 + (size_t)nacc * 16 * MT * 16 * CW * CT) * sizeof(float);
  return a + r;
}

template <typename T, int MT, int CW, int CT, int KW, int NCG, GemmEpi E, bool kMultiA, bool kAF32>
hipError_t launch_k(const GemmArgs &g, int splits, int grid_x, hipStream_t s) {
  auto kern = gemm_kernel<T, MT, CW, CT, KW, NCG, E, kMultiA, kAF32>;
  // allow the dynamic LDS of a work-group that has the CU to itself (set once per instance)
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                          kMaxLds - 1024);
  if (attr != hipSuccess) return attr;
  const size_t lds = lds_bytes<T, MT, CW, CT, KW, E, kAF32>(g);
  if (lds > (size_t)kMaxLds - 1024) return hipErrorInvalidValue;
  const int ncg = (g.N + 16 * CW * CT - 1) / (16 * CW * CT);
  const int gx = grid_x > 0 && grid_x < ncg ? grid_x : ncg;
  if ((long)gx * NCG < ncg) return hipErrorInvalidValue;  // every column group has a work-group
  dim3 grid(gx, splits, (g.M + 16 * MT - 1) / (16 * MT));
  kern<<<grid, CW * KW * 64, lds, s>>>(g);
  return hipGetLastError();
}

template <typename T, GemmEpi E, bool kMultiA, bool kAF32, int CW, int CT, int KW>
hipError_t launch_mt(const GemmArgs &g, const GemmPlan &p, hipStream_t s) {
  switch (gemm_mt(g.M)) {
    case 1: return launch_k<T, 1, CW, CT, KW, 1, E, kMultiA, kAF32>(g, p.splits, 0, s);
    case 2: return launch_k<T, 2, CW, CT, KW, 1, E, kMultiA, kAF32>(g, p.splits, 0, s);
    case 3: return launch_k<T, 3, CW, CT, KW, 1, E, kMultiA, kAF32>(g, p.splits, 0, s);
    default: return launch_k<T, 4, CW, CT, KW, 1, E, kMultiA, kAF32>(g, p.splits, 0, s);
  }
}

// The work-group shapes the plan can choose (instantiated kernels).
template <typename T, GemmEpi E, bool kMultiA, bool kAF32>
hipError_t launch_t(const GemmArgs &g, const GemmPlan &p, hipStream_t s) {
#define DFLASH_SHAPE(X, Y, Z) \
  if (p.cw == X && p.ct == Y && p.kw == Z) return launch_mt<T, E, kMultiA, kAF32, X, Y, Z>(g, p, s);
#define DFLASH_SHAPE_MT1(X, Y, Z)                                                                \
  if (p.cw == X && p.ct == Y && p.kw == Z && mt1)                                              \
    return p.grid_x > 0 ? launch_k<T, 1, X, Y, Z, kMaxGroupsPerWg, E, kMultiA, kAF32>(g, p.splits, p.grid_x, s) \
                        : launch_k<T, 1, X, Y, Z, 1, E, kMultiA, kAF32>(g, p.splits, 0, s);
  const bool mt1 = gemm_mt(g.M) == 1;
  if constexpr (E == GemmEpi::kHeadNormRope || E == GemmEpi::kKvScatter) {
    DFLASH_SHAPE(8, 1, 1)
    DFLASH_SHAPE(4, 1, 2)
  } else {
    DFLASH_SHAPE(2, 1, 2)
    DFLASH_SHAPE_MT1(4, 1, 1)
    DFLASH_SHAPE_MT1(4, 1, 2)
    DFLASH_SHAPE_MT1(8, 1, 1)
    DFLASH_SHAPE_MT1(8, 1, 2)
  }
#undef DFLASH_SHAPE
#undef DFLASH_SHAPE_MT1
  return hipErrorInvalidValue;
}

// fp32 drafters: A and W are fp32. bf16 drafters: W is bf16 and A is either bf16 (the
// auxiliary states of injection, possibly in several segments) or fp32 (every activation).
template <typename T, bool kAF32>
hipError_t launch_dt(const GemmArgs &g, GemmEpi epi, const GemmPlan &p, hipStream_t s) {
  switch (epi) {
    case GemmEpi::kStore:
      if (g.a_nseg > 1) return launch_t<T, GemmEpi::kStore, true, false>(g, p, s);
      return launch_t<T, GemmEpi::kStore, false, kAF32>(g, p, s);
    case GemmEpi::kResidAdd: return launch_t<T, GemmEpi::kResidAdd, false, kAF32>(g, p, s);
    case GemmEpi::kSwiGLU: return launch_t<T, GemmEpi::kSwiGLU, false, kAF32>(g, p, s);
    case GemmEpi::kArgmax: return launch_t<T, GemmEpi::kArgmax, false, kAF32>(g, p, s);
    case GemmEpi::kHeadNormRope: return launch_t<T, GemmEpi::kHeadNormRope, false, kAF32>(g, p, s);
    default: return launch_t<T, GemmEpi::kKvScatter, false, kAF32>(g, p, s);
  }
}

}  // namespace

int gemm_mt(int M) { return M <= 16 ? 1 : M <= 32 ? 2 : M <= 48 ? 3 : 4; }

namespace {
int cu_count() {
  static const int n = [] {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      return 256;
    return cus;
  }();
  return n;
}
}  // namespace

// Work-group shape, K splits and column groups per work-group. At most 16 activation rows
// (one MFMA row tile) the GEMM is a pure weight stream:
//  * more column groups than CUs (the LM head): each work-group owns up to
//    kMaxGroupsPerWg column groups, stages each K pass of the activations once (passes of up
//    to ~132 KiB) and streams all its column groups per pass;
//  * fewer: split-K until there are about two work-groups per CU.
// The shapes were chosen by timing every instantiated shape and split count on the
// Qwen3-8B-shaped projections: 8 wave columns for the LM head and the long-K projections (the
// down projection, fc over the concatenated target states), 4-wave work-groups (several per
// CU) for gate|up, 4 wave columns x 2 K sub-slices otherwise. The head epilogues need
// one head per column group.
GemmPlan gemm_plan(int M, int N, int K, int head_dim, bool bf16, GemmEpi epi, bool multi_a, bool a_f32,
                   int a_segs) {
  GemmPlan p{};
  // many rows: the LDS-tiled kernel (bf16 weights; fp32 activations, or bf16 ones in
  // segments of whole K steps; a head epilogue needs whole heads in a column tile)
  const bool head_fits = (epi != GemmEpi::kHeadNormRope && epi != GemmEpi::kKvScatter) ||
                         ((head_dim == 64 || head_dim == 128) && N % head_dim == 0);
  if (M > 64 && bf16 && K % kTileK == 0 && (a_f32 ? !multi_a : (K / a_segs) % kTileK == 0 && K % a_segs == 0) &&
      head_fits) {
    p.tiled = 1;
    p.cw = 8, p.ct = 1, p.kw = 1;
    // Every column tile rereads all of A, while the row tiles of a column tile run back to
    // back on one XCD and share its weight tile through that XCD's L2 (4 MiB) when it fits.
    // 64 x 256 tiles halve the A rereads (the dominant traffic at batch 128: the LM head's A
    // is 19 MB, read once per column tile), as long as a 256-row weight tile (256 K bf16)
    // still fits the L2; longer K (fc over the concatenated states, the down projection)
    // keeps 128 x 128 tiles.
    // With up to 4 K splits a 256-row weight tile of one split fits (the down projection):
    // the splits' partials cost far less than the A rereads. (fc, whose bf16 input is half
    // the bytes, measured faster unsplit with 128 x 128 tiles.)
    int smin = 1;
    while (a_f32 && (long)256 * (K / smin) * 2 > (4L << 20) && smin < 4) ++smin;
    const bool wide = (long)256 * (K / smin) * 2 <= (4L << 20) && K / kTileK >= 32 * smin;
    p.tile_n = wide ? 256 : 128;
    if (!wide) smin = 1;
    p.tile_m = p.tile_n == 256 ? 64 : 128;
    p.col_groups = epi == GemmEpi::kSwiGLU ? (N + p.tile_n / 2 - 1) / (p.tile_n / 2) : (N + p.tile_n - 1) / p.tile_n;
    p.row_blocks = (M + p.tile_m - 1) / p.tile_m;
    // Split-K when there are fewer tiles than CUs: the split count minimising the rounds (of
    // one work-group per CU: a second one on a CU shares its LDS and matrix cores and adds
    // little) per unit of work, plus a small cost per extra split for the reduction through
    // the workspace; at least 32 K steps per split.
    // The fp32 input rows of the LM head and of gate|up enter the matrix cores as one bf16
    // plane (not a hi + lo pair): half the MFMAs and half the A tile. A CPU study on the
    // batch-128 workload (GEMM inputs rounded to bf16, one projection or a set at a time)
    // changed no draft whose top-2 logit gap is >= 1e-2 when the LM head's and gate|up's inputs
    // were rounded together (0 of 839 such drafts over four samples of 24 sequences); rounding
    // the QKV, O or down inputs as well did change some.
    p.hi_only = a_f32 && (epi == GemmEpi::kArgmax || epi == GemmEpi::kSwiGLU);
    // The bf16-plane projections take the wide 256 x 256 tile (one work-group per CU) when it
    // gives at least about one tile per CU: 2.5 times fewer loaded bytes per flop than 64 x 256
    // (at batch 128: LM head 1.71 -> 1.29 ms, gate|up 0.45 -> 0.38 ms per launch).
    if (p.hi_only && wide && smin == 1 && (long)((M + kWideM - 1) / kWideM) * p.col_groups * 4 >= 3L * cu_count()) {
      p.tile_m = kWideM;
      p.row_blocks = (M + p.tile_m - 1) / p.tile_m;
    }
    const long wgs = (long)p.col_groups * p.row_blocks, slots = cu_count();
    p.splits = smin;
    // A long K already split for the L2 (the down projection) splits further toward three
    // work-groups per CU (what the 64 x 256 kernel runs), with at least 32 K steps a split:
    // batch 32 down 0.95 -> 0.86 ms per step (6 splits). Short K (O, QKV) measured faster at
    // one work-group per CU (below).
    if (smin > 1 && p.tile_m != kWideM && wgs * smin < 3 * slots) {
      double best = 1e30;
      for (int s = smin; s <= 8 && 32 * s <= K / kTileK; ++s) {
        const double cost = (double)((wgs * s + 3 * slots - 1) / (3 * slots)) / s + 0.03 * (s - 1);
        if (cost < best - 1e-9) best = cost, p.splits = s;
      }
    }
    if (smin == 1 && wgs < slots && p.tile_m != kWideM) {  // (the wide tile is never split)
      double best = 1.0;
      for (int s = 2; s <= 8 && 32 * s <= K / kTileK; ++s) {
        const double cost = (double)((wgs * s + slots - 1) / slots) / s + 0.03 * (s - 1);
        if (cost < best - 1e-9) best = cost, p.splits = s;
      }
    }
    // The down projection (residual add, K >= 2 N) of at least four wide row tiles takes the wide
    // tile on the (hi, lo) pair, K split toward one round (batch 128: 2.11 -> 1.89 ms per step);
    // with fewer rows, and for O, the 64 x 256 tiles measured faster.
    if (!p.hi_only && a_f32 && epi == GemmEpi::kResidAdd && wide && K >= 2 * N && M > 3 * kWideM) {
      p.tile_m = kWideM;
      p.tile_n = kWideN;
      p.col_groups = (N + p.tile_n - 1) / p.tile_n;
      p.row_blocks = (M + p.tile_m - 1) / p.tile_m;
      const long tiles = (long)p.col_groups * p.row_blocks;
      double best = 1e30;
      for (int s = smin; s <= 8 && 16 * s <= K / kTileK; ++s) {
        const double cost = (double)((tiles * s + slots - 1) / slots) / s + 0.03 * (s - 1);
        if (cost < best - 1e-9) best = cost, p.splits = s;
      }
    }
    // fc (bf16 rows in K segments, more than one wide row tile) takes the wide tile too, K split
    // toward one round of work-groups (at least 64 K steps a split): batch 128 0.41 -> 0.29 ms,
    // batch 32 0.47 -> 0.40 ms per step
    if (!a_f32 && epi == GemmEpi::kStore && M > kWideM && K / kTileK >= 64) {
      p.tile_n = kWideN;
      p.tile_m = kWideM;
      p.col_groups = (N + p.tile_n - 1) / p.tile_n;
      p.row_blocks = (M + p.tile_m - 1) / p.tile_m;
      const long tiles = (long)p.col_groups * p.row_blocks;
      double best = 1e30;
      for (int s = 1; s <= 8 && 64 * s <= K / kTileK; ++s) {
        const double cost = (double)((tiles * s + slots - 1) / slots) / s + 0.03 * (s - 1);
        if (cost < best - 1e-9) best = cost, p.splits = s;
      }
    }
    return p;
  }
  const bool head = epi == GemmEpi::kHeadNormRope || epi == GemmEpi::kKvScatter;
  const int mt = gemm_mt(M);
  if (head) {
    p.cw = head_dim / 16, p.ct = 1, p.kw = 128 / head_dim;
  } else if (mt > 1) {
    p.cw = 2, p.ct = 1, p.kw = 2;
  } else if (epi == GemmEpi::kArgmax) {
    p.cw = 8, p.ct = 1, p.kw = 1;
  } else if (epi == GemmEpi::kSwiGLU) {
    p.cw = 4, p.ct = 1, p.kw = 1;
  } else if (multi_a) {
    p.cw = 8, p.ct = 1, p.kw = 2;
  } else if (epi == GemmEpi::kResidAdd && K >= 2 * N) {
    p.cw = 8, p.ct = 1, p.kw = 1;
  } else {
    p.cw = 4, p.ct = 1, p.kw = 2;
  }
  p.col_groups = (N + 16 * p.cw * p.ct - 1) / (16 * p.cw * p.ct);
  p.row_blocks = (M + 16 * mt - 1) / (16 * mt);
  p.lds_budget = kDefaultPassBytes;
  p.grid_x = 0;
  const int step = p.kw * (bf16 ? ch_of<uint16_t>() : ch_of<float>());
  const int cus = cu_count();
  if (mt == 1 && !head && p.col_groups > cus) {
    const int per = (p.col_groups + cus - 1) / cus;
    if (per <= kMaxGroupsPerWg) {
      p.grid_x = (p.col_groups + per - 1) / per;
      p.lds_budget = 136 << 10;
    }
  }
  const long wgs = (long)(p.grid_x ? p.grid_x : p.col_groups) * p.row_blocks;
  // splits toward about two work-groups per CU (three 4-wave SwiGLU ones; one for the
  // concatenated-input projection, whose activation staging is the longest)
  const long target = mt > 1                                               ? 4L * cus
                      : (p.cw * p.kw == 4 && epi == GemmEpi::kSwiGLU) ? 3L * cus
                      : multi_a                                        ? cus
                                                                       : 2L * cus;
  int s = 1;
  if (epi != GemmEpi::kArgmax && p.grid_x == 0)
    while (wgs * s * 2 <= target && K % (2 * s * step) == 0 && K / (2 * s) >= 256 && s < 64) s *= 2;
  p.splits = s;
  return p;
}

hipError_t launch_gemm(const GemmArgs &g0, bool bf16, GemmEpi epi, const GemmPlan &p, hipStream_t s) {
  ProfScope prof(g0.tag ? g0.tag : "gemm", s);
  if (p.tiled) {
    const int oc = epi == GemmEpi::kSwiGLU ? p.tile_n / 2 : p.tile_n;
    const bool head = epi == GemmEpi::kHeadNormRope || epi == GemmEpi::kKvScatter;
    const bool a_ok = g0.a_f32 ? g0.a_nseg == 1 && g0.a_split && (!(g0.norm_w || g0.a_out) || g0.ss)
                               : epi == GemmEpi::kStore && g0.a_nseg >= 1 && g0.a_nseg <= 8 &&
                                     g0.K % g0.a_nseg == 0 && (g0.K / g0.a_nseg) % kTileK == 0 && !g0.norm_w &&
                                     !g0.a_out && g0.keep_bs == 0 && g0.lda % 8 == 0;
    // planes written by the producer: the pair of rows with no norm on load or compaction; planes
    // as output: SwiGLU only
    const bool planes_ok = (!g0.a_planes || (g0.a_f32 && !p.hi_only && !g0.norm_w && !g0.a_out && !g0.keep_bs)) &&
                           (!g0.out_planes || epi == GemmEpi::kSwiGLU);
    if (!bf16 || !a_ok || !planes_ok || g0.K % kTileK || g0.M < 1 || g0.keep_bs == 1 ||
        p.col_groups != (g0.N + oc - 1) / oc ||
        p.row_blocks != (g0.M + p.tile_m - 1) / p.tile_m || !((p.tile_m == 128 && p.tile_n == 128) ||
        (p.tile_m == 64 && p.tile_n == 256) ||
        (p.tile_m == kWideM && p.tile_n == kWideN && p.hi_only && p.splits == 1 && g0.a_f32 &&
         (epi == GemmEpi::kSwiGLU || (epi == GemmEpi::kArgmax && g0.b_nseg == 1))) ||
        (p.tile_m == kWideM && p.tile_n == kWideN && !g0.a_f32 && epi == GemmEpi::kStore && g0.b_nseg == 1) ||
        (p.tile_m == kWideM && p.tile_n == kWideN && g0.a_f32 && !p.hi_only && epi == GemmEpi::kResidAdd && g0.b_nseg == 1)) || g0.b_nseg < 1 || g0.b_nseg > 3 || p.splits < 1 ||
        p.splits > g0.K / kTileK || (p.splits > 1 && (!g0.part || !g0.counters)) ||
        (head && ((g0.head_dim != 64 && g0.head_dim != 128) || g0.N % g0.head_dim)))
      return hipErrorInvalidValue;
    switch (epi) {
      case GemmEpi::kStore:
        return g0.a_f32 ? launch_tiled<GemmEpi::kStore, true>(g0, p, s) : launch_tiled<GemmEpi::kStore, false>(g0, p, s);
      case GemmEpi::kResidAdd: return launch_tiled<GemmEpi::kResidAdd, true>(g0, p, s);
      case GemmEpi::kSwiGLU: return launch_tiled<GemmEpi::kSwiGLU, true>(g0, p, s);
      case GemmEpi::kArgmax: return launch_tiled<GemmEpi::kArgmax, true>(g0, p, s);
      case GemmEpi::kHeadNormRope: return launch_tiled<GemmEpi::kHeadNormRope, true>(g0, p, s);
      case GemmEpi::kKvScatter: return launch_tiled<GemmEpi::kKvScatter, true>(g0, p, s);
      default: return hipErrorInvalidValue;
    }
  }
  const int step = p.kw * (bf16 ? ch_of<uint16_t>() : ch_of<float>());
  const int splits = p.splits;
  const bool head = epi == GemmEpi::kHeadNormRope || epi == GemmEpi::kKvScatter;
  if ((epi != GemmEpi::kStore && g0.a_nseg > 1) || g0.N % 16 || g0.K % step || splits < 1 || g0.K % splits ||
      (g0.K / splits) % step || (g0.a_nseg > 1 && (g0.K / g0.a_nseg) % (bf16 ? 8 : 4)) ||
      (splits > 1 && (!g0.part || !g0.counters)) || (head && (g0.head_dim != 64 && g0.head_dim != 128)) ||
      (head && p.cw * p.ct * 16 != g0.head_dim) || ((g0.norm_w || g0.a_out) && (g0.a_nseg > 1 || (bf16 && !g0.a_f32) || !g0.ss)) ||
      (g0.keep_bs == 1) || p.col_groups != (g0.N + 16 * p.cw * p.ct - 1) / (16 * p.cw * p.ct) ||
      g0.a_planes || g0.out_planes)  // (the streaming kernel takes and writes fp32 rows only)
    return hipErrorInvalidValue;
  GemmArgs g = g0;
  g.kt = g.K / splits;
  // K per staged pass: the split cut into equal passes that fit the LDS budget
  const int mt = gemm_mt(g.M);
  const bool af32 = bf16 && g.a_f32 && g.a_nseg == 1;
  const int esz = (bf16 && !af32) ? 2 : 4;  // LDS bytes per staged A element
  const int budget = p.lds_budget > 0 ? p.lds_budget : kDefaultPassBytes;
  const int kp_max = budget / (16 * mt * esz) / step * step;
  if (kp_max < step) return hipErrorInvalidValue;
  int npass = (g.kt + kp_max - 1) / kp_max;
  auto kp_of = [&](int np) { return ((g.kt + np - 1) / np + step - 1) / step * step; };
  g.kp = kp_of(npass);
  // DMA staging rounds rows up to whole 1 KiB segments: more passes if that overflows
  while (af32 && mt == 1 && g.kp > step && 16 * dma_row_bytes(g.kp) + dma_w_bytes(g.kp) > budget)
    g.kp = kp_of(++npass);
  if (!bf16) return launch_dt<float, false>(g, epi, p, s);
  return af32 ? launch_dt<uint16_t, true>(g, epi, p, s) : launch_dt<uint16_t, false>(g, epi, p, s);
}

}  // namespace dflash
