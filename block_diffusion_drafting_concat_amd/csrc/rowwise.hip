// Row-wise kernels of the DFlash path: block embedding, RMSNorm (with the split-K partial
// sum and the residual add folded in), q/k RMSNorm + RoPE of the block, the context K/V
// epilogue of injection (k_norm + RoPE + paged scatter), SwiGLU, the LM-head argmax
// reduction, greedy verification and the RoPE table.
//
// Every consumer of split-K GEMM partials sums them in split order, so results do not
// depend on scheduling.
#include <float.h>

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace dflash {
namespace {

// ---------------------------------------------------------------------------------------
// Block construction + embedding: row m = b*bs + j gets embed[bonus[b]] for j == 0 and
// embed[mask] otherwise, converted to the fp32 residual stream.
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const T *__restrict__ embed, int V, int H,
                                                    const int32_t *__restrict__ bonus, int bs, int mask_id,
                                                    float *__restrict__ x) {
  const int m = blockIdx.x;
  const int b = m / bs, j = m % bs;
  int id = (j == 0) ? bonus[b] : mask_id;
  id = min(max(id, 0), V - 1);
  const T *src = embed + (size_t)id * H;
  for (int i = threadIdx.x * 4; i < H; i += blockDim.x * 4) {
    float4 v;
    v.x = Storage<T>::load(src, i);
    v.y = Storage<T>::load(src, i + 1);
    v.z = Storage<T>::load(src, i + 2);
    v.w = Storage<T>::load(src, i + 3);
    *reinterpret_cast<float4 *>(x + (size_t)m * H + i) = v;
  }
}

// ---------------------------------------------------------------------------------------
// r = (x[m] or 0) + sum_s part[s][m]; x[m] = r; out = r / rms(r) * w (fp32). One work-group
// of up to 1024 threads per row; each thread owns at most kRmsVecs float4 of the row and
// the split loop is unrolled so that the partials stream in parallel.
constexpr int kRmsVecs = 4;
template <typename T>
__global__ __launch_bounds__(1024) void rmsnorm_kernel(int M, int H, float *__restrict__ x,
                                                      const float *__restrict__ part, int splits,
                                                      const T *__restrict__ w, float eps, float *__restrict__ out,
                                                      int keep_bs, float *__restrict__ hidden_out) {
  __shared__ float red[16];
  const int m = blockIdx.x;
  if (keep_bs > 0 && m % keep_bs == 0) return;  // block slot 0 is not drafted
  const int nv = H / 4;
  float4 v[kRmsVecs];
#pragma unroll
  for (int j = 0; j < kRmsVecs; ++j) {
    const int i = threadIdx.x + j * (int)blockDim.x;
    v[j] = (x && i < nv) ? reinterpret_cast<const float4 *>(x + (size_t)m * H)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll 4
  for (int s = 0; s < splits; ++s) {
    const float4 *p = reinterpret_cast<const float4 *>(part + ((size_t)s * M + m) * H);
#pragma unroll
    for (int j = 0; j < kRmsVecs; ++j) {
      const int i = threadIdx.x + j * (int)blockDim.x;
      if (i < nv) {
        const float4 q = p[i];
        v[j].x += q.x;
        v[j].y += q.y;
        v[j].z += q.z;
        v[j].w += q.w;
      }
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < kRmsVecs; ++j) ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
  ss = block_sum(ss, red);
  const float inv = rsqrtf(ss / (float)H + eps);
  const int orow = keep_bs > 0 ? (m / keep_bs) * (keep_bs - 1) + m % keep_bs - 1 : m;
#pragma unroll
  for (int j = 0; j < kRmsVecs; ++j) {
    const int i = threadIdx.x + j * (int)blockDim.x;
    if (i >= nv) break;
    if (x && splits > 0) reinterpret_cast<float4 *>(x + (size_t)m * H)[i] = v[j];
    const float e[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const size_t col = (size_t)i * 4 + c;
      const float y = e[c] * inv * Storage<T>::load(w, col);
      out[(size_t)orow * H + col] = y;
      if (hidden_out) hidden_out[(size_t)orow * H + col] = y;
    }
  }
}

// ---------------------------------------------------------------------------------------
// Per-head RMSNorm + rotate-half RoPE of one head vector held by one wave (D <= 128, so each
// lane owns the pair (i, i + D/2) for i = lane < D/2).
__device__ __forceinline__ void norm_rope_pair(float &x1, float &x2, bool own, int D, float w1, float w2,
                                               float eps, float cs, float sn) {
  const float ss = wave_sum(own ? x1 * x1 + x2 * x2 : 0.f);
  const float inv = rsqrtf(ss / (float)D + eps);
  const float a = x1 * inv * w1, b = x2 * inv * w2;
  x1 = a * cs - b * sn;
  x2 = b * cs + a * sn;
}

// One wave per (row, head). Heads [0, QH) are q, [QH, QH+KVH) k, then v.
template <typename T>
__global__ __launch_bounds__(256) void qk_norm_rope_kernel(int M, int bs, int QH, int KVH, int D,
                                                           const float *__restrict__ qkv, int splits,
                                                           const T *__restrict__ q_norm,
                                                           const T *__restrict__ k_norm, float eps,
                                                           const float *__restrict__ rope_cos,
                                                           const float *__restrict__ rope_sin, int rope_max_pos,
                                                           const int32_t *__restrict__ seq_lens, int max_ctx,
                                                           T *__restrict__ q, T *__restrict__ k, T *__restrict__ v) {
  const int lane = threadIdx.x & 63;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nh = QH + 2 * KVH;
  if (wid >= M * nh) return;
  const int m = wid / nh, h = wid % nh;
  const int N = nh * D, half = D / 2;
  const bool own = lane < half;
  const int i1 = own ? lane : 0, i2 = i1 + half;
  float x1 = 0.f, x2 = 0.f;
  for (int s = 0; s < splits; ++s) {
    const float *p = qkv + ((size_t)s * M + m) * N + (size_t)h * D;
    x1 += p[i1];
    x2 += p[i2];
  }
  if (h >= QH + KVH) {  // value head: round only
    if (own) {
      T *dst = v + ((size_t)m * KVH + (h - QH - KVH)) * D;
      Storage<T>::store(dst, i1, x1);
      Storage<T>::store(dst, i2, x2);
    }
    return;
  }
  const T *w = h < QH ? q_norm : k_norm;
  const int b = m / bs, j = m % bs;
  const int c = min(max(seq_lens[b], 0), max_ctx);
  const int pos = min(c + j, rope_max_pos - 1);
  const float cs = rope_cos[(size_t)pos * half + i1], sn = rope_sin[(size_t)pos * half + i1];
  norm_rope_pair(x1, x2, own, D, Storage<T>::load(w, i1), Storage<T>::load(w, i2), eps, cs, sn);
  if (own) {
    T *dst = h < QH ? q + ((size_t)m * QH + h) * D : k + ((size_t)m * KVH + (h - QH)) * D;
    Storage<T>::store(dst, i1, x1);
    Storage<T>::store(dst, i2, x2);
  }
}

// ---------------------------------------------------------------------------------------
// Context K/V epilogue of injection: one wave per (row, layer, head-of-2*KVH).
template <typename T>
__global__ __launch_bounds__(256) void kv_scatter_kernel(KvScatterArgs a) {
  const int lane = threadIdx.x & 63;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int per_row = a.L * 2 * a.KVH;
  if (wid >= a.N * per_row) return;
  const int r = wid / per_row, rem = wid % per_row;
  const int l = rem / (2 * a.KVH), kvh = rem % (2 * a.KVH);
  const bool is_v = kvh >= a.KVH;
  const int g = is_v ? kvh - a.KVH : kvh;
  const int64_t slot = a.slot_mapping[r];
  if (slot < 0 || slot >= a.num_slots) return;  // padding row / out of range: skipped
  const int D = a.D, half = D / 2;
  const int ncol = per_row * D;
  const bool own = lane < half;
  const int i1 = own ? lane : 0, i2 = i1 + half;
  const size_t col = (size_t)(l * 2 * a.KVH + kvh) * D;
  float x1 = 0.f, x2 = 0.f;
  for (int s = 0; s < a.splits; ++s) {
    const float *p = a.kv + ((size_t)s * a.N + r) * ncol + col;
    x1 += p[i1];
    x2 += p[i2];
  }
  if (!is_v) {
    const T *w = reinterpret_cast<const T *>(a.k_norm[l]);
    const int pos = min(max(a.positions[r], 0), a.rope_max_pos - 1);
    const float cs = a.rope_cos[(size_t)pos * half + i1], sn = a.rope_sin[(size_t)pos * half + i1];
    norm_rope_pair(x1, x2, own, D, Storage<T>::load(w, i1), Storage<T>::load(w, i2), a.eps, cs, sn);
  }
  if (own) {
    T *dst = reinterpret_cast<T *>(is_v ? a.v_cache[l] : a.k_cache[l]) + ((size_t)slot * a.KVH + g) * D;
    Storage<T>::store(dst, i1, x1);
    Storage<T>::store(dst, i2, x2);
  }
}

// ---------------------------------------------------------------------------------------
// act = silu(gate) * up (fp32) from the split partials [splits][M][2I] (gate then up).
template <typename T>
__global__ __launch_bounds__(256) void swiglu_kernel(int M, int I, const float *__restrict__ part, int splits,
                                                     float *__restrict__ act) {
  const size_t idx = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (idx >= (size_t)M * I) return;
  const int m = idx / I, n = idx % I;
  float4 gs = make_float4(0.f, 0.f, 0.f, 0.f), us = gs;
  for (int s = 0; s < splits; ++s) {
    const float *p = part + ((size_t)s * M + m) * (2 * (size_t)I) + n;
    const float4 g4 = *reinterpret_cast<const float4 *>(p);
    const float4 u4 = *reinterpret_cast<const float4 *>(p + I);
    gs.x += g4.x, gs.y += g4.y, gs.z += g4.z, gs.w += g4.w;
    us.x += u4.x, us.y += u4.y, us.z += u4.z, us.w += u4.w;
  }
  const float gv[4] = {gs.x, gs.y, gs.z, gs.w}, uv[4] = {us.x, us.y, us.z, us.w};
#pragma unroll
  for (int c = 0; c < 4; ++c) act[idx + c] = gv[c] / (1.f + expf(-gv[c])) * uv[c];
}

// ---------------------------------------------------------------------------------------
// One work-group per drafted row: reduce the per-group (max, index) pairs val/idx
// [rows][ngroups], lowest index on ties, then assemble [bonus, drafts].
__global__ __launch_bounds__(256) void argmax_reduce_kernel(int B, int K, int ngroups, const float *__restrict__ val,
                                                            const int32_t *__restrict__ idx,
                                                            const int32_t *__restrict__ bonus, int V,
                                                            int32_t *__restrict__ draft_ids,
                                                            int32_t *__restrict__ drafts_only) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const int r = blockIdx.x;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  const float *vr = val + (size_t)r * ngroups;
  const int32_t *ir = idx + (size_t)r * ngroups;
  for (int gi = threadIdx.x; gi < ngroups; gi += blockDim.x) argmax_merge(best, bi, vr[gi], ir[gi]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    argmax_merge(best, bi, ov, oi);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    sv[wave] = best;
    si[wave] = bi;
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) argmax_merge(best, bi, sv[w], si[w]);
  if (bi == 0x7fffffff) bi = 0;  // every logit NaN: unspecified, but a valid id
  const int b = r / K, j = r % K;
  drafts_only[(size_t)b * K + j] = bi;
  draft_ids[(size_t)b * (K + 1) + j + 1] = bi;
  if (j == 0) draft_ids[(size_t)b * (K + 1)] = min(max(bonus[b], 0), V - 1);
}

// ---------------------------------------------------------------------------------------
// Greedy verification: one wave per sequence; lane i compares draft i with target i and the
// first mismatch (lowest set bit of the ballot) ends the accepted prefix.
__global__ void verify_kernel(int B, int K, const int32_t *drafts, const int32_t *target, int32_t *acc,
                              int32_t *out, int32_t *next_bonus) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (b >= B) return;
  const bool mismatch = lane < K && drafts[(size_t)b * K + lane] != target[(size_t)b * (K + 1) + lane];
  const unsigned long long mask = __ballot(mismatch);
  const int n = mask ? (int)__builtin_ctzll(mask) : K;  // accepted drafts
  const int a = n + 1;
  if (lane <= K) out[(size_t)b * (K + 1) + lane] = lane < a ? target[(size_t)b * (K + 1) + lane] : -1;
  if (lane == 0) {
    acc[b] = a;
    next_bonus[b] = target[(size_t)b * (K + 1) + n];
  }
}

// ---------------------------------------------------------------------------------------
__global__ void rope_table_kernel(int D, double theta, int max_pos, float *cs, float *sn) {
  const int half = D / 2;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)max_pos * half) return;
  const int p = idx / half, i = idx % half;
  const double inv_freq = pow(theta, -2.0 * (double)i / (double)D);
  const double ang = (double)p * inv_freq;
  cs[idx] = (float)cos(ang);
  sn[idx] = (float)sin(ang);
}

}  // namespace

// ===========================================================================================
hipError_t launch_embed(bool bf16, const void *embed, int V, int H, const int32_t *bonus, int B, int bs,
                        int mask_id, float *x, hipStream_t s) {
  ProfScope prof("embed", s);
  if (H % 4) return hipErrorInvalidValue;
  if (bf16)
    embed_kernel<uint16_t><<<B * bs, 256, 0, s>>>((const uint16_t *)embed, V, H, bonus, bs, mask_id, x);
  else
    embed_kernel<float><<<B * bs, 256, 0, s>>>((const float *)embed, V, H, bonus, bs, mask_id, x);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(bool bf16, int M, int H, float *x, const float *part, int splits, const void *w,
                          float eps, float *out, int keep_bs, float *hidden_out, hipStream_t s) {
  ProfScope prof("rmsnorm", s);
  if (H % 4 || H > 1024 * 4 * kRmsVecs) return hipErrorInvalidValue;
  const int threads = std::min(1024, (H / 4 + 63) / 64 * 64);
  if (bf16)
    rmsnorm_kernel<uint16_t><<<M, threads, 0, s>>>(M, H, x, part, splits, (const uint16_t *)w, eps, out, keep_bs,
                                                hidden_out);
  else
    rmsnorm_kernel<float><<<M, threads, 0, s>>>(M, H, x, part, splits, (const float *)w, eps, out, keep_bs,
                                            hidden_out);
  return hipGetLastError();
}

hipError_t launch_qk_norm_rope(bool bf16, int M, int bs, int QH, int KVH, int D, const float *qkv, int splits,
                               const void *q_norm, const void *k_norm, float eps, const float *rope_cos,
                               const float *rope_sin, int rope_max_pos, const int32_t *seq_lens, int max_ctx,
                               void *q, void *k, void *v, hipStream_t s) {
  ProfScope prof("qk_norm_rope", s);
  const int waves = M * (QH + 2 * KVH);
  const int grid = (waves + 3) / 4;
  if (bf16)
    qk_norm_rope_kernel<uint16_t><<<grid, 256, 0, s>>>(M, bs, QH, KVH, D, qkv, splits, (const uint16_t *)q_norm,
                                                       (const uint16_t *)k_norm, eps, rope_cos, rope_sin,
                                                       rope_max_pos, seq_lens, max_ctx, (uint16_t *)q,
                                                       (uint16_t *)k, (uint16_t *)v);
  else
    qk_norm_rope_kernel<float><<<grid, 256, 0, s>>>(M, bs, QH, KVH, D, qkv, splits, (const float *)q_norm,
                                                    (const float *)k_norm, eps, rope_cos, rope_sin, rope_max_pos,
                                                    seq_lens, max_ctx, (float *)q, (float *)k, (float *)v);
  return hipGetLastError();
}

hipError_t launch_kv_scatter(bool bf16, const KvScatterArgs &a, hipStream_t s) {
  ProfScope prof("kv_scatter", s);
  const long waves = (long)a.N * a.L * 2 * a.KVH;
  const unsigned grid = (unsigned)((waves + 3) / 4);
  if (bf16)
    kv_scatter_kernel<uint16_t><<<grid, 256, 0, s>>>(a);
  else
    kv_scatter_kernel<float><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_swiglu(bool bf16, int M, int I, const float *part, int splits, float *act, hipStream_t s) {
  ProfScope prof("swiglu", s);
  if (I % 4) return hipErrorInvalidValue;
  const size_t n = (size_t)M * I / 4;
  const unsigned grid = (unsigned)((n + 255) / 256);
  if (bf16)
    swiglu_kernel<uint16_t><<<grid, 256, 0, s>>>(M, I, part, splits, act);
  else
    swiglu_kernel<float><<<grid, 256, 0, s>>>(M, I, part, splits, act);
  return hipGetLastError();
}

hipError_t launch_argmax_reduce(int B, int K, int ngroups, const float *val, const int32_t *idx,
                                const int32_t *bonus, int V, int32_t *draft_ids, int32_t *drafts_only,
                                hipStream_t s) {
  ProfScope prof("argmax_reduce", s);
  argmax_reduce_kernel<<<B * K, 256, 0, s>>>(B, K, ngroups, val, idx, bonus, V, draft_ids, drafts_only);
  return hipGetLastError();
}

hipError_t launch_verify(int B, int K, const int32_t *drafts, const int32_t *target, int32_t *acc, int32_t *out,
                         int32_t *next_bonus, hipStream_t s) {
  ProfScope prof("verify", s);
  verify_kernel<<<(B + 3) / 4, 256, 0, s>>>(B, K, drafts, target, acc, out, next_bonus);
  return hipGetLastError();
}

hipError_t launch_rope_table(int D, double theta, int max_pos, float *cos_out, float *sin_out, hipStream_t s) {
  ProfScope prof("rope_table", s);
  const size_t n = (size_t)max_pos * (D / 2);
  rope_table_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(D, theta, max_pos, cos_out, sin_out);
  return hipGetLastError();
}

}  // namespace dflash
