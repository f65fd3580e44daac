// Row-wise kernels of the DFlash path: block embedding, the LM-head argmax reduction, greedy
// verification (with acceptance counters), proposal-input preparation and the RoPE table. Normalisation, q/k norm + RoPE, SwiGLU and the context
// K/V scatter run as GEMM epilogues or prologues.
#include <float.h>

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace dflash {
namespace {

// ---------------------------------------------------------------------------------------
// Block construction + embedding: row m = b*bs + j gets embed[bonus[b]] for j == 0 and
// embed[mask] otherwise, converted to the fp32 residual stream; ss[m] is the row's sum of
// squares (the first layer's input norm is applied by the QKV GEMM on load). The grid also
// clears the GEMM split-K counters of the call.
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const T *__restrict__ embed, int V, int H,
                                                    const int32_t *__restrict__ bonus, int bs, int mask_id,
                                                    float *__restrict__ x, float *__restrict__ ss,
                                                    unsigned *__restrict__ counters, int n_counters) {
  __shared__ float red[16];
  const int m = blockIdx.x;
  for (int i = m * blockDim.x + threadIdx.x; i < n_counters; i += gridDim.x * blockDim.x) counters[i] = 0u;
  const int b = m / bs, j = m % bs;
  int id = (j == 0) ? bonus[b] : mask_id;
  id = min(max(id, 0), V - 1);
  const T *src = embed + (size_t)id * H;
  float acc = 0.f;
  for (int i = threadIdx.x * 4; i < H; i += blockDim.x * 4) {
    float4 v;
    v.x = Storage<T>::load(src, i);
    v.y = Storage<T>::load(src, i + 1);
    v.z = Storage<T>::load(src, i + 2);
    v.w = Storage<T>::load(src, i + 3);
    acc += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    *reinterpret_cast<float4 *>(x + (size_t)m * H + i) = v;
  }
  acc = block_sum(acc, red);
  if (threadIdx.x == 0) ss[m] = acc;
}

__global__ void zero_kernel(unsigned *p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// ---------------------------------------------------------------------------------------
// One work-group per drafted row: reduce the per-group (max, index) pairs val/idx
// [rows][ngroups], lowest index on ties, then assemble [bonus, drafts].
__global__ __launch_bounds__(256) void argmax_reduce_kernel(int B, int K, int ngroups, const float *__restrict__ val,
                                                            const int32_t *__restrict__ idx,
                                                            const int32_t *__restrict__ bonus, int V,
                                                            const unsigned *__restrict__ abort_word,
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
  if (abort_word && *abort_word) bi = -1;  // the layer stack did not complete: no draft
  const int b = r / K, j = r % K;
  drafts_only[(size_t)b * K + j] = bi;
  draft_ids[(size_t)b * (K + 1) + j + 1] = bi;
  if (j == 0) draft_ids[(size_t)b * (K + 1)] = min(max(bonus[b], 0), V - 1);
}

// ---------------------------------------------------------------------------------------
// Greedy verification: one wave per sequence; lane i compares draft i with target i and the
// first mismatch (lowest set bit of the ballot) ends the accepted prefix. With stats, the
// acceptance counters are accumulated with integer atomics (order-independent).
__global__ void verify_kernel(int B, int K, const int32_t *drafts, const int32_t *target, int32_t *acc,
                              int32_t *out, int32_t *next_bonus, int64_t *stats) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (stats && blockIdx.x == 0 && threadIdx.x == 0) {
    atomicAdd(reinterpret_cast<unsigned long long *>(&stats[0]), (unsigned long long)B);
    atomicAdd(reinterpret_cast<unsigned long long *>(&stats[1]), (unsigned long long)B * K);
  }
  if (b >= B) return;
  const bool mismatch = lane < K && drafts[(size_t)b * K + lane] != target[(size_t)b * (K + 1) + lane];
  const unsigned long long mask = __ballot(mismatch);
  const int n = mask ? (int)__builtin_ctzll(mask) : K;  // accepted drafts
  const int a = n + 1;
  if (lane <= K) out[(size_t)b * (K + 1) + lane] = lane < a ? target[(size_t)b * (K + 1) + lane] : -1;
  if (lane == 0) {
    acc[b] = a;
    next_bonus[b] = target[(size_t)b * (K + 1) + n];
    if (stats && n > 0) atomicAdd(reinterpret_cast<unsigned long long *>(&stats[2]), (unsigned long long)n);
  }
}

// ---------------------------------------------------------------------------------------
// Proposal-input preparation: threads [0, B) correct the requests (sequence length, bonus),
// threads [B, B + n_rows) the context rows (position, slot); each counts the valid entries of
// its request's previous output itself (K + 1 <= 64 reads).
__global__ void prepare_kernel(PrepareArgs a) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= a.B + a.n_rows) return;
  const bool is_req = t < a.B;
  const int r = t - a.B;
  const int b = is_req ? t : min(max(a.row_req[r], 0), a.B - 1);
  const int32_t *prev = a.prev_out + (size_t)b * (a.K + 1);
  int valid = 0, last = -1;
  for (int i = 0; i <= a.K; ++i) {
    const int v = prev[i];
    if (v != -1 && v >= 0 && v < a.V) {
      ++valid;
      last = v;
    }
  }
  const int rejected = a.K + 1 - valid;
  if (is_req) {
    a.seq_lens[b] = a.opt_seq_lens[b] - rejected;
    a.bonus[b] = last >= 0 ? last : 0;
  } else {
    const int pos = a.opt_positions[r] - rejected;
    a.positions[r] = pos;
    int64_t slot = -1;
    if (pos >= 0) {
      const int page = a.block_table[(size_t)b * a.maxb + min(pos / a.P, a.maxb - 1)];
      slot = (int64_t)page * a.P + pos % a.P;
    }
    a.slot_mapping[r] = slot;
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
                        int mask_id, float *x, float *ss, unsigned *counters, int n_counters, hipStream_t s) {
  ProfScope prof("embed", s);
  if (H % 4) return hipErrorInvalidValue;
  if (bf16)
    embed_kernel<uint16_t><<<B * bs, 256, 0, s>>>((const uint16_t *)embed, V, H, bonus, bs, mask_id, x, ss,
                                                  counters, n_counters);
  else
    embed_kernel<float><<<B * bs, 256, 0, s>>>((const float *)embed, V, H, bonus, bs, mask_id, x, ss, counters,
                                               n_counters);
  return hipGetLastError();
}

hipError_t launch_zero(unsigned *p, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  ProfScope prof("zero", s);
  zero_kernel<<<(n + 255) / 256, 256, 0, s>>>(p, n);
  return hipGetLastError();
}

hipError_t launch_argmax_reduce(int B, int K, int ngroups, const float *val, const int32_t *idx,
                                const int32_t *bonus, int V, const unsigned *abort_word, int32_t *draft_ids,
                                int32_t *drafts_only, hipStream_t s) {
  ProfScope prof("argmax_reduce", s);
  argmax_reduce_kernel<<<B * K, 256, 0, s>>>(B, K, ngroups, val, idx, bonus, V, abort_word, draft_ids,
                                             drafts_only);
  return hipGetLastError();
}

hipError_t launch_verify(int B, int K, const int32_t *drafts, const int32_t *target, int32_t *acc, int32_t *out,
                         int32_t *next_bonus, int64_t *stats, hipStream_t s) {
  ProfScope prof("verify", s);
  verify_kernel<<<(B + 3) / 4, 256, 0, s>>>(B, K, drafts, target, acc, out, next_bonus, stats);
  return hipGetLastError();
}

hipError_t launch_prepare(const PrepareArgs &a, hipStream_t s) {
  ProfScope prof("prepare", s);
  const int n = a.B + a.n_rows;
  prepare_kernel<<<(n + 255) / 256, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_rope_table(int D, double theta, int max_pos, float *cos_out, float *sin_out, hipStream_t s) {
  ProfScope prof("rope_table", s);
  const size_t n = (size_t)max_pos * (D / 2);
  rope_table_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(D, theta, max_pos, cos_out, sin_out);
  return hipGetLastError();
}

}  // namespace dflash
