// Host-side launchers of the DFlash kernels (internal to libdflash; the public ABI is
// include/dflash.h). Each launcher enqueues on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "profile.h"

namespace dflash {

// ------------------------------------------------------------------------------------------
// GEMM: C[m, n] = sum_k A[m, k] * B[n, k], A and B of the storage type, fp32 accumulation.
// With one K split the epilogue is applied in the same kernel:
//   kStore    out[m][n] = C                                   (fp32)
//   kResidAdd out[m][n] += C                                  (the fp32 residual stream)
//   kSwiGLU   act[m][n] = silu(C_gate) * C_up (fp32), B = {gate [N,K], up [N,K]}
//   kArgmax   amax_{val,idx}[m][g] = (max, lowest index) over column group g (one split only)
// With `splits` > 1 every split writes fp32 partials part[s][m][N] (SwiGLU: part[s][m][2N],
// gate then up) and the consumer kernel sums them in split order.
// A may be split along K into `a_nseg` equal segments with their own base pointers (the
// auxiliary states of injection; kStore only); B may be split along N into up to 3
// matrices (q|k|v). N must be a multiple of 16.
// ------------------------------------------------------------------------------------------
enum class GemmEpi { kStore, kResidAdd, kSwiGLU, kArgmax };

struct GemmArgs {
  const void *a[8];
  int a_nseg;
  int64_t lda;  // row stride of every A segment, in elements
  const void *b[3];
  int b_end[3];  // exclusive N end of each B segment (b_end[nseg-1] == N)
  int b_nseg;
  int M, N, K;
  float *out;         // kStore / kResidAdd: [M][N]
  float *act;         // kSwiGLU: [M][N] fp32
  float *part;        // splits > 1: [splits][M][N] (SwiGLU [splits][M][2N])
  float *amax_val;    // kArgmax: [M][gemm_col_groups(N)]
  int32_t *amax_idx;  // kArgmax: [M][gemm_col_groups(N)]
  bool a_f32;         // A is fp32 (single segment) while B is bf16: hi+lo bf16 MFMA pairs
  const char *tag;    // name under which the launch is timed when profiling is on
  int kt, kp;         // set by launch_gemm: K per split, K per staged LDS pass
};

int gemm_mt(int M);
int gemm_col_groups(int M, int N, GemmEpi epi);  // work-group column groups (argmax groups)
// Split count for a (M, N, K) problem; shared by workspace planning and launch.
int gemm_plan_splits(int M, int N, int K, bool bf16, GemmEpi epi);
hipError_t launch_gemm(const GemmArgs &g, bool bf16, GemmEpi epi, int splits, hipStream_t s);

// ------------------------------------------------------------------------------------------
// Row-wise kernels
// ------------------------------------------------------------------------------------------
// x[m] = embed[id] with id = bonus[b] for block slot 0 and mask otherwise (m = b*bs + j).
hipError_t launch_embed(bool bf16, const void *embed, int V, int H, const int32_t *bonus,
                        int B, int bs, int mask_id, float *x, hipStream_t s);

// For each row m: r = (x ? x[m] : 0) + sum_s part[s][m] (split order); if x and splits,
// x[m] = r; out[row_map(m)] = rmsnorm(r) * w (fp32). With keep_bs > 0 only rows with
// m % keep_bs != 0 are normalised, and they are written compactly (block slot 0 dropped):
// out row (m / keep_bs) * (keep_bs - 1) + m % keep_bs - 1. hidden_out (optional) gets the
// same rows.
hipError_t launch_rmsnorm(bool bf16, int M, int H, float *x, const float *part, int splits,
                          const void *w, float eps, float *out, int keep_bs, float *hidden_out,
                          hipStream_t s);

// q/k/v of the block from the fp32 QKV projection partials [splits][M][(QH+2KVH)*D]: per-head
// RMSNorm + RoPE on q and k (position seq_lens[b] + j), round; writes q [M][QH][D], k and v
// [M][KVH][D].
hipError_t launch_qk_norm_rope(bool bf16, int M, int bs, int QH, int KVH, int D, const float *qkv,
                               int splits, const void *q_norm, const void *k_norm, float eps,
                               const float *rope_cos, const float *rope_sin, int rope_max_pos,
                               const int32_t *seq_lens, int max_ctx, void *q, void *k, void *v,
                               hipStream_t s);

// Context K/V of injection from the fp32 fused-KV projection partials
// [splits][N][L*2*KVH*D]: k_norm + RoPE on keys, round, scatter both to slot_mapping[r] of
// every layer's cache.
struct KvScatterArgs {
  int N, L, KVH, D;
  const float *kv;
  int splits;
  const void *k_norm[64];
  float eps;
  const float *rope_cos, *rope_sin;
  int rope_max_pos;
  const int32_t *positions;
  const int64_t *slot_mapping;
  int64_t num_slots;
  void *k_cache[64];
  void *v_cache[64];
};
hipError_t launch_kv_scatter(bool bf16, const KvScatterArgs &a, hipStream_t s);

// act[m][n] = silu(sum_s part[s][m][n]) * sum_s part[s][m][I + n] (fp32), part [splits][M][2I].
hipError_t launch_swiglu(bool bf16, int M, int I, const float *part, int splits, float *act,
                         hipStream_t s);

// Final argmax over the column groups val/idx [B*K][ngroups] (lowest index on ties) and
// output assembly.
hipError_t launch_argmax_reduce(int B, int K, int ngroups, const float *val, const int32_t *idx,
                                const int32_t *bonus, int V, int32_t *draft_ids,
                                int32_t *drafts_only, hipStream_t s);

hipError_t launch_verify(int B, int K, const int32_t *drafts, const int32_t *target, int32_t *acc,
                         int32_t *out, int32_t *next_bonus, hipStream_t s);

hipError_t launch_rope_table(int D, double theta, int max_pos, float *cos_out, float *sin_out,
                             hipStream_t s);

// ------------------------------------------------------------------------------------------
// Non-causal paged block attention
// ------------------------------------------------------------------------------------------
struct AttnArgs {
  const void *q, *kb, *vb;  // block q [M][QH][D]; block k/v [M][KVH][D]
  const void *kc, *vc;      // this layer's cache [num_pages*P][KVH][D]
  const int32_t *block_table;
  int maxb, P, num_pages;
  const int32_t *seq_lens;
  int max_ctx;
  int B, bs, QH, KVH, D;
  int chunk, nsplit;  // keys per split (multiple of 64), splits per sequence
  float *po, *pm, *pl;  // partials [B][KVH][nsplit][64][D], [B][KVH][nsplit][64]
  float *o;             // merged output [M][QH*D], fp32
};
void attn_plan(int B, int KVH, int max_keys, int *chunk, int *nsplit);
hipError_t launch_attention(bool bf16, const AttnArgs &a, hipStream_t s);

}  // namespace dflash
