// Host-side launchers of the DFlash kernels (internal to libdflash; the public ABI is
// include/dflash.h). Each launcher enqueues on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "profile.h"

namespace dflash {

// ------------------------------------------------------------------------------------------
// GEMM: C[m, n] = sum_k A[m, k] * B[n, k], B of the storage type, fp32 accumulation.
//
// A is fp32 (every activation) or of the storage type (the auxiliary target states, which
// may come as `a_nseg` equal K segments with their own base pointers). With `norm_w` set, A
// is RMS-normalised while it is staged: row m is scaled by 1/sqrt(ss_m / K + eps) and by the
// norm weight, where ss_m = sum_q ss[q * ss_rows + src_row(m)] are the per-column-group sums
// of squares written by the producer of A (`ss_out`). With `keep_bs` > 0 the GEMM's row m
// reads A row (m / (keep_bs-1)) * keep_bs + m % (keep_bs-1) + 1 (block slot 0 dropped) and
// the normalised rows may be written to `a_out` [M][K].
//
// Split-K (`splits` > 1): every split writes its tile to part[s] ([M][NACC][N]) and the last
// work-group of each output tile to arrive sums the splits in split order and runs the
// epilogue. `counters` holds one zero-initialised counter per output tile
// (GemmPlan::col_groups * row_blocks); the reducing work-group resets it to zero.
//
// Epilogues on the final tile:
//   kStore        out[m][n] = C                                  (fp32)
//   kResidAdd     out[m][n] += C                                 (the fp32 residual stream)
//   kSwiGLU       out[m][n] = silu(C_gate) * C_up, B = {gate [N,K], up [N,K]}
//   kArgmax       amax_{val,idx}[m][col group] = (max, lowest index)
//   kHeadNormRope the block's q | k | v: per-head RMSNorm (q_norm / k_norm) and RoPE at
//                 position min(seq_lens[b], max_ctx) + j on q and k, rounded to the storage
//                 type into q [M][QH][D], k and v [M][KVH][D]; B = {wq, wk, wv}
//   kKvScatter    context K/V of every layer: N = L * 2 * KVH * D (layer-major, k heads then
//                 v heads); k_norm + RoPE at positions[m] on keys; both rounded and written to
//                 slot slot_mapping[m] of the layer's cache (rows with a slot outside
//                 [0, num_slots) are skipped)
// kStore / kResidAdd can also write ss_out[col group][m], the row's sum of squares over
// the tile's columns (for a consumer with norm on load).
// ------------------------------------------------------------------------------------------
enum class GemmEpi { kStore, kResidAdd, kSwiGLU, kArgmax, kHeadNormRope, kKvScatter };

struct GemmArgs {
  const void *a[8];
  int a_nseg;
  int64_t lda;  // row stride of every A segment, in elements
  bool a_f32;   // A is fp32 (single segment): hi+lo bf16 MFMA pairs against bf16 weights
  const void *b[3];
  int b_end[3];  // exclusive N end of each B segment (b_end[nseg-1] == N)
  int b_nseg;
  int M, N, K;
  // norm on load
  const void *norm_w;  // [K] storage type, or null
  const float *ss;     // [ss_groups][ss_rows]
  int ss_groups, ss_rows;
  float eps;
  int keep_bs;    // > 0: compact the rows (drop block slot 0)
  float *a_out;   // optional [M][K]: the normalised A rows
  // split-K
  float *part;
  unsigned *counters;
  // epilogue outputs
  float *out;
  float *ss_out;
  float *amax_val;    // [M][col groups]
  int32_t *amax_idx;  // [M][col groups]
  // head epilogues
  int head_dim, n_q_heads, n_kv_heads, block_size;
  const void *q_norm, *k_norm;
  const int32_t *seq_lens;
  int max_ctx;
  const float *rope_cos, *rope_sin;  // [rope_max_pos][head_dim / 2]
  int rope_max_pos;
  void *q, *k, *v;
  const int32_t *positions;
  const int64_t *slot_mapping;
  int64_t num_slots;
  const void *layer_k_norm[64];
  void *k_cache[64];
  void *v_cache[64];
  const char *tag;  // name under which the launch is timed when profiling is on
  int kt, kp;       // set by launch_gemm: K per split, K per staged LDS pass
  uint16_t *a_split;  // tiled plans: workspace for the (hi, lo) bf16 planes of A, 2 * M * K
  // tiled SwiGLU: write the output as its (hi, lo) bf16 planes [2][M][N] (hi = bf16(f),
  // lo = bf16(f - hi)) instead of fp32 rows
  uint16_t *out_planes;
  // tiled (hi, lo) plans: A's planes [2][M][K] as written by its producer (no split pass; A
  // has no norm on load)
  const uint16_t *a_planes;
};

int gemm_mt(int M);

// Launch plan of one GEMM: work-group shape (cw wave columns x ct column tiles per wave x
// kw K sub-slices), K splits, work-groups along the column groups (0: one per column
// group; fewer: each loops over several), LDS bytes of one staged A pass. Deterministic in
// its arguments, so the workspace planner and the launch agree.
struct GemmPlan {
  int cw, ct, kw;
  int splits;
  int grid_x;
  int lds_budget;
  int col_groups, row_blocks;  // output tiles = col_groups * row_blocks (split-K counters)
  int tiled;                   // 1: the LDS-tiled kernel for many rows (tile_m x tile_n output tiles)
  int hi_only;                 // tiled, fp32 activations: only their bf16 rounding enters the MFMAs
  int tile_m, tile_n;          // tiled: 128 x 128, 64 x 256, or the wide 256 x 256 (gemm_wide_kernel)
};
// a_f32: the activations are fp32 rows (else the storage type, as the auxiliary target states,
// in a_segs equal K segments)
GemmPlan gemm_plan(int M, int N, int K, int head_dim, bool bf16, GemmEpi epi, bool multi_a, bool a_f32 = true,
                   int a_segs = 1);
hipError_t launch_gemm(const GemmArgs &g, bool bf16, GemmEpi epi, const GemmPlan &p, hipStream_t s);

// ------------------------------------------------------------------------------------------
// Row-wise kernels
// ------------------------------------------------------------------------------------------
// x[m] = embed[id] with id = bonus[b] for block slot 0 and mask otherwise (m = b*bs + j);
// ss[m] = sum of squares of x[m]; counters[0, n_counters) = 0.
hipError_t launch_embed(bool bf16, const void *embed, int V, int H, const int32_t *bonus, int B, int bs,
                        int mask_id, float *x, float *ss, unsigned *counters, int n_counters, hipStream_t s);

hipError_t launch_zero(unsigned *p, int n, hipStream_t s);

// Final argmax over the column groups val/idx [B*K][ngroups] (lowest index on ties) and
// output assembly. With `abort_word` set and nonzero (the persistent layer kernel gave up on a
// wait), every draft is -1.
hipError_t launch_argmax_reduce(int B, int K, int ngroups, const float *val, const int32_t *idx,
                                const int32_t *bonus, int V, const unsigned *abort_word, int32_t *draft_ids,
                                int32_t *drafts_only, hipStream_t s);

// stats (optional, [3] int64): += B, B*K, sum(acc - 1)
hipError_t launch_verify(int B, int K, const int32_t *drafts, const int32_t *target, int32_t *acc, int32_t *out,
                         int32_t *next_bonus, int64_t *stats, hipStream_t s);

struct PrepareArgs {
  int B, K, V, n_rows, maxb, P;
  const int32_t *prev_out, *opt_seq_lens, *row_req, *opt_positions, *block_table;
  int32_t *seq_lens, *positions, *bonus;
  int64_t *slot_mapping;
};
hipError_t launch_prepare(const PrepareArgs &a, hipStream_t s);

hipError_t launch_rope_table(int D, double theta, int max_pos, float *cos_out, float *sin_out, hipStream_t s);

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
  int chunk, nsplit;    // keys per split (multiple of 64), splits per sequence
  float *po, *pm, *pl;  // partials [B][KVH][nsplit][64][D], [B][KVH][nsplit][64]
  float *o;             // merged output [M][QH*D], fp32
  // non-null: the merged output as its (hi, lo) bf16 planes [2][M][QH*D] instead (hi =
  // bf16(f), lo = bf16(f - hi)), for an O projection that takes the pair without a split pass
  uint16_t *o_planes;
  // With several sequences: the (sequence, kv head, split) work-groups that have keys, as
  // flat indices (b * KVH + g) * nsplit + split, and their count (written by
  // launch_attention_items once per proposal); null: every index of the grid is launched.
  const int *items, *n_items;
};
void attn_plan(int B, int KVH, int max_keys, int *chunk, int *nsplit);
hipError_t launch_attention(bool bf16, const AttnArgs &a, hipStream_t s);
// items [B * KVH * nsplit] and n_items [1] of `a` from the sequence lengths.
hipError_t launch_attention_items(const AttnArgs &a, int *items, int *n_items, hipStream_t s);

// ------------------------------------------------------------------------------------------
// Persistent layer-stack kernel for one block of at most 16 rows (batch 1), bf16 drafters with
// head_dim 128: every layer's QKV, attention, split merge, O, gate|up and down projections run
// as jobs of one launch with one work-group per CU. Each work-group has four compute waves
// (weights -> MFMA, the next two jobs' weights always in flight), three stager waves (wait for
// the producer tiles a job reads, stage its activations in LDS with the RMSNorm row scale
// applied, stage attention tiles, merge attention splits) and a finisher wave (split-K
// partials, the last contributor's reduction and epilogue, readiness flags, attention tiles).
// The waves hand off through LDS words; work-groups through device-scope flags and counters.
// Every wait is bounded; a work-group that gives up raises an abort word, and the drafts are -1.
// ------------------------------------------------------------------------------------------
constexpr int kPlkMaxLayers = 8;

struct PlkLayerW {
  const uint16_t *in_norm, *wq, *wk, *wv, *q_norm, *k_norm, *wo, *post_norm, *wg, *wu, *wd;
  const uint16_t *kc, *vc;  // this layer's paged cache [num_pages * P][KVH][128]
};

// One GEMM phase: `tiles` output tiles of 128 columns, `chunks` K chunks of `kr` columns per
// tile; the tiles x chunks units are dealt to the work-groups in contiguous ranges (base or
// base + 1 units each, the first `rem` work-groups one more); `slots` bounds the work-groups
// that share one tile.
struct PlkGemm {
  int tiles, chunks, kr, base, rem, slots;
};

struct PlkArgs {
  PlkLayerW lw[kPlkMaxLayers];
  int L, H, QH, KVH, I, bs, G;
  float eps;
  const float *rope_cos, *rope_sin;
  int rope_max_pos;
  const int32_t *seq_lens;
  int max_ctx;
  const int32_t *block_table;
  int maxb, P, num_pages;
  PlkGemm g[4];   // QKV, O, gate|up, down
  int ntile, ns;  // 64-key tiles of the longest key range, splits per kv head
  int rm, nrp;    // block rows per attention merge job, row groups per q head
  int nwg;
  // workspace
  float *x0, *ss0;         // embedding rows [16][H] and sums of squares [1][16]; also the final
                           // rows and their sums of squares per 128-column tile [H/128][16]
  float *xs, *sss;         // x_1 .. x_{2L-1} [2L-1][16][H]; their sums of squares [2L-1][H/128][16]
  uint16_t *qkv;           // the block's q | k | v per layer [L][16][(QH + 2 KVH) * 128]
  float *o, *act;          // merged attention output [L][16][QH * 128]; SwiGLU product [L][16][I]
  float *apo, *apm, *apl;  // attention partials [KVH][ns][64][128], [KVH][ns][64] (reused by layers)
  float *gpart[4];         // GEMM partials [tiles][slots][nacc][16][128] (reused by layers)
  unsigned *sync;          // counters, flags and the abort word (zero before the launch)
  const void *ws;          // the workspace holding every buffer above (ws_bytes < 2^31)
  unsigned ws_bytes;
};

struct PlkPlan {
  int ok;
  PlkGemm g[4];
  int ntile, ns, rm, nrp, nwg;
  size_t off_xs, off_sss, off_qkv, off_o, off_act, off_apo, off_apm, off_apl, off_gpart[4];
  size_t bytes;   // workspace bytes of the regions above (from offset 0)
  int sync_words;  // counters + flags + abort word
};
// The plan of the persistent kernel for this shape, or ok = 0 when it does not apply.
PlkPlan plk_plan(int L, int H, int QH, int KVH, int D, int I, int bs, int batch, int max_ctx, bool bf16);
hipError_t launch_plk(const PlkArgs &a, hipStream_t s);

}  // namespace dflash
