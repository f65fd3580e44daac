// C ABI of the DFlash draft-proposal path (declared in include/dflash.h): argument
// validation, workspace planning and carve-up, and the launch sequence of each call.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cstdlib>
#include <mutex>
#include <string>

#include "../../include/dflash.h"
#include "kernels.h"

using namespace dflash;

namespace {

thread_local std::string g_last_error;

dflash_status fail(dflash_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
dflash_status fail(dflash_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

dflash_status ok() {
  g_last_error.clear();
  return DFLASH_OK;
}

#define HIP_TRY(expr)                                                                          \
  do {                                                                                         \
    hipError_t e_ = (expr);                                                                    \
    if (e_ != hipSuccess) return fail(DFLASH_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool is_bf16(const dflash_config *c) { return c->dtype == DFLASH_BF16; }
size_t elem_size(const dflash_config *c) { return is_bf16(c) ? 2 : 4; }

dflash_status check_config(const dflash_config *c) {
  if (!c) return fail(DFLASH_ERR_INVALID_ARGUMENT, "config is NULL");
  if (c->hidden <= 0 || c->n_layers < 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 ||
      c->intermediate <= 0 || c->vocab <= 0 || c->n_aux <= 0 || c->target_hidden <= 0 || c->block_size <= 0)
    return fail(DFLASH_ERR_INVALID_ARGUMENT, "config dimensions must be positive");
  if (c->dtype != DFLASH_F32 && c->dtype != DFLASH_BF16)
    return fail(DFLASH_ERR_INVALID_ARGUMENT, "unknown dtype %d", c->dtype);
  if (c->n_q_heads % c->n_kv_heads != 0)
    return fail(DFLASH_ERR_INVALID_ARGUMENT, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)", c->n_q_heads,
                c->n_kv_heads);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(DFLASH_ERR_UNSUPPORTED, "head_dim %d is not 64 or 128", c->head_dim);
  if (c->hidden % 128 || c->intermediate % 128 || (c->n_aux * c->target_hidden) % 128 || c->target_hidden % 32)
    return fail(DFLASH_ERR_UNSUPPORTED,
                "hidden, intermediate and n_aux*target_hidden must be multiples of 128, target_hidden of 32");
  if ((c->n_q_heads * c->head_dim) % 128)
    return fail(DFLASH_ERR_UNSUPPORTED, "n_q_heads * head_dim must be a multiple of 128");
  if (c->hidden > 4096 * 4) return fail(DFLASH_ERR_UNSUPPORTED, "hidden %d above 16384", c->hidden);
  if (c->vocab % 16) return fail(DFLASH_ERR_UNSUPPORTED, "vocab %d is not a multiple of 16", c->vocab);
  if (c->block_size < 2 || c->block_size > 64)
    return fail(DFLASH_ERR_UNSUPPORTED, "block_size %d outside [2, 64]", c->block_size);
  if (c->block_size * (c->n_q_heads / c->n_kv_heads) > 64)
    return fail(DFLASH_ERR_UNSUPPORTED, "block_size * q-heads per kv-head exceeds 64");
  if (c->n_layers > 64) return fail(DFLASH_ERR_UNSUPPORTED, "more than 64 layers");
  if (c->n_aux > 8) return fail(DFLASH_ERR_UNSUPPORTED, "more than 8 auxiliary layers");
  if (c->mask_token_id < 0 || c->mask_token_id >= c->vocab)
    return fail(DFLASH_ERR_INVALID_ARGUMENT, "mask_token_id %d outside [0, vocab)", c->mask_token_id);
  if (!(c->rms_eps >= 0.f)) return fail(DFLASH_ERR_INVALID_ARGUMENT, "rms_eps must be >= 0");
  return DFLASH_OK;
}

// ---------------------------------------------------------------------------------------
// Workspace plans. The same functions size the workspace and carve it at launch.
struct Carver {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  }
};

constexpr int kInjectChunk = 4096;  // rows per injection pass

// fp32 partial buffer of a GEMM (split-K only).
size_t gemm_part_floats(const GemmPlan &p, int M, int N, GemmEpi e) {
  if (p.splits <= 1) return 0;
  if (p.tiled) return (size_t)p.splits * p.row_blocks * p.col_groups * p.tile_m * p.tile_n;  // whole tiles
  return (size_t)p.splits * M * N * (e == GemmEpi::kSwiGLU ? 2 : 1);
}
int gemm_tiles(const GemmPlan &p) { return p.col_groups * p.row_blocks; }

struct InjectPlan {
  int rows, n_ctr;
  GemmPlan fc, kv;
  size_t off_y, off_ss, off_part, off_ctr, off_split, total;
};

InjectPlan plan_inject(const dflash_config *c, int rows) {
  InjectPlan p{};
  p.rows = rows;
  const bool bf = is_bf16(c);
  const int H = c->hidden, D = c->head_dim;
  const int kvn = std::max(c->n_layers * 2 * c->n_kv_heads * D, 16);
  p.fc = gemm_plan(rows, H, c->n_aux * c->target_hidden, D, bf, GemmEpi::kStore, c->n_aux > 1, false, c->n_aux);
  p.kv = gemm_plan(rows, kvn, H, D, bf, GemmEpi::kKvScatter, false);
  p.n_ctr = std::max(gemm_tiles(p.fc), gemm_tiles(p.kv));
  const size_t part = std::max(gemm_part_floats(p.fc, rows, H, GemmEpi::kStore),
                               gemm_part_floats(p.kv, rows, kvn, GemmEpi::kKvScatter));
  Carver cv;
  p.off_y = cv.take((size_t)rows * H * sizeof(float));
  p.off_ss = cv.take((size_t)p.fc.col_groups * rows * sizeof(float));
  p.off_part = cv.take(part * sizeof(float));
  p.off_ctr = cv.take((size_t)p.n_ctr * sizeof(unsigned));
  // the (hi, lo) bf16 planes of the normalised context rows when the K/V projection is tiled
  p.off_split = cv.take(p.kv.tiled ? 2 * (size_t)rows * H * sizeof(uint16_t) : 0);
  p.total = cv.off;
  return p;
}

struct ProposePlan {
  int B, M, Mk;
  GemmPlan qkv, o, gu, down, lm;
  PlkPlan plk;  // the persistent layer-stack kernel (batch 1), when it applies
  size_t off_plk;
  int chunk, nsplit, n_ctr, n_zero;  // n_zero: counters + the persistent kernel's sync words
  size_t off_items;  // the attention work-group list (several sequences)
  size_t off_x, off_ss, off_part, off_ctr, off_q, off_k, off_v, off_o, off_act, off_po, off_pm, off_pl, off_amv,
      off_ami, off_split, total;
};

ProposePlan plan_propose(const dflash_config *c, int B, int max_ctx) {
  ProposePlan p{};
  const bool bf = is_bf16(c);
  const int H = c->hidden, D = c->head_dim, QH = c->n_q_heads, KVH = c->n_kv_heads, I = c->intermediate;
  const int K = c->block_size - 1;
  p.B = B;
  p.M = B * c->block_size;
  p.Mk = B * K;
  const int M = p.M;
  const int nqkv = (QH + 2 * KVH) * D;
  p.qkv = gemm_plan(M, nqkv, H, D, bf, GemmEpi::kHeadNormRope, false);
  p.o = gemm_plan(M, H, QH * D, D, bf, GemmEpi::kResidAdd, false);
  p.gu = gemm_plan(M, I, H, D, bf, GemmEpi::kSwiGLU, false);
  p.down = gemm_plan(M, H, I, D, bf, GemmEpi::kResidAdd, false);
  p.lm = gemm_plan(std::max(p.Mk, 1), c->vocab, H, D, bf, GemmEpi::kArgmax, false);
  attn_plan(B, KVH, max_ctx + c->block_size, &p.chunk, &p.nsplit);
  p.plk = c->n_layers <= kPlkMaxLayers
              ? plk_plan(c->n_layers, H, QH, KVH, D, I, c->block_size, B, max_ctx, bf)
              : PlkPlan{};
  p.n_ctr = std::max(std::max(std::max(gemm_tiles(p.qkv), gemm_tiles(p.o)), std::max(gemm_tiles(p.gu), gemm_tiles(p.down))),
                     gemm_tiles(p.lm));
  const size_t part = std::max(std::max(std::max(gemm_part_floats(p.qkv, M, nqkv, GemmEpi::kHeadNormRope),
                                                 gemm_part_floats(p.o, M, H, GemmEpi::kResidAdd)),
                                        std::max(gemm_part_floats(p.gu, M, I, GemmEpi::kSwiGLU),
                                                 gemm_part_floats(p.down, M, H, GemmEpi::kResidAdd))),
                               gemm_part_floats(p.lm, std::max(p.Mk, 1), c->vocab, GemmEpi::kArgmax));
  // the residual-stream producers (O and down projections) write one sum of squares per
  // column group; the embedding writes one
  const int ss_groups = std::max(std::max(p.o.col_groups, p.down.col_groups), 1);
  const size_t es = elem_size(c);
  Carver cv;
  p.off_x = cv.take((size_t)M * H * sizeof(float));
  p.off_ss = cv.take((size_t)ss_groups * M * sizeof(float));
  p.off_part = cv.take(part * sizeof(float));
  p.n_zero = p.n_ctr + (p.plk.ok ? p.plk.sync_words : 0);
  p.off_ctr = cv.take((size_t)p.n_zero * sizeof(unsigned));
  p.off_q = cv.take((size_t)M * QH * D * es);
  p.off_k = cv.take((size_t)M * KVH * D * es);
  p.off_v = cv.take((size_t)M * KVH * D * es);
  p.off_o = cv.take((size_t)M * QH * D * sizeof(float));
  p.off_act = cv.take((size_t)M * I * sizeof(float));
  const size_t nrow = (size_t)B * KVH * p.nsplit * 64;
  p.off_po = cv.take(nrow * D * sizeof(float));
  p.off_pm = cv.take(nrow * sizeof(float));
  p.off_pl = cv.take(nrow * sizeof(float));
  p.off_items = B > 1 ? cv.take(((size_t)B * KVH * p.nsplit + 1) * sizeof(int)) : 0;
  // the (hi, lo) bf16 planes of the activations of the tiled GEMMs (many rows), reused by each
  size_t split = 0;
  if (p.qkv.tiled) split = std::max(split, (size_t)M * H);
  if (p.o.tiled) split = std::max(split, (size_t)M * QH * D);
  if (p.gu.tiled) split = std::max(split, (size_t)M * H);
  if (p.down.tiled) split = std::max(split, (size_t)M * I);
  if (p.lm.tiled) split = std::max(split, (size_t)std::max(p.Mk, 1) * H);
  p.off_split = cv.take(2 * split * sizeof(uint16_t));
  p.off_amv = cv.take((size_t)p.lm.col_groups * std::max(p.Mk, 1) * sizeof(float));
  p.off_ami = cv.take((size_t)p.lm.col_groups * std::max(p.Mk, 1) * sizeof(int32_t));
  p.off_plk = p.plk.ok ? cv.take(p.plk.bytes) : 0;
  p.total = cv.off;
  // the persistent kernel addresses the workspace with 32-bit offsets
  if (p.total >= (size_t(1) << 31)) p.plk.ok = 0;
  return p;
}

template <typename P>
P *at(void *ws, size_t off) {
  return reinterpret_cast<P *>(static_cast<char *>(ws) + off);
}

dflash_status check_weights_common(const dflash_config *c, const dflash_weights *w) {
  if (!w) return fail(DFLASH_ERR_INVALID_ARGUMENT, "weights is NULL");
  if (!w->rope_cos || !w->rope_sin || w->rope_max_pos <= 0)
    return fail(DFLASH_ERR_INVALID_ARGUMENT, "RoPE table missing");
  if (c->n_layers > 0 && !w->k_norm) return fail(DFLASH_ERR_INVALID_ARGUMENT, "k_norm array is NULL");
  for (int l = 0; l < c->n_layers; ++l)
    if (!w->k_norm[l]) return fail(DFLASH_ERR_INVALID_ARGUMENT, "k_norm[%d] is NULL", l);
  return DFLASH_OK;
}

dflash_status check_cache(const dflash_config *c, const dflash_kv_cache *kv) {
  if (!kv) return fail(DFLASH_ERR_INVALID_ARGUMENT, "cache is NULL");
  if (kv->num_pages <= 0 || kv->page_size <= 0)
    return fail(DFLASH_ERR_INVALID_ARGUMENT, "cache num_pages and page_size must be positive");
  if (c->n_layers > 0 && (!kv->k || !kv->v)) return fail(DFLASH_ERR_INVALID_ARGUMENT, "cache layer arrays are NULL");
  for (int l = 0; l < c->n_layers; ++l)
    if (!kv->k[l] || !kv->v[l]) return fail(DFLASH_ERR_INVALID_ARGUMENT, "cache of layer %d is NULL", l);
  return DFLASH_OK;
}

GemmArgs gemm_args(const dflash_config *c, const char *tag, const void *a, int64_t lda, int M, int N, int K,
                   unsigned *counters, float *part) {
  GemmArgs g{};
  g.a[0] = a;
  g.a_nseg = 1;
  g.lda = lda;
  g.a_f32 = true;  // activations are fp32; only the auxiliary states come in the storage type
  g.b_nseg = 1;
  g.M = M;
  g.N = N;
  g.K = K;
  g.eps = c->rms_eps;
  g.head_dim = c->head_dim;
  g.n_q_heads = c->n_q_heads;
  g.n_kv_heads = c->n_kv_heads;
  g.block_size = c->block_size;
  g.counters = counters;
  g.part = part;
  g.tag = tag;
  return g;
}

void set_norm(GemmArgs &g, const void *w, const float *ss, int groups, int rows) {
  g.norm_w = w;
  g.ss = ss;
  g.ss_groups = groups;
  g.ss_rows = rows;
}

void set_rope(GemmArgs &g, const dflash_weights *w) {
  g.rope_cos = w->rope_cos;
  g.rope_sin = w->rope_sin;
  g.rope_max_pos = w->rope_max_pos;
}

}  // namespace

// =========================================================================================
extern "C" {

const char *dflash_status_string(int32_t st) {
  switch (st) {
    case DFLASH_OK: return "ok";
    case DFLASH_ERR_INVALID_ARGUMENT: return "invalid argument";
    case DFLASH_ERR_UNSUPPORTED: return "unsupported configuration";
    case DFLASH_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case DFLASH_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char *dflash_last_error(void) { return g_last_error.c_str(); }

dflash_status dflash_build_rope_table(int32_t head_dim, double theta, int32_t max_pos, float *cos_out,
                                      float *sin_out, void *stream) {
  if (head_dim <= 0 || head_dim % 2) return fail(DFLASH_ERR_INVALID_ARGUMENT, "head_dim must be positive and even");
  if (max_pos <= 0) return fail(DFLASH_ERR_INVALID_ARGUMENT, "max_pos must be positive");
  if (!(theta > 0.0)) return fail(DFLASH_ERR_INVALID_ARGUMENT, "theta must be positive");
  if (!cos_out || !sin_out) return fail(DFLASH_ERR_INVALID_ARGUMENT, "output is NULL");
  HIP_TRY(launch_rope_table(head_dim, theta, max_pos, cos_out, sin_out, (hipStream_t)stream));
  return ok();
}

dflash_status dflash_build_fused_kv_weight(const dflash_config *cfg, const dflash_weights *w, void *out,
                                           void *stream) {
  dflash_status st = check_config(cfg);
  if (st != DFLASH_OK) return st;
  if (!w || !out) return fail(DFLASH_ERR_INVALID_ARGUMENT, "weights or output is NULL");
  if (cfg->n_layers > 0 && (!w->wk || !w->wv)) return fail(DFLASH_ERR_INVALID_ARGUMENT, "wk/wv arrays are NULL");
  const size_t block = (size_t)cfg->n_kv_heads * cfg->head_dim * cfg->hidden * elem_size(cfg);
  for (int l = 0; l < cfg->n_layers; ++l) {
    if (!w->wk[l] || !w->wv[l]) return fail(DFLASH_ERR_INVALID_ARGUMENT, "wk/wv of layer %d is NULL", l);
    char *dst = static_cast<char *>(out) + (size_t)(2 * l) * block;
    HIP_TRY(hipMemcpyAsync(dst, w->wk[l], block, hipMemcpyDeviceToDevice, (hipStream_t)stream));
    HIP_TRY(hipMemcpyAsync(dst + block, w->wv[l], block, hipMemcpyDeviceToDevice, (hipStream_t)stream));
  }
  return ok();
}

size_t dflash_workspace_bytes(const dflash_config *cfg, int32_t op, int32_t max_rows_or_batch,
                              int32_t max_context) {
  if (check_config(cfg) != DFLASH_OK || max_rows_or_batch < 0 || max_context < 0) return 0;
  size_t best = kAlign;
  if (op == DFLASH_OP_INJECT) {
    const int cap = std::min<int>(max_rows_or_batch, kInjectChunk);
    for (int r = 1; r <= cap; ++r) best = std::max(best, plan_inject(cfg, r).total);
    return best;
  }
  if (op == DFLASH_OP_PROPOSE) {
    for (int b = 1; b <= max_rows_or_batch; ++b) best = std::max(best, plan_propose(cfg, b, max_context).total);
    return best;
  }
  return 0;
}

dflash_status dflash_inject_context_kv(const dflash_config *cfg, const dflash_weights *w,
                                       const dflash_kv_cache *cache, const void *const *aux, int64_t aux_row_stride,
                                       int32_t n_rows, const int32_t *positions, const int64_t *slot_mapping,
                                       void *workspace, size_t workspace_bytes, void *stream) {
  dflash_status st = check_config(cfg);
  if (st != DFLASH_OK) return st;
  if (n_rows < 0) return fail(DFLASH_ERR_INVALID_ARGUMENT, "n_rows < 0");
  if (n_rows == 0) return ok();
  if ((st = check_weights_common(cfg, w)) != DFLASH_OK) return st;
  if ((st = check_cache(cfg, cache)) != DFLASH_OK) return st;
  if (!w->fc || !w->hidden_norm || (cfg->n_layers > 0 && !w->kv_fused))
    return fail(DFLASH_ERR_INVALID_ARGUMENT, "fc, hidden_norm or kv_fused is NULL");
  if (!aux) return fail(DFLASH_ERR_INVALID_ARGUMENT, "aux is NULL");
  for (int j = 0; j < cfg->n_aux; ++j)
    if (!aux[j]) return fail(DFLASH_ERR_INVALID_ARGUMENT, "aux[%d] is NULL", j);
  if (aux_row_stride < cfg->target_hidden)
    return fail(DFLASH_ERR_INVALID_ARGUMENT, "aux_row_stride %lld < target_hidden %d", (long long)aux_row_stride,
                cfg->target_hidden);
  const int vec = is_bf16(cfg) ? 8 : 4;
  if (aux_row_stride % vec) return fail(DFLASH_ERR_UNSUPPORTED, "aux_row_stride must be a multiple of %d", vec);
  if (!positions || !slot_mapping) return fail(DFLASH_ERR_INVALID_ARGUMENT, "positions or slot_mapping is NULL");
  if (!workspace) return fail(DFLASH_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (cfg->n_layers == 0) return ok();  // nothing to write

  // Every chunk is planned before the first launch: the chunks are full ones of kInjectChunk
  // rows and one shorter tail, so two plans bound the workspace of the whole call.
  {
    size_t need = plan_inject(cfg, std::min(n_rows, kInjectChunk)).total;
    if (n_rows > kInjectChunk && n_rows % kInjectChunk)
      need = std::max(need, plan_inject(cfg, n_rows % kInjectChunk).total);
    if (need > workspace_bytes)
      return fail(DFLASH_ERR_WORKSPACE_TOO_SMALL, "inject needs %zu workspace bytes, got %zu", need,
                  workspace_bytes);
  }

  hipStream_t s = (hipStream_t)stream;
  const bool bf = is_bf16(cfg);
  const size_t es = elem_size(cfg);
  const int H = cfg->hidden, kvn = cfg->n_layers * 2 * cfg->n_kv_heads * cfg->head_dim;
  for (int r0 = 0; r0 < n_rows; r0 += kInjectChunk) {
    const int rows = std::min(kInjectChunk, n_rows - r0);
    const InjectPlan p = plan_inject(cfg, rows);
    float *y = at<float>(workspace, p.off_y);
    float *ss = at<float>(workspace, p.off_ss);
    float *part = at<float>(workspace, p.off_part);
    unsigned *ctr = at<unsigned>(workspace, p.off_ctr);
    HIP_TRY(launch_zero(ctr, p.n_ctr, s));  // each chunk's plan places the counters anew

    // fc over the concatenated auxiliary states, read in place from the n_aux pointers
    GemmArgs g = gemm_args(cfg, "gemm.fc", nullptr, aux_row_stride, rows, H, cfg->n_aux * cfg->target_hidden, ctr,
                           part);
    for (int j = 0; j < cfg->n_aux; ++j)
      g.a[j] = static_cast<const char *>(aux[j]) + (size_t)r0 * aux_row_stride * es;
    g.a_nseg = cfg->n_aux;
    g.a_f32 = false;  // the auxiliary states come in the storage type
    g.b[0] = w->fc;
    g.b_end[0] = H;
    g.out = y;
    g.ss_out = ss;
    HIP_TRY(launch_gemm(g, bf, GemmEpi::kStore, p.fc, s));

    // hidden_norm on load; K/V of every layer in one projection; k_norm + RoPE + scatter
    GemmArgs k = gemm_args(cfg, "gemm.kv", y, H, rows, kvn, H, ctr, part);
    k.a_split = at<uint16_t>(workspace, p.off_split);
    set_norm(k, w->hidden_norm, ss, p.fc.col_groups, rows);
    k.b[0] = w->kv_fused;
    k.b_end[0] = kvn;
    set_rope(k, w);
    for (int l = 0; l < cfg->n_layers; ++l) {
      k.layer_k_norm[l] = w->k_norm[l];
      k.k_cache[l] = cache->k[l];
      k.v_cache[l] = cache->v[l];
    }
    k.positions = positions + r0;
    k.slot_mapping = slot_mapping + r0;
    k.num_slots = (int64_t)cache->num_pages * cache->page_size;
    HIP_TRY(launch_gemm(k, bf, GemmEpi::kKvScatter, p.kv, s));
  }
  return ok();
}

}  // extern "C"

namespace {
// Validation of a propose call (everything but the workspace pointer) and its plan. Returns
// DFLASH_OK with *nothing = true for an empty batch.
dflash_status propose_check(const dflash_config *cfg, const dflash_weights *w, const dflash_kv_cache *cache,
                            int32_t batch, const int32_t *bonus_tokens, const int32_t *seq_lens, int32_t max_context,
                            int32_t *draft_token_ids, int32_t *drafts_only, size_t workspace_bytes,
                            ProposePlan *plan, bool *nothing) {
  *nothing = false;
  dflash_status st = check_config(cfg);
  if (st != DFLASH_OK) return st;
  if (batch < 0) return fail(DFLASH_ERR_INVALID_ARGUMENT, "batch < 0");
  if (batch == 0) {
    *nothing = true;
    return DFLASH_OK;
  }
  if (max_context < 0) return fail(DFLASH_ERR_INVALID_ARGUMENT, "max_context < 0");
  if ((st = check_weights_common(cfg, w)) != DFLASH_OK) return st;
  if ((st = check_cache(cfg, cache)) != DFLASH_OK) return st;
  if (!cache->block_table || cache->max_blocks_per_seq <= 0)
    return fail(DFLASH_ERR_INVALID_ARGUMENT, "block_table is NULL or max_blocks_per_seq <= 0");
  if (!w->embed || !w->lm_head || !w->final_norm)
    return fail(DFLASH_ERR_INVALID_ARGUMENT, "embed/lm_head/final_norm NULL");
  const int L = cfg->n_layers;
  if (L > 0 && (!w->in_norm || !w->wq || !w->wk || !w->wv || !w->q_norm || !w->wo || !w->post_norm || !w->w_gate ||
                !w->w_up || !w->w_down))
    return fail(DFLASH_ERR_INVALID_ARGUMENT, "a per-layer weight array is NULL");
  for (int l = 0; l < L; ++l)
    if (!w->in_norm[l] || !w->wq[l] || !w->wk[l] || !w->wv[l] || !w->q_norm[l] || !w->wo[l] || !w->post_norm[l] ||
        !w->w_gate[l] || !w->w_up[l] || !w->w_down[l])
      return fail(DFLASH_ERR_INVALID_ARGUMENT, "a weight of layer %d is NULL", l);
  if (!bonus_tokens || !seq_lens || !draft_token_ids || !drafts_only)
    return fail(DFLASH_ERR_INVALID_ARGUMENT, "an input/output pointer is NULL");
  *plan = plan_propose(cfg, batch, max_context);
  if (plan->total > workspace_bytes)
    return fail(DFLASH_ERR_WORKSPACE_TOO_SMALL, "propose needs %zu workspace bytes, got %zu", plan->total,
                workspace_bytes);
  return DFLASH_OK;
}

// The launch sequence of a validated propose call on the workspace `workspace`.
dflash_status propose_enqueue(const dflash_config *cfg, const dflash_weights *w, const dflash_kv_cache *cache,
                              int32_t batch, const int32_t *bonus_tokens, const int32_t *seq_lens,
                              int32_t max_context, int32_t *draft_token_ids, int32_t *drafts_only, float *hidden_out,
                              void *workspace, const ProposePlan &p, void *stream, void *cache_ready = nullptr) {
  const int L = cfg->n_layers;
  hipStream_t s = (hipStream_t)stream;
  // the first launch that reads the cache waits for `cache_ready` (when given)
  bool waited = cache_ready == nullptr;
  auto wait_cache = [&]() -> hipError_t {
    if (waited) return hipSuccess;
    waited = true;
    return hipStreamWaitEvent(s, (hipEvent_t)cache_ready, 0);
  };
  const bool bf = is_bf16(cfg);
  const int H = cfg->hidden, D = cfg->head_dim, QH = cfg->n_q_heads, KVH = cfg->n_kv_heads;
  const int I = cfg->intermediate, bs = cfg->block_size, K = bs - 1, M = p.M;
  float *x = at<float>(workspace, p.off_x);
  float *ss = at<float>(workspace, p.off_ss);
  float *part = at<float>(workspace, p.off_part);
  unsigned *ctr = at<unsigned>(workspace, p.off_ctr);
  void *q = at<char>(workspace, p.off_q);
  void *kb = at<char>(workspace, p.off_k);
  void *vb = at<char>(workspace, p.off_v);
  float *o = at<float>(workspace, p.off_o);
  float *act = at<float>(workspace, p.off_act);
  uint16_t *asplit = at<uint16_t>(workspace, p.off_split);

  HIP_TRY(launch_embed(bf, w->embed, cfg->vocab, H, bonus_tokens, batch, bs, cfg->mask_token_id, x, ss, ctr,
                       p.n_zero, s));
  int ss_groups = 1;  // column groups of the last producer of x (the embedding: one)
  const unsigned *plk_abort = nullptr;
  // the persistent layer-stack kernel, when asked for (it addresses one layer's cache with
  // 32-bit offsets)
  const char *plk_env = getenv("DFLASH_PERSISTENT_LAYERS");
  const bool use_plk = plk_env && plk_env[0] == '1' && p.plk.ok &&
                       (size_t)cache->num_pages * cache->page_size * KVH * D * 2 < (size_t(1) << 31);
  if (use_plk) {
    // the whole layer stack in one persistent launch; it leaves the final rows in x and their
    // sums of squares per 128-column tile in ss
    PlkArgs pa{};
    for (int l = 0; l < L; ++l) {
      PlkLayerW &lw = pa.lw[l];
      lw.in_norm = static_cast<const uint16_t *>(w->in_norm[l]);
      lw.wq = static_cast<const uint16_t *>(w->wq[l]);
      lw.wk = static_cast<const uint16_t *>(w->wk[l]);
      lw.wv = static_cast<const uint16_t *>(w->wv[l]);
      lw.q_norm = static_cast<const uint16_t *>(w->q_norm[l]);
      lw.k_norm = static_cast<const uint16_t *>(w->k_norm[l]);
      lw.wo = static_cast<const uint16_t *>(w->wo[l]);
      lw.post_norm = static_cast<const uint16_t *>(w->post_norm[l]);
      lw.wg = static_cast<const uint16_t *>(w->w_gate[l]);
      lw.wu = static_cast<const uint16_t *>(w->w_up[l]);
      lw.wd = static_cast<const uint16_t *>(w->w_down[l]);
      lw.kc = static_cast<const uint16_t *>(cache->k[l]);
      lw.vc = static_cast<const uint16_t *>(cache->v[l]);
    }
    pa.L = L, pa.H = H, pa.QH = QH, pa.KVH = KVH, pa.I = I, pa.bs = bs, pa.G = QH / KVH;
    pa.eps = cfg->rms_eps;
    pa.rope_cos = w->rope_cos, pa.rope_sin = w->rope_sin, pa.rope_max_pos = w->rope_max_pos;
    pa.seq_lens = seq_lens, pa.max_ctx = max_context;
    pa.block_table = cache->block_table, pa.maxb = cache->max_blocks_per_seq, pa.P = cache->page_size;
    pa.num_pages = cache->num_pages;
    for (int i = 0; i < 4; ++i) pa.g[i] = p.plk.g[i];
    pa.ntile = p.plk.ntile, pa.ns = p.plk.ns, pa.nwg = p.plk.nwg;
    pa.rm = p.plk.rm, pa.nrp = p.plk.nrp;
    char *base = at<char>(workspace, p.off_plk);
    pa.x0 = x, pa.ss0 = ss;
    pa.xs = reinterpret_cast<float *>(base + p.plk.off_xs);
    pa.sss = reinterpret_cast<float *>(base + p.plk.off_sss);
    pa.qkv = reinterpret_cast<uint16_t *>(base + p.plk.off_qkv);
    pa.o = reinterpret_cast<float *>(base + p.plk.off_o);
    pa.act = reinterpret_cast<float *>(base + p.plk.off_act);
    pa.apo = reinterpret_cast<float *>(base + p.plk.off_apo);
    pa.apm = reinterpret_cast<float *>(base + p.plk.off_apm);
    pa.apl = reinterpret_cast<float *>(base + p.plk.off_apl);
    for (int i = 0; i < 4; ++i) pa.gpart[i] = reinterpret_cast<float *>(base + p.plk.off_gpart[i]);
    pa.sync = ctr + p.n_ctr;
    pa.ws = workspace, pa.ws_bytes = (unsigned)p.total;
    plk_abort = pa.sync + p.plk.sync_words - 1;
    HIP_TRY(wait_cache());
    HIP_TRY(launch_plk(pa, s));
    ss_groups = H / 128;
  }
  for (int l = 0; l < (use_plk ? 0 : L); ++l) {
    // input_layernorm on load; q | k | v in one pass; q/k norm + RoPE in the epilogue
    GemmArgs g = gemm_args(cfg, "gemm.qkv", x, H, M, (QH + 2 * KVH) * D, H, ctr, part);
    g.a_split = asplit;
    set_norm(g, w->in_norm[l], ss, ss_groups, M);
    g.b[0] = w->wq[l];
    g.b[1] = w->wk[l];
    g.b[2] = w->wv[l];
    g.b_end[0] = QH * D;
    g.b_end[1] = (QH + KVH) * D;
    g.b_end[2] = (QH + 2 * KVH) * D;
    g.b_nseg = 3;
    g.q_norm = w->q_norm[l];
    g.k_norm = w->k_norm[l];
    g.seq_lens = seq_lens;
    g.max_ctx = max_context;
    set_rope(g, w);
    g.q = q;
    g.k = kb;
    g.v = vb;
    HIP_TRY(launch_gemm(g, bf, GemmEpi::kHeadNormRope, p.qkv, s));

    AttnArgs at_{};
    at_.q = q;
    at_.kb = kb;
    at_.vb = vb;
    at_.kc = cache->k[l];
    at_.vc = cache->v[l];
    at_.block_table = cache->block_table;
    at_.maxb = cache->max_blocks_per_seq;
    at_.P = cache->page_size;
    at_.num_pages = cache->num_pages;
    at_.seq_lens = seq_lens;
    at_.max_ctx = max_context;
    at_.B = batch;
    at_.bs = bs;
    at_.QH = QH;
    at_.KVH = KVH;
    at_.D = D;
    at_.chunk = p.chunk;
    at_.nsplit = p.nsplit;
    at_.po = at<float>(workspace, p.off_po);
    at_.pm = at<float>(workspace, p.off_pm);
    at_.pl = at<float>(workspace, p.off_pl);
    at_.o = o;
    // many rows: the merged output as the (hi, lo) planes the O projection takes, in the o
    // buffer (two bf16 planes fill its M x QH*D floats), so O runs no split pass
    const bool o_planes = p.o.tiled && !p.o.hi_only;
    at_.o_planes = o_planes ? reinterpret_cast<uint16_t *>(o) : nullptr;
    HIP_TRY(wait_cache());
    if (batch > 1) {
      // the work-groups that have keys, listed once for every layer (same sequence lengths)
      int *items = at<int>(workspace, p.off_items), *n_items = items + (size_t)batch * KVH * p.nsplit;
      if (l == 0) HIP_TRY(launch_attention_items(at_, items, n_items, s));
      at_.items = items, at_.n_items = n_items;
    }
    HIP_TRY(launch_attention(bf, at_, s));

    // O projection + residual add; the row sums of squares feed the post-attention norm
    GemmArgs go = gemm_args(cfg, "gemm.o", o, QH * D, M, H, QH * D, ctr, part);
    go.a_split = asplit;
    if (o_planes) go.a_planes = reinterpret_cast<const uint16_t *>(o);
    go.b[0] = w->wo[l];
    go.b_end[0] = H;
    go.out = x;
    go.ss_out = ss;
    HIP_TRY(launch_gemm(go, bf, GemmEpi::kResidAdd, p.o, s));
    ss_groups = p.o.col_groups;

    // post_attention_layernorm on load; gate | up with SwiGLU
    GemmArgs gu = gemm_args(cfg, "gemm.gate_up", x, H, M, I, H, ctr, part);
    gu.a_split = asplit;
    set_norm(gu, w->post_norm[l], ss, ss_groups, M);
    gu.b[0] = w->w_gate[l];
    gu.b[1] = w->w_up[l];
    gu.b_end[0] = I;
    gu.b_end[1] = I;
    gu.b_nseg = 2;
    gu.out = act;
    // many rows: gate|up writes its product as the (hi, lo) planes the down projection takes,
    // in the act buffer (two bf16 planes fill its M x I floats), so no split pass runs
    const bool act_planes = p.gu.tiled && p.down.tiled && !p.down.hi_only;
    if (act_planes) gu.out_planes = reinterpret_cast<uint16_t *>(act);
    HIP_TRY(launch_gemm(gu, bf, GemmEpi::kSwiGLU, p.gu, s));

    GemmArgs gd = gemm_args(cfg, "gemm.down", act, I, M, H, I, ctr, part);
    gd.a_split = asplit;
    if (act_planes) gd.a_planes = reinterpret_cast<const uint16_t *>(act);
    gd.b[0] = w->w_down[l];
    gd.b_end[0] = H;
    gd.out = x;
    gd.ss_out = ss;
    HIP_TRY(launch_gemm(gd, bf, GemmEpi::kResidAdd, p.down, s));
    ss_groups = p.down.col_groups;
  }

  // final norm on load over the drafted rows (block slots 1..K); LM head + per-group argmax
  GemmArgs gl = gemm_args(cfg, "gemm.lm_head", x, H, p.Mk, cfg->vocab, H, ctr, part);
  gl.a_split = asplit;
  set_norm(gl, w->final_norm, ss, ss_groups, M);
  gl.keep_bs = bs;
  gl.a_out = hidden_out;
  gl.b[0] = w->lm_head;
  gl.b_end[0] = cfg->vocab;
  gl.amax_val = at<float>(workspace, p.off_amv);
  gl.amax_idx = at<int32_t>(workspace, p.off_ami);
  HIP_TRY(launch_gemm(gl, bf, GemmEpi::kArgmax, p.lm, s));
  HIP_TRY(launch_argmax_reduce(batch, K, p.lm.col_groups, gl.amax_val, gl.amax_idx, bonus_tokens, cfg->vocab,
                               plk_abort, draft_token_ids, drafts_only, s));
  HIP_TRY(wait_cache());  // no layer read the cache: the call still ends after the event
  return ok();
}

// The static scratch of dflash_propose_block_noalloc: one copy per GPU the library runs on,
// held until the process ends. In host code `scratch` names a host-side stand-in, never the
// device memory: its device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kStaticScratchBytes = (size_t)DFLASH_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (looked up on the first call on a device).
dflash_status static_scratch(void **out) {
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(DFLASH_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(DFLASH_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DFLASH_OK;
}
}  // namespace

extern "C" {

dflash_status dflash_propose_block(const dflash_config *cfg, const dflash_weights *w, const dflash_kv_cache *cache,
                                   int32_t batch, const int32_t *bonus_tokens, const int32_t *seq_lens,
                                   int32_t max_context, int32_t *draft_token_ids, int32_t *drafts_only,
                                   float *hidden_out, void *workspace, size_t workspace_bytes, void *stream) {
  ProposePlan p{};
  bool nothing = false;
  dflash_status st = propose_check(cfg, w, cache, batch, bonus_tokens, seq_lens, max_context, draft_token_ids,
                                   drafts_only, workspace_bytes, &p, &nothing);
  if (st != DFLASH_OK) return st;
  if (nothing) return ok();
  if (!workspace) return fail(DFLASH_ERR_INVALID_ARGUMENT, "workspace is NULL");
  return propose_enqueue(cfg, w, cache, batch, bonus_tokens, seq_lens, max_context, draft_token_ids, drafts_only,
                         hidden_out, workspace, p, stream);
}

dflash_status dflash_propose_block_after(const dflash_config *cfg, const dflash_weights *w,
                                         const dflash_kv_cache *cache, int32_t batch, const int32_t *bonus_tokens,
                                         const int32_t *seq_lens, int32_t max_context, int32_t *draft_token_ids,
                                         int32_t *drafts_only, float *hidden_out, void *workspace,
                                         size_t workspace_bytes, void *cache_ready, void *stream) {
  ProposePlan p{};
  bool nothing = false;
  dflash_status st = propose_check(cfg, w, cache, batch, bonus_tokens, seq_lens, max_context, draft_token_ids,
                                   drafts_only, workspace_bytes, &p, &nothing);
  if (st != DFLASH_OK) return st;
  if (nothing) return ok();
  if (!workspace) return fail(DFLASH_ERR_INVALID_ARGUMENT, "workspace is NULL");
  return propose_enqueue(cfg, w, cache, batch, bonus_tokens, seq_lens, max_context, draft_token_ids, drafts_only,
                         hidden_out, workspace, p, stream, cache_ready);
}

dflash_status dflash_propose_block_noalloc(const dflash_config *cfg, const dflash_weights *w,
                                           const dflash_kv_cache *cache, int32_t batch, const int32_t *bonus_tokens,
                                           const int32_t *seq_lens, int32_t max_context, int32_t *draft_token_ids,
                                           int32_t *drafts_only, float *hidden_out, void *stream) {
  ProposePlan p{};
  bool nothing = false;
  dflash_status st = propose_check(cfg, w, cache, batch, bonus_tokens, seq_lens, max_context, draft_token_ids,
                                   drafts_only, kStaticScratchBytes, &p, &nothing);
  if (st != DFLASH_OK) {
    if (st == DFLASH_ERR_WORKSPACE_TOO_SMALL)
      return fail(st, "propose needs %zu bytes of scratch; the static scratch holds %zu (use dflash_propose_block "
                  "with a workspace)", p.total, kStaticScratchBytes);
    return st;
  }
  if (nothing) return ok();
  void *ws = nullptr;
  if ((st = static_scratch(&ws)) != DFLASH_OK) return st;
  return propose_enqueue(cfg, w, cache, batch, bonus_tokens, seq_lens, max_context, draft_token_ids, drafts_only,
                         hidden_out, ws, p, stream);
}

namespace {
dflash_status verify_impl(int32_t batch, int32_t num_drafts, const int32_t *draft_tokens,
                          const int32_t *target_tokens, int32_t *accepted_len, int32_t *output_tokens,
                          int32_t *next_bonus, int64_t *stats, void *stream) {
  if (batch < 0) return fail(DFLASH_ERR_INVALID_ARGUMENT, "batch < 0");
  if (num_drafts < 1 || num_drafts > 63)
    return fail(DFLASH_ERR_UNSUPPORTED, "num_drafts %d outside [1, 63]", num_drafts);
  if (batch == 0) return ok();
  if (!draft_tokens || !target_tokens || !accepted_len || !output_tokens || !next_bonus)
    return fail(DFLASH_ERR_INVALID_ARGUMENT, "an input/output pointer is NULL");
  HIP_TRY(launch_verify(batch, num_drafts, draft_tokens, target_tokens, accepted_len, output_tokens, next_bonus,
                        stats, (hipStream_t)stream));
  return ok();
}
}  // namespace

dflash_status dflash_greedy_verify(int32_t batch, int32_t num_drafts, const int32_t *draft_tokens,
                                   const int32_t *target_tokens, int32_t *accepted_len, int32_t *output_tokens,
                                   int32_t *next_bonus, void *stream) {
  return verify_impl(batch, num_drafts, draft_tokens, target_tokens, accepted_len, output_tokens, next_bonus,
                     nullptr, stream);
}

dflash_status dflash_greedy_verify_stats(int32_t batch, int32_t num_drafts, const int32_t *draft_tokens,
                                         const int32_t *target_tokens, int32_t *accepted_len,
                                         int32_t *output_tokens, int32_t *next_bonus, int64_t *stats,
                                         void *stream) {
  if (!stats && batch > 0) return fail(DFLASH_ERR_INVALID_ARGUMENT, "stats is NULL");
  return verify_impl(batch, num_drafts, draft_tokens, target_tokens, accepted_len, output_tokens, next_bonus,
                     stats, stream);
}

dflash_status dflash_prepare_proposal_inputs(int32_t batch, int32_t prev_num_drafts, const int32_t *prev_out,
                                             int32_t vocab, const int32_t *opt_seq_lens, int32_t n_rows,
                                             const int32_t *row_req, const int32_t *opt_positions,
                                             const int32_t *block_table, int32_t max_blocks_per_seq,
                                             int32_t page_size, int32_t *seq_lens, int32_t *positions,
                                             int64_t *slot_mapping, int32_t *bonus, void *stream) {
  if (batch < 0 || n_rows < 0) return fail(DFLASH_ERR_INVALID_ARGUMENT, "batch or n_rows < 0");
  if (prev_num_drafts < 0 || prev_num_drafts > 63)
    return fail(DFLASH_ERR_UNSUPPORTED, "prev_num_drafts %d outside [0, 63]", prev_num_drafts);
  if (vocab <= 0 || page_size <= 0 || max_blocks_per_seq <= 0)
    return fail(DFLASH_ERR_INVALID_ARGUMENT, "vocab, page_size and max_blocks_per_seq must be positive");
  if (batch == 0) {
    if (n_rows > 0) return fail(DFLASH_ERR_INVALID_ARGUMENT, "context rows without requests");
    return ok();
  }
  if (!prev_out || !opt_seq_lens || !block_table || !seq_lens || !bonus)
    return fail(DFLASH_ERR_INVALID_ARGUMENT, "a request input/output pointer is NULL");
  if (n_rows > 0 && (!row_req || !opt_positions || !positions || !slot_mapping))
    return fail(DFLASH_ERR_INVALID_ARGUMENT, "a row input/output pointer is NULL");
  PrepareArgs a{};
  a.B = batch;
  a.K = prev_num_drafts;
  a.V = vocab;
  a.n_rows = n_rows;
  a.maxb = max_blocks_per_seq;
  a.P = page_size;
  a.prev_out = prev_out;
  a.opt_seq_lens = opt_seq_lens;
  a.row_req = row_req;
  a.opt_positions = opt_positions;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.positions = positions;
  a.bonus = bonus;
  a.slot_mapping = slot_mapping;
  HIP_TRY(launch_prepare(a, (hipStream_t)stream));
  return ok();
}

}  // extern "C"
