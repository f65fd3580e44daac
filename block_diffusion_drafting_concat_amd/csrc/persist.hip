// Persistent layer-stack kernel: the whole drafter layer stack of one block (batch 1, at most 16
// rows, bf16 weights, head_dim 128) in one launch. Selected by DFLASH_PERSISTENT_LAYERS=1 (the
// per-projection launches are the default: on MI355X they measured faster at the Qwen3-8B shape).
//
// At batch 1 every projection is a weight stream, and a launch per projection pays a ramp (the
// first loads of every work-group arrive together) and a tail (split-K hand-off, slowest
// work-group) each time. Here one work-group per CU runs a fixed list of jobs for every layer:
// QKV chunks, attention tiles, split merges, O chunks, gate|up chunks and down chunks. A GEMM
// job is one K chunk of one 128-column output tile (256 columns of one matrix, or 128 columns
// of gate and of up); the tiles x chunks units of a projection are dealt to the work-groups in
// contiguous ranges, so a work-group accumulates consecutive chunks of one tile in registers and
// hands partial tiles on only where its range starts or ends inside a tile.
//
// Eight waves per work-group:
//  * waves 0-3 compute: each owns 32 output columns (two 16-column MFMA tiles) of the job's
//    tile, streams its weight rows straight into registers and feeds v_mfma_f32_16x16x32_bf16
//    (the fp32 activations as hi = bf16(f), lo = bf16(f - hi), two MFMAs per step). The weights
//    of the next two GEMM jobs are in flight while a job computes: weights do not depend on
//    activations, so HBM keeps streaming while jobs wait for their inputs;
//  * waves 4-6 stage (job k on wave 4 + k % 3): a GEMM job waits for the producer tiles that
//    cover its K range (readiness flags; a normalised input waits for every tile of its rows,
//    whose sums of squares give the RMSNorm row scale) and stages its activations in one of six
//    LDS slots (16 rows x K chunk, times the norm weight and the row scale); an attention job
//    stages q, the tile's 64 keys and V^T; a merge job combines the attention splits of one q
//    head and a few block rows;
//  * wave 7 finishes: it stores a partial tile, counts it on the tile's counter and, as the
//    last contributor, sums the partials in contributor order and runs the epilogue (q/k
//    RMSNorm + RoPE, residual add with row sums of squares, SwiGLU); then it raises the tile's
//    readiness flag. It also computes the attention tiles (every query row of the kv group).
// The waves hand off through LDS words (per activation slot the job staged in it, jobs
// consumed, attention tiles staged and done, output tiles written and finished), so no wave
// waits at a barrier: the stagers run up to six GEMM jobs ahead of the compute waves.
//
// Everything one work-group hands to another inside the launch (activations, partials, flags,
// counters) is written and read with device-scope (sc1) accesses, which are coherent across
// the XCDs' L2 caches. A writer waits for its stores (s_waitcnt) before it raises a flag or
// counts on a counter, and a reader reads data only after it has seen the flag; that the
// stores are then visible to the reader is the same hardware ordering the split-K hand-off of
// the streaming GEMM relies on. Every wait is bounded: past about a second, or once any wave
// has given up, a work-group raises the abort word and runs on without waiting, so the grid
// always drains; the LM-head argmax then reports -1 drafts.
//
// The work-groups must all be resident at once (they wait for each other): one work-group per
// CU (about 152 KiB of LDS each), as many as the GPU has CUs, and nothing else may depend on
// this launch while it runs.
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "stream_core.h"

namespace dflash {
namespace {
using namespace wave;

constexpr int kStagers = 3;  // stager waves 4..6: job k is staged by wave 4 + k % 3
constexpr int kWaves = 4 + kStagers + 1, kThreads = kWaves * 64;
constexpr int kD = 128;     // head dim
constexpr int kKrMax = 256;  // K columns of a chunk (one weight matrix)
constexpr int kArow = kKrMax * 4 + 16;  // LDS bytes of one staged row: 32 B per 8 columns + pad
constexpr int kQs = kD + 8, kKs = kD + 8, kVs = 64 + 8;  // LDS row strides (bf16) of q, K, V^T
constexpr int kNA = 6;                   // activation slots of GEMM jobs
constexpr int kAslot = 16 * kArow;       // one staged GEMM chunk (16640 B)
constexpr int kAttnBytes = (64 * kQs + 64 * kKs + kD * kVs) * 2;  // an attention tile (53248 B)
constexpr int kOslot = 16 * kTN * 4 * 2;  // one output slot (16 KiB)
constexpr int kLds = kNA * kAslot + 2 * kOslot;  // plus the job list
static_assert(kAttnBytes <= kNA * kAslot, "an attention tile fits the activation slots");

enum Stage { kSQkv = 0, kSAttn = 1, kSMerge = 2, kSO = 3, kSGu = 4, kSDown = 5 };
__device__ __forceinline__ int ph_of(int st) { return st == kSQkv ? 0 : st == kSO ? 1 : st == kSGu ? 2 : 3; }

// ---- sync words: per layer [counters of the 4 GEMM phases][their flags][attention counters per
//      kv head][merge flags per q head and row group]; the abort word after the last layer
struct Sync {
  unsigned *base;
  int per_layer, t0, t1, t2, tsum, off_a, off_m;
  __device__ Sync(const PlkArgs &a) : base(a.sync) {
    t0 = a.g[0].tiles;
    t1 = t0 + a.g[1].tiles;
    t2 = t1 + a.g[2].tiles;
    tsum = t2 + a.g[3].tiles;
    off_a = 2 * tsum;
    off_m = off_a + a.KVH;
    per_layer = off_m + a.QH * a.nrp;
  }
  __device__ int off_c(int p) const { return p == 0 ? 0 : p == 1 ? t0 : p == 2 ? t1 : t2; }
  __device__ unsigned *ctr(int l, int p, int t) const { return base + l * per_layer + off_c(p) + t; }
  __device__ unsigned *flag(int l, int p, int t) const { return base + l * per_layer + tsum + off_c(p) + t; }
  __device__ unsigned *actr(int l, int g) const { return base + l * per_layer + off_a + g; }
  __device__ unsigned *mflag(int l, int h) const { return base + l * per_layer + off_m + h; }
  __device__ unsigned *abort_word(int L) const { return base + L * per_layer; }
};

// The abort words: one in global memory for the grid, one in LDS for the work-group. A wave
// that waits past the time limit raises both; a wave that sees either stops waiting.
// (The work-group word is accessed through an LDS pointer: a generic access would also count
// on the vector-memory counter and wait for every weight load in flight.)
struct Abort {
  unsigned *grid;
  int *wg;
  __device__ __forceinline__ bool up() const { return *(lds_vint *)wg != 0; }
  __device__ __forceinline__ void raise() const {
    *(lds_vint *)wg = 1;
    if ((threadIdx.x & 63) == 0) stcu(grid, 1u);
  }
};

// One wave waits until the n words w[i * stride] (i < n) in global memory are all >= want.
// Lanes poll one word each, 64 at a time.
__device__ __forceinline__ void wave_wait(const unsigned *w, int stride, int n, unsigned want, const Abort &ab) {
  const int lane = threadIdx.x & 63;
  const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
  for (int b = 0; b < n; b += 64) {
    while (true) {
      const bool ok = b + lane >= n || ldcu(w + (size_t)(b + lane) * stride) >= want;
      if (__ballot(!ok) == 0) break;
      if (ab.up()) return;
      if (ldcu(ab.grid)) {
        *(lds_vint *)ab.wg = 1;
        return;
      }
      if (__builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) {
        ab.raise();
        return;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
}

// A wave waits until the LDS word *p >= want (hand-offs between the waves of the work-group).
__device__ __forceinline__ void lds_wait(const int *p, int want, const Abort &ab) {
  if (lds_load(p) >= want) return;
  const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
  while (lds_load(p) < want) {
    if (ab.up()) return;
    if (__builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) {
      ab.raise();
      return;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// ---- the job list of work-group w: per layer, its QKV units, attention tiles, merge, O, gate|up
//      and down units
__device__ __forceinline__ int gemm_u0(const PlkGemm &g, int w) { return w * g.base + min(w, g.rem); }
__device__ __forceinline__ int gemm_n(const PlkGemm &g, int w) { return g.base + (w < g.rem ? 1 : 0); }
__device__ __forceinline__ int gemm_owner(const PlkGemm &g, int u) {
  const int big = g.rem * (g.base + 1);
  return u < big ? u / (g.base + 1) : g.rem + (u - big) / g.base;
}
__device__ __forceinline__ int tile_lo(const PlkArgs &a, int s) { return s * a.ntile / a.ns; }
// merge job of work-group w (valid below QH * nrp): q head m / nrp, row group m % nrp; the
// first merge jobs go to the work-groups without attention tiles
__device__ __forceinline__ int merge_index(const PlkArgs &a, int w) {
  int m = (w - a.KVH * a.ns) % a.nwg;
  return m < 0 ? m + a.nwg : m;
}

__device__ __forceinline__ int stage_count(const PlkArgs &a, int w, int st) {
  switch (st) {
    case kSAttn: {
      if (w >= a.KVH * a.ns) return 0;
      const int s = w % a.ns;
      return tile_lo(a, s + 1) - tile_lo(a, s);
    }
    case kSMerge: return merge_index(a, w) < a.QH * a.nrp ? 1 : 0;
    default: return gemm_n(a.g[ph_of(st)], w);
  }
}

struct Cur {
  int l, st, i;
};
__device__ __forceinline__ Cur cur_norm(const PlkArgs &a, int w, Cur c) {
  while (c.l < a.L) {
    if (c.i < stage_count(a, w, c.st)) return c;
    c.i = 0;
    if (++c.st == 6) c.st = 0, ++c.l;
  }
  return c;
}
__device__ __forceinline__ Cur cur_first(const PlkArgs &a, int w) { return cur_norm(a, w, Cur{0, 0, 0}); }
__device__ __forceinline__ Cur cur_next(const PlkArgs &a, int w, Cur c) {
  ++c.i;
  return cur_norm(a, w, c);
}
__device__ __forceinline__ Cur cur_next_gemm(const PlkArgs &a, int w, Cur c) {
  do c = cur_next(a, w, c);
  while (c.l < a.L && (c.st == kSAttn || c.st == kSMerge));
  return c;
}

struct Job {
  int kind;  // 0 end, 1 GEMM chunk, 2 attention tile, 3 merge (t: row group)
  int l, st, ph, t, kc, g, s, tile, head;
  bool flush, last, first;
};
__device__ __forceinline__ Job cur_job(const PlkArgs &a, int w, Cur c) {
  Job j{};
  if (c.l >= a.L) return j;
  j.l = c.l;
  j.st = c.st;
  j.last = c.i == stage_count(a, w, c.st) - 1;
  if (c.st == kSAttn) {
    j.kind = 2;
    j.g = w / a.ns;
    j.s = w % a.ns;
    j.tile = tile_lo(a, j.s) + c.i;
    j.first = c.i == 0;
    j.flush = j.last;
  } else if (c.st == kSMerge) {
    j.kind = 3;
    const int m = merge_index(a, w);
    j.head = m / a.nrp;
    j.t = m % a.nrp;  // row group
    j.g = j.head / a.G;
    j.flush = true;
  } else {
    j.kind = 1;
    j.ph = ph_of(c.st);
    const PlkGemm &g = a.g[j.ph];
    const int u = gemm_u0(g, w) + c.i;
    j.t = u / g.chunks;
    j.kc = u % g.chunks;
    j.flush = j.kc == g.chunks - 1 || j.last;
    j.first = c.i == 0 || j.kc == 0;
  }
  return j;
}

// ---- the work-group's job list, built once in LDS: one descriptor per job
constexpr int kMaxJobs = 256;
struct JobD {
  int kind, ph, l, t, kc, g, s, tile, head;
  int flush, last, first;
  int ng;     // the next GEMM job of the list (this one when none is left)
  int K, kr;  // GEMM: reduction length, K columns of the chunk
  // sequence numbers within the work-group's list: GEMM jobs before this one (a GEMM job's
  // activation slot is gb % kNA), attention tiles before it, GEMM flushes before it (a flush's
  // output slot is fb % 2)
  int gb, ab, fb;
  const uint16_t *w0, *w1;  // GEMM: weight rows of the tile (w1: the up matrix of gate|up)
};
__device__ __forceinline__ Job job_of(const JobD &d) {
  Job j{};
  j.kind = d.kind, j.ph = d.ph, j.l = d.l, j.t = d.t, j.kc = d.kc, j.g = d.g, j.s = d.s, j.tile = d.tile;
  j.head = d.head, j.flush = d.flush, j.last = d.last, j.first = d.first;
  return j;
}

// ---- the x rows and their sums of squares: version 2l is the input of layer l (0: the
//      embedding; 2L: the final rows), 2l + 1 the rows after layer l's attention
__device__ __forceinline__ float *xver(const PlkArgs &a, int k) {
  return (k == 0 || k == 2 * a.L) ? a.x0 : a.xs + (size_t)(k - 1) * 16 * a.H;
}
__device__ __forceinline__ float *ssver(const PlkArgs &a, int k) {
  return (k == 0 || k == 2 * a.L) ? a.ss0 : a.sss + (size_t)(k - 1) * (a.H / kTN) * 16;
}
__device__ __forceinline__ uint16_t *qkv_of(const PlkArgs &a, int l) {
  return a.qkv + (size_t)l * 16 * (a.QH + 2 * a.KVH) * kD;
}

// GEMM phase geometry: the weight rows of tile t (matrix `m` of gate|up), the reduction
// length, the activation source and its norm weight
struct GemmSrc {
  const uint16_t *w0, *w1;  // tile rows [128][K] (w1: the up matrix of gate|up)
  int K, nacc;
  const float *a;          // activation rows [16][K]
  const uint16_t *norm_w;  // normalised input: the norm weight, else null
};
__device__ __forceinline__ GemmSrc gemm_src(const PlkArgs &a, int l, int ph, int t) {
  const PlkLayerW &L = a.lw[l];
  GemmSrc s{};
  s.nacc = 1;
  if (ph == 0) {
    s.K = a.H;
    const uint16_t *b = t < a.QH ? L.wq + (size_t)t * kTN * a.H
                        : t < a.QH + a.KVH ? L.wk + (size_t)(t - a.QH) * kTN * a.H
                                           : L.wv + (size_t)(t - a.QH - a.KVH) * kTN * a.H;
    s.w0 = s.w1 = b;
    s.a = xver(a, 2 * l);
    s.norm_w = L.in_norm;
  } else if (ph == 1) {
    s.K = a.QH * kD;
    s.w0 = s.w1 = L.wo + (size_t)t * kTN * s.K;
    s.a = a.o + (size_t)l * 16 * s.K;
  } else if (ph == 2) {
    s.K = a.H;
    s.nacc = 2;
    s.w0 = L.wg + (size_t)t * kTN * a.H;
    s.w1 = L.wu + (size_t)t * kTN * a.H;
    s.a = xver(a, 2 * l + 1);
    s.norm_w = L.post_norm;
  } else {
    s.K = a.I;
    s.w0 = s.w1 = L.wd + (size_t)t * kTN * a.I;
    s.a = a.act + (size_t)l * 16 * a.I;
  }
  return s;
}

// =============================================================================================
// Compute waves
// =============================================================================================
__device__ __forceinline__ void issue_w(const JobD &d, WBuf &b, int cw, int lane) {
  issue_w(d.w0, d.w1, d.K, d.kc, d.kr, d.ph == 2, b, cw, lane);
}

// Attention tile of job j for query rows 16 * cw + lane % 16 (the finisher wave runs the four
// 16-row tiles in turn): S^T = K Q^T over the
// slot's 64 keys, online softmax, O^T += V^T P^T (the key order inside the MFMAs is permuted so
// that the 8 keys a lane holds after two score tiles are the 8 consecutive keys of its P^T
// operand; P enters the bf16 MFMA as a hi + lo pair).
struct AttnState {
  f32x4_t o[kD / 16];
  float m, l;
};
__device__ __forceinline__ void attn_tile(const PlkArgs &a, const Job &j, const unsigned char *slot, AttnState &st, int c,
                                          int cw, int lane) {
  const uint16_t *qs = reinterpret_cast<const uint16_t *>(slot);
  const uint16_t *ks = qs + 64 * kQs;
  const uint16_t *vts = ks + 64 * kKs;
  const int R = a.bs * a.G;
  if (cw * 16 >= R) return;
  const int T = c + a.bs, t0 = j.tile * 64;
  Vec16 qf[kD / 32];
#pragma unroll
  for (int dc = 0; dc < kD / 32; ++dc)
    qf[dc].u = *reinterpret_cast<const uint4 *>(qs + (cw * 16 + (lane & 15)) * kQs + dc * 32 + (lane >> 4) * 8);
  f32x4_t s[4];
#pragma unroll
  for (int sb = 0; sb < 4; ++sb) {
    s[sb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int rho = lane & 15;
    const int key = (sb / 2) * 32 + 8 * (rho / 4) + 4 * (sb % 2) + rho % 4;
#pragma unroll
    for (int dc = 0; dc < kD / 32; ++dc) {
      Vec16 kf;
      kf.u = *reinterpret_cast<const uint4 *>(ks + key * kKs + dc * 32 + (lane >> 4) * 8);
      mma16<uint16_t>(s[sb], kf, qf[dc]);
    }
  }
  const float scale = 1.4426950408889634f / sqrtf((float)kD);  // log2(e) / sqrt(D)
  float tmax = -INFINITY;
#pragma unroll
  for (int sb = 0; sb < 4; ++sb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = (sb / 2) * 32 + 8 * (lane >> 4) + 4 * (sb % 2) + i;
      const float v = t0 + key < T ? s[sb][i] * scale : -INFINITY;
      s[sb][i] = v;
      tmax = fmaxf(tmax, v);
    }
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
  const float m_new = fmaxf(st.m, tmax);
  const float alpha = m_new == -INFINITY ? 1.f : exp2f(st.m - m_new);
  st.m = m_new;
  st.l *= alpha;
#pragma unroll
  for (int i = 0; i < kD / 16; ++i) st.o[i] *= alpha;
#pragma unroll
  for (int sb = 0; sb < 4; ++sb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = s[sb][i] == -INFINITY ? 0.f : exp2f(s[sb][i] - m_new);
      s[sb][i] = p;
      st.l += p;
    }
#pragma unroll
  for (int ps = 0; ps < 2; ++ps) {
    uint16_t hi[8], lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = s[ps * 2 + e / 4][e % 4];
      hi[e] = f32_to_bf16(p);
      lo[e] = f32_to_bf16(p - bf16_to_f32(hi[e]));
    }
    Vec16 phi, plo;
    __builtin_memcpy(&phi.u, hi, 16);
    __builtin_memcpy(&plo.u, lo, 16);
#pragma unroll
    for (int db = 0; db < kD / 16; ++db) {
      Vec16 vf;
      vf.u = *reinterpret_cast<const uint4 *>(vts + (db * 16 + (lane & 15)) * kVs + ps * 32 + (lane >> 4) * 8);
      mma16<uint16_t>(st.o[db], vf, phi);
      mma16<uint16_t>(st.o[db], vf, plo);
    }
  }
}

// The split's partial (unnormalised output, running max, running sum) of query rows
// 16 rt + lane % 16 to the workspace.
__device__ __forceinline__ void attn_store(const PlkArgs &a, const Ws &ws, const Job &j, AttnState &st, int rt, int lane) {
  const int R = a.bs * a.G;
  if (rt * 16 >= R) return;
  st.l += __shfl_xor(st.l, 16, 64);
  st.l += __shfl_xor(st.l, 32, 64);
  const int r = rt * 16 + (lane & 15);
  const size_t row = (size_t)(j.g * a.ns + j.s) * 64 + r;
  if (r < R) {
#pragma unroll
    for (int db = 0; db < kD / 16; ++db) {
      float *p = a.apo + row * kD + db * 16 + (lane >> 4) * 4;
      wst128(ws, p, make_uint4(__float_as_uint(st.o[db][0]), __float_as_uint(st.o[db][1]),
                               __float_as_uint(st.o[db][2]), __float_as_uint(st.o[db][3])));
    }
    if (lane < 16) {
      wstf(ws, a.apm + row, st.m);
      wstf(ws, a.apl + row, st.l);
    }
  }
}

// =============================================================================================
// Stager wave
// =============================================================================================
// Activations of GEMM job j: rows [16][kr] of the source times the norm weight, as 32-byte
// chunks [8 bf16 hi][8 bf16 lo] per 8 columns; rows past the block are zero.
__device__ __forceinline__ void stage_gemm(const PlkArgs &a, const Ws &ws, const Sync &sy, const Job &j, unsigned char *slot,
                                           const Abort &abort_w) {
  const int lane = threadIdx.x & 63;
  const PlkGemm &g = a.g[j.ph];
  const int kr = g.kr, k0 = j.kc * kr;
  // producer tiles of columns [k0, k0 + kr); a normalised input (QKV, gate|up) needs every tile
  // of its rows, for the rows' sums of squares
  const int p0 = k0 / kTN, np = (k0 + kr - 1) / kTN - p0 + 1;
  const int H128 = a.H / kTN;
  if (j.ph == 0) {
    if (j.l > 0) wave_wait(sy.flag(j.l - 1, 3, 0), 1, H128, 1u, abort_w);
  } else if (j.ph == 1) {
    wave_wait(sy.mflag(j.l, p0 * a.nrp), 1, np * a.nrp, 1u, abort_w);
  } else if (j.ph == 2) {
    wave_wait(sy.flag(j.l, 1, 0), 1, H128, 1u, abort_w);
  } else {
    wave_wait(sy.flag(j.l, 2, p0), 1, np, 1u, abort_w);
  }
  const GemmSrc s = gemm_src(a, j.l, j.ph, j.t);
  // RMSNorm row scale 1 / sqrt(mean(x^2) + eps) of the normalised input's rows, from the per-tile
  // sums of squares (the embedding rows: one sum per row): lane = row + 16 * quarter, each quarter
  // sums a quarter of the tiles; loaded with the activations below
  const int nver = j.ph == 0 ? 2 * j.l : 2 * j.l + 1, groups = nver == 0 ? 1 : H128;
  const float *ssp = ssver(a, nver) + (lane & 15);
  const int gq = (groups + 3) / 4, gb0 = (lane >> 4) * gq;
  float ssum = 0.f;
  if (s.norm_w)
    for (int q = gb0; q < min(gb0 + gq, groups); ++q) ssum += wldf(ws, ssp + q * 16);
  // lane: 8-column group lane % ng of rows u * (64 / ng) + lane / ng; all loads in one batch
  const int ng = kr / 8, rstep = 64 / ng, c8 = lane % ng;
  uint16_t w[8];
  const uint4 wv = s.norm_w ? *reinterpret_cast<const uint4 *>(s.norm_w + k0 + c8 * 8) : make_uint4(0, 0, 0, 0);
  __builtin_memcpy(w, &wv, 16);
  uint4 v[8][2];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int row = u * rstep + lane / ng;
    const bool ok = u < ng / 4 && row < a.bs;
    const float *src = s.a + (size_t)(ok ? row : 0) * s.K + k0 + c8 * 8;
    v[u][0] = wld128(ws, src);  // (rows past the block are zeroed at the LDS write: a select
    v[u][1] = wld128(ws, src + 4);  // here would wait for each load before issuing the next)
  }
  ssum += __shfl_xor(ssum, 16, 64);
  ssum += __shfl_xor(ssum, 32, 64);
  // lane m < bs: row m (rows past the block are zero and stay zero)
  const float rs = (lane & 15) < a.bs ? rsqrtf(ssum / (float)a.H + a.eps) : 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    if (u < ng / 4) {
      const int row = u * rstep + lane / ng;
      float f[8];
      __builtin_memcpy(f, v[u], 32);
      if (row >= a.bs) {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = 0.f;
      }
      if (s.norm_w) {
        const float rs_row = __shfl(rs, row, 64);
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] *= bf16_to_f32(w[e]) * rs_row;
      }
      uint16_t hl[16];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        hl[e] = f32_to_bf16(f[e]);
        hl[8 + e] = f32_to_bf16(f[e] - bf16_to_f32(hl[e]));
      }
      __builtin_memcpy(slot + row * kArow + c8 * 32, hl, 32);
    }
  }
}

// Where an attention tile's keys come from (the tile is one of these for the whole wave).
struct KeySrc {
  __amdgpu_buffer_rsrc_t kc, vc;  // the layer's paged cache (below 2 GiB each)
  const uint16_t *blk;      // the block's q | k | v rows
  int QKVW, QH, KVH, g;     // their row width; heads; the kv group
  int c, T, t0, crow;       // context length, key count, first key; this lane's cache row
};
// 16 bytes (part) of key t's k or v. MODE 0: context keys only (from the paged cache, written
// before the launch); MODE 2: the block's own keys only (this launch's q | k | v rows); MODE 1:
// both kinds in the tile (at most one tile a split): both loads are made into separate registers
// and the choice is taken when the tile is written to LDS. Keys past the end read key T - 1
// (finite values; their scores are masked, so they add nothing). A loaded value is used only at
// the LDS write, after every load of the batch has been issued.
template <int MODE>
__device__ __forceinline__ void key16(const Ws &ws, const KeySrc &ks, int t, int part, bool is_v, uint4 &vctx,
                                      uint4 &vblk) {
  const int tt = min(t, ks.T - 1);
  if (MODE != 2) {
    const int cr = __shfl(ks.crow, max(min(tt, ks.c - 1) - ks.t0, 0), 64);  // (whole wave)
    const u32x4_t t4 = __builtin_amdgcn_raw_buffer_load_b128(is_v ? ks.vc : ks.kc, ((cr * ks.KVH + ks.g) * kD + part * 8) * 2, 0, 0);
    vctx = make_uint4(t4.x, t4.y, t4.z, t4.w);
  }
  if (MODE != 0)
    vblk = wld128(ws, ks.blk + (size_t)max(tt - ks.c, 0) * ks.QKVW + (ks.QH + (is_v ? ks.KVH : 0) + ks.g) * kD + part * 8);
}
template <int MODE>
__device__ __forceinline__ uint4 key_pick(const KeySrc &ks, int t, const uint4 &vctx, const uint4 &vblk) {
  return MODE == 0 ? vctx : MODE == 2 ? vblk : min(t, ks.T - 1) < ks.c ? vctx : vblk;
}
// The tile's 64 keys row-major into kls and V transposed into vts; NB 16-byte loads of K (NB / 2
// key pairs of V) per lane and round trip.
template <int MODE, int NB>
__device__ __forceinline__ void stage_keys(const Ws &ws, const KeySrc &ks, uint16_t *kls, uint16_t *vts, int lane) {
  constexpr int NK = MODE == 1 ? 2 : 1;  // registers per item
  // K: 64 keys x 16 parts of 8
  for (int u0 = 0; u0 < 16; u0 += NB) {
    uint4 k[NB][NK];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int it = (u0 + u) * 64 + lane;
      key16<MODE>(ws, ks, ks.t0 + (it >> 4), it & 15, false, k[u][0], k[u][NK - 1]);
    }
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int it = (u0 + u) * 64 + lane;
      *reinterpret_cast<uint4 *>(kls + (it >> 4) * kKs + (it & 15) * 8) =
          key_pick<MODE>(ks, ks.t0 + (it >> 4), k[u][0], k[u][NK - 1]);
    }
  }
  // V^T: items of two consecutive keys x one part; the pair of each d goes out as one 4-byte write
  for (int u0 = 0; u0 < 8; u0 += NB / 2) {
    uint4 v[NB / 2][2][NK];
#pragma unroll
    for (int u = 0; u < NB / 2; ++u) {
      const int it = (u0 + u) * 64 + lane, kp = it >> 4, part = it & 15;
#pragma unroll
      for (int h = 0; h < 2; ++h) key16<MODE>(ws, ks, ks.t0 + 2 * kp + h, part, true, v[u][h][0], v[u][h][NK - 1]);
    }
#pragma unroll
    for (int u = 0; u < NB / 2; ++u) {
      const int it = (u0 + u) * 64 + lane, kp = it >> 4, part = it & 15;
      const uint4 x0 = key_pick<MODE>(ks, ks.t0 + 2 * kp, v[u][0][0], v[u][0][NK - 1]);
      const uint4 x1 = key_pick<MODE>(ks, ks.t0 + 2 * kp + 1, v[u][1][0], v[u][1][NK - 1]);
      uint16_t v0[8], v1[8];
      __builtin_memcpy(v0, &x0, 16);
      __builtin_memcpy(v1, &x1, 16);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<uint32_t *>(vts + (part * 8 + e) * kVs + 2 * kp) = uint32_t(v0[e]) | (uint32_t(v1[e]) << 16);
    }
  }
}

// q of the kv group, the tile's 64 keys (context keys from the paged cache, then the block's own
// keys, zeros past the end) row-major, and V transposed.
__device__ __forceinline__ void stage_attn(const PlkArgs &a, const Ws &ws, const Sync &sy, const Job &j, unsigned char *slot,
                                           int c, const Abort &abort_w) {
  const int lane = threadIdx.x & 63;
  KeySrc ks;
  const int cbytes = a.num_pages * a.P * a.KVH * kD * 2;
  ks.kc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(a.lw[j.l].kc), (short)0, cbytes, 0x00020000);
  ks.vc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(a.lw[j.l].vc), (short)0, cbytes, 0x00020000);
  ks.blk = qkv_of(a, j.l);
  ks.QKVW = (a.QH + 2 * a.KVH) * kD, ks.QH = a.QH, ks.KVH = a.KVH, ks.g = j.g;
  ks.c = c, ks.T = c + a.bs, ks.t0 = j.tile * 64;
  // the cache row of key t0 + lane (context keys; the block's own keys need no page), looked up
  // before the waits
  const int tl = min(ks.t0 + lane, ks.T - 1);
  ks.crow = tl < c ? min(max(a.block_table[min(tl / a.P, a.maxb - 1)], 0), a.num_pages - 1) * a.P + tl % a.P : 0;
  // the kv group's q heads, its k head and its v head
  wave_wait(sy.flag(j.l, 0, j.g * a.G), 1, a.G, 1u, abort_w);
  wave_wait(sy.flag(j.l, 0, a.QH + j.g), a.KVH, 2, 1u, abort_w);
  uint16_t *qs = reinterpret_cast<uint16_t *>(slot);
  uint16_t *kls = qs + 64 * kQs;
  uint16_t *vts = kls + 64 * kKs;
  const int R = a.bs * a.G;
  // q rows r = hh * bs + jj: 64 rows x 16 parts of 8, issued with the first keys
  uint4 q[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int it = u * 64 + lane, r = it >> 4, part = it & 15;
    const int rq = min(r, R - 1), hh = rq / a.bs, jj = rq % a.bs;
    q[u] = wld128(ws, ks.blk + (size_t)jj * ks.QKVW + (j.g * a.G + hh) * kD + part * 8);
  }
  const int mode = ks.t0 + 64 <= c ? 0 : ks.t0 >= c ? 2 : 1;
  if (mode == 0) stage_keys<0, 16>(ws, ks, kls, vts, lane);
  else if (mode == 2) stage_keys<2, 16>(ws, ks, kls, vts, lane);
  else stage_keys<1, 8>(ws, ks, kls, vts, lane);
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int it = u * 64 + lane, r = it >> 4, part = it & 15;
    *reinterpret_cast<uint4 *>(qs + r * kQs + part * 8) = r < R ? q[u] : make_uint4(0, 0, 0, 0);
  }
}

// Merge of the ns split partials of q head j.head, rows [rm * j.t, rm * j.t + rm) of the block
// (log-sum-exp, splits in order), into the layer's attention output; then the row group's flag.
// Lanes 0-31 take one row, lanes 32-63 the next, four columns per lane.
__device__ __forceinline__ void merge_stage(const PlkArgs &a, const Ws &ws, const Sync &sy, const Job &j,
                                            const Abort &abort_w) {
  const int lane = threadIdx.x & 63;
  wave_wait(sy.actr(j.l, j.g), 1, 1, (unsigned)a.ns, abort_w);
  const int hh = j.head % a.G, d4 = lane & 31;
  const int r_end = min(a.bs, (j.t + 1) * a.rm);
  float *dst = a.o + (size_t)j.l * 16 * a.QH * kD + j.head * kD + d4 * 4;
  for (int r0 = j.t * a.rm; r0 < r_end; r0 += 2) {
    const int row = r0 + (lane >> 5);
    const size_t base = (size_t)j.g * a.ns * 64 + hh * a.bs + min(row, r_end - 1);
    float M = -INFINITY, Ls = 0.f, o[4] = {0.f, 0.f, 0.f, 0.f};
    for (int q0 = 0; q0 < a.ns; q0 += 16) {
      float mq[16], lq[16];
      uint4 v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const size_t rq = base + (size_t)min(q0 + u, a.ns - 1) * 64;
        mq[u] = wldf(ws, a.apm + rq);
        lq[u] = wldf(ws, a.apl + rq);
        v[u] = wld128(ws, a.apo + rq * kD + d4 * 4);
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const float mn = fmaxf(M, mq[u]);
        if (q0 + u >= a.ns || mn == -INFINITY) continue;  // past the splits, or no key yet
        const float sa = exp2f(M - mn), sb = exp2f(mq[u] - mn);
        Ls = Ls * sa + lq[u] * sb;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = o[e] * sa + sb * __uint_as_float(e == 0 ? v[u].x : e == 1 ? v[u].y : e == 2 ? v[u].z : v[u].w);
        M = mn;
      }
    }
    if (row < r_end) {
      const float inv = 1.f / Ls;
      wst128(ws, dst + (size_t)row * a.QH * kD,
             make_uint4(__float_as_uint(o[0] * inv), __float_as_uint(o[1] * inv), __float_as_uint(o[2] * inv),
                        __float_as_uint(o[3] * inv)));
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  if (lane == 0) stcu(sy.mflag(j.l, j.head * a.nrp + j.t), 1u);
}

// =============================================================================================
// Finisher wave
// =============================================================================================
// A flushed tile out[nacc][16][128] (the work-group's partial): with other contributors, store
// it and count it; the last contributor sums every partial and runs the epilogue (q/k RMSNorm +
// RoPE; residual add with the rows' per-tile sums of squares; SwiGLU), then raises the flag.
// The RMSNorm row scale of a normalised input was applied by the staging.
__device__ __forceinline__ void finish_gemm(const PlkArgs &a, const Ws &ws, const Sync &sy, const Job &j, float *out, int w,
                                            int c) {
  const int lane = threadIdx.x & 63;
  const PlkGemm &g = a.g[j.ph];
  const int nacc = j.ph == 2 ? 2 : 1;
  const int first = gemm_owner(g, j.t * g.chunks), lastw = gemm_owner(g, j.t * g.chunks + g.chunks - 1);
  const int count = lastw - first + 1;
  const int bs = a.bs;
  if (count > 1) {
    float *part = a.gpart[j.ph] + (size_t)j.t * g.slots * nacc * 16 * kTN;
    float *mine = part + (size_t)(w - first) * nacc * 16 * kTN;
    for (int i = lane; i < nacc * 16 * kTN / 4; i += 64)
      wst128(ws, mine + i * 4, *reinterpret_cast<const uint4 *>(out + i * 4));
    __builtin_amdgcn_s_waitcnt(0);
    unsigned old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(sy.ctr(j.l, j.ph, j.t), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __shfl(old, 0, 64);
    if (old != (unsigned)(count - 1)) return;  // another contributor finishes this tile
  }
  // Epilogue layout: lane = 4 m + qq handles row m (rows past the block idle). Inputs that do not
  // depend on the sum are loaded before it: the residual row's 32 columns qq * 32 + [0, 32) (O,
  // down), or the RoPE cos | sin of the row's position at rotary indices qq * 16 + [0, 16) (QKV).
  const int m = lane >> 2, qq = lane & 3;
  const bool row_ok = m < bs;
  const int k_in = j.ph == 1 ? 2 * j.l : 2 * j.l + 1;
  uint4 pre[8];
  if (j.ph == 1 || j.ph == 3) {
    const float *xp = xver(a, k_in) + (size_t)min(m, bs - 1) * a.H + j.t * kTN + qq * 32;
#pragma unroll
    for (int e = 0; e < 8; ++e) pre[e] = wld128(ws, xp + 4 * e);
  } else if (j.ph == 0) {
    const size_t pos = (size_t)min(c + min(m, bs - 1), a.rope_max_pos - 1) * (kD / 2) + qq * 16;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pre[e] = *reinterpret_cast<const uint4 *>(a.rope_cos + pos + 4 * e);
      pre[4 + e] = *reinterpret_cast<const uint4 *>(a.rope_sin + pos + 4 * e);
    }
  }
  if (count > 1) {
    const float *part = a.gpart[j.ph] + (size_t)j.t * g.slots * nacc * 16 * kTN;
    if (nacc == 1) reduce_partials<1>(ws, part, count, out, lane);
    else reduce_partials<2>(ws, part, count, out, lane);
  }
  auto u4f = [](const uint4 &v, int i) { return __uint_as_float(i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w); };
  // ---- epilogues on the reduced tile out[nacc][16][128]
  if (j.ph == 0) {
    // q | k | v head t: q/k RMSNorm + RoPE (pairs i, i + 64), rounding to bf16
    const int h = j.t;
    const bool qk = h < a.QH + a.KVH;
    const float *row = out + m * kTN + qq * 16;
    float x1[16], x2[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x1[i] = row[i], x2[i] = row[64 + i];
    if (qk) {
      const uint16_t *nw = (h < a.QH ? a.lw[j.l].q_norm : a.lw[j.l].k_norm) + qq * 16;
      uint16_t w1[16], w2[16];
      const uint4 n0 = *reinterpret_cast<const uint4 *>(nw), n1 = *reinterpret_cast<const uint4 *>(nw + 8);
      const uint4 n2 = *reinterpret_cast<const uint4 *>(nw + 64), n3 = *reinterpret_cast<const uint4 *>(nw + 72);
      __builtin_memcpy(w1, &n0, 16), __builtin_memcpy(w1 + 8, &n1, 16);
      __builtin_memcpy(w2, &n2, 16), __builtin_memcpy(w2 + 8, &n3, 16);
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) ss += x1[i] * x1[i] + x2[i] * x2[i];
      ss += __shfl_xor(ss, 1, 64);
      ss += __shfl_xor(ss, 2, 64);
      const float inv = rsqrtf(ss / (float)kD + a.eps);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = x1[i] * inv * bf16_to_f32(w1[i]), q = x2[i] * inv * bf16_to_f32(w2[i]);
        const float cs = u4f(pre[i >> 2], i & 3), sn = u4f(pre[4 + (i >> 2)], i & 3);
        x1[i] = p * cs - q * sn;
        x2[i] = q * cs + p * sn;
      }
    }
    if (row_ok) {
      uint16_t b1[16], b2[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) b1[i] = f32_to_bf16(x1[i]), b2[i] = f32_to_bf16(x2[i]);
      uint16_t *dst = qkv_of(a, j.l) + (size_t)m * (a.QH + 2 * a.KVH) * kD + h * kD + qq * 16;
      uint4 t[4];
      __builtin_memcpy(t, b1, 32);
      __builtin_memcpy(t + 2, b2, 32);
      wst128(ws, dst, t[0]);
      wst128(ws, dst + 8, t[1]);
      wst128(ws, dst + 64, t[2]);
      wst128(ws, dst + 72, t[3]);
    }
  } else if (j.ph == 1 || j.ph == 3) {
    // residual add into the next x version, with its per-tile row sums of squares
    float *xn = xver(a, k_in + 1) + (size_t)m * a.H + j.t * kTN + qq * 32;
    const float *row = out + m * kTN + qq * 32;
    float ss = 0.f;
    uint4 r[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[i] = u4f(pre[e], i) + row[4 * e + i];
        ss += v[i] * v[i];
      }
      r[e] = make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3]));
    }
    ss += __shfl_xor(ss, 1, 64);
    ss += __shfl_xor(ss, 2, 64);
    if (row_ok) {
#pragma unroll
      for (int e = 0; e < 8; ++e) wst128(ws, xn + 4 * e, r[e]);
      // the final rows' sums of squares are read by the LM head with row stride bs
      if (qq == 0) wstf(ws, ssver(a, k_in + 1) + j.t * (k_in + 1 == 2 * a.L ? bs : 16) + m, ss);
    }
  } else {
    // SwiGLU of the (row-scaled) gate and up tiles
    const float *gr = out + m * kTN + qq * 32, *ur = out + (16 + m) * kTN + qq * 32;
    float *dst = a.act + (size_t)j.l * 16 * a.I + (size_t)m * a.I + j.t * kTN + qq * 32;
    if (row_ok) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float r[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float gt = gr[4 * e + i], up = ur[4 * e + i];
          r[i] = gt / (1.f + expf(-gt)) * up;
        }
        wst128(ws, dst + 4 * e, make_uint4(__float_as_uint(r[0]), __float_as_uint(r[1]), __float_as_uint(r[2]),
                                         __float_as_uint(r[3])));
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  if (lane == 0) stcu(sy.flag(j.l, j.ph, j.t), 1u);
}

// =============================================================================================
__global__ __launch_bounds__(kThreads, 1) void plk_kernel(PlkArgs args) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int s_nj, s_g0, s_ngj, s_ctx;
  // hand-offs between the waves: GEMM jobs consumed (one count per compute wave), the job
  // number + 1 staged in each activation slot, attention tiles staged / computed, output slots
  // written (one count per compute wave) / finished; the work-group's abort word
  __shared__ int s_released, s_ready[kNA], s_attn_ready, s_attn_done, s_out_cnt, s_out_done, s_abort;
  const PlkArgs &a = args;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, w = blockIdx.x;
  const Sync sy(a);
  const Abort ab{sy.abort_word(a.L), &s_abort};
  const Ws wsr{__builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.ws), (short)0, (int)a.ws_bytes, 0x00020000),
               static_cast<const char *>(a.ws)};
  auto aslot = [&](int gb) { return smem + (gb % kNA) * kAslot; };
  auto oslot = [&](int fb) { return reinterpret_cast<float *>(smem + kNA * kAslot + (fb & 1) * kOslot); };
  JobD *jobs = reinterpret_cast<JobD *>(smem + kLds);

  // ---- the job list: every layer has the same stage counts, so job q is (q / J, stage, index)
  {
    int n[6], pre[6], J = 0;
    // GEMM jobs and GEMM flushes of the stages before each stage, and per layer
    int preG[6], preF[6], nG = 0, nF = 0;
#pragma unroll
    for (int st = 0; st < 6; ++st) {
      n[st] = stage_count(a, w, st), pre[st] = J, J += n[st];
      preG[st] = nG, preF[st] = nF;
      if (st != kSAttn && st != kSMerge && n[st] > 0) {
        const PlkGemm &g = a.g[ph_of(st)];
        const int u0 = gemm_u0(g, w);
        nG += n[st];
        nF += (u0 + n[st] - 1) / g.chunks - u0 / g.chunks + 1;
      }
    }
    const int nA = n[kSAttn];
    const int nj = min(a.L * J, kMaxJobs);
    // list index of a cursor
    auto index_of = [&](Cur c) { return c.l >= a.L ? -1 : c.l * J + pre[c.st] + c.i; };
    if (threadIdx.x == 0) {
      s_nj = nj;
      s_ngj = a.L * nG;  // the plan keeps every job of the list within kMaxJobs
      s_ctx = min(max(a.seq_lens[0], 0), a.max_ctx);  // context length of the sequence
      Cur c0 = cur_first(a, w);
      if (c0.l < a.L && (c0.st == kSAttn || c0.st == kSMerge)) c0 = cur_next_gemm(a, w, c0);
      const int g0 = index_of(c0);
      s_g0 = g0 < nj ? g0 : -1;
      s_released = s_attn_ready = s_attn_done = s_out_cnt = s_out_done = s_abort = 0;
    }
    if (threadIdx.x < kNA) s_ready[threadIdx.x] = 0;
    for (int q = threadIdx.x; q < nj; q += kThreads) {
      Cur c{q / J, 0, q % J};
#pragma unroll
      for (int st = 0; st < 5; ++st)
        if (c.st == st && c.i >= n[st]) c.i -= n[st], c.st = st + 1;
      const Job jb = cur_job(a, w, c);
      JobD d{};
      d.kind = jb.kind, d.ph = jb.ph, d.l = jb.l, d.t = jb.t, d.kc = jb.kc, d.g = jb.g, d.s = jb.s;
      d.tile = jb.tile, d.head = jb.head, d.flush = jb.flush, d.last = jb.last, d.first = jb.first;
      const int nx = index_of(cur_next_gemm(a, w, c));  // the next GEMM job (itself when none)
      d.ng = nx >= 0 && nx < nj ? nx : q;
      const bool gemm = jb.kind == 1;
      d.gb = c.l * nG + preG[c.st] + (gemm ? c.i : 0);
      d.ab = c.l * nA + (c.st == kSAttn ? c.i : c.st > kSAttn ? nA : 0);
      d.fb = c.l * nF + preF[c.st];
      if (gemm) {
        const PlkGemm &g = a.g[jb.ph];
        const int u0 = gemm_u0(g, w);
        d.fb += (u0 + c.i) / g.chunks - u0 / g.chunks;
        const GemmSrc gs = gemm_src(a, jb.l, jb.ph, jb.t);
        d.K = gs.K;
        d.kr = g.kr;
        d.w0 = gs.w0;
        d.w1 = gs.w1;
      }
      jobs[q] = d;
    }
    __syncthreads();
  }
  const int NJ = s_nj;

  if (wave < 4) {
    // ---- compute waves: the GEMM jobs in order
    WBuf wb0, wb1;
    f32x4_t acc[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) acc[m][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    int k = s_g0;
    // GEMM job k with its weights in `buf`, which then takes the weights of the GEMM job after
    // the next one: the next job's weights are in flight meanwhile in the other buffer, and both
    // buffers stay live across the loop (a register of a buffer is never reused for anything
    // else, which would make the wave wait for the loads in flight).
    auto gemm_job = [&](WBuf &buf) {
      const JobD d = jobs[k];
      lds_wait(&s_ready[d.gb % kNA], d.gb + 1, ab);
      mma_job(d.ph == 2, kArow, buf, aslot(d.gb), acc, lane);
      lds_add(&s_released, 1);
      // (job indices made wave-uniform, so the loop's branches are scalar ones)
      const int k1 = __builtin_amdgcn_readfirstlane(d.ng);
      issue_w(jobs[__builtin_amdgcn_readfirstlane(jobs[k1].ng)], buf, wave, lane);
      if (d.flush) {
        lds_wait(&s_out_done, d.fb - 1, ab);  // the slot's previous tile is finished
        float *out = oslot(d.fb) + wave * 32 + (lane & 15);
        const bool dual = d.ph == 2;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = (lane >> 4) * 4 + i;
            out[r * kTN + ct * 16] = dual ? acc[0][ct][i] : acc[0][ct][i] + acc[1][ct][i];
            if (dual) out[(16 + r) * kTN + ct * 16] = acc[1][ct][i];
          }
          acc[0][ct] = acc[1][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        lds_add(&s_out_cnt, 1);
      }
      k = k1;
    };
    // A counted loop over pairs with the odd job after it: the loop is entered and left only
    // after wb1's job, so the wait counts at every MFMA see the loads in issue order.
    const int ngj = __builtin_amdgcn_readfirstlane(s_ngj);
    if (k >= 0 && ngj > 0) {
      issue_w(jobs[k], wb0, wave, lane);
      __builtin_amdgcn_sched_barrier(0);  // wb0's loads strictly before wb1's, as in the loop
      issue_w(jobs[jobs[k].ng], wb1, wave, lane);
      for (int i = 0; i + 1 < ngj; i += 2) {
        gemm_job(wb0);
        gemm_job(wb1);
      }
      if (ngj & 1) gemm_job(wb0);
    }
    __builtin_amdgcn_s_waitcnt(0);  // the re-issued weight loads past the last job
  } else if (wave < 4 + kStagers) {
    // ---- stager waves: job k goes to stager k % kStagers; a GEMM job waits for its activation
    //      slot (the job kNA GEMM jobs earlier consumed) and for the attention tiles before it,
    //      which use the slots' memory; an attention tile waits for every job before it
    for (int k = wave - 4; k < NJ; k += kStagers) {
      const JobD d = jobs[k];
      const Job j = job_of(d);
      if (d.kind == 1) {
        lds_wait(&s_released, 4 * (d.gb - kNA + 1), ab);
        lds_wait(&s_attn_done, d.ab, ab);
        stage_gemm(a, wsr, sy, j, aslot(d.gb), ab);
        lds_set(&s_ready[d.gb % kNA], d.gb + 1);
      } else if (d.kind == 2) {
        lds_wait(&s_released, 4 * d.gb, ab);
        lds_wait(&s_attn_done, d.ab, ab);
        stage_attn(a, wsr, sy, j, smem, s_ctx, ab);
        lds_set(&s_attn_ready, d.ab + 1);
      } else if (d.kind == 3) {
        merge_stage(a, wsr, sy, j, ab);
      }
    }
  } else {
    // ---- finisher wave: the GEMM flushes and attention tiles in order; an attention tile
    //      runs every query row (four 16-row tiles in turn) and the split's last tile stores and
    //      counts the split's partial
    for (int k = 0; k < NJ; ++k) {
      const JobD d = jobs[k];
      if (d.kind == 2) {
        // the split's tiles are consecutive jobs, the last one flushes: run them all here, with
        // the state initialised here, so that it is live only in this block
        AttnState ast[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
          for (int i = 0; i < kD / 16; ++i) ast[rt].o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          ast[rt].m = -INFINITY;
          ast[rt].l = 0.f;
        }
        int kk = k;
        bool more = true;
        do {
          const JobD da = jobs[kk];
          lds_wait(&s_attn_ready, da.ab + 1, ab);
          const Job j = job_of(da);
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) attn_tile(a, j, smem, ast[rt], s_ctx, rt, lane);
          lds_add(&s_attn_done, 1);
          more = !j.flush;
          if (more) ++kk;
        } while (more);
        {
          const Job j = job_of(jobs[kk]);
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) attn_store(a, wsr, j, ast[rt], rt, lane);
          __builtin_amdgcn_s_waitcnt(0);
          if (lane == 0) __hip_atomic_fetch_add(sy.actr(j.l, j.g), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        k = kk;
      } else if (d.kind == 1 && d.flush) {
        lds_wait(&s_out_cnt, 4 * (d.fb + 1), ab);
        finish_gemm(a, wsr, sy, job_of(d), oslot(d.fb), w, s_ctx);
        lds_set(&s_out_done, d.fb + 1);
      }
    }
  }
}

}  // namespace

// ---------------------------------------------------------------------------------------------
namespace {
int plk_cus() {
  static const int n = [] {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      return 0;
    return cus;
  }();
  return n;
}

PlkGemm gemm_of(int tiles, int K, int kr, int nwg) {
  PlkGemm g{};
  g.tiles = tiles;
  g.kr = kr;
  g.chunks = K / kr;
  const int units = tiles * g.chunks;
  g.base = units / nwg;
  g.rem = units % nwg;
  // work-groups sharing one tile: a tile of `chunks` units meets at most chunks / base + 2 ranges
  g.slots = g.base > 0 ? std::min(g.chunks, g.chunks / g.base + 2) : std::min(g.chunks, nwg);
  return g;
}
}  // namespace

PlkPlan plk_plan(int L, int H, int QH, int KVH, int D, int I, int bs, int batch, int max_ctx, bool bf16) {
  PlkPlan p{};
  const int nwg = plk_cus();
  const int G = KVH > 0 ? QH / KVH : 0;
  if (!bf16 || batch != 1 || bs > 16 || D != kD || L < 1 || L > kPlkMaxLayers || nwg < 64 || H % kTN ||
      I % kTN || H % 128 || I % 128 || bs * G > 64 || KVH < 1 || QH > nwg || H > 16384)
    return p;
  const int ntile = (max_ctx + bs + 63) / 64;
  int ns = std::min(ntile, std::max(1, nwg / KVH));
  if (KVH * ns > nwg) return p;
  // one weight matrix per job: 256-column chunks (eight 32-column steps, like gate|up's two
  // 128-column chunks)
  if (H % 256 || (QH * D) % 256 || I % 256) return p;
  auto kr1 = [](int) { return 256; };
  p.nwg = nwg;
  p.ntile = ntile;
  p.ns = ns;
  p.g[0] = gemm_of(QH + 2 * KVH, H, kr1(H), nwg);
  p.g[1] = gemm_of(H / kTN, QH * kD, kr1(QH * kD), nwg);
  p.g[2] = gemm_of(I / kTN, H, 128, nwg);  // gate and up: two matrices per job
  p.g[3] = gemm_of(H / kTN, I, kr1(I), nwg);
  // merge jobs: the fewest rows per job that give every (q head, row group) its own work-group
  p.rm = 1;
  while (QH * ((bs + p.rm - 1) / p.rm) > nwg) ++p.rm;
  p.nrp = (bs + p.rm - 1) / p.rm;
  // jobs of one work-group: at most base + 1 units of each projection, the tiles of one
  // attention split and one merge, per layer
  int jobs = (ntile + ns - 1) / ns + 1;
  for (int i = 0; i < 4; ++i) jobs += p.g[i].base + 1;
  if (L * jobs > kMaxJobs) return p;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = (off + bytes + 255) / 256 * 256;
    return o;
  };
  p.off_xs = take((size_t)(2 * L - 1) * 16 * H * 4);
  p.off_sss = take((size_t)(2 * L - 1) * (H / kTN) * 16 * 4);
  p.off_qkv = take((size_t)L * 16 * (QH + 2 * KVH) * kD * 2);
  p.off_o = take((size_t)L * 16 * QH * kD * 4);
  p.off_act = take((size_t)L * 16 * I * 4);
  p.off_apo = take((size_t)KVH * ns * 64 * kD * 4);
  p.off_apm = take((size_t)KVH * ns * 64 * 4);
  p.off_apl = take((size_t)KVH * ns * 64 * 4);
  for (int i = 0; i < 4; ++i)
    p.off_gpart[i] = take((size_t)p.g[i].tiles * p.g[i].slots * (i == 2 ? 2 : 1) * 16 * kTN * 4);
  p.bytes = off;
  int per_layer = 0;
  for (int i = 0; i < 4; ++i) per_layer += 2 * p.g[i].tiles;
  per_layer += KVH + QH * p.nrp;
  p.sync_words = L * per_layer + 1;
  p.ok = 1;
  return p;
}

hipError_t launch_plk(const PlkArgs &a, hipStream_t s) {
  constexpr size_t lds = kLds + kMaxJobs * sizeof(JobD);
  static_assert(lds + 128 <= 160 * 1024, "LDS of one CU");
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void *>(plk_kernel), hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  static const int resident = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, plk_kernel, kThreads, lds) != hipSuccess) return 0;
    return n;
  }();
  // every work-group waits for others: the whole grid must be resident at once
  if (resident < 1 || a.nwg != plk_cus() || a.nwg < 1) return hipErrorInvalidValue;
  ProfScope prof("plk", s);
  plk_kernel<<<a.nwg, kThreads, lds, s>>>(a);
  return hipGetLastError();
}

}  // namespace dflash
