// Non-causal paged block attention of the DFlash drafter.
//
// Every query of a sequence's block sees the sequence's c_b context keys (from the paged
// cache) plus all bs block keys, with no mask. Work-group = (sequence b, kv head g, split s):
// its bs*G query rows (the G q-heads sharing kv head g, times the bs block positions) share
// every K/V tile it loads, so each KV byte is read from HBM once per work-group. The key
// range c_b + bs is cut into splits of `chunk` keys so that one long context (32k) still
// spreads over the whole chip, and so that many contexts of unequal length give even
// work-groups. A second kernel merges the split partials (unnormalised output, running max,
// running sum) with the usual log-sum-exp rescaling; a sequence with one split normalises in
// place.
//
// MFMA layout. Scores are computed transposed, S^T = K Q^T (A = K tile rows, B = Q rows), so
// each lane ends up holding 4 keys of one query row. The output is computed as O^T = V^T P^T,
// where P^T is the B operand. The key order inside each MFMA is permuted so that the 4+4
// keys a lane holds after two score tiles are exactly the 8 consecutive keys the P^T operand
// needs: P never leaves registers. V is staged transposed in LDS so V^T fragments are
// 16-byte LDS reads. P is fed to the bf16 MFMA as a hi/lo pair (p = hi + lo, both bf16),
// which keeps the probabilities at ~16 bits of precision.
#include <float.h>

#include "common.h"
#include "kernels.h"

namespace dflash {
namespace {

constexpr int kTileKeys = 64;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kMaxChunk = 16 * kTileKeys;  // keys per split at most (attn_plan)

template <typename T, int D>
__global__ __launch_bounds__(256, 2) void attn_partial_kernel(AttnArgs a) {
  constexpr int KPV = Storage<T>::kPerVec;
  constexpr int CH = 4 * KPV;                // contraction elements per MFMA step
  constexpr int NB = KPV / 4;                // score tiles per P.V step
  constexpr int KSTR = D + KPV;              // K row stride in LDS (16-byte pad)
  constexpr int VSTR = kTileKeys + KPV;      // V^T row stride in LDS
  constexpr int CPR = D / KPV;               // 16-byte vectors per key row
  __shared__ __attribute__((aligned(16))) T ks[kTileKeys * KSTR];
  __shared__ __attribute__((aligned(16))) T vts[D * VSTR];
  __shared__ int pgs[kMaxChunk + 1];  // page-table entries of the split's key range

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  if (a.items) {  // the blockIdx.x-th work-group that has keys (a 1-D grid)
    if ((int)blockIdx.x >= *a.n_items) return;
    const int f = a.items[blockIdx.x];
    split = f % a.nsplit, g = (f / a.nsplit) % a.KVH, b = f / (a.nsplit * a.KVH);
  }
  const int G = a.QH / a.KVH;
  const int R = a.bs * G;
  const int kbeg = split * a.chunk;
  const int32_t *bt = a.block_table + (size_t)b * a.maxb;
  // The context length, the query fragment and the page-table entries of the split's key
  // range are loaded together (one round trip): the page entries cover keys [kbeg, kbeg +
  // chunk) whatever the length, clamped into the table, and go to LDS, so that the K/V loads
  // of later tiles read them there instead of waiting behind the loads in flight.
  const int pbeg = kbeg / a.P, npg = (a.chunk - 1) / a.P + 2;
  const int c = min(max(a.seq_lens[b], 0), a.max_ctx);
  const int r = wave * 16 + (lane & 15);  // query row hh*bs + j of this wave's 16-row tile
  const bool rvalid = r < R && wave * 16 < R;
  Vec16 qf[D / CH];  // the B operand of S^T
  {
    const int hh = r / a.bs, j = r % a.bs;
    const T *qp = reinterpret_cast<const T *>(a.q) +
                  ((size_t)(b * a.bs + j) * a.QH + g * G + hh) * D + (lane >> 4) * KPV;
#pragma unroll
    for (int dc = 0; dc < D / CH; ++dc) qf[dc] = rvalid ? load_vec16(qp + dc * CH) : zero_vec16();
  }
  for (int i = threadIdx.x; i < npg; i += 256) pgs[i] = bt[min(pbeg + i, a.maxb - 1)];
  __syncthreads();
  const int T_total = c + a.bs;
  if (kbeg >= T_total) return;  // nothing for this split (uniform over the work-group)
  const int kend = min(T_total, kbeg + a.chunk);

  f32x4_t acc_o[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) acc_o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float scale = 1.4426950408889634f / sqrtf((float)D);  // log2(e)/sqrt(D)

  const T *kc = reinterpret_cast<const T *>(a.kc);
  const T *vc = reinterpret_cast<const T *>(a.vc);
  const T *kbk = reinterpret_cast<const T *>(a.kb);
  const T *vbk = reinterpret_cast<const T *>(a.vb);

  // Staging of a 64-key tile. K: item v = (key v / CPR, 16-byte part v % CPR), one row-major
  // vector write each. V is stored transposed (vts[d][key]) by items of two consecutive keys
  // (2 kappa, 2 kappa + 1) and one part: the pair of values of each d goes out as one 4-byte
  // (bf16) or 8-byte (fp32) write. Within a wave, 16 consecutive kappa x 4 parts write each
  // row, so a write instruction touches at most two rows that share banks.
  constexpr int KVEC = kTileKeys * CPR / 256;  // K items per thread
  constexpr int VVEC = (kTileKeys / 2) * CPR / 256;  // V items per thread
  static_assert(kTileKeys * CPR % 256 == 0 && (kTileKeys / 2) * CPR % 256 == 0, "staging items per thread");
  auto v_kappa = [](int v) { return (v & 15) | (((v >> 6) & 1) << 4); };
  auto v_part = [](int v) { return ((v >> 4) & 3) | ((v >> 7) << 2); };
  struct TileRegs {
    Vec16 k[KVEC], v[VVEC][2];
  };
  TileRegs ra, rb;  // two tiles' loads in flight: tile n in ra (n even) or rb (n odd)
  // Loads of a tile, two tiles ahead. Each lane first forms the source row of key t0 + lane
  // (one page lookup per lane and tile): r >= 0 is a slot of the context cache, r < 0 the
  // block's own row -1 - r. Every staging item then takes its key's row from the owning lane
  // (a cross-lane read) and forms its address with no division and no branch. Past the last
  // tile the issues read the last tile again (L2 hits); keys past kend in the last tile are
  // block keys, clamped to the block's last row, and are masked in the scores.
  auto issue = [&](TileRegs &rr, int t0, int tlast) {
    int row;
    {
      const int t = min(t0, tlast) + lane;
      const int page = min(max(pgs[t / a.P - pbeg], 0), a.num_pages - 1);
      row = t < c ? page * a.P + t % a.P : -1 - (b * a.bs + min(t - c, a.bs - 1));
    }
    auto src = [&](const T *cache, const T *blk, int kk, int part) -> const T * {
      const int r = __shfl(row, kk, 64);
      const size_t off = ((size_t)(unsigned)(r ^ (r >> 31)) * a.KVH + g) * D + part * KPV;  // row r or -1 - r
      return (r >= 0 ? cache : blk) + off;
    };
#pragma unroll
    for (int i = 0; i < KVEC; ++i) {
      const int v = threadIdx.x + i * 256;
      rr.k[i] = load_vec16(src(kc, kbk, v / CPR, v % CPR));
    }
#pragma unroll
    for (int i = 0; i < VVEC; ++i) {
      const int v = threadIdx.x + i * 256;
#pragma unroll
      for (int h = 0; h < 2; ++h) rr.v[i][h] = load_vec16(src(vc, vbk, 2 * v_kappa(v) + h, v_part(v)));
    }
  };
  // Tile n's loads go out two tiles ahead, while tiles n - 2 and n - 1 compute. The issues are
  // unconditional (past the last tile they read key kend - 1 again, an L2 hit): a conditional
  // one makes the compiler wait for every load in flight where the paths meet.
  const int ntiles = (kend - kbeg + kTileKeys - 1) / kTileKeys, tlast = kbeg + (ntiles - 1) * kTileKeys;
  issue(ra, kbeg, tlast);
  issue(rb, kbeg + kTileKeys, tlast);

  auto tile = [&](TileRegs &rr, int n) {
    const int t0 = kbeg + n * kTileKeys;
    // ---- the tile's registers into LDS: K row-major, V transposed
    __syncthreads();
#pragma unroll
    for (int i = 0; i < KVEC; ++i) {
      const int v = threadIdx.x + i * 256;
      *reinterpret_cast<uint4 *>(&ks[(v / CPR) * KSTR + (v % CPR) * KPV]) = rr.k[i].u;
    }
#pragma unroll
    for (int i = 0; i < VVEC; ++i) {
      const int v = threadIdx.x + i * 256, kap = v_kappa(v), part = v_part(v);
      T v0[KPV], v1[KPV];
      __builtin_memcpy(v0, &rr.v[i][0].u, 16);
      __builtin_memcpy(v1, &rr.v[i][1].u, 16);
#pragma unroll
      for (int e = 0; e < KPV; ++e) {
        T *dst = &vts[(part * KPV + e) * VSTR + 2 * kap];
        if constexpr (sizeof(T) == 2) {
          *reinterpret_cast<uint32_t *>(dst) = uint32_t(v0[e]) | (uint32_t(v1[e]) << 16);
        } else {
          *reinterpret_cast<float2 *>(dst) = make_float2(v0[e], v1[e]);
        }
      }
    }
    __syncthreads();
    // ---- tile n + 2's loads into the registers just written out
    issue(rr, t0 + 2 * kTileKeys, tlast);
    if (wave * 16 >= R) return;

    // ---- S^T tiles: 4 tiles of 16 keys; tile sb row rho holds key
    //      (sb / NB) * CH + KPV * (rho / 4) + 4 * (sb % NB) + rho % 4
    f32x4_t s[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      s[sb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const int rho = lane & 15;
      const int key = (sb / NB) * CH + KPV * (rho / 4) + 4 * (sb % NB) + rho % 4;
#pragma unroll
      for (int dc = 0; dc < D / CH; ++dc) {
        const Vec16 kf = load_vec16(&ks[key * KSTR + dc * CH + (lane >> 4) * KPV]);
        mma16<T>(s[sb], kf, qf[dc]);
      }
    }
    // lane (group gq = lane/16) holds, for its row, keys (sb/NB)*CH + KPV*gq + 4*(sb%NB) + i
    float tmax = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < 4; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = (sb / NB) * CH + KPV * (lane >> 4) + 4 * (sb % NB) + i;
        const float v = (t0 + key < kend) ? s[sb][i] * scale : -INFINITY;
        s[sb][i] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    // m_new is finite (every computed tile has a key below kend), so the raw exponential needs
    // no guard: the first tile's alpha (m_run = -inf) and masked keys' p (-inf) come out 0
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) acc_o[i] *= alpha;
#pragma unroll
    for (int sb = 0; sb < 4; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(s[sb][i] - m_new);
        s[sb][i] = p;
        l_run += p;
      }

    // ---- O^T += V^T P^T, one P.V step per CH keys
#pragma unroll
    for (int ps = 0; ps < 4 / NB; ++ps) {
      if constexpr (KPV == 8) {
        // hi = bf16(p), lo = bf16(p - hi), two values per conversion instruction (RNE)
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = s[ps * 2 + e / 2][(2 * e) % 4], p1 = s[ps * 2 + e / 2][(2 * e + 1) % 4];
          const bf16x2_t h = __builtin_convertvector(f32x2_t{p0, p1}, bf16x2_t);
          __builtin_memcpy(&hi[e], &h, 4);
          const float h0 = __uint_as_float(hi[e] << 16), h1 = __uint_as_float(hi[e] & 0xffff0000u);
          const bf16x2_t l = __builtin_convertvector(f32x2_t{p0 - h0, p1 - h1}, bf16x2_t);
          __builtin_memcpy(&lo[e], &l, 4);
        }
        Vec16 phi, plo;
        __builtin_memcpy(&phi.u, hi, 16);
        __builtin_memcpy(&plo.u, lo, 16);
#pragma unroll
        for (int db = 0; db < D / 16; ++db) {
          const Vec16 vf = load_vec16(&vts[(db * 16 + (lane & 15)) * VSTR + ps * CH + (lane >> 4) * KPV]);
          mma16<T>(acc_o[db], vf, phi);
          mma16<T>(acc_o[db], vf, plo);
        }
      } else {
        float pv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pv[e] = s[ps][e];
        Vec16 pf;
        __builtin_memcpy(&pf.u, pv, 16);
#pragma unroll
        for (int db = 0; db < D / 16; ++db) {
          const Vec16 vf = load_vec16(&vts[(db * 16 + (lane & 15)) * VSTR + ps * CH + (lane >> 4) * KPV]);
          mma16<T>(acc_o[db], vf, pf);
        }
      }
    }
  };
  // a counted loop over pairs of tiles, the odd tile after it (each register set keeps its role)
  for (int n = 0; n + 1 < ntiles; n += 2) {
    tile(ra, n);
    tile(rb, n + 1);
  }
  if (ntiles & 1) tile(ra, ntiles - 1);
  // ---- O^T lane layout: d = db*16 + (lane/16)*4 + i, row r = wave*16 + lane%16
  const bool active = wave * 16 < R;
  if (active) {
    l_run += __shfl_xor(l_run, 16, 64);
    l_run += __shfl_xor(l_run, 32, 64);
  }
  const int G2 = a.QH / a.KVH;
  auto out_row = [&](int row) {  // merged output element index of query row `row` = hh*bs + j
    return ((size_t)(b * a.bs + row % a.bs) * a.QH + g * G2 + row / a.bs) * D;
  };
  const int ns = (T_total + a.chunk - 1) / a.chunk;  // splits of this sequence
  if (ns == 1) {  // the whole key range: normalise in place
    if (rvalid) {
      const float inv = 1.f / l_run;
      const size_t e0 = out_row(r) + (lane >> 4) * 4;
      if (a.o_planes) {  // 4 consecutive d: packed conversions (round to nearest even), 8-byte stores
        const size_t lo_off = (size_t)a.B * a.bs * a.QH * D;
#pragma unroll
        for (int db = 0; db < D / 16; ++db) {
          const f32x4_t v = acc_o[db] * inv;
          const bf16x2_t h01 = __builtin_convertvector(f32x2_t{v[0], v[1]}, bf16x2_t);
          const bf16x2_t h23 = __builtin_convertvector(f32x2_t{v[2], v[3]}, bf16x2_t);
          const bf16x2_t l01 = __builtin_convertvector(f32x2_t{v[0] - (float)h01[0], v[1] - (float)h01[1]}, bf16x2_t);
          const bf16x2_t l23 = __builtin_convertvector(f32x2_t{v[2] - (float)h23[0], v[3] - (float)h23[1]}, bf16x2_t);
          uint32_t hw[2], lw[2];
          __builtin_memcpy(&hw[0], &h01, 4);
          __builtin_memcpy(&hw[1], &h23, 4);
          __builtin_memcpy(&lw[0], &l01, 4);
          __builtin_memcpy(&lw[1], &l23, 4);
          *reinterpret_cast<uint2 *>(a.o_planes + e0 + db * 16) = make_uint2(hw[0], hw[1]);
          *reinterpret_cast<uint2 *>(a.o_planes + lo_off + e0 + db * 16) = make_uint2(lw[0], lw[1]);
        }
      } else {
#pragma unroll
        for (int db = 0; db < D / 16; ++db) *reinterpret_cast<f32x4_t *>(a.o + e0 + db * 16) = acc_o[db] * inv;
      }
    }
    return;
  }

  // ---- split partials (unnormalised output, running max, running sum), merged by the next
  //      launch
  const size_t base = ((size_t)(b * a.KVH + g) * a.nsplit + split) * 64;
  if (rvalid) {
    float *po = a.po + (base + r) * D + (lane >> 4) * 4;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) *reinterpret_cast<f32x4_t *>(po + db * 16) = acc_o[db];
    if (lane < 16) {
      a.pm[base + r] = m_run;
      a.pl[base + r] = l_run;
    }
  }
}

// Online log-sum-exp accumulation of NU split partials (m, l, o) into a running (m_acc, l_acc,
// o_acc) of four consecutive output elements of one row, in split order: the splits s0, s0 +
// step, ... whose loads (one 16-byte load of o per split) are all issued before any is used, so
// one round trip covers NU splits. The load addresses are clamped to nmax (>= ns) splits; splits
// at or past ns are loaded but never used.
template <int NU>
__device__ __forceinline__ void merge_x4(const float *pm, const float *pl, const float *po, size_t stride_ml,
                                         size_t stride_o, int s0, int step, int ns, int nmax, float &m_acc,
                                         float &l_acc, f32x4_t &o_acc) {
  float mv[NU], lv[NU];
  f32x4_t pv[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int q = min(s0 + u * step, nmax - 1);
    mv[u] = pm[(size_t)q * stride_ml];
    lv[u] = pl[(size_t)q * stride_ml];
    pv[u] = *reinterpret_cast<const f32x4_t *>(po + (size_t)q * stride_o);
  }
  float m_new = m_acc;
#pragma unroll
  for (int u = 0; u < NU; ++u)
    if (s0 + u * step < ns) m_new = fmaxf(m_new, mv[u]);
  // m_acc = -inf at first: r = 0 on empty sums; no split at all so far (a split group of the
  // many-split merge with fewer splits than groups): m_acc = m_new = -inf, and r = 1 keeps the
  // empty sums 0 (exp2f(-inf - -inf) would be NaN and poison the combination)
  const float r = m_acc == m_new ? 1.f : exp2f(m_acc - m_new);
  l_acc *= r;
  o_acc *= r;
#pragma unroll
  for (int u = 0; u < NU; ++u)
    if (s0 + u * step < ns) {
      const float w = exp2f(mv[u] - m_new);
      l_acc += w * lv[u];
      o_acc += w * pv[u];
    }
  m_acc = m_new;
}

// element e.. e + 3 of the merged output: fp32 (one 16-byte store), or its (hi, lo) bf16 planes
// (one 8-byte store each)
__device__ __forceinline__ void store_out4(const AttnArgs &a, size_t e, f32x4_t v) {
  if (a.o_planes) {
    uint16_t h[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[i] = f32_to_bf16(v[i]);
      lo[i] = f32_to_bf16(v[i] - bf16_to_f32(h[i]));
    }
    uint2 hw, lw;
    hw.x = h[0] | (uint32_t(h[1]) << 16), hw.y = h[2] | (uint32_t(h[3]) << 16);
    lw.x = lo[0] | (uint32_t(lo[1]) << 16), lw.y = lo[2] | (uint32_t(lo[3]) << 16);
    *reinterpret_cast<uint2 *>(a.o_planes + e) = hw;
    *reinterpret_cast<uint2 *>(a.o_planes + (size_t)a.B * a.bs * a.QH * a.D + e) = lw;
  } else {
    *reinterpret_cast<f32x4_t *>(a.o + e) = v;
  }
}

// Merge of up to 16 splits per sequence: thread (query row, 4 consecutive d) of a (sequence,
// kv head), 1024 / D rows per work-group, one round trip for all splits (16-byte partial loads,
// 16-byte fp32 or 8 + 8-byte plane stores).
template <typename T>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
  const int D = a.D, tpr = D / 4, rpw = 256 / tpr;
  const int row = blockIdx.x * rpw + (int)threadIdx.x / tpr, d = ((int)threadIdx.x % tpr) * 4;
  const int g = blockIdx.y, b = blockIdx.z;
  const int G = a.QH / a.KVH;
  if (row >= a.bs * G) return;
  const int c = min(max(a.seq_lens[b], 0), a.max_ctx);
  const int ns = (c + a.bs + a.chunk - 1) / a.chunk;
  const size_t base = (size_t)(b * a.KVH + g) * a.nsplit * 64 + row;
  float m = -INFINITY, l = 0.f;
  f32x4_t o = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // One sequence: the first 16 splits' loads go out with the length's (clamped to the
  // workspace's splits). Several: only the sequence's own splits are read.
  const int nmax = a.B == 1 ? a.nsplit : ns;
  int s0 = 0;
  do merge_x4<16>(a.pm + base, a.pl + base, a.po + base * D + d, 64, 64 * (size_t)D, s0, 1, ns, nmax, m, l, o);
  while ((s0 += 16) < ns);
  if (ns == 1) return;  // one split: normalised in place by attn_partial_kernel
  const int hh = row / a.bs, j = row % a.bs;
  store_out4(a, ((size_t)(b * a.bs + j) * a.QH + g * G + hh) * D + d, o / l);
}

// Merge of many splits (more than 16 per sequence: one long context): work-group = one
// (sequence, kv head, query row). Thread (d4, sub) accumulates four consecutive elements over
// the splits s = sub (mod 1024 / D), 8 loads in flight at a time (one round trip up to 64
// splits at D = 128); the sub-accumulators are then combined through LDS in a fixed order.
template <typename T>
__global__ __launch_bounds__(256) void attn_merge_rows_kernel(AttnArgs a) {
  __shared__ float sm[16], sl[16];
  __shared__ f32x4_t so[256];
  const int row = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = a.QH / a.KVH;
  const int D = a.D, tpr = D / 4, nsub = 256 / tpr;  // D = 128: 32 threads a row, 8 subs; 64: 16, 16
  const int t = (int)threadIdx.x % tpr, d = t * 4, sub = (int)threadIdx.x / tpr;
  const int c = min(max(a.seq_lens[b], 0), a.max_ctx);
  const int ns = (c + a.bs + a.chunk - 1) / a.chunk;
  const size_t base = (size_t)(b * a.KVH + g) * a.nsplit * 64 + row;
  float m = -INFINITY, l = 0.f;
  f32x4_t o = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // as in attn_merge_kernel (a sub with no split adds nothing)
  const int nmax = a.B == 1 ? a.nsplit : ns;
  int s0 = sub;
  do merge_x4<8>(a.pm + base, a.pl + base, a.po + base * D + d, 64, 64 * (size_t)D, s0, nsub, ns, nmax, m, l, o);
  while ((s0 += 8 * nsub) < ns);
  if (ns == 1) return;  // one split: normalised in place by attn_partial_kernel (uniform)
  so[threadIdx.x] = o;
  if (t == 0) {
    sm[sub] = m;
    sl[sub] = l;
  }
  __syncthreads();
  if (sub == 0) {
    float mm = -INFINITY;
    for (int q = 0; q < nsub; ++q) mm = fmaxf(mm, sm[q]);
    f32x4_t n = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float dn = 0.f;
    for (int q = 0; q < nsub; ++q) {
      const float w = exp2f(sm[q] - mm);  // a sub with no split: m = -inf, weight 0
      n += w * so[q * tpr + t];
      dn += w * sl[q];
    }
    const int hh = row / a.bs, j = row % a.bs;
    store_out4(a, ((size_t)(b * a.bs + j) * a.QH + g * G + hh) * D + d, n / dn);
  }
}

// The work-groups of the partial kernel that have keys, in (sequence, split, kv head) order:
// one work-group; the sequences' split counts are scanned 256 at a time.
__global__ __launch_bounds__(256) void attn_items_kernel(AttnArgs a, int *items, int *n_items) {
  __shared__ int scan[256];
  __shared__ int carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int b0 = 0; b0 < a.B; b0 += 256) {
    const int b = b0 + (int)threadIdx.x;
    int ns = 0;
    if (b < a.B) {
      const int c = min(max(a.seq_lens[b], 0), a.max_ctx);
      ns = min((c + a.bs + a.chunk - 1) / a.chunk, a.nsplit);
    }
    scan[threadIdx.x] = ns;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {  // inclusive scan
      const int v = threadIdx.x >= (unsigned)o ? scan[threadIdx.x - o] : 0;
      __syncthreads();
      scan[threadIdx.x] += v;
      __syncthreads();
    }
    const int pre = carry + scan[threadIdx.x] - ns;  // splits of the sequences before b
    // (sequence, split, kv head) order: the kv heads of one key range are launched together,
    // and each reads its 256-byte slice of the same 2 KiB cache rows
    for (int sp = 0; sp < ns; ++sp)
      for (int gg = 0; gg < a.KVH; ++gg) items[a.KVH * (pre + sp) + gg] = (b * a.KVH + gg) * a.nsplit + sp;
    __syncthreads();
    if (threadIdx.x == 255) carry += scan[255];
    __syncthreads();
  }
  if (threadIdx.x == 0) *n_items = a.KVH * carry;
}

template <typename T>
hipError_t launch_t(const AttnArgs &a, hipStream_t s) {
  // the partial kernel keeps a split's page-table entries in LDS and pipelines whole tiles
  if (a.chunk < kTileKeys || a.chunk > kMaxChunk || a.chunk % kTileKeys || a.P < 1) return hipErrorInvalidValue;
  dim3 grid = a.items ? dim3(a.nsplit * a.KVH * a.B) : dim3(a.nsplit, a.KVH, a.B);
  {
    ProfScope prof("attn_partial", s);
    if (a.D == 128)
      attn_partial_kernel<T, 128><<<grid, 256, 0, s>>>(a);
    else
      attn_partial_kernel<T, 64><<<grid, 256, 0, s>>>(a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  const int R = a.bs * (a.QH / a.KVH), rpw = 1024 / a.D;  // (attn_merge_kernel's rows per work-group)
  {
    ProfScope prof("attn_merge", s);
    if (a.nsplit > 16)
      attn_merge_rows_kernel<T><<<dim3(R, a.KVH, a.B), 256, 0, s>>>(a);
    else
      attn_merge_kernel<T><<<dim3((R + rpw - 1) / rpw, a.KVH, a.B), 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace

void attn_plan(int B, int KVH, int max_keys, int *chunk, int *nsplit) {
  // Two work-groups fit on a CU. One sequence: at most about 512 work-groups (one round, so no
  // work-group of a long context waits for a slot), in splits of two to sixteen 64-key tiles
  // (at 2048 keys, two-tile splits beat one-tile ones: the second tile costs less than the
  // merge of twice the partials). Several: about 768 (a round and a half), in splits of one to
  // eight tiles: with many sequences of unequal length, short splits keep the work-groups even.
  const long target = B == 1 ? 512 : 768;
  long want = ((long)max_keys * B * KVH + target - 1) / target;
  int ch = (int)((want + kTileKeys - 1) / kTileKeys) * kTileKeys;
  if (ch < (B == 1 ? 2 : 1) * kTileKeys) ch = (B == 1 ? 2 : 1) * kTileKeys;
  if (ch > (B == 1 ? kMaxChunk : kMaxChunk / 2)) ch = B == 1 ? kMaxChunk : kMaxChunk / 2;
  *chunk = ch;
  *nsplit = (max_keys + ch - 1) / ch;
}

hipError_t launch_attention(bool bf16, const AttnArgs &a, hipStream_t s) {
  return bf16 ? launch_t<uint16_t>(a, s) : launch_t<float>(a, s);
}

hipError_t launch_attention_items(const AttnArgs &a, int *items, int *n_items, hipStream_t s) {
  ProfScope prof("attn_items", s);
  attn_items_kernel<<<1, 256, 0, s>>>(a, items, n_items);
  return hipGetLastError();
}

}  // namespace dflash
