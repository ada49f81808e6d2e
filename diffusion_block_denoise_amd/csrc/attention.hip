// Non-causal attention of a row set's queries over every cached position, with grouped K/V heads.
//
// bf16 path (v_mfma_f32_32x32x16_bf16), one wave per tile of 32 query rows of one (batch row,
// K/V head) pair.  Query rows of a pair are (position, head-in-group) combinations, so a group
// of G query heads shares every K/V load.  The wave computes S^T = K Q^T over 32 keys at a time:
// in the MFMA output each lane holds one query and 16 keys, so the row softmax needs a single
// cross-half shuffle.  The probabilities P^T are already laid out as the B operand of the next
// MFMA, O^T += V^T P^T, whose A operand comes from the transposed V cache (bf16: per head,
// 32-key tiles of [hd][32], so a tile is one contiguous run): every lane reads two runs of four
// consecutive keys.  No LDS is used.
// q, K, V^T and P are bf16 hi/lo pairs (hi + lo carries about 16 mantissa bits): every product
// is hi*hi + lo*hi + hi*lo in fp32 accumulators.  A single bf16 rounding of K, V, q or P moves
// the 32-layer, d=4096 model's confidences by several percent; the pairs keep the attention at
// fp32-like accuracy for 1.5x the MFMA work of one bf16 pass per operand pair.
// When the tiles alone cannot fill the GPU (a cached step has few queries) the keys are split
// into chunks; each chunk writes (O, running max, sum) and a merge kernel combines the chunks
// in chunk order.
//
// f32 path: one workgroup per (query row, head): scores in LDS, then weights times V.
//
// Every kernel lets a query see the keys below rs.key_limit of its slot: the context length,
// or with block-causal attention the end of the query's block.
#include "kernels.h"

#include <algorithm>

namespace dllm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

static constexpr int ATTN_MAX_SPLITS = 16;  // key chunks of one query tile (merge width)

static inline int attn_tiles(RowSet rs, int H, int Hkv) {
  return (rs.nR * (H / Hkv) + 31) / 32;
}

static inline void attn_plan(RowSet rs, int H, int Hkv, int &splits, int &chunk) {
  const long waves = (long)attn_tiles(rs, H, Hkv) * rs.B * Hkv;
  const int kt = (rs.L + 31) / 32;  // 32-key tiles of the context
  int want = (int)((256 + waves - 1) / waves);
  if (want > kt) want = kt;
  if (want > ATTN_MAX_SPLITS) want = ATTN_MAX_SPLITS;
  if (want < 1) want = 1;
  chunk = (kt + want - 1) / want * 32;
  splits = (kt * 32 + chunk - 1) / chunk;
}

// Query tiles per workgroup of the many-query kernel for nqt query tiles per (batch row, K/V
// head): 4, or 2 for two or three (then a pair's K/V tiles still come from HBM once and are
// shared through LDS, where one-tile workgroups of the few-query kernel would each stream
// them); 0: the few-query kernel.
static inline int aw_group(int nqt) { return nqt >= 4 ? 4 : nqt >= 2 ? 2 : 0; }

// Many-query kernel (one workgroup per CU with four query tiles, two with two): split the keys
// only when the workgroups fill less than half of the 256 CUs.  A workgroup's time per key tile
// hardly changes with the number of workgroups (measured: 768 queries x 32 heads, 192
// workgroups, 79 us whole; 4 chunks 70 us plus 21 us to merge), so splitting pays only when
// most CUs would idle.
static inline void attn_wide_plan(RowSet rs, int H, int Hkv, int &splits, int &chunk) {
  const int nqt = attn_tiles(rs, H, Hkv), qg = aw_group(nqt);
  const long wgs = (long)((nqt + qg - 1) / qg) * rs.B * Hkv;
  const int kt = (rs.L + 31) / 32;
  int want = wgs * 2 > 256 ? 1 : (int)std::min<long>(4, 256 / wgs);
  want = std::max(1, std::min(want, kt / 2));
  chunk = (kt + want - 1) / want * 32;
  splits = (kt * 32 + chunk - 1) / chunk;
}

size_t attention_part_bytes(RowSet rs, int H, int Hkv, int hd, int dtype) {
  if (dtype == 0) return 0;
  int splits, chunk;
  const int nqt = attn_tiles(rs, H, Hkv), qg = aw_group(nqt);
  if (qg) {
    attn_wide_plan(rs, H, Hkv, splits, chunk);
    if (splits == 1) return 0;
    const int n_qt = (nqt + qg - 1) / qg * qg;
    return (size_t)splits * rs.B * Hkv * n_qt * 32 * (hd + 2) * sizeof(float);
  }
  attn_plan(rs, H, Hkv, splits, chunk);
  if (splits == 1) return 0;
  return (size_t)splits * rs.B * Hkv * nqt * 32 * (hd + 2) * sizeof(float);
}

// Workgroup order of the attention grids (x = blocks of 8 (batch row, K/V head) pairs, each
// block holding the query tiles (or tile groups) of its pairs 8 apart; y = 1; z = key chunk):
// workgroup i runs on XCD i % 8, so the tiles of one pair run on one XCD, where the second
// reader of a K/V tile finds it in the L2, and the workgroups in flight at one time cover few
// pairs.  Pairs past B * Hkv (the last block's padding) return at once.
__device__ inline void attn_grid_order(int x, int npairs, int &pair, int &tile) {
  const int ntiles = gridDim.x / ((npairs + 7) / 8 * 8);
  const int blk = x / (8 * ntiles), r = x - blk * 8 * ntiles;
  tile = r >> 3;
  pair = blk * 8 + (r & 7);
}
static inline unsigned attn_grid_x(int npairs, int ntiles) {
  return (unsigned)((npairs + 7) / 8 * 8 * ntiles);
}

// Reference maximum of the online softmax (log2 units).  The probabilities of a tile are
// exp2(s - m) against a per-query reference m that moves only when a score exceeds it by more
// than REF_SLACK: then m becomes the running maximum and the output and sum so far are rescaled.
// Otherwise p may reach 2^REF_SLACK, far from fp32 and bf16 limits, and since the output and
// the sum share the reference the normalised result is the same as with the exact running
// maximum (up to rounding).  With the exact maximum nearly every tile moved some query's
// maximum in a 32-query tile, so the (register-file) rescale of the output ran every tile.
static constexpr float REF_SLACK = 8.0f;
__device__ inline float ref_max(float mref, float tmax) {
  return tmax > mref + REF_SLACK ? tmax : mref;  // mref = -inf: any visible score sets it
}

template <int HD>
__global__ __launch_bounds__(64) void attn_mfma_kernel(
    const bf16 *__restrict__ q_hi, const bf16 *__restrict__ q_lo, const bf16 *__restrict__ k_hi,
    const bf16 *__restrict__ k_lo, const bf16 *__restrict__ vt_hi, const bf16 *__restrict__ vt_lo,
    RowSet rs, int H, int Hkv, int chunk, float scale_log2, bf16 *o_hi, bf16 *o_lo, float *part,
    int o_packed) {
  constexpr int KS = HD / 16;  // k-steps of the QK^T product
  constexpr int DB = HD / 32;  // 32-dim blocks of the output
  const int G = H / Hkv;
  const int nrows = rs.nR * G;
  const int npairs = rs.B * Hkv, split = blockIdx.z;
  int bg, qt;
  attn_grid_order(blockIdx.x, npairs, bg, qt);
  if (bg >= npairs) return;
  const int nqt = gridDim.x / ((npairs + 7) / 8 * 8);
  const int b = bg / Hkv, g = bg % Hkv;
  const int lane = threadIdx.x, col = lane & 31, half = lane >> 5;

  const int r = qt * 32 + col;
  const bool valid = r < nrows;
  const int pi = valid ? r / G : 0;
  const int head = g * G + (valid ? r % G : 0);
  const int m = b * rs.nR + pi;
  const int ldq = H * HD;
  const int klim = rs.key_limit(rs.start + pi);  // keys this lane's query may see

  // Q^T as the B operand: lane = query column, 8 dims per k-step.
  bf16x8_t qh[KS], ql[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    const size_t o = (size_t)m * ldq + head * HD + kk * 16 + half * 8;
    if (valid) {
      qh[kk] = *(const bf16x8_t *)(q_hi + o);
      ql[kk] = *(const bf16x8_t *)(q_lo + o);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qh[kk][e] = ql[kk][e] = (__bf16)0.f;
    }
  }
  // K [Lp][HD]; V^T in 32-key tiles [Lp/32][HD][32]; both HD * Lp per (batch row, K/V head)
  const size_t kv_off = (size_t)bg * rs.Lp * HD;
  const bf16 *Kh = k_hi + kv_off, *Kl = k_lo + kv_off;
  const bf16 *Vh = vt_hi + kv_off, *Vl = vt_lo + kv_off;

  float mrun = -INFINITY, lsum = 0.f;
  f32x16 o[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[d][i] = 0.f;

  const int kbeg = split * chunk;
  const int kend = min((rs.L + 31) / 32 * 32, kbeg + chunk);
  // One 32-key tile's operands: K rows (hi/lo, 8 dims per k-step) and V^T runs (hi/lo, two runs
  // of four keys per 16-key step).  A tile's K and V are loaded together, and the next tile's
  // while the current one is computed, so the wave waits for one load latency per chunk rather
  // than two per tile.
  struct Tile {
    bf16x8_t kh[KS], kl[KS];
    bf16x8_t vh[DB][2], vl[DB][2];
  };
  auto load_tile = [&](int kb, Tile &t) {
    const size_t krow = (size_t)(kb + col) * HD + half * 8;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      t.kh[kk] = *(const bf16x8_t *)(Kh + krow + kk * 16);
      t.kl[kk] = *(const bf16x8_t *)(Kl + krow + kk * 16);
    }
#pragma unroll
    for (int d = 0; d < DB; ++d) {
      // this lane's keys of 16-key step ks are chunk 2 ks + half of the tile row (vt_key_pos)
      const size_t vrow = (size_t)(kb >> 5) * (HD * 32) + (d * 32 + col) * 32 + 8 * half;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        t.vh[d][ks] = *(const bf16x8_t *)(Vh + vrow + 16 * ks);
        t.vl[d][ks] = *(const bf16x8_t *)(Vl + vrow + 16 * ks);
      }
    }
  };
  auto compute_tile = [&](int kb, const Tile &t) {
    // S^T = K Q^T with hi/lo operands (the lo x lo term is below fp32 resolution).
    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(t.kh[kk], qh[kk], s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(t.kl[kk], qh[kk], s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(t.kh[kk], ql[kk], s, 0, 0, 0);
    }
    // s[i]: key kb + 8*(i/4) + 4*half + i%4, query col
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kb + 8 * (i >> 2) + 4 * half + (i & 3);
      s[i] = key < klim ? s[i] * scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, s[i]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float mnew = ref_max(mrun, tmax);
    const float alpha = mrun == -INFINITY ? 0.f : exp2f(mrun - mnew);
    // P^T as hi/lo B operands of the next product; register i of k-step i/8 holds key slot i%8.
    // (A lane with no visible key yet has mnew = -inf: its probabilities are 0, not NaN.)
    bf16x8_t ph[2], pl[2];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float pv = mnew == -INFINITY ? 0.f : exp2f(s[i] - mnew);
      const __bf16 hi = (__bf16)pv;
      ph[i >> 3][i & 7] = hi;
      pl[i >> 3][i & 7] = (__bf16)(pv - (float)hi);
      psum += pv;
    }
    psum += __shfl_xor(psum, 32, 64);
    lsum = lsum * alpha + psum;
    mrun = mnew;
    // rescale the running output only when some lane's reference moved (alpha is exactly 1
    // otherwise, so skipping changes nothing); after the first tile it rarely moves
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[d][i] *= alpha;
    }
    // consecutive MFMAs update different accumulators (the DB chains run side by side)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int d = 0; d < DB; ++d) o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(t.vh[d][ks], ph[ks], o[d], 0, 0, 0);
#pragma unroll
      for (int d = 0; d < DB; ++d) o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(t.vl[d][ks], ph[ks], o[d], 0, 0, 0);
#pragma unroll
      for (int d = 0; d < DB; ++d) o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(t.vh[d][ks], pl[ks], o[d], 0, 0, 0);
    }
  };
  // Unrolled by two so that the two tile buffers stay in fixed registers.  Past the chunk's end
  // the prefetch re-reads the last tile (values unused), keeping the loads unconditional.
  Tile ta, tb;
  const int last = kend - 32;
  if (kbeg < kend) load_tile(kbeg, ta);
  for (int kb = kbeg; kb < kend; kb += 64) {
    load_tile(min(kb + 32, last), tb);
    compute_tile(kb, ta);
    if (kb + 32 < kend) {
      load_tile(min(kb + 64, last), ta);
      compute_tile(kb + 32, tb);
    }
  }
  if (!valid) return;
  // o[d][i]: dim d*32 + 8*(i/4) + 4*half + i%4 of query col
  if (gridDim.z == 1) {
    const float inv = 1.0f / lsum;
    // output row m, columns head * HD + dim (panel-packed for a large-tile output projection)
    const size_t obase = o_packed ? pa_off(m, head * HD, ldq) : (size_t)m * ldq + head * HD;
    bf16 *oh = o_hi + obase;
    bf16 *ol = o_lo + obase;
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int dim = d * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
        const float v = o[d][i] * inv;
        const bf16 hi = __float2bfloat16(v);
        const size_t od = o_packed ? (size_t)(dim >> 5) * 4096 + (dim & 31) : (size_t)dim;
        oh[od] = hi;
        ol[od] = __float2bfloat16(v - __bfloat162float(hi));
      }
  } else {
    // part[split][bg][qt][col][HD + 2]
    float *pp = part + ((((size_t)split * npairs + bg) * nqt + qt) * 32 + col) * (HD + 2);
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) pp[d * 32 + 8 * (i >> 2) + 4 * half + (i & 3)] = o[d][i];
    if (half == 0) {
      pp[HD] = mrun;
      pp[HD + 1] = lsum;
    }
  }
}

// Many-query variant (block refresh, steps of wide blocks): QT KH waves per workgroup, all of
// the same (batch row, K/V head): QT query tiles of 32 queries (4, or 2 when a pair has only two
// or three).  With QT = 4 each query tile is run by KH = 2 waves that take alternate 32-key tiles
// (key half 0 the even ones, key half 1 the odd ones), so every SIMD holds two waves and one
// wave's MFMAs overlap the other's softmax and LDS reads.  With QT = 2 (KH = 1) each query
// tile's wave takes every key tile: the workgroup needs half the LDS, so two fit a CU (64
// queries x 5120 keys per pair: 555 -> 500 us against key halves, whose 128 KB workgroups ran
// one per CU, when launched alone; within the decode's noise in the long-context cached step).
// Each iteration brings KH key tiles (K and V^T, hi and
// lo) straight from global memory into one of two LDS slots (global_load_lds, 16 bytes per lane,
// no register staging) while the waves work on the other slot; one barrier per iteration.  At
// the end the two waves of a query tile (KH = 2) merge their (reference maximum, sum, output)
// through LDS.  In a tile, row r's 16-byte chunk c sits at chunk
// position r * CPR + (c ^ f(r)) (CPR chunks per row: f(r) = r & 15 for 16, (r >> 1) & 7 for 8,
// (r >> 2) & 3 for 4), so the fragment reads of 16 consecutive rows cover the 64 banks (256
// bytes) of the LDS once.  When the workgroups cannot fill the GPU the keys are split into chunks
// (partials + the merge kernel).

__device__ inline int aw_swz(int r, int cpr) {
  return cpr >= 16 ? (r & 15) : cpr == 8 ? ((r >> 1) & 7) : ((r >> 2) & 3);
}

template <int HD, int QT, int KH>
__global__ __launch_bounds__(64 * QT * KH, 1) void attn_wide_kernel(
    const bf16 *__restrict__ q_hi, const bf16 *__restrict__ q_lo, const bf16 *__restrict__ k_hi,
    const bf16 *__restrict__ k_lo, const bf16 *__restrict__ vt_hi, const bf16 *__restrict__ vt_lo,
    RowSet rs, int H, int Hkv, int chunk, float scale_log2, bf16 *o_hi, bf16 *o_lo, float *part,
    int o_packed) {
  constexpr int KS = HD / 16, DB = HD / 32;
  constexpr int PLANE = 32 * HD * 2;          // bytes of one plane of a 32-key tile
  constexpr int TILE = 4 * PLANE;             // K hi, K lo, V^T hi, V^T lo
  constexpr int PAIR = KH * TILE;          // the tiles of one iteration, one per key half
  constexpr int NW = QT * KH;
  constexpr int LPW = PAIR / 1024 / NW;       // 1 KB loads per wave per iteration
  constexpr int KCPR = HD / 8, VCPR = 4;      // 16-byte chunks per K row / per V^T row
  static_assert(PAIR % (1024 * NW) == 0 && LPW >= 1 && LPW <= 32, "tile staging");
  static_assert(LPW * 64 * QT == TILE / 16, "the waves of key half h load tile h");
  // the merge of the key halves reuses the ring: outputs [query tile][d][i][lane], then
  // (reference maximum, sum) [query tile][2][lane]
  static_assert(KH == 1 || QT * (DB * 16 + 2) * 64 * 4 <= 2 * PAIR, "merge area");
  typedef __attribute__((address_space(3))) void lds_void;
  __shared__ __align__(1024) unsigned char lds[2 * PAIR];

  const int G = H / Hkv;
  const int nrows = rs.nR * G;
  const int npairs = rs.B * Hkv, split = blockIdx.z;
  int bg, grp;
  attn_grid_order(blockIdx.x, npairs, bg, grp);
  if (bg >= npairs) return;  // the whole workgroup, before any barrier
  const int n_qt = gridDim.x / ((npairs + 7) / 8 * 8) * QT;
  const int b = bg / Hkv, g = bg % Hkv;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int qw = wave % QT, kh = wave / QT;
  const int qt = grp * QT + qw;
  const int r = qt * 32 + col;
  const bool valid = r < nrows;
  const int pi = valid ? r / G : 0;
  const int head = g * G + (valid ? r % G : 0);
  const int m = b * rs.nR + pi;
  const int ldq = H * HD;
  const int klim = rs.key_limit(rs.start + pi);  // keys this lane's query may see

  bf16x8_t qh[KS], ql[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    const size_t o = (size_t)m * ldq + head * HD + kk * 16 + half * 8;
    qh[kk] = *(const bf16x8_t *)(q_hi + o);  // invalid rows read row m of batch b: harmless
    ql[kk] = *(const bf16x8_t *)(q_lo + o);
  }
  // K [Lp][HD]; V^T in 32-key tiles [Lp/32][HD][32]: tile kb of either plane starts kb * HD in
  const size_t kv_off = (size_t)bg * rs.Lp * HD;
  // load j of this wave fills chunk position e = (wave * LPW + j) * 64 + lane of the pair slot:
  // tile e / (TILE / 16) = kh of the pair, then plane and position inside the tile
  const uint16_t *src[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int e = (wave * LPW + j) * 64 + lane, et = e % (TILE / 16);
    const int plane = et / (PLANE / 16), pos = et % (PLANE / 16);
    const bf16 *base = plane == 0 ? k_hi : plane == 1 ? k_lo : plane == 2 ? vt_hi : vt_lo;
    int off;
    if (plane < 2) {
      const int rr = pos / KCPR, c = (pos % KCPR) ^ aw_swz(rr, KCPR);
      off = rr * HD + c * 8;
    } else {
      const int rr = pos / VCPR, c = (pos % VCPR) ^ aw_swz(rr, VCPR);
      off = rr * 32 + c * 8;
    }
    src[j] = (const uint16_t *)base + kv_off + off;
  }
  const int ntile = (rs.L + 31) / 32;
  const int t0 = split * (chunk / 32), t1 = min(ntile, t0 + chunk / 32), T = t1 - t0;
  const int NI = (T + KH - 1) / KH;  // iterations
  auto issue = [&](int u) {  // tile t0 + 2u + kh (clamped to the last) into slot u % 2
    unsigned char *dst = lds + (u & 1) * PAIR + wave * LPW * 1024;
    const size_t kb = (size_t)(t0 + min(u * KH + kh, T - 1)) * 32;
#pragma unroll
    for (int j = 0; j < LPW; ++j)
      __builtin_amdgcn_global_load_lds((const void *)(src[j] + kb * HD), (lds_void *)(dst + j * 1024), 16, 0, 0);
  };

  float mrun = -INFINITY, lsum = 0.f;
  f32x16 o[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[d][i] = 0.f;

  // fragment positions (bytes in a plane): K row col, chunk 2 kk + half; V^T row d * 32 + col,
  // chunk 2 ks + half
  const int ksw = aw_swz(col, KCPR), krow = col * KCPR;
  issue(0);
  for (int u = 0; u < NI; ++u) {
    // this wave's loads of pair u have landed (nothing else is outstanding); after the barrier
    // every wave's have, and every wave is done with pair u - 1, whose slot the next issue fills
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (u + 1 < NI) issue(u + 1);
    const int tl = u * KH + kh;  // this wave's tile, counted from t0
    const bool tok = tl < T;        // the odd count's last pair has one tile
    const int kb = (t0 + tl) * 32;
    const unsigned char *cur = lds + (u & 1) * PAIR + kh * TILE;
    __builtin_amdgcn_sched_barrier(0);
    // S^T of the tile (32 keys x 32 queries), three terms of the hi/lo pairs
    f32x16 sc;
    {
      bf16x8_t kfh[KS], kfl[KS];
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const int pos = (krow + ((kk * 2 + half) ^ ksw)) * 16;
        kfh[kk] = *(const bf16x8_t *)(cur + pos);
        kfl[kk] = *(const bf16x8_t *)(cur + PLANE + pos);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfh[kk], qh[kk], sc, 0, 0, 0);
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfl[kk], qh[kk], sc, 0, 0, 0);
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfh[kk], ql[kk], sc, 0, 0, 0);
      }
    }
    // softmax against the reference maximum; lane (col, half) holds keys
    // kb + 8 (k / 4) + 4 half + k % 4 of query col
    float tmax = -INFINITY;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int key = kb + 8 * (k >> 2) + 4 * half + (k & 3);
      sc[k] = tok && key < klim ? sc[k] * scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, sc[k]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float mnew = ref_max(mrun, tmax);
    const float alpha = mrun == -INFINITY ? 0.f : exp2f(mrun - mnew);
    bf16x8_t ph[2], pl[2];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float pv = mnew == -INFINITY ? 0.f : exp2f(sc[i] - mnew);
      const __bf16 hi = (__bf16)pv;
      ph[i >> 3][i & 7] = hi;
      pl[i >> 3][i & 7] = (__bf16)(pv - (float)hi);
      psum += pv;
    }
    psum += __shfl_xor(psum, 32, 64);
    lsum = lsum * alpha + psum;
    mrun = mnew;
    // V^T fragments only now: K and V^T fragments are never live together
    __builtin_amdgcn_sched_barrier(0);
    bf16x8_t vfh[DB][2], vfl[DB][2];
#pragma unroll
    for (int d = 0; d < DB; ++d) {
      const int vr = d * 32 + col, vsw = aw_swz(vr, VCPR);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int pos = (vr * VCPR + ((ks * 2 + half) ^ vsw)) * 16;
        vfh[d][ks] = *(const bf16x8_t *)(cur + 2 * PLANE + pos);
        vfl[d][ks] = *(const bf16x8_t *)(cur + 3 * PLANE + pos);
      }
    }
    // rescale the running output only when some lane's reference moved (alpha is exactly 1
    // otherwise, so skipping changes nothing); after the first tile it rarely moves
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[d][i] *= alpha;
    }
    // consecutive MFMAs update different accumulators (the DB chains run side by side)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int d = 0; d < DB; ++d) o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfh[d][ks], ph[ks], o[d], 0, 0, 0);
#pragma unroll
      for (int d = 0; d < DB; ++d) o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfl[d][ks], ph[ks], o[d], 0, 0, 0);
#pragma unroll
      for (int d = 0; d < DB; ++d) o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfh[d][ks], pl[ks], o[d], 0, 0, 0);
    }
  }
  // merge the key halves: half 1 hands its state to half 0 through the (now idle) ring
  if constexpr (KH == 2) {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no load still writes LDS
  __syncthreads();
  float *xo = (float *)lds;
  float *xm = xo + QT * DB * 16 * 64;
  if (kh == 1) {
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) xo[((qw * DB + d) * 16 + i) * 64 + lane] = o[d][i];
    xm[(qw * 2) * 64 + lane] = mrun;
    xm[(qw * 2 + 1) * 64 + lane] = lsum;
  }
  __syncthreads();
  if (kh == 1 || !valid) return;
  {
    const float m2 = xm[(qw * 2) * 64 + lane], l2 = xm[(qw * 2 + 1) * 64 + lane];
    const float mt = fmaxf(mrun, m2);
    const float a1 = mrun == -INFINITY ? 0.f : exp2f(mrun - mt);
    const float a2 = m2 == -INFINITY ? 0.f : exp2f(m2 - mt);
    lsum = lsum * a1 + l2 * a2;
    mrun = mt;
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[d][i] = o[d][i] * a1 + xo[((qw * DB + d) * 16 + i) * 64 + lane] * a2;
  }
  } else {
    if (!valid) return;
  }
  if (gridDim.z == 1) {
    const float inv = 1.0f / lsum;
    // output row m, columns head * HD + dim (panel-packed for a large-tile output projection)
    const size_t obase = o_packed ? pa_off(m, head * HD, ldq) : (size_t)m * ldq + head * HD;
    bf16 *oh = o_hi + obase;
    bf16 *ol = o_lo + obase;
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int dim = d * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
        const float v = o[d][i] * inv;
        const bf16 hi = __float2bfloat16(v);
        const size_t od = o_packed ? (size_t)(dim >> 5) * 4096 + (dim & 31) : (size_t)dim;
        oh[od] = hi;
        ol[od] = __float2bfloat16(v - __bfloat162float(hi));
      }
  } else {
    // part[split][bg][qt][col][HD + 2], as the few-query kernel writes it
    float *pp = part + ((((size_t)split * npairs + bg) * n_qt + qt) * 32 + col) * (HD + 2);
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) pp[d * 32 + 8 * (i >> 2) + 4 * half + (i & 3)] = o[d][i];
    if (half == 0) {
      pp[HD] = mrun;
      pp[HD + 1] = lsum;
    }
  }
}

// Combine the key chunks: one wave per query row slot, lanes over dims.
static constexpr int MG_ROWS = 4;  // query rows (waves) per merge workgroup

template <int HD>
__global__ __launch_bounds__(64 * MG_ROWS) void attn_merge_kernel(const float *__restrict__ part,
                                                                  RowSet rs, int H, int Hkv,
                                                                  int n_qt, int splits,
                                                                  bf16 *o_hi, bf16 *o_lo,
                                                                  int o_packed) {
  const int G = H / Hkv;
  const int slot = blockIdx.x * MG_ROWS + (threadIdx.x >> 6);  // (bg, qt, col)
  if (slot >= rs.B * Hkv * n_qt * 32) return;
  const int col = slot % 32, qt = (slot / 32) % n_qt, bg = slot / 32 / n_qt;
  const int r = qt * 32 + col;
  if (r >= rs.nR * G) return;
  const int b = bg / Hkv, g = bg % Hkv;
  const int m = b * rs.nR + r / G, head = g * G + r % G;
  const size_t stride = (size_t)rs.B * Hkv * n_qt * 32 * (HD + 2);
  const float *p0 = part + (((size_t)bg * n_qt + qt) * 32 + col) * (HD + 2);
  // lane s holds chunk s's running max and sum; every load of the merge is issued before the
  // first one is used (one memory latency instead of one per chunk), and the sums still run in
  // chunk order
  const int lane = threadIdx.x & 63;
  float m_own = -INFINITY, l_own = 0.f;
  if (lane < splits) {
    m_own = p0[lane * stride + HD];
    l_own = p0[lane * stride + HD + 1];
  }
  constexpr int DPL = (HD + 63) / 64;  // dims per lane (lanes past HD idle when HD < 64)
  const bool dim_ok = lane < HD;
  float v[ATTN_MAX_SPLITS][DPL];
#pragma unroll
  for (int s = 0; s < ATTN_MAX_SPLITS; ++s)
#pragma unroll
    for (int j = 0; j < DPL; ++j) v[s][j] = (s < splits && dim_ok) ? p0[s * stride + lane + 64 * j] : 0.f;
  float mx = -INFINITY;
#pragma unroll
  for (int s = 0; s < ATTN_MAX_SPLITS; ++s)
    if (s < splits) mx = fmaxf(mx, __shfl(m_own, s, 64));
  float l = 0.f, w[ATTN_MAX_SPLITS];
#pragma unroll
  for (int s = 0; s < ATTN_MAX_SPLITS; ++s) {
    const float ms = __shfl(m_own, s, 64), ls = __shfl(l_own, s, 64);
    w[s] = (s < splits && ms > -INFINITY) ? exp2f(ms - mx) : 0.f;
    if (s < splits && ms > -INFINITY) l += ls * w[s];
  }
  const float inv = 1.0f / l;
#pragma unroll
  for (int j = 0; j < DPL; ++j) {
    float acc = 0.f;
#pragma unroll
    for (int s = 0; s < ATTN_MAX_SPLITS; ++s)
      if (w[s] != 0.f) acc += v[s][j] * w[s];
    const float val = acc * inv;
    if (!dim_ok) break;
    const size_t o = o_packed ? pa_off(m, head * HD + lane + 64 * j, H * HD)
                              : (size_t)m * H * HD + head * HD + lane + 64 * j;
    const bf16 hi = __float2bfloat16(val);
    o_hi[o] = hi;
    o_lo[o] = __float2bfloat16(val - __bfloat162float(hi));
  }
}

// fp32: one workgroup of 64 per (row m, head).  Dynamic LDS: Lp scores.
__global__ __launch_bounds__(64) void attn_f32_kernel(const float *__restrict__ q,
                                                      const float *__restrict__ kc,
                                                      const float *__restrict__ vt, RowSet rs,
                                                      int H, int Hkv, int hd, float scale,
                                                      float *o) {
  extern __shared__ float sc[];
  const int m = blockIdx.x, head = blockIdx.y;
  const int b = m / rs.nR;
  const int g = head / (H / Hkv);
  const float *qr = q + (size_t)m * H * hd + head * hd;
  const float *K = kc + ((size_t)b * Hkv + g) * rs.Lp * hd;
  const float *V = vt + ((size_t)b * Hkv + g) * hd * rs.Lp;
  const int lane = threadIdx.x;
  const int nk = rs.key_limit(rs.start + m % rs.nR);  // keys this query may see
  float mx = -INFINITY;
  for (int key = lane; key < nk; key += 64) {
    float s = 0.f;
    for (int d = 0; d < hd; ++d) s = fmaf(qr[d], K[(size_t)key * hd + d], s);
    s *= scale;
    sc[key] = s;
    mx = fmaxf(mx, s);
  }
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  float sum = 0.f;
  for (int key = lane; key < nk; key += 64) {
    const float p = expf(sc[key] - mx);
    sc[key] = p;
    sum += p;
  }
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
  __syncthreads();
  for (int d = lane; d < hd; d += 64) {
    float acc = 0.f;
    const float *vr = V + (size_t)d * rs.Lp;
    for (int key = 0; key < nk; ++key) acc = fmaf(sc[key], vr[key], acc);
    o[(size_t)m * H * hd + head * hd + d] = acc / sum;
  }
}

hipError_t launch_attention(const void *q, const void *q_lo, const void *k_cache,
                            const void *k_cache_lo, const void *vt_cache, const void *vt_cache_lo,
                            RowSet rs, int H, int Hkv, int hd, bf16 *o_hi, bf16 *o_lo, float *o_f32,
                            float *part, int dtype, int o_packed, hipStream_t st) {
  if (rs.M() <= 0) return hipSuccess;
  if (o_packed && (dtype == 0 || (H * hd) % 32 || hd % 32)) return hipErrorInvalidValue;
  if (dtype == 0) {
    dim3 grid(rs.M(), H);
    hipLaunchKernelGGL(attn_f32_kernel, grid, dim3(64), rs.Lp * sizeof(float), st,
                       (const float *)q, (const float *)k_cache, (const float *)vt_cache, rs, H,
                       Hkv, hd, 1.0f / sqrtf((float)hd), o_f32);
    return hipGetLastError();
  }
  const int nqt = attn_tiles(rs, H, Hkv);
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)hd);
  const int qg = aw_group(nqt);
  if (qg) {
    // many queries: K/V tiles shared by the query tiles of a workgroup through LDS
    int wsplits, wchunk;
    attn_wide_plan(rs, H, Hkv, wsplits, wchunk);
    const int groups = (nqt + qg - 1) / qg;
    dim3 wgrid(attn_grid_x(rs.B * Hkv, groups), 1, wsplits);
#define ATTNW_LAUNCH(HDV, QTV)                                                                   \
  hipLaunchKernelGGL((attn_wide_kernel<HDV, QTV, (QTV == 4 ? 2 : 1)>), wgrid,                   \
                     dim3(64 * QTV * (QTV == 4 ? 2 : 1)), 0, st,                                 \
                     (const bf16 *)q, (const bf16 *)q_lo, (const bf16 *)k_cache,                \
                     (const bf16 *)k_cache_lo, (const bf16 *)vt_cache, (const bf16 *)vt_cache_lo, \
                     rs, H, Hkv, wchunk, scale_log2, o_hi, o_lo, part, o_packed)
#define ATTNW_CASE(HDV)                                                                          \
  case HDV:                                                                                      \
    if (qg == 4) ATTNW_LAUNCH(HDV, 4);                                                           \
    else ATTNW_LAUNCH(HDV, 2);                                                                   \
    if (wsplits > 1)                                                                             \
      hipLaunchKernelGGL(attn_merge_kernel<HDV>,                                                 \
                         dim3((rs.B * Hkv * groups * qg * 32 + MG_ROWS - 1) / MG_ROWS),          \
                         dim3(64 * MG_ROWS), 0, st, (const float *)part, rs, H, Hkv,             \
                         groups * qg, wsplits, o_hi, o_lo, o_packed);                            \
    break;
    switch (hd) {
      ATTNW_CASE(32)
      ATTNW_CASE(64)
      ATTNW_CASE(128)
      default:
        return hipErrorInvalidValue;
    }
#undef ATTNW_CASE
#undef ATTNW_LAUNCH
    return hipGetLastError();
  }
  int splits, chunk;
  attn_plan(rs, H, Hkv, splits, chunk);
  dim3 grid(attn_grid_x(rs.B * Hkv, nqt), 1, splits);
#define ATTN_CASE(HDV)                                                                          \
  case HDV:                                                                                     \
    hipLaunchKernelGGL(attn_mfma_kernel<HDV>, grid, dim3(64), 0, st, (const bf16 *)q,           \
                       (const bf16 *)q_lo, (const bf16 *)k_cache, (const bf16 *)k_cache_lo,     \
                       (const bf16 *)vt_cache, (const bf16 *)vt_cache_lo, rs, H, Hkv, chunk,    \
                       scale_log2, o_hi, o_lo, part, o_packed);                                 \
    if (splits > 1)                                                                             \
      hipLaunchKernelGGL(attn_merge_kernel<HDV>, dim3((rs.B * Hkv * nqt * 32 + MG_ROWS - 1) / MG_ROWS), \
                         dim3(64 * MG_ROWS), 0, st, (const float *)part, rs, H, Hkv, nqt, splits, \
                         o_hi, o_lo, o_packed);                                                 \
    break;
  switch (hd) {
    ATTN_CASE(32)
    ATTN_CASE(64)
    ATTN_CASE(128)
    default:
      return hipErrorInvalidValue;
  }
#undef ATTN_CASE
  return hipGetLastError();
}

}  // namespace dllm
