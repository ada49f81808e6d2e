// GEMM C[m][n] = sum_k A[m][k] * W[n][k] for the projections, the feed-forward and the lm_head,
// with fused epilogues.  W is in torch Linear layout [out, in], so both operands are
// K-contiguous.
//
// A operand, bf16 path: two bf16 values (hi, lo) per element with hi + lo equal to the fp32
// activation to about 16 mantissa bits; each K step issues two bf16 MFMAs (hi x W, lo x W) into
// one fp32 accumulator.  At the row counts of a cached step the GEMM is bound by streaming W
// from HBM, so the second MFMA costs no time and keeps the activation error at fp32 level.
//
// Tiles are staged through LDS.  After the K loop the wave accumulators are written to an fp32
// C tile in LDS so that every epilogue has random access to the whole tile (rotary pairs i and
// i + hd/2, gate and up halves, row-wise softmax over a vocabulary tile).  Split-K: every split
// writes its tile to a partial buffer and a reduce kernel sums the splits in split order
// (deterministic) and runs the epilogue; for the residual add that reduce is the caller's
// resid_norm kernel, which also applies the next RMSNorm.
#include "kernels.h"

#include <algorithm>
#include <functional>
#include <map>
#include <mutex>
#include <queue>
#include <tuple>
#include <vector>
#include <float.h>
#include <limits.h>

namespace dllm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

static constexpr int NT = 256;  // threads per workgroup (4 waves)

// ---------------------------------------------------------------------------------------------
// W row addressing (virtual rows: concatenated segments, or interleaved gate/up halves).
template <typename T>
__device__ inline const T *w_row(const GemmArgs &a, int bn, int n0, int c) {
  if (a.epi == EPI_SWIGLU) {
    const int half = bn / 2;
    const int t = n0 / bn;
    const int f = t * half + (c < half ? c : c - half);
    if (f >= a.n_half) return nullptr;
    return (const T *)a.w[c < half ? 0 : 1] + (size_t)f * a.K;
  }
  const int n = n0 + c;
  if (n >= a.N) return nullptr;
  int s = 0, base = 0;
  while (s < 2 && n >= a.seg_end[s]) { base = a.seg_end[s]; ++s; }
  return (const T *)a.w[s] + (size_t)(n - base) * a.K;
}

// ---------------------------------------------------------------------------------------------
// A operand loading: row m of A is row a_row(m) of the hi/lo planes.
__device__ inline int a_row(const GemmArgs &a, int m) {
  return a.row_per ? (m / a.row_per) * a.row_stride + a.row_off + m % a.row_per : m;
}

// ---------------------------------------------------------------------------------------------
// Packed W: start of panel p (128 rows), block kb (32 columns); row r of the block at r * 32.
__device__ inline const uint16_t *wp_block(const GemmArgs &a, int p, int kb) {
  return a.wp + ((size_t)p * (a.K / PW_K) + kb) * (PW_ROWS * PW_K);
}

// Pack kernel: one thread per 16-byte chunk of the packed matrix (coalesced writes).
__global__ __launch_bounds__(256) void pack_weight_kernel(uint16_t *dst, const GemmArgs a, int mode,
                                                          size_t chunks) {
  const size_t q = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  if (q >= chunks) return;
  const int kblocks = a.K / PW_K;
  const size_t blk = q / (PW_ROWS * PW_K / 8);
  const int within = (int)(q % (PW_ROWS * PW_K / 8));
  const int p = (int)(blk / kblocks), kb = (int)(blk % kblocks);
  const int r = within / (PW_K / 8), c8 = (within % (PW_K / 8)) * 8;
  const int n = p * PW_ROWS + r, k = kb * PW_K + c8;
  const uint16_t *src = nullptr;
  if (mode == PACK_SWIGLU) {
    const int c = r, f = p * 64 + (c < 64 ? c : c - 64);
    if (f < a.n_half) src = (const uint16_t *)a.w[c < 64 ? 0 : 1] + (size_t)f * a.K;
  } else if (n < a.N) {
    int sgi = 0, base = 0;
    if (mode == PACK_CONCAT)
      while (sgi < 2 && n >= a.seg_end[sgi]) { base = a.seg_end[sgi]; ++sgi; }
    src = (const uint16_t *)a.w[sgi] + (size_t)(n - base) * a.K;
  }
  s16x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
  if (src) v = *(const s16x8 *)(src + k);
  *(s16x8 *)(dst + q * 8) = v;
}

hipError_t launch_pack_weight(uint16_t *dst, const void *const src[3], const int seg_end[3],
                              int n_half, int mode, int N, int K, hipStream_t st) {
  if (N <= 0 || K <= 0 || K % PW_K) return hipErrorInvalidValue;
  GemmArgs a{};
  for (int i = 0; i < 3; ++i) { a.w[i] = src[i]; a.seg_end[i] = seg_end[i]; }
  a.n_half = n_half; a.N = N; a.K = K;
  const size_t chunks = packed_rows(N) * (size_t)K / 8;
  hipLaunchKernelGGL(pack_weight_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, st, dst, a,
                     mode, chunks);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Epilogues over an fp32 C tile in LDS (ld = ldc).  T is the storage type of q and the cache.
__device__ inline float silu_f(float g) { return g / (1.0f + __expf(-g)); }

__device__ inline void split_hilo(float v, bf16 &hi, bf16 &lo) {
  hi = __float2bfloat16(v);
  lo = __float2bfloat16(v - __bfloat162float(hi));
}

// Store v at element i of an fp32 array, or of a bf16 hi/lo plane pair.
template <typename T> __device__ inline void store_val(void *p, void *p_lo, size_t i, float v);
template <> __device__ inline void store_val<float>(void *p, void *, size_t i, float v) {
  ((float *)p)[i] = v;
}
template <> __device__ inline void store_val<bf16>(void *p, void *p_lo, size_t i, float v) {
  bf16 hi, lo;
  split_hilo(v, hi, lo);
  ((bf16 *)p)[i] = hi;
  ((bf16 *)p_lo)[i] = lo;
}

// Store x[0..3] at elements i..i+3 (i a multiple of 4, the arrays 16-byte aligned): one fp32
// 16-byte store, or one 8-byte store per bf16 plane.
template <typename T> __device__ inline void store_val4(void *p, void *p_lo, size_t i, const float *x);
template <> __device__ inline void store_val4<float>(void *p, void *, size_t i, const float *x) {
  *(float4 *)((float *)p + i) = make_float4(x[0], x[1], x[2], x[3]);
}
template <> __device__ inline void store_val4<bf16>(void *p, void *p_lo, size_t i, const float *x) {
  uint32_t hw[2], lw[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    bf16 h0, l0, h1, l1;
    split_hilo(x[2 * j], h0, l0);
    split_hilo(x[2 * j + 1], h1, l1);
    hw[j] = (uint32_t)__bfloat16_as_ushort(h0) | ((uint32_t)__bfloat16_as_ushort(h1) << 16);
    lw[j] = (uint32_t)__bfloat16_as_ushort(l0) | ((uint32_t)__bfloat16_as_ushort(l1) << 16);
  }
  *(uint2 *)((bf16 *)p + i) = make_uint2(hw[0], hw[1]);
  *(uint2 *)((bf16 *)p_lo + i) = make_uint2(lw[0], lw[1]);
}

struct HeadAcc {
  float m1; int idx; float m2;
};
__device__ inline HeadAcc head_merge(HeadAcc a, HeadAcc b) {
  const bool bw = (b.m1 > a.m1) || (b.m1 == a.m1 && b.idx < a.idx);
  HeadAcc w = bw ? b : a, l = bw ? a : b;
  HeadAcc r;
  r.m1 = w.m1; r.idx = w.idx; r.m2 = fmaxf(w.m2, l.m1);
  return r;
}

template <typename T, int BM, int BN>
__device__ void run_epilogue(const GemmArgs &a, const float *Ct, int ldc, int m0, int n0,
                             int tid) {  // tid: 0..NT-1 among the NT threads that run it
  const int M = a.M;
  switch (a.epi) {
    case EPI_STORE: {
      for (int e = tid; e < BM * BN; e += NT) {
        const int r = e / BN, c = e % BN, m = m0 + r, n = n0 + c;
        if (m < M && n < a.N) a.out_f32[(size_t)m * a.ld_out + n] = a.scale * Ct[r * ldc + c];
      }
    } break;
    case EPI_RESID: {
      if (a.ld_out % 4 == 0 && a.N % 4 == 0) {
        // 4 consecutive columns per access (the residual rows are 16-byte aligned)
        constexpr int C4 = BN / 4;
        for (int e = tid; e < BM * C4; e += NT) {
          const int r = e / C4, c = (e % C4) * 4, m = m0 + r, n = n0 + c;
          if (m >= M || n >= a.N) continue;
          float4 *p = (float4 *)(a.resid + (size_t)m * a.ld_out + n);
          const float4 x = *(const float4 *)(Ct + r * ldc + c);
          float4 v = *p;
          v.x += x.x; v.y += x.y; v.z += x.z; v.w += x.w;
          *p = v;
        }
        break;
      }
      for (int e = tid; e < BM * BN; e += NT) {
        const int r = e / BN, c = e % BN, m = m0 + r, n = n0 + c;
        if (m < M && n < a.N) a.resid[(size_t)m * a.ld_out + n] += Ct[r * ldc + c];
      }
    } break;
    case EPI_QKV: {
      const int hd = a.head_dim, half = hd / 2, H = a.n_heads, Hkv = a.n_kv_heads;
      const int hs = __builtin_ctz(hd);  // head_dim is a power of two (launch_gemm checks)
      const int nq = H * hd, nk = Hkv * hd;
      const RowSet rs = a.rows;
      // q and k columns, row-major: a thread keeps 4 consecutive columns of one head (one side of
      // its rotation halves; consecutive threads write consecutive dims) and walks the rows
      // NT / (BN / 4) apart, its (batch row, slot) advancing with it, so nothing is divided per
      // element and every load and store moves 4 values
      if (n0 < nq + nk) {
        static_assert(NT % (BN / 4) == 0 && BN % 4 == 0, "a thread keeps its 4 columns");
        constexpr int RS = NT / (BN / 4);
        const int c = (tid % (BN / 4)) * 4, n = n0 + c;
        if (n < a.N && n < nq + nk) {
          const int i = n & (hd - 1);               // i..i+3: one side of the halves (half % 4 == 0)
          const int j = i < half ? i : i - half;
          const int pc = i < half ? c + half : c - half;  // the rotation partners (same head)
          const float sg = i < half ? -1.f : 1.f;
          const bool is_q = n < nq;
          const int kvh = (n - nq) >> hs;
          int r = tid / (BN / 4), m = m0 + r;
          int b = m / rs.nR, pr = m - b * rs.nR;
          for (; r < BM && m < M; r += RS, m += RS) {
            const int p = rs.start + pr;
            const size_t rp = (size_t)rs.pos(p) * half + j;  // rotary angles of the slot's position
            const float4 cs = *(const float4 *)(a.rope_cos + rp), sn = *(const float4 *)(a.rope_sin + rp);
            const float4 x = *(const float4 *)(Ct + r * ldc + c), xp = *(const float4 *)(Ct + r * ldc + pc);
            const float y[4] = {x.x * cs.x + sg * (xp.x * sn.x), x.y * cs.y + sg * (xp.y * sn.y),
                                x.z * cs.z + sg * (xp.z * sn.z), x.w * cs.w + sg * (xp.w * sn.w)};
            if (is_q)
              store_val4<T>(a.q_out, a.q_out_lo, (size_t)m * nq + n, y);
            else
              store_val4<T>(a.k_cache, a.k_cache_lo, (((size_t)b * Hkv + kvh) * rs.Lp + p) * hd + i, y);
            pr += RS;
            while (pr >= rs.nR) { pr -= rs.nR; ++b; }
          }
        }
      }
      // v columns, row-fastest: consecutive threads write consecutive positions of one dim, which
      // are adjacent in the transposed cache.  V^T per (batch row, K/V head): fp32 [hd][Lp]; bf16
      // in 32-key tiles [Lp/32][hd][32], so that the attention's key tile is one contiguous run
      // per plane, with the keys of a tile ordered as the attention's probability operand holds
      // them (vt_key_pos)
      if (n0 + BN > nq + nk) {
        auto vt_index = [&](int b, int p, int kvh, int i) -> size_t {
          const size_t base = ((size_t)b * Hkv + kvh) * hd * rs.Lp;
          return sizeof(T) == 2 ? base + (size_t)(p >> 5) * hd * 32 + i * 32 + vt_key_pos(p & 31)
                                : base + (size_t)i * rs.Lp + p;
        };
        if constexpr (NT % BM == 0) {
          // a thread keeps one row and walks the columns NT / BM apart
          constexpr int CS = NT / BM;
          const int r = tid % BM, m = m0 + r;
          if (m < M) {
            const int b = m / rs.nR, p = rs.start + m % rs.nR;
            for (int c = tid / BM; c < BN; c += CS) {
              const int n = n0 + c;
              if (n >= a.N) break;
              if (n < nq + nk) continue;
              const int t = n - nq - nk;
              store_val<T>(a.vt_cache, a.vt_cache_lo, vt_index(b, p, t >> hs, t & (hd - 1)),
                           Ct[r * ldc + c]);
            }
          }
        } else {
          for (int e = tid; e < BM * BN; e += NT) {
            const int r = e % BM, c = e / BM, m = m0 + r, n = n0 + c;
            if (m >= M || n >= a.N || n < nq + nk) continue;
            const int t = n - nq - nk;
            store_val<T>(a.vt_cache, a.vt_cache_lo,
                         vt_index(m / rs.nR, rs.start + m % rs.nR, t >> hs, t & (hd - 1)),
                         Ct[r * ldc + c]);
          }
        }
      }
    } break;
    case EPI_SWIGLU: {
      const int half = BN / 2;
      const int f0 = (n0 / BN) * half;
      if (!a.act_f32 && a.ld_act % 4 == 0 && a.n_half % 4 == 0) {
        // 4 consecutive outputs per thread (one 8-byte store per plane; f and ld_act are
        // multiples of 4, so in the panel-packed layout too they are adjacent)
        constexpr int H4 = BN / 8;
        for (int e = tid; e < BM * H4; e += NT) {
          const int r = e / H4, c = (e % H4) * 4, m = m0 + r, f = f0 + c;
          if (m >= M || f >= a.n_half) continue;
          const float4 g = *(const float4 *)(Ct + r * ldc + c);
          const float4 u = *(const float4 *)(Ct + r * ldc + c + half);
          const float y[4] = {silu_f(g.x) * u.x, silu_f(g.y) * u.y, silu_f(g.z) * u.z, silu_f(g.w) * u.w};
          const size_t o = a.act_packed ? pa_off(m, f, a.ld_act) : (size_t)m * a.ld_act + f;
          store_val4<bf16>(a.act_hi, a.act_lo, o, y);
        }
        break;
      }
      for (int e = tid; e < BM * half; e += NT) {
        const int r = e / half, c = e % half, m = m0 + r, f = f0 + c;
        if (m >= M || f >= a.n_half) continue;
        const float y = silu_f(Ct[r * ldc + c]) * Ct[r * ldc + c + half];
        const size_t o = a.act_packed ? pa_off(m, f, a.ld_act) : (size_t)m * a.ld_act + f;
        if (a.act_f32) {
          a.act_f32[o] = y;
        } else {
          bf16 hi, lo;
          split_hilo(y, hi, lo);
          a.act_hi[o] = hi;
          a.act_lo[o] = lo;
        }
      }
    } break;
    case EPI_LMHEAD: {
      const int lane = tid & 63, wave = tid >> 6;
      for (int r = wave; r < BM; r += NT / 64) {
        const int m = m0 + r;
        if (m >= M) break;
        HeadAcc acc = {-INFINITY, INT_MAX, -INFINITY};
        for (int c = lane; c < BN; c += 64) {
          const int v = n0 + c;
          if (v >= a.vocab || v == a.mask_id) continue;
          HeadAcc x = {a.scale * Ct[r * ldc + c], v, -INFINITY};
          acc = head_merge(acc, x);
        }
        for (int off = 32; off > 0; off >>= 1) {
          HeadAcc o;
          o.m1 = __shfl_xor(acc.m1, off, 64);
          o.idx = __shfl_xor(acc.idx, off, 64);
          o.m2 = __shfl_xor(acc.m2, off, 64);
          acc = head_merge(acc, o);
        }
        float z = 0.f;
        if (acc.m1 > -INFINITY) {
          for (int c = lane; c < BN; c += 64) {
            const int v = n0 + c;
            if (v >= a.vocab || v == a.mask_id) continue;
            z += __expf(a.scale * Ct[r * ldc + c] - acc.m1);
          }
        }
        for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off, 64);
        if (lane == 0) {
          HeadPart hp;
          hp.m1 = acc.m1; hp.idx = acc.idx; hp.m2 = acc.m2; hp.z = z;
          a.head_part[(size_t)m * a.n_vtiles + n0 / BN] = hp;
        }
      }
    } break;
  }
}

// Split-K: each split writes its tile to partial[split][M][N - n_tail0]; a reduce kernel sums
// the splits in split order (deterministic) and runs the epilogue.  No cross-workgroup fence: on
// a multi-XCD GPU an agent-scope release fence writes back the XCD's L2, which costs far more
// than the separate launch.
template <int BM, int BN>
__device__ void write_partial(const GemmArgs &a, int split, const float *Ct, int ldc, int m0,
                              int n0, int tid) {  // tid: 0..NT-1
  const int ld = a.N - a.n_tail0;
  float *P = a.partial + (size_t)split * a.M * ld - a.n_tail0;
  if (ld % 4 == 0) {
    // 4 consecutive columns per access (n0, ldc and, with ld, N are multiples of 4)
    constexpr int C4 = BN / 4;
    for (int e = tid; e < BM * C4; e += NT) {
      const int r = e / C4, c = (e % C4) * 4, m = m0 + r, n = n0 + c;
      if (m < a.M && n < a.N)
        *(float4 *)(P + (size_t)m * ld + n) = *(const float4 *)(Ct + r * ldc + c);
    }
    return;
  }
  for (int e = tid; e < BM * BN; e += NT) {
    const int r = e / BN, c = e % BN, m = m0 + r, n = n0 + c;
    if (m < a.M && n < a.N) P[(size_t)m * ld + n] = Ct[r * ldc + c];
  }
}

static constexpr int RD_BM = 8, RD_BN = 128;

// Tile reduce for the epilogues that need a whole tile (rotary pairs, gate/up halves, lm_head
// softmax partials): 8 x 128 tiles of the columns from n_tail0 on, 4 consecutive columns per
// thread.
__global__ __launch_bounds__(NT) void gemm_reduce_kernel(const GemmArgs a, int splits) {
  constexpr int LDC = RD_BN + 4;
  __shared__ float Ct[RD_BM * LDC];
  const int m0 = blockIdx.y * RD_BM, n0 = a.n_tail0 + blockIdx.x * RD_BN;
  const int ld = a.N - a.n_tail0;
  const size_t MN = (size_t)a.M * ld;
  const int r = threadIdx.x / (RD_BN / 4), c = (threadIdx.x % (RD_BN / 4)) * 4;
  const int m = m0 + r, n = n0 + c;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  if (m < a.M && n + 3 < a.N && ld % 4 == 0) {  // whole, 16-byte aligned column groups
    const float *p = a.partial + (size_t)m * ld + (n - a.n_tail0);
    for (int z = 0; z < splits; ++z) {
      const float4 v = *(const float4 *)(p + z * MN);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
  } else if (m < a.M && n < a.N) {  // a width that is not a multiple of 4 (a vocabulary)
    const float *p = a.partial + (size_t)m * ld + (n - a.n_tail0);
    float t[4] = {0.f, 0.f, 0.f, 0.f};
    for (int z = 0; z < splits; ++z)
      for (int q = 0; q < 4 && n + q < a.N; ++q) t[q] += p[z * MN + q];
    s = make_float4(t[0], t[1], t[2], t[3]);
  }
  *(float4 *)(Ct + r * LDC + c) = s;
  __syncthreads();
  run_epilogue<bf16, RD_BM, RD_BN>(a, Ct, LDC, m0, n0, threadIdx.x);
}

// ---------------------------------------------------------------------------------------------
// Tile t -> (M tile, N tile).  The M tiles form groups of GM rows, taken one after another, so
// the workgroups resident at one time share a few A row blocks (a refresh of many batch rows has
// far more A than the caches hold).  Inside a group, the first c8 columns (a multiple of 8) are
// placed XCD by XCD: workgroup t runs on XCD t % 8 and takes the tiles of columns t % 8,
// t % 8 + 8, ... with the group's M tiles in order, so each W panel is fetched into one XCD's L2;
// the remaining columns follow one after another, M tile index fastest.  Every group's first
// tile index is a multiple of 8 (GM is).  With split tiles (a single group) c8 counts only whole
// columns, so the split columns keep the plain M-fastest order of launch_gemm's plan.
__device__ inline void tile_coords(int t, int mt, int nt, int gm, int c8, int &tm, int &tn) {
  const int g = t / (gm * nt), r = t - g * gm * nt;
  const int rows = min(gm, mt - g * gm);
  if (r < c8 * rows) {
    const int k = r >> 3;
    tn = (r & 7) + 8 * (k / rows);
    tm = g * gm + k % rows;
  } else {
    const int r2 = r - c8 * rows;
    tn = c8 + r2 / rows;
    tm = g * gm + r2 % rows;
  }
}
static constexpr int TILED_GM = 16, BIG_GM = 8;

// Tiled bf16 MFMA kernel for many rows (block refresh).  4 waves as WM x WN; each wave owns
// (BM/WM) x (BN/WN) of the tile in 32x32 blocks (v_mfma_f32_32x32x16_bf16).  BK = 64.
template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(NT) void gemm_mfma_kernel(const GemmArgs a) {
  constexpr int BK = 64, LDK = BK + 8;  // row pitch in bf16 elements (pad 16 B)
  constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
  constexpr int LDC = BN + 4;
  constexpr int STAGE_BYTES = (2 * BM + BN) * LDK * 2;
  constexpr int CT_BYTES = BM * LDC * 4;
  constexpr int SMEM = STAGE_BYTES > CT_BYTES ? STAGE_BYTES : CT_BYTES;
  __shared__ __align__(16) unsigned char smem[SMEM];
  uint16_t *As_hi = (uint16_t *)smem;
  uint16_t *As_lo = As_hi + BM * LDK;
  uint16_t *Ws = As_lo + BM * LDK;
  float *Ct = (float *)smem;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  // work item -> tile (tile_coords; split tiles only occur with a single group of rows, where a
  // split covers whole columns and every row of a column is summed in the same order) and K range
  const int mt = (a.M + BM - 1) / BM;
  const int w = blockIdx.x;
  int tile = w, split = -1, kbeg = 0, kend = a.K;
  if (w >= a.n_full) {
    const int j = w - a.n_full;
    tile = a.n_full + j / a.tail_sp;
    split = j % a.tail_sp;
    kbeg = split * a.k_split;
    kend = min(a.K, kbeg + a.k_split);
    if (a.tail_sp == 1) split = -1;
  }
  int tm, tn;
  tile_coords(tile, mt, (a.N + BN - 1) / BN, TILED_GM, a.xcd_cols, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // Global -> register staging: 16-byte chunks, 8 per 64-wide row.  Native vector types: arrays
  // of HIP's uint4 struct defeat register promotion and end up in scratch memory.
  constexpr int A_CH = BM * BK / 8 / NT;
  constexpr int W_CH = BN * BK / 8 / NT;
  static_assert(A_CH >= 1 && W_CH >= 1, "tile too small");
  s16x8 ra_hi[A_CH], ra_lo[A_CH], rw[W_CH];
  static_assert(BN == PW_ROWS && BK == 2 * PW_K, "one panel, two blocks per K step");
  // packed W: chunk (row r, column c8) of K step k0 is in block k0/32 + c8/32 of panel n0/128
  const uint16_t *wrow[W_CH];
#pragma unroll
  for (int i = 0; i < W_CH; ++i) {
    const int ch = tid + i * NT, r = ch / 8, c8 = (ch % 8) * 8;
    wrow[i] = wp_block(a, n0 / PW_ROWS, c8 / PW_K) + r * PW_K + c8 % PW_K;
  }
  // A row offsets, hoisted out of the K loop (rows past M read row M-1; they only feed output
  // rows that are never written)
  size_t aoff[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int ch = tid + i * NT, r = ch / 8, c8 = (ch % 8) * 8;
    aoff[i] = (size_t)a_row(a, min(m0 + r, a.M - 1)) * a.lda + c8;
  }

  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      ra_hi[i] = *(const s16x8 *)((const uint16_t *)a.a_hi + aoff[i] + k0);
      ra_lo[i] = *(const s16x8 *)((const uint16_t *)a.a_lo + aoff[i] + k0);
    }
#pragma unroll
    for (int i = 0; i < W_CH; ++i) rw[i] = *(const s16x8 *)(wrow[i] + (size_t)(k0 / PW_K) * (PW_ROWS * PW_K));
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int ch = tid + i * NT, r = ch / 8, c8 = (ch % 8) * 8;
      *(s16x8 *)(As_hi + r * LDK + c8) = ra_hi[i];
      *(s16x8 *)(As_lo + r * LDK + c8) = ra_lo[i];
    }
#pragma unroll
    for (int i = 0; i < W_CH; ++i) {
      const int ch = tid + i * NT, r = ch / 8, c8 = (ch % 8) * 8;
      *(s16x8 *)(Ws + r * LDK + c8) = rw[i];
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int frow = lane & 31, fk = (lane >> 5) * 8;
  // Loads are unconditional (the last iteration re-reads its own tile, unused) so the staging
  // registers stay in registers and the wait counts stay static.
  load(kbeg);
  for (int k0 = kbeg; k0 < kend; k0 += BK) {
    __syncthreads();
    store();
    __syncthreads();
    load(min(k0 + BK, kend - BK));
    // keep the next tile's loads ahead of the MFMAs (the scheduler would sink them to the store)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8_t fa_hi[TM], fa_lo[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * (BM / WM) + i * 32 + frow;
        fa_hi[i] = *(const bf16x8_t *)(As_hi + r * LDK + kk * 16 + fk);
        fa_lo[i] = *(const bf16x8_t *)(As_lo + r * LDK + kk * 16 + fk);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = wn * (BN / WN) + j * 32 + frow;
        fb[j] = *(const bf16x8_t *)(Ws + r * LDK + kk * 16 + fk);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa_hi[i], fb[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa_lo[i], fb[j], acc[i][j], 0, 0, 0);
        }
    }
  }
  __syncthreads();
  // Accumulators -> C tile.  32x32 block layout: lane l, reg r -> row 8*(r/4) + 4*(l/32) + r%4,
  // column l%32.
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * (BM / WM) + i * 32 + 8 * (r / 4) + 4 * (lane >> 5) + (r & 3);
        const int col = wn * (BN / WN) + j * 32 + (lane & 31);
        Ct[row * LDC + col] = acc[i][j][r];
      }
  __syncthreads();
  if (split >= 0) {
    write_partial<BM, BN>(a, split, Ct, LDC, m0, n0, tid);
    return;
  }
  run_epilogue<bf16, BM, BN>(a, Ct, LDC, m0, n0, tid);
}

// ---------------------------------------------------------------------------------------------
// Large-tile bf16 MFMA kernels for many rows (block refreshes, and the cached steps of large
// batches).  A workgroup of NWV waves owns a (32 NWV) x BNT tile; wave w owns its rows
// 32 w .. 32 w + 31 across all BNT columns, as 1 x (BNT / 32) blocks of
// v_mfma_f32_32x32x16_bf16.  Two shapes: 256 x 256 (8 waves, two per SIMD, 128 accumulator
// registers each) and 384 x 128 (12 waves, three per SIMD, 64 accumulators each), which tiles
// a 768-row refresh projection of 12288 or 4096 columns into 192 or 64 tiles (whole rounds of the
// XCDs' CUs with or without a K split) where 256 x 256 tiles leave a partly filled round.
// K advances in stages of 32.
//   A (hi and lo planes) goes straight from global memory into the MFMA operand registers: each
//     lane loads its row's 8 k of a 16-k step, one stage ahead of use (a ring of 2 stages in
//     registers).  No wave shares A rows with another, so every A element is loaded once.
//   W is staged in LDS (a ring of 4 slots of [BNT rows][32 k]), written by the waves themselves
//     from registers (loaded a stage and a half ahead), and read as BNT / 32 fragments per 16-k
//     step.  A slot is BNT / 16 loads of 1 KB (64 lanes x 16 bytes); with more waves than that
//     the extra waves load and write a copy of another wave's part (the same bytes to the same
//     place), so every wave runs the same unconditional code.
// Why: with A and W both staged through LDS (by global_load_lds), the LDS took 48 KB of writes
// and 128 KB of fragment reads per stage, and the writes of the tile loads stalled the fragment
// reads feeding the MFMAs (measured: the same loads into registers cost ~3 %, into LDS ~19 %).
// Now LDS carries 16 KB of W writes and 128 KB of W reads per stage, and 1.1-1.2x the MFMA rate
// (long-context gate/up 1.29 -> 1.41 PFLOP/s executed, 768-row down 1.02 -> 1.25).  Plain
// register loads rather than global_load_lds for W as well: with both kinds in flight the
// compiler cannot count them in order and waits for every load at the top of each stage.
// In a W slot, row r's 16-byte chunk c sits at chunk position 4 r + (c ^ ((r >> 2) & 3)), so the
// fragment reads of 16 consecutive rows cover all 64 banks once (conflict-free).
static constexpr int BG_BK = 32, BG_NSW = 4;

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediate: vmcnt vm (6 bits), lgkmcnt lgkm (4 bits), expcnt not waited on
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8);
}

template <int NWV, int BNT>
__global__ __launch_bounds__(64 * NWV, 1) void gemm_big_kernel(const GemmArgs a) {
  constexpr int BMT = 32 * NWV;            // tile rows
  constexpr int WST = BNT * BG_BK * 2;     // one W slot
  constexpr int WLOADS = BNT / 16;         // 1 KB loads per W slot
  constexpr int WL = (WLOADS + NWV - 1) / NWV;  // per wave
  constexpr int LDC = 128 + 4;             // epilogue: 128 x 128 pieces of fp32, two at a time
  constexpr int EPI = 2 * 128 * LDC * 4;
  constexpr int SMEM = BG_NSW * WST > EPI ? BG_NSW * WST : EPI;
  constexpr int NB = BNT / 32;             // 32-column blocks of a wave
  constexpr int NPC = BNT / 128;           // 128-column pieces of a 128-row group
  static_assert(BNT % 128 == 0 && BMT % 128 == 0 && 64 * NWV >= 2 * NT, "epilogue pieces");
  __shared__ __align__(1024) unsigned char smem[SMEM];
  float *Ct = (float *)smem;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // work item -> tile (tile_coords; split tiles only occur with a single group of rows, where a
  // split covers whole columns and every row of a column is summed in the same order) and K range
  const int mt = (a.M + BMT - 1) / BMT;
  const int w = blockIdx.x;
  int tile = w, split = -1, kbeg = 0, kend = a.K;
  if (w >= a.n_full) {
    const int j = w - a.n_full;
    tile = a.n_full + j / a.tail_sp;
    split = j % a.tail_sp;
    kbeg = split * a.k_split;
    kend = min(a.K, kbeg + a.k_split);
    if (a.tail_sp == 1) split = -1;
  }
  int tm, tn;
  tile_coords(tile, mt, (a.N + BNT - 1) / BNT, BIG_GM, a.xcd_cols, tm, tn);
  const int m0 = tm * BMT, n0 = tn * BNT;
  const int T = (kend - kbeg) / BG_BK;  // even: K ranges are multiples of 64

  // W: load j of this wave fills 1 KB block (wave * WL + j) % WLOADS of a slot; its lane's chunk
  // position there is pos = block * 64 + lane: row r = pos >> 2, source chunk (pos & 3) ^
  // ((r >> 2) & 3).  Panels past the last one read the last one (their outputs are never
  // written).
  const int last_panel = (a.N + PW_ROWS - 1) / PW_ROWS - 1;
  const uint16_t *wsrc[WL];
  int wdst[WL];
#pragma unroll
  for (int j = 0; j < WL; ++j) {
    const int blk = (wave * WL + j) % WLOADS;
    const int pos = blk * 64 + lane, r = pos >> 2, c = (pos & 3) ^ ((r >> 2) & 3);
    wsrc[j] = wp_block(a, min(n0 / PW_ROWS + (r >> 7), last_panel), 0) + (r & 127) * PW_K + c * 8;
    wdst[j] = blk * 1024 + lane * 16;
  }
  s16x8 wreg[2][WL];
  auto load_w_to = [&](s16x8 *dst, int t) {  // stage t (past the last: the last again, unused)
    const size_t kw = (size_t)((kbeg + min(t, T - 1) * BG_BK) / PW_K) * (PW_ROWS * PW_K);
#pragma unroll
    for (int j = 0; j < WL; ++j) dst[j] = *(const s16x8 *)(wsrc[j] + kw);
  };
  auto write_w_from = [&](const s16x8 *src, int t) {
    unsigned char *st = smem + (t % BG_NSW) * WST;
#pragma unroll
    for (int j = 0; j < WL; ++j) *(s16x8 *)(st + wdst[j]) = src[j];
  };
  auto load_w = [&](int b, int t) { load_w_to(wreg[b], t); };
  auto write_w = [&](int b, int t) { write_w_from(wreg[b], t); };
  // A: lane l reads row (l & 31) of the wave's 32 rows, 8 k at 8 (l >> 5) of each 16-k step.
  // Rows past M read row M - 1 (their outputs are never written).
  const int frow = lane & 31, fhalf = lane >> 5;
  const size_t row = a_row(a, min(m0 + wave * 32 + frow, a.M - 1));
  const size_t aoff = a.a_packed ? pa_off(row, kbeg + fhalf * 8, a.K) : row * a.lda + kbeg + fhalf * 8;
  const size_t astep = a.a_packed ? (size_t)(PW_ROWS * PW_K) : (size_t)BG_BK;  // per stage
  const uint16_t *ahi = (const uint16_t *)a.a_hi + aoff, *alo = (const uint16_t *)a.a_lo + aoff;
  bf16x8_t ar[2][2][2];  // [ring][plane][16-k step]
  auto load_a = [&](int b, int t) {
    const size_t ks = (size_t)min(t, T - 1) * astep;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      ar[b][0][kk] = *(const bf16x8_t *)(ahi + ks + kk * 16);
      ar[b][1][kk] = *(const bf16x8_t *)(alo + ks + kk * 16);
    }
  };
  // W fragments: row j * 32 + (l & 31) of the slot, chunk kk * 2 + (l >> 5); double-buffered
  const int fsw = (frow >> 2) & 3, wrow = frow * 64;
  bf16x8_t fb[2][NB];
  auto read_w = [&](int t, int kk, int buf) {
    const unsigned char *st = smem + (t % BG_NSW) * WST;
    const int cb = ((kk * 2 + fhalf) ^ fsw) * 16;
#pragma unroll
    for (int j = 0; j < NB; ++j) fb[buf][j] = *(const bf16x8_t *)(st + wrow + j * 2048 + cb);
  };
  f32x16 acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  auto mfmas = [&](int b, int kk, int fbuf) {
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ar[b][0][kk], fb[fbuf][j], acc[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ar[b][1][kk], fb[fbuf][j], acc[j], 0, 0, 0);
  };
  auto barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // Prologue: A(0) into ar[0], W(0..3) into the ring (all of them loaded before the first is
  // written: one memory round trip), W(4) into wreg[0].
  load_a(0, 0);
  {
    s16x8 wpre[2][WL];
    load_w(0, 0);
    load_w(1, 1);
    load_w_to(wpre[0], 2);
    load_w_to(wpre[1], 3);
    write_w(0, 0);
    write_w(1, 1);
    write_w_from(wpre[0], 2);
    write_w_from(wpre[1], 3);
  }
  load_w(0, 4);
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));  // this wave's ring writes are done
  barrier();
  read_w(0, 0, 0);
  // Stage u (b = u & 1): A(u) is in ar[b] and W(u + 4) in wreg[b], both loaded in stage u - 1.
  // The stage starts the loads of A(u + 1) and W(u + 5) (kept ahead of the MFMAs), runs the
  // first 16-k step, waits at a barrier until every wave has read both steps of W(u), writes
  // W(u + 4) into W(u)'s slot and runs the second step.  W(u + 1) was written three stages
  // earlier.  Past the last stage the loads repeat it (unused), so every stage is alike.
  auto stage = [&](int b, int u) {
    load_a(b ^ 1, u + 1);
    load_w(b ^ 1, u + 5);
    __builtin_amdgcn_sched_barrier(0);
    read_w(u, 1, 1);
    mfmas(b, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));  // this wave's LDS reads and writes are done
    barrier();
    write_w(b, u + 4);
    read_w(min(u + 1, T - 1), 0, 0);
    mfmas(b, 1, 1);
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int t0 = 0; t0 < T; t0 += 2) {
    stage(0, t0);
    stage(1, t0 + 1);
  }
  __syncthreads();
  // Epilogue in 128 x 128 pieces, two at a time: piece (g, c) is rows 128 g.., columns 128 c..
  // of the tile, numbered g * NPC + c.  In pass p the waves holding rows of pieces 2p and 2p + 1
  // write them into C tiles 0 and 1, then threads [q NT, (q + 1) NT) run the epilogue of piece
  // 2p + q (with 256 x 256 tiles: both pieces of a 128-row half, every thread working).
  constexpr int NPIECE = BMT / 128 * NPC;
#pragma unroll
  for (int pass = 0; pass < (NPIECE + 1) / 2; ++pass) {
    const int g = wave / 4;  // this wave's 128-row group
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int slot = g * NPC + (j >> 2) - 2 * pass;
      if (slot == 0 || slot == 1) {
        float *Cq = Ct + slot * (128 * LDC);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = (wave & 3) * 32 + 8 * (r / 4) + 4 * fhalf + (r & 3);
          Cq[row * LDC + (j & 3) * 32 + frow] = acc[j][r];
        }
      }
    }
    __syncthreads();
    const int q = tid / NT, et = tid % NT, pc = 2 * pass + q;
    if (q < 2 && pc < NPIECE) {
      const float *Cq = Ct + q * (128 * LDC);
      const int pm = m0 + (pc / NPC) * 128, pn = n0 + (pc % NPC) * 128;
      if (split >= 0)
        write_partial<128, 128>(a, split, Cq, LDC, pm, pn, et);
      else
        run_epilogue<bf16, 128, 128>(a, Cq, LDC, pm, pn, et);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------------
// Weight-streaming bf16 kernel for few rows (M <= 16*MT <= 64): the shape of a cached step, where
// the time is the HBM read of W.  4 waves x 32 W rows = 128 columns per workgroup.
//   W: each lane loads straight into the B-operand registers of v_mfma_f32_16x16x32_bf16 (lane:
//      row l%16 of a 16-row block, 8 consecutive k at 8*(l/16) of each 32-wide k step; 4 lanes
//      read 64 contiguous bytes of a row), through a ring of SK_D chunks of 64 k.
//   A: shared by the 4 waves through LDS, one stage of SK_KA k at a time; the next stage is
//      loaded into registers while the current one is consumed.
// Every load is issued unconditionally and no loaded value is selected on, so the wait counts
// are static and the W ring is only waited on one stage at a time.  Out-of-range addresses are
// clamped instead: a W row past N or an A row past M only feeds output columns or rows that the
// epilogue never writes, and the K range of a workgroup is a whole number of stages (K and the
// split length are multiples of SK_KA).
static constexpr int SK_BN = 128, SK_KA = 256, SK_D = SK_KA / 64;

// NS > 0: the workgroup's K range is exactly NS stages and the stage loop is unrolled, which
// lets the compiler count the loads in flight exactly (with a loop it drains every load at the
// top of each stage); NS = 0: any number of stages.
template <int MT, int NS>
__global__ __launch_bounds__(NT) void gemm_skinny_kernel(const GemmArgs a) {
  constexpr int BM = 16 * MT;
  constexpr int LDA = SK_KA + 8;
  constexpr int LDC = SK_BN + 4;
  constexpr int A_BYTES = 2 * BM * LDA * 2, C_BYTES = BM * LDC * 4;
  constexpr int SMEM = A_BYTES > C_BYTES ? A_BYTES : C_BYTES;
  constexpr int ACH = BM * SK_KA / 8 / NT;  // 16-byte A chunks per thread per stage (hi and lo each)
  static_assert(ACH >= 1, "stage too small");
  __shared__ __align__(16) unsigned char smem[SMEM];
  uint16_t *Ah = (uint16_t *)smem;
  uint16_t *Al = Ah + BM * LDA;
  float *Ct = (float *)smem;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rn = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * SK_BN;
  const int kbeg = blockIdx.z * a.k_split;
  const int kend = min(a.K, kbeg + a.k_split);
  const int nchunk = (kend - kbeg) / 64;
  const int nstage = NS > 0 ? NS : (nchunk + SK_D - 1) / SK_D;

  // W rows of this lane in the packed panel n0/128 (rows past N are zero-padded)
  static_assert(SK_BN == PW_ROWS, "one panel per workgroup");
  const uint16_t *wr[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) wr[cb] = wp_block(a, n0 / PW_ROWS, 0) + (wave * 32 + cb * 16 + rn) * PW_K + 8 * g;
  s16x8 wb[SK_D][2][2];
  auto load_w = [&](int slot, int c) {
    const int kb = (kbeg + min(c, nchunk - 1) * 64) / PW_K;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        wb[slot][cb][ks] = *(const s16x8 *)(wr[cb] + (size_t)(kb + ks) * (PW_ROWS * PW_K));
  };
  // A stage prefetch: chunk e of the stage -> row e / (SK_KA/8), column 8 * (e % (SK_KA/8))
  s16x8 rah[ACH], ral[ACH];
  size_t aoff[ACH];  // row offsets, hoisted out of the stage loop
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    const int e = tid + i * NT, r = e / (SK_KA / 8), c8 = (e % (SK_KA / 8)) * 8;
    aoff[i] = (size_t)a_row(a, min(r, a.M - 1)) * a.lda + kbeg + c8;
  }
  auto load_a = [&](int st) {
    const int k = min(st, nstage - 1) * SK_KA;
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      rah[i] = *(const s16x8 *)((const uint16_t *)a.a_hi + aoff[i] + k);
      ral[i] = *(const s16x8 *)((const uint16_t *)a.a_lo + aoff[i] + k);
    }
  };
  auto store_a = [&]() {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int e = tid + i * NT, r = e / (SK_KA / 8), c8 = (e % (SK_KA / 8)) * 8;
      *(s16x8 *)(Ah + r * LDA + c8) = rah[i];
      *(s16x8 *)(Al + r * LDA + c8) = ral[i];
    }
  };

  f32x4 acc[MT][2];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  load_a(0);
#pragma unroll
  for (int sl = 0; sl < SK_D; ++sl) load_w(sl, sl);
  constexpr int UNROLL = NS > 0 ? NS : 1;
#pragma unroll UNROLL
  for (int st = 0; st < nstage; ++st) {
    store_a();
    __syncthreads();
    load_a(st + 1);  // past the last stage this re-reads a clamped address; the values go unused
#pragma unroll
    for (int sl = 0; sl < SK_D; ++sl) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          const int row = i * 16 + rn, col = sl * 64 + 32 * ks + 8 * g;
          const bf16x8_t fh = *(const bf16x8_t *)(Ah + row * LDA + col);
          const bf16x8_t fl = *(const bf16x8_t *)(Al + row * LDA + col);
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) {
            const bf16x8_t w8 = (bf16x8_t)wb[sl][cb][ks];
            acc[i][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fh, w8, acc[i][cb], 0, 0, 0);
            acc[i][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fl, w8, acc[i][cb], 0, 0, 0);
          }
        }
      }
      load_w(sl, (st + 1) * SK_D + sl);
    }
    __syncthreads();
  }
  // 16x16 block layout: lane l, reg r -> row 4*(l/16) + r, column l%16.
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        Ct[(i * 16 + 4 * g + r) * LDC + wave * 32 + cb * 16 + rn] = acc[i][cb][r];
  __syncthreads();
  if (gridDim.z > 1) {
    write_partial<BM, SK_BN>(a, blockIdx.z, Ct, LDC, 0, n0, tid);
    return;
  }
  run_epilogue<bf16, BM, SK_BN>(a, Ct, LDC, 0, n0, tid);
}

// ---------------------------------------------------------------------------------------------
// fp32 SIMT kernel for the fp32 workloads (small models): 64 x 64 tile, 4 x 4 per thread.
__global__ __launch_bounds__(NT) void gemm_f32_kernel(const GemmArgs a) {
  constexpr int BM = 64, BN = 64, BK = 16, LDC = BN + 4;
  __shared__ float As[BK][BM + 1];
  __shared__ float Ws[BK][BN + 1];
  __shared__ float Ct[BM * LDC];
  const int tid = threadIdx.x;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int tr = tid / 16, tc = tid % 16;
  float acc[4][4] = {};
  const float *wr[4];
  for (int i = 0; i < 4; ++i) {
    const int e = tid + i * NT;  // 1024 elements of a 64x16 tile: row e/16, k e%16
    wr[i] = w_row<float>(a, BN, n0, e / 16);
  }
  for (int k0 = 0; k0 < a.K; k0 += BK) {
    for (int i = 0; i < 4; ++i) {
      const int e = tid + i * NT, r = e / 16, kk = e % 16, m = m0 + r, k = k0 + kk;
      As[kk][r] = (m < a.M && k < a.K) ? a.a_f32[(size_t)a_row(a, m) * a.lda + k] : 0.f;
      Ws[kk][r] = (wr[i] && k < a.K) ? wr[i][k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float av[4], wv[4];
      for (int i = 0; i < 4; ++i) av[i] = As[kk][tr * 4 + i];
      for (int j = 0; j < 4; ++j) wv[j] = Ws[kk][tc * 4 + j];
      for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], wv[j], acc[i][j]);
    }
    __syncthreads();
  }
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) Ct[(tr * 4 + i) * LDC + tc * 4 + j] = acc[i][j];
  __syncthreads();
  run_epilogue<float, BM, BN>(a, Ct, LDC, m0, n0, tid);
}

// ---------------------------------------------------------------------------------------------
int gemm_bn(int M, int dtype) { return dtype == 0 ? 64 : 128; }

// The skinny kernel serves M <= 64 (16-row blocks) when K is a whole number of its 256-wide
// stages; otherwise 128 x 128 tiles.
static bool use_skinny(int M, int K) { return M <= 64 && K % SK_KA == 0; }

static int bm_for(int M, int K) { return use_skinny(M, K) ? 16 * ((M + 15) / 16) : 128; }

// Kernel and split-K plan.
//   Skinny kernel (M <= 64): the fewest power-of-two splits (every tile split alike) that give
//   at least 192 workgroups, with whole stages per split; if K has too few factors of two, as
//   many stage-aligned splits as reach 192 workgroups (or one stage each).
//   Tiled (128 x 128) and large-tile (256 x 256, 384 x 128) kernels: the first n_full work items
//   are whole tiles (whole columns of M tiles) and the remaining columns are split tail_sp ways,
//   so that the last, partly filled round of resident workgroups is spread over the whole GPU.
//   The plan minimises an estimate of the time: the work items, in launch order, placed on the
//   32 CUs of the XCD each one runs on (gpu_makespan), plus the round trip of the fp32 partial
//   tiles (written here, read by the reduce) at ~6 TB/s and ~4 us for the reduce launch.  Fitted
//   on MI355X to the 8B-shape projections at 768 rows: a 128 x 128 workgroup takes 1.25 us per K
//   step of 64 alone on its CU and 1.98 us when two share it (they are limited by the CU, not by
//   latency); a 256 x 256 workgroup (one per CU) 3.0 us, a 384 x 128 one 2.4 us.
enum GemmKind { GK_F32 = 0, GK_SKINNY = 1, GK_TILED = 2, GK_BIG = 3, GK_BIG384 = 4 };

struct SplitPlan {
  int kind;     // GemmKind
  int splits;   // skinny: gridDim.z; tiled / large-tile: tail_sp
  int kc;       // K per split
  int n_full;   // tiled / large-tile: whole-tile work items
  int n_tail0;  // first split column
};

// Estimated time (us) of n_full items of it_full K steps followed by n_tail items of it_tail
// steps on `cus` CUs holding up to per_cu workgroups each.  Items are handed out in launch order
// to the least occupied CUs (round-robin at the start).  A workgroup alone on its CU takes t1 us
// per K step, each of two sharing a CU t2.
static double cu_makespan(long n_full, int it_full, long n_tail, int it_tail, int cus, int per_cu,
                          double t1, double t2) {
  struct Cu { double last; int n; double rem[2]; int ver; };
  std::vector<Cu> cu(cus, Cu{0.0, 0, {0.0, 0.0}, 0});
  const long total = n_full + n_tail;
  long next = 0;
  auto step_time = [&](const Cu &u) { return u.n == 1 ? t1 : t2; };
  auto advance = [&](Cu &u, double T) {  // progress to time T, drop finished items
    if (u.n) {
      const double done = (T - u.last) / step_time(u);
      int k = 0;
      for (int i = 0; i < u.n; ++i)
        if (u.rem[i] - done > 1e-9) u.rem[k++] = u.rem[i] - done;
      u.n = k;
    }
    u.last = T;
  };
  typedef std::pair<double, int> Ev;
  std::priority_queue<Ev, std::vector<Ev>, std::greater<Ev>> q;
  std::vector<int> qver(cus, -1);
  auto schedule = [&](int c) {
    Cu &u = cu[c];
    ++u.ver;
    if (!u.n) return;
    double m = u.rem[0];
    for (int i = 1; i < u.n; ++i) m = std::min(m, u.rem[i]);
    q.push(Ev(u.last + m * step_time(u), c * 4096 + (u.ver & 4095)));
  };
  auto dispatch = [&](double T) {
    for (int want = 0; want < per_cu && next < total; ++want)
      for (int c = 0; c < cus && next < total; ++c) {
        Cu &u = cu[c];
        if (u.n != want) continue;
        advance(u, T);
        if (u.n != want) continue;
        u.rem[u.n++] = next < n_full ? it_full : it_tail;
        ++next;
        schedule(c);
      }
  };
  dispatch(0.0);
  double end = 0.0;
  while (!q.empty()) {
    const double T = q.top().first;
    while (!q.empty() && q.top().first <= T + 1e-9) {
      const int c = q.top().second / 4096, v = q.top().second % 4096;
      q.pop();
      if (v != (cu[c].ver & 4095)) continue;  // superseded
      advance(cu[c], T);
      schedule(c);
    }
    end = std::max(end, T);
    dispatch(T);
  }
  return end;
}

// The same over the whole GPU: workgroup i of a launch runs on XCD i % 8, and each XCD hands its
// own workgroups, in launch order, to its 32 CUs, so the XCDs are scheduled independently and the
// launch ends with the slowest.  (A single queue over 256 CUs would let an XCD with idle CUs take
// another XCD's items: the 768-row gate/up plan then looked balanced, while the XCDs holding a
// 33rd tail item each ran a third round of them: 284 us in place of ~256, measured per workgroup.)
static double gpu_makespan(long n_full, int it_full, long n_tail, int it_tail, int per_cu,
                           double t1, double t2) {
  auto count = [](long n, int x) { return n > x ? (n - x + 7) / 8 : 0L; };  // i < n, i % 8 == x
  double end = 0.0;
  for (int x = 0; x < 8; ++x) {
    const long nf = count(n_full, x), nt = count(n_full + n_tail, x) - nf;
    end = std::max(end, cu_makespan(nf, it_full, nt, it_tail, 32, per_cu, t1, t2));
  }
  return end;
}

// Tile rows and columns of the tiled and large-tile kernels.
static int tile_bm(int kind) { return kind == GK_BIG ? 256 : kind == GK_BIG384 ? 384 : 128; }
static int tile_bn(int kind) { return kind == GK_BIG ? 256 : 128; }

static SplitPlan tile_plan(int kind, int M, int N, int K, double *cost_out) {
  const bool big = kind == GK_BIG || kind == GK_BIG384;
  const int bm = tile_bm(kind), bn = tile_bn(kind), per_cu = big ? 1 : 2;
  const double t1 = kind == GK_BIG ? 3.0 : kind == GK_BIG384 ? 2.4 : 1.25, t2 = 1.98;
  const int mt = (M + bm - 1) / bm, nt = (N + bn - 1) / bn, iters = K / 64;
  const long tiles = (long)mt * nt;
  SplitPlan best_plan{kind, 1, K, (int)tiles, N};
  *cost_out = -1.0;  // not modelled: many rounds of tiles
  // splits need whole columns in launch order: a single group of rows (tile_coords); with many
  // rounds of tiles the tail is negligible
  if (mt > (big ? BIG_GM : TILED_GM) || tiles > 16L * 256 * per_cu) return best_plan;
  double best = 1e30;
  // candidate full-column counts: none, or whole rounds of resident workgroups
  const int cands[2] = {0, (int)((tiles / (256 * per_cu)) * (256 * per_cu) / mt)};
  for (int ci = 0; ci < 2; ++ci) {
    const int c = std::min(cands[ci], nt);
    if (ci == 1 && c == 0) continue;
    const long n_full = (long)c * mt, n_tail_tiles = tiles - n_full;
    const int max_sp = n_tail_tiles == 0 ? 1 : std::min(16, std::max(1, iters / 4));
    for (int sp = 1; sp <= max_sp; ++sp) {
      const int kc = ((K + sp - 1) / sp + 63) / 64 * 64, splits = (K + kc - 1) / kc;
      if (splits != sp) continue;
      const double span = gpu_makespan(n_full, iters, n_tail_tiles * splits, kc / 64, per_cu, t1, t2);
      const int tail_cols = N - c * bn;
      const double partial_us = splits > 1 ? splits * (double)M * tail_cols * 8.0 / 6.0e6 + 4.0 : 0.0;
      const double cost = span + partial_us;
      if (cost < best - 1e-9) {
        best = cost;
        best_plan = SplitPlan{kind, splits, kc, (int)n_full, splits > 1 ? c * bn : N};
      }
    }
  }
  if (best_plan.splits == 1) { best_plan.n_full = (int)tiles; best_plan.n_tail0 = N; }
  *cost_out = best;
  return best_plan;
}

// The tile plans are computed once per shape (the list schedule takes up to a few ms).
static SplitPlan tile_plan_cached(int kind, int M, int N, int K, double *cost_out = nullptr) {
  static std::mutex mu;
  static std::map<std::tuple<int, int, int, int>, std::pair<SplitPlan, double>> cache;
  const auto key = std::make_tuple(kind, M, N, K);
  {
    std::lock_guard<std::mutex> lk(mu);
    auto it = cache.find(key);
    if (it != cache.end()) {
      if (cost_out) *cost_out = it->second.second;
      return it->second.first;
    }
  }
  double cost;
  const SplitPlan pl = tile_plan(kind, M, N, K, &cost);
  std::lock_guard<std::mutex> lk(mu);
  cache.emplace(key, std::make_pair(pl, cost));
  if (cost_out) *cost_out = cost;
  return pl;
}

// Kernel of a GEMM: fp32 SIMT for the fp32 path; the weight-streaming kernel for up to 64 rows;
// from 512 rows a large-tile kernel: 256 x 256 tiles where there are many rounds of them, else
// whichever of the 256 x 256 and 384 x 128 tiles the plan model prices lower (at 768 rows the
// 384 x 128 tiles take q/k/v as 192 whole tiles, 161 against 167 us for 144 large tiles split 3
// ways with their reduce and 205 us for 128 x 128 tiles, and o and down split 4 ways: 49 and
// 126 us against 52 and 131 us; gate/up stays on 256 x 256 tiles, 293 against 300 us; measured
// in isolation with random data), and the 128 x 128 kernel where that plan would split every
// tile K-wise while the 128 x 128 plan runs most tiles whole; the 128 x 128 tiled kernel below
// 512 rows (at 256 and 384 rows it and the 256 x 256 kernel measured alike).
static int choose_kind(int M, int N, int K, int dtype) {
  if (dtype == 0) return GK_F32;
  if (use_skinny(M, K)) return GK_SKINNY;
  if (M < 512 || K % 64) return GK_TILED;
  double c256, c384;
  const SplitPlan p256 = tile_plan_cached(GK_BIG, M, N, K, &c256);
  if (c256 < 0) return GK_BIG;  // many rounds of tiles (not modelled): the faster tile
  const SplitPlan p384 = tile_plan_cached(GK_BIG384, M, N, K, &c384);
  const bool t384 = c384 >= 0 && c384 < c256;
  const SplitPlan &big = t384 ? p384 : p256;
  if (big.splits > 1 && big.n_full == 0 && tile_plan_cached(GK_TILED, M, N, K).n_full > 0)
    return GK_TILED;
  return t384 ? GK_BIG384 : GK_BIG;
}

static SplitPlan split_plan(int M, int N, int K, int dtype) {
  const int kind = choose_kind(M, N, K, dtype);
  SplitPlan pl{kind, 1, K, 0, 0};
  if (kind == GK_F32) return pl;
  if (kind != GK_SKINNY) return tile_plan_cached(kind, M, N, K);
  const long tiles = (N + SK_BN - 1) / SK_BN;  // one 16..64-row tile in M
  // the fewest power-of-two splits that give at least 192 workgroups (3/4 of the CUs): more
  // splits add partial traffic and, for the epilogues that need whole sums, a reduce launch
  int want = 1;
  while (tiles * want < 192 && want < 16 && K % (2 * want * SK_KA) == 0) want *= 2;
  // K not divisible that far: uneven splits of whole stages (the last one shorter)
  if (tiles * want < 192) want = (int)std::min<long>((192 + tiles - 1) / tiles, std::max(1, K / SK_KA));
  pl.kc = ((K + want - 1) / want + SK_KA - 1) / SK_KA * SK_KA;
  pl.splits = (K + pl.kc - 1) / pl.kc;
  return pl;
}

int gemm_num_splits(int M, int N, int K, int dtype) {
  const SplitPlan pl = split_plan(M, N, K, dtype);
  // tiled kernels with whole tiles first: the tail is reduced inside launch_gemm
  if (pl.kind != GK_SKINNY && pl.n_full > 0) return 1;
  return pl.splits;
}

size_t gemm_partial_bytes(int M, int N, int K, int dtype) {
  const SplitPlan pl = split_plan(M, N, K, dtype);
  if (pl.splits <= 1) return 0;
  return (size_t)pl.splits * M * (N - pl.n_tail0) * sizeof(float);
}

bool gemm_a_packed(int M, int N, int K, int dtype) {
  const int kind = choose_kind(M, N, K, dtype);
  return kind == GK_BIG || kind == GK_BIG384;
}

int gemm_kind(int M, int K, int dtype) {
  if (dtype == 0) return 0;
  return use_skinny(M, K) ? 1 : 2;
}

hipError_t launch_gemm(const GemmArgs &a0, int dtype, hipStream_t st, int *splits_out,
                       hipEvent_t ev_begin, hipEvent_t ev_end) {
  GemmArgs a = a0;
  if (splits_out) *splits_out = 1;
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  // panel-packed A only for the large-tile kernel; a packed SwiGLU output needs whole k blocks;
  // the q/k/v epilogue indexes heads with shifts
  if ((a.epi == EPI_QKV && (a.head_dim <= 0 || (a.head_dim & (a.head_dim - 1)))) ||
      (a.a_packed && !gemm_a_packed(a.M, a.N, a.K, dtype)) ||
      (a.epi == EPI_SWIGLU && a.act_packed && (dtype == 0 || a.ld_act % 32)))
    return hipErrorInvalidValue;
  hipError_t e;
  if (ev_begin && (e = hipEventRecord(ev_begin, st)) != hipSuccess) return e;
  if (dtype == 0) {
    a.k_split = a.K;
    dim3 grid((a.N + 63) / 64, (a.M + 63) / 64, 1);
    hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(NT), 0, st, a);
    if (ev_end && (e = hipEventRecord(ev_end, st)) != hipSuccess) return e;
    return hipGetLastError();
  }
  const SplitPlan pl = split_plan(a.M, a.N, a.K, dtype);
  a.k_split = pl.kc;
  static_assert(RD_BN == SK_BN, "reduce tiles must match the GEMM's column tiles");
  if (use_skinny(a.M, a.K)) {
    a.n_full = 0; a.tail_sp = 1; a.n_tail0 = 0; a.xcd_cols = 0;
    if (splits_out) *splits_out = pl.splits;
    const int bm = bm_for(a.M, a.K);
    dim3 grid((a.N + SK_BN - 1) / SK_BN, 1, pl.splits);
    // unrolled variants when every split has the same whole number of stages
    const int ns = (a.K % pl.kc == 0) ? pl.kc / SK_KA : 0;
#define SKINNY_NS(MT_)                                                                         \
  switch (ns) {                                                                                \
    case 1: hipLaunchKernelGGL((gemm_skinny_kernel<MT_, 1>), grid, dim3(NT), 0, st, a); break;   \
    case 2: hipLaunchKernelGGL((gemm_skinny_kernel<MT_, 2>), grid, dim3(NT), 0, st, a); break;   \
    case 3: hipLaunchKernelGGL((gemm_skinny_kernel<MT_, 3>), grid, dim3(NT), 0, st, a); break;   \
    case 4: hipLaunchKernelGGL((gemm_skinny_kernel<MT_, 4>), grid, dim3(NT), 0, st, a); break;   \
    case 6: hipLaunchKernelGGL((gemm_skinny_kernel<MT_, 6>), grid, dim3(NT), 0, st, a); break;   \
    case 8: hipLaunchKernelGGL((gemm_skinny_kernel<MT_, 8>), grid, dim3(NT), 0, st, a); break;   \
    case 16: hipLaunchKernelGGL((gemm_skinny_kernel<MT_, 16>), grid, dim3(NT), 0, st, a); break; \
    default: hipLaunchKernelGGL((gemm_skinny_kernel<MT_, 0>), grid, dim3(NT), 0, st, a); break;  \
  }
    switch (bm) {
      case 16: SKINNY_NS(1) break;
      case 32: SKINNY_NS(2) break;
      case 48: SKINNY_NS(3) break;
      default: SKINNY_NS(4) break;
    }
#undef SKINNY_NS
    if (ev_end && (e = hipEventRecord(ev_end, st)) != hipSuccess) return e;
    if (pl.splits > 1 && a.epi != EPI_RESID) {
      dim3 rgrid((a.N + RD_BN - 1) / RD_BN, (a.M + RD_BM - 1) / RD_BM);
      hipLaunchKernelGGL(gemm_reduce_kernel, rgrid, dim3(NT), 0, st, a, pl.splits);
    }
    return hipGetLastError();
  }
  const int bmt = tile_bm(pl.kind), bnt = tile_bn(pl.kind);
  const int mt = (a.M + bmt - 1) / bmt, nt = (a.N + bnt - 1) / bnt;
  a.n_full = pl.n_full;
  a.tail_sp = pl.splits;
  a.n_tail0 = pl.n_tail0;
  // columns placed XCD by XCD: the whole-tile columns (all of them without splits)
  a.xcd_cols = (mt <= (pl.kind == GK_TILED ? TILED_GM : BIG_GM) ? pl.n_full / mt : nt) / 8 * 8;
  const long items = (long)pl.n_full + ((long)mt * nt - pl.n_full) * pl.splits;
  if (pl.kind == GK_BIG)
    hipLaunchKernelGGL((gemm_big_kernel<8, 256>), dim3((unsigned)items), dim3(512), 0, st, a);
  else if (pl.kind == GK_BIG384)
    hipLaunchKernelGGL((gemm_big_kernel<12, 128>), dim3((unsigned)items), dim3(768), 0, st, a);
  else
    hipLaunchKernelGGL((gemm_mfma_kernel<128, 128, 2, 2>), dim3((unsigned)items), dim3(NT), 0, st, a);
  if (ev_end && (e = hipEventRecord(ev_end, st)) != hipSuccess) return e;
  if (pl.splits > 1) {
    if (pl.n_full == 0 && a.epi == EPI_RESID) {
      if (splits_out) *splits_out = pl.splits;  // the caller folds the partials
    } else {
      dim3 rgrid((a.N - pl.n_tail0 + RD_BN - 1) / RD_BN, (a.M + RD_BM - 1) / RD_BM);
      hipLaunchKernelGGL(gemm_reduce_kernel, rgrid, dim3(NT), 0, st, a, pl.splits);
    }
  }
  return hipGetLastError();
}

}  // namespace dllm
