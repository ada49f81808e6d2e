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
__device__ void run_epilogue(const GemmArgs &a, const float *Ct, int ldc, int m0, int n0) {
  const int tid = threadIdx.x;
  const int M = a.M;
  switch (a.epi) {
    case EPI_STORE: {
      for (int e = tid; e < BM * BN; e += NT) {
        const int r = e / BN, c = e % BN, m = m0 + r, n = n0 + c;
        if (m < M && n < a.N) a.out_f32[(size_t)m * a.ld_out + n] = a.scale * Ct[r * ldc + c];
      }
    } break;
    case EPI_RESID: {
      for (int e = tid; e < BM * BN; e += NT) {
        const int r = e / BN, c = e % BN, m = m0 + r, n = n0 + c;
        if (m < M && n < a.N) a.resid[(size_t)m * a.ld_out + n] += Ct[r * ldc + c];
      }
    } break;
    case EPI_QKV: {
      const int hd = a.head_dim, half = hd / 2, H = a.n_heads, Hkv = a.n_kv_heads;
      const int nq = H * hd, nk = Hkv * hd;
      const RowSet rs = a.rows;
      for (int e = tid; e < BM * BN; e += NT) {
        const int r = e / BN, c = e % BN, m = m0 + r, n = n0 + c;
        if (m >= M || n >= a.N) continue;
        const int b = m / rs.nR, p = rs.start + m % rs.nR;
        const int i = n % hd;
        const float x = Ct[r * ldc + c];
        if (n < nq + nk) {
          const int j = i < half ? i : i - half;
          const size_t rp = (size_t)rs.pos(p) * half + j;  // rotary angle of the slot's position
        const float cs = a.rope_cos[rp], sn = a.rope_sin[rp];
          const float y = i < half ? x * cs - Ct[r * ldc + c + half] * sn
                                   : x * cs + Ct[r * ldc + c - half] * sn;
          if (n < nq) {
            store_val<T>(a.q_out, a.q_out_lo, (size_t)m * nq + n, y);
          } else {
            const int kvh = (n - nq) / hd;
            store_val<T>(a.k_cache, a.k_cache_lo, (((size_t)b * Hkv + kvh) * rs.Lp + p) * hd + i, y);
          }
        } else {
          const int kvh = (n - nq - nk) / hd;
          // V^T per (batch row, K/V head): fp32 [hd][Lp]; bf16 in 32-key tiles [Lp/32][hd][32], so
          // that the attention's key tile is one contiguous run per plane
          const size_t base = ((size_t)b * Hkv + kvh) * hd * rs.Lp;
          const size_t vi = sizeof(T) == 2 ? base + (size_t)(p >> 5) * hd * 32 + i * 32 + (p & 31)
                                           : base + (size_t)i * rs.Lp + p;
          store_val<T>(a.vt_cache, a.vt_cache_lo, vi, x);
        }
      }
    } break;
    case EPI_SWIGLU: {
      const int half = BN / 2;
      const int f0 = (n0 / BN) * half;
      for (int e = tid; e < BM * half; e += NT) {
        const int r = e / half, c = e % half, m = m0 + r, f = f0 + c;
        if (m >= M || f >= a.n_half) continue;
        const float y = silu_f(Ct[r * ldc + c]) * Ct[r * ldc + c + half];
        const size_t o = (size_t)m * a.ld_act + f;
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

// Split-K: each split writes its tile to partial[split][M][N]; a reduce kernel sums the splits
// in split order (deterministic) and runs the epilogue.  No cross-workgroup fence: on a
// multi-XCD GPU an agent-scope release fence writes back the XCD's L2, which costs far more
// than the separate launch.
template <int BM, int BN>
__device__ void write_partial(const GemmArgs &a, const float *Ct, int ldc, int m0, int n0) {
  float *P = a.partial + (size_t)blockIdx.z * a.M * a.N;
  for (int e = threadIdx.x; e < BM * BN; e += NT) {
    const int r = e / BN, c = e % BN, m = m0 + r, n = n0 + c;
    if (m < a.M && n < a.N) P[(size_t)m * a.N + n] = Ct[r * ldc + c];
  }
}

static constexpr int RD_BM = 8, RD_BN = 128;

// Tile reduce for the epilogues that need a whole tile (rotary pairs, gate/up halves, lm_head
// softmax partials): 8 x 128 tiles, 4 consecutive columns per thread.
__global__ __launch_bounds__(NT) void gemm_reduce_kernel(const GemmArgs a, int splits) {
  constexpr int LDC = RD_BN + 4;
  __shared__ float Ct[RD_BM * LDC];
  const int m0 = blockIdx.y * RD_BM, n0 = blockIdx.x * RD_BN;
  const size_t MN = (size_t)a.M * a.N;
  const int r = threadIdx.x / (RD_BN / 4), c = (threadIdx.x % (RD_BN / 4)) * 4;
  const int m = m0 + r, n = n0 + c;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  if (m < a.M && n < a.N) {  // N is a multiple of 4 (widths are multiples of 64)
    const float *p = a.partial + (size_t)m * a.N + n;
    for (int z = 0; z < splits; ++z) {
      const float4 v = *(const float4 *)(p + z * MN);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
  }
  *(float4 *)(Ct + r * LDC + c) = s;
  __syncthreads();
  run_epilogue<bf16, RD_BM, RD_BN>(a, Ct, LDC, m0, n0);
}

// ---------------------------------------------------------------------------------------------
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
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int kbeg = blockIdx.z * a.k_split;
  const int kend = min(a.K, kbeg + a.k_split);

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
  if (gridDim.z > 1) {
    write_partial<BM, BN>(a, Ct, LDC, m0, n0);
    return;
  }
  run_epilogue<bf16, BM, BN>(a, Ct, LDC, m0, n0);
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

template <int MT>
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
  const int nstage = (nchunk + SK_D - 1) / SK_D;

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
    write_partial<BM, SK_BN>(a, Ct, LDC, 0, n0);
    return;
  }
  run_epilogue<bf16, BM, SK_BN>(a, Ct, LDC, 0, n0);
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
  run_epilogue<float, BM, BN>(a, Ct, LDC, m0, n0);
}

// ---------------------------------------------------------------------------------------------
int gemm_bn(int M, int dtype) { return dtype == 0 ? 64 : 128; }

// The skinny kernel serves M <= 64 (16-row blocks) when K is a whole number of its 256-wide
// stages; otherwise 128 x 128 tiles.
static bool use_skinny(int M, int K) { return M <= 64 && K % SK_KA == 0; }

static int bm_for(int M, int K) { return use_skinny(M, K) ? 16 * ((M + 15) / 16) : 128; }

// Split-K plan.  Skinny kernel: as many splits as keep the grid within one round of resident
// workgroups (3 per CU up to 32 rows, 2 up to 48, 1 at 64), at least 512 k per split and at
// most 8 splits (more only adds partial traffic).  Tiled kernel: see below.
static void split_plan(int M, int N, int K, int dtype, int &splits, int &kc) {
  splits = 1;
  kc = K;
  if (dtype == 0) return;
  const bool sk = use_skinny(M, K);
  const int bm = bm_for(M, K), bn = gemm_bn(M, dtype);
  const long tiles = (long)((M + bm - 1) / bm) * ((N + bn - 1) / bn);
  const int unit = sk ? SK_KA : 64;  // split lengths are whole stages / K steps
  int want, max_splits;
  if (sk) {
    const long cap = (M <= 32 ? 3 : (M <= 48 ? 2 : 1)) * 256L;
    want = (int)(cap / tiles);
    max_splits = std::min(K / 512, 8);
  } else {
    // Estimated time (us): rounds of resident workgroups (2 per CU) times the K steps of a
    // split at ~1.8 us per step and round, plus the round trip of the fp32 partial tiles
    // (written here, read by the reduce) at ~5 TB/s when split.  At most 16 splits of at
    // least 4 K steps.  (Fitted to the 768-row projections of the 8B shape on MI355X.)
    const int iters = K / 64;
    const long slots = 512;
    double best = 1e30;
    want = 1;
    for (int sp = 1; sp <= 16 && sp <= std::max(1, iters / 4); ++sp) {
      const long rounds = (tiles * sp + slots - 1) / slots;
      const double partial_us = sp > 1 ? sp * (double)M * N * 8.0 / 5.0e6 : 0.0;
      const double cost = 1.8 * rounds * ((iters + sp - 1) / sp) + partial_us;
      if (cost < best - 1e-9) { best = cost; want = sp; }
    }
    max_splits = std::max(1, K / 256);
  }
  if (want > max_splits) want = max_splits;
  if (want < 1) want = 1;
  kc = ((K + want - 1) / want + unit - 1) / unit * unit;
  splits = (K + kc - 1) / kc;
}

int gemm_num_splits(int M, int N, int K, int dtype) {
  int splits, kc;
  split_plan(M, N, K, dtype, splits, kc);
  return splits;
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
  hipError_t e;
  if (ev_begin && (e = hipEventRecord(ev_begin, st)) != hipSuccess) return e;
  if (dtype == 0) {
    a.k_split = a.K;
    dim3 grid((a.N + 63) / 64, (a.M + 63) / 64, 1);
    hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(NT), 0, st, a);
    if (ev_end && (e = hipEventRecord(ev_end, st)) != hipSuccess) return e;
    return hipGetLastError();
  }
  const int bm = bm_for(a.M, a.K), bn = gemm_bn(a.M, dtype);
  int splits, kc;
  split_plan(a.M, a.N, a.K, dtype, splits, kc);
  a.k_split = kc;
  if (splits_out) *splits_out = splits;
  dim3 grid((a.N + bn - 1) / bn, (a.M + bm - 1) / bm, splits);
  switch (bm) {
    case 16: hipLaunchKernelGGL(gemm_skinny_kernel<1>, grid, dim3(NT), 0, st, a); break;
    case 32: hipLaunchKernelGGL(gemm_skinny_kernel<2>, grid, dim3(NT), 0, st, a); break;
    case 48: hipLaunchKernelGGL(gemm_skinny_kernel<3>, grid, dim3(NT), 0, st, a); break;
    case 64: hipLaunchKernelGGL(gemm_skinny_kernel<4>, grid, dim3(NT), 0, st, a); break;
    default: hipLaunchKernelGGL((gemm_mfma_kernel<128, 128, 2, 2>), grid, dim3(NT), 0, st, a);
  }
  if (ev_end && (e = hipEventRecord(ev_end, st)) != hipSuccess) return e;
  if (splits > 1 && a.epi != EPI_RESID) {
    static_assert(RD_BN == SK_BN, "reduce tiles must match the GEMM's column tiles");
    dim3 rgrid((a.N + RD_BN - 1) / RD_BN, (a.M + RD_BM - 1) / RD_BM);
    hipLaunchKernelGGL(gemm_reduce_kernel, rgrid, dim3(NT), 0, st, a, splits);
  }
  return hipGetLastError();
}

}  // namespace dllm
