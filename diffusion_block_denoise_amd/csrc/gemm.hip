// GEMM C[m][n] = sum_k A[m][k] * W[n][k] for the projections, the feed-forward and the lm_head,
// with fused epilogues.  W is in torch Linear layout [out, in], so both operands are K-contiguous.
//
// bf16 path: A arrives as two bf16 arrays (hi, lo) with hi + lo equal to the fp32 activation to
// about 16 mantissa bits; each K step issues two bf16 MFMAs (hi x W, lo x W) into one fp32
// accumulator.  At the small row counts of a cached step the GEMM is bound by streaming W from
// HBM, so the second MFMA costs no time and keeps the activation error at fp32 level.
//
// Tiles are staged through LDS.  After the K loop the wave accumulators are written to an fp32
// C tile in LDS so that every epilogue has random access to the whole tile (rotary pairs i and
// i + hd/2, gate and up halves, row-wise softmax over a vocabulary tile).  Split-K: every split
// writes its tile to a partial buffer; the last split to arrive (per-tile atomic counter) sums
// the partials in split order (deterministic), resets the counter and runs the epilogue.
#include "kernels.h"

#include <float.h>
#include <limits.h>

namespace dllm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

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
// Epilogues over an fp32 C tile in LDS (ld = ldc).  T is the storage type of q and the cache.
__device__ inline float silu_f(float g) { return g / (1.0f + __expf(-g)); }

__device__ inline void split_hilo(float v, bf16 &hi, bf16 &lo) {
  hi = __float2bfloat16(v);
  lo = __float2bfloat16(v - __bfloat162float(hi));
}

template <typename T> __device__ inline T to_store(float v);
template <> __device__ inline float to_store<float>(float v) { return v; }
template <> __device__ inline bf16 to_store<bf16>(float v) { return __float2bfloat16(v); }

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
          const float cs = a.rope_cos[(size_t)p * half + j], sn = a.rope_sin[(size_t)p * half + j];
          const float y = i < half ? x * cs - Ct[r * ldc + c + half] * sn
                                   : x * cs + Ct[r * ldc + c - half] * sn;
          if (n < nq) {
            ((T *)a.q_out)[(size_t)m * nq + n] = to_store<T>(y);
          } else {
            const int kvh = (n - nq) / hd;
            ((T *)a.k_cache)[(((size_t)b * Hkv + kvh) * rs.Lp + p) * hd + i] = to_store<T>(y);
          }
        } else {
          const int kvh = (n - nq - nk) / hd;
          ((T *)a.vt_cache)[(((size_t)b * Hkv + kvh) * hd + i) * rs.Lp + p] = to_store<T>(x);
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

// Split-K: publish this split's tile, and let the last arriving split reduce all of them in
// split order into Ct.  Returns false for the splits that are not last.
template <int BM, int BN>
__device__ bool splitk_fixup(const GemmArgs &a, float *Ct, int ldc, int m0, int n0) {
  __shared__ int s_last;
  const int tid = threadIdx.x;
  const int splits = gridDim.z;
  const size_t MN = (size_t)a.M * a.N;
  float *P = a.partial + (size_t)blockIdx.z * MN;
  for (int e = tid; e < BM * BN; e += NT) {
    const int r = e / BN, c = e % BN, m = m0 + r, n = n0 + c;
    if (m < a.M && n < a.N) P[(size_t)m * a.N + n] = Ct[r * ldc + c];
  }
  __threadfence();
  __syncthreads();
  const int tile = blockIdx.y * gridDim.x + blockIdx.x;
  if (tid == 0) s_last = (atomicAdd(&a.counters[tile], 1) == splits - 1);
  __syncthreads();
  if (!s_last) return false;
  __threadfence();
  for (int e = tid; e < BM * BN; e += NT) {
    const int r = e / BN, c = e % BN, m = m0 + r, n = n0 + c;
    float s = 0.f;
    if (m < a.M && n < a.N) {
      for (int z = 0; z < splits; ++z)
        s += __hip_atomic_load(a.partial + z * MN + (size_t)m * a.N + n, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    Ct[r * ldc + c] = s;
  }
  if (tid == 0) a.counters[tile] = 0;
  __syncthreads();
  return true;
}

// ---------------------------------------------------------------------------------------------
// bf16 MFMA kernel.  4 waves as WM x WN; each wave owns (BM/WM) x (BN/WN) of the tile in
// 32x32 blocks (v_mfma_f32_32x32x16_bf16).  BK = 64.
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

  // Global -> register staging: 16-byte chunks, 8 per 64-wide row.
  constexpr int A_CH = BM * BK / 8 / NT;  // chunks per thread for each of hi, lo
  constexpr int W_CH = BN * BK / 8 / NT;
  static_assert(A_CH >= 1 && W_CH >= 1, "tile too small");
  uint4 ra_hi[A_CH], ra_lo[A_CH], rw[W_CH];
  const uint16_t *wrow[W_CH];
#pragma unroll
  for (int i = 0; i < W_CH; ++i) {
    const int ch = tid + i * NT, r = ch / 8;
    wrow[i] = w_row<uint16_t>(a, BN, n0, r);
  }

  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int ch = tid + i * NT, r = ch / 8, c8 = (ch % 8) * 8, m = m0 + r;
      if (m < a.M) {
        const size_t off = (size_t)m * a.lda + k0 + c8;
        ra_hi[i] = *(const uint4 *)((const uint16_t *)a.a_hi + off);
        ra_lo[i] = *(const uint4 *)((const uint16_t *)a.a_lo + off);
      } else {
        ra_hi[i] = make_uint4(0, 0, 0, 0);
        ra_lo[i] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < W_CH; ++i) {
      const int ch = tid + i * NT, c8 = (ch % 8) * 8;
      rw[i] = wrow[i] ? *(const uint4 *)(wrow[i] + k0 + c8) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int ch = tid + i * NT, r = ch / 8, c8 = (ch % 8) * 8;
      *(uint4 *)(As_hi + r * LDK + c8) = ra_hi[i];
      *(uint4 *)(As_lo + r * LDK + c8) = ra_lo[i];
    }
#pragma unroll
    for (int i = 0; i < W_CH; ++i) {
      const int ch = tid + i * NT, r = ch / 8, c8 = (ch % 8) * 8;
      *(uint4 *)(Ws + r * LDK + c8) = rw[i];
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
  if (kbeg < kend) load(kbeg);
  for (int k0 = kbeg; k0 < kend; k0 += BK) {
    __syncthreads();
    store();
    __syncthreads();
    if (k0 + BK < kend) load(k0 + BK);
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
  if (gridDim.z > 1 && !splitk_fixup<BM, BN>(a, Ct, LDC, m0, n0)) return;
  run_epilogue<bf16, BM, BN>(a, Ct, LDC, m0, n0);
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
      As[kk][r] = (m < a.M && k < a.K) ? a.a_f32[(size_t)m * a.lda + k] : 0.f;
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

int gemm_bm(int M, int dtype) {
  if (dtype == 0) return 64;
  return M <= 32 ? 32 : (M <= 64 ? 64 : 128);
}

int gemm_num_splits(int M, int N, int K, int dtype) {
  if (dtype == 0) return 1;
  const int bm = gemm_bm(M, dtype), bn = gemm_bn(M, dtype);
  const long tiles = (long)((M + bm - 1) / bm) * ((N + bn - 1) / bn);
  const int target = 512;
  if (tiles >= target) return 1;
  int want = (int)((target + tiles - 1) / tiles);
  const int max_splits = K / 256 > 0 ? K / 256 : 1;
  if (want > max_splits) want = max_splits;
  if (want < 1) want = 1;
  // K per split rounded up to the 64-wide K step; recompute the count that covers K.
  const int kc = ((K + want - 1) / want + 63) / 64 * 64;
  return (K + kc - 1) / kc;
}

hipError_t launch_gemm(const GemmArgs &a0, int dtype, hipStream_t st) {
  GemmArgs a = a0;
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (dtype == 0) {
    a.k_split = a.K;
    dim3 grid((a.N + 63) / 64, (a.M + 63) / 64, 1);
    hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(NT), 0, st, a);
    return hipGetLastError();
  }
  const int bm = gemm_bm(a.M, dtype), bn = gemm_bn(a.M, dtype);
  const int splits = gemm_num_splits(a.M, a.N, a.K, dtype);
  a.k_split = ((a.K + splits - 1) / splits + 63) / 64 * 64;
  dim3 grid((a.N + bn - 1) / bn, (a.M + bm - 1) / bm, splits);
  if (bm == 32)
    hipLaunchKernelGGL((gemm_mfma_kernel<32, 128, 1, 4>), grid, dim3(NT), 0, st, a);
  else if (bm == 64)
    hipLaunchKernelGGL((gemm_mfma_kernel<64, 128, 2, 2>), grid, dim3(NT), 0, st, a);
  else
    hipLaunchKernelGGL((gemm_mfma_kernel<128, 128, 2, 2>), grid, dim3(NT), 0, st, a);
  return hipGetLastError();
}

}  // namespace dllm
