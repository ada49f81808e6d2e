// Row-wise and bookkeeping kernels: embedding gather + RMSNorm, split-K residual add + RMSNorm,
// the merge of the fused lm_head's per-tile softmax partials, the commit rule, token-state
// initialisation, the rotary table, and fills.
#include "kernels.h"

#include <limits.h>

namespace dllm {

template <typename T> __device__ inline float ld_f(const T *p, size_t i);
template <> __device__ inline float ld_f<float>(const float *p, size_t i) { return p[i]; }
template <> __device__ inline float ld_f<bf16>(const bf16 *p, size_t i) { return __bfloat162float(p[i]); }

__device__ inline float block_sum(float v) {
  __shared__ float red[16];
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float s = 0.f;
  const int nw = blockDim.x / 64;
  for (int w = 0; w < nw; ++w) s += red[w];
  return s;
}

// a[i..i+3] = v * r * gain[i..i+3] as hi/lo bf16 planes or fp32.
template <typename T>
__device__ inline void norm_store4(float4 v, float r, const T *gain, size_t o, int i, bf16 *a_hi,
                                   bf16 *a_lo, float *a_f32) {
  const float x[4] = {v.x * r * ld_f<T>(gain, i), v.y * r * ld_f<T>(gain, i + 1),
                      v.z * r * ld_f<T>(gain, i + 2), v.w * r * ld_f<T>(gain, i + 3)};
  if (a_f32) {
    *(float4 *)(a_f32 + o) = make_float4(x[0], x[1], x[2], x[3]);
    return;
  }
  uint32_t hw[2], lw[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const bf16 h0 = __float2bfloat16(x[2 * j]), h1 = __float2bfloat16(x[2 * j + 1]);
    const bf16 l0 = __float2bfloat16(x[2 * j] - __bfloat162float(h0));
    const bf16 l1 = __float2bfloat16(x[2 * j + 1] - __bfloat162float(h1));
    hw[j] = (uint32_t)__bfloat16_as_ushort(h0) | ((uint32_t)__bfloat16_as_ushort(h1) << 16);
    lw[j] = (uint32_t)__bfloat16_as_ushort(l0) | ((uint32_t)__bfloat16_as_ushort(l1) << 16);
  }
  *(uint2 *)(a_hi + o) = make_uint2(hw[0], hw[1]);
  *(uint2 *)(a_lo + o) = make_uint2(lw[0], lw[1]);
}

// One workgroup of RN_NT threads per row; each thread keeps up to RN_MAX_C float4 chunks of the
// row in registers (d <= RN_NT * 4 * RN_MAX_C = 8192).
static constexpr int RN_NT = 1024, RN_MAX_C = 2;

// One workgroup per row: h = embed[token], then a = RMSNorm(h) * gain.
template <typename T>
__global__ __launch_bounds__(RN_NT) void embed_norm_kernel(const int *x, const T *embed,
                                                           const T *gain, RowSet rs, int d,
                                                           float eps, float *h, bf16 *a_hi,
                                                           bf16 *a_lo, float *a_f32, int a_packed) {
  const int m = blockIdx.x;
  const int b = m / rs.nR, p = rs.start + m % rs.nR;
  const int tok = x[(size_t)b * rs.Lx + rs.pos(p)];
  const T *er = embed + (size_t)tok * d;
  float4 v[RN_MAX_C];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < RN_MAX_C; ++c) {
    const int i = (c * RN_NT + threadIdx.x) * 4;
    if (i < d) {
      v[c] = make_float4(ld_f<T>(er, i), ld_f<T>(er, i + 1), ld_f<T>(er, i + 2), ld_f<T>(er, i + 3));
      *(float4 *)(h + (size_t)m * d + i) = v[c];
      ss += v[c].x * v[c].x + v[c].y * v[c].y + v[c].z * v[c].z + v[c].w * v[c].w;
    }
  }
  const float r = rsqrtf(block_sum(ss) / (float)d + eps);
#pragma unroll
  for (int c = 0; c < RN_MAX_C; ++c) {
    const int i = (c * RN_NT + threadIdx.x) * 4;
    if (i < d) norm_store4<T>(v[c], r, gain, a_packed ? pa_off(m, i, d) : (size_t)m * d + i, i, a_hi, a_lo, a_f32);
  }
}

// One workgroup per row: h += sum_z partial[z] (split order), a = RMSNorm(h) * gain.
template <typename T>
__global__ __launch_bounds__(RN_NT) void resid_norm_kernel(int M, int d, float *h,
                                                           const float *__restrict__ part,
                                                           int splits, const T *gain, float eps,
                                                           bf16 *a_hi, bf16 *a_lo, float *a_f32,
                                                           int a_packed) {
  const int m = blockIdx.x;
  const size_t MD = (size_t)M * d;
  float4 v[RN_MAX_C];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < RN_MAX_C; ++c) {
    const int i = (c * RN_NT + threadIdx.x) * 4;
    if (i < d) {
      const size_t o = (size_t)m * d + i;
      float4 acc = *(const float4 *)(h + o);
#pragma unroll 8
      for (int z = 0; z < splits; ++z) {
        const float4 q = *(const float4 *)(part + z * MD + o);
        acc.x += q.x; acc.y += q.y; acc.z += q.z; acc.w += q.w;
      }
      v[c] = acc;
      if (splits) *(float4 *)(h + o) = acc;
      ss += acc.x * acc.x + acc.y * acc.y + acc.z * acc.z + acc.w * acc.w;
    }
  }
  const float r = rsqrtf(block_sum(ss) / (float)d + eps);
#pragma unroll
  for (int c = 0; c < RN_MAX_C; ++c) {
    const int i = (c * RN_NT + threadIdx.x) * 4;
    if (i < d) norm_store4<T>(v[c], r, gain, a_packed ? pa_off(m, i, d) : (size_t)m * d + i, i, a_hi, a_lo, a_f32);
  }
}

hipError_t launch_embed_norm(const int *x, const void *embed, const void *gain, RowSet rs, int d,
                             float eps, float *h, bf16 *a_hi, bf16 *a_lo, float *a_f32, int dtype,
                             int a_packed, hipStream_t st) {
  if (rs.M() <= 0) return hipSuccess;
  if (d % 4 || d > RN_NT * 4 * RN_MAX_C || (a_packed && (dtype == 0 || d % 32)))
    return hipErrorInvalidValue;
  if (dtype == 0)
    hipLaunchKernelGGL(embed_norm_kernel<float>, dim3(rs.M()), dim3(RN_NT), 0, st, x,
                       (const float *)embed, (const float *)gain, rs, d, eps, h, a_hi, a_lo, a_f32, 0);
  else
    hipLaunchKernelGGL(embed_norm_kernel<bf16>, dim3(rs.M()), dim3(RN_NT), 0, st, x,
                       (const bf16 *)embed, (const bf16 *)gain, rs, d, eps, h, a_hi, a_lo, a_f32, a_packed);
  return hipGetLastError();
}

hipError_t launch_resid_norm(int M, int d, float *h, const float *partial, int splits,
                             const void *gain, float eps, bf16 *a_hi, bf16 *a_lo, float *a_f32,
                             int dtype, int a_packed, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  if (d % 4 || d > RN_NT * 4 * RN_MAX_C || (a_packed && (dtype == 0 || d % 32)))
    return hipErrorInvalidValue;
  if (dtype == 0)
    hipLaunchKernelGGL(resid_norm_kernel<float>, dim3(M), dim3(RN_NT), 0, st, M, d, h, partial,
                       splits, (const float *)gain, eps, a_hi, a_lo, a_f32, 0);
  else
    hipLaunchKernelGGL(resid_norm_kernel<bf16>, dim3(M), dim3(RN_NT), 0, st, M, d, h, partial,
                       splits, (const bf16 *)gain, eps, a_hi, a_lo, a_f32, a_packed);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// lm_head partial merge.  One wave per row; lane j folds tiles j, j+64, ... in order, then a
// fixed butterfly combines the lanes, so the result does not depend on scheduling.
struct Part4 {
  float m1; int idx; float m2; float z;
};
__device__ inline Part4 part_merge(Part4 a, Part4 b) {
  const bool bw = (b.m1 > a.m1) || (b.m1 == a.m1 && b.idx < a.idx);
  const Part4 w = bw ? b : a, l = bw ? a : b;
  Part4 r;
  r.m1 = w.m1;
  r.idx = w.idx;
  r.m2 = fmaxf(w.m2, l.m1);
  r.z = w.z + (l.m1 == -INFINITY ? 0.f : l.z * __expf(l.m1 - w.m1));
  return r;
}

__global__ __launch_bounds__(64) void head_merge_kernel(const HeadPart *part, int n_vtiles,
                                                        int *tok, float *conf, float *p2) {
  const int row = blockIdx.x, lane = threadIdx.x;
  Part4 acc = {-INFINITY, INT_MAX, -INFINITY, 0.f};
  const HeadPart *pr = part + (size_t)row * n_vtiles;
  for (int t = lane; t < n_vtiles; t += 64) {
    const HeadPart hp = pr[t];
    Part4 x = {hp.m1, hp.idx, hp.m2, hp.z};
    acc = part_merge(acc, x);
  }
  for (int off = 32; off > 0; off >>= 1) {
    Part4 o;
    o.m1 = __shfl_xor(acc.m1, off, 64);
    o.idx = __shfl_xor(acc.idx, off, 64);
    o.m2 = __shfl_xor(acc.m2, off, 64);
    o.z = __shfl_xor(acc.z, off, 64);
    // both partners must compute the same value: order the operands by lane
    acc = (lane & off) ? part_merge(o, acc) : part_merge(acc, o);
  }
  if (lane == 0) {
    if (acc.idx == INT_MAX) {
      // no finite logit in the row (NaN input): token 0, confidence NaN (ranks last)
      tok[row] = 0;
      conf[row] = __int_as_float(0x7fc00000);
      p2[row] = 0.f;
    } else {
      tok[row] = acc.idx;
      conf[row] = 1.0f / acc.z;
      p2[row] = (acc.m2 == -INFINITY ? 0.f : __expf(acc.m2 - acc.m1)) / acc.z;
    }
  }
}

hipError_t launch_head_merge(const HeadPart *part, int n_rows, int n_vtiles, int *tok, float *conf,
                             float *p2, hipStream_t st) {
  if (n_rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(head_merge_kernel, dim3(n_rows), dim3(64), 0, st, part, n_vtiles, tok, conf,
                     p2);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Commit: one workgroup per batch row, thread i owns block position s + i.  A masked position
// commits when conf > threshold or when fewer than k_floor masked positions rank above it
// (confidence descending, then position ascending; NaN ranks last and is counted).  Schedule
// rules (CommitRules): with first-step scheduling the block's first step uses first_threshold
// and later steps' floors spread the hard positions (masked after the first step) over the
// remaining spb - 1 steps; with early exit each masked position's run (consecutive steps with
// the same argmax above exit_floor) is updated, and when every position still masked after the
// commit has a run of at least exit_steps, they are all committed.
__global__ __launch_bounds__(256) void commit_kernel(int *x, int L, int s, int Bs, const int *tok,
                                                     const float *conf, float threshold,
                                                     int k_floor, int mask_id, uint8_t *committed,
                                                     int *cnt_out, const CommitRules cr) {
  __shared__ float cs[256];
  __shared__ int ms[256];
  __shared__ int cnt[5];  // committed, remaining, NaN, still masked, still masked and not converged
  const int b = blockIdx.x, i = threadIdx.x, B = gridDim.x;
  if (i < 5) cnt[i] = 0;
  __syncthreads();
  const bool first = cr.first_threshold >= 0.f;
  const float tau = first && cr.j == 0 ? cr.first_threshold : threshold;
  int k = k_floor;
  if (first && cr.j >= 1) {  // the hard positions over the remaining steps
    const int nh = cr.n_hard[b], ns = cr.spb - 1 > 1 ? cr.spb - 1 : 1;
    const int kk = nh / ns + ((cr.j - 1) < nh % ns ? 1 : 0);
    k = kk < 1 ? 1 : kk;
  }
  const size_t pi = (size_t)b * Bs + i;
  int masked = 0, t = 0;
  float c = -INFINITY, craw = 0.f;
  if (i < Bs) {
    masked = x[(size_t)b * L + s + i] == mask_id;
    t = tok[pi];
    craw = conf[pi];
    c = craw;
    if (c != c) {
      c = -INFINITY;
      if (masked) atomicAdd(&cnt[2], 1);
    }
    cs[i] = c;
    ms[i] = masked;
  }
  __syncthreads();
  int commit = 0;
  if (i < Bs && masked) {
    int rank = 0;
    for (int q = 0; q < Bs; ++q)
      rank += ms[q] && (cs[q] > c || (cs[q] == c && q < i));
    commit = (c > tau) || (rank < k);
  }
  if (cr.exit_steps > 0) {
    if (i < Bs && masked) {
      const int prev = cr.j == 0 ? -1 : cr.prev_tok[pi];
      int r = cr.j == 0 ? 0 : cr.run[pi];
      r = !(craw > cr.exit_floor) ? 0 : (t == prev ? r + 1 : 1);  // NaN: not above
      cr.prev_tok[pi] = t;
      cr.run[pi] = r;
      if (!commit) {
        atomicAdd(&cnt[3], 1);
        if (r < cr.exit_steps) atomicAdd(&cnt[4], 1);
      }
    }
    __syncthreads();
    if (cnt[3] > 0 && cnt[4] == 0 && i < Bs && masked) commit = 1;  // every rest converged
  }
  if (commit) x[(size_t)b * L + s + i] = t;
  if (i < Bs) committed[pi] = (uint8_t)commit;
  if (commit) atomicAdd(&cnt[0], 1);
  if (masked && !commit) atomicAdd(&cnt[1], 1);
  __syncthreads();
  if (i == 0) {
    cnt_out[b] = cnt[0];
    cnt_out[B + b] = cnt[1];
    cnt_out[2 * B + b] = cnt[2];
    cnt_out[3 * B + b] = cr.exit_steps > 0 && cnt[3] > 0 && cnt[4] == 0;
    if (first && cr.j == 0) cr.n_hard[b] = cnt[1];
  }
}

hipError_t launch_commit(int *x, int L, int B, int s, int Bs, const int *tok, const float *conf,
                         float threshold, int k_floor, int mask_id, uint8_t *committed, int *cnt,
                         const CommitRules &cr, hipStream_t st) {
  if (Bs > 256) return hipErrorInvalidValue;
  if ((cr.exit_steps > 0 && (!cr.prev_tok || !cr.run)) || (cr.first_threshold >= 0.f && !cr.n_hard))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(commit_kernel, dim3(B), dim3(256), 0, st, x, L, s, Bs, tok, conf, threshold,
                     k_floor, mask_id, committed, cnt, cr);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
__global__ void init_tokens_kernel(int *x, int B, int P, int L, int mask_id) {
  const size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  if (i >= (size_t)B * L) return;
  if ((int)(i % L) >= P) x[i] = mask_id;
}

hipError_t launch_init_tokens(int *x, int B, int P, int L, int mask_id, hipStream_t st) {
  const size_t n = (size_t)B * L;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(init_tokens_kernel, dim3((n + 255) / 256), dim3(256), 0, st, x, B, P, L,
                     mask_id);
  return hipGetLastError();
}

__global__ void rope_table_kernel(float *cos_t, float *sin_t, int L, int hd, double base) {
  const int half = hd / 2;
  const size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  if (i >= (size_t)L * half) return;
  const int p = i / half, j = i % half;
  const double theta = (double)p * pow(base, -2.0 * j / (double)hd);
  cos_t[i] = (float)cos(theta);
  sin_t[i] = (float)sin(theta);
}

hipError_t launch_rope_table(float *cos_t, float *sin_t, int L, int hd, float base, hipStream_t st) {
  const size_t n = (size_t)L * (hd / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, st, cos_t, sin_t, L, hd,
                     (double)base);
  return hipGetLastError();
}

__global__ void fill_u32_kernel(uint32_t *p, uint32_t v, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += stride) p[i] = v;
}

hipError_t launch_fill_u32(uint32_t *p, uint32_t v, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_u32_kernel, dim3(blocks), dim3(256), 0, st, p, v, n);
  return hipGetLastError();
}

__global__ void mask_column_kernel(float *logits, int n_rows, int vocab, int mask_id) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r < n_rows) logits[(size_t)r * vocab + mask_id] = -INFINITY;
}

hipError_t launch_mask_column(float *logits, int n_rows, int vocab, int mask_id, hipStream_t st) {
  hipLaunchKernelGGL(mask_column_kernel, dim3((n_rows + 63) / 64), dim3(64), 0, st, logits, n_rows,
                     vocab, mask_id);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Row gather: dst row b * n + j = src row b * src_stride + src_off + j (b < B, j < n), rows of
// row_bytes (a multiple of 16) bytes.  One workgroup per destination row.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint4 *__restrict__ src,
                                                          uint4 *__restrict__ dst, int n,
                                                          int src_stride, int src_off,
                                                          int row_chunks) {
  const int r = blockIdx.x, b = r / n, j = r % n;
  const uint4 *s = src + ((size_t)b * src_stride + src_off + j) * row_chunks;
  uint4 *d = dst + (size_t)r * row_chunks;
  for (int c = threadIdx.x; c < row_chunks; c += 256) d[c] = s[c];
}

hipError_t launch_gather_rows(const void *src, void *dst, int B, int n, int src_stride,
                              int src_off, size_t row_bytes, hipStream_t st) {
  if (B <= 0 || n <= 0) return hipSuccess;
  if (row_bytes % 16 || src_off < 0 || src_off + n > src_stride) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(B * n), dim3(256), 0, st, (const uint4 *)src,
                     (uint4 *)dst, n, src_stride, src_off, (int)(row_bytes / 16));
  return hipGetLastError();
}

}  // namespace dllm
