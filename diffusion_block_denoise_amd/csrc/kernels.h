// Internal interface between the host runtime (dllm.cpp) and the gfx950 kernels.
// Every launcher enqueues on the given stream and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

namespace dllm {

typedef __hip_bfloat16 bf16;

// Rows that one forward processes: for each batch row b, positions [start, start + nR).
// Row m of every activation buffer is (b = m / nR, position = start + m % nR).
// Rows of a forward.  Positions are cache-slot indices c in [0, L): the model's context.
// With suffix pruning the context is the compacted sequence [0, L - 1) plus one slot, the
// `tail`, that carries the last position Lx - 1 of the token state; pos(c) is the position
// (token index and rotary angle) of slot c.  Without pruning tail = -1 and pos(c) = c.
struct RowSet {
  int B;      // batch rows
  int L;      // context length: keys every query attends to (slots [0, L))
  int Lp;     // cache slots per batch row and head: the full length rounded up to 32
  int start;  // first slot of the rows
  int nR;     // rows per batch row
  int Lx;     // token-state length per batch row (prompt + generation)
  int tail;   // slot that holds position Lx - 1, or -1
  // block-causal attention: a query at position p sees keys below the end of p's block (the
  // prompt, P positions, is one block; then blocks of Bs)
  int causal, P, Bs;
  __host__ __device__ int M() const { return B * nR; }
  __host__ __device__ int pos(int c) const { return c == tail ? Lx - 1 : c; }
  // keys [0, key_limit(c)) are visible to the query in slot c
  __host__ __device__ int key_limit(int c) const {
    if (!causal) return L;
    const int e = c < P ? P : P + ((c - P) / Bs + 1) * Bs;
    return e < L ? e : L;
  }
};

// Position of key k (0..31) inside a 32-key row of the bf16 V^T cache.  The P.V product's B
// operand gives the lane of half h in 16-key step s the keys 16s + 4h + {0..3} and
// 16s + 8 + 4h + {0..3}; storing them as the 16-byte chunk 2s + h lets the lane read its eight
// V^T values with one load.
__host__ __device__ inline int vt_key_pos(int k) {
  return ((k >> 4) * 2 + ((k >> 2) & 1)) * 8 + ((k >> 3) & 1) * 4 + (k & 3);
}

// Panel-packed activations: the hi/lo A operand of the large-tile GEMM is stored like the packed
// weights, element (m, k) of an M x K matrix at
// ((m / 128) * (K / 32) + k / 32) * 4096 + (m % 128) * 32 + k % 32 (K a multiple of 32, rows
// padded to a multiple of 128), so a 32-wide k block of a 128-row tile is one contiguous 8 KB
// run.  The other GEMMs read row-major activations (the 128-row tiled kernel, which loads A
// through registers, measured slower on the packed layout).
__host__ __device__ inline size_t pa_off(size_t m, int k, int K) {
  return ((m >> 7) * (size_t)(K >> 5) + (size_t)(k >> 5)) * 4096 + (m & 127) * 32 + (k & 31);
}

// GEMM epilogues.  The GEMM computes C[m][n] = sum_k A[m][k] * W[n][k] (fp32 accumulate).
enum Epi : int {
  EPI_STORE = 0,   // out_f32[m*ld_out + n] = scale * C
  EPI_RESID = 1,   // resid[m*ld_out + n] += C
  EPI_QKV = 2,     // rotary embedding of q and k, q to q_out, k and v to the cache slots
  EPI_SWIGLU = 3,  // tiles hold gate and up halves: act[m][f] = silu(g) * u
  EPI_LMHEAD = 4,  // per row and vocab tile: max, argmax, runner-up max, sum of exp
};

// Per-(row, vocab tile) softmax partial of the fused lm_head.
struct HeadPart {
  float m1;   // max scaled logit in the tile
  int idx;    // its vocab id (lowest among equal maxima)
  float m2;   // best scaled logit among the tile's other ids
  float z;    // sum over the tile of exp(logit - m1)
};

struct GemmArgs {
  // A operand: M x K, row-major with leading dimension lda; row m of A is row
  // (m / row_per) * row_stride + row_off + m % row_per of the array (row_per 0: row m).
  //   bf16 path: a_hi + a_lo (two bf16 arrays whose sum is the fp32 activation)
  //   f32 path : a_f32
  // a_packed: the hi/lo planes are panel-packed (pa_off with K columns; lda unused); taken by
  // the large-tile kernel only, and exactly when gemm_a_packed says so.
  const bf16 *a_hi, *a_lo;
  const float *a_f32;
  int lda;
  int row_per, row_stride, row_off;
  int a_packed;
  // W operand: N x K rows from up to three segments (torch Linear layout, ld = K).
  // Plain mode: virtual row n lives in segment s with seg_end[s-1] <= n < seg_end[s].
  // SwiGLU mode: tile t, column c < BN/2 -> gate row t*BN/2 + c; else up row t*BN/2 + c - BN/2,
  //   rows >= n_half (ffn_dim) are zero.
  const void *w[3];
  int seg_end[3];
  // bf16 path: W packed (pack_weight) into 128-row panels of 32-wide k blocks; virtual row n,
  // column k at ((n / 128) * (K / 32) + k / 32) * 4096 + (n % 128) * 32 + k % 32, rows past N
  // zero up to the next multiple of 128.  w / seg_end are then unused.
  const uint16_t *wp;
  int n_half;     // SwiGLU: ffn_dim
  int M, N, K;    // N is the virtual width (SwiGLU: 2 * ceil(ffn_dim / (BN/2)) * (BN/2))
  int k_split;    // K elements per split (multiple of the kernel's BK)
  // Split-K partial tiles fp32 [splits][M][N - n_tail0]: column n of a split tile is stored at
  // column n - n_tail0.  Skinny kernel: gridDim.z splits of every tile, n_tail0 = 0.  Tiled
  // kernel (1-D grid, M-tile index fastest): work items below n_full are whole tiles with their
  // epilogue; each later tile (all of them columns from n_tail0 on) is split tail_sp ways.
  float *partial;
  int n_full, tail_sp, n_tail0;
  // tiled kernels: in each group of M tiles, the tiles of the first xcd_cols columns (a multiple
  // of 8) are placed XCD by XCD (workgroup b runs on XCD b % 8): XCD x gets columns x, x + 8,
  // ..., each with the group's M tiles, so a W panel is fetched into one L2 only
  int xcd_cols;
  int epi;
  // epilogue operands
  float *out_f32; int ld_out; float scale;        // STORE
  float *resid;                                   // RESID (ld_out)
  // QKV
  RowSet rows; int n_heads, n_kv_heads, head_dim;
  const float *rope_cos, *rope_sin;               // [L][head_dim/2]
  // q [M][n_heads*head_dim]; this layer's K [B][Hkv][Lp][hd] and transposed V [B][Hkv][hd][Lp].
  // f32 path: one fp32 array each.  bf16 path: a hi and a lo bf16 plane each (hi + lo = value).
  void *q_out, *q_out_lo;
  void *k_cache, *k_cache_lo, *vt_cache, *vt_cache_lo;
  // SWIGLU output (bf16 path: hi/lo, panel-packed when act_packed; f32 path: f32), ld = ld_act
  bf16 *act_hi, *act_lo; float *act_f32; int ld_act; int act_packed;
  // LMHEAD
  HeadPart *head_part; int n_vtiles; int vocab; int mask_id;
};

// Packed bf16 weights (the W layout of GemmArgs::wp).  PW_ROWS rows per panel, PW_K columns per
// block.  Virtual rows: PACK_PLAIN: row n of src[0] (n < N); PACK_CONCAT: rows of src[0], then
// src[1], then src[2], segment ends seg_end[0..2]; PACK_SWIGLU: panel t, row c < 64 -> gate row
// 64 t + c of src[0], else up row 64 t + c - 64 of src[1], for rows < n_half.  Other rows are zero.
static constexpr int PW_ROWS = 128, PW_K = 32;
enum PackMode { PACK_PLAIN = 0, PACK_CONCAT = 1, PACK_SWIGLU = 2 };
inline size_t packed_rows(int N) { return (size_t)(N + PW_ROWS - 1) / PW_ROWS * PW_ROWS; }
hipError_t launch_pack_weight(uint16_t *dst, const void *const src[3], const int seg_end[3],
                              int n_half, int mode, int N, int K, hipStream_t st);

// Storage-type tag for templates: 0 = f32, 1 = bf16.
// splits_out (may be NULL) receives the split-K count.  With EPI_RESID and more than one split
// the GEMM only writes partial[split][M][N]; the caller folds them in with launch_resid_norm.
// ev_begin/ev_end (may be NULL): recorded on st right before and after the main GEMM kernel.
hipError_t launch_gemm(const GemmArgs &a, int dtype, hipStream_t st, int *splits_out,
                       hipEvent_t ev_begin = nullptr, hipEvent_t ev_end = nullptr);
// Which kernel launch_gemm uses: 0 = f32 SIMT, 1 = skinny weight-streaming, 2 = tiled MFMA.
int gemm_kind(int M, int K, int dtype);
// Whether the A operand of an M x N x K GEMM is read panel-packed (when launch_gemm runs it on
// the large-tile kernel, whose LDS-DMA stages then take whole 512-byte runs of A): the producers
// of activations write that layout exactly when their consumer's answer is yes.
bool gemm_a_packed(int M, int N, int K, int dtype);
// Tile width (N direction) that launch_gemm uses for a given M and dtype; SwiGLU and
// the lm_head partial layout depend on it.
int gemm_bn(int M, int dtype);
// Splits of the caller-visible partial buffer (EPI_RESID folds them in resid_norm), and the
// partial buffer size in bytes that launch_gemm needs for this shape.
int gemm_num_splits(int M, int N, int K, int dtype);
size_t gemm_partial_bytes(int M, int N, int K, int dtype);

// h[m] = embed[x[b][p]] (fp32); a = RMSNorm(h[m]) * gain as hi/lo planes (bf16; panel-packed
// when a_packed) or f32.
hipError_t launch_embed_norm(const int *x, const void *embed, const void *gain, RowSet rows, int d,
                             float eps, float *h, bf16 *a_hi, bf16 *a_lo, float *a_f32, int dtype,
                             int a_packed, hipStream_t st);
// Per row m < M: h[m] += sum over the splits of partial[z][m] (in split order; splits 0: no
// partials), then a[m] = RMSNorm(h[m]) * gain as hi/lo planes (bf16; panel-packed when
// a_packed) or f32.
hipError_t launch_resid_norm(int M, int d, float *h, const float *partial, int splits,
                             const void *gain, float eps, bf16 *a_hi, bf16 *a_lo, float *a_f32,
                             int dtype, int a_packed, hipStream_t st);
// Non-causal attention of the rows' queries over all L cached positions.
// bf16 path: q, K and V^T come as hi/lo plane pairs, the output o as hi/lo planes [M][H * hd]
// (panel-packed when o_packed); f32 path: the *_lo pointers are unused.
hipError_t launch_attention(const void *q, const void *q_lo, const void *k_cache,
                            const void *k_cache_lo, const void *vt_cache, const void *vt_cache_lo,
                            RowSet rows, int n_heads, int n_kv_heads, int head_dim, bf16 *o_hi,
                            bf16 *o_lo, float *o_f32, float *part, int dtype, int o_packed,
                            hipStream_t st);
size_t attention_part_bytes(RowSet rows, int n_heads, int n_kv_heads, int head_dim, int dtype);
// Merge lm_head partials: tok, conf = 1/Z, p2 = exp(m2 - m1)/Z per row.
hipError_t launch_head_merge(const HeadPart *part, int n_rows, int n_vtiles, int *tok, float *conf,
                             float *p2, hipStream_t st);
// Schedule rules of the commit: early exit for converged tokens (exit_steps > 0) and first-step
// confidence scheduling (first_threshold >= 0); j is the step's index in its block, spb the
// block's step budget.  Per-position state [B][Bs] (argmax of the previous step, run length)
// and per-row state [B] (hard positions left after the first step) live in the workspace; the
// first step of a block starts them afresh.
struct CommitRules {
  int j, spb;
  int exit_steps;
  float exit_floor;
  float first_threshold;
  int *prev_tok, *run, *n_hard;
};
// Commit for each batch row over its block [s, s+Bs); per row, in cnt [4][B]: positions
// committed, masked positions left, masked positions whose confidence is NaN, 1 when the row's
// block ended by the early exit.
hipError_t launch_commit(int *x, int L, int B, int s, int Bs, const int *tok, const float *conf,
                         float threshold, int k_floor, int mask_id, uint8_t *committed, int *cnt,
                         const CommitRules &cr, hipStream_t st);
// x[b][p] = mask_id for P <= p < L (the prompt part is left as it is).
hipError_t launch_init_tokens(int *x, int B, int P, int L, int mask_id, hipStream_t st);
// cos/sin tables [L][hd/2] of theta = p * base^(-2i/hd), computed in fp64 on the device.
hipError_t launch_rope_table(float *cos_t, float *sin_t, int L, int hd, float base, hipStream_t st);
hipError_t launch_fill_u32(uint32_t *p, uint32_t v, size_t n, hipStream_t st);
// dst row b * n + j = src row b * src_stride + src_off + j for b < B, j < n (rows of row_bytes,
// a multiple of 16; src and dst must not overlap).
hipError_t launch_gather_rows(const void *src, void *dst, int B, int n, int src_stride,
                              int src_off, size_t row_bytes, hipStream_t st);
// Static device scratch (scratch.hip): the bytes of the file-scope array, and the device address
// of the current device's copy (looked up once per device).
static constexpr size_t STATIC_SCRATCH_BYTES = (size_t)256 << 20;
hipError_t static_scratch_address(void **ptr);

// Mark the mask id column (-inf) of debug logits rows.
hipError_t launch_mask_column(float *logits, int n_rows, int vocab, int mask_id, hipStream_t st);

}  // namespace dllm
