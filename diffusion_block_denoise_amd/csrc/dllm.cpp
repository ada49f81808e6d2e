// Host runtime behind include/dllm.h: configuration checks, workspace plan, the layer sequence
// of one forward over a row set, the block loop with its cache policy, and the C ABI.
//
// Decode (Fast-dLLM v1, block-wise with confidence-threshold parallel decoding and a KV cache
// refreshed at block boundaries):
//   prefill       x = [prompt | mask^G]; refresh of block 0
//   block_begin   full forward over every position of every batch row: all K/V cache slots are
//                 rewritten and the block rows' statistics serve the block's first step
//   denoise_step  statistics (kept from the refresh on a block's first step; otherwise a
//                 forward over the block rows (dual cache), the block and later rows (prefix
//                 cache) or all rows (no cache)), then the commit on the device
// Every step of the decode runs in the HIP kernels; the host only sequences launches and reads
// back the per-row remaining-mask counts (one small copy per step).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdlib>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/dllm.h"
#include "kernels.h"

using namespace dllm;

static_assert(STATIC_SCRATCH_BYTES == DLLM_STATIC_SCRATCH_BYTES, "static scratch size");

namespace {

std::string g_create_error;

constexpr size_t ALIGN = 256;
inline size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

// ------------------------------------------------------------------------------------------------
// Validation
int check_cfg(const dllm_cfg *c, std::string &msg) {
  auto bad = [&](const char *fmt, ...) {
    char buf[256];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    msg = buf;
    return DLLM_EINVAL;
  };
  if (!c) return bad("cfg is NULL");
  if (c->dtype != DLLM_F32 && c->dtype != DLLM_BF16) return bad("dtype must be DLLM_F32 or DLLM_BF16");
  if (c->n_layers < 1) return bad("n_layers must be >= 1");
  if (c->d_model < 1 || c->n_heads < 1 || c->n_kv_heads < 1 || c->ffn_dim < 1)
    return bad("d_model, n_heads, n_kv_heads and ffn_dim must be >= 1");
  if (c->n_heads % c->n_kv_heads) return bad("n_heads must be a multiple of n_kv_heads");
  if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128)
    return bad("head_dim must be 32, 64 or 128");
  if (c->vocab < 2) return bad("vocab must be >= 2");
  if (c->mask_id < 0 || c->mask_id >= c->vocab) return bad("mask_id must be in [0, vocab)");
  if (!(c->rms_eps >= 0.f) || !std::isfinite(c->rms_eps)) return bad("rms_eps must be finite and >= 0");
  if (!(c->rope_base > 0.f) || !std::isfinite(c->rope_base)) return bad("rope_base must be finite and > 0");
  if (!std::isfinite(c->logit_scale)) return bad("logit_scale must be finite");
  if (c->d_model % 64 || c->d_model > 8192) return bad("d_model must be a multiple of 64 and <= 8192");
  if (c->dtype == DLLM_BF16) {
    if ((c->n_heads * c->head_dim) % 64 || c->ffn_dim % 64)
      return bad("bf16: n_heads*head_dim and ffn_dim must be multiples of 64");
  }
  if (c->batch < 1) return bad("batch must be >= 1");
  if (c->prompt_len < 0) return bad("prompt_len must be >= 0");
  if (c->gen_length < 1 || c->block_size < 1) return bad("gen_length and block_size must be >= 1");
  if (c->block_size > 256) return bad("block_size must be <= 256");
  if (c->gen_length % c->block_size) return bad("gen_length must be a multiple of block_size");
  const int nb = c->gen_length / c->block_size;
  if (c->steps < 0) return bad("steps must be >= 0");
  const int steps = c->steps ? c->steps : c->gen_length;
  if (steps % nb) return bad("steps must be a multiple of gen_length/block_size (%d)", nb);
  if (std::isnan(c->threshold)) return bad("threshold is NaN");
  if (c->attention < 0 || c->attention > 1) return bad("attention must be 0 (full) or 1 (block-causal)");
  if (c->use_cache < 0 || c->use_cache > 2) return bad("use_cache must be 0, 1 or 2");
  if (c->exit_steps < 0) return bad("exit_steps must be >= 0");
  if (std::isnan(c->exit_floor)) return bad("exit_floor is NaN");
  if (std::isnan(c->first_threshold)) return bad("first_threshold is NaN");
  const long long L = (long long)c->prompt_len + c->gen_length;
  if (L * c->batch > (1LL << 26)) return bad("batch * (prompt_len + gen_length) too large");
  if (c->dtype == DLLM_F32 && L > 32768) return bad("f32: prompt_len + gen_length must be <= 32768");
  if ((long long)c->vocab * c->d_model >= (1LL << 40)) return bad("vocab * d_model too large");
  return DLLM_OK;
}

// ------------------------------------------------------------------------------------------------
// Workspace plan
struct Plan {
  int B, P, G, Bs, L, Lp, NB, spb, d, H, Hkv, hd, F, V, nq, nkv, dt;
  int W;       // suffix window (< 0: whole context)
  int causal;  // block-causal attention
  size_t Mmax;  // rows of the largest forward (B*L)
  size_t off_x, off_k, off_v, off_cos, off_sin, off_h, off_ahi, off_alo, off_acthi, off_actlo,
      off_q, off_apart, off_gpart, off_hpart, off_tok, off_conf, off_p2, off_com,
      off_cnt, off_sched, off_wpack, off_hc, off_qc, total;
  // The scratch region [off_scratch, total): partial results that live only within one launch
  // sequence (split-K tiles, attention key-chunk partials, lm_head tile partials).  The
  // static-scratch variant takes it from the library's static device array instead.
  size_t off_scratch;
  // packed bf16 weights (elements): per layer QKV, Wo, gate/up, down, then the lm_head
  int n_gu;  // virtual gate/up width (64 gate + 64 up rows per 128-row panel)
  size_t wp_qkv, wp_o, wp_gu, wp_down, wp_layer, wp_lm;
  size_t kv_layer_elems;  // K (or V) elements per layer
  int n_vtiles;
};

// Virtual width of the fused gate/up GEMM over M rows: gate and up rows interleaved per half tile.
int gateup_width(const Plan &p, int M) {
  const int bn = gemm_bn(M, p.dt);
  return 2 * ((p.F + bn / 2 - 1) / (bn / 2)) * (bn / 2);
}

// Rows [start, start + nR) of every batch row, over the full context.
RowSet rows_of(const Plan &p, int start, int nR) {
  RowSet r;
  r.B = p.B; r.L = p.L; r.Lp = p.Lp; r.start = start; r.nR = nR;
  r.Lx = p.L; r.tail = -1;
  r.causal = p.causal; r.P = p.P; r.Bs = p.Bs;
  return r;
}

// Context of block b (approximate suffix pruning, Streaming-dLLM): the prefix, the block, the
// W positions after it and the last position, compacted to slots [0, e + W] with the last
// position in slot e + W; the whole sequence when W < 0 or the window reaches the end.
int context_len(const Plan &p, int b, int *tail) {
  const int e = p.P + (b + 1) * p.Bs;
  if (p.causal) {  // block-causal: nothing after the block is visible to anyone
    *tail = -1;
    return e;
  }
  if (p.W < 0 || e + p.W >= p.L - 1) {
    *tail = -1;
    return p.L;
  }
  *tail = e + p.W;
  return e + p.W + 1;
}

RowSet rows_in_context(const Plan &p, int b, int start, int nR) {
  RowSet r = rows_of(p, start, nR);
  r.L = context_len(p, b, &r.tail);
  return r;
}

void make_plan(const dllm_cfg *c, Plan &p) {
  p.B = c->batch; p.P = c->prompt_len; p.G = c->gen_length; p.Bs = c->block_size;
  p.L = p.P + p.G; p.Lp = (p.L + 31) / 32 * 32; p.NB = p.G / p.Bs;
  const int steps = c->steps ? c->steps : p.G;
  p.spb = steps / p.NB;
  p.d = c->d_model; p.H = c->n_heads; p.Hkv = c->n_kv_heads; p.hd = c->head_dim;
  p.F = c->ffn_dim; p.V = c->vocab; p.nq = p.H * p.hd; p.nkv = p.Hkv * p.hd;
  p.dt = c->dtype == DLLM_BF16 ? 1 : 0;
  p.W = c->suffix_window;
  p.causal = c->attention == DLLM_ATTN_BLOCK_CAUSAL ? 1 : 0;
  const size_t Mmax = (size_t)p.B * p.L;
  p.Mmax = Mmax;
  p.kv_layer_elems = (size_t)p.B * p.Hkv * p.Lp * p.hd;

  // Row counts that a forward can have: refresh / no cache (B*L, or B*Lc_b with suffix
  // pruning, or two blocks with block-causal attention), dual step (B*Bs), prefix step of
  // block b (B*(L - s_b) or B*(Lc_b - s_b)).
  std::vector<int> Ms = {p.B * p.L, p.B * p.Bs};
  for (int b = 0; b < p.NB; ++b) {
    int tail;
    const int Lc = context_len(p, b, &tail), s0 = p.P + b * p.Bs;
    Ms.push_back(p.B * (p.L - s0));
    Ms.push_back(p.B * Lc);
    Ms.push_back(p.B * (Lc - s0));
    if (p.causal) Ms.push_back(p.B * (b > 0 ? 2 * p.Bs : p.P + p.Bs));  // block-causal refresh
  }
  size_t gpart = 0, apart = 0;
  for (int M : Ms) {
    const int shapes[4][2] = {{p.nq + 2 * p.nkv, p.d}, {p.d, p.nq}, {gateup_width(p, M), p.d}, {p.d, p.F}};
    for (auto &s : shapes) gpart = std::max(gpart, gemm_partial_bytes(M, s[0], s[1], p.dt));
    const int nR = M / p.B;
    apart = std::max(apart, attention_part_bytes(rows_of(p, 0, nR), p.H, p.Hkv, p.hd, p.dt));
  }
  // lm_head over the block rows (and the debug logits GEMM, same shape)
  {
    const int M = p.B * p.Bs, bn = gemm_bn(M, p.dt);
    p.n_vtiles = (p.V + bn - 1) / bn;
    gpart = std::max(gpart, gemm_partial_bytes(M, p.V, p.d, p.dt));
  }

  // packed copies of the bf16 linear weights (the GEMM W layout)
  p.n_gu = 2 * ((p.F + 63) / 64) * 64;
  p.wp_qkv = packed_rows(p.nq + 2 * p.nkv) * p.d;
  p.wp_o = packed_rows(p.d) * p.nq;
  p.wp_gu = packed_rows(p.n_gu) * p.d;
  p.wp_down = packed_rows(p.d) * p.F;
  p.wp_layer = p.wp_qkv + p.wp_o + p.wp_gu + p.wp_down;
  p.wp_lm = packed_rows(p.V) * p.d;

  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = align_up(o + bytes); return r; };
  p.off_wpack = take(p.dt ? (p.wp_layer * c->n_layers + p.wp_lm) * 2 : 0);
  p.off_x = take(Mmax * 4);
  // K and V^T caches, per layer: fp32, or a bf16 hi plane followed by a bf16 lo plane
  p.off_k = take(p.kv_layer_elems * c->n_layers * 4);
  p.off_v = take(p.kv_layer_elems * c->n_layers * 4);
  p.off_cos = take((size_t)p.L * (p.hd / 2) * 4);
  p.off_sin = take((size_t)p.L * (p.hd / 2) * 4);
  p.off_h = take(Mmax * p.d * 4);
  // GEMM input a: RMSNorm(h) [Mmax][d] or the attention output [Mmax][nq]; bf16 hi/lo planes,
  // or fp32 in the hi slot
  // (bf16 planes are panel-packed, 128-row panels, when their consumer GEMM runs on the
  // large-tile kernel: rows are allocated up to the next multiple of 128)
  const size_t wa = std::max(p.d, p.nq), Mpad = (Mmax + 127) / 128 * 128;
  p.off_ahi = take(Mpad * wa * (p.dt ? 2 : 4));
  p.off_alo = take(p.dt ? Mpad * wa * 2 : 0);
  p.off_acthi = take(Mpad * p.F * (p.dt ? 2 : 4));
  p.off_actlo = take(p.dt ? Mpad * p.F * 2 : 0);
  p.off_q = take(Mmax * p.nq * 4);  // fp32, or bf16 hi plane + lo plane
  p.off_tok = take((size_t)p.B * p.Bs * 4);
  p.off_conf = take((size_t)p.B * p.Bs * 4);
  p.off_p2 = take((size_t)p.B * p.Bs * 4);
  p.off_com = take((size_t)p.B * p.Bs);
  // per batch row: committed, remaining masked and NaN-confidence counts of the last step, and
  // whether it ended the row's block by the early exit
  p.off_cnt = take((size_t)4 * p.B * 4);
  // schedule-rule state: previous argmax and run per block position, hard positions per row
  p.off_sched = take(((size_t)2 * p.B * p.Bs + p.B) * 4);
  // the block rows' residual stream and queries in the last layer (forward)
  p.off_hc = take((size_t)p.B * p.Bs * p.d * 4);
  p.off_qc = take((size_t)p.B * p.Bs * p.nq * 4);
  // scratch region last, so that a workspace without it is a prefix of the full one
  p.off_scratch = o;
  p.off_apart = take(apart);
  p.off_gpart = take(gpart);
  p.off_hpart = take((size_t)p.B * p.Bs * p.n_vtiles * sizeof(HeadPart));
  p.total = o;
}

}  // namespace

// ------------------------------------------------------------------------------------------------
struct dllm_handle {
  dllm_cfg cfg;
  Plan p;
  hipStream_t st;
  const void *embed, *final_norm, *lm_head;
  std::vector<const void *> layer;
  char *ws;
  // carved buffers
  uint16_t *wpack;  // packed bf16 weights
  int *x;
  char *kc, *vc;
  float *cos_t, *sin_t, *h;
  float *hc;  // block rows' residual stream in the last layer
  void *qc;   // block rows' queries in the last layer (fp32, or bf16 hi plane + lo plane)
  void *a_hi, *a_lo, *act_hi, *act_lo, *q;
  float *apart, *gpart;
  HeadPart *hpart;
  int *tok;
  float *conf, *p2;
  uint8_t *com;
  int *cnt;  // [4][B]: committed, remaining masked, NaN confidences, early exit (last step)
  int *sched;  // [B][Bs] previous argmax, [B][Bs] run, [B] hard positions (schedule rules)
  // decode state
  bool have_tokens = false;
  int block = -1, j = 0;
  bool fresh = false;
  bool any_forward = false;
  RowSet last_rows{};
  dllm_stats stats{};
  std::vector<int> h_cnt;
  // [4][B] counts in pinned host memory, written by the commit kernel itself (handles made by
  // dllm_create; a static-scratch handle allocates nothing and copies cnt into h_cnt instead)
  int *h_cnt_pin = nullptr, *d_cnt_pin = nullptr;
  std::string err;
  // GPU time of the refreshes and steps: event pairs on the stream, read at the next
  // synchronisation (dllm_block_begin is asynchronous)
  hipEvent_t ev_ref[2] = {nullptr, nullptr}, ev_step[2] = {nullptr, nullptr};
  bool ref_pending = false;
  bool debug_sync = false;  // DLLM_DEBUG_SYNC: synchronise and check after every HIP call
  // per-kernel-class timing (dllm_set_profiling)
  struct Pending {
    int cls;
    hipEvent_t b, e;
    double bytes, flops;
  };
  int prof_mask = 0;
  std::vector<hipEvent_t> ev_pool;
  size_t ev_next = 0;
  std::vector<Pending> pending;
  dllm_kernel_prof prof[DLLM_KC_COUNT] = {};
  ~dllm_handle() {
    if (h_cnt_pin) (void)hipHostFree(h_cnt_pin);
    for (hipEvent_t e : ev_pool) (void)hipEventDestroy(e);
    for (hipEvent_t e : {ev_ref[0], ev_ref[1], ev_step[0], ev_step[1]})
      if (e) (void)hipEventDestroy(e);
  }
};

namespace {

// With DLLM_DEBUG_SYNC set (h->debug_sync) every call is followed by a stream synchronisation,
// so an asynchronous failure is reported by the call that caused it.
#define HIPCHK(expr)                                                                     \
  do {                                                                                   \
    hipError_t e_ = (expr);                                                              \
    if (e_ == hipSuccess && h->debug_sync) e_ = hipStreamSynchronize(h->st);             \
    if (e_ != hipSuccess) {                                                              \
      h->err = std::string(#expr) + ": " + hipGetErrorString(e_);                        \
      return DLLM_EHIP;                                                                  \
    }                                                                                    \
  } while (0)

inline const void *LW(dllm_t *h, int l, int j) { return h->layer[(size_t)9 * l + j]; }

// Packed bf16 weight of layer l: j = 0 QKV, 1 Wo, 2 gate/up, 3 down; l = n_layers: the lm_head.
const uint16_t *WP(dllm_t *h, int l, int j) {
  const Plan &p = h->p;
  if (!p.dt) return nullptr;
  const uint16_t *b = h->wpack + p.wp_layer * l;
  if (l == h->cfg.n_layers) return b;
  const size_t off[4] = {0, p.wp_qkv, p.wp_qkv + p.wp_o, p.wp_qkv + p.wp_o + p.wp_gu};
  return b + off[j];
}

// ---- per-kernel-class timing -------------------------------------------------------------------
// Collect the durations of the pending event pairs (the stream has been synchronised).
int prof_resolve(dllm_t *h) {
  for (const auto &pd : h->pending) {
    float ms = 0.f;
    HIPCHK(hipEventElapsedTime(&ms, pd.b, pd.e));
    dllm_kernel_prof &k = h->prof[pd.cls];
    k.launches++;
    k.ms += ms;
    k.bytes += pd.bytes;
    k.flops += pd.flops;
  }
  h->pending.clear();
  h->ev_next = 0;
  return DLLM_OK;
}

// Event pair for one launch of class cls, or nulls when that class is not being timed.
int prof_events(dllm_t *h, int cls, hipEvent_t *b, hipEvent_t *e) {
  *b = *e = nullptr;
  if (cls < 0 || !(h->prof_mask & (1 << cls))) return DLLM_OK;
  if (h->ev_next + 2 > h->ev_pool.size()) {
    HIPCHK(hipStreamSynchronize(h->st));
    int rc = prof_resolve(h);
    if (rc) return rc;
  }
  *b = h->ev_pool[h->ev_next++];
  *e = h->ev_pool[h->ev_next++];
  return DLLM_OK;
}

void prof_push(dllm_t *h, int cls, hipEvent_t b, hipEvent_t e, double bytes, double flops) {
  if (b) h->pending.push_back({cls, b, e, bytes, flops});
}

// Algorithmic work of a GEMM launch: each weight, A element and output element once.
void gemm_work(dllm_t *h, const GemmArgs &g, int n_real, double out_bytes, double &bytes,
               double &flops) {
  const double esz = h->p.dt ? 2.0 : 4.0;  // weight element
  bytes = (double)n_real * g.K * esz + (double)g.M * g.K * 4.0 + out_bytes;
  flops = 2.0 * g.M * n_real * g.K;
}

int gemm_class(dllm_t *h, const GemmArgs &g) {
  const int kind = gemm_kind(g.M, g.K, h->p.dt);
  return kind == 1 ? DLLM_KC_GEMM_SKINNY : (kind == 2 ? DLLM_KC_GEMM_TILED : -1);
}

// launch_gemm with the timing bracket of its class.
int run_gemm(dllm_t *h, const GemmArgs &g, int n_real, double out_bytes, int *splits) {
  const int cls = gemm_class(h, g);
  hipEvent_t b, e;
  int rc = prof_events(h, cls, &b, &e);
  if (rc) return rc;
  HIPCHK(launch_gemm(g, h->p.dt, h->st, splits, b, e));
  if (b) {
    double bytes, flops;
    gemm_work(h, g, n_real, out_bytes, bytes, flops);
    prof_push(h, cls, b, e, bytes, flops);
  }
  return DLLM_OK;
}

// Layer l of a cache: fp32 array, or (bf16) the hi plane; lo plane follows the hi plane.
void *kv_layer(dllm_t *h, char *base, int l) { return base + (size_t)l * h->p.kv_layer_elems * 4; }
void *kv_layer_lo(dllm_t *h, char *base, int l) {
  return (char *)kv_layer(h, base, l) + h->p.kv_layer_elems * 2;
}
void *q_lo(dllm_t *h) { return (char *)h->q + h->p.Mmax * h->p.nq * 2; }

// Whether the activations that feed an M x N x K GEMM are written panel-packed (the producer
// asks about its consumer's shape).
int a_packed(const dllm_t *h, int M, int N, int K) {
  return h->p.dt == 1 && gemm_a_packed(M, N, K, 1);
}

GemmArgs gemm_base(dllm_t *h, const void *a_hi, const void *a_lo, int lda, int M, int N, int K) {
  GemmArgs g;
  memset(&g, 0, sizeof g);
  if (h->p.dt) {
    g.a_hi = (const bf16 *)a_hi;
    g.a_lo = (const bf16 *)a_lo;
  } else {
    g.a_f32 = (const float *)a_hi;
  }
  g.lda = lda;
  g.a_packed = a_packed(h, M, N, K);
  g.M = M; g.N = N; g.K = K;
  g.partial = h->gpart;
  g.scale = 1.f;
  return g;
}

void set_resid(dllm_t *h, GemmArgs &g, float *hres) {
  g.epi = EPI_RESID;
  g.resid = hres;
  g.ld_out = h->p.d;
}

// Residual GEMM followed by the split-K fold and the next RMSNorm (gain) into a, which feeds a
// GEMM of next_m rows and next_n columns (K = d).
int resid_gemm_norm(dllm_t *h, GemmArgs &g, const void *gain, int next_m, int next_n) {
  const Plan &p = h->p;
  const bool bf = p.dt == 1;
  int splits = 1;
  int rc = run_gemm(h, g, g.N, 8.0 * g.M * g.N, &splits);  // h read and written
  if (rc) return rc;
  HIPCHK(launch_resid_norm(g.M, p.d, g.resid, splits > 1 ? h->gpart : nullptr, splits > 1 ? splits : 0,
                           gain, h->cfg.rms_eps, bf ? (bf16 *)h->a_hi : nullptr,
                           bf ? (bf16 *)h->a_lo : nullptr, bf ? nullptr : (float *)h->a_hi, p.dt,
                           a_packed(h, next_m, next_n, p.d), h->st));
  return DLLM_OK;
}

// One forward over row set rs.  Every layer's K/V are written for all rows of rs, but only the
// current block's rows feed the lm_head: after the last layer's Q/K/V projection the forward
// continues with the block rows alone (their queries and residual stream gathered into hc and
// qc).  Afterwards a holds RMSNorm(h) with the final-norm gain for the rows h->last_rows.
int forward(dllm_t *h, RowSet rs) {
  const Plan &p = h->p;
  const dllm_cfg &c = h->cfg;
  const bool bf = p.dt == 1;
  bf16 *ahi = (bf16 *)h->a_hi, *alo = (bf16 *)h->a_lo;
  float *af = (float *)h->a_hi;
  HIPCHK(launch_embed_norm(h->x, h->embed, LW(h, 0, 0), rs, p.d, c.rms_eps, h->h, bf ? ahi : nullptr,
                           bf ? alo : nullptr, bf ? nullptr : af, p.dt,
                           a_packed(h, rs.M(), p.nq + 2 * p.nkv, p.d),
                           h->st));
  const int s_blk = p.P + h->block * p.Bs;
  const bool narrow = h->block >= 0 && !(rs.start == s_blk && rs.nR == p.Bs) &&
                      rs.start <= s_blk && s_blk + p.Bs <= rs.start + rs.nR;
  RowSet lrs = rs;  // rows carried through the rest of the current layer
  float *hres = h->h;
  void *qb = h->q;
  for (int l = 0; l < c.n_layers; ++l) {
    const int Mq = rs.M();
    // Q, K, V projections of a; rotary embedding; K/V to the cache slots of rows rs
    {
      GemmArgs g = gemm_base(h, h->a_hi, h->a_lo, p.d, Mq, p.nq + 2 * p.nkv, p.d);
      g.w[0] = LW(h, l, 1); g.w[1] = LW(h, l, 2); g.w[2] = LW(h, l, 3);
      g.seg_end[0] = p.nq; g.seg_end[1] = p.nq + p.nkv; g.seg_end[2] = p.nq + 2 * p.nkv;
      g.wp = WP(h, l, 0);
      g.epi = EPI_QKV;
      g.rows = rs; g.n_heads = p.H; g.n_kv_heads = p.Hkv; g.head_dim = p.hd;
      g.rope_cos = h->cos_t; g.rope_sin = h->sin_t;
      g.q_out = h->q;
      g.k_cache = kv_layer(h, h->kc, l);
      g.vt_cache = kv_layer(h, h->vc, l);
      if (bf) {
        g.q_out_lo = q_lo(h);
        g.k_cache_lo = kv_layer_lo(h, h->kc, l);
        g.vt_cache_lo = kv_layer_lo(h, h->vc, l);
      }
      int rc = run_gemm(h, g, g.N, 4.0 * Mq * g.N, nullptr);  // q, K, V as 4-byte pairs
      if (rc) return rc;
    }
    if (l == c.n_layers - 1 && narrow) {
      // last layer: only the block rows go on (their K/V, and everyone else's, are written)
      lrs = rs;
      lrs.start = s_blk;
      lrs.nR = p.Bs;
      const int off = s_blk - rs.start, n = p.Bs;
      const size_t qrow = (size_t)p.nq * (bf ? 2 : 4);
      HIPCHK(launch_gather_rows(h->q, h->qc, p.B, n, rs.nR, off, qrow, h->st));
      if (bf)
        HIPCHK(launch_gather_rows(q_lo(h), (char *)h->qc + (size_t)p.B * n * qrow, p.B, n, rs.nR,
                                  off, qrow, h->st));
      HIPCHK(launch_gather_rows(h->h, h->hc, p.B, n, rs.nR, off, (size_t)p.d * 4, h->st));
      hres = h->hc;
      qb = h->qc;
    }
    const int M = lrs.M();
    const void *qb_lo = bf ? (qb == h->q ? q_lo(h) : (char *)h->qc + (size_t)M * p.nq * 2) : nullptr;
    // attention over all cached positions -> a (input of the output projection)
    {
      hipEvent_t eb, ee;
      int rc = prof_events(h, DLLM_KC_ATTENTION, &eb, &ee);
      if (rc) return rc;
      if (eb) HIPCHK(hipEventRecord(eb, h->st));
      HIPCHK(launch_attention(qb, qb_lo, kv_layer(h, h->kc, l),
                              bf ? kv_layer_lo(h, h->kc, l) : nullptr, kv_layer(h, h->vc, l),
                              bf ? kv_layer_lo(h, h->vc, l) : nullptr, lrs, p.H, p.Hkv, p.hd,
                              bf ? ahi : nullptr, bf ? alo : nullptr, bf ? nullptr : af, h->apart,
                              p.dt, a_packed(h, M, p.d, p.nq), h->st));
      if (ee) {
        HIPCHK(hipEventRecord(ee, h->st));
        // K and V of every cached position once per (batch row, K/V head), q in, o out
        const double kv = 2.0 * p.B * p.Hkv * (double)p.L * p.hd * 4.0;
        const double qo = 2.0 * M * p.nq * 4.0;
        prof_push(h, DLLM_KC_ATTENTION, eb, ee, kv + qo, 4.0 * M * p.H * (double)p.L * p.hd);
      }
    }
    // output projection + residual; a = ffn RMSNorm(h)
    {
      GemmArgs g = gemm_base(h, h->a_hi, h->a_lo, p.nq, M, p.d, p.nq);
      g.w[0] = LW(h, l, 4); g.seg_end[0] = p.d; g.seg_end[1] = g.seg_end[2] = p.d;
      g.wp = WP(h, l, 1);
      set_resid(h, g, hres);
      int rc = resid_gemm_norm(h, g, LW(h, l, 5), M, gateup_width(p, M));
      if (rc) return rc;
    }
    // gate/up + SwiGLU -> act
    {
      GemmArgs g = gemm_base(h, h->a_hi, h->a_lo, p.d, M, gateup_width(p, M), p.d);
      g.w[0] = LW(h, l, 6); g.w[1] = LW(h, l, 7);
      g.wp = WP(h, l, 2);
      g.n_half = p.F;
      g.epi = EPI_SWIGLU;
      g.ld_act = p.F;
      g.act_packed = a_packed(h, M, p.d, p.F);
      if (bf) { g.act_hi = (bf16 *)h->act_hi; g.act_lo = (bf16 *)h->act_lo; }
      else g.act_f32 = (float *)h->act_hi;
      int rc = run_gemm(h, g, 2 * p.F, 4.0 * M * p.F, nullptr);  // act as a 4-byte pair
      if (rc) return rc;
    }
    // down projection + residual; a = next layer's attention RMSNorm(h), or the final norm
    {
      GemmArgs g = gemm_base(h, h->act_hi, h->act_lo, p.F, M, p.d, p.F);
      g.w[0] = LW(h, l, 8); g.seg_end[0] = p.d; g.seg_end[1] = g.seg_end[2] = p.d;
      g.wp = WP(h, l, 3);
      set_resid(h, g, hres);
      // the next layer's Q/K/V projection takes rs's rows, the lm_head the block rows
      const bool last = l + 1 == c.n_layers;
      int rc = resid_gemm_norm(h, g, last ? h->final_norm : LW(h, l + 1, 0),
                               last ? p.B * p.Bs : rs.M(), last ? p.V : p.nq + 2 * p.nkv);
      if (rc) return rc;
    }
  }
  h->last_rows = lrs;
  h->any_forward = true;
  return DLLM_OK;
}

// A operand = the block rows of a after the last forward (final RMSNorm), rows 0..B*Bs-1.
void set_block_rows(dllm_t *h, GemmArgs &g) {
  const Plan &p = h->p;
  const RowSet rs = h->last_rows;
  g.row_per = p.Bs;
  g.row_stride = rs.nR;
  g.row_off = p.P + h->block * p.Bs - rs.start;
}

// Statistics of the block rows: fused lm_head + per-tile softmax partials, then the merge.
int head(dllm_t *h) {
  const Plan &p = h->p;
  const int M = p.B * p.Bs;
  GemmArgs g = gemm_base(h, h->a_hi, h->a_lo, p.d, M, p.V, p.d);
  set_block_rows(h, g);
  g.w[0] = h->lm_head; g.seg_end[0] = g.seg_end[1] = g.seg_end[2] = p.V;
  g.wp = WP(h, h->cfg.n_layers, 0);
  g.epi = EPI_LMHEAD;
  g.scale = h->cfg.logit_scale;
  g.head_part = h->hpart; g.n_vtiles = p.n_vtiles; g.vocab = p.V; g.mask_id = h->cfg.mask_id;
  int rc = run_gemm(h, g, p.V, (double)M * p.n_vtiles * sizeof(HeadPart), nullptr);
  if (rc) return rc;
  HIPCHK(launch_head_merge(h->hpart, M, p.n_vtiles, h->tok, h->conf, h->p2, h->st));
  return DLLM_OK;
}

int refresh(dllm_t *h) {
  int tail;
  const Plan &p = h->p;
  const int Lc = context_len(p, h->block, &tail);
  // block-causal: only the previous block (its tokens are now final; for block 0 the prompt)
  // and the current block; every earlier K/V is final
  const int r0 = p.causal && h->block > 0 ? p.P + (h->block - 1) * p.Bs : 0;
  int rc = forward(h, rows_in_context(p, h->block, r0, Lc - r0));
  if (rc) return rc;
  h->stats.full_forwards++;
  return head(h);
}

int floor_count(const Plan &p, int j) {
  const int base = p.Bs / p.spb, extra = p.Bs % p.spb;
  const int k = base + (j < extra ? 1 : 0);
  return k < 1 ? 1 : k;
}

int hist_bin(int n) {
  if (n <= 3) return n;
  if (n <= 4) return 3;
  if (n <= 8) return 4;
  if (n <= 16) return 5;
  if (n <= 32) return 6;
  if (n <= 64) return 7;
  return 8;
}

// Book the GPU time of an enqueued refresh into the stats once its end event has completed
// (wait: block until it has).
int resolve_refresh_time(dllm_t *h, bool wait) {
  if (!h->ref_pending) return DLLM_OK;
  if (!wait) {
    const hipError_t q = hipEventQuery(h->ev_ref[1]);
    if (q == hipErrorNotReady) return DLLM_OK;
    HIPCHK(q);
  } else {
    HIPCHK(hipEventSynchronize(h->ev_ref[1]));
  }
  float ms = 0.f;
  HIPCHK(hipEventElapsedTime(&ms, h->ev_ref[0], h->ev_ref[1]));
  h->stats.ms_refresh += ms;
  h->ref_pending = false;
  return DLLM_OK;
}

int do_block_begin(dllm_t *h, int b) {
  int rc = resolve_refresh_time(h, true);  // the event pair is reused
  if (rc) return rc;
  h->block = b;
  h->j = 0;
  HIPCHK(hipEventRecord(h->ev_ref[0], h->st));
  rc = refresh(h);
  if (rc) return rc;
  HIPCHK(hipEventRecord(h->ev_ref[1], h->st));
  h->ref_pending = true;
  h->fresh = true;
  return DLLM_OK;
}

int do_step(dllm_t *h, int32_t *n_committed, int32_t *block_done) {
  const Plan &p = h->p;
  int rc;
  HIPCHK(hipEventRecord(h->ev_step[0], h->st));
  if (!h->fresh) {
    const int s = p.P + h->block * p.Bs;
    if (h->cfg.use_cache == DLLM_NO_CACHE || h->cfg.refresh_every_step) {
      rc = refresh(h);
    } else {
      int tail;
      const int Lc = context_len(p, h->block, &tail);
      const int stop = h->cfg.use_cache == DLLM_DUAL_CACHE ? s + p.Bs : Lc;
      rc = forward(h, rows_in_context(p, h->block, s, stop - s));
      if (!rc) {
        h->stats.cached_forwards++;
        rc = head(h);
      }
    }
    if (rc) return rc;
  }
  h->fresh = false;
  const int s = p.P + h->block * p.Bs;
  CommitRules cr;
  cr.j = h->j;
  cr.spb = p.spb;
  cr.exit_steps = h->cfg.exit_steps;
  cr.exit_floor = h->cfg.exit_floor;
  cr.first_threshold = h->cfg.first_threshold;
  cr.prev_tok = h->sched;
  cr.run = h->sched + (size_t)p.B * p.Bs;
  cr.n_hard = h->sched + (size_t)2 * p.B * p.Bs;
  HIPCHK(launch_commit(h->x, p.L, p.B, s, p.Bs, h->tok, h->conf, h->cfg.threshold, floor_count(p, h->j),
                       h->cfg.mask_id, h->com, h->d_cnt_pin ? h->d_cnt_pin : h->cnt, cr, h->st));
  HIPCHK(hipEventRecord(h->ev_step[1], h->st));
  if (!h->d_cnt_pin)
    HIPCHK(hipMemcpyAsync(h->h_cnt.data(), h->cnt, (size_t)4 * p.B * 4, hipMemcpyDeviceToHost, h->st));
  HIPCHK(hipStreamSynchronize(h->st));
  const int *cnt = h->h_cnt_pin ? h->h_cnt_pin : h->h_cnt.data();
  if (!h->pending.empty()) {
    int prc = prof_resolve(h);
    if (prc) return prc;
  }
  rc = resolve_refresh_time(h, true);
  if (rc) return rc;
  float ms = 0.f;
  HIPCHK(hipEventElapsedTime(&ms, h->ev_step[0], h->ev_step[1]));
  h->stats.ms_step += ms;
  h->j++;
  h->stats.steps++;
  int done = 1;
  for (int b = 0; b < p.B; ++b) {
    const int nc = cnt[b], rem = cnt[p.B + b], nan = cnt[2 * p.B + b];
    h->stats.committed += nc;
    h->stats.commits_hist[hist_bin(nc)]++;
    h->stats.nan_count += nan;
    h->stats.early_exits += cnt[3 * p.B + b];
    if (rem) done = 0;
    if (n_committed) n_committed[b] = nc;
  }
  if (block_done) *block_done = done;
  return DLLM_OK;
}

}  // namespace

// ================================================================================================
extern "C" {

int dllm_validate_cfg(const dllm_cfg *cfg) {
  std::string m;
  return check_cfg(cfg, m);
}

int dllm_workspace_bytes(const dllm_cfg *cfg, size_t *bytes) {
  std::string m;
  int rc = check_cfg(cfg, m);
  if (rc) return rc;
  if (!bytes) return DLLM_EINVAL;
  Plan p;
  make_plan(cfg, p);
  *bytes = p.total;
  return DLLM_OK;
}

}  // extern "C"

namespace {

// dllm_create and its static-scratch variant: `scratch` is NULL (the scratch region is the end
// of the workspace) or the device address of the library's static array.
int create_handle(const dllm_weights *w, const dllm_cfg *cfg, void *workspace, size_t ws_bytes,
                  char *scratch, dllm_t **out) {
  if (!out) { g_create_error = "out is NULL"; return DLLM_EINVAL; }
  *out = nullptr;
  std::string m;
  int rc = check_cfg(cfg, m);
  if (rc) { g_create_error = m; return rc; }
  if (!w || !w->embed || !w->final_norm || !w->lm_head || !w->layer) {
    g_create_error = "weights: NULL pointer";
    return DLLM_EINVAL;
  }
  for (int i = 0; i < 9 * cfg->n_layers; ++i)
    if (!w->layer[i]) { g_create_error = "weights: NULL layer pointer"; return DLLM_EINVAL; }
  if (!workspace) { g_create_error = "workspace is NULL"; return DLLM_EINVAL; }
  if ((uintptr_t)workspace % ALIGN) { g_create_error = "workspace must be 256-byte aligned"; return DLLM_EINVAL; }
  Plan p;
  make_plan(cfg, p);
  const size_t need = scratch ? p.off_scratch : p.total;
  if (ws_bytes < need) {
    g_create_error = "workspace too small: need " + std::to_string(need) + " bytes";
    return DLLM_ENOSPACE;
  }
  dllm_t *h = new (std::nothrow) dllm_handle();
  if (!h) { g_create_error = "out of host memory"; return DLLM_EINTERNAL; }
  h->cfg = *cfg;
  h->p = p;
  h->st = (hipStream_t)cfg->stream;
  h->embed = w->embed; h->final_norm = w->final_norm; h->lm_head = w->lm_head;
  h->layer.assign(w->layer, w->layer + 9 * cfg->n_layers);
  char *ws = (char *)workspace;
  h->ws = ws;
  h->wpack = (uint16_t *)(ws + p.off_wpack);
  h->x = (int *)(ws + p.off_x);
  h->kc = ws + p.off_k; h->vc = ws + p.off_v;
  h->cos_t = (float *)(ws + p.off_cos); h->sin_t = (float *)(ws + p.off_sin);
  h->h = (float *)(ws + p.off_h);
  h->hc = (float *)(ws + p.off_hc);
  h->qc = ws + p.off_qc;
  h->a_hi = ws + p.off_ahi; h->a_lo = ws + p.off_alo;
  h->act_hi = ws + p.off_acthi; h->act_lo = ws + p.off_actlo;
  h->q = ws + p.off_q;
  // scratch region: the end of the workspace, or the static array at the same relative offsets
  char *sc = scratch ? scratch - p.off_scratch : ws;
  h->apart = (float *)(sc + p.off_apart);
  h->gpart = (float *)(sc + p.off_gpart);
  h->hpart = (HeadPart *)(sc + p.off_hpart);
  h->tok = (int *)(ws + p.off_tok);
  h->conf = (float *)(ws + p.off_conf); h->p2 = (float *)(ws + p.off_p2);
  h->com = (uint8_t *)(ws + p.off_com);
  h->cnt = (int *)(ws + p.off_cnt);
  h->sched = (int *)(ws + p.off_sched);
  h->h_cnt.assign((size_t)4 * p.B, 0);
  {
    const char *ds = getenv("DLLM_DEBUG_SYNC");
    h->debug_sync = ds && *ds && strcmp(ds, "0") != 0;
  }
  // Zero the K/V cache (its padding slots must hold zeros); rotary table.
  auto fail = [&](hipError_t e, const char *what) {
    g_create_error = std::string(what) + ": " + hipGetErrorString(e);
    delete h;
    return DLLM_EHIP;
  };
  hipError_t e;
  for (hipEvent_t *ev : {&h->ev_ref[0], &h->ev_ref[1], &h->ev_step[0], &h->ev_step[1]})
    if ((e = hipEventCreate(ev)) != hipSuccess) return fail(e, "event");
  if (!scratch) {
    // the step's counts go straight to pinned host memory (no copy command before the host
    // reads them); the static-scratch variant allocates nothing and keeps the copy
    if ((e = hipHostMalloc((void **)&h->h_cnt_pin, (size_t)4 * p.B * sizeof(int), hipHostMallocDefault)) != hipSuccess)
      return fail(e, "pinned counts");
    if ((e = hipHostGetDevicePointer((void **)&h->d_cnt_pin, h->h_cnt_pin, 0)) != hipSuccess)
      return fail(e, "pinned counts");
  }
  if ((e = launch_fill_u32((uint32_t *)h->kc, 0, (p.off_cos - p.off_k) / 4, h->st)) != hipSuccess)
    return fail(e, "zero cache");
  if ((e = launch_rope_table(h->cos_t, h->sin_t, p.L, p.hd, cfg->rope_base, h->st)) != hipSuccess)
    return fail(e, "rope table");
  // Packed copies of the bf16 linear weights; the originals are not read again.
  if (p.dt) {
    for (int l = 0; l < cfg->n_layers; ++l) {
      const void *qkv[3] = {LW(h, l, 1), LW(h, l, 2), LW(h, l, 3)};
      const int qkv_end[3] = {p.nq, p.nq + p.nkv, p.nq + 2 * p.nkv};
      const void *o[3] = {LW(h, l, 4), nullptr, nullptr};
      const int o_end[3] = {p.d, p.d, p.d};
      const void *gu[3] = {LW(h, l, 6), LW(h, l, 7), nullptr};
      const int gu_end[3] = {p.n_gu, p.n_gu, p.n_gu};
      const void *dn[3] = {LW(h, l, 8), nullptr, nullptr};
      if ((e = launch_pack_weight((uint16_t *)WP(h, l, 0), qkv, qkv_end, 0, PACK_CONCAT, p.nq + 2 * p.nkv,
                                  p.d, h->st)) != hipSuccess ||
          (e = launch_pack_weight((uint16_t *)WP(h, l, 1), o, o_end, 0, PACK_PLAIN, p.d, p.nq, h->st)) !=
              hipSuccess ||
          (e = launch_pack_weight((uint16_t *)WP(h, l, 2), gu, gu_end, p.F, PACK_SWIGLU, p.n_gu, p.d,
                                  h->st)) != hipSuccess ||
          (e = launch_pack_weight((uint16_t *)WP(h, l, 3), dn, o_end, 0, PACK_PLAIN, p.d, p.F, h->st)) !=
              hipSuccess)
        return fail(e, "pack weights");
    }
    const void *lm[3] = {h->lm_head, nullptr, nullptr};
    const int lm_end[3] = {p.V, p.V, p.V};
    if ((e = launch_pack_weight((uint16_t *)WP(h, cfg->n_layers, 0), lm, lm_end, 0, PACK_PLAIN, p.V, p.d,
                                h->st)) != hipSuccess)
      return fail(e, "pack lm_head");
  }
  if ((e = hipStreamSynchronize(h->st)) != hipSuccess) return fail(e, "synchronize");
  *out = h;
  return DLLM_OK;
}

}  // namespace

extern "C" {

int dllm_create(const dllm_weights *w, const dllm_cfg *cfg, void *workspace, size_t ws_bytes,
                dllm_t **out) {
  return create_handle(w, cfg, workspace, ws_bytes, nullptr, out);
}

int dllm_create_static_scratch(const dllm_weights *w, const dllm_cfg *cfg, void *workspace,
                               size_t *ws_bytes, dllm_t **out) {
  if (!ws_bytes) { g_create_error = "ws_bytes is NULL"; return DLLM_EINVAL; }
  std::string m;
  int rc = check_cfg(cfg, m);
  if (rc) { g_create_error = m; return rc; }
  Plan p;
  make_plan(cfg, p);
  const size_t sbytes = p.total - p.off_scratch;
  if (sbytes > STATIC_SCRATCH_BYTES) {
    g_create_error = "static scratch too small for this configuration: need " +
                     std::to_string(sbytes) + " bytes, the array holds " +
                     std::to_string((size_t)STATIC_SCRATCH_BYTES);
    return DLLM_ENOSPACE;
  }
  if (!workspace) {  // size query (host only)
    *ws_bytes = p.off_scratch;
    return DLLM_OK;
  }
  void *sp = nullptr;
  const hipError_t e = static_scratch_address(&sp);
  if (e != hipSuccess) {
    g_create_error = std::string("static scratch address: ") + hipGetErrorString(e);
    return DLLM_EHIP;
  }
  return create_handle(w, cfg, workspace, *ws_bytes, (char *)sp, out);
}

int dllm_prefill(dllm_t *h, const int32_t *prompt) {
  if (!h) return DLLM_EINVAL;
  const Plan &p = h->p;
  if (!prompt && p.P > 0) { h->err = "prompt is NULL"; return DLLM_EINVAL; }
  for (size_t i = 0; i < (size_t)p.B * p.P; ++i)
    if (prompt[i] < 0 || prompt[i] >= p.V) { h->err = "prompt id out of range"; return DLLM_EINVAL; }
  if (p.P > 0)
    HIPCHK(hipMemcpy2DAsync(h->x, (size_t)p.L * 4, prompt, (size_t)p.P * 4, (size_t)p.P * 4, p.B,
                            hipMemcpyHostToDevice, h->st));
  HIPCHK(launch_init_tokens(h->x, p.B, p.P, p.L, h->cfg.mask_id, h->st));
  h->have_tokens = true;
  int rc = resolve_refresh_time(h, true);  // a refresh still in flight belongs to the old run
  if (rc) return rc;
  h->stats = dllm_stats{};
  rc = do_block_begin(h, 0);
  if (rc) return rc;
  HIPCHK(hipStreamSynchronize(h->st));
  return resolve_refresh_time(h, true);
}

int dllm_block_begin(dllm_t *h, int32_t block) {
  if (!h) return DLLM_EINVAL;
  if (!h->have_tokens) { h->err = "block_begin before prefill or set_tokens"; return DLLM_ESTATE; }
  if (block < 0 || block >= h->p.NB) { h->err = "block out of range"; return DLLM_EINVAL; }
  return do_block_begin(h, block);
}

int dllm_denoise_step(dllm_t *h, int32_t *n_committed, int32_t *block_done) {
  if (!h) return DLLM_EINVAL;
  if (!h->have_tokens || h->block < 0) { h->err = "denoise_step before block_begin"; return DLLM_ESTATE; }
  return do_step(h, n_committed, block_done);
}

int dllm_generate(dllm_t *h, const int32_t *prompt, int32_t *out, dllm_stats *stats) {
  if (!h) return DLLM_EINVAL;
  int rc = dllm_prefill(h, prompt);  // resets the counters
  if (rc) return rc;
  const int max_steps = h->p.G + h->p.NB;
  int steps = 0;
  for (int b = 0; b < h->p.NB; ++b) {
    if (b > 0 && (rc = do_block_begin(h, b))) return rc;
    int done = 0;
    while (!done) {
      if ((rc = do_step(h, nullptr, &done))) return rc;
      if (++steps > max_steps) { h->err = "step limit exceeded"; return DLLM_EINTERNAL; }
    }
  }
  if (out) {
    HIPCHK(hipMemcpyAsync(out, h->x, (size_t)h->p.B * h->p.L * 4, hipMemcpyDeviceToHost, h->st));
    HIPCHK(hipStreamSynchronize(h->st));
  }
  if (stats) *stats = h->stats;
  return DLLM_OK;
}

int dllm_get_tokens(dllm_t *h, int32_t *x) {
  if (!h || !x) return DLLM_EINVAL;
  HIPCHK(hipMemcpyAsync(x, h->x, (size_t)h->p.B * h->p.L * 4, hipMemcpyDeviceToHost, h->st));
  HIPCHK(hipStreamSynchronize(h->st));
  return DLLM_OK;
}

int dllm_set_tokens(dllm_t *h, const int32_t *x) {
  if (!h || !x) return DLLM_EINVAL;
  const size_t n = (size_t)h->p.B * h->p.L;
  for (size_t i = 0; i < n; ++i)
    if (x[i] < 0 || x[i] >= h->p.V) { h->err = "token id out of range"; return DLLM_EINVAL; }
  HIPCHK(hipMemcpyAsync(h->x, x, n * 4, hipMemcpyHostToDevice, h->st));
  HIPCHK(hipStreamSynchronize(h->st));
  h->have_tokens = true;
  return DLLM_OK;
}

int dllm_get_step_info(dllm_t *h, int32_t *tok, float *conf, float *p2, uint8_t *committed) {
  if (!h) return DLLM_EINVAL;
  if (!h->any_forward) { h->err = "no forward yet"; return DLLM_ESTATE; }
  const size_t n = (size_t)h->p.B * h->p.Bs;
  if (tok) HIPCHK(hipMemcpyAsync(tok, h->tok, n * 4, hipMemcpyDeviceToHost, h->st));
  if (conf) HIPCHK(hipMemcpyAsync(conf, h->conf, n * 4, hipMemcpyDeviceToHost, h->st));
  if (p2) HIPCHK(hipMemcpyAsync(p2, h->p2, n * 4, hipMemcpyDeviceToHost, h->st));
  if (committed) HIPCHK(hipMemcpyAsync(committed, h->com, n, hipMemcpyDeviceToHost, h->st));
  HIPCHK(hipStreamSynchronize(h->st));
  return DLLM_OK;
}

int dllm_debug_block_logits(dllm_t *h, float *logits_dev) {
  if (!h || !logits_dev) return DLLM_EINVAL;
  if (!h->any_forward) { h->err = "no forward yet"; return DLLM_ESTATE; }
  const Plan &p = h->p;
  const int M = p.B * p.Bs;
  GemmArgs g = gemm_base(h, h->a_hi, h->a_lo, p.d, M, p.V, p.d);
  set_block_rows(h, g);
  g.w[0] = h->lm_head; g.seg_end[0] = g.seg_end[1] = g.seg_end[2] = p.V;
  g.wp = WP(h, h->cfg.n_layers, 0);
  g.epi = EPI_STORE; g.out_f32 = logits_dev; g.ld_out = p.V; g.scale = h->cfg.logit_scale;
  HIPCHK(launch_gemm(g, p.dt, h->st, nullptr));
  HIPCHK(launch_mask_column(logits_dev, M, p.V, h->cfg.mask_id, h->st));
  HIPCHK(hipStreamSynchronize(h->st));
  return DLLM_OK;
}

int dllm_get_stats(dllm_t *h, dllm_stats *stats) {
  if (!h || !stats) return DLLM_EINVAL;
  int rc = resolve_refresh_time(h, true);
  if (rc) return rc;
  *stats = h->stats;
  return DLLM_OK;
}

int dllm_set_profiling(dllm_t *h, int class_mask) {
  if (!h) return DLLM_EINVAL;
  if (class_mask & ~((1 << DLLM_KC_COUNT) - 1)) { h->err = "unknown kernel class"; return DLLM_EINVAL; }
  HIPCHK(hipStreamSynchronize(h->st));
  h->pending.clear();
  h->ev_next = 0;
  for (auto &k : h->prof) k = dllm_kernel_prof{};
  if (class_mask && h->ev_pool.empty()) {
    h->ev_pool.resize(4096);
    for (auto &e : h->ev_pool) HIPCHK(hipEventCreate(&e));
  }
  h->prof_mask = class_mask;
  return DLLM_OK;
}

int dllm_get_profile(dllm_t *h, dllm_kernel_prof *out) {
  if (!h || !out) return DLLM_EINVAL;
  HIPCHK(hipStreamSynchronize(h->st));
  int rc = prof_resolve(h);
  if (rc) return rc;
  for (int i = 0; i < DLLM_KC_COUNT; ++i) out[i] = h->prof[i];
  return DLLM_OK;
}

int dllm_get_position(dllm_t *h, int32_t *block, int32_t *step) {
  if (!h) return DLLM_EINVAL;
  if (block) *block = h->block;
  if (step) *step = h->j;
  return DLLM_OK;
}

const char *dllm_last_error(const dllm_t *h) {
  return h ? h->err.c_str() : g_create_error.c_str();
}

void dllm_destroy(dllm_t *h) { delete h; }

}  // extern "C"
