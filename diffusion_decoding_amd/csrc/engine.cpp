// Step engine and C ABI of the block-diffusion denoise library.
//
// One denoise step (DiffusionGemma解析, "换个路数：整片并行去噪的生成机制"; ipcmen.com,
// "工作原理：并行精炼与自我修正"): embed the canvas, run every layer with
// bidirectional attention over [prompt KV ; canvas KV] and the routed + shared
// expert FFN (zhichai.net 深度拆解, "MoE 效率"), apply the final RMSNorm, score
// every position with the fused LM head (entropy + argmax), commit, re-noise.
// The causal commit pass appends a finished canvas to the KV cache
// (zhichai.net 深度拆解, "Block-Autoregressive").  All workspace is allocated
// once at model creation; steps allocate nothing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/dg.h"
#include "kernels.h"

using namespace dg;

namespace {

thread_local std::string g_err;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return status;
}

#define HIP_OK(expr)                                                                        \
  do {                                                                                      \
    int _e = int(expr);                                                                     \
    if (_e) return fail(DG_ERR_HIP, "%s failed: %s (%d)", #expr,                           \
                        hipGetErrorString(hipError_t(_e)), _e);                             \
  } while (0)

}  // namespace

struct dg_model {
  dg_config cfg{};
  std::vector<dg_layer_weights> layers;
  const void* embed = nullptr;
  const void* lm_head = nullptr;
  int max_batch = 0, max_tokens = 0, max_kv = 0;
  int Tmax = 0;  // max_batch * max(max_tokens, canvas_len)
  size_t esz = 0;
  ActType at = ACT_BF16;
  WType wt = W_BF16;   // routed experts
  WType wt_gu = W_BF16;  // routed gate/up (W_FP4A8: MXFP8 token rows)
  WType swt = W_BF16;  // shared expert
  std::vector<void*> allocs;
  // workspace
  void *x = nullptr, *a = nullptr, *qkv = nullptr, *q = nullptr, *kc = nullptr, *vc = nullptr,
       *o = nullptr, *h = nullptr, *hs = nullptr;
  float *attn_po = nullptr, *attn_ml = nullptr;
  void* perm_scratch = nullptr;  // the routing permutation's masks and prefixes above 2048 tokens
  uint8_t* q8 = nullptr;  // MXFP8 experts: the normed rows' codes [Tmax][d], then scales [Tmax][d/32]
  int attn_max_splits = 8;
  float *rlog = nullptr, *topk_w = nullptr, *y = nullptr, *ys = nullptr, *lm_part = nullptr;
  float* rope_tab = nullptr;  // [max_tokens][head_dim / 2] (cos, sin) of the current positions
  int *topk_ids = nullptr, *off = nullptr, *pair_row = nullptr, *pos = nullptr;
  int lm_ntiles = 0;
  float *H = nullptr, *gap = nullptr;
  int* am = nullptr;
  // ctl[0]: status word published by the last step's commit kernel; ctl[1]:
  // flags raised by the kernels since then; ctl[2 .. 2 + max_batch): the
  // per-canvas uncommitted counts.  One copy brings status and counts back.
  int* ctl = nullptr;
  int* n_unc = nullptr;
  int* u_host = nullptr;  // pinned, 2 + max_batch words
  const int* force_ids = nullptr;  // test hook: [n_layers][max_batch * canvas_len][top_k], -1 = not forced
  int* diag_counts = nullptr;      // [n_layers][n_experts] for the step in progress, or null
  // kernel timing
  int prof_id = DG_PROF_NONE;
  std::vector<hipEvent_t> prof_ev;  // start/stop pairs
  int prof_n = 0;
  double prof_ms = 0.0;
  long long prof_launches = 0;
};

namespace {

int alloc(dg_model* m, void** p, size_t bytes) {
  if (bytes == 0) bytes = 16;
  if (hipMalloc(p, bytes) != hipSuccess) {
    (void)hipGetLastError();
    return fail(DG_ERR_OOM, "hipMalloc(%zu) failed", bytes);
  }
  m->allocs.push_back(*p);
  return DG_OK;
}

void free_all(dg_model* m) {
  for (hipEvent_t e : m->prof_ev) (void)hipEventDestroy(e);
  m->prof_ev.clear();
  for (void* p : m->allocs) (void)hipFree(p);
  m->allocs.clear();
  if (m->u_host) (void)hipHostFree(m->u_host);
  m->u_host = nullptr;
}

constexpr int PROF_PAIRS = 1024;

// Accumulate the recorded pairs (waits for the last stop event) and reset.
int prof_drain(dg_model* m) {
  if (m->prof_n == 0) return DG_OK;
  HIP_OK(hipEventSynchronize(m->prof_ev[2 * (m->prof_n - 1) + 1]));
  for (int i = 0; i < m->prof_n; ++i) {
    float ms = 0.f;
    HIP_OK(hipEventElapsedTime(&ms, m->prof_ev[2 * i], m->prof_ev[2 * i + 1]));
    m->prof_ms += ms;
  }
  m->prof_launches += m->prof_n;
  m->prof_n = 0;
  return DG_OK;
}

// Brackets the launches of one kernel class with events when it is selected.
struct ProfScope {
  dg_model* m;
  hipStream_t st;
  bool on;
  ProfScope(dg_model* m_, int id, hipStream_t st_) : m(m_), st(st_), on(m_->prof_id == id) {
    if (on && m->prof_n >= PROF_PAIRS) on = prof_drain(m) == DG_OK;
    if (on) on = hipEventRecord(m->prof_ev[2 * m->prof_n], st) == hipSuccess;
  }
  ~ProfScope() {
    if (on && hipEventRecord(m->prof_ev[2 * m->prof_n + 1], st) == hipSuccess) m->prof_n++;
  }
};

int check_config(const dg_config& c) {
  if (c.n_layers <= 0 || c.d_model <= 0 || c.n_heads <= 0 || c.head_dim <= 0 || c.n_experts <= 0 ||
      c.top_k <= 0 || c.d_expert <= 0 || c.d_shared <= 0 || c.vocab <= 0 || c.canvas_len <= 0 ||
      c.max_steps <= 0)
    return fail(DG_ERR_INVALID_ARG, "config fields must be positive");
  if (c.act_dtype != DG_DTYPE_FP32 && c.act_dtype != DG_DTYPE_BF16)
    return fail(DG_ERR_INVALID_ARG, "act_dtype must be FP32 or BF16");
  if (c.act_dtype == DG_DTYPE_FP32 && c.expert_dtype != DG_DTYPE_FP32)
    return fail(DG_ERR_INVALID_ARG, "FP32 activations need FP32 experts");
  if (c.act_dtype == DG_DTYPE_BF16 && c.expert_dtype != DG_DTYPE_BF16 && c.expert_dtype != DG_DTYPE_FP8_E4M3 &&
      c.expert_dtype != DG_DTYPE_MXFP4 && c.expert_dtype != DG_DTYPE_MXFP4_MXFP8)
    return fail(DG_ERR_INVALID_ARG, "BF16 activations need BF16, FP8_E4M3, MXFP4 or MXFP4_MXFP8 experts");
  if ((c.expert_dtype == DG_DTYPE_MXFP4 || c.expert_dtype == DG_DTYPE_MXFP4_MXFP8) &&
      (c.d_model % 64 || c.d_expert % 64))
    return fail(DG_ERR_SHAPE, "MXFP4 experts need d_model and d_expert multiples of 64");
  if (c.expert_dtype == DG_DTYPE_MXFP4_MXFP8 && c.d_model % 128)
    return fail(DG_ERR_SHAPE, "MXFP4_MXFP8 experts need d_model a multiple of 128");
  const int A = c.n_heads * c.head_dim;
  if (c.d_model % 32 || A % 32 || c.d_expert % 32 || c.d_shared % 32)
    return fail(DG_ERR_SHAPE, "d_model, n_heads*head_dim, d_expert, d_shared must be multiples of 32");
  const bool bf = c.act_dtype == DG_DTYPE_BF16;
  const int dh = c.head_dim;
  if (!(dh == 128 || dh == 64 || dh == 32 || (!bf && dh == 16)))
    return fail(DG_ERR_SHAPE, "head_dim %d unsupported (bf16: 32/64/128, fp32: 16/32/64/128)", dh);
  if (c.n_experts > 256 || c.top_k > 8 || c.top_k > c.n_experts)
    return fail(DG_ERR_SHAPE, "need n_experts <= 256 and top_k <= min(8, n_experts)");
  if (c.canvas_len > 1024) return fail(DG_ERR_SHAPE, "canvas_len must be <= 1024");
  if (!(c.rope_theta >= 0.f) || !(c.rms_eps >= 0.f))
    return fail(DG_ERR_INVALID_ARG, "rope_theta and rms_eps must be >= 0");
  if (c.mask_token < -1 || c.mask_token >= c.vocab)
    return fail(DG_ERR_INVALID_ARG, "mask_token %d must be -1 (uniform noise) or a vocabulary id", c.mask_token);
  if (c.self_condition != 0 && c.self_condition != 1)
    return fail(DG_ERR_INVALID_ARG, "self_condition must be 0 or 1");
  return DG_OK;
}

// ---- phases of a block (shared by the step, the causal pass and the
// test entries, which pass their own buffers)

// rotary embedding applies in the QKV projection's epilogue (bf16, head_dim
// 128, K a multiple of 64); otherwise a separate kernel rotates and scatters
bool fused_rope(const dg_model* m) {
  return m->at == ACT_BF16 && m->cfg.head_dim == 128 && tgemm_supported(m->at, m->cfg.d_model);
}

// q, k, v of the T = B * n rows of a (normed, act_dtype [T][d_model]) at the
// positions whose (cos, sin) rows m->rope_tab holds: q -> q_out
// [B][H][n][dh]; k, v -> (b, h) planes of k_dst / v_dst (dst_bh elements
// apart), rows row0 + i.  Rotary-embedded q and k.
int qkv_rope(dg_model* m, int l, const void* a, int B, int n, void* q_out, void* k_dst, void* v_dst,
             long long dst_bh, int row0, hipStream_t st) {
  const dg_config& c = m->cfg;
  const int T = B * n, d = c.d_model, H = c.n_heads, dh = c.head_dim, A = H * dh;
  const dg_layer_weights& w = m->layers[l];
  GemmArgs g;
  g.A = a; g.lda = d; g.B = w.wqkv; g.ldb = d; g.M = T; g.N = 3 * A; g.K = d;
  if (fused_rope(m)) {
    g.q_out = q_out; g.seq_n = n; g.heads = H; g.rope_tab = m->rope_tab;
    g.k_dst = k_dst; g.v_dst = v_dst; g.dst_bh = dst_bh; g.row0 = row0;
    HIP_OK(gemm(m->at, W_BF16, EPI_QKV, g, 1, st));
    return DG_OK;
  }
  g.C = m->qkv; g.ldc = 3 * A;
  HIP_OK(gemm(m->at, m->at == ACT_BF16 ? W_BF16 : W_F32, EPI_ACT, g, 1, st));
  HIP_OK(rope_scatter(m->at, m->qkv, B, n, H, dh, m->rope_tab, q_out, k_dst, v_dst, dst_bh, row0, st));
  return DG_OK;
}

// Attention of the B x n queries q [B][H][n][dh] into o [B*n][H*dh]:
// bidirectional over cache rows [0, P) of `layer` plus the canvas keys and
// values kc / vc [B][H][n][dh]; causal (kc null): over cache rows [0, P + n)
// with query i seeing rows j <= P + i.
AttnArgs attn_args(const dg_model* m, int l, const void* q, const dg_kv* kv, int P, const void* kc, const void* vc,
                   int B, int n, void* o, long long plane) {
  const dg_config& c = m->cfg;
  const int H = c.n_heads, dh = c.head_dim;
  const long long cap = kv->capacity;
  const long long layer_stride = (long long)kv->batch * H * cap * dh;
  AttnArgs aa{};
  // q and the canvas keys/values: (b, h) planes `plane` elements apart (n * dh: packed)
  if (plane == 0) plane = (long long)n * dh;
  aa.q = q; aa.q_bh = plane; aa.B = B; aa.H = H; aa.n = n; aa.dh = dh; aa.out = o;
  aa.part_o = m->attn_po; aa.part_ml = m->attn_ml;
  aa.k0 = (const char*)kv->k + l * layer_stride * m->esz;
  aa.v0 = (const char*)kv->v + l * layer_stride * m->esz;
  aa.s0_bh = cap * dh;
  if (kc) {
    aa.len0 = P;
    aa.k1 = kc; aa.v1 = vc; aa.s1_bh = plane; aa.len1 = n;
    aa.causal_base = -1;
  } else {
    aa.len0 = P + n;
    aa.k1 = nullptr; aa.v1 = nullptr; aa.s1_bh = 0; aa.len1 = 0;
    aa.causal_base = P;
  }
  aa.splits = std::min(m->attn_max_splits, attn_splits_for(m->at, B, H, n, aa.len0 + aa.len1, dh));
  return aa;
}

int attend(dg_model* m, int l, const void* q, const dg_kv* kv, int P, const void* kc, const void* vc, int B, int n,
           void* o, hipStream_t st, long long plane = 0) {
  HIP_OK(attention(m->at, attn_args(m, l, q, kv, P, kc, vc, B, n, o, plane), st));
  return DG_OK;
}

// shared gate/up + SwiGLU of b [T][d_model] into hs [T][d_shared]; where the
// bf16 direct-load kernel covers it, the router logits (the same rows
// against the E router rows) ride in the same launch as extra tiles and go
// to rlog [T][E] (*router_done = true).
int shared_gate_up(dg_model* m, int l, const void* b, int T, void* hs, float* rlog, bool* router_done,
                   hipStream_t st) {
  const dg_config& c = m->cfg;
  const dg_layer_weights& w = m->layers[l];
  const int d = c.d_model, ds = c.d_shared;
  GemmArgs g;
  g.A = b; g.lda = d; g.B = w.ws_gu; g.ldb = d; g.b_scale = w.ss_gu;
  g.M = T; g.N = ds; g.K = d; g.C = hs; g.ldc = ds; g.swiglu_half = ds;
  int r = int(hipErrorInvalidValue);
  *router_done = false;
  if (m->at == ACT_BF16 && m->swt == W_BF16) {
    GemmArgs gf = g;
    gf.B2 = w.wr; gf.ldb2 = d; gf.N2 = c.n_experts; gf.C2 = rlog; gf.ldc2 = c.n_experts;
    r = gemm(m->at, m->swt, EPI_SWIGLU, gf, 1, st);
    *router_done = r == int(hipSuccess);
  }
  if (r == int(hipErrorInvalidValue)) r = gemm(m->at, m->swt, EPI_SWIGLU, g, 1, st);
  HIP_OK(r);
  return DG_OK;
}

// shared down: ys [T][d_model] (fp32) = hs [T][d_shared] . W_down^T.  With
// rlog (the router logits, already computed), the router top-k into
// m->topk_ids / m->topk_w rides in the same launch where the bf16 kernel
// covers the shape (*topk_done = true): both read only what the shared
// gate/up launch wrote, and the top-k workgroups run beside the product's
// tiles instead of in a launch of their own.
int shared_down(dg_model* m, int l, const void* hs, int T, float* ys, hipStream_t st, const float* rlog = nullptr,
                bool* topk_done = nullptr) {
  const dg_config& c = m->cfg;
  const dg_layer_weights& w = m->layers[l];
  GemmArgs g;
  g.A = hs; g.lda = c.d_shared; g.B = w.ws_d; g.ldb = c.d_shared; g.b_scale = w.ss_d;
  g.M = T; g.N = c.d_model; g.K = c.d_shared; g.C = ys; g.ldc = c.d_model;
  if (rlog && topk_done && m->at == ACT_BF16 && m->swt == W_BF16) {
    GemmArgs gt = g;
    gt.tk_logits = rlog; gt.tk_T = T; gt.tk_E = c.n_experts; gt.tk_k = c.top_k;
    gt.tk_ids = m->topk_ids; gt.tk_w = m->topk_w;
    const int r = gemm_f32_topk(gt, st);
    if (r >= 0) {
      HIP_OK(r);
      *topk_done = true;
      return DG_OK;
    }
  }
  HIP_OK(gemm(m->at, m->swt, EPI_F32, g, 1, st));
  return DG_OK;
}

// router: logits rlog [T][E] of b (unless the shared launch computed them),
// top-k ids [T][k] and weights (unless the shared-down launch computed
// them); `forced` (test hook, nullable) overrides rows.
int route(dg_model* m, int l, const void* b, int T, float* rlog, bool logits_done, int* ids, float* wts,
          const int* forced, hipStream_t st, bool topk_done = false) {
  const dg_config& c = m->cfg;
  const int E = c.n_experts, k = c.top_k, d = c.d_model;
  if (!logits_done) {
    GemmArgs g;
    g.A = b; g.lda = d; g.B = m->layers[l].wr; g.ldb = d; g.M = T; g.N = E; g.K = d; g.C = rlog; g.ldc = E;
    HIP_OK(gemm(m->at, m->at == ACT_BF16 ? W_BF16 : W_F32, EPI_F32, g, 1, st));
  }
  if (!topk_done) HIP_OK(router_topk(rlog, T, E, k, ids, wts, st));
  if (forced) HIP_OK(router_force(rlog, T, E, k, forced, ids, wts, st));
  return DG_OK;
}

// Whether a T-row pass takes the grouped gate/up path: from 24 pairs per
// expert on average (and whenever routing piles onto few experts, as under
// absorbing noise) the gate/up is a grouped GEMM of 128-pair tiles after a
// routing permutation, where the weight stream would need more than one
// 32-token pass for many experts: measured 147 against 162 us at 32 pairs
// per expert (two canvases), 150 against 174 us at 64 (four canvases with
// the pooled 96-token stream), 143 against 198 us under absorbing noise.
// Below that (one canvas: 16 pairs per expert) the weight stream reads each
// expert's weights once with every pair in one pass.  Same bits either way.
bool grouped_route(const dg_model* m, long long T) {
  const dg_config& c = m->cfg;
  return m->at == ACT_BF16 && m->wt == W_BF16 && grouped_supported(true, c.d_model, c.d_expert, c.n_experts) &&
         (T * c.top_k >= 24LL * c.n_experts || c.mask_token >= 0);
}

// routed experts on the top-k ids [T][k]: h [T*k][d_expert] (SwiGLU
// products) and y [T*k][d_model] (fp32 expert outputs), both in pair order
// (expert-major, token-ascending); off [E+1], pair_row [T*k] and pos [T][k]
// (the row of pair (t, j)) describe that order.
// xq / xqs: the rows of b as MXFP8 codes and scales (MXFP4_MXFP8 experts).
int routed(dg_model* m, int l, const void* b, int T, const int* ids, void* h, float* y, int* off, int* pair_row,
           int* pos, hipStream_t st, const uint8_t* xq = nullptr, const uint8_t* xqs = nullptr) {
  const dg_config& c = m->cfg;
  const dg_layer_weights& w = m->layers[l];
  const int E = c.n_experts, k = c.top_k, d = c.d_model, de = c.d_expert;
  if (m->at == ACT_BF16) {
    // Absorbing-state noise: every open position holds the same [MASK] token,
    // so the open rows pile onto a few experts; the pooled kernels' 96-token
    // passes stream a heavy expert's weights a third as often.
    const int pairs = c.mask_token >= 0 ? std::max(T * k, 24 * E + 1) : T * k;
    if (grouped_route(m, T)) {
      HIP_OK(router_permute(ids, T, E, k, off, pair_row, pos, st, m->perm_scratch));
      ProfScope ps(m, DG_PROF_MOE_GATEUP, st);
      HIP_OK(grouped_experts(true, b, pair_row, off, E, T * k, w.w_gu, d, de, h, st));
    } else {
      ProfScope ps(m, DG_PROF_MOE_GATEUP, st);  // routed gate/up + SwiGLU, routing in the kernel
      const MoeRoute r{ids, T, k, off, pair_row, pos};
      HIP_OK(moe_experts(m->wt_gu, true, b, nullptr, nullptr, E, w.w_gu, w.s_gu, d, de, h, st, &r, pairs, xq, xqs));
    }
    {
      // routed down: grouped 128 x 128 tiles from 96 pairs per expert (d_model
      // 2048, 128 experts of 704: 114 against 138 us per layer at 96 pairs per expert, 145
      // against 171 us at 128, and from 256 the pooled weight stream's passes
      // read an expert's weights once per 96 pairs), else the weight stream
      // (88 against 102 us for the grouped tiles at 64).  Under absorbing noise
      // the open rows pile onto a few experts, and the grouped tiles stream only
      // the experts that have pairs: 47.8 against 70.3 us per layer over the
      // first steps of a canvas, 8.98 against 9.05-9.16 ms per step over all 48.
      // Same bits either way.
      ProfScope ps(m, DG_PROF_MOE_DOWN, st);
      if (grouped_route(m, T) && ((long long)T * k >= 96LL * E || c.mask_token >= 0) &&
          grouped_supported(false, de, d, E))
        HIP_OK(grouped_experts(false, h, pair_row, off, E, T * k, w.w_d, de, d, y, st));
      else
        HIP_OK(moe_experts(m->wt, false, h, pair_row, off, E, w.w_d, w.s_d, de, d, y, st, nullptr, pairs));
    }
    return DG_OK;
  }
  HIP_OK(router_permute(ids, T, E, k, off, pair_row, pos, st));
  {
    ProfScope ps(m, DG_PROF_MOE_GATEUP, st);
    GemmArgs g;  // routed gate/up + SwiGLU, rows gathered per expert
    g.A = b; g.lda = d; g.a_rows = pair_row; g.B = w.w_gu; g.ldb = d;
    g.b_gstride = 2LL * de * d; g.b_scale = (const float*)w.s_gu; g.s_gstride = 2LL * de;
    g.M = T * k; g.N = de; g.K = d; g.g_off = off; g.C = h; g.ldc = de; g.swiglu_half = de;
    HIP_OK(gemm(m->at, m->wt, EPI_SWIGLU, g, E, st));
  }
  {
    ProfScope ps(m, DG_PROF_MOE_DOWN, st);
    GemmArgs g;  // routed down
    g.A = h; g.lda = de; g.B = w.w_d; g.ldb = de; g.b_gstride = (long long)d * de;
    g.b_scale = (const float*)w.s_d; g.s_gstride = d;
    g.M = T * k; g.N = d; g.K = de; g.g_off = off; g.C = y; g.ldc = d;
    HIP_OK(gemm(m->at, m->wt, EPI_F32, g, E, st));
  }
  return DG_OK;
}

// Rows per routed-expert launch of a T-row pass.  The grouped path (routing
// permutation, then grouped gate/up tiles) takes all rows at once: its
// permutation scales to any T, and the tiles of one expert weight tile run
// side by side on one XCD, so the weights come from HBM about once however
// many pair tiles an expert has.  The weight-stream kernels derive the
// routing of up to 2048 tokens in LDS (the fp32 path's permutation kernel
// takes 1024); there larger passes run in chunks, each streaming the expert
// weights once.
int route_chunk(const dg_model* m, long long T) {
  if (grouped_route(m, T)) return int(T);
  return m->at == ACT_BF16 ? 2048 : 1024;
}

// Routed experts on the top-k ids of rows [0, T) (normed rows in m->a, the
// shared-expert output in m->ys), then the combine, residual add and next
// RMSNorm of those rows, chunk by chunk.  diag: accumulate the expert pair
// counts of layer l into m->diag_counts.
int moe_chunks(dg_model* m, int l, int T, bool diag, hipStream_t st) {
  const dg_config& c = m->cfg;
  const int k = c.top_k, d = c.d_model, chunk = route_chunk(m, T);
  for (int c0 = 0; c0 < T; c0 += chunk) {
    const int tc = std::min(chunk, T - c0);
    const size_t row = (size_t)d * m->esz;
    const uint8_t* xq = m->q8 ? m->q8 + (size_t)c0 * d : nullptr;
    const uint8_t* xqs = m->q8 ? m->q8 + (size_t)m->Tmax * d + (size_t)c0 * (d / 32) : nullptr;
    int s = routed(m, l, (const char*)m->a + c0 * row, tc, m->topk_ids + (size_t)c0 * k, m->h, m->y, m->off,
                   m->pair_row, m->pos + (size_t)c0 * k, st, xq, xqs);
    if (s) return s;
    if (diag) HIP_OK(expert_counts(m->off, c.n_experts, m->diag_counts + (long long)l * c.n_experts, c0 > 0, st));
    HIP_OK(moe_combine_norm(m->at, (char*)m->x + c0 * row, m->y, m->ys + (size_t)c0 * d, m->topk_w + (size_t)c0 * k,
                            m->pos + (size_t)c0 * k, tc, k, d, c.rms_eps, (char*)m->a + c0 * row, m->ctl + 1, st));
  }
  return DG_OK;
}

// One pre-norm block over T = B * n rows.  causal: rows are new tokens at
// positions P.. written into the cache; otherwise canvas rows attend to the
// first P cache rows plus the canvas.  On entry m->a holds rmsnorm(x); on
// return x is updated and m->a holds rmsnorm of the new x (the next block's
// input norm, or the final norm before the LM head).
int layer_forward(dg_model* m, int l, int B, int n, int P, const dg_kv* kv, bool causal, bool kv_only,
                  hipStream_t st) {
  const dg_config& c = m->cfg;
  const dg_layer_weights& w = m->layers[l];
  const int T = B * n, d = c.d_model, H = c.n_heads, dh = c.head_dim, A = H * dh;
  const long long cap = kv->capacity;
  const long long layer_stride = (long long)kv->batch * H * cap * dh;
  char* kcache = (char*)kv->k + l * layer_stride * m->esz;
  char* vcache = (char*)kv->v + l * layer_stride * m->esz;
  int s;
  {
    ProfScope ps(m, DG_PROF_QKV, st);
    s = causal ? qkv_rope(m, l, m->a, B, n, m->q, kcache, vcache, cap * dh, P, st)
               : qkv_rope(m, l, m->a, B, n, m->q, m->kc, m->vc, (long long)n * dh, 0, st);
    if (s) return s;
  }
  if (causal && kv_only) return DG_OK;
  {
    ProfScope ps(m, DG_PROF_ATTN, st);
    s = causal ? attend(m, l, m->q, kv, P, nullptr, nullptr, B, n, m->o, st)
               : attend(m, l, m->q, kv, P, m->kc, m->vc, B, n, m->o, st);
    if (s) return s;
  }
  {
    GemmArgs g;  // O-projection + residual
    g.A = m->o; g.lda = A; g.B = w.wo; g.ldb = A; g.M = T; g.N = d; g.K = A; g.C = m->x; g.ldc = d;
    HIP_OK(gemm(m->at, m->at == ACT_BF16 ? W_BF16 : W_F32, EPI_RESID, g, 1, st));
  }
  HIP_OK(rmsnorm(m->at, m->x, T, d, c.rms_eps, m->a, st, m->q8, m->q8 ? m->q8 + (size_t)m->Tmax * d : nullptr));
  // The shared expert runs in line, before the router.  (On a second stream,
  // beside the router and the routed experts, its workgroups held CUs that
  // the routed gate/up workgroups (138 KB of LDS each) could not share, and
  // the waits this caused on the main stream cost more than the overlap won.)
  bool router_done = false, topk_done = false;
  {
    ProfScope ps(m, DG_PROF_SHARED, st);
    s = shared_gate_up(m, l, m->a, T, m->hs, m->rlog, &router_done, st);
    if (!s) s = shared_down(m, l, m->hs, T, m->ys, st, router_done ? m->rlog : nullptr, &topk_done);
    if (s) return s;
  }
  {
    ProfScope ps(m, DG_PROF_ROUTER, st);
    const int* forced = (m->force_ids && !causal)
                            ? m->force_ids + (long long)l * m->max_batch * c.canvas_len * c.top_k
                            : nullptr;
    s = route(m, l, m->a, T, m->rlog, router_done, m->topk_ids, m->topk_w, forced, st, topk_done);
    if (s) return s;
  }
  return moe_chunks(m, l, T, m->diag_counts && !causal, st);
}

// ---- mixed-phase batches: requests in different phases in one pass

struct MixedSeg {
  const dg_segment* s;
  int start;  // first row of the segment in the pass
  int P;      // its cache rows before the pass
};

// One block over the rows of a mixed batch (refine segments first, then
// append segments): the dense projections and the experts run once over all
// rows, attention per segment in its own mode over its own cache (all
// segments in one launch); the append segments' new keys and values go into
// their caches first.
int mixed_layer(dg_model* m, int l, const MixedSeg* sg, int n_segs, int T, int T_ref, hipStream_t st) {
  const dg_config& c = m->cfg;
  const int d = c.d_model, H = c.n_heads, dh = c.head_dim, A = H * dh;
  const long long plane = (long long)T * dh;
  int s;
  {
    ProfScope ps(m, DG_PROF_QKV, st);
    s = qkv_rope(m, l, m->a, 1, T, m->q, m->kc, m->vc, plane, 0, st);
    if (s) return s;
  }
  for (int i = 0; i < n_segs; ++i) {
    if (sg[i].s->kind != DG_SEG_APPEND) continue;
    const dg_kv* kv = sg[i].s->kv;
    const long long cap = kv->capacity, lay = (long long)H * cap * dh * m->esz;  // batch-1 cache
    HIP_OK(kv_copy_rows(m->at, (const char*)m->kc + sg[i].start * dh * m->esz,
                        (const char*)m->vc + sg[i].start * dh * m->esz, plane, H, sg[i].s->n, dh,
                        (char*)kv->k + l * lay, (char*)kv->v + l * lay, cap * dh, sg[i].P, st));
  }
  {
    // bf16: every segment's attention in one launch (and one merge); fp32:
    // one launch per segment
    ProfScope ps(m, DG_PROF_ATTN, st);
    static_assert(MAX_SEGMENTS <= ATTN_MAX_SEGS, "one attention launch per pass");
    AttnArgs aa[MAX_SEGMENTS];
    for (int i = 0; i < n_segs; ++i) {
      const int r0 = sg[i].start, n = sg[i].s->n;
      const char* q = (const char*)m->q + (size_t)r0 * dh * m->esz;
      char* o = (char*)m->o + (size_t)r0 * A * m->esz;
      const bool refine = sg[i].s->kind == DG_SEG_REFINE;
      aa[i] = attn_args(m, l, q, sg[i].s->kv, sg[i].P, refine ? (const char*)m->kc + (size_t)r0 * dh * m->esz : nullptr,
                        refine ? (const char*)m->vc + (size_t)r0 * dh * m->esz : nullptr, 1, n, o, plane);
      if (m->at != ACT_BF16) HIP_OK(attention(m->at, aa[i], st));
    }
    if (m->at == ACT_BF16)
      HIP_OK(attention_segments(m->at, aa, n_segs, m->attn_max_splits, m->attn_po, m->attn_ml, st));
  }
  {
    GemmArgs g;  // O-projection + residual
    g.A = m->o; g.lda = A; g.B = m->layers[l].wo; g.ldb = A; g.M = T; g.N = d; g.K = A; g.C = m->x; g.ldc = d;
    HIP_OK(gemm(m->at, m->at == ACT_BF16 ? W_BF16 : W_F32, EPI_RESID, g, 1, st));
  }
  HIP_OK(rmsnorm(m->at, m->x, T, d, c.rms_eps, m->a, st, m->q8, m->q8 ? m->q8 + (size_t)m->Tmax * d : nullptr));
  bool router_done = false, topk_done = false;
  {
    ProfScope ps(m, DG_PROF_SHARED, st);
    s = shared_gate_up(m, l, m->a, T, m->hs, m->rlog, &router_done, st);
    if (!s) s = shared_down(m, l, m->hs, T, m->ys, st, router_done ? m->rlog : nullptr, &topk_done);
    if (s) return s;
  }
  {
    ProfScope ps(m, DG_PROF_ROUTER, st);
    s = route(m, l, m->a, T, m->rlog, router_done, m->topk_ids, m->topk_w, nullptr, st, topk_done);
    if (s) return s;
    if (m->force_ids && T_ref)  // test hook, on the refine rows (the first T_ref)
      HIP_OK(router_force(m->rlog, T_ref, c.n_experts, c.top_k,
                          m->force_ids + (long long)l * m->max_batch * c.canvas_len * c.top_k, m->topk_ids,
                          m->topk_w, st));
  }
  return moe_chunks(m, l, T, false, st);
}

int lm_head_confidence(dg_model* m, const void* hf, int T, float* H, int* am, float* gap,
                       hipStream_t st) {
  ProfScope ps(m, DG_PROF_LM_HEAD, st);
  const dg_config& c = m->cfg;
  GemmArgs g;
  g.A = hf; g.lda = c.d_model; g.B = m->lm_head; g.ldb = c.d_model; g.M = T; g.N = c.vocab;
  g.K = c.d_model; g.part = m->lm_part; g.flags = m->ctl + 1;
  HIP_OK(gemm(m->at, m->at == ACT_BF16 ? W_BF16 : W_F32, EPI_LM, g, 1, st));
  HIP_OK(lm_merge(m->lm_part, T, m->lm_ntiles, H, am, gap, m->ctl + 1, st));
  return DG_OK;
}

int check_canvas(dg_model* m, const dg_canvas* c) {
  if (!c || !c->tokens || !c->committed) return fail(DG_ERR_INVALID_ARG, "null canvas pointer");
  if (m->cfg.self_condition && !c->prediction)
    return fail(DG_ERR_INVALID_ARG, "self-conditioning needs the canvas's prediction array");
  if (c->batch <= 0 || c->batch > m->max_batch)
    return fail(DG_ERR_SHAPE, "canvas batch %d outside [1, %d]", c->batch, m->max_batch);
  return DG_OK;
}

int check_kv(const dg_model* m, const dg_kv* kv, int batch, int extra) {
  if (!kv || !kv->k || !kv->v) return fail(DG_ERR_INVALID_ARG, "null kv pointer");
  if (kv->batch != batch) return fail(DG_ERR_SHAPE, "kv batch %d != %d", kv->batch, batch);
  if (kv->capacity > m->max_kv)
    return fail(DG_ERR_SHAPE, "kv capacity %d exceeds the model's max_kv %d", kv->capacity, m->max_kv);
  if (kv->length < 0 || kv->capacity <= 0 || (long long)kv->length + extra > kv->capacity)
    return fail(DG_ERR_SHAPE, "kv length %d + %d exceeds capacity %d", kv->length, extra, kv->capacity);
  return DG_OK;
}

int denoise_step_impl(dg_model* m, dg_canvas* c, const dg_kv* kv, dg_step_out* out, hipStream_t st) {
  const dg_config& cfg = m->cfg;
  const int B = c->batch, N = cfg.canvas_len, T = B * N, P = kv->length;
  // self-conditioning: from the second step on, the previous step's predictions join the input
  const int* cond = cfg.self_condition && c->step > 0 ? c->prediction : nullptr;
  HIP_OK(embed_gather(m->at, c->tokens, T, m->embed, cfg.d_model, cfg.vocab, m->x, m->ctl + 1, st, cond));
  HIP_OK(rmsnorm(m->at, m->x, T, cfg.d_model, cfg.rms_eps, m->a, st));
  HIP_OK(rope_table(N, cfg.head_dim, P, cfg.rope_theta, m->rope_tab, st));  // canvas positions P..P+N-1
  m->diag_counts = out ? out->expert_counts : nullptr;
  for (int l = 0; l < cfg.n_layers; ++l) {
    int s = layer_forward(m, l, B, N, P, kv, false, false, st);
    if (s) {
      m->diag_counts = nullptr;
      return s;
    }
  }
  m->diag_counts = nullptr;
  // m->a now holds the final RMSNorm of x
  if (out && out->hidden)
    HIP_OK(hipMemcpyAsync(out->hidden, m->a, (size_t)T * cfg.d_model * m->esz, hipMemcpyDeviceToDevice, st));
  float* H = (out && out->entropy) ? out->entropy : m->H;
  int* am = (out && out->argmax) ? out->argmax : m->am;
  float* gap = (out && out->top2_gap) ? out->top2_gap : nullptr;
  int s = lm_head_confidence(m, m->a, T, H, am, gap, st);
  if (s) return s;
  if (cfg.self_condition)  // this step's predictions condition the next
    HIP_OK(hipMemcpyAsync(c->prediction, am, sizeof(int) * T, hipMemcpyDeviceToDevice, st));
  if (out && out->logits) {
    GemmArgs g;
    g.A = m->a; g.lda = cfg.d_model; g.B = m->lm_head; g.ldb = cfg.d_model; g.M = T; g.N = cfg.vocab;
    g.K = cfg.d_model; g.C = out->logits; g.ldc = cfg.vocab;
    HIP_OK(gemm(m->at, m->at == ACT_BF16 ? W_BF16 : W_F32, EPI_F32, g, 1, st));
  }
  {
    ProfScope ps(m, DG_PROF_COMMIT, st);
    HIP_OK(commit_renoise(H, am, c->tokens, c->committed, B, N, c->step, cfg.max_steps,
                          cfg.commit_threshold, c->seed, c->block, cfg.vocab, cfg.mask_token, m->n_unc, m->ctl + 1,
                          m->ctl, st));
  }
  if (out && out->n_uncommitted)
    HIP_OK(hipMemcpyAsync(out->n_uncommitted, m->n_unc, sizeof(int) * B, hipMemcpyDeviceToDevice, st));
  if (out && out->status) HIP_OK(hipMemcpyAsync(out->status, m->ctl, sizeof(int), hipMemcpyDeviceToDevice, st));
  c->step += 1;
  return DG_OK;
}

}  // namespace

extern "C" {

const char* dg_status_str(int s) {
  switch (s) {
    case DG_OK: return "ok";
    case DG_ERR_INVALID_ARG: return "invalid argument";
    case DG_ERR_SHAPE: return "shape error";
    case DG_ERR_HIP: return "HIP error";
    case DG_ERR_OOM: return "out of device memory";
    case DG_ERR_STATE: return "invalid state";
    case DG_ERR_NUMERIC: return "numeric error";
    case DG_ERR_UNIMPLEMENTED: return "unimplemented";
  }
  return "unknown status";
}

const char* dg_last_error(void) { return g_err.c_str(); }

const char* dg_version(void) { return "dg 0.1 gfx950"; }

int dg_model_create(const dg_config* cfg, const dg_weights* w, int32_t max_batch, int32_t max_tokens,
                    int32_t max_kv, dg_model** out) {
  if (!cfg || !w || !out) return fail(DG_ERR_INVALID_ARG, "null argument");
  *out = nullptr;
  int s = check_config(*cfg);
  if (s) return s;
  if (!w->embed || !w->lm_head || !w->layers) return fail(DG_ERR_INVALID_ARG, "null weight pointer");
  for (int l = 0; l < cfg->n_layers; ++l) {
    const dg_layer_weights& L = w->layers[l];
    if (!L.wqkv || !L.wo || !L.wr || !L.w_gu || !L.w_d || !L.ws_gu || !L.ws_d)
      return fail(DG_ERR_INVALID_ARG, "null weight pointer in layer %d", l);
    const bool fp8 = cfg->expert_dtype == DG_DTYPE_FP8_E4M3;
    const bool fp4 = cfg->expert_dtype == DG_DTYPE_MXFP4 || cfg->expert_dtype == DG_DTYPE_MXFP4_MXFP8;
    if (fp8 != (L.s_gu && L.s_d && L.ss_gu && L.ss_d) && !fp4)
      return fail(DG_ERR_INVALID_ARG, "fp8 scales must be given exactly when expert_dtype is FP8 (layer %d)", l);
    if (fp4 && !(L.s_gu && L.s_d && !L.ss_gu && !L.ss_d))
      return fail(DG_ERR_INVALID_ARG, "MXFP4 experts need block scales s_gu, s_d and no shared scales (layer %d)", l);
    if (!fp8 && !fp4 && (L.s_gu || L.s_d || L.ss_gu || L.ss_d))
      return fail(DG_ERR_INVALID_ARG, "scales are given only with FP8 or MXFP4 experts (layer %d)", l);
  }
  if (max_batch <= 0 || max_tokens < 0 || max_kv < 0)
    return fail(DG_ERR_INVALID_ARG, "max_batch must be > 0, max_tokens and max_kv >= 0");
  // attention addresses a (layer, canvas, head) plane of the cache with 32-bit byte offsets
  const long long kv_limit = 0x7fffffffLL / ((long long)cfg->head_dim * (cfg->act_dtype == DG_DTYPE_BF16 ? 2 : 4));
  if (max_kv > kv_limit) return fail(DG_ERR_SHAPE, "max_kv %d exceeds %lld rows", max_kv, kv_limit);
  const int ntok = std::max(max_tokens, cfg->canvas_len);
  // rows of one call (the workspace grows with it; the routed experts take
  // a call's rows at once on the grouped path, else in chunks of 2048 rows,
  // 1024 with fp32)
  const long long max_t = 8192;
  if ((long long)max_batch * ntok > max_t)
    return fail(DG_ERR_SHAPE, "max_batch * max(max_tokens, canvas_len) must be <= %lld", max_t);

  dg_model* m = new dg_model();
  m->cfg = *cfg;
  m->layers.assign(w->layers, w->layers + cfg->n_layers);
  m->embed = w->embed;
  m->lm_head = w->lm_head;
  m->max_batch = max_batch;
  m->max_tokens = ntok;
  m->max_kv = max_kv ? max_kv : int(kv_limit);
  m->Tmax = max_batch * ntok;
  m->at = cfg->act_dtype == DG_DTYPE_BF16 ? ACT_BF16 : ACT_F32;
  m->wt = cfg->expert_dtype == DG_DTYPE_FP8_E4M3 ? W_FP8
        : cfg->expert_dtype == DG_DTYPE_MXFP4 || cfg->expert_dtype == DG_DTYPE_MXFP4_MXFP8 ? W_FP4
                                                 : (m->at == ACT_BF16 ? W_BF16 : W_F32);
  m->wt_gu = cfg->expert_dtype == DG_DTYPE_MXFP4_MXFP8 ? W_FP4A8 : m->wt;
  m->swt = m->wt == W_FP4 ? W_BF16 : m->wt;
  m->esz = m->at == ACT_BF16 ? 2 : 4;
  const size_t T = m->Tmax, d = cfg->d_model, A = (size_t)cfg->n_heads * cfg->head_dim;
  const size_t E = cfg->n_experts, k = cfg->top_k, de = cfg->d_expert, ds = cfg->d_shared;
  const size_t Tc = (size_t)max_batch * cfg->canvas_len;
  const size_t Tr = std::min(T, (size_t)route_chunk(m, (long long)T));  // rows of one routed launch
  m->lm_ntiles = lm_tiles(m->at, cfg->d_model, cfg->vocab);
  const size_t es = m->esz;
  struct Req {
    void** p;
    size_t bytes;
  } reqs[] = {
      {&m->x, T * d * es},
      {&m->a, T * d * es},
      {&m->qkv, T * 3 * A * es},
      {&m->q, T * A * es},
      {&m->kc, T * A * es},
      {&m->vc, T * A * es},
      {&m->o, T * A * es},
      {(void**)&m->attn_po, (size_t)m->attn_max_splits * T * A * 4},
      {(void**)&m->attn_ml, (size_t)m->attn_max_splits * T * cfg->n_heads * 2 * 4},
      {(void**)&m->rlog, T * E * 4},
      {(void**)&m->rope_tab, T * cfg->head_dim * 4},
      {(void**)&m->topk_ids, T * k * 4},
      {(void**)&m->topk_w, T * k * 4},
      {(void**)&m->off, (E + 1) * 4},
      {(void**)&m->pair_row, Tr * k * 4},
      {(void**)&m->pos, T * k * 4},
      {&m->h, Tr * k * de * es},
      {(void**)&m->y, Tr * k * d * 4},
      {&m->hs, T * ds * es},
      {(void**)&m->ys, T * d * 4},
      {(void**)&m->lm_part, Tc * m->lm_ntiles * 5 * 4},
      {(void**)&m->H, Tc * 4},
      {(void**)&m->gap, Tc * 4},
      {(void**)&m->am, Tc * 4},
      {(void**)&m->ctl, (size_t)(2 + max_batch) * 4},
      {&m->perm_scratch, router_permute_scratch(int(Tr), int(E))},
  };
  for (auto& r : reqs) {
    s = alloc(m, r.p, r.bytes);
    if (s) {
      free_all(m);
      delete m;
      return s;
    }
  }
  if (m->wt_gu == W_FP4A8) {  // the normed rows as MXFP8 (only these models have the buffer)
    s = alloc(m, (void**)&m->q8, T * (d + d / 32));
    if (s) {
      free_all(m);
      delete m;
      return s;
    }
  }
  m->n_unc = m->ctl + 2;
  {
    // set-up of the allocation-free entry on this device: the address of its
    // static scratch (a lookup, no allocation)
    void* sp = nullptr;
    const int e = noalloc_scratch(&sp);
    if (e) {
      free_all(m);
      delete m;
      return fail(DG_ERR_HIP, "hipGetSymbolAddress of the static scratch failed: %s", hipGetErrorString(hipError_t(e)));
    }
  }
  if (hipMemset(m->ctl, 0, sizeof(int) * (2 + max_batch)) != hipSuccess) {
    (void)hipGetLastError();
    free_all(m);
    delete m;
    return fail(DG_ERR_HIP, "hipMemset of the status word failed");
  }
  if (hipHostMalloc((void**)&m->u_host, sizeof(int) * (2 + max_batch), hipHostMallocDefault) != hipSuccess) {
    (void)hipGetLastError();
    free_all(m);
    delete m;
    return fail(DG_ERR_OOM, "hipHostMalloc failed");
  }
  *out = m;
  return DG_OK;
}

int dg_model_destroy(dg_model* m) {
  if (!m) return DG_OK;
  (void)hipDeviceSynchronize();
  free_all(m);
  delete m;
  return DG_OK;
}

int dg_canvas_init(dg_model* m, dg_canvas* c, void* stream) {
  if (!m) return fail(DG_ERR_INVALID_ARG, "null model");
  int s = check_canvas(m, c);
  if (s) return s;
  HIP_OK(canvas_init(c->tokens, c->committed, c->batch, m->cfg.canvas_len, c->seed, c->block,
                     m->cfg.vocab, m->cfg.mask_token, (hipStream_t)stream));
  c->step = 0;
  return DG_OK;
}

int dg_canvas_prefill(dg_model* m, dg_canvas* c, const int32_t* tokens, const uint8_t* mask, void* stream) {
  if (!m || !tokens || !mask) return fail(DG_ERR_INVALID_ARG, "null argument");
  int s = check_canvas(m, c);
  if (s) return s;
  if (c->step != 0) return fail(DG_ERR_STATE, "prefill needs a canvas at step 0 (step %d)", c->step);
  HIP_OK(canvas_prefill(c->tokens, c->committed, c->batch * m->cfg.canvas_len, tokens, mask, (hipStream_t)stream));
  return DG_OK;
}

int dg_denoise_step(dg_model* m, dg_canvas* c, const dg_kv* kv, dg_step_out* out, void* stream) {
  if (!m) return fail(DG_ERR_INVALID_ARG, "null model");
  int s = check_canvas(m, c);
  if (s) return s;
  s = check_kv(m, kv, c->batch, 0);
  if (s) return s;
  if (c->step < 0 || c->step >= m->cfg.max_steps)
    return fail(DG_ERR_STATE, "step %d outside [0, max_steps=%d)", c->step, m->cfg.max_steps);
  return denoise_step_impl(m, c, kv, out, (hipStream_t)stream);
}

int dg_generate_canvas(dg_model* m, dg_canvas* c, const dg_kv* kv, int32_t* steps_taken, void* stream) {
  if (!m || !steps_taken) return fail(DG_ERR_INVALID_ARG, "null argument");
  int s = check_canvas(m, c);
  if (s) return s;
  s = check_kv(m, kv, c->batch, 0);
  if (s) return s;
  if (c->step < 0 || c->step > m->cfg.max_steps)
    return fail(DG_ERR_STATE, "step %d outside [0, max_steps]", c->step);
  hipStream_t st = (hipStream_t)stream;
  int taken = 0;
  while (c->step < m->cfg.max_steps) {
    s = denoise_step_impl(m, c, kv, nullptr, st);
    if (s) {
      *steps_taken = taken;
      return s;
    }
    ++taken;
    // the status word and the per-canvas uncommitted counts come back with
    // the step's end (the host waits for it anyway)
    HIP_OK(hipMemcpyAsync(m->u_host, m->ctl, sizeof(int) * (2 + c->batch), hipMemcpyDeviceToHost, st));
    HIP_OK(hipStreamSynchronize(st));
    const int status = m->u_host[0];
    if (status & FLAG_TOKEN) {
      *steps_taken = taken;
      return fail(DG_ERR_INVALID_ARG, "a token id outside [0, %d) reached the embedding (read as id 0) by step %d",
                  m->cfg.vocab, c->step - 1);
    }
    if (status & FLAG_NONFINITE) {
      *steps_taken = taken;
      return fail(DG_ERR_NUMERIC, "non-finite values in the residual stream or the logits by step %d", c->step - 1);
    }
    int left = 0;
    for (int b = 0; b < c->batch; ++b) left += m->u_host[2 + b];
    if (left == 0) break;
  }
  *steps_taken = taken;
  return DG_OK;
}

int dg_commit_canvas(dg_model* m, const int32_t* tokens, int32_t n, dg_kv* kv, void* stream) {
  if (!m || !tokens) return fail(DG_ERR_INVALID_ARG, "null argument");
  if (!kv) return fail(DG_ERR_INVALID_ARG, "null kv");
  if (n <= 0 || n > m->max_tokens) return fail(DG_ERR_SHAPE, "n=%d outside [1, max_tokens=%d]", n, m->max_tokens);
  if (kv->batch <= 0 || kv->batch > m->max_batch) return fail(DG_ERR_SHAPE, "kv batch %d", kv->batch);
  int s = check_kv(m, kv, kv->batch, n);
  if (s) return s;
  hipStream_t st = (hipStream_t)stream;
  const dg_config& cfg = m->cfg;
  const int B = kv->batch, T = B * n, P = kv->length;
  HIP_OK(embed_gather(m->at, tokens, T, m->embed, cfg.d_model, cfg.vocab, m->x, m->ctl + 1, st));
  HIP_OK(rmsnorm(m->at, m->x, T, cfg.d_model, cfg.rms_eps, m->a, st));
  HIP_OK(rope_table(n, cfg.head_dim, P, cfg.rope_theta, m->rope_tab, st));  // positions P..P+n-1
  for (int l = 0; l < cfg.n_layers; ++l) {
    s = layer_forward(m, l, B, n, P, kv, true, l == cfg.n_layers - 1, st);
    if (s) return s;
  }
  kv->length = P + n;
  return DG_OK;
}

int dg_profile_kernel(dg_model* m, int32_t kernel_id) {
  if (!m) return fail(DG_ERR_INVALID_ARG, "null model");
  if (kernel_id < DG_PROF_NONE || kernel_id > DG_PROF_COMMIT) return fail(DG_ERR_INVALID_ARG, "bad kernel id");
  int s = prof_drain(m);
  if (s) return s;
  if (kernel_id != DG_PROF_NONE && m->prof_ev.empty()) {
    m->prof_ev.resize(2 * PROF_PAIRS);
    for (auto& e : m->prof_ev) HIP_OK(hipEventCreate(&e));
  }
  m->prof_id = kernel_id;
  m->prof_ms = 0.0;
  m->prof_launches = 0;
  return DG_OK;
}

int dg_profile_read(dg_model* m, double* total_ms, int64_t* launches) {
  if (!m || !total_ms || !launches) return fail(DG_ERR_INVALID_ARG, "null argument");
  int s = prof_drain(m);
  if (s) return s;
  *total_ms = m->prof_ms;
  *launches = m->prof_launches;
  m->prof_ms = 0.0;
  m->prof_launches = 0;
  return DG_OK;
}

int dg_pack_experts(const void* src, void* dst, int64_t n_mats, int32_t rows, int32_t cols, int32_t dtype,
                    void* stream) {
  if (!src || !dst) return fail(DG_ERR_INVALID_ARG, "null pointer");
  if (dtype != DG_DTYPE_BF16 && dtype != DG_DTYPE_FP8_E4M3 && dtype != DG_DTYPE_MXFP4 && dtype != DG_DTYPE_E8M0)
    return fail(DG_ERR_INVALID_ARG, "dtype must be BF16, FP8_E4M3, MXFP4 or E8M0");
  if (n_mats <= 0 || rows <= 0 || cols <= 0 || rows % 16 || cols % 32)
    return fail(DG_ERR_SHAPE, "need n_mats, rows, cols > 0, rows %% 16 == 0 and cols %% 32 == 0");
  const bool mx = dtype == DG_DTYPE_MXFP4 || dtype == DG_DTYPE_E8M0;
  if (mx && cols % 64) return fail(DG_ERR_SHAPE, "MXFP4 needs cols %% 64 == 0");
  const unsigned long long n = (unsigned long long)n_mats * rows * cols;
  const unsigned long long bytes = dtype == DG_DTYPE_BF16 ? 2 * n : dtype == DG_DTYPE_FP8_E4M3 ? n
                                   : dtype == DG_DTYPE_MXFP4 ? n / 2 : n / 32;
  const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
  if (s0 < d0 + bytes && d0 < s0 + bytes) return fail(DG_ERR_INVALID_ARG, "src and dst overlap");
  hipStream_t st = (hipStream_t)stream;
  if (dtype == DG_DTYPE_E8M0) {
    HIP_OK(moe_pack_scales(src, dst, n_mats, rows, cols, st));
    return DG_OK;
  }
  const WType wt = dtype == DG_DTYPE_BF16 ? W_BF16 : dtype == DG_DTYPE_FP8_E4M3 ? W_FP8 : W_FP4;
  HIP_OK(moe_pack(wt, src, dst, n_mats, rows, cols, st));
  return DG_OK;
}

int dg_test_philox(uint64_t seed, uint32_t pos0, uint32_t step_tag, uint32_t canvas, uint32_t block,
                   uint32_t modulus, int32_t n, uint32_t* out, void* stream) {
  if (!out || n < 0 || n > (1 << 24)) return fail(DG_ERR_INVALID_ARG, "bad philox arguments");
  HIP_OK(philox_fill(seed, pos0, step_tag, canvas, block, modulus, n, out, (hipStream_t)stream));
  return DG_OK;
}

int dg_test_fp4_decode(const uint8_t* packed, const uint8_t* scales, int32_t n_blocks, void* out, void* stream) {
  if (!packed || !scales || !out) return fail(DG_ERR_INVALID_ARG, "null argument");
  if (n_blocks <= 0 || n_blocks > (1 << 24)) return fail(DG_ERR_SHAPE, "n_blocks %d", n_blocks);
  HIP_OK(fp4_decode(packed, scales, n_blocks, out, (hipStream_t)stream));
  return DG_OK;
}

int dg_test_mx8_quantize(const void* x, int32_t rows, int32_t d, int32_t norm, float eps, void* y,
                         uint8_t* codes, uint8_t* scales, void* stream) {
  if (!x || !codes || !scales || (norm && !y)) return fail(DG_ERR_INVALID_ARG, "null argument");
  if (rows <= 0 || d <= 0 || d % 32 || (norm && d > 8192) || (long long)rows * d > (1LL << 30))
    return fail(DG_ERR_SHAPE, "rows=%d d=%d", rows, d);
  if (norm) HIP_OK(rmsnorm(ACT_BF16, x, rows, d, eps, y, (hipStream_t)stream, codes, scales));
  else HIP_OK(mx8_quantize(x, rows, d, codes, scales, (hipStream_t)stream));
  return DG_OK;
}

int dg_test_lm_head(dg_model* m, const void* hf, int32_t T, float* entropy, int32_t* argmax,
                    float* top2_gap, void* stream) {
  if (!m || !hf) return fail(DG_ERR_INVALID_ARG, "null argument");
  if (T <= 0 || T > m->max_batch * m->cfg.canvas_len) return fail(DG_ERR_SHAPE, "T=%d out of range", T);
  return lm_head_confidence(m, hf, T, entropy, argmax, top2_gap, (hipStream_t)stream);
}

int dg_lm_head_confidence_noalloc(const dg_model* m, const void* hf, int32_t T, float* entropy, int32_t* argmax,
                                  float* top2_gap, void* stream) {
  if (!m || !hf || !entropy || !argmax) return fail(DG_ERR_INVALID_ARG, "null argument");
  if (T <= 0) return fail(DG_ERR_SHAPE, "T=%d must be positive", T);
  const size_t per_row = (size_t)m->lm_ntiles * 5 * sizeof(float);
  if ((size_t)T * per_row > NOALLOC_SCRATCH_BYTES)
    return fail(DG_ERR_SHAPE, "%d rows need %zu bytes of partials; the static scratch holds %zu (%zu rows at %d ids)",
                T, (size_t)T * per_row, NOALLOC_SCRATCH_BYTES, NOALLOC_SCRATCH_BYTES / per_row, m->cfg.vocab);
  void* sp = nullptr;
  HIP_OK(noalloc_scratch(&sp));
  hipStream_t st = (hipStream_t)stream;
  const dg_config& c = m->cfg;
  GemmArgs g;
  g.A = hf; g.lda = c.d_model; g.B = m->lm_head; g.ldb = c.d_model; g.M = T; g.N = c.vocab;
  g.K = c.d_model; g.part = (float*)sp;
  HIP_OK(gemm(m->at, m->at == ACT_BF16 ? W_BF16 : W_F32, EPI_LM, g, 1, st));
  HIP_OK(lm_merge((const float*)sp, T, m->lm_ntiles, entropy, argmax, top2_gap, nullptr, st));
  return DG_OK;
}

int dg_test_commit(dg_model* m, dg_canvas* c, const float* entropy, const int32_t* argmax,
                   int32_t* n_uncommitted, void* stream) {
  if (!m || !entropy || !argmax || !n_uncommitted) return fail(DG_ERR_INVALID_ARG, "null argument");
  int s = check_canvas(m, c);
  if (s) return s;
  if (c->step < 0 || c->step >= m->cfg.max_steps) return fail(DG_ERR_STATE, "step out of range");
  HIP_OK(commit_renoise(entropy, argmax, c->tokens, c->committed, c->batch, m->cfg.canvas_len, c->step,
                        m->cfg.max_steps, m->cfg.commit_threshold, c->seed, c->block, m->cfg.vocab, m->cfg.mask_token,
                        n_uncommitted, nullptr, nullptr, (hipStream_t)stream));
  return DG_OK;
}

// ---- unit entries: one phase of a block on caller buffers, through the same
// launches the step makes

namespace {
int check_layer(const dg_model* m, int layer) {
  if (layer < 0 || layer >= m->cfg.n_layers)
    return fail(DG_ERR_INVALID_ARG, "layer %d outside [0, %d)", layer, m->cfg.n_layers);
  return DG_OK;
}
int check_rows(const dg_model* m, long long T) {
  if (T <= 0 || T > m->Tmax) return fail(DG_ERR_SHAPE, "%lld rows outside [1, %d]", T, m->Tmax);
  return DG_OK;
}
}  // namespace

int dg_test_qkv_rope(dg_model* m, int32_t layer, const void* a, int32_t batch, int32_t n, int32_t pos0, void* q,
                     void* k, void* v, void* stream) {
  if (!m || !a || !q || !k || !v) return fail(DG_ERR_INVALID_ARG, "null argument");
  int s = check_layer(m, layer);
  if (!s) s = check_rows(m, (long long)batch * n);
  if (s) return s;
  if (batch <= 0 || n <= 0 || n > m->max_tokens || pos0 < 0)
    return fail(DG_ERR_SHAPE, "batch %d, n %d (max_tokens %d), pos0 %d", batch, n, m->max_tokens, pos0);
  hipStream_t st = (hipStream_t)stream;
  HIP_OK(rope_table(n, m->cfg.head_dim, pos0, m->cfg.rope_theta, m->rope_tab, st));
  return qkv_rope(m, layer, a, batch, n, q, k, v, (long long)n * m->cfg.head_dim, 0, st);
}

int dg_test_attention(dg_model* m, int32_t layer, const void* q, const dg_kv* kv, const void* k_canvas,
                      const void* v_canvas, int32_t n, void* out, void* stream) {
  if (!m || !q || !out || !kv || (!k_canvas) != (!v_canvas)) return fail(DG_ERR_INVALID_ARG, "null argument");
  int s = check_layer(m, layer);
  if (!s) s = check_kv(m, kv, kv->batch, k_canvas ? 0 : n);
  if (!s && (kv->batch <= 0 || kv->batch > m->max_batch)) s = fail(DG_ERR_SHAPE, "kv batch %d", kv->batch);
  if (!s) s = check_rows(m, (long long)kv->batch * n);
  if (s) return s;
  return attend(m, layer, q, kv, kv->length, k_canvas, v_canvas, kv->batch, n, out, (hipStream_t)stream);
}

int dg_test_router(dg_model* m, int32_t layer, const void* b, int32_t T, float* logits, int32_t* ids,
                   float* weights, void* stream) {
  if (!m || !b || !logits || !ids || !weights) return fail(DG_ERR_INVALID_ARG, "null argument");
  int s = check_layer(m, layer);
  if (!s) s = check_rows(m, T);
  if (s) return s;
  hipStream_t st = (hipStream_t)stream;
  bool done = false;
  s = shared_gate_up(m, layer, b, T, m->hs, logits, &done, st);
  if (s) return s;
  return route(m, layer, b, T, logits, done, ids, weights, nullptr, st);
}

int dg_test_shared(dg_model* m, int32_t layer, const void* b, int32_t T, void* hs, float* ys, void* stream) {
  if (!m || !b || !hs || !ys) return fail(DG_ERR_INVALID_ARG, "null argument");
  int s = check_layer(m, layer);
  if (!s) s = check_rows(m, T);
  if (s) return s;
  hipStream_t st = (hipStream_t)stream;
  bool done = false;
  s = shared_gate_up(m, layer, b, T, hs, m->rlog, &done, st);
  if (s) return s;
  return shared_down(m, layer, hs, T, ys, st);
}

int dg_test_moe(dg_model* m, int32_t layer, const void* b, int32_t T, const int32_t* ids, void* h, float* y,
                int32_t* pos, void* stream) {
  if (!m || !b || !ids || !y || !pos) return fail(DG_ERR_INVALID_ARG, "null argument");
  int s = check_layer(m, layer);
  if (!s) s = check_rows(m, T);
  if (s) return s;
  if (T > route_chunk(m, T)) return fail(DG_ERR_SHAPE, "T=%d exceeds one routed launch (%d rows)", T, route_chunk(m, T));
  const int d = m->cfg.d_model;
  uint8_t* xqs = m->q8 ? m->q8 + (size_t)m->Tmax * d : nullptr;
  if (m->q8) HIP_OK(mx8_quantize(b, T, d, m->q8, xqs, (hipStream_t)stream));
  return routed(m, layer, b, T, ids, h ? h : m->h, y, m->off, m->pair_row, pos, (hipStream_t)stream, m->q8, xqs);
}

int dg_mixed_step(dg_model* m, dg_segment* segs, int32_t n_segs, int32_t* status, void* stream) {
  if (!m || !segs) return fail(DG_ERR_INVALID_ARG, "null argument");
  if (n_segs < 1 || n_segs > MAX_SEGMENTS) return fail(DG_ERR_SHAPE, "n_segs %d outside [1, %d]", n_segs, MAX_SEGMENTS);
  const dg_config& cfg = m->cfg;
  long long T = 0, T_ref = 0;
  for (int i = 0; i < n_segs; ++i) {
    const dg_segment& g = segs[i];
    if (g.kind != DG_SEG_APPEND && g.kind != DG_SEG_REFINE)
      return fail(DG_ERR_INVALID_ARG, "segment %d: kind %d", i, g.kind);
    if (!g.kv) return fail(DG_ERR_INVALID_ARG, "segment %d: null kv", i);
    int s = check_kv(m, g.kv, 1, g.kind == DG_SEG_APPEND ? g.n : 0);
    if (s) return s;
    for (int j = 0; j < i; ++j)
      if (segs[j].kv->k == g.kv->k || segs[j].kv->v == g.kv->v)
        return fail(DG_ERR_INVALID_ARG, "segments %d and %d share a KV cache", j, i);
    if (g.kind == DG_SEG_APPEND) {
      if (!g.tokens) return fail(DG_ERR_INVALID_ARG, "segment %d: null tokens", i);
      if (g.n <= 0 || g.n > m->max_tokens)
        return fail(DG_ERR_SHAPE, "segment %d: n=%d outside [1, max_tokens=%d]", i, g.n, m->max_tokens);
    } else {
      if (!g.canvas) return fail(DG_ERR_INVALID_ARG, "segment %d: null canvas", i);
      s = check_canvas(m, g.canvas);
      if (s) return s;
      if (g.canvas->batch != 1) return fail(DG_ERR_SHAPE, "segment %d: a refine segment holds one canvas", i);
      if (g.n != cfg.canvas_len) return fail(DG_ERR_SHAPE, "segment %d: n=%d != canvas_len", i, g.n);
      if (g.canvas->step < 0 || g.canvas->step >= cfg.max_steps)
        return fail(DG_ERR_STATE, "segment %d: step %d outside [0, max_steps)", i, g.canvas->step);
      T_ref += g.n;
    }
    T += g.n;
  }
  if (T > m->Tmax) return fail(DG_ERR_SHAPE, "%lld rows exceed the workspace (%d)", T, m->Tmax);
  if (T_ref > (long long)m->max_batch * cfg.canvas_len)
    return fail(DG_ERR_SHAPE, "%lld refine rows exceed max_batch * canvas_len", T_ref);
  hipStream_t st = (hipStream_t)stream;
  // rows: refine segments first (their LM head and commit read one block), then append segments
  MixedSeg sg[MAX_SEGMENTS];
  RowSegments rs{};
  int n = 0, r = 0;
  for (int pass = 0; pass < 2; ++pass)
    for (int i = 0; i < n_segs; ++i) {
      if ((segs[i].kind == DG_SEG_REFINE) != (pass == 0)) continue;
      sg[n] = MixedSeg{&segs[i], r, segs[i].kv->length};
      rs.start[n] = r;
      rs.pos0[n] = segs[i].kv->length;
      r += segs[i].n;
      ++n;
    }
  rs.n_segs = n;
  rs.start[n] = r;
  for (int i = 0; i < n; ++i) {
    const bool ref = sg[i].s->kind == DG_SEG_REFINE;
    const int32_t* tok = ref ? sg[i].s->canvas->tokens : sg[i].s->tokens;
    const int32_t* cond = ref && cfg.self_condition && sg[i].s->canvas->step > 0 ? sg[i].s->canvas->prediction : nullptr;
    HIP_OK(embed_gather(m->at, tok, sg[i].s->n, m->embed, cfg.d_model, cfg.vocab,
                        (char*)m->x + (size_t)sg[i].start * cfg.d_model * m->esz, m->ctl + 1, st, cond));
  }
  HIP_OK(rmsnorm(m->at, m->x, (int)T, cfg.d_model, cfg.rms_eps, m->a, st));
  HIP_OK(rope_table_rows(rs, cfg.head_dim, cfg.rope_theta, m->rope_tab, st));
  for (int l = 0; l < cfg.n_layers; ++l) {
    int s = mixed_layer(m, l, sg, n, (int)T, (int)T_ref, st);
    if (s) return s;
  }
  int last_ref = -1;
  for (int i = 0; i < n; ++i)
    if (sg[i].s->kind == DG_SEG_REFINE) last_ref = i;
  for (int i = 0; i < n; ++i)
    if (sg[i].s->kind == DG_SEG_REFINE && sg[i].s->hidden)
      HIP_OK(hipMemcpyAsync(sg[i].s->hidden, (const char*)m->a + (size_t)sg[i].start * cfg.d_model * m->esz,
                            (size_t)cfg.canvas_len * cfg.d_model * m->esz, hipMemcpyDeviceToDevice, st));
  if (T_ref > 0) {
    int s = lm_head_confidence(m, m->a, (int)T_ref, m->H, m->am, nullptr, st);
    if (s) return s;
  }
  for (int i = 0; i < n; ++i) {
    const dg_segment& g = *sg[i].s;
    if (g.kind != DG_SEG_REFINE) continue;
    const int r0 = sg[i].start;  // refine rows start at 0, one canvas after another
    dg_canvas* cv = g.canvas;
    ProfScope ps(m, DG_PROF_COMMIT, st);
    // the last commit of the pass publishes the status word
    HIP_OK(commit_renoise(m->H + r0, m->am + r0, cv->tokens, cv->committed, 1, cfg.canvas_len, cv->step,
                          cfg.max_steps, cfg.commit_threshold, cv->seed, cv->block, cfg.vocab, cfg.mask_token,
                          g.n_uncommitted ? g.n_uncommitted : m->n_unc + r0 / cfg.canvas_len,
                          i == last_ref ? m->ctl + 1 : nullptr, i == last_ref ? m->ctl : nullptr, st));
    if (g.entropy)
      HIP_OK(hipMemcpyAsync(g.entropy, m->H + r0, sizeof(float) * cfg.canvas_len, hipMemcpyDeviceToDevice, st));
    if (g.argmax)
      HIP_OK(hipMemcpyAsync(g.argmax, m->am + r0, sizeof(int) * cfg.canvas_len, hipMemcpyDeviceToDevice, st));
    if (cfg.self_condition)
      HIP_OK(hipMemcpyAsync(cv->prediction, m->am + r0, sizeof(int) * cfg.canvas_len, hipMemcpyDeviceToDevice, st));
  }
  if (last_ref < 0) HIP_OK(status_publish(m->ctl + 1, m->ctl, st));
  if (status) HIP_OK(hipMemcpyAsync(status, m->ctl, sizeof(int), hipMemcpyDeviceToDevice, st));
  for (int i = 0; i < n; ++i) {
    if (sg[i].s->kind == DG_SEG_REFINE) sg[i].s->canvas->step += 1;
    else sg[i].s->kv->length += sg[i].s->n;
  }
  return DG_OK;
}

int dg_test_force_routing(dg_model* m, const int32_t* ids) {
  if (!m) return fail(DG_ERR_INVALID_ARG, "null model");
  m->force_ids = ids;
  return DG_OK;
}

}  // extern "C"
