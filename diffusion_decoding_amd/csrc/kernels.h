// Host-side launch interfaces of the gfx950 kernels.  Every launcher enqueues
// on `st` and performs no synchronisation and no allocation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

enum ActType { ACT_F32 = 0, ACT_BF16 = 1 };

// Bits of the device status word the kernels of a step raise (atomic OR):
// a non-finite value in the residual stream or in the logits, a token id
// outside the vocabulary.
constexpr int FLAG_NONFINITE = 1;
constexpr int FLAG_TOKEN = 2;
// W_FP4A8: MXFP4 weights whose gate/up reads its token rows as MXFP8 (the
// gfx950 scaled MFMA; moe_experts gate/up only)
enum WType { W_F32 = 0, W_BF16 = 1, W_FP8 = 2, W_FP4 = 3, W_FP4A8 = 4 };

// ---------------------------------------------------------------- GEMM (k_gemm.hip)
// C[m][n] = sum_k A[row(m)][k] * B[n][k]; epilogue by kind.
enum GemmEpi {
  EPI_F32 = 0,     // C fp32 [m][n]
  EPI_ACT = 1,     // C act  [m][n] (rounded)
  EPI_RESID = 2,   // C act  [m][n] = round(C + acc)
  EPI_SWIGLU = 3,  // C act  [m][j] = round(silu(gate_j) * up_j); B rows: gate j, up half+j
  EPI_LM = 4,      // per-row (max, idx, second, sum e^(z-max), sum e^(z-max)(z-max)) over the tile
  EPI_QKV = 5,     // bf16 QKV projection with head_dim 128: round q/k/v, RoPE q and k (table), scatter
};

struct GemmArgs {
  const void* A = nullptr;
  long long lda = 0;
  const int* a_rows = nullptr;     // optional gather: A row of output row m is a_rows[m]
  const void* B = nullptr;
  long long ldb = 0;
  long long b_gstride = 0;         // elements between consecutive groups' B
  const float* b_scale = nullptr;  // fp8 row scales of B (per output row of B)
  long long s_gstride = 0;
  int M = 0, N = 0, K = 0;         // N: output columns (SWIGLU: outputs j, i.e. gate rows)
  const int* g_off = nullptr;      // [G+1] row ranges of groups (grid.z = G); null: one group
  void* C = nullptr;
  long long ldc = 0;
  int swiglu_half = 0;             // SWIGLU: B row of up_j is swiglu_half + j
  float* part = nullptr;           // EPI_LM partials [M][n_tiles][5]
  int* flags = nullptr;            // EPI_LM: FLAG_NONFINITE when a lane's logits of a row are all NaN/-inf (nullable)
  // EPI_QKV: row m = canvas b * seq_n + token i; q -> q_out [B][heads][seq_n][128];
  // k, v -> (b, h) planes at k_dst / v_dst + (b * heads + h) * dst_bh + (row0 + i) * 128;
  // rope_tab [seq_n][64] (cos, sin) pairs
  void* q_out = nullptr;
  void* k_dst = nullptr;
  void* v_dst = nullptr;
  long long dst_bh = 0;
  int row0 = 0, seq_n = 0, heads = 0;
  const float* rope_tab = nullptr;
  // optional second product over the same A (bf16 direct-load kernel only):
  // C2[m][n] = sum_k A[m][k] * B2[n][k] (fp32), n < N2, in the same launch
  const void* B2 = nullptr;
  long long ldb2 = 0;
  int N2 = 0;
  float* C2 = nullptr;
  long long ldc2 = 0;
  // optional router top-k in the same launch (gemm_f32_topk only): ids and
  // weights [tk_T][tk_k] from the router logits tk_logits [tk_T][tk_E]
  const float* tk_logits = nullptr;
  int tk_T = 0, tk_E = 0, tk_k = 0;
  int* tk_ids = nullptr;
  float* tk_w = nullptr;
};

// Returns 0 or a HIP error code.
int gemm(ActType at, WType wt, GemmEpi epi, const GemmArgs& g, int groups, hipStream_t st);
// EPI_F32 product (bf16 A and B, K = 2048, M <= 512, N >= 1024) with the
// router top-k of g.tk_* in the same launch, on workgroups of their own that
// run beside the product's tiles.  Returns -1 (nothing launched) when the
// shape is not covered (also tk_E > 128 or tk_k > 8), else 0 or a HIP error.
int gemm_f32_topk(const GemmArgs& g, hipStream_t st);
// Routed experts with bf16 weights in the tiled layout, as grouped 128 x 128
// tiles over expert-major pair lists (off [E+1], pair_row [pairs]):
// gate/up (X = normed rows [T][K], gathered by pair_row) -> h [pairs][Nout]
// bf16 SwiGLU; down (X = h [pairs][K], one row per pair) -> y [pairs][Nout]
// fp32.  Same bits as moe_experts.  Shapes: grouped_supported.
bool grouped_supported(bool gate_up, int K, int Nout, int E);
int grouped_experts(bool gate_up, const void* X, const int* pair_row, const int* off, int E, int pairs,
                    const void* W, int K, int Nout, void* out, hipStream_t st);
// Number of vocab tiles the LM epilogue writes per row (depends on the kernel
// gemm() routes the LM head to).
int lm_tiles(ActType at, int K, int vocab);
// Tiled bf16 kernel (k_tgemm.hip): used by gemm() for ungrouped bf16 GEMMs with K % 64 == 0.
bool tgemm_supported(ActType at, int K);
int tgemm(WType wt, GemmEpi epi, const GemmArgs& g, hipStream_t st);
int lm_tiles_tiled(int vocab, int K);
// Merge LM partials of T rows into entropy / argmax / top-2 gap; FLAG_NONFINITE
// (flags nullable) for a row whose entropy is not finite or that has no argmax.
int lm_merge(const float* part, int T, int n_tiles, float* entropy, int* argmax, float* gap, int* flags,
             hipStream_t st);

// ---------------------------------------------------------------- routed experts (k_moe.hip)
// bf16 activations, bf16 or fp8 weights.  gate_up: h[p][j] = bf16(silu(x.Wg_j) * x.Wu_j) with x the
// token row pair_row[p] of X [T][K] and W [E][2*Nout][K]; otherwise y[p][n] = X[p] . W[n] (fp32)
// with W [E][Nout][K].  Pairs of expert e are [off[e], off[e+1]).  W is in the tiled layout of
// moe_pack (Nout and K multiples of 16 and 32).
// route (gate/up only, may be null): derive the routing from the top-k ids in the kernel instead
// of reading off/pair_row, and write off [E+1], pair_row [T*k] and pos [T][k] for later kernels.
struct MoeRoute {
  const int* ids;  // [T][k]
  int T, k;        // T <= 2048
  int* off;
  int* pair_row;
  int* pos;
};
// pairs: T * k (sizes the token passes; 0 = few pairs per expert); with a
// route, the larger of this and route->T * route->k.
// scale: W_FP8 fp32 row scales [E][rows]; W_FP4 / W_FP4A8 the tiled E8M0
// block scales (moe_pack_scales); otherwise null.
// xq, xqs (W_FP4A8 only): the MXFP8 codes [rows][K] and E8M0 scales
// [rows][K/32] of X's rows (mx8_quantize / rmsnorm); K % 128 == 0.
int moe_experts(WType wt, bool gate_up, const void* X, const int* pair_row, const int* off, int E,
                const void* W, const void* scale, int K, int Nout, void* out, hipStream_t st,
                const MoeRoute* route = nullptr, int pairs = 0, const uint8_t* xq = nullptr,
                const uint8_t* xqs = nullptr);
// Row-major [n_mats][rows][cols] expert matrices -> the tiled layout moe_experts reads
// (rows % 16 == 0, cols % 32 == 0, W_FP4: cols % 64 == 0 with two codes per
// byte; src and dst must not overlap).
int moe_pack(WType wt, const void* src, void* dst, long long n_mats, int rows, int cols, hipStream_t st);
// MXFP4 block scales [n_mats][rows][K/32] -> one scale tile per weight tile
// (rows % 16 == 0, K % 64 == 0).
int moe_pack_scales(const void* src, void* dst, long long n_mats, int rows, int K, hipStream_t st);
// out[32 b + i] = bf16(E2M1 code i of block b of packed * 2^(scales[b] - 127)) (test)
int fp4_decode(const void* packed, const uint8_t* scales, int n_blocks, void* out, hipStream_t st);

// ---------------------------------------------------------------- attention (k_attn.hip)
struct AttnArgs {
  const void* q;          // (b,h) planes q_bh elements apart, rows of dh: [B][H][n][dh] when q_bh = n*dh
  long long q_bh;
  const void* k0;         // segment 0 keys: (b,h) at k0 + (b*H+h)*s0_bh, rows [0, len0)
  const void* v0;
  long long s0_bh;        // elements between (b,h) planes of segment 0
  int len0;
  const void* k1;         // segment 1 keys (may be null if len1 == 0)
  const void* v1;
  long long s1_bh;
  int len1;
  int causal_base;        // -1: bidirectional; else query i sees keys j <= causal_base + i
  int B, H, n, dh;
  void* out;              // [B*n][H*dh] act
  float* part_o;          // split partials [splits][B*H][n][dh]
  float* part_ml;         // [splits][B*H][n][2]
  int splits;
};
int attention(ActType at, const AttnArgs& a, hipStream_t st);
int attn_splits_for(ActType at, int B, int H, int n, int keys, int dh);
// Up to ATTN_MAX_SEGS problems (same head_dim) in one launch plus one merge
// launch, bf16 only.  Sets each problem's splits and partial pointers
// (packed from part_o / part_ml; room for max_splits x all their rows).
constexpr int ATTN_MAX_SEGS = 16;
int attention_segments(ActType at, AttnArgs* segs, int n, int max_splits, float* part_o, float* part_ml,
                       hipStream_t st);

// ---------------------------------------------------------------- static scratch (k_scratch.hip)
// Bytes of the file-scope device array the allocation-free LM-head entry
// keeps its partials in: T x (LM tiles) x 5 floats, 40 KB per row at 262144
// ids, so one 256-position canvas fits.
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(16) << 20;
// Device address of that array on the current device (looked up with
// hipGetSymbolAddress on a device's first call and kept).  0 or a HIP error.
int noalloc_scratch(void** ptr);

// ---------------------------------------------------------------- misc (k_misc.hip)
// ids outside [0, vocab) read row 0 and raise FLAG_TOKEN in *flags (nullable);
// tok2 (nullable): add the rows of these ids too (one rounding of the sum)
int embed_gather(ActType at, const int* tok, int T, const void* E, int d, int vocab, void* x, int* flags,
                 hipStream_t st, const int* tok2 = nullptr);
// q8 / q8s (bf16, d % 32 == 0): also write the normed rows as MXFP8 codes
// [T][d] and E8M0 scales [T][d/32], as mx8_quantize does.
int rmsnorm(ActType at, const void* x, int T, int d, float eps, void* y, hipStream_t st, uint8_t* q8 = nullptr,
            uint8_t* q8s = nullptr);
// bf16 rows x [T][d] (d % 32 == 0) -> MXFP8: E4M3FN codes [T][d] and one
// E8M0 scale per 32 elements [T][d/32] (OCP MX conversion, round to nearest
// even, clamp at 448).
int mx8_quantize(const void* x, int T, int d, uint8_t* q8, uint8_t* q8s, hipStream_t st);
// tab[i][j] = (cos, sin) of (pos0 + i) * theta^(-2j/dh), i < n, j < dh/2 (float pairs)
int rope_table(int n, int dh, int pos0, float theta, float* tab, hipStream_t st);
// Rows of a mixed batch: segment s holds rows [start[s], start[s + 1]) at
// positions pos0[s] + (row - start[s]).
constexpr int MAX_SEGMENTS = 16;
struct RowSegments {
  int n_segs;
  int start[MAX_SEGMENTS + 1];
  int pos0[MAX_SEGMENTS];
};
// tab[r][j] = (cos, sin) of the position of row r (as rope_table), r < start[n_segs]
int rope_table_rows(const RowSegments& rs, int dh, float theta, float* tab, hipStream_t st);
// dst planes (h) at dst_k / dst_v + h * dst_bh, rows row0 .. row0 + n - 1 <- src planes
// (src_bh apart) rows 0 .. n - 1 (dh elements of act dtype per row)
int kv_copy_rows(ActType at, const void* src_k, const void* src_v, long long src_bh, int H, int n, int dh,
                 void* dst_k, void* dst_v, long long dst_bh, int row0, hipStream_t st);
// RoPE on q,k from qkv [T][3A] (T = B*n, token i rotated by tab row i) and scatter:
// q -> q_out [B][H][n][dh]; k,v -> (b,h) planes at kdst/vdst + (b*H+h)*dst_bh + (row0+i)*dh.
int rope_scatter(ActType at, const void* qkv, int B, int n, int H, int dh, const float* tab, void* q_out,
                 void* kdst, void* vdst, long long dst_bh, int row0, hipStream_t st);
// x[t] = round(x[t] + sum_j w[t][j] * y[pos[t][j]] + ys[t]); FLAG_NONFINITE in
// *flags when an updated value is not finite
int moe_combine(ActType at, void* x, const float* y, const float* ys, const float* w,
                const int* pos, int T, int k, int d, int* flags, hipStream_t st);
// moe_combine, then a = rmsnorm(x) of the updated rows (one fused kernel for bf16)
int moe_combine_norm(ActType at, void* x, const float* y, const float* ys, const float* w, const int* pos,
                     int T, int k, int d, float eps, void* a, int* flags, hipStream_t st);
// mask_token >= 0: absorbing-state noise (the canvas starts as [MASK] and
// uncommitted positions return to it); -1: uniform Philox draws
int canvas_init(int* tok, uint8_t* committed, int B, int N, uint64_t seed, uint32_t block,
                int vocab, int mask_token, hipStream_t st);
// tok[i] = given[i], committed[i] = 1 wherever mask[i] != 0 (i < n)
int canvas_prefill(int* tok, uint8_t* committed, int n, const int* given, const uint8_t* mask, hipStream_t st);
// live_flags (nullable): the status word the step's kernels raised; it is
// copied to *status (nullable) and cleared.
int commit_renoise(const float* H, const int* am, int* tok, uint8_t* committed, int B, int N,
                   int step, int max_steps, float threshold, uint64_t seed, uint32_t block,
                   int vocab, int mask_token, int* n_unc, int* live_flags, int* status, hipStream_t st);
// *published = *live; *live = 0 (one thread)
int status_publish(int* live, int* published, hipStream_t st);
int philox_fill(uint64_t seed, uint32_t pos0, uint32_t tag, uint32_t canvas, uint32_t block,
                uint32_t modulus, int n, uint32_t* out, hipStream_t st);

// ---------------------------------------------------------------- router (k_router.hip)
// logits [T][E] fp32 -> ids [T][k], w [T][k]
int router_topk(const float* logits, int T, int E, int k, int* ids, float* w, hipStream_t st);
// Rows t with forced[t][0] >= 0 take the ids forced[t][0..k) in that slot order
// and the softmax of their logits as weights (a test hook: lines the routing
// up with a reference where two router logits nearly tie).
int router_force(const float* logits, int T, int E, int k, const int* forced, int* ids, float* w, hipStream_t st);
// ids [T][k] -> off[E+1], pair_row[T*k] (token of each pair slot, expert-major,
// token-ascending), pos[T][k] (slot of pair (t, j)).  Above 2048 tokens it
// needs scratch of router_permute_scratch(T, E) bytes (8-byte aligned).
int router_permute(const int* ids, int T, int E, int k, int* off, int* pair_row, int* pos, hipStream_t st,
                   void* scratch = nullptr);
size_t router_permute_scratch(int T, int E);
// counts[e] (+)= off[e + 1] - off[e] for e < E (diagnostic; accumulate adds)
int expert_counts(const int* off, int E, int* counts, bool accumulate, hipStream_t st);

}  // namespace dg
