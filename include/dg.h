/*
 * dg.h -- C ABI of the block-diffusion denoise library for MI355X (gfx950).
 *
 * The library runs the hot path of DiffusionGemma-style block diffusion
 * decoding on one GPU.  A canvas of `canvas_len` tokens starts from uniform
 * random ids and is refined in denoise steps.  Every step
 *   1. runs the backbone over all canvas positions with bidirectional,
 *      unmasked attention over the prompt KV cache plus the whole canvas
 *      (DiffusionGemma解析, "换个路数：整片并行去噪的生成机制"; zhichai.net
 *      深度拆解, "双向注意力: BERT 的遗产"), each layer holding a mixture of
 *      experts with top-k routing and one shared expert (zhichai.net 深度拆解,
 *      "MoE 效率：128 专家，8 活跃");
 *   2. scores each position by the entropy of its output distribution and
 *      takes its argmax (DiffusionGemma解析, same section: lower entropy means
 *      more certain);
 *   3. commits the most certain uncommitted positions, ranked by entropy
 *      (ipcmen.com, "工作原理：并行精炼与自我修正": lock the most confident
 *      tokens), and
 *   4. redraws every still-uncommitted position uniformly at random
 *      (zhichai.net 深度拆解, "统一状态扩散 vs 掩码扩散").
 * Steps repeat until every position is committed or `max_steps` (48 in the
 * pages: DiffusionGemma解析, "自适应停步机制") have run.  A committed canvas is
 * appended to the KV cache by a causal pass before the next canvas starts
 * (zhichai.net 深度拆解, "Block-Autoregressive：块内并行，块间串行").
 *
 * Conventions for every entry point:
 *  - All pointers inside the structs below are DEVICE pointers unless a field
 *    says "host".  The library never frees caller memory; it owns only the
 *    workspace it allocates in dg_model_create and frees in dg_model_destroy.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    on it asynchronously; only dg_generate_canvas blocks (it reads back the
 *    4-byte count of uncommitted positions after every step).
 *  - Arguments are validated before anything is launched.  On failure the
 *    call returns a negative dg_status, enqueues nothing, and leaves caller
 *    state unchanged; dg_last_error() then describes the failure (per thread).
 *  - Calls on one model must not overlap (the workspace is shared).
 *  - Numeric and token faults are detected on the device: kernels raise bits
 *    of a status word (DG_STATUS_*) in the model, and every denoise step
 *    publishes the bits raised since the previous step (by its own kernels
 *    and by any dg_commit_canvas in between) and clears them.
 *    dg_generate_canvas reads the word back after each step and stops with
 *    DG_ERR_NUMERIC or DG_ERR_INVALID_ARG; dg_denoise_step, which does not
 *    wait for the device, copies it to dg_step_out.status.
 *
 * Layouts (row-major, innermost dimension last; T = batch * tokens):
 *  - activations/weights in `act_dtype` (FP32 or BF16); routed and shared
 *    expert weights in `expert_dtype` (FP32, BF16, FP8_E4M3 codes with one
 *    fp32 scale per output row: w = decode(code) * scale[row], or MXFP4 for the
 *    routed experts with E8M0 block scales and a BF16 shared expert).
 *  - weight matrices are [out][in]: y = W x.
 *  - KV cache: k and v are each [n_layers][batch][n_heads][capacity][head_dim]
 *    in act_dtype, holding rotary-embedded keys and the values.
 */
#ifndef DG_H
#define DG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DG_OK = 0,
  DG_ERR_INVALID_ARG = -1,   /* null pointer, bad enum, unsupported combination */
  DG_ERR_SHAPE = -2,         /* sizes inconsistent or beyond what the model was created for */
  DG_ERR_HIP = -3,           /* a HIP runtime call failed (message in dg_last_error) */
  DG_ERR_OOM = -4,           /* workspace allocation failed */
  DG_ERR_STATE = -5,         /* step counter already at max_steps, or similar */
  DG_ERR_NUMERIC = -6,       /* non-finite values in the residual stream or the logits */
  DG_ERR_UNIMPLEMENTED = -7
} dg_status;

/* DG_DTYPE_MXFP4 (expert_dtype only): routed experts in OCP MX FP4 -- E2M1
 * codes, two per byte (the even element in the low nibble), one E8M0 scale
 * (2^(e-127)) per 32 consecutive weights along the input dimension; the
 * shared expert stays BF16.  The MI355X counterpart of the 4-bit expert
 * weights the pages name (DiffusionGemma深度拆解 (zhichai.net), "MoE 效率：128
 * 专家，8 活跃").  DG_DTYPE_E8M0 names the block scales for dg_pack_experts.
 * DG_DTYPE_MXFP4_MXFP8 (expert_dtype only): the same MXFP4 weights and scales
 * (packed as DG_DTYPE_MXFP4), with the routed gate/up reading its token rows
 * as OCP MX FP8: per row and 32 consecutive elements one E8M0 scale 2^s with
 * s = floor(log2(max |v|)) - 8 (an all-zero block: code 0), each element
 * v / 2^s rounded to E4M3FN, nearest with ties to even, clamped to +-448.
 * The products run on gfx950's scaled MFMA (4-bit x 8-bit operands); the
 * routed down and the shared expert read bf16 as with DG_DTYPE_MXFP4.  Needs
 * d_model % 128 == 0. */
enum {
  DG_DTYPE_FP32 = 0,
  DG_DTYPE_BF16 = 1,
  DG_DTYPE_FP8_E4M3 = 2,
  DG_DTYPE_MXFP4 = 3,
  DG_DTYPE_E8M0 = 4,
  DG_DTYPE_MXFP4_MXFP8 = 5
};

/* Bits of the device status word (dg_step_out.status). */
enum {
  DG_STATUS_NONFINITE = 1,  /* a NaN or infinity after a block's residual add, or among a row's logits */
  DG_STATUS_TOKEN = 2       /* a token id outside [0, vocab) reached the embedding (row 0 was read) */
};

/* Model shape and decoding rule.  All fields are plain values (host). */
typedef struct dg_config {
  int32_t n_layers;
  int32_t d_model;
  int32_t n_heads;
  int32_t head_dim;        /* even; attention scale 1/sqrt(head_dim) */
  int32_t n_experts;       /* routed experts, <= 256 */
  int32_t top_k;           /* experts per token, <= min(n_experts, 8) */
  int32_t d_expert;        /* SwiGLU width of a routed expert */
  int32_t d_shared;        /* SwiGLU width of the shared expert */
  int32_t vocab;
  int32_t canvas_len;      /* positions per canvas, <= 1024 */
  int32_t max_steps;       /* denoise step cap S_max */
  float rope_theta;        /* RoPE base; 0 disables rotary embedding */
  float rms_eps;           /* RMSNorm epsilon (inside the square root) */
  float commit_threshold;  /* nats: uncommitted positions with entropy below it commit */
  int32_t act_dtype;       /* DG_DTYPE_FP32 or DG_DTYPE_BF16 */
  int32_t expert_dtype;    /* FP32 (with act FP32), BF16, FP8_E4M3, MXFP4 or MXFP4_MXFP8 (with act
                              BF16; MXFP4 needs d_model and d_expert multiples of 64, MXFP4_MXFP8
                              also d_model % 128 == 0) */
  int32_t mask_token;      /* -1: uniform-state noise (Philox draws, the method of the pages);
                              0 .. vocab-1: absorbing-state (mask) noise with this [MASK] id --
                              the canvas starts as all [MASK] and every uncommitted position is
                              set back to [MASK] after each step (the masked-diffusion variant
                              the pages contrast it with: DiffusionGemma深度拆解 (zhichai.net),
                              "统一状态扩散 vs 掩码扩散"); nothing else changes */
  int32_t self_condition;  /* 0 or 1: self-conditioning, one of the techniques the model combines
                              (openai-hub.com, "为什么扩散能跑得比自回归快"; named only).  Reading:
                              every step after a canvas's first adds the embedding row of the
                              previous step's argmax at each position (dg_canvas.prediction) to
                              the position's input embedding, one sum rounded once to act_dtype;
                              the first step (step == 0) adds nothing */
} dg_config;

/* One layer's weights (device pointers, borrowed for the model's lifetime).
 *
 * Routed-expert matrices w_gu and w_d in BF16 or FP8_E4M3 are passed in the
 * tiled layout that dg_pack_experts writes from the row-major matrices above
 * (FP32 experts stay row-major): every 16-row by TK-column block of a matrix
 * [rows][cols] is one contiguous tile, tiles ordered by 16-row block, then by
 * column block.  TK is 32 for BF16 and, for FP8, 64 when cols % 64 == 0, else
 * 32.  Inside a tile, slice l = 0..63 (TK/4 elements, 16 or 8 bytes) holds
 * row l % 16 of the block, columns (l / 16) * TK/4 .. +TK/4-1 of the tile.
 * This is the operand layout of the 16x16x32 matrix-core instruction, so a
 * wavefront fetches one weight fragment as a single contiguous 1 KB read.
 * The FP8 scales s_gu/s_d stay per row in row order.  MXFP4 tiles are 16 rows
 * by TK = 128 codes (64 bytes per row; TK = 64 when cols % 128 != 0), slice l
 * holding row l % 16, codes (l / 16) * TK/4 onward; their E8M0 scales
 * s_gu/s_d are tiled alike: per weight tile, 16 x TK/32 bytes, row-major
 * (row, 32-code block). */
typedef struct dg_layer_weights {
  const void* wqkv;    /* [3*n_heads*head_dim][d_model]: q rows, k rows, v rows */
  const void* wo;      /* [d_model][n_heads*head_dim] */
  const void* wr;      /* router [n_experts][d_model] (act_dtype) */
  const void* w_gu;    /* [n_experts][2*d_expert][d_model]: gate rows then up rows (tiled, below) */
  const void* w_d;     /* [n_experts][d_model][d_expert] (tiled, below) */
  const void* s_gu;    /* FP8: fp32 [n_experts][2*d_expert] row scales; MXFP4: E8M0 block
                          scales [n_experts][2*d_expert][d_model/32] (tiled); else NULL */
  const void* s_d;     /* FP8: fp32 [n_experts][d_model]; MXFP4: [n_experts][d_model][d_expert/32] */
  const void* ws_gu;   /* shared expert [2*d_shared][d_model] */
  const void* ws_d;    /* shared expert [d_model][d_shared] */
  const float* ss_gu;  /* FP8 only: [2*d_shared] */
  const float* ss_d;   /* FP8 only: [d_model] */
} dg_layer_weights;

typedef struct dg_weights {
  const void* embed;                  /* [vocab][d_model], act_dtype */
  const void* lm_head;                /* [vocab][d_model], act_dtype (untied) */
  const dg_layer_weights* layers;     /* host array of n_layers entries (copied at create) */
} dg_weights;

/* KV cache (caller-owned device memory, layout in the header comment). */
typedef struct dg_kv {
  void* k;
  void* v;
  int32_t batch;       /* canvases; each has its own cache rows */
  int32_t capacity;    /* rows per (layer, canvas, head) */
  int32_t length;      /* rows in use; advanced by dg_commit_canvas */
} dg_kv;

/* Canvas state.  tokens/committed are device arrays of [batch][canvas_len].
 * Random draws use Philox4x32-10 with key (seed mod 2^32, seed >> 32) and
 * counter (position, step_tag, canvas index b, block): step_tag 0 for
 * dg_canvas_init, s + 1 for the re-noise after step s.  */
typedef struct dg_canvas {
  int32_t* tokens;
  uint8_t* committed;  /* 0 or 1; only ever goes 0 -> 1 */
  int32_t batch;
  int32_t step;        /* host: steps already taken (0-based index of the next step) */
  uint64_t seed;
  uint32_t block;      /* canvas ordinal in block-autoregressive generation */
  int32_t* prediction; /* [batch][canvas_len] device: with self_condition, each step writes its argmax
                          here and every later step reads it (required then; unused otherwise) */
} dg_canvas;

/* Optional per-step outputs (each pointer may be NULL = not written). */
typedef struct dg_step_out {
  float* entropy;          /* [batch][canvas_len] nats, from the fp32 logits */
  int32_t* argmax;         /* [batch][canvas_len] lowest id among maxima */
  float* top2_gap;         /* [batch][canvas_len] largest minus second-largest logit */
  int32_t* n_uncommitted;  /* [batch] after this step's commit */
  float* logits;           /* test/diagnostic: [batch*canvas_len][vocab] fp32 (extra GEMM) */
  void* hidden;            /* test/diagnostic: final normed hidden [batch*canvas_len][d_model] */
  int32_t* status;         /* [1] DG_STATUS_* bits raised since the previous step; 0 = clean */
  int32_t* expert_counts;  /* diagnostic: [n_layers][n_experts] (token, slot) pairs routed to each
                              expert in each layer (all canvases pooled) */
} dg_step_out;

typedef struct dg_model dg_model;

const char* dg_status_str(int status);
const char* dg_last_error(void);
/* Library version string. */
const char* dg_version(void);

/* Create a model over borrowed weights.  `max_batch` canvases per call and up
 * to `max_tokens` tokens per canvas in dg_commit_canvas (>= canvas_len) size
 * the workspace, which is allocated here once.  `max_kv` is the largest KV
 * capacity (rows per layer, canvas and head) any call may pass: calls with a
 * larger kv->capacity fail with DG_ERR_SHAPE.  0 takes the kernels' own
 * limit, 2^31 / (head_dim x element size) rows (attention addresses a cache
 * plane with 32-bit byte offsets); a larger max_kv is refused.  The rows of
 * one call, max_batch x max(max_tokens, canvas_len), may be at most 8192
 * (DG_ERR_SHAPE otherwise).  With BF16 experts at d_model 2048 the routed
 * experts take all of a call's rows in one launch once they hold about 80
 * pairs per expert (grouped tiles); otherwise more than 2048 rows (1024 with
 * fp32 activations) run in chunks, each streaming the expert weights once.
 * Must be called with the target device current. */
int dg_model_create(const dg_config* cfg, const dg_weights* w, int32_t max_batch,
                    int32_t max_tokens, int32_t max_kv, dg_model** out);
int dg_model_destroy(dg_model* m);

/* Draw the initial canvas (step_tag 0) and clear `committed`; sets step = 0.
 * The canvas starts as uniform random ids (DiffusionGemma解析,
 * "换个路数：整片并行去噪的生成机制": generation starts from a canvas of random
 * tokens), or as all [MASK] under absorbing-state noise. */
int dg_canvas_init(dg_model* m, dg_canvas* c, void* stream);

/* Pre-commit known positions of a freshly initialised canvas (fill-in-the-
 * middle and constraint tasks: DiffusionGemma深度拆解 (zhichai.net),
 * "代码填充的结构性优势"; the denoiser refines the open positions around
 * fixed ones).  `tokens` and `mask` are device arrays of
 * [batch][canvas_len] (int32 ids in [0, vocab), uint8 0/1): wherever
 * mask != 0 the canvas takes that token and the position is committed, so
 * the commit schedule counts only the open positions and re-noising never
 * touches it.  Call after dg_canvas_init and before the first step
 * (c->step == 0, else DG_ERR_STATE); stream-ordered.  Token values are not
 * checked on the host (they are device-resident). */
int dg_canvas_prefill(dg_model* m, dg_canvas* c, const int32_t* tokens, const uint8_t* mask, void* stream);

/* One denoise step on every canvas of `c` against the first kv->length cache
 * rows: the canvas refinement phase (ipcmen.com, "模型构建与底层优化": a
 * request's canvas is refined with bidirectional attention; DiffusionGemma解析,
 * "换个路数：整片并行去噪的生成机制": all positions are scored at once, ranked by
 * entropy, the most certain frozen; ipcmen.com, "工作原理：并行精炼与自我修正":
 * the uncertain positions are randomised again).  Forward over all positions
 * (committed ones included), entropy and argmax per position, commit of the
 * ceil(U / (max_steps - step)) lowest-entropy uncommitted positions plus those
 * below commit_threshold, re-noise of the rest.  Requires c->step < max_steps
 * (DG_ERR_STATE otherwise); increments c->step.  kv->batch must equal
 * c->batch.  Asynchronous: the step's status word goes to out->status. */
int dg_denoise_step(dg_model* m, dg_canvas* c, const dg_kv* kv, dg_step_out* out, void* stream);

/* Run denoise steps from the canvas's current state until every position of
 * every canvas is committed or max_steps is reached (DiffusionGemma解析,
 * "自适应停步机制": the loop stops as soon as the canvas is settled, after at
 * most 48 steps).  Blocks: after each step it reads back the uncommitted
 * counts and the status word; a raised DG_STATUS_NONFINITE returns
 * DG_ERR_NUMERIC and DG_STATUS_TOKEN returns DG_ERR_INVALID_ARG, after the
 * step that published it.  Writes the number of steps this call ran to
 * *steps_taken (host), also on those errors. */
int dg_generate_canvas(dg_model* m, dg_canvas* c, const dg_kv* kv, int32_t* steps_taken,
                       void* stream);

/* Causal pass over tokens[batch][n] (device) at positions kv->length ..
 * kv->length+n-1: the prompt read and block commit phases (ipcmen.com,
 * "模型构建与底层优化"; zhichai.net 深度拆解, "Block-Autoregressive：块内并行，
 * 块间串行": a committed canvas is encoded causally and appended to the KV
 * cache before the next canvas starts).  Writes their rotary-embedded keys
 * and values into every layer's cache rows [length, length+n) and advances
 * kv->length by n.  Token i attends to all cached rows and to new tokens
 * j <= i.  Requires length + n <= capacity <= max_kv and n <= max_tokens
 * (DG_ERR_SHAPE, nothing enqueued).  Token ids are not checked on the host;
 * an id outside the vocabulary reads row 0 and raises DG_STATUS_TOKEN, which
 * the next denoise step publishes. */
int dg_commit_canvas(dg_model* m, const int32_t* tokens, int32_t n, dg_kv* kv, void* stream);

/* One segment of a mixed-phase batch (dg_mixed_step).  Each segment is one
 * request with its own batch-1 KV cache (kv->batch == 1; no two segments may
 * share a cache).
 *  - DG_SEG_REFINE: one denoise step of `canvas` (batch 1, step < max_steps)
 *    against the first kv->length cache rows, exactly as dg_denoise_step;
 *    n == canvas_len; entropy/argmax (device, [canvas_len], may be NULL)
 *    receive the step's per-position confidence, n_uncommitted (device [1],
 *    may be NULL) the count after the commit.  Increments canvas->step.
 *  - DG_SEG_APPEND: a causal pass over tokens[n] (device, n <= max_tokens),
 *    exactly as dg_commit_canvas: a prompt read, or a committed canvas being
 *    appended.  Writes the rows' keys and values at kv->length .. +n-1 of every
 *    layer and advances kv->length by n (length + n <= capacity). */
enum { DG_SEG_APPEND = 0, DG_SEG_REFINE = 1 };
typedef struct dg_segment {
  int32_t kind;            /* DG_SEG_APPEND or DG_SEG_REFINE */
  int32_t n;               /* rows: tokens to append, or canvas_len */
  dg_kv* kv;               /* host pointer to the request's cache descriptor (length/step updated) */
  const int32_t* tokens;   /* APPEND: device [n] */
  dg_canvas* canvas;       /* REFINE: host pointer to a batch-1 canvas */
  float* entropy;          /* REFINE, optional: device [canvas_len] */
  int32_t* argmax;         /* REFINE, optional: device [canvas_len] */
  int32_t* n_uncommitted;  /* REFINE, optional: device [1] */
  void* hidden;            /* REFINE, test/diagnostic: final normed hidden [canvas_len][d_model] */
} dg_segment;

/* One pass over a batch of requests in different phases -- prompt reads and
 * block commits (causal) next to canvas refinements (bidirectional): the
 * serving requirement that every request picks its own attention mode within
 * one batch (ipcmen.com, "模型构建与底层优化": requests cycle through prompt
 * reading, canvas refinement and block commit, switching between causal and
 * bidirectional attention).  The segments' rows are stacked (refine segments
 * first) and every block runs its dense projections, shared expert, router
 * and routed experts once over all rows -- the expert weights stream once for
 * the whole mix -- while attention runs per segment in that segment's mode
 * over its own cache.  Each segment's results equal those of its own
 * dg_denoise_step or dg_commit_canvas up to fp32 summation order (row
 * positions and chunking differ).  1 <= n_segs <= 16; the total rows must fit
 * the workspace (max_batch x max(max_tokens, canvas_len)) and the refine rows
 * max_batch x canvas_len, else DG_ERR_SHAPE; every segment is validated
 * before anything is enqueued.  Token and numeric faults raise the status
 * word as in the other entries; the pass publishes it to *status (device [1],
 * may be NULL).  Asynchronous; updates canvas->step and kv->length on the
 * host. */
int dg_mixed_step(dg_model* m, dg_segment* segs, int32_t n_segs, int32_t* status, void* stream);

/* Rewrite n_mats row-major expert matrices src[n_mats][rows][cols] (BF16,
 * FP8_E4M3 codes, or MXFP4 codes two per byte) into the tiled layout
 * dg_layer_weights describes, at dst (same byte size, must not overlap src).
 * rows % 16 == 0, cols % 32 == 0 (MXFP4: cols % 64 == 0; cols counts codes).
 * DG_DTYPE_E8M0 packs the MXFP4 block scales src[n_mats][rows][cols/32] of
 * such matrices into their scale tiles.  Stream-ordered; done once when
 * weights are loaded. */
int dg_pack_experts(const void* src, void* dst, int64_t n_mats, int32_t rows, int32_t cols,
                    int32_t dtype, void* stream);

/* Allocation-free variant of dg_test_lm_head, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the fused LM head + confidence on given
 * normed hidden rows hf[T][d_model] (act_dtype, device) with the model's
 * LM-head weights, writing entropy[T], argmax[T] and (if not NULL)
 * top2_gap[T].  Its per-(row, column tile) partials live in a static device
 * array of 16 MiB instead of the model's workspace: T x 20 bytes per LM tile
 * (40 KB per row at 262144 ids, so up to 409 rows there); a larger T fails
 * with DG_ERR_SHAPE before anything is enqueued.  It calls no allocator.  The
 * array is one per GPU and shared by every call on it: calls that overlap on
 * one GPU (other streams, other threads, other models) race on it.  Nothing
 * in it needs clearing -- each call writes every partial it reads.
 * Stream-ordered; results equal dg_test_lm_head's bit for bit. */
int dg_lm_head_confidence_noalloc(const dg_model* m, const void* hf, int32_t T, float* entropy, int32_t* argmax,
                                  float* top2_gap, void* stream);

/* ---- kernel timing ---------------------------------------------------------
 * Measures one kernel class with HIP events recorded on the stream each of its
 * launches goes to (start before, stop after the launch), so a benchmark can
 * time it inside its own timed region.  dg_profile_kernel selects the class
 * (DG_PROF_NONE disables) and allocates the event pool (1024 pairs) -- call it
 * outside timed or captured regions; dg_profile_read waits for the recorded
 * events, returns the summed duration (ms) and the launch count, and resets. */
enum {
  DG_PROF_NONE = 0,
  DG_PROF_ATTN = 1,        /* canvas attention (+ split merge) */
  DG_PROF_MOE_GATEUP = 2,  /* routed experts: gate/up GEMM + SwiGLU */
  DG_PROF_MOE_DOWN = 3,    /* routed experts: down GEMM */
  DG_PROF_LM_HEAD = 4,     /* LM head + entropy/argmax epilogue + merge */
  DG_PROF_QKV = 5,         /* QKV projection */
  DG_PROF_SHARED = 6,      /* shared expert (gate/up + down) */
  DG_PROF_ROUTER = 7,      /* router GEMM + top-k + permutation */
  DG_PROF_COMMIT = 8       /* commit selection + re-noise */
};
int dg_profile_kernel(dg_model* m, int32_t kernel_id);
int dg_profile_read(dg_model* m, double* total_ms, int64_t* launches);

/* ---- test-only entry points (not part of the product API) ---------------- */

/* out[i] = Philox4x32-10 word 0 of counter (pos0+i, step_tag, canvas, block)
 * under key `seed`, modulo `modulus` (0 = no reduction).  n <= 2^24. */
int dg_test_philox(uint64_t seed, uint32_t pos0, uint32_t step_tag, uint32_t canvas,
                   uint32_t block, uint32_t modulus, int32_t n, uint32_t* out, void* stream);

/* Fused LM head + confidence on given normed hidden rows hf[T][d_model]
 * (act_dtype): writes entropy/argmax/top2_gap for T rows (T <= workspace). */
int dg_test_lm_head(dg_model* m, const void* hf, int32_t T, float* entropy, int32_t* argmax,
                    float* top2_gap, void* stream);

/* E2M1 codes packed[n_blocks * 16] (bytes, two codes each) with E8M0 scales
 * scales[n_blocks] -> out[n_blocks * 32] bf16, through the widening the
 * MXFP4 expert kernels use. */
int dg_test_fp4_decode(const uint8_t* packed, const uint8_t* scales, int32_t n_blocks, void* out, void* stream);

/* bf16 rows x[rows][d] (d % 32 == 0; with norm, d <= 8192) -> MXFP8 as the
 * MXFP4_MXFP8 experts read them: E4M3FN codes[rows][d] and E8M0
 * scales[rows][d/32] (see DG_DTYPE_MXFP4_MXFP8).  norm != 0: first
 * y = bf16(rmsnorm(x)) (eps), written to y, and y is quantized, through the
 * fused RMSNorm kernel; norm == 0: x itself, through the standalone kernel. */
int dg_test_mx8_quantize(const void* x, int32_t rows, int32_t d, int32_t norm, float eps, void* y,
                         uint8_t* codes, uint8_t* scales, void* stream);

/* Commit selection + re-noise alone, on given entropy/argmax [batch][canvas_len]. */
int dg_test_commit(dg_model* m, dg_canvas* c, const float* entropy, const int32_t* argmax,
                   int32_t* n_uncommitted, void* stream);

/* Unit entries: one phase of block `layer` on caller buffers (device, in
 * act_dtype unless stated), through the launches a denoise step makes; the
 * model's workspace holds intermediates.  Row counts up to the workspace
 * (max_batch x max(max_tokens, canvas_len)), else DG_ERR_SHAPE.
 *
 * dg_test_qkv_rope: a [batch*n][d_model] normed rows -> q [batch][H][n][dh]
 * and k, v [batch][H][n][dh], q and k rotary-embedded at positions
 * pos0 .. pos0+n-1 (n <= max_tokens). */
int dg_test_qkv_rope(dg_model* m, int32_t layer, const void* a, int32_t batch, int32_t n, int32_t pos0,
                     void* q, void* k, void* v, void* stream);
/* dg_test_attention: q [kv->batch][H][n][dh] -> out [kv->batch*n][H*dh].
 * With k_canvas/v_canvas ([kv->batch][H][n][dh]): bidirectional over cache
 * rows [0, kv->length) of `layer` and the n canvas rows.  With both NULL:
 * causal over cache rows [0, kv->length + n), query i seeing rows
 * j <= kv->length + i (the new rows must already be in the cache). */
int dg_test_attention(dg_model* m, int32_t layer, const void* q, const dg_kv* kv, const void* k_canvas,
                      const void* v_canvas, int32_t n, void* out, void* stream);
/* dg_test_router: b [T][d_model] normed rows -> fp32 router logits [T][E],
 * top-k ids [T][k] (by logit, ties to the lower id) and weights [T][k] (a
 * softmax over the picked logits). */
int dg_test_router(dg_model* m, int32_t layer, const void* b, int32_t T, float* logits, int32_t* ids,
                   float* weights, void* stream);
/* dg_test_shared: b [T][d_model] -> hs [T][d_shared] (SwiGLU products) and
 * ys [T][d_model] (fp32 shared-expert output). */
int dg_test_shared(dg_model* m, int32_t layer, const void* b, int32_t T, void* hs, float* ys, void* stream);
/* dg_test_moe: b [T][d_model] and top-k ids [T][k] (each in [0, n_experts),
 * distinct within a row; not checked) -> y [T*k][d_model] fp32 expert outputs
 * and, if h is not NULL, h [T*k][d_expert] SwiGLU products, both in pair
 * order (expert-major, token-ascending); pos [T][k] gets the row of pair
 * (t, j). */
int dg_test_moe(dg_model* m, int32_t layer, const void* b, int32_t T, const int32_t* ids, void* h, float* y,
                int32_t* pos, void* stream);
/* dg_test_force_routing: from now on, denoise steps route row t of layer l to
 * the ids ids[l][t][0..k) (device, [n_layers][max_batch*canvas_len][top_k],
 * borrowed) wherever ids[l][t][0] >= 0, weighting them by a softmax over
 * their logits; NULL turns it off.  Lines the routing up with a reference
 * where two router logits nearly tie. */
int dg_test_force_routing(dg_model* m, const int32_t* ids);

#ifdef __cplusplus
}
#endif
#endif /* DG_H */
