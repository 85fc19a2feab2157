// Routed-expert GEMMs of the MoE FFN on gfx950 (zhichai.net 深度拆解, "MoE 效率":
// 128 fine-grained experts, each token routed to 8 of them).  At a 256-token
// canvas an expert sees about 16 tokens per step, so the work is a stream of
// every expert's weights through the MFMA units at 16 FLOP per byte: the
// kernels are written for HBM bandwidth, not for MFMA throughput.
//
// Layout of the work: a few workgroups per expert (gate/up: 2, one per CU at
// 128 experts), each owning a contiguous range of the expert's output rows, so every
// workgroup streams the same number of weight bytes and the grid is balanced
// whatever the routing.  A workgroup first stages the expert's token rows (up
// to 32, all K) in LDS once -- they are the other MFMA operand and are read
// by all of its waves -- then each wave streams its own 16 NB weight rows
// (gate/up: 16 NB gate rows and the matching up rows) from HBM straight into
// MFMA operand registers, MD k-steps ahead.  Staging the tokens once per
// workgroup matters: token loads issued inside the k loop compete with the
// weight stream for the same load path and cut its bandwidth by a third.
// Every weight byte is read once per step (experts with more than 32 pairs
// take one pass per 32).  Weight loads are unconditional -- rows past the end
// are clamped to a valid row and their results are never stored -- so the
// compiler waits for exactly the oldest stage.
//
// MFMA 16x16x32 bf16 with the weights as operand A (16 weight rows) and the
// tokens as operand B (16 tokens): lane l then holds token l % 16 and weight
// rows 4 (l / 16) + 0..3 of the 16x16 result, i.e. four consecutive outputs of
// one token, stored as one 8-byte (bf16) or 16-byte (fp32) write.
//
// gate/up: h[p][j] = bf16(silu(g) * u), g = x_p . W_gate[j], u = x_p . W_up[j]
// down:    y[p][n] = h_p . W_down[n]  (fp32; combined per token later)
// fp8 weights (E4M3FN codes) are widened exactly to bf16 in registers and the
// per-row scale is applied to the fp32 accumulator.
//
// Expert weights are read in a tiled layout made once at load time by
// moe_pack (below): each 16-row x SKE-column block of a matrix is one
// contiguous tile (1 KB for bf16 and for fp8 with 64-column tiles) holding
// exactly one wave's MFMA operand fragment, lane l's bytes at offset
// l * (tile bytes / 64), and the tiles of a 16-row block follow each other
// along k.  A wave's weight load is then one contiguous 1 KB read instead of
// 16 row pieces 4 KB apart, and a wave's stream walks forward through
// memory: pure streaming of the gate/up weights measured 6.1 TB/s this way
// against 5.0 TB/s from the row-major matrices.
#include <cstdint>
#include <type_traits>

#include "dg_common.h"
#include "kernels.h"

namespace dg {
namespace {

constexpr int MTGU = 2;    // 16-token tiles per pass over the gate/up weights (all K staged)
// Weight loads are non-temporal (cache-policy bit nt): every weight byte is
// read once per step, so keeping it in L2 only evicts the token rows and
// outputs; measured at 128 experts x 16 tokens the gate/up stream went from
// 5.9 to 6.6 TB/s and the down stream from 5.2 to 5.5 TB/s.
constexpr int kWeightAux = 2;

struct f8 {
  uint8_t v;
};
struct f4 {  // two E2M1 codes per byte
  uint8_t v;
};

// Weight formats.  A lane loads its slice of a weight tile through a buffer
// resource over one expert's weights: lane offsets are 32-bit, fragment
// offsets are uniform (scalar), and tiles past the expert's end read as
// zero -- a handful of registers however many fragments and stages are in
// flight.  A stage (one tile) is SPS 32-k MFMA steps; lane (c16, g4) holds
// row c16 of the tile and the k range starting at lane_k(g4), and x_k(g4, t)
// gives the k offset, in the stage, of the 8 k-slots it feeds into step t --
// the token operand is read at the same offsets, so any order of k within a
// stage is a valid split of the dot product.
// NIB is the element size in 4-bit units; BSCALE formats carry one E8M0
// scale per 32 weights of a row, applied while the codes are widened (the
// others apply an optional fp32 scale per weight row to the accumulator).
template <typename TW, int SPS_> struct WFmt;
template <> struct WFmt<bf16, 1> {  // 8 bf16 per lane per step
  using raw = u32x4;
  static constexpr int NIB = 4, SPS = 1;
  static constexpr bool BSCALE = false;
  static __device__ __forceinline__ raw load(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kWeightAux);
  }
  static __device__ __forceinline__ int lane_k(int g4) { return 8 * g4; }
  static __device__ __forceinline__ int x_k(int g4, int) { return 8 * g4; }
  static __device__ __forceinline__ u32x4 get(raw v, int, uint32_t) { return v; }
};
template <> struct WFmt<f8, 1> {  // 8 E4M3FN codes per lane per step (K % 64 != 0)
  using raw = u32x2;
  static constexpr int NIB = 2, SPS = 1;
  static constexpr bool BSCALE = false;
  static __device__ __forceinline__ raw load(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kWeightAux);
  }
  static __device__ __forceinline__ int lane_k(int g4) { return 8 * g4; }
  static __device__ __forceinline__ int x_k(int g4, int) { return 8 * g4; }
  static __device__ __forceinline__ u32x4 get(raw c, int, uint32_t) { return e4m3x8_to_bf16x8(c); }
};
template <> struct WFmt<f8, 2> {  // 16 E4M3FN codes per lane: two steps per 16-byte load
  using raw = u32x4;
  static constexpr int NIB = 2, SPS = 2;
  static constexpr bool BSCALE = false;
  static __device__ __forceinline__ raw load(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kWeightAux);
  }
  static __device__ __forceinline__ int lane_k(int g4) { return 16 * g4; }
  static __device__ __forceinline__ int x_k(int g4, int t) { return 16 * g4 + 8 * t; }
  static __device__ __forceinline__ u32x4 get(raw c, int t, uint32_t) {
    return e4m3x8_to_bf16x8(t ? u32x2{c[2], c[3]} : u32x2{c[0], c[1]});
  }
};
// MXFP4: 32 E2M1 codes per lane (16 bytes, four steps; K % 128 == 0) or 16
// (8 bytes, two steps; K % 64 == 0).  A lane's codes are consecutive k of
// one row, inside one 32-weight scale block, so each lane widens with one
// scale.  Step t takes word t: 8 codes, low nibble first.
template <> struct WFmt<f4, 4> {
  using raw = u32x4;
  static constexpr int NIB = 1, SPS = 4;
  static constexpr bool BSCALE = true;
  static __device__ __forceinline__ raw load(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kWeightAux);
  }
  static __device__ __forceinline__ int lane_k(int g4) { return 32 * g4; }
  static __device__ __forceinline__ int x_k(int g4, int t) { return 32 * g4 + 8 * t; }
  static __device__ __forceinline__ u32x4 get(raw c, int t, uint32_t e8) { return e2m1x8_to_bf16x8(c[t], e8); }
};
template <> struct WFmt<f4, 2> {
  using raw = u32x2;
  static constexpr int NIB = 1, SPS = 2;
  static constexpr bool BSCALE = true;
  static __device__ __forceinline__ raw load(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kWeightAux);
  }
  static __device__ __forceinline__ int lane_k(int g4) { return 16 * g4; }
  static __device__ __forceinline__ int x_k(int g4, int t) { return 16 * g4 + 8 * t; }
  static __device__ __forceinline__ u32x4 get(raw c, int t, uint32_t e8) { return e2m1x8_to_bf16x8(c[t], e8); }
};

struct MoeArgs {
  const bf16* X;        // token activations: gate/up [T][K] (rows gathered), down [pairs][K]
  const int* pair_row;  // gate/up: token of each pair slot; down: unused (row = pair)
  const int* off;       // [E+1] pair ranges per expert
  const void* W;        // tiled: gate/up [E][2*Nout][K]; down [E][Nout][K]
  const float* scale;   // fp8: [E][rows of W per expert]
  const uint8_t* bscale;  // mxfp4: E8M0 block scales, tiled like W (see moe_pack_scales)
  int K;                // reduction length (multiple of 32)
  int Nout;             // outputs per token: d_expert (gate/up) or d_model (down)
  void* out;            // gate/up: h bf16 [pairs][Nout]; down: y fp32 [pairs][Nout]
  // gate/up with routing in the kernel (ids != null): the top-k expert ids
  // [T][k]; each expert's workgroups derive its pair range and token list
  // from them, and workgroup 0 of each expert writes off, pair_row and pos
  // (slot of pair (t, j) = off[e] + rank of t among e's tokens) for the
  // kernels after it.
  const int* ids;
  int T, k;
  int* off_out;
  int* pair_row_out;
  int* pos_out;
  // MXFP8 token rows (W_FP4A8 gate/up): codes [rows of X][K], scales [rows of X][K/32]
  const uint8_t* xq;
  const uint8_t* xqs;
};

constexpr int ROUTE_MAX_TOKENS = 2048;
constexpr int ROUTE_MAX_EXPERTS = 256;
// static LDS of the routing lists (tok, slot, flag, hist, red) in the gate/up kernel
constexpr int ROUTE_LDS = ROUTE_MAX_TOKENS * (4 + 1 + 1) + ROUTE_MAX_EXPERTS * 4 + 16;
// static LDS of a routed kernel besides the routing lists (gate/up: the
// largest pair count, one word; 16 bytes are reserved)
constexpr int KERNEL_LDS = 16;

// The routing of one expert e from the top-k ids: pairs of experts below e
// (its pair offset), and its tokens in ascending order with the slot j that
// picked e (each token picks an expert at most once).  Deterministic: the
// order comes from a wave-0 scan over token chunks, not from atomics' order.
struct ExpertRoute {
  int off, cnt;
};
// With hist non-null it also counts the pairs of every expert (hist[0..E)).
__device__ __forceinline__ ExpertRoute route_expert(const MoeArgs& a, int e, int* tok, unsigned char* slot,
                                                    signed char* flag, int* red, int* hist, int E) {
  const int tid = threadIdx.x, nt = blockDim.x;
  if (tid == 0) red[0] = 0;
  if (hist)
    for (int x = tid; x < E; x += nt) hist[x] = 0;
  __syncthreads();
  int less = 0;
  for (int t = tid; t < a.T; t += nt) {
    int m = -1;
    for (int j = 0; j < a.k; ++j) {
      const int id = a.ids[t * a.k + j];
      less += id < e;
      m = id == e ? j : m;
      if (hist) atomicAdd(&hist[id], 1);  // integer counts: order-free
    }
    flag[t] = (signed char)m;
  }
  less = wave_sum_i(less);
  if ((tid & 63) == 0) atomicAdd(&red[0], less);  // integer sum: order-free
  __syncthreads();
  if (tid < 64) {  // wave 0: ordered compaction, 64 tokens per round
    int base = 0;
    for (int t0 = 0; t0 < a.T; t0 += 64) {
      const int t = t0 + tid;
      const int m = t < a.T ? flag[t] : -1;
      const unsigned long long bal = __ballot(m >= 0);
      if (m >= 0) {
        const int r = base + __popcll(bal & ((1ull << tid) - 1ull));
        tok[r] = t;
        slot[r] = (unsigned char)m;
      }
      base += __popcll(bal);
    }
    if (tid == 0) red[1] = base;
  }
  __syncthreads();
  return ExpertRoute{red[0], red[1]};
}

// The expert's token rows of one pass (up to 16 MTP of them, all K) are
// staged once per workgroup in LDS, zero-filled past the last pair; the four
// waves read their operand-B fragments from there, so the only global loads
// in the k loop are the weight stream.
// Pass row r is token row gather[gidx0 + r] of X, or row gidx0 + r when
// gather is null.
template <int MT>
__device__ __forceinline__ void stage_tokens(const MoeArgs& a, bf16* xs, int pitch, const int* gather, int gidx0,
                                             int rows) {
  const int cpr = a.K / 8;  // 16-byte chunks per row
  const int total = 16 * MT * cpr, nt = blockDim.x;
  // batches of 4 loads per thread in flight before their LDS stores
  for (int c0 = threadIdx.x; c0 < total; c0 += 4 * nt) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + u * nt, r = c / cpr, k = (c - r * cpr) * 8;
      v[u] = u32x4{0u, 0u, 0u, 0u};
      if (c < total && r < rows) {
        const long long row = gather ? (long long)gather[gidx0 + r] : (long long)(gidx0 + r);
        v[u] = *(const u32x4*)(a.X + row * a.K + k);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + u * nt, r = c / cpr, k = (c - r * cpr) * 8;
      if (c < total) *(u32x4*)(xs + r * pitch + k) = v[u];
    }
  }
}

// Weight stream of one wave: a buffer resource over expert e's tiles, the
// lane's offsets and a register ring of MD stages.  Slot u of the ring holds
// weight stage k with k % MD == u.  The ring is filled before the workgroup
// stages its tokens, so the first weight tiles are in flight during the
// staging.
template <typename WL, bool GU, int NB, int MD, bool SCALAR_OFFSETS = false>
struct WStream {
  using wraw = typename WL::raw;
  static constexpr bool BS = WL::BSCALE;
  static constexpr int SKE = 32 * WL::SPS;            // k per stage
  static constexpr int TILE = 8 * SKE * WL::NIB;      // bytes of one 16-row tile
  static constexpr int STILE = 16 * SKE / 32;         // bytes of its block scales (BSCALE)
  static constexpr int NW = GU ? 2 * NB : NB;         // fragments per stage: gate blocks, then up blocks
  __amdgpu_buffer_rsrc_t rsrc, srsrc;
  int voff0, svoff0, KS;
  int soff[NW];                           // byte offset of each fragment's first tile
  int ssoff[BS ? NW : 1];                 // and of its first scale tile (BSCALE)
  wraw rw[MD][NW];
  uint32_t rs[BS ? MD : 1][BS ? NW : 1];  // scale codes of the ring's stages

  __device__ __forceinline__ void init(const MoeArgs& a, int e, int n0) {
    const long long wrows = GU ? 2LL * a.Nout : a.Nout;
    const long long mat = wrows * a.K * WL::NIB / 2;  // bytes of one expert's matrix
    rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)a.W + e * mat), (short)0, int(mat), 0x00020000);
    KS = a.K / SKE;
    const int lane = threadIdx.x & 63;
    voff0 = lane * (TILE / 64);
    if constexpr (BS) {
      // lane (row c16, k group g4) reads the scale of its row and of the
      // 32-weight block its codes fall in
      const long long smat = wrows * (a.K / 32);
      srsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(a.bscale + e * smat), (short)0, int(smat), 0x00020000);
      svoff0 = (lane & 15) * (SKE / 32) + (lane >> 4) * SKE / 128;
    }
    // first tile of each fragment's 16-row block (n0 and Nout are multiples
    // of 16).  The offsets are wave-uniform, but the compiler cannot tell
    // (n0 depends on the wave index) and issues each weight load in a loop
    // over the distinct values, which runs once.  SCALAR_OFFSETS moves them
    // to scalar registers (readfirstlane), which removes those loops: the
    // MXFP4 x MXFP8 gate/up then ran 45.0 against 48.3 us, while the bf16
    // and MXFP4 (bf16 widening) streams ran as fast or slower (MXFP4 gate/up
    // and down 49.4 and 34.2 us against 47.0 and 32.5).
#pragma unroll
    for (int f = 0; f < NW; ++f) {
      const int tile0 = ((n0 + 16 * (f % NB) + (f < NB ? 0 : a.Nout)) / 16) * KS;
      soff[f] = SCALAR_OFFSETS ? __builtin_amdgcn_readfirstlane(tile0 * TILE) : tile0 * TILE;
      if constexpr (BS) ssoff[f] = SCALAR_OFFSETS ? __builtin_amdgcn_readfirstlane(tile0 * STILE) : tile0 * STILE;
    }
  }
  __device__ __forceinline__ void ld(int ks, int u) {
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      rw[u][w] = WL::load(rsrc, voff0 + ks * TILE, soff[w]);
      if constexpr (BS)
        rs[u][w] = __builtin_amdgcn_raw_buffer_load_b8(srsrc, svoff0 + ks * STILE, ssoff[w], kWeightAux);
    }
  }
  __device__ __forceinline__ u32x4 get(int u, int w, int t) const {
    if constexpr (BS) return WL::get(rw[u][w], t, rs[u][w]);
    else return WL::get(rw[u][w], t, 0u);
  }
  __device__ __forceinline__ void fill() {
#pragma unroll
    for (int s = 0; s < MD; ++s) ld(min(s, KS - 1), s);
  }
};

// Epilogue of one wave: lane holds token 16 t + c16 of the pass and outputs
// nb + 0..3 of block b; gate/up writes h = bf16(silu(g) * u), down writes y (fp32).
template <typename WL, bool GU, int NB, int MT>
__device__ __forceinline__ void moe_epilogue(const MoeArgs& a, const f32x4 (&acc)[GU ? 2 * NB : NB][MT], int e,
                                             int n0, int pbeg, int rows) {
  const int lane = threadIdx.x & 63, c16 = lane & 15, g4 = lane >> 4;
  const long long wrows = GU ? 2LL * a.Nout : a.Nout;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int nb = n0 + 16 * b + 4 * g4;
    if (nb >= a.Nout) continue;
    float sc[GU ? 2 : 1][4];
#pragma unroll
    for (int h = 0; h < (GU ? 2 : 1); ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = min(nb + r, a.Nout - 1);
        sc[h][r] = a.scale ? a.scale[(long long)e * wrows + (h ? a.Nout : 0) + n] : 1.f;
      }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int r = 16 * t + c16;
      if (r >= rows) continue;
      const long long p = pbeg + r;
      if constexpr (GU) {
        bf16 hv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float gt = acc[b][t][q] * sc[0][q], up = acc[NB + b][t][q] * sc[1][q];
          hv[q] = f32_to_bf16(gt / (1.0f + __expf(-gt)) * up);
        }
        bf16* h = (bf16*)a.out + p * a.Nout + nb;
        if (nb + 3 < a.Nout) {
          *(u32x2*)h = u32x2{uint32_t(hv[0].v) | (uint32_t(hv[1].v) << 16),
                             uint32_t(hv[2].v) | (uint32_t(hv[3].v) << 16)};
        } else {
          for (int q = 0; q < 4 && nb + q < a.Nout; ++q) h[q] = hv[q];
        }
      } else {
        float* y = (float*)a.out + p * a.Nout + nb;
        if (nb + 3 < a.Nout) {
          *(f32x4*)y = f32x4{acc[b][t][0] * sc[0][0], acc[b][t][1] * sc[0][1], acc[b][t][2] * sc[0][2],
                             acc[b][t][3] * sc[0][3]};
        } else {
          for (int q = 0; q < 4 && nb + q < a.Nout; ++q) y[q] = acc[b][t][q] * sc[0][q];
        }
      }
    }
  }
}

// One wave: output rows n0 .. n0 + 16 NB - 1 (for gate/up: those gate rows
// and the matching up rows) of expert e against the MT 16-token tiles staged
// in xs (pass rows pbeg .. pbeg + rows - 1 of the expert's pairs); the weight
// ring of ws has been filled.
template <typename WL, bool GU, int NB, int MD, int MT>
__device__ __forceinline__ void moe_wave(const MoeArgs& a, const bf16* xs, int pitch,
                                         WStream<WL, GU, NB, MD>& ws, int e, int n0, int pbeg, int rows) {
  using WS = WStream<WL, GU, NB, MD>;
  constexpr int SPS = WL::SPS, SKE = WS::SKE, NW = WS::NW;
  const int lane = threadIdx.x & 63, c16 = lane & 15, g4 = lane >> 4;
  const int KS = ws.KS;
  const bf16* xr = xs + c16 * pitch;

  f32x4 acc[NW][MT];
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[w][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The main loop has no conditions and the MFMAs read a slot before its
  // refill is issued into the same registers, so the ring needs no copies
  // and the compiler's wait before a slot is for exactly that slot's loads
  // (the MD - 1 later stages stay in flight); the scheduling barriers keep
  // the loads in stage order.
  auto step = [&](int ks, int u, bool refill, int next) {
#pragma unroll
    for (int t2 = 0; t2 < SPS; ++t2) {
      u32x4 xv[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) xv[t] = *(const u32x4*)(xr + 16 * t * pitch + ks * SKE + WL::x_k(g4, t2));
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const u32x4 wv = ws.get(u, w, t2);
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[w][t] = mfma16x16x32(wv, xv[t], acc[w][t]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (refill) ws.ld(next, u);
    __builtin_amdgcn_sched_barrier(0);
  };
  int k0 = 0;
  for (; k0 + 2 * MD <= KS; k0 += MD) {
#pragma unroll
    for (int u = 0; u < MD; ++u) step(k0 + u, u, true, k0 + u + MD);
  }
  // the last 1 .. 2*MD - 1 stages
#pragma unroll
  for (int u = 0; u < MD; ++u)
    if (k0 + u < KS) step(k0 + u, u, k0 + u + MD < KS, k0 + u + MD);
#pragma unroll
  for (int u = 0; u < MD; ++u)
    if (k0 + MD + u < KS) step(k0 + MD + u, u, false, 0);

  moe_epilogue<WL, GU, NB, MT>(a, acc, e, n0, pbeg, rows);
}

// ---------------------------------------------------------------------------
// MXFP4 weights x MXFP8 tokens on the gfx950 scaled MFMA (16x16x128, E2M1
// operand A, E4M3 operand B, one E8M0 scale per 32 k of each row and column,
// fp32 accumulation).  The MXFP4 weight tiles above are already its A operand
// (lane (c16, g4): row c16, codes k = 32 g4 .. 32 g4 + 31, low nibble first;
// its scale byte is the one of that row and 32-block).  The B operand of lane
// (c16, g4) is token c16's E4M3 codes k = 16 g4 .. 16 g4 + 15 and 64 + 16 g4
// .. 64 + 16 g4 + 15 of the 128-k step (two 16-byte LDS reads), its scale the
// one of token c16 and block g4 (the layout was checked on the device).  The
// token rows arrive quantized (RMSNorm writes them; mx8_quantize for other
// callers): codes [rows][K] and scales [rows][K / 32].

// Stage the pass's token codes [16 MT][K + 16] (an odd multiple of 16 bytes
// per row keeps the 16-row fragment reads conflict-free), then their scales
// [16 MT][K / 32]; rows past the pass are zero.  K % 128 == 0.
template <int MT>
__device__ __forceinline__ void stage_tokens_mx8(const MoeArgs& a, uint8_t* xq, const int* gather, int gidx0,
                                                 int rows) {
  const int cpr = a.K / 16, qp = a.K + 16, nb32 = a.K / 32, spr = a.K / 128;  // 16-byte / 4-byte pieces per row
  uint8_t* sc = xq + 16 * MT * qp;
  const int nt = blockDim.x;
  auto src_row = [&](int r) -> long long {
    return gather ? (long long)gather[gidx0 + r] : (long long)(gidx0 + r);
  };
  const int total = 16 * MT * cpr;
  for (int c0 = threadIdx.x; c0 < total; c0 += 4 * nt) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + u * nt, r = c / cpr, p = c - r * cpr;
      v[u] = u32x4{0u, 0u, 0u, 0u};
      if (c < total && r < rows) v[u] = *(const u32x4*)(a.xq + src_row(r) * a.K + 16 * p);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + u * nt, r = c / cpr, p = c - r * cpr;
      if (c < total) *(u32x4*)(xq + r * qp + 16 * p) = v[u];
    }
  }
  for (int c = threadIdx.x; c < 16 * MT * spr; c += nt) {
    const int r = c / spr, p = c - r * spr;
    const uint32_t v = r < rows ? *(const uint32_t*)(a.xqs + src_row(r) * nb32 + 4 * p) : 0u;
    *(uint32_t*)(sc + r * nb32 + 4 * p) = v;
  }
}

typedef int v8i32 __attribute__((ext_vector_type(8)));

// One wave of the MXFP4 x MXFP8 gate/up: output rows n0 .. n0 + 16 NB - 1
// (and the matching up rows) against the MT token tiles staged by
// stage_tokens_mx8; the weight ring of ws has been filled.
template <bool GU, int NB, int MD, int MT>
__device__ __forceinline__ void moe_wave_mx8(const MoeArgs& a, const uint8_t* xq,
                                             WStream<WFmt<f4, 4>, GU, NB, MD, true>& ws,
                                             int e, int n0, int pbeg, int rows) {
  using WS = WStream<WFmt<f4, 4>, GU, NB, MD, true>;
  constexpr int NW = WS::NW;
  const int lane = threadIdx.x & 63, c16 = lane & 15, g4 = lane >> 4;
  const int KS = ws.KS, qp = a.K + 16, nb32 = a.K / 32;
  const uint8_t* xr = xq + c16 * qp + 16 * g4;
  const uint8_t* sr = xq + 16 * MT * qp + c16 * nb32 + g4;

  f32x4 acc[NW][MT];
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[w][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto step = [&](int ks, int u, bool refill, int next) {
    v8i32 xv[MT];
    int xs8[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const u32x4 lo = *(const u32x4*)(xr + 16 * t * qp + 128 * ks);
      const u32x4 hi = *(const u32x4*)(xr + 16 * t * qp + 128 * ks + 64);
      xv[t] = v8i32{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]), int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
      xs8[t] = sr[16 * t * nb32 + 4 * ks];
    }
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const u32x4 c = ws.rw[u][w];
      const v8i32 wv = v8i32{int(c[0]), int(c[1]), int(c[2]), int(c[3]), 0, 0, 0, 0};
#pragma unroll
      for (int t = 0; t < MT; ++t)
        acc[w][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wv, xv[t], acc[w][t], 4, 0, 0,
                                                                     int(ws.rs[u][w]), 0, xs8[t]);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (refill) ws.ld(next, u);
    __builtin_amdgcn_sched_barrier(0);
  };
  int k0 = 0;
  for (; k0 + 2 * MD <= KS; k0 += MD) {
#pragma unroll
    for (int u = 0; u < MD; ++u) step(k0 + u, u, true, k0 + u + MD);
  }
#pragma unroll
  for (int u = 0; u < MD; ++u)
    if (k0 + u < KS) step(k0 + u, u, k0 + u + MD < KS, k0 + u + MD);
#pragma unroll
  for (int u = 0; u < MD; ++u)
    if (k0 + MD + u < KS) step(k0 + MD + u, u, false, 0);

  moe_epilogue<WFmt<f4, 4>, GU, NB, MT>(a, acc, e, n0, pbeg, rows);
}

// Gate/up with more tokens than fit LDS over all of K (pooled canvases): the
// pass's token rows are staged in chunks of KC columns, double-buffered.  The
// loads of chunk c+1 are issued before chunk c is multiplied and stored after
// it, and one workgroup barrier per chunk hands the buffers over; every
// thread of the workgroup takes part in the staging, the active waves in the
// MFMAs.  One weight stage in flight per wave (the gate/up ring depth).
template <typename WL, int NB, int MT, int KC>
__device__ __forceinline__ void moe_gu_chunked(const MoeArgs& a, bf16* xs, WStream<WL, true, NB, 1>& ws,
                                               bool active, int e, int n0, int pbeg, int rows, const int* gather,
                                               int gidx0) {
  using WS = WStream<WL, true, NB, 1>;
  constexpr int SPS = WL::SPS, SKE = WS::SKE, NW = WS::NW;
  constexpr int CP = KC + 16;  // chunk row pitch: 2 (KC + 16) bytes, an odd multiple of 32
  constexpr int ROWS = 16 * MT, CPR = KC / 8, TOTAL = ROWS * CPR, PB = 4;
  constexpr int KCS = KC / SKE;  // weight stages per chunk
  const int nch = a.K / KC;
  const int lane = threadIdx.x & 63, c16 = lane & 15, g4 = lane >> 4;
  const int tid = threadIdx.x, nt = blockDim.x;
  auto buf = [&](int i) { return xs + (i & 1) * (ROWS * CP); };
  auto xrow = [&](int r) -> const bf16* {
    const long long row = gather ? (long long)gather[gidx0 + r] : (long long)(gidx0 + r);
    return a.X + row * a.K;
  };
  // staging: 16-byte piece q of the chunk is row q / CPR, columns (q % CPR) * 8;
  // rows past the pass are zero
  u32x4 pre[PB];
  auto pre_load = [&](int c) {
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      const int q = tid + u * nt, r = q / CPR, k = (q - r * CPR) * 8;
      pre[u] = u32x4{0u, 0u, 0u, 0u};
      if (q < TOTAL && r < rows) pre[u] = *(const u32x4*)(xrow(r) + c * KC + k);
    }
  };
  auto pre_store = [&](bf16* dst) {
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      const int q = tid + u * nt, r = q / CPR, k = (q - r * CPR) * 8;
      if (q < TOTAL) *(u32x4*)(dst + r * CP + k) = pre[u];
    }
  };
  auto rest = [&](int c, bf16* dst) {  // pieces past PB per thread (small workgroups)
    for (int q = tid + PB * nt; q < TOTAL; q += nt) {
      const int r = q / CPR, k = (q - r * CPR) * 8;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (r < rows) v = *(const u32x4*)(xrow(r) + c * KC + k);
      *(u32x4*)(dst + r * CP + k) = v;
    }
  };

  f32x4 acc[NW][MT];
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[w][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  pre_load(0);
  pre_store(buf(0));
  rest(0, buf(0));
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    if (c + 1 < nch) pre_load(c + 1);
    if (active) {
      const bf16* xr = buf(c) + c16 * CP;
      for (int j = 0; j < KCS; ++j) {
        const int ks = c * KCS + j;
#pragma unroll
        for (int t2 = 0; t2 < SPS; ++t2) {
          u32x4 xv[MT];
#pragma unroll
          for (int t = 0; t < MT; ++t) xv[t] = *(const u32x4*)(xr + 16 * t * CP + j * SKE + WL::x_k(g4, t2));
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            const u32x4 wv = ws.get(0, w, t2);
#pragma unroll
            for (int t = 0; t < MT; ++t) acc[w][t] = mfma16x16x32(wv, xv[t], acc[w][t]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (ks + 1 < ws.KS) ws.ld(ks + 1, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (c + 1 < nch) {
      pre_store(buf(c + 1));
      rest(c + 1, buf(c + 1));
    }
    __syncthreads();
  }
  if (active) moe_epilogue<WL, true, NB, MT>(a, acc, e, n0, pbeg, rows);
}

// grid (split, E), blockDim = 64 * waves, dynamic LDS = 16 MTP rows of
// K + 16 bf16 (KC > 0: two buffers of 16 MTP rows of KC + 16).  Workgroup x
// of expert e owns output rows [x * rows_per_wg, (x + 1) * rows_per_wg); wave
// w of it owns 16 NB of them.  The expert's pairs go in passes of up to
// 16 MTP tokens, each pass staging its tokens in LDS and streaming the wave's
// weights once.
// Gate/up: a workgroup runs the first OWN_PASSES passes of its own expert;
// further passes (an expert holding most of the tokens, as when every open
// position of an absorbing-noise canvas is the same [MASK] token) are spread
// over all workgroups of the grid in a fixed order (pass index, then expert,
// then row range), so they run side by side instead of one after another.
// Each pass is computed by exactly one workgroup with the same arithmetic:
// the results do not depend on which one.
constexpr int OWN_PASSES = 2;
// pairs of expert x: from the in-kernel histogram, else from the offsets
__device__ __forceinline__ int pairs_of(int x, const int* hist, const int* off) {
  return hist ? hist[x] : off[x + 1] - off[x];
}
// Item j of the further passes, ordered by pass index p >= OWN_PASSES, then
// expert, then row range x2 (splits per expert): returns the expert, or -1
// past the last item.  Uniform over the workgroup.
__device__ __forceinline__ int further_pass(int j, int maxc, int PS, int E, int splits, const int* hist,
                                            const int* off, int& p, int& x2) {
  int base = 0;
  for (p = OWN_PASSES; p * PS < maxc; ++p)
    for (int x = 0; x < E; ++x) {
      if (pairs_of(x, hist, off) <= p * PS) continue;
      if (j < base + splits) {
        x2 = j - base;
        return x;
      }
      base += splits;
    }
  return -1;
}
template <typename WL, bool GU, int NB, int MD, int TMAX, int MTP, int KC, bool A8 = false>
__global__ __launch_bounds__(TMAX) void moe_kernel(MoeArgs a, int rows_per_wg) {
  static_assert(KC == 0 || (GU && MD == 1), "chunked staging is the gate/up path with one stage in flight");
  static_assert(!A8 || (std::is_same<WL, WFmt<f4, 4>>::value && KC == 0), "MXFP8 tokens: MXFP4 weights, K % 128 == 0");
  extern __shared__ __attribute__((aligned(16))) bf16 xs[];
  const int pitch = a.K + 16;  // an odd multiple of 32 B when K % 16 == 0: full-rate fragment reads
  constexpr int PS = 16 * MTP;  // pairs per pass
  const int wave = threadIdx.x >> 6;
  // pass rows p0 .. p0 + rows - 1 of expert e; pair p of the expert is X row
  // gather[gbase + p], or X row gbase + p without a gather list (down: X
  // holds one row per pair)
  auto run_pass = [&](WStream<WL, GU, NB, MD, A8>& ws, bool active, int e, int n0, int pbeg, int p0, int rows,
                      const int* gather, int gbase) {
    if constexpr (A8) {
      uint8_t* xq = (uint8_t*)xs;
      if (rows <= 16) stage_tokens_mx8<1>(a, xq, gather, gbase + p0, rows);
      else if (MTP > 2 && rows <= 32) stage_tokens_mx8<2>(a, xq, gather, gbase + p0, rows);
      else stage_tokens_mx8<MTP>(a, xq, gather, gbase + p0, rows);
      __syncthreads();
      if (active) {
        if (rows <= 16) moe_wave_mx8<GU, NB, MD, 1>(a, xq, ws, e, n0, pbeg + p0, rows);
        else if (MTP > 2 && rows <= 32) moe_wave_mx8<GU, NB, MD, 2>(a, xq, ws, e, n0, pbeg + p0, rows);
        else moe_wave_mx8<GU, NB, MD, MTP>(a, xq, ws, e, n0, pbeg + p0, rows);
      }
    } else if constexpr (KC > 0) {
      const int gi = gbase + p0, pb = pbeg + p0;
      if (rows <= 16) moe_gu_chunked<WL, NB, 1, KC>(a, xs, ws, active, e, n0, pb, rows, gather, gi);
      else if (rows <= 32) moe_gu_chunked<WL, NB, 2, KC>(a, xs, ws, active, e, n0, pb, rows, gather, gi);
      else if (MTP > 4 && rows <= 64) moe_gu_chunked<WL, NB, 4, KC>(a, xs, ws, active, e, n0, pb, rows, gather, gi);
      else moe_gu_chunked<WL, NB, MTP, KC>(a, xs, ws, active, e, n0, pb, rows, gather, gi);
    } else {
      if (rows <= 16) stage_tokens<1>(a, xs, pitch, gather, gbase + p0, rows);
      else if (MTP > 2 && rows <= 32) stage_tokens<2>(a, xs, pitch, gather, gbase + p0, rows);
      else stage_tokens<MTP>(a, xs, pitch, gather, gbase + p0, rows);
      __syncthreads();
      if (active) {
        if (rows <= 16) moe_wave<WL, GU, NB, MD, 1>(a, xs, pitch, ws, e, n0, pbeg + p0, rows);
        else if (MTP > 2 && rows <= 32) moe_wave<WL, GU, NB, MD, 2>(a, xs, pitch, ws, e, n0, pbeg + p0, rows);
        else moe_wave<WL, GU, NB, MD, MTP>(a, xs, pitch, ws, e, n0, pbeg + p0, rows);
      }
    }
  };

  const int e = blockIdx.y;
  const int n0 = blockIdx.x * rows_per_wg + wave * 16 * NB;
  const bool active = n0 < min(a.Nout, (blockIdx.x + 1) * rows_per_wg);
  WStream<WL, GU, NB, MD, A8> ws;
  ws.init(a, e, n0);
  if (active) ws.fill();  // the first weight tiles are in flight during the routing and staging

  // wave 0: the most pairs any expert has (read after the next barrier)
  __shared__ int maxc_s;
  auto most_pairs = [&](const int* hist) {
    if (wave == 0) {
      int mx = 0;
      for (int x = threadIdx.x; x < (int)gridDim.y; x += 64) mx = max(mx, pairs_of(x, hist, a.off));
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) mx = max(mx, __shfl_xor(mx, o, 64));
      if (threadIdx.x == 0) maxc_s = mx;
    }
  };

  if constexpr (GU) {
    __shared__ int tok[ROUTE_MAX_TOKENS];
    __shared__ unsigned char slot[ROUTE_MAX_TOKENS];
    __shared__ signed char flag[ROUTE_MAX_TOKENS];
    __shared__ int hist[ROUTE_MAX_EXPERTS];  // pairs per expert (routing in the kernel)
    __shared__ int red[2];
    const int E = gridDim.y;
    int pbeg, pcnt;
    const int* gather;
    int gbase;
    if (a.ids) {
      const ExpertRoute r = route_expert(a, e, tok, slot, flag, red, hist, E);
      pbeg = r.off;
      pcnt = r.cnt;
      gather = tok;
      gbase = 0;
      if (blockIdx.x == 0) {
        for (int i = threadIdx.x; i < pcnt; i += blockDim.x) {
          a.pair_row_out[pbeg + i] = tok[i];
          a.pos_out[tok[i] * a.k + slot[i]] = pbeg + i;
        }
        if (threadIdx.x == 0) {
          a.off_out[e] = pbeg;
          if (e == E - 1) a.off_out[e + 1] = pbeg + pcnt;
        }
      }
    } else {
      pbeg = a.off[e];
      pcnt = a.off[e + 1] - pbeg;
      gather = a.pair_row;
      gbase = pbeg;
    }
    const int* hp = a.ids ? hist : nullptr;
    most_pairs(hp);
    for (int p0 = 0; p0 < min(pcnt, OWN_PASSES * PS); p0 += PS) {
      if (p0) {
        __syncthreads();        // the previous pass is done with xs
        if (active) ws.fill();  // the next pass streams the weights again
      }
      run_pass(ws, active, e, n0, pbeg, p0, min(PS, pcnt - p0), gather, gbase);
    }
    __syncthreads();  // maxc_s is visible; the own passes are done with xs and the lists
    const int maxc = maxc_s;
    if (maxc <= OWN_PASSES * PS) return;  // uniform: no expert has further passes
    const int W = gridDim.x * gridDim.y, wg = blockIdx.y * gridDim.x + blockIdx.x;
    for (int j = wg;; j += W) {
      int p, x2;
      const int e2 = further_pass(j, maxc, PS, E, gridDim.x, hp, a.off, p, x2);
      if (e2 < 0) return;  // uniform: every further pass is taken
      const int n2 = x2 * rows_per_wg + wave * 16 * NB;
      const bool act2 = n2 < min(a.Nout, (x2 + 1) * rows_per_wg);
      ws.init(a, e2, n2);
      if (act2) ws.fill();
      int pb2, gb2;
      const int* g2;
      if (a.ids) {
        pb2 = route_expert(a, e2, tok, slot, flag, red, nullptr, E).off;
        g2 = tok;
        gb2 = 0;
      } else {
        pb2 = a.off[e2];
        g2 = a.pair_row;
        gb2 = pb2;
      }
      run_pass(ws, act2, e2, n2, pb2, p * PS, min(PS, pairs_of(e2, hp, a.off) - p * PS), g2, gb2);
      __syncthreads();  // this pass is done with xs and the lists
    }
  } else {
    // down: each workgroup runs every pass of its own expert (its 2048-odd
    // workgroups already queue behind one another; spreading the further
    // passes over them measured slower)
    const int pbeg = a.off[e], pcnt = a.off[e + 1] - pbeg;
    if (pcnt <= 0) return;  // uniform over the workgroup; nothing was staged
    for (int p0 = 0; p0 < pcnt; p0 += PS) {
      if (p0) {
        __syncthreads();        // the previous pass is done with xs
        if (active) ws.fill();  // the next pass streams the weights again
      }
      run_pass(ws, active, e, n0, pbeg, p0, min(PS, pcnt - p0), nullptr, pbeg);
    }
  }
}

template <typename WL, bool GU, int NB, int MD, int TMAX, int MTP, int KC = 0, bool A8 = false>
int launch_k(const MoeArgs& a, int E, int split, hipStream_t st) {
  if (a.K % (32 * WL::SPS) || (KC > 0 && a.K % KC)) return int(hipErrorInvalidValue);
  const int blocks = (a.Nout + 16 * NB - 1) / (16 * NB);       // 16 NB-row wave blocks per expert
  const int waves = (blocks + split - 1) / split;              // per workgroup
  if (waves * 64 > TMAX) return int(hipErrorInvalidValue);
  const size_t lds = A8 ? size_t(16 * MTP) * (a.K + 16 + a.K / 32)
                   : KC > 0 ? size_t(2 * 16 * MTP) * (KC + 16) * sizeof(bf16)
                            : size_t(16 * MTP) * (a.K + 16) * sizeof(bf16);
  if (lds + (GU ? ROUTE_LDS : 0) + KERNEL_LDS > 160 * 1024) return int(hipErrorInvalidValue);  // + static LDS
  // once per kernel (not inside a graph capture): the largest dynamic LDS any launch may ask for
  static const hipError_t attr = hipFuncSetAttribute((const void*)moe_kernel<WL, GU, NB, MD, TMAX, MTP, KC, A8>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     160 * 1024 - (GU ? ROUTE_LDS : 0) - KERNEL_LDS);
  if (attr != hipSuccess) return int(attr);
  hipLaunchKernelGGL((moe_kernel<WL, GU, NB, MD, TMAX, MTP, KC, A8>), dim3(split, E), dim3(64 * waves), lds, st, a,
                     waves * 16 * NB);
  return int(hipGetLastError());
}

// gate/up: 32 outputs (64 weight rows) per wave, 2 workgroups of up to 12
// waves per expert (704 threads at d_expert 704: the token stage of all K
// takes most of the LDS, so one workgroup per CU), one stage in flight per
// wave; down: 16 outputs per wave, 8 waves per workgroup (K = d_expert is
// short: several workgroups share a CU), 4 stages in flight.  Measured at 128
// experts x 16 tokens: the gate/up stream is fastest with the fewest loads in
// flight (about 11 MB over the chip; 4 stages per wave ran 10-30% slower),
// the short down streams want a deeper ring.  The thread bound sets the register
// budget.
// Many pairs per expert (pooled canvases): up to 96 tokens per pass, so the
// weights are streamed once -- down stages d_expert-wide rows whole, gate/up
// stages d_model-wide rows in chunks.
template <typename WL>
int launch(bool gu, const MoeArgs& a, int E, int pairs, hipStream_t st) {
  if (gu) {
    // many pairs per expert: up to 96 tokens per pass, staged in 256-column
    // chunks; 16 outputs per wave keeps the 96-token accumulators in registers
    if (pairs > 24 * E && a.K % 256 == 0) {
      // MXFP4: 48-token passes.  A 96-token pass spills 170 registers per
      // lane at this thread count (48 tokens: 38): 154 against 178 us per
      // layer at 1024 tokens x 8 slots over 128 experts, although more
      // experts stream their weights twice.  fp8 keeps 96 (168 against 183 us)
      if constexpr (WL::BSCALE) return launch_k<WL, true, 1, 1, 768, 3, 256>(a, E, 4, st);
      return launch_k<WL, true, 1, 1, 768, 6, 256>(a, E, 4, st);
    }
    return launch_k<WL, true, 2, 1, 768, MTGU>(a, E, 2, st);
  }
  // pooled down: 32 outputs per wave (eight waves, 256 outputs per
  // workgroup), so a workgroup's 96 staged token rows (138 KB of LDS, one
  // workgroup per CU) feed twice the weight stream: 86.8 against 100.7 us at
  // 1024 tokens x 8 slots over 128 experts (16 outputs per wave)
  if (pairs > 24 * E && size_t(96) * (a.K + 16) * sizeof(bf16) + KERNEL_LDS <= 160 * 1024)
    return launch_k<WL, false, 2, 4, 512, 6>(a, E, ((a.Nout + 31) / 32 + 7) / 8, st);
  if constexpr (WL::BSCALE) {
    // MXFP4: a quarter of the bf16 bytes per weight row, so a workgroup's
    // token staging (its h rows) weighs as much as its weight stream; 32
    // outputs per wave halve the workgroups per expert (8 of 8 waves) and
    // the staging with them: 32.3 against 36.2 us at 256 tokens x 8 slots
    // (16 outputs per wave, 4 stages in flight; 1024-thread and 64-output
    // variants 33.1-37.5 us)
    const int b32 = (a.Nout + 31) / 32;
    return launch_k<WL, false, 2, 2, 512, 2>(a, E, (b32 + 7) / 8, st);
  }
  const int blocks = (a.Nout + 15) / 16;
  const int split = (blocks + 7) / 8;
  return launch_k<WL, false, 1, 4, 512, 2>(a, E, split, st);
}

// Row-major [n][rows][cols] -> tiled layout (see the top of this file): one
// thread per lane slice of a tile.  Tile k width SKE: 32 for bf16, for fp8 64
// when cols % 64 == 0 (16 codes per lane, two MFMA steps) and else 32.
template <int CH>
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                   long long slices, int rows, int cols, int wb, int ske) {
  const long long c = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= slices) return;
  const int lane = int(c & 63);
  const long long tile = c >> 6;
  const int ks_n = cols / ske;
  const int kt = int(tile % ks_n);
  const long long rb_all = tile / ks_n;  // 16-row block over all matrices
  const long long row = rb_all * 16 + (lane & 15);
  const int col = kt * ske + (lane >> 4) * (ske / 4);
  const uint8_t* s = src + (row * cols + col) * wb;
  if constexpr (CH == 16) {
    *(u32x4*)(dst + c * 16) = *(const u32x4*)s;
  } else {
    *(u32x2*)(dst + c * 8) = *(const u32x2*)s;
  }
}

// Block scales of MXFP4 weights [n][rows][K/32] -> one scale tile per weight
// tile (16 rows x SKE k): 16 x SKE/32 bytes, row-major (row, block), tiles
// in the order of the weight tiles.  One thread per byte.
__global__ __launch_bounds__(256) void pack_scales_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                          long long total, int K, int ske) {
  const long long o = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (o >= total) return;
  const int bpr = ske / 32, stile = 16 * bpr, ks_n = K / ske;
  const long long tile = o / stile;
  const int within = int(o - tile * stile), r = within / bpr, b = within - r * bpr;
  const long long rb_all = tile / ks_n;
  const int kt = int(tile - rb_all * ks_n);
  dst[o] = src[(rb_all * 16 + r) * (K / 32) + kt * bpr + b];
}

// out[8 w .. 8 w + 7] = the 8 E2M1 codes of word w of packed, times the
// scale of their 32-element block, through the conversion the expert
// kernels use (a test of the widening).
__global__ void fp4_decode_kernel(const uint32_t* packed, const uint8_t* scales, int n_words, u32x4* out) {
  const int w = blockIdx.x * blockDim.x + threadIdx.x;
  if (w >= n_words) return;
  out[w] = e2m1x8_to_bf16x8(packed[w], scales[w / 4]);
}

}  // namespace

int moe_pack(WType wt, const void* src, void* dst, long long n_mats, int rows, int cols, hipStream_t st) {
  if (n_mats <= 0 || rows <= 0 || cols <= 0 || rows % 16 || cols % 32) return int(hipErrorInvalidValue);
  int wb, ske;
  if (wt == W_BF16) {
    wb = 2;
    ske = 32;
  } else if (wt == W_FP8) {
    wb = 1;
    ske = cols % 64 == 0 ? 64 : 32;
  } else if (wt == W_FP4) {
    // two codes per byte: tile the packed rows as bytes, 64 bytes (128 k)
    // per tile row when K % 128 == 0, else 32 bytes (64 k)
    if (cols % 64) return int(hipErrorInvalidValue);
    wb = 1;
    ske = cols % 128 == 0 ? 64 : 32;
    cols /= 2;
  } else {
    return int(hipErrorInvalidValue);
  }
  const int ch = ske / 4 * wb;  // bytes per lane slice
  const long long slices = n_mats * rows * (long long)cols * wb / ch;
  const long long blocks = (slices + 255) / 256;
  if (blocks > INT32_MAX) return int(hipErrorInvalidValue);
  if (ch == 16)
    hipLaunchKernelGGL(pack_kernel<16>, dim3((unsigned)blocks), dim3(256), 0, st, (const uint8_t*)src,
                       (uint8_t*)dst, slices, rows, cols, wb, ske);
  else
    hipLaunchKernelGGL(pack_kernel<8>, dim3((unsigned)blocks), dim3(256), 0, st, (const uint8_t*)src,
                       (uint8_t*)dst, slices, rows, cols, wb, ske);
  return int(hipGetLastError());
}

int moe_pack_scales(const void* src, void* dst, long long n_mats, int rows, int K, hipStream_t st) {
  if (n_mats <= 0 || rows <= 0 || K <= 0 || rows % 16 || K % 64) return int(hipErrorInvalidValue);
  const int ske = K % 128 == 0 ? 128 : 64;
  const long long total = n_mats * rows * (long long)(K / 32);
  const long long blocks = (total + 255) / 256;
  if (blocks > INT32_MAX) return int(hipErrorInvalidValue);
  hipLaunchKernelGGL(pack_scales_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (const uint8_t*)src,
                     (uint8_t*)dst, total, K, ske);
  return int(hipGetLastError());
}

int fp4_decode(const void* packed, const uint8_t* scales, int n_blocks, void* out, hipStream_t st) {
  if (n_blocks <= 0) return 0;
  const int n_words = 4 * n_blocks;
  hipLaunchKernelGGL(fp4_decode_kernel, dim3((n_words + 255) / 256), dim3(256), 0, st, (const uint32_t*)packed,
                     scales, n_words, (u32x4*)out);
  return int(hipGetLastError());
}

int moe_experts(WType wt, bool gate_up, const void* X, const int* pair_row, const int* off, int E,
                const void* W, const void* scale, int K, int Nout, void* out, hipStream_t st,
                const MoeRoute* route, int pairs, const uint8_t* xq, const uint8_t* xqs) {
  if (K % 32 || K <= 0 || Nout <= 0 || E <= 0) return int(hipErrorInvalidValue);
  MoeArgs a{};
  a.X = (const bf16*)X;
  a.pair_row = pair_row;
  a.off = off;
  a.W = W;
  if (wt == W_FP4 || wt == W_FP4A8) a.bscale = (const uint8_t*)scale;
  else a.scale = (const float*)scale;
  a.K = K;
  a.Nout = Nout;
  a.out = out;
  if (route) {
    if (!gate_up || route->T > ROUTE_MAX_TOKENS || route->k > 8 || E > ROUTE_MAX_EXPERTS)
      return int(hipErrorInvalidValue);
    pairs = max(pairs, route->T * route->k);
    a.ids = route->ids;
    a.T = route->T;
    a.k = route->k;
    a.off_out = route->off;
    a.pair_row_out = route->pair_row;
    a.pos_out = route->pos;
  }
  if (wt == W_FP4A8) {
    // MXFP4 weights x MXFP8 tokens (gate/up only): 32 outputs per wave, two
    // workgroups per expert and 32 tokens per pass, as for bf16
    if (!gate_up || K % 128 || !a.bscale || !xq || !xqs) return int(hipErrorInvalidValue);
    a.xq = xq;
    a.xqs = xqs;
    a.scale = nullptr;
    return launch_k<WFmt<f4, 4>, true, 2, 1, 768, 2, 0, true>(a, E, 2, st);
  }
  if (wt == W_BF16) return launch<WFmt<bf16, 1>>(gate_up, a, E, pairs, st);
  if (wt == W_FP8 && K % 64 == 0) return launch<WFmt<f8, 2>>(gate_up, a, E, pairs, st);
  if (wt == W_FP8) return launch<WFmt<f8, 1>>(gate_up, a, E, pairs, st);
  if (wt == W_FP4 && !a.bscale) return int(hipErrorInvalidValue);
  if (wt == W_FP4 && K % 128 == 0) return launch<WFmt<f4, 4>>(gate_up, a, E, pairs, st);
  if (wt == W_FP4 && K % 64 == 0) return launch<WFmt<f4, 2>>(gate_up, a, E, pairs, st);
  return int(hipErrorInvalidValue);
}

}  // namespace dg
