// Tiled bf16 GEMM for the dense projections of the denoise step on gfx950
// (QKV, O-projection, router, shared expert, LM head): C = A * B^T with A the
// [M][K] activations and B the [N][K] weights (bf16, or OCP E4M3FN codes with
// one fp32 scale per weight row), fp32 accumulation on MFMA 16x16x32 bf16.
//
// Pipeline: 64-deep k stages; each thread keeps D stages of its share of the
// A and B tiles in flight in registers (global loads of 8 rows x 128 B per
// wave instruction), so the HBM latency is covered by the loads of later
// stages rather than by occupancy; stages pass through a double-buffered LDS
// tile from which the 4 waves read their MFMA fragments.
//
// The LM head at K = 2048 runs on a second kernel (dgemm_kernel, below) that
// moves A and B into LDS with direct global-to-LDS loads instead of a
// register stage, with separate, deeper rings for the weight stream.
//
// Tile order is XCD-aware: workgroup b runs on XCD b % 8, and each XCD gets a
// contiguous run of tiles in which the M tiles of one weight tile are
// neighbours, so the weight tile is fetched from HBM once into that XCD's L2.
//
// Epilogues run from the accumulators.  The LM-head epilogue reduces each row
// of the tile to an online-softmax partial (max, sum e^(z-max),
// sum e^(z-max)(z-max), second max, argmax) so logits never reach HBM; the
// merge kernel folds a row's partials into its entropy and argmax (entropy as
// the confidence of a canvas position: DiffusionGemma解析,
// "换个路数：整片并行去噪的生成机制").
#include <climits>
#include <type_traits>

#include "dg_common.h"
#include "kernels.h"
#include "topk.h"

namespace dg {
namespace {

constexpr int TNT = 256;     // threads per workgroup
constexpr int SK_MIN = 64;   // K must be a multiple of this
// LM-head tile of the register-staged kernel (K != 2048): 128 x 128, four
// waves of 32 rows x 128 columns (one partial per row and tile; four waves
// of 64 x 64 measured 10% slower)
constexpr int LM_BM = 128, LM_BN = 128, LM_WM = 4;
// LM head with K = 2048 (d_model of the full-size workloads): the direct-load
// kernel, 256 x 256 tiles of eight waves (4 x 2, 64 x 128 each, one partial
// per row and 128 columns), A ring 2 and B ring 3 deep (160 KB of LDS).
// Measured at 256 x 262144 x 2048: 344 us against 440 us for the 128 x 128
// register-staged tiles; at M = 1024, 1069 against 1432 us.
constexpr int LMD_BM = 256, LMD_BN = 256, LMD_WM = 4, LMD_NW = 8, LMD_SA = 2, LMD_SB = 3, LMD_KT = 32;
bool lm_direct(int K) { return K == 64 * LMD_KT; }

struct f8 {
  uint8_t v;
};

template <typename TB> struct BChunk;
template <> struct BChunk<bf16> {
  using type = u32x4;  // 8 bf16
  static __device__ __forceinline__ type load(const bf16* p) { return *(const u32x4*)p; }
  static __device__ __forceinline__ u32x4 widen(type v) { return v; }
  static __device__ __forceinline__ type zero() { return u32x4{0u, 0u, 0u, 0u}; }
};
template <> struct BChunk<f8> {
  using type = u32x2;  // 8 codes
  static __device__ __forceinline__ type load(const f8* p) { return *(const u32x2*)p; }
  static __device__ __forceinline__ u32x4 widen(type v) { return e4m3x8_to_bf16x8(v); }
  static __device__ __forceinline__ type zero() { return u32x2{0u, 0u}; }
};

// LM-head epilogue of one wave: acc[i][j] holds rows row0 + 16 i + 4 g4 + r
// and columns col0 + 16 j + c16 of the logits; each row's columns of this
// wave are reduced to one online-softmax partial (max, sum e^(z-max),
// sum e^(z-max)(z-max), second max, argmax), stored at partial index pidx
// of the row's pn partials.
template <int FM, int FN>
__device__ __forceinline__ void lm_partials(const f32x4 (&acc)[FM][FN], const GemmArgs& g, int row0, int col0,
                                            int pn, int pidx) {
  const int lane = threadIdx.x & 63, c16 = lane & 15, g4 = lane >> 4;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      LmPart p = lm_empty_part();
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = col0 + 16 * j + c16;
        if (n < g.N) {
          const float z = acc[i][j][r];
          if (z > p.m) {
            p.sec = p.m;
            p.m = z;
            p.idx = n;
          } else if (z > p.sec) {
            p.sec = z;
          }
        }
      }
      if (p.idx != INT_MAX) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int n = col0 + 16 * j + c16;
          if (n < g.N) {
            const float dz = acc[i][j][r] - p.m;
            const float e = __expf(dz);
            p.s += e;
            p.t += e * dz;
          }
        }
      }
      // a lane with columns but none above -inf: all its logits are NaN or -inf
      if (p.idx == INT_MAX && col0 + c16 < g.N && row0 + 16 * i + 4 * g4 + r < g.M && g.flags)
        atomicOr(g.flags, FLAG_NONFINITE);
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) p = lm_combine(p, lm_shfl_xor(p, o));
      const int m = row0 + 16 * i + 4 * g4 + r;
      if (c16 == 0 && m < g.M) {
        float* o = g.part + ((long long)m * pn + pidx) * 5;
        o[0] = p.m;
        o[1] = p.s;
        o[2] = p.t;
        o[3] = p.sec;
        o[4] = __int_as_float(p.idx);
      }
    }
  }
}

// SwiGLU epilogue of one wave: fragment pair (2q, 2q+1) holds the gate and
// up rows of outputs jbase + 16 q + c16 for rows row0 + 16 i + 4 g4 + r;
// h = bf16(silu(gate) * up) (gate and up scaled by the fp8 row scales, if any).
template <int FM, int FN>
__device__ __forceinline__ void swiglu_store(const f32x4 (&acc)[FM][FN], const GemmArgs& g, int row0, int jbase) {
  const int lane = threadIdx.x & 63, c16 = lane & 15, g4 = lane >> 4;
  const float* Sg = g.b_scale;
#pragma unroll
  for (int q = 0; q < FN / 2; ++q) {
    const int j = jbase + 16 * q + c16;
    if (j >= g.N) continue;
    const float sg = Sg ? Sg[j] : 1.f, su = Sg ? Sg[g.swiglu_half + j] : 1.f;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = row0 + 16 * i + 4 * g4 + r;
        if (m >= g.M) continue;
        const float gt = acc[i][2 * q][r] * sg, up = acc[i][2 * q + 1][r] * su;
        const float h = gt / (1.0f + __expf(-gt)) * up;
        ((bf16*)g.C)[(long long)m * g.ldc + j] = f32_to_bf16(h);
      }
  }
}

// Plain epilogues of one wave (fp32 store, rounded store, rounded residual
// add): fragment j holds columns nbase + 16 j + c16.
template <int EPI, int FM, int FN>
__device__ __forceinline__ void plain_store(const f32x4 (&acc)[FM][FN], const GemmArgs& g, int row0, int nbase) {
  const int lane = threadIdx.x & 63, c16 = lane & 15, g4 = lane >> 4;
  const float* Sg = g.b_scale;
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int n = nbase + 16 * j + c16;
    if (n >= g.N) continue;
    const float sc = Sg ? Sg[n] : 1.f;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = row0 + 16 * i + 4 * g4 + r;
        if (m >= g.M) continue;
        const float v = acc[i][j][r] * sc;
        const long long o = (long long)m * g.ldc + n;
        if constexpr (EPI == EPI_F32) {
          ((float*)g.C)[o] = v;
        } else if constexpr (EPI == EPI_ACT) {
          ((bf16*)g.C)[o] = f32_to_bf16(v);
        } else {
          bf16* C = (bf16*)g.C;
          C[o] = f32_to_bf16(to_f32(C[o]) + v);
        }
      }
  }
}

// BM x BN tile, 4 waves as WAVES_M x (4 / WAVES_M), D stages in flight.
// SWIGLU: the B tile holds gate and up rows interleaved in blocks of 16 (gate
// rows j.., up rows half + j..), so a wave's fragment pair (2q, 2q+1) is the
// gate/up pair of the same 16 outputs and the product is formed in registers.
// KG k-groups: KG x 4 waves per workgroup, group q reducing stages
// [q KT/KG, (q+1) KT/KG) with its own LDS buffers; the groups' accumulators
// are summed through LDS in group order at the end.  More waves per tile
// hide the per-stage LDS and barrier latency that otherwise bounds a tile.
template <typename TB, int BM, int BN, int WAVES_M, int D, int EPI, int SK = 64, int KG = 1>
__global__ __launch_bounds__(TNT * KG) void tgemm_kernel(GemmArgs g, int tiles_m, int tiles_n, int per_xcd) {
  // LDS row pitch SK + 16 elements: fragment reads (16 rows x 64 B per
  // ds_read_b128) run at full LDS rate on gfx950 when the row pitch is an odd
  // multiple of 32 B, at half rate for other multiples of 16 B (measured).
  constexpr int LDK = SK + 16;
  constexpr int WAVES_N = 4 / WAVES_M;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int CPR = SK / 8;  // 8-element chunks per row per stage
  constexpr int A_PT = BM * CPR / TNT, B_PT = BN * CPR / TNT;
  static_assert(BM * CPR % TNT == 0 && BN * CPR % TNT == 0, "tile rows must be multiples of 32");
  static_assert(FM >= 1 && FN >= 1, "wave tile");
  static_assert(EPI != EPI_SWIGLU || FN % 2 == 0, "SWIGLU needs gate/up fragment pairs");

  using BC = BChunk<TB>;
  using bchunk = typename BC::type;

  __shared__ __attribute__((aligned(16))) bf16 lds_all[KG][2][(BM + BN) * LDK];
  static_assert(KG == 1 || (size_t)(KG - 1) * BM * BN * 4 <= sizeof(lds_all), "reduction space");

  // XCD-aware tile index; the exit is uniform over the workgroup.
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int tile = xcd * per_xcd + slot;
  if (slot >= per_xcd || tile >= tiles_m * tiles_n) return;
  const int tn = tile / tiles_m, tm = tile - tn * tiles_m;

  const int lane = threadIdx.x & 63, grp = threadIdx.x / TNT;
  const int tid = threadIdx.x % TNT, wave = tid >> 6;
  const int c16 = lane & 15, g4 = lane >> 4;
  const int wr = (wave / WAVES_N) * WM, wc = (wave % WAVES_N) * WN;
  const int m0 = tm * BM;
  const int KT = g.K / SK / KG;           // stages per group
  const int kbase = grp * KT * SK;        // this group's first k
  bf16 (*As)[(BM + BN) * LDK] = lds_all[grp];
  const int boff = BM * LDK;              // B tile follows the A tile in each buffer

  const bf16* Ag = (const bf16*)g.A;
  const TB* Bg = (const TB*)g.B;

  // this thread's load slots: chunk c -> row c / CPR, k offset (c % CPR) * 8
  const bf16* ap[A_PT];
#pragma unroll
  for (int u = 0; u < A_PT; ++u) {
    const int c = tid + u * TNT, r = c / CPR, kc = (c % CPR) * 8;
    const int m = m0 + r;
    ap[u] = Ag + (long long)(m < g.M ? m : 0) * g.lda + kbase + kc;
  }
  const TB* bp[B_PT];
#pragma unroll
  for (int u = 0; u < B_PT; ++u) {
    const int c = tid + u * TNT, r = c / CPR, kc = (c % CPR) * 8;
    long long brow;
    bool ok;
    if constexpr (EPI == EPI_SWIGLU) {
      const int blk = r >> 4, j = tn * (BN / 2) + (blk >> 1) * 16 + (r & 15);
      ok = j < g.N;
      brow = (blk & 1) ? (long long)g.swiglu_half + j : j;
    } else {
      const int n = tn * BN + r;
      ok = n < g.N;
      brow = n;
    }
    bp[u] = Bg + (ok ? brow : 0) * g.ldb + kbase + kc;
  }

  // Loads are unconditional (rows past M or N read row 0 and only feed
  // accumulator rows/columns the epilogue never stores), so the compiler can
  // wait for exactly the oldest stage instead of draining every load in flight.
  u32x4 ra[D][A_PT];
  bchunk rb[D][B_PT];
  auto gload = [&](int kt, u32x4* ra_, bchunk* rb_) {
#pragma unroll
    for (int u = 0; u < A_PT; ++u) ra_[u] = *(const u32x4*)(ap[u] + kt * SK);
#pragma unroll
    for (int u = 0; u < B_PT; ++u) rb_[u] = BC::load(bp[u] + kt * SK);
  };
  auto lstore = [&](int buf, const u32x4* ra_, const bchunk* rb_) {
#pragma unroll
    for (int u = 0; u < A_PT; ++u) {
      const int c = tid + u * TNT;
      *(u32x4*)&As[buf][(c / CPR) * LDK + (c % CPR) * 8] = ra_[u];
    }
#pragma unroll
    for (int u = 0; u < B_PT; ++u) {
      const int c = tid + u * TNT;
      *(u32x4*)&As[buf][boff + (c / CPR) * LDK + (c % CPR) * 8] = BC::widen(rb_[u]);
    }
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < D; ++s) gload(min(s, KT - 1), ra[s], rb[s]);
  lstore(0, ra[0], rb[0]);
  __syncthreads();

  // One stage: ring slot u held stage kt (already in LDS) and is refilled
  // with stage kt + D (past the end: the last stage again, an L2 hit); the
  // MFMAs read LDS buffer kt & 1 while slot u + 1 (stage kt + 1) goes to the
  // other buffer.
  auto stage = [&](int kt, int u, bool store_next) {
    gload(min(kt + D, KT - 1), ra[u], rb[u]);
    const int buf = kt & 1;
#pragma unroll
    for (int s = 0; s < SK / 32; ++s) {
      u32x4 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *(const u32x4*)&As[buf][(wr + 16 * i + c16) * LDK + 32 * s + 8 * g4];
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = *(const u32x4*)&As[buf][boff + (wc + 16 * j + c16) * LDK + 32 * s + 8 * g4];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma16x16x32(af[i], bfr[j], acc[i][j]);
    }
    if (store_next) lstore(buf ^ 1, ra[(u + 1) % D], rb[(u + 1) % D]);
    __syncthreads();
  };
  // The main loop body has no branches, so the compiler's wait before each
  // LDS store is for exactly the oldest ring slot (a branch inside the loop
  // makes it drain every load in flight at the loop head); the last 1..D
  // stages run after it.
  int kt0 = 0;
  for (; kt0 + D < KT; kt0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) stage(kt0 + u, u, true);
  }
#pragma unroll
  for (int u = 0; u < D; ++u)
    if (kt0 + u < KT) stage(kt0 + u, u, kt0 + u + 1 < KT);

  if constexpr (KG > 1) {
    // groups 1.. hand their accumulators to group 0, which adds them in group order
    float* red = (float*)&lds_all[0][0][0];
    constexpr int PER = FM * FN * 4;  // floats per lane
    if (grp > 0) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            red[(((grp - 1) * 4 + wave) * PER + (i * FN + j) * 4 + r) * 64 + lane] = acc[i][j][r];
    }
    __syncthreads();
    if (grp > 0) return;
#pragma unroll
    for (int q = 1; q < KG; ++q)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[i][j][r] += red[(((q - 1) * 4 + wave) * PER + (i * FN + j) * 4 + r) * 64 + lane];
  }

  // ---------------------------------------------------------------- epilogues
  if constexpr (EPI == EPI_LM) {
    // one partial per (row, wave column block): WAVES_N per tile
    lm_partials<FM, FN>(acc, g, m0 + wr, tn * BN + wc, tiles_n * WAVES_N, tn * WAVES_N + (wave % WAVES_N));
  } else if constexpr (EPI == EPI_QKV) {
    // tile tn is one head of q, k or v (BN = head_dim = 128) and each wave
    // holds whole tile rows, so lane column d = 16 jf + c16 (jf < 4) and its
    // rotate-half partner d + 64 (fragment jf + 4) sit in the same lane:
    // round q/k/v to bf16, rotate q and k in fp32 with the position's
    // (cos, sin), round again, and store into the per-head layouts
    static_assert(BN == 128 && WAVES_N == 1, "QKV epilogue: one head per tile, whole rows per wave");
    const int H = g.heads, which = tn / H, h = tn - which * H;
    const float2* tab = (const float2*)g.rope_tab;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wr + 16 * i + 4 * g4 + r;
        if (m >= g.M) continue;
        const int b = m / g.seq_n, ti = m - b * g.seq_n;
        bf16* dst = which == 0 ? (bf16*)g.q_out + ((long long)(b * H + h) * g.seq_n + ti) * 128
                               : (bf16*)(which == 1 ? g.k_dst : g.v_dst) + (long long)(b * H + h) * g.dst_bh +
                                     (long long)(g.row0 + ti) * 128;
        if (which == 2) {
#pragma unroll
          for (int jf = 0; jf < 8; ++jf) dst[16 * jf + c16] = f32_to_bf16(acc[i][jf][r]);
        } else {
#pragma unroll
          for (int jf = 0; jf < 4; ++jf) {
            const int d = 16 * jf + c16;
            const float x1 = to_f32(f32_to_bf16(acc[i][jf][r])), x2 = to_f32(f32_to_bf16(acc[i][jf + 4][r]));
            const float2 cs = tab[ti * 64 + d];
            dst[d] = f32_to_bf16(x1 * cs.x - x2 * cs.y);
            dst[d + 64] = f32_to_bf16(x2 * cs.x + x1 * cs.y);
          }
        }
      }
  } else if constexpr (EPI == EPI_SWIGLU) {
    swiglu_store<FM, FN>(acc, g, m0 + wr, tn * (BN / 2) + (wc / 2));
  } else {
    plain_store<EPI, FM, FN>(acc, g, m0 + wr, tn * BN + wc);
  }
}

template <typename TB, int BM, int BN, int WAVES_M, int D, int EPI, int SK = 64, int KG = 1>
int launch_t(const GemmArgs& g, hipStream_t st) {
  if (g.K % (SK * KG)) return int(hipErrorInvalidValue);
  const int bn_out = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + bn_out - 1) / bn_out;
  const int total = tiles_m * tiles_n;
  if (total == 0) return 0;
  const int per_xcd = (total + 7) / 8;
  hipLaunchKernelGGL((tgemm_kernel<TB, BM, BN, WAVES_M, D, EPI, SK, KG>), dim3(8 * per_xcd), dim3(TNT * KG), 0,
                     st, g, tiles_m, tiles_n, per_xcd);
  return int(hipGetLastError());
}

// ---------------------------------------------------------------- direct-load GEMM
// bf16 A [M][K] and B [N][K] through LDS without a register stage: each
// global_load_lds_dwordx4 of a wave moves 8 rows x 128 bytes (64 k) of A or
// B -- eight whole cache lines -- into one 1 KB LDS block, lane L's 16 bytes
// landing at byte 16 L of the block.  Lane L loads row L / 8 and 16-byte
// chunk (L % 8) ^ (L / 8) of it, so chunk c of row r sits in slot 8 r + (c ^ r):
// the eight rows of a fragment read hit eight different bank groups.
// A and B stages (64 k each) have rings of their own, SA and SB buffers deep:
// the loads of stage kt + SA - 1 (A) and kt + SB - 1 (B) are issued right
// after the barrier that opens stage kt, so the weight stream (B, from HBM)
// can run further ahead than the activations (A, L2-resident) in the same
// LDS, and no registers hold data in transit.  The wait before that barrier
// counts this thread's loads still allowed in flight (s_waitcnt vmcnt; loads
// complete in issue order); the barrier makes every thread's loads of stage
// kt visible and frees the buffers of stage kt - 1.
namespace dl {

typedef __attribute__((address_space(3))) void* lds_ptr;

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>)
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

// wait until at most N of this thread's vector-memory operations (and no LDS
// operation) are outstanding, then the workgroup barrier.  The wait is the
// s_waitcnt builtin, which the compiler's own wait tracking takes into
// account (so it adds no full wait before reading a stage it knows has
// landed); the empty asm statements keep memory accesses on their side.
template <int N>
__device__ __forceinline__ void wait_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Issue order of the loads: the prologue issues A stages 0 .. SA - 2 and B
// stages 0 .. SB - 2 (step s: A(s), then B(s)); iteration j issues
// A(j + SA - 1), then B(j + SB - 1) (stages past KT - 1 are skipped).  The
// number of loads issued after both A(kt) and B(kt) and before iteration kt:
// what may still be in flight when stage kt is consumed.
template <int SA, int SB, int KT, int LA, int LB>
constexpr int loads_after(int kt) {
  constexpr int SMAX = SA > SB ? SA : SB;
  int seq[2 * SMAX + 2 * KT][2] = {};  // issue order: (0 = A / 1 = B, stage)
  int n = 0;
  for (int st = 0; st < SMAX - 1; ++st) {
    if (st <= SA - 2 && st < KT) { seq[n][0] = 0; seq[n][1] = st; ++n; }
    if (st <= SB - 2 && st < KT) { seq[n][0] = 1; seq[n][1] = st; ++n; }
  }
  for (int j = 0; j < kt; ++j) {
    if (j + SA - 1 < KT) { seq[n][0] = 0; seq[n][1] = j + SA - 1; ++n; }
    if (j + SB - 1 < KT) { seq[n][0] = 1; seq[n][1] = j + SB - 1; ++n; }
  }
  int last = -1;
  for (int i = 0; i < n; ++i)
    if (seq[i][1] == kt) last = i;
  int cnt = 0;
  for (int i = last + 1; i < n; ++i) cnt += seq[i][0] == 0 ? LA : LB;
  return cnt;
}

}  // namespace dl

// Weight row (row of B) that feeds tile row r of tile column tn, and whether
// it exists.  SWIGLU: blocks of 16 rows alternate gate rows j.. and up rows
// swiglu_half + j.., so a wave's fragment pair (2q, 2q+1) is the gate/up pair
// of 16 outputs.  QKV: within each 128-row head, tile rows are ordered so
// that fragment 2P holds head dims 16 P .. 16 P + 15 and fragment 2P + 1 their
// rotate-half partners 64 + 16 P ..; a 32-column wave block then holds whole
// rotation pairs.
template <int EPI, int BN>
__device__ __forceinline__ long long dl_brow(const GemmArgs& g, int tn, int r, bool& ok) {
  if constexpr (EPI == EPI_SWIGLU) {
    const int blk = r >> 4, j = tn * (BN / 2) + (blk >> 1) * 16 + (r & 15);
    ok = j < g.N;
    return (blk & 1) ? (long long)g.swiglu_half + j : j;
  } else if constexpr (EPI == EPI_QKV) {
    const int n = tn * BN + r, f = (n & 127) >> 4;
    ok = n < g.N;
    return (n & ~127) + (f & 1) * 64 + (f >> 1) * 16 + (n & 15);
  } else {
    const int n = tn * BN + r;
    ok = n < g.N;
    return n;
  }
}

// NWV waves as WAVES_M x (NWV / WAVES_M); each wave owns a (BM / WAVES_M) x
// (BN / WAVES_N) block of the tile.  An A stage buffer holds BM / 8 blocks, a
// B stage buffer BN / 8, block q holding rows 8 q .. 8 q + 7 of the tile.
// TK: the launch also holds router top-k workgroups (one token per wave),
// after the tiles in each XCD's run of workgroups: slot s >= per_xcd of XCD x
// is top-k workgroup x * tk_per_xcd + s - per_xcd.
template <int BM, int BN, int WAVES_M, int NWV, int SA, int SB, int EPI, int KT, bool TK = false>
__global__ __launch_bounds__(64 * NWV) void dgemm_kernel(GemmArgs g, int tiles_m, int tiles_n, int tiles_n2,
                                                         int per_xcd, int tk_per_xcd = 0) {
  constexpr int WAVES_N = NWV / WAVES_M;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int LA = BM / 8 / NWV, LB = BN / 8 / NWV;  // loads per wave per stage
  static_assert(LA * 8 * NWV == BM && LB * 8 * NWV == BN && FM >= 1 && FN >= 1, "tile shape");
  static_assert(SA >= 2 && SA <= 8 && SB >= 2 && SB <= 8, "stages");
  static_assert(EPI != EPI_SWIGLU || FN % 2 == 0, "SWIGLU needs gate/up fragment pairs");
  static_assert(EPI != EPI_QKV || (FN % 2 == 0 && BN % 128 == 0), "QKV needs whole rotation pairs and heads");

  // one array per stage buffer, so each LDS access names its buffer statically
#define DG_DL_BUF(X, R, ROWS, I) __shared__ __attribute__((aligned(1024))) bf16 X##I[R > I ? ROWS * 64 : 1];
  DG_DL_BUF(A, SA, BM, 0) DG_DL_BUF(A, SA, BM, 1) DG_DL_BUF(A, SA, BM, 2) DG_DL_BUF(A, SA, BM, 3)
  DG_DL_BUF(A, SA, BM, 4) DG_DL_BUF(A, SA, BM, 5) DG_DL_BUF(A, SA, BM, 6) DG_DL_BUF(A, SA, BM, 7)
  DG_DL_BUF(B, SB, BN, 0) DG_DL_BUF(B, SB, BN, 1) DG_DL_BUF(B, SB, BN, 2) DG_DL_BUF(B, SB, BN, 3)
  DG_DL_BUF(B, SB, BN, 4) DG_DL_BUF(B, SB, BN, 5) DG_DL_BUF(B, SB, BN, 6) DG_DL_BUF(B, SB, BN, 7)
#undef DG_DL_BUF
  auto abuf = [&](auto bc) -> bf16* {
    constexpr int b = decltype(bc)::value % SA;
    if constexpr (b == 0) return A0;
    else if constexpr (b == 1) return A1;
    else if constexpr (b == 2) return A2;
    else if constexpr (b == 3) return A3;
    else if constexpr (b == 4) return A4;
    else if constexpr (b == 5) return A5;
    else if constexpr (b == 6) return A6;
    else return A7;
  };
  auto bbuf = [&](auto bc) -> bf16* {
    constexpr int b = decltype(bc)::value % SB;
    if constexpr (b == 0) return B0;
    else if constexpr (b == 1) return B1;
    else if constexpr (b == 2) return B2;
    else if constexpr (b == 3) return B3;
    else if constexpr (b == 4) return B4;
    else if constexpr (b == 5) return B5;
    else if constexpr (b == 6) return B6;
    else return B7;
  };

  // tiles of the second product (B2, fp32 out; compiled into the SwiGLU
  // kernels only) come first, then the main ones
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  if constexpr (TK) {
    if (slot >= per_xcd) {  // uniform: a top-k workgroup
      __shared__ __attribute__((aligned(16))) unsigned long long tk_keys[NWV][128];
      __shared__ float tk_sel[NWV][8];
      const int w = threadIdx.x >> 6;
      const int t = (xcd * tk_per_xcd + slot - per_xcd) * NWV + w;
      topk_row<2>(g.tk_logits, t, t < g.tk_T, g.tk_E, g.tk_k, g.tk_ids, g.tk_w, tk_keys[w], tk_sel[w]);
      return;
    }
  }
  const int tile0 = xcd * per_xcd + slot, aux_tiles = EPI == EPI_SWIGLU ? tiles_m * tiles_n2 : 0;
  if (slot >= per_xcd || tile0 >= aux_tiles + tiles_m * tiles_n) return;  // uniform over the workgroup
  const bool aux = EPI == EPI_SWIGLU && tile0 < aux_tiles;
  const int tile = aux ? tile0 : tile0 - aux_tiles;
  const int tn = tile / tiles_m, tm = tile - tn * tiles_m;
  // the wave index is uniform: keep it (and the LDS block offsets) scalar
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15, g4 = lane >> 4;
  const int wr = (wave / WAVES_N) * WM, wc = (wave % WAVES_N) * WN;
  const int m0 = tm * BM;

  // this lane's sources of its loads of a stage (A block wave + NWV i, B
  // block wave + NWV i): row lane / 8 of the block, chunk (lane % 8) ^ (lane / 8);
  // rows past M or N read row 0 and only feed outputs that are never stored
  const int rr8 = lane >> 3, ch = (lane & 7) ^ rr8;
  const bf16* asrc[LA];
  const bf16* bsrc[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int r = m0 + 8 * (wave + NWV * i) + rr8;
    asrc[i] = (const bf16*)g.A + (long long)(r < g.M ? r : 0) * g.lda + 8 * ch;
  }
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int r8 = 8 * (wave + NWV * i) + rr8;
    if (aux) {
      const int n = tn * BN + r8;
      bsrc[i] = (const bf16*)g.B2 + (long long)(n < g.N2 ? n : 0) * g.ldb2 + 8 * ch;
    } else {
      bool ok;
      const long long r = dl_brow<EPI, BN>(g, tn, r8, ok);
      bsrc[i] = (const bf16*)g.B + (ok ? r : 0) * g.ldb + 8 * ch;
    }
  }
  auto issue_a = [&](int kt, bf16* b) {
#pragma unroll
    for (int i = 0; i < LA; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(asrc[i] + kt * 64), (dl::lds_ptr)(b + (wave + NWV * i) * 512),
                                       16, 0, 0);
  };
  auto issue_b = [&](int kt, bf16* b) {
#pragma unroll
    for (int i = 0; i < LB; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(bsrc[i] + kt * 64), (dl::lds_ptr)(b + (wave + NWV * i) * 512),
                                       16, 0, 0);
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fragment of 16 rows starting at buffer row r0 (a multiple of 16), k-half
  // ks: lane row r0 + c16 is row c16 % 8 of block (r0 + c16) / 8, chunk 4 ks + g4
  const int rr = lane & 7;
  auto frag_off = [&](int r0, int ks) { return ((r0 >> 3) + (c16 >> 3)) * 512 + (rr * 8 + ((4 * ks + g4) ^ rr)) * 8; };
  // the fragments of both k-halves of a stage (or, for wide wave tiles, of
  // one k-half) are read before their first MFMA: the LDS latency is paid
  // once per group, and the other waves' MFMAs cover it
  constexpr int KH = (FM + FN) <= 8 ? 2 : 1;  // k-halves per fragment group
  auto compute = [&](const bf16* ab, const bf16* bb) {
#pragma unroll
    for (int k0 = 0; k0 < 2; k0 += KH) {
      u32x4 af[KH][FM], bfr[KH][FN];
#pragma unroll
      for (int h = 0; h < KH; ++h) {
#pragma unroll
        for (int i = 0; i < FM; ++i) af[h][i] = *(const u32x4*)(ab + frag_off(wr + 16 * i, k0 + h));
#pragma unroll
        for (int j = 0; j < FN; ++j) bfr[h][j] = *(const u32x4*)(bb + frag_off(wc + 16 * j, k0 + h));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int h = 0; h < KH; ++h)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = mfma16x16x32(af[h][i], bfr[h][j], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // K = 64 KT is a compile-time constant and the stage loop is unrolled
  // completely: every buffer is named statically and the loop has no header
  // at which the compiler's wait tracking of the LDS loads in flight would
  // merge into a full wait
  constexpr int SMAX = SA > SB ? SA : SB;
  dl::static_for<SMAX - 1>([&](auto sc) {
    constexpr int st = decltype(sc)::value;
    if constexpr (st <= SA - 2 && st < KT) issue_a(st, abuf(sc));
    if constexpr (st <= SB - 2 && st < KT) issue_b(st, bbuf(sc));
  });
  dl::static_for<KT>([&](auto kc) {
    constexpr int kt = decltype(kc)::value;
    dl::wait_barrier<dl::loads_after<SA, SB, KT, LA, LB>(kt)>();
    if constexpr (kt + SA - 1 < KT) issue_a(kt + SA - 1, abuf(std::integral_constant<int, kt + SA - 1>{}));
    if constexpr (kt + SB - 1 < KT) issue_b(kt + SB - 1, bbuf(std::integral_constant<int, kt + SB - 1>{}));
    compute(abuf(kc), bbuf(kc));
  });

  if (aux) {
    GemmArgs g2 = g;
    g2.N = g.N2;
    g2.C = g.C2;
    g2.ldc = g.ldc2;
    g2.b_scale = nullptr;
    plain_store<EPI_F32, FM, FN>(acc, g2, m0 + wr, tn * BN + wc);
  } else if constexpr (EPI == EPI_LM) {
    lm_partials<FM, FN>(acc, g, m0 + wr, tn * BN + wc, tiles_n * WAVES_N, tn * WAVES_N + (wave % WAVES_N));
  } else if constexpr (EPI == EPI_SWIGLU) {
    swiglu_store<FM, FN>(acc, g, m0 + wr, tn * (BN / 2) + (wc / 2));
  } else if constexpr (EPI == EPI_QKV) {
    // fragment pair (2q, 2q+1) of the wave: head dims d and d + 64 of one head
    // of q, k or v (see dl_brow); round to bf16, rotate q and k in fp32 with
    // the position's (cos, sin), round again, store into the per-head layouts
    const int H = g.heads;
    const float2* tab = (const float2*)g.rope_tab;
#pragma unroll
    for (int q = 0; q < FN / 2; ++q) {
      const int n = tn * BN + wc + 32 * q;  // first (permuted) column of the pair
      if (n >= g.N) continue;
      const int hg = n >> 7, which = hg / H, h = hg - which * H;
      const int d = ((n & 127) >> 5) * 16 + c16;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + wr + 16 * i + 4 * g4 + r;
          if (m >= g.M) continue;
          const int b = m / g.seq_n, ti = m - b * g.seq_n;
          bf16* dst = which == 0 ? (bf16*)g.q_out + ((long long)(b * H + h) * g.seq_n + ti) * 128
                                 : (bf16*)(which == 1 ? g.k_dst : g.v_dst) + (long long)(b * H + h) * g.dst_bh +
                                       (long long)(g.row0 + ti) * 128;
          if (which == 2) {
            dst[d] = f32_to_bf16(acc[i][2 * q][r]);
            dst[d + 64] = f32_to_bf16(acc[i][2 * q + 1][r]);
          } else {
            const float x1 = to_f32(f32_to_bf16(acc[i][2 * q][r])), x2 = to_f32(f32_to_bf16(acc[i][2 * q + 1][r]));
            const float2 cs = tab[ti * 64 + d];
            dst[d] = f32_to_bf16(x1 * cs.x - x2 * cs.y);
            dst[d + 64] = f32_to_bf16(x2 * cs.x + x1 * cs.y);
          }
        }
    }
  } else {
    plain_store<EPI, FM, FN>(acc, g, m0 + wr, tn * BN + wc);
  }
}

template <int BM, int BN, int WAVES_M, int NWV, int SA, int SB, int EPI, int KT = 32>
int launch_dl(const GemmArgs& g, hipStream_t st) {
  if (g.K != 64 * KT || g.lda % 8 || g.ldb % 8) return int(hipErrorInvalidValue);
  if (g.B2 && (EPI != EPI_SWIGLU || g.ldb2 % 8 || !g.C2 || g.N2 <= 0)) return int(hipErrorInvalidValue);
  const int bn_out = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + bn_out - 1) / bn_out;
  const int tiles_n2 = g.B2 ? (g.N2 + BN - 1) / BN : 0;
  const int total = tiles_m * (tiles_n + tiles_n2);
  if (total == 0) return 0;
  const int per_xcd = (total + 7) / 8;
  hipLaunchKernelGGL((dgemm_kernel<BM, BN, WAVES_M, NWV, SA, SB, EPI, KT>), dim3(8 * per_xcd), dim3(64 * NWV), 0, st,
                     g, tiles_m, tiles_n, tiles_n2, per_xcd);
  return int(hipGetLastError());
}

// Tile shape per epilogue and size (measured at M = 256, K = 2048): the
// dense projections run on 64x64 or 64x32 tiles with two k-groups of 4 waves
// (enough workgroups to cover 256 CUs while weight tiles are shared through
// L2); the LM head on 128x128 tiles with each wave owning whole tile rows,
// which keeps a wave at two per SIMD.  k-groups need K % (64 KG) == 0.
template <typename TB, int BM, int BN, int WM, int D, int EPI>
int launch_kg(const GemmArgs& g, hipStream_t st, int kg_max) {
  if (kg_max >= 4 && g.K % 256 == 0) return launch_t<TB, BM, BN, WM, D, EPI, 64, 4>(g, st);
  if (kg_max >= 2 && g.K % 128 == 0) return launch_t<TB, BM, BN, WM, D, EPI, 64, 2>(g, st);
  return launch_t<TB, BM, BN, WM, D, EPI, 64, 1>(g, st);
}

// Dense projections with K = 2048 (d_model of the full-size workloads) on the
// direct-load kernel, tile shapes and ring depths per epilogue and M from
// measurements with cold weights: at M = 256 the QKV projection (N = 6144)
// took 19.3 us against 26.6 us and the shared gate/up (4096 weight rows)
// 14.5 against 17.7 us; at M = 1024 the QKV 38.7 against 67.7, the shared
// gate/up 25.8 against 44.3 and the N = 2048 projections 19.0 against 24.2.
// The small-M tiles (64 rows) run up to 512 rows: one 512-position canvas or
// two canvases of 256 took 11.76 / 11.13 ms per step against 12.40 / 11.77
// with the large-M tiles (the 128x256 QKV tiles give only 96 workgroups
// there); at 768 rows the large tiles win (13.22 against 13.40 ms).
// Returns -1 when the shape is not covered.
constexpr int SMALL_M = 512;
int dense_direct(GemmEpi epi, const GemmArgs& g, hipStream_t st) {
  if (g.K != 2048 || g.lda % 8 || g.ldb % 8 || g.N < 1024) return -1;
  const bool small = g.M <= SMALL_M;
  if (g.B2 && !(epi == EPI_SWIGLU && small)) return -1;
  // above 4096 rows (batches of 32 canvases): the LM head's 256x256 tiles,
  // which move a third to two thirds fewer bytes per CU than the tiles below
  // (8192 rows at d_model 2048: 69.5 against 73.1 ms per step, same bits;
  // neutral at 4096)
  if (g.M > 4096) {
    switch (epi) {
      case EPI_QKV: return launch_dl<256, 256, 4, 8, 2, 3, EPI_QKV>(g, st);
      case EPI_SWIGLU: return launch_dl<256, 256, 4, 8, 2, 3, EPI_SWIGLU>(g, st);
      case EPI_RESID: return launch_dl<256, 256, 4, 8, 2, 3, EPI_RESID>(g, st);
      case EPI_F32: return launch_dl<256, 256, 4, 8, 2, 3, EPI_F32>(g, st);
      default: return -1;
    }
  }
  switch (epi) {
    case EPI_QKV:
      return small ? launch_dl<64, 128, 2, 8, 3, 6, EPI_QKV>(g, st) : launch_dl<128, 256, 2, 8, 2, 3, EPI_QKV>(g, st);
    case EPI_SWIGLU:
      // with a second product (the router logits) the rings shrink to A 3 /
      // B 6 (72 KB), so two workgroups share a CU and the extra tiles run in
      // the same round
      if (small && g.B2) return launch_dl<64, 64, 4, 8, 3, 6, EPI_SWIGLU>(g, st);
      return small ? launch_dl<64, 64, 4, 8, 4, 8, EPI_SWIGLU>(g, st)
                   : launch_dl<128, 128, 4, 8, 3, 4, EPI_SWIGLU>(g, st);
    // small M: 64x32 tiles of four waves (one 16x32 strip each), 256
    // workgroups at N = 2048, rings of 6 stages (72 KB)
    case EPI_RESID:
      return small ? launch_dl<64, 32, 4, 4, 6, 6, EPI_RESID>(g, st) : launch_dl<64, 128, 2, 8, 3, 6, EPI_RESID>(g, st);
    case EPI_F32:
      return small ? launch_dl<64, 32, 4, 4, 6, 6, EPI_F32>(g, st) : launch_dl<64, 128, 2, 8, 3, 6, EPI_F32>(g, st);
    default:
      return -1;
  }
}

template <typename TB>
int dispatch(GemmEpi epi, const GemmArgs& g, hipStream_t st) {
  const long long tiles64 = (long long)((g.M + 63) / 64) * ((g.N + 63) / 64);
  if (epi == EPI_QKV && (g.N % 128 || !g.seq_n || !g.heads || g.N != 3 * 128 * g.heads))
    return int(hipErrorInvalidValue);
  if constexpr (std::is_same<TB, bf16>::value) {
    const int r = dense_direct(epi, g, st);
    if (r >= 0) return r;
  }
  if (g.B2) return int(hipErrorInvalidValue);  // only the direct-load kernel computes a second product
  switch (epi) {
    case EPI_LM:
      if constexpr (std::is_same<TB, bf16>::value)
        if (lm_direct(g.K)) return launch_dl<LMD_BM, LMD_BN, LMD_WM, LMD_NW, LMD_SA, LMD_SB, EPI_LM, LMD_KT>(g, st);
      return launch_t<TB, LM_BM, LM_BN, LM_WM, 2, EPI_LM>(g, st);
    case EPI_SWIGLU:
      return launch_kg<TB, 64, 64, 2, 2, EPI_SWIGLU>(g, st, 2);
    case EPI_QKV:
      if (g.K % 128 == 0) return launch_t<TB, 64, 128, 4, 2, EPI_QKV, 64, 2>(g, st);
      return launch_t<TB, 64, 128, 4, 2, EPI_QKV, 64, 1>(g, st);
    case EPI_ACT:
      if (tiles64 >= 256) return launch_kg<TB, 64, 64, 2, 2, EPI_ACT>(g, st, 2);
      return launch_kg<TB, 64, 32, 2, 2, EPI_ACT>(g, st, 2);
    case EPI_RESID:
      if (tiles64 >= 256) return launch_kg<TB, 64, 64, 2, 2, EPI_RESID>(g, st, 2);
      return launch_kg<TB, 64, 32, 2, 2, EPI_RESID>(g, st, 2);
    case EPI_F32:
      if (tiles64 >= 256) return launch_kg<TB, 64, 64, 2, 2, EPI_F32>(g, st, 2);
      if (tiles64 >= 64) return launch_kg<TB, 64, 32, 2, 2, EPI_F32>(g, st, 2);
      return launch_kg<TB, 32, 32, 2, 2, EPI_F32>(g, st, 4);
  }
  return int(hipErrorInvalidValue);
}

// ---------------------------------------------------------------------------
// Grouped routed-expert GEMM for many pairs per expert (pooled canvases,
// mixed passes): a plain grid of (expert, 128-output tile, 128-pair tile)
// items over the expert-major pair lists, each a 128 x 128 output tile whose
// operands reach LDS by direct loads.  The expert weights are already tiled
// in the matrix-core operand layout (16 rows x 32 columns per 1 KB block,
// lane l's 16 bytes its fragment), so a block is copied to LDS as is and a
// lane reads its fragment at lane x 16; the pairs' token rows (gathered
// through pair_row for gate/up, contiguous h rows for down) go to 8-row
// blocks with the XOR chunk swizzle of the dense kernel.  The weights are the
// A operand and the tokens the B operand, and every output sums its 32-column
// k blocks in ascending order, as the weight-stream kernels do, so the two
// give the same bits.  Gate/up: 128 gate and 128 up weight rows per tile,
// h = bf16(silu(gate) up); down: 128 weight rows, y fp32.
//
// Waves: 8 = 2 token groups of BM / 2 x 4 output groups of 32; a wave holds
// BM / 32 token blocks x (4 gate/up or 2 down) weight blocks of accumulators.
// BM = 128 with a 3-stage ring up to a few hundred pairs per expert (64-pair
// tiles: 174 against 153 us at 64 pairs per expert, 223 against 196 at 128;
// 145 against 147 us at 32), BM = 256 above (see grouped_experts).
// Items are ordered expert, then output tile, then pair tile, so the pair
// tiles of one expert's weight tile run side by side on one XCD and share it
// in L2; items past the last one exit at once (the grid is a bound).
namespace gex {
constexpr int BN = 128;  // outputs per tile
constexpr int NWV = 8;
}  // namespace gex

// BM: pairs per tile (64, 128 or 256)
template <bool GU, int KT, int S, int BM>
__global__ __launch_bounds__(64 * gex::NWV) void grouped_kernel(const bf16* __restrict__ X, const int* __restrict__ pair_row,
                                                                const int* __restrict__ off, int E, const bf16* __restrict__ W,
                                                                int Nout, void* __restrict__ out, int per_xcd) {
  using namespace gex;
  constexpr int K = 64 * KT;
  constexpr int WB = GU ? 16 : 8;        // 16-row weight blocks per tile
  constexpr int NWB = WB / 4;            // per wave (GU: 2 gate + 2 up)
  constexpr int MT = BM / 32;            // 16-pair blocks per wave (2 token groups)
  constexpr int LA = BM / 8 / NWV;       // token loads per wave per stage
  constexpr int LB = 2 * WB / NWV;       // weight loads per wave per stage (GU 4, down 2)
  static_assert(LA * 8 * NWV == BM && LB * NWV == 2 * WB && S >= 2 && S <= 4, "shape");
#define DG_GX_BUF(X_, R, BYTES, I) __shared__ __attribute__((aligned(1024))) char X_##I[R > I ? BYTES : 1];
  DG_GX_BUF(TS, S, BM * 128, 0) DG_GX_BUF(TS, S, BM * 128, 1) DG_GX_BUF(TS, S, BM * 128, 2) DG_GX_BUF(TS, S, BM * 128, 3)
  DG_GX_BUF(WS, S, WB * 2048, 0) DG_GX_BUF(WS, S, WB * 2048, 1) DG_GX_BUF(WS, S, WB * 2048, 2) DG_GX_BUF(WS, S, WB * 2048, 3)
#undef DG_GX_BUF
  auto tbuf = [&](auto bc) -> char* {
    constexpr int b = decltype(bc)::value % S;
    if constexpr (b == 0) return TS0;
    else if constexpr (b == 1) return TS1;
    else if constexpr (b == 2) return TS2;
    else return TS3;
  };
  auto wbuf = [&](auto bc) -> char* {
    constexpr int b = decltype(bc)::value % S;
    if constexpr (b == 0) return WS0;
    else if constexpr (b == 1) return WS1;
    else if constexpr (b == 2) return WS2;
    else return WS3;
  };

  // item -> (expert, output tile, pair tile): wave 0 scans the experts' pair-tile counts.
  // The grid holds per_xcd slots on each XCD (a bound from the pair count); the
  // items, counted on the device, are dealt out in eight equal contiguous runs,
  // run x on XCD x, so every XCD gets the same share whatever the bound.
  __shared__ int sel[4];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slot = blockIdx.x >> 3;
  if (slot >= per_xcd) return;  // uniform
  const int NT = (Nout + BN - 1) / BN;
  if (wave == 0) {
    // lane l owns experts 4l .. 4l+3
    int c[4], s = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = 4 * lane + u;
      c[u] = e < E ? NT * ((off[e + 1] - off[e] + BM - 1) / BM) : 0;
      s += c[u];
    }
    int incl = s;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    const int total = __shfl(incl, 63, 64);
    const int per = (total + 7) >> 3;  // <= per_xcd: the bound covers every item
    const int item = slot < per ? (blockIdx.x & 7) * per + slot : total;
    int run = incl - s;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (c[u] && item >= run && item < run + c[u]) {
        sel[0] = 4 * lane + u;
        sel[1] = item - run;
      }
      run += c[u];
    }
    if (lane == 63) {
      sel[2] = total;
      sel[3] = item;
    }
  }
  __syncthreads();
  if (sel[3] >= sel[2]) return;  // uniform: past the last item
  const int e = sel[0], j = sel[1];
  const int pbeg = off[e], cnt = off[e + 1] - pbeg;
  const int mtiles = (cnt + BM - 1) / BM;
  const int nt = j / mtiles, m0 = (j - nt * mtiles) * BM, n0 = nt * BN;

  // token row of this lane's loads: block q = wave + NWV i holds pair rows 8q .. 8q+7
  const int rr8 = lane >> 3, ch = (lane & 7) ^ rr8;
  const bf16* tsrc[LA];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int r = min(m0 + 8 * (wave + NWV * i) + rr8, cnt - 1);  // past the pairs: the last pair's row
    const long long row = GU ? (long long)pair_row[pbeg + r] : (long long)(pbeg + r);
    tsrc[i] = X + row * K + 8 * ch;
  }
  // weight load l of this wave: tile block b = (wave LB + l) / 2, k half (wave LB + l) % 2;
  // block b < 8 holds rows n0 + 16 b (gate for GU), b >= 8 the up rows Nout + n0 + 16 (b - 8)
  const long long wrows = GU ? 2LL * Nout : Nout;
  const char* wexp = (const char*)(W + (long long)e * wrows * K);
  const char* wsrc[LB];
  int wdst[LB];
#pragma unroll
  for (int l = 0; l < LB; ++l) {
    const int q = wave * LB + l, b = q >> 1, hf = q & 1;
    const int nb = min(n0 + 16 * (b & 7), ((Nout - 1) >> 4) << 4);  // past Nout: the last block
    const long long rb = (GU && b >= 8 ? Nout + nb : nb) >> 4;
    wsrc[l] = wexp + (rb * (K / 32) + hf) * 1024 + lane * 16;
    wdst[l] = (b * 2 + hf) * 1024;
  }
  auto issue_t = [&](int kt, char* bufp) {
#pragma unroll
    for (int i = 0; i < LA; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(tsrc[i] + kt * 64), (dl::lds_ptr)(bufp + (wave + NWV * i) * 1024),
                                       16, 0, 0);
  };
  auto issue_w = [&](int kt, char* bufp) {
#pragma unroll
    for (int l = 0; l < LB; ++l)
      __builtin_amdgcn_global_load_lds((const void*)(wsrc[l] + kt * 2048), (dl::lds_ptr)(bufp + wdst[l]), 16, 0, 0);
  };

  const int c16 = lane & 15, g4 = lane >> 4, rr = lane & 7;
  const int tg = wave >> 2, og = wave & 3;
  f32x4 acc[NWB][MT];
#pragma unroll
  for (int w = 0; w < NWB; ++w)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[w][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // wave's weight blocks: GU gate 2 og, 2 og + 1, up 8 + 2 og, 8 + 2 og + 1; down 2 og, 2 og + 1
  auto wblk = [&](int w) { return GU ? (w < 2 ? 2 * og + w : 8 + 2 * og + (w - 2)) : 2 * og + w; };
  auto compute = [&](const char* tb, const char* wb) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      u32x4 wf[NWB], tf[MT];
#pragma unroll
      for (int w = 0; w < NWB; ++w) wf[w] = *(const u32x4*)(wb + (wblk(w) * 2 + hf) * 1024 + lane * 16);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int r0 = (BM / 2) * tg + 16 * t;
        tf[t] = *(const u32x4*)(tb + 2 * (((r0 >> 3) + (c16 >> 3)) * 512 + (rr * 8 + ((4 * hf + g4) ^ rr)) * 8));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int w = 0; w < NWB; ++w)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[w][t] = mfma16x16x32(wf[w], tf[t], acc[w][t]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  dl::static_for<S - 1>([&](auto sc) {
    constexpr int st = decltype(sc)::value;
    if constexpr (st < KT) {
      issue_t(st, tbuf(sc));
      issue_w(st, wbuf(sc));
    }
  });
  dl::static_for<KT>([&](auto kc) {
    constexpr int kt = decltype(kc)::value;
    dl::wait_barrier<dl::loads_after<S, S, KT, LA, LB>(kt)>();
    if constexpr (kt + S - 1 < KT) {
      issue_t(kt + S - 1, tbuf(std::integral_constant<int, kt + S - 1>{}));
      issue_w(kt + S - 1, wbuf(std::integral_constant<int, kt + S - 1>{}));
    }
    compute(tbuf(kc), wbuf(kc));
  });

  // epilogue: lane holds pair 64 tg + 16 t + c16 and outputs nb .. nb + 3 of block b
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int nb = n0 + 32 * og + 16 * b + 4 * g4;
    if (nb >= Nout) continue;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int r = m0 + (BM / 2) * tg + 16 * t + c16;
      if (r >= cnt) continue;
      const long long p = pbeg + r;
      if constexpr (GU) {
        bf16 hv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float gt = acc[b][t][q], up = acc[2 + b][t][q];
          hv[q] = f32_to_bf16(gt / (1.0f + __expf(-gt)) * up);
        }
        bf16* h = (bf16*)out + p * Nout + nb;
        if (nb + 3 < Nout) {
          *(u32x2*)h = u32x2{uint32_t(hv[0].v) | (uint32_t(hv[1].v) << 16), uint32_t(hv[2].v) | (uint32_t(hv[3].v) << 16)};
        } else {
          for (int q = 0; q < 4 && nb + q < Nout; ++q) h[q] = hv[q];
        }
      } else {
        float* y = (float*)out + p * Nout + nb;
        if (nb + 3 < Nout) *(f32x4*)y = acc[b][t];
        else
          for (int q = 0; q < 4 && nb + q < Nout; ++q) y[q] = acc[b][t][q];
      }
    }
  }
}

template <bool GU, int KT, int S, int BM>
int launch_grouped(const bf16* X, const int* pair_row, const int* off, int E, int pairs, const bf16* W, int Nout,
                   void* out, hipStream_t st) {
  using namespace gex;
  const int NT = (Nout + BN - 1) / BN;
  const long long items = (long long)NT * ((pairs + BM - 1) / BM + E);  // a bound on the items
  const int per_xcd = int((items + 7) / 8);
  hipLaunchKernelGGL((grouped_kernel<GU, KT, S, BM>), dim3(8 * per_xcd), dim3(64 * NWV), 0, st, X, pair_row, off, E, W,
                     Nout, out, per_xcd);
  return int(hipGetLastError());
}

}  // namespace

int gemm_f32_topk(const GemmArgs& g, hipStream_t st) {
  constexpr int BM = 64, BN = 32, NWV = 4;
  if (g.K != 2048 || g.lda % 8 || g.ldb % 8 || g.N < 1024 || g.M > SMALL_M || g.B2) return -1;
  if (!g.tk_logits || g.tk_T <= 0 || g.tk_E > 128 || g.tk_k > 8 || g.tk_k > g.tk_E) return -1;
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  const int per_xcd = (tiles_m * tiles_n + 7) / 8;
  const int tk_wgs = (g.tk_T + NWV - 1) / NWV, tk_per_xcd = (tk_wgs + 7) / 8;
  hipLaunchKernelGGL((dgemm_kernel<BM, BN, 4, NWV, 6, 6, EPI_F32, 32, true>), dim3(8 * (per_xcd + tk_per_xcd)),
                     dim3(64 * NWV), 0, st, g, tiles_m, tiles_n, 0, per_xcd, tk_per_xcd);
  return int(hipGetLastError());
}

int lm_tiles_tiled(int vocab, int K) {
  if (lm_direct(K)) return (vocab + LMD_BN - 1) / LMD_BN * (LMD_NW / LMD_WM);
  return (vocab + LM_BN - 1) / LM_BN * (4 / LM_WM);
}

bool tgemm_supported(ActType at, int K) { return at == ACT_BF16 && K % SK_MIN == 0; }

bool grouped_supported(bool gate_up, int K, int Nout, int E) {
  return E <= 256 && Nout % 16 == 0 && (gate_up ? K == 2048 : K == 704);
}

int grouped_experts(bool gate_up, const void* X, const int* pair_row, const int* off, int E, int pairs,
                    const void* W, int K, int Nout, void* out, hipStream_t st) {
  if (!grouped_supported(gate_up, K, Nout, E) || pairs <= 0) return int(hipErrorInvalidValue);
  // 256-pair tiles (two stages in LDS for gate/up, three for down) from 384
  // pairs per expert: at 512 (d_model 2048, 128 experts of 704, 8192 tokens)
  // gate/up 451 against 476 us, down 373 against 419 us; at 256 and below the
  // 128-pair tiles win (gate/up 281 against 294 us at 256, 153 against 184 at 64)
  const bool big = pairs >= 384LL * E;
  if (gate_up) {
    if (big) return launch_grouped<true, 32, 2, 256>((const bf16*)X, pair_row, off, E, pairs, (const bf16*)W, Nout, out, st);
    return launch_grouped<true, 32, 3, 128>((const bf16*)X, pair_row, off, E, pairs, (const bf16*)W, Nout, out, st);
  }
  if (big) return launch_grouped<false, 11, 3, 256>((const bf16*)X, pair_row, off, E, pairs, (const bf16*)W, Nout, out, st);
  return launch_grouped<false, 11, 4, 128>((const bf16*)X, pair_row, off, E, pairs, (const bf16*)W, Nout, out, st);
}

int tgemm(WType wt, GemmEpi epi, const GemmArgs& g, hipStream_t st) {
  if (g.K % SK_MIN || g.g_off) return int(hipErrorInvalidValue);
  if (wt == W_BF16) return dispatch<bf16>(epi, g, st);
  if (wt == W_FP8 && epi != EPI_LM) return dispatch<f8>(epi, g, st);
  return int(hipErrorInvalidValue);
}

}  // namespace dg
