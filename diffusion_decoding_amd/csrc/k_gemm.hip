// GEMM family for the denoise step on gfx950: C = A * B^T with both operands
// stored k-contiguous ([rows][K]), LDS-staged 64x64 tiles, 4 waves in a 2x2
// arrangement, MFMA 16x16x32 bf16 (or 16x16x4 f32 for fp32 workloads), and a
// tile epilogue through LDS.  Optional row gather (MoE: token rows of each
// expert) and grouping (grid.z = expert, row range from a device offset table).
//
// The LM-head epilogue turns each row's logits in the tile into an online-
// softmax partial (max, argmax, second max, sum e^(z-max), sum e^(z-max)(z-max))
// so logits never reach HBM; lm_merge folds the partials of a row in a fixed
// order into its entropy H = ln(sum) - t/sum, argmax and top-2 gap.  Entropy as
// the confidence of a position: DiffusionGemma解析, "换个路数：整片并行去噪的生成机制".
#include <climits>
#include <type_traits>

#include "dg_common.h"
#include "kernels.h"

namespace dg {
namespace {

struct fp8 {
  uint8_t v;
};

constexpr int BK = 32;
constexpr int NT = 256;

template <typename CT> struct LdsCfg;
template <> struct LdsCfg<float> {
  static constexpr int PAD = 4, EPC = 4;  // elements per 16-byte chunk
};
template <> struct LdsCfg<bf16> {
  static constexpr int PAD = 8, EPC = 8;
};

// 16-byte chunk of 8 elements of B converted to the bf16 compute type.
__device__ __forceinline__ u32x4 load_chunk_bf(const bf16* p) { return *(const u32x4*)p; }
__device__ __forceinline__ u32x4 load_chunk_bf(const fp8* p) { return e4m3x8_to_bf16x8(*(const u32x2*)p); }
__device__ __forceinline__ u32x4 load_chunk_f(const float* p) { return *(const u32x4*)p; }

template <typename TA, typename TB, int BM, int BN, int EPI>
__global__ __launch_bounds__(NT) void gemm_nt(GemmArgs g) {
  constexpr bool F32 = std::is_same<TA, float>::value;
  using CT = typename std::conditional<F32, float, bf16>::type;
  constexpr int EPC = LdsCfg<CT>::EPC;
  constexpr int LDK = BK + LdsCfg<CT>::PAD;
  constexpr int CPR = BK / EPC;
  constexpr int A_CH = BM * CPR, B_CH = BN * CPR;
  constexpr int A_PT = (A_CH + NT - 1) / NT, B_PT = (B_CH + NT - 1) / NT;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int LDC = BN + 4;
  constexpr int BN_OUT = (EPI == EPI_SWIGLU) ? BN / 2 : BN;

  __shared__ __attribute__((aligned(16))) CT As[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) CT Bs[2][BN * LDK];
  __shared__ float Cs[BM * LDC];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, g4 = lane >> 4;
  const int wr = (wave >> 1) * WM, wc = (wave & 1) * WN;
  const int grp = blockIdx.z;
  int row_begin = 0, row_end = g.M;
  if (g.g_off) {
    row_begin = g.g_off[grp];
    row_end = g.g_off[grp + 1];
  }
  const TA* Ag = (const TA*)g.A;
  const TB* Bg = (const TB*)g.B + (long long)grp * g.b_gstride;
  const float* Sg = g.b_scale ? g.b_scale + (long long)grp * g.s_gstride : nullptr;
  const int n0 = blockIdx.x * BN_OUT;
  const int KT = g.K / BK;

  // B rows of this tile (fixed over the m loop)
  const TB* bptr[B_PT];
  bool bok[B_PT];
  int bkc[B_PT], brl[B_PT];
#pragma unroll
  for (int u = 0; u < B_PT; ++u) {
    int c = tid + u * NT;
    int r = c / CPR;
    bkc[u] = (c % CPR) * EPC;
    brl[u] = r;
    long long brow;
    bool ok;
    if (EPI == EPI_SWIGLU) {
      int j = n0 + (r < BN / 2 ? r : r - BN / 2);
      ok = (c < B_CH) && j < g.N;
      brow = (r < BN / 2) ? j : (long long)g.swiglu_half + j;
    } else {
      int n = n0 + r;
      ok = (c < B_CH) && n < g.N;
      brow = n;
    }
    bok[u] = ok;
    bptr[u] = Bg + (ok ? brow * g.ldb : 0) + bkc[u];
  }

  for (int m0 = row_begin + blockIdx.y * BM; m0 < row_end; m0 += gridDim.y * BM) {
    const TA* aptr[A_PT];
    bool aok[A_PT];
    int akc[A_PT], arl[A_PT];
#pragma unroll
    for (int u = 0; u < A_PT; ++u) {
      int c = tid + u * NT;
      int r = c / CPR;
      akc[u] = (c % CPR) * EPC;
      arl[u] = r;
      int m = m0 + r;
      bool ok = (c < A_CH) && m < row_end;
      long long arow = ok ? (g.a_rows ? g.a_rows[m] : m) : 0;
      aok[u] = ok;
      aptr[u] = Ag + arow * g.lda + akc[u];
    }

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 ra[A_PT], rb[B_PT];
    auto gload = [&](int kt) {
#pragma unroll
      for (int u = 0; u < A_PT; ++u) {
        u32x4 z = {0u, 0u, 0u, 0u};
        if (aok[u]) {
          if constexpr (F32) z = load_chunk_f((const float*)(aptr[u] + kt * BK));
          else z = load_chunk_bf((const bf16*)(aptr[u] + kt * BK));
        }
        ra[u] = z;
      }
#pragma unroll
      for (int u = 0; u < B_PT; ++u) {
        u32x4 z = {0u, 0u, 0u, 0u};
        if (bok[u]) {
          if constexpr (F32) z = load_chunk_f((const float*)(bptr[u] + kt * BK));
          else z = load_chunk_bf(bptr[u] + kt * BK);
        }
        rb[u] = z;
      }
    };
    auto lstore = [&](int buf) {
#pragma unroll
      for (int u = 0; u < A_PT; ++u)
        if (tid + u * NT < A_CH) *(u32x4*)&As[buf][arl[u] * LDK + akc[u]] = ra[u];
#pragma unroll
      for (int u = 0; u < B_PT; ++u)
        if (tid + u * NT < B_CH) *(u32x4*)&Bs[buf][brl[u] * LDK + bkc[u]] = rb[u];
    };

    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < KT) gload(kt + 1);
      if constexpr (F32) {
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          float af[FM], bfv[FN];
#pragma unroll
          for (int i = 0; i < FM; ++i) af[i] = As[buf][(wr + 16 * i + c16) * LDK + 4 * s + g4];
#pragma unroll
          for (int j = 0; j < FN; ++j) bfv[j] = Bs[buf][(wc + 16 * j + c16) * LDK + 4 * s + g4];
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = mfma16x16x4f32(af[i], bfv[j], acc[i][j]);
        }
      } else {
        u32x4 af[FM], bfv[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) af[i] = *(const u32x4*)&As[buf][(wr + 16 * i + c16) * LDK + 8 * g4];
#pragma unroll
        for (int j = 0; j < FN; ++j) bfv[j] = *(const u32x4*)&Bs[buf][(wc + 16 * j + c16) * LDK + 8 * g4];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = mfma16x16x32(af[i], bfv[j], acc[i][j]);
      }
      if (kt + 1 < KT) lstore(buf ^ 1);
      __syncthreads();
    }

    // accumulators -> LDS tile
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          Cs[(wr + 16 * i + 4 * g4 + r) * LDC + wc + 16 * j + c16] = acc[i][j][r];
    __syncthreads();

    if constexpr (EPI == EPI_F32 || EPI == EPI_ACT || EPI == EPI_RESID) {
      for (int e = tid; e < BM * BN; e += NT) {
        int r = e / BN, c = e % BN;
        int m = m0 + r, n = n0 + c;
        if (m >= row_end || n >= g.N) continue;
        float v = Cs[r * LDC + c];
        if (Sg) v *= Sg[n];
        long long o = (long long)m * g.ldc + n;
        if constexpr (EPI == EPI_F32) {
          ((float*)g.C)[o] = v;
        } else if constexpr (EPI == EPI_ACT) {
          ((TA*)g.C)[o] = from_f32<TA>(v);
        } else {
          TA* C = (TA*)g.C;
          C[o] = from_f32<TA>(to_f32(C[o]) + v);
        }
      }
    } else if constexpr (EPI == EPI_SWIGLU) {
      for (int e = tid; e < BM * (BN / 2); e += NT) {
        int r = e / (BN / 2), c = e % (BN / 2);
        int m = m0 + r, j = n0 + c;
        if (m >= row_end || j >= g.N) continue;
        float gt = Cs[r * LDC + c], up = Cs[r * LDC + BN / 2 + c];
        if (Sg) {
          gt *= Sg[j];
          up *= Sg[g.swiglu_half + j];
        }
        float h = gt / (1.0f + __expf(-gt)) * up;
        ((TA*)g.C)[(long long)m * g.ldc + j] = from_f32<TA>(h);
      }
    } else if constexpr (EPI == EPI_LM) {
      // NT / BM threads per row, each over BN / (NT / BM) columns
      constexpr int TPR = NT / BM, CPT = BN / TPR;
      static_assert(TPR >= 1 && (TPR & (TPR - 1)) == 0, "row split");
      const int r = tid / TPR, sub = tid % TPR;
      LmPart p = lm_empty_part();
#pragma unroll 4
      for (int c = sub * CPT; c < sub * CPT + CPT; ++c) {
        int n = n0 + c;
        if (n >= g.N) break;
        float z = Cs[r * LDC + c];
        if (z > p.m) {
          p.sec = p.m;
          p.m = z;
          p.idx = n;
        } else if (z > p.sec) {
          p.sec = z;
        }
      }
      if (p.idx != INT_MAX) {
        for (int c = sub * CPT; c < sub * CPT + CPT; ++c) {
          int n = n0 + c;
          if (n >= g.N) break;
          float d = Cs[r * LDC + c] - p.m;
          float e = __expf(d);
          p.s += e;
          p.t += e * d;
        }
      }
      // no column above -inf while some column exists: every logit NaN or -inf
      if (p.idx == INT_MAX && n0 + sub * CPT < g.N && m0 + r < row_end && g.flags) atomicOr(g.flags, FLAG_NONFINITE);
#pragma unroll
      for (int o = 1; o < TPR; o <<= 1) p = lm_combine(p, lm_shfl_xor(p, o));
      int m = m0 + r;
      if (sub == 0 && m < row_end) {
        float* out = g.part + ((long long)m * gridDim.x + blockIdx.x) * 5;
        out[0] = p.m;
        out[1] = p.s;
        out[2] = p.t;
        out[3] = p.sec;
        out[4] = __int_as_float(p.idx);
      }
    }
    __syncthreads();
  }
}

// one workgroup per row: thread l folds tiles l, l + 256, ... (four loads in
// flight per step), then a fixed xor tree inside each wave and the four wave
// results in wave order.
__global__ __launch_bounds__(256) void lm_merge_kernel(const float* part, int T, int n_tiles,
                                                       float* H, int* am, float* gap, int* flags) {
  __shared__ float wp[4][5];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  LmPart acc = lm_empty_part();
  const float* base = part + (long long)row * n_tiles * 5;
  for (int t0 = tid; t0 < n_tiles; t0 += 1024) {
    LmPart p[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = t0 + 256 * u;
      p[u] = lm_empty_part();
      if (t < n_tiles) {
        p[u].m = base[t * 5 + 0];
        p[u].s = base[t * 5 + 1];
        p[u].t = base[t * 5 + 2];
        p[u].sec = base[t * 5 + 3];
        p[u].idx = __float_as_int(base[t * 5 + 4]);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc = lm_combine(acc, p[u]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc = lm_combine(acc, lm_shfl_xor(acc, o));
  if (lane == 0) {
    wp[wave][0] = acc.m;
    wp[wave][1] = acc.s;
    wp[wave][2] = acc.t;
    wp[wave][3] = acc.sec;
    wp[wave][4] = __int_as_float(acc.idx);
  }
  __syncthreads();
  if (tid == 0) {
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      LmPart p;
      p.m = wp[w][0];
      p.s = wp[w][1];
      p.t = wp[w][2];
      p.sec = wp[w][3];
      p.idx = __float_as_int(wp[w][4]);
      acc = lm_combine(acc, p);
    }
    const float h = logf(acc.s) - acc.t / acc.s;
    // a NaN or infinite logit anywhere in the row makes s or t NaN
    if (flags && (!(fabsf(h) <= 3.402823466e38f) || acc.idx == INT_MAX)) atomicOr(flags, FLAG_NONFINITE);
    if (H) H[row] = h;
    if (am) am[row] = acc.idx;
    if (gap) gap[row] = acc.m - acc.sec;
  }
}

template <typename TA, typename TB, int EPI>
int launch(const GemmArgs& g, int groups, hipStream_t st) {
  constexpr int BM = 64, BN = 64;
  const int bn_out = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  dim3 grid((g.N + bn_out - 1) / bn_out, g.g_off ? 1 : (g.M + BM - 1) / BM, groups);
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return 0;
  hipLaunchKernelGGL((gemm_nt<TA, TB, BM, BN, EPI>), grid, dim3(NT), 0, st, g);
  return int(hipGetLastError());
}

template <typename TA, typename TB>
int launch_epi(GemmEpi epi, const GemmArgs& g, int groups, hipStream_t st) {
  switch (epi) {
    case EPI_F32: return launch<TA, TB, EPI_F32>(g, groups, st);
    case EPI_ACT: return launch<TA, TB, EPI_ACT>(g, groups, st);
    case EPI_RESID: return launch<TA, TB, EPI_RESID>(g, groups, st);
    case EPI_SWIGLU: return launch<TA, TB, EPI_SWIGLU>(g, groups, st);
    case EPI_LM: return launch<TA, TB, EPI_LM>(g, groups, st);
  }
  return int(hipErrorInvalidValue);
}

}  // namespace

int lm_tiles(ActType at, int K, int vocab) {
  return tgemm_supported(at, K) ? lm_tiles_tiled(vocab, K) : (vocab + 63) / 64;
}

int gemm(ActType at, WType wt, GemmEpi epi, const GemmArgs& g, int groups, hipStream_t st) {
  if (g.K % BK) return int(hipErrorInvalidValue);
  if (!g.g_off && tgemm_supported(at, g.K)) return tgemm(wt, epi, g, st);
  if (g.B2) return int(hipErrorInvalidValue);  // a second product needs the bf16 direct-load kernel
  if (at == ACT_F32 && wt == W_F32) return launch_epi<float, float>(epi, g, groups, st);
  if (at == ACT_BF16 && wt == W_BF16) return launch_epi<bf16, bf16>(epi, g, groups, st);
  if (at == ACT_BF16 && wt == W_FP8) {
    if (epi == EPI_LM) return int(hipErrorInvalidValue);
    return launch_epi<bf16, fp8>(epi, g, groups, st);
  }
  return int(hipErrorInvalidValue);
}

int lm_merge(const float* part, int T, int n_tiles, float* entropy, int* argmax, float* gap, int* flags,
             hipStream_t st) {
  if (T <= 0) return 0;
  hipLaunchKernelGGL(lm_merge_kernel, dim3(T), dim3(256), 0, st, part, T, n_tiles, entropy, argmax, gap, flags);
  return int(hipGetLastError());
}

}  // namespace dg
