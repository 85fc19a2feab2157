// Canvas attention on gfx950: flash-style single pass over [prompt KV ; canvas
// KV] per (canvas, head) with no mask -- every canvas position attends to every
// cached key and every canvas key (DiffusionGemma解析, "换个路数：整片并行去噪的
// 生成机制": bidirectional attention over the canvas; zhichai.net 深度拆解,
// "架构解剖": the canvas decoder reads the prompt's KV cache).  The same kernel
// with a causal bound serves the commit pass that appends a canvas to the cache
// (zhichai.net 深度拆解, "Block-Autoregressive").
//
// Work split: a workgroup holds 64 queries (4 waves x 16); K and V tiles of 64
// keys are staged in LDS (V transposed) and shared by the 4 waves.  Each wave
// computes S^T = K Q^T with MFMA, so a lane owns one query column; the online
// softmax then needs only a 4-lane reduction, and the probabilities feed the
// P*V MFMA straight from the accumulator registers as its B operand
// (O^T = V^T P^T).  Key ranges are split across workgroups when the head/query
// grid alone cannot fill the chip; a merge kernel combines the partials.
#include <type_traits>

#include "dg_common.h"
#include "kernels.h"

namespace dg {
namespace {

constexpr int KTILE = 64;

template <typename T, int DH>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a, int keys_per_split) {
  constexpr bool BF = std::is_same<T, bf16>::value;
  constexpr int EPC = BF ? 8 : 4;  // elements per 16-byte chunk
  constexpr int LDKS = DH + EPC;
  constexpr int LDV = KTILE + EPC;
  constexpr int NDF = DH / 16;
  __shared__ __attribute__((aligned(16))) T Ks[KTILE * LDKS];
  __shared__ __attribute__((aligned(16))) T Vt[DH * LDV];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, c16 = lane & 15;
  const int bh = blockIdx.y, b = bh / a.H, h = bh % a.H;
  const int qi = blockIdx.x * 64 + wave * 16 + c16;
  const int total = a.len0 + a.len1;
  const int kbeg = blockIdx.z * keys_per_split;
  const int kend = min(total, kbeg + keys_per_split);
  const float scale = 1.0f / sqrtf(float(DH));

  const T* qrow = (const T*)a.q + ((long long)bh * a.n + min(qi, a.n - 1)) * DH;
  const bool qvalid = qi < a.n;
  const T* K0 = (const T*)a.k0 + (long long)bh * a.s0_bh;
  const T* V0 = (const T*)a.v0 + (long long)bh * a.s0_bh;
  const T* K1 = a.len1 ? (const T*)a.k1 + (long long)bh * a.s1_bh : nullptr;
  const T* V1 = a.len1 ? (const T*)a.v1 + (long long)bh * a.s1_bh : nullptr;

  // Q as the B operand of S^T = K Q^T
  constexpr int NQ = BF ? DH / 32 : DH / 4;
  u32x4 qf[BF ? NQ : 1];
  float qs[BF ? 1 : NQ];
  if constexpr (BF) {
#pragma unroll
    for (int ks = 0; ks < NQ; ++ks) qf[ks] = *(const u32x4*)(qrow + 32 * ks + 8 * g4);
  } else {
#pragma unroll
    for (int ks = 0; ks < NQ; ++ks) qs[ks] = to_f32(qrow[4 * ks + g4]);
  }

  f32x4 o[NDF];
#pragma unroll
  for (int df = 0; df < NDF; ++df) o[df] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  for (int kt0 = kbeg; kt0 < kend; kt0 += KTILE) {
    __syncthreads();
    constexpr int CPRW = DH / EPC;
    for (int c = tid; c < KTILE * CPRW; c += 256) {
      const int row = c / CPRW, col = (c % CPRW) * EPC;
      const int j = kt0 + row;
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (j < kend) {
        const T* kp = j < a.len0 ? K0 + (long long)j * DH : K1 + (long long)(j - a.len0) * DH;
        const T* vp = j < a.len0 ? V0 + (long long)j * DH : V1 + (long long)(j - a.len0) * DH;
        kv = *(const u32x4*)(kp + col);
        vv = *(const u32x4*)(vp + col);
      }
      *(u32x4*)&Ks[row * LDKS + col] = kv;
      if constexpr (BF) {
        const uint16_t* hv = (const uint16_t*)&vv;
#pragma unroll
        for (int e = 0; e < 8; ++e) ((uint16_t*)Vt)[(col + e) * LDV + row] = hv[e];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) Vt[(col + e) * LDV + row] = __uint_as_float(vv[e]);
      }
    }
    __syncthreads();

    // S^T for 64 keys: 4 fragments of 16 keys; lane holds keys 16f + 4g4 + r of query qi
    f32x4 s[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      s[f] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (BF) {
#pragma unroll
        for (int ks = 0; ks < NQ; ++ks) {
          u32x4 ka = *(const u32x4*)&Ks[(16 * f + c16) * LDKS + 32 * ks + 8 * g4];
          s[f] = mfma16x16x32(ka, qf[ks], s[f]);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < NQ; ++ks)
          s[f] = mfma16x16x4f32(to_f32(Ks[(16 * f + c16) * LDKS + 4 * ks + g4]), qs[ks], s[f]);
      }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = kt0 + 16 * f + 4 * g4 + r;
        const bool ok = j < kend && (a.causal_base < 0 || j <= a.causal_base + qi);
        float v = ok ? s[f][r] * scale : -INFINITY;
        s[f][r] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = (m_new == -INFINITY) ? 1.f : __expf(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float p = (s[f][r] == -INFINITY) ? 0.f : __expf(s[f][r] - m_new);
        s[f][r] = p;
        psum += p;
      }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int df = 0; df < NDF; ++df) o[df] *= alpha;

    if constexpr (BF) {
      // 32-key blocks: k-slot t of lane group g4 <-> key 32kb + 4g4 + t (t<4), 32kb + 16 + 4g4 + t-4.
      // P = P_hi + P_lo, both bf16, so P*V keeps ~16 significant bits of P
      // (a single bf16 P would perturb every output by up to 2^-9 relative).
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        u32x4 pb, pl;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const f32x4& sf = s[2 * kb + q];
          uint32_t hb[4], lb[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bf16 hv = f32_to_bf16(sf[r]);
            hb[r] = hv.v;
            lb[r] = f32_to_bf16(sf[r] - to_f32(hv)).v;
          }
          pb[2 * q] = hb[0] | (hb[1] << 16);
          pb[2 * q + 1] = hb[2] | (hb[3] << 16);
          pl[2 * q] = lb[0] | (lb[1] << 16);
          pl[2 * q + 1] = lb[2] | (lb[3] << 16);
        }
#pragma unroll
        for (int df = 0; df < NDF; ++df) {
          const T* vr = &Vt[(16 * df + c16) * LDV + 32 * kb + 4 * g4];
          u32x2 lo = *(const u32x2*)vr;
          u32x2 hi = *(const u32x2*)(vr + 16);
          u32x4 va = {lo[0], lo[1], hi[0], hi[1]};
          o[df] = mfma16x16x32(va, pb, o[df]);
          o[df] = mfma16x16x32(va, pl, o[df]);
        }
      }
    } else {
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int df = 0; df < NDF; ++df)
            o[df] = mfma16x16x4f32(to_f32(Vt[(16 * df + c16) * LDV + 16 * f + 4 * g4 + r]), s[f][r],
                                   o[df]);
    }
  }

  if (!qvalid) return;
  if (a.splits == 1) {
    const float inv = 1.f / l_run;
    T* out = (T*)a.out + ((long long)(b * a.n + qi) * a.H + h) * DH;
#pragma unroll
    for (int df = 0; df < NDF; ++df)
#pragma unroll
      for (int r = 0; r < 4; ++r) out[16 * df + 4 * g4 + r] = from_f32<T>(o[df][r] * inv);
  } else {
    const long long base = ((long long)blockIdx.z * gridDim.y + bh) * a.n + qi;
    float* po = a.part_o + base * DH;
#pragma unroll
    for (int df = 0; df < NDF; ++df)
#pragma unroll
      for (int r = 0; r < 4; ++r) po[16 * df + 4 * g4 + r] = o[df][r];
    if (g4 == 0) {
      a.part_ml[base * 2 + 0] = m_run;
      a.part_ml[base * 2 + 1] = l_run;
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 path.  Work items (canvas-head bh, key split z, 64-query tile qt) are
// linearised with the query tiles, then the splits of one head adjacent, and
// each XCD (workgroup b runs on XCD b % 8) takes a contiguous run of items:
// the query tiles that share a K/V tile, and the splits that are merged
// together, meet in one L2.
//
// Per key tile (64 keys): K is staged in LDS row-major ([key][dim], the A
// operand of S^T = K Q^T); V is staged transposed ([dim][key], the A operand
// of O^T = V^T P^T), each thread moving a 4-key x 8-dim block (four 16-byte
// loads, eight 8-byte LDS writes).  The next tile's loads are issued before
// the current tile's MFMAs so their latency hides behind the compute.
// With several splits, each workgroup writes an unnormalised partial
// (O, running max, running sum) and a second kernel merges them in split
// order.
template <int DH>
__global__ __launch_bounds__(256) void attn_bf16_kernel(AttnArgs a, int keys_per_split, int n_qt,
                                                        int per_xcd) {
  // row pitches: odd multiples of 32 B keep the fragment reads at full LDS rate
  constexpr int LDKS = DH + 16;  // K row pitch (elements)
  constexpr int LDV = 64 + 16;   // V^T row pitch
  constexpr int NDF = DH / 16;
  constexpr int NQ = DH / 32;
  constexpr int KCH = 64 * DH / 8;            // 16-byte K chunks per tile
  constexpr int KPT = (KCH + 255) / 256;      // per thread
  constexpr int VCH = 16 * (DH / 8);          // 4-key x 8-dim V blocks per tile
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][64 * LDKS];
  __shared__ __attribute__((aligned(16))) bf16 Vt[2][DH * LDV];

  const int total_items = a.B * a.H * a.splits * n_qt;
  const int item = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if ((int)(blockIdx.x >> 3) >= per_xcd || item >= total_items) return;  // uniform
  const int qt = item % n_qt;
  const int z = (item / n_qt) % a.splits;
  const int bh = item / (n_qt * a.splits);
  const int b = bh / a.H, h = bh % a.H;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, c16 = lane & 15;
  const int qi = qt * 64 + wave * 16 + c16;
  const int total = a.len0 + a.len1;
  const int kbeg = z * keys_per_split;
  const int kend = min(total, kbeg + keys_per_split);
  const float scale = 1.0f / sqrtf(float(DH));

  const bf16* K0 = (const bf16*)a.k0 + (long long)bh * a.s0_bh;
  const bf16* V0 = (const bf16*)a.v0 + (long long)bh * a.s0_bh;
  const bf16* K1 = a.len1 ? (const bf16*)a.k1 + (long long)bh * a.s1_bh : K0;
  const bf16* V1 = a.len1 ? (const bf16*)a.v1 + (long long)bh * a.s1_bh : V0;
  // key row j of either segment; rows past the split end are clamped to its
  // last key (their scores are masked to -inf)
  auto krow = [&](int j, const bf16* S0, const bf16* S1) -> const bf16* {
    j = min(j, kend - 1);
    return j < a.len0 ? S0 + (long long)j * DH : S1 + (long long)(j - a.len0) * DH;
  };

  // Q as the B operand of S^T = K Q^T
  const bf16* qrow = (const bf16*)a.q + ((long long)bh * a.n + min(qi, a.n - 1)) * DH;
  u32x4 qf[NQ];
#pragma unroll
  for (int ks = 0; ks < NQ; ++ks) qf[ks] = *(const u32x4*)(qrow + 32 * ks + 8 * g4);

  f32x4 o[NDF];
#pragma unroll
  for (int df = 0; df < NDF; ++df) o[df] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  u32x4 kreg[KPT], vreg[4];
  auto gload = [&](int kt0) {
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int c = tid + u * 256;
      if (c < KCH) {
        const int row = c / (DH / 8), col = (c % (DH / 8)) * 8;
        kreg[u] = *(const u32x4*)(krow(kt0 + row, K0, K1) + col);
      }
    }
    if (tid < VCH) {
      const int kb = tid / (DH / 8), col = (tid % (DH / 8)) * 8;
#pragma unroll
      for (int u = 0; u < 4; ++u) vreg[u] = *(const u32x4*)(krow(kt0 + 4 * kb + u, V0, V1) + col);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int c = tid + u * 256;
      if (c < KCH) {
        const int row = c / (DH / 8), col = (c % (DH / 8)) * 8;
        *(u32x4*)&Ks[buf][row * LDKS + col] = kreg[u];
      }
    }
    if (tid < VCH) {
      const int kb = tid / (DH / 8), col = (tid % (DH / 8)) * 8;
      // dim col+e: keys 4kb..4kb+3 as one 8-byte word
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1, sh = (e & 1) * 16;
        const uint32_t k0 = (vreg[0][w] >> sh) & 0xffffu, k1 = (vreg[1][w] >> sh) & 0xffffu;
        const uint32_t k2 = (vreg[2][w] >> sh) & 0xffffu, k3 = (vreg[3][w] >> sh) & 0xffffu;
        *(u32x2*)&Vt[buf][(col + e) * LDV + 4 * kb] = u32x2{k0 | (k1 << 16), k2 | (k3 << 16)};
      }
    }
  };

  const int ntiles = kend > kbeg ? (kend - kbeg + 63) / 64 : 0;
  if (ntiles) {
    gload(kbeg);
    lstore(0);
  }
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int kt0 = kbeg + 64 * t, buf = t & 1;
    if (t + 1 < ntiles) gload(kt0 + 64);
    // S^T for 64 keys: lane holds keys 16f + 4g4 + r of query qi
    f32x4 sc[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      sc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NQ; ++ks) {
        const u32x4 ka = *(const u32x4*)&Ks[buf][(16 * f + c16) * LDKS + 32 * ks + 8 * g4];
        sc[f] = mfma16x16x32(ka, qf[ks], sc[f]);
      }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = kt0 + 16 * f + 4 * g4 + r;
        const bool ok = j < kend && (a.causal_base < 0 || j <= a.causal_base + qi);
        const float v = ok ? sc[f][r] * scale : -INFINITY;
        sc[f][r] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = (m_new == -INFINITY) ? 1.f : __expf(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = (sc[f][r] == -INFINITY) ? 0.f : __expf(sc[f][r] - m_new);
        sc[f][r] = p;
        psum += p;
      }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int df = 0; df < NDF; ++df) o[df] *= alpha;
    // 32-key blocks: k-slot t of lane group g4 <-> key 32kb + 4g4 + t (t < 4),
    // 32kb + 16 + 4g4 + t - 4.  P = P_hi + P_lo, both bf16, so P V keeps about
    // 16 significant bits of P (one bf16 P perturbs every output by up to 2^-9).
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      u32x4 pb, pl;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const f32x4& sf = sc[2 * kb + q];
        uint32_t hb[4], lb[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bf16 hv = f32_to_bf16(sf[r]);
          hb[r] = hv.v;
          lb[r] = f32_to_bf16(sf[r] - to_f32(hv)).v;
        }
        pb[2 * q] = hb[0] | (hb[1] << 16);
        pb[2 * q + 1] = hb[2] | (hb[3] << 16);
        pl[2 * q] = lb[0] | (lb[1] << 16);
        pl[2 * q + 1] = lb[2] | (lb[3] << 16);
      }
#pragma unroll
      for (int df = 0; df < NDF; ++df) {
        const bf16* vr = &Vt[buf][(16 * df + c16) * LDV + 32 * kb + 4 * g4];
        const u32x2 lo = *(const u32x2*)vr;
        const u32x2 hi = *(const u32x2*)(vr + 16);
        const u32x4 va = {lo[0], lo[1], hi[0], hi[1]};
        o[df] = mfma16x16x32(va, pb, o[df]);
        o[df] = mfma16x16x32(va, pl, o[df]);
      }
    }
    if (t + 1 < ntiles) lstore(buf ^ 1);
    __syncthreads();
  }

  const bool qvalid = qi < a.n;
  if (a.splits == 1) {
    if (qvalid) {
      const float inv = 1.f / l_run;
      bf16* out = (bf16*)a.out + ((long long)(b * a.n + qi) * a.H + h) * DH;
#pragma unroll
      for (int df = 0; df < NDF; ++df) {
        u32x2 w;
        w[0] = uint32_t(f32_to_bf16(o[df][0] * inv).v) | (uint32_t(f32_to_bf16(o[df][1] * inv).v) << 16);
        w[1] = uint32_t(f32_to_bf16(o[df][2] * inv).v) | (uint32_t(f32_to_bf16(o[df][3] * inv).v) << 16);
        *(u32x2*)(out + 16 * df + 4 * g4) = w;
      }
    }
    return;
  }
  // split partial (merged by attn_merge_bf16 in split order)
  if (qvalid) {
    const long long base = ((long long)z * a.B * a.H + bh) * a.n + qi;
    float* po = a.part_o + base * DH;
#pragma unroll
    for (int df = 0; df < NDF; ++df) *(f32x4*)(po + 16 * df + 4 * g4) = o[df];
    if (g4 == 0) *(u32x2*)(a.part_ml + base * 2) = u32x2{__float_as_uint(m_run), __float_as_uint(l_run)};
  }
}

// one thread per (b, h, query, 4 dims): combine the split partials in split order
__global__ __launch_bounds__(256) void attn_merge_bf16(AttnArgs a) {
  const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int q4 = a.dh / 4;
  const long long BH = (long long)a.B * a.H;
  if (e >= BH * a.n * q4) return;
  const int d0 = int(e % q4) * 4;
  const long long row = e / q4;  // (bh, i)
  const int i = int(row % a.n), bh = int(row / a.n);
  float M = -INFINITY;
  for (int z = 0; z < a.splits; ++z) M = fmaxf(M, a.part_ml[((z * BH + bh) * a.n + i) * 2]);
  float L = 0.f;
  f32x4 O = {0.f, 0.f, 0.f, 0.f};
  for (int z = 0; z < a.splits; ++z) {
    const long long base = (z * BH + bh) * a.n + i;
    const float mz = a.part_ml[base * 2];
    if (mz == -INFINITY) continue;
    const float w = __expf(mz - M);
    L += a.part_ml[base * 2 + 1] * w;
    O += *(const f32x4*)(a.part_o + base * a.dh + d0) * w;
  }
  const float inv = 1.f / L;
  const int b = bh / a.H, h = bh % a.H;
  bf16* out = (bf16*)a.out + ((long long)(b * a.n + i) * a.H + h) * a.dh + d0;
  *(u32x2*)out = u32x2{uint32_t(f32_to_bf16(O[0] * inv).v) | (uint32_t(f32_to_bf16(O[1] * inv).v) << 16),
                       uint32_t(f32_to_bf16(O[2] * inv).v) | (uint32_t(f32_to_bf16(O[3] * inv).v) << 16)};
}

// one thread per (b, h, query, d): combine the split partials in split order
template <typename T>
__global__ void attn_merge(AttnArgs a) {
  const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int dh = a.dh;
  const long long total = (long long)a.B * a.H * a.n * dh;
  if (e >= total) return;
  const int d = int(e % dh);
  const long long row = e / dh;  // (bh, i)
  const int i = int(row % a.n);
  const int bh = int(row / a.n);
  const long long BH = (long long)a.B * a.H;
  float M = -INFINITY;
  for (int z = 0; z < a.splits; ++z) M = fmaxf(M, a.part_ml[((z * BH + bh) * a.n + i) * 2]);
  float L = 0.f, O = 0.f;
  for (int z = 0; z < a.splits; ++z) {
    const long long base = (z * BH + bh) * a.n + i;
    const float mz = a.part_ml[base * 2];
    if (mz == -INFINITY) continue;
    const float w = __expf(mz - M);
    L += a.part_ml[base * 2 + 1] * w;
    O += a.part_o[base * dh + d] * w;
  }
  const int b = bh / a.H, h = bh % a.H;
  ((T*)a.out)[((long long)(b * a.n + i) * a.H + h) * dh + d] = from_f32<T>(O / L);
}

template <typename T, int DH>
int launch(const AttnArgs& a, hipStream_t st) {
  const int total = a.len0 + a.len1;
  const int per = ((total + a.splits - 1) / a.splits + KTILE - 1) / KTILE * KTILE;
  dim3 grid((a.n + 63) / 64, a.B * a.H, a.splits);
  hipLaunchKernelGGL((attn_kernel<T, DH>), grid, dim3(256), 0, st, a, per);
  int e = int(hipGetLastError());
  if (e || a.splits == 1) return e;
  const long long n = (long long)a.B * a.H * a.n * a.dh;
  hipLaunchKernelGGL((attn_merge<T>), dim3(unsigned((n + 255) / 256)), dim3(256), 0, st, a);
  return int(hipGetLastError());
}

template <int DH>
int launch_bf16(const AttnArgs& a, hipStream_t st) {
  const int total = a.len0 + a.len1;
  const int per = ((total + a.splits - 1) / a.splits + 63) / 64 * 64;
  const int n_qt = (a.n + 63) / 64;
  const int items = a.B * a.H * a.splits * n_qt;
  const int per_xcd = (items + 7) / 8;
  hipLaunchKernelGGL((attn_bf16_kernel<DH>), dim3(8 * per_xcd), dim3(256), 0, st, a, per, n_qt, per_xcd);
  int e = int(hipGetLastError());
  if (e || a.splits == 1) return e;
  const long long n4 = (long long)a.B * a.H * a.n * (DH / 4);
  hipLaunchKernelGGL(attn_merge_bf16, dim3(unsigned((n4 + 255) / 256)), dim3(256), 0, st, a);
  return int(hipGetLastError());
}

}  // namespace

int attn_splits_for(int B, int H, int n, int keys) {
  const int wgs = ((n + 63) / 64) * B * H;
  int s = 1;
  while (wgs * s < 512 && keys / (s * 2) >= 256) s *= 2;
  return s;
}

int attention(ActType at, const AttnArgs& a, hipStream_t st) {
  if (a.n <= 0) return 0;
  if (at == ACT_BF16) {
    if (a.dh == 128) return launch_bf16<128>(a, st);
    if (a.dh == 64) return launch_bf16<64>(a, st);
    if (a.dh == 32) return launch_bf16<32>(a, st);
  } else {
    if (a.dh == 16) return launch<float, 16>(a, st);
    if (a.dh == 32) return launch<float, 32>(a, st);
    if (a.dh == 64) return launch<float, 64>(a, st);
    if (a.dh == 128) return launch<float, 128>(a, st);
  }
  return int(hipErrorInvalidValue);
}

}  // namespace dg
