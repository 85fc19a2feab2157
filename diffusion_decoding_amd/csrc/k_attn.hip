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
// Most bf16 problems take a second kernel with 32-query waves on the
// 32x32x16 MFMA, in 256-query workgroups (long key ranges, batched canvases)
// or 128-query ones (one canvas over a long enough prompt), which stage each
// K/V tile once for four or two times the queries.
#include <algorithm>
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

  const T* qrow = (const T*)a.q + (long long)bh * a.q_bh + (long long)min(qi, a.n - 1) * DH;
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
// bf16 path.  Work items (canvas-head bh, key split z, query tile qt of
// 16 NW queries, one 16-query block per wave) are
// linearised with the query tiles, then the splits of one head adjacent, and
// each XCD (workgroup b runs on XCD b % 8) takes a contiguous run of items:
// the query tiles that share a K/V tile, and the splits that are merged
// together, meet in one L2.
//
// Per key tile (64 keys): K is staged in LDS row-major ([key][dim], the A
// operand of S^T = K Q^T); V is staged transposed ([dim][key], the A operand
// of O^T = V^T P^T), each thread moving a 4-key x 8-dim block (four 16-byte
// loads, eight 8-byte LDS writes).  A register ring keeps the loads of the
// next D key tiles in flight while a tile is computed; all loads are
// unconditional (rows past the split end are clamped to its last key and
// masked to -inf) and the main loop has no branches, so the compiler waits
// for exactly the oldest tile.
// With several splits, each workgroup writes an unnormalised partial
// (O, running max, running sum) and a second kernel merges them in split
// order.
template <int DH, int D, bool SEG, int NW>
__device__ __forceinline__ void attn_bf16_item(const AttnArgs& a, int item, int keys_per_split, int n_qt) {
  // K row pitch: an odd multiple of 32 B keeps the 16-row x 64-byte fragment
  // reads at full LDS rate.  V^T row pitch 72 elements (36 dwords): the
  // 16-byte fragment reads of 16 rows land on 16 distinct 4-bank groups, and
  // in the transposing writes the two 16-lane row groups of a half-wave sit
  // 32 banks apart (8 rows x 36 dwords = 32 mod 64), so neither side
  // conflicts.
  constexpr int LDKS = DH + 16;  // K row pitch (elements)
  constexpr int LDV = 64 + 8;    // V^T row pitch
  constexpr int NDF = DH / 16;
  constexpr int NQ = DH / 32;
  constexpr int NT = 64 * NW;                 // threads
  constexpr int KCH = 64 * DH / 8;            // 16-byte K chunks per tile
  constexpr int KPT = KCH / NT;               // per thread
  // V blocks of 4 keys x VD dims: 8 dims (16-byte loads) with four waves,
  // 4 dims (8-byte loads) with eight, so every thread moves one block
  constexpr int VD = NW == 8 ? 4 : 8;
  constexpr int VCH = 16 * (DH / VD);         // V blocks per tile
  static_assert(KCH % NT == 0 && VCH <= NT && NT % VCH == 0, "tile split");
  using vchunk = typename std::conditional<VD == 8, u32x4, u32x2>::type;
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][64 * LDKS];
  __shared__ __attribute__((aligned(16))) bf16 Vt[2][DH * LDV];

  const int qt = item % n_qt;
  const int z = (item / n_qt) % a.splits;
  const int bh = item / (n_qt * a.splits);
  const int b = bh / a.H, h = bh % a.H;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, c16 = lane & 15;
  const int qi = qt * 16 * NW + wave * 16 + c16;
  const int total = a.len0 + a.len1;
  const int kbeg = z * keys_per_split;
  const int kend = min(total, kbeg + keys_per_split);

  // Keys and values come from two segments (the cache rows, then the canvas
  // rows).  SEG (one segment, or a cache length that is a multiple of 64, so
  // no key tile spans both): each tile is read through a buffer resource built on the scalar
  // unit for its segment, starting at the tile and ending with the segment.
  // Otherwise each segment has one resource covering exactly its rows: a row
  // is loaded from both at 32-bit offsets, the segment that does not hold it
  // returns zeros (its offset is past the end, or negative and so past the
  // end as unsigned), and the two results are OR-ed.  Rows past the split end
  // are other splits' keys (or zeros past the last key); their scores are
  // masked to -inf, so their values meet p = 0.
  constexpr int RB = DH * 2;  // bytes per row
  const __amdgpu_buffer_rsrc_t rk0 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const bf16*)a.k0 + (long long)bh * a.s0_bh), (short)0, a.len0 * RB, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv0 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const bf16*)a.v0 + (long long)bh * a.s0_bh), (short)0, a.len0 * RB, 0x00020000);
  const __amdgpu_buffer_rsrc_t rk1 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.len1 ? (const bf16*)a.k1 + (long long)bh * a.s1_bh : (const bf16*)a.k0), (short)0, a.len1 * RB,
      0x00020000);
  const __amdgpu_buffer_rsrc_t rv1 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.len1 ? (const bf16*)a.v1 + (long long)bh * a.s1_bh : (const bf16*)a.v0), (short)0, a.len1 * RB,
      0x00020000);

  // Q as the B operand of S^T = K Q^T
  const bf16* qrow = (const bf16*)a.q + (long long)bh * a.q_bh + (long long)min(qi, a.n - 1) * DH;
  u32x4 qf[NQ];
#pragma unroll
  for (int ks = 0; ks < NQ; ++ks) qf[ks] = *(const u32x4*)(qrow + 32 * ks + 8 * g4);

  f32x4 o[NDF];
#pragma unroll
  for (int df = 0; df < NDF; ++df) o[df] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int ntiles = kend > kbeg ? (kend - kbeg + 63) / 64 : 0;
  // this thread's V block: 4-key block vkb (fastest over the lanes, so 16
  // lanes write one contiguous 128-byte piece of a V^T row), dims
  // vcol .. vcol + VD - 1.  With 4-dim blocks the four 16-lane groups of a
  // wave take dims +0, +8, +4, +12, so the two groups of a half-wave write
  // rows 8 apart (32 banks) as with 8-dim blocks.  Threads past VCH repeat a
  // block: same loads, same values stored to the same LDS words.
  const int vb = tid % VCH, vkb = vb % 16, vg = vb / 16;
  const int vcol = VD == 8 ? vg * 8 : (vg >> 2) * 16 + (vg & 1) * 8 + ((vg >> 1) & 1) * 4;
  // this thread's byte offsets inside a key tile
  int koff[KPT], voff[4];
#pragma unroll
  for (int p = 0; p < KPT; ++p) {
    const int c = tid + p * NT;
    koff[p] = (c / (DH / 8)) * RB + (c % (DH / 8)) * 16;
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) voff[p] = (4 * vkb + p) * RB + vcol * 2;
  u32x4 kreg[D][KPT];
  vchunk vreg[D][4];
  auto vload = [&](__amdgpu_buffer_rsrc_t r, int off) -> vchunk {
    if constexpr (VD == 8) return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    else return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  };
  auto gload = [&](int t, int u) {
    const int kt0 = kbeg + 64 * min(t, ntiles - 1);
    if constexpr (SEG) {
      const bool s1 = kt0 >= a.len0;  // uniform
      const int r0 = s1 ? kt0 - a.len0 : kt0, rows = s1 ? a.len1 - r0 : a.len0 - r0;
      const bf16* kb = s1 ? (const bf16*)a.k1 + (long long)bh * a.s1_bh : (const bf16*)a.k0 + (long long)bh * a.s0_bh;
      const bf16* vb = s1 ? (const bf16*)a.v1 + (long long)bh * a.s1_bh : (const bf16*)a.v0 + (long long)bh * a.s0_bh;
      const __amdgpu_buffer_rsrc_t rk =
          __builtin_amdgcn_make_buffer_rsrc((void*)(kb + (long long)r0 * DH), (short)0, rows * RB, 0x00020000);
      const __amdgpu_buffer_rsrc_t rv =
          __builtin_amdgcn_make_buffer_rsrc((void*)(vb + (long long)r0 * DH), (short)0, rows * RB, 0x00020000);
#pragma unroll
      for (int p = 0; p < KPT; ++p) kreg[u][p] = __builtin_amdgcn_raw_buffer_load_b128(rk, koff[p], 0, 0);
#pragma unroll
      for (int p = 0; p < 4; ++p) vreg[u][p] = vload(rv, voff[p]);
      return;
    }
    const int b0 = kt0 * RB, b1 = (kt0 - a.len0) * RB;  // tile start in each segment
#pragma unroll
    for (int p = 0; p < KPT; ++p)
      kreg[u][p] = __builtin_amdgcn_raw_buffer_load_b128(rk0, koff[p] + b0, 0, 0) |
                   __builtin_amdgcn_raw_buffer_load_b128(rk1, koff[p] + b1, 0, 0);
#pragma unroll
    for (int p = 0; p < 4; ++p)
      vreg[u][p] = vload(rv0, voff[p] + b0) | vload(rv1, voff[p] + b1);
  };
  // V^T position of this thread's four keys: inside each 32-key block the
  // keys are stored in the order the P.V MFMA consumes them (lane group g
  // takes keys 4g..4g+3 and 16+4g..16+4g+3), so a fragment is one 16-byte read
  const int vpos = 32 * (vkb >> 3) + 8 * (vkb & 3) + 4 * ((vkb >> 2) & 1);
  auto lstore = [&](int buf, int u) {
#pragma unroll
    for (int p = 0; p < KPT; ++p) {
      const int c = tid + p * NT;
      const int row = c / (DH / 8), col = (c % (DH / 8)) * 8;
      *(u32x4*)&Ks[buf][row * LDKS + col] = kreg[u][p];
    }
    // dim vcol+e: keys 4vkb..4vkb+3 as one 8-byte word at their V^T position
#pragma unroll
    for (int e = 0; e < VD; ++e) {
      const int w = e >> 1, sh = (e & 1) * 16;
      const uint32_t k0 = (vreg[u][0][w] >> sh) & 0xffffu, k1 = (vreg[u][1][w] >> sh) & 0xffffu;
      const uint32_t k2 = (vreg[u][2][w] >> sh) & 0xffffu, k3 = (vreg[u][3][w] >> sh) & 0xffffu;
      *(u32x2*)&Vt[buf][(vcol + e) * LDV + vpos] = u32x2{k0 | (k1 << 16), k2 | (k3 << 16)};
    }
  };

  // Softmax in the log2 domain: scores scaled by log2(e)/sqrt(dh), p = 2^(s - m).
  const float sl = 1.4426950408889634f / sqrtf(float(DH));
  // key limit of this lane's query: the split end, or the causal bound
  const int klim = a.causal_base < 0 ? kend : min(kend, a.causal_base + qi + 1);

  // One key tile t from LDS buffer t & 1; ring slot u held tile t and is
  // refilled with tile t + D; slot u + 1 (tile t + 1) goes to the other buffer.
  // MASKED: some key of the tile may lie past klim (the split's last tile, or
  // any tile of a causal pass); then a running max can still be -inf and the
  // exponent base is taken as 0 so that no -inf - -inf arises.
  auto tile = [&](int t, int u, bool store_next, auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    gload(t + D, u);
    const int kt0 = kbeg + 64 * t, buf = t & 1;
    // S^T for 64 keys: lane holds keys 16f + 4g4 + r of query qi.  Every K
    // fragment is read before the first MFMA (the scheduling barriers keep
    // the compiler from interleaving one read and one MFMA at a time, which
    // exposes the LDS latency per MFMA); the V fragments are read right after
    // the S MFMAs and arrive while the softmax runs.
    u32x4 ka[4][NQ];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int ks = 0; ks < NQ; ++ks) ka[f][ks] = *(const u32x4*)&Ks[buf][(16 * f + c16) * LDKS + 32 * ks + 8 * g4];
    __builtin_amdgcn_sched_barrier(0);
    f32x4 sc[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      sc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NQ; ++ks) sc[f] = mfma16x16x32(ka[f][ks], qf[ks], sc[f]);
    }
    __builtin_amdgcn_sched_barrier(0);
    u32x4 va[2][NDF];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int df = 0; df < NDF; ++df) va[kb][df] = *(const u32x4*)&Vt[buf][(16 * df + c16) * LDV + 32 * kb + 8 * g4];
    __builtin_amdgcn_sched_barrier(0);
    // this lane's largest raw score (the scale sl is positive, so it keeps the order)
    float tmax = -INFINITY;
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (MASKED) sc[f][r] = (kt0 + 16 * f + 4 * g4 + r < klim) ? sc[f][r] : -INFINITY;
        tmax = fmaxf(tmax, sc[f][r]);
      }
    tmax *= sl;
    // The exponent base m_run (per query, equal in its four lanes) is raised
    // only when some score of the query exceeds it by more than 2^8 (or it is
    // still -inf), so O and l are rescaled rarely; p stays below 2^8 and the
    // result O / l is unchanged.  The query's maximum over its four lanes is
    // formed only when some lane of the wave sees such a score.
    // v_exp_f32 directly: p below 2^-126 flushes to 0, far below what the sum
    // can resolve.
    // (A lane whose scores are all masked so far keeps m_run = -inf; its
    // exponent base is then 0 and every p of it is exp2(-inf) = 0.)
    if (__any(tmax > m_run + 8.f)) {  // uniform over the wave
      float tq = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tq = fmaxf(tq, __shfl_xor(tq, 32, 64));
      const float m_new = tq > m_run + 8.f ? tq : m_run;
      const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int df = 0; df < NDF; ++df) o[df] *= alpha;
      m_run = m_new;
    }
    float m_base = m_run;
    if constexpr (MASKED) m_base = (m_run == -INFINITY) ? 0.f : m_run;
    // p = 2^(s sl - m) in one fused step; l_run holds this lane's keys only
    // (the four lanes of a query are summed once, at the end)
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[f][r], sl, -m_base));
        sc[f][r] = p;
        l_run += p;
      }
    // 32-key blocks: k-slot t of lane group g4 <-> key 32kb + 4g4 + t (t < 4),
    // 32kb + 16 + 4g4 + t - 4.  P = P_hi + P_lo, both bf16, so P V keeps about
    // 16 significant bits of P (one bf16 P perturbs every output by up to 2^-9).
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      u32x4 pb, pl;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const f32x4& sf = sc[2 * kb + q];
        const uint32_t h01 = pack_bf16x2(sf[0], sf[1]), h23 = pack_bf16x2(sf[2], sf[3]);
        pb[2 * q] = h01;
        pb[2 * q + 1] = h23;
        pl[2 * q] = pack_bf16x2(sf[0] - __uint_as_float(h01 << 16), sf[1] - __uint_as_float(h01 & 0xffff0000u));
        pl[2 * q + 1] = pack_bf16x2(sf[2] - __uint_as_float(h23 << 16), sf[3] - __uint_as_float(h23 & 0xffff0000u));
      }
#pragma unroll
      for (int df = 0; df < NDF; ++df) {
        o[df] = mfma16x16x32(va[kb][df], pb, o[df]);
        o[df] = mfma16x16x32(va[kb][df], pl, o[df]);
      }
    }
    if (store_next) lstore(buf ^ 1, (u + 1) % D);
    __syncthreads();
  };
  using Full = std::integral_constant<bool, false>;
  using Masked = std::integral_constant<bool, true>;

  if (ntiles) {  // uniform over the workgroup
#pragma unroll
    for (int s = 0; s < D; ++s) gload(s, s);
    lstore(0, 0);
    __syncthreads();
    // every tile but the last lies wholly inside the split; only a causal
    // pass masks inside the main loop
    int t0 = 0;
    if (a.causal_base < 0) {
      for (; t0 + D < ntiles; t0 += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) tile(t0 + u, u, true, Full{});
      }
    } else {
      for (; t0 + D < ntiles; t0 += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) tile(t0 + u, u, true, Masked{});
      }
    }
#pragma unroll
    for (int u = 0; u < D; ++u)
      if (t0 + u < ntiles) tile(t0 + u, u, t0 + u + 1 < ntiles, Masked{});
  }

  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  const bool qvalid = qi < a.n;
  if (a.splits == 1) {
    if (qvalid) {
      const float inv = 1.f / l_run;
      bf16* out = (bf16*)a.out + ((long long)(b * a.n + qi) * a.H + h) * DH;
#pragma unroll
      for (int df = 0; df < NDF; ++df) {
        *(u32x2*)(out + 16 * df + 4 * g4) =
            u32x2{pack_bf16x2(o[df][0] * inv, o[df][1] * inv), pack_bf16x2(o[df][2] * inv, o[df][3] * inv)};
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

// ---------------------------------------------------------------------------
// bf16 path with 32-query waves (head_dim 64 or 128).  The same work items
// (query tiles, key splits, XCD order) and key tiles as above, but each wave
// holds 32 queries and computes with the 32x32x16 MFMA: S^T (32 keys x 32
// queries per block) = K Q^T, O^T (32 dims x 32 queries per block) =
// V^T P^T.  A K or V fragment read from LDS then feeds 32 queries instead of
// 16, and NWQ waves (eight in use: 256-query tiles) share each K/V tile
// staged in LDS, so a tile's L2-to-LDS traffic serves four times the queries
// of a 64-query tile.
//
// Layouts of the 32x32x16 MFMA (lane l, half hh = l / 32): an operand lane
// supplies row or column l % 32 and k-slots 8 hh .. 8 hh + 7; a result lane
// holds column l % 32 and, in register 4 b + r, row 8 b + 4 hh + r.  A lane
// of S^T thus holds query l % 32 and keys 8 b + 4 hh + r of a 32-key block.
// As the B operand of the 16-key step c of that block (keys 16 c .. 16 c +
// 15), its registers 8 c .. 8 c + 7 are already in k-slot order when k-slot
// s stands for key 16 c + 8 (s / 4) + 4 hh + s % 4; V^T is stored with the
// keys of every 16-key group in that order (key 8 q + 4 hh + r of the group
// at position 8 hh + 4 q + r), so a V^T fragment is one 16-byte read.
typedef __attribute__((ext_vector_type(16))) float f32x16;

__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

template <int DH, bool SEG, int NWQ>
__device__ __forceinline__ void attn32_item(const AttnArgs& a, int item, int keys_per_split, int n_qt) {
  constexpr int NT = 64 * NWQ;
  constexpr int QTILE = 32 * NWQ;
  // K row pitch DH + 8 elements (68 dwords at dh 128, 36 at 64): the 16-byte
  // fragment reads of 16 consecutive rows land on 16 distinct 4-bank groups.
  // V^T row pitch 72 elements, as in the 16-query kernel.
  constexpr int LDKS = DH + 8;
  constexpr int LDV = 64 + 8;
  constexpr int NKS = DH / 16;  // 16-dim steps of S
  constexpr int NDB = DH / 32;  // 32-dim blocks of O^T
  constexpr int KCH = 64 * DH / 8;
  constexpr int KPT = KCH / NT;
  // V blocks of 4 keys x VD dims: 8 dims (16-byte loads) with four waves,
  // 4 dims (8-byte loads) with eight, so every thread moves one block
  constexpr int VD = NWQ == 8 ? 4 : 8;
  constexpr int VCH = 16 * (DH / VD);
  static_assert(KCH % NT == 0 && VCH <= NT && NT % VCH == 0, "tile split");
  using vchunk = typename std::conditional<VD == 8, u32x4, u32x2>::type;
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][64 * LDKS];
  __shared__ __attribute__((aligned(16))) bf16 Vt[2][DH * LDV];

  const int qt = item % n_qt;
  const int z = (item / n_qt) % a.splits;
  const int bh = item / (n_qt * a.splits);
  const int b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, c32 = lane & 31;
  const int qi = qt * QTILE + wave * 32 + c32;
  const int total = a.len0 + a.len1;
  const int kbeg = z * keys_per_split;
  const int kend = min(total, kbeg + keys_per_split);

  // key/value rows through buffer resources, as in the 16-query kernel
  constexpr int RB = DH * 2;
  const __amdgpu_buffer_rsrc_t rk0 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const bf16*)a.k0 + (long long)bh * a.s0_bh), (short)0, a.len0 * RB, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv0 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const bf16*)a.v0 + (long long)bh * a.s0_bh), (short)0, a.len0 * RB, 0x00020000);
  const __amdgpu_buffer_rsrc_t rk1 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.len1 ? (const bf16*)a.k1 + (long long)bh * a.s1_bh : (const bf16*)a.k0), (short)0, a.len1 * RB,
      0x00020000);
  const __amdgpu_buffer_rsrc_t rv1 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.len1 ? (const bf16*)a.v1 + (long long)bh * a.s1_bh : (const bf16*)a.v0), (short)0, a.len1 * RB,
      0x00020000);

  // Q as the B operand of S^T = K Q^T: query qi, dims 16 ks + 8 hh .. + 7
  const bf16* qrow = (const bf16*)a.q + (long long)bh * a.q_bh + (long long)min(qi, a.n - 1) * DH;
  u32x4 qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) qf[ks] = *(const u32x4*)(qrow + 16 * ks + 8 * hh);

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int ntiles = kend > kbeg ? (kend - kbeg + 63) / 64 : 0;
  // this thread's V block: keys 4 vkb .. 4 vkb + 3 (vkb fastest over the
  // lanes), dims vcol .. vcol + VD - 1 (with 4-dim blocks the four 16-lane
  // groups of a wave take dims +0, +8, +4, +12, as in the 16-query kernel);
  // threads past VCH repeat a block
  const int vb = tid % VCH, vkb = vb % 16, vg = vb / 16;
  const int vcol = VD == 8 ? vg * 8 : (vg >> 2) * 16 + (vg & 1) * 8 + ((vg >> 1) & 1) * 4;
  int koff[KPT], voff[4];
#pragma unroll
  for (int p = 0; p < KPT; ++p) {
    const int c = tid + p * NT;
    koff[p] = (c / (DH / 8)) * RB + (c % (DH / 8)) * 16;
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) voff[p] = (4 * vkb + p) * RB + vcol * 2;
  u32x4 kreg[KPT];
  vchunk vreg[4];
  auto vload = [&](__amdgpu_buffer_rsrc_t r, int off) -> vchunk {
    if constexpr (VD == 8) return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    else return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  };
  auto gload = [&](int t) {
    const int kt0 = kbeg + 64 * min(t, ntiles - 1);
    if constexpr (SEG) {
      const bool s1 = kt0 >= a.len0;  // uniform
      const int r0 = s1 ? kt0 - a.len0 : kt0, rows = s1 ? a.len1 - r0 : a.len0 - r0;
      const bf16* kb = s1 ? (const bf16*)a.k1 + (long long)bh * a.s1_bh : (const bf16*)a.k0 + (long long)bh * a.s0_bh;
      const bf16* vbp = s1 ? (const bf16*)a.v1 + (long long)bh * a.s1_bh : (const bf16*)a.v0 + (long long)bh * a.s0_bh;
      const __amdgpu_buffer_rsrc_t rk =
          __builtin_amdgcn_make_buffer_rsrc((void*)(kb + (long long)r0 * DH), (short)0, rows * RB, 0x00020000);
      const __amdgpu_buffer_rsrc_t rv =
          __builtin_amdgcn_make_buffer_rsrc((void*)(vbp + (long long)r0 * DH), (short)0, rows * RB, 0x00020000);
#pragma unroll
      for (int p = 0; p < KPT; ++p) kreg[p] = __builtin_amdgcn_raw_buffer_load_b128(rk, koff[p], 0, 0);
#pragma unroll
      for (int p = 0; p < 4; ++p) vreg[p] = vload(rv, voff[p]);
      return;
    }
    const int b0 = kt0 * RB, b1 = (kt0 - a.len0) * RB;
#pragma unroll
    for (int p = 0; p < KPT; ++p)
      kreg[p] = __builtin_amdgcn_raw_buffer_load_b128(rk0, koff[p] + b0, 0, 0) |
                __builtin_amdgcn_raw_buffer_load_b128(rk1, koff[p] + b1, 0, 0);
#pragma unroll
    for (int p = 0; p < 4; ++p)
      vreg[p] = vload(rv0, voff[p] + b0) | vload(rv1, voff[p] + b1);
  };
  // V^T position of this thread's four keys (16-key groups in k-slot order)
  const int vpos = 16 * (vkb >> 2) + 8 * (vkb & 1) + 4 * ((vkb >> 1) & 1);
  auto lstore = [&](int buf) {
#pragma unroll
    for (int p = 0; p < KPT; ++p) {
      const int c = tid + p * NT;
      const int row = c / (DH / 8), col = (c % (DH / 8)) * 8;
      *(u32x4*)&Ks[buf][row * LDKS + col] = kreg[p];
    }
#pragma unroll
    for (int e = 0; e < VD; ++e) {
      const int w = e >> 1, sh = (e & 1) * 16;
      const uint32_t k0 = (vreg[0][w] >> sh) & 0xffffu, k1 = (vreg[1][w] >> sh) & 0xffffu;
      const uint32_t k2 = (vreg[2][w] >> sh) & 0xffffu, k3 = (vreg[3][w] >> sh) & 0xffffu;
      *(u32x2*)&Vt[buf][(vcol + e) * LDV + vpos] = u32x2{k0 | (k1 << 16), k2 | (k3 << 16)};
    }
  };

  const float sl = 1.4426950408889634f / sqrtf(float(DH));
  const int klim = a.causal_base < 0 ? kend : min(kend, a.causal_base + qi + 1);

  // one key tile t from LDS buffer t & 1; the loads of tile t + 1 are in
  // flight meanwhile and go to the other buffer at the end
  auto tile = [&](int t, bool store_next, auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    gload(t + 1);
    const int kt0 = kbeg + 64 * t, buf = t & 1;
    f32x16 sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      u32x4 ka[NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) ka[ks] = *(const u32x4*)&Ks[buf][(32 * kb + c32) * LDKS + 16 * ks + 8 * hh];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[kb][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) sc[kb] = mfma32x32x16(ka[ks], qf[ks], sc[kb]);
    }
    __builtin_amdgcn_sched_barrier(0);
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if constexpr (MASKED)
          sc[kb][i] = (kt0 + 32 * kb + 8 * (i >> 2) + 4 * hh + (i & 3) < klim) ? sc[kb][i] : -INFINITY;
        tmax = fmaxf(tmax, sc[kb][i]);
      }
    tmax *= sl;
    // lazy rescaling as in the 16-query kernel; a query's two lanes (halves)
    // hold the same m_run
    if (__any(tmax > m_run + 8.f)) {
      const float tq = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float m_new = tq > m_run + 8.f ? tq : m_run;
      const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] *= alpha;
      m_run = m_new;
    }
    float m_base = m_run;
    if constexpr (MASKED) m_base = (m_run == -INFINITY) ? 0.f : m_run;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][i], sl, -m_base));
        sc[kb][i] = p;
        l_run += p;
      }
    // P = P_hi + P_lo (both bf16) against V^T, one 16-key step at a time
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int kb = c >> 1, i0 = 8 * (c & 1);
      u32x4 pb, pl;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float x0 = sc[kb][i0 + 2 * q], x1 = sc[kb][i0 + 2 * q + 1];
        const uint32_t hi = pack_bf16x2(x0, x1);
        pb[q] = hi;
        pl[q] = pack_bf16x2(x0 - __uint_as_float(hi << 16), x1 - __uint_as_float(hi & 0xffff0000u));
      }
      u32x4 va[NDB];
#pragma unroll
      for (int db = 0; db < NDB; ++db) va[db] = *(const u32x4*)&Vt[buf][(32 * db + c32) * LDV + 16 * c + 8 * hh];
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        o[db] = mfma32x32x16(va[db], pb, o[db]);
        o[db] = mfma32x32x16(va[db], pl, o[db]);
      }
    }
    if (store_next) lstore(buf ^ 1);
    __syncthreads();
  };
  using Full = std::integral_constant<bool, false>;
  using Masked = std::integral_constant<bool, true>;

  if (ntiles) {  // uniform over the workgroup
    gload(0);
    lstore(0);
    __syncthreads();
    int t = 0;
    if (a.causal_base < 0) {
      for (; t + 1 < ntiles; ++t) tile(t, true, Full{});
    } else {
      for (; t + 1 < ntiles; ++t) tile(t, true, Masked{});
    }
    tile(t, false, Masked{});
  }

  l_run += __shfl_xor(l_run, 32, 64);
  if (qi >= a.n) return;
  // lane: query qi, dims 32 db + 8 bb + 4 hh + r in register 4 bb + r of o[db]
  if (a.splits == 1) {
    const float inv = 1.f / l_run;
    bf16* out = (bf16*)a.out + ((long long)(b * a.n + qi) * a.H + h) * DH;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int bb = 0; bb < 4; ++bb)
        *(u32x2*)(out + 32 * db + 8 * bb + 4 * hh) =
            u32x2{pack_bf16x2(o[db][4 * bb] * inv, o[db][4 * bb + 1] * inv),
                  pack_bf16x2(o[db][4 * bb + 2] * inv, o[db][4 * bb + 3] * inv)};
    return;
  }
  const long long base = ((long long)z * a.B * a.H + bh) * a.n + qi;
  float* po = a.part_o + base * DH;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int bb = 0; bb < 4; ++bb)
      *(f32x4*)(po + 32 * db + 8 * bb + 4 * hh) =
          f32x4{o[db][4 * bb], o[db][4 * bb + 1], o[db][4 * bb + 2], o[db][4 * bb + 3]};
  if (hh == 0) *(u32x2*)(a.part_ml + base * 2) = u32x2{__float_as_uint(m_run), __float_as_uint(l_run)};
}

template <int DH, bool SEG, int NWQ>
__global__ __launch_bounds__(64 * NWQ) __attribute__((amdgpu_waves_per_eu(2))) void attn32_kernel(
    AttnArgs a, int keys_per_split, int n_qt, int per_xcd) {
  const int total_items = a.B * a.H * a.splits * n_qt;
  const int item = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if ((int)(blockIdx.x >> 3) >= per_xcd || item >= total_items) return;  // uniform
  attn32_item<DH, SEG, NWQ>(a, item, keys_per_split, n_qt);
}

// One attention problem per launch: work items by XCD as above.
template <int DH, int D, bool SEG, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2))) void attn_bf16_kernel(
    AttnArgs a, int keys_per_split, int n_qt, int per_xcd) {
  const int total_items = a.B * a.H * a.splits * n_qt;
  const int item = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if ((int)(blockIdx.x >> 3) >= per_xcd || item >= total_items) return;  // uniform
  attn_bf16_item<DH, D, SEG, NW>(a, item, keys_per_split, n_qt);
}

// Several problems in one launch (the requests of a mixed batch, each with
// its own queries, cache, mode and key splits): their work items are
// numbered one problem after another, so an XCD's contiguous run of items
// still covers query tiles and splits of the same problem.
struct AttnTable {
  AttnArgs seg[ATTN_MAX_SEGS];
  int item0[ATTN_MAX_SEGS + 1];  // first work item of each problem; item0[n] = all items
  int kps[ATTN_MAX_SEGS];        // keys per split
  int n_qt[ATTN_MAX_SEGS];       // query tiles
  int blk0[ATTN_MAX_SEGS + 1];   // first merge workgroup of each problem (none with one split)
  int n;
};

template <int DH, int D, bool SEG, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2))) void attn_bf16_segs_kernel(
    AttnTable t, int per_xcd) {
  const int item = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if ((int)(blockIdx.x >> 3) >= per_xcd || item >= t.item0[t.n]) return;  // uniform
  int i = 0;
  while (i + 1 < t.n && item >= t.item0[i + 1]) ++i;  // uniform; problems with no items are passed over
  attn_bf16_item<DH, D, SEG, NW>(t.seg[i], item - t.item0[i], t.kps[i], t.n_qt[i]);
}

// one thread per (b, h, query, 4 dims): combine the S split partials in split
// order.  Partial maxima are in the log2 domain of the bf16 kernel.  S is a
// compile-time count, so every partial's loads are issued before the first is
// used.
template <int S>
__device__ __forceinline__ void merge_bf16_item(const AttnArgs& a, long long e) {
  const int q4 = a.dh / 4;
  const long long BH = (long long)a.B * a.H;
  if (e >= BH * a.n * q4) return;
  const int d0 = int(e % q4) * 4;
  const long long row = e / q4;  // (bh, i)
  const int i = int(row % a.n), bh = int(row / a.n);
  const long long zstride = BH * a.n;  // rows between splits
  const long long base0 = (long long)bh * a.n + i;
  u32x2 ml[S];
  f32x4 po[S];
#pragma unroll
  for (int z = 0; z < S; ++z) {
    const long long base = base0 + z * zstride;
    ml[z] = *(const u32x2*)(a.part_ml + base * 2);
    po[z] = *(const f32x4*)(a.part_o + base * a.dh + d0);
  }
  float M = -INFINITY;
#pragma unroll
  for (int z = 0; z < S; ++z) M = fmaxf(M, __uint_as_float(ml[z][0]));
  float L = 0.f;
  f32x4 O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int z = 0; z < S; ++z) {
    const float w = __builtin_amdgcn_exp2f(__uint_as_float(ml[z][0]) - M);  // an empty split (max -inf) weighs 0
    L += __uint_as_float(ml[z][1]) * w;
    O += po[z] * w;
  }
  const float inv = 1.f / L;
  const int b = bh / a.H, h = bh % a.H;
  bf16* out = (bf16*)a.out + ((long long)(b * a.n + i) * a.H + h) * a.dh + d0;
  *(u32x2*)out = u32x2{pack_bf16x2(O[0] * inv, O[1] * inv), pack_bf16x2(O[2] * inv, O[3] * inv)};
}

template <int S>
__global__ __launch_bounds__(256) void attn_merge_bf16(AttnArgs a) {
  merge_bf16_item<S>(a, (long long)blockIdx.x * blockDim.x + threadIdx.x);
}

// the merges of every problem of a table with more than one split, one
// launch; each workgroup belongs to one problem
__global__ __launch_bounds__(256) void attn_merge_bf16_segs(AttnTable t) {
  const int blk = blockIdx.x;
  int i = 0;
  while (i + 1 < t.n && blk >= t.blk0[i + 1]) ++i;  // uniform
  const AttnArgs& a = t.seg[i];
  const long long e = (long long)(blk - t.blk0[i]) * 256 + threadIdx.x;
  switch (a.splits) {
    case 2: merge_bf16_item<2>(a, e); break;
    case 4: merge_bf16_item<4>(a, e); break;
    case 8: merge_bf16_item<8>(a, e); break;
    case 16: merge_bf16_item<16>(a, e); break;
    default: break;
  }
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

// bf16 kernel shape, as queries per workgroup tile: 256 (eight 32-query
// waves; each K/V tile staged in LDS serves four times the queries of a
// 64-query tile) for long key ranges or many canvas-heads; 128 (four 32-query
// waves) when a grid of one workgroup per CU still leaves every key split 256
// keys or more; else 64 (four 16-query waves).  Measured, attention + merge
// per layer: 4 and 8 canvases x 256 queries x 8448 keys 109 and 197 us with
// 256-query tiles against 121 and 216 (eight 16-query waves per 128-query
// tile) and 117 and 211 (128-query tiles); at 2304 keys, per step, 4 / 8 /
// 16 / 32 canvases 1.50 / 2.30 / 3.61 / 6.87 ms against 1.60 / 2.51 / 4.80 /
// 8.99 ms for 64-query tiles.  One canvas x 2304 keys (8 splits of 288 keys)
// 16.3 + 4.6 us against 18.1 + 4.1 with 64-query tiles (4 splits) and 21.6 +
// 4.6 with 256-query tiles; one 512-query canvas x 2560 keys 25.0 + 4.5
// against 27.1 + 4.5; one canvas x 1280 keys keeps 64-query tiles (4 splits:
// 13.9 + 4.2 us against 14.4 + 5.1 for 128-query tiles over 8 splits).
int attn_tile_queries(int B, int H, int n, int keys, int dh) {
  if (dh < 64 || n < 128) return 64;
  if (keys >= 4096 || B * H >= 64) return 256;
  const int wgs = ((n + 127) / 128) * B * H;
  int s = 1;
  while (s < 8 && wgs * s < 256) s *= 2;
  return keys / s >= 256 ? 128 : 64;
}
int attn_tile_waves(int tile_queries) { return tile_queries == 256 ? 8 : 4; }

template <int DH, int NWQ>
int launch_bf16_q32(const AttnArgs& a, hipStream_t st) {
  const int total = a.len0 + a.len1;
  const int per = ((total + a.splits - 1) / a.splits + 63) / 64 * 64;
  const int n_qt = (a.n + 32 * NWQ - 1) / (32 * NWQ);
  const int items = a.B * a.H * a.splits * n_qt;
  const int per_xcd = (items + 7) / 8;
  if (a.len1 == 0 || a.len0 % 64 == 0)  // no key tile spans both segments
    hipLaunchKernelGGL((attn32_kernel<DH, true, NWQ>), dim3(8 * per_xcd), dim3(64 * NWQ), 0, st, a, per, n_qt,
                       per_xcd);
  else
    hipLaunchKernelGGL((attn32_kernel<DH, false, NWQ>), dim3(8 * per_xcd), dim3(64 * NWQ), 0, st, a, per, n_qt,
                       per_xcd);
  return int(hipGetLastError());
}

// 64-query tiles of four 16-query waves, one K/V tile in flight (two would
// spill at four waves)
template <int DH>
int launch_bf16_q16(const AttnArgs& a, hipStream_t st) {
  constexpr int NW = 4;
  const int total = a.len0 + a.len1;
  const int per = ((total + a.splits - 1) / a.splits + 63) / 64 * 64;
  const int n_qt = (a.n + 16 * NW - 1) / (16 * NW);
  const int items = a.B * a.H * a.splits * n_qt;
  const int per_xcd = (items + 7) / 8;
  if (a.len1 == 0 || a.len0 % 64 == 0)  // no key tile spans both segments
    hipLaunchKernelGGL((attn_bf16_kernel<DH, 1, true, NW>), dim3(8 * per_xcd), dim3(64 * NW), 0, st, a, per, n_qt,
                       per_xcd);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<DH, 1, false, NW>), dim3(8 * per_xcd), dim3(64 * NW), 0, st, a, per, n_qt,
                       per_xcd);
  return int(hipGetLastError());
}

template <int DH>
int launch_bf16(const AttnArgs& a, hipStream_t st) {
  int e;
  if constexpr (DH >= 64)
    switch (attn_tile_queries(a.B, a.H, a.n, a.len0 + a.len1, DH)) {
      case 256: e = launch_bf16_q32<DH, 8>(a, st); break;
      case 128: e = launch_bf16_q32<DH, 4>(a, st); break;
      default: e = launch_bf16_q16<DH>(a, st);
    }
  else
    e = launch_bf16_q16<DH>(a, st);
  if (e || a.splits == 1) return e;
  const long long n4 = (long long)a.B * a.H * a.n * (DH / 4);
  const dim3 g(unsigned((n4 + 255) / 256));
  switch (a.splits) {
    case 2: hipLaunchKernelGGL(attn_merge_bf16<2>, g, dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL(attn_merge_bf16<4>, g, dim3(256), 0, st, a); break;
    case 8: hipLaunchKernelGGL(attn_merge_bf16<8>, g, dim3(256), 0, st, a); break;
    case 16: hipLaunchKernelGGL(attn_merge_bf16<16>, g, dim3(256), 0, st, a); break;
    default: return int(hipErrorInvalidValue);
  }
  return int(hipGetLastError());
}

}  // namespace

// Key splits (bf16): double while the grid is under one workgroup per CU and
// each split keeps at least 128 keys, or under 2048 waves (two four-wave or
// one eight-wave workgroup per CU) and each split keeps at least 512 keys
// (shorter splits lose more to the merge and to each workgroup's first tile
// than they gain in parallelism; one canvas x 1280 keys: 4 splits 13.9 + 4.2
// us, 2 splits 19.5 + 4.2).  The fp32 kernel keeps the second rule alone.
int attn_splits_for(ActType at, int B, int H, int n, int keys, int dh) {
  if (at != ACT_BF16) {
    const bool wide = dh >= 64 && n >= 128 && (keys >= 4096 || B * H >= 64);
    const int wgs = ((n + (wide ? 255 : 63)) / (wide ? 256 : 64)) * B * H;
    int s = 1;
    while (s < 16 && wgs * s * (wide ? 8 : 4) < 2048 && keys / (s * 2) >= 512) s *= 2;
    return s;
  }
  const int qt = attn_tile_queries(B, H, n, keys, dh);
  const int wgs = ((n + qt - 1) / qt) * B * H, waves = attn_tile_waves(qt);
  int s = 1;
  while (s < 16 && ((wgs * s < 256 && keys / (s * 2) >= 128) || (wgs * s * waves < 2048 && keys / (s * 2) >= 512)))
    s *= 2;
  return s;
}

// Several problems in one launch (bf16).  Key splits: every problem starts
// at one and all double together, as for a single problem, while the whole
// grid is under 2048 waves and the problem keeps at least 512 keys per split
// (at most max_splits).  Four-wave tiles throughout.  Partials are packed one
// problem after another from part_o / part_ml (at most max_splits x the
// problems' rows, as for one problem of all the rows).
int attention_segments(ActType at, AttnArgs* segs, int n, int max_splits, float* part_o, float* part_ml,
                       hipStream_t st) {
  if (at != ACT_BF16 || n <= 0 || n > ATTN_MAX_SEGS) return int(hipErrorInvalidValue);
  const int dh = segs[0].dh;
  if (dh != 32 && dh != 64 && dh != 128) return int(hipErrorInvalidValue);
  constexpr int NW = 4;
  AttnTable t{};
  t.n = n;
  int wgs[ATTN_MAX_SEGS], keys[ATTN_MAX_SEGS];
  bool seg_tiles = true;  // no key tile of any problem spans its two key segments
  for (int i = 0; i < n; ++i) {
    AttnArgs& a = segs[i];
    if (a.dh != dh || a.n < 0 || a.q_bh < (long long)a.n * a.dh) return int(hipErrorInvalidValue);
    keys[i] = a.len0 + a.len1;
    t.n_qt[i] = (a.n + 16 * NW - 1) / (16 * NW);
    wgs[i] = a.n > 0 ? t.n_qt[i] * a.B * a.H : 0;
    a.splits = 1;
    seg_tiles = seg_tiles && (a.len1 == 0 || a.len0 % 64 == 0);
  }
  for (;;) {
    long long waves = 0;
    for (int i = 0; i < n; ++i) waves += (long long)wgs[i] * segs[i].splits * NW;
    if (waves >= 2048) break;
    bool grew = false;
    for (int i = 0; i < n; ++i)
      if (wgs[i] && segs[i].splits < std::min(16, max_splits) && keys[i] / (segs[i].splits * 2) >= 512) {
        segs[i].splits *= 2;
        grew = true;
      }
    if (!grew) break;
  }
  long long po = 0, ml = 0;
  t.item0[0] = t.blk0[0] = 0;
  for (int i = 0; i < n; ++i) {
    AttnArgs& a = segs[i];
    a.part_o = part_o + po;
    a.part_ml = part_ml + ml;
    const long long rows = (long long)a.B * a.H * a.n;
    if (a.splits > 1) {
      po += a.splits * rows * dh;
      ml += a.splits * rows * 2;
    }
    t.seg[i] = a;
    t.kps[i] = ((keys[i] + a.splits - 1) / a.splits + 63) / 64 * 64;
    t.item0[i + 1] = t.item0[i] + wgs[i] * a.splits;
    t.blk0[i + 1] = t.blk0[i] + (a.splits > 1 ? int((rows * (dh / 4) + 255) / 256) : 0);
  }
  if (t.item0[n] == 0) return 0;
  const int per_xcd = (t.item0[n] + 7) / 8;
  const dim3 grid(8 * per_xcd), block(64 * NW);
#define DG_ATTN_SEGS(DH_)                                                                    \
  if (seg_tiles)                                                                            \
    hipLaunchKernelGGL((attn_bf16_segs_kernel<DH_, 1, true, NW>), grid, block, 0, st, t, per_xcd);  \
  else                                                                                      \
    hipLaunchKernelGGL((attn_bf16_segs_kernel<DH_, 1, false, NW>), grid, block, 0, st, t, per_xcd);
  if (dh == 128) {
    DG_ATTN_SEGS(128)
  } else if (dh == 64) {
    DG_ATTN_SEGS(64)
  } else {
    DG_ATTN_SEGS(32)
  }
#undef DG_ATTN_SEGS
  int e = int(hipGetLastError());
  if (e || t.blk0[n] == 0) return e;
  hipLaunchKernelGGL(attn_merge_bf16_segs, dim3(t.blk0[n]), dim3(256), 0, st, t);
  return int(hipGetLastError());
}

int attention(ActType at, const AttnArgs& a, hipStream_t st) {
  if (a.n <= 0) return 0;
  if (a.q_bh < (long long)a.n * a.dh) return int(hipErrorInvalidValue);
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
