// Small kernels of the denoise step: embedding gather, RMSNorm, RoPE + K/V
// scatter, MoE combine, canvas initialisation, entropy-ranked commit with
// re-noise, and Philox draws.
//
// Commit rule (DiffusionGemma解析, "换个路数：整片并行去噪的生成机制": positions are
// ranked by entropy from low to high and the most certain are frozen; ipcmen.com
// "工作原理：并行精炼与自我修正": the most confident tokens are locked and the
// uncertain positions are randomised for the next step).  With U uncommitted
// positions before step s (0-based) of at most S_max, the m = ceil(U/(S_max-s))
// uncommitted positions with the smallest (entropy, index) commit, together
// with every uncommitted position whose entropy is below the threshold; each
// takes its argmax token.  The last allowed step therefore commits everything
// (DiffusionGemma解析, "自适应停步机制": at most 48 steps).  The rest are redrawn
// uniformly (zhichai.net 深度拆解, "统一状态扩散").
#include <cmath>
#include <type_traits>

#include "dg_common.h"
#include "kernels.h"

namespace dg {
namespace {

// A token id outside [0, vocab) reads row 0 instead and raises FLAG_TOKEN, so
// a bad id from the caller never addresses memory past the table.  With tok2
// (self-conditioning) the row of tok2[t] is added, in fp32, rounded once.
__device__ __forceinline__ int embed_id(int id, int vocab, int* flags) {
  if (id < 0 || id >= vocab) {
    if (threadIdx.x == 0 && flags) atomicOr(flags, FLAG_TOKEN);
    id = 0;
  }
  return id;
}
template <typename T>
__global__ void embed_kernel(const int* tok, const int* tok2, int T_, const T* E, int d, int vocab, T* x,
                             int* flags) {
  const int t = blockIdx.x;
  const long long src = (long long)embed_id(tok[t], vocab, flags) * d;
  if (!tok2) {
    for (int c = threadIdx.x; c < d; c += blockDim.x) x[(long long)t * d + c] = E[src + c];
    return;
  }
  const long long src2 = (long long)embed_id(tok2[t], vocab, flags) * d;
  for (int c = threadIdx.x; c < d; c += blockDim.x)
    x[(long long)t * d + c] = from_f32<T>(to_f32(E[src + c]) + to_f32(E[src2 + c]));
}

// FLAG_NONFINITE when any lane of the wave holds a non-finite value (one
// atomic per wave, only then)
__device__ __forceinline__ void flag_nonfinite(bool bad, int* flags) {
  const unsigned long long any = __ballot(bad);
  if (any && flags && (threadIdx.x & 63) == __ffsll((long long)any) - 1) atomicOr(flags, FLAG_NONFINITE);
}
__device__ __forceinline__ bool nonfinite(float v) { return !(fabsf(v) <= 3.402823466e38f); }

// one workgroup (256 threads) per row
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const T* x, int d, float eps, T* y) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  const T* xr = x + (long long)t * d;
  float ss = 0.f;
  for (int c = threadIdx.x; c < d; c += 256) {
    float v = to_f32(xr[c]);
    ss += v * v;
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  ss = red[0] + red[1] + red[2] + red[3];
  const float inv = 1.0f / sqrtf(ss / float(d) + eps);
  T* yr = y + (long long)t * d;
  for (int c = threadIdx.x; c < d; c += 256) yr[c] = from_f32<T>(to_f32(xr[c]) * inv);
}

// bf16 rows with d % 8 == 0 and d <= 8192: one 16-byte chunk of the row per
// thread, loaded once and kept in registers between the sum of squares and
// the scaled write.
// ---------------------------------------------------------------------------
// MXFP8 token rows (OCP MX conversion of a 32-element block: shared exponent
// floor(log2(max |v|)) - 8 as an E8M0 code clamped to [0, 254], an all-zero
// block code 0; each v / 2^shared rounded to E4M3FN, nearest with ties to
// even, magnitudes past 448 clamped to 448).  Every step is exact fp32
// arithmetic on bf16 inputs, so the codes are the format's own.

// E4M3FN code of y (finite).
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const float a = fminf(fabsf(y), 448.f);
  const int e = max(int((__float_as_uint(a) >> 23) & 255u) - 127, -6);  // binade; below 2^-6 the subnormal grid
  const int q = int(rintf(a * __uint_as_float(uint32_t(130 - e) << 23)));  // a / 2^(e - 3): 0 .. 16
  uint32_t code;
  if (e == -6 && q < 8) {
    code = uint32_t(q);
  } else {
    const int carry = q >> 4;  // 16: the next binade's mantissa 0
    code = (uint32_t(e + 7 + carry) << 3) | uint32_t(q - 8 - 8 * carry);
  }
  return code | ((__float_as_uint(y) >> 24) & 0x80u);
}

// Eight consecutive elements of a 32-element block (the lanes l ^ 1 and
// l ^ 2 hold the rest of it) -> their E4M3 codes; *scale gets the block's
// E8M0 code.  Every lane of the wave must call it.
__device__ __forceinline__ u32x2 mx8_piece(const float (&f)[8], uint32_t* scale) {
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
  m = fmaxf(m, __shfl_xor(m, 1, 64));
  m = fmaxf(m, __shfl_xor(m, 2, 64));
  const int code = max(int((__float_as_uint(m) >> 23) & 255u) - 8, 0);
  *scale = uint32_t(code);
  const float inv = __uint_as_float(uint32_t(254 - code) << 23);  // 2^(127 - code), exact
  uint32_t w0 = 0, w1 = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w0 |= e4m3_code(f[i] * inv) << (8 * i);
    w1 |= e4m3_code(f[4 + i] * inv) << (8 * i);
  }
  return u32x2{w0, w1};
}

// one thread per 8 elements of x [T][d] (d % 32 == 0): codes q8 [T][d],
// scales q8s [T][d/32]
__global__ __launch_bounds__(256) void mx8_quantize_kernel(const bf16* x, long long n8, int d, uint8_t* q8,
                                                           uint8_t* q8s) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const bool live = i < n8;  // whole 4-lane groups share it (d / 8 % 4 == 0)
  float f[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (live) {
    const u32x4 q = *(const u32x4*)(x + 8 * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[2 * j] = __uint_as_float(q[j] << 16);
      f[2 * j + 1] = __uint_as_float(q[j] & 0xffff0000u);
    }
  }
  uint32_t sc;
  const u32x2 c = mx8_piece(f, &sc);
  if (live) {
    *(u32x2*)(q8 + 8 * i) = c;
    if ((i & 3) == 0) q8s[i / 4] = (uint8_t)sc;
  }
}

// q8 / q8s non-null: the normed row is also written as MXFP8 codes and scales
// (the bf16 values, quantized as mx8_quantize does).
__global__ __launch_bounds__(1024) void rmsnorm_bf16_kernel(const bf16* x, int d, float eps, bf16* y, uint8_t* q8,
                                                            uint8_t* q8s) {
  __shared__ float red[16];
  const int t = blockIdx.x, tid = threadIdx.x, c = tid * 8;
  const bool live = c < d;
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (live) {
    const u32x4 q = *(const u32x4*)(x + (long long)t * d + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(q[i] << 16);
      v[2 * i + 1] = __uint_as_float(q[i] & 0xffff0000u);
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss += v[i] * v[i];
  ss = wave_sum(ss);
  const int nw = blockDim.x >> 6;
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  ss = 0.f;
  for (int i = 0; i < nw; ++i) ss += red[i];
  const float inv = 1.0f / sqrtf(ss / float(d) + eps);
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(v[2 * i] * inv, v[2 * i + 1] * inv);
  if (live) *(u32x4*)(y + (long long)t * d + c) = o;
  if (q8) {  // uniform; the non-live lanes hold zeros and take part in the block maxima
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = live ? __uint_as_float(o[i] << 16) : 0.f;
      f[2 * i + 1] = live ? __uint_as_float(o[i] & 0xffff0000u) : 0.f;
    }
    uint32_t sc;
    const u32x2 q = mx8_piece(f, &sc);
    if (live) {
      *(u32x2*)(q8 + (long long)t * d + c) = q;
      if ((tid & 3) == 0) q8s[(long long)t * (d / 32) + c / 32] = (uint8_t)sc;
    }
  }
}

// cos/sin of (pos0 + i) * theta^(-2j/dh) for i < n, j < dh/2, evaluated in
// double precision and rounded to binary32 (binary32 angles at positions in
// the thousands would carry ~1e-3 rad of error); theta == 0 gives the
// identity rotation.  tab[i][j] = (cos, sin).  The table depends only on the
// positions, so one step computes it once for all layers.
__global__ void rope_table_kernel(int n, int dh, int pos0, float theta, float2* tab) {
  const int half = dh / 2;
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n * half) return;
  const int j = e % half, i = e / half;
  float c = 1.f, s = 0.f;
  if (theta > 0.f) {
    const double inv = pow((double)theta, -2.0 * j / dh);
    const double ang = (double)(pos0 + i) * inv;
    c = (float)cos(ang);
    s = (float)sin(ang);
  }
  tab[e] = float2{c, s};
}

// The same table for the rows of a mixed batch, each at its segment's
// position (segments passed by value; a row finds its segment by a scan of
// at most MAX_SEGMENTS starts).
__global__ void rope_table_rows_kernel(RowSegments rs, int dh, float theta, float2* tab) {
  const int half = dh / 2;
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= rs.start[rs.n_segs] * half) return;
  const int j = e % half, r = e / half;
  int s = 0;
  while (s + 1 < rs.n_segs && r >= rs.start[s + 1]) ++s;
  float c = 1.f, sn = 0.f;
  if (theta > 0.f) {
    const double inv = pow((double)theta, -2.0 * j / dh);
    const double ang = (double)(rs.pos0[s] + r - rs.start[s]) * inv;
    c = (float)cos(ang);
    sn = (float)sin(ang);
  }
  tab[e] = float2{c, sn};
}

// One thread per 16-byte chunk of a row: dst row0 + i of plane h <- src row i.
__global__ void kv_copy_rows_kernel(const uint8_t* sk, const uint8_t* sv, long long src_bh_b, int H, int n,
                                    int row_b, uint8_t* dk, uint8_t* dv, long long dst_bh_b, int row0) {
  const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int cpr = row_b / 16;
  if (e >= (long long)H * n * cpr) return;
  const int c = int(e % cpr), i = int((e / cpr) % n), h = int(e / ((long long)cpr * n));
  const long long so = h * src_bh_b + (long long)i * row_b + 16 * c;
  const long long d0 = h * dst_bh_b + (long long)(row0 + i) * row_b + 16 * c;
  *(u32x4*)(dk + d0) = *(const u32x4*)(sk + so);
  *(u32x4*)(dv + d0) = *(const u32x4*)(sv + so);
}

// Rotate-half RoPE on q and k (pairs j, j + dh/2) and scatter q, k, v to
// their per-head layouts; one thread per (token, head, 4 consecutive pairs).
template <typename T>
__global__ void rope_kernel(const T* qkv, int B, int n, int H, int dh, const float2* tab, T* q_out, T* kdst,
                            T* vdst, long long dst_bh, int row0) {
  const int half = dh / 2, g4 = half / 4;
  const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long total = (long long)B * n * H * g4;
  if (e >= total) return;
  const int j = int(e % g4) * 4;
  const int h = int((e / g4) % H);
  const int i = int((e / ((long long)g4 * H)) % n);
  const int b = int(e / ((long long)g4 * H * n));
  const int A = H * dh;
  const T* row = qkv + (long long)(b * n + i) * 3 * A;
  float c[4], s[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const float2 cs = tab[i * half + j + u];
    c[u] = cs.x;
    s[u] = cs.y;
  }
  const int bh = b * H + h;
  T* qo = q_out + ((long long)bh * n + i) * dh;
  T* ko = kdst + (long long)bh * dst_bh + (long long)(row0 + i) * dh;
  T* vo = vdst + (long long)bh * dst_bh + (long long)(row0 + i) * dh;
  if constexpr (std::is_same<T, bf16>::value) {
    // 8-byte accesses: four bf16 of each half-row
    auto ld4 = [](const T* p, float* f) {
      const u32x2 w = *(const u32x2*)p;
      f[0] = __uint_as_float(w[0] << 16);
      f[1] = __uint_as_float(w[0] & 0xffff0000u);
      f[2] = __uint_as_float(w[1] << 16);
      f[3] = __uint_as_float(w[1] & 0xffff0000u);
    };
    auto st4 = [](T* p, const float* f) { *(u32x2*)p = u32x2{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3])}; };
    float a1[4], a2[4], o1[4], o2[4];
    ld4(row + h * dh + j, a1);
    ld4(row + h * dh + j + half, a2);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      o1[u] = a1[u] * c[u] - a2[u] * s[u];
      o2[u] = a2[u] * c[u] + a1[u] * s[u];
    }
    st4(qo + j, o1);
    st4(qo + j + half, o2);
    ld4(row + A + h * dh + j, a1);
    ld4(row + A + h * dh + j + half, a2);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      o1[u] = a1[u] * c[u] - a2[u] * s[u];
      o2[u] = a2[u] * c[u] + a1[u] * s[u];
    }
    st4(ko + j, o1);
    st4(ko + j + half, o2);
    *(u32x2*)(vo + j) = *(const u32x2*)(row + 2 * A + h * dh + j);
    *(u32x2*)(vo + j + half) = *(const u32x2*)(row + 2 * A + h * dh + j + half);
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float q1 = to_f32(row[h * dh + j + u]), q2 = to_f32(row[h * dh + j + u + half]);
      qo[j + u] = from_f32<T>(q1 * c[u] - q2 * s[u]);
      qo[j + u + half] = from_f32<T>(q2 * c[u] + q1 * s[u]);
      const float k1 = to_f32(row[A + h * dh + j + u]), k2 = to_f32(row[A + h * dh + j + u + half]);
      ko[j + u] = from_f32<T>(k1 * c[u] - k2 * s[u]);
      ko[j + u + half] = from_f32<T>(k2 * c[u] + k1 * s[u]);
      vo[j + u] = row[2 * A + h * dh + j + u];
      vo[j + u + half] = row[2 * A + h * dh + j + u + half];
    }
  }
}

template <typename T>
__global__ void combine_kernel(T* x, const float* y, const float* ys, const float* w, const int* pos,
                               int k, int d, int* flags) {
  const int t = blockIdx.x;
  bool bad = false;
  for (int c = threadIdx.x; c < d; c += blockDim.x) {
    float acc = 0.f;
    for (int j = 0; j < k; ++j) acc += w[t * k + j] * y[(long long)pos[t * k + j] * d + c];
    acc += ys[(long long)t * d + c];
    T* xp = x + (long long)t * d + c;
    const T r = from_f32<T>(to_f32(*xp) + acc);
    *xp = r;
    bad |= nonfinite(to_f32(r));
  }
  flag_nonfinite(bad, flags);
}

// bf16, d % 4 == 0: grid (T, ceil(d / 1024)), thread -> 4 consecutive columns.
// Same arithmetic order as combine_kernel: experts in slot order, then the
// shared expert, then one rounding of the residual add.
__global__ __launch_bounds__(256) void combine_bf16_kernel(bf16* x, const float* y, const float* ys,
                                                           const float* w, const int* pos, int k, int d,
                                                           int* flags) {
  const int t = blockIdx.x, c = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (c >= d) return;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) acc += w[t * k + j] * *(const f32x4*)(y + (long long)pos[t * k + j] * d + c);
  acc += *(const f32x4*)(ys + (long long)t * d + c);
  bf16* xp = x + (long long)t * d + c;
  const u32x2 xv = *(const u32x2*)xp;
  const float x0 = __uint_as_float(xv[0] << 16), x1 = __uint_as_float(xv[0] & 0xffff0000u);
  const float x2 = __uint_as_float(xv[1] << 16), x3 = __uint_as_float(xv[1] & 0xffff0000u);
  const bf16 r0 = f32_to_bf16(x0 + acc[0]), r1 = f32_to_bf16(x1 + acc[1]);
  const bf16 r2 = f32_to_bf16(x2 + acc[2]), r3 = f32_to_bf16(x3 + acc[3]);
  *(u32x2*)xp = u32x2{uint32_t(r0.v) | (uint32_t(r1.v) << 16), uint32_t(r2.v) | (uint32_t(r3.v) << 16)};
  if (nonfinite(to_f32(r0)) || nonfinite(to_f32(r1)) || nonfinite(to_f32(r2)) || nonfinite(to_f32(r3)))
    atomicOr(flags, FLAG_NONFINITE);
}

// bf16, d % 4 == 0, d <= 4096: one workgroup per token, one thread per 4
// columns (blockDim = d / 4, rounded up to whole waves).
// x[t] = round(x[t] + sum_j w_j y_j + ys) as combine_bf16_kernel (experts in
// slot order, then the shared expert, one rounding), then the next block's
// (or the final) RMSNorm of the rounded row: a[t] = round(x[t] *
// rsqrt(mean x^2 + eps)).
__global__ __launch_bounds__(1024) void combine_norm_bf16_kernel(bf16* x, const float* y, const float* ys,
                                                                 const float* w, const int* pos, int k, int d,
                                                                 float eps, bf16* a, int* flags) {
  __shared__ float red[16];
  const int t = blockIdx.x, tid = threadIdx.x, c = tid * 4;
  const bool live = c < d;
  float xv[4] = {0.f, 0.f, 0.f, 0.f};
  if (live) {
    // all k expert rows in flight at once; slots past k reread slot 0 with weight 0
    f32x4 yv[8];
    float wj[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int jj = j < k ? j : 0;
      wj[j] = j < k ? w[t * k + jj] : 0.f;
      yv[j] = *(const f32x4*)(y + (long long)pos[t * k + jj] * d + c);
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 8; ++j) acc += wj[j] * yv[j];
    acc += *(const f32x4*)(ys + (long long)t * d + c);
    bf16* xp = x + (long long)t * d + c;
    const u32x2 xo = *(const u32x2*)xp;
    const float x0 = __uint_as_float(xo[0] << 16), x1 = __uint_as_float(xo[0] & 0xffff0000u);
    const float x2 = __uint_as_float(xo[1] << 16), x3 = __uint_as_float(xo[1] & 0xffff0000u);
    const bf16 r0 = f32_to_bf16(x0 + acc[0]), r1 = f32_to_bf16(x1 + acc[1]);
    const bf16 r2 = f32_to_bf16(x2 + acc[2]), r3 = f32_to_bf16(x3 + acc[3]);
    *(u32x2*)xp = u32x2{uint32_t(r0.v) | (uint32_t(r1.v) << 16), uint32_t(r2.v) | (uint32_t(r3.v) << 16)};
    xv[0] = to_f32(r0);
    xv[1] = to_f32(r1);
    xv[2] = to_f32(r2);
    xv[3] = to_f32(r3);
  }
  flag_nonfinite(nonfinite(xv[0]) || nonfinite(xv[1]) || nonfinite(xv[2]) || nonfinite(xv[3]), flags);
  float ss = wave_sum(xv[0] * xv[0] + xv[1] * xv[1] + xv[2] * xv[2] + xv[3] * xv[3]);
  const int nw = blockDim.x >> 6;
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  ss = 0.f;
  for (int i = 0; i < nw; ++i) ss += red[i];
  const float inv = 1.0f / sqrtf(ss / float(d) + eps);
  if (live) {
    const bf16 a0 = f32_to_bf16(xv[0] * inv), a1 = f32_to_bf16(xv[1] * inv);
    const bf16 a2 = f32_to_bf16(xv[2] * inv), a3 = f32_to_bf16(xv[3] * inv);
    *(u32x2*)(a + (long long)t * d + c) =
        u32x2{uint32_t(a0.v) | (uint32_t(a1.v) << 16), uint32_t(a2.v) | (uint32_t(a3.v) << 16)};
  }
}

// Pre-committed positions (fill-in-the-middle, constraint puzzles: the known
// tokens are fixed and the rest of the canvas is denoised around them;
// DiffusionGemma深度拆解 (zhichai.net), "代码填充的结构性优势"): position i
// with mask[i] != 0 takes token given[i] and is marked committed, so the
// commit and re-noise steps never touch it.
__global__ void prefill_kernel(int* tok, uint8_t* committed, int n, const int* given, const uint8_t* mask) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n && mask[i]) {
    tok[i] = given[i];
    committed[i] = 1;
  }
}

__global__ void canvas_init_kernel(int* tok, uint8_t* committed, int N, uint64_t seed, uint32_t block,
                                   int vocab, int mask_token) {
  const int b = blockIdx.y;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N) return;
  tok[b * N + i] = mask_token >= 0 ? mask_token
                                   : int(canvas_draw(seed, uint32_t(i), 0u, uint32_t(b), block, uint32_t(vocab)));
  committed[b * N + i] = 0;
}

// (entropy, index) order as one unsigned key: the entropy's bits mapped so
// that unsigned order is numeric order (-0 taken as +0, every NaN after every
// number), the index in the low word.  Committed positions get the largest
// key, so they never rank before an uncommitted one.
__device__ __forceinline__ unsigned long long commit_key(float h, int i) {
  const uint32_t b = __float_as_uint(h + 0.0f);
  const uint32_t u = (h != h) ? 0xffffffffu : ((b >> 31) ? ~b : (b | 0x80000000u));
  return ((unsigned long long)u << 32) | uint32_t(i);
}

// One workgroup of 1024 threads per canvas; N <= 1024.  Positions are padded
// to whole waves (NR) and each gets 1024 / NR threads, which split the count
// of the keys ranked before it.
// The status word: workgroup 0 copies the flags the step's kernels raised
// (live) to `published` and clears them for the next step; every kernel that
// raises a flag ran before this one on the stream.  An argmax outside the
// vocabulary (a row whose logits were all non-finite, already flagged)
// commits id 0.
__global__ __launch_bounds__(1024) void commit_kernel(const float* H, const int* am, int* tok,
                                                      uint8_t* committed, int N, int step,
                                                      int max_steps, float threshold, uint64_t seed,
                                                      uint32_t block, int vocab, int mask_token,
                                                      int* n_unc, int* live, int* published) {
  __shared__ unsigned long long ks[1024];
  __shared__ int part_s[1024];
  __shared__ int red[16];
  const int b = blockIdx.x, t = threadIdx.x;
  const int NR = (N + 63) & ~63, parts = 1024 / NR;
  const int i = t % NR, q = t / NR;
  const int base = b * N;
  const bool own = q == 0 && i < N;  // the thread that owns position i
  const bool unc = own && committed[base + i] == 0;
  const float hi = own ? H[base + i] : 0.f;
  if (q == 0) ks[i] = unc ? commit_key(hi, i) : ~0ull;
  // U = number of uncommitted positions
  int cnt = wave_sum_i(unc ? 1 : 0);
  if ((t & 63) == 0) red[t >> 6] = cnt;
  __syncthreads();
  int U = 0;
  for (int w = 0; w < 16; ++w) U += red[w];
  const int m = U ? (U + (max_steps - step) - 1) / (max_steps - step) : 0;
  int before = 0;
  if (q < parts && i < N) {
    const unsigned long long mine = ks[i];
    const int len = (N + parts - 1) / parts, j0 = q * len, j1 = min(N, j0 + len);
    for (int j = j0; j < j1; ++j) before += ks[j] < mine ? 1 : 0;
  }
  part_s[t] = before;
  __syncthreads();
  bool take = false;
  if (unc) {
    int tot = 0;
    for (int p = 0; p < parts; ++p) tot += part_s[p * NR + i];
    take = tot < m || hi < threshold;
  }
  if (take) {
    const int a = am[base + i];
    tok[base + i] = (a >= 0 && a < vocab) ? a : 0;
    committed[base + i] = 1;
  }
  const bool still = unc && !take;
  int c2 = wave_sum_i(still ? 1 : 0);
  if ((t & 63) == 0) red[t >> 6] = c2;
  __syncthreads();
  if (still)
    tok[base + i] = mask_token >= 0 ? mask_token
                                    : int(canvas_draw(seed, uint32_t(i), uint32_t(step + 1), uint32_t(b), block,
                                                      uint32_t(vocab)));
  if (t == 0) {
    int Up = 0;
    for (int w = 0; w < 16; ++w) Up += red[w];
    n_unc[b] = Up;
    if (b == 0 && live) {
      if (published) *published = *live;
      *live = 0;
    }
  }
}

__global__ void status_publish_kernel(int* live, int* published) {
  *published = *live;
  *live = 0;
}

__global__ void philox_kernel(uint64_t seed, uint32_t pos0, uint32_t tag, uint32_t canvas,
                              uint32_t block, uint32_t modulus, int n, uint32_t* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  out[i] = canvas_draw(seed, pos0 + uint32_t(i), tag, canvas, block, modulus);
}

}  // namespace

int embed_gather(ActType at, const int* tok, int T, const void* E, int d, int vocab, void* x, int* flags,
                 hipStream_t st, const int* tok2) {
  if (T <= 0) return 0;
  if (at == ACT_BF16)
    hipLaunchKernelGGL(embed_kernel<bf16>, dim3(T), dim3(256), 0, st, tok, tok2, T, (const bf16*)E, d, vocab,
                       (bf16*)x, flags);
  else
    hipLaunchKernelGGL(embed_kernel<float>, dim3(T), dim3(256), 0, st, tok, tok2, T, (const float*)E, d, vocab,
                       (float*)x, flags);
  return int(hipGetLastError());
}

int mx8_quantize(const void* x, int T, int d, uint8_t* q8, uint8_t* q8s, hipStream_t st) {
  if (T <= 0) return 0;
  if (d % 32) return int(hipErrorInvalidValue);
  const long long n8 = (long long)T * d / 8;
  hipLaunchKernelGGL(mx8_quantize_kernel, dim3(unsigned((n8 + 255) / 256)), dim3(256), 0, st, (const bf16*)x, n8,
                     d, q8, q8s);
  return int(hipGetLastError());
}

int rmsnorm(ActType at, const void* x, int T, int d, float eps, void* y, hipStream_t st, uint8_t* q8,
            uint8_t* q8s) {
  if (T <= 0) return 0;
  if (q8 && (at != ACT_BF16 || d % 32 || d > 8192)) return int(hipErrorInvalidValue);
  if (at == ACT_BF16)
  {
    if (d % 8 == 0 && d <= 8192) {
      const int threads = ((d / 8 + 63) / 64) * 64;
      hipLaunchKernelGGL(rmsnorm_bf16_kernel, dim3(T), dim3(threads), 0, st, (const bf16*)x, d, eps, (bf16*)y,
                         q8, q8s);
    } else {
      hipLaunchKernelGGL(rmsnorm_kernel<bf16>, dim3(T), dim3(256), 0, st, (const bf16*)x, d, eps, (bf16*)y);
    }
  }
  else
    hipLaunchKernelGGL(rmsnorm_kernel<float>, dim3(T), dim3(256), 0, st, (const float*)x, d, eps, (float*)y);
  return int(hipGetLastError());
}

int rope_table(int n, int dh, int pos0, float theta, float* tab, hipStream_t st) {
  const int total = n * (dh / 2);
  if (total <= 0) return 0;
  hipLaunchKernelGGL(rope_table_kernel, dim3((total + 255) / 256), dim3(256), 0, st, n, dh, pos0, theta,
                     (float2*)tab);
  return int(hipGetLastError());
}

int rope_table_rows(const RowSegments& rs, int dh, float theta, float* tab, hipStream_t st) {
  if (rs.n_segs <= 0 || rs.n_segs > MAX_SEGMENTS) return int(hipErrorInvalidValue);
  const int total = rs.start[rs.n_segs] * (dh / 2);
  if (total <= 0) return 0;
  hipLaunchKernelGGL(rope_table_rows_kernel, dim3((total + 255) / 256), dim3(256), 0, st, rs, dh, theta,
                     (float2*)tab);
  return int(hipGetLastError());
}

int kv_copy_rows(ActType at, const void* src_k, const void* src_v, long long src_bh, int H, int n, int dh,
                 void* dst_k, void* dst_v, long long dst_bh, int row0, hipStream_t st) {
  const int es = at == ACT_BF16 ? 2 : 4, row_b = dh * es;
  if (row_b % 16) return int(hipErrorInvalidValue);
  const long long total = (long long)H * n * (row_b / 16);
  if (total <= 0) return 0;
  hipLaunchKernelGGL(kv_copy_rows_kernel, dim3(unsigned((total + 255) / 256)), dim3(256), 0, st,
                     (const uint8_t*)src_k, (const uint8_t*)src_v, src_bh * es, H, n, row_b, (uint8_t*)dst_k,
                     (uint8_t*)dst_v, dst_bh * es, row0);
  return int(hipGetLastError());
}

int rope_scatter(ActType at, const void* qkv, int B, int n, int H, int dh, const float* tab, void* q_out,
                 void* kdst, void* vdst, long long dst_bh, int row0, hipStream_t st) {
  if (dh % 8) return int(hipErrorInvalidValue);
  const long long total = (long long)B * n * H * (dh / 8);
  if (total <= 0) return 0;
  dim3 grid(unsigned((total + 255) / 256));
  if (at == ACT_BF16)
    hipLaunchKernelGGL(rope_kernel<bf16>, grid, dim3(256), 0, st, (const bf16*)qkv, B, n, H, dh,
                       (const float2*)tab, (bf16*)q_out, (bf16*)kdst, (bf16*)vdst, dst_bh, row0);
  else
    hipLaunchKernelGGL(rope_kernel<float>, grid, dim3(256), 0, st, (const float*)qkv, B, n, H, dh,
                       (const float2*)tab, (float*)q_out, (float*)kdst, (float*)vdst, dst_bh, row0);
  return int(hipGetLastError());
}

int moe_combine(ActType at, void* x, const float* y, const float* ys, const float* w, const int* pos,
                int T, int k, int d, int* flags, hipStream_t st) {
  if (T <= 0) return 0;
  if (!flags) return int(hipErrorInvalidValue);
  if (at == ACT_BF16 && d % 4 == 0)
    hipLaunchKernelGGL(combine_bf16_kernel, dim3(T, (d + 1023) / 1024), dim3(256), 0, st, (bf16*)x, y, ys, w,
                       pos, k, d, flags);
  else if (at == ACT_BF16)
    hipLaunchKernelGGL(combine_kernel<bf16>, dim3(T), dim3(256), 0, st, (bf16*)x, y, ys, w, pos, k, d, flags);
  else
    hipLaunchKernelGGL(combine_kernel<float>, dim3(T), dim3(256), 0, st, (float*)x, y, ys, w, pos, k, d, flags);
  return int(hipGetLastError());
}

int moe_combine_norm(ActType at, void* x, const float* y, const float* ys, const float* w, const int* pos,
                     int T, int k, int d, float eps, void* a, int* flags, hipStream_t st) {
  if (T <= 0) return 0;
  if (at == ACT_BF16 && d % 4 == 0 && d <= 4096 && k <= 8) {
    const int threads = ((d / 4 + 63) / 64) * 64;
    hipLaunchKernelGGL(combine_norm_bf16_kernel, dim3(T), dim3(threads), 0, st, (bf16*)x, y, ys, w, pos, k, d,
                       eps, (bf16*)a, flags);
    return int(hipGetLastError());
  }
  int e = moe_combine(at, x, y, ys, w, pos, T, k, d, flags, st);
  if (e) return e;
  return rmsnorm(at, x, T, d, eps, a, st);
}

int canvas_init(int* tok, uint8_t* committed, int B, int N, uint64_t seed, uint32_t block, int vocab,
                int mask_token, hipStream_t st) {
  hipLaunchKernelGGL(canvas_init_kernel, dim3((N + 255) / 256, B), dim3(256), 0, st, tok, committed, N,
                     seed, block, vocab, mask_token);
  return int(hipGetLastError());
}

int canvas_prefill(int* tok, uint8_t* committed, int n, const int* given, const uint8_t* mask, hipStream_t st) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(prefill_kernel, dim3((n + 255) / 256), dim3(256), 0, st, tok, committed, n, given, mask);
  return int(hipGetLastError());
}

int commit_renoise(const float* H, const int* am, int* tok, uint8_t* committed, int B, int N, int step,
                   int max_steps, float threshold, uint64_t seed, uint32_t block, int vocab, int mask_token,
                   int* n_unc, int* live_flags, int* status, hipStream_t st) {
  if (N > 1024) return int(hipErrorInvalidValue);
  hipLaunchKernelGGL(commit_kernel, dim3(B), dim3(1024), 0, st, H, am, tok, committed, N, step,
                     max_steps, threshold, seed, block, vocab, mask_token, n_unc, live_flags, status);
  return int(hipGetLastError());
}

int status_publish(int* live, int* published, hipStream_t st) {
  hipLaunchKernelGGL(status_publish_kernel, dim3(1), dim3(1), 0, st, live, published);
  return int(hipGetLastError());
}

int philox_fill(uint64_t seed, uint32_t pos0, uint32_t tag, uint32_t canvas, uint32_t block,
                uint32_t modulus, int n, uint32_t* out, hipStream_t st) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(philox_kernel, dim3((n + 255) / 256), dim3(256), 0, st, seed, pos0, tag, canvas,
                     block, modulus, n, out);
  return int(hipGetLastError());
}

}  // namespace dg
