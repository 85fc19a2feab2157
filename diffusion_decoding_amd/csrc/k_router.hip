// MoE routing on gfx950 (zhichai.net 深度拆解, "MoE 效率": 128 fine-grained
// experts plus one shared expert, each token routed to its top 8).
//
// router_topk: one wave per token picks the k largest router logits (ties to
// the lower expert id) and weights them (topk.h).
// router_permute: one workgroup (three launches above 2048 tokens) builds the
// expert histogram, its exclusive scan, and the expert-major, token-ascending
// permutation of the (token, slot) pairs from per-expert token bitmasks and
// popcount prefix sums; the layout is deterministic.
#include <climits>

#include "dg_common.h"
#include "kernels.h"
#include "topk.h"

namespace dg {
namespace {

// One wave per token (topk.h).
template <int KPL>
__global__ __launch_bounds__(64) void topk_kernel(const float* logits, int T, int E, int k, int* ids,
                                                  float* w) {
  __shared__ __attribute__((aligned(16))) unsigned long long ks[64 * KPL];
  __shared__ float sel[8];
  topk_row<KPL>(logits, blockIdx.x, true, E, k, ids, w, ks, sel);
}

// one thread per token: rows with forced[t][0] >= 0 take the forced ids (in
// their slot order) and a softmax over those ids' logits, summed in slot order
__global__ void force_kernel(const float* logits, int T, int E, int k, const int* forced, int* ids, float* w) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T || forced[t * k] < 0) return;
  float sel[8];
  float m = -INFINITY;
  for (int j = 0; j < k; ++j) {
    const int e = min(max(forced[t * k + j], 0), E - 1);
    sel[j] = logits[(long long)t * E + e];
    m = fmaxf(m, sel[j]);
  }
  float sum = 0.f;
  for (int j = 0; j < k; ++j) sum += __expf(sel[j] - m);
  for (int j = 0; j < k; ++j) {
    ids[t * k + j] = min(max(forced[t * k + j], 0), E - 1);
    w[t * k + j] = __expf(sel[j] - m) / sum;
  }
}

__global__ void counts_kernel(const int* off, int E, int* counts, bool accumulate) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e < E) counts[e] = (accumulate ? counts[e] : 0) + off[e + 1] - off[e];
}

constexpr int PERM_THREADS = 1024;
constexpr int PERM_MAX_TOKENS = 2048;
constexpr int PERM_WORDS = PERM_MAX_TOKENS / 64;
// LDS row stride of an expert's words: odd, so that the per-expert prefix
// pass (lane e reads expert e's words) spreads over the banks
constexpr int PERM_STRIDE = PERM_WORDS + 1;

// One workgroup.  Each expert gets a bitmask over tokens (bit t set when token
// t routes to it), built with LDS OR-atomics -- the result does not depend on
// their order.  Expert e's pairs occupy [off[e], off[e+1]) in token order, so
// the slot of pair (t, j) is off[e] plus the number of earlier tokens in e's
// mask: a per-word prefix plus one popcount.
__global__ __launch_bounds__(PERM_THREADS) void permute_kernel(const int* ids, int T, int E, int k,
                                                               int* off, int* pair_row, int* pos) {
  __shared__ unsigned long long mask[256 * PERM_STRIDE];
  __shared__ unsigned short wpre[256 * PERM_STRIDE];
  __shared__ int cnt_s[256];
  __shared__ int off_s[257];
  // pair rows gathered here first when they fit (k <= 8), then written out
  // in order: scattered 4-byte stores from one workgroup were its slowest part
  __shared__ int prow_s[PERM_MAX_TOKENS * 8];
  const int tid = threadIdx.x;
  const int W = (T + 63) >> 6;
  const int P = T * k;
  for (int i = tid; i < E * W; i += PERM_THREADS) mask[(i / W) * PERM_STRIDE + i % W] = 0ull;
  __syncthreads();
  // eight id loads in flight per thread before their atomics (one at a time
  // left each iteration waiting out a global load)
  for (int p0 = tid; p0 < P; p0 += 8 * PERM_THREADS) {
    int ev[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int p = p0 + u * PERM_THREADS;
      ev[u] = p < P ? ids[p] : -1;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int p = p0 + u * PERM_THREADS, t = p / k;
      if (ev[u] >= 0) atomicOr(&mask[ev[u] * PERM_STRIDE + (t >> 6)], 1ull << (t & 63));
    }
  }
  __syncthreads();
  // per-expert word prefixes and counts (one thread per expert)
  for (int e = tid; e < E; e += PERM_THREADS) {
    int run = 0;
    for (int w = 0; w < W; ++w) {
      wpre[e * PERM_STRIDE + w] = (unsigned short)run;
      run += __popcll(mask[e * PERM_STRIDE + w]);
    }
    cnt_s[e] = run;
  }
  __syncthreads();
  // exclusive scan of the counts by wave 0: lane l owns experts 4l .. 4l+3
  if (tid < 64) {
    int c[4], s = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = 4 * tid + u;
      c[u] = e < E ? cnt_s[e] : 0;
      s += c[u];
    }
    int incl = s;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (tid >= o) incl += v;
    }
    int run = incl - s;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = 4 * tid + u;
      if (e < E) off_s[e] = run;
      run += c[u];
    }
    if (tid == 63) off_s[E] = incl;
  }
  __syncthreads();
  for (int e = tid; e <= E; e += PERM_THREADS) off[e] = off_s[e];
  const bool staged = P <= PERM_MAX_TOKENS * 8;  // uniform
  for (int p0 = tid; p0 < P; p0 += 8 * PERM_THREADS) {
    int ev[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int p = p0 + u * PERM_THREADS;
      ev[u] = p < P ? ids[p] : -1;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int p = p0 + u * PERM_THREADS, t = p / k, e = ev[u];
      if (e < 0) continue;
      const unsigned long long below = (1ull << (t & 63)) - 1ull;
      const int slot = off_s[e] + wpre[e * PERM_STRIDE + (t >> 6)] +
                       __popcll(mask[e * PERM_STRIDE + (t >> 6)] & below);
      if (staged) prow_s[slot] = t;
      else pair_row[slot] = t;
      pos[p] = slot;
    }
  }
  if (staged) {
    __syncthreads();
    for (int p = tid; p < P; p += PERM_THREADS) pair_row[p] = prow_s[p];
  }
}

// More tokens than one workgroup's LDS holds (T > PERM_MAX_TOKENS): the same
// layout from three launches.  Each 64-token block writes one token bitmask
// per expert (masks [W][E]); one workgroup turns the masks' popcounts into
// per-block prefixes (wpre [W][E]) and the expert offsets; then each pair
// finds its slot as in the one-workgroup kernel.
__global__ __launch_bounds__(256) void perm_masks_kernel(const int* ids, int T, int E, int k,
                                                         unsigned long long* masks) {
  __shared__ unsigned long long mask[256];
  const int w = blockIdx.x, t0 = 64 * w, tn = min(64, T - t0);
  for (int e = threadIdx.x; e < E; e += 256) mask[e] = 0ull;
  __syncthreads();
  for (int q = threadIdx.x; q < tn * k; q += 256)
    atomicOr(&mask[ids[(long long)t0 * k + q]], 1ull << (q / k));
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) masks[(long long)w * E + e] = mask[e];
}

__global__ __launch_bounds__(256) void perm_scan_kernel(const unsigned long long* masks, int W, int E, int* wpre,
                                                        int* off) {
  __shared__ int cnt_s[256];
  __shared__ int off_s[257];
  const int tid = threadIdx.x;
  int run = 0;
  if (tid < E)
    for (int w = 0; w < W; ++w) {
      wpre[(long long)w * E + tid] = run;
      run += __popcll(masks[(long long)w * E + tid]);
    }
  cnt_s[tid] = run;
  __syncthreads();
  // exclusive scan of the counts by wave 0: lane l owns experts 4l .. 4l+3
  if (tid < 64) {
    int c[4], sum = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      c[u] = cnt_s[4 * tid + u];
      sum += c[u];
    }
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (tid >= o) incl += v;
    }
    int r = incl - sum;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      off_s[4 * tid + u] = r;
      r += c[u];
    }
    if (tid == 63) off_s[256] = incl;
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) off[e] = off_s[e];
  if (tid == 0) off[E] = off_s[256];
}

__global__ __launch_bounds__(256) void perm_scatter_kernel(const int* ids, int T, int E, int k,
                                                           const unsigned long long* masks, const int* wpre,
                                                           const int* off, int* pair_row, int* pos) {
  const long long p = (long long)blockIdx.x * 256 + threadIdx.x;
  if (p >= (long long)T * k) return;
  const int t = int(p / k), e = ids[p];
  const long long we = (long long)(t >> 6) * E + e;
  const int slot = off[e] + wpre[we] + __popcll(masks[we] & ((1ull << (t & 63)) - 1ull));
  pair_row[slot] = t;
  pos[p] = slot;
}

}  // namespace

size_t router_permute_scratch(int T, int E) {
  return T <= PERM_MAX_TOKENS ? 0 : (size_t)((T + 63) / 64) * E * (sizeof(unsigned long long) + sizeof(int));
}

int router_topk(const float* logits, int T, int E, int k, int* ids, float* w, hipStream_t st) {
  if (T <= 0) return 0;
  if (E > 256 || k > 8 || k > E) return int(hipErrorInvalidValue);
  if (E <= 64)
    hipLaunchKernelGGL(topk_kernel<1>, dim3(T), dim3(64), 0, st, logits, T, E, k, ids, w);
  else if (E <= 128)
    hipLaunchKernelGGL(topk_kernel<2>, dim3(T), dim3(64), 0, st, logits, T, E, k, ids, w);
  else
    hipLaunchKernelGGL(topk_kernel<4>, dim3(T), dim3(64), 0, st, logits, T, E, k, ids, w);
  return int(hipGetLastError());
}

int router_force(const float* logits, int T, int E, int k, const int* forced, int* ids, float* w, hipStream_t st) {
  if (T <= 0) return 0;
  if (k > 8 || k > E) return int(hipErrorInvalidValue);
  hipLaunchKernelGGL(force_kernel, dim3((T + 255) / 256), dim3(256), 0, st, logits, T, E, k, forced, ids, w);
  return int(hipGetLastError());
}

int router_permute(const int* ids, int T, int E, int k, int* off, int* pair_row, int* pos, hipStream_t st,
                   void* scratch) {
  if (T <= 0) return 0;
  if (E > 256 || k > E || k > 64) return int(hipErrorInvalidValue);
  if (T <= PERM_MAX_TOKENS) {
    hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(PERM_THREADS), 0, st, ids, T, E, k, off, pair_row, pos);
    return int(hipGetLastError());
  }
  if (!scratch) return int(hipErrorInvalidValue);
  const int W = (T + 63) / 64;
  unsigned long long* masks = (unsigned long long*)scratch;
  int* wpre = (int*)(masks + (size_t)W * E);
  hipLaunchKernelGGL(perm_masks_kernel, dim3(W), dim3(256), 0, st, ids, T, E, k, masks);
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(256), 0, st, masks, W, E, wpre, off);
  const long long P = (long long)T * k;
  hipLaunchKernelGGL(perm_scatter_kernel, dim3(unsigned((P + 255) / 256)), dim3(256), 0, st, ids, T, E, k, masks,
                     wpre, off, pair_row, pos);
  return int(hipGetLastError());
}

int expert_counts(const int* off, int E, int* counts, bool accumulate, hipStream_t st) {
  hipLaunchKernelGGL(counts_kernel, dim3((E + 255) / 256), dim3(256), 0, st, off, E, counts, accumulate);
  return int(hipGetLastError());
}

}  // namespace dg
