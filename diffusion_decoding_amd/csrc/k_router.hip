// MoE routing on gfx950 (zhichai.net 深度拆解, "MoE 效率": 128 fine-grained
// experts plus one shared expert, each token routed to its top 8).
//
// router_topk: one wave per token picks the k largest router logits (ties to
// the lower expert id) and weights them (topk.h).
// router_permute: one workgroup builds the expert histogram, its exclusive
// scan, and the expert-major, token-ascending permutation of the (token, slot)
// pairs from per-expert token bitmasks and popcount prefix sums; the layout is
// deterministic.
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

// One workgroup.  Each expert gets a bitmask over tokens (bit t set when token
// t routes to it), built with LDS OR-atomics -- the result does not depend on
// their order.  Expert e's pairs occupy [off[e], off[e+1]) in token order, so
// the slot of pair (t, j) is off[e] plus the number of earlier tokens in e's
// mask: a per-word prefix plus one popcount.
__global__ __launch_bounds__(PERM_THREADS) void permute_kernel(const int* ids, int T, int E, int k,
                                                               int* off, int* pair_row, int* pos) {
  __shared__ unsigned long long mask[256 * PERM_WORDS];
  __shared__ unsigned short wpre[256 * PERM_WORDS];
  __shared__ int cnt_s[256];
  __shared__ int off_s[257];
  const int tid = threadIdx.x;
  const int W = (T + 63) >> 6;
  const int P = T * k;
  for (int i = tid; i < E * W; i += PERM_THREADS) mask[(i / W) * PERM_WORDS + i % W] = 0ull;
  __syncthreads();
  for (int p = tid; p < P; p += PERM_THREADS) {
    const int t = p / k, e = ids[p];
    atomicOr(&mask[e * PERM_WORDS + (t >> 6)], 1ull << (t & 63));
  }
  __syncthreads();
  // per-expert word prefixes and counts (one thread per expert)
  for (int e = tid; e < E; e += PERM_THREADS) {
    int run = 0;
    for (int w = 0; w < W; ++w) {
      wpre[e * PERM_WORDS + w] = (unsigned short)run;
      run += __popcll(mask[e * PERM_WORDS + w]);
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
  for (int p = tid; p < P; p += PERM_THREADS) {
    const int t = p / k, e = ids[p];
    const unsigned long long below = (1ull << (t & 63)) - 1ull;
    const int slot = off_s[e] + wpre[e * PERM_WORDS + (t >> 6)] +
                     __popcll(mask[e * PERM_WORDS + (t >> 6)] & below);
    pair_row[slot] = t;
    pos[p] = slot;
  }
}

}  // namespace

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

int router_permute(const int* ids, int T, int E, int k, int* off, int* pair_row, int* pos,
                   hipStream_t st) {
  if (T <= 0) return 0;
  if (T > PERM_MAX_TOKENS || E > 256 || k > E) return int(hipErrorInvalidValue);
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(PERM_THREADS), 0, st, ids, T, E, k, off, pair_row,
                     pos);
  return int(hipGetLastError());
}

int expert_counts(const int* off, int E, int* counts, bool accumulate, hipStream_t st) {
  hipLaunchKernelGGL(counts_kernel, dim3((E + 255) / 256), dim3(256), 0, st, off, E, counts, accumulate);
  return int(hipGetLastError());
}

}  // namespace dg
