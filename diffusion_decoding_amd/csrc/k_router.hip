// MoE routing on gfx950 (zhichai.net 深度拆解, "MoE 效率": 128 fine-grained
// experts plus one shared expert, each token routed to its top 8).
//
// router_topk: one wave per token picks the k largest router logits (ties to
// the lower expert id) and weights them by a softmax over the k picks, which
// equals the full router softmax restricted to the picks and renormalised.
// router_permute: one workgroup builds the expert histogram, its exclusive
// scan, and the expert-major, token-ascending permutation of the (token, slot)
// pairs with wave ballots and popcount prefix sums -- no atomics, so the
// layout is deterministic.
#include <climits>

#include "dg_common.h"
#include "kernels.h"

namespace dg {
namespace {

__global__ __launch_bounds__(256) void topk_kernel(const float* logits, int T, int E, int k, int* ids,
                                                   float* w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (t >= T) return;
  float v[4];
  bool live[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = lane + 64 * u;
    live[u] = e < E;
    v[u] = live[u] ? logits[(long long)t * E + e] : -INFINITY;
  }
  float top[8];
  int topi[8];
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = INT_MAX;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = lane + 64 * u;
      if (live[u] && (v[u] > bv || (v[u] == bv && e < bi))) {
        bv = v[u];
        bi = e;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    top[j] = bv;
    topi[j] = bi;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (lane + 64 * u == bi) live[u] = false;
  }
  if (lane == 0) {
    float s = 0.f, ex[8];
    for (int j = 0; j < k; ++j) {
      ex[j] = __expf(top[j] - top[0]);
      s += ex[j];
    }
    for (int j = 0; j < k; ++j) {
      ids[t * k + j] = topi[j];
      w[t * k + j] = ex[j] / s;
    }
  }
}

constexpr int PERM_THREADS = 1024;
constexpr int PERM_MAX_PAIRS = 8192;

__global__ __launch_bounds__(PERM_THREADS) void permute_kernel(const int* ids, int T, int E, int k,
                                                               int* off, int* pair_row, int* pos) {
  __shared__ int ids_s[PERM_MAX_PAIRS];
  __shared__ int cnt_s[257];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int NW = PERM_THREADS / 64;
  const int P = T * k;
  for (int i = threadIdx.x; i < P; i += PERM_THREADS) ids_s[i] = ids[i];
  __syncthreads();
  const unsigned long long lt = (1ull << lane) - 1ull;
  for (int e = wave; e < E; e += NW) {
    int c = 0;
    for (int t0 = 0; t0 < T; t0 += 64) {
      const int t = t0 + lane;
      bool mem = false;
      if (t < T)
        for (int j = 0; j < k; ++j) mem |= ids_s[t * k + j] == e;
      c += __popcll(__ballot(mem));
    }
    if (lane == 0) cnt_s[e] = c;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int e = 0; e < E; ++e) {
      const int c = cnt_s[e];
      cnt_s[e] = run;
      off[e] = run;
      run += c;
    }
    cnt_s[E] = run;
    off[E] = run;
  }
  __syncthreads();
  for (int e = wave; e < E; e += NW) {
    int base = cnt_s[e];
    for (int t0 = 0; t0 < T; t0 += 64) {
      const int t = t0 + lane;
      int slot = -1;
      if (t < T)
        for (int j = 0; j < k; ++j)
          if (ids_s[t * k + j] == e) slot = j;
      const unsigned long long mask = __ballot(slot >= 0);
      if (slot >= 0) {
        const int p = base + __popcll(mask & lt);
        pair_row[p] = t;
        pos[t * k + slot] = p;
      }
      base += __popcll(mask);
    }
  }
}

}  // namespace

int router_topk(const float* logits, int T, int E, int k, int* ids, float* w, hipStream_t st) {
  if (T <= 0) return 0;
  if (E > 256 || k > 8 || k > E) return int(hipErrorInvalidValue);
  hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, st, logits, T, E, k, ids, w);
  return int(hipGetLastError());
}

int router_permute(const int* ids, int T, int E, int k, int* off, int* pair_row, int* pos,
                   hipStream_t st) {
  if (T * k > PERM_MAX_PAIRS || E > 256) return int(hipErrorInvalidValue);
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(PERM_THREADS), 0, st, ids, T, E, k, off, pair_row,
                     pos);
  return int(hipGetLastError());
}

}  // namespace dg
