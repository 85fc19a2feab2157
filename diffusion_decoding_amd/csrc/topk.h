// Router top-k of one token on one wave (zhichai.net 深度拆解, "MoE 效率":
// each token goes to its 8 best of 128 experts), shared by the router's own
// kernel and the shared-down launch that carries it.
//
// Each (logit, expert) pair becomes one 64-bit key that orders by logit, then
// by lower expert id (the low word holds ~id): a total order, so the top k
// are the keys with fewer than k larger keys.  The wave's E keys go to LDS;
// every lane ranks its own keys (KPL of them: E <= 64 KPL) by counting the
// larger ones, reading the keys as wave-wide broadcasts, and the keys ranked
// below k are written to their slot; the weights are a softmax over the k
// picks, summed in rank order (the full router softmax restricted to the
// picks and renormalised).  No cross-lane shuffles.  (A NaN logit is not
// ranked meaningfully; router logits are finite.)
#pragma once
#include "dg_common.h"

namespace dg {

__device__ __forceinline__ unsigned long long topk_key(float f, int e) {
  uint32_t b = __float_as_uint(f);
  b ^= (b >> 31) ? 0xffffffffu : 0x80000000u;  // order-preserving map to unsigned
  return ((unsigned long long)b << 32) | (0xffffffffu - uint32_t(e));
}

__device__ __forceinline__ float topk_value(unsigned long long key) {
  uint32_t b = uint32_t(key >> 32);
  b = (b & 0x80000000u) ? (b ^ 0x80000000u) : ~b;
  return __uint_as_float(b);
}

// Token t's picks into ids / w [t][k].  ks (64 KPL keys) and sel (8 floats)
// are this wave's LDS.  Every wave of the workgroup calls it the same number
// of times (it holds two workgroup barriers); a wave with valid false reads
// and writes nothing in global memory.
template <int KPL>
__device__ __forceinline__ void topk_row(const float* logits, int t, bool valid, int E, int k, int* ids, float* w,
                                         unsigned long long* ks, float* sel) {
  const int lane = threadIdx.x & 63;
  unsigned long long key[KPL];
#pragma unroll
  for (int u = 0; u < KPL; ++u) {
    const int e = lane + 64 * u;
    key[u] = valid && e < E ? topk_key(logits[(long long)t * E + e], e) : 0ull;
    ks[e] = key[u];  // past E: key 0, ranked below every real key
  }
  __syncthreads();
  const int E2 = (E + 1) & ~1;
  int rank[KPL];
#pragma unroll
  for (int u = 0; u < KPL; ++u) rank[u] = 0;
#pragma unroll 8
  for (int e = 0; e < E2; e += 2) {
    const u32x4 kk = *(const u32x4*)&ks[e];
    const unsigned long long k0 = ((unsigned long long)kk[1] << 32) | kk[0];
    const unsigned long long k1 = ((unsigned long long)kk[3] << 32) | kk[2];
#pragma unroll
    for (int u = 0; u < KPL; ++u) rank[u] += int(k0 > key[u]) + int(k1 > key[u]);
  }
#pragma unroll
  for (int u = 0; u < KPL; ++u) {
    const int e = lane + 64 * u;
    if (e < E && rank[u] < k) sel[rank[u]] = topk_value(key[u]);
  }
  __syncthreads();
  if (!valid) return;
  const float m = sel[0];
  float sum = 0.f;
  for (int j = 0; j < k; ++j) sum += __expf(sel[j] - m);
#pragma unroll
  for (int u = 0; u < KPL; ++u) {
    const int e = lane + 64 * u;
    if (e < E && rank[u] < k) {
      ids[t * k + rank[u]] = e;
      w[t * k + rank[u]] = __expf(sel[rank[u]] - m) / sum;
    }
  }
}

}  // namespace dg
