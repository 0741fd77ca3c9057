// Token grouping by expert.
//
// Routed expert e receives the (token, k) pairs with topk_idx[t][k] == e, kept
// in (t, k) order; shared experts receive every token with weight 1. Grouped
// entries of expert e occupy positions offsets[e] .. offsets[e+1]-1; inv maps
// each (t, slot) back to its position (slot k < K routed, K + s shared). The
// scan is ballot-ordered, not atomic, so the grouping is the same every run.
#include "mpb_device.h"
#include "mpb_internal.h"

namespace mpb {

__global__ __launch_bounds__(256) void k_count(const int32_t* __restrict__ idx, int TK,
                                               int32_t* __restrict__ counts) {
  __shared__ int part[4];
  const int e = blockIdx.x;
  int c = 0;
  for (int j = threadIdx.x; j < TK; j += 256) c += (idx[j] == e);
  for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) counts[e] = part[0] + part[1] + part[2] + part[3];
}

__global__ __launch_bounds__(256) void k_scatter(FfnParams p) {
  __shared__ int s_off;
  __shared__ int wtot[4];
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int T = p.T, K = p.K, S = p.S, E = p.E, KS = K + S;
  if (tid == 0) {
    int off = 0;
    for (int j = 0; j < e; ++j) off += j < E ? p.counts[j] : T;
    s_off = off;
    p.offsets[e] = off;
    const int mine = e < E ? p.counts[e] : T;
    if (e == p.NB - 1) p.offsets[p.NB] = off + mine;
    if (e >= E) p.counts[e] = T;
  }
  __syncthreads();
  const int off = s_off;
  if (e < E) {
    const int TK = T * K;
    int run = 0;
    for (int base = 0; base < TK; base += 256) {
      const int j = base + tid;
      const bool m = j < TK && p.topk_idx[j] == e;
      const unsigned long long bal = __ballot(m);
      const int lp = __popcll(bal & ((1ull << lane) - 1ull));
      if (lane == 0) wtot[w] = __popcll(bal);
      __syncthreads();
      int wp = 0;
      for (int v = 0; v < w; ++v) wp += wtot[v];
      const int tot = wtot[0] + wtot[1] + wtot[2] + wtot[3];
      if (m) {
        const int pos = off + run + wp + lp;
        const int t = j / K, k = j - t * K;
        p.ptok[pos] = t;
        p.pw[pos] = p.topk_w[j];
        p.inv[t * KS + k] = pos;
      }
      run += tot;
      __syncthreads();
    }
  } else {
    const int s = e - E;
    for (int t = tid; t < T; t += 256) {
      const int pos = off + t;
      p.ptok[pos] = t;
      p.pw[pos] = 1.0f;
      p.inv[t * KS + K + s] = pos;
    }
  }
}

hipError_t launch_permute(const FfnParams& p, hipStream_t s) {
  hipLaunchKernelGGL(k_count, dim3(p.E), dim3(256), 0, s, p.topk_idx, p.T * p.K, p.counts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_scatter, dim3(p.NB), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace mpb
