// Token grouping by expert (one launch).
//
// Routed expert e receives the (token, k) pairs with topk_idx[t][k] == e, kept
// in (t, k) order; shared experts receive every token with weight 1. Grouped
// entries of expert e occupy positions offsets[e] .. offsets[e+1]-1; inv maps
// each (t, slot) back to its position (slot k < K routed, K + s shared).
// Every workgroup builds the whole expert histogram in LDS (integer counts,
// order-free), takes its own offset from it, then places its entries with a
// ballot-ordered scan, so the grouping is identical on every run.
//
// The same pass lists the work items of the decode FFN kernels: one per
// 32-token split of every group with tokens, in group order, so that those
// kernels launch no workgroup without work in front of busy ones.
#include "mpb_device.h"
#include "mpb_internal.h"

namespace mpb {

constexpr int kMaxGroups = 512 + 64;

__global__ __launch_bounds__(256) void k_group(FfnParams p) {
  __shared__ int hist[kMaxGroups];
  __shared__ int s_off, s_ioff;
  __shared__ int wtot[4];
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int T = p.T, K = p.K, S = p.S, E = p.E, KS = K + S, TK = T * K;
  for (int i = tid; i < E; i += 256) hist[i] = 0;
  __syncthreads();
  for (int j = tid; j < TK; j += 256) {
    const int x = p.topk_idx[j];
    if (x >= 0 && x < E) atomicAdd(&hist[x], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int off = 0, ioff = 0;
    for (int j = 0; j < e; ++j) {
      const int c = j < E ? hist[j] : T;
      off += c;
      ioff += (c + kDecodeTokensPerWG - 1) / kDecodeTokensPerWG;
    }
    const int mine = e < E ? hist[e] : T;
    s_off = off;
    s_ioff = ioff;
    p.offsets[e] = off;
    p.counts[e] = mine;
    if (e == p.NB - 1) {
      p.offsets[p.NB] = off + mine;
      p.n_items[0] = ioff + (mine + kDecodeTokensPerWG - 1) / kDecodeTokensPerWG;
    }
  }
  __syncthreads();
  const int off = s_off;
  {
    const int mine = e < E ? hist[e] : T;
    const int ni = (mine + kDecodeTokensPerWG - 1) / kDecodeTokensPerWG;
    for (int sp = tid; sp < ni; sp += 256) p.items[s_ioff + sp] = (e << 16) | sp;
  }
  if (e < E) {
    int run = 0;
    for (int b0 = 0; b0 < TK; b0 += 256) {
      const int j = b0 + tid;
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
  hipLaunchKernelGGL(k_group, dim3(p.NB), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace mpb
