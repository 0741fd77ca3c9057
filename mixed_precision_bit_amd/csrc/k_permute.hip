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
// The same pass lists the work items of the FFN kernels: one per tpi-token
// (gate_up) or tpi_dn-token (down) split of every group with tokens. Each kernel gets its own list,
// ordered by that kernel's committed bitwidth of the group, highest first
// (then by group): workgroup time grows with the bitwidth, and starting the
// longest ones first keeps the end of the launch short.
#include "mpb_device.h"
#include "mpb_internal.h"

namespace mpb {

constexpr int kMaxGroups = 512 + 64;

__global__ __launch_bounds__(256) void k_group(FfnParams p) {
  __shared__ int hist[kMaxGroups];
  __shared__ int red[3][4];
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
  // position of this group's entries (group order) and of its items in both
  // bitwidth-ordered lists: sums over the other groups, one per thread, reduced
  const int mine = e < E ? hist[e] : T;
  const int ni = (mine + p.tpi - 1) / p.tpi, ni_dn = (mine + p.tpi_dn - 1) / p.tpi_dn;
  const int qg = p.q[2 * e], qd = p.q[2 * e + 1];
  int a_off = 0, a_gu = 0, a_dn = 0;
  for (int j = tid; j < p.NB; j += 256) {
    const int c = j < E ? hist[j] : T;
    const int n = (c + p.tpi - 1) / p.tpi, n_dn = (c + p.tpi_dn - 1) / p.tpi_dn;
    const int qj = p.q[2 * j], qjd = p.q[2 * j + 1];
    if (j < e) a_off += c;
    if (qj > qg || (qj == qg && j < e)) a_gu += n;
    if (qjd > qd || (qjd == qd && j < e)) a_dn += n_dn;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    a_off += __shfl_xor(a_off, o);
    a_gu += __shfl_xor(a_gu, o);
    a_dn += __shfl_xor(a_dn, o);
  }
  if (lane == 0) { red[0][w] = a_off; red[1][w] = a_gu; red[2][w] = a_dn; }
  __syncthreads();
  const int off = red[0][0] + red[0][1] + red[0][2] + red[0][3];
  const int igu = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  const int idn = red[2][0] + red[2][1] + red[2][2] + red[2][3];
  if (tid == 0) {
    p.offsets[e] = off;
    p.counts[e] = mine;
    if (e == p.NB - 1) p.offsets[p.NB] = off + mine;
  }
  if (e == 0 && tid == 0) {
    int tot = 0, tot_dn = 0;
    for (int j = 0; j < p.NB; ++j) {
      const int c = j < E ? hist[j] : T;
      tot += (c + p.tpi - 1) / p.tpi;
      tot_dn += (c + p.tpi_dn - 1) / p.tpi_dn;
    }
    p.n_items[0] = tot;
    p.n_items[1] = tot_dn;
  }
  for (int sp = tid; sp < ni; sp += 256) p.items[igu + sp] = (e << 16) | sp;
  for (int sp = tid; sp < ni_dn; sp += 256) p.items_dn[idn + sp] = (e << 16) | sp;
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
