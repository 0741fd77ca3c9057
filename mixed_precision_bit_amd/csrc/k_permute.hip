// Token grouping by expert (one launch).
//
// Routed expert e receives the (token, k) pairs with topk_idx[t][k] == e, kept
// in (t, k) order; shared experts receive every token with weight 1. Grouped
// entries of expert e occupy positions offsets[e] .. offsets[e+1]-1; ent holds
// each entry's (token, slot) index t (K + S) + slot (slot k < K routed, K + s
// shared), the row of y the down projection writes for it.
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

constexpr int kIdxCache = 8;  // topk ids kept in registers per thread between the two passes

__global__ __launch_bounds__(256) void k_group(FfnParams p) {
  __shared__ int hist[kMaxGroups];
  __shared__ int red[5][4];
  __shared__ int wtot[4];
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int T = p.T, K = p.K, S = p.S, E = p.E, KS = K + S, TK = T * K;
  // every global read the pass needs is issued up front (one memory round trip)
  int xid[kIdxCache];
#pragma unroll
  for (int c = 0; c < kIdxCache; ++c) {
    const int j = tid + 256 * c;
    xid[c] = j < TK ? p.topk_idx[j] : -1;
  }
  int qjg[3], qjd[3];
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    const int j = tid + 256 * c;  // NB <= 576 < 3 * 256
    qjg[c] = j < p.NB ? p.q[2 * j] : 0;
    qjd[c] = j < p.NB ? p.q[2 * j + 1] : 0;
  }
  const int qg = p.q[2 * e], qd = p.q[2 * e + 1];
  for (int i = tid; i < E; i += 256) hist[i] = 0;
  __syncthreads();
#pragma unroll
  for (int c = 0; c < kIdxCache; ++c)
    if (xid[c] >= 0 && xid[c] < E) atomicAdd(&hist[xid[c]], 1);
  for (int j = tid + 256 * kIdxCache; j < TK; j += 256) {
    const int x = p.topk_idx[j];
    if (x >= 0 && x < E) atomicAdd(&hist[x], 1);
  }
  __syncthreads();
  // position of this group's entries (group order), of its items in both
  // bitwidth-ordered lists, and the item totals: sums over the groups, one per
  // thread, reduced
  const int mine = e < E ? hist[e] : T;
  const int ni = (mine + p.tpi - 1) / p.tpi, ni_dn = (mine + p.tpi_dn - 1) / p.tpi_dn;
  int a[5] = {0, 0, 0, 0, 0};  // offset, gate_up position, down position, gate_up total, down total
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    const int j = tid + 256 * c;
    if (j < p.NB) {
      const int cnt = j < E ? hist[j] : T;
      const int n = (cnt + p.tpi - 1) / p.tpi, n_dn = (cnt + p.tpi_dn - 1) / p.tpi_dn;
      if (j < e) a[0] += cnt;
      if (qjg[c] > qg || (qjg[c] == qg && j < e)) a[1] += n;
      if (qjd[c] > qd || (qjd[c] == qd && j < e)) a[2] += n_dn;
      a[3] += n;
      a[4] += n_dn;
    }
  }
#pragma unroll
  for (int i = 0; i < 5; ++i) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) a[i] += __shfl_xor(a[i], o);
    if (lane == 0) red[i][w] = a[i];
  }
  __syncthreads();
  int r[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) r[i] = red[i][0] + red[i][1] + red[i][2] + red[i][3];
  const int off = r[0], igu = r[1], idn = r[2];
  if (tid == 0) {
    p.offsets[e] = off;
    p.counts[e] = mine;
    if (e == p.NB - 1) p.offsets[p.NB] = off + mine;
    if (e == 0) {
      p.n_items[0] = r[3];
      p.n_items[1] = r[4];
    }
  }
  for (int sp = tid; sp < ni; sp += 256) p.items[igu + sp] = (e << 16) | sp;
  for (int sp = tid; sp < ni_dn; sp += 256) p.items_dn[idn + sp] = (e << 16) | sp;
  if (e < E) {
    int run = 0;
    for (int b0 = 0, c = 0; b0 < TK; b0 += 256, ++c) {
      const int j = b0 + tid;
      int x = -1;
#pragma unroll
      for (int cc = 0; cc < kIdxCache; ++cc)
        if (cc == c) x = xid[cc];
      if (c >= kIdxCache && j < TK) x = p.topk_idx[j];
      const bool m = x == e;
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
        p.ent[pos] = t * KS + k;
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
      p.ent[pos] = t * KS + K + s;
    }
  }
}

// Chunked grouping for large batches (the same result as k_group): k_group
// walks all T*K routed ids once per group, which costs O(groups x T K) at
// prefill sizes. Here the ids are cut into chunks of kGroupChunk entries:
// k_chunk_hist counts every group's entries per chunk, k_chunk_scan turns the
// counts into per-chunk starting ranks and per-group totals, and
// k_chunk_scatter places the entries of one (group, chunk) pair, in (t, k)
// order, starting at the group's offset plus the chunk's starting rank.
__global__ __launch_bounds__(256) void k_chunk_hist(FfnParams p, int32_t* ccnt) {
  __shared__ int hist[kMaxGroups];
  const int c = blockIdx.x, tid = threadIdx.x, E = p.E, TK = p.T * p.K;
  for (int i = tid; i < E; i += 256) hist[i] = 0;
  __syncthreads();
  const int j1 = min(TK, (c + 1) * kGroupChunk);
  for (int j = c * kGroupChunk + tid; j < j1; j += 256) {
    const int x = p.topk_idx[j];
    if (x >= 0 && x < E) atomicAdd(&hist[x], 1);
  }
  __syncthreads();
  for (int i = tid; i < E; i += 256) ccnt[(size_t)c * E + i] = hist[i];
}

// One thread per routed group: exclusive prefix over the chunks (in place)
// and the group's total.
__global__ __launch_bounds__(256) void k_chunk_scan(FfnParams p, int32_t* ccnt, int nchunk) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= p.E) return;
  int run = 0;
  for (int c = 0; c < nchunk; ++c) {
    const int v = ccnt[(size_t)c * p.E + e];
    ccnt[(size_t)c * p.E + e] = run;
    run += v;
  }
  p.counts[e] = run;
}

__global__ __launch_bounds__(256) void k_chunk_scatter(FfnParams p, const int32_t* ccnt) {
  __shared__ int red[5][4];
  __shared__ int wtot[4];
  const int e = blockIdx.x, c = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int T = p.T, K = p.K, E = p.E, KS = K + p.S, TK = T * K;
  // group sizes (routed: totals from the scan; shared: every token), then
  // this group's offset and item positions as in k_group
  const int qg = p.q[2 * e], qd = p.q[2 * e + 1];
  const int mine = e < E ? p.counts[e] : T;
  const int ni = (mine + p.tpi - 1) / p.tpi, ni_dn = (mine + p.tpi_dn - 1) / p.tpi_dn;
  int a[5] = {0, 0, 0, 0, 0};
  for (int j = tid; j < p.NB; j += 256) {
    const int cnt = j < E ? p.counts[j] : T;
    const int n = (cnt + p.tpi - 1) / p.tpi, n_dn = (cnt + p.tpi_dn - 1) / p.tpi_dn;
    const int qjg = p.q[2 * j], qjd = p.q[2 * j + 1];
    if (j < e) a[0] += cnt;
    if (qjg > qg || (qjg == qg && j < e)) a[1] += n;
    if (qjd > qd || (qjd == qd && j < e)) a[2] += n_dn;
    a[3] += n;
    a[4] += n_dn;
  }
#pragma unroll
  for (int i = 0; i < 5; ++i) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) a[i] += __shfl_xor(a[i], o);
    if (lane == 0) red[i][w] = a[i];
  }
  __syncthreads();
  int r[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) r[i] = red[i][0] + red[i][1] + red[i][2] + red[i][3];
  const int off = r[0];
  if (c == 0) {
    if (tid == 0) {
      p.offsets[e] = off;
      if (e >= E) p.counts[e] = mine;
      if (e == p.NB - 1) p.offsets[p.NB] = off + mine;
      if (e == 0) {
        p.n_items[0] = r[3];
        p.n_items[1] = r[4];
      }
    }
    for (int sp = tid; sp < ni; sp += 256) p.items[r[1] + sp] = (e << 16) | sp;
    for (int sp = tid; sp < ni_dn; sp += 256) p.items_dn[r[2] + sp] = (e << 16) | sp;
  }
  if (e < E) {
    int run = off + ccnt[(size_t)c * E + e];
    const int j1 = min(TK, (c + 1) * kGroupChunk);
    for (int b0 = c * kGroupChunk; b0 < j1; b0 += 256) {
      const int j = b0 + tid;
      const int x = j < j1 ? p.topk_idx[j] : -1;
      const bool m = x == e;
      const unsigned long long bal = __ballot(m);
      const int lp = __popcll(bal & ((1ull << lane) - 1ull));
      if (lane == 0) wtot[w] = __popcll(bal);
      __syncthreads();
      int wp = 0;
      for (int v = 0; v < w; ++v) wp += wtot[v];
      const int tot = wtot[0] + wtot[1] + wtot[2] + wtot[3];
      if (m) {
        const int pos = run + wp + lp;
        const int t = j / K, k = j - t * K;
        p.ptok[pos] = t;
        p.pw[pos] = p.topk_w[j];
        p.ent[pos] = t * KS + k;
      }
      run += tot;
      __syncthreads();
    }
  } else if (c == 0) {
    const int sh = e - E;
    for (int t = tid; t < T; t += 256) {
      const int pos = off + t;
      p.ptok[pos] = t;
      p.pw[pos] = 1.0f;
      p.ent[pos] = t * KS + K + sh;
    }
  }
}

int group_chunks(int T, int K) {
  const long long TK = (long long)T * K;
  return TK >= kChunkedFrom ? (int)((TK + kGroupChunk - 1) / kGroupChunk) : 0;
}

hipError_t launch_permute(const FfnParams& p, int32_t* ccnt, hipStream_t s) {
  const int nc = group_chunks(p.T, p.K);
  if (nc == 0) {
    hipLaunchKernelGGL(k_group, dim3(p.NB), dim3(256), 0, s, p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_chunk_hist, dim3(nc), dim3(256), 0, s, p, ccnt);
  hipLaunchKernelGGL(k_chunk_scan, dim3((p.E + 255) / 256), dim3(256), 0, s, p, ccnt, nc);
  hipLaunchKernelGGL(k_chunk_scatter, dim3(p.NB, nc), dim3(256), 0, s, p, (const int32_t*)ccnt);
  return hipGetLastError();
}

}  // namespace mpb
