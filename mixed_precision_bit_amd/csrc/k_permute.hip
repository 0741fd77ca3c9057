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
// longest ones first keeps the end of the launch short. Groups of at least
// wide_from tokens (when set) go to the wide lists instead, split into
// tpi_w-token (gate_up) and tpi_dnw-token (down) items: first every full item
// in the same order, then each group's last, partial item in that order (the
// lighter workgroups come last, where a launch's final round runs).
#include "mpb_device.h"
#include "mpb_internal.h"

namespace mpb {

constexpr int kMaxGroups = 512 + 64;

constexpr int kIdxCache = 8;  // topk ids kept in registers per thread between the two passes

// Items of a group of cnt tokens in the lists: narrow gate_up, narrow down,
// and the wide lists' full and partial items (a group is in the narrow or the
// wide lists; a wide group has at most one partial item per list).
struct GroupItems {
  int gu, dn, gwf, gwp, dwf, dwp;
};
template <bool WIDE>
__device__ __forceinline__ GroupItems group_items(const FfnParams& p, int cnt) {
  const bool wide = WIDE && cnt >= p.wide_from;
  GroupItems n;
  n.gu = wide ? 0 : (cnt + p.tpi - 1) / p.tpi;
  n.dn = wide ? 0 : (cnt + p.tpi_dn - 1) / p.tpi_dn;
  n.gwf = wide ? cnt / p.tpi_w : 0;
  n.gwp = wide && cnt % p.tpi_w ? 1 : 0;
  n.dwf = wide ? cnt / p.tpi_dnw : 0;
  n.dwp = wide && cnt % p.tpi_dnw ? 1 : 0;
  return n;
}

// Sums over group j (count cnt, bitwidths qjg / qjd) that place group e's
// entries and items: a[0] entry offset; positions before e in bitwidth order
// a[1] narrow gate_up, a[2] narrow down, a[3] / a[4] wide gate_up full /
// partial, a[5] / a[6] wide down full / partial; totals a[7] narrow gate_up,
// a[8] narrow down, a[9] / a[10] wide gate_up full / partial, a[11] / a[12]
// wide down full / partial; a[13] the 32-token h panel blocks of the wide
// groups before e.
constexpr int kSums = 14;
__host__ __device__ constexpr bool wide_sum(int i) { return (i >= 3 && i <= 6) || i >= 9; }
template <bool WIDE>
__device__ __forceinline__ void add_group(const FfnParams& p, int (&a)[kSums], int j, int cnt, int qjg, int qjd,
                                          int e, int qg, int qd) {
  const GroupItems n = group_items<WIDE>(p, cnt);
  const bool before_g = qjg > qg || (qjg == qg && j < e);
  const bool before_d = qjd > qd || (qjd == qd && j < e);
  if (j < e) {
    a[0] += cnt;
    a[13] += n.gwf + n.gwp ? (cnt + 31) >> 5 : 0;
  }
  if (before_g) {
    a[1] += n.gu;
    a[3] += n.gwf;
    a[4] += n.gwp;
  }
  if (before_d) {
    a[2] += n.dn;
    a[5] += n.dwf;
    a[6] += n.dwp;
  }
  a[7] += n.gu;
  a[8] += n.dn;
  a[9] += n.gwf;
  a[10] += n.gwp;
  a[11] += n.dwf;
  a[12] += n.dwp;
}

// Writes group e's item entries (and, from group 0, the totals).
template <bool WIDE>
__device__ __forceinline__ void put_items(const FfnParams& p, const int (&r)[kSums], int e, int mine, int tid) {
  const GroupItems n = group_items<WIDE>(p, mine);
  if (tid == 0 && e == 0) {
    p.n_items[0] = r[7];
    p.n_items[1] = r[8];
    p.n_items[2] = r[9] + r[10];
    p.n_items[3] = r[11] + r[12];
  }
  for (int sp = tid; sp < n.gu; sp += 256) p.items[r[1] + sp] = (e << 16) | sp;
  for (int sp = tid; sp < n.dn; sp += 256) p.items_dn[r[2] + sp] = (e << 16) | sp;
  for (int sp = tid; sp < n.gwf; sp += 256) p.items_w[r[3] + sp] = (e << 16) | sp;
  for (int sp = tid; sp < n.dwf; sp += 256) p.items_dnw[r[5] + sp] = (e << 16) | sp;
  if (tid == 0 && WIDE) p.wblk[e] = r[13];
  if (tid == 0 && n.gwp) p.items_w[r[9] + r[4]] = (e << 16) | n.gwf;
  if (tid == 0 && n.dwp) p.items_dnw[r[11] + r[6]] = (e << 16) | n.dwf;
}

template <bool WIDE>
__global__ __launch_bounds__(256) void k_group(FfnParams p) {
  __shared__ int hist[kMaxGroups];
  __shared__ int red[kSums][4];
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
  // position of this group's entries (group order), of its items in the
  // bitwidth-ordered lists, and the item totals: sums over the groups, one per
  // thread, reduced
  const int mine = e < E ? hist[e] : T;
  int a[kSums] = {};
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    const int j = tid + 256 * c;
    if (j < p.NB) add_group<WIDE>(p, a, j, j < E ? hist[j] : T, qjg[c], qjd[c], e, qg, qd);
  }
#pragma unroll
  for (int i = 0; i < kSums; ++i) {
    if (wide_sum(i) && !WIDE) continue;  // zero without wide items
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) a[i] += __shfl_xor(a[i], o);
    if (lane == 0) red[i][w] = a[i];
  }
  __syncthreads();
  int r[kSums];
#pragma unroll
  for (int i = 0; i < kSums; ++i)
    r[i] = wide_sum(i) && !WIDE ? 0 : red[i][0] + red[i][1] + red[i][2] + red[i][3];
  const int off = r[0];
  if (tid == 0) {
    p.offsets[e] = off;
    p.counts[e] = mine;
    if (e == p.NB - 1) p.offsets[p.NB] = off + mine;
  }
  put_items<WIDE>(p, r, e, mine, tid);
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

template <bool WIDE>
__global__ __launch_bounds__(256) void k_chunk_scatter(FfnParams p, const int32_t* ccnt) {
  __shared__ int red[kSums][4];
  __shared__ int wtot[4];
  const int e = blockIdx.x, c = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int T = p.T, K = p.K, E = p.E, KS = K + p.S, TK = T * K;
  // group sizes (routed: totals from the scan; shared: every token), then
  // this group's offset and item positions as in k_group
  const int qg = p.q[2 * e], qd = p.q[2 * e + 1];
  const int mine = e < E ? p.counts[e] : T;
  int a[kSums] = {};
  for (int j = tid; j < p.NB; j += 256)
    add_group<WIDE>(p, a, j, j < E ? p.counts[j] : T, p.q[2 * j], p.q[2 * j + 1], e, qg, qd);
#pragma unroll
  for (int i = 0; i < kSums; ++i) {
    if (wide_sum(i) && !WIDE) continue;  // zero without wide items
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) a[i] += __shfl_xor(a[i], o);
    if (lane == 0) red[i][w] = a[i];
  }
  __syncthreads();
  int r[kSums];
#pragma unroll
  for (int i = 0; i < kSums; ++i)
    r[i] = wide_sum(i) && !WIDE ? 0 : red[i][0] + red[i][1] + red[i][2] + red[i][3];
  const int off = r[0];
  if (c == 0) {
    if (tid == 0) {
      p.offsets[e] = off;
      if (e >= E) p.counts[e] = mine;
      if (e == p.NB - 1) p.offsets[p.NB] = off + mine;
    }
    put_items<WIDE>(p, r, e, mine, tid);
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
  // WIDE: the variants that also list the wide items (a layer and batch that use them)
  const bool wide = p.wide_from > 0;
  if (nc == 0) {
    if (wide) hipLaunchKernelGGL(k_group<true>, dim3(p.NB), dim3(256), 0, s, p);
    else hipLaunchKernelGGL(k_group<false>, dim3(p.NB), dim3(256), 0, s, p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_chunk_hist, dim3(nc), dim3(256), 0, s, p, ccnt);
  hipLaunchKernelGGL(k_chunk_scan, dim3((p.E + 255) / 256), dim3(256), 0, s, p, ccnt, nc);
  if (wide) hipLaunchKernelGGL(k_chunk_scatter<true>, dim3(p.NB, nc), dim3(256), 0, s, p, (const int32_t*)ccnt);
  else hipLaunchKernelGGL(k_chunk_scatter<false>, dim3(p.NB, nc), dim3(256), 0, s, p, (const int32_t*)ccnt);
  return hipGetLastError();
}

}  // namespace mpb
