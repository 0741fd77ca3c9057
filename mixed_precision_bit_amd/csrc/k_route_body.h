// Device code of the router (logits and top-K), shared by the per-phase
// kernels and the fused persistent kernel. See k_route.hip for the method.
#pragma once

#include "mpb_device.h"
#include "mpb_internal.h"

namespace mpb {

constexpr int kTT = 8;  // tokens per logits wave unit

// The matrix-core logits are used once a batch has enough 16 x 16 tiles to
// fill the chip.
__host__ __device__ inline bool logits_use_mfma(int T, int E) {
  return (long long)((T + 15) / 16) * ((E + 15) / 16) >= 1024;
}

template <int XDT>
__device__ __forceinline__ float x_to_f32(uint16_t v) {
  if constexpr (XDT == 0) return (float)__builtin_bit_cast(_Float16, v);
  else return __builtin_bit_cast(float, (uint32_t)v << 16);
}

// Hidden-dimension split of the vector-path logits: small batches give too
// few (token tile, expert) units to fill the chip, so each logit is summed in
// ks parts of the hidden pieces (by different waves) and the parts are added
// in order by the top-K step. Depends on the shapes only.
__host__ __device__ inline int route_ksplit(int T, int H, int E) {
  if (logits_use_mfma(T, E)) return 1;
  const long long units = (long long)((T + kTT - 1) / kTT) * E;
  const int npc = (H + 255) / 256;
  long long ks = 2048 / (units > 0 ? units : 1);
  ks = ks < 1 ? 1 : ks > 8 ? 8 : ks;
  return (int)(ks < npc ? ks : npc);
}

// Logits, first half: wave unit u = (8-token tile, EW-expert group, hidden
// part kp of ks) computes its 64 lanes' partial sums and writes them to part
// ([8 EW][65] doubles, the wave's own LDS region). Units past the last one
// write zeros.
template <int XDT, int EW, int NPC>
__device__ __forceinline__ void logits_partials(const uint16_t* __restrict__ X, const float* __restrict__ W, int T,
                                                int H, int E, int ks, long long u, int lane, double* part) {
  const int ntt = (T + kTT - 1) / kTT, neg = (E + EW - 1) / EW;
  const bool live = u < (long long)ntt * neg * ks;
  const int tt = live ? (int)(u % ntt) : 0;
  const long long rest = live ? u / ntt : 0;
  const int eg = (int)(rest % neg), kp = (int)(rest / neg);
  const int t0 = tt * kTT, e0 = eg * EW;
  double a[kTT][EW];
#pragma unroll
  for (int k = 0; k < kTT; ++k)
#pragma unroll
    for (int j = 0; j < EW; ++j) a[k][j] = 0.0;
  if (live) {
    // pieces [p0, p1) of this part, NPC per pass, all loads of a pass in flight together
    const int npc = (H + 255) / 256, ppk = (npc + ks - 1) / ks;
    const int p0 = kp * ppk, p1 = min(npc, p0 + ppk);
    for (int i0 = p0; i0 < p1; i0 += NPC)
#pragma unroll
    for (int i = i0; i < i0 + NPC; ++i) {
      const int h = 4 * lane + 256 * i;
      const bool hin = h < H && i < p1;  // also false for pieces past the part
      const int hc = hin ? h : 0;
      float4 wv[EW];
#pragma unroll
      for (int j = 0; j < EW; ++j) {
        const int e = e0 + j < E ? e0 + j : E - 1;
        wv[j] = *(const float4*)(W + (size_t)e * H + hc);
      }
      ushort4 xv[kTT];
#pragma unroll
      for (int k = 0; k < kTT; ++k) {
        const int t = t0 + k < T ? t0 + k : T - 1;
        xv[k] = *(const ushort4*)(X + (size_t)t * H + hc);
      }
#pragma unroll
      for (int k = 0; k < kTT; ++k) {
        const double x0 = hin ? (double)x_to_f32<XDT>(xv[k].x) : 0.0;
        const double x1 = hin ? (double)x_to_f32<XDT>(xv[k].y) : 0.0;
        const double x2 = hin ? (double)x_to_f32<XDT>(xv[k].z) : 0.0;
        const double x3 = hin ? (double)x_to_f32<XDT>(xv[k].w) : 0.0;
#pragma unroll
        for (int j = 0; j < EW; ++j) {
          a[k][j] = fma(x0, (double)wv[j].x, a[k][j]);
          a[k][j] = fma(x1, (double)wv[j].y, a[k][j]);
          a[k][j] = fma(x2, (double)wv[j].z, a[k][j]);
          a[k][j] = fma(x3, (double)wv[j].w, a[k][j]);
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < kTT; ++k)
#pragma unroll
    for (int j = 0; j < EW; ++j) part[(k * EW + j) * 65 + lane] = a[k][j];
}

// Logits, second half (after a barrier): lane k EW + j sums the 64 partials of
// (token t0 + k, expert e0 + j) in lane order and stores hidden part kp of that
// logit at logits[kp][t][e] (the bias is added with the parts, by top-K).
template <int EW, bool CO = false>
__device__ __forceinline__ void logits_sum(int T, int E, int ks, long long u, int lane, const double* part,
                                           double* __restrict__ logits) {
  const int ntt = (T + kTT - 1) / kTT, neg = (E + EW - 1) / EW;
  if (u >= (long long)ntt * neg * ks || lane >= kTT * EW) return;
  const long long rest = u / ntt;
  const int t0 = (int)(u % ntt) * kTT, e0 = (int)(rest % neg) * EW, kp = (int)(rest / neg);
  const int k = lane / EW, j = lane % EW, t = t0 + k, e = e0 + j;
  double s = 0.0;
#pragma unroll 16
  for (int l = 0; l < 64; ++l) s += part[lane * 65 + l];
  if (t < T && e < E) {
    double* dst = logits + ((size_t)kp * T + t) * E + e;
    if constexpr (CO) __hip_atomic_store(dst, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *dst = s;
  }
}

// Logits of large batches on the fp64 matrix cores: wave unit u is one 16-token x
// 16-expert tile, v_mfma_f64_16x16x4 with tokens as rows and experts as
// columns. Lane l supplies token tile row l % 16 and expert column l % 16 for
// hidden index h0 + 4 (l / 16) + j in MFMA j of each 16-index step, so every
// logit is summed over h in one fixed order (identical router rows give
// identical logits). Output: lane l, value i holds row 4 i + l / 16, column
// l % 16 of the tile; the bias is added by top-K, as for the vector path.
typedef double f64x4 __attribute__((ext_vector_type(4)));


template <int XDT, bool CO = false>
__device__ __forceinline__ void logits_tile_mfma(const uint16_t* __restrict__ X, const float* __restrict__ W, int T,
                                                 int H, int E, long long u, int lane, double* __restrict__ logits) {
  const int g = lane >> 4, c = lane & 15;
  const int ntt = (T + 15) >> 4, net = (E + 15) >> 4;
  if (u >= (long long)ntt * net) return;
  const int tt = (int)(u % ntt), et = (int)(u / ntt);
  const int t = min(tt * 16 + c, T - 1), e = min(et * 16 + c, E - 1);
  const uint16_t* xr = X + (size_t)t * H + 4 * g;
  const float* wr = W + (size_t)e * H + 4 * g;
  f64x4 acc = {0.0, 0.0, 0.0, 0.0};
  constexpr int kU = 8;  // 16-index steps per pass, loads of a pass in flight together
  for (int h0 = 0; h0 < H; h0 += 16 * kU) {
    ushort4 xv[kU];
    float4 wv[kU];
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      const int h = min(h0 + 16 * j, H - 16);  // past the end: a valid address, skipped below
      xv[j] = *(const ushort4*)(xr + h);
      wv[j] = *(const float4*)(wr + h);
    }
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      if (h0 + 16 * j < H) {
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)x_to_f32<XDT>(xv[j].x), (double)wv[j].x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)x_to_f32<XDT>(xv[j].y), (double)wv[j].y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)x_to_f32<XDT>(xv[j].z), (double)wv[j].z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)x_to_f32<XDT>(xv[j].w), (double)wv[j].w, acc, 0, 0, 0);
      }
    }
  }
  const int ecol = et * 16 + c;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int trow = tt * 16 + 4 * i + g;
    if (trow < T && ecol < E) {
      if constexpr (CO)
        __hip_atomic_store(logits + (size_t)trow * E + ecol, acc[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        logits[(size_t)trow * E + ecol] = acc[i];
    }
  }
}

// Top-K of token t by one wave, in three parts separated by barriers: add up
// the logit's hidden parts and the bias into lg (E doubles of LDS), rank every expert (rank(e) = #experts that
// beat it, ties to the lower index) into sel_v / sel_i (16 entries each), then
// the softmax of the K winners summed in rank order.
template <bool CO = false>
__device__ __forceinline__ void topk_load(const double* __restrict__ logits, const float* __restrict__ bias, int ks,
                                          int t, int T, int E, int lane, double* lg) {
  if (t < T)
    for (int e = lane; e < E; e += 64) {
      double v = 0.0;
      for (int kp = 0; kp < ks; ++kp) {
        const double* a = logits + ((size_t)kp * T + t) * E + e;
        if constexpr (CO) v += __hip_atomic_load(const_cast<double*>(a), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else v += *a;
      }
      lg[e] = v + (bias ? (double)bias[e] : 0.0);
    }
}

__device__ __forceinline__ void topk_rank(int t, int T, int E, int K, int lane, const double* lg, double* sel_v,
                                          int* sel_i) {
  if (t >= T) return;
  for (int e = lane; e < E; e += 64) {
    const double v = lg[e];
    int rank = 0;
#pragma unroll 4
    for (int j = 0; j < E; ++j) {
      const double x = lg[j];
      rank += (x > v || (x == v && j < e)) ? 1 : 0;
    }
    if (rank < K) {
      sel_v[rank] = v;
      sel_i[rank] = e;
    }
  }
}

template <bool CO = false>
__device__ __forceinline__ void topk_finish(int t, int T, int K, int lane, const double* sel_v, const int* sel_i,
                                            int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  if (t >= T || lane >= K) return;
  double sum = 0.0, mine = 0.0;
  for (int kk = 0; kk < K; ++kk) {
    const double ex = exp(sel_v[kk] - sel_v[0]);
    sum += ex;
    if (kk == lane) mine = ex;
  }
  const int32_t id = sel_i[lane];
  const float wt = (float)(mine / sum);
  if constexpr (CO) {
    __hip_atomic_store(idx_out + (size_t)t * K + lane, id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(w_out + (size_t)t * K + lane, wt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    idx_out[(size_t)t * K + lane] = id;
    w_out[(size_t)t * K + lane] = wt;
  }
}

}  // namespace mpb
