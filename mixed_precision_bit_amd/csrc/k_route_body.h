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

template <bool CO>
__device__ __forceinline__ void st_f64(double* p, double v) {
  if constexpr (CO) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}
template <bool CO>
__device__ __forceinline__ double ld_f64(const double* p) {
  if constexpr (CO) return __hip_atomic_load(const_cast<double*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *p;
}

// Router workspace (fp64): the logit parts [ks][T][E], then per hidden part
// the 1-norms of the router rows [ks][E], which bound the logits' rounding
// error (see topk_certify).
__host__ __device__ inline double* route_ws_l1(double* ws, int ks, int T, int E) {
  return ws + (size_t)ks * T * E;
}

constexpr int kMaxParts = 8;  // hidden parts of a logit at most

// Hidden-dimension split of the vector-path logits: small batches give too
// few (token tile, expert) units to fill the chip, so each logit is summed in
// ks parts of the hidden pieces (by different waves) and the parts are added
// in order by the top-K step. Depends on the shapes only.
__host__ __device__ inline int route_ksplit(int T, int H, int E) {
  if (logits_use_mfma(T, E)) return 1;
  const long long units = (long long)((T + kTT - 1) / kTT) * E;
  const int npc = (H + 255) / 256;
  long long ks = 2048 / (units > 0 ? units : 1);
  ks = ks < 1 ? 1 : ks > kMaxParts ? kMaxParts : ks;
  return (int)(ks < npc ? ks : npc);
}

// Logits, first half: wave unit u = (8-token tile, EW-expert group, hidden
// part kp of ks) computes its 64 lanes' partial sums and writes them to part
// ([8 EW][65] doubles, the wave's own LDS region). Units past the last one
// write zeros. The units of the first token tile also store the 1-norms of
// their router rows over part kp (wl1[kp][e]).
template <int XDT, int EW, int NPC, bool CO = false>
__device__ __forceinline__ void logits_partials(const uint16_t* __restrict__ X, const float* __restrict__ W, int T,
                                                int H, int E, int ks, long long u, int lane, double* part,
                                                double* __restrict__ wl1) {
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
  // the 1-norms: only the units that store them (wave-uniform) add them up;
  // in the fused kernel every unit does (its register budget takes no branch)
  const bool do_l1 = live && (CO || tt == 0);
  double l1[EW];
#pragma unroll
  for (int j = 0; j < EW; ++j) l1[j] = 0.0;
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
      if (do_l1)
#pragma unroll
        for (int j = 0; j < EW; ++j)
          l1[j] += hin ? ((double)fabsf(wv[j].x) + (double)fabsf(wv[j].y)) +
                             ((double)fabsf(wv[j].z) + (double)fabsf(wv[j].w))
                       : 0.0;
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
  if (live && tt == 0) {
#pragma unroll
    for (int j = 0; j < EW; ++j) {
      double v = l1[j];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
      if (lane == 0 && e0 + j < E) st_f64<CO>(wl1 + (size_t)kp * E + e0 + j, v);
    }
  }
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
  if (t < T && e < E) st_f64<CO>(logits + ((size_t)kp * T + t) * E + e, s);
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
                                                 int H, int E, long long u, int lane, double* __restrict__ logits,
                                                 double* __restrict__ wl1) {
  const int g = lane >> 4, c = lane & 15;
  const int ntt = (T + 15) >> 4, net = (E + 15) >> 4;
  if (u >= (long long)ntt * net) return;
  const int tt = (int)(u % ntt), et = (int)(u / ntt);
  const int t = min(tt * 16 + c, T - 1), e = min(et * 16 + c, E - 1);
  const uint16_t* xr = X + (size_t)t * H + 4 * g;
  const float* wr = W + (size_t)e * H + 4 * g;
  f64x4 acc = {0.0, 0.0, 0.0, 0.0};
  double l1 = 0.0;  // this lane's share of the 1-norm of router row e (the first tile row only)
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
        if (tt == 0)
          l1 += ((double)fabsf(wv[j].x) + (double)fabsf(wv[j].y)) + ((double)fabsf(wv[j].z) + (double)fabsf(wv[j].w));
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)x_to_f32<XDT>(xv[j].x), (double)wv[j].x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)x_to_f32<XDT>(xv[j].y), (double)wv[j].y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)x_to_f32<XDT>(xv[j].z), (double)wv[j].z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)x_to_f32<XDT>(xv[j].w), (double)wv[j].w, acc, 0, 0, 0);
      }
    }
  }
  if (tt == 0) {
    l1 += __shfl_xor(l1, 16);
    l1 += __shfl_xor(l1, 32);
    if (g == 0 && et * 16 + c < E) st_f64<CO>(wl1 + et * 16 + c, l1);
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
// the logit's hidden parts and the bias into lg (E doubles of LDS), rank every
// expert (rank(e) = #experts that beat it, ties to the lower index) into sel_v
// / sel_i (the K winners and the runner-up: 17 entries each), then the
// softmax of the K winners summed in rank order.
// KP: the most hidden parts the launch can have (1 on the matrix-core path)
template <bool CO = false, int KP = kMaxParts>
__device__ __forceinline__ void topk_load(const double* __restrict__ logits, const float* __restrict__ bias, int ks,
                                          int t, int T, int E, int lane, double* lg) {
  if (t < T)
    for (int e = CO ? lane : lane + 64; e < E; e += 64) {  // outside CO, topk_gather loads the first
      double v = 0.0;
      if constexpr (CO) {  // the fused kernel: no registers to spare
        for (int kp = 0; kp < ks; ++kp) v += ld_f64<CO>(logits + ((size_t)kp * T + t) * E + e);
      } else {
        // every part's load in flight together (parts past ks re-read the
        // last one and are not added), then the parts added in order
        double a[KP];
#pragma unroll
        for (int kp = 0; kp < KP; ++kp) a[kp] = ld_f64<CO>(logits + ((size_t)min(kp, ks - 1) * T + t) * E + e);
#pragma unroll
        for (int kp = 0; kp < KP; ++kp) v = kp < ks ? v + a[kp] : v;
      }
      lg[e] = v + (bias ? (double)bias[e] : 0.0);
    }
}

// The top-K step's reads besides the logits (topk_load), for the rounding
// bound: max over the experts of ||w_e||_1 + |bias_e| (the 1-norms summed over
// the hidden parts) into *nmax, and ||x_t||_inf from token t's row (the same
// value on every lane). Outside the fused kernel the wave finds the maximum
// itself and stores it in its own *nmax: its first expert's logit and norm
// parts and the first 4096 elements of the row are requested at once (one
// memory round trip; lg gets those logits here, topk_load the rest from
// expert 64 on), and both maxima are reduced across the wave together. In the
// fused kernel (CO: no registers to spare) thread tid of nthr takes experts
// tid, tid + nthr, ... and raises the workgroup's *nmax (LDS, zero before;
// non-negative floats order as their bits).
template <int XDT, bool CO = false, int KP = kMaxParts>
__device__ __forceinline__ float topk_gather(const double* __restrict__ logits, const uint16_t* __restrict__ X,
                                             const float* __restrict__ bias, int ks, int t, int T, int H, int E,
                                             int lane, int tid, int nthr, double* lg, unsigned* nmax) {
  const double* wl1 = route_ws_l1(const_cast<double*>(logits), ks, T, E);
  const int tc = min(t, T - 1);
  const uint16_t* x = X + (size_t)tc * H;
  auto amax4 = [](ushort4 v) {
    return fmaxf(fmaxf(fabsf(x_to_f32<XDT>(v.x)), fabsf(x_to_f32<XDT>(v.y))),
                 fmaxf(fabsf(x_to_f32<XDT>(v.z)), fabsf(x_to_f32<XDT>(v.w))));
  };
  float xi = 0.0f;
  constexpr int kXR = 16;  // row pieces of 256 elements requested with the rest
  if constexpr (CO) {      // the fused kernel: no registers to spare
    for (int e = tid; e < E; e += nthr) {
      double v = bias ? fabs((double)bias[e]) : 0.0;
      for (int kp = 0; kp < ks; ++kp) v += ld_f64<CO>(wl1 + (size_t)kp * E + e);
      atomicMax(nmax, __float_as_uint((float)v));
    }
    for (int h = 4 * lane; h < H; h += 256) xi = fmaxf(xi, amax4(*(const ushort4*)(x + h)));
  } else {
    const int el = min(lane, E - 1);
    double a[KP], b[KP];
    ushort4 xv[kXR];
#pragma unroll
    for (int kp = 0; kp < KP; ++kp) {
      const size_t k = (size_t)min(kp, ks - 1);
      a[kp] = logits[(k * T + tc) * E + el];
      b[kp] = wl1[k * E + el];
    }
#pragma unroll
    for (int i = 0; i < kXR; ++i) xv[i] = *(const ushort4*)(x + min(4 * lane + 256 * i, H - 4));  // repeats are harmless
    const double bl = bias ? (double)bias[el] : 0.0, bn = fabs(bl);
    double v = 0.0, nv = bn;
#pragma unroll
    for (int kp = 0; kp < KP; ++kp) {
      v = kp < ks ? v + a[kp] : v;
      nv = kp < ks ? nv + b[kp] : nv;
    }
#pragma unroll
    for (int i = 0; i < kXR; ++i) xi = fmaxf(xi, amax4(xv[i]));
    if (t < T && lane < E) lg[lane] = v + bl;
    float nm = (float)nv;
    for (int h = 4 * lane + 256 * kXR; h < H; h += 256) xi = fmaxf(xi, amax4(*(const ushort4*)(x + h)));
    for (int e = lane + 64; e < E; e += 64) {
      double w = bias ? fabs((double)bias[e]) : 0.0;
      for (int kp = 0; kp < ks; ++kp) w += wl1[(size_t)kp * E + e];
      nm = fmaxf(nm, (float)w);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      xi = fmaxf(xi, __shfl_xor(xi, o));
      nm = fmaxf(nm, __shfl_xor(nm, o));
    }
    *nmax = __float_as_uint(nm);  // the wave's own slot
    return xi;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) xi = fmaxf(xi, __shfl_xor(xi, o));
  return xi;
}

// the calling wave's LDS accesses before it are done before the ones after it
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  __builtin_amdgcn_wave_barrier();
}

// A nan logit (a non-finite activation) ranks as -inf, so the order is total
// and every rank is taken once. The wave replaces its token's nan logits by
// -inf in place first, so the pairwise count below compares plain values and
// topk_certify sees the same order (two -inf never certify as a gap).
__device__ __forceinline__ void topk_rank(int t, int T, int E, int K, int lane, double* lg, double* sel_v,
                                          int* sel_i) {
  if (t >= T) return;
  for (int e = lane; e < E; e += 64)
    if (lg[e] != lg[e]) lg[e] = -__builtin_inf();
  wave_lds_fence();
  for (int e = lane; e < E; e += 64) {
    const double v = lg[e];
    int rank = 0;
#pragma unroll 4
    for (int j = 0; j < E; ++j) {
      const double x = lg[j];
      rank += (x > v || (x == v && j < e)) ? 1 : 0;
    }
    if (rank <= K) {  // the K winners and the runner-up (sel_* hold K + 1 <= 17 entries)
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

// ---------------------------------------------------------------- exact order
// Every fp64 logit is a sum of H exact products x_h w_h (an fp16 or bf16 times
// an fp32 fits the 53-bit significand) and the bias, so whatever the order of
// its additions its rounding error is at most gamma_n (||x_t||_inf ||w_e||_1 +
// |bias_e|) <= B_t = gamma_n max(||x_t||_inf, 1) max_e (||w_e||_1 + |bias_e|)
// with gamma_n = n u / (1 - n u), u = 2^-53 and n the number of additions
// (Higham, Accuracy and Stability of Numerical Algorithms, §4.2; n is taken as
// 2 (H + 64), which also covers a matrix-core sum rounded more than once per
// step). The top-K of a token is certified when each winner's logit exceeds
// the next one's, and the last winner's the runner-up's, by more than 2 B_t:
// every other expert lies at or below the runner-up. Otherwise ("PagedWeight"
// §2.1 ranks the experts by their logits; ties go to the lower index) the
// experts within 2 B_t of the last winner or above it are ranked on their
// exact logits: each product is an integer times a power of two, summed
// exactly into kXL 32-bit digits of weight 2^-282 .. 2^294 (which hold any
// fp16 or bf16 x fp32 product, any fp32 bias and their sums), and the K
// largest are kept, equal values in index order.
constexpr int kXL = 18;
constexpr int kXEmin = -282;

struct ExactScratch {           // one wave's, in LDS
  unsigned long long acc[kXL];  // the candidate's digits, carries pending
  uint32_t top[16][kXL];        // the exact top list: digits in [0, 2^32), the last one signed
  int top_i[16];
  int n;
};

// a finite value's bits as (-1)^neg m 2^e
__device__ __forceinline__ void decode_f16(uint32_t b, uint64_t& m, int& e, bool& neg) {
  const uint32_t ex = (b >> 10) & 31, f = b & 1023;
  neg = (b >> 15) & 1;
  m = ex ? (f | 1024u) : f;
  e = ex ? (int)ex - 25 : -24;
}
__device__ __forceinline__ void decode_bf16(uint32_t b, uint64_t& m, int& e, bool& neg) {
  const uint32_t ex = (b >> 7) & 255, f = b & 127;
  neg = (b >> 15) & 1;
  m = ex ? (f | 128u) : f;
  e = ex ? (int)ex - 134 : -133;
}
__device__ __forceinline__ void decode_f32(uint32_t b, uint64_t& m, int& e, bool& neg) {
  const uint32_t ex = (b >> 23) & 255, f = b & 0x7fffffu;
  neg = b >> 31;
  m = ex ? (f | 0x800000u) : f;
  e = ex ? (int)ex - 150 : -149;
}

// acc += (-1)^neg P 2^e for P < 2^35 and kXEmin <= e <= 226 (inf and nan
// inputs decode into that range too): three digits, LDS atomics
__device__ __forceinline__ void exact_add(unsigned long long* acc, uint64_t P, int e, bool neg) {
  const int off = e - kXEmin, k = off >> 5, r = off & 31;
  const uint64_t lo = (uint32_t)(P << r);
  const uint64_t rest = r ? P >> (32 - r) : P >> 32;
  const uint64_t mid = (uint32_t)rest, hi = rest >> 32;
  atomicAdd(acc + k, neg ? 0ull - lo : lo);
  if (mid) atomicAdd(acc + k + 1, neg ? 0ull - mid : mid);
  if (hi) atomicAdd(acc + k + 2, neg ? 0ull - hi : hi);
}

// Exact logit of (t, e) into sc.acc, by one whole wave.
template <int XDT>
__device__ __forceinline__ void exact_logit(const uint16_t* __restrict__ X, const float* __restrict__ W,
                                            const float* __restrict__ bias, int t, int e, int H, int lane,
                                            ExactScratch& sc) {
  if (lane < kXL) sc.acc[lane] = 0ull;
  wave_lds_fence();
  const uint16_t* x = X + (size_t)t * H;
  const uint32_t* w = (const uint32_t*)W + (size_t)e * H;
  for (int h = lane; h < H; h += 64) {
    uint64_t mx, mw;
    int ex, ew;
    bool sx, sw;
    if constexpr (XDT == 0) decode_f16(x[h], mx, ex, sx);
    else decode_bf16(x[h], mx, ex, sx);
    decode_f32(w[h], mw, ew, sw);
    if (mx && mw) exact_add(sc.acc, mx * mw, ex + ew, sx != sw);
  }
  if (lane == 0 && bias) {
    uint64_t mb;
    int eb;
    bool sb;
    decode_f32(__builtin_bit_cast(uint32_t, bias[e]), mb, eb, sb);
    if (mb) exact_add(sc.acc, mb, eb, sb);
  }
  wave_lds_fence();
}

// a > b for digit lists in the top-list form
__device__ __forceinline__ bool exact_greater(const uint32_t* a, const uint32_t* b) {
  if (a[kXL - 1] != b[kXL - 1]) return (int32_t)a[kXL - 1] > (int32_t)b[kXL - 1];
  for (int k = kXL - 2; k >= 0; --k)
    if (a[k] != b[k]) return a[k] > b[k];
  return false;
}

// B_t of the comment above, from ||x_t||_inf and max_e (||w_e||_1 + |bias_e|)
// (the margin covers that maximum rounded to float and the bound's own
// rounding).
__device__ __forceinline__ double logit_bound(int H, float xi, float nmax) {
  const double n = 2.0 * ((double)H + 64.0), u = 0x1p-53;
  return n * u / (1.0 - n * u) * (1.0 + 0x1p-20) * fmax((double)xi, 1.0) * (double)nmax;
}

// Certificate of the top-K in sel_v / sel_i (after topk_rank: winners and
// runner-up) and, when it fails, the exact ranking in their place. lg: token
// t's fp64 logits, B: their error bound. Called by the whole wave of token t;
// lane i < K checks winner i against the next entry.
template <int XDT>
__device__ __forceinline__ void topk_certify(const uint16_t* __restrict__ X, const float* __restrict__ W,
                                             const float* __restrict__ bias, int t, int T, int H, int E, int K,
                                             int lane, const double* lg, double B, double* sel_v, int* sel_i,
                                             ExactScratch& sc) {
  if (t >= T) return;
  const bool ok = !(lane < K && lane + 1 <= min(K, E - 1)) || sel_v[lane] - B > sel_v[lane + 1] + B;
  if (__all(ok)) return;
  const double thr = sel_v[K - 1] - B;
  const double vK = sel_v[K - 1];
  const int iK = sel_i[K - 1];
  auto winner = [&](int e) { return lg[e] > vK || (lg[e] == vK && e <= iK); };
  // exact ranking of the winners and of every expert within reach of them
  if (lane == 0) sc.n = 0;
  if (lane < 16) sc.top_i[lane] = 0;  // the K winners fill every slot; a valid id regardless
  wave_lds_fence();
  for (int e = 0; e < E; ++e) {
    if (!winner(e) && lg[e] + B < thr) continue;  // the same on every lane
    exact_logit<XDT>(X, W, bias, t, e, H, lane, sc);
    if (lane == 0) {
      long long v[kXL];
      for (int k = 0; k < kXL; ++k) v[k] = (long long)sc.acc[k];
      for (int k = 0; k < kXL - 1; ++k) {
        const long long c = v[k] >> 32;  // floor
        v[k] -= c * 4294967296ll;
        v[k + 1] += c;
      }
      uint32_t d[kXL];
      for (int k = 0; k < kXL; ++k) d[k] = (uint32_t)v[k];
      int pos = sc.n;
      while (pos > 0 && exact_greater(d, sc.top[pos - 1])) --pos;
      if (pos < K) {
        for (int q = min(sc.n, K - 1); q > pos; --q) {
          for (int k = 0; k < kXL; ++k) sc.top[q][k] = sc.top[q - 1][k];
          sc.top_i[q] = sc.top_i[q - 1];
        }
        for (int k = 0; k < kXL; ++k) sc.top[pos][k] = d[k];
        sc.top_i[pos] = e;
        sc.n = min(sc.n + 1, K);
      }
    }
    wave_lds_fence();
  }
  if (lane < K) {
    const int e = sc.top_i[lane];
    sel_i[lane] = e;
    sel_v[lane] = lg[e];
  }
  wave_lds_fence();
}

}  // namespace mpb
