// Router: logits, top-K and routing weights.
//
// "PagedWeight", §2.1: the router assigns routing weights to the E experts and
// selects the top K for each token. Logits are accumulated in fp64: an fp16 or
// bf16 activation times an fp32 router weight is exact in fp64, and each logit
// is summed in one fixed order, so two identical router rows give bit-identical
// logits and the lower expert index wins the tie. The routing weights are the
// softmax over all experts restricted to the K winners and renormalised, which
// equals a softmax over the K winning logits.
#include "mpb_device.h"
#include "mpb_internal.h"

namespace mpb {

constexpr int kRT = 16;      // tokens per workgroup
constexpr int kHC = 64;      // activations staged per step
constexpr int kEMax = 512;   // experts supported by the LDS logit tile

template <int XDT>
__device__ __forceinline__ double x_to_f64(uint16_t v) {
  if constexpr (XDT == 0) return (double)__builtin_bit_cast(_Float16, v);
  else return (double)__builtin_bit_cast(float, (uint32_t)v << 16);
}

__device__ __forceinline__ bool better(double v, int i, double bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

template <int XDT>
__global__ __launch_bounds__(256) void k_route(const uint16_t* __restrict__ X, const float* __restrict__ W,
                                               const float* __restrict__ bias, int T, int H, int E, int K,
                                               int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  __shared__ double xs[kRT][kHC + 1];  // +1: the 16 token rows fall in distinct banks
  __shared__ double lg[kRT][kEMax];
  __shared__ double tv[4][16];
  __shared__ int ti[4][16];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kRT;
  const int tl = tid & 15, eg = tid >> 4;

  // logits: thread (tl, eg) owns experts ep + eg + 16*j, j < 8
  for (int ep = 0; ep < E; ep += 128) {
    double acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.0;
    for (int h0 = 0; h0 < H; h0 += kHC) {
      __syncthreads();
      for (int j = tid; j < kRT * kHC; j += 256) {
        const int t = j / kHC, hh = j % kHC;
        xs[t][hh] = (t0 + t < T) ? x_to_f64<XDT>(X[(size_t)(t0 + t) * H + h0 + hh]) : 0.0;
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int e = ep + eg + 16 * j;
        if (e < E) {
          const float4* wr = (const float4*)(W + (size_t)e * H + h0);
          double a = acc[j];
          for (int h4 = 0; h4 < kHC / 4; ++h4) {
            const float4 wv = wr[h4];
            a = fma(xs[tl][4 * h4 + 0], (double)wv.x, a);
            a = fma(xs[tl][4 * h4 + 1], (double)wv.y, a);
            a = fma(xs[tl][4 * h4 + 2], (double)wv.z, a);
            a = fma(xs[tl][4 * h4 + 3], (double)wv.w, a);
          }
          acc[j] = a;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = ep + eg + 16 * j;
      if (e < E) lg[tl][e] = acc[j] + (bias ? (double)bias[e] : 0.0);
    }
  }
  __syncthreads();

  // top-K: wave w handles token slots w, w+4, w+8, w+12
  const int lane = tid & 63, w = tid >> 6;
  for (int tt = w; tt < kRT; tt += 4) {
    const int t = t0 + tt;
    if (t >= T) break;
    uint32_t taken = 0;
    for (int k = 0; k < K; ++k) {
      double bv = -__builtin_inf();
      int bi = 0x7fffffff;
      for (int i = 0; i < kEMax / 64; ++i) {
        const int e = lane + 64 * i;
        if (e < E && !((taken >> i) & 1u)) {
          const double v = lg[tt][e];
          if (better(v, e, bv, bi)) { bv = v; bi = e; }
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const double ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      }
      if (bi < E && (bi & 63) == lane) taken |= 1u << (bi >> 6);
      if (lane == 0) { tv[w][k] = bv; ti[w][k] = bi; }
    }
    if (lane == 0) {
      double sum = 0.0;
      for (int k = 0; k < K; ++k) sum += exp(tv[w][k] - tv[w][0]);
      for (int k = 0; k < K; ++k) {
        idx_out[(size_t)t * K + k] = ti[w][k];
        w_out[(size_t)t * K + k] = (float)(exp(tv[w][k] - tv[w][0]) / sum);
      }
    }
  }
}

hipError_t launch_route(const uint16_t* X, int xdt, const float* W, const float* bias, int T, int H, int E,
                        int K, int32_t* idx, float* w, hipStream_t s) {
  const dim3 grid((T + kRT - 1) / kRT);
  if (xdt == 0) hipLaunchKernelGGL(k_route<0>, grid, dim3(256), 0, s, X, W, bias, T, H, E, K, idx, w);
  else hipLaunchKernelGGL(k_route<1>, grid, dim3(256), 0, s, X, W, bias, T, H, E, K, idx, w);
  return hipGetLastError();
}

}  // namespace mpb
