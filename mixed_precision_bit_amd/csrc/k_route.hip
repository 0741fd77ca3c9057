// Router: logits, top-K and routing weights.
//
// "PagedWeight", §2.1: the router assigns routing weights to the E experts and
// selects the top K for each token. Logits are accumulated in fp64: an fp16 or
// bf16 activation times an fp32 router weight is exact in fp64, and every
// logit is summed in one fixed order (per-lane partials over a fixed set of
// hidden indices, then a butterfly reduction whose pairwise adds are
// commutative), so two identical router rows give bit-identical logits and the
// lower expert index wins the tie. The routing weights are the softmax over
// all experts restricted to the K winners and renormalised, which equals a
// softmax over the K winning logits.
//
// Mapping: one workgroup (8 waves) per token. Wave w scores experts w, w+8,
// ..., EB at a time so that the router-row loads of EB experts are in flight
// together; lane l owns hidden indices 4l + 256i + {0..3}, holds the token's
// activations for them (exact in fp32, widened to fp64 per product) and reads
// the matching float4 pieces of each router row (one coalesced 1 KiB access
// per wave per piece).
#include "mpb_device.h"
#include "mpb_internal.h"

namespace mpb {

constexpr int kEMax = 512;   // experts supported by the LDS logit row
constexpr int kRouteWaves = 8;

template <int XDT>
__device__ __forceinline__ float x_to_f32(uint16_t v) {
  if constexpr (XDT == 0) return (float)__builtin_bit_cast(_Float16, v);
  else return __builtin_bit_cast(float, (uint32_t)v << 16);
}

__device__ __forceinline__ bool better(double v, int i, double bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

template <int XDT, int NPC, int EB>
__global__ __launch_bounds__(64 * kRouteWaves) void k_route(const uint16_t* __restrict__ X,
                                                            const float* __restrict__ W,
                                                            const float* __restrict__ bias, int T, int H,
                                                            int E, int K, int32_t* __restrict__ idx_out,
                                                            float* __restrict__ w_out) {
  __shared__ double lg[kEMax];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const uint16_t* xr = X + (size_t)t * H;
  float4 x[NPC];
#pragma unroll
  for (int i = 0; i < NPC; ++i) {
    const int h = 4 * lane + 256 * i;
    const ushort4 v = h < H ? *(const ushort4*)(xr + h) : make_ushort4(0, 0, 0, 0);
    x[i] = make_float4(x_to_f32<XDT>(v.x), x_to_f32<XDT>(v.y), x_to_f32<XDT>(v.z), x_to_f32<XDT>(v.w));
  }
  for (int e0 = w; e0 < E; e0 += kRouteWaves * EB) {
    float4 wv[EB][NPC];
#pragma unroll
    for (int b = 0; b < EB; ++b) {
      const int e = e0 + kRouteWaves * b;
      const float* wr = W + (size_t)(e < E ? e : 0) * H;
#pragma unroll
      for (int i = 0; i < NPC; ++i) {
        const int h = 4 * lane + 256 * i;
        wv[b][i] = (e < E && h < H) ? *(const float4*)(wr + h) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
#pragma unroll
    for (int b = 0; b < EB; ++b) {
      const int e = e0 + kRouteWaves * b;
      double a = 0.0;
#pragma unroll
      for (int i = 0; i < NPC; ++i) {
        a = fma((double)x[i].x, (double)wv[b][i].x, a);
        a = fma((double)x[i].y, (double)wv[b][i].y, a);
        a = fma((double)x[i].z, (double)wv[b][i].z, a);
        a = fma((double)x[i].w, (double)wv[b][i].w, a);
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) a += __shfl_xor(a, off);
      if (lane == 0 && e < E) lg[e] = a + (bias ? (double)bias[e] : 0.0);
    }
  }
  __syncthreads();
  if (w != 0) return;
  // top-K on wave 0; lane holds experts lane + 64i
  uint32_t taken = 0;
  double tv[16];
  int ti[16];
  for (int k = 0; k < K; ++k) {
    double bv = -__builtin_inf();
    int bi = 0x7fffffff;
    for (int i = 0; i < kEMax / 64; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((taken >> i) & 1u)) {
        const double v = lg[e];
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
#pragma unroll
    for (int kk = 0; kk < 16; ++kk)
      if (kk == k) { tv[kk] = bv; ti[kk] = bi; }
  }
  if (lane < K) {
    double sum = 0.0, mine = 0.0;
    int myi = 0;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      if (kk < K) {
        const double ex = exp(tv[kk] - tv[0]);
        sum += ex;
        if (kk == lane) { mine = ex; myi = ti[kk]; }
      }
    }
    idx_out[(size_t)t * K + lane] = myi;
    w_out[(size_t)t * K + lane] = (float)(mine / sum);
  }
}

template <int XDT>
static void launch_route_x(const uint16_t* X, const float* W, const float* bias, int T, int H, int E, int K,
                           int32_t* idx, float* w, hipStream_t s) {
  const int npc = (H + 255) / 256;
  const dim3 grid(T), block(64 * kRouteWaves);
  // EB * NPC float4 pieces of router rows in flight per lane (about 64 VGPRs)
  if (npc <= 4) hipLaunchKernelGGL((k_route<XDT, 4, 4>), grid, block, 0, s, X, W, bias, T, H, E, K, idx, w);
  else if (npc <= 8) hipLaunchKernelGGL((k_route<XDT, 8, 2>), grid, block, 0, s, X, W, bias, T, H, E, K, idx, w);
  else if (npc <= 12) hipLaunchKernelGGL((k_route<XDT, 12, 1>), grid, block, 0, s, X, W, bias, T, H, E, K, idx, w);
  else hipLaunchKernelGGL((k_route<XDT, 16, 1>), grid, block, 0, s, X, W, bias, T, H, E, K, idx, w);
}

hipError_t launch_route(const uint16_t* X, int xdt, const float* W, const float* bias, int T, int H, int E,
                        int K, int32_t* idx, float* w, hipStream_t s) {
  if (xdt == 0) launch_route_x<0>(X, W, bias, T, H, E, K, idx, w, s);
  else launch_route_x<1>(X, W, bias, T, H, E, K, idx, w, s);
  return hipGetLastError();
}

}  // namespace mpb
