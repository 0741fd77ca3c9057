// Router: logits, top-K and routing weights (one launch for small batches,
// two otherwise).
//
// "PagedWeight", §2.1: the router assigns routing weights to the E experts and
// selects the top K for each token. Logits are accumulated in fp64: an fp16 or
// bf16 activation times an fp32 router weight is exact in fp64, and every
// logit is summed in one fixed order (per-lane partials over a fixed set of
// hidden indices, then the 64 lane partials in lane order), so two identical
// router rows give bit-identical logits and the lower expert index wins the
// tie. The routing weights are the softmax over all experts restricted to the
// K winners and renormalised, which equals a softmax over the K winning logits.
//
// k_route_logits: one wave per (8-token tile, EW-expert group). Lane l owns
// hidden indices 4l + 256i + {0..3}; per piece i it reads one float4 of each
// of the group's router rows and one ushort4 of each of the tile's tokens
// (coalesced 1 KiB / 512 B accesses per wave) and keeps 8 x EW fp64 partial
// sums. The partials are transposed through LDS and each (token, expert) sum
// is finished by one lane. Logits go to the workspace ([T][E] fp64).
//
// k_route_topk: one wave per token. Expert e is selected at position
// rank(e) = #{experts that beat it} when rank(e) < K. The logits' rounding
// error is bounded from norms the logits kernels store beside them; a top-K
// that the bound cannot certify is ranked again on exact logits
// (topk_certify), so the selection and its order are those of the exact
// logits, ties to the lower index.
//
// k_route_small (batches of up to kSmallT tokens, router matrices of up to
// kSmallEH entries): one workgroup per token sums each of its logits whole
// (wave w of 8 takes experts 2w, 2w + 1, 2w + 16, ...; lane l the hidden
// indices 4l + 256i + {0..3} in order, then the 64 lane sums in a butterfly,
// whose pairwise sums are the same on every lane) and ranks them in LDS, so
// the batch needs neither the partial-sum workspace nor a second launch. Each workgroup streams the whole router matrix through its CU, which
// only pays for small matrices (measured: 8 x 256 layer 4.4 us faster per step;
// with 60 x 2048 the one launch took 29 us against 12.5 us for two).
#include "k_route_body.h"

namespace mpb {

constexpr int kEMaxTopk = 512;
constexpr int kSmallT = 128;    // batches up to this size take k_route_small ...
constexpr int kSmallEH = 16384;  // ... when the router matrix has at most this many entries (64 KiB)
constexpr int kSmallEW = 2;   // experts summed together per wave (independent loads in flight)

template <int XDT, int EW, int NPC>
__global__ __launch_bounds__(256) void k_route_logits(const uint16_t* __restrict__ X, const float* __restrict__ W,
                                                      int T, int H, int E, int ks, double* __restrict__ logits) {
  __shared__ double part[4][kTT * EW * 65];  // +1 column: the summing lanes read rows without bank conflicts
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const long long u = (long long)blockIdx.x * 4 + w;
  logits_partials<XDT, EW, NPC>(X, W, T, H, E, ks, u, lane, part[w], route_ws_l1(logits, ks, T, E));
  __syncthreads();
  logits_sum<EW>(T, E, ks, u, lane, part[w], logits);
}

template <int XDT>
__global__ __launch_bounds__(256) void k_route_logits_mfma(const uint16_t* __restrict__ X, const float* __restrict__ W,
                                                           int T, int H, int E, double* __restrict__ logits) {
  logits_tile_mfma<XDT>(X, W, T, H, E, (long long)blockIdx.x * 4 + (threadIdx.x >> 6), threadIdx.x & 63, logits,
                        route_ws_l1(logits, 1, T, E));
}

template <int XDT, int KP>
__global__ __launch_bounds__(256) void k_route_topk(const double* __restrict__ logits, const uint16_t* __restrict__ X,
                                                    const float* __restrict__ W, const float* __restrict__ bias,
                                                    int ks, int T, int H, int E, int K, int32_t* __restrict__ idx_out,
                                                    float* __restrict__ w_out) {
  __shared__ double lg[4][kEMaxTopk];
  __shared__ double sel_v[4][17];
  __shared__ int sel_i[4][17];
  __shared__ unsigned nmaxw[4];
  __shared__ ExactScratch sc[4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + w;
  const float xi = topk_gather<XDT, false, KP>(logits, X, bias, ks, t, T, H, E, lane, threadIdx.x, 256, lg[w],
                                               &nmaxw[w]);
  const float nm = __uint_as_float(nmaxw[w]);
  topk_load<false, KP>(logits, bias, ks, t, T, E, lane, lg[w]);
  __syncthreads();
  topk_rank(t, T, E, K, lane, lg[w], sel_v[w], sel_i[w]);
  __syncthreads();
  topk_certify<XDT>(X, W, bias, t, T, H, E, K, lane, lg[w], logit_bound(H, xi, nm),
                    sel_v[w], sel_i[w], sc[w]);
  topk_finish(t, T, K, lane, sel_v[w], sel_i[w], idx_out, w_out);
}

template <int XDT>
__global__ __launch_bounds__(512) void k_route_small(const uint16_t* __restrict__ X, const float* __restrict__ W,
                                                     const float* __restrict__ bias, int T, int H, int E, int K,
                                                     int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  __shared__ double lg[kEMaxTopk];
  __shared__ double sel_v[17];
  __shared__ int sel_i[17];
  __shared__ unsigned nmax;
  __shared__ ExactScratch sc;
  const int t = blockIdx.x, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (threadIdx.x == 0) nmax = 0u;
  __syncthreads();
  const uint16_t* x = X + (size_t)t * H;
  float xm = 0.0f;  // max-norm of the token (every wave covers all of it)
  for (int e0 = w * kSmallEW; e0 < E; e0 += 8 * kSmallEW) {
    double a[kSmallEW], n1[kSmallEW];
#pragma unroll
    for (int j = 0; j < kSmallEW; ++j) a[j] = n1[j] = 0.0;
#pragma unroll 8
    for (int h = 4 * lane; h < H; h += 256) {
      const ushort4 xv = *(const ushort4*)(x + h);
      const float f0 = x_to_f32<XDT>(xv.x), f1 = x_to_f32<XDT>(xv.y), f2 = x_to_f32<XDT>(xv.z),
                  f3 = x_to_f32<XDT>(xv.w);
      xm = fmaxf(xm, fmaxf(fmaxf(fabsf(f0), fabsf(f1)), fmaxf(fabsf(f2), fabsf(f3))));
      const double x0 = f0, x1 = f1, x2 = f2, x3 = f3;
#pragma unroll
      for (int j = 0; j < kSmallEW; ++j) {
        const float4 wv = *(const float4*)(W + (size_t)min(e0 + j, E - 1) * H + h);
        a[j] += x0 * (double)wv.x;
        a[j] += x1 * (double)wv.y;
        a[j] += x2 * (double)wv.z;
        a[j] += x3 * (double)wv.w;
        n1[j] += ((double)fabsf(wv.x) + (double)fabsf(wv.y)) + ((double)fabsf(wv.z) + (double)fabsf(wv.w));
      }
    }
#pragma unroll
    for (int j = 0; j < kSmallEW; ++j) {
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        a[j] += __shfl_xor(a[j], o);
        n1[j] += __shfl_xor(n1[j], o);
      }
      if (lane == 0 && e0 + j < E) {
        lg[e0 + j] = a[j] + (bias ? (double)bias[e0 + j] : 0.0);
        atomicMax(&nmax, __float_as_uint((float)(n1[j] + (bias ? fabs((double)bias[e0 + j]) : 0.0))));
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) xm = fmaxf(xm, __shfl_xor(xm, o));
  __syncthreads();
  if (w == 0) topk_rank(t, T, E, K, lane, lg, sel_v, sel_i);
  __syncthreads();
  if (w == 0)
    topk_certify<XDT>(X, W, bias, t, T, H, E, K, lane, lg, logit_bound(H, xm, __uint_as_float(nmax)), sel_v, sel_i,
                      sc);
  if (w == 0) topk_finish(t, T, K, lane, sel_v, sel_i, idx_out, w_out);
}

// Routing mass of one batch ("PagedWeight", §2.1, Eq. 1): m_e = the routing
// weight routed experts' entries carry, summed over tokens and top-K slots,
// over the weight of all entries. One workgroup per expert; each thread sums a
// fixed strided subset of the entries in fp64, and the partials are reduced in
// a fixed tree, so the result is the same on every run. Entries whose expert id
// is out of range count in neither sum.
__global__ __launch_bounds__(256) void k_routing_mass(const int32_t* __restrict__ idx, const float* __restrict__ w,
                                                      int TK, int E, double* __restrict__ mass) {
  __shared__ double red[2][4];
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  double num = 0.0, den = 0.0;
  for (int j = tid; j < TK; j += 256) {
    const int x = idx[j];
    const double r = (double)w[j];
    if (x >= 0 && x < E) {
      den += r;
      if (x == e) num += r;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    num += __shfl_xor(num, o);
    den += __shfl_xor(den, o);
  }
  if (lane == 0) {
    red[0][wv] = num;
    red[1][wv] = den;
  }
  __syncthreads();
  if (tid == 0) {
    const double n = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
    const double d = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
    mass[e] = d > 0.0 ? n / d : 0.0;
  }
}

hipError_t launch_routing_mass(const int32_t* idx, const float* w, int T, int E, int K, double* mass,
                               hipStream_t s) {
  hipLaunchKernelGGL(k_routing_mass, dim3(E), dim3(256), 0, s, idx, w, T * K, E, mass);
  return hipGetLastError();
}

// [ks][T][E] fp64 logit parts and [ks][E] row 1-norms; ks <= 8 on the vector
// path (it depends on H, which the size query does not take), 1 on the
// matrix-core path
size_t route_workspace_bytes(int T, int E) {
  const size_t ks = logits_use_mfma(T, E) ? 1 : kMaxParts;
  return (ks * ((size_t)T * E + E) * 8 + 255) / 256 * 256;
}

template <int XDT>
static void launch_logits(const uint16_t* X, const float* W, int T, int H, int E, int ks, double* lg, hipStream_t s) {
  // large batches: 16 x 16 tiles on the fp64 matrix cores once there are
  // enough tiles to fill the chip
  const long long tiles = (long long)((T + 15) / 16) * ((E + 15) / 16);
  if (logits_use_mfma(T, E)) {
    hipLaunchKernelGGL(k_route_logits_mfma<XDT>, dim3((unsigned)((tiles + 3) / 4)), dim3(256), 0, s, X, W, T, H, E,
                       lg);
    return;
  }
  // experts per wave: grow the group (more reuse of each activation load) only
  // while the launch keeps at least 2048 waves
  const long long ntt = (T + kTT - 1) / kTT;
  const int ew = ntt * ks * ((E + 3) / 4) >= 2048 ? 4 : ntt * ks * ((E + 1) / 2) >= 2048 ? 2 : 1;
  const long long units = ntt * ((E + ew - 1) / ew) * ks;
  const dim3 grid((unsigned)((units + 3) / 4)), block(256);
  // pieces per pass: all of a part when it fits the registers (EW = 1: 8, EW = 2: 4, EW = 4: 2); a
  // pass never loads more pieces than a part has
  const int ppk = ((H + 255) / 256 + ks - 1) / ks;
  if (ew == 4) hipLaunchKernelGGL((k_route_logits<XDT, 4, 2>), grid, block, 0, s, X, W, T, H, E, ks, lg);
  else if (ew == 2) hipLaunchKernelGGL((k_route_logits<XDT, 2, 4>), grid, block, 0, s, X, W, T, H, E, ks, lg);
  else if (ppk <= 2) hipLaunchKernelGGL((k_route_logits<XDT, 1, 2>), grid, block, 0, s, X, W, T, H, E, ks, lg);
  else if (ppk <= 4) hipLaunchKernelGGL((k_route_logits<XDT, 1, 4>), grid, block, 0, s, X, W, T, H, E, ks, lg);
  else hipLaunchKernelGGL((k_route_logits<XDT, 1, 8>), grid, block, 0, s, X, W, T, H, E, ks, lg);
}

hipError_t launch_route(const uint16_t* X, int xdt, const float* W, const float* bias, int T, int H, int E,
                        int K, int32_t* idx, float* w, double* lg, hipStream_t s) {
  if (T <= kSmallT && (long long)E * H <= kSmallEH) {
    if (xdt == 0) hipLaunchKernelGGL(k_route_small<0>, dim3(T), dim3(512), 0, s, X, W, bias, T, H, E, K, idx, w);
    else hipLaunchKernelGGL(k_route_small<1>, dim3(T), dim3(512), 0, s, X, W, bias, T, H, E, K, idx, w);
    return hipGetLastError();
  }
  const int ks = route_ksplit(T, H, E);
  if (xdt == 0) launch_logits<0>(X, W, T, H, E, ks, lg, s);
  else launch_logits<1>(X, W, T, H, E, ks, lg, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((T + 3) / 4)), block(256);
  // the matrix-core path has one hidden part: its top-K loads no others
  if (ks == 1) {
    if (xdt == 0) hipLaunchKernelGGL((k_route_topk<0, 1>), grid, block, 0, s, lg, X, W, bias, ks, T, H, E, K, idx, w);
    else hipLaunchKernelGGL((k_route_topk<1, 1>), grid, block, 0, s, lg, X, W, bias, ks, T, H, E, K, idx, w);
  } else {
    if (xdt == 0)
      hipLaunchKernelGGL((k_route_topk<0, kMaxParts>), grid, block, 0, s, lg, X, W, bias, ks, T, H, E, K, idx, w);
    else
      hipLaunchKernelGGL((k_route_topk<1, kMaxParts>), grid, block, 0, s, lg, X, W, bias, ks, T, H, E, K, idx, w);
  }
  return hipGetLastError();
}

}  // namespace mpb
