// Expert FFN kernels: gate_up + SwiGLU, down, and the weighted combine, one
// launch each (device code in k_ffn_body.h, the gate_up and down kernels and
// their launcher in k_ffn_kernels.h). Items of 32 tokens at decode sizes;
// gate_up takes 128-token items (TC = 4), in the XCD-interleaved order, once
// groups hold 96 tokens on average. Few long down items are split over K
// ranges (one workgroup per range, partial sums added by the combine).
#include "k_ffn_kernels.h"

namespace mpb {

// ---------------------------------------------------------------- combine
// out[t] = sum_k w_tk * y[t, k] + sum_s y[t, K + s], in that order (y in (token, slot) rows).
__global__ __launch_bounds__(256) void k_combine(FfnParams p) {
  const int H4 = p.H >> 2;
  const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (size_t)p.T * H4) return;
  const int t = (int)(gid / H4);
  combine4(p, t, (int)(gid - (size_t)t * H4) * 4);
}

// bf16 activations -> fp16 once per call, one workgroup per token: the
// token's scale shift from its largest finite exponent, then the scaled
// conversion (a plain conversion for tokens within the fp16 range).
__global__ __launch_bounds__(256) void k_x_to_f16(const uint16_t* __restrict__ x, uint16_t* __restrict__ y,
                                                  int32_t* __restrict__ sc, int H) {
  __shared__ int red[4];
  const int t = blockIdx.x, tid = threadIdx.x, n8 = H / 8;
  const uint16_t* xr = x + (size_t)t * H;
  int m = 0;
  for (int i = tid; i < n8; i += 256) m = max(m, max_exp8_bf16(xr + 8 * i));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = max(m, __shfl_xor(m, o));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  const int shift = x_scale_shift(max(max(red[0], red[1]), max(red[2], red[3])));
  if (tid == 0) sc[t] = shift;
  for (int i = tid; i < n8; i += 256) *(f16x8*)(y + (size_t)t * H + 8 * i) = load_x8_bf16(xr + 8 * i, shift);
}

hipError_t launch_x_to_f16(const uint16_t* x, uint16_t* y, int32_t* sc, int T, int H, hipStream_t s) {
  hipLaunchKernelGGL(k_x_to_f16, dim3((unsigned)T), dim3(256), 0, s, x, y, sc, H);
  return hipGetLastError();
}

// LDS per launch: the table region for the highest committed bitwidth plus the
// stage, and at least the epilogue's exchange area (8 waves x 16 x 64 floats).
// Full double-buffered stages pay off where groups hold several 32-token
// items (8 or more tokens per routed expert on average, or 128-token items);
// at smaller batches the larger kernel they need costs more than they save
// (qwen15moe decode: +1 %, with no item taking them).
static bool use_df(const FfnParams& p) { return (long long)p.T * p.K >= 8ll * p.E; }

hipError_t launch_gate_up(const FfnParams& p, int qmax, int tc, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  if (tc == 4 || use_df(p)) return launch_gate_up_df(p, qmax, tc, s, ev0, ev1);
  if (tc != 1) return hipErrorInvalidValue;
  return launch_tc<1, true, true, false>(p, qmax, s, ev0, ev1);
}

hipError_t launch_down(const FfnParams& p, int qmax, bool nt, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  if (!nt || use_df(p)) return launch_down_df(p, qmax, nt, s, ev0, ev1);
  return launch_tc<1, false, true, false>(p, qmax, s, ev0, ev1);
}

hipError_t launch_combine(const FfnParams& p, hipStream_t s) {
  const size_t n = (size_t)p.T * (p.H >> 2);
  hipLaunchKernelGGL(k_combine, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

__global__ void k_set_q(int32_t* q, int i, int b) { q[i] = b; }

hipError_t launch_set_q(int32_t* q, int i, int b, hipStream_t s) {
  hipLaunchKernelGGL(k_set_q, dim3(1), dim3(1), 0, s, q, i, b);
  return hipGetLastError();
}

}  // namespace mpb
