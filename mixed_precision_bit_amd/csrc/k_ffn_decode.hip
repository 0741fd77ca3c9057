// Expert FFN kernels: gate_up + SwiGLU, down, and the weighted combine, one
// launch each (the device code is in k_ffn_body.h). Items of 32 tokens at
// decode sizes; gate_up takes 128-token items (TC = 4), in the XCD-interleaved
// order, once groups hold 96 tokens on average. Few long down items are split
// over K ranges (one workgroup per range, partial sums added by the combine).
#include <hip/hip_ext.h>

#include <algorithm>

#include "k_ffn_body.h"

namespace mpb {

// pr3: the launch holds LDS for a 3-bit pair table and the stage, so 3-bit
// blocks take the pair-table path
template <int TC>
__global__ __launch_bounds__(kThreads) void k_gate_up(FfnParams p, int qmax, int pr3) {
  extern __shared__ __attribute__((aligned(256))) uint16_t lds[];
  int e, it, t0, nt;
  if (!(TC == 4 ? decode_item_xcd(p, true, p.I >> 6, e, it, t0, nt) : decode_item(p, true, p.I >> 6, e, it, t0, nt)))
    return;
  const int q = p.q[2 * e];
  const uint32_t lut_bytes = 256u << qmax;
  // double-buffered stage (one barrier per step): items of <= 16 tokens, and
  // every 128-token item below 8 bits (its stage buffers start at kDbTable4)
  const bool db = TC == 1 ? nt <= kDbTok : q < 8;
  const uint32_t lb = TC == 1 ? lut_bytes : kDbTable4;
#define MPB_GU(Q)                                                                         \
  case Q:                                                                                 \
    if (db) gate_up_body<Q, TC, false, TC == 1, true>(p, e, it, t0, nt, lds, lb, threadIdx.x); \
    else gate_up_body<Q, TC>(p, e, it, t0, nt, lds, lut_bytes, threadIdx.x);            \
    break;
  switch (q < 3 || q > qmax || !tables_at_zero(lds) ? 0 : q) {
    case 3:
      if (pr3) {
        if (db) gate_up_body<3, TC, false, TC == 1, true, true>(p, e, it, t0, nt, lds, kPairTableBytes, threadIdx.x);
        else gate_up_body<3, TC, false, TC == 1, false, true>(p, e, it, t0, nt, lds, kPairTableBytes, threadIdx.x);
      } else {
        if (db) gate_up_body<3, TC, false, TC == 1, true>(p, e, it, t0, nt, lds, lb, threadIdx.x);
        else gate_up_body<3, TC>(p, e, it, t0, nt, lds, lut_bytes, threadIdx.x);
      }
      break;
    MPB_GU(4)
    MPB_GU(5)
    MPB_GU(6)
    MPB_GU(7)
    MPB_GU(8)
#undef MPB_GU
    default: {
      const size_t o = (size_t)(p.offsets[e] + t0) * p.I + it * 64;
      for (int i = threadIdx.x; i < nt * 64; i += blockDim.x) {
        p.hhi[o + (size_t)(i >> 6) * p.I + (i & 63)] = 0x7e00;  // fp16 NaN
        p.hlo[o + (size_t)(i >> 6) * p.I + (i & 63)] = 0;
      }
    }
  }
}


// NT: non-temporal plane loads (decode-size batches, see load_planes)
template <int TC, bool NT>
__global__ __launch_bounds__(kThreads) void k_down(FfnParams p, int qmax, int pr3) {
  extern __shared__ __attribute__((aligned(256))) uint16_t lds[];
  // workgroup b: K range b % dn_split of tile (b / dn_split) % ntile of item
  // (b / dn_split) / ntile
  const int ntile = (p.H + 127) >> 7;
  const int b = blockIdx.x / p.dn_split, ksi = blockIdx.x - b * p.dn_split;
  const int item = b / ntile, it = b - item * ntile;
  int e, t0, nt;
  if (!item_of(p, false, item, e, t0, nt)) return;
  const int q = p.q[2 * e + 1];
  const uint32_t lut_bytes = 256u << qmax;
  const bool db = TC == 1 && nt <= kDbTok;
#define MPB_DN(Q)                                                                                       \
  case Q:                                                                                               \
    if (db) down_body<Q, TC, false, NT, TC == 1>(p, e, it, t0, nt, lds, lut_bytes, threadIdx.x, ksi);   \
    else down_body<Q, TC, false, NT>(p, e, it, t0, nt, lds, lut_bytes, threadIdx.x, ksi);              \
    break;
  switch (q < 3 || q > qmax || !tables_at_zero(lds) ? 0 : q) {
    case 3:
      if (pr3) {
        if (db) down_body<3, TC, false, NT, TC == 1, true>(p, e, it, t0, nt, lds, kPairTableBytes, threadIdx.x, ksi);
        else down_body<3, TC, false, NT, false, true>(p, e, it, t0, nt, lds, kPairTableBytes, threadIdx.x, ksi);
      } else {
        if (db) down_body<3, TC, false, NT, TC == 1>(p, e, it, t0, nt, lds, lut_bytes, threadIdx.x, ksi);
        else down_body<3, TC, false, NT>(p, e, it, t0, nt, lds, lut_bytes, threadIdx.x, ksi);
      }
      break;
    MPB_DN(4)
    MPB_DN(5)
    MPB_DN(6)
    MPB_DN(7)
    MPB_DN(8)
#undef MPB_DN
    default: {
      const int n0 = it * 128;
      poison(p.y + (size_t)ksi * p.T * (p.K + p.S) * p.H + (size_t)(p.offsets[e] + t0) * p.H + n0, p.H, nt,
             min(128, p.H - n0));
    }
  }
}

// ---------------------------------------------------------------- combine
// out[t] = sum_k w_tk * y[entry(t,k)] + sum_s y[entry(t,K+s)], in that order.
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
template <int TC>
static size_t ffn_lds_bytes(int qmax) {
  const size_t single = std::max<size_t>((256u << qmax) + stage_bytes<TC>(), kWaves * 16 * 64 * 4);
  // TC > 1: room for the double-buffered stage of blocks below 8 bits
  return TC == 1 ? single : std::max<size_t>(single, kDbTable4 + 2 * stage_bytes<TC>());
}

// ev0/ev1 (optional): the launch itself records them at the kernel's start and
// end (hipExtLaunchKernelGGL), for timing the kernel alone.
template <int TC, bool GU, bool NT = true>
static hipError_t launch_tc(const FfnParams& p, int qmax, hipStream_t s, hipEvent_t ev0 = nullptr,
                            hipEvent_t ev1 = nullptr) {
  static unsigned long long lds_raised = 0;  // devices on which this kernel's LDS limit is raised
  const void* fn;
  if constexpr (GU) fn = (const void*)k_gate_up<TC>;
  else fn = (const void*)k_down<TC, NT>;
  const hipError_t e = raise_lds_limit(fn, (int)std::max<size_t>(ffn_lds_bytes<TC>(8), kPairTableBytes + stage_bytes<TC>()),
                                       lds_raised);
  if (e != hipSuccess) return e;
  // every launch holds room for a 3-bit pair table and the stage (registers,
  // not LDS, bound these kernels' occupancy: two workgroups per CU at one
  // token chunk, one at four), so a block committed at 3 bits later, under a
  // captured graph, still takes the pair path
  constexpr size_t kPairLds = kPairTableBytes + stage_bytes<TC>();
  const size_t shmem = std::max(ffn_lds_bytes<TC>(qmax), kPairLds);
  const int pr3 = 1;
  // 128-token items take the XCD-interleaved order (decode_item_xcd)
  const int items = TC == 4 ? (p.max_items + 7) / 8 * 8 : p.max_items;
  if constexpr (GU) {
    if (ev0 && ev1)
      hipExtLaunchKernelGGL(k_gate_up<TC>, dim3(items * (p.I >> 6)), dim3(kThreads), shmem, s, ev0, ev1, 0, p, qmax,
                            pr3);
    else
      hipLaunchKernelGGL(k_gate_up<TC>, dim3(items * (p.I >> 6)), dim3(kThreads), shmem, s, p, qmax, pr3);
  } else {
    const dim3 grid(p.max_items * ((p.H + 127) >> 7) * p.dn_split);
    if (ev0 && ev1)
      hipExtLaunchKernelGGL((k_down<TC, NT>), grid, dim3(kThreads), shmem, s, ev0, ev1, 0, p, qmax, pr3);
    else
      hipLaunchKernelGGL((k_down<TC, NT>), grid, dim3(kThreads), shmem, s, p, qmax, pr3);
  }
  return hipGetLastError();
}

hipError_t launch_gate_up(const FfnParams& p, int qmax, int tc, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  switch (tc) {
    case 1: return launch_tc<1, true>(p, qmax, s, ev0, ev1);
    case 4: return launch_tc<4, true>(p, qmax, s, ev0, ev1);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_down(const FfnParams& p, int qmax, bool nt, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  return nt ? launch_tc<1, false, true>(p, qmax, s, ev0, ev1) : launch_tc<1, false, false>(p, qmax, s, ev0, ev1);
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
