// The gate_up and down kernels and their launcher, as templates: each
// translation unit that launches a variant instantiates it (the variants with
// full double-buffered stages live in their own unit, so that the kernels
// without them keep the smaller code).
#pragma once

#include <hip/hip_ext.h>

#include <algorithm>

#include "k_ffn_body.h"

namespace mpb {

// Stage modes of a work item: 0 one buffer (two barriers per step), 1 two
// 16-token buffers in the stage region (items of <= 16 tokens, one token
// chunk), 2 two full buffers after a 32 KiB table region (blocks below 8
// bits); 1 and 2 need one barrier per step (gate_up) or round (down).
template <int Q, int TC, bool PRV, bool DF>
__device__ __forceinline__ void gu_modes(const FfnParams& p, const Item& wi, int it, uint16_t* lds, uint32_t lb,
                                         int mode) {
  if constexpr (TC == 1) {
    if (mode == 1) {
      gate_up_body<Q, 1, false, true, true, PRV, false>(p, wi, it, lds, lb, threadIdx.x);
      return;
    }
  }
  if constexpr (DF && Q < 8) {
    if (mode == 2) {
      gate_up_body<Q, TC, false, TC == 1, true, PRV, true>(p, wi, it, lds, kDbTable4, threadIdx.x);
      return;
    }
  }
  gate_up_body<Q, TC, false, TC == 1, false, PRV, false>(p, wi, it, lds, lb, threadIdx.x);
}

template <int Q, int TC, bool NT, bool PRV, bool DF>
__device__ __forceinline__ void dn_modes(const FfnParams& p, const Item& wi, int it, uint16_t* lds, uint32_t lb,
                                         int mode, int ksi) {
  if (mode == 1) {
    down_body<Q, TC, false, NT, true, PRV, false>(p, wi, it, lds, lb, threadIdx.x, ksi);
    return;
  }
  if constexpr (DF && Q < 8) {
    if (mode == 2) {
      down_body<Q, TC, false, NT, true, PRV, true>(p, wi, it, lds, kDbTable4, threadIdx.x, ksi);
      return;
    }
  }
  down_body<Q, TC, false, NT, false, PRV, false>(p, wi, it, lds, lb, threadIdx.x, ksi);
}

// pr3: the launch holds LDS for a 3-bit pair table and the stage, so 3-bit
// blocks take the pair-table path. DF: items of more than 16 tokens below 8
// bits take full double-buffered stages (stage mode 2); a separate kernel, so
// that launches without them run the smaller code
template <int TC, bool DF>
__global__ __launch_bounds__(kThreads) void k_gate_up(FfnParams p, int qmax, int pr3) {
  extern __shared__ __attribute__((aligned(256))) uint16_t lds[];
  int it;
  Item wi;
  if (!(TC == 4 ? decode_item_xcd(p, true, p.I >> 6, it, wi) : decode_item(p, true, p.I >> 6, it, wi))) return;
  const int q = wi.q;
  const uint32_t lut_bytes = 256u << qmax;
  // stage: double-buffered (one barrier per step) in two 16-token buffers for
  // items of <= 16 tokens (mode 1), in two full buffers after a 32 KiB table
  // region for larger items of blocks below 8 bits (mode 2), else single
  const int mode = TC == 1 && wi.nt <= kDbTok ? 1 : DF && q < 8 ? 2 : 0;
  switch (q < 3 || q > qmax || !tables_at_zero(lds) ? 0 : q) {
    case 3:
      if (pr3) gu_modes<3, TC, true, DF>(p, wi, it, lds, kPairTableBytes, mode);
      else gu_modes<3, TC, false, DF>(p, wi, it, lds, lut_bytes, mode);
      break;
    case 4: gu_modes<4, TC, false, DF>(p, wi, it, lds, lut_bytes, mode); break;
    case 5: gu_modes<5, TC, false, DF>(p, wi, it, lds, lut_bytes, mode); break;
    case 6: gu_modes<6, TC, false, DF>(p, wi, it, lds, lut_bytes, mode); break;
    case 7: gu_modes<7, TC, false, DF>(p, wi, it, lds, lut_bytes, mode); break;
    case 8: gu_modes<8, TC, false, DF>(p, wi, it, lds, lut_bytes, mode); break;
    default: {
      const size_t o = (size_t)wi.base * p.I + it * 64;
      for (int i = threadIdx.x; i < wi.nt * 64; i += blockDim.x) {
        p.hhi[o + (size_t)(i >> 6) * p.I + (i & 63)] = 0x7e00;  // fp16 NaN
        p.hlo[o + (size_t)(i >> 6) * p.I + (i & 63)] = 0;
      }
    }
  }
}


// NT: non-temporal plane loads (decode-size batches, see load_planes)
template <int TC, bool NT, bool DF>
__global__ __launch_bounds__(kThreads) void k_down(FfnParams p, int qmax, int pr3) {
  extern __shared__ __attribute__((aligned(256))) uint16_t lds[];
  // workgroup b: K range b % dn_split of tile (b / dn_split) % ntile of item
  // (b / dn_split) / ntile
  const int ntile = (p.H + 127) >> 7;
  const int b = blockIdx.x / p.dn_split, ksi = blockIdx.x - b * p.dn_split;
  const int item = b / ntile, it = b - item * ntile;
  Item wi;
  if (!item_of(p, false, item, wi)) return;
  const int q = wi.q;
  const uint32_t lut_bytes = 256u << qmax;
  // round buffers as for gate_up: 16-token halves (mode 1), full buffers after
  // a 32 KiB table region (mode 2), or one buffer
  const int mode = TC == 1 && wi.nt <= kDbTok ? 1 : TC == 1 && DF && q < 8 ? 2 : 0;
  switch (q < 3 || q > qmax || !tables_at_zero(lds) ? 0 : q) {
    case 3:
      if (pr3) dn_modes<3, TC, NT, true, DF>(p, wi, it, lds, kPairTableBytes, mode, ksi);
      else dn_modes<3, TC, NT, false, DF>(p, wi, it, lds, lut_bytes, mode, ksi);
      break;
    case 4: dn_modes<4, TC, NT, false, DF>(p, wi, it, lds, lut_bytes, mode, ksi); break;
    case 5: dn_modes<5, TC, NT, false, DF>(p, wi, it, lds, lut_bytes, mode, ksi); break;
    case 6: dn_modes<6, TC, NT, false, DF>(p, wi, it, lds, lut_bytes, mode, ksi); break;
    case 7: dn_modes<7, TC, NT, false, DF>(p, wi, it, lds, lut_bytes, mode, ksi); break;
    case 8: dn_modes<8, TC, NT, false, DF>(p, wi, it, lds, lut_bytes, mode, ksi); break;
    default: poison_y(p, ksi, wi.base, wi.nt, it * 128);
  }
}


// ev0/ev1 (optional, each may be null): the launch itself records them at the
// kernel's start and end (hipExtLaunchKernelGGL), for timing the kernel alone.
template <int TC, bool GU, bool NT, bool DF>
static hipError_t launch_tc(const FfnParams& p, int qmax, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  static unsigned long long lds_raised = 0;  // devices on which this kernel's LDS limit is raised
  const void* fn;
  if constexpr (GU) fn = (const void*)k_gate_up<TC, DF>;
  else fn = (const void*)k_down<TC, NT, DF>;
  const hipError_t e = raise_lds_limit(fn, (int)ffn_shmem<TC, DF>(8), lds_raised);
  if (e != hipSuccess) return e;
  const size_t shmem = ffn_shmem<TC, DF>(qmax);
  const int pr3 = 1;
  // 128-token items take the XCD-interleaved order (decode_item_xcd)
  const int items = TC == 4 ? (p.max_items + 7) / 8 * 8 : p.max_items;
  if constexpr (GU) {
    if (ev0 || ev1)
      hipExtLaunchKernelGGL((k_gate_up<TC, DF>), dim3(items * (p.I >> 6)), dim3(kThreads), shmem, s, ev0, ev1, 0, p,
                            qmax, pr3);
    else
      hipLaunchKernelGGL((k_gate_up<TC, DF>), dim3(items * (p.I >> 6)), dim3(kThreads), shmem, s, p, qmax, pr3);
  } else {
    const dim3 grid(p.max_items * ((p.H + 127) >> 7) * p.dn_split);
    if (ev0 || ev1)
      hipExtLaunchKernelGGL((k_down<TC, NT, DF>), grid, dim3(kThreads), shmem, s, ev0, ev1, 0, p, qmax, pr3);
    else
      hipLaunchKernelGGL((k_down<TC, NT, DF>), grid, dim3(kThreads), shmem, s, p, qmax, pr3);
  }
  return hipGetLastError();
}

}  // namespace mpb
