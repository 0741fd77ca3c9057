// Bit-plane packer and the dequantisation test kernel.
//
// The packer turns a block's canonical planes (bit j of word w = element
// 32w+j, plane 0 = code MSB) into the plane-major packed pages the FFN kernels
// read: a block at bitwidth q touches its first q pages and nothing else
// ("PagedWeight", §3.1: one bit-plane is one weight page; §2.2: the top planes
// form the lower-bitwidth weights).
#include "mpb_device.h"
#include "mpb_internal.h"

namespace mpb {

struct PagePtrs {
  uint32_t* p[8];
};
struct CPagePtrs {
  const uint32_t* p[8];
};

// One thread per (plane, row, word): each of the word's 32 element bits moves
// to its packed position (packed_pos). Runs once per weight load.
__global__ __launch_bounds__(256) void k_pack(const uint32_t* __restrict__ canon, int N, int W,
                                              PagePtrs pages) {
  const size_t per_plane = (size_t)N * W;
  const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= 8 * per_plane) return;
  const int p = (int)(gid / per_plane);
  const size_t rem = gid - (size_t)p * per_plane;
  const int n = (int)(rem / W), w = (int)(rem % W);
  const uint32_t c = canon[gid];
  uint32_t out = 0;
#pragma unroll
  for (int e = 0; e < 32; ++e) out |= ((c >> e) & 1u) << packed_pos(e, p);
  pages.p[p][((size_t)(n >> 5) * W + w) * 32 + (n & 31)] = out;
}

hipError_t launch_pack(const uint32_t* canon, int N, int Kd, uint32_t* const* pages, hipStream_t s) {
  PagePtrs pp;
  for (int p = 0; p < 8; ++p) pp.p[p] = pages[p];
  const int W = Kd / 32;
  const size_t n = (size_t)8 * N * W;
  const unsigned grid = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(k_pack, dim3(grid), dim3(256), 0, s, canon, N, W, pp);
  return hipGetLastError();
}

// One wave per 32-row tile: stage the tile's Q-bit tables in LDS, then run the
// FFN kernels' assemble + lookup over every word and write fp16 weights in
// canonical element order.
template <int Q>
__device__ void dequant_tile(const CPagePtrs& pages, const uint16_t* __restrict__ lut, int N, int W,
                             uint16_t* __restrict__ out, uint16_t* lds) {
  const int lane = threadIdx.x, r = lane & 31, g = lane >> 5;
  const int row0 = blockIdx.x * 32;
  stage_luts<Q>(lds, lut, row0, lane, 0);
  __syncthreads();
  const uint32_t slot = lut_slot(r, 0);
  const int Kd = W * 32;
  for (int w0 = 0; w0 < W; w0 += 2) {
    const int word = w0 + g;
    uint32_t P[Q];
#pragma unroll
    for (int p = 0; p < Q; ++p) P[p] = pages.p[p][((size_t)blockIdx.x * W + word) * 32 + r];
    uint32_t O[8];
    assemble<Q>(P, O);
    uint16_t* dst = out + (size_t)(row0 + r) * Kd + word * 32;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const f16x8 a = lookup8(lds, O[2 * m], O[2 * m + 1], slot);
      *(f16x8*)(dst + 8 * m) = a;  // elements 8m..8m+7
    }
  }
}

__global__ __launch_bounds__(64) void k_dequant(CPagePtrs pages, const uint16_t* __restrict__ lut, int N,
                                                int W, int b, uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(256))) uint16_t lds[32768];
  switch (b) {
    case 3: dequant_tile<3>(pages, lut, N, W, out, lds); break;
    case 4: dequant_tile<4>(pages, lut, N, W, out, lds); break;
    case 5: dequant_tile<5>(pages, lut, N, W, out, lds); break;
    case 6: dequant_tile<6>(pages, lut, N, W, out, lds); break;
    case 7: dequant_tile<7>(pages, lut, N, W, out, lds); break;
    case 8: dequant_tile<8>(pages, lut, N, W, out, lds); break;
    default: break;
  }
}

hipError_t launch_dequant(const uint32_t* const* pages, const uint16_t* lut, int N, int Kd, int b,
                          uint16_t* out, hipStream_t s) {
  CPagePtrs pp;
  for (int p = 0; p < 8; ++p) pp.p[p] = p < b ? pages[p] : nullptr;
  hipLaunchKernelGGL(k_dequant, dim3(N / 32), dim3(64), 0, s, pp, lut, N, Kd / 32, b, out);
  return hipGetLastError();
}

}  // namespace mpb
