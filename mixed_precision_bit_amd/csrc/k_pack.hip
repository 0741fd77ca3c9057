// Bit-plane packer and the dequantisation test kernel.
//
// The packer turns a block's canonical planes (bit j of word w = element
// 32w+j, plane 0 = code MSB) into the plane-major packed pages the FFN kernels
// read: a block at bitwidth q touches its first q pages and nothing else
// ("PagedWeight", §3.1: one bit-plane is one weight page; §2.2: the top planes
// form the lower-bitwidth weights).
#include "k_ffn_body.h"
#include "mpb_device.h"
#include "mpb_internal.h"

namespace mpb {

struct PagePtrs {
  uint32_t* p[8];
};
struct CPagePtrs {
  const uint32_t* p[8];
};

// One thread per (plane, row, padded word): each of the word's 32 element bits
// moves to its packed position (packed_pos); words past the row end are zero.
// Runs once per weight load.
__global__ __launch_bounds__(256) void k_pack(const uint32_t* __restrict__ canon, int N, int W, int NC,
                                              PagePtrs pages) {
  const int WP = 4 * NC;  // padded words per row
  const size_t per_plane = (size_t)N * WP;
  const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= 8 * per_plane) return;
  const int p = (int)(gid / per_plane);
  const size_t rem = gid - (size_t)p * per_plane;
  const int n = (int)(rem / WP), w = (int)(rem % WP);
  uint32_t out = 0;
  if (w < W) {
    const uint32_t c = canon[((size_t)p * N + n) * W + w];
#pragma unroll
    for (int e = 0; e < 32; ++e) out |= ((c >> e) & 1u) << packed_pos(e, p);
  }
  uint32_t* dst = p == 0 ? pages.p[0] : p == 1 ? pages.p[1] : p == 2 ? pages.p[2] : p == 3 ? pages.p[3]
                : p == 4 ? pages.p[4] : p == 5 ? pages.p[5] : p == 6 ? pages.p[6] : pages.p[7];
  dst[page_word(n, w, NC)] = out;
}

hipError_t launch_pack(const uint32_t* canon, int N, int Kd, uint32_t* const* pages, hipStream_t s) {
  PagePtrs pp;
  for (int p = 0; p < 8; ++p) pp.p[p] = pages[p];
  const int W = Kd / 32, NC = page_chunks(Kd);
  const size_t n = (size_t)8 * N * 4 * NC;
  const unsigned grid = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(k_pack, dim3(grid), dim3(256), 0, s, canon, N, W, NC, pp);
  return hipGetLastError();
}

// Table images. The FFN kernels hold, per workgroup, the b-bit tables of 128
// rows (four waves of 32) with entry u of row r of wave w at byte
// u * 256 + lut_slot(r, w), u the bit-reversed index. An image is that LDS
// content for every workgroup tile, tile after tile (256 << b bytes each), so a
// workgroup fills its table region with plain 16-byte copies. Wave w of tile t
// holds rows
//   kind 0 (gate_up, N = 2I): (w / 2) * N/2 + 64 t + 32 (w % 2) + r
//   kind 1 (down,    N = H ): 128 t + 32 w + r   (zero past N)
// One thread per image fp16.
__global__ __launch_bounds__(256) void k_pack_table(const uint16_t* __restrict__ lut, int kind, int N, int b,
                                                    uint16_t* __restrict__ img, size_t total) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int j = (int)(i & 127);                 // fp16 slot inside a 256-byte entry line
  const size_t tu = i >> 7;
  const int u = (int)(tu & ((1u << b) - 1));     // bit-reversed index
  const int t = (int)(tu >> b);                  // tile
  const int wh = j >> 6, rem = j & 63, r = rem >> 1, wl = rem & 1, w = 2 * wh + wl;
  const int row = kind == 0 ? wh * (N / 2) + 64 * t + 32 * wl + r : 128 * t + 32 * w + r;
  const uint32_t c = __builtin_bitreverse32((uint32_t)u) >> (32 - b);
  img[i] = row < N ? lut[(size_t)row * (1u << b) + c] : (uint16_t)0;
}

hipError_t launch_pack_table(const uint16_t* lut, int kind, int N, int b, uint16_t* img, hipStream_t s) {
  const size_t total = (size_t)((N + 127) / 128) * ((size_t)128 << b);
  hipLaunchKernelGGL(k_pack_table, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, lut, kind, N, b, img,
                     total);
  return hipGetLastError();
}

// One wave per 32-row tile: stage the tile's Q-bit tables in LDS, then run the
// FFN kernels' assemble + lookup over every word and write fp16 weights in
// canonical element order.
template <int Q>
__device__ void dequant_tile(const CPagePtrs& pages, const uint16_t* __restrict__ lut, int W,
                             uint16_t* __restrict__ out, uint16_t* lds) {
  const int lane = threadIdx.x, r = lane & 31, g = lane >> 5;
  const int row0 = blockIdx.x * 32;
  const int NC = (W + 3) / 4, Kd = W * 32;
  stage_luts<Q>(lds, lut, row0, lane, 0);
  __syncthreads();
  const uint32_t slot = lut_slot(r, 0);
  for (int c = g; c < NC; c += 2) {
    uint4 P4[Q];
#pragma unroll
    for (int p = 0; p < Q; ++p)
      P4[p] = *(const uint4*)(pages.p[p] + page_word(row0 + r, 4 * c, NC));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int word = 4 * c + j;
      if (word >= W) break;
      uint32_t P[Q];
#pragma unroll
      for (int p = 0; p < Q; ++p) P[p] = j == 0 ? P4[p].x : j == 1 ? P4[p].y : j == 2 ? P4[p].z : P4[p].w;
      uint32_t O[8];
      assemble<Q>(P, O);
      uint16_t* dst = out + (size_t)(row0 + r) * Kd + word * 32;
#pragma unroll
      for (int m = 0; m < 4; ++m) *(f16x8*)(dst + 8 * m) = lookup8(O[2 * m], O[2 * m + 1], slot);
    }
  }
}

__global__ __launch_bounds__(64) void k_dequant(CPagePtrs pages, const uint16_t* __restrict__ lut, int W, int b,
                                                uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(256))) uint16_t lds[32768];
  switch (tables_at_zero(lds) ? b : 0) {
    case 3: dequant_tile<3>(pages, lut, W, out, lds); break;
    case 4: dequant_tile<4>(pages, lut, W, out, lds); break;
    case 5: dequant_tile<5>(pages, lut, W, out, lds); break;
    case 6: dequant_tile<6>(pages, lut, W, out, lds); break;
    case 7: dequant_tile<7>(pages, lut, W, out, lds); break;
    case 8: dequant_tile<8>(pages, lut, W, out, lds); break;
    default:  // table region misplaced: NaN rows
      for (int i = threadIdx.x; i < 32 * W * 32; i += 64) out[(size_t)blockIdx.x * 32 * W * 32 + i] = 0x7e00;
  }
}

hipError_t launch_dequant(const uint32_t* const* pages, const uint16_t* lut, int N, int Kd, int b,
                          uint16_t* out, hipStream_t s) {
  CPagePtrs pp;
  for (int p = 0; p < 8; ++p) pp.p[p] = p < b ? pages[p] : nullptr;
  hipLaunchKernelGGL(k_dequant, dim3(N / 32), dim3(64), 0, s, pp, lut, Kd / 32, b, out);
  return hipGetLastError();
}

// Dequantisation through a table image, as the FFN kernels read it: one
// 512-thread workgroup per image tile copies the tile's image to LDS with
// their load_table_image, and wave w < 4 dequantises the rows that wave w of
// an FFN workgroup looks up (kind 0, gate_up: (w / 2) N/2 + 64 t + 32 (w % 2) +
// r; kind 1, down: 128 t + 32 w + r) with table slot lut_slot(r, w), writing
// fp16 weights in canonical element order. Used to check mpb_pack_table's
// images bit for bit against the canonical tables.
template <int Q>
__device__ void dequant_tile_image(const CPagePtrs& pages, const uint16_t* __restrict__ img, int kind, int N, int W,
                                   uint16_t* __restrict__ out) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 31, g = lane >> 5;
  const int t = blockIdx.x, NC = (W + 3) / 4, Kd = W * 32;
  load_table_image<Q>(img + (size_t)t * (128u << Q), w, lane);
  wait_vmem_all();
  __syncthreads();
  if (w >= 4) return;
  const int row = kind == 0 ? (w >> 1) * (N / 2) + 64 * t + 32 * (w & 1) + r : 128 * t + 32 * w + r;
  if (row >= N) return;  // past the last tile's rows (kind 1; whole waves, N % 64 == 0)
  const uint32_t slot = lut_slot(r, w);
  for (int c = g; c < NC; c += 2) {
    uint4 P4[Q];
#pragma unroll
    for (int p = 0; p < Q; ++p) P4[p] = *(const uint4*)(pages.p[p] + page_word(row, 4 * c, NC));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int word = 4 * c + j;
      if (word >= W) break;
      uint32_t P[Q];
#pragma unroll
      for (int p = 0; p < Q; ++p) P[p] = j == 0 ? P4[p].x : j == 1 ? P4[p].y : j == 2 ? P4[p].z : P4[p].w;
      uint32_t O[8];
      assemble<Q>(P, O);
      uint16_t* dst = out + (size_t)row * Kd + word * 32;
#pragma unroll
      for (int m = 0; m < 4; ++m) *(f16x8*)(dst + 8 * m) = lookup8(O[2 * m], O[2 * m + 1], slot);
    }
  }
}

__global__ __launch_bounds__(512) void k_dequant_image(CPagePtrs pages, const uint16_t* __restrict__ img, int kind,
                                                       int N, int W, int b, uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(256))) uint16_t lds[32768];
  switch (tables_at_zero(lds) ? b : 0) {
    case 3: dequant_tile_image<3>(pages, img, kind, N, W, out); break;
    case 4: dequant_tile_image<4>(pages, img, kind, N, W, out); break;
    case 5: dequant_tile_image<5>(pages, img, kind, N, W, out); break;
    case 6: dequant_tile_image<6>(pages, img, kind, N, W, out); break;
    case 7: dequant_tile_image<7>(pages, img, kind, N, W, out); break;
    case 8: dequant_tile_image<8>(pages, img, kind, N, W, out); break;
    default:  // table region misplaced: NaN for the tile's rows
      if (threadIdx.x < 256) {
        const int w = threadIdx.x >> 6, t = blockIdx.x;
        for (int r = 0; r < 32; ++r) {
          const int row = kind == 0 ? (w >> 1) * (N / 2) + 64 * t + 32 * (w & 1) + r : 128 * t + 32 * w + r;
          if (row < N)
            for (int i = threadIdx.x & 63; i < W * 32; i += 64) out[(size_t)row * W * 32 + i] = 0x7e00;
        }
      }
  }
}

hipError_t launch_dequant_image(const uint32_t* const* pages, const uint16_t* img, int kind, int N, int Kd, int b,
                                uint16_t* out, hipStream_t s) {
  CPagePtrs pp;
  for (int p = 0; p < 8; ++p) pp.p[p] = p < b ? pages[p] : nullptr;
  const int tiles = kind == 0 ? N / 128 : (N + 127) / 128;
  hipLaunchKernelGGL(k_dequant_image, dim3(tiles), dim3(512), 0, s, pp, img, kind, N, Kd / 32, b, out);
  return hipGetLastError();
}

}  // namespace mpb
