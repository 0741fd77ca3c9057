// Grouped GEMM for large expert groups: the gate_up and down projections of
// groups of at least kWideFrom tokens (prefill-size batches).
//
// "PagedWeight", §3.3 ("Fused Mixed-Precision MoE Kernel"): the expert FFN
// reads each linear-block's bit-planes and centroid table at its committed
// bitwidth and dequantises on the fly. At this size the expert FFN is a dense
// contraction, so a weight tile is dequantised once per K step into LDS and
// shared by every wave of the workgroup, each multiplying it with its own
// token columns on the matrix cores (fp16 operands, fp32 accumulation).
//
// A workgroup (4 waves, one per SIMD) owns one 128-row weight tile of one
// block and one item of the group: 512 tokens (gate_up) or 256 tokens (down,
// whose columns are h hi and h lo of each token, hi + lo carrying h to about
// 22 bits). Per step of 64 K elements:
//   * dequantisation: thread (row r of row group w, word j = lane / 32) reads
//     word j of the step from each of the q plane pages (loaded two steps
//     ahead), assembles the 32 indices of that word and looks them up in the
//     tile's table, writing them to the LDS A stage of the next step (two
//     stages, one barrier per step);
//   * contraction: wave w multiplies all 128 rows (four 32-row blocks from the
//     A stage) with its 128 columns (four 32-column blocks read straight from
//     memory into registers: each substep's operands of the next step are
//     requested into the registers its MFMAs have just read, which frees the
//     registers of a second operand set): sixteen 32x32x16 MFMAs per
//     16 K into 256 accumulators, the dequantisation of the next step placed
//     between them. The K order inside a step is permuted (the same for both
//     operands): 16-K substep ks takes K octets ks and 4 + ks, so that the
//     lanes holding the upper half of an MFMA's K read octets 4..7 and each
//     lane's four operand pieces of a column in a step are 64 contiguous
//     bytes, requested back to back.
// gate_up tiles hold 64 gate rows (blocks 0, 1) and the matching 64 up rows
// (blocks 2, 3), so SiLU(gate) * up is formed in registers. Down adds each
// token's hi and lo accumulators and writes the (token, slot) row of y that the
// combine pass reads.
//
// h of the wide groups goes to panels laid out for down's operand loads: per
// 32-token block of a group and 64-element step of I, 4 KiB of hi then 4 KiB
// of lo, each [substep ks][half g][token r][8 fp16] holding h[r][64 s + 8 (4 g
// + ks) + j]. A down operand load of 64 lanes (token r, half g) then reads 1
// KiB in one piece: a load whose lanes reach 32 rows of a row-major array
// touches 32 cache lines, and those line lookups, not the bytes, bounded the
// loop (measured: the same loads over contiguous bytes took gate_up 586 ->
// 479 us and down 632 -> 535 us at the 4096-token bf16 prefill layer). The
// gate_up epilogue writes the panels with 512-byte stores.
#include <hip/hip_ext.h>

#include "k_ffn_body.h"

namespace mpb {

constexpr uint32_t kWideAStage = 128u * 64u * 2u;  // one A stage: 128 rows x 64 K fp16

__host__ __device__ constexpr uint32_t wide_shmem(int qmax) { return (256u << qmax) + 2u * kWideAStage; }

// A stage: piece o (8 fp16, K elements 8 o .. 8 o + 7 of the step) of tile row
// R sits at 128 R + 16 (o ^ ((R >> 1) & 7)); the 16 lanes of one LDS phase,
// which touch one piece of 16 consecutive rows, then hit distinct banks.
__device__ __forceinline__ uint32_t wa_off(int R, int o) {
  return (uint32_t)R * 128u + ((uint32_t)(o ^ ((R >> 1) & 7)) << 4);
}

// Element offset in the h panels: block blk, step s of I (NSI steps), half hl
// (0 hi, 1 lo), element kk of the step, token r of the block.
__device__ __forceinline__ size_t hpan_off(int blk, int NSI, int s, int hl, int kk, int r) {
  const int o = kk >> 3;  // octet 4 g + ks
  return ((((size_t)blk * NSI + s) * 2 + hl) << 11) + ((o & 3) << 9) + (((o >> 2) * 32 + r) << 3) + (kk & 7);
}

// Item and tile of workgroup blockIdx.x in the wide list of gate_up (gu) or
// down: all tiles of an item run on one XCD (the dispatcher hands workgroup b
// to XCD b % 8), so the item's activations are read through one L2. blk0: the
// item's first h panel block.
__device__ __forceinline__ bool wide_item(const FfnParams& p, bool gu, int ntile, int& tile, Item& m, int& blk0) {
  const int k = blockIdx.x >> 3, li = k / ntile;
  tile = k - li * ntile;
  const int item = 8 * li + (blockIdx.x & 7);
  const int n = p.n_items[gu ? 2 : 3];
  const int v = (gu ? p.items_w : p.items_dnw)[min(item, p.max_items_w - 1)];
  if ((item >= n) | (v < 0)) return false;
  const int tpi = gu ? p.tpi_w : p.tpi_dnw;
  const int e = v >> 16;
  item_fields<false>(p, 2 * e + (gu ? 0 : 1), e, (v & 0xffff) * tpi, tpi, m);
  blk0 = p.wblk[e] + (v & 0xffff) * (tpi >> 5);
  return true;
}

constexpr int kWideWaves = 4;
constexpr int kWideThreads = 64 * kWideWaves;

// Copy a tile's table image (256 << Q bytes) into LDS at byte 0 with direct
// global-to-LDS loads, 1 KiB per wave and load.
template <int Q>
__device__ __forceinline__ void wide_table_image(const uint16_t* img, int w, int lane) {
  const char* src = (const char*)img + 16 * lane;
#pragma unroll
  for (int c = 0; c < (1 << Q) / 4; c += kWideWaves)
    if (c + w < (1 << Q) / 4)
      __builtin_amdgcn_global_load_lds(src + 1024 * (c + w), (lds_void*)(uintptr_t)(1024u * (c + w)), 16, 0, 0);
}

template <int Q, bool GU>
__device__ __forceinline__ void wide_body(const FfnParams& p, const Item& wi, int it, int blk0, uint16_t* lds,
                                          uint32_t tb) {
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 31, g = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Kd = GU ? p.H : p.I;
  const int NC = (Kd / 32 + 3) >> 2;  // 128-element chunks per row in the pages
  const int NS = Kd >> 6;             // steps of 64
  const int nt = wi.nt, base = wi.base;
  char* abuf = (char*)lds + tb;

  // ---- dequantisation role: row group w, row r, word g of the step
  int row0;  // first block row of row group w
  bool live_rows = true;
  if constexpr (GU) {
    row0 = (w >> 1) * p.I + it * 64 + (w & 1) * 32;
  } else {
    row0 = it * 128 + w * 32;
    live_rows = row0 < p.H;
  }
  rsrc_t rs[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q)
    rs[q] = tile_rsrc(wi.planes[q], live_rows ? (size_t)(row0 >> 5) * NC * 512 : 0, live_rows ? NC * 512 : 0);
  // word j = g of half-chunk s of row r: byte (s / 2) 512 + 16 r + 8 (s % 2) + 4 j
  const int voff = 16 * r + 4 * g;
  auto load_words = [&](uint32_t (&P)[Q], int s) {
#pragma unroll
    for (int q = 0; q < Q; ++q)
      P[q] = __builtin_amdgcn_raw_buffer_load_b32(rs[q], (s >> 1) * 512 + 8 * (s & 1) + voff, 0, 0);
  };
  const uint32_t slot = lut_slot(r, w);
  const int R = 32 * w + r;
  uint32_t aw[4];  // the word's four pieces (K octets 4 g .. 4 g + 3 of the step)
#pragma unroll
  for (int i = 0; i < 4; ++i) aw[i] = wa_off(R, 4 * g + i);

  // ---- contraction role: columns 128 w .. 128 w + 127 in four blocks c of 32
  // (gate_up: tokens 128 w + 32 c + r; down: token 64 w + 32 (c / 2) + r, its
  // h hi for even c, h lo for odd c). Tokens past the item read the item's
  // last token (gate_up) or its last panel block (down): in bounds, and those
  // columns are never stored.
  rsrc_t brs;
  uint32_t boff[4];
  constexpr uint32_t bstep = GU ? 128 : 8192;  // bytes from one step's operands to the next
  constexpr uint32_t bks = GU ? 16 : 1024;      // bytes from one substep's operands to the next
  bool cl[4];  // wave-uniform: the column block holds a token of the item
  if constexpr (GU) {
    brs = rows_rsrc(p.xh, (size_t)p.T * p.H * 2);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int t = 128 * w + 32 * c + r;
      cl[c] = 128 * w + 32 * c < nt;
      boff[c] = (uint32_t)p.ptok[base + min(t, nt - 1)] * (uint32_t)p.H * 2u + 64u * g;
    }
  } else {
    const int NSI = p.I >> 6;
    brs = rows_rsrc(p.hpan, ((size_t)blk0 + ((nt + 31) >> 5)) * NSI * 8192);
#pragma unroll
    for (int tc = 0; tc < 2; ++tc) {
      const uint32_t blk = (uint32_t)(blk0 + min(2 * w + tc, (nt - 1) >> 5));
      boff[2 * tc] = blk * (uint32_t)NSI * 8192u + 16u * (uint32_t)lane;
      boff[2 * tc + 1] = boff[2 * tc] + 4096u;
      cl[2 * tc] = cl[2 * tc + 1] = 64 * w + 32 * tc < nt;
    }
  }
  // B[c][ks]: column block c, substep ks = K octet 4 g + ks of the step (the
  // lane's 64 bytes of the row, g = 0 the first half, g = 1 the second; for
  // down, the panel's substep ks).
  // Every load of the K loop is issued unconditionally (column blocks without
  // tokens read the item's last token; steps past the end re-read the last
  // step, plane words past the row read zeros): a load under a branch leaves
  // the compiler an unknown count of loads in flight, and it then waits for
  // all of them, which would expose the full memory latency every step.
  typedef f16x8 Bops[4][4];
  auto load_b1 = [&](Bops& B, int s, int ks) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      B[c][ks] = __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(brs, boff[c] + bks * ks, bstep * s, 0));
  };

  // A operand of row block rb, substep ks: tile row 32 rb + r, piece 4 g + ks
  // (the swizzle does not depend on rb)
  uint32_t ard[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) ard[ks] = wa_off(r, 4 * g + ks);

  // ---- prologue: table image, the first two steps' planes, the first
  // columns; step 0 dequantised before the loop
  wide_table_image<Q>(wi.luts[Q - 3] + (size_t)it * (128u << Q), w, lane);
  uint32_t PR[2][Q];
  load_words(PR[0], 0);
  load_words(PR[1], 1);
  Bops BB;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) load_b1(BB, 0, ks);
  wait_vmem_all();
  __syncthreads();
  {
    uint32_t O[8];
    assemble<Q>(PR[0], O);
#pragma unroll
    for (int i = 0; i < 4; ++i) *(f16x8*)(abuf + aw[i]) = lookup8(O[2 * i], O[2 * i + 1], slot);
  }
  load_words(PR[0], 2);
  __syncthreads();

  f32x16 acc[4][4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[rb][c] = (f32x16){};

  // step s: request step s + 1's columns; multiply step s's stage with step s's
  // columns substep by substep (the A operands of the next substep read ahead),
  // placing the dequantisation of step s + 1 into the other stage between the
  // substeps (assembly, two lookup halves, stores); request step s + 3's
  // planes; one barrier. In the last step the dequantisation fills the idle
  // stage with unused values.
  auto step = [&](int s, uint32_t (&Pn)[Q], Bops& Bc) {
    const char* ab = abuf + (uint32_t)(s & 1) * kWideAStage;
    char* an = abuf + (uint32_t)((s + 1) & 1) * kWideAStage;
    f16x8 A[2][4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) A[0][rb] = *(const f16x8*)(ab + 4096u * rb + ard[0]);
    uint32_t O[8];
    f16x8 d[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks < 3)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) A[(ks + 1) & 1][rb] = *(const f16x8*)(ab + 4096u * rb + ard[ks + 1]);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (!cl[c]) continue;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) acc[rb][c] = mfma32(A[ks & 1][rb], Bc[c][ks], acc[rb][c]);
      }
      // substep ks of the next step, into the registers these MFMAs have read
      load_b1(Bc, min(s + 1, NS - 1), ks);
      if (ks == 0) assemble<Q>(Pn, O);
      if (ks == 1) {
        d[0] = lookup8(O[0], O[1], slot);
        d[1] = lookup8(O[2], O[3], slot);
      }
      if (ks == 2) {
        d[2] = lookup8(O[4], O[5], slot);
        d[3] = lookup8(O[6], O[7], slot);
      }
      if (ks == 3)
#pragma unroll
        for (int i = 0; i < 4; ++i) *(f16x8*)(an + aw[i]) = d[i];
    }
    load_words(Pn, s + 3);
    __syncthreads();
  };
  for (int s0 = 0; s0 < NS; s0 += 2)
    unroll_const<2>([&](auto u) {
      const int s = s0 + u;
      if (s < NS) step(s, PR[(u + 1) % 2], BB);
    });

  // ---- epilogue. acc[rb][c][v] is tile row 32 rb + 8 (v / 4) + 4 g + v % 4,
  // column 32 c + r of the wave's block.
  if constexpr (GU) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int t = 128 * w + 32 * c + r;
      if (t >= nt) continue;
      // a token converted scaled by 2^-sc (bf16 beyond the fp16 range): gate
      // and up scaled back, h carried as h 2^(-2 sc)
      const int sc = p.xsc ? p.xsc[p.ptok[base + t]] : 0;
      const int blk = blk0 + 4 * w + c;  // panel block of token t, which is its row r
#pragma unroll
      for (int rh = 0; rh < 2; ++rh)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          uint16_t hv[4], lv[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float gate = __builtin_amdgcn_ldexpf(acc[rh][c][4 * v4 + k], sc);
            const float up = __builtin_amdgcn_ldexpf(acc[2 + rh][c][4 * v4 + k], sc);
            const split16 h = split_hi_lo(__builtin_amdgcn_ldexpf(silu(gate) * up, -2 * sc));
            hv[k] = __builtin_bit_cast(uint16_t, h.hi);
            lv[k] = __builtin_bit_cast(uint16_t, h.lo);
          }
          uint16_t* hp = p.hpan + hpan_off(blk, p.I >> 6, it, 0, 32 * rh + 8 * v4 + 4 * g, r);
          *(uint64_t*)hp = __builtin_bit_cast(uint64_t, make_ushort4(hv[0], hv[1], hv[2], hv[3]));
          *(uint64_t*)(hp + 2048) = __builtin_bit_cast(uint64_t, make_ushort4(lv[0], lv[1], lv[2], lv[3]));
        }
    }
  } else {
#pragma unroll
    for (int tc = 0; tc < 2; ++tc) {
      const int t = 64 * w + 32 * tc + r;
      if (t >= nt) continue;
      const int sc = p.xsc ? p.xsc[p.ptok[base + t]] : 0;
      float* yrow = p.y + (size_t)p.ent[base + t] * p.H + it * 128 + 4 * g;
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        if (it * 128 + 32 * rb >= p.H) continue;
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          f32x4 o;
#pragma unroll
          for (int k = 0; k < 4; ++k)
            o[k] = __builtin_amdgcn_ldexpf(acc[rb][2 * tc][4 * v4 + k] + acc[rb][2 * tc + 1][4 * v4 + k], 2 * sc);
          *(f32x4*)(yrow + 32 * rb + 8 * v4) = o;
        }
      }
    }
  }
}

// A block whose committed bitwidth is outside 3..qmax (the launch's table
// region was sized for qmax), or a table region not at LDS byte 0, gives NaN
// for the item's outputs of this tile instead of a silently wrong value.
template <bool GU>
__global__ __launch_bounds__(kWideThreads) void k_wide(FfnParams p, int qmax) {
  extern __shared__ __attribute__((aligned(256))) uint16_t lds[];
  const int ntile = GU ? p.I >> 6 : (p.H + 127) >> 7;
  int it, blk0;
  Item wi;
  if (!wide_item(p, GU, ntile, it, wi, blk0)) return;
  const uint32_t tb = 256u << qmax;
  switch (wi.q < 3 || wi.q > qmax || !tables_at_zero(lds) ? 0 : wi.q) {
    case 3: wide_body<3, GU>(p, wi, it, blk0, lds, tb); break;
    case 4: wide_body<4, GU>(p, wi, it, blk0, lds, tb); break;
    case 5: wide_body<5, GU>(p, wi, it, blk0, lds, tb); break;
    case 6: wide_body<6, GU>(p, wi, it, blk0, lds, tb); break;
    case 7: wide_body<7, GU>(p, wi, it, blk0, lds, tb); break;
    case 8: wide_body<8, GU>(p, wi, it, blk0, lds, tb); break;
    default:
      if constexpr (GU) {
        for (int i = threadIdx.x; i < wi.nt * 64; i += blockDim.x) {
          const size_t o = hpan_off(blk0 + (i >> 11), p.I >> 6, it, 0, i & 63, (i >> 6) & 31);
          p.hpan[o] = 0x7e00;  // fp16 NaN
          p.hpan[o + 2048] = 0;
        }
      } else {
        poison_y(p, 0, wi.base, wi.nt, it * 128);
      }
  }
}

hipError_t launch_wide(const FfnParams& p, bool gu, int qmax, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  if (!p.wide_from || p.max_items_w <= 0) return hipSuccess;
  static unsigned long long lds_raised[2] = {0, 0};  // devices on which each kernel's LDS limit is raised
  const void* fn = gu ? (const void*)k_wide<true> : (const void*)k_wide<false>;
  const hipError_t e = raise_lds_limit(fn, (int)wide_shmem(8), lds_raised[gu ? 0 : 1]);
  if (e != hipSuccess) return e;
  const int ntile = gu ? p.I >> 6 : (p.H + 127) >> 7;
  const dim3 grid((unsigned)((p.max_items_w + 7) / 8 * 8 * ntile));
  const size_t shmem = wide_shmem(qmax);
  if (gu) {
    if (ev0 || ev1)
      hipExtLaunchKernelGGL(k_wide<true>, grid, dim3(kWideThreads), shmem, s, ev0, ev1, 0, p, qmax);
    else
      hipLaunchKernelGGL(k_wide<true>, grid, dim3(kWideThreads), shmem, s, p, qmax);
  } else {
    if (ev0 || ev1)
      hipExtLaunchKernelGGL(k_wide<false>, grid, dim3(kWideThreads), shmem, s, ev0, ev1, 0, p, qmax);
    else
      hipLaunchKernelGGL(k_wide<false>, grid, dim3(kWideThreads), shmem, s, p, qmax);
  }
  return hipGetLastError();
}

}  // namespace mpb
