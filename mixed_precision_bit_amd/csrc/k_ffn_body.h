// Device code of the decode-size expert FFN, shared by the per-phase
// kernels and the fused persistent kernel.
//
//
// "PagedWeight", §3.3: the fused kernel reads the weight pages directly and
// follows the committed bitwidth of every gate_up and down block. Here each
// workgroup reads its block's q_i once from the device page table and runs the
// matching instantiation, so a launch mixes bitwidths freely and a change of
// q_i between launches takes effect on the next launch.
//
// Mapping (MFMA 32x32x16 fp16 -> fp32): a workgroup of 8 waves handles up to
// TC x 32 tokens of one expert (TC = 1 at decode sizes, 4 for prefill-size
// groups) and 128 weight rows: wave w owns row group w % 4 (32 rows) and K
// half w / 4, so two waves share every row's centroid table and the table
// region costs half as much LDS per wave. Lane l holds row l%32; in step s it
// reads half-chunk 2s + l/32 of its K half (2 words = 64 elements) from each
// of the q plane pages: one 8-byte load per page, the 64 lanes of a wave
// covering one 512-byte chunk of 32 rows, issued three steps ahead. Each
// dequantised A operand feeds TC MFMAs, one per 32-token chunk.
//
// The B operand (the tokens) is staged into LDS by the whole workgroup between
// the two barriers of a step and read with ds_read_b128, so the waits of the
// multiply part of a step are on plane loads only (vector-memory completions
// are counted in issue order).
//
// LDS: [centroid tables: 2^qmax * 256 bytes][stage: 2 halves x TC x 32 tokens
// x 256 bytes]. Piece p (16 bytes) of token t of a half sits at p ^ (t % 16),
// so the 16 lanes of one ds_read_b128 phase, which read one piece of 16
// tokens, hit distinct banks.
#pragma once

#include <algorithm>
#include <type_traits>
#include <utility>

#include "mpb_device.h"
#include "mpb_internal.h"

namespace mpb {

constexpr int kTok = kChunkTokens;  // 32 tokens per MFMA column block
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;

// Stage: [K half][token of the item (32 TC)][16 pieces of 16 bytes]; piece p
// of token t sits at p ^ (t % 16).
template <int TC>
__device__ __forceinline__ uint32_t stage_off(int kh, int t, int piece) {
  return (uint32_t)kh * (TC * kTok * 256u) + t * 256u + ((piece ^ (t & 15)) << 4);
}
template <int TC>
constexpr int stage_bytes() { return 2 * TC * kTok * 256; }
// Full double-buffered stages (items of more than 16 tokens, blocks below 8
// bits): the table region (the 7-bit table, or the 3-bit pair table) is 32 KiB,
// the two stage buffers follow it (160 KiB in all for 128-token items)
constexpr uint32_t kDbTable4 = 32768;
static_assert(kDbTable4 + 2 * 2 * 4 * 32 * 256 <= 163840, "two 128-token stage buffers fit the LDS");

// LDS bytes of a per-phase FFN launch for blocks of at most qmax bits: the
// table region and the stage, the SwiGLU exchange, and room for a 3-bit pair
// table and the stage in every launch (registers, not LDS, bound these
// kernels' occupancy: two workgroups per CU at one token chunk, one at four),
// so that a block committed at 3 bits later, under a captured graph, still
// takes the pair path; with DF also the two full stage buffers after a 32 KiB
// table region. The kernels read it too (the room left beside a block's own
// table decides whether its activations stay resident).
template <int TC, bool DF>
__host__ __device__ constexpr uint32_t ffn_shmem(int qmax) {
  constexpr uint32_t kSwiglu = TC * kWaves * 16 * 64 * 4;  // the exchanged accumulators of every chunk
  uint32_t b = (256u << qmax) + (uint32_t)stage_bytes<TC>();
  b = b > kSwiglu ? b : kSwiglu;
  const uint32_t pr = kPairTableBytes + (uint32_t)stage_bytes<TC>();
  b = b > pr ? b : pr;
  const uint32_t df = kDbTable4 + 2u * (uint32_t)stage_bytes<TC>();
  return DF && df > b ? df : b;
}

// Items of at most 16 tokens (TC = 1) split the same region into two stage
// buffers of [K half][16 tokens][16 pieces]; step s reads buffer s % 2 while
// the activations of step s + 1 are written to the other one, so a step needs
// one workgroup barrier instead of two. MFMA columns 16..31 read tokens 0..15
// again; those output columns are never stored.
constexpr int kDbTok = 16;
__device__ __forceinline__ uint32_t stage_off_db(int s, int kh, int t, int piece) {
  return (uint32_t)(s & 1) * (2 * kDbTok * 256u) + (uint32_t)kh * (kDbTok * 256u) + t * 256u +
         ((piece ^ (t & 15)) << 4);
}

// Plane loads go through buffer descriptors, one per plane page, based at the
// wave's 32-row tile and spanning its NC chunks; an offset past the tile
// (padding half-chunks, prefetches past the end) reads zeros without touching
// memory.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t tile_rsrc(const void* page, size_t tile_off, uint32_t bytes) {
  // the operands are wave-uniform; say so, or the compiler wraps every load
  // in a loop over distinct descriptors
  const uint64_t a = (uint64_t)((const char*)page + tile_off);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const int n = __builtin_amdgcn_readfirstlane((int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0, n, 0x00020000);
}

// Copy a tile's table image (256 << Q bytes) into LDS at byte 0 with direct
// global-to-LDS loads: wave w moves 1 KiB pieces w, w + 8, ... (no registers,
// no LDS store instructions). The caller waits for vector memory and
// synchronises the workgroup before the first lookup.
typedef __attribute__((address_space(3))) void lds_void;

template <int Q>
__device__ __forceinline__ void load_table_image(const uint16_t* img, int w, int lane, uint32_t dst = 0) {
  const char* src = (const char*)img + 16 * lane;
#pragma unroll
  for (int c = 0; c < (1 << Q) / 4; c += kWaves)
    if (c + w < (1 << Q) / 4)
      __builtin_amdgcn_global_load_lds(src + 1024 * (c + w), (lds_void*)(uintptr_t)(dst + 1024u * (c + w)), 16, 0,
                                       0);
}

__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// wait until at most N vector memory operations of the wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Half-chunk s of the wave's K half for every plane: lane (r, g) reads the 8
// bytes at chunk cb + s, row r, half g. NT: the loads carry the non-temporal
// hint (cache policy bit 1), for launches that read each plane byte about
// once (decode-size batches: one item per group); the weight stream then does
// not displace activations and tables in the caches (measured: gate_up -4 %,
// down -5 % at the qwen15moe decode size). Where the several items of a group
// re-read its planes (prefill-size batches) the hint costs 5-12 %.
template <int Q, bool NT>
__device__ __forceinline__ void load_planes(uint2 (&P)[Q], const rsrc_t (&rs)[Q], int cb, int s, int voff) {
  constexpr int kPolicy = NT ? 2 : 0;
#pragma unroll
  for (int q = 0; q < Q; ++q)
    P[q] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs[q], (cb + s) * 512 + voff, 0, kPolicy));
}

template <int Q>
__device__ __forceinline__ void word_of(const uint2 (&P2)[Q], int j, uint32_t (&P)[Q]) {
#pragma unroll
  for (int q = 0; q < Q; ++q) P[q] = j == 0 ? P2[q].x : P2[q].y;
}

// Data that one workgroup of the fused kernel hands to another (grouping
// results, h, y, converted activations) is written with device-coherent
// stores (agent-scope relaxed atomics, written through to memory) when CO is
// set, so a unit can hand data to the next with a counter alone, without
// cache write-back. Small shared values (offsets, token ids, counts) are also
// read with device-coherent loads. Bulk data (activations, h, y) is read with
// plain loads: each of its cache lines is written by exactly one unit and
// read only after that unit has counted itself done, so no cache holds an
// older copy of it within the launch (caches start clean at every launch).
// The per-phase kernels use plain accesses throughout.
template <bool CO, typename T>
__device__ __forceinline__ T ld_co(const T* p) {
  if constexpr (CO) return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *p;
}
template <bool CO, typename T>
__device__ __forceinline__ void st_co(T* p, T v) {
  if constexpr (CO) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}
template <bool CO>
__device__ __forceinline__ void st_co16(void* p, uint4 v) {
  if constexpr (CO) {
    st_co<true>((uint64_t*)p, (uint64_t)v.x | ((uint64_t)v.y << 32));
    st_co<true>((uint64_t*)p + 1, (uint64_t)v.z | ((uint64_t)v.w << 32));
  } else {
    *(uint4*)p = v;
  }
}

// Activation pieces staged per thread and step (or round): thread tid stages
// piece p = tid % 16 of token 32 c + tid / 16 of both K halves, c < TC.
template <int TC>
struct StagePlan {
  rsrc_t rs;                // the activation rows (x, or h hi and lo), one descriptor for the wave
  uint32_t off[TC];         // byte offset of the slot's row in rs
  int lim[TC];              // elements of the row the slot reads (0 for token slots >= nt)
  uint32_t dst[2][TC];      // stage byte offsets per K half
  bool wl[TC];              // the wave holds a token slot < nt in chunk c (wave-uniform)
  bool wr;                  // the thread's slots land in the stage (16-token buffers: slots 16..31 do not)
};

// wave-uniform: some token slot of the calling wave's chunk c is live (a wave
// stages the four consecutive slots st & ~3 .. st | 3)
__device__ __forceinline__ bool wave_has_tokens(int c, int st, int nt) {
  return __builtin_amdgcn_readfirstlane(kTok * c + (st & ~3)) < nt;
}

// A window element k of slot c: its byte offset in the rows' descriptor, or
// kNoRow, past any buffer, for elements the slot does not read (the load then
// returns zeros without touching memory), so staging needs no branches.
template <int TC>
__device__ __forceinline__ uint32_t win_off(const StagePlan<TC>& sp, int c, int k) {
  return k < sp.lim[c] ? sp.off[c] + 2u * (uint32_t)k : kNoRow;
}

// The descriptor over [lo, lo + bytes) for the staged rows; bytes < kNoRow
// (rows_fit: the host refuses batches whose activation or h arrays are larger).
__device__ __forceinline__ rsrc_t rows_rsrc(const void* lo, size_t bytes) {
  return tile_rsrc(lo, 0, (uint32_t)bytes);
}

template <int TC>
__device__ __forceinline__ void load_window(uint4 (&v)[2][TC], const StagePlan<TC>& sp, const int (&k)[2]) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int c = 0; c < TC; ++c)
      if (sp.wl[c])
        v[i][c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(sp.rs, win_off(sp, c, k[i]), 0, 0));
}

template <int TC>
__device__ __forceinline__ void store_window(char* stage, const uint4 (&v)[2][TC], const StagePlan<TC>& sp) {
  if (!sp.wr) return;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int c = 0; c < TC; ++c)
      if (sp.wl[c]) *(uint4*)(stage + sp.dst[i][c]) = v[i][c];
}

// Pair-order staging (3-bit pair tables): a piece holds elements e..e+3 and
// e+32..e+35 of a half-chunk interleaved (one from each word per fp16 pair),
// matching the order of lookup_pairs4. k[i] is the first element (e) of the
// piece for K half i.
template <int TC>
__device__ __forceinline__ void load_window_pairs(uint4 (&v)[2][TC], const StagePlan<TC>& sp, const int (&k)[2]) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int c = 0; c < TC; ++c) {
      if (!sp.wl[c]) continue;
      const uint2 a = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(sp.rs, win_off(sp, c, k[i]), 0, 0));
      const uint2 b =
          __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(sp.rs, win_off(sp, c, k[i] + 32), 0, 0));
      v[i][c] = make_uint4(a.x, a.y, b.x, b.y);
    }
}

template <int TC>
__device__ __forceinline__ void store_window_pairs(char* stage, const uint4 (&v)[2][TC], const StagePlan<TC>& sp) {
  if (!sp.wr) return;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int c = 0; c < TC; ++c) {
      if (!sp.wl[c]) continue;
      // (a0 a1 | a2 a3) and (b0 b1 | b2 b3) -> a0 b0, a1 b1, a2 b2, a3 b3
      const uint4 x = v[i][c];
      *(uint4*)(stage + sp.dst[i][c]) =
          make_uint4(__builtin_amdgcn_perm(x.z, x.x, 0x05040100u), __builtin_amdgcn_perm(x.z, x.x, 0x07060302u),
                     __builtin_amdgcn_perm(x.w, x.y, 0x05040100u), __builtin_amdgcn_perm(x.w, x.y, 0x07060302u));
    }
}

// A work item as the FFN bodies take it: group e, the item's first token t0
// within the group and its token count nt, its first grouped entry base =
// offsets[e] + t0, the block's committed bitwidth q, its plane pages and its
// row of table-image pointers (b = 3..8; the body reads the one it needs
// after its first plane loads are out, so that round trip overlaps them).
struct Item {
  int e, t0, nt, base, q;
  const uint32_t* planes[8];
  const uint16_t* const* luts;
};
// The same with the block's row of page pointers instead of the pointers (the
// body reads the ones it needs): for the fused kernel, where eight more live
// pointers would push its waves past their register budget.
struct ItemRow {
  int e, t0, nt, base, q;
  const uint32_t* const* planes;
  const uint16_t* const* luts;
};

// The group-indexed fields of an item: token count, offset, bitwidth and page
// pointers, loaded together (one round trip).
template <bool CO, typename It>
__device__ __forceinline__ void item_fields(const FfnParams& p, int blk, int e, int t0, int tpi, It& m) {
  const int cnt = ld_co<CO>(p.counts + e);
  const int off = ld_co<CO>(p.offsets + e);
  m.q = p.q[blk];
  if constexpr (std::is_same<It, Item>::value) {
#pragma unroll
    for (int k = 0; k < 8; ++k) m.planes[k] = p.planes[blk * 8 + k];
  } else {
    m.planes = p.planes + blk * 8;
  }
  m.luts = p.luts + blk * 6;
  m.e = e;
  m.t0 = t0;
  m.nt = min(cnt - t0, tpi);
  m.base = off + t0;
}

// Item `item` of the gate_up (gu) or down list; false past the end of the
// list. The list entry is read together with the list length (at an index
// clamped to the list's capacity, so the read stays inside it), then the
// group's fields.
__device__ __forceinline__ bool item_of(const FfnParams& p, bool gu, int item, Item& m) {
  const int n = p.n_items[gu ? 0 : 1];
  const int v = (gu ? p.items : p.items_dn)[min(item, p.max_items - 1)];
  // a list entry is never negative (group << 16 | split); testing it too
  // keeps its load ahead of the test, beside the length's
  if ((item >= n) | (v < 0)) return false;
  const int tpi = gu ? p.tpi : p.tpi_dn;
  const int e = v >> 16;
  item_fields<false>(p, 2 * e + (gu ? 0 : 1), e, (v & 0xffff) * tpi, tpi, m);
  return true;
}

// Work item of a launch: workgroup id = item * ntile + tile, so the
// consecutive workgroups that the dispatcher spreads over the chip carry the
// tiles of one item and every workgroup below n_items * ntile has tokens.
__device__ __forceinline__ bool decode_item(const FfnParams& p, bool gu, int ntile, int& tile, Item& m) {
  const int item = blockIdx.x / ntile;
  tile = blockIdx.x - item * ntile;
  return item_of(p, gu, item, m);
}

// The same items for launches that stream activations from L2 (128-token
// items): the dispatcher hands workgroup b to XCD b % 8, and workgroup b takes
// tile k % ntile of item 8 (k / ntile) + b % 8, k = b / 8. All tiles of an
// item then run on one XCD, one after another, so its L2 serves the item's
// activations to every tile; items are dealt to the XCDs in turn, which keeps
// the bitwidth mix (the list is ordered by bitwidth) the same on every XCD.
// Needs a grid of 8 * ceil(max_items / 8) * ntile workgroups.
__device__ __forceinline__ bool decode_item_xcd(const FfnParams& p, bool gu, int ntile, int& tile, Item& m) {
  const int k = blockIdx.x >> 3, li = k / ntile;
  tile = k - li * ntile;
  return item_of(p, gu, 8 * li + (blockIdx.x & 7), m);
}

// K split: a row has HC = Kd / 64 half-chunks; half 0 takes the first HH (even,
// >= HC / 2), half 1 the rest, both in NSW = HH / 2 steps of two half-chunks.
struct KSplit {
  int HC, HH, NSW;
  __device__ KSplit(int Kd) : HC(Kd >> 6), HH((((Kd >> 6) + 1) / 2 + 1) & ~1), NSW((((Kd >> 6) + 1) / 2 + 1) / 2) {}
};

// f(integral_constant<int, 0>) .. f(integral_constant<int, N - 1>) in order:
// an unrolled loop whose index is a constant in every copy (so ring slots
// stay in registers), however large the body
template <typename F, int... I>
__device__ __forceinline__ void each_const(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void unroll_const(F&& f) {
  each_const(f, std::make_integer_sequence<int, N>{});
}

// Steps of plane loads in flight per wave (the plane ring). Three at every
// bitwidth: rings of about 48 VGPRs at each bitwidth (6 steps at 3 and 4
// bits, 4 at 5 and 6) were measured no faster at the qwen15moe decode shape
// (gate_up +1 %, down +2 %) and mixed at the Mixtral shape (4-bit gate_up
// +6 %, 3-bit down -3 %): with three steps in flight the plane stream is not
// what holds these kernels back.
template <int Q, int TC>
constexpr int plane_ring() {
  return 3;
}

// ---------------------------------------------------------------- gate_up
// Waves 0/1 take gate rows c0..c0+31 / c0+32..c0+63, waves 2/3 the matching up
// rows, waves 4..7 the same rows over the second K half. Each dequantised
// A operand feeds TC MFMAs, one per 32-token chunk of the item. After the K
// loop the waves exchange their accumulators through LDS; each then adds the
// halves for a quarter of a row half, applies SiLU(gate) * up and stores h as
// an fp16 (hi, lo) pair (hi + lo carries ~22 significant bits of the fp32
// value into the down projection).
//
// Issue order per step s (vector memory completes in issue order, so a wait
// for one load also waits for every older one): compute on the planes of step
// s, barrier, write the activations of step s+1 (loaded one step earlier) to
// the stage, load the activations of step s+2, load the planes of step s+3,
// barrier. DB: the stage is double-buffered and the first of the two barriers
// is dropped; items of <= 16 tokens (TC = 1) split the stage region into two
// 16-token buffers, 128-token items (TC = 4) of blocks below 8 bits take two
// full stage buffers after a 32 KiB table region (the 8-bit table needs 64 KiB).
//
// PR (3-bit blocks): pair tables. lut_bytes is kPairTableBytes; the
// tile's 3-bit table image is copied to the stage region, expanded into the
// pair table before the first activations are staged, and each step runs
// eight lookup_pairs4 groups over both words of the lane's half-chunk, with
// the activations staged in pair order (piece 8 g' + m: elements 4m..4m+3 of
// both words of half-chunk 2s + g').
template <int Q, int TC, bool CO = false, bool NT = (TC == 1), bool DB = false, bool PR = false, bool DF = false,
          typename It = Item>
__device__ __forceinline__ void gate_up_body(const FfnParams& p, const It& wi, int it, uint16_t* lds,
                                             uint32_t lut_bytes, int tid) {
  static_assert(!PR || Q == 3, "pair tables: 3-bit blocks");
  // DB with one token chunk: two 16-token buffers in the 16 KiB stage region
  // (HALF), or with DF two full 32-token buffers after a 32 KiB table region
  constexpr bool HALF = DB && TC == 1 && !DF;
  const int lane = tid & 63, r = lane & 31, g = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: plane descriptors stay scalar
  const int rg = w & 3, kh = w >> 2;
  const int I = p.I, H = p.H, NC = (H / 32 + 3) >> 2;
  const KSplit ks(H);
  const int c0 = it * 64 + (rg & 1) * 32;
  const int row0 = (rg >> 1) * I + c0;
  const int nt = wi.nt, base = wi.base;
  const uint32_t slot = PR ? pair_slot(r, rg) : lut_slot(r, rg);
  char* stage = (char*)lds + lut_bytes;

  // staging: piece p = 8 g' + 4 j + m of a token holds elements 32 j + 8 m .. + 7
  // of half-chunk 2 s + g' of the K half (PR: piece 8 g' + m, elements 4 m ..
  // 4 m + 3 of both words)
  StagePlan<TC> sp;
  const int st = tid >> 4, spc = tid & 15;
  sp.rs = rows_rsrc(p.xh, (size_t)p.T * H * 2);
  sp.wr = !HALF || st < 16;
  // the token ids are loaded first (the entry of the item's last token stands
  // in for slots past it) and turned into row offsets only after the table
  // and the first planes are requested, so those loads do not wait for them
  int tok[TC];
#pragma unroll
  for (int c = 0; c < TC; ++c) {
    const int t = kTok * c + st;
    tok[c] = ld_co<CO>(p.ptok + base + min(t, nt - 1));
    sp.wl[c] = wave_has_tokens(c, st, nt);
    sp.lim[c] = t < nt ? H : 0;
    sp.dst[0][c] = HALF ? stage_off_db(0, 0, t & 15, spc) : stage_off<TC>(0, t, spc);
    sp.dst[1][c] = HALF ? stage_off_db(0, 1, t & 15, spc) : stage_off<TC>(1, t, spc);
  }
  auto row_offsets = [&]() {
#pragma unroll
    for (int c = 0; c < TC; ++c) sp.off[c] = kTok * c + st < nt ? (uint32_t)tok[c] * (uint32_t)H * 2u : 0u;
  };
  // bf16 input: the epilogue's tokens (column r of each chunk), whose scale
  // shifts it reads; requested now so that the epilogue waits for one load
  int etok[TC];
#pragma unroll
  for (int c = 0; c < TC; ++c) etok[c] = p.xsc ? ld_co<CO>(p.ptok + base + min(kTok * c + r, nt - 1)) : 0;
  // stage byte offset of piece `pc` of token chunk c, row r, in buffer par
  auto rd_off = [&](int par, int c, int pc) -> uint32_t {
    if constexpr (HALF) return stage_off_db(par, kh, r & 15, pc);
    else return (DB ? (uint32_t)par * stage_bytes<TC>() : 0u) + stage_off<TC>(kh, kTok * c + r, pc);
  };
  auto kwin = [&](int s, int (&k)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) k[i] = (i * ks.HH + 2 * s + (spc >> 3)) * 64 + (PR ? 4 : 8) * (spc & 7);
  };
  auto ld_win = [&](uint4 (&v)[2][TC], const int (&k)[2]) {
    if constexpr (PR) load_window_pairs<TC>(v, sp, k);
    else load_window<TC>(v, sp, k);
  };
  auto st_win = [&](char* dst, const uint4 (&v)[2][TC], const int (&k)[2]) {
    if constexpr (PR) store_window_pairs<TC>(dst, v, sp);
    else store_window<TC>(dst, v, sp);
  };
  // DMA (double-buffered stage, natural piece order): the window of step s
  // goes from memory straight into stage buffer par with buffer-to-LDS loads
  // (no registers, no LDS stores). One load moves 1 KiB: lane L writes slot
  // L % 16 of token (L / 16) of the wave's four token rows, so it reads piece
  // (L % 16) ^ (t % 16) of its token t (the stage's swizzle); rows past the
  // item and elements past the row read as zeros.
  constexpr bool DMA = DB && !PR;
  const int pdma = spc ^ (st & 15);
  auto dma_win = [&](int par, int s) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int k = (i * ks.HH + 2 * s + (pdma >> 3)) * 64 + 8 * (pdma & 7);
#pragma unroll
      for (int c = 0; c < TC; ++c) {
        if (!sp.wl[c] || !sp.wr) continue;
        // the wave's first token row (slot 0, before the swizzle)
        const uint32_t row0b = HALF ? (uint32_t)par * (2 * kDbTok * 256u) + (uint32_t)i * (kDbTok * 256u)
                                    : (uint32_t)par * stage_bytes<TC>() + (uint32_t)i * (TC * kTok * 256u);
        const uint32_t dst = lut_bytes + row0b + (uint32_t)(kTok * c + (st & ~3)) * 256u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(sp.rs, (lds_void*)(uintptr_t)__builtin_amdgcn_readfirstlane(dst), 16,
                                                 win_off(sp, c, k), 0, 0, 0);
      }
    }
  };

  // the descriptor of K half 0 ends where half 1 begins, so the prefetches
  // past the half read zeros instead of half 1's pages
  const int cb = kh * (ks.HH >> 1);  // first chunk of the wave's K half
  const int ce = kh ? NC : ks.HH >> 1;
  rsrc_t rs[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) rs[q] = tile_rsrc(wi.planes[q], (size_t)(row0 >> 5) * NC * 512, ce * 512);
  const int voff = 16 * r + 8 * g;

  constexpr int D = plane_ring<Q, TC>();
  uint2 P[D][Q];
  uint4 xr[2][TC];
  int kk[2];
  // PR: the 3-bit image goes to the stage region, which is staged only after
  // the pair table has been built from it
  // step 0's planes first: their pointers are known a round trip before the
  // table's
  load_planes<Q, NT>(P[0], rs, cb, 0, voff);
  load_table_image<Q>(wi.luts[Q - 3] + (size_t)it * (128u << Q), w, lane, PR ? lut_bytes : 0u);
  row_offsets();
  if constexpr (DMA) {
    dma_win(0, 0);
#pragma unroll
    for (int d = 1; d < D; ++d) load_planes<Q, NT>(P[d], rs, cb, d, voff);
    wait_vmem_le<(D - 1) * Q>();  // step 0's planes, the table and step 0's activations
    __syncthreads();
  } else {
    kwin(0, kk);
    ld_win(xr, kk);
    load_planes<Q, NT>(P[1], rs, cb, 1, voff);
    wait_vmem_le<Q>();  // step 0's planes, the table and step 0's activations
    if constexpr (PR) {
      __syncthreads();
      build_pair_table3(lut_bytes, tid);
      __syncthreads();
    }
    st_win(stage, xr, kk);
    kwin(1, kk);
    ld_win(xr, kk);
#pragma unroll
    for (int d = 2; d < D; ++d) load_planes<Q, NT>(P[d], rs, cb, d, voff);
    __syncthreads();
  }

  f32x16 acc[TC];
#pragma unroll
  for (int c = 0; c < TC; ++c) acc[c] = (f32x16){};
  // par = s % 2 (the stage buffer of step s when DB), passed as a constant so
  // that the buffer offset folds into the LDS instructions' offset field
  auto step = [&](int s, uint2 (&Ps)[Q], int par) {
    // DMA: the buffer of step s + 1 was last read in step s - 1
    if constexpr (DMA)
      if (s + 1 < ks.NSW) dma_win(par ^ 1, s + 1);
    if constexpr (PR) {
      uint32_t Pa[3], Pb[3], O[8];
      word_of<3>(Ps, 0, Pa);
      word_of<3>(Ps, 1, Pb);
      assemble_pairs3(Pa, Pb, rg >> 1, O);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const f16x8 a = lookup_pairs4(O[m], slot);
#pragma unroll
        for (int c = 0; c < TC; ++c) {
          const uint32_t bo = rd_off(par, c, 8 * g + m);
          acc[c] = mfma32(a, *(const f16x8*)(stage + bo), acc[c]);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        uint32_t Pw[Q], O[8];
        word_of<Q>(Ps, j, Pw);
        assemble<Q>(Pw, O);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const f16x8 a = lookup8(O[2 * m], O[2 * m + 1], slot);
#pragma unroll
          for (int c = 0; c < TC; ++c) {
            const uint32_t bo = rd_off(par, c, 8 * g + 4 * j + m);
            const f16x8 b = *(const f16x8*)(stage + bo);
            acc[c] = mfma32(a, b, acc[c]);
          }
        }
      }
    }
    if constexpr (DMA) {
      load_planes<Q, NT>(Ps, rs, cb, s + D, voff);
      wait_vmem_le<Q>();  // step s + 1's activations (older than these planes)
      __syncthreads();
      return;
    }
    if (!DB) __syncthreads();
    if (s + 1 < ks.NSW) {
      kwin(s + 1, kk);
      st_win(stage + (!DB ? 0u : HALF ? stage_off_db(par ^ 1, 0, 0, 0) : (uint32_t)(par ^ 1) * stage_bytes<TC>()),
             xr, kk);
    }
    kwin(s + 2, kk);
    ld_win(xr, kk);
    load_planes<Q, NT>(Ps, rs, cb, s + D, voff);
    __syncthreads();
  };
  // whole ring turns in the loop, the remainder after it: the loop's back edge
  // then always follows the ring's last step, which keeps the wait counts
  // exact (DB with an odd ring: two turns per pass, so that the buffer parity
  // is fixed per position)
  constexpr int U = DB && (D & 1) ? 2 * D : D;
  int s = 0;
  for (; s + U <= ks.NSW; s += U)
    unroll_const<U>([&](auto u) { step(s + u, P[u % D], u & 1); });
  unroll_const<U - 1>([&](auto u) {
    if (s + u < ks.NSW) step(s + u, P[u % D], u & 1);
  });

  // SwiGLU: every wave puts the accumulators of every token chunk in LDS
  // (layout [chunk][wave][v][lane], TC x 32 KiB, which every launch holds),
  // then wave w finishes v = 4 (w >> 1) .. + 3 of row half hr = w & 1
  // (columns it * 64 + 32 hr + ...) of each chunk, with gate = the partials of
  // waves hr and hr + 4 and up = those of waves hr + 2 and hr + 6, each sum in
  // that order; all eight waves share the SiLU work, behind one barrier
  float* xb = (float*)lds;
  const int hr = w & 1, v4 = w >> 1;
  // a token converted scaled by 2^-sc (bf16 beyond the fp16 range) gets gate
  // and up scaled back, and h carried as h 2^(-2 sc)
  int scs[TC];
#pragma unroll
  for (int c = 0; c < TC; ++c) scs[c] = p.xsc ? ld_co<CO>(p.xsc + etok[c]) : 0;
#pragma unroll
  for (int c = 0; c < TC; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) xb[((c * kWaves + w) * 16 + v) * 64 + lane] = acc[c][v];
  __syncthreads();
#pragma unroll
  for (int c = 0; c < TC; ++c) {
    const int t = kTok * c + r;
    if (t < nt) {
      // acc[c][v] is row 8*(v/4) + 4*g + v%4 of a wave's 32 rows, token t
      const int sc = scs[c];
      const float* xc = xb + c * kWaves * 16 * 64;
      const size_t o = (size_t)(base + t) * I + it * 64 + hr * 32 + 4 * g;
      uint16_t hv[4], lv[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int v = 4 * v4 + k;
        const float gate =
            __builtin_amdgcn_ldexpf(xc[(hr * 16 + v) * 64 + lane] + xc[((hr + 4) * 16 + v) * 64 + lane], sc);
        const float up =
            __builtin_amdgcn_ldexpf(xc[((hr + 2) * 16 + v) * 64 + lane] + xc[((hr + 6) * 16 + v) * 64 + lane], sc);
        const split16 sp2 = split_hi_lo(__builtin_amdgcn_ldexpf(silu(gate) * up, -2 * sc));
        hv[k] = __builtin_bit_cast(uint16_t, sp2.hi);
        lv[k] = __builtin_bit_cast(uint16_t, sp2.lo);
      }
      st_co<CO>((uint64_t*)(p.hhi + o + 8 * v4), __builtin_bit_cast(uint64_t, make_ushort4(hv[0], hv[1], hv[2], hv[3])));
      st_co<CO>((uint64_t*)(p.hlo + o + 8 * v4), __builtin_bit_cast(uint64_t, make_ushort4(lv[0], lv[1], lv[2], lv[3])));
    }
  }
}

// A block whose committed bitwidth is outside 3..qmax (the table region of
// this launch was sized for qmax), or a table region not at LDS byte 0,
// produces NaN instead of a silently wrong value.
__device__ __forceinline__ void poison_y(const FfnParams& p, int ksi, int base, int nt, int n0) {
  const int cols = min(128, p.H - n0);
  float* y = p.y + (size_t)ksi * p.T * (p.K + p.S) * p.H + n0;
  for (int i = threadIdx.x; i < nt * cols; i += blockDim.x)
    y[(size_t)p.ent[base + i / cols] * p.H + i % cols] = __builtin_nanf("");
}

// ---------------------------------------------------------------- down
// Waves w and w+4 take output rows n0 + 32 (w % 4) .. +31 over the two K
// halves. B operand = h as its fp16 hi and lo parts, two MFMAs per word and
// token chunk into the same fp32 accumulator; items of <= 16 tokens put hi in
// MFMA columns 0..15 and lo in columns 16..31 instead (one MFMA per word),
// and each column adds its lo partner after the K loop. A step is staged in two rounds,
// one per word of the half-chunk; piece p = 8 hl + 4 g' + m of a token holds
// elements 32 j + 8 m .. + 7 of half-chunk 2 s + g', hi (hl = 0) or lo
// (hl = 1), for round j. Each window is loaded one step before it is staged,
// ahead of the plane load that follows it. DB (TC = 1): round j reads stage
// buffer j while the next round's window is written to the other one, two
// barriers per step instead of four; the buffers are 16-token halves of the
// stage region for items of <= 16 tokens, or with DF full 32-token buffers
// after a 32 KiB table region.
template <int Q, int TC, bool CO = false, bool NT = true, bool DB = false, bool PR = false, bool DF = false,
          typename It = Item>
__device__ __forceinline__ void down_body(const FfnParams& p, const It& wi, int it, uint16_t* lds,
                                          uint32_t lut_bytes, int tid, int ksi = 0) {
  // DB: two 16-token round buffers in the 16 KiB stage region (HALF), or with
  // DF two full 32-token round buffers after a 32 KiB table region
  constexpr bool HALF = DB && !DF;
  const int lane = tid & 63, r = lane & 31, g = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = w & 3, kh = w >> 2;
  const int I = p.I, H = p.H, NC = (I / 32 + 3) >> 2;
  // K range ksi: half-chunks hc0 .. hc1-1 (whole chunks; the last range ends at
  // the row's end, whose chunk is zero-padded), split in two halves as a row
  const int hc0 = ksi * p.dn_hcs, hc1 = min(I >> 6, hc0 + p.dn_hcs);
  const int klen = hc1 * 64;  // activation elements at and past klen read as zero
  const KSplit ks((hc1 - hc0) * 64);
  const int n0 = it * 128 + rg * 32;
  const bool active = n0 < H;
  const int nt = wi.nt, base = wi.base;
  static_assert(!PR || Q == 3, "pair tables: 3-bit blocks");
  const uint32_t slot = PR ? pair_slot(r, rg) : lut_slot(r, rg);
  char* stage = (char*)lds + lut_bytes;

  StagePlan<TC> sp;
  const int st = tid >> 4, spc = tid & 15, hl = spc >> 3;
  // the y row of each token chunk's entry in this lane's column (its (token,
  // slot) index), read now so the epilogue's stores do not wait for it
  int yent[TC];
#pragma unroll
  for (int c = 0; c < TC; ++c) yent[c] = ld_co<CO>(p.ent + base + min(kTok * c + r, nt - 1));
  {
    // one descriptor over both halves of h
    const size_t hbytes = (size_t)p.T * (p.K + p.S) * I * 2;
    const char* a = (const char*)p.hhi;
    const char* b = (const char*)p.hlo;
    const char* lo = a < b ? a : b;
    sp.rs = rows_rsrc(lo, (size_t)((a < b ? b : a) - lo) + hbytes);
    const uint32_t half = (uint32_t)((hl ? b : a) - lo);
    sp.wr = !HALF || st < 16;
#pragma unroll
    for (int c = 0; c < TC; ++c) {
      const int t = kTok * c + st;
      sp.wl[c] = wave_has_tokens(c, st, nt);
      sp.lim[c] = t < nt ? klen : 0;
      sp.off[c] = t < nt ? half + (uint32_t)(base + t) * (uint32_t)I * 2u : 0u;
      sp.dst[0][c] = HALF ? stage_off_db(0, 0, t & 15, spc) : stage_off<TC>(0, t, spc);
      sp.dst[1][c] = HALF ? stage_off_db(0, 1, t & 15, spc) : stage_off<TC>(1, t, spc);
    }
  }
  static_assert(!DB || TC == 1, "double-buffered stage: one token chunk");
  // stage buffer of round j (DB)
  auto rbuf = [&](int j) -> uint32_t {
    return !DB ? 0u : HALF ? stage_off_db(j, 0, 0, 0) : (uint32_t)j * stage_bytes<TC>();
  };
  // window (s, j): for K half i, element 64 (hc0 + i HH + 2 s + g') + 32 j + 8 m
  // (PR: round j takes pair groups 4 j .. 4 j + 3, elements 4 m .. 4 m + 3 of
  // both words, m = 4 j + (piece & 3), staged in pair order)
  auto kwin = [&](int s, int j, int (&k)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      k[i] = (hc0 + i * ks.HH + 2 * s + ((spc >> 2) & 1)) * 64 + (PR ? 4 * (4 * j + (spc & 3)) : 32 * j + 8 * (spc & 3));
  };
  auto ld_win = [&](uint4 (&v)[2][TC], const int (&k)[2]) {
    if constexpr (PR) load_window_pairs<TC>(v, sp, k);
    else load_window<TC>(v, sp, k);
  };
  auto st_win = [&](char* dst, const uint4 (&v)[2][TC], const int (&k)[2]) {
    if constexpr (PR) store_window_pairs<TC>(dst, v, sp);
    else store_window<TC>(dst, v, sp);
  };

  const int cb = (hc0 >> 1) + kh * (ks.HH >> 1);
  const int ce = kh ? min(NC, (hc1 + 1) >> 1) : (hc0 >> 1) + (ks.HH >> 1);
  rsrc_t rs[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q)
    rs[q] = tile_rsrc(wi.planes[q], active ? (size_t)(n0 >> 5) * NC * 512 : 0, active ? ce * 512 : 0);
  const int voff = 16 * r + 8 * g;

  constexpr int D = plane_ring<Q, TC>();
  uint2 P[D][Q];
  uint4 ha[2][TC], hb[2][TC];
  int ka[2], kb[2];
  // (requesting steps 1 and 2's planes before this first wait as well, or
  // step 0's planes before the table, measured 1-3 % slower)
  load_table_image<Q>(wi.luts[Q - 3] + (size_t)it * (128u << Q), w, lane, PR ? lut_bytes : 0u);
  kwin(0, 0, ka);
  ld_win(ha, ka);
  load_planes<Q, NT>(P[0], rs, cb, 0, voff);
  wait_vmem_all();
  if constexpr (PR) {
    __syncthreads();
    build_pair_table3(lut_bytes, tid);
    __syncthreads();
  }
  st_win(stage, ha, ka);
  kwin(0, 1, kb);
  ld_win(hb, kb);
  kwin(1, 0, ka);
  ld_win(ha, ka);
#pragma unroll
  for (int d = 1; d < D; ++d) load_planes<Q, NT>(P[d], rs, cb, d, voff);
  __syncthreads();

  f32x16 acc[TC];
#pragma unroll
  for (int c = 0; c < TC; ++c) acc[c] = (f32x16){};
  // O: PR, the pair words of both rounds (assembled in round 0)
  auto round = [&](int j, const uint2 (&Ps)[Q], uint32_t (&Op)[8]) {
    uint32_t Pw[Q], O[8];
    if constexpr (PR) {
      if (j == 0) {
        uint32_t Pa[3], Pb[3];
        word_of<3>(Ps, 0, Pa);
        word_of<3>(Ps, 1, Pb);
        assemble_pairs3(Pa, Pb, rg >> 1, Op);
      }
    } else {
      word_of<Q>(Ps, j, Pw);
      assemble<Q>(Pw, O);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const f16x8 a = PR ? lookup_pairs4(Op[4 * j + m], slot) : lookup8(O[2 * m], O[2 * m + 1], slot);
#pragma unroll
      for (int c = 0; c < TC; ++c) {
        if constexpr (HALF) {
          // columns 0..15: h hi of the item's tokens, 16..31: h lo of the
          // same tokens (one MFMA and one operand read instead of two)
          const f16x8 b = *(const f16x8*)(stage + stage_off_db(j, kh, r & 15, 8 * (r >> 4) + 4 * g + m));
          acc[c] = mfma32(a, b, acc[c]);
        } else {
          const uint32_t oh = rbuf(j) + stage_off<TC>(kh, kTok * c + r, 4 * g + m);
          const uint32_t ol = rbuf(j) + stage_off<TC>(kh, kTok * c + r, 8 + 4 * g + m);
          const f16x8 bh = *(const f16x8*)(stage + oh);
          const f16x8 bl = *(const f16x8*)(stage + ol);
          acc[c] = mfma32(a, bh, acc[c]);
          acc[c] = mfma32(a, bl, acc[c]);
        }
      }
    }
    if (!DB) __syncthreads();
  };
  auto step = [&](int s, uint2 (&Ps)[Q]) {
    uint32_t Op[8];
    round(0, Ps, Op);
    kwin(s, 1, kb);
    st_win(stage + rbuf(1), hb, kb);
    kwin(s + 1, 1, kb);
    ld_win(hb, kb);
    __syncthreads();
    round(1, Ps, Op);
    if (s + 1 < ks.NSW) {
      kwin(s + 1, 0, ka);
      st_win(stage + rbuf(0), ha, ka);
    }
    kwin(s + 2, 0, ka);
    ld_win(ha, ka);
    load_planes<Q, NT>(Ps, rs, cb, s + D, voff);
    __syncthreads();
  };
  // whole ring turns in the loop, the remainder after it (exact wait counts)
  int s = 0;
  for (; s + D <= ks.NSW; s += D) unroll_const<D>([&](auto u) { step(s + u, P[u]); });
  unroll_const<D - 1>([&](auto u) {
    if (s + u < ks.NSW) step(s + u, P[u]);
  });

  // 16-token buffers: each column c < 16 takes its h lo partner from column
  // c + 16, so column c holds the whole sum over the wave's K half
  if constexpr (HALF) {
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[0][v] += __shfl_xor(acc[0][v], 16);
  }
  // second K half -> first through LDS, one token chunk at a time; layout
  // [row group][v][lane]
  float* xb = (float*)lds;
#pragma unroll
  for (int c = 0; c < TC; ++c) {
    if (c) __syncthreads();
    if (kh == 1) {
#pragma unroll
      for (int v = 0; v < 16; ++v) xb[(rg * 16 + v) * 64 + lane] = acc[c][v];
    }
    __syncthreads();
    const int t = kTok * c + r;
    if (kh == 0 && active && t < nt) {
      // h of a scaled token was carried as h 2^(-2 sc)
      const int sc = p.xsc ? ld_co<CO>(p.xsc + ld_co<CO>(p.ptok + base + t)) : 0;
      float* yrow = p.y + (size_t)ksi * p.T * (p.K + p.S) * H + (size_t)yent[c] * H + n0 + 4 * g;
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        f32x4 o;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          o[k] = __builtin_amdgcn_ldexpf(acc[c][4 * v4 + k] + xb[(rg * 16 + 4 * v4 + k) * 64 + lane], 2 * sc);
        st_co16<CO>(yrow + 8 * v4, __builtin_bit_cast(uint4, o));
      }
    }
  }
}

// out[t][n..n+3] = sum_k w_tk * y[t, k] + sum_s y[t, K + s], in that order
// (the same order for every output, so the result is deterministic). y holds
// one row per (token, slot), so a token's rows are known without reading the
// grouping: the ids, weights and rows are all requested together (one round
// trip); a dead slot's row (an out-of-range id) is read but not added.
template <bool CO = false>
__device__ __forceinline__ void combine4(const FfnParams& p, int t, int n) {
  const int KS = p.K + p.S;
  f32x4 s = (f32x4){};
  for (int k0 = 0; k0 < KS; k0 += 8) {
    float w[8];
    bool live[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = k0 + j;
      live[j] = k < KS;
      w[j] = 1.0f;
      if (k < p.K) {
        const int ex = ld_co<CO>(p.topk_idx + t * p.K + k);
        live[j] = ex >= 0 && ex < p.E;
        w[j] = ld_co<CO>(p.topk_w + t * p.K + k);
      }
    }
    const float* yt = p.y + (size_t)t * KS * p.H + n;
    f32x4 y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = k0 + j < KS ? *(const f32x4*)(yt + (size_t)(k0 + j) * p.H) : (f32x4){};
    // partial sums of the other K ranges, added in range order
    const size_t slice = (size_t)p.T * KS * p.H;
    for (int r = 1; r < p.dn_split; ++r) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (live[j]) y[j] += *(const f32x4*)(yt + r * slice + (size_t)(k0 + j) * p.H);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (!live[j]) continue;
      if (k0 + j < p.K) s += w[j] * y[j];
      else s += y[j];
    }
  }
  *(f32x4*)(p.out + (size_t)t * p.H + n) = s;
}

}  // namespace mpb
