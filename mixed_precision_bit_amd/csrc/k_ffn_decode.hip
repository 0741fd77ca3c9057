// Decode-size expert FFN: gate_up + SwiGLU, down, and the weighted combine.
//
// "PagedWeight", §3.3: the fused kernel reads the weight pages directly and
// follows the committed bitwidth of every gate_up and down block. Here each
// workgroup reads its block's q_i once from the device page table and runs the
// matching instantiation, so a launch mixes bitwidths freely and a change of
// q_i between launches takes effect on the next launch.
//
// Mapping (MFMA 32x32x16 fp16 -> fp32): a workgroup of 4 waves handles up to
// 32 tokens of one expert. A wave owns 32 weight rows; lane l holds row l%32
// and, in step s, chunk 2s + l/32 of that row (4 words = 128 elements) from
// each of the q plane pages: one 16-byte load per page, issued three steps
// ahead. Each word feeds four MFMAs as the A operand.
//
// The B operand (the tokens) is staged per step into LDS by the whole
// workgroup and read with ds_read_b128: with the weights the only vector
// memory traffic in the loop, waits on the activations never queue behind the
// long-latency plane loads (vector-memory completions are counted in issue
// order). All loads are unconditional (clamped addresses), so the wait counts
// are static.
//
// LDS: [centroid tables: 2^qmax * 256 bytes][stage: 32 tokens x 512 bytes].
// Stage rows are 512 bytes; 16-byte piece c of row t sits at piece c ^ t, so
// the 32 lanes reading one piece column of 32 rows spread over the banks.
#include "mpb_device.h"
#include "mpb_internal.h"

namespace mpb {

constexpr int kTok = kDecodeTokensPerWG;  // 32
constexpr int kStageBytes = kTok * 512;

__device__ __forceinline__ uint32_t stage_off(int t, int piece) { return t * 512u + ((piece ^ t) << 4); }

// Plane loads go through buffer descriptors, one per plane page, based at the
// wave's 32-row tile and spanning its NC chunks: lane l reads chunk 2s + l/32
// of its row at byte offset 1024 s + 16 l, and an offset past the tile (the
// lanes of the last odd chunk, prefetches past the end) reads zeros without
// touching memory.
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
// global-to-LDS loads: wave w moves 1 KiB pieces w, w + 4, ... (no registers,
// no LDS store instructions). The caller waits for vector memory and
// synchronises the workgroup before the first lookup.
typedef __attribute__((address_space(3))) void lds_void;

template <int Q>
__device__ __forceinline__ void load_table_image(const uint16_t* img, int w, int lane) {
  const char* src = (const char*)img + 16 * lane;
#pragma unroll
  for (int c = 0; c < (1 << Q) / 4; c += 4)
    if (c + w < (1 << Q) / 4)
      __builtin_amdgcn_global_load_lds(src + 1024 * (c + w), (lds_void*)(uintptr_t)(1024u * (c + w)), 16, 0, 0);
}

__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int Q>
__device__ __forceinline__ void load_chunk(uint4 (&P)[Q], const rsrc_t (&rs)[Q], int s, int lane) {
#pragma unroll
  for (int q = 0; q < Q; ++q)
    P[q] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs[q], 1024 * s + 16 * lane, 0, 0));
}

template <int Q>
__device__ __forceinline__ void word_of(const uint4 (&P4)[Q], int j, uint32_t (&P)[Q]) {
#pragma unroll
  for (int q = 0; q < Q; ++q) P[q] = j == 0 ? P4[q].x : j == 1 ? P4[q].y : j == 2 ? P4[q].z : P4[q].w;
}

// One word: assemble indices, look the 32 weights up, multiply with the four
// B pieces of the word.
template <int Q>
__device__ __forceinline__ void word_mfma(const uint4 (&P4)[Q], int j, const uint16_t* lds, uint32_t slot,
                                          const char* stage, int r, int bpiece0, f32x16& acc) {
  uint32_t P[Q], O[8];
  word_of<Q>(P4, j, P);
  assemble<Q>(P, O);
  f16x8 b[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) b[m] = *(const f16x8*)(stage + stage_off(r, bpiece0 + m));
#pragma unroll
  for (int m = 0; m < 4; ++m) acc = mfma32(lookup8(O[2 * m], O[2 * m + 1], slot), b[m], acc);
}

// ---------------------------------------------------------------- gate_up
// Workgroup = 4 waves = 64 h columns of one expert: waves 0/1 take gate rows
// c0..c0+31 / c0+32..c0+63, waves 2/3 the matching up rows. After the K loop
// the up waves hand their accumulators to the gate waves through LDS, which
// apply SiLU(gate) * up and store h as an fp16 (hi, lo) pair (hi + lo carries
// ~22 significant bits of the fp32 value into the down projection).
//
// Issue order per step s (vector memory completes in issue order, so a wait
// for one load also waits for every older one): compute on the planes of step
// s, barrier, write the activations of step s+1 (loaded one step earlier) to
// the stage, load the activations of step s+2, load the planes of step s+3,
// barrier. A plane load thus has two steps of compute to arrive before the
// activation wait that follows it, an activation load one step.

// 16-byte activation pieces staged per thread and step: piece pc = tid + 256 i
// is token slot pc / 32, piece column pc % 32.
struct StagePlan {
  const uint16_t* row[4];  // source row start (token slots >= nt load nothing)
  int col[4];              // element offset of the piece inside a step window
  uint32_t dst[4];         // stage byte offset
  bool live[4];            // token slot < nt (rows past nt stay zero)
};

__device__ __forceinline__ void load_window(uint4 (&v)[4], const StagePlan& sp, int k0, int len) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = k0 + sp.col[i];
    if (sp.live[i]) v[i] = *(const uint4*)(sp.row[i] + (k < len ? k : 0));
  }
}

__device__ __forceinline__ void store_window(char* stage, const uint4 (&v)[4], const StagePlan& sp, int k0, int len) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (sp.live[i]) *(uint4*)(stage + sp.dst[i]) = k0 + sp.col[i] < len ? v[i] : make_uint4(0u, 0u, 0u, 0u);
}

__device__ __forceinline__ void zero_dead_rows(char* stage, const StagePlan& sp) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (!sp.live[i]) *(uint4*)(stage + sp.dst[i]) = make_uint4(0u, 0u, 0u, 0u);
}

template <int Q>
__device__ __forceinline__ void gate_up_body(const FfnParams& p, int e, int it, int t0, int nt, uint16_t* lds,
                             uint32_t lut_bytes) {
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 31, g = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: plane descriptors stay scalar
  const int I = p.I, H = p.H, W = H >> 5, NC = (W + 3) >> 2, NS = (NC + 1) >> 1;
  const int c0 = it * 64 + (w & 1) * 32;
  const int row0 = (w >> 1) * I + c0;
  const int base = p.offsets[e] + t0;
  const uint32_t slot = lut_slot(r, w);
  const int blk = 2 * e;
  char* stage = (char*)lds + lut_bytes;

  StagePlan sp;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int pc = tid + 256 * i, tt = pc >> 5, cl = pc & 31;
    sp.live[i] = tt < nt;
    sp.row[i] = p.xh + (size_t)p.ptok[base + (sp.live[i] ? tt : 0)] * H;
    sp.col[i] = 8 * cl;
    sp.dst[i] = stage_off(tt, cl);
  }
  rsrc_t rs[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) rs[q] = tile_rsrc(p.planes[blk * 8 + q], (size_t)(row0 >> 5) * NC * 512, NC * 512);

  // prologue: tables, the first activation window and the first planes in one
  // memory round trip; the next two steps' planes are issued after the wait
  uint4 PA[Q], PB[Q], PC[Q], xr[4];
  load_table_image<Q>(p.luts[blk * 6 + (Q - 3)] + (size_t)it * (128u << Q), w, lane);
  load_window(xr, sp, 0, H);
  load_chunk<Q>(PA, rs, 0, lane);
  wait_vmem_all();
  zero_dead_rows(stage, sp);
  store_window(stage, xr, sp, 0, H);
  load_chunk<Q>(PB, rs, 1, lane);
  load_window(xr, sp, NS > 1 ? 256 : 0, H);
  load_chunk<Q>(PC, rs, 2, lane);
  __syncthreads();

  f32x16 acc = (f32x16){};
  auto step = [&](int s, uint4 (&P)[Q]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) word_mfma<Q>(P, j, lds, slot, stage, r, 16 * g + 4 * j, acc);
    __syncthreads();
    if (s + 1 < NS) store_window(stage, xr, sp, 256 * (s + 1), H);
    load_window(xr, sp, 256 * (s + 2 < NS ? s + 2 : NS - 1), H);
    load_chunk<Q>(P, rs, s + 3, lane);
    __syncthreads();
  };
  // whole ring turns in the loop, the remainder after it: the loop's back edge
  // then always follows a PC step, which keeps the wait counts exact
  int s = 0;
  for (; s + 3 <= NS; s += 3) {
    step(s, PA);
    step(s + 1, PB);
    step(s + 2, PC);
  }
  if (s < NS) step(s, PA);
  if (s + 1 < NS) step(s + 1, PB);

  // hand the up accumulators to the gate waves; layout [wave-2][v][lane]
  float* xb = (float*)lds;
  if (w >= 2) {
#pragma unroll
    for (int v = 0; v < 16; ++v) xb[((w - 2) * 16 + v) * 64 + lane] = acc[v];
  }
  __syncthreads();
  if (w >= 2 || r >= nt) return;
  // acc[v] is row 8*(v/4) + 4*g + v%4 of the wave's 32 rows, token slot r
  const size_t o = (size_t)(base + r) * I + c0 + 4 * g;
#pragma unroll
  for (int v4 = 0; v4 < 4; ++v4) {
    uint16_t hv[4], lv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int v = 4 * v4 + k;
      const split16 sp2 = split_hi_lo(silu(acc[v]) * xb[(w * 16 + v) * 64 + lane]);
      hv[k] = __builtin_bit_cast(uint16_t, sp2.hi);
      lv[k] = __builtin_bit_cast(uint16_t, sp2.lo);
    }
    *(ushort4*)(p.hhi + o + 8 * v4) = make_ushort4(hv[0], hv[1], hv[2], hv[3]);
    *(ushort4*)(p.hlo + o + 8 * v4) = make_ushort4(lv[0], lv[1], lv[2], lv[3]);
  }
}

// Work item of a decode launch: workgroup id = item * ntile + tile, so the
// consecutive workgroups that the dispatcher spreads over the chip carry the
// tiles of one item and every workgroup below n_items * ntile has tokens.
__device__ __forceinline__ bool decode_item(const FfnParams& p, const int32_t* items, int ntile, int& e, int& tile,
                                            int& t0, int& nt) {
  const int item = blockIdx.x / ntile;
  tile = blockIdx.x - item * ntile;
  if (item >= p.n_items[0]) return false;
  const int v = items[item];
  e = v >> 16;
  t0 = (v & 0xffff) * kTok;
  nt = min(p.counts[e] - t0, kTok);
  return true;
}

// A block whose committed bitwidth is outside 3..qmax (the table region of
// this launch was sized for qmax), or a table region not at LDS byte 0,
// produces NaN instead of a silently wrong value.
__device__ __forceinline__ void poison(float* dst, size_t ld, int rows, int cols) {
  for (int i = threadIdx.x; i < rows * cols; i += blockDim.x) dst[(size_t)(i / cols) * ld + i % cols] = __builtin_nanf("");
}

__global__ __launch_bounds__(256) void k_gate_up_decode(FfnParams p, int qmax) {
  extern __shared__ __attribute__((aligned(256))) uint16_t lds[];
  int e, it, t0, nt;
  if (!decode_item(p, p.items, p.I >> 6, e, it, t0, nt)) return;
  const int q = p.q[2 * e];
  const uint32_t lut_bytes = 256u << qmax;
  switch (q < 3 || q > qmax || !tables_at_zero(lds) ? 0 : q) {
    case 3: gate_up_body<3>(p, e, it, t0, nt, lds, lut_bytes); break;
    case 4: gate_up_body<4>(p, e, it, t0, nt, lds, lut_bytes); break;
    case 5: gate_up_body<5>(p, e, it, t0, nt, lds, lut_bytes); break;
    case 6: gate_up_body<6>(p, e, it, t0, nt, lds, lut_bytes); break;
    case 7: gate_up_body<7>(p, e, it, t0, nt, lds, lut_bytes); break;
    case 8: gate_up_body<8>(p, e, it, t0, nt, lds, lut_bytes); break;
    default: {
      const size_t o = (size_t)(p.offsets[e] + t0) * p.I + it * 64;
      for (int i = threadIdx.x; i < nt * 64; i += blockDim.x) {
        p.hhi[o + (size_t)(i >> 6) * p.I + (i & 63)] = 0x7e00;  // fp16 NaN
        p.hlo[o + (size_t)(i >> 6) * p.I + (i & 63)] = 0;
      }
    }
  }
}

// ---------------------------------------------------------------- down
// Workgroup = 4 waves x 32 output rows. B operand = h as its fp16 hi and lo
// parts, two MFMAs per word into the same fp32 accumulator. A step is staged
// in two rounds; round rd holds words 2rd, 2rd+1 of both lane groups' chunks,
// hi parts in pieces 0..15 and lo parts in pieces 16..31 of each token row.
// Each window is loaded one step before it is staged, ahead of the plane load
// that follows it, so a plane load has about one and a half steps to arrive.
template <int Q>
__device__ __forceinline__ void down_body(const FfnParams& p, int e, int it, int t0, int nt, uint16_t* lds,
                          uint32_t lut_bytes) {
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 31, g = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: plane descriptors stay scalar
  const int I = p.I, H = p.H, W = I >> 5, NC = (W + 3) >> 2, NS = (NC + 1) >> 1;
  const int n0 = it * 128 + w * 32;
  const bool active = n0 < H;
  const int base = p.offsets[e] + t0;
  const uint32_t slot = lut_slot(r, w);
  const int blk = 2 * e + 1;
  char* stage = (char*)lds + lut_bytes;

  // piece column cl: hl = cl/16 (hi/lo), gg = (cl/8)%2 (lane group), q8 = cl%8;
  // window (s, rd) = chunk 2s+gg, elements 64rd .. 64rd+63 of the chunk
  StagePlan sp;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int pc = tid + 256 * i, tt = pc >> 5, cl = pc & 31;
    const int hl = cl >> 4, gg = (cl >> 3) & 1, q8 = cl & 7;
    sp.live[i] = tt < nt;
    sp.row[i] = (hl ? p.hlo : p.hhi) + (size_t)(base + (sp.live[i] ? tt : 0)) * I;
    sp.col[i] = 128 * gg + 8 * q8;
    sp.dst[i] = stage_off(tt, cl);
  }
  // window (s, rd) -> element offset of its start; windows past the last are clamped
  auto win = [&](int s, int rd) { return s < NS ? 256 * s + 64 * rd : 256 * (NS - 1) + 64; };

  rsrc_t rs[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q)
    rs[q] = tile_rsrc(p.planes[blk * 8 + q], active ? (size_t)(n0 >> 5) * NC * 512 : 0, active ? NC * 512 : 0);

  // ha holds the next round-0 window, hb the next round-1 window; each is
  // loaded one step before it is staged
  uint4 PA[Q], PB[Q], PC[Q], ha[4], hb[4];
  load_table_image<Q>(p.luts[blk * 6 + (Q - 3)] + (size_t)it * (128u << Q), w, lane);
  load_window(ha, sp, win(0, 0), I);
  load_chunk<Q>(PA, rs, 0, lane);
  wait_vmem_all();
  zero_dead_rows(stage, sp);
  store_window(stage, ha, sp, win(0, 0), I);
  load_window(hb, sp, win(0, 1), I);
  load_window(ha, sp, win(1, 0), I);
  load_chunk<Q>(PB, rs, 1, lane);
  load_chunk<Q>(PC, rs, 2, lane);
  __syncthreads();

  f32x16 acc = (f32x16){};
  auto round = [&](int rd, const uint4 (&P)[Q]) {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int j = 2 * rd + jj;
      uint32_t Pw[Q], O[8];
      word_of<Q>(P, j, Pw);
      assemble<Q>(Pw, O);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const f16x8 bh = *(const f16x8*)(stage + stage_off(r, 8 * g + 4 * jj + m));
        const f16x8 bl = *(const f16x8*)(stage + stage_off(r, 16 + 8 * g + 4 * jj + m));
        const f16x8 a = lookup8(O[2 * m], O[2 * m + 1], slot);
        acc = mfma32(a, bh, acc);
        acc = mfma32(a, bl, acc);
      }
    }
    __syncthreads();
  };
  auto step = [&](int s, uint4 (&P)[Q]) {
    round(0, P);
    store_window(stage, hb, sp, win(s, 1), I);
    load_window(hb, sp, win(s + 1, 1), I);
    __syncthreads();
    round(1, P);
    if (s + 1 < NS) store_window(stage, ha, sp, win(s + 1, 0), I);
    load_window(ha, sp, win(s + 2, 0), I);
    load_chunk<Q>(P, rs, s + 3, lane);
    __syncthreads();
  };
  // whole ring turns in the loop, the remainder after it: the loop's back edge
  // then always follows a PC step, which keeps the wait counts exact
  int s = 0;
  for (; s + 3 <= NS; s += 3) {
    step(s, PA);
    step(s + 1, PB);
    step(s + 2, PC);
  }
  if (s < NS) step(s, PA);
  if (s + 1 < NS) step(s + 1, PB);
  if (!active || r >= nt) return;
  float* yrow = p.y + (size_t)(base + r) * H + n0 + 4 * g;
#pragma unroll
  for (int v4 = 0; v4 < 4; ++v4) {
    f32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = acc[4 * v4 + k];
    *(f32x4*)(yrow + 8 * v4) = o;
  }
}

__global__ __launch_bounds__(256) void k_down_decode(FfnParams p, int qmax) {
  extern __shared__ __attribute__((aligned(256))) uint16_t lds[];
  int e, it, t0, nt;
  if (!decode_item(p, p.items_dn, (p.H + 127) >> 7, e, it, t0, nt)) return;
  const int q = p.q[2 * e + 1];
  const uint32_t lut_bytes = 256u << qmax;
  switch (q < 3 || q > qmax || !tables_at_zero(lds) ? 0 : q) {
    case 3: down_body<3>(p, e, it, t0, nt, lds, lut_bytes); break;
    case 4: down_body<4>(p, e, it, t0, nt, lds, lut_bytes); break;
    case 5: down_body<5>(p, e, it, t0, nt, lds, lut_bytes); break;
    case 6: down_body<6>(p, e, it, t0, nt, lds, lut_bytes); break;
    case 7: down_body<7>(p, e, it, t0, nt, lds, lut_bytes); break;
    case 8: down_body<8>(p, e, it, t0, nt, lds, lut_bytes); break;
    default: {
      const int n0 = it * 128;
      poison(p.y + (size_t)(p.offsets[e] + t0) * p.H + n0, p.H, nt, min(128, p.H - n0));
    }
  }
}

// ---------------------------------------------------------------- combine
// out[t] = sum_k w_tk * y[entry(t,k)] + sum_s y[entry(t,K+s)], in that order.
__global__ __launch_bounds__(256) void k_combine(FfnParams p) {
  const int H4 = p.H >> 2;
  const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (size_t)p.T * H4) return;
  const int t = (int)(gid / H4), n = (int)(gid - (size_t)t * H4) * 4;
  const int KS = p.K + p.S;
  f32x4 s = (f32x4){};
  for (int k = 0; k < p.K; ++k) {
    const int ex = p.topk_idx[t * p.K + k];
    if (ex >= 0 && ex < p.E) {
      const int pos = p.inv[t * KS + k];
      s += p.topk_w[t * p.K + k] * *(const f32x4*)(p.y + (size_t)pos * p.H + n);
    }
  }
  for (int sh = 0; sh < p.S; ++sh) {
    const int pos = p.inv[t * KS + p.K + sh];
    s += *(const f32x4*)(p.y + (size_t)pos * p.H + n);
  }
  *(f32x4*)(p.out + (size_t)t * p.H + n) = s;
}

// bf16 activations -> fp16 once per call (exact in the fp16 normal range).
__global__ __launch_bounds__(256) void k_x_to_f16(const uint16_t* __restrict__ x, uint16_t* __restrict__ y,
                                                  size_t n8) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n8) *(f16x8*)(y + 8 * i) = load_x8_bf16(x + 8 * i);
}

hipError_t launch_x_to_f16(const uint16_t* x, uint16_t* y, size_t n, hipStream_t s) {
  const size_t n8 = n / 8;
  hipLaunchKernelGGL(k_x_to_f16, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, x, y, n8);
  return hipGetLastError();
}

static bool lds_attr_set = false;

static hipError_t set_lds_attr() {
  if (lds_attr_set) return hipSuccess;
  const int maxb = (256 << 8) + kStageBytes;
  hipError_t e = hipFuncSetAttribute((const void*)k_gate_up_decode, hipFuncAttributeMaxDynamicSharedMemorySize, maxb);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute((const void*)k_down_decode, hipFuncAttributeMaxDynamicSharedMemorySize, maxb);
  if (e == hipSuccess) lds_attr_set = true;
  return e;
}

hipError_t launch_gate_up(const FfnParams& p, int qmax, hipStream_t s) {
  hipError_t e = set_lds_attr();
  if (e != hipSuccess) return e;
  const size_t shmem = (256u << qmax) + kStageBytes;
  hipLaunchKernelGGL(k_gate_up_decode, dim3(p.max_items * (p.I >> 6)), dim3(256), shmem, s, p, qmax);
  return hipGetLastError();
}

hipError_t launch_down(const FfnParams& p, int qmax, hipStream_t s) {
  hipError_t e = set_lds_attr();
  if (e != hipSuccess) return e;
  const size_t shmem = (256u << qmax) + kStageBytes;
  hipLaunchKernelGGL(k_down_decode, dim3(p.max_items * ((p.H + 127) >> 7)), dim3(256), shmem, s, p, qmax);
  return hipGetLastError();
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
