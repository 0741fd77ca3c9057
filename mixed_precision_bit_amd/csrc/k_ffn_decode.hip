// Decode-size expert FFN: gate_up + SwiGLU, down, and the weighted combine.
//
// "PagedWeight", §3.3: the fused kernel reads the weight pages directly and
// follows the committed bitwidth of every gate_up and down block. Here each
// workgroup reads its block's q_i once from the device page table and runs the
// matching instantiation, so a launch mixes bitwidths freely and a change of
// q_i between launches takes effect on the next launch.
//
// Mapping (MFMA 32x32x16 fp16 -> fp32): a wave owns 32 weight rows. Lane l
// holds row l%32; in step s it reads chunk 2s + l/32 (4 words = 128 elements)
// of that row from each of the q plane pages, one 16-byte load per page, while
// the next step's chunk is already in flight. Each word feeds four MFMAs as
// the A operand; the B operand is the expert's tokens (32 per chunk, up to two
// chunks per workgroup), element-aligned with the A words. Weights are
// dequantised once per step and reused for every token chunk.
#include "mpb_device.h"
#include "mpb_internal.h"

namespace mpb {

constexpr int MAXC = kDecodeChunks;

template <int Q>
__device__ __forceinline__ void load_chunk(uint4 (&P)[Q], const uint4* const (&pp)[Q], int c, bool ok) {
#pragma unroll
  for (int q = 0; q < Q; ++q) P[q] = ok ? pp[q][(size_t)c * 32] : make_uint4(0u, 0u, 0u, 0u);
}

template <int Q>
__device__ __forceinline__ void word_of(const uint4 (&P4)[Q], int j, uint32_t (&P)[Q]) {
#pragma unroll
  for (int q = 0; q < Q; ++q) P[q] = j == 0 ? P4[q].x : j == 1 ? P4[q].y : j == 2 ? P4[q].z : P4[q].w;
}

// B operands (8 fp16 each) of the four MFMAs of one word, for every token chunk.
__device__ __forceinline__ void load_b_word(f16x8 (&b)[MAXC][4], const uint16_t* const (&row)[MAXC],
                                            const bool (&v)[MAXC], int nch, int word, bool wok) {
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const bool ok = wok && c < nch && v[c];
#pragma unroll
    for (int m = 0; m < 4; ++m) b[c][m] = ok ? *(const f16x8*)(row[c] + 32 * word + 8 * m) : (f16x8){};
  }
}

// ---------------------------------------------------------------- gate_up
// Workgroup = 4 waves = 64 h columns of one expert: waves 0/1 take gate rows
// c0..c0+31 / c0+32..c0+63, waves 2/3 the matching up rows. After the K loop
// the up waves hand their accumulators to the gate waves through LDS, which
// apply SiLU(gate) * up and store h as an fp16 (hi, lo) pair (hi + lo carries
// ~22 significant bits of the fp32 value into the down projection).
template <int Q>
__device__ void gate_up_body(const FfnParams& p, int e, int it, int t0, int nt, uint16_t* lds) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, r = lane & 31, g = lane >> 5;
  const int I = p.I, H = p.H, W = H >> 5, NC = (W + 3) >> 2, NS = (NC + 1) >> 1;
  const int c0 = it * 64 + (w & 1) * 32;
  const int row0 = (w >> 1) * I + c0;
  const int nch = (nt + 31) >> 5;
  const int base = p.offsets[e] + t0;
  const uint32_t slot = lut_slot(r, w);
  const int blk = 2 * e;

  const uint16_t* xrow[MAXC];
  bool xv[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int j = 32 * c + r;
    xv[c] = j < nt;
    xrow[c] = p.xh + (size_t)(xv[c] ? p.ptok[base + j] : 0) * H;
  }
  const uint4* pp[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) pp[q] = (const uint4*)p.planes[blk * 8 + q] + (size_t)(row0 >> 5) * NC * 32 + r;

  uint4 Pc[Q], Pn[Q];
  load_chunk<Q>(Pc, pp, g, g < NC);
  f16x8 bc[MAXC][4], bn[MAXC][4];
  load_b_word(bc, xrow, xv, nch, 4 * g, 4 * g < W);
  stage_luts<Q>(lds, p.luts[blk * 6 + (Q - 3)], row0, lane, w);
  __syncthreads();

  f32x16 acc[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) acc[c] = (f32x16){};
  for (int s = 0; s < NS; ++s) {
    const int c = 2 * s + g;
    load_chunk<Q>(Pn, pp, c + 2, c + 2 < NC);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int nword = j < 3 ? 4 * c + j + 1 : 4 * (c + 2);
      load_b_word(bn, xrow, xv, nch, nword, nword < W);
      uint32_t P[Q], O[8];
      word_of<Q>(Pc, j, P);
      assemble<Q>(P, O);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const f16x8 a = lookup8(lds, O[2 * m], O[2 * m + 1], slot);
#pragma unroll
        for (int cc = 0; cc < MAXC; ++cc)
          if (cc < nch) acc[cc] = mfma32(a, bc[cc][m], acc[cc]);
      }
#pragma unroll
      for (int cc = 0; cc < MAXC; ++cc)
#pragma unroll
        for (int m = 0; m < 4; ++m) bc[cc][m] = bn[cc][m];
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) Pc[q] = Pn[q];
  }

  // hand the up accumulators to the gate waves; layout [wave-2][chunk][v][lane]
  __syncthreads();
  float* xb = (float*)lds;
  if (w >= 2) {
#pragma unroll
    for (int cc = 0; cc < MAXC; ++cc)
      if (cc < nch)
#pragma unroll
        for (int v = 0; v < 16; ++v) xb[(((w - 2) * MAXC + cc) * 16 + v) * 64 + lane] = acc[cc][v];
  }
  __syncthreads();
  if (w >= 2) return;
  // acc[c][v] is row 8*(v/4) + 4*g + v%4 of the wave's 32 rows, token slot r
#pragma unroll
  for (int cc = 0; cc < MAXC; ++cc) {
    const int j = 32 * cc + r;
    if (cc < nch && j < nt) {
      const size_t o = (size_t)(base + j) * I + c0 + 4 * g;
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        ushort4 hi, lo;
        uint16_t hv[4], lv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int v = 4 * v4 + k;
          const float up = xb[((w * MAXC + cc) * 16 + v) * 64 + lane];
          const split16 sp = split_hi_lo(silu(acc[cc][v]) * up);
          const _Float16 h1 = sp.hi, h2 = sp.lo;
          hv[k] = __builtin_bit_cast(uint16_t, h1);
          lv[k] = __builtin_bit_cast(uint16_t, h2);
        }
        hi = make_ushort4(hv[0], hv[1], hv[2], hv[3]);
        lo = make_ushort4(lv[0], lv[1], lv[2], lv[3]);
        *(ushort4*)(p.hhi + o + 8 * v4) = hi;
        *(ushort4*)(p.hlo + o + 8 * v4) = lo;
      }
    }
  }
}

__global__ __launch_bounds__(256) void k_gate_up_decode(FfnParams p) {
  __shared__ __attribute__((aligned(256))) uint16_t lds[32768];
  const int nit = p.I >> 6;
  const int e = blockIdx.x / nit, it = blockIdx.x - e * nit;
  const int cnt = p.counts[e];
  const int t0 = blockIdx.y * kDecodeTokensPerWG;
  if (t0 >= cnt) return;
  const int nt = min(cnt - t0, kDecodeTokensPerWG);
  switch (p.q[2 * e]) {
    case 3: gate_up_body<3>(p, e, it, t0, nt, lds); break;
    case 4: gate_up_body<4>(p, e, it, t0, nt, lds); break;
    case 5: gate_up_body<5>(p, e, it, t0, nt, lds); break;
    case 6: gate_up_body<6>(p, e, it, t0, nt, lds); break;
    case 7: gate_up_body<7>(p, e, it, t0, nt, lds); break;
    case 8: gate_up_body<8>(p, e, it, t0, nt, lds); break;
    default: break;
  }
}

// ---------------------------------------------------------------- down
// Workgroup = 4 waves x 32 output rows. B operand = h as its fp16 hi and lo
// parts, two MFMAs into the same fp32 accumulator.
template <int Q>
__device__ void down_body(const FfnParams& p, int e, int nt_, int t0, int nt, uint16_t* lds) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, r = lane & 31, g = lane >> 5;
  const int I = p.I, H = p.H, W = I >> 5, NC = (W + 3) >> 2, NS = (NC + 1) >> 1;
  const int n0 = nt_ * 128 + w * 32;
  const bool active = n0 < H;
  const int nch = (nt + 31) >> 5;
  const int base = p.offsets[e] + t0;
  const uint32_t slot = lut_slot(r, w);
  const int blk = 2 * e + 1;

  const uint16_t* hrow[MAXC];
  const uint16_t* lrow[MAXC];
  bool hv[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int j = 32 * c + r;
    hv[c] = j < nt;
    const size_t o = (size_t)(base + (hv[c] ? j : 0)) * I;
    hrow[c] = p.hhi + o;
    lrow[c] = p.hlo + o;
  }
  const uint4* pp[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q)
    pp[q] = (const uint4*)p.planes[blk * 8 + q] + (size_t)((active ? n0 : 0) >> 5) * NC * 32 + r;

  uint4 Pc[Q], Pn[Q];
  if (active) {
    load_chunk<Q>(Pc, pp, g, g < NC);
    stage_luts<Q>(lds, p.luts[blk * 6 + (Q - 3)], n0, lane, w);
  }
  __syncthreads();
  if (!active) return;

  f32x16 acc[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) acc[c] = (f32x16){};
  for (int s = 0; s < NS; ++s) {
    const int c = 2 * s + g;
    load_chunk<Q>(Pn, pp, c + 2, c + 2 < NC);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int word = 4 * c + j;
      f16x8 bh[MAXC][4], bl[MAXC][4];
      load_b_word(bh, hrow, hv, nch, word, word < W);
      load_b_word(bl, lrow, hv, nch, word, word < W);
      uint32_t P[Q], O[8];
      word_of<Q>(Pc, j, P);
      assemble<Q>(P, O);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const f16x8 a = lookup8(lds, O[2 * m], O[2 * m + 1], slot);
#pragma unroll
        for (int cc = 0; cc < MAXC; ++cc) {
          if (cc < nch) {
            acc[cc] = mfma32(a, bh[cc][m], acc[cc]);
            acc[cc] = mfma32(a, bl[cc][m], acc[cc]);
          }
        }
      }
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) Pc[q] = Pn[q];
  }
#pragma unroll
  for (int cc = 0; cc < MAXC; ++cc) {
    const int j = 32 * cc + r;
    if (cc < nch && j < nt) {
      float* yrow = p.y + (size_t)(base + j) * H + n0 + 4 * g;
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        f32x4 o;
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = acc[cc][4 * v4 + k];
        *(f32x4*)(yrow + 8 * v4) = o;
      }
    }
  }
}

__global__ __launch_bounds__(256) void k_down_decode(FfnParams p) {
  __shared__ __attribute__((aligned(256))) uint16_t lds[32768];
  const int nnt = (p.H + 127) >> 7;
  const int e = blockIdx.x / nnt, nt_ = blockIdx.x - e * nnt;
  const int cnt = p.counts[e];
  const int t0 = blockIdx.y * kDecodeTokensPerWG;
  if (t0 >= cnt) return;
  const int nt = min(cnt - t0, kDecodeTokensPerWG);
  switch (p.q[2 * e + 1]) {
    case 3: down_body<3>(p, e, nt_, t0, nt, lds); break;
    case 4: down_body<4>(p, e, nt_, t0, nt, lds); break;
    case 5: down_body<5>(p, e, nt_, t0, nt, lds); break;
    case 6: down_body<6>(p, e, nt_, t0, nt, lds); break;
    case 7: down_body<7>(p, e, nt_, t0, nt, lds); break;
    case 8: down_body<8>(p, e, nt_, t0, nt, lds); break;
    default: break;
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

hipError_t launch_gate_up(const FfnParams& p, hipStream_t s) {
  const int ty = (p.T + kDecodeTokensPerWG - 1) / kDecodeTokensPerWG;
  hipLaunchKernelGGL(k_gate_up_decode, dim3(p.NB * (p.I >> 6), ty), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_down(const FfnParams& p, hipStream_t s) {
  const int ty = (p.T + kDecodeTokensPerWG - 1) / kDecodeTokensPerWG;
  hipLaunchKernelGGL(k_down_decode, dim3(p.NB * ((p.H + 127) >> 7), ty), dim3(256), 0, s, p);
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
