// Decode-size expert FFN: gate_up + SwiGLU, down, and the weighted combine.
//
// "PagedWeight", §3.3: the fused kernel reads the weight pages directly and
// follows the committed bitwidth of every gate_up and down block. Here each
// workgroup reads its block's q_i once from the device page table and runs the
// matching instantiation, so a launch mixes bitwidths freely and a change of
// q_i between launches takes effect on the next launch.
//
// Mapping (MFMA 32x32x16 fp16 -> fp32): a wave owns 32 weight rows. Lane l
// holds row l%32 and, per step, word w0 + l/32 of that row (32 elements) from
// each of the q plane pages; the 32 weights of the word feed four MFMAs as the
// A operand. The B operand is 32 tokens of the expert's group, element-aligned
// with the A words. Weights are dequantised once per step and reused for every
// 32-token chunk the workgroup holds.
#include "mpb_device.h"
#include "mpb_internal.h"

namespace mpb {

constexpr int MAXC = kDecodeChunks;

// ---------------------------------------------------------------- gate_up
template <int Q, int XDT>
__device__ void gate_up_body(const FfnParams& p, int e, int it, int t0, int nt, uint16_t* lds) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, r = lane & 31, g = lane >> 5;
  const int I = p.I, H = p.H, Wd = H >> 5;
  const int c0 = it * 128 + w * 32;  // first h column (gate row) of this wave
  const bool active = c0 < I;
  const int nch = (nt + 31) >> 5;
  const int base = p.offsets[e] + t0;
  const uint32_t slot = lut_slot(r, w);

  const uint16_t* xrow[MAXC];
  bool xv[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int j = 32 * c + r;
    xv[c] = j < nt;
    const int tok = xv[c] ? p.ptok[base + j] : 0;
    xrow[c] = p.X + (size_t)tok * H + 32 * g;
  }
  const int blk = 2 * e;
  const uint16_t* lut = p.luts[blk * 6 + (Q - 3)];
  f32x16 accg[MAXC], accu[MAXC];

#pragma unroll
  for (int ph = 0; ph < 2; ++ph) {
    const int row0 = ph * I + c0;
    if (active) stage_luts<Q>(lds, lut, row0, lane, w);
    __syncthreads();
    if (active) {
      f32x16 acc[MAXC];
#pragma unroll
      for (int c = 0; c < MAXC; ++c) acc[c] = (f32x16){};
      const uint32_t* pp[Q];
#pragma unroll
      for (int q = 0; q < Q; ++q) pp[q] = p.planes[blk * 8 + q] + (size_t)(row0 >> 5) * Wd * 32 + 32 * g + r;
      for (int w0 = 0; w0 < Wd; w0 += 2) {
        uint32_t P[Q];
#pragma unroll
        for (int q = 0; q < Q; ++q) P[q] = pp[q][w0 * 32];
        uint32_t O[8];
        assemble<Q>(P, O);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const f16x8 a = lookup8(lds, O[2 * m], O[2 * m + 1], slot);
#pragma unroll
          for (int c = 0; c < MAXC; ++c) {
            if (c < nch) {
              const f16x8 b = xv[c] ? load_x8<XDT>(xrow[c] + 32 * w0 + 8 * m) : (f16x8){};
              acc[c] = mfma32(a, b, acc[c]);
            }
          }
        }
      }
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        if (ph == 0) accg[c] = acc[c];
        else accu[c] = acc[c];
      }
    }
    __syncthreads();
  }
  if (!active) return;
  // acc[c][v] is row 8*(v/4) + 4*g + v%4 of the wave's 32 rows, token slot r
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int j = 32 * c + r;
    if (c < nch && j < nt) {
      float* hrow = p.h + (size_t)(base + j) * I + c0 + 4 * g;
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        f32x4 o;
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = silu(accg[c][4 * v4 + k]) * accu[c][4 * v4 + k];
        *(f32x4*)(hrow + 8 * v4) = o;
      }
    }
  }
}

template <int XDT>
__global__ __launch_bounds__(256) void k_gate_up_decode(FfnParams p) {
  __shared__ __attribute__((aligned(256))) uint16_t lds[32768];
  const int nit = (p.I + 127) >> 7;
  const int e = blockIdx.x / nit, it = blockIdx.x - e * nit;
  const int cnt = p.counts[e];
  const int t0 = blockIdx.y * kDecodeTokensPerWG;
  if (t0 >= cnt) return;
  const int nt = min(cnt - t0, kDecodeTokensPerWG);
  switch (p.q[2 * e]) {
    case 3: gate_up_body<3, XDT>(p, e, it, t0, nt, lds); break;
    case 4: gate_up_body<4, XDT>(p, e, it, t0, nt, lds); break;
    case 5: gate_up_body<5, XDT>(p, e, it, t0, nt, lds); break;
    case 6: gate_up_body<6, XDT>(p, e, it, t0, nt, lds); break;
    case 7: gate_up_body<7, XDT>(p, e, it, t0, nt, lds); break;
    case 8: gate_up_body<8, XDT>(p, e, it, t0, nt, lds); break;
    default: break;
  }
}

// ---------------------------------------------------------------- down
// B operand = h (fp32) split into fp16 hi + lo parts, two MFMAs per step, so h
// keeps ~22 significant bits through the contraction.
template <int Q>
__device__ void down_body(const FfnParams& p, int e, int nt_, int t0, int nt, uint16_t* lds) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, r = lane & 31, g = lane >> 5;
  const int I = p.I, H = p.H, Wd = I >> 5;
  const int n0 = nt_ * 128 + w * 32;
  const bool active = n0 < H;
  const int nch = (nt + 31) >> 5;
  const int base = p.offsets[e] + t0;
  const uint32_t slot = lut_slot(r, w);
  const int blk = 2 * e + 1;
  if (active) stage_luts<Q>(lds, p.luts[blk * 6 + (Q - 3)], n0, lane, w);
  __syncthreads();
  if (!active) return;

  const float* hrow[MAXC];
  bool hv[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int j = 32 * c + r;
    hv[c] = j < nt;
    hrow[c] = p.h + (size_t)(base + (hv[c] ? j : 0)) * I + 32 * g;
  }
  f32x16 acc[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) acc[c] = (f32x16){};
  const uint32_t* pp[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) pp[q] = p.planes[blk * 8 + q] + (size_t)(n0 >> 5) * Wd * 32 + 32 * g + r;
  for (int w0 = 0; w0 < Wd; w0 += 2) {
    uint32_t P[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) P[q] = pp[q][w0 * 32];
    uint32_t O[8];
    assemble<Q>(P, O);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const f16x8 a = lookup8(lds, O[2 * m], O[2 * m + 1], slot);
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        if (c < nch) {
          f32x4 v0 = (f32x4){}, v1 = (f32x4){};
          if (hv[c]) {
            v0 = *(const f32x4*)(hrow[c] + 32 * w0 + 8 * m);
            v1 = *(const f32x4*)(hrow[c] + 32 * w0 + 8 * m + 4);
          }
          f16x8 hi, lo;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            hi[j] = (_Float16)v0[j];
            lo[j] = (_Float16)(v0[j] - (float)hi[j]);
            hi[4 + j] = (_Float16)v1[j];
            lo[4 + j] = (_Float16)(v1[j] - (float)hi[4 + j]);
          }
          acc[c] = mfma32(a, hi, acc[c]);
          acc[c] = mfma32(a, lo, acc[c]);
        }
      }
    }
  }
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int j = 32 * c + r;
    if (c < nch && j < nt) {
      float* yrow = p.y + (size_t)(base + j) * H + n0 + 4 * g;
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        f32x4 o;
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = acc[c][4 * v4 + k];
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

hipError_t launch_gate_up(const FfnParams& p, int xdt, hipStream_t s) {
  const int ty = (p.T + kDecodeTokensPerWG - 1) / kDecodeTokensPerWG;
  const dim3 g1(p.NB * ((p.I + 127) >> 7), ty);
  if (xdt == 0) hipLaunchKernelGGL(k_gate_up_decode<0>, g1, dim3(256), 0, s, p);
  else hipLaunchKernelGGL(k_gate_up_decode<1>, g1, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_down(const FfnParams& p, hipStream_t s) {
  const int ty = (p.T + kDecodeTokensPerWG - 1) / kDecodeTokensPerWG;
  const dim3 g2(p.NB * ((p.H + 127) >> 7), ty);
  hipLaunchKernelGGL(k_down_decode, g2, dim3(256), 0, s, p);
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
