// Host-side declarations shared by the libmpb translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mpb {

// Token chunks of 32 held per workgroup by the decode FFN kernels.
constexpr int kDecodeChunks = 2;
constexpr int kDecodeTokensPerWG = 32 * kDecodeChunks;

struct FfnParams {
  const uint16_t* xh;         // [T][H] fp16 activations (converted copy for bf16 input)
  int T, H, I, E, S, K, NB;   // NB = E + S
  const int32_t* topk_idx;    // [T][K]
  const float* topk_w;        // [T][K]
  const uint32_t* const* planes;  // [2*NB][8]
  const uint16_t* const* luts;    // [2*NB][6]
  const int32_t* q;           // [2*NB]
  // workspace
  int32_t* counts;            // [NB]
  int32_t* offsets;           // [NB+1]
  int32_t* ptok;              // [P] token of each grouped entry
  float* pw;                  // [P] routing weight of each entry
  int32_t* inv;               // [T][K+S] entry position of (t, slot)
  uint16_t* hhi;              // [P][I] fp16 high part of h = SiLU(gate) * up
  uint16_t* hlo;              // [P][I] fp16 remainder h - hi
  float* y;                   // [P][H] per-entry down projection
  float* out;                 // [T][H]
};

struct WsLayout {
  size_t counts, offsets, ptok, pw, inv, hhi, hlo, y, xh, total;
};
WsLayout ws_layout(int T, int H, int I, int E, int S, int K, bool bf16);

hipError_t launch_pack(const uint32_t* canon, int N, int Kd, uint32_t* const* pages, hipStream_t s);
hipError_t launch_dequant(const uint32_t* const* pages, const uint16_t* lut, int N, int Kd, int b,
                          uint16_t* out, hipStream_t s);
hipError_t launch_route(const uint16_t* X, int xdt, const float* W, const float* bias, int T, int H,
                        int E, int K, int32_t* idx, float* w, hipStream_t s);
hipError_t launch_permute(const FfnParams& p, hipStream_t s);
hipError_t launch_x_to_f16(const uint16_t* x, uint16_t* y, size_t n, hipStream_t s);
hipError_t launch_gate_up(const FfnParams& p, hipStream_t s);
hipError_t launch_down(const FfnParams& p, hipStream_t s);
hipError_t launch_combine(const FfnParams& p, hipStream_t s);
hipError_t launch_set_q(int32_t* q, int i, int b, hipStream_t s);

}  // namespace mpb
