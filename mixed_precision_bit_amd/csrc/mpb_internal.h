// Host-side declarations shared by the libmpb translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mpb {

// Tokens per MFMA tile column block: a work item of the FFN kernels holds
// TC chunks of kChunkTokens tokens of one group.
constexpr int kChunkTokens = 32;

// Token chunks per work item of the gate_up kernel: one dequantised weight
// operand feeds TC MFMAs, one per 32-token chunk, so large groups (prefill)
// take four chunks and decode-size groups one. The down kernel always takes
// one (with its two MFMAs per word, h hi and lo, more chunks cost more in
// registers and LDS reads than the shared dequantisation saves). Two chunks
// for groups of 24 to 95 tokens (one item per Mixtral-shaped decode expert)
// were measured slower in both kernels: the second accumulator takes the
// kernels to three waves per SIMD, which costs more than the dequantisation
// it saves. Decided from the shapes only (the workspace layout depends on it).
inline int ffn_token_chunks(int T, int E, int K) {
  const long long avg = (long long)T * K / E;  // tokens per routed group on average
  return avg >= 96 ? 4 : 1;
}

struct FfnParams {
  const uint16_t* xh;         // [T][H] fp16 activations (converted copy for bf16 input)
  const int32_t* xsc;         // [T] per-token scale exponent of the converted copy, or null (fp16 input)
  int T, H, I, E, S, K, NB;   // NB = E + S
  const int32_t* topk_idx;    // [T][K]
  const float* topk_w;        // [T][K]
  const uint32_t* const* planes;  // [2*NB][8]
  const uint16_t* const* luts;    // [2*NB][6] table images (k_pack_table layout)
  const int32_t* q;           // [2*NB]
  // workspace
  int32_t* counts;            // [NB]
  int32_t* offsets;           // [NB+1]
  int32_t* ptok;              // [P] token of each grouped entry
  float* pw;                  // [P] routing weight of each entry
  int32_t* ent;               // [P] (token, slot) of each grouped entry: t (K + S) + slot
  int32_t* items;             // [max_items] gate_up work items: (group << 16) | token split
  int32_t* items_dn;          // [max_items] down work items, same encoding
  int32_t* n_items;           // [4] number of valid items: gate_up, down, wide gate_up, wide down
  int max_items;              // capacity of items (host bound)
  int tpi;                    // gate_up tokens per item: kChunkTokens * TC
  int tpi_dn;                 // down tokens per item: kChunkTokens
  // wide items (groups of at least wide_from tokens; 0: none): the grouped-GEMM
  // kernels of k_ffn_wide.hip take them, the kernels above only the other groups
  int32_t* items_w;           // [max_items_w] wide gate_up items, same encoding (tpi_w tokens each)
  int32_t* items_dnw;         // [max_items_w] wide down items (tpi_dnw tokens each)
  int max_items_w;            // capacity of items_w and items_dnw
  int wide_from;              // smallest group that takes the wide kernels (0: none)
  int tpi_w;                  // wide gate_up tokens per item
  int tpi_dnw;                // wide down tokens per item
  uint16_t* hhi;              // [P][I] fp16 high part of h = SiLU(gate) * up
  uint16_t* hlo;              // [P][I] fp16 remainder h - hi
  int32_t* wblk;              // [NB] first h panel block of each wide group
  uint16_t* hpan;             // h of the wide groups as down operand panels (k_ffn_wide.hip)
  float* y;                   // [dn_split][T (K + S)][H] down projection of each (token, slot) (partial sums over K ranges)
  float* out;                 // [T][H]
  int dn_split;               // K ranges of the down projection (1: whole K per workgroup)
  int dn_hcs;                 // half-chunks (64 elements) per K range, even
};

// Down-projection K split: a layer whose down launch would hold fewer than
// 1024 workgroups (few, long items: Mixtral-shaped experts) splits K into
// ranges of whole 128-element chunks, one workgroup each, with at least 16
// half-chunks per range; the combine pass adds the partial sums in range
// order. Decided from the shapes only (the workspace layout depends on it).
inline int dn_splits(int T, int H, int I, int E, int S, int K) {
  const long long P = (long long)T * (K + S), NB = (long long)E + S;
  const long long items = (P < NB ? P : NB) + P / kChunkTokens;
  const long long wgs = items * ((H + 127) / 128);
  if (wgs >= 1024) return 1;
  long long sp = (1536 + wgs - 1) / (wgs > 0 ? wgs : 1);
  const long long most = (I / 64) / 16;
  if (sp > most) sp = most;
  return sp < 1 ? 1 : (int)sp;
}
// half-chunks per K range for n ranges of HC half-chunks (even, ranges cover HC)
inline int dn_range_hcs(int I, int n) {
  const int HC = I / 64;
  const int per = (HC + n - 1) / n;
  return (per + 1) & ~1;
}

struct WsLayout {
  size_t counts, offsets, ptok, pw, ent, items, items_dn, items_w, items_dnw, wblk, n_items, ccnt, hhi, hlo, hpan,
      y, xh, xsc, total;
  size_t hpan_size;  // bytes of the h panels (0 without wide items)
  int max_items, max_items_w;
};
// Upper bound on work items (one per tpi-token split of a group with tokens):
// sum_g ceil(cnt_g / tpi) <= min(NB, P) + P / tpi for P grouped entries; the
// down list (tpi = kChunkTokens) is the longer one.
inline int max_decode_items(int T, int E, int S, int K) {
  const long long P = (long long)T * (K + S), NB = (long long)E + S;
  return (int)((P < NB ? P : NB) + P / kChunkTokens);
}
WsLayout ws_layout(int T, int H, int I, int E, int S, int K, bool bf16);

// Wide items: a group of at least kWideFrom tokens runs as a grouped GEMM whose
// workgroups dequantise a 128-row weight tile once per K step into LDS and
// multiply it with kWideTokGu (gate_up) or kWideTokDn (down: h hi and lo, two
// columns per token) tokens. Used where a layer's groups can reach that size
// (batches of at least kWideBatch tokens: smaller ones hold too few such
// groups to fill the chip with these long workgroups, and their 32-token items
// finish sooner) and its down projection is not split over K ranges.
constexpr int kWideFrom = 96;
constexpr int kWideBatch = 2048;
constexpr int kWideTokGu = 512;
constexpr int kWideTokDn = 256;
inline int ffn_wide_from(int T, int H, int I, int E, int S, int K) {
  return T >= kWideBatch && dn_splits(T, H, I, E, S, K) == 1 ? kWideFrom : 0;
}
// Upper bound on wide items of either list: sum_g ceil(cnt_g / kWideTokDn) over
// groups of at least kWideFrom entries.
inline int max_wide_items(int T, int E, int S, int K) {
  const long long P = (long long)T * (K + S), NB = (long long)E + S;
  const long long g = P / kWideFrom;
  return (int)(P / kWideTokDn + (g < NB ? g : NB));
}

// h panels of the wide groups: one per 32-token block of a group and 64-row
// step of I, hi then lo, 4 KiB each; a group's blocks are consecutive. Upper
// bound on the blocks: sum_g ceil(cnt_g / 32) <= P / 32 + NB.
inline size_t hpan_bytes(int T, int I, int E, int S, int K) {
  const size_t P = (size_t)T * (K + S);
  return ((P + 31) / 32 + (size_t)E + S) * (size_t)I * 128;
}

// The FFN kernels stage activation and h rows through buffer descriptors with
// 32-bit byte offsets, kNoRow standing for "no row" (reads as zeros): the
// activations ([T][H] fp16), the span of h's two halves and the h panels must
// stay below it.
constexpr uint32_t kNoRow = 0xfffffff0u;
inline bool rows_fit(const WsLayout& L, int T, int H, int I, int K, int S) {
  const size_t P = (size_t)T * (K + S);
  return (size_t)T * H * 2 < kNoRow && (L.hlo - L.hhi) + P * I * 2 < kNoRow && L.hpan_size < kNoRow;
}

// Raise a kernel's dynamic LDS limit to `bytes` on the current device, once
// per device (bit d of `done` records device d; the library is driven from
// one host thread).
inline hipError_t raise_lds_limit(const void* fn, int bytes, unsigned long long& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const unsigned long long bit = dev < 64 ? 1ull << dev : 0ull;
  if (done & bit) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done |= bit;
  return e;
}

hipError_t launch_pack(const uint32_t* canon, int N, int Kd, uint32_t* const* pages, hipStream_t s);
hipError_t launch_pack_table(const uint16_t* lut, int kind, int N, int b, uint16_t* img, hipStream_t s);
hipError_t launch_dequant(const uint32_t* const* pages, const uint16_t* lut, int N, int Kd, int b,
                          uint16_t* out, hipStream_t s);
hipError_t launch_dequant_image(const uint32_t* const* pages, const uint16_t* img, int kind, int N, int Kd, int b,
                                uint16_t* out, hipStream_t s);
size_t route_workspace_bytes(int T, int E);
hipError_t launch_routing_mass(const int32_t* idx, const float* w, int T, int E, int K, double* mass,
                               hipStream_t s);
hipError_t launch_route(const uint16_t* X, int xdt, const float* W, const float* bias, int T, int H,
                        int E, int K, int32_t* idx, float* w, double* logits, hipStream_t s);
// Grouping: one pass per group for small batches; for T*K >= kChunkedFrom the
// routed ids are processed in chunks of kGroupChunk (group_chunks(T, K)
// chunks, 0 below the threshold), with ccnt = [chunks][E] int32 scratch.
constexpr int kGroupChunk = 2048;
constexpr long long kChunkedFrom = 8192;
int group_chunks(int T, int K);
hipError_t launch_permute(const FfnParams& p, int32_t* ccnt, hipStream_t s);
// bf16 activations [T][H] -> fp16 y = x * 2^-sc[t] per token: sc[t] = 0 (a
// plain conversion) when every finite |x| of the token is below 2^15, else the
// shift that brings them below 2^8
hipError_t launch_x_to_f16(const uint16_t* x, uint16_t* y, int32_t* sc, int T, int H, hipStream_t s);
// qmax: highest committed bitwidth among the launch's blocks (sizes the LDS
// table region; a block above it yields NaN)
// ev0/ev1: optional events the launch records at the kernel's start and end
hipError_t launch_gate_up(const FfnParams& p, int qmax, int tc, hipStream_t s, hipEvent_t ev0 = nullptr,
                          hipEvent_t ev1 = nullptr);
// the variants with full double-buffered stages (their own translation unit)
hipError_t launch_gate_up_df(const FfnParams& p, int qmax, int tc, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1);
hipError_t launch_down_df(const FfnParams& p, int qmax, bool nt, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1);
// nt: non-temporal plane loads (decode-size batches, one item per group)
// ev0/ev1: optional events the launch records at the kernel's start and end
hipError_t launch_down(const FfnParams& p, int qmax, bool nt, hipStream_t s, hipEvent_t ev0 = nullptr,
                       hipEvent_t ev1 = nullptr);
hipError_t launch_combine(const FfnParams& p, hipStream_t s);
// The wide (grouped-GEMM) gate_up and down launches; no-ops when p.wide_from is 0.
hipError_t launch_wide(const FfnParams& p, bool gu, int qmax, hipStream_t s, hipEvent_t ev0 = nullptr,
                       hipEvent_t ev1 = nullptr);
hipError_t launch_set_q(int32_t* q, int i, int b, hipStream_t s);

// The whole layer in one persistent launch (k_fused.hip).
struct FusedLaunch {
  FfnParams f;          // FFN view of the call (tpi = tpi_dn = kChunkTokens)
  const uint16_t* x;    // activations as given
  int xdt;              // 0 fp16, 1 bf16
  const float* W;       // router weights [E][H]
  const float* bias;    // [E] or null
  double* logits;       // [T][E] workspace
  int32_t* idx_out;     // [T][K]
  float* w_out;         // [T][K]
  uint32_t* ctr;        // fused_counter_bytes() of counters, zero at launch
  int qmax;             // highest committed bitwidth (sizes the table region)
};
size_t fused_counter_bytes();
hipError_t launch_fused(const FusedLaunch& L, hipStream_t s);

// Records msg as the calling thread's last error and returns code.
int set_error(int code, const char* msg);
// Checks a layer geometry against the ranges the library supports; on failure
// returns false and points *why at a message.
bool geometry_ok(int H, int I, int E, int S, int K, const char** why);

}  // namespace mpb
