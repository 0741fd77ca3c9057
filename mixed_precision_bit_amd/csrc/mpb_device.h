// Device-side building blocks shared by every kernel that reads Any-Precision
// weights: the packed bit-plane word layout, index assembly from the top q
// planes, the LDS staging of per-row centroid tables and the table lookup.
//
// Source: "PagedWeight: Efficient MoE LLM Serving with Dynamic Quality-Aware
// Weight Quantization", §2.2 (a b-bit weight is a subset of the bit-planes
// plus the b-bit lookup table) and §3.3 (the fused kernel reads the planes and
// tables directly at each block's committed bitwidth).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

namespace mpb {

// ----------------------------------------------------------------------------
// Packed plane page layout.
//
// A page holds one bit-plane of an [N][Kd] block. Rows are grouped in tiles of
// 32; each row's W = Kd/32 words are grouped in chunks of 4 (128 elements),
// NC = ceil(W/4) chunks per row, the last one zero-padded. Chunk c of row n is
// 16 contiguous bytes at word ((n/32 * NC + c) * 32 + n%32) * 4, so a wave whose
// 32 lanes hold 32 rows reads one chunk of each with a single 512-byte
// dwordx4 access.
//
// Inside a word, element e = 4*s + b (s = 0..7, b = 0..3) of plane p sits at
// bit (8*b + s + p) mod 32: plane p is the word with element 4s+b at bit
// 8b + s, rotated left by p. With that placement the q-bit indices come out
// of q plane words with bit-field inserts alone (assemble).
// ----------------------------------------------------------------------------
__host__ __device__ constexpr int packed_pos(int e, int p) { return (8 * (e & 3) + (e >> 2) + p) & 31; }

__host__ __device__ constexpr int page_chunks(int Kd) { return (Kd / 32 + 3) / 4; }

__host__ __device__ constexpr size_t page_word(int n, int w, int NC) {
  return (((size_t)(n >> 5) * NC + (w >> 2)) * 32 + (n & 31)) * 4 + (w & 3);
}

__host__ __device__ constexpr uint32_t rotl_c(uint32_t x, int r) {
  return (r & 31) ? (x << (r & 31)) | (x >> (32 - (r & 31))) : x;
}

// (a & m) | (c & ~m): one v_bfi_b32 (the compiler matches this form).
__device__ __forceinline__ uint32_t bfi(uint32_t m, uint32_t a, uint32_t c) { return (a & m) | (c & ~m); }

// Index assembly. P[p] = plane-p word (p < Q) of one (row, word). On return
// byte b of O[s] is u = sum_p bit_p(e=4s+b) << p, the Q-bit index with its bit
// order reversed (plane 0, the code MSB, lands in bit 0). Tables are staged in
// the same reversed order, so no per-weight reversal is needed.
//
// Per byte lane b this is the transpose of an 8x8 bit matrix: row p (plane
// p) holds, at bit s, plane p of element 4s+b, and row s of the result must
// hold, at bit p, the same bit. It runs as the usual three rounds of block
// swaps (4x4, 2x2, 1x1 blocks), each of which moves bits k = 4, 2, 1 places
// between rows p and p+k. Because plane p is stored rotated left by p bits
// (packed_pos), row p+k already sits k bits to the left of row p, so each new
// row is one bit-field insert of the two old rows under a rotated mask; no
// shift is needed (rotating instead of shifting only moves bits into positions
// the mask takes from the other row). Row s ends rotated by s and is rotated
// back once. Cost per 32 elements: 24 inserts and 7 rotates for every Q (the
// and-or gathering it replaces took 8Q + 7). Rows at and above Q are a zero
// the compiler cannot see through: folded constants turned the inserts into
// longer and/or sequences.
template <int K>
__device__ __forceinline__ void bfly_round(uint32_t (&X)[8], uint32_t M) {
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    if (p & K) continue;
    const uint32_t a = X[p], c = X[p + K];
    X[p] = bfi(rotl_c(M, p), a, c);
    X[p + K] = bfi(rotl_c(M, p + K), a, c);
  }
}

template <int Q>
__device__ __forceinline__ void assemble(const uint32_t (&P)[Q], uint32_t (&O)[8]) {
  uint32_t z = 0u;
  asm("" : "+v"(z));
  uint32_t X[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) X[p] = p < Q ? P[p] : z;
  bfly_round<4>(X, 0x0F0F0F0Fu);
  bfly_round<2>(X, 0x33333333u);
  bfly_round<1>(X, 0x55555555u);
#pragma unroll
  for (int s = 0; s < 8; ++s) O[s] = s ? __builtin_amdgcn_alignbit(X[s], X[s], s) : X[s];
}

// Pair indices of two words at 3 bits. PA/PB = planes 0..2 of word A and word
// B of one (row, half-chunk). On return byte b of O[s] is
//   hb + 2 (uA + 8 uB),
// uA, uB the reversed 3-bit indices of element 4s+b of word A and word B and
// hb = 1 when h (wave-uniform) is set: the same transpose with word A's planes
// in rows 1..3, word B's in rows 4..6 and row 0 all ones or all zeros.
// Rows 1..3 need their plane rotated left by one more bit than stored, rows
// 4..6 by four more.
__device__ __forceinline__ void assemble_pairs3(const uint32_t (&PA)[3], const uint32_t (&PB)[3], bool h,
                                                uint32_t (&O)[8]) {
  uint32_t z = 0u;
  asm("" : "+v"(z));
  uint32_t X[8];
  X[0] = h ? ~z : z;
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    X[1 + q] = __builtin_amdgcn_alignbit(PA[q], PA[q], 31);  // rotl 1
    X[4 + q] = __builtin_amdgcn_alignbit(PB[q], PB[q], 28);  // rotl 4
  }
  X[7] = z;
  bfly_round<4>(X, 0x0F0F0F0Fu);
  bfly_round<2>(X, 0x33333333u);
  bfly_round<1>(X, 0x55555555u);
#pragma unroll
  for (int s = 0; s < 8; ++s) O[s] = s ? __builtin_amdgcn_alignbit(X[s], X[s], s) : X[s];
}

template <int Q>
__device__ __forceinline__ uint32_t bitrev(uint32_t v) {
  return __builtin_bitreverse32(v) >> (32 - Q);
}

// ----------------------------------------------------------------------------
// LDS centroid tables.
//
// A workgroup of up to 4 waves keeps, for each wave, the tables of the 32 rows
// it is dequantising. Entry u (reversed index, see assemble) of row r of wave w
// is the fp16 at byte
//     u * 256 + slot(r, w),   slot(r, w) = 4*r + 2*(w & 1) + 128*(w >> 1).
// Row r always lives in LDS bank r (dword address = 64u + r + 32*(w>>1)), so the
// 32 lanes of a half-wave, which hold 32 different rows, never conflict. The
// table region starts at LDS byte 0 and spans 2^Q * 256 bytes (64 KiB at Q=8).
// ----------------------------------------------------------------------------
__device__ __forceinline__ uint32_t lut_slot(int r, int w) {
  return 4u * r + 2u * (w & 1) + 128u * (w >> 1);
}

// Stage the Q-bit tables of rows row0..row0+31 (canonical [N][2^Q] fp16 at
// lut, canonical index order) into table slot set w. Called by all 64 lanes of
// one wave; lane (r, half) copies 16-byte pieces half, half+2, ... of row r.
// Split in a load phase and a store phase so that a caller can issue other
// loads between them.
template <int Q>
struct LutPieces {
  static constexpr int NP = (1 << Q) / 8;  // 16-byte pieces per row
  static constexpr int NI = (NP + 1) / 2;  // pieces per lane
  uint4 v[NI];
};

template <int Q>
__device__ __forceinline__ void load_luts(LutPieces<Q>& L, const uint16_t* __restrict__ lut, int row0, int lane) {
  const int r = lane & 31, half = lane >> 5;
  const uint4* src = (const uint4*)(lut + (size_t)(row0 + r) * (1u << Q));
#pragma unroll
  for (int i = 0; i < LutPieces<Q>::NI; ++i)
    if (half + 2 * i < LutPieces<Q>::NP) L.v[i] = src[half + 2 * i];
}

template <int Q>
__device__ __forceinline__ void store_luts(uint16_t* lds, const LutPieces<Q>& L, int lane, int w) {
  const int r = lane & 31, half = lane >> 5;
  const uint32_t slot = lut_slot(r, w);
#pragma unroll
  for (int i = 0; i < LutPieces<Q>::NI; ++i) {
    if (half + 2 * i < LutPieces<Q>::NP) {
      const uint32_t wd[4] = {L.v[i].x, L.v[i].y, L.v[i].z, L.v[i].w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t u = bitrev<Q>(8 * (half + 2 * i) + j);
        lds[(u * 256u + slot) >> 1] = (uint16_t)(wd[j >> 1] >> (16 * (j & 1)));
      }
    }
  }
}

template <int Q>
__device__ __forceinline__ void stage_luts(uint16_t* lds, const uint16_t* __restrict__ lut, int row0,
                                           int lane, int w) {
  LutPieces<Q> L;
  load_luts<Q>(L, lut, row0, lane);
  store_luts<Q>(lds, L, lane, w);
}

// LDS byte address of the entry named by byte b of an assembled word O.
__device__ __forceinline__ uint32_t lut_addr(uint32_t O, uint32_t slot, int b) {
  // result byte 0 = slot, byte 1 = O.byte[b], bytes 2..3 = 0
  return __builtin_amdgcn_perm(O, slot, 0x0c0c0000u | ((4u + (uint32_t)b) << 8));
}

// Table reads address LDS directly by byte offset: the table region must start
// at LDS byte 0 (the kernels that use it hold no other LDS object in front of
// it; tables_at_zero checks this). Going through the shared array's generic
// pointer instead costs one add per lookup.
typedef const __attribute__((address_space(3))) uint16_t lds_u16;

__device__ __forceinline__ bool tables_at_zero(const void* lds) { return (uint32_t)(uintptr_t)lds == 0u; }

__device__ __forceinline__ _Float16 lut_read(uint32_t addr) {
  return __builtin_bit_cast(_Float16, *(lds_u16*)(uintptr_t)addr);
}

// ----------------------------------------------------------------------------
// Pair tables (3-bit blocks). A 128-row tile's 3-bit table expands in LDS into
// a table of 64 pairs per row: entry P = uA + 8 uB of tile row R = 32 g + r
// (row group g) is the dword at byte P * 512 + 4 R holding (LUT[uA],
// LUT[uB]), word A's value in the low half. With hb = g >> 1 in bit 0 of the
// assembled pair byte (assemble_pairs3) and pair_slot below, lut_addr gives
// the entry's address, and one ds_read_b32 yields two dequantised weights
// packed as the MFMA operand wants them (half the table reads of lookup8 and
// no packing). Lanes r = 0..31 hit banks r.
// ----------------------------------------------------------------------------
constexpr uint32_t kPairTableBytes = 64u * 512u;

__device__ __forceinline__ uint32_t pair_slot(int r, int g) { return 4u * r + 128u * (g & 1); }

// Builds the pair table at LDS byte 0 from the tile's 3-bit table image,
// already copied to LDS at byte `src` (image layout of lut_slot). Every
// thread of a 512-thread workgroup writes 16 entries of one row. The caller
// synchronises the workgroup before and after.
__device__ __forceinline__ void build_pair_table3(uint32_t src, int tid) {
  typedef __attribute__((address_space(3))) uint32_t lds_u32;
  const int R = tid & 127, p0 = tid >> 7;
  const uint32_t ss = src + lut_slot(R & 31, R >> 5);
  uint32_t T[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) T[u] = *(lds_u16*)(uintptr_t)(ss + 256u * u);
  const uint32_t a0 = *(lds_u16*)(uintptr_t)(ss + 256u * p0), a1 = *(lds_u16*)(uintptr_t)(ss + 256u * (p0 + 4));
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int P = p0 + 4 * i;  // uA = p0 + 4 (i & 1), uB = i >> 1
    *(lds_u32*)(uintptr_t)(P * 512u + 4u * R) = ((i & 1) ? a1 : a0) | (T[i >> 1] << 16);
  }
}

// Eight dequantised weights from one assembled pair word: the pairs of
// elements 4s..4s+3 of words A and B, as an MFMA A-operand (A, B alternating).
__device__ __forceinline__ f16x8 lookup_pairs4(uint32_t O, uint32_t slot) {
  typedef const __attribute__((address_space(3))) uint32_t lds_cu32;
  uint32_t v[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) v[b] = *(lds_cu32*)(uintptr_t)lut_addr(O, slot, b);
  return __builtin_bit_cast(f16x8, v);
}

// Eight dequantised weights, elements 8m..8m+7 of the word (O0 = O[2m],
// O1 = O[2m+1]), as an MFMA A-operand.
__device__ __forceinline__ f16x8 lookup8(uint32_t O0, uint32_t O1, uint32_t slot) {
  f16x8 a;
#pragma unroll
  for (int b = 0; b < 4; ++b) a[b] = lut_read(lut_addr(O0, slot, b));
#pragma unroll
  for (int b = 0; b < 4; ++b) a[4 + b] = lut_read(lut_addr(O1, slot, b));
  return a;
}

// ----------------------------------------------------------------------------
// Activations: bf16 -> fp16 conversion of 8 consecutive elements (16-byte
// aligned), scaled by 2^-sc. The fp16 range ends at 65504, the bf16 one near
// 3.4e38: a token holding larger values is converted scaled down by a power
// of two (exact) and the FFN kernels undo the scale in fp32, so it stays on
// the fp16 matrix cores without overflowing.
// ----------------------------------------------------------------------------
// Largest biased exponent among the finite bf16 values of 8 elements (0 for zeros).
__device__ __forceinline__ int max_exp8_bf16(const uint16_t* p) {
  const u16x8 v = *(const u16x8*)p;
  int m = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int e = (v[j] >> 7) & 0xff;
    m = e == 0xff ? m : max(m, e);
  }
  return m;
}
// Scale shift of a token whose largest finite |x| has biased bf16 exponent
// emax, i.e. |x| < 2^(emax - 126): 0 when every |x| < 2^15 (the conversion is
// exact in the fp16 normal range), else the shift that brings |x| below 2^8,
// which also leaves room for h = SiLU(gate) * up, quadratic in x, carried at
// 2^(-2 sc) through fp16.
__device__ __forceinline__ int x_scale_shift(int emax) { return emax > 141 ? emax - 134 : 0; }

// bf16 -> fp16 of x * 2^-sc (exact for results in the fp16 normal range;
// rounded below it).
__device__ __forceinline__ f16x8 load_x8_bf16(const uint16_t* p, int sc = 0) {
  const u16x8 v = *(const u16x8*)p;
  f16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    r[j] = (_Float16)__builtin_amdgcn_ldexpf(__builtin_bit_cast(float, (uint32_t)v[j] << 16), -sc);
  return r;
}

__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// h = hi + lo with hi = fp16(h) and lo = fp16(h - hi). h is pinned to one fp32
// value first: otherwise floating-point contraction may fold the product that
// produced h into the two conversions separately (v_fma_mix), rounding hi two
// different ways and making hi + lo wrong by one fp16 ulp near rounding ties.
struct split16 {
  _Float16 hi, lo;
};
__device__ __forceinline__ split16 split_hi_lo(float h) {
  asm volatile("" : "+v"(h));
  const _Float16 hi = (_Float16)h;
  const float r = h - (float)hi;  // exact: hi is within half an fp16 ulp of h
  return {hi, (_Float16)r};
}

}  // namespace mpb
