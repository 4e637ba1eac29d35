// device.h -- gfx950 device helpers shared by the libqlora kernels:
// vector types, the NF4 / Q8 codebooks, the byte-permute NF4 decoder,
// LDS tile addressing and the bf16 MFMA wrapper.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlora {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef uint16_t bf16_t;  // bf16 bit pattern in global memory

constexpr int kBlock = 64;         // weights per absmax block
constexpr int kGroupBlocks = 256;  // blocks per second-level group

// NF4 levels as fp32 bit patterns, ascending.  Construction (deepfa.ir blog,
// "1. 4-bit NormalFloat (NF4)": normal quantiles, equal mass per bucket,
// normalised to [-1, 1], exact zero): with delta = 929/960, 8 positive
// levels Phi^-1(delta + (1/2 - delta) j/8), j = 0..7, 7 negative levels
// -Phi^-1(delta + (1/2 - delta) j/7), j = 0..6, and 0, all divided by
// Phi^-1(delta) and rounded to fp32.
__constant__ constexpr uint32_t kNf4LevelBits[16] = {
    0xBF800000u, 0xBF3239B1u, 0xBF066B2Eu, 0xBECA329Eu, 0xBE91A24Bu, 0xBE3D353Du,
    0xBDBA7869u, 0x00000000u, 0x3DA2FB01u, 0x3E24CADFu, 0x3E7C04DAu, 0x3EAD0336u,
    0x3EE1A4B5u, 0x3F1007A9u, 0x3F3913B0u, 0x3F800000u};

// Encoder thresholds: T_k is the exact midpoint of levels k and k+1 rounded
// toward -inf to fp32.  For any fp32 x, #{k : x > T_k} is the index of the
// nearest level with ties going to the lower index.
__constant__ constexpr uint32_t kNf4ThreshBits[15] = {
    0xBF591CD9u, 0xBF1C5270u, 0xBEEB847Du, 0xBEADEA75u, 0xBE703CEAu,
    0xBE0D38B9u, 0xBD3A7869u, 0x3D22FB01u, 0x3DF6485Fu, 0x3E5067DCu,
    0x3E9582D1u, 0x3EC753F5u, 0x3F006D01u, 0x3F248DACu, 0x3F5C89D8u};

// The two other 4-bit codebooks that the pages compare NF4 with (deepfa.ir
// blog, "1. 4-bit NormalFloat (NF4)" and its results list), quantized and
// dequantized the same way.  FP4 is E2M1 (sign, two exponent bits with
// bias 1, one mantissa bit: +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}) divided by 6;
// its two zeros are both +0 (codes 7 and 8).  Int4 is k/7 for the
// two's-complement k = -8..7.  Levels rounded to fp32, ascending.
__constant__ constexpr uint32_t kFp4LevelBits[16] = {
    0xBF800000u, 0xBF2AAAABu, 0xBF000000u, 0xBEAAAAABu, 0xBE800000u, 0xBE2AAAABu,
    0xBDAAAAABu, 0x00000000u, 0x00000000u, 0x3DAAAAABu, 0x3E2AAAABu, 0x3E800000u,
    0x3EAAAAABu, 0x3F000000u, 0x3F2AAAABu, 0x3F800000u};
__constant__ constexpr uint32_t kInt4LevelBits[16] = {
    0xBF924925u, 0xBF800000u, 0xBF5B6DB7u, 0xBF36DB6Eu, 0xBF124925u, 0xBEDB6DB7u,
    0xBE924925u, 0xBE124925u, 0x00000000u, 0x3E124925u, 0x3E924925u, 0x3EDB6DB7u,
    0x3F124925u, 0x3F36DB6Eu, 0x3F5B6DB7u, 0x3F800000u};
// Their thresholds, as for NF4; FP4's zero pair gets the threshold of the
// next distinct pair twice (T_7 = T_8), so that code 8 is never produced
// (ties go to the lower index).
__constant__ constexpr uint32_t kFp4ThreshBits[15] = {
    0xBF555556u, 0xBF155556u, 0xBED55556u, 0xBE955556u, 0xBE555556u,
    0xBE000001u, 0xBD2AAAABu, 0x3D2AAAABu, 0x3D2AAAABu, 0x3E000000u,
    0x3E555555u, 0x3E955555u, 0x3ED55555u, 0x3F155555u, 0x3F555555u};
__constant__ constexpr uint32_t kInt4ThreshBits[15] = {
    0xBF892493u, 0xBF6DB6DCu, 0xBF492493u, 0xBF24924Au, 0xBF000001u,
    0xBEB6DB6Eu, 0xBE5B6DB8u, 0xBD924925u, 0x3D924925u, 0x3E5B6DB7u,
    0x3EB6DB6Eu, 0x3F000000u, 0x3F249249u, 0x3F492492u, 0x3F6DB6DBu};

// Codebook selectors (the values of qlora_codebook).
constexpr int kCbNf4 = 0, kCbFp4 = 1, kCbInt4 = 2;
template <int CB>
__device__ __forceinline__ uint32_t cb_level_bits(int i) {
  return CB == kCbNf4 ? kNf4LevelBits[i] : CB == kCbFp4 ? kFp4LevelBits[i] : kInt4LevelBits[i];
}
template <int CB>
__device__ __forceinline__ uint32_t cb_thresh_bits(int i) {
  return CB == kCbNf4 ? kNf4ThreshBits[i] : CB == kCbFp4 ? kFp4ThreshBits[i] : kInt4ThreshBits[i];
}
// The code of an all-zero block: the lowest index of a zero level.
template <int CB>
constexpr uint32_t cb_zero_code() { return CB == kCbInt4 ? 8u : 7u; }

__device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }

// Second-level code value Q8[q] = RN32(q / 255).  The fp64 product
// q * RN64(1/255) is within 2^-52 relative of q / 255, while q / 255 (an
// 8-bit by 8-bit quotient) is never closer than 2^-33 relative to an fp32
// rounding boundary, so rounding the product to fp32 gives RN32(q / 255)
// for every q in 0..255.
__device__ __forceinline__ float q8_value(uint32_t q) {
  return (float)((double)q * (1.0 / 255.0));
}

// bf16 bit pattern -> fp32 (exact)
__device__ __forceinline__ float bf2f(uint32_t b) { return u2f(b << 16); }

// Two fp32 -> packed bf16 pair {lo, hi}, round to nearest even
// (one v_cvt_pk_bf16_f32 on gfx950).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint32_t perm(uint32_t s0, uint32_t s1, uint32_t sel) {
  return __builtin_amdgcn_perm(s0, s1, sel);
}

// ---------------------------------------------------------------------------
// Byte-permute NF4 decoder.
//
// A per-block table of the 16 dequantized bf16 values v[c] = RNE_bf16(RN32(
// L[c] * t)) is kept as two byte planes of four dwords each: lo[j] holds the
// low bytes of v[4j..4j+3], hi[j] the high bytes.  v_perm_b32 selects bytes
// from a 64-bit pair with selectors 0..7 and returns 0xFF for selectors >= 13,
// so a 16-entry byte lookup is two perms ANDed: entries 0..7 use selector
// sa = c + (c & 8) (c for c < 8, >= 16 otherwise) and entries 8..15 use
// sb = sa ^ 0x10 (c - 8 for c >= 8, >= 16 otherwise).
// ---------------------------------------------------------------------------
struct Nf4Table {
  uint32_t lo[4];
  uint32_t hi[4];
};

template <int CB = kCbNf4>
__device__ __forceinline__ Nf4Table make_table(float t) {
  uint32_t p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    p[i] = pack_bf16x2(u2f(cb_level_bits<CB>(2 * i)) * t, u2f(cb_level_bits<CB>(2 * i + 1)) * t);
  Nf4Table T;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    T.lo[j] = perm(p[2 * j + 1], p[2 * j], 0x06040200u);
    T.hi[j] = perm(p[2 * j + 1], p[2 * j], 0x07050301u);
  }
  return T;
}

// Four lookups: idx holds four codes (0..15), one per byte.
__device__ __forceinline__ void lookup4(uint32_t idx, const Nf4Table& T, uint32_t& lo, uint32_t& hi) {
  const uint32_t sa = idx + (idx & 0x08080808u);
  const uint32_t sb = sa ^ 0x10101010u;
  lo = perm(T.lo[1], T.lo[0], sa) & perm(T.lo[3], T.lo[2], sb);
  hi = perm(T.hi[1], T.hi[0], sa) & perm(T.hi[3], T.hi[2], sb);
}

// Eight codes (one packed dword, element i in nibble i) -> eight bf16 in
// natural order: out[d] = {v[c_2d], v[c_2d+1]}.
__device__ __forceinline__ void dequant8(uint32_t c, const Nf4Table& T, uint32_t out[4]) {
  const uint32_t e = c & 0x0F0F0F0Fu;           // elements 0,2,4,6
  const uint32_t o = (c >> 4) & 0x0F0F0F0Fu;    // elements 1,3,5,7
  uint32_t le, he, lo, ho;
  lookup4(e, T, le, he);
  lookup4(o, T, lo, ho);
  const uint32_t l01 = perm(lo, le, 0x05010400u);   // lo bytes of elements 0..3
  const uint32_t h01 = perm(ho, he, 0x05010400u);
  const uint32_t l23 = perm(lo, le, 0x07030602u);   // lo bytes of elements 4..7
  const uint32_t h23 = perm(ho, he, 0x07030602u);
  out[0] = perm(h01, l01, 0x05010400u);
  out[1] = perm(h01, l01, 0x07030602u);
  out[2] = perm(h23, l23, 0x05010400u);
  out[3] = perm(h23, l23, 0x07030602u);
}

// Four consecutive codes (nibbles 0..3 of the low half, or 4..7 of the high
// half of c) spread into one byte each.
__device__ __forceinline__ uint32_t spread4(uint32_t c, bool high_half) {
  const uint32_t t = perm(0u, c, high_half ? 0x0C030C02u : 0x0C010C00u);
  return ((t << 4) | t) & 0x0F0F0F0Fu;
}

// Two rows of eight codes each (same columns) -> eight dwords, one per
// column k: out[k] = {v0[c0_k], v1[c1_k]}  (row pair packed along k-major).
__device__ __forceinline__ void dequant8x2_pairs(uint32_t c0, uint32_t c1, const Nf4Table& T0,
                                                 const Nf4Table& T1, uint32_t out[8]) {
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    uint32_t l0, h0, l1, h1;
    lookup4(spread4(c0, half), T0, l0, h0);
    lookup4(spread4(c1, half), T1, l1, h1);
    const uint32_t P = perm(l1, l0, 0x05010400u);
    const uint32_t Q = perm(h1, h0, 0x05010400u);
    const uint32_t P2 = perm(l1, l0, 0x07030602u);
    const uint32_t Q2 = perm(h1, h0, 0x07030602u);
    out[4 * half + 0] = perm(Q, P, 0x05010400u);
    out[4 * half + 1] = perm(Q, P, 0x07030602u);
    out[4 * half + 2] = perm(Q2, P2, 0x05010400u);
    out[4 * half + 3] = perm(Q2, P2, 0x07030602u);
  }
}

// Second-level formats of the block constants (the values of
// qlora_absmax_format): the linear code Q8 above, or FP8 E4M3 (sign 0, four
// exponent bits with bias 7, three mantissa bits, largest finite value 448)
// divided by 448: Q[q] = RN32(e4m3(q) / 448), q = 0..126.  e4m3(q) is
// (8 + m) 2^(e - 10) (exponent field e > 0) or m 2^-9 (e = 0), exact in fp64;
// the product with RN64(1/448) is within 2^-52 relative of the quotient,
// which is either exact in fp32 (8 + m = 14) or has the period-3 binary
// expansion of a seventh and so lies at least about 2^-27 relative from
// every fp32 rounding boundary: rounding the product gives RN32(e4m3 / 448).
constexpr int kAbsLinear = 0, kAbsFp8 = 1;
__device__ __forceinline__ float fp8_value(uint32_t q) {
  const uint32_t e = (q >> 3) & 15u, m = q & 7u;
  const double v = e ? (double)(8u + m) * (double)(1u << e) * (1.0 / 1024.0) : (double)m * (1.0 / 512.0);
  return (float)(v * (1.0 / 448.0));
}
__device__ __forceinline__ float absmax_value(uint32_t q, int fmt) {
  return fmt == kAbsFp8 ? fp8_value(q) : q8_value(q);
}

// Block scale t = RN32(Q[q] * s2) for the second-level format fmt.
__device__ __forceinline__ float block_scale(uint32_t q, float s2, int fmt) { return absmax_value(q, fmt) * s2; }

// ---------------------------------------------------------------------------
// LDS tiles: rows of 64 bf16 (128 B = 8 chunks of 16 B); chunk c of row r is
// stored at chunk position c ^ swz(r), swz(r) = (r ^ r>>3 ^ r>>6) & 7.
// Eight consecutive rows reading one logical chunk (MFMA operand reads) and
// rows 8 or 32 apart writing one column (transposing producers) both land
// on eight different 16-byte bank groups.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lds_swz(int row) { return (row ^ (row >> 3) ^ (row >> 6)) & 7; }
__device__ __forceinline__ int lds_chunk_off(int row, int chunk) {  // in bf16 elements
  return row * 64 + ((chunk ^ lds_swz(row)) << 3);
}

// Scheduling hints: interleave instruction classes inside one basic block.
enum : int { kSchedValu = 0x002, kSchedMfma = 0x008, kSchedDsRead = 0x100, kSchedDsWrite = 0x200 };
#define QLORA_SCHED(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)

__device__ __forceinline__ f32x16_t mfma32x32x16(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

}  // namespace qlora
