// lds.h -- buffer loads, buffer->LDS DMA, LDS accesses and waits shared by
// the GEMM kernels (gfx950).
#pragma once
#include "device.h"

namespace qlora {

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

// Raw buffer resource over `bytes` bytes: loads past the end return zero.
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
// 16 bytes per lane from global memory straight into LDS (lane-linear at `lds`).
__device__ __forceinline__ void dma16(rsrc_t r, char* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ uint4 buf_load16(rsrc_t r, uint32_t voff, uint32_t soff) {
  const u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// s_waitcnt with vmcnt = vm and lgkmcnt = lgkm (expcnt not waited).
constexpr int wait_imm(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8); }
#define QLORA_WAIT(vm, lgkm) __builtin_amdgcn_s_waitcnt(wait_imm((vm), (lgkm)))

// LDS accesses use native vector types: the compiler can then tell them
// apart from the DMA destinations instead of waiting for every DMA in flight.
__device__ __forceinline__ bf16x8_t rd16(const char* p) { return *reinterpret_cast<const bf16x8_t*>(p); }
__device__ __forceinline__ uint4 rdu16(const char* p) {
  const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void wr16(char* p, const uint4& v) {
  const u32x4_t x = {v.x, v.y, v.z, v.w};
  *reinterpret_cast<u32x4_t*>(p) = x;
}
// Transposed LDS read (ds_read_b64_tr_b16).
__device__ __forceinline__ uint2 rd_tr(const char* p) {
  const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p));
  return __builtin_bit_cast(uint2, v);
}

// Transposed-read fragment of a tile whose rows (32 per stage, 2 k16 steps)
// are the contraction and whose columns are an MFMA operand's rows: row
// pitch PB bytes, 32-byte column block b of row n stored at b ^ (n & 3).
// Lane (g = lane >> 4, sl = lane & 15) reads row 8 (g >> 1) + (sl >> 2),
// columns 32 f + 16 (g & 1) + 4 (sl & 3) .. +3; a second read 4 rows down
// completes the lane's 8 contraction elements.
template <int PB>
__device__ __forceinline__ int tr_off(int f) {
  const int lane = threadIdx.x & 63, g = lane >> 4, sl = lane & 15, n0 = 8 * (g >> 1) + (sl >> 2);
  return n0 * PB + 32 * ((2 * f + (g & 1)) ^ (n0 & 3)) + 8 * (sl & 3);
}
template <int PB>
__device__ __forceinline__ bf16x8_t tr_frag(const char* p) {
  const uint2 lo = rd_tr(p), hi = rd_tr(p + 4 * PB);
  return __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
}
// Batched transposed reads.  The compiler cannot tell a ds_read_b64_tr_b16
// builtin apart from the buffer->LDS DMA writes in flight, so before the
// first such read it waits for every DMA: a ring that keeps stages in flight
// would be drained at every stage.  Here the reads of up to three tr_frag
// fragments (fragment i at p_i, second half O_i bytes further) are issued
// from one asm block that also waits for them, so its outputs are complete
// when the block ends; the caller's own vmcnt wait and barrier order the
// reads after the DMA of the stage they read.
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
__device__ __forceinline__ bf16x8_t cat_frag(u32x2_t lo, u32x2_t hi) {
  return __builtin_bit_cast(bf16x8_t, u32x4_t{lo.x, lo.y, hi.x, hi.y});
}
template <int O0>
__device__ __forceinline__ void tr_read1(const char* p0, bf16x8_t& f0) {
  u32x2_t a0, a1;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %2\n\t"
      "ds_read_b64_tr_b16 %1, %2 offset:%3\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a0), "=&v"(a1)
      : "v"(lds_addr(p0)), "i"(O0));
  f0 = cat_frag(a0, a1);
}
template <int O0, int O1>
__device__ __forceinline__ void tr_read2(const char* p0, const char* p1, bf16x8_t& f0, bf16x8_t& f1) {
  u32x2_t a0, a1, b0, b1;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\t"
      "ds_read_b64_tr_b16 %1, %4 offset:%6\n\t"
      "ds_read_b64_tr_b16 %2, %5\n\t"
      "ds_read_b64_tr_b16 %3, %5 offset:%7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a0), "=&v"(a1), "=&v"(b0), "=&v"(b1)
      : "v"(lds_addr(p0)), "v"(lds_addr(p1)), "i"(O0), "i"(O1));
  f0 = cat_frag(a0, a1);
  f1 = cat_frag(b0, b1);
}
template <int O0, int O1, int O2>
__device__ __forceinline__ void tr_read3(const char* p0, const char* p1, const char* p2, bf16x8_t& f0, bf16x8_t& f1,
                                         bf16x8_t& f2) {
  u32x2_t a0, a1, b0, b1, c0, c1;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %6\n\t"
      "ds_read_b64_tr_b16 %1, %6 offset:%9\n\t"
      "ds_read_b64_tr_b16 %2, %7\n\t"
      "ds_read_b64_tr_b16 %3, %7 offset:%10\n\t"
      "ds_read_b64_tr_b16 %4, %8\n\t"
      "ds_read_b64_tr_b16 %5, %8 offset:%11\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a0), "=&v"(a1), "=&v"(b0), "=&v"(b1), "=&v"(c0), "=&v"(c1)
      : "v"(lds_addr(p0)), "v"(lds_addr(p1)), "v"(lds_addr(p2)), "i"(O0), "i"(O1), "i"(O2));
  f0 = cat_frag(a0, a1);
  f1 = cat_frag(b0, b1);
  f2 = cat_frag(c0, c1);
}

// Position of 16-byte chunk c of row r in a 64-byte-row tile.
__device__ __forceinline__ int spos(int r, int c) { return r * 64 + 16 * (c ^ ((r >> 2) & 3)); }

}  // namespace qlora
