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

// Position of 16-byte chunk c of row r in a 64-byte-row tile.
__device__ __forceinline__ int spos(int r, int c) { return r * 64 + 16 * (c ^ ((r >> 2) & 3)); }

}  // namespace qlora
