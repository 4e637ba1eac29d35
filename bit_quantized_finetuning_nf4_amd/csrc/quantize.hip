// quantize.hip -- blockwise NF4 quantization with double-quantized absmax
// constants, and standalone dequantization to bf16.
//
// Method (glossary "QLoRA", Definition; deepfa.ir blog "1. 4-bit NormalFloat"
// and "2. Double Quantization"): each block of 64 consecutive weights is
// scaled by its absmax and every scaled weight is stored as the index of the
// nearest NF4 level; the block absmaxes are quantized a second time to 8-bit
// codes against one fp32 scale per group of 256 blocks.
#include "device.h"
#include "kernels.h"

namespace qlora {

// 4-bit codes of eight fp32 values x = RN32(w / a): c = #{k : x > T_k} over
// the 15 ascending thresholds of codebook CB (FP4's has one threshold twice,
// which the count handles alike), by binary search with the code's bits found
// most significant first.  The first step compares with T_7 (a constant),
// the others with T_{8c+3}, T_{4c+1}, T_{2c} from an LDS copy of the table:
// 4 compares instead of 15.  A compare is the sign of T - x: the difference
// of two finite floats is rounded without changing its sign and is +0 when
// they are equal, so its sign bit is [x > T] (no threshold is zero).  The
// funnel shift (c : d) >> 31 appends that bit to c in one instruction.  The
// eight searches advance step by step together, so that each step's eight
// LDS reads are in flight at once.
__device__ __forceinline__ uint32_t gt_bit(float t, float x) { return __builtin_bit_cast(uint32_t, t - x); }
template <int CB>
__device__ __forceinline__ uint32_t nf4_codes8(const float (&x)[8], const float* thr) {
  uint32_t c[8];
  float t[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = gt_bit(u2f(cb_thresh_bits<CB>(7)), x[i]) >> 31;
#pragma unroll
  for (int i = 0; i < 8; ++i) t[i] = thr[8 * c[i] + 3];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = __builtin_amdgcn_alignbit(c[i], gt_bit(t[i], x[i]), 31);
#pragma unroll
  for (int i = 0; i < 8; ++i) t[i] = thr[4 * c[i] + 1];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = __builtin_amdgcn_alignbit(c[i], gt_bit(t[i], x[i]), 31);
#pragma unroll
  for (int i = 0; i < 8; ++i) t[i] = thr[2 * c[i]];
  uint32_t packed = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) packed |= __builtin_amdgcn_alignbit(c[i], gt_bit(t[i], x[i]), 31) << (4 * i);
  return packed;
}

// max over the eight lanes 8j .. 8j+7 of a non-negative float, on its bits
// (ordered as the values): swap neighbours, swap pairs, then mirror the two
// quads (DPP)
__device__ __forceinline__ float max8_lanes(float m) {
  uint32_t u = __builtin_bit_cast(uint32_t, m);
  u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0xB1, 0xF, 0xF, true));
  u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x4E, 0xF, 0xF, true));
  u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x141, 0xF, 0xF, true));
  return u2f(u);
}

// Nearest Q8 level to y in [0, 1], ties to the lower index.  The nearest
// level is within one step of rint(255 y); distances of two fp32 values are
// exact in fp64.
__device__ __forceinline__ uint32_t q8_code(float y) {
  int c = (int)rintf(y * 255.0f);
  c = c < 0 ? 0 : (c > 255 ? 255 : c);
  int best = c > 0 ? c - 1 : 0;
  double bd = fabs((double)y - (double)q8_value(best));
  const int hi = c < 255 ? c + 1 : 255;
  for (int k = best + 1; k <= hi; ++k) {
    const double d = fabs((double)y - (double)q8_value(k));
    if (d < bd) { bd = d; best = k; }
  }
  return (uint32_t)best;
}

// One workgroup of 256 threads per group of 256 blocks.  Each lane encodes
// 8 consecutive weights per pass; 8 lanes form one block, 32 blocks per
// pass, 8 passes per group.  Block absmaxes go to LDS for the second level.
template <int CB>
__global__ __launch_bounds__(256) void quantize_kernel(const bf16_t* __restrict__ W, int64_t numel,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ absmax_q,
                                                       float* __restrict__ group_scale, int64_t nb) {
  __shared__ float amax[kGroupBlocks];
  __shared__ float red[8];
  __shared__ float thr[16];
  const int tid = threadIdx.x;
  if (tid < 15) thr[tid] = u2f(cb_thresh_bits<CB>(tid));
  __syncthreads();
  const int64_t g = blockIdx.x;
  const int64_t gbase = g * (int64_t)kGroupBlocks * kBlock;
  const int64_t code_bytes = (numel + 1) >> 1;

  // all eight passes' loads first: 128 bytes per lane in flight
  uint4 wv[8];
  if (gbase + (int64_t)kGroupBlocks * kBlock <= numel) {   // a whole group (uniform branch)
#pragma unroll
    for (int pass = 0; pass < 8; ++pass)
      wv[pass] = *reinterpret_cast<const uint4*>(W + gbase + (int64_t)pass * 2048 + tid * 8);
  } else {
#pragma unroll
    for (int pass = 0; pass < 8; ++pass) {
      const int64_t e0 = gbase + (int64_t)pass * 2048 + tid * 8;
      uint32_t w[4] = {0u, 0u, 0u, 0u};
      if (e0 + 8 <= numel) {
        const uint4 v = *reinterpret_cast<const uint4*>(W + e0);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
      } else if (e0 < numel) {
        for (int i = 0; i < 8; ++i)
          if (e0 + i < numel) w[i >> 1] |= (uint32_t)W[e0 + i] << (16 * (i & 1));
      }
      wv[pass] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
#pragma unroll
  for (int pass = 0; pass < 8; ++pass) {
    const int64_t e0 = gbase + (int64_t)pass * 2048 + tid * 8;
    const uint32_t w[4] = {wv[pass].x, wv[pass].y, wv[pass].z, wv[pass].w};
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = u2f(w[i] << 16);
      f[2 * i + 1] = u2f(w[i] & 0xFFFF0000u);
    }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
    // absmax of the 64-element block held by 8 consecutive lanes
    m = max8_lanes(m);
    const int blk = pass * 32 + (tid >> 3);
    if ((tid & 7) == 0) amax[blk] = m;

    uint32_t packed = cb_zero_code<CB>() * 0x11111111u;   // all-zero block: the code of the level 0
    if (m > 0.0f) {
      // x = RN32(w / a) from the fp64 product w * r, r ~ 1/a.  w and a are
      // bf16 (at most 8 significant bits) and an fp32 rounding boundary B is
      // an odd multiple of a power of two with 25 significant bits, so
      // w - aB is a nonzero multiple of a power of two that is at least
      // about 2^-33 |w|: w / a is at least that far, relatively, from every
      // boundary.  r from the hardware reciprocal and two Newton steps is
      // within 2^-50 relative of 1/a, the product adds 2^-53, so the product
      // lies on the same side of every boundary as w / a and rounding it to
      // fp32 gives RN32(w / a).
      const double ad = (double)m;
      double r = __builtin_amdgcn_rcp(ad);
      r = fma(r, fma(-ad, r, 1.0), r);
      r = fma(r, fma(-ad, r, 1.0), r);
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = (float)((double)f[i] * r);
      packed = nf4_codes8<CB>(x, thr);
    }
    if (e0 + 8 <= numel) {
      *reinterpret_cast<uint32_t*>(codes + (e0 >> 1)) = packed;
    } else if (e0 < numel) {
      // ragged tail: codes of absent elements are 0, bytes past the end are
      // not written
      for (int i = 0; i < 8; i += 2) {
        const int64_t e = e0 + i;
        if (e >= numel) break;
        uint32_t b = (packed >> (4 * i)) & 0xFu;
        if (e + 1 < numel) b |= ((packed >> (4 * (i + 1))) & 0xFu) << 4;
        if ((e >> 1) < code_bytes) codes[e >> 1] = (uint8_t)b;
      }
    }
  }
  __syncthreads();

  // second level: s2 = max block absmax of the group
  float m = amax[tid];
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  const float s2 = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int64_t b = g * kGroupBlocks + tid;
  if (b < nb) {
    uint32_t q = 0;
    if (s2 > 0.0f) {
      const float y = (float)((double)amax[tid] / (double)s2);  // RN32(a / s2)
      q = q8_code(y);
    }
    absmax_q[b] = (uint8_t)q;
  }
  if (tid == 0) group_scale[g] = s2;
}

// One lane per block of 64 weights: 32 bytes of codes -> 128 bytes of bf16.
template <int CB>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ absmax_q,
                                                      const float* __restrict__ group_scale,
                                                      int64_t numel, int64_t nb,
                                                      bf16_t* __restrict__ out) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nb) return;
  const float t = block_scale(absmax_q[b], group_scale[b / kGroupBlocks]);
  const Nf4Table T = make_table<CB>(t);
  const int64_t e0 = b * kBlock;
  if (e0 + kBlock <= numel) {
    const uint4* src = reinterpret_cast<const uint4*>(codes + (e0 >> 1));
    const uint4 c0 = src[0], c1 = src[1];
    const uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    uint4* dst = reinterpret_cast<uint4*>(out + e0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t o[4];
      dequant8(cw[i], T, o);
      dst[i] = make_uint4(o[0], o[1], o[2], o[3]);
    }
  } else {
    // ragged last block
    const int64_t n = numel - e0;
    for (int64_t i = 0; i < n; i += 8) {
      uint32_t cw = 0;
      for (int j = 0; j < 8 && i + j < n; j += 2)
        cw |= (uint32_t)codes[(e0 + i + j) >> 1] << (4 * j);
      uint32_t o[4];
      dequant8(cw, T, o);
      for (int j = 0; j < 8 && i + j < n; ++j)
        out[e0 + i + j] = (bf16_t)(o[j >> 1] >> (16 * (j & 1)));
    }
  }
}

int device_cu_count() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 256;
  return cus > 0 ? cus : 256;
}

hipError_t launch_quantize(const bf16_t* W, int64_t numel, uint8_t* codes, uint8_t* absmax_q,
                           float* group_scale, int codebook, hipStream_t s) {
  const int64_t nb = (numel + kBlock - 1) / kBlock;
  const int64_t ng = (nb + kGroupBlocks - 1) / kGroupBlocks;
  auto* fn = codebook == kCbFp4 ? &quantize_kernel<kCbFp4> : codebook == kCbInt4 ? &quantize_kernel<kCbInt4>
                                                                                  : &quantize_kernel<kCbNf4>;
  hipLaunchKernelGGL(fn, dim3((unsigned)ng), dim3(256), 0, s, W, numel, codes, absmax_q, group_scale, nb);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* codes, const uint8_t* absmax_q, const float* group_scale,
                          int64_t numel, int codebook, bf16_t* out, hipStream_t s) {
  const int64_t nb = (numel + kBlock - 1) / kBlock;
  auto* fn = codebook == kCbFp4 ? &dequant_kernel<kCbFp4> : codebook == kCbInt4 ? &dequant_kernel<kCbInt4>
                                                                                : &dequant_kernel<kCbNf4>;
  hipLaunchKernelGGL(fn, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, s, codes, absmax_q, group_scale, numel,
                     nb, out);
  return hipGetLastError();
}

}  // namespace qlora
