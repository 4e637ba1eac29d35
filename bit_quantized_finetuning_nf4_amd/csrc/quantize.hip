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

// NF4 code of an fp32 value x = RN32(w / a).
// #{k : x > T_k} for the 15 ascending thresholds, by binary search: the
// first step against T_7 (a constant), then three steps against thresholds
// picked from an LDS copy of the table (T_{c+3}, T_{c+1}, T_c for the count
// c found so far).  4 compares instead of 15.
__device__ __forceinline__ uint32_t nf4_code(float x, const float* thr) {
  uint32_t c = x > u2f(kNf4ThreshBits[7]) ? 8u : 0u;
  c += x > thr[c + 3] ? 4u : 0u;
  c += x > thr[c + 1] ? 2u : 0u;
  c += x > thr[c] ? 1u : 0u;
  return c;
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
__global__ __launch_bounds__(256) void quantize_kernel(const bf16_t* __restrict__ W, int64_t numel,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ absmax_q,
                                                       float* __restrict__ group_scale, int64_t nb) {
  __shared__ float amax[kGroupBlocks];
  __shared__ float red[8];
  __shared__ float thr[16];
  const int tid = threadIdx.x;
  if (tid < 15) thr[tid] = u2f(kNf4ThreshBits[tid]);
  __syncthreads();
  const int64_t g = blockIdx.x;
  const int64_t gbase = g * (int64_t)kGroupBlocks * kBlock;
  const int64_t code_bytes = (numel + 1) >> 1;

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
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    m = fmaxf(m, __shfl_xor(m, 4));
    const int blk = pass * 32 + (tid >> 3);
    if ((tid & 7) == 0) amax[blk] = m;

    uint32_t packed = 0x77777777u;
    if (m > 0.0f) {
      // x = RN32(w / a): the fp64 product w * RN64(1/a) is within 2^-52
      // relative of w / a, and an fp32 rounding boundary is never closer
      // than 2^-49 relative to such a quotient in the range where the code
      // depends on it, so rounding the product to fp32 gives RN32(w / a).
      const double rinv = 1.0 / (double)m;
      packed = 0u;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = (float)((double)f[i] * rinv);
        packed |= nf4_code(x, thr) << (4 * i);
      }
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
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ absmax_q,
                                                      const float* __restrict__ group_scale,
                                                      int64_t numel, int64_t nb,
                                                      bf16_t* __restrict__ out) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nb) return;
  const float t = block_scale(absmax_q[b], group_scale[b / kGroupBlocks]);
  const Nf4Table T = make_table(t);
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

hipError_t launch_quantize(const bf16_t* W, int64_t numel, uint8_t* codes, uint8_t* absmax_q,
                           float* group_scale, hipStream_t s) {
  const int64_t nb = (numel + kBlock - 1) / kBlock;
  const int64_t ng = (nb + kGroupBlocks - 1) / kGroupBlocks;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)ng), dim3(256), 0, s, W, numel, codes, absmax_q,
                     group_scale, nb);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* codes, const uint8_t* absmax_q, const float* group_scale,
                          int64_t numel, bf16_t* out, hipStream_t s) {
  const int64_t nb = (numel + kBlock - 1) / kBlock;
  hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, s, codes, absmax_q,
                     group_scale, numel, nb, out);
  return hipGetLastError();
}

}  // namespace qlora
