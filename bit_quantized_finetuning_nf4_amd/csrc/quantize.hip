// quantize.hip -- blockwise NF4 quantization with double-quantized absmax
// constants, and standalone dequantization to bf16.
//
// Method (glossary "QLoRA", Definition; deepfa.ir blog "1. 4-bit NormalFloat"
// and "2. Double Quantization"): each block of 64 consecutive weights is
// scaled by its absmax and every scaled weight is stored as the index of the
// nearest NF4 level; the block absmaxes are quantized a second time to 8-bit
// codes against one fp32 scale per group of 256 blocks.
#include <mutex>
#include <utility>
#include <vector>

#include "device.h"
#include "kernels.h"

namespace qlora {

// Codes without a division.  The code of w is c = #{k : RN32(w / a) > T_k}
// over the 15 ascending fp32 thresholds T_k of codebook CB (FP4's has one
// twice, which the count handles alike).  With B_k the midpoint of T_k and
// the next fp32 above it, RN32(w / a) > T_k exactly when w / a > B_k: w / a
// is never a rounding boundary itself (w and a are bf16, a boundary has 25
// significant bits, see below), so it rounds above T_k exactly when it lies
// above B_k.  For a > 0 that is w > a B_k, and a B_k (8 by 25 significant
// bits) is exact in fp64.  For any w representable in fp32, w > p holds
// exactly when w > RD32(p), the largest fp32 value not above p.  So the
// block's thresholds c_k = RD32(a B_k) are computed once per block (two per
// lane of the block's eight) and each weight is compared with them as it is.
//
// Why w / a is never a boundary: an fp32 rounding boundary B is an odd
// multiple of a power of two with 25 significant bits, and a B then has at
// least 25 significant bits, while w has at most 8.

// The midpoint of T_k and the next fp32 value above it (toward +inf; no
// threshold is zero), exact in fp64.
template <int CB>
__device__ __forceinline__ double thresh_mid(int k) {
  const uint32_t t = cb_thresh_bits<CB>(k);
  const uint32_t up = (t & 0x80000000u) ? t - 1u : t + 1u;
  return 0.5 * ((double)u2f(t) + (double)u2f(up));
}
// RD32(p): the largest fp32 value not above p.
__device__ __forceinline__ float rd32(double p) {
  const float f = (float)p;
  if (!((double)f > p)) return f;
  const uint32_t u = f2u(f);
  return u2f((u & 0x7FFFFFFFu) == 0u ? 0x80000001u : (f > 0.0f ? u - 1u : u + 1u));
}

// 4-bit codes of eight weights against the block's thresholds c_0 .. c_14 at
// tb (LDS): c = #{k : w > c_k} by binary search, the code's bits found most
// significant first, comparing with c_7, then c_{8c+3}, c_{4c+1}, c_{2c}: 4
// compares instead of 15.  A compare is the sign of c_k - w: the difference
// of two floats is rounded without changing its sign and is +0 when they are
// equal, so its sign bit is [w > c_k] (an infinite c_k gives the right sign
// too).  The funnel shift (c : d) >> 31 appends that bit to c in one
// instruction.  The eight searches advance step by step together, so that
// each step's eight LDS reads are in flight at once.
__device__ __forceinline__ uint32_t gt_bit(float t, float x) { return __builtin_bit_cast(uint32_t, t - x); }
__device__ __forceinline__ uint32_t codes8(const float (&w)[8], const float* tb) {
  uint32_t c[8];
  float t[8];
  const float t7 = tb[7];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = gt_bit(t7, w[i]) >> 31;
#pragma unroll
  for (int i = 0; i < 8; ++i) t[i] = tb[8 * c[i] + 3];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = __builtin_amdgcn_alignbit(c[i], gt_bit(t[i], w[i]), 31);
#pragma unroll
  for (int i = 0; i < 8; ++i) t[i] = tb[4 * c[i] + 1];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = __builtin_amdgcn_alignbit(c[i], gt_bit(t[i], w[i]), 31);
#pragma unroll
  for (int i = 0; i < 8; ++i) t[i] = tb[2 * c[i]];
  uint32_t packed = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) packed |= __builtin_amdgcn_alignbit(c[i], gt_bit(t[i], w[i]), 31) << (4 * i);
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

// Nearest FP8 second-level value to y in [0, 1], ties to the lower index:
// the largest code whose value is <= y (a binary search over the increasing
// 127 values), then the nearer of it and the next one by exact fp64
// distances.
__device__ __forceinline__ uint32_t fp8_code(float y) {
  int lo = 0, hi = 126;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (fp8_value((uint32_t)mid) <= y) lo = mid; else hi = mid - 1;
  }
  if (lo < 126 && (double)fp8_value((uint32_t)lo + 1u) - (double)y < (double)y - (double)fp8_value((uint32_t)lo)) ++lo;
  return (uint32_t)lo;
}

// One workgroup of 256 threads per group of 256 blocks.  Each lane encodes
// 8 consecutive weights per pass; 8 lanes form one block, 32 blocks per
// pass, 8 passes per group.  Block absmaxes go to LDS for the second level.
template <int CB>
__global__ __launch_bounds__(256) void quantize_kernel(const bf16_t* __restrict__ W, int64_t numel,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ absmax_q,
                                                       float* __restrict__ group_scale, int64_t nb,
                                                       int absfmt) {
  __shared__ float amax[kGroupBlocks];
  __shared__ float red[8];
  __shared__ float thr[32 * 16];   // a pass's 32 blocks: thresholds c_0 .. c_14 each
  const int tid = threadIdx.x;
  // this lane computes c_{2j} and c_{2j+1} of its block, j = tid & 7 (c_15
  // does not exist and is never read)
  const int j2 = 2 * (tid & 7);
  const double bm0 = thresh_mid<CB>(j2), bm1 = j2 + 1 < 15 ? thresh_mid<CB>(j2 + 1) : 0.0;
  float* tb = thr + (tid >> 3) * 16;   // only this wave's lanes touch its blocks' rows
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
      const double ad = (double)m;
      tb[j2] = rd32(ad * bm0);
      if (j2 + 1 < 15) tb[j2 + 1] = rd32(ad * bm1);
      // the block's eight lanes are in this wave: its LDS writes above are
      // done before the reads below
      packed = codes8(f, tb);
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
      q = absfmt == kAbsFp8 ? fp8_code(y) : q8_code(y);
    }
    absmax_q[b] = (uint8_t)q;
  }
  if (tid == 0) group_scale[g] = s2;
}

// Four lanes per block of 64 weights: lane p of the four takes weights
// 16 p .. 16 p + 15 (8 code bytes -> 32 bytes of bf16), so a wave reads 512
// contiguous code bytes and writes 2 KiB of contiguous bf16.  Each lane builds
// its block's table (the block scale and the 16 products with the levels).
// Grid y selects one of the launch's weights (all of one shape): weight i
// goes to out + i out_gs.
template <int CB>
__global__ __launch_bounds__(256) void dequant_kernel(DeqSrcs src, int64_t numel, int64_t nb, int absfmt,
                                                      bf16_t* __restrict__ out, int64_t out_gs, int rev) {
  const int wi = rev ? (int)gridDim.y - 1 - (int)blockIdx.y : (int)blockIdx.y;
  const uint8_t* __restrict__ codes = src.codes[wi];
  const uint8_t* __restrict__ absmax_q = src.absmax_q[wi];
  const float* __restrict__ group_scale = src.group_scale[wi];
  out += wi * out_gs;
  const int64_t bx = rev ? (int64_t)gridDim.x - 1 - blockIdx.x : (int64_t)blockIdx.x;
  const int64_t g = bx * blockDim.x + threadIdx.x;
  const int64_t b = g >> 2;
  if (b >= nb) return;
  const float t = block_scale(absmax_q[b], group_scale[b / kGroupBlocks], absfmt);
  const Nf4Table T = make_table<CB>(t);
  const int64_t e0 = (g << 4);   // first of the lane's 16 weights
  if (e0 + 16 <= numel) {
    const uint2 c = *reinterpret_cast<const uint2*>(codes + (e0 >> 1));
    uint32_t o[8];
    dequant8(c.x, T, o);
    dequant8(c.y, T, o + 4);
    uint4* dst = reinterpret_cast<uint4*>(out + e0);
    dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
    dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
  } else if (e0 < numel) {
    // ragged end of the last block
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

// Transposed dequantization, WdT [K x N] = deq(W)^T for W [N x K] with
// K % 64 == 0 (the dense backward multiplies by it).  A workgroup takes 64
// rows x 256 columns of W, so each row's codes are one whole 128-byte line:
// thread t decodes rows 2 (t & 31) and 2 (t & 31) + 1, columns 32 (t >> 5)
// .. +31 (half a block of each row), packs each column's two rows into one
// dword and stores it to LDS at [column][row pair] (rows of 33 dwords: the
// 32 row pairs of a wave's half fall in 32 consecutive banks, the other half
// 32 banks on); then the waves write WdT rows k0 .. k0 + 255, 128 bytes (64
// rows of W) each, eight whole rows per store instruction.  Rows past N
// decode as zero and are not written; columns past K are neither read nor
// written.  Grid z selects one of the launch's weights (all of one shape):
// weight i goes to the columns from i out_gs on.
constexpr int kTrStride = 33;
template <int CB>
__global__ __launch_bounds__(256) void dequant_t_kernel(DeqSrcs src, int64_t N, int64_t K, int absfmt,
                                                        bf16_t* __restrict__ out, int64_t ldo, int64_t out_gs,
                                                        int rev) {
  const int wi = rev ? (int)gridDim.z - 1 - (int)blockIdx.z : (int)blockIdx.z;
  const uint8_t* __restrict__ codes = src.codes[wi];
  const uint8_t* __restrict__ absmax_q = src.absmax_q[wi];
  const float* __restrict__ group_scale = src.group_scale[wi];
  out += wi * out_gs;
  __shared__ uint32_t tile[256 * kTrStride];
  const int t = threadIdx.x, rp = t & 31, cg = t >> 5;
  const int64_t by = rev ? (int64_t)gridDim.y - 1 - blockIdx.y : (int64_t)blockIdx.y;
  const int64_t n0 = by * 64, k0 = (int64_t)blockIdx.x * 256;
  const int64_t kc = k0 + 32 * cg;
  if (kc < K) {
    uint4 c[2];
    Nf4Table T[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t row = n0 + 2 * rp + i;
      if (row < N) {
        const int64_t b = (row * K + kc) >> 6;
        T[i] = make_table<CB>(block_scale(absmax_q[b], group_scale[b / kGroupBlocks], absfmt));
        c[i] = *reinterpret_cast<const uint4*>(codes + ((row * K + kc) >> 1));
      } else {
        T[i] = make_table<CB>(0.0f);
        c[i] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
    const uint32_t w0[4] = {c[0].x, c[0].y, c[0].z, c[0].w}, w1[4] = {c[1].x, c[1].y, c[1].z, c[1].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t o[8];
      dequant8x2_pairs(w0[j], w1[j], T[0], T[1], o);
#pragma unroll
      for (int k = 0; k < 8; ++k) tile[(32 * cg + 8 * j + k) * kTrStride + rp] = o[k];
    }
  }
  __syncthreads();
  // write-out: each store instruction of a wave covers 8 whole 128-byte rows
  // of WdT (lane l: row 8 q + (l >> 3) of the wave's 64, 16-byte chunk l & 7)
  const int lane = t & 63, w = t >> 6, c = lane & 7;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int kk = 64 * w + 8 * q + (lane >> 3);
    if (k0 + kk >= K) continue;
    const uint32_t* src = tile + kk * kTrStride + 4 * c;
    const uint4 v = make_uint4(src[0], src[1], src[2], src[3]);
    bf16_t* dst = out + (k0 + kk) * ldo + n0 + 8 * c;
    if (n0 + 8 * c + 8 <= N) {
      *reinterpret_cast<uint4*>(dst) = v;
    } else {
      const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
      for (int e = 0; e < 8 && n0 + 8 * c + e < N; ++e) dst[e] = (bf16_t)(vw[e >> 1] >> (16 * (e & 1)));
    }
  }
}

// Kernels whose dynamic-LDS limit has been raised, per device: the
// attribute call costs a few microseconds of host time, which per-token
// decode loops and small products would pay on every launch.
hipError_t allow_lds(const void* fn, int bytes) {
  static std::mutex mu;
  static std::vector<std::pair<const void*, int>> done;   // (kernel, device)
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  for (const auto& d : done)
    if (d.first == fn && d.second == dev) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.emplace_back(fn, dev);
  return e;
}

int device_cu_count() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 256;
  return cus > 0 ? cus : 256;
}

hipError_t launch_quantize(const bf16_t* W, int64_t numel, uint8_t* codes, uint8_t* absmax_q,
                           float* group_scale, int codebook, int absfmt, hipStream_t s) {
  const int64_t nb = (numel + kBlock - 1) / kBlock;
  const int64_t ng = (nb + kGroupBlocks - 1) / kGroupBlocks;
  auto* fn = codebook == kCbFp4 ? &quantize_kernel<kCbFp4> : codebook == kCbInt4 ? &quantize_kernel<kCbInt4>
                                                                                  : &quantize_kernel<kCbNf4>;
  hipLaunchKernelGGL(fn, dim3((unsigned)ng), dim3(256), 0, s, W, numel, codes, absmax_q, group_scale, nb, absfmt);
  return hipGetLastError();
}

// Write order of a dequantization.  The dense GEMM that follows starts on the
// first weight rows (forward) or the first contraction columns (dX), so when
// the bf16 output is larger than the 256 MB last-level cache the workgroups
// run in reverse: the part written last, which the cache still holds, is the
// part read first.  Each workgroup computes the same values in either order.
constexpr int64_t kLlcBytes = (int64_t)256 << 20;

hipError_t launch_dequant_group(const DeqSrcs& src, int n, int64_t N, int64_t K, int codebook, int absfmt,
                                bool transposed, bf16_t* out, int64_t ldo, int64_t out_gs, hipStream_t s) {
  if (n < 1 || n > kDeqMax) return hipErrorInvalidValue;
  const int rev = (int64_t)n * N * K * 2 > kLlcBytes ? 1 : 0;
  if (!transposed) {
    const int64_t numel = N * K, nb = (numel + kBlock - 1) / kBlock;
    auto* fn = codebook == kCbFp4 ? &dequant_kernel<kCbFp4> : codebook == kCbInt4 ? &dequant_kernel<kCbInt4>
                                                                                  : &dequant_kernel<kCbNf4>;
    hipLaunchKernelGGL(fn, dim3((unsigned)((4 * nb + 255) / 256), (unsigned)n), dim3(256), 0, s, src, numel, nb,
                       absfmt, out, out_gs, rev);
  } else {
    auto* fn = codebook == kCbFp4 ? &dequant_t_kernel<kCbFp4> : codebook == kCbInt4 ? &dequant_t_kernel<kCbInt4>
                                                                                    : &dequant_t_kernel<kCbNf4>;
    hipLaunchKernelGGL(fn, dim3((unsigned)((K + 255) / 256), (unsigned)((N + 63) / 64), (unsigned)n), dim3(256), 0,
                       s, src, N, K, absfmt, out, ldo, out_gs, rev);
  }
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* codes, const uint8_t* absmax_q, const float* group_scale,
                          int64_t numel, int codebook, int absfmt, bf16_t* out, hipStream_t s) {
  DeqSrcs src{};
  src.codes[0] = codes;
  src.absmax_q[0] = absmax_q;
  src.group_scale[0] = group_scale;
  return launch_dequant_group(src, 1, 1, numel, codebook, absfmt, false, out, 0, 0, s);
}

hipError_t launch_dequant_t(const uint8_t* codes, const uint8_t* absmax_q, const float* group_scale, int64_t N,
                            int64_t K, int codebook, int absfmt, bf16_t* out, int64_t ldo, hipStream_t s) {
  DeqSrcs src{};
  src.codes[0] = codes;
  src.absmax_q[0] = absmax_q;
  src.group_scale[0] = group_scale;
  return launch_dequant_group(src, 1, N, K, codebook, absfmt, true, out, ldo, 0, s);
}

}  // namespace qlora
