// gemv.hip -- batch-1 decode y = deq(W) x + s B (A x) over many linears.
//
// whatthefuture.ai article, closing paragraphs: 4-bit inference is slow and
// an 8-16x speed-up is expected; glossary "QLoRA", Definition: the frozen
// weights are 4-bit NF4 with double-quantized constants.
//
// The product streams 0.516 bytes per weight from HBM, so the kernel is
// built around the per-weight ALU cost of decoding:
//   * codes are decoded by byte permutes against the constant table of the
//     16 unscaled levels in bf16; the block scale t = Q8[q] s2 multiplies
//     the block's fp32 partial dot product afterwards;
//   * the multiply-adds run on the matrix cores: v_mfma_f32_32x32x16_bf16
//     with the decoded weights as the B operand (lane j <-> weight row j)
//     and x broadcast to every row of the A operand, a fresh accumulator per
//     block;
//   * a workgroup of 4 waves owns 128 weight rows; each lane pair (j, j+32)
//     streams the two 16-byte halves of each block of row j, so a wave reads
//     whole 128-byte lines over four blocks.
// x is staged once per workgroup in LDS, with each group of 8 elements in
// the order (0,2,4,6,1,3,5,7) that the decoder produces.
#include "device.h"
#include "kernels.h"

namespace qlora {

constexpr int kGemvThreads = 256;
constexpr int kGemvRows = 128;       // weight rows per workgroup
constexpr int kDownRows = 4;         // LoRA-A rows per workgroup in phase 1 (one per wave)
constexpr int kMaxBatch = 24;        // jobs per launch (kernel-argument batch)

struct GemvBatch {
  GemvJob jobs[kMaxBatch];
  int wg_begin[kMaxBatch + 1];
  int njobs;
};

namespace {

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer resource over `bytes` bytes: loads past the end return zero.
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(rsrc_t r, uint32_t voff) {
  const u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ int find_job(const GemvBatch& b) {
  int j = 0;
  while (j + 1 < b.njobs && (int)blockIdx.x >= b.wg_begin[j + 1]) ++j;
  return j;
}

__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float dot8(uint4 a, uint4 x) {
  const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, xw[4] = {x.x, x.y, x.z, x.w};
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    s += bf2f(aw[e] & 0xFFFFu) * bf2f(xw[e] & 0xFFFFu);
    s += bf2f(aw[e] >> 16) * bf2f(xw[e] >> 16);
  }
  return s;
}

// Decode 8 codes into bf16 pairs in the order {0,2},{4,6},{1,3},{5,7}.
__device__ __forceinline__ bf16x8_t dequant8_eo(uint32_t c, const Nf4Table& T) {
  uint32_t le, he, lo, ho;
  lookup4(c & 0x0F0F0F0Fu, T, le, he);
  lookup4((c >> 4) & 0x0F0F0F0Fu, T, lo, ho);
  return __builtin_bit_cast(bf16x8_t, make_uint4(perm(he, le, 0x05010400u), perm(he, le, 0x07030602u),
                                                 perm(ho, lo, 0x05010400u), perm(ho, lo, 0x07030602u)));
}

}  // namespace

// Phase 1: u = A x for every job with r > 0 (fp32, into the job's scratch);
// one wave per adapter row, four 16-byte loads of A and x in flight per lane.
__global__ __launch_bounds__(kGemvThreads) void lora_down_kernel(GemvBatch b) {
  const int j = find_job(b);
  const GemvJob& J = b.jobs[j];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int row = (blockIdx.x - b.wg_begin[j]) * kDownRows + w;
  if (row >= J.r) return;   // uniform per wave; the kernel has no barrier
  const bf16_t* a = J.A + (int64_t)row * J.K;
  float acc = 0.0f;
  for (int k0 = lane * 8; k0 < J.K; k0 += 4 * 512) {
    uint4 av[4], xv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = k0 + 512 * u;
      av[u] = xv[u] = make_uint4(0u, 0u, 0u, 0u);
      if (k < J.K) {
        av[u] = *reinterpret_cast<const uint4*>(a + k);
        xv[u] = *reinterpret_cast<const uint4*>(J.x + k);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc += dot8(av[u], xv[u]);
  }
  acc = wave_sum(acc);
  if (lane == 0) J.u[row] = acc;
}

// Phase 2: the NF4 GEMV with the LoRA up-projection in the epilogue.
//
// Wave w of a workgroup owns weight rows 32 w .. 32 w + 31 of the group's
// 128; lanes j and j + 32 stream the two 16-byte halves of each block of row
// j.  Per block, four MFMAs take x (broadcast to every row of the A operand)
// against the decoded unscaled levels of the 32 rows (B operand), starting
// from a zero accumulator, so every row of the result holds the 32 rows'
// partial dot products for the block; the block scale multiplies them in
// fp32.  The codes of the next four blocks are in flight while the current
// four are decoded.
__global__ __launch_bounds__(kGemvThreads) void nf4_gemv_kernel(GemvBatch b) {
  extern __shared__ __align__(16) uint32_t xs[];  // K/2 dwords
  const int j = find_job(b);
  const GemvJob& J = b.jobs[j];
  const int K = J.K, N = J.N, nblk = K >> 6;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int jr = lane & 31, h = lane >> 5;

  // stage x, each group of 8 reordered to (0,2,4,6,1,3,5,7)
  for (int i = threadIdx.x; i < K / 8; i += kGemvThreads) {
    const uint4 v = *reinterpret_cast<const uint4*>(J.x + 8 * i);
    *reinterpret_cast<uint4*>(xs + 4 * i) =
        make_uint4(perm(v.y, v.x, 0x05040100u), perm(v.w, v.z, 0x05040100u), perm(v.y, v.x, 0x07060302u),
                   perm(v.w, v.z, 0x07060302u));
  }
  __syncthreads();

  const Nf4Table T = make_table(1.0f);  // bf16 of the unscaled levels
  const int64_t n = (int64_t)(blockIdx.x - b.wg_begin[j]) * kGemvRows + 32 * w + jr;
  // Rows past N address the first byte past the arrays: the range check
  // returns zero codes and absmax code 0, i.e. block scale 0.
  const int64_t nc = n < N ? n : N;
  const int64_t nb = (int64_t)N * nblk;
  const rsrc_t cr = make_rsrc(J.codes, (uint32_t)(nb * 32));
  const rsrc_t ar = make_rsrc(J.absmax_q, (uint32_t)nb);
  const uint32_t crow = (uint32_t)(nc * nblk * 32) + 16u * h;
  const uint32_t brow = (uint32_t)(nc * nblk);
  const bool quad = (nblk & 3) == 0;
  float acc = 0.0f;

  uint4 cw[4];
#pragma unroll
  for (int bi = 0; bi < 4; ++bi) cw[bi] = buf_load16(cr, crow + 32u * bi);
  for (int b0 = 0; b0 < nblk; b0 += 4) {
    // scales of blocks b0 .. b0+3 (zero past the last block)
    float t[4];
    if (quad) {
      const uint32_t q4 = __builtin_amdgcn_raw_buffer_load_b32(ar, brow + b0, 0, 0);
      const float s2 = J.group_scale[(brow + b0 < nb ? brow + b0 : nb - 1) >> 8];
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) t[bi] = block_scale((q4 >> (8 * bi)) & 0xFFu, s2);
    } else {
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        const uint32_t blk = brow + b0 + bi;
        const uint32_t q = __builtin_amdgcn_raw_buffer_load_b8(ar, blk, 0, 0);
        const float s2 = J.group_scale[(blk < nb ? blk : nb - 1) >> 8];
        t[bi] = b0 + bi < nblk ? block_scale(q, s2) : 0.0f;
      }
    }
    // codes of the next four blocks (past the row end they are never used)
    uint4 cn[4];
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) cn[bi] = buf_load16(cr, crow + 32u * (b0 + 4 + bi));
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) {
      if (b0 + bi >= nblk) break;   // uniform: a ragged last quad of blocks
      const uint32_t* xb = xs + 32 * (b0 + bi) + 16 * h;
      const uint32_t words[4] = {cw[bi].x, cw[bi].y, cw[bi].z, cw[bi].w};
      f32x16_t D = {};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8_t xa = *reinterpret_cast<const bf16x8_t*>(xb + 4 * kk);
        D = mfma32x32x16(xa, dequant8_eo(words[kk], T), D);
      }
      acc += t[bi] * D[0];
    }
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) cw[bi] = cn[bi];
  }

  // LoRA up-projection: lanes j and j+32 take alternate groups of 8 ranks
  const bool valid = n < N;
  float lora = 0.0f;
  if (J.r > 0 && valid) {
    const bf16_t* brp = J.B + n * J.r;
    for (int i = 8 * h; i < J.r; i += 16) {
      const uint4 v = *reinterpret_cast<const uint4*>(brp + i);
      const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lora += bf2f(vw[e] & 0xFFFFu) * J.u[i + 2 * e];
        lora += bf2f(vw[e] >> 16) * J.u[i + 2 * e + 1];
      }
    }
  }
  lora += __shfl_xor(lora, 32);
  if (h == 0 && valid) {
    const float y = acc + J.s * lora;
    J.y[n] = (bf16_t)(pack_bf16x2(y, 0.0f) & 0xFFFFu);
  }
}

hipError_t launch_gemv(const GemvJob* jobs, int njobs, hipStream_t st) {
  for (int base = 0; base < njobs; base += kMaxBatch) {
    const int cnt = njobs - base < kMaxBatch ? njobs - base : kMaxBatch;
    GemvBatch down{}, main{};
    int wd = 0, wm = 0, maxK = 0, nd = 0;
    for (int i = 0; i < cnt; ++i) {
      const GemvJob& J = jobs[base + i];
      main.jobs[i] = J;
      main.wg_begin[i] = wm;
      wm += (J.N + kGemvRows - 1) / kGemvRows;
      if (J.K > maxK) maxK = J.K;
      if (J.r > 0) {
        down.jobs[nd] = J;
        down.wg_begin[nd] = wd;
        wd += (J.r + kDownRows - 1) / kDownRows;
        ++nd;
      }
    }
    main.wg_begin[cnt] = wm;
    main.njobs = cnt;
    down.wg_begin[nd] = wd;
    down.njobs = nd;
    if (nd > 0) {
      hipLaunchKernelGGL(lora_down_kernel, dim3(wd), dim3(kGemvThreads), 0, st, down);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    const size_t lds = (size_t)maxK * sizeof(bf16_t);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&nf4_gemv_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(nf4_gemv_kernel, dim3(wm), dim3(kGemvThreads), lds, st, main);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace qlora
