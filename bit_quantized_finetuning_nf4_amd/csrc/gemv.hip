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
//     and x as A-operand row bi for block bi of the iteration, so one
//     accumulator tile collects four blocks' partial dots in rows 0..3;
//   * a workgroup of 4 waves owns 128 weight rows; each lane pair (j, j+32)
//     streams the two 16-byte halves of each block of row j, so a wave reads
//     whole 128-byte lines.
// x is staged once per workgroup in LDS, with each group of 8 elements in
// the order (0,2,4,6,1,3,5,7) that the decoder produces.
#include "device.h"
#include "kernels.h"

namespace qlora {

constexpr int kGemvThreads = 256;
constexpr int kGemvRows = 128;       // weight rows per workgroup
constexpr int kDownRows = 16;        // LoRA-A rows per workgroup in phase 1
constexpr int kMaxBatch = 24;        // jobs per launch (kernel-argument batch)

struct GemvBatch {
  GemvJob jobs[kMaxBatch];
  int wg_begin[kMaxBatch + 1];
  int njobs;
};

__device__ __forceinline__ int find_job(const GemvBatch& b) {
  int j = 0;
  while (j + 1 < b.njobs && (int)blockIdx.x >= b.wg_begin[j + 1]) ++j;
  return j;
}

__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Phase 1: u = A x for every job with r > 0 (fp32, into the job's scratch).
__global__ __launch_bounds__(kGemvThreads) void lora_down_kernel(GemvBatch b) {
  const int j = find_job(b);
  const GemvJob& J = b.jobs[j];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int row0 = (blockIdx.x - b.wg_begin[j]) * kDownRows + 4 * w;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int k = lane * 8; k < J.K; k += 512) {
    const uint4 xv = *reinterpret_cast<const uint4*>(J.x + k);
    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int row = row0 + rr;
      if (row < J.r) {
        const uint4 av = *reinterpret_cast<const uint4*>(J.A + (int64_t)row * J.K + k);
        const uint32_t aw[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[rr] += bf2f(aw[e] & 0xFFFFu) * bf2f(xw[e] & 0xFFFFu);
          acc[rr] += bf2f(aw[e] >> 16) * bf2f(xw[e] >> 16);
        }
      }
    }
  }
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const float v = wave_sum(acc[rr]);
    if (lane == 0 && row0 + rr < J.r) J.u[row0 + rr] = v;
  }
}

// Decode 8 codes into bf16 pairs in the order {0,2},{4,6},{1,3},{5,7}.
__device__ __forceinline__ void dequant8_eo(uint32_t c, const Nf4Table& T, uint32_t out[4]) {
  uint32_t le, he, lo, ho;
  lookup4(c & 0x0F0F0F0Fu, T, le, he);
  lookup4((c >> 4) & 0x0F0F0F0Fu, T, lo, ho);
  out[0] = perm(he, le, 0x05010400u);
  out[1] = perm(he, le, 0x07030602u);
  out[2] = perm(ho, lo, 0x05010400u);
  out[3] = perm(ho, lo, 0x07030602u);
}

// Phase 2: the NF4 GEMV with the LoRA up-projection in the epilogue.
__global__ __launch_bounds__(kGemvThreads) void nf4_gemv_kernel(GemvBatch b) {
  extern __shared__ __align__(16) uint32_t xs[];  // K/2 dwords
  const int j = find_job(b);
  const GemvJob& J = b.jobs[j];
  const int K = J.K, N = J.N;
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
  const bool valid = n < N;
  const int nblk = K >> 6;
  const uint8_t* crow = J.codes + (n * K >> 1) + 16 * h;
  const int64_t brow = n * nblk;
  const bool quad_aligned = (nblk & 3) == 0;
  float acc = 0.0f;

  for (int b0 = 0; b0 < nblk; b0 += 4) {
    uint4 cw[4];
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) {
      if (valid && b0 + bi < nblk) {
        cw[bi] = *reinterpret_cast<const uint4*>(crow + 32 * (b0 + bi));
      } else {
        cw[bi].x = cw[bi].y = cw[bi].z = cw[bi].w = 0x77777777u;  // code 7 = level 0
      }
    }
    float t[4] = {0.f, 0.f, 0.f, 0.f};
    if (valid) {
      if (quad_aligned) {
        const uint32_t q4 = *reinterpret_cast<const uint32_t*>(J.absmax_q + brow + b0);
        const float s2 = J.group_scale[(brow + b0) >> 8];
#pragma unroll
        for (int bi = 0; bi < 4; ++bi) t[bi] = block_scale((q4 >> (8 * bi)) & 0xFFu, s2);
      } else {
#pragma unroll
        for (int bi = 0; bi < 4; ++bi)
          if (b0 + bi < nblk)
            t[bi] = block_scale(J.absmax_q[brow + b0 + bi], J.group_scale[(brow + b0 + bi) >> 8]);
      }
    }
    f32x16_t C;
#pragma unroll
    for (int e = 0; e < 16; ++e) C[e] = 0.0f;
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) {
      const uint32_t words[4] = {cw[bi].x, cw[bi].y, cw[bi].z, cw[bi].w};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        uint32_t o[4];
        dequant8_eo(words[kk], T, o);
        const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
        uint4 av = make_uint4(0u, 0u, 0u, 0u);
        if (jr == bi && b0 + bi < nblk) av = *reinterpret_cast<const uint4*>(xs + 32 * (b0 + bi) + 16 * h + 4 * kk);
        C = mfma32x32x16(__builtin_bit_cast(bf16x8_t, av), bop, C);
      }
    }
    acc += t[0] * C[0] + t[1] * C[1] + t[2] * C[2] + t[3] * C[3];
  }

  // LoRA up-projection: lanes j and j+32 take alternate groups of 8 ranks
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
