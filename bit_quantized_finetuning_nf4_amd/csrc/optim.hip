// optim.hip -- the AdamW step on the LoRA matrices, the step after the
// backward pass.  The pages name paged optimizers, whose states move
// between GPU and CPU memory (glossary "Definition"; deepfa.ir blog "3.
// Paged Optimizers"); the optimizer itself is read as AdamW with bias
// correction and decoupled weight decay on fp32 master values, fp32 moments
// and the fp32 gradients of the backward pass.
//
// An HBM stream: 30 bytes per parameter (p, g, m, v read; p, m, v and the
// bf16 copy written), four parameters per lane per iteration.  Every pointer
// may be device memory or pinned host memory (the GPU reads and writes such
// memory in place over the host link): states kept on the host are the
// CPU-resident side of a paged optimizer.
#include <algorithm>
#include <cmath>

#include "device.h"
#include "kernels.h"

namespace qlora {

namespace {

struct AdamW {
  float lr, b1, b2, eps, wd, bc1, bc2;   // bc = 1 - beta^t
};

__device__ __forceinline__ float adamw1(float& p, float g, float& m, float& v, const AdamW& o) {
  m = o.b1 * m + (1.0f - o.b1) * g;
  v = o.b2 * v + (1.0f - o.b2) * g * g;
  const float mh = m / o.bc1, vh = v / o.bc2;
  p = p - o.lr * (mh / (sqrtf(vh) + o.eps) + o.wd * p);
  return p;
}

__global__ __launch_bounds__(256) void adamw_kernel(float* __restrict__ p, bf16_t* __restrict__ pb,
                                                    const float* __restrict__ g, float* __restrict__ m,
                                                    float* __restrict__ v, int64_t n, AdamW o) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * 4;
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < n; i += stride) {
    if (i + 4 <= n) {
      float4 pv = *reinterpret_cast<const float4*>(p + i);
      const float4 gv = *reinterpret_cast<const float4*>(g + i);
      float4 mv = *reinterpret_cast<const float4*>(m + i);
      float4 vv = *reinterpret_cast<const float4*>(v + i);
      adamw1(pv.x, gv.x, mv.x, vv.x, o);
      adamw1(pv.y, gv.y, mv.y, vv.y, o);
      adamw1(pv.z, gv.z, mv.z, vv.z, o);
      adamw1(pv.w, gv.w, mv.w, vv.w, o);
      *reinterpret_cast<float4*>(p + i) = pv;
      *reinterpret_cast<float4*>(m + i) = mv;
      *reinterpret_cast<float4*>(v + i) = vv;
      if (pb) *reinterpret_cast<uint2*>(pb + i) = make_uint2(pack_bf16x2(pv.x, pv.y), pack_bf16x2(pv.z, pv.w));
    } else {
      for (int64_t j = i; j < n; ++j) {
        float pj = p[j], mj = m[j], vj = v[j];
        adamw1(pj, g[j], mj, vj, o);
        p[j] = pj;
        m[j] = mj;
        v[j] = vj;
        if (pb) pb[j] = (bf16_t)(pack_bf16x2(pj, 0.0f) & 0xFFFFu);
      }
    }
  }
}

}  // namespace

hipError_t launch_adamw(float* p, bf16_t* p_bf16, const float* g, float* m, float* v, int64_t n, float lr,
                        float beta1, float beta2, float eps, float weight_decay, int step, hipStream_t st) {
  AdamW o;
  o.lr = lr;
  o.b1 = beta1;
  o.b2 = beta2;
  o.eps = eps;
  o.wd = weight_decay;
  o.bc1 = (float)(1.0 - std::pow((double)beta1, (double)step));
  o.bc2 = (float)(1.0 - std::pow((double)beta2, (double)step));
  const int64_t quads = (n + 3) / 4;
  const int64_t want = (quads + 255) / 256;
  const int grid = (int)std::min<int64_t>(want, (int64_t)device_cu_count() * 8);
  hipLaunchKernelGGL(adamw_kernel, dim3(grid), dim3(256), 0, st, p, p_bf16, g, m, v, n, o);
  return hipGetLastError();
}

}  // namespace qlora
