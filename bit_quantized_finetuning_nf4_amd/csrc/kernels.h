// kernels.h -- launch helpers implemented by the .hip files (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlora {

typedef uint16_t bf16_t;

struct Nf4View {
  const uint8_t* codes;
  const uint8_t* absmax_q;
  const float* group_scale;
  int64_t N;  // rows
  int64_t K;  // cols, K % 64 == 0 on the GEMM/GEMV paths
  int codebook;  // 0 NF4, 1 FP4, 2 Int4 (the values of qlora_codebook)
};

// Compute units of the current device (256 if the query fails).
int device_cu_count();

// codebook: 0 NF4, 1 FP4, 2 Int4 (the values of qlora_codebook)
// One AdamW step over n parameters (p_bf16 may be null); see optim.hip.
hipError_t launch_adamw(float* p, bf16_t* p_bf16, const float* g, float* m, float* v, int64_t n, float lr,
                        float beta1, float beta2, float eps, float weight_decay, int step, hipStream_t st);

hipError_t launch_quantize(const bf16_t* W, int64_t numel, uint8_t* codes, uint8_t* absmax_q,
                           float* group_scale, int codebook, hipStream_t s);
hipError_t launch_dequant(const uint8_t* codes, const uint8_t* absmax_q, const float* group_scale,
                          int64_t numel, int codebook, bf16_t* out, hipStream_t s);

// Y = X deq(W)^T + s * U * B^T  (U already holds X A^T in bf16; r may be 0)
hipError_t launch_fwd(const Nf4View& W, const bf16_t* X, int64_t M, const bf16_t* U, const bf16_t* B,
                      int r, float s, bf16_t* Y, hipStream_t st);

// dX = dY deq(W) + s * G * A  (G = dY B in bf16; r may be 0)
hipError_t launch_dx(const Nf4View& W, const bf16_t* dY, int64_t M, const bf16_t* G, const bf16_t* A,
                     int r, float s, bf16_t* dX, hipStream_t st);

// Skinny products with a deterministic split-contraction reduction.
// out_bf16 / out_f32 (either may be null) receive scale * result.
size_t skinny_partial_bytes(int64_t rows, int64_t cols, int64_t contraction, int kind);
enum SkinnyKind { kXAt = 0, kDyB = 1, kGtX = 2, kDytU = 3 };
hipError_t launch_xat(const bf16_t* X, const bf16_t* A, int64_t M, int64_t K, int r, float* part,
                      bf16_t* out, bf16_t* out2, float scale, hipStream_t st);
hipError_t launch_dyb(const bf16_t* dY, const bf16_t* B, int64_t M, int64_t N, int r, float* part,
                      bf16_t* out, float scale, hipStream_t st);
hipError_t launch_gtx(const bf16_t* G, const bf16_t* X, int64_t M, int64_t K, int r, float* part,
                      float* dA, float scale, hipStream_t st);
hipError_t launch_dytu(const bf16_t* dY, const bf16_t* U, int64_t M, int64_t N, int r, float* part,
                       float* dB, float scale, hipStream_t st);

// Batch-1 decode.
struct GemvJob {
  const uint8_t* codes;
  const uint8_t* absmax_q;
  const float* group_scale;
  const bf16_t* x;
  const bf16_t* A;
  const bf16_t* B;
  bf16_t* y;
  float* u;  // m x r fp32 scratch (A x per token)
  int32_t N;
  int32_t K;
  int32_t r;
  float s;
  int32_t m;  // tokens: x is [m x K], y [m x N]
};
// gemv_prepare writes the job table (jobs, per-workgroup tile segments and
// the u = A x map) into `table` (device memory of at least
// gemv_table_bound(njobs, max rows) bytes) by one host-to-device copy on
// `st`; gemv_run then launches u = A x and the NF4 GEMV (two launches of it
// when some jobs need the byte-wise absmax path).
size_t gemv_table_bound(int njobs, int64_t max_rows);
size_t gemv_lds_bytes(int64_t K);
// What gemv_run needs besides the table in device memory.
constexpr int kGvKinds = 4;   // launches per call: batch-1 and several tokens, two absmax layouts each
struct GemvLaunch {
  void* table;
  uint64_t seg_off[kGvKinds], rng_off[kGvKinds], down_off;
  int32_t groups[kGvKinds], max_steps[kGvKinds];
  int32_t n_down;
  int32_t codebook;  // shared by every job of the call
};
hipError_t gemv_prepare(const GemvJob* jobs, int njobs, int codebook, void* table, size_t table_bytes,
                        GemvLaunch* out, hipStream_t st);
hipError_t gemv_run(const GemvLaunch& L, hipStream_t st);

}  // namespace qlora
