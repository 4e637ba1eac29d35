// kernels.h -- launch helpers implemented by the .hip files (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qlora.h"

namespace qlora {

typedef uint16_t bf16_t;

struct Nf4View {
  const uint8_t* codes;
  const uint8_t* absmax_q;
  const float* group_scale;
  int64_t N;  // rows
  int64_t K;  // cols, K % 64 == 0 on the GEMM/GEMV paths
  int codebook;  // 0 NF4, 1 FP4, 2 Int4 (the values of qlora_codebook)
  int absfmt;    // second-level format (the values of qlora_absmax_format)
};

// Compute units of the current device (256 if the query fails).
int device_cu_count();

// Raise kernel fn's dynamic-LDS limit to `bytes` (the most any of its
// launches asks for) on the current device, once per device.
hipError_t allow_lds(const void* fn, int bytes);
constexpr int kMaxLds = 160 * 1024;

// codebook: 0 NF4, 1 FP4, 2 Int4 (the values of qlora_codebook)
// One AdamW step over n parameters (p_bf16 may be null); see optim.hip.
hipError_t launch_adamw(float* p, bf16_t* p_bf16, const float* g, float* m, float* v, int64_t n, float lr,
                        float beta1, float beta2, float eps, float weight_decay, int step, hipStream_t st);

hipError_t launch_quantize(const bf16_t* W, int64_t numel, uint8_t* codes, uint8_t* absmax_q,
                           float* group_scale, int codebook, int absfmt, hipStream_t s);
hipError_t launch_dequant(const uint8_t* codes, const uint8_t* absmax_q, const float* group_scale,
                          int64_t numel, int codebook, int absfmt, bf16_t* out, hipStream_t s);

// WdT [K x N] = deq(W)^T (bf16) for W [N x K], K % 64 == 0, N < 65536 * 64;
// rows of WdT are ldo >= N elements apart (a column block of a wider matrix).
hipError_t launch_dequant_t(const uint8_t* codes, const uint8_t* absmax_q, const float* group_scale, int64_t N,
                            int64_t K, int codebook, int absfmt, bf16_t* out, int64_t ldo, hipStream_t s);

// Up to kDeqMax weights of one shape (N x K), one codebook and one absmax
// format, dequantized by one launch: weight i to out + i out_gs, as
// launch_dequant (N K weights) or, transposed, as launch_dequant_t.
constexpr int kDeqMax = 8;
struct DeqSrcs {
  const uint8_t* codes[kDeqMax];
  const uint8_t* absmax_q[kDeqMax];
  const float* group_scale[kDeqMax];
};
hipError_t launch_dequant_group(const DeqSrcs& src, int n, int64_t N, int64_t K, int codebook, int absfmt,
                                bool transposed, bf16_t* out, int64_t ldo, int64_t out_gs, hipStream_t s);

// Y = X deq(W)^T + s * U * B^T  (U already holds X A^T in bf16; r may be 0)
hipError_t launch_fwd(const Nf4View& W, const bf16_t* X, int64_t M, const bf16_t* U, const bf16_t* B,
                      int r, float s, bf16_t* Y, hipStream_t st);

// dX = dY deq(W) + s * G * A  (G = dY B in bf16; r may be 0)
hipError_t launch_dx(const Nf4View& W, const bf16_t* dY, int64_t M, const bf16_t* G, const bf16_t* A,
                     int r, float s, bf16_t* dX, hipStream_t st);

// Dense bf16 product on a weight already in bf16, Wd [N x K]:
// Y [M x N] = X Wd^T + s * U * B'^T (r may be 0), where B' [N x r] is B, or,
// with b_trans, the transpose of B [r x N].  The backward runs it on the
// transposed weight: dX = dY (W^T)^T + s G (A^T)^T.  part (part_bytes of
// fp32 scratch, may be null) lets shapes with few tiles and a long
// contraction split it (dense_split_bytes(N, K, M) bytes are enough).
hipError_t launch_bf16_fwd(const bf16_t* Wd, int64_t N, int64_t K, const bf16_t* X, int64_t M, const bf16_t* U,
                           const bf16_t* B, bool b_trans, int r, float s, bf16_t* Y, hipStream_t st,
                           float* part = nullptr, size_t part_bytes = 0);
// The same over a stack of weights with one adapter each: weight rows come in
// groups of gn (the last may be shorter), and the rows of group g take
// columns g r .. g r + r - 1 of U (row stride ldu) in the tail.  gn = N and
// ldu = r is launch_bf16_fwd.
hipError_t launch_bf16_group(const bf16_t* Wd, int64_t N, int64_t K, const bf16_t* X, int64_t M, const bf16_t* U,
                             int ldu, const bf16_t* B, bool b_trans, int r, int64_t gn, float s, bf16_t* Y,
                             hipStream_t st, float* part = nullptr, size_t part_bytes = 0);
// Scratch for a split contraction of the dense product Y [M x N] over K
// (0 when such a shape is not split).
size_t dense_split_bytes(int64_t N, int64_t K, int64_t M);

// Skinny products with a deterministic split-contraction reduction.
// out_bf16 / out_f32 (either may be null) receive scale * result.
size_t skinny_partial_bytes(int64_t rows, int64_t cols, int64_t contraction, int kind);
enum SkinnyKind { kXAt = 0, kDyB = 1, kGtX = 2, kDytU = 3 };
hipError_t launch_xat(const bf16_t* X, const bf16_t* A, int64_t M, int64_t K, int r, float* part,
                      bf16_t* out, bf16_t* out2, float scale, hipStream_t st);
hipError_t launch_dyb(const bf16_t* dY, const bf16_t* B, int64_t M, int64_t N, int r, float* part,
                      bf16_t* out, float scale, hipStream_t st);
// G groups: group g reads columns g N .. of dY [M x ldy] and B + g N r, and
// writes columns g r .. of out [M x G r]; partials: skinny_partial_bytes(M,
// G r, N, kDyB).
hipError_t launch_dyb_group(const bf16_t* dY, int64_t ldy, const bf16_t* B, int64_t M, int64_t N, int r, int G,
                            float* part, bf16_t* out, float scale, hipStream_t st);
// The adapter gradients: dA [G r x K] = scale G^T X (Gm [M x G r], X [M x
// K]) and, per group g, dB_g = scale dY_g^T U_g (columns g N .. of dY [M x
// ldy], columns g r .. of U [M x ldu]) into dB + g N r; the two split
// reductions run as one launch.  Partials: grads_partial_bytes(M, N, K, r, G).
size_t grads_partial_bytes(int64_t M, int64_t N, int64_t K, int r, int G);
hipError_t launch_grads(const bf16_t* Gm, const bf16_t* X, const bf16_t* dY, int64_t ldy, const bf16_t* U, int ldu,
                        int64_t M, int64_t N, int64_t K, int r, int G, float* part, float* dA, float* dB, float scale,
                        hipStream_t st);

// The paged optimizer's layout and step (paged.hip).
bool paged_plan(const qlora_paged_tensor* t, int nt, size_t dev_bytes, qlora_paged_layout* L);
hipError_t paged_adamw(const qlora_paged_tensor* t, int nt, char* ws, const qlora_paged_layout& L, float lr,
                       float b1, float b2, float eps, float wd, int step, int flags, hipStream_t st,
                       hipStream_t copy_stream);

// Decode of one to 16 tokens per linear.
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
// `st`; gemv_run then launches u = A x (one launch for the one-token jobs,
// one for the others) and the NF4 GEMV (one launch per kind of job present:
// one token or several, with absmax rows read two or four bytes at a time or
// byte by byte).
size_t gemv_table_bound(int njobs, int64_t max_rows);
size_t gemv_lds_bytes(int64_t K);
// What gemv_run needs besides the table in device memory.
constexpr int kGvKinds = 4;   // launches per call: batch-1 and several tokens, two absmax layouts each
struct GemvLaunch {
  void* table;
  uint64_t seg_off[kGvKinds], rng_off[kGvKinds], down_off;
  int32_t groups[kGvKinds], max_steps[2];   // max_steps: the two one-token launches
  int32_t n_down, n_rows;                    // u = A x map entries, the first n_rows of them one per adapter row
  int32_t codebook;  // shared by every job of the call: 4-bit codebook | second-level format << 8
};
hipError_t gemv_prepare(const GemvJob* jobs, int njobs, int codebook, void* table, size_t table_bytes,
                        GemvLaunch* out, hipStream_t st);
hipError_t gemv_run(const GemvLaunch& L, hipStream_t st);

}  // namespace qlora
