// capi.hip -- the extern "C" boundary of libqlora (declared in include/qlora.h).
//
// Every entry point validates all of its arguments before it enqueues
// anything, never allocates and never synchronizes.  Scratch memory comes
// from the caller's workspace, carved as follows (each piece 256-byte
// aligned):
//   FWD  (r > 0): U bf16 [M x r] | split partials of X A^T (fp32)
//   BWD  (r > 0): G bf16 [M x r] | U bf16 [M x r] | split partials (fp32,
//                 the largest of X A^T, dY B, G^T X, dY^T U)
//   GEMV        : per job, 128 fp32 for u = A x | the device job table
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "../../include/qlora.h"
#include "kernels.h"

using namespace qlora;

namespace {

thread_local int g_last_hip_error = 0;

constexpr size_t kAlign = 256;
constexpr int kMaxRank = 128;
constexpr int kMaxJobs = 4096;
constexpr int64_t kMaxGemvCols = 32768;
constexpr int32_t kMaxGemvTokens = 16;
constexpr uint64_t kPlanMagic = 0x51474D56504C414EULL;   // marks a plan filled by qlora_gemv_prepare  // x is staged whole in LDS beside the 64 KiB table

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// GEMV scratch for u = A x: kMaxRank fp32 per token slot, max(m, 1) slots per job.
size_t gemv_u_bytes(int64_t njobs, int64_t max_m) {
  return align_up((size_t)njobs * (size_t)std::max<int64_t>(max_m, 1) * kMaxRank * sizeof(float));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

qlora_status hip_status(hipError_t e) {
  if (e == hipSuccess) return QLORA_OK;
  g_last_hip_error = (int)e;
  return QLORA_E_HIP;
}

qlora_status check_weight(const qlora_nf4_weight* q) {
  if (!q) return QLORA_E_NULL;
  if (q->rows <= 0 || q->cols <= 0) return QLORA_E_SHAPE;
  if (q->blocksize != 64 || q->group_blocks != 256) return QLORA_E_UNSUPPORTED;
  if (q->codebook != QLORA_CODEBOOK_NF4 && q->codebook != QLORA_CODEBOOK_FP4 && q->codebook != QLORA_CODEBOOK_INT4)
    return QLORA_E_UNSUPPORTED;
  if (!q->codes || !q->absmax_q || !q->group_scale) return QLORA_E_NULL;
  if (!aligned16(q->codes) || (reinterpret_cast<uintptr_t>(q->group_scale) & 3u)) return QLORA_E_ALIGN;
  return QLORA_OK;
}

// GEMM paths: K % 64 == 0 (blocks never straddle rows), N % 8 == 0 (16-byte
// rows of dY / Y), codes addressed with 32-bit byte offsets (N K / 2 below
// 2^32).
qlora_status check_gemm_weight(const qlora_nf4_weight* q) {
  qlora_status st = check_weight(q);
  if (st != QLORA_OK) return st;
  if (q->cols % 64 != 0 || q->rows % 8 != 0) return QLORA_E_UNSUPPORTED;
  if (q->rows > (int64_t)0xFFFFFFFF / (q->cols / 2)) return QLORA_E_UNSUPPORTED;
  return QLORA_OK;
}

// The fused GEMMs address the token-side matrices (X [M x K], dY [M x N])
// with 32-bit byte offsets: M K and M N below 2^31 elements.
qlora_status check_tokens(int64_t M, const qlora_nf4_weight* q) {
  if (M <= 0 || M > 0x7FFFFFFF) return QLORA_E_SHAPE;
  if (M > (int64_t)0x7FFFFFFF / q->cols || M > (int64_t)0x7FFFFFFF / q->rows) return QLORA_E_UNSUPPORTED;
  return QLORA_OK;
}

qlora_status check_rank(int32_t r, const void* A, const void* B) {
  if (r < 0 || r > kMaxRank || r % 8 != 0) return QLORA_E_UNSUPPORTED;
  if (r > 0) {
    if (!A || !B) return QLORA_E_NULL;
    if (!aligned16(A) || !aligned16(B)) return QLORA_E_ALIGN;
  }
  return QLORA_OK;
}

Nf4View view(const qlora_nf4_weight* q) {
  return Nf4View{q->codes, q->absmax_q, q->group_scale, q->rows, q->cols, q->codebook};
}

struct FwdLayout {
  size_t u, part, total;
};
FwdLayout fwd_layout(int64_t M, int64_t N, int64_t K, int32_t r) {
  FwdLayout L{0, 0, 0};
  if (r == 0) return L;
  L.u = 0;
  L.part = align_up((size_t)M * r * 2);
  L.total = L.part + align_up(skinny_partial_bytes(M, r, K, kXAt));
  (void)N;
  return L;
}

size_t lora_part_bytes(int64_t M, int64_t N, int64_t K, int32_t r);

struct BwdLayout {
  size_t g, u, part, total;
};
BwdLayout bwd_layout(int64_t M, int64_t N, int64_t K, int32_t r) {
  BwdLayout L{0, 0, 0, 0};
  if (r == 0) return L;
  const size_t mr = align_up((size_t)M * r * 2);
  L.g = 0;
  L.u = mr;
  L.part = 2 * mr;
  L.total = L.part + lora_part_bytes(M, N, K, r);
  return L;
}

char* ws_at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

size_t lora_part_bytes(int64_t M, int64_t N, int64_t K, int32_t r) {
  if (r == 0) return 0;
  size_t p = skinny_partial_bytes(M, r, K, kXAt);
  p = std::max(p, skinny_partial_bytes(M, r, N, kDyB));
  p = std::max(p, skinny_partial_bytes(r, K, M, kGtX));
  p = std::max(p, skinny_partial_bytes(N, r, M, kDytU));
  return align_up(p);
}

qlora_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (ws_bytes < need) return QLORA_E_WORKSPACE;
  if (need > 0 && !ws) return QLORA_E_NULL;
  if (need > 0 && !aligned16(ws)) return QLORA_E_ALIGN;
  return QLORA_OK;
}

qlora_status check_adapter_rank(int32_t r) {
  return (r <= 0 || r > kMaxRank || r % 8 != 0) ? QLORA_E_UNSUPPORTED : QLORA_OK;
}

}  // namespace

extern "C" {

const char* qlora_status_str(qlora_status s) {
  switch (s) {
    case QLORA_OK: return "QLORA_OK";
    case QLORA_E_NULL: return "QLORA_E_NULL: a required pointer is NULL";
    case QLORA_E_ALIGN: return "QLORA_E_ALIGN: a pointer is not 16-byte aligned";
    case QLORA_E_SHAPE: return "QLORA_E_SHAPE: a size is not positive or sizes disagree";
    case QLORA_E_UNSUPPORTED: return "QLORA_E_UNSUPPORTED: unsupported blocksize, group, shape or rank";
    case QLORA_E_WORKSPACE: return "QLORA_E_WORKSPACE: workspace smaller than qlora_workspace_bytes()";
    case QLORA_E_HIP: return "QLORA_E_HIP: HIP launch error (see qlora_last_hip_error)";
  }
  return "QLORA_E_UNKNOWN";
}

int qlora_last_hip_error(void) { return g_last_hip_error; }

const char* qlora_version(void) { return "0.1.0"; }

void qlora_nf4_levels(float out[16]) {
  // Same bit patterns as the device table (device.h); see the construction
  // there.
  static const uint32_t bits[16] = {
      0xBF800000u, 0xBF3239B1u, 0xBF066B2Eu, 0xBECA329Eu, 0xBE91A24Bu, 0xBE3D353Du,
      0xBDBA7869u, 0x00000000u, 0x3DA2FB01u, 0x3E24CADFu, 0x3E7C04DAu, 0x3EAD0336u,
      0x3EE1A4B5u, 0x3F1007A9u, 0x3F3913B0u, 0x3F800000u};
  if (!out) return;
  std::memcpy(out, bits, sizeof(bits));
}

qlora_status qlora_codebook_levels(qlora_codebook cb, float out[16]) {
  // Same bit patterns as the device tables (device.h), where the
  // constructions are given.
  static const uint32_t fp4[16] = {
      0xBF800000u, 0xBF2AAAABu, 0xBF000000u, 0xBEAAAAABu, 0xBE800000u, 0xBE2AAAABu,
      0xBDAAAAABu, 0x00000000u, 0x00000000u, 0x3DAAAAABu, 0x3E2AAAABu, 0x3E800000u,
      0x3EAAAAABu, 0x3F000000u, 0x3F2AAAABu, 0x3F800000u};
  static const uint32_t int4[16] = {
      0xBF924925u, 0xBF800000u, 0xBF5B6DB7u, 0xBF36DB6Eu, 0xBF124925u, 0xBEDB6DB7u,
      0xBE924925u, 0xBE124925u, 0x00000000u, 0x3E124925u, 0x3E924925u, 0x3EDB6DB7u,
      0x3F124925u, 0x3F36DB6Eu, 0x3F5B6DB7u, 0x3F800000u};
  if (!out) return QLORA_E_NULL;
  switch (cb) {
    case QLORA_CODEBOOK_NF4: qlora_nf4_levels(out); return QLORA_OK;
    case QLORA_CODEBOOK_FP4: std::memcpy(out, fp4, sizeof(fp4)); return QLORA_OK;
    case QLORA_CODEBOOK_INT4: std::memcpy(out, int4, sizeof(int4)); return QLORA_OK;
  }
  return QLORA_E_UNSUPPORTED;
}

qlora_status qlora_sizes(int64_t rows, int64_t cols, int32_t blocksize, int32_t group_blocks,
                         size_t* codes_bytes, size_t* absmax_q_bytes, size_t* scale_bytes) {
  if (rows <= 0 || cols <= 0) return QLORA_E_SHAPE;
  if (blocksize != 64 || group_blocks != 256) return QLORA_E_UNSUPPORTED;
  if (rows > (int64_t)1 << 40 || cols > (int64_t)1 << 40 || rows > INT64_MAX / cols) return QLORA_E_SHAPE;
  const int64_t n = rows * cols;
  const int64_t nb = (n + 63) / 64;
  const int64_t ng = (nb + 255) / 256;
  if (codes_bytes) *codes_bytes = (size_t)((n + 1) / 2);
  if (absmax_q_bytes) *absmax_q_bytes = (size_t)nb;
  if (scale_bytes) *scale_bytes = (size_t)ng * sizeof(float);
  return QLORA_OK;
}

size_t qlora_workspace_bytes(qlora_op op, int64_t M, int64_t N, int64_t K, int32_t r, int32_t njobs) {
  switch (op) {
    case QLORA_OP_FWD:
      if (M <= 0 || N <= 0 || K <= 0 || r < 0 || r > kMaxRank) return 0;
      return fwd_layout(M, N, K, r).total;
    case QLORA_OP_BWD:
      if (M <= 0 || N <= 0 || K <= 0 || r < 0 || r > kMaxRank) return 0;
      return bwd_layout(M, N, K, r).total;
    case QLORA_OP_GEMV:
      if (njobs <= 0 || njobs > kMaxJobs || N <= 0 || M < 0 || M > kMaxGemvTokens) return 0;
      return gemv_u_bytes(njobs, M) + gemv_table_bound(njobs, N);
    case QLORA_OP_LORA:
      if (M <= 0 || N <= 0 || K <= 0 || r < 0 || r > kMaxRank) return 0;
      return lora_part_bytes(M, N, K, r);
  }
  return 0;
}

qlora_status qlora_adamw(float* p, uint16_t* p_bf16, const float* grad, float* m, float* v, int64_t n,
                         float lr, float beta1, float beta2, float eps, float weight_decay, int32_t step,
                         void* stream) {
  if (!p || !grad || !m || !v) return QLORA_E_NULL;
  if (!aligned16(p) || !aligned16(grad) || !aligned16(m) || !aligned16(v) || (p_bf16 && !aligned16(p_bf16)))
    return QLORA_E_ALIGN;
  if (n <= 0 || step < 1) return QLORA_E_SHAPE;
  if (!(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f) || !(eps > 0.0f) ||
      !std::isfinite(lr) || !std::isfinite(weight_decay))
    return QLORA_E_SHAPE;
  return hip_status(launch_adamw(p, p_bf16, grad, m, v, n, lr, beta1, beta2, eps, weight_decay, step,
                                 (hipStream_t)stream));
}

qlora_status qlora_quantize(const uint16_t* W, const qlora_nf4_weight* q, void* stream) {
  qlora_status st = check_weight(q);
  if (st != QLORA_OK) return st;
  if (!W) return QLORA_E_NULL;
  if (!aligned16(W)) return QLORA_E_ALIGN;
  if (q->rows > INT64_MAX / q->cols) return QLORA_E_SHAPE;
  const int64_t n = q->rows * q->cols;
  if ((n + 16383) / 16384 > 0x7FFFFFFF) return QLORA_E_SHAPE;
  return hip_status(
      launch_quantize(W, n, q->codes, q->absmax_q, q->group_scale, q->codebook, (hipStream_t)stream));
}

qlora_status qlora_dequant(const qlora_nf4_weight* q, uint16_t* W_out, void* stream) {
  qlora_status st = check_weight(q);
  if (st != QLORA_OK) return st;
  if (!W_out) return QLORA_E_NULL;
  if (!aligned16(W_out)) return QLORA_E_ALIGN;
  if (q->rows > INT64_MAX / q->cols) return QLORA_E_SHAPE;
  const int64_t n = q->rows * q->cols;
  if ((n + 63) / 64 / 256 > 0x7FFFFFFF) return QLORA_E_SHAPE;
  return hip_status(
      launch_dequant(q->codes, q->absmax_q, q->group_scale, n, q->codebook, W_out, (hipStream_t)stream));
}

qlora_status qlora_linear_fwd(const qlora_nf4_weight* W, const uint16_t* X, int64_t M, const uint16_t* A,
                              const uint16_t* B, int32_t r, float alpha, uint16_t* Y, uint16_t* U_save,
                              void* ws, size_t ws_bytes, void* stream) {
  qlora_status st = check_gemm_weight(W);
  if (st != QLORA_OK) return st;
  if ((st = check_tokens(M, W)) != QLORA_OK) return st;
  if (!X || !Y) return QLORA_E_NULL;
  if (!aligned16(X) || !aligned16(Y) || (U_save && !aligned16(U_save))) return QLORA_E_ALIGN;
  if ((st = check_rank(r, A, B)) != QLORA_OK) return st;
  const FwdLayout L = fwd_layout(M, W->rows, W->cols, r);
  if (ws_bytes < L.total) return QLORA_E_WORKSPACE;
  if (L.total > 0 && !ws) return QLORA_E_NULL;
  if (L.total > 0 && !aligned16(ws)) return QLORA_E_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  const Nf4View v = view(W);
  const bf16_t* U = nullptr;
  float sc = 0.0f;
  if (r > 0) {
    sc = (float)((double)alpha / (double)r);  // s = RN32(alpha / r)
    bf16_t* Ud = U_save ? U_save : reinterpret_cast<bf16_t*>(ws_at(ws, L.u));
    float* part = reinterpret_cast<float*>(ws_at(ws, L.part));
    st = hip_status(launch_xat(X, A, M, W->cols, r, part, Ud, nullptr, 1.0f, s));
    if (st != QLORA_OK) return st;
    U = Ud;
  }
  return hip_status(launch_fwd(v, X, M, U, B, r, sc, Y, s));
}

qlora_status qlora_linear_bwd(const qlora_nf4_weight* W, const uint16_t* X, const uint16_t* dY, int64_t M,
                              const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                              const uint16_t* U_saved, uint16_t* dX, float* dA, float* dB, void* ws,
                              size_t ws_bytes, void* stream) {
  qlora_status st = check_gemm_weight(W);
  if (st != QLORA_OK) return st;
  if ((st = check_tokens(M, W)) != QLORA_OK) return st;
  if (!dY) return QLORA_E_NULL;
  if (!aligned16(dY) || (dX && !aligned16(dX)) || (U_saved && !aligned16(U_saved))) return QLORA_E_ALIGN;
  if ((st = check_rank(r, A, B)) != QLORA_OK) return st;
  if (r > 0) {
    if (!dA || !dB || !X) return QLORA_E_NULL;
    if (!aligned16(dA) || !aligned16(dB) || !aligned16(X)) return QLORA_E_ALIGN;
  } else {
    if (dA || dB) return QLORA_E_SHAPE;  // no adapter, no adapter gradients
  }
  const BwdLayout L = bwd_layout(M, W->rows, W->cols, r);
  if (ws_bytes < L.total) return QLORA_E_WORKSPACE;
  if (L.total > 0 && !ws) return QLORA_E_NULL;
  if (L.total > 0 && !aligned16(ws)) return QLORA_E_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  const Nf4View v = view(W);
  const int64_t N = W->rows, K = W->cols;
  if (r == 0) {
    if (!dX) return QLORA_OK;
    return hip_status(launch_dx(v, dY, M, nullptr, nullptr, 0, 0.0f, dX, s));
  }
  const float sc = (float)((double)alpha / (double)r);
  bf16_t* G = reinterpret_cast<bf16_t*>(ws_at(ws, L.g));
  float* part = reinterpret_cast<float*>(ws_at(ws, L.part));
  const bf16_t* U = U_saved;
  if (!U) {
    bf16_t* Ud = reinterpret_cast<bf16_t*>(ws_at(ws, L.u));
    st = hip_status(launch_xat(X, A, M, K, r, part, Ud, nullptr, 1.0f, s));
    if (st != QLORA_OK) return st;
    U = Ud;
  }
  st = hip_status(launch_dyb(dY, B, M, N, r, part, G, 1.0f, s));
  if (st != QLORA_OK) return st;
  if (dX) {
    st = hip_status(launch_dx(v, dY, M, G, A, r, sc, dX, s));
    if (st != QLORA_OK) return st;
  }
  st = hip_status(launch_gtx(G, X, M, K, r, part, dA, sc, s));
  if (st != QLORA_OK) return st;
  return hip_status(launch_dytu(dY, U, M, N, r, part, dB, sc, s));
}

qlora_status qlora_lora_down(const uint16_t* X, const uint16_t* A, int64_t M, int64_t K, int32_t r, uint16_t* U,
                             void* ws, size_t ws_bytes, void* stream) {
  qlora_status st = check_adapter_rank(r);
  if (st != QLORA_OK) return st;
  if (M <= 0 || M > 0x7FFFFFFF || K <= 0 || K % 8 != 0) return QLORA_E_SHAPE;
  if (!X || !A || !U) return QLORA_E_NULL;
  if (!aligned16(X) || !aligned16(A) || !aligned16(U)) return QLORA_E_ALIGN;
  if ((st = check_ws(ws, ws_bytes, align_up(skinny_partial_bytes(M, r, K, kXAt)))) != QLORA_OK) return st;
  return hip_status(launch_xat(X, A, M, K, r, static_cast<float*>(ws), U, nullptr, 1.0f, (hipStream_t)stream));
}

qlora_status qlora_lora_dy_b(const uint16_t* dY, const uint16_t* B, int64_t M, int64_t N, int32_t r, uint16_t* G,
                             void* ws, size_t ws_bytes, void* stream) {
  qlora_status st = check_adapter_rank(r);
  if (st != QLORA_OK) return st;
  if (M <= 0 || M > 0x7FFFFFFF || N <= 0 || N % 8 != 0) return QLORA_E_SHAPE;
  if (!dY || !B || !G) return QLORA_E_NULL;
  if (!aligned16(dY) || !aligned16(B) || !aligned16(G)) return QLORA_E_ALIGN;
  if ((st = check_ws(ws, ws_bytes, align_up(skinny_partial_bytes(M, r, N, kDyB)))) != QLORA_OK) return st;
  return hip_status(launch_dyb(dY, B, M, N, r, static_cast<float*>(ws), G, 1.0f, (hipStream_t)stream));
}

qlora_status qlora_lora_grads(const uint16_t* X, const uint16_t* dY, const uint16_t* U, const uint16_t* G,
                              int64_t M, int64_t N, int64_t K, int32_t r, float alpha, float* dA, float* dB,
                              void* ws, size_t ws_bytes, void* stream) {
  qlora_status st = check_adapter_rank(r);
  if (st != QLORA_OK) return st;
  if (M <= 0 || M > 0x7FFFFFFF || N <= 0 || N % 8 != 0 || K <= 0 || K % 8 != 0) return QLORA_E_SHAPE;
  // X and dY are addressed with 32-bit byte offsets
  if (M > (int64_t)0x7FFFFFFF / K || M > (int64_t)0x7FFFFFFF / N) return QLORA_E_UNSUPPORTED;
  if (!X || !dY || !U || !G || !dA || !dB) return QLORA_E_NULL;
  if (!aligned16(X) || !aligned16(dY) || !aligned16(U) || !aligned16(G) || !aligned16(dA) || !aligned16(dB))
    return QLORA_E_ALIGN;
  const size_t need = align_up(std::max(skinny_partial_bytes(r, K, M, kGtX), skinny_partial_bytes(N, r, M, kDytU)));
  if ((st = check_ws(ws, ws_bytes, need)) != QLORA_OK) return st;
  const float sc = (float)((double)alpha / (double)r);
  hipStream_t s = (hipStream_t)stream;
  st = hip_status(launch_gtx(G, X, M, K, r, static_cast<float*>(ws), dA, sc, s));
  if (st != QLORA_OK) return st;
  return hip_status(launch_dytu(dY, U, M, N, r, static_cast<float*>(ws), dB, sc, s));
}

qlora_status qlora_nf4_fwd(const qlora_nf4_weight* W, const uint16_t* X, int64_t M, const uint16_t* U,
                           const uint16_t* B, int32_t r, float alpha, uint16_t* Y, void* stream) {
  qlora_status st = check_gemm_weight(W);
  if (st != QLORA_OK) return st;
  if ((st = check_tokens(M, W)) != QLORA_OK) return st;
  if (!X || !Y) return QLORA_E_NULL;
  if (!aligned16(X) || !aligned16(Y)) return QLORA_E_ALIGN;
  if ((st = check_rank(r, U, B)) != QLORA_OK) return st;
  const float sc = r > 0 ? (float)((double)alpha / (double)r) : 0.0f;
  return hip_status(launch_fwd(view(W), X, M, r > 0 ? U : nullptr, r > 0 ? B : nullptr, r, sc, Y,
                               (hipStream_t)stream));
}

qlora_status qlora_nf4_dx(const qlora_nf4_weight* W, const uint16_t* dY, int64_t M, const uint16_t* G,
                          const uint16_t* A, int32_t r, float alpha, uint16_t* dX, void* stream) {
  qlora_status st = check_gemm_weight(W);
  if (st != QLORA_OK) return st;
  if ((st = check_tokens(M, W)) != QLORA_OK) return st;
  if (!dY || !dX) return QLORA_E_NULL;
  if (!aligned16(dY) || !aligned16(dX)) return QLORA_E_ALIGN;
  if ((st = check_rank(r, G, A)) != QLORA_OK) return st;
  const float sc = r > 0 ? (float)((double)alpha / (double)r) : 0.0f;
  return hip_status(launch_dx(view(W), dY, M, r > 0 ? G : nullptr, r > 0 ? A : nullptr, r, sc, dX,
                              (hipStream_t)stream));
}

qlora_status qlora_gemv_prepare(const qlora_gemv_job* jobs, int32_t njobs, void* ws, size_t ws_bytes,
                                qlora_gemv_plan* plan, void* stream) {
  if (!jobs || !plan) return QLORA_E_NULL;
  if (njobs <= 0) return QLORA_E_SHAPE;
  if (njobs > kMaxJobs) return QLORA_E_UNSUPPORTED;
  int32_t max_m = 1;
  for (int i = 0; i < njobs; ++i) {
    const qlora_gemv_job& J = jobs[i];
    qlora_status st = check_weight(J.W);
    if (st != QLORA_OK) return st;
    if (J.m < 0) return QLORA_E_SHAPE;
    if (J.m > kMaxGemvTokens) return QLORA_E_UNSUPPORTED;
    max_m = std::max(max_m, J.m);
    // one codebook per call: the kernel builds its decode table once
    if (J.W->codebook != jobs[0].W->codebook) return QLORA_E_UNSUPPORTED;
    if (J.W->cols % 64 != 0 || J.W->cols > kMaxGemvCols || J.W->rows > 0x7FFFFFFF) return QLORA_E_UNSUPPORTED;
    // codes addressed with 32-bit byte offsets, including the prefetch of
    // one row's worth of blocks past the last row
    if (J.W->rows + 1 > ((int64_t)0xFFFFFFFF - 256) / (J.W->cols / 2)) return QLORA_E_UNSUPPORTED;
    if (!J.x || !J.y) return QLORA_E_NULL;
    if (!aligned16(J.x) || !aligned16(J.y)) return QLORA_E_ALIGN;
    if ((st = check_rank(J.r, J.A, J.B)) != QLORA_OK) return st;
    // B [rows x r] addressed with 32-bit byte offsets
    if (J.r > 0 && J.W->rows > (int64_t)0xFFFFFFFF / (2 * (int64_t)J.r)) return QLORA_E_UNSUPPORTED;
  }
  if (!ws) return QLORA_E_NULL;
  if (!aligned16(ws)) return QLORA_E_ALIGN;
  std::vector<GemvJob> buf((size_t)njobs);
  for (int i = 0; i < njobs; ++i) {
    const qlora_gemv_job& J = jobs[i];
    GemvJob& D = buf[(size_t)i];
    D.codes = J.W->codes;
    D.absmax_q = J.W->absmax_q;
    D.group_scale = J.W->group_scale;
    D.x = J.x;
    D.A = J.r > 0 ? J.A : nullptr;
    D.B = J.r > 0 ? J.B : nullptr;
    D.y = J.y;
    D.u = J.r > 0 ? reinterpret_cast<float*>(ws_at(ws, (size_t)i * (size_t)max_m * kMaxRank * sizeof(float)))
                  : nullptr;
    D.N = (int32_t)J.W->rows;
    D.K = (int32_t)J.W->cols;
    D.r = J.r;
    D.s = J.r > 0 ? (float)((double)J.alpha / (double)J.r) : 0.0f;
    D.m = std::max(J.m, 1);
  }
  const size_t u_bytes = gemv_u_bytes(njobs, max_m);
  const size_t table_bytes = gemv_table_bound(njobs, 1);
  if (ws_bytes < u_bytes || ws_bytes - u_bytes < table_bytes) return QLORA_E_WORKSPACE;
  GemvLaunch L{};
  qlora_status st = hip_status(
      gemv_prepare(buf.data(), njobs, jobs[0].W->codebook, ws_at(ws, u_bytes), table_bytes, &L, (hipStream_t)stream));
  if (st != QLORA_OK) return st;
  static_assert(sizeof(GemvLaunch) + sizeof(uint64_t) <= sizeof(qlora_gemv_plan), "plan storage");
  std::memset(plan, 0, sizeof(*plan));
  plan->priv[0] = kPlanMagic;
  std::memcpy(&plan->priv[1], &L, sizeof(L));
  return QLORA_OK;
}

qlora_status qlora_gemv_run(const qlora_gemv_plan* plan, void* stream) {
  if (!plan) return QLORA_E_NULL;
  if (plan->priv[0] != kPlanMagic) return QLORA_E_SHAPE;
  GemvLaunch L;
  std::memcpy(&L, &plan->priv[1], sizeof(L));
  return hip_status(gemv_run(L, (hipStream_t)stream));
}

qlora_status qlora_gemv(const qlora_gemv_job* jobs, int32_t njobs, void* ws, size_t ws_bytes, void* stream) {
  qlora_gemv_plan plan;
  const qlora_status st = qlora_gemv_prepare(jobs, njobs, ws, ws_bytes, &plan, stream);
  return st != QLORA_OK ? st : qlora_gemv_run(&plan, stream);
}

}  // extern "C"
