// capi.hip -- the extern "C" boundary of libqlora (declared in include/qlora.h).
//
// Every entry point validates all of its arguments before it enqueues
// anything, never allocates and never synchronizes.  Scratch memory comes
// from the caller's workspace, carved as follows (each piece 256-byte
// aligned):
//   FWD  (r > 0): U bf16 [M x r] | split partials of X A^T (fp32)
//        staged : ... | deq(W) bf16 [N x K]
//   BWD  (r > 0): G bf16 [M x r] | U bf16 [M x r] | split partials (fp32,
//                 the largest of X A^T, dY B and G^T X with dY^T U side by
//                 side)
//        staged : ... | deq(W)^T bf16 [K x N]
// A staged call dequantizes W once into the workspace and multiplies with
// the dense bf16 kernel; otherwise the fused kernels decode W inside each
// 256-token tile.  Staging pays off once a weight would be decoded several
// times, so it is taken from kStagedMinTokens tokens on, when the workspace
// holds the bf16 weight.
//   GEMV        : per job, 128 fp32 for u = A x | the device job table
// qlora_linear_fwd_noalloc carves the FWD layout out of `scratch` below
// instead of a caller workspace.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
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
constexpr uint64_t kPlanMagic = 0x51474D56504C414EULL;   // marks a plan filled by qlora_gemv_prepare

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
  if (q->absmax_format != QLORA_ABSMAX_LINEAR8 && q->absmax_format != QLORA_ABSMAX_FP8) return QLORA_E_UNSUPPORTED;
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

// The LoRA side products address a 128-row tile of the large operand
// (128 C bf16) and the rank-side operand (r C bf16, r <= 128) with 32-bit
// byte ranges: C (K or N) below 2^24.
constexpr int64_t kMaxSkinnyCols = (int64_t)1 << 24;
bool skinny_cols_ok(int64_t C) { return C < kMaxSkinnyCols; }

qlora_status check_rank(int32_t r, const void* A, const void* B) {
  if (r < 0 || r > kMaxRank || r % 8 != 0) return QLORA_E_UNSUPPORTED;
  if (r > 0) {
    if (!A || !B) return QLORA_E_NULL;
    if (!aligned16(A) || !aligned16(B)) return QLORA_E_ALIGN;
  }
  return QLORA_OK;
}

Nf4View view(const qlora_nf4_weight* q) {
  return Nf4View{q->codes, q->absmax_q, q->group_scale, q->rows, q->cols, q->codebook, q->absmax_format};
}

constexpr int64_t kStagedMinTokens = 1024;

// Order of the staged backward.  G = dY B reads dY, which the dX product
// reads again; when dY (M x N bf16) is at most half the 256 MB last-level
// cache, G runs after the transposed dequantization, right before the dX
// product, so that dY is still in the cache there.  A larger dY would push
// the dequantized weight out instead, so G runs first.
bool dy_late(int64_t M, int64_t N) { return M * N * 2 <= ((int64_t)128 << 20); }

// The staged path's bf16 weight is addressed with 32-bit byte offsets, and
// the transposing dequant grid has ceil(N / 64) rows.  The dense kernel runs
// its contraction in whole pairs of 32-wide stages: K % 64 == 0 holds on
// every GEMM path; dX contracts over N, so its staged form needs N % 64 == 0.
bool staged_ok(int64_t M, int64_t N, int64_t K) {
  return M >= kStagedMinTokens && N <= (int64_t)0x7FFFFFFF / K && (N + 63) / 64 <= 65535;
}
bool staged_bwd_ok(int64_t M, int64_t N, int64_t K) { return staged_ok(M, N, K) && N % 64 == 0; }

struct FwdLayout {
  size_t u, part, wd, total;
};
FwdLayout fwd_layout(int64_t M, int64_t N, int64_t K, int32_t r, bool staged) {
  FwdLayout L{0, 0, 0, 0};
  if (r > 0) {
    L.u = 0;
    L.part = align_up((size_t)M * r * 2);
    L.total = L.part + align_up(skinny_partial_bytes(M, r, K, kXAt));
  }
  if (staged) {
    L.wd = L.total;
    L.total += align_up((size_t)N * (size_t)K * 2);
  }
  return L;
}

size_t lora_part_bytes(int64_t M, int64_t N, int64_t K, int32_t r);

struct BwdLayout {
  size_t g, u, part, wdt, split, split_bytes, total;
};
BwdLayout bwd_layout(int64_t M, int64_t N, int64_t K, int32_t r, bool staged) {
  BwdLayout L{0, 0, 0, 0, 0, 0, 0};
  if (r > 0) {
    const size_t mr = align_up((size_t)M * r * 2);
    L.g = 0;
    L.u = mr;
    L.part = 2 * mr;
    L.total = L.part + lora_part_bytes(M, N, K, r);
  }
  if (staged) {
    L.wdt = L.total;
    L.total += align_up((size_t)N * (size_t)K * 2);
    // dX [M x K] contracts over N
    L.split = L.total;
    L.split_bytes = dense_split_bytes(K, N, M);
    L.total += align_up(L.split_bytes);
  }
  return L;
}

char* ws_at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

size_t lora_part_bytes(int64_t M, int64_t N, int64_t K, int32_t r) {
  if (r == 0) return 0;
  size_t p = skinny_partial_bytes(M, r, K, kXAt);
  p = std::max(p, skinny_partial_bytes(M, r, N, kDyB));
  p = std::max(p, grads_partial_bytes(M, N, K, r, 1));
  return align_up(p);
}

// Layer-set groups: G weights of one shape N x K read the same input, with
// the adapters stacked (A [G r x K], B [G N x r]) and the outputs side by
// side (Y, dY [M x G N]).  Always staged.
//   GROUP_FWD: U bf16 [M x G r] | partials of X A^T | deq(W_g) stacked [G N x K]
//   GROUP_BWD: G bf16 [M x G r] | U bf16 [M x G r] | partials (the largest
//              of X A^T, dY B and the two gradients' side by side) |
//              deq(W_g)^T side by side [K x G N] and the dense product's
//              split partials, if it splits (with dX)
constexpr int kMaxGroupRank = 256;   // G r: the largest rank tile of the side products

bool group_sizes_ok(int64_t M, int64_t N, int64_t K, int32_t r, int32_t G) {
  if (M <= 0 || N <= 0 || K <= 0 || G < 1 || r < 0 || r > kMaxRank || (int64_t)G * r > kMaxGroupRank) return false;
  const int64_t NG = (int64_t)G * N;
  return NG <= (int64_t)0x7FFFFFFF / K;
}

// Split partial sums of the group's side products: U = X A^T at rank G r,
// dY B over all groups, and the gradients (G^T X at rank G r and dY^T U per
// group, side by side).
size_t group_part_bytes(int64_t M, int64_t N, int64_t K, int32_t r, int32_t G) {
  if (r == 0) return 0;
  const int32_t rg = G * r;
  size_t p = skinny_partial_bytes(M, rg, K, kXAt);
  p = std::max(p, skinny_partial_bytes(M, rg, N, kDyB));
  p = std::max(p, grads_partial_bytes(M, N, K, r, G));
  return align_up(p);
}

FwdLayout group_fwd_layout(int64_t M, int64_t N, int64_t K, int32_t r, int32_t G) {
  FwdLayout L{0, 0, 0, 0};
  const int32_t rg = G * r;
  if (r > 0) {
    L.part = align_up((size_t)M * rg * 2);
    L.total = L.part + align_up(skinny_partial_bytes(M, rg, K, kXAt));
  }
  L.wd = L.total;
  L.total += align_up((size_t)G * (size_t)N * (size_t)K * 2);
  return L;
}

BwdLayout group_bwd_layout(int64_t M, int64_t N, int64_t K, int32_t r, int32_t G, bool with_dx) {
  BwdLayout L{0, 0, 0, 0, 0, 0, 0};
  const int32_t rg = G * r;
  if (r > 0) {
    const size_t mr = align_up((size_t)M * rg * 2);
    L.u = mr;
    L.part = 2 * mr;
    L.total = L.part + group_part_bytes(M, N, K, r, G);
  }
  if (with_dx) {
    L.wdt = L.total;
    L.total += align_up((size_t)G * (size_t)N * (size_t)K * 2);
    L.split = L.total;
    L.split_bytes = dense_split_bytes(K, (int64_t)G * N, M);
    L.total += align_up(L.split_bytes);
  }
  return L;
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

// Scratch of qlora_linear_fwd_noalloc: one array per device, held until the
// process ends.  In host code `scratch` only names the symbol; its device
// address comes from hipGetSymbolAddress, looked up once per device.
static __device__ __align__(256) unsigned char scratch[QLORA_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device

// The device address of `scratch` on the current device.
qlora_status static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return QLORA_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (!p) return QLORA_E_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return QLORA_OK;
}

// Argument checks of the forward, before any workspace is looked at.
qlora_status check_fwd(const qlora_nf4_weight* W, const uint16_t* X, int64_t M, const uint16_t* A,
                       const uint16_t* B, int32_t r, const uint16_t* Y, const uint16_t* U_save) {
  qlora_status st = check_gemm_weight(W);
  if (st != QLORA_OK) return st;
  if ((st = check_tokens(M, W)) != QLORA_OK) return st;
  if (!X || !Y) return QLORA_E_NULL;
  if (!aligned16(X) || !aligned16(Y) || (U_save && !aligned16(U_save))) return QLORA_E_ALIGN;
  if ((st = check_rank(r, A, B)) != QLORA_OK) return st;
  if (r > 0 && !skinny_cols_ok(W->cols)) return QLORA_E_UNSUPPORTED;
  return QLORA_OK;
}

// The forward's launches, on a workspace of the FWD layout.
qlora_status run_fwd(const qlora_nf4_weight* W, const uint16_t* X, int64_t M, const uint16_t* A,
                     const uint16_t* B, int32_t r, float alpha, uint16_t* Y, uint16_t* U_save, void* ws,
                     bool staged, hipStream_t s) {
  const FwdLayout L = fwd_layout(M, W->rows, W->cols, r, staged);
  const Nf4View v = view(W);
  const bf16_t* U = nullptr;
  float sc = 0.0f;
  if (r > 0) {
    sc = (float)((double)alpha / (double)r);  // s = RN32(alpha / r)
    bf16_t* Ud = U_save ? U_save : reinterpret_cast<bf16_t*>(ws_at(ws, L.u));
    float* part = reinterpret_cast<float*>(ws_at(ws, L.part));
    qlora_status st = hip_status(launch_xat(X, A, M, W->cols, r, part, Ud, nullptr, 1.0f, s));
    if (st != QLORA_OK) return st;
    U = Ud;
  }
  if (staged) {
    bf16_t* Wd = reinterpret_cast<bf16_t*>(ws_at(ws, L.wd));
    qlora_status st = hip_status(launch_dequant(W->codes, W->absmax_q, W->group_scale, W->rows * W->cols,
                                                W->codebook, W->absmax_format, Wd, s));
    if (st != QLORA_OK) return st;
    return hip_status(launch_bf16_fwd(Wd, W->rows, W->cols, X, M, U, B, false, r, sc, Y, s));
  }
  return hip_status(launch_fwd(v, X, M, U, B, r, sc, Y, s));
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
    case QLORA_E_FORMAT: return "QLORA_E_FORMAT: not a serialized weight header (magic, version or size)";
    case QLORA_E_TABLE: return "QLORA_E_TABLE: the weight was written with other level tables";
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
    case QLORA_OP_FWD_FUSED:
      if (M <= 0 || N <= 0 || K <= 0 || r < 0 || r > kMaxRank) return 0;
      return fwd_layout(M, N, K, r, op == QLORA_OP_FWD && staged_ok(M, N, K)).total;
    case QLORA_OP_BWD:
    case QLORA_OP_BWD_FUSED:
      if (M <= 0 || N <= 0 || K <= 0 || r < 0 || r > kMaxRank) return 0;
      return bwd_layout(M, N, K, r, op == QLORA_OP_BWD && staged_bwd_ok(M, N, K)).total;
    case QLORA_OP_GEMV:
      if (njobs <= 0 || njobs > kMaxJobs || N <= 0 || M < 0 || M > kMaxGemvTokens) return 0;
      return gemv_u_bytes(njobs, M) + gemv_table_bound(njobs, N);
    case QLORA_OP_LORA:   // ranks above 128: qlora_lora_down on a group's stacked adapters
      if (M <= 0 || N <= 0 || K <= 0 || r < 0 || r > kMaxGroupRank) return 0;
      return lora_part_bytes(M, N, K, r);
    case QLORA_OP_GROUP_FWD:
      if (!group_sizes_ok(M, N, K, r, njobs)) return 0;
      return group_fwd_layout(M, N, K, r, njobs).total;
    case QLORA_OP_GROUP_BWD:
      if (!group_sizes_ok(M, N, K, r, njobs)) return 0;
      return group_bwd_layout(M, N, K, r, njobs, true).total;
    case QLORA_OP_GROUP_LORA:
      if (!group_sizes_ok(M, N, K, r, njobs)) return 0;
      return group_part_bytes(M, N, K, r, njobs);
    case QLORA_OP_BF16_DX:
      if (!group_sizes_ok(M, N, K, r, njobs)) return 0;
      return dense_split_bytes(K, (int64_t)njobs * N, M);
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

qlora_status qlora_paged_layout_of(const qlora_paged_tensor* t, int32_t ntensors, size_t dev_bytes,
                                   qlora_paged_layout* out) {
  if (!t || !out) return QLORA_E_NULL;
  if (ntensors <= 0) return QLORA_E_SHAPE;
  for (int i = 0; i < ntensors; ++i)
    if (t[i].n <= 0 || t[i].n > ((int64_t)1 << 40)) return QLORA_E_SHAPE;
  return paged_plan(t, ntensors, dev_bytes, out) ? QLORA_OK : QLORA_E_WORKSPACE;
}

qlora_status qlora_paged_adamw(const qlora_paged_tensor* t, int32_t ntensors, void* dev_ws, size_t dev_bytes,
                               float lr, float beta1, float beta2, float eps, float weight_decay, int32_t step,
                               int32_t flags, void* stream, void* copy_stream) {
  if (!t) return QLORA_E_NULL;
  if (ntensors <= 0 || step < 1) return QLORA_E_SHAPE;
  if (flags & ~(QLORA_PAGED_LOAD | QLORA_PAGED_STORE)) return QLORA_E_UNSUPPORTED;
  if (!(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f) || !(eps > 0.0f) ||
      !std::isfinite(lr) || !std::isfinite(weight_decay))
    return QLORA_E_SHAPE;
  for (int i = 0; i < ntensors; ++i) {
    const qlora_paged_tensor& x = t[i];
    if (!x.p || !x.grad || !x.m || !x.v) return QLORA_E_NULL;
    if (!aligned16(x.p) || !aligned16(x.grad) || !aligned16(x.m) || !aligned16(x.v) ||
        (x.p_bf16 && !aligned16(x.p_bf16)))
      return QLORA_E_ALIGN;
    if (x.n <= 0 || x.n > ((int64_t)1 << 40)) return QLORA_E_SHAPE;
  }
  qlora_paged_layout L;
  if (!paged_plan(t, ntensors, dev_bytes, &L)) return QLORA_E_WORKSPACE;
  if (!dev_ws) return QLORA_E_NULL;
  if (reinterpret_cast<uintptr_t>(dev_ws) & 255u) return QLORA_E_ALIGN;
  return hip_status(paged_adamw(t, ntensors, static_cast<char*>(dev_ws), L, lr, beta1, beta2, eps, weight_decay,
                                step, flags, (hipStream_t)stream, (hipStream_t)copy_stream));
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
      launch_quantize(W, n, q->codes, q->absmax_q, q->group_scale, q->codebook, q->absmax_format,
                      (hipStream_t)stream));
}

qlora_status qlora_dequant(const qlora_nf4_weight* q, uint16_t* W_out, void* stream) {
  qlora_status st = check_weight(q);
  if (st != QLORA_OK) return st;
  if (!W_out) return QLORA_E_NULL;
  if (!aligned16(W_out)) return QLORA_E_ALIGN;
  if (q->rows > INT64_MAX / q->cols) return QLORA_E_SHAPE;
  const int64_t n = q->rows * q->cols;
  if ((n + 63) / 64 / 64 > 0x7FFFFFFF) return QLORA_E_SHAPE;   // the launch's workgroup count
  return hip_status(
      launch_dequant(q->codes, q->absmax_q, q->group_scale, n, q->codebook, q->absmax_format, W_out,
                     (hipStream_t)stream));
}

qlora_status qlora_dequant_t(const qlora_nf4_weight* q, uint16_t* Wt_out, void* stream) {
  qlora_status st = check_weight(q);
  if (st != QLORA_OK) return st;
  if (!Wt_out) return QLORA_E_NULL;
  if (!aligned16(Wt_out)) return QLORA_E_ALIGN;
  if (q->cols % 64 != 0 || q->rows % 8 != 0) return QLORA_E_UNSUPPORTED;
  if (q->cols / 64 > 0x7FFFFFFF || (q->rows + 63) / 64 > 65535) return QLORA_E_UNSUPPORTED;
  return hip_status(launch_dequant_t(q->codes, q->absmax_q, q->group_scale, q->rows, q->cols, q->codebook,
                                     q->absmax_format, Wt_out, q->rows, (hipStream_t)stream));
}

qlora_status qlora_linear_fwd(const qlora_nf4_weight* W, const uint16_t* X, int64_t M, const uint16_t* A,
                              const uint16_t* B, int32_t r, float alpha, uint16_t* Y, uint16_t* U_save,
                              void* ws, size_t ws_bytes, void* stream) {
  qlora_status st = check_fwd(W, X, M, A, B, r, Y, U_save);
  if (st != QLORA_OK) return st;
  const bool staged = staged_ok(M, W->rows, W->cols) &&
                      ws_bytes >= fwd_layout(M, W->rows, W->cols, r, true).total;
  const FwdLayout L = fwd_layout(M, W->rows, W->cols, r, staged);
  if (ws_bytes < L.total) return QLORA_E_WORKSPACE;
  if (L.total > 0 && !ws) return QLORA_E_NULL;
  if (L.total > 0 && !aligned16(ws)) return QLORA_E_ALIGN;
  return run_fwd(W, X, M, A, B, r, alpha, Y, U_save, ws, staged, (hipStream_t)stream);
}

qlora_status qlora_linear_fwd_noalloc(const qlora_nf4_weight* W, const uint16_t* X, int64_t M, const uint16_t* A,
                                      const uint16_t* B, int32_t r, float alpha, uint16_t* Y, uint16_t* U_save,
                                      void* stream) {
  qlora_status st = check_fwd(W, X, M, A, B, r, Y, U_save);
  if (st != QLORA_OK) return st;
  const FwdLayout L = fwd_layout(M, W->rows, W->cols, r, false);   // the fused path: no bf16 weight
  if (L.total > QLORA_STATIC_SCRATCH_BYTES) return QLORA_E_WORKSPACE;
  void* ws = nullptr;
  if (L.total > 0 && (st = static_scratch(&ws)) != QLORA_OK) return st;
  return run_fwd(W, X, M, A, B, r, alpha, Y, U_save, ws, false, (hipStream_t)stream);
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
    if (!skinny_cols_ok(W->cols) || !skinny_cols_ok(W->rows)) return QLORA_E_UNSUPPORTED;
  } else {
    if (dA || dB) return QLORA_E_SHAPE;  // no adapter, no adapter gradients
  }
  const bool staged = dX && staged_bwd_ok(M, W->rows, W->cols) &&
                      ws_bytes >= bwd_layout(M, W->rows, W->cols, r, true).total;
  const BwdLayout L = bwd_layout(M, W->rows, W->cols, r, staged);
  if (ws_bytes < L.total) return QLORA_E_WORKSPACE;
  if (L.total > 0 && !ws) return QLORA_E_NULL;
  if (L.total > 0 && !aligned16(ws)) return QLORA_E_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  const Nf4View v = view(W);
  const int64_t N = W->rows, K = W->cols;
  bf16_t* WdT = staged ? reinterpret_cast<bf16_t*>(ws_at(ws, L.wdt)) : nullptr;
  auto dequant_t = [&]() -> qlora_status {
    return hip_status(
        launch_dequant_t(W->codes, W->absmax_q, W->group_scale, N, K, W->codebook, W->absmax_format, WdT, N, s));
  };
  // dX = dY deq(W) + s G A: the dense kernel on deq(W)^T, or the fused one
  auto run_dx = [&](const bf16_t* G, float sc) -> qlora_status {
    if (!staged) return hip_status(launch_dx(v, dY, M, G, r > 0 ? A : nullptr, r, sc, dX, s));
    return hip_status(launch_bf16_fwd(WdT, K, N, dY, M, G, r > 0 ? A : nullptr, true, r, sc, dX, s,
                                      reinterpret_cast<float*>(ws_at(ws, L.split)), L.split_bytes));
  };
  if (r == 0) {
    if (!dX) return QLORA_OK;
    if (staged && (st = dequant_t()) != QLORA_OK) return st;
    return run_dx(nullptr, 0.0f);
  }
  const bool g_late = staged && dy_late(M, N);
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
  if (staged && g_late && (st = dequant_t()) != QLORA_OK) return st;
  st = hip_status(launch_dyb(dY, B, M, N, r, part, G, 1.0f, s));
  if (st != QLORA_OK) return st;
  if (dX) {
    if (staged && !g_late && (st = dequant_t()) != QLORA_OK) return st;
    st = run_dx(G, sc);
    if (st != QLORA_OK) return st;
  }
  return hip_status(launch_grads(G, X, dY, N, U, r, M, N, K, r, 1, part, dA, dB, sc, s));
}

namespace {

// A group's weights: G >= 1 descriptors of one GEMM-path shape.
qlora_status check_group_weights(const qlora_nf4_weight* W, int32_t G) {
  if (!W) return QLORA_E_NULL;
  if (G < 1) return QLORA_E_SHAPE;
  for (int32_t g = 0; g < G; ++g) {
    qlora_status st = check_gemm_weight(&W[g]);
    if (st != QLORA_OK) return st;
    if (W[g].rows != W[0].rows || W[g].cols != W[0].cols) return QLORA_E_SHAPE;
  }
  return QLORA_OK;
}

// Sizes of a group's products: N % 64 == 0 and K % 64 == 0, G r <= 256, and
// the stack, X and dY addressed with 32-bit byte offsets (G N K, M K and
// M G N below 2^31).
qlora_status check_group_shape(int64_t M, int64_t N, int64_t K, int32_t r, int32_t G) {
  if (G < 1 || M <= 0 || M > 0x7FFFFFFF || N <= 0 || K <= 0) return QLORA_E_SHAPE;
  if (r < 0 || r % 8 != 0 || r > kMaxRank || (int64_t)G * r > kMaxGroupRank) return QLORA_E_UNSUPPORTED;
  if (N % 64 != 0 || K % 64 != 0) return QLORA_E_UNSUPPORTED;
  const int64_t NG = (int64_t)G * N;
  if (NG > (int64_t)0x7FFFFFFF / K || M > (int64_t)0x7FFFFFFF / K || M > (int64_t)0x7FFFFFFF / NG)
    return QLORA_E_UNSUPPORTED;
  if (r > 0 && (!skinny_cols_ok(K) || !skinny_cols_ok(NG))) return QLORA_E_UNSUPPORTED;
  return QLORA_OK;
}

// deq(W_g) into rows g N .. of the stack, or deq(W_g)^T into columns g N ..;
// consecutive weights with the same codebook and absmax format (up to
// kDeqMax of them) share one launch.
qlora_status group_dequant(const qlora_nf4_weight* W, int32_t G, bool transposed, bf16_t* out, hipStream_t s) {
  const int64_t N = W[0].rows, K = W[0].cols;
  for (int32_t g = 0; g < G;) {
    DeqSrcs src{};
    int n = 0;
    while (g + n < G && n < kDeqMax && W[g + n].codebook == W[g].codebook &&
           W[g + n].absmax_format == W[g].absmax_format) {
      src.codes[n] = W[g + n].codes;
      src.absmax_q[n] = W[g + n].absmax_q;
      src.group_scale[n] = W[g + n].group_scale;
      ++n;
    }
    hipError_t e = transposed ? launch_dequant_group(src, n, N, K, W[g].codebook, W[g].absmax_format, true,
                                                     out + g * N, (int64_t)G * N, N, s)
                              : launch_dequant_group(src, n, N, K, W[g].codebook, W[g].absmax_format, false,
                                                     out + g * N * K, 0, N * K, s);
    if (e != hipSuccess) return hip_status(e);
    g += n;
  }
  return QLORA_OK;
}

float lora_s(float alpha, int32_t r) { return r > 0 ? (float)((double)alpha / (double)r) : 0.0f; }

// The group's products on validated arguments (the building blocks below
// and the two group calls share them).
qlora_status group_fwd_product(const bf16_t* Wd, int32_t G, int64_t N, int64_t K, const bf16_t* X, int64_t M,
                               const bf16_t* U, const bf16_t* B, int32_t r, float alpha, bf16_t* Y, hipStream_t s) {
  return hip_status(launch_bf16_group(Wd, (int64_t)G * N, K, X, M, r > 0 ? U : nullptr, G * r, r > 0 ? B : nullptr,
                                      false, r, N, lora_s(alpha, r), Y, s));
}
// dX = sum_g dY_g deq(W_g) + s sum_g G_g A_g: one dense product contracting
// over the G N columns of dY, with the stacked adapters as a rank-G r tail
qlora_status group_dx_product(const bf16_t* WdT, int32_t G, int64_t N, int64_t K, const bf16_t* dY, int64_t M,
                              const bf16_t* Gm, const bf16_t* A, int32_t r, float alpha, bf16_t* dX, hipStream_t s,
                              float* split, size_t split_bytes) {
  return hip_status(launch_bf16_group(WdT, K, (int64_t)G * N, dY, M, r > 0 ? Gm : nullptr, G * r,
                                      r > 0 ? A : nullptr, true, G * r, K, lora_s(alpha, r), dX, s, split,
                                      split_bytes));
}
qlora_status group_grads(const bf16_t* X, const bf16_t* dY, const bf16_t* U, const bf16_t* Gm, int64_t M, int64_t N,
                         int64_t K, int32_t r, int32_t G, float alpha, float* dA, float* dB, float* part,
                         hipStream_t s) {
  const float sc = lora_s(alpha, r);
  // dA [G r x K] = s G^T X in one pass over X; dB_g = s dY_g^T U_g
  return hip_status(launch_grads(Gm, X, dY, (int64_t)G * N, U, G * r, M, N, K, r, G, part, dA, dB, sc, s));
}

}  // namespace

qlora_status qlora_group_fwd(const qlora_nf4_weight* W, int32_t G, const uint16_t* X, int64_t M,
                             const uint16_t* A, const uint16_t* B, int32_t r, float alpha, uint16_t* Y,
                             uint16_t* U_save, void* ws, size_t ws_bytes, void* stream) {
  qlora_status st = check_group_weights(W, G);
  if (st != QLORA_OK) return st;
  if ((st = check_rank(r, A, B)) != QLORA_OK) return st;
  const int64_t N = W[0].rows, K = W[0].cols;
  if ((st = check_group_shape(M, N, K, r, G)) != QLORA_OK) return st;
  if (!X || !Y) return QLORA_E_NULL;
  if (!aligned16(X) || !aligned16(Y) || (U_save && !aligned16(U_save))) return QLORA_E_ALIGN;
  const FwdLayout L = group_fwd_layout(M, N, K, r, G);
  if ((st = check_ws(ws, ws_bytes, L.total)) != QLORA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  bf16_t* U = nullptr;
  if (r > 0) {
    U = U_save ? U_save : reinterpret_cast<bf16_t*>(ws_at(ws, L.u));
    // every adapter's U in one pass over X: U [M x G r] = X [A_0; A_1; ..]^T
    st = hip_status(launch_xat(X, A, M, K, G * r, reinterpret_cast<float*>(ws_at(ws, L.part)), U, nullptr, 1.0f, s));
    if (st != QLORA_OK) return st;
  }
  bf16_t* Wd = reinterpret_cast<bf16_t*>(ws_at(ws, L.wd));
  if ((st = group_dequant(W, G, false, Wd, s)) != QLORA_OK) return st;
  return group_fwd_product(Wd, G, N, K, X, M, U, B, r, alpha, Y, s);
}

qlora_status qlora_group_bwd(const qlora_nf4_weight* W, int32_t G, const uint16_t* X, const uint16_t* dY,
                             int64_t M, const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                             const uint16_t* U_saved, uint16_t* dX, float* dA, float* dB, void* ws,
                             size_t ws_bytes, void* stream) {
  qlora_status st = check_group_weights(W, G);
  if (st != QLORA_OK) return st;
  if ((st = check_rank(r, A, B)) != QLORA_OK) return st;
  const int64_t N = W[0].rows, K = W[0].cols, NG = (int64_t)G * N;
  if ((st = check_group_shape(M, N, K, r, G)) != QLORA_OK) return st;
  if (!dY) return QLORA_E_NULL;
  if (!aligned16(dY) || (dX && !aligned16(dX)) || (U_saved && !aligned16(U_saved))) return QLORA_E_ALIGN;
  if (r > 0) {
    if (!dA || !dB || !X) return QLORA_E_NULL;
    if (!aligned16(dA) || !aligned16(dB) || !aligned16(X)) return QLORA_E_ALIGN;
  } else if (dA || dB) {
    return QLORA_E_SHAPE;   // no adapter, no adapter gradients
  }
  const BwdLayout L = group_bwd_layout(M, N, K, r, G, dX != nullptr);
  if ((st = check_ws(ws, ws_bytes, L.total)) != QLORA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  bf16_t* WdT = dX ? reinterpret_cast<bf16_t*>(ws_at(ws, L.wdt)) : nullptr;
  if (r == 0) {
    if (!dX) return QLORA_OK;
    if ((st = group_dequant(W, G, true, WdT, s)) != QLORA_OK) return st;
    return group_dx_product(WdT, G, N, K, dY, M, nullptr, nullptr, 0, alpha, dX, s,
                            reinterpret_cast<float*>(ws_at(ws, L.split)), L.split_bytes);
  }
  bf16_t* Gm = reinterpret_cast<bf16_t*>(ws_at(ws, L.g));
  float* part = reinterpret_cast<float*>(ws_at(ws, L.part));
  const bf16_t* U = U_saved;
  if (!U) {
    bf16_t* Ud = reinterpret_cast<bf16_t*>(ws_at(ws, L.u));
    if ((st = hip_status(launch_xat(X, A, M, K, G * r, part, Ud, nullptr, 1.0f, s))) != QLORA_OK) return st;
    U = Ud;
  }
  // G [M x G r]: group g is dY_g B_g
  const bool g_late = dX && dy_late(M, NG);
  if (g_late && (st = group_dequant(W, G, true, WdT, s)) != QLORA_OK) return st;
  if ((st = hip_status(launch_dyb_group(dY, NG, B, M, N, r, G, part, Gm, 1.0f, s))) != QLORA_OK) return st;
  if (dX) {
    if (!g_late && (st = group_dequant(W, G, true, WdT, s)) != QLORA_OK) return st;
    if ((st = group_dx_product(WdT, G, N, K, dY, M, Gm, A, r, alpha, dX, s,
                               reinterpret_cast<float*>(ws_at(ws, L.split)), L.split_bytes)) != QLORA_OK)
      return st;
  }
  return group_grads(X, dY, U, Gm, M, N, K, r, G, alpha, dA, dB, part, s);
}

qlora_status qlora_group_dequant(const qlora_nf4_weight* W, int32_t G, uint16_t* Wd_out, void* stream) {
  qlora_status st = check_group_weights(W, G);
  if (st != QLORA_OK) return st;
  if (!Wd_out) return QLORA_E_NULL;
  if (!aligned16(Wd_out)) return QLORA_E_ALIGN;
  return group_dequant(W, G, false, Wd_out, (hipStream_t)stream);
}

qlora_status qlora_group_dequant_t(const qlora_nf4_weight* W, int32_t G, uint16_t* WdT_out, void* stream) {
  qlora_status st = check_group_weights(W, G);
  if (st != QLORA_OK) return st;
  if (!WdT_out) return QLORA_E_NULL;
  if (!aligned16(WdT_out)) return QLORA_E_ALIGN;
  // the transposing grid has ceil(N / 64) rows; rows of the result are G N apart
  if ((W[0].rows + 63) / 64 > 65535 || W[0].cols / 64 > 0x7FFFFFFF) return QLORA_E_UNSUPPORTED;
  return group_dequant(W, G, true, WdT_out, (hipStream_t)stream);
}

qlora_status qlora_bf16_group_fwd(const uint16_t* Wd, int32_t G, int64_t N, int64_t K, const uint16_t* X, int64_t M,
                                  const uint16_t* U, const uint16_t* B, int32_t r, float alpha, uint16_t* Y,
                                  void* stream) {
  qlora_status st = check_group_shape(M, N, K, r, G);
  if (st != QLORA_OK) return st;
  if (!Wd || !X || !Y) return QLORA_E_NULL;
  if (!aligned16(Wd) || !aligned16(X) || !aligned16(Y)) return QLORA_E_ALIGN;
  if ((st = check_rank(r, U, B)) != QLORA_OK) return st;
  return group_fwd_product(Wd, G, N, K, X, M, U, B, r, alpha, Y, (hipStream_t)stream);
}

qlora_status qlora_bf16_group_dx(const uint16_t* WdT, int32_t G, int64_t N, int64_t K, const uint16_t* dY,
                                 int64_t M, const uint16_t* Gm, const uint16_t* A, int32_t r, float alpha,
                                 uint16_t* dX, void* ws, size_t ws_bytes, void* stream) {
  qlora_status st = check_group_shape(M, N, K, r, G);
  if (st != QLORA_OK) return st;
  if (!WdT || !dY || !dX) return QLORA_E_NULL;
  if (!aligned16(WdT) || !aligned16(dY) || !aligned16(dX) || (ws && !aligned16(ws))) return QLORA_E_ALIGN;
  if ((st = check_rank(r, Gm, A)) != QLORA_OK) return st;
  return group_dx_product(WdT, G, N, K, dY, M, Gm, A, r, alpha, dX, (hipStream_t)stream, static_cast<float*>(ws),
                          ws ? ws_bytes : 0);
}

qlora_status qlora_group_lora_dy_b(const uint16_t* dY, const uint16_t* B, int64_t M, int64_t N, int32_t r,
                                   int32_t G, uint16_t* Gm, void* ws, size_t ws_bytes, void* stream) {
  qlora_status st = check_adapter_rank(r);
  if (st != QLORA_OK) return st;
  if (G < 1 || M <= 0 || M > 0x7FFFFFFF || N <= 0 || N % 8 != 0) return QLORA_E_SHAPE;
  if ((int64_t)G * r > kMaxGroupRank || !skinny_cols_ok((int64_t)G * N)) return QLORA_E_UNSUPPORTED;
  if (!dY || !B || !Gm) return QLORA_E_NULL;
  if (!aligned16(dY) || !aligned16(B) || !aligned16(Gm)) return QLORA_E_ALIGN;
  if ((st = check_ws(ws, ws_bytes, align_up(skinny_partial_bytes(M, G * r, N, kDyB)))) != QLORA_OK) return st;
  return hip_status(launch_dyb_group(dY, (int64_t)G * N, B, M, N, r, G, static_cast<float*>(ws), Gm, 1.0f,
                                     (hipStream_t)stream));
}

qlora_status qlora_group_lora_grads(const uint16_t* X, const uint16_t* dY, const uint16_t* U, const uint16_t* Gm,
                                    int64_t M, int64_t N, int64_t K, int32_t r, int32_t G, float alpha, float* dA,
                                    float* dB, void* ws, size_t ws_bytes, void* stream) {
  qlora_status st = check_adapter_rank(r);
  if (st != QLORA_OK) return st;
  if (G < 1 || M <= 0 || M > 0x7FFFFFFF || N <= 0 || N % 8 != 0 || K <= 0 || K % 8 != 0) return QLORA_E_SHAPE;
  const int64_t NG = (int64_t)G * N;
  if ((int64_t)G * r > kMaxGroupRank) return QLORA_E_UNSUPPORTED;
  // X and dY are addressed with 32-bit byte offsets
  if (M > (int64_t)0x7FFFFFFF / K || M > (int64_t)0x7FFFFFFF / NG) return QLORA_E_UNSUPPORTED;
  if (!X || !dY || !U || !Gm || !dA || !dB) return QLORA_E_NULL;
  if (!aligned16(X) || !aligned16(dY) || !aligned16(U) || !aligned16(Gm) || !aligned16(dA) || !aligned16(dB))
    return QLORA_E_ALIGN;
  const size_t need = align_up(grads_partial_bytes(M, N, K, r, G));
  if ((st = check_ws(ws, ws_bytes, need)) != QLORA_OK) return st;
  return group_grads(X, dY, U, Gm, M, N, K, r, G, alpha, dA, dB, static_cast<float*>(ws), (hipStream_t)stream);
}

qlora_status qlora_lora_down(const uint16_t* X, const uint16_t* A, int64_t M, int64_t K, int32_t r, uint16_t* U,
                             void* ws, size_t ws_bytes, void* stream) {
  // up to kMaxGroupRank: a group's stacked adapters
  if (r <= 0 || r > kMaxGroupRank || r % 8 != 0) return QLORA_E_UNSUPPORTED;
  qlora_status st = QLORA_OK;
  if (M <= 0 || M > 0x7FFFFFFF || K <= 0 || K % 8 != 0) return QLORA_E_SHAPE;
  if (!skinny_cols_ok(K)) return QLORA_E_UNSUPPORTED;
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
  if (!skinny_cols_ok(N)) return QLORA_E_UNSUPPORTED;
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
  const size_t need = align_up(grads_partial_bytes(M, N, K, r, 1));
  if ((st = check_ws(ws, ws_bytes, need)) != QLORA_OK) return st;
  const float sc = (float)((double)alpha / (double)r);
  hipStream_t s = (hipStream_t)stream;
  return hip_status(launch_grads(G, X, dY, N, U, r, M, N, K, r, 1, static_cast<float*>(ws), dA, dB, sc, s));
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

qlora_status qlora_bf16_fwd(const uint16_t* Wd, int64_t N, int64_t K, const uint16_t* X, int64_t M,
                            const uint16_t* U, const uint16_t* B, int32_t r, float alpha, uint16_t* Y,
                            void* stream) {
  if (N <= 0 || K <= 0 || M <= 0) return QLORA_E_SHAPE;
  if (K % 64 != 0 || N % 8 != 0) return QLORA_E_UNSUPPORTED;
  // Wd, X and Y are addressed with 32-bit byte offsets
  if (N > (int64_t)0x7FFFFFFF / K || M > (int64_t)0x7FFFFFFF / K || M > (int64_t)0x7FFFFFFF / N)
    return QLORA_E_UNSUPPORTED;
  if (!Wd || !X || !Y) return QLORA_E_NULL;
  if (!aligned16(Wd) || !aligned16(X) || !aligned16(Y)) return QLORA_E_ALIGN;
  qlora_status st = check_rank(r, U, B);
  if (st != QLORA_OK) return st;
  const float sc = r > 0 ? (float)((double)alpha / (double)r) : 0.0f;
  return hip_status(launch_bf16_fwd(Wd, N, K, X, M, r > 0 ? U : nullptr, r > 0 ? B : nullptr, false, r, sc, Y,
                                    (hipStream_t)stream));
}

qlora_status qlora_bf16_dx(const uint16_t* WdT, int64_t N, int64_t K, const uint16_t* dY, int64_t M,
                           const uint16_t* G, const uint16_t* A, int32_t r, float alpha, uint16_t* dX,
                           void* ws, size_t ws_bytes, void* stream) {
  if (N <= 0 || K <= 0 || M <= 0) return QLORA_E_SHAPE;
  if (K % 64 != 0 || N % 64 != 0) return QLORA_E_UNSUPPORTED;
  if (N > (int64_t)0x7FFFFFFF / K || M > (int64_t)0x7FFFFFFF / K || M > (int64_t)0x7FFFFFFF / N)
    return QLORA_E_UNSUPPORTED;
  if (!WdT || !dY || !dX) return QLORA_E_NULL;
  if (!aligned16(WdT) || !aligned16(dY) || !aligned16(dX) || (ws && !aligned16(ws))) return QLORA_E_ALIGN;
  qlora_status st = check_rank(r, G, A);
  if (st != QLORA_OK) return st;
  const float sc = r > 0 ? (float)((double)alpha / (double)r) : 0.0f;
  // dX [M x K] = dY [M x N] (WdT [K x N])^T + s G (A^T)^T
  return hip_status(launch_bf16_fwd(WdT, K, N, dY, M, r > 0 ? G : nullptr, r > 0 ? A : nullptr, true, r, sc, dX,
                                    (hipStream_t)stream, static_cast<float*>(ws), ws ? ws_bytes : 0));
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
    // one codebook and second-level format per call: the kernel builds its
    // decode tables once
    if (J.W->codebook != jobs[0].W->codebook || J.W->absmax_format != jobs[0].W->absmax_format)
      return QLORA_E_UNSUPPORTED;
    if (J.W->cols % 64 != 0 || J.W->cols > kMaxGemvCols || J.W->rows > 0x7FFFFFFF) return QLORA_E_UNSUPPORTED;
    // codes addressed with 32-bit byte offsets, including the prefetch of
    // up to one row and 1 KiB past the last row
    if (J.W->rows + 1 > ((int64_t)0xFFFFFFFF - 1024) / (J.W->cols / 2)) return QLORA_E_UNSUPPORTED;
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
      gemv_prepare(buf.data(), njobs, jobs[0].W->codebook | (jobs[0].W->absmax_format << 8), ws_at(ws, u_bytes),
                   table_bytes, &L, (hipStream_t)stream));
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
