/*
 * qlora.h -- C ABI of libqlora: the frozen NF4 linear layer with
 * double-quantized block constants and a trainable bf16 LoRA adapter, on
 * one AMD Instinct MI355X (gfx950).
 *
 * What the operations compute comes from the QLoRA pages:
 *   - glossary page "QLoRA" (mangrove.ai), section "Definition": frozen
 *     pretrained weights stored as 4-bit NormalFloat (NF4) numbers, converted
 *     back to BFloat16 each time a layer is used; LoRA matrices trained in
 *     16-bit; weight gradients only for the LoRA matrices; double
 *     quantization of the scaling constants;
 *   - deepfa.ir blog "QLoRA: Fine-Tuning 65-Billion Parameter Models on a
 *     Single Consumer GPU", sections "LoRA: Prerequisite", "1. 4-bit
 *     NormalFloat (NF4)", "2. Double Quantization", "QLoRA's Working Process";
 *   - whatthefuture.ai "One GPU, 24 hours...", closing paragraphs: 4-bit
 *     inference (batch-1 decode) is slow and is to be sped up.
 *
 * Storage format (fixed by this library; the pages give none):
 *   - W is [rows x cols] (out x in), row-major.  A block is 64 consecutive
 *     elements of the flattened W; a group is 256 consecutive blocks.
 *   - codes: ceil(rows*cols/2) bytes.  Element 2j is the low nibble of byte
 *     j, element 2j+1 the high nibble.  A code indexes the ascending NF4
 *     table (0 = -1, 7 = 0, 15 = +1).
 *   - absmax_q: one byte per block, the index of the nearest level of
 *     Q8[k] = RN32(k/255) to RN32(absmax_b / s2_g) (ties to the lower index).
 *   - group_scale: one fp32 per group, s2_g = largest block absmax.
 *   - Dequantized value: RNE_bf16(RN32(L[c] * RN32(Q8[q] * s2))).
 *
 * Conventions for every call:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  bf16
 *     tensors travel as uint16_t bit patterns; all are row-major, contiguous.
 *   - The library never allocates or frees memory and never synchronizes.
 *     Scratch memory is the caller's `ws` buffer, sized by
 *     qlora_workspace_bytes().
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the
 *     default stream).  Device-side faults surface at the caller's next
 *     synchronization.
 *   - All argument checks happen before any launch: a status other than
 *     QLORA_OK means nothing was enqueued.
 *   - The library keeps no mutable global state and is thread-safe; two
 *     calls that share an output or workspace buffer must be ordered by the
 *     caller (same stream, or events).
 *   - Alignment: codes, X, dY, Y, dX, A, B, U, x, y and ws must be 16-byte
 *     aligned (QLORA_E_ALIGN otherwise).
 */
#ifndef QLORA_H
#define QLORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QLORA_OK = 0,
  QLORA_E_NULL = 1,        /* a required pointer is NULL                     */
  QLORA_E_ALIGN = 2,       /* a pointer is not 16-byte aligned               */
  QLORA_E_SHAPE = 3,       /* a size is not positive, or sizes disagree      */
  QLORA_E_UNSUPPORTED = 4, /* blocksize != 64, group != 256, cols % 64 != 0
                              on the GEMM/GEMV paths, rows % 8 != 0 or
                              rows*cols/2 >= 2^32 on the GEMM paths, M*rows
                              or M*cols >= 2^31 on the fused GEMMs, r
                              outside [0,128] or r % 8 != 0, too many jobs,
                              an unknown codebook, GEMV jobs of different
                              codebooks in one call */
  QLORA_E_WORKSPACE = 5,   /* ws_bytes smaller than qlora_workspace_bytes()  */
  QLORA_E_HIP = 6          /* a HIP launch/copy error; see qlora_last_hip_error */
} qlora_status;

typedef enum {
  QLORA_OP_FWD = 0,   /* qlora_linear_fwd                                   */
  QLORA_OP_BWD = 1,   /* qlora_linear_bwd                                   */
  QLORA_OP_GEMV = 2,  /* qlora_gemv                                         */
  QLORA_OP_LORA = 3   /* qlora_lora_down, qlora_lora_dy_b, qlora_lora_grads */
} qlora_op;

/* A quantized weight: host struct holding device pointers.
 * codes: ceil(rows*cols/2) bytes; absmax_q: nb bytes; group_scale: ng fp32,
 * with nb = ceil(rows*cols/64), ng = ceil(nb/256). */
/* 4-bit codebooks.  The pages compare NF4 with FP4 and Int4 and report that
 * NF4 has the lower quantization error (deepfa.ir blog, "1. 4-bit
 * NormalFloat (NF4)" and its results list).  FP4 is E2M1 (sign, two exponent
 * bits with bias 1, one mantissa bit) divided by its largest value 6; its
 * two zeros are both +0 (codes 7 and 8, and code 8 is never produced).
 * Int4 is k/7 for the two's-complement k = -8..7 (code 0, -8/7, is never
 * produced from absmax-normalised values).  All three are quantized the
 * same way: blockwise absmax, nearest level with ties to the lower index,
 * 8-bit double quantization; an all-zero block stores the code of the
 * level 0 (7 for NF4 and FP4, 8 for Int4).  A weight descriptor names its
 * codebook, and every call that reads or writes the weight uses it. */
typedef enum {
  QLORA_CODEBOOK_NF4 = 0,
  QLORA_CODEBOOK_FP4 = 1,
  QLORA_CODEBOOK_INT4 = 2
} qlora_codebook;

typedef struct {
  int64_t rows;           /* N, output features                       */
  int64_t cols;           /* K, input features                        */
  int32_t blocksize;      /* must be 64                               */
  int32_t group_blocks;   /* must be 256                              */
  uint8_t* codes;
  uint8_t* absmax_q;
  float* group_scale;
  int32_t codebook;       /* qlora_codebook of the 4-bit codes (0 = NF4) */
} qlora_nf4_weight;

/* One batch-1 decode product y = deq(W) x + (alpha/r) B (A x). */
typedef struct {
  const qlora_nf4_weight* W;  /* host pointer to the descriptor            */
  const uint16_t* x;          /* [m x cols] bf16 ([cols] for one token)    */
  const uint16_t* A;          /* [r x cols] bf16, NULL when r == 0         */
  const uint16_t* B;          /* [rows x r] bf16, NULL when r == 0         */
  int32_t r;
  float alpha;
  uint16_t* y;                /* [m x rows] bf16, overwritten              */
  int32_t m;                  /* tokens: 0 or 1 for one, at most 16        */
} qlora_gemv_job;

/* Name of a status code (static string). */
const char* qlora_status_str(qlora_status s);

/* The hipError_t of the last QLORA_E_HIP returned on this thread. */
int qlora_last_hip_error(void);

/* Library version, e.g. "0.1.0". */
const char* qlora_version(void);

/* The library's NF4 table: 16 fp32 levels, ascending (host memory).
 * deepfa.ir blog, "1. 4-bit NormalFloat (NF4)": 16 levels from normal
 * quantiles with equal probability per bucket, normalised to [-1, 1],
 * with an exact zero. */
void qlora_nf4_levels(float out[16]);

/* Host-only size arithmetic for a rows x cols weight.  Any output pointer
 * may be NULL.  Returns QLORA_E_SHAPE for non-positive sizes and
 * QLORA_E_UNSUPPORTED for blocksize != 64 or group_blocks != 256. */
qlora_status qlora_sizes(int64_t rows, int64_t cols, int32_t blocksize, int32_t group_blocks,
                         size_t* codes_bytes, size_t* absmax_q_bytes, size_t* scale_bytes);

/* Bytes of scratch the given call needs (0 when none).  FWD/BWD: M tokens,
 * N = rows, K = cols, LoRA rank r; GEMV: njobs jobs, with N and K the
 * largest rows/cols among them; LORA: the split-contraction partial sums of
 * the LoRA side products of one M x N x K, rank-r layer.  Returns 0 for
 * invalid sizes. */
size_t qlora_workspace_bytes(qlora_op op, int64_t M, int64_t N, int64_t K, int32_t r, int32_t njobs);

/* Quantize bf16 W [rows x cols] into q (codes, absmax_q, group_scale are
 * overwritten) with the levels of q->codebook.  Any rows*cols >= 1 (ragged
 * last block and group allowed).
 * Glossary "Definition" and deepfa.ir "1. NF4" / "2. Double Quantization". */
qlora_status qlora_quantize(const uint16_t* W, const qlora_nf4_weight* q, void* stream);

/* Dequantize q into bf16 W_out [rows x cols] (overwritten).
 * Glossary "Definition": converted back to BFloat16 for the calculation. */
qlora_status qlora_dequant(const qlora_nf4_weight* q, uint16_t* W_out, void* stream);

/* One AdamW step on n trainable values (the LoRA matrices after a backward
 * pass; the pages' paged optimizers keep such states movable between GPU
 * and CPU memory: glossary "Definition", deepfa.ir "3. Paged Optimizers").
 * p [n] fp32 master values, grad [n] fp32 (dA or dB), m and v [n] fp32
 * moments, all updated in place; p_bf16 [n] (nullable) receives the bf16
 * copy the layer reads (round to nearest even).  For step >= 1:
 *   m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2;
 *   p = p - lr ((m / (1 - b1^step)) / (sqrt(v / (1 - b2^step)) + eps) + wd p).
 * Any pointer may be device memory or pinned host memory (hipHostMalloc):
 * the kernel reads and writes host memory in place over the host link.
 * Pointers 16-byte aligned, n >= 1, 0 <= beta < 1, eps > 0, step >= 1;
 * QLORA_E_NULL / _ALIGN / _SHAPE otherwise. */
qlora_status qlora_adamw(float* p, uint16_t* p_bf16, const float* grad, float* m, float* v, int64_t n,
                         float lr, float beta1, float beta2, float eps, float weight_decay, int32_t step,
                         void* stream);

/* The 16 fp32 levels of a codebook, ascending, as the device tables hold
 * them.  QLORA_E_NULL for a NULL out, QLORA_E_UNSUPPORTED for an unknown
 * codebook. */
qlora_status qlora_codebook_levels(qlora_codebook cb, float out[16]);

/* Forward: Y [M x N] = X deq(W)^T + s (X A^T) B^T, s = RN32(alpha / r).
 * X [M x K], A [r x K], B [N x r], Y bf16 (overwritten).  r == 0 (A = B =
 * NULL) gives the frozen layer alone.  U_save (nullable) receives
 * U = X A^T [M x r] in bf16 for the backward pass.  Requires K % 64 == 0.
 * deepfa.ir "LoRA: Prerequisite" and "QLoRA's Working Process". */
qlora_status qlora_linear_fwd(const qlora_nf4_weight* W, const uint16_t* X, int64_t M,
                              const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                              uint16_t* Y, uint16_t* U_save,
                              void* ws, size_t ws_bytes, void* stream);

/* Backward: dX [M x K] = dY deq(W) + s (dY B) A (bf16, overwritten; NULL
 * skips it); dA [r x K] = s (dY B)^T X and dB [N x r] = s dY^T (X A^T)
 * (fp32, overwritten, not accumulated).  No gradient for the frozen W.
 * U_saved (nullable) is X A^T from the forward pass; when NULL it is
 * recomputed.  When r == 0, dA and dB must be NULL.  Requires K % 64 == 0.
 * Glossary "Definition" (weight gradients only for the LoRA matrices);
 * insights4ai page (gradients backpropagated through the frozen 4-bit
 * model into the adapters). */
qlora_status qlora_linear_bwd(const qlora_nf4_weight* W, const uint16_t* X, const uint16_t* dY,
                              int64_t M, const uint16_t* A, const uint16_t* B, int32_t r,
                              float alpha, const uint16_t* U_saved, uint16_t* dX,
                              float* dA, float* dB, void* ws, size_t ws_bytes, void* stream);

/* ---- Building blocks of the forward and backward passes ----------------
 * qlora_linear_fwd = qlora_lora_down + qlora_nf4_fwd;
 * qlora_linear_bwd = [qlora_lora_down] + qlora_lora_dy_b + qlora_nf4_dx
 *                    + qlora_lora_grads.
 * They let a caller keep U and G, reuse them, or time the two fused NF4
 * GEMMs on their own.  Same conventions as above; ws is sized by
 * qlora_workspace_bytes(QLORA_OP_LORA, M, N, K, r, 0). */

/* U [M x r] = X A^T (bf16).  deepfa.ir "LoRA: Prerequisite": the adapter's
 * down-projection.  r in (0, 128], r % 8 == 0, K % 8 == 0. */
qlora_status qlora_lora_down(const uint16_t* X, const uint16_t* A, int64_t M, int64_t K, int32_t r,
                             uint16_t* U, void* ws, size_t ws_bytes, void* stream);

/* G [M x r] = dY B (bf16): the gradient reaching the adapter's
 * down-projection output.  N % 8 == 0. */
qlora_status qlora_lora_dy_b(const uint16_t* dY, const uint16_t* B, int64_t M, int64_t N, int32_t r,
                             uint16_t* G, void* ws, size_t ws_bytes, void* stream);

/* dA [r x K] = s G^T X and dB [N x r] = s dY^T U (fp32, overwritten),
 * s = RN32(alpha / r).  M*K and M*N must be < 2^31 (QLORA_E_UNSUPPORTED
 * otherwise).  Glossary "Definition": weight gradients only for the LoRA
 * matrices. */
qlora_status qlora_lora_grads(const uint16_t* X, const uint16_t* dY, const uint16_t* U, const uint16_t* G,
                              int64_t M, int64_t N, int64_t K, int32_t r, float alpha, float* dA, float* dB,
                              void* ws, size_t ws_bytes, void* stream);

/* The fused forward GEMM: Y = X deq(W)^T + s U B^T, with U = X A^T given
 * (r == 0: U = B = NULL).  No workspace.  deepfa.ir "QLoRA's Working
 * Process": dequantization to BF16 on the fly inside the product. */
qlora_status qlora_nf4_fwd(const qlora_nf4_weight* W, const uint16_t* X, int64_t M, const uint16_t* U,
                           const uint16_t* B, int32_t r, float alpha, uint16_t* Y, void* stream);

/* The fused backward GEMM: dX = dY deq(W) + s G A, with G = dY B given
 * (r == 0: G = A = NULL).  No workspace.  insights4ai page: gradients flow
 * through the frozen 4-bit weights. */
qlora_status qlora_nf4_dx(const qlora_nf4_weight* W, const uint16_t* dY, int64_t M, const uint16_t* G,
                          const uint16_t* A, int32_t r, float alpha, uint16_t* dX, void* stream);

/* Decode for njobs independent products (host job array, read before
 * return): for each of the job's m tokens (rows of x and y),
 * y = deq(W) x + s B (A x), s = RN32(alpha / r), y bf16 (overwritten); the
 * forward product at a batch of m <= 16 tokens.  Each job needs
 * cols % 64 == 0 and cols <= 32768, and rows * r * 2 < 2^32.
 * njobs <= 4096.  A job's m may be 0 or 1 (one token, x [cols], y [rows])
 * up to 16 (x [m x cols], y [m x rows]); m < 0 is QLORA_E_SHAPE, m > 16
 * QLORA_E_UNSUPPORTED.  ws is sized by qlora_workspace_bytes(QLORA_OP_GEMV,
 * largest m (0 or 1 for one token), max rows, max cols, 0, njobs); it holds
 * u = A x and the job table, which the call writes with an asynchronous
 * host-to-device copy on `stream`.  Equivalent to qlora_gemv_prepare
 * followed by qlora_gemv_run.
 * whatthefuture.ai article: 4-bit inference is slow (the 8-16x speed-up
 * its authors expected). */
qlora_status qlora_gemv(const qlora_gemv_job* jobs, int32_t njobs, void* ws, size_t ws_bytes,
                        void* stream);

/* A prepared decode call, for callers that repeat the same jobs (a decode
 * loop over fixed layers and buffers).  The fields belong to the library. */
typedef struct {
  uint64_t priv[16];
} qlora_gemv_plan;

/* Validate the jobs and write their table into ws (as qlora_gemv does);
 * fill *plan.  The copy is ordered on `stream`.  Same errors as
 * qlora_gemv; nothing is enqueued on error. */
qlora_status qlora_gemv_prepare(const qlora_gemv_job* jobs, int32_t njobs, void* ws, size_t ws_bytes,
                                qlora_gemv_plan* plan, void* stream);

/* Launch a prepared decode call on `stream`.  The workspace and every
 * buffer the jobs name must still hold what they held at prepare time (the
 * inputs may have new values); a stream other than the prepare stream must
 * be ordered after it by the caller.  QLORA_E_SHAPE for a plan that
 * qlora_gemv_prepare did not fill. */
qlora_status qlora_gemv_run(const qlora_gemv_plan* plan, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_H */
