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
 *     Q8[k] = RN32(k/255) (or of the FP8 levels, see qlora_absmax_format) to
 *     RN32(absmax_b / s2_g) (ties to the lower index).
 *   - group_scale: one fp32 per group, s2_g = largest block absmax.
 *   - Dequantized value: RNE_bf16(RN32(L[c] * RN32(Q8[q] * s2))).
 *
 * Conventions for every call:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  bf16
 *     tensors travel as uint16_t bit patterns; all are row-major, contiguous.
 *   - The library never allocates or frees memory and never synchronizes.
 *     Scratch memory is the caller's `ws` buffer, sized by
 *     qlora_workspace_bytes(), except for qlora_linear_fwd_noalloc, whose
 *     scratch is a fixed array the library holds on each device.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the
 *     default stream).  Device-side faults surface at the caller's next
 *     synchronization.
 *   - All argument checks happen before any launch: a status other than
 *     QLORA_OK means nothing was enqueued.
 *   - The library is thread-safe.  Its only mutable global state is the
 *     per-device address of the scratch array of qlora_linear_fwd_noalloc,
 *     looked up once under a lock.  Two calls that share an output or
 *     workspace buffer must be ordered by the caller (same stream, or
 *     events).
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
                              or M*cols >= 2^31 on the fused GEMMs, rows
                              or cols >= 2^24 where a LoRA side product
                              runs over them, r outside [0,128] or
                              r % 8 != 0, too many jobs,
                              an unknown codebook or second-level format,
                              GEMV jobs of different codebooks or formats
                              in one call */
  QLORA_E_WORKSPACE = 5,   /* ws_bytes smaller than qlora_workspace_bytes()  */
  QLORA_E_HIP = 6,         /* a HIP launch/copy error; see qlora_last_hip_error */
  QLORA_E_FORMAT = 7,      /* not a serialized weight header: wrong magic,
                              version, header size, or a buffer too short   */
  QLORA_E_TABLE = 8        /* a serialized weight was written with level
                              tables other than this library's             */
} qlora_status;

typedef enum {
  QLORA_OP_FWD = 0,   /* qlora_linear_fwd (room for the staged path)        */
  QLORA_OP_BWD = 1,   /* qlora_linear_bwd (room for the staged path)        */
  QLORA_OP_GEMV = 2,  /* qlora_gemv                                         */
  QLORA_OP_LORA = 3,  /* qlora_lora_down, qlora_lora_dy_b, qlora_lora_grads */
  QLORA_OP_FWD_FUSED = 4,  /* qlora_linear_fwd, fused path only             */
  QLORA_OP_BWD_FUSED = 5,  /* qlora_linear_bwd, fused path only             */
  QLORA_OP_GROUP_FWD = 6,  /* qlora_group_fwd (njobs = G, the group size)   */
  QLORA_OP_GROUP_BWD = 7,  /* qlora_group_bwd (njobs = G, the group size)   */
  QLORA_OP_GROUP_LORA = 8, /* the group building blocks' side products:
                              qlora_lora_down at rank G r,
                              qlora_group_lora_dy_b, qlora_group_lora_grads
                              (njobs = G)                                    */
  QLORA_OP_BF16_DX = 9     /* the split contraction of qlora_bf16_dx
                              (njobs = 1) and qlora_bf16_group_dx (njobs = G):
                              0 for shapes that do not split                 */
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

/* Second-level format of the 8-bit block-constant codes (double
 * quantization: glossary "Definition", deepfa.ir "2. Double Quantization";
 * the pages name no format).  Both encode y = RN32(absmax_b / s2_g) as the
 * nearest level, ties to the lower index, and decode t = RN32(Q[q] * s2):
 *   LINEAR8: Q[k] = RN32(k / 255), k = 0..255;
 *   FP8:     Q[k] = RN32(e4m3(k) / 448), k = 0..126, where e4m3(k) is the
 *            value of the FP8 E4M3 bit pattern k (sign 0, 4 exponent bits
 *            with bias 7 and subnormals, 3 mantissa bits; 448 = code 126 is
 *            the largest finite value).  Relative rather than absolute steps:
 *            constants far below their group's largest keep about 3 bits of
 *            precision instead of rounding to zero. */
typedef enum {
  QLORA_ABSMAX_LINEAR8 = 0,
  QLORA_ABSMAX_FP8 = 1
} qlora_absmax_format;

typedef struct {
  int64_t rows;           /* N, output features                       */
  int64_t cols;           /* K, input features                        */
  int32_t blocksize;      /* must be 64                               */
  int32_t group_blocks;   /* must be 256                              */
  uint8_t* codes;
  uint8_t* absmax_q;
  float* group_scale;
  int32_t codebook;       /* qlora_codebook of the 4-bit codes (0 = NF4) */
  int32_t absmax_format;  /* qlora_absmax_format of absmax_q (0 = linear) */
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
 * the LoRA side products of one M x N x K, rank-r layer (r up to 256 for
 * qlora_lora_down on a group's stacked adapters).  Returns 0 for invalid
 * sizes. */
size_t qlora_workspace_bytes(qlora_op op, int64_t M, int64_t N, int64_t K, int32_t r, int32_t njobs);

/* Quantize bf16 W [rows x cols] into q (codes, absmax_q, group_scale are
 * overwritten) with the levels of q->codebook.  Any rows*cols >= 1 (ragged
 * last block and group allowed).
 * Glossary "Definition" and deepfa.ir "1. NF4" / "2. Double Quantization". */
qlora_status qlora_quantize(const uint16_t* W, const qlora_nf4_weight* q, void* stream);

/* Dequantize q into bf16 W_out [rows x cols] (overwritten).
 * Glossary "Definition": converted back to BFloat16 for the calculation. */
qlora_status qlora_dequant(const qlora_nf4_weight* q, uint16_t* W_out, void* stream);

/* Dequantize q into the transposed bf16 weight Wt_out [cols x rows]
 * (overwritten): Wt_out[k][n] = deq(W)[n][k], bit-identical to
 * qlora_dequant's values.  cols % 64 == 0, rows % 8 == 0, rows < 4194240
 * (QLORA_E_UNSUPPORTED otherwise).  The staged backward multiplies dY by it. */
qlora_status qlora_dequant_t(const qlora_nf4_weight* q, uint16_t* Wt_out, void* stream);

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

/* ---- The paged optimizer ------------------------------------------------
 * The pages' paged optimizers (glossary "Definition": they manage memory
 * spikes; deepfa.ir "3. Paged Optimizers": states move between GPU and CPU
 * memory).  The moments of every tensor live in a pinned host backing store
 * (hipHostMalloc or torch pin_memory; pageable memory works but serializes
 * the copies); the step pages them through a device buffer of the caller's
 * size:
 *   - when every tensor's moments fit, all are resident in the buffer;
 *   - otherwise two staging slots of `chunk` values are carved first and the
 *     leading tensors whose moments fit the rest are resident; the others
 *     are copied host -> device chunk by chunk on copy_stream, updated on
 *     stream, and copied back, each chunk's copy overlapping the update of
 *     the one before (events order the streams; a NULL copy_stream, or the
 *     compute stream itself, runs everything in order on `stream`).
 * Resident moments stay in the buffer between calls: pass QLORA_PAGED_LOAD
 * on the first step (and after changing the buffer) to fill them from the
 * backing store, QLORA_PAGED_STORE to write them back after the step.  The
 * layout depends only on the tensor sizes and dev_bytes. */
typedef struct {
  float* p;              /* device [n] fp32 master values, updated in place */
  uint16_t* p_bf16;      /* device [n] bf16 copy of p (nullable)             */
  const float* grad;     /* device [n] fp32 gradient                         */
  float* m;              /* host [n] backing store of the first moment       */
  float* v;              /* host [n] backing store of the second moment      */
  int64_t n;
} qlora_paged_tensor;

typedef struct {
  int32_t resident;      /* leading tensors whose moments stay on the device */
  size_t resident_bytes; /* their share of the buffer                        */
  size_t chunk;          /* values per staging slot (0: nothing is paged)    */
  size_t staging_bytes;  /* the two slots' share of the buffer               */
} qlora_paged_layout;

#define QLORA_PAGED_LOAD 1
#define QLORA_PAGED_STORE 2

/* Host only: the layout qlora_paged_adamw uses for these tensors and a
 * dev_bytes buffer.  A staging slot holds chunk = min(4M, dev_bytes / 32)
 * values rounded down to a multiple of 64, so the slots take at most half
 * the buffer; QLORA_E_WORKSPACE when not every state fits and dev_bytes is
 * below 2 KiB. */
qlora_status qlora_paged_layout_of(const qlora_paged_tensor* t, int32_t ntensors, size_t dev_bytes,
                                   qlora_paged_layout* out);

/* One AdamW step (the update of qlora_adamw) on every tensor, with its
 * moments paged as above.  dev_ws: device buffer of dev_bytes, 256-byte
 * aligned.  step >= 1; flags: QLORA_PAGED_LOAD | QLORA_PAGED_STORE.  Every
 * p, grad, p_bf16 16-byte aligned, n >= 1.  Errors as qlora_adamw, and
 * QLORA_E_WORKSPACE as qlora_paged_layout_of.  The call creates and releases
 * a few HIP events; it allocates no memory. */
qlora_status qlora_paged_adamw(const qlora_paged_tensor* t, int32_t ntensors, void* dev_ws, size_t dev_bytes,
                               float lr, float beta1, float beta2, float eps, float weight_decay, int32_t step,
                               int32_t flags, void* stream, void* copy_stream);

/* The 16 fp32 levels of a codebook, ascending, as the device tables hold
 * them.  QLORA_E_NULL for a NULL out, QLORA_E_UNSUPPORTED for an unknown
 * codebook. */
qlora_status qlora_codebook_levels(qlora_codebook cb, float out[16]);

/* Two paths compute qlora_linear_fwd and qlora_linear_bwd; both give the
 * defined result within the stated tolerances (they differ only in the
 * order of fp32 accumulation):
 *   - fused: the product kernels decode W to bf16 inside each 256-token
 *     tile (deepfa.ir "QLoRA's Working Process": converted to BF16 on the
 *     fly); workspace qlora_workspace_bytes(QLORA_OP_FWD_FUSED / _BWD_FUSED);
 *   - staged: W is dequantized once into the workspace (deq(W) for the
 *     forward, deq(W)^T for dX), then multiplied by the dense bf16 kernel,
 *     so each weight is decoded once per call instead of once per 256
 *     tokens.  Taken when M >= 1024, rows * cols < 2^31 (and, for dX,
 *     rows % 64 == 0) and ws_bytes >= qlora_workspace_bytes(QLORA_OP_FWD /
 *     _BWD), which then includes rows * cols * 2 bytes for the bf16 weight.
 * Forward: Y [M x N] = X deq(W)^T + s (X A^T) B^T, s = RN32(alpha / r).
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

/* Bytes of the scratch array of qlora_linear_fwd_noalloc on each device. */
#define QLORA_STATIC_SCRATCH_BYTES ((size_t)32 << 20)

/* qlora_linear_fwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments, result and errors as
 * qlora_linear_fwd; the scratch it would take from `ws` (U when U_save is
 * NULL, and the split partial sums of X A^T) comes from a 32 MiB array the
 * library holds on each device from its first use until the process ends.
 * It calls no allocating routine.  A call needing more than
 * QLORA_STATIC_SCRATCH_BYTES, i.e. qlora_workspace_bytes(QLORA_OP_FWD, M,
 * N, K, r, 0) > QLORA_STATIC_SCRATCH_BYTES (for example M = 65536 at
 * r = 128), returns QLORA_E_WORKSPACE before enqueuing anything.  The array
 * is shared by every call on one device and keeps the last call's
 * contents: calls that overlap on one device (concurrent streams, several
 * host threads) race on it and must be ordered by the caller.  The current
 * device must be the one `stream` belongs to. */
qlora_status qlora_linear_fwd_noalloc(const qlora_nf4_weight* W, const uint16_t* X, int64_t M,
                                      const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                                      uint16_t* Y, uint16_t* U_save, void* stream);

/* ---- Layer-set groups ----------------------------------------------------
 * LoRA adapts several linears of each transformer layer (deepfa.ir blog,
 * "Optimization Tips", target modules: query and value, extendable to key
 * and output; the layer sets here adapt all seven linears of a LLaMA layer),
 * and some of them read the same input: q, k and v read the normalised
 * hidden state, gate and up the second normalised state.  A group call
 * computes G such linears as one: each has its own NF4 weight W_g [N x K]
 * (all G of one shape, N % 64 == 0) and its own adapter (A_g, B_g) of rank
 * r, with alpha shared.  The adapters are stacked, A [G r x K] = A_0 over
 * A_1 .., and B [G N x r] = B_0 over B_1 ..; outputs sit side by side,
 * Y [M x G N] with Y_g in columns g N .. g N + N - 1.  Per linear the
 * result is the one of qlora_linear_fwd / _bwd; only the data movement is
 * shared:
 *   - the G weights are dequantized into one stack and multiplied by one
 *     dense bf16 product over G N rows (each row group with its own LoRA
 *     tail), so the token tiles of X are read once per G N rows;
 *   - U = X A^T for all G adapters is one pass over X (U [M x G r]);
 *   - dX = sum_g (dY_g deq(W_g) + s G_g A_g) is one product contracting
 *     over G N, with the G adapters as one rank-G r tail; dA is one pass over
 *     X.
 * G r <= 256, G N K < 2^31, M G N < 2^31.  Y_g, U_g, dA_g and dB_g equal
 * those of qlora_linear_fwd / _bwd on the staged path bit for bit; dX differs
 * from the bf16 sum of G per-linear dX only in rounding (it is rounded to
 * bf16 once).  Workspace: qlora_workspace_bytes(QLORA_OP_GROUP_FWD / _BWD,
 * M, N, K, r, G).  Errors as for qlora_linear_fwd, plus QLORA_E_SHAPE when
 * the G weights differ in shape and QLORA_E_UNSUPPORTED when N % 64 != 0
 * or G r > 256. */

/* Y [M x G N] (bf16, overwritten); U_save (nullable) receives U [M x G r]. */
qlora_status qlora_group_fwd(const qlora_nf4_weight* W, int32_t G, const uint16_t* X, int64_t M,
                             const uint16_t* A, const uint16_t* B, int32_t r, float alpha, uint16_t* Y,
                             uint16_t* U_save, void* ws, size_t ws_bytes, void* stream);

/* dY [M x G N]; dX [M x K] (bf16, overwritten; NULL skips it); dA [G r x K]
 * and dB [G N x r] (fp32, overwritten).  U_saved (nullable) is U [M x G r]
 * from qlora_group_fwd; when NULL it is recomputed. */
qlora_status qlora_group_bwd(const qlora_nf4_weight* W, int32_t G, const uint16_t* X, const uint16_t* dY,
                             int64_t M, const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                             const uint16_t* U_saved, uint16_t* dX, float* dA, float* dB, void* ws,
                             size_t ws_bytes, void* stream);

/* Building blocks of the group calls, for callers that keep U and G, or time
 * the dense products on their own:
 *   qlora_group_fwd = qlora_lora_down (rank G r, the stacked A)
 *                     + qlora_group_dequant + qlora_bf16_group_fwd;
 *   qlora_group_bwd = [qlora_lora_down] + qlora_group_lora_dy_b
 *                     + qlora_group_dequant_t + qlora_bf16_group_dx
 *                     + qlora_group_lora_grads.
 * Same layouts and conditions as the group calls; ws is sized by
 * qlora_workspace_bytes(QLORA_OP_GROUP_LORA, M, N, K, r, G). */

/* Wd_out [G N x K] bf16: deq(W_g) in rows g N .. g N + N - 1. */
qlora_status qlora_group_dequant(const qlora_nf4_weight* W, int32_t G, uint16_t* Wd_out, void* stream);

/* WdT_out [K x G N] bf16: deq(W_g)^T in columns g N .. g N + N - 1.
 * Requires rows < 65536 * 64. */
qlora_status qlora_group_dequant_t(const qlora_nf4_weight* W, int32_t G, uint16_t* WdT_out, void* stream);

/* Y [M x G N] = X Wd^T + s (U_g B_g^T side by side), Wd [G N x K] the stack,
 * U [M x G r] and B [G N x r] (r == 0: U = B = NULL).  No workspace. */
qlora_status qlora_bf16_group_fwd(const uint16_t* Wd, int32_t G, int64_t N, int64_t K, const uint16_t* X,
                                  int64_t M, const uint16_t* U, const uint16_t* B, int32_t r, float alpha,
                                  uint16_t* Y, void* stream);

/* dX [M x K] = dY WdT^T + s Gm A, WdT [K x G N], dY [M x G N], Gm [M x G r]
 * (Gm_g = dY_g B_g) and the stacked A [G r x K] (r == 0: Gm = A = NULL).
 * ws (may be NULL): with at least qlora_workspace_bytes(QLORA_OP_BF16_DX, M,
 * N, K, r, G) bytes, a shape with few output tiles and a long contraction
 * (G N) splits the contraction in two and adds the two fp32 halves; with
 * less room it runs unsplit.  The two differ only in rounding.  A call
 * that splits overwrites ws. */
qlora_status qlora_bf16_group_dx(const uint16_t* WdT, int32_t G, int64_t N, int64_t K, const uint16_t* dY,
                                 int64_t M, const uint16_t* Gm, const uint16_t* A, int32_t r, float alpha,
                                 uint16_t* dX, void* ws, size_t ws_bytes, void* stream);

/* Gm [M x G r] (bf16): columns g r .. are dY_g B_g, dY [M x G N], B [G N x r].
 * r in (0, 128], G r <= 256, N % 8 == 0, G N < 2^24. */
qlora_status qlora_group_lora_dy_b(const uint16_t* dY, const uint16_t* B, int64_t M, int64_t N, int32_t r,
                                   int32_t G, uint16_t* Gm, void* ws, size_t ws_bytes, void* stream);

/* dA [G r x K] = s Gm^T X and dB [G N x r] with dB_g = s dY_g^T U_g (fp32,
 * overwritten); U, Gm [M x G r].  M K and M G N below 2^31. */
qlora_status qlora_group_lora_grads(const uint16_t* X, const uint16_t* dY, const uint16_t* U, const uint16_t* Gm,
                                    int64_t M, int64_t N, int64_t K, int32_t r, int32_t G, float alpha,
                                    float* dA, float* dB, void* ws, size_t ws_bytes, void* stream);

/* ---- Building blocks of the forward and backward passes ----------------
 * qlora_linear_fwd = qlora_lora_down + qlora_nf4_fwd;
 * qlora_linear_bwd = [qlora_lora_down] + qlora_lora_dy_b + qlora_nf4_dx
 *                    + qlora_lora_grads.
 * They let a caller keep U and G, reuse them, or time the two fused NF4
 * GEMMs on their own.  Same conventions as above; ws is sized by
 * qlora_workspace_bytes(QLORA_OP_LORA, M, N, K, r, 0). */

/* U [M x r] = X A^T (bf16).  deepfa.ir "LoRA: Prerequisite": the adapter's
 * down-projection.  r in (0, 256] (above 128: the stacked adapters of a
 * group, with ws sized by QLORA_OP_GROUP_LORA), r % 8 == 0, K % 8 == 0,
 * K < 2^24 (QLORA_E_UNSUPPORTED otherwise). */
qlora_status qlora_lora_down(const uint16_t* X, const uint16_t* A, int64_t M, int64_t K, int32_t r,
                             uint16_t* U, void* ws, size_t ws_bytes, void* stream);

/* G [M x r] = dY B (bf16): the gradient reaching the adapter's
 * down-projection output.  N % 8 == 0, N < 2^24. */
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

/* The dense forward GEMM on a weight already dequantized to bf16 (for
 * example by qlora_dequant): Y [M x N] = X Wd^T + s U B^T, with Wd [N x K]
 * bf16 and U = X A^T given (r == 0: U = B = NULL).  K % 64 == 0, N % 8 == 0,
 * N*K, M*K and M*N below 2^31 (QLORA_E_UNSUPPORTED otherwise).  No
 * workspace.  deepfa.ir "QLoRA's Working Process": the weights are converted
 * to BF16 for the computation; here the conversion is a separate pass, so a
 * weight is decoded once per product instead of once per token tile. */
qlora_status qlora_bf16_fwd(const uint16_t* Wd, int64_t N, int64_t K, const uint16_t* X, int64_t M,
                            const uint16_t* U, const uint16_t* B, int32_t r, float alpha, uint16_t* Y,
                            void* stream);

/* The dense backward GEMM on the transposed bf16 weight (for example from
 * qlora_dequant_t): dX [M x K] = dY WdT^T + s G A, with WdT [K x N] bf16,
 * dY [M x N], G = dY B [M x r] given and A [r x K] (r == 0: G = A = NULL).
 * N % 64 == 0, K % 64 == 0, N*K, M*K and M*N below 2^31
 * (QLORA_E_UNSUPPORTED otherwise).  ws (may be NULL) as for
 * qlora_bf16_group_dx, sized by qlora_workspace_bytes(QLORA_OP_BF16_DX, M,
 * N, K, r, 1).  insights4ai page: gradients flow through the frozen weights
 * into the adapters. */
qlora_status qlora_bf16_dx(const uint16_t* WdT, int64_t N, int64_t K, const uint16_t* dY, int64_t M,
                           const uint16_t* G, const uint16_t* A, int32_t r, float alpha, uint16_t* dX,
                           void* ws, size_t ws_bytes, void* stream);

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
 * u = A x and the job table, which the call writes with a host-to-device
 * copy on `stream` from a temporary (pageable) host buffer: HIP stages such
 * a copy before the call returns, so the call may wait for work already
 * queued on `stream`.  Equivalent to qlora_gemv_prepare followed by
 * qlora_gemv_run; a decode loop over fixed layers prepares once and runs
 * the plan, which enqueues only the launches.
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

/* ---- Serialized quantized weights -------------------------------------
 * An adapter is trained against one exact quantized base weight: the pages
 * store the adapters apart from the frozen model and note that they only
 * work with the base model (and quantization) they were trained on
 * (deepfa.ir blog, "LoRA: Prerequisite").  A weight quantized once can be
 * written out and read back byte for byte; the header records the level
 * tables it was encoded with, so a file from a library whose tables differ
 * is refused instead of being decoded with the wrong levels.
 *
 * File = header (QLORA_QTENSOR_HEADER_BYTES) | codes | absmax_q |
 * group_scale (fp32), the three arrays exactly as qlora_sizes() sizes them.
 * Header, all fields little-endian:
 *    0  char[8]  magic "QLORAQT1"
 *    8  uint32   version (1)
 *   12  uint32   header bytes (64)
 *   16  int64    rows
 *   24  int64    cols
 *   32  int32    blocksize (64)      36  int32  group_blocks (256)
 *   40  int32    codebook            44  int32  absmax_format
 *   48  uint64   level-table id (qlora_level_table_id)
 *   56  uint64   payload bytes (codes + absmax_q + group_scale)
 * All calls below are host-only and touch no device memory. */
#define QLORA_QTENSOR_HEADER_BYTES 64

/* 64-bit FNV-1a digest of the tables a weight of this codebook and
 * second-level format is decoded with: the 16 fp32 levels of the 4-bit
 * codebook and the fp32 levels of the block-constant code (256 for LINEAR8,
 * 127 for FP8), as bit patterns, after a version tag.  QLORA_E_NULL for a
 * NULL id, QLORA_E_UNSUPPORTED for an unknown codebook or format. */
qlora_status qlora_level_table_id(int32_t codebook, int32_t absmax_format, uint64_t* id);

/* Write the header of q (its sizes, codebook and format; the device
 * pointers are not read) into out[0 .. QLORA_QTENSOR_HEADER_BYTES).
 * QLORA_E_NULL, QLORA_E_FORMAT when out_bytes is too small, and the errors
 * of qlora_sizes / qlora_level_table_id for an invalid descriptor. */
qlora_status qlora_qtensor_header_write(const qlora_nf4_weight* q, uint8_t* out, size_t out_bytes);

/* Parse a header: fill q's rows, cols, blocksize, group_blocks, codebook and
 * absmax_format (its pointers are left as they are) and *payload_bytes
 * (nullable).  QLORA_E_FORMAT for a short buffer, wrong magic, version or
 * header size, or a payload size that disagrees with the sizes;
 * QLORA_E_UNSUPPORTED / QLORA_E_SHAPE for sizes or tables this library
 * does not handle; QLORA_E_TABLE when the recorded level-table id differs
 * from this library's for that codebook and format. */
qlora_status qlora_qtensor_header_read(const uint8_t* in, size_t in_bytes, qlora_nf4_weight* q,
                                       uint64_t* payload_bytes);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_H */
