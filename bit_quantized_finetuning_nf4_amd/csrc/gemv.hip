// gemv.hip -- decode y = deq(W) x + s B (A x) over many linears: batch 1
// (this header, nf4_gemv_kernel) and up to 16 tokens per linear
// (nf4_gemv_batch_kernel, further down); u = A x first (lora_row_kernel,
// lora_down_kernel).
//
// whatthefuture.ai article, closing paragraphs: 4-bit inference is slow and
// an 8-16x speed-up is expected; glossary "QLoRA", Definition: the frozen
// weights are 4-bit NF4 with double-quantized constants.
//
// The product streams 0.516 bytes per weight from HBM.  A wave64 VALU
// instruction costs four cycles on a 16-lane SIMD, so at 8 TB/s a decode
// that spends more than about three lane-instructions per weight becomes the
// bound.  This kernel spends one v_perm and one LDS read per two weights:
//
//   * LDS lookup table.  Entry e (a code byte: two weights) is the bf16 pair
//     {L[e & 15], L[e >> 4]} of unscaled levels.  The 256 entries are stored
//     once per lane column: entry e of column c sits at byte e*256 + c*4, so
//     lane c always reads bank c and a wave's 64 lookups never conflict
//     (64 KiB).  One v_perm builds the address from a code byte and the lane
//     column; one ds_read_b32 returns two ready bf16 weights.
//   * Loads.  A step covers 256 code bytes (eight NF4 blocks) of each row.
//     One 16-byte load per lane brings four whole rows' steps: lanes
//     4r+p + 16g (r, p, g in 0..3) read chunk 4p+g of row r, so every load
//     touches eight 128-byte lines of four rows.  (Loads spread over sixteen
//     rows stall in the vector L1's address translation.)
//   * MFMA v_mfma_f32_16x16x32_bf16.  B column c = 4r + p is (row r,
//     position p); its four k-groups g are chunks 4p+g, so one MFMA covers
//     dword j of the sixteen chunks of four rows.  A row m carries x for
//     position m >> 2, restricted to the k-groups of one block: rows with
//     m & 1 = h keep k-groups 2h, 2h+1 (block 2p+h of the step) and are zero
//     elsewhere.  Result row 4p + h of column c is then the partial dot
//     product of row r with block 2p+h alone; lane c + 16p holds it and
//     applies the block's scale t = Q8[q_b] s2 in fp32.  x is shared by the
//     row sets of a wave, so one A operand serves all of them.
//   * Persistent workgroups.  One 16-wave workgroup per CU (the 64 KiB table
//     and x fill its LDS) walks a contiguous, cost-balanced range of row
//     tiles.  The tables are built once; x is restaged only when the job's
//     x pointer or length changes; the code loads run one step ahead
//     straight across tile boundaries, and each tile's LoRA rows and the
//     next tile's group scales are fetched when the tile starts, so no tile
//     boundary waits on memory.
//   * y (and u) are stored through global-address-space pointers: through
//     generic ones they become FLAT stores, and while one may be in flight
//     the compiler turns each wait for a code load into a wait for all
//     loads, draining the loads that run ahead.
//
// The job table lives in device memory (written by one copy per call), so
// one launch per kind of job covers every job.
#include <algorithm>
#include <mutex>
#include <cstring>
#include <vector>

#include "device.h"
#include "kernels.h"

namespace qlora {

namespace {

constexpr int kGvWaves = 16;                               // waves per workgroup
constexpr int kGvThreads = 64 * kGvWaves;
constexpr int kGvSets = 2;                                 // sets of four rows per wave
constexpr int kGvRows = kGvWaves * 4 * kGvSets;            // weight rows per workgroup
constexpr int kStepBlocks = 8;                             // NF4 blocks per row per step (256 code bytes)
constexpr int kLutBytes = 256 * 64 * 4;                    // 256 entries x 64 lane columns
constexpr int kZeroBytes = 512;                            // zero run read by the off-diagonal A lanes
constexpr int kQ8Bytes = 256 * 4;                          // Q8[q] = RN32(q / 255) as fp32
constexpr int kQ8Off = kLutBytes, kZeroOff = kQ8Off + kQ8Bytes, kXOff = kZeroOff + kZeroBytes;   // LDS layout
constexpr int kMaxGvGroups = 1024;                         // persistent workgroups per launch, at most
constexpr int kRowThreads = 256;                           // u = A x of one-token jobs: one workgroup per adapter row
constexpr int kRowUnroll = 4;                              // 16-byte loads of A (and of x) per thread in flight
constexpr int kDownWaves = 4;                              // u = A x of several tokens: one workgroup per 16 adapter rows
constexpr int kDownThreads = 64 * kDownWaves;
constexpr int kDownUnroll = 4;                             // 32-column steps per wave and batch
constexpr int kBtWaves = 16;                               // small-batch kernel: waves per workgroup
constexpr int kBtThreads = 64 * kBtWaves;
constexpr int kBtSets = 2;                                 // 16-row sets per wave
constexpr int kBtRows = kBtWaves * kBtSets * 16;           // weight rows per tile (512)
constexpr int kBtTokens = 16;                              // most tokens per job
constexpr int kBtRank = 128;                               // largest adapter rank the library accepts
constexpr int kBtChunkCols = 1024;                         // columns per staged x chunk (four 256-column spans)
constexpr int kBtXRow = kBtChunkCols * 2 + 16;             // LDS bytes per token row of a chunk (padded)
constexpr int kBtXBuf = kBtTokens * kBtXRow;
constexpr int kBtSuRow = kBtRank * 2 + 16;                 // LDS bytes per token row of s u (padded)
constexpr int kBtSuOff = kQ8Off + kQ8Bytes, kBtXOff = kBtSuOff + kBtTokens * kBtSuRow;
constexpr int kBtLds = kBtXOff + 2 * kBtXBuf;              // 136,960 bytes
static_assert(kBtLds <= 160 * 1024, "LDS of the small-batch kernel");
static_assert(kGvThreads == 1024, "the table fill below assumes 16 waves");

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

__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// bf16 (round to nearest even) of the unscaled level c of codebook CB.
template <int CB>
__device__ __forceinline__ uint32_t level_bf16(int c) {
  return pack_bf16x2(u2f(cb_level_bits<CB>(c)), 0.0f) & 0xFFFFu;
}

__device__ __forceinline__ f32x4_t mfma16x16x32(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// The kernel has no static LDS, so its dynamic LDS starts at address 0 and
// plain 32-bit LDS addresses index it (no base add per access).
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) u32x4_t lds_u128;
__device__ __forceinline__ uint32_t lds_ld32(uint32_t addr) { return *(const lds_u32*)(size_t)addr; }
__device__ __forceinline__ float lds_ldf(uint32_t addr) { return __builtin_bit_cast(float, lds_ld32(addr)); }
__device__ __forceinline__ u32x4_t lds_ld128(uint32_t addr) { return *(const lds_u128*)(size_t)addr; }
__device__ __forceinline__ void lds_st32(uint32_t addr, uint32_t v) { *(lds_u32*)(size_t)addr = v; }
__device__ __forceinline__ void lds_st128(uint32_t addr, uint4 v) {
  *(lds_u128*)(size_t)addr = u32x4_t{v.x, v.y, v.z, v.w};
}

// The job table's y and u pointers as global-memory pointers.  Through a
// generic pointer the accesses become FLAT instructions, and while one of
// those may be in flight the compiler turns every later wait for a vector
// load into a wait for all of them, which drains the loads running ahead.
template <class T>
__device__ __forceinline__ __attribute__((address_space(1))) T* global_ptr(T* p) {
  return (__attribute__((address_space(1))) T*)p;
}

// The value of lane group G (lanes 16G..16G+15) in every group, lane by lane
// within the group: a permlane32 swap of v with itself pairs groups 0-2 and
// 1-3, a permlane16 swap of the result with itself then pairs neighbours.
__device__ __forceinline__ float from_group(float v, int G) {
  const uint32_t x = __builtin_bit_cast(uint32_t, v);
  const auto h = __builtin_amdgcn_permlane32_swap(x, x, false, false);   // [0 1 0 1], [2 3 2 3]
  const uint32_t y = G < 2 ? h[0] : h[1];
  const auto q = __builtin_amdgcn_permlane16_swap(y, y, false, false);   // even groups everywhere, odd ones
  return __builtin_bit_cast(float, (G & 1) ? q[1] : q[0]);
}

// Eight weights (one code dword, element i in nibble i) -> bf16 x 8.  Table
// address of code byte i: byte << 8 | lane column << 2, built by one v_perm.
__device__ __forceinline__ bf16x8_t decode8(uint32_t c, uint32_t col) {
  const uint4 v = make_uint4(lds_ld32(perm(c, col, 0x0C0C0400u)), lds_ld32(perm(c, col, 0x0C0C0500u)),
                             lds_ld32(perm(c, col, 0x0C0C0600u)), lds_ld32(perm(c, col, 0x0C0C0700u)));
  return __builtin_bit_cast(bf16x8_t, v);
}

}  // namespace

// Phase 1: u = A x for every job with r > 0 (fp32, into the job's scratch;
// u[t r + j] for token t).
//
// One-token jobs: one workgroup per adapter row, so that a call of a few
// jobs still spreads over every CU.  Each thread keeps kRowUnroll 16-byte
// loads of A and of x in flight (columns past K read zero), and the
// workgroup adds its threads' dot products in a fixed order.
__global__ __launch_bounds__(kRowThreads) void lora_row_kernel(const GemvJob* __restrict__ jobs,
                                                               const int2* __restrict__ map) {
  __shared__ float part[kRowThreads / 64];
  const int2 mp = map[blockIdx.x];
  const GemvJob& J = jobs[mp.x];
  const int K = J.K, row = mp.y;
  const uint32_t kb = (uint32_t)K * 2u;
  const rsrc_t arr = make_rsrc(J.A + (int64_t)row * K, kb);
  const rsrc_t xr = make_rsrc(J.x, kb);
  float acc = 0.0f;
  for (int c0 = 0; c0 < K / 8; c0 += kRowThreads * kRowUnroll) {
    uint4 av[kRowUnroll], xv[kRowUnroll];
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const uint32_t off = 16u * (uint32_t)(c0 + (int)threadIdx.x + u * kRowThreads);
      av[u] = buf_load16(arr, off);
      xv[u] = buf_load16(xr, off);
    }
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) acc += dot8(av[u], xv[u]);
  }
  const float v = wave_sum(acc);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < kRowThreads / 64; ++i) sum += part[i];
    global_ptr(J.u)[row] = sum;
  }
}

// Jobs of several tokens: one workgroup per 16 adapter rows of a job:
// U [16 tokens x 16 rows] = X A^T by v_mfma_f32_16x16x32_bf16, A operand =
// x (lane c + 16g: token c, columns 8g..8g+7 of a 32-column step), B operand
// = the adapter rows (lane c + 16g: row c, the same columns).  The four waves
// take every fourth step, two batches of four steps in flight each, and add
// their partials in LDS.  Tokens past m and rows past r read zero (buffer
// range checks).
__global__ __launch_bounds__(kDownThreads) void lora_down_kernel(const GemvJob* __restrict__ jobs,
                                                                 const int2* __restrict__ map) {
  __shared__ float part[kDownWaves][16][17];
  const int2 mp = map[blockIdx.x];
  const GemvJob& J = jobs[mp.x];
  const int K = J.K, row0 = mp.y, m = J.m, R = J.r;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, c = lane & 15, g = lane >> 4;
  const uint32_t kb = (uint32_t)K * 2u;
  const rsrc_t xr = make_rsrc(J.x, (uint32_t)m * kb);
  const rsrc_t arr = make_rsrc(J.A + (int64_t)row0 * K, (uint32_t)min(16, R - row0) * kb);
  const uint32_t lane_off = (uint32_t)c * kb + 16u * (uint32_t)g;
  const int nst = K / 32;   // K is a multiple of 64
  f32x4_t D = {0.0f, 0.0f, 0.0f, 0.0f};
  // Batches of kDownUnroll steps (every fourth step), double buffered: the
  // next batch is issued before this one's MFMAs, so loads stay in flight.
  // Steps past the row read past both ranges: zero.
  constexpr int kBatch = kDownWaves * kDownUnroll;
  auto load = [&](uint4 (&xv)[kDownUnroll], uint4 (&av)[kDownUnroll], int s0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kDownUnroll; ++u) {
      const int s = s0 + kDownWaves * u;
      const uint32_t off = s < nst ? lane_off + 64u * (uint32_t)s : 0xFFFFFFF0u;
      xv[u] = buf_load16(xr, off);
      av[u] = buf_load16(arr, off);
    }
  };
  auto mma = [&](const uint4 (&xv)[kDownUnroll], const uint4 (&av)[kDownUnroll]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kDownUnroll; ++u)
      D = mfma16x16x32(__builtin_bit_cast(bf16x8_t, xv[u]), __builtin_bit_cast(bf16x8_t, av[u]), D);
  };
  uint4 xa[kDownUnroll], aa[kDownUnroll], xb[kDownUnroll], ab[kDownUnroll];
  load(xa, aa, w);
  for (int s0 = w; s0 < nst; s0 += 2 * kBatch) {
    load(xb, ab, s0 + kBatch);
    __builtin_amdgcn_sched_barrier(0);
    mma(xa, aa);
    load(xa, aa, s0 + 2 * kBatch);   // unconditional: past the row it reads zero and keeps the waits exact
    __builtin_amdgcn_sched_barrier(0);
    mma(xb, ab);
  }
  // lane (c, g) holds tokens 4g..4g+3 of adapter row row0 + c
#pragma unroll
  for (int i = 0; i < 4; ++i) part[w][4 * g + i][c] = D[i];
  __syncthreads();
  const int t = threadIdx.x >> 4, n = threadIdx.x & 15;
  if (t < m && row0 + n < R) {
    float v = 0.0f;
#pragma unroll
    for (int i = 0; i < kDownWaves; ++i) v += part[i][t][n];
    global_ptr(J.u)[t * R + row0 + n] = v;
  }
}

// Phase 2: the NF4 GEMV and the LoRA up-projection, persistent.
//
// Workgroup b owns segments segs[range[b] .. range[b+1]); a segment is
// (job, first tile, tile count) of consecutive tiles of one job.  Within a
// tile of kGvRows rows, wave w owns rows 4 kGvSets w + 4k + r (set k, row r
// of the set).  Lane l = c + 16g, c = 4r + p: row r, position p, k-group g.
// With kPair (even block count per row, 2-byte aligned absmax_q) a lane
// reads its two blocks' absmax codes with one 2-byte load, otherwise with two
// byte loads.  A row of at most 32768 columns touches at most three
// 256-block groups, so three group scales per row cover a tile.
template <bool kPair, int CB>
__global__ __launch_bounds__(kGvThreads) void nf4_gemv_kernel(const GemvJob* __restrict__ jobs,
                                                              const int4* __restrict__ segs,
                                                              const int* __restrict__ range, int max_steps,
                                                              int absfmt) {
  extern __shared__ __align__(16) uint8_t lds_dyn[];  // addressed from 0 (see lds_ld32)
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = lane & 15, g = lane >> 4, r = c >> 2, p = c & 3;
  const uint32_t col = 4u * lane;

  // tables, once: thread (w, lane) writes code-byte entries e = w + 16 i of
  // column lane; the first 256 threads write Q8; the first 32 the zero run
  {
    const uint32_t lo = level_bf16<CB>(__builtin_amdgcn_readfirstlane(w));   // w is wave-uniform: a scalar load
#pragma unroll
    for (int i = 0; i < 16; ++i)
      lds_st32((uint32_t)(w + 16 * i) * 256u + 4u * lane, lo | (level_bf16<CB>(i) << 16));
    if (tid < 256) lds_st32(kQ8Off + 4u * tid, __builtin_bit_cast(uint32_t, absmax_value((uint32_t)tid, absfmt)));
    if (tid < kZeroBytes / 16) lds_st128(kZeroOff + 16u * tid, make_uint4(0u, 0u, 0u, 0u));
  }

  // A lane (row m = c, k-group g) carries x for position m >> 2 when g lies
  // in block half m & 1, else reads the zero run.
  const bool xon = (g >> 1) == (c & 1);
  const uint32_t xa0 = xon ? kXOff + 256u * (uint32_t)(c >> 2) + 64u * (uint32_t)g : kZeroOff;
  const uint32_t xinc = xon ? 1024u : 0u;
  const bool holds = g == p;                       // the lane's accumulators are (row r, blocks 2p, 2p+1)
  const uint32_t chunk = 16u * (uint32_t)(4 * p + g);   // code byte of the lane's chunk within a step
  const uint32_t pblk = 2u * (uint32_t)p;               // first of the lane's two blocks within a step
  const uint32_t rchunk = (uint32_t)(4 * g + p);        // the lane's 8-rank chunk of the LoRA term

  // x in LDS belongs to (staged, staged_k); two jobs may share an x
  // pointer with different K, and the zero padding past K differs.
  const void* staged = nullptr;
  int staged_k = 0;
  for (int si = range[blockIdx.x]; si < range[blockIdx.x + 1]; ++si) {
    const int4 sg = segs[si];
    const GemvJob& J = jobs[sg.x];
    const int K = J.K, N = J.N, nblk = K >> 6, R = J.r;
    const int nsteps = (nblk + kStepBlocks - 1) / kStepBlocks;
    const uint32_t nb = (uint32_t)N * (uint32_t)nblk;
    const rsrc_t cr = make_rsrc(J.codes, nb * 32u);
    const rsrc_t ar = make_rsrc(J.absmax_q, nb);
    const rsrc_t sr = make_rsrc(J.group_scale, ((nb + 255u) >> 8) * 4u);
    const rsrc_t br = make_rsrc(J.B, (uint32_t)N * (uint32_t)R * 2u);
    const rsrc_t ur = make_rsrc(J.u, (uint32_t)R * 4u);

    if (J.x != staged || K != staged_k) {   // uniform: restage x (zero-padded to whole steps)
      const rsrc_t xr = make_rsrc(J.x, (uint32_t)K * 2u);
      constexpr int kXChunks = 4;   // 16-byte chunks per thread: K <= 32768
      uint4 xv[kXChunks];
#pragma unroll
      for (int i = 0; i < kXChunks; ++i) xv[i] = buf_load16(xr, 16u * (uint32_t)(tid + i * kGvThreads));
      __syncthreads();   // every wave is done with the previous x
#pragma unroll
      for (int i = 0; i < kXChunks; ++i) {
        const int ci = tid + i * kGvThreads;
        if (ci < max_steps * 64) lds_st128(kXOff + 16u * ci, xv[i]);
      }
      __syncthreads();
      staged = J.x;
      staged_k = K;
    }

    // The lane's u chunk (zero past r: range check).
    const uint4 u0b = buf_load16(ur, 32u * rchunk), u1b = buf_load16(ur, 32u * rchunk + 16u);
    const float uv[8] = {u2f(u0b.x), u2f(u0b.y), u2f(u0b.z), u2f(u0b.w),
                         u2f(u1b.x), u2f(u1b.y), u2f(u1b.z), u2f(u1b.w)};

    // Row of set k in tile t; rows past N read the first byte past the
    // arrays (zero codes, absmax code 0, so block scale 0).
    const int t_first = sg.y, t_last = sg.y + sg.z - 1;
    auto row_of = [&](int t, int k) __attribute__((always_inline)) {
      return t * kGvRows + 4 * kGvSets * w + 4 * k + r;
    };
    auto rbase_of = [&](int t, int k) __attribute__((always_inline)) -> uint32_t {
      const int row = row_of(t, k);
      return (uint32_t)(row < N ? row : N) * (uint32_t)nblk;
    };
    uint32_t rbc[kGvSets], rbn[kGvSets];   // first block of the row: this tile, next tile
    float s2c[kGvSets][3], s2n[kGvSets][3];
    auto load_s2 = [&](float (&dst)[kGvSets][3], const uint32_t (&rb)[kGvSets]) __attribute__((always_inline)) {
#pragma unroll
      for (int k = 0; k < kGvSets; ++k)
#pragma unroll
        for (int i = 0; i < 3; ++i)
          dst[k][i] = u2f(__builtin_amdgcn_raw_buffer_load_b32(sr, ((rb[k] >> 8) + i) * 4u, 0, 0));
    };
    // one step's loads: the chunk of codes and the two absmax codes per set
    uint4 cs[kGvSets];
    uint32_t aq[kGvSets];
    auto load_step = [&](uint4 (&c_)[kGvSets], uint32_t (&a_)[kGvSets], const uint32_t (&rb)[kGvSets], int s)
                         __attribute__((always_inline)) {
#pragma unroll
      for (int k = 0; k < kGvSets; ++k) {
        c_[k] = buf_load16(cr, rb[k] * 32u + 256u * (uint32_t)s + chunk);
        const uint32_t b = rb[k] + kStepBlocks * (uint32_t)s + pblk;
        if constexpr (kPair) {
          a_[k] = __builtin_amdgcn_raw_buffer_load_b16(ar, b, 0, 0);
        } else {
          a_[k] = __builtin_amdgcn_raw_buffer_load_b8(ar, b, 0, 0) |
                  ((uint32_t)__builtin_amdgcn_raw_buffer_load_b8(ar, b + 1u, 0, 0) << 8);
        }
      }
    };
#pragma unroll
    for (int k = 0; k < kGvSets; ++k) {
      rbc[k] = rbase_of(t_first, k);
      rbn[k] = rbase_of(t_first + 1 <= t_last ? t_first + 1 : t_last, k);
    }
    load_s2(s2c, rbc);
    // Loads run one step ahead of use, straight across tile
    // boundaries: (tl, sl) is the next step to load; past the segment's
    // last step it stays on that step (a re-read of cached lines).
    int tl = t_first, sl = 0;
    auto load_next = [&](uint4 (&c_)[kGvSets], uint32_t (&a_)[kGvSets]) __attribute__((always_inline)) {
      uint32_t rb[kGvSets];
#pragma unroll
      for (int k = 0; k < kGvSets; ++k) rb[k] = rbase_of(tl, k);
      load_step(c_, a_, rb, sl);
      if (tl < t_last || sl + 1 < nsteps) {   // uniform scalar bookkeeping
        if (++sl == nsteps) {
          sl = 0;
          ++tl;
        }
      }
    };
    load_next(cs, aq);

    for (int t = t_first; t <= t_last; ++t) {
      // tile start: this tile's LoRA rows and the next tile's group scales
      uint4 bq[kGvSets];
#pragma unroll
      for (int k = 0; k < kGvSets; ++k) {
        const int row = row_of(t, k);
        bq[k] = buf_load16(br, (uint32_t)(row < N ? row : N) * (uint32_t)R * 2u + 16u * rchunk);
      }
      load_s2(s2n, rbn);
      uint32_t gb1[kGvSets], gb2[kGvSets];   // first block (within the row) of its second and third group
#pragma unroll
      for (int k = 0; k < kGvSets; ++k) {
        gb1[k] = 256u - (rbc[k] & 255u);
        gb2[k] = gb1[k] + 256u;
      }
      float acc[kGvSets];
#pragma unroll
      for (int k = 0; k < kGvSets; ++k) acc[k] = 0.0f;
      uint32_t xa = xa0;

      for (int s = 0; s < nsteps; ++s) {
        // the next step's loads first
        uint4 csn[kGvSets];
        uint32_t aqn[kGvSets];
        load_next(csn, aqn);
        __builtin_amdgcn_sched_barrier(0);   // keep the loads ahead of this step's work

        // this step: two chains of four MFMAs per set, then the block scales
        f32x4_t D[kGvSets];
#pragma unroll
        for (int k = 0; k < kGvSets; ++k) D[k] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x8_t a = __builtin_bit_cast(bf16x8_t, lds_ld128(xa + 16u * j));
#pragma unroll
          for (int k = 0; k < kGvSets; ++k) {
            const uint32_t cw = j == 0 ? cs[k].x : j == 1 ? cs[k].y : j == 2 ? cs[k].z : cs[k].w;
            D[k] = mfma16x16x32(a, decode8(cw, col), D[k]);
          }
        }
        // Blocks past the row end (a ragged last step) meet zero-padded x:
        // their partial is zero and their (finite) scale needs no mask.
        const uint32_t bi = kStepBlocks * (uint32_t)s + pblk;
#pragma unroll
        for (int k = 0; k < kGvSets; ++k) {
          const float q0 = lds_ldf(kQ8Off + 4u * (aq[k] & 0xFFu));
          const float q1 = lds_ldf(kQ8Off + 4u * ((aq[k] >> 8) & 0xFFu));
          const float s20 = bi >= gb2[k] ? s2c[k][2] : bi >= gb1[k] ? s2c[k][1] : s2c[k][0];
          const float s21 = kPair ? s20 : (bi + 1u >= gb2[k] ? s2c[k][2] : bi + 1u >= gb1[k] ? s2c[k][1] : s2c[k][0]);
          acc[k] += (q0 * s20) * D[k][0] + (q1 * s21) * D[k][1];
        }
        xa += xinc;
#pragma unroll
        for (int k = 0; k < kGvSets; ++k) {
          cs[k] = csn[k];
          aq[k] = aqn[k];
        }
      }

      // Tile end.  Per set: the row total is the sum over the four lanes
      // holding it (c = 4r + p, g = p); the LoRA up-projection is split
      // over the sixteen lanes of the row by 8-rank chunk 4g + p.  One
      // reduction over g (lanes 16 and 32 apart) and p (1 and 2 apart)
      // adds both.
#pragma unroll
      for (int k = 0; k < kGvSets; ++k) {
        const int row = row_of(t, k);
        const uint32_t bw[4] = {bq[k].x, bq[k].y, bq[k].z, bq[k].w};
        float lora = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) lora += bf2f(bw[e] & 0xFFFFu) * uv[2 * e] + bf2f(bw[e] >> 16) * uv[2 * e + 1];
        float part = (holds ? acc[k] : 0.0f) + J.s * lora;
        part += __shfl_xor(part, 16);
        part += __shfl_xor(part, 32);
        part += __shfl_xor(part, 1);
        part += __shfl_xor(part, 2);
        if (lane == 4 * r && row < N) global_ptr(J.y)[row] = (bf16_t)(pack_bf16x2(part, 0.0f) & 0xFFFFu);
      }
#pragma unroll
      for (int k = 0; k < kGvSets; ++k) {
        rbc[k] = rbn[k];
        rbn[k] = rbase_of(t + 2 <= t_last ? t + 2 : t_last, k);
#pragma unroll
        for (int i = 0; i < 3; ++i) s2c[k][i] = s2n[k][i];
      }
    }
  }
}

// Small-batch decode: jobs of m = 2..16 tokens, Y [m x N] = X deq(W)^T +
// s (X A^T) B^T.
//
// The batch-1 kernel packs (row, position) pairs into the MFMA columns and
// spends its spare A rows on block masking; with m tokens that layout costs
// m/2 times the MFMAs and m copies of x in LDS.  Here the product takes the
// plain layout: B operand = decoded weights (column c = weight row c, k-group
// g), A operand = x (row = token, zero past m), so lane c + 16g ends with
// tokens 4g..4g+3 of row c and applies that row's block scales to its fp32
// partials.
//
//   * Spans.  A span is 256 columns (four NF4 blocks, 128 code bytes) of a
//     16-row set.  Its codes arrive in two loads that each cover eight whole
//     rows (8 rows x 128 bytes, eight full lines: loads spread over sixteen
//     rows stall in the vector L1's address translation).  Load i gives lane
//     (c, g) bytes 64 (c >> 3) + 16 g of row 8i + (c & 7).
//   * Two transposes put them in MFMA layout.  DPP row shifts by 8 lanes
//     under bank masks exchange the load index with lane bit 3, so lane
//     (c, g) then holds 16-byte chunk 4j + g of its own row c in register j.
//     permlane32/16 swaps exchange the dword index with lane bits 4-5, so
//     register (j, d) of lane (c, g) holds dword g of chunk 4j + d.  MFMA
//     u = 4j + d thus covers the 32 columns of chunk u, all in block u >> 1;
//     two MFMAs make a block's partial, which gets the block's scale
//     t = Q8[q] s2 in fp32.
//   * x in LDS.  The eight waves of a workgroup walk the same columns in
//     lockstep, one 1024-column chunk (four spans) of all sixteen token rows
//     (zero past m and past K) at a time, double buffered: a chunk's spans
//     run between the global loads of the next chunk and their LDS stores,
//     then one barrier.  Lane (t, g) reads the x of MFMA u at byte
//     64 u + 16 g of token t's span, once for the two sets of its wave.
//   * Block scales.  Lane (c, g) computes t = Q8[q] s2 of blocks 4g..4g+3
//     of the chunk for its row c once per chunk; span sp takes its four from
//     lane group sp by two permlane swaps each.
//   * Decode table, persistence, cost-balanced tile ranges and loads running
//     a span ahead across tile boundaries as in the batch-1 kernel; a tile is
//     512 rows (sixteen waves of two sets).
//   * LoRA.  s u (bf16, zero past m and r) is staged per job; the
//     up-projection s U B^T is r/32 MFMAs per set at tile end, with B read
//     straight from memory.
template <bool kQuad, int CB>
__global__ __launch_bounds__(kBtThreads) void nf4_gemv_batch_kernel(const GemvJob* __restrict__ jobs,
                                                                    const int4* __restrict__ segs,
                                                                    const int* __restrict__ range, int absfmt) {
  extern __shared__ __align__(16) uint8_t lds_dyn[];  // addressed from 0 (see lds_ld32)
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const uint32_t col = 4u * lane;

  // tables, once: wave w writes code-byte entries e = w + kBtWaves i of column lane
  {
    const int wu = __builtin_amdgcn_readfirstlane(w);
#pragma unroll
    for (int i = 0; i < 256 / kBtWaves; ++i) {
      const int e = wu + kBtWaves * i;
      lds_st32((uint32_t)e * 256u + 4u * lane, level_bf16<CB>(e & 15) | (level_bf16<CB>(e >> 4) << 16));
    }
    if (tid < 256) lds_st32(kQ8Off + 4u * tid, __builtin_bit_cast(uint32_t, absmax_value((uint32_t)tid, absfmt)));
  }

  const uint32_t xlane = kBtXOff + (uint32_t)c * kBtXRow + 16u * (uint32_t)g;   // x of lane (token c, k-group g)
  const uint32_t lrow = (uint32_t)(c & 7), lbyte = 64u * (uint32_t)(c >> 3) + 16u * (uint32_t)g;   // code loads
  const bool bit3 = (c & 8) != 0;
  int cc = 0;   // x chunks staged so far: buffer cc & 1 holds the current one

  for (int si = range[blockIdx.x]; si < range[blockIdx.x + 1]; ++si) {
    const int4 sg = segs[si];
    const GemvJob& J = jobs[sg.x];
    const int K = J.K, N = J.N, nblk = K >> 6, R = J.r, m = J.m;
    // chunks of 16 blocks per row; the spans past the row meet zero x (staged
    // zero past K), so they add exactly zero
    const int nch = (nblk + 15) / 16, nsp = 4 * nch;
    const uint32_t nb = (uint32_t)N * (uint32_t)nblk;
    const rsrc_t cr = make_rsrc(J.codes, nb * 32u);
    const rsrc_t ar = make_rsrc(J.absmax_q, nb);
    const rsrc_t sr = make_rsrc(J.group_scale, ((nb + 255u) >> 8) * 4u);
    const uint32_t bend = (uint32_t)N * (uint32_t)R * 2u;
    const rsrc_t br = make_rsrc(J.B, bend);
    const uint32_t xend = (uint32_t)m * (uint32_t)K * 2u;
    const rsrc_t xr = make_rsrc(J.x, xend);

    // x chunk ch: 16-byte piece p = tid + kBtThreads q is columns
    // 1024 ch + 8 (p & 127) of token p >> 7 (zero past m or K)
    constexpr int kXq = kBtTokens * 128 / kBtThreads;   // 16-byte x pieces per thread and chunk
    // A wave's pieces all belong to one token (64 of its 128), so pieces of
    // tokens past m are skipped wave by wave: their rows of both buffers are
    // zeroed when the job is staged and stay zero.
    auto load_x = [&](uint4 (&v)[kXq], int ch) __attribute__((always_inline)) {
#pragma unroll
      for (int q = 0; q < kXq; ++q) {
        const int p = tid + kBtThreads * q, t = p >> 7, k = kBtChunkCols * ch + 8 * (p & 127);
        if (t < m)   // uniform
          v[q] = buf_load16(xr, k < K ? ((uint32_t)t * (uint32_t)K + (uint32_t)k) * 2u : xend);
      }
    };
    auto store_x = [&](const uint4 (&v)[kXq], int buf) __attribute__((always_inline)) {
#pragma unroll
      for (int q = 0; q < kXq; ++q) {
        const int p = tid + kBtThreads * q;
        if ((p >> 7) < m)   // uniform
          lds_st128(kBtXOff + (uint32_t)buf * kBtXBuf + (uint32_t)(p >> 7) * kBtXRow + 16u * (uint32_t)(p & 127),
                    v[q]);
      }
    };
    {   // stage the job: x chunk 0, zero rows past m in both buffers, and s u
      uint4 xv[kXq];
      load_x(xv, 0);
      constexpr int kSq = kBtTokens * kBtRank / 2 / kBtThreads;   // s u pairs per thread
      uint32_t su[kSq];
#pragma unroll
      for (int q = 0; q < kSq; ++q) {
        const int p = tid + kBtThreads * q, t = p >> 6, j = 2 * (p & 63);
        const bool on = t < m && j < R;   // R is a multiple of 8
        const __attribute__((address_space(1))) float* u = global_ptr(J.u);
        su[q] = on ? pack_bf16x2(J.s * u[t * R + j], J.s * u[t * R + j + 1]) : 0u;
      }
      __syncthreads();   // every wave is done with the previous job's buffers
      store_x(xv, cc & 1);
#pragma unroll
      for (int q = 0; q < kXq; ++q) {
        const int p = tid + kBtThreads * q;
        if ((p >> 7) >= m)   // uniform
#pragma unroll
          for (int bf = 0; bf < 2; ++bf)
            lds_st128(kBtXOff + (uint32_t)bf * kBtXBuf + (uint32_t)(p >> 7) * kBtXRow + 16u * (uint32_t)(p & 127),
                      make_uint4(0u, 0u, 0u, 0u));
      }
#pragma unroll
      for (int q = 0; q < kSq; ++q) {
        const int p = tid + kBtThreads * q;
        lds_st32(kBtSuOff + (uint32_t)(p >> 6) * kBtSuRow + 4u * (uint32_t)(p & 63), su[q]);
      }
      __syncthreads();
    }

    // Row `rr` of set k in tile t; rows past N read the first byte past the
    // arrays (zero codes, absmax code 0, so block scale 0).
    const int t_first = sg.y, t_last = sg.y + sg.z - 1;
    auto rbase = [&](int t, int k, int rr) __attribute__((always_inline)) -> uint32_t {
      const int row = t * kBtRows + 16 * kBtSets * w + 16 * k + rr;
      return (uint32_t)(row < N ? row : N) * (uint32_t)nblk;
    };
    // The group scales of the MFMA-layout row c of each set in tile t: a row
    // of at most 32768 columns touches at most three 256-block groups.
    float s2c[kBtSets][3];
    auto load_s2 = [&](int t) __attribute__((always_inline)) {
#pragma unroll
      for (int k = 0; k < kBtSets; ++k) {
        const uint32_t rb = rbase(t, k, c);
#pragma unroll
        for (int i = 0; i < 3; ++i)
          s2c[k][i] = u2f(__builtin_amdgcn_raw_buffer_load_b32(sr, ((rb >> 8) + i) * 4u, 0, 0));
      }
    };
    // The absmax codes of a chunk (16 blocks per row): lane (c, g) loads
    // blocks 4g..4g+3 of row c once per chunk, a chunk ahead; span sp takes
    // its four from lane c + 16 sp.
    auto load_aq = [&](uint32_t (&a_)[kBtSets], int t, int ch) __attribute__((always_inline)) {
#pragma unroll
      for (int k = 0; k < kBtSets; ++k) {
        const uint32_t b = rbase(t, k, c) + 16u * (uint32_t)ch + 4u * (uint32_t)g;
        if constexpr (kQuad) {   // 4-byte aligned: one load
          a_[k] = __builtin_amdgcn_raw_buffer_load_b32(ar, b, 0, 0);
          continue;
        }
        a_[k] = __builtin_amdgcn_raw_buffer_load_b8(ar, b, 0, 0) |
                ((uint32_t)__builtin_amdgcn_raw_buffer_load_b8(ar, b + 1u, 0, 0) << 8) |
                ((uint32_t)__builtin_amdgcn_raw_buffer_load_b8(ar, b + 2u, 0, 0) << 16) |
                ((uint32_t)__builtin_amdgcn_raw_buffer_load_b8(ar, b + 3u, 0, 0) << 24);
      }
    };
    // Code loads run a span ahead, across tile boundaries; past the
    // segment's last span they stay on it.  lb holds the byte offsets of span
    // 0 of the load tile's rows, plus the lane's bytes.
    uint32_t lb[kBtSets][2];
    auto set_lb = [&](int t) __attribute__((always_inline)) {
#pragma unroll
      for (int k = 0; k < kBtSets; ++k)
#pragma unroll
        for (int i = 0; i < 2; ++i) lb[k][i] = rbase(t, k, 8 * i + (int)lrow) * 32u + lbyte;
    };
    int tl = t_first, sl = 0;
    set_lb(tl);
    auto load_next = [&](uint4 (&c_)[kBtSets][2]) __attribute__((always_inline)) {
#pragma unroll
      for (int k = 0; k < kBtSets; ++k)
#pragma unroll
        for (int i = 0; i < 2; ++i) c_[k][i] = buf_load16(cr, lb[k][i] + 128u * (uint32_t)sl);
      if (tl < t_last || sl + 1 < nsp) {   // uniform scalar bookkeeping
        if (++sl == nsp) {
          sl = 0;
          ++tl;
          set_lb(tl);
        }
      }
    };
    load_s2(t_first);
    uint4 ca[kBtSets][2], cb[kBtSets][2];   // codes of the current and the next span
    load_next(ca);
    uint32_t aqc[kBtSets];
    load_aq(aqc, t_first, 0);

    for (int t = t_first; t <= t_last; ++t) {
      float acc[kBtSets][4];
#pragma unroll
      for (int k = 0; k < kBtSets; ++k)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[k][i] = 0.0f;
      float tq[kBtSets][4];   // block scales of the lane's four blocks of the current chunk

      // One span: `cur` holds its codes, `nxt` receives the next span's; sp is
      // the span within chunk ch, xb the chunk's x of this lane.
      auto span = [&](uint4 (&cur)[kBtSets][2], uint4 (&nxt)[kBtSets][2], int ch, int sp, uint32_t xb)
                      __attribute__((always_inline)) {
        load_next(nxt);
        __builtin_amdgcn_sched_barrier(0);   // keep the loads ahead of this span's work
        // MFMA layout: T[k][4 j + d] = dword g of chunk 4j + d of row c
        uint32_t T[kBtSets][8];
#pragma unroll
        for (int k = 0; k < kBtSets; ++k) {
          uint32_t V[2][4] = {{cur[k][0].x, cur[k][0].y, cur[k][0].z, cur[k][0].w},
                              {cur[k][1].x, cur[k][1].y, cur[k][1].z, cur[k][1].w}};
          // load index <-> lane bit 3: lanes with bit 3 set take the other
          // load from 8 lanes below, the others from 8 lanes above
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t lo = V[0][e], hi = V[1][e];
            const uint32_t down = (uint32_t)__builtin_amdgcn_mov_dpp((int)hi, 0x118, 0xF, 0xF, false);   // row_shr:8
            const uint32_t up = (uint32_t)__builtin_amdgcn_mov_dpp((int)lo, 0x108, 0xF, 0xF, false);     // row_shl:8
            V[0][e] = bit3 ? down : lo;
            V[1][e] = bit3 ? hi : up;
          }
          // dword index <-> lane bits 4-5
#pragma unroll
          for (int j = 0; j < 2; ++j) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const auto v = __builtin_amdgcn_permlane32_swap(V[j][e], V[j][e + 2], false, false);
              V[j][e] = v[0];
              V[j][e + 2] = v[1];
            }
#pragma unroll
            for (int e = 0; e < 4; e += 2) {
              const auto v = __builtin_amdgcn_permlane16_swap(V[j][e], V[j][e + 1], false, false);
              V[j][e] = v[0];
              V[j][e + 1] = v[1];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) T[k][4 * j + e] = V[j][e];
          }
        }
        // the span's block scales: blocks 4 sp..4 sp + 3 of the chunk, from lane group sp
        float ts[kBtSets][4];
#pragma unroll
        for (int k = 0; k < kBtSets; ++k)
#pragma unroll
          for (int b = 0; b < 4; ++b) ts[k][b] = from_group(tq[k][b], sp);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          f32x4_t D[kBtSets];
#pragma unroll
          for (int k = 0; k < kBtSets; ++k) D[k] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int u = 2 * b + h;
            const bf16x8_t a = __builtin_bit_cast(bf16x8_t, lds_ld128(xb + 512u * (uint32_t)sp + 64u * (uint32_t)u));
#pragma unroll
            for (int k = 0; k < kBtSets; ++k) D[k] = mfma16x16x32(a, decode8(T[k][u], col), D[k]);
          }
#pragma unroll
          for (int k = 0; k < kBtSets; ++k) {
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[k][i] += ts[k][b] * D[k][i];
            // apply the block's partial now: left to itself the compiler
            // defers these products to the chunk's end and keeps every
            // block's MFMA result alive until then
            asm volatile("" : "+v"(acc[k][0]), "+v"(acc[k][1]), "+v"(acc[k][2]), "+v"(acc[k][3]));
          }
        }
      };

      for (int ch = 0; ch < nch; ++ch) {
        uint4 xv[kXq];
        load_x(xv, ch + 1 < nch ? ch + 1 : 0);   // the next chunk (of the next tile after the last)
        uint32_t aqn[kBtSets];
        load_aq(aqn, ch + 1 < nch ? t : (t + 1 <= t_last ? t + 1 : t_last), ch + 1 < nch ? ch + 1 : 0);
        // this chunk's block scales: blocks 4g..4g+3 of row c
#pragma unroll
        for (int k = 0; k < kBtSets; ++k) {
          const uint32_t gb1 = 256u - (rbase(t, k, c) & 255u), gb2 = gb1 + 256u;   // first block of groups 2, 3
          // the group scales as register values: a select over the array's
          // elements would become a select of addresses and keep the array
          // in memory
          float v0 = s2c[k][0], v1 = s2c[k][1], v2 = s2c[k][2];
          asm volatile("" : "+v"(v0), "+v"(v1), "+v"(v2));
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t bi = 16u * (uint32_t)ch + 4u * (uint32_t)g + (uint32_t)j;   // block within the row
            const float s2 = bi >= gb2 ? v2 : bi >= gb1 ? v1 : v0;
            tq[k][j] = lds_ldf(kQ8Off + 4u * ((aqc[k] >> (8 * j)) & 0xFFu)) * s2;
          }
        }
        const uint32_t xb = xlane + (uint32_t)(cc & 1) * kBtXBuf;
        span(ca, cb, ch, 0, xb);
        span(cb, ca, ch, 1, xb);
        span(ca, cb, ch, 2, xb);
        span(cb, ca, ch, 3, xb);
        store_x(xv, (cc + 1) & 1);
#pragma unroll
        for (int k = 0; k < kBtSets; ++k) aqc[k] = aqn[k];
        __syncthreads();
        ++cc;
      }

      // Tile end: the next tile's group scales (loaded here, where the LoRA
      // loads below wait for memory anyway), the LoRA term by MFMA (A = s u
      // of token c, B = ranks of weight row c; ranks past r read zero on both
      // sides), then y.
      load_s2(t + 1 <= t_last ? t + 1 : t_last);
#pragma unroll
      for (int k = 0; k < kBtSets; ++k) {
        const int row = t * kBtRows + 16 * kBtSets * w + 16 * k + c;
        const uint32_t roff = (uint32_t)(row < N ? row : N) * (uint32_t)R * 2u;
        f32x4_t L = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < kBtRank / 32; ++kk) {
          if (32 * kk < R) {   // uniform
            const uint32_t rk = 32u * (uint32_t)kk + 8u * (uint32_t)g;
            const uint4 bv = buf_load16(br, rk < (uint32_t)R ? roff + 2u * rk : bend);
            const u32x4_t av = lds_ld128(kBtSuOff + (uint32_t)c * kBtSuRow + 2u * rk);
            L = mfma16x16x32(__builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, bv), L);
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = 4 * g + i;
          if (tok < m && row < N)
            global_ptr(J.y)[(int64_t)tok * N + row] = (bf16_t)(pack_bf16x2(acc[k][i] + L[i], 0.0f) & 0xFFFFu);
        }
      }
    }
  }
}

namespace {

// Jobs whose absmax codes can be read two at a time (an even number of
// blocks per row and a 2-byte aligned array).
bool pair_job(const GemvJob& J) {
  return (J.K % 128) == 0 && (reinterpret_cast<uintptr_t>(J.absmax_q) & 1u) == 0;
}

size_t up256(size_t x) { return (x + 255) / 256 * 256; }

// One launch's work: its tiles cut into `groups` contiguous ranges of about
// equal cost (rows x columns), each range a list of per-job segments.
struct LaunchPlan {
  std::vector<int4> segs;
  std::vector<int> range;   // groups + 1 offsets into segs; empty when the launch has no tiles
  int max_steps = 0;
  int groups() const { return range.empty() ? 0 : (int)range.size() - 1; }
};

// Jobs of several tokens whose absmax rows can be read four bytes at a
// time (a multiple of 4 blocks per row and a 4-byte aligned array).
bool quad_job(const GemvJob& J) {
  return (J.K % 256) == 0 && (reinterpret_cast<uintptr_t>(J.absmax_q) & 3u) == 0;
}

// The four launches of a call: batch-1 jobs whose absmax codes pair up,
// the other batch-1 jobs, jobs of two or more tokens with 4-byte aligned
// absmax rows, and the other jobs of several tokens.
int job_kind(const GemvJob& J) { return J.m > 1 ? (quad_job(J) ? 2 : 3) : pair_job(J) ? 0 : 1; }

LaunchPlan plan_launch(const GemvJob* jobs, int njobs, int kind, int max_groups) {
  LaunchPlan lp;
  struct Tile { int job, t; double cost; };
  std::vector<Tile> tiles;
  double total = 0.0;
  const int tile_rows = kind >= 2 ? kBtRows : kGvRows;
  for (int i = 0; i < njobs; ++i) {
    if (job_kind(jobs[i]) != kind) continue;
    const int nt = (jobs[i].N + tile_rows - 1) / tile_rows;
    for (int t = 0; t < nt; ++t) {
      const int rows = std::min(tile_rows, jobs[i].N - t * tile_rows);
      const double cost = (double)rows * (double)jobs[i].K;
      tiles.push_back({i, t, cost});
      total += cost;
    }
    const int steps = (jobs[i].K / 64 + kStepBlocks - 1) / kStepBlocks;
    if (steps > lp.max_steps) lp.max_steps = steps;
  }
  if (tiles.empty()) return lp;
  const int groups = std::min<int>(max_groups, (int)tiles.size());
  lp.range.push_back(0);
  double acc = 0.0;
  size_t ti = 0;
  for (int b = 0; b < groups; ++b) {
    const double target = total * (double)(b + 1) / (double)groups;
    const size_t first = ti;
    // take tiles while the cumulative cost stays at or below the target,
    // at least one per group, and leave one tile for each later group
    while (ti < tiles.size() && (ti == first || acc + tiles[ti].cost <= target * (1.0 + 1e-12)) &&
           tiles.size() - ti > (size_t)(groups - 1 - b)) {
      acc += tiles[ti].cost;
      ++ti;
    }
    if (b == groups - 1)
      while (ti < tiles.size()) acc += tiles[ti++].cost;
    for (size_t k = first; k < ti;) {
      size_t e = k + 1;
      while (e < ti && tiles[e].job == tiles[k].job) ++e;
      lp.segs.push_back(make_int4(tiles[k].job, tiles[k].t, (int)(e - k), 0));
      k = e;
    }
    lp.range.push_back((int)lp.segs.size());
  }
  return lp;
}

int device_cus() { return std::min(device_cu_count(), kMaxGvGroups); }

// Both decode kernels address their LDS from 0, which holds only while the
// compiler has given them no static LDS.  Checked once per kernel, with the
// dynamic-LDS limit raised to the most any launch asks for.
hipError_t gemv_lds_ready(const void* fn) {
  static std::mutex mu;
  static std::vector<const void*> checked;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (std::find(checked.begin(), checked.end(), fn) == checked.end()) {
      hipFuncAttributes fa{};
      hipError_t e = hipFuncGetAttributes(&fa, fn);
      if (e != hipSuccess) return e;
      if (fa.sharedSizeBytes != 0) return hipErrorInvalidKernelFile;
      checked.push_back(fn);
    }
  }
  return allow_lds(fn, kMaxLds);
}

template <bool kPair, int CB>
hipError_t launch_main(const GemvJob* djobs, const int4* segs, const int* range, int groups, int max_steps,
                       int absfmt, hipStream_t st) {
  if (groups <= 0) return hipSuccess;
  // The kernel addresses its LDS from 0, which holds only while the
  // compiler has given it no static LDS (checked once, with the LDS limit).
  hipError_t e = gemv_lds_ready(reinterpret_cast<const void*>(&nf4_gemv_kernel<kPair, CB>));
  if (e != hipSuccess) return e;
  const size_t lds = (size_t)kXOff + (size_t)max_steps * 1024;
  hipLaunchKernelGGL((nf4_gemv_kernel<kPair, CB>), dim3(groups), dim3(kGvThreads), lds, st, djobs, segs, range,
                     max_steps, absfmt);
  return hipGetLastError();
}

template <bool kQuad, int CB>
hipError_t launch_batch(const GemvJob* djobs, const int4* segs, const int* range, int groups, int absfmt,
                        hipStream_t st) {
  if (groups <= 0) return hipSuccess;
  hipError_t e = gemv_lds_ready(reinterpret_cast<const void*>(&nf4_gemv_batch_kernel<kQuad, CB>));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((nf4_gemv_batch_kernel<kQuad, CB>), dim3(groups), dim3(kBtThreads), kBtLds, st, djobs, segs,
                     range, absfmt);
  return hipGetLastError();
}

// The four launches of the GEMV (see job_kind), for codebook CB.
template <int CB>
hipError_t launch_all(const GemvLaunch& L, const GemvJob* djobs, const uint8_t* dev, int absfmt, hipStream_t st) {
  hipError_t e = launch_main<true, CB>(djobs, reinterpret_cast<const int4*>(dev + L.seg_off[0]),
                                       reinterpret_cast<const int*>(dev + L.rng_off[0]), L.groups[0],
                                       L.max_steps[0], absfmt, st);
  if (e != hipSuccess) return e;
  e = launch_main<false, CB>(djobs, reinterpret_cast<const int4*>(dev + L.seg_off[1]),
                             reinterpret_cast<const int*>(dev + L.rng_off[1]), L.groups[1], L.max_steps[1], absfmt,
                             st);
  if (e != hipSuccess) return e;
  e = launch_batch<true, CB>(djobs, reinterpret_cast<const int4*>(dev + L.seg_off[2]),
                             reinterpret_cast<const int*>(dev + L.rng_off[2]), L.groups[2], absfmt, st);
  if (e != hipSuccess) return e;
  return launch_batch<false, CB>(djobs, reinterpret_cast<const int4*>(dev + L.seg_off[3]),
                                 reinterpret_cast<const int*>(dev + L.rng_off[3]), L.groups[3], absfmt, st);
}

}  // namespace

size_t gemv_table_bound(int njobs, int64_t max_rows) {
  if (njobs <= 0 || max_rows <= 0) return 0;
  // jobs | per launch kind: segments (at most one per job plus one per
  // group boundary) and group offsets | lora_down map
  const size_t segs = (size_t)njobs + kMaxGvGroups;
  const size_t downs = (size_t)njobs * 128;
  return up256((size_t)njobs * sizeof(GemvJob)) + kGvKinds * (up256(segs * sizeof(int4)) + up256((kMaxGvGroups + 1) * sizeof(int))) +
         up256(downs * sizeof(int2));
}

size_t gemv_lds_bytes(int64_t K) {
  const int64_t nsteps = (K / 64 + kStepBlocks - 1) / kStepBlocks;
  return (size_t)kXOff + (size_t)nsteps * 1024;
}

hipError_t gemv_prepare(const GemvJob* jobs, int njobs, int codebook, void* table, size_t table_bytes,
                        GemvLaunch* out, hipStream_t st) {
  const int groups = device_cus();
  LaunchPlan lp[kGvKinds];
  for (int k = 0; k < kGvKinds; ++k) lp[k] = plan_launch(jobs, njobs, k, groups);
  // u = A x map: an entry per adapter row of the one-token jobs, then an
  // entry per 16 adapter rows of the others
  std::vector<int2> down;
  for (int i = 0; i < njobs; ++i)
    if (jobs[i].m <= 1)
      for (int t = 0; t < jobs[i].r; ++t) down.push_back(make_int2(i, t));
  const int n_rows = (int)down.size();
  for (int i = 0; i < njobs; ++i)
    if (jobs[i].m > 1)
      for (int t = 0; t < jobs[i].r; t += 16) down.push_back(make_int2(i, t));
  // layout: jobs | per launch kind: segments, group offsets | u = A x map
  GemvLaunch L{};
  size_t off = up256((size_t)njobs * sizeof(GemvJob));
  for (int k = 0; k < kGvKinds; ++k) {
    L.seg_off[k] = off;
    off += up256(lp[k].segs.size() * sizeof(int4));
    L.rng_off[k] = off;
    off += up256(lp[k].range.size() * sizeof(int));
    L.groups[k] = lp[k].groups();
    if (k < 2) L.max_steps[k] = lp[k].max_steps;
  }
  L.down_off = off;
  L.n_down = (int)down.size();
  L.n_rows = n_rows;
  L.codebook = codebook;
  off += up256(down.size() * sizeof(int2));
  if (off > table_bytes) return hipErrorInvalidValue;   // the caller's check makes this unreachable
  std::vector<uint8_t> host(off, 0);
  std::memcpy(host.data(), jobs, (size_t)njobs * sizeof(GemvJob));
  for (int k = 0; k < kGvKinds; ++k) {
    if (!lp[k].segs.empty()) std::memcpy(host.data() + L.seg_off[k], lp[k].segs.data(), lp[k].segs.size() * sizeof(int4));
    if (!lp[k].range.empty()) std::memcpy(host.data() + L.rng_off[k], lp[k].range.data(), lp[k].range.size() * sizeof(int));
  }
  if (!down.empty()) std::memcpy(host.data() + L.down_off, down.data(), down.size() * sizeof(int2));
  L.table = table;
  hipError_t e = hipMemcpyAsync(table, host.data(), off, hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return e;
  *out = L;
  return hipSuccess;
}

hipError_t gemv_run(const GemvLaunch& L, hipStream_t st) {
  const uint8_t* dev = static_cast<const uint8_t*>(L.table);
  const GemvJob* djobs = reinterpret_cast<const GemvJob*>(dev);
  const int2* map = reinterpret_cast<const int2*>(dev + L.down_off);
  if (L.n_rows > 0) {
    hipLaunchKernelGGL(lora_row_kernel, dim3((unsigned)L.n_rows), dim3(kRowThreads), 0, st, djobs, map);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (L.n_down > L.n_rows) {
    hipLaunchKernelGGL(lora_down_kernel, dim3((unsigned)(L.n_down - L.n_rows)), dim3(kDownThreads), 0, st, djobs,
                       map + L.n_rows);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int cb = L.codebook & 0xFF, absfmt = L.codebook >> 8;
  if (cb == kCbFp4) return launch_all<kCbFp4>(L, djobs, dev, absfmt, st);
  if (cb == kCbInt4) return launch_all<kCbInt4>(L, djobs, dev, absfmt, st);
  return launch_all<kCbNf4>(L, djobs, dev, absfmt, st);
}

}  // namespace qlora
