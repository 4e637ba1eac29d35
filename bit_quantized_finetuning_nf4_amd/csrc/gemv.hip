// gemv.hip -- batch-1 decode y = deq(W) x + s B (A x) over many linears.
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
//     x changes; the code loads run one step ahead straight across tile
//     boundaries, and each tile's LoRA rows and the next tile's group scales
//     are fetched when the tile starts, so no tile boundary waits on memory.
//
// The job table lives in device memory (written by one copy per call), so
// one launch covers every job.
#include <algorithm>
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
#ifndef QLORA_GEMV_AHEAD
#define QLORA_GEMV_AHEAD 1
#endif
constexpr int kGvAhead = QLORA_GEMV_AHEAD;                 // steps of code loads in flight per wave (1 or 2)
constexpr int kStepBlocks = 8;                             // NF4 blocks per row per step (256 code bytes)
constexpr int kLutBytes = 256 * 64 * 4;                    // 256 entries x 64 lane columns
constexpr int kZeroBytes = 512;                            // zero run read by the off-diagonal A lanes
constexpr int kQ8Bytes = 256 * 4;                          // Q8[q] = RN32(q / 255) as fp32
constexpr int kQ8Off = kLutBytes, kZeroOff = kQ8Off + kQ8Bytes, kXOff = kZeroOff + kZeroBytes;   // LDS layout
constexpr int kMaxGvGroups = 1024;                         // persistent workgroups per launch, at most
constexpr int kDownThreads = 256;                          // u = A x: one workgroup per adapter row
constexpr int kDownUnroll = 4;                             // 16-byte loads of A per thread in flight
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

// Eight weights (one code dword, element i in nibble i) -> bf16 x 8.  Table
// address of code byte i: byte << 8 | lane column << 2, built by one v_perm.
__device__ __forceinline__ bf16x8_t decode8(uint32_t c, uint32_t col) {
  const uint4 v = make_uint4(lds_ld32(perm(c, col, 0x0C0C0400u)), lds_ld32(perm(c, col, 0x0C0C0500u)),
                             lds_ld32(perm(c, col, 0x0C0C0600u)), lds_ld32(perm(c, col, 0x0C0C0700u)));
  return __builtin_bit_cast(bf16x8_t, v);
}

}  // namespace

// Phase 1: u = A x for every job with r > 0 (fp32, into the job's scratch).
// One workgroup per adapter row: each thread keeps up to kDownUnroll
// 16-byte loads of A (and of x, an L2 hit) in flight, then the workgroup
// sums its partials.
__global__ __launch_bounds__(kDownThreads) void lora_down_kernel(const GemvJob* __restrict__ jobs,
                                                                 const int2* __restrict__ map) {
  __shared__ float part[kDownThreads / 64];
  const int2 m = map[blockIdx.x];
  const GemvJob& J = jobs[m.x];
  const int K = J.K, row = m.y;
  const rsrc_t arr = make_rsrc(J.A + (int64_t)row * K, (uint32_t)K * 2u);   // zero past the row
  const rsrc_t xr = make_rsrc(J.x, (uint32_t)K * 2u);
  float acc = 0.0f;
  for (int c0 = 0; c0 < K / 8; c0 += kDownThreads * kDownUnroll) {
    uint4 av[kDownUnroll], xv[kDownUnroll];
#pragma unroll
    for (int u = 0; u < kDownUnroll; ++u) {
      const uint32_t off = 16u * (uint32_t)(c0 + (int)threadIdx.x + u * kDownThreads);
      av[u] = buf_load16(arr, off);
      xv[u] = buf_load16(xr, off);
    }
#pragma unroll
    for (int u = 0; u < kDownUnroll; ++u) acc += dot8(av[u], xv[u]);
  }
  acc = wave_sum(acc);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.0f;
#pragma unroll
    for (int i = 0; i < kDownThreads / 64; ++i) t += part[i];
    J.u[row] = t;
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
                                                              const int* __restrict__ range, int max_steps) {
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
    if (tid < 256) lds_st32(kQ8Off + 4u * tid, __builtin_bit_cast(uint32_t, q8_value((uint32_t)tid)));
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

  const void* staged = nullptr;
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

    if (J.x != staged) {   // uniform: restage x (zero-padded to whole steps)
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
    // Loads run kGvAhead steps ahead of use, straight across tile
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
    uint4 cs1[kGvSets];
    uint32_t aq1[kGvSets];
    if constexpr (kGvAhead == 2) load_next(cs1, aq1);

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
        // the loads kGvAhead steps ahead first
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
          if constexpr (kGvAhead == 2) {
            cs[k] = cs1[k];
            aq[k] = aq1[k];
            cs1[k] = csn[k];
            aq1[k] = aqn[k];
          } else {
            cs[k] = csn[k];
            aq[k] = aqn[k];
          }
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
        if (lane == 4 * r && row < N) J.y[row] = (bf16_t)(pack_bf16x2(part, 0.0f) & 0xFFFFu);
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

LaunchPlan plan_launch(const GemvJob* jobs, int njobs, bool pair, int max_groups) {
  LaunchPlan lp;
  struct Tile { int job, t; double cost; };
  std::vector<Tile> tiles;
  double total = 0.0;
  for (int i = 0; i < njobs; ++i) {
    if (pair_job(jobs[i]) != pair) continue;
    const int nt = (jobs[i].N + kGvRows - 1) / kGvRows;
    for (int t = 0; t < nt; ++t) {
      const int rows = std::min(kGvRows, jobs[i].N - t * kGvRows);
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

template <bool kPair, int CB>
hipError_t launch_main(const GemvJob* djobs, const int4* segs, const int* range, int groups, int max_steps,
                       hipStream_t st) {
  if (groups <= 0) return hipSuccess;
  // The kernel addresses its LDS from 0, which holds only while the
  // compiler has given it no static LDS.
  hipFuncAttributes fa{};
  hipError_t e = hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(&nf4_gemv_kernel<kPair, CB>));
  if (e != hipSuccess) return e;
  if (fa.sharedSizeBytes != 0) return hipErrorInvalidKernelFile;
  const size_t lds = (size_t)kXOff + (size_t)max_steps * 1024;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&nf4_gemv_kernel<kPair, CB>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((nf4_gemv_kernel<kPair, CB>), dim3(groups), dim3(kGvThreads), lds, st, djobs, segs, range,
                     max_steps);
  return hipGetLastError();
}

// The two launches of the GEMV (jobs whose absmax codes pair up, then the
// rest), for codebook CB.
template <int CB>
hipError_t launch_both(const GemvLaunch& L, const GemvJob* djobs, const uint8_t* dev, hipStream_t st) {
  const hipError_t e = launch_main<true, CB>(djobs, reinterpret_cast<const int4*>(dev + L.seg_off[0]),
                                             reinterpret_cast<const int*>(dev + L.rng_off[0]), L.groups[0],
                                             L.max_steps[0], st);
  if (e != hipSuccess) return e;
  return launch_main<false, CB>(djobs, reinterpret_cast<const int4*>(dev + L.seg_off[1]),
                                reinterpret_cast<const int*>(dev + L.rng_off[1]), L.groups[1], L.max_steps[1], st);
}

}  // namespace

size_t gemv_table_bound(int njobs, int64_t max_rows) {
  if (njobs <= 0 || max_rows <= 0) return 0;
  // jobs | per launch kind: segments (at most one per job plus one per
  // group boundary) and group offsets | lora_down map
  const size_t segs = (size_t)njobs + kMaxGvGroups;
  const size_t downs = (size_t)njobs * 128;
  return up256((size_t)njobs * sizeof(GemvJob)) + 2 * (up256(segs * sizeof(int4)) + up256((kMaxGvGroups + 1) * sizeof(int))) +
         up256(downs * sizeof(int2));
}

size_t gemv_lds_bytes(int64_t K) {
  const int64_t nsteps = (K / 64 + kStepBlocks - 1) / kStepBlocks;
  return (size_t)kXOff + (size_t)nsteps * 1024;
}

hipError_t gemv_prepare(const GemvJob* jobs, int njobs, int codebook, void* table, size_t table_bytes,
                        GemvLaunch* out, hipStream_t st) {
  const int groups = device_cus();
  const LaunchPlan lp[2] = {plan_launch(jobs, njobs, true, groups), plan_launch(jobs, njobs, false, groups)};
  std::vector<int2> down;
  for (int i = 0; i < njobs; ++i)
    for (int t = 0; t < jobs[i].r; ++t) down.push_back(make_int2(i, t));
  // layout: jobs | per launch kind: segments, group offsets | u = A x map
  GemvLaunch L{};
  size_t off = up256((size_t)njobs * sizeof(GemvJob));
  for (int k = 0; k < 2; ++k) {
    L.seg_off[k] = off;
    off += up256(lp[k].segs.size() * sizeof(int4));
    L.rng_off[k] = off;
    off += up256(lp[k].range.size() * sizeof(int));
    L.groups[k] = lp[k].groups();
    L.max_steps[k] = lp[k].max_steps;
  }
  L.down_off = off;
  L.n_down = (int)down.size();
  L.codebook = codebook;
  off += up256(down.size() * sizeof(int2));
  if (off > table_bytes) return hipErrorInvalidValue;   // the caller's check makes this unreachable
  std::vector<uint8_t> host(off, 0);
  std::memcpy(host.data(), jobs, (size_t)njobs * sizeof(GemvJob));
  for (int k = 0; k < 2; ++k) {
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
  if (L.n_down > 0) {
    hipLaunchKernelGGL(lora_down_kernel, dim3((unsigned)L.n_down), dim3(kDownThreads), 0, st, djobs,
                       reinterpret_cast<const int2*>(dev + L.down_off));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (L.codebook == kCbFp4) return launch_both<kCbFp4>(L, djobs, dev, st);
  if (L.codebook == kCbInt4) return launch_both<kCbInt4>(L, djobs, dev, st);
  return launch_both<kCbNf4>(L, djobs, dev, st);
}

}  // namespace qlora
