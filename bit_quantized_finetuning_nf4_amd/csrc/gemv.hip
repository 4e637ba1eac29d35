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
//     four rows, so one A operand serves four row sets.
//   * x is staged in LDS (zero-padded to whole steps) behind the table, with
//     a zero run for the A lanes outside their block.
//
// The job table lives in device memory (written by one copy per call), so
// one launch covers every job and the partial last wave of workgroups is
// paid once per call instead of once per small batch.
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
constexpr int kGvDepth = 2;                                // steps of loads in flight per wave (a round)
constexpr int kStepBlocks = 8;                             // NF4 blocks per row per step (256 code bytes)
constexpr int kLutBytes = 256 * 64 * 4;                    // 256 entries x 64 lane columns
constexpr int kZeroBytes = 512;                           // zero run read by the off-diagonal A lanes
constexpr int kDownThreads = 256;
constexpr int kDownRows = 4;                               // adapter rows per workgroup (one per wave)
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

// bf16 (round to nearest even) of the unscaled NF4 level c.
__device__ __forceinline__ uint32_t level_bf16(int c) {
  return pack_bf16x2(u2f(kNf4LevelBits[c]), 0.0f) & 0xFFFFu;
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

// Phase 1: u = A x for every job with r > 0 (fp32, into the job's scratch);
// one wave per adapter row, four 16-byte loads of A and x in flight per lane.
__global__ __launch_bounds__(kDownThreads) void lora_down_kernel(const GemvJob* __restrict__ jobs,
                                                                 const int2* __restrict__ map) {
  const int2 m = map[blockIdx.x];
  const GemvJob& J = jobs[m.x];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int row = m.y * kDownRows + w;
  if (row >= J.r) return;   // uniform per wave; the kernel has no barrier
  const bf16_t* a = J.A + (int64_t)row * J.K;
  float acc = 0.0f;
  for (int k0 = lane * 8; k0 < J.K; k0 += 4 * 512) {
    uint4 av[4], xv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = k0 + 512 * u;
      av[u] = xv[u] = make_uint4(0u, 0u, 0u, 0u);
      if (k < J.K) {
        av[u] = *reinterpret_cast<const uint4*>(a + k);
        xv[u] = *reinterpret_cast<const uint4*>(J.x + k);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc += dot8(av[u], xv[u]);
  }
  acc = wave_sum(acc);
  if (lane == 0) J.u[row] = acc;
}

// Phase 2: the NF4 GEMV with the LoRA up-projection in the epilogue.
// Workgroup = (job, tile of kGvRows rows); wave w owns rows
// tile*kGvRows + 4 kGvSets w onwards as kGvSets sets of four.  Lane l = c + 16g,
// c = 4r + p: row r of each set, position p, k-group g.  With kPair (even
// block count per row, 2-byte aligned absmax_q) a lane reads its two blocks'
// absmax codes with one 2-byte load, otherwise with two byte loads.  Loads
// run a round (kGvDepth steps) ahead; a row of at most 32768 columns touches
// at most three 256-block groups, so their scales are loaded once per tile.
template <bool kPair>
__global__ __launch_bounds__(kGvThreads) void nf4_gemv_kernel(const GemvJob* __restrict__ jobs,
                                                              const int2* __restrict__ map) {
  extern __shared__ __align__(16) uint8_t lds_dyn[];  // addressed from 0 (see lds_ld32)
  const int2 m = map[blockIdx.x];
  const GemvJob& J = jobs[m.x];
  const int K = J.K, N = J.N, nblk = K >> 6;
  const int nsteps = (nblk + kStepBlocks - 1) / kStepBlocks;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = lane & 15, g = lane >> 4, r = c >> 2, p = c & 3;
  // LDS: code-byte table | x (nsteps * 1024 bytes) | zero run | Q8 table
  const uint32_t xoff = kLutBytes, zoff = kLutBytes + (uint32_t)nsteps * 1024u, q8off = zoff + kZeroBytes;

  const uint32_t nb = (uint32_t)N * (uint32_t)nblk;
  const rsrc_t cr = make_rsrc(J.codes, nb * 32u);
  const rsrc_t ar = make_rsrc(J.absmax_q, nb);
  const rsrc_t sr = make_rsrc(J.group_scale, ((nb + 255u) >> 8) * 4u);
  const rsrc_t xr = make_rsrc(J.x, (uint32_t)K * 2u);   // zero padding comes from the range check

  // Row of each set; rows past N read the first byte past the arrays (zero
  // codes, absmax code 0, so block scale 0).
  uint32_t rb[kGvSets];   // first block of the row
#pragma unroll
  for (int k = 0; k < kGvSets; ++k) {
    const int row = m.y * kGvRows + 4 * kGvSets * w + 4 * k + r;
    rb[k] = (uint32_t)(row < N ? row : N) * (uint32_t)nblk;
  }
  const uint32_t chunk = 16u * (uint32_t)(4 * p + g);   // code byte of the lane's chunk within a step
  const uint32_t pblk = 2u * (uint32_t)p;                // first of the lane's two blocks within a step

  // x first (waited for before the barrier), then the group scales and the
  // first round of codes and absmax codes.
  constexpr int kXChunks = 4;   // 16-byte chunks per thread: K <= 32768
  uint4 xv[kXChunks];
#pragma unroll
  for (int i = 0; i < kXChunks; ++i) xv[i] = buf_load16(xr, 16u * (uint32_t)(tid + i * kGvThreads));
  float s2v[kGvSets][3];
#pragma unroll
  for (int k = 0; k < kGvSets; ++k)
#pragma unroll
    for (int i = 0; i < 3; ++i)
      s2v[k][i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sr, ((rb[k] >> 8) + i) * 4u, 0, 0));
  uint4 cs[kGvDepth][kGvSets];
  uint32_t aq[kGvDepth][kGvSets];   // the lane's two absmax codes, byte 0 and byte 1
  auto load_step = [&](int i, int si) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < kGvSets; ++k) {
      const uint32_t b = rb[k] + kStepBlocks * (uint32_t)si + pblk;
      cs[i][k] = buf_load16(cr, rb[k] * 32u + 256u * (uint32_t)si + chunk);
      if constexpr (kPair) {
        aq[i][k] = __builtin_amdgcn_raw_buffer_load_b16(ar, b, 0, 0);
      } else {
        aq[i][k] = __builtin_amdgcn_raw_buffer_load_b8(ar, b, 0, 0) |
                   ((uint32_t)__builtin_amdgcn_raw_buffer_load_b8(ar, b + 1u, 0, 0) << 8);
      }
    }
  };
#pragma unroll
  for (int i = 0; i < kGvDepth; ++i) load_step(i, i < nsteps ? i : nsteps - 1);

  // table: thread (w, lane) writes entries e = w + 16 i, column lane
  {
    const uint32_t lo = level_bf16(__builtin_amdgcn_readfirstlane(w));   // w is wave-uniform: a scalar load
#pragma unroll
    for (int i = 0; i < 16; ++i)
      lds_st32((uint32_t)(w + 16 * i) * 256u + 4u * lane, lo | (level_bf16(i) << 16));
  }
  // chunks past the staged x are zero (range check) and land in the zero run
#pragma unroll
  for (int i = 0; i < kXChunks; ++i) {
    const int ci = tid + i * kGvThreads;
    lds_st128(ci < nsteps * 64 ? xoff + 16u * ci : zoff + 16u * (ci & 7), xv[i]);
  }
  if (tid < kZeroBytes / 16) lds_st128(zoff + 16u * tid, make_uint4(0u, 0u, 0u, 0u));
  if (tid < 256) lds_st32(q8off + 4u * tid, __builtin_bit_cast(uint32_t, q8_value((uint32_t)tid)));
  __syncthreads();

  const uint32_t col = 4u * lane;
  // A lane (row m = c, k-group g) carries x for position m >> 2 when g lies
  // in block half m & 1, else reads the zero run.
  const bool xon = (g >> 1) == (c & 1);
  uint32_t xa = xon ? xoff + 256u * (uint32_t)(c >> 2) + 64u * (uint32_t)g : zoff;
  const uint32_t xinc = xon ? 1024u : 0u;
  const bool holds = g == p;   // this lane's accumulator is (row r, blocks 2p, 2p+1)
  float acc[kGvSets];
#pragma unroll
  for (int k = 0; k < kGvSets; ++k) acc[k] = 0.0f;

  // Block scales.  The lane's two blocks of a step lie in one 256-block
  // group when the row has an even number of blocks (kPair); otherwise each
  // block finds its own group.  Q8[q] comes from a table in LDS.  Blocks
  // past the row end (a ragged last step) meet zero-padded x, so their
  // partial is zero and their scale (finite) needs no masking.  The group
  // scales come in by value: choosing among variables captured by reference
  // would make the compiler pick among their addresses and keep them in
  // scratch memory.
  uint32_t gb1[kGvSets], gb2[kGvSets];   // first block (within the row) of the row's second and third group
#pragma unroll
  for (int k = 0; k < kGvSets; ++k) {
    gb1[k] = 256u - (rb[k] & 255u);
    gb2[k] = gb1[k] + 256u;
  }
  auto group_scale = [&](int k, uint32_t bi, float sa, float sb, float sc) __attribute__((always_inline)) {
    return bi >= gb2[k] ? sc : bi >= gb1[k] ? sb : sa;
  };
  auto step = [&](int i, int s) __attribute__((always_inline)) {
    f32x4_t D[kGvSets];
#pragma unroll
    for (int k = 0; k < kGvSets; ++k) D[k] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, lds_ld128(xa + 16u * j));
#pragma unroll
      for (int k = 0; k < kGvSets; ++k) {
        const uint32_t cw = j == 0 ? cs[i][k].x : j == 1 ? cs[i][k].y : j == 2 ? cs[i][k].z : cs[i][k].w;
        D[k] = mfma16x16x32(a, decode8(cw, col), D[k]);
      }
    }
    const uint32_t bi = kStepBlocks * (uint32_t)s + pblk;
#pragma unroll
    for (int k = 0; k < kGvSets; ++k) {
      const float q0 = lds_ldf(q8off + 4u * (aq[i][k] & 0xFFu));
      const float q1 = lds_ldf(q8off + 4u * ((aq[i][k] >> 8) & 0xFFu));
      const float s20 = group_scale(k, bi, s2v[k][0], s2v[k][1], s2v[k][2]);
      const float s21 = kPair ? s20 : group_scale(k, bi + 1u, s2v[k][0], s2v[k][1], s2v[k][2]);
      acc[k] += (q0 * s20) * D[k][0] + (q1 * s21) * D[k][1];
    }
    xa += xinc;
  };

  // Rounds of kGvDepth steps with no branch inside, so the load counters
  // are tracked exactly; each step refills its slot with the step one round
  // later (clamped to the last step: a re-read of lines already in cache).
  int s0 = 0;
  for (; s0 + kGvDepth <= nsteps; s0 += kGvDepth) {
#pragma unroll
    for (int i = 0; i < kGvDepth; ++i) {
      const int s = s0 + i;
      step(i, s);
      load_step(i, s + kGvDepth < nsteps ? s + kGvDepth : nsteps - 1);
      __builtin_amdgcn_sched_barrier(0);   // issue the refill here, a round ahead of its use
    }
  }
#pragma unroll
  for (int i = 0; i < kGvDepth - 1; ++i)
    if (s0 + i < nsteps) step(i, s0 + i);   // uniform

  // Per set: the row total is the sum over the four lanes holding it
  // (c = 4r + p, g = p); the LoRA up-projection is split over the sixteen
  // lanes of the row by 8-rank chunks 4g + p.  One reduction over g (lanes
  // 16 and 32 apart) and p (1 and 2 apart) adds both.
#pragma unroll
  for (int k = 0; k < kGvSets; ++k) {
    const int row = m.y * kGvRows + 4 * kGvSets * w + 4 * k + r;
    const bool valid = row < N;
    float lora = 0.0f;
    if (J.r > 0 && valid) {
      const bf16_t* brp = J.B + (int64_t)row * J.r;
      for (int i = 8 * (4 * g + p); i < J.r; i += 128) {
        const uint4 v = *reinterpret_cast<const uint4*>(brp + i);
        const float4 u0 = *reinterpret_cast<const float4*>(J.u + i);
        const float4 u1 = *reinterpret_cast<const float4*>(J.u + i + 4);
        lora += bf2f(v.x & 0xFFFFu) * u0.x + bf2f(v.x >> 16) * u0.y + bf2f(v.y & 0xFFFFu) * u0.z +
                bf2f(v.y >> 16) * u0.w + bf2f(v.z & 0xFFFFu) * u1.x + bf2f(v.z >> 16) * u1.y +
                bf2f(v.w & 0xFFFFu) * u1.z + bf2f(v.w >> 16) * u1.w;
      }
    }
    float part = (holds ? acc[k] : 0.0f) + J.s * lora;
    part += __shfl_xor(part, 16);
    part += __shfl_xor(part, 32);
    part += __shfl_xor(part, 1);
    part += __shfl_xor(part, 2);
    if (lane == 4 * r && valid) J.y[row] = (bf16_t)(pack_bf16x2(part, 0.0f) & 0xFFFFu);
  }
}

namespace {

// Tiles of jobs whose absmax codes can be read two at a time (an even
// number of blocks per row and a 2-byte aligned array).
bool pair_job(const GemvJob& J) {
  return (J.K % 128) == 0 && (reinterpret_cast<uintptr_t>(J.absmax_q) & 1u) == 0;
}

struct TablePlan {
  size_t jobs_off, pair_off, other_off, down_off, total;
  int n_pair, n_other, n_down;
};

size_t up256(size_t x) { return (x + 255) / 256 * 256; }

TablePlan plan_table(const GemvJob* jobs, int njobs) {
  TablePlan p{};
  for (int i = 0; i < njobs; ++i) {
    (pair_job(jobs[i]) ? p.n_pair : p.n_other) += (jobs[i].N + kGvRows - 1) / kGvRows;
    if (jobs[i].r > 0) p.n_down += (jobs[i].r + kDownRows - 1) / kDownRows;
  }
  p.jobs_off = 0;
  p.pair_off = up256((size_t)njobs * sizeof(GemvJob));
  p.other_off = p.pair_off + up256((size_t)p.n_pair * sizeof(int2));
  p.down_off = p.other_off + up256((size_t)p.n_other * sizeof(int2));
  p.total = p.down_off + up256((size_t)p.n_down * sizeof(int2));
  return p;
}

template <bool kPair>
hipError_t launch_main(const GemvJob* djobs, const int2* map, int n, size_t lds, hipStream_t st) {
  if (n == 0) return hipSuccess;
  // The kernel addresses its LDS from 0, which holds only while the
  // compiler has given it no static LDS.
  hipFuncAttributes fa{};
  hipError_t e = hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(&nf4_gemv_kernel<kPair>));
  if (e != hipSuccess) return e;
  if (fa.sharedSizeBytes != 0) return hipErrorInvalidKernelFile;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&nf4_gemv_kernel<kPair>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(nf4_gemv_kernel<kPair>, dim3(n), dim3(kGvThreads), lds, st, djobs, map);
  return hipGetLastError();
}

}  // namespace

size_t gemv_table_bound(int njobs, int64_t max_rows) {
  if (njobs <= 0 || max_rows <= 0) return 0;
  const size_t tiles = (size_t)njobs * (size_t)((max_rows + kGvRows - 1) / kGvRows);
  const size_t downs = (size_t)njobs * (128 / kDownRows);
  // two tile maps (each padded to 256 bytes) share the tiles
  return up256((size_t)njobs * sizeof(GemvJob)) + up256(tiles * sizeof(int2)) + 256 + up256(downs * sizeof(int2));
}

size_t gemv_table_bytes(const GemvJob* jobs, int njobs) { return plan_table(jobs, njobs).total; }

size_t gemv_lds_bytes(int64_t K) {
  const int64_t nsteps = (K / 64 + kStepBlocks - 1) / kStepBlocks;
  return (size_t)kLutBytes + (size_t)nsteps * 1024 + kZeroBytes + 256 * sizeof(float);
}

hipError_t launch_gemv(const GemvJob* jobs, int njobs, void* table, hipStream_t st) {
  const TablePlan p = plan_table(jobs, njobs);
  std::vector<uint8_t> host(p.total, 0);
  std::memcpy(host.data() + p.jobs_off, jobs, (size_t)njobs * sizeof(GemvJob));
  int2* pm = reinterpret_cast<int2*>(host.data() + p.pair_off);
  int2* om = reinterpret_cast<int2*>(host.data() + p.other_off);
  int2* dm = reinterpret_cast<int2*>(host.data() + p.down_off);
  int maxK = 0;
  for (int i = 0, ip = 0, io = 0, id = 0; i < njobs; ++i) {
    const GemvJob& J = jobs[i];
    const bool pair = pair_job(J);
    for (int t = 0; t < (J.N + kGvRows - 1) / kGvRows; ++t) (pair ? pm[ip++] : om[io++]) = make_int2(i, t);
    if (J.r > 0)
      for (int t = 0; t < (J.r + kDownRows - 1) / kDownRows; ++t) dm[id++] = make_int2(i, t);
    if (J.K > maxK) maxK = J.K;
  }
  uint8_t* dev = static_cast<uint8_t*>(table);
  hipError_t e = hipMemcpyAsync(dev, host.data(), p.total, hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return e;
  const GemvJob* djobs = reinterpret_cast<const GemvJob*>(dev + p.jobs_off);
  if (p.n_down > 0) {
    hipLaunchKernelGGL(lora_down_kernel, dim3(p.n_down), dim3(kDownThreads), 0, st, djobs,
                       reinterpret_cast<const int2*>(dev + p.down_off));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const size_t lds = gemv_lds_bytes(maxK);
  e = launch_main<true>(djobs, reinterpret_cast<const int2*>(dev + p.pair_off), p.n_pair, lds, st);
  if (e != hipSuccess) return e;
  return launch_main<false>(djobs, reinterpret_cast<const int2*>(dev + p.other_off), p.n_other, lds, st);
}

}  // namespace qlora
