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
//   * MFMA v_mfma_f32_16x16x32_bf16.  Lane l = (n, q), n = l % 16, q = l / 16,
//     supplies B operand column n (weight row n of its 16-row group) for one
//     NF4 block, the block 4s + q of step s; eight MFMAs cover the block's
//     64 weights.  The A operand is "diagonal": rows 4q .. 4q+3 of A hold x
//     over block 4s + q and zero elsewhere.  Row m of the 16 x 16 result is
//     then the partial dot product of weight row n with block 4s + m/4 alone,
//     so every lane finds its own block's partial in its accumulator and
//     applies that block's scale t = Q8[q_b] s2 in fp32.
//   * x is staged in LDS (zero-padded to whole four-block steps) behind the
//     table, with a 128-byte zero run for the off-diagonal A lanes.
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
constexpr int kGvGroups = 2;                               // 16-row groups per wave
constexpr int kGvDepth = 3;                                // steps of loads in flight per wave
constexpr int kGvRows = kGvWaves * 16 * kGvGroups;         // weight rows per workgroup
constexpr int kLutBytes = 256 * 64 * 4;                    // 256 entries x 64 lane columns
constexpr int kZeroBytes = 128;
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

// One step's loads for the lane's kGvGroups rows: the 32 code bytes of block
// 4s + q, its absmax code and its group's scale.
struct Stage {
  uint4 c0[kGvGroups], c1[kGvGroups];
  uint32_t aq[kGvGroups];
  float s2[kGvGroups];
};

__device__ __forceinline__ void load_stage(Stage& st, rsrc_t cr, rsrc_t ar, rsrc_t sr,
                                           const uint32_t (&bidx)[kGvGroups], int s) {
#pragma unroll
  for (int g = 0; g < kGvGroups; ++g) {
    const uint32_t b = bidx[g] + 4u * (uint32_t)s;
    st.c0[g] = buf_load16(cr, b * 32u);
    st.c1[g] = buf_load16(cr, b * 32u + 16u);
    st.aq[g] = __builtin_amdgcn_raw_buffer_load_b8(ar, b, 0, 0);
    st.s2[g] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sr, (b >> 8) * 4u, 0, 0));
  }
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
// tile*kGvRows + 32w .. +31 as two 16-row groups.
__global__ __launch_bounds__(kGvThreads) void nf4_gemv_kernel(const GemvJob* __restrict__ jobs,
                                                              const int2* __restrict__ map) {
  extern __shared__ __align__(16) uint8_t lds_dyn[];  // addressed from 0 (see lds_ld32)
  const int2 m = map[blockIdx.x];
  const GemvJob& J = jobs[m.x];
  const int K = J.K, N = J.N, nblk = K >> 6;
  const int nsteps = (nblk + 3) >> 2;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nl = lane & 15, q = lane >> 4;
  const uint32_t xoff = kLutBytes, zoff = kLutBytes + (uint32_t)nsteps * 512u;

  const uint32_t nb = (uint32_t)N * (uint32_t)nblk;
  const rsrc_t cr = make_rsrc(J.codes, nb * 32u);
  const rsrc_t ar = make_rsrc(J.absmax_q, nb);
  const rsrc_t sr = make_rsrc(J.group_scale, ((nb + 255u) >> 8) * 4u);

  // Per group: the lane's row (rows past N read the first byte past the
  // arrays: zero codes, absmax code 0 and so block scale 0) and the offset
  // of its first block, 4s + q at s = 0.
  int row[kGvGroups];
  uint32_t bidx[kGvGroups];
#pragma unroll
  for (int g = 0; g < kGvGroups; ++g) {
    row[g] = m.y * kGvRows + w * (16 * kGvGroups) + 16 * g + nl;
    bidx[g] = (uint32_t)(row[g] < N ? row[g] : N) * (uint32_t)nblk + (uint32_t)q;
  }

  // x (zero-padded to nsteps * 256 elements) is fetched first, then the
  // first kGvDepth steps' loads, so that waiting for x before the barrier
  // does not wait for the codes.
  constexpr int kXChunks = 4;   // 16-byte chunks per thread: K <= 32768
  const rsrc_t xr = make_rsrc(J.x, (uint32_t)K * 2u);   // the zero padding comes from the range check
  uint4 xv[kXChunks];
#pragma unroll
  for (int c = 0; c < kXChunks; ++c) xv[c] = buf_load16(xr, 16u * (uint32_t)(tid + c * kGvThreads));
  Stage st[kGvDepth];
#pragma unroll
  for (int i = 0; i < kGvDepth; ++i) load_stage(st[i], cr, ar, sr, bidx, i < nsteps ? i : nsteps - 1);

  // table: thread (w, lane) writes entries e = w + 16 i, column lane
  {
    const uint32_t lo = level_bf16(__builtin_amdgcn_readfirstlane(w));   // w is wave-uniform: a scalar load
#pragma unroll
    for (int i = 0; i < 16; ++i)
      lds_st32((uint32_t)(w + 16 * i) * 256u + 4u * lane, lo | (level_bf16(i) << 16));
  }
  // chunks past the staged x are zero (range check) and land in the zero run
#pragma unroll
  for (int c = 0; c < kXChunks; ++c) {
    const int i = tid + c * kGvThreads;
    lds_st128(i < nsteps * 32 ? xoff + 16u * i : zoff + 16u * (i & 7), xv[c]);
  }
  if (tid < kZeroBytes / 16) lds_st128(zoff + 16u * tid, make_uint4(0u, 0u, 0u, 0u));
  __syncthreads();

  const uint32_t col = 4u * lane;
  const bool diag = (nl >> 2) == q;
  uint32_t xa = diag ? xoff + 128u * q : zoff;
  const uint32_t xinc = diag ? 512u : 0u;

  float acc[kGvGroups];
#pragma unroll
  for (int g = 0; g < kGvGroups; ++g) acc[g] = 0.0f;

  // Step s consumes the stage loaded kGvDepth steps earlier and refills it
  // with step s + kGvDepth (clamped to the last step: a re-read of lines
  // already in cache, never used).  The main loop runs whole rounds of
  // kGvDepth steps with no branch inside, so the load counters are tracked
  // exactly across the round; the last partial round follows.
  auto step = [&](Stage& cur, int s, bool refill) {
    const bool live = 4 * s + q < nblk;   // false only in a ragged last step
    float t[kGvGroups];
    f32x4_t D[kGvGroups];
#pragma unroll
    for (int g = 0; g < kGvGroups; ++g) {
      t[g] = live ? block_scale(cur.aq[g] & 0xFFu, cur.s2[g]) : 0.0f;
      D[g] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, lds_ld128(xa + 16u * j));
#pragma unroll
      for (int g = 0; g < kGvGroups; ++g) {
        const uint32_t cw = j < 4 ? (j == 0 ? cur.c0[g].x : j == 1 ? cur.c0[g].y : j == 2 ? cur.c0[g].z : cur.c0[g].w)
                                  : (j == 4 ? cur.c1[g].x : j == 5 ? cur.c1[g].y : j == 6 ? cur.c1[g].z : cur.c1[g].w);
        D[g] = mfma16x16x32(a, decode8(cw, col), D[g]);
      }
    }
#pragma unroll
    for (int g = 0; g < kGvGroups; ++g) acc[g] += t[g] * D[g][0];
    xa += xinc;
    if (refill) {
      const int sn = s + kGvDepth;
      load_stage(cur, cr, ar, sr, bidx, sn < nsteps ? sn : nsteps - 1);
    }
  };
  int s0 = 0;
  for (; s0 + kGvDepth <= nsteps; s0 += kGvDepth) {
#pragma unroll
    for (int i = 0; i < kGvDepth; ++i) step(st[i], s0 + i, true);
  }
#pragma unroll
  for (int i = 0; i < kGvDepth - 1; ++i)
    if (s0 + i < nsteps) step(st[i], s0 + i, false);

  // LoRA up-projection: the four lanes of a row take alternate 8-rank chunks
#pragma unroll
  for (int g = 0; g < kGvGroups; ++g) {
    const bool valid = row[g] < N;
    float lora = 0.0f;
    if (J.r > 0 && valid) {
      const bf16_t* brp = J.B + (int64_t)row[g] * J.r;
      for (int i = 8 * q; i < J.r; i += 32) {
        const uint4 v = *reinterpret_cast<const uint4*>(brp + i);
        const float4 u0 = *reinterpret_cast<const float4*>(J.u + i);
        const float4 u1 = *reinterpret_cast<const float4*>(J.u + i + 4);
        lora += bf2f(v.x & 0xFFFFu) * u0.x + bf2f(v.x >> 16) * u0.y + bf2f(v.y & 0xFFFFu) * u0.z +
                bf2f(v.y >> 16) * u0.w + bf2f(v.z & 0xFFFFu) * u1.x + bf2f(v.z >> 16) * u1.y +
                bf2f(v.w & 0xFFFFu) * u1.z + bf2f(v.w >> 16) * u1.w;
      }
    }
    float part = acc[g];
    part += __shfl_xor(part, 16);
    part += __shfl_xor(part, 32);
    lora += __shfl_xor(lora, 16);
    lora += __shfl_xor(lora, 32);
    if (q == 0 && valid) {
      const float y = part + J.s * lora;
      J.y[row[g]] = (bf16_t)(pack_bf16x2(y, 0.0f) & 0xFFFFu);
    }
  }
}

namespace {

struct TablePlan {
  size_t jobs_off, main_off, down_off, total;
  int n_main, n_down;
};

TablePlan plan_table(const GemvJob* jobs, int njobs) {
  TablePlan p{};
  for (int i = 0; i < njobs; ++i) {
    p.n_main += (jobs[i].N + kGvRows - 1) / kGvRows;
    if (jobs[i].r > 0) p.n_down += (jobs[i].r + kDownRows - 1) / kDownRows;
  }
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  p.jobs_off = 0;
  p.main_off = up((size_t)njobs * sizeof(GemvJob));
  p.down_off = p.main_off + up((size_t)p.n_main * sizeof(int2));
  p.total = p.down_off + up((size_t)p.n_down * sizeof(int2));
  return p;
}

}  // namespace

size_t gemv_table_bound(int njobs, int64_t max_rows) {
  if (njobs <= 0 || max_rows <= 0) return 0;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t tiles = (size_t)njobs * (size_t)((max_rows + kGvRows - 1) / kGvRows);
  const size_t downs = (size_t)njobs * (128 / kDownRows);
  return up((size_t)njobs * sizeof(GemvJob)) + up(tiles * sizeof(int2)) + up(downs * sizeof(int2));
}

size_t gemv_table_bytes(const GemvJob* jobs, int njobs) { return plan_table(jobs, njobs).total; }

size_t gemv_lds_bytes(int64_t K) {
  const int64_t nsteps = (K / 64 + 3) / 4;
  return (size_t)kLutBytes + (size_t)nsteps * 512 + kZeroBytes;
}

hipError_t launch_gemv(const GemvJob* jobs, int njobs, void* table, hipStream_t st) {
  const TablePlan p = plan_table(jobs, njobs);
  std::vector<uint8_t> host(p.total, 0);
  std::memcpy(host.data() + p.jobs_off, jobs, (size_t)njobs * sizeof(GemvJob));
  int2* mm = reinterpret_cast<int2*>(host.data() + p.main_off);
  int2* dm = reinterpret_cast<int2*>(host.data() + p.down_off);
  int maxK = 0;
  for (int i = 0, im = 0, id = 0; i < njobs; ++i) {
    const GemvJob& J = jobs[i];
    for (int t = 0; t < (J.N + kGvRows - 1) / kGvRows; ++t) mm[im++] = make_int2(i, t);
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
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&nf4_gemv_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(nf4_gemv_kernel, dim3(p.n_main), dim3(kGvThreads), lds, st, djobs,
                     reinterpret_cast<const int2*>(dev + p.main_off));
  return hipGetLastError();
}

}  // namespace qlora
