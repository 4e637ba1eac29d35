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
//     supplies B operand column n (weight row n of its 16-row group).  A
//     step covers four NF4 blocks (128 code bytes) of each of the 16 rows;
//     lane q loads bytes 16q .. 16q+15 and 64+16q .. 64+16q+15 of its row, so
//     the four lanes of a row read two contiguous 64-byte runs, and each of
//     its two 16-byte pieces is half of one block.  Each piece feeds a chain
//     of four MFMAs whose A operand is "diagonal": rows 4q .. 4q+3 of A hold
//     the x values under lane-group q's piece and zero elsewhere.  Row m of
//     the 16 x 16 result is then the partial dot product of weight row n
//     with lane-group m/4's piece alone, so every lane finds its own piece's
//     partial in its accumulator and applies that block's scale
//     t = Q8[q_b] s2 in fp32.
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
constexpr int kGvRows = kGvWaves * 16;                     // weight rows per workgroup, 16 per wave
constexpr int kGvDepth = 4;                                // steps of codes in flight per wave (a round)
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

// Absmax codes of 16 blocks from `block` (a multiple of 8), as two separate
// 8-byte loads: with K % 512 == 0 a row's absmax codes are a whole number of
// 8-byte units, so neither load straddles the end of the array (the second
// one takes its +8 through the scalar offset, which keeps the compiler from
// fusing the pair into one 16-byte access).
__device__ __forceinline__ void load_absmax16(rsrc_t ar, uint32_t block, uint2 (&out)[2]) {
  out[0] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(ar, block, 0, 0));
  out[1] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(ar, block, 8, 0));
}

// The lane's two 16-byte code pieces in one step: `off` and `off` + 64.
struct Codes {
  uint4 lo, hi;
};
__device__ __forceinline__ Codes load_codes(rsrc_t cr, uint32_t off) {
  return Codes{buf_load16(cr, off), buf_load16(cr, off + 64u)};
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
// tile*kGvRows + 16w .. +15, lane (n, q) row n of them.  Loads run a round
// (kGvDepth steps) ahead:
//   * codes: two 16-byte loads per lane per step;
//   * absmax codes: with kQuad (K % 512 == 0, absmax_q 8-byte aligned), one
//     8-byte load per row per two steps, lane q taking byte q of each 4-byte
//     step; otherwise one byte load per step;
//   * group scales: a row of at most 32768 columns touches at most three
//     256-block groups, so the three scales are loaded once per tile.
template <bool kQuad>
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
  const rsrc_t xr = make_rsrc(J.x, (uint32_t)K * 2u);   // zero padding comes from the range check

  // The lane's row; rows past N read the first byte past the arrays (zero
  // codes, absmax code 0, so block scale 0).  Its two pieces in step s are
  // half (q & 1) of blocks 4s + hb and 4s + 2 + hb, hb = q >> 1.
  const int row = m.y * kGvRows + 16 * w + nl;
  const uint32_t rbase = (uint32_t)(row < N ? row : N) * (uint32_t)nblk;   // first block of the row
  const uint32_t hb = (uint32_t)q >> 1;
  const uint32_t cbase = rbase * 32u + 16u * (uint32_t)q;                   // code byte of the first piece at s = 0

  // x first (waited for before the barrier), then the row's group scales,
  // absmax codes and the first round of codes.
  constexpr int kXChunks = 4;   // 16-byte chunks per thread: K <= 32768
  uint4 xv[kXChunks];
#pragma unroll
  for (int c = 0; c < kXChunks; ++c) xv[c] = buf_load16(xr, 16u * (uint32_t)(tid + c * kGvThreads));
  const uint32_t g0 = rbase >> 8;
  const float s2a = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sr, g0 * 4u, 0, 0));
  const float s2b = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sr, g0 * 4u + 4u, 0, 0));
  const float s2c = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sr, g0 * 4u + 8u, 0, 0));
  uint2 aqr[2];                  // kQuad: absmax codes of the round's 16 blocks (steps 4k .. 4k+3)
  uint32_t aqs[kGvDepth][2];     // !kQuad: the two pieces' absmax codes per step
  if constexpr (kQuad) load_absmax16(ar, rbase, aqr);
  Codes cs[kGvDepth];
  auto load_step = [&](int i, int si) __attribute__((always_inline)) {
    cs[i] = load_codes(cr, cbase + 128u * (uint32_t)si);
    if constexpr (!kQuad) {
      const uint32_t b = rbase + 4u * (uint32_t)si + hb;
      aqs[i][0] = __builtin_amdgcn_raw_buffer_load_b8(ar, b, 0, 0);
      aqs[i][1] = __builtin_amdgcn_raw_buffer_load_b8(ar, b + 2u, 0, 0);
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
  for (int c = 0; c < kXChunks; ++c) {
    const int i = tid + c * kGvThreads;
    lds_st128(i < nsteps * 32 ? xoff + 16u * i : zoff + 16u * (i & 7), xv[c]);
  }
  if (tid < kZeroBytes / 16) lds_st128(zoff + 16u * tid, make_uint4(0u, 0u, 0u, 0u));
  __syncthreads();

  const uint32_t col = 4u * lane;
  const bool diag = (nl >> 2) == q;
  // diagonal lanes: x under the first piece at 64q (bytes) into the step,
  // the second 256 bytes further; off-diagonal lanes read the zero run
  uint32_t xa = diag ? xoff + 64u * q : zoff;
  const uint32_t xinc = diag ? 512u : 0u;
  float acc = 0.0f;

  // Block scale of block `b` (its absmax code `aq`), zero past the row end.
  // (The group scales are passed by value: choosing among variables
  // captured by reference would make the compiler pick among their
  // addresses and keep them in scratch memory.)
  auto scale = [&](uint32_t aq, uint32_t bi, float s2a_, float s2b_, float s2c_) __attribute__((always_inline)) {
    const uint32_t gi = ((rbase + bi) >> 8) - g0;
    const float s2 = gi == 0 ? s2a_ : gi == 1 ? s2b_ : s2c_;
    return bi < (uint32_t)nblk ? block_scale(aq, s2) : 0.0f;   // ragged last step
  };
  // One step: two chains of four MFMAs over the lane's two pieces.
  auto step = [&](const Codes& c, uint32_t aq0, uint32_t aq1, int s, float s2a_, float s2b_, float s2c_)
                  __attribute__((always_inline)) {
    const uint32_t bi = 4u * (uint32_t)s + hb;   // block index within the row
    const float t0 = scale(aq0, bi, s2a_, s2b_, s2c_);
    const float t1 = scale(aq1, bi + 2u, s2a_, s2b_, s2c_);
    f32x4_t D0 = {0.0f, 0.0f, 0.0f, 0.0f}, D1 = {0.0f, 0.0f, 0.0f, 0.0f};
    const uint32_t lw[4] = {c.lo.x, c.lo.y, c.lo.z, c.lo.w}, hw[4] = {c.hi.x, c.hi.y, c.hi.z, c.hi.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8_t a0 = __builtin_bit_cast(bf16x8_t, lds_ld128(xa + 16u * j));
      const bf16x8_t a1 = __builtin_bit_cast(bf16x8_t, lds_ld128(xa + 256u + 16u * j));
      D0 = mfma16x16x32(a0, decode8(lw[j], col), D0);
      D1 = mfma16x16x32(a1, decode8(hw[j], col), D1);
    }
    acc += t0 * D0[0];
    acc += t1 * D1[0];
    xa += xinc;
  };
  auto aq_of = [&](int i, uint32_t byte) __attribute__((always_inline)) -> uint32_t {   // kQuad
    const uint32_t d = (i & 1) ? aqr[i >> 1].y : aqr[i >> 1].x;
    return __builtin_amdgcn_ubfe(d, 8u * byte, 8u);
  };
  auto run_step = [&](int i, int s) __attribute__((always_inline)) {
    if constexpr (kQuad) step(cs[i], aq_of(i, hb), aq_of(i, hb + 2u), s, s2a, s2b, s2c);
    else step(cs[i], aqs[i][0], aqs[i][1], s, s2a, s2b, s2c);
  };

  // Rounds of kGvDepth steps with no branch inside, so the load counters
  // are tracked exactly; each step refills its slot with the step one round
  // later (clamped to the last step: a re-read of lines already in cache).
  int s0 = 0;
  for (; s0 + kGvDepth <= nsteps; s0 += kGvDepth) {
    uint2 aqn[2];
    if constexpr (kQuad) {
      load_absmax16(ar, rbase + 4u * (uint32_t)(s0 + kGvDepth), aqn);   // the next round
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < kGvDepth; ++i) {
      const int s = s0 + i;
      run_step(i, s);
      load_step(i, s + kGvDepth < nsteps ? s + kGvDepth : nsteps - 1);
      __builtin_amdgcn_sched_barrier(0);   // issue the refill here, a round ahead of its use
    }
    if constexpr (kQuad) {
      aqr[0] = aqn[0];
      aqr[1] = aqn[1];
    }
  }
#pragma unroll
  for (int i = 0; i < kGvDepth - 1; ++i)
    if (s0 + i < nsteps) run_step(i, s0 + i);   // uniform

  // LoRA up-projection: the four lanes of a row take alternate 8-rank chunks
  const bool valid = row < N;
  float lora = 0.0f;
  if (J.r > 0 && valid) {
    const bf16_t* brp = J.B + (int64_t)row * J.r;
    for (int i = 8 * q; i < J.r; i += 32) {
      const uint4 v = *reinterpret_cast<const uint4*>(brp + i);
      const float4 u0 = *reinterpret_cast<const float4*>(J.u + i);
      const float4 u1 = *reinterpret_cast<const float4*>(J.u + i + 4);
      lora += bf2f(v.x & 0xFFFFu) * u0.x + bf2f(v.x >> 16) * u0.y + bf2f(v.y & 0xFFFFu) * u0.z +
              bf2f(v.y >> 16) * u0.w + bf2f(v.z & 0xFFFFu) * u1.x + bf2f(v.z >> 16) * u1.y +
              bf2f(v.w & 0xFFFFu) * u1.z + bf2f(v.w >> 16) * u1.w;
    }
  }
  float part = acc;
  part += __shfl_xor(part, 16);
  part += __shfl_xor(part, 32);
  lora += __shfl_xor(lora, 16);
  lora += __shfl_xor(lora, 32);
  if (q == 0 && valid) {
    const float y = part + J.s * lora;
    J.y[row] = (bf16_t)(pack_bf16x2(y, 0.0f) & 0xFFFFu);
  }
}

namespace {

// Tiles of jobs whose absmax rows can be read 8 bytes at a time.
bool quad_job(const GemvJob& J) {
  return (J.K % 512) == 0 && (reinterpret_cast<uintptr_t>(J.absmax_q) & 7u) == 0;
}

struct TablePlan {
  size_t jobs_off, quad_off, other_off, down_off, total;
  int n_quad, n_other, n_down;
};

size_t up256(size_t x) { return (x + 255) / 256 * 256; }

TablePlan plan_table(const GemvJob* jobs, int njobs) {
  TablePlan p{};
  for (int i = 0; i < njobs; ++i) {
    (quad_job(jobs[i]) ? p.n_quad : p.n_other) += (jobs[i].N + kGvRows - 1) / kGvRows;
    if (jobs[i].r > 0) p.n_down += (jobs[i].r + kDownRows - 1) / kDownRows;
  }
  p.jobs_off = 0;
  p.quad_off = up256((size_t)njobs * sizeof(GemvJob));
  p.other_off = p.quad_off + up256((size_t)p.n_quad * sizeof(int2));
  p.down_off = p.other_off + up256((size_t)p.n_other * sizeof(int2));
  p.total = p.down_off + up256((size_t)p.n_down * sizeof(int2));
  return p;
}

template <bool kQuad>
hipError_t launch_main(const GemvJob* djobs, const int2* map, int n, size_t lds, hipStream_t st) {
  if (n == 0) return hipSuccess;
  // The kernel addresses its LDS from 0, which holds only while the
  // compiler has given it no static LDS.
  hipFuncAttributes fa{};
  hipError_t e = hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(&nf4_gemv_kernel<kQuad>));
  if (e != hipSuccess) return e;
  if (fa.sharedSizeBytes != 0) return hipErrorInvalidKernelFile;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&nf4_gemv_kernel<kQuad>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(nf4_gemv_kernel<kQuad>, dim3(n), dim3(kGvThreads), lds, st, djobs, map);
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
  const int64_t nsteps = (K / 64 + 3) / 4;
  return (size_t)kLutBytes + (size_t)nsteps * 512 + kZeroBytes;
}

hipError_t launch_gemv(const GemvJob* jobs, int njobs, void* table, hipStream_t st) {
  const TablePlan p = plan_table(jobs, njobs);
  std::vector<uint8_t> host(p.total, 0);
  std::memcpy(host.data() + p.jobs_off, jobs, (size_t)njobs * sizeof(GemvJob));
  int2* qm = reinterpret_cast<int2*>(host.data() + p.quad_off);
  int2* om = reinterpret_cast<int2*>(host.data() + p.other_off);
  int2* dm = reinterpret_cast<int2*>(host.data() + p.down_off);
  int maxK = 0;
  for (int i = 0, iq = 0, io = 0, id = 0; i < njobs; ++i) {
    const GemvJob& J = jobs[i];
    const bool quad = quad_job(J);
    for (int t = 0; t < (J.N + kGvRows - 1) / kGvRows; ++t) (quad ? qm[iq++] : om[io++]) = make_int2(i, t);
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
  e = launch_main<true>(djobs, reinterpret_cast<const int2*>(dev + p.quad_off), p.n_quad, lds, st);
  if (e != hipSuccess) return e;
  return launch_main<false>(djobs, reinterpret_cast<const int2*>(dev + p.other_off), p.n_other, lds, st);
}

}  // namespace qlora
