// gemm.hip -- LDS-tiled bf16 MFMA products of the QLoRA linear layer.
//
//   U = X A^T,  G = dY B,  dA = s (dY B)^T X,  dB = s dY^T (X A^T)
// (the fused NF4 GEMMs live in gemm_nf4.hip)
//
// deepfa.ir blog, "LoRA: Prerequisite" and "QLoRA's Working Process" (the
// 4-bit weights are dequantized to BF16 on the fly in the forward and
// backward passes, only the adapters are trained); glossary "QLoRA",
// Definition (weight gradients only for the LoRA matrices).
//
// Engine: 256 threads (4 waves of 64), v_mfma_f32_32x32x16_bf16, fp32
// accumulation.  The MFMA "A" operand is the output-column side (W rows,
// LoRA ranks, ...) and the "B" operand the output-row side (tokens), so each
// lane ends with four consecutive output columns of one row.  Both operands
// are staged in LDS as rows of 64 contraction elements (see lds_chunk_off),
// double buffered: the global loads of step s+1 are issued before the MFMAs
// of step s and written to LDS (dequantizing on the way) after them.
#include "device.h"
#include "kernels.h"

namespace qlora {

constexpr int kThreads = 256;

// A bf16 matrix seen by a tile producer: src[i * ld + j], i < rows, j < cols.
struct TileDesc {
  const bf16_t* src;
  int64_t ld, rows, cols;
};

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

__device__ __forceinline__ uint32_t scale_pair(uint32_t w, float s) {
  return pack_bf16x2(bf2f(w & 0xFFFFu) * s, bf2f(w >> 16) * s);
}

// ---------------------------------------------------------------------------
// Tile producers.  Each fills one LDS tile of BR rows x 64 contraction
// elements for contraction step `step` (elements [64 step, 64 step + 64)).
// ---------------------------------------------------------------------------

// Source rows are contiguous along the contraction: src[row * ld + c].
// cols (the contraction extent) must be a multiple of 8.
template <int BR>
struct RowTile {
  static constexpr int kPer = BR * 8 / kThreads;
  static_assert(kPer >= 1, "tile too small");
  const bf16_t* src;
  int64_t ld, rows, cols, row0;
  uint4 v[kPer];
  __device__ __forceinline__ RowTile(const TileDesc& d, int64_t origin)
      : src(d.src), ld(d.ld), rows(d.rows), cols(d.cols), row0(origin) {}

  __device__ __forceinline__ void load(int step) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int idx = threadIdx.x + i * kThreads;
      const int r = idx >> 3, ch = idx & 7;
      const int64_t gr = row0 + r, gc = (int64_t)step * 64 + ch * 8;
      v[i] = (gr < rows && gc < cols) ? *reinterpret_cast<const uint4*>(src + gr * ld + gc) : zero4();
    }
  }
  __device__ __forceinline__ void store(bf16_t* lds) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int idx = threadIdx.x + i * kThreads;
      *reinterpret_cast<uint4*>(lds + lds_chunk_off(idx >> 3, idx & 7)) = v[i];
    }
  }
  // store s * v, rounded back to bf16
  __device__ __forceinline__ void store_scaled(bf16_t* lds, float s) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int idx = threadIdx.x + i * kThreads;
      const uint4 w = make_uint4(scale_pair(v[i].x, s), scale_pair(v[i].y, s), scale_pair(v[i].z, s),
                                 scale_pair(v[i].w, s));
      *reinterpret_cast<uint4*>(lds + lds_chunk_off(idx >> 3, idx & 7)) = w;
    }
  }
};

// Source is contraction-major: src[c * ld + x]; the tile holds rows x in
// [x0, x0 + BX), so it is a transpose.  A task is a pair of contraction rows
// (2p, 2p+1) times 8 consecutive x; its two 16-byte loads become eight
// dwords {src[2p][x], src[2p+1][x]}.  Tasks are laid out in 8x8 squares
// (8 row pairs x 8 x-groups per wave) so a wave reads whole 128-byte lines.
// xcols must be a multiple of 8.
template <int BX>
struct TransTile {
  static constexpr int kTasks = 4 * BX;
  static constexpr int kPer = (kTasks + kThreads - 1) / kThreads;
  const bf16_t* src;
  int64_t ld, crows, xcols, x0;
  uint4 v0[kPer], v1[kPer];
  // d.rows is the contraction extent, d.cols the x extent
  __device__ __forceinline__ TransTile(const TileDesc& d, int64_t origin)
      : src(d.src), ld(d.ld), crows(d.rows), xcols(d.cols), x0(origin) {}

  __device__ __forceinline__ static void coords(int t, int& p, int& g) {
    const int sq = t >> 6;
    p = ((sq & 3) << 3) | (t & 7);
    g = ((sq >> 2) << 3) | ((t >> 3) & 7);
  }
  __device__ __forceinline__ void load(int step) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int t = threadIdx.x + i * kThreads;
      v0[i] = zero4();
      v1[i] = zero4();
      if (kTasks % kThreads == 0 || t < kTasks) {
        int p, g;
        coords(t, p, g);
        const int64_t c = (int64_t)step * 64 + 2 * p, x = x0 + 8 * g;
        if (x < xcols) {
          if (c < crows) v0[i] = *reinterpret_cast<const uint4*>(src + c * ld + x);
          if (c + 1 < crows) v1[i] = *reinterpret_cast<const uint4*>(src + (c + 1) * ld + x);
        }
      }
    }
  }
  __device__ __forceinline__ void store(bf16_t* lds) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int t = threadIdx.x + i * kThreads;
      if (kTasks % kThreads == 0 || t < kTasks) {
        int p, g;
        coords(t, p, g);
        const uint32_t a[4] = {v0[i].x, v0[i].y, v0[i].z, v0[i].w};
        const uint32_t b[4] = {v1[i].x, v1[i].y, v1[i].z, v1[i].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t w = perm(b[e >> 1], a[e >> 1], (e & 1) ? 0x07060302u : 0x05040100u);
          *reinterpret_cast<uint32_t*>(lds + lds_chunk_off(8 * g + e, p >> 2) + 2 * (p & 3)) = w;
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// MFMA core: wave tile of FI x FJ 32x32 sub-tiles; As rows = output columns
// (starting at ia), Bs rows = output rows (starting at jb).
// ---------------------------------------------------------------------------
template <int FI, int FJ>
__device__ __forceinline__ void mma_step(f32x16_t (&acc)[FI][FJ], const bf16_t* As, const bf16_t* Bs,
                                         int ia, int jb) {
  const int lane = threadIdx.x & 63, lr = lane & 31, h = lane >> 5;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    bf16x8_t a[FI], b[FJ];
#pragma unroll
    for (int i = 0; i < FI; ++i)
      a[i] = *reinterpret_cast<const bf16x8_t*>(As + lds_chunk_off(ia + 32 * i + lr, 2 * kk + h));
#pragma unroll
    for (int j = 0; j < FJ; ++j)
      b[j] = *reinterpret_cast<const bf16x8_t*>(Bs + lds_chunk_off(jb + 32 * j + lr, 2 * kk + h));
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
      for (int j = 0; j < FJ; ++j) acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j]);
  }
}

struct StoreBf16 {
  bf16_t* out;
  int64_t ld, rows, cols;
  __device__ __forceinline__ void operator()(int64_t row, int64_t col, float v0, float v1, float v2,
                                             float v3) const {
    if (row >= rows) return;
    bf16_t* p = out + row * ld + col;
    if (col + 3 < cols) {
      *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
    } else {
      const float v[4] = {v0, v1, v2, v3};
      for (int e = 0; e < 4; ++e)
        if (col + e < cols) p[e] = (bf16_t)(pack_bf16x2(v[e], 0.0f) & 0xFFFFu);
    }
  }
};

struct StoreF32 {
  float* out;
  int64_t ld, rows, cols;
  __device__ __forceinline__ void operator()(int64_t row, int64_t col, float v0, float v1, float v2,
                                             float v3) const {
    if (row >= rows) return;
    float* p = out + row * ld + col;
    if (col + 3 < cols) {
      *reinterpret_cast<float4*>(p) = make_float4(v0, v1, v2, v3);
    } else {
      const float v[4] = {v0, v1, v2, v3};
      for (int e = 0; e < 4; ++e)
        if (col + e < cols) p[e] = v[e];
    }
  }
};

// lane holds column lr of each 32x32 sub-tile and rows 8q + 4h + 0..3 of the
// A side, i.e. four consecutive output columns of one output row.
template <int FI, int FJ, class Store>
__device__ __forceinline__ void epilogue(const f32x16_t (&acc)[FI][FJ], int64_t col0, int64_t row0,
                                         const Store& st) {
  const int lane = threadIdx.x & 63, lr = lane & 31, h = lane >> 5;
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        st(row0 + 32 * j + lr, col0 + 32 * i + 8 * q + 4 * h, acc[i][j][4 * q + 0], acc[i][j][4 * q + 1],
           acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
}

// Workgroup id -> tile: ids are first gathered per XCD (dispatch places
// consecutive ids on consecutive XCDs), then walked column-fastest so the
// tiles resident on one XCD share their token rows in its L2.
__device__ __forceinline__ void map_tile(int tiles_c, int tiles_r, int& tc, int& tr) {
  const int nwg = tiles_c * tiles_r;
  int id = blockIdx.x;
  if ((nwg & 7) == 0) id = (id & 7) * (nwg >> 3) + (id >> 3);
  tc = id % tiles_c;
  tr = id / tiles_c;
}

// ---------------------------------------------------------------------------
// Skinny products (one side is the LoRA rank): out_part[split] = partial
// contraction over a contiguous range of steps; a second kernel sums the
// splits in a fixed order (deterministic) and applies the scale.
// ---------------------------------------------------------------------------
template <bool T, int B>
struct Producer;
template <int B>
struct Producer<false, B> { using type = RowTile<B>; };
template <int B>
struct Producer<true, B> { using type = TransTile<B>; };

template <int BR, int BC, int WR, int WC, bool ROW_T, bool COL_T>
__global__ __launch_bounds__(kThreads) void skinny_kernel(TileDesc rd, TileDesc cd, int64_t rows, int64_t cols,
                                                          int total_steps, int steps_per_split, int tiles_r,
                                                          int tiles_c, float* __restrict__ part) {
  constexpr int TJ = BR / WR, TI = BC / WC, FJ = TJ / 32, FI = TI / 32;
  extern __shared__ __align__(16) bf16_t smem[];
  bf16_t* const As0 = smem;
  bf16_t* const As1 = smem + BC * 64;
  bf16_t* const Bs0 = smem + 2 * BC * 64;
  bf16_t* const Bs1 = smem + 2 * BC * 64 + BR * 64;
  const int tiles = tiles_r * tiles_c;
  const int split = blockIdx.x / tiles, rem = blockIdx.x % tiles;
  const int tr = rem / tiles_c, tc = rem % tiles_c;
  const int w = threadIdx.x >> 6, wr = w / WC, wc = w % WC;
  const int64_t r0 = (int64_t)tr * BR, c0 = (int64_t)tc * BC;
  typename Producer<ROW_T, BR>::type rl(rd, r0);
  typename Producer<COL_T, BC>::type cl(cd, c0);

  f32x16_t acc[FI][FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int s_begin = split * steps_per_split;
  const int s_end = min(total_steps, s_begin + steps_per_split);
  if (s_begin < s_end) {
    rl.load(s_begin);
    cl.load(s_begin);
    rl.store(Bs0);
    cl.store(As0);
    __syncthreads();
    for (int st = s_begin; st < s_end; ++st) {
      const bool odd = (st - s_begin) & 1;
      if (st + 1 < s_end) {
        rl.load(st + 1);
        cl.load(st + 1);
      }
      mma_step<FI, FJ>(acc, odd ? As1 : As0, odd ? Bs1 : Bs0, wc * TI, wr * TJ);
      if (st + 1 < s_end) {
        rl.store(odd ? Bs0 : Bs1);
        cl.store(odd ? As0 : As1);
      }
      __syncthreads();
    }
  }
  epilogue<FI, FJ>(acc, c0 + wc * TI, r0 + wr * TJ, StoreF32{part + (int64_t)split * rows * cols, cols, rows, cols});
}

// out = scale * sum_s part[s]; optional bf16 outputs (two copies) or fp32.
__global__ __launch_bounds__(kThreads) void reduce_kernel(const float* __restrict__ part, int splits, int64_t n,
                                                          float scale, float* __restrict__ out_f32,
                                                          bf16_t* __restrict__ out_bf16,
                                                          bf16_t* __restrict__ out_bf16_2) {
  const int64_t i = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 4;
  if (i >= n) return;
  float4 acc = *reinterpret_cast<const float4*>(part + i);
  for (int sp = 1; sp < splits; ++sp) {
    const float4 v = *reinterpret_cast<const float4*>(part + (int64_t)sp * n + i);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  acc.x *= scale;
  acc.y *= scale;
  acc.z *= scale;
  acc.w *= scale;
  if (out_f32) *reinterpret_cast<float4*>(out_f32 + i) = acc;
  if (out_bf16 || out_bf16_2) {
    const uint2 p = make_uint2(pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w));
    if (out_bf16) *reinterpret_cast<uint2*>(out_bf16 + i) = p;
    if (out_bf16_2) *reinterpret_cast<uint2*>(out_bf16_2 + i) = p;
  }
}

// ---------------------------------------------------------------------------
// Host-side launchers.
// ---------------------------------------------------------------------------
static hipError_t set_lds(const void* fn, size_t bytes) {
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

// Split of the contraction: enough workgroups to cover the chip, at least
// four 64-element steps per split.
struct SkinnyShape {
  int BR, BC, tiles_r, tiles_c, total_steps, sps, splits;
};

static SkinnyShape skinny_shape(int64_t rows, int64_t cols, int64_t contraction, int BR, int BC) {
  SkinnyShape sh;
  sh.BR = BR;
  sh.BC = BC;
  sh.tiles_r = (int)((rows + BR - 1) / BR);
  sh.tiles_c = (int)((cols + BC - 1) / BC);
  sh.total_steps = (int)((contraction + 63) / 64);
  const int tiles = sh.tiles_r * sh.tiles_c;
  int want = (512 + tiles - 1) / tiles;   // about two workgroups per CU: fewer partial sums to write and re-read
  const int max_splits = sh.total_steps / 4 > 0 ? sh.total_steps / 4 : 1;
  if (want > max_splits) want = max_splits;
  if (want < 1) want = 1;
  sh.sps = (sh.total_steps + want - 1) / want;
  sh.splits = (sh.total_steps + sh.sps - 1) / sh.sps;
  return sh;
}

static void kind_tiles(int kind, int r, int& BR, int& BC) {
  const bool wide = r > 64;
  switch (kind) {
    case kGtX: BR = wide ? 128 : 64; BC = 256; break;   // rows = rank, cols = K
    default: BR = 128; BC = wide ? 128 : 64; break;     // rows = tokens / N, cols = rank
  }
}

size_t skinny_partial_bytes(int64_t rows, int64_t cols, int64_t contraction, int kind) {
  int BR, BC;
  const int r = (kind == kGtX) ? (int)rows : (int)cols;
  kind_tiles(kind, r, BR, BC);
  const SkinnyShape sh = skinny_shape(rows, cols, contraction, BR, BC);
  return (size_t)sh.splits * (size_t)rows * (size_t)cols * sizeof(float);
}

template <int BR, int BC, int WR, int WC, bool ROW_T, bool COL_T>
static hipError_t run_skinny(const TileDesc& rl, const TileDesc& cl, int64_t rows, int64_t cols, int64_t contraction,
                             float* part, float scale, float* out_f32, bf16_t* out_bf16, bf16_t* out_bf16_2,
                             hipStream_t st) {
  const SkinnyShape sh = skinny_shape(rows, cols, contraction, BR, BC);
  const size_t lds = 2u * (BR + BC) * 64 * sizeof(bf16_t);
  auto* fn = &skinny_kernel<BR, BC, WR, WC, ROW_T, COL_T>;
  hipError_t e = set_lds(reinterpret_cast<const void*>(fn), lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3(sh.tiles_r * sh.tiles_c * sh.splits), dim3(kThreads), lds, st, rl, cl, rows, cols,
                     sh.total_steps, sh.sps, sh.tiles_r, sh.tiles_c, part);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = rows * cols;  // multiple of 4: cols is the rank (r % 16 == 0) or K
  hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)((n / 4 + kThreads - 1) / kThreads)), dim3(kThreads), 0, st,
                     part, sh.splits, n, scale, out_f32, out_bf16, out_bf16_2);
  return hipGetLastError();
}

// U = X A^T  [M x r]   (rows = tokens, cols = rank, contraction K)
hipError_t launch_xat(const bf16_t* X, const bf16_t* A, int64_t M, int64_t K, int r, float* part, bf16_t* out,
                      bf16_t* out2, float scale, hipStream_t st) {
  const TileDesc rl{X, K, M, K}, cl{A, K, r, K};
  if (r <= 64) return run_skinny<128, 64, 4, 1, false, false>(rl, cl, M, r, K, part, scale, nullptr, out, out2, st);
  return run_skinny<128, 128, 4, 1, false, false>(rl, cl, M, r, K, part, scale, nullptr, out, out2, st);
}

// G = dY B  [M x r]   (contraction N; B [N x r] is contraction-major)
hipError_t launch_dyb(const bf16_t* dY, const bf16_t* B, int64_t M, int64_t N, int r, float* part, bf16_t* out,
                      float scale, hipStream_t st) {
  const TileDesc rl{dY, N, M, N}, cl{B, r, N, r};
  if (r <= 64) return run_skinny<128, 64, 4, 1, false, true>(rl, cl, M, r, N, part, scale, nullptr, out, nullptr, st);
  return run_skinny<128, 128, 4, 1, false, true>(rl, cl, M, r, N, part, scale, nullptr, out, nullptr, st);
}

// dA = scale * G^T X  [r x K]   (rows = rank, cols = K, contraction M)
hipError_t launch_gtx(const bf16_t* G, const bf16_t* X, int64_t M, int64_t K, int r, float* part, float* dA,
                      float scale, hipStream_t st) {
  const TileDesc rl{G, r, M, r}, cl{X, K, M, K};
  if (r <= 64) return run_skinny<64, 256, 1, 4, true, true>(rl, cl, r, K, M, part, scale, dA, nullptr, nullptr, st);
  return run_skinny<128, 256, 2, 2, true, true>(rl, cl, r, K, M, part, scale, dA, nullptr, nullptr, st);
}

// dB = scale * dY^T U  [N x r]   (rows = N, cols = rank, contraction M)
hipError_t launch_dytu(const bf16_t* dY, const bf16_t* U, int64_t M, int64_t N, int r, float* part, float* dB,
                       float scale, hipStream_t st) {
  const TileDesc rl{dY, N, M, N}, cl{U, r, M, r};
  if (r <= 64) return run_skinny<128, 64, 4, 1, true, true>(rl, cl, N, r, M, part, scale, dB, nullptr, nullptr, st);
  return run_skinny<128, 128, 4, 1, true, true>(rl, cl, N, r, M, part, scale, dB, nullptr, nullptr, st);
}

}  // namespace qlora
