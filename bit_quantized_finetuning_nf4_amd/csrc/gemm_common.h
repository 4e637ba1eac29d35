// gemm_common.h -- tile geometry, tile order, output store and LoRA-tail
// staging shared by the fused NF4 GEMMs and the dense bf16 GEMMs (gfx950).
//
// 256 threads (4 waves), 256 x 256 output tiles, stages of 32 along the
// contraction; operand tiles in LDS are rows of 32 bf16 (64 bytes) with
// 16-byte chunk c of row r at c ^ ((r >> 2) & 3) (spos, lds.h).
#pragma once
#include "device.h"
#include "kernels.h"
#include "lds.h"

namespace qlora {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 256;
constexpr int kStages = 4;                       // ring depth
constexpr int kOp = kTile * 64;                  // 16 KiB: 256 rows x 32 bf16
constexpr int kStage = 2 * kOp;                  // weight half at 0, token half at kOp

// Fragment read offsets in a 64-byte-row tile for the two k16 halves of a
// stage: lane (lr, h) reads chunk 2 kk + h of row lr.
struct FragOffs {
  int o0, o1;
};
__device__ __forceinline__ FragOffs frag_offs(int lane) {
  const int lr = lane & 31, h = lane >> 5;
  return FragOffs{spos(lr, h), spos(lr, 2 + h)};
}

__device__ __forceinline__ void zero_acc(f32x16_t (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
}

template <int FI, int FJ>
__device__ __forceinline__ void mfma_block(f32x16_t (&acc)[FI][FJ], const bf16x8_t (&a)[FI], const bf16x8_t (&b)[FJ]) {
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j) acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j]);
}

// Tile order: consecutive workgroups share the token tile (the column-side
// tiles vary fastest); the eight XCDs receive contiguous ranges.
__device__ __forceinline__ void map_tile(int tiles_c, int tiles_r, int& tc, int& tr) {
  (void)tiles_r;
  const int nwg = (int)gridDim.x;   // the launch may cover only the first tiles of the grid
  int id = blockIdx.x;
  if ((nwg & 7) == 0) id = (id & 7) * (nwg >> 3) + (id >> 3);
  tc = id % tiles_c;
  tr = id / tiles_c;
}

// Output tiles through LDS, for kernels whose LDS is free at the end (16
// bytes per output column of the tile, 64 KiB per 128 columns of 256
// tokens).  In the MFMA output layout a lane holds four consecutive columns
// of one row, so direct 8-byte stores would cover 32 rows per instruction,
// 32 partial cache lines each.  Instead each lane puts its 8-byte pieces
// into LDS rows of U 8-byte units (unit u of row R at u ^ (R & SM): the 32
// rows of one write instruction fall on different banks, and with U a
// multiple of 16 and SM < 16, or U a multiple of 32, the unit stays inside
// its row), then the workgroup writes the tile out row by row, 16 bytes per
// lane, a wave instruction covering whole rows.  Units c, c + 1 (c even) sit
// at the aligned pair (c ^ s) & ~1, swapped when s is odd.
template <int U, int SM>
__device__ __forceinline__ void lds_put4(char* smem, int R, int u, float x0, float x1, float x2, float x3) {
  static_assert(U % 32 == 0 || (U % 16 == 0 && SM < 16), "the swizzle must stay inside the row");
  *reinterpret_cast<u32x2_t*>(smem + (R * U + (u ^ (R & SM))) * 8) = u32x2_t{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
}
// The tile's 256 rows out: row R to out + (row0 + R) ld + col0 .. (4 U
// columns), rows >= rows and columns >= cols skipped (cols % 8 == 0).
template <int U, int SM>
__device__ __forceinline__ void lds_tile_out(const char* smem, bf16_t* out, int64_t ld, int64_t rows, int64_t cols,
                                             int64_t row0, int64_t col0) {
  const int t = threadIdx.x;
#pragma unroll 4
  for (int k = 0; k < U / 2; ++k) {
    const int g = k * kThreads + t, R = g / (U / 2), c = 2 * (g % (U / 2)), sw = R & SM;
    u32x4_t v = *reinterpret_cast<const u32x4_t*>(smem + (R * U + ((c ^ sw) & ~1)) * 8);
    if (sw & 1) v = u32x4_t{v.z, v.w, v.x, v.y};
    const int64_t row = row0 + R, col = col0 + 4 * c;
    if (row < rows && col < cols) *reinterpret_cast<u32x4_t*>(out + row * ld + col) = v;
  }
}
// No load into LDS still in flight, and every wave done with the LDS.
__device__ __forceinline__ void lds_free_for_output() {
  QLORA_WAIT(0, 0);
  __syncthreads();
}

// The 256-token x 64 FI-column tile of the 2 x 2 wave grid: lane (lr, h) of
// wave (wr, wc) holds token row0 + 128 wr + 32 j + lr and columns col0 + 32
// FI wc + 32 i + 8 q + 4 h + 0..3 (16 FI KiB of LDS).
template <int FI>
__device__ __forceinline__ void store_tile_lds(const f32x16_t (&acc)[FI][4], bf16_t* out, int64_t ld, int64_t rows,
                                               int64_t cols, int64_t row0, int64_t col0, char* smem) {
  constexpr int U = 16 * FI, SM = FI == 3 ? 15 : 31;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wr = w >> 1, wc = w & 1, lr = lane & 31, h = lane >> 5;
  lds_free_for_output();
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        lds_put4<U, SM>(smem, wr * 128 + 32 * j + lr, wc * 8 * FI + 8 * i + 2 * q + h, acc[i][j][4 * q],
                        acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
  __syncthreads();
  lds_tile_out<U, SM>(smem, out, ld, rows, cols, row0, col0);
}

// 16 bytes of a bf16 row scaled by s (fp32 product rounded to bf16).
__device__ __forceinline__ uint4 scale16(uint4 v, float s) {
  v.x = pack_bf16x2(bf2f(v.x & 0xFFFFu) * s, bf2f(v.x >> 16) * s);
  v.y = pack_bf16x2(bf2f(v.y & 0xFFFFu) * s, bf2f(v.y >> 16) * s);
  v.z = pack_bf16x2(bf2f(v.z & 0xFFFFu) * s, bf2f(v.z >> 16) * s);
  v.w = pack_bf16x2(bf2f(v.w & 0xFFFFu) * s, bf2f(v.w >> 16) * s);
  return v;
}

// Token half of the LoRA tail: (s T)[row0 + row, j0 + 8 c ..] into a
// 64-byte-row tile (T is rows x rank with row stride ld, zero past the rank
// and the last row).
__device__ __forceinline__ void tail_tokens(char* dst, const bf16_t* T, int64_t ld, int64_t rows, int r,
                                            int64_t row0, int j0, float s) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int idx = threadIdx.x + kThreads * e;
    const int row = idx >> 2, c = idx & 3, col = j0 + 8 * c;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (col < r && row0 + row < rows) v = scale16(*reinterpret_cast<const uint4*>(T + (row0 + row) * ld + col), s);
    wr16(dst + spos(row, c), v);
  }
}
__device__ __forceinline__ void tail_tokens(char* dst, const bf16_t* T, int64_t rows, int r, int64_t row0, int j0,
                                            float s) {
  tail_tokens(dst, T, r, rows, r, row0, j0, s);
}

// DMA pattern for a 256-row x 64-byte tile: wave w, instruction q covers
// rows 64 q + 16 w .. +15 (1 KiB, lane-linear); lane j -> row + (j >> 2),
// position j & 3, which holds chunk (j & 3) ^ ((j >> 4) & 3).
__device__ __forceinline__ int dma_row(int q, int w, int j) { return 64 * q + 16 * w + (j >> 2); }
__device__ __forceinline__ int dma_chunk(int j) { return (j & 3) ^ ((j >> 4) & 3); }

// Operand fragments of a 128 x 128 wave sub-tile: A (column side) and B
// (token side), k16 steps 0 and 1.
struct Frags {
  bf16x8_t a0[4], b0[4], a1[4], b1[4];
};

}  // namespace
}  // namespace qlora
