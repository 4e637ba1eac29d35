// gemm_bf16.hip -- dense bf16 GEMMs on a dequantized weight.
//
//   forward   Y = X Wd^T + s U B^T     (Wd = deq(W) as bf16, U = X A^T)
//
// deepfa.ir blog, "QLoRA's Working Process": the 4-bit weights are converted
// to BF16 for the computation.  These kernels take that bf16 weight from
// memory instead of decoding it inside the tile, so a weight is decoded once
// per product (by the dequant kernel) rather than once per 256-token tile.
//
// 256 threads (4 waves), 256 x 256 output tile, wave (wr, wc) a 128 x 128
// sub-tile (tokens 128 wr.., weight rows 128 wc..) in 256 accumulator
// registers, bf16 MFMA 32x32x16 with fp32 accumulation.  The contraction runs
// in stages of 32 through a ring of five LDS stage buffers (weight half +
// token half, 64-byte rows), filled by buffer->LDS DMA three and four stages
// ahead, in pairs of stages that cover whole 128-byte lines; one barrier per
// stage.
#include "gemm_common.h"

namespace qlora {
namespace {

constexpr int kDRing = 5;                               // stage s in ring slot s mod 5
constexpr size_t kLdsDense = (size_t)kDRing * kStage;   // 160 KiB
constexpr int kDGroup = 4;                              // token tiles per tile group (tile order)

// Tile order of the dense GEMMs.  The eight XCDs receive contiguous ranges of
// tile ids (the hardware hands workgroups to XCDs round robin); ids run over
// groups of kDGroup token tiles, each group column-tile-major, so that the
// tiles one XCD holds at a time share a few token tiles and a few weight
// tiles and both stream through its L2.
__device__ __forceinline__ void map_tile_grouped(int tiles_c, int tiles_r, int& tc, int& tr) {
  const int nwg = (int)gridDim.x;
  int id = blockIdx.x;
  if ((nwg & 7) == 0) id = (id & 7) * (nwg >> 3) + (id >> 3);
  const int per_group = kDGroup * tiles_c;
  const int g = id / per_group, first = g * kDGroup;
  const int size = min(kDGroup, tiles_r - first);
  const int local = id - g * per_group;
  tr = first + local % size;
  tc = local / size;
}

struct DenseOps {
  rsrc_t wr_, xr;           // weight rows, token rows
  uint32_t wo[4], xo[4];    // lane offsets of the four DMA instructions per operand (stage 0)
  int nsub, w;
};

// Stage `stage` of both operands into ring slot `slot`: DMA instruction q of
// wave w fills tile rows 64 q + 16 w .. +15 (lane j: row + (j >> 2), holding
// chunk dma_chunk(j) at position j & 3).  Past the last stage the last one
// is re-loaded (never read).
__device__ __forceinline__ void dense_dma(char* smem, const DenseOps& f, int stage, int slot) {
  const uint32_t soff = (uint32_t)min(stage, f.nsub - 1) * 64u;
  char* dst = smem + slot * kStage + 16 * f.w * 64;
#pragma unroll
  for (int q = 0; q < 4; ++q) dma16(f.wr_, dst + 64 * q * 64, f.wo[q], soff);
#pragma unroll
  for (int q = 0; q < 4; ++q) dma16(f.xr, dst + kOp + 64 * q * 64, f.xo[q], soff);
}

// MFMA slot X (0..31) of substep s (stage s at cur, s+1 at nxt; stage
// s+3 and s+4 go to fill0 and fill1): X = 16 kk + 4 i + j is fragment pair (i, j) of
// k16 step kk.  The LDS reads and the DMAs are spread one per two slots, so
// that the four waves (which leave each barrier together) do not queue their
// reads on the LDS at once:
//   LDS reads   read q (fragments A0, B0, B1, B2, B3, A1, A2, A3 in that
//               order) in slot 2 q: step 1 of stage s; in slot 16 + 2 q: step
//               0 of stage s+1, into the registers step 0 of stage s has
//               finished with.  The MFMA of slot 16 + 4 i + j uses read
//               max(i + 4 [i > 0], 1 + j), issued at least ten slots before.
//   DMA         odd substeps only, odd slots: stages s+3 and s+4, the two
//               halves of the same 128-byte lines (a stage is 64 bytes of a
//               row), one after the other, so that the second request of a
//               line meets the first one's pending miss in the L1 instead of
//               going to L2 again: slot 4 q + 1 and 4 q + 3 are instruction
//               q (four weight-row, then four token-row) of stage s+3 and of
//               stage s+4.
template <int X, bool ODD>
__device__ __forceinline__ void fwd_dense_slot(const char* cur, const char* nxt, char* fill0, char* fill1,
                                               const DenseOps& f, int s, f32x16_t (&acc)[4][4], Frags& F, int am,
                                               int bm, FragOffs fo) {
  constexpr int kk = X >> 4, i = (X >> 2) & 3, j = X & 3, y = X & 15;
  if constexpr (kk == 0)
    acc[i][j] = mfma32x32x16(F.a0[i], F.b0[j], acc[i][j]);
  else
    acc[i][j] = mfma32x32x16(F.a1[i], F.b1[j], acc[i][j]);
  if constexpr ((y & 1) == 0) {
    constexpr int q = y >> 1;                               // read 0..7
    constexpr bool isA = q == 0 || q >= 5;
    constexpr int fr = q == 0 ? 0 : q >= 5 ? q - 4 : q - 1;   // fragment index
    const char* base = (kk == 0 ? cur : nxt) + (isA ? am : kOp + bm) + fr * 2048;
    const int o = kk == 0 ? fo.o1 : fo.o0;
    if constexpr (isA) {
      if constexpr (kk == 0) F.a1[fr] = rd16(base + o); else F.a0[fr] = rd16(base + o);
    } else {
      if constexpr (kk == 0) F.b1[fr] = rd16(base + o); else F.b0[fr] = rd16(base + o);
    }
  }
  if constexpr (ODD && (X & 1)) {
    constexpr int q = X >> 2, second = (X >> 1) & 1;   // instruction 0..7, stage s+3 or s+4
    const uint32_t soff = (uint32_t)min(s + 3 + second, f.nsub - 1) * 64u;
    char* dst = (second ? fill1 : fill0) + (q >= 4 ? kOp : 0) + (64 * (q & 3) + 16 * f.w) * 64;
    if constexpr (q < 4)
      dma16(f.wr_, dst, f.wo[q], soff);
    else
      dma16(f.xr, dst, f.xo[q - 4], soff);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// One barrier per substep.  Before it, this wave's DMAs of stage s+1 must
// have landed: at an even substep (stage s+1 was DMA'd three substeps ago)
// only the sixteen DMAs of the last odd substep may still be in flight; at an
// odd one (stage s+1 DMA'd two substeps ago, interleaved with stage s+2) only
// the last DMA, of stage s+2.  The barrier then makes stage s+1 visible to
// every wave and certifies that every wave has finished reading stage s-1,
// whose slot (with stage s-2's) an odd substep refills.  Stage t sits in ring
// slot t mod 5; sl is stage s's.
template <bool ODD>
__device__ __forceinline__ void fwd_dense_substep(char* smem, const DenseOps& f, int s, int sl,
                                                  f32x16_t (&acc)[4][4], Frags& F, int am, int bm, FragOffs fo) {
  auto slot = [](int v) { return v >= kDRing ? v - kDRing : v; };
  const char* cur = smem + sl * kStage;
  const char* nxt = smem + slot(sl + 1) * kStage;
  char* fill0 = smem + slot(sl + 3) * kStage;
  char* fill1 = smem + slot(sl + 4) * kStage;
  __builtin_amdgcn_sched_barrier(0);
  QLORA_WAIT(ODD ? 1 : 16, 0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
#define QLORA_FD_SLOT(x) fwd_dense_slot<x, ODD>(cur, nxt, fill0, fill1, f, s, acc, F, am, bm, fo)
#define QLORA_FD_SLOT4(x) QLORA_FD_SLOT(x); QLORA_FD_SLOT(x + 1); QLORA_FD_SLOT(x + 2); QLORA_FD_SLOT(x + 3)
  QLORA_FD_SLOT4(0); QLORA_FD_SLOT4(4); QLORA_FD_SLOT4(8); QLORA_FD_SLOT4(12);
  QLORA_FD_SLOT4(16); QLORA_FD_SLOT4(20); QLORA_FD_SLOT4(24); QLORA_FD_SLOT4(28);
#undef QLORA_FD_SLOT4
#undef QLORA_FD_SLOT
}

// Weight half of the LoRA tail: B'[row0 + row, j0 + 8 c ..] into a 64-byte-row
// tile (zero past the rank and past the last row), where B' is B [rows x r]
// or, with b_trans, the transpose of B [r x rows] (read column-wise).
__device__ __forceinline__ void tail_rows(char* dst, const bf16_t* Bm, bool b_trans, int64_t rows, int r,
                                          int64_t row0, int j0) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int idx = threadIdx.x + kThreads * e;
    const int row = idx >> 2, c = idx & 3, col = j0 + 8 * c;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (col < r && row0 + row < rows) {
      if (!b_trans) {
        v = *reinterpret_cast<const uint4*>(Bm + (row0 + row) * r + col);
      } else {
        const bf16_t* p = Bm + (int64_t)col * rows + row0 + row;
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = (uint32_t)p[2 * q * rows] | ((uint32_t)p[(2 * q + 1) * rows] << 16);
        v = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
    wr16(dst + spos(row, c), v);
  }
}

__global__ __launch_bounds__(kThreads, 1) void bf16_fwd_kernel(const bf16_t* __restrict__ Wd, int64_t N, int64_t K,
                                                               const bf16_t* __restrict__ X, int64_t M,
                                                               const bf16_t* __restrict__ U,
                                                               const bf16_t* __restrict__ Bl, int b_trans, int r,
                                                               float s, bf16_t* __restrict__ Y, int tiles_n,
                                                               int tiles_m) {
  extern __shared__ __align__(16) char smem[];
  int tn, tm;
  map_tile_grouped(tiles_n, tiles_m, tn, tm);
  const int64_t n0 = (int64_t)tn * kTile, m0 = (int64_t)tm * kTile;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6, wr = wv >> 1, wc = wv & 1;

  DenseOps f;
  f.w = __builtin_amdgcn_readfirstlane(wv);
  __builtin_assume(f.w >= 0 && f.w < 4);
  f.nsub = (int)(K >> 5);
  f.wr_ = make_rsrc(Wd, (uint32_t)(N * K * 2));
  f.xr = make_rsrc(X, (uint32_t)(M * K * 2));
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    // rows past the end re-read the last row: finite data, never stored
    const int row = dma_row(q, f.w, lane);
    f.wo[q] = (uint32_t)(min(n0 + row, N - 1) * K * 2 + dma_chunk(lane) * 16);
    f.xo[q] = (uint32_t)(min(m0 + row, M - 1) * K * 2 + dma_chunk(lane) * 16);
  }
  const FragOffs fo = frag_offs(lane);
  const int am = wc * 128 * 64, bm = wr * 128 * 64;

  f32x16_t acc[4][4];
  zero_acc(acc);

  // stages 0..3 in slots 0..3; substep 1 starts the pairs (4, 5)
#pragma unroll
  for (int st = 0; st < 4; ++st) dense_dma(smem, f, st, st);
  QLORA_WAIT(0, 0);
  __builtin_amdgcn_s_barrier();
  Frags F;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    F.a0[i] = rd16(smem + am + i * 2048 + fo.o0);
    F.b0[i] = rd16(smem + kOp + bm + i * 2048 + fo.o0);
  }
  // K % 64 == 0: the stage count is even
  int sl = 0;
  for (int st = 0; st < f.nsub; st += 2) {
    fwd_dense_substep<false>(smem, f, st, sl, acc, F, am, bm, fo);
    sl = sl + 1 == kDRing ? 0 : sl + 1;
    fwd_dense_substep<true>(smem, f, st + 1, sl, acc, F, am, bm, fo);
    sl = sl + 1 == kDRing ? 0 : sl + 1;
  }
  // drain the DMAs still in flight (clamped re-loads) before reusing the ring
  QLORA_WAIT(0, 0);
  __builtin_amdgcn_s_barrier();

  if (r > 0) {
    // acc += B (s U)^T over the rank, 32 at a time
    for (int j0 = 0; j0 < r; j0 += 32) {
      tail_rows(smem, Bl, b_trans != 0, N, r, n0, j0);
      tail_tokens(smem + kOp, U, M, r, m0, j0, s);
      QLORA_WAIT(0, 0);
      __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int o = kk ? fo.o1 : fo.o0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          F.a0[i] = rd16(smem + am + i * 2048 + o);
          F.b0[i] = rd16(smem + kOp + bm + i * 2048 + o);
        }
        mfma_block<4, 4>(acc, F.a0, F.b0);
      }
      QLORA_WAIT(0, 0);
      __builtin_amdgcn_s_barrier();
    }
  }
  store_tile<4>(acc, Y, N, M, N, m0, n0);
}

}  // namespace

hipError_t launch_bf16_fwd(const bf16_t* Wd, int64_t N, int64_t K, const bf16_t* X, int64_t M, const bf16_t* U,
                           const bf16_t* B, bool b_trans, int r, float s, bf16_t* Y, hipStream_t st) {
  const int tiles_n = (int)((N + kTile - 1) / kTile);
  const int tiles_m = (int)((M + kTile - 1) / kTile);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bf16_fwd_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsDense);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bf16_fwd_kernel, dim3(tiles_n * tiles_m), dim3(kThreads), kLdsDense, st, Wd, N, K, X, M, U, B,
                     (int)b_trans, r, s, Y, tiles_n, tiles_m);
  return hipGetLastError();
}

}  // namespace qlora
