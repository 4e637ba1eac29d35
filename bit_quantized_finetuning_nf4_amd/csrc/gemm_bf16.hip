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
// in pairs of 32-wide stages: a pair (64 columns: one 128-byte line of every
// row) comes into one of two LDS pair slots by buffer->LDS DMA, each
// instruction moving 8 whole rows, one pair ahead; one barrier per pair.
//
//   dX        the same kernel on deq(W)^T: dX = dY (W^T)^T + s G (A^T)^T,
//             with A read column-wise in the LoRA tail;
//   groups    weight rows in groups of gn, each with its own adapter (the
//             stacked q/k/v or gate/up weights of one layer).
#include <algorithm>

#include "gemm_common.h"

namespace qlora {
namespace {

constexpr int kPairOp = kTile * 128;                    // 32 KiB: 256 rows x 64 bf16 (two stages)
constexpr int kPairSlot = 2 * kPairOp;                  // weight rows at 0, token rows at kPairOp
constexpr size_t kLdsPairs = 2 * (size_t)kPairSlot;     // 128 KiB: two pair slots
constexpr size_t kLdsDense = kLdsPairs + 2 * kOp;       // + 32 KiB: the first LoRA tail chunk
constexpr int kDGroup = 4;                              // token tiles per tile group (tile order)

// Pair slots hold two consecutive 32-wide stages (one 64-wide stage): rows of
// 128 bytes, 16-byte chunk c of row r at position c ^ ((r >> 1) & 7), so the
// 16 lanes of one read quarter (16 consecutive rows, one chunk) and a DMA
// instruction's 64 lanes (8 whole rows) cover all 64 LDS banks.  Chunks
// 0..3 are the even stage, 4..7 the odd one.
__device__ __forceinline__ int pos128(int r, int c) { return r * 128 + 16 * (c ^ ((r >> 1) & 7)); }

// Tile order of the dense GEMMs.  The eight XCDs receive contiguous ranges of
// tile ids (the hardware hands workgroups to XCDs round robin); ids run over
// groups of kDGroup token tiles, each group column-tile-major, so that the
// tiles one XCD holds at a time share a few token tiles and a few weight
// tiles and both stream through its L2.
// With the contraction split, ids run split-major: the tiles of one split
// (which share its column range of both operands) sit on the same XCDs.
__device__ __forceinline__ int xcd_tile_id() {
  const int nwg = (int)gridDim.x;
  int id = blockIdx.x;
  if ((nwg & 7) == 0) id = (id & 7) * (nwg >> 3) + (id >> 3);
  return id;
}
// With 16 token tiles or more a group holds 8 of them, so each weight tile
// streams through an XCD's L2 half as often (the weight is the larger
// operand of these products): at 4096 tokens the 65B products ran 1.4 %
// faster than with 4; at 2048 tokens (8 token tiles) 4 stays slightly ahead.
__device__ __forceinline__ void map_tile_grouped(int id, int tiles_c, int tiles_r, int& tc, int& tr) {
  const int grp = tiles_r >= 16 ? 2 * kDGroup : kDGroup;
  const int per_group = grp * tiles_c;
  const int g = id / per_group, first = g * grp;
  const int size = min(grp, tiles_r - first);
  const int local = id - g * per_group;
  tr = first + local % size;
  tc = local / size;
}

struct DenseOps {
  rsrc_t wr_, xr;           // weight rows, token rows
  uint32_t wo[8], xo[8];    // lane offsets of the eight DMA instructions per operand (pair 0)
  int npair, w;
};

// DMA of pair `pair` (64 columns of every row) of both operands into pair
// slot `dst`: weight instruction q < 2 FI and token instruction q < 8 of
// wave w fill rows 8 (4 q + w) .. +7 of their tile, 128 bytes each (lane j:
// row + (j >> 3), position j & 7).  DMA d of a pair is weight instruction d
// for d < 2 FI, token instruction d - 2 FI after.  Past the last pair the last
// one is re-loaded (never read).
template <int FI>
__device__ __forceinline__ void pair_dma(char* dst, const DenseOps& f, int pair, int d) {
  const uint32_t soff = (uint32_t)min(pair, f.npair - 1) * 128u;
  const bool wrow = d < 2 * FI;
  const int q = wrow ? d : d - 2 * FI;
  char* dd = dst + (wrow ? 0 : kPairOp) + 8 * (4 * q + f.w) * 128;
  if (wrow)
    dma16(f.wr_, dd, f.wo[q], soff);
  else
    dma16(f.xr, dd, f.xo[q], soff);
}

// Read offsets of the lane within a pair slot: stage half hf, k16 step kk ->
// chunk 4 hf + 2 kk + h of row lr.
struct PairOffs {
  int o[2][2];
};

// MFMA slot X (0 .. 8 FI - 1) of substep s: X = 4 FI kk + 4 i + j is
// fragment pair (i, j) of k16 step kk (FI weight fragments of 32 rows, four
// token fragments).  Stage s is half HF of the pair slot at cur; stage s+1 is
// the other half of cur (HF = 0) or half 0 of the next slot (HF = 1).
//   LDS reads   read q (fragments A0, B0, B1, B2, B3, A1, .., A(FI-1) in
//               that order) in slot rd_slot(q): step 1 of stage s; in slot
//               4 FI + rd_slot(q): step 0 of stage s+1, into the registers
//               step 0 of stage s has finished with.
//   barrier     odd substeps, before slot 4 FI: this wave's DMAs of the next
//               pair have landed and its reads of this pair have completed;
//               after it the next pair is visible to every wave and no wave
//               reads this pair's slot any more.
//   DMA         the pair after next into this pair's slot (2 FI weight-row,
//               then 8 token-row instructions of 8 whole 128-byte rows each):
//               the first FI + 4 in the odd substep's slots 4 FI .., every
//               other slot; the other FI + 4 in the next pair's even substep,
//               one every fourth slot.  Issued all in the odd substep's
//               second half, 16 instructions per wave in 16 MFMA slots
//               overran the texture address queue (its FIFO full about 10 %
//               of the cycles) and stalled issue; split, the product ran
//               about 7 % faster.
template <int FI>
constexpr int rd_slot(int q) { return q * 4 * FI / (FI + 4); }
template <int FI>
constexpr int dma_half = FI + 4;   // DMAs of a pair issued in its odd substep
template <int FI>
constexpr int dma_slot_a(int d) { return 4 * FI + d * 4 * FI / dma_half<FI>; }
template <int FI>
constexpr int dma_slot_b(int d) { return (d - dma_half<FI>) * 8 * FI / dma_half<FI>; }

template <int FI, int X, int HF>
__device__ __forceinline__ void dense_slot(const char* cur, const char* nxt, char* fill, const DenseOps& f,
                                           int pair, f32x16_t (&acc)[FI][4], Frags& F, int am, int bm,
                                           const PairOffs& po) {
  constexpr int H = 4 * FI;   // slots per k16 step
  constexpr int kk = X / H, y = X % H, i = y >> 2, j = y & 3;
  if constexpr (HF == 1 && X == H) {
    QLORA_WAIT(0, 0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (kk == 0)
    acc[i][j] = mfma32x32x16(F.a0[i], F.b0[j], acc[i][j]);
  else
    acc[i][j] = mfma32x32x16(F.a1[i], F.b1[j], acc[i][j]);
#pragma unroll
  for (int q = 0; q < FI + 4; ++q) {
    if (rd_slot<FI>(q) != y) continue;
    const bool isA = q == 0 || q >= 5;
    const int fr = q == 0 ? 0 : q >= 5 ? q - 4 : q - 1;   // fragment index
    // step 1 of stage s (half HF of cur), or step 0 of stage s+1
    const char* slot = kk == 0 ? cur : (HF == 0 ? cur : nxt);
    const int o = kk == 0 ? po.o[HF][1] : po.o[HF ^ 1][0];
    const char* base = slot + (isA ? am : kPairOp + bm) + fr * 32 * 128 + o;
    if (isA) {
      if (kk == 0) F.a1[fr] = rd16(base); else F.a0[fr] = rd16(base);
    } else {
      if (kk == 0) F.b1[fr] = rd16(base); else F.b0[fr] = rd16(base);
    }
  }
  if constexpr (HF == 1 && kk == 1) {
#pragma unroll
    for (int d = 0; d < dma_half<FI>; ++d)
      if (dma_slot_a<FI>(d) == X) pair_dma<FI>(fill, f, pair + 2, d);
  }
  if constexpr (HF == 0) {
    // the rest of pair + 1's DMAs into nxt, which no wave reads before the
    // barrier of this pair (in the first pair they re-load what the
    // prologue loaded: the same bytes to the same place)
#pragma unroll
    for (int d = dma_half<FI>; d < 2 * FI + 8; ++d)
      if (dma_slot_b<FI>(d) == X) pair_dma<FI>(const_cast<char*>(nxt), f, pair + 1, d);
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <int FI, int HF, int X>
__device__ __forceinline__ void dense_slots(const char* cur, const char* nxt, char* fill, const DenseOps& f,
                                            int pair, f32x16_t (&acc)[FI][4], Frags& F, int am, int bm,
                                            const PairOffs& po) {
  if constexpr (X < 8 * FI) {
    dense_slot<FI, X, HF>(cur, nxt, fill, f, pair, acc, F, am, bm, po);
    dense_slots<FI, HF, X + 1>(cur, nxt, fill, f, pair, acc, F, am, bm, po);
  }
}

// One 32-wide chunk of the LoRA tail, in registers: the weight half
// B'[row0 + row, j0 ..] (zero past the rank, and for rows outside [lo, hi))
// and the token half T[trow0 + row, j0 + 8 c ..] (T is trows x rank with
// row stride ld; zero past the rank and the last row).  Token half: thread t
// holds row (t + 256 e) >> 2, 16-byte chunk (t + 256 e) & 3.  Weight half:
// B' is B [rows x r], held like the tokens; or, with b_trans, the transpose
// of B [r x rows], read along its rows (coalesced): thread t holds B[j0 +
// (i >> 5)][row0 + 8 (i & 31) ..] for i = t + 256 e.
struct TailRegs {
  uint4 w[4], t[4];
};
__device__ __forceinline__ void tail_load(TailRegs& R, const bf16_t* Bm, bool b_trans, int64_t rows, int r,
                                          int64_t row0, int j0, int64_t lo, int64_t hi, const bf16_t* T,
                                          int64_t ld, int64_t trows, int64_t trow0) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int idx = threadIdx.x + kThreads * e;
    const int row = idx >> 2, c = idx & 3, col = j0 + 8 * c;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (!b_trans) {
      if (col < r && row0 + row >= lo && row0 + row < hi)
        v = *reinterpret_cast<const uint4*>(Bm + (row0 + row) * r + col);
    } else {
      // rows % 8 == 0 and lo, hi multiples of 8: the 8 rows are all in or all out
      const int j = j0 + (idx >> 5);
      const int64_t rr = row0 + 8 * (idx & 31);
      if (j < r && rr >= lo && rr < hi) v = *reinterpret_cast<const uint4*>(Bm + (int64_t)j * rows + rr);
    }
    R.w[e] = v;
    uint4 u = make_uint4(0u, 0u, 0u, 0u);
    if (col < r && trow0 + row < trows) u = *reinterpret_cast<const uint4*>(T + (trow0 + row) * ld + col);
    R.t[e] = u;
  }
}
// The chunk into LDS: s T as a 64-byte-row tile at dst + kOp; the weights
// at dst, as a 64-byte-row tile or, with b_trans, as a tile of 32 rank rows
// x 256 weight rows (512-byte rows, 32-byte block b of rank row n at
// b ^ (n & 3)) for transposed fragment reads.
__device__ __forceinline__ void tail_store(char* dst, const TailRegs& R, bool b_trans, float s) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int idx = threadIdx.x + kThreads * e;
    const int row = idx >> 2, c = idx & 3;
    if (!b_trans) {
      wr16(dst + spos(row, c), R.w[e]);
    } else {
      const int n = idx >> 5, sg = idx & 31;
      wr16(dst + n * 512 + 32 * ((sg >> 1) ^ (n & 3)) + 16 * (sg & 1), R.w[e]);
    }
    wr16(dst + kOp + spos(row, c), scale16(R.t[e], s));
  }
}

// The LoRA tail by DMA, for tiles inside one adapter group with the rank in
// whole 32-wide chunks.  A chunk takes 32 KiB of LDS in the layouts of
// tail_store, but the token half holds T itself (unscaled): s is applied to
// each fragment as it is read, which rounds exactly as tail_store does.
struct TailSrc {
  rsrc_t wr, tr;         // weight half (B, or A with b_trans), token half (T)
  int64_t n0, m0, rows;  // first weight row, first token row, weight rows (N)
  int r, ld, col0;       // rank, T's row stride, T's first column (the group's)
  bool bt;
};
// DMA of chunk c (ranks 32 c ..) into dst: per wave 4 token and 4 weight
// instructions of 1 KiB.  Token rows / weight rows (no b_trans): the
// 256-row x 64-byte pattern of dma_row / dma_chunk.  With b_trans: rank rows
// n = 2 (4 w + q) + (lane >> 5) of 512 bytes, lane position pc = lane & 31
// holding 32-byte block (pc >> 1) ^ (n & 3), half pc & 1.  Rows past the
// arrays read zero (buffer range) or another row's finite values, which only
// reach outputs past M or N.
__device__ __forceinline__ void tail_dma(char* dst, const TailSrc& S, int c, int w, int lane) {
  const int j0 = 32 * c;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = dma_row(q, w, lane), ch = dma_chunk(lane);
    dma16(S.tr, dst + kOp + (64 * q + 16 * w) * 64,
          (uint32_t)(((S.m0 + row) * S.ld + S.col0 + j0 + 8 * ch) * 2), 0u);
    if (!S.bt) {
      dma16(S.wr, dst + (64 * q + 16 * w) * 64, (uint32_t)(((S.n0 + row) * S.r + j0 + 8 * ch) * 2), 0u);
    } else {
      const int n = 2 * (4 * w + q) + (lane >> 5), pc = lane & 31;
      const int e = 8 * (2 * ((pc >> 1) ^ (n & 3)) + (pc & 1));
      dma16(S.wr, dst + 1024 * (4 * w + q), (uint32_t)(((int64_t)(j0 + n) * S.rows + S.n0 + e) * 2), 0u);
    }
  }
}
__device__ __forceinline__ bf16x8_t scale_frag(bf16x8_t v, float s) {
  return __builtin_bit_cast(bf16x8_t, scale16(__builtin_bit_cast(uint4, v), s));
}

// fp32 sums of the tile (the lane layout of store_tile_lds): lane (lr, h) of
// wave (wr, wc) holds token row0 + 128 wr + 32 j + lr, columns col0 + 32 FI
// wc + 32 i + 8 q + 4 h + 0..3, stored as one 16-byte piece (cols % 4 == 0).
template <int FI>
__device__ __forceinline__ void store_tile_f32(const f32x16_t (&acc)[FI][4], float* out, int64_t ld, int64_t rows,
                                               int64_t cols, int64_t row0, int64_t col0) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wr = w >> 1, wc = w & 1, lr = lane & 31, h = lane >> 5;
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t row = row0 + 128 * wr + 32 * j + lr;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t col = col0 + 32 * FI * wc + 32 * i + 8 * q + 4 * h;
        if (row < rows && col < cols)
          *reinterpret_cast<float4*>(out + row * ld + col) =
              make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
      }
    }
}

// FI: weight fragments per wave, so the tile is 64 FI weight rows x 256
// tokens (FI = 4, 3 or 2); its tiles start at weight row n_begin.
// Split contraction (part != null): the grid holds the tiles once per split;
// split p takes contraction pairs p pps .. (64-column pairs), split 0 alone
// adds the LoRA tail, and each split stores its fp32 sums at part + p M N
// ([M x N], row stride N) instead of Y.
template <int FI, bool TD>
__global__ __launch_bounds__(kThreads, 1) void bf16_fwd_kernel(const bf16_t* __restrict__ Wd, int64_t N, int64_t K,
                                                               const bf16_t* __restrict__ X, int64_t M,
                                                               const bf16_t* __restrict__ U,
                                                               const bf16_t* __restrict__ Bl, int b_trans, int r,
                                                               int ldu, int64_t gn, float s, bf16_t* __restrict__ Y,
                                                               int64_t n_begin, int tiles_n, int tiles_m, int pps,
                                                               float* __restrict__ part) {
  extern __shared__ __align__(16) char smem[];
  int tn, tm;
  int id = xcd_tile_id();
  const int split = id / (tiles_n * tiles_m);
  map_tile_grouped(id - split * tiles_n * tiles_m, tiles_n, tiles_m, tn, tm);
  const int64_t n0 = n_begin + (int64_t)tn * 64 * FI, m0 = (int64_t)tm * kTile;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6, wr = wv >> 1, wc = wv & 1;

  DenseOps f;
  f.w = __builtin_amdgcn_readfirstlane(wv);
  __builtin_assume(f.w >= 0 && f.w < 4);
  const int p0 = split * pps;
  f.npair = min((int)(K >> 6) - p0, pps);
  f.wr_ = make_rsrc(Wd, (uint32_t)(N * K * 2));
  f.xr = make_rsrc(X, (uint32_t)(M * K * 2));
  {
    // lane j of DMA instruction q: row 8 (4 q + w) + (j >> 3), position j & 7
    // holding chunk (j & 7) ^ ((row >> 1) & 7) = (j & 7) ^ ((4 w + (j >> 4)) & 7)
    const int c = (lane & 7) ^ ((4 * f.w + (lane >> 4)) & 7);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      // rows past the end re-read the last row: finite data, never stored
      const int row = 8 * (4 * q + f.w) + (lane >> 3);
      if (q < 2 * FI) f.wo[q] = (uint32_t)(min(n0 + row, N - 1) * K * 2 + p0 * 128 + c * 16);
      f.xo[q] = (uint32_t)(min(m0 + row, M - 1) * K * 2 + p0 * 128 + c * 16);
    }
  }
  PairOffs po;
  {
    const int lr = lane & 31, h = lane >> 5;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) po.o[hf][kk] = pos128(lr, 4 * hf + 2 * kk + h);
  }
  const int am = wc * 32 * FI * 128, bm = wr * 128 * 128;

  f32x16_t acc[FI][4];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // TD: the LoRA tail by DMA (the launch checked that the rank comes in whole
  // chunks, that no tile straddles two adapter groups and that the side
  // arrays fit 32-bit byte offsets); otherwise through registers
  const int64_t g0 = n0 / gn;
  const bool tail = r > 0 && split == 0;
  const bool tdma = TD && tail;
  // (built where used, so nothing of it stays live through the main loop)
  auto tail_src = [&]() __attribute__((always_inline)) {
    TailSrc ts;
    ts.wr = make_rsrc(Bl, (uint32_t)(N * r * 2));
    ts.tr = make_rsrc(U, (uint32_t)(M * ldu * 2));
    ts.n0 = n0;
    ts.m0 = m0;
    ts.rows = N;
    ts.r = r;
    ts.ld = ldu;
    ts.col0 = (int)(g0 * r);
    ts.bt = b_trans != 0;
    return ts;
  };
  if (tdma) tail_dma(smem + kLdsPairs, tail_src(), 0, f.w, lane);   // chunk 0 past the pair slots
  // pairs 0 and 1 into slots 0 and 1
#pragma unroll
  for (int d = 0; d < 2 * FI + 8; ++d) {
    pair_dma<FI>(smem, f, 0, d);
    pair_dma<FI>(smem + kPairSlot, f, 1, d);
  }
  QLORA_WAIT(0, 0);
  __builtin_amdgcn_s_barrier();
  Frags F;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < FI) F.a0[i] = rd16(smem + am + i * 32 * 128 + po.o[0][0]);
    F.b0[i] = rd16(smem + kPairOp + bm + i * 32 * 128 + po.o[0][0]);
  }
  // K % 64 == 0: whole pairs of 32-wide stages
  for (int pr = 0; pr < f.npair; ++pr) {
    char* cur = smem + (pr & 1) * kPairSlot;
    char* nxt = smem + ((pr & 1) ^ 1) * kPairSlot;
    __builtin_amdgcn_sched_barrier(0);
    dense_slots<FI, 0, 0>(cur, nxt, cur, f, pr, acc, F, am, bm, po);
    __builtin_amdgcn_sched_barrier(0);
    dense_slots<FI, 1, 0>(cur, nxt, cur, f, pr, acc, F, am, bm, po);
  }
  // drain the DMAs still in flight (clamped re-loads) before reusing LDS
  QLORA_WAIT(0, 0);
  __builtin_amdgcn_s_barrier();

  const FragOffs fo = frag_offs(lane);
  const int am64 = wc * 32 * FI * 64, bm64 = wr * 128 * 64;
  // acc += the chunk at buf (weights at buf, tokens at buf + kOp); the tokens
  // are scaled by s as they are read when `raw`
  auto tail_chunk = [&](const char* buf, bool raw) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int o = kk ? fo.o1 : fo.o0;
      if (b_trans) {
        // transposed reads in asm blocks, so that the DMAs of later chunks
        // stay in flight (see tr_read2)
        const char* tb = buf + kk * 16 * 512;
        const int f0 = wc * FI;
        if constexpr (FI == 3) {
          tr_read3<2048, 2048, 2048>(tb + tr_off<512>(f0), tb + tr_off<512>(f0 + 1), tb + tr_off<512>(f0 + 2), F.a0[0],
                                     F.a0[1], F.a0[2]);
        } else {
#pragma unroll
          for (int i = 0; i < FI; i += 2)
            tr_read2<2048, 2048>(tb + tr_off<512>(f0 + i), tb + tr_off<512>(f0 + i + 1), F.a0[i], F.a0[i + 1]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < FI; ++i) F.a0[i] = rd16(buf + am64 + i * 2048 + o);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8_t b = rd16(buf + kOp + bm64 + i * 2048 + o);
        F.b0[i] = raw ? scale_frag(b, s) : b;
      }
#pragma unroll
      for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32x32x16(F.a0[i], F.b0[j], acc[i][j]);
    }
  };
  if constexpr (TD) {
    if (tdma) {
      // chunk 0 landed before the drain above; chunks 1 .. go four at a time
      // into the pair slots, the first four while chunk 0 is multiplied
      const TailSrc ts = tail_src();
      const int nt = r / 32;
      int b0 = 1, bn = min(4, nt - 1);
      for (int c = 0; c < bn; ++c) tail_dma(smem + c * 2 * kOp, ts, b0 + c, f.w, lane);
      tail_chunk(smem + kLdsPairs, true);
      while (bn > 0) {
        QLORA_WAIT(0, 0);
        __builtin_amdgcn_s_barrier();
        for (int c = 0; c < bn; ++c) tail_chunk(smem + c * 2 * kOp, true);
        b0 += bn;
        bn = min(4, nt - b0);
        if (bn > 0) {
          QLORA_WAIT(0, 0);
          __builtin_amdgcn_s_barrier();   // every wave is done with the batch's slots
          for (int c = 0; c < bn; ++c) tail_dma(smem + c * 2 * kOp, ts, b0 + c, f.w, lane);
        }
      }
    }
  } else if (tail) {
    // acc += B (s U)^T over the rank, 32 at a time, through 64-byte-row tiles.
    // Weight rows come in groups of gn, each with its own adapter: rows of
    // group g take columns g r .. of U (row stride ldu) and their rows of B;
    // a tile that straddles groups runs the tail once per group, with the
    // other groups' rows zero.  Chunks alternate between two tile pairs:
    // chunk c + 1 is loaded into registers while chunk c is multiplied, and
    // one barrier per chunk both publishes a chunk and retires the buffer
    // the next store overwrites (its readers finished before they stored
    // their part of the chunk in between).
    const int64_t g_last = (min(n0 + 64 * FI, N) - 1) / gn;
    const int nj = (r + 31) / 32;
    const int nt = (int)(g_last - g0 + 1) * nj;
    TailRegs R;
    auto load = [&](int t) {
      const int64_t g = g0 + t / nj;
      tail_load(R, Bl, b_trans != 0, N, r, n0, 32 * (t % nj), g * gn, min((g + 1) * gn, N), U + g * r, ldu, M,
                m0);
    };
    load(0);
    for (int t = 0; t < nt; ++t) {
      char* buf = smem + (t & 1) * 2 * kOp;
      tail_store(buf, R, b_trans != 0, s);
      if (t + 1 < nt) load(t + 1);
      __syncthreads();
      tail_chunk(buf, false);
    }
  }
  if (part != nullptr)
    store_tile_f32<FI>(acc, part + (int64_t)split * M * N, N, M, N, m0, n0);
  else
    store_tile_lds<FI>(acc, Y, N, M, N, m0, n0, smem);
}

}  // namespace

namespace {

// Tiles of 64 FI weight rows over rows [n_begin, n_begin + n_rows) of the
// N-row weight (N is every array's extent and leading dimension).
// Whether the launch's tiles can take the LoRA tail by DMA: the rank in whole
// 32-wide chunks, no tile across two adapter groups, and U (M x ldu) and B
// or A (N x r) within 32-bit byte offsets.
bool tail_by_dma(int64_t N, int64_t M, int r, int ldu, int64_t gn, int64_t n_begin, int tiles_n, int rows) {
  if (r <= 0 || r % 32 != 0 || M * ldu >= ((int64_t)1 << 30) || N * r >= ((int64_t)1 << 30)) return false;
  for (int t = 0; t < tiles_n; ++t) {
    const int64_t lo = n_begin + (int64_t)t * rows, hi = std::min(lo + rows, N) - 1;
    if (lo / gn != hi / gn) return false;
  }
  return true;
}

// splits > 1: the contraction in that many parts of whole 64-column pairs,
// fp32 sums to part (splits x M x N floats), not Y.
template <int FI>
hipError_t launch_fi(const bf16_t* Wd, int64_t N, int64_t K, const bf16_t* X, int64_t M, const bf16_t* U,
                     const bf16_t* B, bool b_trans, int r, int ldu, int64_t gn, float s, bf16_t* Y, int64_t n_begin,
                     int64_t n_rows, hipStream_t st, int splits = 1, float* part = nullptr) {
  const int tiles_n = (int)((n_rows + 64 * FI - 1) / (64 * FI));
  const int tiles_m = (int)((M + kTile - 1) / kTile);
  const bool td = tail_by_dma(N, M, r, ldu, gn, n_begin, tiles_n, 64 * FI);
  auto* fn = td ? &bf16_fwd_kernel<FI, true> : &bf16_fwd_kernel<FI, false>;
  const size_t lds = td ? kLdsDense : kLdsPairs;
  hipError_t e = allow_lds(reinterpret_cast<const void*>(fn), (int)lds);
  if (e != hipSuccess) return e;
  const int npair = (int)(K >> 6);
  const int pps = splits > 1 ? (npair + splits - 1) / splits : npair;
  hipLaunchKernelGGL(fn, dim3(tiles_n * tiles_m * splits), dim3(kThreads), lds, st, Wd, N, K, X, M, U, B,
                     (int)b_trans, r, ldu, gn, s, Y, n_begin, tiles_n, tiles_m, pps, splits > 1 ? part : nullptr);
  return hipGetLastError();
}

// Y [M x N] (bf16) = the sum of the splits' fp32 partials, added in split
// order; four values per thread (N % 4 == 0).
__global__ __launch_bounds__(kThreads) void split_sum_kernel(const float* __restrict__ part, int splits, int64_t n,
                                                             bf16_t* __restrict__ Y) {
  const int64_t i = 4 * ((int64_t)blockIdx.x * kThreads + threadIdx.x);
  if (i >= n) return;
  float4 a = *reinterpret_cast<const float4*>(part + i);
  for (int p = 1; p < splits; ++p) {
    const float4 v = *reinterpret_cast<const float4*>(part + (int64_t)p * n + i);
    a.x += v.x;
    a.y += v.y;
    a.z += v.z;
    a.w += v.w;
  }
  *reinterpret_cast<uint2*>(Y + i) = make_uint2(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w));
}

// Time of weight rows [n_begin, N) in 64 FI-row tiles, in units of one round
// of 256-row tiles: rounds x FI / 4, with a small charge for the narrower
// tiles' extra LDS reads per MFMA.
double tile_cost(int64_t rows, int64_t tiles_m, int fi, int cus) {
  const int64_t tiles = (rows + 64 * fi - 1) / (64 * fi) * tiles_m;
  const double eff = fi == 4 ? 1.0 : fi == 3 ? 1.06 : 1.12;
  return (double)((tiles + cus - 1) / cus) * fi / 4.0 * eff;
}
int best_fi(int64_t rows, int64_t tiles_m, int cus) {
  int best = 4;
  for (int fi = 3; fi >= 2; --fi)
    if (tile_cost(rows, tiles_m, fi, cus) < tile_cost(rows, tiles_m, best, cus)) best = fi;
  return best;
}

hipError_t launch_rows(int fi, const bf16_t* Wd, int64_t N, int64_t K, const bf16_t* X, int64_t M,
                       const bf16_t* U, const bf16_t* B, bool b_trans, int r, int ldu, int64_t gn, float s,
                       bf16_t* Y, int64_t n_begin, hipStream_t st) {
  const int64_t n_rows = N - n_begin;
  if (fi == 3) return launch_fi<3>(Wd, N, K, X, M, U, B, b_trans, r, ldu, gn, s, Y, n_begin, n_rows, st);
  if (fi == 2) return launch_fi<2>(Wd, N, K, X, M, U, B, b_trans, r, ldu, gn, s, Y, n_begin, n_rows, st);
  return launch_fi<4>(Wd, N, K, X, M, U, B, b_trans, r, ldu, gn, s, Y, n_begin, n_rows, st);
}

}  // namespace

// Split contraction.  A shape with at most half as many 256 x 256 tiles as
// CUs, which would otherwise run narrower tiles, and a long contraction runs
// its 256 x 256 tiles twice, each over half the contraction, and adds the
// two fp32 partials: the 7B gate/up dX product (128 tiles, 22016 columns)
// took 411 us on 128-row tiles.  The CU count the size of the partials
// assumes is fixed (256), so that the workspace a caller queries does not
// depend on the device; the launch splits only if it has that room.
constexpr int kSplitCus = 256;
constexpr int64_t kSplitMinK = 16384;
int dense_splits(int64_t N, int64_t K, int64_t M, int cus) {
  const int64_t tiles = ((N + kTile - 1) / kTile) * ((M + kTile - 1) / kTile);
  return (K >= kSplitMinK && N % 4 == 0 && 2 * tiles <= cus) ? 2 : 1;
}

size_t dense_split_bytes(int64_t N, int64_t K, int64_t M) {
  const int sp = dense_splits(N, K, M, kSplitCus);
  return sp > 1 ? (size_t)sp * (size_t)M * (size_t)N * sizeof(float) : 0;
}

// The grid is sized for the CU count.  Weight rows are cut into a part that
// fills whole rounds of 256-row tiles and a remainder, whose tile width (256,
// 192 or 128 rows) minimizes its time; a shape with fewer 256-row tiles than
// CUs is all remainder, or a split contraction (above) when part has room.
hipError_t launch_bf16_group(const bf16_t* Wd, int64_t N, int64_t K, const bf16_t* X, int64_t M, const bf16_t* U,
                             int ldu, const bf16_t* B, bool b_trans, int r, int64_t gn, float s, bf16_t* Y,
                             hipStream_t st, float* part, size_t part_bytes) {
  const int cus = device_cu_count();
  const int64_t tiles_m = (M + kTile - 1) / kTile;
  const int64_t tiles_n = (N + kTile - 1) / kTile;
  const int sp = dense_splits(N, K, M, cus);
  if (sp > 1 && part != nullptr && part_bytes >= (size_t)sp * (size_t)M * (size_t)N * sizeof(float)) {
    hipError_t e = launch_fi<4>(Wd, N, K, X, M, U, B, b_trans, r, ldu, gn, s, Y, 0, N, st, sp, part);
    if (e != hipSuccess) return e;
    const int64_t n = M * N;
    hipLaunchKernelGGL(split_sum_kernel, dim3((unsigned)((n / 4 + kThreads - 1) / kThreads)), dim3(kThreads), 0, st,
                       part, sp, n, Y);
    return hipGetLastError();
  }
  int64_t n_split = 0;   // rows of the whole-round part
  if (tiles_n * tiles_m > cus && cus % tiles_m == 0) {
    const int64_t per_round = cus / tiles_m;   // 256-row column tiles per round
    n_split = std::min(N, (tiles_n * tiles_m / cus) * per_round * kTile);
    if (n_split >= N || tile_cost(N - n_split, tiles_m, best_fi(N - n_split, tiles_m, cus), cus) >=
                            tile_cost(N - n_split, tiles_m, 4, cus))
      n_split = 0;   // nothing left over, or the remainder gains nothing from narrower tiles: one launch
  }
  if (n_split > 0) {
    hipError_t e = launch_fi<4>(Wd, N, K, X, M, U, B, b_trans, r, ldu, gn, s, Y, 0, n_split, st);
    if (e != hipSuccess) return e;
    // the remainder's tiles address rows from n_split on, in the same arrays
    return launch_rows(best_fi(N - n_split, tiles_m, cus), Wd, N, K, X, M, U, B, b_trans, r, ldu, gn, s, Y, n_split,
                       st);
  }
  return launch_rows(best_fi(N, tiles_m, cus), Wd, N, K, X, M, U, B, b_trans, r, ldu, gn, s, Y, 0, st);
}

hipError_t launch_bf16_fwd(const bf16_t* Wd, int64_t N, int64_t K, const bf16_t* X, int64_t M, const bf16_t* U,
                           const bf16_t* B, bool b_trans, int r, float s, bf16_t* Y, hipStream_t st, float* part,
                           size_t part_bytes) {
  return launch_bf16_group(Wd, N, K, X, M, U, r, B, b_trans, r, N, s, Y, st, part, part_bytes);
}

}  // namespace qlora
