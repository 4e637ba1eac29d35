// gemm_nf4.hip -- the two fused NF4 GEMMs of the QLoRA linear layer.
//
//   forward   Y  = X deq(W)^T + s U B^T     (U = X A^T)
//   backward  dX = dY deq(W) + s G A        (G = dY B)
//
// deepfa.ir blog, "QLoRA's Working Process": the 4-bit weights are converted
// to BF16 on the fly in the forward and backward passes; "LoRA:
// Prerequisite": the adapter adds a low-rank product to the frozen weight.
//
// Both kernels: 256 threads (4 waves), 256 x 256 output tile, each wave a
// 128 x 128 sub-tile held in 256 accumulator registers, bf16 MFMA 32x32x16
// with fp32 accumulation, contraction in steps of 64 with two LDS buffers.
// While the MFMAs of step s run, the producers fill the other buffer for
// step s+1: the NF4 codes of step s+1 (loaded two steps ahead) are
// dequantized into LDS between the MFMA groups, and the token-side tile of
// step s+1 is loaded into registers at the start of step s and written to
// LDS at its end.  The MFMA "A" operand is the output-column side and "B"
// the output-row (token) side; both hold their contraction elements in
// natural order (the MFMA pairs slot e of every A row with slot e of every
// B column).
//
// LDS layouts.  On gfx950 8-byte LDS reads stream at about twice the rate
// of 16-byte reads, and sixteen lanes are served together, so:
//   R  row-fragment tiles: rows of 64 bf16 padded to 136 bytes.  A fragment
//      (16 bytes of one row) is read as two adjacent 8-byte halves; sixteen
//      consecutive rows reading the same half sit 17 units of 8 bytes apart
//      and so hit sixteen different bank groups.
//   T  transposed tiles (backward weight side): rows = contraction index,
//      256 bf16 padded to 544 bytes; read with ds_read_b64_tr_b16, which
//      hands each lane of a 16-lane group one column of a 4-row block.  The
//      four rows of a block sit 68 units apart (4 bank groups), so the 16
//      addresses hit 16 different bank groups.
#include "device.h"
#include "kernels.h"

namespace qlora {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 256;
constexpr int kRS = 136;                         // R-layout row stride (bytes)
constexpr int kTS = 544;                         // T-layout row stride (bytes)
constexpr int kRTileBytes = kTile * kRS;         // 34816
constexpr int kTTileBytes = 64 * kTS;            // 34816
static_assert(kRTileBytes == kTTileBytes, "tiles share one buffer size");
constexpr int kBuf = kRTileBytes;
constexpr size_t kLds = 4u * kBuf;               // 2 buffers x 2 operands = 136 KiB

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

__device__ __forceinline__ uint2 lds_read8(const char* p) { return *reinterpret_cast<const uint2*>(p); }
__device__ __forceinline__ void lds_write8(char* p, uint32_t a, uint32_t b) {
  *reinterpret_cast<uint2*>(p) = make_uint2(a, b);
}
__device__ __forceinline__ uint2 lds_read_tr(const char* p) {
  const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p));
  return __builtin_bit_cast(uint2, v);
}
__device__ __forceinline__ bf16x8_t frag(uint2 lo, uint2 hi) {
  return __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
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

// Interleave one contraction sub-step: 16 MFMAs, the fragment reads of the
// next sub-step early, the producer's VALU work spread between the MFMAs
// and its LDS writes at the end.
__device__ __forceinline__ void schedule_substep() {
#pragma unroll
  for (int x = 0; x < 16; ++x) {
    QLORA_SCHED(kSchedMfma, 1);
    if (x < 8) QLORA_SCHED(kSchedDsRead, 1);
    QLORA_SCHED(kSchedValu, 5);
    if (x >= 12) QLORA_SCHED(kSchedDsWrite, 1);
  }
}

__device__ __forceinline__ void map_tile(int tiles_c, int tiles_r, int& tc, int& tr) {
  const int nwg = tiles_c * tiles_r;
  int id = blockIdx.x;
  if ((nwg & 7) == 0) id = (id & 7) * (nwg >> 3) + (id >> 3);
  tc = id % tiles_c;
  tr = id / tiles_c;
}

// ---------------------------------------------------------------------------
// NF4 codes of one (row, 64-block): 32 bytes of codes + absmax code + scale.
// ---------------------------------------------------------------------------
struct BlockCodes {
  uint4 c0, c1;
  uint32_t q;
  float s2;
};

// Block index of (row n, 64-block blk) is n K/64 + blk: `boff` = n K/64 per
// lane (32-bit), blk uniform.
__device__ __forceinline__ void load_block(BlockCodes& bc, const Nf4View& W, uint32_t boff, int64_t blk, bool valid) {
  if (valid) {
    const uint4* p = reinterpret_cast<const uint4*>(W.codes + blk * 32 + (uint64_t)boff * 32u);
    bc.c0 = p[0];
    bc.c1 = p[1];
    bc.q = (W.absmax_q + blk)[boff];
    bc.s2 = W.group_scale[(boff + (uint32_t)blk) >> 8];
  } else {
    bc.c0 = bc.c1 = make_uint4(0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u);
    bc.q = 0;
    bc.s2 = 0.0f;
  }
}

__device__ __forceinline__ uint32_t code_word(const BlockCodes& bc, int ch) {
  switch (ch) {
    case 0: return bc.c0.x; case 1: return bc.c0.y; case 2: return bc.c0.z; case 3: return bc.c0.w;
    case 4: return bc.c1.x; case 5: return bc.c1.y; case 6: return bc.c1.z; default: return bc.c1.w;
  }
}

// ---------------------------------------------------------------------------
// Token-side tile (layout R) staged through registers: 256 rows x 128 bytes
// per step, 8 x 16 bytes per thread; 8 consecutive lanes read one row.
// Rows past the end re-read the last row (finite data, never stored);
// columns past `cols` (rank and contraction tails) are zero.
// ---------------------------------------------------------------------------
struct RTileRegs {
  uint4 v[8];
};

// Per-lane byte offsets of the 8 rows a thread loads (rows past the end are
// clamped to the last row); `ld` in elements.
struct RTileOffs {
  uint32_t o[8];
};

__device__ __forceinline__ void r_offsets(RTileOffs& O, int64_t ld, int64_t rows, int64_t row0) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int idx = threadIdx.x + kThreads * q;
    int64_t gr = row0 + (idx >> 3);
    gr = gr < rows ? gr : rows - 1;
    O.o[q] = (uint32_t)(2 * (gr * ld + 8 * (idx & 7)));
  }
}

// Load step `step` of a row-major tile: uniform base (src + 64 step) plus the
// lane's 32-bit byte offset.  `col_clamp` (bytes, multiple of 16) keeps a
// ragged last step inside each row; the excess columns meet zero weights.
__device__ __forceinline__ void r_load(RTileRegs& R, const bf16_t* src, const RTileOffs& O, int step,
                                       uint32_t col_bytes_left) {
  const char* base = reinterpret_cast<const char*>(src + (int64_t)step * 64);
  const uint32_t cmax = col_bytes_left - 16;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint32_t c16 = 16u * ((threadIdx.x + kThreads * q) & 7);
    const uint32_t off = O.o[q] - c16 + (c16 < cmax ? c16 : cmax);
    R.v[q] = *reinterpret_cast<const uint4*>(base + off);
  }
}

__device__ __forceinline__ void r_load_masked(RTileRegs& R, const bf16_t* src, int64_t ld, int64_t rows,
                                              int64_t cols, int64_t row0, int step) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int idx = threadIdx.x + kThreads * q;
    const int64_t gr = row0 + (idx >> 3), gc = (int64_t)step * 64 + 8 * (idx & 7);
    R.v[q] = make_uint4(0u, 0u, 0u, 0u);
    if (gr < rows && gc < cols) R.v[q] = *reinterpret_cast<const uint4*>(src + gr * ld + gc);
  }
}

__device__ __forceinline__ void r_store(char* lds, const RTileRegs& R) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int idx = threadIdx.x + kThreads * q;
    char* p = lds + (idx >> 3) * kRS + 16 * (idx & 7);
    lds_write8(p, R.v[q].x, R.v[q].y);
    lds_write8(p + 8, R.v[q].z, R.v[q].w);
  }
}

__device__ __forceinline__ void r_scale(RTileRegs& R, float s) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    uint4& v = R.v[q];
    v.x = pack_bf16x2(bf2f(v.x & 0xFFFFu) * s, bf2f(v.x >> 16) * s);
    v.y = pack_bf16x2(bf2f(v.y & 0xFFFFu) * s, bf2f(v.y >> 16) * s);
    v.z = pack_bf16x2(bf2f(v.z & 0xFFFFu) * s, bf2f(v.z >> 16) * s);
    v.w = pack_bf16x2(bf2f(v.w & 0xFFFFu) * s, bf2f(v.w >> 16) * s);
  }
}

// Fragment (layout R) for sub-step kk: lane (lr, h) reads the 16 bytes of
// chunk 2kk + h of its fragment row; `base` already holds the lane's row
// and h offset.
__device__ __forceinline__ bf16x8_t r_frag(const char* base, int kk) {
  const char* p = base + 32 * kk;
  return frag(lds_read8(p), lds_read8(p + 8));
}

// Per-lane byte offset of a lane's fragment row within a tile.
__device__ __forceinline__ int r_lane_off(int lane) { return (lane & 31) * kRS + 16 * (lane >> 5); }

__device__ __forceinline__ void store_acc_bf16(const f32x16_t (&acc)[4][4], bf16_t* out, int64_t ld, int64_t rows,
                                               int64_t cols, int64_t col0, int64_t row0) {
  const int lane = threadIdx.x & 63, lr = lane & 31, h = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t row = row0 + 32 * j + lr;
      if (row >= rows) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t col = col0 + 32 * i + 8 * q + 4 * h;
        if (col < cols) {  // cols % 8 == 0, so the 4 columns are all in range
          *reinterpret_cast<uint2*>(out + row * ld + col) =
              make_uint2(pack_bf16x2(acc[i][j][4 * q + 0], acc[i][j][4 * q + 1]),
                         pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]));
        }
      }
    }
}

// ---------------------------------------------------------------------------
// Forward kernel
// ---------------------------------------------------------------------------
// Weight-side producer: thread t owns W row t of the tile and dequantizes
// chunks [ch0, ch0 + n) of its 64-element block into LDS row t (layout R).
__device__ __forceinline__ void fwd_dequant_chunks(char* As, const BlockCodes& bc, const Nf4Table& T, int ch0,
                                                   int n) {
  char* row = As + threadIdx.x * kRS;
#pragma unroll
  for (int k = 0; k < n; ++k) {
    const int ch = ch0 + k;
    uint32_t o[4];
    dequant8(code_word(bc, ch), T, o);
    lds_write8(row + 16 * ch, o[0], o[1]);
    lds_write8(row + 16 * ch + 8, o[2], o[3]);
  }
}

struct FwdCtx {
  Nf4View W;
  const bf16_t* X;
  RTileOffs xo;
  uint32_t wboff;  // owned W row * K / 64
  bool wvalid;
  int nsteps;
};

// One contraction step: MFMAs on (Ac, Bc) while producing step st+1 into
// (An, Bn) from `cur` (the codes of step st+1); the codes of step st+2 are
// loaded into `nxt`.
__device__ __forceinline__ void fwd_step(f32x16_t (&acc)[4][4], bf16x8_t (&fa)[2][4], bf16x8_t (&fb)[2][4],
                                         const FwdCtx& c, int st, const char* Ac, const char* Bc, char* An,
                                         char* Bn, const BlockCodes& cur, BlockCodes& nxt, RTileRegs& xr,
                                         int aoff, int boff) {
  const bool more = st + 1 < c.nsteps;
  if (more) r_load(xr, c.X, c.xo, st + 1, 128u);
  if (st + 2 < c.nsteps) load_block(nxt, c.W, c.wboff, st + 2, c.wvalid);
  // Branch-free producer (on the last step it fills a buffer nobody reads)
  // so that the scheduler can interleave it with the MFMAs.
  const Nf4Table T = make_table(block_scale(cur.q, cur.s2));
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    if (kk < 3) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fa[(kk + 1) & 1][i] = r_frag(Ac + aoff + 32 * kRS * i, kk + 1);
        fb[(kk + 1) & 1][i] = r_frag(Bc + boff + 32 * kRS * i, kk + 1);
      }
    }
    mfma_block<4, 4>(acc, fa[kk & 1], fb[kk & 1]);
    fwd_dequant_chunks(An, cur, T, 2 * kk, 2);
    schedule_substep();
  }
  if (more) r_store(Bn, xr);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    fa[0][i] = r_frag(An + aoff + 32 * kRS * i, 0);
    fb[0][i] = r_frag(Bn + boff + 32 * kRS * i, 0);
  }
}

__global__ __launch_bounds__(kThreads, 1) void nf4_fwd_kernel(Nf4View W, const bf16_t* __restrict__ X, int64_t M,
                                                              const bf16_t* __restrict__ U,
                                                              const bf16_t* __restrict__ Bl, int r, float s,
                                                              bf16_t* __restrict__ Y, int tiles_n, int tiles_m) {
  extern __shared__ __align__(16) char smem[];
  char* const A0 = smem;
  char* const A1 = smem + kBuf;
  char* const B0 = smem + 2 * kBuf;
  char* const B1 = smem + 3 * kBuf;
  int tn, tm;
  map_tile(tiles_n, tiles_m, tn, tm);
  const int64_t n0 = (int64_t)tn * kTile, m0 = (int64_t)tm * kTile;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, wr = w >> 1, wc = w & 1;
  FwdCtx c;
  c.W = W;
  c.X = X;
  r_offsets(c.xo, W.K, M, m0);
  c.wboff = (uint32_t)((n0 + t) * (W.K >> 6));
  c.wvalid = n0 + t < W.N;
  c.nsteps = (int)(W.K >> 6);
  const int aoff = wc * 128 * kRS + r_lane_off(lane);
  const int boff = wr * 128 * kRS + r_lane_off(lane);

  f32x16_t acc[4][4];
  zero_acc(acc);

  // prologue: step 0 into buffer 0, codes of step 1 in flight
  BlockCodes bcA, bcB;
  RTileRegs xr;
  r_load(xr, X, c.xo, 0, 128u);
  load_block(bcA, W, c.wboff, 0, c.wvalid);
  bcB = bcA;
  if (c.nsteps > 1) load_block(bcB, W, c.wboff, 1, c.wvalid);
  {
    const Nf4Table T = make_table(block_scale(bcA.q, bcA.s2));
    fwd_dequant_chunks(A0, bcA, T, 0, 8);
  }
  r_store(B0, xr);
  __syncthreads();

  bf16x8_t fa[2][4], fb[2][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    fa[0][i] = r_frag(A0 + aoff + 32 * kRS * i, 0);
    fb[0][i] = r_frag(B0 + boff + 32 * kRS * i, 0);
  }
  // two steps per iteration: buffers and code registers alternate
  // statically; an odd last step is peeled
  int st = 0;
  for (; st + 1 < c.nsteps; st += 2) {
    fwd_step(acc, fa, fb, c, st, A0, B0, A1, B1, bcB, bcA, xr, aoff, boff);
    fwd_step(acc, fa, fb, c, st + 1, A1, B1, A0, B0, bcA, bcB, xr, aoff, boff);
  }
  if (st < c.nsteps) fwd_step(acc, fa, fb, c, st, A0, B0, A1, B1, bcB, bcA, xr, aoff, boff);

  if (r > 0) {
    // LoRA up-projection: extra contraction steps over the rank,
    // acc += (s U) B^T, through the same LDS layout.
    for (st = 0; st * 64 < r; ++st) {
      r_load_masked(xr, Bl, r, W.N, r, n0, st);
      r_store(A0, xr);
      r_load_masked(xr, U, r, M, r, m0, st);
      r_scale(xr, s);
      r_store(B0, xr);
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          fa[0][i] = r_frag(A0 + aoff + 32 * kRS * i, kk);
          fb[0][i] = r_frag(B0 + boff + 32 * kRS * i, kk);
        }
        mfma_block<4, 4>(acc, fa[0], fb[0]);
      }
      __syncthreads();
    }
  }
  store_acc_bf16(acc, Y, W.N, M, W.N, n0 + wc * 128, m0 + wr * 128);
}

// ---------------------------------------------------------------------------
// Backward dX kernel
// ---------------------------------------------------------------------------
// Weight-side tile (layout T): 64 contraction rows x 256 columns.  Thread t
// owns row t >> 2 and 64-column block t & 3.
__device__ __forceinline__ char* t_chunk(char* lds, int row, int blk, int ch) {
  return lds + row * kTS + 128 * blk + 16 * ch;
}

// Per-lane byte offset of the first transpose read of fragment i at kk = 0:
// as a source lane of its 16-lane group (g, s) it addresses row
// 8h + (s >> 2), columns ia + 32 i + 16 half16 + 4 (s & 3) .. +3.  kk adds
// 16 rows, the second read 4 rows.
__device__ __forceinline__ int t_frag_off(int lane, int ia, int i) {
  const int g = lane >> 4, s = lane & 15, h = g >> 1, half16 = g & 1;
  return (8 * h + (s >> 2)) * kTS + 2 * (ia + 32 * i + 16 * half16 + 4 * (s & 3));
}

__device__ __forceinline__ bf16x8_t t_frag(const char* p, int kk) {
  const char* q = p + kk * 16 * kTS;
  return frag(lds_read_tr(q), lds_read_tr(q + 4 * kTS));
}

struct DxCtx {
  Nf4View W;
  const bf16_t* dY;
  RTileOffs yo;
  uint32_t ybytes;  // 2 N: bytes per dY row
  uint32_t wboff;   // block index of (row orow, column kcol)
  int64_t kcol;
  int orow, oblk;
  bool kvalid;
  int nsteps;
};

// Codes of contraction step `step`: W row 64 step + orow, 64-column block
// kcol / 64; its block index is wboff + 64 step K/64 (the uniform part).
__device__ __forceinline__ void dx_wload(BlockCodes& bc, const DxCtx& c, int step) {
  const int64_t n = (int64_t)step * 64 + c.orow;
  load_block(bc, c.W, c.wboff, (int64_t)step * 64 * (c.W.K >> 6), c.kvalid && n < c.W.N);
}

__device__ __forceinline__ void dx_dequant(char* As, const DxCtx& c, const BlockCodes& bc, const Nf4Table& T, int ch0,
                                           int cnt) {
#pragma unroll
  for (int k = 0; k < cnt; ++k) {
    uint32_t o[4];
    dequant8(code_word(bc, ch0 + k), T, o);
    *reinterpret_cast<uint4*>(t_chunk(As, c.orow, c.oblk, ch0 + k)) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

__device__ __forceinline__ void dx_step(f32x16_t (&acc)[4][4], bf16x8_t (&fa)[2][4], bf16x8_t (&fb)[2][4],
                                        const DxCtx& c, int st, const char* Ac, const char* Bc, char* An, char* Bn,
                                        const BlockCodes& cur, BlockCodes& nxt, RTileRegs& yr, const int (&aoff)[4],
                                        int boff) {
  const bool more = st + 1 < c.nsteps;
  if (more) r_load(yr, c.dY, c.yo, st + 1, c.ybytes - 128u * (st + 1));
  if (st + 2 < c.nsteps) dx_wload(nxt, c, st + 2);
  const Nf4Table T = make_table(block_scale(cur.q, cur.s2));
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    if (kk < 3) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fa[(kk + 1) & 1][i] = t_frag(Ac + aoff[i], kk + 1);
        fb[(kk + 1) & 1][i] = r_frag(Bc + boff + 32 * kRS * i, kk + 1);
      }
    }
    mfma_block<4, 4>(acc, fa[kk & 1], fb[kk & 1]);
    dx_dequant(An, c, cur, T, 2 * kk, 2);
    schedule_substep();
  }
  if (more) r_store(Bn, yr);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    fa[0][i] = t_frag(An + aoff[i], 0);
    fb[0][i] = r_frag(Bn + boff + 32 * kRS * i, 0);
  }
}

__global__ __launch_bounds__(kThreads, 1) void nf4_dx_kernel(Nf4View W, const bf16_t* __restrict__ dY, int64_t M,
                                                             const bf16_t* __restrict__ G,
                                                             const bf16_t* __restrict__ Al, int r, float s,
                                                             bf16_t* __restrict__ dX, int tiles_k, int tiles_m) {
  extern __shared__ __align__(16) char smem[];
  char* const A0 = smem;
  char* const A1 = smem + kBuf;
  char* const B0 = smem + 2 * kBuf;
  char* const B1 = smem + 3 * kBuf;
  int tk, tm;
  map_tile(tiles_k, tiles_m, tk, tm);
  const int64_t k0 = (int64_t)tk * kTile, m0 = (int64_t)tm * kTile;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, wr = w >> 1, wc = w & 1;
  DxCtx c;
  c.W = W;
  c.dY = dY;
  r_offsets(c.yo, W.N, M, m0);
  c.ybytes = (uint32_t)(2 * W.N);
  c.orow = t >> 2;
  c.oblk = t & 3;
  c.kcol = k0 + 64 * (t & 3);
  c.kvalid = c.kcol < W.K;
  c.wboff = (uint32_t)(c.orow * (W.K >> 6) + (c.kvalid ? (c.kcol >> 6) : 0));
  c.nsteps = (int)((W.N + 63) >> 6);

  int aoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) aoff[i] = t_frag_off(lane, wc * 128, i);
  const int boff = wr * 128 * kRS + r_lane_off(lane);

  f32x16_t acc[4][4];
  zero_acc(acc);

  BlockCodes bcA, bcB;
  RTileRegs yr;
  r_load(yr, dY, c.yo, 0, c.ybytes);
  dx_wload(bcA, c, 0);
  bcB = bcA;
  if (c.nsteps > 1) dx_wload(bcB, c, 1);
  {
    const Nf4Table T = make_table(block_scale(bcA.q, bcA.s2));
    dx_dequant(A0, c, bcA, T, 0, 8);
  }
  r_store(B0, yr);
  __syncthreads();

  bf16x8_t fa[2][4], fb[2][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    fa[0][i] = t_frag(A0 + aoff[i], 0);
    fb[0][i] = r_frag(B0 + boff + 32 * kRS * i, 0);
  }
  int st = 0;
  for (; st + 1 < c.nsteps; st += 2) {
    dx_step(acc, fa, fb, c, st, A0, B0, A1, B1, bcB, bcA, yr, aoff, boff);
    dx_step(acc, fa, fb, c, st + 1, A1, B1, A0, B0, bcA, bcB, yr, aoff, boff);
  }
  if (st < c.nsteps) dx_step(acc, fa, fb, c, st, A0, B0, A1, B1, bcB, bcA, yr, aoff, boff);

  if (r > 0) {
    // acc += (s G) A over the rank: A [r x K] rows are contraction rows of
    // the weight-side layout, copied without dequantization.
    for (st = 0; st * 64 < r; ++st) {
      {
        const int64_t j = (int64_t)st * 64 + c.orow;
        const bool ok = j < r && c.kvalid;
        const bf16_t* src = Al + j * W.K + c.kcol;
#pragma unroll
        for (int ch = 0; ch < 8; ++ch) {
          uint4 v = make_uint4(0u, 0u, 0u, 0u);
          if (ok) v = *reinterpret_cast<const uint4*>(src + 8 * ch);
          *reinterpret_cast<uint4*>(t_chunk(A0, c.orow, c.oblk, ch)) = v;
        }
      }
      r_load_masked(yr, G, r, M, r, m0, st);
      r_scale(yr, s);
      r_store(B0, yr);
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          fa[0][i] = t_frag(A0 + aoff[i], kk);
          fb[0][i] = r_frag(B0 + boff + 32 * kRS * i, kk);
        }
        mfma_block<4, 4>(acc, fa[0], fb[0]);
      }
      __syncthreads();
    }
  }
  store_acc_bf16(acc, dX, W.K, M, W.K, k0 + wc * 128, m0 + wr * 128);
}

}  // namespace

hipError_t launch_fwd(const Nf4View& W, const bf16_t* X, int64_t M, const bf16_t* U, const bf16_t* B, int r,
                      float s, bf16_t* Y, hipStream_t st) {
  const int tiles_n = (int)((W.N + kTile - 1) / kTile);
  const int tiles_m = (int)((M + kTile - 1) / kTile);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&nf4_fwd_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(nf4_fwd_kernel, dim3(tiles_n * tiles_m), dim3(kThreads), kLds, st, W, X, M, U, B, r, s, Y,
                     tiles_n, tiles_m);
  return hipGetLastError();
}

hipError_t launch_dx(const Nf4View& W, const bf16_t* dY, int64_t M, const bf16_t* G, const bf16_t* A, int r,
                     float s, bf16_t* dX, hipStream_t st) {
  const int tiles_k = (int)((W.K + kTile - 1) / kTile);
  const int tiles_m = (int)((M + kTile - 1) / kTile);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&nf4_dx_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(nf4_dx_kernel, dim3(tiles_k * tiles_m), dim3(kThreads), kLds, st, W, dY, M, G, A, r, s, dX,
                     tiles_k, tiles_m);
  return hipGetLastError();
}

}  // namespace qlora
