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
// with fp32 accumulation.  The contraction runs in stages of 32 through a
// ring of four LDS stage buffers (weight half + token half), one barrier per
// stage, placed between its two MFMA halves:
//
//   substep s:  issue the loads of stage s+3 (token tile) and of the codes
//               ahead; dequantize stage s+2 into its ring slot; MFMAs on
//               stage s (first half) | barrier | MFMAs on stage s (second
//               half) while the first fragments of stage s+1 are read.
//
// The dequantization (NF4 code -> block-scaled bf16 by a byte-permute table,
// see device.h) is interleaved with the MFMAs of the same wave; a weight
// element is dequantized once per 256-token tile.
//
// Token-side tiles are stored as rows of 32 bf16 (64 bytes), 16-byte chunk c
// of row r at position c ^ ((r >> 2) & 3): sixteen consecutive rows reading
// one logical chunk (the MFMA fragment pattern) cover all 64 LDS banks, and
// so do the producers' 16-byte writes.  The MFMA "A" operand is the output
// column side (weight rows / columns), "B" the token side.
#include "gemm_common.h"

namespace qlora {
namespace {

// Second-level constants of a block: its 8-bit absmax code and group scale.
struct Scale {
  uint32_t q;
  float s2;
};

// ===========================================================================
// Forward with the weight operand in registers.  Wave w owns weight rows
// n0 + 64 w .. +63 (two 32-row A fragments) against all 256 tokens of the
// tile (eight 32-token B fragments): still 16 accumulator tiles per wave,
// but every weight element a wave multiplies is one it dequantized itself,
// straight into its MFMA A registers.  Only the token tile (DMA, a ring of
// kRSlots stages shared by the four waves) and the wave's own NF4 codes
// (DMA, two stages per chunk, four chunk buffers) pass through LDS; no
// dequantized weight is written to LDS.
//
// k order inside a 32-wide stage: lane half h of an MFMA takes k 16h + 8kk
// .. +7 in k16 step kk, so a lane's weight codes for a stage are the 8
// contiguous bytes 8h .. 8h+7 of its row's 16, and its token fragment of
// step kk is 16-byte chunk 2h + kk of the token row.
//
// Substep s (U8 = s mod 8; token stage s sits in ring slot s & 7), one
// barrier each:
//   wait until token stage s+1 and the code chunk of stage s+2 have landed;
//   barrier (the token stage is then visible from every wave, and every
//   wave has finished reading the slot about to be refilled);
//   DMA token stage s + kRAhead; odd s: DMA code chunk (s+7)/2; even s:
//   load the scales of block s/2 + 3;
//   read the codes of stage s+2 (used by the next substep); odd s: build
//   the tables of block (s+1)/2 (stage s+1 starts it);
//   first half:  MFMAs of k16 step 0 of stage s; read step 1 of stage s;
//                dequantize step 1 of stage s+1;
//   second half: MFMAs of step 1 of stage s; read step 0 of stage s+1;
//                dequantize step 0 of stage s+1 into the registers step 0
//                of stage s has just freed.
// ===========================================================================
constexpr int kRSlots = 8;                                            // token ring depth (stage s in slot s & 7)
constexpr int kRAhead = 6;                                            // token stages DMA'd ahead of use
// The refilled slot (stage s + kRAhead - 8) was last read in substep s-1 at
// the latest; the code chunk DMA'd at substep 2c-7 is read at substep 2c-2.
static_assert(kRAhead >= 2 && kRAhead <= 6, "ring / code-chunk schedule");
constexpr int kRChunk = kTile * 32;                                   // 8 KiB: codes of two stages
constexpr int kRCodeBase = kRSlots * kOp;                             // 128 KiB
constexpr size_t kLdsFwdR = (size_t)kRCodeBase + 4 * kRChunk;         // 160 KiB

// Loads issued by substep v of the register-A forward: 4 token DMAs, then
// 2 code DMAs at odd v or 4 scale loads at even v.
constexpr int fwdr_loads(int v) { return 4 + ((v & 1) ? 2 : 4); }
// vmcnt at the start of substep u: token stage u+1 (issued at substep
// u + 1 - kRAhead) has landed once only the loads of substeps
// u + 2 - kRAhead .. u - 1 may be in flight.
constexpr int fwdr_vmcnt(int u) {
  int n = 0;
  for (int v = u + 2 - kRAhead; v <= u - 1; ++v) n += fwdr_loads(v & 7);
  return n;
}
static_assert(fwdr_vmcnt(0) < 64 && fwdr_vmcnt(1) < 64, "vmcnt field");

struct FwdR {
  rsrc_t xr, cr;          // X, NF4 codes
  uint32_t xo[4];         // per-lane byte offsets of the four token DMA instructions
  uint32_t co[2];         // ... of the two code DMA instructions (row 64 w + lane, stage half p)
  const uint8_t* aq[2];   // absmax codes of the lane's two rows (block 0)
  const float* gs;        // group scales
  uint32_t ablk0[2];      // block index of (row, block 0)
  int nsub, nblk, w;
  int crow[2];            // code-chunk byte offset of the lane's 8-byte piece in row i
  int absfmt;             // second-level format of the block constants
};

__device__ __forceinline__ void fwdr_dma_x(char* smem, const FwdR& f, int stage, int slot) {
  const uint32_t soff = (uint32_t)min(stage, f.nsub - 1) * 64u;
  char* dst = smem + slot * kOp;
#pragma unroll
  for (int q = 0; q < 4; ++q) dma16(f.xr, dst + (64 * q + 16 * f.w) * 64, f.xo[q], soff);
}
// Code chunk c (stages 2c, 2c+1) of the wave's 64 rows into buffer BUF:
// stage half p of row r at BUF * kRChunk + p * 4096 + 16 r.
template <int BUF>
__device__ __forceinline__ void fwdr_dma_codes(char* smem, const FwdR& f, int chunk) {
  const uint32_t soff = (uint32_t)min(chunk, (f.nsub >> 1) - 1) * 32u;
  char* dst = smem + kRCodeBase + BUF * kRChunk + 64 * f.w * 16;
#pragma unroll
  for (int p = 0; p < 2; ++p) dma16(f.cr, dst + p * 4096, f.co[p], soff);
}
__device__ __forceinline__ Scale fwdr_scale(const FwdR& f, int i, int blk) {
  const int b = min(blk, f.nblk - 1);
  return Scale{f.aq[i][b], f.gs[(f.ablk0[i] + (uint32_t)b) >> 8]};
}
// The lane's 8 code bytes (16 weights) of row i in stage st.
__device__ __forceinline__ uint2 fwdr_codes(const char* smem, const FwdR& f, int i, int st) {
  const char* p = smem + kRCodeBase + ((st >> 1) & 3) * kRChunk + (st & 1) * 4096 + f.crow[i];
  const u32x2_t v = *reinterpret_cast<const u32x2_t*>(p);   // a native vector type (see rd16)
  return make_uint2(v.x, v.y);
}

// LDS read bases of the loop: token ring half [slot / 4] at chunk 2h (0) or
// 2h + 1 (1), and the code chunks (row 0 of the lane; row 1 is 512 B on).
struct RdBase {
  int tok[2][2];
  int code;
};
// Codes of row i in stage ST (mod 8), read from the loop's code base.
template <int ST>
__device__ __forceinline__ uint2 fwdr_codes_at(const char* smem, const RdBase& rb, int i) {
  constexpr int off = ((ST >> 1) & 3) * kRChunk + (ST & 1) * 4096;
  const u32x2_t v = *reinterpret_cast<const u32x2_t*>(smem + rb.code + off + 512 * i);
  return make_uint2(v.x, v.y);
}

struct FragsR {
  bf16x8_t b0[8], b1[8];   // token fragments of k16 steps 0 and 1
  bf16x8_t a0[2], a1[2];   // weight fragments of the current stage, steps 0 and 1 [row]
  uint2 c[2];              // codes of the next stage [row]
};

template <int FI, int FJ>
__device__ __forceinline__ void mfma_rows(f32x16_t (&acc)[FI][FJ], const bf16x8_t (&a)[FI], const bf16x8_t (&b)[FJ]) {
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j) acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j]);
}

// Eight weights (a code dword) -> bf16 x 8 fragment.
__device__ __forceinline__ bf16x8_t deq_frag(uint32_t c, const Nf4Table& T) {
  uint32_t o[4];
  dequant8(c, T, o);
  return __builtin_bit_cast(bf16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
}

// The dequantization work of a substep is cut into chunks of five or six
// VALU instructions, one chunk after each MFMA, and every MFMA slot is fenced
// so that the compiler keeps the interleave (left to itself it bunches a
// whole decode between two MFMAs and leaves the matrix unit idle).
//
// Decode of one code dword (eight weights) in five chunks; the steps are
// those of dequant8.
struct DqState {
  uint32_t sa, sb, o, le, he, lo, ho, l01, h01;
};
template <int K>
__device__ __forceinline__ void dq_chunk(DqState& d, uint32_t c, const Nf4Table& T, bf16x8_t& out) {
  if constexpr (K == 0) {
    const uint32_t e = c & 0x0F0F0F0Fu;
    d.o = (c >> 4) & 0x0F0F0F0Fu;
    d.sa = e + (e & 0x08080808u);
    d.sb = d.sa ^ 0x10101010u;
  } else if constexpr (K == 1) {
    d.le = perm(T.lo[1], T.lo[0], d.sa) & perm(T.lo[3], T.lo[2], d.sb);
    d.he = perm(T.hi[1], T.hi[0], d.sa) & perm(T.hi[3], T.hi[2], d.sb);
  } else if constexpr (K == 2) {
    d.sa = d.o + (d.o & 0x08080808u);
    d.sb = d.sa ^ 0x10101010u;
    d.lo = perm(T.lo[1], T.lo[0], d.sa) & perm(T.lo[3], T.lo[2], d.sb);
  } else if constexpr (K == 3) {
    d.ho = perm(T.hi[1], T.hi[0], d.sa) & perm(T.hi[3], T.hi[2], d.sb);
    d.l01 = perm(d.lo, d.le, 0x05010400u);
    d.h01 = perm(d.ho, d.he, 0x05010400u);
  } else {
    const uint32_t l23 = perm(d.lo, d.le, 0x07030602u);
    const uint32_t h23 = perm(d.ho, d.he, 0x07030602u);
    out = __builtin_bit_cast(bf16x8_t, make_uint4(perm(d.h01, d.l01, 0x05010400u), perm(d.h01, d.l01, 0x07030602u),
                                                  perm(h23, l23, 0x05010400u), perm(h23, l23, 0x07030602u)));
  }
}
// Table of one block in six chunks; the steps are those of make_table.
struct TbState {
  float t;
  uint32_t p[8];
  Nf4Table T;   // the table of the lane's own row, before the lane-half swap
};
// Product of level i of codebook CB with t; the levels 0 and 1 give 0 and t
// exactly (t is finite and not negative), so they are not multiplied out.
template <int CB>
__device__ __forceinline__ float level_times(int i, float t) {
  const uint32_t l = cb_level_bits<CB>(i);
  return l == 0u ? 0.0f : l == 0x3F800000u ? t : u2f(l) * t;
}
template <int CB, int K>
__device__ __forceinline__ void tb_chunk(TbState& b, const Scale& sc, Nf4Table& T, int fmt) {
  auto pair = [&](int i) { b.p[i] = pack_bf16x2(level_times<CB>(2 * i, b.t), level_times<CB>(2 * i + 1, b.t)); };
  if constexpr (K == 0) {
    b.t = block_scale(sc.q, sc.s2, fmt);
    pair(0);
  } else if constexpr (K < 4) {
    pair(2 * K - 1);
    pair(2 * K);
  } else if constexpr (K == 4) {
    pair(7);
    T.lo[0] = perm(b.p[1], b.p[0], 0x06040200u);
    T.hi[0] = perm(b.p[1], b.p[0], 0x07050301u);
    T.lo[1] = perm(b.p[3], b.p[2], 0x06040200u);
  } else {
    T.hi[1] = perm(b.p[3], b.p[2], 0x07050301u);
#pragma unroll
    for (int j = 2; j < 4; ++j) {
      T.lo[j] = perm(b.p[2 * j + 1], b.p[2 * j], 0x06040200u);
      T.hi[j] = perm(b.p[2 * j + 1], b.p[2 * j], 0x07050301u);
    }
  }
}

// MFMA slot X (0..31) of a register-A forward substep: slot X < 16 is
// fragment pair (row X & 1, token fragment X >> 1) of k16 step 0, slot
// X >= 16 the same for step 1.  Besides its MFMA a slot carries:
//   global loads  token DMA (stage s + kRAhead) in slots 1, 3, 5, 7; odd s:
//                 code DMA (chunk (s+7)/2) in slots 9, 11; even s: the
//                 absmax code and group scale of block s/2 + 3 in slots 9, 11
//                 (row 0) and 13, 15 (row 1)
//   LDS reads     slots 0..7: step 1 of stage s, fragment X; slots 16..23:
//                 step 0 of stage s+1, fragment X - 16 (its register was last
//                 read by slot 2(X-16)+1)
//   VALU chunks   odd s:  in slots 0..5 lane half h builds the table of block
//                         (s+1)/2 for row h, and slot 6 swaps lane halves
//                         so that every lane holds both rows' tables; step 1
//                         of stage s+1 in 7..16, step 0 in 17..26
//                 even s: step 1 of stage s+1 in 0..9, step 0 in 16..25
//                 (step 0 is written over the step 0 registers of stage s,
//                 last read by slot 15)
template <int CB, int U8, int X>
__device__ __forceinline__ void fwdr_slot(char* smem, const FwdR& f, int s, f32x16_t (&acc)[2][8], FragsR& F,
                                          Nf4Table (&T)[2], Scale (&sc)[4][2], bf16x8_t (&n1)[2], DqState& dq,
                                          TbState& tb, const RdBase& rb) {
  constexpr bool kOdd = (U8 & 1) != 0;
  constexpr int i = X & 1, j = (X & 15) >> 1;
  // the step-1 fragments (read in slots 0..7) and the codes: one wait for all
  if constexpr (X == 16) QLORA_WAIT(63, 0);
  if constexpr (X < 16)
    acc[i][j] = mfma32x32x16(F.a0[i], F.b0[j], acc[i][j]);
  else
    acc[i][j] = mfma32x32x16(F.a1[i], F.b1[j], acc[i][j]);
  // global loads
  if constexpr (X < 8 && (X & 1)) {
    const uint32_t soff = (uint32_t)min(s + kRAhead, f.nsub - 1) * 64u;
    dma16(f.xr, smem + ((U8 + kRAhead) & 7) * kOp + (64 * (X >> 1) + 16 * f.w) * 64, f.xo[X >> 1], soff);
  } else if constexpr (kOdd && (X == 9 || X == 11)) {
    constexpr int c8 = (U8 + 7) >> 1;   // chunk (s+7)/2 is c8 mod 4
    const uint32_t soff = (uint32_t)min((s + 7) >> 1, (f.nsub >> 1) - 1) * 32u;
    dma16(f.cr, smem + kRCodeBase + (c8 & 3) * kRChunk + 64 * f.w * 16 + ((X - 9) >> 1) * 4096, f.co[(X - 9) >> 1],
          soff);
  } else if constexpr (!kOdd && X >= 9 && X <= 15 && (X & 1)) {
    constexpr int SL = ((U8 >> 1) + 3) & 3, row = (X - 9) >> 2;
    const int b = min((s >> 1) + 3, f.nblk - 1);
    if constexpr (((X - 9) >> 1) & 1)
      sc[SL][row].s2 = f.gs[(f.ablk0[row] + (uint32_t)b) >> 8];
    else
      sc[SL][row].q = f.aq[row][b];
  }
  // LDS reads
  if constexpr (X < 8) F.b1[X] = rd16(smem + rb.tok[U8 >> 2][1] + (U8 & 3) * kOp + X * 2048);
  if constexpr (X >= 16 && X < 24) {
    constexpr int SN = (U8 + 1) & 7;
    F.b0[X - 16] = rd16(smem + rb.tok[SN >> 2][0] + (SN & 3) * kOp + (X - 16) * 2048);
  }
  // VALU chunks
  if constexpr (kOdd) {
    constexpr int SL = ((U8 + 1) >> 1) & 3;
    if constexpr (X < 6) {
      const bool hi = (threadIdx.x & 32) != 0;
      const Scale mine{hi ? sc[SL][1].q : sc[SL][0].q, hi ? sc[SL][1].s2 : sc[SL][0].s2};
      tb_chunk<CB, X>(tb, mine, tb.T, f.absfmt);
    } else if constexpr (X == 6) {
      // lanes 0..31 hold row 0's table and lanes 32..63 row 1's: swapping the
      // upper half of one copy with the lower half of another gives each row's
      // table in every lane
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x2_t lo = __builtin_amdgcn_permlane32_swap(tb.T.lo[q], tb.T.lo[q], false, false);
        const u32x2_t hi = __builtin_amdgcn_permlane32_swap(tb.T.hi[q], tb.T.hi[q], false, false);
        T[0].lo[q] = lo[0];
        T[1].lo[q] = lo[1];
        T[0].hi[q] = hi[0];
        T[1].hi[q] = hi[1];
      }
    } else if constexpr (X >= 7 && X < 17) {
      dq_chunk<(X - 7) % 5>(dq, F.c[(X - 7) / 5].y, T[(X - 7) / 5], n1[(X - 7) / 5]);
    } else if constexpr (X >= 17 && X < 27) {
      dq_chunk<(X - 17) % 5>(dq, F.c[(X - 17) / 5].x, T[(X - 17) / 5], F.a0[(X - 17) / 5]);
    }
  } else {
    if constexpr (X < 10) dq_chunk<X % 5>(dq, F.c[X / 5].y, T[X / 5], n1[X / 5]);
    else if constexpr (X >= 16 && X < 26) dq_chunk<(X - 16) % 5>(dq, F.c[(X - 16) / 5].x, T[(X - 16) / 5], F.a0[(X - 16) / 5]);
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <int CB, int U8>
__device__ __forceinline__ void fwdr_substep(char* smem, const FwdR& f, int s, f32x16_t (&acc)[2][8], FragsR& F,
                                             Nf4Table (&T)[2], Scale (&sc)[4][2], const RdBase& rb) {
  __builtin_amdgcn_sched_barrier(0);
  // the LDS reads of the last substep (step 0 of stage s, issued 16 slots
  // ago) are waited for here too
  QLORA_WAIT(fwdr_vmcnt(U8), 0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  // codes of stage s+2, for the next substep
  const uint2 cn0 = fwdr_codes_at<U8 + 2>(smem, rb, 0), cn1 = fwdr_codes_at<U8 + 2>(smem, rb, 1);
  bf16x8_t n1[2];
  DqState dq;
  TbState tb;
#define QLORA_FWDR_SLOT(x) fwdr_slot<CB, U8, x>(smem, f, s, acc, F, T, sc, n1, dq, tb, rb)
#define QLORA_FWDR_SLOT4(x) QLORA_FWDR_SLOT(x); QLORA_FWDR_SLOT(x + 1); QLORA_FWDR_SLOT(x + 2); QLORA_FWDR_SLOT(x + 3)
  QLORA_FWDR_SLOT4(0); QLORA_FWDR_SLOT4(4); QLORA_FWDR_SLOT4(8); QLORA_FWDR_SLOT4(12);
  QLORA_FWDR_SLOT4(16); QLORA_FWDR_SLOT4(20); QLORA_FWDR_SLOT4(24); QLORA_FWDR_SLOT4(28);
#undef QLORA_FWDR_SLOT4
#undef QLORA_FWDR_SLOT
  F.a1[0] = n1[0];
  F.a1[1] = n1[1];
  F.c[0] = cn0;
  F.c[1] = cn1;
}

template <int CB>
__global__ __launch_bounds__(kThreads, 1) void nf4_fwd_r_kernel(Nf4View W, const bf16_t* __restrict__ X, int64_t M,
                                                                const bf16_t* __restrict__ U,
                                                                const bf16_t* __restrict__ Bl, int r, float s,
                                                                bf16_t* __restrict__ Y, int tiles_n, int tiles_m) {
  extern __shared__ __align__(16) char smem[];
  int tn, tm;
  map_tile(tiles_n, tiles_m, tn, tm);
  const int64_t n0 = (int64_t)tn * kTile, m0 = (int64_t)tm * kTile;
  const int t = threadIdx.x, lane = t & 63, lr = lane & 31, h = lane >> 5;
  const int64_t N = W.N, K = W.K;

  FwdR f;
  f.w = __builtin_amdgcn_readfirstlane(t >> 6);
  __builtin_assume(f.w >= 0 && f.w < 4);
  f.xr = make_rsrc(X, (uint32_t)(M * K * 2));
  f.cr = make_rsrc(W.codes, (uint32_t)(N * K / 2));
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    // rows past the end re-read the last row: finite data, never stored
    const int64_t xm = min(m0 + dma_row(q, t >> 6, lane), M - 1);
    f.xo[q] = (uint32_t)(xm * K * 2 + dma_chunk(lane) * 16);
  }
  {
    const int64_t wn = min(n0 + 64 * f.w + lane, N - 1);
#pragma unroll
    for (int p = 0; p < 2; ++p) f.co[p] = (uint32_t)(wn * (K / 2) + 16 * p);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rt = 64 * f.w + 32 * i + lr;   // row within the tile
    const int64_t own = min(n0 + rt, N - 1);
    f.ablk0[i] = (uint32_t)(own * (K >> 6));
    f.aq[i] = W.absmax_q + f.ablk0[i];
    f.crow[i] = rt * 16 + 8 * h;
  }
  f.gs = W.group_scale;
  f.nsub = (int)(K >> 5);
  f.absfmt = W.absfmt;
  f.nblk = (int)(K >> 6);
  // token fragment offsets: lane (lr, h) reads chunk 2h + kk of token row lr (+ 32 j)
  const int fo0 = spos(lr, 2 * h), fo1 = spos(lr, 2 * h + 1);

  f32x16_t acc[2][8];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // prologue: code chunks 0..3, scales of blocks 0..2, token stages
  // 0 .. kRAhead - 1
  fwdr_dma_codes<0>(smem, f, 0);
  fwdr_dma_codes<1>(smem, f, 1);
  fwdr_dma_codes<2>(smem, f, 2);
  fwdr_dma_codes<3>(smem, f, 3);
  Scale sc[4][2];
#pragma unroll
  for (int b = 0; b < 3; ++b)
#pragma unroll
    for (int i = 0; i < 2; ++i) sc[b][i] = fwdr_scale(f, i, b);
#pragma unroll
  for (int st = 0; st < kRAhead; ++st) fwdr_dma_x(smem, f, st, st);
  QLORA_WAIT(0, 0);
  __builtin_amdgcn_s_barrier();
  Nf4Table T[2];
  FragsR F;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    T[i] = make_table<CB>(block_scale(sc[0][i].q, sc[0][i].s2, f.absfmt));
    const uint2 c = fwdr_codes(smem, f, i, 0);
    F.a0[i] = deq_frag(c.x, T[i]);
    F.a1[i] = deq_frag(c.y, T[i]);
    F.c[i] = fwdr_codes(smem, f, i, 1);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) F.b0[j] = rd16(smem + j * 2048 + fo0);
  // Base addresses of the loop's LDS reads.  The ring spans 128 KiB and the
  // codes sit above it, past the 16-bit offset field of ds_read, so the loop
  // keeps a base per ring half and one for the codes; hiding them from the
  // compiler stops it from folding them back into per-read address adds.
  RdBase rb;
  rb.tok[0][0] = fo0;
  rb.tok[0][1] = fo1;
  rb.tok[1][0] = fo0 + 4 * kOp;
  rb.tok[1][1] = fo1 + 4 * kOp;
  rb.code = kRCodeBase + f.crow[0];
  asm volatile("" : "+v"(rb.tok[1][0]), "+v"(rb.tok[1][1]), "+v"(rb.code));
  // K % 64 == 0, so the stage count is even; the loop's stage counter stays a
  // multiple of 8, so ring positions follow from the substep index alone
  int st = 0;
#define QLORA_FWDR_SUB(u) fwdr_substep<CB, u>(smem, f, st + u, acc, F, T, sc, rb)
  for (; st + 8 <= f.nsub; st += 8) {
    QLORA_FWDR_SUB(0); QLORA_FWDR_SUB(1); QLORA_FWDR_SUB(2); QLORA_FWDR_SUB(3);
    QLORA_FWDR_SUB(4); QLORA_FWDR_SUB(5); QLORA_FWDR_SUB(6); QLORA_FWDR_SUB(7);
  }
  const int rem = f.nsub - st;
  if (rem >= 2) { QLORA_FWDR_SUB(0); QLORA_FWDR_SUB(1); }
  if (rem >= 4) { QLORA_FWDR_SUB(2); QLORA_FWDR_SUB(3); }
  if (rem >= 6) { QLORA_FWDR_SUB(4); QLORA_FWDR_SUB(5); }
#undef QLORA_FWDR_SUB
  // drain the DMAs still in flight (clamped re-loads) before reusing the ring
  QLORA_WAIT(0, 0);
  __builtin_amdgcn_s_barrier();
  if (r > 0) {
    // LoRA up-projection: acc += B (s U)^T over the rank, 32 at a time; the
    // weight operand comes straight from B (rows of the lane, ranks 16h + 8kk)
    for (int j0 = 0; j0 < r; j0 += 32) {
      char* xb = smem;
      tail_tokens(xb, U, M, r, m0, j0, s);
      bf16x8_t a[2][2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int64_t n = n0 + 64 * f.w + 32 * i + lr;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int col = j0 + 16 * h + 8 * kk;
          uint4 v = make_uint4(0u, 0u, 0u, 0u);
          if (col < r && n < N) v = *reinterpret_cast<const uint4*>(Bl + n * r + col);
          a[i][kk] = __builtin_bit_cast(bf16x8_t, v);
        }
      }
      QLORA_WAIT(0, 0);
      __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8_t b[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) b[j] = rd16(xb + j * 2048 + (kk ? fo1 : fo0));
        const bf16x8_t ak[2] = {a[0][kk], a[1][kk]};
        mfma_rows<2, 8>(acc, ak, b);
      }
      QLORA_WAIT(0, 0);
      __builtin_amdgcn_s_barrier();
    }
  }
  // Output: lane (lr, h) of wave w holds token m0 + 32 j + lr and weight
  // columns n0 + 64 w + 32 i + 8 q + 4 h + 0..3; out through LDS (128 KiB)
  lds_free_for_output();
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        lds_put4<64, 31>(smem, 32 * j + lr, 16 * f.w + 8 * i + 2 * q + h, acc[i][j][4 * q], acc[i][j][4 * q + 1],
                         acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
  __syncthreads();
  lds_tile_out<64, 31>(smem, Y, N, M, N, m0, n0);
}

// ===========================================================================
// Forward with 32 weight rows per wave: the tile is WAVES x 32 weight rows
// x 256 tokens, and wave w owns weight rows n0 + 32 w .. +31 (one A
// fragment) against all 256 tokens: 8 accumulator tiles (128 registers).
// With WAVES = 4 it runs 128-row tiles: the halves of a launch's ragged last
// round, and whole launches whose 256-row tiles would leave CUs idle.  The
// decode per MFMA is the 256-row kernel's (each weight still feeds 256
// tokens); the token fragments are read from LDS twice as often (1 KiB per
// MFMA).
//
// Substep s (stage s, ring slot s & 7), one barrier each, 16 MFMA slots
// x = 8 kk + j (fragment j, k16 step kk), fenced from one another:
//   after the MFMA of slot x, the LDS read of the fragment slot x + 8 needs
//   (step 1 of stage s, or step 0 of stage s+1) into the register slot x
//   has just used; slot 0 also reads the lane's codes of stage s+2;
//   slots 1, 3: token DMA of stage s + kR8Ahead; odd s, slot 5: the wave's
//   code DMA of chunk (s+7)/2; even s, slots 5, 7: absmax code and group
//   scale of block s/2 + 3;
//   VALU chunks: odd s builds the table of block (s+1)/2 (slots 0..5);
//   step 1 of stage s+1 is decoded next, step 0 after slot 7 (into the
//   registers of step 0 of stage s).
// ===========================================================================
constexpr int kR8Ahead = 6;                                          // token stages DMA'd ahead of use
static_assert(kR8Ahead >= 2 && kR8Ahead <= 6, "ring / code-chunk schedule");
// Loads of substep v, token DMAs first: 16 / WAVES token DMAs per wave, then
// 1 code DMA (odd v) or 2 scale loads (even v).
constexpr int fwd8_tail(int v) { return (v & 1) ? 1 : 2; }
template <int WAVES>
constexpr int fwd8_loads(int v) { return 16 / WAVES + fwd8_tail(v); }
// vmcnt at the start of substep u: every load of substep u + 1 - kR8Ahead
// has landed once only the loads of the later substeps may be in flight.
// That covers token stage u+1 and the code chunk c DMA'd at substep 2c - 7,
// which substep 2c - 2 reads first.
template <int WAVES>
constexpr int fwd8_vmcnt(int u) {
  int n = 0;
  for (int v = u + 2 - kR8Ahead; v <= u - 1; ++v) n += fwd8_loads<WAVES>(v);
  return n;
}
static_assert(fwd8_vmcnt<4>(0) < 64 && fwd8_vmcnt<4>(1) < 64, "vmcnt field");

struct Fwd8 {
  rsrc_t xr, cr;
  uint32_t xo[4];         // lane offsets of the wave's token DMA instructions (16 / WAVES of them)
  uint32_t co;            // lane offset of the wave's code DMA (row 32 w + (lane & 31), stage half lane >> 5)
  const uint8_t* aq;      // absmax codes of the lane's row (block 0)
  const float* gs;
  uint32_t ablk0;
  int nsub, nblk, w;
  int crow;               // byte offset of the lane's 8 code bytes in a chunk buffer (stage half 0)
  int absfmt;             // second-level format of the block constants
};

// Token DMA instruction q of wave w fills tile rows 16 ((16 / WAVES) w + q) .. +15.
template <int WAVES>
__device__ __forceinline__ void fwd8_dma_x(char* smem, const Fwd8& f, int q, int stage, int slot) {
  const uint32_t soff = (uint32_t)min(stage, f.nsub - 1) * 64u;
  dma16(f.xr, smem + slot * kOp + ((16 / WAVES) * f.w + q) * 1024, f.xo[q], soff);
}
template <int BUF>
__device__ __forceinline__ void fwd8_dma_codes(char* smem, const Fwd8& f, int chunk) {
  const uint32_t soff = (uint32_t)min(chunk, (f.nsub >> 1) - 1) * 32u;
  dma16(f.cr, smem + kRCodeBase + BUF * kRChunk + f.w * 1024, f.co, soff);
}
__device__ __forceinline__ uint2 fwd8_codes(const char* smem, const Fwd8& f, int st) {
  const u32x2_t v = *reinterpret_cast<const u32x2_t*>(smem + kRCodeBase + ((st >> 1) & 3) * kRChunk + (st & 1) * 512 +
                                                      f.crow);
  return make_uint2(v.x, v.y);
}

template <int CB, int WAVES, int U8, int X>
__device__ __forceinline__ void fwd8_slot(char* smem, const Fwd8& f, int s, f32x16_t (&acc)[8], bf16x8_t (&b)[8],
                                          bf16x8_t& a0, bf16x8_t& a1, bf16x8_t& n1, uint2& c, uint2& cn,
                                          Nf4Table& T, Scale (&sc)[4], DqState& dq, TbState& tb, int fo0, int fo1) {
  constexpr bool kOdd = (U8 & 1) != 0;
  constexpr int kk = X >> 3, j = X & 7;
  acc[j] = mfma32x32x16(kk ? a1 : a0, b[j], acc[j]);
  if constexpr (kk == 0)
    b[j] = rd16(smem + U8 * kOp + j * 2048 + fo1);
  else
    b[j] = rd16(smem + ((U8 + 1) & 7) * kOp + j * 2048 + fo0);
  if constexpr (X == 0) cn = fwd8_codes(smem, f, s + 2);
  // global loads
  if constexpr (X >= 1 && X <= 16 / WAVES) fwd8_dma_x<WAVES>(smem, f, X - 1, s + kR8Ahead, (U8 + kR8Ahead) & 7);
  if constexpr (kOdd && X == 5) fwd8_dma_codes<((U8 + 7) >> 1) & 3>(smem, f, (s + 7) >> 1);
  if constexpr (!kOdd && (X == 5 || X == 7)) {
    constexpr int SL = ((U8 >> 1) + 3) & 3;
    const int bk = min((s >> 1) + 3, f.nblk - 1);
    if constexpr (X == 5)
      sc[SL].q = f.aq[bk];
    else
      sc[SL].s2 = f.gs[(f.ablk0 + (uint32_t)bk) >> 8];
  }
  // VALU chunks
  if constexpr (kOdd) {
    constexpr int SL = ((U8 + 1) >> 1) & 3;
    if constexpr (X < 6) tb_chunk<CB, X>(tb, sc[SL], T, f.absfmt);
    else if constexpr (X < 11) dq_chunk<X - 6>(dq, c.y, T, n1);
    else dq_chunk<X - 11>(dq, c.x, T, a0);
  } else {
    if constexpr (X < 5) dq_chunk<X>(dq, c.y, T, n1);
    else if constexpr (X >= 8 && X < 13) dq_chunk<X - 8>(dq, c.x, T, a0);
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <int CB, int WAVES, int U8>
__device__ __forceinline__ void fwd8_substep(char* smem, const Fwd8& f, int s, f32x16_t (&acc)[8], bf16x8_t (&b)[8],
                                             bf16x8_t& a0, bf16x8_t& a1, uint2& c, Nf4Table& T, Scale (&sc)[4],
                                             int fo0, int fo1) {
  __builtin_amdgcn_sched_barrier(0);
  QLORA_WAIT(fwd8_vmcnt<WAVES>(U8), 15);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  bf16x8_t n1;
  uint2 cn;
  DqState dq;
  TbState tb;
#define QLORA_FWD8_SLOT(x) fwd8_slot<CB, WAVES, U8, x>(smem, f, s, acc, b, a0, a1, n1, c, cn, T, sc, dq, tb, fo0, fo1)
#define QLORA_FWD8_SLOT4(x) QLORA_FWD8_SLOT(x); QLORA_FWD8_SLOT(x + 1); QLORA_FWD8_SLOT(x + 2); QLORA_FWD8_SLOT(x + 3)
  QLORA_FWD8_SLOT4(0); QLORA_FWD8_SLOT4(4); QLORA_FWD8_SLOT4(8); QLORA_FWD8_SLOT4(12);
#undef QLORA_FWD8_SLOT4
#undef QLORA_FWD8_SLOT
  a1 = n1;
  c = cn;
}

// Token half of the LoRA tail with THREADS threads: (s U)[m0 + row, j0 + 8 c ..].
template <int THREADS>
__device__ __forceinline__ void tail_tokens8(char* dst, const bf16_t* Ut, int64_t rows, int r, int64_t row0, int j0,
                                             float s) {
#pragma unroll
  for (int e = 0; e < 1024 / THREADS; ++e) {
    const int idx = threadIdx.x + THREADS * e;
    const int row = idx >> 2, cc = idx & 3, col = j0 + 8 * cc;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (col < r && row0 + row < rows) v = scale16(*reinterpret_cast<const uint4*>(Ut + (row0 + row) * r + col), s);
    wr16(dst + spos(row, cc), v);
  }
}

// WAVES waves own 32 WAVES weight rows of a 256-token tile.  TAIL_BASE < 0:
// the tiles are those of a grid of 32 WAVES-row tiles (map_tile).  Otherwise
// (WAVES == 4) workgroup b takes half b & 1 (128 rows) of 256-row tile
// tail_base + b / 2 in the row-major order of a tiles_n x tiles_m grid of
// 256 x 256 tiles: the split last round of a launch whose tile count is not
// a multiple of the CU count.
template <int CB, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 1) void nf4_fwd_n32_kernel(Nf4View W, const bf16_t* __restrict__ X,
                                                                    int64_t M, const bf16_t* __restrict__ U,
                                                                    const bf16_t* __restrict__ Bl, int r, float s,
                                                                    bf16_t* __restrict__ Y, int tiles_n, int tiles_m,
                                                                    int tail_base) {
  extern __shared__ __align__(16) char smem[];
  int64_t n0, m0;
  if (tail_base < 0) {
    int tn, tm;
    map_tile(tiles_n, tiles_m, tn, tm);
    n0 = (int64_t)tn * 32 * WAVES;
    m0 = (int64_t)tm * kTile;
  } else {
    const int p = tail_base + (int)(blockIdx.x >> 1);
    n0 = (int64_t)(p % tiles_n) * kTile + 128 * (blockIdx.x & 1);
    m0 = (int64_t)(p / tiles_n) * kTile;
  }
  const int t = threadIdx.x, lane = t & 63, lr = lane & 31, h = lane >> 5;
  const int64_t N = W.N, K = W.K;

  Fwd8 f;
  f.w = __builtin_amdgcn_readfirstlane(t >> 6);
  __builtin_assume(f.w >= 0 && f.w < WAVES);
  f.nsub = (int)(K >> 5);
  f.absfmt = W.absfmt;
  f.nblk = (int)(K >> 6);
  f.xr = make_rsrc(X, (uint32_t)(M * K * 2));
  f.cr = make_rsrc(W.codes, (uint32_t)(N * K / 2));
  // token DMA: instruction q of wave w fills tile rows 16 ((16 / WAVES) w +
  // q) .. +15, four lanes per row (lane j: row j >> 2, position j & 3
  // holding chunk dma_chunk(j))
#pragma unroll
  for (int q = 0; q < 16 / WAVES; ++q) {
    const int row = 16 * ((16 / WAVES) * f.w + q) + (lane >> 2);
    const int64_t xm = min(m0 + row, M - 1);   // rows past the end re-read the last row: never stored
    f.xo[q] = (uint32_t)(xm * K * 2 + dma_chunk(lane) * 16);
  }
  const int64_t own = min(n0 + 32 * f.w + lr, N - 1);
  // code DMA: lane l brings stage half l >> 5 of row 32 w + (l & 31)
  f.co = (uint32_t)(own * (K / 2) + 16 * h);
  f.crow = f.w * 1024 + lr * 16 + 8 * h;
  f.ablk0 = (uint32_t)(own * (K >> 6));
  f.aq = W.absmax_q + f.ablk0;
  f.gs = W.group_scale;
  const int fo0 = spos(lr, 2 * h), fo1 = spos(lr, 2 * h + 1);

  f32x16_t acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;

  // prologue: code chunks 0..3, scales of blocks 0..2, token stages 0 .. kR8Ahead - 1
  fwd8_dma_codes<0>(smem, f, 0);
  fwd8_dma_codes<1>(smem, f, 1);
  fwd8_dma_codes<2>(smem, f, 2);
  fwd8_dma_codes<3>(smem, f, 3);
  Scale sc[4];
#pragma unroll
  for (int bk = 0; bk < 3; ++bk) {
    const int b2 = min(bk, f.nblk - 1);
    sc[bk] = Scale{f.aq[b2], f.gs[(f.ablk0 + (uint32_t)b2) >> 8]};
  }
#pragma unroll
  for (int st = 0; st < kR8Ahead; ++st)
#pragma unroll
    for (int q = 0; q < 16 / WAVES; ++q) fwd8_dma_x<WAVES>(smem, f, q, st, st);
  QLORA_WAIT(0, 0);
  __builtin_amdgcn_s_barrier();
  Nf4Table T = make_table<CB>(block_scale(sc[0].q, sc[0].s2, f.absfmt));
  bf16x8_t a0, a1;
  {
    const uint2 c0 = fwd8_codes(smem, f, 0);
    a0 = deq_frag(c0.x, T);
    a1 = deq_frag(c0.y, T);
  }
  uint2 c = fwd8_codes(smem, f, 1);
  bf16x8_t b[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) b[j] = rd16(smem + j * 2048 + fo0);
  // K % 64 == 0, so the stage count is even
  int st = 0;
#define QLORA_FWD8_SUB(u) fwd8_substep<CB, WAVES, u>(smem, f, st + u, acc, b, a0, a1, c, T, sc, fo0, fo1)
  for (; st + 8 <= f.nsub; st += 8) {
    QLORA_FWD8_SUB(0); QLORA_FWD8_SUB(1); QLORA_FWD8_SUB(2); QLORA_FWD8_SUB(3);
    QLORA_FWD8_SUB(4); QLORA_FWD8_SUB(5); QLORA_FWD8_SUB(6); QLORA_FWD8_SUB(7);
  }
  const int rem = f.nsub - st;
  if (rem >= 2) { QLORA_FWD8_SUB(0); QLORA_FWD8_SUB(1); }
  if (rem >= 4) { QLORA_FWD8_SUB(2); QLORA_FWD8_SUB(3); }
  if (rem >= 6) { QLORA_FWD8_SUB(4); QLORA_FWD8_SUB(5); }
#undef QLORA_FWD8_SUB
  // drain the DMAs and reads still in flight (clamped re-loads) before reusing the ring
  QLORA_WAIT(0, 0);
  __builtin_amdgcn_s_barrier();

  if (r > 0) {
    // LoRA up-projection: acc += B (s U)^T over the rank, 32 at a time; the
    // weight operand comes straight from B (row of the lane, ranks 16h + 8kk)
    for (int j0 = 0; j0 < r; j0 += 32) {
      tail_tokens8<64 * WAVES>(smem, U, M, r, m0, j0, s);
      bf16x8_t a[2];
      const int64_t n = n0 + 32 * f.w + lr;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int col = j0 + 16 * h + 8 * kk;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (col < r && n < N) v = *reinterpret_cast<const uint4*>(Bl + n * r + col);
        a[kk] = __builtin_bit_cast(bf16x8_t, v);
      }
      QLORA_WAIT(0, 0);
      __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = mfma32x32x16(a[kk], rd16(smem + j * 2048 + (kk ? fo1 : fo0)), acc[j]);
      QLORA_WAIT(0, 0);
      __builtin_amdgcn_s_barrier();
    }
  }
  // Output: lane (lr, h) of wave w holds token m0 + 32 j + lr and weight
  // columns n0 + 32 w + 8 q + 4 h + 0..3; out through LDS (16 WAVES KiB)
  static_assert(64 * WAVES == kThreads, "the LDS write-out runs on kThreads threads");
  lds_free_for_output();
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      lds_put4<8 * WAVES, 31>(smem, 32 * j + lr, 8 * f.w + 2 * q + h, acc[j][4 * q], acc[j][4 * q + 1],
                              acc[j][4 * q + 2], acc[j][4 * q + 3]);
  __syncthreads();
  lds_tile_out<8 * WAVES, 31>(smem, Y, N, M, N, m0, n0);
}

// ===========================================================================
// Backward: dX = dY deq(W) + s G A.  Output tile 256 (m) x 256 (k); the
// contraction runs over n.  Weight half of a stage = 32 rows n x 256
// columns k, rows of 512 bytes with 32-byte block b of row n at position
// b ^ (n & 3), read transposed (ds_read_b64_tr_b16) as the A operand: the
// four rows that one 16-lane group of a transposed read touches land on
// four different 32-byte bank groups.  Thread t dequantizes row t >> 3,
// columns 32 (t & 7) .. +31 (its codes are 16 coalesced bytes), chunk p in
// order p ^ ((t >> 2) & 1), which keeps the 16-byte writes conflict-free.
// The dY tile goes through registers: the transposed reads cannot be told
// apart from DMA destinations by the compiler, which would then wait for
// every DMA in flight before each of them.
// ===========================================================================
constexpr int kWRow = 512;
constexpr size_t kLdsDx = (size_t)kStages * kStage;   // 128 KiB
__device__ __forceinline__ int tpos(int n, int b) { return n * kWRow + 32 * (b ^ (n & 3)); }

// A fragment: columns of 8 contraction rows (two transposed reads 4 rows apart).
__device__ __forceinline__ bf16x8_t tfrag(const char* p) {
  const uint2 lo = rd_tr(p), hi = rd_tr(p + 4 * kWRow);
  return __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

struct Dx {
  rsrc_t yr, cr, ar, gr;      // dY, codes, absmax codes, group scales
  uint32_t yo[4];             // dY lane offsets of the four 16-byte pieces (stage 0)
  int ypos[4];                // their LDS offsets within a token half
  uint32_t co, ao;            // codes / absmax lane offsets at stage 0
  uint32_t cstride, astride;  // per-stage strides (32 rows)
  uint32_t ablk, kb;          // block index at stage 0, K / 64
  int nsub;
  int absfmt;             // second-level format of the block constants
};
struct Codes {
  uint4 c;
  uint32_t q;
  float s2;
};
struct YRegs {
  uint4 v[4];
};

// Codes, absmax code and group scale of a stage for this thread.  Rows past
// N read as zero through the buffer range check: absmax code 0 gives block
// scale 0, so those rows dequantize to zero and meet the padded dY columns.
__device__ __forceinline__ void dx_load_codes(Codes& c, const Dx& d, int stage) {
  const uint32_t st = (uint32_t)min(stage, d.nsub - 1);
  c.c = buf_load16(d.cr, d.co, st * d.cstride);
  c.q = __builtin_amdgcn_raw_buffer_load_b8(d.ar, d.ao, st * d.astride, 0);
  const uint32_t g = (d.ablk + st * 32u * d.kb) >> 8;
  c.s2 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(d.gr, g * 4u, 0, 0));
}
__device__ __forceinline__ void dx_load_y(YRegs& y, const Dx& d, int stage) {
  const uint32_t soff = (uint32_t)min(stage, d.nsub - 1) * 64u;
#pragma unroll
  for (int q = 0; q < 4; ++q) y.v[q] = buf_load16(d.yr, d.yo[q], soff);
}
__device__ __forceinline__ void dx_store_y(char* smem, const Dx& d, const YRegs& y, int buf) {
  char* dst = smem + buf * kStage + kOp;
#pragma unroll
  for (int q = 0; q < 4; ++q) wr16(dst + d.ypos[q], y.v[q]);
}
// Dequantize chunks 2 half, 2 half + 1 of this thread's 32 columns into
// ring buffer `buf`.
__device__ __forceinline__ void dx_produce(char* smem, const Codes& c, const Nf4Table& T, int buf, int half) {
  const int t = threadIdx.x, n = t >> 3, j = t & 7, flip = (t >> 2) & 1;
  char* base = smem + buf * kStage;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int p = (2 * half + k) ^ flip;
    const uint32_t word = p == 0 ? c.c.x : p == 1 ? c.c.y : p == 2 ? c.c.z : c.c.w;
    uint32_t o[4];
    dequant8(word, T, o);
    const int ch = 4 * j + p;   // 16-byte chunk of the row (8 columns)
    wr16(base + tpos(n, ch >> 1) + 16 * (ch & 1), make_uint4(o[0], o[1], o[2], o[3]));
  }
}

// Substep s, U8 = s mod 8, one barrier at its start: the barrier makes stage
// s+1 (dequantized and stored during substep s-1) visible, and every wave has
// finished reading stage s-2, whose ring buffer (s+2) & 3 this substep fills.
// 32 MFMA slots, fenced one from another; slot x = 16 kk + 4 i + j is
// fragment (i, j) of k16 step kk.  Besides its MFMA a slot carries:
//   LDS reads     slots 0..11: step 1 of stage s (A fragment i in slots 2i,
//                 2i + 1, B fragment j in slot 8 + j); slots 16..27: step 0
//                 of stage s+1 in the same pattern, into the registers
//                 step 0 of stage s has finished with
//   global loads  slots 1, 3, 5, 7: dY of stage s+3; slots 9, 11, 13:
//                 codes, absmax code and group scale of stage s+4
//   LDS writes    slots 2, 6, 10, 14: dY of stage s+2 (loaded last
//                 substep); slots 11, 16, 21, 26: the four dequantized
//                 16-byte chunks of stage s+2
//   VALU chunks   slots 0..5: table of the thread's row and block; slots
//                 6..25: the four decodes, five chunks each
template <int I>
__device__ __forceinline__ uint32_t u4_word(const uint4& v) {
  return I == 0 ? v.x : I == 1 ? v.y : I == 2 ? v.z : v.w;
}

template <int CB, int U8, int X>
__device__ __forceinline__ void dx_slot(char* smem, const Dx& d, int s, f32x16_t (&acc)[4][4], Frags& F,
                                        Codes (&cs)[4], YRegs (&ys)[2], const int (&ao)[4], int bm, FragOffs fo,
                                        TbState& tb, Nf4Table& T, DqState& dq, bf16x8_t& dqo) {
  constexpr int U = U8 & 3;
  constexpr int kk = X >> 4, i = (X >> 2) & 3, j = X & 3, y = X & 15;
  const char* cur = smem + U * kStage;
  const char* nxt = smem + ((U + 1) & 3) * kStage;
  if constexpr (kk == 0)
    acc[i][j] = mfma32x32x16(F.a0[i], F.b0[j], acc[i][j]);
  else
    acc[i][j] = mfma32x32x16(F.a1[i], F.b1[j], acc[i][j]);
  // LDS reads: A fragment r = y / 2 is two transposed reads 4 rows apart
  if constexpr (y < 8) {
    constexpr int r = y >> 1, part = y & 1;
    const char* p = (kk == 0 ? cur + 16 * kWRow : nxt) + ao[r] + part * 4 * kWRow;
    const uint2 v = rd_tr(p);
    bf16x8_t& a = kk == 0 ? F.a1[r] : F.a0[r];
    uint4 w = __builtin_bit_cast(uint4, a);
    if constexpr (part == 0) {
      w.x = v.x;
      w.y = v.y;
    } else {
      w.z = v.x;
      w.w = v.y;
    }
    a = __builtin_bit_cast(bf16x8_t, w);
  } else if constexpr (y < 12) {
    if constexpr (kk == 0)
      F.b1[y - 8] = rd16(cur + kOp + bm + (y - 8) * 2048 + fo.o1);
    else
      F.b0[y - 8] = rd16(nxt + kOp + bm + (y - 8) * 2048 + fo.o0);
  }
  // global loads
  if constexpr (kk == 0 && y < 8 && (y & 1)) {
    const uint32_t soff = (uint32_t)min(s + 3, d.nsub - 1) * 64u;
    ys[U8 & 1].v[y >> 1] = buf_load16(d.yr, d.yo[y >> 1], soff);
  }
  if constexpr (kk == 0 && (y == 9 || y == 11 || y == 13)) {
    const uint32_t st = (uint32_t)min(s + 4, d.nsub - 1);
    if constexpr (y == 9) cs[U].c = buf_load16(d.cr, d.co, st * d.cstride);
    if constexpr (y == 11) cs[U].q = __builtin_amdgcn_raw_buffer_load_b8(d.ar, d.ao, st * d.astride, 0);
    if constexpr (y == 13) {
      const uint32_t g = (d.ablk + st * 32u * d.kb) >> 8;
      cs[U].s2 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(d.gr, g * 4u, 0, 0));
    }
  }
  // LDS writes
  if constexpr (kk == 0 && (y & 3) == 2) wr16(smem + ((U + 2) & 3) * kStage + kOp + d.ypos[y >> 2],
                                                ys[(U8 + 1) & 1].v[y >> 2]);
  constexpr int kProduced = (X == 11) ? 0 : (X == 16) ? 1 : (X == 21) ? 2 : (X == 26) ? 3 : -1;
  if constexpr (kProduced >= 0) {
    const int t = threadIdx.x, n = t >> 3, jj = t & 7, flip = (t >> 2) & 1;
    const int p = kProduced ^ flip, ch = 4 * jj + p;   // 16-byte chunk of the row (8 columns)
    wr16(smem + ((U + 2) & 3) * kStage + tpos(n, ch >> 1) + 16 * (ch & 1), __builtin_bit_cast(uint4, dqo));
  }
  // VALU chunks: stage s+2 from code set (U + 2) & 3
  {
    const Codes& pc = cs[(U + 2) & 3];
    if constexpr (X < 6) {
      tb_chunk<CB, X>(tb, Scale{pc.q, pc.s2}, T, d.absfmt);
    } else if constexpr (X < 26) {
      constexpr int dd = (X - 6) / 5, kc = (X - 6) % 5;
      // chunk dd ^ flip: a select between two fixed words (a runtime index
      // into the code registers would send them to scratch)
      const bool flip = (threadIdx.x & 4) != 0;
      const uint32_t word = flip ? u4_word<dd ^ 1>(pc.c) : u4_word<dd>(pc.c);
      dq_chunk<kc>(dq, word, T, dqo);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <int CB, int U8>
__device__ __forceinline__ void dx_substep(char* smem, const Dx& d, int s, f32x16_t (&acc)[4][4], Frags& F,
                                           Codes (&cs)[4], YRegs (&ys)[2], const int (&ao)[4], int bm,
                                           FragOffs fo) {
  __builtin_amdgcn_sched_barrier(0);
  QLORA_WAIT(63, 0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  TbState tb;
  Nf4Table T;
  DqState dq;
  bf16x8_t dqo;
#define QLORA_DX_SLOT(x) dx_slot<CB, U8, x>(smem, d, s, acc, F, cs, ys, ao, bm, fo, tb, T, dq, dqo)
#define QLORA_DX_SLOT4(x) QLORA_DX_SLOT(x); QLORA_DX_SLOT(x + 1); QLORA_DX_SLOT(x + 2); QLORA_DX_SLOT(x + 3)
  QLORA_DX_SLOT4(0); QLORA_DX_SLOT4(4); QLORA_DX_SLOT4(8); QLORA_DX_SLOT4(12);
  QLORA_DX_SLOT4(16); QLORA_DX_SLOT4(20); QLORA_DX_SLOT4(24); QLORA_DX_SLOT4(28);
#undef QLORA_DX_SLOT4
#undef QLORA_DX_SLOT
}

template <int CB>
__global__ __launch_bounds__(kThreads, 1) void nf4_dx_kernel(Nf4View W, const bf16_t* __restrict__ dY, int64_t M,
                                                             const bf16_t* __restrict__ G,
                                                             const bf16_t* __restrict__ Al, int r, float s,
                                                             bf16_t* __restrict__ dX, int tiles_k, int tiles_m) {
  extern __shared__ __align__(16) char smem[];
  int tk, tm;
  map_tile(tiles_k, tiles_m, tk, tm);
  const int64_t k0 = (int64_t)tk * kTile, m0 = (int64_t)tm * kTile;
  const int t = threadIdx.x, lane = t & 63, wr = (t >> 6) >> 1, wc = (t >> 6) & 1;
  const int64_t N = W.N, K = W.K;

  Dx d;
  d.yr = make_rsrc(dY, (uint32_t)(M * N * 2));
  d.cr = make_rsrc(W.codes, (uint32_t)(N * K / 2));
  d.ar = make_rsrc(W.absmax_q, (uint32_t)(N * (K >> 6)));
  d.gr = make_rsrc(W.group_scale, (uint32_t)(((N * (K >> 6) + 255) >> 8) * 4));
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int idx = t + kThreads * q, row = idx >> 2, c = idx & 3;
    const int64_t ym = min(m0 + row, M - 1);
    d.yo[q] = (uint32_t)(ym * N * 2 + c * 16);
    d.ypos[q] = spos(row, c);
  }
  {
    const int64_t kc = min(k0 + 32 * (t & 7), K - 32);   // columns past K: any in-range block
    const int64_t n = t >> 3;
    d.kb = (uint32_t)(K >> 6);
    d.co = (uint32_t)(n * (K / 2) + kc / 2);
    d.ao = (uint32_t)(n * (K >> 6) + (kc >> 6));
    d.ablk = d.ao;
    d.cstride = (uint32_t)(32 * (K / 2));
    d.astride = (uint32_t)(32 * (K >> 6));
  }
  d.nsub = (int)((N + 31) >> 5);
  d.absfmt = W.absfmt;
  // A fragment i: as a source lane of its 16-lane group (g, sl) a lane reads
  // row 8 (g >> 1) + (sl >> 2) and columns 128 wc + 32 i + 16 (g & 1) + 4 (sl & 3)
  int ao[4];
  {
    const int g = lane >> 4, sl = lane & 15, n0 = 8 * (g >> 1) + (sl >> 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) ao[i] = tpos(n0, wc * 8 + 2 * i + (g & 1)) + 8 * (sl & 3);
  }
  const FragOffs fo = frag_offs(lane);
  const int bm = wr * 128 * 64;

  f32x16_t acc[4][4];
  zero_acc(acc);

  Codes cs[4];
  YRegs ys[2];
#pragma unroll
  for (int p = 0; p < 4; ++p) dx_load_codes(cs[p], d, p);
  dx_load_y(ys[0], d, 0);
  dx_store_y(smem, d, ys[0], 0);
  dx_load_y(ys[0], d, 1);
  dx_store_y(smem, d, ys[0], 1);
  dx_load_y(ys[1], d, 2);   // stored by substep 0
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const Nf4Table T = make_table<CB>(block_scale(cs[p].q, cs[p].s2, d.absfmt));
    dx_produce(smem, cs[p], T, p, 0);
    dx_produce(smem, cs[p], T, p, 1);
  }
  QLORA_WAIT(0, 0);
  __builtin_amdgcn_s_barrier();
  Frags F;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    F.a0[i] = tfrag(smem + ao[i]);
    F.b0[i] = rd16(smem + kOp + bm + i * 2048 + fo.o0);
  }
  int st = 0;
#define QLORA_DX_SUB(u) dx_substep<CB, u>(smem, d, st + u, acc, F, cs, ys, ao, bm, fo)
  for (; st + 8 <= d.nsub; st += 8) {
    QLORA_DX_SUB(0); QLORA_DX_SUB(1); QLORA_DX_SUB(2); QLORA_DX_SUB(3);
    QLORA_DX_SUB(4); QLORA_DX_SUB(5); QLORA_DX_SUB(6); QLORA_DX_SUB(7);
  }
  const int rem = d.nsub - st;
  if (rem >= 1) QLORA_DX_SUB(0);
  if (rem >= 2) QLORA_DX_SUB(1);
  if (rem >= 3) QLORA_DX_SUB(2);
  if (rem >= 4) QLORA_DX_SUB(3);
  if (rem >= 5) QLORA_DX_SUB(4);
  if (rem >= 6) QLORA_DX_SUB(5);
  if (rem >= 7) QLORA_DX_SUB(6);
#undef QLORA_DX_SUB
  QLORA_WAIT(0, 0);
  __builtin_amdgcn_s_barrier();

  if (r > 0) {
    // acc += (s G) A over the rank, 32 at a time: rows j of A are
    // contraction rows of the weight half, copied without dequantization
    for (int j0 = 0; j0 < r; j0 += 32) {
      char* wb = smem;
      char* yb = smem + kOp;
      {
        const int n = t >> 3, jj = t & 7, flip = (t >> 2) & 1;
        const int64_t row = j0 + n;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int p = k ^ flip, ch = 4 * jj + p;
          const int64_t col = k0 + 8 * ch;
          uint4 v = make_uint4(0u, 0u, 0u, 0u);
          if (row < r && col < K) v = *reinterpret_cast<const uint4*>(Al + row * K + col);
          wr16(wb + tpos(n, ch >> 1) + 16 * (ch & 1), v);
        }
      }
      tail_tokens(yb, G, M, r, m0, j0, s);
      QLORA_WAIT(0, 0);
      __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int o = kk ? fo.o1 : fo.o0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          F.a0[i] = tfrag(wb + ao[i] + kk * 16 * kWRow);
          F.b0[i] = rd16(yb + bm + i * 2048 + o);
        }
        mfma_block<4, 4>(acc, F.a0, F.b0);
      }
      QLORA_WAIT(0, 0);
      __builtin_amdgcn_s_barrier();
    }
  }
  store_tile_lds(acc, dX, K, M, K, m0, k0, smem);
}

// ===========================================================================
// dX half tile: 256 tokens x 128 columns, for the last round of a launch
// whose full tiles would leave at least half of the CUs idle.  The ring,
// the substep and its single barrier are those of nf4_dx_kernel with half
// the weight columns: the weight half of a stage is 32 rows x 128 columns in
// rows of 256 bytes (32-byte block b of row n at b ^ (n & 3)), each thread
// dequantizes 16 weights (row t >> 3, columns 16 (t & 7) .. +15: 8 code
// bytes and one block), and wave (wr, wc) owns tokens 128 wr .. +127 against
// columns 64 wc .. +63, 16 MFMAs per stage.  Block b of the launch takes
// half b & 1 of tile tile_base + b / 2.
// ===========================================================================
constexpr int kWRowH = 256;
__device__ __forceinline__ int tposh(int n, int b) { return n * kWRowH + 32 * (b ^ (n & 3)); }
__device__ __forceinline__ bf16x8_t tfragh(const char* p) {
  const uint2 lo = rd_tr(p), hi = rd_tr(p + 4 * kWRowH);
  return __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

struct CodesH {
  uint2 c;
  uint32_t q;
  float s2;
};
struct FragsH {
  bf16x8_t a0[2], b0[4], a1[2], b1[4];
};

__device__ __forceinline__ void dxh_load_codes(CodesH& c, const Dx& d, int stage) {
  const uint32_t st = (uint32_t)min(stage, d.nsub - 1);
  const u32x2_t v = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(d.cr, d.co, st * d.cstride, 0));
  c.c = make_uint2(v.x, v.y);
  c.q = __builtin_amdgcn_raw_buffer_load_b8(d.ar, d.ao, st * d.astride, 0);
  const uint32_t g = (d.ablk + st * 32u * d.kb) >> 8;
  c.s2 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(d.gr, g * 4u, 0, 0));
}
// 16-byte chunk p (0, 1) of this thread's 16 columns, dequantized with T,
// into ring buffer `buf`; chunk p of thread (n, jj) is chunk 2 jj + p of row n
__device__ __forceinline__ void dxh_store_chunk(char* smem, int buf, int p, const bf16x8_t& v) {
  const int t = threadIdx.x, n = t >> 3, ch = 2 * (t & 7) + p;
  wr16(smem + buf * kStage + tposh(n, ch >> 1) + 16 * (ch & 1), __builtin_bit_cast(uint4, v));
}

// Slot x (0..15) of substep s: the MFMA of fragment pair (i, j) = ((x >> 2)
// & 1, x & 3) of k16 step x >> 3.  Besides it:
//   LDS reads     slots 0..7: step 1 of stage s (A fragment i in slots 2i,
//                 2i + 1, B fragment j in slot 4 + j); slots 8..15: step 0
//                 of stage s+1 in the same pattern, into the registers
//                 step 0 of stage s has finished with
//   global loads  slots 1, 3, 5, 7: dY of stage s+3; slots 9, 11, 13:
//                 codes, absmax code and group scale of stage s+4
//   LDS writes    slots 2, 6, 10, 14: dY of stage s+2 (loaded last
//                 substep); slot 11: the first dequantized chunk of stage
//                 s+2 (the second follows the last slot)
//   VALU chunks   slots 0..5: table of the thread's row and block; slots
//                 6..15: the two decodes, five chunks each
template <int CB, int U8, int X>
__device__ __forceinline__ void dxh_slot(char* smem, const Dx& d, int s, f32x16_t (&acc)[2][4], FragsH& F,
                                         CodesH (&cs)[4], YRegs (&ys)[2], const int (&ao)[2], int bm, FragOffs fo,
                                         TbState& tb, Nf4Table& T, DqState& dq, bf16x8_t& dqo) {
  constexpr int U = U8 & 3;
  constexpr int kk = X >> 3, i = (X >> 2) & 1, j = X & 3, y = X & 7;
  const char* cur = smem + U * kStage;
  const char* nxt = smem + ((U + 1) & 3) * kStage;
  if constexpr (kk == 0)
    acc[i][j] = mfma32x32x16(F.a0[i], F.b0[j], acc[i][j]);
  else
    acc[i][j] = mfma32x32x16(F.a1[i], F.b1[j], acc[i][j]);
  // LDS reads: A fragment r = y / 2 is two transposed reads 4 rows apart
  if constexpr (y < 4) {
    constexpr int r = y >> 1, part = y & 1;
    const char* p = (kk == 0 ? cur + 16 * kWRowH : nxt) + ao[r] + part * 4 * kWRowH;
    const uint2 v = rd_tr(p);
    bf16x8_t& a = kk == 0 ? F.a1[r] : F.a0[r];
    uint4 w = __builtin_bit_cast(uint4, a);
    if constexpr (part == 0) {
      w.x = v.x;
      w.y = v.y;
    } else {
      w.z = v.x;
      w.w = v.y;
    }
    a = __builtin_bit_cast(bf16x8_t, w);
  } else {
    if constexpr (kk == 0)
      F.b1[y - 4] = rd16(cur + kOp + bm + (y - 4) * 2048 + fo.o1);
    else
      F.b0[y - 4] = rd16(nxt + kOp + bm + (y - 4) * 2048 + fo.o0);
  }
  // global loads
  if constexpr (kk == 0 && (y & 1)) {
    const uint32_t soff = (uint32_t)min(s + 3, d.nsub - 1) * 64u;
    ys[U8 & 1].v[y >> 1] = buf_load16(d.yr, d.yo[y >> 1], soff);
  }
  if constexpr (X == 9 || X == 11 || X == 13) {
    const uint32_t st = (uint32_t)min(s + 4, d.nsub - 1);
    if constexpr (X == 9) {
      const u32x2_t v =
          __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(d.cr, d.co, st * d.cstride, 0));
      cs[U].c = make_uint2(v.x, v.y);
    }
    if constexpr (X == 11) cs[U].q = __builtin_amdgcn_raw_buffer_load_b8(d.ar, d.ao, st * d.astride, 0);
    if constexpr (X == 13) {
      const uint32_t g = (d.ablk + st * 32u * d.kb) >> 8;
      cs[U].s2 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(d.gr, g * 4u, 0, 0));
    }
  }
  // LDS writes
  if constexpr ((X & 3) == 2)
    wr16(smem + ((U + 2) & 3) * kStage + kOp + d.ypos[X >> 2], ys[(U8 + 1) & 1].v[X >> 2]);
  if constexpr (X == 11) dxh_store_chunk(smem, (U + 2) & 3, (threadIdx.x >> 2) & 1, dqo);
  // VALU chunks: stage s+2 from code set (U + 2) & 3
  {
    const CodesH& pc = cs[(U + 2) & 3];
    if constexpr (X < 6) {
      tb_chunk<CB, X>(tb, Scale{pc.q, pc.s2}, T, d.absfmt);
    } else {
      constexpr int dd = (X - 6) / 5, kc = (X - 6) % 5;
      // decode dd is chunk dd ^ flip: a select between the two code words as
      // values (a select between the fields would go through scratch)
      const bool flip = (threadIdx.x & 4) != 0;
      const uint32_t cx = pc.c.x, cy = pc.c.y;
      const uint32_t word = (flip != (dd != 0)) ? cy : cx;
      dq_chunk<kc>(dq, word, T, dqo);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <int CB, int U8>
__device__ __forceinline__ void dxh_substep(char* smem, const Dx& d, int s, f32x16_t (&acc)[2][4], FragsH& F,
                                            CodesH (&cs)[4], YRegs (&ys)[2], const int (&ao)[2], int bm,
                                            FragOffs fo) {
  constexpr int U = U8 & 3;
  __builtin_amdgcn_sched_barrier(0);
  QLORA_WAIT(63, 0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  TbState tb;
  Nf4Table T;
  DqState dq;
  bf16x8_t dqo;
#define QLORA_DXH_SLOT(x) dxh_slot<CB, U8, x>(smem, d, s, acc, F, cs, ys, ao, bm, fo, tb, T, dq, dqo)
#define QLORA_DXH_SLOT4(x) QLORA_DXH_SLOT(x); QLORA_DXH_SLOT(x + 1); QLORA_DXH_SLOT(x + 2); QLORA_DXH_SLOT(x + 3)
  QLORA_DXH_SLOT4(0); QLORA_DXH_SLOT4(4); QLORA_DXH_SLOT4(8); QLORA_DXH_SLOT4(12);
#undef QLORA_DXH_SLOT4
#undef QLORA_DXH_SLOT
  // the second dequantized chunk of stage s+2
  dxh_store_chunk(smem, (U + 2) & 3, ((threadIdx.x >> 2) & 1) ^ 1, dqo);
}

template <int CB>
__global__ __launch_bounds__(kThreads, 1) void nf4_dx_half_kernel(Nf4View W, const bf16_t* __restrict__ dY,
                                                                  int64_t M, const bf16_t* __restrict__ G,
                                                                  const bf16_t* __restrict__ Al, int r, float s,
                                                                  bf16_t* __restrict__ dX, int tiles_k,
                                                                  int tile_base) {
  extern __shared__ __align__(16) char smem[];
  const int tile = tile_base + (int)(blockIdx.x >> 1);
  const int tk = tile % tiles_k, tm = tile / tiles_k;
  const int64_t k0 = (int64_t)tk * kTile + 128 * (int64_t)(blockIdx.x & 1), m0 = (int64_t)tm * kTile;
  const int t = threadIdx.x, lane = t & 63, wr = (t >> 6) >> 1, wc = (t >> 6) & 1;
  const int64_t N = W.N, K = W.K;

  Dx d;
  d.yr = make_rsrc(dY, (uint32_t)(M * N * 2));
  d.cr = make_rsrc(W.codes, (uint32_t)(N * K / 2));
  d.ar = make_rsrc(W.absmax_q, (uint32_t)(N * (K >> 6)));
  d.gr = make_rsrc(W.group_scale, (uint32_t)(((N * (K >> 6) + 255) >> 8) * 4));
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int idx = t + kThreads * q, row = idx >> 2, c = idx & 3;
    const int64_t ym = min(m0 + row, M - 1);
    d.yo[q] = (uint32_t)(ym * N * 2 + c * 16);
    d.ypos[q] = spos(row, c);
  }
  {
    const int64_t kc = min(k0 + 16 * (t & 7), K - 16);   // columns past K: any in-range block
    const int64_t n = t >> 3;
    d.kb = (uint32_t)(K >> 6);
    d.co = (uint32_t)(n * (K / 2) + kc / 2);
    d.ao = (uint32_t)(n * (K >> 6) + (kc >> 6));
    d.ablk = d.ao;
    d.cstride = (uint32_t)(32 * (K / 2));
    d.astride = (uint32_t)(32 * (K >> 6));
  }
  d.nsub = (int)((N + 31) >> 5);
  d.absfmt = W.absfmt;
  // A fragment i: as a source lane of its 16-lane group (g, sl) a lane reads
  // row 8 (g >> 1) + (sl >> 2) and columns 64 wc + 32 i + 16 (g & 1) + 4 (sl & 3)
  int ao[2];
  {
    const int g = lane >> 4, sl = lane & 15, n0 = 8 * (g >> 1) + (sl >> 2);
#pragma unroll
    for (int i = 0; i < 2; ++i) ao[i] = tposh(n0, wc * 4 + 2 * i + (g & 1)) + 8 * (sl & 3);
  }
  const FragOffs fo = frag_offs(lane);
  const int bm = wr * 128 * 64;

  f32x16_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  CodesH cs[4];
  YRegs ys[2];
#pragma unroll
  for (int p = 0; p < 4; ++p) dxh_load_codes(cs[p], d, p);
  dx_load_y(ys[0], d, 0);
  dx_store_y(smem, d, ys[0], 0);
  dx_load_y(ys[0], d, 1);
  dx_store_y(smem, d, ys[0], 1);
  dx_load_y(ys[1], d, 2);   // stored by substep 0
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const Nf4Table T = make_table<CB>(block_scale(cs[p].q, cs[p].s2, d.absfmt));
    const int flip = (t >> 2) & 1;
    const uint32_t cx = cs[p].c.x, cy = cs[p].c.y;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      uint32_t o[4];
      dequant8((k ^ flip) ? cy : cx, T, o);
      dxh_store_chunk(smem, p, k ^ flip, __builtin_bit_cast(bf16x8_t, make_uint4(o[0], o[1], o[2], o[3])));
    }
  }
  QLORA_WAIT(0, 0);
  __builtin_amdgcn_s_barrier();
  FragsH F;
#pragma unroll
  for (int i = 0; i < 2; ++i) F.a0[i] = tfragh(smem + ao[i]);
#pragma unroll
  for (int j = 0; j < 4; ++j) F.b0[j] = rd16(smem + kOp + bm + j * 2048 + fo.o0);
  int st = 0;
#define QLORA_DXH_SUB(u) dxh_substep<CB, u>(smem, d, st + u, acc, F, cs, ys, ao, bm, fo)
  for (; st + 8 <= d.nsub; st += 8) {
    QLORA_DXH_SUB(0); QLORA_DXH_SUB(1); QLORA_DXH_SUB(2); QLORA_DXH_SUB(3);
    QLORA_DXH_SUB(4); QLORA_DXH_SUB(5); QLORA_DXH_SUB(6); QLORA_DXH_SUB(7);
  }
  const int rem = d.nsub - st;
  if (rem >= 1) QLORA_DXH_SUB(0);
  if (rem >= 2) QLORA_DXH_SUB(1);
  if (rem >= 3) QLORA_DXH_SUB(2);
  if (rem >= 4) QLORA_DXH_SUB(3);
  if (rem >= 5) QLORA_DXH_SUB(4);
  if (rem >= 6) QLORA_DXH_SUB(5);
  if (rem >= 7) QLORA_DXH_SUB(6);
#undef QLORA_DXH_SUB
  QLORA_WAIT(0, 0);
  __builtin_amdgcn_s_barrier();

  if (r > 0) {
    // acc += (s G) A over the rank, 32 at a time (as in nf4_dx_kernel)
    for (int j0 = 0; j0 < r; j0 += 32) {
      char* wb = smem;
      char* yb = smem + kOp;
      {
        const int n = t >> 3, jj = t & 7, flip = (t >> 2) & 1;
        const int64_t row = j0 + n;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int p = k ^ flip, ch = 2 * jj + p;
          const int64_t col = k0 + 8 * ch;
          uint4 v = make_uint4(0u, 0u, 0u, 0u);
          if (row < r && col < K) v = *reinterpret_cast<const uint4*>(Al + row * K + col);
          wr16(wb + tposh(n, ch >> 1) + 16 * (ch & 1), v);
        }
      }
      tail_tokens(yb, G, M, r, m0, j0, s);
      QLORA_WAIT(0, 0);
      __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int o = kk ? fo.o1 : fo.o0;
#pragma unroll
        for (int i = 0; i < 2; ++i) F.a0[i] = tfragh(wb + ao[i] + kk * 16 * kWRowH);
#pragma unroll
        for (int j = 0; j < 4; ++j) F.b0[j] = rd16(yb + bm + j * 2048 + o);
        mfma_block<2, 4>(acc, F.a0, F.b0);
      }
      QLORA_WAIT(0, 0);
      __builtin_amdgcn_s_barrier();
    }
  }
  store_tile_lds(acc, dX, K, M, K, m0, k0, smem);
}

}  // namespace

namespace {

template <int CB>
hipError_t launch_fwd_cb(const Nf4View& W, const bf16_t* X, int64_t M, const bf16_t* U, const bf16_t* B, int r,
                        float s, bf16_t* Y, hipStream_t st) {
  const int tiles_n = (int)((W.N + kTile - 1) / kTile);
  const int tiles_m = (int)((M + kTile - 1) / kTile);
  const int tiles = tiles_n * tiles_m;
  // When the last round of 256 x 256 tiles would leave at least half the CUs
  // idle, its tiles run as two 128-row halves each, in a second launch of
  // the 32-rows-per-wave kernel, so that round takes about half as long.
  const int cus = device_cu_count();   // the tail split needs the round size
  const int rest = tiles % cus;
  const int main_tiles = (tiles > cus && rest > 0 && 2 * rest <= cus) ? tiles - rest : tiles;
  hipError_t e = allow_lds(reinterpret_cast<const void*>(&nf4_fwd_r_kernel<CB>), (int)kLdsFwdR);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(nf4_fwd_r_kernel<CB>, dim3(main_tiles), dim3(kThreads), kLdsFwdR, st, W, X, M, U, B, r, s, Y,
                     tiles_n, tiles_m);
  e = hipGetLastError();
  if (e != hipSuccess || main_tiles == tiles) return e;
  auto* tail = &nf4_fwd_n32_kernel<CB, 4>;
  e = allow_lds(reinterpret_cast<const void*>(tail), (int)kLdsFwdR);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(tail, dim3(2 * (tiles - main_tiles)), dim3(kThreads), kLdsFwdR, st, W, X, M, U, B, r, s, Y,
                     tiles_n, tiles_m, main_tiles);
  return hipGetLastError();
}

template <int CB>
hipError_t launch_dx_cb(const Nf4View& W, const bf16_t* dY, int64_t M, const bf16_t* G, const bf16_t* A, int r,
                       float s, bf16_t* dX, hipStream_t st) {
  const int tiles_k = (int)((W.K + kTile - 1) / kTile);
  const int tiles_m = (int)((M + kTile - 1) / kTile);
  const int tiles = tiles_k * tiles_m;
  // As in the forward: a last round that would leave at least half of the
  // CUs idle runs as 128-column halves in a second launch.
  const int cus = device_cu_count();
  const int rest = tiles % cus;
  const int main_tiles = (tiles > cus && rest > 0 && 2 * rest <= cus) ? tiles - rest : tiles;
  hipError_t e = allow_lds(reinterpret_cast<const void*>(&nf4_dx_kernel<CB>), (int)kLdsDx);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(nf4_dx_kernel<CB>, dim3(main_tiles), dim3(kThreads), kLdsDx, st, W, dY, M, G, A, r, s, dX,
                     tiles_k, tiles_m);
  e = hipGetLastError();
  if (e != hipSuccess || main_tiles == tiles) return e;
  e = allow_lds(reinterpret_cast<const void*>(&nf4_dx_half_kernel<CB>), (int)kLdsDx);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(nf4_dx_half_kernel<CB>, dim3(2 * (tiles - main_tiles)), dim3(kThreads), kLdsDx, st, W, dY, M, G, A,
                     r, s, dX, tiles_k, main_tiles);
  return hipGetLastError();
}

}  // namespace

// The codebook is a template parameter of the kernels (its levels are
// literals in the block-table code).
hipError_t launch_fwd(const Nf4View& W, const bf16_t* X, int64_t M, const bf16_t* U, const bf16_t* B, int r,
                      float s, bf16_t* Y, hipStream_t st) {
  if (W.codebook == kCbFp4) return launch_fwd_cb<kCbFp4>(W, X, M, U, B, r, s, Y, st);
  if (W.codebook == kCbInt4) return launch_fwd_cb<kCbInt4>(W, X, M, U, B, r, s, Y, st);
  return launch_fwd_cb<kCbNf4>(W, X, M, U, B, r, s, Y, st);
}

hipError_t launch_dx(const Nf4View& W, const bf16_t* dY, int64_t M, const bf16_t* G, const bf16_t* A, int r,
                     float s, bf16_t* dX, hipStream_t st) {
  if (W.codebook == kCbFp4) return launch_dx_cb<kCbFp4>(W, dY, M, G, A, r, s, dX, st);
  if (W.codebook == kCbInt4) return launch_dx_cb<kCbInt4>(W, dY, M, G, A, r, s, dX, st);
  return launch_dx_cb<kCbNf4>(W, dY, M, G, A, r, s, dX, st);
}

}  // namespace qlora
