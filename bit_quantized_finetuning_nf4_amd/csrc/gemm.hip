// gemm.hip -- the four LoRA products of the QLoRA linear layer:
//
//   U = X A^T,  G = dY B            (contraction along the rows of X / dY)
//   dA = s G^T X,  dB = s dY^T U    (contraction over the tokens)
// (the fused NF4 GEMMs live in gemm_nf4.hip)
//
// deepfa.ir blog, "LoRA: Prerequisite" and "QLoRA's Working Process" (the
// 4-bit weights are dequantized to BF16 on the fly in the forward and
// backward passes, only the adapters are trained); glossary "QLoRA",
// Definition (weight gradients only for the LoRA matrices).
//
// All four read one large bf16 matrix (X or dY, M x K or M x N) once and a
// small one (A, B, G or U) with the rank r <= 128 on one side, so they are
// HBM streams with little arithmetic.  Both kernels below bring the large
// matrix into LDS by buffer->LDS DMA through a ring of six 32-row (or
// 32-column) stages, five stages ahead, one barrier per stage, and run a few
// bf16 MFMAs (32x32x16, fp32 accumulation) per stage.  The contraction is
// split over workgroups (about one per CU); each split writes fp32 partial
// sums and reduce_kernel adds them in a fixed order, so results do not
// depend on timing.  The rank side is padded to RP = 64 or 128 with values
// that only reach output columns >= r, which are never stored.
#include "device.h"
#include "kernels.h"
#include "lds.h"

namespace qlora {

namespace {

constexpr int kThreads = 256;
constexpr int kRing = 6;    // stages in the LDS ring
constexpr int kAhead = 5;   // stages DMA'd ahead of the one being multiplied

// DMA of a 32-row x (PB / 2)-column tile in the layout above: instruction q
// covers rows (512 / PB) q .. ; lane l writes byte 16 (l mod (PB / 16)) of
// its row, which holds global column 8 (2 ((p >> 1) ^ (row & 3)) + (p & 1))
// for p = l mod (PB / 16).
template <int PB>
__device__ __forceinline__ void tr_dma_coords(int q, int lane, int& row, int& col) {
  constexpr int kLanesPerRow = PB / 16;
  row = (64 / kLanesPerRow) * q + lane / kLanesPerRow;
  const int p = lane % kLanesPerRow;
  col = 8 * (2 * ((p >> 1) ^ (row & 3)) + (p & 1));
}

// ---------------------------------------------------------------------------
// Row contraction: out[m][j] = sum_c P[m][c] Q(c, j), 128 rows m per
// workgroup (wave w: rows 32 w .. +31, the MFMA B operand), all RP ranks j
// (the A operand), stages of 32 c.  P rows are DMA'd as 64-byte rows
// (16-byte chunk c of row m at c ^ ((m >> 2) & 3)).  Q is A [r x C] (QT =
// false: rows j, read like P) or B [C x r] (QT = true: rows c, read
// transposed).  Output D[j][m]: a lane holds four consecutive j of one m.
// ---------------------------------------------------------------------------
template <int RP, bool QT>
struct RowShape {
  static constexpr int kP = 128 * 64;                      // 8 KiB of P per stage
  static constexpr int kQ = RP * 64;                       // Q per stage (RP rows x 64 B, or 32 rows x 2 RP B)
  static constexpr int kStage = kP + kQ;
  static constexpr int kQDma = kQ / 1024 / 4;              // Q DMA instructions per wave per stage
  static constexpr int kLoads = 2 + kQDma;                 // all DMA instructions per wave per stage
};

template <int RP, bool QT>
__global__ __launch_bounds__(kThreads, 1) void rskinny_kernel(const bf16_t* __restrict__ P, int64_t M, int64_t C,
                                                              int64_t ldp, int64_t p_gs,
                                                              const bf16_t* __restrict__ Q, int r, int64_t q_gs,
                                                              int stages_per_split, int tiles_m, int ldo,
                                                              float* __restrict__ part) {
  using S = RowShape<RP, QT>;
  extern __shared__ __align__(16) char smem[];
  const int tm = blockIdx.x % tiles_m, sp = blockIdx.x / tiles_m, g = blockIdx.y;
  const int t = threadIdx.x, w = t >> 6, lane = t & 63, lr = lane & 31, h = lane >> 5;
  const int64_t m0 = (int64_t)tm * 128;
  const int nst = (int)((C + 31) / 32);
  const int s0 = sp * stages_per_split, s1 = min(nst, s0 + stages_per_split);
  P += g * p_gs;
  Q += g * q_gs;
  // P rows of this tile only (rows past M read as zero); Q whole
  const rsrc_t pr = make_rsrc(P + m0 * ldp, (uint32_t)(((min((int64_t)128, M - m0) - 1) * ldp + C) * 2));
  const rsrc_t qr = make_rsrc(Q, (uint32_t)((int64_t)r * C * 2));
  uint32_t po[2], qo[S::kQDma > 0 ? S::kQDma : 1];
  int pl[2], ql[S::kQDma > 0 ? S::kQDma : 1];
#pragma unroll
  for (int q = 0; q < 2; ++q) {   // P: instruction q of wave w fills rows 16 (2w + q) .. +15
    const int row = 16 * (2 * w + q) + (lane >> 2), ch = (lane & 3) ^ ((lane >> 4) & 3);
    po[q] = (uint32_t)(row * ldp * 2 + ch * 16);
    pl[q] = 16 * (2 * w + q) * 64;
  }
#pragma unroll
  for (int q = 0; q < S::kQDma; ++q) {
    const int gi = S::kQDma * w + q;   // 1 KiB piece of the stage's Q tile
    if constexpr (!QT) {               // rows j of A, 64 bytes per stage
      const int row = 16 * gi + (lane >> 2), ch = (lane & 3) ^ ((lane >> 4) & 3);
      qo[q] = (uint32_t)(row * C * 2 + ch * 16);
    } else {                           // rows c of B, 2 RP bytes, transposed layout
      int row, col;
      tr_dma_coords<2 * RP>(gi, lane, row, col);
      qo[q] = (uint32_t)(row * r * 2 + col * 2);
    }
    ql[q] = S::kP + gi * 1024;
  }
  auto dma = [&](int st, int slot) {
    const int ss = min(st, s1 - 1);    // past the split: re-load its last stage (never read)
    char* base = smem + slot * S::kStage;
#pragma unroll
    for (int q = 0; q < 2; ++q) dma16(pr, base + pl[q], po[q], (uint32_t)ss * 64u);
#pragma unroll
    for (int q = 0; q < S::kQDma; ++q)
      dma16(qr, base + ql[q], qo[q], QT ? (uint32_t)ss * 32u * (uint32_t)r * 2u : (uint32_t)ss * 64u);
  };

  constexpr int FJ = RP / 32;
  static_assert(!QT || FJ == 2 || FJ == 4, "transposed rank side: RP 64 or 128");
  f32x16_t acc[FJ];
#pragma unroll
  for (int f = 0; f < FJ; ++f)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[f][e] = 0.0f;

  if (s0 < s1) {
#pragma unroll
    for (int a = 0; a < kAhead; ++a) dma(s0 + a, a);
    int slot = 0;
    for (int st = s0; st < s1; ++st) {
      // stage st was issued kAhead - 1 stages before the last kAhead - 1 issues
      QLORA_WAIT((kAhead - 1) * S::kLoads, 0);
      __builtin_amdgcn_s_barrier();
      dma(st + kAhead, slot == 0 ? kRing - 1 : slot - 1);   // the slot stage st - 1 used
      const char* base = smem + slot * S::kStage;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        // P fragment (B operand): row 32 w + lr, the 8 columns that lane half h
        // takes in k16 step kk.  Both operands must agree on that: a 64-byte
        // row read takes chunk 2h + kk (columns 16 h + 8 kk ..), a transposed
        // read of 32 Q rows takes rows 16 kk + 8 h .. (chunk 2 kk + h)
        const int ch = QT ? 2 * kk + h : 2 * h + kk;
        bf16x8_t b = rd16(base + spos(32 * w + lr, ch));
        if (32 * st + 8 * ch >= C) b = bf16x8_t{};   // columns past C (C % 8 == 0)
        bf16x8_t a[FJ];
        if constexpr (!QT) {
#pragma unroll
          for (int f = 0; f < FJ; ++f) a[f] = rd16(base + S::kP + spos(32 * f + lr, 2 * h + kk));
        } else {
          // transposed reads in asm blocks (see tr_read2): FJ is 2 or 4
          constexpr int O = 4 * 2 * RP;
          const char* qb = base + S::kP + kk * 16 * 2 * RP;
#pragma unroll
          for (int f = 0; f < FJ; f += 2) tr_read2<O, O>(qb + tr_off<2 * RP>(f), qb + tr_off<2 * RP>(f + 1), a[f], a[f + 1]);
        }
#pragma unroll
        for (int f = 0; f < FJ; ++f) acc[f] = mfma32x32x16(a[f], b, acc[f]);
      }
      slot = slot == kRing - 1 ? 0 : slot + 1;
    }
    QLORA_WAIT(0, 0);
  }
  // D[j][m]: lane (lr, h) holds m = m0 + 32 w + lr, j = 32 f + 8 q + 4 h + 0..3,
  // stored at column g r + j of the split's [M x ldo] partial
  float* out = part + (int64_t)sp * M * ldo + (int64_t)g * r;
  const int64_t m = m0 + 32 * w + lr;
  if (m < M) {
#pragma unroll
    for (int f = 0; f < FJ; ++f)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = 32 * f + 8 * q + 4 * h;
        if (j < r)
          *reinterpret_cast<float4*>(out + m * ldo + j) =
              make_float4(acc[f][4 * q], acc[f][4 * q + 1], acc[f][4 * q + 2], acc[f][4 * q + 3]);
      }
  }
}

// ---------------------------------------------------------------------------
// Token contraction: D = sum_m Big[m][c] Sm[m][j] for 128 columns c per
// workgroup (wave w: columns 32 w .. +31) and all RP ranks j, stages of 32
// tokens.  Both tiles are rows m, read transposed.  DB = false stores dA
// [r x C] (A operand = Big, D[c][j]: four consecutive c per lane); DB = true
// stores dB [C x r] (A operand = Sm, D[j][c]: four consecutive j per lane).
// ---------------------------------------------------------------------------
template <int RP>
struct ColShape {
  static constexpr int kBig = 32 * 256;                    // 8 KiB: 32 rows x 128 columns
  static constexpr int kSm = 32 * 2 * RP;                  // 32 rows x RP ranks
  static constexpr int kStage = kBig + kSm;
  static constexpr int kSmDma = kSm / 1024 / 4;
  static constexpr int kLoads = 2 + kSmDma;
};

template <int RP, bool DB>
__global__ __launch_bounds__(kThreads, 1) void cskinny_kernel(const bf16_t* __restrict__ Big, int64_t M, int64_t C,
                                                              int64_t ldb, int64_t big_gs,
                                                              const bf16_t* __restrict__ Sm, int r, int lds,
                                                              int64_t sm_gs, int stages_per_split, int tiles_c,
                                                              float* __restrict__ part) {
  using S = ColShape<RP>;
  extern __shared__ __align__(16) char smem[];
  const int tc = blockIdx.x % tiles_c, sp = blockIdx.x / tiles_c, g = blockIdx.y;
  const int t = threadIdx.x, w = t >> 6, lane = t & 63, lr = lane & 31, h = lane >> 5;
  const int64_t c0 = (int64_t)tc * 128;
  const int nst = (int)((M + 31) / 32);
  const int s0 = sp * stages_per_split, s1 = min(nst, s0 + stages_per_split);
  Big += g * big_gs;
  Sm += g * sm_gs;
  // rows past M read as zero
  const rsrc_t br = make_rsrc(Big, (uint32_t)(((M - 1) * ldb + C) * 2));
  const rsrc_t sr = make_rsrc(Sm, (uint32_t)(((M - 1) * lds + r) * 2));
  uint32_t bo[2], so[S::kSmDma];
  int bl[2], sl[S::kSmDma];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    int row, col;
    tr_dma_coords<256>(2 * w + q, lane, row, col);
    bo[q] = (uint32_t)(row * ldb * 2 + (c0 + col) * 2);   // columns past C: never stored
    bl[q] = (2 * w + q) * 1024;
  }
#pragma unroll
  for (int q = 0; q < S::kSmDma; ++q) {
    int row, col;
    tr_dma_coords<2 * RP>(S::kSmDma * w + q, lane, row, col);
    so[q] = (uint32_t)(row * lds * 2 + col * 2);   // ranks past r: never stored
    sl[q] = S::kBig + (S::kSmDma * w + q) * 1024;
  }
  auto dma = [&](int st, int slot) {
    const uint32_t ss = (uint32_t)min(st, s1 - 1);
    char* base = smem + slot * S::kStage;
#pragma unroll
    for (int q = 0; q < 2; ++q) dma16(br, base + bl[q], bo[q], ss * 32u * (uint32_t)ldb * 2u);
#pragma unroll
    for (int q = 0; q < S::kSmDma; ++q) dma16(sr, base + sl[q], so[q], ss * 32u * (uint32_t)lds * 2u);
  };

  constexpr int FJ = RP / 32;
  static_assert(FJ == 2 || FJ == 4 || FJ == 8, "RP 64, 128 or 256");
  f32x16_t acc[FJ];
#pragma unroll
  for (int f = 0; f < FJ; ++f)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[f][e] = 0.0f;
  const int bo_frag = tr_off<256>(w);

  if (s0 < s1) {
#pragma unroll
    for (int a = 0; a < kAhead; ++a) dma(s0 + a, a);
    int slot = 0;
    for (int st = s0; st < s1; ++st) {
      QLORA_WAIT((kAhead - 1) * S::kLoads, 0);
      __builtin_amdgcn_s_barrier();
      dma(st + kAhead, slot == 0 ? kRing - 1 : slot - 1);
      const char* base = smem + slot * S::kStage;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        // transposed reads in asm blocks (see tr_read3): the big tile's
        // fragment and the first two rank fragments, then three at a time
        constexpr int O = 4 * 2 * RP;
        const char* sb = base + S::kBig + kk * 16 * 2 * RP;
        bf16x8_t bg, sm[FJ];
        tr_read3<4 * 256, O, O>(base + kk * 16 * 256 + bo_frag, sb + tr_off<2 * RP>(0), sb + tr_off<2 * RP>(1), bg,
                                sm[0], sm[1]);
        if constexpr (FJ == 4) tr_read2<O, O>(sb + tr_off<2 * RP>(2), sb + tr_off<2 * RP>(3), sm[2], sm[3]);
        if constexpr (FJ == 8) {
#pragma unroll
          for (int f = 2; f < 8; f += 3)
            tr_read3<O, O, O>(sb + tr_off<2 * RP>(f), sb + tr_off<2 * RP>(f + 1), sb + tr_off<2 * RP>(f + 2), sm[f],
                              sm[f + 1], sm[f + 2]);
        }
#pragma unroll
        for (int f = 0; f < FJ; ++f)
          acc[f] = DB ? mfma32x32x16(sm[f], bg, acc[f]) : mfma32x32x16(bg, sm[f], acc[f]);
      }
      slot = slot == kRing - 1 ? 0 : slot + 1;
    }
    QLORA_WAIT(0, 0);
  }
  // the split's partial holds all groups' outputs, group g at g C r
  float* out = part + ((int64_t)sp * gridDim.y + g) * C * r;
#pragma unroll
  for (int f = 0; f < FJ; ++f)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (!DB) {   // D[c][j]: c = c0 + 32 w + 8 q + 4 h + 0..3, j = 32 f + lr -> dA[j][c..]
        const int j = 32 * f + lr;
        const int64_t c = c0 + 32 * w + 8 * q + 4 * h;
        if (j < r && c < C)
          *reinterpret_cast<float4*>(out + j * C + c) =
              make_float4(acc[f][4 * q], acc[f][4 * q + 1], acc[f][4 * q + 2], acc[f][4 * q + 3]);
      } else {               // D[j][c]: j = 32 f + 8 q + 4 h + 0..3, c = c0 + 32 w + lr -> dB[c][j..]
        const int j = 32 * f + 8 * q + 4 * h;
        const int64_t c = c0 + 32 * w + lr;
        if (j < r && c < C)
          *reinterpret_cast<float4*>(out + c * r + j) =
              make_float4(acc[f][4 * q], acc[f][4 * q + 1], acc[f][4 * q + 2], acc[f][4 * q + 3]);
      }
    }
}

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

// The reductions of dA and dB in one launch: elements [0, n0) of the
// output are out0 (partials at part0, splits0 of them), the next n1 are out1
// (part1, splits1); each sums its splits in order, as reduce_kernel does.
__global__ __launch_bounds__(kThreads) void reduce2_kernel(const float* __restrict__ part0, int splits0, int64_t n0,
                                                           float* __restrict__ out0,
                                                           const float* __restrict__ part1, int splits1, int64_t n1,
                                                           float* __restrict__ out1, float scale) {
  int64_t i = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 4;
  const float* part = part0;
  float* out = out0;
  int splits = splits0;
  int64_t n = n0;
  if (i >= n0) {
    i -= n0;
    part = part1, out = out1, splits = splits1, n = n1;
  }
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
  *reinterpret_cast<float4*>(out + i) = acc;
}

// Splits of the contraction (stages of 32) for about `target` workgroups,
// at least 32 stages each: shorter splits spend most of their time filling
// the ring and add partials (the 7B and 13B steps ran 1.1-1.4 % faster than
// with 8).  The target (256, one per CU of the part this is
// tuned for) was measured; it is fixed, not the device's CU count, because
// the workspace size a caller queries must not depend on which device is
// current.  It does not depend on the number of groups a launch covers
// either, so that a group call sums in the order of the per-linear calls.
struct Split {
  int tiles, sps, splits;
};
Split split_for(int64_t tiles, int64_t contraction, int target) {
  const int nst = (int)((contraction + 31) / 32);
  int want = (int)((target + tiles - 1) / tiles);
  want = std::max(1, std::min(want, std::max(1, nst / 32)));
  Split s;
  s.tiles = (int)tiles;
  s.sps = (nst + want - 1) / want;
  s.splits = (nst + s.sps - 1) / s.sps;
  return s;
}

Split kind_split(int64_t rows, int64_t cols, int64_t contraction, int kind) {
  // rows x cols is the output: kXAt, kDyB [M x r]; kGtX [r x K]; kDytU [N x r]
  const int64_t tiles = (kind == kGtX) ? (cols + 127) / 128 : (rows + 127) / 128;
  return split_for(tiles, contraction, 256);
}

hipError_t reduce(const float* part, int splits, int64_t n, float scale, float* out_f32, bf16_t* out_bf16,
                  bf16_t* out_bf16_2, hipStream_t st) {
  hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)((n / 4 + kThreads - 1) / kThreads)), dim3(kThreads), 0, st,
                     part, splits, n, scale, out_f32, out_bf16, out_bf16_2);
  return hipGetLastError();
}

// Row contraction over G groups (grid y): group g reads P + g p_gs (rows of
// stride ldp, C columns) and Q + g q_gs, and writes columns g r .. of the
// [M x ldo] result.
struct RowArgs {
  const bf16_t* P;
  int64_t M, C, ldp, p_gs;
  const bf16_t* Q;
  int r;
  int64_t q_gs;
  int G, ldo;
};

template <int RP, bool QT>
hipError_t run_rows(const RowArgs& a, float* part, float scale, bf16_t* out, bf16_t* out2, hipStream_t st) {
  const Split sp = split_for((a.M + 127) / 128, a.C, 256);
  auto* fn = &rskinny_kernel<RP, QT>;
  const size_t lds = (size_t)kRing * RowShape<RP, QT>::kStage;
  hipError_t e = allow_lds(reinterpret_cast<const void*>(fn), (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3(sp.tiles * sp.splits, a.G), dim3(kThreads), lds, st, a.P, a.M, a.C, a.ldp, a.p_gs, a.Q,
                     a.r, a.q_gs, sp.sps, sp.tiles, a.ldo, part);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return reduce(part, sp.splits, a.M * a.ldo, scale, nullptr, out, out2, st);
}

// Token contraction over G groups (grid y): group g reads Big + g big_gs
// (rows of stride ldb, C columns) and Sm + g sm_gs (rows of stride lds, r
// ranks), and writes the g-th C x r block of the result.
struct ColArgs {
  const bf16_t* Big;
  int64_t M, C, ldb, big_gs;
  const bf16_t* Sm;
  int r, lds;
  int64_t sm_gs;
  int G;
};

// The token-contraction product's partials (no reduction); *splits gets
// their count.
template <int RP, bool DB>
hipError_t run_cols(const ColArgs& a, float* part, int* splits, hipStream_t st) {
  const Split sp = split_for((a.C + 127) / 128, a.M, 256);
  auto* fn = &cskinny_kernel<RP, DB>;
  const size_t lds = (size_t)kRing * ColShape<RP>::kStage;
  hipError_t e = allow_lds(reinterpret_cast<const void*>(fn), (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3(sp.tiles * sp.splits, a.G), dim3(kThreads), lds, st, a.Big, a.M, a.C, a.ldb,
                     a.big_gs, a.Sm, a.r, a.lds, a.sm_gs, sp.sps, sp.tiles, part);
  *splits = sp.splits;
  return hipGetLastError();
}

}  // namespace

size_t skinny_partial_bytes(int64_t rows, int64_t cols, int64_t contraction, int kind) {
  const Split sp = kind_split(rows, cols, contraction, kind);
  return (size_t)sp.splits * (size_t)rows * (size_t)cols * sizeof(float);
}

hipError_t launch_xat(const bf16_t* X, const bf16_t* A, int64_t M, int64_t K, int r, float* part, bf16_t* out,
                      bf16_t* out2, float scale, hipStream_t st) {
  const RowArgs a{X, M, K, K, 0, A, r, 0, 1, r};
  if (r <= 64) return run_rows<64, false>(a, part, scale, out, out2, st);
  if (r <= 128) return run_rows<128, false>(a, part, scale, out, out2, st);
  if (r <= 192) return run_rows<192, false>(a, part, scale, out, out2, st);
  return run_rows<256, false>(a, part, scale, out, out2, st);
}

hipError_t launch_dyb_group(const bf16_t* dY, int64_t ldy, const bf16_t* B, int64_t M, int64_t N, int r, int G,
                            float* part, bf16_t* out, float scale, hipStream_t st) {
  const RowArgs a{dY, M, N, ldy, N, B, r, N * r, G, G * r};
  if (r <= 64) return run_rows<64, true>(a, part, scale, out, nullptr, st);
  return run_rows<128, true>(a, part, scale, out, nullptr, st);
}

hipError_t launch_dyb(const bf16_t* dY, const bf16_t* B, int64_t M, int64_t N, int r, float* part, bf16_t* out,
                      float scale, hipStream_t st) {
  return launch_dyb_group(dY, N, B, M, N, r, 1, part, out, scale, st);
}

size_t grads_partial_bytes(int64_t M, int64_t N, int64_t K, int r, int G) {
  const size_t a = skinny_partial_bytes(G * r, K, M, kGtX);
  return (a + 255) / 256 * 256 + (size_t)G * skinny_partial_bytes(N, r, M, kDytU);
}

hipError_t launch_grads(const bf16_t* Gm, const bf16_t* X, const bf16_t* dY, int64_t ldy, const bf16_t* U, int ldu,
                        int64_t M, int64_t N, int64_t K, int r, int G, float* part, float* dA, float* dB, float scale,
                        hipStream_t st) {
  // dA [G r x K] = s G^T X in one pass over X (the stacked rank as one)
  const int ra = G * r;
  const ColArgs a{X, M, K, K, 0, Gm, ra, ra, 0, 1};
  int sa = 0, sb = 0;
  hipError_t e = ra <= 64    ? run_cols<64, false>(a, part, &sa, st)
                 : ra <= 128 ? run_cols<128, false>(a, part, &sa, st)
                             : run_cols<256, false>(a, part, &sa, st);
  if (e != hipSuccess) return e;
  // dB_g [N x r] = s dY_g^T U_g for every group, partials after dA's
  float* part_b = part + (skinny_partial_bytes(ra, K, M, kGtX) + 255) / 256 * 256 / sizeof(float);
  const ColArgs b{dY, M, N, ldy, N, U, r, ldu, r, G};
  e = r <= 64 ? run_cols<64, true>(b, part_b, &sb, st) : run_cols<128, true>(b, part_b, &sb, st);
  if (e != hipSuccess) return e;
  const int64_t na = (int64_t)ra * K, nb = (int64_t)G * N * r;
  hipLaunchKernelGGL(reduce2_kernel, dim3((unsigned)(((na + nb) / 4 + kThreads - 1) / kThreads)), dim3(kThreads), 0, st,
                     part, sa, na, dA, part_b, sb, nb, dB, scale);
  return hipGetLastError();
}

}  // namespace qlora
