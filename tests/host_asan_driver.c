/* Host-side AddressSanitizer driver of the C ABI's argument checks.
 *
 * Linked against a build of libqlora whose host code (capi.hip, qtensor.cpp)
 * is instrumented with -fsanitize=address.  Every call below is one the
 * library must refuse during validation, before any HIP call, so the driver
 * runs without a GPU and launches nothing; device pointers are fake, aligned
 * or not, and are never dereferenced.  Host arrays the library reads (job
 * tables, descriptors, header bytes) are heap blocks of exactly the size
 * passed, so any read past them is reported by the sanitizer.  Exits 0 and
 * prints "host asan driver OK" when every status is the expected one.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "qlora.h"

static int failures = 0;

#define EXPECT(call, want)                                                            \
  do {                                                                                \
    int got_ = (int)(call);                                                           \
    if (got_ != (int)(want)) {                                                        \
      fprintf(stderr, "line %d: %s -> %d, expected %d\n", __LINE__, #call, got_, (int)(want)); \
      ++failures;                                                                     \
    }                                                                                 \
  } while (0)

static void* fake(uintptr_t a) { return (void*)a; }

static qlora_nf4_weight weight(int64_t rows, int64_t cols) {
  qlora_nf4_weight w;
  memset(&w, 0, sizeof(w));
  w.rows = rows;
  w.cols = cols;
  w.blocksize = 64;
  w.group_blocks = 256;
  w.codes = (uint8_t*)fake(0x10000);
  w.absmax_q = (uint8_t*)fake(0x20000);
  w.group_scale = (float*)fake(0x30000);
  w.codebook = QLORA_CODEBOOK_NF4;
  w.absmax_format = QLORA_ABSMAX_LINEAR8;
  return w;
}

static uint64_t lcg(uint64_t* s) {
  *s = *s * 6364136223846793005ULL + 1442695040888963407ULL;
  return *s >> 33;
}

int main(void) {
  /* status strings for every code and an unknown one */
  for (int s = 0; s <= 9; ++s)
    if (!qlora_status_str((qlora_status)s)) ++failures;

  /* size arithmetic */
  size_t c, a, sc;
  EXPECT(qlora_sizes(0, 64, 64, 256, &c, &a, &sc), QLORA_E_SHAPE);
  EXPECT(qlora_sizes(64, 64, 32, 256, &c, &a, &sc), QLORA_E_UNSUPPORTED);
  EXPECT(qlora_sizes((int64_t)1 << 39, (int64_t)1 << 39, 64, 256, &c, &a, &sc), QLORA_E_SHAPE);
  EXPECT(qlora_sizes(3, 1000, 64, 256, NULL, NULL, NULL), QLORA_OK);
  if (qlora_workspace_bytes(QLORA_OP_FWD, -1, 64, 64, 8, 0) != 0) ++failures;
  if (qlora_workspace_bytes((qlora_op)99, 64, 64, 64, 8, 0) != 0) ++failures;

  float lv[16];
  EXPECT(qlora_codebook_levels((qlora_codebook)7, lv), QLORA_E_UNSUPPORTED);
  EXPECT(qlora_codebook_levels(QLORA_CODEBOOK_NF4, NULL), QLORA_E_NULL);

  /* quantize / dequant descriptors */
  qlora_nf4_weight* w = (qlora_nf4_weight*)malloc(sizeof(qlora_nf4_weight));
  *w = weight(64, 128);
  EXPECT(qlora_quantize(NULL, w, NULL), QLORA_E_NULL);
  EXPECT(qlora_quantize((const uint16_t*)fake(0x1000), NULL, NULL), QLORA_E_NULL);
  w->blocksize = 128;
  EXPECT(qlora_dequant(w, (uint16_t*)fake(0x1000), NULL), QLORA_E_UNSUPPORTED);
  *w = weight(64, 128);
  w->codebook = 5;
  EXPECT(qlora_dequant(w, (uint16_t*)fake(0x1000), NULL), QLORA_E_UNSUPPORTED);
  *w = weight(64, 128);
  w->codes = (uint8_t*)fake(0x10008);
  EXPECT(qlora_dequant(w, (uint16_t*)fake(0x1000), NULL), QLORA_E_ALIGN);
  *w = weight(64, 100);
  EXPECT(qlora_dequant_t(w, (uint16_t*)fake(0x1000), NULL), QLORA_E_UNSUPPORTED);

  /* forward / backward */
  const uint16_t* X = (const uint16_t*)fake(0x100000);
  uint16_t* Y = (uint16_t*)fake(0x200000);
  const uint16_t* Aa = (const uint16_t*)fake(0x300000);
  const uint16_t* Bb = (const uint16_t*)fake(0x400000);
  *w = weight(64, 128);
  EXPECT(qlora_linear_fwd(w, X, 0, Aa, Bb, 8, 16.f, Y, NULL, NULL, 0, NULL), QLORA_E_SHAPE);
  EXPECT(qlora_linear_fwd(w, X, 16, Aa, Bb, 7, 16.f, Y, NULL, NULL, 0, NULL), QLORA_E_UNSUPPORTED);
  EXPECT(qlora_linear_fwd(w, X, 16, Aa, Bb, 256, 16.f, Y, NULL, NULL, 0, NULL), QLORA_E_UNSUPPORTED);
  EXPECT(qlora_linear_fwd(w, X, 16, NULL, Bb, 8, 16.f, Y, NULL, NULL, 0, NULL), QLORA_E_NULL);
  EXPECT(qlora_linear_fwd(w, (const uint16_t*)fake(0x100002), 16, Aa, Bb, 8, 16.f, Y, NULL, NULL, 0, NULL),
         QLORA_E_ALIGN);
  EXPECT(qlora_linear_fwd(w, X, 16, Aa, Bb, 8, 16.f, Y, NULL, NULL, 0, NULL), QLORA_E_WORKSPACE);
  EXPECT(qlora_linear_fwd(w, X, (int64_t)1 << 32, Aa, Bb, 8, 16.f, Y, NULL, NULL, 0, NULL), QLORA_E_SHAPE);
  *w = weight(64, 100);
  EXPECT(qlora_linear_fwd(w, X, 16, Aa, Bb, 8, 16.f, Y, NULL, NULL, 0, NULL), QLORA_E_UNSUPPORTED);
  *w = weight(64, (int64_t)1 << 24);
  EXPECT(qlora_linear_fwd(w, X, 1, Aa, Bb, 8, 16.f, Y, NULL, NULL, 0, NULL), QLORA_E_UNSUPPORTED);
  *w = weight(64, 128);
  EXPECT(qlora_linear_fwd_noalloc(w, X, 16, Aa, Bb, 7, 16.f, Y, NULL, NULL), QLORA_E_UNSUPPORTED);
  float* dA = (float*)fake(0x500000);
  float* dB = (float*)fake(0x600000);
  EXPECT(qlora_linear_bwd(w, X, NULL, 16, Aa, Bb, 8, 16.f, NULL, Y, dA, dB, NULL, 0, NULL), QLORA_E_NULL);
  EXPECT(qlora_linear_bwd(w, X, X, 16, NULL, NULL, 0, 16.f, NULL, Y, dA, dB, NULL, 0, NULL), QLORA_E_SHAPE);
  EXPECT(qlora_linear_bwd(w, X, X, 16, Aa, Bb, 8, 16.f, NULL, Y, NULL, dB, NULL, 0, NULL), QLORA_E_NULL);
  EXPECT(qlora_linear_bwd(w, X, X, 16, Aa, Bb, 8, 16.f, NULL, Y, dA, dB, NULL, 0, NULL), QLORA_E_WORKSPACE);

  /* groups: a descriptor array of exactly G entries, one of them bad */
  qlora_nf4_weight* g3 = (qlora_nf4_weight*)malloc(3 * sizeof(qlora_nf4_weight));
  g3[0] = weight(64, 128);
  g3[1] = weight(64, 128);
  g3[2] = weight(64, 256);
  EXPECT(qlora_group_fwd(g3, 3, X, 16, Aa, Bb, 8, 16.f, Y, NULL, NULL, 0, NULL), QLORA_E_SHAPE);
  EXPECT(qlora_group_fwd(g3, 0, X, 16, Aa, Bb, 8, 16.f, Y, NULL, NULL, 0, NULL), QLORA_E_SHAPE);
  g3[2] = weight(64, 128);
  g3[2].group_blocks = 128;
  EXPECT(qlora_group_dequant(g3, 3, Y, NULL), QLORA_E_UNSUPPORTED);

  /* LoRA side products: 32-bit byte ranges */
  EXPECT(qlora_lora_down(X, Aa, 1, (int64_t)1 << 24, 8, Y, NULL, 0, NULL), QLORA_E_UNSUPPORTED);
  EXPECT(qlora_lora_dy_b(X, Bb, 1, (int64_t)1 << 24, 8, Y, NULL, 0, NULL), QLORA_E_UNSUPPORTED);

  /* decode jobs: a table of exactly njobs entries */
  qlora_gemv_job* jobs = (qlora_gemv_job*)malloc(2 * sizeof(qlora_gemv_job));
  *w = weight(64, 128);
  for (int i = 0; i < 2; ++i) {
    memset(&jobs[i], 0, sizeof(jobs[i]));
    jobs[i].W = w;
    jobs[i].x = X;
    jobs[i].y = Y;
    jobs[i].m = 1;
  }
  jobs[1].m = 17;
  EXPECT(qlora_gemv(jobs, 2, fake(0x700000), 1 << 20, NULL), QLORA_E_UNSUPPORTED);
  jobs[1].m = -1;
  EXPECT(qlora_gemv(jobs, 2, fake(0x700000), 1 << 20, NULL), QLORA_E_SHAPE);
  jobs[1].m = 1;
  jobs[1].r = 8;
  EXPECT(qlora_gemv(jobs, 2, fake(0x700000), 1 << 20, NULL), QLORA_E_NULL);
  jobs[1].r = 0;
  EXPECT(qlora_gemv(jobs, 2, NULL, 1 << 20, NULL), QLORA_E_NULL);
  EXPECT(qlora_gemv(jobs, 0, fake(0x700000), 1 << 20, NULL), QLORA_E_SHAPE);
  qlora_gemv_plan* plan = (qlora_gemv_plan*)calloc(1, sizeof(qlora_gemv_plan));
  EXPECT(qlora_gemv_prepare(jobs, 2, fake(0x700000), 16, plan, NULL), QLORA_E_WORKSPACE);
  EXPECT(qlora_gemv_run(plan, NULL), QLORA_E_SHAPE);

  /* optimizer */
  float* p = (float*)fake(0x800000);
  EXPECT(qlora_adamw(p, NULL, p, p, p, 0, 1e-3f, 0.9f, 0.999f, 1e-8f, 0.f, 1, NULL), QLORA_E_SHAPE);
  EXPECT(qlora_adamw(p, NULL, p, p, p, 64, 1e-3f, 1.0f, 0.999f, 1e-8f, 0.f, 1, NULL), QLORA_E_SHAPE);
  qlora_paged_tensor* pt = (qlora_paged_tensor*)calloc(2, sizeof(qlora_paged_tensor));
  for (int i = 0; i < 2; ++i) {
    pt[i].p = p;
    pt[i].grad = p;
    pt[i].m = p;
    pt[i].v = p;
    pt[i].n = 1 << 20;
  }
  qlora_paged_layout lay;
  EXPECT(qlora_paged_layout_of(pt, 2, 1024, &lay), QLORA_E_WORKSPACE);
  EXPECT(qlora_paged_layout_of(pt, 2, (size_t)1 << 30, &lay), QLORA_OK);
  if (lay.resident != 2 || lay.chunk != 0) ++failures;

  /* serialized-weight headers: exact-size heap buffers, valid and mutated */
  uint64_t id = 0;
  EXPECT(qlora_level_table_id(QLORA_CODEBOOK_NF4, QLORA_ABSMAX_LINEAR8, NULL), QLORA_E_NULL);
  EXPECT(qlora_level_table_id(QLORA_CODEBOOK_NF4, 3, &id), QLORA_E_UNSUPPORTED);
  EXPECT(qlora_level_table_id(QLORA_CODEBOOK_INT4, QLORA_ABSMAX_FP8, &id), QLORA_OK);
  uint8_t* hdr = (uint8_t*)malloc(QLORA_QTENSOR_HEADER_BYTES);
  uint8_t* small = (uint8_t*)malloc(QLORA_QTENSOR_HEADER_BYTES - 1);
  *w = weight(3, 1000);
  EXPECT(qlora_qtensor_header_write(w, small, QLORA_QTENSOR_HEADER_BYTES - 1), QLORA_E_FORMAT);
  EXPECT(qlora_qtensor_header_write(w, hdr, QLORA_QTENSOR_HEADER_BYTES), QLORA_OK);
  qlora_nf4_weight* back = (qlora_nf4_weight*)malloc(sizeof(qlora_nf4_weight));
  memset(back, 0, sizeof(*back));
  uint64_t payload = 0;
  EXPECT(qlora_qtensor_header_read(hdr, QLORA_QTENSOR_HEADER_BYTES, back, &payload), QLORA_OK);
  if (back->rows != 3 || back->cols != 1000 || payload != 1500 + 47 + 4) {
    fprintf(stderr, "header read back: %lld x %lld, payload %llu\n", (long long)back->rows, (long long)back->cols, (unsigned long long)payload);
    ++failures;
  }
  memcpy(small, hdr, QLORA_QTENSOR_HEADER_BYTES - 1);
  EXPECT(qlora_qtensor_header_read(small, QLORA_QTENSOR_HEADER_BYTES - 1, back, &payload), QLORA_E_FORMAT);
  uint8_t* mut = (uint8_t*)malloc(QLORA_QTENSOR_HEADER_BYTES);
  uint64_t seed = 12345;
  int accepted = 0;
  for (int t = 0; t < 20000; ++t) {
    memcpy(mut, hdr, QLORA_QTENSOR_HEADER_BYTES);
    if (t % 2) {
      for (int b = 0; b < QLORA_QTENSOR_HEADER_BYTES; ++b) mut[b] = (uint8_t)lcg(&seed);
    } else {
      const int flips = 1 + (int)(lcg(&seed) % 3);
      for (int f = 0; f < flips; ++f) mut[lcg(&seed) % QLORA_QTENSOR_HEADER_BYTES] ^= (uint8_t)(1 + lcg(&seed) % 255);
    }
    if (qlora_qtensor_header_read(mut, QLORA_QTENSOR_HEADER_BYTES, back, &payload) == QLORA_OK) ++accepted;
  }
  /* a mutated header is accepted only when the flips landed in nothing the
     reader checks; random bytes never are */
  if (accepted > 200) {
    fprintf(stderr, "%d mutated headers accepted\n", accepted);
    ++failures;
  }

  free(mut);
  free(back);
  free(small);
  free(hdr);
  free(pt);
  free(plan);
  free(jobs);
  free(g3);
  free(w);
  if (failures) {
    fprintf(stderr, "host asan driver: %d failure(s)\n", failures);
    return 1;
  }
  printf("host asan driver OK\n");
  return 0;
}
