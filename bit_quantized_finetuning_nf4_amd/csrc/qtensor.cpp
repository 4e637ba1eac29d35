// qtensor.cpp -- host-only header of a serialized quantized weight
// (declared in include/qlora.h, "Serialized quantized weights").
//
// The pages keep the trained adapters apart from the frozen 4-bit model and
// tie them to it (deepfa.ir blog, "LoRA: Prerequisite"), so a stored weight
// must be decoded with exactly the level tables it was encoded with.  The
// header records a digest of those tables; reading a header whose digest
// differs from the library's own is refused.
//
// Everything here is plain C++ on host memory: no HIP call, no device
// pointer is dereferenced.
#include <cstdint>
#include <cstring>

#include "../../include/qlora.h"

namespace {

constexpr char kMagic[8] = {'Q', 'L', 'O', 'R', 'A', 'Q', 'T', '1'};
constexpr uint32_t kVersion = 1;

struct Fnv1a {
  uint64_t h = 0xcbf29ce484222325ULL;
  void bytes(const void* p, size_t n) {
    const unsigned char* b = static_cast<const unsigned char*>(p);
    for (size_t i = 0; i < n; ++i) {
      h ^= b[i];
      h *= 0x100000001b3ULL;
    }
  }
  void u32(uint32_t v) {
    unsigned char b[4];
    for (int i = 0; i < 4; ++i) b[i] = (unsigned char)(v >> (8 * i));
    bytes(b, 4);
  }
  void f32(float f) {
    uint32_t v;
    std::memcpy(&v, &f, 4);
    u32(v);
  }
};

// Value of the FP8 E4M3 bit pattern k (k < 128: sign 0): four exponent bits
// with bias 7, three mantissa bits, a zero exponent field is subnormal.
double e4m3_value(int k) {
  const int e = k >> 3, m = k & 7;
  if (e == 0) return m / 512.0;                        // m / 8 * 2^(1 - 7)
  double v = 1.0 + m / 8.0;
  for (int i = 7; i < e; ++i) v *= 2.0;
  for (int i = e; i < 7; ++i) v *= 0.5;
  return v;
}

void put_u32(uint8_t* p, uint32_t v) {
  for (int i = 0; i < 4; ++i) p[i] = (uint8_t)(v >> (8 * i));
}
void put_u64(uint8_t* p, uint64_t v) {
  for (int i = 0; i < 8; ++i) p[i] = (uint8_t)(v >> (8 * i));
}
uint32_t get_u32(const uint8_t* p) {
  uint32_t v = 0;
  for (int i = 0; i < 4; ++i) v |= (uint32_t)p[i] << (8 * i);
  return v;
}
uint64_t get_u64(const uint8_t* p) {
  uint64_t v = 0;
  for (int i = 0; i < 8; ++i) v |= (uint64_t)p[i] << (8 * i);
  return v;
}

qlora_status payload_of(int64_t rows, int64_t cols, int32_t bs, int32_t gb, uint64_t* out) {
  size_t c = 0, a = 0, s = 0;
  const qlora_status st = qlora_sizes(rows, cols, bs, gb, &c, &a, &s);
  if (st != QLORA_OK) return st;
  *out = (uint64_t)c + (uint64_t)a + (uint64_t)s;
  return QLORA_OK;
}

}  // namespace

extern "C" {

qlora_status qlora_level_table_id(int32_t codebook, int32_t absmax_format, uint64_t* id) {
  if (!id) return QLORA_E_NULL;
  float lv[16];
  const qlora_status st = qlora_codebook_levels((qlora_codebook)codebook, lv);
  if (st != QLORA_OK) return st;
  if (absmax_format != QLORA_ABSMAX_LINEAR8 && absmax_format != QLORA_ABSMAX_FP8) return QLORA_E_UNSUPPORTED;
  Fnv1a f;
  f.bytes("qlora-levels-1", 14);
  f.u32((uint32_t)codebook);
  for (float v : lv) f.f32(v);
  f.u32((uint32_t)absmax_format);
  // Second-level code points.  A quotient of two small integers is never
  // within an fp64 rounding error of an fp32 rounding boundary, so rounding
  // the fp64 quotient to fp32 gives RN32 of the exact quotient.
  if (absmax_format == QLORA_ABSMAX_LINEAR8) {
    for (int k = 0; k < 256; ++k) f.f32((float)(k / 255.0));
  } else {
    for (int k = 0; k < 127; ++k) f.f32((float)(e4m3_value(k) / 448.0));
  }
  *id = f.h;
  return QLORA_OK;
}

qlora_status qlora_qtensor_header_write(const qlora_nf4_weight* q, uint8_t* out, size_t out_bytes) {
  if (!q || !out) return QLORA_E_NULL;
  if (out_bytes < QLORA_QTENSOR_HEADER_BYTES) return QLORA_E_FORMAT;
  uint64_t payload = 0, id = 0;
  qlora_status st = payload_of(q->rows, q->cols, q->blocksize, q->group_blocks, &payload);
  if (st != QLORA_OK) return st;
  if ((st = qlora_level_table_id(q->codebook, q->absmax_format, &id)) != QLORA_OK) return st;
  uint8_t h[QLORA_QTENSOR_HEADER_BYTES];
  std::memcpy(h, kMagic, 8);
  put_u32(h + 8, kVersion);
  put_u32(h + 12, QLORA_QTENSOR_HEADER_BYTES);
  put_u64(h + 16, (uint64_t)q->rows);
  put_u64(h + 24, (uint64_t)q->cols);
  put_u32(h + 32, (uint32_t)q->blocksize);
  put_u32(h + 36, (uint32_t)q->group_blocks);
  put_u32(h + 40, (uint32_t)q->codebook);
  put_u32(h + 44, (uint32_t)q->absmax_format);
  put_u64(h + 48, id);
  put_u64(h + 56, payload);
  std::memcpy(out, h, sizeof(h));
  return QLORA_OK;
}

qlora_status qlora_qtensor_header_read(const uint8_t* in, size_t in_bytes, qlora_nf4_weight* q,
                                       uint64_t* payload_bytes) {
  if (!in || !q) return QLORA_E_NULL;
  if (in_bytes < QLORA_QTENSOR_HEADER_BYTES) return QLORA_E_FORMAT;
  if (std::memcmp(in, kMagic, 8) != 0 || get_u32(in + 8) != kVersion ||
      get_u32(in + 12) != QLORA_QTENSOR_HEADER_BYTES)
    return QLORA_E_FORMAT;
  const int64_t rows = (int64_t)get_u64(in + 16), cols = (int64_t)get_u64(in + 24);
  const int32_t bs = (int32_t)get_u32(in + 32), gb = (int32_t)get_u32(in + 36);
  const int32_t cb = (int32_t)get_u32(in + 40), af = (int32_t)get_u32(in + 44);
  uint64_t payload = 0, id = 0;
  qlora_status st = payload_of(rows, cols, bs, gb, &payload);
  if (st != QLORA_OK) return st;
  if (get_u64(in + 56) != payload) return QLORA_E_FORMAT;
  if ((st = qlora_level_table_id(cb, af, &id)) != QLORA_OK) return st;
  if (get_u64(in + 48) != id) return QLORA_E_TABLE;
  q->rows = rows;
  q->cols = cols;
  q->blocksize = bs;
  q->group_blocks = gb;
  q->codebook = cb;
  q->absmax_format = af;
  if (payload_bytes) *payload_bytes = payload;
  return QLORA_OK;
}

}  // extern "C"
