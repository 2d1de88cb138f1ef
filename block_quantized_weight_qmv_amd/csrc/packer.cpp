// Host block packer: integer codes + fp16 scale bit patterns -> canonical
// block bytes.  Layouts as in qmv.h (VTE, feature list: llama.cpp's reference
// Q8_0 / Q4_K / Q6_K layouts; hipEngine 0.3.0, "GGUF Support": Q5_K, read as
// GGUF's published block; INT4 group-128 planes as this library reads the
// datastack.it summary of "annotated-llm-runtime").  Every range is checked
// before the first byte is written, so a failed call leaves `out` untouched.
#include <string.h>

#include "api_internal.h"

namespace {

void put16(uint8_t* p, uint16_t v) {
  p[0] = static_cast<uint8_t>(v & 0xFF);
  p[1] = static_cast<uint8_t>(v >> 8);
}

int32_t check_common(int32_t fmt, const void* a, const void* b, int64_t rows, int64_t cols,
                     const uint8_t* out, uint64_t out_bytes) {
  if (!a || !b || !out) return qmv::fail(QMV_ERR_NULL, "packer: NULL pointer argument");
  const uint64_t need = qmv_packed_size(fmt, rows, cols);
  if (need == 0) return qmv::fail(QMV_ERR_SHAPE, "packer: bad shape %lld x %lld", (long long)rows, (long long)cols);
  if (out_bytes < need)
    return qmv::fail(QMV_ERR_SIZE, "packer: output holds %llu bytes, %llu needed",
                     (unsigned long long)out_bytes, (unsigned long long)need);
  return QMV_OK;
}

// The twelve scale bytes shared by Q4_K and Q5_K: eight 6-bit scales and
// eight 6-bit mins; entries 0-3 sit in the low six bits of bytes 0-3 / 4-7,
// entries 4-7 split into a low nibble in bytes 8-11 and two high bits in the
// top of bytes 0-3 / 4-7.
void put_k_scales(uint8_t* s, const uint8_t* sc, const uint8_t* m) {
  for (int k = 0; k < 4; ++k) {
    s[k] = static_cast<uint8_t>(sc[k] | ((sc[k + 4] >> 4) << 6));
    s[k + 4] = static_cast<uint8_t>(m[k] | ((m[k + 4] >> 4) << 6));
    s[k + 8] = static_cast<uint8_t>((sc[k + 4] & 15) | ((m[k + 4] & 15) << 4));
  }
}

int32_t check_k_scales(const char* name, const uint8_t* sc6, const uint8_t* m6, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (sc6[i] > 63 || m6[i] > 63)
      return qmv::fail(QMV_ERR_RANGE, "%s: 6-bit scale/min out of range at %lld", name, (long long)i);
  return QMV_OK;
}

}  // namespace

extern "C" {

int32_t qmv_pack_q8_0(const uint16_t* d_bits, const int8_t* q, int64_t rows, int64_t cols,
                      uint8_t* out, uint64_t out_bytes) {
  const int32_t st = check_common(QMV_Q8_0, d_bits, q, rows, cols, out, out_bytes);
  if (st != QMV_OK) return st;
  const int64_t nb = cols / 32;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t j = 0; j < nb; ++j) {
      uint8_t* blk = out + (r * nb + j) * 34;
      put16(blk, d_bits[r * nb + j]);
      memcpy(blk + 2, q + r * cols + j * 32, 32);
    }
  return qmv::ok();
}

int32_t qmv_pack_q4_k(const uint16_t* d_bits, const uint16_t* dmin_bits, const uint8_t* sc6,
                      const uint8_t* m6, const uint8_t* q4, int64_t rows, int64_t cols,
                      uint8_t* out, uint64_t out_bytes) {
  int32_t st = check_common(QMV_Q4_K, d_bits, q4, rows, cols, out, out_bytes);
  if (st != QMV_OK) return st;
  if (!dmin_bits || !sc6 || !m6) return qmv::fail(QMV_ERR_NULL, "packer: NULL pointer argument");
  const int64_t nb = cols / 256;
  if ((st = check_k_scales("q4_k", sc6, m6, rows * nb * 8)) != QMV_OK) return st;
  for (int64_t i = 0; i < rows * cols; ++i)
    if (q4[i] > 15) return qmv::fail(QMV_ERR_RANGE, "q4_k: code > 15 at %lld", (long long)i);
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t j = 0; j < nb; ++j) {
      const int64_t bi = r * nb + j;
      uint8_t* blk = out + bi * 144;
      put16(blk, d_bits[bi]);
      put16(blk + 2, dmin_bits[bi]);
      put_k_scales(blk + 4, sc6 + bi * 8, m6 + bi * 8);
      const uint8_t* u = q4 + r * cols + j * 256;
      uint8_t* qs = blk + 16;
      for (int c = 0; c < 4; ++c)
        for (int l = 0; l < 32; ++l)
          qs[32 * c + l] = static_cast<uint8_t>(u[64 * c + l] | (u[64 * c + 32 + l] << 4));
    }
  return qmv::ok();
}

int32_t qmv_pack_q5_k(const uint16_t* d_bits, const uint16_t* dmin_bits, const uint8_t* sc6,
                      const uint8_t* m6, const uint8_t* q5, int64_t rows, int64_t cols,
                      uint8_t* out, uint64_t out_bytes) {
  int32_t st = check_common(QMV_Q5_K, d_bits, q5, rows, cols, out, out_bytes);
  if (st != QMV_OK) return st;
  if (!dmin_bits || !sc6 || !m6) return qmv::fail(QMV_ERR_NULL, "packer: NULL pointer argument");
  const int64_t nb = cols / 256;
  if ((st = check_k_scales("q5_k", sc6, m6, rows * nb * 8)) != QMV_OK) return st;
  for (int64_t i = 0; i < rows * cols; ++i)
    if (q5[i] > 31) return qmv::fail(QMV_ERR_RANGE, "q5_k: code > 31 at %lld", (long long)i);
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t j = 0; j < nb; ++j) {
      const int64_t bi = r * nb + j;
      uint8_t* blk = out + bi * 176;
      put16(blk, d_bits[bi]);
      put16(blk + 2, dmin_bits[bi]);
      put_k_scales(blk + 4, sc6 + bi * 8, m6 + bi * 8);
      const uint8_t* u = q5 + r * cols + j * 256;
      uint8_t* qh = blk + 16;
      uint8_t* qs = blk + 48;
      for (int l = 0; l < 32; ++l) {
        uint8_t h = 0;
        for (int s = 0; s < 8; ++s) h = static_cast<uint8_t>(h | ((u[32 * s + l] >> 4) << s));
        qh[l] = h;
      }
      for (int c = 0; c < 4; ++c)
        for (int l = 0; l < 32; ++l)
          qs[32 * c + l] = static_cast<uint8_t>((u[64 * c + l] & 15) | ((u[64 * c + 32 + l] & 15) << 4));
    }
  return qmv::ok();
}

int32_t qmv_pack_q6_k(const uint16_t* d_bits, const int8_t* sc8, const uint8_t* q6, int64_t rows,
                      int64_t cols, uint8_t* out, uint64_t out_bytes) {
  int32_t st = check_common(QMV_Q6_K, d_bits, q6, rows, cols, out, out_bytes);
  if (st != QMV_OK) return st;
  if (!sc8) return qmv::fail(QMV_ERR_NULL, "packer: NULL pointer argument");
  for (int64_t i = 0; i < rows * cols; ++i)
    if (q6[i] > 63) return qmv::fail(QMV_ERR_RANGE, "q6_k: code > 63 at %lld", (long long)i);
  const int64_t nb = cols / 256;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t j = 0; j < nb; ++j) {
      const int64_t bi = r * nb + j;
      uint8_t* blk = out + bi * 210;
      const uint8_t* q = q6 + r * cols + j * 256;
      uint8_t* ql = blk;
      uint8_t* qh = blk + 128;
      for (int h = 0; h < 2; ++h)
        for (int l = 0; l < 32; ++l) {
          const uint8_t* t = q + 128 * h + l;  // weights 128h + 32g + l, g = 0..3
          ql[64 * h + l] = static_cast<uint8_t>((t[0] & 15) | ((t[64] & 15) << 4));
          ql[64 * h + 32 + l] = static_cast<uint8_t>((t[32] & 15) | ((t[96] & 15) << 4));
          qh[32 * h + l] = static_cast<uint8_t>((t[0] >> 4) | ((t[32] >> 4) << 2) |
                                                ((t[64] >> 4) << 4) | ((t[96] >> 4) << 6));
        }
      memcpy(blk + 192, sc8 + bi * 16, 16);
      put16(blk + 208, d_bits[bi]);
    }
  return qmv::ok();
}

int32_t qmv_pack_int4_g128(const uint16_t* s_bits, const int8_t* q, int64_t rows, int64_t cols,
                           uint8_t* out, uint64_t out_bytes) {
  const int32_t st = check_common(QMV_INT4_G128, s_bits, q, rows, cols, out, out_bytes);
  if (st != QMV_OK) return st;
  for (int64_t i = 0; i < rows * cols; ++i)
    if (q[i] < -8 || q[i] > 7) return qmv::fail(QMV_ERR_RANGE, "int4: code outside [-8, 7] at %lld", (long long)i);
  for (int64_t i = 0; i < rows * cols / 2; ++i)
    out[i] = static_cast<uint8_t>((q[2 * i] + 8) | ((q[2 * i + 1] + 8) << 4));
  uint8_t* sp = out + rows * cols / 2;
  for (int64_t i = 0; i < rows * (cols / 128); ++i) put16(sp + 2 * i, s_bits[i]);
  return qmv::ok();
}

}  // extern "C"
