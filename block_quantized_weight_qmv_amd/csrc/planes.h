// Plane layouts of Q4_K, Q5_K and Q6_K weights ("decode-repacked" layouts, after hipEngine
// 0.3.0, "GGUF Support": GGUF blocks are repacked into decode layouts on load
// and the repacked copy replaces the source).
//
// The canonical layout keeps each 144-byte block whole, so the GEMV's three
// load instructions per lane (block header, code quarter A, code quarter B)
// all touch the same 128-byte lines.  The plane layout moves the same bytes
// into three planes, so that each code load instruction of a wave reads 1 KB
// of consecutive bytes that no other instruction reads:
//
//   N = rows * (cols / 256) blocks, block b = r * (cols / 256) + j,
//   a = 16 N rounded up to a multiple of 256,
//   H  plane at 0:     header of block b (its first 16 bytes: d, dmin,
//                      scales[12]) at 16 b;
//   QA plane at a:     qs[32c .. 32c+16) of block b at a + 64 b + 16 c;
//   QB plane at 5 a:   qs[32c+16 .. 32c+32) of block b at 5 a + 64 b + 16 c;
//   total 5 a + 64 N bytes (the 144 N bytes of the blocks plus under
//   1280 bytes of padding between the planes).
//
// a is recorded in the descriptor's scales_offset field.
//
// Q6_K (210-byte blocks: ql[128] | qh[64] | sc[16] | d), same N, b and a,
// with p = 2h + i for the GEMV lane (h, i) of a block (h, i in {0, 1}):
//   L0 plane at 0:     ql[64h + 16i .. +16)        of block b at 64 b + 16 p;
//   L1 plane at 4 a:   ql[64h + 32 + 16i .. +16)   of block b at 4 a + 64 b + 16 p;
//   QH plane at 8 a:   qh[32h + 16i .. +16)        of block b at 8 a + 64 b + 16 p;
//   SC plane at 12 a:  sc[0 .. 16)                 of block b at 12 a + 16 b;
//   D  plane at 13 a:  d                           of block b at 13 a + 2 b;
//   total 13 a + 2 N bytes (210 N plus under 3328 bytes of padding).
// The three 64-byte planes are read with nontemporal loads, 1 KB of
// consecutive bytes per wave instruction; the sub-scales and d, whose lines
// the next row's instructions share, with plain loads.
//
// Q5_K (176-byte blocks: d | dmin | scales[12] | qh[32] | qs[128]), same N,
// b and a:
//   H   plane at 0:     bytes 0..15 of block b (d, dmin, scales) at 16 b;
//   QH0 plane at a:     qh[0 .. 16) of block b at a + 16 b;
//   QH1 plane at 2 a:   qh[16 .. 32) of block b at 2 a + 16 b;
//   QA  plane at 3 a:   qs[32c .. 32c+16) of block b at 3 a + 64 b + 16 c;
//   QB  plane at 7 a:   qs[32c+16 .. 32c+32) of block b at 7 a + 64 b + 16 c;
//   total 7 a + 64 N bytes (176 N plus under 1792 bytes of padding).
// QA and QB are read with nontemporal loads; the header and qh planes, which
// the four lanes of a block share, with plain loads.
#pragma once

#include <stdint.h>

namespace qmv {

struct Q4KPlanes {
  uint64_t a;      // the plane unit a (16 N rounded up to 256); plane offsets are multiples of it
  uint64_t total;  // bytes of the whole layout
};

__host__ __device__ inline Q4KPlanes q4k_planes(int64_t rows, int64_t cols) {
  const uint64_t n = static_cast<uint64_t>(rows) * static_cast<uint64_t>(cols / 256);
  const uint64_t a = (16 * n + 255) / 256 * 256;
  return Q4KPlanes{a, 5 * a + 64 * n};
}

__host__ __device__ inline Q4KPlanes q5k_planes(int64_t rows, int64_t cols) {
  const uint64_t n = static_cast<uint64_t>(rows) * static_cast<uint64_t>(cols / 256);
  const uint64_t a = (16 * n + 255) / 256 * 256;
  return Q4KPlanes{a, 7 * a + 64 * n};
}

__host__ __device__ inline Q4KPlanes q6k_planes(int64_t rows, int64_t cols) {
  const uint64_t n = static_cast<uint64_t>(rows) * static_cast<uint64_t>(cols / 256);
  const uint64_t a = (16 * n + 255) / 256 * 256;
  return Q4KPlanes{a, 13 * a + 2 * n};
}

}  // namespace qmv
