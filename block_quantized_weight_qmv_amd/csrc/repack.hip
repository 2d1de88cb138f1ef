// Repack of canonical Q4_K, Q5_K and Q6_K blocks into the plane layouts of
// planes.h, on the device, once per weight tensor (hipEngine 0.3.0, "GGUF Support": the
// decode repack happens at load time).  Q4_K: one thread per block, nine
// 16-byte loads of the block, one 16-byte store to each plane slot.  Bytes are moved,
// never changed, so the repacked tensor decodes to exactly the same weights.
#include "device_util.h"
#include "launch.h"
#include "planes.h"

namespace qmv {

__global__ void __launch_bounds__(256)
repack_q4_k_planes_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int64_t nblocks,
                          uint64_t a) {
  const int64_t b = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (b >= nblocks) return;
  const uint4* s = reinterpret_cast<const uint4*>(src + b * 144);
  uint4 v[9];
#pragma unroll
  for (int i = 0; i < 9; ++i) v[i] = s[i];
  reinterpret_cast<uint4*>(dst + 16 * b)[0] = v[0];
  uint4* qa = reinterpret_cast<uint4*>(dst + a + 64 * b);
  uint4* qb = reinterpret_cast<uint4*>(dst + 5 * a + 64 * b);
  // qs[32c .. 32c+16) is block chunk 1 + 2c, qs[32c+16 .. 32c+32) chunk 2 + 2c
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    qa[c] = v[1 + 2 * c];
    qb[c] = v[2 + 2 * c];
  }
}

// Q5_K: one thread per block, eleven 16-byte loads, one store per plane slot.
__global__ void __launch_bounds__(256)
repack_q5_k_planes_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int64_t nblocks,
                          uint64_t a) {
  const int64_t b = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (b >= nblocks) return;
  const uint4* s = reinterpret_cast<const uint4*>(src + b * 176);
  uint4 v[11];
#pragma unroll
  for (int i = 0; i < 11; ++i) v[i] = s[i];
  reinterpret_cast<uint4*>(dst)[b] = v[0];                // header
  reinterpret_cast<uint4*>(dst + a)[b] = v[1];            // qh[0 .. 16)
  reinterpret_cast<uint4*>(dst + 2 * a)[b] = v[2];        // qh[16 .. 32)
  uint4* qa = reinterpret_cast<uint4*>(dst + 3 * a + 64 * b);
  uint4* qb = reinterpret_cast<uint4*>(dst + 7 * a + 64 * b);
  // qs[32c .. 32c+16) is block chunk 3 + 2c, qs[32c+16 .. 32c+32) chunk 4 + 2c
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    qa[c] = v[3 + 2 * c];
    qb[c] = v[4 + 2 * c];
  }
}

hipError_t repack_q5_k_planes(const qmv_weights& src, void* dst, hipStream_t s) {
  const int64_t nblocks = src.rows * (src.cols / 256);
  const Q4KPlanes pl = q5k_planes(src.rows, src.cols);
  const int64_t grid = (nblocks + 255) / 256;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(repack_q5_k_planes_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, s,
                     static_cast<const uint8_t*>(src.data), static_cast<uint8_t*>(dst), nblocks,
                     pl.a);
  return hipGetLastError();
}

// Q6_K: one thread per (2-byte aligned) block, read with unaligned 16-byte
// loads (ql 8, qh 4, sc 1) and a 2-byte load of d.
__global__ void __launch_bounds__(256)
repack_q6_k_planes_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int64_t nblocks,
                          uint64_t a) {
  const int64_t b = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (b >= nblocks) return;
  const uint8_t* p = src + b * 210;
  uint4 ql[8], qh[4];
#pragma unroll
  for (int k = 0; k < 8; ++k) ql[k] = ld16_any(p + 16 * k);
#pragma unroll
  for (int k = 0; k < 4; ++k) qh[k] = ld16_any(p + 128 + 16 * k);
  const uint4 sc = ld16_any(p + 192);
  const uint16_t d = static_cast<uint16_t>(ld_u16(p + 208));
  uint4* l0 = reinterpret_cast<uint4*>(dst + 64 * b);
  uint4* l1 = reinterpret_cast<uint4*>(dst + 4 * a + 64 * b);
  uint4* h = reinterpret_cast<uint4*>(dst + 8 * a + 64 * b);
  // slot p = 2h + i: ql chunk 4h + i (L0), 4h + 2 + i (L1), qh chunk 2h + i
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      l0[2 * hh + i] = ql[4 * hh + i];
      l1[2 * hh + i] = ql[4 * hh + 2 + i];
      h[2 * hh + i] = qh[2 * hh + i];
    }
  reinterpret_cast<uint4*>(dst + 12 * a)[b] = sc;
  reinterpret_cast<uint16_t*>(dst + 13 * a)[b] = d;
}

hipError_t repack_q6_k_planes(const qmv_weights& src, void* dst, hipStream_t s) {
  const int64_t nblocks = src.rows * (src.cols / 256);
  const Q4KPlanes pl = q6k_planes(src.rows, src.cols);
  const int64_t grid = (nblocks + 255) / 256;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(repack_q6_k_planes_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, s,
                     static_cast<const uint8_t*>(src.data), static_cast<uint8_t*>(dst), nblocks,
                     pl.a);
  return hipGetLastError();
}

hipError_t repack_q4_k_planes(const qmv_weights& src, void* dst, hipStream_t s) {
  const int64_t nblocks = src.rows * (src.cols / 256);
  const Q4KPlanes pl = q4k_planes(src.rows, src.cols);
  const int64_t grid = (nblocks + 255) / 256;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(repack_q4_k_planes_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, s,
                     static_cast<const uint8_t*>(src.data), static_cast<uint8_t*>(dst), nblocks,
                     pl.a);
  return hipGetLastError();
}

}  // namespace qmv
