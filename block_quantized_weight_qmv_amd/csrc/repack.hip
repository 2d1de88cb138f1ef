// Repack of canonical Q4_K blocks into the plane layout of planes.h, on the
// device, once per weight tensor (hipEngine 0.3.0, "GGUF Support": the
// decode repack happens at load time).  One thread per block: nine 16-byte
// loads of the block, one 16-byte store to each plane slot.  Bytes are moved,
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
