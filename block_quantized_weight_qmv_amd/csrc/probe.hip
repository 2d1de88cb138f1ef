// HBM roofline probes: a 128-bit streaming read and a 128-bit copy.  They are
// the "plain kernels of known size" against which GEMV bandwidth and the
// FETCH_SIZE / WRITE_SIZE counters are calibrated on the same GPU.
#include "device_util.h"
#include "launch.h"

namespace qmv {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;

int64_t probe_read_blocks(uint64_t nbytes) {
  const int64_t vec = static_cast<int64_t>(nbytes / 16);
  int64_t blocks = (vec + kProbeThreads * kProbeUnroll - 1) / (kProbeThreads * kProbeUnroll);
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  return blocks;
}

__global__ void __launch_bounds__(kProbeThreads)
probe_read_kernel(const uint4* __restrict__ src, int64_t nvec, float* __restrict__ out) {
  uint32_t acc = 0;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kProbeThreads;
  int64_t i = static_cast<int64_t>(blockIdx.x) * kProbeThreads + threadIdx.x;
  for (; i + (kProbeUnroll - 1) * stride < nvec; i += kProbeUnroll * stride) {
    uint4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < nvec; i += stride) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  __shared__ uint32_t red[kProbeThreads];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int k = 0; k < kProbeThreads; ++k) t ^= red[k];
    out[blockIdx.x] = static_cast<float>(t & 0xFFFFu);
  }
}

__global__ void __launch_bounds__(kProbeThreads)
probe_copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, int64_t nvec) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kProbeThreads;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kProbeThreads + threadIdx.x; i < nvec;
       i += stride)
    dst[i] = src[i];
}

hipError_t probe_read(const void* src, uint64_t nbytes, float* out, hipStream_t s) {
  const int blocks = static_cast<int>(probe_read_blocks(nbytes));
  hipLaunchKernelGGL(probe_read_kernel, dim3(blocks), dim3(kProbeThreads), 0, s,
                     static_cast<const uint4*>(src), static_cast<int64_t>(nbytes / 16), out);
  return hipGetLastError();
}

hipError_t probe_copy(const void* src, void* dst, uint64_t nbytes, hipStream_t s) {
  const int64_t nvec = static_cast<int64_t>(nbytes / 16);
  int64_t blocks = (nvec + kProbeThreads - 1) / kProbeThreads;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(probe_copy_kernel, dim3(static_cast<int>(blocks)), dim3(kProbeThreads), 0, s,
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), nvec);
  return hipGetLastError();
}

}  // namespace qmv
