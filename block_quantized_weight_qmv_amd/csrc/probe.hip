// HBM roofline probes: a 128-bit streaming read and a 128-bit copy.  They are
// the "plain kernels of known size" against which GEMV bandwidth and the
// FETCH_SIZE / WRITE_SIZE counters are calibrated on the same GPU.
#include "device_util.h"
#include "launch.h"

namespace qmv {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;
constexpr int64_t kProbeMaxBlocks = 1024;

int64_t probe_read_blocks(uint64_t nbytes) {
  const int64_t vec = static_cast<int64_t>(nbytes / 16);
  int64_t blocks = (vec + kProbeThreads * kProbeUnroll - 1) / (kProbeThreads * kProbeUnroll);
  if (blocks > kProbeMaxBlocks) blocks = kProbeMaxBlocks;
  if (blocks < 1) blocks = 1;
  return blocks;
}

// Each workgroup reads one contiguous chunk (a whole number of
// threads x unroll vectors) with nontemporal 128-bit loads, so every 128-byte
// line is requested by exactly one load instruction.  Among the access
// patterns, grid shapes and cache hints measured on gfx950 (grid-stride,
// chunk per workgroup, chunk per wave; plain and nontemporal; 256-8192
// workgroups), this is the fastest family for a 2 GiB stream: about 7.0 TB/s,
// against 5.5-6.2 TB/s for the same loads without the hint.
__global__ void __launch_bounds__(kProbeThreads)
probe_read_kernel(const uint4* __restrict__ src, int64_t nvec, float* __restrict__ out) {
  typedef uint32_t v4_t __attribute__((ext_vector_type(4)));
  const v4_t* p = reinterpret_cast<const v4_t*>(src);
  constexpr int64_t kStep = static_cast<int64_t>(kProbeThreads) * kProbeUnroll;
  int64_t chunk = (nvec + gridDim.x - 1) / gridDim.x;
  chunk = (chunk + kStep - 1) / kStep * kStep;
  const int64_t begin = static_cast<int64_t>(blockIdx.x) * chunk;
  const int64_t end = begin + chunk < nvec ? begin + chunk : nvec;
  uint32_t acc = 0;
  int64_t i = begin + threadIdx.x;
  for (; i + (kProbeUnroll - 1) * kProbeThreads < end; i += kStep) {
    v4_t v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * kProbeThreads);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < end; i += kProbeThreads) {
    const v4_t v = __builtin_nontemporal_load(p + i);
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
