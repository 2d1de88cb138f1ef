// Decode GEMV skeleton for gfx950, shared by the four block formats.
//
// Work split (one launch, y = W x for one activation row per grid.y):
//  * `kw` waves split K: wave k owns the columns [k*P::kColsPerWave, ...) and
//    keeps that slice of x in VGPRs (converted to fp32) for the whole kernel,
//    so every activation is read once per wave, not once per row.
//  * Rows are cut into `nsets` contiguous, balanced row sets; each set is
//    processed by one group of kw waves, R rows at a time.  All loads of the R
//    rows are issued before any arithmetic, so each lane has R independent
//    128-bit weight streams in flight.
//  * Within a wave, lanes split the slice along K so that one load
//    instruction of the wave reads consecutive bytes of a row (coalesced).
//  * Per row, the lane partial sums are added by a fixed-order wave64 DPP
//    reduction; with kw > 1 the kw wave totals meet in LDS and are added in
//    wave order.  The result is deterministic and y is overwritten.
//
// A format policy P provides: kColsPerWave, Params, XSlice, Frag, a
// constructor (params, cols, kslot, lane) setting `ok` for lanes that own
// columns, load_x(x, XSlice&), load(row, Frag&), zero(Frag&) and
// dot(Frag, XSlice) -> this lane's partial of W[row] . x.
#pragma once

#include "device_util.h"
#include "launch.h"

namespace qmv {

template <class P, typename XT, int R, int MAXT>
__global__ void __launch_bounds__(MAXT)
gemv_kernel(typename P::Params prm, const XT* __restrict__ x, float* __restrict__ y,
            int rows, int cols, int nsets, int kw) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int kslot = wave % kw;
  const int sets_per_wg = (blockDim.x >> 6) / kw;
  const int set = blockIdx.x * sets_per_wg + wave / kw;
  x += static_cast<size_t>(blockIdx.y) * cols;
  y += static_cast<size_t>(blockIdx.y) * rows;

  const P pol(prm, cols, kslot, lane);
  typename P::XSlice xs;
  pol.load_x(x, xs);

  int r_begin = 0, r_end = 0;
  if (set < nsets) {
    r_begin = part_begin(set, rows, nsets);
    r_end = part_begin(set + 1, rows, nsets);
  }

  __shared__ float part[(MAXT / 64) * R];

  for (int r0 = r_begin; r0 < r_end; r0 += R) {
    typename P::Frag f[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (pol.ok && r0 + r < r_end)
        pol.load(r0 + r, f[r]);
      else
        P::zero(f[r]);
    }
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = pol.dot(f[r], xs);

    if (kw == 1) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float t = wave_sum(acc[r]);
        if (lane == r && r0 + r < r_end) y[r0 + r] = t;
      }
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float t = wave_sum(acc[r]);
        if (lane == r) part[wave * R + r] = t;
      }
      __syncthreads();
      if (wave == 0 && lane < R && r0 + lane < r_end) {
        float t = 0.f;
        for (int k = 0; k < kw; ++k) t += part[k * R + lane];
        y[r0 + lane] = t;
      }
      __syncthreads();
    }
  }
}

// Launch P's GEMV for every activation row of `a`.
template <class P, typename XT>
hipError_t launch_gemv_typed(const GemvArgs& a, const typename P::Params& prm) {
  const int rows = static_cast<int>(a.W->rows);
  const int cols = static_cast<int>(a.W->cols);
  const int kw = (cols + P::kColsPerWave - 1) / P::kColsPerWave;
  if (kw > 16) return hipErrorInvalidValue;
  const Split s = make_split(rows, kw, 2048);
  const dim3 grid(s.grid, static_cast<unsigned>(a.batch));
  const dim3 block(s.threads);
  const XT* x = static_cast<const XT*>(a.x);
  if (s.threads <= 256) {
    hipLaunchKernelGGL((gemv_kernel<P, XT, 4, 256>), grid, block, 0, a.stream, prm, x, a.y,
                       rows, cols, s.nsets, kw);
  } else if (s.threads <= 512) {
    hipLaunchKernelGGL((gemv_kernel<P, XT, 4, 512>), grid, block, 0, a.stream, prm, x, a.y,
                       rows, cols, s.nsets, kw);
  } else {
    hipLaunchKernelGGL((gemv_kernel<P, XT, 2, 1024>), grid, block, 0, a.stream, prm, x, a.y,
                       rows, cols, s.nsets, kw);
  }
  return hipGetLastError();
}

template <class P>
hipError_t launch_gemv(const GemvArgs& a, const typename P::Params& prm) {
  switch (a.x_dtype) {
    case QMV_F32: return launch_gemv_typed<P, float>(a, prm);
    case QMV_F16: return launch_gemv_typed<P, _Float16>(a, prm);
    case QMV_BF16: return launch_gemv_typed<P, bf16_t>(a, prm);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qmv
