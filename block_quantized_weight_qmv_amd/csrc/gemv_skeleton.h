// Decode GEMV skeleton for gfx950, shared by the four block formats.  One
// launch computes up to kMaxItems independent GEMVs y_i = W_i x_i of the same
// format and activation type (the single-matrix call is the case n = 1).
//
// Work split:
//  * For matrix i, `kw_i` waves split K: wave k owns the columns
//    [k*P::kColsPerWave, ...) and keeps that slice of x_i in VGPRs (fp32) for
//    its whole life, so activations are read once per wave, not once per row.
//  * The rows of matrix i are cut into nsets_i contiguous row sets of q_i or
//    q_i+1 rows; a set is processed by kw_i waves of one workgroup, R rows per
//    tile.  All workgroups have the same size (the largest kw among the
//    matrices, at least 4 waves); with kw_i == 1 a workgroup serves one set
//    per wave, with kw_i > 1 one set (spare waves leave at once).  Set sizes
//    are chosen so that every wave streams about the same number of bytes and
//    the launch is about one resident generation of waves: long-lived waves
//    with many tiles keep memory and arithmetic overlapped, and the small
//    matrices of a launch share the ramp-up and tail of the big ones.
//  * Loads are plain 128-bit global loads issued unconditionally (rows past
//    the set's end re-read its last row; lanes without columns read a valid
//    block and carry a zero x slice), so the compiler can track them exactly:
//    the x slice and two tiles are requested before the first wait, and the
//    next tile is requested before the current one is consumed.
//  * The R row partials of a tile are reduced together: two DPP exchange
//    steps leave each lane of a quad with one row's quad sum, then rotations
//    within rows of 16 lanes and swaps across rows finish the sum.  The order
//    is fixed, so results are deterministic; with kw > 1 the wave totals are
//    added in wave order through LDS.  y is overwritten.
//
// A format policy P provides kColsPerWave, kXElems, XSlice, Frag, a
// constructor (w, scales_offset, cols, kslot, lane), load_x_raw(x, uint4*),
// finish_x<XT>(raw, XSlice&), load(row, Frag&) and dot(Frag, XSlice) -> this
// lane's partial of W[row] . x.
#pragma once

#include "device_util.h"
#include "launch.h"

namespace qmv {

// DPP move with a compile-time control word.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float xor_lane(float v, int lane, int mask) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __float_as_int(v)));
}

// Sum each of the R (1, 2 or 4) per-lane partials over the wave.  On return,
// lane q < R holds the total of partial q.
template <int R>
__device__ __forceinline__ float reduce_rows(const float* a, int lane) {
  float v;
  if (R == 1) {
    v = a[0];
    v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  } else if (R == 2) {
    const bool odd = lane & 1;
    v = odd ? a[1] : a[0];
    v += dpp<0xB1>(odd ? a[0] : a[1]);
    v += dpp<0x4E>(v);
  } else {
    const bool odd = lane & 1, b1 = lane & 2;
    float ka = odd ? a[1] : a[0];
    float kb = odd ? a[3] : a[2];
    ka += dpp<0xB1>(odd ? a[0] : a[1]);
    kb += dpp<0xB1>(odd ? a[2] : a[3]);
    v = b1 ? kb : ka;
    v += dpp<0x4E>(b1 ? ka : kb);
  }
  v += dpp<0x124>(v);    // row_ror:4
  v += dpp<0x128>(v);    // row_ror:8
  v += xor_lane(v, lane, 16);
  v += xor_lane(v, lane, 32);
  return v;
}

template <class P, int R>
__device__ __forceinline__ void load_tile(const P& pol, typename P::Frag* f, int row0, int r_last) {
#pragma unroll
  for (int r = 0; r < R; ++r) pol.load(min(row0 + r, r_last), f[r]);
}

template <class P, int R>
__device__ __forceinline__ void finish_tile(const P& pol, const typename P::Frag* f,
                                            const typename P::XSlice& xs, float* y, int row0,
                                            int r_end, int kw, int lane, int wave, float* part) {
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = pol.dot(f[r], xs);
  const float t = reduce_rows<R>(acc, lane);
  if (kw == 1) {
    if (lane < R && row0 + lane < r_end) y[row0 + lane] = t;
  } else {
    if (lane < R) part[wave * R + lane] = t;
    __syncthreads();
    if (wave == 0 && lane < R && row0 + lane < r_end) {
      float s = 0.f;
      for (int k = 0; k < kw; ++k) s += part[k * R + lane];
      y[row0 + lane] = s;
    }
    __syncthreads();
  }
}

// One matrix of a launch, as laid out by plan_gemv (host).
struct GemvItem {
  const uint8_t* w;
  uint64_t scales_offset;
  const void* x;      // [batch][cols]
  float* y;           // [batch][rows]
  int rows, cols;
  int kw;             // waves along K
  int sets_per_wg;    // row sets per workgroup
  int nsets, q, rem;  // rows = q * nsets + rem; set s has q + (s < rem) rows
  int wg_begin;       // first workgroup of this matrix
};

struct GemvLaunch {
  int n;
  GemvItem item[kMaxItems];
};

template <class P, typename XT, int R, int MAXT>
__global__ void __launch_bounds__(MAXT)
gemv_kernel(const GemvLaunch args) {
  // This workgroup's matrix (wave-uniform scan over at most kMaxItems).
  int it = 0;
#pragma unroll 1
  for (int k = 1; k < args.n; ++k)
    if (static_cast<int>(blockIdx.x) >= args.item[k].wg_begin) it = k;
  const GemvItem& m = args.item[it];

  const int lane = __lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kw = m.kw;
  if (wave >= kw * m.sets_per_wg) return;  // spare waves of a kw > 1 workgroup
  const int kslot = wave % kw;
  const int set = (blockIdx.x - m.wg_begin) * m.sets_per_wg + wave / kw;
  if (set >= m.nsets) return;  // only with kw == 1, where no barrier is shared
  const XT* x = static_cast<const XT*>(m.x) + static_cast<size_t>(blockIdx.y) * m.cols;
  float* y = m.y + static_cast<size_t>(blockIdx.y) * m.rows;
  const int r_begin = set * m.q + min(set, m.rem);
  const int r_end = r_begin + m.q + (set < m.rem ? 1 : 0);
  const int r_last = r_end - 1;

  __shared__ float part[(MAXT / 64) * R];
  const P pol(m.w, m.scales_offset, m.cols, kslot, lane);

  // Issue order: x slice, tile 0, tile 1; only then wait for x.
  uint4 raw[P::kXElems * sizeof(XT) / 16];
  pol.load_x_raw(x, raw);
  __builtin_amdgcn_sched_barrier(0);
  typename P::Frag fa[R], fb[R];
  load_tile<P, R>(pol, fa, r_begin, r_last);
  load_tile<P, R>(pol, fb, r_begin + R, r_last);
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  typename P::XSlice xs;
  pol.template finish_x<XT>(raw, xs);

  // Each prefetch is pinned right after the tile whose registers it reuses:
  // left alone, the compiler sinks the loads below the next tile's arithmetic
  // (across the basic blocks of the reduction), which leaves one tile in
  // flight per wave.  An empty asm with a memory clobber keeps the loads in
  // program order without waiting for them (the weight pointer is
  // deliberately not __restrict__: a restrict-qualified read-only pointer
  // lets the compiler move its loads across the clobber).
  int r0 = r_begin;  // every set has at least one row
  do {
    finish_tile<P, R>(pol, fa, xs, y, r0, r_end, kw, lane, wave, part);
    load_tile<P, R>(pol, fa, r0 + 2 * R, r_last);
    __asm__ __volatile__("" ::: "memory");
    if (r0 + R >= r_end) break;
    finish_tile<P, R>(pol, fb, xs, y, r0 + R, r_end, kw, lane, wave, part);
    load_tile<P, R>(pol, fb, r0 + 3 * R, r_last);
    __asm__ __volatile__("" ::: "memory");
    r0 += 2 * R;
  } while (r0 < r_end);
}

// Widest K split among the matrices of a launch.
template <class P>
inline int max_kw(const GemvCall* calls, int n) {
  int m = 1;
  for (int i = 0; i < n; ++i) {
    const int kw = static_cast<int>((calls[i].W->cols + P::kColsPerWave - 1) / P::kColsPerWave);
    m = kw > m ? kw : m;
  }
  return m;
}

// Lay out a launch over `n` matrices with `waves` waves per workgroup: K split
// and row sets per matrix, workgroup ranges.  Rows per set are the same for
// every matrix, chosen so that the launch holds about `target_waves` waves.
template <class P>
inline int plan_gemv(const GemvCall* calls, int n, int waves, int64_t target_waves,
                     GemvLaunch* L) {
  int64_t wave_rows = 0;  // sum over matrices of rows * kw
  for (int i = 0; i < n; ++i)
    wave_rows += calls[i].W->rows *
                 ((calls[i].W->cols + P::kColsPerWave - 1) / P::kColsPerWave);
  int64_t rps = (wave_rows + target_waves - 1) / target_waves;
  if (rps < 1) rps = 1;
  int wg = 0;
  L->n = n;
  for (int i = 0; i < n; ++i) {
    GemvItem& m = L->item[i];
    const qmv_weights* W = calls[i].W;
    m.w = static_cast<const uint8_t*>(W->data);
    m.scales_offset = W->scales_offset;
    m.x = calls[i].x;
    m.y = calls[i].y;
    m.rows = static_cast<int>(W->rows);
    m.cols = static_cast<int>(W->cols);
    m.kw = static_cast<int>((W->cols + P::kColsPerWave - 1) / P::kColsPerWave);
    m.sets_per_wg = m.kw == 1 ? waves : 1;  // a kw > 1 set shares its workgroup's barrier
    m.nsets = static_cast<int>((m.rows + rps - 1) / rps);
    m.q = m.rows / m.nsets;
    m.rem = m.rows % m.nsets;
    m.wg_begin = wg;
    wg += (m.nsets + m.sets_per_wg - 1) / m.sets_per_wg;
  }
  return wg;
}

// Workgroups of `kernel` (block threads) the current device holds at once;
// queried once per kernel and device.
template <typename K>
inline int64_t resident_workgroups(K kernel, int block) {
  static int cache[64];  // per device; 0 = not yet queried
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cache[dev] == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0) != hipSuccess ||
        cus <= 0 || per_cu <= 0) {
      cus = 256;
      per_cu = 1;
    }
    cache[dev] = cus * per_cu;
  }
  return cache[dev];
}

template <class P, typename XT, int R, int MAXT>
hipError_t launch_cfg(const GemvCall* calls, int n, int waves, int64_t batch, hipStream_t stream) {
  auto kernel = gemv_kernel<P, XT, R, MAXT>;
  const int block = 64 * waves;
  const int64_t target = resident_workgroups(kernel, block) * waves;
  GemvLaunch L;
  const int grid = plan_gemv<P>(calls, n, waves, target, &L);
  hipLaunchKernelGGL(kernel, dim3(grid, static_cast<unsigned>(batch)), dim3(block), 0, stream, L);
  return hipGetLastError();
}

template <class P, typename XT>
hipError_t launch_gemv_typed(const GemvCall* calls, int n, int64_t batch, hipStream_t stream) {
  const int kw = max_kw<P>(calls, n);
  if (kw > 16) return hipErrorInvalidValue;
  const int waves = kw < 4 ? 4 : kw;
  if (waves <= 4) return launch_cfg<P, XT, 4, 256>(calls, n, waves, batch, stream);
  if (waves <= 8) return launch_cfg<P, XT, 4, 512>(calls, n, waves, batch, stream);
  return launch_cfg<P, XT, 2, 1024>(calls, n, waves, batch, stream);
}

template <class P>
hipError_t launch_gemv(const GemvCall* calls, int n, int x_dtype, int64_t batch,
                       hipStream_t stream) {
  switch (x_dtype) {
    case QMV_F32: return launch_gemv_typed<P, float>(calls, n, batch, stream);
    case QMV_F16: return launch_gemv_typed<P, _Float16>(calls, n, batch, stream);
    case QMV_BF16: return launch_gemv_typed<P, bf16_t>(calls, n, batch, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qmv
