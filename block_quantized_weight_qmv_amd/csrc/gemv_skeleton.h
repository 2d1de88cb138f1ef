// Decode GEMV skeleton for gfx950, shared by the four block formats.  One
// launch computes up to kMaxItems independent GEMVs y_i = W_i x_i of the same
// format and activation type (the single-matrix call is the case n = 1).
//
// Work split:
//  * For matrix i, `kw_i` waves split K: wave k owns the columns
//    [k*P::kColsPerWave, ...) and keeps that slice of x_i in VGPRs (fp32) for
//    its whole life, so activations are read once per wave, not once per row.
//  * The rows of matrix i are cut into nsets_i contiguous row sets of q_i or
//    q_i+R rows (q_i a multiple of R; only the matrix's last set can end in
//    a partial tile); a set is processed by kw_i waves of one workgroup, R
//    rows per tile.  Whole tiles matter for streams read with the
//    nontemporal hint: a partial tile re-reads its last row, and such a line
//    is no longer in L2.  All workgroups have the same size (the largest kw among the
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
//  * When every matrix of the launch fits one wave's K slice (kw == 1, the
//    SX kernels), all waves of a workgroup need the same activations: the
//    workgroup reads x from global memory once, a quarter per wave, into LDS,
//    and each wave takes its slice from there.  Read per wave instead, x
//    (16 KB per wave for fp32 x and 4096 columns) is a large share of what
//    the compute unit's vector memory path has to move before the first
//    weights arrive.
//  * The R row partials of a tile are reduced together: two DPP exchange
//    steps leave each lane of a quad with one row's quad sum, then rotations
//    within rows of 16 lanes and swaps across rows finish the sum.  The order
//    is fixed, so results are deterministic; with kw > 1 the wave totals are
//    added in wave order through LDS.  y is overwritten.
//
// A format policy P provides kColsPerWave, kXElems, XSliceT<XT> (the lane's
// activations as the policy multiplies activations of type XT), Frag, a
// constructor (w, scales_offset, cols, kslot, lane), load_x_raw(x, uint4*),
// finish_x<XT>(raw, XSliceT<XT>&), load(row, Frag&),
// dot<XT>(Frag, XSliceT<XT>) -> this lane's partial of W[row] . x, and, for
// the multi-row kernels below, dot_rows<XT, NBR>(Frag, const XSliceT<XT>*,
// float* out) -> out[m] = dot<XT>(Frag, slice m), bit for bit.
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

// Paired launches: two matrices of one shape and one activation as a single
// launch of 2 x rows rows, rows 2i and 2i + 1 being row i of the first
// matrix (w) and of the second (w_up), so each two-row tile holds both
// matrices' row i.  kPairOut writes both results (y, y_up); kPairGlu, the
// gate and up projections of a SwiGLU FFN, writes h = silu(gate . x) *
// (up . x) to y in their place.
constexpr int kPairNone = 0, kPairOut = 1, kPairGlu = 2;

// A tile of a paired launch: rows 2i and 2i + 1 are row i of the first
// matrix (pol) and of the second (pol_up); row0 is even.
template <class P, int R, int PM>
__device__ __forceinline__ void load_tile_of(const P& pol, const P& pol_up, typename P::Frag* f, int row0,
                                             int r_last) {
  if constexpr (PM != kPairNone) {
    const int i = min(row0, r_last) >> 1;
    pol.load(i, f[0]);
    pol_up.load(i, f[1]);
  } else {
    load_tile<P, R>(pol, f, row0, r_last);
  }
}

// silu(g) = g / (1 + e^-g), the gate nonlinearity of a SwiGLU FFN, as
// g * rcp(1 + 2^(-g log2 e)) with the hardware exp2 and reciprocal (each
// about 1 ulp; six instructions per tile against about 25 for expf and an
// IEEE division, on a path bound by VALU issue).  The rounded product
// -g log2 e adds about |g| 2^-24 relative error to e^-g, which reaches h only
// in proportion e^-g / (1 + e^-g): where g is very negative and silu(g) is
// already tiny.  Below about -88, e^-g overflows to +inf and the result is
// -0, the limit.
__device__ __forceinline__ float silu(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * 1.44269504088896341f));
}

// Reduce a tile and store its rows: to y when this wave covers all of K, else
// this wave's K-slice sums to its LDS column `part` (indexed by row - r_begin).
template <class P, typename XT, int R, int PM = kPairNone>
__device__ __forceinline__ void finish_tile(const P& pol, const typename P::Frag* f,
                                            const typename P::template XSliceT<XT>& xs, float* y, int row0,
                                            int r_begin, int r_end, int kw, int lane, float* part,
                                            float* y_up = nullptr) {
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = pol.template dot<XT>(f[r], xs);
  const float t = reduce_rows<R>(acc, lane);
  // paired launches: even lanes hold the first matrix's row total, odd lanes
  // the second's
  if constexpr (PM == kPairGlu) {
    // lane 0 takes lane 1's and writes h[i] = silu(g) * u for the pair's row i
    const float u = dpp<0xB1>(t);  // quad_perm [1,0,3,2]
    if (lane == 0 && row0 < r_end) y[row0 >> 1] = silu(t) * u;
    return;
  }
  if constexpr (PM == kPairOut) {
    if (lane < 2 && row0 < r_end) (lane ? y_up : y)[row0 >> 1] = t;
    return;
  }
  if (lane < R && row0 + lane < r_end) {
    // The LDS write is a relaxed atomic store (a plain ds_write) so that the
    // compiler cannot merge the two stores into one generic-pointer store:
    // a flat store counts against both wait counters, and the wait-count
    // pass would then drain the weight prefetch at every tile.
    if (kw == 1)
      y[row0 + lane] = t;
    else
      __hip_atomic_store(part + (row0 - r_begin + lane), t, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_WORKGROUP);
  }
}

// One matrix of a launch, as laid out by plan_gemv (host).
struct GemvItem {
  const uint8_t* w;
  const uint8_t* w_up;  // paired launches: the second matrix
  uint64_t scales_offset;
  const void* x;      // [batch][cols]
  float* y;           // [batch][rows]; paired: [batch][rows / 2] (kPairGlu: h)
  float* y_up;        // kPairOut: the second matrix's [batch][rows / 2]
  int rows, cols;
  int kw;             // waves along K
  int sets_per_wg;    // row sets per workgroup (kw waves each)
  int nsets, q, rem;  // set s has q + R (s < rem) or q rows, the last one clamped to rows
  int wg_begin;       // first workgroup of this matrix
};

struct GemvLaunch {
  int n;
  int part_stride;    // LDS floats per wave for K-split partial sums (>= rows of a set)
  GemvItem item[kMaxItems];
};

// The body of gemv_kernel, gemv_pair_kernel and gemv_glu_kernel (PM: the
// paired modes above, only with SX and R = 2: every row within one wave's K
// slice).
template <class P, typename XT, int R, int D, int MAXT, bool SX, int PM>
__device__ __forceinline__ void gemv_body(const GemvLaunch& args) {
  static_assert(PM == kPairNone || (SX && R == 2), "paired tiles are two rows within one wave's K slice");
  // This workgroup's matrix (wave-uniform scan over at most kMaxItems).
  int it = 0;
#pragma unroll 1
  for (int k = 1; k < args.n; ++k)
    if (static_cast<int>(blockIdx.x) >= args.item[k].wg_begin) it = k;
  const GemvItem& m = args.item[it];

  const int lane = __lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kw = SX ? 1 : m.kw;
  if (!SX && wave >= kw * m.sets_per_wg) return;  // spare waves of a kw > 1 workgroup
  const int kslot = wave % kw;
  const int set = (blockIdx.x - m.wg_begin) * m.sets_per_wg + wave / kw;
  // Only with kw == 1, where no barrier is shared.  The SX kernels keep such
  // waves to the x copy and give them no rows.
  if (!SX && set >= m.nsets) return;
  const XT* x = static_cast<const XT*>(m.x) + static_cast<size_t>(blockIdx.y) * m.cols;
  float* y = m.y + static_cast<size_t>(blockIdx.y) * (PM != kPairNone ? m.rows / 2 : m.rows);
  float* y_up = PM == kPairOut ? m.y_up + static_cast<size_t>(blockIdx.y) * (m.rows / 2) : nullptr;
  int r_begin = set * m.q + R * min(set, m.rem);
  int r_end = min(r_begin + m.q + (set < m.rem ? R : 0), m.rows);
  if (SX && set >= m.nsets) r_begin = r_end = m.rows;  // tile loads clamp to the last row
  const int r_last = r_end - 1;

  // K-split partial sums: one column of part_stride floats per wave; in the
  // SX kernels, the workgroup's copy of x.
  extern __shared__ float part_lds[];
  float* part = part_lds + wave * args.part_stride;
  const P pol(m.w, m.scales_offset, m.cols, kslot, lane);
  const P pol_up(PM != kPairNone ? m.w_up : m.w, m.scales_offset, m.cols, kslot, lane);  // paired only

  uint4 raw[P::kXElems * sizeof(XT) / 16];
  typename P::Frag f[D][R];
  if constexpr (SX) {
    // Issue order: this thread's x chunks, tile 0, tile 1; the chunks are
    // stored to LDS once they arrive (the tiles stay in flight), then every
    // wave reads its slice.  Chunk indices past the row's end are clamped:
    // those threads re-read and re-store the last chunk.
    constexpr int kChunks = P::kColsPerWave * static_cast<int>(sizeof(XT)) / 16;
    constexpr int kPerThread = (kChunks + MAXT - 1) / MAXT;
    // (A native vector type: copies of uint4, a struct, become memcpy calls
    // that keep the array in scratch memory.)
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const int nchunks = m.cols * static_cast<int>(sizeof(XT)) / 16;
    const u32x4* gx = reinterpret_cast<const u32x4*>(x);
    u32x4 xc[kPerThread];
    int slot[kPerThread];
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const int g = min(static_cast<int>(threadIdx.x) + k * MAXT, nchunks - 1);
      xc[k] = gx[g];
      slot[k] = xshared_slot(g);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < D; ++j) load_tile_of<P, R, PM>(pol, pol_up, f[j], r_begin + j * R, r_last);
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    u32x4* xl = reinterpret_cast<u32x4*>(part_lds);
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) xl[slot[k]] = xc[k];
    lds_barrier();
    pol.load_x_raw(XShared<XT>{reinterpret_cast<const uint4*>(part_lds)}, raw);
  } else {
    // Issue order: x slice, tile 0, tile 1; only then wait for x.
    pol.load_x_raw(XGlobal<XT>{x}, raw);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < D; ++j) load_tile_of<P, R, PM>(pol, pol_up, f[j], r_begin + j * R, r_last);
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  }
  typename P::template XSliceT<XT> xs;
  pol.template finish_x<XT>(raw, xs);

  // Each prefetch is pinned right after the tile whose registers it reuses:
  // left alone, the compiler sinks the loads below the next tile's arithmetic
  // (across the basic blocks of the reduction), which leaves one tile in
  // flight per wave.  An empty asm with a memory clobber keeps the loads in
  // program order without waiting for them (the weight pointer is
  // deliberately not __restrict__: a restrict-qualified read-only pointer
  // lets the compiler move its loads across the clobber), and a scheduling
  // barrier stops the next tile's arithmetic, which touches no memory, from
  // being hoisted above them.
  //
  // The loop has a single exit, at its bottom.  A second exit between the two
  // tiles reaches the loop header in the compiler's wait-count analysis on a
  // path where only one tile was requested, and the merged state makes the
  // first tile of every iteration wait for all outstanding loads, draining
  // the prefetch.  So the loop runs D tiles per iteration while a tile past
  // them exists, and the last at most D tiles are finished after it.
  const int ntiles = (r_end - r_begin + R - 1) / R;
  int r0 = r_begin;
#pragma unroll 1
  for (int t = D; t < ntiles; t += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      finish_tile<P, XT, R, PM>(pol, f[j], xs, y, r0 + j * R, r_begin, r_end, kw, lane, part, y_up);
      load_tile_of<P, R, PM>(pol, pol_up, f[j], r0 + (j + D) * R, r_last);
      __asm__ __volatile__("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    }
    r0 += D * R;
  }
#pragma unroll
  for (int j = 0; j < D; ++j)
    if (r0 + j * R < r_end)
      finish_tile<P, XT, R, PM>(pol, f[j], xs, y, r0 + j * R, r_begin, r_end, kw, lane, part, y_up);

  // K split: after one barrier, the kw waves of the set add the columns of
  // their set in slot order, row by row (waves that left early count as
  // arrived at a barrier).
  if (!SX && kw > 1) {
    __syncthreads();
    const float* cols = part_lds + (wave - kslot) * args.part_stride;
    for (int j = kslot * 64 + lane; j < r_end - r_begin; j += kw * 64) {
      float v = cols[j];
      for (int k = 1; k < kw; ++k) v += cols[k * args.part_stride + j];
      y[r_begin + j] = v;
    }
  }
}

template <class P, typename XT, int R, int D, int MAXT, bool SX>
__global__ void __launch_bounds__(MAXT)
gemv_kernel(const GemvLaunch args) {
  gemv_body<P, XT, R, D, MAXT, SX, kPairNone>(args);
}

// Two matrices of one shape on one activation, paired row by row (kPairOut).
template <class P, typename XT, int MAXT>
__global__ void __launch_bounds__(MAXT)
gemv_pair_kernel(const GemvLaunch args) {
  gemv_body<P, XT, 2, 2, MAXT, true, kPairOut>(args);
}

// The gate/up launch of a SwiGLU FFN (kPairGlu).
template <class P, typename XT, int MAXT>
__global__ void __launch_bounds__(MAXT)
gemv_glu_kernel(const GemvLaunch args) {
  gemv_body<P, XT, 2, 2, MAXT, true, kPairGlu>(args);
}

// Batches of activation rows against matrices within one wave's K slice: the
// work split and tile pipeline of the shared-activation gemv_kernel, but each
// wave carries NBR (2 or 4) activation rows, so W is read once per NBR rows
// instead of once per row.  All waves of a workgroup need the same NBR activation slices
// (every matrix fits one wave's K slice): wave m < NBR reads row m from global
// memory, converts it and leaves each lane's slice in LDS (word k of lane l at
// [m][k][l]); after a barrier every wave reads all NBR slices.
// P::dot_rows<XT, NBR> gives a row tile's NBR partials, sharing the block
// decode, and the R x NBR partials (at most 4) are reduced together.  Grid y
// covers the batch in steps of NBR (rows past the batch re-read the last row
// and are not stored).
template <class P, typename XT, int R, int D, int MAXT, int NBR>
__global__ void __launch_bounds__(MAXT) __attribute__((amdgpu_waves_per_eu(2)))
gemv_rows_kernel(const GemvLaunch args, int batch) {
  static_assert(R * NBR <= 4, "reduce_rows handles at most four partials");
  static_assert(NBR <= MAXT / 64, "one converting wave per activation row");
  typedef typename P::template XSliceT<XT> XS;
  static_assert(sizeof(XS) % 4 == 0, "slices move through LDS as 32-bit words");
  constexpr int kWords = static_cast<int>(sizeof(XS) / 4);
  int it = 0;
#pragma unroll 1
  for (int k = 1; k < args.n; ++k)
    if (static_cast<int>(blockIdx.x) >= args.item[k].wg_begin) it = k;
  const GemvItem& m = args.item[it];

  const int lane = __lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int set = (blockIdx.x - m.wg_begin) * m.sets_per_wg + wave;
  const int mb0 = static_cast<int>(blockIdx.y) * NBR;  // first activation row
  int r_begin = set * m.q + R * min(set, m.rem);
  int r_end = min(r_begin + m.q + (set < m.rem ? R : 0), m.rows);
  if (set >= m.nsets) r_begin = r_end = m.rows;  // slices only; tile loads clamp to the last row
  const int r_last = r_end - 1;

  extern __shared__ float part_lds[];
  uint32_t* slices = reinterpret_cast<uint32_t*>(part_lds);
  const P pol(m.w, m.scales_offset, m.cols, 0, lane);
  typename P::Frag f[D][R];

  // Issue order: the converting wave's x slice, tile 0, tile 1.
  const bool conv = wave < NBR;
  uint4 raw[P::kXElems * sizeof(XT) / 16];
  if (conv) {
    const XT* xr = static_cast<const XT*>(m.x) + static_cast<size_t>(min(mb0 + wave, batch - 1)) * m.cols;
    pol.load_x_raw(XGlobal<XT>{xr}, raw);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < D; ++j) load_tile<P, R>(pol, f[j], r_begin + j * R, r_last);
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  if (conv) {
    XS own;
    pol.template finish_x<XT>(raw, own);
    uint32_t w[kWords];
    __builtin_memcpy(w, &own, sizeof(XS));
#pragma unroll
    for (int k = 0; k < kWords; ++k) slices[(wave * kWords + k) * 64 + lane] = w[k];
  }
  lds_barrier();
  XS xs[NBR];
#pragma unroll
  for (int mi = 0; mi < NBR; ++mi) {
    uint32_t w[kWords];
#pragma unroll
    for (int k = 0; k < kWords; ++k) w[k] = slices[(mi * kWords + k) * 64 + lane];
    __builtin_memcpy(&xs[mi], w, sizeof(XS));
  }

  auto finish = [&](const typename P::Frag* fr, int row0) {
    // three partials (one weight row, three activation rows) are reduced as
    // four, the fourth zero and not stored
    constexpr int kParts = R * NBR == 3 ? 4 : R * NBR;
    float acc[kParts];
    if constexpr (kParts > R * NBR) acc[kParts - 1] = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) pol.template dot_rows<XT, NBR>(fr[r], xs, acc + r * NBR);
    const float t = reduce_rows<kParts>(acc, lane);
    const int r = lane / NBR, mi = lane - (lane / NBR) * NBR;
    if (lane < R * NBR && row0 + r < r_end && mb0 + mi < batch)
      m.y[static_cast<size_t>(mb0 + mi) * m.rows + row0 + r] = t;
  };
  // Single-exit tile loop with pinned prefetches, as in gemv_kernel.
  const int ntiles = (r_end - r_begin + R - 1) / R;
  int r0 = r_begin;
#pragma unroll 1
  for (int t = D; t < ntiles; t += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      finish(f[j], r0 + j * R);
      load_tile<P, R>(pol, f[j], r0 + (j + D) * R, r_last);
      __asm__ __volatile__("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    }
    r0 += D * R;
  }
#pragma unroll
  for (int j = 0; j < D; ++j)
    if (r0 + j * R < r_end) finish(f[j], r0 + j * R);
}

// Two activation rows against matrices split along K (kw > 1 waves per row
// set): gemv_kernel's K-split structure with gemv_rows_kernel's shared block
// decode.  Each wave needs both rows' slices of its own K slot, so it reads
// and converts them itself, one row at a time.  A tile's R x 2 wave totals go
// to the wave's LDS column ([row - r_begin][activation row]); after one
// barrier the kw waves of the set add their columns in slot order, the batch-1
// K split's order, so every output equals the batch-1 GEMV's bit for bit.
// Grid y covers the batch in steps of two (a last odd row re-reads its
// predecessor's neighbour, clamped, and is not stored).
template <class P, typename XT, int R, int D, int MAXT>
__global__ void __launch_bounds__(MAXT) __attribute__((amdgpu_waves_per_eu(2)))
gemv_rows_split_kernel(const GemvLaunch args, int batch) {
  constexpr int NBR = 2;
  static_assert(R * NBR <= 4, "reduce_rows handles at most four partials");
  int it = 0;
#pragma unroll 1
  for (int k = 1; k < args.n; ++k)
    if (static_cast<int>(blockIdx.x) >= args.item[k].wg_begin) it = k;
  const GemvItem& m = args.item[it];

  const int lane = __lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kw = m.kw;
  if (wave >= kw * m.sets_per_wg) return;  // spare waves (they count as arrived at the barrier)
  const int kslot = wave % kw;
  const int set = (blockIdx.x - m.wg_begin) * m.sets_per_wg + wave / kw;
  if (set >= m.nsets) return;  // a whole set absent: all its waves leave together
  const int mb0 = static_cast<int>(blockIdx.y) * NBR;
  const int r_begin = set * m.q + R * min(set, m.rem);
  const int r_end = min(r_begin + m.q + (set < m.rem ? R : 0), m.rows);
  const int r_last = r_end - 1;

  extern __shared__ float part_lds[];
  float* part = part_lds + wave * args.part_stride * NBR;
  const P pol(m.w, m.scales_offset, m.cols, kslot, lane);
  typename P::Frag f[D][R];

  // Issue order: both rows' x slices, tile 0, tile 1; then convert row by row.
  uint4 raw[NBR][P::kXElems * sizeof(XT) / 16];
#pragma unroll
  for (int mi = 0; mi < NBR; ++mi) {
    const XT* xr = static_cast<const XT*>(m.x) + static_cast<size_t>(min(mb0 + mi, batch - 1)) * m.cols;
    pol.load_x_raw(XGlobal<XT>{xr}, raw[mi]);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < D; ++j) load_tile<P, R>(pol, f[j], r_begin + j * R, r_last);
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  typename P::template XSliceT<XT> xs[NBR];
#pragma unroll
  for (int mi = 0; mi < NBR; ++mi) {
    pol.template finish_x<XT>(raw[mi], xs[mi]);
    __builtin_amdgcn_sched_barrier(0);  // one row's conversion temporaries at a time
  }

  auto finish = [&](const typename P::Frag* fr, int row0) {
    float acc[R * NBR];
#pragma unroll
    for (int r = 0; r < R; ++r) pol.template dot_rows<XT, NBR>(fr[r], xs, acc + r * NBR);
    const float t = reduce_rows<R * NBR>(acc, lane);
    // lane q < R x NBR holds partial q = r x NBR + mi of rows row0 + r
    if (lane < R * NBR && row0 + lane / NBR < r_end)
      __hip_atomic_store(part + (row0 - r_begin) * NBR + lane, t, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_WORKGROUP);
  };
  // Single-exit tile loop with pinned prefetches, as in gemv_kernel.
  const int ntiles = (r_end - r_begin + R - 1) / R;
  int r0 = r_begin;
#pragma unroll 1
  for (int t = D; t < ntiles; t += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      finish(f[j], r0 + j * R);
      load_tile<P, R>(pol, f[j], r0 + (j + D) * R, r_last);
      __asm__ __volatile__("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    }
    r0 += D * R;
  }
#pragma unroll
  for (int j = 0; j < D; ++j)
    if (r0 + j * R < r_end) finish(f[j], r0 + j * R);

  // K split: the kw waves of the set add their columns in slot order.
  __syncthreads();
  const float* cols = part_lds + (wave - kslot) * args.part_stride * NBR;
  const int n_out = (r_end - r_begin) * NBR;
  for (int j = kslot * 64 + lane; j < n_out; j += kw * 64) {
    float v = cols[j];
    for (int k = 1; k < kw; ++k) v += cols[k * args.part_stride * NBR + j];
    const int mi = j % NBR;
    if (mb0 + mi < batch) m.y[static_cast<size_t>(mb0 + mi) * m.rows + r_begin + j / NBR] = v;
  }
}

// Matrices split along K (kw > 1 K slots), any batch row by grid y: the
// activation slices in LDS.
//
// In gemv_kernel's K split every wave of a row set holds a private slice of
// x in VGPRs (16 KB of fp32 for Q4_K, read from L2 before its first tile)
// and the set's waves add their partial sums through LDS at the end; with
// one set per compute unit that leaves 1.25 waves per SIMD to hide the
// arithmetic behind the loads.  Here the workgroup first stages every lane
// slice of the row once -- slice (k, l) is exactly what lane l of a wave at
// K slot k multiplies, converted (fp32: scaled, with its sub-block sums) by
// the policy's finish_x, and stored as 16-byte words at [k][word][lane] so
// that a wave's reads are consecutive -- and then each wave streams whole
// rows, R at a time, K slot after K slot, reading each slot's slice from LDS
// into VGPRs for the tile.  The R partials of a tile are reduced across the
// wave as in gemv_kernel, and the slot totals are added in slot order (lane
// r < R keeps row r's running total), which are the K-split gemv_kernel's
// operations in its order: outputs are equal bit for bit.  Rows are dealt to
// the launch's waves in contiguous groups of R.
struct GemvLxArgs {
  const uint8_t* w;
  uint64_t scales_offset;
  const void* x;      // [batch][cols]
  float* y;           // [batch][rows]
  int rows, cols;
  int nslots;         // K slots (waves' worth of columns) per row
  int groups;         // row groups of R rows
};

template <class P, typename XT>
constexpr int lx_slice_words() {  // 16-byte words of one lane slice
  return static_cast<int>((sizeof(typename P::template XSliceT<XT>) + 15) / 16);
}

template <class P, typename XT, int R, int D, int MAXT>
__global__ void __launch_bounds__(MAXT)
gemv_lx_kernel(const GemvLxArgs a) {
  typedef typename P::template XSliceT<XT> XS;
  constexpr int kW4 = lx_slice_words<P, XT>();
  const int lane = __lane_id();
  const int waves = static_cast<int>(blockDim.x) >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = static_cast<int>(gridDim.x) * waves;
  const int gw = static_cast<int>(blockIdx.x) * waves + wave;
  // this wave's row groups [g0, g1)
  const int g0 = static_cast<int>(static_cast<int64_t>(gw) * a.groups / nw);
  const int g1 = static_cast<int>(static_cast<int64_t>(gw + 1) * a.groups / nw);
  const int ntiles = (g1 - g0) * a.nslots;
  const int r_last = a.rows - 1;
  const XT* x = static_cast<const XT*>(a.x) + static_cast<size_t>(blockIdx.y) * a.cols;
  float* y = a.y + static_cast<size_t>(blockIdx.y) * a.rows;
  extern __shared__ uint4 lx_slices[];

  // Tile t of this wave: row group g0 + t / nslots, K slot t % nslots;
  // tracked incrementally for the tile being loaded and the one finished.
  // Prefetches past the wave's own tiles re-read the matrix's last row,
  // which every wave shares (L2 hits), rather than rows of the next wave.
  int ld_g = g0, ld_k = 0;
  auto load_next = [&](typename P::Frag* f) {
    const P pol(a.w, a.scales_offset, a.cols, ld_k, lane);
    const int rb = ld_g < g1 ? ld_g * R : r_last;
#pragma unroll
    for (int r = 0; r < R; ++r) pol.load(min(rb + r, r_last), f[r]);
    if (++ld_k == a.nslots) {
      ld_k = 0;
      ++ld_g;
    }
  };

  // Issue order: the activations of the slice this thread stages (threads
  // nslots x 64 and above re-read the last slice and store nothing; the
  // launch gives a workgroup at least nslots waves), then the first D tiles;
  // the slice is converted and stored once its loads arrive.
  const int sidx = min(static_cast<int>(threadIdx.x), a.nslots * 64 - 1);
  const P pk(a.w, a.scales_offset, a.cols, sidx >> 6, sidx & 63);
  uint4 raw[P::kXElems * sizeof(XT) / 16];
  pk.load_x_raw(XGlobal<XT>{x}, raw);
  __builtin_amdgcn_sched_barrier(0);
  typename P::Frag f[D][R];
#pragma unroll
  for (int j = 0; j < D; ++j) load_next(f[j]);
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  {
    XS sl;
    pk.template finish_x<XT>(raw, sl);
    uint4 wds[kW4];
    wds[kW4 - 1] = make_uint4(0, 0, 0, 0);
    __builtin_memcpy(wds, &sl, sizeof(XS));
    if (static_cast<int>(threadIdx.x) < a.nslots * 64) {
#pragma unroll
      for (int i = 0; i < kW4; ++i) lx_slices[((sidx >> 6) * kW4 + i) * 64 + (sidx & 63)] = wds[i];
    }
  }
  lds_barrier();

  const P pol(a.w, a.scales_offset, a.cols, 0, lane);  // dot() uses lane constants only
  int fin_g = g0, fin_k = 0;
  float tot = 0.f;  // lane r < R: running total of row fin_g * R + r over the slots so far
  auto finish = [&](const typename P::Frag* fr) {
    uint4 wds[kW4];
#pragma unroll
    for (int i = 0; i < kW4; ++i) wds[i] = lx_slices[(fin_k * kW4 + i) * 64 + lane];
    XS xs;
    __builtin_memcpy(&xs, wds, sizeof(XS));
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = pol.template dot<XT>(fr[r], xs);
    const float t = reduce_rows<R>(acc, lane);
    tot = fin_k == 0 ? t : tot + t;
    if (++fin_k == a.nslots) {
      const int row = fin_g * R + lane;
      if (lane < R && row < a.rows) y[row] = tot;
      fin_k = 0;
      ++fin_g;
    }
  };
  // Single-exit tile loop with pinned prefetches, as in gemv_kernel.
  int t = D;
#pragma unroll 1
  for (; t < ntiles; t += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      finish(f[j]);
      load_next(f[j]);
      __asm__ __volatile__("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int j = 0; j < D; ++j)
    if (t - D + j < ntiles) finish(f[j]);
}

// Rows of a K-split set are capped so that the partial sums of a workgroup
// (waves x rows floats) stay within 16 waves x kMaxPartStride x 4 bytes.
constexpr int kMaxPartStride = 256;

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
// every matrix, a whole number of R-row tiles, chosen so that the launch
// holds about `target_waves` waves.
template <class P, int R>
inline int plan_gemv(const GemvCall* calls, int n, int waves, int64_t target_waves,
                     GemvLaunch* L) {
  int64_t wave_rows = 0;  // sum over matrices of rows * kw
  for (int i = 0; i < n; ++i)
    wave_rows += calls[i].W->rows *
                 ((calls[i].W->cols + P::kColsPerWave - 1) / P::kColsPerWave);
  int64_t rps = (wave_rows + target_waves - 1) / target_waves;
  rps = (rps + R - 1) / R * R;  // a wave's tile count is ceil(rows / R) either way
  if (rps < R) rps = R;
  int wg = 0;
  L->n = n;
  L->part_stride = 0;
  for (int i = 0; i < n; ++i) {
    GemvItem& m = L->item[i];
    const qmv_weights* W = calls[i].W;
    m.w = static_cast<const uint8_t*>(W->data);
    m.w_up = nullptr;
    m.y_up = nullptr;
    m.scales_offset = W->scales_offset;
    m.x = calls[i].x;
    m.y = calls[i].y;
    m.rows = static_cast<int>(W->rows);
    m.cols = static_cast<int>(W->cols);
    m.kw = static_cast<int>((W->cols + P::kColsPerWave - 1) / P::kColsPerWave);
    m.sets_per_wg = waves / m.kw;
    int64_t set_rows = rps;
    if (m.kw > 1 && set_rows > kMaxPartStride) set_rows = kMaxPartStride;  // LDS of the partials
    const int units = (m.rows + R - 1) / R;  // tiles of R rows
    m.nsets = static_cast<int>((units + set_rows / R - 1) / (set_rows / R));
    m.q = (units / m.nsets) * R;
    m.rem = units % m.nsets;
    if (m.kw > 1) {
      const int need = m.q + (m.rem ? R : 0);
      L->part_stride = need > L->part_stride ? need : L->part_stride;
    }
    m.wg_begin = wg;
    wg += (m.nsets + m.sets_per_wg - 1) / m.sets_per_wg;
  }
  return wg;
}

// Launch shape.  Waves stream their rows with two tiles in flight; the HBM
// queue holds all of them, so a request waits about (bytes in flight) /
// bandwidth.  Enough waves keep the memory busy and the SIMDs fed, but every
// extra byte in flight lengthens the ramp-up before the first tiles arrive
// and the tail after the last: measured on gfx950, two waves per SIMD at
// most, at least one per SIMD, and at least kMinRowsPerWave rows per wave
// (short-lived waves pay the activation load and the first-tile latency for
// little work).
#ifndef QMV_WAVES_PER_SIMD
#define QMV_WAVES_PER_SIMD 2
#endif
#ifndef QMV_MIN_ROWS_PER_WAVE
#define QMV_MIN_ROWS_PER_WAVE 8
#endif
constexpr int kMaxWavesPerSimd = QMV_WAVES_PER_SIMD;
constexpr int kMinRowsPerWave = QMV_MIN_ROWS_PER_WAVE;
// Launches long enough to give every wave at least this many rows at two
// waves per SIMD run three: the ramp-up that more bytes in flight costs is
// then small against the whole (measured on the 152064-row lm-head: 72.1-72.4
// us against 73.2-73.3 us; on the 7B layer's launches, all far below, three
// waves per SIMD was slower).
constexpr int kLongRowsPerWave = 48;

// LDS of the shared-activation kernels: the x copy of the launch's longest
// row, in 16-byte chunks rounded up to a multiple of 16 (xshared_slot).
template <typename XT>
inline size_t sx_lds_bytes(const GemvCall* calls, int n) {
  int64_t cols = 0;
  for (int i = 0; i < n; ++i) cols = calls[i].W->cols > cols ? calls[i].W->cols : cols;
  const int64_t chunks = (cols * static_cast<int64_t>(sizeof(XT)) / 16 + 15) / 16 * 16;
  return static_cast<size_t>(chunks) * 16;
}

template <class P, typename XT, int R, int D, int MAXT, bool SX, int PM = kPairNone>
hipError_t launch_cfg(const GemvCall* calls, int n, int waves, int64_t batch, hipStream_t stream,
                      int waves_per_simd, const void* w_up = nullptr, float* y_up = nullptr) {
  const auto kernel = [] {
    if constexpr (PM == kPairGlu)
      return gemv_glu_kernel<P, XT, MAXT>;
    else if constexpr (PM == kPairOut)
      return gemv_pair_kernel<P, XT, MAXT>;
    else
      return gemv_kernel<P, XT, R, D, MAXT, SX>;
  }();
  const int block = 64 * waves;
  if (SX && block != MAXT) return hipErrorInvalidValue;  // the x copy assumes MAXT threads
  const int cus = device_cus();
  int64_t wave_rows = 0;
  for (int i = 0; i < n; ++i)
    wave_rows += calls[i].W->rows * ((calls[i].W->cols + P::kColsPerWave - 1) / P::kColsPerWave);
  // dynamic LDS: the x copy (SX), else at most kMaxPartStride partial sums per wave
  size_t lds_max = static_cast<size_t>(waves) * kMaxPartStride * sizeof(float);
  if (SX) lds_max = sx_lds_bytes<XT>(calls, n);
  const int64_t resident = resident_workgroups(kernel, block, lds_max) * waves;
  if (waves_per_simd == 2 && wave_rows >= static_cast<int64_t>(cus) * 4 * 2 * kLongRowsPerWave)
    waves_per_simd = 3;
  int64_t target = wave_rows / kMinRowsPerWave;
  if (target > static_cast<int64_t>(cus) * 4 * waves_per_simd)
    target = static_cast<int64_t>(cus) * 4 * waves_per_simd;
  if (target < static_cast<int64_t>(cus) * 4) target = static_cast<int64_t>(cus) * 4;
  // whole workgroups per CU, so that no CU carries an extra one
  int64_t per_cu = target / (static_cast<int64_t>(cus) * waves);
  if (per_cu < 1) per_cu = 1;
  target = per_cu * cus * waves;
  if (target > resident) target = resident;
  GemvLaunch L;
  const int grid = plan_gemv<P, R>(calls, n, waves, target, &L);
  if (PM != kPairNone) {
    L.item[0].w_up = static_cast<const uint8_t*>(w_up);
    L.item[0].y_up = y_up;
  }
  size_t lds = static_cast<size_t>(waves) * L.part_stride * sizeof(float);
  if (SX) lds = sx_lds_bytes<XT>(calls, n);
  hipLaunchKernelGGL(kernel, dim3(grid, static_cast<unsigned>(batch)), dim3(block), lds, stream,
                     L);
  return hipGetLastError();
}

// Tiles in flight per wave of gemv_rows_kernel: two with two activation rows
// (R = 2), three with three or four (R = 1).  (Measured on the 18944 x 3584
// FFN shape: deeper pipelines were slower at both sizes, two tiles of four
// rows 0.3 us slower.)
template <int NBR>
constexpr int rows_tiles_in_flight() { return NBR >= 3 ? 3 : 2; }

// Launch of gemv_rows_kernel: every matrix within one wave's K slice, NBR
// activation rows per wave (R rows per tile, R x NBR <= 4), four-wave
// workgroups, the launch shape of the shared-activation GEMV.
template <class P, typename XT, int R, int NBR>
hipError_t launch_rows(const GemvCall* calls, int n, int64_t batch, hipStream_t stream) {
  constexpr int kWaves = 4;
  auto kernel = gemv_rows_kernel<P, XT, R, rows_tiles_in_flight<NBR>(), 64 * kWaves, NBR>;
  const int cus = device_cus();
  int64_t wave_rows = 0;
  for (int i = 0; i < n; ++i) {
    if (calls[i].W->cols > P::kColsPerWave) return hipErrorInvalidValue;
    wave_rows += calls[i].W->rows;
  }
  const size_t lds = static_cast<size_t>(NBR) * sizeof(typename P::template XSliceT<XT>) * 64;
  const int64_t resident = resident_workgroups(kernel, 64 * kWaves, lds) * kWaves;
  int64_t target = wave_rows / kMinRowsPerWave;
  if (target > static_cast<int64_t>(cus) * 4 * kMaxWavesPerSimd) target = static_cast<int64_t>(cus) * 4 * kMaxWavesPerSimd;
  if (target < static_cast<int64_t>(cus) * 4) target = static_cast<int64_t>(cus) * 4;
  int64_t per_cu = target / (static_cast<int64_t>(cus) * kWaves);
  if (per_cu < 1) per_cu = 1;
  target = per_cu * cus * kWaves;
  if (target > resident) target = resident;
  GemvLaunch L;
  const int grid = plan_gemv<P, R>(calls, n, kWaves, target, &L);
  hipLaunchKernelGGL(kernel, dim3(grid, static_cast<unsigned>((batch + NBR - 1) / NBR)),
                     dim3(64 * kWaves), lds, stream, L, static_cast<int>(batch));
  return hipGetLastError();
}

// Launch of gemv_rows_split_kernel: matrices of two to eight waves along K,
// max(4, widest K split) waves per workgroup, the launch shape of the K-split
// GEMV.
template <class P, typename XT, int MAXT>
hipError_t launch_rows_split(const GemvCall* calls, int n, int64_t batch, hipStream_t stream) {
  // Two weight rows per tile; one where a row's fragment is above 64 bytes
  // (Q5_K), which would not fit two waves per SIMD without spilling.
  constexpr int R = sizeof(typename P::Frag) > 64 ? 1 : 2;
  auto kernel = gemv_rows_split_kernel<P, XT, R, 2, MAXT>;
  const int kw = max_kw<P>(calls, n);
  const int waves = kw < 4 ? 4 : kw;
  if (64 * waves > MAXT) return hipErrorInvalidValue;
  const int cus = device_cus();
  int64_t wave_rows = 0;
  for (int i = 0; i < n; ++i)
    wave_rows += calls[i].W->rows * ((calls[i].W->cols + P::kColsPerWave - 1) / P::kColsPerWave);
  const int64_t resident =
      resident_workgroups(kernel, 64 * waves, static_cast<size_t>(waves) * kMaxPartStride * 2 * sizeof(float)) * waves;
  int64_t target = wave_rows / kMinRowsPerWave;
  if (target > static_cast<int64_t>(cus) * 4 * kMaxWavesPerSimd) target = static_cast<int64_t>(cus) * 4 * kMaxWavesPerSimd;
  if (target < static_cast<int64_t>(cus) * 4) target = static_cast<int64_t>(cus) * 4;
  int64_t per_cu = target / (static_cast<int64_t>(cus) * waves);
  if (per_cu < 1) per_cu = 1;
  target = per_cu * cus * waves;
  if (target > resident) target = resident;
  GemvLaunch L;
  const int grid = plan_gemv<P, R>(calls, n, waves, target, &L);
  const size_t lds = static_cast<size_t>(waves) * L.part_stride * 2 * sizeof(float);
  hipLaunchKernelGGL(kernel, dim3(grid, static_cast<unsigned>((batch + 1) / 2)), dim3(64 * waves), lds,
                     stream, L, static_cast<int>(batch));
  return hipGetLastError();
}

// Two or more fp16 or bf16 activation rows against matrices split along K
// (two to eight waves): one pass over W per two rows.
template <class P>
hipError_t launch_gemv_rows_split(const GemvCall* calls, int n, int x_dtype, int64_t batch,
                                  hipStream_t stream) {
  // (fp32: two rows' raw activations and slices do not fit beside the tiles)
  if (batch < 2 || x_dtype == QMV_F32) return hipErrorInvalidValue;
  const int kw = max_kw<P>(calls, n);
  if (kw < 2 || kw > 8) return hipErrorInvalidValue;
  switch (x_dtype) {
    case QMV_F16:
      return kw <= 4 ? launch_rows_split<P, _Float16, 256>(calls, n, batch, stream)
                     : launch_rows_split<P, _Float16, 512>(calls, n, batch, stream);
    case QMV_BF16:
      return kw <= 4 ? launch_rows_split<P, bf16_t, 256>(calls, n, batch, stream)
                     : launch_rows_split<P, bf16_t, 512>(calls, n, batch, stream);
    default: return hipErrorInvalidValue;
  }
}

// Batches of two or more activation rows.  Against matrices no wider than one
// wave's K slice: fp16 and bf16 two or three rows in one pass over W,
// otherwise groups of four rows, one pass per group; fp32 (66-word slices)
// groups of two rows.
// Against matrices split along K (two to eight waves, every matrix of the
// launch), fp16 and bf16 only: one pass per two rows.
template <class P>
hipError_t launch_gemv_rows(const GemvCall* calls, int n, int x_dtype, int64_t batch,
                            hipStream_t stream) {
  if (batch < 2) return hipErrorInvalidValue;
  if (max_kw<P>(calls, n) > 1) return launch_gemv_rows_split<P>(calls, n, x_dtype, batch, stream);
  switch (x_dtype) {
    case QMV_F32:  // 66-word slices: two rows per pass
      return launch_rows<P, float, 2, 2>(calls, n, batch, stream);
    case QMV_F16:
      return batch == 2   ? launch_rows<P, _Float16, 2, 2>(calls, n, batch, stream)
             : batch == 3 ? launch_rows<P, _Float16, 1, 3>(calls, n, batch, stream)
                          : launch_rows<P, _Float16, 1, 4>(calls, n, batch, stream);
    case QMV_BF16:
      return batch == 2   ? launch_rows<P, bf16_t, 2, 2>(calls, n, batch, stream)
             : batch == 3 ? launch_rows<P, bf16_t, 1, 3>(calls, n, batch, stream)
                          : launch_rows<P, bf16_t, 1, 4>(calls, n, batch, stream);
    default: return hipErrorInvalidValue;
  }
}

// K slots whose slices gemv_lx_kernel stages (LDS bytes per workgroup:
// slots x slice words x 1 KB; fp32 Q4_K slices are 17 words).
constexpr int kLxMaxSlots = 8;
// Rows per group of gemv_lx_kernel.
#ifndef QMV_LX_ROWS
#define QMV_LX_ROWS 2
#endif
// Waves per workgroup (one workgroup per compute unit) at most.
#ifndef QMV_LX_MAX_WAVES
#define QMV_LX_MAX_WAVES 8
#endif

template <class P, typename XT>
inline size_t lx_lds_bytes(int nslots) {
  return static_cast<size_t>(nslots) * lx_slice_words<P, XT>() * 64 * 16;
}

// One matrix split along K (2..kLxMaxSlots slots): gemv_lx_kernel with one
// workgroup per compute unit and enough waves that each takes about one row
// group (at least 4, at most QMV_LX_MAX_WAVES waves per workgroup).
#ifndef QMV_LX_TILES
#define QMV_LX_TILES 2
#endif

template <class P, typename XT>
hipError_t launch_lx(const GemvCall& c, int64_t batch, hipStream_t stream) {
  constexpr int R = QMV_LX_ROWS;
  constexpr int D = QMV_LX_TILES;
  constexpr int kMaxT = 64 * QMV_LX_MAX_WAVES;
  auto kernel = gemv_lx_kernel<P, XT, R, D, kMaxT>;
  const qmv_weights* W = c.W;
  GemvLxArgs a;
  a.w = static_cast<const uint8_t*>(W->data);
  a.scales_offset = W->scales_offset;
  a.x = c.x;
  a.y = c.y;
  a.rows = static_cast<int>(W->rows);
  a.cols = static_cast<int>(W->cols);
  a.nslots = static_cast<int>((W->cols + P::kColsPerWave - 1) / P::kColsPerWave);
  a.groups = static_cast<int>((W->rows + R - 1) / R);
  if (a.nslots > kLxMaxSlots) return hipErrorInvalidValue;
  const int cus = device_cus();
  int waves = (a.groups + cus - 1) / cus;
  waves = waves < 4 ? 4 : (waves > QMV_LX_MAX_WAVES ? QMV_LX_MAX_WAVES : waves);
  if (waves < a.nslots) waves = a.nslots;  // one staging thread per lane slice
  int grid = (a.groups + waves - 1) / waves;
  grid = grid > cus ? cus : grid;
  const size_t lds = lx_lds_bytes<P, XT>(a.nslots);
  hipLaunchKernelGGL(kernel, dim3(grid, static_cast<unsigned>(batch)), dim3(64 * waves), lds, stream, a);
  return hipGetLastError();
}

// Rows per tile and tiles in flight of the shared-activation GEMV: two of
// two rows, unless the format's policy names its own (P::kSxRows,
// P::kSxTiles).  Measured on the 7B shapes: two-row tiles are best for the
// K-quants (one-row tiles with three in flight: Q4_K gate+up 15.6 against
// 15.2 us), one-row tiles with three in flight for INT4 (gate+up 14.0
// against 14.4 us).
template <class P, class = void>
struct SxShape {
  static constexpr int kRows = 2, kTiles = 2;
};
template <class P>
struct SxShape<P, decltype(void(P::kSxRows))> {
  static constexpr int kRows = P::kSxRows, kTiles = P::kSxTiles;
};

template <class P, typename XT>
hipError_t launch_gemv_typed(const GemvCall* calls, int n, int64_t batch, hipStream_t stream) {
  const int kw = max_kw<P>(calls, n);
  if (kw > 16) return hipErrorInvalidValue;
  // A single matrix split along K: the activation slices in LDS.
  if (n == 1 && kw > 1 && kw <= kLxMaxSlots) return launch_lx<P, XT>(calls[0], batch, stream);
  const int waves = kw < 4 ? 4 : kw;
  // Two tiles in flight per wave, two waves per SIMD.  (Measured alternatives
  // on the 7B layer shapes: one wave per SIMD with 3, 4, 6 or 8 tiles in
  // flight, or two waves with 4, were no faster in total; the younger wave of
  // a SIMD trails the older one under the oldest-first issue order, but a
  // deeper single wave loses more on the small matrices and at steady state.)
  if (kw == 1)
    return launch_cfg<P, XT, SxShape<P>::kRows, SxShape<P>::kTiles, 256, true>(calls, n, waves, batch, stream,
                                                                              kMaxWavesPerSimd);
  if (waves <= 4) return launch_cfg<P, XT, 2, 2, 256, false>(calls, n, waves, batch, stream, kMaxWavesPerSimd);
  if (waves <= 8) return launch_cfg<P, XT, 2, 2, 512, false>(calls, n, waves, batch, stream, kMaxWavesPerSimd);
  return launch_cfg<P, XT, 1, 2, 1024, false>(calls, n, waves, batch, stream, kMaxWavesPerSimd);
}

// A paired launch: `a` describes the first matrix with twice its rows (rows
// 2i, 2i + 1 = row i of the first and of the second matrix) and a.y its
// output (glu: h); `b_w` is the second matrix's data, of the same format,
// layout and shape, and `b_y` its output (kPairOut only).  Every row within
// one wave's K slice (checked by the caller).
template <class P, int PM>
hipError_t launch_gemv_pair_mode(const GemvCall& a, const void* b_w, float* b_y, int x_dtype, int64_t batch,
                                 hipStream_t stream) {
  if (max_kw<P>(&a, 1) != 1 || (a.W->rows & 1)) return hipErrorInvalidValue;
  switch (x_dtype) {
    case QMV_F32:
      return launch_cfg<P, float, 2, 2, 256, true, PM>(&a, 1, 4, batch, stream, kMaxWavesPerSimd, b_w, b_y);
    case QMV_F16:
      return launch_cfg<P, _Float16, 2, 2, 256, true, PM>(&a, 1, 4, batch, stream, kMaxWavesPerSimd, b_w, b_y);
    case QMV_BF16:
      return launch_cfg<P, bf16_t, 2, 2, 256, true, PM>(&a, 1, 4, batch, stream, kMaxWavesPerSimd, b_w, b_y);
    default: return hipErrorInvalidValue;
  }
}

template <class P>
hipError_t launch_gemv_pair(const GemvCall& a, const void* b_w, float* b_y, int x_dtype, int64_t batch,
                            bool glu, hipStream_t stream) {
  return glu ? launch_gemv_pair_mode<P, kPairGlu>(a, b_w, nullptr, x_dtype, batch, stream)
             : launch_gemv_pair_mode<P, kPairOut>(a, b_w, b_y, x_dtype, batch, stream);
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
