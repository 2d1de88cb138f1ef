// Batched Q4_K on the gfx950 matrix cores, dequantized tiles: Y[m][n] =
// sum_k X[m][k] W[n][k] for a few hundred activation rows X (bf16 or fp16)
// and Q4_K weights W (canonical or plane layout), y layout [batch][rows].
//
// The batched-prefill reading of the pages' kernel families (hipEngine
// "Quickstart": WMMA prefill beside GEMV decode; the dequantize-to-tile
// scheme of the bulk-prefill passage): once a weight is met by a few hundred
// activation rows, converting it to the matrix-core type once per tile costs
// less than applying its scales to every product.  The factored kernels of
// gemm_q4_k_mfma.hip keep the codes exact and spend four VALU FMAs per
// matrix-core product on the sub-block scale (as many issue cycles as the
// product); here each workgroup dequantizes its weight tile once into LDS
// as fp16, converts its activation tile to fp16, and every product
// accumulates straight into the result.
//
// Tile: 256 weight rows x 128 batch rows per workgroup (512 threads), K in
// steps of 64 columns (two sub-blocks).  Two LDS buffers: step k + 1 is
// dequantized and stored while step k is multiplied, one barrier per step.
// Weight and activation loads run four steps ahead of their use.  Waves are
// 4 (weight rows) x 2 (batch rows) with 64 x 64 outputs each: 4 x 4
// v_mfma_f32_16x16x32_f16 tiles, A = weights, B = activations; accumulator
// r of lane l is the output (weight row 4 (l / 16) + r, batch row l % 16) of
// its tile.
//
// Weights: w = d sc_s u - dmin m_s, evaluated per element as
// fma(u, fp16(d sc_s), -fp16(dmin m_s)) in packed fp16.  The codes enter as
// fp16(1024 + u) (one AND-OR per two codes) and lose the 1024 exactly in a
// packed add.  Each weight carries about one and a half fp16 roundings
// (relative error near 2^-11) against its fp32 value.
// Activations, bf16: each batch row is scaled by a power of two 2^-e, e set
// from the largest |x| of the row seen so far along K (raised at most once
// per Q4_K block, from that block's maximum), so the fp16 copy is exact from
// that maximum down to 2^-38 of it.  When a block raises e, the row's
// accumulators are first multiplied by the exact power of two
// 2^(e_old - e_new); the results are multiplied by 2^e at the end.  fp16
// activations enter as given.
//
// K order within a sub-block: operand slot 8 g + i holds element
// 8 g + (0, 2, 1, 3, 4, 6, 5, 7)[i] on both sides (the order in which masking
// a dword of code bytes yields fp16 pairs).
//
// LDS, per buffer: weights [256 rows][2 sub-blocks x 4 g] then activations
// [128 rows][2 x 4 g] in 16-byte units, the 8 units of a row permuted so that
// the operand reads and the staging stores are free of bank conflicts.
#include <type_traits>

#include "device_util.h"
#include "launch.h"

namespace qmv {

namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

constexpr int kDqThreads = 512;
constexpr int kDqRows = static_cast<int>(kDqTileRows);    // weight rows per workgroup
constexpr int kDqBatch = static_cast<int>(kDqTileBatch);  // batch rows per workgroup
constexpr int kDqBufUnits = 2 * kDqRows * 4 + 2 * kDqBatch * 4;
constexpr size_t kDqLdsBytes = 2 * static_cast<size_t>(kDqBufUnits) * 16 + 3 * kDqBatch * sizeof(float);

// 16-byte unit (sub-block kc, 8-column group g) of a row: rows of 128 bytes,
// the eight units of a row permuted by h(row) = bits (0, 2, 1) of row & 7.
// Every access of a wave touches eight rows at one (kc, g) (operand reads),
// or four rows at two units each, or two rows at four (staging stores); in
// each case any eight lanes in a row of the wave land on eight different
// 16-byte bank groups of a 128-byte bank line.
__device__ __forceinline__ int dq_unit(int kc, int row, int g) {
  const int h = (row & 1) | ((row & 2) << 1) | ((row & 4) >> 1);
  return row * 8 + ((kc * 4 + g) ^ h);
}

__device__ __forceinline__ float byte_f32(uint32_t v, int j) {
  return static_cast<float>((v >> (8 * j)) & 0xFFu);
}

// fp16 pair (lo, hi) of two fp32 values, rounded to nearest even.
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  const h2_t v = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// Largest of the sign-cleared bf16 bit patterns of two packed values.
__device__ __forceinline__ u16x2_t abs_max_bf16(u16x2_t m, uint32_t v) {
  return __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, v & 0x7FFF7FFFu));
}

}  // namespace

template <bool PL, bool F16X>
__global__ void __launch_bounds__(kDqThreads)
gemm_q4_k_dqtile(const uint8_t* w, uint64_t pa, int N, int K, const uint16_t* x, float* y, int M) {
  extern __shared__ __attribute__((aligned(16))) uint4 dq_lds[];
  float* ratio_lds = reinterpret_cast<float*>(dq_lds + 2 * kDqBufUnits);  // [block parity][128 rows]
  float* fin_lds = ratio_lds + 2 * kDqBatch;                               // [128 rows]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 3, wm = wave >> 2;
  const int nb = K >> 8;
  const int n0 = static_cast<int>(blockIdx.x) * kDqRows, m0 = static_cast<int>(blockIdx.y) * kDqBatch;

  // Weight staging role: row rw of the tile, 16-byte piece p of each 32-byte
  // code chunk (chunk s of a block holds sub-blocks 2s and 2s + 1).  Rows
  // past N re-read the last row (results not stored).
  const int rw = tid >> 1, p = tid & 1;
  const size_t wblk = static_cast<size_t>(min(n0 + rw, N - 1)) * nb;
  constexpr size_t kH = PL ? 16 : 144, kQ = PL ? 64 : 144, kC = PL ? 16 : 32;
  const uint8_t* qbase = PL ? w + (p == 0 ? pa : 5 * pa) : w + 16 + 16 * p;
  // Activation staging role: batch row rx of the tile, columns
  // 64 s + 16 qx .. + 16 of each step s of a block.  Rows past M re-read the
  // last row.
  const int rx = tid >> 2, qx = tid & 3;
  const uint16_t* xrow = x + static_cast<size_t>(min(m0 + rx, M - 1)) * K + 16 * qx;

  // Loads past the last step re-read the last block (in bounds, unused).
  uint4 wq[4];     // code pieces, ring by step
  uint4 hd_cur, hd_next;  // block headers: the block being staged, the next
  uint4 xr[4][2];  // activation chunks of one block, ring by step within the block
  // (ring slots are indexed by the compile-time step s)
  auto load_w = [&](int b, int s) {
    wq[s] = *reinterpret_cast<const uint4*>(qbase + (wblk + min(b, nb - 1)) * kQ + s * kC);
  };
  auto load_h = [&](int b) { hd_next = *reinterpret_cast<const uint4*>(w + (wblk + min(b, nb - 1)) * kH); };
  auto load_x = [&](int b, int s) {
    const uint4* src = reinterpret_cast<const uint4*>(xrow + 256 * min(b, nb - 1) + 64 * s);
    xr[s][0] = src[0];
    xr[s][1] = src[1];
  };

  int e_run = -126;     // bf16: this row's scale exponent so far
  float cscale = 1.f;   // 2^-e_run

  // Dequantize / convert step (block b, step s) into LDS buffer s & 1 and
  // refill the rings with the step four later.  s is a compile-time
  // constant: no load sits under a run-time branch (the wait-count analysis
  // would then wait for every outstanding load).
  auto stage = [&](int b, auto s_c) {
    constexpr int s = decltype(s_c)::value;
    uint4* buf = dq_lds + (s & 1) * kDqBufUnits;
    // weights: sub-blocks 2s (low nibbles) and 2s + 1 (high nibbles)
    {
      if constexpr (s == 0) hd_cur = hd_next;
      const uint4 h = hd_cur;
      const float d = f16_to_f32(h.x & 0xFFFFu), dmin = f16_to_f32(h.x >> 16);
      // byte j of scw / mw: the 6-bit scale / min of sub-block j (s < 2) or 4 + j
      const uint32_t scw = s < 2 ? (h.y & 0x3F3F3F3Fu) : ((h.w & 0x0F0F0F0Fu) | ((h.y >> 2) & 0x30303030u));
      const uint32_t mw = s < 2 ? (h.z & 0x3F3F3F3Fu) : (((h.w >> 4) & 0x0F0F0F0Fu) | ((h.z >> 2) & 0x30303030u));
      const int j0 = (2 * s) & 3;
      const _Float16 ds0 = static_cast<_Float16>(d * byte_f32(scw, j0));
      const _Float16 ds1 = static_cast<_Float16>(d * byte_f32(scw, j0 + 1));
      const _Float16 dm0 = static_cast<_Float16>(-(dmin * byte_f32(mw, j0)));
      const _Float16 dm1 = static_cast<_Float16>(-(dmin * byte_f32(mw, j0 + 1)));
      const h2_t dsl = {ds0, ds0}, dsh = {ds1, ds1}, dml = {dm0, dm0}, dmh = {dm1, dm1};
      const h2_t off = {static_cast<_Float16>(-1024.f), static_cast<_Float16>(-1024.f)};
      const uint4 q4 = wq[s];
      const uint32_t q[4] = {q4.x, q4.y, q4.z, q4.w};
      uint32_t lo[8], hi[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t a = (q[i] & 0x000F000Fu) | 0x64006400u;
        const uint32_t bq = ((q[i] >> 8) & 0x000F000Fu) | 0x64006400u;
        const uint32_t c = ((q[i] >> 4) & 0x000F000Fu) | 0x64006400u;
        const uint32_t dq = ((q[i] >> 12) & 0x000F000Fu) | 0x64006400u;
        lo[2 * i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(h2_t, a) + off, dsl, dml));
        lo[2 * i + 1] =
            __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(h2_t, bq) + off, dsl, dml));
        hi[2 * i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(h2_t, c) + off, dsh, dmh));
        hi[2 * i + 1] =
            __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(h2_t, dq) + off, dsh, dmh));
      }
      buf[dq_unit(0, rw, 2 * p)] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
      buf[dq_unit(0, rw, 2 * p + 1)] = make_uint4(lo[4], lo[5], lo[6], lo[7]);
      buf[dq_unit(1, rw, 2 * p)] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      buf[dq_unit(1, rw, 2 * p + 1)] = make_uint4(hi[4], hi[5], hi[6], hi[7]);
      load_w(b + 1, s);
      if constexpr (s == 0) load_h(b + 1);
    }
    // activations: columns 64 s + 16 qx .. + 16 of row rx
    {
      if constexpr (!F16X && s == 0) {
        // the block's largest |x| in this row (four threads, its four chunks all in)
        u16x2_t m2 = {0, 0};
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const uint4 v = xr[c][hh];
            m2 = abs_max_bf16(m2, v.x);
            m2 = abs_max_bf16(m2, v.y);
            m2 = abs_max_bf16(m2, v.z);
            m2 = abs_max_bf16(m2, v.w);
          }
        int mx = max(static_cast<int>(m2.x), static_cast<int>(m2.y));
        mx = max(mx, __builtin_amdgcn_update_dpp(0, mx, 0xB1, 0xF, 0xF, false));  // lane ^ 1
        mx = max(mx, __builtin_amdgcn_update_dpp(0, mx, 0x4E, 0xF, 0xF, false));  // lane ^ 2
        // largest |x| in [2^E, 2^(E+1)), E = (bits >> 7) - 127: scaled into [2^14, 2^15)
        int eb = (mx >> 7) - 127 - 14;
        eb = eb < -126 ? -126 : (eb > 113 ? 113 : eb);
        const int e_new = max(e_run, eb);
        if (qx == 0) ratio_lds[(b & 1) * kDqBatch + rx] = __builtin_amdgcn_ldexpf(1.f, e_run - e_new);
        e_run = e_new;
        cscale = __builtin_amdgcn_ldexpf(1.f, -e_new);
      }
      const uint4 v0 = xr[s][0], v1 = xr[s][1];  // 16 columns: x0..x7, x8..x15
      uint4 o0, o1;
      if constexpr (F16X) {
        o0 = make_uint4((v0.x & 0xFFFFu) | (v0.y << 16), (v0.x >> 16) | (v0.y & 0xFFFF0000u),
                        (v0.z & 0xFFFFu) | (v0.w << 16), (v0.z >> 16) | (v0.w & 0xFFFF0000u));
        o1 = make_uint4((v1.x & 0xFFFFu) | (v1.y << 16), (v1.x >> 16) | (v1.y & 0xFFFF0000u),
                        (v1.z & 0xFFFFu) | (v1.w << 16), (v1.z >> 16) | (v1.w & 0xFFFF0000u));
      } else {
        auto lo_f = [&](uint32_t v) { return __uint_as_float(v << 16) * cscale; };
        auto hi_f = [&](uint32_t v) { return __uint_as_float(v & 0xFFFF0000u) * cscale; };
        o0 = make_uint4(pack_f16(lo_f(v0.x), lo_f(v0.y)), pack_f16(hi_f(v0.x), hi_f(v0.y)),
                        pack_f16(lo_f(v0.z), lo_f(v0.w)), pack_f16(hi_f(v0.z), hi_f(v0.w)));
        o1 = make_uint4(pack_f16(lo_f(v1.x), lo_f(v1.y)), pack_f16(hi_f(v1.x), hi_f(v1.y)),
                        pack_f16(lo_f(v1.z), lo_f(v1.w)), pack_f16(hi_f(v1.z), hi_f(v1.w)));
      }
      uint4* xb = buf + 2 * kDqRows * 4;
      xb[dq_unit(qx >> 1, rx, 2 * (qx & 1))] = o0;
      xb[dq_unit(qx >> 1, rx, 2 * (qx & 1) + 1)] = o1;
      load_x(b + 1, s);
    }
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // The products of step (block b, step s) from LDS buffer s & 1.
  auto multiply = [&](int b, auto s_c) {
    constexpr int s = decltype(s_c)::value;
    const uint4* buf = dq_lds + (s & 1) * kDqBufUnits;
    const uint4* xb = buf + 2 * kDqRows * 4;
    const int g = lane >> 4, r16 = lane & 15;
    if constexpr (!F16X && s == 0) {
      {  // the block may have raised the scale of some of this wave's rows
        float f[4];
        bool all_one = true;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f[j] = ratio_lds[(b & 1) * kDqBatch + 64 * wm + 16 * j + r16];
          all_one = all_one && f[j] == 1.f;
        }
        if (__builtin_amdgcn_ballot_w64(!all_one) != 0) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] *= f[j];
        }
      }
    }
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      h8_t B[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        B[j] = __builtin_bit_cast(h8_t, xb[dq_unit(kc, 64 * wm + 16 * j + r16, g)]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const h8_t A = __builtin_bit_cast(h8_t, buf[dq_unit(kc, 64 * wn + 16 * i + r16, g)]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B[j], acc[i][j], 0, 0, 0);
      }
    }
  };

  typedef std::integral_constant<int, 0> S0;
  typedef std::integral_constant<int, 1> S1;
  typedef std::integral_constant<int, 2> S2;
  typedef std::integral_constant<int, 3> S3;
  // Prologue: the header of block 0, steps 0..3 of the rings, step 0 staged.
  load_h(0);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    load_w(0, s);
    load_x(0, s);
  }
  stage(0, S0{});
  lds_barrier();
  // Each step multiplies one buffer while the next step is staged into the
  // other.  The last step stages a step past the end (block nb: clamped
  // loads of the last block, never multiplied), which keeps the loop body
  // free of branches; its activation maximum is the last block's again, so
  // it leaves the row scale as it was.
#pragma unroll 1
  for (int b = 0; b < nb; ++b) {
    multiply(b, S0{});
    stage(b, S1{});
    lds_barrier();
    multiply(b, S1{});
    stage(b, S2{});
    lds_barrier();
    multiply(b, S2{});
    stage(b, S3{});
    lds_barrier();
    multiply(b, S3{});
    stage(b + 1, S0{});
    lds_barrier();
  }

  if constexpr (!F16X) {
    if (qx == 0) fin_lds[rx] = __builtin_amdgcn_ldexpf(1.f, e_run);
    lds_barrier();
  }
  // Lane (q4, r16) holds outputs n .. n + 3 of activation row mrow: one
  // 16-byte store when the row length keeps it aligned.
  const int r16 = lane & 15, q4 = lane >> 4;
  const bool row4 = (N & 3) == 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int mrow = 64 * wm + 16 * j + r16;
    const int m = m0 + mrow;
    const float fs = F16X ? 1.f : fin_lds[mrow];
    if (m < M) {
      float* yr = y + static_cast<size_t>(m) * N;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = n0 + 64 * wn + 16 * i + 4 * q4;
        const f32x4_t v = acc[i][j] * fs;
        if (row4 && n + 4 <= N) {
          *reinterpret_cast<f32x4_t*>(yr + n) = v;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < N) yr[n + r] = v[r];
        }
      }
    }
  }
}


hipError_t gemm_q4_k_dq(const qmv_weights& W, const void* x, bool f16x, float* y, int64_t batch,
                        hipStream_t stream) {
  // This kernel while its grid fills between half and all of the compute
  // units in one round; otherwise (a second round of workgroups, or too few
  // weight rows to fill the device) the register-dequantized kernel, whose
  // tile height follows the shape (measured on the 7B FFN shapes, bf16: 18944
  // rows at 256-384 batch rows 86-87 us here against 87-106 us there; at 512
  // rows 165 against 111 us; 3584 rows at 192-512 batch rows 333-350 against
  // 208 us).
  const int64_t wgs = (W.rows + kDqTileRows - 1) / kDqTileRows * ((batch + kDqTileBatch - 1) / kDqTileBatch);
  const int64_t cus = device_cus();
  if ((wgs > cus || 2 * wgs < cus) && gemm_q4_k_dqreg_fits(W, batch))
    return gemm_q4_k_dqreg(W, x, f16x, y, batch, stream);
  const int N = static_cast<int>(W.rows), K = static_cast<int>(W.cols), M = static_cast<int>(batch);
  const uint8_t* w = static_cast<const uint8_t*>(W.data);
  const uint16_t* xh = static_cast<const uint16_t*>(x);
  const dim3 grid((N + kDqRows - 1) / kDqRows, (M + kDqBatch - 1) / kDqBatch);
  const bool pl = W.layout == QMV_LAYOUT_PLANES;
  if (pl && f16x)
    hipLaunchKernelGGL((gemm_q4_k_dqtile<true, true>), grid, dim3(kDqThreads), kDqLdsBytes, stream, w, W.scales_offset,
                       N, K, xh, y, M);
  else if (pl)
    hipLaunchKernelGGL((gemm_q4_k_dqtile<true, false>), grid, dim3(kDqThreads), kDqLdsBytes, stream, w,
                       W.scales_offset, N, K, xh, y, M);
  else if (f16x)
    hipLaunchKernelGGL((gemm_q4_k_dqtile<false, true>), grid, dim3(kDqThreads), kDqLdsBytes, stream, w,
                       W.scales_offset, N, K, xh, y, M);
  else
    hipLaunchKernelGGL((gemm_q4_k_dqtile<false, false>), grid, dim3(kDqThreads), kDqLdsBytes, stream, w,
                       W.scales_offset, N, K, xh, y, M);
  return hipGetLastError();
}

}  // namespace qmv
