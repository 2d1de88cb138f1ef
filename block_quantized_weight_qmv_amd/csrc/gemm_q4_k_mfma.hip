// Batched Q4_K multiply on the gfx950 matrix cores: Y[m][n] = sum_k X[m][k] W[n][k]
// for bf16 activations X [M][K] and Q4_K weights W [N][K] (y layout [batch][rows]).
//
// Used when the batch makes the product a real dense contraction (M >= 64:
// prefill chunks, speculative-decode verify).  The pages keep two kernel
// families for this reason: hipEngine 0.3.0 ("Quickstart") pairs WMMA prefill
// with GEMV decode, LLM170 runs speculative verify as a batched forward, and
// hipfire's multi-weight WMMA dispatch rules (K a whole number of blocks, one
// dtype per dispatch, disjoint output tiles) apply here unchanged.
//
// Per workgroup (4 waves) an output tile of 64 rows of W x 64 activation rows,
// K stepped 64 weights at a time (one Q4_K sub-block pair):
//   1. every thread decodes 16 weights of one W row to their exact fp32 value
//      w = fma(d*sc, u, -dmin*m) (the one rounding of the format), then splits
//      it into bf16 hi = RNE(w) and lo = RNE(w - hi): hi + lo carries 16
//      significant bits (relative error <= 2^-17), so the bf16 products stay
//      far inside the 2e-3 GEMV bound while X is used exactly as given;
//   2. hi, lo and the X tile go to LDS (rows padded to 144 bytes so that the
//      MFMA operand reads of 32 rows hit distinct banks);
//   3. each wave runs v_mfma_f32_32x32x16_bf16 on its 32 x 32 block, twice per
//      16-wide K slice (hi and lo), accumulating in fp32.
// The next step's global loads are issued before the MFMA phase.
//
// Operand layouts of v_mfma_f32_32x32x16_bf16 (checked on the device): lane l
// holds A[l % 32][8 (l / 32) + e] and B[8 (l / 32) + e][l % 32] for e = 0..7;
// accumulator r of lane l is D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
#include "device_util.h"
#include "launch.h"

namespace qmv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kTileN = 64, kTileM = 64, kTileK = 64;
constexpr int kRowPad = kTileK + 8;  // bf16 per LDS row: 144 bytes

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// 6-bit scale and min of sub-block s (0..7) from the 12 scale bytes, held in
// the header dwords h1 (bytes 0-3), h2 (4-7), h3 (8-11).
__device__ __forceinline__ void q4k_scale_min(uint32_t h1, uint32_t h2, uint32_t h3, int s,
                                              uint32_t& sc, uint32_t& mn) {
  const uint64_t lo = (static_cast<uint64_t>(h2) << 32) | h1;  // scales[0..7]
  auto byte = [&](int i) -> uint32_t {
    return i < 8 ? static_cast<uint32_t>(lo >> (8 * i)) & 0xFFu : (h3 >> (8 * (i - 8))) & 0xFFu;
  };
  if (s < 4) {
    sc = byte(s) & 63u;
    mn = byte(s + 4) & 63u;
  } else {
    sc = (byte(s + 4) & 15u) | ((byte(s - 4) >> 6) << 4);
    mn = (byte(s + 4) >> 4) | ((byte(s) >> 6) << 4);
  }
}

__global__ void __launch_bounds__(256)
gemm_q4_k_bf16_kernel(const uint8_t* w, int N, int K, const uint16_t* x, float* y, int M,
                      int m_tiles) {
  __shared__ __attribute__((aligned(16))) uint16_t wh[kTileN][kRowPad];
  __shared__ __attribute__((aligned(16))) uint16_t wl[kTileN][kRowPad];
  __shared__ __attribute__((aligned(16))) uint16_t xs[kTileM][kRowPad];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int mt = static_cast<int>(blockIdx.x) % m_tiles, nt = static_cast<int>(blockIdx.x) / m_tiles;
  const int n0 = nt * kTileN, m0 = mt * kTileM;
  const int nb = K / 256;
  const size_t row_bytes = static_cast<size_t>(nb) * 144;
  const int steps = nb * 4;

  // Decode assignment: W row r, 16 weights = half h (low / high nibbles) of
  // qs bytes [32c + 16q, +16) of the step's chunk c.
  const int r = tid >> 2, h = (tid >> 1) & 1, q = tid & 1;
  const uint8_t* wrow = w + static_cast<size_t>(min(n0 + r, N - 1)) * row_bytes;
  // X assignment: activation row xr, 16 consecutive elements of the step.
  const int xr = tid >> 2, xk = 16 * (tid & 3);
  const uint16_t* xrow = x + static_cast<size_t>(min(m0 + xr, M - 1)) * K + xk;

  uint4 hd, qv, x0, x1;
  auto load = [&](int step) {
    const uint8_t* p = wrow + static_cast<size_t>(step >> 2) * 144;
    hd = *reinterpret_cast<const uint4*>(p);
    qv = *reinterpret_cast<const uint4*>(p + 16 + 32 * (step & 3) + 16 * q);
    const uint16_t* px = xrow + step * kTileK;
    x0 = *reinterpret_cast<const uint4*>(px);
    x1 = *reinterpret_cast<const uint4*>(px + 8);
  };

  // Output block of this wave: W rows [32 wn, +32) x activation rows [32 wm, +32).
  const int wn = wave >> 1, wm = wave & 1;
  f32x16_t acc = {};

  load(0);
  for (int step = 0; step < steps; ++step) {
    // 1-2: decode and stage this step's tiles.
    {
      const int c = step & 3, s = 2 * c + h;
      uint32_t sc, mn;
      q4k_scale_min(hd.y, hd.z, hd.w, s, sc, mn);
      const float ds = f16_to_f32(hd.x & 0xFFFFu) * static_cast<float>(sc);
      const float dm = f16_to_f32(hd.x >> 16) * static_cast<float>(mn);
      const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
      uint32_t hw[8], lw[8];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t byte = (qw[i >> 2] >> (8 * (i & 3))) & 0xFFu;
        const uint32_t u = h ? (byte >> 4) : (byte & 15u);
        const float v = fmaf(ds, static_cast<float>(u), -dm);
        const uint32_t hb = f32_to_bf16_rne(v);
        const uint32_t lb = f32_to_bf16_rne(v - __uint_as_float(hb << 16));
        if (i & 1) {
          hw[i >> 1] |= hb << 16;
          lw[i >> 1] |= lb << 16;
        } else {
          hw[i >> 1] = hb;
          lw[i >> 1] = lb;
        }
      }
      const int col = 32 * h + 16 * q;
      *reinterpret_cast<uint4*>(&wh[r][col]) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      *reinterpret_cast<uint4*>(&wh[r][col + 8]) = make_uint4(hw[4], hw[5], hw[6], hw[7]);
      *reinterpret_cast<uint4*>(&wl[r][col]) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
      *reinterpret_cast<uint4*>(&wl[r][col + 8]) = make_uint4(lw[4], lw[5], lw[6], lw[7]);
      *reinterpret_cast<uint4*>(&xs[xr][xk]) = x0;
      *reinterpret_cast<uint4*>(&xs[xr][xk + 8]) = x1;
    }
    __syncthreads();
    if (step + 1 < steps) load(step + 1);
    // 3: four 16-wide K slices, hi and lo.
#pragma unroll
    for (int ks = 0; ks < kTileK / 16; ++ks) {
      const int kk = 16 * ks + 8 * (lane >> 5);
      const bf16x8_t a_hi = *reinterpret_cast<const bf16x8_t*>(&wh[32 * wn + (lane & 31)][kk]);
      const bf16x8_t a_lo = *reinterpret_cast<const bf16x8_t*>(&wl[32 * wn + (lane & 31)][kk]);
      const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(&xs[32 * wm + (lane & 31)][kk]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_hi, b, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_lo, b, acc, 0, 0, 0);
    }
    __syncthreads();
  }

  const int m = m0 + 32 * wm + (lane & 31);
  if (m < M) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int n = n0 + 32 * wn + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      if (n < N) y[static_cast<size_t>(m) * N + n] = acc[i];
    }
  }
}

hipError_t gemm_q4_k_bf16(const qmv_weights& W, const void* x, float* y, int64_t batch,
                          hipStream_t stream) {
  const int N = static_cast<int>(W.rows), K = static_cast<int>(W.cols), M = static_cast<int>(batch);
  const int m_tiles = (M + kTileM - 1) / kTileM, n_tiles = (N + kTileN - 1) / kTileN;
  hipLaunchKernelGGL(gemm_q4_k_bf16_kernel, dim3(m_tiles * n_tiles), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(W.data), N, K, static_cast<const uint16_t*>(x), y,
                     M, m_tiles);
  return hipGetLastError();
}

}  // namespace qmv
