// Batched Q4_K multiply on the gfx950 matrix cores: Y[m][n] = sum_k X[m][k] W[n][k]
// for bf16 activations X [M][K] and Q4_K weights W [N][K] (y layout [batch][rows]).
//
// Used once the batch makes the product a dense contraction (prefill chunks,
// speculative-decode verify).  The pages keep two kernel families for this
// reason: hipEngine 0.3.0 ("Quickstart") pairs WMMA prefill with GEMV decode,
// LLM170 runs speculative verify as a batched forward, and hipfire's
// multi-weight WMMA dispatch rules (K a whole number of blocks, one dtype per
// dispatch, disjoint output tiles) apply unchanged.
//
// Factored form.  A Q4_K weight is d*sc_s*u - dmin*m_s with a 4-bit code u and
// per-(row, sub-block) scales, so for every sub-block s of 32 weights
//   sum_k W[n][k] X[m][k] = d sc_s (sum_k u X) - dmin m_s (sum_k X).
// The code sum is a small-integer dot product that the matrix cores compute
// exactly: the codes enter v_mfma_f32_16x16x32_bf16 as the bf16 value 128 + u
// (bits 0x4300 | u, one AND-OR per two codes), X enters as given, and one
// instruction covers one sub-block (K = 32).  With S = sum (128 + u) X and
// Xs = sum X, the row's contribution is ds S - (128 ds + dm) Xs with
// ds = d sc_s, dm = dmin m_s, applied in fp32 to the 16x16 result.  Nothing
// is dequantized to memory, W is read once per tile of up to 64 batch rows,
// and the products are exact (the 2e-3 GEMV bound is spent only on fp32
// summation).
//
// Workgroup: 4 waves, 64 rows of W (16 per wave), MT = 16 MB batch rows,
// stepping one Q4_K block (256 K) at a time:
//   * X's block for the tile is staged in LDS (double buffered, one barrier
//     per block, its global loads issued two blocks ahead) with each group of
//     8 columns permuted to the code order below, together with its 8
//     sub-block sums;
//   * each lane streams its row's header and 4 x 8 code bytes straight into
//     registers (two blocks in flight) and builds the A operands there;
//   * ds and 128 ds + dm of its 16 rows are exchanged through per-wave LDS.
//
// v_mfma_f32_16x16x32_bf16 (layout checked on the device): lane l holds
// A[l % 16][8 (l / 16) + e] and B[8 (l / 16) + e][l % 16], e = 0..7, and
// accumulator r of lane l is D[4 (l / 16) + r][l % 16].  Code slot 8q + e of a
// sub-block maps to weight 8q + (0, 2, 1, 3, 4, 6, 5, 7)[e], the order in which
// masking one dword of code bytes yields bf16 pairs.
#include "device_util.h"
#include "launch.h"

namespace qmv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kXRow = 256 + 8;  // bf16 per staged X row (528 bytes)

// 6-bit scale and min of sub-block s (0..7) from the header dwords holding
// scales[0..3] (h1), [4..7] (h2) and [8..11] (h3).
__device__ __forceinline__ void q4k_scale_min(uint32_t h1, uint32_t h2, uint32_t h3, int s,
                                              uint32_t& sc, uint32_t& mn) {
  auto byte = [&](int i) -> uint32_t {
    const uint32_t word = i < 4 ? h1 : (i < 8 ? h2 : h3);
    return (word >> (8 * (i & 3))) & 0xFFu;
  };
  if (s < 4) {
    sc = byte(s) & 63u;
    mn = byte(s + 4) & 63u;
  } else {
    sc = (byte(s + 4) & 15u) | ((byte(s - 4) >> 6) << 4);
    mn = (byte(s + 4) >> 4) | ((byte(s) >> 6) << 4);
  }
}

// Two columns of a permuted 8-group: (x0, x2) and (x1, x3) from (x0, x1), (x2, x3).
__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) { return (a & 0xFFFFu) | (b << 16); }
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }

struct WRegs {
  uint4 hd;     // block header of this lane's row
  uint2 q[4];   // code bytes 32c + 8 (lane / 16) .. +7 of chunks c = 0..3
};

template <int MB>
__global__ void __launch_bounds__(256)
gemm_q4_k_bf16_kernel(const uint8_t* w, int N, int K, const uint16_t* x, float* y, int M) {
  constexpr int MT = 16 * MB;
  constexpr int kPairs = MT * 8;                 // (batch row, sub-block) sums per block
  constexpr int kPairsPerThread = (kPairs + 255) / 256;
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][MT][kXRow];
  __shared__ __attribute__((aligned(16))) float xsum[2][8][MT];
  __shared__ __attribute__((aligned(16))) float sds[4][8][16];   // ds per (wave, s, row)
  __shared__ __attribute__((aligned(16))) float sdm[4][8][16];   // 128 ds + dm

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, l16 = lane & 15;
  const int nb = K / 256;
  const int n0 = static_cast<int>(blockIdx.x) * 64 + wave * 16;
  const int m0 = static_cast<int>(blockIdx.y) * MT;
  const uint8_t* wrow = w + static_cast<size_t>(min(n0 + l16, N - 1)) * (static_cast<size_t>(nb) * 144);

  auto load_w = [&](int b, WRegs& r) {
    const uint8_t* p = wrow + static_cast<size_t>(min(b, nb - 1)) * 144;
    r.hd = *reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int c = 0; c < 4; ++c) r.q[c] = *reinterpret_cast<const uint2*>(p + 16 + 32 * c + 8 * q);
  };
  // X staging: thread handles pairs (m, s) = (pi / 8, pi % 8): 32 columns.
  uint4 xr[2][kPairsPerThread][4];  // X of the next two blocks in flight
  auto load_x = [&](int b, int slot) {
#pragma unroll
    for (int t = 0; t < kPairsPerThread; ++t) {
      const int pi = min(tid + 256 * t, kPairs - 1);
      const int m = pi >> 3, s = pi & 7;
      const uint16_t* p = x + static_cast<size_t>(min(m0 + m, M - 1)) * K +
                          static_cast<size_t>(min(b, nb - 1)) * 256 + 32 * s;
#pragma unroll
      for (int g = 0; g < 4; ++g) xr[slot][t][g] = reinterpret_cast<const uint4*>(p)[g];
    }
  };
  auto stage_x = [&](int buf) {
#pragma unroll
    for (int t = 0; t < kPairsPerThread; ++t) {
      const int pi = tid + 256 * t;
      if (pi < kPairs) {
        const int m = pi >> 3, s = pi & 7;
        float sum = 0.f;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint4 v = xr[buf][t][g];
          const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sum += __uint_as_float(d[i] << 16);
            sum += __uint_as_float(d[i] & 0xFFFF0000u);
          }
          *reinterpret_cast<uint4*>(&xs[buf][m][32 * s + 8 * g]) =
              make_uint4(lo_pair(v.x, v.y), hi_pair(v.x, v.y), lo_pair(v.z, v.w), hi_pair(v.z, v.w));
        }
        xsum[buf][s][m] = sum;
      }
    }
  };

  f32x4_t acc[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto step = [&](int b, const WRegs& r) {
    const int buf = b & 1;
    stage_x(buf);
    __syncthreads();
    load_x(b + 2, buf);
    // Scales of this lane's row for sub-blocks 2q and 2q + 1.
    {
      const float d = f16_to_f32(r.hd.x & 0xFFFFu), dmin = f16_to_f32(r.hd.x >> 16);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int s = 2 * q + i;
        uint32_t sc, mn;
        q4k_scale_min(r.hd.y, r.hd.z, r.hd.w, s, sc, mn);
        const float ds = d * static_cast<float>(sc);
        sds[wave][s][l16] = ds;
        sdm[wave][s][l16] = fmaf(128.f, ds, dmin * static_cast<float>(mn));
      }
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint2 pc = r.q[s >> 1];
      const uint32_t v0 = (s & 1) ? pc.x >> 4 : pc.x, v1 = (s & 1) ? pc.y >> 4 : pc.y;
      const uint32_t a[4] = {(v0 & 0x000F000Fu) | 0x43004300u, ((v0 >> 8) & 0x000F000Fu) | 0x43004300u,
                             (v1 & 0x000F000Fu) | 0x43004300u, ((v1 >> 8) & 0x000F000Fu) | 0x43004300u};
      const bf16x8_t A = __builtin_bit_cast(bf16x8_t, a);
      const f32x4_t ds4 = *reinterpret_cast<const f32x4_t*>(&sds[wave][s][4 * q]);
      const f32x4_t dm4 = *reinterpret_cast<const f32x4_t*>(&sdm[wave][s][4 * q]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const bf16x8_t B = *reinterpret_cast<const bf16x8_t*>(&xs[buf][16 * mb + l16][32 * s + 8 * q]);
        const f32x4_t S =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        const float xsv = xsum[buf][s][16 * mb + l16];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mb][i] = fmaf(-dm4[i], xsv, fmaf(ds4[i], S[i], acc[mb][i]));
      }
    }
  };

  WRegs ra, rb;
  load_w(0, ra);
  load_w(1, rb);
  load_x(0, 0);
  load_x(1, 1);
  int b = 0;
#pragma unroll 1
  for (; b + 2 < nb; b += 2) {
    step(b, ra);
    load_w(b + 2, ra);
    step(b + 1, rb);
    load_w(b + 3, rb);
  }
  step(b, ra);
  if (b + 1 < nb) step(b + 1, rb);

#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = m0 + 16 * mb + l16;
    if (m < M) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = n0 + 4 * q + i;
        if (n < N) y[static_cast<size_t>(m) * N + n] = acc[mb][i];
      }
    }
  }
}

hipError_t gemm_q4_k_bf16(const qmv_weights& W, const void* x, float* y, int64_t batch,
                          hipStream_t stream) {
  const int N = static_cast<int>(W.rows), K = static_cast<int>(W.cols), M = static_cast<int>(batch);
  const uint8_t* w = static_cast<const uint8_t*>(W.data);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const unsigned n_tiles = static_cast<unsigned>((N + 63) / 64);
  if (M <= 16) {
    hipLaunchKernelGGL(gemm_q4_k_bf16_kernel<1>, dim3(n_tiles, 1), dim3(256), 0, stream, w, N, K, xb,
                       y, M);
  } else if (M <= 32) {
    hipLaunchKernelGGL(gemm_q4_k_bf16_kernel<2>, dim3(n_tiles, 1), dim3(256), 0, stream, w, N, K, xb,
                       y, M);
  } else {
    const unsigned m_tiles = static_cast<unsigned>((M + 63) / 64);
    hipLaunchKernelGGL(gemm_q4_k_bf16_kernel<4>, dim3(n_tiles, m_tiles), dim3(256), 0, stream, w, N,
                       K, xb, y, M);
  }
  return hipGetLastError();
}

}  // namespace qmv
