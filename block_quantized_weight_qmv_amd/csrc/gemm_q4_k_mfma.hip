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


// ---------------------------------------------------------------------------
// Small batches (M <= 32): K split over the waves of a workgroup.
//
// Operands swapped relative to the tile kernel above: A = 16 batch rows of X,
// B = the codes of 16 weight rows, so accumulator r of lane (q, c) is
// Y[4q + r][c] -- batch rows 4q..4q+3 of weight row c, the row whose block
// header that lane loads itself.  Every scale is then applied from the lane's
// own registers, with no exchange.  The sub-block sums of X come from one
// more matrix-core product per sub-block, against a B of bf16 ones, which
// lands them in the same accumulator layout (Xs[4q + r] in every lane).
//
// A workgroup owns 16 NB weight rows and 16 MB batch rows; its kw waves take
// consecutive, near-equal runs of blocks along K.  X is read straight from
// memory (it is small and L2-resident), so the K loop has no barrier; the kw
// partial tiles are added in wave order through LDS at the end (results do
// not depend on timing).  W and X of the next block are in flight while the
// current one is multiplied.
template <int NB, int MB>
struct KsRegs {
  uint4 hd[NB];       // block header of this lane's row, per row tile
  uint2 q[NB][4];     // code bytes 32c + 8 (lane / 16) .. +7, chunks c = 0..3
  uint4 x[MB][8];     // X[16 mb + lane % 16][32 s + 8 (lane / 16) .. +7], s = 0..7
};

template <int NB, int MB>
__global__ void __launch_bounds__(512)
gemm_q4_k_bf16_ksplit(const uint8_t* w, int N, int K, const uint16_t* x, float* y, int M, int kw) {
  extern __shared__ float ks_part[];  // [kw][NB * MB * 4][64]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int q = lane >> 4, c = lane & 15;
  const int nb = K >> 8;
  const int b0 = wave * nb / kw, b1 = (wave + 1) * nb / kw;  // kw <= nb: never empty
  const int n0 = static_cast<int>(blockIdx.x) * 16 * NB;
  const int m0 = static_cast<int>(blockIdx.y) * 16 * MB;
  const size_t row_bytes = static_cast<size_t>(nb) * 144;
  const uint8_t* wr[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t)
    wr[t] = w + static_cast<size_t>(min(n0 + 16 * t + c, N - 1)) * row_bytes + 16 + 8 * q;
  const uint16_t* xr[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
    xr[mb] = x + static_cast<size_t>(min(m0 + 16 * mb + c, M - 1)) * K + 8 * q;

  // Loads of block b (clamped to the last block: in bounds, results unused).
  auto load = [&](int b, KsRegs<NB, MB>& r) {
    const int bb = min(b, nb - 1);
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const uint8_t* p = wr[t] + static_cast<size_t>(bb) * 144;
      r.hd[t] = *reinterpret_cast<const uint4*>(p - 16 - 8 * q);
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) r.q[t][cc] = *reinterpret_cast<const uint2*>(p + 32 * cc);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int s = 0; s < 8; ++s)
        r.x[mb][s] = *reinterpret_cast<const uint4*>(xr[mb] + static_cast<size_t>(bb) * 256 + 32 * s);
  };

  f32x4_t acc[NB][MB];
#pragma unroll
  for (int t = 0; t < NB; ++t)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[t][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const uint32_t one2 = 0x3F803F80u;  // two bf16 ones
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, make_uint4(one2, one2, one2, one2));

  auto step = [&](const KsRegs<NB, MB>& r) {
    float d[NB], dmin[NB];
    uint32_t sc03[NB], m03[NB], sc47[NB], m47[NB];
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const uint4 h = r.hd[t];
      d[t] = f16_to_f32(h.x & 0xFFFFu);
      dmin[t] = f16_to_f32(h.x >> 16);
      // Byte j of these words is sc_j / m_j (j < 4) or sc_{4+j} / m_{4+j}.
      sc03[t] = h.y & 0x3F3F3F3Fu;
      m03[t] = h.z & 0x3F3F3F3Fu;
      sc47[t] = (h.w & 0x0F0F0F0Fu) | ((h.y >> 2) & 0x30303030u);
      m47[t] = ((h.w >> 4) & 0x0F0F0F0Fu) | ((h.z >> 2) & 0x30303030u);
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      bf16x8_t A[MB];
      f32x4_t xs[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const uint4 v = r.x[mb][s];
        A[mb] = __builtin_bit_cast(bf16x8_t, make_uint4(lo_pair(v.x, v.y), hi_pair(v.x, v.y),
                                                        lo_pair(v.z, v.w), hi_pair(v.z, v.w)));
        xs[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mb], ones, f32x4_t{0.f, 0.f, 0.f, 0.f},
                                                         0, 0, 0);
      }
#pragma unroll
      for (int t = 0; t < NB; ++t) {
        const uint32_t scw = s < 4 ? sc03[t] : sc47[t], mw = s < 4 ? m03[t] : m47[t];
        const float ds = d[t] * static_cast<float>((scw >> (8 * (s & 3))) & 0xFFu);
        const float dmp = fmaf(128.f, ds, dmin[t] * static_cast<float>((mw >> (8 * (s & 3))) & 0xFFu));
        const uint2 pc = r.q[t][s >> 1];
        const uint32_t v0 = (s & 1) ? pc.x >> 4 : pc.x, v1 = (s & 1) ? pc.y >> 4 : pc.y;
        const uint32_t b[4] = {(v0 & 0x000F000Fu) | 0x43004300u, ((v0 >> 8) & 0x000F000Fu) | 0x43004300u,
                               (v1 & 0x000F000Fu) | 0x43004300u, ((v1 >> 8) & 0x000F000Fu) | 0x43004300u};
        const bf16x8_t B = __builtin_bit_cast(bf16x8_t, b);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const f32x4_t S =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mb], B, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[t][mb][i] = fmaf(-dmp, xs[mb][i], fmaf(ds, S[i], acc[t][mb][i]));
        }
      }
    }
  };

  KsRegs<NB, MB> ra, rb;
  load(b0, ra);
  load(b0 + 1, rb);
  int b = b0;
#pragma unroll 1
  for (; b + 1 < b1; b += 2) {
    step(ra);
    load(b + 2, ra);
    step(rb);
    load(b + 3, rb);
  }
  if (b < b1) step(ra);

  constexpr int kTiles = NB * MB * 4;  // accumulator floats per lane
  auto store = [&](int j, int ln, float v) {  // j = (t * MB + mb) * 4 + r
    const int r = j & 3, mb = (j >> 2) % MB, t = (j >> 2) / MB;
    const int m = m0 + 16 * mb + 4 * (ln >> 4) + r, n = n0 + 16 * t + (ln & 15);
    if (m < M && n < N) y[static_cast<size_t>(m) * N + n] = v;
  };
  if (kw == 1) {
#pragma unroll
    for (int t = 0; t < NB; ++t)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) store((t * MB + mb) * 4 + i, lane, acc[t][mb][i]);
    return;
  }
  float* mine = ks_part + wave * kTiles * 64;
#pragma unroll
  for (int t = 0; t < NB; ++t)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) mine[((t * MB + mb) * 4 + i) * 64 + lane] = acc[t][mb][i];
  __syncthreads();
  for (int e = static_cast<int>(threadIdx.x); e < kTiles * 64; e += kw * 64) {
    float v = ks_part[e];
    for (int k = 1; k < kw; ++k) v += ks_part[k * kTiles * 64 + e];
    store(e >> 6, e & 63, v);
  }
}


// ---------------------------------------------------------------------------
// Batches of at most 16 rows with X small enough for LDS: one resident
// workgroup per CU streams its share of W past an LDS copy of all of X.
//
// At these batch sizes the product is bound by reading W once, and what
// decides the time is how many bytes of W are in flight and how evenly the
// rows are spread.  Each workgroup (8 waves) owns a run of 16-row tiles; its
// (tile, block) units are cut into 8 near-equal runs, one per wave, so every
// wave streams about the same number of W bytes whatever the tile count.  A
// wave keeps kDepth units of W in flight in registers.  X is read from memory
// once per workgroup (rows read whole by consecutive lanes), permuted into
// the operand order and stored in LDS together with its sub-block sums; the
// A operands then come from LDS with one conflict-free ds_read_b128 per
// sub-block.  The first W loads are issued only once X is in: issued
// before, they queue ahead of it in the memory system and every wave waits
// longer for X (measured with per-wave timestamps: the X phase is the
// largest fixed cost of this kernel).  A wave's run spans at most
// two tiles; its partial tiles are parked in LDS and added in wave order at
// the end (results do not depend on timing).
//
// Operand roles as in the K-split kernel: A = X (rows = batch), B = codes,
// accumulator r of lane (q, c) is Y[4q + r][c] of weight row c.
#ifndef QMV_STREAM_WAVES
#define QMV_STREAM_WAVES 8
#endif
#ifndef QMV_STREAM_DEPTH
#define QMV_STREAM_DEPTH 2
#endif
constexpr int kStreamWaves = QMV_STREAM_WAVES;
static_assert((kStreamWaves & (kStreamWaves - 1)) == 0 && kStreamWaves <= 16, "power of two, at most 16");
constexpr int kDepth = QMV_STREAM_DEPTH;

// Byte k (0..3, a constant after unrolling) of v as fp32: one v_cvt_f32_ubyte{k}.
__device__ __forceinline__ float ubyte_f32(uint32_t v, int k) {
  switch (k & 3) {
    case 0: return cvt_ubyte<0>(v);
    case 1: return cvt_ubyte<1>(v);
    case 2: return cvt_ubyte<2>(v);
    default: return cvt_ubyte<3>(v);
  }
}

// A value the compiler cannot see through, held in a VGPR: lets
// (v & mask) | c become one v_and_or_b32 (mask from an SGPR, c from this
// VGPR) -- gfx950's VOP3 encodings take no literal operand.
__device__ __forceinline__ uint32_t vgpr_const(uint32_t c) {
  __asm__("" : "+v"(c));
  return c;
}

struct UnitRegs {
  uint4 hd;    // block header of this lane's row
  uint2 q[4];  // code bytes 32c + 8 (lane / 16) .. +7, chunks c = 0..3
};

// LDS bytes of the streaming kernel for nb blocks along K.
__host__ __device__ constexpr size_t stream_lds_bytes(int nb) {
  return static_cast<size_t>(nb) * 8 * (16 * 32 * 2 + 16 * 4) +  // X operands + sub-block sums
         static_cast<size_t>(kStreamWaves) * 2 * 4 * 64 * 4;      // two partial tiles per wave
}

__global__ void __launch_bounds__(64 * kStreamWaves)
gemm_q4_k_bf16_stream(const uint8_t* w, int N, int K, const uint16_t* x, float* y, int M) {
  extern __shared__ __attribute__((aligned(16))) uint8_t st_lds[];
  const int nb = K >> 8;
  // X operands: [nb][8 s][4 q][16 slots][16 B], batch row m of quarter q of
  // sub-block s in slot m ^ ((4 s + q) & 15): the staging stores (lanes along
  // q and s, one row m) and the operand reads (lanes along m) both spread
  // over all 32 banks.
  uint8_t* xa = st_lds;
  float* xsum = reinterpret_cast<float*>(st_lds + static_cast<size_t>(nb) * 8 * 1024);  // [nb][8][16]
  float* part = xsum + nb * 8 * 16;                            // [wave][2][4][64]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, c = lane & 15;
  // This workgroup's tiles [t0, t1) and this wave's units [u0, u1).
  const int T = (N + 15) >> 4, G = static_cast<int>(gridDim.x), g = static_cast<int>(blockIdx.x);
  const int t0 = g * (T / G) + min(g, T % G);
  const int nt = T / G + (g < T % G ? 1 : 0);
  const int U = nt * nb;
  const int u0 = wave * U / kStreamWaves, u1 = (wave + 1) * U / kStreamWaves;
  const size_t row_bytes = static_cast<size_t>(nb) * 144;

  auto load = [&](int u, UnitRegs& r) {
    const int uu = min(u, max(u1 - 1, 0));   // clamped: in bounds, results unused
    const int tr = t0 + uu / nb, b = uu - (uu / nb) * nb;
    const uint8_t* p = w + static_cast<size_t>(min(16 * tr + c, N - 1)) * row_bytes +
                       static_cast<size_t>(b) * 144;
    r.hd = *reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) r.q[cc] = *reinterpret_cast<const uint2*>(p + 16 + 32 * cc + 8 * q);
  };

  // Row m of X is 32 nb chunks of 16 bytes; thread j reads chunk j of every
  // row (consecutive lanes, consecutive bytes), which is sub-block s = j / 4
  // % 8, quarter k = j % 4 of block b = j / 32.  nb <= 16 here (the LDS
  // bound), so 32 nb <= 512 threads cover a row.
  const bool xl = tid < 32 * nb;
  const int xb_ = tid >> 5, xs_ = (tid >> 2) & 7, xk = tid & 3;
  uint4 xv[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    xv[m] = make_uint4(0u, 0u, 0u, 0u);
    if (xl && m < M) xv[m] = *reinterpret_cast<const uint4*>(x + static_cast<size_t>(m) * K + 8 * tid);
  }
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const uint4 v = xv[m];
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) sum += __uint_as_float(d[e] << 16) + __uint_as_float(d[e] & 0xFFFF0000u);
    sum += __shfl_xor(sum, 1);  // the four quarters of a sub-block are lanes 4i..4i+3
    sum += __shfl_xor(sum, 2);
    if (xl) {
      *reinterpret_cast<uint4*>(xa + ((static_cast<size_t>(xb_) * 8 + xs_) * 4 + xk) * 256 +
                                (m ^ ((4 * xs_ + xk) & 15)) * 16) =
          make_uint4(lo_pair(v.x, v.y), hi_pair(v.x, v.y), lo_pair(v.z, v.w), hi_pair(v.z, v.w));
      if (xk == 0) xsum[(xb_ * 8 + xs_) * 16 + m] = sum;
    }
  }
  // W of the first units only now: issued earlier, it queued ahead of X.
  UnitRegs f[kDepth];
#pragma unroll
  for (int j = 0; j < kDepth; ++j) load(u0 + j, f[j]);
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  // First tile of wave k's run: floor(floor(k U / W) / nb) = floor(k nt / W).
  const int tf = wave * nt / kStreamWaves;

  const uint32_t bias = vgpr_const(0x43004300u);  // two bf16 128.0

  auto unit = [&](int u, const UnitRegs& r) {
    const int b = u - (u / nb) * nb;
    const uint4 h = r.hd;
    const float d = f16_to_f32(h.x & 0xFFFFu), dmin = f16_to_f32(h.x >> 16);
    const uint32_t sc03 = h.y & 0x3F3F3F3Fu, m03 = h.z & 0x3F3F3F3Fu;
    const uint32_t sc47 = (h.w & 0x0F0F0F0Fu) | ((h.y >> 2) & 0x30303030u);
    const uint32_t m47 = ((h.w >> 4) & 0x0F0F0F0Fu) | ((h.z >> 2) & 0x30303030u);
    const uint8_t* xb = xa + static_cast<size_t>(b) * 8 * 1024 + q * 256;
    const float* xsb = xsum + b * 8 * 16 + 4 * q;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8_t A = *reinterpret_cast<const bf16x8_t*>(xb + s * 1024 + ((c ^ ((4 * s + q) & 15)) * 16));
      const f32x4_t xs = *reinterpret_cast<const f32x4_t*>(xsb + s * 16);
      const float ds = d * ubyte_f32(s < 4 ? sc03 : sc47, s);
      const float dmp = fmaf(128.f, ds, dmin * ubyte_f32(s < 4 ? m03 : m47, s));
      const uint2 pc = r.q[s >> 1];
      const int sh = 4 * (s & 1);
      const uint32_t bw[4] = {((pc.x >> sh) & 0x000F000Fu) | bias, ((pc.x >> (8 + sh)) & 0x000F000Fu) | bias,
                              ((pc.y >> sh) & 0x000F000Fu) | bias, ((pc.y >> (8 + sh)) & 0x000F000Fu) | bias};
      const f32x4_t S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8_t, bw),
                                                                f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = fmaf(-dmp, xs[i], fmaf(ds, S[i], acc[i]));
    }
    // End of a tile (or of the run): park the partial tile.
    if (b == nb - 1 || u == u1 - 1) {
      float* dst = part + ((wave * 2 + (u / nb - tf)) * 4) * 64 + lane;
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i * 64] = acc[i];
      acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  };

  // Single-exit loop over groups of kDepth units (as in the GEMV skeleton: a
  // second exit would make the wait-count analysis drain the prefetch).
  int u = u0;
#pragma unroll 1
  for (; u + kDepth < u1; u += kDepth) {
#pragma unroll
    for (int j = 0; j < kDepth; ++j) {
      unit(u + j, f[j]);
      load(u + j + kDepth, f[j]);
      __asm__ __volatile__("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int j = 0; j < kDepth; ++j)
    if (u + j < u1) unit(u + j, f[j]);

  __syncthreads();
  // Tile t of the workgroup gets the partials of the waves whose run meets
  // it, in wave order.  Wave k's run is [floor(k U / W), floor((k+1) U / W))
  // (W a power of two: no division); its partial of tile t sits in slot
  // t - floor(k nt / W).
  for (int e = tid; e < nt * 256; e += 64 * kStreamWaves) {
    const int tt = e >> 8, r = (e >> 6) & 3, ln = e & 63;
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < kStreamWaves; ++k) {
      const int ku0 = k * U / kStreamWaves, ku1 = (k + 1) * U / kStreamWaves;
      if (ku1 > ku0 && ku0 < (tt + 1) * nb && ku1 > tt * nb)
        v += part[((k * 2 + (tt - k * nt / kStreamWaves)) * 4 + r) * 64 + ln];
    }
    const int m = 4 * (ln >> 4) + r, n = 16 * (t0 + tt) + (ln & 15);
    if (m < M && n < N) y[static_cast<size_t>(m) * N + n] = v;
  }
}

hipError_t gemm_q4_k_bf16(const qmv_weights& W, const void* x, float* y, int64_t batch,
                          hipStream_t stream) {
  const int N = static_cast<int>(W.rows), K = static_cast<int>(W.cols), M = static_cast<int>(batch);
  const uint8_t* w = static_cast<const uint8_t*>(W.data);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const int nb = K / 256;
  if (M <= 16 && stream_lds_bytes(nb) <= static_cast<size_t>(device_lds_per_block())) {
    // One workgroup per CU (more only if a workgroup would hold over 8 tiles).
    const int T = (N + 15) / 16;
    int G = device_cus();
    if (G > T) G = T;
    if (G < (T + 7) / 8) G = (T + 7) / 8;
    hipLaunchKernelGGL(gemm_q4_k_bf16_stream, dim3(G), dim3(64 * kStreamWaves), stream_lds_bytes(nb),
                       stream, w, N, K, xb, y, M);
    return hipGetLastError();
  }
  if (M <= 32) {
    // K split: enough waves for about eight per SIMD, at most 8 per workgroup
    // and never more than one per block.
    const unsigned n_groups = static_cast<unsigned>((N + 15) / 16);
    int kw = static_cast<int>((8192 + n_groups - 1) / n_groups);
    kw = kw < 1 ? 1 : (kw > 8 ? 8 : kw);
    kw = kw > nb ? nb : kw;
    const size_t lds = static_cast<size_t>(kw) * (M <= 16 ? 1 : 2) * 4 * 64 * sizeof(float);
    if (M <= 16)
      hipLaunchKernelGGL((gemm_q4_k_bf16_ksplit<1, 1>), dim3(n_groups, 1), dim3(64 * kw), lds, stream,
                         w, N, K, xb, y, M, kw);
    else
      hipLaunchKernelGGL((gemm_q4_k_bf16_ksplit<1, 2>), dim3(n_groups, 1), dim3(64 * kw), lds, stream,
                         w, N, K, xb, y, M, kw);
    return hipGetLastError();
  }
  const unsigned n_tiles = static_cast<unsigned>((N + 63) / 64);
  const unsigned m_tiles = static_cast<unsigned>((M + 63) / 64);
  hipLaunchKernelGGL(gemm_q4_k_bf16_kernel<4>, dim3(n_tiles, m_tiles), dim3(256), 0, stream, w, N,
                     K, xb, y, M);
  return hipGetLastError();
}

}  // namespace qmv
