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
// ds = d sc_s, dm = dmin m_s, applied in fp32.  Nothing is dequantized to
// memory and the products are exact (the 2e-3 GEMV bound is spent only on
// fp32 summation).
//
// Operand roles: A = 16 batch rows of X, B = the codes of 16 weight rows, so
// accumulator r of lane (q, c) = (l / 16, l % 16) is Y[4q + r][c]: batch rows
// 4q..4q+3 of weight row c, the row whose block header that lane loads.
// Every scale is applied from the lane's own registers.
//
// Three kernels, by batch (routing in gemm_q4_k_bf16 below):
//   * M <= 16 and X fits in LDS: gemm_q4_k_stream (also for fp16 X) -- one workgroup per
//     CU streams its share of W past an LDS copy of all of X;
//   * 17 <= M: gemm_q4_k_tile (also for fp16 X) -- 64 NB x 16 MB WM tiles, X staged per
//     block through double-buffered LDS, min and offset terms as two extra
//     matrix-core products per block;
//   * M <= 16 with X too large for LDS: gemm_q4_k_ksplit (also fp16 X) -- K split over
//     the waves of a workgroup, X read from memory.
//
// v_mfma_f32_16x16x32_bf16 (layout checked on the device): lane l holds
// A[l % 16][8 (l / 16) + e] and B[8 (l / 16) + e][l % 16], e = 0..7, and
// accumulator r of lane l is D[4 (l / 16) + r][l % 16].  Code slot 8q + e of a
// sub-block maps to weight 8q + (0, 2, 1, 3, 4, 6, 5, 7)[e], the order in which
// masking one dword of code bytes yields bf16 pairs; X is permuted to match
// where it is staged.
#include <type_traits>

#include "device_util.h"
#include "launch.h"

namespace qmv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// v with every bit cleared unless keep: an AND with a mask the compiler cannot
// see through.  A select of a loaded value is turned into a branch around the
// load, and a load under a branch makes the wait-count analysis wait for
// every outstanding load.
__device__ __forceinline__ uint4 keep_if(uint4 v, bool keep) {
  uint32_t k = keep ? 0xFFFFFFFFu : 0u;
  __asm__("" : "+v"(k));
  return make_uint4(v.x & k, v.y & k, v.z & k, v.w & k);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Sum of the eight bf16 values of a 16-byte chunk in fp32: four
// v_dot2c_f32_bf16 against bf16 ones (exact products, fp32 sums).
__device__ __forceinline__ float bf16x8_sum(uint4 v) {
  const bf16x2_t one = __builtin_bit_cast(bf16x2_t, 0x3F803F80u);
  float s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, v.x), one, 0.f, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, v.y), one, s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, v.z), one, s, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, v.w), one, s, false);
}

// Sum over the four lanes of a quad (lanes 4i..4i+3) with DPP quad
// permutes -- register-to-register, unlike __shfl_xor (ds_bpermute).
__device__ __forceinline__ float quad_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));  // lane ^ 1
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));  // lane ^ 2
  return v;
}

// Two columns of a permuted 8-group: (x0, x2) and (x1, x3) from (x0, x1), (x2, x3).
__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) { return (a & 0xFFFFu) | (b << 16); }
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }

// The activation type of the matrix-core kernels.  bf16: the codes enter the
// matrix cores as bf16(128 + u) (0x4300 | u).  fp16: as fp16(1024 + u)
// (0x6400 | u, exact, the same one AND-OR per two codes); products are exact
// in fp32 either way, and the 1024 X offset removed afterwards costs at most
// about 2^-24 * 1024 / 8 relative to a sub-block's sum.
template <bool F16>
struct StreamX {
  typedef bf16x8_t vec8;
  static constexpr uint32_t kBias2 = 0x43004300u;  // two bf16 128.0
  static constexpr float kBias = 128.f;
  static constexpr uint32_t kOne2 = 0x3F803F80u;   // two bf16 ones
  __device__ static float sum8(uint4 v) { return bf16x8_sum(v); }
  __device__ static f32x4_t mfma(vec8 a, vec8 b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  }
};
template <>
struct StreamX<true> {
  typedef _Float16 vec8 __attribute__((ext_vector_type(8)));
  static constexpr uint32_t kBias2 = 0x64006400u;  // two fp16 1024.0
  static constexpr float kBias = 1024.f;
  static constexpr uint32_t kOne2 = 0x3C003C00u;   // two fp16 ones
  // Sum of the eight fp16 values of a chunk in fp32: four v_dot2_f32_f16
  // against fp16 ones (exact products, fp32 sums).
  __device__ static float sum8(uint4 v) {
    const h2_t one = __builtin_bit_cast(h2_t, 0x3C003C00u);
    float s = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, v.x), one, 0.f, false);
    s = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, v.y), one, s, false);
    s = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, v.z), one, s, false);
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, v.w), one, s, false);
  }
  __device__ static f32x4_t mfma(vec8 a, vec8 b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  }
};

// ---------------------------------------------------------------------------
// Small batches with X too large for LDS: K split over the waves of a workgroup.
//
// The sub-block sums of X come from one more matrix-core product per
// sub-block, against a B of bf16 ones, which lands them in the accumulator
// layout (Xs[4q + r] in every lane).
//
// A workgroup owns 16 NB weight rows and 16 MB batch rows; its kw waves take
// consecutive, near-equal runs of blocks along K.  X is read straight from
// memory (it is small and L2-resident), so the K loop has no barrier; the kw
// partial tiles are added in wave order through LDS at the end (results do
// not depend on timing).  W and X of the next block are in flight while the
// current one is multiplied.
// Where a lane finds Q4_K block `blk` (= row * blocks per row + block): its
// 16-byte header, and its 8-byte piece qs[32 cc + 8 q .. +8) of code chunk
// cc, in the canonical layout (PL = false: 144-byte blocks) or the plane
// layout of planes.h (PL = true: header plane; qs[32cc .. 32cc+16) in code
// plane A at a, qs[32cc+16 .. 32cc+32) in plane B at 5a, 64 bytes per block).
template <bool PL>
struct Q4KBlockAddr {
  static constexpr size_t kH = PL ? 16 : 144;  // header stride per block
  static constexpr size_t kQ = PL ? 64 : 144;  // code stride per block
  static constexpr int kC = PL ? 16 : 32;      // code chunk stride
  const uint8_t* hbase;
  const uint8_t* qbase;
  __device__ Q4KBlockAddr(const uint8_t* w, uint64_t a, int q) {
    hbase = w;
    if constexpr (PL)
      qbase = w + (q < 2 ? a : 5 * a) + 8 * (q & 1);
    else
      qbase = w + 16 + 8 * q;
  }
  __device__ const uint8_t* hd(size_t blk) const { return hbase + blk * kH; }
  __device__ const uint8_t* qs(size_t blk, int cc) const { return qbase + blk * kQ + cc * kC; }
};

template <int NB, int MB>
struct KsRegs {
  uint4 hd[NB];       // block header of this lane's row, per row tile
  uint2 q[NB][4];     // code bytes 32c + 8 (lane / 16) .. +7, chunks c = 0..3
  uint4 x[MB][8];     // X[16 mb + lane % 16][32 s + 8 (lane / 16) .. +7], s = 0..7
};

template <int NB, int MB, bool PL, bool F16>
__global__ void __launch_bounds__(512)
gemm_q4_k_ksplit(const uint8_t* w, uint64_t pa, int N, int K, const uint16_t* x, float* y, int M, int kw) {
  typedef StreamX<F16> XT;
  typedef typename XT::vec8 vec8;
  extern __shared__ float ks_part[];  // [kw][NB * MB * 4][64]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int q = lane >> 4, c = lane & 15;
  const int nb = K >> 8;
  const int b0 = wave * nb / kw, b1 = (wave + 1) * nb / kw;  // kw <= nb: never empty
  const int n0 = static_cast<int>(blockIdx.x) * 16 * NB;
  const int m0 = static_cast<int>(blockIdx.y) * 16 * MB;
  const Q4KBlockAddr<PL> wa(w, pa, q);
  size_t wr[NB];  // first block of this lane's row, per row tile
#pragma unroll
  for (int t = 0; t < NB; ++t) wr[t] = static_cast<size_t>(min(n0 + 16 * t + c, N - 1)) * nb;
  const uint16_t* xr[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
    xr[mb] = x + static_cast<size_t>(min(m0 + 16 * mb + c, M - 1)) * K + 8 * q;

  // Loads of block b (clamped to the last block: in bounds, results unused).
  auto load = [&](int b, KsRegs<NB, MB>& r) {
    const int bb = min(b, nb - 1);
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const size_t blk = wr[t] + bb;
      r.hd[t] = *reinterpret_cast<const uint4*>(wa.hd(blk));
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) r.q[t][cc] = *reinterpret_cast<const uint2*>(wa.qs(blk, cc));
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
  const uint32_t one2 = XT::kOne2;
  const vec8 ones = __builtin_bit_cast(vec8, make_uint4(one2, one2, one2, one2));

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
      vec8 A[MB];
      f32x4_t xs[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const uint4 v = r.x[mb][s];
        A[mb] = __builtin_bit_cast(vec8, make_uint4(lo_pair(v.x, v.y), hi_pair(v.x, v.y),
                                                    lo_pair(v.z, v.w), hi_pair(v.z, v.w)));
        xs[mb] = XT::mfma(A[mb], ones);
      }
#pragma unroll
      for (int t = 0; t < NB; ++t) {
        const uint32_t scw = s < 4 ? sc03[t] : sc47[t], mw = s < 4 ? m03[t] : m47[t];
        const float ds = d[t] * static_cast<float>((scw >> (8 * (s & 3))) & 0xFFu);
        const float dmp = fmaf(XT::kBias, ds, dmin[t] * static_cast<float>((mw >> (8 * (s & 3))) & 0xFFu));
        const uint2 pc = r.q[t][s >> 1];
        const uint32_t v0 = (s & 1) ? pc.x >> 4 : pc.x, v1 = (s & 1) ? pc.y >> 4 : pc.y;
        const uint32_t b[4] = {(v0 & 0x000F000Fu) | XT::kBias2, ((v0 >> 8) & 0x000F000Fu) | XT::kBias2,
                               (v1 & 0x000F000Fu) | XT::kBias2, ((v1 >> 8) & 0x000F000Fu) | XT::kBias2};
        const vec8 B = __builtin_bit_cast(vec8, b);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const f32x4_t S = XT::mfma(A[mb], B);
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

template <bool PL, bool F16>
__global__ void __launch_bounds__(64 * kStreamWaves)
gemm_q4_k_stream(const uint8_t* w, uint64_t pa, int N, int K, const uint16_t* x, float* y, int M) {
  typedef StreamX<F16> XT;
  typedef typename XT::vec8 vec8;
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
  const Q4KBlockAddr<PL> wa(w, pa, q);

  auto load = [&](int u, UnitRegs& r) {
    const int uu = min(u, max(u1 - 1, 0));   // clamped: in bounds, results unused
    const int tr = t0 + uu / nb, b = uu - (uu / nb) * nb;
    const size_t blk = static_cast<size_t>(min(16 * tr + c, N - 1)) * nb + b;
    r.hd = *reinterpret_cast<const uint4*>(wa.hd(blk));
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) r.q[cc] = *reinterpret_cast<const uint2*>(wa.qs(blk, cc));
  };

  // Row m of X is 32 nb chunks of 16 bytes; thread j reads chunk j of every
  // row (consecutive lanes, consecutive bytes), which is sub-block s = j / 4
  // % 8, quarter k = j % 4 of block b = j / 32.  nb <= 16 here (the LDS
  // bound), so 32 nb <= 512 threads cover a row.
  const bool xl = tid < 32 * nb;
  const int xb_ = tid >> 5, xs_ = (tid >> 2) & 7, xk = tid & 3;
  // Only the M real rows are read and stored: the operand rows past M (left
  // as whatever LDS holds) feed only accumulator rows past M, which are never
  // stored.  The loads may sit under the (uniform) row test: nothing else is
  // in flight yet, so waiting for them waits for nothing more.
  const int xt = min(tid, 32 * nb - 1);
  uint4 xv[16];
#pragma unroll
  for (int m = 0; m < 16; ++m)
    if (m < M) xv[m] = *reinterpret_cast<const uint4*>(x + static_cast<size_t>(m) * K + 8 * xt);
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    if (m >= M) continue;  // uniform; the loop stays unrolled
    const uint4 v = xv[m];
    const float sum = quad_sum(XT::sum8(v));  // the four quarters of a sub-block are lanes 4i..4i+3
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
  lds_barrier();

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  // First tile of wave k's run: floor(floor(k U / W) / nb) = floor(k nt / W).
  const int tf = wave * nt / kStreamWaves;

  const uint32_t bias = vgpr_const(XT::kBias2);

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
      const vec8 A = *reinterpret_cast<const vec8*>(xb + s * 1024 + ((c ^ ((4 * s + q) & 15)) * 16));
      const f32x4_t xs = *reinterpret_cast<const f32x4_t*>(xsb + s * 16);
      const float ds = d * ubyte_f32(s < 4 ? sc03 : sc47, s);
      const float dmp = fmaf(XT::kBias, ds, dmin * ubyte_f32(s < 4 ? m03 : m47, s));
      const uint2 pc = r.q[s >> 1];
      const int sh = 4 * (s & 1);
      const uint32_t bw[4] = {((pc.x >> sh) & 0x000F000Fu) | bias, ((pc.x >> (8 + sh)) & 0x000F000Fu) | bias,
                              ((pc.y >> sh) & 0x000F000Fu) | bias, ((pc.y >> (8 + sh)) & 0x000F000Fu) | bias};
      const f32x4_t S = XT::mfma(A, __builtin_bit_cast(vec8, bw));
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

  lds_barrier();
  // Tile t of the workgroup gets the partials of the waves whose run meets
  // it, in wave order.  Wave k's run is [floor(k U / W), floor((k+1) U / W))
  // (W a power of two: no division); its partial of tile t sits in slot
  // t - floor(k nt / W).
  for (int e = tid; e < nt * 256; e += 64 * kStreamWaves) {
    const int tt = e >> 8, r = (e >> 6) & 3, ln = e & 63;
    // All slots are read first (clamped to a valid one), then the ones that
    // hold a partial of this tile are added in wave order: reads under the
    // per-wave test would each wait out the LDS latency in turn.
    float p[kStreamWaves];
#pragma unroll
    for (int k = 0; k < kStreamWaves; ++k) {
      const int slot = min(max(tt - k * nt / kStreamWaves, 0), 1);
      p[k] = part[((k * 2 + slot) * 4 + r) * 64 + ln];
    }
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < kStreamWaves; ++k) {
      const int ku0 = k * U / kStreamWaves, ku1 = (k + 1) * U / kStreamWaves;
      if (ku1 > ku0 && ku0 < (tt + 1) * nb && ku1 > tt * nb) v += p[k];
    }
    const int m = 4 * (ln >> 4) + r, n = 16 * (t0 + tt) + (ln & 15);
    if (m < M && n < N) y[static_cast<size_t>(m) * N + n] = v;
  }
}



// ---------------------------------------------------------------------------
// Larger batches: workgroups of WN x WM waves over a run of 16-row tiles of W
// and 16 MB WM batch rows.
//
// Workgroup g owns a run of nt <= WN NB consecutive 16-row tiles of W (runs
// as equal as the tile count allows, so that with one workgroup per CU every
// CU gets the same work up to one tile); wave (wn, wm) owns NB tiles of that
// run (wn < nt / NB; a wave whose slot lies past the run only stages X) and
// MB 16-row tiles of the batch (rows 16 MB wm ..).  X
// advances one block (256 columns) at a time through two LDS buffers with one
// barrier per block: the loads of block b + 2 are issued while block b is
// multiplied and stored after it, so their latency is hidden by a whole block
// of work.  W comes straight from memory into registers, two blocks ahead.
// Operand roles as in the kernels above (A = X, B = codes, lane (q, c)
// accumulates Y[4q + r][c]).
//
// Per sub-block s the matrix cores give S = sum_k (128 + u_k) X_k, which the
// lane scales by its row's ds = d sc_s (one FMA per accumulator).  The rest
// of each weight, -128 ds - dm per sub-block, is a product over sub-blocks:
//   sum_s (128 d sc_s + dmin m_s) Xs_s = 128 d T1 + dmin T2,
//   T1 = sum_s sc_s Xs_s,  T2 = sum_s m_s Xs_s,
// two more matrix-core products per block with K = the 8 sub-blocks: A holds
// each sub-block sum split exactly into three bf16 parts (8 + 8 + 8
// significant bits; K slots 8j + s for part j, the fourth group zero) and B
// the 6-bit sc_s or m_s, exact in bf16.  The products are exact and the sums
// fp32, as for S.
template <int NB>
struct TileRegs {
  uint4 hd[NB];
  uint2 q[NB][4];
};

// LDS bytes per buffer: X operands of 16 MT rows x 256 columns, then the
// split sub-block sums (1 KB per 16 rows).
template <int MT>
__host__ __device__ constexpr size_t tile_buf_bytes() {
  return static_cast<size_t>(MT) * 512 + static_cast<size_t>(MT / 16) * 1024;
}

// F16: fp16 X.  Only the main products change (codes as fp16(1024 + u), X
// as given, fp16 sums of eight); the split sub-block sums are fp32 values
// either way and keep their bf16 products.
template <int NB, int MB, int WM, int WN, bool PL, bool F16>
__global__ void __launch_bounds__(64 * WN * WM)
gemm_q4_k_tile(const uint8_t* w, uint64_t pa, int N, int K, const uint16_t* x, float* y, int M) {
  typedef StreamX<F16> XT;
  typedef typename XT::vec8 vec8;
  extern __shared__ __attribute__((aligned(16))) uint8_t tl_lds[];
  constexpr int MT = 16 * MB * WM;             // batch rows of the workgroup
  constexpr int kThreads = 64 * WN * WM;
  constexpr size_t kXBytes = static_cast<size_t>(MT) * 512;
  constexpr size_t kBuf = tile_buf_bytes<MT>();
  constexpr int kItems = (MT * 8 + kThreads - 1) / kThreads;  // (row, sub-block) items per thread
  // Buffer layout: X operands [8 s][MT / 16][4 q][16 slots][16 B], batch row
  // m (within its 16-row tile) of quarter q of sub-block s in slot
  // m ^ ((s + 4 q) & 15); then the split sums [MT / 16][4 j][16 m][8 s] bf16
  // (j = 3 stays zero).  The swizzle spreads both the staging stores (lanes
  // along s, one row, one quarter) and the operand reads (lanes along m) over
  // all 32 banks.

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % WN, wm = wave / WN;
  const int q = lane >> 4, c = lane & 15;
  const int nb = K >> 8;
  const int T = (N + 15) >> 4, G = static_cast<int>(gridDim.x), g = static_cast<int>(blockIdx.x);
  const int t0 = g * (T / G) + min(g, T % G);
  const int nt = T / G + (g < T % G ? 1 : 0);
  const bool active = wn * NB < nt;  // wave-uniform
  const int n0 = 16 * (t0 + wn * NB);
  const int mw0 = static_cast<int>(blockIdx.y) * MT;           // first batch row of the workgroup
  const Q4KBlockAddr<PL> wa(w, pa, q);
  size_t wr[NB];  // first block of this lane's row, per row tile
#pragma unroll
  for (int t = 0; t < NB; ++t) wr[t] = static_cast<size_t>(min(n0 + 16 * t + c, N - 1)) * nb;

  // Zero the fourth part group of both split-sum buffers once.
  for (int i = tid; i < 2 * (MT / 16) * 16; i += kThreads) {
    const int buf = i / ((MT / 16) * 16), mb = (i >> 4) % (MT / 16), e = i & 15;
    *reinterpret_cast<uint4*>(tl_lds + buf * kBuf + kXBytes + (mb * 4 + 3) * 256 + e * 16) =
        make_uint4(0u, 0u, 0u, 0u);
  }

  auto load_w = [&](int b, TileRegs<NB>& r) {
    const int bb = min(b, nb - 1);
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const size_t blk = wr[t] + bb;
      r.hd[t] = *reinterpret_cast<const uint4*>(wa.hd(blk));
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) r.q[t][cc] = *reinterpret_cast<const uint2*>(wa.qs(blk, cc));
    }
  };
  // Item i = tid + kThreads j: batch row i / 8 of the workgroup, sub-block
  // i % 8 -- 64 contiguous bytes of X, read as four 16-byte quarters.
  // Loads are unconditional (clamped): a load under a branch makes the
  // compiler's wait-count analysis wait for every outstanding load.
  auto load_x = [&](int b, uint4 (&v)[kItems][4]) {
    const int bb = min(b, nb - 1);
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
      const int i = min(tid + kThreads * j, MT * 8 - 1);
      const int m = min(mw0 + (i >> 3), M - 1);
      const uint4* p = reinterpret_cast<const uint4*>(x + static_cast<size_t>(m) * K + 256 * bb + 32 * (i & 7));
#pragma unroll
      for (int k = 0; k < 4; ++k) v[j][k] = p[k];
    }
  };
  const bool ragged = mw0 + MT > M;  // only the last batch tile has rows past M
  auto stage_x = [&](uint4 (&v)[kItems][4], int buf) {
    uint8_t* base = tl_lds + buf * kBuf;
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
      const int i = tid + kThreads * j;
      if (kItems * kThreads > MT * 8 && i >= MT * 8) continue;
      const int row = i >> 3, s = i & 7, mb = row >> 4, mr = row & 15;
      if (ragged) {
#pragma unroll
        for (int k = 0; k < 4; ++k) v[j][k] = keep_if(v[j][k], mw0 + row < M);
      }
      float sum = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint4 u = v[j][k];
        sum += XT::sum8(u);
        *reinterpret_cast<uint4*>(base + ((s * (MT / 16) + mb) * 4 + k) * 256 + (mr ^ ((s + 4 * k) & 15)) * 16) =
            make_uint4(lo_pair(u.x, u.y), hi_pair(u.x, u.y), lo_pair(u.z, u.w), hi_pair(u.z, u.w));
      }
      // exact three-way bf16 split: truncations, each residual exact in fp32
      const uint32_t hb = __float_as_uint(sum) & 0xFFFF0000u;
      const float r1 = sum - __uint_as_float(hb);
      const uint32_t mbits = __float_as_uint(r1) & 0xFFFF0000u;
      const float r2 = r1 - __uint_as_float(mbits);
      uint16_t* t = reinterpret_cast<uint16_t*>(base + kXBytes + mb * 1024 + mr * 16) + s;
      t[0] = static_cast<uint16_t>(hb >> 16);
      t[256 / 2] = static_cast<uint16_t>(mbits >> 16);
      t[512 / 2] = static_cast<uint16_t>(__float_as_uint(r2) >> 16);
    }
  };

  f32x4_t acc[NB][MB];
#pragma unroll
  for (int t = 0; t < NB; ++t)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[t][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const uint32_t bias = vgpr_const(XT::kBias2);

  auto compute = [&](const TileRegs<NB>& r, int buf) {
    const uint8_t* base = tl_lds + buf * kBuf;
    float ds[NB][8], d128[NB], dmin[NB];
    uint32_t bt1[NB][4], bt2[NB][4];
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const uint4 h = r.hd[t];
      const float d = f16_to_f32(h.x & 0xFFFFu);
      d128[t] = XT::kBias * d;
      dmin[t] = f16_to_f32(h.x >> 16);
      const uint32_t sc03 = h.y & 0x3F3F3F3Fu, m03 = h.z & 0x3F3F3F3Fu;
      const uint32_t sc47 = (h.w & 0x0F0F0F0Fu) | ((h.y >> 2) & 0x30303030u);
      const uint32_t m47 = ((h.w >> 4) & 0x0F0F0F0Fu) | ((h.z >> 2) & 0x30303030u);
      float scf[8], mf[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        scf[s] = ubyte_f32(s < 4 ? sc03 : sc47, s);
        mf[s] = ubyte_f32(s < 4 ? m03 : m47, s);
        ds[t][s] = d * scf[s];
      }
      // small integers: the top half of the fp32 value is the exact bf16
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bt1[t][e] = (__float_as_uint(scf[2 * e]) >> 16) | (__float_as_uint(scf[2 * e + 1]) & 0xFFFF0000u);
        bt2[t][e] = (__float_as_uint(mf[2 * e]) >> 16) | (__float_as_uint(mf[2 * e + 1]) & 0xFFFF0000u);
      }
    }
    // Two orders of the sub-block loop, both pinning each step's scaling in
    // place with an empty asm (left alone, the compiler sinks every FMA below
    // all the block's products and parks those products in registers --
    // hundreds of them).  With one or two batch tiles per wave the loop is
    // software-pipelined: iteration s reads the A operands of s + 1, issues
    // the products of s and then scales those of s - 1, so neither the LDS
    // nor the matrix-core latency sits in front of a dependent instruction.
    // With four batch tiles the products of a step already cover that
    // latency, and the straight order measured faster.
    if constexpr (MB <= 2) {
      auto read_a = [&](int s, vec8 (&A)[MB]) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          A[mb] = *reinterpret_cast<const vec8*>(base + ((s * (MT / 16) + MB * wm + mb) * 4 + q) * 256 +
                                                 (c ^ ((s + 4 * q) & 15)) * 16);
      };
      auto scale = [&](int s, const f32x4_t (&S)[NB][MB]) {
#pragma unroll
        for (int t = 0; t < NB; ++t)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[t][mb][i] = fmaf(ds[t][s], S[t][mb][i], acc[t][mb][i]);
            __asm__ __volatile__("" : "+v"(acc[t][mb]));
          }
      };
      vec8 A[2][MB];
      f32x4_t S[2][NB][MB];
      read_a(0, A[0]);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        if (s < 7) read_a(s + 1, A[(s + 1) & 1]);
#pragma unroll
        for (int t = 0; t < NB; ++t) {
          const uint2 pc = r.q[t][s >> 1];
          const int sh = 4 * (s & 1);
          const uint32_t bw[4] = {((pc.x >> sh) & 0x000F000Fu) | bias, ((pc.x >> (8 + sh)) & 0x000F000Fu) | bias,
                                  ((pc.y >> sh) & 0x000F000Fu) | bias, ((pc.y >> (8 + sh)) & 0x000F000Fu) | bias};
          const vec8 B = __builtin_bit_cast(vec8, bw);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) S[s & 1][t][mb] = XT::mfma(A[s & 1][mb], B);
        }
        if (s > 0) scale(s - 1, S[(s - 1) & 1]);
      }
      scale(7, S[1]);
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        vec8 A[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          A[mb] = *reinterpret_cast<const vec8*>(base + ((s * (MT / 16) + MB * wm + mb) * 4 + q) * 256 +
                                                 (c ^ ((s + 4 * q) & 15)) * 16);
#pragma unroll
        for (int t = 0; t < NB; ++t) {
          const uint2 pc = r.q[t][s >> 1];
          const int sh = 4 * (s & 1);
          const uint32_t bw[4] = {((pc.x >> sh) & 0x000F000Fu) | bias, ((pc.x >> (8 + sh)) & 0x000F000Fu) | bias,
                                  ((pc.y >> sh) & 0x000F000Fu) | bias, ((pc.y >> (8 + sh)) & 0x000F000Fu) | bias};
          const vec8 B = __builtin_bit_cast(vec8, bw);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            const f32x4_t S = XT::mfma(A[mb], B);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[t][mb][i] = fmaf(ds[t][s], S[i], acc[t][mb][i]);
            __asm__ __volatile__("" : "+v"(acc[t][mb]));
          }
        }
      }
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const bf16x8_t AT =
          *reinterpret_cast<const bf16x8_t*>(base + kXBytes + ((MB * wm + mb) * 4 + q) * 256 + c * 16);
#pragma unroll
      for (int t = 0; t < NB; ++t) {
        const f32x4_t T1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            AT, __builtin_bit_cast(bf16x8_t, bt1[t]), f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        const f32x4_t T2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            AT, __builtin_bit_cast(bf16x8_t, bt2[t]), f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t][mb][i] = fmaf(-d128[t], T1[i], fmaf(-dmin[t], T2[i], acc[t][mb][i]));
      }
    }
  };

  // The block loop, once with the products and once staging only (a wave
  // whose tile slot lies past the run): two copies rather than a branch in
  // the loop, so that the wait counts of the working copy stay exact.  Both
  // meet the same barriers in the same order.
  auto run = [&](auto with_products) {
    constexpr bool kWork = decltype(with_products)::value;
    TileRegs<NB> ra, rb;
    uint4 xv[kItems][4];
    load_x(0, xv);
    if constexpr (kWork) {
      load_w(0, ra);
      load_w(1, rb);
    }
    stage_x(xv, 0);
    load_x(1, xv);
    lds_barrier();
    int b = 0;
#pragma unroll 1
    for (; b + 2 < nb; b += 2) {
      if constexpr (kWork) {
        compute(ra, 0);
        load_w(b + 2, ra);
      }
      stage_x(xv, 1);
      lds_barrier();
      load_x(b + 2, xv);
      if constexpr (kWork) {
        compute(rb, 1);
        load_w(b + 3, rb);
      }
      stage_x(xv, 0);
      lds_barrier();
      load_x(b + 3, xv);
    }
    if constexpr (kWork) compute(ra, 0);
    if (b + 1 < nb) {
      stage_x(xv, 1);
      lds_barrier();
      if constexpr (kWork) compute(rb, 1);
    }
  };
  if (active) {
    run(std::true_type{});
  } else {
    run(std::false_type{});
    return;
  }

#pragma unroll
  for (int t = 0; t < NB; ++t)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = mw0 + 16 * (MB * wm + mb) + 4 * q + i, n = n0 + 16 * t + c;
        if (m < M && n < N) y[static_cast<size_t>(m) * N + n] = acc[t][mb][i];
      }
}

// M <= 16 with X too large for LDS: K split over up to 8 waves per workgroup
// (about eight waves per SIMD in all, never more than one per block).
template <bool PL, bool F16>
static hipError_t launch_ksplit(const uint8_t* w, uint64_t pa, int N, int K, const uint16_t* xb, float* y,
                                int M, hipStream_t stream) {
  const int nb = K / 256;
  const unsigned n_groups = static_cast<unsigned>((N + 15) / 16);
  int kw = static_cast<int>((8192 + n_groups - 1) / n_groups);
  kw = kw < 1 ? 1 : (kw > 8 ? 8 : kw);
  kw = kw > nb ? nb : kw;
  const size_t lds = static_cast<size_t>(kw) * 4 * 64 * sizeof(float);
  hipLaunchKernelGGL((gemm_q4_k_ksplit<1, 1, PL, F16>), dim3(n_groups, 1), dim3(64 * kw), lds, stream, w, pa, N,
                     K, xb, y, M, kw);
  return hipGetLastError();
}

// 17 <= M: runs of 4-5 weight tiles, one workgroup per CU for each batch
// tile of 32, 64 or 128 rows (every CU gets the same work up to one tile).
template <bool PL, bool F16>
static hipError_t launch_tile(const uint8_t* w, uint64_t pa, int N, int K, const uint16_t* xb, float* y,
                              int M, hipStream_t stream) {
  const int T = (N + 15) / 16;
  int G = device_cus();
  if (G > T) G = T;
  if (G < (T + 4) / 5) G = (T + 4) / 5;
  if (M <= 64) {
    if (M <= 32)
      hipLaunchKernelGGL((gemm_q4_k_tile<1, 1, 2, 5, PL, F16>), dim3(G, 1), dim3(640), 2 * tile_buf_bytes<32>(),
                         stream, w, pa, N, K, xb, y, M);
    else
      hipLaunchKernelGGL((gemm_q4_k_tile<1, 2, 2, 5, PL, F16>), dim3(G, 1), dim3(640), 2 * tile_buf_bytes<64>(),
                         stream, w, pa, N, K, xb, y, M);
  } else {
    hipLaunchKernelGGL((gemm_q4_k_tile<1, 4, 2, 5, PL, F16>), dim3(G, (M + 127) / 128), dim3(640),
                       2 * tile_buf_bytes<128>(), stream, w, pa, N, K, xb, y, M);
  }
  return hipGetLastError();
}

template <bool PL>
static hipError_t gemm_q4_k_bf16_layout(const qmv_weights& W, const void* x, float* y, int64_t batch,
                                        hipStream_t stream) {
  const uint64_t pa = W.scales_offset;  // plane unit a (planes); 0 (canonical)
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
    hipLaunchKernelGGL((gemm_q4_k_stream<PL, false>), dim3(G), dim3(64 * kStreamWaves), stream_lds_bytes(nb),
                       stream, w, pa, N, K, xb, y, M);
    return hipGetLastError();
  }
  if (M <= 16) return launch_ksplit<PL, false>(w, pa, N, K, xb, y, M, stream);
  return launch_tile<PL, false>(w, pa, N, K, xb, y, M, stream);
}

// fp16 activations: the kernels of the bf16 path with fp16 operands (up to
// 16 rows the streaming kernel where X fits its LDS copy, else the K-split
// kernel; from 17 rows the tile kernels).
bool gemm_q4_k_f16_fits(int64_t cols, int64_t batch) { return cols >= 256 && batch >= 1; }

hipError_t gemm_q4_k_f16(const qmv_weights& W, const void* x, float* y, int64_t batch,
                         hipStream_t stream) {
  if (!gemm_q4_k_f16_fits(W.cols, batch)) return hipErrorInvalidValue;
  const int N = static_cast<int>(W.rows), K = static_cast<int>(W.cols);
  const uint8_t* w = static_cast<const uint8_t*>(W.data);
  if (batch >= 17) {
    const uint16_t* xh = static_cast<const uint16_t*>(x);
    return W.layout == QMV_LAYOUT_PLANES
               ? launch_tile<true, true>(w, W.scales_offset, N, K, xh, y, static_cast<int>(batch), stream)
               : launch_tile<false, true>(w, W.scales_offset, N, K, xh, y, static_cast<int>(batch), stream);
  }
  const int T = (N + 15) / 16;
  int G = device_cus();
  if (G > T) G = T;
  if (G < (T + 7) / 8) G = (T + 7) / 8;
  const int M = static_cast<int>(batch);
  const uint16_t* xh = static_cast<const uint16_t*>(x);
  if (stream_lds_bytes(K / 256) > static_cast<size_t>(device_lds_per_block()))
    return W.layout == QMV_LAYOUT_PLANES ? launch_ksplit<true, true>(w, W.scales_offset, N, K, xh, y, M, stream)
                                         : launch_ksplit<false, true>(w, W.scales_offset, N, K, xh, y, M, stream);
  if (W.layout == QMV_LAYOUT_PLANES)
    hipLaunchKernelGGL((gemm_q4_k_stream<true, true>), dim3(G), dim3(64 * kStreamWaves), stream_lds_bytes(K / 256),
                       stream, w, W.scales_offset, N, K, xh, y, M);
  else
    hipLaunchKernelGGL((gemm_q4_k_stream<false, true>), dim3(G), dim3(64 * kStreamWaves), stream_lds_bytes(K / 256),
                       stream, w, W.scales_offset, N, K, xh, y, M);
  return hipGetLastError();
}

hipError_t gemm_q4_k_bf16(const qmv_weights& W, const void* x, float* y, int64_t batch,
                          hipStream_t stream) {
  return W.layout == QMV_LAYOUT_PLANES ? gemm_q4_k_bf16_layout<true>(W, x, y, batch, stream)
                                       : gemm_q4_k_bf16_layout<false>(W, x, y, batch, stream);
}

}  // namespace qmv
