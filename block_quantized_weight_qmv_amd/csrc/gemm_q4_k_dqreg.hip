// Batched Q4_K on the gfx950 matrix cores, weights dequantized into operand
// registers: Y[m][n] = sum_k X[m][k] W[n][k] for tens to hundreds of
// activation rows X (bf16 or fp16) and Q4_K weights W (canonical or plane
// layout), y layout [batch][rows].
//
// The batched-prefill reading of the pages' kernel families (hipEngine
// "Quickstart": matrix-core prefill beside GEMV decode): once a weight meets
// tens of activation rows, it is cheaper to convert it to the matrix-core
// type once than to apply its scales to every product.
//
// Three kernels per run of one to four matrices on the same activations
// (the consecutive items of a multi-matrix launch, e.g. q+k+v), in stream
// order:
// 1. act_rows_f16: the activations to fp16 once, into the workspace (not
//    again for a following run on the same activations): bf16
//    rows scaled by a power of two 2^-e per row (e from the row's largest
//    |x|, which lands in [2^14, 2^15)), fp16 rows as given; each group of
//    eight columns in the operand order (0, 2, 1, 3, 4, 6, 5, 7) below.
// 2. gemm_q4_k_dqreg: the products of every matrix of the run (each
//    workgroup finds its matrix by its row tile) over one of S slices of K
//    (whole 256-column blocks); with S = 1 straight into y, else into S
//    partial outputs in the workspace.  Results are multiplied by 2^e at the
//    end.
// 3. (S > 1) dqreg_sum: y = the sum of the partial outputs in slice order,
//    so results are independent of timing.
//
// Workgroup: four waves, one per SIMD.  Wave w owns 16 T consecutive weight
// rows (T tiles of 16, T = 1..5) and all 16 NB activation rows of the
// workgroup's batch tile (NB = 4 or 8).  Each wave dequantizes its own weight tiles straight into A operand
// registers: weights never pass through LDS and are converted once.  The
// fp16 activation tile is copied into LDS per half block (no arithmetic),
// where all four waves read it as B operands.  Per 32-column step a wave
// issues NB T v_mfma_f32_16x16x32_f16 against NB LDS reads.
//
// What sets the time (gfx950, measured): one wave issues about two
// independent VALU instructions under each 16-cycle product for free; beyond
// that the VALU issue sets the pace.  Forming an A operand costs about 16
// VALU instructions (two per product at NB = 8, four at NB = 4).  Each B
// operand read (1 KB per wave) serves T products, so T = 1 leaves the four
// waves bound by LDS bandwidth.  The host picks T, NB and S per run from a
// model fitted to such measurements and from how many workgroups fill the
// compute units.
//
// K order.  A block is walked in two halves of four steps, half h covering
// columns 128 h .. 128 h + 128 (code chunks c = 2h and 2h + 1: sub-blocks
// 2c, low nibbles of code bytes 32c .. 32c + 32, and 2c + 1, high nibbles).
// In half h, A operand lane (g, r) (g = lane / 16) holds the 16-byte code
// piece 16 (g & 1) .. + 16 of chunk c = 2h + (g >> 1); step t takes one dword
// pair of it: sub-block 2c + (t & 1), elements 16 (g & 1) + 8 (t >> 1) +
// (0, 2, 1, 3, 4, 6, 5, 7), the order in which masking a dword yields fp16
// pairs.  The B operand holds the same columns of X in the same order, so a
// half's activations are 128 consecutive columns of each row.
//
// Weights: w = d sc u - dmin m, evaluated per element as
// fma(u, fp16(d sc), -fp16(dmin m)) in packed fp16; the codes enter as
// fp16(1024 + u) (one AND-OR per two codes) and lose the 1024 exactly in a
// packed add.  Each weight carries about one and a half fp16 roundings
// (relative error near 2^-11) against its fp32 value.
//
// LDS unit (16 bytes) of activation row n, step t of the half, k-group g:
// 16 n + 8 (t & 1) + (f(t, g) ^ s(n)) with f(t, g) = (t >> 1) + 2 (g & 1) +
// 4 ((t & 1) ^ (g >> 1)) and s(n) = 4 (n & 1) + ((n >> 1) & 3).  The operand
// reads (eight rows at one (t, g)) and the staging stores (two rows, four
// consecutive 16-byte pieces each) both land any eight lanes of a row of the
// wave on eight different 16-byte bank groups of a 128-byte line.
#include <algorithm>
#include <mutex>
#include <type_traits>
#include <utility>

#include "device_util.h"
#include "launch.h"

namespace qmv {

namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

constexpr int kRgThreads = 256;  // four waves
constexpr int kRgRowUnits = 16;  // 16-byte units per activation row and half block
constexpr int kRgNB = 8;         // B tiles per workgroup: 128 activation rows

__host__ __device__ constexpr int rg_batch(int nb) { return 16 * nb; }
__host__ __device__ constexpr int rg_buf_units(int nb) { return rg_batch(nb) * kRgRowUnits; }
__host__ __device__ constexpr size_t rg_lds_bytes(int nb) { return 2 * static_cast<size_t>(rg_buf_units(nb)) * 16; }

__device__ __forceinline__ int rg_swz(int n) { return ((n & 1) << 2) | ((n >> 1) & 3); }
__device__ __forceinline__ int rg_unit(int n, int t, int g) {
  return 16 * n + 8 * (t & 1) + (((t >> 1) | ((g & 1) << 1) | (((t & 1) ^ (g >> 1)) << 2)) ^ rg_swz(n));
}

template <int V>
using IC = std::integral_constant<int, V>;

// f(IC<0>{}), ..., f(IC<N - 1>{}) in order.
template <typename F, int... I>
__device__ __forceinline__ void rg_static_for(F&& f, std::integer_sequence<int, I...>) {
  (f(IC<I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void rg_static_for(F&& f) {
  rg_static_for(f, std::make_integer_sequence<int, N>{});
}

// Nothing may be scheduled across this point.
__device__ __forceinline__ void rg_fence() { __builtin_amdgcn_sched_barrier(0); }

// Two fp16 bit patterns a (low), b (high) as one dword.
__device__ __forceinline__ uint32_t rg_pack(_Float16 a, _Float16 b) {
  return static_cast<uint32_t>(__builtin_bit_cast(unsigned short, a)) |
         (static_cast<uint32_t>(__builtin_bit_cast(unsigned short, b)) << 16);
}

}  // namespace

// Activations [M][K] (bf16 when BF16, else fp16) to the operand form of
// gemm_q4_k_dqreg: out [M][K] fp16, each group of eight columns in the order
// (0, 2, 1, 3, 4, 6, 5, 7); scale[m] = 2^e, the factor the products of row m
// carry back.  bf16 row m is multiplied by 2^-e with e set from its largest
// |x| (bit patterns with the sign cleared order as the magnitudes do): the
// largest lands in [2^14, 2^15), so no value overflows fp16 and values down
// to 2^-24 of the largest keep full fp16 precision; each value is rounded to
// nearest once.  e = 0 for an all-zero row; e stays within [-126, 127].  One
// workgroup per row; rows of up to 20480 columns are read once and held in
// registers for both the maximum and the conversion, longer ones are read
// twice (the second time from L2).  K a multiple of 8, x and out 16-byte
// aligned.
template <bool BF16>
__global__ void __launch_bounds__(256) act_rows_f16(const uint16_t* x, int K, uint16_t* out, float* scale) {
  constexpr int kHeld = 10;  // 16-byte pieces a thread keeps between the two passes (rows up to 20480 columns)
  __shared__ int wmax[4];
  const int tid = static_cast<int>(threadIdx.x), lane = tid & 63;
  const int row = static_cast<int>(blockIdx.x);
  const uint4* xr = reinterpret_cast<const uint4*>(x + static_cast<size_t>(row) * K);
  uint4* orow = reinterpret_cast<uint4*>(out + static_cast<size_t>(row) * K);
  const int n8 = K >> 3;
  const bool held = n8 <= kHeld * 256;
  uint4 v[kHeld];
  if (held) {
#pragma unroll
    for (int u = 0; u < kHeld; ++u) v[u] = tid + 256 * u < n8 ? xr[tid + 256 * u] : make_uint4(0u, 0u, 0u, 0u);
  }
  int e = 0;
  if constexpr (BF16) {
    u16x2_t m2 = {0, 0};
    auto fold = [&](const uint4& q) {
      m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2_t, q.x & 0x7FFF7FFFu));
      m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2_t, q.y & 0x7FFF7FFFu));
      m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2_t, q.z & 0x7FFF7FFFu));
      m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2_t, q.w & 0x7FFF7FFFu));
    };
    if (held) {
#pragma unroll
      for (int u = 0; u < kHeld; ++u) fold(v[u]);  // the zero fill adds nothing to a maximum
    } else {
      int i = tid;
      for (; i + 3 * 256 < n8; i += 4 * 256) {
        uint4 q[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) q[u] = xr[i + 256 * u];
#pragma unroll
        for (int u = 0; u < 4; ++u) fold(q[u]);
      }
      for (; i < n8; i += 256) fold(xr[i]);
    }
    int mx = max(static_cast<int>(m2.x), static_cast<int>(m2.y));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = max(mx, __shfl_xor(mx, o));
    if (lane == 0) wmax[tid >> 6] = mx;
    __syncthreads();
    mx = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
    // the largest lies in [2^E, 2^(E+1)) with E = (bits >> 7) - 127
    e = mx == 0 ? 0 : (mx >> 7) - 127 - 14;
    e = e < -126 ? -126 : (e > 127 ? 127 : e);
  }
  const float s = __builtin_amdgcn_ldexpf(1.f, -e);
  auto convert = [&](const uint4& q) {  // (x0 x1) (x2 x3) (x4 x5) (x6 x7)
    if constexpr (BF16) {
      const uint32_t w[4] = {q.x, q.y, q.z, q.w};
      _Float16 h[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        h[2 * k] = static_cast<_Float16>(__builtin_bit_cast(float, w[k] << 16) * s);
        h[2 * k + 1] = static_cast<_Float16>(__builtin_bit_cast(float, w[k] & 0xFFFF0000u) * s);
      }
      return make_uint4(rg_pack(h[0], h[2]), rg_pack(h[1], h[3]), rg_pack(h[4], h[6]), rg_pack(h[5], h[7]));
    } else {
      return make_uint4(__builtin_amdgcn_perm(q.y, q.x, 0x05040100u), __builtin_amdgcn_perm(q.y, q.x, 0x07060302u),
                        __builtin_amdgcn_perm(q.w, q.z, 0x05040100u), __builtin_amdgcn_perm(q.w, q.z, 0x07060302u));
    }
  };
  if (held) {
#pragma unroll
    for (int u = 0; u < kHeld; ++u)
      if (tid + 256 * u < n8) orow[tid + 256 * u] = convert(v[u]);
  } else {
    for (int i = tid; i < n8; i += 256) orow[i] = convert(xr[i]);
  }
  if (tid == 0) scale[row] = __builtin_amdgcn_ldexpf(1.f, e);
}

// T: 16-row weight tiles per wave.  NB: 16-row activation (B) tiles per
// workgroup.  XD: activation loads run XD half blocks ahead (1 or 2).  CD:
// code loads run CD half blocks ahead (1 or 2).  PL: plane layout.  mats:
// one to kDqregMaxMats matrices of K columns against the same activations,
// the row tiles of matrix i being blockIdx.x = tile0[i] .. tile0[i + 1];
// x: the activations in act_rows_f16's form; xs[m]: the factor of row m.
// Blocks kb0 = z bps .. min(kb0 + bps, K / 256) of the slice z = blockIdx.z;
// out[i]: matrix i's y when there is one slice, else its partial outputs of
// slice z at out[i] + z zs[i] ([M][N] each).  All byte offsets fit in 32
// bits (checked by the launcher).
struct DqregMats {
  const uint8_t* w[kDqregMaxMats];
  float* out[kDqregMaxMats];
  size_t zs[kDqregMaxMats];
  uint32_t pa[kDqregMaxMats];
  int n[kDqregMaxMats];
  int tile0[kDqregMaxMats + 1];
  int count;
};

template <int T, int NB, int XD, int CD, bool PL>
__global__ void __launch_bounds__(kRgThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_q4_k_dqreg(const DqregMats mats, int K, const uint16_t* x, const float* xs, int M, int bps) {
  constexpr int kBatch = rg_batch(NB), kBufUnits = rg_buf_units(NB);
  constexpr int RS = NB / 4;  // activation rows staged per lane
  extern __shared__ __attribute__((aligned(16))) uint4 rg_lds[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nb = K >> 8;
  const int kb0 = static_cast<int>(blockIdx.z) * bps;
  const int kb1 = min(kb0 + bps, nb);
  const int m0 = static_cast<int>(blockIdx.y) * kBatch;
  const int g = lane >> 4, r16 = lane & 15;
  const uint8_t* xbytes = reinterpret_cast<const uint8_t*>(x);
  // this workgroup's matrix (blockIdx.x is uniform, so is mi)
  int mi = 0;
#pragma unroll
  for (int k = 1; k < kDqregMaxMats; ++k) mi += k < mats.count && static_cast<int>(blockIdx.x) >= mats.tile0[k];
  const uint8_t* w = mats.w[mi];
  const uint32_t pa = mats.pa[mi];
  const int N = mats.n[mi];
  float* y = mats.out[mi] + blockIdx.z * mats.zs[mi];

  // Weight role: tile i of this wave is weight rows nw0 + 16 i .. + 16; lane
  // (g, r16) loads row nw0 + 16 i + r16 (rows past N re-read the last row,
  // results not stored): per block the header and, for half h, code piece
  // 16 (g & 1) of chunk 2h + (g >> 1).
  const int nw0 = (static_cast<int>(blockIdx.x) - mats.tile0[mi]) * (64 * T) + wave * (16 * T);
  uint32_t bidx[T];  // block index of the row's block 0
#pragma unroll
  for (int i = 0; i < T; ++i) bidx[i] = static_cast<uint32_t>(min(nw0 + 16 * i + r16, N - 1)) * nb;

  uint4 hdr[T];            // header of the next block to decode
  uint4 qc[CD][2][T];      // code pieces [block parity (CD = 2)][half][tile]
  uint32_t scl[T][2][2];   // [tile][half h][nibble]: (fp16(d sc), -fp16(dmin m)) of sub-block 2c + nibble
  // The code pieces of half h of block b into ring slot (sp, h) (loads past
  // the slice read the next blocks, up to the last, unused).
  auto load_codes = [&](int b, auto sp_c, auto h_c) {
    constexpr int sp = decltype(sp_c)::value, h = decltype(h_c)::value;
    const uint32_t bc = static_cast<uint32_t>(min(b, nb - 1));
#pragma unroll
    for (int i = 0; i < T; ++i) {
      const uint32_t blk = bidx[i] + bc;
      if constexpr (PL)
        qc[sp][h][i] = ld16(w + (((g & 1) ? 5u * pa : pa) + 64u * blk + 32u * h + 16u * (g >> 1)));
      else
        qc[sp][h][i] = ld16(w + (144u * blk + 16u + 64u * h + 16u * g));
    }
  };
  auto load_header = [&](int b) {
    const uint32_t bc = static_cast<uint32_t>(min(b, nb - 1));
#pragma unroll
    for (int i = 0; i < T; ++i) hdr[i] = ld16(w + (PL ? 16u : 144u) * (bidx[i] + bc));
  };
  auto decode = [&]() {
#pragma unroll
    for (int i = 0; i < T; ++i) {
      const uint4 h = hdr[i];
      const float d = f16_to_f32(h.x & 0xFFFFu), dmin = f16_to_f32(h.x >> 16);
      // byte j of the low / high words: the 6-bit scale or min of sub-block j / 4 + j
      const uint32_t scw[2] = {h.y & 0x3F3F3F3Fu, (h.w & 0x0F0F0F0Fu) | ((h.y >> 2) & 0x30303030u)};
      const uint32_t mw[2] = {h.z & 0x3F3F3F3Fu, ((h.w >> 4) & 0x0F0F0F0Fu) | ((h.z >> 2) & 0x30303030u)};
      const int sh = 16 * (g >> 1);  // sub-blocks 2 (g >> 1) + (0, 1) of each word
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        // shifted once, so that each value is one byte-to-float conversion
        const uint32_t sw = scw[hh] >> sh, mh = mw[hh] >> sh;
#pragma unroll
        for (int nib = 0; nib < 2; ++nib) {
          const float sc = static_cast<float>((sw >> (8 * nib)) & 0xFFu);
          const float mm = static_cast<float>((mh >> (8 * nib)) & 0xFFu);
          const h2_t v = {static_cast<_Float16>(d * sc), static_cast<_Float16>(-(dmin * mm))};
          scl[i][hh][nib] = __builtin_bit_cast(uint32_t, v);
        }
      }
    }
  };

  // Staging role: lane 4 q + gs of the wave copies the 8-column pieces
  // 4 k + gs (k = 0..3) of the half of activation rows n = 16 wave + q + 64 s
  // (s < RS; rows past M re-read the last row): the four lanes of a row read
  // 64 consecutive bytes per load instruction.
  const int gs = lane & 3, ns = 16 * wave + (lane >> 2);
  uint32_t xoff[RS];  // byte offset of (row, column 8 gs)
#pragma unroll
  for (int s = 0; s < RS; ++s)
    xoff[s] = 2u * (static_cast<uint32_t>(min(m0 + ns + 64 * s, M - 1)) * static_cast<uint32_t>(K) + 8u * gs);
  uint4 xr[XD][RS][4];  // pieces in flight [ring slot][row][k]
  // Loads of half block H (clamped to the last): columns 128 H + 32 k + 8 gs.
  auto load_x = [&](int H, auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    const uint32_t kb = 256u * static_cast<uint32_t>(min(H, 2 * nb - 1));
#pragma unroll
    for (int s = 0; s < RS; ++s)
#pragma unroll
      for (int k = 0; k < 4; ++k) xr[slot][s][k] = ld16(xbytes + (xoff[s] + kb + 64u * k));
  };
  // Staging chunk c of a half: piece k of row r (columns 32 k + 8 gs of the
  // half: step t = 2 (gs & 1) + (k & 1), k-group g = 2 (k >> 1) + (gs >> 1)).
  constexpr int kChunks = 4 * RS;
  auto chunk = [&](auto c_c, auto xs_c, auto nx_c) {
    constexpr int c = decltype(c_c)::value, xsl = decltype(xs_c)::value, nx = decltype(nx_c)::value;
    constexpr int r = c / 4, k = c % 4;
    const int n = ns + 64 * r;
    rg_lds[nx * kBufUnits + rg_unit(n, 2 * (gs & 1) + (k & 1), 2 * (k >> 1) + (gs >> 1))] = xr[xsl][r][k];
  };

  f32x4_t acc[T][NB];

  // LDS unit offsets of this lane's B operand reads, per step
  int bofs[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) bofs[t] = rg_unit(r16, t, g);

  // B operand j of step t of a half from LDS buffer par.
  auto read_b = [&](auto par_c, auto t_c, int j) -> h8_t {
    constexpr int par = decltype(par_c)::value, t = decltype(t_c)::value;
    return __builtin_bit_cast(h8_t, rg_lds[par * kBufUnits + bofs[t] + 256 * j]);
  };
  // The code mask and the fp16(1024) pattern in registers the compiler cannot
  // fold back into literals: a VOP3 instruction takes no literal on this
  // architecture, so as literals every (q & mask) | magic needed an AND and an
  // OR; from an SGPR and a VGPR it is one v_and_or_b32.
  uint32_t kmask, kmagic;
  __asm__ volatile("s_mov_b32 %0, 0x000f000f" : "=s"(kmask));
  __asm__ volatile("v_mov_b32 %0, 0x64006400" : "=v"(kmagic));
  // Pair q (of four) of the A operand of tile i for step t of a half: codes
  // qc[cpar][par].  Pairs 0, 1 come from the step's first code dword, 2, 3
  // from its second; odd pairs take the codes 8 bits up.
  auto dq_pair = [&](auto cpar_c, auto par_c, auto t_c, auto i_c, auto q_c) -> h2_t {
    constexpr int cpar = decltype(cpar_c)::value, par = decltype(par_c)::value, t = decltype(t_c)::value;
    constexpr int i = decltype(i_c)::value, q = decltype(q_c)::value;
    constexpr int sh = 4 * (t & 1) + 8 * (q & 1);
    const h2_t off = {static_cast<_Float16>(-1024.f), static_cast<_Float16>(-1024.f)};
    const uint4 c4 = qc[CD == 2 ? cpar : 0][par][i];
    const uint32_t qd = q < 2 ? ((t >> 1) ? c4.z : c4.x) : ((t >> 1) ? c4.w : c4.y);
    const h2_t sc = __builtin_bit_cast(h2_t, scl[i][par][t & 1]);
    const h2_t ds = {sc.x, sc.x}, dm = {sc.y, sc.y};
    const uint32_t a = ((qd >> sh) & kmask) | kmagic;
    return __builtin_elementwise_fma(__builtin_bit_cast(h2_t, a) + off, ds, dm);
  };
  auto pack_a = [](const h2_t(&wq)[4]) {
    return h8_t{wq[0].x, wq[0].y, wq[1].x, wq[1].y, wq[2].x, wq[2].y, wq[3].x, wq[3].y};
  };
  // Slots behind the products of a tile: behind product j, a quarter of the
  // next A operand when j % QG == 0 (QG = NB / 4), else a staging slot; in
  // the last step the last tile forms no next A operand and every slot
  // stages.  Staging slots per step: T (NB - 4), plus 4 in the last step.
  constexpr int QG = NB / 4;
  // The products of step t of a half, in a fixed order of groups of four:
  // each product is written with a little VALU work behind it, and the
  // compiler interleaves the instructions within a group of four products
  // (fences between groups; one fence per product kept every dependent
  // VALU chain in line with its product and was 7 % slower).  a_cur holds
  // tile 0's A operand and leaves with the next step's; bb holds the B
  // operands, and behind the last tile's product j the next step's operand
  // j is read into the register that product has finished with.  stage(c)
  // runs staging slot c of the step.
  auto mstep = [&](auto cpar_c, auto par_c, auto t_c, h8_t(&bb)[NB], h8_t& a_cur, auto&& stage) {
    constexpr int t = decltype(t_c)::value;
    constexpr int tn = t < 3 ? t + 1 : 3;
    rg_static_for<T>([&](auto i_c) {
      constexpr int i = decltype(i_c)::value;
      constexpr bool next_a = i + 1 < T || t < 3;
      h2_t wq[4];
      rg_static_for<NB>([&](auto j_c) {
        constexpr int j = decltype(j_c)::value;
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_cur, bb[j], acc[i][j], 0, 0, 0);
        if constexpr (i + 1 == T && t < 3) bb[j] = read_b(par_c, IC<tn>{}, j);
        if constexpr (j % QG == 0 && next_a) {
          if constexpr (i + 1 < T)
            wq[j / QG] = dq_pair(cpar_c, par_c, t_c, IC<i + 1>{}, IC<j / QG>{});
          else
            wq[j / QG] = dq_pair(cpar_c, par_c, IC<tn>{}, IC<0>{}, IC<j / QG>{});
        } else {
          stage(IC<i*(NB - 4) + (next_a ? (j / QG) * (QG - 1) + (j % QG) - 1 : j)>{});
        }
        if constexpr (j % 4 == 3) rg_fence();
      });
      if constexpr (next_a) a_cur = pack_a(wq);
      rg_fence();
    });
  };

  // Half block H = 2 b + par of block b (codes in set cpar): loads for the
  // halves ahead, the four steps with the next half's staging in their free
  // slots, barrier.
  auto half = [&](int H, auto cpar_c, auto par_c) {
    constexpr int par = decltype(par_c)::value;
    // activations of half H + XD into ring slot (H + XD) & (XD - 1); with a
    // one-half code distance, the next half's code pieces
    load_x(H + XD, IC<XD == 2 ? par : 0>{});
    if constexpr (CD == 1) load_codes((H + 1) >> 1, IC<0>{}, IC<par ^ 1>{});
    h8_t bb[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) bb[j] = read_b(par_c, IC<0>{}, j);
    h8_t a_cur;
    {
      h2_t wq[4];
      rg_static_for<4>([&](auto q_c) { wq[decltype(q_c)::value] = dq_pair(cpar_c, par_c, IC<0>{}, IC<0>{}, q_c); });
      a_cur = pack_a(wq);
    }
    // The next half's staging (ring slot xsl, LDS buffer par ^ 1) in the
    // slots of steps t0..3: every step when its activations were loaded two
    // halves ahead, the last two when one half ahead.
    constexpr int nx = par ^ 1, xsl = XD == 2 ? nx : 0, t0 = XD == 2 ? 0 : 2;
    constexpr int per_step = T * (NB - 4);
    constexpr int slots = (3 - t0) * per_step + per_step + 4;
    constexpr int cps = (kChunks + slots - 1) / slots;  // chunks per slot
    auto stage_in = [&](auto t_c) {
      constexpr int t = decltype(t_c)::value;
      return [&](auto c_c) {
        constexpr int c = decltype(c_c)::value;
        if constexpr (t >= t0) {
          constexpr int slot = (t - t0) * per_step + c;
          rg_static_for<cps>([&](auto k_c) {
            constexpr int ch = slot * cps + decltype(k_c)::value;
            if constexpr (ch < kChunks) chunk(IC<ch>{}, IC<xsl>{}, IC<nx>{});
          });
        }
      };
    };
    mstep(cpar_c, par_c, IC<0>{}, bb, a_cur, stage_in(IC<0>{}));
    mstep(cpar_c, par_c, IC<1>{}, bb, a_cur, stage_in(IC<1>{}));
    mstep(cpar_c, par_c, IC<2>{}, bb, a_cur, stage_in(IC<2>{}));
    mstep(cpar_c, par_c, IC<3>{}, bb, a_cur, stage_in(IC<3>{}));
    lds_barrier();
  };
  auto block = [&](int b, auto cpar_c) {
    constexpr int cpar = decltype(cpar_c)::value;
    decode();
    load_header(b + 1);
    if constexpr (CD == 2) {
      load_codes(b + 1, IC<cpar ^ 1>{}, IC<0>{});
      load_codes(b + 1, IC<cpar ^ 1>{}, IC<1>{});
    }
    half(2 * b, cpar_c, IC<0>{});
    half(2 * b + 1, cpar_c, IC<1>{});
  };

#pragma unroll
  for (int i = 0; i < T; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // Prologue: the first block's codes and header, the first halves of X in
  // flight, the first half staged.
  load_header(kb0);
  load_codes(kb0, IC<0>{}, IC<0>{});
  if constexpr (CD == 2) load_codes(kb0, IC<0>{}, IC<1>{});
  load_x(2 * kb0, IC<0>{});
  if constexpr (XD == 2) load_x(2 * kb0 + 1, IC<1>{});
  rg_static_for<kChunks>([&](auto c_c) { chunk(c_c, IC<0>{}, IC<0>{}); });
  lds_barrier();
  // The last half stages a half past the slice (loads clamped to the last
  // half of K, never multiplied).
  int b = kb0;
#pragma unroll 1
  for (; b + 2 <= kb1; b += 2) {
    block(b, IC<0>{});
    block(b + 1, IC<1>{});
  }
  if (b < kb1) block(b, IC<0>{});

  // Lane (g, r16) holds outputs n .. n + 3 (n = 16 i + 4 g) of activation
  // row 16 j + r16: one 16-byte store when the row length keeps it aligned
  // (scattered 4-byte stores cost about a fifth of the kernel at five tiles).
  const bool row4 = (N & 3) == 0;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int m = m0 + 16 * j + r16;
    if (m < M) {
      const float fs = xs[m];
      float* yr = y + static_cast<size_t>(m) * N;
#pragma unroll
      for (int i = 0; i < T; ++i) {
        const int n = nw0 + 16 * i + 4 * g;
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

// For item i = blockIdx.y: y[e] = the sum over s < S of part[s zs + e] in
// order of s, for e < n (zs a multiple of 4; part and y 16-byte aligned).
struct DqregSums {
  const float* part[kDqregMaxMats];
  float* y[kDqregMaxMats];
  size_t zs[kDqregMaxMats];
  size_t n[kDqregMaxMats];
};

__global__ void __launch_bounds__(256) dqreg_sum(const DqregSums items, int S) {
  const int it = static_cast<int>(blockIdx.y);
  const float* part = items.part[it];
  float* y = items.y[it];
  const size_t zs = items.zs[it], n = items.n[it];
  const size_t n4 = n / 4, z4 = zs / 4;
  const f32x4_t* p = reinterpret_cast<const f32x4_t*>(part);
  f32x4_t* o = reinterpret_cast<f32x4_t*>(y);
  const size_t i0 = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x;
  const size_t step = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = i0; i < n4; i += step) {
    f32x4_t v = p[i];
    for (int s = 1; s < S; ++s) v += p[s * z4 + i];
    o[i] = v;
  }
  for (size_t e = 4 * n4 + i0; e < n; e += step) {
    float v = part[e];
    for (int s = 1; s < S; ++s) v += part[s * zs + e];
    y[e] = v;
  }
}

namespace {

// Prefetch distances: activations and codes two half blocks ahead up to
// two tiles per wave, else one.  From three tiles a step is long enough to
// cover the loads, and the registers of a second half in flight cost more
// than they save (measured at four tiles: 202 against 184 us on the 7B FFN
// gate at 512 rows).
constexpr int rg_xd(int t) { return t >= 3 ? 1 : 2; }

size_t rg_align(size_t v) { return (v + 255) / 256 * 256; }
// Floats from one slice's partial outputs to the next: 256-byte aligned.
size_t rg_slice_floats(int64_t rows, int64_t batch) { return rg_align(static_cast<size_t>(rows) * batch * 4) / 4; }

template <int T, int NB>
hipError_t launch_dqreg(const DqregMats& mats, int K, const uint16_t* x16, const float* xs, int M, int splits,
                        int bps, bool pl, hipStream_t stream) {
  constexpr int D = rg_xd(T);
  const dim3 grid(mats.tile0[mats.count], (M + rg_batch(NB) - 1) / rg_batch(NB), splits);
  const size_t lds = rg_lds_bytes(NB);
  if (pl)
    hipLaunchKernelGGL((gemm_q4_k_dqreg<T, NB, D, D, true>), grid, dim3(kRgThreads), lds, stream, mats, K, x16, xs, M,
                       bps);
  else
    hipLaunchKernelGGL((gemm_q4_k_dqreg<T, NB, D, D, false>), grid, dim3(kRgThreads), lds, stream, mats, K, x16, xs,
                       M, bps);
  return hipGetLastError();
}

template <int NB>
hipError_t launch_dqreg_t(int t, const DqregMats& mats, int K, const uint16_t* x16, const float* xs, int M,
                          int splits, int bps, bool pl, hipStream_t stream) {
  switch (t) {
    case 1: return launch_dqreg<1, NB>(mats, K, x16, xs, M, splits, bps, pl, stream);
    case 2: return launch_dqreg<2, NB>(mats, K, x16, xs, M, splits, bps, pl, stream);
    case 3: return launch_dqreg<3, NB>(mats, K, x16, xs, M, splits, bps, pl, stream);
    case 4: return launch_dqreg<4, NB>(mats, K, x16, xs, M, splits, bps, pl, stream);
    default: return launch_dqreg<5, NB>(mats, K, x16, xs, M, splits, bps, pl, stream);
  }
}

// Modelled time (us) of one launch: workgroup rounds over the compute units
// times a workgroup's time, (14 + 17 / T) ns per product of a wave at
// NB = 8 and (20 + 16 / T) ns at NB = 4 (where each A operand serves four
// products), plus 5.5 us of prologue and epilogue; with several slices, the
// sum kernel, 3 us plus the partial outputs read and y written once at
// 8 TB/s.  Fitted to kernel traces of the 7B layer's matrices at 128 to 512
// rows (T = 1..5, 2 to 74 blocks per slice: within 10 %).
double dqreg_cost(const int64_t* rows, int n, int64_t batch, int64_t cus, int t, int nbt, int splits, int bps) {
  int64_t tiles = 0, all_rows = 0;
  for (int i = 0; i < n; ++i) {
    tiles += (rows[i] + 64 * t - 1) / (64 * t);
    all_rows += rows[i];
  }
  const int64_t wgs = tiles * ((batch + rg_batch(nbt) - 1) / rg_batch(nbt)) * splits;
  const double products = static_cast<double>(bps) * 8 * nbt * t;
  const double per = nbt == 4 ? 20.0 + 16.0 / t : 14.0 + 17.0 / t;
  double us = static_cast<double>((wgs + cus - 1) / cus) * (products * per * 1e-3 + 5.5);
  if (splits > 1) us += 3.0 + static_cast<double>(splits + 1) * all_rows * batch * 4 / 8e6;
  return us;
}

}  // namespace

bool dqreg_eligible(const qmv_weights& W, int64_t batch) {
  if (W.fmt != QMV_Q4_K || W.rows < kDqMinRows || batch < kDqMinBatchRun) return false;
  const uint64_t wbytes = W.layout == QMV_LAYOUT_PLANES ? 5 * W.scales_offset + 64 * (W.rows * (W.cols / 256))
                                                        : 144 * static_cast<uint64_t>(W.rows) * (W.cols / 256);
  return wbytes < (1ull << 32) && 2 * static_cast<uint64_t>(batch) * W.cols < (1ull << 32);
}

DqregPlan dqreg_plan(const int64_t* rows, int n, int64_t cols, int64_t batch) {
  const int64_t cus = device_cus();
  const int nb = static_cast<int>(cols / 256);
  DqregPlan best{1, 8, 1, nb};
  double best_us = -1;
  for (int nbt : {8, 4})
    for (int t = 1; t <= 5; ++t)
      for (int s = 1; s <= kDqregMaxSplits && s <= nb; ++s) {
        const int bps = (nb + s - 1) / s;
        const int splits = (nb + bps - 1) / bps;  // every slice holds at least one block
        if (splits != s) continue;
        const double us = dqreg_cost(rows, n, batch, cus, t, nbt, splits, bps);
        if (best_us < 0 || us < best_us) {
          best = DqregPlan{t, nbt, splits, bps};
          best_us = us;
        }
      }
  return best;
}

size_t dqreg_workspace_bytes(const int64_t* rows, int n, int64_t cols, int64_t batch, const DqregPlan& p) {
  size_t b = rg_align(static_cast<size_t>(batch) * cols * 2) + rg_align(static_cast<size_t>(batch) * 4);
  if (p.splits > 1)
    for (int i = 0; i < n; ++i) b += static_cast<size_t>(p.splits) * rg_slice_floats(rows[i], batch) * 4;
  return b;
}

hipError_t gemm_q4_k_dqreg_ws(const GemvCall* calls, int n, bool f16x, int64_t batch, const DqregPlan& p, void* ws,
                              bool convert, hipStream_t stream) {
  const int M = static_cast<int>(batch), K = static_cast<int>(calls[0].W->cols);
  uint8_t* base = static_cast<uint8_t*>(ws);
  uint16_t* x16 = reinterpret_cast<uint16_t*>(base);
  float* xs = reinterpret_cast<float*>(base + rg_align(static_cast<size_t>(M) * K * 2));
  float* part = reinterpret_cast<float*>(base + rg_align(static_cast<size_t>(M) * K * 2) +
                                         rg_align(static_cast<size_t>(M) * 4));
  hipError_t e = hipSuccess;
  if (convert) {
    const uint16_t* x = static_cast<const uint16_t*>(calls[0].x);
    if (f16x)
      hipLaunchKernelGGL((act_rows_f16<false>), dim3(M), dim3(256), 0, stream, x, K, x16, xs);
    else
      hipLaunchKernelGGL((act_rows_f16<true>), dim3(M), dim3(256), 0, stream, x, K, x16, xs);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  DqregMats mats{};
  DqregSums sums{};
  mats.count = n;
  size_t n_max = 0;
  for (int i = 0; i < n; ++i) {
    const qmv_weights& W = *calls[i].W;
    mats.w[i] = static_cast<const uint8_t*>(W.data);
    mats.pa[i] = static_cast<uint32_t>(W.scales_offset);
    mats.n[i] = static_cast<int>(W.rows);
    mats.tile0[i + 1] = mats.tile0[i] + static_cast<int>((W.rows + 64 * p.t - 1) / (64 * p.t));
    mats.zs[i] = rg_slice_floats(W.rows, M);
    if (p.splits > 1) {
      mats.out[i] = part;
      sums.part[i] = part;
      sums.y[i] = calls[i].y;
      sums.zs[i] = mats.zs[i];
      sums.n[i] = static_cast<size_t>(M) * W.rows;
      n_max = std::max(n_max, sums.n[i]);
      part += static_cast<size_t>(p.splits) * mats.zs[i];
    } else {
      mats.out[i] = calls[i].y;
    }
  }
  const bool pl = calls[0].W->layout == QMV_LAYOUT_PLANES;
  e = p.nb == 4 ? launch_dqreg_t<4>(p.t, mats, K, x16, xs, M, p.splits, p.bps, pl, stream)
                : launch_dqreg_t<8>(p.t, mats, K, x16, xs, M, p.splits, p.bps, pl, stream);
  if (e != hipSuccess || p.splits == 1) return e;
  const int blocks = static_cast<int>(std::min<size_t>((n_max / 4 + 255) / 256 + 1, 4096));
  hipLaunchKernelGGL(dqreg_sum, dim3(blocks, n), dim3(256), 0, stream, sums, p.splits);
  return hipGetLastError();
}

// The fixed workspace of qmv_gemv_noalloc, for callers that cannot allocate:
// one copy per device, held from module load until the process ends.  In
// host code `scratch` only names the symbol; its device address, per device,
// comes from hipGetSymbolAddress on the first use there.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

hipError_t scratch_workspace(size_t bytes, void** out) {
  if (bytes > kScratchBytes) return hipErrorOutOfMemory;
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return hipSuccess;
}

namespace {

// The register-dequantized runs of a launch's matrix-core calls: reg[i] for
// calls on those kernels, run[i] the calls in the run starting at i (0 inside
// a run), plans[i] its plan; returns the workspace bytes the runs need (they
// run one after another in one workspace).
size_t plan_runs(const GemvCall* calls, int n, int64_t batch, bool* reg, int* run, DqregPlan* plans) {
  size_t bytes = 0;
  for (int i = 0; i < n; ++i) reg[i] = dqreg_eligible(*calls[i].W, batch);
  for (int i = 0; i < n;) {
    int k = 1;
    if (reg[i]) {
      while (i + k < n && k < kDqregMaxMats && reg[i + k] && calls[i + k].x == calls[i].x &&
             calls[i + k].W->cols == calls[i].W->cols && calls[i + k].W->layout == calls[i].W->layout)
        ++k;
      // a lone matrix below kDqMinBatch rows stays on the tile kernels
      // unless its K is long
      if (k == 1 && batch < kDqMinBatch && calls[i].W->cols < kDqLongK) reg[i] = false;
    }
    run[i] = k;
    for (int j = 1; j < k; ++j) run[i + j] = 0;
    if (reg[i]) {
      int64_t rows[kDqregMaxMats];
      for (int j = 0; j < k; ++j) rows[j] = calls[i + j].W->rows;
      plans[i] = dqreg_plan(rows, k, calls[i].W->cols, batch);
      bytes = std::max(bytes, dqreg_workspace_bytes(rows, k, calls[i].W->cols, batch, plans[i]));
    }
    i += k;
  }
  return bytes;
}

}  // namespace

size_t gemm_q4_k_mfma_items_workspace(const GemvCall* calls, int n, int64_t batch) {
  bool reg[kMaxItems];
  int run[kMaxItems];
  DqregPlan plans[kMaxItems];
  return plan_runs(calls, n, batch, reg, run, plans);
}

hipError_t gemm_q4_k_mfma_items(const GemvCall* calls, int n, bool f16x, int64_t batch, hipStream_t stream,
                                void* ws) {
  // runs of consecutive register-dequantized calls on the same activations
  // and widths (up to kDqregMaxMats) share one conversion, one product
  // launch and one sum launch; without a workspace every call takes the
  // kernels of gemm_q4_k_bf16 / gemm_q4_k_f16
  bool reg[kMaxItems];
  int run[kMaxItems];
  DqregPlan plans[kMaxItems];
  if (ws) {
    plan_runs(calls, n, batch, reg, run, plans);
  } else {
    for (int i = 0; i < n; ++i) {
      reg[i] = false;
      run[i] = 1;
    }
  }
  hipError_t e = hipSuccess;
  const GemvCall* converted = nullptr;  // the run whose activations the workspace holds
  for (int i = 0; i < n && e == hipSuccess; i += run[i]) {
    const GemvCall& c = calls[i];
    if (reg[i]) {
      const bool same = converted && converted->x == c.x && converted->W->cols == c.W->cols;
      e = gemm_q4_k_dqreg_ws(calls + i, run[i], f16x, batch, plans[i], ws, !same, stream);
      converted = &c;
    } else {
      e = f16x ? gemm_q4_k_f16(*c.W, c.x, c.y, batch, stream) : gemm_q4_k_bf16(*c.W, c.x, c.y, batch, stream);
      converted = nullptr;
    }
  }
  return e;
}

}  // namespace qmv
