// Batched Q4_K on the gfx950 matrix cores, weights dequantized into operand
// registers: Y[m][n] = sum_k X[m][k] W[n][k] for a hundred or more activation
// rows X (bf16 or fp16) and Q4_K weights W (canonical or plane layout),
// y layout [batch][rows].
//
// The batched-prefill reading of the pages' kernel families (hipEngine
// "Quickstart": matrix-core prefill beside GEMV decode): once a weight meets
// a hundred or more activation rows, it is cheaper to convert it to the
// matrix-core type once than to apply its scales to every product.
//
// Workgroup: four waves, one per SIMD.  Wave w owns 16 T consecutive weight
// rows (T tiles of 16) and all 16 NB activation rows of the workgroup's batch
// tile (NB = 8 or 16 B tiles).  Each wave dequantizes its own weight tiles
// straight into A operand registers: weights never pass through LDS and are
// converted once.  The activation tile is converted to fp16 once per
// workgroup into LDS, where all four waves read it as B operands.  Per
// 32-column step a wave issues NB T v_mfma_f32_16x16x32_f16 against NB LDS
// reads.
//
// What sets the time (measured on gfx950 with an issue probe): one wave
// issues about two independent VALU instructions under each 16-cycle
// product for free; beyond that the VALU issue sets the pace.  Forming an A
// operand costs about 16 VALU instructions (two per product at NB = 8, one
// at NB = 16); converting the activation tile costs about 3 per value, i.e.
// about 6 / T per product.  The host picks (T, NB) per shape from that and
// from how many workgroups fill the compute units.
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
// Activations are staged per half block (16 NB rows x 128 columns of fp16)
// into one of two LDS buffers, one barrier per half block; their loads run
// one or two half blocks ahead.  bf16 rows are scaled by a power of two 2^-e
// fixed per row for the whole of K: e is set from the row's largest |x| in
// the first half block with 8 bits of headroom (and at least -112), so that
// the fp16 copy is exact from 256 times that maximum down to 2^-20 of it;
// the conversion is integer arithmetic on the bit patterns (exponent minus
// 112 + e, saturating at zero, mantissa moved up three bits), and bf16
// subnormals become zero.  Every later half block checks its own maximum
// against the headroom; if any row of the workgroup would overflow, the
// workgroup computes its tile once more with each row's e taken from its
// largest |x| over all of K (found on the first pass).  A rising magnitude
// along K costs a second pass; no accumulator is ever rescaled.  Results are
// multiplied by 2^e at the end.  fp16 activations enter as given.
//
// LDS unit (16 bytes) of activation row n, step t of the half, k-group g:
// 16 n + 8 (t & 1) + (f(t, g) ^ s(n)) with f(t, g) = (t >> 1) + 2 (g & 1) +
// 4 ((t & 1) ^ (g >> 1)) and s(n) = 4 (n & 1) + ((n >> 1) & 3).  The operand
// reads (eight rows at one (t, g)) and the staging stores (two rows, four
// consecutive 16-byte pieces each) both land any eight lanes of a row of the
// wave on eight different 16-byte bank groups of a 128-byte line.
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
constexpr int kRgHeadroom = 8;   // bits of bf16 row-scale headroom over the first half block

__host__ __device__ constexpr int rg_batch(int nb) { return 16 * nb; }
__host__ __device__ constexpr int rg_buf_units(int nb) { return rg_batch(nb) * kRgRowUnits; }
__host__ __device__ constexpr size_t rg_lds_bytes(int nb) {
  return 2 * static_cast<size_t>(rg_buf_units(nb)) * 16 + rg_batch(nb) * sizeof(float) + 16;
}

__device__ __forceinline__ int rg_swz(int n) { return ((n & 1) << 2) | ((n >> 1) & 3); }
__device__ __forceinline__ int rg_unit(int n, int t, int g) {
  return 16 * n + 8 * (t & 1) + (((t >> 1) | ((g & 1) << 1) | (((t & 1) ^ (g >> 1)) << 2)) ^ rg_swz(n));
}

// Exponent index of a row's largest |x| (from its sign-cleared bf16 bit
// patterns, the four lanes of the row combined): eb such that the maximum
// scaled by 2^-eb lies in [2^14, 2^15).
__device__ __forceinline__ int rg_eb(u16x2_t m2) {
  int mx = max(static_cast<int>(m2.x), static_cast<int>(m2.y));
  mx = max(mx, __builtin_amdgcn_update_dpp(0, mx, 0xB1, 0xF, 0xF, false));  // lane ^ 1
  mx = max(mx, __builtin_amdgcn_update_dpp(0, mx, 0x4E, 0xF, 0xF, false));  // lane ^ 2
  const int eb = (mx >> 7) - 127 - 14;  // the maximum lies in [2^E, 2^(E+1)), E = (bits >> 7) - 127
  return eb < -126 ? -126 : (eb > 113 ? 113 : eb);
}

// bf16 pair (sign-cleared m, original v) scaled by 2^-e to an fp16 pair:
// exponent field minus 112 + e (sub = that << 7 in both halves), saturating
// at zero, mantissa up three bits, sign back.
__device__ __forceinline__ uint32_t rg_bf16x2_to_f16x2(uint32_t m, uint32_t v, u16x2_t sub) {
  const u16x2_t t = __builtin_elementwise_sub_sat(__builtin_bit_cast(u16x2_t, m), sub) << 3;
  return __builtin_bit_cast(uint32_t, t) | (v & 0x80008000u);
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

// Nothing may be scheduled across this point: the instruction order of a
// step is the order written.
__device__ __forceinline__ void rg_fence() { __builtin_amdgcn_sched_barrier(0); }

}  // namespace

// T: 16-row weight tiles per wave.  NB: 16-row activation (B) tiles per
// workgroup, 8 or 16.  XD: activation loads run XD half blocks ahead (1 or
// 2).  CD: code loads run CD half blocks ahead (1 or 2).  PL: plane layout.
// F16X: fp16 activations (else bf16).  All byte offsets fit in 32 bits
// (checked by the launcher).
template <int T, int NB, int XD, int CD, bool PL, bool F16X>
__global__ void __launch_bounds__(kRgThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_q4_k_dqreg(const uint8_t* w, uint32_t pa, int N, int K, const uint16_t* x, float* y, int M) {
  constexpr int kBatch = rg_batch(NB), kBufUnits = rg_buf_units(NB);
  constexpr int RS = NB / 4;  // activation rows staged per lane
  extern __shared__ __attribute__((aligned(16))) uint4 rg_lds[];
  float* fin_lds = reinterpret_cast<float*>(rg_lds + 2 * kBufUnits);  // [activation row]: 2^e
  int* ovf_lds = reinterpret_cast<int*>(fin_lds + kBatch);             // [wave]: a row would overflow

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nb = K >> 8;
  const int m0 = static_cast<int>(blockIdx.y) * kBatch;
  const int g = lane >> 4, r16 = lane & 15;
  const uint8_t* xbytes = reinterpret_cast<const uint8_t*>(x);

  // Weight role: tile i of this wave is weight rows nw0 + 16 i .. + 16; lane
  // (g, r16) loads row nw0 + 16 i + r16 (rows past N re-read the last row,
  // results not stored): per block the header and, for half h, code piece
  // 16 (g & 1) of chunk 2h + (g >> 1).
  const int nw0 = static_cast<int>(blockIdx.x) * (64 * T) + wave * (16 * T);
  uint32_t bidx[T];  // block index of the row's block 0
#pragma unroll
  for (int i = 0; i < T; ++i) bidx[i] = static_cast<uint32_t>(min(nw0 + 16 * i + r16, N - 1)) * nb;

  uint4 hdr[T];            // header of the next block to decode
  uint4 qc[CD][2][T];      // code pieces [block parity (CD = 2)][half][tile]
  uint32_t scl[T][2][2];   // [tile][half h][nibble]: (fp16(d sc), -fp16(dmin m)) of sub-block 2c + nibble
  // The code pieces of half h of block b into ring slot (sp, h).
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
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int nib = 0; nib < 2; ++nib) {
          const float sc = static_cast<float>((scw[hh] >> (sh + 8 * nib)) & 0xFFu);
          const float mm = static_cast<float>((mw[hh] >> (sh + 8 * nib)) & 0xFFu);
          const h2_t v = {static_cast<_Float16>(d * sc), static_cast<_Float16>(-(dmin * mm))};
          scl[i][hh][nib] = __builtin_bit_cast(uint32_t, v);
        }
    }
  };

  // Staging role: lane 4 q + gs of the wave stages the 8-column pieces
  // 4 k + gs (k = 0..3) of the half of activation rows n = 16 wave + q + 64 s
  // (s < RS; rows past M re-read the last row): the four lanes of a row read
  // 64 consecutive bytes per load instruction.
  const int gs = lane & 3, ns = 16 * wave + (lane >> 2);
  uint32_t xoff[RS];  // byte offset of (row, column 8 gs)
#pragma unroll
  for (int s = 0; s < RS; ++s)
    xoff[s] = 2u * (static_cast<uint32_t>(min(m0 + ns + 64 * s, M - 1)) * static_cast<uint32_t>(K) + 8u * gs);
  uint4 xr[XD][RS][4];  // raw pieces [ring slot][row][k]
  // Loads of half block H (clamped to the last): columns 128 H + 32 k + 8 gs.
  auto load_x = [&](int H, auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    const uint32_t kb = 256u * static_cast<uint32_t>(min(H, 2 * nb - 1));
#pragma unroll
    for (int s = 0; s < RS; ++s)
#pragma unroll
      for (int k = 0; k < 4; ++k) xr[slot][s][k] = ld16(xbytes + (xoff[s] + kb + 64u * k));
  };

  // bf16 row scales of this lane's staged rows: the exponent in use, the
  // largest seen over K, the packed exponent subtrahend, and whether a row
  // would overflow.
  int e_fix[RS], e_max[RS];
  u16x2_t esub[RS];
  u16x2_t mrow[RS];  // running |x| maxima over a half
#pragma unroll
  for (int s = 0; s < RS; ++s) {
    e_fix[s] = 0;
    e_max[s] = -126;
    esub[s] = u16x2_t{0, 0};
    mrow[s] = u16x2_t{0, 0};
  }
  uint32_t ovf = 0;
  int pass = 0;
  uint32_t ostage[2] = {0, 0};  // the first two dwords of a piece being converted
  auto set_scale = [&](int s, int e) {
    e_fix[s] = e < -112 ? -112 : (e > 126 ? 126 : e);
    const unsigned short v = static_cast<unsigned short>((112 + e_fix[s]) << 7);
    esub[s] = u16x2_t{v, v};
  };

  // Staging pieces.  store (r, k, h) converts dwords 2 h, 2 h + 1 of piece k
  // of row r (h = 1 stores the piece: columns 32 k + 8 gs of the half, step
  // t = 2 (gs & 1) + (k & 1), k-group g = 2 (k >> 1) + (gs >> 1)), folding
  // the values into the row's running maximum when tracked; check (r) checks
  // the row's maximum against its scale.
  auto store = [&](auto xs_c, auto nx_c, auto r_c, auto k_c, auto h_c, bool track) {
    constexpr int xs = decltype(xs_c)::value, nx = decltype(nx_c)::value, r = decltype(r_c)::value;
    constexpr int k = decltype(k_c)::value, h = decltype(h_c)::value;
    const uint4 v = xr[xs][r][k];  // columns c .. c + 8: (x0 x1) (x2 x3) (x4 x5) (x6 x7)
    const uint32_t lo = h ? v.z : v.x, hi = h ? v.w : v.y;
    uint32_t cl, ch;
    if constexpr (F16X) {
      cl = lo;
      ch = hi;
    } else {
      const uint32_t ml = lo & 0x7FFF7FFFu, mh = hi & 0x7FFF7FFFu;
      if (track) {
        const u16x2_t m = (k == 0 && h == 0) ? u16x2_t{0, 0} : mrow[r];
        mrow[r] = __builtin_elementwise_max(__builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, ml)),
                                            __builtin_bit_cast(u16x2_t, mh));
      }
      cl = rg_bf16x2_to_f16x2(ml, lo, esub[r]);
      ch = rg_bf16x2_to_f16x2(mh, hi, esub[r]);
    }
    const uint32_t o0 = __builtin_amdgcn_perm(ch, cl, 0x05040100u);  // (x0, x2) / (x4, x6)
    const uint32_t o1 = __builtin_amdgcn_perm(ch, cl, 0x07060302u);  // (x1, x3) / (x5, x7)
    if constexpr (h == 0) {
      ostage[0] = o0;
      ostage[1] = o1;
    } else {
      const int n = ns + 64 * r;
      rg_lds[nx * kBufUnits + rg_unit(n, 2 * (gs & 1) + (k & 1), 2 * (k >> 1) + (gs >> 1))] =
          make_uint4(ostage[0], ostage[1], o0, o1);
    }
  };
  auto check = [&](auto r_c) {
    constexpr int r = decltype(r_c)::value;
    const int eb = rg_eb(mrow[r]);
    // values below 2^(eb + 15) stay below 65504 after scaling by 2^-e iff eb <= e + 1
    ovf |= eb > e_fix[r] + 1 ? 1u : 0u;
    e_max[r] = max(e_max[r], eb);
  };
  // The staging chunks of a half: 8 RS stores (tracking the maxima), then RS
  // checks.
  constexpr int kChunks = 8 * RS + (F16X ? 0 : RS);
  auto chunk = [&](auto c_c, auto xs_c, auto nx_c) {
    constexpr int c = decltype(c_c)::value;
    if constexpr (c < 8 * RS)
      store(xs_c, nx_c, IC<c / 8>{}, IC<(c % 8) / 2>{}, IC<c % 2>{}, true);
    else
      check(IC<c - 8 * RS>{});
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
  // The products of step t of a half, in a fixed order: each product is
  // followed by a little VALU work, so that the matrix core runs while the
  // VALU works, with no scheduling heuristics involved.  a_cur holds tile
  // 0's A operand and leaves with the next step's; bb holds the B operands,
  // and behind the last tile's product j the next step's operand j is read
  // into the register that product has finished with.  stage(c) runs staging
  // slot c of the step.
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
        rg_fence();
        if constexpr (j % QG == 0 && next_a) {
          if constexpr (i + 1 < T)
            wq[j / QG] = dq_pair(cpar_c, par_c, t_c, IC<i + 1>{}, IC<j / QG>{});
          else
            wq[j / QG] = dq_pair(cpar_c, par_c, IC<tn>{}, IC<0>{}, IC<j / QG>{});
        } else {
          stage(IC<i*(NB - 4) + (next_a ? (j / QG) * (QG - 1) + (j % QG) - 1 : j)>{});
        }
        rg_fence();
      });
      if constexpr (next_a) a_cur = pack_a(wq);
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
    // The next half's staging (ring slot xs, LDS buffer par ^ 1) in the
    // slots of steps t0..3: every step when its activations were loaded two
    // halves ahead, the last two when one half ahead.
    constexpr int nx = par ^ 1, xs = XD == 2 ? nx : 0, t0 = XD == 2 ? 0 : 2;
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
            if constexpr (ch < kChunks) chunk(IC<ch>{}, IC<xs>{}, IC<nx>{});
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

  for (;; ++pass) {
    // (the address bases pass through an empty asm: otherwise their derived
    // addresses are computed once before this loop and all held live through
    // the block loop)
#pragma unroll
    for (int i = 0; i < T; ++i) __asm__ volatile("" : "+v"(bidx[i]));
#pragma unroll
    for (int s = 0; s < RS; ++s) __asm__ volatile("" : "+v"(xoff[s]));
#pragma unroll
    for (int t = 0; t < 4; ++t) __asm__ volatile("" : "+v"(bofs[t]));
#pragma unroll
    for (int i = 0; i < T; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // Prologue: block 0's codes and header, the first halves of X in flight,
    // half 0 staged (on the first pass its maxima set the row scales first).
    load_header(0);
    load_codes(0, IC<0>{}, IC<0>{});
    if constexpr (CD == 2) load_codes(0, IC<0>{}, IC<1>{});
    load_x(0, IC<0>{});
    if constexpr (XD == 2) load_x(1, IC<1>{});
    if constexpr (!F16X) {
      if (pass == 0) {
        rg_static_for<RS>([&](auto r_c) {
          constexpr int r = decltype(r_c)::value;
          u16x2_t m2 = {0, 0};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint4 v = xr[0][r][k];
            m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2_t, v.x & 0x7FFF7FFFu));
            m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2_t, v.y & 0x7FFF7FFFu));
            m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2_t, v.z & 0x7FFF7FFFu));
            m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2_t, v.w & 0x7FFF7FFFu));
          }
          const int eb = rg_eb(m2);
          e_max[r] = eb;
          set_scale(r, eb + kRgHeadroom);
        });
      }
    }
    rg_static_for<8 * RS>([&](auto c_c) {
      constexpr int c = decltype(c_c)::value;
      store(IC<0>{}, IC<0>{}, IC<c / 8>{}, IC<(c % 8) / 2>{}, IC<c % 2>{}, false);
    });
    lds_barrier();
    // The last half stages a half past the end (clamped loads of the last
    // half, never multiplied; its maximum is the last half's again).
    int b = 0;
#pragma unroll 1
    for (; b + 2 <= nb; b += 2) {
      block(b, IC<0>{});
      block(b + 1, IC<1>{});
    }
    if (b < nb) block(b, IC<0>{});
    if constexpr (F16X) {
      break;
    } else {
      // a second pass only if some row of the workgroup would have overflowed
      if (lane == 0) ovf_lds[wave] = __builtin_amdgcn_ballot_w64(ovf != 0) != 0 ? 1 : 0;
      lds_barrier();
      const bool again = pass == 0 && (ovf_lds[0] | ovf_lds[1] | ovf_lds[2] | ovf_lds[3]) != 0;
      lds_barrier();
      if (!again) break;
#pragma unroll
      for (int s = 0; s < RS; ++s) set_scale(s, e_max[s]);
      ovf = 0;
    }
  }

  if constexpr (!F16X) {
    if (gs == 0) {
#pragma unroll
      for (int s = 0; s < RS; ++s) fin_lds[ns + 64 * s] = __builtin_amdgcn_ldexpf(1.f, e_fix[s]);
    }
    lds_barrier();
  }
  // Lane (g, r16) holds outputs n .. n + 3 (n = 16 i + 4 g) of activation
  // row 16 j + r16: one 16-byte store when the row length keeps it aligned
  // (scattered 4-byte stores cost about a fifth of the kernel at five tiles).
  const bool row4 = (N & 3) == 0;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int mr = 16 * j + r16;
    const int m = m0 + mr;
    const float fs = F16X ? 1.f : fin_lds[mr];
    if (m < M) {
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

namespace {

// Prefetch distances: activations and codes two half blocks ahead up to
// two tiles per wave, else one.  From three tiles a step is long enough to
// cover the loads, and the registers of a second half in flight cost more
// than they save (measured at four tiles: 202 against 184 us on the 7B FFN
// gate at 512 rows).
#ifndef QMV_DQREG_XD
#define QMV_DQREG_XD(T, NB) ((T) >= 3 || (NB) > 8 ? 1 : 2)
#endif
#ifndef QMV_DQREG_CD
#define QMV_DQREG_CD(T, NB) ((T) >= 3 || (NB) > 8 ? 1 : 2)
#endif

template <int T, int NB>
hipError_t launch_dqreg(const qmv_weights& W, const uint16_t* x, bool f16x, float* y, int M, hipStream_t stream) {
  constexpr int XD = QMV_DQREG_XD(T, NB), CD = QMV_DQREG_CD(T, NB);
  const int N = static_cast<int>(W.rows), K = static_cast<int>(W.cols);
  const uint8_t* w = static_cast<const uint8_t*>(W.data);
  const uint32_t pa = static_cast<uint32_t>(W.scales_offset);
  const dim3 grid((N + 64 * T - 1) / (64 * T), (M + rg_batch(NB) - 1) / rg_batch(NB));
  const size_t lds = rg_lds_bytes(NB);
  const bool pl = W.layout == QMV_LAYOUT_PLANES;
  if (pl && f16x)
    hipLaunchKernelGGL((gemm_q4_k_dqreg<T, NB, XD, CD, true, true>), grid, dim3(kRgThreads), lds, stream, w, pa, N, K,
                       x, y, M);
  else if (pl)
    hipLaunchKernelGGL((gemm_q4_k_dqreg<T, NB, XD, CD, true, false>), grid, dim3(kRgThreads), lds, stream, w, pa, N,
                       K, x, y, M);
  else if (f16x)
    hipLaunchKernelGGL((gemm_q4_k_dqreg<T, NB, XD, CD, false, true>), grid, dim3(kRgThreads), lds, stream, w, pa, N,
                       K, x, y, M);
  else
    hipLaunchKernelGGL((gemm_q4_k_dqreg<T, NB, XD, CD, false, false>), grid, dim3(kRgThreads), lds, stream, w, pa, N,
                       K, x, y, M);
  return hipGetLastError();
}

// The (tiles per wave, B tiles) forms built, and the modelled time of one:
// workgroup rounds over the compute units times the issue time of a
// workgroup, from the probe: about 18 cycles per product while the VALU work
// per product stays within two instructions, about 4.5 cycles per further
// instruction.
struct DqregForm {
  int t, nb;
};
constexpr DqregForm kDqregForms[] = {{1, 8}, {2, 8}, {3, 8}, {4, 8}, {5, 8}};
constexpr int kDqregFormCount = static_cast<int>(sizeof(kDqregForms) / sizeof(kDqregForms[0]));

double dqreg_cost(int64_t rows, int64_t batch, int64_t cus, DqregForm f) {
  const int64_t wgs = (rows + 64 * f.t - 1) / (64 * f.t) * ((batch + rg_batch(f.nb) - 1) / rg_batch(f.nb));
  const double valu_per_product = 16.0 / (2 * f.nb) + 6.0 / f.t + 0.4;
  const double per_product = valu_per_product <= 2 ? 18.0 : 18.0 + 4.5 * (valu_per_product - 2);
  return static_cast<double>((wgs + cus - 1) / cus) * f.t * f.nb * per_product;
}

}  // namespace

int dqreg_form(int64_t rows, int64_t batch) {
  const int64_t cus = device_cus();
  int best = 0;
  for (int k = 1; k < kDqregFormCount; ++k)
    if (dqreg_cost(rows, batch, cus, kDqregForms[k]) < dqreg_cost(rows, batch, cus, kDqregForms[best])) best = k;
  return best;
}

bool gemm_q4_k_dqreg_fits(const qmv_weights& W, int64_t batch) {
  const uint64_t wbytes = W.layout == QMV_LAYOUT_PLANES ? 5 * W.scales_offset + 64 * (W.rows * (W.cols / 256))
                                                        : 144 * static_cast<uint64_t>(W.rows) * (W.cols / 256);
  return wbytes < (1ull << 32) && 2 * static_cast<uint64_t>(batch) * W.cols < (1ull << 32);
}

hipError_t gemm_q4_k_dqreg(const qmv_weights& W, const void* x, bool f16x, float* y, int64_t batch,
                           hipStream_t stream) {
  const uint16_t* xh = static_cast<const uint16_t*>(x);
  const int M = static_cast<int>(batch);
#ifdef QMV_DQREG_FORM
  const int form = QMV_DQREG_FORM;
#else
  const int form = dqreg_form(W.rows, batch);
#endif
  switch (form) {
    case 0: return launch_dqreg<1, 8>(W, xh, f16x, y, M, stream);
    case 1: return launch_dqreg<2, 8>(W, xh, f16x, y, M, stream);
    case 2: return launch_dqreg<3, 8>(W, xh, f16x, y, M, stream);
    case 3: return launch_dqreg<4, 8>(W, xh, f16x, y, M, stream);
    default: return launch_dqreg<5, 8>(W, xh, f16x, y, M, stream);
  }
}

}  // namespace qmv
