// Q4_K decode GEMV for gfx950.
//
// Block (VTE, feature list: llama.cpp's reference Q4_K layout), 144 bytes:
// d fp16 | dmin fp16 | scales[12] | qs[128]; weight t = 64c + 32h + l takes
// nibble h of qs[32c + l]; sub-block s = 2c + h; w = d*sc_s*u - dmin*m_s.
//
// Lane mapping: four lanes per block, lane c (0..3) owns qs[32c .. 32c+32),
// i.e. the 64 weights of sub-blocks 2c (low nibbles) and 2c+1 (high nibbles),
// whose activations x[64c .. 64c+64) are contiguous.  One wave covers 16
// blocks (4096 columns) with three 16-byte loads per lane and row: the block
// header (shared by the four lanes) and the lane's two qs quarters.
//
// Arithmetic per lane and row, all fp32:
//   S0 = sum_l u_lo[l] * x[l],  S1 = sum_l (16 u_hi[l]) * x[32 + l]
//   partial = d * (sc0 * S0 + sc1/16 * S1) - dmin * (m0 * X0 + m1 * X1)
// with X0, X1 the sub-block sums of x, computed once per wave.  Codes become
// floats with v_cvt_f32_ubyte{0..3} after one AND each for the low nibbles
// (mask 0x0F0F0F0F) and for the high nibbles (mask 0xF0F0F0F0, which leaves
// 16*u in each byte; the 1/16 is folded into sc1).
#include "gemv_skeleton.h"

namespace qmv {

struct Q4KPolicy {
  static constexpr int kColsPerWave = 16 * 256;
  struct Params {
    const uint8_t* w;
  };
  struct XSlice {
    float v[64];
    float s0, s1;
  };
  struct Frag {
    uint4 hd, qa, qb;
  };

  const uint8_t* base;
  size_t row_bytes;
  int col0;
  int c;
  bool ok;
  bool hi;
  uint32_t sh0, sh1, hoff, moff;

  __device__ Q4KPolicy(const Params& p, int cols, int kslot, int lane) {
    const int nb = cols / 256;
    const int j = kslot * 16 + (lane >> 2);
    c = lane & 3;
    ok = j < nb;
    row_bytes = static_cast<size_t>(nb) * 144;
    base = p.w + static_cast<size_t>(j) * 144;
    col0 = j * 256 + c * 64;
    // Sub-blocks 2c and 2c+1.  Their 6-bit scale and min come from
    //   j < 4 : sc = scales[j] & 63,                 m = scales[j+4] & 63
    //   j >= 4: sc = (scales[j+4] & 15) | (scales[j-4] >> 6) << 4
    //           m  = (scales[j+4] >> 4) | (scales[j]   >> 6) << 4
    // Both cases read as  low4 | high2 << 4  with per-lane shifts below
    // (H1, H2, H3 = header dwords holding scales[0..3], [4..7], [8..11]).
    hi = c >= 2;
    sh0 = static_cast<uint32_t>((2 * c) & 3) * 8;
    sh1 = sh0 + 8;
    hoff = hi ? 6u : 4u;
    moff = hi ? 4u : 0u;
  }

  template <typename XT>
  __device__ void load_x(const XT* x, XSlice& s) const {
    s.s0 = 0.f;
    s.s1 = 0.f;
    if (!ok) {
#pragma unroll
      for (int i = 0; i < 64; ++i) s.v[i] = 0.f;
      return;
    }
    qmv::load_x<64>(x + col0, s.v);
#pragma unroll
    for (int i = 0; i < 32; ++i) s.s0 += s.v[i];
#pragma unroll
    for (int i = 32; i < 64; ++i) s.s1 += s.v[i];
  }

  __device__ void load(int row, Frag& f) const {
    const uint8_t* p = base + static_cast<size_t>(row) * row_bytes;
    f.hd = *reinterpret_cast<const uint4*>(p);
    f.qa = *reinterpret_cast<const uint4*>(p + 16 + 32 * c);
    f.qb = *reinterpret_cast<const uint4*>(p + 32 + 32 * c);
  }

  __device__ static void zero(Frag& f) {
    f.hd = make_uint4(0, 0, 0, 0);
    f.qa = f.hd;
    f.qb = f.hd;
  }

  __device__ float dot(const Frag& f, const XSlice& s) const {
    const uint32_t H1 = f.hd.y, H2 = f.hd.z, H3 = f.hd.w;
    const uint32_t A = hi ? H3 : H1;
    const uint32_t B = hi ? H3 : H2;
    const uint32_t sc0 = ((A >> sh0) & 15u) | (((H1 >> (sh0 + hoff)) & 3u) << 4);
    const uint32_t sc1 = ((A >> sh1) & 15u) | (((H1 >> (sh1 + hoff)) & 3u) << 4);
    const uint32_t m0 = ((B >> (sh0 + moff)) & 15u) | (((H2 >> (sh0 + hoff)) & 3u) << 4);
    const uint32_t m1 = ((B >> (sh1 + moff)) & 15u) | (((H2 >> (sh1 + hoff)) & 3u) << 4);
    const float d = f16_to_f32(f.hd.x & 0xFFFFu);
    const float dmin = f16_to_f32(f.hd.x >> 16);

    const uint32_t q[8] = {f.qa.x, f.qa.y, f.qa.z, f.qa.w, f.qb.x, f.qb.y, f.qb.z, f.qb.w};
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t lo = q[i] & 0x0F0F0F0Fu;
      const uint32_t hv = q[i] & 0xF0F0F0F0u;
      s0 = fmaf(ubyte<0>(lo), s.v[4 * i + 0], s0);
      s0 = fmaf(ubyte<1>(lo), s.v[4 * i + 1], s0);
      s0 = fmaf(ubyte<2>(lo), s.v[4 * i + 2], s0);
      s0 = fmaf(ubyte<3>(lo), s.v[4 * i + 3], s0);
      s1 = fmaf(ubyte<0>(hv), s.v[32 + 4 * i + 0], s1);
      s1 = fmaf(ubyte<1>(hv), s.v[32 + 4 * i + 1], s1);
      s1 = fmaf(ubyte<2>(hv), s.v[32 + 4 * i + 2], s1);
      s1 = fmaf(ubyte<3>(hv), s.v[32 + 4 * i + 3], s1);
    }
    const float t = fmaf(static_cast<float>(sc1) * 0.0625f, s1, static_cast<float>(sc0) * s0);
    const float mm = fmaf(static_cast<float>(m1), s.s1, static_cast<float>(m0) * s.s0);
    return fmaf(d, t, -dmin * mm);
  }
};

hipError_t gemv_q4_k(const GemvArgs& a) {
  Q4KPolicy::Params prm{static_cast<const uint8_t*>(a.W->data)};
  return launch_gemv<Q4KPolicy>(a, prm);
}

}  // namespace qmv
