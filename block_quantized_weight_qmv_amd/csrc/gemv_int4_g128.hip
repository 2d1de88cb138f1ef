// INT4 symmetric group-128 decode GEMV for gfx950.
//
// Format ("Costruire un runtime di inference LLM da zero", datastack.it, "Tre
// bug che insegnano": symmetric INT4 weights, one scale per 128; the plane
// layout is this library's reading): a codes plane where byte j of a row holds
// u_{2j} in bits 0-3 and u_{2j+1} in bits 4-7 (u = q + 8), then an fp16 scales
// plane [rows][cols/128].  w_k = s_{k/128} * (u_k - 8).
//
// Lane mapping: each lane owns 64 consecutive weights (32 code bytes, two
// 16-byte loads, half of one group) plus that group's 2-byte scale; a wave
// covers 4096 columns.  Per lane and row, in fp32:
//   Se = sum u_even * x_even,  So = sum (16 u_odd) * x_odd
//   partial = s * (Se + So/16 - 8 * X),  X = sum of the lane's 64 activations
#include "gemv_skeleton.h"

namespace qmv {

struct Int4G128Policy {
  static constexpr int kColsPerWave = 64 * 64;
  struct Params {
    const uint8_t* w;
    uint64_t scales_offset;
  };
  struct XSlice {
    float v[64];
    float s;
  };
  struct Frag {
    uint4 qa, qb;
    uint32_t sbits;
  };

  const uint8_t* codes;
  const uint8_t* scales;
  size_t code_row, scale_row;
  int col0;
  bool ok;

  __device__ Int4G128Policy(const Params& p, int cols, int kslot, int lane) {
    col0 = kslot * kColsPerWave + 64 * lane;
    ok = col0 < cols;
    code_row = static_cast<size_t>(cols) / 2;
    scale_row = static_cast<size_t>(cols / 128) * 2;
    codes = p.w + col0 / 2;
    scales = p.w + p.scales_offset + static_cast<size_t>(col0 / 128) * 2;
  }

  template <typename XT>
  __device__ void load_x(const XT* x, XSlice& s) const {
    s.s = 0.f;
    if (!ok) {
#pragma unroll
      for (int i = 0; i < 64; ++i) s.v[i] = 0.f;
      return;
    }
    qmv::load_x<64>(x + col0, s.v);
#pragma unroll
    for (int i = 0; i < 64; ++i) s.s += s.v[i];
  }

  __device__ void load(int row, Frag& f) const {
    const uint8_t* p = codes + static_cast<size_t>(row) * code_row;
    f.qa = *reinterpret_cast<const uint4*>(p);
    f.qb = *reinterpret_cast<const uint4*>(p + 16);
    f.sbits = load_u16(scales + static_cast<size_t>(row) * scale_row);
  }

  __device__ static void zero(Frag& f) {
    f.qa = make_uint4(0, 0, 0, 0);
    f.qb = f.qa;
    f.sbits = 0;
  }

  __device__ float dot(const Frag& f, const XSlice& s) const {
    const uint32_t q[8] = {f.qa.x, f.qa.y, f.qa.z, f.qa.w, f.qb.x, f.qb.y, f.qb.z, f.qb.w};
    float se = 0.f, so = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t lo = q[i] & 0x0F0F0F0Fu;  // u_{8i}, u_{8i+2}, u_{8i+4}, u_{8i+6}
      const uint32_t hv = q[i] & 0xF0F0F0F0u;  // 16 u_{8i+1}, 16 u_{8i+3}, ...
      se = fmaf(ubyte<0>(lo), s.v[8 * i + 0], se);
      se = fmaf(ubyte<1>(lo), s.v[8 * i + 2], se);
      se = fmaf(ubyte<2>(lo), s.v[8 * i + 4], se);
      se = fmaf(ubyte<3>(lo), s.v[8 * i + 6], se);
      so = fmaf(ubyte<0>(hv), s.v[8 * i + 1], so);
      so = fmaf(ubyte<1>(hv), s.v[8 * i + 3], so);
      so = fmaf(ubyte<2>(hv), s.v[8 * i + 5], so);
      so = fmaf(ubyte<3>(hv), s.v[8 * i + 7], so);
    }
    const float t = fmaf(so, 0.0625f, se);
    return f16_to_f32(f.sbits) * fmaf(-8.f, s.s, t);
  }
};

hipError_t gemv_int4_g128(const GemvArgs& a) {
  Int4G128Policy::Params prm{static_cast<const uint8_t*>(a.W->data), a.W->scales_offset};
  return launch_gemv<Int4G128Policy>(a, prm);
}

}  // namespace qmv
