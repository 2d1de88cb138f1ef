// Q8_0 decode GEMV for gfx950.
//
// Block (VTE, feature list: llama.cpp's reference Q8_0 layout), 34 bytes:
// d fp16 | q[32] int8; w_i = d * q_i.  Blocks are only 2-byte aligned, so the
// 32 codes are fetched with two unaligned 16-byte loads (global_load_dwordx4
// accepts any alignment on gfx950).
//
// Lane mapping: one lane per block (32 weights); a wave covers 64 blocks
// (2048 columns).  Codes are made unsigned by flipping bit 7 of every byte
// (u = q + 128) so v_cvt_f32_ubyte applies; per lane and row, in fp32:
//   partial = d * (sum u * x - 128 * X),  X = sum of the lane's 32 activations
#include "gemv_skeleton.h"

namespace qmv {

struct Q80Policy {
  static constexpr int kColsPerWave = 64 * 32;
  struct Params {
    const uint8_t* w;
  };
  struct XSlice {
    float v[32];
    float s;
  };
  struct Frag {
    uint4 qa, qb;
    uint32_t d;
  };

  const uint8_t* base;
  size_t row_bytes;
  int col0;
  bool ok;

  __device__ Q80Policy(const Params& p, int cols, int kslot, int lane) {
    const int nb = cols / 32;
    const int j = kslot * 64 + lane;
    ok = j < nb;
    row_bytes = static_cast<size_t>(nb) * 34;
    base = p.w + static_cast<size_t>(j) * 34;
    col0 = j * 32;
  }

  template <typename XT>
  __device__ void load_x(const XT* x, XSlice& s) const {
    s.s = 0.f;
    if (!ok) {
#pragma unroll
      for (int i = 0; i < 32; ++i) s.v[i] = 0.f;
      return;
    }
    qmv::load_x<32>(x + col0, s.v);
#pragma unroll
    for (int i = 0; i < 32; ++i) s.s += s.v[i];
  }

  __device__ void load(int row, Frag& f) const {
    const uint8_t* p = base + static_cast<size_t>(row) * row_bytes;
    f.d = load_u16(p);
    f.qa = load16_any(p + 2);
    f.qb = load16_any(p + 18);
  }

  __device__ static void zero(Frag& f) {
    f.qa = make_uint4(0, 0, 0, 0);
    f.qb = f.qa;
    f.d = 0;
  }

  __device__ float dot(const Frag& f, const XSlice& s) const {
    const uint32_t q[8] = {f.qa.x, f.qa.y, f.qa.z, f.qa.w, f.qb.x, f.qb.y, f.qb.z, f.qb.w};
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t u = q[i] ^ 0x80808080u;
      acc = fmaf(ubyte<0>(u), s.v[4 * i + 0], acc);
      acc = fmaf(ubyte<1>(u), s.v[4 * i + 1], acc);
      acc = fmaf(ubyte<2>(u), s.v[4 * i + 2], acc);
      acc = fmaf(ubyte<3>(u), s.v[4 * i + 3], acc);
    }
    return f16_to_f32(f.d) * fmaf(-128.f, s.s, acc);
  }
};

hipError_t gemv_q8_0(const GemvArgs& a) {
  Q80Policy::Params prm{static_cast<const uint8_t*>(a.W->data)};
  return launch_gemv<Q80Policy>(a, prm);
}

}  // namespace qmv
