// Q8_0 decode GEMV for gfx950.
//
// Block (VTE, feature list: llama.cpp's reference Q8_0 layout), 34 bytes:
// d fp16 | q[32] int8; w_i = d * q_i.  Blocks are only 2-byte aligned, so the
// 32 codes are fetched with two unaligned 16-byte loads (global_load_dwordx4
// accepts any alignment on gfx950).
//
// Lane mapping: one lane per block (32 weights); a wave covers 64 blocks
// (2048 columns).  Codes are made unsigned by flipping bit 7 of every byte
// (u = q + 128 < 1024) and enter the FMAs as fp16 subnormals (device_util.h):
//   partial = d (2^24 sum u x 2^-24 - 128 X),  X = sum of the lane's activations
#include "gemv_skeleton.h"

namespace qmv {

struct Q80Policy {
  static constexpr int kColsPerWave = 64 * 32;
  static constexpr int kXElems = 32;
  struct XSlice {
    float v[32];
    float s;
  };
  template <typename XT>
  using XSliceT = XSlice;  // fp32 activations for every activation type
  struct Frag {
    uint4 qa, qb;
    uint32_t d;
  };

  const uint8_t* base;
  uint32_t row_bytes;
  int col0;
  bool ok;

  __device__ Q80Policy(const uint8_t* w, uint64_t, int cols, int kslot, int lane) {
    const int nb = cols / 32;
    const int j = kslot * 64 + lane;
    ok = j < nb;
    const int jc = ok ? j : nb - 1;  // lanes past the row end read a valid block
    row_bytes = static_cast<uint32_t>(nb) * 34;
    base = w + static_cast<size_t>(jc) * 34;
    col0 = jc * 32;
  }

  template <class XS>
  __device__ void load_x_raw(const XS& x, uint4* raw) const {
    qmv::load_x_raw<32>(x, col0, raw);
  }

  template <typename XT>
  __device__ void finish_x(const uint4* raw, XSlice& s) const {
    x_to_f32<32>(raw, s.v, static_cast<const XT*>(nullptr));
    s.s = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      s.v[i] = ok ? s.v[i] : 0.f;
      s.s += s.v[i];
    }
  }

  __device__ void load(int row, Frag& f) const {
    const uint8_t* p = base + static_cast<size_t>(row) * row_bytes;
    f.d = ld_u16(p);
    f.qa = ld16_any(p + 2);
    f.qb = ld16_any(p + 18);
  }

  template <typename XT>
  __device__ float dot(const Frag& f, const XSlice& s) const {
    const uint32_t q[8] = {f.qa.x, f.qa.y, f.qa.z, f.qa.w, f.qb.x, f.qb.y, f.qb.z, f.qb.w};
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t u = q[i] ^ 0x80808080u;
      const uint32_t a = u & 0x00FF00FFu, b = (u >> 8) & 0x00FF00FFu;  // codes 0,2 | 1,3
      acc = fma_lo(a, s.v[4 * i + 0], acc);
      acc = fma_lo(b, s.v[4 * i + 1], acc);
      acc = fma_hi(a, s.v[4 * i + 2], acc);
      acc = fma_hi(b, s.v[4 * i + 3], acc);
    }
    return f16_to_f32(f.d) * fmaf(kTwo24, acc, -128.f * s.s);
  }
};

hipError_t gemv_q8_0(const GemvCall* calls, int n, int x_dtype, int64_t batch, hipStream_t s) {
  return launch_gemv<Q80Policy>(calls, n, x_dtype, batch, s);
}

}  // namespace qmv
