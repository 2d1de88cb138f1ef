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
// one v_fma_mix_f32 per weight for fp32 activations; fp16 and bf16 ones enter
// as fp16 (bf16 scaled per lane by a power of two, exact; half_scale_exp),
// two products per v_dot2_f32_f16 (exact: 8 + 11 significant bits), with
// 2^(24+e) in place of 2^24.
#include "gemv_skeleton.h"

namespace qmv {

struct Q80Policy {
  static constexpr int kColsPerWave = 64 * 32;
  static constexpr int kXElems = 32;
  struct XSlice {
    float v[32];  // scaled by 2^-e (f32_slice_factor)
    float s;      // sum of the lane's 32 unscaled activations
    float xs;     // 2^(24 + e)
  };
  struct XSliceHalf {
    h2_t h[16];  // h[2i + p]: pair p of dword i: (4i, 4i+2), (4i+1, 4i+3)
    float s;     // fp32 sum of the lane's 32 activations
    float xs;    // 2^(24 + e)
  };
  template <typename XT>
  using XSliceT = typename XSliceFor<XT, XSlice, XSliceHalf>::type;
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
  __device__ void finish_x(const uint4* raw, XSliceT<XT>& s) const {
    float v[32];
    float* dst = v;
    if constexpr (__is_same(XT, float)) dst = s.v;
    x_to_f32<32>(raw, dst, static_cast<const XT*>(nullptr));
    s.s = 0.f;
    if constexpr (__is_same(XT, float)) {
      float un;
      const float f = f32_slice_factor<32>(s.v, ok, s.xs, un);
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        s.v[i] *= f;
        s.s += s.v[i];
      }
      s.s *= un;
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        dst[i] = ok ? dst[i] : 0.f;
        s.s += dst[i];
      }
      const int e = half_scale_exp<XT, 32>(v);
      s.xs = __builtin_amdgcn_ldexpf(1.0f, 24 + e);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        s.h[2 * i] = h2_t{scaled_f16(v[4 * i], e), scaled_f16(v[4 * i + 2], e)};
        s.h[2 * i + 1] = h2_t{scaled_f16(v[4 * i + 1], e), scaled_f16(v[4 * i + 3], e)};
      }
    }
  }

  __device__ void load(int row, Frag& f) const {
    const uint8_t* p = base + static_cast<size_t>(row) * row_bytes;
    f.d = ld_u16(p);
    f.qa = ld16_any(p + 2);
    f.qb = ld16_any(p + 18);
  }

  template <typename XT>
  __device__ float dot(const Frag& f, const XSliceT<XT>& s) const {
    const uint32_t q[8] = {f.qa.x, f.qa.y, f.qa.z, f.qa.w, f.qb.x, f.qb.y, f.qb.z, f.qb.w};
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t u = q[i] ^ 0x80808080u;
      const uint32_t a = u & 0x00FF00FFu, b = (u >> 8) & 0x00FF00FFu;  // codes 0,2 | 1,3
      if constexpr (__is_same(XT, float)) {
        acc = fma_lo(a, s.v[4 * i + 0], acc);
        acc = fma_lo(b, s.v[4 * i + 1], acc);
        acc = fma_hi(a, s.v[4 * i + 2], acc);
        acc = fma_hi(b, s.v[4 * i + 3], acc);
      } else {
        acc = dot2_lo_hi(a, s.h[2 * i], acc);
        acc = dot2_lo_hi(b, s.h[2 * i + 1], acc);
      }
    }
    float xs;
    if constexpr (__is_same(XT, float))
      xs = s.xs;
    else
      xs = s.xs;
    return f16_to_f32(f.d) * fmaf(xs, acc, -128.f * s.s);
  }

  // dot<XT> for NBR activation rows at once: the offset codes are formed
  // once, then each row's sum follows dot's operations in dot's order, so
  // out[m] equals dot(f, s[m]) bit for bit.
  template <typename XT, int NBR>
  __device__ void dot_rows(const Frag& f, const XSliceT<XT>* s, float* out) const {
    const uint32_t q[8] = {f.qa.x, f.qa.y, f.qa.z, f.qa.w, f.qb.x, f.qb.y, f.qb.z, f.qb.w};
    float acc[NBR];
#pragma unroll
    for (int m = 0; m < NBR; ++m) acc[m] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t u = q[i] ^ 0x80808080u;
      const uint32_t a = u & 0x00FF00FFu, b = (u >> 8) & 0x00FF00FFu;
#pragma unroll
      for (int m = 0; m < NBR; ++m) {
        if constexpr (__is_same(XT, float)) {
          acc[m] = fma_lo(a, s[m].v[4 * i + 0], acc[m]);
          acc[m] = fma_lo(b, s[m].v[4 * i + 1], acc[m]);
          acc[m] = fma_hi(a, s[m].v[4 * i + 2], acc[m]);
          acc[m] = fma_hi(b, s[m].v[4 * i + 3], acc[m]);
        } else {
          acc[m] = dot2_lo_hi(a, s[m].h[2 * i], acc[m]);
          acc[m] = dot2_lo_hi(b, s[m].h[2 * i + 1], acc[m]);
        }
      }
    }
    const float d = f16_to_f32(f.d);
#pragma unroll
    for (int m = 0; m < NBR; ++m) {
      float xs;
      if constexpr (__is_same(XT, float))
        xs = s[m].xs;
      else
        xs = s[m].xs;
      out[m] = d * fmaf(xs, acc[m], -128.f * s[m].s);
    }
  }
};

hipError_t gemv_q8_0_rows(const GemvCall* calls, int n, int x_dtype, int64_t batch, hipStream_t s) {
  return launch_gemv_rows<Q80Policy>(calls, n, x_dtype, batch, s);
}

hipError_t gemv_q8_0(const GemvCall* calls, int n, int x_dtype, int64_t batch, hipStream_t s) {
  return launch_gemv<Q80Policy>(calls, n, x_dtype, batch, s);
}

hipError_t gemv_q8_0_pair(const GemvCall& a, const void* b_w, float* b_y, int x_dtype, int64_t batch, bool glu,
                          hipStream_t s) {
  return launch_gemv_pair<Q80Policy>(a, b_w, b_y, x_dtype, batch, glu, s);
}

}  // namespace qmv
