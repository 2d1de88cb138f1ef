// INT4 symmetric group-128 decode GEMV for gfx950.
//
// Format ("Costruire un runtime di inference LLM da zero", datastack.it, "Tre
// bug che insegnano": symmetric INT4 weights, one scale per 128; the plane
// layout is this library's reading): a codes plane where byte j of a row holds
// u_{2j} in bits 0-3 and u_{2j+1} in bits 4-7 (u = q + 8), then an fp16 scales
// plane [rows][cols/128].  w_k = s_{k/128} * (u_k - 8).
//
// Lane mapping: a wave covers 4096 columns = 2048 code bytes of a row.  Lane l
// owns code bytes [16l, 16l+16) and [1024+16l, 1024+16l+16), so each of the two
// 16-byte load instructions reads 1 KB of consecutive bytes, plus the fp16
// scale of each half's group.  The code loads carry the nontemporal hint: no
// other instruction reads their lines (a row's code bytes are a multiple of
// 64 B, so only a row boundary can split a line).  Per lane, half and row,
// codes enter as fp16 subnormals (see device_util.h), sums in fp32:
//   Se = sum u_even x_even 2^-24,  So = sum 16 u_odd x_odd 2^-24
//   partial += s (2^24 (Se + So/16) - 8 X),  X = fp32 sum of the half's 32 activations
// fp32 activations: one v_fma_mix_f32 per weight.  fp16 activations (the
// datastack runtime's FP16 activations) and bf16: two products per
// v_dot2_f32_f16 against the activations as fp16 -- fp16 as given, bf16
// scaled per lane by a power of two (half_scale_exp; exact) -- with 2^(24+e)
// in place of 2^24.
#include "gemv_skeleton.h"

namespace qmv {

struct Int4G128Policy {
  static constexpr int kColsPerWave = 64 * 64;
  static constexpr int kXElems = 64;
  // shared-activation GEMV: one-row tiles, three in flight (SxShape)
  static constexpr int kSxRows = 1, kSxTiles = 3;
  struct XSliceF32 {
    float v[64];  // v[32h + k]: activation of column col[h] + k, scaled by 2^-e (f32_slice_factor)
    float s[2];   // sums of each half's 32 unscaled activations
    float xs;     // 2^(24 + e)
  };
  struct XSliceHalf {
    h2_t h[32];  // h[16 hf + 4 i + p]: fp16 activation pairs of half hf, dword i, pair p
    float s[2];  // fp32 sums of each half's 32 activations
    float xs;    // 2^(24 + e)
  };
  template <typename XT>
  using XSliceT = typename XSliceFor<XT, XSliceF32, XSliceHalf>::type;
  struct Frag {
    uint4 q[2];
    uint32_t sb[2];
  };

  const uint8_t* codes[2];
  const uint8_t* scales[2];
  uint32_t code_row, scale_row;
  int col[2];
  bool okh[2];

  __device__ Int4G128Policy(const uint8_t* w, uint64_t scales_offset, int cols, int kslot,
                            int lane) {
    code_row = static_cast<uint32_t>(cols) / 2;
    scale_row = static_cast<uint32_t>(cols / 128) * 2;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int c = kslot * kColsPerWave + 2048 * h + 32 * lane;
      okh[h] = c < cols;
      if (!okh[h]) c = cols - 32;  // past the row end: read valid columns, x zeroed
      col[h] = c;
      codes[h] = w + c / 2;
      scales[h] = w + scales_offset + static_cast<size_t>(c / 128) * 2;
    }
  }

  template <class XS>
  __device__ void load_x_raw(const XS& x, uint4* raw) const {
    constexpr int kPer = 32 * static_cast<int>(sizeof(typename XS::elem)) / 16;
    qmv::load_x_raw<32>(x, col[0], raw);
    qmv::load_x_raw<32>(x, col[1], raw + kPer);
  }

  template <typename XT>
  __device__ void finish_x(const uint4* raw, XSliceT<XT>& s) const {
    float v[64];  // v[32 hf + k]: activation of column col[hf] + k
    float* dst = v;
    if constexpr (__is_same(XT, float)) dst = s.v;
    x_to_f32<64>(raw, dst, static_cast<const XT*>(nullptr));
    if constexpr (__is_same(XT, float)) {
      float un;
      const float f = f32_slice_factor<64>(s.v, true, s.xs, un);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const float fh = okh[hf] ? f : 0.f;
        s.s[hf] = 0.f;
#pragma unroll
        for (int k = 0; k < 32; ++k) {
          s.v[32 * hf + k] *= fh;
          s.s[hf] += s.v[32 * hf + k];
        }
        s.s[hf] *= un;
      }
    } else {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        s.s[hf] = 0.f;
#pragma unroll
        for (int k = 0; k < 32; ++k) {
          dst[32 * hf + k] = okh[hf] ? dst[32 * hf + k] : 0.f;
          s.s[hf] += dst[32 * hf + k];
        }
      }
      const int e = half_scale_exp<XT, 64>(v);
      s.xs = __builtin_amdgcn_ldexpf(1.0f, 24 + e);
      // dword i of a half holds weights 8i..8i+7, two per byte; the code pairs
      // are (8i, 8i+4), (8i+2, 8i+6) from the low nibbles and (8i+1, 8i+5),
      // (8i+3, 8i+7) from the high nibbles
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float* x = v + 32 * hf + 8 * i;
          h2_t* o = s.h + 16 * hf + 4 * i;
          o[0] = h2_t{scaled_f16(x[0], e), scaled_f16(x[4], e)};
          o[1] = h2_t{scaled_f16(x[2], e), scaled_f16(x[6], e)};
          o[2] = h2_t{scaled_f16(x[1], e), scaled_f16(x[5], e)};
          o[3] = h2_t{scaled_f16(x[3], e), scaled_f16(x[7], e)};
        }
    }
  }

  __device__ void load(int row, Frag& f) const {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f.q[h] = ld16_stream(codes[h] + static_cast<size_t>(row) * code_row);
      f.sb[h] = ld_u16(scales[h] + static_cast<size_t>(row) * scale_row);
    }
  }

  template <typename XT>
  __device__ float dot(const Frag& f, const XSliceT<XT>& s) const {
    float out = 0.f;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const uint32_t q[4] = {f.q[hf].x, f.q[hf].y, f.q[hf].z, f.q[hf].w};
      float se = 0.f, so = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // dword i holds weights 8i..8i+7: byte b = u_{8i+2b} (low) | u_{8i+2b+1} (high)
        const uint32_t w0 = q[i], w8 = q[i] >> 8;
        const uint32_t a = w0 & 0x000F000Fu, b = w8 & 0x000F000Fu;  // u_{8i}, u_{8i+4} | u_{8i+2}, u_{8i+6}
        const uint32_t e = w0 & 0x00F000F0u, g = w8 & 0x00F000F0u;  // 16 u_{8i+1}, ... (odd weights)
        if constexpr (__is_same(XT, float)) {
          const float* x = s.v + 32 * hf + 8 * i;
          se = fma_lo(a, x[0], se);
          se = fma_lo(b, x[2], se);
          se = fma_hi(a, x[4], se);
          se = fma_hi(b, x[6], se);
          so = fma_lo(e, x[1], so);
          so = fma_lo(g, x[3], so);
          so = fma_hi(e, x[5], so);
          so = fma_hi(g, x[7], so);
        } else {
          const h2_t* x = s.h + 16 * hf + 4 * i;
          se = dot2_lo_hi(a, x[0], se);
          se = dot2_lo_hi(b, x[1], se);
          so = dot2_lo_hi(e, x[2], so);
          so = dot2_lo_hi(g, x[3], so);
        }
      }
      float xs;
      if constexpr (__is_same(XT, float))
        xs = s.xs;
      else
        xs = s.xs;
      const float t = fmaf(xs, fmaf(so, 0.0625f, se), -8.f * s.s[hf]);
      out = fmaf(f16_to_f32(f.sb[hf]), t, out);
    }
    return out;
  }

  // dot<XT> for NBR activation rows at once: the code masks are computed
  // once, then each row's sums follow dot's operations in dot's order, so
  // out[m] equals dot(f, s[m]) bit for bit.
  template <typename XT, int NBR>
  __device__ void dot_rows(const Frag& f, const XSliceT<XT>* s, float* out) const {
#pragma unroll
    for (int m = 0; m < NBR; ++m) out[m] = 0.f;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const uint32_t q[4] = {f.q[hf].x, f.q[hf].y, f.q[hf].z, f.q[hf].w};
      float se[NBR], so[NBR];
#pragma unroll
      for (int m = 0; m < NBR; ++m) se[m] = so[m] = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w0 = q[i], w8 = q[i] >> 8;
        const uint32_t a = w0 & 0x000F000Fu, b = w8 & 0x000F000Fu;
        const uint32_t e = w0 & 0x00F000F0u, g = w8 & 0x00F000F0u;
#pragma unroll
        for (int m = 0; m < NBR; ++m) {
          if constexpr (__is_same(XT, float)) {
            const float* x = s[m].v + 32 * hf + 8 * i;
            se[m] = fma_lo(a, x[0], se[m]);
            se[m] = fma_lo(b, x[2], se[m]);
            se[m] = fma_hi(a, x[4], se[m]);
            se[m] = fma_hi(b, x[6], se[m]);
            so[m] = fma_lo(e, x[1], so[m]);
            so[m] = fma_lo(g, x[3], so[m]);
            so[m] = fma_hi(e, x[5], so[m]);
            so[m] = fma_hi(g, x[7], so[m]);
          } else {
            const h2_t* x = s[m].h + 16 * hf + 4 * i;
            se[m] = dot2_lo_hi(a, x[0], se[m]);
            se[m] = dot2_lo_hi(b, x[1], se[m]);
            so[m] = dot2_lo_hi(e, x[2], so[m]);
            so[m] = dot2_lo_hi(g, x[3], so[m]);
          }
        }
      }
      const float sc = f16_to_f32(f.sb[hf]);
#pragma unroll
      for (int m = 0; m < NBR; ++m) {
        float xs;
        if constexpr (__is_same(XT, float))
          xs = s[m].xs;
        else
          xs = s[m].xs;
        const float t = fmaf(xs, fmaf(so[m], 0.0625f, se[m]), -8.f * s[m].s[hf]);
        out[m] = fmaf(sc, t, out[m]);
      }
    }
  }
};

hipError_t gemv_int4_g128_rows(const GemvCall* calls, int n, int x_dtype, int64_t batch,
                               hipStream_t s) {
  return launch_gemv_rows<Int4G128Policy>(calls, n, x_dtype, batch, s);
}

hipError_t gemv_int4_g128(const GemvCall* calls, int n, int x_dtype, int64_t batch, hipStream_t s) {
  return launch_gemv<Int4G128Policy>(calls, n, x_dtype, batch, s);
}

hipError_t gemv_int4_g128_pair(const GemvCall& a, const void* b_w, float* b_y, int x_dtype, int64_t batch,
                               bool glu, hipStream_t s) {
  return launch_gemv_pair<Int4G128Policy>(a, b_w, b_y, x_dtype, batch, glu, s);
}

}  // namespace qmv
