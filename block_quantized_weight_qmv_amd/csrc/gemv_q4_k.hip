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
// Arithmetic per lane and row.  fp32 activations (exact, one rounding per FMA):
//   S0 = sum_l u_lo[l] x[l] 2^-24,  S1 = sum_l 16 u_hi[l] x[32+l] 2^-24
//   partial = d 2^24 (sc0 S0 + sc1/16 S1) - dmin (m0 X0 + m1 X1)
// X0, X1 are the sub-block sums of x, computed once per wave.  Each dword of
// qs (8 codes) costs one shift and four ANDs (masks 0x000F000F / 0x00F000F0
// leave two codes per dword as fp16 subnormals) and eight v_fma_mix_f32.
// fp16 and bf16 activations (HalfXSlice, exact): the same sums with two
// products per v_dot2_f32_f16, four per dword instead of eight FMAs, and
// 2^(24+e) in place of 2^24 for the lane's power-of-two activation scale.
#include "gemv_skeleton.h"

namespace qmv {

struct Q4KPolicy {
  static constexpr int kColsPerWave = 16 * 256;
  static constexpr int kXElems = 64;
  struct XSliceF32 {
    float v[64];   // scaled by 2^-e (f32_slice_factor)
    float s0, s1;  // sums of the unscaled activations of the two sub-blocks
    float xs;      // 2^(24 + e)
  };
  template <typename XT>
  using XSliceT = typename XSliceFor<XT, XSliceF32, HalfXSlice>::type;
  struct Frag {
    uint4 hd, qa, qb;
  };

  const uint8_t* base;
  uint32_t row_bytes;
  int col0;
  int c;
  bool ok;
  bool hi;
  uint32_t sh, mask_a, mask_b;

  __device__ Q4KPolicy(const uint8_t* w, uint64_t, int cols, int kslot, int lane) {
    const int nb = cols / 256;
    const int j = kslot * 16 + (lane >> 2);
    c = lane & 3;
    ok = j < nb;
    const int jc = ok ? j : nb - 1;  // lanes past the row end read a valid block
    row_bytes = static_cast<uint32_t>(nb) * 144;
    base = w + static_cast<size_t>(jc) * 144;
    col0 = jc * 256 + c * 64;
    // Scale and min of sub-blocks 2c, 2c+1, both as two bytes of one dword
    // (H1, H2, H3 = header dwords with scales[0..3], [4..7], [8..11]):
    //   c < 2 : sc = (H1 >> 16c) & 0x3F3F,  m = (H2 >> 16c) & 0x3F3F
    //   c >= 2: sc = (H3 >> sh) & 0x0F0F | (H1 >> sh >> 2) & 0x3030
    //           m  = (H3 >> sh >> 4) & 0x0F0F | (H2 >> sh >> 2) & 0x3030
    // with sh = 16 (c & 1): low nibbles from scales[8+j'], top two bits from
    // bits 6-7 of scales[j'] (scale) or scales[4+j'] (min).
    hi = c >= 2;
    sh = 16u * static_cast<uint32_t>(c & 1);
    mask_a = hi ? 0x0F0Fu : 0x3F3Fu;
    mask_b = hi ? 0x3030u : 0u;
  }

  template <class XS>
  __device__ void load_x_raw(const XS& x, uint4* raw) const {
    qmv::load_x_raw<64>(x, col0, raw);
  }

  template <typename XT>
  __device__ void finish_x(const uint4* raw, XSliceT<XT>& s) const {
    if constexpr (__is_same(XT, float)) {
      x_to_f32<64>(raw, s.v, static_cast<const XT*>(nullptr));
      float un;
      const float f = f32_slice_factor<64>(s.v, ok, s.xs, un);
#pragma unroll
      for (int i = 0; i < 64; ++i) s.v[i] *= f;
      s.s0 = 0.f;
      s.s1 = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) s.s0 += s.v[i];
#pragma unroll
      for (int i = 32; i < 64; ++i) s.s1 += s.v[i];
      s.s0 *= un;
      s.s1 *= un;
    } else {
      finish_half_xslice<XT>(raw, ok, s);
    }
  }

  __device__ void load(int row, Frag& f) const {
    const uint8_t* p = base + static_cast<size_t>(row) * row_bytes;
    f.hd = ld16(p);
    f.qa = ld16(p + 16 + 32 * c);
    f.qb = ld16(p + 32 + 32 * c);
  }

  template <typename XT>
  __device__ float dot(const Frag& f, const XSliceT<XT>& s) const {
    const uint32_t t1 = f.hd.y >> sh, t2 = f.hd.z >> sh, t3 = f.hd.w >> sh;
    const uint32_t sc = ((hi ? t3 : t1) & mask_a) | ((t1 >> 2) & mask_b);
    const uint32_t mn = ((hi ? (t3 >> 4) : t2) & mask_a) | ((t2 >> 2) & mask_b);
    const float dmin = f16_to_f32(f.hd.x >> 16);

    const uint32_t q[8] = {f.qa.x, f.qa.y, f.qa.z, f.qa.w, f.qb.x, f.qb.y, f.qb.z, f.qb.w};
    float s0 = 0.f, s1 = 0.f;
    float d;
    if constexpr (__is_same(XT, float)) {
      d = f16_to_f32(f.hd.x & 0xFFFFu) * s.xs;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t w0 = q[i], w8 = q[i] >> 8;
        const uint32_t a = w0 & 0x000F000Fu, b = w8 & 0x000F000Fu;  // low nibbles, bytes 0/2 and 1/3
        const uint32_t e = w0 & 0x00F000F0u, g = w8 & 0x00F000F0u;  // high nibbles (x16)
        const float* x0 = s.v + 4 * i;
        const float* x1 = s.v + 32 + 4 * i;
        s0 = fma_lo(a, x0[0], s0);
        s0 = fma_lo(b, x0[1], s0);
        s0 = fma_hi(a, x0[2], s0);
        s0 = fma_hi(b, x0[3], s0);
        s1 = fma_lo(e, x1[0], s1);
        s1 = fma_lo(g, x1[1], s1);
        s1 = fma_hi(e, x1[2], s1);
        s1 = fma_hi(g, x1[3], s1);
      }
    } else {
      d = f16_to_f32(f.hd.x & 0xFFFFu) * s.xs;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t w0 = q[i], w8 = q[i] >> 8;
        const uint32_t a = w0 & 0x000F000Fu, b = w8 & 0x000F000Fu;
        const uint32_t e = w0 & 0x00F000F0u, g = w8 & 0x00F000F0u;
        s0 = dot2_lo_hi(a, s.h[4 * i + 0], s0);
        s0 = dot2_lo_hi(b, s.h[4 * i + 1], s0);
        s1 = dot2_lo_hi(e, s.h[4 * i + 2], s1);
        s1 = dot2_lo_hi(g, s.h[4 * i + 3], s1);
      }
    }
    const float t = fmaf(cvt_ubyte<1>(sc) * 0.0625f, s1, cvt_ubyte<0>(sc) * s0);
    const float mm = fmaf(cvt_ubyte<1>(mn), s.s1, cvt_ubyte<0>(mn) * s.s0);
    return fmaf(d, t, -dmin * mm);
  }

  // dot<XT> for NBR activation rows at once: the header decode and the code
  // masks are computed once, then each row's sums follow dot's operations in
  // dot's order, so out[m] equals dot(f, s[m]) bit for bit.
  template <typename XT, int NBR>
  __device__ void dot_rows(const Frag& f, const XSliceT<XT>* s, float* out) const {
    const uint32_t t1 = f.hd.y >> sh, t2 = f.hd.z >> sh, t3 = f.hd.w >> sh;
    const uint32_t sc = ((hi ? t3 : t1) & mask_a) | ((t1 >> 2) & mask_b);
    const uint32_t mn = ((hi ? (t3 >> 4) : t2) & mask_a) | ((t2 >> 2) & mask_b);
    const float dmin = f16_to_f32(f.hd.x >> 16);
    const float d16 = f16_to_f32(f.hd.x & 0xFFFFu);

    const uint32_t q[8] = {f.qa.x, f.qa.y, f.qa.z, f.qa.w, f.qb.x, f.qb.y, f.qb.z, f.qb.w};
    float s0[NBR], s1[NBR];
#pragma unroll
    for (int m = 0; m < NBR; ++m) s0[m] = s1[m] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t w0 = q[i], w8 = q[i] >> 8;
      const uint32_t a = w0 & 0x000F000Fu, b = w8 & 0x000F000Fu;
      const uint32_t e = w0 & 0x00F000F0u, g = w8 & 0x00F000F0u;
#pragma unroll
      for (int m = 0; m < NBR; ++m) {
        if constexpr (__is_same(XT, float)) {
          const float* x0 = s[m].v + 4 * i;
          const float* x1 = s[m].v + 32 + 4 * i;
          s0[m] = fma_lo(a, x0[0], s0[m]);
          s0[m] = fma_lo(b, x0[1], s0[m]);
          s0[m] = fma_hi(a, x0[2], s0[m]);
          s0[m] = fma_hi(b, x0[3], s0[m]);
          s1[m] = fma_lo(e, x1[0], s1[m]);
          s1[m] = fma_lo(g, x1[1], s1[m]);
          s1[m] = fma_hi(e, x1[2], s1[m]);
          s1[m] = fma_hi(g, x1[3], s1[m]);
        } else {
          s0[m] = dot2_lo_hi(a, s[m].h[4 * i + 0], s0[m]);
          s0[m] = dot2_lo_hi(b, s[m].h[4 * i + 1], s0[m]);
          s1[m] = dot2_lo_hi(e, s[m].h[4 * i + 2], s1[m]);
          s1[m] = dot2_lo_hi(g, s[m].h[4 * i + 3], s1[m]);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < NBR; ++m) {
      float d;
      if constexpr (__is_same(XT, float))
        d = d16 * s[m].xs;
      else
        d = d16 * s[m].xs;
      const float t = fmaf(cvt_ubyte<1>(sc) * 0.0625f, s1[m], cvt_ubyte<0>(sc) * s0[m]);
      const float mm = fmaf(cvt_ubyte<1>(mn), s[m].s1, cvt_ubyte<0>(mn) * s[m].s0);
      out[m] = fmaf(d, t, -dmin * mm);
    }
  }
};

// The same GEMV over the plane layout of planes.h: the lane mapping, the
// arithmetic and its order are Q4KPolicy's, only the addresses differ.  Lane
// (j, c) reads block j's header from the header plane (16 headers = 256
// consecutive bytes per instruction; the four lanes of a block share one
// address) and its two code quarters from planes A and B, where one
// instruction of the wave reads 16 blocks x 64 bytes = 1 KB of consecutive
// bytes that no other instruction reads.  Those code loads carry the
// nontemporal hint; the header loads, whose lines are shared with the next
// row's headers, do not.
struct Q4KPlanesPolicy : Q4KPolicy {
  const uint8_t* hdr;
  const uint8_t* qa;
  const uint8_t* qb;
  uint32_t nb;

  __device__ Q4KPlanesPolicy(const uint8_t* w, uint64_t a, int cols, int kslot, int lane)
      : Q4KPolicy(w, 0, cols, kslot, lane) {
    nb = static_cast<uint32_t>(cols / 256);
    const int jc = col0 / 256;  // this lane's block in the row (clamped as in Q4KPolicy)
    hdr = w + static_cast<size_t>(jc) * 16;
    qa = w + a + static_cast<size_t>(jc) * 64 + 16 * c;
    qb = w + 5 * a + static_cast<size_t>(jc) * 64 + 16 * c;
  }

  __device__ void load(int row, Frag& f) const {
    const size_t b = static_cast<size_t>(row) * nb;
    f.hd = ld16(hdr + 16 * b);
    f.qa = ld16_stream(qa + 64 * b);
    f.qb = ld16_stream(qb + 64 * b);
  }
};

hipError_t gemv_q4_k(const GemvCall* calls, int n, int x_dtype, int64_t batch, hipStream_t s) {
  return launch_gemv<Q4KPolicy>(calls, n, x_dtype, batch, s);
}

hipError_t gemv_q4_k_planes(const GemvCall* calls, int n, int x_dtype, int64_t batch,
                            hipStream_t s) {
  return launch_gemv<Q4KPlanesPolicy>(calls, n, x_dtype, batch, s);
}

hipError_t gemv_q4_k_pair(const GemvCall& a, const void* b_w, float* b_y, int x_dtype, int64_t batch,
                          bool planes, bool glu, hipStream_t s) {
  return planes ? launch_gemv_pair<Q4KPlanesPolicy>(a, b_w, b_y, x_dtype, batch, glu, s)
                : launch_gemv_pair<Q4KPolicy>(a, b_w, b_y, x_dtype, batch, glu, s);
}

hipError_t gemv_q4_k_rows(const GemvCall* calls, int n, int x_dtype, int64_t batch, bool planes,
                          hipStream_t s) {
  return planes ? launch_gemv_rows<Q4KPlanesPolicy>(calls, n, x_dtype, batch, s)
                : launch_gemv_rows<Q4KPolicy>(calls, n, x_dtype, batch, s);
}

}  // namespace qmv
