// Q5_K decode GEMV for gfx950.
//
// Block (hipEngine 0.3.0, "GGUF Support", names the type; the bytes are
// GGUF's published Q5_K block), 176 bytes:
//   d fp16 | dmin fp16 | scales[12] (as Q4_K) | qh[32] | qs[128] (as Q4_K).
// Weight t = 64c + 32h + l: u = (nibble h of qs[32c + l]) | (bit 2c + h of
// qh[l]) << 4, sub-block s = 2c + h, w = d*sc_s*u - dmin*m_s.
//
// Lane mapping as in the Q4_K GEMV: four lanes per block, lane c owns
// qs[32c .. 32c+32) (sub-blocks 2c and 2c+1, activations x[64c .. 64c+64)).
// Every lane also needs bits 2c and 2c+1 of all 32 qh bytes, so each lane
// loads the whole qh array: five 16-byte loads per lane and row (header, qh
// twice, its two qs quarters); the four lanes of a block share those lines.
//
// Arithmetic: the fifth code bit is merged into the fp16-subnormal code
// before the v_fma_mix_f32.  For qs dword i (bytes l = 4i .. 4i+3) the
// matching high bits sit in qh dword i, byte k = l - 4i, at bit 8k + 2c (low
// nibble's sub-block) and 8k + 2c + 1 (high nibble's).  One rotate of that
// dword per code pair puts the bits where the pair needs them:
//   a = bytes 0, 2 low nibbles at bits 0-3 / 16-19, fifth bit to 4 / 20
//   b = bytes 1, 3 low nibbles (after >> 8),        fifth bit to 4 / 20
//   e = bytes 0, 2 high nibbles at bits 4-7 / 20-23, fifth bit to 8 / 24
//   g = bytes 1, 3 high nibbles (after >> 8),        fifth bit to 8 / 24
// so a and b carry u (0..31) and e and g carry 16u (0..496) as fp16
// subnormals, and the sums are as in Q4_K:
//   S0 = sum u x 2^-24, S1 = sum 16 u x 2^-24,
//   partial = d 2^24 (sc0 S0 + sc1/16 S1) - dmin (m0 X0 + m1 X1),
// one v_fma_mix_f32 per weight for fp32 activations; for fp16 and bf16
// activations two products per v_dot2_f32_f16 (HalfXSlice; exact, 9 + 11
// significant bits), with 2^(24+e) for the lane's activation scale.
#include "gemv_skeleton.h"

namespace qmv {

struct Q5KPolicy {
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
    uint4 hd, h0, h1, qa, qb;
  };

  const uint8_t* base;
  uint32_t row_bytes;
  int col0;
  int c;
  bool ok;
  bool hi;
  uint32_t sh, mask_a, mask_b;
  uint32_t ra, rb, re, rg;  // right-rotate counts that align the fifth bits

  __device__ Q5KPolicy(const uint8_t* w, uint64_t, int cols, int kslot, int lane) {
    const int nb = cols / 256;
    const int j = kslot * 16 + (lane >> 2);
    c = lane & 3;
    ok = j < nb;
    const int jc = ok ? j : nb - 1;  // lanes past the row end read a valid block
    row_bytes = static_cast<uint32_t>(nb) * 176;
    base = w + static_cast<size_t>(jc) * 176;
    col0 = jc * 256 + c * 64;
    // Scale/min decode of sub-blocks 2c, 2c+1 exactly as in the Q4_K GEMV.
    hi = c >= 2;
    sh = 16u * static_cast<uint32_t>(c & 1);
    mask_a = hi ? 0x0F0Fu : 0x3F3Fu;
    mask_b = hi ? 0x3030u : 0u;
    // bit 8k + 2c -> 8k + 4 (k even), bit 8k + 2c -> 8k - 4 (k odd),
    // bit 8k + 2c + 1 -> 8k + 8 (k even), bit 8k + 2c + 1 -> 8k (k odd).
    const uint32_t c2 = 2u * static_cast<uint32_t>(c);
    ra = (c2 + 28u) & 31u;
    rb = c2 + 4u;
    re = (c2 + 25u) & 31u;
    rg = c2 + 1u;
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
    f.h0 = ld16(p + 16);
    f.h1 = ld16(p + 32);
    f.qa = ld16(p + 48 + 32 * c);
    f.qb = ld16(p + 64 + 32 * c);
  }

  template <typename XT>
  __device__ float dot(const Frag& f, const XSliceT<XT>& s) const {
    const uint32_t t1 = f.hd.y >> sh, t2 = f.hd.z >> sh, t3 = f.hd.w >> sh;
    const uint32_t sc = ((hi ? t3 : t1) & mask_a) | ((t1 >> 2) & mask_b);
    const uint32_t mn = ((hi ? (t3 >> 4) : t2) & mask_a) | ((t2 >> 2) & mask_b);
    float d;
    if constexpr (__is_same(XT, float))
      d = f16_to_f32(f.hd.x & 0xFFFFu) * s.xs;
    else
      d = f16_to_f32(f.hd.x & 0xFFFFu) * s.xs;
    const float dmin = f16_to_f32(f.hd.x >> 16);

    const uint32_t q[8] = {f.qa.x, f.qa.y, f.qa.z, f.qa.w, f.qb.x, f.qb.y, f.qb.z, f.qb.w};
    const uint32_t h[8] = {f.h0.x, f.h0.y, f.h0.z, f.h0.w, f.h1.x, f.h1.y, f.h1.z, f.h1.w};
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t w0 = q[i], w8 = q[i] >> 8;
      const uint32_t a = (w0 & 0x000F000Fu) | (__builtin_rotateright32(h[i], ra) & 0x00100010u);
      const uint32_t b = (w8 & 0x000F000Fu) | (__builtin_rotateright32(h[i], rb) & 0x00100010u);
      const uint32_t e = (w0 & 0x00F000F0u) | (__builtin_rotateright32(h[i], re) & 0x01000100u);
      const uint32_t g = (w8 & 0x00F000F0u) | (__builtin_rotateright32(h[i], rg) & 0x01000100u);
      if constexpr (__is_same(XT, float)) {
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
      } else {
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

  // dot<XT> for NBR activation rows at once: the header decode and the
  // five-bit codes are formed once, then each row's sums follow dot's
  // operations in dot's order, so out[m] equals dot(f, s[m]) bit for bit.
  template <typename XT, int NBR>
  __device__ void dot_rows(const Frag& f, const XSliceT<XT>* s, float* out) const {
    const uint32_t t1 = f.hd.y >> sh, t2 = f.hd.z >> sh, t3 = f.hd.w >> sh;
    const uint32_t sc = ((hi ? t3 : t1) & mask_a) | ((t1 >> 2) & mask_b);
    const uint32_t mn = ((hi ? (t3 >> 4) : t2) & mask_a) | ((t2 >> 2) & mask_b);
    const float d16 = f16_to_f32(f.hd.x & 0xFFFFu);
    const float dmin = f16_to_f32(f.hd.x >> 16);

    const uint32_t q[8] = {f.qa.x, f.qa.y, f.qa.z, f.qa.w, f.qb.x, f.qb.y, f.qb.z, f.qb.w};
    const uint32_t h[8] = {f.h0.x, f.h0.y, f.h0.z, f.h0.w, f.h1.x, f.h1.y, f.h1.z, f.h1.w};
    float s0[NBR], s1[NBR];
#pragma unroll
    for (int m = 0; m < NBR; ++m) s0[m] = s1[m] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t w0 = q[i], w8 = q[i] >> 8;
      const uint32_t a = (w0 & 0x000F000Fu) | (__builtin_rotateright32(h[i], ra) & 0x00100010u);
      const uint32_t b = (w8 & 0x000F000Fu) | (__builtin_rotateright32(h[i], rb) & 0x00100010u);
      const uint32_t e = (w0 & 0x00F000F0u) | (__builtin_rotateright32(h[i], re) & 0x01000100u);
      const uint32_t g = (w8 & 0x00F000F0u) | (__builtin_rotateright32(h[i], rg) & 0x01000100u);
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

// The same GEMV over the Q5_K plane layout of planes.h: lane mapping,
// arithmetic and its order are Q5KPolicy's.  Lane (j, c) reads block j's
// header and both qh halves from the H, QH0 and QH1 planes (plain loads: the
// four lanes of a block share them) and its two code quarters from the QA
// and QB planes, where one instruction of the wave reads 16 blocks x 64 bytes
// = 1 KB of consecutive bytes that no other instruction reads (nontemporal
// loads).
struct Q5KPlanesPolicy : Q5KPolicy {
  const uint8_t* hdr;
  const uint8_t* qh0;
  const uint8_t* qh1;
  const uint8_t* qa;
  const uint8_t* qb;
  uint32_t nb;

  __device__ Q5KPlanesPolicy(const uint8_t* w, uint64_t a, int cols, int kslot, int lane)
      : Q5KPolicy(w, 0, cols, kslot, lane) {
    nb = static_cast<uint32_t>(cols / 256);
    const size_t jc = static_cast<size_t>(col0 / 256);  // this lane's block (clamped as in Q5KPolicy)
    hdr = w + jc * 16;
    qh0 = w + a + jc * 16;
    qh1 = w + 2 * a + jc * 16;
    qa = w + 3 * a + jc * 64 + 16 * c;
    qb = w + 7 * a + jc * 64 + 16 * c;
  }

  __device__ void load(int row, Frag& f) const {
    const size_t b = static_cast<size_t>(row) * nb;
    f.hd = ld16(hdr + 16 * b);
    f.h0 = ld16(qh0 + 16 * b);
    f.h1 = ld16(qh1 + 16 * b);
    f.qa = ld16_stream(qa + 64 * b);
    f.qb = ld16_stream(qb + 64 * b);
  }
};

hipError_t gemv_q5_k_rows(const GemvCall* calls, int n, int x_dtype, int64_t batch, bool planes,
                          hipStream_t s) {
  return planes ? launch_gemv_rows<Q5KPlanesPolicy>(calls, n, x_dtype, batch, s)
                : launch_gemv_rows<Q5KPolicy>(calls, n, x_dtype, batch, s);
}

hipError_t gemv_q5_k(const GemvCall* calls, int n, int x_dtype, int64_t batch, hipStream_t s) {
  return launch_gemv<Q5KPolicy>(calls, n, x_dtype, batch, s);
}

hipError_t gemv_q5_k_planes(const GemvCall* calls, int n, int x_dtype, int64_t batch,
                            hipStream_t s) {
  return launch_gemv<Q5KPlanesPolicy>(calls, n, x_dtype, batch, s);
}

hipError_t gemv_q5_k_pair(const GemvCall& a, const void* b_w, float* b_y, int x_dtype, int64_t batch,
                          bool planes, bool glu, hipStream_t s) {
  return planes ? launch_gemv_pair<Q5KPlanesPolicy>(a, b_w, b_y, x_dtype, batch, glu, s)
                : launch_gemv_pair<Q5KPolicy>(a, b_w, b_y, x_dtype, batch, glu, s);
}

}  // namespace qmv
