// Q6_K decode GEMV for gfx950.
//
// Block (VTE, feature list: llama.cpp's reference Q6_K layout), 210 bytes:
// ql[128] | qh[64] | sc[16] int8 | d fp16.  Weight t = 128h + 32g + l has
// low4 = nibble (g>>1) of ql[64h + 32(g&1) + l], high2 = bits 2g of
// qh[32h + l], q6 = low4 | high2 << 4 and w = d * sc[t/16] * (q6 - 32).
// Blocks are 2-byte aligned; loads are unaligned global_load_dwordx4.
//
// Lane mapping: four lanes per block, lane (h, i) owns l in [16i, 16i+16) of
// half h for all four g: 64 weights in sub-blocks 8h + 2g + i, read as three
// 16-byte loads (ql for g = 0/2, ql for g = 1/3, qh) plus the 8 sub-scales of
// half h and d.  A wave covers 16 blocks.  The 6-bit codes are assembled four
// per dword:
//   q6 = (ql >> 4(g>>1)) & 0x0F0F0F0F  |  (qh shifted so bits 2g land on 4..5) & 0x30303030
// and enter the FMAs two per dword as fp16 subnormals (device_util.h):
//   partial = d sum_g sc_g (2^24 S_g - 32 X_g)
// one v_fma_mix_f32 per weight for fp32 activations; fp16 and bf16 ones enter
// as fp16 (bf16 scaled per lane by a power of two, exact; half_scale_exp),
// two products per v_dot2_f32_f16 (exact: 6 + 11 significant bits), with
// 2^(24+e) in place of 2^24.
#include "gemv_skeleton.h"

namespace qmv {

struct Q6KPolicy {
  static constexpr int kColsPerWave = 16 * 256;
  static constexpr int kXElems = 64;
  struct XSlice {
    float v[64];  // v[16g + t] = x[col0 + 32g + t], scaled by 2^-e (f32_slice_factor)
    float s[4];   // sums of each group's 16 unscaled activations
    float xs;     // 2^(24 + e)
  };
  struct XSliceHalf {
    h2_t h[32];  // h[8g + 2k + p]: pair p of dword k of group g: (4k, 4k+2), (4k+1, 4k+3)
    float s[4];  // fp32 sums of each group's 16 activations
    float xs;    // 2^(24 + e)
  };
  template <typename XT>
  using XSliceT = typename XSliceFor<XT, XSlice, XSliceHalf>::type;
  struct Frag {
    uint4 la, lb, qh;
    uint2 sc;
    uint32_t d;
  };

  const uint8_t* base;
  uint32_t row_bytes;
  int col0;
  int h, i;
  bool ok;

  __device__ Q6KPolicy(const uint8_t* w, uint64_t, int cols, int kslot, int lane) {
    const int nb = cols / 256;
    const int j = kslot * 16 + (lane >> 2);
    h = (lane >> 1) & 1;
    i = lane & 1;
    ok = j < nb;
    const int jc = ok ? j : nb - 1;  // lanes past the row end read a valid block
    row_bytes = static_cast<uint32_t>(nb) * 210;
    base = w + static_cast<size_t>(jc) * 210;
    col0 = jc * 256 + 128 * h + 16 * i;
  }

  template <class XS>
  __device__ void load_x_raw(const XS& x, uint4* raw) const {
    constexpr int kPer = 16 * static_cast<int>(sizeof(typename XS::elem)) / 16;  // uint4 words per run of 16
#pragma unroll
    for (int g = 0; g < 4; ++g) qmv::load_x_raw<16>(x, col0 + 32 * g, raw + g * kPer);
  }

  template <typename XT>
  __device__ void finish_x(const uint4* raw, XSliceT<XT>& s) const {
    float v[64];  // v[16g + t] = x[col0 + 32g + t]
    float* dst = v;
    if constexpr (__is_same(XT, float)) dst = s.v;
    x_to_f32<64>(raw, dst, static_cast<const XT*>(nullptr));
    if constexpr (__is_same(XT, float)) {
      float un;
      const float f = f32_slice_factor<64>(s.v, ok, s.xs, un);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        s.s[g] = 0.f;
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          s.v[16 * g + t] *= f;
          s.s[g] += s.v[16 * g + t];
        }
        s.s[g] *= un;
      }
    } else {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        s.s[g] = 0.f;
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          dst[16 * g + t] = ok ? dst[16 * g + t] : 0.f;
          s.s[g] += dst[16 * g + t];
        }
      }
      const int e = half_scale_exp<XT, 64>(v);
      s.xs = __builtin_amdgcn_ldexpf(1.0f, 24 + e);
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float* x = v + 16 * g + 4 * k;
          s.h[8 * g + 2 * k] = h2_t{scaled_f16(x[0], e), scaled_f16(x[2], e)};
          s.h[8 * g + 2 * k + 1] = h2_t{scaled_f16(x[1], e), scaled_f16(x[3], e)};
        }
    }
  }

  __device__ void load(int row, Frag& f) const {
    const uint8_t* p = base + static_cast<size_t>(row) * row_bytes;
    f.la = ld16_any(p + 64 * h + 16 * i);
    f.lb = ld16_any(p + 64 * h + 32 + 16 * i);
    f.qh = ld16_any(p + 128 + 32 * h + 16 * i);
    f.sc = ld8_any(p + 192 + 8 * h);
    f.d = ld_u16(p + 208);
  }

  template <typename XT>
  __device__ float dot(const Frag& f, const XSliceT<XT>& s) const {
    const uint32_t la[4] = {f.la.x, f.la.y, f.la.z, f.la.w};
    const uint32_t lb[4] = {f.lb.x, f.lb.y, f.lb.z, f.lb.w};
    const uint32_t qh[4] = {f.qh.x, f.qh.y, f.qh.z, f.qh.w};
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t q6[4] = {
          (la[k] & 0x0F0F0F0Fu) | ((qh[k] << 4) & 0x30303030u),
          (lb[k] & 0x0F0F0F0Fu) | ((qh[k] << 2) & 0x30303030u),
          ((la[k] >> 4) & 0x0F0F0F0Fu) | (qh[k] & 0x30303030u),
          ((lb[k] >> 4) & 0x0F0F0F0Fu) | ((qh[k] >> 2) & 0x30303030u)};
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t a = q6[g] & 0x003F003Fu, b = (q6[g] >> 8) & 0x003F003Fu;  // l 0,2 | 1,3
        if constexpr (__is_same(XT, float)) {
          const float* x = s.v + 16 * g + 4 * k;
          acc[g] = fma_lo(a, x[0], acc[g]);
          acc[g] = fma_lo(b, x[1], acc[g]);
          acc[g] = fma_hi(a, x[2], acc[g]);
          acc[g] = fma_hi(b, x[3], acc[g]);
        } else {
          acc[g] = dot2_lo_hi(a, s.h[8 * g + 2 * k], acc[g]);
          acc[g] = dot2_lo_hi(b, s.h[8 * g + 2 * k + 1], acc[g]);
        }
      }
    }
    // sub-scale of g is sc[8h + 2g + i] = byte (2g + i) of the 8 loaded scales
    float t = 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t word = g < 2 ? f.sc.x : f.sc.y;
      const int sc = static_cast<int8_t>((word >> (8 * (2 * (g & 1) + i))) & 0xFFu);
      float xs;
      if constexpr (__is_same(XT, float))
        xs = s.xs;
      else
        xs = s.xs;
      t = fmaf(static_cast<float>(sc), fmaf(xs, acc[g], -32.f * s.s[g]), t);
    }
    return f16_to_f32(f.d) * t;
  }

  // dot<XT> for NBR activation rows at once: the 6-bit codes and the
  // sub-scales are assembled once, then each row's sums follow dot's
  // operations in dot's order, so out[m] equals dot(f, s[m]) bit for bit.
  template <typename XT, int NBR>
  __device__ void dot_rows(const Frag& f, const XSliceT<XT>* s, float* out) const {
    const uint32_t la[4] = {f.la.x, f.la.y, f.la.z, f.la.w};
    const uint32_t lb[4] = {f.lb.x, f.lb.y, f.lb.z, f.lb.w};
    const uint32_t qh[4] = {f.qh.x, f.qh.y, f.qh.z, f.qh.w};
    float acc[NBR][4];
#pragma unroll
    for (int m = 0; m < NBR; ++m)
#pragma unroll
      for (int g = 0; g < 4; ++g) acc[m][g] = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t q6[4] = {
          (la[k] & 0x0F0F0F0Fu) | ((qh[k] << 4) & 0x30303030u),
          (lb[k] & 0x0F0F0F0Fu) | ((qh[k] << 2) & 0x30303030u),
          ((la[k] >> 4) & 0x0F0F0F0Fu) | (qh[k] & 0x30303030u),
          ((lb[k] >> 4) & 0x0F0F0F0Fu) | ((qh[k] >> 2) & 0x30303030u)};
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t a = q6[g] & 0x003F003Fu, b = (q6[g] >> 8) & 0x003F003Fu;
#pragma unroll
        for (int m = 0; m < NBR; ++m) {
          if constexpr (__is_same(XT, float)) {
            const float* x = s[m].v + 16 * g + 4 * k;
            acc[m][g] = fma_lo(a, x[0], acc[m][g]);
            acc[m][g] = fma_lo(b, x[1], acc[m][g]);
            acc[m][g] = fma_hi(a, x[2], acc[m][g]);
            acc[m][g] = fma_hi(b, x[3], acc[m][g]);
          } else {
            acc[m][g] = dot2_lo_hi(a, s[m].h[8 * g + 2 * k], acc[m][g]);
            acc[m][g] = dot2_lo_hi(b, s[m].h[8 * g + 2 * k + 1], acc[m][g]);
          }
        }
      }
    }
    float scf[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t word = g < 2 ? f.sc.x : f.sc.y;
      scf[g] = static_cast<float>(static_cast<int8_t>((word >> (8 * (2 * (g & 1) + i))) & 0xFFu));
    }
    const float d = f16_to_f32(f.d);
#pragma unroll
    for (int m = 0; m < NBR; ++m) {
      float xs;
      if constexpr (__is_same(XT, float))
        xs = s[m].xs;
      else
        xs = s[m].xs;
      float t = 0.f;
#pragma unroll
      for (int g = 0; g < 4; ++g) t = fmaf(scf[g], fmaf(xs, acc[m][g], -32.f * s[m].s[g]), t);
      out[m] = d * t;
    }
  }
};

// The same GEMV over the Q6_K plane layout of planes.h: lane mapping,
// arithmetic and its order are Q6KPolicy's.  Lane p = 2h + i of block j reads
// its two ql chunks and its qh chunk from the L0, L1 and QH planes, where one
// instruction of the wave reads 16 blocks x 64 bytes = 1 KB of consecutive
// bytes that no other instruction reads (nontemporal loads), and its eight
// sub-scales and d from the SC and D planes (plain loads: those lines are
// shared with the neighbouring rows' instructions).
struct Q6KPlanesPolicy : Q6KPolicy {
  const uint8_t* l0;
  const uint8_t* l1;
  const uint8_t* qh;
  const uint8_t* scp;
  const uint8_t* dp;
  uint32_t nb;

  __device__ Q6KPlanesPolicy(const uint8_t* w, uint64_t a, int cols, int kslot, int lane)
      : Q6KPolicy(w, 0, cols, kslot, lane) {
    nb = static_cast<uint32_t>(cols / 256);
    const int jc = (col0 - 128 * h - 16 * i) / 256;  // this lane's block (clamped as in Q6KPolicy)
    const int p = 2 * h + i;
    l0 = w + static_cast<size_t>(jc) * 64 + 16 * p;
    l1 = w + 4 * a + static_cast<size_t>(jc) * 64 + 16 * p;
    qh = w + 8 * a + static_cast<size_t>(jc) * 64 + 16 * p;
    scp = w + 12 * a + static_cast<size_t>(jc) * 16 + 8 * h;
    dp = w + 13 * a + static_cast<size_t>(jc) * 2;
  }

  __device__ void load(int row, Frag& f) const {
    const size_t b = static_cast<size_t>(row) * nb;
    f.la = ld16_stream(l0 + 64 * b);
    f.lb = ld16_stream(l1 + 64 * b);
    f.qh = ld16_stream(qh + 64 * b);
    f.sc = ld8_any(scp + 16 * b);
    f.d = ld_u16(dp + 2 * b);
  }
};

hipError_t gemv_q6_k_rows(const GemvCall* calls, int n, int x_dtype, int64_t batch, bool planes,
                          hipStream_t s) {
  return planes ? launch_gemv_rows<Q6KPlanesPolicy>(calls, n, x_dtype, batch, s)
                : launch_gemv_rows<Q6KPolicy>(calls, n, x_dtype, batch, s);
}

hipError_t gemv_q6_k(const GemvCall* calls, int n, int x_dtype, int64_t batch, hipStream_t s) {
  return launch_gemv<Q6KPolicy>(calls, n, x_dtype, batch, s);
}

hipError_t gemv_q6_k_planes(const GemvCall* calls, int n, int x_dtype, int64_t batch,
                            hipStream_t s) {
  return launch_gemv<Q6KPlanesPolicy>(calls, n, x_dtype, batch, s);
}

hipError_t gemv_q6_k_pair(const GemvCall& a, const void* b_w, float* b_y, int x_dtype, int64_t batch,
                          bool planes, bool glu, hipStream_t s) {
  return planes ? launch_gemv_pair<Q6KPlanesPolicy>(a, b_w, b_y, x_dtype, batch, glu, s)
                : launch_gemv_pair<Q6KPolicy>(a, b_w, b_y, x_dtype, batch, glu, s);
}

}  // namespace qmv
