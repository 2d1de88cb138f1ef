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
// half h and d.  A wave covers 16 blocks.  For each group of four weights the
// 6-bit codes are assembled in place, four per dword:
//   q6 = (ql >> 4(g>>1)) & 0x0F0F0F0F  |  (qh shifted so bits 2g land on 4..5) & 0x30303030
// then converted with v_cvt_f32_ubyte; per lane and row, in fp32:
//   partial = d * sum_g sc_g * (S_g - 32 X_g)
#include "gemv_skeleton.h"

namespace qmv {

struct Q6KPolicy {
  static constexpr int kColsPerWave = 16 * 256;
  struct Params {
    const uint8_t* w;
  };
  struct XSlice {
    float v[64];  // v[16g + t] = x[col0 + 32g + t]
    float s[4];
  };
  struct Frag {
    uint4 la, lb, qh;
    uint2 sc;
    uint32_t d;
  };

  const uint8_t* base;
  size_t row_bytes;
  int col0;
  int h, i;
  bool ok;

  __device__ Q6KPolicy(const Params& p, int cols, int kslot, int lane) {
    const int nb = cols / 256;
    const int j = kslot * 16 + (lane >> 2);
    h = (lane >> 1) & 1;
    i = lane & 1;
    ok = j < nb;
    row_bytes = static_cast<size_t>(nb) * 210;
    base = p.w + static_cast<size_t>(j) * 210;
    col0 = j * 256 + 128 * h + 16 * i;
  }

  template <typename XT>
  __device__ void load_x(const XT* x, XSlice& s) const {
#pragma unroll
    for (int g = 0; g < 4; ++g) s.s[g] = 0.f;
    if (!ok) {
#pragma unroll
      for (int k = 0; k < 64; ++k) s.v[k] = 0.f;
      return;
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      qmv::load_x<16>(x + col0 + 32 * g, s.v + 16 * g);
#pragma unroll
      for (int t = 0; t < 16; ++t) s.s[g] += s.v[16 * g + t];
    }
  }

  __device__ void load(int row, Frag& f) const {
    const uint8_t* p = base + static_cast<size_t>(row) * row_bytes;
    f.la = load16_any(p + 64 * h + 16 * i);
    f.lb = load16_any(p + 64 * h + 32 + 16 * i);
    f.qh = load16_any(p + 128 + 32 * h + 16 * i);
    f.sc = load8_any(p + 192 + 8 * h);
    f.d = load_u16(p + 208);
  }

  __device__ static void zero(Frag& f) {
    f.la = make_uint4(0, 0, 0, 0);
    f.lb = f.la;
    f.qh = f.la;
    f.sc = make_uint2(0, 0);
    f.d = 0;
  }

  __device__ float dot(const Frag& f, const XSlice& s) const {
    const uint32_t la[4] = {f.la.x, f.la.y, f.la.z, f.la.w};
    const uint32_t lb[4] = {f.lb.x, f.lb.y, f.lb.z, f.lb.w};
    const uint32_t qh[4] = {f.qh.x, f.qh.y, f.qh.z, f.qh.w};
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t q0 = (la[k] & 0x0F0F0F0Fu) | ((qh[k] << 4) & 0x30303030u);
      const uint32_t q1 = (lb[k] & 0x0F0F0F0Fu) | ((qh[k] << 2) & 0x30303030u);
      const uint32_t q2 = ((la[k] >> 4) & 0x0F0F0F0Fu) | (qh[k] & 0x30303030u);
      const uint32_t q3 = ((lb[k] >> 4) & 0x0F0F0F0Fu) | ((qh[k] >> 2) & 0x30303030u);
      const uint32_t qq[4] = {q0, q1, q2, q3};
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        acc[g] = fmaf(ubyte<0>(qq[g]), s.v[16 * g + 4 * k + 0], acc[g]);
        acc[g] = fmaf(ubyte<1>(qq[g]), s.v[16 * g + 4 * k + 1], acc[g]);
        acc[g] = fmaf(ubyte<2>(qq[g]), s.v[16 * g + 4 * k + 2], acc[g]);
        acc[g] = fmaf(ubyte<3>(qq[g]), s.v[16 * g + 4 * k + 3], acc[g]);
      }
    }
    // sub-scale of g is sc[8h + 2g + i] = byte (2g + i) of the 8 loaded scales
    float t = 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t word = g < 2 ? f.sc.x : f.sc.y;
      const int sc = static_cast<int8_t>((word >> (8 * (2 * (g & 1) + i))) & 0xFFu);
      t = fmaf(static_cast<float>(sc), fmaf(-32.f, s.s[g], acc[g]), t);
    }
    return f16_to_f32(f.d) * t;
  }
};

hipError_t gemv_q6_k(const GemvArgs& a) {
  Q6KPolicy::Params prm{static_cast<const uint8_t*>(a.W->data)};
  return launch_gemv<Q6KPolicy>(a, prm);
}

}  // namespace qmv
