// Dequantization kernels: packed blocks -> dense [rows][cols] fp32 / fp16 / bf16.
//
// VTE (kyuubyn.github.io/VTE), feature list: blocks are decoded byte for byte
// in llama.cpp's reference layout and checked against a NumPy decoder.  Each
// thread decodes four consecutive weights of one row, reading the bytes named
// by the layout tables below one at a time, and stores them as one vector.
//
// Q5_K (hipEngine 0.3.0, "GGUF Support", read as GGUF's published block) is
// decoded the same way.
//
// Exactness: every product here is exact in fp32 (Q8_0 11+7 bits, Q6_K
// 11 + 12 bits, INT4 11+3 bits, Q4_K d*sc*u 21 bits, Q5_K 22 bits, dmin*m
// 17 bits), so the fp32 result is the exact weight, except Q4_K and Q5_K,
// which round once at the subtraction.  fp16 / bf16 outputs are that fp32 value rounded to nearest even.
#include "device_util.h"
#include "launch.h"
#include "planes.h"

namespace qmv {

__device__ __forceinline__ uint32_t ld_u8(const uint8_t* p) { return *p; }
__device__ __forceinline__ uint32_t ld_le16(const uint8_t* p) { return p[0] | (p[1] << 8); }

// Q8_0: d fp16 | q[32] int8; w = d*q.
__device__ __forceinline__ void dq_q8_0(const uint8_t* row, int k, float* w) {
  const uint8_t* b = row + (k / 32) * 34;
  const float d = f16_to_f32(ld_le16(b));
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int t = (k + e) % 32;
    w[e] = d * static_cast<float>(static_cast<int8_t>(ld_u8(b + 2 + t)));
  }
}

// Six-bit scale and min of sub-block s from the twelve scale bytes of a Q4_K or
// Q5_K block.
__device__ __forceinline__ void k_scale_min(const uint8_t* sc, int s, uint32_t& scale,
                                            uint32_t& mn) {
  if (s < 4) {
    scale = ld_u8(sc + s) & 63;
    mn = ld_u8(sc + s + 4) & 63;
  } else {
    scale = (ld_u8(sc + s + 4) & 15) | ((ld_u8(sc + s - 4) >> 6) << 4);
    mn = (ld_u8(sc + s + 4) >> 4) | ((ld_u8(sc + s) >> 6) << 4);
  }
}

// Q4_K: d | dmin | scales[12] | qs[128]; t = 64c + 32h + l, u = nibble h of qs[32c+l].
__device__ __forceinline__ void dq_q4_k(const uint8_t* row, int k, float* w) {
  const uint8_t* b = row + (k / 256) * 144;
  const float d = f16_to_f32(ld_le16(b));
  const float dmin = f16_to_f32(ld_le16(b + 2));
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int t = (k + e) % 256;
    const int c = t >> 6, h = (t >> 5) & 1, l = t & 31, s = t >> 5;
    uint32_t scale, mn;
    k_scale_min(b + 4, s, scale, mn);
    const uint32_t u = (ld_u8(b + 16 + 32 * c + l) >> (4 * h)) & 15;
    w[e] = (d * static_cast<float>(scale)) * static_cast<float>(u) - dmin * static_cast<float>(mn);
  }
}

// Q4_K in the plane layout (planes.h): the header of block b at 16 b,
// qs[32c + l] at a + 64 b + 16 c + l (l < 16) or 5 a + 64 b + 16 c + l - 16.
// Same decode as dq_q4_k, byte addresses aside.
constexpr int kQ4KPlanes = 0x102;  // kernel template tag, not a public format

__device__ __forceinline__ void dq_q4_k_planes(const uint8_t* w, uint64_t a, int64_t b, int k,
                                               float* out) {
  const uint8_t* h = w + 16 * b;
  const float d = f16_to_f32(ld_le16(h));
  const float dmin = f16_to_f32(ld_le16(h + 2));
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int t = (k + e) % 256;
    const int c = t >> 6, hh = (t >> 5) & 1, l = t & 31, s = t >> 5;
    uint32_t scale, mn;
    k_scale_min(h + 4, s, scale, mn);
    const uint8_t* q = l < 16 ? w + a + 64 * b + 16 * c + l : w + 5 * a + 64 * b + 16 * c + (l - 16);
    const uint32_t u = (ld_u8(q) >> (4 * hh)) & 15;
    out[e] = (d * static_cast<float>(scale)) * static_cast<float>(u) - dmin * static_cast<float>(mn);
  }
}

// Q5_K: d | dmin | scales[12] | qh[32] | qs[128]; t = 64c + 32h + l,
// u = (nibble h of qs[32c+l]) | (bit 2c+h of qh[l]) << 4.
__device__ __forceinline__ void dq_q5_k(const uint8_t* row, int k, float* w) {
  const uint8_t* b = row + (k / 256) * 176;
  const float d = f16_to_f32(ld_le16(b));
  const float dmin = f16_to_f32(ld_le16(b + 2));
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int t = (k + e) % 256;
    const int c = t >> 6, h = (t >> 5) & 1, l = t & 31, s = t >> 5;
    uint32_t scale, mn;
    k_scale_min(b + 4, s, scale, mn);
    const uint32_t lo = (ld_u8(b + 48 + 32 * c + l) >> (4 * h)) & 15;
    const uint32_t hi = (ld_u8(b + 16 + l) >> s) & 1;
    const uint32_t u = lo | (hi << 4);
    w[e] = (d * static_cast<float>(scale)) * static_cast<float>(u) - dmin * static_cast<float>(mn);
  }
}

// Q6_K: ql[128] | qh[64] | sc[16] | d; t = 128h + 32g + l.
__device__ __forceinline__ void dq_q6_k(const uint8_t* row, int k, float* w) {
  const uint8_t* b = row + (k / 256) * 210;
  const float d = f16_to_f32(ld_le16(b + 208));
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int t = (k + e) % 256;
    const int h = t >> 7, g = (t >> 5) & 3, l = t & 31;
    const uint32_t lo = (ld_u8(b + 64 * h + 32 * (g & 1) + l) >> (4 * (g >> 1))) & 15;
    const uint32_t hi = (ld_u8(b + 128 + 32 * h + l) >> (2 * g)) & 3;
    const int q6 = static_cast<int>(lo | (hi << 4)) - 32;
    const int sc = static_cast<int8_t>(ld_u8(b + 192 + t / 16));
    w[e] = (d * static_cast<float>(sc)) * static_cast<float>(q6);
  }
}

// Q6_K in the plane layout (planes.h): ql[64h + 32m + 16i + t] of block b at
// 4 m a + 64 b + 16 (2h + i) + t, qh[32h + 16i + t] at 8 a + 64 b +
// 16 (2h + i) + t, sc[k] at 12 a + 16 b + k, d at 13 a + 2 b.  Same decode as
// dq_q6_k, byte addresses aside.
constexpr int kQ6KPlanes = 0x103;  // kernel template tag, not a public format
constexpr int kQ5KPlanes = 0x105;  // kernel template tag, not a public format

// Q5_K in the plane layout (planes.h): header of block b at 16 b, qh[l] at
// a + 16 b + l (l < 16) or 2 a + 16 b + l - 16, qs[32c + l] at
// 3 a + 64 b + 16 c + l (l < 16) or 7 a + 64 b + 16 c + l - 16.  Same decode
// as dq_q5_k, byte addresses aside.
__device__ __forceinline__ void dq_q5_k_planes(const uint8_t* w, uint64_t a, int64_t b, int k,
                                               float* out) {
  const uint8_t* h = w + 16 * b;
  const float d = f16_to_f32(ld_le16(h));
  const float dmin = f16_to_f32(ld_le16(h + 2));
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int t = (k + e) % 256;
    const int c = t >> 6, hh = (t >> 5) & 1, l = t & 31, s = t >> 5;
    uint32_t scale, mn;
    k_scale_min(h + 4, s, scale, mn);
    const uint8_t* q = l < 16 ? w + 3 * a + 64 * b + 16 * c + l : w + 7 * a + 64 * b + 16 * c + (l - 16);
    const uint8_t* qh = l < 16 ? w + a + 16 * b + l : w + 2 * a + 16 * b + (l - 16);
    const uint32_t lo = (ld_u8(q) >> (4 * hh)) & 15;
    const uint32_t hi = (ld_u8(qh) >> s) & 1;
    const uint32_t u = lo | (hi << 4);
    out[e] = (d * static_cast<float>(scale)) * static_cast<float>(u) - dmin * static_cast<float>(mn);
  }
}

__device__ __forceinline__ void dq_q6_k_planes(const uint8_t* w, uint64_t a, int64_t b, int k,
                                               float* out) {
  const float d = f16_to_f32(ld_le16(w + 13 * a + 2 * b));
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int t = (k + e) % 256;
    const int h = t >> 7, g = (t >> 5) & 3, l = t & 31;
    const int m = g & 1, i = l >> 4, tt = l & 15, p = 2 * h + i;
    const uint32_t lo = (ld_u8(w + 4 * m * a + 64 * b + 16 * p + tt) >> (4 * (g >> 1))) & 15;
    const uint32_t hi = (ld_u8(w + 8 * a + 64 * b + 16 * p + tt) >> (2 * g)) & 3;
    const int q6 = static_cast<int>(lo | (hi << 4)) - 32;
    const int sc = static_cast<int8_t>(ld_u8(w + 12 * a + 16 * b + t / 16));
    out[e] = (d * static_cast<float>(sc)) * static_cast<float>(q6);
  }
}

// INT4_G128: codes plane (u_{2j} low nibble, u_{2j+1} high) then fp16 scales.
__device__ __forceinline__ void dq_int4(const uint8_t* codes_row, const uint8_t* scales_row,
                                        int k, float* w) {
  const float s = f16_to_f32(ld_le16(scales_row + 2 * (k / 128)));
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int t = k + e;
    const int u = (ld_u8(codes_row + t / 2) >> (4 * (t & 1))) & 15;
    w[e] = s * static_cast<float>(u - 8);
  }
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t f32_to_f16_rne(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

template <int FMT, int OUT>
__global__ void __launch_bounds__(256)
dequant_kernel(const uint8_t* __restrict__ w, uint64_t scales_offset, int rows, int cols,
               void* __restrict__ out) {
  const int64_t quads_per_row = cols / 4;
  const int64_t total = static_cast<int64_t>(rows) * quads_per_row;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int r = static_cast<int>(idx / quads_per_row);
    const int k = static_cast<int>(idx % quads_per_row) * 4;
    float v[4];
    if (FMT == QMV_Q8_0) {
      dq_q8_0(w + static_cast<size_t>(r) * (cols / 32) * 34, k, v);
    } else if (FMT == QMV_Q4_K) {
      dq_q4_k(w + static_cast<size_t>(r) * (cols / 256) * 144, k, v);
    } else if (FMT == kQ4KPlanes) {
      dq_q4_k_planes(w, scales_offset, static_cast<int64_t>(r) * (cols / 256) + k / 256, k, v);
    } else if (FMT == kQ5KPlanes) {
      dq_q5_k_planes(w, scales_offset, static_cast<int64_t>(r) * (cols / 256) + k / 256, k, v);
    } else if (FMT == kQ6KPlanes) {
      dq_q6_k_planes(w, scales_offset, static_cast<int64_t>(r) * (cols / 256) + k / 256, k, v);
    } else if (FMT == QMV_Q5_K) {
      dq_q5_k(w + static_cast<size_t>(r) * (cols / 256) * 176, k, v);
    } else if (FMT == QMV_Q6_K) {
      dq_q6_k(w + static_cast<size_t>(r) * (cols / 256) * 210, k, v);
    } else {
      dq_int4(w + static_cast<size_t>(r) * (cols / 2),
              w + scales_offset + static_cast<size_t>(r) * (cols / 128) * 2, k, v);
    }
    const size_t o = static_cast<size_t>(r) * cols + k;
    if (OUT == QMV_F32) {
      *reinterpret_cast<float4*>(static_cast<float*>(out) + o) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
      uint32_t h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) h[e] = OUT == QMV_F16 ? f32_to_f16_rne(v[e]) : f32_to_bf16_rne(v[e]);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + o) =
          make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
    }
  }
}

template <int FMT>
static hipError_t dequant_fmt(const qmv_weights& W, void* out, int out_dtype, hipStream_t s) {
  const int rows = static_cast<int>(W.rows), cols = static_cast<int>(W.cols);
  const int64_t total = W.rows * (W.cols / 4);
  const int64_t want = (total + 255) / 256;
  const int grid = static_cast<int>(want < 65536 ? want : 65536);
  const uint8_t* w = static_cast<const uint8_t*>(W.data);
  switch (out_dtype) {
    case QMV_F32:
      hipLaunchKernelGGL((dequant_kernel<FMT, QMV_F32>), dim3(grid), dim3(256), 0, s, w,
                         W.scales_offset, rows, cols, out);
      break;
    case QMV_F16:
      hipLaunchKernelGGL((dequant_kernel<FMT, QMV_F16>), dim3(grid), dim3(256), 0, s, w,
                         W.scales_offset, rows, cols, out);
      break;
    case QMV_BF16:
      hipLaunchKernelGGL((dequant_kernel<FMT, QMV_BF16>), dim3(grid), dim3(256), 0, s, w,
                         W.scales_offset, rows, cols, out);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t dequant(const qmv_weights& W, void* out, int out_dtype, hipStream_t s) {
  if (W.layout == QMV_LAYOUT_PLANES) {
    if (W.fmt == QMV_Q4_K) return dequant_fmt<kQ4KPlanes>(W, out, out_dtype, s);
    if (W.fmt == QMV_Q5_K) return dequant_fmt<kQ5KPlanes>(W, out, out_dtype, s);
    if (W.fmt == QMV_Q6_K) return dequant_fmt<kQ6KPlanes>(W, out, out_dtype, s);
    return hipErrorInvalidValue;
  }
  switch (W.fmt) {
    case QMV_Q8_0: return dequant_fmt<QMV_Q8_0>(W, out, out_dtype, s);
    case QMV_Q4_K: return dequant_fmt<QMV_Q4_K>(W, out, out_dtype, s);
    case QMV_Q5_K: return dequant_fmt<QMV_Q5_K>(W, out, out_dtype, s);
    case QMV_Q6_K: return dequant_fmt<QMV_Q6_K>(W, out, out_dtype, s);
    case QMV_INT4_G128: return dequant_fmt<QMV_INT4_G128>(W, out, out_dtype, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qmv
