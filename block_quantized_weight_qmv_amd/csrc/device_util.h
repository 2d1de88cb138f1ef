// Device helpers shared by the gfx950 kernels of libqmv: fp16/bf16 decoding,
// activation loads converted to fp32, and the wave64 sum.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmv {

// Activation element types as seen by the kernels.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float f16_to_f32(uint32_t bits) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits) {
  return __uint_as_float(bits << 16);
}

// 16 bytes from an address with any alignment.  On gfx950 the compiler emits
// one global_load_dwordx4 (unaligned global access is enabled for amdhsa).
__device__ __forceinline__ uint4 load16_any(const uint8_t* p) {
  uint4 v;
  __builtin_memcpy(&v, p, 16);
  return v;
}

__device__ __forceinline__ uint2 load8_any(const uint8_t* p) {
  uint2 v;
  __builtin_memcpy(&v, p, 8);
  return v;
}

__device__ __forceinline__ uint32_t load_u16(const uint8_t* p) {
  uint16_t v;
  __builtin_memcpy(&v, p, 2);
  return v;
}

// N contiguous activations starting at a 16-byte aligned element, as fp32.
template <int N>
__device__ __forceinline__ void load_x(const float* p, float* out) {
#pragma unroll
  for (int i = 0; i < N; i += 4) {
    const float4 v = *reinterpret_cast<const float4*>(p + i);
    out[i] = v.x; out[i + 1] = v.y; out[i + 2] = v.z; out[i + 3] = v.w;
  }
}

template <int N>
__device__ __forceinline__ void load_x(const _Float16* p, float* out) {
#pragma unroll
  for (int i = 0; i < N; i += 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(p + i);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      out[i + 2 * k] = f16_to_f32(w[k] & 0xFFFFu);
      out[i + 2 * k + 1] = f16_to_f32(w[k] >> 16);
    }
  }
}

template <int N>
__device__ __forceinline__ void load_x(const bf16_t* p, float* out) {
#pragma unroll
  for (int i = 0; i < N; i += 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(p + i);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      out[i + 2 * k] = __uint_as_float(w[k] << 16);
      out[i + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
  }
}

// Byte b of a dword, converted to fp32 (v_cvt_f32_ubyte{0..3}).
template <int B>
__device__ __forceinline__ float ubyte(uint32_t v) {
  return static_cast<float>((v >> (8 * B)) & 0xFFu);
}

// Sum over the 64 lanes of a wave, returned to every lane.  Fixed order:
// quad butterflies, half-row and row mirrors, then row broadcasts 15 and 31
// (lane 63 ends with the total), read back with readlane.
__device__ __forceinline__ float wave_sum(float v) {
  int iv;
  iv = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
  v += __int_as_float(iv);
  iv = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
  v += __int_as_float(iv);
  iv = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false); // row_half_mirror
  v += __int_as_float(iv);
  iv = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false); // row_mirror
  v += __int_as_float(iv);
  iv = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false); // row_bcast:15
  v += __int_as_float(iv);
  iv = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false); // row_bcast:31
  v += __int_as_float(iv);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Balanced contiguous partition of n items into parts: [begin, end) of part p.
__device__ __forceinline__ int part_begin(int p, int n, int parts) {
  return static_cast<int>((static_cast<int64_t>(p) * n) / parts);
}

}  // namespace qmv
