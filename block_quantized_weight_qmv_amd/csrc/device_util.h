// Device helpers shared by the gfx950 kernels of libqmv: fp16/bf16 decoding,
// activation loads converted to fp32, and the wave64 sum.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <map>
#include <mutex>
#include <tuple>

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

// Weight loads: plain 128-bit global loads.  Used where several load
// instructions of a wave touch the same 128-byte line (a block header and its
// code quarters): the line stays in L2 between them.
__device__ __forceinline__ uint4 ld16(const uint8_t* p) {  // 16-byte aligned
  return *reinterpret_cast<const uint4*>(p);
}

// Streaming weight loads with the nontemporal hint (global_load_dwordx4 ... nt),
// for access patterns in which every 128-byte line is read by one load
// instruction of one wave and never again.  Measured on gfx950 with 128-bit
// reads: such a stream reaches about 7.0 TB/s with the hint against 5.5-6.1
// without; where three instructions share each line (a block header and two
// code quarters), the hint drops it to 4.8 TB/s: a line marked for early
// eviction is gone before the next instruction asks for it, and is fetched
// again.
__device__ __forceinline__ uint4 ld16_stream(const uint8_t* p) {  // 16-byte aligned
  typedef uint32_t v4_t __attribute__((ext_vector_type(4)));
  const v4_t v = __builtin_nontemporal_load(reinterpret_cast<const v4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

typedef uint32_t u32x4_a1 __attribute__((ext_vector_type(4), aligned(1)));
typedef uint32_t u32x2_a1 __attribute__((ext_vector_type(2), aligned(1)));

// Any alignment: on gfx950 the compiler emits one global_load_dwordx4
// (unaligned global access is enabled for amdhsa).
__device__ __forceinline__ uint4 ld16_any(const uint8_t* p) {
  const u32x4_a1 v = *reinterpret_cast<const u32x4_a1*>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint2 ld8_any(const uint8_t* p) {
  const u32x2_a1 v = *reinterpret_cast<const u32x2_a1*>(p);
  return make_uint2(v.x, v.y);
}

__device__ __forceinline__ uint32_t ld_u16(const uint8_t* p) {  // 2-byte aligned
  return *reinterpret_cast<const uint16_t*>(p);
}

// Small integer codes as fp16 *subnormal* bit patterns.  A 16-bit half holding
// an integer u < 1024 in its low bits is the fp16 value u * 2^-24, so
//   fma(float(half), x, acc)
// is exactly fma(u, x, acc) scaled by 2^-24 (one rounding either way; the
// power-of-two scale is undone once per row).  The compiler folds the fp16
// operand into v_fma_mix_f32 with op_sel, so two codes masked out of one
// dword (bits 0-15 and 16-31) feed two FMAs with no conversion instruction.
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float fma_lo(uint32_t bits, float x, float acc) {
  return fmaf(static_cast<float>(__builtin_bit_cast(h2_t, bits).x), x, acc);
}
__device__ __forceinline__ float fma_hi(uint32_t bits, float x, float acc) {
  return fmaf(static_cast<float>(__builtin_bit_cast(h2_t, bits).y), x, acc);
}

// Two codes held as fp16 subnormals in the halves of `bits`, times two fp16
// activations, both products added to acc in fp32 (v_dot2_f32_f16).  The
// products are exact (4 + 11 significant bits).
__device__ __forceinline__ float dot2_lo_hi(uint32_t bits, h2_t x, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, bits), x, acc, false);
}

// Byte B of v as fp32 via v_cvt_f32_ubyte{B}.  The empty asm hides how v was
// computed, which keeps the compiler from rewriting mask-then-convert into a
// bitfield extract per byte.
template <int B>
__device__ __forceinline__ float cvt_ubyte(uint32_t v) {
  __asm__("" : "+v"(v));
  return static_cast<float>((v >> (8 * B)) & 0xFFu);
}

// Where activations are read from.  Both sources hand out 16-byte chunks by
// element index (the index of the chunk's first element, a multiple of
// 16 / sizeof(XT)).
//  * XGlobal: the activation row in global memory.
//  * XShared: a copy of the row in LDS, written by xshared_slot().  Chunk g
//    of the row sits in slot g ^ ((g >> 4) & 15): the low four bits of the
//    slot (its group of four banks) are rotated by bits 4-7 of g, so lanes
//    whose chunks lie 256 bytes apart (the GEMV lane mappings) fall on
//    different banks.  Slots stay within the row's chunk count rounded up to
//    a multiple of 16.
template <typename XT>
struct XGlobal {
  typedef XT elem;
  const XT* p;
  __device__ uint4 chunk(int e) const { return *reinterpret_cast<const uint4*>(p + e); }
};

__device__ __forceinline__ int xshared_slot(int g) { return g ^ ((g >> 4) & 15); }

template <typename XT>
struct XShared {
  typedef XT elem;
  const uint4* lds;
  __device__ uint4 chunk(int e) const {
    return lds[xshared_slot(e / static_cast<int>(16 / sizeof(XT)))];
  }
};

// Raw activation loads: N elements starting at element e (16-byte aligned),
// as N * sizeof(XT) / 16 uint4 words; converted later by x_to_f32 so that the
// conversion does not force a wait before the weight loads are issued.
template <int N, class XS>
__device__ __forceinline__ void load_x_raw(const XS& x, int e, uint4* raw) {
  constexpr int kPer = 16 / static_cast<int>(sizeof(typename XS::elem));
#pragma unroll
  for (int i = 0; i < N / kPer; ++i) raw[i] = x.chunk(e + i * kPer);
}

// Workgroup barrier for LDS hand-offs: waits only for this wave's LDS
// operations (lgkmcnt(0); vmcnt and expcnt left at their maxima), then
// s_barrier.  __syncthreads() also fences global memory, which makes every
// wave wait for all of its outstanding loads, the weight prefetch included.
// The empty asm statements keep the compiler from moving memory accesses
// across.
__device__ __forceinline__ void lds_barrier() {
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  __asm__ __volatile__("" ::: "memory");
}

template <int N>
__device__ __forceinline__ void x_to_f32(const uint4* raw, float* out, const float*) {
#pragma unroll
  for (int i = 0; i < N / 4; ++i) {
    out[4 * i] = __uint_as_float(raw[i].x); out[4 * i + 1] = __uint_as_float(raw[i].y);
    out[4 * i + 2] = __uint_as_float(raw[i].z); out[4 * i + 3] = __uint_as_float(raw[i].w);
  }
}

template <int N>
__device__ __forceinline__ void x_to_f32(const uint4* raw, float* out, const _Float16*) {
#pragma unroll
  for (int i = 0; i < N / 8; ++i) {
    const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      out[8 * i + 2 * k] = f16_to_f32(w[k] & 0xFFFFu);
      out[8 * i + 2 * k + 1] = f16_to_f32(w[k] >> 16);
    }
  }
}

template <int N>
__device__ __forceinline__ void x_to_f32(const uint4* raw, float* out, const bf16_t*) {
#pragma unroll
  for (int i = 0; i < N / 8; ++i) {
    const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      out[8 * i + 2 * k] = __uint_as_float(w[k] << 16);
      out[8 * i + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
  }
}

// A lane's 64 fp16 or bf16 activations as the Q4_K and Q5_K GEMVs multiply
// them: fp16 activations as they are (e = 0); bf16 ones scaled by 2^-e, a
// power of two chosen per lane so that the largest |x| lands in
// [2^14, 2^15), and converted to fp16 -- exact, bf16's 8 significant bits
// fitting fp16's 11, for every element above 2^-31 of the lane's largest
// (smaller ones fall into fp16's subnormal range: absolute error at most
// 2^-40 of the largest),
// paired in the order the code halves come (dword i of the lane's codes:
// (byte 0, byte 2) and (byte 1, byte 3), low nibbles against activations
// 4i.., high nibbles against 32 + 4i..).  xs = 2^(24+e) undoes both the
// scaling and the 2^-24 of the subnormal codes; s0 and s1 are fp32 sums of
// the unrounded activations of the two sub-blocks, which the min terms take.
// e is kept where 2^(24+e) is a normal float (|x| below 2^117).
struct HalfXSlice {
  h2_t h[32];
  float s0, s1;
  float xs;
};

// Activation slice type of a policy by activation type: fp32 activations keep
// the exact fp32 slice F32 (one FMA per weight); fp16 and bf16 activations use
// Half (two products per instruction).  Rounding fp32 activations to fp16
// instead would cost up to 2^-11 of each product, which a row whose terms
// cancel turns into a relative error above 2e-3 (measured: one 128-wide INT4
// row at 2.3e-3).
template <typename XT, class F32, class Half>
struct XSliceFor {
  typedef Half type;
};
template <class F32, class Half>
struct XSliceFor<float, F32, Half> {
  typedef F32 type;
};

// fp32 activations enter v_fma_mix_f32 against codes held as u * 2^-24, so a
// product falls below float32's normal range (2^-126) once |x| is below about
// 2^-102 and then loses bits.  A lane whose largest |x| lies outside
// [2^-60, 2^60] therefore scales its slice by 2^-e, e the binary exponent of
// that largest |x| (clamped to [-100, 64], so xs times an fp16 scale stays
// finite), and undoes it with xs = 2^(24 + e); inside that range (the usual
// case) e = 0.  Either way every product of a nonzero code and an element
// within 2^-40 of the lane's largest stays normal.  Scaling by a power of two
// is exact and no product is subnormal, so 2x still gives 2y bit for bit.
//
// f32_slice_factor returns the factor every activation of the lane is
// multiplied by -- 2^-e, or 0 for a lane past the row's end, whose
// activations must not count -- and sets xs and un = 2^e, which turns sums of
// the scaled activations back into sums of the given ones (exactly).  The
// multiply replaces the select that zeroes such lanes, so the scaling costs
// only the maximum.
template <int N>
__device__ __forceinline__ float f32_slice_factor(const float* v, bool ok, float& xs, float& un) {
  float mx = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) mx = fmaxf(mx, fabsf(v[i]));
  const bool mid = mx <= 0x1p60f && (mx >= 0x1p-60f || mx == 0.f);
  int e = __builtin_amdgcn_frexp_expf(mx);
  e = mid ? 0 : (e < -100 ? -100 : (e > 64 ? 64 : e));
  xs = __builtin_amdgcn_ldexpf(1.0f, 24 + e);
  un = __builtin_amdgcn_ldexpf(1.0f, e);
  return ok ? __builtin_amdgcn_ldexpf(1.0f, -e) : 0.f;
}

__device__ __forceinline__ _Float16 scaled_f16(float v, int e) {
  return static_cast<_Float16>(__builtin_amdgcn_ldexpf(v, -e));
}

// The power of two e of a lane's n activations: 0 for fp16 activations (they
// are used as given, exactly), else the one that puts the largest |x| into
// [2^14, 2^15), kept where 2^(24+e) is a normal float (bf16 reaches 2^127:
// e <= 103 covers |x| below 2^117).
template <typename XT, int N>
__device__ __forceinline__ int half_scale_exp(const float* v) {
  if constexpr (__is_same(XT, _Float16)) {
    return 0;
  } else {
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < N; ++i) mx = fmaxf(mx, fabsf(v[i]));
    // mx = m 2^E with m in [0.5, 1): scaled by 2^-(E-15) it lies in [2^14, 2^15)
    const int e = __builtin_amdgcn_frexp_expf(mx) - 15;
    return e < -150 ? -150 : (e > 103 ? 103 : e);
  }
}

template <typename XT>
__device__ __forceinline__ void finish_half_xslice(const uint4* raw, bool ok, HalfXSlice& s) {
  float v[64];
  x_to_f32<64>(raw, v, static_cast<const XT*>(nullptr));
#pragma unroll
  for (int i = 0; i < 64; ++i) v[i] = ok ? v[i] : 0.f;
  s.s0 = 0.f;
  s.s1 = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) s.s0 += v[i];
#pragma unroll
  for (int i = 32; i < 64; ++i) s.s1 += v[i];
  const int e = half_scale_exp<XT, 64>(v);
  s.xs = __builtin_amdgcn_ldexpf(1.0f, 24 + e);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    s.h[4 * i + 0] = h2_t{scaled_f16(v[4 * i], e), scaled_f16(v[4 * i + 2], e)};
    s.h[4 * i + 1] = h2_t{scaled_f16(v[4 * i + 1], e), scaled_f16(v[4 * i + 3], e)};
    s.h[4 * i + 2] = h2_t{scaled_f16(v[32 + 4 * i], e), scaled_f16(v[32 + 4 * i + 2], e)};
    s.h[4 * i + 3] = h2_t{scaled_f16(v[32 + 4 * i + 1], e), scaled_f16(v[32 + 4 * i + 3], e)};
  }
}

// Host side: compute units and LDS bytes per workgroup of the current device,
// queried once per device (gfx950: 256 CUs, 160 KB).  The entries are atomics:
// host threads may race to fill one, and each stores the same value.
inline int device_attr_cached(hipDeviceAttribute_t attr, std::atomic<int> (&cache)[64], int fallback) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, attr, dev) != hipSuccess || v <= 0) v = fallback;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

inline int device_cus() {
  static std::atomic<int> cache[64];
  return device_attr_cached(hipDeviceAttributeMultiprocessorCount, cache, 256);
}

inline int device_lds_per_block() {
  static std::atomic<int> cache[64];
  return device_attr_cached(hipDeviceAttributeMaxSharedMemoryPerBlock, cache, 65536);
}

// Workgroups of kernel `fn` the current device holds at once, for a launch of
// `block` threads and `lds` bytes of dynamic LDS: compute units x the
// occupancy query.  One entry per (device, kernel, block, lds), filled on
// first use under a lock.
inline int64_t resident_workgroups_of(const void* fn, int block, size_t lds) {
  static std::mutex mu;
  static std::map<std::tuple<int, const void*, int, size_t>, int64_t> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  const auto key = std::make_tuple(dev, fn, block, lds);
  {
    std::lock_guard<std::mutex> g(mu);
    const auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, block, lds) != hipSuccess || per_cu <= 0)
    per_cu = 1;
  const int64_t v = static_cast<int64_t>(device_cus()) * per_cu;
  std::lock_guard<std::mutex> g(mu);
  cache[key] = v;
  return v;
}

template <typename K>
inline int64_t resident_workgroups(K kernel, int block, size_t lds) {
  return resident_workgroups_of(reinterpret_cast<const void*>(kernel), block, lds);
}

}  // namespace qmv
