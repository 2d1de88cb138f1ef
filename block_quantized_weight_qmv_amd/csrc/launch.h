// Internal interface between the C ABI (api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmv.h"

namespace qmv {

// Arguments of one GEMV call after validation: x is [batch][cols] of x_dtype,
// y is [batch][rows] fp32.
struct GemvArgs {
  const qmv_weights* W;
  const void* x;
  int x_dtype;
  float* y;
  int64_t batch;
  hipStream_t stream;
};

// Largest batch a single GEMV call accepts (grid y dimension).
constexpr int64_t kMaxBatch = 65535;

hipError_t gemv_q8_0(const GemvArgs& a);
hipError_t gemv_q4_k(const GemvArgs& a);
hipError_t gemv_q6_k(const GemvArgs& a);
hipError_t gemv_int4_g128(const GemvArgs& a);

hipError_t dequant(const qmv_weights& W, void* out, int out_dtype, hipStream_t s);

int64_t probe_read_blocks(uint64_t nbytes);
hipError_t probe_read(const void* src, uint64_t nbytes, float* out, hipStream_t s);
hipError_t probe_copy(const void* src, void* dst, uint64_t nbytes, hipStream_t s);

// Work split of a GEMV launch: `nsets` row sets, each handled by `kw` waves
// that split K; `sets_per_wg` sets per workgroup (1 whenever kw > 1, so the
// cross-wave reduction barrier is only ever shared by waves of one set).
struct Split {
  int kw;
  int sets_per_wg;
  int nsets;
  int threads;
  int grid;
};

// Choose a split for `rows` rows and `kw` waves along K, aiming at about
// `target_waves` resident waves in total.
inline Split make_split(int64_t rows, int kw, int target_waves) {
  Split s;
  s.kw = kw;
  s.sets_per_wg = kw == 1 ? 4 : 1;
  int64_t target_sets = target_waves / kw;
  if (target_sets < 1) target_sets = 1;
  const int64_t rows_per_set = (rows + target_sets - 1) / target_sets;
  s.nsets = static_cast<int>((rows + rows_per_set - 1) / rows_per_set);
  s.threads = 64 * kw * s.sets_per_wg;
  s.grid = (s.nsets + s.sets_per_wg - 1) / s.sets_per_wg;
  return s;
}

}  // namespace qmv
