// Internal interface between the C ABI (api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmv.h"

namespace qmv {

// One matrix of a GEMV launch after validation: W [rows][cols] packed,
// x [batch][cols] of the launch's activation type, y [batch][rows] fp32.
struct GemvCall {
  const qmv_weights* W;
  const void* x;
  float* y;
};

// Most matrices one launch accepts.
constexpr int kMaxItems = 16;

// Largest batch a single GEMV call accepts (grid y dimension).
constexpr int64_t kMaxBatch = 65535;

hipError_t gemv_q8_0(const GemvCall* calls, int n, int x_dtype, int64_t batch, hipStream_t s);
hipError_t gemv_q4_k(const GemvCall* calls, int n, int x_dtype, int64_t batch, hipStream_t s);
// Q4_K / Q5_K / Q6_K weights in the plane layout (planes.h); every item in that layout.
hipError_t gemv_q4_k_planes(const GemvCall* calls, int n, int x_dtype, int64_t batch,
                            hipStream_t s);
// Every format with two or more activation rows: matrices within one wave's K
// slice (4096 columns; Q8_0 2048) take one pass over the weights per two or
// four rows (gemv_rows_kernel; fp32: two), and, for fp16/bf16 rows, matrices
// of 2..kRowsSplitMaxWaves waves along K one pass per two rows
// (gemv_rows_split_kernel; every item of one call of the same kind).  Q4_K bf16 batches above kRowsMaxBf16Batch, and
// Q4_K bf16 batches above two against matrices split along K, go to the
// matrix cores.
#ifndef QMV_ROWS_MAX_BF16_BATCH
#define QMV_ROWS_MAX_BF16_BATCH 4
#endif
constexpr int64_t kRowsMaxBf16Batch = QMV_ROWS_MAX_BF16_BATCH;
// Matrices of two to kRowsSplitMaxWaves waves along K take the K-split form
// of the multi-row GEMV (two activation rows per pass); wider ones run the
// GEMV once per activation row.
#ifndef QMV_ROWS_SPLIT_MAX_WAVES
#define QMV_ROWS_SPLIT_MAX_WAVES 8
#endif
constexpr int64_t kRowsSplitMaxWaves = QMV_ROWS_SPLIT_MAX_WAVES;
// Q4_K calls of two or more matrices within one wave's K slice, at most
// kRowsSmallMultiMaxRows rows in all, at 5..kRowsSmallMultiMaxBatch fp16/bf16
// rows: one multi-row launch instead of a matrix-core launch per matrix.
constexpr int64_t kRowsSmallMultiMaxBatch = 16;
constexpr int64_t kRowsSmallMultiMaxRows = 8192;
hipError_t gemv_q4_k_rows(const GemvCall* calls, int n, int x_dtype, int64_t batch, bool planes,
                          hipStream_t s);
hipError_t gemv_q6_k_rows(const GemvCall* calls, int n, int x_dtype, int64_t batch, bool planes,
                          hipStream_t s);
hipError_t gemv_int4_g128_rows(const GemvCall* calls, int n, int x_dtype, int64_t batch,
                               hipStream_t s);
hipError_t gemv_q5_k_rows(const GemvCall* calls, int n, int x_dtype, int64_t batch, bool planes,
                          hipStream_t s);
hipError_t gemv_q8_0_rows(const GemvCall* calls, int n, int x_dtype, int64_t batch, hipStream_t s);
hipError_t gemv_q5_k(const GemvCall* calls, int n, int x_dtype, int64_t batch, hipStream_t s);
hipError_t gemv_q5_k_planes(const GemvCall* calls, int n, int x_dtype, int64_t batch,
                            hipStream_t s);
hipError_t gemv_q6_k(const GemvCall* calls, int n, int x_dtype, int64_t batch, hipStream_t s);
hipError_t gemv_q6_k_planes(const GemvCall* calls, int n, int x_dtype, int64_t batch,
                            hipStream_t s);
hipError_t gemv_int4_g128(const GemvCall* calls, int n, int x_dtype, int64_t batch,
                          hipStream_t s);

// Batched Q4_K x bf16 on MFMA (gemm_q4_k_mfma.hip); the GEMV entry points use
// it for batches of at least kMfmaMinBatch rows.
#ifndef QMV_MFMA_MIN_BATCH
#define QMV_MFMA_MIN_BATCH 2
#endif
constexpr int64_t kMfmaMinBatch = QMV_MFMA_MIN_BATCH;
hipError_t gemm_q4_k_bf16(const qmv_weights& W, const void* x, float* y, int64_t batch,
                          hipStream_t s);
// Batches of at least kDqMinBatch rows (bf16 or fp16 activations) against
// matrices of at least kDqMinRows rows: the dequantized-tile kernels
// (gemm_q4_k_dq.hip, which hands shapes whose grid would not fill one round
// well to gemm_q4_k_dqreg.hip), entered from the launchers of
// gemm_q4_k_mfma.hip.  They round each weight to fp16 (relative error near
// 2^-11), which the normwise bound absorbs over a matrix of a few hundred
// rows (about 4e-4 on the 7B FFN shapes) but not over a handful of rows,
// where one output's cancellation sets the error; smaller matrices keep the
// exact-product kernels.  Measured against the 64-row tile kernel on the 7B
// FFN shapes (bf16): 18944 x 3584 at 128 rows 65 against 47 us, at 192-256
// rows 86-87 against 90 us, at 512 rows 111 against 171 us; 3584 x 18944 at
// 128 rows 209 against 169 us, at 192 rows 207 against 333 us.
#ifndef QMV_DQ_MIN_BATCH
#define QMV_DQ_MIN_BATCH 192
#endif
constexpr int64_t kDqMinBatch = QMV_DQ_MIN_BATCH;
constexpr int64_t kDqMinRows = 256;
// Tile of gemm_q4_k_dq: weight rows x activation rows per workgroup.
constexpr int64_t kDqTileRows = 256, kDqTileBatch = 128;
hipError_t gemm_q4_k_dq(const qmv_weights& W, const void* x, bool f16x, float* y, int64_t batch,
                        hipStream_t s);
// The register-dequantized kernel (gemm_q4_k_dqreg.hip): tile shape chosen
// by dqreg_form; byte offsets must fit in 32 bits.
bool gemm_q4_k_dqreg_fits(const qmv_weights& W, int64_t batch);
int dqreg_form(int64_t rows, int64_t batch);
hipError_t gemm_q4_k_dqreg(const qmv_weights& W, const void* x, bool f16x, float* y, int64_t batch,
                           hipStream_t s);
// Q4_K x fp16 on the matrix cores with fp16 operands: the kernels of the
// bf16 path (streaming or K-split up to 16 rows, tiles from 17).  qmv_gemv
// takes it from kMfmaMinF16Batch rows; below, the multi-row GEMV is faster.
#ifndef QMV_MFMA_MIN_F16_BATCH
#define QMV_MFMA_MIN_F16_BATCH 5
#endif
constexpr int64_t kMfmaMinF16Batch = QMV_MFMA_MIN_F16_BATCH;
bool gemm_q4_k_f16_fits(int64_t cols, int64_t batch);
hipError_t gemm_q4_k_f16(const qmv_weights& W, const void* x, float* y, int64_t batch,
                         hipStream_t s);

hipError_t dequant(const qmv_weights& W, void* out, int out_dtype, hipStream_t s);

// Canonical Q4_K / Q5_K / Q6_K blocks -> plane layout (planes.h) at dst.
hipError_t repack_q4_k_planes(const qmv_weights& src, void* dst, hipStream_t s);
hipError_t repack_q5_k_planes(const qmv_weights& src, void* dst, hipStream_t s);
hipError_t repack_q6_k_planes(const qmv_weights& src, void* dst, hipStream_t s);

int64_t probe_read_blocks(uint64_t nbytes);
hipError_t probe_read(const void* src, uint64_t nbytes, float* out, hipStream_t s);
hipError_t probe_copy(const void* src, void* dst, uint64_t nbytes, hipStream_t s);

}  // namespace qmv
