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

// Two matrices of one format, layout and shape on one activation as one
// launch whose two-row tiles pair row i of each (gemv_pair_kernel): `a`
// describes the first matrix with twice its rows, a.y its output; b_w is
// the second matrix's data and b_y its output.  glu: the gate and up
// projections of a SwiGLU FFN, whose epilogue writes h = silu(gate . x) *
// (up . x) to a.y in place of both (gemv_glu_kernel; b_y unused).  Matrices
// within one wave's K slice only (4096 columns; Q8_0 2048).
hipError_t gemv_q8_0_pair(const GemvCall& a, const void* b_w, float* b_y, int x_dtype, int64_t batch, bool glu,
                          hipStream_t s);
hipError_t gemv_q4_k_pair(const GemvCall& a, const void* b_w, float* b_y, int x_dtype, int64_t batch,
                          bool planes, bool glu, hipStream_t s);
hipError_t gemv_q5_k_pair(const GemvCall& a, const void* b_w, float* b_y, int x_dtype, int64_t batch,
                          bool planes, bool glu, hipStream_t s);
hipError_t gemv_q6_k_pair(const GemvCall& a, const void* b_w, float* b_y, int x_dtype, int64_t batch,
                          bool planes, bool glu, hipStream_t s);
hipError_t gemv_int4_g128_pair(const GemvCall& a, const void* b_w, float* b_y, int x_dtype, int64_t batch,
                               bool glu, hipStream_t s);

// Batched Q4_K x bf16 on MFMA (gemm_q4_k_mfma.hip); the GEMV entry points use
// it for batches of at least kMfmaMinBatch rows.
#ifndef QMV_MFMA_MIN_BATCH
#define QMV_MFMA_MIN_BATCH 2
#endif
constexpr int64_t kMfmaMinBatch = QMV_MFMA_MIN_BATCH;
hipError_t gemm_q4_k_bf16(const qmv_weights& W, const void* x, float* y, int64_t batch,
                          hipStream_t s);
// Q4_K x bf16/fp16 batches on the register-dequantized kernels
// (gemm_q4_k_dqreg.hip), for matrices of at least kDqMinRows rows whose byte
// offsets fit in 32 bits (dqreg_eligible): from kDqMinBatchRun rows for runs
// of two or more consecutive matrices of a launch on the same activations
// (q+k+v, gate+up: one launch for the run) and for matrices of at least
// kDqLongK columns, from kDqMinBatch rows for any matrix.  They round each
// weight to fp16 (relative error near 2^-11), which the normwise bound
// absorbs over a matrix of a few hundred rows (about 4e-4 on the 7B FFN
// shapes) but not over a handful of rows, where one output's cancellation
// sets the error; smaller matrices keep the exact-product kernels.
// Measured against the tile kernels on the 7B decoder layer (bf16, graph
// replays, whole layer): 17 rows 151.1 against 101.5 us, 24 rows 152.3
// against 103.7, 32 rows 149.5 against 108.1, 48 rows 197.6 against 114.2,
// 64 rows 153.6 against 120.1, 96 rows 282.1 against 152.7;
// a lone 3584 x 3584 matrix at 32 rows 12.9 (tile) against 15.5 us, the
// 18944 x 3584 gate alone at 64 rows 26 (tile) against 39 us; above 64 rows
// the tile kernels take 128-row tiles (the layer's o at 96 rows 35.7 us
// against 24.5 at 128 rows on the register kernels).
constexpr int64_t kDqMinBatch = 65, kDqMinBatchRun = 17, kDqLongK = 8192, kDqMinRows = 256;
// The activations converted once into a workspace, T 16-row tiles per wave
// against NB 16-row activation tiles per workgroup, K in `splits` slices of
// `bps` blocks (partial outputs summed in slice order).
struct DqregPlan {
  int t, nb, splits, bps;
};
constexpr int kDqregMaxSplits = 8;
// Matrices one launch of the register-dequantized kernels covers.
constexpr int kDqregMaxMats = 4;
bool dqreg_eligible(const qmv_weights& W, int64_t batch);
// The plan for n (1..kDqregMaxMats) matrices of rows[i] x cols in one launch.
DqregPlan dqreg_plan(const int64_t* rows, int n, int64_t cols, int64_t batch);
size_t dqreg_workspace_bytes(const int64_t* rows, int n, int64_t cols, int64_t batch, const DqregPlan& p);
// The n calls (same x, cols and layout) in one launch, with the caller's
// workspace ws (dqreg_workspace_bytes, 256-byte aligned); convert = false
// reuses the converted activations a previous call on the same stream left
// in ws (same x, batch and cols).
hipError_t gemm_q4_k_dqreg_ws(const GemvCall* calls, int n, bool f16x, int64_t batch, const DqregPlan& p, void* ws,
                              bool convert, hipStream_t s);
// The matrix-core calls of one launch (Q4_K, bf16 or fp16 rows, batch >= 2)
// in order: with a device workspace ws (gemm_q4_k_mfma_items_workspace
// bytes, 256-byte aligned), each on the register-dequantized kernels where
// the rules above say so (runs of consecutive such calls on the same
// activations, widths and layout, up to kDqregMaxMats, share one
// conversion, one product launch and one sum), else on the kernels of
// gemm_q4_k_bf16 / gemm_q4_k_f16; without one (ws = nullptr), every call on
// the latter.
hipError_t gemm_q4_k_mfma_items(const GemvCall* calls, int n, bool f16x, int64_t batch, hipStream_t s, void* ws);
// Workspace bytes gemm_q4_k_mfma_items needs for these calls (0: none).
size_t gemm_q4_k_mfma_items_workspace(const GemvCall* calls, int n, int64_t batch);
// The fixed device array of qmv_gemv_noalloc, QMV_NOALLOC_SCRATCH_BYTES,
// on the current device (its address looked up once per device).
constexpr size_t kScratchBytes = QMV_NOALLOC_SCRATCH_BYTES;
hipError_t scratch_workspace(size_t bytes, void** out);

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
