// C ABI of libqmv: argument validation, status codes and kernel dispatch.
//
// Validation happens before any HIP call, so every error code except
// QMV_ERR_HIP can be produced and tested on a machine without a GPU.
// Unsupported combinations are refused, never routed to another path
// (hipEngine 0.3.0, "Quickstart": unsupported registry combinations fail
// rather than fall back; hipfire, "Implementation requirements for
// multi-weight Q8 WMMA dispatch": check dtypes and that K is a whole number
// of blocks so no kernel silently drops a tail).
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <initializer_list>

#include <hip/hip_runtime.h>

#include "api_internal.h"
#include "launch.h"
#include "planes.h"

namespace qmv {

static thread_local char g_last_error[512];

int32_t fail(int32_t status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int32_t ok() {
  g_last_error[0] = '\0';
  return QMV_OK;
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// How a launch gets the workspace of the register-dequantized kernels: none
// (those kernels are not used), the caller's buffer, or the library's fixed
// scratch; with `need` set, nothing is launched and the bytes the launch
// needs are stored there.
struct WsMode {
  void* ptr;
  uint64_t bytes;
  bool fixed;
  uint64_t* need;
};

// The workspace for a launch that needs `need` bytes of it (nullptr: the
// register-dequantized kernels are not used).  Fails before any launch when
// the caller's buffer or the fixed scratch is too small.
static int32_t take_workspace(const WsMode& ws, uint64_t need, void** out);

static int32_t from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(QMV_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), static_cast<int>(e));
}

// Largest cols a single GEMV launch supports: 16 waves along K.
static int64_t gemv_max_cols(int32_t fmt) {
  switch (fmt) {
    case QMV_Q8_0: return 16 * 64 * 32;
    case QMV_Q4_K: return 16 * 16 * 256;
    case QMV_Q6_K: return 16 * 16 * 256;
    case QMV_Q5_K: return 16 * 16 * 256;
    case QMV_INT4_G128: return 16 * 64 * 64;
    default: return 0;
  }
}

static int32_t check_weights(const qmv_weights* W) {
  if (!W) return fail(QMV_ERR_NULL, "weights descriptor is NULL");
  if (!W->data) return fail(QMV_ERR_NULL, "weights data pointer is NULL");
  if (qmv_block_size(W->fmt) == 0) return fail(QMV_ERR_FORMAT, "unknown format %d", W->fmt);
  if (W->layout != QMV_LAYOUT_BLOCKS && W->layout != QMV_LAYOUT_PLANES)
    return fail(QMV_ERR_FORMAT, "unknown layout %d", W->layout);
  const bool planes = W->layout == QMV_LAYOUT_PLANES;
  if (planes && W->fmt != QMV_Q4_K && W->fmt != QMV_Q5_K && W->fmt != QMV_Q6_K)
    return fail(QMV_ERR_UNSUPPORTED, "format %d has no plane layout", W->fmt);
  const uint64_t need = planes ? qmv_planes_size(W->fmt, W->rows, W->cols)
                               : qmv_packed_size(W->fmt, W->rows, W->cols);
  if (need == 0)
    return fail(QMV_ERR_SHAPE, "bad weight shape %lld x %lld for format %d", (long long)W->rows,
                (long long)W->cols, W->fmt);
  if (W->nbytes != need)
    return fail(QMV_ERR_SIZE, "weights hold %llu bytes, format needs %llu",
                (unsigned long long)W->nbytes, (unsigned long long)need);
  const uint64_t soff = W->fmt == QMV_INT4_G128 ? static_cast<uint64_t>(W->rows * W->cols / 2)
                        : planes                ? q4k_planes(W->rows, W->cols).a  // same unit for Q5_K, Q6_K
                                                : 0;
  if (W->scales_offset != soff)
    return fail(QMV_ERR_FORMAT, "scales_offset %llu, expected %llu",
                (unsigned long long)W->scales_offset, (unsigned long long)soff);
  if (!aligned16(W->data)) return fail(QMV_ERR_ALIGN, "weights data not 16-byte aligned");
  if (W->rows > INT32_MAX || W->cols > INT32_MAX || W->rows * W->cols > (int64_t{1} << 40))
    return fail(QMV_ERR_UNSUPPORTED, "weight tensor too large");
  return QMV_OK;
}

}  // namespace qmv

using qmv::fail;

namespace qmv {

// A paired launch of two matrices of one format, layout and shape (`a` with
// twice its rows; launch.h): both outputs, or with glu the SwiGLU input.
static hipError_t pair_launch(int32_t fmt, const GemvCall& a, const void* b_w, float* b_y, int32_t x_dtype,
                              int64_t batch, bool planes, bool glu, hipStream_t s) {
  switch (fmt) {
    case QMV_Q8_0: return gemv_q8_0_pair(a, b_w, b_y, x_dtype, batch, glu, s);
    case QMV_Q4_K: return gemv_q4_k_pair(a, b_w, b_y, x_dtype, batch, planes, glu, s);
    case QMV_Q5_K: return gemv_q5_k_pair(a, b_w, b_y, x_dtype, batch, planes, glu, s);
    case QMV_Q6_K: return gemv_q6_k_pair(a, b_w, b_y, x_dtype, batch, planes, glu, s);
    default: return gemv_int4_g128_pair(a, b_w, b_y, x_dtype, batch, glu, s);
  }
}

static int32_t take_workspace(const WsMode& ws, uint64_t need, void** out) {
  if (out) *out = nullptr;
  if (ws.need) {
    *ws.need = need;
    return ok();
  }
  if (need == 0) return ok();
  if (ws.fixed) {
    if (need > kScratchBytes)
      return fail(QMV_ERR_SIZE, "qmv_gemv_noalloc: this call needs %llu bytes of workspace, more than the %llu "
                                "of the library's fixed scratch (fewer activation rows fit)",
                  (unsigned long long)need, (unsigned long long)kScratchBytes);
    return from_hip(scratch_workspace(need, out), "qmv_gemv_noalloc: scratch lookup");
  }
  if (!ws.ptr) return ok();  // no workspace: the exact-product kernels
  if (ws.bytes < need)
    return fail(QMV_ERR_SIZE, "workspace holds %llu bytes, this launch needs %llu (qmv_workspace_size)",
                (unsigned long long)ws.bytes, (unsigned long long)need);
  *out = ws.ptr;
  return ok();
}

}  // namespace qmv

extern "C" {

int32_t qmv_block_size(int32_t fmt) {
  switch (fmt) {
    case QMV_Q8_0: return 32;
    case QMV_Q4_K: return 256;
    case QMV_Q6_K: return 256;
    case QMV_Q5_K: return 256;
    case QMV_INT4_G128: return 128;
    default: return 0;
  }
}

uint64_t qmv_packed_size(int32_t fmt, int64_t rows, int64_t cols) {
  const int32_t qk = qmv_block_size(fmt);
  if (qk == 0 || rows < 1 || cols < 1 || cols % qk != 0) return 0;
  if (rows > (int64_t{1} << 40) / cols) return 0;
  const uint64_t nblk = static_cast<uint64_t>(rows) * static_cast<uint64_t>(cols / qk);
  switch (fmt) {
    case QMV_Q8_0: return nblk * 34;
    case QMV_Q4_K: return nblk * 144;
    case QMV_Q6_K: return nblk * 210;
    case QMV_Q5_K: return nblk * 176;
    default: return static_cast<uint64_t>(rows) * cols / 2 + nblk * 2;
  }
}

uint64_t qmv_planes_size(int32_t fmt, int64_t rows, int64_t cols) {
  if ((fmt != QMV_Q4_K && fmt != QMV_Q5_K && fmt != QMV_Q6_K) || qmv_packed_size(fmt, rows, cols) == 0)
    return 0;
  return fmt == QMV_Q4_K   ? qmv::q4k_planes(rows, cols).total
         : fmt == QMV_Q5_K ? qmv::q5k_planes(rows, cols).total
                           : qmv::q6k_planes(rows, cols).total;
}

int32_t qmv_create_weights_planes(int32_t fmt, int64_t rows, int64_t cols, const void* dev_planes,
                                  uint64_t nbytes, qmv_weights* out) {
  if (!out) return fail(QMV_ERR_NULL, "output descriptor is NULL");
  if (!dev_planes) return fail(QMV_ERR_NULL, "planes data pointer is NULL");
  if (qmv_block_size(fmt) == 0) return fail(QMV_ERR_FORMAT, "unknown format %d", fmt);
  if (fmt != QMV_Q4_K && fmt != QMV_Q5_K && fmt != QMV_Q6_K)
    return fail(QMV_ERR_UNSUPPORTED, "format %d has no plane layout", fmt);
  const uint64_t need = qmv_planes_size(fmt, rows, cols);
  if (need == 0)
    return fail(QMV_ERR_SHAPE, "bad shape %lld x %lld (cols must be a positive multiple of 256)",
                (long long)rows, (long long)cols);
  if (nbytes != need)
    return fail(QMV_ERR_SIZE, "got %llu bytes, planes need %llu", (unsigned long long)nbytes,
                (unsigned long long)need);
  if (!qmv::aligned16(dev_planes)) return fail(QMV_ERR_ALIGN, "planes data not 16-byte aligned");
  qmv_weights w;
  w.fmt = fmt;
  w.layout = QMV_LAYOUT_PLANES;
  w.rows = rows;
  w.cols = cols;
  w.data = dev_planes;
  w.nbytes = nbytes;
  w.scales_offset = qmv::q4k_planes(rows, cols).a;  // the plane unit, the same for every format
  *out = w;
  return qmv::ok();
}

int32_t qmv_repack_planes(const qmv_weights* src, void* dst, uint64_t dst_bytes, qmv_weights* out,
                          void* stream) {
  if (!out) return fail(QMV_ERR_NULL, "output descriptor is NULL");
  if (!dst) return fail(QMV_ERR_NULL, "destination is NULL");
  int32_t st = qmv::check_weights(src);
  if (st != QMV_OK) return st;
  if (src->layout != QMV_LAYOUT_BLOCKS)
    return fail(QMV_ERR_UNSUPPORTED, "source is not in the canonical block layout");
  if (src->fmt != QMV_Q4_K && src->fmt != QMV_Q5_K && src->fmt != QMV_Q6_K)
    return fail(QMV_ERR_UNSUPPORTED, "format %d has no plane layout", src->fmt);
  const uint64_t need = qmv_planes_size(src->fmt, src->rows, src->cols);
  if (dst_bytes < need)
    return fail(QMV_ERR_SIZE, "destination holds %llu bytes, planes need %llu",
                (unsigned long long)dst_bytes, (unsigned long long)need);
  if (!qmv::aligned16(dst)) return fail(QMV_ERR_ALIGN, "destination not 16-byte aligned");
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(src->data), s1 = s0 + src->nbytes;
  const uintptr_t d0 = reinterpret_cast<uintptr_t>(dst), d1 = d0 + need;
  if (s0 < d1 && d0 < s1) return fail(QMV_ERR_SHAPE, "destination overlaps the source");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = src->fmt == QMV_Q4_K   ? qmv::repack_q4_k_planes(*src, dst, s)
                       : src->fmt == QMV_Q5_K ? qmv::repack_q5_k_planes(*src, dst, s)
                                              : qmv::repack_q6_k_planes(*src, dst, s);
  if (e != hipSuccess) return qmv::from_hip(e, "qmv_repack_planes launch");
  qmv_weights w = *src;
  w.layout = QMV_LAYOUT_PLANES;
  w.data = dst;
  w.nbytes = need;
  w.scales_offset = qmv::q4k_planes(src->rows, src->cols).a;
  *out = w;
  return qmv::ok();
}

int32_t qmv_create_weights(int32_t fmt, int64_t rows, int64_t cols, const void* dev_packed,
                           uint64_t nbytes, qmv_weights* out) {
  if (!out) return fail(QMV_ERR_NULL, "output descriptor is NULL");
  if (!dev_packed) return fail(QMV_ERR_NULL, "packed data pointer is NULL");
  if (qmv_block_size(fmt) == 0) return fail(QMV_ERR_FORMAT, "unknown format %d", fmt);
  const uint64_t need = qmv_packed_size(fmt, rows, cols);
  if (need == 0)
    return fail(QMV_ERR_SHAPE, "bad shape %lld x %lld (cols must be a positive multiple of %d)",
                (long long)rows, (long long)cols, qmv_block_size(fmt));
  if (nbytes != need)
    return fail(QMV_ERR_SIZE, "got %llu bytes, format needs %llu", (unsigned long long)nbytes,
                (unsigned long long)need);
  if ((reinterpret_cast<uintptr_t>(dev_packed) & 15u) != 0)
    return fail(QMV_ERR_ALIGN, "packed data not 16-byte aligned");
  qmv_weights w;
  w.fmt = fmt;
  w.layout = QMV_LAYOUT_BLOCKS;
  w.rows = rows;
  w.cols = cols;
  w.data = dev_packed;
  w.nbytes = nbytes;
  w.scales_offset = fmt == QMV_INT4_G128 ? static_cast<uint64_t>(rows * cols / 2) : 0;
  *out = w;
  return qmv::ok();
}

int32_t qmv_gemv(int32_t fmt, const qmv_weights* W, const void* x, int32_t x_dtype, float* y,
                 int64_t rows, int64_t cols, int64_t batch, void* stream) {
  if (!W) return fail(QMV_ERR_NULL, "weights descriptor is NULL");
  if (fmt != W->fmt || rows != W->rows || cols != W->cols)
    return fail(QMV_ERR_FORMAT, "call (fmt %d, %lld x %lld) disagrees with weights (fmt %d, %lld x %lld)",
                fmt, (long long)rows, (long long)cols, W->fmt, (long long)W->rows,
                (long long)W->cols);
  const qmv_gemv_item item{W, x, y};
  return qmv_gemv_multi(fmt, x_dtype, batch, &item, 1, stream);
}

static int32_t gemv_multi_impl(int32_t fmt, int32_t x_dtype, int64_t batch, const qmv_gemv_item* items,
                               int32_t n, void* stream, const qmv::WsMode& ws);

int32_t qmv_gemv_noalloc(int32_t fmt, const qmv_weights* W, const void* x, int32_t x_dtype, float* y,
                         int64_t rows, int64_t cols, int64_t batch, void* stream) {
  if (!W) return fail(QMV_ERR_NULL, "weights descriptor is NULL");
  if (fmt != W->fmt || rows != W->rows || cols != W->cols)
    return fail(QMV_ERR_FORMAT, "call (fmt %d, %lld x %lld) disagrees with weights (fmt %d, %lld x %lld)",
                fmt, (long long)rows, (long long)cols, W->fmt, (long long)W->rows,
                (long long)W->cols);
  const qmv_gemv_item item{W, x, y};
  return gemv_multi_impl(fmt, x_dtype, batch, &item, 1, stream, qmv::WsMode{nullptr, 0, true, nullptr});
}

int32_t qmv_gemv_multi(int32_t fmt, int32_t x_dtype, int64_t batch, const qmv_gemv_item* items,
                       int32_t n, void* stream) {
  return gemv_multi_impl(fmt, x_dtype, batch, items, n, stream, qmv::WsMode{nullptr, 0, false, nullptr});
}

int32_t qmv_gemv_multi_ws(int32_t fmt, int32_t x_dtype, int64_t batch, const qmv_gemv_item* items,
                          int32_t n, void* workspace, uint64_t workspace_bytes, void* stream) {
  if (workspace_bytes && !workspace) return fail(QMV_ERR_NULL, "workspace is NULL");
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return fail(QMV_ERR_ALIGN, "workspace not 256-byte aligned");
  return gemv_multi_impl(fmt, x_dtype, batch, items, n, stream,
                         qmv::WsMode{workspace, workspace_bytes, false, nullptr});
}

int32_t qmv_workspace_size(int32_t fmt, int32_t x_dtype, int64_t batch, const qmv_gemv_item* items,
                           int32_t n, uint64_t* bytes) {
  if (!bytes) return fail(QMV_ERR_NULL, "bytes is NULL");
  *bytes = 0;
  uint64_t need = 0;
  const int32_t st =
      gemv_multi_impl(fmt, x_dtype, batch, items, n, nullptr, qmv::WsMode{nullptr, 0, false, &need});
  if (st == QMV_OK) *bytes = need;
  return st;
}

static int32_t gemv_multi_impl(int32_t fmt, int32_t x_dtype, int64_t batch, const qmv_gemv_item* items,
                               int32_t n, void* stream, const qmv::WsMode& ws) {
  if (!items) return fail(QMV_ERR_NULL, "items is NULL");
  if (n < 1) return fail(QMV_ERR_SHAPE, "item count %d < 1", n);
  if (n > qmv::kMaxItems)
    return fail(QMV_ERR_UNSUPPORTED, "item count %d above %d", n, qmv::kMaxItems);
  if (qmv_block_size(fmt) == 0) return fail(QMV_ERR_FORMAT, "unknown format %d", fmt);
  if (batch < 1) return fail(QMV_ERR_SHAPE, "batch %lld < 1", (long long)batch);
  if (x_dtype != QMV_F32 && x_dtype != QMV_F16 && x_dtype != QMV_BF16)
    return fail(QMV_ERR_UNSUPPORTED, "activation dtype %d", x_dtype);
  if (batch > qmv::kMaxBatch)
    return fail(QMV_ERR_UNSUPPORTED, "batch %lld above %lld", (long long)batch,
                (long long)qmv::kMaxBatch);
  qmv::GemvCall calls[qmv::kMaxItems];
  for (int i = 0; i < n; ++i) {
    const qmv_gemv_item& it = items[i];
    int32_t st = qmv::check_weights(it.W);
    if (st != QMV_OK) return st;
    if (it.W->fmt != fmt)
      return fail(QMV_ERR_FORMAT, "item %d has format %d, launch format %d", i, it.W->fmt, fmt);
    if (it.W->layout != items[0].W->layout)
      return fail(QMV_ERR_UNSUPPORTED, "item %d has layout %d, item 0 layout %d", i, it.W->layout,
                  items[0].W->layout);
    if (!it.x || !it.y) return fail(QMV_ERR_NULL, "item %d: x or y is NULL", i);
    if (!qmv::aligned16(it.x) || !qmv::aligned16(it.y))
      return fail(QMV_ERR_ALIGN, "item %d: x or y not 16-byte aligned", i);
    if (it.W->cols > qmv::gemv_max_cols(fmt))
      return fail(QMV_ERR_UNSUPPORTED, "item %d: cols %lld above the GEMV limit %lld", i,
                  (long long)it.W->cols, (long long)qmv::gemv_max_cols(fmt));
    calls[i] = qmv::GemvCall{it.W, it.x, it.y};
  }
  // Outputs must not overlap: each item's y is written by its own workgroups.
  for (int i = 0; i < n; ++i)
    for (int j = i + 1; j < n; ++j) {
      const uintptr_t a0 = reinterpret_cast<uintptr_t>(items[i].y);
      const uintptr_t a1 = a0 + static_cast<uintptr_t>(batch * items[i].W->rows) * 4;
      const uintptr_t b0 = reinterpret_cast<uintptr_t>(items[j].y);
      const uintptr_t b1 = b0 + static_cast<uintptr_t>(batch * items[j].W->rows) * 4;
      if (a0 < b1 && b0 < a1) return fail(QMV_ERR_SHAPE, "outputs of items %d and %d overlap", i, j);
    }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  // Q4_K with bf16 activations and a batch of at least kMfmaMinBatch rows: the
  // matrix-core kernel, one launch per matrix (the GEMV path would read the
  // weights once per activation row).
  const bool planes = items[0].W->layout == QMV_LAYOUT_PLANES;
  // Two or more rows (Q4_K bf16: up to kRowsMaxBf16Batch): the matrices
  // within one wave's K slice take the multi-row GEMV (one launch, one pass
  // over the weights per two or four activation rows, two for fp32), those of
  // two to eight waves along K its K-split form (fp16/bf16; one launch, one
  // pass per two rows; Q4_K x bf16 above two rows keeps the matrix cores),
  // the wider ones the GEMV once per row; Q4_K x fp16 from five rows takes
  // the matrix cores with fp16 operands (gemm_q4_k_f16_fits).  Every item's
  // result is the same as that of the item called alone, except in runs of
  // register-dequantized matrices (gemm_q4_k_mfma_items), whose shared K
  // slicing can change the float32 summation order.
  const bool half_x = x_dtype == QMV_F16 || x_dtype == QMV_BF16;
  const int64_t wave_cols = fmt == QMV_Q8_0 ? 2048 : 4096;
  // Several small Q4_K matrices (the q, k, v of a layer) at 5..16 fp16/bf16
  // rows: one multi-row launch for all of them beats a matrix-core launch per
  // matrix (7B q+k+v at 8 bf16 rows: 9.7 against 19.5 us; a single matrix,
  // or large ones, stay on the matrix cores).  Each output row then equals
  // the batch-1 GEMV's bit for bit.
  if (fmt == QMV_Q4_K && half_x && batch >= 5 && batch <= qmv::kRowsSmallMultiMaxBatch && n >= 2) {
    bool small = true;
    int64_t rows_sum = 0;
    for (int i = 0; i < n; ++i) {
      small = small && items[i].W->cols <= wave_cols;
      rows_sum += items[i].W->rows;
    }
    if (small && rows_sum <= qmv::kRowsSmallMultiMaxRows) {
      if (ws.need) return qmv::take_workspace(ws, 0, nullptr);
      return qmv::from_hip(qmv::gemv_q4_k_rows(calls, n, x_dtype, batch, planes, s),
                           "qmv_gemv (multi-row, several matrices) launch");
    }
  }
  if (batch >= 2 &&
      !(fmt == QMV_Q4_K && x_dtype == QMV_BF16 && batch > qmv::kRowsMaxBf16Batch)) {
    qmv::GemvCall narrow[qmv::kMaxItems], split[qmv::kMaxItems], wide[qmv::kMaxItems];
    qmv::GemvCall mfma16[qmv::kMaxItems];
    int nn = 0, ns = 0, nw = 0, nm = 0;
    // Q4_K x fp16 from 5 rows: the matrix cores with fp16 operands
    const bool f16_mfma = fmt == QMV_Q4_K && x_dtype == QMV_F16 && batch >= qmv::kMfmaMinF16Batch;
    // Q4_K x bf16 against wide matrices: the K-split form for two rows, the
    // matrix cores above (3584 x 18944: 14.7 against 24.8 us at two rows,
    // 27.0 against 25.1 us at three)
    const bool q4k_mfma = fmt == QMV_Q4_K && x_dtype == QMV_BF16 && batch >= qmv::kMfmaMinBatch;
    const bool mfma_split = q4k_mfma && batch > 2;
    for (int i = 0; i < n; ++i) {
      if (f16_mfma && qmv::gemm_q4_k_f16_fits(calls[i].W->cols, batch))
        mfma16[nm++] = calls[i];
      else if (calls[i].W->cols <= wave_cols)
        narrow[nn++] = calls[i];
      else if (calls[i].W->cols <= qmv::kRowsSplitMaxWaves * wave_cols && half_x && !mfma_split)
        split[ns++] = calls[i];
      else
        wide[nw++] = calls[i];
    }
    auto rows = [&](const qmv::GemvCall* c, int k) -> hipError_t {
      switch (fmt) {
        case QMV_Q4_K: return qmv::gemv_q4_k_rows(c, k, x_dtype, batch, planes, s);
        case QMV_Q6_K: return qmv::gemv_q6_k_rows(c, k, x_dtype, batch, planes, s);
        case QMV_Q5_K: return qmv::gemv_q5_k_rows(c, k, x_dtype, batch, planes, s);
        case QMV_Q8_0: return qmv::gemv_q8_0_rows(c, k, x_dtype, batch, s);
        default: return qmv::gemv_int4_g128_rows(c, k, x_dtype, batch, s);
      }
    };
    // the register-dequantized kernels' workspace, checked before any launch
    const uint64_t need = std::max(nm ? qmv::gemm_q4_k_mfma_items_workspace(mfma16, nm, batch) : 0,
                                   q4k_mfma && nw ? qmv::gemm_q4_k_mfma_items_workspace(wide, nw, batch) : 0);
    void* wsp = nullptr;
    const int32_t wst = qmv::take_workspace(ws, need, &wsp);
    if (wst != QMV_OK || ws.need) return wst;
    if (nn) e = rows(narrow, nn);
    if (e == hipSuccess && ns) e = rows(split, ns);
    if (e == hipSuccess && nm) e = qmv::gemm_q4_k_mfma_items(mfma16, nm, true, batch, s, wsp);
    if (e == hipSuccess && nw) {
      if (q4k_mfma) {
        e = qmv::gemm_q4_k_mfma_items(wide, nw, false, batch, s, wsp);
      } else {
        switch (fmt) {
          case QMV_Q4_K:
            e = planes ? qmv::gemv_q4_k_planes(wide, nw, x_dtype, batch, s)
                       : qmv::gemv_q4_k(wide, nw, x_dtype, batch, s);
            break;
          case QMV_Q6_K:
            e = planes ? qmv::gemv_q6_k_planes(wide, nw, x_dtype, batch, s)
                       : qmv::gemv_q6_k(wide, nw, x_dtype, batch, s);
            break;
          case QMV_Q5_K:
            e = planes ? qmv::gemv_q5_k_planes(wide, nw, x_dtype, batch, s)
                       : qmv::gemv_q5_k(wide, nw, x_dtype, batch, s);
            break;
          case QMV_Q8_0: e = qmv::gemv_q8_0(wide, nw, x_dtype, batch, s); break;
          default: e = qmv::gemv_int4_g128(wide, nw, x_dtype, batch, s); break;
        }
      }
    }
    return qmv::from_hip(e, "qmv_gemv (multi-row) launch");
  }
  if (fmt == QMV_Q4_K && x_dtype == QMV_BF16 && batch >= qmv::kMfmaMinBatch) {
    void* wsp = nullptr;
    const int32_t st = qmv::take_workspace(ws, qmv::gemm_q4_k_mfma_items_workspace(calls, n, batch), &wsp);
    if (st != QMV_OK || ws.need) return st;
    return qmv::from_hip(qmv::gemm_q4_k_mfma_items(calls, n, false, batch, s, wsp),
                         "qmv_gemv (matrix-core) launch");
  }
  if (ws.need) return qmv::take_workspace(ws, 0, nullptr);
  // Two matrices of one shape on one activation within one wave's K slice
  // (gate and up): one launch whose two-row tiles pair row i of each
  // (7B gate+up, Q4_K planes, fp32 x: 15.3 against 15.5 us as two items;
  // INT4, fp16 x: 13.2 against 13.9 us).
  if (batch == 1 && n == 2 && items[0].x == items[1].x && items[0].W->rows == items[1].W->rows &&
      items[0].W->cols == items[1].W->cols && items[0].W->cols <= wave_cols &&
      items[0].W->rows <= INT32_MAX / 2) {
    qmv_weights pair = *items[0].W;
    pair.rows = 2 * items[0].W->rows;
    const qmv::GemvCall a{&pair, items[0].x, items[0].y};
    return qmv::from_hip(qmv::pair_launch(fmt, a, items[1].W->data, items[1].y, x_dtype, batch, planes, false, s),
                         "qmv_gemv (paired matrices) launch");
  }
  switch (fmt) {
    case QMV_Q8_0: e = qmv::gemv_q8_0(calls, n, x_dtype, batch, s); break;
    case QMV_Q4_K:
      e = planes ? qmv::gemv_q4_k_planes(calls, n, x_dtype, batch, s)
                 : qmv::gemv_q4_k(calls, n, x_dtype, batch, s);
      break;
    case QMV_Q5_K:
      e = planes ? qmv::gemv_q5_k_planes(calls, n, x_dtype, batch, s)
                 : qmv::gemv_q5_k(calls, n, x_dtype, batch, s);
      break;
    case QMV_Q6_K:
      e = planes ? qmv::gemv_q6_k_planes(calls, n, x_dtype, batch, s)
                 : qmv::gemv_q6_k(calls, n, x_dtype, batch, s);
      break;
    default: e = qmv::gemv_int4_g128(calls, n, x_dtype, batch, s); break;
  }
  return qmv::from_hip(e, "qmv_gemv launch");
}

int32_t qmv_gemv_swiglu(int32_t fmt, const qmv_weights* Wg, const qmv_weights* Wu, const void* x,
                        int32_t x_dtype, float* h, int64_t rows, int64_t cols, int64_t batch, void* stream) {
  for (const qmv_weights* W : {Wg, Wu}) {
    const int32_t st = qmv::check_weights(W);
    if (st != QMV_OK) return st;
    if (fmt != W->fmt || rows != W->rows || cols != W->cols)
      return fail(QMV_ERR_FORMAT, "call (fmt %d, %lld x %lld) disagrees with weights (fmt %d, %lld x %lld)",
                  fmt, (long long)rows, (long long)cols, W->fmt, (long long)W->rows, (long long)W->cols);
  }
  if (Wg->layout != Wu->layout)
    return fail(QMV_ERR_UNSUPPORTED, "gate layout %d, up layout %d", Wg->layout, Wu->layout);
  if (!x || !h) return fail(QMV_ERR_NULL, "x or h is NULL");
  if (!qmv::aligned16(x) || !qmv::aligned16(h)) return fail(QMV_ERR_ALIGN, "x or h not 16-byte aligned");
  if (batch < 1) return fail(QMV_ERR_SHAPE, "batch %lld < 1", (long long)batch);
  if (batch > qmv::kMaxBatch)
    return fail(QMV_ERR_UNSUPPORTED, "batch %lld above %lld", (long long)batch, (long long)qmv::kMaxBatch);
  if (x_dtype != QMV_F32 && x_dtype != QMV_F16 && x_dtype != QMV_BF16)
    return fail(QMV_ERR_UNSUPPORTED, "activation dtype %d", x_dtype);
  const int64_t slice = fmt == QMV_Q8_0 ? 2048 : 4096;  // one wave's K slice
  if (cols > slice)
    return fail(QMV_ERR_UNSUPPORTED, "cols %lld above %lld: the fused gate/up launch needs every row within "
                "one wave's K slice (call qmv_gemv_multi for gate and up instead)", (long long)cols,
                (long long)slice);
  if (rows > INT32_MAX / 2) return fail(QMV_ERR_UNSUPPORTED, "rows %lld too large", (long long)rows);
  const uintptr_t x0 = reinterpret_cast<uintptr_t>(x);
  const uintptr_t x1 = x0 + static_cast<uintptr_t>(batch * cols) * (x_dtype == QMV_F32 ? 4 : 2);
  const uintptr_t h0 = reinterpret_cast<uintptr_t>(h);
  const uintptr_t h1 = h0 + static_cast<uintptr_t>(batch * rows) * 4;
  if (x0 < h1 && h0 < x1) return fail(QMV_ERR_SHAPE, "h overlaps x");
  qmv_weights pair = *Wg;  // launch rows 2i, 2i + 1 = gate row i, up row i
  pair.rows = 2 * rows;
  const qmv::GemvCall gate{&pair, x, h};
  return qmv::from_hip(qmv::pair_launch(fmt, gate, Wu->data, nullptr, x_dtype, batch,
                                       Wg->layout == QMV_LAYOUT_PLANES, true, static_cast<hipStream_t>(stream)),
                       "qmv_gemv_swiglu launch");
}

int32_t qmv_dequant(const qmv_weights* W, void* out, int32_t out_dtype, void* stream) {
  int32_t st = qmv::check_weights(W);
  if (st != QMV_OK) return st;
  if (!out) return fail(QMV_ERR_NULL, "output is NULL");
  if (out_dtype != QMV_F32 && out_dtype != QMV_F16 && out_dtype != QMV_BF16)
    return fail(QMV_ERR_UNSUPPORTED, "output dtype %d", out_dtype);
  if (!qmv::aligned16(out)) return fail(QMV_ERR_ALIGN, "output not 16-byte aligned");
  return qmv::from_hip(qmv::dequant(*W, out, out_dtype, static_cast<hipStream_t>(stream)),
                       "qmv_dequant launch");
}

int64_t qmv_probe_read_outputs(uint64_t nbytes) { return qmv::probe_read_blocks(nbytes); }

int32_t qmv_probe_read(const void* src, uint64_t nbytes, float* out, void* stream) {
  if (!src || !out) return fail(QMV_ERR_NULL, "probe: NULL pointer");
  if (nbytes % 16 != 0) return fail(QMV_ERR_SIZE, "probe: nbytes not a multiple of 16");
  if (!qmv::aligned16(src) || !qmv::aligned16(out)) return fail(QMV_ERR_ALIGN, "probe: misaligned");
  return qmv::from_hip(qmv::probe_read(src, nbytes, out, static_cast<hipStream_t>(stream)),
                       "qmv_probe_read launch");
}

int32_t qmv_probe_copy(const void* src, void* dst, uint64_t nbytes, void* stream) {
  if (!src || !dst) return fail(QMV_ERR_NULL, "probe: NULL pointer");
  if (nbytes % 16 != 0) return fail(QMV_ERR_SIZE, "probe: nbytes not a multiple of 16");
  if (!qmv::aligned16(src) || !qmv::aligned16(dst)) return fail(QMV_ERR_ALIGN, "probe: misaligned");
  return qmv::from_hip(qmv::probe_copy(src, dst, nbytes, static_cast<hipStream_t>(stream)),
                       "qmv_probe_copy launch");
}

const char* qmv_status_string(int32_t status) {
  switch (status) {
    case QMV_OK: return "ok";
    case QMV_ERR_NULL: return "null pointer";
    case QMV_ERR_FORMAT: return "format or descriptor mismatch";
    case QMV_ERR_SHAPE: return "bad shape";
    case QMV_ERR_ALIGN: return "pointer not 16-byte aligned";
    case QMV_ERR_SIZE: return "byte count mismatch";
    case QMV_ERR_UNSUPPORTED: return "unsupported combination";
    case QMV_ERR_RANGE: return "value out of range";
    case QMV_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* qmv_last_error(void) { return qmv::g_last_error; }

}  // extern "C"
