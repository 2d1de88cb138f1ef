/*
 * qmv.h -- block-quantized weight dequantize-and-multiply on AMD gfx950.
 *
 * C ABI of libqmv.so.  Plain C types only: integers, sizes and pointers.
 * Device pointers come from the caller (for example torch tensors'
 * data_ptr()); the library allocates no memory, creates no stream and never
 * synchronizes (its one device array, the fixed scratch of qmv_gemv_noalloc,
 * is part of the loaded code object).  Workspace, where a kernel needs one,
 * comes from the caller too (qmv_workspace_size, qmv_gemv_multi_ws).
 * `stream` arguments are hipStream_t values passed as void* (NULL = the
 * legacy default stream).
 *
 * Operation (what every entry point computes):
 *   W is a rows x cols matrix stored as blocks of quantized codes plus
 *   per-block scales, row-major, each row being cols / QK consecutive blocks.
 *     - VTE (kyuubyn.github.io/VTE), feature list: Q4_K, Q6_K and Q8_0 blocks
 *       are decoded byte for byte in llama.cpp's reference block layout.
 *     - "Costruire un runtime di inference LLM da zero" (datastack.it),
 *       "Tre bug che insegnano": the seven projections of each layer use
 *       symmetric INT4 weights with one scale per group of 128, multiplied
 *       against FP16 activations by a dedicated GEMV (an unpack of the 4-bit
 *       codes feeding FP16 activations beat an INT8-activation dot product).
 *   Byte maps (all fp16 little-endian IEEE binary16):
 *     Q8_0 (QK 32, 34 B):  d fp16 | q[32] int8.             w_i = d*q_i
 *     Q4_K (QK 256, 144 B): d fp16 | dmin fp16 | scales[12] (eight 6-bit
 *         scales sc_j and mins m_j) | qs[128].  Weight t = 64c+32h+l uses
 *         nibble h of qs[32c+l] and sub-block s = t/32:
 *         w_t = d*sc_s*u - dmin*m_s.
 *         j<4:  sc_j = scales[j]&63, m_j = scales[j+4]&63
 *         j>=4: sc_j = (scales[j+4]&15) | (scales[j-4]>>6)<<4,
 *               m_j  = (scales[j+4]>>4) | (scales[j]>>6)<<4
 *     Q5_K (QK 256, 176 B): d fp16 | dmin fp16 | scales[12] as Q4_K |
 *         qh[32] | qs[128] as Q4_K.  hipEngine 0.3.0, "GGUF Support", counts
 *         the type in a Q4_K_M file's payload; the bytes are GGUF's published
 *         Q5_K block.  Weight t = 64c+32h+l: u = (nibble h of qs[32c+l]) |
 *         (bit 2c+h of qh[l]) << 4 in 0..31, w_t = d*sc_s*u - dmin*m_s.
 *     Q6_K (QK 256, 210 B): ql[128] | qh[64] | sc[16] int8 | d fp16.
 *         Weight t = 128h+32g+l: low4 = nibble (g>>1) of ql[64h+32(g&1)+l],
 *         high2 = bits 2g..2g+1 of qh[32h+l], q6 = low4 | high2<<4,
 *         w_t = d*sc[t/16]*(q6-32).
 *     INT4_G128 (QK 128): codes plane rows*cols/2 bytes, byte j of a row
 *         holding u_{2j} (bits 0-3) and u_{2j+1} (bits 4-7), u = q+8; then a
 *         scales plane of rows*(cols/128) fp16 at scales_offset = rows*cols/2.
 *         w_k = s_{k/128}*(u_k-8).
 *   GEMV: y[b][r] = sum_k W[r][k] * x[b][k], x [batch][cols] row-major,
 *   y [batch][rows] fp32 row-major, overwritten.  Products and sums are
 *   carried in fp32; activations are converted exactly to fp32 (f16 and
 *   bf16 are subsets of fp32).  Any finite activations are accepted: the
 *   kernels scale each lane's activations by a power of two where their
 *   magnitudes would push products out of fp32's normal range, so results
 *   meet the same bound from |x| near 1e-38 to 1e38 (elements more than
 *   2^40 below the largest of their 64-element slice contribute with a
 *   relative error of at most 2^-24 of that largest).
 *
 * Errors: every entry point returns a qmv_status.  Argument validation runs
 * before any HIP call, so it needs no GPU.  After a launch, a failed
 * hipGetLastError maps to QMV_ERR_HIP; qmv_last_error() then holds the HIP
 * error text (thread-local).  Faults inside a kernel surface at the caller's
 * next synchronization, as for any HIP kernel.  The library never prints and
 * never aborts.
 */
#ifndef QMV_H
#define QMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  QMV_Q8_0 = 1,
  QMV_Q4_K = 2,
  QMV_Q6_K = 3,
  QMV_INT4_G128 = 4,
  QMV_Q5_K = 5
};

enum { QMV_F32 = 0, QMV_F16 = 1, QMV_BF16 = 2 };

/* Byte layouts of a weight tensor in device memory.
 *   QMV_LAYOUT_BLOCKS: the canonical blocks above, row-major.
 *   QMV_LAYOUT_PLANES (Q4_K, Q5_K, Q6_K): the same bytes rearranged for streaming,
 *     a decode-repacked layout in the sense of hipEngine 0.3.0, "GGUF
 *     Support" (GGUF blocks repacked at load time into decode layouts that
 *     replace the source).  With N = rows*(cols/256) blocks, block
 *     b = r*(cols/256) + j, and a = 16*N rounded up to a multiple of 256:
 *       header plane at 0:   bytes 0..15 of block b (d, dmin, scales) at 16*b;
 *       code plane A at a:   qs[32c .. 32c+16) of block b at a + 64*b + 16*c;
 *       code plane B at 5*a: qs[32c+16 .. 32c+32) of block b at
 *                            5*a + 64*b + 16*c   (c = 0..3);
 *     Q5_K, same N, b and a: bytes 0..15 of block b at 16*b; qh[0 .. 16)
 *       at a + 16*b; qh[16 .. 32) at 2*a + 16*b; qs[32c .. 32c+16) at
 *       3*a + 64*b + 16*c; qs[32c+16 .. 32c+32) at 7*a + 64*b + 16*c.
 *     Q6_K, same N, b and a, with p = 2h + i (h, i in {0, 1}):
 *       ql[64h + 16i .. +16) of block b at 64*b + 16*p;
 *       ql[64h + 32 + 16i .. +16) at 4*a + 64*b + 16*p;
 *       qh[32h + 16i .. +16) at 8*a + 64*b + 16*p;
 *       sc[0 .. 16) at 12*a + 16*b;   d at 13*a + 2*b.
 *     qmv_planes_size bytes in all; the descriptor's scales_offset holds a.
 *     Made on the device by qmv_repack_planes.  The GEMV streams each code
 *     plane with load instructions that read whole 128-byte lines no other
 *     instruction reads (which lets it use nontemporal loads), so the plane
 *     base should be 256-byte aligned for full speed (16 is required). */
enum { QMV_LAYOUT_BLOCKS = 0, QMV_LAYOUT_PLANES = 1 };

enum {
  QMV_OK = 0,
  QMV_ERR_NULL = -1,        /* a required pointer is NULL                    */
  QMV_ERR_FORMAT = -2,      /* unknown format, or fmt/rows/cols disagree     */
                            /* with the weights descriptor                   */
  QMV_ERR_SHAPE = -3,       /* rows/cols/batch < 1, or cols % QK != 0        */
  QMV_ERR_ALIGN = -4,       /* a device pointer is not 16-byte aligned       */
  QMV_ERR_SIZE = -5,        /* a byte count differs from qmv_packed_size or  */
                            /* an output buffer is too small                 */
  QMV_ERR_UNSUPPORTED = -6, /* dtype combination not provided                */
  QMV_ERR_RANGE = -7,       /* packer: a code or scale outside its range     */
  QMV_ERR_HIP = -8          /* the HIP runtime reported an error             */
};

/* Descriptor of packed weights resident in device memory.  Plain data,
 * caller-owned; it only points at the packed bytes, which must stay alive
 * (and unmodified) until every enqueued call that reads them has finished. */
typedef struct qmv_weights {
  int32_t fmt;            /* QMV_Q8_0 .. QMV_Q5_K                            */
  int32_t layout;         /* QMV_LAYOUT_BLOCKS (0) or QMV_LAYOUT_PLANES      */
  int64_t rows, cols;     /* logical shape of W                              */
  const void* data;       /* device pointer to the packed bytes (16 B aligned)*/
  uint64_t nbytes;        /* == qmv_packed_size(fmt, rows, cols), or         */
                          /* qmv_planes_size for QMV_LAYOUT_PLANES           */
  uint64_t scales_offset; /* INT4_G128: byte offset of the scales plane;     */
                          /* QMV_LAYOUT_PLANES: offset a of code plane A;    */
                          /* 0 for the block formats                         */
} qmv_weights;

/* Codes per block: 32, 256, 256, 128, 256 (Q8_0, Q4_K, Q6_K, INT4_G128,
 * Q5_K); 0 for an unknown format. */
int32_t qmv_block_size(int32_t fmt);

/* Bytes of a packed rows x cols tensor; 0 if fmt is unknown, rows or cols < 1
 * or cols is not a multiple of the block size. */
uint64_t qmv_packed_size(int32_t fmt, int64_t rows, int64_t cols);

/* ---- Host block packer (host memory in and out, caller-owned) ----------
 * Each packer writes the canonical bytes of the layouts above into `out`
 * (out_bytes must be >= qmv_packed_size).  Codes are given per weight in
 * natural [rows][cols] order; scales are fp16 bit patterns.  Range errors
 * (QMV_ERR_RANGE) are detected before anything is written. */

/* Q8_0: d_bits [rows][cols/32], q [rows][cols] (any int8). */
int32_t qmv_pack_q8_0(const uint16_t* d_bits, const int8_t* q, int64_t rows,
                      int64_t cols, uint8_t* out, uint64_t out_bytes);

/* Q4_K: d_bits, dmin_bits [rows][cols/256]; sc6, m6 [rows][cols/256][8] each
 * in 0..63; q4 [rows][cols] in 0..15. */
int32_t qmv_pack_q4_k(const uint16_t* d_bits, const uint16_t* dmin_bits,
                      const uint8_t* sc6, const uint8_t* m6, const uint8_t* q4,
                      int64_t rows, int64_t cols, uint8_t* out,
                      uint64_t out_bytes);

/* Q5_K: d_bits, dmin_bits [rows][cols/256]; sc6, m6 [rows][cols/256][8] each
 * in 0..63; q5 [rows][cols] in 0..31. */
int32_t qmv_pack_q5_k(const uint16_t* d_bits, const uint16_t* dmin_bits,
                      const uint8_t* sc6, const uint8_t* m6, const uint8_t* q5,
                      int64_t rows, int64_t cols, uint8_t* out,
                      uint64_t out_bytes);

/* Q6_K: d_bits [rows][cols/256]; sc8 [rows][cols/256][16] (any int8);
 * q6 [rows][cols] in 0..63. */
int32_t qmv_pack_q6_k(const uint16_t* d_bits, const int8_t* sc8,
                      const uint8_t* q6, int64_t rows, int64_t cols,
                      uint8_t* out, uint64_t out_bytes);

/* INT4_G128: s_bits [rows][cols/128]; q [rows][cols] in -8..7. */
int32_t qmv_pack_int4_g128(const uint16_t* s_bits, const int8_t* q,
                           int64_t rows, int64_t cols, uint8_t* out,
                           uint64_t out_bytes);

/* Bytes of the QMV_LAYOUT_PLANES layout of a rows x cols tensor; 0 if the
 * format has no plane layout (Q8_0, INT4_G128) or the shape is
 * invalid. */
uint64_t qmv_planes_size(int32_t fmt, int64_t rows, int64_t cols);

/* Enqueue the repack of canonical Q4_K, Q5_K or Q6_K blocks (src, QMV_LAYOUT_BLOCKS) into
 * the plane layout at dst (device memory of dst_bytes >= qmv_planes_size
 * bytes, 16-byte aligned, 256 recommended, not overlapping src) and fill
 * *out with a QMV_LAYOUT_PLANES descriptor of dst.  Bytes are moved, not
 * changed: qmv_dequant of the result equals qmv_dequant of src bit for bit.
 * src must stay alive until the repack has run (stream order); after that
 * the caller may free it.  Errors: QMV_ERR_NULL, QMV_ERR_UNSUPPORTED (a
 * format without a plane layout, or src already in planes), QMV_ERR_SIZE
 * (dst_bytes too small), QMV_ERR_ALIGN, QMV_ERR_SHAPE (dst overlaps src),
 * or any error of the src descriptor's validation. */
int32_t qmv_repack_planes(const qmv_weights* src, void* dst,
                          uint64_t dst_bytes, qmv_weights* out, void* stream);

/* Descriptor for plane-layout bytes already in device memory (for example
 * planes made by qmv_repack_planes earlier and kept): validates format,
 * shape, size (nbytes == qmv_planes_size; QMV_ERR_SIZE) and alignment and
 * fills *out with layout QMV_LAYOUT_PLANES.  No HIP call, no allocation; the
 * bytes are not inspected. */
int32_t qmv_create_weights_planes(int32_t fmt, int64_t rows, int64_t cols,
                                  const void* dev_planes, uint64_t nbytes,
                                  qmv_weights* out);

/* Validate shape and size and fill *out.  No HIP call, no allocation.
 * dev_packed must be 16-byte aligned (QMV_ERR_ALIGN) and nbytes must equal
 * qmv_packed_size (QMV_ERR_SIZE). */
int32_t qmv_create_weights(int32_t fmt, int64_t rows, int64_t cols,
                           const void* dev_packed, uint64_t nbytes,
                           qmv_weights* out);

/* y = W x for `batch` activation rows (the decode GEMV; see top of file).
 * fmt, rows and cols must repeat the descriptor's (QMV_ERR_FORMAT otherwise),
 * x is [batch][cols] of x_dtype (QMV_F32, QMV_F16 or QMV_BF16), y is
 * [batch][rows] fp32; x and y device pointers, 16-byte aligned.  Enqueues on
 * `stream` and returns; legal inside HIP stream capture.  batch >= 2 rows
 * (Q4_K x bf16: 2..4 rows) run the multi-row GEMV in every format: weights
 * read once per two or four activation rows (fp32: two) for cols <= 4096
 * (Q8_0: 2048), and, for fp16/bf16 rows, once per two rows up to eight times
 * that width (Q4_K x bf16: at two rows); each output row equals bit for bit
 * the batch-1 call on that activation row.  Q4_K x fp16 with 5 or more rows
 * runs on the matrix cores with fp16 operands (exact products, fp32 sums).
 * Other Q4_K x bf16 calls with batch >= 2 run the matrix-core path (weights
 * read once for up to 16 activation rows, once per tile of 32, 64 or 128
 * rows above; exact products, fp32 sums, results independent of timing).
 * Otherwise each activation row is a GEMV over the packed weights.  Q4_K,
 * Q5_K and Q6_K weights in QMV_LAYOUT_PLANES run the same arithmetic, in the
 * same order, as the canonical layout on every one of these paths, so
 * results equal bit for bit.  This call uses no workspace; the faster
 * register-dequantized kernels for large batches need one and run through
 * qmv_gemv_multi_ws (or qmv_gemv_noalloc). */
int32_t qmv_gemv(int32_t fmt, const qmv_weights* W, const void* x,
                 int32_t x_dtype, float* y, int64_t rows, int64_t cols,
                 int64_t batch, void* stream);

/* qmv_gemv for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc) and
 * have no workspace to give: the same arguments and checks as qmv_gemv and
 * the kernels and results, bit for bit, of qmv_gemv_multi_ws with this one
 * item and a large enough workspace -- but the register-dequantized
 * kernels take the library's fixed device array of QMV_NOALLOC_SCRATCH_BYTES
 * (64 MiB, one per GPU, held from library load until the process ends) as
 * their workspace.  No path of this call allocates.  A call whose workspace
 * (qmv_workspace_size of that item) would exceed the array fails with
 * QMV_ERR_SIZE before any launch; the 7B decoder layer's matrices fit up to
 * 512 activation rows.  Nothing in the array needs to start at zero.  Every
 * call on one GPU shares the array and leaves it holding its own
 * intermediates: calls that overlap on one GPU (several streams or
 * threads, or graph replays of such calls) race and must be serialized by
 * the caller. */
#define QMV_NOALLOC_SCRATCH_BYTES (64ull << 20)
int32_t qmv_gemv_noalloc(int32_t fmt, const qmv_weights* W, const void* x,
                         int32_t x_dtype, float* y, int64_t rows,
                         int64_t cols, int64_t batch, void* stream);

/* One matrix of a multi-matrix GEMV launch. */
typedef struct qmv_gemv_item {
  const qmv_weights* W; /* packed W_i (all items share the launch's format)  */
  const void* x;        /* [batch][W->cols] activations of the launch's dtype */
  float* y;             /* [batch][W->rows] fp32, overwritten                 */
} qmv_gemv_item;

/* y_i = W_i x_i for n (1..16) matrices in one launch: the matrices' rows are
 * spread over one resident generation of workgroups, so small matrices share
 * the ramp-up and tail of large ones.  Meant for the projections of a decode
 * step that read the same activation (q/k/v, gate/up) -- the fused-QKV and
 * multi-weight dispatch of hipfire ("Review hipfire prefill optimization
 * levers"; "Implementation requirements for multi-weight Q8 WMMA dispatch":
 * one dtype for every weight of a dispatch, K a whole number of blocks, and
 * output tiles that never overlap).  Each item is validated as in qmv_gemv;
 * the y ranges must be disjoint (QMV_ERR_SHAPE otherwise); every x and y is a
 * 16-byte aligned device pointer; all items share one layout
 * (QMV_ERR_UNSUPPORTED otherwise).  Results equal n separate qmv_gemv calls
 * up to float32 summation order; where the calls would take the multi-row
 * GEMV or the matrix-core path, the launch routes each item as its own call
 * would, and results equal bit for bit -- except for two or more Q4_K
 * matrices of at most 4096 columns and 8192 rows in all at 5..16 fp16/bf16
 * rows, which share one multi-row launch (each output row then equals the
 * batch-1 result bit for bit) where a call of one of them alone would take
 * the matrix cores.  One activation row against exactly two matrices of one
 * shape within one wave's K slice on the same x pointer (gate and up) runs
 * as one launch whose two-row tiles pair row i of both: results equal the
 * lone calls bit for bit, except INT4 (its lone call runs one-row tiles),
 * which differs in float32 summation order.  Uses no workspace. */
int32_t qmv_gemv_multi(int32_t fmt, int32_t x_dtype, int64_t batch,
                       const qmv_gemv_item* items, int32_t n, void* stream);

/* *bytes = the device workspace that qmv_gemv_multi_ws needs for exactly
 * these arguments (the same fmt, x_dtype, batch and items, whose weight
 * descriptors and shapes are read; x and y are only checked, never read):
 * 0 when the launch takes no register-dequantized kernel.  Returns the
 * status the launch would return for these arguments (bytes NULL:
 * QMV_ERR_NULL), with *bytes = 0 on error.  No HIP call.  The size is (a
 * run's cols x activation rows x 2 bytes, rounded up to 256) + (activation
 * rows x 4, rounded up to 256), plus, where K is cut into S = 2..8 slices, S
 * partial outputs of weight rows x activation rows x 4 bytes per matrix; at
 * 512 bf16 rows the 7B FFN gate needs 3.7 MB, the down matrix (K in slices)
 * 56 MB. */
int32_t qmv_workspace_size(int32_t fmt, int32_t x_dtype, int64_t batch,
                           const qmv_gemv_item* items, int32_t n,
                           uint64_t* bytes);

/* qmv_gemv_multi with a caller-owned device workspace, which lets large
 * batches run the register-dequantized kernels: against Q4_K matrices of at
 * least 256 weight rows, from 65 fp16/bf16 activation rows (from 17 against
 * matrices of 8192 columns and more, and for runs of two to four
 * consecutive items on the same x pointer with the same cols and layout).
 * There the activations are converted once to fp16 (a bf16 row scaled by
 * the power of two that brings its largest |x| into [2^14, 2^15)) and each
 * weight is rounded to fp16 (relative error near 2^-11), so the products
 * are no longer exact; the normwise bound still holds (about 4e-4 on the 7B
 * FFN shapes).  K may be cut into slices whose partial outputs are summed in
 * a fixed order, so results stay independent of timing.  A run shares one
 * activation conversion, one product launch and one partial-output sum;
 * its items meet the same bound as their own calls but may differ from them
 * in float32 summation order, since the run's K slicing follows all its
 * rows.  Every other item runs as in qmv_gemv_multi, bit for bit.
 * workspace: device pointer, 256-byte aligned (QMV_ERR_ALIGN), NULL only
 * with workspace_bytes 0 (QMV_ERR_NULL); workspace_bytes below
 * qmv_workspace_size of the same arguments fails with QMV_ERR_SIZE before
 * any launch.  NULL with 0 bytes means no workspace: qmv_gemv_multi's
 * kernels.  The caller owns the buffer; the launch writes intermediates
 * there (converted activations, row scales, partial outputs) that need no
 * initial value, and stream order keeps them apart: launches that may run
 * at the same time (other streams) need buffers of their own.  Enqueues
 * only; legal inside HIP stream capture. */
int32_t qmv_gemv_multi_ws(int32_t fmt, int32_t x_dtype, int64_t batch,
                          const qmv_gemv_item* items, int32_t n,
                          void* workspace, uint64_t workspace_bytes,
                          void* stream);

/* h = silu(W_gate x) * (W_up x), elementwise, for `batch` activation rows:
 * the input of a SwiGLU FFN's down projection (hipfire, the Qwen2 decoder's
 * "Key Technical Specifications": a SwiGLU FFN), silu(g) = g / (1 + e^-g),
 * in one launch whose epilogue combines the two projections of each output,
 * so neither g nor u is written to memory.  The unfused chain stays
 * available and is the correctness baseline (hipEngine 0.3.0, "Core
 * principles": fused composites coexist with a numerically equivalent
 * unfused chain): qmv_gemv_multi over the two matrices, then silu(g) * u.
 * Wg and Wu are the gate and up matrices, of format fmt, both rows x cols
 * and in one layout (QMV_ERR_FORMAT / QMV_ERR_UNSUPPORTED otherwise); x is
 * [batch][cols] of x_dtype (QMV_F32, QMV_F16 or QMV_BF16), h is
 * [batch][rows] fp32, overwritten; both device pointers, 16-byte aligned,
 * not overlapping (QMV_ERR_SHAPE).  Every row must lie within one wave's K
 * slice: cols <= 4096 (Q8_0: 2048), else QMV_ERR_UNSUPPORTED.  Each
 * activation row is one pass over both matrices (the batch-1 GEMV per
 * row), each output pair (g, u) is computed with the arithmetic of the
 * GEMV's two-row tiles, and silu(g) = g * rcp(1 + 2^(-g log2 e)) uses the
 * hardware exp2 and reciprocal (about 1 ulp each): h differs from
 * silu(g) * u of the same kernel's g and u only in the rounding of the
 * epilogue (relative error within a few ulp, plus about |g| 2^-24 where g is
 * very negative and h tiny; -0 below g = -88).
 * Enqueues on `stream` and returns; no workspace; legal inside HIP stream
 * capture. */
int32_t qmv_gemv_swiglu(int32_t fmt, const qmv_weights* Wg,
                        const qmv_weights* Wu, const void* x, int32_t x_dtype,
                        float* h, int64_t rows, int64_t cols, int64_t batch,
                        void* stream);

/* out = W as a dense [rows][cols] matrix of out_dtype (QMV_F32: the exact
 * value rounded once to fp32, bit-exact; QMV_F16 / QMV_BF16: that fp32 value
 * rounded to nearest-even).  out is a 16-byte aligned device pointer to
 * rows*cols elements. */
int32_t qmv_dequant(const qmv_weights* W, void* out, int32_t out_dtype,
                    void* stream);

/* Measurement kernels for the HBM roofline (not part of the GEMV path).
 * qmv_probe_read streams nbytes (multiple of 16) from src with nontemporal
 * 128-bit loads, one contiguous chunk per workgroup (the fastest streaming
 * read measured on the part), and writes one fp32 per workgroup to out (out
 * must hold
 * qmv_probe_read_outputs(nbytes) floats).  qmv_probe_copy copies nbytes
 * (multiple of 16) from src to dst with 128-bit loads and stores. */
int64_t qmv_probe_read_outputs(uint64_t nbytes);
int32_t qmv_probe_read(const void* src, uint64_t nbytes, float* out,
                       void* stream);
int32_t qmv_probe_copy(const void* src, void* dst, uint64_t nbytes,
                       void* stream);

/* Static text for a status code; "unknown status" otherwise. */
const char* qmv_status_string(int32_t status);

/* Details of the last error raised on the calling thread ("" if none). */
const char* qmv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QMV_H */
