/*
 * libwq -- group-wise asymmetric INT4 weight quantization and the fused
 * dequantize-and-multiply y = x * What^T for AMD Instinct MI355X (gfx950).
 *
 * The method (from "Quantization for LLM inference: FP8, INT4 (GPTQ, AWQ) and
 * GGUF - the model's accounting zoom", section "The minimum maths: scale and
 * zero-point"): a weight row is cut into groups of g consecutive weights along
 * K; each group gets a scale s = (max - min) / 15 and an integer zero-point
 * z = round(-min / s), each weight the 4-bit code q = clip(round(w/s + z), 0, 15),
 * and decoding is What = s * (q - z).  The matrix product with fp16 activations
 * is the weight-only ("W4A16") matmul that decode runs as a memory-bound GEMV
 * and large batches run as a dense GEMM ("Quantization Methods Compared: INT8,
 * GPTQ, AWQ, FP8, FP4 and KV-Cache Quantization", section "Hardware, formats and
 * the roofline: why INT4 gave no speedup at batch 128": kernels dequantize to
 * fp16 inside the matmul).
 *
 * Numerics fixed by this library where the pages leave them open:
 *   - the scale is stored as IEEE fp16, converted from the fp32 value
 *     fl32(fl32(hi - lo) / 15) with round-to-nearest-even, subnormals kept,
 *     where lo = min(0, min of group) and hi = max(0, max of group);
 *   - z = clamp(rne(fl32(-lo / s)), 0, 15) and
 *     q = clamp(rne(fl32(fl32(w / s) + z)), 0, 15), with s the stored fp16 scale,
 *     every operation a single correctly rounded binary32 operation;
 *   - a group whose fp16 scale is 0 stores s = 0, z = 0 and codes 0;
 *   - What = s * (q - z) is exact in fp32; fp16 and bf16 outputs are one
 *     round-to-nearest-even of that value;
 *   - y is fp16 (round-to-nearest-even) of an fp32 accumulation.
 *
 * Layouts (all row-major, the weight matrix is W[N][K]: row = output channel):
 *   x        [M][K] fp16                        activations
 *   y        [M][N] fp16                        outputs
 *   s_f16    [N][G] fp16 bit patterns, G = K / group
 *   z_codes  [N][G] uint8, values 0..15          (unpacked zero-points)
 *   q_codes  [N][K] uint8, values 0..15          (unpacked codes)
 *   zpacked  [N][ceil(G/2)] bytes, group j in the low nibble of byte j/2 when j
 *            is even, in the high nibble when j is odd
 *   qpacked  device tile layout: rows padded to Np = ceil(N/16)*16, columns to
 *            Kp = ceil(K/128)*128 (pad codes are 0); tile (nb, kt) of 16 rows x
 *            128 columns occupies 1024 bytes at byte offset
 *            (nb * Kp/128 + kt) * 1024; inside it, "lane" l = r + 16*c
 *            (r = 0..15 row in tile, c = 0..3) owns the 16 bytes at 16*l, read
 *            as four little-endian 32-bit words j = 0..3; word j holds columns
 *            32*j + 8*c + e (e = 0..7) of the tile, column e in nibble
 *            4*(e%2) + e/2 (so a word splits into four fp16 pairs of
 *            neighbouring columns with one shift and mask each).
 *
 * Conventions:
 *   - Every pointer argument is device memory (hipMalloc or equivalent) unless
 *     stated otherwise.  The caller owns every buffer; libwq allocates nothing.
 *   - `stream` is a hipStream_t (NULL = the default stream).  All work is
 *     enqueued asynchronously on it; no call synchronizes.
 *   - Return values: WQ_OK, or a negative wq_status.  Argument errors are
 *     detected on the host before anything is enqueued.  WQ_EHIP reports a
 *     failed launch (including an asynchronous error left by earlier work).
 *   - Preconditions not checked on the fast path: weights are finite and every
 *     group's range is below 15 * 65520 (so the fp16 scale is finite); codes
 *     and zero-points passed to wq_pack_int4 are 0..15 (higher bits ignored);
 *     buffers do not overlap.
 *   - libwq keeps no state; calls on different streams may run concurrently
 *     as long as they do not share output or workspace buffers.
 */
#ifndef LIBWQ_H
#define LIBWQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    WQ_OK = 0,
    WQ_EINVAL = -1,       /* null pointer, non-positive size, bad dtype, path or scheme */
    WQ_EUNSUPPORTED = -2, /* group not 32 or 128, K not a multiple of group (or of 32 / 128 where stated) */
    WQ_EALIGN = -3,       /* pointer not aligned as documented */
    WQ_EWORKSPACE = -4,   /* workspace missing or smaller than required */
    WQ_EHIP = -5          /* a HIP runtime call or kernel launch failed */
} wq_status;

typedef enum { WQ_F32 = 0, WQ_BF16 = 1, WQ_F16 = 2 } wq_dtype;

typedef enum {
    WQ_ASYM = 0, /* asymmetric: s = (max - min) / 15, z = round(-min / s) */
    WQ_SYM = 1   /* symmetric: s = max|w| / 7, codes q + 8 (q in -7..7), z = 8 */
} wq_scheme;

typedef enum {
    WQ_PATH_AUTO = 0, /* the GEMV or the MFMA GEMM kernel by the rule below */
    WQ_PATH_GEMV = 1, /* force the split-K GEMV kernel (any M; dot products on the matrix cores) */
    WQ_PATH_MFMA = 2  /* force the MFMA tile GEMM kernel (any M) */
} wq_path;

/* WQ_PATH_AUTO.  The GEMV kernel for few rows of x, the MFMA GEMM otherwise
 * (every GEMV takes its dot products on the matrix cores, so its time grows
 * slowly with M up to its 16-row activation tile).  Every format keeps the
 * GEMV up to WQ_AUTO_NARROW_GEMV_MAX_M rows when N is at most
 * WQ_AUTO_GEMV_MAX_N (the MFMA GEMM's 128-column workgroups are then too few
 * to fill the GPU).  Otherwise the GEMV runs up to WQ_AUTO_INT4_GEMV_MAX_M
 * rows of 4-bit integer codes (up to WQ_AUTO_INT4_G32_LONG_K_GEMV_MAX_M rows
 * at group 32 with K above WQ_AUTO_INT4_G32_LONG_K), up to
 * WQ_AUTO_FP4_GEMV_MAX_M rows of MXFP4 or NVFP4 codes and up to
 * WQ_AUTO_INT8_GEMV_MAX_M rows of int8 codes.  Measured (back-to-back calls,
 * us, GEMV / MFMA GEMM, N = 8192): 4-bit codes, K = 8192: M = 8, g = 32
 * 11.3 / 16.1; M = 16, g = 32 13.1 / 16.6, g = 128 12.5 / 15.7; M = 24, g = 32
 * 23.8 / 18.1; K = 16384, M = 16: g = 128 20.9 / 24.1, g = 32 22.8 / 25.5;
 * K = 28672, M = 16: g = 128 33.5 / 33.5, g = 32 38.0 / 35.8, M = 8, g = 32
 * 31.1 / 34.3; N = 28672, K = 8192, M = 16, g = 128: 32.8 / 34.6.  MXFP4,
 * M = 16: K = 8192 11.3 / 15.7, K = 28672 31.4 / 33.1; NVFP4, M = 16: K = 8192
 * 12.3 / 16.2, K = 28672 32.8 / 33.5.  int8, g = 128, K = 8192: M = 8 14.5 /
 * 19.3, M = 16 18.8 / 18.1.  M = 32, N = 2048: MXFP4 10.5 / 12.5, NVFP4
 * 10.4 / 13.0, int8 12.3 / 13.3; 4-bit at N = 1024 6.6 / 13.3. */
#define WQ_AUTO_GEMV_MAX_N 2048
#define WQ_AUTO_NARROW_GEMV_MAX_M 32
#define WQ_AUTO_INT4_GEMV_MAX_M 16
#define WQ_AUTO_INT4_G32_LONG_K 16384
#define WQ_AUTO_INT4_G32_LONG_K_GEMV_MAX_M 8
#define WQ_AUTO_FP4_GEMV_MAX_M 16
#define WQ_AUTO_INT8_GEMV_MAX_M 8

/* A product that splits K across workgroups uses a caller-provided workspace:
 * WQ_WORKSPACE_COUNTER_BYTES bytes of 32-bit counters (one per output tile),
 * then the fp32 partial sums.  The counter bytes must be zero before a
 * workspace's first use and every call puts back to zero those it used; the
 * partial sums are overwritten by each call and need no clearing. */
#define WQ_WORKSPACE_COUNTER_BYTES 2048

/* Library version, major * 10000 + minor * 100 + patch. */
int wq_version(void);

/* Static string describing a status code. */
const char* wq_strerror(int status);

/* Byte sizes of the device layouts for an [N][K] weight matrix with the given
 * group: qpacked (tile layout, padded), s_f16 ([N][G] fp16) and zpacked
 * ([N][ceil(G/2)]).  Host-only.  Any output pointer may be NULL. */
int wq_layout_bytes(int64_t N, int64_t K, int group,
                    size_t* qpacked_bytes, size_t* s_bytes, size_t* zpacked_bytes);

/* Group quantization (steps: per-group min/max, scale and zero-point, encoding,
 * packing) -- "The minimum maths: scale and zero-point", equations for s, z and
 * the encoding, with the readings listed above.
 *   W        [N][K] weights, w_dtype WQ_F32, WQ_BF16 or WQ_F16; 16-byte aligned,
 *            K * element size a multiple of 16 bytes when K > group
 *   s_f16    [N][G] output scales (required, 2-byte aligned)
 *   q_codes  [N][K] output codes, or NULL
 *   z_codes  [N][G] output zero-points, or NULL
 *   qpacked  tile-layout output codes (wq_layout_bytes), 16-byte aligned, or NULL
 *   zpacked  [N][ceil(G/2)] output packed zero-points, or NULL
 * Deterministic: the same input gives the same bytes on every run. */
int wq_quantize_groups(const void* W, int w_dtype, int64_t N, int64_t K, int group,
                       uint8_t* q_codes, uint16_t* s_f16, uint8_t* z_codes,
                       uint32_t* qpacked, uint8_t* zpacked, void* stream);

/* As wq_quantize_groups, with the quantization scheme (wq_scheme).  WQ_SYM is
 * the symmetric 4-bit quantizer of "Test-time quantization", section "The
 * maths that matter" (s = M / (2^(b-1) - 1) at b = 4, M = max|w| over the
 * group) with the code q = round(w / s) of "Quantization Methods Compared",
 * section "What quantisation does", read as:
 *   s = fp16(fl32(M / 7)) (round-to-nearest-even, subnormals kept);
 *   q = clamp(rne(fl32(w / s)), -7, 7), stored as the code q + 8;
 *   zero-point 8 for every group (z_codes / zpacked hold 8), so
 *   s * (code - zero-point) = s * q and every other entry point (dequant,
 *   product) applies unchanged;
 *   a group whose fp16 scale is 0 stores s = 0 and codes 8.
 * Same arguments, layouts and error behaviour as wq_quantize_groups; WQ_EINVAL
 * for an unknown scheme. */
int wq_quantize_groups_ex(const void* W, int w_dtype, int64_t N, int64_t K, int group, int scheme,
                          uint8_t* q_codes, uint16_t* s_f16, uint8_t* z_codes,
                          uint32_t* qpacked, uint8_t* zpacked, void* stream);

/* ---- AWQ-style per-input-channel scaling -------------------------------------
 * "Quantization for LLM inference", section "AWQ": the weights of a salient
 * input channel (one with large mean activation magnitude) are multiplied by a
 * factor before quantizing and that channel's activations are divided by it,
 * so the product is unchanged while the salient weights get a finer effective
 * step ("Quantization Methods Compared", section "The methods compared").
 * Read as: W' = W diag(alpha) with alpha[k] > 0 per input channel, quantized
 * with the usual group quantizer; x' = x / alpha at run time; y = x' W'hat^T.
 * In a model x / alpha folds into the preceding operation's weights; the
 * standalone kernel below serves callers without one. */

/* As wq_quantize_groups_ex, each weight first multiplied by alpha[k] (device
 * fp32 [K], 16-byte aligned, positive and finite; one fp32 multiplication)
 * before the group min/max, scale, zero-point and encoding.  alpha == NULL is
 * wq_quantize_groups_ex.  The scaled weights must meet the same range
 * precondition. */
int wq_quantize_groups_scaled(const void* W, int w_dtype, int64_t N, int64_t K, int group, int scheme,
                              const float* alpha, uint8_t* q_codes, uint16_t* s_f16, uint8_t* z_codes,
                              uint32_t* qpacked, uint8_t* zpacked, void* stream);

/* x_out[m][k] = fp16(fl32(x[m][k] / alpha[k])) (correctly rounded division,
 * then round-to-nearest-even to fp16).  x_f16, x_out_f16 [M][K] and alpha [K]
 * 16-byte aligned; K a multiple of 8 (WQ_EUNSUPPORTED otherwise); x_out may
 * equal x (in place). */
int wq_scale_activations(const uint16_t* x_f16, int64_t M, int64_t K, const float* alpha,
                         uint16_t* x_out_f16, void* stream);

/* out[k] = (|x[0][k]| + |x[1][k]| + ... + |x[M-1][k]|) / M, the sum taken in row
 * order in fp32 and divided in fp32: the mean activation magnitude per input
 * channel over calibration rows x [M][K], from which salient channels are
 * chosen.  Deterministic. */
int wq_channel_absmean(const uint16_t* x_f16, int64_t M, int64_t K, float* out, void* stream);

/* Packing of codes and zero-points into the device layouts -- "Numerical
 * example" (eight 4-bit codes occupy four bytes; a 4-bit zero-point takes half
 * a byte).  q_codes [N][K] and z_codes [N][G] in, qpacked (16-byte aligned,
 * padding written as 0) and zpacked out. */
int wq_pack_int4(const uint8_t* q_codes, const uint8_t* z_codes, int64_t N, int64_t K, int group,
                 uint32_t* qpacked, uint8_t* zpacked, void* stream);

/* Dequantization What = s * (q - z) -- "The minimum maths", decoding equation.
 * Writes W_hat [N][K] as out_dtype (WQ_F32 exact; WQ_F16 / WQ_BF16 one
 * round-to-nearest-even of the exact value).  W_hat 16-byte aligned. */
int wq_dequant(const uint32_t* qpacked, const uint16_t* s_f16, const uint8_t* zpacked,
               int64_t N, int64_t K, int group, int out_dtype, void* W_hat, void* stream);

/* Workspace bytes wq_gemm_w4a16 / wq_gemm_w4a16_ex need for this shape, enough
 * for either kernel family (may be 0).  Either kernel needs one only when it
 * splits K across workgroups to fill the GPU (fp32 partial sums plus one
 * counter per output tile): the GEMV for few row blocks, the MFMA GEMM for few
 * 128-column blocks.  Host-only. */
size_t wq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int group);

/* Workspace bytes of the one kernel family `path` (wq_path) selects for this
 * shape: what wq_gemm_w4a16_ex with that path requires (0 for bad arguments).
 * Host-only. */
size_t wq_gemm_workspace_bytes_ex(int64_t M, int64_t N, int64_t K, int group, int path);

/* y = x * What^T with What = s * (q - z) dequantized inside the kernel -- the
 * fused weight-only matmul of "Hardware, formats and the roofline".  The
 * WQ_PATH_AUTO rule (wq_path) picks the split-K GEMV kernel or the MFMA tile
 * GEMM kernel (which also splits K when its grid is small).
 *   x_f16     [M][K] fp16, 16-byte aligned, finite
 *   qpacked   tile-layout codes, 16-byte aligned; s_f16 [N][G]; zpacked [N][ceil(G/2)]
 *   y_f16     [M][N] fp16 output, 2-byte aligned
 *   workspace at least wq_gemm_workspace_bytes(M, N, K, group) bytes of device
 *             memory, 256-byte aligned, its first WQ_WORKSPACE_COUNTER_BYTES
 *             bytes zero before its first use; may be NULL when that size is
 *             0.  Every call leaves those counter bytes zero again, so one
 *             workspace serves later calls of any shape without clearing;
 *             calls that may run concurrently need separate workspaces.
 * Results are deterministic (fixed summation order). */
int wq_gemm_w4a16(int64_t M, int64_t N, int64_t K, int group,
                  const uint16_t* x_f16, const uint32_t* qpacked, const uint16_t* s_f16,
                  const uint8_t* zpacked, uint16_t* y_f16,
                  void* workspace, size_t workspace_bytes, void* stream);

/* count products of one shape issued back to back on `stream`, in order:
 * y_f16[i] = x_f16[i] * What_i^T with What_i from (qpacked[i], s_f16[i],
 * zpacked[i]), as wq_gemm_w4a16 would compute each.  The five arrays are host
 * arrays of count device pointers.  Every product is checked before the first
 * is enqueued, so an argument error enqueues nothing; the products run in
 * stream order, so one workspace (sized for the shape) serves all of them.
 * For decode loops whose per-call host cost would exceed a kernel's time. */
int wq_gemm_w4a16_seq(int count, int64_t M, int64_t N, int64_t K, int group,
                      const uint16_t* const* x_f16, const uint32_t* const* qpacked,
                      const uint16_t* const* s_f16, const uint8_t* const* zpacked,
                      uint16_t* const* y_f16, void* workspace, size_t workspace_bytes, void* stream);

/* Describes, as one NUL-terminated line written into buf (host memory,
 * buf_len bytes, truncated to fit), the kernel and launch shape that
 * wq_gemm_w4a16_ex would use for this problem and path: kernel template
 * parameters, grid, block, LDS bytes and (GEMV) the number of K splits.
 * Host-only; launches nothing.  WQ_EINVAL for a NULL or empty buffer or a bad
 * size or path, WQ_EUNSUPPORTED as for wq_gemm_w4a16. */
int wq_gemm_plan(int64_t M, int64_t N, int64_t K, int group, int path, char* buf, size_t buf_len);

/* As wq_gemm_w4a16, with the kernel family chosen by `path` (wq_path). */
int wq_gemm_w4a16_ex(int64_t M, int64_t N, int64_t K, int group,
                     const uint16_t* x_f16, const uint32_t* qpacked, const uint16_t* s_f16,
                     const uint8_t* zpacked, uint16_t* y_f16,
                     void* workspace, size_t workspace_bytes, int path, void* stream);

/* Bytes of the fixed per-GPU scratch of wq_gemm_w4a16_noalloc: the split-K
 * counter region and 16 MiB of fp32 partial sums (enough for every product
 * whose kernel splits K at K <= 28672 with N up to 8192 at M = 128, e.g. the
 * 8192 x 28672 down projection). */
#define WQ_NOALLOC_SCRATCH_BYTES (WQ_WORKSPACE_COUNTER_BYTES + (16 << 20))

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * wq_gemm_w4a16 with the workspace taken from a fixed device array of
 * WQ_NOALLOC_SCRATCH_BYTES that the library holds once per GPU for the life of
 * the process, instead of from the caller.  Same arguments (minus the
 * workspace), kernels, results and errors as wq_gemm_w4a16; calls no
 * allocating routine.  WQ_EWORKSPACE when the product's kernel would need more
 * scratch than WQ_NOALLOC_SCRATCH_BYTES (nothing is enqueued).  The first call
 * on a device looks up that device's scratch address and clears its counters
 * with a kernel on `stream`; each product leaves them zero again.  Every call
 * on one GPU shares that GPU's scratch: calls that may overlap on one GPU (on
 * different streams, or from different threads without ordering) race and
 * must be serialized by the caller. */
int wq_gemm_w4a16_noalloc(int64_t M, int64_t N, int64_t K, int group,
                          const uint16_t* x_f16, const uint32_t* qpacked, const uint16_t* s_f16,
                          const uint8_t* zpacked, uint16_t* y_f16, void* stream);

/* ---- Group absmax int8 weights (W8A16) --------------------------------------
 * The int8 rule of "Quantization Methods Compared: INT8, GPTQ, AWQ, FP8, FP4
 * and KV-Cache Quantization", section "What quantisation does: scale, round,
 * and the outlier that ruins a group" (s = max|w| / 127, q = round(w / s),
 * decoding q * s), with one scale per group of `group` (32 or 128) weights
 * along K, read as:
 *   s = fp16(fl32(M / 127)), M = max|w| over the group (round-to-nearest-even,
 *   subnormals kept);
 *   q = clamp(rne(fl32(w / s)), -127, 127) with the stored scale s;
 *   a group whose fp16 scale is 0 stores s = 0 and codes 0;
 *   What = s * q, exact in fp32.
 * No zero-points.  Layouts:
 *   q_codes  [N][K] int8 (two's complement)
 *   s_f16    [N][G] fp16 bit patterns, G = K / group
 *   qpacked  2048-byte tiles of 16 rows x 128 columns (rows padded to
 *            ceil(N/16)*16, columns to ceil(K/128)*128 with code 0), tile
 *            (nb, kt) at byte offset (nb * Kp/128 + kt) * 2048; inside it half
 *            h = 0, 1 at byte 1024*h, lane l = r + 16*c at byte 16*l of the
 *            half, and byte 8*i + e (i = 0, 1; e = 0..7) of that holds the code
 *            of column 32*(2h + i) + 8*c + e of row r.
 * Same conventions as the 4-bit entry points (device pointers, caller-owned
 * buffers, asynchronous on `stream`, status codes). */

/* Byte sizes of qpacked (2048-byte tiles) and s_f16 for [N][K] at `group`.
 * Host-only; either output may be NULL. */
int wq_layout_bytes_w8(int64_t N, int64_t K, int group, size_t* qpacked_bytes, size_t* s_bytes);

/* Group absmax int8 quantization of W [N][K] (w_dtype WQ_F32, WQ_BF16 or
 * WQ_F16; 16-byte aligned).  s_f16 [N][G] required; q_codes [N][K] (8-byte
 * aligned) and qpacked (16-byte aligned) may each be NULL.  Deterministic. */
int wq_quantize_w8(const void* W, int w_dtype, int64_t N, int64_t K, int group,
                   int8_t* q_codes, uint16_t* s_f16, uint8_t* qpacked, void* stream);

/* int8 codes [N][K] -> qpacked tiles (padding written as 0).  K must be a
 * multiple of 32 (WQ_EUNSUPPORTED otherwise); q_codes 8-byte aligned,
 * qpacked 16-byte aligned. */
int wq_pack_int8(const int8_t* q_codes, int64_t N, int64_t K, uint8_t* qpacked, void* stream);

/* What = s * q into W_hat [N][K] as out_dtype (WQ_F32 exact; WQ_F16 / WQ_BF16
 * one round-to-nearest-even of it); W_hat 16-byte aligned. */
int wq_dequant_w8(const uint8_t* qpacked, const uint16_t* s_f16, int64_t N, int64_t K, int group,
                  int out_dtype, void* W_hat, void* stream);

/* Workspace bytes for wq_gemm_w8a16 / wq_gemm_w8a16_ex, enough for either
 * kernel family with int8 codes (as wq_gemm_workspace_bytes, but the int8 GEMV
 * may split K across more workgroups than the 4-bit one).  Host-only. */
size_t wq_gemm_w8a16_workspace_bytes(int64_t M, int64_t N, int64_t K, int group);

/* y = x * What^T with What = s * q dequantized inside the kernel (the
 * weight-only product of "Hardware, formats and the roofline" with 8-bit
 * weights): the split-K GEMV or the MFMA tile GEMM by the WQ_PATH_AUTO rule.  Arguments, workspace contract, alignment, determinism and errors as
 * wq_gemm_w4a16,
 * without zero-points. */
int wq_gemm_w8a16(int64_t M, int64_t N, int64_t K, int group,
                  const uint16_t* x_f16, const uint8_t* qpacked, const uint16_t* s_f16,
                  uint16_t* y_f16, void* workspace, size_t workspace_bytes, void* stream);

/* As wq_gemm_w8a16, with the kernel family chosen by `path` (wq_path). */
int wq_gemm_w8a16_ex(int64_t M, int64_t N, int64_t K, int group,
                     const uint16_t* x_f16, const uint8_t* qpacked, const uint16_t* s_f16,
                     uint16_t* y_f16, void* workspace, size_t workspace_bytes, int path, void* stream);

/* As wq_gemm_plan, for wq_gemm_w8a16_ex. */
int wq_gemm_w8a16_plan(int64_t M, int64_t N, int64_t K, int group, int path, char* buf, size_t buf_len);

/* ---- MXFP4 weights ----------------------------------------------------------
 * "Quantization for LLM inference", section "Microscaling: NVFP4 and MXFP4":
 * 4-bit floating-point weights with one 8-bit scale per small block, in the
 * format of the microscaling paper that section cites: E2M1 elements (sign,
 * two exponent bits with bias 1, one mantissa bit: magnitudes 0, 0.5, 1, 1.5,
 * 2, 3, 4, 6), blocks of 32 consecutive weights along K, an E8M0 scale byte e8
 * meaning 2^(e8 - 127).  Read as:
 *   e8 = clamp(floor(log2 max|w|) - 2 + 127, 0, 254), 0 for an all-zero block
 *   (so the block maximum lands in [4, 8) before rounding);
 *   code = nearest E2M1 value of w / 2^(e8 - 127), ties to the even mantissa
 *   bit, saturating at 6; sign in bit 3 (kept when a negative value rounds to 0);
 *   What = E2M1(code) * 2^(e8 - 127).
 * 4.25 bits per weight.  Layouts: q_codes [N][K] uint8 (0..15); e8 [N][K/32];
 * qpacked the INT4 tile geometry (wq_layout_bytes) with column e of a word in
 * nibble e (two neighbouring columns per byte, the even one low).  K a
 * multiple of 32 (WQ_EUNSUPPORTED otherwise).  Same conventions as above. */

/* Byte sizes of qpacked and e8 for [N][K].  Host-only. */
int wq_layout_bytes_mxfp4(int64_t N, int64_t K, size_t* qpacked_bytes, size_t* e8_bytes);

/* MXFP4 quantization of W [N][K] (WQ_F32, WQ_BF16 or WQ_F16, 16-byte aligned;
 * finite).  e8 [N][K/32] required; q_codes (8-byte aligned) and qpacked
 * (16-byte aligned) may each be NULL.  Deterministic. */
int wq_quantize_mxfp4(const void* W, int w_dtype, int64_t N, int64_t K, uint8_t* q_codes, uint8_t* e8,
                      uint32_t* qpacked, void* stream);

/* Codes [N][K] (low 4 bits used) -> qpacked (padding written as 0). */
int wq_pack_mxfp4(const uint8_t* q_codes, int64_t N, int64_t K, uint32_t* qpacked, void* stream);

/* What = E2M1(code) * 2^(e8 - 127) into W_hat [N][K] (WQ_F32 exact; WQ_F16 /
 * WQ_BF16 one round-to-nearest-even of it); W_hat 16-byte aligned. */
int wq_dequant_mxfp4(const uint32_t* qpacked, const uint8_t* e8, int64_t N, int64_t K, int out_dtype,
                     void* W_hat, void* stream);

/* Workspace bytes for wq_gemm_mxfp4 / _ex (either kernel family).  Host-only. */
size_t wq_gemm_mxfp4_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* y = x * What^T with MXFP4 weights decoded inside the kernel: the GEMV
 * (WQ_PATH_AUTO rule) has the matrix cores sum exact E2M1 values times x per
 * block in fp32 and applies the block's power of two in fp32 (exact for every
 * e8); the MFMA GEMM (larger M) takes fp16
 * operands fp16(E2M1 * 2^(e8 - 127)), exact while the block exponent lies in
 * [-23, 13] (outside, the operand rounds to fp16's range).  Arguments,
 * workspace contract and errors as wq_gemm_w4a16 with e8 for the scales and no
 * zero-points. */
int wq_gemm_mxfp4(int64_t M, int64_t N, int64_t K, const uint16_t* x_f16, const uint32_t* qpacked,
                  const uint8_t* e8, uint16_t* y_f16, void* workspace, size_t workspace_bytes, void* stream);

/* As wq_gemm_mxfp4, with the kernel family chosen by `path` (wq_path). */
int wq_gemm_mxfp4_ex(int64_t M, int64_t N, int64_t K, const uint16_t* x_f16, const uint32_t* qpacked,
                     const uint8_t* e8, uint16_t* y_f16, void* workspace, size_t workspace_bytes, int path,
                     void* stream);

/* As wq_gemm_plan, for wq_gemm_mxfp4_ex. */
int wq_gemm_mxfp4_plan(int64_t M, int64_t N, int64_t K, int path, char* buf, size_t buf_len);

/* ---- NVFP4 weights ----------------------------------------------------------
 * "Quantization Methods Compared: INT8, GPTQ, AWQ, FP8, FP4 and KV-Cache
 * Quantization", section "Hardware, formats and the roofline" (its key box):
 * 4-bit values with one FP8 E4M3 scale per 16 values plus one fp32 scale per
 * tensor, 4.5 bits per value; "Quantization for LLM inference", section
 * "Microscaling: NVFP4 and MXFP4".  Elements are E2M1 as in MXFP4; E4M3 has 4
 * exponent bits (bias 7) and 3 mantissa bits, largest finite value 448.  The
 * pages leave the two scales' choice open; read as:
 *   S = fp32(fp64(max|W| / (6 * 448))) over the whole tensor (1 when all zero);
 *   s8 = the E4M3 value nearest to the block's max|w| / (6 S), ties to even,
 *   saturating at 448;
 *   code = the E2M1 value nearest to w / (E4M3(s8) * S), ties to even,
 *   saturating at 6, sign in bit 3; a block with s8 = 0 stores codes 0;
 *   What = fp32(E2M1(code) * E4M3(s8) * S) (one rounding).
 * Layouts: q_codes [N][K] uint8; s8 [N][K/16]; qpacked the MXFP4 tiles
 * (wq_pack_mxfp4 packs codes); tensor_scale one fp32 in device memory.  K a
 * multiple of 32 (WQ_EUNSUPPORTED otherwise).  Input weights must be finite
 * (a non-finite weight gives unspecified codes). */

/* Byte sizes of qpacked and s8 for [N][K].  Host-only. */
int wq_layout_bytes_nvfp4(int64_t N, int64_t K, size_t* qpacked_bytes, size_t* s8_bytes);

/* NVFP4 quantization of W [N][K] (WQ_F32, WQ_BF16 or WQ_F16, 16-byte aligned).
 * tensor_scale (device, 4-byte aligned) receives S and s8 [N][K/16] the block
 * scales (both required); q_codes (8-byte aligned) and qpacked (16-byte
 * aligned) may each be NULL.  Four launches on `stream`: a fill and a
 * reduction for S, then the quantizer.  Deterministic. */
int wq_quantize_nvfp4(const void* W, int w_dtype, int64_t N, int64_t K, uint8_t* q_codes, uint8_t* s8,
                      float* tensor_scale, uint32_t* qpacked, void* stream);

/* What = fp32(E2M1(code) * E4M3(s8) * S) into W_hat [N][K] (WQ_F32; WQ_F16 /
 * WQ_BF16 one round-to-nearest-even of that fp32 value); W_hat 16-byte aligned. */
int wq_dequant_nvfp4(const uint32_t* qpacked, const uint8_t* s8, const float* tensor_scale, int64_t N, int64_t K,
                     int out_dtype, void* W_hat, void* stream);

/* Workspace bytes for wq_gemm_nvfp4 / _ex (either kernel family).  Host-only. */
size_t wq_gemm_nvfp4_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* y = x * What^T with NVFP4 weights decoded inside the kernel.  The tensor
 * scale factors out of every output: y = fp16(S * sum_k x * E2M1 * E4M3), the
 * GEMV and the MFMA GEMM both giving the matrix cores the exact fp16 operands
 * E2M1 * E4M3 (fp32 sums).  Arguments, workspace contract and errors as
 * wq_gemm_w4a16 with s8 for the scales and tensor_scale (device) for S. */
int wq_gemm_nvfp4(int64_t M, int64_t N, int64_t K, const uint16_t* x_f16, const uint32_t* qpacked, const uint8_t* s8,
                  const float* tensor_scale, uint16_t* y_f16, void* workspace, size_t workspace_bytes, void* stream);

/* As wq_gemm_nvfp4, with the kernel family chosen by `path` (wq_path). */
int wq_gemm_nvfp4_ex(int64_t M, int64_t N, int64_t K, const uint16_t* x_f16, const uint32_t* qpacked,
                     const uint8_t* s8, const float* tensor_scale, uint16_t* y_f16, void* workspace,
                     size_t workspace_bytes, int path, void* stream);

/* As wq_gemm_plan, for wq_gemm_nvfp4_ex. */
int wq_gemm_nvfp4_plan(int64_t M, int64_t N, int64_t K, int path, char* buf, size_t buf_len);

/* ---- INT4 KV cache in blocks of 128 -----------------------------------------
 * "Quantization for LLM inference", section "KV cache quantization": the K/V
 * cache stored as int4 in blocks of 128 values (half a byte per value plus
 * the scale overhead).  Read as: each token's K (or V) vector of hd values
 * (all KV heads of one layer, hd a multiple of 128) is cut into hd/128 blocks
 * of 128 consecutive values, and each block is quantized exactly like one
 * weight group of 128 (wq_quantize_groups' numerics: fp16 scale, 4-bit
 * zero-point, 4-bit codes).  A cache of S rows (token slots) holds per row:
 *   codes   hd/2 bytes; block b at byte 64*b, as 16 little-endian 32-bit words,
 *           word j holding values 8j + e (e = 0..7) of the block, value e in
 *           nibble 4*(e%2) + e/2 (the word format of the weight tiles)
 *   s_f16   hd/128 fp16 scales
 *   zpacked ceil(hd/256) bytes, block b's zero-point in the low nibble of
 *           byte b/2 when b is even, in the high nibble when b is odd (an odd
 *           block count leaves the last high nibble 0)
 * so 0.5 + 2.5/128 bytes per value (3.85x smaller than an fp16 cache).  Arrays
 * are row-major [S][...]; device memory, caller-owned. */

/* Byte sizes of the three cache arrays for S rows of hd values.  Host-only.
 * WQ_EUNSUPPORTED when hd is not a multiple of 128. */
int wq_kv_layout_bytes(int64_t S, int64_t hd, size_t* codes_bytes, size_t* s_bytes, size_t* z_bytes);

/* Quantizes X [T][hd] (x_dtype WQ_F32, WQ_BF16 or WQ_F16; 16-byte aligned)
 * token by token into cache row slot[t] (slot: device int32 [T], 4-byte
 * aligned, or NULL for rows 0..T-1).  Tokens whose slot lies outside [0, S)
 * are skipped; rows not named keep their contents; two tokens naming the same
 * row in one call leave either token's values there.  codes 8-byte aligned.
 * Preconditions as wq_quantize_groups (finite values, block range below
 * 15 * 65520).  Deterministic. */
int wq_kv_quantize(const void* X, int x_dtype, int64_t T, int64_t hd, const int32_t* slot, int64_t S,
                   uint8_t* codes, uint16_t* s_f16, uint8_t* zpacked, void* stream);

/* Decodes cache rows slot[t] (NULL: rows 0..T-1) into out [T][hd] as out_dtype
 * (WQ_F32 exact s * (q - z); WQ_F16 / WQ_BF16 one round-to-nearest-even of it);
 * tokens whose slot lies outside [0, S) decode to zeros.  out 16-byte
 * aligned. */
int wq_kv_dequant(const uint8_t* codes, const uint16_t* s_f16, const uint8_t* zpacked, int64_t T, int64_t hd,
                  const int32_t* slot, int64_t S, int out_dtype, void* out, void* stream);

/* ---- Streaming-read probe (a measurement aid, not a step of the method) -----
 * A decode product's time is the reading of its weights ("Hardware, formats
 * and the roofline": decode is bound by memory bandwidth), so the rate at which
 * this GPU reads the same number of bytes once is that product's ceiling on
 * this part, next to the nominal HBM peak.  Issues `count` kernel launches
 * back to back on `stream`; launch i reads the window_bytes bytes at
 * src + (i mod (span_bytes / window_bytes)) * window_bytes, once, with
 * `chunks` (1, 2, 4, 8 or 16) 16-byte loads per thread, plain (nontemporal
 * 0) or with the non-temporal streaming hint (1), and writes nothing to
 * memory except, if the XOR of one thread's words equals a fixed 32-bit value,
 * that value to *sink.  Rotating over a span larger than the last-level cache
 * keeps every launch reading from HBM.
 *   src     device memory, 16-byte aligned, span_bytes readable
 *   window_bytes  a positive multiple of 256, at most span_bytes (and 2^40)
 *   sink    one device word, 4-byte aligned
 * WQ_EINVAL for a NULL pointer, a negative count or a bad size, chunk count
 * or nontemporal flag; WQ_EALIGN for misaligned pointers; count == 0 enqueues nothing. */
int wq_read_probe(const void* src, size_t window_bytes, size_t span_bytes, int count, int chunks,
                  int nontemporal, uint32_t* sink, void* stream);

/* ---- Matrix-core probe (a measurement aid, not a step of the method) --------
 * Past the ridge point the batched product is bound by its matrix-core work
 * ("Hardware, formats and the roofline"), so the rate at which this GPU
 * sustains the fp16 MFMA instruction the product kernels issue
 * (v_mfma_f32_16x16x32_f16, 16,384 FLOP each), with no memory traffic and no
 * other vector work and at the clock the part holds under that load, is that
 * product's ceiling on this part, next to the nominal dense fp16 peak.
 * Issues `count` launches back to back on `stream`, each of `workgroups`
 * workgroups of 256 threads (four waves); every wave issues iters x 8 MFMAs,
 * so one launch performs workgroups * 4 * iters * 8 * 16384 FLOP.  Writes
 * nothing to memory except, on one fixed result, a word to *sink.
 *   sink    one device word, 4-byte aligned
 * WQ_EINVAL for a NULL sink or a non-positive size (count == 0 enqueues
 * nothing), WQ_EALIGN for a misaligned sink. */
int wq_mfma_probe(int workgroups, int iters, int count, uint32_t* sink, void* stream);

/* ---- Clock probe (a measurement aid) ----------------------------------------
 * The matrix-core and read ceilings above depend on the core clock the part
 * holds under load, so timed regions are paired with a reading of it: one
 * launch of `workgroups` workgroups of one wave, each spinning for `ticks`
 * ticks of the constant 100 MHz real-time counter (s_memrealtime) and writing
 * how far the shader clock counter (s_memtime) and the real-time counter
 * advanced: out[2b] and out[2b + 1] for workgroup b (device memory, 8-byte
 * aligned, 2 * workgroups entries).  Core clock = 100 MHz * out[2b] / out[2b+1].
 * The spin also ends after a fixed number of counter reads.
 * WQ_EINVAL for a NULL out, workgroups outside 1..65536 or ticks outside
 * 1..10^7; WQ_EALIGN for a misaligned out. */
int wq_clock_probe(int workgroups, uint32_t ticks, unsigned long long* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBWQ_H */
