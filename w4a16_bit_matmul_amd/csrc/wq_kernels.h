// Launch entry points of the libwq kernels (host side of each .hip file).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace wq {

// Raises a kernel's dynamic LDS limit to `lds` bytes (needed above 64 KiB)
// once per device: the attribute stays with the function on that device, so
// later launches skip the runtime call.  `done` is the kernel instance's own
// set of devices already raised (one bit per device; devices past 63 raise it
// on every launch).
inline hipError_t raise_lds_limit(const void* kernel, size_t lds, std::atomic<uint64_t>& done) {
  if (lds <= 65536) return hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? uint64_t(1) << dev : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return e;
}

// sym: the symmetric 4-bit scheme (codes q + 8, zero-point 8) instead of the
// asymmetric one.  alpha (fp32 [K] or NULL): per-input-channel factors applied
// to the weights before quantizing (the AWQ fold).
hipError_t launch_quantize(const void* W, int dtype, int64_t N, int64_t K, int group, int sym, const float* alpha,
                           uint8_t* q_codes, uint16_t* s, uint8_t* z_codes, uint32_t* qpacked, uint8_t* zpacked,
                           hipStream_t stream);

// The activation side of the AWQ fold, x' = fp16(x / alpha[k]) (K a multiple
// of 8), and the per-channel mean |x| (fp32, row order) that finds salient
// channels.
hipError_t launch_scale_activations(const uint16_t* x, int64_t M, int64_t K, const float* alpha, uint16_t* out,
                                    hipStream_t stream);
hipError_t launch_channel_absmean(const uint16_t* x, int64_t M, int64_t K, float* out, hipStream_t stream);

hipError_t launch_pack(const uint8_t* q_codes, const uint8_t* z_codes, int64_t N, int64_t K, int group,
                       uint32_t* qpacked, uint8_t* zpacked, hipStream_t stream);

hipError_t launch_dequant(const uint32_t* qpacked, const uint16_t* s, const uint8_t* zpacked, int64_t N, int64_t K,
                          int group, int out_dtype, void* out, hipStream_t stream);

// Group absmax int8: codes [N][K] int8 (or NULL), scales [N][G], 2048-byte
// tiles (or NULL).
hipError_t launch_quantize_w8(const void* W, int dtype, int64_t N, int64_t K, int group, int8_t* q_codes,
                              uint16_t* s, uint8_t* qpacked, hipStream_t stream);
hipError_t launch_pack_w8(const int8_t* q_codes, int64_t N, int64_t K, uint8_t* qpacked, hipStream_t stream);
hipError_t launch_dequant_w8(const uint8_t* qpacked, const uint16_t* s, int64_t N, int64_t K, int group,
                             int out_dtype, void* out, hipStream_t stream);

// MXFP4: E2M1 codes [N][K] (or NULL), E8M0 scale bytes [N][K/32], 1 KB tiles
// with natural nibble order (or NULL).
hipError_t launch_quantize_mxfp4(const void* W, int dtype, int64_t N, int64_t K, uint8_t* q_codes, uint8_t* e8,
                                 uint8_t* qpacked, hipStream_t stream);
hipError_t launch_pack_mxfp4(const uint8_t* q_codes, int64_t N, int64_t K, uint8_t* qpacked, hipStream_t stream);
hipError_t launch_dequant_mxfp4(const uint8_t* qpacked, const uint8_t* e8, int64_t N, int64_t K, int out_dtype,
                                void* out, hipStream_t stream);

// NVFP4: the per-tensor fp32 scale (device, written by the quantizer), E2M1
// codes [N][K] (or NULL), E4M3 scale bytes [N][K/16], 1 KB tiles in the MXFP4
// layout (or NULL).  K a multiple of 32.
hipError_t launch_quantize_nvfp4(const void* W, int dtype, int64_t N, int64_t K, float* tensor_scale, uint8_t* q_codes,
                                 uint8_t* s8, uint8_t* qpacked, hipStream_t stream);
hipError_t launch_dequant_nvfp4(const uint8_t* qpacked, const uint8_t* s8, const float* tensor_scale, int64_t N,
                                int64_t K, int out_dtype, void* out, hipStream_t stream);

// INT4 KV cache in blocks of 128: token t's hd values (X [T][hd]) into cache
// row slot[t] (slot NULL: row t; rows outside [0, S) skipped), and back.
hipError_t launch_kv_quantize(const void* X, int dtype, int64_t T, int64_t hd, const int32_t* slot, int64_t S,
                              uint8_t* codes, uint16_t* s, uint8_t* zp, hipStream_t stream);
hipError_t launch_kv_dequant(const uint8_t* codes, const uint16_t* s, const uint8_t* zp, int64_t T, int64_t hd,
                             const int32_t* slot, int64_t S, int out_dtype, void* out, hipStream_t stream);

// Split-K GEMV for small M (dot products on the matrix cores).  It needs a workspace (a counter region that
// is zero on entry and left zero, then fp32 partial sums) only when it splits K
// across workgroups; gemv_workspace_bytes gives the size (0 otherwise).
size_t gemv_workspace_bytes(int64_t M, int64_t N, int64_t K, int group, int fmt);
// Writes a one-line description of the kernel and launch shape chosen for this
// problem (snprintf semantics).  fmt (wq_device.h): kFmtInt4 (tile codes +
// zero-points), kFmtInt8 (2048-byte int8 tiles; zpacked unused) or kFmtMxfp4
// (E2M1 tiles; zpacked holds the E8M0 scale bytes, s unused, group 32).
// kFmtNvfp4: zpacked holds the E4M3 scale bytes, tscale the per-tensor fp32
// scale (device), group 16.
int describe_gemv(int64_t M, int64_t N, int64_t K, int group, int fmt, char* buf, size_t len);
hipError_t launch_gemv(int64_t M, int64_t N, int64_t K, int group, int fmt, const uint16_t* x,
                       const void* qpacked, const uint16_t* s, const uint8_t* zpacked, uint16_t* y, void* workspace,
                       hipStream_t stream, const float* tscale = nullptr);

// MFMA tile GEMM.  Workspace layout and size come from gemm_workspace_bytes.
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int group);
int describe_gemm(int64_t M, int64_t N, int64_t K, int group, int fmt, char* buf, size_t len);
hipError_t launch_gemm(int64_t M, int64_t N, int64_t K, int group, int fmt, const uint16_t* x, const void* qpacked,
                       const uint16_t* s, const uint8_t* zpacked, uint16_t* y, void* workspace, hipStream_t stream,
                       const float* tscale = nullptr);

// Streaming-read probe: count launches back to back, launch i reading the
// window_bytes at src + (i mod (span_bytes / window_bytes)) * window_bytes once,
// with chunks (1, 2, 4, 8 or 16) 16-byte loads per thread, plain or
// non-temporal.  sink: one device word, written only if a thread's XOR of its
// words hits a fixed value.
hipError_t launch_read_probe(const void* src, size_t window_bytes, size_t span_bytes, int count, int chunks,
                             int nontemporal, uint32_t* sink, hipStream_t stream);

// Matrix-core probe: count launches of `workgroups` workgroups of four waves,
// each wave issuing iters x 8 v_mfma_f32_16x16x32_f16 on register operands
// (16,384 FLOP each).  sink: one device word, written only on a fixed result.
hipError_t launch_mfma_probe(int workgroups, int iters, int count, uint32_t* sink, hipStream_t stream);

// Clock probe: `workgroups` workgroups of one wave spin for `ticks` ticks of
// the 100 MHz real-time counter; workgroup b writes the shader clock counter's
// and the real-time counter's advance to out[2b], out[2b + 1].
hipError_t launch_clock_probe(int workgroups, uint32_t ticks, unsigned long long* out, hipStream_t stream);

}  // namespace wq
