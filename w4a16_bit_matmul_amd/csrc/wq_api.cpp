// libwq C ABI: argument validation (host only, before anything is enqueued),
// kernel selection and launch.  Declarations and the contract of every entry
// point are in include/libwq.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/libwq.h"
#include "wq_device.h"
#include "wq_kernels.h"

static_assert(wq::kSplitCounterBytes == WQ_WORKSPACE_COUNTER_BYTES, "split-K counter region size");

// Kernel family for a product of code format fmt (wq_device.h): the
// WQ_PATH_AUTO rule of libwq.h.  The GEMV takes its dot products on the matrix
// cores at a cost nearly flat in M up to its 8- or 16-row activation tile, and
// hands over to the MFMA tile GEMM where re-reading the weights per activation
// tile costs more than the GEMM's staging.  Narrow outputs give the GEMM's
// 128-column workgroups too few to fill the chip, so the GEMV keeps more rows
// there.
static bool auto_mfma(int64_t M, int64_t N, int64_t K, int group, int fmt, int path) {
  if (path != WQ_PATH_AUTO) return path == WQ_PATH_MFMA;
  if (M <= WQ_AUTO_NARROW_GEMV_MAX_M && N <= WQ_AUTO_GEMV_MAX_N) return false;
  if (fmt == wq::kFmtInt4)
    return M > (group == 32 && K > WQ_AUTO_INT4_G32_LONG_K ? WQ_AUTO_INT4_G32_LONG_K_GEMV_MAX_M
                                                           : WQ_AUTO_INT4_GEMV_MAX_M);
  if (fmt == wq::kFmtMxfp4 || fmt == wq::kFmtNvfp4) return M > WQ_AUTO_FP4_GEMV_MAX_M;
  return M > WQ_AUTO_INT8_GEMV_MAX_M;
}

namespace {

constexpr int kVersion = 100;  // 0.1.0

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_shape(int64_t N, int64_t K, int group) {
  if (N <= 0 || K <= 0) return WQ_EINVAL;
  if (group != 32 && group != 128) return WQ_EUNSUPPORTED;
  if (K % group != 0) return WQ_EUNSUPPORTED;
  // int32 grid dimensions and tile counts stay far below these limits
  if (N > (int64_t(1) << 31) || K > (int64_t(1) << 31)) return WQ_EINVAL;
  return WQ_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? WQ_OK : WQ_EHIP; }

}  // namespace

extern "C" {

int wq_version(void) { return kVersion; }

const char* wq_strerror(int status) {
  switch (status) {
    case WQ_OK: return "success";
    case WQ_EINVAL: return "invalid argument (null pointer, non-positive size, bad dtype, path or scheme)";
    case WQ_EUNSUPPORTED: return "unsupported shape (group must be 32 or 128 and divide K)";
    case WQ_EALIGN: return "pointer not aligned as required";
    case WQ_EWORKSPACE: return "workspace missing or too small";
    case WQ_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int wq_layout_bytes(int64_t N, int64_t K, int group, size_t* qpacked_bytes, size_t* s_bytes, size_t* zpacked_bytes) {
  int st = check_shape(N, K, group);
  if (st) return st;
  const int64_t Np = (N + 15) / 16 * 16, Kp = (K + 127) / 128 * 128, G = K / group;
  if (qpacked_bytes) *qpacked_bytes = (size_t)(Np * Kp / 2);
  if (s_bytes) *s_bytes = (size_t)(N * G * 2);
  if (zpacked_bytes) *zpacked_bytes = (size_t)(N * ((G + 1) / 2));
  return WQ_OK;
}

int wq_quantize_groups_scaled(const void* W, int w_dtype, int64_t N, int64_t K, int group, int scheme,
                              const float* alpha, uint8_t* q_codes, uint16_t* s_f16, uint8_t* z_codes,
                              uint32_t* qpacked, uint8_t* zpacked, void* stream) {
  if (!W || !s_f16) return WQ_EINVAL;
  if (w_dtype != WQ_F32 && w_dtype != WQ_BF16 && w_dtype != WQ_F16) return WQ_EINVAL;
  if (scheme != WQ_ASYM && scheme != WQ_SYM) return WQ_EINVAL;
  int st = check_shape(N, K, group);
  if (st) return st;
  if (!aligned(W, 16) || !aligned(s_f16, 2) || (qpacked && !aligned(qpacked, 16)) || (q_codes && !aligned(q_codes, 8)) ||
      (alpha && !aligned(alpha, 16)))
    return WQ_EALIGN;
  return hip_status(wq::launch_quantize(W, w_dtype, N, K, group, scheme == WQ_SYM, alpha, q_codes, s_f16, z_codes,
                                        qpacked, zpacked, static_cast<hipStream_t>(stream)));
}

int wq_quantize_groups_ex(const void* W, int w_dtype, int64_t N, int64_t K, int group, int scheme,
                          uint8_t* q_codes, uint16_t* s_f16, uint8_t* z_codes, uint32_t* qpacked, uint8_t* zpacked,
                          void* stream) {
  return wq_quantize_groups_scaled(W, w_dtype, N, K, group, scheme, nullptr, q_codes, s_f16, z_codes, qpacked,
                                   zpacked, stream);
}

int wq_scale_activations(const uint16_t* x_f16, int64_t M, int64_t K, const float* alpha, uint16_t* x_out_f16,
                         void* stream) {
  if (!x_f16 || !alpha || !x_out_f16) return WQ_EINVAL;
  if (M <= 0 || K <= 0 || M > (int64_t(1) << 31) || K > (int64_t(1) << 31)) return WQ_EINVAL;
  if (K % 8 != 0) return WQ_EUNSUPPORTED;
  if (!aligned(x_f16, 16) || !aligned(alpha, 16) || !aligned(x_out_f16, 16)) return WQ_EALIGN;
  return hip_status(wq::launch_scale_activations(x_f16, M, K, alpha, x_out_f16, static_cast<hipStream_t>(stream)));
}

int wq_channel_absmean(const uint16_t* x_f16, int64_t M, int64_t K, float* out, void* stream) {
  if (!x_f16 || !out) return WQ_EINVAL;
  if (M <= 0 || K <= 0 || M > (int64_t(1) << 31) || K > (int64_t(1) << 31)) return WQ_EINVAL;
  if (!aligned(x_f16, 2) || !aligned(out, 4)) return WQ_EALIGN;
  return hip_status(wq::launch_channel_absmean(x_f16, M, K, out, static_cast<hipStream_t>(stream)));
}

int wq_quantize_groups(const void* W, int w_dtype, int64_t N, int64_t K, int group, uint8_t* q_codes,
                       uint16_t* s_f16, uint8_t* z_codes, uint32_t* qpacked, uint8_t* zpacked, void* stream) {
  return wq_quantize_groups_ex(W, w_dtype, N, K, group, WQ_ASYM, q_codes, s_f16, z_codes, qpacked, zpacked, stream);
}

int wq_pack_int4(const uint8_t* q_codes, const uint8_t* z_codes, int64_t N, int64_t K, int group, uint32_t* qpacked,
                 uint8_t* zpacked, void* stream) {
  if (!q_codes || !z_codes || !qpacked || !zpacked) return WQ_EINVAL;
  int st = check_shape(N, K, group);
  if (st) return st;
  if (!aligned(q_codes, 8) || !aligned(qpacked, 16)) return WQ_EALIGN;
  return hip_status(
      wq::launch_pack(q_codes, z_codes, N, K, group, qpacked, zpacked, static_cast<hipStream_t>(stream)));
}

int wq_dequant(const uint32_t* qpacked, const uint16_t* s_f16, const uint8_t* zpacked, int64_t N, int64_t K,
               int group, int out_dtype, void* W_hat, void* stream) {
  if (!qpacked || !s_f16 || !zpacked || !W_hat) return WQ_EINVAL;
  if (out_dtype != WQ_F32 && out_dtype != WQ_BF16 && out_dtype != WQ_F16) return WQ_EINVAL;
  int st = check_shape(N, K, group);
  if (st) return st;
  if (!aligned(qpacked, 16) || !aligned(s_f16, 2) || !aligned(W_hat, 16)) return WQ_EALIGN;
  return hip_status(wq::launch_dequant(qpacked, s_f16, zpacked, N, K, group, out_dtype, W_hat,
                                       static_cast<hipStream_t>(stream)));
}

size_t wq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int group) {
  if (M <= 0 || M > (int64_t(1) << 31) || check_shape(N, K, group)) return 0;
  const size_t a = wq::gemv_workspace_bytes(M, N, K, group, wq::kFmtInt4), b = wq::gemm_workspace_bytes(M, N, K, group);
  return a > b ? a : b;
}

size_t wq_gemm_workspace_bytes_ex(int64_t M, int64_t N, int64_t K, int group, int path) {
  if (M <= 0 || M > (int64_t(1) << 31) || check_shape(N, K, group)) return 0;
  if (path != WQ_PATH_AUTO && path != WQ_PATH_GEMV && path != WQ_PATH_MFMA) return 0;
  const bool mfma = auto_mfma(M, N, K, group, wq::kFmtInt4, path);
  return mfma ? wq::gemm_workspace_bytes(M, N, K, group) : wq::gemv_workspace_bytes(M, N, K, group, wq::kFmtInt4);
}

int wq_gemm_plan(int64_t M, int64_t N, int64_t K, int group, int path, char* buf, size_t buf_len) {
  if (!buf || buf_len == 0) return WQ_EINVAL;
  buf[0] = 0;
  if (M <= 0 || M > (int64_t(1) << 31)) return WQ_EINVAL;
  if (path != WQ_PATH_AUTO && path != WQ_PATH_GEMV && path != WQ_PATH_MFMA) return WQ_EINVAL;
  int st = check_shape(N, K, group);
  if (st) return st;
  const bool mfma = auto_mfma(M, N, K, group, wq::kFmtInt4, path);
  if (mfma)
    wq::describe_gemm(M, N, K, group, 4, buf, buf_len);
  else
    wq::describe_gemv(M, N, K, group, 4, buf, buf_len);
  return WQ_OK;
}

namespace {

// Argument checks of one product (host only); 0 or a wq_status.  fmt: the code
// format (wq_device.h); int8 takes no zero-points, MXFP4 takes its scale
// bytes in zpacked and no fp16 scales.
int check_gemm(int64_t M, int64_t N, int64_t K, int group, int fmt, const uint16_t* x_f16, const void* qpacked,
               const uint16_t* s_f16, const uint8_t* zpacked, const uint16_t* y_f16, const void* workspace,
               size_t workspace_bytes, int path, bool* mfma) {
  const bool fp16_scales = fmt == wq::kFmtInt4 || fmt == wq::kFmtInt8;
  if (!x_f16 || !qpacked || (fp16_scales && !s_f16) || (fmt != wq::kFmtInt8 && !zpacked) || !y_f16)
    return WQ_EINVAL;
  if (M <= 0 || M > (int64_t(1) << 31)) return WQ_EINVAL;
  if (path != WQ_PATH_AUTO && path != WQ_PATH_GEMV && path != WQ_PATH_MFMA) return WQ_EINVAL;
  int st = check_shape(N, K, fmt == wq::kFmtNvfp4 ? 32 : group);  // NVFP4: blocks of 16, K a multiple of 32
  if (st) return st;
  if (!aligned(x_f16, 16) || !aligned(qpacked, 16) || !aligned(s_f16, 2) || !aligned(y_f16, 2)) return WQ_EALIGN;
  *mfma = auto_mfma(M, N, K, group, fmt, path);
  const size_t need = *mfma ? wq::gemm_workspace_bytes(M, N, K, group) : wq::gemv_workspace_bytes(M, N, K, group, fmt);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return WQ_EWORKSPACE;
    if (!aligned(workspace, 256)) return WQ_EALIGN;
  }
  return WQ_OK;
}

hipError_t launch_one(bool mfma, int64_t M, int64_t N, int64_t K, int group, int bits, const uint16_t* x_f16,
                      const void* qpacked, const uint16_t* s_f16, const uint8_t* zpacked, uint16_t* y_f16,
                      void* workspace, hipStream_t s, const float* tscale = nullptr) {
  if (!mfma) return wq::launch_gemv(M, N, K, group, bits, x_f16, qpacked, s_f16, zpacked, y_f16, workspace, s, tscale);
  return wq::launch_gemm(M, N, K, group, bits, x_f16, qpacked, s_f16, zpacked, y_f16, workspace, s, tscale);
}

}  // namespace

int wq_gemm_w4a16_ex(int64_t M, int64_t N, int64_t K, int group, const uint16_t* x_f16, const uint32_t* qpacked,
                     const uint16_t* s_f16, const uint8_t* zpacked, uint16_t* y_f16, void* workspace,
                     size_t workspace_bytes, int path, void* stream) {
  bool mfma = false;
  const int st = check_gemm(M, N, K, group, 4, x_f16, qpacked, s_f16, zpacked, y_f16, workspace, workspace_bytes,
                            path, &mfma);
  if (st) return st;
  return hip_status(launch_one(mfma, M, N, K, group, 4, x_f16, qpacked, s_f16, zpacked, y_f16, workspace,
                               static_cast<hipStream_t>(stream)));
}

int wq_gemm_w4a16_seq(int count, int64_t M, int64_t N, int64_t K, int group, const uint16_t* const* x_f16,
                      const uint32_t* const* qpacked, const uint16_t* const* s_f16, const uint8_t* const* zpacked,
                      uint16_t* const* y_f16, void* workspace, size_t workspace_bytes, void* stream) {
  if (count < 0 || (count > 0 && (!x_f16 || !qpacked || !s_f16 || !zpacked || !y_f16))) return WQ_EINVAL;
  bool mfma = false;
  for (int i = 0; i < count; ++i) {
    const int st = check_gemm(M, N, K, group, 4, x_f16[i], qpacked[i], s_f16[i], zpacked[i], y_f16[i], workspace,
                              workspace_bytes, WQ_PATH_AUTO, &mfma);
    if (st) return st;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int i = 0; i < count; ++i) {
    const hipError_t e = launch_one(mfma, M, N, K, group, 4, x_f16[i], qpacked[i], s_f16[i], zpacked[i], y_f16[i],
                                    workspace, s);
    if (e != hipSuccess) return WQ_EHIP;
  }
  return WQ_OK;
}

int wq_gemm_w4a16(int64_t M, int64_t N, int64_t K, int group, const uint16_t* x_f16, const uint32_t* qpacked,
                  const uint16_t* s_f16, const uint8_t* zpacked, uint16_t* y_f16, void* workspace,
                  size_t workspace_bytes, void* stream) {
  return wq_gemm_w4a16_ex(M, N, K, group, x_f16, qpacked, s_f16, zpacked, y_f16, workspace, workspace_bytes,
                          WQ_PATH_AUTO, stream);
}

// ---- group absmax int8 (W8A16) ---------------------------------------------

int wq_layout_bytes_w8(int64_t N, int64_t K, int group, size_t* qpacked_bytes, size_t* s_bytes) {
  int st = check_shape(N, K, group);
  if (st) return st;
  const int64_t Np = (N + 15) / 16 * 16, Kp = (K + 127) / 128 * 128;
  if (qpacked_bytes) *qpacked_bytes = (size_t)(Np * Kp);
  if (s_bytes) *s_bytes = (size_t)(N * (K / group) * 2);
  return WQ_OK;
}

int wq_quantize_w8(const void* W, int w_dtype, int64_t N, int64_t K, int group, int8_t* q_codes, uint16_t* s_f16,
                   uint8_t* qpacked, void* stream) {
  if (!W || !s_f16) return WQ_EINVAL;
  if (w_dtype != WQ_F32 && w_dtype != WQ_BF16 && w_dtype != WQ_F16) return WQ_EINVAL;
  int st = check_shape(N, K, group);
  if (st) return st;
  if (!aligned(W, 16) || !aligned(s_f16, 2) || (qpacked && !aligned(qpacked, 16)) || (q_codes && !aligned(q_codes, 8)))
    return WQ_EALIGN;
  return hip_status(
      wq::launch_quantize_w8(W, w_dtype, N, K, group, q_codes, s_f16, qpacked, static_cast<hipStream_t>(stream)));
}

int wq_pack_int8(const int8_t* q_codes, int64_t N, int64_t K, uint8_t* qpacked, void* stream) {
  if (!q_codes || !qpacked) return WQ_EINVAL;
  if (N <= 0 || K <= 0 || N > (int64_t(1) << 31) || K > (int64_t(1) << 31)) return WQ_EINVAL;
  if (K % 32 != 0) return WQ_EUNSUPPORTED;
  if (!aligned(q_codes, 8) || !aligned(qpacked, 16)) return WQ_EALIGN;
  return hip_status(wq::launch_pack_w8(q_codes, N, K, qpacked, static_cast<hipStream_t>(stream)));
}

int wq_dequant_w8(const uint8_t* qpacked, const uint16_t* s_f16, int64_t N, int64_t K, int group, int out_dtype,
                  void* W_hat, void* stream) {
  if (!qpacked || !s_f16 || !W_hat) return WQ_EINVAL;
  if (out_dtype != WQ_F32 && out_dtype != WQ_BF16 && out_dtype != WQ_F16) return WQ_EINVAL;
  int st = check_shape(N, K, group);
  if (st) return st;
  if (!aligned(qpacked, 16) || !aligned(s_f16, 2) || !aligned(W_hat, 16)) return WQ_EALIGN;
  return hip_status(
      wq::launch_dequant_w8(qpacked, s_f16, N, K, group, out_dtype, W_hat, static_cast<hipStream_t>(stream)));
}

size_t wq_gemm_w8a16_workspace_bytes(int64_t M, int64_t N, int64_t K, int group) {
  if (M <= 0 || M > (int64_t(1) << 31) || check_shape(N, K, group)) return 0;
  // the int8 GEMV may split K differently from the 4-bit one
  const size_t a = wq::gemv_workspace_bytes(M, N, K, group, wq::kFmtInt8), b = wq::gemm_workspace_bytes(M, N, K, group);
  return a > b ? a : b;
}

int wq_gemm_w8a16_ex(int64_t M, int64_t N, int64_t K, int group, const uint16_t* x_f16, const uint8_t* qpacked,
                     const uint16_t* s_f16, uint16_t* y_f16, void* workspace, size_t workspace_bytes, int path,
                     void* stream) {
  bool mfma = false;
  const int st = check_gemm(M, N, K, group, 8, x_f16, qpacked, s_f16, nullptr, y_f16, workspace, workspace_bytes,
                            path, &mfma);
  if (st) return st;
  return hip_status(launch_one(mfma, M, N, K, group, 8, x_f16, qpacked, s_f16, nullptr, y_f16, workspace,
                               static_cast<hipStream_t>(stream)));
}

int wq_gemm_w8a16(int64_t M, int64_t N, int64_t K, int group, const uint16_t* x_f16, const uint8_t* qpacked,
                  const uint16_t* s_f16, uint16_t* y_f16, void* workspace, size_t workspace_bytes, void* stream) {
  return wq_gemm_w8a16_ex(M, N, K, group, x_f16, qpacked, s_f16, y_f16, workspace, workspace_bytes, WQ_PATH_AUTO,
                          stream);
}

int wq_gemm_w8a16_plan(int64_t M, int64_t N, int64_t K, int group, int path, char* buf, size_t buf_len) {
  if (!buf || buf_len == 0) return WQ_EINVAL;
  buf[0] = 0;
  if (M <= 0 || M > (int64_t(1) << 31)) return WQ_EINVAL;
  if (path != WQ_PATH_AUTO && path != WQ_PATH_GEMV && path != WQ_PATH_MFMA) return WQ_EINVAL;
  int st = check_shape(N, K, group);
  if (st) return st;
  const bool mfma = auto_mfma(M, N, K, group, wq::kFmtInt8, path);
  if (mfma)
    wq::describe_gemm(M, N, K, group, 8, buf, buf_len);
  else
    wq::describe_gemv(M, N, K, group, 8, buf, buf_len);
  return WQ_OK;
}

// ---- INT4 KV cache in blocks of 128 ------------------------------------------

namespace {
int check_kv(int64_t T, int64_t hd, int64_t S) {
  if (T <= 0 || hd <= 0 || S <= 0) return WQ_EINVAL;
  if (hd % 128 != 0) return WQ_EUNSUPPORTED;
  if (T > (int64_t(1) << 31) || S > (int64_t(1) << 31) || hd > (int64_t(1) << 24)) return WQ_EINVAL;
  return WQ_OK;
}
}  // namespace

int wq_kv_layout_bytes(int64_t S, int64_t hd, size_t* codes_bytes, size_t* s_bytes, size_t* z_bytes) {
  const int st = check_kv(1, hd, S);
  if (st) return st;
  const int64_t nb = hd / 128;
  if (codes_bytes) *codes_bytes = (size_t)(S * (hd / 2));
  if (s_bytes) *s_bytes = (size_t)(S * nb * 2);
  if (z_bytes) *z_bytes = (size_t)(S * ((nb + 1) / 2));
  return WQ_OK;
}

int wq_kv_quantize(const void* X, int x_dtype, int64_t T, int64_t hd, const int32_t* slot, int64_t S,
                   uint8_t* codes, uint16_t* s_f16, uint8_t* zpacked, void* stream) {
  if (!X || !codes || !s_f16 || !zpacked) return WQ_EINVAL;
  if (x_dtype != WQ_F32 && x_dtype != WQ_BF16 && x_dtype != WQ_F16) return WQ_EINVAL;
  const int st = check_kv(T, hd, S);
  if (st) return st;
  if (!aligned(X, 16) || !aligned(codes, 8) || !aligned(s_f16, 2) || (slot && !aligned(slot, 4))) return WQ_EALIGN;
  return hip_status(
      wq::launch_kv_quantize(X, x_dtype, T, hd, slot, S, codes, s_f16, zpacked, static_cast<hipStream_t>(stream)));
}

int wq_kv_dequant(const uint8_t* codes, const uint16_t* s_f16, const uint8_t* zpacked, int64_t T, int64_t hd,
                  const int32_t* slot, int64_t S, int out_dtype, void* out, void* stream) {
  if (!codes || !s_f16 || !zpacked || !out) return WQ_EINVAL;
  if (out_dtype != WQ_F32 && out_dtype != WQ_BF16 && out_dtype != WQ_F16) return WQ_EINVAL;
  const int st = check_kv(T, hd, S);
  if (st) return st;
  if (!aligned(codes, 8) || !aligned(s_f16, 2) || !aligned(out, 16) || (slot && !aligned(slot, 4))) return WQ_EALIGN;
  return hip_status(wq::launch_kv_dequant(codes, s_f16, zpacked, T, hd, slot, S, out_dtype, out,
                                          static_cast<hipStream_t>(stream)));
}

// ---- MXFP4 (E2M1 codes, blocks of 32, E8M0 scales) ---------------------------

namespace {
int check_mx_shape(int64_t N, int64_t K) { return check_shape(N, K, 32); }
}  // namespace

int wq_layout_bytes_mxfp4(int64_t N, int64_t K, size_t* qpacked_bytes, size_t* e8_bytes) {
  const int st = check_mx_shape(N, K);
  if (st) return st;
  const int64_t Np = (N + 15) / 16 * 16, Kp = (K + 127) / 128 * 128;
  if (qpacked_bytes) *qpacked_bytes = (size_t)(Np * Kp / 2);
  if (e8_bytes) *e8_bytes = (size_t)(N * (K / 32));
  return WQ_OK;
}

int wq_quantize_mxfp4(const void* W, int w_dtype, int64_t N, int64_t K, uint8_t* q_codes, uint8_t* e8,
                      uint32_t* qpacked, void* stream) {
  if (!W || !e8) return WQ_EINVAL;
  if (w_dtype != WQ_F32 && w_dtype != WQ_BF16 && w_dtype != WQ_F16) return WQ_EINVAL;
  const int st = check_mx_shape(N, K);
  if (st) return st;
  if (!aligned(W, 16) || (qpacked && !aligned(qpacked, 16)) || (q_codes && !aligned(q_codes, 8))) return WQ_EALIGN;
  return hip_status(wq::launch_quantize_mxfp4(W, w_dtype, N, K, q_codes, e8, reinterpret_cast<uint8_t*>(qpacked),
                                              static_cast<hipStream_t>(stream)));
}

int wq_pack_mxfp4(const uint8_t* q_codes, int64_t N, int64_t K, uint32_t* qpacked, void* stream) {
  if (!q_codes || !qpacked) return WQ_EINVAL;
  const int st = check_mx_shape(N, K);
  if (st) return st;
  if (!aligned(q_codes, 8) || !aligned(qpacked, 16)) return WQ_EALIGN;
  return hip_status(wq::launch_pack_mxfp4(q_codes, N, K, reinterpret_cast<uint8_t*>(qpacked),
                                          static_cast<hipStream_t>(stream)));
}

int wq_dequant_mxfp4(const uint32_t* qpacked, const uint8_t* e8, int64_t N, int64_t K, int out_dtype, void* W_hat,
                     void* stream) {
  if (!qpacked || !e8 || !W_hat) return WQ_EINVAL;
  if (out_dtype != WQ_F32 && out_dtype != WQ_BF16 && out_dtype != WQ_F16) return WQ_EINVAL;
  const int st = check_mx_shape(N, K);
  if (st) return st;
  if (!aligned(qpacked, 16) || !aligned(W_hat, 16)) return WQ_EALIGN;
  return hip_status(wq::launch_dequant_mxfp4(reinterpret_cast<const uint8_t*>(qpacked), e8, N, K, out_dtype, W_hat,
                                             static_cast<hipStream_t>(stream)));
}

// the larger of the two kernel families' needs, for the format's own GEMV plan
static size_t workspace_fmt(int64_t M, int64_t N, int64_t K, int group, int fmt) {
  if (M <= 0 || M > (int64_t(1) << 31) || check_shape(N, K, 32)) return 0;
  const size_t a = wq::gemv_workspace_bytes(M, N, K, group, fmt), b = wq::gemm_workspace_bytes(M, N, K, group);
  return a > b ? a : b;
}

size_t wq_gemm_mxfp4_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  return workspace_fmt(M, N, K, 32, wq::kFmtMxfp4);
}

int wq_gemm_mxfp4_ex(int64_t M, int64_t N, int64_t K, const uint16_t* x_f16, const uint32_t* qpacked,
                     const uint8_t* e8, uint16_t* y_f16, void* workspace, size_t workspace_bytes, int path,
                     void* stream) {
  bool mfma = false;
  const int st = check_gemm(M, N, K, 32, wq::kFmtMxfp4, x_f16, qpacked, nullptr, e8, y_f16, workspace,
                            workspace_bytes, path, &mfma);
  if (st) return st;
  return hip_status(launch_one(mfma, M, N, K, 32, wq::kFmtMxfp4, x_f16, qpacked, nullptr, e8, y_f16, workspace,
                               static_cast<hipStream_t>(stream)));
}

int wq_gemm_mxfp4(int64_t M, int64_t N, int64_t K, const uint16_t* x_f16, const uint32_t* qpacked, const uint8_t* e8,
                  uint16_t* y_f16, void* workspace, size_t workspace_bytes, void* stream) {
  return wq_gemm_mxfp4_ex(M, N, K, x_f16, qpacked, e8, y_f16, workspace, workspace_bytes, WQ_PATH_AUTO, stream);
}

int wq_gemm_mxfp4_plan(int64_t M, int64_t N, int64_t K, int path, char* buf, size_t buf_len) {
  if (!buf || buf_len == 0) return WQ_EINVAL;
  buf[0] = 0;
  if (M <= 0 || M > (int64_t(1) << 31)) return WQ_EINVAL;
  if (path != WQ_PATH_AUTO && path != WQ_PATH_GEMV && path != WQ_PATH_MFMA) return WQ_EINVAL;
  const int st = check_mx_shape(N, K);
  if (st) return st;
  const bool mfma = auto_mfma(M, N, K, 32, wq::kFmtMxfp4, path);
  if (mfma)
    wq::describe_gemm(M, N, K, 32, wq::kFmtMxfp4, buf, buf_len);
  else
    wq::describe_gemv(M, N, K, 32, wq::kFmtMxfp4, buf, buf_len);
  return WQ_OK;
}


// ---- streaming-read probe (measurement aid) ----------------------------------

int wq_read_probe(const void* src, size_t window_bytes, size_t span_bytes, int count, int chunks, int nontemporal,
                  uint32_t* sink, void* stream) {
  if (!src || !sink || count < 0 || window_bytes == 0 || window_bytes % 256 != 0 || span_bytes < window_bytes ||
      window_bytes > (size_t(1) << 40) || (chunks != 1 && chunks != 2 && chunks != 4 && chunks != 8 && chunks != 16) ||
      (nontemporal != 0 && nontemporal != 1))
    return WQ_EINVAL;
  if (!aligned(src, 16) || !aligned(sink, 4)) return WQ_EALIGN;
  if (count == 0) return WQ_OK;
  return hip_status(wq::launch_read_probe(src, window_bytes, span_bytes, count, chunks, nontemporal, sink,
                                          static_cast<hipStream_t>(stream)));
}

int wq_mfma_probe(int workgroups, int iters, int count, uint32_t* sink, void* stream) {
  if (!sink || workgroups <= 0 || iters <= 0 || count < 0) return WQ_EINVAL;
  if (!aligned(sink, 4)) return WQ_EALIGN;
  if (count == 0) return WQ_OK;
  return hip_status(wq::launch_mfma_probe(workgroups, iters, count, sink, static_cast<hipStream_t>(stream)));
}

int wq_clock_probe(int workgroups, uint32_t ticks, unsigned long long* out, void* stream) {
  if (!out || workgroups <= 0 || workgroups > 65536 || ticks == 0 || ticks > 10000000u) return WQ_EINVAL;
  if (!aligned(out, 8)) return WQ_EALIGN;
  return hip_status(wq::launch_clock_probe(workgroups, ticks, out, static_cast<hipStream_t>(stream)));
}

// ---- NVFP4 --------------------------------------------------------------------

int wq_layout_bytes_nvfp4(int64_t N, int64_t K, size_t* qpacked_bytes, size_t* s8_bytes) {
  const int st = check_mx_shape(N, K);
  if (st) return st;
  const int64_t Np = (N + 15) / 16 * 16, Kp = (K + 127) / 128 * 128;
  if (qpacked_bytes) *qpacked_bytes = (size_t)(Np * Kp / 2);
  if (s8_bytes) *s8_bytes = (size_t)(N * (K / 16));
  return WQ_OK;
}

int wq_quantize_nvfp4(const void* W, int w_dtype, int64_t N, int64_t K, uint8_t* q_codes, uint8_t* s8,
                      float* tensor_scale, uint32_t* qpacked, void* stream) {
  if (!W || !s8 || !tensor_scale) return WQ_EINVAL;
  if (w_dtype != WQ_F32 && w_dtype != WQ_BF16 && w_dtype != WQ_F16) return WQ_EINVAL;
  const int st = check_mx_shape(N, K);
  if (st) return st;
  if (!aligned(W, 16) || !aligned(tensor_scale, 4) || (qpacked && !aligned(qpacked, 16)) ||
      (q_codes && !aligned(q_codes, 8)))
    return WQ_EALIGN;
  return hip_status(wq::launch_quantize_nvfp4(W, w_dtype, N, K, tensor_scale, q_codes, s8,
                                              reinterpret_cast<uint8_t*>(qpacked), static_cast<hipStream_t>(stream)));
}

int wq_dequant_nvfp4(const uint32_t* qpacked, const uint8_t* s8, const float* tensor_scale, int64_t N, int64_t K,
                     int out_dtype, void* W_hat, void* stream) {
  if (!qpacked || !s8 || !tensor_scale || !W_hat) return WQ_EINVAL;
  if (out_dtype != WQ_F32 && out_dtype != WQ_BF16 && out_dtype != WQ_F16) return WQ_EINVAL;
  const int st = check_mx_shape(N, K);
  if (st) return st;
  if (!aligned(qpacked, 16) || !aligned(tensor_scale, 4) || !aligned(W_hat, 16)) return WQ_EALIGN;
  return hip_status(wq::launch_dequant_nvfp4(reinterpret_cast<const uint8_t*>(qpacked), s8, tensor_scale, N, K,
                                             out_dtype, W_hat, static_cast<hipStream_t>(stream)));
}

size_t wq_gemm_nvfp4_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  return workspace_fmt(M, N, K, 16, wq::kFmtNvfp4);
}

int wq_gemm_nvfp4_ex(int64_t M, int64_t N, int64_t K, const uint16_t* x_f16, const uint32_t* qpacked,
                     const uint8_t* s8, const float* tensor_scale, uint16_t* y_f16, void* workspace,
                     size_t workspace_bytes, int path, void* stream) {
  if (!tensor_scale) return WQ_EINVAL;
  bool mfma = false;
  const int st = check_gemm(M, N, K, 16, wq::kFmtNvfp4, x_f16, qpacked, nullptr, s8, y_f16, workspace,
                            workspace_bytes, path, &mfma);
  if (st) return st;
  if (!aligned(tensor_scale, 4)) return WQ_EALIGN;
  return hip_status(launch_one(mfma, M, N, K, 16, wq::kFmtNvfp4, x_f16, qpacked, nullptr, s8, y_f16, workspace,
                               static_cast<hipStream_t>(stream), tensor_scale));
}

int wq_gemm_nvfp4(int64_t M, int64_t N, int64_t K, const uint16_t* x_f16, const uint32_t* qpacked, const uint8_t* s8,
                  const float* tensor_scale, uint16_t* y_f16, void* workspace, size_t workspace_bytes, void* stream) {
  return wq_gemm_nvfp4_ex(M, N, K, x_f16, qpacked, s8, tensor_scale, y_f16, workspace, workspace_bytes, WQ_PATH_AUTO,
                          stream);
}

int wq_gemm_nvfp4_plan(int64_t M, int64_t N, int64_t K, int path, char* buf, size_t buf_len) {
  if (!buf || buf_len == 0) return WQ_EINVAL;
  buf[0] = 0;
  if (M <= 0 || M > (int64_t(1) << 31)) return WQ_EINVAL;
  if (path != WQ_PATH_AUTO && path != WQ_PATH_GEMV && path != WQ_PATH_MFMA) return WQ_EINVAL;
  const int st = check_mx_shape(N, K);
  if (st) return st;
  if (auto_mfma(M, N, K, 16, wq::kFmtNvfp4, path))
    wq::describe_gemm(M, N, K, 16, wq::kFmtNvfp4, buf, buf_len);
  else
    wq::describe_gemv(M, N, K, 16, wq::kFmtNvfp4, buf, buf_len);
  return WQ_OK;
}

}  // extern "C"
