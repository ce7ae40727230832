// Allocation-free variant of the W4A16 product (wq_gemm_w4a16_noalloc).
//
// For callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops): the split-K workspace that wq_gemm_w4a16
// takes from its caller lives here in a fixed device array instead, one copy
// per GPU for the life of the process.  Layout as any workspace: the
// WQ_WORKSPACE_COUNTER_BYTES of split-K counters, then the fp32 partial sums.
//
// The array's name is a host-side stand-in in host code, not a device address:
// on its first call on a device the entry point asks the runtime for that
// device's address of the array (hipGetSymbolAddress, with the device current)
// and keeps it; kernels and fills only ever receive that pointer.  The first
// call also clears the counters with a fill kernel on the caller's stream (no
// memset node, so a captured graph replays correctly); every product then
// leaves them zero again.  Calls that overlap on one GPU share the array and
// race: callers serialize them (one stream, or their own ordering).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/libwq.h"
#include "wq_device.h"
#include "wq_kernels.h"

namespace {

static_assert(WQ_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static_assert(WQ_NOALLOC_SCRATCH_BYTES > WQ_WORKSPACE_COUNTER_BYTES, "scratch holds the counters");

static __device__ __align__(256) uint8_t scratch[WQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;      // this device's address of `scratch`
  hipError_t err = hipSuccess;
};
ScratchSlot g_slots[kMaxDevices];

__global__ void zero_words_kernel(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// The current device's scratch pointer, set up on the first call on that
// device: its address from the runtime, then the counters cleared on `stream`.
hipError_t scratch_for_current_device(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  ScratchSlot& slot = g_slots[dev];
  std::call_once(slot.once, [&] {
    void* p = nullptr;
    slot.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (slot.err != hipSuccess) return;
    constexpr int nwords = WQ_WORKSPACE_COUNTER_BYTES / 4;
    zero_words_kernel<<<(nwords + 255) / 256, 256, 0, stream>>>(static_cast<uint32_t*>(p), nwords);
    slot.err = hipGetLastError();
    if (slot.err == hipSuccess) slot.ptr = p;
  });
  *out = slot.ptr;
  return slot.err;
}

}  // namespace

extern "C" int wq_gemm_w4a16_noalloc(int64_t M, int64_t N, int64_t K, int group, const uint16_t* x_f16,
                                     const uint32_t* qpacked, const uint16_t* s_f16, const uint8_t* zpacked,
                                     uint16_t* y_f16, void* stream) {
  // the scratch the product needs, checked before anything is set up or enqueued
  const size_t need = wq_gemm_workspace_bytes_ex(M, N, K, group, WQ_PATH_AUTO);
  if (need > (size_t)WQ_NOALLOC_SCRATCH_BYTES) return WQ_EWORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    if (scratch_for_current_device(static_cast<hipStream_t>(stream), &ws) != hipSuccess || !ws) return WQ_EHIP;
  }
  return wq_gemm_w4a16_ex(M, N, K, group, x_f16, qpacked, s_f16, zpacked, y_f16, ws,
                          need > 0 ? (size_t)WQ_NOALLOC_SCRATCH_BYTES : 0, WQ_PATH_AUTO, stream);
}
