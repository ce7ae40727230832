// Streaming-read probe: how fast this GPU reads a buffer of a given size once.
// A decode product's time is the reading of its weights (the roofline argument
// of "Hardware, formats and the roofline"), so the probe's rate on the same
// byte count is the ceiling that kernel can reach on this part, next to the
// nominal 8 TB/s.
//
// One pass, no grid-stride loop: workgroup b of 256 threads reads chunks
// [256*U*b, 256*U*(b+1)) of 16 bytes, thread t the chunks t, t + 256, ... (so
// each of the U loads of a wave covers 1 KB contiguously).  Chunks past the end
// re-read the last one (no branch, so all U loads are in flight together);
// plain or non-temporal (streaming-hint) loads.  The
// XOR of a thread's words is stored only if it equals a fixed value, which
// keeps the loads and practically never writes.
#include "wq_device.h"
#include "wq_kernels.h"

namespace wq {
namespace {

constexpr uint32_t kProbeMagic = 0x9e3779b9u;

template <int U, bool NTL>
__global__ __launch_bounds__(256) void read_probe_kernel(const u4* __restrict__ src, int64_t n16,
                                                         uint32_t* __restrict__ sink) {
  const int64_t base = (int64_t)blockIdx.x * 256 * U + threadIdx.x;
  u4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const u4* p = src + min(base + 256 * u, n16 - 1);
    if constexpr (NTL) v[u] = __builtin_nontemporal_load(p);
    else v[u] = *p;
  }
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  if (acc == kProbeMagic) sink[0] = acc;
}

template <int U, bool NTL>
void launch_u(const uint8_t* src, size_t window, size_t nwin, int count, uint32_t* sink, hipStream_t s) {
  const int64_t n16 = (int64_t)(window / 16);
  const unsigned grid = (unsigned)((n16 + 256 * U - 1) / (256 * U));
  for (int i = 0; i < count; ++i)
    read_probe_kernel<U, NTL><<<grid, 256, 0, s>>>(reinterpret_cast<const u4*>(src + (size_t)(i % nwin) * window),
                                                   n16, sink);
}

template <bool NTL>
void launch_nt(const uint8_t* p, size_t window, size_t nwin, int count, int chunks, uint32_t* sink, hipStream_t s) {
  if (chunks == 1) launch_u<1, NTL>(p, window, nwin, count, sink, s);
  else if (chunks == 2) launch_u<2, NTL>(p, window, nwin, count, sink, s);
  else if (chunks == 4) launch_u<4, NTL>(p, window, nwin, count, sink, s);
  else if (chunks == 8) launch_u<8, NTL>(p, window, nwin, count, sink, s);
  else launch_u<16, NTL>(p, window, nwin, count, sink, s);
}

}  // namespace

hipError_t launch_read_probe(const void* src, size_t window_bytes, size_t span_bytes, int count, int chunks,
                             int nontemporal, uint32_t* sink, hipStream_t stream) {
  const uint8_t* p = static_cast<const uint8_t*>(src);
  const size_t nwin = span_bytes / window_bytes;
  if (nontemporal) launch_nt<true>(p, window_bytes, nwin, count, chunks, sink, stream);
  else launch_nt<false>(p, window_bytes, nwin, count, chunks, sink, stream);
  return hipGetLastError();
}

}  // namespace wq
