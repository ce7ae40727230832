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
//
// Matrix-core probe: the rate at which this GPU sustains the fp16 MFMA
// instruction the product kernels use (v_mfma_f32_16x16x32_f16) when nothing
// else runs -- no memory traffic, no other vector work -- under the clock the
// part holds at that load.  It is the compute-side counterpart of the read
// probe: the ceiling of a product that is bound by its matrix-core work, next
// to the nominal dense fp16 peak.  Each wave keeps eight independent
// accumulators and issues `iters` rounds of eight MFMAs on register operands.
//
// Clock probe: the rate of the shader clock counter (s_memtime) against the
// constant 100 MHz real-time counter (s_memrealtime) over a short spin of one
// wave per workgroup; launched right after a timed region, it gives the core
// clock the part was holding there.  The spin ends after `ticks` real-time
// ticks or a fixed number of reads, whichever comes first.
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

__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  h8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)((lane + i) & 7) * (_Float16)0.125f;
    b[i] = (_Float16)((lane * 3 + i) & 7) * (_Float16)0.0625f;
  }
  f4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[j], 0, 0, 0);
  }
  float t = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) t += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  if (__builtin_bit_cast(uint32_t, t) == kProbeMagic) sink[0] = kProbeMagic;
}

__global__ __launch_bounds__(64) void clock_probe_kernel(uint32_t ticks, unsigned long long* __restrict__ out) {
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  uint64_t r = r0;
  for (int i = 0; i < (1 << 22) && r - r0 < ticks; ++i) r = __builtin_amdgcn_s_memrealtime();
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    out[2 * blockIdx.x] = c1 - c0;
    out[2 * blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace

hipError_t launch_clock_probe(int workgroups, uint32_t ticks, unsigned long long* out, hipStream_t stream) {
  clock_probe_kernel<<<workgroups, 64, 0, stream>>>(ticks, out);
  return hipGetLastError();
}

hipError_t launch_mfma_probe(int workgroups, int iters, int count, uint32_t* sink, hipStream_t stream) {
  for (int i = 0; i < count; ++i) mfma_probe_kernel<<<workgroups, 256, 0, stream>>>(iters, sink);
  return hipGetLastError();
}

hipError_t launch_read_probe(const void* src, size_t window_bytes, size_t span_bytes, int count, int chunks,
                             int nontemporal, uint32_t* sink, hipStream_t stream) {
  const uint8_t* p = static_cast<const uint8_t*>(src);
  const size_t nwin = span_bytes / window_bytes;
  if (nontemporal) launch_nt<true>(p, window_bytes, nwin, count, chunks, sink, stream);
  else launch_nt<false>(p, window_bytes, nwin, count, chunks, sink, stream);
  return hipGetLastError();
}

}  // namespace wq
