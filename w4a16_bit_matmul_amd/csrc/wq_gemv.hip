// Split-K dequantize-and-multiply GEMV for small M (gfx950, VALU path).
//
// Computes y[m][n] = sum_k x[m][k] * s[n][g(k)] * (q[n][k] - z[n][g(k)]) -- the
// fused weight-only product of "Quantization Methods Compared: INT8, GPTQ, AWQ,
// FP8, FP4 and KV-Cache Quantization", section "Hardware, formats and the
// roofline" (decode reads every weight once and is bound by memory bandwidth),
// with the decoding of "Quantization for LLM inference: FP8, INT4 (GPTQ, AWQ)
// and GGUF", section "The minimum maths".
//
// Arithmetic: a packed word becomes four fp16 pairs (1024 + 64q) with one shift
// and one AND-OR each; v_dot2_f32_f16 multiplies them with fp16 activation
// pairs into fp32.  Per group,
//   sum_k x * s * (q - z) = (s/64) * (sum_k x * (1024 + 64q) - (1024 + 64z) * sum_k x),
// so the scale and zero-point are applied once per lane and group, not per
// weight.  All products are exact in fp32; the sums round in fp32.  Putting
// the code in the upper mantissa bits (64q rather than q) keeps the bias term
// within a few times the code term, so the subtraction cancels few bits.
//
// Decomposition: a workgroup owns NB consecutive 16-row blocks and MT rows of
// x, over all of K; its waves split the 128-column tiles round-robin (split-K
// inside the workgroup), every lane streaming 16 bytes of codes per tile.
// Partial sums meet in LDS in a fixed order, so results are deterministic.
#include "wq_device.h"
#include "wq_kernels.h"

namespace wq {
namespace {

__device__ __forceinline__ float dot2(h2 a, h2 b, float c) { return __builtin_amdgcn_fdot2(a, b, c, false); }

template <int MT, int NB, int G, int KU, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void gemv_kernel(
    int64_t M, int64_t N, int64_t K, const uint16_t* __restrict__ x, const uint32_t* __restrict__ qpacked,
    const uint16_t* __restrict__ s_in, const uint8_t* __restrict__ zpacked, uint16_t* __restrict__ y,
    int64_t KT) {
  constexpr int JG = (G == 128) ? 1 : 4;  // groups per 16-byte lane chunk
  __shared__ float red[WAVES][NB][MT][16];

  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, c = lane >> 4;
  const int64_t nb0 = (int64_t)blockIdx.x * NB;
  const int64_t m0 = (int64_t)blockIdx.y * MT;
  const int64_t Gtot = K / G, GB = (Gtot + 1) / 2;
  const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};

  const int64_t NBLK = (N + 15) / 16;
  int64_t nrow[NB];
  bool blk_ok[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    blk_ok[b] = nb0 + b < NBLK;  // the last workgroup may own fewer row blocks
    int64_t n = (nb0 + b) * 16 + r;
    nrow[b] = n < N ? n : N - 1;  // pad rows read a valid scale; their output is dropped
  }

  float acc[NB][MT];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[b][m] = 0.0f;

  const uint8_t* qbase = reinterpret_cast<const uint8_t*>(qpacked) + 16 * lane;

  for (int64_t kt0 = wv; kt0 < KT; kt0 += (int64_t)WAVES * KU) {
    u4 wword[KU][NB];
    uint4 xraw[KU][MT][4];
    float sc[KU][NB][JG];
    float zb[KU][NB][JG];
    // ---- issue every load of this step first
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int64_t kt = kt0 + (int64_t)u * WAVES;
      const bool kt_ok = kt < KT;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if (kt_ok && blk_ok[b]) {
          wword[u][b] = *reinterpret_cast<const u4*>(qbase + tile_offset_bytes(nb0 + b, kt, KT));
        } else {
          wword[u][b] = u4{0, 0, 0, 0};
        }
#pragma unroll
        for (int jg = 0; jg < JG; ++jg) {
          int64_t gi = (G == 128) ? kt : kt * 4 + jg;
          gi = gi < Gtot ? gi : Gtot - 1;
          // s/64 and 1024 + 64z: both exact in fp32
          sc[u][b][jg] = kt_ok ? f16_bits_to_f32(s_in[nrow[b] * Gtot + gi]) * 0.015625f : 0.0f;
          zb[u][b][jg] = kt_ok ? 1024.0f + 64.0f * (float)load_zero(zpacked, GB, nrow[b], gi) : 0.0f;
        }
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t k0 = kt * 128 + 32 * j + 8 * c;
          if (kt_ok && m0 + m < M && kt * 128 + 32 * j < K) {
            xraw[u][m][j] = *reinterpret_cast<const uint4*>(x + (m0 + m) * K + k0);
          } else {
            xraw[u][m][j] = make_uint4(0, 0, 0, 0);
          }
        }
      }
    }
    // ---- compute
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      // per-group activation sums of this lane's columns
      float xs[MT][JG];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
#pragma unroll
        for (int jg = 0; jg < JG; ++jg) xs[m][jg] = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint4 v = xraw[u][m][j];
          const int jg = (G == 128) ? 0 : j;
          xs[m][jg] = dot2(as_h2(v.x), ones, xs[m][jg]);
          xs[m][jg] = dot2(as_h2(v.y), ones, xs[m][jg]);
          xs[m][jg] = dot2(as_h2(v.z), ones, xs[m][jg]);
          xs[m][jg] = dot2(as_h2(v.w), ones, xs[m][jg]);
        }
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        float t[MT][JG];
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int jg = 0; jg < JG; ++jg) t[m][jg] = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t word = wword[u][b][j];
          const h2 p0 = biased_pair64(word, 0), p1 = biased_pair64(word, 1);
          const h2 p2 = biased_pair64(word, 2), p3 = biased_pair64(word, 3);
          const int jg = (G == 128) ? 0 : j;
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            const uint4 v = xraw[u][m][j];
            float a = t[m][jg];
            a = dot2(p0, as_h2(v.x), a);
            a = dot2(p1, as_h2(v.y), a);
            a = dot2(p2, as_h2(v.z), a);
            a = dot2(p3, as_h2(v.w), a);
            t[m][jg] = a;
          }
        }
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int jg = 0; jg < JG; ++jg)
            acc[b][m] = fmaf(sc[u][b][jg], fmaf(-zb[u][b][jg], xs[m][jg], t[m][jg]), acc[b][m]);
      }
    }
  }

  // ---- reduce: the four lanes of a row, then the waves, in a fixed order
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float v = acc[b][m];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      if (c == 0) red[wv][b][m][r] = v;
    }
  __syncthreads();
  for (int i = threadIdx.x; i < NB * MT * 16; i += WAVES * 64) {
    const int rr = i & 15, m = (i >> 4) % MT, b = (i >> 4) / MT;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) v += red[w][b][m][rr];
    const int64_t n = (nb0 + b) * 16 + rr;
    if (n < N && m0 + m < M) y[(m0 + m) * N + n] = f32_to_f16_bits(v);
  }
}

template <int MT, int NB, int KU128, int KU32, int WAVES>
hipError_t launch_t(int64_t M, int64_t N, int64_t K, int group, const uint16_t* x, const uint32_t* qpacked,
                    const uint16_t* s, const uint8_t* zpacked, uint16_t* y, hipStream_t stream) {
  const int64_t NBLK = (N + 15) / 16, KT = (K + 127) / 128;
  dim3 grid((unsigned)((NBLK + NB - 1) / NB), (unsigned)((M + MT - 1) / MT)), block(WAVES * 64);
  if (group == 128)
    gemv_kernel<MT, NB, 128, KU128, WAVES><<<grid, block, 0, stream>>>(M, N, K, x, qpacked, s, zpacked, y, KT);
  else
    gemv_kernel<MT, NB, 32, KU32, WAVES><<<grid, block, 0, stream>>>(M, N, K, x, qpacked, s, zpacked, y, KT);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(int64_t M, int64_t N, int64_t K, int group, const uint16_t* x, const uint32_t* qpacked,
                       const uint16_t* s, const uint8_t* zpacked, uint16_t* y, hipStream_t stream) {
  if (M == 1) return launch_t<1, 2, 2, 1, 16>(M, N, K, group, x, qpacked, s, zpacked, y, stream);
  if (M == 2) return launch_t<2, 2, 2, 1, 16>(M, N, K, group, x, qpacked, s, zpacked, y, stream);
  if (M <= 4) return launch_t<4, 2, 1, 1, 16>(M, N, K, group, x, qpacked, s, zpacked, y, stream);
  return launch_t<8, 2, 1, 1, 8>(M, N, K, group, x, qpacked, s, zpacked, y, stream);
}

}  // namespace wq
