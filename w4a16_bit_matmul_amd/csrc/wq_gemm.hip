// Dequantize-to-fp16 tile GEMM on CDNA4 matrix cores (gfx950).
//
// y = x * What^T with What = s * (q - z) formed inside the kernel: the dense
// regime of "Quantization Methods Compared: INT8, GPTQ, AWQ, FP8, FP4 and
// KV-Cache Quantization", section "Hardware, formats and the roofline" (past
// the ridge point the product is compute-bound and the in-kernel dequantization
// is extra instructions), decoding from "Quantization for LLM inference: FP8,
// INT4 (GPTQ, AWQ) and GGUF", section "The minimum maths".
//
// MFMA: v_mfma_f32_16x16x32_f16.  Lane l = r + 16*c supplies A row r and B
// column r, each with the eight k-slots 8c..8c+7 of the 32-deep step.  The
// packed tile layout gives lane l exactly those slots for column r: word j of
// its 16 bytes holds columns 32j + 8c + e, so step j of a 128-column tile uses
// word j as the B operand and x[m][32j + 8c .. 32j + 8c + 7] (one 16-byte load)
// as the A operand.
//
// B dequantization per pair of columns: shift + AND-OR (1024 + q, exact fp16),
// v_pk_add_f16 with -(1024 + z) (exact q - z), v_pk_mul_f16 with the scale
// (one round-to-nearest-even: fp16(What)).  Accumulation is fp32 in the MFMA.
//
// Decomposition: a workgroup (4 waves) owns a (16*MB) x (16*NBW) output tile;
// wave w takes the 128-column tiles kt = w, w+4, ... of K, dequantizes its own
// B operands in registers (no weight is dequantized twice) and accumulates a
// full-tile partial; the four partials are added through LDS in a fixed order.
#include "wq_device.h"
#include "wq_kernels.h"

namespace wq {
namespace {

constexpr int kWaves = 4;

__device__ __forceinline__ f4 mfma16(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// fp16(s * (q - z)) for the eight columns held by one packed word.
__device__ __forceinline__ h8 dequant_word(uint32_t word, h2 neg_bias, h2 scale) {
  h2 p0 = (biased_pair(word, 0) + neg_bias) * scale;
  h2 p1 = (biased_pair(word, 1) + neg_bias) * scale;
  h2 p2 = (biased_pair(word, 2) + neg_bias) * scale;
  h2 p3 = (biased_pair(word, 3) + neg_bias) * scale;
  h8 out;
  out[0] = p0[0]; out[1] = p0[1]; out[2] = p1[0]; out[3] = p1[1];
  out[4] = p2[0]; out[5] = p2[1]; out[6] = p3[0]; out[7] = p3[1];
  return out;
}

template <int MB, int NBW, int G>
__global__ __launch_bounds__(kWaves * 64) void gemm_kernel(
    int64_t M, int64_t N, int64_t K, const uint16_t* __restrict__ x, const uint32_t* __restrict__ qpacked,
    const uint16_t* __restrict__ s_in, const uint8_t* __restrict__ zpacked, uint16_t* __restrict__ y, int64_t KT) {
  constexpr int JG = (G == 128) ? 1 : 4;
  constexpr int NACC = MB * NBW * 4;
  __shared__ float red[2][NACC][64];

  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, c = lane >> 4;
  const int64_t nb0 = (int64_t)blockIdx.x * NBW;
  const int64_t mrow0 = (int64_t)blockIdx.y * (16 * MB);
  const int64_t NBLK = (N + 15) / 16;
  const int64_t Gtot = K / G, GB = (Gtot + 1) / 2;

  int64_t nrow[NBW];
  bool blk_ok[NBW];
#pragma unroll
  for (int b = 0; b < NBW; ++b) {
    blk_ok[b] = nb0 + b < NBLK;
    int64_t n = (nb0 + b) * 16 + r;
    nrow[b] = n < N ? n : N - 1;
  }
  bool row_ok[MB];
  const uint16_t* xrow[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    int64_t m = mrow0 + 16 * i + r;
    row_ok[i] = m < M;
    xrow[i] = x + (row_ok[i] ? m : 0) * K + 8 * c;
  }

  f4 acc[MB][NBW];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int b = 0; b < NBW; ++b) acc[i][b] = f4{0.f, 0.f, 0.f, 0.f};

  const uint8_t* qbase = reinterpret_cast<const uint8_t*>(qpacked) + 16 * lane;

  for (int64_t kt = wv; kt < KT; kt += kWaves) {
    u4 bw[NBW];
    h2 nbias[NBW][JG], scl[NBW][JG];
#pragma unroll
    for (int b = 0; b < NBW; ++b) {
      bw[b] = blk_ok[b] ? *reinterpret_cast<const u4*>(qbase + tile_offset_bytes(nb0 + b, kt, KT)) : u4{0, 0, 0, 0};
#pragma unroll
      for (int jg = 0; jg < JG; ++jg) {
        int64_t gi = (G == 128) ? kt : kt * 4 + jg;
        gi = gi < Gtot ? gi : Gtot - 1;
        _Float16 sv = __builtin_bit_cast(_Float16, s_in[nrow[b] * Gtot + gi]);
        _Float16 zv = (_Float16)(-(1024.0f + (float)load_zero(zpacked, GB, nrow[b], gi)));
        scl[b][jg] = h2{sv, sv};
        nbias[b][jg] = h2{zv, zv};
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int jg = (G == 128) ? 0 : j;
      const bool col_ok = kt * 128 + 32 * j < K;
      h8 a[MB];
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        if (row_ok[i] && col_ok) {
          a[i] = __builtin_bit_cast(h8, *reinterpret_cast<const uint4*>(xrow[i] + kt * 128 + 32 * j));
        } else {
          a[i] = h8{0, 0, 0, 0, 0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int b = 0; b < NBW; ++b) {
        const h8 bf = dequant_word(bw[b][j], nbias[b][jg], scl[b][jg]);
#pragma unroll
        for (int i = 0; i < MB; ++i) acc[i][b] = mfma16(a[i], bf, acc[i][b]);
      }
    }
  }

  // ---- add the four partial tiles: (2,3) -> (0,1), then 1 -> 0
  auto put = [&](int slot) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int b = 0; b < NBW; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[slot][(i * NBW + b) * 4 + e][lane] = acc[i][b][e];
  };
  auto add = [&](int slot) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int b = 0; b < NBW; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][b][e] += red[slot][(i * NBW + b) * 4 + e][lane];
  };
  if (wv >= 2) put(wv - 2);
  __syncthreads();
  if (wv < 2) add(wv);
  __syncthreads();
  if (wv == 1) put(0);
  __syncthreads();
  if (wv != 0) return;
  add(0);

  // ---- epilogue: lane (r, c) holds rows 4c..4c+3 of column r of each block
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int b = 0; b < NBW; ++b) {
      const int64_t n = (nb0 + b) * 16 + r;
      if (n >= N) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t m = mrow0 + 16 * i + 4 * c + e;
        if (m < M) y[m * N + n] = f32_to_f16_bits(acc[i][b][e]);
      }
    }
}

template <int MB, int NBW>
hipError_t launch_t(int64_t M, int64_t N, int64_t K, int group, const uint16_t* x, const uint32_t* qpacked,
                    const uint16_t* s, const uint8_t* zpacked, uint16_t* y, hipStream_t stream) {
  const int64_t NBLK = (N + 15) / 16, KT = (K + 127) / 128;
  dim3 grid((unsigned)((NBLK + NBW - 1) / NBW), (unsigned)((M + 16 * MB - 1) / (16 * MB))), block(kWaves * 64);
  if (group == 128)
    gemm_kernel<MB, NBW, 128><<<grid, block, 0, stream>>>(M, N, K, x, qpacked, s, zpacked, y, KT);
  else
    gemm_kernel<MB, NBW, 32><<<grid, block, 0, stream>>>(M, N, K, x, qpacked, s, zpacked, y, KT);
  return hipGetLastError();
}

}  // namespace

size_t gemm_workspace_bytes(int64_t, int64_t, int64_t, int) { return 0; }

hipError_t launch_gemm(int64_t M, int64_t N, int64_t K, int group, const uint16_t* x, const uint32_t* qpacked,
                       const uint16_t* s, const uint8_t* zpacked, uint16_t* y, void* /*workspace*/,
                       hipStream_t stream) {
  const int64_t NBLK = (N + 15) / 16;
  if (M <= 16) return launch_t<1, 4>(M, N, K, group, x, qpacked, s, zpacked, y, stream);
  if (M <= 32) return launch_t<2, 4>(M, N, K, group, x, qpacked, s, zpacked, y, stream);
  if (M <= 64) return launch_t<4, 4>(M, N, K, group, x, qpacked, s, zpacked, y, stream);
  if (NBLK % 7 == 0 && NBLK / 7 >= 192) return launch_t<8, 7>(M, N, K, group, x, qpacked, s, zpacked, y, stream);
  return launch_t<8, 4>(M, N, K, group, x, qpacked, s, zpacked, y, stream);
}

}  // namespace wq
