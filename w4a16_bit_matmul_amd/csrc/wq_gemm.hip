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
// column r, each with the eight k-slots 8c..8c+7 of the 32-deep step, and
// receives D rows 4c..4c+3 of column r.  The packed tile layout gives lane l
// exactly those slots for column r: word j of its 16 bytes holds columns
// 32j + 8c + e, so step j of a 128-column tile uses word j as the B operand and
// x[m][32j + 8c .. 32j + 8c + 7] (one 16-byte load) as the A operand.
//
// B dequantization per pair of columns: shift + AND-OR (1024 + q, exact fp16),
// packed fp16 add of -(1024 + z) (exact q - z), packed fp16 multiply by the
// scale (one round-to-nearest-even: fp16(What)).  Accumulation is fp32 in the
// matrix cores.
//
// Decomposition: a workgroup (4 waves, one per SIMD) owns a (16*MB) x (64*NPW)
// output tile.  The activation tile of each 128-column K step (16*MB rows) is
// loaded once per workgroup into LDS (double-buffered, rows padded against
// bank conflicts) and read by all four waves; wave w owns NPW 16-column blocks,
// dequantizes its own B operands in registers (no weight is dequantized
// twice) and accumulates its columns over all of K, so no partial sums cross
// waves.  Code tiles, scales and zero-points are loaded three K steps ahead of
// use, activations one K step ahead.
#include "wq_device.h"
#include "wq_kernels.h"

namespace wq {
namespace {

constexpr int kWaves = 4;

struct GemmArgs {
  const uint16_t* x;
  const uint8_t* qp;
  const uint16_t* s;
  const uint8_t* zp;
  uint16_t* y;
  int M, N, K, KT, Gtot, GB, NBLK, sz_vec;
};

__device__ __forceinline__ f4 mfma16(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Forces a value into a VGPR and hides it from constant folding, so that
// v_and_or_b32 takes the mask from an SGPR and the fp16 exponent from here.
__device__ __forceinline__ uint32_t in_vgpr(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Scales and zero-points of one row for one 128-column K tile, as loaded:
// g = 128: one group (scale bits in s, zero-point byte in z, nibble zsh);
// g = 32: four groups (scales in the four halves of s / s2, nibbles of z).
template <int G>
struct TileSZ {
  uint32_t s, s2, z;
};

template <int G>
__device__ __forceinline__ TileSZ<G> load_tile_sz(const GemmArgs& a, uint32_t srow, uint32_t zrow, int kt) {
  TileSZ<G> v;
  if constexpr (G == 128) {
    v.s = a.s[srow + kt];
    v.z = a.zp[zrow + (kt >> 1)];
    v.s2 = 0;
  } else {
    const int g0 = kt * 4;
    if (a.sz_vec) {
      const uint2 t = *reinterpret_cast<const uint2*>(a.s + srow + g0);
      v.s = t.x;
      v.s2 = t.y;
      v.z = *reinterpret_cast<const uint16_t*>(a.zp + zrow + g0 / 2);
    } else {
      uint32_t sh[4], zz = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int gi = min(g0 + j, a.Gtot - 1);
        sh[j] = a.s[srow + gi];
        const uint32_t zb = a.zp[zrow + (gi >> 1)];
        zz |= ((gi & 1) ? (zb >> 4) : (zb & 15u)) << (4 * j);
      }
      v.s = sh[0] | (sh[1] << 16);
      v.s2 = sh[2] | (sh[3] << 16);
      v.z = zz;
    }
  }
  return v;
}

// (scale, scale) and (-(1024 + z), -(1024 + z)) fp16 pairs of group j (word j).
template <int G>
__device__ __forceinline__ void tile_consts(const TileSZ<G>& v, int kt, int j, uint32_t magic, h2& sc, h2& nb) {
  uint32_t sb, z;
  if constexpr (G == 128) {
    sb = v.s & 0xffffu;
    z = (v.z >> (4 * (kt & 1))) & 15u;
  } else {
    sb = ((j < 2 ? v.s : v.s2) >> (16 * (j & 1))) & 0xffffu;
    z = (v.z >> (4 * j)) & 15u;
  }
  sc = as_h2(sb * 0x00010001u);
  nb = -as_h2(z * 0x00010001u + magic);
}

// fp16(s * (q - z)) for the eight columns held by one packed word.
__device__ __forceinline__ h8 dequant_word(uint32_t w, uint32_t magic, h2 nb, h2 sc) {
  const h2 p0 = (as_h2((w & 0x000F000Fu) | magic) + nb) * sc;
  const h2 p1 = (as_h2(((w >> 4) & 0x000F000Fu) | magic) + nb) * sc;
  const h2 p2 = (as_h2(((w >> 8) & 0x000F000Fu) | magic) + nb) * sc;
  const h2 p3 = (as_h2(((w >> 12) & 0x000F000Fu) | magic) + nb) * sc;
  h8 out;
  out[0] = p0[0]; out[1] = p0[1]; out[2] = p1[0]; out[3] = p1[1];
  out[4] = p2[0]; out[5] = p2[1]; out[6] = p3[0]; out[7] = p3[1];
  return out;
}

constexpr int kArow = 128 * 2 + 16;  // LDS bytes per activation row of a K step (padded)
constexpr int kBdepth = 3;           // K steps of codes in flight ahead of use

template <int MB, int NPW, int G>
__global__ __launch_bounds__(kWaves * 64) void gemm_kernel(GemmArgs a) {
  constexpr int ROWS = 16 * MB;
  constexpr int ACH = ROWS * 16 / (kWaves * 64);  // 16-byte activation chunks per thread and K step
  static_assert(ACH >= 1 && ROWS * 16 % (kWaves * 64) == 0, "whole chunks per thread");
  extern __shared__ __align__(16) uint8_t smem[];  // [2][ROWS][kArow]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, c = lane >> 4;
  const int nbw0 = blockIdx.x * (kWaves * NPW) + wv * NPW;  // this wave's first column block
  const int mrow0 = blockIdx.y * ROWS;
  const uint32_t magic = in_vgpr(kMagicPair);
  const int KT = a.KT;

  // wave-uniform B tile bases of this wave's column blocks (blocks past the end
  // re-read the last one), per-lane offsets of the row's scales / zeros
  const uint8_t* tb[NPW];
  uint32_t srow[NPW], zrow[NPW];
#pragma unroll
  for (int b = 0; b < NPW; ++b) {
    tb[b] = a.qp + (size_t)min(nbw0 + b, a.NBLK - 1) * KT * kTileBytes + 16u * lane;
    const uint32_t n = (uint32_t)min((nbw0 + b) * 16 + r, a.N - 1);
    srow[b] = n * (uint32_t)a.Gtot;
    zrow[b] = n * (uint32_t)a.GB;
  }
  // activation chunks this thread stages: chunk q = tid + 256*i is row q / 16,
  // columns 8*(q % 16) .. +8 of the K step (rows past M re-read row M - 1,
  // columns past K are stored as zeros)
  uint32_t xoff[ACH], loff[ACH];
  int xcol[ACH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    const int q = tid + kWaves * 64 * i, row = q >> 4, cc = q & 15;
    xoff[i] = (uint32_t)min(mrow0 + row, a.M - 1) * (uint32_t)a.K;
    xcol[i] = 8 * cc;
    loff[i] = (uint32_t)(row * kArow + 16 * cc);
  }
  auto load_x = [&](int kt, uint4 (&v)[ACH]) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int col = min(kt * 128 + xcol[i], a.K - 8);
      v[i] = *reinterpret_cast<const uint4*>(a.x + xoff[i] + col);
    }
  };
  auto store_x = [&](int kt, int buf, const uint4 (&v)[ACH]) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const bool ok = kt * 128 + xcol[i] < a.K;
      *reinterpret_cast<uint4*>(smem + buf * (ROWS * kArow) + loff[i]) = ok ? v[i] : make_uint4(0, 0, 0, 0);
    }
  };
  struct BStep {
    u4 codes[NPW];
    TileSZ<G> sz[NPW];
  };
  auto load_b = [&](int kt, BStep& d) {
    kt = min(kt, KT - 1);  // steps past the end re-load the last (unused)
#pragma unroll
    for (int b = 0; b < NPW; ++b) d.sz[b] = load_tile_sz<G>(a, srow[b], zrow[b], kt);
#pragma unroll
    for (int b = 0; b < NPW; ++b) d.codes[b] = *reinterpret_cast<const u4*>(tb[b] + (size_t)kt * kTileBytes);
  };

  f4 acc[MB][NPW];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int b = 0; b < NPW; ++b) acc[i][b] = f4{0.f, 0.f, 0.f, 0.f};

  // ---- prologue: codes of steps 0..kBdepth-1, activations of step 0 in LDS
  BStep bq[kBdepth + 1];
  {
    uint4 xv[ACH];
    load_x(0, xv);
#pragma unroll
    for (int d = 0; d < kBdepth; ++d) load_b(d, bq[d]);
    store_x(0, 0, xv);
  }
  __syncthreads();

  // lane (r, c) reads A rows 16i + r, columns 32j + 8c .. +8 of the step
  const uint32_t aread = (uint32_t)(r * kArow + 16 * c);

  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < KT;
    uint4 xv[ACH];
    if (more) load_x(kt + 1, xv);
    load_b(kt + kBdepth, bq[kBdepth]);
    const BStep& cur = bq[0];
    const uint8_t* abase = smem + buf * (ROWS * kArow) + aread;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (kt * 128 + 32 * j >= a.K) break;  // ragged last step: no columns left
      h8 af[MB];
#pragma unroll
      for (int i = 0; i < MB; ++i)
        af[i] = __builtin_bit_cast(h8, *reinterpret_cast<const uint4*>(abase + i * 16 * kArow + 64 * j));
#pragma unroll
      for (int b = 0; b < NPW; ++b) {
        h2 sc, nbias;
        tile_consts<G>(cur.sz[b], kt, j, magic, sc, nbias);
        const h8 bf = dequant_word(cur.codes[b][j], magic, nbias, sc);
#pragma unroll
        for (int i = 0; i < MB; ++i) acc[i][b] = mfma16(af[i], bf, acc[i][b]);
      }
    }
    if (more) store_x(kt + 1, buf ^ 1, xv);
    __syncthreads();
#pragma unroll
    for (int d = 0; d < kBdepth; ++d) bq[d] = bq[d + 1];
  }

  // ---- epilogue: lane (r, c) holds rows 4c..4c+3 of column r of each block
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int b = 0; b < NPW; ++b) {
      const int n = (nbw0 + b) * 16 + r;
      if (n >= a.N) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = mrow0 + 16 * i + 4 * c + e;
        if (m < a.M) a.y[(size_t)m * a.N + n] = f32_to_f16_bits(acc[i][b][e]);
      }
    }
}

template <int MB, int NPW>
hipError_t launch_t(int group, const GemmArgs& a, hipStream_t stream) {
  const int cols = kWaves * NPW;  // column blocks per workgroup
  dim3 grid((unsigned)((a.NBLK + cols - 1) / cols), (unsigned)((a.M + 16 * MB - 1) / (16 * MB))),
      block(kWaves * 64);
  const size_t lds = (size_t)2 * 16 * MB * kArow;
  if (group == 128) {
    auto k = gemm_kernel<MB, NPW, 128>;
    if (lds > 65536) hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    k<<<grid, block, lds, stream>>>(a);
  } else {
    auto k = gemm_kernel<MB, NPW, 32>;
    if (lds > 65536) hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    k<<<grid, block, lds, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace

size_t gemm_workspace_bytes(int64_t, int64_t, int64_t, int) { return 0; }

hipError_t launch_gemm(int64_t M, int64_t N, int64_t K, int group, const uint16_t* x, const uint32_t* qpacked,
                       const uint16_t* s, const uint8_t* zpacked, uint16_t* y, void* /*workspace*/,
                       hipStream_t stream) {
  GemmArgs a;
  a.x = x;
  a.qp = reinterpret_cast<const uint8_t*>(qpacked);
  a.s = s;
  a.zp = zpacked;
  a.y = y;
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  a.KT = (int)((K + 127) / 128);
  a.Gtot = (int)(K / group);
  a.GB = (a.Gtot + 1) / 2;
  a.NBLK = (int)((N + 15) / 16);
  // g = 32: a tile's four scales (8 bytes) and zero-points (2 bytes) load as
  // one vector each when every row starts suitably aligned
  a.sz_vec = (group == 32 && a.Gtot % 4 == 0 && (reinterpret_cast<uintptr_t>(s) & 7) == 0 &&
              (reinterpret_cast<uintptr_t>(zpacked) & 1) == 0)
                 ? 1
                 : 0;
  if (M <= 16) return launch_t<1, 1>(group, a, stream);
  if (M <= 32) return launch_t<2, 1>(group, a, stream);
  if (M <= 64) return launch_t<4, 2>(group, a, stream);
  return launch_t<8, 2>(group, a, stream);
}

}  // namespace wq
