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
// Decomposition: a workgroup of eight waves (two per SIMD) owns a (16*MB) x
// (64*NPW) output tile.  Waves 0-3 take the first half of the 128-column K
// steps and waves 4-7 the second; within a half, wave w owns NPW 16-column
// blocks, dequantizes its own B operands in registers (no weight is
// dequantized twice) and accumulates its columns over its half of K.  Each
// half loads the activation tile of its current K step once into LDS
// (double-buffered, rows padded against bank conflicts), read by its four
// waves.  Code tiles, scales and zero-points are loaded three K steps ahead of
// use, activations one step ahead.  At the end the second half's sums are
// added to the first half's through LDS, in a fixed order.
#include <stdio.h>

#include <type_traits>

#include "wq_device.h"
#include "wq_kernels.h"

namespace wq {
namespace {

constexpr int kWaves = 8;      // per workgroup: two K halves of four waves
constexpr int kHalfThreads = 256;

struct GemmArgs {
  const uint16_t* x;
  const uint8_t* qp;
  const uint16_t* s;
  const uint8_t* zp;
  uint16_t* y;
  int M, N, K, KT, Gtot, GB, NBLK, sz_vec;
};

// Workgroup barrier that orders LDS only.  __syncthreads() also releases
// global memory, which on gfx9 means waiting for every outstanding global load
// (vmcnt(0)) -- including the prefetches meant to stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

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
  constexpr int ACH = ROWS * 16 / kHalfThreads;  // 16-byte activation chunks per thread and K step
  static_assert(ACH >= 1 && ROWS * 16 % kHalfThreads == 0, "whole chunks per thread");
  constexpr int TILE = ROWS * kArow;              // LDS bytes of one activation tile
  extern __shared__ __align__(16) uint8_t smem[];  // [2 halves][2 buffers][ROWS][kArow]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = wv >> 2, wn = wv & 3;            // K half, column group
  const int th = tid & (kHalfThreads - 1);        // thread index within the half
  const int r = lane & 15, c = lane >> 4;
  const int nbw0 = blockIdx.x * (4 * NPW) + wn * NPW;  // this wave's first column block
  const int mrow0 = blockIdx.y * ROWS;
  const uint32_t magic = in_vgpr(kMagicPair);
  const int KT = a.KT;
  const int S = (KT + 1) / 2;                     // K steps per half (the second may have one less)
  const int kt0 = kh * S, kt_end = min(KT, kt0 + S);
  uint8_t* lds = smem + kh * 2 * TILE;

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
  // activation chunks this thread stages: chunk q = th + 256*i is row
  // q / 16 = th / 16 + 16i, columns 8*(th % 16) .. +8 of the K step (rows past
  // M re-read row M - 1; columns past K re-read the last columns and are never
  // used: K is a multiple of 32, so an MFMA step is wholly inside K or skipped)
  const int xr0 = mrow0 + (th >> 4), xcol = 8 * (th & 15);
  const uint32_t lds_x = (uint32_t)((th >> 4) * kArow + 16 * (th & 15));
  auto load_x = [&](int kt, u4 (&v)[ACH]) {
    kt = min(kt, KT - 1);
    const int col = min(kt * 128 + xcol, a.K - 8);
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const uint32_t row = (uint32_t)min(xr0 + 16 * i, a.M - 1);
      v[i] = *reinterpret_cast<const u4*>(a.x + row * (uint32_t)a.K + col);
    }
  };
  auto store_x = [&](int buf, const u4 (&v)[ACH]) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) *reinterpret_cast<u4*>(lds + buf * TILE + lds_x + i * 16 * kArow) = v[i];
  };
  struct BStep {
    u4 codes[NPW];
    TileSZ<G> sz[NPW];
  };
  f4 acc[MB][NPW];
  auto load_b = [&](int kt, BStep& d) {
    kt = min(kt, KT - 1);  // steps past the end re-load the last (unused)
#pragma unroll
    for (int b = 0; b < NPW; ++b) d.sz[b] = load_tile_sz<G>(a, srow[b], zrow[b], kt);
#pragma unroll
    for (int b = 0; b < NPW; ++b) d.codes[b] = *reinterpret_cast<const u4*>(tb[b] + (size_t)kt * kTileBytes);
  };

#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int b = 0; b < NPW; ++b) acc[i][b] = f4{0.f, 0.f, 0.f, 0.f};

  // ---- prologue: codes of this half's steps 0..2, activations of step 0 in LDS
  static_assert(kBdepth == 3, "the K loop below is unrolled over a ring of four code buffers");
  BStep b0, b1, b2, b3;
  {
    u4 xv[ACH];
    load_x(kt0, xv);
    load_b(kt0, b0);
    load_b(kt0 + 1, b1);
    load_b(kt0 + 2, b2);
    store_x(0, xv);
  }
  lds_barrier();

  // lane (r, c) reads A rows 16i + r, columns 32j + 8c .. +8 of the step
  const uint32_t aread = (uint32_t)(r * kArow + 16 * c);

  // One K step of this half (both halves run the same number of steps and
  // barriers; a half past its last step only keeps the barriers): prefetch the
  // activations of the next step and the codes three steps ahead (into the
  // ring slot the previous step used), multiply with this step's activations
  // from LDS, then store the prefetched activations.  Buffers have fixed ring
  // slots, so nothing still in flight is ever copied.  FULL steps (both
  // halves' tiles whole, next tiles exist) have no branch at all: every load is
  // issued unconditionally (addresses clamped into the arrays), so the
  // compiler's wait counting stays exact and the prefetches stay in flight.
  auto step = [&](auto full_tag, int s, const BStep& cur, BStep& nxt) {
    constexpr bool FULL = decltype(full_tag)::value;
    const int kt = kt0 + s;
    const int buf = s & 1;
    const bool live = FULL || kt < kt_end, more = FULL || kt + 1 < kt_end;
    // activations first: loads complete in issue order, so storing them at the
    // end of the step does not wait for the code prefetch issued after them
    u4 xv[ACH];
    if (more) load_x(kt + 1, xv);
    __builtin_amdgcn_sched_barrier(0);
    load_b(kt + kBdepth, nxt);
    if (live) {
      const uint8_t* abase = lds + buf * TILE + aread;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (!FULL && kt * 128 + 32 * j >= a.K) break;  // ragged last step: no columns left
        h8 af[MB];
#pragma unroll
        for (int i = 0; i < MB; ++i) af[i] = *reinterpret_cast<const h8*>(abase + i * 16 * kArow + 64 * j);
#pragma unroll
        for (int b = 0; b < NPW; ++b) {
          h2 sc, nbias;
          tile_consts<G>(cur.sz[b], kt, j, magic, sc, nbias);
          const h8 bf = dequant_word(cur.codes[b][j], magic, nbias, sc);
#pragma unroll
          for (int i = 0; i < MB; ++i) acc[i][b] = mfma16(af[i], bf, acc[i][b]);
        }
      }
    }
    if (more) store_x(buf ^ 1, xv);
    lds_barrier();
  };
  using Full = std::integral_constant<bool, true>;
  using Part = std::integral_constant<bool, false>;

  // steps where both halves have whole tiles with a successor, in groups of
  // four (the ring size)
  const int s_full = min(a.K / 128 - S, S - 1) & ~3;
  int s0 = 0;
  for (; s0 < s_full; s0 += 4) {
    step(Full{}, s0, b0, b3);
    step(Full{}, s0 + 1, b1, b0);
    step(Full{}, s0 + 2, b2, b1);
    step(Full{}, s0 + 3, b3, b2);
  }
  for (; s0 < S; s0 += 4) {
    step(Part{}, s0, b0, b3);
    if (s0 + 1 < S) step(Part{}, s0 + 1, b1, b0);
    if (s0 + 2 < S) step(Part{}, s0 + 2, b2, b1);
    if (s0 + 3 < S) step(Part{}, s0 + 3, b3, b2);
  }

  // ---- add the second half's sums to the first half's (LDS reused), then
  // lane (r, c) of the first half holds rows 4c..4c+3 of column r of each block
  float* red = reinterpret_cast<float*>(smem);  // [4 column groups][MB*NPW*4][64]
  constexpr int NACC = MB * NPW * 4;
  if (kh == 1) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int b = 0; b < NPW; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[(wn * NACC + (i * NPW + b) * 4 + e) * 64 + lane] = acc[i][b][e];
  }
  lds_barrier();
  if (kh == 1) return;
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int b = 0; b < NPW; ++b) {
      const int n = (nbw0 + b) * 16 + r;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = acc[i][b][e] + red[(wn * NACC + (i * NPW + b) * 4 + e) * 64 + lane];
        const int m = mrow0 + 16 * i + 4 * c + e;
        if (n < a.N && m < a.M) a.y[(size_t)m * a.N + n] = f32_to_f16_bits(v);
      }
    }
}

// Row blocks (MB) and column blocks per wave (NPW) for a problem of M rows.
struct GemmTiles {
  int MB, NPW;
};
GemmTiles gemm_tiles(int64_t M) {
  if (M <= 16) return {1, 1};
  if (M <= 32) return {2, 1};
  if (M <= 64) return {4, 2};
  return {8, 2};
}

dim3 gemm_grid(int MB, int NPW, int64_t M, int64_t N) {
  const int64_t cols = 4 * NPW;  // column blocks per workgroup
  return dim3((unsigned)(((N + 15) / 16 + cols - 1) / cols), (unsigned)((M + 16 * MB - 1) / (16 * MB)));
}

size_t gemm_lds(int MB, int NPW) {
  // two halves x two buffers of activation tiles; the final reduction reuses it
  const size_t lds_tiles = (size_t)4 * 16 * MB * kArow, lds_red = (size_t)4 * MB * NPW * 4 * 64 * sizeof(float);
  return lds_tiles > lds_red ? lds_tiles : lds_red;
}

template <int MB, int NPW>
hipError_t launch_t(int group, const GemmArgs& a, hipStream_t stream) {
  const dim3 grid = gemm_grid(MB, NPW, a.M, a.N), block(kWaves * 64);
  const size_t lds = gemm_lds(MB, NPW);
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

int describe_gemm(int64_t M, int64_t N, int64_t, int group, char* buf, size_t len) {
  const GemmTiles t = gemm_tiles(M);
  const dim3 g = gemm_grid(t.MB, t.NPW, M, N);
  return snprintf(buf, len, "gemm_kernel<MB=%d, NPW=%d, G=%d> grid=(%u,%u,1) block=%d lds=%zu", t.MB, t.NPW, group,
                  g.x, g.y, kWaves * 64, gemm_lds(t.MB, t.NPW));
}

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
  const GemmTiles t = gemm_tiles(M);
  if (t.MB == 1) return launch_t<1, 1>(group, a, stream);
  if (t.MB == 2) return launch_t<2, 1>(group, a, stream);
  if (t.MB == 4) return launch_t<4, 2>(group, a, stream);
  return launch_t<8, 2>(group, a, stream);
}

}  // namespace wq
