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
// 32j + 8c + e, so MFMA step j of a 128-column K tile uses word j as the B
// operand and x[m][32j + 8c .. 32j + 8c + 7] as the A operand.
//
// B dequantization per pair of columns: shift + AND-OR (1024 + q, exact fp16),
// packed fp16 add of -(1024 + z) (exact q - z), packed fp16 multiply by the
// scale (one round-to-nearest-even: fp16(What)).  Accumulation is fp32 in the
// matrix cores.  8-bit codes (group absmax int8, What = s * q): sign-bit flip
// and byte permute (1152 + q, exact fp16), packed subtraction of 1152, packed
// multiply by the scale; each wave's 16-byte load then holds its two MFMA
// steps of a 2048-byte tile.  MXFP4 codes (E2M1, one E8M0 scale per block of
// 32 = one MFMA step): v_cvt_scalef32_pk_f16_fp4 turns each byte of a code
// word into the fp16 pair of E2M1 value times the block's power of two, four
// instructions per operand.
//
// Decomposition.  A workgroup of eight waves (two per SIMD) owns a (16*MB) x
// 128 output tile and walks K one 128-column tile per step, all waves on the
// same tile.  Wave w = 4p + cg takes MFMA steps 2p and 2p + 1 of every tile
// for the two 16-column blocks of column group cg: it dequantizes its own B
// operands in registers (no weight is dequantized twice), using two of the
// four code words in each lane's 16 bytes, loaded three tiles ahead into a
// four-slot register ring.  The activations of a tile are staged in LDS once
// for the workgroup: every thread loads whole 256-byte row segments with
// 16-byte loads (sixteen threads per row) three tiles ahead of use into one
// of two register sets and stores them, one tile before their use, into one
// of two LDS buffers; chunk cc of row R sits in slot cc ^ (R % 16) of its row, so the
// A-operand reads (lane l = r + 16c takes chunk 4j + c of row 16i + r) spread
// over all banks.  Scales and zero-points of eight tiles at a time are staged
// into LDS with wide loads (a row's scales for eight tiles in one load instead
// of one load per tile), half a chunk ahead.  The steady state runs in groups
// of eight tiles without a branch, so the compiler's wait counts stay exact
// and every load stays in flight until its first use; barriers order LDS only
// (__syncthreads() on gfx9 would also wait for every outstanding global load).
// At the end the second step pair's sums are added to the first pair's
// through LDS, in a fixed order.  A grid too small to fill the GPU (few
// 128-column blocks) splits K across workgroups in runs of whole eight-tile
// chunks: each split writes fp32 partial sums to the workspace, and the last
// workgroup of an output tile (a device-scope counter) adds them in split order,
// writes y and puts the counter back to zero.
#include <stdio.h>

#include <algorithm>
#include <type_traits>

#include "wq_device.h"
#include "wq_kernels.h"

namespace wq {
namespace {

constexpr int kWaves = 8;     // per workgroup: four column groups x two MFMA-step pairs
constexpr int kSzChunk = 8;   // K tiles per staged chunk of scales / zero-points
constexpr int kNPW = 2;       // 16-column blocks per wave (eight per workgroup)

struct GemmArgs {
  const uint16_t* x;
  const uint8_t* qp;
  const uint16_t* s;
  const uint8_t* zp;
  uint16_t* y;
  float* partial;      // [KS][M][N] fp32 (KS > 1 only)
  unsigned* counters;  // [gridDim.y][gridDim.x] (KS > 1 only)
  const float* tscale; // NVFP4: the per-tensor scale (device)
  int M, N, K, KT, Gtot, GB, NBLK, kt_per_split, KS;
};

// Workgroup barrier that orders LDS only.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ f4 mfma16(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// A raw buffer of `bytes` bytes at `base` (32-bit data format, no swizzle).
// Loads take a per-lane offset and a wave-uniform offset; only the per-lane
// one takes part in the buffer's range check, so callers keep both inside
// the buffer themselves.
constexpr uint32_t kBufferFlags = 0x00020000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, (int)kBufferFlags);
}

// Forces a value into a VGPR and hides it from constant folding, so that
// v_and_or_b32 takes the mask from an SGPR and the fp16 exponent from here.
__device__ __forceinline__ uint32_t in_vgpr(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// fp16(E2M1(q) * 2^e) for the eight columns of an MXFP4 code word (column e in
// nibble e); the scale's exponent field gives e.
__device__ __forceinline__ h8 dequant_word_mx(uint32_t w, float scale) {
  const h2 p0 = fp4_pair<0>(w, scale), p1 = fp4_pair<1>(w, scale), p2 = fp4_pair<2>(w, scale),
           p3 = fp4_pair<3>(w, scale);
  h8 out;
  out[0] = p0[0]; out[1] = p0[1]; out[2] = p1[0]; out[3] = p1[1];
  out[4] = p2[0]; out[5] = p2[1]; out[6] = p3[0]; out[7] = p3[1];
  return out;
}

// fp16(s * q) for the eight columns held by two words of 8-bit codes.
__device__ __forceinline__ h8 dequant_words8(uint32_t lo, uint32_t hi, h2 sc) {
  const h2 bias = as_h2(0x64806480u);  // (1152, 1152)
  lo ^= 0x80808080u;
  hi ^= 0x80808080u;
  const h2 p0 = (as_h2(byte_pair(lo, 0x04010400u)) - bias) * sc;
  const h2 p1 = (as_h2(byte_pair(lo, 0x04030402u)) - bias) * sc;
  const h2 p2 = (as_h2(byte_pair(hi, 0x04010400u)) - bias) * sc;
  const h2 p3 = (as_h2(byte_pair(hi, 0x04030402u)) - bias) * sc;
  h8 out;
  out[0] = p0[0]; out[1] = p0[1]; out[2] = p1[0]; out[3] = p1[1];
  out[4] = p2[0]; out[5] = p2[1]; out[6] = p3[0]; out[7] = p3[1];
  return out;
}

// LDS bytes of one staged chunk of scales / zero-points (kSzChunk tiles) for
// the workgroup's 128 weight rows:
//   4-bit and int8 codes, g = 128: [tile][row] 8 bytes: the scale as an fp16
//     pair (s, s), then the fp16 pair -(1024 + z) (4-bit; zero for int8);
//   g = 32: [tile][step pair jp][row] 16 bytes: those two pairs for group
//     4t + 2jp, then for group 4t + 2jp + 1;
//   MXFP4: [tile][row] u32, the tile's four E8M0 scale bytes, block 4t first;
//   NVFP4: [tile][row] 16 bytes, the tile's eight E4M3 block scales as fp16.
template <int G, int FMT = kFmtInt4>
constexpr int sz_chunk_bytes() {
  return FMT == kFmtMxfp4   ? kSzChunk * 128 * 4
         : FMT == kFmtNvfp4 ? kSzChunk * 128 * 16
         : G == 128         ? kSzChunk * 128 * 8
                            : kSzChunk * 2 * 128 * 16;
}

// The fp16 pair -(1024 + z) (exact) as bits.
__device__ __forceinline__ uint32_t neg_bias_pair(uint32_t z) { return (0xE400u | z) * 0x00010001u; }

// fp16(s * (q - z)) for the eight columns of one packed word, given the scale
// pair and the pairs -(1024 + z) and -(64 + z): columns 0, 1 and 4, 5 come as
// 1024 + q (low code bits), columns 2, 3 and 6, 7 as 64 + q (code bits 4..7
// under the exponent of 64, whose unit spacing is 2^-4).
__device__ __forceinline__ h8 dequant_word(uint32_t w, uint32_t m1024, uint32_t m64, h2 nb, h2 nb64, h2 sc) {
  const uint32_t w8 = w >> 8;
  const h2 p0 = (as_h2((w & 0x000F000Fu) | m1024) + nb) * sc;
  const h2 p1 = (as_h2((w & 0x00F000F0u) | m64) + nb64) * sc;
  const h2 p2 = (as_h2((w8 & 0x000F000Fu) | m1024) + nb) * sc;
  const h2 p3 = (as_h2((w8 & 0x00F000F0u) | m64) + nb64) * sc;
  h8 out;
  out[0] = p0[0]; out[1] = p0[1]; out[2] = p1[0]; out[3] = p1[1];
  out[4] = p2[0]; out[5] = p2[1]; out[6] = p3[0]; out[7] = p3[1];
  return out;
}

// SZV: every row of s (and zpacked) is aligned for the wide staging loads.
// FMT: kFmtInt4 (codes and zero-points), kFmtInt8 (int8 codes, no
// zero-points) or kFmtMxfp4 (E2M1 codes, E8M0 scale bytes in a.zp, G = 32).
//
// Software pipeline.  Each K tile is two phases of a wave: phase A runs the
// MFMAs of the wave's first step of the tile (step 2jp) while it reads the A
// fragments of its second step from LDS and dequantizes that step's B
// operands; phase B runs the second step's MFMAs while it prepares the next
// tile's first step the same way.  So the matrix cores always have operands
// that were formed one phase earlier, and the LDS reads and dequantization
// overlap the MFMAs of the other phase.  One barrier per tile, between its
// two phases: the activations of tile kt + 1 are stored in phase A (into the
// buffer tile kt - 1 used, whose last reads were in phase A of step kt - 1,
// before that step's barrier) and first read in phase B.
template <int MB, int G, bool SZV, int FMT>
__global__ __launch_bounds__(kWaves * 64) void gemm_kernel(GemmArgs a) {
  static_assert(FMT == kFmtInt4 || FMT == kFmtInt8 || (FMT == kFmtMxfp4 && G == 32) || (FMT == kFmtNvfp4 && G == 16),
                "code format");
  constexpr int BITS = FMT == kFmtInt8 ? 8 : 4;
  using CodeT = std::conditional_t<BITS == 4, uint2, u4>;  // one wave's two MFMA steps of a tile
  constexpr int TB = BITS == 4 ? kTileBytes : kTileBytes8;
  constexpr int NPW = kNPW;
  constexpr int NTH = kWaves * 64;
  constexpr int ROWS = 16 * MB;
  constexpr int XTILE = ROWS * 256;                            // one K tile of activations in LDS
  constexpr int XCH = ROWS * 16 >= NTH ? ROWS * 16 / NTH : 1;  // 16-byte chunks per thread per tile
  constexpr int SZB = sz_chunk_bytes<G, FMT>();
  constexpr int SZW = FMT == kFmtMxfp4 || FMT == kFmtNvfp4 ? 1 : 2;  // staged words per block and step
  static_assert(ROWS * 16 % NTH == 0 || NTH % (ROWS * 16) == 0, "whole chunks per thread");
  extern __shared__ __align__(16) uint8_t smem[];  // [2][XTILE] activations, [2][SZB] scales

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int jp = wv >> 2, cgp = wv & 3;
  const int r = lane & 15, c = lane >> 4;
  const int nwg0 = blockIdx.x * 8 * 16;  // first weight row of the workgroup
  const int nbw0 = blockIdx.x * 8 + cgp * NPW;
  const int mrow0 = blockIdx.y * ROWS;
  const uint32_t m1024 = in_vgpr(kMagicPair), m64 = in_vgpr(0x54005400u);
  const int KT = a.KT;

  // the codes of MFMA steps 2jp, 2jp + 1 in each of the wave's blocks: 4-bit,
  // words 2jp and 2jp + 1 of the lane's 16 bytes; 8-bit, the lane's 16 bytes
  // of half jp.  One buffer over the wave's blocks: the lane's offset in a
  // tile is fixed, the tile and block offsets are wave-uniform (blocks past
  // the end re-read the last one, tiles past the end the last one).
  // (wave-uniform values; the explicit readfirstlane keeps the compiler from
  // treating the buffer descriptor as per-lane)
  const int qb0 = __builtin_amdgcn_readfirstlane(min(nbw0, a.NBLK - 1));
  const int qbn = __builtin_amdgcn_readfirstlane(min(nbw0 + NPW - 1, a.NBLK - 1) - qb0 + 1);
  const __amdgpu_buffer_rsrc_t qres = buffer_of(a.qp + (size_t)qb0 * KT * TB, (uint32_t)(qbn * KT * TB));
  const uint32_t qvoff = 16u * lane + (BITS == 4 ? 8u : 1024u) * jp;
  // With few rows (MB <= 2) the kernel streams codes at HBM speed and
  // non-temporal loads measure faster; with more rows they do not.
  constexpr int kCodeAux = MB > 2 ? 0 : 2;  // cache policy: non-temporal
  auto load_b = [&](int kt, CodeT (&d)[NPW]) {
    kt = min(kt, KT - 1);
#pragma unroll
    for (int b = 0; b < NPW; ++b) {
      const uint32_t so = (uint32_t)(min(b, qbn - 1) * KT + kt) * TB;
      if constexpr (BITS == 4)
        d[b] = __builtin_bit_cast(CodeT, __builtin_amdgcn_raw_buffer_load_b64(qres, qvoff, so, kCodeAux));
      else
        d[b] = __builtin_bit_cast(CodeT, __builtin_amdgcn_raw_buffer_load_b128(qres, qvoff, so, kCodeAux));
    }
  };

  // activation chunk q = tid + NTH * i: row q / 16 of the tile, global chunk
  // q % 16 (with fewer chunks than threads, threads share chunks and store
  // the same bytes); rows past M re-read row M - 1.  The loads of tile kt go
  // through a buffer that starts at column 128 kt of the workgroup's first
  // row and ends with its last row, so the lane's offset (its row and chunk)
  // is fixed and range-checked: in a ragged last tile, chunks past K read
  // the next row's first columns, or zeros past the last row (K is a
  // multiple of 32, so an MFMA step lies wholly inside K or is skipped).
  const int xrows = min(a.M - mrow0, ROWS);
  const uint16_t* const xbase = a.x + (size_t)mrow0 * a.K;
  uint32_t xvoff[XCH];
  uint32_t xlds[XCH];
  const int xcc = tid & 15;
#pragma unroll
  for (int i = 0; i < XCH; ++i) {
    const int row = ((tid >> 4) + (NTH / 16) * i) % ROWS;
    xvoff[i] = (uint32_t)min(row, xrows - 1) * a.K * 2u + 16u * xcc;
    xlds[i] = (uint32_t)(row * 256 + 16 * (xcc ^ (row & 15)));
  }
  auto load_x = [&](int kt, u4 (&v)[XCH]) {
    kt = min(kt, KT - 1);
    const __amdgpu_buffer_rsrc_t xres = buffer_of(xbase + kt * 128, (uint32_t)(xrows * a.K - kt * 128) * 2u);
#pragma unroll
    for (int i = 0; i < XCH; ++i)
      v[i] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(xres, xvoff[i], 0u, 0));
  };
  auto store_x = [&](int kt, const u4 (&v)[XCH]) {
#pragma unroll
    for (int i = 0; i < XCH; ++i) *reinterpret_cast<u4*>(smem + (kt & 1) * XTILE + xlds[i]) = v[i];
  };

  // ---- scale / zero-point staging: thread (row n = tid / 4, part p = tid % 4)
  // covers tiles 2p, 2p + 1 of a chunk (groups past the end re-read the last)
  const int sn = tid >> 2, sp = tid & 3;
  const size_t srow = (size_t)min(nwg0 + sn, a.N - 1) * a.Gtot;
  const size_t zrow = (size_t)min(nwg0 + sn, a.N - 1) * a.GB;
  struct SzStage {
    uint32_t s[4], z;
  };
  auto sz_load = [&](int chunk, SzStage& v) {
    const int t0 = chunk * kSzChunk + 2 * sp;  // first of this thread's two tiles
    if constexpr (FMT == kFmtMxfp4) {  // eight scale bytes: blocks 4 t0 .. 4 t0 + 7
      if constexpr (SZV) {  // Gtot % 8 == 0
        const uint2 t = *reinterpret_cast<const uint2*>(a.zp + srow + min(4 * t0, a.Gtot - 8));
        v.s[0] = t.x;
        v.s[1] = t.y;
      } else {
        uint32_t b[2] = {0u, 0u};
#pragma unroll
        for (int q = 0; q < 8; ++q) b[q >> 2] |= (uint32_t)a.zp[srow + min(4 * t0 + q, a.Gtot - 1)] << (8 * (q & 3));
        v.s[0] = b[0];
        v.s[1] = b[1];
      }
      v.z = 0u;
    } else if constexpr (FMT == kFmtNvfp4) {  // sixteen scale bytes: blocks 8 t0 .. 8 t0 + 15
      if constexpr (SZV) {  // Gtot % 16 == 0
        const u4 t = *reinterpret_cast<const u4*>(a.zp + srow + min(8 * t0, a.Gtot - 16));
        v.s[0] = t.x; v.s[1] = t.y; v.s[2] = t.z; v.s[3] = t.w;
      } else {
        uint32_t b[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int q = 0; q < 16; ++q) b[q >> 2] |= (uint32_t)a.zp[srow + min(8 * t0 + q, a.Gtot - 1)] << (8 * (q & 3));
        v.s[0] = b[0]; v.s[1] = b[1]; v.s[2] = b[2]; v.s[3] = b[3];
      }
      v.z = 0u;
    } else if constexpr (G == 128) {
      if constexpr (SZV) {  // Gtot even: one u32 holds both scales
        v.s[0] = *reinterpret_cast<const uint32_t*>(a.s + srow + min(t0, a.Gtot - 2));
      } else {
        v.s[0] = a.s[srow + min(t0, a.Gtot - 1)];
        v.s[1] = a.s[srow + min(t0 + 1, a.Gtot - 1)];
      }
      v.z = FMT == kFmtInt4 ? a.zp[zrow + (min(t0, a.Gtot - 1) >> 1)] : 0u;
    } else {
      if constexpr (SZV) {  // Gtot % 8 == 0: 16 bytes of scales, 4 bytes of zero-points
        const int g = min(4 * t0, a.Gtot - 8);
        const u4 t = *reinterpret_cast<const u4*>(a.s + srow + g);
        v.s[0] = t.x; v.s[1] = t.y; v.s[2] = t.z; v.s[3] = t.w;
        v.z = FMT == kFmtInt4 ? *reinterpret_cast<const uint32_t*>(a.zp + zrow + g / 2) : 0u;
      } else {
        uint32_t zz = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int g0 = min(4 * t0 + 2 * q, a.Gtot - 1), g1 = min(4 * t0 + 2 * q + 1, a.Gtot - 1);
          v.s[q] = (uint32_t)a.s[srow + g0] | ((uint32_t)a.s[srow + g1] << 16);
          if constexpr (FMT == kFmtInt4) {
            const uint32_t zb0 = a.zp[zrow + (g0 >> 1)], zb1 = a.zp[zrow + (g1 >> 1)];
            zz |= (((g0 & 1) ? zb0 >> 4 : zb0 & 15u) | (((g1 & 1) ? zb1 >> 4 : zb1 & 15u) << 4)) << (8 * q);
          }
        }
        v.z = zz;
      }
    }
  };
  uint8_t* const szbase = smem + 2 * XTILE;
  // scale pair and -(1024 + z) pair of one group (int8: no zero-point)
  auto entry = [&](uint32_t s16, uint32_t z) -> uint2 {
    return uint2{(s16 & 0xffffu) * 0x00010001u, FMT == kFmtInt4 ? neg_bias_pair(z & 15u) : 0u};
  };
  auto sz_store = [&](int chunk, const SzStage& v) {
    uint8_t* buf = szbase + (chunk & 1) * SZB;
    if constexpr (FMT == kFmtMxfp4) {
      *reinterpret_cast<uint32_t*>(buf + (2 * sp) * 512 + 4 * sn) = v.s[0];
      *reinterpret_cast<uint32_t*>(buf + (2 * sp + 1) * 512 + 4 * sn) = v.s[1];
    } else if constexpr (FMT == kFmtNvfp4) {
      // tile 2p + e: bytes of s[2e], s[2e + 1] (blocks 8 t .. 8 t + 7) as fp16
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        uint32_t h[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t wd = v.s[2 * e + (k >> 1)];
          h[k] = as_u32((k & 1) ? e4m3_pair_f16<true>(wd) : e4m3_pair_f16<false>(wd));
        }
        *reinterpret_cast<u4*>(buf + ((2 * sp + e) * 128 + sn) * 16) = u4{h[0], h[1], h[2], h[3]};
      }
    } else if constexpr (G == 128) {
      const uint32_t s0 = SZV ? v.s[0] & 0xffffu : v.s[0];
      const uint32_t s1 = SZV ? v.s[0] >> 16 : v.s[1];
      // tiles 2p (low nibble) and 2p + 1 (high nibble) share a zero-point byte
      *reinterpret_cast<uint2*>(buf + ((2 * sp) * 128 + sn) * 8) = entry(s0, v.z);
      *reinterpret_cast<uint2*>(buf + ((2 * sp + 1) * 128 + sn) * 8) = entry(s1, v.z >> 4);
    } else {
      // the thread's eight groups: i = 4e + q for tile 2p + e; scale i in half
      // i % 2 of s[i / 2], zero-point i in nibble i of z
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int i = 4 * e + 2 * h;
          const uint2 ea = entry(v.s[i >> 1], v.z >> (4 * i)), eb = entry(v.s[i >> 1] >> 16, v.z >> (4 * i + 4));
          *reinterpret_cast<u4*>(buf + (((2 * sp + e) * 2 + h) * 128 + sn) * 16) = u4{ea.x, ea.y, eb.x, eb.y};
        }
    }
  };

  f4 acc[MB][NPW];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int b = 0; b < NPW; ++b) acc[i][b] = f4{0.f, 0.f, 0.f, 0.f};

  // this workgroup's K tiles [kt_lo, kt_hi): all of K, or one split (kt_lo a
  // multiple of the eight-tile chunk)
  const int kt_lo = blockIdx.z * a.kt_per_split;
  const int kt_hi = min(KT, kt_lo + a.kt_per_split);

  // this lane's A reads: row r of block i, chunk 4j + c at slot (4j + c) ^ r;
  // its scale / zero entries: rows (cg*NPW + b)*16 + r of the workgroup
  const uint8_t* const arow = smem + r * 256;
  const int szrow = cgp * NPW * 16 + r;

  // staged scale / zero-point words of one step (jj) of tile kt for the
  // wave's blocks: the scale pair and the -(1024 + z) pair (MXFP4: the tile's
  // scale bytes)
  struct SzRegs {
    uint32_t w[NPW][SZW];
  };
  auto read_sz = [&](int kt, int jj, SzRegs& v) {
    const uint8_t* szt = szbase + ((kt / kSzChunk) & 1) * SZB;
    const int tt = kt % kSzChunk;
#pragma unroll
    for (int b = 0; b < NPW; ++b) {
      const int row = szrow + 16 * b;
      if constexpr (FMT == kFmtMxfp4) {
        v.w[b][0] = *reinterpret_cast<const uint32_t*>(szt + tt * 512 + 4 * row);
      } else if constexpr (FMT == kFmtNvfp4) {
        // the lane's eight columns of step j lie in block 2j + c / 2 of the tile
        const int j = 2 * jp + jj;
        v.w[b][0] = *reinterpret_cast<const uint16_t*>(szt + (tt * 128 + row) * 16 + 2 * (2 * j + (c >> 1)));
      } else {
        const uint2 t = *reinterpret_cast<const uint2*>(
            szt + (G == 128 ? (tt * 128 + row) * 8 : ((tt * 2 + jp) * 128 + row) * 16 + 8 * jj));
        v.w[b][0] = t.x;
        v.w[b][1] = t.y;
      }
    }
  };
  // A fragments of step jj (MFMA step 2jp + jj) of tile kt, from its LDS buffer
  auto read_a = [&](int kt, int jj, h8 (&af)[MB]) {
    const int j = 2 * jp + jj;
    const uint8_t* abuf = arow + (kt & 1) * XTILE + ((4 * j + c) ^ r) * 16;
#pragma unroll
    for (int i = 0; i < MB; ++i) af[i] = *reinterpret_cast<const h8*>(abuf + i * 16 * 256);
  };
  // B operands of step jj of tile kt (kt only picks the MXFP4 scale byte)
  auto deq = [&](int kt, int jj, const CodeT (&cur)[NPW], const SzRegs& sz, h8 (&bf)[NPW]) {
#pragma unroll
    for (int b = 0; b < NPW; ++b) {
      if constexpr (FMT == kFmtMxfp4) {
        // block 4 kt + j: byte j of the tile's scale word (exponent field only)
        const int j = 2 * jp + jj;
        const float scale = __builtin_bit_cast(float, ((sz.w[b][0] >> (8 * j)) & 0xffu) << 23);
        bf[b] = dequant_word_mx(jj ? cur[b].y : cur[b].x, scale);
      } else if constexpr (FMT == kFmtNvfp4) {
        // E2M1 values (exact) times the block's E4M3 scale: exact in fp16
        const h8 v = dequant_word_mx(jj ? cur[b].y : cur[b].x, 1.0f);
        const _Float16 s = __builtin_bit_cast(_Float16, (uint16_t)sz.w[b][0]);
        bf[b] = v * s;
      } else if constexpr (FMT == kFmtInt4) {
        const h2 nb = as_h2(sz.w[b][1]), nb64 = nb + h2{(_Float16)960.0f, (_Float16)960.0f};  // -(64 + z), exact
        bf[b] = dequant_word(jj ? cur[b].y : cur[b].x, m1024, m64, nb, nb64, as_h2(sz.w[b][0]));
      } else {
        bf[b] = dequant_words8(jj ? cur[b][2] : cur[b][0], jj ? cur[b][3] : cur[b][1], as_h2(sz.w[b][0]));
      }
    }
  };
  auto mma = [&](const h8 (&af)[MB], const h8 (&bf)[NPW]) {
#pragma unroll
    for (int b = 0; b < NPW; ++b)
#pragma unroll
      for (int i = 0; i < MB; ++i) acc[i][b] = mfma16(af[i], bf[b], acc[i][b]);
  };
  // in a ragged last tile, a step that starts at or past K is skipped
  auto step_in_k = [&](int kt, int jj) { return kt * 128 + 32 * (2 * jp + jj) < a.K; };

  // ---- prologue: activations of the first tile (in LDS) and of the second
  // and third (in registers), codes of the first three tiles, scales /
  // zero-points of the first chunk; then the operands of the first tile's
  // first step
  // the code ring: RING slots, loaded RING - 1 tiles ahead
  constexpr int RING = 4;
  CodeT ring[RING][NPW];
  u4 xs[2][XCH];  // activations of even / odd tiles
  SzStage szs;
  // scales / zero-points for the dequantization: with EARLY_SZ (below) two
  // sets, step 0 of alternate tiles; otherwise one, read before each use
  // READS_FIRST: phase A issues its LDS reads before anything else (below);
  // EARLY_SZ: phase A also reads step 0 of the next tile's scales (one group
  // per tile).  Both take registers: the 128-row int8 instances and the ones
  // with unaligned scale rows do not have them to spare (they would spill
  // inside the K loop); the 4-bit g = 32 instance reloads two loop-invariant
  // values per eight tiles and still measured 2 % faster.
  constexpr bool READS_FIRST =
      MB <= 4 || (FMT == kFmtInt4 && (G == 128 || SZV)) || ((FMT == kFmtMxfp4 || FMT == kFmtNvfp4) && SZV);
  constexpr bool EARLY_SZ = READS_FIRST && G == 128;
  constexpr int NSZ = EARLY_SZ ? 2 : 1;
  SzRegs szr[NSZ];
  h8 af0[MB], af1[MB], bf0[NPW], bf1[NPW];
  load_x(kt_lo, xs[0]);
  load_x(kt_lo + 1, xs[1]);
#pragma unroll
  for (int s = 0; s < RING - 1; ++s) load_b(kt_lo + s, ring[s]);
  sz_load(kt_lo / kSzChunk, szs);
  store_x(kt_lo, xs[0]);
  load_x(kt_lo + 2, xs[0]);
  sz_store(kt_lo / kSzChunk, szs);
  lds_barrier();
  read_sz(kt_lo, 0, szr[0]);
  read_a(kt_lo, 0, af0);
  deq(kt_lo, 0, ring[0], szr[0], bf0);

  // One tile kt.  xs: the register set holding the activations of tile
  // kt + 1 (loaded two tiles earlier), which are stored to LDS and replaced
  // by those of tile kt + 3.  cur: codes of tile kt; nxt: codes of tile
  // kt + 1; ld: the ring slot that receives tile kt + RING - 1.
  // szc: the set holding step 0 of tile kt's scales / zero-points; szn: the
  // set that receives step 0 of tile kt + 1's (the same set without
  // EARLY_SZ).  EARLY_SZ reads szn in phase A, which saves phase B a wait on
  // LDS (one group per tile: step 1 reuses szc).
  auto tile = [&](auto full_tag, int kt, u4 (&xs)[XCH], const CodeT (&cur)[NPW], const CodeT (&nxt)[NPW],
                  CodeT (&ld)[NPW], SzRegs& szc, SzRegs& szn) {
    constexpr bool FULL = decltype(full_tag)::value;
    // phase A: MFMAs of step 0 (operands formed earlier); prepare step 1.
    // With READS_FIRST the phase's LDS reads go first: the barrier at the
    // end of the phase waits for every LDS access of the wave, so reads
    // issued late would expose their whole latency there.
    if constexpr (READS_FIRST) {
      if constexpr (EARLY_SZ) read_sz(kt + 1, 0, szn);  // (staged half a chunk ahead)
      else read_sz(kt, 1, szc);
      read_a(kt, 1, af1);
      __builtin_amdgcn_sched_barrier(0);
    }
    store_x(kt + 1, xs);
    load_x(kt + 3, xs);
    __builtin_amdgcn_sched_barrier(0);
    load_b(kt + RING - 1, ld);
    if constexpr (!READS_FIRST) {
      read_sz(kt, 1, szc);
      read_a(kt, 1, af1);
    }
    deq(kt, 1, cur, szc, bf1);
    if (FULL || step_in_k(kt, 0)) mma(af0, bf0);
    lds_barrier();
    // phase B: MFMAs of step 1; prepare step 0 of tile kt + 1
    if constexpr (!EARLY_SZ) read_sz(kt + 1, 0, szn);
    read_a(kt + 1, 0, af0);
    deq(kt + 1, 0, nxt, szn, bf0);
    if (FULL || step_in_k(kt, 1)) mma(af1, bf1);
  };
  using Full = std::integral_constant<bool, true>;
  using Part = std::integral_constant<bool, false>;

  // whole tiles in groups of eight (one or two turns of the code ring, four
  // of the activation registers); the next chunk's scales / zero-points are
  // loaded at tile 1 and stored at tile 4
  const int kt_full = kt_lo + ((min(kt_hi, a.K / 128) - kt_lo) & ~(kSzChunk - 1));
  int kt = kt_lo;
  for (; kt < kt_full; kt += kSzChunk) {
    const int ch = kt / kSzChunk;
#pragma unroll
    for (int u = 0; u < kSzChunk; ++u) {
      if (u == 1) sz_load(ch + 1, szs);
      if (u == 4) sz_store(ch + 1, szs);
      tile(Full{}, kt + u, xs[(u + 1) % 2], ring[u % RING], ring[(u + 1) % RING], ring[(u + RING - 1) % RING],
           szr[u % NSZ], szr[(u + 1) % NSZ]);
    }
  }
  // the rest (fewer than eight tiles, the last one possibly ragged); their
  // chunk was staged during the previous chunk or before the loop
  if (kt < kt_hi) {
#pragma unroll
    for (int u = 0; u < kSzChunk; ++u)
      if (kt + u < kt_hi)
        tile(Part{}, kt + u, xs[(u + 1) % 2], ring[u % RING], ring[(u + 1) % RING], ring[(u + RING - 1) % RING],
             szr[u % NSZ], szr[(u + 1) % NSZ]);
  }

  // every wave's last LDS reads are done before the reduction reuses LDS
  lds_barrier();
  // NVFP4: the per-tensor scale multiplies each output (partial sums stay unscaled)
  const float ys = FMT == kFmtNvfp4 ? *a.tscale : 1.0f;

  // ---- add the second step pair's sums to the first's (LDS reused), then
  // lane (r, c) of the first pair holds rows 4c..4c+3 of column r of each block
  float* red = reinterpret_cast<float*>(smem);  // [column group][MB*NPW*4][64]
  constexpr int NACC = MB * NPW * 4;
  if (jp == 1) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int b = 0; b < NPW; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[(cgp * NACC + (i * NPW + b) * 4 + e) * 64 + lane] = acc[i][b][e];
  }
  lds_barrier();
  if (jp == 0) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int b = 0; b < NPW; ++b) {
        const int n = (nbw0 + b) * 16 + r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = acc[i][b][e] + red[(cgp * NACC + (i * NPW + b) * 4 + e) * 64 + lane];
          const int m = mrow0 + 16 * i + 4 * c + e;
          if (a.KS > 1)  // padded plane: every element of the tile is inside it
            split_store(a.partial + ((size_t)blockIdx.z * gridDim.y * ROWS + m) * (gridDim.x * 128) + n, v);
          else if (n < a.N && m < a.M)
            a.y[(size_t)m * a.N + n] = f32_to_f16_bits(FMT == kFmtNvfp4 ? v * ys : v);
        }
      }
  }
  if (a.KS == 1) return;

  // ---- split K: the last workgroup of this output tile adds the partial sums
  unsigned* ctr = a.counters + blockIdx.y * gridDim.x + blockIdx.x;
  if (!split_arrive(ctr, a.KS)) return;
  {
    // every thread sums, in split order, one column of the tile at rows
    // row0 + 4j: consecutive threads read consecutive columns (coalesced) and
    // a thread's loads differ by a uniform stride, all in flight together
    constexpr int RPP = NTH / 128, PER = ROWS / RPP;  // rows per pass, elements per thread
    const int col = tid & 127, row0 = tid / 128;
    const size_t Np = (size_t)gridDim.x * 128, plane = (size_t)gridDim.y * ROWS * Np;
    const float* base = a.partial + (size_t)(mrow0 + row0) * Np + blockIdx.x * 128 + col;
    float v[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) v[j] = 0.0f;
    for (int k2 = 0; k2 < a.KS; ++k2) {
      float t[PER];
#pragma unroll
      for (int j = 0; j < PER; ++j) t[j] = split_load(base + k2 * plane + (size_t)(RPP * j) * Np);
#pragma unroll
      for (int j = 0; j < PER; ++j) v[j] += t[j];
    }
    const int n = blockIdx.x * 128 + col;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int m = mrow0 + row0 + RPP * j;
      if (n < a.N && m < a.M) a.y[(size_t)m * a.N + n] = f32_to_f16_bits(FMT == kFmtNvfp4 ? v[j] * ys : v[j]);
    }
  }
  if (tid == 0) split_reset(ctr);
}

// Row blocks per workgroup for a problem of M rows, N columns and depth K.
// Eight row blocks (128 rows) per workgroup only when the grid has enough
// 128-column blocks to fill the GPU: with fewer of them (N below 24,576) four
// row blocks give twice the workgroups before K is split, and fewer split
// planes to write and add, and with very few (N below 4,096) two do (M=128:
// N=K=8192 31.8 -> 29.2 us with four; N=1024, K=8192 24.1 -> 16.8 us with
// four, 13.3 us with two; at N=28672 eight measured 8 % faster than four).
// Fewer row blocks dequantize every weight once per block of rows, which a
// long K does not repay: at N=8192, K=28672 four measured 91 us against 81
// with eight, so the smaller blocks are used only up to K = 16384.
int gemm_mb(int64_t M, int64_t N, int64_t K) {
  const int64_t gx = ((N + 15) / 16 + 7) / 8;
  const bool short_k = K <= 16384;
  return M <= 16 ? 1 : (M <= 32 || (short_k && gx < 32)) ? 2 : (M <= 64 || (short_k && gx < 192)) ? 4 : 8;
}

// Launch shape: (128-column blocks, 16*MB-row blocks, K splits).  A grid of
// fewer than 192 workgroups splits K so that about 256 run (one per CU), in
// runs of whole eight-tile chunks.
struct GemmPlan {
  int MB, KS, kt_per_split;
  unsigned gx, gy;
};

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K) {
  GemmPlan p;
  p.MB = gemm_mb(M, N, K);
  p.gx = (unsigned)(((N + 15) / 16 + 7) / 8);
  p.gy = (unsigned)((M + 16 * p.MB - 1) / (16 * p.MB));
  const int KT = (int)((K + 127) / 128);
  const int64_t wgs = (int64_t)p.gx * p.gy;
  int ks = 1;
  if (wgs < 192 && wgs <= kSplitMaxTiles)
    ks = (int)std::min<int64_t>((256 + wgs - 1) / wgs, std::max(1, KT / kSzChunk));
  p.kt_per_split = (KT + ks - 1) / ks;
  p.kt_per_split = (p.kt_per_split + kSzChunk - 1) / kSzChunk * kSzChunk;
  p.KS = (KT + p.kt_per_split - 1) / p.kt_per_split;
  return p;
}

size_t gemm_lds(int MB, int group, int fmt) {
  // two activation buffers and two staged chunks of scales / zero-points; the
  // final reduction ([4][MB*NPW*4][64] fp32) reuses the front of it
  const size_t tiles =
      (size_t)2 * MB * 16 * 256 +
      2 * (size_t)(fmt == kFmtMxfp4   ? sz_chunk_bytes<32, kFmtMxfp4>()
                   : fmt == kFmtNvfp4 ? sz_chunk_bytes<16, kFmtNvfp4>()
                   : group == 128     ? sz_chunk_bytes<128>()
                                      : sz_chunk_bytes<32>());
  const size_t red = (size_t)4 * MB * kNPW * 4 * 64 * sizeof(float);
  return tiles > red ? tiles : red;
}

template <int MB, int G, bool SZV, int FMT>
hipError_t launch_kg(const GemmPlan& p, const GemmArgs& a, hipStream_t stream) {
  const dim3 grid(p.gx, p.gy, (unsigned)p.KS), block(kWaves * 64);
  const size_t lds = gemm_lds(MB, G, FMT);
  auto k = gemm_kernel<MB, G, SZV, FMT>;
  static std::atomic<uint64_t> lds_raised{0};
  const hipError_t e = raise_lds_limit((const void*)k, lds, lds_raised);
  if (e != hipSuccess) return e;
  k<<<grid, block, lds, stream>>>(a);
  return hipGetLastError();
}

template <int MB, int FMT>
hipError_t launch_t(int group, const GemmPlan& p, const GemmArgs& a, hipStream_t stream) {
  // wide staging loads of scales / zero-points when every row is aligned for
  // them: g = 128 two scales (4 bytes); g = 32 eight scales (16 bytes) and
  // eight zero-points (4 bytes); MXFP4 eight scale bytes
  const uintptr_t sp = reinterpret_cast<uintptr_t>(a.s), zp = reinterpret_cast<uintptr_t>(a.zp);
  if constexpr (FMT == kFmtMxfp4) {
    if (a.Gtot % 8 == 0 && zp % 8 == 0) return launch_kg<MB, 32, true, FMT>(p, a, stream);
    return launch_kg<MB, 32, false, FMT>(p, a, stream);
  } else if constexpr (FMT == kFmtNvfp4) {  // sixteen E4M3 scale bytes
    if (a.Gtot % 16 == 0 && zp % 16 == 0) return launch_kg<MB, 16, true, FMT>(p, a, stream);
    return launch_kg<MB, 16, false, FMT>(p, a, stream);
  } else {
    if (group == 128) {
      if (a.Gtot % 2 == 0 && sp % 4 == 0) return launch_kg<MB, 128, true, FMT>(p, a, stream);
      return launch_kg<MB, 128, false, FMT>(p, a, stream);
    }
    if (a.Gtot % 8 == 0 && sp % 16 == 0 && (FMT == kFmtInt8 || zp % 4 == 0))
      return launch_kg<MB, 32, true, FMT>(p, a, stream);
    return launch_kg<MB, 32, false, FMT>(p, a, stream);
  }
}

template <int FMT>
hipError_t launch_f(int group, const GemmPlan& p, const GemmArgs& a, hipStream_t stream) {
  switch (p.MB) {
    case 1: return launch_t<1, FMT>(group, p, a, stream);
    case 2: return launch_t<2, FMT>(group, p, a, stream);
    case 4: return launch_t<4, FMT>(group, p, a, stream);
    default: return launch_t<8, FMT>(group, p, a, stream);
  }
}

}  // namespace

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int) {
  const GemmPlan p = plan_gemm(M, N, K);
  if (p.KS == 1) return 0;
  // partial-sum planes padded to whole tiles: [KS][gy * 16 * MB][gx * 128]
  return kSplitCounterBytes + (size_t)p.KS * p.gy * 16 * p.MB * p.gx * 128 * sizeof(float);
}

int describe_gemm(int64_t M, int64_t N, int64_t K, int group, int fmt, char* buf, size_t len) {
  const GemmPlan p = plan_gemm(M, N, K);
  return snprintf(buf, len, "gemm_kernel<MB=%d, NPW=%d, G=%d%s> grid=(%u,%u,%d) block=%d lds=%zu split_k=%d", p.MB,
                  kNPW, group,
                  fmt == kFmtInt8 ? ", BITS=8" : fmt == kFmtMxfp4 ? ", MXFP4" : fmt == kFmtNvfp4 ? ", NVFP4" : "", p.gx,
                  p.gy, p.KS,
                  kWaves * 64, gemm_lds(p.MB, group, fmt), p.KS);
}

hipError_t launch_gemm(int64_t M, int64_t N, int64_t K, int group, int fmt, const uint16_t* x, const void* qpacked,
                       const uint16_t* s, const uint8_t* zpacked, uint16_t* y, void* workspace,
                       hipStream_t stream, const float* tscale) {
  const GemmPlan p = plan_gemm(M, N, K);
  GemmArgs a;
  a.tscale = tscale;
  a.KS = p.KS;
  a.kt_per_split = p.kt_per_split;
  a.partial = nullptr;
  a.counters = nullptr;
  if (p.KS > 1) {
    a.counters = static_cast<unsigned*>(workspace);
    a.partial = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + kSplitCounterBytes);
  }
  a.x = x;
  a.qp = static_cast<const uint8_t*>(qpacked);
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
  if (fmt == kFmtInt8) return launch_f<kFmtInt8>(group, p, a, stream);
  if (fmt == kFmtMxfp4) return launch_f<kFmtMxfp4>(group, p, a, stream);
  if (fmt == kFmtNvfp4) return launch_f<kFmtNvfp4>(group, p, a, stream);
  return launch_f<kFmtInt4>(group, p, a, stream);
}

}  // namespace wq
