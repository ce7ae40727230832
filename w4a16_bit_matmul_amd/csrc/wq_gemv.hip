// Split-K dequantize-and-multiply GEMV for small M (gfx950).
//
// Computes y[m][n] = sum_k x[m][k] * What[n][k] -- the fused weight-only
// product of "Quantization Methods Compared: INT8, GPTQ, AWQ, FP8, FP4 and
// KV-Cache Quantization", section "Hardware, formats and the roofline" (decode
// reads every weight once and is bound by memory bandwidth), with the decodings
// of "Quantization for LLM inference: FP8, INT4 (GPTQ, AWQ) and GGUF", sections
// "The minimum maths" (What = s (q - z) for 4-bit and s q for 8-bit integer
// codes) and "Microscaling: NVFP4 and MXFP4" (E2M1 codes times an E8M0 or an
// E4M3 block scale).
//
// Kernels.  gemv_mfma_kernel (4-bit and 8-bit integer, MXFP4 and NVFP4 codes)
// takes the dot products on the matrix cores: every code word of a lane
// becomes the exact fp16 B operand of one v_mfma_f32_16x16x32_f16 (the
// decodings are described beside it), and gemv_mfma_half_kernel is its one-row
// form for 4-bit codes over half a 16-row block.
//
// 8-bit codes (group absmax int8, decoding s * q, no zero-point): a word holds
// four two's-complement codes; XOR-ing the sign bits and placing two bytes
// under the fp16 exponent of 1024 (v_perm_b32) gives (1152 + q) pairs, and one
// packed fp16 subtraction of 1152 leaves q exactly: the matrix core sums x * q
// over a group in fp32, and one multiply-add applies the group's scale.
//
// Decomposition.  A workgroup owns one 16-row block (the matrix-core kernel
// with eight or sixteen rows of x: RB = 1, 2 or 4 consecutive blocks, which
// share each x slice), MT rows of x and a range of 128-column K tiles (all of K
// unless the grid splits K).  Wave w walks
// segments of KQ consecutive K tiles (w, w + W, w + 2W, ... in segment units).
// For each segment it first loads the segment's slice of x (one 16-byte load
// per lane and x row), then the segment's scales and zero-points (one or two
// vector loads per lane when the layout allows), then the KQ code tiles (with
// non-temporal loads: each code byte is read once, and the streaming hint
// measured 2-8 % faster), and copies the x slice into its own LDS region: no
// workgroup barrier stands between the loads and the arithmetic, so each wave
// starts as soon as its own data arrives.  Two 1024-thread workgroups share
// a CU only if every wave holds at most 64 VGPRs (eight waves per SIMD), so the
// one-row 4-bit, MXFP4 and NVFP4 instances are compiled to that bound; the
// instances that need more registers (8-bit codes, two or more rows of x) run
// eight-wave workgroups instead, two or three per CU (sixteen-row tiles over
// four blocks: four-wave workgroups, two per CU; eight-row tiles over two
// blocks, or over one block of a narrow output: sixteen waves, one workgroup
// per CU, at most 128 VGPRs).  The waves' partial sums meet in
// LDS in a fixed order.  When the grid splits K, each
// workgroup writes fp32 partial sums to the workspace and the last workgroup of
// a row range (found with a device-scope atomic counter) adds them in split
// order and writes y, so results stay deterministic; it then puts the counter
// back to zero for the next call.
#include <stdio.h>

#include <algorithm>

#include "wq_device.h"
#include "wq_kernels.h"

namespace wq {
namespace {

struct GemvArgs {
  const uint16_t* x;
  const uint8_t* qp;
  const uint16_t* s;
  const uint8_t* zp;
  uint16_t* y;
  float* partial;      // [KS][M][N] fp32 (KS > 1 only)
  unsigned* counters;  // [gridDim.y][gridDim.x] (KS > 1 only)
  const float* tscale; // NVFP4: the per-tensor scale (device)
  int M, N, K, kt_per_split, KS, sz_vec;
};

// Tile and group counts derived in the kernel from K (and the group size G),
// so that every kernel argument arrives in the first batch of scalar loads
// (a field first used after a branch is otherwise fetched there, adding a
// second kernel-argument round trip before the first weight load).
struct Dims {
  int KT, Gtot, GB;
};
template <int G>
__device__ __forceinline__ Dims dims_of(int K) {
  const int gtot = K / G;
  return Dims{(K + 127) >> 7, gtot, (gtot + 1) >> 1};
}

// Forces a value into a VGPR and hides it from constant folding, so that
// v_and_or_b32 can take the mask from an SGPR and the fp16 exponent bits from
// this register (a VOP3 instruction takes no literal and one SGPR at most).
__device__ __forceinline__ uint32_t in_vgpr(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Scales and zero-points of the NS = KQ * 128 / G groups one segment covers in
// one row, kept as loaded until use (so that issuing the loads never waits):
// group t's scale is half t of sv, its zero-point nibble t of zv.
template <int NS>
struct SZ {
  uint32_t sv[NS / 2];
  uint32_t zv[(NS + 7) / 8];
  __device__ __forceinline__ float scale(int t) const {
    return f16_bits_to_f32((uint16_t)(sv[t >> 1] >> (16 * (t & 1))));
  }
  __device__ __forceinline__ uint32_t zero(int t) const { return (zv[t >> 3] >> (4 * (t & 7))) & 15u; }
};

// (srow / zrow as below; ZP = false: no zero-points, zv stays zero.)
// srow / zrow: element offsets of the row's scales and zero-point bytes (rows
// past N are clamped to row N - 1 by the caller: their outputs are never
// stored); g0: first group of the segment (wave-uniform).  With a.sz_vec the
// segment's groups lie inside the row and are aligned for vector loads;
// otherwise each group is loaded alone, clamped into the row (groups past the
// row meet zero activations and zero codes).
template <int NS, bool ZP>
__device__ __forceinline__ SZ<NS> load_sz(const GemvArgs& a, int Gtot, uint32_t srow, uint32_t zrow, int g0) {
  SZ<NS> v;
#pragma unroll
  for (int i = 0; i < (NS + 7) / 8; ++i) v.zv[i] = 0;
  if (a.sz_vec) {
    const uint16_t* sp = a.s + srow + g0;
    const uint8_t* zp = ZP ? a.zp + zrow + g0 / 2 : nullptr;
    if constexpr (NS == 4) {
      const uint2 t = *reinterpret_cast<const uint2*>(sp);
      v.sv[0] = t.x;
      v.sv[1] = t.y;
      if constexpr (ZP) v.zv[0] = *reinterpret_cast<const uint16_t*>(zp);
    } else if constexpr (NS == 8) {
      const uint4 t = *reinterpret_cast<const uint4*>(sp);
      v.sv[0] = t.x; v.sv[1] = t.y; v.sv[2] = t.z; v.sv[3] = t.w;
      if constexpr (ZP) v.zv[0] = *reinterpret_cast<const uint32_t*>(zp);
    } else {
      static_assert(NS == 16, "segment of 4 or 8 groups at g = 128, 16 at g = 32");
      const uint4 t0 = *reinterpret_cast<const uint4*>(sp), t1 = *reinterpret_cast<const uint4*>(sp + 8);
      v.sv[0] = t0.x; v.sv[1] = t0.y; v.sv[2] = t0.z; v.sv[3] = t0.w;
      v.sv[4] = t1.x; v.sv[5] = t1.y; v.sv[6] = t1.z; v.sv[7] = t1.w;
      if constexpr (ZP) {
        const uint2 zz = *reinterpret_cast<const uint2*>(zp);
        v.zv[0] = zz.x;
        v.zv[1] = zz.y;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < NS / 2; ++i) v.sv[i] = 0;
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      const int gi = min(g0 + t, Gtot - 1);
      v.sv[t >> 1] |= (uint32_t)a.s[srow + gi] << (16 * (t & 1));
      if constexpr (ZP) {
        const uint32_t zb = a.zp[zrow + (gi >> 1)];
        v.zv[t >> 3] |= ((gi & 1) ? (zb >> 4) : (zb & 15u)) << (4 * (t & 7));
      }
    }
  }
  return v;
}

// E8M0 scale bytes of the NS blocks one segment covers in one row.
template <int NS>
struct E8 {
  uint32_t v[NS / 4];
  __device__ __forceinline__ float scale(int t) const { return e8m0_to_f32((v[t >> 2] >> (8 * (t & 3))) & 0xffu); }
};

// (scale bytes of NS = 16 blocks (MXFP4) or 32 blocks (NVFP4) per segment)
template <int NS>
__device__ __forceinline__ E8<NS> load_e8(const GemvArgs& a, int Gtot, uint32_t erow, int g0) {
  static_assert(NS == 16 || NS == 32, "segment of four tiles of four or eight blocks");
  E8<NS> v;
  if (a.sz_vec) {
#pragma unroll
    for (int h = 0; h < NS / 16; ++h) {
      const u4 t = *reinterpret_cast<const u4*>(a.zp + erow + g0 + 16 * h);
      v.v[4 * h] = t[0]; v.v[4 * h + 1] = t[1]; v.v[4 * h + 2] = t[2]; v.v[4 * h + 3] = t[3];
    }
  } else {
#pragma unroll
    for (int i = 0; i < NS / 4; ++i) v.v[i] = 0;
#pragma unroll
    for (int t = 0; t < NS; ++t) v.v[t >> 2] |= (uint32_t)a.zp[erow + min(g0 + t, Gtot - 1)] << (8 * (t & 3));
  }
  return v;
}

// ---- GEMV with the dot products on the matrix cores (M <= 16 rows of x per tile).
//
// Each code word j of a tile (the decomposition above) becomes one
// v_mfma_f32_16x16x32_f16 B operand: lane l = r + 16c supplies B column r (weight
// row nb*16 + r) with k-slots 8c..8c+7 of step j, which is exactly word j of
// its 16 bytes, and A row r (activation row m0 + r, clamped to the block's
// last row; the D rows it produces past MT are never read) with the same
// k-slots, read from the wave's LDS slice.  The B operand is the exact fp16
// q - z of each code:
//   word & 0x000F000F | 0x6400 6400     = (1024 + q0, 1024 + q1)
//   word & 0x00F000F0 | 0x5400 5400     = (  64 + q2,   64 + q3)
// and the same two of (word >> 8) for columns 4..7 (an fp16 with exponent
// 2^6 has unit spacing 2^-4, so code bits 4..7 land on whole numbers), minus
// the group's (1024 + z) or (64 + z) pair; the matrix core accumulates the
// exact products x * (q - z) in fp32 over a group, and one fp32 multiply-add
// per group applies the scale: 9 VALU instructions per code word, against 13
// for the same exact arithmetic on the vector units with v_dot2_f32_f16.  Lane
// (r, c) receives D rows 4c..4c+3 (activation rows) of column r.
// Halves between the rows of a wave's x slice in the matrix-core GEMV: KQ
// tiles, plus 16 bytes with several rows (A-fragment reads then start the
// sixteen rows on different banks; with one row every lane reads the same one).
constexpr __host__ __device__ int gemv_xrow(int MT, int KQ) { return KQ * 128 + (MT > 1 ? 8 : 0); }

// RB > 1: the workgroup owns RB consecutive 16-row blocks, and each wave
// applies its segment's x slice to the codes of all of them, so x is read
// from L2 once per RB blocks.
// (Register bounds: the one-row sixteen-wave instances run two workgroups per
// CU at 64 VGPRs; the eight-row instances over up to two blocks two eight-wave
// workgroups, or one sixteen-wave workgroup, at 128; the four-wave
// sixteen-row instances two at 256.)
// FMT: kFmtInt4 (above), kFmtInt8 (2048-byte tiles, 32 bytes per lane: step
// j's eight codes are words 2 (j % 2) and 2 (j % 2) + 1 of half j / 2, decoded
// to exact fp16 q), kFmtMxfp4 or kFmtNvfp4.  The E2M1 codes share the
// tile layout, so word j of a lane's 16 bytes is again the B operand of step j:
// v_cvt_scalef32_pk_f16_fp4 at scale 1 gives its eight exact E2M1 values.
// MXFP4 (one E8M0 scale per 32 columns = one step): the matrix core sums each
// step, and one fp32 multiply-add applies the block's power of two (exact over
// the whole E8M0 range).  NVFP4 (one E4M3 scale per 16 columns, so two blocks
// per step): the lane's eight values lie in one block and are multiplied by
// its scale as an fp16 pair (the FP8 conversion gives the E4M3 value exactly;
// the product is exact too: E2M1 x E4M3 has at most 6 significant bits inside
// fp16's normal range), so the matrix core sums the whole K range and the
// per-tensor scale multiplies each output.
template <int MT, int W, int KQ, int G, int RB = 1, int FMT = kFmtInt4>
__global__ __launch_bounds__(W * 64, (W == 16 && MT == 1) ? 8 : (MT == 8 && RB <= 2) ? 4 : W == 4 ? 2 : 1) void
gemv_mfma_kernel(GemvArgs a) {
  static_assert(FMT == kFmtInt4 || FMT == kFmtInt8 || (FMT == kFmtMxfp4 && G == 32) || (FMT == kFmtNvfp4 && G == 16),
                "code format");
  constexpr int TB = FMT == kFmtInt8 ? kTileBytes8 : kTileBytes;
  constexpr int HALVES = FMT == kFmtInt8 ? 2 : 1;  // 16-byte loads per lane and tile
  constexpr int GPT = 128 / G;       // groups per 128-column tile
  constexpr int SPG = GPT <= 4 ? 4 / GPT : 1;  // MFMA steps per group (integer and MXFP4 codes)
  constexpr int NS = KQ * GPT;       // groups per segment
  constexpr int NE = FMT == kFmtNvfp4 ? 32 : 16;  // scale bytes per segment and row (MXFP4, NVFP4)
  constexpr int NT = W * 64;
  constexpr int XCH = MT * KQ / 4;   // 16-byte x chunks per lane and segment
  constexpr int NA = MT < 4 ? MT : 4;  // D elements per lane that can hold real rows
  constexpr int XROW = gemv_xrow(MT, KQ);  // halves between slice rows
  static_assert(KQ % 4 == 0 && XCH >= 1, "a segment is a multiple of four tiles");
  extern __shared__ __align__(16) uint8_t smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, c = lane >> 4;
  const int nb0 = blockIdx.x * RB, m0 = blockIdx.y * MT, ks = blockIdx.z;
  const int nblk = (a.N + 15) >> 4;
  const Dims d = dims_of<G>(a.K);
  const int kt_lo = ks * a.kt_per_split;
  const int nkt = min(d.KT, kt_lo + a.kt_per_split) - kt_lo;
  uint16_t* xw = reinterpret_cast<uint16_t*>(smem) + wv * (MT * XROW);
  // the cross-wave sums [W][RB][MT][16]: after the x slices (RB = 1), or in
  // their place once every wave is done with its slice
  float* red = reinterpret_cast<float*>(smem + (RB == 1 ? (size_t)W * MT * XROW * 2 : 0));

  // per row block: its tiles (blocks past the last re-read it; their outputs
  // are never stored) and this lane's row of scales and zero-points
  const uint8_t* tbase[RB];
  uint32_t srow[RB], zrow[RB];
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int nb = min(nb0 + b, nblk - 1);
    tbase[b] = a.qp + (size_t)nb * d.KT * TB;
    const uint32_t n = (uint32_t)min(nb * 16 + r, a.N - 1);
    srow[b] = n * (uint32_t)d.Gtot;
    zrow[b] = n * (uint32_t)d.GB;
  }
  const uint32_t lane16 = 16u * lane;
  const uint32_t m1024 = in_vgpr(kMagicPair), m64 = in_vgpr(0x54005400u);
  const h2 b1152 = as_h2(in_vgpr(0x64806480u));  // (1152, 1152): 8-bit codes
  // this lane's A row of the slice (rows past MT repeat the last one); slice
  // rows are XROW halves apart, KQ tiles plus 16 bytes, so that the sixteen
  // rows an A-fragment read touches start on different banks
  const uint16_t* arow = xw + (r < MT ? r : MT - 1) * XROW + 8 * c;

  float acc[RB][NA];
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int i = 0; i < NA; ++i) acc[b][i] = 0.0f;
  f4 accv[RB];  // NVFP4: the matrix core's running sums
#pragma unroll
  for (int b = 0; b < RB; ++b) accv[b] = f4{0.f, 0.f, 0.f, 0.f};

  for (int sg = wv; sg * KQ < nkt; sg += W) {
    const int q0 = sg * KQ;
    const int nq = min(KQ, nkt - q0);
    const int kt0 = kt_lo + q0;

    u4 buf[RB][KQ][HALVES];
    uint4 xc[XCH];
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int ci = i * 64 + lane, m = ci / (KQ * 16), cc = ci % (KQ * 16);
      const int row = min(m0 + m, a.M - 1), col = min(kt0 * 128 + cc * 8, a.K - 8);
      xc[i] = *reinterpret_cast<const uint4*>(a.x + (size_t)row * a.K + col);
    }
    SZ<(FMT == kFmtInt4 || FMT == kFmtInt8) ? NS : 4> sz[RB];
    E8<NE> e8s[RB];
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      if constexpr (FMT == kFmtInt4 || FMT == kFmtInt8)
        sz[b] = load_sz<NS, FMT == kFmtInt4>(a, d.Gtot, srow[b], zrow[b], kt0 * GPT);
      else
        e8s[b] = load_e8<NE>(a, d.Gtot, srow[b], kt0 * GPT);
    }
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int t = 0; t < KQ; ++t)
#pragma unroll
        for (int h = 0; h < HALVES; ++h)
          buf[b][t][h] = __builtin_nontemporal_load(
              reinterpret_cast<const u4*>(tbase[b] + (size_t)min(kt0 + t, d.KT - 1) * TB + 1024u * h + lane16));
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int ci = i * 64 + lane, m = ci / (KQ * 16), cc = ci % (KQ * 16);
      const bool ok = m0 + m < a.M && kt0 * 128 + cc * 8 < a.K;
      *reinterpret_cast<uint4*>(xw + m * XROW + cc * 8) = ok ? xc[i] : make_uint4(0, 0, 0, 0);
    }
    // the slice is read back by other lanes of this wave only
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();

#pragma unroll
    for (int t = 0; t < KQ; ++t) {
      if (t >= nq) break;
      const uint16_t* xr = arow + t * 128;
      if constexpr (FMT == kFmtNvfp4) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const h8 afr = *reinterpret_cast<const h8*>(xr + 32 * j);
#pragma unroll
          for (int b = 0; b < RB; ++b) {
            // step j: the lane's columns lie in block 2j + c / 2 of the tile,
            // byte 2 (j % 2) + c / 2 of scale word 2t + j / 2
            const uint32_t sw = e8s[b].v[2 * t + (j >> 1)] >> (8 * (c >> 1));
            const h2 sp = (j & 1) ? e4m3_pair_f16<true>(sw) : e4m3_pair_f16<false>(sw);
            const h2 s2 = h2{sp[0], sp[0]};
            const uint32_t w = buf[b][t][0][j];
            const h2 p0 = fp4_pair<0>(w, 1.0f) * s2, p1 = fp4_pair<1>(w, 1.0f) * s2;
            const h2 p2 = fp4_pair<2>(w, 1.0f) * s2, p3 = fp4_pair<3>(w, 1.0f) * s2;
            h8 bfr;
            bfr[0] = p0[0]; bfr[1] = p0[1]; bfr[2] = p1[0]; bfr[3] = p1[1];
            bfr[4] = p2[0]; bfr[5] = p2[1]; bfr[6] = p3[0]; bfr[7] = p3[1];
            accv[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(afr, bfr, accv[b], 0, 0, 0);
          }
        }
        continue;
      }
      if constexpr (FMT == kFmtMxfp4) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const h8 afr = *reinterpret_cast<const h8*>(xr + 32 * j);
#pragma unroll
          for (int b = 0; b < RB; ++b) {
            const uint32_t w = buf[b][t][0][j];
            const h2 p0 = fp4_pair<0>(w, 1.0f), p1 = fp4_pair<1>(w, 1.0f);
            const h2 p2 = fp4_pair<2>(w, 1.0f), p3 = fp4_pair<3>(w, 1.0f);
            h8 bfr;
            bfr[0] = p0[0]; bfr[1] = p0[1]; bfr[2] = p1[0]; bfr[3] = p1[1];
            bfr[4] = p2[0]; bfr[5] = p2[1]; bfr[6] = p3[0]; bfr[7] = p3[1];
            const f4 T = __builtin_amdgcn_mfma_f32_16x16x32_f16(afr, bfr, f4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            const float sc = e8s[b].scale(t * 4 + j);
#pragma unroll
            for (int i = 0; i < NA; ++i) acc[b][i] = fmaf(sc, T[i], acc[b][i]);
          }
        }
        continue;
      }
      if constexpr (FMT == kFmtInt8) {
        // step j: the lane's eight codes are words 2 (j % 2) and 2 (j % 2) + 1
        // of half j / 2 of the tile, (1152 + q) pairs minus 1152 in fp16
#pragma unroll
        for (int gi = 0; gi < GPT; ++gi) {
#pragma unroll
          for (int b = 0; b < RB; ++b) {
            f4 T;
#pragma unroll
            for (int jj = 0; jj < SPG; ++jj) {
              const int j = gi * SPG + jj;
              const u4& hv = buf[b][t][j >> 1];
              const uint32_t lo = hv[2 * (j & 1)] ^ 0x80808080u, hi = hv[2 * (j & 1) + 1] ^ 0x80808080u;
              const h2 p0 = as_h2(byte_pair(lo, 0x04010400u)) - b1152, p1 = as_h2(byte_pair(lo, 0x04030402u)) - b1152;
              const h2 p2 = as_h2(byte_pair(hi, 0x04010400u)) - b1152, p3 = as_h2(byte_pair(hi, 0x04030402u)) - b1152;
              h8 bfr;
              bfr[0] = p0[0]; bfr[1] = p0[1]; bfr[2] = p1[0]; bfr[3] = p1[1];
              bfr[4] = p2[0]; bfr[5] = p2[1]; bfr[6] = p3[0]; bfr[7] = p3[1];
              const h8 afr = *reinterpret_cast<const h8*>(xr + 32 * j);
              T = jj == 0 ? __builtin_amdgcn_mfma_f32_16x16x32_f16(afr, bfr, f4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0)
                          : __builtin_amdgcn_mfma_f32_16x16x32_f16(afr, bfr, T, 0, 0, 0);
            }
            const float sc = sz[b].scale(t * GPT + gi);
#pragma unroll
            for (int i = 0; i < NA; ++i) acc[b][i] = fmaf(sc, T[i], acc[b][i]);
          }
        }
        continue;
      }
#pragma unroll
      for (int gi = 0; gi < GPT; ++gi) {
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          const uint32_t z = sz[b].zero(t * GPT + gi);
          const h2 zq = as_h2(z * 0x00010001u + kMagicPair);     // (1024 + z) twice
          const h2 z64 = as_h2(z * 0x00100010u + 0x54005400u);   // (64 + z) twice: z in mantissa bits 4..7
          f4 T;
#pragma unroll
          for (int jj = 0; jj < SPG; ++jj) {
            const int j = gi * SPG + jj;
            const uint32_t w = buf[b][t][0][j], w8 = w >> 8;
            const h2 p0 = as_h2((w & 0x000F000Fu) | m1024) - zq;
            const h2 p1 = as_h2((w & 0x00F000F0u) | m64) - z64;
            const h2 p2 = as_h2((w8 & 0x000F000Fu) | m1024) - zq;
            const h2 p3 = as_h2((w8 & 0x00F000F0u) | m64) - z64;
            h8 bfr;
            bfr[0] = p0[0]; bfr[1] = p0[1]; bfr[2] = p1[0]; bfr[3] = p1[1];
            bfr[4] = p2[0]; bfr[5] = p2[1]; bfr[6] = p3[0]; bfr[7] = p3[1];
            const h8 afr = *reinterpret_cast<const h8*>(xr + 32 * j);
            T = jj == 0 ? __builtin_amdgcn_mfma_f32_16x16x32_f16(afr, bfr, f4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0)
                        : __builtin_amdgcn_mfma_f32_16x16x32_f16(afr, bfr, T, 0, 0, 0);
          }
          const float sc = sz[b].scale(t * GPT + gi);
#pragma unroll
          for (int i = 0; i < NA; ++i) acc[b][i] = fmaf(sc, T[i], acc[b][i]);
        }
      }
    }
    // the next segment overwrites this wave's slice: finish reading it first
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
  }

  if constexpr (FMT == kFmtNvfp4) {
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int i = 0; i < NA; ++i) acc[b][i] = accv[b][i];
  }
  // NVFP4: the per-tensor scale multiplies each output (partial sums stay unscaled)
  const float ys = FMT == kFmtNvfp4 ? *a.tscale : 1.0f;

  // ---- reduce: lane (r, c) holds rows 4c + i of column r of each block; the
  // W waves' sums of each (block, row, column) meet in LDS and are added in
  // wave order
  constexpr int NOUT = MT * 16;   // outputs per row block
  if constexpr (RB > 1) __syncthreads();  // every wave is done with its x slice
  if (4 * c < MT) {
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int i = 0; i < NA; ++i)
        if (4 * c + i < MT) red[((wv * RB + b) * MT + 4 * c + i) * 16 + r] = acc[b][i];
  }
  __syncthreads();
  for (int i = tid; i < RB * NOUT; i += NT) {
    const int b = i / NOUT, o = i % NOUT;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w) v += red[(w * RB + b) * NOUT + o];
    const int rr = o & 15, m = o >> 4;
    const int nn = (nb0 + b) * 16 + rr, mm = m0 + m;
    if (a.KS > 1)  // padded plane [gridDim.y * MT][gridDim.x * RB * 16]: always in bounds
      split_store(a.partial + ((size_t)ks * gridDim.y * MT + mm) * (gridDim.x * RB * 16) + nn, v);
    else if (nn < a.N && mm < a.M)
      a.y[(size_t)mm * a.N + nn] = f32_to_f16_bits(FMT == kFmtNvfp4 ? v * ys : v);
  }
  if (a.KS == 1) return;

  // ---- split-K: the last workgroup of this row range adds the partial sums
  unsigned* ctr = a.counters + blockIdx.y * gridDim.x + blockIdx.x;
  if (!split_arrive(ctr, a.KS)) return;
  for (int i = tid; i < RB * NOUT; i += NT) {
    const int b = i / NOUT, o = i % NOUT;
    const int rr = o & 15, m = o >> 4;
    const int nn = (nb0 + b) * 16 + rr, mm = m0 + m;
    if (nn < a.N && mm < a.M) {
      const float* pp = a.partial + (size_t)mm * (gridDim.x * RB * 16) + nn;
      const size_t plane = (size_t)gridDim.y * MT * gridDim.x * RB * 16;
      float v = 0.0f;
      for (int k0 = 0; k0 < a.KS; k0 += 4) {  // four loads in flight, added in split order
        float t[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) t[j] = split_load(pp + (size_t)min(k0 + j, a.KS - 1) * plane);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (k0 + j < a.KS) v += t[j];
      }
      a.y[(size_t)mm * a.N + nn] = f32_to_f16_bits(FMT == kFmtNvfp4 ? v * ys : v);
    }
  }
  if (tid == 0) split_reset(ctr);
}

// ---- One activation row (M = 1): eight weight rows per workgroup.
//
// Streaming a weight matrix once reads fastest in units of 16-32 KB per
// workgroup; a 16-row block of a K = 8192 matrix is 64 KB.  With one row of
// activations only row 0 of the matrix core's sixteen A rows carries data, so
// a wave covers HALF the rows of two neighbouring K tiles at once: lanes
// r = 0..7 hold rows 8h + r of tile t, lanes r = 8..15 rows 8h + r - 8 of
// tile t + 1 (each lane still reads 16 bytes of a tile: eight rows x 16 bytes
// = 128 contiguous bytes per tile and lane column c), and A row 0 is x over
// tile t, A rows 1..15 are x over tile t + 1.  Then D row 0 of columns 0..7
// and D row 1 of columns 8..15 are the two tiles' dot products for the same
// eight weight rows; the lanes of a weight row add them.  The workgroup
// (one half h of a 16-row block, all of K) reads half as many bytes.
template <int W, int KQ, int G>
__global__ __launch_bounds__(W * 64, W == 16 ? 8 : 4) void gemv_mfma_half_kernel(GemvArgs a) {
  constexpr int GPT = 128 / G;       // groups per 128-column tile
  constexpr int SPG = 4 / GPT;       // MFMA steps per group
  constexpr int NS = KQ * GPT;       // groups per segment
  constexpr int NP = KQ / 2;         // tile pairs per segment
  static_assert(KQ == 4, "a segment is four tiles: one 16-byte x chunk per lane");
  extern __shared__ __align__(16) uint8_t smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, c = lane >> 4;
  const int rr = r & 7, tsel = r >> 3;  // row within the half, which tile of the pair
  const int hb = blockIdx.x, nb = hb >> 1, h = hb & 1, ks = blockIdx.z;
  const Dims d = dims_of<G>(a.K);
  const int kt_lo = ks * a.kt_per_split;
  const int nkt = min(d.KT, kt_lo + a.kt_per_split) - kt_lo;
  uint16_t* xw = reinterpret_cast<uint16_t*>(smem) + wv * (KQ * 128);
  float* red = reinterpret_cast<float*>(smem + (size_t)W * KQ * 256);  // [W][16]

  const uint8_t* tbase = a.qp + (size_t)nb * d.KT * kTileBytes + 16u * (8 * h + rr + 16 * c);
  const uint32_t n = (uint32_t)min(hb * 8 + rr, a.N - 1);
  const uint32_t srow = n * (uint32_t)d.Gtot, zrow = n * (uint32_t)d.GB;
  const uint32_t m1024 = in_vgpr(kMagicPair), m64 = in_vgpr(0x54005400u);
  const int aoff = (r == 0 ? 0 : 128) + 8 * c;  // A row 0: the pair's first tile; rows 1..15: its second

  float acc = 0.0f;
  for (int sg = wv; sg * KQ < nkt; sg += W) {
    const int q0 = sg * KQ;
    const int nq = min(KQ, nkt - q0);
    const int kt0 = kt_lo + q0;

    // x over the segment's four tiles: one 16-byte chunk per lane; scales and
    // zero-points of the segment's groups; this lane's two code words
    const uint4 xc = *reinterpret_cast<const uint4*>(a.x + min(kt0 * 128 + lane * 8, a.K - 8));
    const SZ<NS> sz = load_sz<NS, true>(a, d.Gtot, srow, zrow, kt0 * GPT);
    u4 buf[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p)
      buf[p] = __builtin_nontemporal_load(
          reinterpret_cast<const u4*>(tbase + (size_t)min(kt0 + 2 * p + tsel, d.KT - 1) * kTileBytes));
    *reinterpret_cast<uint4*>(xw + lane * 8) = kt0 * 128 + lane * 8 < a.K ? xc : make_uint4(0, 0, 0, 0);
    // the slice is read back by other lanes of this wave only
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();

#pragma unroll
    for (int p = 0; p < NP; ++p) {
      if (2 * p >= nq) break;  // (a second tile past K meets zero activations)
      const uint16_t* xr = xw + 2 * p * 128 + aoff;
#pragma unroll
      for (int gi = 0; gi < GPT; ++gi) {
        // this lane's group: gi of local tile 2p + tsel
        const int t = (2 * p + tsel) * GPT + gi;
        const uint32_t z = (sz.zv[((2 * p) * GPT + gi) >> 3] >> (4 * (t & 7))) & 15u;
        const uint32_t sw = tsel ? sz.sv[((2 * p + 1) * GPT + gi) >> 1] : sz.sv[((2 * p) * GPT + gi) >> 1];
        const float sc = f16_bits_to_f32((uint16_t)(sw >> (16 * (t & 1))));
        const h2 zq = as_h2(z * 0x00010001u + kMagicPair);     // (1024 + z) twice
        const h2 z64 = as_h2(z * 0x00100010u + 0x54005400u);   // (64 + z) twice: z in mantissa bits 4..7
        f4 T;
#pragma unroll
        for (int jj = 0; jj < SPG; ++jj) {
          const int j = gi * SPG + jj;
          const uint32_t w = buf[p][j], w8 = w >> 8;
          const h2 p0 = as_h2((w & 0x000F000Fu) | m1024) - zq;
          const h2 p1 = as_h2((w & 0x00F000F0u) | m64) - z64;
          const h2 p2 = as_h2((w8 & 0x000F000Fu) | m1024) - zq;
          const h2 p3 = as_h2((w8 & 0x00F000F0u) | m64) - z64;
          h8 bfr;
          bfr[0] = p0[0]; bfr[1] = p0[1]; bfr[2] = p1[0]; bfr[3] = p1[1];
          bfr[4] = p2[0]; bfr[5] = p2[1]; bfr[6] = p3[0]; bfr[7] = p3[1];
          const h8 afr = *reinterpret_cast<const h8*>(xr + 32 * j);
          T = jj == 0 ? __builtin_amdgcn_mfma_f32_16x16x32_f16(afr, bfr, f4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0)
                      : __builtin_amdgcn_mfma_f32_16x16x32_f16(afr, bfr, T, 0, 0, 0);
        }
        acc = fmaf(sc, tsel ? T[1] : T[0], acc);
      }
    }
    // the next segment overwrites this wave's slice: finish reading it first
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
  }

  // ---- reduce: lane (r, 0) holds weight row 8h + (r & 7) over one tile of
  // each pair; the W waves' sums and the two lanes of a row meet in LDS
  if (c == 0) red[wv * 16 + r] = acc;
  __syncthreads();
  if (tid < 8) {
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w) v += red[w * 16 + tid] + red[w * 16 + tid + 8];
    const int nn = hb * 8 + tid;
    if (a.KS > 1)  // padded plane [gridDim.x * 8]: always in bounds
      split_store(a.partial + (size_t)ks * gridDim.x * 8 + nn, v);
    else if (nn < a.N)
      a.y[nn] = f32_to_f16_bits(v);
  }
  if (a.KS == 1) return;

  // ---- split-K: the last workgroup of this half block adds the partial sums
  unsigned* ctr = a.counters + blockIdx.x;
  if (!split_arrive(ctr, a.KS)) return;
  if (tid < 8) {
    const int nn = hb * 8 + tid;
    if (nn < a.N) {
      const float* pp = a.partial + nn;
      const size_t plane = (size_t)gridDim.x * 8;
      float v = 0.0f;
      for (int k0 = 0; k0 < a.KS; k0 += 4) {  // four loads in flight, added in split order
        float t4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) t4[j] = split_load(pp + (size_t)min(k0 + j, a.KS - 1) * plane);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (k0 + j < a.KS) v += t4[j];
      }
      a.y[nn] = f32_to_f16_bits(v);
    }
  }
  if (tid == 0) split_reset(ctr);
}

// Launch shape of the GEMV for one problem; shared by the launcher and the
// workspace query so both agree.
constexpr int kKQ = 4;  // K tiles per wave segment

struct GemvPlan {
  int MT, W, RB, KS, kt_per_split;
  bool half;  // gemv_mfma_half_kernel: eight weight rows per workgroup (4-bit codes, one row of x)
  unsigned gx, gy;
  size_t lds;
};

GemvPlan plan_gemv(int64_t M, int64_t N, int64_t K, int fmt) {
  GemvPlan p;
  // past eight rows a sixteen-row activation tile reads the
  // weights once for sixteen rows (M = 16, N = 28672, K = 8192: 52.6 against
  // 75.9 us with two eight-row tiles), unless that leaves fewer than 128
  // workgroups before K is split (N = 1024, M = 16: 7.90 against 6.93 us;
  // M = 32: 9.05 against 11.0 us)
  const int64_t nblk = (N + 15) / 16;
  p.MT = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4
         : (M <= 8 || nblk * ((M + 15) / 16) < 128) ? 8 : 16;
  // one row of 4-bit or FP4 codes: sixteen waves, two workgroups per CU at
  // 64 VGPRs.  Instances that need more registers (two to eight rows, and int8
  // codes with twice the bytes in flight per lane) measured 4-20 % faster with
  // eight-wave workgroups (two or three per CU) than with one sixteen-wave
  // workgroup per CU.
  p.W = (p.MT <= 1 && fmt != kFmtInt8) ? 16 : 8;
  // eight-row workgroups only while they still fit the GPU in one round (two
  // per CU): at M=1, N=1024, K=8192 they took 4.66 us against 5.60 us with
  // 16-row workgroups, but at N=8192 (1024 workgroups, two rounds) 9.8 us
  // against 7.9 us
  p.half = p.MT == 1 && fmt == kFmtInt4 && (N + 15) / 16 * 2 <= 512;
  const int64_t NBLK = (N + 15) / 16, KT = (K + 127) / 128;
  // narrow outputs (N <= 2048) with 9..32 rows of x: eight-row tiles in
  // sixteen-wave workgroups, each covering all of K.  The row tiles of a
  // column block re-read its codes from L2 (from the same XCD's when the
  // grid's x extent is a multiple of eight: workgroups go round the eight
  // XCDs in order); what is saved is the split-K hand-off and half of each
  // wave's x slice.  N = 1024, K = 8192, g = 32: M = 16 6.87 ->
  // 6.67 us, M = 32 7.80 -> 6.59 us; N = 2048, M = 16 7.98 -> 6.82 us;
  // N = 1024, K = 14336, M = 32 12.84 -> 9.46 us; MXFP4 and NVFP4 gain as
  // much.  Taken only where it fills the GPU: at least 64 workgroups (N = 64,
  // M = 16: 6.05 -> 6.33 us), at least eight K segments for the sixteen waves
  // (K = 2048, N = 2048, M = 32: 4.03 -> 5.68 us, the 141 KB of LDS holding
  // one workgroup per CU), sixteen past one round of 256 workgroups, and one
  // pass over K unless the grid fills one round (N = 1024, K = 14336, M = 16,
  // 128 workgroups over two passes: 8.48 -> 9.64 us).  8-bit codes keep
  // eight-wave workgroups (registers).
  const int64_t nwg8 = NBLK * ((M + 7) / 8), segs = (KT + kKQ - 1) / kKQ;
  const bool narrow = fmt != kFmtInt8 && M > 8 && M <= 32 && N <= 2048 && nwg8 >= 64 && segs >= 8 &&
                      (segs >= 16 || nwg8 <= 256) && (KT <= 16 * kKQ || nwg8 >= 256);
  if (narrow) p.MT = 8;
  p.gy = (unsigned)((M + p.MT - 1) / p.MT);
  // eight or sixteen rows of x: each workgroup applies its x
  // slices to RB row blocks (x read from L2 once per RB blocks), as many as
  // still leave the grid more than one round of workgroups (eight-row tiles
  // run two workgroups per CU, sixteen-row tiles one) and no reason to split
  // K.  M = 16, N = 28672, K = 8192, g = 128: 52.8 -> 33.7 us with four
  // blocks (32.9 us in four-wave workgroups, below); M = 8, g = 32: 35.1 ->
  // 32.5 us with two.  Both tile heights also take two blocks where that
  // still leaves one workgroup per CU (eight-row tiles: sixteen waves, below):
  // re-reading x from L2 costs more than the second round saves (M = 8,
  // N = 8192, g = 32: K = 8192 12.13 -> 11.18 us, K = 28672 36.7 -> 30.7 us;
  // M = 16, N = K = 8192, MXFP4 14.7 -> 11.3 us).
  p.RB = 1;
  if (!narrow && fmt != kFmtInt8 && p.MT >= 8) {  // (8-bit codes: twice the code registers per block)
    const int64_t round = p.MT == 8 ? 512 : 256;
    for (int rb = 4; rb > 1; rb /= 2)
      if ((NBLK + rb - 1) / rb * p.gy > round) {
        p.RB = rb;
        break;
      }
    if (p.RB == 1 && (NBLK + 1) / 2 * p.gy >= 256) p.RB = 2;
  }
  // sixteen-row tiles over four row blocks: four-wave workgroups, two per CU,
  // so that the grid runs in one round (M = 16, N = 28672, g = 32: 40.0 ->
  // 37.5 us); eight-row tiles over two blocks in a grid of at most 256
  // workgroups: sixteen waves, one workgroup per CU
  if (p.MT == 16 && p.RB == 4) p.W = 4;
  if (p.MT == 8 && p.RB == 2 && (NBLK + 1) / 2 * p.gy <= 256) p.W = 16;
  if (narrow) p.W = 16;
  p.gx = (unsigned)(p.half ? 2 * NBLK : (NBLK + p.RB - 1) / p.RB);
  // split K across workgroups only where a workgroup would otherwise take
  // more than one pass of its waves over K, and only up to about two
  // workgroups per CU: a split that leaves waves without a segment, or that
  // merely adds workgroups, pays the hand-off at the tail for nothing
  // (N = 1024, K = 8192: 5.32 -> 4.43 us without the split; N = 4096: 6.80 ->
  // 5.31 us)
  int64_t ks = 1;
  const int64_t wgs = (int64_t)p.gx * p.gy, pass = (int64_t)p.W * kKQ;
  const int64_t passes = (KT + pass - 1) / pass;
  const int64_t target = p.half ? 1024 : 512;  // about two workgroups per CU
  while (wgs * ks * 2 <= target && ks < passes) ks *= 2;
  if (wgs > kSplitMaxTiles) ks = 1;  // (never taken: a split grid has < 512 row ranges)
  if (p.RB > 1) ks = 1;  // (never taken either: row blocks are shared only past one round)
  if (narrow) ks = 1;     // (K = 14336, M = 32: 9.46 us whole, 14.26 us split two ways)
  // split boundaries on whole segments
  p.kt_per_split = (int)(((KT + ks - 1) / ks + kKQ - 1) / kKQ * kKQ);
  p.KS = (int)((KT + p.kt_per_split - 1) / p.kt_per_split);
  // x slices (the eight-row kernel: [W][KQ * 128] halves), then the
  // cross-wave sums [W][MT][16] fp32; with several row blocks the sums
  // [W][RB][MT][16] reuse the slices' space
  const size_t slices = !p.half ? (size_t)p.W * p.MT * gemv_xrow(p.MT, kKQ) * 2 : (size_t)p.W * p.MT * kKQ * 256;
  if (p.RB > 1)
    p.lds = std::max(slices, (size_t)p.W * p.RB * p.MT * 16 * 4);
  else
    p.lds = slices + (size_t)p.W * p.MT * 16 * 4;
  return p;
}

template <int W, int G>
hipError_t launch_kh(const GemvPlan& p, const GemvArgs& a, hipStream_t stream) {
  if (!p.half || p.MT != 1 || p.W != W || p.RB != 1) return hipErrorInvalidValue;
  auto k = gemv_mfma_half_kernel<W, kKQ, G>;
  static std::atomic<uint64_t> lds_raised{0};
  const hipError_t e = raise_lds_limit((const void*)k, p.lds, lds_raised);
  if (e != hipSuccess) return e;
  k<<<dim3(p.gx, p.gy, p.KS), dim3(W * 64), p.lds, stream>>>(a);
  return hipGetLastError();
}

template <int MT, int W, int G, int RB, int FMT>
hipError_t launch_km(const GemvPlan& p, const GemvArgs& a, hipStream_t stream) {
  // the plan sized the grid and the LDS for its own (MT, W, RB): launch only
  // the instance it describes
  if (p.half || p.MT != MT || p.W != W || p.RB != RB) return hipErrorInvalidValue;
  auto k = gemv_mfma_kernel<MT, W, kKQ, G, RB, FMT>;
  static std::atomic<uint64_t> lds_raised{0};
  const hipError_t e = raise_lds_limit((const void*)k, p.lds, lds_raised);
  if (e != hipSuccess) return e;
  k<<<dim3(p.gx, p.gy, p.KS), dim3(W * 64), p.lds, stream>>>(a);
  return hipGetLastError();
}

// the matrix-core GEMV over p.RB row blocks (sixteen-row tiles over four
// blocks run four-wave workgroups; sixteen-wave eight-row workgroups exist
// over one block, for narrow outputs, and over two)
template <int MT, int W, int G, int FMT>
hipError_t launch_mk(const GemvPlan& p, const GemvArgs& a, hipStream_t stream) {
  if constexpr (FMT == kFmtInt8) {  // one row block per workgroup, eight waves
    if (p.RB != 1 || W != 8) return hipErrorInvalidValue;
    return launch_km<MT, 8, G, 1, FMT>(p, a, stream);
  } else if constexpr (MT == 8 && W == 16) {
    if (p.RB == 1) return launch_km<8, 16, G, 1, FMT>(p, a, stream);
    if (p.RB != 2) return hipErrorInvalidValue;
    return launch_km<8, 16, G, 2, FMT>(p, a, stream);
  } else {
    if constexpr (MT == 8) {
      if (p.RB == 4) return launch_km<8, W, G, 4, FMT>(p, a, stream);
      if (p.RB == 2) return launch_km<8, W, G, 2, FMT>(p, a, stream);
    }
    if constexpr (MT == 16) {
      if (p.RB == 4) return launch_km<16, 4, G, 4, FMT>(p, a, stream);
      if (p.RB == 2) return launch_km<16, 8, G, 2, FMT>(p, a, stream);
    }
    if (p.RB != 1) return hipErrorInvalidValue;
    return launch_km<MT, W, G, 1, FMT>(p, a, stream);
  }
}

template <int MT, int W>
hipError_t launch_t(const GemvPlan& p, int group, int fmt, GemvArgs a, hipStream_t stream) {
  if (fmt == kFmtMxfp4) return launch_mk<MT, W, 32, kFmtMxfp4>(p, a, stream);
  if (fmt == kFmtNvfp4) return launch_mk<MT, W, 16, kFmtNvfp4>(p, a, stream);
  if (fmt == kFmtInt8)
    return group == 128 ? launch_mk<MT, W, 128, kFmtInt8>(p, a, stream) : launch_mk<MT, W, 32, kFmtInt8>(p, a, stream);
  if constexpr (MT == 1 && W == 16) {
    if (p.half) return group == 128 ? launch_kh<W, 128>(p, a, stream) : launch_kh<W, 32>(p, a, stream);
  } else {
    // the eight-row grid (two workgroups per 16-row block) exists only for the
    // one-row sixteen-wave kernel; any other kernel on it would read past N
    if (p.half) return hipErrorInvalidValue;
  }
  return group == 128 ? launch_mk<MT, W, 128, kFmtInt4>(p, a, stream) : launch_mk<MT, W, 32, kFmtInt4>(p, a, stream);
}

}  // namespace

int describe_gemv(int64_t M, int64_t N, int64_t K, int group, int fmt, char* buf, size_t len) {
  const GemvPlan p = plan_gemv(M, N, K, fmt);
  if (fmt == kFmtMxfp4 || fmt == kFmtNvfp4 || fmt == kFmtInt8)
    return snprintf(buf, len,
                    "gemv_mfma_kernel<MT=%d, W=%d, KQ=%d, G=%d, RB=%d, %s> grid=(%u,%u,%d) block=%d lds=%zu split_k=%d",
                    p.MT, p.W, kKQ, group, p.RB, fmt == kFmtMxfp4 ? "MXFP4" : fmt == kFmtNvfp4 ? "NVFP4" : "BITS=8",
                    p.gx, p.gy, p.KS, p.W * 64,
                    p.lds, p.KS);
  if (p.half)
    return snprintf(buf, len, "gemv_mfma_half_kernel<W=%d, KQ=%d, G=%d> grid=(%u,%u,%d) block=%d lds=%zu split_k=%d",
                    p.W, kKQ, group, p.gx, p.gy, p.KS, p.W * 64, p.lds, p.KS);
  if (p.RB > 1)
    return snprintf(buf, len,
                    "gemv_mfma_kernel<MT=%d, W=%d, KQ=%d, G=%d, RB=%d> grid=(%u,%u,%d) block=%d lds=%zu split_k=%d",
                    p.MT, p.W, kKQ, group, p.RB, p.gx, p.gy, p.KS, p.W * 64, p.lds, p.KS);
  return snprintf(buf, len, "gemv_mfma_kernel<MT=%d, W=%d, KQ=%d, G=%d> grid=(%u,%u,%d) block=%d lds=%zu split_k=%d",
                  p.MT, p.W, kKQ, group, p.gx, p.gy, p.KS, p.W * 64, p.lds, p.KS);
}

size_t gemv_workspace_bytes(int64_t M, int64_t N, int64_t K, int, int fmt) {
  const GemvPlan p = plan_gemv(M, N, K, fmt);
  if (p.KS == 1) return 0;
  // partial-sum planes padded to whole tiles: [KS][gy * MT][gx * 16] (gx * 8
  // columns for eight-row workgroups)
  return kSplitCounterBytes + (size_t)p.KS * p.gy * p.MT * p.gx * (p.half ? 8 : 16 * p.RB) * sizeof(float);
}

hipError_t launch_gemv(int64_t M, int64_t N, int64_t K, int group, int fmt, const uint16_t* x,
                       const void* qpacked, const uint16_t* s, const uint8_t* zpacked, uint16_t* y, void* workspace,
                       hipStream_t stream, const float* tscale) {
  const GemvPlan p = plan_gemv(M, N, K, fmt);
  GemvArgs a;
  a.tscale = tscale;
  a.x = x;
  a.qp = static_cast<const uint8_t*>(qpacked);
  a.s = s;
  a.zp = zpacked;
  a.y = y;
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  const int KT = (int)((K + 127) / 128), Gtot = (int)(K / group);
  a.kt_per_split = p.kt_per_split;
  a.KS = p.KS;
  // a segment's scales / zero-points load as vectors when every segment lies
  // inside its row and starts suitably aligned
  const int ns = kKQ * (128 / group);  // groups per segment
  a.sz_vec = (Gtot % ns == 0 && KT % kKQ == 0 && p.kt_per_split % kKQ == 0 &&
              (reinterpret_cast<uintptr_t>(s) & (uintptr_t)(2 * ns > 16 ? 15 : 2 * ns - 1)) == 0 &&
              (fmt == kFmtInt8 || (reinterpret_cast<uintptr_t>(zpacked) & (uintptr_t)(ns / 2 > 8 ? 7 : ns / 2 - 1)) == 0))
                 ? 1
                 : 0;
  if (fmt == kFmtMxfp4 || fmt == kFmtNvfp4)  // 16 (32) scale bytes per segment, one (two) 16-byte loads
    a.sz_vec = (Gtot % ns == 0 && KT % kKQ == 0 && p.kt_per_split % kKQ == 0 &&
                (reinterpret_cast<uintptr_t>(zpacked) & 15) == 0)
                   ? 1
                   : 0;
  a.partial = nullptr;
  a.counters = nullptr;
  if (p.KS > 1) {
    a.counters = static_cast<unsigned*>(workspace);
    a.partial = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + kSplitCounterBytes);
  }
  if (p.MT == 1) return p.W == 16 ? launch_t<1, 16>(p, group, fmt, a, stream) : launch_t<1, 8>(p, group, fmt, a, stream);
  if (p.MT == 2) return launch_t<2, 8>(p, group, fmt, a, stream);
  if (p.MT == 4) return launch_t<4, 8>(p, group, fmt, a, stream);
  if (p.MT == 8) return p.W == 16 ? launch_t<8, 16>(p, group, fmt, a, stream) : launch_t<8, 8>(p, group, fmt, a, stream);
  return launch_t<16, 8>(p, group, fmt, a, stream);
}

}  // namespace wq
