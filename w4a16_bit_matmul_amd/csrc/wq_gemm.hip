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
// 16-byte loads (sixteen threads per row) two tiles ahead of use into
// registers and stores them, one step before their use, into one of two LDS
// buffers; chunk cc of row R sits in slot cc ^ (R % 16) of its row, so the
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

// Forces a value into a VGPR and hides it from constant folding, so that
// v_and_or_b32 takes the mask from an SGPR and the fp16 exponent from here.
__device__ __forceinline__ uint32_t in_vgpr(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
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

// LDS bytes of one staged chunk for the workgroup's 128 weight rows:
// g = 128: [tile][row] u32 (scale bits, zero-point in bits 16..19);
// g = 32: [tile][pair][row] u32 (scales of groups 4t + 2q, 4t + 2q + 1), then
// [tile][row] u16 (the tile's four zero-points, group 4t in bits 0..3);
// MXFP4: [tile][row] u32 (the tile's four E8M0 scale bytes, block 4t first).
template <int G, int FMT = kFmtInt4>
constexpr int sz_chunk_bytes() {
  return (G == 128 || FMT == kFmtMxfp4) ? kSzChunk * 128 * 4 : kSzChunk * 2 * 128 * 4 + kSzChunk * 128 * 2;
}

// SZV: every row of s (and zpacked) is aligned for the wide staging loads.
// FMT: kFmtInt4 (codes and zero-points), kFmtInt8 (int8 codes, no
// zero-points) or kFmtMxfp4 (E2M1 codes, E8M0 scale bytes in a.zp, G = 32).
template <int MB, int G, bool SZV, int FMT>
__global__ __launch_bounds__(kWaves * 64) void gemm_kernel(GemmArgs a) {
  static_assert(FMT == kFmtInt4 || FMT == kFmtInt8 || (FMT == kFmtMxfp4 && G == 32), "code format");
  constexpr int BITS = FMT == kFmtInt8 ? 8 : 4;
  using CodeT = std::conditional_t<BITS == 4, uint2, u4>;  // one wave's two MFMA steps of a tile
  constexpr int TB = BITS == 4 ? kTileBytes : kTileBytes8;
  constexpr int NPW = kNPW;
  constexpr int NTH = kWaves * 64;
  constexpr int ROWS = 16 * MB;
  constexpr int XTILE = ROWS * 256;                            // one K tile of activations in LDS
  constexpr int XCH = ROWS * 16 >= NTH ? ROWS * 16 / NTH : 1;  // 16-byte chunks per thread per tile
  constexpr int SZB = sz_chunk_bytes<G, FMT>();
  static_assert(ROWS * 16 % NTH == 0 || NTH % (ROWS * 16) == 0, "whole chunks per thread");
  extern __shared__ __align__(16) uint8_t smem[];  // [2][XTILE] activations, [2][SZB] scales

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int jp = wv >> 2, cgp = wv & 3;
  const int r = lane & 15, c = lane >> 4;
  const int nwg0 = blockIdx.x * 8 * 16;  // first weight row of the workgroup
  const int nbw0 = blockIdx.x * 8 + cgp * NPW;
  const int mrow0 = blockIdx.y * ROWS;
  const uint32_t magic = in_vgpr(kMagicPair);
  const int KT = a.KT;

  // the codes of MFMA steps 2jp, 2jp + 1 in each of the wave's blocks: 4-bit,
  // words 2jp and 2jp + 1 of the lane's 16 bytes; 8-bit, the lane's 16 bytes
  // of half jp (blocks past the end re-read the last one)
  const uint8_t* tb[NPW];
#pragma unroll
  for (int b = 0; b < NPW; ++b)
    tb[b] = a.qp + (size_t)min(nbw0 + b, a.NBLK - 1) * KT * TB + 16u * lane + (BITS == 4 ? 8u : 1024u) * jp;
  // With few rows (MB <= 2) the kernel streams codes at HBM speed and
  // non-temporal loads measure faster; with more rows they do not.
  auto load_b = [&](int kt, CodeT (&d)[NPW]) {
    kt = min(kt, KT - 1);  // tiles past the end re-load the last (unused)
#pragma unroll
    for (int b = 0; b < NPW; ++b) {
      const uint8_t* p = tb[b] + (size_t)kt * TB;
      if constexpr (MB > 2) {
        d[b] = *reinterpret_cast<const CodeT*>(p);
      } else if constexpr (BITS == 4) {
        typedef uint32_t v2 __attribute__((ext_vector_type(2)));
        const v2 t = __builtin_nontemporal_load(reinterpret_cast<const v2*>(p));
        d[b] = CodeT{t.x, t.y};
      } else {
        d[b] = __builtin_nontemporal_load(reinterpret_cast<const CodeT*>(p));
      }
    }
  };

  // activation chunk q = tid + NTH * i: row q / 16 of the tile, global chunk
  // q % 16 (with fewer chunks than threads, threads share chunks and store
  // the same bytes).  Rows past M re-read row M - 1; in a ragged last tile,
  // chunks past K re-read the last chunk inside K (K is a multiple of 32, so
  // an MFMA step lies wholly inside K or is skipped).
  const uint16_t* xrow[XCH];
  uint32_t xlds[XCH];
  const int xcc = tid & 15;
#pragma unroll
  for (int i = 0; i < XCH; ++i) {
    const int row = ((tid >> 4) + (NTH / 16) * i) % ROWS;
    xrow[i] = a.x + (size_t)min(mrow0 + row, a.M - 1) * a.K;
    xlds[i] = (uint32_t)(row * 256 + 16 * (xcc ^ (row & 15)));
  }
  auto load_x = [&](int kt, u4 (&v)[XCH]) {
    const int col = min(min(kt, KT - 1) * 128 + 8 * xcc, a.K - 8);
#pragma unroll
    for (int i = 0; i < XCH; ++i) v[i] = *reinterpret_cast<const u4*>(xrow[i] + col);
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
  auto sz_store = [&](int chunk, const SzStage& v) {
    uint8_t* buf = szbase + (chunk & 1) * SZB;
    if constexpr (FMT == kFmtMxfp4) {
      *reinterpret_cast<uint32_t*>(buf + (2 * sp) * 512 + 4 * sn) = v.s[0];
      *reinterpret_cast<uint32_t*>(buf + (2 * sp + 1) * 512 + 4 * sn) = v.s[1];
    } else if constexpr (G == 128) {
      const uint32_t s0 = SZV ? v.s[0] & 0xffffu : v.s[0];
      const uint32_t s1 = SZV ? v.s[0] >> 16 : v.s[1];
      // tiles 2p (low nibble) and 2p + 1 (high nibble) share a zero-point byte
      *reinterpret_cast<uint32_t*>(buf + (2 * sp) * 512 + 4 * sn) = s0 | ((v.z & 15u) << 16);
      *reinterpret_cast<uint32_t*>(buf + (2 * sp + 1) * 512 + 4 * sn) = s1 | ((v.z >> 4) << 16);
    } else {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
#pragma unroll
        for (int q = 0; q < 2; ++q)
          *reinterpret_cast<uint32_t*>(buf + ((2 * sp + e) * 2 + q) * 512 + 4 * sn) = v.s[2 * e + q];
        *reinterpret_cast<uint16_t*>(buf + kSzChunk * 1024 + (2 * sp + e) * 256 + 2 * sn) =
            (uint16_t)(v.z >> (16 * e));
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

  // ---- prologue: activations of the first tile (in LDS) and the second (in
  // registers), codes of the first three tiles, scales / zero-points of the
  // first chunk
  CodeT b0[NPW], b1[NPW], b2[NPW], b3[NPW];
  u4 xs0[XCH], xs1[XCH];
  SzStage szs;
  load_x(kt_lo, xs0);
  load_x(kt_lo + 1, xs1);
  load_b(kt_lo, b0);
  load_b(kt_lo + 1, b1);
  load_b(kt_lo + 2, b2);
  sz_load(kt_lo / kSzChunk, szs);
  store_x(kt_lo, xs0);
  sz_store(kt_lo / kSzChunk, szs);
  lds_barrier();

  // this lane's A reads: row r of block i, chunk 4j + c at slot (4j + c) ^ r;
  // its scale / zero entries: rows (cg*NPW + b)*16 + r of the workgroup
  const uint8_t* const arow = smem + r * 256;
  const int szrow = cgp * NPW * 16 + r;

  // One step (K tile kt): load the activations of tile kt + 2 and the codes
  // of tile kt + 3, multiply tile kt, and store the activations of tile
  // kt + 1 (loaded one step earlier) into the other LDS buffer.
  auto step = [&](auto full_tag, int kt, u4 (&xld)[XCH], const u4 (&xst)[XCH], const CodeT (&cur)[NPW],
                  CodeT (&nxt)[NPW]) {
    constexpr bool FULL = decltype(full_tag)::value;
    load_x(kt + 2, xld);
    __builtin_amdgcn_sched_barrier(0);
    load_b(kt + 3, nxt);
    // scale / zero-point of this tile for the wave's blocks
    const uint8_t* szt = szbase + ((kt / kSzChunk) & 1) * SZB;
    const int tt = kt % kSzChunk;
    uint32_t sv[NPW], zv[NPW];
#pragma unroll
    for (int b = 0; b < NPW; ++b) {
      if constexpr (FMT == kFmtMxfp4) {
        sv[b] = *reinterpret_cast<const uint32_t*>(szt + tt * 512 + 4 * (szrow + 16 * b));
        zv[b] = 0u;
      } else if constexpr (G == 128) {
        sv[b] = *reinterpret_cast<const uint32_t*>(szt + tt * 512 + 4 * (szrow + 16 * b));
        zv[b] = sv[b] >> 16;
      } else {
        sv[b] = *reinterpret_cast<const uint32_t*>(szt + (tt * 2 + jp) * 512 + 4 * (szrow + 16 * b));
        zv[b] = (uint32_t)*reinterpret_cast<const uint16_t*>(szt + kSzChunk * 1024 + tt * 256 + 2 * (szrow + 16 * b)) >>
                (8 * jp);
      }
    }
    const uint8_t* abuf = arow + (kt & 1) * XTILE;
    auto mstep = [&](int jj) {
      const int j = 2 * jp + jj;
      if (!FULL && kt * 128 + 32 * j >= a.K) return;  // ragged last tile
      const int slot = ((4 * j + c) ^ r) * 16;
      h8 af[MB];
#pragma unroll
      for (int i = 0; i < MB; ++i) af[i] = *reinterpret_cast<const h8*>(abuf + i * 16 * 256 + slot);
#pragma unroll
      for (int b = 0; b < NPW; ++b) {
        h8 bf;
        const uint32_t sb = G == 128 ? sv[b] & 0xffffu : (jj ? sv[b] >> 16 : sv[b] & 0xffffu);
        const h2 sc = as_h2(sb * 0x00010001u);
        if constexpr (FMT == kFmtMxfp4) {
          // block 4 kt + j: byte j of the tile's scale word (exponent field only)
          const float scale = __builtin_bit_cast(float, ((sv[b] >> (8 * j)) & 0xffu) << 23);
          bf = dequant_word_mx(jj ? cur[b].y : cur[b].x, scale);
        } else if constexpr (FMT == kFmtInt4) {
          const uint32_t z = G == 128 ? zv[b] & 15u : (zv[b] >> (4 * jj)) & 15u;
          const h2 nbias = -as_h2(z * 0x00010001u + magic);
          bf = dequant_word(jj ? cur[b].y : cur[b].x, magic, nbias, sc);
        } else {
          bf = dequant_words8(jj ? cur[b][2] : cur[b][0], jj ? cur[b][3] : cur[b][1], sc);
        }
#pragma unroll
        for (int i = 0; i < MB; ++i) acc[i][b] = mfma16(af[i], bf, acc[i][b]);
      }
    };
    mstep(0);
    // the other buffer was last read before the previous barrier
    store_x(kt + 1, xst);
    mstep(1);
    lds_barrier();
  };
  using Full = std::integral_constant<bool, true>;
  using Part = std::integral_constant<bool, false>;

  // whole tiles in groups of eight (two turns of the code ring, four of the
  // activation registers); the next chunk's scales / zero-points are loaded
  // at step 1 and stored at step 5
  const int kt_full = kt_lo + ((min(kt_hi, a.K / 128) - kt_lo) & ~(kSzChunk - 1));
  int kt = kt_lo;
  for (; kt < kt_full; kt += kSzChunk) {
    const int ch = kt / kSzChunk;
    step(Full{}, kt, xs0, xs1, b0, b3);
    sz_load(ch + 1, szs);
    step(Full{}, kt + 1, xs1, xs0, b1, b0);
    step(Full{}, kt + 2, xs0, xs1, b2, b1);
    step(Full{}, kt + 3, xs1, xs0, b3, b2);
    step(Full{}, kt + 4, xs0, xs1, b0, b3);
    sz_store(ch + 1, szs);
    step(Full{}, kt + 5, xs1, xs0, b1, b0);
    step(Full{}, kt + 6, xs0, xs1, b2, b1);
    step(Full{}, kt + 7, xs1, xs0, b3, b2);
  }
  // the rest (fewer than eight tiles, the last one possibly ragged); their
  // chunk was staged during the previous chunk or before the loop
  for (; kt < kt_hi; kt += 4) {
    step(Part{}, kt, xs0, xs1, b0, b3);
    if (kt + 1 < kt_hi) step(Part{}, kt + 1, xs1, xs0, b1, b0);
    if (kt + 2 < kt_hi) step(Part{}, kt + 2, xs0, xs1, b2, b1);
    if (kt + 3 < kt_hi) step(Part{}, kt + 3, xs1, xs0, b3, b2);
  }

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
            a.y[(size_t)m * a.N + n] = f32_to_f16_bits(v);
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
      if (n < a.N && m < a.M) a.y[(size_t)m * a.N + n] = f32_to_f16_bits(v[j]);
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

dim3 gemm_grid(int MB, int64_t M, int64_t N) {
  return dim3((unsigned)(((N + 15) / 16 + 7) / 8), (unsigned)((M + 16 * MB - 1) / (16 * MB)));
}

size_t gemm_lds(int MB, int group, int fmt) {
  // two activation buffers and two staged chunks of scales / zero-points; the
  // final reduction ([4][MB*NPW*4][64] fp32) reuses the front of it
  const size_t tiles =
      (size_t)2 * MB * 16 * 256 +
      2 * (size_t)(fmt == kFmtMxfp4 ? sz_chunk_bytes<32, kFmtMxfp4>()
                                    : group == 128 ? sz_chunk_bytes<128>() : sz_chunk_bytes<32>());
  const size_t red = (size_t)4 * MB * kNPW * 4 * 64 * sizeof(float);
  return tiles > red ? tiles : red;
}

template <int MB, int G, bool SZV, int FMT>
hipError_t launch_kg(const GemmArgs& a, hipStream_t stream) {
  const dim3 g2 = gemm_grid(MB, a.M, a.N), grid(g2.x, g2.y, (unsigned)a.KS), block(kWaves * 64);
  const size_t lds = gemm_lds(MB, G, FMT);
  auto k = gemm_kernel<MB, G, SZV, FMT>;
  static std::atomic<uint64_t> lds_raised{0};
  const hipError_t e = raise_lds_limit((const void*)k, lds, lds_raised);
  if (e != hipSuccess) return e;
  k<<<grid, block, lds, stream>>>(a);
  return hipGetLastError();
}

template <int MB, int FMT>
hipError_t launch_t(int group, const GemmArgs& a, hipStream_t stream) {
  // wide staging loads of scales / zero-points when every row is aligned for
  // them: g = 128 two scales (4 bytes); g = 32 eight scales (16 bytes) and
  // eight zero-points (4 bytes); MXFP4 eight scale bytes
  const uintptr_t sp = reinterpret_cast<uintptr_t>(a.s), zp = reinterpret_cast<uintptr_t>(a.zp);
  if constexpr (FMT == kFmtMxfp4) {
    if (a.Gtot % 8 == 0 && zp % 8 == 0) return launch_kg<MB, 32, true, FMT>(a, stream);
    return launch_kg<MB, 32, false, FMT>(a, stream);
  } else {
    if (group == 128) {
      if (a.Gtot % 2 == 0 && sp % 4 == 0) return launch_kg<MB, 128, true, FMT>(a, stream);
      return launch_kg<MB, 128, false, FMT>(a, stream);
    }
    if (a.Gtot % 8 == 0 && sp % 16 == 0 && (FMT == kFmtInt8 || zp % 4 == 0))
      return launch_kg<MB, 32, true, FMT>(a, stream);
    return launch_kg<MB, 32, false, FMT>(a, stream);
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
                  kNPW, group, fmt == kFmtInt8 ? ", BITS=8" : fmt == kFmtMxfp4 ? ", MXFP4" : "", p.gx, p.gy, p.KS,
                  kWaves * 64, gemm_lds(p.MB, group, fmt), p.KS);
}

hipError_t launch_gemm(int64_t M, int64_t N, int64_t K, int group, int fmt, const uint16_t* x, const void* qpacked,
                       const uint16_t* s, const uint8_t* zpacked, uint16_t* y, void* workspace,
                       hipStream_t stream) {
  const GemmPlan p = plan_gemm(M, N, K);
  GemmArgs a;
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
  if (fmt == kFmtInt8) {
    switch (gemm_mb(M, N, K)) {
      case 1: return launch_t<1, kFmtInt8>(group, a, stream);
      case 2: return launch_t<2, kFmtInt8>(group, a, stream);
      case 4: return launch_t<4, kFmtInt8>(group, a, stream);
      default: return launch_t<8, kFmtInt8>(group, a, stream);
    }
  }
  if (fmt == kFmtMxfp4) {
    switch (gemm_mb(M, N, K)) {
      case 1: return launch_t<1, kFmtMxfp4>(group, a, stream);
      case 2: return launch_t<2, kFmtMxfp4>(group, a, stream);
      case 4: return launch_t<4, kFmtMxfp4>(group, a, stream);
      default: return launch_t<8, kFmtMxfp4>(group, a, stream);
    }
  }
  switch (gemm_mb(M, N, K)) {
    case 1: return launch_t<1, kFmtInt4>(group, a, stream);
    case 2: return launch_t<2, kFmtInt4>(group, a, stream);
    case 4: return launch_t<4, kFmtInt4>(group, a, stream);
    default: return launch_t<8, kFmtInt4>(group, a, stream);
  }
}

}  // namespace wq
