// Device-side helpers shared by the libwq kernels (gfx950 only).
//
// Packed-code tile layout (one 1024-byte tile = 16 rows x 128 columns):
//   lane l = r + 16*c owns bytes [16*l, 16*l + 16) of the tile: four 32-bit
//   words j = 0..3; word j holds columns 32*j + 8*c + e (e = 0..7), column e in
//   nibble 4*(e%2) + e/2.  Shifting a word right by 4*p (p = 0..3) and masking
//   with 0x000F000F leaves the codes of columns 2p and 2p+1 in the two 16-bit
//   halves, which is one fp16 pair after OR-ing in the exponent of 1024.0.
//   That lane/column assignment is also the A/B operand assignment of
//   v_mfma_f32_16x16x32_f16 (lane l: row l%16, eight k values 8*(l/16)..+7),
//   so a word is directly one MFMA B-fragment for the k-slots of step j.
//
// 8-bit codes (group absmax int8) use 2048-byte tiles of the same 16 x 128
// shape: half h = 0, 1 at byte 1024*h holds MFMA steps 2h and 2h + 1; in it
// lane l = r + 16*c owns the 16 bytes at 16*l, whose byte 8*i + e (i = 0, 1)
// is the two's-complement code of column 32*(2h + i) + 8*c + e.  So one
// 16-byte load gives a lane its B operands for two MFMA steps, and a wave's
// load covers 1024 contiguous bytes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wq {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// Code formats of the product kernels: 4-bit asymmetric / symmetric INT4 (with
// fp16 scales and 4-bit zero-points), group absmax int8 (fp16 scales), MXFP4
// (E2M1 codes in the INT4 tile geometry, natural nibble order, one E8M0 scale
// byte per block of 32), NVFP4 (the same codes and layout, one E4M3 scale byte
// per block of 16, one fp32 scale per tensor).
enum : int { kFmtInt4 = 4, kFmtInt8 = 8, kFmtMxfp4 = 2, kFmtNvfp4 = 3 };

// E4M3 scale bytes (0..126: 4 exponent bits with bias 7, 3 mantissa bits;
// exponent field 0 is m * 2^-9) of one 32-bit word, converted in pairs by
// gfx950's OCP FP8 conversions at scale 1: bytes 2 HI and 2 HI + 1 as an fp16
// pair or an fp32 pair, low byte first.  Every E4M3 value is exact in both.
template <bool HI>
__device__ __forceinline__ h2 e4m3_pair_f16(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, HI);
}
template <bool HI>
__device__ __forceinline__ float e4m3_lo_f32(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(word, 1.0f, HI)[0];
}

constexpr int kTileRows = 16;
constexpr int kTileCols = 128;
constexpr int kTileBytes = 1024;
constexpr int kTileBytes8 = 2048;

// fp16 bit pattern of 1024.0: OR-ing a 4-bit code q into the low mantissa bits
// gives exactly 1024 + q.
constexpr uint32_t kMagicPair = 0x64006400u;

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

// (1024 + q_{2p}, 1024 + q_{2p+1}) of one packed word, p = 0..3.
__device__ __forceinline__ h2 biased_pair(uint32_t word, int p) {
  return as_h2(((word >> (4 * p)) & 0x000F000Fu) | kMagicPair);
}

// (1024 + 64*q_{2p}, 1024 + 64*q_{2p+1}) of one packed word, p = 0..3: the code
// lands in mantissa bits 6..9, so the bias 1024 is small next to the code term
// (1024 + 64*15 = 1984 < 2048 keeps every value an exact fp16 integer).
__device__ __forceinline__ h2 biased_pair64(uint32_t word, int p) {
  const uint32_t sh = p == 0 ? (word << 6) : p == 1 ? (word << 2) : p == 2 ? (word >> 2) : (word >> 6);
  return as_h2((sh & 0x03C003C0u) | kMagicPair);
}

// fp16 pair (1152 + q_a, 1152 + q_b) of two int8 codes of a 32-bit word (four
// codes, little-endian): flipping the sign bits turns each code q into the
// unsigned byte q + 128, which v_perm_b32 places under the fp16 exponent of
// 1024.0 (bytes 0x64); sel picks the two bytes (0x04010400: bytes 0 and 1,
// 0x04030402: bytes 2 and 3).  Subtracting 1152 leaves q exactly.
constexpr uint32_t kMagicBytes = 0x64646464u;
__device__ __forceinline__ uint32_t byte_pair(uint32_t word_flipped, uint32_t sel) {
  return __builtin_amdgcn_perm(kMagicBytes, word_flipped, sel);
}

// The fp16 pair (E2M1 code of byte b's low nibble, high nibble) * 2^e, where the
// scale argument's exponent field gives e (v_cvt_scalef32_pk_f16_fp4: fp16
// rounding of the exact product).
template <int B>
__device__ __forceinline__ h2 fp4_pair(uint32_t word, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, scale, B);
}

// 2^(e8 - 127) as fp32 (e8 = 0: the fp32 subnormal 2^-127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t e8) {
  return __builtin_bit_cast(float, e8 == 0 ? 0x00400000u : e8 << 23);
}

// Round-to-nearest-even fp32 -> fp16 bits.
__device__ __forceinline__ uint16_t f32_to_f16_bits(float v) {
  return __builtin_bit_cast(uint16_t, (_Float16)v);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs; NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ int64_t tile_offset_bytes(int64_t nb, int64_t kt, int64_t KT) {
  return (nb * KT + kt) * kTileBytes;
}
__device__ __forceinline__ int64_t tile8_offset_bytes(int64_t nb, int64_t kt, int64_t KT) {
  return (nb * KT + kt) * kTileBytes8;
}

// Zero-point of (row n, group gi) from the packed [N][ceil(G/2)] array.
__device__ __forceinline__ uint32_t load_zero(const uint8_t* zpacked, int64_t GB, int64_t n, int64_t gi) {
  uint32_t b = zpacked[n * GB + (gi >> 1)];
  return (gi & 1) ? (b >> 4) : (b & 15u);
}

// ---- Split-K hand-off between the workgroups that share one output tile.
// The workspace starts with a fixed counter region (one 32-bit counter per
// output tile; a split launch never has more than kSplitMaxTiles tiles) and
// holds the fp32 partial sums after it.  Counters start at zero and the last
// workgroup of a tile puts its counter back to zero, so one zero-filled
// workspace serves later launches of any shape; the partial sums are fully
// overwritten by every launch and need no clearing.
constexpr int kSplitMaxTiles = 512;
constexpr size_t kSplitCounterBytes = kSplitMaxTiles * sizeof(unsigned);

// Partial sums travel through device-scope relaxed atomic stores and loads
// (cache-coherent across the chiplets' separate L2 caches), so no whole-cache
// write-back or invalidate is needed: a workgroup's stores are complete before
// its counter increment (waitcnt + barrier below), and the last workgroup
// issues its loads only after its own increment has returned.
__device__ __forceinline__ void split_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float split_load(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Called by every thread of the workgroup after its split_store calls; true in
// the workgroup that arrives last at counter `ctr` (of KS arrivals).
__device__ __forceinline__ bool split_arrive(unsigned* ctr, int KS) {
  __shared__ unsigned last;
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's stores are acknowledged
  __syncthreads();
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(KS - 1);
  __syncthreads();
  return last != 0;
}

// The last workgroup of a tile resets its counter for the next launch.
__device__ __forceinline__ void split_reset(unsigned* ctr) {
  __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace wq
