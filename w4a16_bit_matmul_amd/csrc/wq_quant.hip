// Group quantization, packing and dequantization kernels (gfx950).
//
// Method: "Quantization for LLM inference: FP8, INT4 (GPTQ, AWQ) and GGUF -
// the model's accounting zoom", section "The minimum maths: scale and
// zero-point" (s = (max - min) / 15, z = round(-min / s),
// q = clip(round(w / s + z), 0, 15), decoding s * (q - z)) and section
// "Numerical example" (8 codes in 4 bytes, a 4-bit zero-point in half a byte).
// Symmetric variant: "Test-time quantization", section "The maths that
// matter" (b-bit symmetric range, s = M / (2^(b-1) - 1)) with the code of
// "Quantization Methods Compared", section "What quantisation does"
// (q = round(w / s)); at b = 4 the code q in [-7, 7] is stored as q + 8 with
// zero-point 8, so every kernel that decodes s * (q - z) decodes it.
// Group absmax int8 (same page and section: s = max|w| / 127, q = round(w / s),
// decoding q * s) keeps one fp16 scale per group, no zero-point, and 8-bit
// codes in 2048-byte tiles (16 rows x 128 columns).
// MXFP4 ("Quantization for LLM inference", section "Microscaling: NVFP4 and
// MXFP4", in the format of the microscaling paper it cites): E2M1 codes, one
// E8M0 power-of-two scale per block of 32 along K, in the 1 KB tiles with
// natural nibble order (two neighbouring columns per byte, as the hardware's
// FP4 conversion takes them).
// INT4 KV cache ("Quantization for LLM inference", section "KV cache
// quantization": int4 in blocks of 128): each token's K or V vector is cut into
// blocks of 128 values, each block quantized like a weight group, the rows
// scattered to caller-chosen cache slots.
//
// This translation unit is compiled with -ffp-contract=off: every fp32
// operation below is one correctly rounded IEEE operation (division is the
// correctly rounded HIP default), so codes, scales and zero-points are
// bit-identical to any other implementation of the same steps.
//
// Work decomposition: one wavefront per (16-row block, pair of 128-column
// tiles).  Lane l = r + 16*c reads the 32 weights of row r that its 16 bytes of
// the packed tile hold (columns 32*j + 8*c + e), so each wave writes whole
// 1024-byte tiles with one 16-byte store per lane, and a group's min/max is a
// reduction over the four lanes r, r+16, r+32, r+48 (two xor-shuffles).
#include <algorithm>

#include "wq_device.h"
#include "wq_kernels.h"

namespace wq {
namespace {

constexpr int kWavesPerBlock = 4;

template <int DT>
__device__ __forceinline__ void load8(const void* W, int64_t idx, float* out) {
  if constexpr (DT == 0) {  // fp32
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(W) + idx);
    float4 a = p[0], b = p[1];
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  } else {
    uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(W) + idx);
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (DT == 1) {  // bf16: exact widening
        out[2 * i] = __builtin_bit_cast(float, w[i] << 16);
        out[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
      } else {  // fp16: exact widening
        out[2 * i] = f16_bits_to_f32((uint16_t)(w[i] & 0xffffu));
        out[2 * i + 1] = f16_bits_to_f32((uint16_t)(w[i] >> 16));
      }
    }
  }
}

__device__ __forceinline__ float wave_min4(float v) {
  v = fminf(v, __shfl_xor(v, 16));
  v = fminf(v, __shfl_xor(v, 32));
  return v;
}
__device__ __forceinline__ float wave_max4(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

// Scale (fp16 bits), its fp32 value, an approximate reciprocal of it and the
// zero-point of a group whose min and max are lo and hi.
struct GroupParams {
  uint16_t s_bits;
  float s;
  float r;  // v_rcp_f32(s): only steers the rounding shortcut below
  float z;
};

__device__ __forceinline__ GroupParams group_params(float lo, float hi) {
  lo = fminf(lo, 0.0f);  // range widened to contain 0: z is then a code
  hi = fmaxf(hi, 0.0f);
  float range = hi - lo;
  float s32 = range / 15.0f;
  GroupParams p;
  p.s_bits = f32_to_f16_bits(s32);
  p.s = f16_bits_to_f32(p.s_bits);
  p.r = __builtin_amdgcn_rcpf(p.s);
  if (p.s == 0.0f) {  // degenerate group: s = 0, z = 0, codes 0
    p.s_bits = 0;
    p.z = 0.0f;
    return p;
  }
  float z = rintf(-lo / p.s);
  p.z = fminf(fmaxf(z, 0.0f), 15.0f);
  return p;
}

// Symmetric 4-bit: s = max|w| / 7 (max|w| = max(hi, -lo)), zero-point 8; a
// group whose fp16 scale is 0 stores s = 0 and codes 8.
__device__ __forceinline__ GroupParams group_params_sym(float lo, float hi) {
  const float m = fmaxf(hi, -lo);
  const float s32 = m / 7.0f;
  GroupParams p;
  p.s_bits = f32_to_f16_bits(s32);
  p.s = f16_bits_to_f32(p.s_bits);
  p.r = __builtin_amdgcn_rcpf(p.s);
  p.z = 8.0f;
  if (p.s == 0.0f) p.s_bits = 0;
  return p;
}

// rne(fl32(fl32(w / s) + z)) -- the encoding's two correctly rounded fp32
// operations and the rounding to an integer -- without the division wherever
// it cannot matter.  t = fma(w, r, z) with r = v_rcp_f32(s) (1 ulp) lies within
// |w/s| * 2^-22 + ulp(t) of the real w/s + z, and the exact steps lie within
// 2^-24 * (|w/s| + |t|) of it; with |w/s| <= 2^(B-1) + 1 for B-bit codes both
// are below 2^(B-1) * 2^-21.  So when t is farther than `margin` (2^-14 for
// 4-bit codes, 2^-10 for 8-bit: room for an rcp error of 16 ulp) from every
// half-integer, t, the real value and the exact result all round to the same
// integer; otherwise the exact steps run.
__device__ __forceinline__ float round_quotient(float w, const GroupParams& p, float z, float margin) {
  const float t = fmaf(w, p.r, z);
  const float f = t - floorf(t);  // exact for |t| < 2^23
  if (fabsf(f - 0.5f) > margin) return rintf(t);
  const float u = w / p.s;  // correctly rounded
  return rintf(u + z);
}

__device__ __forceinline__ uint32_t encode_sym(float w, const GroupParams& p) {
  if (p.s == 0.0f) return 8u;
  float r = round_quotient(w, p, 0.0f, 0x1p-14f);
  r = fminf(fmaxf(r, -7.0f), 7.0f);
  return (uint32_t)(r + 8.0f);
}

__device__ __forceinline__ uint32_t encode(float w, const GroupParams& p) {
  if (p.s == 0.0f) return 0u;
  float r = round_quotient(w, p, p.z, 0x1p-14f);
  r = fminf(fmaxf(r, 0.0f), 15.0f);
  return (uint32_t)r;
}

// Group absmax int8: s = max|w| / 127; a group whose fp16 scale is 0 stores
// s = 0 and codes 0.
__device__ __forceinline__ GroupParams group_params_w8(float lo, float hi) {
  const float m = fmaxf(hi, -lo);
  const float s32 = m / 127.0f;
  GroupParams p;
  p.s_bits = f32_to_f16_bits(s32);
  p.s = f16_bits_to_f32(p.s_bits);
  p.r = __builtin_amdgcn_rcpf(p.s);
  p.z = 0.0f;
  if (p.s == 0.0f) p.s_bits = 0;
  return p;
}

__device__ __forceinline__ uint32_t encode_w8(float w, const GroupParams& p) {
  if (p.s == 0.0f) return 0u;
  float r = round_quotient(w, p, 0.0f, 0x1p-10f);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (uint32_t)(int)r & 0xffu;  // two's-complement byte
}

// Nibble position of column e (0..7) inside a packed word.
__device__ __forceinline__ int nibble_pos(int e) { return 4 * (e & 1) + (e >> 1); }

// SCALED: each weight is first multiplied by its input channel's factor
// alpha[k] (the AWQ fold, one fp32 multiplication).  At g = 128 without the
// fold the kernel fits 64 VGPRs, which lets eight workgroups share a CU instead
// of six or seven (bf16 8192 x 8192: 56.3 -> 44.0 us); the other instances
// would spill at that bound (g = 32 measured 59 -> 78 us) and keep theirs.
template <int DT, int G, bool SYM, bool SCALED>
__global__ __launch_bounds__(256, (G == 128 && !SCALED) ? 8 : 1) void quantize_kernel(
    const void* __restrict__ W, int64_t N, int64_t K, int64_t NBLK, int64_t KT, const float* __restrict__ alpha,
    uint8_t* __restrict__ q_codes, uint16_t* __restrict__ s_out, uint8_t* __restrict__ z_codes,
    uint32_t* __restrict__ qpacked, uint8_t* __restrict__ zpacked) {
  const int lane = threadIdx.x & 63;
  const int64_t ST = (KT + 1) / 2;
  const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (item >= NBLK * ST) return;  // whole wave exits together
  const int64_t nb = item / ST, st = item % ST;
  const int r = lane & 15, c = lane >> 4;
  const int64_t n = nb * 16 + r;
  const bool row_ok = n < N;
  const int64_t Gtot = K / G;
  const int64_t GB = (Gtot + 1) / 2;

  uint32_t zkeep[2][4] = {{0, 0, 0, 0}, {0, 0, 0, 0}};

  for (int t = 0; t < 2; ++t) {
    const int64_t kt = 2 * st + t;
    if (kt >= KT) break;
    float w[4][8];
    bool jok[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t k0 = kt * 128 + 32 * j + 8 * c;
      jok[j] = row_ok && (kt * 128 + 32 * j < K);
      if (jok[j]) {
        load8<DT>(W, n * K + k0, w[j]);
        if constexpr (SCALED) {
          const float4 a0 = *reinterpret_cast<const float4*>(alpha + k0);
          const float4 a1 = *reinterpret_cast<const float4*>(alpha + k0 + 4);
          const float a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) w[j][e] = w[j][e] * a[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) w[j][e] = 0.0f;
      }
    }

    GroupParams gp[4];
    if constexpr (G == 128) {
      float lo = w[0][0], hi = w[0][0];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) { lo = fminf(lo, w[j][e]); hi = fmaxf(hi, w[j][e]); }
      lo = wave_min4(lo);
      hi = wave_max4(hi);
      GroupParams p = SYM ? group_params_sym(lo, hi) : group_params(lo, hi);
#pragma unroll
      for (int j = 0; j < 4; ++j) gp[j] = p;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float lo = w[j][0], hi = w[j][0];
#pragma unroll
        for (int e = 1; e < 8; ++e) { lo = fminf(lo, w[j][e]); hi = fmaxf(hi, w[j][e]); }
        lo = wave_min4(lo);
        hi = wave_max4(hi);
        gp[j] = SYM ? group_params_sym(lo, hi) : group_params(lo, hi);
      }
    }

    uint32_t words[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t word = 0;
      uint32_t codes[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        codes[e] = jok[j] ? (SYM ? encode_sym(w[j][e], gp[j]) : encode(w[j][e], gp[j])) : 0u;
        word |= codes[e] << (4 * nibble_pos(e));
      }
      words[j] = word;
      if (q_codes && jok[j]) {
        const int64_t k0 = kt * 128 + 32 * j + 8 * c;
        uint2 lohi;
        lohi.x = codes[0] | (codes[1] << 8) | (codes[2] << 16) | (codes[3] << 24);
        lohi.y = codes[4] | (codes[5] << 8) | (codes[6] << 16) | (codes[7] << 24);
        *reinterpret_cast<uint2*>(q_codes + n * K + k0) = lohi;
      }
      zkeep[t][j] = (uint32_t)gp[j].z;
    }
    if (qpacked) {
      u4 v = {words[0], words[1], words[2], words[3]};
      *reinterpret_cast<u4*>(reinterpret_cast<uint8_t*>(qpacked) + tile_offset_bytes(nb, kt, KT) + 16 * lane) = v;
    }
    if (row_ok) {
      if constexpr (G == 128) {
        if (c == 0) {
          s_out[n * Gtot + kt] = gp[0].s_bits;
          if (z_codes) z_codes[n * Gtot + kt] = (uint8_t)gp[0].z;
        }
      } else {
        // lane c writes group j = c of this tile
        const int64_t gi = kt * 4 + c;
        if (gi < Gtot) {
          uint16_t sb = c == 0 ? gp[0].s_bits : c == 1 ? gp[1].s_bits : c == 2 ? gp[2].s_bits : gp[3].s_bits;
          float zz = c == 0 ? gp[0].z : c == 1 ? gp[1].z : c == 2 ? gp[2].z : gp[3].z;
          s_out[n * Gtot + gi] = sb;
          if (z_codes) z_codes[n * Gtot + gi] = (uint8_t)zz;
        }
      }
    }
  }

  if (zpacked && row_ok) {
    if constexpr (G == 128) {
      // groups 2*st and 2*st + 1 share byte st
      if (c == 0 && st < GB) zpacked[n * GB + st] = (uint8_t)(zkeep[0][0] | (zkeep[1][0] << 4));
    } else {
      // groups 8*st .. 8*st+7 -> bytes 4*st .. 4*st+3; lane c writes byte 4*st + c
      const int64_t b = st * 4 + c;
      if (b < GB) {
        const int t = c >> 1;            // tile of group 8*st + 2c
        const int j0 = (2 * c) & 3;      // its column group inside the tile
        uint32_t lo = zkeep[t][j0];
        uint32_t hi = (2 * b + 1 < Gtot) ? zkeep[t][j0 + 1] : 0u;
        zpacked[n * GB + b] = (uint8_t)(lo | (hi << 4));
      }
    }
  }
}

// Codes [N][K] and zero-points [N][G] -> tile-layout codes and packed zeros.
template <int G>
__global__ __launch_bounds__(256) void pack_kernel(
    const uint8_t* __restrict__ q_codes, const uint8_t* __restrict__ z_codes, int64_t N, int64_t K,
    int64_t NBLK, int64_t KT, uint32_t* __restrict__ qpacked, uint8_t* __restrict__ zpacked) {
  const int lane = threadIdx.x & 63;
  const int64_t ST = (KT + 1) / 2;
  const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (item >= NBLK * ST) return;
  const int64_t nb = item / ST, st = item % ST;
  const int r = lane & 15, c = lane >> 4;
  const int64_t n = nb * 16 + r;
  const bool row_ok = n < N;
  const int64_t Gtot = K / G;
  const int64_t GB = (Gtot + 1) / 2;

  for (int t = 0; t < 2; ++t) {
    const int64_t kt = 2 * st + t;
    if (kt >= KT) break;
    uint32_t words[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t k0 = kt * 128 + 32 * j + 8 * c;
      uint32_t word = 0;
      if (row_ok && kt * 128 + 32 * j < K) {
        uint2 v = *reinterpret_cast<const uint2*>(q_codes + n * K + k0);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          uint32_t code = ((e < 4 ? v.x >> (8 * e) : v.y >> (8 * (e - 4)))) & 15u;
          word |= code << (4 * nibble_pos(e));
        }
      }
      words[j] = word;
    }
    u4 out = {words[0], words[1], words[2], words[3]};
    *reinterpret_cast<u4*>(reinterpret_cast<uint8_t*>(qpacked) + tile_offset_bytes(nb, kt, KT) + 16 * lane) = out;
  }
  if (row_ok) {
    // this item's 256 columns hold 256/G groups -> 128/G bytes of zpacked
    constexpr int kBytes = 128 / G;
    if (c < kBytes) {
      const int64_t b = st * kBytes + c;
      if (b < GB) {
        uint32_t lo = z_codes[n * Gtot + 2 * b] & 15u;
        uint32_t hi = (2 * b + 1 < Gtot) ? (z_codes[n * Gtot + 2 * b + 1] & 15u) : 0u;
        zpacked[n * GB + b] = (uint8_t)(lo | (hi << 4));
      }
    }
  }
}

// Tile-layout codes + scales + zeros -> What[N][K] = s * (q - z).
template <int OUT, int G>
__global__ __launch_bounds__(256) void dequant_kernel(
    const uint32_t* __restrict__ qpacked, const uint16_t* __restrict__ s_in, const uint8_t* __restrict__ zpacked,
    int64_t N, int64_t K, int64_t NBLK, int64_t KT, void* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (item >= NBLK * KT) return;
  const int64_t nb = item / KT, kt = item % KT;
  const int r = lane & 15, c = lane >> 4;
  const int64_t n = nb * 16 + r;
  if (n >= N) return;
  const int64_t Gtot = K / G;
  const int64_t GB = (Gtot + 1) / 2;
  const u4 v = *reinterpret_cast<const u4*>(reinterpret_cast<const uint8_t*>(qpacked) +
                                            tile_offset_bytes(nb, kt, KT) + 16 * lane);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t k0 = kt * 128 + 32 * j + 8 * c;
    if (k0 >= K) continue;
    const int64_t gi = k0 / G;
    const float s = f16_bits_to_f32(s_in[n * Gtot + gi]);
    const int z = (int)load_zero(zpacked, GB, n, gi);
    const uint32_t word = v[j];
    float d[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int q = (int)((word >> (4 * nibble_pos(e))) & 15u);
      d[e] = s * (float)(q - z);  // exact: 11-bit significand times |q - z| <= 15
    }
    if constexpr (OUT == 0) {
      float4* o = reinterpret_cast<float4*>(static_cast<float*>(out) + n * K + k0);
      o[0] = make_float4(d[0], d[1], d[2], d[3]);
      o[1] = make_float4(d[4], d[5], d[6], d[7]);
    } else {
      uint32_t p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t a = OUT == 2 ? f32_to_f16_bits(d[2 * i]) : f32_to_bf16_bits(d[2 * i]);
        uint32_t b = OUT == 2 ? f32_to_f16_bits(d[2 * i + 1]) : f32_to_bf16_bits(d[2 * i + 1]);
        p[i] = a | (b << 16);
      }
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + n * K + k0) = make_uint4(p[0], p[1], p[2], p[3]);
    }
  }
}

// ---- group absmax int8 -------------------------------------------------------
// One wavefront per (16-row block, 128-column tile).  Lane l = r + 16*c reads
// the 32 weights of row r that its bytes of the tile hold (columns
// 32*j + 8*c + e) and writes them with two 16-byte stores, one per half tile.

// Loads the 32 weights of lane (r, c) of tile kt, zeros past K or N.
template <int DT>
__device__ __forceinline__ void load_lane_tile(const void* W, int64_t n, bool row_ok, int64_t K, int64_t kt, int c,
                                               float (&w)[4][8], bool (&jok)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    jok[j] = row_ok && (kt * 128 + 32 * j < K);
    if (jok[j]) {
      load8<DT>(W, n * K + kt * 128 + 32 * j + 8 * c, w[j]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) w[j][e] = 0.0f;
    }
  }
}

template <int DT, int G>
__global__ __launch_bounds__(256) void quantize_w8_kernel(const void* __restrict__ W, int64_t N, int64_t K,
                                                          int64_t NBLK, int64_t KT, int8_t* __restrict__ q_codes,
                                                          uint16_t* __restrict__ s_out, uint8_t* __restrict__ qpacked) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (item >= NBLK * KT) return;  // whole wave exits together
  const int64_t nb = item / KT, kt = item % KT;
  const int r = lane & 15, c = lane >> 4;
  const int64_t n = nb * 16 + r;
  const bool row_ok = n < N;
  const int64_t Gtot = K / G;

  float w[4][8];
  bool jok[4];
  load_lane_tile<DT>(W, n, row_ok, K, kt, c, w, jok);

  GroupParams gp[4];
  if constexpr (G == 128) {
    float lo = w[0][0], hi = w[0][0];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) { lo = fminf(lo, w[j][e]); hi = fmaxf(hi, w[j][e]); }
    const GroupParams p = group_params_w8(wave_min4(lo), wave_max4(hi));
#pragma unroll
    for (int j = 0; j < 4; ++j) gp[j] = p;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float lo = w[j][0], hi = w[j][0];
#pragma unroll
      for (int e = 1; e < 8; ++e) { lo = fminf(lo, w[j][e]); hi = fmaxf(hi, w[j][e]); }
      gp[j] = group_params_w8(wave_min4(lo), wave_max4(hi));
    }
  }

  uint32_t words[4][2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t b[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) b[e] = jok[j] ? encode_w8(w[j][e], gp[j]) : 0u;
    words[j][0] = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
    words[j][1] = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
    if (q_codes && jok[j])
      *reinterpret_cast<uint2*>(q_codes + n * K + kt * 128 + 32 * j + 8 * c) = make_uint2(words[j][0], words[j][1]);
  }
  if (qpacked) {
    uint8_t* t = qpacked + tile8_offset_bytes(nb, kt, KT) + 16 * lane;
    *reinterpret_cast<u4*>(t) = u4{words[0][0], words[0][1], words[1][0], words[1][1]};
    *reinterpret_cast<u4*>(t + 1024) = u4{words[2][0], words[2][1], words[3][0], words[3][1]};
  }
  if (row_ok) {
    if constexpr (G == 128) {
      if (c == 0) s_out[n * Gtot + kt] = gp[0].s_bits;
    } else {
      const int64_t gi = kt * 4 + c;  // lane c writes group c of this tile
      if (gi < Gtot) s_out[n * Gtot + gi] = c == 0 ? gp[0].s_bits : c == 1 ? gp[1].s_bits : c == 2 ? gp[2].s_bits : gp[3].s_bits;
    }
  }
}

// int8 codes [N][K] -> 2048-byte tiles.
__global__ __launch_bounds__(256) void pack_w8_kernel(const int8_t* __restrict__ q_codes, int64_t N, int64_t K,
                                                      int64_t NBLK, int64_t KT, uint8_t* __restrict__ qpacked) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (item >= NBLK * KT) return;
  const int64_t nb = item / KT, kt = item % KT;
  const int r = lane & 15, c = lane >> 4;
  const int64_t n = nb * 16 + r;
  uint2 v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t k0 = kt * 128 + 32 * j + 8 * c;
    v[j] = (n < N && kt * 128 + 32 * j < K) ? *reinterpret_cast<const uint2*>(q_codes + n * K + k0) : make_uint2(0, 0);
  }
  uint8_t* t = qpacked + tile8_offset_bytes(nb, kt, KT) + 16 * lane;
  *reinterpret_cast<u4*>(t) = u4{v[0].x, v[0].y, v[1].x, v[1].y};
  *reinterpret_cast<u4*>(t + 1024) = u4{v[2].x, v[2].y, v[3].x, v[3].y};
}

// 2048-byte tiles + scales -> What[N][K] = s * q (exact in fp32).
template <int OUT, int G>
__global__ __launch_bounds__(256) void dequant_w8_kernel(const uint8_t* __restrict__ qpacked,
                                                         const uint16_t* __restrict__ s_in, int64_t N, int64_t K,
                                                         int64_t NBLK, int64_t KT, void* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (item >= NBLK * KT) return;
  const int64_t nb = item / KT, kt = item % KT;
  const int r = lane & 15, c = lane >> 4;
  const int64_t n = nb * 16 + r;
  if (n >= N) return;
  const int64_t Gtot = K / G;
  const uint8_t* t = qpacked + tile8_offset_bytes(nb, kt, KT) + 16 * lane;
  const u4 h0 = *reinterpret_cast<const u4*>(t), h1 = *reinterpret_cast<const u4*>(t + 1024);
  const uint32_t wd[4][2] = {{h0[0], h0[1]}, {h0[2], h0[3]}, {h1[0], h1[1]}, {h1[2], h1[3]}};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t k0 = kt * 128 + 32 * j + 8 * c;
    if (k0 >= K) continue;
    const float s = f16_bits_to_f32(s_in[n * Gtot + k0 / G]);
    float d[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int q = (int)(int8_t)(uint8_t)(wd[j][e >> 2] >> (8 * (e & 3)));
      d[e] = s * (float)q;  // exact: 11-bit significand times |q| <= 127
    }
    if constexpr (OUT == 0) {
      float4* o = reinterpret_cast<float4*>(static_cast<float*>(out) + n * K + k0);
      o[0] = make_float4(d[0], d[1], d[2], d[3]);
      o[1] = make_float4(d[4], d[5], d[6], d[7]);
    } else {
      uint32_t p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t a = OUT == 2 ? f32_to_f16_bits(d[2 * i]) : f32_to_bf16_bits(d[2 * i]);
        uint32_t b = OUT == 2 ? f32_to_f16_bits(d[2 * i + 1]) : f32_to_bf16_bits(d[2 * i + 1]);
        p[i] = a | (b << 16);
      }
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + n * K + k0) = make_uint4(p[0], p[1], p[2], p[3]);
    }
  }
}

// ---- MXFP4 --------------------------------------------------------------------

// E8M0 scale byte of a block whose max |v| is amax: the shared exponent
// floor(log2 amax) - 2 (the exponent field of amax minus 129 for normal amax),
// clamped at -127; 0 for an all-zero or fp32-subnormal maximum.
__device__ __forceinline__ uint32_t mx_scale_byte(float amax) {
  const int E = (int)((__builtin_bit_cast(uint32_t, amax) >> 23) & 0xffu);
  return (uint32_t)max(E - 2, 0);
}

// E2M1 code of v / 2^(e8 - 127): nearest of {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to
// the even mantissa bit, saturating at 6, sign in bit 3 (kept for negative
// values that round to zero).  The scaled magnitude m is below 8; on the
// grids 0.5 (m < 2), 1 (m < 4) and 2 (m >= 4) an integer's parity is the
// mantissa bit, so rint on each grid rounds ties to even.
__device__ __forceinline__ uint32_t mx_encode(float v, uint32_t e8) {
  const float inv = __builtin_bit_cast(float, (254u - e8) << 23);  // 2^(127 - e8), exact
  const float m = fabsf(v) * inv;
  uint32_t code;
  if (m < 2.0f) code = (uint32_t)rintf(2.0f * m);           // 0 .. 4
  else if (m < 4.0f) code = (uint32_t)rintf(m) + 2u;        // 4 .. 6
  else code = min((uint32_t)rintf(0.5f * m) + 4u, 7u);      // 6, 7 (saturating)
  return code | (v < 0.0f ? 8u : 0u);
}

// E2M1 magnitude of code bits 0..2 (exact in fp32).
__device__ __forceinline__ float mx_magnitude(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, f = c & 1u;
  return e == 0 ? 0.5f * (float)f : __builtin_bit_cast(float, (e + 126u) << 23) * (1.0f + 0.5f * (float)f);
}

template <int DT>
__global__ __launch_bounds__(256) void quantize_mxfp4_kernel(const void* __restrict__ W, int64_t N, int64_t K,
                                                             int64_t NBLK, int64_t KT, uint8_t* __restrict__ q_codes,
                                                             uint8_t* __restrict__ e8_out, uint8_t* __restrict__ qpacked) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (item >= NBLK * KT) return;  // whole wave exits together
  const int64_t nb = item / KT, kt = item % KT;
  const int r = lane & 15, c = lane >> 4;
  const int64_t n = nb * 16 + r;
  const bool row_ok = n < N;
  const int64_t Gtot = K / 32;

  float w[4][8];
  bool jok[4];
  load_lane_tile<DT>(W, n, row_ok, K, kt, c, w, jok);
  uint32_t words[4], e8[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(w[j][e]));
    amax = wave_max4(amax);
    e8[j] = amax > 0.0f ? mx_scale_byte(amax) : 0u;
    uint32_t word = 0;
    uint32_t b[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      b[e] = jok[j] ? mx_encode(w[j][e], e8[j]) : 0u;
      word |= b[e] << (4 * e);
    }
    words[j] = word;
    if (q_codes && jok[j])
      *reinterpret_cast<uint2*>(q_codes + n * K + kt * 128 + 32 * j + 8 * c) =
          make_uint2(b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24), b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24));
  }
  if (qpacked)
    *reinterpret_cast<u4*>(qpacked + tile_offset_bytes(nb, kt, KT) + 16 * lane) = u4{words[0], words[1], words[2], words[3]};
  if (row_ok) {
    const int64_t gi = kt * 4 + c;  // lane c writes block c of this tile
    if (gi < Gtot) e8_out[n * Gtot + gi] = (uint8_t)(c == 0 ? e8[0] : c == 1 ? e8[1] : c == 2 ? e8[2] : e8[3]);
  }
}

// MXFP4 codes [N][K] (low 4 bits) -> tiles with natural nibble order.
__global__ __launch_bounds__(256) void pack_mxfp4_kernel(const uint8_t* __restrict__ q_codes, int64_t N, int64_t K,
                                                         int64_t NBLK, int64_t KT, uint8_t* __restrict__ qpacked) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (item >= NBLK * KT) return;
  const int64_t nb = item / KT, kt = item % KT;
  const int r = lane & 15, c = lane >> 4;
  const int64_t n = nb * 16 + r;
  uint32_t words[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t word = 0;
    if (n < N && kt * 128 + 32 * j < K) {
      const uint2 v = *reinterpret_cast<const uint2*>(q_codes + n * K + kt * 128 + 32 * j + 8 * c);
#pragma unroll
      for (int e = 0; e < 8; ++e) word |= (((e < 4 ? v.x : v.y) >> (8 * (e & 3))) & 15u) << (4 * e);
    }
    words[j] = word;
  }
  *reinterpret_cast<u4*>(qpacked + tile_offset_bytes(nb, kt, KT) + 16 * lane) = u4{words[0], words[1], words[2], words[3]};
}

// Tiles + E8M0 scales -> What[N][K] = E2M1(q) * 2^(e8 - 127) (exact in fp32).
template <int OUT>
__global__ __launch_bounds__(256) void dequant_mxfp4_kernel(const uint8_t* __restrict__ qpacked,
                                                            const uint8_t* __restrict__ e8_in, int64_t N, int64_t K,
                                                            int64_t NBLK, int64_t KT, void* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (item >= NBLK * KT) return;
  const int64_t nb = item / KT, kt = item % KT;
  const int r = lane & 15, c = lane >> 4;
  const int64_t n = nb * 16 + r;
  if (n >= N) return;
  const int64_t Gtot = K / 32;
  const u4 v = *reinterpret_cast<const u4*>(qpacked + tile_offset_bytes(nb, kt, KT) + 16 * lane);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t k0 = kt * 128 + 32 * j + 8 * c;
    if (k0 >= K) continue;
    const uint32_t e8 = e8_in[n * Gtot + k0 / 32];
    const float sc = __builtin_bit_cast(float, e8 == 0 ? 0x00400000u : e8 << 23);  // 2^(e8 - 127)
    // magnitudes (exact, >= 0) converted first, the sign then set as a bit: a
    // code of -0 must give -0 in every output format (the compiler may fuse
    // the product and the fp16 conversion into one fma with a +0 addend)
    float d[8];
    uint32_t neg[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t c = (v[j] >> (4 * e)) & 15u;
      d[e] = mx_magnitude(c) * sc;
      neg[e] = c >> 3;
    }
    if constexpr (OUT == 0) {
      uint32_t b[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) b[e] = __builtin_bit_cast(uint32_t, d[e]) | (neg[e] << 31);
      uint4* o = reinterpret_cast<uint4*>(static_cast<float*>(out) + n * K + k0);
      o[0] = make_uint4(b[0], b[1], b[2], b[3]);
      o[1] = make_uint4(b[4], b[5], b[6], b[7]);
    } else {
      uint32_t p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t a = OUT == 2 ? f32_to_f16_bits(d[2 * i]) : f32_to_bf16_bits(d[2 * i]);
        uint32_t b = OUT == 2 ? f32_to_f16_bits(d[2 * i + 1]) : f32_to_bf16_bits(d[2 * i + 1]);
        p[i] = (a | (neg[2 * i] << 15)) | ((b | (neg[2 * i + 1] << 15)) << 16);
      }
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + n * K + k0) = make_uint4(p[0], p[1], p[2], p[3]);
    }
  }
}

// ---- NVFP4 --------------------------------------------------------------------
// E2M1 codes (the MXFP4 tile layout), one E4M3 scale byte per block of 16
// along K, one fp32 scale per tensor.  The tensor scale comes from the largest
// |w| of the whole tensor: a zero fill, a reduction (one atomic max of the
// value's bits per wave: non-negative fp32 values order as their bits), then
// one thread turns that maximum into S in place; the quantizer reads S.
// Every choice of an E4M3 or E2M1 value is the nearest value of the exact
// quotient, decided by exact comparisons with the midpoints between
// neighbouring values in fp64 (both factors have few significant bits, so
// each product is exact), ties to the even code, saturating.

__global__ void nvfp4_zero_kernel(float* tensor_scale) { *tensor_scale = 0.0f; }

template <int DT>
__global__ __launch_bounds__(256) void nvfp4_amax_kernel(const void* __restrict__ W, int64_t n8,
                                                         float* __restrict__ tensor_scale) {
  float m = 0.0f;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    float w[8];
    load8<DT>(W, i * 8, w);
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(w[e]));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0)
    atomicMax(reinterpret_cast<unsigned*>(tensor_scale), __builtin_bit_cast(unsigned, m));
}

// S = fp32(fp64(amax / (6 * 448))), 1 for an all-zero tensor.
__global__ void nvfp4_tensor_scale_kernel(float* tensor_scale) {
  const float amax = *tensor_scale;
  *tensor_scale = amax > 0.0f ? (float)((double)amax / 2688.0) : 1.0f;
}

// E4M3 magnitude of code c = 0..126 (bias 7; exponent field 0 is m * 2^-9).
__device__ __forceinline__ double e4m3_value(int c) {
  const int e = c >> 3, f = c & 7;
  return e == 0 ? (double)f * 0x1p-9 : (double)(8 + f) * __builtin_bit_cast(double, (uint64_t)(e - 10 + 1023) << 52);
}
// E2M1 magnitude of code m = 0..7.
__device__ __forceinline__ double e2m1_value(int m) {
  const int e = m >> 1, f = m & 1;
  return e == 0 ? 0.5 * f : (double)(2 + f) * (double)(1 << e) * 0.25;
}

// The E4M3 code nearest to a / d (a, d >= 0; d > 0), ties to even, 126 (448)
// past the last midpoint.
__device__ __forceinline__ int e4m3_nearest(double a, double d) {
  int c = 0;
  for (int k = 0; k < 126; ++k) {
    const double rhs = 0.5 * (e4m3_value(k) + e4m3_value(k + 1)) * d;
    if (a > rhs || (a == rhs && ((k + 1) & 1) == 0)) c = k + 1;
    else break;
  }
  return c;
}
// The E2M1 magnitude code nearest to a / d, ties to even, 7 (6) past 5.
__device__ __forceinline__ uint32_t e2m1_nearest(double a, double d) {
  uint32_t c = 0;
#pragma unroll
  for (int k = 0; k < 7; ++k) {
    const double rhs = 0.5 * (e2m1_value(k) + e2m1_value(k + 1)) * d;
    if (a > rhs || (a == rhs && ((k + 1) & 1) == 0)) c = (uint32_t)(k + 1);
    else break;
  }
  return c;
}

// One wavefront per (16-row block, 128-column tile), the MXFP4 decomposition:
// lane (r, c) holds columns 32j + 8c .. +7 of row r, so the block of 16 at
// columns 32j + 16h is shared by lanes c = 2h and 2h + 1 (lane index xor 16).
template <int DT>
__global__ __launch_bounds__(256) void quantize_nvfp4_kernel(const void* __restrict__ W, int64_t N, int64_t K,
                                                             int64_t NBLK, int64_t KT,
                                                             const float* __restrict__ tensor_scale,
                                                             uint8_t* __restrict__ q_codes, uint8_t* __restrict__ s8_out,
                                                             uint8_t* __restrict__ qpacked) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (item >= NBLK * KT) return;  // whole wave exits together
  const int64_t nb = item / KT, kt = item % KT;
  const int r = lane & 15, c = lane >> 4;
  const int64_t n = nb * 16 + r;
  const bool row_ok = n < N;
  const int64_t Gtot = K / 16;
  const double S = (double)*tensor_scale;

  float w[4][8];
  bool jok[4];
  load_lane_tile<DT>(W, n, row_ok, K, kt, c, w, jok);
  uint32_t words[4], sb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(w[j][e]));
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    sb[j] = amax > 0.0f ? (uint32_t)e4m3_nearest((double)amax, 6.0 * S) : 0u;
    const double d = e4m3_value((int)sb[j]) * S;
    uint32_t word = 0;
    uint32_t b[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t mag = sb[j] == 0 ? 0u : e2m1_nearest(fabs((double)w[j][e]), d);
      b[e] = jok[j] ? (mag | (w[j][e] < 0.0f ? 8u : 0u)) : 0u;
      word |= b[e] << (4 * e);
    }
    words[j] = word;
    if (q_codes && jok[j])
      *reinterpret_cast<uint2*>(q_codes + n * K + kt * 128 + 32 * j + 8 * c) =
          make_uint2(b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24), b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24));
  }
  if (qpacked)
    *reinterpret_cast<u4*>(qpacked + tile_offset_bytes(nb, kt, KT) + 16 * lane) = u4{words[0], words[1], words[2], words[3]};
  if (row_ok && (c & 1) == 0) {  // lanes c = 0 and 2 write the blocks 2j and 2j + 1 of each step j
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t gi = kt * 8 + 2 * j + (c >> 1);
      if (gi < Gtot) s8_out[n * Gtot + gi] = (uint8_t)sb[j];
    }
  }
}

// Tiles + E4M3 scale bytes + tensor scale -> What[N][K] =
// fp32(E2M1(q) * E4M3(s8) * S): the first product is exact in fp32, the
// multiplication by S rounds once.
template <int OUT>
__global__ __launch_bounds__(256) void dequant_nvfp4_kernel(const uint8_t* __restrict__ qpacked,
                                                            const uint8_t* __restrict__ s8_in,
                                                            const float* __restrict__ tensor_scale, int64_t N, int64_t K,
                                                            int64_t NBLK, int64_t KT, void* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (item >= NBLK * KT) return;
  const int64_t nb = item / KT, kt = item % KT;
  const int r = lane & 15, c = lane >> 4;
  const int64_t n = nb * 16 + r;
  if (n >= N) return;
  const int64_t Gtot = K / 16;
  const float S = *tensor_scale;
  const u4 v = *reinterpret_cast<const u4*>(qpacked + tile_offset_bytes(nb, kt, KT) + 16 * lane);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t k0 = kt * 128 + 32 * j + 8 * c;
    if (k0 >= K) continue;
    const float sc = (float)e4m3_value(s8_in[n * Gtot + k0 / 16] & 127);  // exact
    // magnitudes first, the sign then set as a bit (a code of -0 gives -0)
    float d[8];
    uint32_t neg[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t cc = (v[j] >> (4 * e)) & 15u;
      d[e] = (mx_magnitude(cc) * sc) * S;
      neg[e] = cc >> 3;
    }
    if constexpr (OUT == 0) {
      uint32_t b[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) b[e] = __builtin_bit_cast(uint32_t, d[e]) | (neg[e] << 31);
      uint4* o = reinterpret_cast<uint4*>(static_cast<float*>(out) + n * K + k0);
      o[0] = make_uint4(b[0], b[1], b[2], b[3]);
      o[1] = make_uint4(b[4], b[5], b[6], b[7]);
    } else {
      uint32_t p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t a = OUT == 2 ? f32_to_f16_bits(d[2 * i]) : f32_to_bf16_bits(d[2 * i]);
        uint32_t b = OUT == 2 ? f32_to_f16_bits(d[2 * i + 1]) : f32_to_bf16_bits(d[2 * i + 1]);
        p[i] = (a | (neg[2 * i] << 15)) | ((b | (neg[2 * i + 1] << 15)) << 16);
      }
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + n * K + k0) = make_uint4(p[0], p[1], p[2], p[3]);
    }
  }
}

// ---- INT4 KV cache in blocks of 128 ------------------------------------------
// A 16-lane group owns a pair of blocks (2p, 2p + 1) of one token: lanes 0..7
// block 2p, lanes 8..15 block 2p + 1, each lane 16 consecutive values (two
// code words).  A block's min / max is a reduction over its 8 lanes; the
// pair's zero-points share one byte, composed with one shuffle inside the
// group.  Cache row of hd values: codes hd/2 bytes (block b at byte 64*b, word
// j = values 8j..8j+7 in the weight-tile nibble order), hd/128 fp16 scales,
// ceil(hd/256) zero-point bytes.

template <int DT>
__device__ __forceinline__ void load16(const void* X, int64_t idx, float (&v)[16]) {
  load8<DT>(X, idx, v);
  load8<DT>(X, idx + 8, v + 8);
}

template <int DT>
__global__ __launch_bounds__(256) void kv_quantize_kernel(const void* __restrict__ X, int64_t T, int64_t hd,
                                                          const int32_t* __restrict__ slot, int64_t S,
                                                          uint8_t* __restrict__ codes, uint16_t* __restrict__ s_out,
                                                          uint8_t* __restrict__ zp) {
  const int64_t gl = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nb = hd / 128, ppt = (nb + 1) / 2, zb = ppt;
  const int64_t pid = gl >> 4;
  const int half = (int)(gl >> 3) & 1, part = (int)gl & 7;
  const int64_t t = min(pid / ppt, T - 1);      // clamped: lanes past the end compute on real data, store nothing
  const int64_t b = min(2 * (pid % ppt) + half, nb - 1);
  const bool active = pid < T * ppt && 2 * (pid % ppt) + half < nb;
  float v[16];
  load16<DT>(X, t * hd + b * 128 + part * 16, v);
  float lo = v[0], hi = v[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) { lo = fminf(lo, v[i]); hi = fmaxf(hi, v[i]); }
#pragma unroll
  for (int m = 1; m < 8; m <<= 1) {
    lo = fminf(lo, __shfl_xor(lo, m));
    hi = fmaxf(hi, __shfl_xor(hi, m));
  }
  const GroupParams p = group_params(lo, hi);
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 16; ++i) w[i >> 3] |= encode(v[i], p) << (4 * nibble_pos(i & 7));
  const uint32_t z = (uint32_t)p.z;
  const uint32_t z_next = (uint32_t)__shfl_down((int)z, 8, 16);  // zero-point of block 2p + 1 (lanes 0..7)
  const int64_t row = slot ? (int64_t)slot[t] : t;
  if (!active || row < 0 || row >= S) return;
  *reinterpret_cast<uint2*>(codes + row * (hd / 2) + b * 64 + part * 8) = make_uint2(w[0], w[1]);
  if (part == 0) {
    s_out[row * nb + b] = p.s_bits;
    if (half == 0) zp[row * zb + b / 2] = (uint8_t)(z | ((b + 1 < nb ? z_next : 0u) << 4));
  }
}

// Cache rows slot[t] -> out[t][hd] = s * (q - z); rows outside [0, S) give 0.
template <int OUT>
__global__ __launch_bounds__(256) void kv_dequant_kernel(const uint8_t* __restrict__ codes,
                                                         const uint16_t* __restrict__ s_in,
                                                         const uint8_t* __restrict__ zp, int64_t T, int64_t hd,
                                                         const int32_t* __restrict__ slot, int64_t S,
                                                         void* __restrict__ out) {
  const int64_t gl = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nb = hd / 128, zb = (nb + 1) / 2;
  const int64_t bid = gl >> 3;
  if (bid >= T * nb) return;
  const int part = (int)gl & 7;
  const int64_t t = bid / nb, b = bid % nb;
  const int64_t row = slot ? (int64_t)slot[t] : t;
  const bool ok = row >= 0 && row < S;
  float d[16];
  if (ok) {
    const uint2 w = *reinterpret_cast<const uint2*>(codes + row * (hd / 2) + b * 64 + part * 8);
    const float sc = f16_bits_to_f32(s_in[row * nb + b]);
    const uint32_t zbyte = zp[row * zb + b / 2];
    const int z = (int)((b & 1) ? zbyte >> 4 : zbyte & 15u);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int q = (int)((((i < 8) ? w.x : w.y) >> (4 * nibble_pos(i & 7))) & 15u);
      d[i] = sc * (float)(q - z);  // exact
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) d[i] = 0.0f;
  }
  const int64_t o = t * hd + b * 128 + part * 16;
  if constexpr (OUT == 0) {
    float4* po = reinterpret_cast<float4*>(static_cast<float*>(out) + o);
#pragma unroll
    for (int i = 0; i < 4; ++i) po[i] = make_float4(d[4 * i], d[4 * i + 1], d[4 * i + 2], d[4 * i + 3]);
  } else {
    uint32_t pk[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t a = OUT == 2 ? f32_to_f16_bits(d[2 * i]) : f32_to_bf16_bits(d[2 * i]);
      const uint32_t c = OUT == 2 ? f32_to_f16_bits(d[2 * i + 1]) : f32_to_bf16_bits(d[2 * i + 1]);
      pk[i] = a | (c << 16);
    }
    uint4* po = reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + o);
    po[0] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    po[1] = make_uint4(pk[4], pk[5], pk[6], pk[7]);
  }
}

// ---- the activation side of the AWQ fold, and its channel statistic --------

// x'[m][k] = fp16(fl32(x[m][k] / alpha[k])); eight values per thread.
__global__ __launch_bounds__(256) void scale_activations_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                                const float* __restrict__ alpha,
                                                                uint16_t* __restrict__ out) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= M * K) return;
  const int64_t k = i % K;  // K is a multiple of 8: the eight values share a row
  const uint4 v = *reinterpret_cast<const uint4*>(x + i);
  const float4 a0 = *reinterpret_cast<const float4*>(alpha + k), a1 = *reinterpret_cast<const float4*>(alpha + k + 4);
  const float a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
  const uint32_t in[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float lo = f16_bits_to_f32((uint16_t)(in[p] & 0xffffu)) / a[2 * p];
    const float hi = f16_bits_to_f32((uint16_t)(in[p] >> 16)) / a[2 * p + 1];
    o[p] = (uint32_t)f32_to_f16_bits(lo) | ((uint32_t)f32_to_f16_bits(hi) << 16);
  }
  *reinterpret_cast<uint4*>(out + i) = make_uint4(o[0], o[1], o[2], o[3]);
}

// out[k] = (sum over m in row order of |x[m][k]|, in fp32) / M; one thread per
// channel, consecutive threads on consecutive channels.
__global__ __launch_bounds__(256) void channel_absmean_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                              float* __restrict__ out) {
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (k >= K) return;
  float acc = 0.0f;
  for (int64_t m = 0; m < M; ++m) acc = acc + fabsf(f16_bits_to_f32(x[m * K + k]));
  out[k] = acc / (float)M;
}

inline int64_t blocks_for(int64_t waves) { return (waves + kWavesPerBlock - 1) / kWavesPerBlock; }

}  // namespace

hipError_t launch_quantize(const void* W, int dtype, int64_t N, int64_t K, int group, int sym, const float* alpha,
                           uint8_t* q_codes, uint16_t* s, uint8_t* z_codes, uint32_t* qpacked, uint8_t* zpacked,
                           hipStream_t stream) {
  const int64_t NBLK = (N + 15) / 16, KT = (K + 127) / 128, ST = (KT + 1) / 2;
  dim3 grid((unsigned)blocks_for(NBLK * ST)), block(256);
#define WQ_Q(DT, G, S, A)                                                                                \
  quantize_kernel<DT, G, S, A><<<grid, block, 0, stream>>>(W, N, K, NBLK, KT, alpha, q_codes, s, z_codes, qpacked, \
                                                           zpacked)
#define WQ_QS(DT, G)                              \
  do {                                            \
    if (sym) {                                    \
      if (alpha) WQ_Q(DT, G, true, true);         \
      else WQ_Q(DT, G, true, false);              \
    } else {                                      \
      if (alpha) WQ_Q(DT, G, false, true);        \
      else WQ_Q(DT, G, false, false);             \
    }                                             \
  } while (0)
  if (group == 128) {
    if (dtype == 0) WQ_QS(0, 128); else if (dtype == 1) WQ_QS(1, 128); else WQ_QS(2, 128);
  } else {
    if (dtype == 0) WQ_QS(0, 32); else if (dtype == 1) WQ_QS(1, 32); else WQ_QS(2, 32);
  }
#undef WQ_QS
#undef WQ_Q
  return hipGetLastError();
}

hipError_t launch_pack(const uint8_t* q_codes, const uint8_t* z_codes, int64_t N, int64_t K, int group,
                       uint32_t* qpacked, uint8_t* zpacked, hipStream_t stream) {
  const int64_t NBLK = (N + 15) / 16, KT = (K + 127) / 128, ST = (KT + 1) / 2;
  dim3 grid((unsigned)blocks_for(NBLK * ST)), block(256);
  if (group == 128)
    pack_kernel<128><<<grid, block, 0, stream>>>(q_codes, z_codes, N, K, NBLK, KT, qpacked, zpacked);
  else
    pack_kernel<32><<<grid, block, 0, stream>>>(q_codes, z_codes, N, K, NBLK, KT, qpacked, zpacked);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint32_t* qpacked, const uint16_t* s, const uint8_t* zpacked, int64_t N, int64_t K,
                          int group, int out_dtype, void* out, hipStream_t stream) {
  const int64_t NBLK = (N + 15) / 16, KT = (K + 127) / 128;
  dim3 grid((unsigned)blocks_for(NBLK * KT)), block(256);
#define WQ_D(O, G) dequant_kernel<O, G><<<grid, block, 0, stream>>>(qpacked, s, zpacked, N, K, NBLK, KT, out)
  if (group == 128) {
    if (out_dtype == 0) WQ_D(0, 128); else if (out_dtype == 1) WQ_D(1, 128); else WQ_D(2, 128);
  } else {
    if (out_dtype == 0) WQ_D(0, 32); else if (out_dtype == 1) WQ_D(1, 32); else WQ_D(2, 32);
  }
#undef WQ_D
  return hipGetLastError();
}

hipError_t launch_quantize_w8(const void* W, int dtype, int64_t N, int64_t K, int group, int8_t* q_codes,
                              uint16_t* s, uint8_t* qpacked, hipStream_t stream) {
  const int64_t NBLK = (N + 15) / 16, KT = (K + 127) / 128;
  dim3 grid((unsigned)blocks_for(NBLK * KT)), block(256);
#define WQ_Q8(DT, G) quantize_w8_kernel<DT, G><<<grid, block, 0, stream>>>(W, N, K, NBLK, KT, q_codes, s, qpacked)
  if (group == 128) {
    if (dtype == 0) WQ_Q8(0, 128); else if (dtype == 1) WQ_Q8(1, 128); else WQ_Q8(2, 128);
  } else {
    if (dtype == 0) WQ_Q8(0, 32); else if (dtype == 1) WQ_Q8(1, 32); else WQ_Q8(2, 32);
  }
#undef WQ_Q8
  return hipGetLastError();
}

hipError_t launch_pack_w8(const int8_t* q_codes, int64_t N, int64_t K, uint8_t* qpacked, hipStream_t stream) {
  const int64_t NBLK = (N + 15) / 16, KT = (K + 127) / 128;
  pack_w8_kernel<<<dim3((unsigned)blocks_for(NBLK * KT)), dim3(256), 0, stream>>>(q_codes, N, K, NBLK, KT, qpacked);
  return hipGetLastError();
}

hipError_t launch_dequant_w8(const uint8_t* qpacked, const uint16_t* s, int64_t N, int64_t K, int group,
                             int out_dtype, void* out, hipStream_t stream) {
  const int64_t NBLK = (N + 15) / 16, KT = (K + 127) / 128;
  dim3 grid((unsigned)blocks_for(NBLK * KT)), block(256);
#define WQ_D8(O, G) dequant_w8_kernel<O, G><<<grid, block, 0, stream>>>(qpacked, s, N, K, NBLK, KT, out)
  if (group == 128) {
    if (out_dtype == 0) WQ_D8(0, 128); else if (out_dtype == 1) WQ_D8(1, 128); else WQ_D8(2, 128);
  } else {
    if (out_dtype == 0) WQ_D8(0, 32); else if (out_dtype == 1) WQ_D8(1, 32); else WQ_D8(2, 32);
  }
#undef WQ_D8
  return hipGetLastError();
}

hipError_t launch_kv_quantize(const void* X, int dtype, int64_t T, int64_t hd, const int32_t* slot, int64_t S,
                              uint8_t* codes, uint16_t* s, uint8_t* zp, hipStream_t stream) {
  const int64_t lanes = T * ((hd / 128 + 1) / 2) * 16;
  const dim3 grid((unsigned)((lanes + 255) / 256)), block(256);
  if (dtype == 0) kv_quantize_kernel<0><<<grid, block, 0, stream>>>(X, T, hd, slot, S, codes, s, zp);
  else if (dtype == 1) kv_quantize_kernel<1><<<grid, block, 0, stream>>>(X, T, hd, slot, S, codes, s, zp);
  else kv_quantize_kernel<2><<<grid, block, 0, stream>>>(X, T, hd, slot, S, codes, s, zp);
  return hipGetLastError();
}

hipError_t launch_kv_dequant(const uint8_t* codes, const uint16_t* s, const uint8_t* zp, int64_t T, int64_t hd,
                             const int32_t* slot, int64_t S, int out_dtype, void* out, hipStream_t stream) {
  const int64_t lanes = T * (hd / 128) * 8;
  const dim3 grid((unsigned)((lanes + 255) / 256)), block(256);
  if (out_dtype == 0) kv_dequant_kernel<0><<<grid, block, 0, stream>>>(codes, s, zp, T, hd, slot, S, out);
  else if (out_dtype == 1) kv_dequant_kernel<1><<<grid, block, 0, stream>>>(codes, s, zp, T, hd, slot, S, out);
  else kv_dequant_kernel<2><<<grid, block, 0, stream>>>(codes, s, zp, T, hd, slot, S, out);
  return hipGetLastError();
}

hipError_t launch_scale_activations(const uint16_t* x, int64_t M, int64_t K, const float* alpha, uint16_t* out,
                                    hipStream_t stream) {
  const int64_t threads = M * K / 8;
  scale_activations_kernel<<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream>>>(x, M, K, alpha, out);
  return hipGetLastError();
}

hipError_t launch_channel_absmean(const uint16_t* x, int64_t M, int64_t K, float* out, hipStream_t stream) {
  channel_absmean_kernel<<<dim3((unsigned)((K + 255) / 256)), dim3(256), 0, stream>>>(x, M, K, out);
  return hipGetLastError();
}

hipError_t launch_quantize_mxfp4(const void* W, int dtype, int64_t N, int64_t K, uint8_t* q_codes, uint8_t* e8,
                                 uint8_t* qpacked, hipStream_t stream) {
  const int64_t NBLK = (N + 15) / 16, KT = (K + 127) / 128;
  dim3 grid((unsigned)blocks_for(NBLK * KT)), block(256);
  if (dtype == 0) quantize_mxfp4_kernel<0><<<grid, block, 0, stream>>>(W, N, K, NBLK, KT, q_codes, e8, qpacked);
  else if (dtype == 1) quantize_mxfp4_kernel<1><<<grid, block, 0, stream>>>(W, N, K, NBLK, KT, q_codes, e8, qpacked);
  else quantize_mxfp4_kernel<2><<<grid, block, 0, stream>>>(W, N, K, NBLK, KT, q_codes, e8, qpacked);
  return hipGetLastError();
}

hipError_t launch_pack_mxfp4(const uint8_t* q_codes, int64_t N, int64_t K, uint8_t* qpacked, hipStream_t stream) {
  const int64_t NBLK = (N + 15) / 16, KT = (K + 127) / 128;
  pack_mxfp4_kernel<<<dim3((unsigned)blocks_for(NBLK * KT)), dim3(256), 0, stream>>>(q_codes, N, K, NBLK, KT, qpacked);
  return hipGetLastError();
}

hipError_t launch_quantize_nvfp4(const void* W, int dtype, int64_t N, int64_t K, float* tensor_scale, uint8_t* q_codes,
                                 uint8_t* s8, uint8_t* qpacked, hipStream_t stream) {
  const int64_t NBLK = (N + 15) / 16, KT = (K + 127) / 128;
  const int64_t n8 = N * K / 8;
  const unsigned rgrid = (unsigned)std::min<int64_t>((n8 + 255) / 256, 2048);
  nvfp4_zero_kernel<<<1, 1, 0, stream>>>(tensor_scale);
  if (dtype == 0) nvfp4_amax_kernel<0><<<rgrid, 256, 0, stream>>>(W, n8, tensor_scale);
  else if (dtype == 1) nvfp4_amax_kernel<1><<<rgrid, 256, 0, stream>>>(W, n8, tensor_scale);
  else nvfp4_amax_kernel<2><<<rgrid, 256, 0, stream>>>(W, n8, tensor_scale);
  nvfp4_tensor_scale_kernel<<<1, 1, 0, stream>>>(tensor_scale);
  dim3 grid((unsigned)blocks_for(NBLK * KT)), block(256);
  if (dtype == 0)
    quantize_nvfp4_kernel<0><<<grid, block, 0, stream>>>(W, N, K, NBLK, KT, tensor_scale, q_codes, s8, qpacked);
  else if (dtype == 1)
    quantize_nvfp4_kernel<1><<<grid, block, 0, stream>>>(W, N, K, NBLK, KT, tensor_scale, q_codes, s8, qpacked);
  else
    quantize_nvfp4_kernel<2><<<grid, block, 0, stream>>>(W, N, K, NBLK, KT, tensor_scale, q_codes, s8, qpacked);
  return hipGetLastError();
}

hipError_t launch_dequant_nvfp4(const uint8_t* qpacked, const uint8_t* s8, const float* tensor_scale, int64_t N,
                                int64_t K, int out_dtype, void* out, hipStream_t stream) {
  const int64_t NBLK = (N + 15) / 16, KT = (K + 127) / 128;
  dim3 grid((unsigned)blocks_for(NBLK * KT)), block(256);
  if (out_dtype == 0) dequant_nvfp4_kernel<0><<<grid, block, 0, stream>>>(qpacked, s8, tensor_scale, N, K, NBLK, KT, out);
  else if (out_dtype == 1)
    dequant_nvfp4_kernel<1><<<grid, block, 0, stream>>>(qpacked, s8, tensor_scale, N, K, NBLK, KT, out);
  else dequant_nvfp4_kernel<2><<<grid, block, 0, stream>>>(qpacked, s8, tensor_scale, N, K, NBLK, KT, out);
  return hipGetLastError();
}

hipError_t launch_dequant_mxfp4(const uint8_t* qpacked, const uint8_t* e8, int64_t N, int64_t K, int out_dtype,
                                void* out, hipStream_t stream) {
  const int64_t NBLK = (N + 15) / 16, KT = (K + 127) / 128;
  dim3 grid((unsigned)blocks_for(NBLK * KT)), block(256);
  if (out_dtype == 0) dequant_mxfp4_kernel<0><<<grid, block, 0, stream>>>(qpacked, e8, N, K, NBLK, KT, out);
  else if (out_dtype == 1) dequant_mxfp4_kernel<1><<<grid, block, 0, stream>>>(qpacked, e8, N, K, NBLK, KT, out);
  else dequant_mxfp4_kernel<2><<<grid, block, 0, stream>>>(qpacked, e8, N, K, NBLK, KT, out);
  return hipGetLastError();
}

}  // namespace wq
