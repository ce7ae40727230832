/*
 * wq_oracle.c -- plain, slow CPU oracle for group-wise asymmetric INT4 weight
 * quantization and the dequantize-and-multiply product y = x * What^T.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or
 * calls this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark load it.  It shares no code, header, table or constant with the
 * HIP path.
 *
 * Sources (web pages; cited by title and section):
 *   [Q]  "Quantization for LLM inference: FP8, INT4 (GPTQ, AWQ) and GGUF - the
 *        model's accounting zoom", sections "The minimum maths: scale and
 *        zero-point" (equations for s, z, the encoding and the decoding) and
 *        "Numerical example" (the 8-weight INT4 table and the storage count).
 *   [C]  "Quantization Methods Compared: INT8, GPTQ, AWQ, FP8, FP4 and KV-Cache
 *        Quantization", section "What quantisation does: scale, round, and the
 *        outlier that ruins a group" (symmetric absmax int8 rule, per-group
 *        scales, bits per weight).
 *   [T]  "Test-time quantization", section "The maths that matter" (symmetric
 *        b-bit scale M/(2^(b-1)-1) and the half-step error bound).
 *   [Q]  also section "KV cache quantization" (the cache stored as int4 in
 *        blocks of 128 values, half a byte per value plus the scale overhead)
 *        and section "AWQ" (a salient input channel's weights multiplied by a
 *        factor before quantizing, its activations divided by it).
 *   [C]  also section "The methods compared" (the activation-aware scaling of
 *        salient channels and its toy example in symmetric int4).
 *   [Q]  also section "Microscaling: NVFP4 and MXFP4" (4-bit floating-point
 *        elements with one 8-bit scale per small block of 16 or 32), with the
 *        format of the microscaling paper that section cites: E2M1 elements
 *        (sign, 2 exponent bits with bias 1, 1 mantissa bit), blocks of 32,
 *        an E8M0 power-of-two scale.
 *   [C]  also section "Hardware, formats and the roofline" (its key box:
 *        NVFP4 stores 4-bit values with one FP8 E4M3 scale per 16 values and
 *        one fp32 scale per tensor, 4.5 bits per value, 39.4 GB for 70B).
 *        The pages leave the choice of the two scales open; read here as
 *        S = fp32(amax / (6 * 448)) over the tensor, the block scale the E4M3
 *        value nearest to the block's max|w| / (6 S), and every rounding to
 *        E4M3 or E2M1 to the nearest value of the exact quotient, ties to
 *        even, saturating at the format's largest finite value.
 *
 * Where the pages leave a step open, the readings below are used (each is also
 * listed in the design notes):
 *   - rounding to an integer is round-half-to-even ("rne");
 *   - the scale is stored as IEEE fp16 (round to nearest even, subnormals kept)
 *     and the STORED scale is the one used to encode and to decode;
 *   - s, z and the codes are computed with single IEEE binary32 operations, in
 *     the order written, with no fused multiply-add;
 *   - the group range is widened to include zero (lo' = min(lo,0),
 *     hi' = max(hi,0)) so that the zero-point is a code in [0, 15];
 *   - a group whose stored scale is 0 stores s = 0, z = 0 and all codes 0;
 *   - a group whose range would give a non-finite fp16 scale is an error.
 *
 * The symmetric variant ([T] "The maths that matter": b-bit symmetric range,
 * s = M / (2^(b-1) - 1); [C] "What quantisation does": q = round(w / s)) at
 * b = 4 uses the same storage: s = fp16(fl32(max|w| / 7)), q = clip(rne(fl32(w
 * / s)), -7, 7), stored as the code q + 8 with zero-point 8, so that
 * s * (code - 8) decodes it; a group whose stored scale is 0 stores s = 0,
 * zero-point 8 and codes 8.
 *
 * Packed layouts:
 *   canonical: [N][K/2] bytes, byte b of a row holds k = 2b in its low nibble
 *              and k = 2b+1 in its high nibble (the page only fixes that eight
 *              4-bit codes take four bytes);
 *   device:    16-row x 128-column tiles, tile (nb, kt) at byte offset
 *              (nb * ceil(K/128) + kt) * 1024; inside a tile, lane
 *              l = r + 16*c (r = row in tile 0..15, c = 0..3) owns 16 bytes
 *              at offset 16*l, made of four little-endian 32-bit words j = 0..3;
 *              word j holds the eight columns kk = 32*j + 8*c + e (e = 0..7)
 *              of the tile, column e in nibble p(e) = 4*(e%2) + e/2.  Rows are
 *              padded to a multiple of 16 and columns to a multiple of 128 with
 *              code 0.  (Parity unpinned by the pages: the layout is a
 *              definition; the tests check it is a bijection.)
 *   zeros:     [N][ceil(G/2)] bytes, G = K/g groups per row, group j in the
 *              low nibble of byte j/2 when j is even, high nibble when odd.
 *
 * Group absmax int8 ([C] "What quantisation does": s = max|w| / 127,
 * q = round(w / s), w_hat = q * s, one scale per group of g weights), read the
 * same way: s = fp16(fl32(max|w| / 127)), q = clip(rne(fl32(w / s)), -127, 127)
 * with the stored scale s, no zero-point, and a group whose stored scale is 0
 * stores s = 0 and codes 0.  w_hat = s * q is exact in fp32 (an 11-bit
 * significand times a 7-bit integer).  Its device layout (a definition, parity
 * unpinned by the pages; the tests check it is a bijection):
 *   device8:   16-row x 128-column tiles of 2048 bytes, tile (nb, kt) at byte
 *              offset (nb * ceil(K/128) + kt) * 2048; inside a tile, half
 *              h = 0, 1 at 1024 * h; in it lane l = r + 16*c owns the 16 bytes
 *              at 16*l, whose byte 8*i + e (i = 0, 1; e = 0..7) holds column
 *              32*(2h + i) + 8*c + e of row r, as a two's-complement byte.
 *              Padding rows and columns hold code 0.
 */
#include "wq_oracle.h"

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int g_threads = 1;

void orc_set_threads(int n) { g_threads = n > 0 ? n : 1; }
int orc_get_threads(void) { return g_threads; }

/* ------------------------------------------------------------------------- */
/* Number formats                                                            */
/* ------------------------------------------------------------------------- */

static float bits_to_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f32_to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* IEEE fp16 -> fp32, exact.  Value = (-1)^s * 2^(e-15) * (1 + m/1024) for
 * normal numbers and 2^-24 * m for subnormals. */
float orc_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 31) {
        if (m) return bits_to_f32(0x7fc00000u | ((uint32_t)sign << 31));
        v = INFINITY;
    } else if (e == 0) {
        v = ldexp((double)m, -24);
    } else {
        v = ldexp(1024.0 + m, e - 25);
    }
    return (float)(sign ? -v : v);
}

/* fp32 -> IEEE fp16 with round-to-nearest-even, subnormals kept.  The value is
 * taken exactly in double, divided by the fp16 spacing of its binade (a power
 * of two, so exact), rounded half-to-even, and re-encoded. */
uint16_t orc_f32_to_f16(float f)
{
    uint16_t sign = (f32_to_bits(f) >> 16) & 0x8000u;
    if (isnan(f)) return (uint16_t)(sign | 0x7e00u);
    double a = fabs((double)f);
    if (a >= 65520.0) return (uint16_t)(sign | 0x7c00u); /* rounds past 65504 */
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: spacing 2^-24; n = 1024 encodes 2^-14 correctly */
        double n = nearbyint(a / ldexp(1.0, -24));
        return (uint16_t)(sign | (uint16_t)n);
    }
    int e;
    frexp(a, &e); /* a in [2^(e-1), 2^e) */
    double ulp = ldexp(1.0, e - 1 - 10);
    double n = nearbyint(a / ulp); /* in [1024, 2048] */
    uint32_t bits = ((uint32_t)(e - 1 + 15) << 10) + (uint32_t)(n - 1024.0);
    return (uint16_t)(sign | bits);
}

float orc_bf16_to_f32(uint16_t b) { return bits_to_f32((uint32_t)b << 16); }

/* fp32 -> bfloat16 with round-to-nearest-even (8 significant bits, fp32's
 * exponent range, subnormal spacing 2^-133). */
uint16_t orc_f32_to_bf16(float f)
{
    uint32_t u = f32_to_bits(f);
    uint16_t sign = (u >> 16) & 0x8000u;
    if (isnan(f)) return (uint16_t)(sign | 0x7fc0u);
    double a = fabs((double)f);
    if (isinf(f)) return (uint16_t)(sign | 0x7f80u);
    double n;
    uint32_t mag;
    if (a < ldexp(1.0, -126)) {
        n = nearbyint(a / ldexp(1.0, -133)); /* 0..128; 128 encodes 2^-126 */
        mag = (uint32_t)n;
    } else {
        int e;
        frexp(a, &e);
        double ulp = ldexp(1.0, e - 1 - 7);
        n = nearbyint(a / ulp); /* in [128, 256] */
        mag = ((uint32_t)(e - 1 + 127) << 7) + (uint32_t)(n - 128.0);
        if (mag >= 0x7f80u) mag = 0x7f80u; /* overflow to infinity */
    }
    return (uint16_t)(sign | mag);
}

void orc_f32_to_f16_array(const float* a, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_f16(a[i]);
}

void orc_f32_to_bf16_array(const float* a, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_bf16(a[i]);
}

/* ------------------------------------------------------------------------- */
/* Group-wise asymmetric INT4 quantizer  ([Q] "The minimum maths")           */
/* ------------------------------------------------------------------------- */

static float load_w(const void* W, int dtype, int64_t idx)
{
    if (dtype == ORC_F32) return ((const float*)W)[idx];
    if (dtype == ORC_BF16) return orc_bf16_to_f32(((const uint16_t*)W)[idx]);
    return orc_f16_to_f32(((const uint16_t*)W)[idx]);
}

/* One group of g weights -> one fp16 scale, one zero-point, g codes.
 *   s = (max - min) / (2^4 - 1)          range over the group, widened to 0
 *   z = round(-min / s)                  integer zero-point in [0, 15]
 *   q = clip(round(w / s + z), 0, 15)    the encoding
 * Returns 0, or ORC_ERANGE if the scale is not a finite fp16 number. */
static int quantize_one_group(const float* w, int g, uint8_t* q, uint16_t* s_out, uint8_t* z_out)
{
    float lo = w[0], hi = w[0];
    for (int i = 1; i < g; ++i) {
        if (w[i] < lo) lo = w[i];
        if (w[i] > hi) hi = w[i];
    }
    if (!isfinite(lo) || !isfinite(hi)) return ORC_ERANGE;
    if (lo > 0.0f) lo = 0.0f;
    if (hi < 0.0f) hi = 0.0f;

    float range = hi - lo;          /* one fp32 subtraction */
    float s32 = range / 15.0f;      /* one fp32 division    */
    uint16_t sh_bits = orc_f32_to_f16(s32);
    float sh = orc_f16_to_f32(sh_bits);
    if (!isfinite(sh)) return ORC_ERANGE;

    if (sh == 0.0f) { /* degenerate group: everything decodes to 0 */
        *s_out = 0;
        *z_out = 0;
        for (int i = 0; i < g; ++i) q[i] = 0;
        return 0;
    }
    *s_out = sh_bits;

    float zf = nearbyintf(-lo / sh);
    if (zf < 0.0f) zf = 0.0f;
    if (zf > 15.0f) zf = 15.0f;
    *z_out = (uint8_t)zf;

    for (int i = 0; i < g; ++i) {
        float t = w[i] / sh;        /* fp32 division */
        t = t + zf;                 /* fp32 addition, not fused */
        float r = nearbyintf(t);
        if (r < 0.0f) r = 0.0f;
        if (r > 15.0f) r = 15.0f;
        q[i] = (uint8_t)r;
    }
    return 0;
}

/* One group, symmetric 4-bit ([T] "The maths that matter", b = 4):
 *   s = M / (2^3 - 1),  M = max |w| over the group
 *   q = clip(round(w / s), -7, 7), kept as the code q + 8 (zero-point 8)
 * Returns 0, or ORC_ERANGE if the scale is not a finite fp16 number. */
static int quantize_one_group_sym(const float* w, int g, uint8_t* q, uint16_t* s_out, uint8_t* z_out)
{
    float m = 0.0f;
    for (int i = 0; i < g; ++i) {
        if (!isfinite(w[i])) return ORC_ERANGE;
        float a = fabsf(w[i]);
        if (a > m) m = a;
    }
    float s32 = m / 7.0f;           /* one fp32 division */
    uint16_t sh_bits = orc_f32_to_f16(s32);
    float sh = orc_f16_to_f32(sh_bits);
    if (!isfinite(sh)) return ORC_ERANGE;
    *z_out = 8;
    if (sh == 0.0f) { /* degenerate group: everything decodes to 0 */
        *s_out = 0;
        for (int i = 0; i < g; ++i) q[i] = 8;
        return 0;
    }
    *s_out = sh_bits;
    for (int i = 0; i < g; ++i) {
        float r = nearbyintf(w[i] / sh);  /* fp32 division, then rne */
        if (r < -7.0f) r = -7.0f;
        if (r > 7.0f) r = 7.0f;
        q[i] = (uint8_t)(r + 8.0f);
    }
    return 0;
}

int orc_quantize_groups(const void* W, int dtype, int64_t N, int64_t K, int g,
                        uint8_t* q, uint16_t* s, uint8_t* z)
{
    return orc_quantize_groups_ex(W, dtype, N, K, g, ORC_ASYM, q, s, z);
}

int orc_quantize_groups_ex(const void* W, int dtype, int64_t N, int64_t K, int g, int scheme,
                           uint8_t* q, uint16_t* s, uint8_t* z)
{
    return orc_quantize_groups_scaled(W, dtype, N, K, g, scheme, NULL, q, s, z);
}

/* As orc_quantize_groups_ex, each weight first multiplied by its input
 * channel's factor alpha[k] (one fp32 multiplication; alpha == NULL: no
 * scaling) -- the AWQ fold W' = W diag(alpha) ([Q] "AWQ"). */
int orc_quantize_groups_scaled(const void* W, int dtype, int64_t N, int64_t K, int g, int scheme,
                               const float* alpha, uint8_t* q, uint16_t* s, uint8_t* z)
{
    if (!W || !q || !s || !z || N <= 0 || K <= 0 || g <= 0 || K % g) return ORC_EINVAL;
    if (scheme != ORC_ASYM && scheme != ORC_SYM) return ORC_EINVAL;
    if (dtype != ORC_F32 && dtype != ORC_BF16 && dtype != ORC_F16) return ORC_EINVAL;
    int64_t G = K / g;
    int status = 0;
#pragma omp parallel for num_threads(g_threads) schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        float* buf = (float*)malloc(sizeof(float) * (size_t)g);
        for (int64_t j = 0; j < G; ++j) {
            for (int i = 0; i < g; ++i) {
                buf[i] = load_w(W, dtype, n * K + j * g + i);
                if (alpha) buf[i] = buf[i] * alpha[j * g + i];
            }
            int st = scheme == ORC_SYM
                         ? quantize_one_group_sym(buf, g, q + n * K + j * g, s + n * G + j, z + n * G + j)
                         : quantize_one_group(buf, g, q + n * K + j * g, s + n * G + j, z + n * G + j);
            if (st) {
#pragma omp critical
                status = st;
            }
        }
        free(buf);
    }
    return status;
}

/* Decoding  w_hat = s * (q - z).  With an fp16 scale and |q - z| <= 15 the
 * product has at most 15 significant bits, so it is exact in fp32. */
int orc_dequant(const uint8_t* q, const uint16_t* s, const uint8_t* z,
                int64_t N, int64_t K, int g, int out_dtype, void* out)
{
    if (!q || !s || !z || !out || N <= 0 || K <= 0 || g <= 0 || K % g) return ORC_EINVAL;
    int64_t G = K / g;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int64_t j = k / g;
            float sc = orc_f16_to_f32(s[n * G + j]);
            float d = (float)((int)q[n * K + k] - (int)z[n * G + j]);
            float v = sc * d;
            if (out_dtype == ORC_F32) ((float*)out)[n * K + k] = v;
            else if (out_dtype == ORC_F16) ((uint16_t*)out)[n * K + k] = orc_f32_to_f16(v);
            else if (out_dtype == ORC_BF16) ((uint16_t*)out)[n * K + k] = orc_f32_to_bf16(v);
            else return ORC_EINVAL;
        }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Packing  ([Q] "Numerical example": eight 4-bit codes take four bytes)      */
/* ------------------------------------------------------------------------- */

int orc_pack_canonical(const uint8_t* q, int64_t N, int64_t K, uint8_t* out)
{
    if (!q || !out || N <= 0 || K <= 0 || K % 2) return ORC_EINVAL;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < K / 2; ++b)
            out[n * (K / 2) + b] = (uint8_t)((q[n * K + 2 * b] & 15) | ((q[n * K + 2 * b + 1] & 15) << 4));
    return 0;
}

int64_t orc_device_bytes(int64_t N, int64_t K)
{
    int64_t Np = (N + 15) / 16 * 16, Kp = (K + 127) / 128 * 128;
    return Np * Kp / 2;
}

/* Byte offset and nibble of element (n, k) in the device layout. */
static void device_pos(int64_t n, int64_t k, int64_t K, int64_t* byte, int* high)
{
    int64_t KT = (K + 127) / 128;
    int64_t nb = n / 16, r = n % 16, kt = k / 128, kk = k % 128;
    int64_t j = kk / 32, c = (kk % 32) / 8, e = kk % 8;
    int64_t lane = r + 16 * c;
    int p = (int)(4 * (e % 2) + e / 2);
    *byte = (nb * KT + kt) * 1024 + lane * 16 + j * 4 + p / 2;
    *high = p % 2;
}

int orc_pack_device(const uint8_t* q, int64_t N, int64_t K, uint8_t* out)
{
    if (!q || !out || N <= 0 || K <= 0) return ORC_EINVAL;
    memset(out, 0, (size_t)orc_device_bytes(N, K));
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int64_t byte;
            int high;
            device_pos(n, k, K, &byte, &high);
            uint8_t v = q[n * K + k] & 15;
            out[byte] = (uint8_t)(high ? (out[byte] & 0x0f) | (v << 4) : (out[byte] & 0xf0) | v);
        }
    return 0;
}

int orc_unpack_device(const uint8_t* packed, int64_t N, int64_t K, uint8_t* q)
{
    if (!packed || !q || N <= 0 || K <= 0) return ORC_EINVAL;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int64_t byte;
            int high;
            device_pos(n, k, K, &byte, &high);
            q[n * K + k] = high ? (packed[byte] >> 4) : (packed[byte] & 15);
        }
    return 0;
}

int orc_pack_zeros(const uint8_t* z, int64_t N, int64_t G, uint8_t* out)
{
    if (!z || !out || N <= 0 || G <= 0) return ORC_EINVAL;
    int64_t GB = (G + 1) / 2;
    memset(out, 0, (size_t)(N * GB));
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < G; ++j) {
            uint8_t v = z[n * G + j] & 15;
            uint8_t* b = out + n * GB + j / 2;
            *b = (uint8_t)((j % 2) ? (*b & 0x0f) | (v << 4) : (*b & 0xf0) | v);
        }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* The product y = x * What^T in fp64, summed in k order                     */
/* ------------------------------------------------------------------------- */

/* The activations as fp64 (exact: every fp16 value is a double), converted once
 * per call so the products below need no conversion per multiply. */
static double* x_to_f64(const uint16_t* x_f16, int64_t n)
{
    double* xd = (double*)malloc(sizeof(double) * (size_t)n);
    if (xd)
        for (int64_t i = 0; i < n; ++i) xd[i] = (double)orc_f16_to_f32(x_f16[i]);
    return xd;
}

int orc_gemm_f64(int64_t M, int64_t N, int64_t K, const uint16_t* x_f16, const float* w_hat, double* y)
{
    if (!x_f16 || !w_hat || !y || M <= 0 || N <= 0 || K <= 0) return ORC_EINVAL;
    double* xd = x_to_f64(x_f16, M * K);
    if (!xd) return ORC_EINVAL;
#pragma omp parallel for num_threads(g_threads) schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += xd[m * K + k] * (double)w_hat[n * K + k];
            y[m * N + n] = acc;
        }
    free(xd);
    return 0;
}

/* Rows [n0, n0 + nrows) of the same product, quantized weights given as codes,
 * scales and zero-points: the oracle's dequantization followed by the fp64
 * product, one row at a time (any range of rows, up to all of them, for the
 * full-size checks). */
int orc_gemm_rows_f64(int64_t M, int64_t N, int64_t K, int g, const uint16_t* x_f16,
                      const uint8_t* q, const uint16_t* s, const uint8_t* z,
                      int64_t n0, int64_t nrows, double* y_rows /* [M][nrows] */)
{
    if (!x_f16 || !q || !s || !z || !y_rows || M <= 0 || N <= 0 || K <= 0 || g <= 0 || K % g) return ORC_EINVAL;
    if (n0 < 0 || nrows <= 0 || n0 + nrows > N) return ORC_EINVAL;
    int64_t G = K / g;
    double* xd = x_to_f64(x_f16, M * K);
    if (!xd) return ORC_EINVAL;
#pragma omp parallel for num_threads(g_threads) schedule(static)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t n = n0 + i;
        float* wr = (float*)malloc(sizeof(float) * (size_t)K);
        orc_dequant(q + n * K, s + n * G, z + n * G, 1, K, g, ORC_F32, wr);
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += xd[m * K + k] * (double)wr[k];
            y_rows[m * nrows + i] = acc;
        }
        free(wr);
    }
    free(xd);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Group absmax int8  ([C] "What quantisation does")                         */
/* ------------------------------------------------------------------------- */

/* One group of g weights -> one fp16 scale and g int8 codes:
 *   s = max|w| / 127,  q = clip(round(w / s), -127, 127)
 * Returns 0, or ORC_ERANGE for a non-finite weight or fp16 scale. */
static int quantize_one_group_w8(const float* w, int g, int8_t* q, uint16_t* s_out)
{
    float m = 0.0f;
    for (int i = 0; i < g; ++i) {
        if (!isfinite(w[i])) return ORC_ERANGE;
        float a = fabsf(w[i]);
        if (a > m) m = a;
    }
    float s32 = m / 127.0f;         /* one fp32 division */
    uint16_t sh_bits = orc_f32_to_f16(s32);
    float sh = orc_f16_to_f32(sh_bits);
    if (!isfinite(sh)) return ORC_ERANGE;
    if (sh == 0.0f) { /* degenerate group: everything decodes to 0 */
        *s_out = 0;
        for (int i = 0; i < g; ++i) q[i] = 0;
        return 0;
    }
    *s_out = sh_bits;
    for (int i = 0; i < g; ++i) {
        float r = nearbyintf(w[i] / sh);  /* fp32 division, then rne */
        if (r < -127.0f) r = -127.0f;
        if (r > 127.0f) r = 127.0f;
        q[i] = (int8_t)r;
    }
    return 0;
}

int orc_quantize_w8(const void* W, int dtype, int64_t N, int64_t K, int g, int8_t* q, uint16_t* s)
{
    if (!W || !q || !s || N <= 0 || K <= 0 || g <= 0 || K % g) return ORC_EINVAL;
    if (dtype != ORC_F32 && dtype != ORC_BF16 && dtype != ORC_F16) return ORC_EINVAL;
    int64_t G = K / g;
    int status = 0;
#pragma omp parallel for num_threads(g_threads) schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        float* buf = (float*)malloc(sizeof(float) * (size_t)g);
        for (int64_t j = 0; j < G; ++j) {
            for (int i = 0; i < g; ++i) buf[i] = load_w(W, dtype, n * K + j * g + i);
            int st = quantize_one_group_w8(buf, g, q + n * K + j * g, s + n * G + j);
            if (st) {
#pragma omp critical
                status = st;
            }
        }
        free(buf);
    }
    return status;
}

/* Decoding  w_hat = s * q, exact in fp32; fp16 / bf16 are one rounding of it. */
int orc_dequant_w8(const int8_t* q, const uint16_t* s, int64_t N, int64_t K, int g, int out_dtype, void* out)
{
    if (!q || !s || !out || N <= 0 || K <= 0 || g <= 0 || K % g) return ORC_EINVAL;
    if (out_dtype != ORC_F32 && out_dtype != ORC_F16 && out_dtype != ORC_BF16) return ORC_EINVAL;
    int64_t G = K / g;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            float v = orc_f16_to_f32(s[n * G + k / g]) * (float)q[n * K + k];
            if (out_dtype == ORC_F32) ((float*)out)[n * K + k] = v;
            else if (out_dtype == ORC_F16) ((uint16_t*)out)[n * K + k] = orc_f32_to_f16(v);
            else ((uint16_t*)out)[n * K + k] = orc_f32_to_bf16(v);
        }
    return 0;
}

int64_t orc_device_bytes_w8(int64_t N, int64_t K)
{
    int64_t Np = (N + 15) / 16 * 16, Kp = (K + 127) / 128 * 128;
    return Np * Kp;
}

/* Byte offset of element (n, k) in the device8 layout. */
static int64_t device8_pos(int64_t n, int64_t k, int64_t K)
{
    int64_t KT = (K + 127) / 128;
    int64_t nb = n / 16, r = n % 16, kt = k / 128, kk = k % 128;
    int64_t j = kk / 32, c = (kk % 32) / 8, e = kk % 8;
    int64_t h = j / 2, i = j % 2, lane = r + 16 * c;
    return (nb * KT + kt) * 2048 + h * 1024 + lane * 16 + i * 8 + e;
}

int orc_pack_device_w8(const int8_t* q, int64_t N, int64_t K, uint8_t* out)
{
    if (!q || !out || N <= 0 || K <= 0) return ORC_EINVAL;
    memset(out, 0, (size_t)orc_device_bytes_w8(N, K));
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) out[device8_pos(n, k, K)] = (uint8_t)q[n * K + k];
    return 0;
}

int orc_unpack_device_w8(const uint8_t* packed, int64_t N, int64_t K, int8_t* q)
{
    if (!packed || !q || N <= 0 || K <= 0) return ORC_EINVAL;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) q[n * K + k] = (int8_t)packed[device8_pos(n, k, K)];
    return 0;
}

/* Rows [n0, n0 + nrows) of y = x * What^T with What = s * q (int8 codes),
 * dequantized by orc_dequant_w8 and multiplied in fp64 in k order. */
int orc_gemm_rows_w8_f64(int64_t M, int64_t N, int64_t K, int g, const uint16_t* x_f16,
                         const int8_t* q, const uint16_t* s, int64_t n0, int64_t nrows, double* y_rows)
{
    if (!x_f16 || !q || !s || !y_rows || M <= 0 || N <= 0 || K <= 0 || g <= 0 || K % g) return ORC_EINVAL;
    if (n0 < 0 || nrows <= 0 || n0 + nrows > N) return ORC_EINVAL;
    int64_t G = K / g;
    double* xd = x_to_f64(x_f16, M * K);
    if (!xd) return ORC_EINVAL;
#pragma omp parallel for num_threads(g_threads) schedule(static)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t n = n0 + i;
        float* wr = (float*)malloc(sizeof(float) * (size_t)K);
        orc_dequant_w8(q + n * K, s + n * G, 1, K, g, ORC_F32, wr);
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += xd[m * K + k] * (double)wr[k];
            y_rows[m * nrows + i] = acc;
        }
        free(wr);
    }
    free(xd);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* AWQ-style per-input-channel scaling  ([Q] "AWQ", [C] "The methods compared") */
/* ------------------------------------------------------------------------- */

/* The activation side of the fold: x'[m][k] = fp16(fl32(x[m][k] / alpha[k])),
 * so that x' W'^T = x W^T up to rounding. */
int orc_scale_activations(const uint16_t* x_f16, int64_t M, int64_t K, const float* alpha, uint16_t* out)
{
    if (!x_f16 || !alpha || !out || M <= 0 || K <= 0) return ORC_EINVAL;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) {
            float v = orc_f16_to_f32(x_f16[m * K + k]) / alpha[k];
            out[m * K + k] = orc_f32_to_f16(v);
        }
    return 0;
}

/* The statistic that finds salient channels: mean |x| of each input channel
 * over the M rows, summed in row order in fp32, then divided by M in fp32. */
int orc_channel_absmean(const uint16_t* x_f16, int64_t M, int64_t K, float* out)
{
    if (!x_f16 || !out || M <= 0 || K <= 0) return ORC_EINVAL;
    for (int64_t k = 0; k < K; ++k) {
        float acc = 0.0f;
        for (int64_t m = 0; m < M; ++m) acc = acc + fabsf(orc_f16_to_f32(x_f16[m * K + k]));
        out[k] = acc / (float)M;
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* MXFP4  ([Q] "Microscaling: NVFP4 and MXFP4")                              */
/* ------------------------------------------------------------------------- */

/* The eight E2M1 magnitudes, code m = 0..7 (exponent field m >> 1, mantissa
 * bit m & 1): exponent field 0 is subnormal, 0.5 * mantissa; otherwise
 * 2^(e - 1) * (1 + mantissa / 2). */
static double e2m1_magnitude(int m)
{
    int e = m >> 1, f = m & 1;
    return e == 0 ? 0.5 * f : ldexp(1.0 + 0.5 * f, e - 1);
}

/* Nearest E2M1 magnitude code to v >= 0 (ties to the code with an even
 * mantissa bit; anything past 6 gives 6, the largest: the saturating
 * conversion). */
static int e2m1_encode_magnitude(double v)
{
    int best = 0;
    double best_d = fabs(v - e2m1_magnitude(0));
    for (int m = 1; m < 8; ++m) {
        double d = fabs(v - e2m1_magnitude(m));
        if (d < best_d || (d == best_d && (m & 1) == 0 && (best & 1) == 1)) {
            best = m;
            best_d = d;
        }
    }
    return best;
}

/* One block of 32 values -> E8M0 scale byte and 32 E2M1 codes (sign in bit 3).
 * The shared exponent is floor(log2(max|v|)) - 2 (2 = the largest E2M1
 * exponent, so the block maximum lands in [4, 8) before rounding), clamped to
 * the E8M0 range [-127, 127]; an all-zero block stores exponent -127 and codes
 * 0.  A value below zero keeps its sign bit even when it rounds to zero. */
static int quantize_block_mxfp4(const float* v, uint8_t* q, uint8_t* e8)
{
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) {
        if (!isfinite(v[i])) return ORC_ERANGE;
        if (fabs((double)v[i]) > amax) amax = fabs((double)v[i]);
    }
    int shared = -127;
    if (amax > 0.0) {
        int ex;
        frexp(amax, &ex);       /* amax = f * 2^ex, f in [0.5, 1) */
        shared = ex - 1 - 2;
        if (shared < -127) shared = -127;
        if (shared > 127) shared = 127;
    }
    *e8 = (uint8_t)(shared + 127);
    for (int i = 0; i < 32; ++i) {
        double x = ldexp((double)v[i], -shared);  /* exact */
        int m = e2m1_encode_magnitude(fabs(x));
        q[i] = (uint8_t)(((v[i] < 0.0f) ? 8 : 0) | m);
    }
    return 0;
}

int orc_quantize_mxfp4(const void* W, int dtype, int64_t N, int64_t K, uint8_t* q, uint8_t* e8)
{
    if (!W || !q || !e8 || N <= 0 || K <= 0 || K % 32) return ORC_EINVAL;
    if (dtype != ORC_F32 && dtype != ORC_BF16 && dtype != ORC_F16) return ORC_EINVAL;
    int64_t G = K / 32;
    int status = 0;
#pragma omp parallel for num_threads(g_threads) schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        float buf[32];
        for (int64_t j = 0; j < G; ++j) {
            for (int i = 0; i < 32; ++i) buf[i] = load_w(W, dtype, n * K + j * 32 + i);
            int st = quantize_block_mxfp4(buf, q + n * K + j * 32, e8 + n * G + j);
            if (st) {
#pragma omp critical
                status = st;
            }
        }
    }
    return status;
}

/* w_hat = E2M1(q) * 2^(e8 - 127), exact in fp32 (fp32 subnormals cover the
 * smallest block exponent); fp16 / bf16 outputs are one rounding of it. */
int orc_dequant_mxfp4(const uint8_t* q, const uint8_t* e8, int64_t N, int64_t K, int out_dtype, void* out)
{
    if (!q || !e8 || !out || N <= 0 || K <= 0 || K % 32) return ORC_EINVAL;
    if (out_dtype != ORC_F32 && out_dtype != ORC_F16 && out_dtype != ORC_BF16) return ORC_EINVAL;
    int64_t G = K / 32;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int c = q[n * K + k] & 15;
            double mag = e2m1_magnitude(c & 7);
            double v = ldexp((c & 8) ? -mag : mag, (int)e8[n * G + k / 32] - 127);
            float f = (float)v;
            if (out_dtype == ORC_F32) ((float*)out)[n * K + k] = f;
            else if (out_dtype == ORC_F16) ((uint16_t*)out)[n * K + k] = orc_f32_to_f16(f);
            else ((uint16_t*)out)[n * K + k] = orc_f32_to_bf16(f);
        }
    return 0;
}

/* Device layout of MXFP4 codes: the 1024-byte tiles of the INT4 layout
 * (16 rows x 128 columns, lane l = r + 16c owns 16 bytes, word j = columns
 * 32j + 8c + e), with column e in nibble e of its word (two neighbouring
 * columns per byte, the even one in the low nibble). */
int orc_pack_device_mxfp4(const uint8_t* q, int64_t N, int64_t K, uint8_t* out)
{
    if (!q || !out || N <= 0 || K <= 0) return ORC_EINVAL;
    int64_t KT = (K + 127) / 128;
    memset(out, 0, (size_t)orc_device_bytes(N, K));
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int64_t nb = n / 16, r = n % 16, kt = k / 128, kk = k % 128;
            int64_t j = kk / 32, c = (kk % 32) / 8, e = kk % 8;
            int64_t byte = (nb * KT + kt) * 1024 + (r + 16 * c) * 16 + j * 4 + e / 2;
            uint8_t v = q[n * K + k] & 15;
            out[byte] = (uint8_t)((e % 2) ? (out[byte] & 0x0f) | (v << 4) : (out[byte] & 0xf0) | v);
        }
    return 0;
}

/* Rows [n0, n0 + nrows) of y = x * What^T for MXFP4 weights, in fp64. */
int orc_gemm_rows_mxfp4_f64(int64_t M, int64_t N, int64_t K, const uint16_t* x_f16, const uint8_t* q,
                            const uint8_t* e8, int64_t n0, int64_t nrows, double* y_rows)
{
    if (!x_f16 || !q || !e8 || !y_rows || M <= 0 || N <= 0 || K <= 0 || K % 32) return ORC_EINVAL;
    if (n0 < 0 || nrows <= 0 || n0 + nrows > N) return ORC_EINVAL;
    int64_t G = K / 32;
    double* xd = x_to_f64(x_f16, M * K);
    if (!xd) return ORC_EINVAL;
#pragma omp parallel for num_threads(g_threads) schedule(static)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t n = n0 + i;
        float* wr = (float*)malloc(sizeof(float) * (size_t)K);
        orc_dequant_mxfp4(q + n * K, e8 + n * G, 1, K, ORC_F32, wr);
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += xd[m * K + k] * (double)wr[k];
            y_rows[m * nrows + i] = acc;
        }
        free(wr);
    }
    free(xd);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* NVFP4  ([C] "Hardware, formats and the roofline" key box: 4-bit values,    */
/* one E4M3 scale per 16 values and a per-tensor fp32 scale, 4.5 bits per    */
/* value; [Q] "Microscaling: NVFP4 and MXFP4")                               */
/* ------------------------------------------------------------------------- */

/* The E4M3 magnitude of code c = 0..126 (4 exponent bits with bias 7, 3
 * mantissa bits; exponent field 0 is subnormal, m * 2^-9; 0x7F would be NaN,
 * so 448 = code 126 is the largest finite value). */
static double e4m3_magnitude(int c)
{
    int e = c >> 3, f = c & 7;
    return e == 0 ? ldexp((double)f, -9) : ldexp(1.0 + f / 8.0, e - 7);
}

/* The code c in [0, ncodes) whose value val(c) * d is nearest to a >= 0, ties
 * to the even code, beyond the last midpoint the last code (saturation).
 * Values increase with c; each comparison a <> mid * d is exact in fp64 for
 * the operands used here (a: an fp32 value; mid: a midpoint of two format
 * values, at most five significant bits; d: at most 28 significant bits). */
static int nearest_scaled(double a, double d, double (*val)(int), int ncodes)
{
    int c = 0;
    for (int k = 0; k + 1 < ncodes; ++k) {
        double mid = 0.5 * (val(k) + val(k + 1));
        double rhs = mid * d;
        if (a > rhs || (a == rhs && ((k + 1) & 1) == 0)) c = k + 1;
        else break;
    }
    return c;
}

/* The per-tensor scale of a tensor whose largest |w| is amax:
 * S = fp32(fp64(amax / (6 * 448))) (6 and 448 are the largest E2M1 and E4M3
 * magnitudes, so the largest block scale lands on 448); S = 1 for an
 * all-zero tensor. */
static float nvfp4_tensor_scale(double amax)
{
    return amax > 0.0 ? (float)(amax / 2688.0) : 1.0f;
}

/* NVFP4 quantization of W[N][K] (K a multiple of 16): the per-tensor scale S
 * from the largest |w| of the whole tensor; per block of 16 along K the E4M3
 * scale byte s8 = the E4M3 value nearest to max|w| / (6 S) (ties to even,
 * saturating at 448); the E2M1 codes (sign in bit 3) nearest to
 * w / (E4M3(s8) * S) (ties to even, saturating at 6).  A block whose scale
 * byte is 0 stores codes 0 (a negative value keeps its sign bit, as in MXFP4).
 * A non-finite input is an error. */
int orc_quantize_nvfp4(const void* W, int dtype, int64_t N, int64_t K, uint8_t* q, uint8_t* s8,
                       float* tensor_scale)
{
    if (!W || !q || !s8 || !tensor_scale || N <= 0 || K <= 0 || K % 16) return ORC_EINVAL;
    if (dtype != ORC_F32 && dtype != ORC_BF16 && dtype != ORC_F16) return ORC_EINVAL;
    double amax = 0.0;
    for (int64_t i = 0; i < N * K; ++i) {
        float v = load_w(W, dtype, i);
        if (!isfinite(v)) return ORC_ERANGE;
        if (fabs((double)v) > amax) amax = fabs((double)v);
    }
    const float S = nvfp4_tensor_scale(amax);
    *tensor_scale = S;
    const int64_t G = K / 16;
#pragma omp parallel for num_threads(g_threads) schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t j = 0; j < G; ++j) {
            float v[16];
            double bmax = 0.0;
            for (int i = 0; i < 16; ++i) {
                v[i] = load_w(W, dtype, n * K + j * 16 + i);
                if (fabs((double)v[i]) > bmax) bmax = fabs((double)v[i]);
            }
            int sc = nearest_scaled(bmax, 6.0 * (double)S, e4m3_magnitude, 127);
            s8[n * G + j] = (uint8_t)sc;
            double d = e4m3_magnitude(sc) * (double)S;
            for (int i = 0; i < 16; ++i) {
                int m = sc == 0 ? 0 : nearest_scaled(fabs((double)v[i]), d, e2m1_magnitude, 8);
                q[n * K + j * 16 + i] = (uint8_t)(((v[i] < 0.0f) ? 8 : 0) | m);
            }
        }
    }
    return 0;
}

/* w_hat = fp32(E2M1(q) * E4M3(s8) * S): the product of the two format values
 * is exact, and one rounding to fp32 applies the per-tensor scale; fp16 /
 * bf16 outputs are one further rounding of that fp32 value. */
int orc_dequant_nvfp4(const uint8_t* q, const uint8_t* s8, float tensor_scale, int64_t N, int64_t K,
                      int out_dtype, void* out)
{
    if (!q || !s8 || !out || N <= 0 || K <= 0 || K % 16) return ORC_EINVAL;
    if (out_dtype != ORC_F32 && out_dtype != ORC_F16 && out_dtype != ORC_BF16) return ORC_EINVAL;
    int64_t G = K / 16;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int c = q[n * K + k] & 15;
            double mag = e2m1_magnitude(c & 7) * e4m3_magnitude(s8[n * G + k / 16] & 127);
            float f = (float)(((c & 8) ? -mag : mag) * (double)tensor_scale);
            if (out_dtype == ORC_F32) ((float*)out)[n * K + k] = f;
            else if (out_dtype == ORC_F16) ((uint16_t*)out)[n * K + k] = orc_f32_to_f16(f);
            else ((uint16_t*)out)[n * K + k] = orc_f32_to_bf16(f);
        }
    return 0;
}

/* Rows [n0, n0 + nrows) of y = x * What^T for NVFP4 weights, in fp64, with
 * the exact decoded weights E2M1(q) * E4M3(s8) * S (before any rounding). */
int orc_gemm_rows_nvfp4_f64(int64_t M, int64_t N, int64_t K, const uint16_t* x_f16, const uint8_t* q,
                            const uint8_t* s8, float tensor_scale, int64_t n0, int64_t nrows, double* y_rows)
{
    if (!x_f16 || !q || !s8 || !y_rows || M <= 0 || N <= 0 || K <= 0 || K % 16) return ORC_EINVAL;
    if (n0 < 0 || nrows <= 0 || n0 + nrows > N) return ORC_EINVAL;
    int64_t G = K / 16;
    double* xd = x_to_f64(x_f16, M * K);
    if (!xd) return ORC_EINVAL;
#pragma omp parallel for num_threads(g_threads) schedule(static)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t n = n0 + i;
        double* wr = (double*)malloc(sizeof(double) * (size_t)K);
        for (int64_t k = 0; k < K; ++k) {
            int c = q[n * K + k] & 15;
            double mag = e2m1_magnitude(c & 7) * e4m3_magnitude(s8[n * G + k / 16] & 127) * (double)tensor_scale;
            wr[k] = (c & 8) ? -mag : mag;
        }
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += xd[m * K + k] * wr[k];
            y_rows[m * nrows + i] = acc;
        }
        free(wr);
    }
    free(xd);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* INT4 KV cache in blocks of 128  ([Q] "KV cache quantization")             */
/* ------------------------------------------------------------------------- */

/* Each token's K (or V) vector of hd values (all heads, hd a multiple of 128)
 * is cut into hd/128 blocks of 128 consecutive values, and each block goes
 * through the same group quantizer as the weights (scale, zero-point, 4-bit
 * codes).  Token t of a call is written to cache row slot[t] (slot == NULL:
 * row t); tokens whose slot lies outside [0, S) are skipped.  Cache layout of
 * one row:
 *   codes  hd/2 bytes: block b at byte 64*b; its 16 little-endian 32-bit words
 *          j = 0..15 hold values 8j + e (e = 0..7), value e in nibble
 *          4*(e%2) + e/2 (the word format of the weight tiles);
 *   s      hd/128 fp16 scales;
 *   z      ceil(hd/256) bytes, block b's zero-point in the low nibble of byte
 *          b/2 when b is even, in the high nibble when b is odd. */
static int64_t kv_nibble_byte(int64_t v, int* high)
{
    int64_t b = v / 128, i = v % 128, j = i / 8, e = i % 8;
    int p = (int)(4 * (e % 2) + e / 2);
    *high = p % 2;
    return b * 64 + j * 4 + p / 2;
}

int orc_kv_quantize(const void* X, int dtype, int64_t T, int64_t hd, const int32_t* slot, int64_t S,
                    uint8_t* codes, uint16_t* s, uint8_t* z)
{
    if (!X || !codes || !s || !z || T <= 0 || hd <= 0 || hd % 128 || S <= 0) return ORC_EINVAL;
    if (dtype != ORC_F32 && dtype != ORC_BF16 && dtype != ORC_F16) return ORC_EINVAL;
    int64_t nb = hd / 128, zb = (nb + 1) / 2;
    float w[128];
    uint8_t q[128];
    for (int64_t t = 0; t < T; ++t) {
        int64_t row = slot ? (int64_t)slot[t] : t;
        if (row < 0 || row >= S) continue;
        uint8_t* crow = codes + row * (hd / 2);
        uint8_t* zrow = z + row * zb;
        if (nb % 2) zrow[zb - 1] &= 0x0f;  /* an odd block count leaves the last high nibble 0 */
        for (int64_t b = 0; b < nb; ++b) {
            for (int i = 0; i < 128; ++i) w[i] = load_w(X, dtype, t * hd + b * 128 + i);
            uint8_t zz;
            int st = quantize_one_group(w, 128, q, s + row * nb + b, &zz);
            if (st) return st;
            zrow[b / 2] = (uint8_t)((b % 2) ? (zrow[b / 2] & 0x0f) | (zz << 4) : (zrow[b / 2] & 0xf0) | zz);
            for (int i = 0; i < 128; ++i) {
                int high;
                int64_t byte = kv_nibble_byte(b * 128 + i, &high);
                crow[byte] = (uint8_t)(high ? (crow[byte] & 0x0f) | (q[i] << 4) : (crow[byte] & 0xf0) | q[i]);
            }
        }
    }
    return 0;
}

/* Rows slot[t] (slot == NULL: row t) of the cache decoded to x_hat[t][hd] =
 * s * (q - z) (fp32 exact; fp16 / bf16 one rounding); rows outside [0, S)
 * decode to zeros. */
int orc_kv_dequant(const uint8_t* codes, const uint16_t* s, const uint8_t* z, int64_t T, int64_t hd,
                   const int32_t* slot, int64_t S, int out_dtype, void* out)
{
    if (!codes || !s || !z || !out || T <= 0 || hd <= 0 || hd % 128 || S <= 0) return ORC_EINVAL;
    if (out_dtype != ORC_F32 && out_dtype != ORC_F16 && out_dtype != ORC_BF16) return ORC_EINVAL;
    int64_t nb = hd / 128, zb = (nb + 1) / 2;
    for (int64_t t = 0; t < T; ++t) {
        int64_t row = slot ? (int64_t)slot[t] : t;
        int ok = row >= 0 && row < S;
        for (int64_t v = 0; v < hd; ++v) {
            float val = 0.0f;
            if (ok) {
                int high;
                int64_t byte = kv_nibble_byte(v, &high);
                int q = high ? codes[row * (hd / 2) + byte] >> 4 : codes[row * (hd / 2) + byte] & 15;
                int64_t b = v / 128;
                uint8_t zbyte = z[row * zb + b / 2];
                int zz = (b % 2) ? zbyte >> 4 : zbyte & 15;
                val = orc_f16_to_f32(s[row * nb + b]) * (float)(q - zz);
            }
            if (out_dtype == ORC_F32) ((float*)out)[t * hd + v] = val;
            else if (out_dtype == ORC_F16) ((uint16_t*)out)[t * hd + v] = orc_f32_to_f16(val);
            else ((uint16_t*)out)[t * hd + v] = orc_f32_to_bf16(val);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Symmetric quantizers ([C] absmax int8; [T] symmetric b-bit), in fp64      */
/* ------------------------------------------------------------------------- */

/* Symmetric absmax: s = max|w| / (2^(b-1) - 1), q = round(w / s) clipped to
 * +-(2^(b-1) - 1), w_hat = q * s.  b = 8 gives the int8 rule s = max|w|/127;
 * b = 4 gives the +-7 INT4 variant. */
int orc_symmetric(const double* w, int64_t n, int bits, int32_t* q, double* s_out, double* w_hat)
{
    if (!w || !q || !s_out || n <= 0 || bits < 2 || bits > 16) return ORC_EINVAL;
    double amax = 0.0;
    for (int64_t i = 0; i < n; ++i) if (fabs(w[i]) > amax) amax = fabs(w[i]);
    int32_t qmax = (1 << (bits - 1)) - 1;
    double s = amax / (double)qmax;
    *s_out = s;
    for (int64_t i = 0; i < n; ++i) {
        double r = s > 0.0 ? nearbyint(w[i] / s) : 0.0;
        if (r > qmax) r = qmax;
        if (r < -qmax) r = -qmax;
        q[i] = (int32_t)r;
        if (w_hat) w_hat[i] = r * s;
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Storage accounting ([Q] "Numerical example"; [C] per-group scales)        */
/* ------------------------------------------------------------------------- */

/* Bits per weight of b-bit codes with one scale of scale_bits and one zero-point
 * of zero_bits per group of g weights. */
double orc_bits_per_weight(int bits, int g, int scale_bits, int zero_bits)
{
    return (double)bits + (double)(scale_bits + zero_bits) / (double)g;
}

/* Bytes needed to store n weights that way (groups rounded up). */
double orc_storage_bytes(int64_t n, int bits, int g, int scale_bits, int zero_bits)
{
    int64_t groups = (n + g - 1) / g;
    return ((double)n * bits + (double)groups * (scale_bits + zero_bits)) / 8.0;
}
