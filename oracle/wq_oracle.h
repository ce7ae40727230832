/*
 * wq_oracle.h -- declarations of the CPU oracle (test infrastructure only).
 * The product library never includes this header.  See wq_oracle.c for the
 * definitions, the pages each function follows and the readings it takes.
 */
#ifndef WQ_ORACLE_H
#define WQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F16 = 2 };
enum { ORC_OK = 0, ORC_EINVAL = -1, ORC_ERANGE = -6 };
enum { ORC_ASYM = 0, ORC_SYM = 1 };  /* quantization scheme */

void orc_set_threads(int n);
int orc_get_threads(void);

float orc_f16_to_f32(uint16_t h);
uint16_t orc_f32_to_f16(float f);
float orc_bf16_to_f32(uint16_t b);
uint16_t orc_f32_to_bf16(float f);
void orc_f32_to_f16_array(const float* a, int64_t n, uint16_t* out);
void orc_f32_to_bf16_array(const float* a, int64_t n, uint16_t* out);

int orc_quantize_groups(const void* W, int dtype, int64_t N, int64_t K, int g,
                        uint8_t* q, uint16_t* s, uint8_t* z);
/* As orc_quantize_groups, with the scheme ORC_ASYM or ORC_SYM (symmetric 4-bit,
 * codes q + 8 with zero-point 8). */
int orc_quantize_groups_ex(const void* W, int dtype, int64_t N, int64_t K, int g, int scheme,
                           uint8_t* q, uint16_t* s, uint8_t* z);
/* AWQ fold: each weight multiplied by alpha[k] (fp32) before quantizing. */
int orc_quantize_groups_scaled(const void* W, int dtype, int64_t N, int64_t K, int g, int scheme,
                               const float* alpha, uint8_t* q, uint16_t* s, uint8_t* z);
int orc_dequant(const uint8_t* q, const uint16_t* s, const uint8_t* z,
                int64_t N, int64_t K, int g, int out_dtype, void* out);
/* x' = fp16(x / alpha[k]); mean |x| per channel (fp32, row order). */
int orc_scale_activations(const uint16_t* x_f16, int64_t M, int64_t K, const float* alpha, uint16_t* out);
int orc_channel_absmean(const uint16_t* x_f16, int64_t M, int64_t K, float* out);

int orc_pack_canonical(const uint8_t* q, int64_t N, int64_t K, uint8_t* out);
int64_t orc_device_bytes(int64_t N, int64_t K);
int orc_pack_device(const uint8_t* q, int64_t N, int64_t K, uint8_t* out);
int orc_unpack_device(const uint8_t* packed, int64_t N, int64_t K, uint8_t* q);
int orc_pack_zeros(const uint8_t* z, int64_t N, int64_t G, uint8_t* out);

int orc_gemm_f64(int64_t M, int64_t N, int64_t K, const uint16_t* x_f16, const float* w_hat, double* y);
int orc_gemm_rows_f64(int64_t M, int64_t N, int64_t K, int g, const uint16_t* x_f16,
                      const uint8_t* q, const uint16_t* s, const uint8_t* z,
                      int64_t n0, int64_t nrows, double* y_rows);

/* Group absmax int8: s = fp16(max|w| / 127), q = clip(rne(w / s), -127, 127). */
int orc_quantize_w8(const void* W, int dtype, int64_t N, int64_t K, int g, int8_t* q, uint16_t* s);
int orc_dequant_w8(const int8_t* q, const uint16_t* s, int64_t N, int64_t K, int g, int out_dtype, void* out);
int64_t orc_device_bytes_w8(int64_t N, int64_t K);
int orc_pack_device_w8(const int8_t* q, int64_t N, int64_t K, uint8_t* out);
int orc_unpack_device_w8(const uint8_t* packed, int64_t N, int64_t K, int8_t* q);
int orc_gemm_rows_w8_f64(int64_t M, int64_t N, int64_t K, int g, const uint16_t* x_f16,
                         const int8_t* q, const uint16_t* s, int64_t n0, int64_t nrows, double* y_rows);

/* INT4 KV cache: blocks of 128 values of each token's vector, the group
 * quantizer per block, scattered to cache rows slot[t] (NULL: row t). */
int orc_kv_quantize(const void* X, int dtype, int64_t T, int64_t hd, const int32_t* slot, int64_t S,
                    uint8_t* codes, uint16_t* s, uint8_t* z);
int orc_kv_dequant(const uint8_t* codes, const uint16_t* s, const uint8_t* z, int64_t T, int64_t hd,
                   const int32_t* slot, int64_t S, int out_dtype, void* out);

/* MXFP4: E2M1 codes (sign in bit 3) and E8M0 scale bytes per block of 32. */
int orc_quantize_mxfp4(const void* W, int dtype, int64_t N, int64_t K, uint8_t* q, uint8_t* e8);
int orc_dequant_mxfp4(const uint8_t* q, const uint8_t* e8, int64_t N, int64_t K, int out_dtype, void* out);
int orc_pack_device_mxfp4(const uint8_t* q, int64_t N, int64_t K, uint8_t* out);
int orc_gemm_rows_mxfp4_f64(int64_t M, int64_t N, int64_t K, const uint16_t* x_f16, const uint8_t* q,
                            const uint8_t* e8, int64_t n0, int64_t nrows, double* y_rows);

/* NVFP4: E2M1 codes (sign in bit 3), E4M3 scale bytes per block of 16 and one
 * fp32 scale per tensor (device layout: orc_pack_device_mxfp4). */
int orc_quantize_nvfp4(const void* W, int dtype, int64_t N, int64_t K, uint8_t* q, uint8_t* s8,
                       float* tensor_scale);
int orc_dequant_nvfp4(const uint8_t* q, const uint8_t* s8, float tensor_scale, int64_t N, int64_t K,
                      int out_dtype, void* out);
int orc_gemm_rows_nvfp4_f64(int64_t M, int64_t N, int64_t K, const uint16_t* x_f16, const uint8_t* q,
                            const uint8_t* s8, float tensor_scale, int64_t n0, int64_t nrows, double* y_rows);

int orc_symmetric(const double* w, int64_t n, int bits, int32_t* q, double* s_out, double* w_hat);

double orc_bits_per_weight(int bits, int g, int scale_bits, int zero_bits);
double orc_storage_bytes(int64_t n, int bits, int g, int scale_bits, int zero_bits);

#ifdef __cplusplus
}
#endif

#endif
