/*
 * CPU oracle for the BitLinear W1.58A8 layer -- TEST INFRASTRUCTURE ONLY.
 * Declarations for oracle.c; see that file for the definitions, the page
 * citations and the readings taken where the pages are silent.
 * All buffers are host memory owned by the caller, row-major.
 */
#ifndef BITLINEAR_ORACLE_H
#define BITLINEAR_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

float   oracle_absmean_scale(const float *W, int64_t N, int64_t K);
void    oracle_ternarize(const float *W, int64_t N, int64_t K, float gamma, int8_t *T);
int64_t oracle_packed_bytes(int64_t N, int64_t K);
void    oracle_pack(const int8_t *T, int64_t N, int64_t K, uint8_t *P);
int64_t oracle_unpack(const uint8_t *P, int64_t N, int64_t K, int8_t *T);
int64_t oracle_packed5_bytes(int64_t N, int64_t K);
void    oracle_pack5(const int8_t *T, int64_t N, int64_t K, uint8_t *P);
int64_t oracle_unpack5(const uint8_t *P, int64_t N, int64_t K, int8_t *T);
void    oracle_matmul_packed5_rows(const int8_t *Q, const uint8_t *P, int64_t M, int64_t N,
                                   int64_t K, const int64_t *rows, int64_t nrows,
                                   int32_t *acc);
void    oracle_quant_act(const float *X, int64_t M, int64_t K,
                         int8_t *Q, float *absmax, int32_t *rowsum);
void    oracle_rmsnorm_quant_act(const float *X, int64_t M, int64_t K, const float *g,
                                 float eps, float *Xn, float *inv_out, int8_t *Q,
                                 float *absmax, int32_t *rowsum);
void    oracle_add_rmsnorm_quant_act(const float *X, const float *R, int64_t M, int64_t K,
                                     const float *g, float eps, float *S, float *Xn, float *inv_out,
                                     int8_t *Q, float *absmax, int32_t *rowsum);
void    oracle_relu2_gate_quant_act(const float *G, const float *U, int64_t M, int64_t N,
                                    float *H, int8_t *Q, float *absmax, int32_t *rowsum);
void    oracle_matmul(const int8_t *Q, const int8_t *T, int64_t M, int64_t N, int64_t K,
                      int32_t *acc);
void    oracle_matmul_addsub(const int8_t *Q, const int8_t *T, int64_t M, int64_t N,
                             int64_t K, int32_t *acc);
void    oracle_matmul_packed_rows(const int8_t *Q, const uint8_t *P, int64_t M, int64_t N,
                                  int64_t K, const int64_t *rows, int64_t nrows,
                                  int32_t *acc);
void    oracle_epilogue(const int32_t *acc, int64_t M, int64_t N, float gamma,
                        const float *absmax, float *Y);
void    oracle_epilogue_f64(const int32_t *acc, int64_t M, int64_t N, float gamma,
                            const float *absmax, double *Y);
int     oracle_threads(void);
int64_t oracle_forward_packed(const float *X, int64_t M, int64_t K, const uint8_t *P,
                              float gamma, int64_t N, float *Y,
                              int8_t *Q, float *absmax, int32_t *rowsum,
                              int8_t *T, int32_t *acc);

#ifdef __cplusplus
}
#endif
#endif
