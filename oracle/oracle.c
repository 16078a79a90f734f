/*
 * CPU oracle for the BitNet b1.58 BitLinear layer (W1.58A8).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or helper
 * with the HIP library; the two are written independently from the same
 * definitions, so that agreement between them means something.
 *
 * Style: plain scalar C, one obvious loop per definition, no SIMD, no
 * blocking, no fusion.  Built with -O2 -fno-fast-math -ffp-contract=off so
 * that every fp32 operation is a single IEEE-754 rounding in the default
 * round-to-nearest-even mode.  The loops over independent outputs (rows of
 * the contraction, tokens of the activation cast, rows of the unpack) carry
 * an OpenMP work-sharing pragma, so the CPU-baseline leg of the benchmark
 * can use every host core: each output is still produced by one thread in
 * one sequential loop, so no result depends on the thread count.
 *
 * Sources (page title, section):
 *  [AN]  anthology note-168 on arXiv 2402.17764 (dmarx.github.io),
 *        "What it does" and "The part that is a bet rather than a measurement".
 *  [YT]  BitNet b1.58 2B4T video transcript (yousumm.com), "Transcription".
 *  [BH]  "Bit Happens: How Tiny Weights Are Shaking It Off"
 *        (michaelmallari.bitbucket.io), "From High-Precision Bloat to Elegant
 *        Bit-Level Efficiency".
 *
 * Readings taken where the pages are silent, numbered R1 .. R17:
 *  R1  absmean scale = mean of |W| over the whole matrix (one scale per
 *      tensor), accumulated in fp64, divided by N*K in fp64, rounded once to
 *      fp32, then floored at 1e-5.
 *  R2  ternary code = clamp(rintf(w / gamma), -1, 1), fp32 IEEE division,
 *      round-half-to-even (so |w| == gamma/2 gives 0).
 *  R3  activation scale = per-token max |x|, floored at 1e-5;
 *      q = clamp(rintf(x * (127 / a)), -127, 127), the multiplier computed
 *      once per token by an fp32 IEEE division.
 *  R4  output y = (float)acc * c with c = (gamma * a) / 127 in fp32
 *      (multiply, then divide).
 *  R5  the 2-bit packed format "BL2-T64" defined at oracle_pack below.
 *  R15 the ~0.4 GB footprint of the 2B model read as five codes per byte:
 *      the base-3 format "BT5-T32" defined at oracle_pack5 below.
 *  R13 the sub-layer norm before the activation cast is RMSNorm with a
 *      per-channel gain (oracle_rmsnorm_quant_act).
 *  R14 the squared-ReLU feed-forward is gated: h = relu(gate)^2 * up
 *      (oracle_relu2_gate_quant_act).
 *  R17 blocks are pre-norm with an fp32 residual add before the next
 *      sub-layer norm (oracle_add_rmsnorm_quant_act).
 *
 * Parity pins: every function below is pinned by tests/test_oracle_pins.py
 * against closed forms, hand-derived fixtures (tests/golden/), library
 * routines or brute force.  The exact last bit of the absmean scale for a
 * random matrix depends on the fp64 summation order and is the one value
 * that is "parity unpinned" beyond a 1e-6 relative bound.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

/* ------------------------------------------------------------------------ */
/* Weight side: absmean scale and ternary codes.   [AN] "What it does";      */
/* [YT] the absmean quantizer chooses -1, 0 or +1 for every weight.          */
/* ------------------------------------------------------------------------ */

float oracle_absmean_scale(const float *W, int64_t N, int64_t K)
{
    double s = 0.0;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            s += fabs((double)W[n * K + k]);
    double mean = s / ((double)N * (double)K);
    float gamma = (float)mean;
    if (!(gamma >= 1e-5f)) gamma = 1e-5f;
    return gamma;
}

void oracle_ternarize(const float *W, int64_t N, int64_t K, float gamma, int8_t *T)
{
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            float r = rintf(W[n * K + k] / gamma);
            int8_t t = 0;
            if (r >= 1.0f) t = 1;
            else if (r <= -1.0f) t = -1;
            T[n * K + k] = t;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Packed format BL2-T64: four ternary codes per byte ([YT]: four codes are  */
/* bundled into one byte, moved to the compute unit and unpacked there).     */
/*                                                                           */
/* Field value = code + 1, so {-1, 0, +1} -> {0, 1, 2}; the value 3 is never */
/* written and a byte of four zero codes is 0x55.                            */
/*                                                                           */
/* The N x K matrix is cut into row tiles of 64 rows and K units of 64       */
/* codes (K is padded up to a multiple of 64 and N up to a multiple of 64    */
/* with zero codes).  Tile t, unit u is a 1024-byte block at byte            */
/* (t * KU + u) * 1024, KU = ceil(K / 64).  The block is 64 slots of 16      */
/* bytes; slot L holds four little-endian 32-bit words d = 0..3.  With       */
/* d = 2*s + h, word d of slot L holds row 64*t + 32*s + (L mod 32) and      */
/* codes k = 64*u + 32*h + 16*(L div 32) + c for c = 0..15, code c in byte   */
/* (c mod 4) at bit 2*(c div 4) of the word.                                 */
/* ------------------------------------------------------------------------ */

int64_t oracle_packed_bytes(int64_t N, int64_t K)
{
    int64_t tiles = (N + 63) / 64;
    int64_t units = (K + 63) / 64;
    return tiles * units * 1024;
}

/* Position of code (n, k): byte index into the packed buffer and the bit
 * shift of its 2-bit field inside that byte.                                */
static void bl2_position(int64_t n, int64_t k, int64_t K, int64_t *byte, int *shift)
{
    int64_t units = (K + 63) / 64;
    int64_t t = n / 64, r = n % 64;
    int64_t u = k / 64, kk = k % 64;
    int64_t s = r / 32, row_in_half = r % 32;
    int64_t h = kk / 32, g = (kk % 32) / 16, c = kk % 16;
    int64_t slot = row_in_half + 32 * g;
    int64_t word = 2 * s + h;
    *byte = (t * units + u) * 1024 + 16 * slot + 4 * word + (c % 4);
    *shift = (int)(2 * (c / 4));
}

void oracle_pack(const int8_t *T, int64_t N, int64_t K, uint8_t *P)
{
    int64_t bytes = oracle_packed_bytes(N, K);
    for (int64_t i = 0; i < bytes; ++i) P[i] = 0x55; /* every field = zero code */
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            int64_t b; int sh;
            bl2_position(n, k, K, &b, &sh);
            uint8_t field = (uint8_t)(T[n * K + k] + 1);
            P[b] = (uint8_t)((P[b] & ~(3u << sh)) | ((unsigned)field << sh));
        }
    }
}

/* Returns the number of fields holding the forbidden value 3 among the N*K
 * real positions, plus the number of padding fields that are not the zero
 * code; T receives the decoded codes (a forbidden field decodes as 0).      */
int64_t oracle_unpack(const uint8_t *P, int64_t N, int64_t K, int8_t *T)
{
    int64_t bad = 0;
    int64_t tiles = (N + 63) / 64, units = (K + 63) / 64;
#pragma omp parallel for schedule(static) reduction(+ : bad) if (N * K >= (1 << 20))
    for (int64_t n = 0; n < tiles * 64; ++n) {
        for (int64_t k = 0; k < units * 64; ++k) {
            int64_t b; int sh;
            bl2_position(n, k, K, &b, &sh);
            int field = (P[b] >> sh) & 3;
            if (n < N && k < K) {
                if (field == 3) { ++bad; field = 1; }
                T[n * K + k] = (int8_t)(field - 1);
            } else if (field != 1) {
                ++bad;
            }
        }
    }
    return bad;
}

/* ------------------------------------------------------------------------ */
/* Packed format BT5-T32: five ternary codes per byte.  [YT] "Transcription" */
/* puts the 2B model at about 0.4 GB; four codes per byte gives 0.52 GB for  */
/* its 2.08 G BitLinear weights, five per byte (1.6 bits) gives 0.42 GB, so  */
/* the figure is read as base-3 packing (reading R15).                       */
/*                                                                           */
/* Byte value: the five codes of a byte, digit i = 0..4 (0 most significant) */
/* with digit value code + 1, form b = sum_i (code_i + 1) * 3^(4-i), an      */
/* integer in [0, 242].  The stored byte is s = ceil(256 * b / 243), so that */
/* s / 256 is b / 243 rounded up; b comes back as floor(243 * s / 256).     */
/* Five zero codes give b = 121, s = 128.                                    */
/*                                                                           */
/* Layout: row tiles of 32 rows, K units of 160 codes (K padded to a        */
/* multiple of 160 and N to a multiple of 32 with zero codes), KU5 =         */
/* ceil(K / 160).  Tile t, unit u is a 1024-byte block at byte               */
/* (t * KU5 + u) * 1024, made of 64 slots of 16 bytes.  Byte p (0..15) of    */
/* slot L holds row 32*t + (L mod 32) and, as digit i, the code              */
/* k = 160*u + 32*i + 16*(L div 32) + p.                                     */
/* ------------------------------------------------------------------------ */

int64_t oracle_packed5_bytes(int64_t N, int64_t K)
{
    int64_t tiles = (N + 31) / 32;
    int64_t units = (K + 159) / 160;
    return tiles * units * 1024;
}

/* Byte of the packed buffer that holds row n, unit u, slot half g (= L div
 * 32) and byte p of the slot.                                               */
static int64_t bt5_byte(int64_t n, int64_t u, int64_t g, int64_t p, int64_t units)
{
    int64_t t = n / 32, slot = n % 32 + 32 * g;
    return (t * units + u) * 1024 + 16 * slot + p;
}

void oracle_pack5(const int8_t *T, int64_t N, int64_t K, uint8_t *P)
{
    int64_t units = (K + 159) / 160, rows = (N + 31) / 32 * 32;
    for (int64_t n = 0; n < rows; ++n) {
        for (int64_t u = 0; u < units; ++u) {
            for (int64_t g = 0; g < 2; ++g) {
                for (int64_t p = 0; p < 16; ++p) {
                    int64_t b = 0;
                    for (int64_t i = 0; i < 5; ++i) {
                        int64_t k = 160 * u + 32 * i + 16 * g + p;
                        int code = (n < N && k < K) ? T[n * K + k] : 0;
                        b = 3 * b + (code + 1);          /* base-3 digit, most significant first */
                    }
                    int64_t s = (256 * b + 242) / 243;   /* ceil(256 b / 243) */
                    P[bt5_byte(n, u, g, p, units)] = (uint8_t)s;
                }
            }
        }
    }
}

/* Returns the number of bytes that are not the image of any five codes
 * (s != ceil(256 b / 243) for b = floor(243 s / 256)), plus the number of
 * padding positions that do not hold the zero code; T receives the decoded
 * codes.                                                                    */
int64_t oracle_unpack5(const uint8_t *P, int64_t N, int64_t K, int8_t *T)
{
    int64_t bad = 0;
    int64_t units = (K + 159) / 160, rows = (N + 31) / 32 * 32;
    for (int64_t n = 0; n < rows; ++n) {
        for (int64_t u = 0; u < units; ++u) {
            for (int64_t g = 0; g < 2; ++g) {
                for (int64_t p = 0; p < 16; ++p) {
                    int64_t s = P[bt5_byte(n, u, g, p, units)];
                    int64_t b = (243 * s) / 256;
                    if ((256 * b + 242) / 243 != s) ++bad;
                    for (int64_t i = 4; i >= 0; --i) {   /* least significant digit first */
                        int code = (int)(b % 3) - 1;
                        b /= 3;
                        int64_t k = 160 * u + 32 * i + 16 * g + p;
                        if (n < N && k < K) T[n * K + k] = (int8_t)code;
                        else if (code != 0) ++bad;
                    }
                }
            }
        }
    }
    return bad;
}

/* acc[m * nrows + r] = sum_k T[rows[r], k] * Q[m, k] with the codes read
 * straight from a BT5-T32 buffer (one byte decoded per code visit).         */
void oracle_matmul_packed5_rows(const int8_t *Q, const uint8_t *P, int64_t M, int64_t N,
                                int64_t K, const int64_t *rows, int64_t nrows, int32_t *acc)
{
    (void)N;
    int64_t units = (K + 159) / 160;
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t n = rows[r];
        for (int64_t m = 0; m < M; ++m) {
            int32_t sum = 0;
            for (int64_t k = 0; k < K; ++k) {
                int64_t u = k / 160, i = (k % 160) / 32, g = (k % 32) / 16, p = k % 16;
                int64_t b = (243 * (int64_t)P[bt5_byte(n, u, g, p, units)]) / 256;
                for (int64_t j = 4; j > i; --j) b /= 3;  /* drop the digits below digit i */
                int t = (int)(b % 3) - 1;
                sum += t * (int32_t)Q[m * K + k];
            }
            acc[m * nrows + r] = sum;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Activation side: per-token absmax to int8 ([AN] "What it does":           */
/* activations at 8 bits; [YT]: values are squeezed into eight-bit numbers). */
/* ------------------------------------------------------------------------ */

void oracle_quant_act(const float *X, int64_t M, int64_t K,
                      int8_t *Q, float *absmax, int32_t *rowsum)
{
#pragma omp parallel for schedule(static) if (M > 1 && M * K >= (1 << 20))
    for (int64_t m = 0; m < M; ++m) {
        float a = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float v = fabsf(X[m * K + k]);
            if (v > a) a = v;
        }
        if (!(a >= 1e-5f)) a = 1e-5f;
        float s = 127.0f / a;
        int32_t sum = 0;
        for (int64_t k = 0; k < K; ++k) {
            float r = rintf(X[m * K + k] * s);
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            int8_t q = (int8_t)r;
            Q[m * K + k] = q;
            sum += q;
        }
        absmax[m] = a;
        if (rowsum) rowsum[m] = sum;
    }
}

/* ------------------------------------------------------------------------ */
/* Sub-layer norm before the activation cast ([YT] "Transcription": BitNet   */
/* adds a sub-layer norm for stability; the pages give no formula).          */
/* Reading R13: RMSNorm with a per-channel gain g (all ones when absent):    */
/*   inv = (float)(1 / sqrt(sum_k x_k^2 / K + eps)), fp64 throughout, one     */
/*         rounding to fp32 at the end;                                      */
/*   xn_k = (x_k * inv) * g_k, two fp32 roundings in that order;             */
/* then the absmax int8 cast of xn (R3).  Xn (nullable) receives xn.         */
/* ------------------------------------------------------------------------ */

void oracle_rmsnorm_quant_act(const float *X, int64_t M, int64_t K, const float *g, float eps,
                              float *Xn, float *inv_out, int8_t *Q, float *absmax,
                              int32_t *rowsum)
{
    float *row = (float *)malloc((size_t)K * sizeof(float));
    for (int64_t m = 0; m < M; ++m) {
        double s2 = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double v = (double)X[m * K + k];
            s2 += v * v;
        }
        float inv = (float)(1.0 / sqrt(s2 / (double)K + (double)eps));
        for (int64_t k = 0; k < K; ++k) {
            float v = X[m * K + k] * inv;
            row[k] = v * (g ? g[k] : 1.0f);
            if (Xn) Xn[m * K + k] = row[k];
        }
        if (inv_out) inv_out[m] = inv;
        oracle_quant_act(row, 1, K, Q + m * K, absmax + m, rowsum ? rowsum + m : NULL);
    }
    free(row);
}

/* ------------------------------------------------------------------------ */
/* Gated squared-ReLU feed-forward activation before the down projection's  */
/* int8 cast ([YT] "Transcription": BitNet swaps its activation function for */
/* a squared ReLU; the pages give no formula).  Reading R14: the FFN hidden  */
/* value is h = relu(g)^2 * u from the gate and up projections' outputs,     */
/* evaluated in fp32 as r = max(g, 0); h = (r * r) * u (two roundings in     */
/* that order); then the absmax int8 cast of h (R3).  H (nullable) gets h.   */
/* Residual add before the sub-layer norm (reading R17: pre-norm blocks,
 * x_next = x + sublayer(norm(x)), with the addition in fp32): S = X + R,
 * then oracle_rmsnorm_quant_act on S.                                       */
void oracle_add_rmsnorm_quant_act(const float *X, const float *R, int64_t M, int64_t K,
                                  const float *g, float eps, float *S, float *Xn, float *inv_out,
                                  int8_t *Q, float *absmax, int32_t *rowsum)
{
    for (int64_t i = 0; i < M * K; ++i) S[i] = X[i] + R[i];
    oracle_rmsnorm_quant_act(S, M, K, g, eps, Xn, inv_out, Q, absmax, rowsum);
}

/* ------------------------------------------------------------------------ */

void oracle_relu2_gate_quant_act(const float *G, const float *U, int64_t M, int64_t N, float *H,
                                 int8_t *Q, float *absmax, int32_t *rowsum)
{
    float *row = (float *)malloc((size_t)N * sizeof(float));
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            float g = G[m * N + n];
            float r = g > 0.0f ? g : 0.0f;
            float sq = r * r;
            row[n] = sq * U[m * N + n];
            if (H) H[m * N + n] = row[n];
        }
        oracle_quant_act(row, 1, N, Q + m * N, absmax + m, rowsum ? rowsum + m : NULL);
    }
    free(row);
}

/* ------------------------------------------------------------------------ */
/* Contraction ([AN] "The part that is a bet...": with ternary weights the   */
/* product needs only integer additions).  acc[m][n] = sum_k T[n][k]Q[m][k]. */
/* ------------------------------------------------------------------------ */

void oracle_matmul(const int8_t *Q, const int8_t *T, int64_t M, int64_t N, int64_t K,
                   int32_t *acc)
{
#pragma omp parallel for collapse(2) schedule(static) if (M * N * K >= (1 << 20))
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int32_t s = 0;
            for (int64_t k = 0; k < K; ++k)
                s += (int32_t)T[n * K + k] * (int32_t)Q[m * K + k];
            acc[m * N + n] = s;
        }
}

/* The same result written as the pages phrase it: additions of the          */
/* activations where the weight is +1, subtractions where it is -1, nothing  */
/* where it is 0.  No multiplication is used.                                */
void oracle_matmul_addsub(const int8_t *Q, const int8_t *T, int64_t M, int64_t N, int64_t K,
                          int32_t *acc)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int32_t plus = 0, minus = 0;
            for (int64_t k = 0; k < K; ++k) {
                int8_t t = T[n * K + k];
                if (t == 1) plus += Q[m * K + k];
                else if (t == -1) minus += Q[m * K + k];
            }
            acc[m * N + n] = plus - minus;
        }
}

/* Contraction straight from the packed buffer for a chosen list of output
 * rows (used for sampled checks at full model sizes).  acc is M x nrows.    */
void oracle_matmul_packed_rows(const int8_t *Q, const uint8_t *P, int64_t M, int64_t N,
                               int64_t K, const int64_t *rows, int64_t nrows, int32_t *acc)
{
    (void)N;
#pragma omp parallel for schedule(static) if (nrows * M * K >= (1 << 20))
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t n = rows[i];
        for (int64_t m = 0; m < M; ++m) {
            int32_t s = 0;
            for (int64_t k = 0; k < K; ++k) {
                int64_t b; int sh;
                bl2_position(n, k, K, &b, &sh);
                int t = ((P[b] >> sh) & 3) - 1;
                s += t * (int32_t)Q[m * K + k];
            }
            acc[m * nrows + i] = s;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Rescale back to real values (BitLinear replaces nn.Linear, [AN] "What it  */
/* does", so the layer returns real numbers).                                */
/* ------------------------------------------------------------------------ */

void oracle_epilogue(const int32_t *acc, int64_t M, int64_t N, float gamma,
                     const float *absmax, float *Y)
{
    for (int64_t m = 0; m < M; ++m) {
        float c = (gamma * absmax[m]) / 127.0f;
        for (int64_t n = 0; n < N; ++n)
            Y[m * N + n] = (float)acc[m * N + n] * c;
    }
}

/* Tolerance reference: the same rescale carried out in fp64.                */
void oracle_epilogue_f64(const int32_t *acc, int64_t M, int64_t N, float gamma,
                         const float *absmax, double *Y)
{
    for (int64_t m = 0; m < M; ++m) {
        double c = ((double)gamma * (double)absmax[m]) / 127.0;
        for (int64_t n = 0; n < N; ++n)
            Y[m * N + n] = (double)acc[m * N + n] * c;
    }
}

/* ------------------------------------------------------------------------ */
/* Whole layer from fp32 activations and packed weights: unpack, quantize    */
/* the activations, contract, rescale.  Q/T/acc are caller scratch           */
/* (M*K, N*K, M*N).  Returns the number of bad packed fields.                */
/* ------------------------------------------------------------------------ */
int64_t oracle_forward_packed(const float *X, int64_t M, int64_t K, const uint8_t *P,
                              float gamma, int64_t N, float *Y,
                              int8_t *Q, float *absmax, int32_t *rowsum,
                              int8_t *T, int32_t *acc)
{
    int64_t bad = oracle_unpack(P, N, K, T);
    oracle_quant_act(X, M, K, Q, absmax, rowsum);
    oracle_matmul(Q, T, M, N, K, acc);
    oracle_epilogue(acc, M, N, gamma, absmax, Y);
    return bad;
}

/* Threads the OpenMP loops above use (the CPU-baseline leg reports it). */
int oracle_threads(void) { return omp_get_max_threads(); }
