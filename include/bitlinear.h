/*
 * bitlinear.h -- C ABI of the MI355X (gfx950) BitLinear W1.58A8 library.
 *
 * The layer (anthology note-168 on arXiv 2402.17764, "What it does"):
 * BitLinear stands in for nn.Linear; its weights are ternary {-1, 0, +1},
 * chosen by an absmean quantizer, and its activations are 8-bit.  The
 * product of ternary weights with integer activations needs only integer
 * additions (same note, "The part that is a bet rather than a measurement").
 * For inference the weights are quantized once and stored packed, four
 * codes to a byte, then streamed to the compute units and unpacked there
 * next to the 8-bit multiply (BitNet b1.58 2B4T video transcript,
 * yousumm.com, "Transcription").
 *
 * Definitions implemented (readings of the pages; they print no formula):
 *   gamma  = max(1e-5, fp32(mean |W|))        mean over all N*K, fp64 sum
 *   T[n,k] = clamp(rint(W[n,k] / gamma), -1, 1)   fp32 IEEE divide, half-even
 *   a[m]   = max(1e-5, max_k |X[m,k]|)
 *   Q[m,k] = clamp(rint(X[m,k] * (127 / a[m])), -127, 127)
 *   acc[m,n] = sum_k T[n,k] * Q[m,k]           exact int32
 *   Y[m,n] = float(acc[m,n]) * ((gamma * a[m]) / 127)
 *
 * The hot path and where each step lives (every other call is an extension
 * built from the same kernels):
 *   bitlinear_quantize_weights  absmean scale + ternarize (once per weight)
 *   bitlinear_pack              four codes per byte, BL2-T64 (once per weight)
 *   bitlinear_quant_act         per-token absmax + int8 cast + row sums
 *   bitlinear_forward           quant_act + ternary x int8 contraction
 *                               (exact int32) + fp32 rescale, per call
 *   bitlinear_workspace_bytes, bitlinear_strerror, bitlinear_last_error,
 *   bitlinear_abi_version       helpers of those four
 * Extensions: bitlinear_matmul (the contraction on caller-quantized
 * activations), the cast variants (_rmsnorm, _add_rmsnorm, _relu2_gate),
 * multi-matrix and cast + multi-matrix launches, grouped plans, BT5-T32
 * (five codes per byte), bitlinear_forward_noalloc, and the calibration
 * probes of bitlinear_probe.h.
 * Two deliberate differences from a minimal contract: every call takes
 * `void *stream`, which is a hipStream_t (void * keeps HIP headers out of
 * this file), and bitlinear_quant_act takes a row stride ldq so that the
 * codes land directly in the padded rows the contraction reads.
 *
 * Conventions for every call
 *   - Matrices are row-major.  W and T are N x K (N = out features, K = in
 *     features); X and Q are M x K (M tokens); Y and acc are M x N.
 *   - Every buffer pointer is DEVICE memory allocated and owned by the
 *     caller.  The library never allocates, frees or synchronizes; every
 *     call only enqueues kernels on `stream` (a hipStream_t; NULL = the
 *     default stream) and returns.  Results are ready when the stream is.
 *   - Every device buffer must be 16-byte aligned (BITLINEAR_ERR_ALIGN).
 *   - Return value: BITLINEAR_OK (0) or a negative status.  On a
 *     validation error nothing is enqueued.  bitlinear_strerror() names a
 *     status; bitlinear_last_error() gives the calling thread's last
 *     detailed message (including the HIP error text on BITLINEAR_ERR_HIP).
 *   - Sizes: 1 <= M, N <= 2^24 and 1 <= K <= 131072, so |acc| <= 127*K
 *     < 2^24 is exact in int32 and converts to fp32 exactly.  Any M, N, K
 *     in range is accepted (no multiple-of-64 requirement); internally K
 *     is padded to a multiple of 64 with zero codes / zero activations.
 *   - NaN or infinite inputs give unspecified (but memory-safe) results.
 *   - Calls are reentrant; the library holds no mutable global state beyond
 *     the scratch array of bitlinear_forward_noalloc.  Two calls that share
 *     a workspace must not run concurrently.
 *
 * Packed weight format "BL2-T64" (the buffer bitlinear_pack writes and the
 * matmul calls read; bitlinear_packed_bytes(N, K) bytes):
 *   field = code + 1 in 2 bits, so {-1, 0, +1} -> {0, 1, 2}; 3 never occurs;
 *   0x55 is four zero codes.  Rows are grouped in tiles of 64 (t = n / 64),
 *   K in units of 64 codes (u = k / 64), KU = ceil(K / 64) units per row.
 *   Tile t, unit u is a 1024-byte block at (t * KU + u) * 1024 made of 64
 *   slots of 16 bytes; 32-bit little-endian word d = 2*s + h of slot L
 *   holds row 64*t + 32*s + (L % 32), codes k = 64*u + 32*h + 16*(L / 32)
 *   + c for c = 0..15, code c at bit 8*(c % 4) + 2*(c / 4).  Rows >= N and
 *   codes >= K are padding and hold zero codes.
 *   Why this order: one 16-byte load per lane gives a 64-row x 64-code
 *   block; (word >> 2j) & 0x03030303 yields four consecutive codes as
 *   bytes, ready for a 4-way int8 dot product, and the four planes of one
 *   word are exactly the 16-byte int8 operand of one lane of the gfx950
 *   32x32x32 int8 matrix instruction.
 *
 * Packed weight format "BT5-T32" (five codes per byte, 1.6 bits per weight;
 * bitlinear_pack5 writes it, the *5 calls read it; bitlinear_packed5_bytes
 * (N, K) bytes).  The pages quote about 0.4 GB for the 2B model (BitNet
 * b1.58 2B4T video transcript, yousumm.com, "Transcription"), which four
 * codes per byte (0.52 GB) cannot reach and five per byte (0.42 GB) does:
 *   the five codes of a byte, digit i = 0..4 (0 most significant), form
 *   b = sum_i (code_i + 1) * 3^(4-i) in [0, 242]; the byte stores
 *   s = ceil(256 b / 243) (five zero codes: 0x80).  Rows are grouped in
 *   tiles of 32 (t = n / 32), K in units of 160 codes (u = k / 160), KU5 =
 *   ceil(K / 160).  Tile t, unit u is a 1024-byte block at (t * KU5 + u) *
 *   1024 made of 64 slots of 16 bytes; byte p of slot L holds row 32 t +
 *   L % 32 and, as digit i, code k = 160 u + 32 i + 16 (L / 32) + p.  Rows
 *   >= N and codes >= K are padding and hold zero codes.
 *   Why: floor(s * 3^j / 256) is exactly the integer of the top j digits
 *   (243 < 256), so a packed byte decodes with one multiply and one byte
 *   select per digit plane, and a lane's 16-byte load is the B operand of
 *   the 32x32x32 int8 matrix instruction for each of the five planes.
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BITLINEAR_ABI_VERSION 2

enum bitlinear_status {
    BITLINEAR_OK = 0,
    BITLINEAR_ERR_NULL = -1,      /* a required pointer is NULL                 */
    BITLINEAR_ERR_SHAPE = -2,     /* a size is out of range or inconsistent     */
    BITLINEAR_ERR_ALIGN = -3,     /* a buffer or stride is not 16-byte aligned  */
    BITLINEAR_ERR_WORKSPACE = -4, /* workspace missing or smaller than needed   */
    BITLINEAR_ERR_HIP = -5,       /* the HIP runtime refused a launch           */
    BITLINEAR_ERR_ARG = -6        /* any other bad argument (op code, table)    */
};

/* Workspace kinds for bitlinear_workspace_bytes. */
enum bitlinear_ws_op {
    BITLINEAR_WS_QUANTIZE_WEIGHTS = 1,
    BITLINEAR_WS_MATMUL = 2,
    BITLINEAR_WS_FORWARD = 3,
    BITLINEAR_WS_MATMUL5 = 4,
    BITLINEAR_WS_FORWARD5 = 5
};

/* Packed weight formats (bitlinear_problem.format). */
enum bitlinear_format {
    BITLINEAR_FORMAT_BL2 = 0, /* BL2-T64, four codes per byte */
    BITLINEAR_FORMAT_BT5 = 1  /* BT5-T32, five codes per byte */
};

/* Library ABI version (BITLINEAR_ABI_VERSION of the build). */
int bitlinear_abi_version(void);

/* Static text for a status code. */
const char *bitlinear_strerror(int status);

/* The calling thread's last detailed error message ("" if none). */
const char *bitlinear_last_error(void);

/* Bytes of the BL2-T64 buffer for an N x K matrix:
 * ceil(N/64) * ceil(K/64) * 1024 (= N*K/4 when 64 divides N and K).
 * Returns 0 for sizes out of range. */
size_t bitlinear_packed_bytes(int64_t N, int64_t K);

/* Smallest row stride (bytes) of an int8 activation matrix that the matmul
 * calls accept: K rounded up to a multiple of 64. */
int64_t bitlinear_q_stride(int64_t K);

/* Bytes of the BT5-T32 buffer for an N x K matrix:
 * ceil(N/32) * ceil(K/160) * 1024 (= N*K/5 when 32 divides N and 160 divides
 * K).  Returns 0 for sizes out of range. */
size_t bitlinear_packed5_bytes(int64_t N, int64_t K);

/* Smallest row stride (bytes) of the int8 activations bitlinear_matmul5
 * accepts: K rounded up to a multiple of 160. */
int64_t bitlinear_q_stride5(int64_t K);

/* Workspace bytes that `op` needs for these sizes (0 if none; SIZE_MAX if
 * the sizes are invalid).  M is ignored for BITLINEAR_WS_QUANTIZE_WEIGHTS. */
size_t bitlinear_workspace_bytes(int op, int64_t M, int64_t N, int64_t K);

/*
 * Weight quantization (absmean -> ternary), once per weight matrix: one
 * absmean scale per matrix, codes in {-1, 0, +1} (anthology note-168 on
 * arXiv 2402.17764, "What it does"; the scale is quantized once, ahead of
 * inference: BitNet b1.58 2B4T video transcript, yousumm.com,
 * "Transcription").
 *   W         [in]  N x K fp32.
 *   gamma_in  [in]  NULL: compute gamma = absmean of W (deterministic fp64
 *                   two-stage reduction, rounded once to fp32).  Non-NULL:
 *                   device pointer to one fp32 used as gamma instead.
 *   T_out     [out] N x K int8 codes in {-1, 0, +1}.
 *   gamma_out [out] one fp32: the scale used.
 *   ws        workspace of bitlinear_workspace_bytes(BITLINEAR_WS_QUANTIZE_
 *             WEIGHTS, 0, N, K) bytes (may be NULL when that is 0).
 */
int bitlinear_quantize_weights(const float *W, int64_t N, int64_t K, const float *gamma_in,
                               int8_t *T_out, float *gamma_out, void *ws, size_t ws_bytes,
                               void *stream);

/*
 * Pack ternary codes into BL2-T64, four codes per byte (BitNet b1.58 2B4T
 * video transcript, yousumm.com, "Transcription": four codes are packed
 * into one byte and unpacked next to the math units).
 *   T      [in]  N x K int8 codes; values outside {-1, 0, +1} are clamped.
 *   P_out  [out] bitlinear_packed_bytes(N, K) bytes; padding is written too.
 */
int bitlinear_pack(const int8_t *T, int64_t N, int64_t K, uint8_t *P_out, void *stream);

/*
 * Unpack BL2-T64 back to N x K int8 codes (inverse of bitlinear_pack; a
 * malformed field 3 decodes as 0).
 */
int bitlinear_unpack(const uint8_t *P, int64_t N, int64_t K, int8_t *T_out, void *stream);

/*
 * Per-token absmax int8 activation quantization (anthology note-168 on
 * arXiv 2402.17764, "What it does": the activations are 8-bit; per-token
 * absmax scaling is the reading taken).
 *   X          [in]  M x K fp32.
 *   Q_out      [out] M rows of ldq bytes: K int8 codes, then zeros up to ldq.
 *   ldq        row stride of Q_out in bytes, ldq >= K, ldq % 16 == 0.
 *   absmax_out [out] M fp32 scales a[m].
 *   rowsum_out [out] M int32 sums of each row of Q (nullable).
 */
int bitlinear_quant_act(const float *X, int64_t M, int64_t K, int8_t *Q_out, int64_t ldq,
                        float *absmax_out, int32_t *rowsum_out, void *stream);

/*
 * Sub-layer norm, then the per-token absmax int8 cast, in one pass over X
 * (BitNet b1.58 2B4T video transcript, yousumm.com, "Transcription": a
 * sub-layer norm sits before the quantized layers; the formula is not
 * given -- the reading taken is RMSNorm with a per-channel gain):
 *   inv[m]   = (float)(1 / sqrt(sum_k X[m][k]^2 / K + eps)), fp64 inside;
 *   Xhat[m][k] = (X[m][k] * inv[m]) * norm_weight[k] (two fp32 roundings);
 *   then exactly bitlinear_quant_act on Xhat (absmax_out is max |Xhat|).
 *   norm_weight [in] K fp32 gains, 4-byte aligned; NULL means all ones.
 *   eps          >= 0 and finite, else BITLINEAR_ERR_ARG.
 *   Other arguments, layouts and errors as bitlinear_quant_act.
 */
int bitlinear_quant_act_rmsnorm(const float *X, int64_t M, int64_t K, const float *norm_weight,
                                float eps, int8_t *Q_out, int64_t ldq, float *absmax_out,
                                int32_t *rowsum_out, void *stream);

/*
 * Residual add, then bitlinear_quant_act_rmsnorm, in one pass: the input of
 * the next sub-layer of a stack of BitLinear blocks (the sub-layer norm of
 * the BitNet b1.58 2B4T video transcript, yousumm.com, "Transcription",
 * applied to the residual stream; the reading taken is the pre-norm block
 * x_next = x + sublayer(norm(x))):
 *   Xsum[m][k] = X[m][k] + R[m][k]   (fp32, one rounding; written out)
 *   then exactly bitlinear_quant_act_rmsnorm on Xsum.
 *   X, R      [in]  M x K fp32 (16-byte aligned): residual stream and the
 *                   sub-layer output added to it.
 *   Xsum_out  [out] M x K fp32 (16-byte aligned); it may be X or R itself
 *                   (in-place update), but may not otherwise overlap X, R or
 *                   Q_out (BITLINEAR_ERR_ARG).
 *   Other arguments, layouts and errors as bitlinear_quant_act_rmsnorm.
 */
int bitlinear_quant_act_add_rmsnorm(const float *X, const float *R, int64_t M, int64_t K,
                                    const float *norm_weight, float eps, float *Xsum_out,
                                    int8_t *Q_out, int64_t ldq, float *absmax_out,
                                    int32_t *rowsum_out, void *stream);

/*
 * Gated squared-ReLU feed-forward activation, then the per-token absmax
 * int8 cast, in one pass: the input of a feed-forward block's down
 * projection (BitNet b1.58 2B4T video transcript, yousumm.com,
 * "Transcription": the activation function is a squared ReLU; the formula
 * is not given -- the reading taken is the gated form
 *   H[m][n] = (r * r) * U[m][n],  r = max(G[m][n], 0), in fp32),
 * then exactly bitlinear_quant_act on H (absmax_out is max |H|).
 *   G, U      [in]  M x N fp32: the gate and up projections' outputs
 *                   (row-major, 16-byte aligned).
 *   Q_out, ldq, absmax_out, rowsum_out: as bitlinear_quant_act with K = N.
 */
int bitlinear_quant_act_relu2_gate(const float *G, const float *U, int64_t M, int64_t N,
                                   int8_t *Q_out, int64_t ldq, float *absmax_out,
                                   int32_t *rowsum_out, void *stream);

/*
 * Ternary x int8 contraction and rescale from already-quantized activations
 * (lets a caller supply Q, a and the row sums itself).
 *   Q       [in]  M rows of ldq bytes, bitlinear_q_stride(K) <= ldq <= 2^26,
 *                 ldq % 16 == 0; bytes K..ldq-1 of each row must be 0.
 *   absmax  [in]  M fp32 activation scales.
 *   rowsum  [in]  M int32, rowsum[m] = sum_k Q[m,k].
 *   P       [in]  BL2-T64 weights of an N x K matrix.
 *   gamma   [in]  one fp32 weight scale (device).
 *   Y_out   [out] M x N fp32.
 *   acc_out [out] M x N int32 exact accumulators (nullable; for checking).
 *   ws      bitlinear_workspace_bytes(BITLINEAR_WS_MATMUL, M, N, K) bytes.
 */
int bitlinear_matmul(const int8_t *Q, int64_t ldq, const float *absmax, const int32_t *rowsum,
                     int64_t M, int64_t K, const uint8_t *P, const float *gamma, int64_t N,
                     float *Y_out, int32_t *acc_out, void *ws, size_t ws_bytes, void *stream);

/*
 * BT5-T32 packing of ternary codes (five per byte, format above).
 *   T      [in]  N x K int8 codes (values outside {-1, 0, +1} are clamped).
 *   P5_out [out] bitlinear_packed5_bytes(N, K) bytes; padding is written.
 */
int bitlinear_pack5(const int8_t *T, int64_t N, int64_t K, uint8_t *P5_out, void *stream);

/* Inverse of bitlinear_pack5 (for checking): T_out receives N x K codes,
 * decoded with the same digit planes the contraction uses. */
int bitlinear_unpack5(const uint8_t *P5, int64_t N, int64_t K, int8_t *T_out, void *stream);

/*
 * bitlinear_matmul over BT5-T32 weights: the same results, bit for bit
 * (acc exact, Y = float(acc) * ((gamma * a) / 127)).
 *   Q       [in]  M rows of ldq bytes, ldq >= bitlinear_q_stride5(K), a
 *                 multiple of 16 and <= 2^26; bytes k >= K of each row up to
 *                 bitlinear_q_stride5(K) must be zero.
 *   P5      [in]  BT5-T32 weights of an N x K matrix.
 *   others  as for bitlinear_matmul; ws of bitlinear_workspace_bytes(
 *           BITLINEAR_WS_MATMUL5, M, N, K) bytes (0 when K is not split).
 * Any M is accepted; the kernel takes 16 tokens per pass over the weights,
 * so it is meant for decode and small batches.
 */
int bitlinear_matmul5(const int8_t *Q, int64_t ldq, const float *absmax, const int32_t *rowsum,
                      int64_t M, int64_t K, const uint8_t *P5, const float *gamma, int64_t N,
                      float *Y_out, int32_t *acc_out, void *ws, size_t ws_bytes, void *stream);

/*
 * The whole BitLinear forward over BT5-T32 weights (quantize X, then
 * bitlinear_matmul5).  ws: bitlinear_workspace_bytes(BITLINEAR_WS_FORWARD5,
 * M, N, K) bytes; it receives Q (stride bitlinear_q_stride5(K)), a and the
 * row sums.
 */
int bitlinear_forward5(const float *X, int64_t M, int64_t K, const uint8_t *P5,
                       const float *gamma, int64_t N, float *Y_out, int32_t *acc_out,
                       void *ws, size_t ws_bytes, void *stream);

/*
 * The whole BitLinear forward: quantize X per token, contract with the
 * packed ternary weights, rescale -- BitLinear in place of nn.Linear
 * (anthology note-168 on arXiv 2402.17764, "What it does"), the product
 * exact in integers (same note, "The part that is a bet rather than a
 * measurement").
 *   X       [in]  M x K fp32.          P, gamma as for bitlinear_matmul.
 *   Y_out   [out] M x N fp32.          acc_out as for bitlinear_matmul.
 *   ws      bitlinear_workspace_bytes(BITLINEAR_WS_FORWARD, M, N, K) bytes;
 *           it receives Q, a and the row sums (layout private).
 */
int bitlinear_forward(const float *X, int64_t M, int64_t K, const uint8_t *P,
                      const float *gamma, int64_t N, float *Y_out, int32_t *acc_out,
                      void *ws, size_t ws_bytes, void *stream);

/*
 * bitlinear_forward for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Results
 * are bit-identical to bitlinear_forward.  The workspace (int8 activations,
 * scales, row sums, split-K partial sums and arrival counters) is a fixed
 * device array inside the library, bitlinear_noalloc_scratch_bytes() bytes
 * (16 MiB) on each GPU, held until the process ends; its device address is
 * looked up once per device on the first call.  The call allocates and
 * frees nothing; the arrival counters it needs are cleared by its own
 * kernels.
 *   X, M, K, P, gamma, N, Y_out, acc_out  as bitlinear_forward.
 *   stream  must belong to the current device (else BITLINEAR_ERR_ARG).
 *   Sizes whose bitlinear_workspace_bytes(BITLINEAR_WS_FORWARD, M, N, K)
 *   exceed the array are rejected with BITLINEAR_ERR_WORKSPACE before
 *   anything is enqueued.
 * Every call on a GPU uses that GPU's one array: calls that can overlap on
 * one GPU (other streams, other host threads) race and must be serialized
 * by the caller.
 */
int bitlinear_forward_noalloc(const float *X, int64_t M, int64_t K, const uint8_t *P,
                              const float *gamma, int64_t N, float *Y_out, int32_t *acc_out,
                              void *stream);

/* Bytes of the scratch array bitlinear_forward_noalloc works in. */
size_t bitlinear_noalloc_scratch_bytes(void);

/* ---------------------------------------------------------------------- */
/* Several weight matrices on one int8 input (q|k|v, gate|up): one launch.  */
/* ---------------------------------------------------------------------- */

typedef struct bitlinear_weight {
    const uint8_t *P;   /* packed weights of an N x K matrix (device)        */
    const float *gamma; /* one fp32 weight scale (device)                    */
    float *Y;           /* M x N fp32 output (device)                        */
    int32_t *acc;       /* M x N int32 accumulators (device, nullable)       */
    int64_t N;
    int32_t format;     /* bitlinear_format of P; the same for all weights   */
    int32_t reserved;   /* must be 0                                         */
} bitlinear_weight;

/* Workspace bytes of bitlinear_matmul_multi for these weights (only N,
 * format and reserved are read; SIZE_MAX on invalid input; 0 when no matrix
 * splits K). */
size_t bitlinear_multi_workspace_bytes(const bitlinear_weight *w, int count, int64_t M, int64_t K);

/*
 * bitlinear_matmul (or bitlinear_matmul5, by format) for 1..4 weight
 * matrices that read the same activations, in one launch; each result is
 * bit-identical to the single call's.
 *   Q, ldq, absmax, rowsum, M, K  as bitlinear_matmul (bitlinear_matmul5
 *                 for BITLINEAR_FORMAT_BT5: ldq >= bitlinear_q_stride5(K)).
 *   w, count      the weight matrices (1 <= count <= 4).
 *   ws            bitlinear_multi_workspace_bytes(w, count, M, K) bytes.  Its
 *                 start holds split-K arrival counters: ZERO-FILL the
 *                 workspace once before its first use.  Every completed call
 *                 leaves the counters zero again, so later calls with the
 *                 same weights and sizes reuse it without a clearing launch;
 *                 calls with other sizes need their own zeroed workspace.
 *                 Calls that share a workspace must not run concurrently.
 */
int bitlinear_matmul_multi(const int8_t *Q, int64_t ldq, const float *absmax, const int32_t *rowsum,
                           int64_t M, int64_t K, const bitlinear_weight *w, int count, void *ws,
                           size_t ws_bytes, void *stream);

/* What bitlinear_cast_matmul_multi casts to int8 (the activation casts
 * above: quant_act, quant_act_rmsnorm, quant_act_relu2_gate,
 * quant_act_add_rmsnorm). */
enum bitlinear_cast_mode {
    BITLINEAR_CAST_PLAIN = 0,      /* X                                      */
    BITLINEAR_CAST_RMSNORM = 1,    /* RMSNorm(X) with gains aux (NULL: ones) */
    BITLINEAR_CAST_RELU2_GATE = 2, /* relu(X)^2 * aux (X gate, aux up)       */
    BITLINEAR_CAST_ADD_RMSNORM = 3 /* RMSNorm(X + R), X + R to X_out         */
};

/* Workspace bytes of bitlinear_cast_matmul_multi in `mode` (only N, format
 * and reserved of w are read; SIZE_MAX on invalid input). */
size_t bitlinear_cast_multi_workspace_bytes(int mode, const bitlinear_weight *w, int count, int64_t M, int64_t K);

/*
 * How many kernels bitlinear_cast_matmul_multi enqueues for these arguments:
 * 1 when the contraction's workgroups cast the row themselves, 2 when the
 * cast runs as its own kernel first (the rule is stated at that call).  Host
 * only: nothing is enqueued and no device memory is read.  Returns -1 where
 * bitlinear_cast_multi_workspace_bytes returns SIZE_MAX (bad mode, shapes
 * or weights).
 */
int bitlinear_cast_multi_launches(int mode, const bitlinear_weight *w, int count, int64_t M, int64_t K);

/*
 * The activation cast of `mode` followed by bitlinear_matmul_multi on its
 * int8 codes: a decode layer's sub-layer norm (or gated squared ReLU) and
 * the BitLinear matrices that read it, as the pages describe a BitNet block
 * (BitNet b1.58 2B4T video transcript, yousumm.com, "Transcription": a
 * norm before each BitLinear, squared ReLU in the feed-forward part; the
 * int8 cast: anthology note-168 on arXiv 2402.17764, "What it does").
 * Every Y (and acc) equals that of the cast call followed by
 * bitlinear_matmul_multi, bit for bit, and X_out that of the add mode's
 * cast -- except that with 8 waves per workgroup (launches of 257..512 row
 * tiles) the norm modes add the fp64 squares in another order, which moves
 * the fp32 norm factor only where the exact value lies within that rounding
 * of an fp32 rounding boundary.
 * One token whose weights take the wide one-token kernel (BL2-T64, few row
 * tiles, K <= 65536) in at most one workgroup per compute unit, each
 * reading fewer cast-input bytes than packed weights, is cast inside every
 * workgroup of the contraction launch, so the call is one launch; otherwise
 * the cast runs as its own kernel into the workspace.
 *   mode   a bitlinear_cast_mode.
 *   X      M x K fp32 rows (device; the gate projection's output for
 *          BITLINEAR_CAST_RELU2_GATE), 16-byte aligned.
 *   aux    RMSNorm gains [K] (nullable, 4-byte aligned) for the norm modes;
 *          the up projection's output (M x K, 16-byte aligned, required)
 *          for the gate; ignored for BITLINEAR_CAST_PLAIN.
 *   R      the addend of the residual sum (M x K, add mode only).
 *   eps    RMSNorm epsilon (finite, >= 0; norm modes only).
 *   X_out  receives X + R (add mode only); must not overlap X or R, which
 *          every workgroup reads while one writes X_out.
 *   M, K, w, count  as bitlinear_matmul_multi (K is the cast rows' length).
 *   ws     bitlinear_cast_multi_workspace_bytes(mode, w, count, M, K) bytes,
 *          ZERO-FILLED once before first use as for bitlinear_matmul_multi
 *          (the same reuse rules; calls sharing it must not overlap).
 * Errors: NULL (missing X, aux, R or X_out), SHAPE, ALIGN, ARG (mode, eps,
 * overlap, weights), WORKSPACE; nothing is enqueued on an error.
 */
int bitlinear_cast_matmul_multi(int mode, const float *X, const float *aux, const float *R, float eps,
                                float *X_out, int64_t M, int64_t K, const bitlinear_weight *w, int count,
                                void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------- */
/* Grouped forward: many independent BitLinear layers in one launch per    */
/* stage (e.g. every weight matrix of a model, or q|k|v sharing an input). */
/* ---------------------------------------------------------------------- */

typedef struct bitlinear_problem {
    const float *X;     /* M x K fp32 activations (device)                  */
    const uint8_t *P;   /* packed weights of the N x K matrix (device)      */
    const float *gamma; /* one fp32 weight scale (device)                   */
    float *Y;           /* M x N fp32 output (device)                       */
    int32_t *acc;       /* M x N int32 accumulators (device, nullable)      */
    int64_t M, N, K;
    int32_t format;     /* bitlinear_format of P (0 = BL2-T64)              */
    int32_t reserved;   /* must be 0                                        */
} bitlinear_problem;

/* Host bytes of the plan table for these problems (0 on invalid input),
 * and the device workspace bytes the group needs. */
size_t bitlinear_group_table_bytes(const bitlinear_problem *probs, int count);
size_t bitlinear_group_workspace_bytes(const bitlinear_problem *probs, int count);

/*
 * Validate the problems and write the plan table into HOST memory
 * (table_host, table_bytes >= bitlinear_group_table_bytes).  The plan binds
 * the problems' buffers and the device workspace `ws` (ws_bytes >=
 * bitlinear_group_workspace_bytes).  The caller copies the table byte for
 * byte to a 16-byte aligned device buffer and passes both copies to the
 * calls below; host copy gives launch sizes, device copy feeds the kernels.
 */
int bitlinear_group_plan(const bitlinear_problem *probs, int count, void *ws, size_t ws_bytes,
                         void *table_host, size_t table_bytes);

/* Stage 1 of the grouped forward: quantize every problem's activations. */
int bitlinear_group_quant_act(const void *table_host, const void *table_dev, void *stream);
/* Stage 2: contract and rescale every problem (reads stage 1's results). */
int bitlinear_group_matmul(const void *table_host, const void *table_dev, void *stream);
/* Both stages. */
int bitlinear_group_forward(const void *table_host, const void *table_dev, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* BITLINEAR_H */
