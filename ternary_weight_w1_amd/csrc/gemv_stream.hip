// Streaming contraction for small token counts (decode): M = 1 and 2 with
// packed int8 dot products, 3 <= M <= 32 with int8 matrix instructions (the
// split point is a host-side setting; the dot4 kernels take up to 4 tokens).
//
// The pages describe the decode kernel as: weights packed four codes per
// byte are streamed across the GPU and unpacked next to the math units,
// then multiplied with 8-bit activations (BitNet b1.58 2B4T video
// transcript, yousumm.com, "Transcription"); the product needs only
// integer additions (anthology note-168 on arXiv 2402.17764, "The part that
// is a bet rather than a measurement").  On gfx950 this regime is bound by
// HBM: every packed byte is read once and carries 4 codes, so the kernel is
// built to keep many 16-byte non-temporal loads in flight and to spend as
// few VALU operations per code as possible.
//
// Work item = (problem, 64-row weight tile, K split).  A 256-thread
// workgroup owns one item; its four waves take every fourth 64-code unit of
// the split, so together they stream 4 KiB of contiguous packed weights per
// step.  Each lane loads one 16-byte slot of the unit's 1 KiB block: words
// (s, h) hold 16 codes of rows r and 32 + r (r = lane % 32) for code chunk
// lane / 32 of half h.
//
// M = 1 (dot4):   plane j of a word times the matching 4 activation bytes
//                 with v_dot4c_i32_i8: per 16 codes 7 bit operations + 4
//                 dot products.  The (t+1) fields make the sum exceed the
//                 ternary dot product by the activation row sum, which the
//                 epilogue subtracts once.  With 2..4 tokens the planes are
//                 unpacked once and serve every token.
// M <= 32 (mfma): the four planes of a word are exactly one lane's B operand
//                 of v_mfma_i32_32x32x32_i8 (A = 32 token rows of int8
//                 activations, zero beyond M), so per 1 KiB unit a wave
//                 issues 4 MFMAs after 28 bit operations, whatever M is.
//
// Partial sums of the four waves meet in LDS; with K split over several
// workgroups the last one to arrive (atomic ticket) adds the splits.
// Integer addition is associative, so every order gives the same bits.
#include "mm_common.hpp"

namespace bl {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;

__device__ inline int dot16(unsigned w, v4i q, int acc)
{
    acc = __builtin_amdgcn_sdot4((int)(w & 0x03030303u), q.x, acc, false);
    acc = __builtin_amdgcn_sdot4((int)((w >> 2) & 0x03030303u), q.y, acc, false);
    acc = __builtin_amdgcn_sdot4((int)((w >> 4) & 0x03030303u), q.z, acc, false);
    acc = __builtin_amdgcn_sdot4((int)((w >> 6) & 0x03030303u), q.w, acc, false);
    return acc;
}

// Activations of the workgroup's K range, staged once per workgroup when
// the dot4 kernel runs with QLDS (dynamic LDS, 64 bytes per unit).
extern __shared__ __attribute__((aligned(16))) int8_t stream_q_lds[];

// Copies n 16-byte chunks into the staged activations, chunk i from src(i):
// each thread issues up to eight loads before its first LDS store, so a
// workgroup's staging costs one memory round trip per 8 * 256 chunks
// rather than one per 256.
template <typename Src>
__device__ __forceinline__ void stage_chunks(int n, Src src)
{
    v4i *dst = reinterpret_cast<v4i *>(stream_q_lds);
    for (int base = threadIdx.x; base < n; base += 8 * kThreads) {
        v4i v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (base + k * kThreads < n) v[k] = src(base + k * kThreads);
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (base + k * kThreads < n) dst[base + k * kThreads] = v[k];
    }
}

// Stages units [u0, u1) of the first M token rows of Q (row stride ldq) with
// MT slots per unit: slot m of unit u0 + uu at byte (uu * MT + m) * 64,
// slots M .. MT-1 zero.  Thread t always copies chunk t % 4 of slot
// (t / 4) % MT, for every (256 / (4 MT))-th unit, with up to eight loads in
// flight before its first LDS store.
template <int MT>
__device__ __forceinline__ void stage_token_slots(const Problem &p, int u0, int u1)
{
    static_assert(MT >= 1 && 4 * MT <= kThreads, "one pass covers at least one unit");
    constexpr int kPer = kThreads / (4 * MT);  // units per pass
    const int t = threadIdx.x, ch = t & 3, m = (t >> 2) % MT, uo = t / (4 * MT);
    const bool live = m < p.M && uo < kPer;
    const BL_GLOBAL int8_t *src = gload_ptr<int8_t>(p.Q) + (int64_t)(m < p.M ? m : 0) * p.ldq + 64 * u0 + 16 * ch;
    v4i *dst = reinterpret_cast<v4i *>(stream_q_lds) + m * 4 + ch;
    const v4i zero = {0, 0, 0, 0};
    const int nu = u1 - u0;
    for (int ub = uo; ub < nu; ub += 8 * kPer) {
        v4i v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (ub + k * kPer < nu) v[k] = live ? *reinterpret_cast<const BL_GLOBAL v4i *>(src + 64 * (ub + k * kPer)) : zero;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (ub + k * kPer < nu && uo < kPer) dst[(ub + k * kPer) * MT * 4] = v[k];
    }
}

// Fused prologue (decode, one token): quantize the token's fp32 activations
// straight into LDS -- absmax over the whole row (block reduction), then
// the same per-element code as the quantization kernel -- keeping the codes
// of units [u0, u1) and the row sum of all of them.  Replaces a separate
// quantization launch; the row is re-read from L1/L2 in the second pass.
__device__ void fused_quant_token(const Problem &p, int u0, int u1, float &absmax, int &rowsum)
{
    __shared__ float fmax_l[kWaves];
    __shared__ int isum_l[kWaves];
    const int tid = threadIdx.x, K = p.K;
    const BL_GLOBAL float *x = gload_ptr<float>(p.X);
    typedef float v4f __attribute__((ext_vector_type(4)));
    const bool vec = ((K & 3) == 0) && ((reinterpret_cast<uintptr_t>(p.X) & 15) == 0);
    const BL_GLOBAL v4f *x4 = reinterpret_cast<const BL_GLOBAL v4f *>(x);
    float a = 0.0f;
    if (vec) {
        for (int i = tid; i < (K >> 2); i += kThreads) {
            const v4f w = x4[i];
            a = fmaxf(a, fmaxf(fmaxf(fabsf(w.x), fabsf(w.y)), fmaxf(fabsf(w.z), fabsf(w.w))));
        }
    } else {
        for (int i = tid; i < K; i += kThreads) a = fmaxf(a, fabsf(x[i]));
    }
    for (int off = 32; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
    if ((tid & 63) == 0) fmax_l[tid >> 6] = a;
    __syncthreads();
    a = fmaxf(fmaxf(fmax_l[0], fmax_l[1]), fmaxf(fmax_l[2], fmax_l[3]));
    if (!(a >= 1e-5f)) a = 1e-5f;
    const float s = 127.0f / a;

    const int k0 = 64 * u0, k1 = 64 * u1;  // LDS holds codes k0 .. k1-1
    int sum = 0;
    if (vec) {
        for (int i = tid; i < (K >> 2); i += kThreads) {
            const v4f w = x4[i];
            const int8_t c0 = quant_code(w.x, s), c1 = quant_code(w.y, s);
            const int8_t c2 = quant_code(w.z, s), c3 = quant_code(w.w, s);
            sum += (int)c0 + (int)c1 + (int)c2 + (int)c3;
            const int k = 4 * i;
            if (k >= k0 && k < k1)
                *reinterpret_cast<uint32_t *>(stream_q_lds + (k - k0)) =
                    (uint32_t)(uint8_t)c0 | ((uint32_t)(uint8_t)c1 << 8) |
                    ((uint32_t)(uint8_t)c2 << 16) | ((uint32_t)(uint8_t)c3 << 24);
        }
    } else {
        for (int k = tid; k < K; k += kThreads) {
            const int8_t c = quant_code(x[k], s);
            sum += c;
            if (k >= k0 && k < k1) stream_q_lds[k - k0] = c;
        }
    }
    for (int k = (K > k0 ? K : k0) + tid; k < k1; k += kThreads) stream_q_lds[k - k0] = 0;
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
    if ((tid & 63) == 0) isum_l[tid >> 6] = sum;
    __syncthreads();
    absmax = a;
    rowsum = isum_l[0] + isum_l[1] + isum_l[2] + isum_l[3];
}

// Table-lookup variant, kept to compare against the dot4 stream: the pages
// say the existing GPU path of the model uses lookup tables rather than
// native tensor operations ("BitNet: Microsoft's AI Revolution Shows Why
// Precision May be Overrated", promptinjection.net, "4. GPU Support: The
// Fragile Boost").  Reading taken: for every pair of codes a nibble of the
// packed word holds (two 2-bit fields f0, f1), the workgroup tabulates the
// 16 possible partial sums f0 * q0 + f1 * q1 of the token's activations once;
// the stream then replaces each nibble's multiply by one 16-bit LDS read.
// Byte b of a word holds codes b, b + 4, b + 8, b + 12 of its 16 (bits 0, 2,
// 4, 6), so nibble x of byte b pairs codes b + 8x and b + 8x + 4.
// Table layout: for unit u of the range, word wi = 2 h + g of the unit and
// pair pi = 2 b + x, the 16 int16 entries sit at byte
// ((u - u0) * 32 + wi * 8 + pi) * 32 -- 1 KiB per 64-code unit.
constexpr int kLutUnitBytes = 1024;

__device__ inline int lut16(unsigned w, const int8_t *base)
{
    int s = 0;
#pragma unroll
    for (int pi = 0; pi < 8; ++pi) {
        const unsigned v = (w >> (4 * pi)) & 0xFu;  // bit 8 b + 4 x = 4 pi
        s += *reinterpret_cast<const int16_t *>(base + 32 * pi + 2 * v);
    }
    return s;
}

__device__ void build_lut(const Problem &p, int u0, int u1)
{
    const BL_GLOBAL int8_t *q = gload_ptr<int8_t>(p.Q);  // token 0, zero beyond K
    for (int pg = threadIdx.x; pg < 32 * (u1 - u0); pg += kThreads) {
        const int uu = pg >> 5, wi = (pg >> 3) & 3, pi = pg & 7;
        const int k = 64 * (u0 + uu) + 32 * (wi >> 1) + 16 * (wi & 1) + (pi >> 1) + 8 * (pi & 1);
        const int q0 = q[k], q1 = q[k + 4];
        int e[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) e[v] = (v & 3) * q0 + (v >> 2) * q1;
        v4i lo, hi;
        lo.x = (e[0] & 0xFFFF) | (e[1] << 16);
        lo.y = (e[2] & 0xFFFF) | (e[3] << 16);
        lo.z = (e[4] & 0xFFFF) | (e[5] << 16);
        lo.w = (e[6] & 0xFFFF) | (e[7] << 16);
        hi.x = (e[8] & 0xFFFF) | (e[9] << 16);
        hi.y = (e[10] & 0xFFFF) | (e[11] << 16);
        hi.z = (e[12] & 0xFFFF) | (e[13] << 16);
        hi.w = (e[14] & 0xFFFF) | (e[15] << 16);
        v4i *dst = reinterpret_cast<v4i *>(stream_q_lds + 32 * pg);
        dst[0] = lo;
        dst[1] = hi;
    }
}

// QLDS: read the activations with broadcast LDS reads (2 distinct 16-byte
// addresses per half wave) instead of two 16-byte global loads per lane per
// unit, which would triple the vector-memory instructions of the stream.
// FUSED: the activations are quantized in the prologue (implies QLDS).
// LUT: the table-lookup variant above instead of dot products.
template <int UNROLL, bool QLDS, bool FUSED = false, bool LUT = false>
__device__ void stream_dot4(const Problem &p, int local)
{
    static_assert(!FUSED || QLDS, "the fused prologue writes the LDS activations");
    static_assert(!LUT || (QLDS && !FUSED), "the table takes the LDS");
    __shared__ int red[kWaves][64];
    const int tile = local / p.ks, split = local - tile * p.ks;
    const int u0 = split * p.upsplit;
    const int u1 = min(p.KU, u0 + p.upsplit);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 5;
    const BL_GLOBAL v4u *blk = gload_ptr<v4u>(p.P + (int64_t)tile * p.KU * kBlockBytes) + lane;
    const BL_GLOBAL int8_t *qg = gload_ptr<int8_t>(p.Q) + 16 * g;  // token 0; chunk g of each 32-code half
    float tok_absmax = 0.0f;
    int tok_rowsum = 0;
    if constexpr (FUSED) {
        fused_quant_token(p, u0, u1, tok_absmax, tok_rowsum);
    } else if constexpr (LUT) {
        build_lut(p, u0, u1);
        __syncthreads();
    } else if constexpr (QLDS) {
        const BL_GLOBAL v4i *src = gload_ptr<v4i>(p.Q + 64 * u0);
        stage_chunks(4 * (u1 - u0), [&](int i) { return src[i]; });
        __syncthreads();
    }
    auto finish = [&](int n, int32_t fields, float gamma) {
        if constexpr (FUSED)
            finish_output_with(p, gamma, 0, n, fields, tok_rowsum, tok_absmax);
        else
            finish_output(p, gamma, 0, n, fields);
    };
    // activation bytes 64*u + 16*g (+32 for the second half) of unit u
    auto qload = [&](int u, int off) -> v4i {
        if constexpr (QLDS)
            return *reinterpret_cast<const v4i *>(stream_q_lds + 64 * (u - u0) + 16 * g + off);
        else
            return *reinterpret_cast<const BL_GLOBAL v4i *>(qg + 64 * u + off);
    };

    int acc0 = 0, acc1 = 0;  // rows r and 32 + r of the tile
    int u = u0 + wave;
    if constexpr (LUT) {
        // words (s, h): x = (0, 0), y = (0, 1), z = (1, 0), w = (1, 1); lane
        // half g selects the table of code chunk g
        for (; u + kWaves * (UNROLL - 1) < u1; u += kWaves * UNROLL) {
            v4u w[UNROLL];
#pragma unroll
            for (int j = 0; j < UNROLL; ++j) w[j] = load_packed(blk + (int64_t)(u + kWaves * j) * 64);
#pragma unroll
            for (int j = 0; j < UNROLL; ++j) {
                const int8_t *t0 = stream_q_lds + (u + kWaves * j - u0) * kLutUnitBytes + g * 256;
                acc0 += lut16(w[j].x, t0) + lut16(w[j].y, t0 + 512);
                acc1 += lut16(w[j].z, t0) + lut16(w[j].w, t0 + 512);
            }
        }
        for (; u < u1; u += kWaves) {
            const v4u w = load_packed(blk + (int64_t)u * 64);
            const int8_t *t0 = stream_q_lds + (u - u0) * kLutUnitBytes + g * 256;
            acc0 += lut16(w.x, t0) + lut16(w.y, t0 + 512);
            acc1 += lut16(w.z, t0) + lut16(w.w, t0 + 512);
        }
        u = u1;  // the dot4 loops below have nothing left
    }
    for (; u + kWaves * (UNROLL - 1) < u1; u += kWaves * UNROLL) {
        v4u w[UNROLL];
        v4i qa[UNROLL], qb[UNROLL];
#pragma unroll
        for (int j = 0; j < UNROLL; ++j) w[j] = load_packed(blk + (int64_t)(u + kWaves * j) * 64);
#pragma unroll
        for (int j = 0; j < UNROLL; ++j) {
            qa[j] = qload(u + kWaves * j, 0);
            qb[j] = qload(u + kWaves * j, 32);
        }
#pragma unroll
        for (int j = 0; j < UNROLL; ++j) {
            acc0 = dot16(w[j].x, qa[j], acc0);
            acc0 = dot16(w[j].y, qb[j], acc0);
            acc1 = dot16(w[j].z, qa[j], acc1);
            acc1 = dot16(w[j].w, qb[j], acc1);
        }
    }
    if (u < u1) {
        // the last (fewer than UNROLL) units of this wave, loaded together:
        // with K split finely (small launches) they are all a wave has
        v4u w[UNROLL - 1];
#pragma unroll
        for (int j = 0; j < UNROLL - 1; ++j)
            if (u + kWaves * j < u1) w[j] = load_packed(blk + (int64_t)(u + kWaves * j) * 64);
#pragma unroll
        for (int j = 0; j < UNROLL - 1; ++j)
            if (u + kWaves * j < u1) {
                const v4i qa = qload(u + kWaves * j, 0);
                const v4i qb = qload(u + kWaves * j, 32);
                acc0 = dot16(w[j].x, qa, acc0);
                acc0 = dot16(w[j].y, qb, acc0);
                acc1 = dot16(w[j].z, qa, acc1);
                acc1 = dot16(w[j].w, qb, acc1);
            }
    }
    // lanes r and r + 32 hold the two code chunks of the same rows
    acc0 += __shfl_xor(acc0, 32, 64);
    acc1 += __shfl_xor(acc1, 32, 64);
    if (lane < 32) {
        red[wave][lane] = acc0;
        red[wave][32 + lane] = acc1;
    }
    __syncthreads();

    const int t = threadIdx.x;
    const int n = 64 * tile + t;
    const float gamma = *p.gamma;
    int total = 0;
    if (t < 64) total = red[0][t] + red[1][t] + red[2][t] + red[3][t];
    if (p.ks == 1) {
        if (t < 64 && n < p.N) finish(n, total, gamma);
        return;
    }
    const int64_t ldp = (int64_t)p.NT * 64;  // partial row stride
    if (t < 64) put_partial(p.acc_ws + ((int64_t)split * p.M * ldp + n), total);
    if (!arrive_last(p, tile)) return;
    const int64_t off[1] = {n};
    const bool ok[1] = {t < 64 && n < p.N};
    int32_t sum[1];
    sum_partials<1>(p.acc_ws, off, ok, (int64_t)p.M * ldp, p.ks, sum);
    if (ok[0]) finish(n, sum[0], gamma);
}

// 1..4 tokens (dot4): the four planes of a packed word are unpacked once
// and serve every token, so each token costs 4 dot products per 16 codes on
// top of the 7 shared bit operations.  The K range's activations are staged
// once per workgroup in LDS, unit by unit and token by token within a unit
// (64 bytes per token per unit: ((u - u0) * MT + m) * 64), so the reads of
// one unit are broadcast reads as in the one-token kernel.  Split K, the
// cross-wave sum and the epilogue work as there, with one row of partials
// per token; workgroup thread t finishes token t / 64, row t % 64.
template <int UNROLL, int MT>
__device__ __forceinline__ void stream_dot4_tokens(const Problem &p, int local)
{
    static_assert(MT >= 1 && MT * 64 <= kThreads, "one epilogue thread per (token, row)");
    __shared__ int red[kWaves][MT][64];
    const int tile = local / p.ks, split = local - tile * p.ks;
    const int u0 = split * p.upsplit;
    const int u1 = min(p.KU, u0 + p.upsplit);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 5;
    const BL_GLOBAL v4u *blk = gload_ptr<v4u>(p.P + (int64_t)tile * p.KU * kBlockBytes) + lane;
    stage_token_slots<MT>(p, u0, u1);
    __syncthreads();
    int acc0[MT], acc1[MT];  // rows r and 32 + r of the tile, per token
#pragma unroll
    for (int m = 0; m < MT; ++m) acc0[m] = acc1[m] = 0;
    auto dot4x4 = [](v4i pl, v4i q, int acc) {
        acc = __builtin_amdgcn_sdot4(pl.x, q.x, acc, false);
        acc = __builtin_amdgcn_sdot4(pl.y, q.y, acc, false);
        acc = __builtin_amdgcn_sdot4(pl.z, q.z, acc, false);
        acc = __builtin_amdgcn_sdot4(pl.w, q.w, acc, false);
        return acc;
    };
    // words (s, h): x = (0, 0), y = (0, 1), z = (1, 0), w = (1, 1)
    auto unit = [&](v4u w, int u) {
        const v4i px = planes(w.x), py = planes(w.y), pz = planes(w.z), pw = planes(w.w);
        const int8_t *qu = stream_q_lds + (u - u0) * MT * 64 + 16 * g;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const v4i qa = *reinterpret_cast<const v4i *>(qu + 64 * m);
            const v4i qb = *reinterpret_cast<const v4i *>(qu + 64 * m + 32);
            acc0[m] = dot4x4(py, qb, dot4x4(px, qa, acc0[m]));
            acc1[m] = dot4x4(pw, qb, dot4x4(pz, qa, acc1[m]));
        }
    };
    int u = u0 + wave;
    for (; u + kWaves * (UNROLL - 1) < u1; u += kWaves * UNROLL) {
        v4u w[UNROLL];
#pragma unroll
        for (int j = 0; j < UNROLL; ++j) w[j] = load_packed(blk + (int64_t)(u + kWaves * j) * 64);
#pragma unroll
        for (int j = 0; j < UNROLL; ++j) unit(w[j], u + kWaves * j);
    }
    if (u < u1) {
        // the last (fewer than UNROLL) units of this wave, loaded together
        v4u w[UNROLL - 1];
#pragma unroll
        for (int j = 0; j < UNROLL - 1; ++j)
            if (u + kWaves * j < u1) w[j] = load_packed(blk + (int64_t)(u + kWaves * j) * 64);
#pragma unroll
        for (int j = 0; j < UNROLL - 1; ++j)
            if (u + kWaves * j < u1) unit(w[j], u + kWaves * j);
    }
    // lanes r and r + 32 hold the two code chunks of the same rows
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        acc0[m] += __shfl_xor(acc0[m], 32, 64);
        acc1[m] += __shfl_xor(acc1[m], 32, 64);
    }
    if (lane < 32) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            red[wave][m][lane] = acc0[m];
            red[wave][m][32 + lane] = acc1[m];
        }
    }
    __syncthreads();

    const int t = threadIdx.x;
    const int m = t >> 6, row = t & 63;
    const int n = 64 * tile + row;
    const bool mine = t < 64 * MT && m < p.M;
    const float gamma = *p.gamma;
    int total = 0;
    if (mine) total = red[0][m][row] + red[1][m][row] + red[2][m][row] + red[3][m][row];
    if (p.ks == 1) {
        if (mine && n < p.N) finish_output(p, gamma, m, n, total);
        return;
    }
    const int64_t ldp = (int64_t)p.NT * 64;  // partial row stride
    if (mine) put_partial(p.acc_ws + (((int64_t)split * p.M + m) * ldp + n), total);
    if (!arrive_last(p, tile)) return;
    const int64_t off[1] = {(int64_t)m * ldp + n};
    const bool ok[1] = {mine && n < p.N};
    int32_t sum[1];
    sum_partials<1>(p.acc_ws, off, ok, (int64_t)p.M * ldp, p.ks, sum);
    if (ok[0]) finish_output(p, gamma, m, n, sum[0]);
}

// 3..32 tokens (2..32 when the dot4 kernels are limited to one): the same
// packed stream feeds v_mfma_i32_32x32x32_i8 with the token rows as the A
// operand.  A workgroup covers 4 * TPW
// 64-row tiles over one K range: each wave owns TPW tiles and
// every wave walks the same units in the same order, so a wave streams its
// tiles' blocks contiguously, one activation fragment serves all its tiles,
// the four waves fetch that fragment at about the same time (one L2 read,
// three L1 hits), and each wave ends with complete sums -- no cross-wave
// reduction, no LDS, no barrier.  Loads run one group of UNROLL units ahead
// of the MFMAs through a two-slot register ring (branch-free: unit indices
// clamp to the range end and surplus units get zero weights, which add
// nothing).
template <int UNROLL, int TPW>
__device__ void stream_mfma(const Problem &p, int local)
{
    const int grp = local / p.ks, split = local - grp * p.ks;
    const int u0 = split * p.upsplit;
    const int u1 = min(p.KU, u0 + p.upsplit);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, g = lane >> 5, r = lane & 31;
    const int tile0 = 4 * TPW * grp + TPW * wave;
    // tiles past NT stream tile NT-1 (valid memory); their sums are dropped
    const BL_GLOBAL v4u *blk[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
        blk[t] = gload_ptr<v4u>(p.P + (int64_t)min(tile0 + t, p.NT - 1) * p.KU * kBlockBytes) + lane;
    // A operand of unit u, half h: fragment-ordered activations hold it as one
    // contiguous 1 KiB block (16 bytes per lane); row-major activations give
    // each lane 16 bytes of its token row (lanes of rows past M load nothing).
    const bool rv = p.qtiled || r < p.M;
    const BL_GLOBAL int8_t *qbase;
    int64_t ustride, hoff;
    if (p.qtiled) {
        qbase = gload_ptr<int8_t>(p.Q) + 16 * lane;
        ustride = 2048;
        hoff = 1024;
    } else {
        qbase = gload_ptr<int8_t>(p.Q) + (int64_t)min(r, p.M - 1) * p.ldq + 16 * g;
        ustride = 64;
        hoff = 32;
    }
    const v4i zero = {0, 0, 0, 0};
    const v4u zw = {0u, 0u, 0u, 0u};
    // the tokens' row sums and absmax, fetched now so that their latency
    // hides under the stream (read per output element at the end)
    __shared__ int s_rowsum[kStreamMaxTokens];
    __shared__ float s_absmax[kStreamMaxTokens];
    if (threadIdx.x < p.M) {
        s_rowsum[threadIdx.x] = gload_ptr<int32_t>(p.rowsum)[threadIdx.x];
        s_absmax[threadIdx.x] = gload_ptr<float>(p.absmax)[threadIdx.x];
    }

    const int n_units = u1 - u0;
    const int groups = (n_units + UNROLL - 1) / UNROLL;
    v4u w[2][UNROLL][TPW];
    v4i qa[2][UNROLL], qb[2][UNROLL];
    auto load_group = [&](int slot, int i) {
#pragma unroll
        for (int j = 0; j < UNROLL; ++j) {
            const int u = min(u0 + UNROLL * i + j, u1 - 1);
#pragma unroll
            for (int t = 0; t < TPW; ++t) w[slot][j][t] = load_packed(blk[t] + (int64_t)u * 64);
            const BL_GLOBAL int8_t *qu = qbase + ustride * u;
            qa[slot][j] = rv ? *reinterpret_cast<const BL_GLOBAL v4i *>(qu) : zero;
            qb[slot][j] = rv ? *reinterpret_cast<const BL_GLOBAL v4i *>(qu + hoff) : zero;
        }
    };
    v16i acc[TPW][2];
#pragma unroll
    for (int t = 0; t < TPW; ++t) acc[t][0] = acc[t][1] = (v16i){};
    // Both halves of every unit of the group, first half first: consecutive
    // updates of one accumulator are 2 * TPW MFMAs apart, so the matrix pipe
    // never waits on its own previous result.
    auto run_group = [&](int slot, int i) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < UNROLL; ++j) {
                const bool live = UNROLL * i + j < n_units;
                const v4i a = h ? qb[slot][j] : qa[slot][j];
#pragma unroll
                for (int t = 0; t < TPW; ++t) {
                    const v4u wj = live ? w[slot][j][t] : zw;
                    acc[t][0] = mfma_i8(a, planes(h ? wj.y : wj.x), acc[t][0]);
                    acc[t][1] = mfma_i8(a, planes(h ? wj.w : wj.z), acc[t][1]);
                }
            }
    };
    load_group(0, 0);
    int i = 0;
    for (; i + 2 <= groups; i += 2) {
        load_group(1, i + 1);
        run_group(0, i);
        load_group(0, i + 2);
        run_group(1, i + 1);
    }
    if (i < groups) run_group(0, i);

    // element e of lane l is token 8*(e/4) + 4*(l/32) + e%4, row 32*s + l%32
    const float gamma = *p.gamma;
    const int64_t ldp = (int64_t)p.NT * 64;
    __syncthreads();  // the token scales are in LDS
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        if (tile0 + t >= p.NT) continue;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const int n = 64 * (tile0 + t) + 32 * s2 + r;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int m = 8 * (e >> 2) + 4 * g + (e & 3);
                if (m < p.M && n < p.N) {
                    if (p.ks == 1)
                        finish_output_with(p, gamma, m, n, acc[t][s2][e], s_rowsum[m], s_absmax[m]);
                    else
                        put_partial(p.acc_ws + (((int64_t)split * p.M + m) * ldp + n), acc[t][s2][e]);
                }
            }
        }
    }
    if (p.ks == 1) return;
    // split K: the last workgroup of the tile group sums its tiles
    constexpr int kRows = 256 * TPW;
    if (!arrive_last(p, 4 * TPW * grp)) return;
    const int total = p.M * kRows;
    for (int base = threadIdx.x; base < total; base += 4 * kThreads) {
        int64_t off[4];
        bool ok[4];
        int mm[4], nn[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int idx = base + r * kThreads;
            mm[r] = idx / kRows;
            nn[r] = kRows * grp + idx % kRows;
            ok[r] = idx < total && nn[r] < p.N;
            off[r] = (int64_t)mm[r] * ldp + nn[r];
        }
        int32_t sums[4];
        sum_partials<4>(p.acc_ws, off, ok, (int64_t)p.M * ldp, p.ks, sums);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (ok[r]) finish_output_with(p, gamma, mm[r], nn[r], sums[r], s_rowsum[mm[r]], s_absmax[mm[r]]);
    }
}

// 0: dot4, activations from global; 1: MFMA (2..32 tokens, tile groups per
// workgroup); 2: dot4 with
// LDS-staged activations; 3: as 2 with 8 units in flight per wave; 4: as 3
// with the activation quantization fused into the prologue; 5: the
// table-lookup comparison variant (one token); 6, 7, 8: the dot4 token-loop
// kernel with V - 4 token slots per unit, for launches whose problems have
// at most V - 4 tokens (one-token problems take the one-slot loop, whose
// LDS layout and stream are those of 3); 9: as 1 with one tile per wave.
template <int V>
__device__ inline void stream_body(const Problem &p, int local)
{
    if constexpr (V >= 6 && V <= 8) {
        if (p.M == 1)
            stream_dot4_tokens<8, 1>(p, local);
        else
            stream_dot4_tokens<8, V - 4>(p, local);
    } else if constexpr (V == 0)
        stream_dot4<4, false>(p, local);
    else if constexpr (V == 1)
        stream_mfma<2, kStreamMfmaTiles>(p, local);
    else if constexpr (V == 9)
        stream_mfma<2, 1>(p, local);
    else if constexpr (V == 2)
        stream_dot4<4, true>(p, local);
    else if constexpr (V == 3)
        stream_dot4<8, true>(p, local);
    else if constexpr (V == 4)
        stream_dot4<8, true, true>(p, local);
    else
        stream_dot4<8, true, false, true>(p, local);
}

template <int V>
__global__ __launch_bounds__(kThreads) void stream_single_kernel(Problem p)
{
    stream_body<V>(p, blockIdx.x);
}

template <int V>
__global__ __launch_bounds__(kThreads) void stream_group_kernel(const Problem *__restrict__ probs,
                                                                const uint2 *__restrict__ item_map)
{
    const uint2 it = item_map[blockIdx.x];
    if (it.x == 0xFFFFFFFFu) return;
    stream_body<V>(probs[it.x], (int)it.y);
}

template <int V>
__global__ __launch_bounds__(kThreads) void stream_multi_kernel(ProblemSet ps)
{
    const int i = multi_index(ps, blockIdx.x);
    stream_body<V>(ps.p[i], (int)blockIdx.x - ps.begin[i]);
}

}  // namespace

hipError_t launch_stream_multi(const ProblemSet &ps, int variant, int lds_bytes, hipStream_t s)
{
    const dim3 grid((unsigned)ps.begin[ps.count]), block(kThreads);
    const unsigned lds = (variant >= 2 && variant <= 8) ? (unsigned)lds_bytes : 0u;
    switch (variant) {
    case 0: hipLaunchKernelGGL(stream_multi_kernel<0>, grid, block, 0, s, ps); break;
    case 1: hipLaunchKernelGGL(stream_multi_kernel<1>, grid, block, 0, s, ps); break;
    case 9: hipLaunchKernelGGL(stream_multi_kernel<9>, grid, block, 0, s, ps); break;
    case 2: hipLaunchKernelGGL(stream_multi_kernel<2>, grid, block, lds, s, ps); break;
    case 5: hipLaunchKernelGGL(stream_multi_kernel<5>, grid, block, lds, s, ps); break;
    case 6: hipLaunchKernelGGL(stream_multi_kernel<6>, grid, block, lds, s, ps); break;
    case 7: hipLaunchKernelGGL(stream_multi_kernel<7>, grid, block, lds, s, ps); break;
    case 8: hipLaunchKernelGGL(stream_multi_kernel<8>, grid, block, lds, s, ps); break;
    default: hipLaunchKernelGGL(stream_multi_kernel<3>, grid, block, lds, s, ps); break;
    }
    return hipGetLastError();
}

hipError_t launch_stream_single(const Problem &p, int variant, hipStream_t s)
{
    // the MFMA variants' work items are tile groups (p.ntt of them)
    const int64_t tiles = (variant == 1 || variant == 9) ? (int64_t)p.ntt : (int64_t)p.NT;
    const dim3 grid((unsigned)(tiles * p.ks)), block(kThreads);
    const unsigned slot = variant >= 6 ? 64u * (unsigned)(variant - 4) : 64u;
    const unsigned lds =
        (variant >= 2 && variant <= 8) ? (variant == 5 ? kLutUnitBytes : slot) * (unsigned)p.upsplit : 0u;
    switch (variant) {
    case 0: hipLaunchKernelGGL(stream_single_kernel<0>, grid, block, 0, s, p); break;
    case 1: hipLaunchKernelGGL(stream_single_kernel<1>, grid, block, 0, s, p); break;
    case 9: hipLaunchKernelGGL(stream_single_kernel<9>, grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL(stream_single_kernel<2>, grid, block, lds, s, p); break;
    case 3: hipLaunchKernelGGL(stream_single_kernel<3>, grid, block, lds, s, p); break;
    case 5: hipLaunchKernelGGL(stream_single_kernel<5>, grid, block, lds, s, p); break;
    case 6: hipLaunchKernelGGL(stream_single_kernel<6>, grid, block, lds, s, p); break;
    case 7: hipLaunchKernelGGL(stream_single_kernel<7>, grid, block, lds, s, p); break;
    case 8: hipLaunchKernelGGL(stream_single_kernel<8>, grid, block, lds, s, p); break;
    default: hipLaunchKernelGGL(stream_single_kernel<4>, grid, block, lds, s, p); break;
    }
    return hipGetLastError();
}

hipError_t launch_stream_group(const Problem *probs, const uint2 *item_map, int n_items,
                               int variant, int lds_bytes, hipStream_t s)
{
    const dim3 grid((unsigned)n_items), block(kThreads);
    const unsigned lds = (variant >= 2 && variant <= 8) ? (unsigned)lds_bytes : 0u;
    switch (variant) {
    case 0: hipLaunchKernelGGL(stream_group_kernel<0>, grid, block, 0, s, probs, item_map); break;
    case 1: hipLaunchKernelGGL(stream_group_kernel<1>, grid, block, 0, s, probs, item_map); break;
    case 9: hipLaunchKernelGGL(stream_group_kernel<9>, grid, block, 0, s, probs, item_map); break;
    case 2: hipLaunchKernelGGL(stream_group_kernel<2>, grid, block, lds, s, probs, item_map); break;
    case 3: hipLaunchKernelGGL(stream_group_kernel<3>, grid, block, lds, s, probs, item_map); break;
    case 5: hipLaunchKernelGGL(stream_group_kernel<5>, grid, block, lds, s, probs, item_map); break;
    case 6: hipLaunchKernelGGL(stream_group_kernel<6>, grid, block, lds, s, probs, item_map); break;
    case 7: hipLaunchKernelGGL(stream_group_kernel<7>, grid, block, lds, s, probs, item_map); break;
    case 8: hipLaunchKernelGGL(stream_group_kernel<8>, grid, block, lds, s, probs, item_map); break;
    default: hipLaunchKernelGGL(stream_group_kernel<4>, grid, block, lds, s, probs, item_map); break;
    }
    return hipGetLastError();
}

}  // namespace bl
