// Streaming contraction for small token counts (decode): M = 1 and 2 with
// packed int8 dot products, 3 <= M <= 32 with int8 matrix instructions (the
// split point is a host-side setting), and, for launches of few tiles (the
// matrices of one decode layer), wide workgroups of eight waves per tile
// that may also cast their own input row.
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
// workgroup owns one item (the dot4 kernels; the MFMA stream takes groups of
// tiles, the wide kernels 512 threads per item); its four waves take every
// fourth 64-code unit of the split, so together they stream 4 KiB of
// contiguous packed weights per step.  Each lane loads one 16-byte slot of the unit's 1 KiB block: words
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
#include "quant_row.hpp"

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
// the dot4 kernels run (dynamic LDS, 64 bytes per token slot per unit).
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

// The activations of the workgroup's K range are staged once in LDS and
// read with broadcast LDS reads (2 distinct 16-byte addresses per half
// wave) instead of two 16-byte global loads per lane per unit, which would
// triple the vector-memory instructions of the stream.
// LUT: the table-lookup variant above instead of dot products.
template <int UNROLL, bool LUT = false>
__device__ void stream_dot4(const Problem &p, int local)
{
    __shared__ int red[kWaves][64];
    const int tile = local / p.ks, split = local - tile * p.ks;
    const int u0 = split * p.upsplit;
    const int u1 = min(p.KU, u0 + p.upsplit);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 5;
    const BL_GLOBAL v4u *blk = gload_ptr<v4u>(p.P + (int64_t)tile * p.KU * kBlockBytes) + lane;
    if constexpr (LUT) {
        build_lut(p, u0, u1);
    } else {
        const BL_GLOBAL v4i *src = gload_ptr<v4i>(p.Q + 64 * u0);
        stage_chunks(4 * (u1 - u0), [&](int i) { return src[i]; });
    }
    __syncthreads();
    auto finish = [&](int n, int32_t fields, float gamma) { finish_output(p, gamma, 0, n, fields); };
    // activation bytes 64*u + 16*g (+32 for the second half) of unit u
    auto qload = [&](int u, int off) -> v4i {
        return *reinterpret_cast<const v4i *>(stream_q_lds + 64 * (u - u0) + 16 * g + off);
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

// One token over few tiles (the matrices of one decode layer, launched on
// their own): the launch is too small to be bound by bandwidth, and its time
// is the chain of memory round trips of one workgroup.  W waves
// (kWideWaves) share one 64-row tile and K range; wave w takes units u0 + w, u0 + w + W,
// ... (at most kWideUnits) and requests all of them before the activations
// are staged, so the weight and activation round trips overlap and nothing
// waits on memory after the barrier.  The waves' sums meet in LDS; where
// W * kWideUnits units cover K there is no K split and no hand-off through
// memory, otherwise splits work as in the other streaming kernels.
// CAST >= 0: the workgroup casts the token row itself (quant_row.hpp mode
// CAST, input ci) into LDS, the whole row (byte k = code k), after its
// weight loads are requested; the epilogue takes the row's absmax and code
// sum from that cast.
template <int W, int CAST = -1>
__device__ void stream_dot4_wide(const Problem &p, int local, const CastIn *ci = nullptr)
{
    constexpr int kThr = 64 * W;
    __shared__ int red[W][64];
    const int tile = local / p.ks, split = local - tile * p.ks;
    const int u0 = split * p.upsplit;
    const int u1 = min(p.KU, u0 + p.upsplit);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, g = lane >> 5;
    const BL_GLOBAL v4u *blk = gload_ptr<v4u>(p.P + (int64_t)tile * p.KU * kBlockBytes) + lane;
    // units of this wave (the host keeps the split within W * kWideUnits)
    const int nu = u1 - u0 > wave ? (u1 - u0 - wave + W - 1) / W : 0;
    v4u w[kWideUnits];
#pragma unroll
    for (int j = 0; j < kWideUnits; ++j)
        if (j < nu) w[j] = load_packed(blk + (int64_t)(u0 + wave + W * j) * 64);
    RowScale rsc{0.0f, 0};
    int lds_u0 = u0;  // unit staged at LDS byte 0
    if constexpr (CAST >= 0) {
        const LdsDest dst{stream_q_lds, p.KU};
        rsc = quant_row<W, CAST>(ci->x, ci->K, dst, ci->aux, ci->eps, ci->res, blockIdx.x == 0 ? ci->xo : nullptr);
        lds_u0 = 0;
    } else {
        const int n = 4 * (u1 - u0);  // 16-byte chunks of the range
        const BL_GLOBAL v4i *src = gload_ptr<v4i>(p.Q + 64 * u0);
        v4i *dst = reinterpret_cast<v4i *>(stream_q_lds);
        for (int i = threadIdx.x; i < n; i += kThr) dst[i] = src[i];
    }
    __syncthreads();
    int acc0 = 0, acc1 = 0;  // rows r and 32 + r of the tile
#pragma unroll
    for (int j = 0; j < kWideUnits; ++j)
        if (j < nu) {
            const int8_t *q = stream_q_lds + 64 * (u0 - lds_u0 + wave + W * j) + 16 * g;
            const v4i qa = *reinterpret_cast<const v4i *>(q);
            const v4i qb = *reinterpret_cast<const v4i *>(q + 32);
            acc0 = dot16(w[j].x, qa, acc0);
            acc0 = dot16(w[j].y, qb, acc0);
            acc1 = dot16(w[j].z, qa, acc1);
            acc1 = dot16(w[j].w, qb, acc1);
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
    auto finish = [&](int32_t fields) {
        if constexpr (CAST >= 0)
            finish_output_with(p, gamma, 0, n, fields, rsc.sum, rsc.a);
        else
            finish_output(p, gamma, 0, n, fields);
    };
    int total = 0;
    if (t < 64) {
#pragma unroll
        for (int i = 0; i < W; ++i) total += red[i][t];
    }
    if (p.ks == 1) {
        if (t < 64 && n < p.N) finish(total);
        return;
    }
    const int64_t ldp = (int64_t)p.NT * 64;  // partial row stride
    if (t < 64) put_partial(p.acc_ws + ((int64_t)split * p.M * ldp + n), total);
    if (!arrive_last(p, tile)) return;
    const int64_t off[1] = {n};
    const bool ok[1] = {t < 64 && n < p.N};
    int32_t sum[1];
    sum_partials<1>(p.acc_ws, off, ok, (int64_t)p.M * ldp, p.ks, sum);
    if (ok[0]) finish(sum[0]);
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
// of the MFMAs through a two-slot register ring (branch-free: activation
// unit indices clamp to the range end, and surplus units read zero weights
// through an empty buffer resource, which add nothing).
// ALDS: the activations of the workgroup's K range are staged once in LDS
// (row-major, at most 16 tokens): token m's 64 bytes of unit u at byte
// ((u - u0) * M + m) * kTokStride; each wave reads its A operands with
// ds_read_b128 (lanes of rows past M read row M-1, whose sums in those
// rows are never stored) instead of two global loads per unit.
constexpr int kTokStride = 80;  // 64 bytes + 16: 16 rows at one column hit distinct bank groups

// Stages units [0, n_units) of the K range at q (the first M token rows,
// row stride ldq) row-major into LDS: token m's 64 bytes of unit uu at
// (uu * M + m) * kTokStride.  Thread t always copies part t % 4 of token
// (t / 4) % M, for every (THR / (4 M))-th unit from t / (4 M) on -- so no
// thread divides per chunk -- with up to UNR loads in flight before its
// first LDS store; threads past the last whole pass of 4 M copy nothing.
template <int THR, int UNR>
__device__ __forceinline__ void stage_rows(const BL_GLOBAL int8_t *q, int64_t ldq, int M, int n_units)
{
    const int cpu = 4 * M, per = THR / cpu;
    const int slot = threadIdx.x % cpu, uo = threadIdx.x / cpu;
    if (uo >= per) return;
    const BL_GLOBAL int8_t *src = q + (int64_t)(slot >> 2) * ldq + 16 * (slot & 3);
    int8_t *dst = stream_q_lds + (slot >> 2) * kTokStride + 16 * (slot & 3);
    const int ustride = M * kTokStride;
    for (int ub = uo; ub < n_units; ub += UNR * per) {
        v4i v[UNR];
#pragma unroll
        for (int k = 0; k < UNR; ++k)
            if (ub + k * per < n_units) v[k] = *reinterpret_cast<const BL_GLOBAL v4i *>(src + 64 * (ub + k * per));
#pragma unroll
        for (int k = 0; k < UNR; ++k)
            if (ub + k * per < n_units) *reinterpret_cast<v4i *>(dst + (ub + k * per) * ustride) = v[k];
    }
}
template <int UNROLL, int TPW, bool ALDS = false>
__device__ __forceinline__ void stream_mfma(const Problem &p, int local)
{
    const int ks = uni(p.ks), KU = uni(p.KU), NT = uni(p.NT), M = uni(p.M);
    const int grp = local / ks, split = local - grp * ks;
    const int u0 = split * uni(p.upsplit);
    const int u1 = min(KU, u0 + uni(p.upsplit));
    const int n_units = u1 - u0;
    const int wave = uni(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, g = lane >> 5, r = lane & 31;
    const int tile0 = 4 * TPW * grp + TPW * wave;
    // Each tile's units of the range are read through a buffer resource of
    // exactly those bytes, and a unit past the range through a resource of
    // none, which returns the all-zero word: zero fields add nothing, so the
    // loop needs no selects.  Tiles past NT stream tile NT-1 (valid memory);
    // their sums are dropped.
    __amdgpu_buffer_rsrc_t rw[TPW];
    const __amdgpu_buffer_rsrc_t rz = buffer_rsrc(uni(p.P), 0);
#pragma unroll
    for (int t = 0; t < TPW; ++t)
        rw[t] = buffer_rsrc(uni(p.P) + ((int64_t)min(tile0 + t, NT - 1) * KU + u0) * kBlockBytes, n_units * kBlockBytes);
    const int woff = 16 * lane;
    // A operand of unit u, half h: fragment-ordered activations hold it as one
    // contiguous 1 KiB block (16 bytes per lane); row-major activations give
    // each lane 16 bytes of its token row.  Lanes of rows past M read row
    // M-1: an A row only feeds the same output row, which is never stored.
    const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(uni(p.Q), -1);
    const int qtiled = uni(p.qtiled);
    const int ldq = uni((int)p.ldq);
    const int qlane = qtiled ? 16 * lane : min(r, M - 1) * ldq + 16 * g;
    const int ustride = qtiled ? 2048 : 64, hoff = qtiled ? 1024 : 32;
    // the tokens' row sums and rescale factors, fetched now so that their
    // latency hides under the stream (read per output element at the end)
    __shared__ int s_rowsum[kStreamMaxTokens];
    __shared__ float s_scale[kStreamMaxTokens];
    if (threadIdx.x < M) {
        s_rowsum[threadIdx.x] = gload_ptr<int32_t>(p.rowsum)[threadIdx.x];
        s_scale[threadIdx.x] = token_scale(*p.gamma, gload_ptr<float>(p.absmax)[threadIdx.x]);
    }

    const int groups = (n_units + UNROLL - 1) / UNROLL;
    int a_lane = 0;  // this lane's byte offset within a staged unit (ALDS)
    v4u w[2][UNROLL][TPW];
    v4i qa[2][UNROLL], qb[2][UNROLL];
    auto load_group = [&](int slot, int i) {
#pragma unroll
        for (int j = 0; j < UNROLL; ++j) {
            const int ur = UNROLL * i + j;  // unit within the range
#pragma unroll
            for (int t = 0; t < TPW; ++t)
                w[slot][j][t] = __builtin_amdgcn_raw_buffer_load_b128(ur < n_units ? rw[t] : rz, woff,
                                                                      ur * kBlockBytes, kNonTemporal);
            if constexpr (!ALDS) {
                const int uoff = ustride * (u0 + min(ur, n_units - 1));
                qa[slot][j] = (v4i)__builtin_amdgcn_raw_buffer_load_b128(rq, qlane, uoff, 0);
                qb[slot][j] = (v4i)__builtin_amdgcn_raw_buffer_load_b128(rq, qlane + hoff, uoff, 0);
            }
        }
    };
    // the first group's packed weights are requested before the activations
    // are staged (they do not depend on them): the two round trips overlap
    if constexpr (ALDS) load_group(0, 0);
    if constexpr (ALDS) {
        stage_rows<kThreads, 8>(gload_ptr<int8_t>(p.Q) + 64 * u0, p.ldq, M, n_units);
        a_lane = min(r, M - 1) * kTokStride + 16 * g;
        __syncthreads();
    }
    v16i acc[TPW][2];
#pragma unroll
    for (int t = 0; t < TPW; ++t) acc[t][0] = acc[t][1] = (v16i){};
    // Word x of a lane's slot holds rows 0..31 of the unit's first half of
    // codes, y the same rows' second half, z and w rows 32..63; the pairs
    // (x, y) and (z, w) share the unpack's 64-bit shifts.  Consecutive
    // updates of one accumulator are two MFMAs apart, so the matrix pipe
    // never waits on its own previous result.
    auto run_group = [&](int slot, int i) {
#pragma unroll
        for (int j = 0; j < UNROLL; ++j) {
            v4i a0, a1;
            if constexpr (ALDS) {
                // units past the range read any staged unit: their weights are zero
                const int uu = min(UNROLL * i + j, n_units - 1);
                const int8_t *q = stream_q_lds + a_lane + uu * M * kTokStride;
                a0 = *reinterpret_cast<const v4i *>(q);
                a1 = *reinterpret_cast<const v4i *>(q + 32);
            } else {
                a0 = qa[slot][j];
                a1 = qb[slot][j];
            }
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                const v4u wj = w[slot][j][t];
                v4i bx, by, bz, bw;
                planes2(wj.x, wj.y, bx, by);
                planes2(wj.z, wj.w, bz, bw);
                acc[t][0] = mfma_i8(a0, bx, acc[t][0]);
                acc[t][1] = mfma_i8(a0, bz, acc[t][1]);
                acc[t][0] = mfma_i8(a1, by, acc[t][0]);
                acc[t][1] = mfma_i8(a1, bw, acc[t][1]);
            }
        }
    };
    if constexpr (!ALDS) load_group(0, 0);
    // each group's loads are issued before the previous group's MFMAs (the
    // barriers keep the scheduler from sinking them behind the MFMAs, which
    // would shorten the stream's lookahead)
    int i = 0;
    for (; i + 2 <= groups; i += 2) {
        load_group(1, i + 1);
        __builtin_amdgcn_sched_barrier(0);
        run_group(0, i);
        __builtin_amdgcn_sched_barrier(0);
        load_group(0, i + 2);
        __builtin_amdgcn_sched_barrier(0);
        run_group(1, i + 1);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (i < groups) run_group(0, i);

    // element e of lane l is token 8*(e/4) + 4*(l/32) + e%4, row 32*s + l%32
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
                        finish_output_scaled(p, m, n, acc[t][s2][e], s_rowsum[m], s_scale[m]);
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
            if (ok[r]) finish_output_scaled(p, mm[r], nn[r], sums[r], s_rowsum[mm[r]], s_scale[mm[r]]);
    }
}

// 2..16 tokens over few tiles: the wide kernel's decomposition (W waves per
// 64-row tile and K range, every wave's units requested before the staging)
// with the matrix-instruction stream.  The activations of the range are
// staged row-major as in variant 10 (token m's 64 bytes of unit u at
// ((u - u0) * M + m) * kTokStride); each wave
// accumulates its units into two 32 x 32 tiles (rows 0..31 and 32..63 of
// the weight tile), and the waves' sums meet in LDS, in the space the
// staged activations held: eight slots, word (slot * M + m) * 64 + row for
// token m.
template <int W>
__device__ void stream_mfma_wide(const Problem &p, int local)
{
    constexpr int kThr = 64 * W;
    const int tile = local / p.ks, split = local - tile * p.ks;
    const int u0 = split * p.upsplit;
    const int u1 = min(p.KU, u0 + p.upsplit);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, g = lane >> 5, r = lane & 31;
    const int M = p.M;
    const BL_GLOBAL v4u *blk = gload_ptr<v4u>(p.P + (int64_t)tile * p.KU * kBlockBytes) + lane;
    const int nu = u1 - u0 > wave ? (u1 - u0 - wave + W - 1) / W : 0;
    v4u w[kWideUnits];
#pragma unroll
    for (int j = 0; j < kWideUnits; ++j)
        if (j < nu) w[j] = load_packed(blk + (int64_t)(u0 + wave + W * j) * 64);
    __shared__ int s_rowsum[kStreamMaxTokens];
    __shared__ float s_scale[kStreamMaxTokens];
    if (threadIdx.x < M) {
        s_rowsum[threadIdx.x] = gload_ptr<int32_t>(p.rowsum)[threadIdx.x];
        s_scale[threadIdx.x] = token_scale(*p.gamma, gload_ptr<float>(p.absmax)[threadIdx.x]);
    }
    const int n_units = u1 - u0;
    stage_rows<kThr, 4>(gload_ptr<int8_t>(p.Q) + 64 * u0, p.ldq, M, n_units);
    __syncthreads();
    // lanes of rows past M read row M-1: an A row only feeds the same output
    // row, which is never stored
    const int a_lane = min(r, M - 1) * kTokStride + 16 * g;
    v16i acc0 = (v16i){}, acc1 = (v16i){};
#pragma unroll
    for (int j = 0; j < kWideUnits; ++j)
        if (j < nu) {
            const int8_t *a = stream_q_lds + a_lane + (wave + W * j) * M * kTokStride;
            const v4i a0 = *reinterpret_cast<const v4i *>(a);
            const v4i a1 = *reinterpret_cast<const v4i *>(a + 32);
            v4i bx, by, bz, bw;
            planes2(w[j].x, w[j].y, bx, by);
            planes2(w[j].z, w[j].w, bz, bw);
            acc0 = mfma_i8(a0, bx, acc0);
            acc1 = mfma_i8(a0, bz, acc1);
            acc0 = mfma_i8(a1, by, acc0);
            acc1 = mfma_i8(a1, bw, acc1);
        }
    __syncthreads();  // the staged activations are no longer read
    // element e of lane l is token 8*(e/4) + 4*(l/32) + e%4, row 32*s + l%32;
    // at most 16 tokens: elements 0..7.  Eight slots of M * 64 sums: waves
    // 0..7 store theirs, then waves 8..15 (when W = 16) add theirs to slot
    // wave - 8, each lane to the words it stored itself.
    int *red = reinterpret_cast<int *>(stream_q_lds);
    constexpr int kSlots = 8;
    auto put = [&](bool add) {
        const int slot = wave % kSlots;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int m = 8 * (e >> 2) + 4 * g + (e & 3);
            if (m < M) {
                int *d = red + (slot * M + m) * 64 + r;
                d[0] = add ? d[0] + acc0[e] : acc0[e];
                d[32] = add ? d[32] + acc1[e] : acc1[e];
            }
        }
    };
    if (wave < kSlots) put(false);
    if constexpr (W > kSlots) {
        __syncthreads();
        if (wave >= kSlots) put(true);
    }
    __syncthreads();
    // thread t finishes outputs t + kThr * i: token (t + kThr * i) / 64, row % 64
    constexpr int kR = (16 * 64 + kThr - 1) / kThr;
    int mm[kR], nn[kR], tot[kR];
    bool mine[kR];
#pragma unroll
    for (int i = 0; i < kR; ++i) {
        const int idx = threadIdx.x + kThr * i;
        mm[i] = idx >> 6;
        nn[i] = 64 * tile + (idx & 63);
        mine[i] = mm[i] < M;
        tot[i] = 0;
        if (mine[i]) {
#pragma unroll
            for (int v = 0; v < kSlots; ++v) tot[i] += red[(v * M + mm[i]) * 64 + (idx & 63)];
        }
    }
    if (p.ks == 1) {
#pragma unroll
        for (int i = 0; i < kR; ++i)
            if (mine[i] && nn[i] < p.N) finish_output_scaled(p, mm[i], nn[i], tot[i], s_rowsum[mm[i]], s_scale[mm[i]]);
        return;
    }
    const int64_t ldp = (int64_t)p.NT * 64;  // partial row stride
#pragma unroll
    for (int i = 0; i < kR; ++i)
        if (mine[i]) put_partial(p.acc_ws + (((int64_t)split * M + mm[i]) * ldp + nn[i]), tot[i]);
    if (!arrive_last(p, tile)) return;
    int64_t off[kR];
    bool ok[kR];
#pragma unroll
    for (int i = 0; i < kR; ++i) {
        off[i] = (int64_t)mm[i] * ldp + nn[i];
        ok[i] = mine[i] && nn[i] < p.N;
    }
    int32_t sum[kR];
    sum_partials<kR>(p.acc_ws, off, ok, (int64_t)M * ldp, p.ks, sum);
#pragma unroll
    for (int i = 0; i < kR; ++i)
        if (ok[i]) finish_output_scaled(p, mm[i], nn[i], sum[i], s_rowsum[mm[i]], s_scale[mm[i]]);
}

// Instantiations: 1: MFMA stream (17..32 tokens; two tiles per wave); 3:
// dot4 with LDS-staged activations, 8 units in flight per wave (one token);
// 5: the table-lookup comparison variant (one token); 6: the dot4 token
// loop for launches whose problems have at most two tokens (one-token
// problems take the one-slot loop, whose LDS layout and stream are those
// of 3); 9: as 1 with one tile per wave; 10: the MFMA stream for 3..16
// tokens with LDS-staged activations, one tile per wave, loads four units
// ahead; 12: the one-token wide kernel; 13: the wide kernel's MFMA stream
// for 2..16 tokens (kWideWaves waves per workgroup, both).
template <int V>
__device__ __forceinline__ void stream_body(const Problem &p, int local)
{
    if constexpr (V == 6) {
        if (p.M == 1)
            stream_dot4_tokens<8, 1>(p, local);
        else
            stream_dot4_tokens<8, kDot4MaxTokens>(p, local);
    } else if constexpr (V == 1)
        stream_mfma<2, kStreamMfmaTiles>(p, local);
    else if constexpr (V == 9)
        stream_mfma<2, 1>(p, local);
    else if constexpr (V == 10 || V == 11)
        stream_mfma<4, 1, true>(p, local);
    else if constexpr (V == 12)
        stream_dot4_wide<kWideWaves>(p, local);
    else if constexpr (V == 13)
        stream_mfma_wide<kWideWaves>(p, local);
    else if constexpr (V == 5)
        stream_dot4<8, true>(p, local);
    else
        stream_dot4<8>(p, local);
}

// threads per workgroup of variant V
__host__ __device__ constexpr int stream_threads(int V) { return (V == 12 || V == 13) ? 64 * kWideWaves : kThreads; }

template <int V>
__global__ __launch_bounds__(stream_threads(V)) void stream_single_kernel(Problem p)
{
    stream_body<V>(p, blockIdx.x);
}

template <int V>
__global__ __launch_bounds__(stream_threads(V)) void stream_group_kernel(const Problem *__restrict__ probs,
                                                                const uint2 *__restrict__ item_map)
{
    const uint2 it = item_map[blockIdx.x];
    if (it.x == 0xFFFFFFFFu) return;
    stream_body<V>(probs[it.x], (int)it.y);
}

template <int V>
__global__ __launch_bounds__(stream_threads(V)) void stream_multi_kernel(ProblemSet ps)
{
    const int i = multi_index(ps, blockIdx.x);
    stream_body<V>(ps.p[i], (int)blockIdx.x - ps.begin[i]);
}

// Variant 11: the body of 10 held to 128 VGPRs (four waves per SIMD), so that
// four workgroups share a compute unit where their staged activations fit
// (10 takes 136, three waves per SIMD).
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void stream_single_kernel_w4(Problem p)
{
    stream_body<11>(p, blockIdx.x);
}
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void stream_group_kernel_w4(
    const Problem *__restrict__ probs, const uint2 *__restrict__ item_map)
{
    const uint2 it = item_map[blockIdx.x];
    if (it.x == 0xFFFFFFFFu) return;
    stream_body<11>(probs[it.x], (int)it.y);
}
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void stream_multi_kernel_w4(ProblemSet ps)
{
    const int i = multi_index(ps, blockIdx.x);
    stream_body<11>(ps.p[i], (int)blockIdx.x - ps.begin[i]);
}

// One-token launches that cast their own input: W waves, cast mode MODE.
template <int W, int MODE>
__global__ __launch_bounds__(64 * W) void stream_cast_multi_kernel(ProblemSet ps, CastIn ci)
{
    const int i = multi_index(ps, blockIdx.x);
    stream_dot4_wide<W, MODE>(ps.p[i], (int)blockIdx.x - ps.begin[i], &ci);
}

}  // namespace

hipError_t launch_stream_cast_multi(const ProblemSet &ps, const CastIn &ci, int mode, hipStream_t s)
{
    const dim3 grid((unsigned)ps.begin[ps.count]), block(64 * kWideWaves);
    const unsigned lds = 64u * (unsigned)ps.p[0].KU;  // the whole row's codes
    constexpr int W = kWideWaves;
    switch (mode) {
    case kRmsNorm: hipLaunchKernelGGL((stream_cast_multi_kernel<W, kRmsNorm>), grid, block, lds, s, ps, ci); break;
    case kRelu2Gate: hipLaunchKernelGGL((stream_cast_multi_kernel<W, kRelu2Gate>), grid, block, lds, s, ps, ci); break;
    case kAddRmsNorm: hipLaunchKernelGGL((stream_cast_multi_kernel<W, kAddRmsNorm>), grid, block, lds, s, ps, ci); break;
    default: hipLaunchKernelGGL((stream_cast_multi_kernel<W, kPlain>), grid, block, lds, s, ps, ci); break;
    }
    return hipGetLastError();
}

// one case per instantiation; unknown values take 3
#define BL_STREAM_CASES(KERNEL, LDS, ...)                                                   \
    switch (variant) {                                                                     \
    case 1: hipLaunchKernelGGL(KERNEL<1>, grid, block, 0, s, __VA_ARGS__); break;          \
    case 9: hipLaunchKernelGGL(KERNEL<9>, grid, block, 0, s, __VA_ARGS__); break;          \
    case 10: hipLaunchKernelGGL(KERNEL<10>, grid, block, LDS, s, __VA_ARGS__); break;      \
    case 11: hipLaunchKernelGGL(KERNEL##_w4, grid, block, LDS, s, __VA_ARGS__); break;     \
    case 5: hipLaunchKernelGGL(KERNEL<5>, grid, block, LDS, s, __VA_ARGS__); break;        \
    case 6: hipLaunchKernelGGL(KERNEL<6>, grid, block, LDS, s, __VA_ARGS__); break;        \
    case 12: hipLaunchKernelGGL(KERNEL<12>, grid, block, LDS, s, __VA_ARGS__); break;      \
    case 13: hipLaunchKernelGGL(KERNEL<13>, grid, block, LDS, s, __VA_ARGS__); break;      \
    default: hipLaunchKernelGGL(KERNEL<3>, grid, block, LDS, s, __VA_ARGS__); break;       \
    }

hipError_t launch_stream_multi(const ProblemSet &ps, int variant, int lds_bytes, hipStream_t s)
{
    const dim3 grid((unsigned)ps.begin[ps.count]), block(stream_threads(variant));
    BL_STREAM_CASES(stream_multi_kernel, (unsigned)lds_bytes, ps)
    return hipGetLastError();
}

hipError_t launch_stream_single(const Problem &p, int variant, hipStream_t s)
{
    // the MFMA variants' work items are tile groups (p.ntt of them)
    const int64_t tiles = (variant == 1 || variant == 9 || variant == 10 || variant == 11) ? (int64_t)p.ntt : (int64_t)p.NT;
    const dim3 grid((unsigned)(tiles * p.ks)), block(stream_threads(variant));
    const unsigned slot = variant == 6 ? 64u * kDot4MaxTokens : 64u;
    unsigned lds = (variant == 10 || variant == 11) ? (unsigned)(kTokStride * p.M * p.upsplit + 16)
                                 : (variant == 5 ? kLutUnitBytes : slot) * (unsigned)p.upsplit;
    if (variant == 13) {
        // staged activations, then the waves' sums (eight slots) in the same space
        const unsigned red = (unsigned)(8 * p.M * 256);
        lds = (unsigned)(kTokStride * p.M * p.upsplit + 16);
        lds = lds > red ? lds : red;
    }
    BL_STREAM_CASES(stream_single_kernel, lds, p)
    return hipGetLastError();
}

hipError_t launch_stream_group(const Problem *probs, const uint2 *item_map, int n_items,
                               int variant, int lds_bytes, hipStream_t s)
{
    const dim3 grid((unsigned)n_items), block(stream_threads(variant));
    BL_STREAM_CASES(stream_group_kernel, (unsigned)lds_bytes, probs, item_map)
    return hipGetLastError();
}

#undef BL_STREAM_CASES

}  // namespace bl
