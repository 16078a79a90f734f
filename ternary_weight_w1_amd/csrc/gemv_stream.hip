// Streaming contraction for small token counts (decode): M = 1 with packed
// int8 dot products, 2 <= M <= 32 with int8 matrix instructions.
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
//                 epilogue subtracts once.
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

// QLDS: read the activations with broadcast LDS reads (2 distinct 16-byte
// addresses per half wave) instead of two 16-byte global loads per lane per
// unit, which would triple the vector-memory instructions of the stream.
// FUSED: the activations are quantized in the prologue (implies QLDS).
template <int UNROLL, bool QLDS, bool FUSED = false>
__device__ void stream_dot4(const Problem &p, int local)
{
    static_assert(!FUSED || QLDS, "the fused prologue writes the LDS activations");
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
    } else if constexpr (QLDS) {
        const BL_GLOBAL v4i *src = gload_ptr<v4i>(p.Q + 64 * u0);
        v4i *dst = reinterpret_cast<v4i *>(stream_q_lds);
        for (int i = threadIdx.x; i < 4 * (u1 - u0); i += kThreads) dst[i] = src[i];
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
    for (; u < u1; u += kWaves) {
        const v4u w = load_packed(blk + (int64_t)u * 64);
        const v4i qa = qload(u, 0);
        const v4i qb = qload(u, 32);
        acc0 = dot16(w.x, qa, acc0);
        acc0 = dot16(w.y, qb, acc0);
        acc1 = dot16(w.z, qa, acc1);
        acc1 = dot16(w.w, qb, acc1);
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
    if (t < 64) gstore_ptr<int32_t>(p.acc_ws)[(int64_t)split * p.M * ldp + n] = total;
    if (!arrive_last(p, tile)) return;
    if (t < 64 && n < p.N) {
        int sum = 0;
        for (int j = 0; j < p.ks; ++j) sum += gload_ptr<int32_t>(p.acc_ws)[(int64_t)j * p.M * ldp + n];
        finish(n, sum, gamma);
    }
}

template <int UNROLL>
__device__ void stream_mfma(const Problem &p, int local)
{
    // per wave, per 32-row half s, per accumulator element e, per lane
    __shared__ int red[kWaves][2][16][64];
    const int tile = local / p.ks, split = local - tile * p.ks;
    const int u0 = split * p.upsplit;
    const int u1 = min(p.KU, u0 + p.upsplit);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 5, r = lane & 31;
    const BL_GLOBAL v4u *blk = gload_ptr<v4u>(p.P + (int64_t)tile * p.KU * kBlockBytes) + lane;
    const bool rv = r < p.M;
    const BL_GLOBAL int8_t *qrow = gload_ptr<int8_t>(p.Q + (int64_t)(rv ? r : 0) * p.ldq + 16 * g);
    const v4i zero = {0, 0, 0, 0};

    v16i acc0 = {}, acc1 = {};
    int u = u0 + wave;
    for (; u + kWaves * (UNROLL - 1) < u1; u += kWaves * UNROLL) {
        v4u w[UNROLL];
        v4i qa[UNROLL], qb[UNROLL];
#pragma unroll
        for (int j = 0; j < UNROLL; ++j) w[j] = load_packed(blk + (int64_t)(u + kWaves * j) * 64);
#pragma unroll
        for (int j = 0; j < UNROLL; ++j) {
            const BL_GLOBAL int8_t *qu = qrow + 64 * (u + kWaves * j);
            qa[j] = rv ? *reinterpret_cast<const BL_GLOBAL v4i *>(qu) : zero;
            qb[j] = rv ? *reinterpret_cast<const BL_GLOBAL v4i *>(qu + 32) : zero;
        }
#pragma unroll
        for (int j = 0; j < UNROLL; ++j) {
            acc0 = mfma_i8(qa[j], planes(w[j].x), acc0);
            acc0 = mfma_i8(qb[j], planes(w[j].y), acc0);
            acc1 = mfma_i8(qa[j], planes(w[j].z), acc1);
            acc1 = mfma_i8(qb[j], planes(w[j].w), acc1);
        }
    }
    for (; u < u1; u += kWaves) {
        const v4u w = load_packed(blk + (int64_t)u * 64);
        const BL_GLOBAL int8_t *qu = qrow + 64 * u;
        const v4i qa = rv ? *reinterpret_cast<const BL_GLOBAL v4i *>(qu) : zero;
        const v4i qb = rv ? *reinterpret_cast<const BL_GLOBAL v4i *>(qu + 32) : zero;
        acc0 = mfma_i8(qa, planes(w.x), acc0);
        acc0 = mfma_i8(qb, planes(w.y), acc0);
        acc1 = mfma_i8(qa, planes(w.z), acc1);
        acc1 = mfma_i8(qb, planes(w.w), acc1);
    }
    // element e of lane l is token 8*(e/4) + 4*(l/32) + e%4, row 32*s + l%32;
    // only element groups that hold real tokens are exchanged
    const int eg = (p.M + 7) >> 3;  // 1..4
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        if ((e >> 2) < eg) {
            red[wave][0][e][lane] = acc0[e];
            red[wave][1][e][lane] = acc1[e];
        }
    }
    __syncthreads();

    const float gamma = *p.gamma;
    const int64_t ldp = (int64_t)p.NT * 64;
    const int entries = 2 * 4 * eg * 64;
    int *flat = &red[0][0][0][0];
    constexpr int kWaveStride = 2 * 16 * 64;
    for (int idx = threadIdx.x; idx < entries; idx += kThreads) {
        const int s = idx / (4 * eg * 64);
        const int e = (idx >> 6) % (4 * eg);
        const int l = idx & 63;
        const int m = 8 * (e >> 2) + 4 * (l >> 5) + (e & 3);
        const int n = 64 * tile + 32 * s + (l & 31);
        if (m >= p.M || n >= p.N) continue;
        const int off = (s * 16 + e) * 64 + l;
        const int total = flat[off] + flat[kWaveStride + off] + flat[2 * kWaveStride + off] +
                          flat[3 * kWaveStride + off];
        if (p.ks == 1)
            finish_output(p, gamma, m, n, total);
        else
            gstore_ptr<int32_t>(p.acc_ws)[((int64_t)split * p.M + m) * ldp + n] = total;
    }
    if (p.ks == 1) return;
    if (!arrive_last(p, tile)) return;
    for (int idx = threadIdx.x; idx < p.M * 64; idx += kThreads) {
        const int m = idx >> 6;
        const int n = 64 * tile + (idx & 63);
        if (n >= p.N) continue;
        int sum = 0;
        for (int j = 0; j < p.ks; ++j) sum += gload_ptr<int32_t>(p.acc_ws)[((int64_t)j * p.M + m) * ldp + n];
        finish_output(p, gamma, m, n, sum);
    }
}

// 0: dot4, activations from global; 1: MFMA (2..32 tokens); 2: dot4 with
// LDS-staged activations; 3: as 2 with 8 units in flight per wave; 4: as 3
// with the activation quantization fused into the prologue.
template <int V>
__device__ inline void stream_body(const Problem &p, int local)
{
    if constexpr (V == 0)
        stream_dot4<4, false>(p, local);
    else if constexpr (V == 1)
        stream_mfma<2>(p, local);
    else if constexpr (V == 2)
        stream_dot4<4, true>(p, local);
    else if constexpr (V == 3)
        stream_dot4<8, true>(p, local);
    else
        stream_dot4<8, true, true>(p, local);
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

}  // namespace

hipError_t launch_stream_single(const Problem &p, int variant, hipStream_t s)
{
    const dim3 grid((unsigned)(p.NT * p.ks)), block(kThreads);
    const unsigned lds = variant >= 2 ? 64u * (unsigned)p.upsplit : 0u;
    switch (variant) {
    case 0: hipLaunchKernelGGL(stream_single_kernel<0>, grid, block, 0, s, p); break;
    case 1: hipLaunchKernelGGL(stream_single_kernel<1>, grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL(stream_single_kernel<2>, grid, block, lds, s, p); break;
    case 3: hipLaunchKernelGGL(stream_single_kernel<3>, grid, block, lds, s, p); break;
    default: hipLaunchKernelGGL(stream_single_kernel<4>, grid, block, lds, s, p); break;
    }
    return hipGetLastError();
}

hipError_t launch_stream_group(const Problem *probs, const uint2 *item_map, int n_items,
                               int variant, int lds_bytes, hipStream_t s)
{
    const dim3 grid((unsigned)n_items), block(kThreads);
    const unsigned lds = variant >= 2 ? (unsigned)lds_bytes : 0u;
    switch (variant) {
    case 0: hipLaunchKernelGGL(stream_group_kernel<0>, grid, block, 0, s, probs, item_map); break;
    case 1: hipLaunchKernelGGL(stream_group_kernel<1>, grid, block, 0, s, probs, item_map); break;
    case 2: hipLaunchKernelGGL(stream_group_kernel<2>, grid, block, lds, s, probs, item_map); break;
    case 3: hipLaunchKernelGGL(stream_group_kernel<3>, grid, block, lds, s, probs, item_map); break;
    default: hipLaunchKernelGGL(stream_group_kernel<4>, grid, block, lds, s, probs, item_map); break;
    }
    return hipGetLastError();
}

}  // namespace bl
