// Per-token absmax int8 activation quantization for gfx950.
//
// anthology note-168 on arXiv 2402.17764, "What it does": BitLinear's
// activations are 8-bit.  Reading implemented (the pages print no formula):
// a = max(1e-5, max_k |x_k|) for each token, s = 127 / a (one fp32 IEEE
// division per token), q_k = clamp(rint(x_k * s), -127, 127).  The row sum
// of q is produced too: the contraction kernels multiply by (code + 1)
// fields and subtract it once per output.
//
// One 256-thread workgroup per token: the row is read with 16-byte loads
// (kept in registers up to 8192 values), |x| is reduced with wave
// butterflies and then across the four waves through LDS, and the codes are
// written 16 per 16-byte store.  The max is order-free and the row sum is an
// integer sum, so both are exact whatever the reduction order.
#include "common.hpp"

namespace bl {
namespace {

constexpr int kThreads = 256;
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

__device__ inline float block_max(float v, float *lds)
{
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    const int wave = threadIdx.x >> 6;
    __syncthreads();  // lds may still be read by a previous reduction
    if ((threadIdx.x & 63) == 0) lds[wave] = v;
    __syncthreads();
    return fmaxf(fmaxf(lds[0], lds[1]), fmaxf(lds[2], lds[3]));
}

__device__ inline int block_sum_i32(int v, int *lds)
{
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) lds[wave] = v;
    __syncthreads();
    return lds[0] + lds[1] + lds[2] + lds[3];
}

// Where code k of the row goes: row-major (Q + m*ldq + k) or fragment order.
// In both layouts each aligned 16-code chunk is 16 contiguous bytes.
struct QDest {
    int8_t *Q;
    int64_t ldq;  // row-major stride; unused in fragment order
    int64_t m;
    int64_t KU;
    int tiled;
    __device__ int64_t at(int64_t k) const { return tiled ? qf32_offset(m, k, KU) : m * ldq + k; }
    __device__ int64_t fill_end() const { return tiled ? 64 * KU : ldq; }
};

// One token row.  Each thread owns 16-code chunks (four 16-byte loads, one
// 16-byte store); rows of up to kRegChunks * 16 * 256 values stay in
// registers between the max and the rounding pass, so X is read from HBM
// once; longer rows read it twice (the second pass mostly from L2).
constexpr int kRegChunks = 2;

__device__ void quant_row(const float *x_, int K, const QDest &dst, float *absmax_,
                          int32_t *rowsum_)
{
    __shared__ float fl[4];
    __shared__ int il[4];
    const BL_GLOBAL float *x = gload_ptr<float>(x_);
    BL_GLOBAL int8_t *q = gstore_ptr<int8_t>(dst.Q);
    const int tid = threadIdx.x;
    // chunk path: K a multiple of 16 and X rows 16-byte aligned
    const bool vec = ((K & 15) == 0) && ((reinterpret_cast<uintptr_t>(x_) & 15) == 0);
    const int nc = K >> 4;
    const BL_GLOBAL v4f *x4 = reinterpret_cast<const BL_GLOBAL v4f *>(x);
    const bool in_regs = vec && nc <= kRegChunks * kThreads;
    const v4f zero4 = {0.f, 0.f, 0.f, 0.f};

    auto amax4 = [](v4f w) {
        return fmaxf(fmaxf(fabsf(w.x), fabsf(w.y)), fmaxf(fabsf(w.z), fabsf(w.w)));
    };
    v4f v[kRegChunks][4];
    float a = 0.0f;
    if (in_regs) {
#pragma unroll
        for (int j = 0; j < kRegChunks; ++j) {
            const int c = tid + j * kThreads;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                v[j][t] = c < nc ? x4[4 * c + t] : zero4;
                a = fmaxf(a, amax4(v[j][t]));
            }
        }
    } else if (vec) {
        for (int c = tid; c < nc; c += kThreads)
#pragma unroll
            for (int t = 0; t < 4; ++t) a = fmaxf(a, amax4(x4[4 * c + t]));
    } else {
        for (int i = tid; i < K; i += kThreads) a = fmaxf(a, fabsf(x[i]));
    }
    a = block_max(a, fl);
    if (!(a >= 1e-5f)) a = 1e-5f;
    const float s = 127.0f / a;

    int sum = 0;
    auto pack4 = [&](v4f w) {
        const int8_t c0 = quant_code(w.x, s), c1 = quant_code(w.y, s);
        const int8_t c2 = quant_code(w.z, s), c3 = quant_code(w.w, s);
        sum += (int)c0 + (int)c1 + (int)c2 + (int)c3;
        return (uint32_t)(uint8_t)c0 | ((uint32_t)(uint8_t)c1 << 8) | ((uint32_t)(uint8_t)c2 << 16) |
               ((uint32_t)(uint8_t)c3 << 24);
    };
    auto put16 = [&](int c, const v4f *w) {
        v4u o;
        o.x = pack4(w[0]);
        o.y = pack4(w[1]);
        o.z = pack4(w[2]);
        o.w = pack4(w[3]);
        *reinterpret_cast<BL_GLOBAL v4u *>(q + dst.at(16 * c)) = o;
    };
    if (in_regs) {
#pragma unroll
        for (int j = 0; j < kRegChunks; ++j) {
            const int c = tid + j * kThreads;
            if (c < nc) put16(c, v[j]);
        }
    } else if (vec) {
        for (int c = tid; c < nc; c += kThreads) {
            v4f w[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) w[t] = x4[4 * c + t];
            put16(c, w);
        }
    } else {
        for (int i = tid; i < K; i += kThreads) {
            const int8_t c = quant_code(x[i], s);
            sum += c;
            q[dst.at(i)] = c;
        }
    }
    for (int64_t i = K + tid; i < dst.fill_end(); i += kThreads) q[dst.at(i)] = 0;
    sum = block_sum_i32(sum, il);
    if (tid == 0) {
        *gstore_ptr<float>(absmax_) = a;
        if (rowsum_) *gstore_ptr<int32_t>(rowsum_) = sum;
    }
}

__global__ __launch_bounds__(kThreads) void quant_act_kernel(const float *__restrict__ X, int K,
                                                             int8_t *__restrict__ Q, int64_t ldq,
                                                             int qtiled,
                                                             float *__restrict__ absmax,
                                                             int32_t *__restrict__ rowsum,
                                                             uint32_t *__restrict__ zero_ptr,
                                                             int zero_n)
{
    const int64_t m = blockIdx.x;
    if (m == 0 && zero_ptr)
        for (int i = threadIdx.x; i < zero_n; i += kThreads) zero_ptr[i] = 0u;
    const QDest dst{Q, ldq, m, (K + 63) / 64, qtiled};
    quant_row(X + m * K, K, dst, absmax + m, rowsum ? rowsum + m : nullptr);
}

__global__ __launch_bounds__(kThreads) void quant_act_group_kernel(const Problem *__restrict__ probs,
                                                                   const uint32_t *__restrict__ tok_map)
{
    const int tok = blockIdx.x;
    const Problem &p = probs[tok_map[tok]];
    const int64_t m = tok - p.tok_begin;
    if (m == 0 && p.tickets)
        for (int i = threadIdx.x; i < p.NT; i += kThreads) p.tickets[i] = 0u;
    const QDest dst{p.Q, p.ldq, m, p.KU, p.qtiled};
    quant_row(p.X + m * p.K, p.K, dst, p.absmax + m, p.rowsum + m);
}

__global__ __launch_bounds__(kThreads) void zero_words_kernel(uint32_t *__restrict__ p, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) p[i] = 0u;
}

}  // namespace

hipError_t launch_quant_act(const float *X, int64_t M, int64_t K, int8_t *Q, int64_t ldq,
                            int qtiled, float *absmax, int32_t *rowsum, uint32_t *zero_ptr,
                            int zero_n, hipStream_t s)
{
    hipLaunchKernelGGL(quant_act_kernel, dim3((unsigned)M), dim3(kThreads), 0, s, X, (int)K, Q, ldq,
                       qtiled, absmax, rowsum, zero_ptr, zero_n);
    return hipGetLastError();
}

hipError_t launch_quant_act_group(const Problem *probs, const uint32_t *tok_map, int n_tokens,
                                  hipStream_t s)
{
    hipLaunchKernelGGL(quant_act_group_kernel, dim3((unsigned)n_tokens), dim3(kThreads), 0, s,
                       probs, tok_map);
    return hipGetLastError();
}

hipError_t launch_zero_words(uint32_t *p, int64_t n, hipStream_t s)
{
    int64_t blocks = (n + kThreads - 1) / kThreads;
    if (blocks < 1) blocks = 1;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, p, n);
    return hipGetLastError();
}

}  // namespace bl
