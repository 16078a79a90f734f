// Per-token absmax int8 activation quantization for gfx950.
//
// anthology note-168 on arXiv 2402.17764, "What it does": BitLinear's
// activations are 8-bit.  Reading implemented (the pages print no formula):
// a = max(1e-5, max_k |x_k|) for each token, s = 127 / a (one fp32 IEEE
// division per token), q_k = clamp(rint(x_k * s), -127, 127).  The row sum
// of q is produced too: the contraction kernels multiply by (code + 1)
// fields and subtract it once per output.
//
// One 256-thread workgroup per token: pass 1 reads the row with 16-byte
// loads and reduces |x| with wave butterflies, then across the four waves
// through LDS; pass 2 re-reads the row (L1/L2 resident) and writes four
// codes per 32-bit store.  The max is order-free and the row sum is an
// integer sum, so both are exact whatever the reduction order.
#include "common.hpp"

namespace bl {
namespace {

constexpr int kThreads = 256;

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

__device__ inline int8_t quant_code(float x, float s)
{
    float r = rintf(x * s);
    r = r > 127.0f ? 127.0f : r;
    r = r < -127.0f ? -127.0f : r;
    return (int8_t)(int)r;
}

__device__ void quant_row(const float *__restrict__ x, int K, int8_t *__restrict__ q, int64_t ldq,
                          float *__restrict__ absmax, int32_t *__restrict__ rowsum)
{
    __shared__ float fl[4];
    __shared__ int il[4];
    const int tid = threadIdx.x;
    const bool vec = ((K & 3) == 0) && ((reinterpret_cast<uintptr_t>(x) & 15) == 0);

    float a = 0.0f;
    if (vec) {
        const float4 *x4 = reinterpret_cast<const float4 *>(x);
        for (int i = tid; i < (K >> 2); i += kThreads) {
            const float4 v = x4[i];
            a = fmaxf(a, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
        }
    } else {
        for (int i = tid; i < K; i += kThreads) a = fmaxf(a, fabsf(x[i]));
    }
    a = block_max(a, fl);
    if (!(a >= 1e-5f)) a = 1e-5f;
    const float s = 127.0f / a;

    int sum = 0;
    if (vec) {
        const float4 *x4 = reinterpret_cast<const float4 *>(x);
        uint32_t *q4 = reinterpret_cast<uint32_t *>(q);
        for (int i = tid; i < (K >> 2); i += kThreads) {
            const float4 v = x4[i];
            const int8_t c0 = quant_code(v.x, s), c1 = quant_code(v.y, s);
            const int8_t c2 = quant_code(v.z, s), c3 = quant_code(v.w, s);
            sum += (int)c0 + (int)c1 + (int)c2 + (int)c3;
            q4[i] = (uint32_t)(uint8_t)c0 | ((uint32_t)(uint8_t)c1 << 8) |
                    ((uint32_t)(uint8_t)c2 << 16) | ((uint32_t)(uint8_t)c3 << 24);
        }
    } else {
        for (int i = tid; i < K; i += kThreads) {
            const int8_t c = quant_code(x[i], s);
            sum += c;
            q[i] = c;
        }
    }
    for (int64_t i = K + tid; i < ldq; i += kThreads) q[i] = 0;
    sum = block_sum_i32(sum, il);
    if (tid == 0) {
        *absmax = a;
        if (rowsum) *rowsum = sum;
    }
}

__global__ __launch_bounds__(kThreads) void quant_act_kernel(const float *__restrict__ X, int K,
                                                             int8_t *__restrict__ Q, int64_t ldq,
                                                             float *__restrict__ absmax,
                                                             int32_t *__restrict__ rowsum,
                                                             uint32_t *__restrict__ zero_ptr,
                                                             int zero_n)
{
    const int64_t m = blockIdx.x;
    if (m == 0 && zero_ptr)
        for (int i = threadIdx.x; i < zero_n; i += kThreads) zero_ptr[i] = 0u;
    quant_row(X + m * K, K, Q + m * ldq, ldq, absmax + m, rowsum ? rowsum + m : nullptr);
}

__global__ __launch_bounds__(kThreads) void quant_act_group_kernel(const Problem *__restrict__ probs,
                                                                   const uint32_t *__restrict__ tok_map)
{
    const int tok = blockIdx.x;
    const Problem &p = probs[tok_map[tok]];
    const int64_t m = tok - p.tok_begin;
    if (m == 0 && p.tickets)
        for (int i = threadIdx.x; i < p.NT; i += kThreads) p.tickets[i] = 0u;
    quant_row(p.X + m * p.K, p.K, p.Q + m * p.ldq, p.ldq, p.absmax + m, p.rowsum + m);
}

__global__ __launch_bounds__(kThreads) void zero_words_kernel(uint32_t *__restrict__ p, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) p[i] = 0u;
}

}  // namespace

hipError_t launch_quant_act(const float *X, int64_t M, int64_t K, int8_t *Q, int64_t ldq,
                            float *absmax, int32_t *rowsum, uint32_t *zero_ptr, int zero_n,
                            hipStream_t s)
{
    hipLaunchKernelGGL(quant_act_kernel, dim3((unsigned)M), dim3(kThreads), 0, s, X, (int)K, Q, ldq,
                       absmax, rowsum, zero_ptr, zero_n);
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
