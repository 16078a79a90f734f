// Per-token absmax int8 activation quantization for gfx950 (the row cast
// itself, its readings of the pages and its citations are in quant_row.hpp).
//
// One workgroup per token: one wave when there are many tokens (2048 or
// more), four for 512..2047, sixteen for fewer than 512 (decode and short
// prefill chains, where each cast is a few workgroups' latency problem).  Variants cast the RMSNorm of the row
// (the sub-layer norm before a BitLinear), the residual sum and its RMSNorm,
// or the gated squared-ReLU of two rows (the feed-forward hidden value
// before the down projection), computed in the same pass over the inputs.
#include "quant_row.hpp"

namespace bl {
namespace {

constexpr int kThreads = 256;
constexpr int kFewTokens = 2048;
constexpr int kSingleTokens = 512;  // fewer rows: sixteen waves per row

// One workgroup per token.
template <int WAVES, int MODE>
__global__ __launch_bounds__(64 * WAVES) void quant_act_kernel(const float *__restrict__ X, int K,
                                                               int8_t *__restrict__ Q, int64_t ldq,
                                                               int qtiled, float *__restrict__ absmax,
                                                               int32_t *__restrict__ rowsum,
                                                               uint32_t *__restrict__ zero_ptr,
                                                               int zero_n, const float *__restrict__ g,
                                                               float eps, const float *res = nullptr,
                                                               float *xo = nullptr)
{
    const int64_t m = blockIdx.x;
    if (m == 0 && zero_ptr)
        for (int i = threadIdx.x; i < zero_n; i += 64 * WAVES) zero_ptr[i] = 0u;
    const QDest dst{Q, ldq, m, (K + 63) / 64, qtiled};
    // the gate/up mode reads a second M x K array (g) row by row
    const float *aux = MODE == kRelu2Gate ? g + m * K : g;
    RowScale rsc;
    if constexpr (MODE == kAddRmsNorm)
        rsc = quant_row<WAVES, MODE>(X + m * K, K, dst, aux, eps, res + m * K, xo + m * K);
    else
        rsc = quant_row<WAVES, MODE>(X + m * K, K, dst, aux, eps);
    if (threadIdx.x == 0) {
        absmax[m] = rsc.a;
        if (rowsum) rowsum[m] = rsc.sum;
    }
}

template <int WAVES>
__global__ __launch_bounds__(64 * WAVES) void quant_act_group_kernel(const Problem *__restrict__ probs,
                                                                     const uint32_t *__restrict__ tok_map)
{
    const int tok = blockIdx.x;
    const Problem &p = probs[tok_map[tok]];
    const int64_t m = tok - p.tok_begin;
    if (m == 0 && p.tickets)
        for (int64_t i = threadIdx.x; i < ticket_count(p); i += 64 * WAVES) p.tickets[i] = 0u;
    const QDest dst{p.Q, p.ldq, m, p.KU, p.qtiled};
    const RowScale rsc = quant_row<WAVES, kPlain>(p.X + m * p.K, p.K, dst, nullptr, 0.0f);
    if (threadIdx.x == 0) {
        p.absmax[m] = rsc.a;
        p.rowsum[m] = rsc.sum;
    }
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
    if (M < kSingleTokens)
        hipLaunchKernelGGL((quant_act_kernel<16, kPlain>), dim3((unsigned)M), dim3(1024), 0, s, X, (int)K, Q,
                           ldq, qtiled, absmax, rowsum, zero_ptr, zero_n, nullptr, 0.0f);
    else if (M < kFewTokens)
        hipLaunchKernelGGL((quant_act_kernel<4, kPlain>), dim3((unsigned)M), dim3(256), 0, s, X, (int)K, Q,
                           ldq, qtiled, absmax, rowsum, zero_ptr, zero_n, nullptr, 0.0f);
    else
        hipLaunchKernelGGL((quant_act_kernel<1, kPlain>), dim3((unsigned)M), dim3(64), 0, s, X, (int)K, Q,
                           ldq, qtiled, absmax, rowsum, zero_ptr, zero_n, nullptr, 0.0f);
    return hipGetLastError();
}

hipError_t launch_quant_act_rmsnorm(const float *X, int64_t M, int64_t K, const float *g, float eps,
                                    int8_t *Q, int64_t ldq, float *absmax, int32_t *rowsum,
                                    hipStream_t s)
{
    if (M < kSingleTokens)
        hipLaunchKernelGGL((quant_act_kernel<16, kRmsNorm>), dim3((unsigned)M), dim3(1024), 0, s, X, (int)K, Q,
                           ldq, 0, absmax, rowsum, nullptr, 0, g, eps);
    else if (M < kFewTokens)
        hipLaunchKernelGGL((quant_act_kernel<4, kRmsNorm>), dim3((unsigned)M), dim3(256), 0, s, X, (int)K, Q,
                           ldq, 0, absmax, rowsum, nullptr, 0, g, eps);
    else
        hipLaunchKernelGGL((quant_act_kernel<1, kRmsNorm>), dim3((unsigned)M), dim3(64), 0, s, X, (int)K, Q,
                           ldq, 0, absmax, rowsum, nullptr, 0, g, eps);
    return hipGetLastError();
}

hipError_t launch_quant_act_add_rmsnorm(const float *X, const float *R, int64_t M, int64_t K, const float *g,
                                        float eps, float *Xsum, int8_t *Q, int64_t ldq, float *absmax,
                                        int32_t *rowsum, hipStream_t s)
{
    if (M < kSingleTokens)
        hipLaunchKernelGGL((quant_act_kernel<16, kAddRmsNorm>), dim3((unsigned)M), dim3(1024), 0, s, X, (int)K,
                           Q, ldq, 0, absmax, rowsum, nullptr, 0, g, eps, R, Xsum);
    else if (M < kFewTokens)
        hipLaunchKernelGGL((quant_act_kernel<4, kAddRmsNorm>), dim3((unsigned)M), dim3(256), 0, s, X, (int)K,
                           Q, ldq, 0, absmax, rowsum, nullptr, 0, g, eps, R, Xsum);
    else
        hipLaunchKernelGGL((quant_act_kernel<1, kAddRmsNorm>), dim3((unsigned)M), dim3(64), 0, s, X, (int)K,
                           Q, ldq, 0, absmax, rowsum, nullptr, 0, g, eps, R, Xsum);
    return hipGetLastError();
}

hipError_t launch_quant_act_relu2_gate(const float *G, const float *U, int64_t M, int64_t N, int8_t *Q,
                                       int64_t ldq, float *absmax, int32_t *rowsum, hipStream_t s)
{
    if (M < kSingleTokens)
        hipLaunchKernelGGL((quant_act_kernel<16, kRelu2Gate>), dim3((unsigned)M), dim3(1024), 0, s, G, (int)N,
                           Q, ldq, 0, absmax, rowsum, nullptr, 0, U, 0.0f);
    else if (M < kFewTokens)
        hipLaunchKernelGGL((quant_act_kernel<4, kRelu2Gate>), dim3((unsigned)M), dim3(256), 0, s, G, (int)N,
                           Q, ldq, 0, absmax, rowsum, nullptr, 0, U, 0.0f);
    else
        hipLaunchKernelGGL((quant_act_kernel<1, kRelu2Gate>), dim3((unsigned)M), dim3(64), 0, s, G, (int)N,
                           Q, ldq, 0, absmax, rowsum, nullptr, 0, U, 0.0f);
    return hipGetLastError();
}

hipError_t launch_quant_act_group(const Problem *probs, const uint32_t *tok_map, int n_tokens,
                                  hipStream_t s)
{
    if (n_tokens < kFewTokens)
        hipLaunchKernelGGL(quant_act_group_kernel<4>, dim3((unsigned)n_tokens), dim3(256), 0, s, probs,
                           tok_map);
    else
        hipLaunchKernelGGL(quant_act_group_kernel<1>, dim3((unsigned)n_tokens), dim3(64), 0, s, probs,
                           tok_map);
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
