// Absmean ternary weight quantization for gfx950.
//
// anthology note-168 on arXiv 2402.17764, "What it does": BitLinear weights
// are restricted to {-1, 0, +1} by an absmean quantizer.  The pages print no
// formula; the reading implemented here is gamma = mean |W| over the whole
// matrix, t = clamp(rint(w / gamma), -1, 1) with round-half-to-even.
//
// Off the per-token path (runs once per weight matrix), HBM-bound:
//   pass 1  absmean_partial : fixed-shape fp64 partial sums of |W|
//   pass 2  absmean_final   : fixed-order fp64 sum -> one fp32 rounding
//   pass 3  ternarize       : 16 weights per thread, 16-byte code stores
// The reduction order depends only on the matrix size and the block count,
// so gamma is identical from run to run.
#include "common.hpp"

namespace bl {
namespace {

constexpr int kThreads = 256;

__device__ inline double block_sum_f64(double v, double *lds)
{
    // fixed pairing order: xor butterflies inside the wave, then the four
    // wave sums added in wave order by thread 0
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) lds[wave] = v;
    __syncthreads();
    double s = 0.0;
    if (threadIdx.x == 0) s = ((lds[0] + lds[1]) + lds[2]) + lds[3];
    return s;
}

__global__ __launch_bounds__(kThreads) void absmean_partial_kernel(const float *__restrict__ W,
                                                                   int64_t count, int64_t chunk,
                                                                   double *__restrict__ partial)
{
    __shared__ double lds[4];
    const int64_t begin = (int64_t)blockIdx.x * chunk;
    const int64_t end = begin + chunk < count ? begin + chunk : count;
    double s = 0.0;
    // chunk is a multiple of 4 and W is 16-byte aligned: float4 body
    const int64_t vec_end = begin + ((end - begin) & ~(int64_t)3);
    for (int64_t i = begin + 4 * (int64_t)threadIdx.x; i < vec_end; i += 4 * kThreads) {
        const float4 w = *reinterpret_cast<const float4 *>(W + i);
        s += fabs((double)w.x);
        s += fabs((double)w.y);
        s += fabs((double)w.z);
        s += fabs((double)w.w);
    }
    for (int64_t i = vec_end + threadIdx.x; i < end; i += kThreads) s += fabs((double)W[i]);
    s = block_sum_f64(s, lds);
    if (threadIdx.x == 0) partial[blockIdx.x] = s;
}

__global__ __launch_bounds__(kThreads) void absmean_final_kernel(const double *__restrict__ partial,
                                                                 int nblocks, int64_t count,
                                                                 const float *__restrict__ gamma_in,
                                                                 float *__restrict__ gamma_out)
{
    __shared__ double lds[4];
    if (gamma_in != nullptr) {
        if (threadIdx.x == 0) *gamma_out = *gamma_in;
        return;
    }
    double s = 0.0;
    for (int i = threadIdx.x; i < nblocks; i += kThreads) s += partial[i];
    s = block_sum_f64(s, lds);
    if (threadIdx.x == 0) {
        const double mean = s / (double)count;
        float g = (float)mean;
        if (!(g >= 1e-5f)) g = 1e-5f;
        *gamma_out = g;
    }
}

__device__ inline int8_t ternary_code(float w, float g)
{
    const float r = rintf(w / g);  // IEEE division (no fast-math), round half to even
    return r >= 1.0f ? (int8_t)1 : (r <= -1.0f ? (int8_t)-1 : (int8_t)0);
}

__global__ __launch_bounds__(kThreads) void ternarize_kernel(const float *__restrict__ W,
                                                             int64_t count,
                                                             const float *__restrict__ gamma,
                                                             int8_t *__restrict__ T)
{
    const float g = *gamma;
    const int64_t groups = count >> 4;  // 16 weights per thread
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < groups; i += stride) {
        const float4 *src = reinterpret_cast<const float4 *>(W + 16 * i);
        uint32_t word[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float4 w = src[j];
            const uint32_t b0 = (uint8_t)ternary_code(w.x, g);
            const uint32_t b1 = (uint8_t)ternary_code(w.y, g);
            const uint32_t b2 = (uint8_t)ternary_code(w.z, g);
            const uint32_t b3 = (uint8_t)ternary_code(w.w, g);
            word[j] = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
        }
        *reinterpret_cast<uint4 *>(T + 16 * i) = make_uint4(word[0], word[1], word[2], word[3]);
    }
    // tail (count % 16 weights), handled by the first block
    if (blockIdx.x == 0) {
        const int64_t t = 16 * groups + threadIdx.x;
        if (t < count) T[t] = ternary_code(W[t], g);
    }
}

}  // namespace

hipError_t launch_absmean_partial(const float *W, int64_t count, double *partial, int nblocks,
                                  hipStream_t s)
{
    int64_t chunk = (count + nblocks - 1) / nblocks;
    chunk = (chunk + 3) & ~(int64_t)3;
    hipLaunchKernelGGL(absmean_partial_kernel, dim3(nblocks), dim3(kThreads), 0, s, W, count,
                       chunk, partial);
    return hipGetLastError();
}

hipError_t launch_absmean_final(const double *partial, int nblocks, int64_t count,
                                const float *gamma_in, float *gamma_out, hipStream_t s)
{
    hipLaunchKernelGGL(absmean_final_kernel, dim3(1), dim3(kThreads), 0, s, partial, nblocks,
                       count, gamma_in, gamma_out);
    return hipGetLastError();
}

hipError_t launch_ternarize(const float *W, int64_t count, const float *gamma, int8_t *T,
                            hipStream_t s)
{
    const int64_t groups = count >> 4;
    int64_t blocks = (groups + kThreads - 1) / kThreads;
    if (blocks < 1) blocks = 1;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(ternarize_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, W, count,
                       gamma, T);
    return hipGetLastError();
}

}  // namespace bl
