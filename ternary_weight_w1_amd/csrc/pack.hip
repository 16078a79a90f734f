// BL2-T64 packing of ternary codes, four to a byte (BitNet b1.58 2B4T video
// transcript, yousumm.com, "Transcription": four codes are bundled into one
// byte, streamed to the compute unit and unpacked beside the multiplier).
//
// One thread builds one 32-bit word of the packed buffer: 16 codes of one
// row.  Word index i -> block b = i / 256 (tile t = b / KU, unit u = b % KU),
// slot L = (i % 256) / 4, word d = i % 4 = 2*s + h; the word holds row
// 64*t + 32*s + L%32, codes 64*u + 32*h + 16*(L/32) + c, c = 0..15, with
// field (code + 1) at bit 8*(c%4) + 2*(c/4).  Out-of-range rows and codes
// are written as zero codes (field 1).  Consecutive threads write
// consecutive words, so the stores are fully coalesced.
#include "common.hpp"

namespace bl {
namespace {

constexpr int kThreads = 256;

__device__ inline uint32_t field_of(int8_t t)
{
    const int c = t > 1 ? 1 : (t < -1 ? -1 : (int)t);
    return (uint32_t)(c + 1);
}

__global__ __launch_bounds__(kThreads) void pack_kernel(const int8_t *__restrict__ T, int64_t N,
                                                        int64_t K, int64_t KU, int64_t words,
                                                        uint32_t *__restrict__ P)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < words; i += stride) {
        const int64_t b = i >> 8;
        const int w = (int)(i & 255);
        const int L = w >> 2, d = w & 3;
        const int64_t t = b / KU, u = b - t * KU;
        const int64_t n = 64 * t + 32 * (d >> 1) + (L & 31);
        const int64_t k0 = 64 * u + 32 * (d & 1) + 16 * (L >> 5);
        uint32_t word = 0x55555555u;  // all zero codes
        if (n < N) {
            const int8_t *row = T + n * K;
            if ((K & 15) == 0 && k0 + 16 <= K) {
                const uint4 v = *reinterpret_cast<const uint4 *>(row + k0);
                const uint32_t q[4] = {v.x, v.y, v.z, v.w};
                word = 0;
#pragma unroll
                for (int c = 0; c < 16; ++c) {
                    const int8_t code = (int8_t)((q[c >> 2] >> (8 * (c & 3))) & 0xFF);
                    word |= field_of(code) << (8 * (c & 3) + 2 * (c >> 2));
                }
            } else {
                word = 0;
                for (int c = 0; c < 16; ++c) {
                    const int8_t code = (k0 + c < K) ? row[k0 + c] : (int8_t)0;
                    word |= field_of(code) << (8 * (c & 3) + 2 * (c >> 2));
                }
            }
        }
        P[i] = word;
    }
}

__global__ __launch_bounds__(kThreads) void unpack_kernel(const uint32_t *__restrict__ P,
                                                          int64_t N, int64_t K, int64_t KU,
                                                          int64_t words, int8_t *__restrict__ T)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < words; i += stride) {
        const int64_t b = i >> 8;
        const int w = (int)(i & 255);
        const int L = w >> 2, d = w & 3;
        const int64_t t = b / KU, u = b - t * KU;
        const int64_t n = 64 * t + 32 * (d >> 1) + (L & 31);
        const int64_t k0 = 64 * u + 32 * (d & 1) + 16 * (L >> 5);
        if (n >= N) continue;
        const uint32_t word = P[i];
        for (int c = 0; c < 16; ++c) {
            if (k0 + c >= K) break;
            const int f = (word >> (8 * (c & 3) + 2 * (c >> 2))) & 3;
            T[n * K + k0 + c] = (int8_t)(f == 3 ? 0 : f - 1);
        }
    }
}

int grid_for(int64_t work)
{
    int64_t blocks = (work + kThreads - 1) / kThreads;
    if (blocks < 1) blocks = 1;
    if (blocks > 65536) blocks = 65536;
    return (int)blocks;
}

}  // namespace

hipError_t launch_pack(const int8_t *T, int64_t N, int64_t K, uint8_t *P, hipStream_t s)
{
    const int64_t KU = (K + 63) / 64, NT = (N + 63) / 64;
    const int64_t words = NT * KU * 256;
    hipLaunchKernelGGL(pack_kernel, dim3(grid_for(words)), dim3(kThreads), 0, s, T, N, K, KU,
                       words, reinterpret_cast<uint32_t *>(P));
    return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t *P, int64_t N, int64_t K, int8_t *T, hipStream_t s)
{
    const int64_t KU = (K + 63) / 64, NT = (N + 63) / 64;
    const int64_t words = NT * KU * 256;
    hipLaunchKernelGGL(unpack_kernel, dim3(grid_for(words)), dim3(kThreads), 0, s,
                       reinterpret_cast<const uint32_t *>(P), N, K, KU, words, T);
    return hipGetLastError();
}

}  // namespace bl
