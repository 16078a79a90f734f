// BT5-T32 packing: five ternary codes per byte in base 3 (the format and
// the reason for it are described in bt5.hpp).
//
// One thread builds one 32-bit word of the packed buffer, i.e. four packed
// bytes p = 4 d .. 4 d + 3 of one slot.  Word index i -> block b = i / 256
// (tile t = b / KU5, unit u = b % KU5), slot L = (i % 256) / 4, word d = i % 4;
// byte p holds row 32 t + L % 32 and codes 160 u + 32 i' + 16 (L / 32) + p
// for digit i' = 0..4.  Out-of-range rows and codes are zero codes.
#include "bt5.hpp"

namespace bl {
namespace {

constexpr int kThreads = 256;

__device__ inline int digit_of(int8_t t)
{
    return (t > 0 ? 1 : (t < 0 ? -1 : 0)) + 1;
}

__global__ __launch_bounds__(kThreads) void pack5_kernel(const int8_t *__restrict__ T, int64_t N,
                                                         int64_t K, int64_t KU5, int64_t words,
                                                         uint32_t *__restrict__ P)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < words; i += stride) {
        const int64_t b = i >> 8;
        const int w = (int)(i & 255);
        const int L = w >> 2, d = w & 3;
        const int64_t t = b / KU5, u = b - t * KU5;
        const int64_t n = kBt5TileRows * t + (L & 31);
        const int64_t k0 = kBt5UnitCodes * u + 16 * (L >> 5) + 4 * d;
        uint32_t word = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            unsigned v = 0;  // base-3 value, digit 0 most significant
#pragma unroll
            for (int dig = 0; dig < 5; ++dig) {
                const int64_t k = k0 + 32 * dig + q;
                const int8_t code = (n < N && k < K) ? T[n * K + k] : (int8_t)0;
                v = 3 * v + (unsigned)digit_of(code);
            }
            const unsigned s = (256u * v + 242u) / 243u;  // ceil(256 v / 243)
            word |= s << (8 * q);
        }
        P[i] = word;
    }
}

// Decodes with the contraction kernel's prefix planes, so a round trip
// through pack5 and unpack5 checks that decode on every byte.
__global__ __launch_bounds__(kThreads) void unpack5_kernel(const uint32_t *__restrict__ P,
                                                           int64_t N, int64_t K, int64_t KU5,
                                                           int64_t words, int8_t *__restrict__ T)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < words; i += stride) {
        const int64_t b = i >> 8;
        const int w = (int)(i & 255);
        const int L = w >> 2, d = w & 3;
        const int64_t t = b / KU5, u = b - t * KU5;
        const int64_t n = kBt5TileRows * t + (L & 31);
        if (n >= N) continue;
        const int64_t k0 = kBt5UnitCodes * u + 16 * (L >> 5) + 4 * d;
        const Bt5Planes pl = bt5_planes(P[i]);
        // digit bytes: d_0 = H_1, d_i = H_(i+1) - 3 H_i, d_4 from the planes
        unsigned dg[5];
        dg[0] = pl.h[0];
#pragma unroll
        for (int j = 1; j < 4; ++j) dg[j] = pl.h[j] - (pl.h[j - 1] + (pl.h[j - 1] << 1));
        dg[4] = pl.h[4];
#pragma unroll
        for (int dig = 0; dig < 5; ++dig)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t k = k0 + 32 * dig + q;
                if (k < K) T[n * K + k] = (int8_t)((int)((dg[dig] >> (8 * q)) & 0xFF) - 1);
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

hipError_t launch_pack5(const int8_t *T, int64_t N, int64_t K, uint8_t *P, hipStream_t s)
{
    const int64_t KU5 = (K + kBt5UnitCodes - 1) / kBt5UnitCodes;
    const int64_t NT = (N + kBt5TileRows - 1) / kBt5TileRows;
    const int64_t words = NT * KU5 * 256;
    hipLaunchKernelGGL(pack5_kernel, dim3(grid_for(words)), dim3(kThreads), 0, s, T, N, K, KU5,
                       words, reinterpret_cast<uint32_t *>(P));
    return hipGetLastError();
}

hipError_t launch_unpack5(const uint8_t *P, int64_t N, int64_t K, int8_t *T, hipStream_t s)
{
    const int64_t KU5 = (K + kBt5UnitCodes - 1) / kBt5UnitCodes;
    const int64_t NT = (N + kBt5TileRows - 1) / kBt5TileRows;
    const int64_t words = NT * KU5 * 256;
    hipLaunchKernelGGL(unpack5_kernel, dim3(grid_for(words)), dim3(kThreads), 0, s,
                       reinterpret_cast<const uint32_t *>(P), N, K, KU5, words, T);
    return hipGetLastError();
}

}  // namespace bl
