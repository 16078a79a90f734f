// Calibration kernels for the two roofline denominators the contraction
// kernels are reported against: a plain streaming read of a device buffer
// (the HBM bound of the one-token sweep) and a chain of int8 matrix
// instructions with no memory traffic at all (the bound of the prefill
// contraction).  Neither does any of the layer's arithmetic; each leaves a
// checksum so that its work cannot be dropped and its result can be checked.
#include "mm_common.hpp"
#include "probe.hpp"

namespace bl {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeReadUnroll = 8;  // 16-byte loads in flight per thread

// Workgroup b streams the 16-byte words [b * chunk16, (b + 1) * chunk16) of
// the buffer (the last chunk may be short): consecutive lanes read
// consecutive words, eight loads in flight per thread, all folded with XOR.
__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const v4u *__restrict__ p, int64_t n16,
                                                                   int64_t chunk16, uint32_t *__restrict__ sink)
{
    const int64_t begin = (int64_t)blockIdx.x * chunk16;
    const int64_t end = begin + chunk16 < n16 ? begin + chunk16 : n16;
    const BL_GLOBAL v4u *src = gload_ptr<v4u>(p);
    v4u acc = {0u, 0u, 0u, 0u};
    int64_t i = begin + threadIdx.x;
    for (; i + (kProbeReadUnroll - 1) * kProbeThreads < end; i += kProbeReadUnroll * kProbeThreads) {
        v4u v[kProbeReadUnroll];
#pragma unroll
        for (int j = 0; j < kProbeReadUnroll; ++j) v[j] = load_packed(src + i + j * kProbeThreads);
#pragma unroll
        for (int j = 0; j < kProbeReadUnroll; ++j) acc ^= v[j];
    }
    for (; i < end; i += kProbeThreads) acc ^= load_packed(src + i);
    gstore_ptr<uint32_t>(sink)[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

// Four independent accumulator chains of v_mfma_i32_32x32x32_i8 per wave,
// every operand byte equal to a (A) or b (B): each accumulator element gains
// 32 a b per instruction, so after `iters` rounds every thread's 64 elements
// sum to 2048 a b iters, which is what it writes.
__global__ __launch_bounds__(kProbeThreads) void probe_mfma_kernel(int64_t iters, int a, int b,
                                                                   int32_t *__restrict__ sink)
{
    const int ab = (int)((uint32_t)(a & 0xff) * 0x01010101u);
    const int bb = (int)((uint32_t)(b & 0xff) * 0x01010101u);
    const v4i av = {ab, ab, ab, ab}, bv = {bb, bb, bb, bb};
    v16i acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = (v16i){};
    for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = mfma_i8(av, bv, acc[j]);
    }
    int32_t s = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[j][e];
    gstore_ptr<int32_t>(sink)[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_probe_read(const void *buf, int64_t bytes, int64_t chunk_bytes, uint32_t *sink, hipStream_t s)
{
    const int64_t chunks = (bytes + chunk_bytes - 1) / chunk_bytes;
    hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)chunks), dim3(kProbeThreads), 0, s,
                       static_cast<const v4u *>(buf), bytes / 16, chunk_bytes / 16, sink);
    return hipGetLastError();
}

hipError_t launch_probe_mfma(int64_t iters, int a, int b, int blocks, int32_t *sink, hipStream_t s)
{
    hipLaunchKernelGGL(probe_mfma_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0, s, iters, a, b, sink);
    return hipGetLastError();
}

hipError_t probe_mfma_resident_blocks(int *blocks)
{
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(probe_mfma_kernel),
                                                         kProbeThreads, 0);
    if (e == hipSuccess) *blocks = cus * per_cu;
    return e;
}

}  // namespace bl
