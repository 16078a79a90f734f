// Calibration kernels for the two roofline denominators the contraction
// kernels are reported against: a plain streaming read of a device buffer
// (the HBM bound of the one-token sweep) and a chain of int8 matrix
// instructions with no memory traffic at all (the bound of the prefill
// contraction); and the cost of a grid-wide barrier with data exchange,
// the price a persistent kernel would pay per dependent stage.  None does
// any of the layer's arithmetic; each leaves a checksum so that its work
// cannot be dropped and its result can be checked.
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

// The same four chains with operands taken from memory: kProbeSets pairs of
// (A, B) fragments, 16 bytes per lane each, loaded once into registers; chain
// j multiplies set j, so consecutive matrix instructions take different
// operand bits, as they do in a contraction over real data (the constant
// operands above toggle almost nothing).  Thread 0 of each workgroup records
// the shader-clock count over its loop and the reference-clock counter at
// its start and end, so the clock the part sustains under this load can be
// read off.
constexpr int kProbeSets = 4;
__global__ __launch_bounds__(kProbeThreads) void probe_mfma_data_kernel(int64_t iters, const v4i *__restrict__ ops,
                                                                        int32_t *__restrict__ sink,
                                                                        uint64_t *__restrict__ clocks)
{
    const int lane = threadIdx.x & 63;
    v4i av[kProbeSets], bv[kProbeSets];
#pragma unroll
    for (int j = 0; j < kProbeSets; ++j) {
        av[j] = gload_ptr<v4i>(ops)[(2 * j) * 64 + lane];
        bv[j] = gload_ptr<v4i>(ops)[(2 * j + 1) * 64 + lane];
    }
    v16i acc[kProbeSets];
#pragma unroll
    for (int j = 0; j < kProbeSets; ++j) acc[j] = (v16i){};
    const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < kProbeSets; ++j) acc[j] = mfma_i8(av[j], bv[j], acc[j]);
    }
    int32_t s = 0;
#pragma unroll
    for (int j = 0; j < kProbeSets; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[j][e];
    const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    gstore_ptr<int32_t>(sink)[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
    if (threadIdx.x == 0) {
        gstore_ptr<uint64_t>(clocks)[3 * blockIdx.x] = t1 - t0;
        gstore_ptr<uint64_t>(clocks)[3 * blockIdx.x + 1] = r0;
        gstore_ptr<uint64_t>(clocks)[3 * blockIdx.x + 2] = r1;
    }
}

// `rounds` grid-wide barriers among the launch's workgroups (at most one per
// compute unit, so all are resident at once).  At barrier r every workgroup
// publishes one word (r * G + b) with a device-scope store, waits until the
// store has completed, increments the device-scope arrival counter and polls
// it until all G have arrived; then it reads every workgroup's word of round
// r with device-scope loads and adds them up.  Words alternate between two
// slot sets by round parity: a workgroup can overwrite its round-r slot (in
// round r + 2) only after the barrier of round r + 1, which every reader of
// round r has passed.  The poll is bounded: a workgroup that polls
// spin_limit times without seeing everyone counts a give-up and stops, so
// every wave exits whatever the others do.
// state: [0] arrival counter, [1] give-ups, [2 + (r & 1) * G + b] the words.
__global__ __launch_bounds__(kProbeThreads) void probe_barrier_kernel(int rounds, int spin_limit,
                                                                      uint32_t *__restrict__ state,
                                                                      uint32_t *__restrict__ sink)
{
    const int b = blockIdx.x, G = gridDim.x, t = threadIdx.x;
    __shared__ int s_ok;
    uint32_t sum = 0;
    for (int r = 0; r < rounds; ++r) {
        uint32_t *words = state + 2 + (r & 1) * G;
        if (t == 0) __hip_atomic_store(&words[b], (uint32_t)r * G + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);  // the word is at the coherence point
        __syncthreads();
        if (t == 0) {
            __hip_atomic_fetch_add(&state[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint32_t target = (uint32_t)(r + 1) * G;
            int spins = 0;
            while (__hip_atomic_load(&state[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target &&
                   spins < spin_limit) {
                __builtin_amdgcn_s_sleep(1);
                ++spins;
            }
            s_ok = spins < spin_limit;
            if (!s_ok) __hip_atomic_fetch_add(&state[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        if (!s_ok) break;
        for (int i = t; i < G; i += kProbeThreads)
            sum += __hip_atomic_load(&words[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    gstore_ptr<uint32_t>(sink)[(int64_t)b * kProbeThreads + t] = sum;
}

}  // namespace

hipError_t launch_probe_barrier(int rounds, int blocks, int spin_limit, uint32_t *state, uint32_t *sink,
                                hipStream_t s)
{
    hipLaunchKernelGGL(probe_barrier_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0, s, rounds, spin_limit,
                       state, sink);
    return hipGetLastError();
}

hipError_t probe_compute_units(int *cus)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
    return e;
}

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

hipError_t launch_probe_mfma_data(int64_t iters, const void *ops, int blocks, int32_t *sink, uint64_t *clocks,
                                  hipStream_t s)
{
    hipLaunchKernelGGL(probe_mfma_data_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0, s, iters,
                       static_cast<const v4i *>(ops), sink, clocks);
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
