// Device helpers shared by the two contraction kernels.
#pragma once

#include "common.hpp"

namespace bl {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));


// The four 2-bit planes of a packed word as four int8x4 words: plane j holds
// the (code + 1) fields of codes 4j..4j+3 as bytes.  Together they are the
// 16 consecutive fields of the word, in code order.
__device__ inline v4i planes(unsigned w)
{
    v4i r;
    r.x = (int)(w & 0x03030303u);
    r.y = (int)((w >> 2) & 0x03030303u);
    r.z = (int)((w >> 4) & 0x03030303u);
    r.w = (int)((w >> 6) & 0x03030303u);
    return r;
}

// The planes of two words at once: one 64-bit shift serves both (the bits a
// word receives from its neighbour land above bit 25 of its top byte, which
// the mask clears), 11 operations instead of 14.
__device__ inline void planes2(unsigned a, unsigned b, v4i &pa, v4i &pb)
{
    const uint64_t ab = ((uint64_t)b << 32) | a;
    const uint64_t m = 0x0303030303030303ull;
    const uint64_t s1 = (ab >> 2) & m, s2 = (ab >> 4) & m, s3 = (ab >> 6) & m;
    pa.x = (int)(a & 0x03030303u);
    pb.x = (int)(b & 0x03030303u);
    pa.y = (int)(uint32_t)s1;
    pb.y = (int)(uint32_t)(s1 >> 32);
    pa.z = (int)(uint32_t)s2;
    pb.z = (int)(uint32_t)(s2 >> 32);
    pa.w = (int)(uint32_t)s3;
    pb.w = (int)(uint32_t)(s3 >> 32);
}

// Streaming read of one 16-byte slot of the packed weights (read once, so
// marked non-temporal).
__device__ inline v4u load_packed(const BL_GLOBAL v4u *p) { return __builtin_nontemporal_load(p); }

__device__ inline v16i mfma_i8(v4i a, v4i b, v16i c)
{
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// Rescale epilogue (anthology note-168 on arXiv 2402.17764, "What it does":
// the layer replaces nn.Linear, so it returns real values).  The kernels
// accumulate sum_k (t+1) q = acc + rowsum; the exact integer acc is
// recovered here, then y = float(acc) * ((gamma * a) / 127) in fp32.
__device__ inline float token_scale(float gamma, float absmax) { return (gamma * absmax) / 127.0f; }
__device__ inline void finish_output_with(const Problem &p, float gamma, int m, int n, int32_t fields,
                                          int32_t rowsum, float absmax)
{
    const int32_t acc = fields - rowsum;
    const float c = token_scale(gamma, absmax);
    const int64_t o = (int64_t)m * p.N + n;
    gstore_ptr<float>(p.Y)[o] = (float)acc * c;
    if (p.acc_out) gstore_ptr<int32_t>(p.acc_out)[o] = acc;
}

// The same with the token's factor c = token_scale(gamma, a) computed once
// per token by the caller (kernels that finish many outputs per token).
__device__ inline void finish_output_scaled(const Problem &p, int m, int n, int32_t fields, int32_t rowsum, float c)
{
    const int32_t acc = fields - rowsum;
    const int64_t o = (int64_t)m * p.N + n;
    gstore_ptr<float>(p.Y)[o] = (float)acc * c;
    if (p.acc_out) gstore_ptr<int32_t>(p.acc_out)[o] = acc;
}

__device__ inline void finish_output(const Problem &p, float gamma, int m, int n, int32_t fields)
{
    finish_output_with(p, gamma, m, n, fields, gload_ptr<int32_t>(p.rowsum)[m],
                       gload_ptr<float>(p.absmax)[m]);
}

// Split-K exchange.  The workgroups of one tile may run on different XCDs,
// each with its own L2, so their int32 partial sums travel as device-scope
// relaxed atomic stores and loads (written through to, and read from, the
// device's coherence point) instead of through fences: a device-scope fence
// writes back and invalidates the whole local L2 in every workgroup.
__device__ inline void put_partial(int32_t *p, int32_t v)
{
    __hip_atomic_store(gstore_ptr<int32_t>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline int32_t get_partial(const int32_t *p)
{
    return __hip_atomic_load(const_cast<BL_GLOBAL int32_t *>(gload_ptr<int32_t>(p)), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}

// Split-K sums of R outputs at once: out[r] = sum_j part[off[r] + j * stride]
// over the ks splits, for the outputs with ok[r].  The loads of four splits
// of all R outputs are issued before any is added, so a thread waits once
// per four splits instead of once per partial (each load crosses to the
// device's coherence point).
template <int R>
__device__ inline void sum_partials(const int32_t *part, const int64_t (&off)[R], const bool (&ok)[R],
                                    int64_t stride, int ks, int32_t (&out)[R])
{
#pragma unroll
    for (int r = 0; r < R; ++r) out[r] = 0;
    int j = 0;
    for (; j + 4 <= ks; j += 4) {
        int32_t v[R][4];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) v[r][i] = ok[r] ? get_partial(part + off[r] + (j + i) * stride) : 0;
#pragma unroll
        for (int r = 0; r < R; ++r) out[r] += (v[r][0] + v[r][1]) + (v[r][2] + v[r][3]);
    }
    for (; j < ks; ++j) {
        int32_t v[R];
#pragma unroll
        for (int r = 0; r < R; ++r) v[r] = ok[r] ? get_partial(part + off[r] + j * stride) : 0;
#pragma unroll
        for (int r = 0; r < R; ++r) out[r] += v[r];
    }
}

// Split-K arrival: every workgroup of a tile publishes its partial sums
// (put_partial), waits until those stores have completed, then takes a
// ticket; the one that takes the last ticket reads every partial
// (get_partial, issued only after its ticket came back) and puts the
// counter back to zero (every other workgroup of the tile has already taken
// its ticket), so the counters are clean for the next launch.
__device__ inline bool arrive_last(const Problem &p, int tile)
{
    __shared__ int s_last;
    __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores are complete
    __syncthreads();
    if (threadIdx.x == 0) {
        BL_GLOBAL uint32_t *t = gstore_ptr<uint32_t>(p.tickets) + tile;
        const unsigned old = __hip_atomic_fetch_add(t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = old == (unsigned)(p.ks - 1);
        if (last) __hip_atomic_store(t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = last ? 1 : 0;
    }
    __syncthreads();
    return s_last != 0;
}

}  // namespace bl
