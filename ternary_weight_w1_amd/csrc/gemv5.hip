// Streaming contraction over BT5-T32 weights (five ternary codes per byte,
// bt5.hpp), for up to 16 tokens per pass: acc[m, n] = sum_k T[n, k] Q[m, k]
// exact in int32, then the rescale epilogue.
//
// The base-3 decode is the expensive part, so it is cut to one multiply and
// one byte select per prefix plane (bt5_planes), and the linear part of the
// contraction goes to the matrix cores.  For one packed byte with digits d_i
// and prefix integers H_j = floor(s 3^j / 256):
//     sum_i d_i q_i = sum_(j=1..3) H_j (q_(j-1) - 3 q_j) + H_4 q_3 + d_4 q_4
// (d_4 = H_5 - 3 H_4), where q_i is the activation of the code at digit i.
// Each of the five planes (H_1, H_2, H_3, H_4, d_4) is the B operand of one
// 32x32x32 int8 matrix instruction; the A operand holds, for token m, the
// activations of the plane's first coefficient in row 2m and of its second
// (times -3 after the product) in row 2m + 1.  With the layout of bt5.hpp the
// A operand of a lane is 16 contiguous bytes of a Q row: digit i of packed
// bytes p = 0..15 of slot half g are codes 160 u + 32 i + 16 g + p.
// out[2m] - 3 out[2m+1] is then sum_k (t + 1) q; the row sum of Q is taken
// off in the epilogue as for the 2-bit kernels.
//
// Work item: (group of four 32-row tiles, group of 16 tokens, K split); each
// wave owns one tile and walks the split's 160-code units with three or four
// units in flight.  Per unit a wave loads the packed block (16 bytes a lane) and the
// unit's activation rows -- ten 16-byte chunks per token, spread over the
// lanes, NA = ceil(10 * tokens / 64) loads -- into a private LDS slot; the
// five A operands are then LDS reads (rows of absent tokens and the zero
// second rows of planes 4 and 5 read a zero patch).  Five operand loads per
// unit straight from memory would occupy the vector memory path five times
// longer than the weights do.  Loads are raw buffer loads: lanes past the
// data get an offset past the resource and read zeros, and a unit past the
// split's end is read that way too, so it decodes to all-zero planes; the
// loop has no branches and no barriers.
#include "bt5.hpp"
#include "mm_common.hpp"

namespace bl {
namespace {

constexpr int kThreads = 256;  // four waves, one tile each

// Units loaded ahead per wave: four, or three when three activation loads
// per unit would push the wave past 128 VGPRs (four waves per SIMD).
template <int NA>
constexpr int ring_of() { return NA >= 3 ? 3 : 4; }

// LDS of one wave: the ring's slots of NA KiB (chunk i of a slot at 16 i) and
// a 16-byte zero patch after them.
template <int NA>
constexpr int wave_lds_bytes() { return ring_of<NA>() * NA * 1024 + 16; }

template <int NA>
__device__ __forceinline__ void bt5_body(const Problem &p, int local)
{
    constexpr int kRing = ring_of<NA>();
    __shared__ __attribute__((aligned(16))) int8_t lds[4 * wave_lds_bytes<NA>()];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // problem fields as wave-uniform values (they feed buffer resources and
    // scalar offsets)
    const int ks = uni(p.ks), ntt = uni(p.ntt), NT = uni(p.NT), KU5 = uni(p.KU5);
    const int M = uni(p.M), ldq = uni((int)p.ldq);
    const int split = uni(local % ks);
    const int rest = uni(local / ks);
    const int grp = rest % ntt;
    const int tg = rest / ntt;
    const int tile = uni(4 * grp + wave);
    const bool tv = tile < NT;
    const int u0 = uni(split * p.upsplit);
    const int u1 = uni(min(KU5, u0 + p.upsplit));
    const int m0 = tg * kBt5Tokens;
    const int mg = uni(min(kBt5Tokens, M - m0));
    const int c = lane >> 5;

    v16i acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0;

    if (tv) {
        int8_t *wl = lds + wave * wave_lds_bytes<NA>();
        constexpr int kZero = kRing * NA * 1024;
        if (lane == 0) *reinterpret_cast<v4i *>(wl + kZero) = (v4i){0, 0, 0, 0};
        const int bbytes = KU5 * kBlockBytes;
        const uint8_t *wp = static_cast<const uint8_t *>(uni(p.P));
        const int8_t *qp = static_cast<const int8_t *>(uni(p.Q));
        const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(wp + (int64_t)tile * KU5 * kBlockBytes, bbytes);
        const int qbytes = mg * ldq;
        const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(qp + (int64_t)m0 * ldq, qbytes);
        // chunk i = 10 m + q (token m, 16-byte chunk q of its 160-byte unit
        // row) is loaded by lane i % 64 in load i / 64
        int coff[NA];
#pragma unroll
        for (int a = 0; a < NA; ++a) {
            const int i = lane + 64 * a, m = i / 10, q = i - 10 * m;
            coff[a] = m < mg ? m * ldq + 16 * q : qbytes;
        }
        // A row r = 2 m + h of this lane, chunk half c: plane j reads chunk
        // 2 (j + h) + c of token m (h = 1 only for planes 1..3)
        const int r = lane & 31, ml = r >> 1, h = r & 1;
        int aoff[5];
#pragma unroll
        for (int j = 0; j < 5; ++j)
            aoff[j] = (ml < mg && (h == 0 || j <= 2)) ? 16 * (10 * ml + 2 * (j + h) + c) : kZero;
        const int boff = 16 * lane;

        v4u bq[kRing];
        v4i araw[kRing][NA];
        auto load = [&](int s, int u) {
            const int uc = min(u, u1 - 1);
            bq[s] = __builtin_amdgcn_raw_buffer_load_b128(rb, u < u1 ? boff : bbytes, uc * kBlockBytes, 2);
#pragma unroll
            for (int a = 0; a < NA; ++a)
                araw[s][a] = (v4i)__builtin_amdgcn_raw_buffer_load_b128(rq, coff[a], uc * kBt5UnitCodes, 0);
        };
        auto run = [&](int s) {
            int8_t *slot = wl + s * NA * 1024;
#pragma unroll
            for (int a = 0; a < NA; ++a) *reinterpret_cast<v4i *>(slot + 16 * (lane + 64 * a)) = araw[s][a];
            const Bt5Planes p0 = bt5_planes(bq[s].x), p1 = bt5_planes(bq[s].y);
            const Bt5Planes p2 = bt5_planes(bq[s].z), p3 = bt5_planes(bq[s].w);
#pragma unroll
            for (int j = 0; j < 5; ++j) {
                const v4i a = *reinterpret_cast<const v4i *>((aoff[j] == kZero ? wl : slot) + aoff[j]);
                v4i b;
                b.x = (int)p0.h[j];
                b.y = (int)p1.h[j];
                b.z = (int)p2.h[j];
                b.w = (int)p3.h[j];
                acc = mfma_i8(a, b, acc);
            }
        };
        // loads stay in slot order (prologue and loop alike), so each wait
        // for a slot counts only the slots issued after it
#pragma unroll
        for (int s = 0; s < kRing; ++s) {
            load(s, u0 + s);
            __builtin_amdgcn_sched_barrier(0);
        }
        for (int u = u0; u < u1; u += kRing) {
#pragma unroll
            for (int s = 0; s < kRing; ++s) {
                run(s);
                load(s, u + s + kRing);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

    // lane (c, r') holds rows 8 (e / 4) + 4 c + e % 4 of column n: the pair
    // (e, e + 1), e even, is token m's rows 2m and 2m + 1
    const int n = kBt5TileRows * tile + (lane & 31);
    const float gamma = *gload_ptr<float>(p.gamma);
    const int64_t ldp = (int64_t)NT * kBt5TileRows;
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
        const int m = m0 + ((8 * (e >> 2) + 4 * c + (e & 3)) >> 1);
        if (!tv || n >= p.N || m >= M) continue;
        const int32_t v = acc[e] - 3 * acc[e + 1];
        if (ks == 1)
            finish_output(p, gamma, m, n, v);
        else
            put_partial(p.acc_ws + ((int64_t)split * M + m) * ldp + n, v);
    }
    if (ks == 1) return;
    if (!arrive_last(p, rest)) return;
    int64_t off[8];
    bool ok[8];
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
        const int m = m0 + ((8 * (e >> 2) + 4 * c + (e & 3)) >> 1);
        ok[e >> 1] = tv && n < p.N && m < M;
        off[e >> 1] = (int64_t)m * ldp + n;
    }
    int32_t sums[8];
    sum_partials<8>(p.acc_ws, off, ok, (int64_t)M * ldp, ks, sums);
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
        const int m = m0 + ((8 * (e >> 2) + 4 * c + (e & 3)) >> 1);
        if (ok[e >> 1]) finish_output(p, gamma, m, n, sums[e >> 1]);
    }
}

template <int NA>
__global__ __launch_bounds__(kThreads, 2) void bt5_single_kernel(Problem p)
{
    bt5_body<NA>(p, (int)blockIdx.x);
}

template <int NA>
__global__ __launch_bounds__(kThreads, 2) void bt5_group_kernel(const Problem *__restrict__ probs,
                                                                const uint2 *__restrict__ item_map)
{
    const uint2 it = item_map[blockIdx.x];
    if (it.x != 0xFFFFFFFFu) bt5_body<NA>(probs[it.x], (int)it.y);
}

template <int NA>
__global__ __launch_bounds__(kThreads, 2) void bt5_multi_kernel(ProblemSet ps)
{
    const int i = multi_index(ps, blockIdx.x);
    bt5_body<NA>(ps.p[i], (int)blockIdx.x - ps.begin[i]);
}

}  // namespace

int bt5_chunk_loads(int max_tokens)
{
    const int m = max_tokens < kBt5Tokens ? max_tokens : kBt5Tokens;
    return (10 * m + 63) / 64;
}

hipError_t launch_bt5_single(const Problem &p, hipStream_t s)
{
    const dim3 grid((unsigned)((int64_t)p.ntt * p.mt * p.ks)), block(kThreads);
    switch (bt5_chunk_loads(p.M)) {
    case 1: hipLaunchKernelGGL(bt5_single_kernel<1>, grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL(bt5_single_kernel<2>, grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL(bt5_single_kernel<3>, grid, block, 0, s, p); break;
    }
    return hipGetLastError();
}

hipError_t launch_bt5_group(const Problem *probs, const uint2 *item_map, int n_items, int max_tokens,
                            hipStream_t s)
{
    const dim3 grid((unsigned)n_items), block(kThreads);
    switch (bt5_chunk_loads(max_tokens)) {
    case 1: hipLaunchKernelGGL(bt5_group_kernel<1>, grid, block, 0, s, probs, item_map); break;
    case 2: hipLaunchKernelGGL(bt5_group_kernel<2>, grid, block, 0, s, probs, item_map); break;
    default: hipLaunchKernelGGL(bt5_group_kernel<3>, grid, block, 0, s, probs, item_map); break;
    }
    return hipGetLastError();
}

hipError_t launch_bt5_multi(const ProblemSet &ps, int max_tokens, hipStream_t s)
{
    const dim3 grid((unsigned)ps.begin[ps.count]), block(kThreads);
    switch (bt5_chunk_loads(max_tokens)) {
    case 1: hipLaunchKernelGGL(bt5_multi_kernel<1>, grid, block, 0, s, ps); break;
    case 2: hipLaunchKernelGGL(bt5_multi_kernel<2>, grid, block, 0, s, ps); break;
    default: hipLaunchKernelGGL(bt5_multi_kernel<3>, grid, block, 0, s, ps); break;
    }
    return hipGetLastError();
}

}  // namespace bl
