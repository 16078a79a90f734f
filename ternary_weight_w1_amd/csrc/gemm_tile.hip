// Tiled int8-MFMA contraction for many tokens (prefill, large decode
// batches).
//
// Same arithmetic as the streaming kernel -- ternary fields times int8
// activations, exact int32 sums, rescale (anthology note-168 on arXiv
// 2402.17764, "What it does" and "The part that is a bet rather than a
// measurement") -- but here 2*M*N*K int8 operations dominate the packed
// weight bytes and the matrix cores set the pace.  The pages call running
// ternary weights through int8 hardware a stopgap until ternary logic
// exists (BitNet b1.58 2B4T video transcript, yousumm.com, "Transcription");
// on gfx950 the int8 matrix instruction v_mfma_i32_32x32x32_i8 is that path.
//
// Work item = (problem, BM-token tile, 256-row weight tile).  Each of the
// four waves owns one 64-row BL2-T64 tile: per 64-code unit it loads its
// 1 KiB block (16 bytes per lane), and the four 2-bit planes of each word
// are directly its MFMA B operands -- the ternary tile is unpacked in
// registers and never takes a trip through LDS.  The activation tile
// (BM x 64 bytes per unit) is shared by the four waves, so it is staged in
// LDS, double buffered, with rows padded to 80 bytes so that the 16-byte
// fragment reads of 8 consecutive lanes hit distinct banks.  Per unit a wave
// issues 4*RM MFMAs against 8 LDS reads and one global load.
#include "mm_common.hpp"

namespace bl {
namespace {

constexpr int kThreads = 256;
constexpr int kLda = 80;  // padded LDS row stride of the activation tile

template <int RM>
__device__ void tile_body(const Problem &p, int local)
{
    constexpr int BM = 32 * RM;
    constexpr int CH = BM * 4 / kThreads;  // 16-byte activation chunks per thread per unit
    static_assert(CH >= 1, "tile too small for the staging pattern");
    __shared__ __attribute__((aligned(16))) int8_t As[2][BM * kLda];

    const int mtile = local % p.mt;
    const int nt = local / p.mt;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, g = lane >> 5, r = lane & 31;
    const int tile = 4 * nt + wave;
    const bool wv = tile < p.NT;
    const v4u *blk =
        reinterpret_cast<const v4u *>(p.P + (int64_t)(wv ? tile : 0) * p.KU * kBlockBytes) + lane;
    const int m0 = mtile * BM;
    const int KU = p.KU;
    const v4i zero = {0, 0, 0, 0};
    const v4u zero_codes = {0x55555555u, 0x55555555u, 0x55555555u, 0x55555555u};

    v4i areg[CH];
    auto load_a = [&](int u) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = tid + kThreads * i;
            const int m = m0 + (c >> 2);
            areg[i] = (m < p.M)
                          ? *reinterpret_cast<const v4i *>(p.Q + (int64_t)m * p.ldq + 64 * u + 16 * (c & 3))
                          : zero;
        }
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = tid + kThreads * i;
            *reinterpret_cast<v4i *>(&As[buf][(c >> 2) * kLda + 16 * (c & 3)]) = areg[i];
        }
    };

    v16i acc[RM][2];
#pragma unroll
    for (int i = 0; i < RM; ++i) acc[i][0] = acc[i][1] = (v16i){};

    load_a(0);
    store_a(0);
    v4u w = wv ? load_packed(blk) : zero_codes;
    __syncthreads();

    for (int u = 0; u < KU; ++u) {
        const int buf = u & 1;
        const bool more = u + 1 < KU;
        v4u wn = zero_codes;
        if (more) {
            load_a(u + 1);
            if (wv) wn = load_packed(blk + (int64_t)(u + 1) * 64);
        }
        const v4i b00 = planes(w.x), b01 = planes(w.y), b10 = planes(w.z), b11 = planes(w.w);
#pragma unroll
        for (int i = 0; i < RM; ++i) {
            const int8_t *arow = &As[buf][(32 * i + r) * kLda + 16 * g];
            const v4i a0 = *reinterpret_cast<const v4i *>(arow);
            const v4i a1 = *reinterpret_cast<const v4i *>(arow + 32);
            acc[i][0] = mfma_i8(a0, b00, acc[i][0]);
            acc[i][0] = mfma_i8(a1, b01, acc[i][0]);
            acc[i][1] = mfma_i8(a0, b10, acc[i][1]);
            acc[i][1] = mfma_i8(a1, b11, acc[i][1]);
        }
        if (more) {
            store_a(buf ^ 1);
            w = wn;
        }
        __syncthreads();
    }

    if (!wv) return;
    const float gamma = *p.gamma;
#pragma unroll
    for (int i = 0; i < RM; ++i) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int n = 64 * tile + 32 * s + r;
            if (n >= p.N) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int m = m0 + 32 * i + 8 * (e >> 2) + 4 * g + (e & 3);
                if (m < p.M) finish_output(p, gamma, m, n, acc[i][s][e]);
            }
        }
    }
}

template <int V>
__device__ inline void tile_dispatch(const Problem &p, int local)
{
    if constexpr (V == 0)
        tile_body<2>(p, local);
    else
        tile_body<4>(p, local);
}

template <int V>
__global__ __launch_bounds__(kThreads) void tile_single_kernel(Problem p)
{
    tile_dispatch<V>(p, blockIdx.x);
}

template <int V>
__global__ __launch_bounds__(kThreads) void tile_group_kernel(const Problem *__restrict__ probs,
                                                              const uint32_t *__restrict__ item_map)
{
    const Problem &p = probs[item_map[blockIdx.x]];
    tile_dispatch<V>(p, (int)blockIdx.x - p.item_begin);
}

}  // namespace

hipError_t launch_tile_single(const Problem &p, int variant, hipStream_t s)
{
    const dim3 grid((unsigned)(p.mt * p.ntt)), block(kThreads);
    if (variant == 0)
        hipLaunchKernelGGL(tile_single_kernel<0>, grid, block, 0, s, p);
    else
        hipLaunchKernelGGL(tile_single_kernel<1>, grid, block, 0, s, p);
    return hipGetLastError();
}

hipError_t launch_tile_group(const Problem *probs, const uint32_t *item_map, int n_items,
                             int variant, hipStream_t s)
{
    const dim3 grid((unsigned)n_items), block(kThreads);
    if (variant == 0)
        hipLaunchKernelGGL(tile_group_kernel<0>, grid, block, 0, s, probs, item_map);
    else
        hipLaunchKernelGGL(tile_group_kernel<1>, grid, block, 0, s, probs, item_map);
    return hipGetLastError();
}

}  // namespace bl
