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
// issues 4*RM MFMAs against 2*RM LDS reads and one global load.
//
// Latency: global loads run D units ahead of the MFMAs through register
// rings (activation chunks and packed words), the activation chunk of unit
// u+1 is written to LDS behind unit u's MFMAs, and one barrier per unit
// separates the two LDS buffers.
#include "mm_common.hpp"

namespace bl {
namespace {

constexpr int kThreads = 256;
constexpr int kLda = 80;  // padded LDS row stride of the activation tile
constexpr int kDepth = 3; // units of global-load lookahead

template <int RM>
__device__ void tile_body(const Problem &p, int local)
{
    constexpr int BM = 32 * RM;
    constexpr int CH = BM * 4 / kThreads;  // 16-byte activation chunks per thread per unit
    static_assert(CH >= 1, "tile too small for the staging pattern");
    __shared__ __attribute__((aligned(16))) int8_t As[2][BM * kLda];
    __shared__ float cs[BM];
    __shared__ int rsum[BM];

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
    const v4u zero_codes = {0x55555555u, 0x55555555u, 0x55555555u, 0x55555555u};

    // activation chunk c of a unit: row c/4, 16 bytes at 16*(c%4); rows past
    // M read row M-1 (their results are never stored)
    const int8_t *asrc[CH];
    int adst[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int c = tid + kThreads * i;
        const int m = min(m0 + (c >> 2), p.M - 1);
        asrc[i] = p.Q + (int64_t)m * p.ldq + 16 * (c & 3);
        adst[i] = (c >> 2) * kLda + 16 * (c & 3);
    }

    if (tid < BM) {
        const int m = min(m0 + tid, p.M - 1);
        cs[tid] = (*p.gamma * p.absmax[m]) / 127.0f;
        rsum[tid] = p.rowsum[m];
    }

    v4i ar[kDepth][CH];
    v4u br[kDepth];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
        if (d < KU) {
#pragma unroll
            for (int i = 0; i < CH; ++i) ar[d][i] = *reinterpret_cast<const v4i *>(asrc[i] + 64 * d);
            br[d] = wv ? load_packed(blk + (int64_t)d * 64) : zero_codes;
        }
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) *reinterpret_cast<v4i *>(&As[0][adst[i]]) = ar[0][i];
    __syncthreads();

    v16i acc[RM][2];
#pragma unroll
    for (int i = 0; i < RM; ++i) acc[i][0] = acc[i][1] = (v16i){};

    for (int u0 = 0; u0 < KU; u0 += kDepth) {
#pragma unroll
        for (int s = 0; s < kDepth; ++s) {
            const int u = u0 + s;
            if (u >= KU) break;
            const int buf = u & 1;
            const v4u w = br[s];
            const v4i b00 = planes(w.x), b01 = planes(w.y), b10 = planes(w.z), b11 = planes(w.w);
            if (u + kDepth < KU) {
#pragma unroll
                for (int i = 0; i < CH; ++i)
                    ar[s][i] = *reinterpret_cast<const v4i *>(asrc[i] + 64 * (u + kDepth));
                if (wv) br[s] = load_packed(blk + (int64_t)(u + kDepth) * 64);
            }
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
            if (u + 1 < KU) {
                const int ns = (s + 1) % kDepth;
#pragma unroll
                for (int i = 0; i < CH; ++i) *reinterpret_cast<v4i *>(&As[buf ^ 1][adst[i]]) = ar[ns][i];
            }
            __syncthreads();
        }
    }

    if (!wv) return;
#pragma unroll
    for (int i = 0; i < RM; ++i) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int n = 64 * tile + 32 * s + r;
            if (n >= p.N) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = 32 * i + 8 * (e >> 2) + 4 * g + (e & 3);
                const int m = m0 + row;
                if (m < p.M) {
                    const int32_t a = acc[i][s][e] - rsum[row];
                    const int64_t o = (int64_t)m * p.N + n;
                    p.Y[o] = (float)a * cs[row];
                    if (p.acc_out) p.acc_out[o] = a;
                }
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

// Workgroup b runs on XCD b % 8; the logical item order is split into eight
// contiguous slices, one per XCD, so the tiles that share activation rows
// and packed weight columns meet in the same L2.
__device__ inline int xcd_logical(int b, int per)
{
    return (b & 7) * per + (b >> 3);
}

// 128-token tiles hold 128 accumulators per lane and run one wave per SIMD;
// 64-token tiles fit two.
template <int V>
__global__ __launch_bounds__(kThreads, V == 0 ? 2 : 1) void tile_single_kernel(Problem p, int items, int per)
{
    const int j = xcd_logical(blockIdx.x, per);
    if (j >= items) return;
    tile_dispatch<V>(p, j);
}

template <int V>
__global__ __launch_bounds__(kThreads, V == 0 ? 2 : 1) void tile_group_kernel(const Problem *__restrict__ probs,
                                                                 const uint2 *__restrict__ item_map)
{
    const uint2 it = item_map[blockIdx.x];
    if (it.x == 0xFFFFFFFFu) return;
    tile_dispatch<V>(probs[it.x], (int)it.y);
}

}  // namespace

hipError_t launch_tile_single(const Problem &p, int variant, hipStream_t s)
{
    const int items = p.mt * p.ntt;
    const int per = (items + 7) / 8;
    const dim3 grid((unsigned)(8 * per)), block(kThreads);
    if (variant == 0)
        hipLaunchKernelGGL(tile_single_kernel<0>, grid, block, 0, s, p, items, per);
    else
        hipLaunchKernelGGL(tile_single_kernel<1>, grid, block, 0, s, p, items, per);
    return hipGetLastError();
}

hipError_t launch_tile_group(const Problem *probs, const uint2 *item_map, int n_items,
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
