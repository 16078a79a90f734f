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
// Work item = (problem, BM-token tile, 256-row weight tile).  Each wave owns
// one or two 64-row BL2-T64 tiles: per 64-code unit it loads each tile's
// 1 KiB block (16 bytes per lane), and the four 2-bit planes of each word
// are directly its MFMA B operands -- the ternary tile is unpacked in
// registers and never takes a trip through LDS.  The activation tile
// (BM x 64 bytes per unit) is shared by the waves, so it is staged in LDS,
// double buffered, with rows padded to 80 bytes so that the 16-byte fragment
// reads of 8 consecutive lanes hit distinct banks.
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

// WMS: 32-token subtiles per wave; WNT: 64-row weight tiles per wave;
// WAVES_M x (4 / WAVES_M) waves.  The workgroup covers BM = WAVES_M*WMS*32
// tokens and always 256 weight rows.
// FRAG: the activations arrive in fragment order (see qf32_offset) and are
// staged into LDS unchanged, so the global loads are whole 1 KiB blocks and
// both the LDS writes and the operand reads are linear (conflict-free,
// unpadded); otherwise row-major activations are staged into padded rows.
template <int WMS, int WNT, int WAVES_M, bool FRAG>
__device__ void tile_body(const Problem &p, int local)
{
    constexpr int WAVES_N = 4 / WAVES_M;
    static_assert(WAVES_N * WNT == 4, "a workgroup spans 256 weight rows");
    constexpr int BM = WAVES_M * WMS * 32;
    constexpr int CH = BM * 4 / kThreads;  // 16-byte activation chunks per thread per unit
    static_assert(CH >= 1, "tile too small for the staging pattern");
    constexpr int kRowBytes = FRAG ? 64 : kLda;
    __shared__ __attribute__((aligned(16))) int8_t As[2][BM * kRowBytes];
    __shared__ float cs[BM];
    __shared__ int rsum[BM];

    const int mtile = local % p.mt;
    const int nt = local / p.mt;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, g = lane >> 5, r = lane & 31;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int m0 = mtile * BM;
    const int KU = p.KU;
    const v4u zero_codes = {0x55555555u, 0x55555555u, 0x55555555u, 0x55555555u};

    // weight tiles past NT load tile NT-1 (valid memory; never stored)
    int tile[WNT];
    bool tv[WNT];
    const BL_GLOBAL v4u *blk[WNT];
#pragma unroll
    for (int j = 0; j < WNT; ++j) {
        tile[j] = 4 * nt + wn * WNT + j;
        tv[j] = tile[j] < p.NT;
        blk[j] = gload_ptr<v4u>(p.P + (int64_t)min(tile[j], p.NT - 1) * KU * kBlockBytes) + lane;
    }

    // activation chunk c of a unit: row c/4, 16 bytes at 16*(c%4); rows past
    // M read row M-1 (their results are never stored)
    // fragment order: chunk c is 16 bytes at 16*(c%128) of the 2 KiB
    // (block m0/32 + c/128, unit) pair of 1 KiB fragments; blocks past the
    // last one re-read the last (never stored)
    const BL_GLOBAL int8_t *asrc[CH];
    int adst[CH];
    int64_t astep;  // bytes between consecutive units
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int c = tid + kThreads * i;
        if constexpr (FRAG) {
            const int64_t b = min((m0 >> 5) + (c >> 7), ((p.M + 31) >> 5) - 1);
            asrc[i] = gload_ptr<int8_t>(p.Q + b * KU * 2048 + 16 * (c & 127));
            adst[i] = 16 * c;
        } else {
            const int m = min(m0 + (c >> 2), p.M - 1);
            asrc[i] = gload_ptr<int8_t>(p.Q + (int64_t)m * p.ldq + 16 * (c & 3));
            adst[i] = (c >> 2) * kLda + 16 * (c & 3);
        }
    }
    astep = FRAG ? 2048 : 64;

    __syncthreads();  // the previous work item of this workgroup may still read LDS
    if (tid < BM) {
        const int m = min(m0 + tid, p.M - 1);
        cs[tid] = (*gload_ptr<float>(p.gamma) * gload_ptr<float>(p.absmax)[m]) / 127.0f;
        rsum[tid] = gload_ptr<int32_t>(p.rowsum)[m];
    }

    // Register rings: slot s holds unit u with u % kDepth == s.  Every load
    // is unconditional (unit indices clamp to KU-1, a harmless re-read at
    // the end) so the loop body has no branches and the compiler keeps the
    // slots in fixed registers with precise wait counts.
    v4i ar[kDepth][CH];
    v4u br[kDepth][WNT];
    auto load_unit = [&](int slot, int u) {
        const int uc = min(u, KU - 1);
#pragma unroll
        for (int i = 0; i < CH; ++i) ar[slot][i] = *reinterpret_cast<const BL_GLOBAL v4i *>(asrc[i] + astep * uc);
#pragma unroll
        for (int j = 0; j < WNT; ++j) br[slot][j] = blk[j][(int64_t)uc * 64];
    };
#pragma unroll
    for (int d = 0; d < kDepth; ++d) load_unit(d, d);
#pragma unroll
    for (int i = 0; i < CH; ++i) *reinterpret_cast<v4i *>(&As[0][adst[i]]) = ar[0][i];
    __syncthreads();

    v16i acc[WMS][2 * WNT];
#pragma unroll
    for (int i = 0; i < WMS; ++i)
#pragma unroll
        for (int j = 0; j < 2 * WNT; ++j) acc[i][j] = (v16i){};

    const int arow0 = wm * WMS * 32;
    // one unit: MFMAs on LDS buffer u&1 and ring slot s, refill slot s with
    // unit u+kDepth, stage unit u+1's activations into the other buffer
    auto step = [&](int s, int u) {
        const int buf = u & 1;
        v4i b[WNT][4];
#pragma unroll
        for (int j = 0; j < WNT; ++j) {
            const v4u w = br[s][j];
            b[j][0] = planes(w.x);
            b[j][1] = planes(w.y);
            b[j][2] = planes(w.z);
            b[j][3] = planes(w.w);
        }
        v4i a[WMS][2];
#pragma unroll
        for (int i = 0; i < WMS; ++i) {
            if constexpr (FRAG) {
                const int8_t *f = &As[buf][((arow0 >> 5) + i) * 2048 + 16 * lane];
                a[i][0] = *reinterpret_cast<const v4i *>(f);
                a[i][1] = *reinterpret_cast<const v4i *>(f + 1024);
            } else {
                const int8_t *arow = &As[buf][(arow0 + 32 * i + r) * kLda + 16 * g];
                a[i][0] = *reinterpret_cast<const v4i *>(arow);
                a[i][1] = *reinterpret_cast<const v4i *>(arow + 32);
            }
        }
        load_unit(s, u + kDepth);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < WMS; ++i)
#pragma unroll
                for (int j = 0; j < WNT; ++j) {
                    acc[i][2 * j] = mfma_i8(a[i][h], b[j][h], acc[i][2 * j]);
                    acc[i][2 * j + 1] = mfma_i8(a[i][h], b[j][2 + h], acc[i][2 * j + 1]);
                }
        const int ns = (s + 1) % kDepth;
#pragma unroll
        for (int i = 0; i < CH; ++i) *reinterpret_cast<v4i *>(&As[buf ^ 1][adst[i]]) = ar[ns][i];
        __syncthreads();
    };
    int u0 = 0;
    for (; u0 + kDepth <= KU; u0 += kDepth) {
#pragma unroll
        for (int s = 0; s < kDepth; ++s) step(s, u0 + s);
    }
#pragma unroll
    for (int s = 0; s < kDepth - 1; ++s)
        if (u0 + s < KU) step(s, u0 + s);

#pragma unroll
    for (int j = 0; j < WNT; ++j) {
        if (!tv[j]) continue;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const int n = 64 * tile[j] + 32 * s2 + r;
            if (n >= p.N) continue;
#pragma unroll
            for (int i = 0; i < WMS; ++i) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = arow0 + 32 * i + 8 * (e >> 2) + 4 * g + (e & 3);
                    const int m = m0 + row;
                    if (m < p.M) {
                        const int32_t a = acc[i][2 * j + s2][e] - rsum[row];
                        const int64_t o = (int64_t)m * p.N + n;
                        gstore_ptr<float>(p.Y)[o] = (float)a * cs[row];
                        if (p.acc_out) gstore_ptr<int32_t>(p.acc_out)[o] = a;
                    }
                }
            }
        }
    }
}

// Barrier-free variant: every wave loads its own MFMA A operands straight
// from global memory (fragment-ordered activations: one contiguous 1 KiB
// load per operand; row-major activations: two 32-byte row pieces per lane
// pair) next to its packed weight block, through a kDirect-deep register
// ring.  The four waves of a workgroup share their 128 token rows through
// L1 instead of LDS, so there is no LDS staging, no bank conflict and no
// per-unit barrier; one wave per SIMD, latency covered by the ring depth.
constexpr int kDirect = 4;

template <bool TILED>
__device__ void tile_direct_body(const Problem &p, int local)
{
    constexpr int WMS = 4;       // 32-token subtiles per wave (128 tokens)
    constexpr int BM = 32 * WMS;
    __shared__ float cs[BM];
    __shared__ int rsum[BM];

    const int mtile = local % p.mt;
    const int nt = local / p.mt;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, g = lane >> 5, r = lane & 31;
    const int m0 = mtile * BM;
    const int KU = p.KU;
    const int tile = 4 * nt + wave;
    const bool tv = tile < p.NT;
    const BL_GLOBAL v4u *blk = gload_ptr<v4u>(p.P + (int64_t)min(tile, p.NT - 1) * KU * kBlockBytes) + lane;

    // A operand (i, h) of unit u:
    //   TILED: block min(m0/32 + i, last block), 16 bytes at 16*lane
    //   row-major: row min(m0 + 32 i + r, M - 1), bytes 64u + 32h + 16g
    const BL_GLOBAL v4i *abase[WMS];
#pragma unroll
    for (int i = 0; i < WMS; ++i) {
        if constexpr (TILED) {
            const int64_t b = min((m0 >> 5) + i, ((p.M + 31) >> 5) - 1);
            abase[i] = gload_ptr<v4i>(p.Q + b * KU * 2048) + lane;
        } else {
            const int64_t m = min(m0 + 32 * i + r, p.M - 1);
            abase[i] = gload_ptr<v4i>(p.Q + m * p.ldq + 16 * g);
        }
    }

    __syncthreads();  // the previous work item of this workgroup may still read LDS
    if (tid < BM) {
        const int m = min(m0 + tid, p.M - 1);
        cs[tid] = (*gload_ptr<float>(p.gamma) * gload_ptr<float>(p.absmax)[m]) / 127.0f;
        rsum[tid] = gload_ptr<int32_t>(p.rowsum)[m];
    }
    __syncthreads();

    v4i ar[kDirect][WMS][2];
    v4u br[kDirect];
    auto load_unit = [&](int slot, int u) {
        const int uc = min(u, KU - 1);
#pragma unroll
        for (int i = 0; i < WMS; ++i)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if constexpr (TILED)
                    ar[slot][i][h] = abase[i][(int64_t)(2 * uc + h) * 64];
                else
                    ar[slot][i][h] = abase[i][4 * uc + 2 * h];
            }
        br[slot] = blk[(int64_t)uc * 64];
    };
#pragma unroll
    for (int d = 0; d < kDirect; ++d) load_unit(d, d);

    v16i acc[WMS][2];
#pragma unroll
    for (int i = 0; i < WMS; ++i) acc[i][0] = acc[i][1] = (v16i){};

    auto step = [&](int s, int u) {
        const v4u w = br[s];
        const v4i b0 = planes(w.x), b1 = planes(w.y), b2 = planes(w.z), b3 = planes(w.w);
        v4i a[WMS][2];
#pragma unroll
        for (int i = 0; i < WMS; ++i) {
            a[i][0] = ar[s][i][0];
            a[i][1] = ar[s][i][1];
        }
        load_unit(s, u + kDirect);
#pragma unroll
        for (int i = 0; i < WMS; ++i) {
            acc[i][0] = mfma_i8(a[i][0], b0, acc[i][0]);
            acc[i][1] = mfma_i8(a[i][0], b2, acc[i][1]);
        }
#pragma unroll
        for (int i = 0; i < WMS; ++i) {
            acc[i][0] = mfma_i8(a[i][1], b1, acc[i][0]);
            acc[i][1] = mfma_i8(a[i][1], b3, acc[i][1]);
        }
    };
    int u0 = 0;
    for (; u0 + kDirect <= KU; u0 += kDirect) {
#pragma unroll
        for (int s = 0; s < kDirect; ++s) step(s, u0 + s);
    }
#pragma unroll
    for (int s = 0; s < kDirect - 1; ++s)
        if (u0 + s < KU) step(s, u0 + s);

    if (!tv) return;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
        const int n = 64 * tile + 32 * s2 + r;
        if (n >= p.N) continue;
#pragma unroll
        for (int i = 0; i < WMS; ++i) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = 32 * i + 8 * (e >> 2) + 4 * g + (e & 3);
                const int m = m0 + row;
                if (m < p.M) {
                    const int32_t a = acc[i][s2][e] - rsum[row];
                    const int64_t o = (int64_t)m * p.N + n;
                    gstore_ptr<float>(p.Y)[o] = (float)a * cs[row];
                    if (p.acc_out) gstore_ptr<int32_t>(p.acc_out)[o] = a;
                }
            }
        }
    }
}

// Variant 0: 64 tokens x 256 rows, each wave 64 x 64 (four waves along N).
// Variant 1: 128 tokens x 256 rows, each wave 64 x 128 (2 x 2 waves): half
// the LDS reads and L2 reads per MFMA of variant 0.
// Variant 3: the barrier-free direct kernel on fragment-ordered
// activations; variant 4: the same on row-major activations.
template <int V>
__device__ inline void tile_dispatch(const Problem &p, int local)
{
    if constexpr (V == 0)
        tile_body<2, 1, 1, false>(p, local);
    else if constexpr (V == 1)
        tile_body<2, 2, 2, false>(p, local);
    else if constexpr (V == 2)
        tile_body<4, 1, 1, false>(p, local);
    else if constexpr (V == 3)
        tile_direct_body<true>(p, local);
    else if constexpr (V == 4)
        tile_direct_body<false>(p, local);
    else if constexpr (V == 5)
        tile_body<4, 1, 1, true>(p, local);
    else if constexpr (V == 6)
        tile_body<2, 1, 1, true>(p, local);
    else
        tile_body<2, 2, 2, true>(p, local);
}

template <int V>
constexpr int tile_min_waves()
{
    return (V == 3 || V == 4) ? 1 : 2;
}

// Workgroup b runs on XCD b % 8; the logical item order is split into eight
// contiguous slices, one per XCD (slot b stands for logical item
// (b % 8) * per + b / 8), so the tiles that share activation rows and packed
// weight columns meet in the same L2.
__device__ inline int xcd_logical(int b, int per)
{
    return (b & 7) * per + (b >> 3);
}

template <int V>
__global__ __launch_bounds__(kThreads, tile_min_waves<V>()) void tile_single_kernel(Problem p, int items, int per)
{
    const int j = xcd_logical(blockIdx.x, per);
    if (j < items) tile_dispatch<V>(p, j);
}

template <int V>
__global__ __launch_bounds__(kThreads, tile_min_waves<V>()) void tile_group_kernel(const Problem *__restrict__ probs,
                                                                 const uint2 *__restrict__ item_map)
{
    const uint2 it = item_map[blockIdx.x];
    if (it.x != 0xFFFFFFFFu) tile_dispatch<V>(probs[it.x], (int)it.y);
}

}  // namespace

hipError_t launch_tile_single(const Problem &p, int variant, hipStream_t s)
{
    const int items = p.mt * p.ntt;
    const int per = (items + 7) / 8;
    const dim3 grid((unsigned)(8 * per)), block(kThreads);
    switch (variant) {
    case 0: hipLaunchKernelGGL(tile_single_kernel<0>, grid, block, 0, s, p, items, per); break;
    case 1: hipLaunchKernelGGL(tile_single_kernel<1>, grid, block, 0, s, p, items, per); break;
    case 2: hipLaunchKernelGGL(tile_single_kernel<2>, grid, block, 0, s, p, items, per); break;
    case 3: hipLaunchKernelGGL(tile_single_kernel<3>, grid, block, 0, s, p, items, per); break;
    case 4: hipLaunchKernelGGL(tile_single_kernel<4>, grid, block, 0, s, p, items, per); break;
    case 5: hipLaunchKernelGGL(tile_single_kernel<5>, grid, block, 0, s, p, items, per); break;
    case 6: hipLaunchKernelGGL(tile_single_kernel<6>, grid, block, 0, s, p, items, per); break;
    default: hipLaunchKernelGGL(tile_single_kernel<7>, grid, block, 0, s, p, items, per); break;
    }
    return hipGetLastError();
}

hipError_t launch_tile_group(const Problem *probs, const uint2 *item_map, int n_items,
                             int variant, hipStream_t s)
{
    const dim3 grid((unsigned)n_items), block(kThreads);
    switch (variant) {
    case 0: hipLaunchKernelGGL(tile_group_kernel<0>, grid, block, 0, s, probs, item_map); break;
    case 1: hipLaunchKernelGGL(tile_group_kernel<1>, grid, block, 0, s, probs, item_map); break;
    case 2: hipLaunchKernelGGL(tile_group_kernel<2>, grid, block, 0, s, probs, item_map); break;
    case 3: hipLaunchKernelGGL(tile_group_kernel<3>, grid, block, 0, s, probs, item_map); break;
    case 4: hipLaunchKernelGGL(tile_group_kernel<4>, grid, block, 0, s, probs, item_map); break;
    case 5: hipLaunchKernelGGL(tile_group_kernel<5>, grid, block, 0, s, probs, item_map); break;
    case 6: hipLaunchKernelGGL(tile_group_kernel<6>, grid, block, 0, s, probs, item_map); break;
    default: hipLaunchKernelGGL(tile_group_kernel<7>, grid, block, 0, s, probs, item_map); break;
    }
    return hipGetLastError();
}

}  // namespace bl
