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
// Work item = (problem, 64-token tile, 256-row weight tile[, K split]).
// Each of the four waves owns one 64-row BL2-T64 tile: per 64-code unit it
// loads the tile's 1 KiB block (16 bytes per lane), and the four 2-bit
// planes of each word are directly its MFMA B operands -- the ternary tile
// is unpacked in registers and never takes a trip through LDS.  The
// activation tile (64 tokens x 64 bytes per unit) is shared by the waves,
// so it is staged in LDS, double buffered, two units per stage and barrier.
// Global loads run two stages ahead of the MFMAs through register rings.
// Four workgroups share a CU (126 VGPRs, about 37 KiB of LDS each), so
// while one stages or stores, three keep the matrix cores busy.
#include <type_traits>

#include "mm_common.hpp"

namespace bl {
namespace {

constexpr int kThreads = 256;
typedef float v4f_t __attribute__((ext_vector_type(4)));
// floats per LDS row of the epilogue transpose of blocks at the edge of Y:
// their rescaled outputs go through LDS, 32 rows at a time per wave, so
// that Y is written with 16-byte stores covering whole 256-byte row pieces
// (interior blocks store straight from the accumulators).  Output stores are
// non-temporal: the fp32 result (M*N*4 bytes, the largest stream of the
// kernel) is written once and must not evict the activation and weight
// tiles that other workgroups still reuse from L2.
constexpr int kEpiStride = 72;

// WMS*32-token x 64-row-per-wave tile with UPS units of K per LDS stage and
// barrier: the fixed cost of a barrier
// round (the wait itself and the LDS read latency before the first MFMA)
// is paid once per UPS units.  A stage's unit past the K range gets an
// all-zero packed word -- zero fields add nothing -- so odd unit counts need
// no branch; its activation chunk re-reads the range's last unit (valid
// memory).
//
// K split (launches with few work items): work item = (item, split), item =
// (M tile, four N tiles); split j covers units [j upsplit, (j + 1) upsplit).
// Each split publishes its 32 WMS accumulators per thread as device-scope
// stores, [item][split][accumulator][thread], takes the item's ticket, and
// the last one adds the other splits into its registers and runs the
// epilogue.  Integer addition is associative: the bits do not depend on the
// order.
// LDS stage rows: 128 bytes (two units of one token) + 16 of padding, so
// that 16 consecutive lanes reading 16 consecutive rows at one 16-byte
// column (the operand reads: lane r reads row r) hit 16 distinct 4-bank
// groups (36 r mod 64 over r = 0..15), and rows r, r + 4, r + 8, r + 12
// start 16 banks apart, so a 16-lane staging write of four whole 64-byte
// row pieces from those rows is conflict-free too (see the chunk map).
constexpr int kLda2 = 144;

template <int UPS, int WMS>
__device__ __forceinline__ void tile_body(const Problem &p, int local)
{
    constexpr int BM = 32 * WMS, CH = BM / 64;  // CH: 16-byte chunks per thread per unit
    constexpr int kRow = 64 * UPS + 16;
    static_assert(UPS == 2 && kRow == kLda2, "stage rows are 128 bytes + padding");
    constexpr int kStageBytes = BM * kRow;
    constexpr int kEpiBytes = 4 * 32 * kEpiStride * 4;
    constexpr int kSmem = 2 * kStageBytes > kEpiBytes ? 2 * kStageBytes : kEpiBytes;
    constexpr int kD = 2;  // stages of global-load lookahead
    __shared__ __attribute__((aligned(16))) int8_t smem[kSmem];
    int8_t (*As)[kStageBytes] = reinterpret_cast<int8_t (*)[kStageBytes]>(smem);
    __shared__ float cs[BM];
    __shared__ __attribute__((aligned(16))) int nrsum[BM];

    const int ks = uni(p.ks), mt = uni(p.mt), NT = uni(p.NT), M = uni(p.M), N = uni(p.N);
    const int ldq = uni((int)p.ldq);  // at most 2^26: 64 rows stay below 2^32 bytes
    const int split = local % ks;
    const int item = local / ks;
    const int mtile = item % mt;
    const int nt = item / mt;
    const int tid = threadIdx.x;
    const int wave = uni(tid >> 6), lane = tid & 63, g = lane >> 5, r = lane & 31;
    const int m0 = mtile * BM;
    const int KU = uni(p.KU);
    const int ub = split * uni(p.upsplit);           // first unit of the split
    const int nu = min(KU, ub + uni(p.upsplit)) - ub;  // its units
    const int KS = (nu + UPS - 1) / UPS;
    const int tile = 4 * nt + wave;
    const bool tv = tile < NT;
    // this wave's 64-row tile over the split's units, read through a buffer
    // resource of exactly those bytes; a unit past them is read through a
    // resource of none, which returns the all-zero word (zero fields add
    // nothing), so odd unit counts and the loads run ahead of the last
    // stage need no selects
    const uint8_t *wp = uni(p.P) + ((int64_t)min(tile, NT - 1) * KU + ub) * kBlockBytes;
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(wp, nu * kBlockBytes), rz = buffer_rsrc(wp, 0);
    const int woff = 16 * lane;
    // the work item's activation rows; every offset stays in them (rows past
    // M re-read row M-1, units past the split re-read its last unit)
    const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(uni(p.Q) + (int64_t)m0 * ldq, -1);

    // 16-byte chunk c of a unit: column c % 4 of token row ((c / 16) % 4) +
    // 4 ((c / 4) % 4) + 16 (c / 64): four consecutive lanes read one
    // contiguous 64-byte row piece, a wave reads 16 whole row pieces, and
    // each 16-lane group of the LDS writes covers rows r, r+4, r+8, r+12
    // (rows past M re-read row M-1; their results are never stored)
    int aoff[CH];
    int adst[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int c = tid + kThreads * i;
        const int row = ((c >> 4) & 3) + 4 * ((c >> 2) & 3) + 16 * (c >> 6), col = c & 3;
        aoff[i] = (min(m0 + row, M - 1) - m0) * ldq + 16 * col;
        adst[i] = row * kRow + 16 * col;
    }

    v4i ar[kD][UPS][CH];
    v4u br[kD][UPS];
    auto load_stage = [&](int slot, int st) {
#pragma unroll
        for (int h = 0; h < UPS; ++h) {
            const int u = st * UPS + h;
            const int uc = ub + min(u, nu - 1);
#pragma unroll
            for (int i = 0; i < CH; ++i)
                ar[slot][h][i] = (v4i)__builtin_amdgcn_raw_buffer_load_b128(rq, aoff[i], 64 * uc, 0);
            br[slot][h] = __builtin_amdgcn_raw_buffer_load_b128(u < nu ? rw : rz, woff, u * kBlockBytes, 0);
        }
    };
    auto stage_lds = [&](int buf, int slot) {
#pragma unroll
        for (int h = 0; h < UPS; ++h)
#pragma unroll
            for (int i = 0; i < CH; ++i) *reinterpret_cast<v4i *>(&As[buf][adst[i] + 64 * h]) = ar[slot][h][i];
    };
    // stage 0 is requested first, then the token scales and row sums (the
    // row sums start the accumulators), then stage 1: the round trips
    // overlap, and the wait for the scales leaves stage 1's loads in flight
    load_stage(0, 0);
    __builtin_amdgcn_sched_barrier(0);
    float s_gamma = 0.0f, s_absmax = 0.0f;
    int32_t s_rowsum = 0;
    if (tid < BM) {
        const int m = min(m0 + tid, M - 1);
        s_gamma = *gload_ptr<float>(p.gamma);
        s_absmax = gload_ptr<float>(p.absmax)[m];
        s_rowsum = gload_ptr<int32_t>(p.rowsum)[m];
    }
    __builtin_amdgcn_sched_barrier(0);
    static_assert(kD == 2, "two stages of lookahead");
    load_stage(1, 1);
    __builtin_amdgcn_sched_barrier(0);
    if (tid < BM) {
        cs[tid] = token_scale(s_gamma, s_absmax);
        nrsum[tid] = -s_rowsum;
    }
    stage_lds(0, 0);
    __syncthreads();

    // the accumulators start at minus the token's row sum (in the first K
    // split only), so they end as sum (t + 1) q - sum q = sum t q
    v16i acc[WMS][2];
#pragma unroll
    for (int i = 0; i < WMS; ++i) acc[i][0] = acc[i][1] = (v16i){};
    if (split == 0) {
#pragma unroll
        for (int i = 0; i < WMS; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const v4i n4 = *reinterpret_cast<const v4i *>(&nrsum[32 * i + 8 * q + 4 * g]);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][0][4 * q + e] = acc[i][1][4 * q + e] = n4[e];
            }
    }

    auto step = [&](int s, int st) {
        __builtin_amdgcn_sched_barrier(0);
        const int buf = st & 1;
        v4u w[UPS];
#pragma unroll
        for (int h = 0; h < UPS; ++h) w[h] = br[s][h];
        const int8_t *abase = &As[buf][r * kRow + 16 * g];
#pragma unroll
        for (int h = 0; h < UPS; ++h) {
            v4i a[WMS][2];
#pragma unroll
            for (int i = 0; i < WMS; ++i) {
                const int8_t *arow = abase + 32 * i * kRow + 64 * h;
                a[i][0] = *reinterpret_cast<const v4i *>(arow);
                a[i][1] = *reinterpret_cast<const v4i *>(arow + 32);
            }
            v4i b0, b1, b2, b3;
            planes2(w[h].x, w[h].y, b0, b1);
            planes2(w[h].z, w[h].w, b2, b3);
            if (h == UPS - 1) {
                // every word of slot s has become planes: refill it
                __builtin_amdgcn_sched_barrier(0);
                load_stage(s, st + kD);
            }
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
        }
        if (st + 1 < KS) {  // the last stage has no successor to stage
            stage_lds(buf ^ 1, (s + 1) % kD);
            __syncthreads();
        }
    };
    int s0 = 0;
    for (; s0 + kD <= KS; s0 += kD) {
#pragma unroll
        for (int s = 0; s < kD; ++s) step(s, s0 + s);
    }
#pragma unroll
    for (int s = 0; s < kD - 1; ++s)
        if (s0 + s < KS) step(s, s0 + s);

    {
        if (ks > 1) {
            constexpr int kAcc = 32 * WMS;  // accumulators per thread
            int32_t *part = p.acc_ws + (int64_t)item * ks * (kAcc * kThreads);
#pragma unroll
            for (int i = 0; i < WMS; ++i)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        put_partial(part + ((int64_t)split * kAcc + (i * 2 + s2) * 16 + e) * kThreads + tid,
                                    acc[i][s2][e]);
            if (!arrive_last(p, item)) return;
            for (int j = 0; j < ks; ++j) {
                if (j == split) continue;
#pragma unroll
                for (int i = 0; i < WMS; ++i)
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) {
                        int32_t v[16];
#pragma unroll
                        for (int e = 0; e < 16; ++e)
                            v[e] = get_partial(part + ((int64_t)j * kAcc + (i * 2 + s2) * 16 + e) * kThreads + tid);
#pragma unroll
                        for (int e = 0; e < 16; ++e) acc[i][s2][e] += v[e];
                    }
            }
        }
    }

    // epilogue: rescale and store, non-temporal.  A wave whose 64 x 64 block
    // lies wholly inside Y (N a multiple of 4) stores straight from its
    // accumulators through a buffer resource at scalar row offsets: no LDS,
    // no per-row bounds tests, no address arithmetic in vector registers.
    // Other waves transpose through LDS for 16-byte stores with tests.
    float *ep = reinterpret_cast<float *>(smem) + wave * (32 * kEpiStride);
    const bool vec_ok = (N & 3) == 0;
    const bool interior = tv && vec_ok && m0 + BM <= M && 64 * tile + 64 <= N && N <= (1 << 23);
    // only blocks at the edge of Y reuse the stage buffers (for the
    // transpose): where every wave's block is interior, no wave waits
    if (!(vec_ok && m0 + BM <= M && 64 * (4 * nt + 3) + 64 <= N && N <= (1 << 23)))
        __syncthreads();  // every wave is done with the activation stages
    BL_GLOBAL float *Y = gstore_ptr<float>(p.Y);
    float *yp = uni(p.Y) + (int64_t)m0 * N;
    const __amdgpu_buffer_rsrc_t ry = buffer_rsrc(yp, -1);
    const int yoff = 4 * ((lane >> 4) * N + 64 * tile + 4 * (lane & 15));
    auto epilogue = [&](auto whole) {
#pragma unroll
        for (int i = 0; i < WMS; ++i) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = 8 * (e >> 2) + 4 * g + (e & 3);
                    ep[row * kEpiStride + 32 * s2 + r] = (float)acc[i][s2][e] * cs[32 * i + row];
                }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int row = (lane >> 4) + 4 * k;
                const int c4 = 4 * (lane & 15);
                const v4f_t v = *reinterpret_cast<const v4f_t *>(&ep[row * kEpiStride + c4]);
                if constexpr (decltype(whole)::value) {
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), ry, yoff,
                                                           4 * (32 * i + 4 * k) * N, kNonTemporal);
                } else {
                    const int m = m0 + 32 * i + row;
                    const int n = 64 * tile + c4;
                    if (tv && m < M) {
                        const int64_t o = (int64_t)m * N + n;
                        if (vec_ok && n + 3 < N) {
                            __builtin_nontemporal_store(v, reinterpret_cast<BL_GLOBAL v4f_t *>(Y + o));
                        } else {
                            if (n < N) __builtin_nontemporal_store(v.x, Y + o);
                            if (n + 1 < N) __builtin_nontemporal_store(v.y, Y + o + 1);
                            if (n + 2 < N) __builtin_nontemporal_store(v.z, Y + o + 2);
                            if (n + 3 < N) __builtin_nontemporal_store(v.w, Y + o + 3);
                        }
                    }
                }
            }
        }
    };
    if (interior) {
        // straight from the accumulators: element e of lane l is token
        // 8 (e / 4) + 4 (l / 32) + e % 4 of the half, row 32 s2 + l % 32, so
        // one 4-byte store of the wave writes two whole 128-byte row pieces
        const int doff = 4 * (4 * g * N + 64 * tile + r);
#pragma unroll
        for (int i = 0; i < WMS; ++i)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = 8 * (e >> 2) + 4 * g + (e & 3);
                    const float v = (float)acc[i][s2][e] * cs[32 * i + row];
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), ry, doff + 128 * s2,
                                                          4 * (32 * i + 8 * (e >> 2) + (e & 3)) * N, kNonTemporal);
                }
    } else {
        epilogue(std::false_type{});
    }
    if (p.acc_out && tv) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const int n = 64 * tile + 32 * s2 + r;
            if (n >= N) continue;
#pragma unroll
            for (int i = 0; i < WMS; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = 32 * i + 8 * (e >> 2) + 4 * g + (e & 3);
                    const int m = m0 + row;
                    if (m < M) gstore_ptr<int32_t>(p.acc_out)[(int64_t)m * N + n] = acc[i][s2][e];
                }
        }
    }
}

// Workgroup b runs on XCD b % 8; the logical item order is split into eight
// contiguous slices, one per XCD (slot b stands for logical item
// (b % 8) * per + b / 8), so the tiles that share activation rows and packed
// weight columns meet in the same L2.
__device__ inline int xcd_logical(int b, int per)
{
    return (b & 7) * per + (b >> 3);
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
void tile_single_kernel(Problem p, int items, int per)
{
    const int j = xcd_logical(blockIdx.x, per);
    if (j < items) tile_body<2, 2>(p, j);
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
void tile_group_kernel(const Problem *__restrict__ probs, const uint2 *__restrict__ item_map)
{
    const uint2 it = item_map[blockIdx.x];
    if (it.x != 0xFFFFFFFFu) tile_body<2, 2>(probs[it.x], (int)it.y);
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
void tile_multi_kernel(ProblemSet ps)
{
    const int i = multi_index(ps, blockIdx.x);
    tile_body<2, 2>(ps.p[i], (int)blockIdx.x - ps.begin[i]);
}

}  // namespace

hipError_t launch_tile_single(const Problem &p, hipStream_t s)
{
    const int items = p.mt * p.ntt * p.ks;
    const int per = (items + 7) / 8;
    hipLaunchKernelGGL(tile_single_kernel, dim3((unsigned)(8 * per)), dim3(kThreads), 0, s, p, items, per);
    return hipGetLastError();
}

hipError_t launch_tile_group(const Problem *probs, const uint2 *item_map, int n_items, hipStream_t s)
{
    hipLaunchKernelGGL(tile_group_kernel, dim3((unsigned)n_items), dim3(kThreads), 0, s, probs, item_map);
    return hipGetLastError();
}

hipError_t launch_tile_multi(const ProblemSet &ps, hipStream_t s)
{
    hipLaunchKernelGGL(tile_multi_kernel, dim3((unsigned)ps.begin[ps.count]), dim3(kThreads), 0, s, ps);
    return hipGetLastError();
}

}  // namespace bl
