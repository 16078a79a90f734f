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
typedef float v4f_t __attribute__((ext_vector_type(4)));
constexpr int kDepth = 3; // units of global-load lookahead

// WMS: 32-token subtiles per wave; WNT: 64-row weight tiles per wave;
// WAVES_M x (4 / WAVES_M) waves.  The workgroup covers BM = WAVES_M*WMS*32
// tokens and always 256 weight rows.
// Activation staging (ALAY):
//   0  row-major activations -> LDS rows padded to 80 bytes;
//   1  fragment-ordered activations (see qf32_offset) -> LDS unchanged: the
//      global loads are whole 1 KiB blocks;
//   2  row-major activations -> LDS in fragment order: each wave instruction
//      fills one 1 KiB operand fragment (32 rows x 32 bytes from global).
// In 1 and 2 the LDS writes and the operand reads are linear (conflict-free,
// no padding).
// EPI: the rescaled outputs go through LDS, 32 rows at a time per wave, so
// that Y is written with 16-byte stores covering whole 256-byte row pieces
// instead of one 4-byte store per accumulator element.
// Output stores are non-temporal: the fp32 result (M*N*4 bytes, the largest
// stream of the kernel) is written once and must not evict the activation
// and weight tiles that other workgroups still reuse from L2.
constexpr int kEpiStride = 72;  // floats per LDS row of the epilogue transpose

template <int WMS, int WNT, int WAVES_M, int ALAY, bool EPI = false>
__device__ __forceinline__ void tile_body(const Problem &p, int local)
{
    constexpr bool FRAG = ALAY != 0;
    constexpr int WAVES_N = 4 / WAVES_M;
    static_assert(WAVES_N * WNT == 4, "a workgroup spans 256 weight rows");
    constexpr int BM = WAVES_M * WMS * 32;
    constexpr int CH = BM * 4 / kThreads;  // 16-byte activation chunks per thread per unit
    static_assert(CH >= 1, "tile too small for the staging pattern");
    constexpr int kRowBytes = FRAG ? 64 : kLda;
    constexpr int kStageBytes = BM * kRowBytes;
    constexpr int kEpiBytes = EPI ? 4 * 32 * kEpiStride * 4 : 0;
    constexpr int kSmem = 2 * kStageBytes > kEpiBytes ? 2 * kStageBytes : kEpiBytes;
    __shared__ __attribute__((aligned(16))) int8_t smem[kSmem];
    int8_t (*As)[kStageBytes] = reinterpret_cast<int8_t (*)[kStageBytes]>(smem);
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
        if constexpr (ALAY == 1) {
            const int64_t b = min((m0 >> 5) + (c >> 7), ((p.M + 31) >> 5) - 1);
            asrc[i] = gload_ptr<int8_t>(p.Q + b * KU * 2048 + 16 * (c & 127));
            adst[i] = 16 * c;
        } else if constexpr (ALAY == 2) {
            // fragment f = c / 64 = (32-row block, half), lane l = c % 64:
            // row 32*(f/2) + l%32, 16 bytes at 32*(f%2) + 16*(l/32) of the unit
            const int f = c >> 6, l = c & 63;
            const int m = min(m0 + 32 * (f >> 1) + (l & 31), p.M - 1);
            asrc[i] = gload_ptr<int8_t>(p.Q + (int64_t)m * p.ldq + 32 * (f & 1) + 16 * (l >> 5));
            adst[i] = 16 * c;
        } else {
            const int m = min(m0 + (c >> 2), p.M - 1);
            asrc[i] = gload_ptr<int8_t>(p.Q + (int64_t)m * p.ldq + 16 * (c & 3));
            adst[i] = (c >> 2) * kLda + 16 * (c & 3);
        }
    }
    astep = ALAY == 1 ? 2048 : 64;

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

    if constexpr (EPI) {
        __syncthreads();  // every wave is done with the activation stages
        float *ep = reinterpret_cast<float *>(smem) + wave * (32 * kEpiStride);
        const bool vec_ok = (p.N & 3) == 0;  // 16-byte aligned output rows
        BL_GLOBAL float *Y = gstore_ptr<float>(p.Y);
#pragma unroll
        for (int j = 0; j < WNT; ++j) {
#pragma unroll
            for (int i = 0; i < WMS; ++i) {
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int row = 8 * (e >> 2) + 4 * g + (e & 3);
                        const int rr = arow0 + 32 * i + row;
                        ep[row * kEpiStride + 32 * s2 + r] = (float)(acc[i][2 * j + s2][e] - rsum[rr]) * cs[rr];
                    }
                // 16 lanes per 64-float row piece, 4 rows per pass, 8 passes
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int row = (lane >> 4) + 4 * k;
                    const int c4 = 4 * (lane & 15);
                    const int m = m0 + arow0 + 32 * i + row;
                    const int n = 64 * tile[j] + c4;
                    const v4f_t v = *reinterpret_cast<const v4f_t *>(&ep[row * kEpiStride + c4]);
                    if (tv[j] && m < p.M) {
                        const int64_t o = (int64_t)m * p.N + n;
                        if (vec_ok && n + 3 < p.N) {
                            __builtin_nontemporal_store(v, reinterpret_cast<BL_GLOBAL v4f_t *>(Y + o));
                        } else {
                            if (n < p.N) __builtin_nontemporal_store(v.x, Y + o);
                            if (n + 1 < p.N) __builtin_nontemporal_store(v.y, Y + o + 1);
                            if (n + 2 < p.N) __builtin_nontemporal_store(v.z, Y + o + 2);
                            if (n + 3 < p.N) __builtin_nontemporal_store(v.w, Y + o + 3);
                        }
                    }
                }
            }
        }
    }
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
                        if constexpr (!EPI)
                            __builtin_nontemporal_store((float)a * cs[row], gstore_ptr<float>(p.Y) + o);
                        if (p.acc_out) gstore_ptr<int32_t>(p.acc_out)[o] = a;
                    }
                }
            }
        }
    }
}

// WMS*32-token x 64-row-per-wave tile (as tile_body<WMS, 1, 1, 0, true>) with
// UPS units of K per LDS stage and barrier: the fixed cost of a barrier
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
constexpr int kLda2 = 144;  // 128 bytes + 16 of padding: 8 lanes on distinct banks

template <int UPS, int WMS>
__device__ __forceinline__ void tile_body_ups(const Problem &p, int local)
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
    __shared__ int rsum[BM];

    const int split = local % p.ks;
    const int item = local / p.ks;
    const int mtile = item % p.mt;
    const int nt = item / p.mt;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, g = lane >> 5, r = lane & 31;
    const int m0 = mtile * BM;
    const int KU = p.KU;
    const int ub = split * p.upsplit;           // first unit of the split
    const int nu = min(KU, ub + p.upsplit) - ub;  // its units
    const int KS = (nu + UPS - 1) / UPS;
    const int tile = 4 * nt + wave;
    const bool tv = tile < p.NT;
    const BL_GLOBAL v4u *blk = gload_ptr<v4u>(p.P + (int64_t)min(tile, p.NT - 1) * KU * kBlockBytes) + lane;

    const BL_GLOBAL int8_t *asrc[CH];
    int adst[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int c = tid + kThreads * i;
        const int m = min(m0 + (c >> 2), p.M - 1);
        asrc[i] = gload_ptr<int8_t>(p.Q + (int64_t)m * p.ldq + 16 * (c & 3));
        adst[i] = (c >> 2) * kRow + 16 * (c & 3);
    }

    __syncthreads();  // the previous work item of this workgroup may still read LDS

    v4i ar[kD][UPS][CH];
    v4u br[kD][UPS];
    auto load_stage = [&](int slot, int st) {
#pragma unroll
        for (int h = 0; h < UPS; ++h) {
            const int u = st * UPS + h;
            const int uc = ub + min(u, nu - 1);
#pragma unroll
            for (int i = 0; i < CH; ++i) ar[slot][h][i] = *reinterpret_cast<const BL_GLOBAL v4i *>(asrc[i] + 64 * uc);
            br[slot][h] = blk[(int64_t)uc * 64];
        }
    };
    auto stage_lds = [&](int buf, int slot) {
#pragma unroll
        for (int h = 0; h < UPS; ++h)
#pragma unroll
            for (int i = 0; i < CH; ++i) *reinterpret_cast<v4i *>(&As[buf][adst[i] + 64 * h]) = ar[slot][h][i];
    };
#pragma unroll
    for (int d = 0; d < kD; ++d) load_stage(d, d);
    // the token scales (read by the epilogue only) are requested behind the
    // first stages, so the two memory round trips overlap
    __builtin_amdgcn_sched_barrier(0);
    if (tid < BM) {
        const int m = min(m0 + tid, p.M - 1);
        cs[tid] = (*gload_ptr<float>(p.gamma) * gload_ptr<float>(p.absmax)[m]) / 127.0f;
        rsum[tid] = gload_ptr<int32_t>(p.rowsum)[m];
    }
    stage_lds(0, 0);
    __syncthreads();

    v16i acc[WMS][2];
#pragma unroll
    for (int i = 0; i < WMS; ++i) acc[i][0] = acc[i][1] = (v16i){};

    auto step = [&](int s, int st) {
        __builtin_amdgcn_sched_barrier(0);
        const int buf = st & 1;
        v4u w[UPS];
        const v4u z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int h = 0; h < UPS; ++h) w[h] = st * UPS + h < nu ? br[s][h] : z;
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
            const v4i b0 = planes(w[h].x), b1 = planes(w[h].y), b2 = planes(w[h].z), b3 = planes(w[h].w);
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
        stage_lds(buf ^ 1, (s + 1) % kD);
        __syncthreads();
    };
    int s0 = 0;
    for (; s0 + kD <= KS; s0 += kD) {
#pragma unroll
        for (int s = 0; s < kD; ++s) step(s, s0 + s);
    }
#pragma unroll
    for (int s = 0; s < kD - 1; ++s)
        if (s0 + s < KS) step(s, s0 + s);

    if constexpr (WMS == 2) {  // the host splits K for the 64-token instantiation only
        if (p.ks > 1) {
            constexpr int kAcc = 32 * WMS;  // accumulators per thread
            int32_t *part = p.acc_ws + (int64_t)item * p.ks * (kAcc * kThreads);
#pragma unroll
            for (int i = 0; i < WMS; ++i)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        put_partial(part + ((int64_t)split * kAcc + (i * 2 + s2) * 16 + e) * kThreads + tid,
                                    acc[i][s2][e]);
            if (!arrive_last(p, item)) return;
            for (int j = 0; j < p.ks; ++j) {
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

    // epilogue: rescale, transpose through LDS, 16-byte non-temporal stores
    __syncthreads();  // every wave is done with the activation stages
    float *ep = reinterpret_cast<float *>(smem) + wave * (32 * kEpiStride);
    const bool vec_ok = (p.N & 3) == 0;
    BL_GLOBAL float *Y = gstore_ptr<float>(p.Y);
#pragma unroll
    for (int i = 0; i < WMS; ++i) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = 8 * (e >> 2) + 4 * g + (e & 3);
                const int rr = 32 * i + row;
                ep[row * kEpiStride + 32 * s2 + r] = (float)(acc[i][s2][e] - rsum[rr]) * cs[rr];
            }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int row = (lane >> 4) + 4 * k;
            const int c4 = 4 * (lane & 15);
            const int m = m0 + 32 * i + row;
            const int n = 64 * tile + c4;
            const v4f_t v = *reinterpret_cast<const v4f_t *>(&ep[row * kEpiStride + c4]);
            if (tv && m < p.M) {
                const int64_t o = (int64_t)m * p.N + n;
                if (vec_ok && n + 3 < p.N) {
                    __builtin_nontemporal_store(v, reinterpret_cast<BL_GLOBAL v4f_t *>(Y + o));
                } else {
                    if (n < p.N) __builtin_nontemporal_store(v.x, Y + o);
                    if (n + 1 < p.N) __builtin_nontemporal_store(v.y, Y + o + 1);
                    if (n + 2 < p.N) __builtin_nontemporal_store(v.z, Y + o + 2);
                    if (n + 3 < p.N) __builtin_nontemporal_store(v.w, Y + o + 3);
                }
            }
        }
    }
    if (p.acc_out && tv) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const int n = 64 * tile + 32 * s2 + r;
            if (n >= p.N) continue;
#pragma unroll
            for (int i = 0; i < WMS; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = 32 * i + 8 * (e >> 2) + 4 * g + (e & 3);
                    const int m = m0 + row;
                    if (m < p.M) gstore_ptr<int32_t>(p.acc_out)[(int64_t)m * p.N + n] = acc[i][s2][e] - rsum[row];
                }
        }
    }
}

// 64-token x 256-row tile with the activation tile moved by the buffer
// unit straight into LDS (buffer_load ... lds) instead of through a
// register ring and ds_write: no VGPRs hold in-flight activations, the LDS
// stages are laid out in MFMA fragment order (each wave instruction fills
// one 1 KiB fragment, lane l's 16 bytes at 16 l, and each operand read is
// the same linear 1 KiB: no bank conflicts, no padding), and NB stages sit
// in LDS, D of them in flight.  Weights come through buffer loads too; every
// address of the loop is scalar: the buffer resource of unit u starts at
// unit u, and units past the K range get a record count of zero, so their
// loads return zeros -- zero fields add nothing -- with no per-lane select.
// Waits are placed by hand: the DMA's LDS writes are not tracked by the
// compiler, so every stage waits until at most the loads of the stages
// after it are outstanding (loads complete in order), then meets the
// other waves at a barrier.
__device__ inline __amdgpu_buffer_rsrc_t unit_rsrc(const void *base, int64_t off, bool live, uint32_t bytes)
{
    // CDNA buffer resource: 32-bit data format, no stride, raw addressing
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(static_cast<const char *>(base)) + off, 0,
                                             live ? bytes : 0u, 0x00020000);
}

template <int WMS, int WNT, int NB, int D, int UPS = 2, bool PRIO = false>
__device__ __forceinline__ void tile_body_dma(const Problem &p, int local)
{
    // WMS 32-token blocks x WNT 64-row weight tiles per wave; the four waves
    // share the tokens and take consecutive weight tiles
    constexpr int BM = 32 * WMS;
    constexpr int kFrags = 2 * WMS;                 // 1 KiB fragments per unit (block, half)
    constexpr int kFragsPerWave = kFrags / 4;       // moved by each wave per unit
    static_assert(kFrags % 4 == 0, "every wave moves whole fragments");
    constexpr int kUnitBytes = kFrags * 1024;
    constexpr int kStageBytes = UPS * kUnitBytes;
    constexpr int kEpiBytes = 4 * 32 * kEpiStride * 4;
    constexpr int kSmem = NB * kStageBytes > kEpiBytes ? NB * kStageBytes : kEpiBytes;
    static_assert(NB >= D + 1, "a stage's LDS buffer is refilled only after every wave has read it");
    __shared__ __attribute__((aligned(1024))) int8_t smem[kSmem];
    __shared__ float cs[BM];
    __shared__ int rsum[BM];

    const int split = local % p.ks;
    const int item = local / p.ks;
    const int mtile = item % p.mt;
    const int nt = item / p.mt;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, g = lane >> 5, r = lane & 31;
    const int m0 = mtile * BM;
    const int KU = p.KU;
    const int ub = split * p.upsplit;             // first unit of the split
    const int nu = min(KU, ub + p.upsplit) - ub;  // its units
    const int KS = (nu + UPS - 1) / UPS;
    int tile[WNT];
    bool tv[WNT];
    const uint8_t *bbase[WNT];
#pragma unroll
    for (int j = 0; j < WNT; ++j) {
        tile[j] = 4 * WNT * nt + WNT * wave + j;
        tv[j] = tile[j] < p.NT;
        bbase[j] = p.P + (int64_t)min(tile[j], p.NT - 1) * KU * kBlockBytes;
    }

    // the token scales (read by the epilogue only), requested first so that
    // every later wait covers them; kept in registers until the epilogue
    float cs_r = 0.0f;
    int rs_r = 0;
    if (tid < BM) {
        const int m = min(m0 + tid, p.M - 1);
        cs_r = (*gload_ptr<float>(p.gamma) * gload_ptr<float>(p.absmax)[m]) / 127.0f;
        rs_r = gload_ptr<int32_t>(p.rowsum)[m];
    }

    // fragment f = 2 b + h of a unit: 32-token block b, code half h; lane l
    // brings token 32 b + l % 32, codes 32 h + 16 (l / 32) .. + 15.  Wave w
    // moves fragments w * kFragsPerWave + i.  Row-major activations: 16
    // bytes of the token's row (rows past M re-read row M - 1, never
    // stored); fragment-ordered ones: the 1 KiB block of (32-row block,
    // unit, half).
    const int8_t *abase[kFragsPerWave];
    int64_t astride;
    uint32_t avoff[kFragsPerWave], abytes;
#pragma unroll
    for (int i = 0; i < kFragsPerWave; ++i) {
        const int f = wave * kFragsPerWave + i, fb = f >> 1, fh = f & 1;
        if (p.qtiled) {
            // 32-row blocks past the last one re-read the last
            const int64_t blk = min(m0 / 32 + fb, (p.M + 31) / 32 - 1);
            abase[i] = p.Q + ((blk * KU) * 2 + fh) * 1024;
            avoff[i] = 16u * (uint32_t)lane;
        } else {
            const int m = min(m0 + 32 * fb + r, p.M - 1);
            abase[i] = p.Q + (int64_t)m0 * p.ldq + 32 * fh;
            avoff[i] = (uint32_t)((m - m0) * p.ldq + 16 * g);
        }
    }
    astride = p.qtiled ? 2048 : 64;
    abytes = p.qtiled ? 1024u : (uint32_t)(BM * p.ldq);
    // LDS: stage buffer b holds UPS units of kFrags fragments; fragment f of
    // unit h lands at b * kStageBytes + h * kUnitBytes + f * 1024
    auto issue_a = [&](int st) {
        const int buf = st % NB;
#pragma unroll
        for (int h = 0; h < UPS; ++h) {
            const int u = st * UPS + h;
#pragma unroll
            for (int i = 0; i < kFragsPerWave; ++i) {
                const int f = wave * kFragsPerWave + i;
                const __amdgpu_buffer_rsrc_t rs = unit_rsrc(abase[i], astride * (ub + u), u < nu, abytes);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rs, (__attribute__((address_space(3))) void *)(smem + buf * kStageBytes + h * kUnitBytes + f * 1024),
                    16, avoff[i], 0, 0, 0);
            }
        }
    };
    v4u br[D][UPS][WNT];
    auto issue_b = [&](int slot, int st) {
#pragma unroll
        for (int h = 0; h < UPS; ++h) {
            const int u = st * UPS + h;
#pragma unroll
            for (int j = 0; j < WNT; ++j) {
                const __amdgpu_buffer_rsrc_t rs =
                    unit_rsrc(bbase[j], (int64_t)(ub + u) * kBlockBytes, u < nu, kBlockBytes);
                br[slot][h][j] =
                    __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rs, 16u * (uint32_t)lane, 0, 0));
            }
        }
    };

    __syncthreads();  // the previous work item of this workgroup may still read LDS
#pragma unroll
    for (int d = 0; d < D; ++d) {
        issue_a(d);
        issue_b(d, d);
    }

    v16i acc[WMS][2 * WNT];
#pragma unroll
    for (int i = 0; i < WMS; ++i)
#pragma unroll
        for (int j = 0; j < 2 * WNT; ++j) acc[i][j] = (v16i){};

    // s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding:
    // vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
    constexpr int kAfter = (D - 1) * UPS * (kFragsPerWave + WNT);  // loads of the later stages
    constexpr int kWaitLater = 0x0F70 | (kAfter & 15) | ((kAfter >> 4) << 14);
    static_assert(kAfter < 64, "wait count fits the counter");
    auto step = [&](int s, int st) {
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
        __builtin_amdgcn_s_waitcnt(kWaitLater);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        issue_a(st + D);
        const int8_t *sb = smem + (st % NB) * kStageBytes + 16 * lane;
        v4i b[UPS][WNT][4];
#pragma unroll
        for (int h = 0; h < UPS; ++h)
#pragma unroll
            for (int j = 0; j < WNT; ++j) {
                const v4u w = br[s][h][j];
                b[h][j][0] = planes(w.x);
                b[h][j][1] = planes(w.y);
                b[h][j][2] = planes(w.z);
                b[h][j][3] = planes(w.w);
            }
        __builtin_amdgcn_sched_barrier(0);
        issue_b(s, st + D);
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int h = 0; h < UPS; ++h) {
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                v4i a[WMS];
#pragma unroll
                for (int i = 0; i < WMS; ++i)
                    a[i] = *reinterpret_cast<const v4i *>(sb + h * kUnitBytes + (2 * i + kh) * 1024);
#pragma unroll
                for (int i = 0; i < WMS; ++i)
#pragma unroll
                    for (int j = 0; j < WNT; ++j) {
                        // word (s, kh) of the slot: rows 32 s of the tile, code half kh
                        acc[i][2 * j] = mfma_i8(a[i], b[h][j][kh], acc[i][2 * j]);
                        acc[i][2 * j + 1] = mfma_i8(a[i], b[h][j][2 + kh], acc[i][2 * j + 1]);
                    }
            }
        }
    };
    int s0 = 0;
    for (; s0 + D <= KS; s0 += D) {
#pragma unroll
        for (int s = 0; s < D; ++s) step(s, s0 + s);
    }
#pragma unroll
    for (int s = 0; s < D - 1; ++s)
        if (s0 + s < KS) step(s, s0 + s);

    // the surplus stages' loads (zeros) must land before LDS is reused
    __builtin_amdgcn_s_waitcnt(0x0F70);
    if (tid < BM) {
        cs[tid] = cs_r;
        rsum[tid] = rs_r;
    }

    if (p.ks > 1) {
        constexpr int kAcc = 32 * WMS * WNT;  // accumulators per thread
        int32_t *part = p.acc_ws + (int64_t)item * p.ks * (kAcc * kThreads);
#pragma unroll
        for (int i = 0; i < WMS; ++i)
#pragma unroll
            for (int s2 = 0; s2 < 2 * WNT; ++s2)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    put_partial(part + ((int64_t)split * kAcc + (i * 2 * WNT + s2) * 16 + e) * kThreads + tid,
                                acc[i][s2][e]);
        if (!arrive_last(p, item)) return;
        for (int jj = 0; jj < p.ks; ++jj) {
            if (jj == split) continue;
#pragma unroll
            for (int i = 0; i < WMS; ++i)
#pragma unroll
                for (int s2 = 0; s2 < 2 * WNT; ++s2) {
                    int32_t v[16];
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        v[e] = get_partial(part + ((int64_t)jj * kAcc + (i * 2 * WNT + s2) * 16 + e) * kThreads + tid);
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[i][s2][e] += v[e];
                }
        }
    }

    // epilogue: rescale, transpose through LDS (32 token rows x 64 weight
    // rows per wave at a time), 16-byte non-temporal stores
    __syncthreads();  // every wave is done with the activation stages; scales visible
    float *ep = reinterpret_cast<float *>(smem) + wave * (32 * kEpiStride);
    const bool vec_ok = (p.N & 3) == 0;
    BL_GLOBAL float *Y = gstore_ptr<float>(p.Y);
#pragma unroll
    for (int j = 0; j < WNT; ++j)
#pragma unroll
        for (int i = 0; i < WMS; ++i) {
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = 8 * (e >> 2) + 4 * g + (e & 3);
                    const int rr = 32 * i + row;
                    ep[row * kEpiStride + 32 * s2 + r] = (float)(acc[i][2 * j + s2][e] - rsum[rr]) * cs[rr];
                }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int row = (lane >> 4) + 4 * k;
                const int c4 = 4 * (lane & 15);
                const int m = m0 + 32 * i + row;
                const int n = 64 * tile[j] + c4;
                const v4f_t v = *reinterpret_cast<const v4f_t *>(&ep[row * kEpiStride + c4]);
                if (tv[j] && m < p.M) {
                    const int64_t o = (int64_t)m * p.N + n;
                    if (vec_ok && n + 3 < p.N) {
                        __builtin_nontemporal_store(v, reinterpret_cast<BL_GLOBAL v4f_t *>(Y + o));
                    } else {
                        if (n < p.N) __builtin_nontemporal_store(v.x, Y + o);
                        if (n + 1 < p.N) __builtin_nontemporal_store(v.y, Y + o + 1);
                        if (n + 2 < p.N) __builtin_nontemporal_store(v.z, Y + o + 2);
                        if (n + 3 < p.N) __builtin_nontemporal_store(v.w, Y + o + 3);
                    }
                }
            }
        }
    if (p.acc_out) {
#pragma unroll
        for (int j = 0; j < WNT; ++j) {
            if (!tv[j]) continue;
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const int n = 64 * tile[j] + 32 * s2 + r;
                if (n >= p.N) continue;
#pragma unroll
                for (int i = 0; i < WMS; ++i)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int row = 32 * i + 8 * (e >> 2) + 4 * g + (e & 3);
                        const int m = m0 + row;
                        if (m < p.M)
                            gstore_ptr<int32_t>(p.acc_out)[(int64_t)m * p.N + n] = acc[i][2 * j + s2][e] - rsum[row];
                    }
            }
        }
    }
}

// Instantiations (the value of the tile-variant knob):
//   0  64 tokens x 256 rows, each wave 64 x 64 (four waves along N);
//   1  128 tokens x 256 rows, each wave 64 x 128 (2 x 2 waves): half the LDS
//      reads and L2 reads per MFMA of 0;
//   2  128 tokens x 256 rows, each wave 128 x 64, 4-byte output stores;
//   5, 6, 7  as 2, 0, 1 on fragment-ordered activations;
//   10, 12  as 2 with activations staged in fragment order (10 with the
//      LDS-transposed epilogue);
//   11  as 2 with the LDS-transposed epilogue;
//   18  as 11 with two 64-code units per LDS stage;
//   19  as 18 with 64-token tiles (64 x 64 per wave; the default).
template <int V>
__device__ __forceinline__ void tile_dispatch(const Problem &p, int local)
{
    if constexpr (V == 0)
        tile_body<2, 1, 1, 0>(p, local);
    else if constexpr (V == 1)
        tile_body<2, 2, 2, 0>(p, local);
    else if constexpr (V == 2)
        tile_body<4, 1, 1, 0>(p, local);
    else if constexpr (V == 5)
        tile_body<4, 1, 1, 1>(p, local);
    else if constexpr (V == 6)
        tile_body<2, 1, 1, 1>(p, local);
    else if constexpr (V == 7)
        tile_body<2, 2, 2, 1>(p, local);
    else if constexpr (V == 10)
        tile_body<4, 1, 1, 2, true>(p, local);
    else if constexpr (V == 11)
        tile_body<4, 1, 1, 0, true>(p, local);
    else if constexpr (V == 12)
        tile_body<4, 1, 1, 2, false>(p, local);
    else if constexpr (V == 19)
        tile_body_ups<2, 2>(p, local);
    else if constexpr (V == 20)
        tile_body_dma<2, 1, 3, 2>(p, local);
    else if constexpr (V == 21)
        tile_body_dma<2, 1, 4, 3>(p, local);
    else if constexpr (V == 23)
        tile_body_dma<4, 1, 3, 2>(p, local);
    else if constexpr (V == 24)
        tile_body_dma<2, 2, 3, 2>(p, local);
    else if constexpr (V == 27)
        tile_body_dma<2, 1, 3, 2, 2, true>(p, local);
    else if constexpr (V == 28)
        tile_body_dma<2, 1, 2, 1, 4>(p, local);
    else
        tile_body_ups<2, 4>(p, local);
}

// Workgroup b runs on XCD b % 8; the logical item order is split into eight
// contiguous slices, one per XCD (slot b stands for logical item
// (b % 8) * per + b / 8), so the tiles that share activation rows and packed
// weight columns meet in the same L2.
__device__ inline int xcd_logical(int b, int per)
{
    return (b & 7) * per + (b >> 3);
}

// Waves per SIMD each instantiation is compiled for (the register budget):
// the DMA-staged 64 x 64-per-wave tile fits 128 VGPRs (four waves), the
// larger per-wave tiles hold 128 or 256 accumulators.
template <int V>
struct TileWaves {
    static constexpr int lo = (V == 19 || V == 20 || V == 27) ? 4 : (V == 21 || V == 28) ? 3 : 2;
    static constexpr int hi = (V == 19 || V == 20 || V == 27) ? 4 : (V == 21 || V == 28) ? 3 : (V >= 23) ? 2 : 8;
};

template <int V>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(TileWaves<V>::lo, TileWaves<V>::hi)))
void tile_single_kernel(Problem p, int items, int per)
{
    const int j = xcd_logical(blockIdx.x, per);
    if (j < items) tile_dispatch<V>(p, j);
}

template <int V>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(TileWaves<V>::lo, TileWaves<V>::hi)))
void tile_group_kernel(const Problem *__restrict__ probs,
                                                                 const uint2 *__restrict__ item_map)
{
    const uint2 it = item_map[blockIdx.x];
    if (it.x != 0xFFFFFFFFu) tile_dispatch<V>(probs[it.x], (int)it.y);
}

template <int V>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(TileWaves<V>::lo, TileWaves<V>::hi)))
void tile_multi_kernel(ProblemSet ps)
{
    const int i = multi_index(ps, blockIdx.x);
    tile_dispatch<V>(ps.p[i], (int)blockIdx.x - ps.begin[i]);
}

}  // namespace

// one case per instantiation; unknown values take 18
#define BL_TILE_CASES(KERNEL, ...)                                                         \
    switch (variant) {                                                                     \
    case 0: hipLaunchKernelGGL(KERNEL<0>, __VA_ARGS__); break;                             \
    case 1: hipLaunchKernelGGL(KERNEL<1>, __VA_ARGS__); break;                             \
    case 2: hipLaunchKernelGGL(KERNEL<2>, __VA_ARGS__); break;                             \
    case 5: hipLaunchKernelGGL(KERNEL<5>, __VA_ARGS__); break;                             \
    case 6: hipLaunchKernelGGL(KERNEL<6>, __VA_ARGS__); break;                             \
    case 7: hipLaunchKernelGGL(KERNEL<7>, __VA_ARGS__); break;                             \
    case 10: hipLaunchKernelGGL(KERNEL<10>, __VA_ARGS__); break;                           \
    case 11: hipLaunchKernelGGL(KERNEL<11>, __VA_ARGS__); break;                           \
    case 12: hipLaunchKernelGGL(KERNEL<12>, __VA_ARGS__); break;                           \
    case 19: hipLaunchKernelGGL(KERNEL<19>, __VA_ARGS__); break;                           \
    case 20: hipLaunchKernelGGL(KERNEL<20>, __VA_ARGS__); break;                           \
    case 21: hipLaunchKernelGGL(KERNEL<21>, __VA_ARGS__); break;                           \
    case 23: hipLaunchKernelGGL(KERNEL<23>, __VA_ARGS__); break;                           \
    case 24: hipLaunchKernelGGL(KERNEL<24>, __VA_ARGS__); break;                           \
    case 27: hipLaunchKernelGGL(KERNEL<27>, __VA_ARGS__); break;                           \
    case 28: hipLaunchKernelGGL(KERNEL<28>, __VA_ARGS__); break;                           \
    default: hipLaunchKernelGGL(KERNEL<18>, __VA_ARGS__); break;                           \
    }

hipError_t launch_tile_single(const Problem &p, int variant, hipStream_t s)
{
    const int items = p.mt * p.ntt * p.ks;
    const int per = (items + 7) / 8;
    const dim3 grid((unsigned)(8 * per)), block(kThreads);
    BL_TILE_CASES(tile_single_kernel, grid, block, 0, s, p, items, per)
    return hipGetLastError();
}

hipError_t launch_tile_group(const Problem *probs, const uint2 *item_map, int n_items,
                             int variant, hipStream_t s)
{
    const dim3 grid((unsigned)n_items), block(kThreads);
    BL_TILE_CASES(tile_group_kernel, grid, block, 0, s, probs, item_map)
    return hipGetLastError();
}

hipError_t launch_tile_multi(const ProblemSet &ps, int variant, hipStream_t s)
{
    const dim3 grid((unsigned)ps.begin[ps.count]), block(kThreads);
    BL_TILE_CASES(tile_multi_kernel, grid, block, 0, s, ps)
    return hipGetLastError();
}

#undef BL_TILE_CASES

}  // namespace bl
