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

#include <cstdlib>

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

// 128-token x 64-row-per-wave tile (as tile_body<4, 1, 1, 0, true>) with
// UPS units of K per LDS stage and barrier: the fixed cost of a barrier
// round (the wait itself and the LDS read latency before the first MFMA)
// is paid once per UPS units.  A stage's unit past KU gets an all-zero
// packed word -- zero fields add nothing -- so odd unit counts need no
// branch; its activation chunk re-reads unit KU-1 (valid memory).
constexpr int kLda2 = 144;  // 128 bytes + 16 of padding: 8 lanes on distinct banks

template <int UPS>
__device__ __forceinline__ void tile_body_ups(const Problem &p, int local)
{
    constexpr int WMS = 4, BM = 128, CH = 2;  // CH: 16-byte chunks per thread per unit
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

    const int mtile = local % p.mt;
    const int nt = local / p.mt;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, g = lane >> 5, r = lane & 31;
    const int m0 = mtile * BM;
    const int KU = p.KU;
    const int KS = (KU + UPS - 1) / UPS;
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
    if (tid < BM) {
        const int m = min(m0 + tid, p.M - 1);
        cs[tid] = (*gload_ptr<float>(p.gamma) * gload_ptr<float>(p.absmax)[m]) / 127.0f;
        rsum[tid] = gload_ptr<int32_t>(p.rowsum)[m];
    }

    v4i ar[kD][UPS][CH];
    v4u br[kD][UPS];
    auto load_stage = [&](int slot, int st) {
#pragma unroll
        for (int h = 0; h < UPS; ++h) {
            const int u = st * UPS + h;
            const int uc = min(u, KU - 1);
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
        for (int h = 0; h < UPS; ++h) w[h] = st * UPS + h < KU ? br[s][h] : z;
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

// Software-pipelined variant (row-major activations, four waves along N,
// WMS 32-token subtiles per wave).  The activation tile goes through a
// three-stage LDS ring: while the MFMAs of unit u run, each wave already
// reads unit u+1's operands from LDS and unpacks its weight planes, stores
// unit u+2's activations into the third stage, and issues the global loads
// of unit u+4 (activations) and u+3 (weights).  One barrier per unit.
template <int WMS>
__device__ void tile_pipe_body(const Problem &p, int local)
{
    constexpr int BM = 32 * WMS;
    constexpr int CH = BM * 4 / kThreads;
    static_assert(CH >= 1, "tile too small for the staging pattern");
    __shared__ __attribute__((aligned(16))) int8_t As[3][BM * kLda];
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

    const BL_GLOBAL int8_t *asrc[CH];
    int adst[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int c = tid + kThreads * i;
        const int m = min(m0 + (c >> 2), p.M - 1);
        asrc[i] = gload_ptr<int8_t>(p.Q + (int64_t)m * p.ldq + 16 * (c & 3));
        adst[i] = (c >> 2) * kLda + 16 * (c & 3);
    }
    if (tid < BM) {
        const int m = min(m0 + tid, p.M - 1);
        cs[tid] = (*gload_ptr<float>(p.gamma) * gload_ptr<float>(p.absmax)[m]) / 127.0f;
        rsum[tid] = gload_ptr<int32_t>(p.rowsum)[m];
    }

    // register rings (slot = unit % 3): activation chunks of units u+2..u+4,
    // packed weights of units u+1..u+3
    v4i ar[3][CH];
    v4u br[3];
    auto load_a = [&](int slot, int u) {
        const int uc = min(u, KU - 1);
#pragma unroll
        for (int i = 0; i < CH; ++i) ar[slot][i] = *reinterpret_cast<const BL_GLOBAL v4i *>(asrc[i] + 64 * uc);
    };
    auto load_b = [&](int slot, int u) { br[slot] = blk[(int64_t)min(u, KU - 1) * 64]; };
    auto store_a = [&](int stage, int slot) {
#pragma unroll
        for (int i = 0; i < CH; ++i) *reinterpret_cast<v4i *>(&As[stage][adst[i]]) = ar[slot][i];
    };
    v4i fa[2][WMS][2];  // activation operands of the current / next unit
    v4i fb[2][4];       // weight planes of the current / next unit
    auto read_a = [&](int buf, int stage) {
#pragma unroll
        for (int i = 0; i < WMS; ++i) {
            const int8_t *arow = &As[stage][(32 * i + r) * kLda + 16 * g];
            fa[buf][i][0] = *reinterpret_cast<const v4i *>(arow);
            fa[buf][i][1] = *reinterpret_cast<const v4i *>(arow + 32);
        }
    };
    auto unpack_b = [&](int buf, int slot) {
        const v4u w = br[slot];
        fb[buf][0] = planes(w.x);
        fb[buf][1] = planes(w.y);
        fb[buf][2] = planes(w.z);
        fb[buf][3] = planes(w.w);
    };

    // prologue: units 0 and 1 staged, unit 0's operands in registers
    load_a(0, 0);
    load_a(1, 1);
    load_a(2, 2);
    load_b(0, 0);
    load_b(1, 1);
    load_b(2, 2);
    store_a(0, 0);
    store_a(1, 1);
    load_a(0, 3);
    load_a(1, 4);
    __syncthreads();
    read_a(0, 0);
    unpack_b(0, 0);
    load_b(0, 3);

    v16i acc[WMS][2];
#pragma unroll
    for (int i = 0; i < WMS; ++i) acc[i][0] = acc[i][1] = (v16i){};

    // unit u (cur = u & 1 operand buffer, u % 3 ring slot and LDS stage)
    auto step = [&](int u, int cur, int s3) {
        const int s1 = (s3 + 1) % 3, s2 = (s3 + 2) % 3;
        read_a(cur ^ 1, s1);    // unit u+1 (staged one unit ago)
        unpack_b(cur ^ 1, s1);  // unit u+1
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < WMS; ++i) {
                acc[i][0] = mfma_i8(fa[cur][i][h], fb[cur][h], acc[i][0]);
                acc[i][1] = mfma_i8(fa[cur][i][h], fb[cur][2 + h], acc[i][1]);
            }
        store_a(s2, s2);        // unit u+2 into the free stage
        load_a(s2, u + 5);      // that ring slot now takes unit u+5
        load_b(s1, u + 4);      // unit u+1's weights are unpacked: slot takes u+4
        __syncthreads();
    };
    int u = 0;
    for (; u + 6 <= KU; u += 6) {
        step(u + 0, 0, 0);
        step(u + 1, 1, 1);
        step(u + 2, 0, 2);
        step(u + 3, 1, 0);
        step(u + 4, 0, 1);
        step(u + 5, 1, 2);
    }
#pragma unroll
    for (int t = 0; t < 5; ++t)
        if (u + t < KU) step(u + t, t & 1, t % 3);

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

// Persistent variant of the 128-token x 64-row-per-wave tile (row-major
// activations, padded LDS rows).  The grid holds the resident workgroups;
// each walks its XCD slice of work items.  At the end of a tile's K loop it
// first issues the NEXT tile's first kDepth units of loads, then the
// current tile's output stores: on gfx9 loads and stores share one in-order
// completion counter, so stores issued before the next tile's loads would
// stall its first wait; issued after them, the fp32 output drains while the
// next tile's loop runs instead of in a separate burst.
// Work cursor of a persistent workgroup: slots b, b + stride, ...; a slot
// names a logical item through the XCD-slice order (single problem) or the
// plan's slot map (grouped launch).
struct TileCursor {
    int b;
    int stride;
    int n_slots;
    const Problem *single;
    const Problem *probs;
    const uint2 *item_map;
    int single_items, single_per;  // single-problem cursors (unused by the grouped launch)
};

__device__ inline bool cursor_fetch(TileCursor &c, const Problem *&pp, int &local)
{
    for (; c.b < c.n_slots; c.b += c.stride) {
        if (c.single) {
            const int j = (c.b & 7) * c.single_per + (c.b >> 3);
            if (j < c.single_items) {
                pp = c.single;
                local = j;
                return true;
            }
        } else {
            const uint2 it = c.item_map[c.b];
            if (it.x != 0xFFFFFFFFu) {
                pp = c.probs + it.x;
                local = (int)it.y;
                return true;
            }
        }
    }
    return false;
}

__device__ void tile_persist_body(TileCursor cur)
{
    constexpr int WMS = 4, BM = 128, CH = 2;
    __shared__ __attribute__((aligned(16))) int8_t As[2][BM * kLda];
    __shared__ float cs[BM];
    __shared__ int rsum[BM];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, g = lane >> 5, r = lane & 31;

    const Problem *pp = nullptr;
    int local = 0;
    if (!cursor_fetch(cur, pp, local)) return;

    // per-tile state
    int KU = 0, m0 = 0, tile = 0;
    const BL_GLOBAL v4u *blk = nullptr;
    const BL_GLOBAL int8_t *asrc[CH];
    int adst[CH];
    v4i ar[kDepth][CH];
    v4u br[kDepth];

    auto setup = [&](const Problem &p, int loc) {
        const int mtile = loc % p.mt, nt = loc / p.mt;
        KU = p.KU;
        m0 = mtile * BM;
        tile = 4 * nt + wave;
        blk = gload_ptr<v4u>(p.P + (int64_t)min(tile, p.NT - 1) * KU * kBlockBytes) + lane;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = tid + kThreads * i;
            const int m = min(m0 + (c >> 2), p.M - 1);
            asrc[i] = gload_ptr<int8_t>(p.Q + (int64_t)m * p.ldq + 16 * (c & 3));
            adst[i] = (c >> 2) * kLda + 16 * (c & 3);
        }
    };
    auto load_unit = [&](int slot, int u) {
        const int uc = min(u, KU - 1);
#pragma unroll
        for (int i = 0; i < CH; ++i) ar[slot][i] = *reinterpret_cast<const BL_GLOBAL v4i *>(asrc[i] + 64 * uc);
        br[slot] = blk[(int64_t)uc * 64];
    };
    auto begin_tile = [&](const Problem &p) {
        if (tid < BM) {
            const int m = min(m0 + tid, p.M - 1);
            cs[tid] = (*gload_ptr<float>(p.gamma) * gload_ptr<float>(p.absmax)[m]) / 127.0f;
            rsum[tid] = gload_ptr<int32_t>(p.rowsum)[m];
        }
#pragma unroll
        for (int i = 0; i < CH; ++i) *reinterpret_cast<v4i *>(&As[0][adst[i]]) = ar[0][i];
        __syncthreads();
    };

    v16i acc[WMS][2];
    auto step = [&](int s, int u) {
        const int buf = u & 1;
        const v4u w = br[s];
        const v4i b0 = planes(w.x), b1 = planes(w.y), b2 = planes(w.z), b3 = planes(w.w);
        v4i a[WMS][2];
#pragma unroll
        for (int i = 0; i < WMS; ++i) {
            const int8_t *arow = &As[buf][(32 * i + r) * kLda + 16 * g];
            a[i][0] = *reinterpret_cast<const v4i *>(arow);
            a[i][1] = *reinterpret_cast<const v4i *>(arow + 32);
        }
        load_unit(s, u + kDepth);
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
        const int ns = (s + 1) % kDepth;
#pragma unroll
        for (int i = 0; i < CH; ++i) *reinterpret_cast<v4i *>(&As[buf ^ 1][adst[i]]) = ar[ns][i];
        __syncthreads();
    };

    setup(*pp, local);
#pragma unroll
    for (int d = 0; d < kDepth; ++d) load_unit(d, d);
    begin_tile(*pp);

    bool more = true;
    while (more) {
#pragma unroll
        for (int i = 0; i < WMS; ++i) acc[i][0] = acc[i][1] = (v16i){};
        int u0 = 0;
        for (; u0 + kDepth <= KU; u0 += kDepth) {
#pragma unroll
            for (int s = 0; s < kDepth; ++s) step(s, u0 + s);
        }
#pragma unroll
        for (int s = 0; s < kDepth - 1; ++s)
            if (u0 + s < KU) step(s, u0 + s);

        // this tile's output coordinates, then the next tile's first loads
        const Problem *pc = pp;
        const int c_m0 = m0, c_tile = tile;
        cur.b += cur.stride;
        more = cursor_fetch(cur, pp, local);
        if (more) {
            setup(*pp, local);
#pragma unroll
            for (int d = 0; d < kDepth; ++d) load_unit(d, d);
        }
        // epilogue of the finished tile (its scales are still in LDS)
        const int M = pc->M, N = pc->N;
        if (c_tile < pc->NT) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const int n = 64 * c_tile + 32 * s2 + r;
                if (n >= N) continue;
#pragma unroll
                for (int i = 0; i < WMS; ++i) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int row = 32 * i + 8 * (e >> 2) + 4 * g + (e & 3);
                        const int m = c_m0 + row;
                        if (m < M) {
                            const int32_t a = acc[i][s2][e] - rsum[row];
                            const int64_t o = (int64_t)m * N + n;
                            gstore_ptr<float>(pc->Y)[o] = (float)a * cs[row];
                            if (pc->acc_out) gstore_ptr<int32_t>(pc->acc_out)[o] = a;
                        }
                    }
                }
            }
        }
        if (more) {
            __syncthreads();  // every wave has read this tile's scales
            begin_tile(*pp);
        }
    }
}

template <int V>
__global__ __launch_bounds__(kThreads, 2) void tile_persist_group_kernel(const Problem *__restrict__ probs,
                                                                         const uint2 *__restrict__ item_map,
                                                                         int n_slots)
{
    TileCursor c{(int)blockIdx.x, (int)gridDim.x, n_slots, nullptr, probs, item_map, 0, 0};
    tile_persist_body(c);
}

// Persistent tile kernel whose fp32 outputs leave during the next tile's
// K loop.  Tile = 64 tokens x 256 weight rows (four waves, 64 rows each).
// At the end of a tile's K loop the rescaled outputs are written to an LDS
// staging tile (64 x 256 fp32); during the next tile's loop each wave sends
// one 1 KiB staged row to Y per unit (16 rows per wave), so the output
// stream, the largest HBM stream of a prefill contraction, runs under the
// MFMAs instead of in a burst after them.  The drain stores are buffer
// stores whose record count is 0 when there is nothing to send (the
// hardware drops out-of-range lanes), so every unit issues the same memory
// instructions and the load ring keeps static wait counts.  LDS: 10 KiB
// activation stages + 66 KiB output stage per workgroup, two per CU.
constexpr int kDrainBM = 64;
constexpr int kYsStride = 264;  // floats per staged row: rows 4 apart land 32 banks apart
constexpr int kDrainRows = kDrainBM / 4;  // rows each wave sends per tile

// the staged tile still to be sent (wave-uniform values)
struct DrainState {
    float *Y;
    int64_t N;
    int m0, rows, n0, bytes;  // rows == 0: nothing staged
};

__device__ __forceinline__ void tile_drain_body(TileCursor cur)
{
    constexpr int WMS = 2, BM = kDrainBM, CH = 1;
    __shared__ __attribute__((aligned(16))) int8_t As[2][BM * kLda];
    __shared__ __attribute__((aligned(16))) float Ys[BM * kYsStride];
    __shared__ float cs[BM];
    __shared__ int rsum[BM];
    const int tid = threadIdx.x;
    const int lane = tid & 63, g = lane >> 5, r = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    const Problem *pp = nullptr;
    int local = 0;
    if (!cursor_fetch(cur, pp, local)) return;

    int KU = 0, m0 = 0, tile = 0;
    const BL_GLOBAL v4u *blk = nullptr;
    const BL_GLOBAL int8_t *asrc[CH];
    int adst[CH];
    v4i ar[kDepth][CH];
    v4u br[kDepth];
    DrainState d{nullptr, 0, 0, 0, 0, 0};

    auto setup = [&](const Problem &p, int loc) {
        const int mtile = loc % p.mt, nt = loc / p.mt;
        KU = p.KU;
        m0 = mtile * BM;
        tile = 4 * nt + wave;
        blk = gload_ptr<v4u>(p.P + (int64_t)min(tile, p.NT - 1) * KU * kBlockBytes) + lane;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = tid + kThreads * i;
            const int m = min(m0 + (c >> 2), p.M - 1);
            asrc[i] = gload_ptr<int8_t>(p.Q + (int64_t)m * p.ldq + 16 * (c & 3));
            adst[i] = (c >> 2) * kLda + 16 * (c & 3);
        }
    };
    auto load_unit = [&](int slot, int u) {
        const int uc = min(u, KU - 1);
#pragma unroll
        for (int i = 0; i < CH; ++i) ar[slot][i] = *reinterpret_cast<const BL_GLOBAL v4i *>(asrc[i] + 64 * uc);
        br[slot] = blk[(int64_t)uc * 64];
    };
    auto begin_tile = [&](const Problem &p) {
        if (tid < BM) {
            const int m = min(m0 + tid, p.M - 1);
            cs[tid] = (*gload_ptr<float>(p.gamma) * gload_ptr<float>(p.absmax)[m]) / 127.0f;
            rsum[tid] = gload_ptr<int32_t>(p.rowsum)[m];
        }
#pragma unroll
        for (int i = 0; i < CH; ++i) *reinterpret_cast<v4i *>(&As[0][adst[i]]) = ar[0][i];
        __syncthreads();
    };
    // staged row j (< kDrainRows) of this wave -> Y; j >= kDrainRows sends nothing
    auto drain_row = [&](int j) {
        const int jr = min(j, kDrainRows - 1);
        const int rt = 4 * jr + wave;
        const v4u v = *reinterpret_cast<const v4u *>(&Ys[rt * kYsStride + 4 * lane]);
        const bool ok = j < kDrainRows && rt < d.rows;
        float *base = d.Y + ((int64_t)d.m0 + (ok ? rt : 0)) * d.N + d.n0;
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc(base, (short)0, ok ? d.bytes : 0, 0x00020000);
        __builtin_amdgcn_raw_buffer_store_b128(v, rs, 16 * lane, 0, 2 /* non-temporal */);
    };

    v16i acc[WMS][2];
    auto step = [&](int s, int u) {
        // keep each unit's work inside its own step: hoisting a later unit's
        // plane extraction would wait on loads that are still in flight
        __builtin_amdgcn_sched_barrier(0);
        const int buf = u & 1;
        const v4u w = br[s];
        const v4i b0 = planes(w.x), b1 = planes(w.y), b2 = planes(w.z), b3 = planes(w.w);
        v4i a[WMS][2];
#pragma unroll
        for (int i = 0; i < WMS; ++i) {
            const int8_t *arow = &As[buf][(32 * i + r) * kLda + 16 * g];
            a[i][0] = *reinterpret_cast<const v4i *>(arow);
            a[i][1] = *reinterpret_cast<const v4i *>(arow + 32);
        }
        // slot s is refilled only after its previous contents became planes,
        // so the ring slots keep fixed registers across iterations
        __builtin_amdgcn_sched_barrier(0);
        load_unit(s, u + kDepth);
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
        const int ns = (s + 1) % kDepth;
#pragma unroll
        for (int i = 0; i < CH; ++i) *reinterpret_cast<v4i *>(&As[buf ^ 1][adst[i]]) = ar[ns][i];
        // the drain goes last: its LDS read shares the barrier's wait, and
        // placed between the MFMAs it made the compiler copy ring registers
        // that still had loads in flight
        drain_row(u);
        __syncthreads();
    };

    // The ring registers are filled and drained within one pass of the tile
    // loop (nothing in flight crosses its back-edge), which keeps them in
    // fixed registers; the previous tile's staged outputs are what carries
    // over.
    do {
        setup(*pp, local);
#pragma unroll
        for (int d0 = 0; d0 < kDepth; ++d0) load_unit(d0, d0);
        begin_tile(*pp);
#pragma unroll
        for (int i = 0; i < WMS; ++i) acc[i][0] = acc[i][1] = (v16i){};
        int u0 = 0;
        for (; u0 + kDepth <= KU; u0 += kDepth) {
#pragma unroll
            for (int s = 0; s < kDepth; ++s) step(s, u0 + s);
        }
#pragma unroll
        for (int s = 0; s < kDepth - 1; ++s)
            if (u0 + s < KU) step(s, u0 + s);
        // a loop shorter than kDrainRows units leaves staged rows behind
        for (int j = KU; j < kDrainRows; ++j) drain_row(j);
        __syncthreads();  // every staged row has been read

        // this tile's outputs -> LDS stage (or straight to Y when its rows are
        // not 16-byte aligned pieces)
        const Problem &pc = *pp;
        const int M = pc.M, N = pc.N;
        const bool staged = (N & 3) == 0 && (reinterpret_cast<uintptr_t>(pc.Y) & 15) == 0;
        const int n0 = 256 * (tile >> 2);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const int col = 64 * wave + 32 * s2 + r;
            const int n = n0 + col;
#pragma unroll
            for (int i = 0; i < WMS; ++i) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = 32 * i + 8 * (e >> 2) + 4 * g + (e & 3);
                    const int32_t a = acc[i][s2][e] - rsum[row];
                    const float y = (float)a * cs[row];
                    Ys[row * kYsStride + col] = y;
                    const int m = m0 + row;
                    if (m < M && n < N) {
                        const int64_t o = (int64_t)m * N + n;
                        if (!staged) gstore_ptr<float>(pc.Y)[o] = y;
                        if (pc.acc_out) gstore_ptr<int32_t>(pc.acc_out)[o] = a;
                    }
                }
            }
        }
        d.Y = pc.Y;
        d.N = N;
        d.m0 = m0;
        d.n0 = n0;
        d.rows = staged ? min(BM, M - m0) : 0;
        d.bytes = 4 * min(256, N - n0);
        __syncthreads();  // the stage is complete and every wave has read the scales
        cur.b += cur.stride;
    } while (cursor_fetch(cur, pp, local));
    for (int j = 0; j < kDrainRows; ++j) drain_row(j);
}

template <int V>
__global__ __launch_bounds__(kThreads, 2) void tile_drain_group_kernel(const Problem *__restrict__ probs,
                                                                       const uint2 *__restrict__ item_map,
                                                                       int n_slots)
{
    TileCursor c{(int)blockIdx.x, (int)gridDim.x, n_slots, nullptr, probs, item_map, 0, 0};
    tile_drain_body(c);
}

// Wave-specialized persistent tile kernel: 320-thread workgroups, two per
// CU.  Waves 0-3 compute 64-token x 256-row tiles exactly like the 64-token
// LDS-staged kernel, but end each tile by writing the rescaled outputs to an
// LDS stage instead of storing them; wave 4 sends the previous tile's staged
// rows (1 KiB each) to Y while the compute waves run the next tile's K loop,
// and takes part in every barrier of that loop.  The output stream
// thus runs under the MFMAs, and since the store waves issue no loads, the
// single in-order memory counter never makes a compute wave wait for a
// store.  LDS per workgroup: 10 KiB activation stages + 66 KiB output stage.
constexpr int kWsThreads = 320;
// The kernel is declared for up to 512 threads so that the compiler budgets
// registers for four waves per SIMD (<= 128 VGPRs): the first and fifth wave
// of a 5-wave workgroup share a SIMD, so two co-resident workgroups put four
// waves on it.

template <int V>
__global__ __launch_bounds__(512, 4) void tile_ws_group_kernel(const Problem *__restrict__ probs,
                                                                      const uint2 *__restrict__ item_map,
                                                                      int n_slots)
{
    constexpr int WMS = 2, BM = kDrainBM, CH = 1;
    __shared__ __attribute__((aligned(16))) int8_t As[2][BM * kLda];
    __shared__ __attribute__((aligned(16))) float Ys[BM * kYsStride];
    __shared__ float cs[BM];
    __shared__ int rsum[BM];
    const int tid = threadIdx.x;
    const int lane = tid & 63, g = lane >> 5, r = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool compute = wave < 4;
    const int cw = wave & 3;  // compute wave index

    TileCursor cur{(int)blockIdx.x, (int)gridDim.x, n_slots, nullptr, probs, item_map, 0, 0};
    const Problem *pp = nullptr;
    int local = 0;
    if (!cursor_fetch(cur, pp, local)) return;

    int KU = 0, m0 = 0, tile = 0;
    const BL_GLOBAL v4u *blk = nullptr;
    const BL_GLOBAL int8_t *asrc = nullptr;
    int adst = 0;
    v4i ar[kDepth];
    v4u br[kDepth];
    DrainState d{nullptr, 0, 0, 0, 0, 0};

    auto setup = [&](const Problem &p, int loc) {
        const int mtile = loc % p.mt, nt = loc / p.mt;
        KU = p.KU;
        m0 = mtile * BM;
        tile = 4 * nt + cw;
        blk = gload_ptr<v4u>(p.P + (int64_t)min(tile, p.NT - 1) * KU * kBlockBytes) + lane;
        const int c = tid & 255;
        const int m = min(m0 + (c >> 2), p.M - 1);
        asrc = gload_ptr<int8_t>(p.Q + (int64_t)m * p.ldq + 16 * (c & 3));
        adst = (c >> 2) * kLda + 16 * (c & 3);
    };
    auto load_unit = [&](int slot, int u) {
        const int uc = min(u, KU - 1);
        ar[slot] = *reinterpret_cast<const BL_GLOBAL v4i *>(asrc + 64 * uc);
        br[slot] = blk[(int64_t)uc * 64];
    };
    // the store wave sends staged rows [j0, j1)
    auto drain_rows = [&](int j0, int j1) {
        for (int rt = j0; rt < j1; ++rt) {
            if (rt < d.rows && 16 * lane < d.bytes) {
                const v4f_t v = *reinterpret_cast<const v4f_t *>(&Ys[rt * kYsStride + 4 * lane]);
                __builtin_nontemporal_store(
                    v, reinterpret_cast<BL_GLOBAL v4f_t *>(gstore_ptr<float>(d.Y) + ((int64_t)d.m0 + rt) * d.N + d.n0) +
                           lane);
            }
        }
    };

    v16i acc[WMS][2];
    // Register budget (two 5-wave workgroups per CU need <= 128 VGPRs): the
    // planes of each half unit are extracted right before its MFMAs and the
    // activation operands are read one half at a time.
    auto step = [&](int s, int u) {
        __builtin_amdgcn_sched_barrier(0);
        const int buf = u & 1;
        const v4u w = br[s];
        const int8_t *arow = &As[buf][r * kLda + 16 * g];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            v4i a[WMS];
#pragma unroll
            for (int i = 0; i < WMS; ++i) a[i] = *reinterpret_cast<const v4i *>(arow + 32 * i * kLda + 32 * h);
            const v4i bl = planes(h ? w.y : w.x), bh = planes(h ? w.w : w.z);
            __builtin_amdgcn_sched_barrier(0);
            if (h == 0) load_unit(s, u + kDepth);  // slot s is free once w is read
#pragma unroll
            for (int i = 0; i < WMS; ++i) {
                acc[i][0] = mfma_i8(a[i], bl, acc[i][0]);
                acc[i][1] = mfma_i8(a[i], bh, acc[i][1]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        const int ns = (s + 1) % kDepth;
        *reinterpret_cast<v4i *>(&As[buf ^ 1][adst]) = ar[ns];
        __syncthreads();
    };

    // The two roles walk the same work list and meet at the same barriers:
    // one at a tile's start, one per unit of its K loop, two at its end.
    if (!compute) {
        do {
            const int ku = pp->KU;
            __syncthreads();  // tile start
            // the previous tile's BM rows, spread over this tile's loop
            for (int u = 0; u < ku; ++u) {
                drain_rows((u * BM + ku - 1) / ku, ((u + 1) * BM + ku - 1) / ku);
                __syncthreads();
            }
            __syncthreads();  // the stage has been read
            const Problem &pc = *pp;
            const bool staged = (pc.N & 3) == 0 && (reinterpret_cast<uintptr_t>(pc.Y) & 15) == 0;
            d.Y = pc.Y;
            d.N = pc.N;
            d.m0 = (local % pc.mt) * BM;
            d.n0 = 256 * (local / pc.mt);
            d.rows = staged ? min(BM, pc.M - d.m0) : 0;
            d.bytes = 4 * min(256, pc.N - d.n0);
            __syncthreads();  // the stage holds this tile
            cur.b += cur.stride;
        } while (cursor_fetch(cur, pp, local));
        drain_rows(0, BM);
        return;
    }

    do {
        setup(*pp, local);
#pragma unroll
        for (int d0 = 0; d0 < kDepth; ++d0) load_unit(d0, d0);
        if (tid < BM) {
            const int m = min(m0 + tid, pp->M - 1);
            cs[tid] = (*gload_ptr<float>(pp->gamma) * gload_ptr<float>(pp->absmax)[m]) / 127.0f;
            rsum[tid] = gload_ptr<int32_t>(pp->rowsum)[m];
        }
        *reinterpret_cast<v4i *>(&As[0][adst]) = ar[0];
        __syncthreads();  // tile start

#pragma unroll
        for (int i = 0; i < WMS; ++i) acc[i][0] = acc[i][1] = (v16i){};
        int u0 = 0;
        for (; u0 + kDepth <= KU; u0 += kDepth) {
#pragma unroll
            for (int s = 0; s < kDepth; ++s) step(s, u0 + s);
        }
#pragma unroll
        for (int s = 0; s < kDepth - 1; ++s)
            if (u0 + s < KU) step(s, u0 + s);
        __syncthreads();  // the stage has been read

        const Problem &pc = *pp;
        const int M = pc.M, N = pc.N;
        const bool staged = (N & 3) == 0 && (reinterpret_cast<uintptr_t>(pc.Y) & 15) == 0;
        const int n0 = 256 * (tile >> 2);
        // one 32-row block at a time: its 16 scales and row sums per lane
        // plus the accumulators fit the register budget
#pragma unroll
        for (int i = 0; i < WMS; ++i) {
            __builtin_amdgcn_sched_barrier(0);
            float csv[16];
            int rsv[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = 32 * i + 8 * (e >> 2) + 4 * g + (e & 3);
                csv[e] = cs[row];
                rsv[e] = rsum[row];
            }
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const int col = 64 * cw + 32 * s2 + r;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = 32 * i + 8 * (e >> 2) + 4 * g + (e & 3);
                    Ys[row * kYsStride + col] = (float)(acc[i][s2][e] - rsv[e]) * csv[e];
                }
            }
        }
        if (!staged || pc.acc_out) {
            // rows that are not 16-byte pieces, and the optional int32 sums
            for (int i = 0; i < WMS; ++i)
                for (int s2 = 0; s2 < 2; ++s2)
                    for (int e = 0; e < 16; ++e) {
                        const int row = 32 * i + 8 * (e >> 2) + 4 * g + (e & 3);
                        const int n = n0 + 64 * cw + 32 * s2 + r;
                        const int m = m0 + row;
                        if (m < M && n < N) {
                            const int32_t a = acc[i][s2][e] - rsum[row];
                            const int64_t o = (int64_t)m * N + n;
                            if (!staged) gstore_ptr<float>(pc.Y)[o] = (float)a * cs[row];
                            if (pc.acc_out) gstore_ptr<int32_t>(pc.acc_out)[o] = a;
                        }
                    }
        }
        __syncthreads();  // the stage holds this tile; the scales are free
        cur.b += cur.stride;
    } while (cursor_fetch(cur, pp, local));
}

// Wave-specialized persistent tile kernel, one 576-thread workgroup per CU:
// tile = 128 tokens x 256 weight rows.  Waves 0-7 compute (two per SIMD,
// each 64 tokens x 64 rows: two 64-token halves x four 64-row weight
// tiles) and end each tile by writing the rescaled outputs to an LDS stage;
// wave 8 sends the previous tile's staged rows to Y during the next tile's
// K loop and meets the compute waves at every barrier.  LDS: 20 KiB
// activation stages + 132 KiB output stage.
constexpr int kWs2Threads = 576;

template <int V>
__global__ __launch_bounds__(kWs2Threads) void tile_ws2_group_kernel(const Problem *__restrict__ probs,
                                                                      const uint2 *__restrict__ item_map,
                                                                      int n_slots)
{
    constexpr int WMS = 2, BM = 2 * kDrainBM, CH = 1;
    __shared__ __attribute__((aligned(16))) int8_t As[2][BM * kLda];
    __shared__ __attribute__((aligned(16))) float Ys[BM * kYsStride];
    __shared__ float cs[BM];
    __shared__ int rsum[BM];
    const int tid = threadIdx.x;
    const int lane = tid & 63, g = lane >> 5, r = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool compute = wave < 8;
    const int cw = wave & 3;  // weight tile of a compute wave
    const int wm = (wave >> 2) & 1;  // 64-token half of a compute wave

    TileCursor cur{(int)blockIdx.x, (int)gridDim.x, n_slots, nullptr, probs, item_map, 0, 0};
    const Problem *pp = nullptr;
    int local = 0;
    if (!cursor_fetch(cur, pp, local)) return;

    int KU = 0, m0 = 0, tile = 0;
    const BL_GLOBAL v4u *blk = nullptr;
    const BL_GLOBAL int8_t *asrc = nullptr;
    int adst = 0;
    v4i ar[kDepth];
    v4u br[kDepth];
    DrainState d{nullptr, 0, 0, 0, 0, 0};

    auto setup = [&](const Problem &p, int loc) {
        const int mtile = loc % p.mt, nt = loc / p.mt;
        KU = p.KU;
        m0 = mtile * BM;
        tile = 4 * nt + cw;
        blk = gload_ptr<v4u>(p.P + (int64_t)min(tile, p.NT - 1) * KU * kBlockBytes) + lane;
        const int c = tid & 511;
        const int m = min(m0 + (c >> 2), p.M - 1);
        asrc = gload_ptr<int8_t>(p.Q + (int64_t)m * p.ldq + 16 * (c & 3));
        adst = (c >> 2) * kLda + 16 * (c & 3);
    };
    auto load_unit = [&](int slot, int u) {
        const int uc = min(u, KU - 1);
        ar[slot] = *reinterpret_cast<const BL_GLOBAL v4i *>(asrc + 64 * uc);
        br[slot] = blk[(int64_t)uc * 64];
    };
    // the store wave sends staged rows [j0, j1)
    auto drain_rows = [&](int j0, int j1) {
        for (int rt = j0; rt < j1; ++rt) {
            if (rt < d.rows && 16 * lane < d.bytes) {
                const v4f_t v = *reinterpret_cast<const v4f_t *>(&Ys[rt * kYsStride + 4 * lane]);
                __builtin_nontemporal_store(
                    v, reinterpret_cast<BL_GLOBAL v4f_t *>(gstore_ptr<float>(d.Y) + ((int64_t)d.m0 + rt) * d.N + d.n0) +
                           lane);
            }
        }
    };

    v16i acc[WMS][2];
    // Register budget (two 5-wave workgroups per CU need <= 128 VGPRs): the
    // planes of each half unit are extracted right before its MFMAs and the
    // activation operands are read one half at a time.
    auto step = [&](int s, int u) {
        __builtin_amdgcn_sched_barrier(0);
        const int buf = u & 1;
        const v4u w = br[s];
        const int8_t *arow = &As[buf][(64 * wm + r) * kLda + 16 * g];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            v4i a[WMS];
#pragma unroll
            for (int i = 0; i < WMS; ++i) a[i] = *reinterpret_cast<const v4i *>(arow + 32 * i * kLda + 32 * h);
            const v4i bl = planes(h ? w.y : w.x), bh = planes(h ? w.w : w.z);
            __builtin_amdgcn_sched_barrier(0);
            if (h == 0) load_unit(s, u + kDepth);  // slot s is free once w is read
#pragma unroll
            for (int i = 0; i < WMS; ++i) {
                acc[i][0] = mfma_i8(a[i], bl, acc[i][0]);
                acc[i][1] = mfma_i8(a[i], bh, acc[i][1]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        const int ns = (s + 1) % kDepth;
        *reinterpret_cast<v4i *>(&As[buf ^ 1][adst]) = ar[ns];
        __syncthreads();
    };

    // The two roles walk the same work list and meet at the same barriers:
    // one at a tile's start, one per unit of its K loop, two at its end.
    if (!compute) {
        do {
            const int ku = pp->KU;
            __syncthreads();  // tile start
            // the previous tile's BM rows, spread over this tile's loop
            for (int u = 0; u < ku; ++u) {
                drain_rows((u * BM + ku - 1) / ku, ((u + 1) * BM + ku - 1) / ku);
                __syncthreads();
            }
            __syncthreads();  // the stage has been read
            const Problem &pc = *pp;
            const bool staged = (pc.N & 3) == 0 && (reinterpret_cast<uintptr_t>(pc.Y) & 15) == 0;
            d.Y = pc.Y;
            d.N = pc.N;
            d.m0 = (local % pc.mt) * BM;
            d.n0 = 256 * (local / pc.mt);
            d.rows = staged ? min(BM, pc.M - d.m0) : 0;
            d.bytes = 4 * min(256, pc.N - d.n0);
            __syncthreads();  // the stage holds this tile
            cur.b += cur.stride;
        } while (cursor_fetch(cur, pp, local));
        drain_rows(0, BM);
        return;
    }

    do {
        setup(*pp, local);
#pragma unroll
        for (int d0 = 0; d0 < kDepth; ++d0) load_unit(d0, d0);
        if (tid < BM) {
            const int m = min(m0 + tid, pp->M - 1);
            cs[tid] = (*gload_ptr<float>(pp->gamma) * gload_ptr<float>(pp->absmax)[m]) / 127.0f;
            rsum[tid] = gload_ptr<int32_t>(pp->rowsum)[m];
        }
        *reinterpret_cast<v4i *>(&As[0][adst]) = ar[0];
        __syncthreads();  // tile start

#pragma unroll
        for (int i = 0; i < WMS; ++i) acc[i][0] = acc[i][1] = (v16i){};
        int u0 = 0;
        for (; u0 + kDepth <= KU; u0 += kDepth) {
#pragma unroll
            for (int s = 0; s < kDepth; ++s) step(s, u0 + s);
        }
#pragma unroll
        for (int s = 0; s < kDepth - 1; ++s)
            if (u0 + s < KU) step(s, u0 + s);
        __syncthreads();  // the stage has been read

        const Problem &pc = *pp;
        const int M = pc.M, N = pc.N;
        const bool staged = (N & 3) == 0 && (reinterpret_cast<uintptr_t>(pc.Y) & 15) == 0;
        const int n0 = 256 * (tile >> 2);
        // one 32-row block at a time: its 16 scales and row sums per lane
        // plus the accumulators fit the register budget
#pragma unroll
        for (int i = 0; i < WMS; ++i) {
            __builtin_amdgcn_sched_barrier(0);
            float csv[16];
            int rsv[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = 64 * wm + 32 * i + 8 * (e >> 2) + 4 * g + (e & 3);
                csv[e] = cs[row];
                rsv[e] = rsum[row];
            }
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const int col = 64 * cw + 32 * s2 + r;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = 64 * wm + 32 * i + 8 * (e >> 2) + 4 * g + (e & 3);
                    Ys[row * kYsStride + col] = (float)(acc[i][s2][e] - rsv[e]) * csv[e];
                }
            }
        }
        if (!staged || pc.acc_out) {
            // rows that are not 16-byte pieces, and the optional int32 sums
            for (int i = 0; i < WMS; ++i)
                for (int s2 = 0; s2 < 2; ++s2)
                    for (int e = 0; e < 16; ++e) {
                        const int row = 64 * wm + 32 * i + 8 * (e >> 2) + 4 * g + (e & 3);
                        const int n = n0 + 64 * cw + 32 * s2 + r;
                        const int m = m0 + row;
                        if (m < M && n < N) {
                            const int32_t a = acc[i][s2][e] - rsum[row];
                            const int64_t o = (int64_t)m * N + n;
                            if (!staged) gstore_ptr<float>(pc.Y)[o] = (float)a * cs[row];
                            if (pc.acc_out) gstore_ptr<int32_t>(pc.acc_out)[o] = a;
                        }
                    }
        }
        __syncthreads();  // the stage holds this tile; the scales are free
        cur.b += cur.stride;
    } while (cursor_fetch(cur, pp, local));
}

// Persistent form of the 128-token tile with the LDS-transposed epilogue:
// the resident workgroups walk the work list, one tile body per item (its
// load ring lives within the item).  Two workgroups share each CU; started
// together they would reach their epilogues together, every CU storing at
// once while its matrix cores idle.  The second half of the grid therefore
// starts `stagger` ticks of the 100 MHz real-time counter late, so that on
// each CU one workgroup's output burst falls inside the other's K loop.
template <int V>
__global__ __launch_bounds__(kThreads, 2) void tile_persist_epi_kernel(const Problem *__restrict__ probs,
                                                                       const uint2 *__restrict__ item_map,
                                                                       int n_slots, int stagger)
{
    if (stagger > 0 && blockIdx.x >= gridDim.x / 2) {
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        while (__builtin_amdgcn_s_memrealtime() - t0 < (uint64_t)stagger) __builtin_amdgcn_s_sleep(8);
    }
    for (int b = blockIdx.x; b < n_slots; b += gridDim.x) {
        const uint2 it = item_map[b];
        if (it.x != 0xFFFFFFFFu) tile_body<4, 1, 1, 0, true>(probs[it.x], (int)it.y);
    }
}

// resident workgroups of a kernel on the current device, a multiple of 8
template <typename Kern>
int resident_grid(Kern kernel)
{
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 8;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 8;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) != hipSuccess) return 8;
    const int g = (cus * per_cu) & ~7;
    return g < 8 ? 8 : g;
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
        tile_body<2, 1, 1, 0>(p, local);
    else if constexpr (V == 1)
        tile_body<2, 2, 2, 0>(p, local);
    else if constexpr (V == 2)
        tile_body<4, 1, 1, 0>(p, local);
    else if constexpr (V == 3)
        tile_direct_body<true>(p, local);
    else if constexpr (V == 4)
        tile_direct_body<false>(p, local);
    else if constexpr (V == 5)
        tile_body<4, 1, 1, 1>(p, local);
    else if constexpr (V == 6)
        tile_body<2, 1, 1, 1>(p, local);
    else if constexpr (V == 7)
        tile_body<2, 2, 2, 1>(p, local);
    else if constexpr (V == 8)
        tile_pipe_body<2>(p, local);
    else if constexpr (V == 9)
        tile_pipe_body<4>(p, local);
    else if constexpr (V == 10)
        tile_body<4, 1, 1, 2, true>(p, local);
    else if constexpr (V == 11)
        tile_body<4, 1, 1, 0, true>(p, local);
    else if constexpr (V == 18)
        tile_body_ups<2>(p, local);
    else
        tile_body<4, 1, 1, 2, false>(p, local);
}

template <int V>
constexpr int tile_min_waves()
{
    return (V == 3 || V == 4 || V == 9) ? 1 : 2;
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
    // the persistent variants walk device-side plans only
    if (variant == 13) variant = 2;
    if (variant == 14 || variant == 15) variant = 0;   // same 64-token tile, not persistent
    if (variant == 16 || variant == 17) variant = 11;
    switch (variant) {
    case 0: hipLaunchKernelGGL(tile_single_kernel<0>, grid, block, 0, s, p, items, per); break;
    case 1: hipLaunchKernelGGL(tile_single_kernel<1>, grid, block, 0, s, p, items, per); break;
    case 2: hipLaunchKernelGGL(tile_single_kernel<2>, grid, block, 0, s, p, items, per); break;
    case 3: hipLaunchKernelGGL(tile_single_kernel<3>, grid, block, 0, s, p, items, per); break;
    case 4: hipLaunchKernelGGL(tile_single_kernel<4>, grid, block, 0, s, p, items, per); break;
    case 5: hipLaunchKernelGGL(tile_single_kernel<5>, grid, block, 0, s, p, items, per); break;
    case 6: hipLaunchKernelGGL(tile_single_kernel<6>, grid, block, 0, s, p, items, per); break;
    case 7: hipLaunchKernelGGL(tile_single_kernel<7>, grid, block, 0, s, p, items, per); break;
    case 8: hipLaunchKernelGGL(tile_single_kernel<8>, grid, block, 0, s, p, items, per); break;
    case 9: hipLaunchKernelGGL(tile_single_kernel<9>, grid, block, 0, s, p, items, per); break;
    case 10: hipLaunchKernelGGL(tile_single_kernel<10>, grid, block, 0, s, p, items, per); break;
    case 11: hipLaunchKernelGGL(tile_single_kernel<11>, grid, block, 0, s, p, items, per); break;
    case 18: hipLaunchKernelGGL(tile_single_kernel<18>, grid, block, 0, s, p, items, per); break;
    default: hipLaunchKernelGGL(tile_single_kernel<12>, grid, block, 0, s, p, items, per); break;
    }
    return hipGetLastError();
}

hipError_t launch_tile_group(const Problem *probs, const uint2 *item_map, int n_items,
                             int variant, hipStream_t s)
{
    const dim3 grid((unsigned)n_items), block(kThreads);
    if (variant == 13) {
        const int g = resident_grid(tile_persist_group_kernel<13>);
        const dim3 pg((unsigned)(n_items < g ? n_items : g));
        hipLaunchKernelGGL(tile_persist_group_kernel<13>, pg, block, 0, s, probs, item_map, n_items);
        return hipGetLastError();
    }
    if (variant == 17) {
        int dev = 0, cus = 0, per_cu = 0;
        hipGetDevice(&dev);
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, tile_ws2_group_kernel<17>, kWs2Threads, 0);
        int g = (cus * per_cu) & ~7;
        if (g < 8) g = 8;
        const dim3 pg((unsigned)(n_items < g ? n_items : g));
        hipLaunchKernelGGL(tile_ws2_group_kernel<17>, pg, dim3(kWs2Threads), 0, s, probs, item_map, n_items);
        return hipGetLastError();
    }
    if (variant == 16) {
        static const int stagger = [] {
            const char *e = getenv("BITLINEAR_TILE_STAGGER");
            return e ? atoi(e) : 2000;
        }();
        const int g = resident_grid(tile_persist_epi_kernel<16>);
        const dim3 pg((unsigned)(n_items < g ? n_items : g));
        hipLaunchKernelGGL(tile_persist_epi_kernel<16>, pg, block, 0, s, probs, item_map, n_items, stagger);
        return hipGetLastError();
    }
    if (variant == 15) {
        int dev = 0, cus = 0, per_cu = 0;
        hipGetDevice(&dev);
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, tile_ws_group_kernel<15>, kWsThreads, 0);
        int g = (cus * per_cu) & ~7;
        if (g < 8) g = 8;
        const dim3 pg((unsigned)(n_items < g ? n_items : g));
        hipLaunchKernelGGL(tile_ws_group_kernel<15>, pg, dim3(kWsThreads), 0, s, probs, item_map, n_items);
        return hipGetLastError();
    }
    if (variant == 14) {
        const int g = resident_grid(tile_drain_group_kernel<14>);
        const dim3 pg((unsigned)(n_items < g ? n_items : g));
        hipLaunchKernelGGL(tile_drain_group_kernel<14>, pg, block, 0, s, probs, item_map, n_items);
        return hipGetLastError();
    }
    switch (variant) {
    case 0: hipLaunchKernelGGL(tile_group_kernel<0>, grid, block, 0, s, probs, item_map); break;
    case 1: hipLaunchKernelGGL(tile_group_kernel<1>, grid, block, 0, s, probs, item_map); break;
    case 2: hipLaunchKernelGGL(tile_group_kernel<2>, grid, block, 0, s, probs, item_map); break;
    case 3: hipLaunchKernelGGL(tile_group_kernel<3>, grid, block, 0, s, probs, item_map); break;
    case 4: hipLaunchKernelGGL(tile_group_kernel<4>, grid, block, 0, s, probs, item_map); break;
    case 5: hipLaunchKernelGGL(tile_group_kernel<5>, grid, block, 0, s, probs, item_map); break;
    case 6: hipLaunchKernelGGL(tile_group_kernel<6>, grid, block, 0, s, probs, item_map); break;
    case 7: hipLaunchKernelGGL(tile_group_kernel<7>, grid, block, 0, s, probs, item_map); break;
    case 8: hipLaunchKernelGGL(tile_group_kernel<8>, grid, block, 0, s, probs, item_map); break;
    case 9: hipLaunchKernelGGL(tile_group_kernel<9>, grid, block, 0, s, probs, item_map); break;
    case 10: hipLaunchKernelGGL(tile_group_kernel<10>, grid, block, 0, s, probs, item_map); break;
    case 11: hipLaunchKernelGGL(tile_group_kernel<11>, grid, block, 0, s, probs, item_map); break;
    case 18: hipLaunchKernelGGL(tile_group_kernel<18>, grid, block, 0, s, probs, item_map); break;
    default: hipLaunchKernelGGL(tile_group_kernel<12>, grid, block, 0, s, probs, item_map); break;
    }
    return hipGetLastError();
}

}  // namespace bl
