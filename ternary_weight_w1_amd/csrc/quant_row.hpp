// Cast of one token row to int8 codes by one workgroup, shared by the
// activation-quantization kernels and the contraction kernels that cast
// their own input (a decode layer's norm or gate followed by a BitLinear).
//
// anthology note-168 on arXiv 2402.17764, "What it does": BitLinear's
// activations are 8-bit.  Reading implemented (the pages print no formula):
// a = max(1e-5, max_k |x_k|) for each token, s = 127 / a (one fp32 IEEE
// division per token), q_k = clamp(rint(x_k * s), -127, 127).  The row sum
// of q is produced too: the contraction kernels multiply by (code + 1)
// fields and subtract it once per output.  The max is order-free and the
// row sum is an integer sum, so both are exact whatever the reduction order.
#pragma once

#include "common.hpp"

namespace bl {

typedef float v4f __attribute__((ext_vector_type(4)));

// Where code k of the row goes: row-major (Q + m*ldq + k) or fragment order
// in global memory.  In both layouts each aligned 16-code chunk is 16
// contiguous bytes.
struct QDest {
    int8_t *Q;
    int64_t ldq;  // row-major stride; unused in fragment order
    int64_t m;
    int64_t KU;
    int tiled;
    __device__ int64_t at(int64_t k) const { return tiled ? qf32_offset(m, k, KU) : m * ldq + k; }
    __device__ int64_t fill_end() const { return tiled ? 64 * KU : ldq; }
    __device__ void put4(int64_t k, uint32_t codes) const
    {
        *reinterpret_cast<BL_GLOBAL uint32_t *>(gstore_ptr<int8_t>(Q) + at(k)) = codes;
    }
    __device__ void put1(int64_t k, int8_t c) const { gstore_ptr<int8_t>(Q)[at(k)] = c; }
};

// Codes of the row at byte k of an LDS buffer, zero-filled to 64 * KU.
struct LdsDest {
    int8_t *q;
    int64_t KU;
    __device__ int64_t fill_end() const { return 64 * KU; }
    __device__ void put4(int64_t k, uint32_t codes) const { *reinterpret_cast<uint32_t *>(q + k) = codes; }
    __device__ void put1(int64_t k, int8_t c) const { q[k] = c; }
};

// Wave-wide reductions whose result every lane holds: DPP moves within each
// 16-lane row (swap neighbours, swap pairs, mirror within 8, mirror within
// 16 -- after each step all lanes of a group hold the same combination,
// since both operands of every combine meet in the same order up to
// commutation), then the four row results read as scalars and combined as
// (r0 op r1) op (r2 op r3).  Fixed order, so the same bits in every lane,
// every wave and every kernel that casts a row.
constexpr int kDppSwap1 = 0xB1;        // quad_perm(1, 0, 3, 2)
constexpr int kDppSwap2 = 0x4E;        // quad_perm(2, 3, 0, 1)
constexpr int kDppHalfMirror = 0x141;  // lane i <- lane 7 - i within 8
constexpr int kDppMirror = 0x140;      // lane i <- lane 15 - i within 16
template <int CTRL>
__device__ inline int dpp_i(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ inline double dpp_d(double v)
{
    const int2 b = __builtin_bit_cast(int2, v);
    return __builtin_bit_cast(double, make_int2(dpp_i<CTRL>(b.x), dpp_i<CTRL>(b.y)));
}
template <int CTRL>
__device__ inline float dpp_f(float v)
{
    return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, v)));
}
__device__ inline int wave_sum(int v)
{
    v += dpp_i<kDppSwap1>(v);
    v += dpp_i<kDppSwap2>(v);
    v += dpp_i<kDppHalfMirror>(v);
    v += dpp_i<kDppMirror>(v);
    return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
           (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}
__device__ inline float wave_max(float v)
{
    v = fmaxf(v, dpp_f<kDppSwap1>(v));
    v = fmaxf(v, dpp_f<kDppSwap2>(v));
    v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
    v = fmaxf(v, dpp_f<kDppMirror>(v));
    auto lane_f = [](float x, int l) { return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l)); };
    return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}
__device__ inline double wave_sum(double v)
{
    v += dpp_d<kDppSwap1>(v);
    v += dpp_d<kDppSwap2>(v);
    v += dpp_d<kDppHalfMirror>(v);
    v += dpp_d<kDppMirror>(v);
    auto lane_d = [](double x, int l) {
        const int2 b = __builtin_bit_cast(int2, x);
        return __builtin_bit_cast(double, make_int2(__builtin_amdgcn_readlane(b.x, l), __builtin_amdgcn_readlane(b.y, l)));
    };
    return (lane_d(v, 0) + lane_d(v, 16)) + (lane_d(v, 32) + lane_d(v, 48));
}

// absmax and code sum of a cast row (the same in every thread)
struct RowScale {
    float a;
    int32_t sum;
};

// MODE (what is cast; BitNet b1.58 2B4T video transcript, yousumm.com,
// "Transcription", names a sub-layer norm and a squared ReLU but gives no
// formulas -- the readings taken are these):
//   kPlain     x itself;
//   kRmsNorm   x_hat = (x * inv) * g with inv = (float)(1 / sqrt(sum x^2 /
//              K + eps)), the sum and the square root in fp64 (g = NULL:
//              all ones).  The fp64 sum runs per thread, then across lanes
//              (wave_sum), then across waves in a fixed order:
//              deterministic;
//   kRelu2Gate h = (r * r) * u with r = max(x, 0), x the gate projection's
//              output and u the up projection's (passed as g);
//   kAddRmsNorm the residual sum s = x + r (fp32, one rounding; r = res_)
//              is cast as kRmsNorm casts x, and written to xo_ unless xo_
//              is NULL.  Every element is read and written by one thread,
//              load before store, so xo_ may be x_ or res_ when a single
//              workgroup casts the row (an in-place residual update).
constexpr int kRegF4 = 32;
enum { kPlain = 0, kRmsNorm = 1, kRelu2Gate = 2, kAddRmsNorm = 3 };

// One token row per workgroup of WAVES waves.  Thread t owns the float4
// groups t, t + 64 * WAVES, ... of the row, so each 16-byte load of a wave
// reads 1 KiB of contiguous X and each 4-byte code store writes 256
// contiguous bytes.  Rows of up to 8192 values (one or four waves) or 12288
// (eight or sixteen) stay in registers between the passes, so X is read
// from memory once (longer rows are read again, mostly from L2).  The
// reductions are wave_sum / wave_max, joined through LDS when WAVES > 1.
template <int WAVES, int MODE, typename Dest>
__device__ RowScale quant_row(const float *x_, int K, const Dest &dst, const float *g_, float eps,
                              const float *res_ = nullptr, float *xo_ = nullptr)
{
    constexpr bool NORM = MODE == kRmsNorm || MODE == kAddRmsNorm;
    constexpr bool ADD = MODE == kAddRmsNorm;
    constexpr int kThr = 64 * WAVES;
    // float4 groups per thread kept in registers
    constexpr int kRegs = WAVES == 1 ? kRegF4 : WAVES == 4 ? kRegF4 / 4 : WAVES == 8 ? 6 : 3;
    __shared__ float red_a[WAVES];
    __shared__ int red_s[WAVES];
    __shared__ double red_d[WAVES];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const BL_GLOBAL float *x = gload_ptr<float>(x_);
    const BL_GLOBAL float *gw = gload_ptr<float>(g_);
    // float4 path: K a multiple of 4 and the rows (and gains) 16-byte aligned
    const bool vec = ((K & 3) == 0) && ((reinterpret_cast<uintptr_t>(x_) & 15) == 0) &&
                     (MODE == kPlain || !g_ || (reinterpret_cast<uintptr_t>(g_) & 15) == 0) &&
                     (!ADD || ((reinterpret_cast<uintptr_t>(res_) | reinterpret_cast<uintptr_t>(xo_)) & 15) == 0);
    const bool wxo = ADD && xo_ != nullptr;
    const BL_GLOBAL float *rs = gload_ptr<float>(res_);
    BL_GLOBAL float *xo = gstore_ptr<float>(xo_);
    const BL_GLOBAL v4f *r4 = reinterpret_cast<const BL_GLOBAL v4f *>(rs);
    BL_GLOBAL v4f *xo4 = reinterpret_cast<BL_GLOBAL v4f *>(xo);
    const int nf = K >> 2;
    const BL_GLOBAL v4f *x4 = reinterpret_cast<const BL_GLOBAL v4f *>(x);
    const BL_GLOBAL v4f *g4 = reinterpret_cast<const BL_GLOBAL v4f *>(gw);
    const bool in_regs = vec && nf <= kRegs * kThr;
    const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
    // the row value before the norm: x, or x + r in the residual mode
    auto ld4 = [&](int f) {
        v4f u = x4[f];
        if constexpr (ADD) u = u + r4[f];
        return u;
    };
    auto ld1 = [&](int i) {
        float u = x[i];
        if constexpr (ADD) u = u + rs[i];
        return u;
    };

    auto relu2 = [](float gv, float uv) {
        const float r = gv > 0.0f ? gv : 0.0f;
        return (r * r) * uv;
    };
    auto relu2_4 = [&](v4f gv, v4f uv) {
        v4f h;
        h.x = relu2(gv.x, uv.x);
        h.y = relu2(gv.y, uv.y);
        h.z = relu2(gv.z, uv.z);
        h.w = relu2(gv.w, uv.w);
        return h;
    };
    v4f v[kRegs];
    // with eight or more waves (few tokens: every memory round trip is on
    // the critical path) the norm's gains come with the row
    constexpr bool kGainRegs = NORM && WAVES >= 8;
    v4f gv[kGainRegs ? kRegs : 1];
    if (in_regs) {
#pragma unroll
        for (int j = 0; j < kRegs; ++j) {
            const int f = t + kThr * j;
            v[j] = f < nf ? __builtin_nontemporal_load(x4 + f) : zero4;
            if constexpr (kGainRegs) gv[j] = (g_ && f < nf) ? g4[f] : zero4;
            if constexpr (MODE == kRelu2Gate)
                if (f < nf) v[j] = relu2_4(v[j], __builtin_nontemporal_load(g4 + f));
            if constexpr (ADD)
                if (f < nf) {
                    v[j] = v[j] + __builtin_nontemporal_load(r4 + f);
                    if (wxo) xo4[f] = v[j];
                }
        }
    }

    float inv = 1.0f;
    if constexpr (NORM) {
        auto sq4 = [](v4f u) {
            double d = (double)u.x * (double)u.x;
            d += (double)u.y * (double)u.y;
            d += (double)u.z * (double)u.z;
            d += (double)u.w * (double)u.w;
            return d;
        };
        double s2 = 0.0;
        if (in_regs) {
#pragma unroll
            for (int j = 0; j < kRegs; ++j) s2 += sq4(v[j]);
        } else if (vec) {
            for (int f = t; f < nf; f += kThr) s2 += sq4(ld4(f));
        } else {
            for (int i = t; i < K; i += kThr) {
                const double u = (double)ld1(i);
                s2 += u * u;
            }
        }
        s2 = wave_sum(s2);
        if constexpr (WAVES > 1) {
            if (lane == 0) red_d[w] = s2;
            __syncthreads();
            s2 = red_d[0];
#pragma unroll
            for (int i = 1; i < WAVES; ++i) s2 += red_d[i];
        }
        inv = (float)(1.0 / sqrt(s2 / (double)K + (double)eps));
    }
    // the value cast, for float4 group f (given x's group) / element i
    auto norm4 = [&](v4f u, int f) {
        if constexpr (NORM) {
            u = u * inv;
            if (g_) u = u * g4[f];
        } else if constexpr (MODE == kRelu2Gate) {
            u = relu2_4(u, g4[f]);
        }
        return u;
    };
    // the value cast for element i, given its pre-norm value u
    auto norm1v = [&](float u, int i) {
        if constexpr (NORM) {
            u = u * inv;
            if (g_) u = u * gw[i];
        } else if constexpr (MODE == kRelu2Gate) {
            u = relu2(u, gw[i]);
        }
        return u;
    };
    auto norm1 = [&](int i) { return norm1v(ld1(i), i); };
    if constexpr (NORM) {
        if (in_regs) {
#pragma unroll
            for (int j = 0; j < kRegs; ++j) {
                const int f = t + kThr * j;
                if constexpr (kGainRegs) {
                    // (x * inv) * g: the same two roundings as norm4
                    if (f < nf) {
                        v[j] = v[j] * inv;
                        if (g_) v[j] = v[j] * gv[j];
                    }
                } else {
                    if (f < nf) v[j] = norm4(v[j], f);
                }
            }
        }
    }

    auto amax4 = [](v4f u) {
        return fmaxf(fmaxf(fabsf(u.x), fabsf(u.y)), fmaxf(fabsf(u.z), fabsf(u.w)));
    };
    float a = 0.0f;
    if (in_regs) {
#pragma unroll
        for (int j = 0; j < kRegs; ++j) a = fmaxf(a, amax4(v[j]));
    } else if (vec) {
        for (int f = t; f < nf; f += kThr) a = fmaxf(a, amax4(norm4(ld4(f), f)));
    } else {
        for (int i = t; i < K; i += kThr) a = fmaxf(a, fabsf(norm1(i)));
    }
    a = wave_max(a);
    if constexpr (WAVES > 1) {
        if (lane == 0) red_a[w] = a;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < WAVES; ++i) a = fmaxf(a, red_a[i]);
    }
    if (!(a >= 1e-5f)) a = 1e-5f;
    const float s = 127.0f / a;

    int sum = 0;
    // codes 4f .. 4f+3 are contiguous in every destination layout
    auto put4 = [&](int f, v4f v4) {
        const int8_t c0 = quant_code(v4.x, s), c1 = quant_code(v4.y, s);
        const int8_t c2 = quant_code(v4.z, s), c3 = quant_code(v4.w, s);
        sum += (int)c0 + (int)c1 + (int)c2 + (int)c3;
        dst.put4(4 * (int64_t)f, (uint32_t)(uint8_t)c0 | ((uint32_t)(uint8_t)c1 << 8) |
                                     ((uint32_t)(uint8_t)c2 << 16) | ((uint32_t)(uint8_t)c3 << 24));
    };
    if (in_regs) {
#pragma unroll
        for (int j = 0; j < kRegs; ++j) {
            const int f = t + kThr * j;
            if (f < nf) put4(f, v[j]);
        }
    } else if (vec) {
        for (int f = t; f < nf; f += kThr) {
            const v4f u = ld4(f);
            if (wxo) xo4[f] = u;
            put4(f, norm4(u, f));
        }
    } else {
        for (int i = t; i < K; i += kThr) {
            const float u = ld1(i);  // read once: xo may alias x or r
            if (wxo) xo[i] = u;
            const int8_t c = quant_code(norm1v(u, i), s);
            sum += c;
            dst.put1(i, c);
        }
    }
    for (int64_t i = K + t; i < dst.fill_end(); i += kThr) dst.put1(i, 0);
    sum = wave_sum(sum);
    if constexpr (WAVES > 1) {
        if (lane == 0) red_s[w] = sum;
        __syncthreads();
        sum = 0;
#pragma unroll
        for (int i = 0; i < WAVES; ++i) sum += red_s[i];
    }
    return RowScale{a, sum};
}

}  // namespace bl
