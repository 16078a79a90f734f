// Per-token absmax int8 activation quantization for gfx950.
//
// anthology note-168 on arXiv 2402.17764, "What it does": BitLinear's
// activations are 8-bit.  Reading implemented (the pages print no formula):
// a = max(1e-5, max_k |x_k|) for each token, s = 127 / a (one fp32 IEEE
// division per token), q_k = clamp(rint(x_k * s), -127, 127).  The row sum
// of q is produced too: the contraction kernels multiply by (code + 1)
// fields and subtract it once per output.
//
// One workgroup per token (one wave when there are many tokens, four for
// few): the row is read with 16-byte loads (kept in registers up to 8192
// values), |x| and the code sum are reduced with wave butterflies, and the
// codes are written four per 4-byte store.  Variants cast the RMSNorm of
// the row (the sub-layer norm before a BitLinear) or the gated squared-ReLU
// of two rows (the feed-forward hidden value before the down projection),
// computed in the same pass over the inputs.  The max is order-free and the row sum is an
// integer sum, so both are exact whatever the reduction order.
#include "common.hpp"

namespace bl {
namespace {

constexpr int kThreads = 256;
typedef float v4f __attribute__((ext_vector_type(4)));



// Where code k of the row goes: row-major (Q + m*ldq + k) or fragment order.
// In both layouts each aligned 16-code chunk is 16 contiguous bytes.
struct QDest {
    int8_t *Q;
    int64_t ldq;  // row-major stride; unused in fragment order
    int64_t m;
    int64_t KU;
    int tiled;
    __device__ int64_t at(int64_t k) const { return tiled ? qf32_offset(m, k, KU) : m * ldq + k; }
    __device__ int64_t fill_end() const { return tiled ? 64 * KU : ldq; }
};

// One token row per workgroup of WAVES waves.  Thread t owns the float4
// groups t, t + 64 * WAVES, ... of the row, so each 16-byte load of a wave
// reads 1 KiB of contiguous X and each 4-byte code store writes 256
// contiguous bytes of Q.  Rows of up to kRegF4 * 64 * 4 values stay in
// registers between the passes, so X is read from HBM once (longer rows are
// read again, mostly from L2).  The reductions are wave butterflies, joined
// through LDS when WAVES > 1.  Many tokens: one wave each (no barrier); few
// tokens (decode): four waves each, so the loads of one row are spread over
// more lanes.
//
// MODE (what is cast; BitNet b1.58 2B4T video transcript, yousumm.com,
// "Transcription", names a sub-layer norm and a squared ReLU but gives no
// formulas -- the readings taken are these):
//   kPlain     x itself;
//   kRmsNorm   x_hat = (x * inv) * g with inv = (float)(1 / sqrt(sum x^2 /
//              K + eps)), the sum and the square root in fp64 (aux = g,
//              NULL = all ones).  The fp64 sum runs per thread, then across
//              lanes, then across waves in a fixed order: deterministic;
//   kRelu2Gate h = (r * r) * u with r = max(x, 0), x the gate projection's
//              output and u the up projection's (aux = u);
//   kAddRmsNorm the residual sum s = x + r (fp32, one rounding; r = res_)
//              is written to xo_ and cast as kRmsNorm casts x.  Every element
//              is read and written by one thread, load before store, so xo_
//              may be x_ or res_ (an in-place residual update).
constexpr int kRegF4 = 32;
constexpr int kFewTokens = 2048;
constexpr int kSingleTokens = 16;  // fewer rows: sixteen waves per row
enum { kPlain = 0, kRmsNorm = 1, kRelu2Gate = 2, kAddRmsNorm = 3 };

template <int WAVES, int MODE>
__device__ void quant_row(const float *x_, int K, const QDest &dst, float *absmax_, int32_t *rowsum_,
                          const float *g_, float eps, const float *res_ = nullptr, float *xo_ = nullptr)
{
    constexpr bool NORM = MODE == kRmsNorm || MODE == kAddRmsNorm;
    constexpr bool ADD = MODE == kAddRmsNorm;
    constexpr int kThr = 64 * WAVES;
    // float4 groups per thread kept in registers: 32 with one wave, 8 with
    // four, 3 with sixteen (rows up to 8192, 8192 and 12288 values)
    constexpr int kRegs = WAVES == 1 ? kRegF4 : WAVES == 4 ? kRegF4 / 4 : 3;
    __shared__ float red_a[WAVES];
    __shared__ int red_s[WAVES];
    __shared__ double red_d[WAVES];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const BL_GLOBAL float *x = gload_ptr<float>(x_);
    const BL_GLOBAL float *gw = gload_ptr<float>(g_);
    BL_GLOBAL int8_t *q = gstore_ptr<int8_t>(dst.Q);
    // float4 path: K a multiple of 4 and the rows (and gains) 16-byte aligned
    const bool vec = ((K & 3) == 0) && ((reinterpret_cast<uintptr_t>(x_) & 15) == 0) &&
                     (MODE == kPlain || !g_ || (reinterpret_cast<uintptr_t>(g_) & 15) == 0) &&
                     (!ADD || ((reinterpret_cast<uintptr_t>(res_) | reinterpret_cast<uintptr_t>(xo_)) & 15) == 0);
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
    // sixteen waves serve single tokens (decode chains), where every memory
    // round trip is on the critical path: the norm's gains come with the row
    constexpr bool kGainRegs = NORM && WAVES == 16;
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
                    xo4[f] = v[j];
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
        for (int off = 32; off > 0; off >>= 1) s2 += __shfl_xor(s2, off, 64);
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
    for (int off = 32; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
    if constexpr (WAVES > 1) {
        if (lane == 0) red_a[w] = a;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < WAVES; ++i) a = fmaxf(a, red_a[i]);
    }
    if (!(a >= 1e-5f)) a = 1e-5f;
    const float s = 127.0f / a;

    int sum = 0;
    // codes 4f .. 4f+3 are contiguous in both Q layouts (16-code chunks are)
    auto put4 = [&](int f, v4f v4) {
        const int8_t c0 = quant_code(v4.x, s), c1 = quant_code(v4.y, s);
        const int8_t c2 = quant_code(v4.z, s), c3 = quant_code(v4.w, s);
        sum += (int)c0 + (int)c1 + (int)c2 + (int)c3;
        *reinterpret_cast<BL_GLOBAL uint32_t *>(q + dst.at(4 * (int64_t)f)) =
            (uint32_t)(uint8_t)c0 | ((uint32_t)(uint8_t)c1 << 8) | ((uint32_t)(uint8_t)c2 << 16) |
            ((uint32_t)(uint8_t)c3 << 24);
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
            if constexpr (ADD) xo4[f] = u;
            put4(f, norm4(u, f));
        }
    } else {
        for (int i = t; i < K; i += kThr) {
            const float u = ld1(i);  // read once: xo may alias x or r
            if constexpr (ADD) xo[i] = u;
            const int8_t c = quant_code(norm1v(u, i), s);
            sum += c;
            q[dst.at(i)] = c;
        }
    }
    for (int64_t i = K + t; i < dst.fill_end(); i += kThr) q[dst.at(i)] = 0;
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
    if constexpr (WAVES > 1) {
        if (lane == 0) red_s[w] = sum;
        __syncthreads();
        sum = 0;
#pragma unroll
        for (int i = 0; i < WAVES; ++i) sum += red_s[i];
    }
    if (t == 0) {
        *gstore_ptr<float>(absmax_) = a;
        if (rowsum_) *gstore_ptr<int32_t>(rowsum_) = sum;
    }
}

// One workgroup per token.
template <int WAVES, int MODE>
__global__ __launch_bounds__(64 * WAVES) void quant_act_kernel(const float *__restrict__ X, int K,
                                                               int8_t *__restrict__ Q, int64_t ldq,
                                                               int qtiled, float *__restrict__ absmax,
                                                               int32_t *__restrict__ rowsum,
                                                               uint32_t *__restrict__ zero_ptr,
                                                               int zero_n, const float *__restrict__ g,
                                                               float eps, const float *res = nullptr,
                                                               float *xo = nullptr)
{
    const int64_t m = blockIdx.x;
    if (m == 0 && zero_ptr)
        for (int i = threadIdx.x; i < zero_n; i += 64 * WAVES) zero_ptr[i] = 0u;
    const QDest dst{Q, ldq, m, (K + 63) / 64, qtiled};
    // the gate/up mode reads a second M x K array (g) row by row
    const float *aux = MODE == kRelu2Gate ? g + m * K : g;
    if constexpr (MODE == kAddRmsNorm)
        quant_row<WAVES, MODE>(X + m * K, K, dst, absmax + m, rowsum ? rowsum + m : nullptr, aux, eps,
                               res + m * K, xo + m * K);
    else
        quant_row<WAVES, MODE>(X + m * K, K, dst, absmax + m, rowsum ? rowsum + m : nullptr, aux, eps);
}

template <int WAVES>
__global__ __launch_bounds__(64 * WAVES) void quant_act_group_kernel(const Problem *__restrict__ probs,
                                                                     const uint32_t *__restrict__ tok_map)
{
    const int tok = blockIdx.x;
    const Problem &p = probs[tok_map[tok]];
    const int64_t m = tok - p.tok_begin;
    if (m == 0 && p.tickets)
        for (int64_t i = threadIdx.x; i < ticket_count(p); i += 64 * WAVES) p.tickets[i] = 0u;
    const QDest dst{p.Q, p.ldq, m, p.KU, p.qtiled};
    quant_row<WAVES, kPlain>(p.X + m * p.K, p.K, dst, p.absmax + m, p.rowsum + m, nullptr, 0.0f);
}

__global__ __launch_bounds__(kThreads) void zero_words_kernel(uint32_t *__restrict__ p, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) p[i] = 0u;
}

}  // namespace

hipError_t launch_quant_act(const float *X, int64_t M, int64_t K, int8_t *Q, int64_t ldq,
                            int qtiled, float *absmax, int32_t *rowsum, uint32_t *zero_ptr,
                            int zero_n, hipStream_t s)
{
    if (M < kSingleTokens)
        hipLaunchKernelGGL((quant_act_kernel<16, kPlain>), dim3((unsigned)M), dim3(1024), 0, s, X, (int)K, Q,
                           ldq, qtiled, absmax, rowsum, zero_ptr, zero_n, nullptr, 0.0f);
    else if (M < kFewTokens)
        hipLaunchKernelGGL((quant_act_kernel<4, kPlain>), dim3((unsigned)M), dim3(256), 0, s, X, (int)K, Q,
                           ldq, qtiled, absmax, rowsum, zero_ptr, zero_n, nullptr, 0.0f);
    else
        hipLaunchKernelGGL((quant_act_kernel<1, kPlain>), dim3((unsigned)M), dim3(64), 0, s, X, (int)K, Q,
                           ldq, qtiled, absmax, rowsum, zero_ptr, zero_n, nullptr, 0.0f);
    return hipGetLastError();
}

hipError_t launch_quant_act_rmsnorm(const float *X, int64_t M, int64_t K, const float *g, float eps,
                                    int8_t *Q, int64_t ldq, float *absmax, int32_t *rowsum,
                                    hipStream_t s)
{
    if (M < kSingleTokens)
        hipLaunchKernelGGL((quant_act_kernel<16, kRmsNorm>), dim3((unsigned)M), dim3(1024), 0, s, X, (int)K, Q,
                           ldq, 0, absmax, rowsum, nullptr, 0, g, eps);
    else if (M < kFewTokens)
        hipLaunchKernelGGL((quant_act_kernel<4, kRmsNorm>), dim3((unsigned)M), dim3(256), 0, s, X, (int)K, Q,
                           ldq, 0, absmax, rowsum, nullptr, 0, g, eps);
    else
        hipLaunchKernelGGL((quant_act_kernel<1, kRmsNorm>), dim3((unsigned)M), dim3(64), 0, s, X, (int)K, Q,
                           ldq, 0, absmax, rowsum, nullptr, 0, g, eps);
    return hipGetLastError();
}

hipError_t launch_quant_act_add_rmsnorm(const float *X, const float *R, int64_t M, int64_t K, const float *g,
                                        float eps, float *Xsum, int8_t *Q, int64_t ldq, float *absmax,
                                        int32_t *rowsum, hipStream_t s)
{
    if (M < kSingleTokens)
        hipLaunchKernelGGL((quant_act_kernel<16, kAddRmsNorm>), dim3((unsigned)M), dim3(1024), 0, s, X, (int)K,
                           Q, ldq, 0, absmax, rowsum, nullptr, 0, g, eps, R, Xsum);
    else if (M < kFewTokens)
        hipLaunchKernelGGL((quant_act_kernel<4, kAddRmsNorm>), dim3((unsigned)M), dim3(256), 0, s, X, (int)K,
                           Q, ldq, 0, absmax, rowsum, nullptr, 0, g, eps, R, Xsum);
    else
        hipLaunchKernelGGL((quant_act_kernel<1, kAddRmsNorm>), dim3((unsigned)M), dim3(64), 0, s, X, (int)K,
                           Q, ldq, 0, absmax, rowsum, nullptr, 0, g, eps, R, Xsum);
    return hipGetLastError();
}

hipError_t launch_quant_act_relu2_gate(const float *G, const float *U, int64_t M, int64_t N, int8_t *Q,
                                       int64_t ldq, float *absmax, int32_t *rowsum, hipStream_t s)
{
    if (M < kSingleTokens)
        hipLaunchKernelGGL((quant_act_kernel<16, kRelu2Gate>), dim3((unsigned)M), dim3(1024), 0, s, G, (int)N,
                           Q, ldq, 0, absmax, rowsum, nullptr, 0, U, 0.0f);
    else if (M < kFewTokens)
        hipLaunchKernelGGL((quant_act_kernel<4, kRelu2Gate>), dim3((unsigned)M), dim3(256), 0, s, G, (int)N,
                           Q, ldq, 0, absmax, rowsum, nullptr, 0, U, 0.0f);
    else
        hipLaunchKernelGGL((quant_act_kernel<1, kRelu2Gate>), dim3((unsigned)M), dim3(64), 0, s, G, (int)N,
                           Q, ldq, 0, absmax, rowsum, nullptr, 0, U, 0.0f);
    return hipGetLastError();
}

hipError_t launch_quant_act_group(const Problem *probs, const uint32_t *tok_map, int n_tokens,
                                  hipStream_t s)
{
    if (n_tokens < kFewTokens)
        hipLaunchKernelGGL(quant_act_group_kernel<4>, dim3((unsigned)n_tokens), dim3(256), 0, s, probs,
                           tok_map);
    else
        hipLaunchKernelGGL(quant_act_group_kernel<1>, dim3((unsigned)n_tokens), dim3(64), 0, s, probs,
                           tok_map);
    return hipGetLastError();
}

hipError_t launch_zero_words(uint32_t *p, int64_t n, hipStream_t s)
{
    int64_t blocks = (n + kThreads - 1) / kThreads;
    if (blocks < 1) blocks = 1;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, p, n);
    return hipGetLastError();
}

}  // namespace bl
