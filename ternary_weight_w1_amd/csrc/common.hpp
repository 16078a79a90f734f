// Shared definitions of the BitLinear HIP library (device and host side).
// Everything here is private to the library; the public contract is
// include/bitlinear.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

// Global-memory views of the problem's buffers.  Pointers read from a
// problem descriptor are generic; the explicit address space makes every
// access a global_load/global_store (flat accesses would also count against
// the LDS wait counter and serialize LDS waits behind in-flight loads).
#define BL_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ inline const BL_GLOBAL T *gload_ptr(const void *p)
{
    return (const BL_GLOBAL T *)p;
}
template <typename T>
__device__ inline BL_GLOBAL T *gstore_ptr(void *p)
{
    return (BL_GLOBAL T *)p;
}

// Wave-uniform copy of a value every lane holds (problem fields read from
// a plan table can arrive in vector registers); buffer resources and scalar
// offsets must live in scalar registers.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
template <typename T>
__device__ __forceinline__ T *uni(T *p)
{
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    return reinterpret_cast<T *>(((uint64_t)hi << 32) | lo);
}

// cache-policy operand of a buffer access that marks it non-temporal (nt)
constexpr int kNonTemporal = 2;

// Buffer resource over `bytes` bytes at p (both wave-uniform; 32-bit data
// format, unstrided).  A raw access whose lane offset reaches past `bytes`
// reads zeros (a store is dropped); bytes = 0 makes every access miss, and
// -1 admits every offset below 2^32.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *p, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, bytes, 0x00020000);
}

// int8 code of one activation: clamp(rint(x * s), -127, 127) with s = 127 / a
// computed once per token (anthology note-168 on arXiv 2402.17764, "What it
// does": 8-bit activations; per-token absmax scaling is the reading taken).
// The only definition in the library: the quantization kernel and the fused
// decode prologue both call it.
__device__ inline int8_t quant_code(float x, float s)
{
    float r = rintf(x * s);
    r = r > 127.0f ? 127.0f : r;
    r = r < -127.0f ? -127.0f : r;
    return (int8_t)(int)r;
}

// BL2-T64 geometry: 64-row tiles, 64-code units, 1 KiB blocks.
constexpr int kTileRows = 64;
constexpr int kUnitCodes = 64;
constexpr int kBlockBytes = 1024;
// token counts the streaming kernels take; larger ones take the tile kernel
constexpr int kStreamMaxTokens = 32;
// 64-row tiles per wave of the streaming MFMA kernel (a workgroup takes 4x)
// in launches with enough tile groups to fill the part; smaller launches
// take one per wave, twice as many workgroups
constexpr int kStreamMfmaTiles = 2;
// token counts above which that kernel reads fragment-ordered activations
constexpr int kStreamFragTokens = 16;
// launches of 1..16 tokens over few tiles take the wide kernels: kWideWaves
// waves per 64-row tile, each holding up to kWideUnits 64-code units in flight
constexpr int kWideWaves = 8;
constexpr int kWideUnits = 12;
// most tokens the packed-dot4 streaming kernels take (64 LDS bytes per token
// per unit of the workgroup's K range): one, and two in the token loop;
// from three tokens on the matrix-instruction stream is faster
constexpr int kDot4MaxTokens = 2;

// Everything the contraction kernels need to know about one BitLinear
// problem.  Single calls pass one of these by value; the grouped path keeps
// an array of them in device memory (the plan table).
struct Problem {
    const float *X;        // fp32 activations, M x K (quantization input)
    const uint8_t *P;      // packed weights (BL2-T64, or BT5-T32 when fmt == 1)
    const float *gamma;    // device scalar
    float *Y;              // M x N fp32 output
    int32_t *acc_out;      // optional M x N int32 accumulators
    int8_t *Q;             // int8 activations, M rows of ldq bytes
    float *absmax;         // [M]
    int32_t *rowsum;       // [M]
    int32_t *acc_ws;       // split-K partial sums, M x (NT*64), or null
    uint32_t *tickets;     // split-K arrival counters, [NT], or null
    int64_t ldq;           // row stride of Q in bytes (>= 64*KU, % 16 == 0)
    int32_t M, N, K;
    int32_t KU;            // ceil(K/64)
    int32_t NT;            // row tiles: ceil(N/64), or ceil(N/32) for BT5-T32
    int32_t ks;            // K splits of the streaming kernel (1 = none)
    int32_t upsplit;       // units per split (last split may be shorter)
    int32_t kind;          // 0 = streaming kernel (small M), 1 = tile kernel, 2 = BT5-T32 kernel
    int32_t mtile;         // rows of M per tile-kernel work item
    int32_t qtiled;        // 1: Q is stored in MFMA fragment order (see below)
    int32_t mt;            // M tiles of the tile kernel (token groups of the BT5 kernel)
    int32_t ntt;           // N tiles of the tile kernel; tile groups of the streaming MFMA
                           // kernel (4 * stiles tiles each); four-tile groups of the BT5 kernel
    int32_t tok_begin;     // first row of this problem in the grouped quant grid
    int32_t item_begin;    // first work item of this problem in its kernel's grid
    int32_t fmt;           // 0: BL2-T64 weights, 1: BT5-T32 weights
    int32_t KU5;           // ceil(K/160), the BT5-T32 units (0 for BL2-T64)
    int32_t stiles;        // 64-row tiles per wave of the streaming MFMA kernel (1 or 2; else 0)
    int32_t wide;          // 1: the wide kernels (kWideWaves waves per tile); else 0
};
static_assert(sizeof(Problem) == 160, "Problem layout is shared by host and device");

// Split-K arrival counters of a problem: one per N tile of the 2-bit
// streaming kernels, one per (four-tile group, token group) of the BT5
// kernel, one per (M tile, four N tiles) item of the tile kernel.
__host__ __device__ inline int64_t ticket_count(const Problem &p)
{
    return p.kind == 0 ? (int64_t)p.NT : (int64_t)p.ntt * p.mt;
}

// int32 words of a problem's split-K partial sums (ks > 1): one row of N
// tiles per split and token for the streaming kernels (64 or 32 rows per
// tile), mtile accumulators per thread of every (item, split) for the tile
// kernel.
__host__ __device__ inline int64_t partial_words(const Problem &p)
{
    if (p.kind == 1) return (int64_t)p.ks * p.mt * p.ntt * p.mtile * 256;
    return (int64_t)p.ks * p.M * p.NT * (p.kind == 2 ? 32 : 64);
}

// Up to kMultiMax problems that read the same int8 activations, passed by
// value to one launch (q|k|v, gate|up): workgroup b belongs to the last
// problem i with begin[i] <= b, as its local item b - begin[i].
constexpr int kMultiMax = 4;
struct ProblemSet {
    Problem p[kMultiMax];
    int32_t begin[kMultiMax + 1];
    int32_t count;
    int32_t pad_;
};
__device__ inline int multi_index(const ProblemSet &ps, int b)
{
    int i = 0;
#pragma unroll
    for (int j = 1; j < kMultiMax; ++j)
        if (j < ps.count && b >= ps.begin[j]) i = j;
    return i;
}

// Input of a one-token contraction launch whose workgroups cast the
// activations themselves (quant_row.hpp modes): every workgroup casts the
// whole row into LDS and keeps its absmax and code sum.
struct CastIn {
    const float *x;    // the row (the gate projection's output for the gated squared ReLU)
    const float *aux;  // RMSNorm gains (NULL: ones), or the up projection's output
    const float *res;  // the addend of the residual sum, or NULL
    float *xo;         // the residual sum, written by workgroup 0, or NULL
    float eps;
    int32_t K;
};

// Fragment order of the int8 activations ("QF32"), used by the streaming
// MFMA kernel above 16 tokens so that each wave reads an A operand with one
// contiguous 1 KiB load:
// for 32-row block b = m / 32, 64-code unit u and half h, a 1 KiB block at
// ((b * KU + u) * 2 + h) * 1024 holds, at byte 16 * l + c (lane l = 0..63,
// c = 0..15), Q[32 b + l % 32][64 u + 32 h + 16 (l / 32) + c].  Rows past M
// in the last block are never written and never stored from.
__host__ __device__ inline int64_t qf32_offset(int64_t m, int64_t k, int64_t KU)
{
    const int64_t b = m >> 5;
    const int64_t u = k >> 6, h = (k >> 5) & 1, g = (k >> 4) & 1;
    return ((b * KU + u) * 2 + h) * 1024 + 16 * ((m & 31) + 32 * g) + (k & 15);
}

// Plan table header (first bytes of the grouped-forward table).
struct GroupHeader {
    uint32_t magic;
    int32_t count;          // problems
    int32_t n_tokens;       // total rows over all problems (quant grid)
    int32_t n_items_stream; // work items of the streaming kernel
    int32_t n_items_tile;   // work items of the tile kernel
    int32_t n_zero;         // problems whose split-K scratch must be zeroed
    int32_t dot4_items;     // unused by the kernels (diagnostics)
    int32_t stream_variant; // streaming kernel instantiation (see api.hip)
    int32_t reserved_;      // unused
    int32_t stream_lds;     // dynamic LDS bytes of the streaming kernel
    int32_t n_items_bt5;    // work items of the BT5-T32 kernel
    int32_t bt5_max_m;      // largest token count among the BT5-T32 problems
    int64_t ws_bytes;       // workspace the plan was built for
    int64_t off_probs;      // byte offsets inside the table
    int64_t off_tok_map;    // uint32 per token: problem index
    int64_t off_stream_map; // uint2 per workgroup: {problem, local item} ({~0u, 0} = idle)
    int64_t off_tile_map;   // uint2 per workgroup: {problem, local item}
    int64_t off_bt5_map;    // uint2 per workgroup: {problem, local item}
    int64_t total_bytes;
};
constexpr uint32_t kGroupMagic = 0xB17E0002u;

// Kernel launchers (each defined next to its kernels).
hipError_t launch_absmean_partial(const float *W, int64_t count, double *partial, int nblocks,
                                  hipStream_t s);
hipError_t launch_absmean_final(const double *partial, int nblocks, int64_t count,
                                const float *gamma_in, float *gamma_out, hipStream_t s);
hipError_t launch_ternarize(const float *W, int64_t count, const float *gamma, int8_t *T,
                            hipStream_t s);
hipError_t launch_pack(const int8_t *T, int64_t N, int64_t K, uint8_t *P, hipStream_t s);
hipError_t launch_unpack(const uint8_t *P, int64_t N, int64_t K, int8_t *T, hipStream_t s);
hipError_t launch_pack5(const int8_t *T, int64_t N, int64_t K, uint8_t *P, hipStream_t s);
hipError_t launch_unpack5(const uint8_t *P, int64_t N, int64_t K, int8_t *T, hipStream_t s);
hipError_t launch_quant_act(const float *X, int64_t M, int64_t K, int8_t *Q, int64_t ldq,
                            int qtiled, float *absmax, int32_t *rowsum, uint32_t *zero_ptr,
                            int zero_n, hipStream_t s);
hipError_t launch_quant_act_rmsnorm(const float *X, int64_t M, int64_t K, const float *g, float eps,
                                    int8_t *Q, int64_t ldq, float *absmax, int32_t *rowsum,
                                    hipStream_t s);
hipError_t launch_quant_act_add_rmsnorm(const float *X, const float *R, int64_t M, int64_t K, const float *g,
                                        float eps, float *Xsum, int8_t *Q, int64_t ldq, float *absmax,
                                        int32_t *rowsum, hipStream_t s);
hipError_t launch_quant_act_relu2_gate(const float *G, const float *U, int64_t M, int64_t N, int8_t *Q,
                                       int64_t ldq, float *absmax, int32_t *rowsum, hipStream_t s);
hipError_t launch_quant_act_group(const Problem *probs, const uint32_t *tok_map, int n_tokens,
                                  hipStream_t s);
hipError_t launch_zero_words(uint32_t *p, int64_t n, hipStream_t s);
hipError_t launch_stream_single(const Problem &p, int variant, hipStream_t s);
hipError_t launch_stream_group(const Problem *probs, const uint2 *item_map, int n_items,
                               int variant, int lds_bytes, hipStream_t s);
hipError_t launch_tile_single(const Problem &p, hipStream_t s);
hipError_t launch_tile_group(const Problem *probs, const uint2 *item_map, int n_items, hipStream_t s);
hipError_t launch_bt5_single(const Problem &p, hipStream_t s);
hipError_t launch_stream_multi(const ProblemSet &ps, int variant, int lds_bytes, hipStream_t s);
hipError_t launch_stream_cast_multi(const ProblemSet &ps, const CastIn &ci, int mode, hipStream_t s);
hipError_t launch_tile_multi(const ProblemSet &ps, hipStream_t s);
hipError_t launch_bt5_multi(const ProblemSet &ps, int max_tokens, hipStream_t s);
hipError_t launch_bt5_group(const Problem *probs, const uint2 *item_map, int n_items, int max_tokens,
                            hipStream_t s);

}  // namespace bl
