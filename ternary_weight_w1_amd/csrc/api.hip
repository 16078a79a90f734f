// Host side of the C ABI declared in include/bitlinear.h: argument
// validation, workspace layout, kernel selection and launches.  No call
// allocates, frees, copies or synchronizes; validation happens before the
// first launch, so a rejected call enqueues nothing.
#include <bitlinear.h>
#include <bitlinear_probe.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "bt5.hpp"
#include "common.hpp"
#include "probe.hpp"

using bl::Problem;

namespace {

thread_local std::string g_last_error;

int fail(int status, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int hip_fail(hipError_t e, const char *what)
{
    return fail(BITLINEAR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kMaxMN = int64_t(1) << 24;
constexpr int64_t kMaxK = 131072;
constexpr int kStreamMaxM = bl::kStreamMaxTokens;
constexpr int kGroupTiles = 4 * bl::kStreamMfmaTiles;  // tiles per streaming MFMA workgroup

bool a16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
bool a4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3) == 0; }
int64_t up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

int check_nk(int64_t N, int64_t K)
{
    if (N < 1 || N > kMaxMN) return fail(BITLINEAR_ERR_SHAPE, "N=%lld out of range [1, 2^24]", (long long)N);
    if (K < 1 || K > kMaxK) return fail(BITLINEAR_ERR_SHAPE, "K=%lld out of range [1, 131072]", (long long)K);
    return BITLINEAR_OK;
}

int check_mnk(int64_t M, int64_t N, int64_t K)
{
    if (M < 1 || M > kMaxMN) return fail(BITLINEAR_ERR_SHAPE, "M=%lld out of range [1, 2^24]", (long long)M);
    return check_nk(N, K);
}

// Measurement knobs, read once from the environment (immutable afterwards).
struct Knobs {
    int lut = 0;                 // one-token problems take the table-lookup comparison kernel
    int split_target = 1024;     // aim for at least this many workgroups
    int xcd_order = 3;           // bit 0: streaming kernel, bit 1: tile kernel
    int mfma_tiles = 0;          // tiles per wave of the streaming MFMA kernel above 16 tokens: 0 = by launch size, 1, 2
    int wide = 1;                // launches of 1..16 tokens over few tiles take the wide kernels
    int cast_fuse = 1;           // one-token cast + contraction calls cast inside the contraction:
                                 // 0 never, 1 where it pays (the default rule), 2 wherever it can
};
const Knobs &knobs()
{
    static const Knobs k = [] {
        Knobs v;
        if (const char *s = getenv("BITLINEAR_SPLIT_TARGET")) v.split_target = atoi(s) > 0 ? atoi(s) : 1;
        if (const char *s = getenv("BITLINEAR_DOT4_VARIANT")) v.lut = atoi(s) == 5;
        if (const char *s = getenv("BITLINEAR_XCD_ORDER")) v.xcd_order = atoi(s) & 3;
        if (const char *s = getenv("BITLINEAR_MFMA_TILES")) v.mfma_tiles = (atoi(s) == 1 || atoi(s) == 2) ? atoi(s) : 0;
        if (const char *s = getenv("BITLINEAR_WIDE")) v.wide = atoi(s) != 0;
        if (const char *s = getenv("BITLINEAR_CAST_FUSE")) v.cast_fuse = (atoi(s) >= 0 && atoi(s) <= 2) ? atoi(s) : 1;
        return v;
    }();
    return k;
}

// Token rows per tile-kernel work item (64-token tiles, two units per stage:
// against a 128-token tile it is as fast at M = 256 and 512 and pads less
// elsewhere -- M = 64: 0.27 vs 0.40 ms; 176: 0.40 vs 0.49 ms on 3B/2B stacks)
// and weight rows per item (four 64-row tiles, one per wave).
constexpr int kTileTokens = 64;
constexpr int kTileRowTiles = 4;

// The dot4 kernels hold 64 bytes of activations per token slot per unit of
// the workgroup's K range (decompose caps the range to fit 64 KiB).
constexpr int kStreamLdsMax = 64 * 1024;
// The table-lookup dot4 variant (knob value 5) runs single-token problems
// with at most kLutMaxUnits units (64 KiB of table) per workgroup.
constexpr int kLutMaxUnits = 64;
bool lut_variant(int64_t M) { return knobs().lut && M == 1; }
// The dot4 kernel for two tokens stages 64 bytes per token slot per unit:
// at most kDot4TokMaxUnits units (64 KiB) per workgroup.
constexpr int kDot4TokMaxUnits = 64 * 1024 / (64 * bl::kDot4MaxTokens);
bool dot4_tokens(int64_t M) { return M >= 2 && M <= bl::kDot4MaxTokens; }
// Token counts the 32x32x32 MFMA stream takes (its work items are groups of
// 4 * tiles-per-wave row tiles; the dot4 kernels work per tile).
bool mfma32_stream(int64_t M) { return M <= kStreamMaxM && M > bl::kDot4MaxTokens; }
// Up to 16 tokens the MFMA stream stages the workgroup's activations in LDS
// (row-major, 80 bytes per token per unit of the K range) and takes one
// tile per wave (variant 10); beyond, it reads fragment-ordered activations
// from memory.  Staging cut the 2B sweeps 8-10% (M = 8: 128.5 -> 117.6 us;
// M = 16: 145.4 -> 131.6 us) and the 3B sweep at M = 8 12% (186.9 -> 164.5).
// A K range longer than the staging holds is split; problems that would
// need more than three such splits (the 70B class at 16 tokens: 448 units)
// keep the launch on the global-load stream, whose larger tiles per wave
// win there (70B M = 16: 3.69 ms, against 3.97 ms staged).
constexpr int kAldsMaxTokens = 16;
constexpr int64_t kAldsMaxSplits = 3;
int64_t alds_max_units(int64_t M) { return kStreamLdsMax / (80 * M); }
bool alds_for(int64_t maxM) { return maxM > bl::kDot4MaxTokens && maxM <= kAldsMaxTokens; }
bool alds_fits(int64_t M, int64_t K)
{
    const int64_t ku = (K + 63) / 64, cap = alds_max_units(M);
    return (ku + cap - 1) / cap <= kAldsMaxSplits;
}
// Its instantiation for a launch whose workgroups stage `lds` bytes: held to
// 128 VGPRs (11, four waves per SIMD) where four such workgroups fit in a
// compute unit's 160 KiB of LDS, else 10 (136 VGPRs, three per SIMD).
constexpr int64_t kAlds4Lds = 160 * 1024 / 4 - 512;
int alds_variant(int64_t lds) { return lds <= kAlds4Lds ? 11 : 10; }
// Tiles per wave of that stream for a launch with `groups` kGroupTiles-tile
// groups: two when the groups alone fill the part (the split target), else
// one, which doubles the workgroups without more split-K reductions.
int mfma_tiles_for(int64_t groups)
{
    if (knobs().mfma_tiles) return knobs().mfma_tiles;
    return groups < knobs().split_target ? 1 : bl::kStreamMfmaTiles;
}

// Launches of 1..16 tokens of at most two workgroups per compute unit take
// the wide kernels: a workgroup's kWideWaves waves share one 64-row tile and
// K range, so the launch is one memory round trip per workgroup and, where
// one split covers K, needs no hand-off through memory.  Eight waves beat
// sixteen on every decode-layer shape measured (one token: q|k|v 3.95 vs
// 4.21 us, o 3.79 vs 4.02, gate|up 5.66 vs 5.78; eight tokens: q|k|v 4.92
// vs 5.41, o 4.74 vs 5.16).
constexpr int64_t kWideSlots = 512;
// With 2..16 tokens (the MFMA stream) a split also holds at most what fits
// 64 KiB of LDS with the kernel's own 512 bytes: staged activations (80
// bytes per token per unit); the waves' sums (8 * M * 256 bytes) reuse
// that space.
constexpr int64_t kWideMaxTokens = 16;
int64_t wide_units(int64_t M)
{
    const int64_t u = (int64_t)bl::kWideWaves * bl::kWideUnits;
    return M == 1 ? u : std::min<int64_t>(u, (65536 - 512) / (80 * M));
}
// A K range longer than a workgroup holds is split into parts of about
// kWideSplitUnits units: a split costs a hand-off through memory (about
// 2 us), so it pays only where it takes the per-workgroup stream well below
// that (3200 x 8640 at one token: 7.5 us unsplit with 16 waves, 6.5 in three
// parts, 5.8 in five; at eight tokens 8.1 in two parts, 7.4 in three).
constexpr int64_t kWideSplitUnits = 28;
int64_t wide_splits(int64_t M, int64_t KU)
{
    return KU <= wide_units(M) ? 1 : (KU + kWideSplitUnits - 1) / kWideSplitUnits;
}
bool wide_for(int64_t M, int64_t tiles, int64_t KU)
{
    if (M < 1 || M > kWideMaxTokens || !knobs().wide || (M == 1 && knobs().lut)) return false;
    return tiles * wide_splits(M, KU) <= kWideSlots;
}
// Decomposition of a problem for the wide kernels.
void decompose_wide(Problem &p)
{
    p.kind = 0;
    p.KU = (int32_t)((p.K + 63) / 64);
    p.NT = (int32_t)((p.N + 63) / 64);
    p.mt = p.ntt = p.mtile = p.qtiled = p.stiles = 0;
    p.wide = 1;
    p.ks = (int32_t)wide_splits(p.M, p.KU);
    p.upsplit = (p.KU + p.ks - 1) / p.ks;
    p.ks = (p.KU + p.upsplit - 1) / p.upsplit;
}
int wide_variant(int64_t M) { return M == 1 ? 12 : 13; }

// Most K splits of a tile-kernel problem (measured on the chained 3B step at
// M = 64 with one split count for every launch: 3.16 ms unsplit, 2.70 at
// two, 2.74 at four, 3.06 at eight, 3.33 at up to sixteen).  Two, except in
// launches of at most kTileFewItems items (a layer's o or down at 64 tokens:
// 13 items), which take up to four of at least 16 units (chained 3B step at
// M = 64: 2.353 -> 2.280 ms; four splits for launches of up to ~50 items
// made M = 256 3% slower).
constexpr int64_t kTileMaxSplits = 4;
constexpr int64_t kTileFewItems = 32;

// Kernel kind and decomposition of one problem.  `base_items` is the number
// of streaming work items the whole launch has without K splits; splits are
// added only while the launch is short of workgroups.  own_q: the library
// quantizes the activations itself and may choose their layout.  groups4:
// the launch runs the streaming MFMA kernel, whose work items are groups of
// 4 * tpw 64-row tiles (p.ntt of them).
void decompose(Problem &p, int64_t base_items, bool own_q, bool groups4 = false, int tpw = bl::kStreamMfmaTiles,
               int64_t tile_base = 0, bool alds = false)
{
    p.KU = (int32_t)((p.K + 63) / 64);
    p.NT = (int32_t)((p.N + 63) / 64);
    p.ks = 1;
    p.upsplit = p.KU;
    p.mt = p.ntt = p.mtile = p.qtiled = p.stiles = p.wide = 0;
    if (p.M <= kStreamMaxM) {
        p.kind = 0;
        if (groups4) {
            p.stiles = tpw;
            p.ntt = (p.NT + 4 * tpw - 1) / (4 * tpw);
            // past 16 tokens the MFMA kernel reads each A operand as one
            // 1 KiB block when the library lays the activations out itself
            p.qtiled = own_q && p.M > bl::kStreamFragTokens ? 1 : 0;
        }
        const int64_t target = knobs().split_target;
        if (base_items < target) {
            int64_t ks = (target + base_items - 1) / base_items;
            int64_t cap = p.KU / 8;  // keep >= 8 units (2 per wave) per split
            if (cap < 1) cap = 1;
            if (ks > cap) ks = cap;
            const int64_t upsplit = (p.KU + ks - 1) / ks;
            p.upsplit = (int32_t)upsplit;
            p.ks = (int32_t)((p.KU + upsplit - 1) / upsplit);
        }
        // the table-lookup variant holds 1 KiB of table per unit in LDS, the
        // 2..4-token dot4 kernel 256 bytes of activations
        if (lut_variant(p.M) && p.upsplit > kLutMaxUnits) {
            p.upsplit = kLutMaxUnits;
            p.ks = (p.KU + kLutMaxUnits - 1) / kLutMaxUnits;
        }
        if (dot4_tokens(p.M) && p.upsplit > kDot4TokMaxUnits) {
            p.upsplit = kDot4TokMaxUnits;
            p.ks = (p.KU + kDot4TokMaxUnits - 1) / kDot4TokMaxUnits;
        }
        // the MFMA stream with staged activations: 80 bytes per token per unit
        if (groups4 && alds && p.upsplit > alds_max_units(p.M)) {
            const int64_t cap = alds_max_units(p.M);
            const int32_t ks = (int32_t)((p.KU + cap - 1) / cap);
            p.upsplit = (p.KU + ks - 1) / ks;
            p.ks = (p.KU + p.upsplit - 1) / p.upsplit;
        }
        // the one-token kernel stages 64 bytes per unit: longer ranges are
        // split into equal parts that fit 64 KiB
        if (p.M == 1 && !groups4 && p.upsplit > kStreamLdsMax / 64) {
            const int32_t ks = (p.KU + kStreamLdsMax / 64 - 1) / (kStreamLdsMax / 64);
            p.upsplit = (p.KU + ks - 1) / ks;
            p.ks = (p.KU + p.upsplit - 1) / p.upsplit;
        }
    } else {
        p.kind = 1;
        p.mtile = kTileTokens;
        p.mt = (int32_t)((p.M + p.mtile - 1) / p.mtile);
        p.ntt = (p.NT + kTileRowTiles - 1) / kTileRowTiles;
        // K splits while the launch's work items (tile_base, or this
        // problem's alone) are short of the target (see kTileMaxSplits).
        // Each split's partials are 64 KiB per item, read back by the
        // item's last split, so more splits cost more than they gain.
        const int64_t items = tile_base > 0 ? tile_base : (int64_t)p.mt * p.ntt;
        const int64_t target = knobs().split_target;
        if (items < target) {
            int64_t ks = (target + items - 1) / items;
            // launches of very few items (a single layer's o or down at 64
            // tokens) split up to four ways, at least 16 units each; others
            // in two, at least 8 units each
            const bool few = items <= kTileFewItems;
            int64_t cap = few ? p.KU / 16 : p.KU / 8;
            const int64_t max_splits = few ? kTileMaxSplits : 2;
            if (cap > max_splits) cap = max_splits;
            if (cap < 1) cap = 1;
            if (ks > cap) ks = cap;
            const int64_t upsplit = (p.KU + ks - 1) / ks;
            p.upsplit = (int32_t)upsplit;
            p.ks = (int32_t)((p.KU + upsplit - 1) / upsplit);
        }
    }
}

// BT5-T32 weights always take the BT5 kernel, for any M: its work items are
// (four 32-row tiles, 16 tokens, K split).  Splits are added while the
// launch is short of workgroups, keeping at least four 160-code units each.
int64_t bt5_items(int64_t M, int64_t N)
{
    const int64_t nt = (N + bl::kBt5TileRows - 1) / bl::kBt5TileRows;
    return (nt + 3) / 4 * ((M + bl::kBt5Tokens - 1) / bl::kBt5Tokens);
}
void decompose5(Problem &p, int64_t base_items)
{
    p.fmt = 1;
    p.kind = 2;
    p.KU = (int32_t)((p.K + 63) / 64);
    p.KU5 = (int32_t)((p.K + bl::kBt5UnitCodes - 1) / bl::kBt5UnitCodes);
    p.NT = (int32_t)((p.N + bl::kBt5TileRows - 1) / bl::kBt5TileRows);
    p.ntt = (p.NT + 3) / 4;
    p.mt = (int32_t)((p.M + bl::kBt5Tokens - 1) / bl::kBt5Tokens);
    p.mtile = p.qtiled = 0;
    p.ks = 1;
    p.upsplit = p.KU5;
    const int64_t target = knobs().split_target;
    if (base_items < target) {
        int64_t ks = (target + base_items - 1) / base_items;
        int64_t cap = p.KU5 / 4;
        if (cap < 1) cap = 1;
        if (ks > cap) ks = cap;
        const int64_t upsplit = (p.KU5 + ks - 1) / ks;
        p.upsplit = (int32_t)upsplit;
        p.ks = (int32_t)((p.KU5 + upsplit - 1) / upsplit);
    }
}

int64_t items_of(const Problem &p)
{
    if (p.kind == 0) return (int64_t)(p.ntt > 0 ? p.ntt : p.NT) * p.ks;
    return (int64_t)p.ntt * p.mt * p.ks;
}

// Row stride of the library's own int8 activations: whole 64-code units,
// or whole 160-code units for BT5-T32 weights (the quantizer zero-fills the
// row up to the stride, so every unit the kernels read is complete).
int64_t own_ldq(const Problem &p) { return p.fmt ? 160 * (int64_t)p.KU5 : 64 * (int64_t)p.KU; }

// Decomposition of a problem launched alone: the streaming MFMA kernel (more
// tokens than the dot4 kernel takes) works on tile groups.
void decompose_single(Problem &p, bool own_q)
{
    const int64_t nt = (p.N + 63) / 64;
    if (wide_for(p.M, nt, (p.K + 63) / 64)) {
        decompose_wide(p);
        return;
    }
    const bool g4 = mfma32_stream(p.M);
    const bool alds = g4 && alds_for(p.M) && alds_fits(p.M, p.K);
    const int tpw = alds ? 1 : g4 ? mfma_tiles_for((nt + kGroupTiles - 1) / kGroupTiles) : bl::kStreamMfmaTiles;
    decompose(p, g4 ? (nt + 4 * tpw - 1) / (4 * tpw) : nt, own_q, g4, tpw, 0, alds);
}

int stream_variant_for(int64_t M, int64_t upsplit)
{
    if (M > bl::kDot4MaxTokens) return 1;
    if (M >= 2) return 6;  // decompose keeps upsplit <= kDot4TokMaxUnits
    if (knobs().lut && upsplit <= kLutMaxUnits) return 5;
    return 3;
}


// Dynamic LDS a problem of M tokens whose workgroups take upsplit units
// needs under a streaming-kernel variant: activations, 64 bytes per token
// slot per unit (one slot for 3; two for 6 except one-token problems), or
// the lookup table (1 KiB per unit, 5); none for the MFMA stream (1, 9).
int64_t stream_lds_need(int variant, int64_t M, int64_t upsplit)
{
    if (variant == 1 || variant == 9) return 0;
    if (variant == 10 || variant == 11) return 80 * M * upsplit;
    if (variant == 13) return std::max<int64_t>(80 * M * upsplit, 8 * M * 256);
    if (variant == 5) return 1024 * upsplit;
    const int64_t slots = (variant == 6 && M > 1) ? bl::kDot4MaxTokens : 1;
    return 64 * slots * upsplit;
}

// Workspace layout of one problem: [Q][absmax][rowsum][partials][tickets],
// each region 256-byte aligned.  with_act = false leaves out the first three.
struct WsLayout {
    int64_t q = 0, absmax = 0, rowsum = 0, part = 0, tick = 0, total = 0;
};
WsLayout ws_layout(const Problem &p, bool with_act)
{
    WsLayout L;
    int64_t off = 0;
    const int64_t ldq = own_ldq(p);
    if (with_act) {
        L.q = off;
        off = up(off + (p.qtiled ? up(p.M, 32) : (int64_t)p.M) * ldq, 256);
        L.absmax = off;
        off = up(off + 4 * (int64_t)p.M, 256);
        L.rowsum = off;
        off = up(off + 4 * (int64_t)p.M, 256);
    }
    if (p.ks > 1) {
        L.part = off;
        off = up(off + 4 * bl::partial_words(p), 256);
        L.tick = off;
        off = up(off + 4 * bl::ticket_count(p), 256);
    }
    L.total = off;
    return L;
}

int quant_weight_blocks(int64_t count)
{
    int64_t b = (count + 65535) / 65536;
    if (b < 1) b = 1;
    if (b > 1024) b = 1024;
    return (int)b;
}

Problem make_problem(int64_t M, int64_t N, int64_t K)
{
    Problem p;
    memset(&p, 0, sizeof p);
    p.M = (int32_t)M;
    p.N = (int32_t)N;
    p.K = (int32_t)K;
    return p;
}

hipError_t launch_contraction(const Problem &p, bool own_q, hipStream_t s)
{
    if (p.kind == 2) return bl::launch_bt5_single(p, s);
    if (p.kind == 0) {
        if (p.wide) return bl::launch_stream_single(p, wide_variant(p.M), s);
        const int v = stream_variant_for(p.M, p.upsplit);
        const int sv = v != 1                                     ? v
                       : (alds_for(p.M) && alds_fits(p.M, p.K)) ? alds_variant(80 * p.M * p.upsplit)
                       : p.stiles == 1                          ? 9
                                                                : 1;
        return bl::launch_stream_single(p, sv, s);
    }
    (void)own_q;
    return bl::launch_tile_single(p, s);
}

// Validation shared by the forward calls (nothing is enqueued on failure).
int forward_check(const char *who, const float *X, int64_t M, int64_t K, const uint8_t *P, const float *gamma,
                  int64_t N, float *Y_out, int32_t *acc_out)
{
    if (!X || !P || !gamma || !Y_out) return fail(BITLINEAR_ERR_NULL, "%s: X, P, gamma and Y_out are required", who);
    if (int st = check_mnk(M, N, K)) return st;
    if (!a16(X) || !a16(P) || !a16(Y_out) || (acc_out && !a16(acc_out)) || !a4(gamma))
        return fail(BITLINEAR_ERR_ALIGN, "%s: arrays need 16-byte, gamma 4-byte alignment", who);
    return BITLINEAR_OK;
}

// bitlinear_forward on the workspace ws (the caller's, or the library's
// scratch for bitlinear_forward_noalloc).
int forward_impl(const char *who, const float *X, int64_t M, int64_t K, const uint8_t *P, const float *gamma,
                 int64_t N, float *Y_out, int32_t *acc_out, void *ws, size_t ws_bytes, void *stream)
{
    if (int st = forward_check(who, X, M, K, P, gamma, N, Y_out, acc_out)) return st;
    Problem p = make_problem(M, N, K);
    decompose_single(p, true);
    const WsLayout L = ws_layout(p, true);
    if (!ws || ws_bytes < (size_t)L.total || !a16(ws))
        return fail(BITLINEAR_ERR_WORKSPACE, "%s: needs %lld workspace bytes (16-byte aligned)", who, (long long)L.total);
    if (p.kind == 1 && items_of(p) >= (int64_t(1) << 31))
        return fail(BITLINEAR_ERR_SHAPE, "%s: grid too large", who);
    char *base = static_cast<char *>(ws);
    p.X = X;
    p.P = P;
    p.gamma = gamma;
    p.Y = Y_out;
    p.acc_out = acc_out;
    p.ldq = 64 * (int64_t)p.KU;
    p.Q = reinterpret_cast<int8_t *>(base + L.q);
    p.absmax = reinterpret_cast<float *>(base + L.absmax);
    p.rowsum = reinterpret_cast<int32_t *>(base + L.rowsum);
    if (p.ks > 1) {
        p.acc_ws = reinterpret_cast<int32_t *>(base + L.part);
        p.tickets = reinterpret_cast<uint32_t *>(base + L.tick);
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (hipError_t e = bl::launch_quant_act(X, M, K, p.Q, p.ldq, p.qtiled, p.absmax, p.rowsum,
                                            p.tickets, p.tickets ? (int)bl::ticket_count(p) : 0, s))
        return hip_fail(e, who);
    if (hipError_t e = launch_contraction(p, true, s)) return hip_fail(e, who);
    return BITLINEAR_OK;
}

}  // namespace

extern "C" {

int bitlinear_abi_version(void) { return BITLINEAR_ABI_VERSION; }

const char *bitlinear_strerror(int status)
{
    switch (status) {
    case BITLINEAR_OK: return "ok";
    case BITLINEAR_ERR_NULL: return "a required pointer is NULL";
    case BITLINEAR_ERR_SHAPE: return "a size is out of range or inconsistent";
    case BITLINEAR_ERR_ALIGN: return "a buffer or stride is not aligned";
    case BITLINEAR_ERR_WORKSPACE: return "workspace missing or too small";
    case BITLINEAR_ERR_HIP: return "HIP runtime error";
    case BITLINEAR_ERR_ARG: return "invalid argument";
    default: return "unknown status";
    }
}

const char *bitlinear_last_error(void) { return g_last_error.c_str(); }

size_t bitlinear_packed_bytes(int64_t N, int64_t K)
{
    if (N < 1 || N > kMaxMN || K < 1 || K > kMaxK) return 0;
    return (size_t)((N + 63) / 64) * (size_t)((K + 63) / 64) * 1024u;
}

int64_t bitlinear_q_stride(int64_t K) { return (K < 1 || K > kMaxK) ? 0 : up(K, 64); }

size_t bitlinear_packed5_bytes(int64_t N, int64_t K)
{
    if (N < 1 || N > kMaxMN || K < 1 || K > kMaxK) return 0;
    return (size_t)((N + bl::kBt5TileRows - 1) / bl::kBt5TileRows) *
           (size_t)((K + bl::kBt5UnitCodes - 1) / bl::kBt5UnitCodes) * 1024u;
}

int64_t bitlinear_q_stride5(int64_t K) { return (K < 1 || K > kMaxK) ? 0 : up(K, bl::kBt5UnitCodes); }

size_t bitlinear_workspace_bytes(int op, int64_t M, int64_t N, int64_t K)
{
    if (op == BITLINEAR_WS_QUANTIZE_WEIGHTS) {
        if (check_nk(N, K) != BITLINEAR_OK) return SIZE_MAX;
        return (size_t)quant_weight_blocks(N * K) * sizeof(double);
    }
    if (op < BITLINEAR_WS_MATMUL || op > BITLINEAR_WS_FORWARD5) return SIZE_MAX;
    if (check_mnk(M, N, K) != BITLINEAR_OK) return SIZE_MAX;
    Problem p = make_problem(M, N, K);
    const bool with_act = op == BITLINEAR_WS_FORWARD || op == BITLINEAR_WS_FORWARD5;
    if (op >= BITLINEAR_WS_MATMUL5)
        decompose5(p, bt5_items(M, N));
    else
        decompose_single(p, with_act);
    return (size_t)ws_layout(p, with_act).total;
}

int bitlinear_quantize_weights(const float *W, int64_t N, int64_t K, const float *gamma_in,
                               int8_t *T_out, float *gamma_out, void *ws, size_t ws_bytes,
                               void *stream)
{
    if (!W || !T_out || !gamma_out) return fail(BITLINEAR_ERR_NULL, "quantize_weights: W, T_out and gamma_out are required");
    if (int st = check_nk(N, K)) return st;
    if (!a16(W) || !a16(T_out) || !a4(gamma_out) || (gamma_in && !a4(gamma_in)))
        return fail(BITLINEAR_ERR_ALIGN, "quantize_weights: W/T_out need 16-byte, gamma 4-byte alignment");
    const int64_t count = N * K;
    const int nb = quant_weight_blocks(count);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!gamma_in) {
        if (!ws || ws_bytes < (size_t)nb * sizeof(double) || !a16(ws))
            return fail(BITLINEAR_ERR_WORKSPACE, "quantize_weights: needs %zu workspace bytes (16-byte aligned)",
                        (size_t)nb * sizeof(double));
        double *partial = static_cast<double *>(ws);
        if (hipError_t e = bl::launch_absmean_partial(W, count, partial, nb, s)) return hip_fail(e, "absmean_partial");
        if (hipError_t e = bl::launch_absmean_final(partial, nb, count, nullptr, gamma_out, s)) return hip_fail(e, "absmean_final");
    } else {
        if (hipError_t e = bl::launch_absmean_final(nullptr, 0, count, gamma_in, gamma_out, s)) return hip_fail(e, "absmean_final");
    }
    if (hipError_t e = bl::launch_ternarize(W, count, gamma_out, T_out, s)) return hip_fail(e, "ternarize");
    return BITLINEAR_OK;
}

int bitlinear_pack(const int8_t *T, int64_t N, int64_t K, uint8_t *P_out, void *stream)
{
    if (!T || !P_out) return fail(BITLINEAR_ERR_NULL, "pack: T and P_out are required");
    if (int st = check_nk(N, K)) return st;
    if (!a16(T) || !a16(P_out)) return fail(BITLINEAR_ERR_ALIGN, "pack: buffers need 16-byte alignment");
    if (hipError_t e = bl::launch_pack(T, N, K, P_out, static_cast<hipStream_t>(stream))) return hip_fail(e, "pack");
    return BITLINEAR_OK;
}

int bitlinear_unpack(const uint8_t *P, int64_t N, int64_t K, int8_t *T_out, void *stream)
{
    if (!P || !T_out) return fail(BITLINEAR_ERR_NULL, "unpack: P and T_out are required");
    if (int st = check_nk(N, K)) return st;
    if (!a16(P) || !a16(T_out)) return fail(BITLINEAR_ERR_ALIGN, "unpack: buffers need 16-byte alignment");
    if (hipError_t e = bl::launch_unpack(P, N, K, T_out, static_cast<hipStream_t>(stream))) return hip_fail(e, "unpack");
    return BITLINEAR_OK;
}

int bitlinear_pack5(const int8_t *T, int64_t N, int64_t K, uint8_t *P_out, void *stream)
{
    if (!T || !P_out) return fail(BITLINEAR_ERR_NULL, "pack5: T and P_out are required");
    if (int st = check_nk(N, K)) return st;
    if (!a16(T) || !a16(P_out)) return fail(BITLINEAR_ERR_ALIGN, "pack5: buffers need 16-byte alignment");
    if (hipError_t e = bl::launch_pack5(T, N, K, P_out, static_cast<hipStream_t>(stream))) return hip_fail(e, "pack5");
    return BITLINEAR_OK;
}

int bitlinear_unpack5(const uint8_t *P, int64_t N, int64_t K, int8_t *T_out, void *stream)
{
    if (!P || !T_out) return fail(BITLINEAR_ERR_NULL, "unpack5: P and T_out are required");
    if (int st = check_nk(N, K)) return st;
    if (!a16(P) || !a16(T_out)) return fail(BITLINEAR_ERR_ALIGN, "unpack5: buffers need 16-byte alignment");
    if (hipError_t e = bl::launch_unpack5(P, N, K, T_out, static_cast<hipStream_t>(stream))) return hip_fail(e, "unpack5");
    return BITLINEAR_OK;
}

int bitlinear_quant_act(const float *X, int64_t M, int64_t K, int8_t *Q_out, int64_t ldq,
                        float *absmax_out, int32_t *rowsum_out, void *stream)
{
    if (!X || !Q_out || !absmax_out) return fail(BITLINEAR_ERR_NULL, "quant_act: X, Q_out and absmax_out are required");
    if (int st = check_mnk(M, 1, K)) return st;
    if (ldq < K || ldq % 16 != 0) return fail(BITLINEAR_ERR_SHAPE, "quant_act: ldq=%lld must be >= K and a multiple of 16", (long long)ldq);
    if (!a16(X) || !a16(Q_out) || !a4(absmax_out) || (rowsum_out && !a4(rowsum_out)))
        return fail(BITLINEAR_ERR_ALIGN, "quant_act: X/Q_out need 16-byte, absmax/rowsum 4-byte alignment");
    if (hipError_t e = bl::launch_quant_act(X, M, K, Q_out, ldq, 0, absmax_out, rowsum_out, nullptr, 0,
                                            static_cast<hipStream_t>(stream)))
        return hip_fail(e, "quant_act");
    return BITLINEAR_OK;
}

int bitlinear_quant_act_rmsnorm(const float *X, int64_t M, int64_t K, const float *norm_weight, float eps,
                                int8_t *Q_out, int64_t ldq, float *absmax_out, int32_t *rowsum_out,
                                void *stream)
{
    if (!X || !Q_out || !absmax_out)
        return fail(BITLINEAR_ERR_NULL, "quant_act_rmsnorm: X, Q_out and absmax_out are required");
    if (int st = check_mnk(M, 1, K)) return st;
    if (ldq < K || ldq % 16 != 0)
        return fail(BITLINEAR_ERR_SHAPE, "quant_act_rmsnorm: ldq=%lld must be >= K and a multiple of 16", (long long)ldq);
    if (!(eps >= 0.0f) || !(eps <= 3.0e38f))
        return fail(BITLINEAR_ERR_ARG, "quant_act_rmsnorm: eps must be finite and >= 0");
    if (!a16(X) || !a16(Q_out) || !a4(absmax_out) || (rowsum_out && !a4(rowsum_out)) ||
        (norm_weight && !a4(norm_weight)))
        return fail(BITLINEAR_ERR_ALIGN, "quant_act_rmsnorm: X/Q_out need 16-byte, absmax/rowsum/norm_weight 4-byte alignment");
    if (hipError_t e = bl::launch_quant_act_rmsnorm(X, M, K, norm_weight, eps, Q_out, ldq, absmax_out,
                                                    rowsum_out, static_cast<hipStream_t>(stream)))
        return hip_fail(e, "quant_act_rmsnorm");
    return BITLINEAR_OK;
}

int bitlinear_quant_act_add_rmsnorm(const float *X, const float *R, int64_t M, int64_t K,
                                    const float *norm_weight, float eps, float *Xsum_out, int8_t *Q_out,
                                    int64_t ldq, float *absmax_out, int32_t *rowsum_out, void *stream)
{
    if (!X || !R || !Xsum_out || !Q_out || !absmax_out)
        return fail(BITLINEAR_ERR_NULL, "quant_act_add_rmsnorm: X, R, Xsum_out, Q_out and absmax_out are required");
    if (int st = check_mnk(M, 1, K)) return st;
    if (ldq < K || ldq % 16 != 0)
        return fail(BITLINEAR_ERR_SHAPE, "quant_act_add_rmsnorm: ldq=%lld must be >= K and a multiple of 16", (long long)ldq);
    if (!(eps >= 0.0f) || !(eps <= 3.0e38f))
        return fail(BITLINEAR_ERR_ARG, "quant_act_add_rmsnorm: eps must be finite and >= 0");
    if (!a16(X) || !a16(R) || !a16(Xsum_out) || !a16(Q_out) || !a4(absmax_out) || (rowsum_out && !a4(rowsum_out)) ||
        (norm_weight && !a4(norm_weight)))
        return fail(BITLINEAR_ERR_ALIGN, "quant_act_add_rmsnorm: X/R/Xsum_out/Q_out need 16-byte, absmax/rowsum/norm_weight 4-byte alignment");
    // Xsum_out may be X or R itself; any other overlap with X, R or Q is not allowed
    auto overlaps = [](const void *a, int64_t na, const void *b, int64_t nb) {
        const char *pa = static_cast<const char *>(a), *pb = static_cast<const char *>(b);
        return pa < pb + nb && pb < pa + na;
    };
    const int64_t fb = 4 * M * K;
    if ((Xsum_out != X && overlaps(Xsum_out, fb, X, fb)) || (Xsum_out != R && overlaps(Xsum_out, fb, R, fb)) ||
        overlaps(Xsum_out, fb, Q_out, M * ldq))
        return fail(BITLINEAR_ERR_ARG, "quant_act_add_rmsnorm: Xsum_out must be X, R or a separate buffer");
    if (hipError_t e = bl::launch_quant_act_add_rmsnorm(X, R, M, K, norm_weight, eps, Xsum_out, Q_out, ldq, absmax_out,
                                                        rowsum_out, static_cast<hipStream_t>(stream)))
        return hip_fail(e, "quant_act_add_rmsnorm");
    return BITLINEAR_OK;
}

int bitlinear_quant_act_relu2_gate(const float *G, const float *U, int64_t M, int64_t N, int8_t *Q_out,
                                   int64_t ldq, float *absmax_out, int32_t *rowsum_out, void *stream)
{
    if (!G || !U || !Q_out || !absmax_out)
        return fail(BITLINEAR_ERR_NULL, "quant_act_relu2_gate: G, U, Q_out and absmax_out are required");
    if (int st = check_mnk(M, 1, N)) return st;
    if (ldq < N || ldq % 16 != 0)
        return fail(BITLINEAR_ERR_SHAPE, "quant_act_relu2_gate: ldq=%lld must be >= N and a multiple of 16", (long long)ldq);
    if (!a16(G) || !a16(U) || !a16(Q_out) || !a4(absmax_out) || (rowsum_out && !a4(rowsum_out)))
        return fail(BITLINEAR_ERR_ALIGN, "quant_act_relu2_gate: G/U/Q_out need 16-byte, absmax/rowsum 4-byte alignment");
    if (hipError_t e = bl::launch_quant_act_relu2_gate(G, U, M, N, Q_out, ldq, absmax_out, rowsum_out,
                                                       static_cast<hipStream_t>(stream)))
        return hip_fail(e, "quant_act_relu2_gate");
    return BITLINEAR_OK;
}

int bitlinear_matmul(const int8_t *Q, int64_t ldq, const float *absmax, const int32_t *rowsum,
                     int64_t M, int64_t K, const uint8_t *P, const float *gamma, int64_t N,
                     float *Y_out, int32_t *acc_out, void *ws, size_t ws_bytes, void *stream)
{
    if (!Q || !absmax || !rowsum || !P || !gamma || !Y_out)
        return fail(BITLINEAR_ERR_NULL, "matmul: Q, absmax, rowsum, P, gamma and Y_out are required");
    if (int st = check_mnk(M, N, K)) return st;
    if (ldq < up(K, 64) || ldq % 16 != 0 || ldq > (int64_t(1) << 26))
        return fail(BITLINEAR_ERR_SHAPE, "matmul: ldq=%lld must be in [%lld, 2^26] and a multiple of 16", (long long)ldq,
                    (long long)up(K, 64));
    if (!a16(Q) || !a16(P) || !a16(Y_out) || (acc_out && !a16(acc_out)) || !a4(absmax) || !a4(rowsum) || !a4(gamma))
        return fail(BITLINEAR_ERR_ALIGN, "matmul: arrays need 16-byte, scalars 4-byte alignment");
    Problem p = make_problem(M, N, K);
    decompose_single(p, false);
    const WsLayout L = ws_layout(p, false);
    if (L.total > 0 && (!ws || ws_bytes < (size_t)L.total || !a16(ws)))
        return fail(BITLINEAR_ERR_WORKSPACE, "matmul: needs %lld workspace bytes (16-byte aligned)", (long long)L.total);
    if (p.kind == 1 && items_of(p) >= (int64_t(1) << 31))
        return fail(BITLINEAR_ERR_SHAPE, "matmul: grid too large");
    p.Q = const_cast<int8_t *>(Q);
    p.ldq = ldq;
    p.absmax = const_cast<float *>(absmax);
    p.rowsum = const_cast<int32_t *>(rowsum);
    p.P = P;
    p.gamma = gamma;
    p.Y = Y_out;
    p.acc_out = acc_out;
    char *base = static_cast<char *>(ws);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (p.ks > 1) {
        p.acc_ws = reinterpret_cast<int32_t *>(base + L.part);
        p.tickets = reinterpret_cast<uint32_t *>(base + L.tick);
        if (hipError_t e = bl::launch_zero_words(p.tickets, bl::ticket_count(p), s)) return hip_fail(e, "zero tickets");
    }
    if (hipError_t e = launch_contraction(p, false, s)) return hip_fail(e, "matmul");
    return BITLINEAR_OK;
}

int bitlinear_forward(const float *X, int64_t M, int64_t K, const uint8_t *P,
                      const float *gamma, int64_t N, float *Y_out, int32_t *acc_out,
                      void *ws, size_t ws_bytes, void *stream)
{
    return forward_impl("forward", X, M, K, P, gamma, N, Y_out, acc_out, ws, ws_bytes, stream);
}

int bitlinear_matmul5(const int8_t *Q, int64_t ldq, const float *absmax, const int32_t *rowsum,
                      int64_t M, int64_t K, const uint8_t *P5, const float *gamma, int64_t N,
                      float *Y_out, int32_t *acc_out, void *ws, size_t ws_bytes, void *stream)
{
    if (!Q || !absmax || !rowsum || !P5 || !gamma || !Y_out)
        return fail(BITLINEAR_ERR_NULL, "matmul5: Q, absmax, rowsum, P5, gamma and Y_out are required");
    if (int st = check_mnk(M, N, K)) return st;
    const int64_t k5 = up(K, bl::kBt5UnitCodes);
    if (ldq < k5 || ldq % 16 != 0 || ldq > (int64_t(1) << 26))
        return fail(BITLINEAR_ERR_SHAPE, "matmul5: ldq=%lld must be in [%lld, 2^26] and a multiple of 16",
                    (long long)ldq, (long long)k5);
    if (!a16(Q) || !a16(P5) || !a16(Y_out) || (acc_out && !a16(acc_out)) || !a4(absmax) || !a4(rowsum) || !a4(gamma))
        return fail(BITLINEAR_ERR_ALIGN, "matmul5: arrays need 16-byte, scalars 4-byte alignment");
    Problem p = make_problem(M, N, K);
    decompose5(p, bt5_items(M, N));
    const WsLayout L = ws_layout(p, false);
    if (L.total > 0 && (!ws || ws_bytes < (size_t)L.total || !a16(ws)))
        return fail(BITLINEAR_ERR_WORKSPACE, "matmul5: needs %lld workspace bytes (16-byte aligned)", (long long)L.total);
    if (items_of(p) >= (int64_t(1) << 31)) return fail(BITLINEAR_ERR_SHAPE, "matmul5: grid too large");
    p.Q = const_cast<int8_t *>(Q);
    p.ldq = ldq;
    p.absmax = const_cast<float *>(absmax);
    p.rowsum = const_cast<int32_t *>(rowsum);
    p.P = P5;
    p.gamma = gamma;
    p.Y = Y_out;
    p.acc_out = acc_out;
    char *base = static_cast<char *>(ws);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (p.ks > 1) {
        p.acc_ws = reinterpret_cast<int32_t *>(base + L.part);
        p.tickets = reinterpret_cast<uint32_t *>(base + L.tick);
        if (hipError_t e = bl::launch_zero_words(p.tickets, bl::ticket_count(p), s)) return hip_fail(e, "zero tickets");
    }
    if (hipError_t e = launch_contraction(p, false, s)) return hip_fail(e, "matmul5");
    return BITLINEAR_OK;
}

int bitlinear_forward5(const float *X, int64_t M, int64_t K, const uint8_t *P5,
                       const float *gamma, int64_t N, float *Y_out, int32_t *acc_out,
                       void *ws, size_t ws_bytes, void *stream)
{
    if (!X || !P5 || !gamma || !Y_out) return fail(BITLINEAR_ERR_NULL, "forward5: X, P5, gamma and Y_out are required");
    if (int st = check_mnk(M, N, K)) return st;
    if (!a16(X) || !a16(P5) || !a16(Y_out) || (acc_out && !a16(acc_out)) || !a4(gamma))
        return fail(BITLINEAR_ERR_ALIGN, "forward5: arrays need 16-byte, gamma 4-byte alignment");
    Problem p = make_problem(M, N, K);
    decompose5(p, bt5_items(M, N));
    const WsLayout L = ws_layout(p, true);
    if (!ws || ws_bytes < (size_t)L.total || !a16(ws))
        return fail(BITLINEAR_ERR_WORKSPACE, "forward5: needs %lld workspace bytes (16-byte aligned)", (long long)L.total);
    if (items_of(p) >= (int64_t(1) << 31)) return fail(BITLINEAR_ERR_SHAPE, "forward5: grid too large");
    char *base = static_cast<char *>(ws);
    p.X = X;
    p.P = P5;
    p.gamma = gamma;
    p.Y = Y_out;
    p.acc_out = acc_out;
    p.ldq = own_ldq(p);
    p.Q = reinterpret_cast<int8_t *>(base + L.q);
    p.absmax = reinterpret_cast<float *>(base + L.absmax);
    p.rowsum = reinterpret_cast<int32_t *>(base + L.rowsum);
    if (p.ks > 1) {
        p.acc_ws = reinterpret_cast<int32_t *>(base + L.part);
        p.tickets = reinterpret_cast<uint32_t *>(base + L.tick);
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (hipError_t e = bl::launch_quant_act(X, M, K, p.Q, p.ldq, 0, p.absmax, p.rowsum, p.tickets,
                                            p.tickets ? (int)bl::ticket_count(p) : 0, s))
        return hip_fail(e, "forward5: quant_act");
    if (hipError_t e = launch_contraction(p, true, s)) return hip_fail(e, "forward5: matmul5");
    return BITLINEAR_OK;
}

}  // extern "C"

// --------------------------------------------------------------------------
// Several weight matrices on one int8 input, one launch.
// --------------------------------------------------------------------------
namespace {

struct MultiPlan {
    bl::ProblemSet ps;
    int kind = 0, variant = 0, lds = 0;
    int64_t tick_bytes = 0, total_bytes = 0;  // workspace: all tickets first, then all partials
    int64_t tick_off[bl::kMultiMax] = {}, part_off[bl::kMultiMax] = {};
};

// check_ptrs = false: sizing only (buffer pointers may still be unset)
int multi_plan(const int8_t *Q, int64_t ldq, int64_t M, int64_t K, const bitlinear_weight *w, int count,
               MultiPlan &mp, bool check_ptrs = true)
{
    if (!w) return fail(BITLINEAR_ERR_NULL, "matmul_multi: weight array is NULL");
    if (count < 1 || count > bl::kMultiMax) return fail(BITLINEAR_ERR_SHAPE, "matmul_multi: count=%d not in [1, 4]", count);
    const int fmt = w[0].format;
    for (int i = 0; i < count; ++i) {
        if (check_ptrs && (!w[i].P || !w[i].gamma || !w[i].Y))
            return fail(BITLINEAR_ERR_NULL, "matmul_multi: weight %d lacks P, gamma or Y", i);
        if (w[i].format != fmt || (fmt != BITLINEAR_FORMAT_BL2 && fmt != BITLINEAR_FORMAT_BT5) || w[i].reserved != 0)
            return fail(BITLINEAR_ERR_ARG, "matmul_multi: weights need one known format and reserved == 0");
        if (int st = check_mnk(M, w[i].N, K)) return st;
        if (check_ptrs && (!a16(w[i].P) || !a16(w[i].Y) || (w[i].acc && !a16(w[i].acc)) || !a4(w[i].gamma)))
            return fail(BITLINEAR_ERR_ALIGN, "matmul_multi: weight %d buffers misaligned", i);
    }
    const int64_t kq = fmt ? up(K, bl::kBt5UnitCodes) : up(K, 64);
    if (ldq < kq || ldq % 16 != 0 || ldq > (int64_t(1) << 26))
        return fail(BITLINEAR_ERR_SHAPE, "matmul_multi: ldq=%lld must be in [%lld, 2^26] and a multiple of 16",
                    (long long)ldq, (long long)kq);
    (void)Q;
    memset(&mp.ps, 0, sizeof mp.ps);
    // decomposition over the whole launch: K is split only while all the
    // problems together are short of workgroups
    const bool g4 = !fmt && mfma32_stream(M);
    int64_t base = 0, max_upsplit = 0;
    int tpw = bl::kStreamMfmaTiles;
    for (int pass = 0; pass < (g4 ? 2 : 1); ++pass) {
        // the MFMA stream's groups: kGroupTiles tiles first, then as many
        // tiles as the tiles-per-wave choice gives
        if (pass == 1) tpw = (alds_for(M) && alds_fits(M, K)) ? 1 : mfma_tiles_for(base);
        base = 0;
        for (int i = 0; i < count; ++i) {
            const int64_t nt = (w[i].N + 63) / 64;
            base += fmt ? bt5_items(M, w[i].N) : (g4 ? (nt + 4 * tpw - 1) / (4 * tpw) : nt);
        }
        if (base < 1) base = 1;
    }
    // the tile kernel's work items over the whole launch (M > 32)
    int64_t tile_base = 0;
    if (!fmt && M > kStreamMaxM) {
        for (int i = 0; i < count; ++i)
            tile_base += (M + kTileTokens - 1) / kTileTokens * (((w[i].N + 63) / 64 + kTileRowTiles - 1) / kTileRowTiles);
    }
    int64_t all_tiles = 0;
    for (int i = 0; i < count; ++i) all_tiles += (w[i].N + 63) / 64;
    const bool W = !fmt && wide_for(M, all_tiles, (K + 63) / 64);
    int64_t items = 0, tick = 0, part = 0;
    for (int i = 0; i < count; ++i) {
        Problem &p = mp.ps.p[i];
        p = make_problem(M, w[i].N, K);
        if (fmt)
            decompose5(p, base);
        else if (W)
            decompose_wide(p);
        else
            decompose(p, base, false, g4, tpw, tile_base, g4 && alds_for(M) && alds_fits(M, K));
        mp.ps.begin[i] = (int32_t)items;
        items += items_of(p);
        max_upsplit = max_upsplit > p.upsplit ? max_upsplit : p.upsplit;
        if (p.ks > 1) {
            mp.tick_off[i] = tick;
            tick += 4 * bl::ticket_count(p);
            mp.part_off[i] = part;
            part = up(part + 4 * bl::partial_words(p), 256);
        } else {
            mp.tick_off[i] = mp.part_off[i] = -1;
        }
    }
    if (items >= (int64_t(1) << 31)) return fail(BITLINEAR_ERR_SHAPE, "matmul_multi: grid too large");
    mp.ps.begin[count] = (int32_t)items;
    mp.ps.count = count;
    mp.kind = mp.ps.p[0].kind;
    if (mp.kind == 0 && W) {
        mp.variant = wide_variant(M);
        mp.lds = (int)stream_lds_need(mp.variant, M, max_upsplit);
    } else if (mp.kind == 0) {
        mp.variant = stream_variant_for(M, max_upsplit);
        if (mp.variant == 1) mp.variant = (alds_for(M) && alds_fits(M, K)) ? 10 : tpw == 1 ? 9 : 1;
        mp.lds = (int)stream_lds_need(mp.variant, M, max_upsplit);
        if (mp.variant == 10) mp.variant = alds_variant(mp.lds);
    }
    mp.tick_bytes = up(tick, 256);
    mp.total_bytes = mp.tick_bytes + part;
    return BITLINEAR_OK;
}

}  // namespace

extern "C" {

size_t bitlinear_multi_workspace_bytes(const bitlinear_weight *w, int count, int64_t M, int64_t K)
{
    MultiPlan mp;
    const int64_t ldq = (w && count >= 1 && w[0].format == BITLINEAR_FORMAT_BT5) ? up(K, bl::kBt5UnitCodes) : up(K, 64);
    if (multi_plan(nullptr, ldq, M, K, w, count, mp, false) != BITLINEAR_OK) return SIZE_MAX;
    return (size_t)mp.total_bytes;
}

int bitlinear_matmul_multi(const int8_t *Q, int64_t ldq, const float *absmax, const int32_t *rowsum,
                           int64_t M, int64_t K, const bitlinear_weight *w, int count, void *ws,
                           size_t ws_bytes, void *stream)
{
    if (!Q || !absmax || !rowsum) return fail(BITLINEAR_ERR_NULL, "matmul_multi: Q, absmax and rowsum are required");
    if (!a16(Q) || !a4(absmax) || !a4(rowsum)) return fail(BITLINEAR_ERR_ALIGN, "matmul_multi: Q needs 16-byte, scales 4-byte alignment");
    MultiPlan mp;
    if (int st = multi_plan(Q, ldq, M, K, w, count, mp)) return st;
    if (mp.total_bytes > 0 && (!ws || ws_bytes < (size_t)mp.total_bytes || !a16(ws)))
        return fail(BITLINEAR_ERR_WORKSPACE, "matmul_multi: needs %lld workspace bytes (16-byte aligned)",
                    (long long)mp.total_bytes);
    char *base = static_cast<char *>(ws);
    for (int i = 0; i < count; ++i) {
        Problem &p = mp.ps.p[i];
        p.Q = const_cast<int8_t *>(Q);
        p.ldq = ldq;
        p.absmax = const_cast<float *>(absmax);
        p.rowsum = const_cast<int32_t *>(rowsum);
        p.P = w[i].P;
        p.gamma = w[i].gamma;
        p.Y = w[i].Y;
        p.acc_out = w[i].acc;
        if (mp.tick_off[i] >= 0) {
            p.tickets = reinterpret_cast<uint32_t *>(base + mp.tick_off[i]);
            p.acc_ws = reinterpret_cast<int32_t *>(base + mp.tick_bytes + mp.part_off[i]);
        }
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (mp.kind == 0)
        e = bl::launch_stream_multi(mp.ps, mp.variant, mp.lds, s);
    else if (mp.kind == 1)
        e = bl::launch_tile_multi(mp.ps, s);
    else
        e = bl::launch_bt5_multi(mp.ps, (int)(M < bl::kBt5Tokens ? M : bl::kBt5Tokens), s);
    if (e) return hip_fail(e, "matmul_multi");
    return BITLINEAR_OK;
}

}  // extern "C"

// --------------------------------------------------------------------------
// Cast + multi-matrix contraction.
// --------------------------------------------------------------------------
namespace {

// One token whose launch takes the wide kernel (BL2-T64 weights) casts its
// row inside every workgroup: the whole row's codes sit in LDS (64 KiB
// cap).  Otherwise the cast runs as its own kernel into the workspace,
// which then holds [multi-matrix workspace][Q][absmax][rowsum].
constexpr int64_t kCastMaxK = 65536, kCastMaxItems = 256;
struct CastPlan {
    MultiPlan mp;
    bool fused = false;
    int64_t ldq = 0, q_off = 0, a_off = 0, rs_off = 0, total = 0;
};
int cast_plan(int mode, int64_t M, int64_t K, const bitlinear_weight *w, int count, CastPlan &cp, bool check_ptrs)
{
    const bool bt5 = w && count >= 1 && w[0].format == BITLINEAR_FORMAT_BT5;
    cp.ldq = bt5 ? up(K, bl::kBt5UnitCodes) : up(K, 64);
    if (int st = multi_plan(nullptr, cp.ldq, M, K, w, count, cp.mp, check_ptrs)) return st;
    // casting in every workgroup pays where each workgroup reads fewer cast
    // input bytes than packed weights and the launch has at most one
    // workgroup per compute unit (measured per 3B-class decode-layer call,
    // graph replay: q|k|v after the residual add + norm 7.25 us against
    // 4.31 + 3.93 in two launches, o 5.22 against 2.77 + 3.81; gate|up, 270
    // workgroups, 10.39 against 4.31 + 5.66; down after the gated squared
    // ReLU, 69 KiB of input per workgroup, 10.14 against 3.49 + 5.85)
    int64_t items = 0, upsplit = 0;
    for (int i = 0; i < count; ++i) {
        items += items_of(cp.mp.ps.p[i]);
        upsplit = std::max<int64_t>(upsplit, cp.mp.ps.p[i].upsplit);
    }
    const int64_t arrays = (mode == BITLINEAR_CAST_ADD_RMSNORM) ? 3 : (mode == BITLINEAR_CAST_PLAIN) ? 1 : 2;
    cp.fused = knobs().cast_fuse && !bt5 && M == 1 && cp.mp.kind == 0 && cp.mp.variant == 12 && K <= kCastMaxK &&
               (knobs().cast_fuse == 2 || (items <= kCastMaxItems && arrays * 4 * K <= 1024 * upsplit));
    if (cp.fused) {
        cp.total = cp.mp.total_bytes;
        return BITLINEAR_OK;
    }
    cp.q_off = up(cp.mp.total_bytes, 256);
    cp.a_off = cp.q_off + up(M * cp.ldq, 256);
    cp.rs_off = cp.a_off + up(4 * M, 256);
    cp.total = cp.rs_off + up(4 * M, 256);
    return BITLINEAR_OK;
}

}  // namespace

extern "C" {

size_t bitlinear_cast_multi_workspace_bytes(int mode, const bitlinear_weight *w, int count, int64_t M, int64_t K)
{
    CastPlan cp;
    if (mode < BITLINEAR_CAST_PLAIN || mode > BITLINEAR_CAST_ADD_RMSNORM) return SIZE_MAX;
    if (cast_plan(mode, M, K, w, count, cp, false) != BITLINEAR_OK) return SIZE_MAX;
    return (size_t)cp.total;
}

int bitlinear_cast_multi_launches(int mode, const bitlinear_weight *w, int count, int64_t M, int64_t K)
{
    CastPlan cp;
    if (mode < BITLINEAR_CAST_PLAIN || mode > BITLINEAR_CAST_ADD_RMSNORM) return -1;
    if (cast_plan(mode, M, K, w, count, cp, false) != BITLINEAR_OK) return -1;
    return cp.fused ? 1 : 2;
}

int bitlinear_cast_matmul_multi(int mode, const float *X, const float *aux, const float *R, float eps,
                                float *X_out, int64_t M, int64_t K, const bitlinear_weight *w, int count,
                                void *ws, size_t ws_bytes, void *stream)
{
    const char *who = "cast_matmul_multi";
    if (mode < BITLINEAR_CAST_PLAIN || mode > BITLINEAR_CAST_ADD_RMSNORM)
        return fail(BITLINEAR_ERR_ARG, "%s: unknown cast mode %d", who, mode);
    const bool norm = mode == BITLINEAR_CAST_RMSNORM || mode == BITLINEAR_CAST_ADD_RMSNORM;
    const bool add = mode == BITLINEAR_CAST_ADD_RMSNORM, gate = mode == BITLINEAR_CAST_RELU2_GATE;
    if (!X || (gate && !aux) || (add && (!R || !X_out)))
        return fail(BITLINEAR_ERR_NULL, "%s: X (and U for the gate, R and X_out for the residual sum) are required", who);
    if (int st = check_mnk(M, 1, K)) return st;
    if (norm && (!(eps >= 0.0f) || !(eps <= 3.0e38f))) return fail(BITLINEAR_ERR_ARG, "%s: eps must be finite and >= 0", who);
    if (!a16(X) || (gate && !a16(aux)) || (norm && aux && !a4(aux)) || (add && (!a16(R) || !a16(X_out))))
        return fail(BITLINEAR_ERR_ALIGN, "%s: X, U, R and X_out need 16-byte, norm weights 4-byte alignment", who);
    if (add) {
        auto overlaps = [](const void *a, int64_t na, const void *b, int64_t nb) {
            const char *pa = static_cast<const char *>(a), *pb = static_cast<const char *>(b);
            return pa < pb + nb && pb < pa + na;
        };
        const int64_t fb = 4 * M * K;
        if (overlaps(X_out, fb, X, fb) || overlaps(X_out, fb, R, fb))
            return fail(BITLINEAR_ERR_ARG, "%s: X_out must not overlap X or R", who);
    }
    CastPlan cp;
    if (int st = cast_plan(mode, M, K, w, count, cp, true)) return st;
    if (cp.total > 0 && (!ws || ws_bytes < (size_t)cp.total || !a16(ws)))
        return fail(BITLINEAR_ERR_WORKSPACE, "%s: needs %lld workspace bytes (16-byte aligned)", who, (long long)cp.total);
    char *base = static_cast<char *>(ws);
    hipStream_t s = static_cast<hipStream_t>(stream);
    int8_t *Q = cp.fused ? nullptr : reinterpret_cast<int8_t *>(base + cp.q_off);
    float *absmax = cp.fused ? nullptr : reinterpret_cast<float *>(base + cp.a_off);
    int32_t *rowsum = cp.fused ? nullptr : reinterpret_cast<int32_t *>(base + cp.rs_off);
    MultiPlan &mp = cp.mp;
    for (int i = 0; i < count; ++i) {
        Problem &p = mp.ps.p[i];
        p.Q = Q;
        p.ldq = cp.ldq;
        p.absmax = absmax;
        p.rowsum = rowsum;
        p.P = w[i].P;
        p.gamma = w[i].gamma;
        p.Y = w[i].Y;
        p.acc_out = w[i].acc;
        if (mp.tick_off[i] >= 0) {
            p.tickets = reinterpret_cast<uint32_t *>(base + mp.tick_off[i]);
            p.acc_ws = reinterpret_cast<int32_t *>(base + mp.tick_bytes + mp.part_off[i]);
        }
    }
    hipError_t e;
    if (cp.fused) {
        bl::CastIn ci{X, aux, add ? R : nullptr, add ? X_out : nullptr, eps, (int32_t)K};
        e = bl::launch_stream_cast_multi(mp.ps, ci, mode, s);
        if (e) return hip_fail(e, who);
        return BITLINEAR_OK;
    }
    switch (mode) {
    case BITLINEAR_CAST_RMSNORM: e = bl::launch_quant_act_rmsnorm(X, M, K, aux, eps, Q, cp.ldq, absmax, rowsum, s); break;
    case BITLINEAR_CAST_ADD_RMSNORM:
        e = bl::launch_quant_act_add_rmsnorm(X, R, M, K, aux, eps, X_out, Q, cp.ldq, absmax, rowsum, s);
        break;
    case BITLINEAR_CAST_RELU2_GATE: e = bl::launch_quant_act_relu2_gate(X, aux, M, K, Q, cp.ldq, absmax, rowsum, s); break;
    default: e = bl::launch_quant_act(X, M, K, Q, cp.ldq, 0, absmax, rowsum, nullptr, 0, s); break;
    }
    if (e) return hip_fail(e, who);
    if (mp.kind == 0)
        e = bl::launch_stream_multi(mp.ps, mp.variant, mp.lds, s);
    else if (mp.kind == 1)
        e = bl::launch_tile_multi(mp.ps, s);
    else
        e = bl::launch_bt5_multi(mp.ps, (int)(M < bl::kBt5Tokens ? M : bl::kBt5Tokens), s);
    if (e) return hip_fail(e, who);
    return BITLINEAR_OK;
}

}  // extern "C"

// --------------------------------------------------------------------------
// Grouped forward: plan table construction.
// --------------------------------------------------------------------------
namespace {

struct GroupPlan {
    std::vector<Problem> probs;
    bl::GroupHeader h;
    int64_t items_s = 0, items_t = 0, items_5 = 0;  // logical work items before XCD padding
};

// Units of K that work item j of problem p streams (every kernel numbers
// the K splits of an item consecutively: split = j % ks).
int64_t item_units(const Problem &p, int64_t j)
{
    const int64_t ku = p.kind == 2 ? p.KU5 : p.KU, split = j % p.ks;
    return std::min<int64_t>(ku, (split + 1) * p.upsplit) - split * p.upsplit;
}

// Work-item map of one kernel: logical items in problem order; with
// xcd = true, workgroup b takes logical item (b % 8) * per + b / 8, so each
// of the eight XCDs walks a contiguous slice of the list.  With
// longest_first, items run longest first within a slice (the whole list
// without xcd), stably: a slice that ended on its longest items (a stack's
// down projections, K 2.7 times the others') would leave its compute units
// idle while the last of them ran.  The streaming kernels take it (few
// rounds of workgroups: the 2B decode sweep at one token 85.8 -> 83.3 us,
// at eight tokens 110.6 -> 103.4); the tile kernel does not (some 24
// rounds, and the 2B prefill sweep 0.917 -> 0.934 ms with it).
void fill_map(const std::vector<Problem> &probs, int kind, int64_t logical, int64_t slots,
              bool xcd, bool longest_first, uint32_t *map)
{
    struct It {
        uint32_t p, j;
        int64_t units;
    };
    std::vector<It> it;
    it.reserve(logical);
    for (size_t i = 0; i < probs.size(); ++i) {
        if (probs[i].kind != kind) continue;
        const int64_t n = items_of(probs[i]);
        for (int64_t j = 0; j < n; ++j) it.push_back({(uint32_t)i, (uint32_t)j, item_units(probs[i], j)});
    }
    const int64_t per = xcd ? slots / 8 : slots;
    for (int64_t b0 = 0; longest_first && b0 < logical; b0 += per) {
        const int64_t b1 = std::min<int64_t>(logical, b0 + per);
        std::stable_sort(it.begin() + b0, it.begin() + b1, [](const It &a, const It &b) { return a.units > b.units; });
    }
    for (int64_t b = 0; b < slots; ++b) {
        const int64_t j = xcd ? (b % 8) * per + b / 8 : b;
        map[2 * b] = j < logical ? it[j].p : 0xFFFFFFFFu;
        map[2 * b + 1] = j < logical ? it[j].j : 0u;
    }
}

// Validates the problems and computes the whole plan.  With ws == nullptr
// the problems' workspace pointers are left null (sizing only).
int build_group(const bitlinear_problem *in, int count, char *ws, GroupPlan &out)
{
    if (!in) return fail(BITLINEAR_ERR_NULL, "group: problem array is NULL");
    if (count < 1 || count > (1 << 20)) return fail(BITLINEAR_ERR_SHAPE, "group: count=%d out of range", count);
    memset(&out.h, 0, sizeof out.h);
    out.probs.assign(count, make_problem(1, 1, 1));
    int64_t base_items = 0, base5 = 0, max_m5 = 0;
    for (int i = 0; i < count; ++i) {
        const bitlinear_problem &q = in[i];
        if (!q.X || !q.P || !q.gamma || !q.Y) return fail(BITLINEAR_ERR_NULL, "group: problem %d lacks X, P, gamma or Y", i);
        if (int st = check_mnk(q.M, q.N, q.K)) return st;
        if (!a16(q.X) || !a16(q.P) || !a16(q.Y) || (q.acc && !a16(q.acc)) || !a4(q.gamma))
            return fail(BITLINEAR_ERR_ALIGN, "group: problem %d buffers misaligned", i);
        if ((q.format != BITLINEAR_FORMAT_BL2 && q.format != BITLINEAR_FORMAT_BT5) || q.reserved != 0)
            return fail(BITLINEAR_ERR_ARG, "group: problem %d has unknown weight format %d (or reserved != 0)", i, q.format);
        if (q.format == BITLINEAR_FORMAT_BT5) {
            base5 += bt5_items(q.M, q.N);
            max_m5 = q.M > max_m5 ? q.M : max_m5;
        }
        else if (q.M <= kStreamMaxM)
            base_items += (q.N + 63) / 64;
    }
    if (base_items < 1) base_items = 1;
    if (base5 < 1) base5 = 1;
    // the tile kernel's work items over the whole launch
    int64_t tile_base = 0;
    for (int i = 0; i < count; ++i)
        if (in[i].format != BITLINEAR_FORMAT_BT5 && in[i].M > kStreamMaxM)
            tile_base += (in[i].M + kTileTokens - 1) / kTileTokens *
                         (((in[i].N + 63) / 64 + kTileRowTiles - 1) / kTileRowTiles);
    int64_t tokens = 0, items_s = 0, items_t = 0, items_5 = 0, off = 0;
    // streaming instantiation for the whole launch: LDS-staged dot4 when every
    // streaming problem has at most two tokens (the one-token kernel if all
    // have one), MFMA otherwise
    int64_t max_upsplit = 0, max_m = 1;
    std::vector<std::pair<int64_t, int64_t>> mu;  // (M, upsplit) of the streaming problems
    for (int i = 0; i < count; ++i) {
        if (in[i].format == BITLINEAR_FORMAT_BT5) continue;
        Problem p = make_problem(in[i].M, in[i].N, in[i].K);
        decompose(p, base_items, true, false, bl::kStreamMfmaTiles, tile_base);
        if (p.kind != 0) continue;
        max_m = max_m > p.M ? max_m : p.M;
        max_upsplit = max_upsplit > p.upsplit ? max_upsplit : p.upsplit;
        mu.emplace_back(p.M, p.upsplit);
    }
    // one instantiation for the launch, from its largest token count; the
    // staged-activation variants size their LDS for every problem (a
    // one-token problem's K range is not capped) and give way to the MFMA
    // stream when that exceeds 64 KiB
    int stream_variant = stream_variant_for(max_m, max_upsplit);
    int64_t lds_tok = 0;
    if (stream_variant == 6) {
        for (const auto &x : mu) {
            const int64_t b = stream_lds_need(stream_variant, x.first, x.second);
            lds_tok = lds_tok > b ? lds_tok : b;
        }
        if (lds_tok > kStreamLdsMax) stream_variant = 1;
    }
    const bool groups4 = stream_variant == 1;
    // staged activations for the whole launch: every streaming problem fits
    bool alds_ok = groups4 && alds_for(max_m);
    for (int i = 0; i < count && alds_ok; ++i)
        if (in[i].format != BITLINEAR_FORMAT_BT5 && in[i].M <= kStreamMaxM && !alds_fits(max_m, in[i].K))
            alds_ok = false;
    int tpw = bl::kStreamMfmaTiles;
    if (groups4) {
        // the MFMA kernel's work items are tile groups: kGroupTiles tiles,
        // or 4 when the launch is too small for two tiles per wave
        for (int pass = 0; pass < 2; ++pass) {
            if (pass == 1) tpw = alds_ok ? 1 : mfma_tiles_for(base_items);
            base_items = 0;
            for (int i = 0; i < count; ++i)
                if (in[i].format != BITLINEAR_FORMAT_BT5 && in[i].M <= kStreamMaxM)
                    base_items += ((in[i].N + 63) / 64 + 4 * tpw - 1) / (4 * tpw);
            if (base_items < 1) base_items = 1;
        }
        if (tpw == 1) stream_variant = 9;
    }
    const bool alds = alds_ok;
    if (alds) stream_variant = 10;
    int64_t lds_alds = 0;
    for (int i = 0; i < count; ++i) {
        const bitlinear_problem &q = in[i];
        Problem &p = out.probs[i];
        p = make_problem(q.M, q.N, q.K);
        if (q.format == BITLINEAR_FORMAT_BT5)
            decompose5(p, base5);
        else
            decompose(p, base_items, true, groups4, tpw, tile_base, alds);
        if (alds && p.kind == 0) {
            const int64_t b = stream_lds_need(stream_variant, p.M, p.upsplit);
            lds_alds = lds_alds > b ? lds_alds : b;
        }
        p.X = q.X;
        p.P = q.P;
        p.gamma = q.gamma;
        p.Y = q.Y;
        p.acc_out = q.acc;
        p.ldq = own_ldq(p);
        const WsLayout L = ws_layout(p, true);
        if (ws) {
            char *b = ws + off;
            p.Q = reinterpret_cast<int8_t *>(b + L.q);
            p.absmax = reinterpret_cast<float *>(b + L.absmax);
            p.rowsum = reinterpret_cast<int32_t *>(b + L.rowsum);
            if (p.ks > 1) {
                p.acc_ws = reinterpret_cast<int32_t *>(b + L.part);
                p.tickets = reinterpret_cast<uint32_t *>(b + L.tick);
            }
        }
        off += L.total;
        p.tok_begin = (int32_t)tokens;
        tokens += p.M;
        if (p.kind == 0) {
            p.item_begin = (int32_t)items_s;
            items_s += items_of(p);
        } else if (p.kind == 2) {
            p.item_begin = (int32_t)items_5;
            items_5 += items_of(p);
        } else {
            p.item_begin = (int32_t)items_t;
            items_t += items_of(p);
        }
        if (tokens >= (int64_t(1) << 31) || items_s >= (int64_t(1) << 31) || items_t >= (int64_t(1) << 31) ||
            items_5 >= (int64_t(1) << 31))
            return fail(BITLINEAR_ERR_SHAPE, "group: too many tokens or work items");
    }
    bl::GroupHeader &h = out.h;
    h.magic = bl::kGroupMagic;
    h.count = count;
    h.n_tokens = (int32_t)tokens;
    out.items_s = items_s;
    out.items_t = items_t;
    out.items_5 = items_5;
    if (knobs().xcd_order & 1) items_s = up(items_s, 8);
    if (knobs().xcd_order & 2) items_t = up(items_t, 8);
    if (knobs().xcd_order & 1) items_5 = up(items_5, 8);
    h.n_items_stream = (int32_t)items_s;
    h.n_items_tile = (int32_t)items_t;
    h.n_items_bt5 = (int32_t)items_5;
    h.bt5_max_m = (int32_t)(max_m5 < bl::kBt5Tokens ? max_m5 : bl::kBt5Tokens);
    if (alds) stream_variant = alds_variant(lds_alds);
    h.stream_variant = stream_variant;
    h.stream_lds = h.stream_variant == 6 ? (int32_t)lds_tok
                   : alds ? (int32_t)lds_alds : (int32_t)stream_lds_need(h.stream_variant, 1, max_upsplit);
    h.ws_bytes = off;
    int64_t t = up(sizeof(bl::GroupHeader), 16);
    h.off_probs = t;
    t = up(t + (int64_t)count * sizeof(Problem), 16);
    h.off_tok_map = t;
    t = up(t + 4 * tokens, 16);
    h.off_stream_map = t;
    t = up(t + 8 * items_s, 16);
    h.off_tile_map = t;
    t = up(t + 8 * items_t, 16);
    h.off_bt5_map = t;
    t = up(t + 8 * items_5, 16);
    h.total_bytes = t;
    return BITLINEAR_OK;
}

int read_header(const void *table_host, const void *table_dev, bl::GroupHeader &h)
{
    if (!table_host || !table_dev) return fail(BITLINEAR_ERR_NULL, "group: table pointers are required");
    if (!a16(table_dev) || !a16(table_host)) return fail(BITLINEAR_ERR_ALIGN, "group: tables need 16-byte alignment");
    memcpy(&h, table_host, sizeof h);
    if (h.magic != bl::kGroupMagic || h.count < 1) return fail(BITLINEAR_ERR_ARG, "group: not a plan table");
    return BITLINEAR_OK;
}

}  // namespace

extern "C" {

size_t bitlinear_group_table_bytes(const bitlinear_problem *probs, int count)
{
    GroupPlan g;
    if (build_group(probs, count, nullptr, g) != BITLINEAR_OK) return 0;
    return (size_t)g.h.total_bytes;
}

size_t bitlinear_group_workspace_bytes(const bitlinear_problem *probs, int count)
{
    GroupPlan g;
    if (build_group(probs, count, nullptr, g) != BITLINEAR_OK) return SIZE_MAX;
    return (size_t)g.h.ws_bytes;
}

int bitlinear_group_plan(const bitlinear_problem *probs, int count, void *ws, size_t ws_bytes,
                         void *table_host, size_t table_bytes)
{
    if (!table_host) return fail(BITLINEAR_ERR_NULL, "group_plan: table_host is required");
    if (!a16(table_host)) return fail(BITLINEAR_ERR_ALIGN, "group_plan: table_host needs 16-byte alignment");
    GroupPlan g;
    if (int st = build_group(probs, count, nullptr, g)) return st;
    if (g.h.ws_bytes > 0 && (!ws || ws_bytes < (size_t)g.h.ws_bytes || !a16(ws)))
        return fail(BITLINEAR_ERR_WORKSPACE, "group_plan: needs %lld workspace bytes (16-byte aligned)", (long long)g.h.ws_bytes);
    if (table_bytes < (size_t)g.h.total_bytes)
        return fail(BITLINEAR_ERR_ARG, "group_plan: table needs %lld bytes", (long long)g.h.total_bytes);
    if (int st = build_group(probs, count, static_cast<char *>(ws), g)) return st;
    char *t = static_cast<char *>(table_host);
    memset(t, 0, (size_t)g.h.total_bytes);
    memcpy(t, &g.h, sizeof g.h);
    memcpy(t + g.h.off_probs, g.probs.data(), g.probs.size() * sizeof(Problem));
    uint32_t *tok = reinterpret_cast<uint32_t *>(t + g.h.off_tok_map);
    for (int i = 0; i < count; ++i) {
        const Problem &p = g.probs[i];
        if (p.tok_begin >= 0)
            for (int m = 0; m < p.M; ++m) tok[p.tok_begin + m] = (uint32_t)i;
    }
    fill_map(g.probs, 0, g.items_s, g.h.n_items_stream, knobs().xcd_order & 1, true,
             reinterpret_cast<uint32_t *>(t + g.h.off_stream_map));
    fill_map(g.probs, 1, g.items_t, g.h.n_items_tile, (knobs().xcd_order & 2) != 0, false,
             reinterpret_cast<uint32_t *>(t + g.h.off_tile_map));
    fill_map(g.probs, 2, g.items_5, g.h.n_items_bt5, knobs().xcd_order & 1, true,
             reinterpret_cast<uint32_t *>(t + g.h.off_bt5_map));
    return BITLINEAR_OK;
}

int bitlinear_group_quant_act(const void *table_host, const void *table_dev, void *stream)
{
    bl::GroupHeader h;
    if (int st = read_header(table_host, table_dev, h)) return st;
    const char *d = static_cast<const char *>(table_dev);
    if (h.n_tokens == 0) return BITLINEAR_OK;  // every problem quantizes in its contraction kernel
    if (hipError_t e = bl::launch_quant_act_group(reinterpret_cast<const Problem *>(d + h.off_probs),
                                                  reinterpret_cast<const uint32_t *>(d + h.off_tok_map),
                                                  h.n_tokens, static_cast<hipStream_t>(stream)))
        return hip_fail(e, "group quant_act");
    return BITLINEAR_OK;
}

int bitlinear_group_matmul(const void *table_host, const void *table_dev, void *stream)
{
    bl::GroupHeader h;
    if (int st = read_header(table_host, table_dev, h)) return st;
    const char *d = static_cast<const char *>(table_dev);
    const Problem *probs = reinterpret_cast<const Problem *>(d + h.off_probs);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (h.n_items_stream > 0)
        if (hipError_t e = bl::launch_stream_group(probs, reinterpret_cast<const uint2 *>(d + h.off_stream_map),
                                                   h.n_items_stream, h.stream_variant, h.stream_lds, s))
            return hip_fail(e, "group stream kernel");
    if (h.n_items_tile > 0)
        if (hipError_t e = bl::launch_tile_group(probs, reinterpret_cast<const uint2 *>(d + h.off_tile_map),
                                                 h.n_items_tile, s))
            return hip_fail(e, "group tile kernel");
    if (h.n_items_bt5 > 0)
        if (hipError_t e = bl::launch_bt5_group(probs, reinterpret_cast<const uint2 *>(d + h.off_bt5_map),
                                                h.n_items_bt5, h.bt5_max_m, s))
            return hip_fail(e, "group BT5 kernel");
    return BITLINEAR_OK;
}

int bitlinear_group_forward(const void *table_host, const void *table_dev, void *stream)
{
    if (int st = bitlinear_group_quant_act(table_host, table_dev, stream)) return st;
    return bitlinear_group_matmul(table_host, table_dev, stream);
}


// ---------------------------------------------------------------- probes

int64_t bitlinear_probe_read_sink_words(int64_t bytes, int64_t chunk_bytes)
{
    if (bytes <= 0 || bytes % 16 != 0 || chunk_bytes <= 0 || chunk_bytes % 4096 != 0) return 0;
    const int64_t chunks = (bytes + chunk_bytes - 1) / chunk_bytes;
    return chunks > (int64_t(1) << 31) - 1 ? 0 : chunks * 256;
}

int bitlinear_probe_read(const void *buf, int64_t bytes, int64_t chunk_bytes, uint32_t *sink, void *stream)
{
    if (!buf || !sink) return fail(BITLINEAR_ERR_NULL, "probe_read: buf and sink are required");
    if (!a16(buf) || !a4(sink)) return fail(BITLINEAR_ERR_ALIGN, "probe_read: buf must be 16-byte aligned");
    if (bitlinear_probe_read_sink_words(bytes, chunk_bytes) == 0)
        return fail(BITLINEAR_ERR_SHAPE, "probe_read: bytes=%lld (multiple of 16) chunk_bytes=%lld (multiple of 4096)",
                    (long long)bytes, (long long)chunk_bytes);
    const hipError_t e = bl::launch_probe_read(buf, bytes, chunk_bytes, sink, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? BITLINEAR_OK : hip_fail(e, "probe_read");
}

int bitlinear_probe_mfma(int64_t iters, int32_t a, int32_t b, int32_t blocks, int32_t *sink, void *stream)
{
    if (!sink) return fail(BITLINEAR_ERR_NULL, "probe_mfma: sink is required");
    if (!a4(sink)) return fail(BITLINEAR_ERR_ALIGN, "probe_mfma: sink must be 4-byte aligned");
    if (a < -128 || a > 127 || b < -128 || b > 127)
        return fail(BITLINEAR_ERR_ARG, "probe_mfma: a=%d b=%d outside the int8 range", a, b);
    const int64_t ab = (int64_t)(a < 0 ? -a : a) * (b < 0 ? -b : b);
    if (iters < 1 || blocks < 1 || 2048 * ab * iters >= (int64_t(1) << 31))
        return fail(BITLINEAR_ERR_SHAPE, "probe_mfma: iters=%lld blocks=%d (2048 |a b| iters must stay below 2^31)",
                    (long long)iters, blocks);
    const hipError_t e = bl::launch_probe_mfma(iters, a, b, blocks, sink, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? BITLINEAR_OK : hip_fail(e, "probe_mfma");
}

int bitlinear_probe_mfma_data(int64_t iters, const void *operands, int32_t blocks, int32_t *sink, uint64_t *clocks,
                              void *stream)
{
    if (!operands || !sink || !clocks)
        return fail(BITLINEAR_ERR_NULL, "probe_mfma_data: operands, sink and clocks are required");
    if (!a16(operands) || !a4(sink) || (reinterpret_cast<uintptr_t>(clocks) & 7) != 0)
        return fail(BITLINEAR_ERR_ALIGN, "probe_mfma_data: operands 16-byte, sink 4-byte, clocks 8-byte aligned");
    if (iters < 1 || blocks < 1)
        return fail(BITLINEAR_ERR_SHAPE, "probe_mfma_data: iters=%lld blocks=%d must be >= 1", (long long)iters, blocks);
    const hipError_t e =
        bl::launch_probe_mfma_data(iters, operands, blocks, sink, clocks, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? BITLINEAR_OK : hip_fail(e, "probe_mfma_data");
}

int bitlinear_probe_compute_units(int32_t *cus)
{
    if (!cus) return fail(BITLINEAR_ERR_NULL, "probe_compute_units: cus is required");
    int n = 0;
    if (hipError_t e = bl::probe_compute_units(&n)) return hip_fail(e, "probe_compute_units");
    *cus = n;
    return BITLINEAR_OK;
}

int bitlinear_probe_barrier(int32_t rounds, int32_t blocks, int32_t spin_limit, uint32_t *state, uint32_t *sink,
                            void *stream)
{
    if (!state || !sink) return fail(BITLINEAR_ERR_NULL, "probe_barrier: state and sink are required");
    if (!a4(state) || !a4(sink)) return fail(BITLINEAR_ERR_ALIGN, "probe_barrier: state and sink must be 4-byte aligned");
    if (rounds < 1) return fail(BITLINEAR_ERR_SHAPE, "probe_barrier: rounds=%d must be >= 1", rounds);
    if (spin_limit < 1) return fail(BITLINEAR_ERR_ARG, "probe_barrier: spin_limit=%d must be >= 1", spin_limit);
    int cus = 0;
    if (hipError_t e = bl::probe_compute_units(&cus)) return hip_fail(e, "probe_barrier");
    if (blocks < 1 || blocks > cus)
        return fail(BITLINEAR_ERR_SHAPE, "probe_barrier: blocks=%d must be in [1, %d] (one per compute unit)", blocks, cus);
    const hipError_t e = bl::launch_probe_barrier(rounds, blocks, spin_limit, state, sink, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? BITLINEAR_OK : hip_fail(e, "probe_barrier");
}

int bitlinear_probe_mfma_blocks(int32_t *blocks)
{
    if (!blocks) return fail(BITLINEAR_ERR_NULL, "probe_mfma_blocks: blocks is required");
    int n = 0;
    const hipError_t e = bl::probe_mfma_resident_blocks(&n);
    if (e != hipSuccess) return hip_fail(e, "probe_mfma_blocks");
    *blocks = n;
    return BITLINEAR_OK;
}

}  // extern "C"

// --------------------------------------------------------------------------
// The forward for callers that cannot allocate (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc): the
// workspace of bitlinear_forward -- int8 activations, scales, row sums,
// split-K partial sums and arrival tickets -- lives in a fixed device array
// of the library instead of a caller buffer.
// --------------------------------------------------------------------------
namespace {
constexpr size_t kScratchBytes = size_t(16) << 20;
constexpr int kScratchDevices = 64;
}  // namespace

// One copy per GPU, alive until the process ends.  In host code this name is
// only a handle for hipGetSymbolAddress: its device address comes from
// scratch_on_current_device() and is the only thing ever passed to kernels.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
void *g_scratch_addr[kScratchDevices];  // device address of `scratch`, per device

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and cached.
int scratch_on_current_device(const char *who, void *stream, void **out)
{
    int dev = -1;
    if (hipError_t e = hipGetDevice(&dev)) return hip_fail(e, who);
    if (stream) {
        int sdev = -1;
        if (hipError_t e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev)) return hip_fail(e, who);
        if (sdev != dev)
            return fail(BITLINEAR_ERR_ARG, "%s: the stream belongs to device %d, the current device is %d", who,
                        sdev, dev);
    }
    if (dev < 0 || dev >= kScratchDevices)
        return fail(BITLINEAR_ERR_ARG, "%s: device %d is beyond the %d the library serves", who, dev,
                    kScratchDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void *p = nullptr;
        if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) return hip_fail(e, who);
        if (!p || !a16(p)) return fail(BITLINEAR_ERR_HIP, "%s: no usable device address for the scratch array", who);
        g_scratch_addr[dev] = p;
    }
    *out = g_scratch_addr[dev];
    return BITLINEAR_OK;
}

}  // namespace

extern "C" {

size_t bitlinear_noalloc_scratch_bytes(void) { return kScratchBytes; }

int bitlinear_forward_noalloc(const float *X, int64_t M, int64_t K, const uint8_t *P, const float *gamma,
                              int64_t N, float *Y_out, int32_t *acc_out, void *stream)
{
    const char *who = "forward_noalloc";
    if (int st = forward_check(who, X, M, K, P, gamma, N, Y_out, acc_out)) return st;
    const size_t need = bitlinear_workspace_bytes(BITLINEAR_WS_FORWARD, M, N, K);
    if (need > kScratchBytes)
        return fail(BITLINEAR_ERR_WORKSPACE,
                    "%s: M=%lld N=%lld K=%lld need %zu bytes of scratch, more than the %zu the library holds "
                    "(use bitlinear_forward with a workspace)",
                    who, (long long)M, (long long)N, (long long)K, need, kScratchBytes);
    void *ws = nullptr;
    if (int st = scratch_on_current_device(who, stream, &ws)) return st;
    return forward_impl(who, X, M, K, P, gamma, N, Y_out, acc_out, ws, kScratchBytes, stream);
}

}  // extern "C"
