// BT5-T32: five ternary codes per byte (base 3), the packing that matches
// the ~0.4 GB footprint quoted for the 2B model (BitNet b1.58 2B4T video
// transcript, yousumm.com, "Transcription").  Geometry and the device-side
// byte decode shared by the pack and contraction kernels.
//
// A byte holds digits d_i = code_i + 1 (i = 0..4, 0 most significant) as
// b = sum_i d_i 3^(4-i) and stores s = ceil(256 b / 243).  Because 243 <
// 256, the prefix integers H_j = floor(s 3^j / 256) (j = 1..5) are exactly
// the top j digits of b read as a base-3 number, so every digit comes out of
// one multiply and one byte select:  d_0 = H_1, d_i = H_(i+1) - 3 H_i.
//
// Layout: tile t of 32 rows, unit u of 160 codes, KU5 = ceil(K / 160); the
// 1 KiB block (t * KU5 + u) holds 64 slots of 16 bytes; byte p of slot L is
// row 32 t + L % 32 with, as digit i, code k = 160 u + 32 i + 16 (L / 32) + p.
#pragma once

#include "common.hpp"

namespace bl {

constexpr int kBt5TileRows = 32;
constexpr int kBt5UnitCodes = 160;
constexpr int kBt5Tokens = 16;  // tokens per pass of the contraction kernel (two A rows each)

// The five contraction planes of one packed word (bytes p = 0..3 of the word
// are four packed bytes).  Each output word holds, byte for byte, H_1, H_2,
// H_3, H_4 and d_4 = H_5 - 3 H_4 of those bytes.  Byte-wise this is exact in
// 32-bit arithmetic: H_j <= 80 for j <= 4, so 3 H_4 <= 240 carries nowhere,
// and H_5 - 3 H_4 = d_4 >= 0 borrows nowhere.
struct Bt5Planes {
    unsigned h[5];
};
__device__ __forceinline__ Bt5Planes bt5_planes(unsigned w)
{
    // even bytes (0, 2) and odd bytes (1, 3) spread to 16-bit lanes: s * 3^j
    // <= 255 * 243 < 2^16 keeps each product inside its lane
    const unsigned e = __builtin_amdgcn_perm(0u, w, 0x0c020c00u);
    const unsigned o = __builtin_amdgcn_perm(0u, w, 0x0c030c01u);
    // byte 1 of each lane product is floor(s 3^j / 256); gather them back in
    // byte order p = 0, 1, 2, 3
    auto prefix = [&](unsigned m) {
        return __builtin_amdgcn_perm(__umul24(o, m), __umul24(e, m), 0x07030501u);
    };
    Bt5Planes r;
    r.h[0] = prefix(3u);
    r.h[1] = prefix(9u);
    r.h[2] = prefix(27u);
    r.h[3] = prefix(81u);
    const unsigned h5 = prefix(243u);
    // 3 H_4 as a shift-add kept apart from the subtraction (fused, the
    // compiler picks a 64-bit multiply-add, a multi-pass instruction)
    unsigned t3 = r.h[3] + (r.h[3] << 1);
    asm volatile("" : "+v"(t3));
    r.h[4] = h5 - t3;
    return r;
}

}  // namespace bl
