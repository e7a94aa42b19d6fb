// kperm.h -- the K-permuted operand order of the register-resident backward scan.
//
// A v_mfma_f32_16x16x32_bf16 operand lane l (row or column l%16, lane group
// g = l/16) supplies the eight K values at positions 8g..8g+7 of a 32-long K
// block, while an accumulator tile leaves lane l holding rows 4g..4g+3 of its
// 16 rows.  If every operand a scan reads from memory supplies its K index,
// inside each block of 32, in the order
//     stored position 8g + j  <-  index 4g + j          (j = 0..3)
//     stored position 8g + j  <-  index 16 + 4g + j - 4 (j = 4..7)
// then the eight values a lane must supply for K block kb are exactly the four
// it holds in accumulator tile 2kb and the four in tile 2kb + 1.  A state or
// delta tile computed by one product is then the operand of the next one
// straight from the registers that hold it, as either operand: as A with the
// M index along its columns, or as B with the N index along its columns.  The
// sum over K does not depend on the order of its terms, so the products are
// those of the unpermuted matrices.
#pragma once

#include "common.h"

namespace gdn {

// operand fragment from two accumulator tiles (rows 32kb.. and 32kb + 16..),
// rounded to bf16 nearest-even
__device__ __forceinline__ bf16x8 frag_acc(f32x4 lo, f32x4 hi)
{
    const u32x4 w = {cvt2_bf16(lo[0], lo[1]), cvt2_bf16(lo[2], lo[3]), cvt2_bf16(hi[0], hi[1]),
                     cvt2_bf16(hi[2], hi[3])};
    return __builtin_bit_cast(bf16x8, w);
}

__device__ __forceinline__ bf16x8 frag_neg(bf16x8 a)
{
    const u32x4 w = __builtin_bit_cast(u32x4, a) ^ u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
    return __builtin_bit_cast(bf16x8, w);
}

// B operand that moves K position k to output column nn: with an accumulator
// fragment of K block kb as the A operand (M along the tile's columns), the
// product is the transpose of accumulator tile 2kb (half 0) or 2kb + 1 (half 1),
// exactly (each output is one bf16 value times 1).
__device__ __forceinline__ bf16x8 frag_ident(int half)
{
    const int l = lane_id(), n = l & 15, g = l >> 4;
    u32x4 w = {0u, 0u, 0u, 0u};
    if ((n >> 2) == g) {
        const int j = 4 * half + (n & 3);  // the slot holding index 16 half + n
        const uint32_t one = 0x3F80u << (16 * (j & 1));
        w[j >> 1] = one;
    }
    return __builtin_bit_cast(bf16x8, w);
}

}  // namespace gdn
