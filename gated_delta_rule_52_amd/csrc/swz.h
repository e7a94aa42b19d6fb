// swz.h -- swizzled LDS tables of bf16 rows and their MFMA operand reads.
//
// A table holds rows of U 16-byte units (8 bf16 each); unit u of row r sits at
// slot r * U + (u ^ f(r)).  The gfx950 LDS has 64 banks of 4 bytes.  A 16-byte
// read is served in four phases of 16 lanes, a lane's phase being
// 2 * bit5 + (bit2 ^ bit3 ^ bit4) of its lane id, and a phase is free of bank
// conflicts when its lanes touch distinct 16-byte bank groups (address bits
// 4..7).  An 8-byte read (plain or transposing) is served in two phases of 32
// lanes over 256 bytes; 8-byte writes in four phases of 16 lanes, 16-byte
// writes in eight phases of 8 lanes, both over 128 bytes.  (Measured with the
// hardware's bank-conflict counter on single-wave access patterns.)  Each f
// below was chosen, by checking every access pattern of its tables against
// these rules, so that the operand reads of its tables hit every bank once.
#pragma once

#include "common.h"

namespace gdn {

// 4 units (32 bf16) a row: 16-byte row reads and transposing reads
struct SwzU4 {
    static constexpr int U = 4;
    __device__ static int f(int r) { return (((r >> 1) & 1) << 1) ^ (((r >> 3) & 1) * 3); }
};
// 8 units (64 bf16) a row: 16-byte row reads and transposing reads
struct SwzU8 {
    static constexpr int U = 8;
    __device__ static int f(int r) { return (r & 2) | ((r >> 1) & 4); }
};
// 8 units a row: 16-byte row reads, rows written as four-row column pieces
struct SwzU8w {
    static constexpr int U = 8;
    __device__ static int f(int r) { return (r >> 1) & 7; }
};
// 16 units (128 bf16) a row: 16-byte row reads
struct SwzU16 {
    static constexpr int U = 16;
    __device__ static int f(int r) { return r & 15; }
};

// 8 units a row, written as 16-byte units of consecutive rows (lane L: row
// r0 + L, one unit) and read as 16-byte row fragments (frag_rows)
struct SwzR8 {
    static constexpr int U = 8;
    __device__ static int f(int r) { return r & 7; }
};
// 16 units a row, written as whole rows of 16-byte words and read by
// transposing loads (frag_cols)
struct SwzV16 {
    static constexpr int U = 16;
    __device__ static int f(int r) { return 2 * ((r & 3) | (((r >> 3) & 1) << 2)); }
};

// 8 units a row, written as 16-byte units of consecutive rows (lane L: row
// r0 + L, one unit) and read by transposing loads (frag_cols): a channel-major
// table whose rows are channels and whose columns are tokens
struct SwzT8 {
    static constexpr int U = 8;
    __device__ static int f(int r) { return (r & 3) | ((((r >> 2) ^ (r >> 3)) & 1) << 2); }
};

// 4 units a row, read only by transposing loads in the K-permuted order
// (frag_cols_kperm): rows r and r + 4 of a load phase take different unit pairs
struct SwzK4 {
    static constexpr int U = 4;
    __device__ static int f(int r) { return ((r >> 2) & 1) << 1; }
};

// 8 (16) units a row, read only by transposing loads in the K-permuted order
// of kperm.h (frag_cols_kperm)
struct SwzK8 {
    static constexpr int U = 8;
    __device__ static int f(int r) { return r & 6; }
};
struct SwzK16 {
    static constexpr int U = 16;
    __device__ static int f(int r) { return 2 * (r & 7); }
};

template <class S>
__device__ __forceinline__ int swz_slot(int r, int u)
{
    return r * S::U + (u ^ S::f(r));
}

// index (in bf16 elements) of column c of row r
template <class S>
__device__ __forceinline__ int swz_elem(int r, int c)
{
    return swz_slot<S>(r, c >> 3) * 8 + (c & 7);
}

// address of bf16 column c of row r
template <class S>
__device__ __forceinline__ bf16* swz_at(void* tab, int r, int c)
{
    return reinterpret_cast<bf16*>(reinterpret_cast<uint4*>(tab) + swz_slot<S>(r, c >> 3)) + (c & 7);
}

// MFMA operand with K along the rows (v_mfma_f32_16x16x32_bf16 A, or B given as
// B^T rows): lane (r, kk) supplies unit u0 + kk of row r0 + r, i.e. operand row
// r, K = 8 u0 + 8 kk .. + 7.  HALF (K = 16): lanes kk >= 2 repeat kk - 2 (the
// caller zeros the other operand there).
template <class S, bool HALF = false>
__device__ __forceinline__ bf16x8 frag_rows(const void* tab, int r0, int u0)
{
    const int l = lane_id(), kk = HALF ? (l >> 4) & 1 : l >> 4;
    return __builtin_bit_cast(bf16x8, reinterpret_cast<const uint4*>(tab)[swz_slot<S>(r0 + (l & 15), u0 + kk)]);
}

// MFMA operand with K down the rows: operand(m, k) = X(k0 + k, m0 + m), from two
// transposing loads (ds_read_b64_tr_b16).  Within each group of 16 lanes such a
// load hands lane i element i & 3 of the four 16-bit values read by lane
// 4 e + (i >> 2), as its element e (e = 0..3).  So lane j of group g reads row
// k0 + 8 g + 4 h + (j >> 2), columns m0 + 4 (j & 3) .. + 3, and lane m receives
// X(k0 + 8 g + 4 h + e, m0 + m), the operand's K = 8 g + 4 h + e.  m0 is a
// multiple of 16.  HALF (K = 16): groups g >= 2 repeat g - 2.
template <class S, bool HALF = false>
__device__ __forceinline__ bf16x8 frag_cols(const void* tab, int k0, int m0)
{
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    const int l = lane_id(), j = l & 15, g = HALF ? (l >> 4) & 1 : l >> 4;
    s16x4 v[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int k = k0 + 8 * g + 4 * h + (j >> 2);
        const bf16* p = swz_at<S>(const_cast<void*>(tab), k, m0 + 4 * (j & 3));
        v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
    }
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

// As frag_cols, with the operand's K index in the order of kperm.h: position
// 8 g + e (e < 4) holds K index 4 g + e and position 8 g + 4 + e index
// 16 + 4 g + e, within the 32-long block from k0.  Lane j of group g reads row
// k0 + 16 h + 4 g + (j >> 2) in load h.
template <class S>
__device__ __forceinline__ bf16x8 frag_cols_kperm(const void* tab, int k0, int m0)
{
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    const int l = lane_id(), j = l & 15, g = l >> 4;
    s16x4 v[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int k = k0 + 16 * h + 4 * g + (j >> 2);
        const bf16* p = swz_at<S>(const_cast<void*>(tab), k, m0 + 4 * (j & 3));
        v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
    }
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

// ---------------------------------------------------------------------------
// fp32 tables: rows of U 16-byte units (4 floats each), U a multiple of 16,
// unit u of row r at slot r * U + (u ^ f(r)), f(r) = 2 h(r) with
//   h = (bit0 of r) | (bit1 ^ bit2 of r) << 1 | (bit3 of r) << 2.
// Two reads are free of bank conflicts on it (v_mfma_f32_16x16x4_f32 operands,
// r0, k0, c0 multiples of 16, u0 of 4):
//  * 16-byte row fragments: lane (m, g) = (l % 16, l / 16) reads unit u0 + g of
//    row r0 + m.  f leaves bit 0 alone, so the two lane groups of a 16-byte
//    read phase differ in it; inside a group the eight rows of the phase give
//    eight different h.
//  * 4-byte column reads: lane (m, g) reads row k0 + 4 g + e, column c0 + m.
//    Bit 1 of f permutes the four units of a 16-column block, bits 2 and 3
//    move the block by g: the 64 lanes hit 64 different banks.
// The 4-byte writes of accumulator tiles (lane (m, g) writing row x + 4 g + r,
// column y + m) are the column pattern and free of conflicts too.
template <int U_>
struct SwzF {
    static constexpr int U = U_;
    static_assert(U % 16 == 0, "bank groups repeat every 16 units");
    __device__ static int f(int r) { return 2 * ((r & 1) | (((r >> 1) ^ (r >> 2)) & 1) << 1 | ((r >> 3) & 1) << 2); }
};

// index (in floats) of column c of row r
template <class S>
__device__ __forceinline__ int swzf_idx(int r, int c)
{
    return swz_slot<S>(r, c >> 2) * 4 + (c & 3);
}

// K-contiguous operand: lane (m, g) receives unit u0 + g of row r0 + m, its
// element e being the operand's K index 4 (u0 + g) + e of MFMA e
template <class S>
__device__ __forceinline__ f32x4 ffrag_rows(const void* tab, int r0, int u0)
{
    const int l = lane_id();
    return reinterpret_cast<const f32x4*>(tab)[swz_slot<S>(r0 + (l & 15), u0 + (l >> 4))];
}

// Operand with K down the rows: lane (m, g) receives X(k0 + 4 g + e, c0 + m)
// as element e, matching the K order of ffrag_rows over the same 16-block
template <class S>
__device__ __forceinline__ f32x4 ffrag_cols(const void* tab, int k0, int c0)
{
    const int l = lane_id(), m = l & 15, g = l >> 4;
    const float* t = reinterpret_cast<const float*>(tab);
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = t[swzf_idx<S>(k0 + 4 * g + e, c0 + m)];
    return v;
}

// acc += A B over one 16-long K block given as the four fp32 MFMAs of two
// matching fragments
__device__ __forceinline__ f32x4 mma_f32_k16(f32x4 a, f32x4 b, f32x4 acc)
{
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = mfma_f32_16x16x4(a[e], b[e], acc);
    return acc;
}

}  // namespace gdn
