// chunk_common.h -- geometry and small device helpers of the chunked kernels.
#pragma once

#include "common.h"
#include "mma.h"

namespace gdn {

constexpr int NTHR = 256;  // threads per workgroup of every chunk kernel (4 waves)

constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <int C_, int DK_, int DV_>
struct Geo {
    static constexpr int C = C_, DK = DK_, DV = DV_;
    static constexpr int NB = C / 16;                    // 16-row tiles per chunk
    static constexpr int PD = cmax(cmax(DK, DV), C) + 4; // pitch of [C][*] LDS tables
    static constexpr int PC = C + 4;                     // pitch of [C][C] LDS tables
    static constexpr int HALF = C / 2;                   // rows per column-pass part
    static constexpr int NOFF = NB * (NB - 1) / 2;       // strictly-lower 16-tiles
    static constexpr int MAXOFF = (NOFF + 3) / 4;        // per wave
    static_assert(C % 16 == 0 && DK % 16 == 0 && DV % 16 == 0, "16-multiples only");
};

// k-th strictly lower 16-tile (ti > tj), row-major over ti then tj
__device__ __forceinline__ void off_tile(int idx, int& ti, int& tj)
{
    ti = 1;
    while ((ti * (ti + 1)) / 2 <= idx) ++ti;
    tj = idx - (ti * (ti - 1)) / 2;
}

// Level (half-block length) at which the block-boundary split separates tile
// rows ti from tile columns tj: the two 16-tiles sit in the two halves of one
// block of 2*h tokens.
__device__ __forceinline__ int off_tile_level(int ti, int tj)
{
    return 16 << (31 - __clz(ti ^ tj));
}

// Inside a diagonal 16-tile: is (i, j) (tile-local) split at level h, i.e. in
// the same 2h-block, i in its later half and j in its earlier half?
__device__ __forceinline__ bool in_level(int i, int j, int h)
{
    return (i / (2 * h) == j / (2 * h)) && ((i / h) & 1) && !((j / h) & 1);
}

// bf16 inputs at chunk 64 keep the chunk tables (W, Qg, Kh, P) in bf16, laid
// out for the K-contiguous MFMA operands of the scans; other shapes keep fp32.
template <typename TIn, int C, int DK>
constexpr bool bf16_tables()
{
    return sizeof(TIn) == 2 && C == 64 && DK >= 64;
}

template <typename TIn>
__device__ __forceinline__ float4 load4(const TIn* p);
template <>
__device__ __forceinline__ float4 load4<float>(const float* p)
{
    return *reinterpret_cast<const float4*>(p);
}
template <>
__device__ __forceinline__ float4 load4<bf16>(const bf16* p)
{
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    return float4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                  __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u)};
}

__device__ __forceinline__ void st4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }

}  // namespace gdn
