// mma.h -- 16x16 output tiles on the gfx950 matrix cores, operands from LDS
// (or any addressable float memory) with arbitrary row/column strides, so one
// helper serves A*B, A^T*B, A*B^T and A^T*B^T.
//
// A 16x16 tile D(i, j) += sum_k A(i, k) B(k, j), i, j in [0, 16), k in [0, K):
//   A(i, k) = A[i * ars + k * acs],   B(k, j) = B[k * brs + j * bcs].
// Result layout (both MFMA kinds): lane l holds D(4*(l/16) + r, l%16) in acc[r].
//
// MT selects the matrix-core instruction: MT_F32 uses v_mfma_f32_16x16x4_f32
// (fp32 operands, exact products), MT_BF16 v_mfma_f32_16x16x32_bf16 (operands
// rounded to bf16 nearest-even, fp32 accumulation).
#pragma once

#include "common.h"

namespace gdn {

enum { MT_F32 = 0, MT_BF16 = 1 };

__device__ __forceinline__ int acc_row(int r) { return 4 * (lane_id() >> 4) + r; }
__device__ __forceinline__ int acc_col() { return lane_id() & 15; }

template <int MT>
__device__ __forceinline__ f32x4 mma16(f32x4 acc, const float* __restrict__ A, int ars, int acs,
                                       const float* __restrict__ B, int brs, int bcs, int K)
{
    const int l = lane_id();
    const int r = l & 15, kk = l >> 4;
    if (MT == MT_F32) {
        for (int k = 0; k < K; k += 4)
            acc = mfma_f32_16x16x4(A[r * ars + (k + kk) * acs], B[(k + kk) * brs + r * bcs], acc);
    } else {
        for (int k = 0; k < K; k += 32) {
            bf16x8 a, b;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int kx = k + 8 * kk + e;
                const bool in = kx < K;
                const int kc = in ? kx : K - 1;  // in-range index: the loads stay unconditional
                const float va = A[r * ars + kc * acs], vb = B[kc * brs + r * bcs];
                a[e] = (__bf16)(in ? va : 0.f);
                b[e] = (__bf16)(in ? vb : 0.f);
            }
            acc = mfma_bf16_16x16x32(a, b, acc);
        }
    }
    return acc;
}

// Compile-time K (fully unrolled).
template <int MT, int K>
__device__ __forceinline__ f32x4 mma16k(f32x4 acc, const float* __restrict__ A, int ars, int acs,
                                        const float* __restrict__ B, int brs, int bcs)
{
    const int l = lane_id();
    const int r = l & 15, kk = l >> 4;
    if (MT == MT_F32) {
#pragma unroll
        for (int k = 0; k < K; k += 4)
            acc = mfma_f32_16x16x4(A[r * ars + (k + kk) * acs], B[(k + kk) * brs + r * bcs], acc);
    } else {
#pragma unroll
        for (int k = 0; k < K; k += 32) {
            bf16x8 a, b;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int kx = k + 8 * kk + e;
                const bool in = (K % 32 == 0) || kx < K;
                const int kc = in ? kx : K - 1;
                const float va = A[r * ars + kc * acs], vb = B[kc * brs + r * bcs];
                a[e] = (__bf16)(in ? va : 0.f);
                b[e] = (__bf16)(in ? vb : 0.f);
            }
            acc = mfma_bf16_16x16x32(a, b, acc);
        }
    }
    return acc;
}

}  // namespace gdn

namespace gdn {

// Functor form: fa(i, k) and fb(k, j) return the operand elements (masks,
// per-row scalings, transposes are expressed inside them).  K is the
// contraction length; fa / fb are called with k < K only (the bf16 paths
// clamp the index of the padding lanes to K - 1 and zero the value).
template <int MT, int K, typename FA, typename FB>
__device__ __forceinline__ f32x4 mma16f(f32x4 acc, FA fa, FB fb)
{
    const int l = lane_id();
    const int r = l & 15, kk = l >> 4;
    if (MT == MT_F32) {
#pragma unroll
        for (int k = 0; k < K; k += 4) acc = mfma_f32_16x16x4(fa(r, k + kk), fb(k + kk, r), acc);
    } else {
#pragma unroll
        for (int k = 0; k < K; k += 32) {
            bf16x8 a, b;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int kx = k + 8 * kk + e;
                const bool in = (K % 32 == 0) || kx < K;
                const int kc = in ? kx : K - 1;
                const float va = fa(r, kc), vb = fb(kc, r);
                a[e] = (__bf16)(in ? va : 0.f);
                b[e] = (__bf16)(in ? vb : 0.f);
            }
            acc = mfma_bf16_16x16x32(a, b, acc);
        }
    }
    return acc;
}

// Runtime contraction length (multiple of 4 for MT_F32).
template <int MT, typename FA, typename FB>
__device__ __forceinline__ f32x4 mma16fd(f32x4 acc, FA fa, FB fb, int K)
{
    const int l = lane_id();
    const int r = l & 15, kk = l >> 4;
    if (MT == MT_F32) {
        for (int k = 0; k < K; k += 4) acc = mfma_f32_16x16x4(fa(r, k + kk), fb(k + kk, r), acc);
    } else {
        for (int k = 0; k < K; k += 32) {
            bf16x8 a, b;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int kx = k + 8 * kk + e;
                const bool in = kx < K;
                const int kc = in ? kx : K - 1;
                const float va = fa(r, kc), vb = fb(kc, r);
                a[e] = (__bf16)(in ? va : 0.f);
                b[e] = (__bf16)(in ? vb : 0.f);
            }
            acc = mfma_bf16_16x16x32(a, b, acc);
        }
    }
    return acc;
}

}  // namespace gdn

namespace gdn {

// K-contiguous bf16 operands: A is [16 rows][K] and Bt is [16 columns][K]
// (B transposed), both with K contiguous, so each lane fetches its eight
// operand elements with one 16-byte LDS read.  Rows must be 16-byte aligned.
//   D(i, j) += sum_k A[i*lda + k] * Bt[j*ldb + k]
template <int K>
__device__ __forceinline__ f32x4 mma_kc(f32x4 acc, const bf16* __restrict__ A, int lda,
                                        const bf16* __restrict__ Bt, int ldb)
{
    const int l = lane_id();
    const int r = l & 15, kk = l >> 4;
#pragma unroll
    for (int k = 0; k < K; k += 32) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(A + r * lda + k + 8 * kk);
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(Bt + r * ldb + k + 8 * kk);
        acc = mfma_bf16_16x16x32(a, b, acc);
    }
    return acc;
}

__device__ __forceinline__ f32x4 mma_kc_dyn(f32x4 acc, const bf16* __restrict__ A, int lda,
                                            const bf16* __restrict__ Bt, int ldb, int K)
{
    const int l = lane_id();
    const int r = l & 15, kk = l >> 4;
    for (int k = 0; k < K; k += 32) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(A + r * lda + k + 8 * kk);
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(Bt + r * ldb + k + 8 * kk);
        acc = mfma_bf16_16x16x32(a, b, acc);
    }
    return acc;
}

// K = 16 on the 16x16x32 instruction: the lanes of the upper K half read an
// in-range copy of the lower half and supply a zero B operand.
__device__ __forceinline__ f32x4 mma_kc16(f32x4 acc, const bf16* __restrict__ A, int lda,
                                          const bf16* __restrict__ Bt, int ldb)
{
    const int l = lane_id();
    const int r = l & 15, kk = l >> 4, ko = 8 * (kk & 1);
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(A + r * lda + ko);
    bf16x8 b = *reinterpret_cast<const bf16x8*>(Bt + r * ldb + ko);
    if (kk >= 2) b = bf16x8{};
    return mfma_bf16_16x16x32(a, b, acc);
}

// four consecutive bf16 (8 bytes) from four floats, round to nearest even
__device__ __forceinline__ uint2 pack4_bf16(float a, float b, float c, float d)
{
    return uint2{cvt2_bf16(a, b), cvt2_bf16(c, d)};
}

}  // namespace gdn
