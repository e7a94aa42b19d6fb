// common.h -- device helpers shared by the gfx950 kernels of the gated
// delta-rule library: element conversion, MFMA fragments, launch checks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gdn.h"

namespace gdn {

// ---------------------------------------------------------------------------
// element types
// ---------------------------------------------------------------------------
struct bf16 {
    uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return __uint_as_float(((uint32_t)x.bits) << 16); }

// float -> bf16, round to nearest even, on the gfx950 conversion instruction
// (v_cvt_pk_bf16_f32: two values per instruction)
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// two floats -> two bf16 in one 32-bit word, a in the low half
__device__ __forceinline__ uint32_t cvt2_bf16(float a, float b)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), bf16x2_t));
}

__device__ __forceinline__ bf16 f32_to_bf16(float f)
{
    bf16 r;
    r.bits = __builtin_bit_cast(uint16_t, (__bf16)f);
    return r;
}

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return f32_to_bf16(x); }

// exp(x) as 2^(x*log2 e) on the hardware exp2 unit
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Element `off` of a workgroup-uniform base pointer, with the byte offset
// formed in 32 bits: the access then takes the scalar base plus a 32-bit lane
// offset, instead of a 64-bit address computed per lane.  The caller
// guarantees off * sizeof(T) < 2^32.
template <typename T> __device__ __forceinline__ T ld32(const T* base, uint32_t off)
{
    return *reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + off * (uint32_t)sizeof(T));
}
template <typename T> __device__ __forceinline__ void st32(T* base, uint32_t off, T x)
{
    *reinterpret_cast<T*>(reinterpret_cast<char*>(base) + off * (uint32_t)sizeof(T)) = x;
}

// Lane sums inside a DPP row (16 lanes) by DPP moves, which stay in the VALU
// instead of a round trip through the LDS crossbar (ds_bpermute).  Every lane
// of a group receives the group's sum, bitwise equal across the group.  All 16
// lanes of the row must be active.
template <int CTRL> __device__ __forceinline__ float dpp_mov(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
// sum over aligned groups of 4 lanes: neighbour swap, pair swap
__device__ __forceinline__ float lane4_sum(float x)
{
    x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
    return x;
}
// sum over aligned groups of 8 lanes: neighbour swap, pair swap, mirror in 8
__device__ __forceinline__ float lane8_sum(float x)
{
    x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp_mov<0x141>(x);  // row_half_mirror: lane i <- 7-i
    return x;
}
// sum over a whole row of 16 lanes
__device__ __forceinline__ float lane16_sum(float x)
{
    x = lane8_sum(x);
    x += dpp_mov<0x140>(x);  // row_mirror: lane i <- 15-i
    return x;
}

// ---------------------------------------------------------------------------
// MFMA (CDNA3/CDNA4 matrix cores), wave64
//
// v_mfma_f32_16x16x4_f32:  D[16x16] += A[16x4] * B[4x16]
//   lane l supplies A[l%16][l/16] and B[l/16][l%16];
//   lane l holds D[4*(l/16)+r][l%16] in acc[r], r = 0..3.
// v_mfma_f32_16x16x32_bf16: D[16x16] += A[16x32] * B[32x16]
//   lane l supplies A[l%16][8*(l/16)+e] and B[8*(l/16)+e][l%16], e = 0..7;
//   same D layout.
// ---------------------------------------------------------------------------
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
// 16 bytes as a native vector: unlike HIP's uint4 (a struct copied with
// memcpy), an array of these stays in registers when it is held across loops
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma_f32_16x16x4(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// bf16 pairs of neighbouring columns of an MFMA accumulator tile: lanes l and
// l ^ 1 hold columns j and j ^ 1 of the same four rows 4 (l / 16) + r.  After one
// exchange the even lane holds rows 0, 1 and the odd lane rows 2, 3 of those
// four, each as one 32-bit word of columns (j & ~1, j | 1) rounded to bf16:
// .x is row 4 (l / 16) + 2 (l & 1), .y the row after it.  Both lanes of every
// pair must be active.
__device__ __forceinline__ uint2 acc_colpairs(f32x4 v)
{
    const bool odd = (lane_id() & 1) != 0;
    const float s0 = odd ? v[0] : v[2], s1 = odd ? v[1] : v[3];  // the rows the neighbour writes
    const float n0 = dpp_mov<0xB1>(s0), n1 = dpp_mov<0xB1>(s1);  // quad_perm [1,0,3,2]
    const float a0 = odd ? n0 : v[0], b0 = odd ? v[2] : n0;
    const float a1 = odd ? n1 : v[1], b1 = odd ? v[3] : n1;
    return uint2{cvt2_bf16(a0, b0), cvt2_bf16(a1, b1)};
}

// 16-byte direct load from global memory into LDS: lane i's word lands at
// lds_wave_base + 16 i (the base is the same for the whole wave).  Written as
// inline assembly so that the compiler sees no pending LDS write (it would
// otherwise wait for the load before every LDS access it cannot tell apart
// from the target, and at every barrier); the caller waits for it with an
// explicit vmcnt and a barrier before reading the words.  The memory clobber
// keeps the compiler's memory operations on their side of the load, so the
// number of vector memory operations issued after it is what the code shows.
__device__ __forceinline__ void dma16(const void* gptr, const void* lds_wave_base)
{
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)lds_wave_base);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0v), "v"(gptr) : "memory", "m0");
}

// Touch the 128-byte line holding gptr so that it is in the L2 when the real
// load comes: a 4-byte direct load into an LDS sink that nobody reads (lane i
// writes sink_wave_base + 4 i).  Counted by vmcnt like any load.
__device__ __forceinline__ void warm_line(const void* gptr, const void* sink_wave_base)
{
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)sink_wave_base);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(m0v), "v"(gptr) : "memory", "m0");
}

// s_waitcnt with only the vector memory count limited, 0 <= N < 64 (gfx9
// encoding: vmcnt[3:0] in bits 3:0 and vmcnt[5:4] in bits 15:14)
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// s_waitcnt with only the vector memory count limited (expcnt and lgkmcnt at
// their maxima); N < 16
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x3F70 | N);
}

// Call f with std::true_type or std::false_type: a runtime flag picks a
// template instance.
template <typename F>
auto with_bool(bool b, F&& f)
{
    return b ? f(std::true_type{}) : f(std::false_type{});
}

#ifdef GDN_PROFILE
// launch recorder (include/gdn_profile.h), only in the measurement build
// (libgdn_prof.so); no-ops unless a tool enabled it
void prof_begin(const char* name, hipStream_t st);
void prof_end(hipStream_t st);
#endif

}  // namespace gdn

#ifdef GDN_PROFILE
// Launch a kernel on `st` between the recorder's marks, then check the launch.
#define GDN_LAUNCH(name, kernel, grid, block, st, ...)                   \
    do {                                                                 \
        ::gdn::prof_begin(name, st);                                     \
        hipLaunchKernelGGL(kernel, grid, block, 0, st, __VA_ARGS__);     \
        ::gdn::prof_end(st);                                             \
        if (hipGetLastError() != hipSuccess) return GDN_ERR_HIP;         \
    } while (0)
#else
// Launch a kernel on `st`, then check the launch.
#define GDN_LAUNCH(name, kernel, grid, block, st, ...)                   \
    do {                                                                 \
        (void)(name);                                                    \
        hipLaunchKernelGGL(kernel, grid, block, 0, st, __VA_ARGS__);     \
        if (hipGetLastError() != hipSuccess) return GDN_ERR_HIP;         \
    } while (0)
#endif

#define GDN_HIP_CHECK_LAUNCH()                                   \
    do {                                                         \
        if (hipGetLastError() != hipSuccess) return GDN_ERR_HIP; \
    } while (0)
