// chunk_common.h -- geometry and small device helpers of the chunked kernels.
#pragma once

#include <atomic>

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

// Element (i, c) of a chunk-head's [R][Dv] array stored in 32-column slices,
// [ch][Dv / 32][R][32]: a 32-column tile of R rows is one contiguous block.  The
// bf16 path keeps its saved states, deltas and their gradients this way: the
// scans write one 32-column slice per workgroup and bchunk1b reads 32-column
// tiles, each then whole 128-byte lines.
__host__ __device__ __forceinline__ size_t slice32(size_t ch, int R, int DV, int i, int c)
{
    return ((ch * (size_t)(DV / 32) + (size_t)(c >> 5)) * (size_t)R + (size_t)i) * 32 + (size_t)(c & 31);
}

// fp32 inputs at chunk 64 run the fp32-operand scans: their tables stay fp32,
// with Kh stored transposed (Kh^T [DK][C], like the bf16 tables) so that every
// operand of the forward scan is a K-contiguous row read.
template <typename TIn, int C, int DK>
constexpr bool f32_tables()
{
    return sizeof(TIn) == 4 && C == 64 && DK >= 64;
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

// ---------------------------------------------------------------------------
// Numerical-safety options of the chunked forward (gdn_shape wy_eps, clip,
// diag): damping of the WY solve's diagonal, clipping at the stage boundaries,
// and per-stage counts of non-finite and large (|x| > 1e6) values.
// ---------------------------------------------------------------------------
struct Safety {
    float clip;          // > 0: NaN -> 0, +-inf -> +-clip, clamp to [-clip, clip]
    float dinv;          // 1 / (1 + wy_eps)
    unsigned int* diag;  // GDN_DIAG_WORDS counters, or null
    __host__ __device__ bool on() const { return clip > 0.f || diag != nullptr; }
};

constexpr int NDIAG_PREP = 2 * (GDN_DIAG_W + 1);  // counter words of the prep stages P..W

// One value at a stage boundary: counted into the workgroup's LDS counters
// sd[0] (non-finite) or sd[1] (|x| > 1e6) when sd is set, then clipped when
// clip > 0.  The count branch is taken only for such values.
__device__ __forceinline__ float guard(float x, float clip, unsigned int* sd)
{
    if (sd && !(fabsf(x) <= 1e6f)) atomicAdd(&sd[isfinite(x) ? 1 : 0], 1u);
    if (clip > 0.f) x = isnan(x) ? 0.f : fminf(fmaxf(x, -clip), clip);
    return x;
}

// Add a workgroup's LDS counters to the global ones (after a barrier); integer
// sums, so the totals do not depend on the order.
__device__ __forceinline__ void flush_counts(const unsigned int* sd, unsigned int* diag, int n)
{
    const int t = threadIdx.x;
    if (diag && t < n && sd[t]) atomicAdd(&diag[t], sd[t]);
}

// Stage boundaries that no kernel of its own writes through (the outputs o and
// hT, and with clip the gradient outputs): up to 8 tensors per launch, one per
// blockIdx.y.  Each value is counted (cnt[0] non-finite, cnt[1] |x| > 1e6, when
// cnt is set) and clipped (clip > 0) in place; 16 bytes per thread per step,
// and a word is stored only when clipping changed one of its values.
struct SafeSeg {
    void* p;
    size_t n;            // elements
    int bf16;            // element type: bf16 or float
    unsigned int* cnt;   // two counters or null
};
struct SafeSegs {
    SafeSeg s[8];
    float clip;
};

template <typename T>
__device__ __forceinline__ void safe_seg(const SafeSeg& sg, float clip)
{
    constexpr int EPL = 16 / (int)sizeof(T);
    const size_t nv = sg.n / EPL;
    const size_t stride = (size_t)gridDim.x * 256;
    const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
    unsigned int nf = 0, big = 0;
    auto one = [&](float v, bool& changed) {
        if (!(fabsf(v) <= 1e6f)) {
            if (isfinite(v)) ++big;
            else ++nf;
        }
        if (clip > 0.f) {
            const float y = isnan(v) ? 0.f : fminf(fmaxf(v, -clip), clip);
            changed |= !(y == v);
            return y;
        }
        return v;
    };
    T* base = reinterpret_cast<T*>(sg.p);
    for (size_t i = gid; i < nv; i += stride) {
        uint4 u = reinterpret_cast<const uint4*>(base)[i];
        uint32_t w[4] = {u.x, u.y, u.z, u.w};
        bool changed = false;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float lo = one(__uint_as_float(w[e] << 16), changed);
                const float hi = one(__uint_as_float(w[e] & 0xFFFF0000u), changed);
                w[e] = (uint32_t)f32_to_bf16(lo).bits | ((uint32_t)f32_to_bf16(hi).bits << 16);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = __float_as_uint(one(__uint_as_float(w[e]), changed));
        }
        if (changed) reinterpret_cast<uint4*>(base)[i] = uint4{w[0], w[1], w[2], w[3]};
    }
    for (size_t i = nv * EPL + gid; i < sg.n; i += stride) {  // tail
        bool changed = false;
        const float y = one(to_f32(base[i]), changed);
        if (changed) base[i] = from_f32<T>(y);
    }
    if (sg.cnt) {
        if (nf) atomicAdd(&sg.cnt[0], nf);
        if (big) atomicAdd(&sg.cnt[1], big);
    }
}

template <int N_SEG>  // a template, so the translation units that include this share one kernel
__global__ void __launch_bounds__(256) safe_pass_kernel(SafeSegs segs)
{
    static_assert(N_SEG == 8, "SafeSegs holds 8 segments");
    const SafeSeg& sg = segs.s[blockIdx.y];
    if (sg.n == 0) return;
    if (sg.bf16) safe_seg<bf16>(sg, segs.clip);
    else safe_seg<float>(sg, segs.clip);
}

// Compute units of the current device, cached per device: the grid of a
// persistent kernel that keeps one workgroup per CU.  Only the grid size
// depends on it (not the results); a failed query falls back to 256.
inline int device_cus()
{
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Launch one pass over `count` segments (no-op when nothing is asked for).
inline gdn_status safe_pass(const SafeSeg* segs, int count, float clip, hipStream_t st)
{
    SafeSegs a{};
    a.clip = clip;
    size_t most = 0;
    int m = 0;
    for (int i = 0; i < count; ++i) {
        if (!segs[i].p || segs[i].n == 0 || (clip <= 0.f && !segs[i].cnt)) continue;
        a.s[m++] = segs[i];
        const size_t nv = segs[i].n / (segs[i].bf16 ? 8 : 4) + 1;
        if (nv > most) most = nv;
    }
    if (m == 0) return GDN_OK;
    size_t blocks = (most + 255) / 256;
    if (blocks > 2048) blocks = 2048;
    GDN_LAUNCH("safe_pass", safe_pass_kernel<8>, dim3((unsigned)blocks, (unsigned)m), dim3(256), st, a);
    return GDN_OK;
}

}  // namespace gdn
