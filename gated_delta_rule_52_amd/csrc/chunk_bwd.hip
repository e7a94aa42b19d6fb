// chunk_bwd.hip -- backward of the chunked gated delta rule on gfx950.
//
// Gradients of L(o, hT) with respect to q, k, v, g, beta and h0, given dO and
// dhT (atomic_ops card, "Features": the backward is a chain of stage kernels
// after the forward).  Nothing is kept from the forward call: the forward
// intermediates are recomputed (prep with T, then the state scan saving the
// state at the start of every chunk), then
//
//  bscan    one workgroup per (b, h, Dv-slice), chunks in reverse, carrying
//           dS = dL/dS (the state at the end of the chunk):
//             dD = scale P^T dO + Kh dS'           (gradient of the deltas)
//             dS <- Qg^T dO + gam o dS' - W^T dD
//           and dh0 = dS after chunk 0.
//  bchunk1  one workgroup per chunk-head; streams the Dv columns of S, dS',
//           dO, dD and U in 32-wide tiles and accumulates the contractions
//           over Dv:  dQg = dO S^T, dW = -dD S^T, dKh = D dS'^T,
//           dPs = dO D^T, dT(U) = dD (beta V)^T, dgam = rowsum(dS' o S),
//           plus dX_V = T^T dD -> dv = beta dX_V and <dX_V, v> (part of dbeta).
//  bchunk2  one workgroup per chunk-head (8 waves); dX_K = T^T dW,
//           dT = dT(U) + dW X_K^T, dA = -T^T dT T^T (strictly lower), then the
//           score gradients through the same block-boundary split as the
//           forward (every (i, j) pair belongs to exactly one level; at level h
//           the decay factors of the query rows and key rows are separate, so
//           sum_j dP_ij k_j o E_ij = F_i o (dP KF)_i is a matrix product), the
//           gradients of the decay factors (Gamma, Kh, gam, the level
//           factors) and finally dg = reverse cumulative sum of dG over the
//           chunk, where G is the chunk-local cumulative log-decay.
#include <type_traits>

#include "chunk_common.h"
#include "kperm.h"
#include "plan.h"
#include "swz.h"

namespace gdn {

gdn_status recompute_dispatch(const Plan& p, const void* q, const void* k, const void* v,
                              const float* g, const float* beta, const float* h0, void* o,
                              float* hT, bool out, void* ws, hipStream_t st);

template <int DV>
struct BScanCfg {
    static constexpr int BV = DV >= 32 ? 32 : DV;
    static constexpr int NS = DV / BV;
    static constexpr int PS = BV + 4;
};

// ---------------------------------------------------------------------------
// bscan (fp32 tables; the chunk-16 configurations: chunk 64 runs bscan4 or
// bscanf)
// ---------------------------------------------------------------------------
template <typename TIn, int C, int DK, int DV, int MT>
__global__ void __launch_bounds__(NTHR)
bscan_kernel(const float* __restrict__ Qgi, const float* __restrict__ Khi,
             const float* __restrict__ Wi, const float* __restrict__ Psi,
             const float* __restrict__ gami, const TIn* __restrict__ dO,
             const float* __restrict__ dhT, float* __restrict__ dSt, float* __restrict__ dDt,
             float* __restrict__ dh0, int BH, int T, int H, int NC)
{
    static_assert(!bf16_tables<TIn, C, DK>() && !f32_tables<TIn, C, DK>(), "chunk 64 runs bscan4 or bscanf");
    using G = Geo<C, DK, DV>;
    using SC = BScanCfg<DV>;
    constexpr int PD = G::PD, PC = G::PC, BV = SC::BV, NS = SC::NS, PS = SC::PS;
    __shared__ float sdS[DK][PS], sQ[C][PD], sK[C][PD], sW[C][PD], sP[C][PC], sdO[C][PS],
        sdD[C][PS], sg[DK];

    const int x = blockIdx.x;
    const int grp = x / (8 * NS), rem = x % (8 * NS);
    const int sl = rem / 8, bh = grp * 8 + rem % 8;
    if (bh >= BH) return;
    const int b = bh / H, h = bh % H;
    const int v0 = sl * BV;
    const int tid = threadIdx.x, w = tid >> 6;

    for (int idx = tid; idx < DK * BV; idx += NTHR) {
        const int i = idx / BV, j = idx % BV;
        sdS[i][j] = dhT ? dhT[((size_t)bh * DK + i) * DV + v0 + j] : 0.f;
    }
    __syncthreads();

    constexpr int TD = (C / 16) * (BV / 16);
    constexpr int TS = (DK / 16) * (BV / 16);
    constexpr int MD = (TD + 3) / 4, MS = (TS + 3) / 4;

    for (int n = NC - 1; n >= 0; --n) {
        const size_t ch = (size_t)bh * NC + n;
        {
            float* dp = dSt + ch * DK * DV;
            for (int idx = tid; idx < DK * BV; idx += NTHR) {
                const int i = idx / BV, j = idx % BV;
                dp[i * DV + v0 + j] = sdS[i][j];
            }
            const float* Qp = Qgi + ch * C * DK;
            const float* Kp = Khi + ch * C * DK;
            const float* Wp = Wi + ch * C * DK;
            for (int idx = tid; idx < C * DK / 4; idx += NTHR) {
                const int r = idx / (DK / 4), c4 = (idx % (DK / 4)) * 4;
                st4(&sQ[r][c4], load4<float>(Qp + r * DK + c4));
                st4(&sK[r][c4], load4<float>(Kp + r * DK + c4));
                st4(&sW[r][c4], load4<float>(Wp + r * DK + c4));
            }

            const float* Pp = Psi + ch * C * C;
            for (int idx = tid; idx < C * C / 4; idx += NTHR) {
                const int r = idx / (C / 4), c4 = (idx % (C / 4)) * 4;
                st4(&sP[r][c4], load4<float>(Pp + r * C + c4));
            }
            for (int i = tid; i < DK; i += NTHR) sg[i] = gami[ch * DK + i];
            for (int idx = tid; idx < C * BV; idx += NTHR) {
                const int r = idx / BV, j = idx % BV;
                const int t = n * C + r;
                sdO[r][j] = t < T ? to_f32(dO[(((size_t)b * T + t) * H + h) * DV + v0 + j]) : 0.f;
            }
        }
        __syncthreads();
        float* dDp = dDt + ch * C * DV;
#pragma unroll
        for (int m = 0; m < MD; ++m) {
            const int idx = w + 4 * m;
            if (idx < TD) {
                const int ti = idx / (BV / 16), tj = idx % (BV / 16);
                f32x4 acc = mma16k<MT, C>(zero4(), &sP[0][ti * 16], 1, PC, &sdO[0][tj * 16], PS, 1);
                acc = mma16k<MT, DK>(acc, &sK[ti * 16][0], PD, 1, &sdS[0][tj * 16], PS, 1);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = ti * 16 + acc_row(r), j = tj * 16 + acc_col();
                    sdD[i][j] = acc[r];
                    dDp[i * DV + v0 + j] = acc[r];
                }
            }
        }
        __syncthreads();
        f32x4 sn[MS];
#pragma unroll
        for (int m = 0; m < MS; ++m) {
            const int idx = w + 4 * m;
            if (idx < TS) {
                const int si = idx / (BV / 16), sj = idx % (BV / 16);
                f32x4 acc;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = si * 16 + acc_row(r);
                    acc[r] = sg[i] * sdS[i][sj * 16 + acc_col()];
                }
                acc = mma16k<MT, C>(acc, &sQ[0][si * 16], 1, PD, &sdO[0][sj * 16], PS, 1);
                f32x4 wd = mma16k<MT, C>(zero4(), &sW[0][si * 16], 1, PD, &sdD[0][sj * 16], PS, 1);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] -= wd[r];
                sn[m] = acc;
            }
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < MS; ++m) {
            const int idx = w + 4 * m;
            if (idx < TS) {
                const int si = idx / (BV / 16), sj = idx % (BV / 16);
#pragma unroll
                for (int r = 0; r < 4; ++r) sdS[si * 16 + acc_row(r)][sj * 16 + acc_col()] = sn[m][r];
            }
        }
        __syncthreads();
    }
    if (dh0) {
        for (int idx = tid; idx < DK * BV; idx += NTHR) {
            const int i = idx / BV, j = idx % BV;
            dh0[((size_t)bh * DK + i) * DV + v0 + j] = sdS[i][j];
        }
    }
}


// ---------------------------------------------------------------------------
// bscanf: the reverse scan over fp32 chunk tables (fp32 inputs, chunk 64) on
// v_mfma_f32_16x16x4_f32, the counterpart of scanf.  8 waves, one (b, h,
// 32-wide Dv slice) per workgroup; the state gradient dS' lives transposed in
// the MFMA accumulators of its owner waves (a lane's four values are four
// consecutive Dv columns of one row of dS').  Per chunk, two phases:
//   A: dD^T = dS'^T Kh^T + dO^T P                      (reads Kh^T, P, dO)
//   B: dS^T = gam dS'^T + dO^T Qg - dD^T W              (reads Qg, W, dO, gam)
// dS'^T and -dD^T go through LDS as K-contiguous A operands; the forward's
// tables are read down their columns (4-byte reads, K = 4 g + e, on the fp32
// row swizzle that keeps them free of bank conflicts), and so is the dO slice,
// whose rows are stored in an order (row s at s ^ bit2(s), its units XOR-ed by
// 4 bit3) that makes those reads conflict-free too.  Direct loads bring Qg, W
// and the decay of this chunk during phase A and Kh^T, P and dO of the next
// (earlier) chunk during phase B; dO has two buffers, being read in both
// phases.  dO rows past the sequence end are loaded from its last row: the
// rows of P and Qg they meet are zero there.
// ---------------------------------------------------------------------------
template <int DK, int DV>
__global__ void __launch_bounds__(512)
bscanf_kernel(const float* __restrict__ KhTt, const float* __restrict__ Pst,
              const float* __restrict__ Qgt, const float* __restrict__ Wt,
              const float* __restrict__ gami, const float* __restrict__ dO,
              const float* __restrict__ dhT, float* __restrict__ dSt, float* __restrict__ dDt,
              float* __restrict__ dh0, int BH, int T, int H, int NC)
{
    constexpr int C = 64, BV = 32, NS = DV / BV, NW = 8, NT = 64 * NW;
    constexpr int TS = (DK / 16) * (BV / 16), MS = TS / NW;
    static_assert(DK == 128 || DK == 64, "64 or 128 key channels");
    static_assert((C / 16) * (BV / 16) == NW && TS % NW == 0, "one dD tile and whole state tiles per wave");
    using SK = SwzF<DK / 4>;  // rows of DK floats
    using SC = SwzF<C / 4>;   // rows of C floats
    constexpr int UK = DK / 4, UC = C / 4, UB = BV / 4;
    // LDS in 16-byte units.  group A: Kh^T [DK][C], P [C][C]; group B: Qg, W [C][DK], decay
    constexpr int OK = 0, OP = OK + DK * UC, OQ = OP + C * UC, OW = OQ + C * UK, OG = OW + C * UK;
    constexpr int NTAB = OG + 64;
    constexpr int NQK = C * UK / NT, NQC = DK * UC / NT, NQP = C * UC / NT;
    static_assert(C * UK % NT == 0 && C * UC % NT == 0 && C * UB == NT,
                  "every direct-load instruction lies in one table");
    __shared__ __align__(16) f32x4 tab[NTAB];
    __shared__ __align__(16) f32x4 sdO0[C * UB], sdO1[C * UB];
    __shared__ __align__(16) f32x4 sSt[BV * UK], sDt[BV * UC];
    float* const St = reinterpret_cast<float*>(sSt);
    float* const Dt = reinterpret_cast<float*>(sDt);

    const int x = blockIdx.x;
    const int grp = x / (8 * NS), rem = x % (8 * NS);
    const int sl = rem / 8, bh = grp * 8 + rem % 8;
    if (bh >= BH) return;
    const int b = bh / H, h = bh % H;
    const int v0 = sl * BV;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int lr = l & 15, lq = l >> 4;
    const int tj = w & 1, ti = w >> 1;

    int gk[NQK], gc[NQC];
#pragma unroll
    for (int q = 0; q < NQK; ++q) {
        const int s = q * NT + tid, row = s / UK, u = s % UK;
        gk[q] = (row * UK + (u ^ SK::f(row))) * 4;
    }
#pragma unroll
    for (int q = 0; q < NQC; ++q) {
        const int s = q * NT + tid, row = s / UC, u = s % UC;
        gc[q] = (row * UC + (u ^ SC::f(row))) * 4;
    }
    // dO slot tid: stored row pr holds token row pr ^ bit2(pr), stored unit
    // pu holds unit pu ^ 4 bit3(pr) of the slice
    const int pr = tid / UB, pu = tid % UB;
    const int orow = pr ^ ((pr >> 2) & 1), ocol = v0 + 4 * (pu ^ (((pr >> 3) & 1) << 2));
    auto fetchA = [&](int n, f32x4* sdo) {
        const size_t ch = (size_t)bh * NC + n;
#pragma unroll
        for (int q = 0; q < NQC; ++q) dma16(KhTt + ch * C * DK + gc[q], tab + OK + q * NT + 64 * w);
#pragma unroll
        for (int q = 0; q < NQP; ++q) dma16(Pst + ch * C * C + gc[q], tab + OP + q * NT + 64 * w);
        const int t = min(n * C + orow, T - 1);
        dma16(dO + (((size_t)b * T + t) * H + h) * DV + ocol, sdo + 64 * w);
    };
    auto fetchB = [&](int n) {
        const size_t ch = (size_t)bh * NC + n;
        if (w == 0) dma16(gami + ch * DK + 4 * (l % (DK / 4)), tab + OG);
#pragma unroll
        for (int q = 0; q < NQK; ++q) {
            dma16(Qgt + ch * C * DK + gk[q], tab + OQ + q * NT + 64 * w);
            dma16(Wt + ch * C * DK + gk[q], tab + OW + q * NT + 64 * w);
        }
    };
    // operand with K = token rows: lane (m, g) receives dO(k0 + 4 g + e, tj*16 + m)
    auto dO_cols = [&](const f32x4* sdo, int k0) {
        const float* t = reinterpret_cast<const float*>(sdo);
        const int c = tj * 16 + lr;
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int s = k0 + 4 * lq + e, r = s ^ ((s >> 2) & 1);
            v[e] = t[(r * UB + ((c >> 2) ^ (((r >> 3) & 1) << 2))) * 4 + (c & 3)];
        }
        return v;
    };

    // state tile m: sacc[m][r] = dS'[si*16 + lr][v0 + tj*16 + 4 lq + r], si = ti + 4 m
    f32x4 sacc[MS];
#pragma unroll
    for (int m = 0; m < MS; ++m) {
        const int si = ti + (NW / 2) * m;
        sacc[m] = zero4();
        if (dhT)
            sacc[m] = *reinterpret_cast<const f32x4*>(dhT + ((size_t)bh * DK + si * 16 + lr) * DV + v0 + tj * 16 + 4 * lq);
#pragma unroll
        for (int r = 0; r < 4; ++r) St[swzf_idx<SK>(tj * 16 + 4 * lq + r, si * 16 + lr)] = sacc[m][r];
    }
    fetchA(NC - 1, ((NC - 1) & 1) ? sdO1 : sdO0);
    wait_vmcnt<0>();
    __syncthreads();

    constexpr int AFTERB = MS + 1;  // dS' and dD stores issued after group B
    static_assert(AFTERB < 16, "vmcnt field");
    auto step = [&](int n, const f32x4* sdo, f32x4* sdo_next, auto last_c) {
        constexpr bool LAST = decltype(last_c)::value;
        const size_t ch = (size_t)bh * NC + n;
        fetchB(n);
#pragma unroll
        for (int m = 0; m < MS; ++m) {
            const int si = ti + (NW / 2) * m;
            *reinterpret_cast<f32x4*>(dSt + (ch * DK + si * 16 + lr) * DV + v0 + tj * 16 + 4 * lq) = sacc[m];
        }
        // phase A: acc[r] = dD^T[tj*16 + 4 lq + r][ti*16 + lr]
        f32x4 dd = zero4();
#pragma unroll
        for (int u0 = 0; u0 < UK; u0 += 4)
            dd = mma_f32_k16(ffrag_rows<SK>(sSt, tj * 16, u0), ffrag_cols<SC>(tab + OK, 4 * u0, ti * 16), dd);
        // P^T dO: P[s][t] is zero for s < t, so K runs from the tile's first row
        for (int k0 = ti * 16; k0 < C; k0 += 16)
            dd = mma_f32_k16(dO_cols(sdo, k0), ffrag_cols<SC>(tab + OP, k0, ti * 16), dd);
        *reinterpret_cast<f32x4*>(dDt + (ch * C + ti * 16 + lr) * DV + v0 + tj * 16 + 4 * lq) = dd;
#pragma unroll
        for (int r = 0; r < 4; ++r) Dt[swzf_idx<SC>(tj * 16 + 4 * lq + r, ti * 16 + lr)] = -dd[r];
        wait_vmcnt<AFTERB>();  // Qg, W, gam of this chunk have landed
        __syncthreads();
        if constexpr (!LAST) fetchA(n - 1, sdo_next);
        // phase B: dS^T = gam dS'^T + dO^T Qg + (-dD^T) W
        const float* sg = reinterpret_cast<const float*>(tab + OG);
        f32x4 acc[MS];
#pragma unroll
        for (int m = 0; m < MS; ++m) {
            const float gk = sg[(ti + (NW / 2) * m) * 16 + lr];
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[m][r] = gk * sacc[m][r];
        }
#pragma unroll
        for (int kb = 0; kb < C / 16; ++kb) {
            const f32x4 ao = dO_cols(sdo, 16 * kb);
            const f32x4 ad = ffrag_rows<SC>(sDt, tj * 16, 4 * kb);
#pragma unroll
            for (int m = 0; m < MS; ++m) {
                const int si = ti + (NW / 2) * m;
                acc[m] = mma_f32_k16(ao, ffrag_cols<SK>(tab + OQ, 16 * kb, si * 16), acc[m]);
                acc[m] = mma_f32_k16(ad, ffrag_cols<SK>(tab + OW, 16 * kb, si * 16), acc[m]);
            }
        }
#pragma unroll
        for (int m = 0; m < MS; ++m) {
            const int si = ti + (NW / 2) * m;
            sacc[m] = acc[m];
#pragma unroll
            for (int r = 0; r < 4; ++r) St[swzf_idx<SK>(tj * 16 + 4 * lq + r, si * 16 + lr)] = acc[m][r];
        }
        if constexpr (!LAST) {
            wait_vmcnt<0>();  // Kh^T, P, dO of the next chunk have landed
            __syncthreads();
        }
    };
    // chunk n reads dO buffer n & 1
    for (int n = NC - 1; n > 0; --n) {
        if (n & 1) step(n, sdO1, sdO0, std::false_type{});
        else step(n, sdO0, sdO1, std::false_type{});
    }
    step(0, sdO0, sdO1, std::true_type{});
    if (dh0) {
#pragma unroll
        for (int m = 0; m < MS; ++m) {
            const int si = ti + (NW / 2) * m;
            *reinterpret_cast<f32x4*>(dh0 + ((size_t)bh * DK + si * 16 + lr) * DV + v0 + tj * 16 + 4 * lq) = sacc[m];
        }
    }
}

// ---------------------------------------------------------------------------
// bscan4: the reverse scan of the state gradient over bf16 chunk tables (bf16
// inputs, chunk 64): two compute waves per (b, h, 32-wide Dv slice),
// wave w owning 16 columns of dS for the whole sequence in MFMA accumulators
// that are the operands of the next products (kperm.h).  Per chunk n, from the
// last to the first, with dS' the gradient at the chunk's end and the chunk's
// forward tables Kh^T, Ps, Qg, W, the dO slice and the decay in LDS (the
// transposes Kh, P^T, Qg^T, W^T are their operands, read with transposing
// loads in the K order of kperm.h):
//     dD  = Kh dS' + P^T dO                 (P^T upper triangular)
//     dS <- gam o dS' + Qg^T dO - W^T dD    (the gradient at the chunk's start)
// dS' and dD leave as bf16 rows for bchunk1 (transposed by a 0/1 MFMA so a
// lane stores four consecutive columns).  The dO operand (K along tokens) is
// read from the LDS copy of the slice by transposing loads in the same K order.
// Two load waves bring the next chunk into the other of two LDS buffers by
// direct loads and touch the lines of the chunk three ahead into the L2.
// ---------------------------------------------------------------------------
constexpr int NTHR_B4 = 256;  // waves 0, 1 compute; waves 2, 3 load

template <int DK, int DV>
__global__ void __launch_bounds__(NTHR_B4) __attribute__((amdgpu_waves_per_eu(1, 1)))
bscan4_kernel(const bf16* __restrict__ KhTp, const bf16* __restrict__ Psp,
              const bf16* __restrict__ Qgp, const bf16* __restrict__ Wp,
              const float* __restrict__ gami, const bf16* __restrict__ dO, const float* dhT,
              bf16* __restrict__ dSt, bf16* __restrict__ dDt, float* dh0, int BH, int T, int H,
              int NC)
{
    constexpr int C = 64, BV = 32, NS = DV / BV;
    constexpr int NT = DK / 16, KB = DK / 32;
    constexpr int WK = DK / 8, WC = C / 8;
    // a buffer in 16-byte words: Kh^T [DK][WC], Ps [C][WC] (SwzK8), Qg [C][WK],
    // W [C][WK] (SK), the dO slice [C][BV] bf16 (SwzK4), the decay
    using SK = std::conditional_t<DK == 128, SwzK16, SwzK8>;
    static_assert(WC == SwzK8::U && WK == SK::U, "row widths of the swizzles");
    constexpr int OKh = 0, OPs = OKh + DK * WC, OQg = OPs + C * WC, OW = OQg + C * WK;
    constexpr int OdO = OW + C * WK, OG = OdO + C * BV / 8, QB = OG + 64;
    constexpr int NL = 128;  // threads of the two load waves
    constexpr int NQT = OdO / NL, NQO = (C * BV / 8) / NL;
    static_assert(OPs % NL == 0 && OQg % NL == 0 && OW % NL == 0 && OdO % NL == 0 &&
                  NQO * NL == C * BV / 8, "each load lies in one table");
    // 128-byte lines of a chunk's tables and decay (the dO slice: one line a row)
    constexpr int LT = (C * DK + C * C + 2 * DK * C) * 2 / 128, LG = DK * 4 / 128;
    constexpr int NWARM = 2;
    static_assert(C + (NWARM * NL - C) * NS >= LT + LG, "every line of a chunk is warmed");
    __shared__ __align__(16) uint4 sTab0[QB], sTab1[QB];
    __shared__ __align__(16) uint32_t sSink[2][64];

    const int x = blockIdx.x;
    const int grp = x / (8 * NS), rem = x % (8 * NS);
    const int sl = rem / 8, bh = grp * 8 + rem % 8;
    if (bh >= BH) return;
    const int b = bh / H, h = bh % H;
    const int v0 = sl * BV;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int ln = l & 15, lg = l >> 4;
    const bool loader = w >= 2;
    const int lt = tid & (NL - 1), lw = w & 1;
    const int vc = v0 + 16 * lw;

    // dS tile t: ds[t][r] = dS[16 t + 4 lg + r][vc + ln]
    f32x4 ds[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) ds[t] = zero4();
    if (dhT && !loader) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) ds[t][r] = dhT[((size_t)bh * DK + 16 * t + 4 * lg + r) * DV + vc + ln];
    }
    const bf16x8 id_lo = frag_ident(0), id_hi = frag_ident(1);

    auto fetch = [&](int n, uint4* buf) __attribute__((always_inline)) {
        const size_t ch = (size_t)bh * NC + n;
        if (lw == 0) dma16(gami + ch * DK + 4 * (l % (DK / 4)), buf + OG);
#pragma unroll
        for (int q = 0; q < NQT; ++q) {
            const int s0 = q * NL;
            const bool kq = s0 >= OQg;  // Qg and W rows; Kh^T and Ps rows otherwise
            const int wpr = kq ? WK : WC;
            const int off = s0 < OPs ? OKh : s0 < OQg ? OPs : s0 < OW ? OQg : OW;
            const bf16* tab = s0 < OPs ? KhTp + ch * C * DK
                            : s0 < OQg ? Psp + ch * C * C
                            : s0 < OW  ? Qgp + ch * C * DK
                                       : Wp + ch * C * DK;
            // slot (r, ws) of the swizzled table holds the row's unit ws ^ f(r)
            const int ls = s0 + lt - off, r = ls / wpr, ws = ls % wpr;
            const int wd = ws ^ (kq ? SK::f(r) : SwzK8::f(r));
            dma16(tab + (r * wpr + wd) * 8, buf + s0 + 64 * lw);
        }
        // dO rows of the chunk (rows past T repeat the last one: their P^T and
        // Qg^T columns are zero); slot (r, ws) holds the row's unit ws ^ f(r)
#pragma unroll
        for (int q = 0; q < NQO; ++q) {
            const int su = q * NL + lt, r = su / (BV / 8);
            const int t = min(n * C + r, T - 1);
            dma16(dO + (((size_t)b * T + t) * H + h) * DV + v0 + 8 * ((su % (BV / 8)) ^ SwzK4::f(r)),
                  buf + OdO + q * NL + 64 * lw);
        }
    };
    // chunk n's lines -> L2: the dO slice, and every NS-th line of the tables
    // and decay (the other slices of the head, on the same XCD, take the rest)
    auto warm = [&](int n) __attribute__((always_inline)) {
        const size_t ch = (size_t)bh * NC + n;
#pragma unroll
        for (int q = 0; q < NWARM; ++q) {
            const int s = q * NL + lt;
            const char* p;
            if (s < C) {
                const int t = min(n * C + s, T - 1);
                p = reinterpret_cast<const char*>(dO + (((size_t)b * T + t) * H + h) * DV + v0);
            } else {
                const int L = min((s - C) * NS + sl, LT + LG - 1);
                constexpr int L1 = C * DK * 2 / 128, L2 = L1 + C * C * 2 / 128, L3 = L2 + DK * C * 2 / 128;
                p = L < L1 ? reinterpret_cast<const char*>(KhTp + ch * C * DK) + 128 * L
                  : L < L2 ? reinterpret_cast<const char*>(Psp + ch * C * C) + 128 * (L - L1)
                  : L < L3 ? reinterpret_cast<const char*>(Qgp + ch * DK * C) + 128 * (L - L2)
                  : L < LT ? reinterpret_cast<const char*>(Wp + ch * DK * C) + 128 * (L - L3)
                           : reinterpret_cast<const char*>(gami + ch * DK) + 128 * (L - LT);
            }
            warm_line(p, &sSink[lw][0]);
        }
    };

    auto compute = [&](int n, const uint4* tb) __attribute__((always_inline)) {
        const size_t ch = (size_t)bh * NC + n;
        const f32x4* tG = reinterpret_cast<const f32x4*>(tb + OG);
        bf16x8 dsb[KB];  // dS' (the chunk's end) as operand fragments
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) dsb[kb] = frag_acc(ds[2 * kb], ds[2 * kb + 1]);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const f32x4 tr = mfma_bf16_16x16x32(dsb[t / 2], (t & 1) ? id_hi : id_lo, zero4());
            *reinterpret_cast<uint2*>(&dSt[slice32(ch, DK, DV, 16 * t + ln, vc + 4 * lg)]) =
                pack4_bf16(tr[0], tr[1], tr[2], tr[3]);
        }
        // dO as the operand with K along tokens (in the K order of kperm.h),
        // this wave's 16 columns
        bf16x8 dob[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) dob[kb] = frag_cols_kperm<SwzK4>(tb + OdO, 32 * kb, 16 * lw);
        // dD = Kh dS' + P^T dO (the fragments of a product are read before its
        // MFMAs: one wave per SIMD has no other wave to cover the LDS latency)
        bf16x8 kf[KB][4], pf[4][2];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) kf[kb][ti] = frag_cols_kperm<SwzK8>(tb + OKh, 32 * kb, 16 * ti);
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
            for (int kb = ti / 2; kb < 2; ++kb) pf[ti][kb] = frag_cols_kperm<SwzK8>(tb + OPs, 32 * kb, 16 * ti);
        f32x4 dd[4];
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) dd[ti] = zero4();
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) dd[ti] = mfma_bf16_16x16x32(kf[kb][ti], dsb[kb], dd[ti]);
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
            for (int kb = ti / 2; kb < 2; ++kb) dd[ti] = mfma_bf16_16x16x32(pf[ti][kb], dob[kb], dd[ti]);
        const bf16x8 ddb[2] = {frag_acc(dd[0], dd[1]), frag_acc(dd[2], dd[3])};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const f32x4 tr = mfma_bf16_16x16x32(ddb[t / 2], (t & 1) ? id_hi : id_lo, zero4());
            *reinterpret_cast<uint2*>(&dDt[slice32(ch, C, DV, 16 * t + ln, vc + 4 * lg)]) =
                pack4_bf16(tr[0], tr[1], tr[2], tr[3]);
        }
        const bf16x8 ddn[2] = {frag_neg(ddb[0]), frag_neg(ddb[1])};
        // dS <- gam o dS' + Qg^T dO - W^T dD
        bf16x8 qf[NT][2], wf[NT][2];
        f32x4 gv[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            gv[t] = tG[4 * t + lg];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                qf[t][kb] = frag_cols_kperm<SK>(tb + OQg, 32 * kb, 16 * t);
                wf[t][kb] = frag_cols_kperm<SK>(tb + OW, 32 * kb, 16 * t);
            }
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            f32x4 acc;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = gv[t][r] * ds[t][r];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) acc = mfma_bf16_16x16x32(qf[t][kb], dob[kb], acc);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) acc = mfma_bf16_16x16x32(wf[t][kb], ddn[kb], acc);
            ds[t] = acc;
        }
    };

    auto step = [&](int n, const uint4* cur, uint4* nxt) __attribute__((always_inline)) {
        if (loader) {
            fetch(max(n - 1, 0), nxt);
            warm(max(n - 3, 0));
            wait_vm<NWARM>();  // chunk n - 1 has landed
        } else {
            compute(n, cur);
        }
        __syncthreads();
    };
    if (loader) {
        fetch(NC - 1, sTab0);
        warm(max(NC - 2, 0));
        warm(max(NC - 3, 0));
        wait_vm<2 * NWARM>();
    }
    __syncthreads();
    int i = 0;
    for (; i + 1 < NC; i += 2) {
        step(NC - 1 - i, sTab0, sTab1);
        step(NC - 2 - i, sTab1, sTab0);
    }
    if (i < NC) step(NC - 1 - i, sTab0, sTab1);
    wait_vm<0>();  // no direct load may still write the LDS when the workgroup ends
    if (dh0 && !loader) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dh0[((size_t)bh * DK + 16 * t + 4 * lg + r) * DV + vc + ln] = ds[t][r];
    }
}

// ---------------------------------------------------------------------------
// bchunk1 (fp32 tables; the chunk-16 configurations: chunk 64 runs bchunk1b or
// bchunk1f)
// ---------------------------------------------------------------------------
template <typename TIn, int C, int DK, int DV, int MT>
__global__ void __launch_bounds__(NTHR)
bchunk1_kernel(const TIn* __restrict__ v, const float* __restrict__ beta,
               const TIn* __restrict__ dO, const float* __restrict__ Wi,
               const float* __restrict__ Ui, const float* __restrict__ Tmi,
               const float* __restrict__ Sst, const float* __restrict__ dSt,
               const float* __restrict__ dDt, TIn* __restrict__ dvo, float* __restrict__ dQgo,
               float* __restrict__ dWgo, float* __restrict__ dKho, float* __restrict__ dPso,
               float* __restrict__ dT1o, float* __restrict__ dgmo, float* __restrict__ dbpo, int T,
               int H, int NC)
{
    static_assert(!bf16_tables<TIn, C, DK>() && !f32_tables<TIn, C, DK>(), "chunk 64 runs bchunk1b or bchunk1f");
    using G = Geo<C, DK, DV>;
    constexpr int PD = G::PD, PC = G::PC, NB = G::NB;
    constexpr int BW = DV >= 32 ? 32 : DV, PW = BW + 4;
    __shared__ float sW[C][PD], sT[C][PC], sS[DK][PW], sdS[DK][PW], sdO[C][PW], sdD[C][PW],
        sD[C][PW], sv[C][PW], sxv[C][PW], sdx[C][PW], sbeta[C], sred[NTHR];

    const int ch = blockIdx.x;
    const int n = ch % NC, bh = ch / NC, h = bh % H, b = bh / H;
    const int t0 = n * C;
    const int nvalid = min(C, T - t0);
    const int tid = threadIdx.x, w = tid >> 6;
    const size_t tok0 = ((size_t)b * T + t0) * H + h;
    const size_t rsV = (size_t)H * DV;

    {
        for (int idx = tid; idx < C * DK / 4; idx += NTHR) {
            const int r = idx / (DK / 4), c4 = (idx % (DK / 4)) * 4;
            st4(&sW[r][c4], load4<float>(Wi + (size_t)ch * C * DK + r * DK + c4));
        }
        const float* Tp = Tmi + (size_t)ch * C * C;
        for (int idx = tid; idx < C * C / 4; idx += NTHR) {
            const int r = idx / (C / 4), c4 = (idx % (C / 4)) * 4;
            st4(&sT[r][c4], load4<float>(Tp + r * C + c4));
        }
        for (int r = tid; r < C; r += NTHR) sbeta[r] = r < nvalid ? beta[tok0 + (size_t)r * H] : 0.f;
    }

    constexpr int T3 = NB * (DK / 16), M3 = (T3 + 3) / 4;  // [C x DK] tiles per wave
    constexpr int T2 = NB * NB, M2 = (T2 + 3) / 4;         // [C x C] tiles per wave
    constexpr int TD = NB * (BW / 16), MD = (TD + 3) / 4;   // [C x BW] tiles per wave
    f32x4 aQ[M3], aW[M3], aK[M3], aP[M2], aT[M2];
#pragma unroll
    for (int m = 0; m < M3; ++m) aQ[m] = aW[m] = aK[m] = zero4();
#pragma unroll
    for (int m = 0; m < M2; ++m) aP[m] = aT[m] = zero4();
    constexpr int NG = (NTHR / DK) > 0 ? NTHR / DK : 1;  // threads per key channel
    const int gc = tid % DK, gg = tid / DK;
    float dgm_part = 0.f, dbp_part = 0.f;

    const float* Sp = Sst + (size_t)ch * DK * DV;
    const float* dSp = dSt + (size_t)ch * DK * DV;
    const float* dDp = dDt + (size_t)ch * C * DV;
    const float* Up = Ui + (size_t)ch * C * DV;

    for (int v0 = 0; v0 < DV; v0 += BW) {
        __syncthreads();
        for (int idx = tid; idx < DK * BW; idx += NTHR) {
            const int i = idx / BW, j = idx % BW;
            sS[i][j] = Sp[i * DV + v0 + j];
            sdS[i][j] = dSp[i * DV + v0 + j];
        }
        for (int idx = tid; idx < C * BW; idx += NTHR) {
            const int r = idx / BW, j = idx % BW;
            float dov = 0.f, vv = 0.f;
            if (r < nvalid) {
                dov = to_f32(dO[(tok0 + (size_t)r * H) * DV + v0 + j]);
                vv = to_f32(v[tok0 * DV + r * rsV + v0 + j]);
            }
            sdO[r][j] = dov;
            sv[r][j] = vv;
            sxv[r][j] = sbeta[r] * vv;
            sdD[r][j] = dDp[r * DV + v0 + j];
            sD[r][j] = Up[r * DV + v0 + j];
        }
        __syncthreads();
        // D = U - W S ; dX_V = T^T dD (dv = beta dX_V)
#pragma unroll
        for (int m = 0; m < MD; ++m) {
            const int idx = w + 4 * m;
            if (idx < TD) {
                const int ti = idx / (BW / 16), tj = idx % (BW / 16);
                f32x4 ws = mma16k<MT_F32, DK>(zero4(), &sW[ti * 16][0], PD, 1, &sS[0][tj * 16], PW, 1);
                f32x4 dx = mma16k<MT, C>(zero4(), &sT[0][ti * 16], 1, PC, &sdD[0][tj * 16], PW, 1);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = ti * 16 + acc_row(r), j = tj * 16 + acc_col();
                    sD[i][j] -= ws[r];
                    sdx[i][j] = dx[r];
                    if (i < nvalid) dvo[(tok0 + (size_t)i * H) * DV + v0 + j] = from_f32<TIn>(sbeta[i] * dx[r]);
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < M3; ++m) {
            const int idx = w + 4 * m;
            if (idx < T3) {
                const int ti = idx / (DK / 16), tj = idx % (DK / 16);
                aQ[m] = mma16k<MT, BW>(aQ[m], &sdO[ti * 16][0], PW, 1, &sS[tj * 16][0], 1, PW);
                aW[m] = mma16k<MT, BW>(aW[m], &sdD[ti * 16][0], PW, 1, &sS[tj * 16][0], 1, PW);
                aK[m] = mma16k<MT, BW>(aK[m], &sD[ti * 16][0], PW, 1, &sdS[tj * 16][0], 1, PW);
            }
        }
#pragma unroll
        for (int m = 0; m < M2; ++m) {
            const int idx = w + 4 * m;
            if (idx < T2) {
                const int ti = idx / NB, tj = idx % NB;
                aP[m] = mma16k<MT, BW>(aP[m], &sdO[ti * 16][0], PW, 1, &sD[tj * 16][0], 1, PW);
                aT[m] = mma16k<MT, BW>(aT[m], &sdD[ti * 16][0], PW, 1, &sxv[tj * 16][0], 1, PW);
            }
        }
        if (gg < NG) {
            for (int j = gg; j < BW; j += NG) dgm_part += sdS[gc][j] * sS[gc][j];
        }
        for (int r = tid; r < C; r += NTHR) {
            float s = 0.f;
            for (int j = 0; j < BW; ++j) s += sdx[r][j] * sv[r][j];
            dbp_part += s;
        }
    }

    // outputs
    float* dQp = dQgo + (size_t)ch * C * DK;
    float* dWp = dWgo + (size_t)ch * C * DK;
    float* dKp = dKho + (size_t)ch * C * DK;
#pragma unroll
    for (int m = 0; m < M3; ++m) {
        const int idx = w + 4 * m;
        if (idx < T3) {
            const int ti = idx / (DK / 16), tj = idx % (DK / 16);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = ti * 16 + acc_row(r), j = tj * 16 + acc_col();
                dQp[i * DK + j] = aQ[m][r];
                dWp[i * DK + j] = -aW[m][r];
                dKp[i * DK + j] = aK[m][r];
            }
        }
    }
    float* dPp = dPso + (size_t)ch * C * C;
    float* dTp = dT1o + (size_t)ch * C * C;
#pragma unroll
    for (int m = 0; m < M2; ++m) {
        const int idx = w + 4 * m;
        if (idx < T2) {
            const int ti = idx / NB, tj = idx % NB;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = ti * 16 + acc_row(r), j = tj * 16 + acc_col();
                dPp[i * C + j] = aP[m][r];
                dTp[i * C + j] = aT[m][r];
            }
        }
    }
    sred[tid] = dgm_part;
    __syncthreads();
    if (tid < DK) {
        float s = 0.f;
        for (int gi = 0; gi < NG; ++gi) s += sred[gi * DK + tid];
        dgmo[(size_t)ch * DK + tid] = s;
    }
    for (int r = tid; r < C; r += NTHR) dbpo[(size_t)ch * C + r] = dbp_part;
}


// ---------------------------------------------------------------------------
// bchunk1f: the chunk-local contractions of the backward over fp32 operands
// (fp32 inputs, chunk 64) on v_mfma_f32_16x16x4_f32, one workgroup of 8 waves
// per chunk-head, streaming Dv in 64-column slices through LDS (S, dS, dO,
// dD, v and the chunk deltas D saved by the forward scan, rows on the fp32
// swizzle).  Per slice:
//   1: dX_V^T = dD^T T (dv = beta dX_V, dbeta through U)
//   2: dQg^T += S dO^T, dW^T += S dD^T, dKh^T += dS D^T, dPs^T += D dO^T,
//      dT1^T += v dD^T (times beta of the key row at the end), dgam += dS o S
// Every product is computed transposed, so that each result leaves as
// 16-byte rows of the [C][*] outputs; its A operands are rows of the [*][Dv]
// slice tables and its B operands rows of the [C][Dv] ones, both read along
// Dv (the contraction index).  Phase 1 reads dD and T down their columns
// instead.
// ---------------------------------------------------------------------------
template <int DK, int DV>
__global__ void __launch_bounds__(512)
bchunk1f_kernel(const float* __restrict__ v, const float* __restrict__ beta,
                const float* __restrict__ dO, const float* __restrict__ Dsti,
                const float* __restrict__ Tmi,
                const float* __restrict__ Sst, const float* __restrict__ dSt,
                const float* __restrict__ dDt, float* __restrict__ dvo, float* __restrict__ dQgo,
                float* __restrict__ dWgo, float* __restrict__ dKho, float* __restrict__ dPso,
                float* __restrict__ dT1o, float* __restrict__ dgmo, float* __restrict__ dbpo, int T,
                int H, int NC)
{
    constexpr int C = 64, BW = 64, NT = 512, NSL = DV / BW;
    constexpr int NI = DK / 16, MI = NI / 2;  // key-channel tiles, per wave
    static_assert(DK == 128 || DK == 64, "64 or 128 key channels");
    static_assert(DV % BW == 0, "whole 64-column slices");
    using SF = SwzF<BW / 4>;  // every slice table: rows of 64 floats
    constexpr int UW = BW / 4;
    __shared__ __align__(16) f32x4 sS[DK * UW], sdS[DK * UW], sdO[C * UW], sdD[C * UW], sD[C * UW], sv[C * UW];
    __shared__ __align__(16) f32x4 sT[C * (C / 4)];  // T [C][C], the same row swizzle
    __shared__ float sred[2][C];

    const int ch = blockIdx.x;
    const int n = ch % NC, bh = ch / NC, h = bh % H, b = bh / H;
    const int t0 = n * C;
    const int nvalid = min(C, T - t0);
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int lr = l & 15, lq = l >> 4;
    const size_t tok0 = ((size_t)b * T + t0) * H + h;  // token index of row 0
    // this wave: tokens ti*16.. (the B side), key-channel tiles ih*MI.., key
    // rows sh*32.. (dPs, dT1), and in phase 1 the slice's column tiles jh, jh + 2
    const int ti = w & 3, ih = w >> 2, sh = w >> 2, jh = w >> 2;
    const int tr = ti * 16 + lr;  // this lane's token row on the B side

    const float btr = tr < nvalid ? beta[tok0 + (size_t)tr * H] : 0.f;
    // T: loaded with the first slice
#pragma unroll
    for (int q = 0; q < C * (C / 4) / NT; ++q) {
        const int s = q * NT + tid, row = s / (C / 4), u = (s % (C / 4)) ^ SF::f(row);
        dma16(Tmi + ((size_t)ch * C + row) * C + 4 * u, sT + q * NT + 64 * w);
    }

    // slice loads: slot q * NT + tid of a table takes unit (row, u ^ f(row))
    auto fetch = [&](int v0) {
#pragma unroll
        for (int q = 0; q < DK * UW / NT; ++q) {
            const int s = q * NT + tid, row = s / UW, u = (s % UW) ^ SF::f(row);
            const size_t go = ((size_t)ch * DK + row) * DV + v0 + 4 * u;
            dma16(Sst + go, sS + q * NT + 64 * w);
            dma16(dSt + go, sdS + q * NT + 64 * w);
        }
#pragma unroll
        for (int q = 0; q < C * UW / NT; ++q) {
            const int s = q * NT + tid, row = s / UW, u = (s % UW) ^ SF::f(row);
            const int rc = min(row, nvalid - 1);  // rows past the end: zeroed after the wait
            const size_t tk = (tok0 + (size_t)rc * H) * DV + v0 + 4 * u;
            dma16(dO + tk, sdO + q * NT + 64 * w);
            dma16(v + tk, sv + q * NT + 64 * w);
            dma16(dDt + ((size_t)ch * C + row) * DV + v0 + 4 * u, sdD + q * NT + 64 * w);
            dma16(Dsti + ((size_t)ch * C + row) * DV + v0 + 4 * u, sD + q * NT + 64 * w);
        }
    };

    f32x4 aQ[MI], aW[MI], aK[MI], aP[2], aT[2];
#pragma unroll
    for (int m = 0; m < MI; ++m) aQ[m] = aW[m] = aK[m] = zero4();
    aP[0] = aP[1] = aT[0] = aT[1] = zero4();
    float dbp = 0.f;
    // dgam: TPR threads per key-channel row, UPT units of the slice each
    f32x4 dgm = zero4();
    constexpr int TPR = NT / DK, UPT = UW / TPR;
    const int grow = tid / TPR, gu0 = (tid % TPR) * UPT;

    fetch(0);
    for (int sl = 0; sl < NSL; ++sl) {
        const int v0 = sl * BW;
        wait_vmcnt<0>();
        __syncthreads();
        if (nvalid < C) {  // zero dO and v past the sequence end (its last chunk only)
            for (int idx = tid; idx < (C - nvalid) * UW; idx += NT) {
                const int row = nvalid + idx / UW, u = idx % UW;
                sdO[row * UW + u] = zero4();
                sv[row * UW + u] = zero4();
            }
            __syncthreads();
        }
        // phase 1: dX_V^T for column tiles jh, jh + 2 (acc[r] at column
        // jt*16 + 4 lq + r of the slice, token tr)
#pragma unroll
        for (int jm = 0; jm < 2; ++jm) {
            const int jt = jh + 2 * jm;
            f32x4 dx = zero4();
            // T lower triangular: T[s][t] = 0 for s < t
            for (int kb = ti; kb < C / 16; ++kb)
                dx = mma_f32_k16(ffrag_cols<SF>(sdD, 16 * kb, jt * 16), ffrag_cols<SF>(sT, 16 * kb, ti * 16), dx);
            const f32x4 vv = sv[swz_slot<SF>(tr, jt * 4 + lq)];
#pragma unroll
            for (int r = 0; r < 4; ++r) dbp += dx[r] * vv[r];
            if (tr < nvalid) {
                f32x4 o;
#pragma unroll
                for (int r = 0; r < 4; ++r) o[r] = btr * dx[r];
                *reinterpret_cast<f32x4*>(dvo + (tok0 + (size_t)tr * H) * DV + v0 + jt * 16 + 4 * lq) = o;
            }
        }
        // dgam partial: sum over this thread's units of its row of dS o S
#pragma unroll
        for (int u = 0; u < UPT; ++u) {
            const f32x4 a = sS[swz_slot<SF>(grow, gu0 + u)], c = sdS[swz_slot<SF>(grow, gu0 + u)];
#pragma unroll
            for (int r = 0; r < 4; ++r) dgm[r] += a[r] * c[r];
        }
        __syncthreads();
        // phase 2: the contractions over the slice's Dv columns
#pragma unroll 1
        for (int kb = 0; kb < UW / 4; ++kb) {
            const int u0 = 4 * kb;
            const f32x4 bO = ffrag_rows<SF>(sdO, ti * 16, u0), bD = ffrag_rows<SF>(sdD, ti * 16, u0),
                        bX = ffrag_rows<SF>(sD, ti * 16, u0);
#pragma unroll
            for (int m = 0; m < MI; ++m) {
                const int i0 = (ih * MI + m) * 16;
                const f32x4 aS = ffrag_rows<SF>(sS, i0, u0), adS = ffrag_rows<SF>(sdS, i0, u0);
                aQ[m] = mma_f32_k16(aS, bO, aQ[m]);
                aW[m] = mma_f32_k16(aS, bD, aW[m]);
                aK[m] = mma_f32_k16(adS, bX, aK[m]);
            }
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int s0 = sh * 32 + 16 * m;
                aP[m] = mma_f32_k16(ffrag_rows<SF>(sD, s0, u0), bO, aP[m]);
                aT[m] = mma_f32_k16(ffrag_rows<SF>(sv, s0, u0), bD, aT[m]);
            }
        }
        if (sl + 1 < NSL) {
            __syncthreads();
            fetch(v0 + BW);
        }
    }

    // outputs: lane values are 16-byte pieces of row tr
    {
        const size_t rk = ((size_t)ch * C + tr) * DK + 4 * lq;
#pragma unroll
        for (int m = 0; m < MI; ++m) {
            const int i0 = (ih * MI + m) * 16;
            *reinterpret_cast<f32x4*>(dQgo + rk + i0) = aQ[m];
            *reinterpret_cast<f32x4*>(dWgo + rk + i0) = -aW[m];
            *reinterpret_cast<f32x4*>(dKho + rk + i0) = aK[m];
        }
        const size_t rc = ((size_t)ch * C + tr) * C + 4 * lq;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int s0 = sh * 32 + 16 * m;
            // dT1 = dD (beta v)^T: beta of the key rows s0 + 4 lq + r
            f32x4 bk;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int sr = s0 + 4 * lq + r;
                bk[r] = sr < nvalid ? beta[tok0 + (size_t)sr * H] : 0.f;
            }
            *reinterpret_cast<f32x4*>(dPso + rc + s0) = aP[m];
            *reinterpret_cast<f32x4*>(dT1o + rc + s0) = aT[m] * bk;
        }
    }
    // dgam: the TPR threads of a row are neighbouring lanes
    {
        float sgm = dgm[0] + dgm[1] + dgm[2] + dgm[3];
#pragma unroll
        for (int o = 1; o < TPR; o <<= 1) sgm += __shfl_xor(sgm, o);
        if (tid % TPR == 0) dgmo[(size_t)ch * DK + grow] = sgm;
    }
    // dbeta through U: the four lane groups, then the two waves of a token tile
    dbp += __shfl_xor(dbp, 16);
    dbp += __shfl_xor(dbp, 32);
    if (lq == 0) sred[jh][tr] = dbp;
    __syncthreads();
    if (tid < C) dbpo[(size_t)ch * C + tid] = sred[0][tid] + sred[1][tid];
}

// ---------------------------------------------------------------------------
// bchunk1 over bf16 tables (bf16 inputs): 8 waves, Dv streamed in 32-column
// tiles with the next tile prefetched into registers; D comes from the forward
// (saved by the scan); the five contractions over Dv are single K = 32 bf16
// MFMAs on K-contiguous LDS tiles; dgam is summed from the states as they are
// loaded; dX_V = T^T dD stays in fp32.  Persistent, one workgroup per CU (the
// LDS allows no second): each workgroup takes every gridDim.x-th chunk-head and
// loads the next one's first tile, T, beta and W while it computes the WY
// adjoint of the keys of the current one.
// ---------------------------------------------------------------------------
constexpr int NTHR_C = 512;

template <int C, int DK, int DV>
__global__ void __launch_bounds__(NTHR_C)
bchunk1b_kernel(const bf16* __restrict__ v, const float* __restrict__ beta,
                const bf16* __restrict__ dO, const bf16* __restrict__ Dst,
                const float* __restrict__ Tmi,
                const bf16* __restrict__ Wbi, const bf16* __restrict__ Sst,
                const bf16* __restrict__ dSt, const bf16* __restrict__ dDt,
                bf16* __restrict__ dvo, float* __restrict__ dQgo, float* __restrict__ dWgo,
                float* __restrict__ dKho, float* __restrict__ dPso, float* __restrict__ dT1o,
                float* __restrict__ dgmo, float* __restrict__ dbpo, int T, int H, int NC, int nch)
{
    constexpr int BW = 32, NW = NTHR_C / 64, NB = C / 16;
    constexpr int PF = BW + 4;
    static_assert(BW == 4 * 8 && C == 8 * 8 && (DK == 128 || DK == 64), "table row widths of the swizzles");
    using SwK = std::conditional_t<DK == 128, SwzU16, SwzU8>;  // [C][DK] tables
    constexpr int T3 = NB * (DK / 16), M3 = (T3 + NW - 1) / NW;
    constexpr int T2 = NB * NB, M2 = (T2 + NW - 1) / NW;
    constexpr int TD = NB * (BW / 16), MD = (TD + NW - 1) / NW;
    constexpr int SWE = DK * BW / NTHR_C;            // bf16 of an S (dS) tile per thread: 8 or 4
    constexpr int SPR = BW / SWE;                    // threads per S row
    using SWord = std::conditional_t<SWE == 8, uint4, uint2>;
    static_assert(SWE * NTHR_C == DK * BW && (SWE == 8 || SWE == 4), "one S word and one dS word per thread");
    constexpr int NB8 = C * BW / 8;                  // uint4 words of a bf16 [C][BW] tile
    static_assert(NB8 == NTHR_C / 2, "two [C][BW] words per thread");
    // Dv-streaming tiles, and after the Dv loop the key WY-adjoint tables, share
    // sbuf.  bf16 tables are swizzled rows (swz.h): the [rows][BW] tiles SwzU4,
    // dW^T [DK][C] SwzU8w, W and dX_K [C][DK] SwK; T [C][C] (SwzU8) is read
    // transposed by transposing loads, and so is dD for dX_V = T^T dD.
    constexpr int R4 = BW * 2;  // bytes of a [rows][BW] bf16 row
    constexpr int O_dS = DK * R4, O_dO = 2 * DK * R4, O_D = O_dO + C * R4;
    constexpr int O_dD = O_D + C * R4, O_U = O_dD + C * R4, O_dX = O_U + C * R4;
    constexpr int O_v = O_dX + C * R4, STREAM = O_v + C * PF * 4;
    constexpr int O_W = DK * C * 2;
    constexpr int O_Xh = O_W + C * DK * 2, O_Xl = O_Xh + C * DK * 2, ENDP = O_Xl + C * DK * 2;
    // the tail's M diag(beta) parts (2 x C x C bf16): in the dv staging bytes
    // when they fit there (Dv = 128), else after the tail's tables
    constexpr bool M_IN_DV = 2 * C * C * 2 <= C * (DV + 8) * 2;
    constexpr int ENDM = M_IN_DV ? ENDP : ENDP + 2 * C * C * 2;
    __shared__ __align__(16) char sbuf[cmax(STREAM, ENDM)];
    // T as high + low bf16 parts (16 significant bits), for dX_V = T^T dD in the
    // Dv loop and dX_K = T^T dW after it; built once from the loaded T
    __shared__ __align__(16) uint4 sTh[C * C / 8], sTl[C * C / 8];
    __shared__ __align__(16) bf16 sDV[C][DV + 8];  // dv, written out after the Dv loop
    // dA of the previous chunk-head, staged from its accumulator tiles (32-bit
    // words of column pairs) until its rows are stored whole, 16 bytes a thread
    __shared__ __align__(16) bf16 sdA[C][C + 8];
    static_assert(C * C / 8 == NTHR_C, "one 16-byte dA word per thread");
    __shared__ float sbeta[C], sred[BW / 16][C];
    char* const sS = sbuf;
    char* const sdS = sbuf + O_dS;
    char* const sdO = sbuf + O_dO;
    char* const sD = sbuf + O_D;
    char* const sdD = sbuf + O_dD;
    char* const sV = sbuf + O_U;    // v and dX_V tiles, for
    char* const sdX = sbuf + O_dX;  // M = dX_V V^T
    float (*sv)[PF] = reinterpret_cast<float (*)[PF]>(sbuf + O_v);
    char* const sdWT = sbuf;  // dW^T
    char* const sW = sbuf + O_W;
    char* const sXh = sbuf + O_Xh;  // dX_K, high part
    char* const sXl = sbuf + O_Xl;  // dX_K, low part
    // 8 bf16 at column c of row r of a [rows][BW] tile
    auto at8 = [](char* t, int r, int c) { return reinterpret_cast<uint4*>(swz_at<SwzU4>(t, r, c)); };

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int lr = l & 15, lq = l >> 4;
    if ((int)blockIdx.x >= nch) return;  // whole workgroup
    // chunk-head ch -> its valid rows and first token
    auto geo = [&](int c, int& nv, size_t& tk) {
        const int n = c % NC, bh = c / NC, h = bh % H, b = bh / H;
        nv = min(C, T - n * C);
        tk = ((size_t)b * T + (size_t)n * C) * H + h;
    };
    // the chunk the prefetch reads (the current one inside the Dv loop, the
    // next one of this workgroup during the current one's WY-adjoint tail)
    const bf16 *Sp, *dSp, *dDp, *Dp;  // bf16 chunk-start states, chunk-end state gradients, delta gradients, D
    size_t tokr;  // this thread's token row of dO and v
    int nvalid;   // of the chunk being computed
    size_t tok0;
    bool row8;

    // Prefetch of one Dv tile, branch-free (a load under a divergent branch makes
    // the compiler wait for it where the branches join): every thread loads one
    // S word and one dS word (the same elements), and two 16-byte words of the
    // [C][BW] tiles: threads < NB8 a D word and a v word, the others a dO word
    // and a dD word; rows past the end are clamped on load and zeroed in stash().
    SWord pS, pdS;
    uint4 pa, pb;
    const bool lowh = tid < NB8;
    const int e8 = lowh ? tid : tid - NB8;
    const int r8 = e8 / (BW / 8), j8 = (e8 % (BW / 8)) * 8;
    const int rs = tid / SPR, js = (tid % SPR) * SWE;  // S (dS) row and first column of this thread
    auto fetch_from = [&](int c) {
        int nv;
        size_t tk;
        geo(c, nv, tk);
        // the saved bf16 arrays are in 32-column slices (slice32): a Dv tile
        // is one contiguous [rows][32] block at slice v0 / 32
        Sp = Sst + (size_t)c * DK * DV;
        dSp = dSt + (size_t)c * DK * DV;
        dDp = dDt + (size_t)c * C * DV;
        Dp = Dst + (size_t)c * C * DV;
        tokr = (tk + (size_t)min(r8, nv - 1) * H) * DV;
        return tk + (size_t)min(tid % C, nv - 1) * H;  // this thread's beta token
    };
    auto fetch = [&](int v0) {
        pS = *reinterpret_cast<const SWord*>(Sp + v0 * DK + rs * BW + js);
        pdS = *reinterpret_cast<const SWord*>(dSp + v0 * DK + rs * BW + js);
        const bf16* src = lowh ? Dp + v0 * C + r8 * BW + j8 : dO + tokr + v0 + j8;
        pa = *reinterpret_cast<const uint4*>(src);
        const bf16* srcb = lowh ? v + tokr + v0 + j8 : dDp + v0 * C + r8 * BW + j8;
        pb = *reinterpret_cast<const uint4*>(srcb);
    };
    float dgm_part = 0.f;
    auto stash = [&]() {
        // keep the use of the prefetched words here: hoisted into the compute
        // phase they would make it wait for the prefetch
        __builtin_amdgcn_sched_barrier(0);
        {
            constexpr int NWD = SWE / 2;  // 32-bit words of a thread's S word
            const uint32_t* sw = reinterpret_cast<const uint32_t*>(&pS);
            const uint32_t* dw = reinterpret_cast<const uint32_t*>(&pdS);
#pragma unroll
            for (int z = 0; z < NWD; ++z)
                dgm_part += __uint_as_float(sw[z] << 16) * __uint_as_float(dw[z] << 16) +
                            __uint_as_float(sw[z] & 0xFFFF0000u) * __uint_as_float(dw[z] & 0xFFFF0000u);
            *reinterpret_cast<SWord*>(swz_at<SwzU4>(sS, rs, js)) = pS;
            *reinterpret_cast<SWord*>(swz_at<SwzU4>(sdS, rs, js)) = pdS;
        }
        if (lowh) {
            *at8(sD, r8, j8) = pa;
            const uint4 vb = row8 ? pb : uint4{0u, 0u, 0u, 0u};
            *at8(sV, r8, j8) = vb;
            const uint32_t u[4] = {vb.x, vb.y, vb.z, vb.w};
            float vv[8];
#pragma unroll
            for (int z = 0; z < 4; ++z) {
                vv[2 * z] = __uint_as_float(u[z] << 16);
                vv[2 * z + 1] = __uint_as_float(u[z] & 0xFFFF0000u);
            }
            st4(&sv[r8][j8], float4{vv[0], vv[1], vv[2], vv[3]});
            st4(&sv[r8][j8 + 4], float4{vv[4], vv[5], vv[6], vv[7]});
        } else {
            *at8(sdO, r8, j8) = row8 ? pa : uint4{0u, 0u, 0u, 0u};
            *at8(sdD, r8, j8) = pb;
        }
    };

    // prologue loads of a chunk: its first Dv tile, T, beta and W (W is used
    // after the Dv loop); issued for the first chunk here and for each next one
    // during the tail of the one before, so the tail hides their latency
    constexpr int NT4 = (C * C / 4 + NTHR_C - 1) / NTHR_C;
    constexpr int NK8 = (C * DK / 8 + NTHR_C - 1) / NTHR_C;
    float4 tv[NT4];
    float bv0;
    u32x4 wv[NK8];  // W rows (bf16) for the keys' WY adjoint after the Dv loop
    auto prologue_loads = [&](int c) {
        const size_t tb = fetch_from(c);
        fetch(0);
        const float* Tp = Tmi + (size_t)c * C * C;
#pragma unroll
        for (int u = 0; u < NT4; ++u) tv[u] = load4<float>(Tp + 4 * min(tid + NTHR_C * u, C * C / 4 - 1));
        bv0 = beta[tb];
        const bf16* Wp = Wbi + (size_t)c * C * DK;
#pragma unroll
        for (int u = 0; u < NK8; ++u)
            wv[u] = *reinterpret_cast<const u32x4*>(Wp + 8 * min(tid + NTHR_C * u, C * DK / 8 - 1));
    };
    prologue_loads(blockIdx.x);

    // the WY-adjoint tail's outputs of the previous chunk (chunk-head pch),
    // held in registers and stored after the next chunk's prologue: a global
    // store issued after the prefetch would be waited for with it (the memory
    // counter completes in issue order)
    constexpr int NX8 = (C * DK / 8 + NTHR_C - 1) / NTHR_C;
    u32x4 oX[NX8];
    float oG, oB;
    int pch = -1;
    auto put_tail = [&]() {
        bf16* dXp = reinterpret_cast<bf16*>(dWgo) + (size_t)pch * C * DK;
#pragma unroll
        for (int u = 0; u < NX8; ++u) {
            const int idx = tid + NTHR_C * u;
            if (idx < C * DK / 8) *reinterpret_cast<u32x4*>(dXp + idx * 8) = oX[u];
        }
        bf16* dAp = reinterpret_cast<bf16*>(dT1o) + (size_t)pch * C * C;
        {
            const int r = tid / (C / 8), c8 = (tid % (C / 8)) * 8;
            *reinterpret_cast<uint4*>(&dAp[r * C + c8]) = *reinterpret_cast<const uint4*>(&sdA[r][c8]);
        }
        if (tid % SPR == 0) dgmo[(size_t)pch * DK + rs] = oG;
        if (tid < C) dbpo[(size_t)pch * C + tid] = oB;
    };

    // persistent: this workgroup takes chunk-heads blockIdx.x, + gridDim.x, ...
    for (int ch = blockIdx.x;;) {
        geo(ch, nvalid, tok0);
        row8 = r8 < nvalid;
        dgm_part = 0.f;
        f32x4 aQ[M3], aW[M3], aK[M3], aP[M2], aT[M2];
#pragma unroll
        for (int m = 0; m < M3; ++m) aQ[m] = aW[m] = aK[m] = zero4();
#pragma unroll
        for (int m = 0; m < M2; ++m) aP[m] = aT[m] = zero4();
        float dbr[MD][4];
#pragma unroll
        for (int m = 0; m < MD; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) dbr[m][r] = 0.f;

        // T (high and low parts) and beta into LDS, the first tile stashed
#pragma unroll
        for (int u = 0; u < NT4; ++u) {  // T[r][c0 .. c0 + 3]
            const int idx = tid + NTHR_C * u;
            if (idx < C * C / 4) {
                const int r = idx / (C / 4), c0 = (idx % (C / 4)) * 4;
                const float tt[4] = {tv[u].x, tv[u].y, tv[u].z, tv[u].w};
                float hi[4], lo[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    hi[e] = to_f32(f32_to_bf16(tt[e]));
                    lo[e] = tt[e] - hi[e];
                }
                *reinterpret_cast<uint2*>(swz_at<SwzU8>(sTh, r, c0)) = pack4_bf16(hi[0], hi[1], hi[2], hi[3]);
                *reinterpret_cast<uint2*>(swz_at<SwzU8>(sTl, r, c0)) = pack4_bf16(lo[0], lo[1], lo[2], lo[3]);
            }
        }
        if (tid < C) sbeta[tid] = tid < nvalid ? bv0 : 0.f;
        stash();
        __syncthreads();
        if (pch >= 0) put_tail();  // the previous chunk's, now that the prefetch is used
        // one Dv tile; the last one is peeled (MORE = false) so that the prefetch and
        // its stash need no run-time guard: with one, the compiler cannot match the
        // two and waits for every outstanding load and store at the top of the loop
        auto tile = [&](int v0, auto more_c) {
            constexpr bool MORE = decltype(more_c)::value;
            if constexpr (MORE) fetch(v0 + BW);
            // dX_V = T^T dD (dD bf16, T as high + low bf16 parts, fp32
            // accumulation; T^T and dD read with K down their rows): dv = beta
            // dX_V, and <dX_V, v> for dbeta
#pragma unroll
            for (int m = 0; m < MD; ++m) {
                const int idx = w + NW * m;
                if (idx < TD) {
                    const int ti = idx / (BW / 16), tj = idx % (BW / 16);
                    f32x4 dx = zero4();
#pragma unroll 1  // one K block's fragments live at a time (the kernel sits at the VGPR limit)
                    for (int k0 = 0; k0 < C; k0 += 32) {
                        const bf16x8 bd = frag_cols<SwzU4>(sdD, k0, tj * 16);
                        dx = mfma_bf16_16x16x32(frag_cols<SwzU8>(sTh, k0, ti * 16), bd, dx);
                        dx = mfma_bf16_16x16x32(frag_cols<SwzU8>(sTl, k0, ti * 16), bd, dx);
                    }
                    f32x4 bdx;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = ti * 16 + 4 * lq + r, j = tj * 16 + lr;
                        bdx[r] = sbeta[i] * dx[r];
                        dbr[m][r] += dx[r] * sv[i][j];
                    }
                    // dv and dX_V as 32-bit words of column pairs
                    const uint2 wv2 = acc_colpairs(bdx), wx2 = acc_colpairs(dx);
                    const int i2 = ti * 16 + 4 * lq + 2 * (lr & 1), j2 = tj * 16 + (lr & ~1);
                    *reinterpret_cast<uint32_t*>(&sDV[i2][v0 + j2]) = wv2.x;
                    *reinterpret_cast<uint32_t*>(&sDV[i2 + 1][v0 + j2]) = wv2.y;
                    *reinterpret_cast<uint32_t*>(swz_at<SwzU4>(sdX, i2, j2)) = wx2.x;
                    *reinterpret_cast<uint32_t*>(swz_at<SwzU4>(sdX, i2 + 1, j2)) = wx2.y;
                }
            }
#pragma unroll
            for (int m = 0; m < M3; ++m) {
                const int idx = w + NW * m;
                if (idx < T3) {
                    const int ti = idx / (DK / 16), tj = idx % (DK / 16);
                    const bf16x8 bs = frag_rows<SwzU4>(sS, tj * 16, 0);
                    aQ[m] = mfma_bf16_16x16x32(frag_rows<SwzU4>(sdO, ti * 16, 0), bs, aQ[m]);
                    aW[m] = mfma_bf16_16x16x32(frag_rows<SwzU4>(sdD, ti * 16, 0), bs, aW[m]);
                    aK[m] = mfma_bf16_16x16x32(frag_rows<SwzU4>(sD, ti * 16, 0), frag_rows<SwzU4>(sdS, tj * 16, 0), aK[m]);
                }
            }
#pragma unroll
            for (int m = 0; m < M2; ++m) {
                const int idx = w + NW * m;
                if (idx < T2) {
                    const int ti = idx / NB, tj = idx % NB;
                    aP[m] = mfma_bf16_16x16x32(frag_rows<SwzU4>(sdO, ti * 16, 0), frag_rows<SwzU4>(sD, tj * 16, 0), aP[m]);
                }
            }
            __syncthreads();  // the dX_V tile is complete
#pragma unroll
            for (int m = 0; m < M2; ++m) {
                const int idx = w + NW * m;
                if (idx < T2) {
                    const int ti = idx / NB, tj = idx % NB;
                    aT[m] = mfma_bf16_16x16x32(frag_rows<SwzU4>(sdX, ti * 16, 0), frag_rows<SwzU4>(sV, tj * 16, 0), aT[m]);
                }
            }
            __syncthreads();
            if constexpr (MORE) {
                stash();
                __syncthreads();
            }
        };
        for (int v0 = 0; v0 + BW < DV; v0 += BW) tile(v0, std::true_type{});
        tile(DV - BW, std::false_type{});

        // dv out: the loop stores nothing to global memory (a store there would be
        // waited for with the next prefetch)
        for (int idx = tid; idx < C * DV / 8; idx += NTHR_C) {
            const int r = idx / (DV / 8), c0 = (idx % (DV / 8)) * 8;
            if (r < nvalid)
                *reinterpret_cast<uint4*>(dvo + (tok0 + (size_t)r * H) * DV + c0) =
                    *reinterpret_cast<const uint4*>(&sDV[r][c0]);
        }
        // outputs (bf16: the consumer reads them as gradients of bf16-rounded products)
        bf16* dQp = reinterpret_cast<bf16*>(dQgo) + (size_t)ch * C * DK;
        bf16* dKp = reinterpret_cast<bf16*>(dKho) + (size_t)ch * C * DK;
#pragma unroll
        for (int m = 0; m < M3; ++m) {
            const int idx = w + NW * m;
            if (idx < T3) {
                const int ti = idx / (DK / 16), tj = idx % (DK / 16);
                {
                    const uint2 wq = acc_colpairs(aQ[m]), wk = acc_colpairs(aK[m]);
                    const int i2 = ti * 16 + 4 * lq + 2 * (lr & 1), j2 = tj * 16 + (lr & ~1);
                    *reinterpret_cast<uint32_t*>(&dQp[i2 * DK + j2]) = wq.x;
                    *reinterpret_cast<uint32_t*>(&dQp[(i2 + 1) * DK + j2]) = wq.y;
                    *reinterpret_cast<uint32_t*>(&dKp[i2 * DK + j2]) = wk.x;
                    *reinterpret_cast<uint32_t*>(&dKp[(i2 + 1) * DK + j2]) = wk.y;
                }
                // dW = -aW, stored transposed for dX_K = T^T dW (4 consecutive rows per lane)
                *reinterpret_cast<uint2*>(swz_at<SwzU8w>(sdWT, tj * 16 + lr, ti * 16 + 4 * lq)) =
                    pack4_bf16(-aW[m][0], -aW[m][1], -aW[m][2], -aW[m][3]);
            }
        }
        bf16* dPp = reinterpret_cast<bf16*>(dPso) + (size_t)ch * C * C;
#pragma unroll
        for (int m = 0; m < M2; ++m) {
            const int idx = w + NW * m;
            if (idx < T2) {
                const int ti = idx / NB, tj = idx % NB;
                const uint2 wp = acc_colpairs(aP[m]);
                const int i2 = ti * 16 + 4 * lq + 2 * (lr & 1), j2 = tj * 16 + (lr & ~1);
                *reinterpret_cast<uint32_t*>(&dPp[i2 * C + j2]) = wp.x;
                *reinterpret_cast<uint32_t*>(&dPp[(i2 + 1) * C + j2]) = wp.y;
            }
        }

        // ---- WY adjoint of the keys (W = T X_K):  dX_K = T^T dW and
        //   dA = -T^T (dU X_V^T + dW X_K^T) T^T = -(dX_V U^T + dX_K W^T) = -(G1 + dX_K W^T),
        // with G1 = dX_V U^T = M diag(beta) T^T (U = T diag(beta) V, M = dX_V V^T
        // from the Dv loop): U is not read, and with clip the product is the
        // unclipped one by construction.  bf16 MFMA with T, M diag(beta) and dX_K
        // as high + low bf16 parts (16 significant bits).
#pragma unroll
        for (int u = 0; u < NK8; ++u) {
            const int idx = tid + NTHR_C * u;
            if (idx < C * DK / 8) *reinterpret_cast<u32x4*>(swz_at<SwK>(sW, idx / (DK / 8), (idx % (DK / 8)) * 8)) = wv[u];
        }
        __syncthreads();
        // the next chunk's prologue loads, in flight through the tail (the last
        // workgroup's final chunk repeats itself: loads stay unconditional)
        prologue_loads((int)min((long long)ch + gridDim.x, (long long)nch - 1));
        // M diag(beta) (rows i, columns k) as high + low parts (the dv staging
        // was written out before the barrier above)
        char* const sMh = M_IN_DV ? reinterpret_cast<char*>(&sDV[0][0]) : sbuf + ENDP;
        char* const sMl = sMh + C * C * 2;
#pragma unroll
        for (int m = 0; m < M2; ++m) {
            const int idx = w + NW * m;
            if (idx < T2) {
                const int ti = idx / NB, tj = idx % NB;
                const float bk = sbeta[tj * 16 + lr];
                f32x4 hi, lo;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float x = aT[m][r] * bk;
                    hi[r] = to_f32(f32_to_bf16(x));
                    lo[r] = x - hi[r];
                }
                const uint2 wh = acc_colpairs(hi), wl = acc_colpairs(lo);
                const int i2 = ti * 16 + 4 * lq + 2 * (lr & 1), j2 = tj * 16 + (lr & ~1);
                *reinterpret_cast<uint32_t*>(swz_at<SwzU8>(sMh, i2, j2)) = wh.x;
                *reinterpret_cast<uint32_t*>(swz_at<SwzU8>(sMh, i2 + 1, j2)) = wh.y;
                *reinterpret_cast<uint32_t*>(swz_at<SwzU8>(sMl, i2, j2)) = wl.x;
                *reinterpret_cast<uint32_t*>(swz_at<SwzU8>(sMl, i2 + 1, j2)) = wl.y;
            }
        }
#pragma unroll
        for (int m = 0; m < M3; ++m) {
            const int idx = w + NW * m;
            if (idx < T3) {
                const int ti = idx / (DK / 16), tj = idx % (DK / 16);
                f32x4 acc = zero4();
#pragma unroll
                for (int k0 = 0; k0 < C; k0 += 32) {
                    const bf16x8 bw = frag_rows<SwzU8w>(sdWT, tj * 16, k0 / 8);
                    acc = mfma_bf16_16x16x32(frag_cols<SwzU8>(sTh, k0, ti * 16), bw, acc);
                    acc = mfma_bf16_16x16x32(frag_cols<SwzU8>(sTl, k0, ti * 16), bw, acc);
                }
                f32x4 hi, lo;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    hi[r] = to_f32(f32_to_bf16(acc[r]));
                    lo[r] = acc[r] - hi[r];
                }
                const uint2 wh = acc_colpairs(hi), wl = acc_colpairs(lo);
                const int i2 = ti * 16 + 4 * lq + 2 * (lr & 1), j2 = tj * 16 + (lr & ~1);
                *reinterpret_cast<uint32_t*>(swz_at<SwK>(sXh, i2, j2)) = wh.x;
                *reinterpret_cast<uint32_t*>(swz_at<SwK>(sXh, i2 + 1, j2)) = wh.y;
                *reinterpret_cast<uint32_t*>(swz_at<SwK>(sXl, i2, j2)) = wl.x;
                *reinterpret_cast<uint32_t*>(swz_at<SwK>(sXl, i2 + 1, j2)) = wl.y;
            }
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < NX8; ++u) {  // dX_K (bf16) rows, stored in place of dW
            const int idx = min(tid + NTHR_C * u, C * DK / 8 - 1);
            oX[u] = *reinterpret_cast<const u32x4*>(swz_at<SwK>(sXh, idx / (DK / 8), (idx % (DK / 8)) * 8));
        }
#pragma unroll
        for (int m = 0; m < M2; ++m) {
            const int idx = w + NW * m;
            if (idx < T2) {
                const int ti = idx / NB, tj = idx % NB;
                f32x4 acc = zero4();
                if (ti >= tj) {  // dA is strictly lower: tiles above the diagonal are zero
                    // G1 = (M diag(beta)) T^T; T is lower triangular, so the K block
                    // from k0 contributes only if k0 <= the tile's last row of T
#pragma unroll
                    for (int k0 = 0; k0 < C; k0 += 32) {
                        if (k0 <= tj * 16 + 15) {
                            const bf16x8 th = frag_rows<SwzU8>(sTh, tj * 16, k0 / 8);
                            const bf16x8 tl = frag_rows<SwzU8>(sTl, tj * 16, k0 / 8);
                            const bf16x8 mh = frag_rows<SwzU8>(sMh, ti * 16, k0 / 8);
                            acc = mfma_bf16_16x16x32(mh, th, acc);
                            acc = mfma_bf16_16x16x32(mh, tl, acc);
                            acc = mfma_bf16_16x16x32(frag_rows<SwzU8>(sMl, ti * 16, k0 / 8), th, acc);
                        }
                    }
#pragma unroll
                    for (int u0 = 0; u0 < DK / 8; u0 += 4) {
                        const bf16x8 bw = frag_rows<SwK>(sW, tj * 16, u0);
                        acc = mfma_bf16_16x16x32(frag_rows<SwK>(sXh, ti * 16, u0), bw, acc);
                        acc = mfma_bf16_16x16x32(frag_rows<SwK>(sXl, ti * 16, u0), bw, acc);
                    }
                }
                f32x4 da;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = ti * 16 + 4 * lq + r, j = tj * 16 + lr;
                    da[r] = i > j ? -acc[r] : 0.f;
                }
                const uint2 wa = acc_colpairs(da);
                const int i2 = ti * 16 + 4 * lq + 2 * (lr & 1), j2 = tj * 16 + (lr & ~1);
                *reinterpret_cast<uint32_t*>(&sdA[i2][j2]) = wa.x;
                *reinterpret_cast<uint32_t*>(&sdA[i2 + 1][j2]) = wa.y;
            }
        }
        // dgam: the SPR threads of one state row (aligned lanes) hold its partial sums
        static_assert(SPR == 4 || SPR == 8, "four or eight threads per state row");
        if constexpr (SPR == 4) oG = lane4_sum(dgm_part);
        else oG = lane8_sum(dgm_part);
        // dbeta part: row sums of dX_V o v over the 16 columns of each tile (one
        // slot per row and column tile, each written by the tile's wave), then
        // over the column tiles (fixed order)
#pragma unroll
        for (int m = 0; m < MD; ++m) {
            const int idx = w + NW * m;
            if (idx < TD) {
                const int ti = idx / (BW / 16), tj = idx % (BW / 16);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float sb = lane16_sum(dbr[m][r]);
                    if (lr == 0) sred[tj][ti * 16 + 4 * lq + r] = sb;
                }
            }
        }
        __syncthreads();
        static_assert(C <= NTHR_C, "one dbeta row per thread");
        oB = 0.f;
        if (tid < C)
            for (int jj = 0; jj < BW / 16; ++jj) oB += sred[jj][tid];
        pch = ch;
        if ((long long)ch + gridDim.x >= nch) break;
        ch += gridDim.x;
        __syncthreads();  // the tail's LDS reads are done before the next chunk's writes
    }
    put_tail();
}

// Score gradients, decay chain rule and outputs, shared by both bchunk2
// kernels: on entry sdP holds scale * dPs (lower incl. diagonal), sdA holds dA
// (strictly lower), and each column thread (channel c, rows p0 .. p0+RPP-1)
// holds a = exp(g), q, k and its partial dq, dk, dG (= dL/dG before the
// reverse cumsum) and dbeta terms; sX, sY, sZ are free [C][PD] fp32 tables.
template <typename TIn, int C, int DK, bool PCH, int MT, int NTH, int RPP, int PC, int PD>
__device__ __forceinline__ void score_grad_tail(
    float (&a)[RPP], float (&qv)[RPP], float (&kv)[RPP], float (&dq)[RPP], float (&dk)[RPP],
    float (&dG)[RPP], float (&dbr)[RPP], float (*sdP)[PC], float (*sdA)[PC], float (*sX)[PD],
    float (*sY)[PD], float (*sZ)[PD], const float* sbeta, float (*stot)[DK], float (*sext)[DK],
    bool cp, int c, int part, int p0, int nvalid, int ch, size_t tok0, size_t rsK, int H,
    const float* __restrict__ dbpi, TIn* __restrict__ dqo, TIn* __restrict__ dko,
    float* __restrict__ dgo, float* __restrict__ dbo)
{
    constexpr int NB = C / 16, NW = NTH / 64, NPART = C / RPP;
    const int tid = threadIdx.x, w = tid >> 6;
    // diagonal scores (E = 1): P_ii = q_i . k_i
    if (cp) {
#pragma unroll
        for (int i = 0; i < RPP; ++i) {
            const int r = p0 + i;
            const float dp = sdP[r][r];
            dq[i] += dp * kv[i];
            dk[i] += dp * qv[i];
        }
    }

    // ---- score gradients of pairs that span two 16-token tiles: the levels
    // h = C/2 .. 16 of the block-boundary split, as MFMA products of the score
    // gradients and factored rows (each own row is in the query half or the key
    // half of its 2h-block at every such level)
#pragma unroll
    for (int lvl = 0; (C >> (lvl + 1)) >= 16; ++lvl) {
        const int hl = C >> (lvl + 1);
        float F[RPP];
        // level-hl factor of each own row: query rows prod_{s=m+1..r} a_s,
        // key rows prod_{s=r+1..m} a_s, m the last token of the earlier half
        const int base = (p0 / (2 * hl)) * (2 * hl);
        const bool qs = p0 >= base + hl;
        if (qs) {
            float pre = 1.f;
            for (int pp = (base + hl) / RPP; pp < part; ++pp) pre *= stot[pp][c];
            float Fr = pre;
#pragma unroll
            for (int i = 0; i < RPP; ++i) {
                Fr *= a[i];
                F[i] = Fr;
            }
        } else {
            float suf = 1.f;
            for (int pp = part + 1; pp < (base + hl) / RPP; ++pp) suf *= stot[pp][c];
            float Fr = suf;
#pragma unroll
            for (int i = RPP - 1; i >= 0; --i) {
                F[i] = Fr;
                Fr *= a[i];
            }
        }
        if (cp) {
#pragma unroll
            for (int i = 0; i < RPP; ++i) {
                sX[p0 + i][c] = qv[i] * F[i];  // QK
                sY[p0 + i][c] = kv[i] * F[i];  // KK
            }
        }
        __syncthreads();
        // R1 = dP_h KK (query rows) + dP_h^T QK (key rows);
        // R2 = dA_h KK (query rows) + (diag(beta) dA_h)^T KK (key rows)
        constexpr int T3 = NB * (DK / 16), M3 = (T3 + NW - 1) / NW;
        f32x4 r2[M3];
#pragma unroll
        for (int m = 0; m < M3; ++m) {
            const int idx = w + NW * m;
            if (idx >= T3) continue;
            const int ti = idx / (DK / 16), tj = idx % (DK / 16);
            f32x4 r1 = zero4();
            r2[m] = zero4();
            const int tbase = (ti * 16 / (2 * hl)) * (2 * hl);
            if (ti * 16 >= tbase + hl) {
                r1 = mma16fd<MT>(r1, [&](int i, int kx) { return sdP[ti * 16 + i][tbase + kx]; },
                                 [&](int kx, int j) { return sY[tbase + kx][tj * 16 + j]; }, hl);
                r2[m] = mma16fd<MT>(r2[m], [&](int i, int kx) { return sdA[ti * 16 + i][tbase + kx]; },
                                    [&](int kx, int j) { return sY[tbase + kx][tj * 16 + j]; }, hl);
            } else {
                const int qb = tbase + hl;
                r1 = mma16fd<MT>(r1, [&](int i, int kx) { return sdP[qb + kx][ti * 16 + i]; },
                                 [&](int kx, int j) { return sX[qb + kx][tj * 16 + j]; }, hl);
                r2[m] = mma16fd<MT>(r2[m], [&](int i, int kx) { return sbeta[qb + kx] * sdA[qb + kx][ti * 16 + i]; },
                                    [&](int kx, int j) { return sY[qb + kx][tj * 16 + j]; }, hl);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) sZ[ti * 16 + acc_row(r)][tj * 16 + acc_col()] = r1[r];
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < M3; ++m) {
            const int idx = w + NW * m;
            if (idx >= T3) continue;
            const int ti = idx / (DK / 16), tj = idx % (DK / 16);
#pragma unroll
            for (int r = 0; r < 4; ++r) sX[ti * 16 + acc_row(r)][tj * 16 + acc_col()] = r2[m][r];
        }
        __syncthreads();
        if (cp) {
#pragma unroll
            for (int i = 0; i < RPP; ++i) {
                const int r = p0 + i;
                const float R1 = sZ[r][c], R2 = sX[r][c];
                if (qs) {
                    const float bt = sbeta[r];
                    dq[i] += F[i] * R1;
                    dk[i] += bt * F[i] * R2;
                    dG[i] += qv[i] * F[i] * R1 + bt * kv[i] * F[i] * R2;
                    dbr[i] += kv[i] * F[i] * R2;
                } else {
                    dk[i] += F[i] * (R1 + R2);
                    dG[i] -= kv[i] * F[i] * (R1 + R2);
                }
            }
        }
        __syncthreads();
    }

    // ---- score gradients of pairs inside one 16-token tile (j < i), on VALU:
    // this thread owns channel c of all 16 rows of its tile, so every pair's
    // contribution to its rows is local (no reduction across lanes); the decay
    // between the two tokens is the running product E_ij = prod_{s=j+1..i} a_s.
    // Per row i the sums over j are kept in two scalars and per column j one
    // sum over i; the decay gradient follows from them, since d/dG_i of
    // E_ij = +E_ij and d/dG_j = -E_ij: dG_i += q_i rq_i + beta_i k_i ra_i and
    // dG_j -= k_j cs_j (rq, ra: row sums of dP E k and dA E k; cs: column sums
    // of dP E q + dA E beta k).
    if (cp) {
        float cs[RPP];
#pragma unroll
        for (int j = 0; j < RPP; ++j) cs[j] = 0.f;
#pragma unroll
        for (int i = 1; i < RPP; ++i) {
            const int r = p0 + i;
            const float bi = sbeta[r], bki = bi * kv[i];
            float rq = 0.f, ra = 0.f, E = 1.f;
#pragma unroll
            for (int j = i - 1; j >= 0; --j) {
                E *= a[j + 1];
                const float tP = sdP[r][p0 + j] * E;
                const float tA = sdA[r][p0 + j] * E;
                rq += tP * kv[j];
                ra += tA * kv[j];
                cs[j] += tP * qv[i] + tA * bki;
            }
            dq[i] += rq;
            dk[i] += bi * ra;
            dG[i] += qv[i] * rq + bki * ra;
            dbr[i] += kv[i] * ra;
        }
#pragma unroll
        for (int j = 0; j < RPP; ++j) {
            dk[j] += cs[j];
            dG[j] -= kv[j] * cs[j];
        }
    }

    // ---- dg = reverse cumulative sum of dG over the chunk; dbeta; dq, dk out
    if (cp) {
        float s = 0.f;
#pragma unroll
        for (int i = RPP - 1; i >= 0; --i) {
            s += dG[i];
            dG[i] = s;
        }
        sext[part][c] = s;
    }
    __syncthreads();
    if (cp) {
        float add = 0.f;
        for (int pp = part + 1; pp < NPART; ++pp) add += sext[pp][c];
#pragma unroll
        for (int i = 0; i < RPP; ++i) {
            const int r = p0 + i;
            dG[i] += add;
            sZ[r][c] = dG[i];
            sX[r][c] = dbr[i];
            if (r < nvalid) {
                dqo[tok0 * DK + r * rsK + c] = from_f32<TIn>(dq[i]);
                dko[tok0 * DK + r * rsK + c] = from_f32<TIn>(dk[i]);
                if (PCH) dgo[(tok0 + (size_t)r * H) * DK + c] = dG[i];
            }
        }
    }
    __syncthreads();
    for (int r = tid; r < nvalid; r += NTH) {
        float sb = dbpi[(size_t)ch * C + r];
        for (int cc = 0; cc < DK; ++cc) sb += sX[r][cc];
        dbo[tok0 + (size_t)r * H] = sb;
        if (!PCH) {
            float sg = 0.f;
            for (int cc = 0; cc < DK; ++cc) sg += sZ[r][cc];
            dgo[tok0 + (size_t)r * H] = sg;
        }
    }
}

// ---------------------------------------------------------------------------
// bchunk2
// ---------------------------------------------------------------------------
constexpr int NTHR2 = 512;  // 8 waves

template <typename TIn, int C, int DK, int DV, bool PCH, int MT>
__global__ void __launch_bounds__(NTHR2)
bchunk2_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k, const float* __restrict__ g,
               const float* __restrict__ beta, const float* __restrict__ Tmi,
               const float* __restrict__ dQgi, const float* __restrict__ dWgi,
               const float* __restrict__ dKhi, const float* __restrict__ dPsi,
               const float* __restrict__ dT1i, const float* __restrict__ dgmi,
               const float* __restrict__ dbpi, TIn* __restrict__ dqo, TIn* __restrict__ dko,
               float* __restrict__ dgo, float* __restrict__ dbo, int T, int H, int NC, float scale,
               const float* __restrict__ rni)
{
    using G = Geo<C, DK, DV>;
    constexpr int PD = G::PD, PC = G::PC, NB = G::NB;
    constexpr int RPP = 16;         // rows per column-thread part: one 16-token tile
    constexpr int NPART = C / RPP;  // parts per chunk
    constexpr int NW = NTHR2 / 64;
    __shared__ float sT[C][PC], sdP[C][PC], sdA[C][PC], sX[C][PD], sY[C][PD], sZ[C][PD];
    __shared__ float sbeta[C], stot[NPART][DK], sext[NPART][DK];

    const int ch = blockIdx.x;
    const int n = ch % NC, bh = ch / NC, h = bh % H, b = bh / H;
    const int t0 = n * C;
    const int nvalid = min(C, T - t0);
    const int tid = threadIdx.x, w = tid >> 6;
    const size_t tok0 = ((size_t)b * T + t0) * H + h;
    const size_t rsK = (size_t)H * DK;

    // intermediate gradients from bchunk1 (fp32)
    static_assert(!bf16_tables<TIn, C, DK>(), "bf16 inputs at chunk 64 run bchunk2c");
    using IT = float;
    const IT* dQgI = dQgi;
    const IT* dWgI = dWgi;
    const IT* dKhI = dKhi;
    const IT* dPsI = dPsi;
    const IT* dT1I = dT1i;

    // column threads: channel c, rows [p0, p0 + RPP)
    const bool cp = tid < NPART * DK;
    const int c = tid % DK, part = cp ? tid / DK : 0, p0 = part * RPP;

    float a[RPP], qv[RPP], kv[RPP], Gm[RPP];
    float dq[RPP], dk[RPP], dG[RPP], dbr[RPP];
#pragma unroll
    for (int i = 0; i < RPP; ++i) {
        const int r = p0 + i;
        // rows past the end read the last valid row (every load unconditional,
        // so all rows are in flight at once) and are then replaced by g = q = k = 0
        const int rr = min(r, nvalid - 1);
        const float gx = PCH ? g[(tok0 + (size_t)rr * H) * DK + c] : g[tok0 + (size_t)rr * H];
        const float qx = to_f32(q[tok0 * DK + rr * rsK + c]);
        const float kx = to_f32(k[tok0 * DK + rr * rsK + c]);
        const bool ok = cp && r < nvalid;
        a[i] = ok ? gx : 0.f;  // log-decay for now; exponentiated once the other loads are out
        qv[i] = ok ? qx : 0.f;
        kv[i] = ok ? kx : 0.f;
        dq[i] = dk[i] = dG[i] = dbr[i] = 0.f;
    }
    if (rni) {  // use_qk_l2norm: the rows the forward used, r x (dq, dk are then d/dx_hat)
#pragma unroll
        for (int i = 0; i < RPP; ++i) {
            qv[i] *= rni[((size_t)ch * 2) * C + p0 + i];
            kv[i] *= rni[((size_t)ch * 2 + 1) * C + p0 + i];
        }
    }
    {
        // T, dW and beta: every load issued before the first LDS write
        constexpr int NT1 = (C * C + NTHR2 - 1) / NTHR2, NW4 = (C * DK / 4 + NTHR2 - 1) / NTHR2;
        const float* Tp = Tmi + (size_t)ch * C * C;
        const IT* dWp = dWgI + (size_t)ch * C * DK;
        float tv[NT1];
        float4 wv[NW4];
#pragma unroll
        for (int u = 0; u < NT1; ++u) tv[u] = Tp[min(tid + NTHR2 * u, C * C - 1)];
#pragma unroll
        for (int u = 0; u < NW4; ++u) {
            const int idx = min(tid + NTHR2 * u, C * DK / 4 - 1);
            wv[u] = load4<IT>(dWp + (idx / (DK / 4)) * DK + (idx % (DK / 4)) * 4);
        }
        const float bv = beta[tok0 + (size_t)min(tid % C, nvalid - 1) * H];
#pragma unroll
        for (int u = 0; u < NT1; ++u) {
            const int idx = tid + NTHR2 * u;
            if (idx < C * C) sT[idx / C][idx % C] = tv[u];
        }
#pragma unroll
        for (int u = 0; u < NW4; ++u) {
            const int idx = tid + NTHR2 * u;
            if (idx < C * DK / 4) st4(&sY[idx / (DK / 4)][(idx % (DK / 4)) * 4], wv[u]);
        }
        if (tid < C) sbeta[tid] = tid < nvalid ? bv : 0.f;
    }
#pragma unroll
    for (int i = 0; i < RPP; ++i) a[i] = expf(a[i]);
    {
        float pt = 1.f;
#pragma unroll
        for (int i = 0; i < RPP; ++i) pt *= a[i];
        if (cp) stot[part][c] = pt;
    }
    __syncthreads();

    // ---- Gamma, Kh factor, X_K; contributions of dQg, dKh, dgam
    if (cp) {
        const IT* dQp = dQgI + (size_t)ch * C * DK;
        const IT* dKp = dKhI + (size_t)ch * C * DK;
        float pre = 1.f, suf = 1.f;
        for (int pp = 0; pp < part; ++pp) pre *= stot[pp][c];
        for (int pp = part + 1; pp < NPART; ++pp) suf *= stot[pp][c];
        float Gr = pre;
#pragma unroll
        for (int i = 0; i < RPP; ++i) {
            Gr *= a[i];
            Gm[i] = Gr;
        }
        float kap = suf, sumKh = 0.f;
#pragma unroll
        for (int i = RPP - 1; i >= 0; --i) {
            const int r = p0 + i;
            const float dqg = to_f32(dQp[r * DK + c]), dkh = to_f32(dKp[r * DK + c]);
            dq[i] += scale * Gm[i] * dqg;
            dG[i] += scale * qv[i] * Gm[i] * dqg;
            const float khv = kv[i] * kap;
            dk[i] += kap * dkh;
            dG[i] -= khv * dkh;
            sumKh += khv * dkh;
            sX[r][c] = sbeta[r] * kv[i] * Gm[i];  // X_K
            kap *= a[i];
        }
        sext[part][c] = sumKh;
    }
    __syncthreads();
    if (cp && part == NPART - 1) {
        float s = 0.f;
        for (int pp = 0; pp < NPART; ++pp) s += sext[pp][c];
        dG[RPP - 1] += s + Gm[RPP - 1] * dgmi[(size_t)ch * DK + c];
    }

    // this wave's 16x16 tiles of the C x C gradients dT(U) and dPs, fetched
    // before the products below so that their latency overlaps them
    constexpr int MA = (NB * NB + NW - 1) / NW;
    float pT1[MA][4], pPs[MA][4];
    {
        const IT* dT1p = dT1I + (size_t)ch * C * C;
        const IT* dPp = dPsI + (size_t)ch * C * C;
#pragma unroll
        for (int m = 0; m < MA; ++m) {
            const int idx = w + NW * m;
            const int ti = (idx % (NB * NB)) / NB, tj = idx % NB;  // in range for every wave
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int e = (ti * 16 + acc_row(r)) * C + tj * 16 + acc_col();
                pT1[m][r] = to_f32(dT1p[e]);
                pPs[m][r] = to_f32(dPp[e]);
            }
        }
    }
    // ---- dX_K = T^T dW (-> sZ);  dT = dT(U) + dW X_K^T (-> sdA)
    {
        constexpr int T3 = NB * (DK / 16);
        for (int idx = w; idx < T3; idx += NW) {
            const int ti = idx / (DK / 16), tj = idx % (DK / 16);
            f32x4 acc = mma16k<MT_F32, C>(zero4(), &sT[0][ti * 16], 1, PC, &sY[0][tj * 16], PD, 1);
#pragma unroll
            for (int r = 0; r < 4; ++r) sZ[ti * 16 + acc_row(r)][tj * 16 + acc_col()] = acc[r];
        }
#pragma unroll
        for (int m = 0; m < MA; ++m) {
            const int idx = w + NW * m;
            if (idx < NB * NB) {
                const int ti = idx / NB, tj = idx % NB;
                f32x4 acc;
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] = pT1[m][r];
                acc = mma16k<MT_F32, DK>(acc, &sY[ti * 16][0], PD, 1, &sX[tj * 16][0], 1, PD);
#pragma unroll
                for (int r = 0; r < 4; ++r) sdA[ti * 16 + acc_row(r)][tj * 16 + acc_col()] = acc[r];
            }
        }
    }
    __syncthreads();
    // X_K contributions: dk += beta Gamma dX_K, dG += X_K o dX_K, dbeta += <k Gamma, dX_K>
    if (cp) {
#pragma unroll
        for (int i = 0; i < RPP; ++i) {
            const int r = p0 + i;
            const float dx = sZ[r][c];
            const float kg = kv[i] * Gm[i];
            dk[i] += sbeta[r] * Gm[i] * dx;
            dG[i] += sbeta[r] * kg * dx;
            dbr[i] += kg * dx;
        }
    }
    // Y = dT T^T (-> sdP as scratch)
    for (int idx = w; idx < NB * NB; idx += NW) {
        const int ti = idx / NB, tj = idx % NB;
        f32x4 acc = mma16k<MT_F32, C>(zero4(), &sdA[ti * 16][0], PC, 1, &sT[tj * 16][0], 1, PC);
#pragma unroll
        for (int r = 0; r < 4; ++r) sdP[ti * 16 + acc_row(r)][tj * 16 + acc_col()] = acc[r];
    }
    __syncthreads();
    // dA = -T^T Y, strictly lower
    f32x4 dAt[MA];
#pragma unroll
    for (int m = 0; m < MA; ++m) {
        const int idx = w + NW * m;
        if (idx < NB * NB) {
            const int ti = idx / NB, tj = idx % NB;
            dAt[m] = mma16k<MT_F32, C>(zero4(), &sT[0][ti * 16], 1, PC, &sdP[0][tj * 16], PC, 1);
        }
    }
    __syncthreads();
    {
#pragma unroll
        for (int m = 0; m < MA; ++m) {
            const int idx = w + NW * m;
            if (idx < NB * NB) {
                const int ti = idx / NB, tj = idx % NB;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = ti * 16 + acc_row(r), j = tj * 16 + acc_col();
                    sdA[i][j] = i > j ? -dAt[m][r] : 0.f;
                    sdP[i][j] = i >= j ? scale * pPs[m][r] : 0.f;
                }
            }
        }
    }
    __syncthreads();
    score_grad_tail<TIn, C, DK, PCH, MT, NTHR2, RPP, PC, PD>(
        a, qv, kv, dq, dk, dG, dbr, sdP, sdA, sX, sY, sZ, sbeta, stot, sext, cp, c, part, p0, nvalid,
        ch, tok0, rsK, H, dbpi, dqo, dko, dgo, dbo);
}

// ---------------------------------------------------------------------------
// bchunk2c: bf16 inputs at chunk 64, after bchunk1b has taken the WY adjoint
// (dX_K and dA).  One workgroup takes one chunk-head and half of its key
// channels: score gradients by the block-boundary split, the decay chain rule
// and the outputs dq, dk, dg of those channels.  A thread owns one channel of
// eight consecutive token rows (a part); < 80 KB of LDS and < 128 VGPRs let
// two workgroups (four waves per SIMD) share a CU.
// dbeta (and dg for per-head decay) are row sums over all channels: each half
// writes its partial sums and bchunk2_finish adds them in a fixed order.
// With L2N (use_qk_l2norm) q and k rows are scaled by the forward's r and
// dq, dk are written with respect to the normalised rows; l2norm_bwd maps
// them to the raw rows, which needs whole rows.
// ---------------------------------------------------------------------------
// threads of a bchunk2c workgroup: one per (8-row part, key channel of the half)
template <int C, int DK>
constexpr int bchunk2c_threads()
{
    return (C / 8) * (DK / 2);
}

// Channel-major bf16 tables of bchunk2c (a channel's C = 64 token rows as eight
// 16-byte slots of 8 rows): slot s of channel ch sits at ch * 8 + (s ^ (ch & 7)),
// so both the B fragments (16 channels, one or two slots) and the slot writes of
// a part (consecutive channels, one slot) meet no bank conflict under the
// measured LDS phase rules (swz.h).
__device__ __forceinline__ int ctab_slot(int ch, int s) { return ch * 8 + (s ^ (ch & 7)); }

// B fragment of a channel-major table: lane (r, kk) supplies 8-row slot
// slot0 + kk of channel ch0 + r; HALF (K = 16): lanes kk >= 2 supply zeros and
// the others slots slot0, slot0 + 1
template <bool HALF>
__device__ __forceinline__ bf16x8 ctab_frag(const uint4* __restrict__ tab, int ch0, int slot0)
{
    const int l = lane_id(), kk = l >> 4;
    const bf16x8 b = __builtin_bit_cast(bf16x8, tab[ctab_slot(ch0 + (l & 15), slot0 + (HALF ? kk & 1 : kk))]);
    return HALF && kk >= 2 ? bf16x8{} : b;
}

template <int C, int DK, bool PCH, bool L2N>
__global__ void __launch_bounds__((C / 8) * (DK / 2)) __attribute__((amdgpu_waves_per_eu(4)))  // bchunk2c_threads; 4 waves per SIMD: 2 workgroups a CU
bchunk2c_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k, const float* __restrict__ g,
                const float* __restrict__ beta, const bf16* __restrict__ dQgi,
                const bf16* __restrict__ dXKi, const bf16* __restrict__ dKhi,
                const bf16* __restrict__ dPsi, const bf16* __restrict__ dAi,
                const float* __restrict__ dgmi, bf16* __restrict__ dqo, bf16* __restrict__ dko,
                float* __restrict__ dgo, float* __restrict__ dbq, float* __restrict__ dgq, int T,
                int H, int NC, int nch, float scale, const float* __restrict__ rni)
{
    static_assert(C == 64, "bchunk2c: chunk 64");
    constexpr int HC = DK / 2;  // key channels per workgroup
    constexpr int NTHR_F = bchunk2c_threads<C, DK>();
    constexpr int NB = C / 16, NW = NTHR_F / 64;
    constexpr int RPP = 8, NPART = C / RPP;
    static_assert(NPART * HC == NTHR_F, "one column thread per (part, channel)");
    // LDS, one buffer with named parts:
    //  score gradients, bf16, by rows (SwzU8): dPs (unscaled, lower incl.
    //  diagonal) and dA (strictly lower); their transposes are read from the
    //  same tables with transposing loads;
    //  level tables (channel-major, ctab_slot): q and k rows times the level
    //  factor, and the k rows times beta as well (the key side of dA^T);
    //  level results (fp32 [rows][HC], ridx): query rows scale*R1, key rows
    //  scale*R1 + R2 (sR), query rows' R2 (sR2, C/2 rows).  Before the levels sR
    //  also holds the dKh row-sum partials.  Per-head decay uses, after its score
    //  products, the first three C x HC fp32 tables' worth of bytes for their
    //  results.
    static_assert(C == 8 * 8, "score rows and channel-major tables of eight 16-byte units");
    constexpr int TB = C * C * 2, O_QK = 2 * TB, O_KK = O_QK + HC * C * 2, O_KB = O_KK + HC * C * 2;
    // fp32 [rows][HC] tables, rows padded by four words: the accumulator-tile
    // writes (rows 4 apart) and the 4-lanes-a-row reads meet no bank conflicts
    constexpr int PH = HC + 4;
    constexpr int O_R = O_KB + HC * C * 2, O_R2 = O_R + C * PH * 4, LDSB = O_R2 + (C / 2) * PH * 4;
    static_assert(3 * C * PH * 4 <= O_R2, "per-head results fit below sR2 (sR is not live then)");
    __shared__ __align__(16) char sbuf[LDSB];
    uint4* sPv = reinterpret_cast<uint4*>(sbuf);        // dPs rows
    uint4* sAv = reinterpret_cast<uint4*>(sbuf + TB);   // dA rows
    uint4* sQK = reinterpret_cast<uint4*>(sbuf + O_QK);  // q rows (times a factor), by channel
    uint4* sKK = reinterpret_cast<uint4*>(sbuf + O_KK);  // k rows (times a factor), by channel
    uint4* sKB = reinterpret_cast<uint4*>(sbuf + O_KB);  // beta k rows (times a factor), by channel
    float* sR = reinterpret_cast<float*>(sbuf + O_R);
    float* sR2 = reinterpret_cast<float*>(sbuf + O_R2);
    auto ridx = [](int i, int j) { return i * PH + j; };
    // element (R, c) of a score table
    auto sel = [](const uint4* X, int R, int c) {
        return to_f32(reinterpret_cast<const bf16*>(X + swz_slot<SwzU8>(R, c >> 3))[c & 7]);
    };
    __shared__ float sbeta[C], stot[NPART][HC];
    __shared__ float sG[C];  // per-head decay: chunk-local inclusive cumsum of g
    float (*sext)[HC] = reinterpret_cast<float (*)[HC]>(sR);

    // block -> (chunk-head, half): the two halves of a chunk-head are 8 ids
    // apart, so they run on the same XCD and share its L2 for the C x C tables
    const int bid = blockIdx.x;
    const int half = (bid >> 3) & 1;
    const int ch = (bid >> 4) * 8 + (bid & 7);
    if (ch >= nch) return;  // whole workgroup: no barrier is skipped by part of it
    const int n = ch % NC, bh = ch / NC, h = bh % H, b = bh / H;
    const int t0 = n * C;
    const int nvalid = min(C, T - t0);
    const int tid = threadIdx.x, w = tid >> 6;
    // the wave index as a wave-uniform value: the MFMA tile loops' tile
    // choice and coordinates then live in scalar registers and branches
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const size_t tok0 = ((size_t)b * T + t0) * H + h;
    const size_t rsK = (size_t)H * DK;
    const bool cp = tid < NPART * HC;
    const int cl = tid % HC, part = cp ? tid / HC : 0, p0 = part * RPP;
    const int c = half * HC + cl;  // key channel

    float a[RPP], qv[RPP], kv[RPP], Gm[RPP];
    float dq[RPP], dk[RPP], dG[RPP], dbr[RPP];
    // token-row offsets from the chunk's first row: 32-bit (rsK * C < 2^31)
    const uint32_t rs32 = (uint32_t)rsK;
    const bf16* qb = q + tok0 * DK;
    const bf16* kb = k + tok0 * DK;
    const float* gb = PCH ? g + tok0 * DK : g + tok0;
#pragma unroll
    for (int i = 0; i < RPP; ++i) {
        const int r = p0 + i;
        // rows past the end read the last valid row (all loads unconditional)
        // and are then replaced by g = q = k = 0
        const uint32_t rr = (uint32_t)min(r, nvalid - 1);
        const uint32_t off = rr * rs32 + (uint32_t)c;
        const float gx = PCH ? ld32(gb, off) : ld32(gb, rr * (uint32_t)H);
        const float qx = to_f32(ld32(qb, off));
        const float kx = to_f32(ld32(kb, off));
        const bool ok = cp && r < nvalid;
        a[i] = ok ? gx : 0.f;  // log-decay until the table loads are out
        qv[i] = ok ? qx : 0.f;
        kv[i] = ok ? kx : 0.f;
        dq[i] = dk[i] = dG[i] = dbr[i] = 0.f;
    }
    // the bchunk1 hand-offs of this thread's rows, in the same round of loads
    // (two bf16 per word); used after the first barrier
    uint32_t hQ[RPP / 2], hK[RPP / 2], hX[RPP / 2];
    {
        const bf16* hQb = dQgi + (size_t)ch * C * DK;
        const bf16* hKb = dKhi + (size_t)ch * C * DK;
        const bf16* hXb = dXKi + (size_t)ch * C * DK;
#pragma unroll
        for (int i = 0; i < RPP; i += 2) {
            const uint32_t a0 = (uint32_t)((p0 + i) * DK + c), a1 = a0 + DK;
            hQ[i / 2] = (uint32_t)ld32(hQb, a0).bits | ((uint32_t)ld32(hQb, a1).bits << 16);
            hK[i / 2] = (uint32_t)ld32(hKb, a0).bits | ((uint32_t)ld32(hKb, a1).bits << 16);
            hX[i / 2] = (uint32_t)ld32(hXb, a0).bits | ((uint32_t)ld32(hXb, a1).bits << 16);
        }
    }
    auto hw = [](const uint32_t* h, int i) {
        return __uint_as_float((i & 1) ? (h[i / 2] & 0xFFFF0000u) : (h[i / 2] << 16));
    };
    float rq[L2N ? RPP : 1], rk[L2N ? RPP : 1];
    // per-head decay with L2N: all rows' r (q rows, then k rows) in the bytes
    // of sR2, which only the per-channel levels use
    float* sRn = reinterpret_cast<float*>(sbuf + O_R2);
    if constexpr (L2N) {
#pragma unroll
        for (int i = 0; i < RPP; ++i) {
            rq[i] = rni[((size_t)ch * 2) * C + p0 + i];
            rk[i] = rni[((size_t)ch * 2 + 1) * C + p0 + i];
        }
        if (!PCH && tid < 2 * C) sRn[tid] = rni[(size_t)ch * 2 * C + tid];
    }
    {
        // dPs and dA (C x C bf16): rows as they are, and transposed
        constexpr int NC8 = C * C / 8, NU = (NC8 + NTHR_F - 1) / NTHR_F;
        const bf16* Pp = dPsi + (size_t)ch * C * C;
        const bf16* Ap = dAi + (size_t)ch * C * C;
        uint4 pw[NU], aw[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int idx = min(tid + NTHR_F * u, NC8 - 1);
            pw[u] = *reinterpret_cast<const uint4*>(Pp + 8 * idx);
            aw[u] = *reinterpret_cast<const uint4*>(Ap + 8 * idx);
        }
        const float bv = beta[tok0 + (size_t)min(tid % C, nvalid - 1) * H];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int idx = tid + NTHR_F * u;
            if (idx < NC8) {
                const int i = idx / (C / 8), uu = idx % (C / 8);
                sPv[swz_slot<SwzU8>(i, uu)] = pw[u];
                sAv[swz_slot<SwzU8>(i, uu)] = aw[u];
            }
        }
        if (tid < C) sbeta[tid] = tid < nvalid ? bv : 0.f;
    }
    if constexpr (!PCH) {
        if (w == 0) {  // G_i = g_0 + ... + g_i, inclusive prefix sum across the wave (C = 64)
            float x = tid < nvalid ? g[tok0 + (size_t)min(tid, nvalid - 1) * H] : 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(x, off);
                if (tid >= off) x += y;
            }
            sG[tid] = x;
        }
    }
#pragma unroll
    for (int i = 0; i < RPP; ++i) a[i] = fast_exp(a[i]);
    if constexpr (L2N) {  // the rows the forward used
#pragma unroll
        for (int i = 0; i < RPP; ++i) {
            qv[i] *= rq[i];
            kv[i] *= rk[i];
        }
    }
    {
        float pt = 1.f;
#pragma unroll
        for (int i = 0; i < RPP; ++i) pt *= a[i];
        if (cp) stot[part][cl] = pt;
    }
    __syncthreads();

    // ---- Gamma, Kh factor; contributions of dQg, dKh; X_K = diag(beta) K o Gamma
    if (cp) {
        float pre = 1.f, suf = 1.f;
        for (int pp = 0; pp < part; ++pp) pre *= stot[pp][cl];
        for (int pp = part + 1; pp < NPART; ++pp) suf *= stot[pp][cl];
        float Gr = pre;
#pragma unroll
        for (int i = 0; i < RPP; ++i) {
            Gr *= a[i];
            Gm[i] = Gr;
        }
        float kap = suf, sumKh = 0.f;
#pragma unroll
        for (int i = RPP - 1; i >= 0; --i) {
            const int r = p0 + i;
            const float dqg = hw(hQ, i), dkh = hw(hK, i), dx = hw(hX, i);
            dq[i] += scale * Gm[i] * dqg;
            dG[i] += scale * qv[i] * Gm[i] * dqg;
            const float khv = kv[i] * kap;
            dk[i] += kap * dkh;
            dG[i] -= khv * dkh;
            sumKh += khv * dkh;
            kap *= a[i];
            // dk += beta Gamma dX_K, dG += X_K o dX_K, dbeta += <k Gamma, dX_K>
            const float kg = kv[i] * Gm[i], bt = sbeta[r];
            dk[i] += bt * Gm[i] * dx;
            dG[i] += bt * kg * dx;
            dbr[i] += kg * dx;
        }
        sext[part][cl] = sumKh;
    }
    __syncthreads();
    if (cp && part == NPART - 1) {
        float sacc = 0.f;
        for (int pp = 0; pp < NPART; ++pp) sacc += sext[pp][cl];
        dG[RPP - 1] += sacc + Gm[RPP - 1] * dgmi[(size_t)ch * DK + c];
    }
    if constexpr (!PCH) {
        // ---- Per-head decay: the decay between tokens j <= i is the scalar
        // E_ij = exp(G_i - G_j), the same for every channel, so with dP~ = dPs o E
        // and dA~ = dA o E all score gradients are three MFMA products per tile:
        //   X = scale dP~ K  (dq),   R = dA~ K  (query side of dk and dbeta),
        //   Y = scale dP~^T Q + (diag(beta) dA~)^T K  (key side of dk),
        // and dG = q o X + beta k o R - k o Y (the diagonal, E = 1, cancels in dG).
        // Scale the score tables by E in place; the transposed operands are read
        // from the same scaled values.  With L2N (x_hat = r x) the operand tables
        // hold the raw bf16 rows, and dP~ takes r_q(i) r_k(j), dA~ r_k(i) r_k(j);
        // the products X', R', Y' against raw rows then give X = X' / r_q(i),
        // R = R' / r_k(i), Y = Y' / r_k(j), and dG = q o X' + beta k o R' - k o Y'
        // with the raw q, k: the plain path's arithmetic, whose pairs (i, j)
        // cancel in dG's reverse sum because both sides read one rounded value.
        for (int e = tid; e < C * (C / 8); e += NTHR_F) {
            const int rr = e / (C / 8), uu = e % (C / 8), c0 = uu * 8;
            uint4* t1 = &sPv[swz_slot<SwzU8>(rr, uu)];
            uint4* t2 = &sAv[swz_slot<SwzU8>(rr, uu)];
            uint4 w1 = *t1, w2 = *t2;
            uint32_t u1[4] = {w1.x, w1.y, w1.z, w1.w}, u2[4] = {w2.x, w2.y, w2.z, w2.w};
            float ev[8];
            float ev2[8];
#pragma unroll
            for (int z = 0; z < 8; ++z) {
                const int i = rr, j = c0 + z;  // element (i, j) of the C x C matrix
                ev[z] = j <= i ? fast_exp(sG[i] - sG[j]) : 0.f;
                ev2[z] = ev[z];
                if constexpr (L2N) {
                    ev[z] *= sRn[i] * sRn[C + j];
                    ev2[z] *= sRn[C + i] * sRn[C + j];
                }
            }
#pragma unroll
            for (int z = 0; z < 4; ++z) {
                const float p0v = __uint_as_float(u1[z] << 16) * ev[2 * z], p1v = __uint_as_float(u1[z] & 0xFFFF0000u) * ev[2 * z + 1];
                const float a0v = __uint_as_float(u2[z] << 16) * ev2[2 * z], a1v = __uint_as_float(u2[z] & 0xFFFF0000u) * ev2[2 * z + 1];
                u1[z] = (uint32_t)f32_to_bf16(p0v).bits | ((uint32_t)f32_to_bf16(p1v).bits << 16);
                u2[z] = (uint32_t)f32_to_bf16(a0v).bits | ((uint32_t)f32_to_bf16(a1v).bits << 16);
            }
            *t1 = uint4{u1[0], u1[1], u1[2], u1[3]};
            *t2 = uint4{u2[0], u2[1], u2[2], u2[3]};
        }
        // q^T, k^T and (beta k)^T, channel-major (the level tables with factor 1).  With L2N
        // the raw rows: x_hat / r is within 2^-23 of the raw bf16 value, far
        // inside half a bf16 step, so the bf16 rounding gives it back exactly.
        auto raw_q = [&](int i) {
            return L2N ? to_f32(f32_to_bf16(qv[i] / sRn[p0 + i])) : qv[i];
        };
        auto raw_k = [&](int i) {
            return L2N ? to_f32(f32_to_bf16(kv[i] / sRn[C + p0 + i])) : kv[i];
        };
        if (cp) {
            float qx[RPP], kx[RPP];
#pragma unroll
            for (int i = 0; i < RPP; ++i) {
                qx[i] = raw_q(i);
                kx[i] = raw_k(i);
            }
#pragma unroll
            for (int i = 0; i < RPP; i += 8) {
                const uint2 q0 = pack4_bf16(qx[i], qx[i + 1], qx[i + 2], qx[i + 3]);
                const uint2 q1 = pack4_bf16(qx[i + 4], qx[i + 5], qx[i + 6], qx[i + 7]);
                const uint2 k0 = pack4_bf16(kx[i], kx[i + 1], kx[i + 2], kx[i + 3]);
                const uint2 k1 = pack4_bf16(kx[i + 4], kx[i + 5], kx[i + 6], kx[i + 7]);
                float bk[8];
#pragma unroll
                for (int z = 0; z < 8; ++z) bk[z] = sbeta[p0 + i + z] * kx[i + z];
                const uint2 b0 = pack4_bf16(bk[0], bk[1], bk[2], bk[3]);
                const uint2 b1 = pack4_bf16(bk[4], bk[5], bk[6], bk[7]);
                sQK[ctab_slot(cl, (p0 + i) / 8)] = uint4{q0.x, q0.y, q1.x, q1.y};
                sKK[ctab_slot(cl, (p0 + i) / 8)] = uint4{k0.x, k0.y, k1.x, k1.y};
                sKB[ctab_slot(cl, (p0 + i) / 8)] = uint4{b0.x, b0.y, b1.x, b1.y};
            }
        }
        __syncthreads();
        constexpr int T3 = NB * (HC / 16), M3 = (T3 + NW - 1) / NW;
        f32x4 xr[M3], rr2[M3], yr[M3];
#pragma unroll
        for (int m = 0; m < M3; ++m) {
            const int idx = w + NW * m;
            const int ti = (idx % T3) / (HC / 16), tj = idx % (HC / 16);
            f32x4 y1 = zero4();
            xr[m] = rr2[m] = yr[m] = zero4();
#pragma unroll
            for (int kb = 0; kb < C; kb += 32) {
                const bf16x8 ap = frag_rows<SwzU8, false>(sPv, ti * 16, kb / 8), aa = frag_rows<SwzU8, false>(sAv, ti * 16, kb / 8);
                const bf16x8 tp = frag_cols<SwzU8, false>(sPv, kb, ti * 16), ta = frag_cols<SwzU8, false>(sAv, kb, ti * 16);
                const bf16x8 bk = ctab_frag<false>(sKK, tj * 16, kb / 8);
                xr[m] = mfma_bf16_16x16x32(ap, bk, xr[m]);
                rr2[m] = mfma_bf16_16x16x32(aa, bk, rr2[m]);
                y1 = mfma_bf16_16x16x32(tp, ctab_frag<false>(sQK, tj * 16, kb / 8), y1);
                yr[m] = mfma_bf16_16x16x32(ta, ctab_frag<false>(sKB, tj * 16, kb / 8), yr[m]);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                xr[m][r] *= scale;
                yr[m][r] += scale * y1[r];
            }
        }
        __syncthreads();  // every read of the tables is done: their bytes take the results
        float* sX = reinterpret_cast<float*>(sbuf);
        float* sRq = reinterpret_cast<float*>(sbuf + C * PH * 4);
        float* sY = reinterpret_cast<float*>(sbuf + 2 * C * PH * 4);
#pragma unroll
        for (int m = 0; m < M3; ++m) {
            const int idx = w + NW * m;
            if (idx < T3) {
                const int ti = idx / (HC / 16), tj = idx % (HC / 16);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = ti * 16 + acc_row(r), j = tj * 16 + acc_col();
                    sX[ridx(i, j)] = xr[m][r];
                    sRq[ridx(i, j)] = rr2[m][r];
                    sY[ridx(i, j)] = yr[m][r];
                }
            }
        }
        __syncthreads();
        if (cp) {
#pragma unroll
            for (int i = 0; i < RPP; ++i) {
                const int r = p0 + i;
                const float X = sX[ridx(r, cl)], R = sRq[ridx(r, cl)], Y = sY[ridx(r, cl)], bt = sbeta[r];
                if constexpr (L2N) {
                    const float qr = raw_q(i), kr = raw_k(i);
                    dq[i] += X / sRn[r];
                    dk[i] += (bt * R + Y) / sRn[C + r];
                    dG[i] += qr * X + bt * kr * R - kr * Y;
                    dbr[i] += kr * R;
                } else {
                    dq[i] += X;
                    dk[i] += bt * R + Y;
                    dG[i] += qv[i] * X + bt * kv[i] * R - kv[i] * Y;
                    dbr[i] += kv[i] * R;
                }
            }
        }
    } else {
    // ---- diagonal scores (decay 1): P_ii = q_i . k_i
    if (cp) {
#pragma unroll
        for (int i = 0; i < RPP; ++i) {
            const float dp = scale * sel(sPv, p0 + i, p0 + i);
            dq[i] += dp * kv[i];
            dk[i] += dp * qv[i];
        }
    }

    // ---- pairs inside one 8-token part (j < i), on VALU: this thread owns
    // channel c of all 8 rows of its part; E_ij = prod_{s=j+1..i} a_s.  Row
    // sums rq (of dP E k), ra (of dA E k) and column sums cs (of dP E q +
    // dA E beta k) give the decay gradient too: d/dG_i E_ij = E_ij = -d/dG_j E_ij.
    if (cp) {
        float cs[RPP];
#pragma unroll
        for (int j = 0; j < RPP; ++j) cs[j] = 0.f;
#pragma unroll
        for (int i = 1; i < RPP; ++i) {
            const int r = p0 + i;
            const float bi = sbeta[r], bki = bi * kv[i], sqi = scale * qv[i];
            // this row's columns p0 .. p0 + 7: one 16-byte unit of each table
            const u32x4 pu = __builtin_bit_cast(u32x4, sPv[swz_slot<SwzU8>(r, p0 >> 3)]);
            const u32x4 au = __builtin_bit_cast(u32x4, sAv[swz_slot<SwzU8>(r, p0 >> 3)]);
            auto ext = [](const u32x4& u, int j) {
                return __uint_as_float((j & 1) ? (u[j >> 1] & 0xFFFF0000u) : (u[j >> 1] << 16));
            };
            float rq = 0.f, ra = 0.f, E = 1.f;
#pragma unroll
            for (int j = i - 1; j >= 0; --j) {
                E *= a[j + 1];
                const float tP = ext(pu, j) * E;
                const float tA = ext(au, j) * E;
                rq = fmaf(tP, kv[j], rq);
                ra = fmaf(tA, kv[j], ra);
                cs[j] = fmaf(tA, bki, fmaf(tP, sqi, cs[j]));
            }
            rq *= scale;
            dq[i] += rq;
            dk[i] = fmaf(bi, ra, dk[i]);
            dG[i] = fmaf(bki, ra, fmaf(qv[i], rq, dG[i]));
            dbr[i] = fmaf(kv[i], ra, dbr[i]);
        }
#pragma unroll
        for (int j = 0; j < RPP; ++j) {
            dk[j] += cs[j];
            dG[j] -= kv[j] * cs[j];
        }
    }

    // ---- pairs that span two 8-token parts: levels h = 32, 16, 8 of the
    // block-boundary split.  With F the level factor of each own row (query
    // rows prod_{s=m+1..r} a_s, key rows prod_{s=r+1..m} a_s, m the last token
    // of the earlier half) the tables hold (q o F)^T and (k o F)^T, and
    //   query rows: R1 = dPs KK,      R2 = dA KK
    //   key rows:   R1 = dPs^T QK,    R2 = (diag(beta) dA)^T KK
    // At h = 32, 16 a 16-row MFMA tile is all query or all key rows.  At h = 8
    // its rows 8..15 are query rows and 0..7 key rows of one 16-token block: a
    // lane of the A operand supplies dPs (query row, key columns) or dPs^T (key
    // row, query columns) and zeros elsewhere, and the B operand's key rows come
    // from KK and its query rows from QK, so one product gives both sides.
#pragma unroll
    for (int lvl = 0; lvl < 3; ++lvl) {
        const int hl = C >> (lvl + 1);
        float F[RPP];
        const int base = (p0 / (2 * hl)) * (2 * hl);
        const bool qs = p0 >= base + hl;
        if (qs) {
            float pre = 1.f;
            for (int pp = (base + hl) / RPP; pp < part; ++pp) pre *= stot[pp][cl];
            float Fr = pre;
#pragma unroll
            for (int i = 0; i < RPP; ++i) {
                Fr *= a[i];
                F[i] = Fr;
            }
        } else {
            float suf = 1.f;
            for (int pp = part + 1; pp < (base + hl) / RPP; ++pp) suf *= stot[pp][cl];
            float Fr = suf;
#pragma unroll
            for (int i = RPP - 1; i >= 0; --i) {
                F[i] = Fr;
                Fr *= a[i];
            }
        }
        // a level's products read the key half's rows from KK and the query
        // half's from QK and KB only, so each part writes just those
        if (cp) {
#pragma unroll
            for (int i = 0; i < RPP; i += 8) {
                float kf[8];
#pragma unroll
                for (int z = 0; z < 8; ++z) kf[z] = kv[i + z] * F[i + z];
                if (qs) {
                    const uint2 q0 = pack4_bf16(qv[i] * F[i], qv[i + 1] * F[i + 1], qv[i + 2] * F[i + 2], qv[i + 3] * F[i + 3]);
                    const uint2 q1 = pack4_bf16(qv[i + 4] * F[i + 4], qv[i + 5] * F[i + 5], qv[i + 6] * F[i + 6], qv[i + 7] * F[i + 7]);
                    const uint2 b0 = pack4_bf16(sbeta[p0 + i] * kf[0], sbeta[p0 + i + 1] * kf[1], sbeta[p0 + i + 2] * kf[2], sbeta[p0 + i + 3] * kf[3]);
                    const uint2 b1 = pack4_bf16(sbeta[p0 + i + 4] * kf[4], sbeta[p0 + i + 5] * kf[5], sbeta[p0 + i + 6] * kf[6], sbeta[p0 + i + 7] * kf[7]);
                    sQK[ctab_slot(cl, (p0 + i) / 8)] = uint4{q0.x, q0.y, q1.x, q1.y};
                    sKB[ctab_slot(cl, (p0 + i) / 8)] = uint4{b0.x, b0.y, b1.x, b1.y};
                } else {
                    const uint2 k0 = pack4_bf16(kf[0], kf[1], kf[2], kf[3]);
                    const uint2 k1 = pack4_bf16(kf[4], kf[5], kf[6], kf[7]);
                    sKK[ctab_slot(cl, (p0 + i) / 8)] = uint4{k0.x, k0.y, k1.x, k1.y};
                }
            }
        }
        __syncthreads();
        constexpr int T3 = NB * (HC / 16), M3 = (T3 + NW - 1) / NW;
#pragma unroll 2  // two tiles a wave: both in flight (118 VGPRs, no spill)
        for (int m = 0; m < M3; ++m) {
            const int idx = wu + NW * m;
            if (idx < T3) {
                const int ti = idx / (HC / 16), tj = idx % (HC / 16);
                const int tbase = (ti * 16 / (2 * hl)) * (2 * hl);
                const bool qt = ti * 16 >= tbase + hl;
                f32x4 r1, r2;
                if (hl >= 16) {
                    // query tiles: dPs and dA rows against k F; key tiles: their
                    // transposes against q F and beta k F
                    const int kb = qt ? tbase : tbase + hl;  // first row of the summed half
                    if (hl == 32) {
                        const bf16x8 a1 = qt ? frag_rows<SwzU8, false>(sPv, ti * 16, kb / 8) : frag_cols<SwzU8, false>(sPv, kb, ti * 16);
                        const bf16x8 a2 = qt ? frag_rows<SwzU8, false>(sAv, ti * 16, kb / 8) : frag_cols<SwzU8, false>(sAv, kb, ti * 16);
                        r1 = mfma_bf16_16x16x32(a1, ctab_frag<false>(qt ? sKK : sQK, tj * 16, kb / 8), zero4());
                        r2 = mfma_bf16_16x16x32(a2, ctab_frag<false>(qt ? sKK : sKB, tj * 16, kb / 8), zero4());
                    } else {
                        const bf16x8 a1 = qt ? frag_rows<SwzU8, true>(sPv, ti * 16, kb / 8) : frag_cols<SwzU8, true>(sPv, kb, ti * 16);
                        const bf16x8 a2 = qt ? frag_rows<SwzU8, true>(sAv, ti * 16, kb / 8) : frag_cols<SwzU8, true>(sAv, kb, ti * 16);
                        r1 = mfma_bf16_16x16x32(a1, ctab_frag<true>(qt ? sKK : sQK, tj * 16, kb / 8), zero4());
                        r2 = mfma_bf16_16x16x32(a2, ctab_frag<true>(qt ? sKK : sKB, tj * 16, kb / 8), zero4());
                    }
                } else {
                    // h = 8, K = the tile's own 16 rows on the K = 32 instruction:
                    // lane (row rr, K half kk & 1); lanes kk >= 2 supply zeros.  A
                    // query row takes its dPs / dA row over the key half (a row
                    // read), a key row dPs^T / dA^T over the query half (a
                    // transposing read); both reads run on every lane
                    const int l = lane_id(), rr = l & 15, kk = l >> 4, kh = kk & 1;
                    const bool qrow = rr >= 8;
                    const bool live = kk < 2 && (qrow ? kh == 0 : kh == 1);
                    // B: the key half's rows (kh = 0) k F, the query half's q F and
                    // beta k F
                    const int slot = ctab_slot(tj * 16 + rr, 2 * ti + kh);
                    {
                        const bf16x8 p_row = frag_rows<SwzU8, true>(sPv, ti * 16, 2 * ti);
                        const bf16x8 p_tr = frag_cols<SwzU8, true>(sPv, ti * 16, ti * 16);
                        const bf16x8 a1 = live ? (qrow ? p_row : p_tr) : bf16x8{};
                        bf16x8 b1 = __builtin_bit_cast(bf16x8, kh == 0 ? sKK[slot] : sQK[slot]);
                        if (kk >= 2) b1 = bf16x8{};
                        r1 = mfma_bf16_16x16x32(a1, b1, zero4());
                    }
                    {
                        const bf16x8 a_row = frag_rows<SwzU8, true>(sAv, ti * 16, 2 * ti);
                        const bf16x8 a_tr = frag_cols<SwzU8, true>(sAv, ti * 16, ti * 16);
                        const bf16x8 a2 = live ? (qrow ? a_row : a_tr) : bf16x8{};
                        bf16x8 b2 = __builtin_bit_cast(bf16x8, kh == 0 ? sKK[slot] : sKB[slot]);
                        if (kk >= 2) b2 = bf16x8{};
                        r2 = mfma_bf16_16x16x32(a2, b2, zero4());
                    }
                }
                // results: a lane's four rows acc_row(0) + r of column
                // acc_col(), at one lane address plus immediate row offsets.
                // Query rows keep R1 and R2 apart (R2 in sR2, whose rows are
                // the query halves' rows packed), key rows take R1 + R2.
                const int lrow = acc_row(0), lcol = acc_col();
                float* const pR = sR + ridx(ti * 16, tj * 16) + ridx(lrow, lcol);
                const bool qrows = hl >= 16 ? qt : lrow >= 8;  // the lane's four rows alike
                if (qrows) {
                    // first row of this tile's query rows in sR2: the tile's
                    // first query row i0 maps to (i0 / (2 hl)) hl + i0 % hl, and
                    // the rows after it follow on
                    const int i0 = ti * 16 + (hl >= 16 ? 0 : 8);
                    float* const pR2 = sR2 + ridx((i0 / (2 * hl)) * hl + (i0 % hl), tj * 16) +
                                       ridx(lrow - (hl >= 16 ? 0 : 8), lcol);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        pR[r * PH] = scale * r1[r];
                        pR2[r * PH] = r2[r];
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) pR[r * PH] = scale * r1[r] + r2[r];
                }
            }
        }
        __syncthreads();
        if (cp) {
            if (qs) {
#pragma unroll
                for (int i = 0; i < RPP; ++i) {
                    const int r = p0 + i;
                    const float R1 = sR[ridx(r, cl)], R2 = sR2[ridx((r / (2 * hl)) * hl + (r % hl), cl)];
                    const float bt = sbeta[r];
                    const float t1 = F[i] * R1, t2 = F[i] * R2, kt2 = kv[i] * t2;
                    dq[i] += t1;
                    dk[i] = fmaf(bt, t2, dk[i]);
                    dG[i] = fmaf(bt, kt2, fmaf(qv[i], t1, dG[i]));
                    dbr[i] += kt2;
                }
            } else {
#pragma unroll
                for (int i = 0; i < RPP; ++i) {
                    const float t = F[i] * sR[ridx(p0 + i, cl)];
                    dk[i] += t;
                    dG[i] = fmaf(-kv[i], t, dG[i]);
                }
            }
        }
    }

    }  // per-channel decay

    // ---- dg = reverse cumulative sum of dG over the chunk (the part sums go
    // through stot, no longer needed); dq, dk, dg out; dbeta partials
    float (*spart)[HC] = stot;  // every level factor was formed before the last level's barriers
    if (cp) {
        float s = 0.f;
#pragma unroll
        for (int i = RPP - 1; i >= 0; --i) {
            s += dG[i];
            dG[i] = s;
        }
        spart[part][cl] = s;
    }
    __syncthreads();
    if (cp) {
        float add = 0.f;
        for (int pp = part + 1; pp < NPART; ++pp) add += spart[pp][cl];
#pragma unroll
        for (int i = 0; i < RPP; ++i) {
            const int r = p0 + i;
            dG[i] += add;
            sR[ridx(r, cl)] = dbr[i];
            if (r < nvalid) {
                const uint32_t off = (uint32_t)r * rs32 + (uint32_t)c;
                st32(dqo + tok0 * DK, off, f32_to_bf16(dq[i]));
                st32(dko + tok0 * DK, off, f32_to_bf16(dk[i]));
                if (PCH) st32(dgo + tok0 * DK, off, dG[i]);
            }
        }
    }
    __syncthreads();
    // dbeta partial: row sums of dbr over this half's channels, 4 threads per row
    {
        const int r = tid >> 2, sub = tid & 3;
        float sb = 0.f;
        if (r < C) {
#pragma unroll
            for (int cc = sub; cc < HC; cc += 4) sb += sR[ridx(r, cc)];
        }
        sb += dpp_mov<0xB1>(sb);  // quad sum: neighbour swap, pair swap
        sb += dpp_mov<0x4E>(sb);
        if (r < C && sub == 0) dbq[((size_t)ch * 2 + half) * C + r] = sb;
    }
    if (!PCH) {
        // per-head decay: dg of a row is the sum of dG over all channels
        __syncthreads();
        if (cp) {
#pragma unroll
            for (int i = 0; i < RPP; ++i) sR[ridx(p0 + i, cl)] = dG[i];
        }
        __syncthreads();
        const int r = tid >> 2, sub = tid & 3;
        float sg = 0.f;
        if (r < C) {
#pragma unroll
            for (int cc = sub; cc < HC; cc += 4) sg += sR[ridx(r, cc)];
        }
        sg += dpp_mov<0xB1>(sg);  // quad sum: neighbour swap, pair swap
        sg += dpp_mov<0x4E>(sg);
        if (r < C && sub == 0) dgq[((size_t)ch * 2 + half) * C + r] = sg;
    }
}

// dbeta = (part through U, from bchunk1b) + the two channel halves' partials;
// for per-head decay also dg = sum of the two halves.  Fixed order: repeatable.
template <bool PCH>
__global__ void __launch_bounds__(256)
bchunk2_finish_kernel(const float* __restrict__ dbpi, const float* __restrict__ dbq,
                      const float* __restrict__ dgq, float* __restrict__ dbo,
                      float* __restrict__ dgo, int T, int H, int NC, int C, long long total)
{
    const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
    if (e >= total) return;
    const int r = (int)(e % C);
    const long long ch = e / C;
    const int n = (int)(ch % NC), bh = (int)(ch / NC), h = bh % H, b = bh / H;
    const int t = n * C + r;
    if (t >= T) return;
    const size_t tok = ((size_t)b * T + t) * H + h;
    dbo[tok] = dbpi[ch * C + r] + dbq[(ch * 2) * C + r] + dbq[(ch * 2 + 1) * C + r];
    if (!PCH) dgo[tok] = dgq[(ch * 2) * C + r] + dgq[(ch * 2 + 1) * C + r];
}

// ---------------------------------------------------------------------------
// l2norm_bwd: the adjoint of use_qk_l2norm, in place.  dq and dk hold the
// gradients with respect to the normalised rows x_hat = r x; the raw rows'
// gradients are dx = r (dx_hat - x_hat (x_hat . dx_hat)).  One row (the Dk
// values of one token and head) per LPR lanes, 16 bytes per lane; the row dot
// is a fixed butterfly over those lanes (repeatable).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void load16(const bf16* p, float (&x)[8])
{
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[2 * e] = __uint_as_float(w[e] << 16);
        x[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
}
__device__ __forceinline__ void load16(const float* p, float (&x)[4])
{
    const float4 v = *reinterpret_cast<const float4*>(p);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
}
__device__ __forceinline__ void store16(bf16* p, const float (&x)[8])
{
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
        w[e] = (uint32_t)f32_to_bf16(x[2 * e]).bits | ((uint32_t)f32_to_bf16(x[2 * e + 1]).bits << 16);
    *reinterpret_cast<uint4*>(p) = uint4{w[0], w[1], w[2], w[3]};
}
__device__ __forceinline__ void store16(float* p, const float (&x)[4])
{
    *reinterpret_cast<float4*>(p) = float4{x[0], x[1], x[2], x[3]};
}

constexpr int NTHR_L = 256;

template <typename TIn, int DK>
__global__ void __launch_bounds__(NTHR_L)
l2norm_bwd_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k, const float* __restrict__ rn,
                  TIn* __restrict__ dq, TIn* __restrict__ dk, int T, int H, int NC, int C,
                  long long ntok)
{
    constexpr int EPL = 16 / (int)sizeof(TIn);  // elements per lane
    constexpr int LPR = DK / EPL;               // lanes per row
    static_assert(LPR >= 1 && LPR <= 64 && (LPR & (LPR - 1)) == 0 && NTHR_L % LPR == 0,
                  "a row is a power-of-two group of lanes inside one wave");
    const long long gid = (long long)blockIdx.x * NTHR_L + threadIdx.x;
    // lanes past the last row work on row 0 (every lane joins the butterfly)
    // and store nothing
    const bool ok = gid / LPR < ntok;
    const long long tok = ok ? gid / LPR : 0;
    const int ln = (int)(gid % LPR);
    const int h = (int)(tok % H);
    const long long bt = tok / H;
    const int t = (int)(bt % T);
    const long long b = bt / T;
    const size_t ch = ((size_t)b * H + h) * NC + t / C;
    const int r = t % C;
    const float rq = rn[(ch * 2) * C + r], rk = rn[(ch * 2 + 1) * C + r];
    const size_t e0 = (size_t)tok * DK + (size_t)ln * EPL;
    float xq[EPL], xk[EPL], gq[EPL], gk[EPL];
    load16(q + e0, xq);
    load16(k + e0, xk);
    load16(dq + e0, gq);
    load16(dk + e0, gk);
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        xq[e] *= rq;
        xk[e] *= rk;
        sq += xq[e] * gq[e];
        sk += xk[e] * gk[e];
    }
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) {
        sq += __shfl_xor(sq, off);
        sk += __shfl_xor(sk, off);
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        gq[e] = rq * (gq[e] - xq[e] * sq);
        gk[e] = rk * (gk[e] - xk[e] * sk);
    }
    if (ok) {
        store16(dq + e0, gq);
        store16(dk + e0, gk);
    }
}

template <typename TIn, int DK>
gdn_status run_l2norm_bwd(const Plan& p, const void* q, const void* k, void* dq, void* dk,
                          const char* ws, hipStream_t st)
{
    constexpr int LPR = DK / (16 / (int)sizeof(TIn));
    const long long ntok = (long long)p.B * p.T * p.H;
    const long long nthr = ntok * LPR;
    dim3 grid((unsigned)((nthr + NTHR_L - 1) / NTHR_L));
    GDN_LAUNCH("l2norm_bwd", (l2norm_bwd_kernel<TIn, DK>), grid, dim3(NTHR_L), st, (const TIn*)q,
               (const TIn*)k, (const float*)(ws + p.o_rn), (TIn*)dq, (TIn*)dk, p.T, p.H, p.NC,
               p.C, ntok);
    return GDN_OK;
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
template <typename TIn, int C, int DK, int DV>
gdn_status backward_t(const Plan& p, const void* q, const void* k, const void* v, const float* g,
                      const float* beta, const float* h0, const void* dO, const float* dhT,
                      void* dq, void* dk, void* dv, float* dg, float* dbeta, float* dh0, char* ws,
                      bool recompute, hipStream_t st)
{
    constexpr int MT = std::is_same<TIn, bf16>::value ? MT_BF16 : MT_F32;
    if (recompute) {
        gdn_status s = recompute_dispatch(p, q, k, v, g, beta, h0, nullptr, nullptr, false, ws, st);
        if (s != GDN_OK) return s;
    }
    const int BH = p.B * p.H;
    const float* rn = p.l2n ? (const float*)(ws + p.o_rn) : nullptr;
    if constexpr (bf16_tables<TIn, C, DK>()) {
        // the forward tables (plan.h)
        dim3 grid((unsigned)(((BH + 7) / 8) * 8 * (DV / 32))), block(NTHR_B4);
        GDN_LAUNCH("bscan", (bscan4_kernel<DK, DV>), grid, block, st,
                   (const bf16*)(ws + p.o_Kh), (const bf16*)(ws + p.o_Ps),
                   (const bf16*)(ws + p.o_Qg), (const bf16*)(ws + p.o_W),
                   (const float*)(ws + p.o_gam), (const bf16*)dO, dhT, (bf16*)(ws + p.o_dSt),
                   (bf16*)(ws + p.o_dDt), dh0, BH, p.T, p.H, p.NC);
    } else if constexpr (f32_tables<TIn, C, DK>()) {
        dim3 grid((unsigned)(((BH + 7) / 8) * 8 * (DV / 32))), block(512);
        GDN_LAUNCH("bscan", (bscanf_kernel<DK, DV>), grid, block, st,
                   (const float*)(ws + p.o_Kh), (const float*)(ws + p.o_Ps),
                   (const float*)(ws + p.o_Qg), (const float*)(ws + p.o_W),
                   (const float*)(ws + p.o_gam), (const float*)dO, dhT, (float*)(ws + p.o_dSt),
                   (float*)(ws + p.o_dDt), dh0, BH, p.T, p.H, p.NC);
    } else {
        using SC = BScanCfg<DV>;
        dim3 grid((unsigned)(((BH + 7) / 8) * 8 * SC::NS)), block(NTHR);
        GDN_LAUNCH("bscan", (bscan_kernel<TIn, C, DK, DV, MT>), grid, block, st,
                           (const float*)(ws + p.o_Qg), (const float*)(ws + p.o_Kh),
                           (const float*)(ws + p.o_W), (const float*)(ws + p.o_Ps),
                           (const float*)(ws + p.o_gam), (const TIn*)dO, dhT,
                           (float*)(ws + p.o_dSt), (float*)(ws + p.o_dDt), dh0, BH, p.T, p.H, p.NC);
        GDN_HIP_CHECK_LAUNCH();
    }
    dim3 gch((unsigned)p.n_ch);
    if constexpr (bf16_tables<TIn, C, DK>()) {
        // the WY adjoint takes W = T X_K as a product: with clip the unclipped
        // copy (clipping is differentiated as the identity; its U side is formed
        // from T and v in the kernel)
        const bool raw = p.clip > 0.f;
        // persistent, one workgroup per CU (its LDS allows no second one)
        const dim3 gp((unsigned)std::min<long long>(p.n_ch, device_cus()));
        GDN_LAUNCH("bchunk1", (bchunk1b_kernel<C, DK, DV>), gp, dim3(NTHR_C), st, (const bf16*)v,
                   beta, (const bf16*)dO, (const bf16*)(ws + p.o_Dst), (const float*)(ws + p.o_Tm),
                   (const bf16*)(ws + (raw ? p.o_Wr : p.o_W)),
                   (const bf16*)(ws + p.o_Sst), (const bf16*)(ws + p.o_dSt),
                   (const bf16*)(ws + p.o_dDt), (bf16*)dv, (float*)(ws + p.o_dQg),
                   (float*)(ws + p.o_dWg), (float*)(ws + p.o_dKh), (float*)(ws + p.o_dPs),
                   (float*)(ws + p.o_dT1), (float*)(ws + p.o_dgm), (float*)(ws + p.o_dbp), p.T, p.H,
                   p.NC, (int)p.n_ch);
    } else if constexpr (f32_tables<TIn, C, DK>()) {
        GDN_LAUNCH("bchunk1", (bchunk1f_kernel<DK, DV>), gch, dim3(512), st, (const float*)v, beta,
                   (const float*)dO, (const float*)(ws + p.o_Dst),
                   (const float*)(ws + p.o_Tm), (const float*)(ws + p.o_Sst),
                   (const float*)(ws + p.o_dSt), (const float*)(ws + p.o_dDt), (float*)dv,
                   (float*)(ws + p.o_dQg), (float*)(ws + p.o_dWg), (float*)(ws + p.o_dKh),
                   (float*)(ws + p.o_dPs), (float*)(ws + p.o_dT1), (float*)(ws + p.o_dgm),
                   (float*)(ws + p.o_dbp), p.T, p.H, p.NC);
    } else
    GDN_LAUNCH("bchunk1", (bchunk1_kernel<TIn, C, DK, DV, MT>), gch, dim3(NTHR), st,
                       (const TIn*)v, beta, (const TIn*)dO, (const float*)(ws + p.o_W),
                       (const float*)(ws + p.o_U), (const float*)(ws + p.o_Tm),
                       (const float*)(ws + p.o_Sst), (const float*)(ws + p.o_dSt),
                       (const float*)(ws + p.o_dDt), (TIn*)dv, (float*)(ws + p.o_dQg),
                       (float*)(ws + p.o_dWg), (float*)(ws + p.o_dKh), (float*)(ws + p.o_dPs),
                       (float*)(ws + p.o_dT1), (float*)(ws + p.o_dgm), (float*)(ws + p.o_dbp), p.T,
                       p.H, p.NC);
    GDN_HIP_CHECK_LAUNCH();
    if constexpr (bf16_tables<TIn, C, DK>()) {
        // here the dW region holds dX_K and the dT1 region dA (bchunk1b)
        const int nch = (int)p.n_ch;
        dim3 g2((unsigned)(((p.n_ch + 7) / 8) * 16));
        auto launch2 = [&](auto pch, auto l2n) {
            GDN_LAUNCH("bchunk2",
                       (bchunk2c_kernel<C, DK, decltype(pch)::value, decltype(l2n)::value>), g2,
                       dim3(bchunk2c_threads<C, DK>()), st, (const bf16*)q, (const bf16*)k, g, beta,
                       (const bf16*)(ws + p.o_dQg), (const bf16*)(ws + p.o_dWg),
                       (const bf16*)(ws + p.o_dKh), (const bf16*)(ws + p.o_dPs),
                       (const bf16*)(ws + p.o_dT1), (const float*)(ws + p.o_dgm), (bf16*)dq,
                       (bf16*)dk, dg, (float*)(ws + p.o_dbq), (float*)(ws + p.o_dgq), p.T, p.H,
                       p.NC, nch, p.scale, rn);
            return GDN_OK;
        };
        using TT = std::true_type;
        using FF = std::false_type;
        gdn_status s2 = p.decay == GDN_DECAY_PER_CHANNEL
                            ? (p.l2n ? launch2(TT{}, TT{}) : launch2(TT{}, FF{}))
                            : (p.l2n ? launch2(FF{}, TT{}) : launch2(FF{}, FF{}));
        if (s2 != GDN_OK) return s2;
        const long long tot = (long long)p.n_ch * C;
        dim3 gf((unsigned)((tot + 255) / 256));
        if (p.decay == GDN_DECAY_PER_CHANNEL)
            GDN_LAUNCH("bchunk2_finish", (bchunk2_finish_kernel<true>), gf, dim3(256), st,
                       (const float*)(ws + p.o_dbp), (const float*)(ws + p.o_dbq),
                       (const float*)(ws + p.o_dgq), dbeta, dg, p.T, p.H, p.NC, C, tot);
        else
            GDN_LAUNCH("bchunk2_finish", (bchunk2_finish_kernel<false>), gf, dim3(256), st,
                       (const float*)(ws + p.o_dbp), (const float*)(ws + p.o_dbq),
                       (const float*)(ws + p.o_dgq), dbeta, dg, p.T, p.H, p.NC, C, tot);
        if (p.l2n) return run_l2norm_bwd<TIn, DK>(p, q, k, dq, dk, ws, st);
        return GDN_OK;
    } else {
    if (p.decay == GDN_DECAY_PER_CHANNEL)
        GDN_LAUNCH("bchunk2", (bchunk2_kernel<TIn, C, DK, DV, true, MT>), gch, dim3(NTHR2), st,
                           (const TIn*)q, (const TIn*)k, g, beta, (const float*)(ws + p.o_Tm),
                           (const float*)(ws + p.o_dQg), (const float*)(ws + p.o_dWg),
                           (const float*)(ws + p.o_dKh), (const float*)(ws + p.o_dPs),
                           (const float*)(ws + p.o_dT1), (const float*)(ws + p.o_dgm),
                           (const float*)(ws + p.o_dbp), (TIn*)dq, (TIn*)dk, dg, dbeta, p.T, p.H,
                           p.NC, p.scale, rn);
    else
        GDN_LAUNCH("bchunk2", (bchunk2_kernel<TIn, C, DK, DV, false, MT>), gch, dim3(NTHR2), st,
                           (const TIn*)q, (const TIn*)k, g, beta, (const float*)(ws + p.o_Tm),
                           (const float*)(ws + p.o_dQg), (const float*)(ws + p.o_dWg),
                           (const float*)(ws + p.o_dKh), (const float*)(ws + p.o_dPs),
                           (const float*)(ws + p.o_dT1), (const float*)(ws + p.o_dgm),
                           (const float*)(ws + p.o_dbp), (TIn*)dq, (TIn*)dk, dg, dbeta, p.T, p.H,
                           p.NC, p.scale, rn);
    GDN_HIP_CHECK_LAUNCH();
    if (p.l2n) return run_l2norm_bwd<TIn, DK>(p, q, k, dq, dk, ws, st);
    return GDN_OK;
    }
}

template <typename TIn>
gdn_status backward_dt(const Plan& p, const void* q, const void* k, const void* v, const float* g,
                       const float* beta, const float* h0, const void* dO, const float* dhT,
                       void* dq, void* dk, void* dv, float* dg, float* dbeta, float* dh0, char* ws,
                       bool recompute, hipStream_t st)
{
#define GDN_BWD(C_, D_)                                                                           \
    if (p.C == C_ && p.Dk == D_ && p.Dv == D_)                                                     \
        return backward_t<TIn, C_, D_, D_>(p, q, k, v, g, beta, h0, dO, dhT, dq, dk, dv, dg, dbeta, \
                                           dh0, ws, recompute, st);
    GDN_BWD(64, 128) GDN_BWD(64, 64) GDN_BWD(16, 16)
#undef GDN_BWD
    return GDN_ERR_UNSUPPORTED;
}

gdn_status backward_dispatch(const Plan& p, const void* q, const void* k, const void* v,
                             const float* g, const float* beta, const float* h0, const void* dO,
                             const float* dhT, void* dq, void* dk, void* dv, float* dg,
                             float* dbeta, float* dh0, void* ws, bool recompute, hipStream_t st)
{
    gdn_status s =
        p.dtype == GDN_BF16
            ? backward_dt<bf16>(p, q, k, v, g, beta, h0, dO, dhT, dq, dk, dv, dg, dbeta, dh0,
                                (char*)ws, recompute, st)
            : backward_dt<float>(p, q, k, v, g, beta, h0, dO, dhT, dq, dk, dv, dg, dbeta, dh0,
                                 (char*)ws, recompute, st);
    if (s != GDN_OK || !(p.clip > 0.f)) return s;
    // clip: the gradient outputs cross the layer's boundary
    const size_t tok = (size_t)p.B * p.T * p.H;
    const size_t nq = tok * p.Dk, nv = tok * p.Dv;
    const size_t ng = p.decay == GDN_DECAY_PER_CHANNEL ? nq : tok;
    const int bf = p.dtype == GDN_BF16;
    const SafeSeg segs[6] = {{dq, nq, bf, nullptr},  {dk, nq, bf, nullptr},
                             {dv, nv, bf, nullptr},  {dg, ng, 0, nullptr},
                             {dbeta, tok, 0, nullptr},
                             {dh0, (size_t)p.B * p.H * p.Dk * p.Dv, 0, nullptr}};
    return safe_pass(segs, 6, p.clip, st);
}

}  // namespace gdn
