// chunk_fwd.hip -- chunked forward of the gated delta rule on gfx950.
//
// Two kernels (atomic_ops card, "Features": chunk scores -> WY block solve ->
// recompute -> inter-chunk scan):
//
//  prep  one workgroup per chunk-head (C tokens of one (b, h)), fully parallel.
//        Per key channel c and token r, a_rc = exp(g_rc).  The decayed scores
//          P_ij = sum_c q_ic k_jc E_ijc  (j <= i),
//          A_ij = beta_i sum_c k_ic k_jc E_ijc  (j < i),  E_ijc = prod_{s=j+1..i} a_sc
//        are formed with the decay split at a block boundary (Marin note,
//        "Approach"): the chunk is cut into two halves, a pair (i, j) that spans
//        them takes E_ij = [prod_{s=m+1..i} a_s] * [prod_{s=j+1..m} a_s] with m
//        the last token of the earlier half, so scaling each query row and each
//        key row by its own factor (both <= 1) turns the spanning scores into
//        one dense product on the matrix cores.  The split is applied again
//        inside every half, down to single tokens, so every score is produced
//        by MFMA; the diagonal (E = 1) is a plain dot product.  The factors are
//        running products of a, one exp per token-channel.
//        Then T = (I + A)^-1 (16-row diagonal blocks by forward substitution,
//        merged pairwise by T21 = -T22 A21 T11 on MFMA), and the WY form
//          W = T diag(beta) (K o Gamma),  U = T diag(beta) V,
//        with Gamma_r = prod_{s<=r} a_s; also Qg = scale Q o Gamma,
//        Kh = K o prod_{s>r} a_s and gam = prod_s a_s.
//  scan  one workgroup per (b, h, Dv-slice), sequential over chunks, the fp32
//        state slice resident in LDS:
//          D = U - W S;  O = Qg S + scale P D;  S <- gam o S + Kh^T D.
//        Each Dv column of S evolves on its own, which is what allows the
//        slicing; the slices of one (b, h) are given workgroup ids that land
//        on the same XCD so their shared W/Qg/Kh/P reads hit one L2.
#include <type_traits>

#include "chunk_common.h"
#include "plan.h"

namespace gdn {

// ---------------------------------------------------------------------------
// prep
// ---------------------------------------------------------------------------
template <typename TIn, int C, int DK, int DV, bool PCH, int MT>
__global__ void __launch_bounds__(NTHR)
prep_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
            const float* __restrict__ g, const float* __restrict__ beta, int T, int H, int NC,
            float scale, float* __restrict__ Wo, float* __restrict__ Uo, float* __restrict__ Qgo,
            float* __restrict__ Kho, float* __restrict__ Pso, float* __restrict__ gamo,
            float* __restrict__ Tmo)
{
    using G = Geo<C, DK, DV>;
    constexpr int PD = G::PD, PC = G::PC, NB = G::NB, HALF = G::HALF;
    __shared__ float sq[C][PD], sk[C][PD], sX[C][PD], sY[C][PD], sA[C][PC];
    __shared__ float sbeta[C], sdiag[C], stot[2][DK];

    const int ch = blockIdx.x;
    const int n = ch % NC, bh = ch / NC, h = bh % H, b = bh / H;
    const int t0 = n * C;
    const int nvalid = min(C, T - t0);
    const int tid = threadIdx.x, w = tid >> 6;
    const size_t tok0 = ((size_t)b * T + t0) * H + h;  // token index of row 0
    const TIn* qb = q + tok0 * DK;
    const TIn* kb = k + tok0 * DK;
    const TIn* vb = v + tok0 * DV;
    const size_t rsK = (size_t)H * DK, rsV = (size_t)H * DV;

    // ---- loads: q, k rows (zero past T), beta (zero past T)
    for (int idx = tid; idx < C * DK / 4; idx += NTHR) {
        const int r = idx / (DK / 4), c4 = (idx % (DK / 4)) * 4;
        float4 qv = {0.f, 0.f, 0.f, 0.f}, kv = qv;
        if (r < nvalid) {
            qv = load4<TIn>(qb + r * rsK + c4);
            kv = load4<TIn>(kb + r * rsK + c4);
        }
        st4(&sq[r][c4], qv);
        st4(&sk[r][c4], kv);
    }
    for (int r = tid; r < C; r += NTHR) sbeta[r] = r < nvalid ? beta[(tok0 + (size_t)r * H)] : 0.f;

    // ---- column-pass threads: channel c, rows [part*HALF, part*HALF + HALF)
    const bool cp = tid < 2 * DK;
    const int c = tid % DK, part = (tid / DK) & 1;
    float a[HALF];
#pragma unroll
    for (int i = 0; i < HALF; ++i) {
        const int r = part * HALF + i;
        float gv = 0.f;
        if (cp && r < nvalid) gv = PCH ? g[(tok0 + (size_t)r * H) * DK + c] : g[tok0 + (size_t)r * H];
        a[i] = expf(gv);
    }
    __syncthreads();

    // ---- diagonal scores P_ii = q_i . k_i
    for (int r = tid; r < C; r += NTHR) {
        float s = 0.f;
        for (int cc = 0; cc < DK; ++cc) {
            const int c2 = (cc + r) % DK;  // skewed to spread LDS banks
            s += sq[r][c2] * sk[r][c2];
        }
        sdiag[r] = s;
    }

    // ---- hierarchical block-boundary split, levels h = C/2 .. 1
    f32x4 accP[G::MAXOFF > 0 ? G::MAXOFF : 1], accA[G::MAXOFF > 0 ? G::MAXOFF : 1];
#pragma unroll
    for (int s = 0; s < (G::MAXOFF > 0 ? G::MAXOFF : 1); ++s) accP[s] = accA[s] = zero4();
    f32x4 dP = zero4(), dA = zero4();

#pragma unroll
    for (int lvl = 0; (C >> (lvl + 1)) >= 1; ++lvl) {
        const int hl = C >> (lvl + 1);
        // factor tables: sX[r] = q_r F_r, sY[r] = k_r F_r, F the level-hl factor of row r
        if (cp) {
#pragma unroll
            for (int u0 = 0; u0 < HALF; u0 += hl) {
                const int r0 = part * HALF + u0;
                const bool query = (r0 / hl) & 1;
                if (query) {  // F_r = prod_{s=r0..r} a_s
                    float F = 1.f;
#pragma unroll
                    for (int i = 0; i < hl; ++i) {
                        F *= a[u0 + i];
                        sX[r0 + i][c] = sq[r0 + i][c] * F;
                        sY[r0 + i][c] = sk[r0 + i][c] * F;
                    }
                } else {      // F_r = prod_{s=r+1..r0+hl-1} a_s
                    float F = 1.f;
#pragma unroll
                    for (int i = hl - 1; i >= 0; --i) {
                        sX[r0 + i][c] = sq[r0 + i][c] * F;
                        sY[r0 + i][c] = sk[r0 + i][c] * F;
                        F *= a[u0 + i];
                    }
                }
            }
        }
        __syncthreads();
        if (hl >= 16) {
#pragma unroll
            for (int s = 0; s < G::MAXOFF; ++s) {
                const int idx = w + 4 * s;
                if (idx < G::NOFF) {
                    int ti, tj;
                    off_tile(idx, ti, tj);
                    if (off_tile_level(ti, tj) == hl) {
                        accP[s] = mma16k<MT, DK>(accP[s], &sX[ti * 16][0], PD, 1, &sY[tj * 16][0], 1, PD);
                        accA[s] = mma16k<MT, DK>(accA[s], &sY[ti * 16][0], PD, 1, &sY[tj * 16][0], 1, PD);
                    }
                }
            }
        } else if (w < NB) {
            const int t = w;
            f32x4 tp = mma16k<MT, DK>(zero4(), &sX[t * 16][0], PD, 1, &sY[t * 16][0], 1, PD);
            f32x4 ta = mma16k<MT, DK>(zero4(), &sY[t * 16][0], PD, 1, &sY[t * 16][0], 1, PD);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (in_level(acc_row(r), acc_col(), hl)) {
                    dP[r] += tp[r];
                    dA[r] += ta[r];
                }
            }
        }
        __syncthreads();
    }

    // ---- scores out: Ps = scale P (global, upper part zero), A (x beta) to LDS
    float* Ps = Pso + (size_t)ch * C * C;
#pragma unroll
    for (int s = 0; s < G::MAXOFF; ++s) {
        const int idx = w + 4 * s;
        if (idx < G::NOFF) {
            int ti, tj;
            off_tile(idx, ti, tj);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = ti * 16 + acc_row(r), j = tj * 16 + acc_col();
                Ps[i * C + j] = scale * accP[s][r];
                sA[i][j] = sbeta[i] * accA[s][r];
            }
        }
    }
    if (w < NB) {
        const int t = w;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = t * 16 + acc_row(r), j = t * 16 + acc_col();
            const float pv = i > j ? dP[r] : (i == j ? sdiag[i] : 0.f);
            Ps[i * C + j] = scale * pv;
            sA[i][j] = i > j ? sbeta[i] * dA[r] : 0.f;
        }
    }
    for (int idx = tid; idx < C * C; idx += NTHR) {
        const int i = idx / C, j = idx % C;
        if (i / 16 < j / 16) {
            Ps[idx] = 0.f;
            sA[i][j] = 0.f;
        }
    }

    // ---- Gamma, Kh, gam, Qg and X_K = beta K o Gamma (into sY)
    float ptot = 1.f;
#pragma unroll
    for (int i = 0; i < HALF; ++i) ptot *= a[i];
    if (cp) stot[part][c] = ptot;
    float* sT = &sX[0][0];  // T = (I + A)^-1, [C][PC] view of sX
    for (int idx = tid; idx < C * PC; idx += NTHR) sT[idx] = 0.f;
    __syncthreads();
    if (cp) {
        float Gm = part ? stot[0][c] : 1.f;
        float* Qg = Qgo + (size_t)ch * C * DK;
        float* Kh = Kho + (size_t)ch * C * DK;
#pragma unroll
        for (int i = 0; i < HALF; ++i) {
            const int r = part * HALF + i;
            Gm *= a[i];
            Qg[r * DK + c] = scale * sq[r][c] * Gm;
            sY[r][c] = sbeta[r] * sk[r][c] * Gm;
        }
        if (part == 1) gamo[(size_t)ch * DK + c] = Gm;
        float kap = part ? 1.f : stot[1][c];
#pragma unroll
        for (int i = HALF - 1; i >= 0; --i) {
            const int r = part * HALF + i;
            Kh[r * DK + c] = sk[r][c] * kap;
            kap *= a[i];
        }
    }

    // ---- WY solve: 16x16 diagonal blocks of (I + A)^-1 by forward substitution
    if (w == 0) {
        const int lane = tid & 63, bb = lane >> 4, j = lane & 15;
        if (bb < NB) {
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float s = (i == j) ? 1.f : 0.f;
#pragma unroll
                for (int m = 0; m < i; ++m) s -= sA[bb * 16 + i][bb * 16 + m] * x[m];
                x[i] = s;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) sT[(bb * 16 + i) * PC + bb * 16 + j] = x[i];
        }
    }
    __syncthreads();
    // merge neighbouring diagonal blocks: T21 = -T22 (A21 T11)
    float* sYt = &sq[0][0];  // [C][PC] scratch (q no longer needed)
#pragma unroll
    for (int s = 16; 2 * s <= C; s *= 2) {
        const int tps = (s / 16) * (s / 16);       // 16-tiles per s x s block
        const int ntile = (C / (2 * s)) * tps;
        for (int idx = w; idx < ntile; idx += 4) {
            const int p = idx / tps, ti = (idx % tps) / (s / 16), tj = idx % (s / 16);
            const int b0 = p * 2 * s;
            f32x4 y = mma16<MT_F32>(zero4(), &sA[b0 + s + 16 * ti][b0], PC, 1,
                                    &sT[b0 * PC + b0 + 16 * tj], PC, 1, s);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sYt[(b0 + s + 16 * ti + acc_row(r)) * PC + b0 + 16 * tj + acc_col()] = y[r];
        }
        __syncthreads();
        for (int idx = w; idx < ntile; idx += 4) {
            const int p = idx / tps, ti = (idx % tps) / (s / 16), tj = idx % (s / 16);
            const int b0 = p * 2 * s;
            f32x4 t21 = mma16<MT_F32>(zero4(), &sT[(b0 + s + 16 * ti) * PC + b0 + s], PC, 1,
                                      &sYt[(b0 + s) * PC + b0 + 16 * tj], PC, 1, s);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sT[(b0 + s + 16 * ti + acc_row(r)) * PC + b0 + 16 * tj + acc_col()] = -t21[r];
        }
        __syncthreads();
    }
    if (Tmo) {
        float* Tm = Tmo + (size_t)ch * C * C;
        for (int idx = tid; idx < C * C; idx += NTHR) Tm[idx] = sT[(idx / C) * PC + idx % C];
    }

    // ---- X_V = beta V into sq, then W = T X_K and U = T X_V
    for (int idx = tid; idx < C * DV / 4; idx += NTHR) {
        const int r = idx / (DV / 4), c4 = (idx % (DV / 4)) * 4;
        float4 vv = {0.f, 0.f, 0.f, 0.f};
        if (r < nvalid) vv = load4<TIn>(vb + r * rsV + c4);
        const float bt = sbeta[r];
        st4(&sq[r][c4], float4{bt * vv.x, bt * vv.y, bt * vv.z, bt * vv.w});
    }
    __syncthreads();
    float* Wp = Wo + (size_t)ch * C * DK;
    for (int idx = w; idx < NB * (DK / 16); idx += 4) {
        const int ti = idx / (DK / 16), tj = idx % (DK / 16);
        f32x4 acc = mma16<MT_F32>(zero4(), &sT[ti * 16 * PC], PC, 1, &sY[0][tj * 16], PD, 1, 16 * (ti + 1));
#pragma unroll
        for (int r = 0; r < 4; ++r) Wp[(ti * 16 + acc_row(r)) * DK + tj * 16 + acc_col()] = acc[r];
    }
    float* Up = Uo + (size_t)ch * C * DV;
    for (int idx = w; idx < NB * (DV / 16); idx += 4) {
        const int ti = idx / (DV / 16), tj = idx % (DV / 16);
        f32x4 acc = mma16<MT_F32>(zero4(), &sT[ti * 16 * PC], PC, 1, &sq[0][tj * 16], PD, 1, 16 * (ti + 1));
#pragma unroll
        for (int r = 0; r < 4; ++r) Up[(ti * 16 + acc_row(r)) * DV + tj * 16 + acc_col()] = acc[r];
    }
}

// ---------------------------------------------------------------------------
// scan
// ---------------------------------------------------------------------------
template <int DV>
struct ScanCfg {
    static constexpr int BV = DV >= 32 ? 32 : DV;  // Dv columns per workgroup
    static constexpr int NS = DV / BV;              // slices per (b, h)
    static constexpr int PS = BV + 4;               // LDS pitch of [*][BV] tiles
};

template <typename TIn, int C, int DK, int DV, int MT, bool SAVE, bool OUT>
__global__ void __launch_bounds__(NTHR)
scan_kernel(const float* __restrict__ Wi, const float* __restrict__ Ui,
            const float* __restrict__ Qgi, const float* __restrict__ Khi,
            const float* __restrict__ Psi, const float* __restrict__ gami,
            const float* __restrict__ h0, TIn* __restrict__ o, float* __restrict__ hT,
            float* __restrict__ Sst, int BH, int T, int H, int NC)
{
    using G = Geo<C, DK, DV>;
    using SC = ScanCfg<DV>;
    constexpr int PD = G::PD, PC = G::PC, BV = SC::BV, NS = SC::NS, PS = SC::PS;
    __shared__ float sS[DK][PS], sW[C][PD], sQ[C][PD], sK[C][PD], sP[C][PC], sD[C][PS], sg[DK];

    // XCD-aware id: the NS slices of one (b, h) share blockIdx % 8
    const int x = blockIdx.x;
    const int grp = x / (8 * NS), rem = x % (8 * NS);
    const int sl = rem / 8, bh = grp * 8 + rem % 8;
    if (bh >= BH) return;
    const int b = bh / H, h = bh % H;
    const int v0 = sl * BV;
    const int tid = threadIdx.x, w = tid >> 6;

    for (int idx = tid; idx < DK * BV; idx += NTHR) {
        const int i = idx / BV, j = idx % BV;
        sS[i][j] = h0 ? h0[((size_t)bh * DK + i) * DV + v0 + j] : 0.f;
    }
    __syncthreads();

    constexpr int TD = (C / 16) * (BV / 16);   // D / O tiles
    constexpr int TS = (DK / 16) * (BV / 16);  // state tiles
    constexpr int MD = (TD + 3) / 4, MS = (TS + 3) / 4;

    for (int n = 0; n < NC; ++n) {
        const size_t ch = (size_t)bh * NC + n;
        if (SAVE) {
            float* Sp = Sst + ch * DK * DV;
            for (int idx = tid; idx < DK * BV; idx += NTHR) {
                const int i = idx / BV, j = idx % BV;
                Sp[i * DV + v0 + j] = sS[i][j];
            }
        }
        {
            const float* Wp = Wi + ch * C * DK;
            const float* Qp = Qgi + ch * C * DK;
            const float* Kp = Khi + ch * C * DK;
            for (int idx = tid; idx < C * DK / 4; idx += NTHR) {
                const int r = idx / (DK / 4), c4 = (idx % (DK / 4)) * 4;
                st4(&sW[r][c4], load4<float>(Wp + r * DK + c4));
                if (OUT) st4(&sQ[r][c4], load4<float>(Qp + r * DK + c4));
                st4(&sK[r][c4], load4<float>(Kp + r * DK + c4));
            }
            if (OUT) {
                const float* Pp = Psi + ch * C * C;
                for (int idx = tid; idx < C * C / 4; idx += NTHR) {
                    const int r = idx / (C / 4), c4 = (idx % (C / 4)) * 4;
                    st4(&sP[r][c4], load4<float>(Pp + r * C + c4));
                }
            }
            for (int i = tid; i < DK; i += NTHR) sg[i] = gami[ch * DK + i];
        }
        __syncthreads();

        f32x4 o1[MD];
        const float* Up = Ui + ch * C * DV;
#pragma unroll
        for (int m = 0; m < MD; ++m) {
            const int idx = w + 4 * m;
            if (idx < TD) {
                const int ti = idx / (BV / 16), tj = idx % (BV / 16);
                f32x4 ws = mma16k<MT, DK>(zero4(), &sW[ti * 16][0], PD, 1, &sS[0][tj * 16], PS, 1);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = ti * 16 + acc_row(r), j = tj * 16 + acc_col();
                    sD[i][j] = Up[i * DV + v0 + j] - ws[r];
                }
                if (OUT) o1[m] = mma16k<MT, DK>(zero4(), &sQ[ti * 16][0], PD, 1, &sS[0][tj * 16], PS, 1);
            }
        }
        __syncthreads();
        if (OUT) {
#pragma unroll
            for (int m = 0; m < MD; ++m) {
                const int idx = w + 4 * m;
                if (idx < TD) {
                    const int ti = idx / (BV / 16), tj = idx % (BV / 16);
                    f32x4 acc = mma16<MT>(o1[m], &sP[ti * 16][0], PC, 1, &sD[0][tj * 16], PS, 1, 16 * (ti + 1));
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = ti * 16 + acc_row(r), j = tj * 16 + acc_col();
                        const int t = n * C + i;
                        if (t < T) o[(((size_t)b * T + t) * H + h) * DV + v0 + j] = from_f32<TIn>(acc[r]);
                    }
                }
            }
        }
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
                    acc[r] = sg[i] * sS[i][sj * 16 + acc_col()];
                }
                sn[m] = mma16k<MT, C>(acc, &sK[0][si * 16], 1, PD, &sD[0][sj * 16], PS, 1);
            }
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < MS; ++m) {
            const int idx = w + 4 * m;
            if (idx < TS) {
                const int si = idx / (BV / 16), sj = idx % (BV / 16);
#pragma unroll
                for (int r = 0; r < 4; ++r) sS[si * 16 + acc_row(r)][sj * 16 + acc_col()] = sn[m][r];
            }
        }
        __syncthreads();
    }
    if (hT) {
        for (int idx = tid; idx < DK * BV; idx += NTHR) {
            const int i = idx / BV, j = idx % BV;
            hT[((size_t)bh * DK + i) * DV + v0 + j] = sS[i][j];
        }
    }
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
template <typename TIn, int C, int DK, int DV, int MT>
gdn_status run_prep(const Plan& p, const void* q, const void* k, const void* v, const float* g,
                    const float* beta, char* ws, bool want_T, hipStream_t st)
{
    float* W = (float*)(ws + p.o_W);
    float* U = (float*)(ws + p.o_U);
    float* Qg = (float*)(ws + p.o_Qg);
    float* Kh = (float*)(ws + p.o_Kh);
    float* Ps = (float*)(ws + p.o_Ps);
    float* gam = (float*)(ws + p.o_gam);
    float* Tm = want_T ? (float*)(ws + p.o_Tm) : nullptr;
    dim3 grid((unsigned)p.n_ch), block(NTHR);
    if (p.decay == GDN_DECAY_PER_CHANNEL)
        GDN_LAUNCH(want_T ? "prep_T" : "prep", (prep_kernel<TIn, C, DK, DV, true, MT>), grid, block, st,
                           (const TIn*)q, (const TIn*)k, (const TIn*)v, g, beta, p.T, p.H, p.NC,
                           p.scale, W, U, Qg, Kh, Ps, gam, Tm);
    else
        GDN_LAUNCH(want_T ? "prep_T" : "prep", (prep_kernel<TIn, C, DK, DV, false, MT>), grid, block, st,
                           (const TIn*)q, (const TIn*)k, (const TIn*)v, g, beta, p.T, p.H, p.NC,
                           p.scale, W, U, Qg, Kh, Ps, gam, Tm);
    GDN_HIP_CHECK_LAUNCH();
    return GDN_OK;
}

template <typename TIn, int C, int DK, int DV, int MT, bool SAVE, bool OUT>
gdn_status run_scan(const Plan& p, const float* h0, void* o, float* hT, char* ws, hipStream_t st)
{
    using SC = ScanCfg<DV>;
    const int BH = p.B * p.H;
    const int ngrp = (BH + 7) / 8;
    dim3 grid((unsigned)(ngrp * 8 * SC::NS)), block(NTHR);
    GDN_LAUNCH(SAVE ? (OUT ? "scan_train" : "scan_save") : "scan", (scan_kernel<TIn, C, DK, DV, MT, SAVE, OUT>), grid, block, st,
                       (const float*)(ws + p.o_W), (const float*)(ws + p.o_U),
                       (const float*)(ws + p.o_Qg), (const float*)(ws + p.o_Kh),
                       (const float*)(ws + p.o_Ps), (const float*)(ws + p.o_gam), h0, (TIn*)o, hT,
                       SAVE ? (float*)(ws + p.o_Sst) : nullptr, BH, p.T, p.H, p.NC);
    GDN_HIP_CHECK_LAUNCH();
    return GDN_OK;
}

template <typename TIn, int C, int DK, int DV>
gdn_status forward_t(const Plan& p, const void* q, const void* k, const void* v, const float* g,
                     const float* beta, const float* h0, void* o, float* hT, char* ws,
                     hipStream_t st)
{
    constexpr int MT = std::is_same<TIn, bf16>::value ? MT_BF16 : MT_F32;
    gdn_status s = run_prep<TIn, C, DK, DV, MT>(p, q, k, v, g, beta, ws, false, st);
    if (s != GDN_OK) return s;
    return run_scan<TIn, C, DK, DV, MT, false, true>(p, h0, o, hT, ws, st);
}

template <typename TIn>
gdn_status forward_dt(const Plan& p, const void* q, const void* k, const void* v, const float* g,
                      const float* beta, const float* h0, void* o, float* hT, char* ws,
                      hipStream_t st)
{
#define GDN_FWD(C_, D_)                                                                  \
    if (p.C == C_ && p.Dk == D_ && p.Dv == D_)                                            \
        return forward_t<TIn, C_, D_, D_>(p, q, k, v, g, beta, h0, o, hT, ws, st);
    GDN_FWD(64, 128) GDN_FWD(64, 64) GDN_FWD(16, 16)
#undef GDN_FWD
    return GDN_ERR_UNSUPPORTED;
}

gdn_status forward_dispatch(const Plan& p, const void* q, const void* k, const void* v,
                            const float* g, const float* beta, const float* h0, void* o, float* hT,
                            void* ws, hipStream_t st)
{
    if (p.dtype == GDN_BF16)
        return forward_dt<bf16>(p, q, k, v, g, beta, h0, o, hT, (char*)ws, st);
    return forward_dt<float>(p, q, k, v, g, beta, h0, o, hT, (char*)ws, st);
}

// Forward recompute for the backward pass: the prep outputs (with T) and the
// state at the start of every chunk; no outputs are written.  With `out`, the
// same pass also writes o and hT (the training forward, which leaves these
// residuals in the workspace for the backward).
template <typename TIn, int C, int DK, int DV>
gdn_status recompute_t(const Plan& p, const void* q, const void* k, const void* v, const float* g,
                       const float* beta, const float* h0, void* o, float* hT, bool out, char* ws,
                       hipStream_t st)
{
    constexpr int MT = std::is_same<TIn, bf16>::value ? MT_BF16 : MT_F32;
    gdn_status s = run_prep<TIn, C, DK, DV, MT>(p, q, k, v, g, beta, ws, true, st);
    if (s != GDN_OK) return s;
    if (out) return run_scan<TIn, C, DK, DV, MT, true, true>(p, h0, o, hT, ws, st);
    return run_scan<TIn, C, DK, DV, MT, true, false>(p, h0, nullptr, nullptr, ws, st);
}

gdn_status recompute_dispatch(const Plan& p, const void* q, const void* k, const void* v,
                              const float* g, const float* beta, const float* h0, void* o,
                              float* hT, bool out, void* ws, hipStream_t st)
{
#define GDN_REC(C_, D_)                                                                        \
    if (p.C == C_ && p.Dk == D_ && p.Dv == D_)                                                  \
        return p.dtype == GDN_BF16                                                              \
                   ? recompute_t<bf16, C_, D_, D_>(p, q, k, v, g, beta, h0, o, hT, out,         \
                                                   (char*)ws, st)                               \
                   : recompute_t<float, C_, D_, D_>(p, q, k, v, g, beta, h0, o, hT, out,        \
                                                    (char*)ws, st);
    GDN_REC(64, 128) GDN_REC(64, 64) GDN_REC(16, 16)
#undef GDN_REC
    return GDN_ERR_UNSUPPORTED;
}

}  // namespace gdn
