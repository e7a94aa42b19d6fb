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
#include "swz.h"
#include "plan.h"

namespace gdn {

// ---------------------------------------------------------------------------
// prep (fp32 tables; the chunk-16 configurations: chunk 64 runs prep2 or prepf)
// ---------------------------------------------------------------------------
template <typename TIn, int C, int DK, int DV, bool PCH, int MT>
__global__ void __launch_bounds__(NTHR)
prep_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
            const float* __restrict__ g, const float* __restrict__ beta, int T, int H, int NC,
            float scale, float* __restrict__ Wo, float* __restrict__ Uo, float* __restrict__ Qgo,
            float* __restrict__ Kho, float* __restrict__ Pso, float* __restrict__ gamo,
            float* __restrict__ Tmo, float* __restrict__ rno, Safety sf)
{
    static_assert(!bf16_tables<TIn, C, DK>() && !f32_tables<TIn, C, DK>(), "chunk 64 runs prep2 or prepf");
    using G = Geo<C, DK, DV>;
    constexpr int PD = G::PD, PC = G::PC, NB = G::NB, HALF = G::HALF;
    __shared__ float sq[C][PD], sk[C][PD], sX[C][PD], sY[C][PD], sA[C][PC];
    __shared__ float sbeta[C], sdiag[C], stot[2][DK], sRn[2 * C];
    __shared__ unsigned int sdg[NDIAG_PREP];  // stage counts (clip or diag set)

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
    const bool safe = sf.on();
    if (tid < NDIAG_PREP) sdg[tid] = 0u;
    auto grd = [&](float x, int stage) {
        return safe ? guard(x, sf.clip, sf.diag ? &sdg[2 * stage] : nullptr) : x;
    };

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

    // ---- use_qk_l2norm (rno set): every q and k row scaled by
    // r = 1/sqrt(|x|^2 + eps) in place; r kept in rno for the backward
    if (rno) {
        for (int r = tid; r < 2 * C; r += NTHR) {
            const float* row = r < C ? &sq[r][0] : &sk[r - C][0];
            float s = 0.f;
            for (int cc = 0; cc < DK; ++cc) {
                const float x = row[(cc + r) % DK];  // skewed to spread LDS banks
                s += x * x;
            }
            const float rr = 1.f / sqrtf(s + GDN_L2NORM_EPS);
            sRn[r] = rr;
            rno[(size_t)ch * 2 * C + r] = rr;
        }
        __syncthreads();
        for (int idx = tid; idx < C * DK; idx += NTHR) {
            const int r = idx / DK, cc = idx % DK;
            sq[r][cc] *= sRn[r];
            sk[r][cc] *= sRn[C + r];
        }
        __syncthreads();
    }

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
    auto put_ps = [&](int i0, int j, const float (&pv)[4]) {  // rows i0..i0+3, column j
#pragma unroll
        for (int r = 0; r < 4; ++r) Ps[(i0 + r) * C + j] = pv[r];
    };
#pragma unroll
    for (int s = 0; s < G::MAXOFF; ++s) {
        const int idx = w + 4 * s;
        if (idx < G::NOFF) {
            int ti, tj;
            off_tile(idx, ti, tj);
            float pv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = ti * 16 + acc_row(r), j = tj * 16 + acc_col();
                pv[r] = scale * grd(accP[s][r], GDN_DIAG_P);
                sA[i][j] = grd(sbeta[i] * accA[s][r], GDN_DIAG_A);
            }
            put_ps(ti * 16 + acc_row(0), tj * 16 + acc_col(), pv);
        }
    }
    if (w < NB) {
        const int t = w;
        float pv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = t * 16 + acc_row(r), j = t * 16 + acc_col();
            pv[r] = scale * (i > j ? grd(dP[r], GDN_DIAG_P) : (i == j ? grd(sdiag[i], GDN_DIAG_P) : 0.f));
            sA[i][j] = i > j ? grd(sbeta[i] * dA[r], GDN_DIAG_A) : 0.f;
        }
        put_ps(t * 16 + acc_row(0), t * 16 + acc_col(), pv);
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
        float qgv[HALF], khv[HALF];
#pragma unroll
        for (int i = 0; i < HALF; ++i) {
            const int r = part * HALF + i;
            Gm *= a[i];
            qgv[i] = scale * sq[r][c] * Gm;
            sY[r][c] = sbeta[r] * sk[r][c] * Gm;
        }
        if (part == 1) gamo[(size_t)ch * DK + c] = Gm;
        float kap = part ? 1.f : stot[1][c];
#pragma unroll
        for (int i = HALF - 1; i >= 0; --i) {
            const int r = part * HALF + i;
            khv[i] = sk[r][c] * kap;
            kap *= a[i];
        }
        float* Qg = Qgo + (size_t)ch * C * DK;
        float* Kh = Kho + (size_t)ch * C * DK;
#pragma unroll
        for (int i = 0; i < HALF; ++i) {
            Qg[(part * HALF + i) * DK + c] = qgv[i];
            Kh[(part * HALF + i) * DK + c] = khv[i];
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
                x[i] = s * sf.dinv;  // diagonal (1 + wy_eps)
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
    if (safe) {  // the solve's output crosses a stage boundary
        for (int idx = tid; idx < C * C; idx += NTHR) {
            float* t = &sT[(idx / C) * PC + idx % C];
            *t = grd(*t, GDN_DIAG_T);
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
        for (int r = 0; r < 4; ++r) acc[r] = grd(acc[r], GDN_DIAG_W);
#pragma unroll
        for (int r = 0; r < 4; ++r) Wp[(ti * 16 + acc_row(r)) * DK + tj * 16 + acc_col()] = acc[r];
    }
    float* Up = Uo + (size_t)ch * C * DV;
    for (int idx = w; idx < NB * (DV / 16); idx += 4) {
        const int ti = idx / (DV / 16), tj = idx % (DV / 16);
        f32x4 acc = mma16<MT_F32>(zero4(), &sT[ti * 16 * PC], PC, 1, &sq[0][tj * 16], PD, 1, 16 * (ti + 1));
#pragma unroll
        for (int r = 0; r < 4; ++r) Up[(ti * 16 + acc_row(r)) * DV + tj * 16 + acc_col()] = grd(acc[r], GDN_DIAG_U);
    }
    if (safe) {
        __syncthreads();
        flush_counts(sdg, sf.diag, NDIAG_PREP);
    }
}


// ---------------------------------------------------------------------------
// prep over bf16 tables (bf16 inputs, chunk 64): 8 waves.  A column thread
// owns one key channel of one 16-token tile and keeps its q, k and exp(g) in
// registers; the level tables are bf16 rows with the channel index contiguous
// (one 16-byte LDS read per MFMA operand); the diagonal scores are a chain of
// the unscaled rows kept on the diagonal; W = T X_K is a bf16 MFMA product
// with X_K^T written by the column threads; U = T X_V likewise, with X_V^T =
// (beta V)^T stashed into the level-table bytes once T is done.  v is loaded
// right after the level loop, before any table store: a load issued after
// them would wait for them (one completion counter for loads and stores).
// With L2N (use_qk_l2norm) every q and k row is scaled by r = 1/sqrt(|x|^2 +
// eps): the squared lengths are the diagonals of the Q Q^T and K K^T tiles of
// the raw rows, r is folded into the products of raw rows and into the rows
// each thread keeps, and r goes to rno for the backward.
// With SAFE (clip or diag) the stage values P, A, T, U, W pass through guard();
// the solve's diagonal is damped by sf.dinv = 1 / (1 + wy_eps) in every instance.
// Wro (training with clip): W also before clipping, which the backward's WY
// adjoint needs (clipping is differentiated as the identity).
// ---------------------------------------------------------------------------
constexpr int NTHR_P = 512;

template <int C, int DK, int DV, bool PCH, bool L2N, bool SAFE>
__global__ void __launch_bounds__(NTHR_P, 4)
prep2_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
             const float* __restrict__ g, const float* __restrict__ beta, int T, int H, int NC,
             float scale, bf16* __restrict__ Wb, float* __restrict__ Uo,
             bf16* __restrict__ Qgb, bf16* __restrict__ KhTb, bf16* __restrict__ Psb,
             float* __restrict__ gamo, float* __restrict__ Tmo, float* __restrict__ rno,
             Safety sf, bf16* __restrict__ Wro)
{
    static_assert(C == 64 && DK == DV, "prep2: chunk 64, Dk == Dv");
    constexpr int NW = NTHR_P / 64, RPP = 16, NPART = C / RPP, NB = C / 16;
    constexpr int PA = DK + 8, PT = C + 8, PC = C + 4;
    constexpr int NOFF = NB * (NB - 1) / 2;
    // level tables; after the level loop the same bytes hold T and the merge scratch (fp32)
    constexpr int SBUF = cmax(2 * C * PA * 2, 2 * C * PC * 4);
    __shared__ __align__(16) char sbuf[SBUF];
    __shared__ __align__(16) float sA[C][PC];  // A (beta rows), strictly lower; later T in bf16
    // X_K^T, channel rows (SwzR8): a column thread writes its rows of one
    // channel as two 16-byte units, the W product reads 16-byte row fragments
    __shared__ __align__(16) uint4 sXT[DK * C / 8];
    __shared__ float sbeta[C], stot[NPART][DK];
    __shared__ float sG[C];  // per-head decay: chunk-local inclusive cumsum of g
    __shared__ float sRn[2][L2N ? C : 1];  // L2N: 1/sqrt(|q_i|^2 + eps), same for k
    __shared__ unsigned int sdg[SAFE ? NDIAG_PREP : 1];  // SAFE: this workgroup's stage counts
    // level tables, channel-major (rows = key channels, columns = tokens; SwzT8):
    // a column thread writes its rows of one channel as whole 16-byte units,
    // and the score products read them with transposing loads
    uint4* const sX = reinterpret_cast<uint4*>(sbuf);
    uint4* const sY = reinterpret_cast<uint4*>(sbuf + DK * C * 2);
    static_assert(2 * DK * C * 2 <= SBUF && RPP % 8 == 0, "channel-major level tables");
    float (*sT)[PC] = reinterpret_cast<float (*)[PC]>(sbuf);
    float (*sYt)[PC] = reinterpret_cast<float (*)[PC]>(sbuf + C * PC * 4);
    // T in bf16 over sA once T is formed (SwzR8 rows; 16-byte row-fragment reads)
    uint4* const sTb = reinterpret_cast<uint4*>(&sA[0][0]);
    static_assert(C * C * 2 <= (int)sizeof(sA), "bf16 T fits sA");

    const int ch = blockIdx.x;
    const int n = ch % NC, bh = ch / NC, h = bh % H, b = bh / H;
    const int t0 = n * C;
    const int nvalid = min(C, T - t0);
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int lr = l & 15, lq = l >> 4;
    const size_t tok0 = ((size_t)b * T + t0) * H + h;
    const size_t rsK = (size_t)H * DK;
    const bool bwdt = Tmo != nullptr;
    const bool cp = tid < NPART * DK;
    const int c = tid % DK, part = cp ? tid / DK : 0, p0 = part * RPP;
    // this thread's rows of channel c in a level table (row i's value x(i)),
    // 8 at a time
    auto put_rows = [&](uint4* tab, auto x) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < RPP; i += 8) {
            const uint2 lo = pack4_bf16(x(i), x(i + 1), x(i + 2), x(i + 3));
            const uint2 hi = pack4_bf16(x(i + 4), x(i + 5), x(i + 6), x(i + 7));
            tab[swz_slot<SwzT8>(c, (p0 + i) / 8)] = uint4{lo.x, lo.y, hi.x, hi.y};
        }
    };
    // 16 x 16 score tile: rows ti*16.. of table A against rows tj*16.. of table
    // B, summed over the DK channels
    auto cm_prod = [&](f32x4 acc, const uint4* A, int ti, const uint4* B, int tj) {
#pragma unroll 2
        for (int k0 = 0; k0 < DK; k0 += 32)
            acc = mfma_bf16_16x16x32(frag_cols<SwzT8>(A, k0, ti * 16), frag_cols<SwzT8>(B, k0, tj * 16), acc);
        return acc;
    };
    if (SAFE && tid < NDIAG_PREP) sdg[tid] = 0u;
    auto sd = [&](int stage) -> unsigned int* { return SAFE && sf.diag ? &sdg[2 * stage] : nullptr; };
    auto grd = [&](float x, int stage) { return SAFE ? guard(x, sf.clip, sd(stage)) : x; };

    float a[RPP], qv[RPP], kv[RPP];
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
        a[i] = fast_exp(ok ? gx : 0.f);
        qv[i] = ok ? qx : 0.f;
        kv[i] = ok ? kx : 0.f;
    }
    for (int r = tid; r < C; r += NTHR_P) sbeta[r] = r < nvalid ? beta[tok0 + (size_t)r * H] : 0.f;
    {
        float pt = 1.f;
#pragma unroll
        for (int i = 0; i < RPP; ++i) pt *= a[i];
        if (cp) stot[part][c] = pt;
    }
    if constexpr (!PCH) {
        static_assert(C == 64, "one token per lane of wave 0");
        if (w == 0) {  // G_i = g_0 + ... + g_i, inclusive prefix sum across the wave
            float x = l < nvalid ? g[tok0 + (size_t)min(l, nvalid - 1) * H] : 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(x, off);
                if (l >= off) x += y;
            }
            sG[l] = x;
        }
    }
    // level 0: unscaled rows, the diagonal P_ii = q_i . k_i
    if (cp) {
        put_rows(sX, [&](int i) { return qv[i]; });
        put_rows(sY, [&](int i) { return kv[i]; });
    }
    __syncthreads();
    // L2N, waves w < NB: squared lengths of rows 16w.. from the raw tables
    // (published to sRn by the next barrier)
    auto row_norms = [&]() {
        if constexpr (L2N) {
            const f32x4 nq = cm_prod(zero4(), sX, w, sX, w);
            const f32x4 nk = cm_prod(zero4(), sY, w, sY, w);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (4 * lq + r == lr) {
                    const int i = w * 16 + lr;
                    const float rq = 1.f / sqrtf(nq[r] + GDN_L2NORM_EPS);
                    const float rk = 1.f / sqrtf(nk[r] + GDN_L2NORM_EPS);
                    sRn[0][i] = rq;
                    sRn[1][i] = rk;
                    rno[((size_t)ch * 2) * C + i] = rq;
                    rno[((size_t)ch * 2 + 1) * C + i] = rk;
                }
            }
        }
    };
    // L2N, after the barrier that publishes sRn: the rows this thread keeps
    auto scale_rows = [&]() {
        if constexpr (L2N) {
#pragma unroll
            for (int i = 0; i < RPP; ++i) {
                qv[i] *= sRn[0][p0 + i];
                kv[i] *= sRn[1][p0 + i];
            }
        }
    };
    f32x4 dP = zero4(), dA = zero4();
    // off-diagonal 16-tiles: waves NB.. own tile idx with (idx % (NW - NB)) == w - NB
    // (per-head decay)
    constexpr int OW = NW - NB, MOFF = (NOFF + OW - 1) / OW;
    // Per-channel decay: the P (= X Y^T) and A (= Y Y^T) products of each level
    // are spread over all eight waves, one product a wave: level 32's tiles
    // (2,0) (2,1) (3,0) (3,1), level 16's (1,0) (3,2) (waves 0-3), and at the
    // levels below the four diagonal tiles
    static_assert(C == 64 && NW == 8, "four 16-tiles a chunk, eight waves");
    const int pa = w & 1;                                      // 0: P, 1: A
    const int ti32 = 2 + (w >> 2), tj32 = (w >> 1) & 1;        // level-32 tile
    const int ti16 = (w >> 1) == 0 ? 1 : 3, tj16 = ti16 - 1;   // level-16 tile (waves 0-3)
    const int td = w & 3, pd = w >> 2;                         // diagonal tile and product
    f32x4 a32 = zero4(), a16 = zero4(), ad = zero4();
    f32x4 accP[MOFF], accA[MOFF];
#pragma unroll
    for (int m = 0; m < MOFF; ++m) accP[m] = accA[m] = zero4();
    if constexpr (!PCH) {
        // Per-head decay: the decay between tokens j <= i is the scalar
        // exp(G_i - G_j) <= 1, the same for every key channel, so each score is
        // the plain product q_i . k_j (or k_i . k_j) times it: one MFMA product
        // per 16-tile instead of the block-boundary split.
        if (w < NB) {
            const f32x4 tp = cm_prod(zero4(), sX, w, sY, w);
            const f32x4 ta = cm_prod(zero4(), sY, w, sY, w);
            row_norms();
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 4 * lq + r, j = lr;
                const float e = j <= i ? fast_exp(sG[w * 16 + i] - sG[w * 16 + j]) : 0.f;
                dP[r] = tp[r] * e;
                dA[r] = j < i ? ta[r] * e : 0.f;
            }
        } else {
#pragma unroll
            for (int m = 0; m < MOFF; ++m) {
                const int idx = (w - NB) + OW * m;
                if (idx < NOFF) {
                    int ti, tj;
                    off_tile(idx, ti, tj);
                    accP[m] = cm_prod(zero4(), sX, ti, sY, tj);
                    accA[m] = cm_prod(zero4(), sY, ti, sY, tj);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float e = fast_exp(sG[ti * 16 + 4 * lq + r] - sG[tj * 16 + lr]);
                        accP[m][r] *= e;
                        accA[m][r] *= e;
                    }
                }
            }
        }
        __syncthreads();
        if constexpr (L2N) {  // products of raw rows times r_i r_j
            if (w < NB) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = w * 16 + 4 * lq + r, j = w * 16 + lr;
                    dP[r] *= sRn[0][i] * sRn[1][j];
                    dA[r] *= sRn[1][i] * sRn[1][j];
                }
            } else {
#pragma unroll
                for (int m = 0; m < MOFF; ++m) {
                    const int idx = (w - NB) + OW * m;
                    if (idx < NOFF) {
                        int ti, tj;
                        off_tile(idx, ti, tj);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int i = ti * 16 + 4 * lq + r, j = tj * 16 + lr;
                            accP[m][r] *= sRn[0][i] * sRn[1][j];
                            accA[m][r] *= sRn[1][i] * sRn[1][j];
                        }
                    }
                }
            }
            scale_rows();
        }
    } else {
    if (w < NB) {  // waves 0-3 hold the diagonal P tiles (pd = 0, td = w)
        const f32x4 tp = cm_prod(zero4(), sX, w, sY, w);
        row_norms();
#pragma unroll
        for (int r = 0; r < 4; ++r) ad[r] = (4 * lq + r == lr) ? tp[r] : 0.f;
    }
    __syncthreads();
    if constexpr (L2N) {
        if (w < NB) {  // P_ii of the raw rows times r_q r_k
            const int i = w * 16 + lr;
#pragma unroll
            for (int r = 0; r < 4; ++r) ad[r] *= sRn[0][i] * sRn[1][i];
        }
    }
    scale_rows();  // the level tables below are built from the normalised rows

#pragma unroll
    for (int lvl = 0; (C >> (lvl + 1)) >= 1; ++lvl) {
        const int hl = C >> (lvl + 1);
        float F[RPP];
        if (hl >= RPP) {
            const int base = (p0 / (2 * hl)) * (2 * hl);
            if (p0 >= base + hl) {
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
        } else {
#pragma unroll
            for (int u0 = 0; u0 < RPP; u0 += (hl < RPP ? hl : RPP)) {
                if (((p0 + u0) / hl) & 1) {
                    float Fr = 1.f;
#pragma unroll
                    for (int i = 0; i < hl; ++i) {
                        Fr *= a[u0 + i];
                        F[u0 + i] = Fr;
                    }
                } else {
                    float Fr = 1.f;
#pragma unroll
                    for (int i = hl - 1; i >= 0; --i) {
                        F[u0 + i] = Fr;
                        Fr *= a[u0 + i];
                    }
                }
            }
        }
        if (cp) {
            put_rows(sX, [&](int i) { return qv[i] * F[i]; });
            put_rows(sY, [&](int i) { return kv[i] * F[i]; });
        }
        __syncthreads();
        if (hl == 32) {
            a32 = cm_prod(a32, pa ? sY : sX, ti32, sY, tj32);
        } else if (hl == 16) {
            if (w < 4) a16 = cm_prod(a16, pa ? sY : sX, ti16, sY, tj16);
        } else {
            const f32x4 t = cm_prod(zero4(), pd ? sY : sX, td, sY, td);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (in_level(4 * lq + r, lr, hl)) ad[r] += t[r];
        }
        __syncthreads();
    }
    }  // per-channel decay


    // v rows for U = T X_V at the end, loaded before any table store (a load
    // issued after them would wait for them: one completion counter for loads
    // and stores) and after the level loop (kept out of its registers); rows
    // past the end are clamped here and zeroed through beta = 0
    constexpr int NV8 = C * DV / 8, QV = NV8 / NTHR_P;
    static_assert(QV * NTHR_P == NV8, "whole v words per thread");
    uint4 vw[QV];
#pragma unroll
    for (int u = 0; u < QV; ++u) {
        const int idx = tid + NTHR_P * u, r = idx / (DV / 8), j0 = (idx % (DV / 8)) * 8;
        vw[u] = *reinterpret_cast<const uint4*>(v + tok0 * DV + (size_t)min(r, nvalid - 1) * H * DV + j0);
    }

    // ---- scores out: Ps (bf16); A (x beta) to LDS.  Ps is staged in the
    // level-table bytes (free after the score products) and leaves as whole
    // rows, 16 bytes per thread
    bf16 (*sPs)[PT] = reinterpret_cast<bf16 (*)[PT]>(sbuf);
    static_assert(C * PT * 2 <= SBUF, "staged Ps fits the level-table bytes");
    bf16* Psc = Psb + (size_t)ch * C * C;
    auto put_ps = [&](int i0, int j, const float (&pv)[4]) {
#pragma unroll
        for (int r = 0; r < 4; ++r) sPs[i0 + r][j] = f32_to_bf16(pv[r]);
    };
    if constexpr (PCH) {
        // one P or A item of a tile: P scaled into the staging, A times beta to sA;
        // on the diagonal P keeps j <= i and A j < i
        auto put_item = [&](int ti, int tj, int prod, const f32x4& acc, bool diag) {
            if (prod == 0) {
                float pv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = ti * 16 + 4 * lq + r, j = tj * 16 + lr;
                    pv[r] = (!diag || i >= j) ? scale * grd(acc[r], GDN_DIAG_P) : 0.f;
                }
                put_ps(ti * 16 + 4 * lq, tj * 16 + lr, pv);
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = ti * 16 + 4 * lq + r, j = tj * 16 + lr;
                    sA[i][j] = (!diag || i > j) ? grd(sbeta[i] * acc[r], GDN_DIAG_A) : 0.f;
                }
            }
        };
        put_item(ti32, tj32, pa, a32, false);
        if (w < 4) put_item(ti16, tj16, pa, a16, false);
        put_item(td, td, pd, ad, true);
    } else if (w >= NB) {
#pragma unroll
        for (int m = 0; m < MOFF; ++m) {
            const int idx = (w - NB) + OW * m;
            if (idx < NOFF) {
                int ti, tj;
                off_tile(idx, ti, tj);
                float pv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = ti * 16 + 4 * lq + r, j = tj * 16 + lr;
                    pv[r] = scale * grd(accP[m][r], GDN_DIAG_P);
                    sA[i][j] = grd(sbeta[i] * accA[m][r], GDN_DIAG_A);
                }
                put_ps(ti * 16 + 4 * lq, tj * 16 + lr, pv);
            }
        }
    } else {
        const int t = w;
        float pv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = t * 16 + 4 * lq + r, j = t * 16 + lr;
            pv[r] = i >= j ? scale * grd(dP[r], GDN_DIAG_P) : 0.f;
            sA[i][j] = i > j ? grd(sbeta[i] * dA[r], GDN_DIAG_A) : 0.f;
        }
        put_ps(t * 16 + 4 * lq, t * 16 + lr, pv);
    }
    for (int idx = tid; idx < C * C; idx += NTHR_P) {
        const int i = idx / C, j = idx % C;
        if (i / 16 < j / 16) {
            sPs[i][j] = f32_to_bf16(0.f);
            sA[i][j] = 0.f;
        }
    }
    __syncthreads();  // staged Ps rows complete
    for (int idx = tid; idx < C * C / 8; idx += NTHR_P) {
        const int r = idx / (C / 8), c0 = (idx % (C / 8)) * 8;
        *reinterpret_cast<uint4*>(&Psc[r * C + c0]) = *reinterpret_cast<const uint4*>(&sPs[r][c0]);
    }
    __syncthreads();  // the staged Ps rows are read: Qg takes their bytes

    // ---- Gamma, Kh factor, gam: Qg, Kh^T outputs and X_K^T = (beta K o Gamma)^T.
    // Qg rows are staged in the level-table bytes (free after the score
    // products) and leave as whole rows, 16 bytes per thread, instead of one
    // 2-byte store per row and thread.
    bf16 (*sQs)[PA] = reinterpret_cast<bf16 (*)[PA]>(sbuf);
    static_assert(C * PA * 2 <= SBUF, "staged Qg fits the level-table bytes");
    bf16* Qgc = Qgb + (size_t)ch * C * DK;
    if (cp) {
        float pre = 1.f, suf = 1.f;
        for (int pp = 0; pp < part; ++pp) pre *= stot[pp][c];
        for (int pp = part + 1; pp < NPART; ++pp) suf *= stot[pp][c];
        float qg[RPP], kh[RPP], xk[RPP];
        float Gm = pre;
#pragma unroll
        for (int i = 0; i < RPP; ++i) {
            Gm *= a[i];
            qg[i] = scale * qv[i] * Gm;
            xk[i] = sbeta[p0 + i] * kv[i] * Gm;
        }
        if (part == NPART - 1) gamo[(size_t)ch * DK + c] = Gm;
        float kap = suf;
#pragma unroll
        for (int i = RPP - 1; i >= 0; --i) {
            kh[i] = kv[i] * kap;
            kap *= a[i];
        }
        bf16* KhTc = KhTb + (size_t)ch * C * DK;
#pragma unroll
        for (int i = 0; i < RPP; ++i) sQs[p0 + i][c] = f32_to_bf16(qg[i]);
        // a thread's 16 rows of one channel are 32 contiguous bytes of the
        // transposed tables: two 16-byte stores each
#pragma unroll
        for (int i = 0; i < RPP; i += 8) {
            const uint2 k0 = pack4_bf16(kh[i], kh[i + 1], kh[i + 2], kh[i + 3]);
            const uint2 k1 = pack4_bf16(kh[i + 4], kh[i + 5], kh[i + 6], kh[i + 7]);
            *reinterpret_cast<uint4*>(&KhTc[c * C + p0 + i]) = uint4{k0.x, k0.y, k1.x, k1.y};
        }
#pragma unroll
        for (int i = 0; i < RPP; i += 8) {
            const uint2 lo = pack4_bf16(xk[i], xk[i + 1], xk[i + 2], xk[i + 3]);
            const uint2 hi = pack4_bf16(xk[i + 4], xk[i + 5], xk[i + 6], xk[i + 7]);
            sXT[swz_slot<SwzR8>(c, (p0 + i) / 8)] = uint4{lo.x, lo.y, hi.x, hi.y};
        }
    }
    __syncthreads();  // staged rows complete
    for (int idx = tid; idx < C * DK / 8; idx += NTHR_P) {
        const int r = idx / (DK / 8), c0 = (idx % (DK / 8)) * 8;
        *reinterpret_cast<uint4*>(&Qgc[r * DK + c0]) = *reinterpret_cast<const uint4*>(&sQs[r][c0]);
    }
    __syncthreads();  // the staged rows are read: sT takes their bytes
    for (int idx = tid; idx < C * PC; idx += NTHR_P) (&sT[0][0])[idx] = 0.f;
    __syncthreads();

    // ---- WY solve: 16x16 diagonal blocks of (I + A)^-1 by forward substitution
    if (w == 0) {
        const int bb = lq, j = lr;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float sacc = (i == j) ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < i; ++m) sacc -= sA[bb * 16 + i][bb * 16 + m] * x[m];
            x[i] = sacc * sf.dinv;  // diagonal (1 + wy_eps)
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sT[bb * 16 + i][bb * 16 + j] = x[i];
    }
    __syncthreads();
    // merge neighbouring diagonal blocks: T21 = -T22 (A21 T11)
#pragma unroll
    for (int sz = 16; 2 * sz <= C; sz *= 2) {
        const int tps = (sz / 16) * (sz / 16);
        const int ntile = (C / (2 * sz)) * tps;
        for (int idx = w; idx < ntile; idx += NW) {
            const int pi = idx / tps, ti = (idx % tps) / (sz / 16), tj = idx % (sz / 16);
            const int b0 = pi * 2 * sz;
            f32x4 y = mma16<MT_F32>(zero4(), &sA[b0 + sz + 16 * ti][b0], PC, 1, &sT[b0][b0 + 16 * tj], PC, 1, sz);
#pragma unroll
            for (int r = 0; r < 4; ++r) sYt[b0 + sz + 16 * ti + 4 * lq + r][b0 + 16 * tj + lr] = y[r];
        }
        __syncthreads();
        for (int idx = w; idx < ntile; idx += NW) {
            const int pi = idx / tps, ti = (idx % tps) / (sz / 16), tj = idx % (sz / 16);
            const int b0 = pi * 2 * sz;
            f32x4 t21 = mma16<MT_F32>(zero4(), &sT[b0 + sz + 16 * ti][b0 + sz], PC, 1, &sYt[b0 + sz][b0 + 16 * tj], PC, 1, sz);
#pragma unroll
            for (int r = 0; r < 4; ++r) sT[b0 + sz + 16 * ti + 4 * lq + r][b0 + 16 * tj + lr] = -t21[r];
        }
        __syncthreads();
    }
    // T out (fp32, training) and its bf16 copy (over sA, no longer needed)
    for (int idx = tid; idx < C * C / 4; idx += NTHR_P) {  // 4 consecutive columns per thread
        const int i = idx / (C / 4), j = (idx % (C / 4)) * 4;
        float tv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) tv[e] = grd(sT[i][j + e], GDN_DIAG_T);
        if (bwdt) *reinterpret_cast<float4*>(&Tmo[(size_t)ch * C * C + i * C + j]) = float4{tv[0], tv[1], tv[2], tv[3]};
        *reinterpret_cast<uint2*>(swz_at<SwzR8>(sTb, i, j)) = pack4_bf16(tv[0], tv[1], tv[2], tv[3]);
    }
    __syncthreads();
    // X_V = beta V (token rows) into the level-table bytes (free now that T is
    // in sTb), one 16-byte word per store; the U product reads it transposed
    using SXV = std::conditional_t<DV == 128, SwzV16, SwzT8>;
    static_assert(SXV::U * 8 == DV && C * DV * 2 <= SBUF, "X_V fits the level-table bytes");
    uint4* const sXV = reinterpret_cast<uint4*>(sbuf);
#pragma unroll
    for (int u = 0; u < QV; ++u) {
        const int idx = tid + NTHR_P * u, r = idx / (DV / 8), j0 = (idx % (DV / 8)) * 8;
        const float bt = sbeta[r];
        const uint32_t wd[4] = {vw[u].x, vw[u].y, vw[u].z, vw[u].w};
        uint32_t xw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            xw[e] = cvt2_bf16(bt * __uint_as_float(wd[e] << 16), bt * __uint_as_float(wd[e] & 0xFFFF0000u));
        sXV[swz_slot<SXV>(r, j0 / 8)] = uint4{xw[0], xw[1], xw[2], xw[3]};
    }
    // ---- W = T X_K (bf16 out).  The tile of W^T = X_K^T T^T: a lane holds 4
    // consecutive columns of one W row, one 8-byte store
    constexpr int TW = NB * (DK / 16);
    for (int idx = w; idx < TW; idx += NW) {
        const int ti = idx / (DK / 16), tj = idx % (DK / 16);
        const int K = ((16 * (ti + 1) + 31) / 32) * 32;  // T is lower triangular
        f32x4 acc = zero4();
        for (int k0 = 0; k0 < K; k0 += 32)
            acc = mfma_bf16_16x16x32(frag_rows<SwzR8>(sXT, tj * 16, k0 / 8), frag_rows<SwzR8>(sTb, ti * 16, k0 / 8), acc);
        const size_t e = (size_t)ch * C * DK + (ti * 16 + lr) * DK + tj * 16 + 4 * lq;
        if (SAFE && Wro) *reinterpret_cast<uint2*>(&Wro[e]) = pack4_bf16(acc[0], acc[1], acc[2], acc[3]);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = grd(acc[r], GDN_DIAG_W);
        *reinterpret_cast<uint2*>(&Wb[e]) = pack4_bf16(acc[0], acc[1], acc[2], acc[3]);
    }
    __syncthreads();  // X_V^T complete
    // ---- U = T X_V (fp32 out).
    // The tile of U^T = X_V^T T^T: a lane holds 4 consecutive columns of one U row
    constexpr int TU = NB * (DV / 16);
    float* Uc = Uo + (size_t)ch * C * DV;
    for (int idx = w; idx < TU; idx += NW) {
        const int ti = idx / (DV / 16), tj = idx % (DV / 16);
        const int K = ((16 * (ti + 1) + 31) / 32) * 32;  // T is lower triangular
        f32x4 acc = zero4();
        for (int k0 = 0; k0 < K; k0 += 32)
            acc = mfma_bf16_16x16x32(frag_cols<SXV>(sXV, k0, tj * 16), frag_rows<SwzR8>(sTb, ti * 16, k0 / 8), acc);
        const size_t e = (size_t)(ti * 16 + lr) * DV + tj * 16 + 4 * lq;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = grd(acc[r], GDN_DIAG_U);
        *reinterpret_cast<float4*>(&Uc[e]) = float4{acc[0], acc[1], acc[2], acc[3]};
    }
    if constexpr (SAFE) {
        __syncthreads();
        flush_counts(sdg, sf.diag, NDIAG_PREP);
    }
}

// ---------------------------------------------------------------------------
// prepf: prep over fp32 tables (fp32 inputs, chunk 64) on
// v_mfma_f32_16x16x4_f32, with prep2's structure: 8 waves; a column thread
// owns one key channel of one 16-token part and keeps its q, k and exp(g) in
// registers; the level tables are fp32 rows with the channel index contiguous
// on the fp32 row swizzle (one 16-byte LDS read per lane per four MFMAs).  The
// score tiles, W and U are computed transposed (P^T = Y X^T and so on), so a
// lane's four values are four consecutive columns of one output row, stored
// as 16 bytes.  Kh goes out transposed (Kh^T [DK][C]).  exp is the library
// expf throughout.  With SAFE the stage values P, A, T, U, W pass through
// guard(); the solve's diagonal is damped by sf.dinv in every instance.
// ---------------------------------------------------------------------------
template <int C, int DK, int DV, bool PCH, bool L2N, bool SAFE>
__global__ void __launch_bounds__(NTHR_P)
prepf_kernel(const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
             const float* __restrict__ g, const float* __restrict__ beta, int T, int H, int NC,
             float scale, float* __restrict__ Wo, float* __restrict__ Uo,
             float* __restrict__ Qgo, float* __restrict__ KhTo, float* __restrict__ Pso,
             float* __restrict__ gamo, float* __restrict__ Tmo, float* __restrict__ rno, Safety sf)
{
    static_assert(C == 64 && DK == DV && (DK == 64 || DK == 128), "prepf: chunk 64, Dk == Dv");
    constexpr int NW = NTHR_P / 64, RPP = 16, NPART = C / RPP, NB = C / 16;
    constexpr int PC = C + 4, UK = DK / 4, UC = C / 4;
    constexpr int NOFF = NB * (NB - 1) / 2;
    using SK = SwzF<UK>;  // rows of DK floats
    using SC = SwzF<UC>;  // rows of C floats
    // level tables (fp32, swizzled); after the level loop the same bytes hold
    // T and the merge scratch, then X_V^T
    constexpr int SBUF = cmax(2 * C * DK * 4, cmax(2 * C * PC * 4, DV * C * 4));
    __shared__ __align__(16) char sbuf[SBUF];
    __shared__ __align__(16) float sA[C][PC];  // A (beta rows), strictly lower; later T (swizzled)
    __shared__ __align__(16) f32x4 sXT[DK * UC];  // X_K^T [DK][C]
    __shared__ float sbeta[C], stot[NPART][DK];
    __shared__ float sG[C];  // per-head decay: chunk-local inclusive cumsum of g
    __shared__ float sRn[2][L2N ? C : 1];
    __shared__ unsigned int sdg[SAFE ? NDIAG_PREP : 1];
    f32x4* const sX = reinterpret_cast<f32x4*>(sbuf);
    f32x4* const sY = reinterpret_cast<f32x4*>(sbuf + C * DK * 4);
    float* const Xf = reinterpret_cast<float*>(sX);
    float* const Yf = reinterpret_cast<float*>(sY);
    float (*sT)[PC] = reinterpret_cast<float (*)[PC]>(sbuf);
    float (*sYt)[PC] = reinterpret_cast<float (*)[PC]>(sbuf + C * PC * 4);
    f32x4* const sTs = reinterpret_cast<f32x4*>(&sA[0][0]);  // T [C][C] swizzled (SC)
    static_assert(C * C * 4 <= C * PC * 4, "swizzled T fits the A bytes");

    const int ch = blockIdx.x;
    const int n = ch % NC, bh = ch / NC, h = bh % H, b = bh / H;
    const int t0 = n * C;
    const int nvalid = min(C, T - t0);
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int lr = l & 15, lq = l >> 4;
    const size_t tok0 = ((size_t)b * T + t0) * H + h;
    const size_t rsK = (size_t)H * DK;
    const bool bwdt = Tmo != nullptr;
    const bool cp = tid < NPART * DK;
    const int c = tid % DK, part = cp ? tid / DK : 0, p0 = part * RPP;
    if (SAFE && tid < NDIAG_PREP) sdg[tid] = 0u;
    auto sd = [&](int stage) -> unsigned int* { return SAFE && sf.diag ? &sdg[2 * stage] : nullptr; };
    auto grd = [&](float x, int stage) { return SAFE ? guard(x, sf.clip, sd(stage)) : x; };
    // Y_a X_b^T over the key channels: acc[r] = sum_c Y[a0 + 4 lq + r][c] X[b0 + lr][c]
    auto kc = [&](f32x4 acc, const f32x4* A, int a0, const f32x4* B, int b0) {
#pragma unroll
        for (int u0 = 0; u0 < UK; u0 += 4) acc = mma_f32_k16(ffrag_rows<SK>(A, a0, u0), ffrag_rows<SK>(B, b0, u0), acc);
        return acc;
    };

    float a[RPP], qv[RPP], kv[RPP];
#pragma unroll
    for (int i = 0; i < RPP; ++i) {
        const int r = p0 + i;
        const int rr = min(r, nvalid - 1);
        const float gx = PCH ? g[(tok0 + (size_t)rr * H) * DK + c] : g[tok0 + (size_t)rr * H];
        const float qx = q[tok0 * DK + rr * rsK + c];
        const float kx = k[tok0 * DK + rr * rsK + c];
        const bool ok = cp && r < nvalid;
        a[i] = expf(ok ? gx : 0.f);
        qv[i] = ok ? qx : 0.f;
        kv[i] = ok ? kx : 0.f;
    }
    for (int r = tid; r < C; r += NTHR_P) sbeta[r] = r < nvalid ? beta[tok0 + (size_t)r * H] : 0.f;
    {
        float pt = 1.f;
#pragma unroll
        for (int i = 0; i < RPP; ++i) pt *= a[i];
        if (cp) stot[part][c] = pt;
    }
    if constexpr (!PCH) {
        if (w == 0) {  // G_i = g_0 + ... + g_i, inclusive prefix sum across the wave
            float x = l < nvalid ? g[tok0 + (size_t)min(l, nvalid - 1) * H] : 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(x, off);
                if (l >= off) x += y;
            }
            sG[l] = x;
        }
    }
    // level 0: unscaled rows
    if (cp) {
#pragma unroll
        for (int i = 0; i < RPP; ++i) {
            Xf[swzf_idx<SK>(p0 + i, c)] = qv[i];
            Yf[swzf_idx<SK>(p0 + i, c)] = kv[i];
        }
    }
    __syncthreads();
    auto row_norms = [&]() {
        if constexpr (L2N) {
            const f32x4 nq = kc(zero4(), sX, w * 16, sX, w * 16);
            const f32x4 nk = kc(zero4(), sY, w * 16, sY, w * 16);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (4 * lq + r == lr) {
                    const int i = w * 16 + lr;
                    const float rq = 1.f / sqrtf(nq[r] + GDN_L2NORM_EPS);
                    const float rk = 1.f / sqrtf(nk[r] + GDN_L2NORM_EPS);
                    sRn[0][i] = rq;
                    sRn[1][i] = rk;
                    rno[((size_t)ch * 2) * C + i] = rq;
                    rno[((size_t)ch * 2 + 1) * C + i] = rk;
                }
            }
        }
    };
    auto scale_rows = [&]() {
        if constexpr (L2N) {
#pragma unroll
            for (int i = 0; i < RPP; ++i) {
                qv[i] *= sRn[0][p0 + i];
                kv[i] *= sRn[1][p0 + i];
            }
        }
    };
    // score tiles, transposed: acc[r] = P[ti*16 + lr][tj*16 + 4 lq + r] (and A)
    f32x4 dP = zero4(), dA = zero4();
    constexpr int OW = NW - NB, MOFF = (NOFF + OW - 1) / OW;
    f32x4 accP[MOFF], accA[MOFF];
#pragma unroll
    for (int m = 0; m < MOFF; ++m) accP[m] = accA[m] = zero4();
    if constexpr (!PCH) {
        // per head: plain products times exp(G_i - G_j) (<= 1 for j <= i)
        if (w < NB) {
            const f32x4 tp = kc(zero4(), sY, w * 16, sX, w * 16);
            const f32x4 ta = kc(zero4(), sY, w * 16, sY, w * 16);
            row_norms();
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = lr, j = 4 * lq + r;
                const float e = j <= i ? expf(sG[w * 16 + i] - sG[w * 16 + j]) : 0.f;
                dP[r] = tp[r] * e;
                dA[r] = j < i ? ta[r] * e : 0.f;
            }
        } else {
#pragma unroll
            for (int m = 0; m < MOFF; ++m) {
                const int idx = (w - NB) + OW * m;
                if (idx < NOFF) {
                    int ti, tj;
                    off_tile(idx, ti, tj);
                    accP[m] = kc(zero4(), sY, tj * 16, sX, ti * 16);
                    accA[m] = kc(zero4(), sY, tj * 16, sY, ti * 16);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float e = expf(sG[ti * 16 + lr] - sG[tj * 16 + 4 * lq + r]);
                        accP[m][r] *= e;
                        accA[m][r] *= e;
                    }
                }
            }
        }
        __syncthreads();
        if constexpr (L2N) {
            if (w < NB) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = w * 16 + lr, j = w * 16 + 4 * lq + r;
                    dP[r] *= sRn[0][i] * sRn[1][j];
                    dA[r] *= sRn[1][i] * sRn[1][j];
                }
            } else {
#pragma unroll
                for (int m = 0; m < MOFF; ++m) {
                    const int idx = (w - NB) + OW * m;
                    if (idx < NOFF) {
                        int ti, tj;
                        off_tile(idx, ti, tj);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int i = ti * 16 + lr, j = tj * 16 + 4 * lq + r;
                            accP[m][r] *= sRn[0][i] * sRn[1][j];
                            accA[m][r] *= sRn[1][i] * sRn[1][j];
                        }
                    }
                }
            }
            scale_rows();
        }
    } else {
    if (w < NB) {
        const f32x4 tp = kc(zero4(), sY, w * 16, sX, w * 16);
        row_norms();
#pragma unroll
        for (int r = 0; r < 4; ++r) dP[r] = (4 * lq + r == lr) ? tp[r] : 0.f;
    }
    __syncthreads();
    if constexpr (L2N) {
        if (w < NB) {
            const int i = w * 16 + lr;
#pragma unroll
            for (int r = 0; r < 4; ++r) dP[r] *= sRn[0][i] * sRn[1][i];
        }
    }
    scale_rows();

#pragma unroll
    for (int lvl = 0; (C >> (lvl + 1)) >= 1; ++lvl) {
        const int hl = C >> (lvl + 1);
        float F[RPP];
        if (hl >= RPP) {
            const int base = (p0 / (2 * hl)) * (2 * hl);
            if (p0 >= base + hl) {
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
        } else {
#pragma unroll
            for (int u0 = 0; u0 < RPP; u0 += (hl < RPP ? hl : RPP)) {
                if (((p0 + u0) / hl) & 1) {
                    float Fr = 1.f;
#pragma unroll
                    for (int i = 0; i < hl; ++i) {
                        Fr *= a[u0 + i];
                        F[u0 + i] = Fr;
                    }
                } else {
                    float Fr = 1.f;
#pragma unroll
                    for (int i = hl - 1; i >= 0; --i) {
                        F[u0 + i] = Fr;
                        Fr *= a[u0 + i];
                    }
                }
            }
        }
        if (cp) {
#pragma unroll
            for (int i = 0; i < RPP; ++i) {
                Xf[swzf_idx<SK>(p0 + i, c)] = qv[i] * F[i];
                Yf[swzf_idx<SK>(p0 + i, c)] = kv[i] * F[i];
            }
        }
        __syncthreads();
        if (hl >= 16) {
            if (w >= NB) {
#pragma unroll
                for (int m = 0; m < MOFF; ++m) {
                    const int idx = (w - NB) + OW * m;
                    if (idx < NOFF) {
                        int ti, tj;
                        off_tile(idx, ti, tj);
                        if (off_tile_level(ti, tj) == hl) {
                            accP[m] = kc(accP[m], sY, tj * 16, sX, ti * 16);
                            accA[m] = kc(accA[m], sY, tj * 16, sY, ti * 16);
                        }
                    }
                }
            }
        } else if (w < NB) {
            const f32x4 tp = kc(zero4(), sY, w * 16, sX, w * 16);
            const f32x4 ta = kc(zero4(), sY, w * 16, sY, w * 16);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (in_level(lr, 4 * lq + r, hl)) {
                    dP[r] += tp[r];
                    dA[r] += ta[r];
                }
            }
        }
        __syncthreads();
    }
    }  // per-channel decay

    // v rows for U at the end (clamped past the end, zeroed through beta = 0)
    constexpr int NV4 = C * DV / 4, QV = NV4 / NTHR_P;
    static_assert(QV * NTHR_P == NV4, "whole v words per thread");
    f32x4 vw[QV];
#pragma unroll
    for (int u = 0; u < QV; ++u) {
        const int idx = tid + NTHR_P * u, r = idx / (DV / 4), j0 = (idx % (DV / 4)) * 4;
        vw[u] = *reinterpret_cast<const f32x4*>(v + tok0 * DV + (size_t)min(r, nvalid - 1) * H * DV + j0);
    }

    // ---- scores out: Ps rows (16 bytes a lane), A (x beta) to LDS
    float* Psc = Pso + (size_t)ch * C * C;
    if (w >= NB) {
#pragma unroll
        for (int m = 0; m < MOFF; ++m) {
            const int idx = (w - NB) + OW * m;
            if (idx < NOFF) {
                int ti, tj;
                off_tile(idx, ti, tj);
                const int i = ti * 16 + lr, j0 = tj * 16 + 4 * lq;
                f32x4 pv, av;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    pv[r] = scale * grd(accP[m][r], GDN_DIAG_P);
                    av[r] = grd(sbeta[i] * accA[m][r], GDN_DIAG_A);
                }
                *reinterpret_cast<f32x4*>(&Psc[i * C + j0]) = pv;
                *reinterpret_cast<f32x4*>(&sA[i][j0]) = av;
            }
        }
    } else {
        const int i = w * 16 + lr, j0 = w * 16 + 4 * lq;
        f32x4 pv, av;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = j0 + r;
            pv[r] = i >= j ? scale * grd(dP[r], GDN_DIAG_P) : 0.f;
            av[r] = i > j ? grd(sbeta[i] * dA[r], GDN_DIAG_A) : 0.f;
        }
        *reinterpret_cast<f32x4*>(&Psc[i * C + j0]) = pv;
        *reinterpret_cast<f32x4*>(&sA[i][j0]) = av;
    }
    for (int idx = tid; idx < C * C / 4; idx += NTHR_P) {  // tiles above the diagonal
        const int i = idx / (C / 4), j0 = (idx % (C / 4)) * 4;
        if (i / 16 < j0 / 16) {
            *reinterpret_cast<f32x4*>(&Psc[i * C + j0]) = zero4();
            *reinterpret_cast<f32x4*>(&sA[i][j0]) = zero4();
        }
    }

    // ---- Gamma, Kh factor, gam: Qg, Kh^T outputs and X_K^T = (beta K o Gamma)^T
    if (cp) {
        float pre = 1.f, suf = 1.f;
        for (int pp = 0; pp < part; ++pp) pre *= stot[pp][c];
        for (int pp = part + 1; pp < NPART; ++pp) suf *= stot[pp][c];
        float qg[RPP], kh[RPP], xk[RPP];
        float Gm = pre;
#pragma unroll
        for (int i = 0; i < RPP; ++i) {
            Gm *= a[i];
            qg[i] = scale * qv[i] * Gm;
            xk[i] = sbeta[p0 + i] * kv[i] * Gm;
        }
        if (part == NPART - 1) gamo[(size_t)ch * DK + c] = Gm;
        float kap = suf;
#pragma unroll
        for (int i = RPP - 1; i >= 0; --i) {
            kh[i] = kv[i] * kap;
            kap *= a[i];
        }
        float* Qgc = Qgo + (size_t)ch * C * DK;
#pragma unroll
        for (int i = 0; i < RPP; ++i) Qgc[(p0 + i) * DK + c] = qg[i];
        float* KhTc = KhTo + (size_t)ch * C * DK;
#pragma unroll
        for (int i = 0; i < RPP; i += 4) {
            *reinterpret_cast<f32x4*>(&KhTc[c * C + p0 + i]) = f32x4{kh[i], kh[i + 1], kh[i + 2], kh[i + 3]};
            sXT[swz_slot<SC>(c, (p0 + i) / 4)] = f32x4{xk[i], xk[i + 1], xk[i + 2], xk[i + 3]};
        }
    }
    __syncthreads();  // the level tables are free: sT takes their bytes
    for (int idx = tid; idx < C * PC; idx += NTHR_P) (&sT[0][0])[idx] = 0.f;
    __syncthreads();

    // ---- WY solve: 16x16 diagonal blocks of (I + A)^-1 by forward substitution
    if (w == 0) {
        const int bb = lq, j = lr;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float sacc = (i == j) ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < i; ++m) sacc -= sA[bb * 16 + i][bb * 16 + m] * x[m];
            x[i] = sacc * sf.dinv;  // diagonal (1 + wy_eps)
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sT[bb * 16 + i][bb * 16 + j] = x[i];
    }
    __syncthreads();
    // merge neighbouring diagonal blocks: T21 = -T22 (A21 T11)
#pragma unroll
    for (int sz = 16; 2 * sz <= C; sz *= 2) {
        const int tps = (sz / 16) * (sz / 16);
        const int ntile = (C / (2 * sz)) * tps;
        for (int idx = w; idx < ntile; idx += NW) {
            const int pi = idx / tps, ti = (idx % tps) / (sz / 16), tj = idx % (sz / 16);
            const int b0 = pi * 2 * sz;
            f32x4 y = mma16<MT_F32>(zero4(), &sA[b0 + sz + 16 * ti][b0], PC, 1, &sT[b0][b0 + 16 * tj], PC, 1, sz);
#pragma unroll
            for (int r = 0; r < 4; ++r) sYt[b0 + sz + 16 * ti + 4 * lq + r][b0 + 16 * tj + lr] = y[r];
        }
        __syncthreads();
        for (int idx = w; idx < ntile; idx += NW) {
            const int pi = idx / tps, ti = (idx % tps) / (sz / 16), tj = idx % (sz / 16);
            const int b0 = pi * 2 * sz;
            f32x4 t21 = mma16<MT_F32>(zero4(), &sT[b0 + sz + 16 * ti][b0 + sz], PC, 1, &sYt[b0 + sz][b0 + 16 * tj], PC, 1, sz);
#pragma unroll
            for (int r = 0; r < 4; ++r) sT[b0 + sz + 16 * ti + 4 * lq + r][b0 + 16 * tj + lr] = -t21[r];
        }
        __syncthreads();
    }
    // T out (training) and its swizzled copy over sA (no longer needed)
    for (int idx = tid; idx < C * C / 4; idx += NTHR_P) {
        const int i = idx / (C / 4), j = (idx % (C / 4)) * 4;
        f32x4 tv;
#pragma unroll
        for (int e = 0; e < 4; ++e) tv[e] = grd(sT[i][j + e], GDN_DIAG_T);
        if (bwdt) *reinterpret_cast<f32x4*>(&Tmo[(size_t)ch * C * C + i * C + j]) = tv;
        sTs[swz_slot<SC>(i, j / 4)] = tv;
    }
    __syncthreads();
    // X_V = beta V (token rows) into the level-table bytes (free now that T is
    // in sTs), one 16-byte word per store; the U product reads it down its
    // columns (transposed 4-byte writes were 8-way bank conflicted)
    using SV = SwzF<DV / 4>;  // rows of DV floats
    static_assert(C * DV * 4 <= SBUF, "X_V fits the level-table bytes");
    f32x4* const sXV = reinterpret_cast<f32x4*>(sbuf);
#pragma unroll
    for (int u = 0; u < QV; ++u) {
        const int idx = tid + NTHR_P * u, r = idx / (DV / 4), j0 = (idx % (DV / 4)) * 4;
        sXV[swz_slot<SV>(r, j0 / 4)] = sbeta[r] * vw[u];
    }
    // ---- W^T = X_K^T T^T: acc[r] = W[ti*16 + lr][tj*16 + 4 lq + r]
    constexpr int TW = NB * (DK / 16);
    float* Wc = Wo + (size_t)ch * C * DK;
    for (int idx = w; idx < TW; idx += NW) {
        const int ti = idx / (DK / 16), tj = idx % (DK / 16);
        f32x4 acc = zero4();
        for (int u0 = 0; u0 < 4 * (ti + 1); u0 += 4)  // T lower triangular
            acc = mma_f32_k16(ffrag_rows<SC>(sXT, tj * 16, u0), ffrag_rows<SC>(sTs, ti * 16, u0), acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = grd(acc[r], GDN_DIAG_W);
        *reinterpret_cast<f32x4*>(&Wc[(ti * 16 + lr) * DK + tj * 16 + 4 * lq]) = acc;
    }
    __syncthreads();  // X_V^T complete
    // ---- U^T = X_V^T T^T
    constexpr int TU = NB * (DV / 16);
    float* Uc = Uo + (size_t)ch * C * DV;
    for (int idx = w; idx < TU; idx += NW) {
        const int ti = idx / (DV / 16), tj = idx % (DV / 16);
        f32x4 acc = zero4();
        for (int u0 = 0; u0 < 4 * (ti + 1); u0 += 4)
            acc = mma_f32_k16(ffrag_cols<SV>(sXV, 4 * u0, tj * 16), ffrag_rows<SC>(sTs, ti * 16, u0), acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = grd(acc[r], GDN_DIAG_U);
        *reinterpret_cast<f32x4*>(&Uc[(ti * 16 + lr) * DV + tj * 16 + 4 * lq]) = acc;
    }
    if constexpr (SAFE) {
        __syncthreads();
        flush_counts(sdg, sf.diag, NDIAG_PREP);
    }
}

// ---------------------------------------------------------------------------
// scan (fp32 tables; the chunk-16 configurations: chunk 64 runs scan2, scan3
// or scanf)
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
            const float* h0, TIn* __restrict__ o, float* hT,
            float* __restrict__ Sst, int BH, int T, int H, int NC)
{
    static_assert(!bf16_tables<TIn, C, DK>() && !f32_tables<TIn, C, DK>(), "chunk 64 runs scan2, scan3 or scanf");
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
// scan2: the state-saving forward scans (training forward, backward
// recompute) over bf16 chunk tables (bf16 inputs): 8 waves; the fp32 state slice
// lives in the MFMA accumulators of its owner waves for the whole sequence,
// its bf16 copy S^T [BV][DK] in LDS is the B operand of W S and Qg S; every
// operand is K-contiguous (one 16-byte LDS read per lane per MFMA); the next
// chunk's tables are fetched into registers while the current one computes.
// ---------------------------------------------------------------------------
constexpr int NTHR_S = 512;

template <int C, int DK, int DV, bool SAVE, bool OUT>
__global__ void __launch_bounds__(NTHR_S)
scan2_kernel(const bf16* __restrict__ Wb, const bf16* __restrict__ Qgb,
             const bf16* __restrict__ KhTb, const bf16* __restrict__ Psb,
             const float* __restrict__ Ui, const float* __restrict__ gami,
             const float* h0, bf16* __restrict__ o, float* hT,
             bf16* __restrict__ Sst, bf16* __restrict__ Dst, int BH, int T, int H, int NC)
{
    constexpr int BV = 32, NS = DV / BV, NW = NTHR_S / 64;
    constexpr int TD = (C / 16) * (BV / 16), TS = (DK / 16) * (BV / 16);
    constexpr int MD = (TD + NW - 1) / NW, MS = (TS + NW - 1) / NW;
    // bf16 tables as swizzled rows (swz.h): rows of DK values SA, rows of C values SC
    using SA = std::conditional_t<DK == 128, SwzU16, SwzU8w>;
    using SC = SwzU8w;
    static_assert(C == 64 && (DK == 128 || DK == 64), "row widths of the swizzles");
    // 16-byte words of one chunk's tables.  Each table is a whole number of words
    // per thread, so the table of word slot q is known at compile time and the
    // prefetch has no branches: the compiler then waits exactly for it, not also
    // for the state and output stores issued after it.
    constexpr int QW = C * DK / 8, QK = DK * C / 8, QP = C * C / 8;
    constexpr int QALL = 2 * QW + QK + QP, QPT = (QALL + NTHR_S - 1) / NTHR_S;
    static_assert(QW % NTHR_S == 0 && QK % NTHR_S == 0 && QP % NTHR_S == 0, "table split");
    static_assert(TD % NW == 0 && TS % NW == 0, "tile split");
    // W, Qg [C][DK], Kh^T [DK][C], Ps [C][C], and the bf16 copies S^T [BV][DK], D^T [BV][C]
    __shared__ __align__(16) uint4 sW[C * DK / 8], sQ[C * DK / 8], sKT[DK * C / 8], sP[C * C / 8],
        sSt[BV * DK / 8], sDt[BV * C / 8];
    // staging of each step's outputs (double-buffered by step parity), written
    // out with 16-byte stores: the next chunk's start state, D and o (bf16; the
    // saved states feed the backward's bf16 products and its decay-gradient sums)
    constexpr int PO = BV + 8;
    __shared__ __align__(16) bf16 sSf[2][DK][PO];
    // the chunk's U slice (fp32 rows, padded so the accumulator-layout reads of
    // four rows 4 apart hit distinct banks) and decay
    constexpr int PU = BV + 4;
    static_assert(C * BV / 4 == NTHR_S && DK / 4 <= NTHR_S, "one U word and at most one decay word per thread");
    __shared__ __align__(16) float sU[C][PU], sGm[DK];
    __shared__ __align__(16) bf16 sDr[2][C][PO], sOr[2][C][PO];

    const int x = blockIdx.x;
    const int grp = x / (8 * NS), rem = x % (8 * NS);
    const int sl = rem / 8, bh = grp * 8 + rem % 8;
    if (bh >= BH) return;
    const int b = bh / H, h = bh % H;
    const int v0 = sl * BV;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int lr = l & 15, lq = l >> 4;

    // state tiles owned by this wave: S[si*16 + 4lq + r][sj*16 + lr]
    f32x4 sacc[MS];
#pragma unroll
    for (int m = 0; m < MS; ++m) {
        const int idx = w + NW * m;
        sacc[m] = zero4();
        if (idx < TS) {
            const int si = idx / (BV / 16), sj = idx % (BV / 16);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sacc[m][r] = h0 ? h0[((size_t)bh * DK + si * 16 + 4 * lq + r) * DV + v0 + sj * 16 + lr] : 0.f;
            *reinterpret_cast<uint2*>(swz_at<SA>(sSt, sj * 16 + lr, si * 16 + 4 * lq)) =
                pack4_bf16(sacc[m][0], sacc[m][1], sacc[m][2], sacc[m][3]);
        }
    }

    // Two register sets of prefetched tables: chunk n + 1 arrives in one while
    // chunk n + 2 is fetched into the other, so two steps of compute cover the
    // latency.  Fetches are unconditional (the chunk index is clamped; the tail
    // re-reads the last chunk) and the loop body is a pair of steps with the
    // sets fixed, so the waits are exact.
    // U and the decay go through LDS too: one 16-byte word of each per thread
    // (the decay word repeats across threads) instead of one 4-byte load per
    // accumulator value.
    using PFW = uint4[QPT];
    using UF = float4;
    using GF = float4;
    uint4 pfA[QPT], pfB[QPT];
    float4 upA, upB, gpA, gpB;
    auto fetch = [&](int n, PFW& pf, UF& upf, GF& gpf) {  // chunk n tables -> registers
        const size_t ch = (size_t)bh * NC + n;
#pragma unroll
        for (int q = 0; q < QPT; ++q) {
            const int idx = tid + NTHR_S * q;
            uint4 val = uint4{0u, 0u, 0u, 0u};
            if (q * NTHR_S < QW) val = reinterpret_cast<const uint4*>(Wb + ch * C * DK)[idx];
            else if (q * NTHR_S < 2 * QW) val = reinterpret_cast<const uint4*>(Qgb + ch * C * DK)[idx - QW];
            else if (q * NTHR_S < 2 * QW + QK) val = reinterpret_cast<const uint4*>(KhTb + ch * C * DK)[idx - 2 * QW];
            else val = reinterpret_cast<const uint4*>(Psb + ch * C * C)[idx - 2 * QW - QK];
            pf[q] = val;
        }
        upf = load4<float>(Ui + (ch * C + tid / (BV / 4)) * DV + v0 + 4 * (tid % (BV / 4)));
        gpf = load4<float>(gami + ch * DK + 4 * (tid % (DK / 4)));
    };
    // Registers -> LDS in two halves, each written while the other half's
    // tables are read: W and Qg (read in the first phase of a step) during the
    // second phase of the step before, Kh^T and P (read in the second phase)
    // during the first phase, so a step needs two barriers.  Keep the use of
    // the prefetched words inside the stashes: hoisted into the compute phase
    // they would make it wait for the prefetch.
    auto stash_wq = [&](PFW& pf, UF& upf) {  // W and Qg words, U
        __builtin_amdgcn_sched_barrier(0);
        st4(&sU[tid / (BV / 4)][4 * (tid % (BV / 4))], upf);
#pragma unroll
        for (int q = 0; q < QPT; ++q) {
            const int idx = tid + NTHR_S * q;
            if (q * NTHR_S < QW) {
                *reinterpret_cast<uint4*>(swz_at<SA>(sW, idx / (DK / 8), (idx % (DK / 8)) * 8)) = pf[q];
            } else if (q * NTHR_S < 2 * QW) {
                const int e = idx - QW;
                *reinterpret_cast<uint4*>(swz_at<SA>(sQ, e / (DK / 8), (e % (DK / 8)) * 8)) = pf[q];
            }
        }
    };
    auto stash_kp = [&](PFW& pf, UF& upf, GF& gpf) {  // Kh^T and P words; U and gam
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < QPT; ++q) {
            const int idx = tid + NTHR_S * q;
            if (q * NTHR_S < 2 * QW) {
            } else if (q * NTHR_S < 2 * QW + QK) {
                const int e = idx - 2 * QW;
                *reinterpret_cast<uint4*>(swz_at<SC>(sKT, e / (C / 8), (e % (C / 8)) * 8)) = pf[q];
            } else {
                const int e = idx - 2 * QW - QK;
                *reinterpret_cast<uint4*>(swz_at<SC>(sP, e / (C / 8), (e % (C / 8)) * 8)) = pf[q];
            }
        }
        if (tid < DK / 4) st4(&sGm[4 * tid], gpf);
    };
    fetch(0, pfA, upA, gpA);
    fetch(min(1, NC - 1), pfB, upB, gpB);
    stash_wq(pfA, upA);
    __syncthreads();

    // Each step's outputs are staged in LDS and written with 16-byte stores after
    // the step's stash (issued before the wait for the prefetch, that wait would
    // also cover them: loads and stores share one counter).
    if (SAVE) {  // chunk 0 starts from h0
#pragma unroll
        for (int m = 0; m < MS; ++m) {
            const int idx = w + NW * m;
            const int si = idx / (BV / 16), sj = idx % (BV / 16);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Sst[slice32((size_t)bh * NC, DK, DV, si * 16 + 4 * lq + r, v0 + sj * 16 + lr)] = f32_to_bf16(sacc[m][r]);
        }
    }
    // one step: chunk n, whose W, Qg and U are in LDS; `cu` holds chunk n (its
    // Kh^T, P and decay are stashed first) and then takes chunk n + 2, `nx`
    // holds chunk n + 1 (its W, Qg and U are stashed in the second phase)
    auto step = [&](int n, PFW& pcu, UF& ucu, GF& gcu, PFW& pnx, UF& unx) {
        const size_t ch = (size_t)bh * NC + n;
        const int pb = n & 1;
        stash_kp(pcu, ucu, gcu);
        fetch(min(n + 2, NC - 1), pcu, ucu, gcu);
        // D = U - W S  and  O1 = Qg S
        f32x4 o1[MD];
#pragma unroll
        for (int m = 0; m < MD; ++m) {
            const int idx = w + NW * m;
            const int ti = idx / (BV / 16), tj = idx % (BV / 16);
            f32x4 ws = zero4();
#pragma unroll
            for (int u0 = 0; u0 < DK / 8; u0 += 4)
                ws = mfma_bf16_16x16x32(frag_rows<SA>(sW, ti * 16, u0), frag_rows<SA>(sSt, tj * 16, u0), ws);
            float dv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) dv[r] = sU[ti * 16 + 4 * lq + r][tj * 16 + lr] - ws[r];
            *reinterpret_cast<uint2*>(swz_at<SC>(sDt, tj * 16 + lr, ti * 16 + 4 * lq)) = pack4_bf16(dv[0], dv[1], dv[2], dv[3]);
            if (SAVE) {  // staged as 32-bit words of column pairs
                const uint2 wd = acc_colpairs(f32x4{dv[0], dv[1], dv[2], dv[3]});
                const int i2 = ti * 16 + 4 * lq + 2 * (lr & 1), j2 = tj * 16 + (lr & ~1);
                *reinterpret_cast<uint32_t*>(&sDr[pb][i2][j2]) = wd.x;
                *reinterpret_cast<uint32_t*>(&sDr[pb][i2 + 1][j2]) = wd.y;
            }
            if (OUT) {
                o1[m] = zero4();
#pragma unroll
                for (int u0 = 0; u0 < DK / 8; u0 += 4)
                    o1[m] = mfma_bf16_16x16x32(frag_rows<SA>(sQ, ti * 16, u0), frag_rows<SA>(sSt, tj * 16, u0), o1[m]);
            }
        }
        __syncthreads();
        stash_wq(pnx, unx);  // chunk n + 1 (at the last step a harmless repeat)
        if (OUT) {
#pragma unroll
            for (int m = 0; m < MD; ++m) {
                const int idx = w + NW * m;
                const int ti = idx / (BV / 16), tj = idx % (BV / 16);
                // P is lower triangular: columns past the tile row are zero
                const int K = ((16 * (ti + 1) + 31) / 32) * 32;
                f32x4 acc = o1[m];
                for (int u0 = 0; u0 < K / 8; u0 += 4)
                    acc = mfma_bf16_16x16x32(frag_rows<SC>(sP, ti * 16, u0), frag_rows<SC>(sDt, tj * 16, u0), acc);
                const uint2 wo = acc_colpairs(acc);
                const int i2 = ti * 16 + 4 * lq + 2 * (lr & 1), j2 = tj * 16 + (lr & ~1);
                *reinterpret_cast<uint32_t*>(&sOr[pb][i2][j2]) = wo.x;
                *reinterpret_cast<uint32_t*>(&sOr[pb][i2 + 1][j2]) = wo.y;
            }
        }
        // S <- gam o S + Kh^T D
#pragma unroll
        for (int m = 0; m < MS; ++m) {
            const int idx = w + NW * m;
            const int si = idx / (BV / 16), sj = idx % (BV / 16);
            const f32x4 gv = *reinterpret_cast<const f32x4*>(&sGm[si * 16 + 4 * lq]);
            f32x4 acc;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = gv[r] * sacc[m][r];
#pragma unroll
            for (int u0 = 0; u0 < C / 8; u0 += 4)
                acc = mfma_bf16_16x16x32(frag_rows<SC>(sKT, si * 16, u0), frag_rows<SC>(sDt, sj * 16, u0), acc);
            sacc[m] = acc;
            *reinterpret_cast<uint2*>(swz_at<SA>(sSt, sj * 16 + lr, si * 16 + 4 * lq)) =
                pack4_bf16(sacc[m][0], sacc[m][1], sacc[m][2], sacc[m][3]);
            if (SAVE) {
                const uint2 wsf = acc_colpairs(sacc[m]);
                const int i2 = si * 16 + 4 * lq + 2 * (lr & 1), j2 = sj * 16 + (lr & ~1);
                *reinterpret_cast<uint32_t*>(&sSf[pb][i2][j2]) = wsf.x;
                *reinterpret_cast<uint32_t*>(&sSf[pb][i2 + 1][j2]) = wsf.y;
            }
        }
        __syncthreads();
        // this step's stores, from the staging: the start state of chunk n + 1,
        // then D and o of chunk n (rows of BV contiguous elements)
        if (SAVE && n + 1 < NC) {
            constexpr int NF8 = DK * BV / 8;  // 16-byte words of the bf16 state slice
#pragma unroll
            for (int u = 0; u < (NF8 + NTHR_S - 1) / NTHR_S; ++u) {
                const int e = tid + NTHR_S * u;
                if (e < NF8) {
                    const int i = e / (BV / 8), j8 = (e % (BV / 8)) * 8;
                    *reinterpret_cast<uint4*>(&Sst[slice32(ch + 1, DK, DV, i, v0 + j8)]) =
                        *reinterpret_cast<const uint4*>(&sSf[pb][i][j8]);
                }
            }
        }
        {
            constexpr int NB8 = C * BV / 8;  // 16-byte words of a [C][BV] bf16 tile
            static_assert(2 * NB8 <= NTHR_S, "D and o words, one per thread");
            if (tid < NB8) {
                const int i = tid / (BV / 8), j8 = (tid % (BV / 8)) * 8;
                if (SAVE)
                    *reinterpret_cast<uint4*>(&Dst[slice32(ch, C, DV, i, v0 + j8)]) =
                        *reinterpret_cast<const uint4*>(&sDr[pb][i][j8]);
            } else if (tid < 2 * NB8) {
                const int e = tid - NB8, i = e / (BV / 8), j8 = (e % (BV / 8)) * 8;
                const int t = n * C + i;
                if (OUT && t < T)
                    *reinterpret_cast<uint4*>(&o[(((size_t)b * T + t) * H + h) * DV + v0 + j8]) =
                        *reinterpret_cast<const uint4*>(&sOr[pb][i][j8]);
            }
        }
    };
    int n = 0;
    for (; n + 1 < NC; n += 2) {
        step(n, pfA, upA, gpA, pfB, upB);
        step(n + 1, pfB, upB, gpB, pfA, upA);
    }
    if (n < NC) step(n, pfA, upA, gpA, pfB, upB);
    if (hT) {
#pragma unroll
        for (int m = 0; m < MS; ++m) {
            const int idx = w + NW * m;
            if (idx < TS) {
                const int si = idx / (BV / 16), sj = idx % (BV / 16);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    hT[((size_t)bh * DK + si * 16 + 4 * lq + r) * DV + v0 + sj * 16 + lr] = sacc[m][r];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// scan3: the forward scan without saved states (gdn_forward), over bf16 chunk
// tables.  8 waves, one (b, h, 32-wide Dv slice) per workgroup.  The fp32
// state slice lives in the MFMA accumulators of its owner waves for the whole
// sequence, computed transposed (rows along Dv): a lane's four accumulator
// values are four consecutive Dv columns of one row of S (or of o); the bf16
// copies S^T [BV][DK] and D^T [BV][C] in LDS are the K-contiguous A operands
// of the products.  Everything a chunk reads (P, W, Qg, Kh^T: the B operands;
// the U slice; the decay) goes straight from global memory into one of two
// LDS buffers (swizzled rows, one chunk ahead) by direct loads waited for
// explicitly: the loop holds no register loads, so the compiler places no
// waits of its own, and the only vector memory operations after a chunk's
// loads are the step's output stores, counted exactly.  (The state-saving
// scans keep scan2: their extra stores, issued after a register prefetch two
// chunks ahead, measured faster there.)
// ---------------------------------------------------------------------------
template <int C, int DK, int DV>
__global__ void __launch_bounds__(NTHR_S)
scan3_kernel(const bf16* __restrict__ Wb, const bf16* __restrict__ Qgb,
             const bf16* __restrict__ KhTb, const bf16* __restrict__ Psb,
             const float* __restrict__ Ui, const float* __restrict__ gami,
             const float* h0, bf16* __restrict__ o, float* hT,
             int BH, int T, int H, int NC)
{
    constexpr int BV = 32, NS = DV / BV, NW = NTHR_S / 64;
    constexpr int TD = (C / 16) * (BV / 16), TS = (DK / 16) * (BV / 16);
    constexpr int MD = TD / NW, MS = TS / NW;
    // bf16 tables as swizzled rows (swz.h): rows of DK values SA, rows of C values SC
    using SA = std::conditional_t<DK == 128, SwzU16, SwzU8w>;
    using SC = SwzU8w;
    static_assert(C == 64 && (DK == 128 || DK == 64), "row widths of the swizzles");
    static_assert(TD % NW == 0 && TS % NW == 0, "every wave owns whole tiles");
    // a buffer as 16-byte words: the four tables (row widths WC, WK), then the
    // U slice [C][BV] fp32 (BV / 4 words a row) and the decay (DK / 4 words,
    // loaded by wave 0: a whole wave of words, the upper ones repeats)
    constexpr int WC = C / 8, WK = DK / 8, WU = BV / 4;
    constexpr int OP = 0, OW = OP + C * WC, OQ = OW + C * WK, OK = OQ + C * WK, QT = OK + DK * WC;
    constexpr int OU = QT, OG = OU + C * WU, QB = OG + 64;
    constexpr int NQ = QT / NTHR_S;
    static_assert(OW % NTHR_S == 0 && OQ % NTHR_S == 0 && OK % NTHR_S == 0 && QT % NTHR_S == 0,
                  "every load instruction lies in one table");
    static_assert(C * WU == NTHR_S && WU == 8 && DK / 4 <= 64, "one U word per thread, decay in one wave");
    // two buffers, separate arrays: the compiler then sees that reads of one
    // cannot alias the direct loads into the other and does not wait for them
    __shared__ __align__(16) uint4 sTab0[QB], sTab1[QB];
    __shared__ __align__(16) uint4 sSt[BV * DK / 8], sDt[BV * C / 8];  // S^T, D^T (SA, SC)
    // 2-byte views for the transposed writes: one index expression per write
    // keeps each address a single step from its array (the alias information
    // that spares those writes a wait for the direct loads is kept)
    uint16_t* const St16 = reinterpret_cast<uint16_t*>(sSt);
    uint16_t* const Dt16 = reinterpret_cast<uint16_t*>(sDt);

    const int x = blockIdx.x;
    const int grp = x / (8 * NS), rem = x % (8 * NS);
    const int sl = rem / 8, bh = grp * 8 + rem % 8;
    if (bh >= BH) return;
    const int b = bh / H, h = bh % H;
    const int v0 = sl * BV;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int lr = l & 15, lq = l >> 4;

    // state tile m of this wave: sacc[m][r] = S[si*16 + lr][v0 + sj*16 + 4 lq + r]
    f32x4 sacc[MS];
#pragma unroll
    for (int m = 0; m < MS; ++m) {
        const int idx = w + NW * m;
        const int si = idx / (BV / 16), sj = idx % (BV / 16);
        sacc[m] = zero4();
        if (h0)
            sacc[m] = *reinterpret_cast<const f32x4*>(
                h0 + ((size_t)bh * DK + si * 16 + lr) * DV + v0 + sj * 16 + 4 * lq);
#pragma unroll
        for (int r = 0; r < 4; ++r) St16[swz_elem<SA>(sj * 16 + 4 * lq + r, si * 16 + lr)] = f32_to_bf16(sacc[m][r]).bits;
    }

    // slot tid + NTHR_S q of a buffer takes table word (row, w ^ f(row)), (row, w)
    // being the slot's place in its table (rows of DK values SA, of C values
    // SC); the U slice takes word (row, w ^ (row & 7))
    int goff[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int g0 = q * NTHR_S;
        const int wpr = (g0 >= OW && g0 < OK) ? WK : WC;
        const int s = g0 + tid - (g0 < OW ? OP : g0 < OQ ? OW : g0 < OK ? OQ : OK);
        const int row = s / wpr, wd = s % wpr;
        goff[q] = (row * wpr + (wd ^ (wpr == WK ? SA::f(row) : SC::f(row)))) * 8;
    }
    const int urow = tid / WU, uoff = urow * DV + v0 + 4 * ((tid % WU) ^ (urow & 7));
    auto fetch = [&](int n, uint4* buf) {
        const size_t ch = (size_t)bh * NC + n;
        if (w == 0) dma16(gami + ch * DK + 4 * (l % (DK / 4)), buf + OG);
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int g0 = q * NTHR_S;
            const bf16* src = g0 < OW ? Psb + ch * C * C
                            : g0 < OQ ? Wb + ch * C * DK
                            : g0 < OK ? Qgb + ch * C * DK
                                      : KhTb + ch * C * DK;
            dma16(src + goff[q], buf + g0 + 64 * w);
        }
        dma16(Ui + ch * C * DV + uoff, buf + OU + 64 * w);
    };
    // vector memory operations issued after a chunk's loads and before the
    // wait for them: the step's output stores (the last step, whose stores may
    // be skipped past T, does not wait)
    constexpr int AFTER = MD;
    static_assert(AFTER < 16, "vmcnt field");

    // chunk n sits in buffer n & 1: the steps of a pair of chunks use fixed buffers
    fetch(0, sTab0);
    wait_vmcnt<0>();
    __syncthreads();

    // LAST: the sequence's last chunk (a harmless reload of it into the idle
    // buffer, output rows past T skipped, no wait)
    auto step = [&](int n, const uint4* tb, uint4* tnx, auto last_c) {
        constexpr bool LAST = decltype(last_c)::value;
        fetch(LAST ? n : n + 1, tnx);
        // D^T = U^T - S^T W^T and O1^T = S^T Qg^T: acc[r] = D[ti*16 + lr][v0 + tj*16 + 4 lq + r]
        f32x4 o1[MD];
#pragma unroll
        for (int m = 0; m < MD; ++m) {
            const int idx = w + NW * m;
            const int ti = idx / (BV / 16), tj = idx % (BV / 16);
            f32x4 ws = zero4();
#pragma unroll
            for (int u0 = 0; u0 < WK; u0 += 4)
                ws = mfma_bf16_16x16x32(frag_rows<SA>(sSt, tj * 16, u0), frag_rows<SA>(tb + OW, ti * 16, u0), ws);
            const f32x4 u4 = *reinterpret_cast<const f32x4*>(tb + OU + (ti * 16 + lr) * WU + ((tj * 4 + lq) ^ (lr & 7)));
#pragma unroll
            for (int r = 0; r < 4; ++r) Dt16[swz_elem<SC>(tj * 16 + 4 * lq + r, ti * 16 + lr)] = f32_to_bf16(u4[r] - ws[r]).bits;
            o1[m] = zero4();
#pragma unroll
            for (int u0 = 0; u0 < WK; u0 += 4)
                o1[m] = mfma_bf16_16x16x32(frag_rows<SA>(sSt, tj * 16, u0), frag_rows<SA>(tb + OQ, ti * 16, u0), o1[m]);
        }
        __syncthreads();
        // O^T += D^T P^T (P lower triangular: columns past the tile row are zero)
#pragma unroll
        for (int m = 0; m < MD; ++m) {
            const int idx = w + NW * m;
            const int ti = idx / (BV / 16), tj = idx % (BV / 16);
            f32x4 acc = mfma_bf16_16x16x32(frag_rows<SC>(sDt, tj * 16, 0), frag_rows<SC>(tb + OP, ti * 16, 0), o1[m]);
            if (16 * (ti + 1) > 32)
                acc = mfma_bf16_16x16x32(frag_rows<SC>(sDt, tj * 16, 4), frag_rows<SC>(tb + OP, ti * 16, 4), acc);
            const int t = n * C + ti * 16 + lr;
            if (!LAST || t < T)
                *reinterpret_cast<uint2*>(o + (((size_t)b * T + t) * H + h) * DV + v0 + tj * 16 + 4 * lq) =
                    pack4_bf16(acc[0], acc[1], acc[2], acc[3]);
        }
        // S^T <- S^T o gam + D^T Kh
        const float* sg = reinterpret_cast<const float*>(tb + OG);
#pragma unroll
        for (int m = 0; m < MS; ++m) {
            const int idx = w + NW * m;
            const int si = idx / (BV / 16), sj = idx % (BV / 16);
            const float gk = sg[si * 16 + lr];
            f32x4 acc;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = gk * sacc[m][r];
#pragma unroll
            for (int u0 = 0; u0 < WC; u0 += 4)
                acc = mfma_bf16_16x16x32(frag_rows<SC>(sDt, sj * 16, u0), frag_rows<SC>(tb + OK, si * 16, u0), acc);
            sacc[m] = acc;
#pragma unroll
            for (int r = 0; r < 4; ++r) St16[swz_elem<SA>(sj * 16 + 4 * lq + r, si * 16 + lr)] = f32_to_bf16(sacc[m][r]).bits;
        }
        if constexpr (!LAST) {
            wait_vmcnt<AFTER>();  // chunk n + 1's loads have landed
            __syncthreads();
        }
    };
    int n = 0;
    for (; n + 2 < NC; n += 2) {
        step(n, sTab0, sTab1, std::false_type{});
        step(n + 1, sTab1, sTab0, std::false_type{});
    }
    if (n + 2 == NC) {
        step(n, sTab0, sTab1, std::false_type{});
        step(n + 1, sTab1, sTab0, std::true_type{});
    } else {
        step(n, sTab0, sTab1, std::true_type{});
    }
    wait_vmcnt<0>();  // the last step's reload into the idle buffer
    if (hT) {
#pragma unroll
        for (int m = 0; m < MS; ++m) {
            const int idx = w + NW * m;
            const int si = idx / (BV / 16), sj = idx % (BV / 16);
            *reinterpret_cast<f32x4*>(hT + ((size_t)bh * DK + si * 16 + lr) * DV + v0 + sj * 16 + 4 * lq) = sacc[m];
        }
    }
}

// ---------------------------------------------------------------------------
// scanf: the forward scans over fp32 chunk tables (fp32 inputs, chunk 64) on
// v_mfma_f32_16x16x4_f32.  8 waves, one (b, h, 32-wide Dv slice) per
// workgroup, the fp32 state slice in the MFMA accumulators of its owner waves
// for the whole sequence, computed transposed (a lane's four values are four
// consecutive Dv columns of one row of S, of D or of o).  S^T [BV][DK] and
// D^T [BV][C] go through LDS as the K-contiguous A operands; the tables W, Qg
// (rows t), P (rows t) and Kh^T (rows of channels) are the B operands, read
// along their rows too, so every operand read is one 16-byte LDS read per lane
// per four MFMAs, on the fp32 row swizzle (SwzF) that keeps them free of bank
// conflicts.  Per chunk, two phases split by a barrier:
//   1: D^T = U^T - S^T W^T and O1^T = S^T Qg^T   (reads W, Qg, U)
//   2: O^T = O1^T + D^T P^T and S^T <- gam S^T + D^T Kh   (reads P, Kh^T, gam)
// The tables are loaded straight into LDS by direct loads, each group while
// the other phase runs: P, Kh^T and gam of this chunk during phase 1, W, Qg and
// U of the next chunk during phase 2 (fp32 tables of two chunks do not fit the
// LDS together).  The waits count the stores issued after each group.  The
// state-saving instances also store each chunk's start state and its D.
// ---------------------------------------------------------------------------
template <int C, int DK, int DV, bool SAVE, bool OUT>
__global__ void __launch_bounds__(NTHR_S)
scanf_kernel(const float* __restrict__ Wt, const float* __restrict__ Qgt,
             const float* __restrict__ KhTt, const float* __restrict__ Pst,
             const float* __restrict__ Ui, const float* __restrict__ gami,
             const float* h0, float* __restrict__ o, float* hT, float* __restrict__ Sst,
             float* __restrict__ Dst, int BH, int T, int H, int NC)
{
    constexpr int BV = 32, NS = DV / BV, NW = NTHR_S / 64;
    constexpr int TS = (DK / 16) * (BV / 16), MS = TS / NW;
    static_assert(C == 64 && (DK == 128 || DK == 64), "chunk 64, 64 or 128 key channels");
    static_assert((C / 16) * (BV / 16) == NW && TS % NW == 0, "one D tile and whole state tiles per wave");
    using SK = SwzF<DK / 4>;  // rows of DK floats
    using SC = SwzF<C / 4>;   // rows of C floats
    constexpr int UK = DK / 4, UC = C / 4, UB = BV / 4;
    // LDS in 16-byte units.  group 1: W [C][DK], Qg [C][DK], the U slice [C][BV]
    constexpr int OW = 0, OQ = OW + C * UK, OU = OQ + C * UK, G1 = OU + C * UB;
    // group 2: P [C][C], Kh^T [DK][C], the decay (one wave of words, repeats above DK)
    constexpr int OP = G1, OK = OP + C * UC, OG = OK + DK * UC, NTAB = OG + 64;
    constexpr int NQK = C * UK / NTHR_S, NQC = DK * UC / NTHR_S, NQP = C * UC / NTHR_S;
    static_assert(C * UK % NTHR_S == 0 && C * UC % NTHR_S == 0 && C * UB == NTHR_S,
                  "every direct-load instruction lies in one table");
    static_assert(DK / 4 <= 64, "decay in one wave of words");
    __shared__ __align__(16) f32x4 tab[NTAB];
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
    // this wave's D tile (rows of D^T tj, columns ti) and state tiles (sj = tj, si)
    const int tj = w & 1, ti = w >> 1;

    // slot tid + NTHR_S q of a table takes the table's unit (row, u ^ f(row))
    int gk[NQK], gc[NQC];
#pragma unroll
    for (int q = 0; q < NQK; ++q) {
        const int s = q * NTHR_S + tid, row = s / UK, u = s % UK;
        gk[q] = (row * UK + (u ^ SK::f(row))) * 4;
    }
#pragma unroll
    for (int q = 0; q < NQC; ++q) {
        const int s = q * NTHR_S + tid, row = s / UC, u = s % UC;
        gc[q] = (row * UC + (u ^ SC::f(row))) * 4;
    }
    const int urow = tid / UB, uoff = urow * DV + v0 + 4 * ((tid % UB) ^ (urow & 7));
    auto fetch1 = [&](int n) {
        const size_t ch = (size_t)bh * NC + n;
#pragma unroll
        for (int q = 0; q < NQK; ++q) {
            dma16(Wt + ch * C * DK + gk[q], tab + OW + q * NTHR_S + 64 * w);
            dma16(Qgt + ch * C * DK + gk[q], tab + OQ + q * NTHR_S + 64 * w);
        }
        dma16(Ui + ch * C * DV + uoff, tab + OU + 64 * w);
    };
    auto fetch2 = [&](int n) {
        const size_t ch = (size_t)bh * NC + n;
        if (w == 0) dma16(gami + ch * DK + 4 * (l % (DK / 4)), tab + OG);
#pragma unroll
        for (int q = 0; q < NQP; ++q) dma16(Pst + ch * C * C + gc[q], tab + OP + q * NTHR_S + 64 * w);
#pragma unroll
        for (int q = 0; q < NQC; ++q) dma16(KhTt + ch * C * DK + gc[q], tab + OK + q * NTHR_S + 64 * w);
    };

    // state tile m: sacc[m][r] = S[si*16 + lr][v0 + tj*16 + 4 lq + r], si = ti + 4 m
    f32x4 sacc[MS];
#pragma unroll
    for (int m = 0; m < MS; ++m) {
        const int si = ti + (NW / 2) * m;
        sacc[m] = zero4();
        if (h0)
            sacc[m] = *reinterpret_cast<const f32x4*>(h0 + ((size_t)bh * DK + si * 16 + lr) * DV + v0 + tj * 16 + 4 * lq);
#pragma unroll
        for (int r = 0; r < 4; ++r) St[swzf_idx<SK>(tj * 16 + 4 * lq + r, si * 16 + lr)] = sacc[m][r];
    }
    fetch1(0);
    wait_vmcnt<0>();
    __syncthreads();

    constexpr int AFTER2 = SAVE ? MS + 1 : 0;  // stores issued after group 2 (S, D)
    constexpr int AFTER1 = OUT ? 1 : 0;    // stores issued after group 1
    auto step = [&](int n, auto last_c) {
        constexpr bool LAST = decltype(last_c)::value;
        const size_t ch = (size_t)bh * NC + n;
        fetch2(n);
        if (SAVE) {
#pragma unroll
            for (int m = 0; m < MS; ++m) {
                const int si = ti + (NW / 2) * m;
                *reinterpret_cast<f32x4*>(Sst + (ch * DK + si * 16 + lr) * DV + v0 + tj * 16 + 4 * lq) = sacc[m];
            }
        }
        // phase 1: acc[r] = D^T[tj*16 + 4 lq + r][ti*16 + lr] = D[ti*16 + lr][v0 + tj*16 + 4 lq + r]
        f32x4 ws = zero4(), o1 = zero4();
#pragma unroll
        for (int u0 = 0; u0 < UK; u0 += 4) {
            const f32x4 a = ffrag_rows<SK>(sSt, tj * 16, u0);
            ws = mma_f32_k16(a, ffrag_rows<SK>(tab + OW, ti * 16, u0), ws);
            if (OUT) o1 = mma_f32_k16(a, ffrag_rows<SK>(tab + OQ, ti * 16, u0), o1);
        }
        {
            const int ur = ti * 16 + lr;
            const f32x4 u4 = tab[OU + ur * UB + ((tj * 4 + lq) ^ (ur & 7))];
            f32x4 d;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                d[r] = u4[r] - ws[r];
                Dt[swzf_idx<SC>(tj * 16 + 4 * lq + r, ti * 16 + lr)] = d[r];
            }
            if (SAVE) *reinterpret_cast<f32x4*>(Dst + (ch * C + ur) * DV + v0 + tj * 16 + 4 * lq) = d;
        }
        wait_vmcnt<AFTER2>();  // P, Kh^T, gam of this chunk have landed
        __syncthreads();
        if constexpr (!LAST) fetch1(n + 1);
        // phase 2: O^T += D^T P^T (P lower triangular: K up to the tile's last row)
        if (OUT) {
            for (int u0 = 0; u0 < 4 * (ti + 1); u0 += 4)
                o1 = mma_f32_k16(ffrag_rows<SC>(sDt, tj * 16, u0), ffrag_rows<SC>(tab + OP, ti * 16, u0), o1);
            const int t = n * C + ti * 16 + lr;
            if (!LAST || t < T)
                *reinterpret_cast<f32x4*>(o + (((size_t)b * T + t) * H + h) * DV + v0 + tj * 16 + 4 * lq) = o1;
        }
        // S^T <- S^T o gam + D^T Kh
        const float* sg = reinterpret_cast<const float*>(tab + OG);
#pragma unroll
        for (int m = 0; m < MS; ++m) {
            const int si = ti + (NW / 2) * m;
            const float gk = sg[si * 16 + lr];
            f32x4 acc;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = gk * sacc[m][r];
#pragma unroll
            for (int u0 = 0; u0 < UC; u0 += 4)
                acc = mma_f32_k16(ffrag_rows<SC>(sDt, tj * 16, u0), ffrag_rows<SC>(tab + OK, si * 16, u0), acc);
            sacc[m] = acc;
#pragma unroll
            for (int r = 0; r < 4; ++r) St[swzf_idx<SK>(tj * 16 + 4 * lq + r, si * 16 + lr)] = acc[r];
        }
        if constexpr (!LAST) {
            wait_vmcnt<AFTER1>();  // W, Qg, U of the next chunk have landed
            __syncthreads();
        }
    };
    for (int n = 0; n + 1 < NC; ++n) step(n, std::false_type{});
    step(NC - 1, std::true_type{});
    if (hT) {
#pragma unroll
        for (int m = 0; m < MS; ++m) {
            const int si = ti + (NW / 2) * m;
            *reinterpret_cast<f32x4*>(hT + ((size_t)bh * DK + si * 16 + lr) * DV + v0 + tj * 16 + 4 * lq) = sacc[m];
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
    float* rn = p.l2n ? (float*)(ws + p.o_rn) : nullptr;
    const Safety sf{p.clip, p.dinv, p.diag ? (unsigned int*)(ws + p.o_dgc) : nullptr};
    const bool raw = want_T && p.clip > 0.f;  // the training forward keeps W unclipped too
    bf16* Wro = raw ? (bf16*)(ws + p.o_Wr) : nullptr;
    dim3 grid((unsigned)p.n_ch), block(NTHR);
    if constexpr (bf16_tables<TIn, C, DK>()) {
        bf16* Wb = (bf16*)W;
        bf16* Qb = (bf16*)Qg;
        bf16* Kb = (bf16*)Kh;
        bf16* Pb = (bf16*)Ps;
        auto launch = [&](auto pch, auto l2n, auto safe) {
            GDN_LAUNCH(want_T ? "prep_T" : "prep",
                       (prep2_kernel<C, DK, DV, decltype(pch)::value, decltype(l2n)::value,
                                     decltype(safe)::value>),
                       grid, dim3(NTHR_P), st, (const bf16*)q, (const bf16*)k, (const bf16*)v, g,
                       beta, p.T, p.H, p.NC, p.scale, Wb, U, Qb, Kb, Pb, gam, Tm, rn, sf, Wro);
            return GDN_OK;
        };
        return with_bool(p.decay == GDN_DECAY_PER_CHANNEL, [&](auto pch) {
            return with_bool(p.l2n, [&](auto l2n) {
                return with_bool(sf.on(), [&](auto safe) { return launch(pch, l2n, safe); });
            });
        });
    }
    if constexpr (f32_tables<TIn, C, DK>()) {
        auto launch = [&](auto pch, auto l2n, auto safe) {
            GDN_LAUNCH(want_T ? "prep_T" : "prep",
                       (prepf_kernel<C, DK, DV, decltype(pch)::value, decltype(l2n)::value,
                                     decltype(safe)::value>),
                       grid, dim3(NTHR_P), st, (const float*)q, (const float*)k, (const float*)v, g,
                       beta, p.T, p.H, p.NC, p.scale, W, U, Qg, Kh, Ps, gam, Tm, rn, sf);
            return GDN_OK;
        };
        return with_bool(p.decay == GDN_DECAY_PER_CHANNEL, [&](auto pch) {
            return with_bool(p.l2n, [&](auto l2n) {
                return with_bool(sf.on(), [&](auto safe) { return launch(pch, l2n, safe); });
            });
        });
    }
    if constexpr (!bf16_tables<TIn, C, DK>() && !f32_tables<TIn, C, DK>()) {
        if (p.decay == GDN_DECAY_PER_CHANNEL)
            GDN_LAUNCH(want_T ? "prep_T" : "prep", (prep_kernel<TIn, C, DK, DV, true, MT>), grid, block, st,
                       (const TIn*)q, (const TIn*)k, (const TIn*)v, g, beta, p.T, p.H, p.NC,
                       p.scale, W, U, Qg, Kh, Ps, gam, Tm, rn, sf);
        else
            GDN_LAUNCH(want_T ? "prep_T" : "prep", (prep_kernel<TIn, C, DK, DV, false, MT>), grid, block, st,
                       (const TIn*)q, (const TIn*)k, (const TIn*)v, g, beta, p.T, p.H, p.NC,
                       p.scale, W, U, Qg, Kh, Ps, gam, Tm, rn, sf);
    }
    return GDN_OK;
}

template <typename TIn, int C, int DK, int DV, int MT, bool SAVE, bool OUT>
gdn_status run_scan(const Plan& p, const float* h0, void* o, float* hT, char* ws, hipStream_t st)
{
    using SC = ScanCfg<DV>;
    const int BH = p.B * p.H;
    const int ngrp = (BH + 7) / 8;
    if constexpr (bf16_tables<TIn, C, DK>()) {
        const size_t n = p.n_ch;
        dim3 grid((unsigned)(ngrp * 8 * (DV / 32))), block(NTHR_S);
        if constexpr (!SAVE) {
            GDN_LAUNCH("scan", (scan3_kernel<C, DK, DV>), grid, block, st,
                       (const bf16*)(ws + p.o_W), (const bf16*)(ws + p.o_Qg),
                       (const bf16*)(ws + p.o_Kh), (const bf16*)(ws + p.o_Ps),
                       (const float*)(ws + p.o_U), (const float*)(ws + p.o_gam), h0, (bf16*)o, hT,
                       BH, p.T, p.H, p.NC);
        } else {
            GDN_LAUNCH(SAVE ? (OUT ? "scan_train" : "scan_save") : "scan",
                       (scan2_kernel<C, DK, DV, SAVE, OUT>), grid, block, st,
                       (const bf16*)(ws + p.o_W), (const bf16*)(ws + p.o_Qg),
                       (const bf16*)(ws + p.o_Kh), (const bf16*)(ws + p.o_Ps),
                       (const float*)(ws + p.o_U), (const float*)(ws + p.o_gam), h0, (bf16*)o, hT,
                       SAVE ? (bf16*)(ws + p.o_Sst) : nullptr, SAVE ? (bf16*)(ws + p.o_Dst) : nullptr,
                       BH, p.T, p.H, p.NC);
        }
        (void)n;
        return GDN_OK;
    }
    if constexpr (f32_tables<TIn, C, DK>()) {
        dim3 grid((unsigned)(ngrp * 8 * (DV / 32))), block(NTHR_S);
        GDN_LAUNCH(SAVE ? (OUT ? "scan_train" : "scan_save") : "scan", (scanf_kernel<C, DK, DV, SAVE, OUT>),
                   grid, block, st, (const float*)(ws + p.o_W), (const float*)(ws + p.o_Qg),
                   (const float*)(ws + p.o_Kh), (const float*)(ws + p.o_Ps),
                   (const float*)(ws + p.o_U), (const float*)(ws + p.o_gam), h0, (float*)o, hT,
                   SAVE ? (float*)(ws + p.o_Sst) : nullptr, SAVE ? (float*)(ws + p.o_Dst) : nullptr,
                   BH, p.T, p.H, p.NC);
        return GDN_OK;
    }
    if constexpr (!bf16_tables<TIn, C, DK>() && !f32_tables<TIn, C, DK>()) {
        dim3 grid((unsigned)(ngrp * 8 * SC::NS)), block(NTHR);
        GDN_LAUNCH(SAVE ? (OUT ? "scan_train" : "scan_save") : "scan", (scan_kernel<TIn, C, DK, DV, MT, SAVE, OUT>),
                   grid, block, st, (const float*)(ws + p.o_W), (const float*)(ws + p.o_U),
                   (const float*)(ws + p.o_Qg), (const float*)(ws + p.o_Kh),
                   (const float*)(ws + p.o_Ps), (const float*)(ws + p.o_gam), h0, (TIn*)o, hT,
                   SAVE ? (float*)(ws + p.o_Sst) : nullptr, BH, p.T, p.H, p.NC);
    }
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

__global__ void zero_words_kernel(unsigned int* __restrict__ w, int n)
{
    if ((int)threadIdx.x < n) w[threadIdx.x] = 0u;
}

// Numerical-safety options around a forward pass: the stage counters start at
// zero (a fill kernel, so the pass can be captured), and after the scan the
// outputs o and hT cross their stage boundary.
static gdn_status safety_begin(const Plan& p, char* ws, hipStream_t st)
{
    if (!p.diag) return GDN_OK;
    GDN_LAUNCH("zero_words", zero_words_kernel, dim3(1), dim3(64), st,
               (unsigned int*)(ws + p.o_dgc), GDN_DIAG_WORDS);
    return GDN_OK;
}

static gdn_status safety_outputs(const Plan& p, void* o, float* hT, char* ws, hipStream_t st)
{
    unsigned int* dg = p.diag ? (unsigned int*)(ws + p.o_dgc) : nullptr;
    const size_t no = (size_t)p.B * p.T * p.H * p.Dv, nh = (size_t)p.B * p.H * p.Dk * p.Dv;
    const SafeSeg segs[2] = {{o, no, p.dtype == GDN_BF16, dg ? dg + 2 * GDN_DIAG_O : nullptr},
                             {hT, nh, 0, dg ? dg + 2 * GDN_DIAG_HT : nullptr}};
    return safe_pass(segs, 2, p.clip, st);
}

gdn_status forward_dispatch(const Plan& p, const void* q, const void* k, const void* v,
                            const float* g, const float* beta, const float* h0, void* o, float* hT,
                            void* ws, hipStream_t st)
{
    gdn_status s = safety_begin(p, (char*)ws, st);
    if (s != GDN_OK) return s;
    s = p.dtype == GDN_BF16 ? forward_dt<bf16>(p, q, k, v, g, beta, h0, o, hT, (char*)ws, st)
                            : forward_dt<float>(p, q, k, v, g, beta, h0, o, hT, (char*)ws, st);
    if (s != GDN_OK) return s;
    return safety_outputs(p, o, hT, (char*)ws, st);
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

static gdn_status recompute_sized(const Plan& p, const void* q, const void* k, const void* v,
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

gdn_status recompute_dispatch(const Plan& p, const void* q, const void* k, const void* v,
                              const float* g, const float* beta, const float* h0, void* o,
                              float* hT, bool out, void* ws, hipStream_t st)
{
    gdn_status s = safety_begin(p, (char*)ws, st);
    if (s != GDN_OK) return s;
    s = recompute_sized(p, q, k, v, g, beta, h0, o, hT, out, ws, st);
    if (s != GDN_OK || !out) return s;
    return safety_outputs(p, o, hT, (char*)ws, st);
}

}  // namespace gdn
