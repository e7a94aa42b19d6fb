// replay.hip -- decode with the state kept as a checkpoint plus a buffer of
// recent tokens (the ReplaySSM idea in the news digest's blurb, page "Gated
// DeltaNet" topic: checkpoint + recent-input buffer, the checkpoint written only
// when the buffer fills, outputs computed directly on the other steps).
//
// For the gated delta rule (gated-deltanet card, "Method") with checkpoint S_c
// after some token, buffered tokens i = 1..n since it, and G_i the log-decay
// accumulated from the checkpoint through token i (per key channel, or one per
// head), the state before token t's write is
//     S'_t = diag(e^{G_t}) S_c + sum_{i<t} diag(e^{G_t - G_i}) k_i d_i^T,
// so, with alpha_ti = sum_c k_tc k_ic e^{G_tc - G_ic} and gamma_ti the same
// with q_t in place of k_t,
//     m_t = S_c^T (e^{G_t} o k_t) + sum_{i<t} alpha_ti d_i,   d_t = beta_t (v_t - m_t),
//     o_t = scale (S_c^T (e^{G_t} o q_t) + sum_{i<t} gamma_ti d_i + (q_t . k_t) d_t).
// A step reads the checkpoint once and writes only the new token's (k, G, d)
// into the buffer; when the buffer holds `depth` tokens the kernel folds it
// into the checkpoint, S_c <- diag(e^{G_t}) S_c + sum_i diag(e^{G_t - G_i}) k_i d_i^T,
// and empties it.  The arithmetic is the recurrence's, reassociated.
//
// Buffer layout (gdn_replay_buffer_bytes): n[B*H] int32 (tokens held), then
// K [B*H][depth][Dk] fp32, G [B*H][depth][Dk or 1] fp32, D [B*H][depth][Dv] fp32.
// Thread map as the plain decode step: thread t owns float4 column c4 = t % VPR
// of rows r0 + p*RPP of the checkpoint, r0 = t / VPR.
#include <type_traits>

#include "common.h"

namespace gdn {

constexpr int REPLAY_MAX_DEPTH = 16;

template <int DK, int DV>
struct ReplayCfg {
    static constexpr int VPR = DV / 4;
    static constexpr int NT = (DK * VPR < 256) ? DK * VPR : 256;
    static constexpr int RPP = NT / VPR;
    static constexpr int NP = DK / RPP;
    static constexpr int NW = NT / 64;
    static constexpr int SUB = 16;             // lanes per buffered token in the dot phase
    static constexpr int CPS = DK / SUB;       // key channels per lane there
    static_assert(NT % 64 == 0 && DK % SUB == 0, "replay geometry");
};

struct ReplayBuf {
    int* n;
    float* K;
    float* G;
    float* D;
};

inline size_t align256r(size_t x) { return (x + 255) & ~(size_t)255; }

inline ReplayBuf replay_layout(void* buf, int BH, int Dk, int Dv, int depth, bool pch)
{
    char* p = (char*)buf;
    ReplayBuf b;
    size_t off = 0;
    b.n = (int*)(p + off);   off = align256r(off + sizeof(int) * BH);
    b.K = (float*)(p + off); off = align256r(off + sizeof(float) * BH * depth * Dk);
    b.G = (float*)(p + off); off = align256r(off + sizeof(float) * BH * depth * (pch ? Dk : 1));
    b.D = (float*)(p + off);
    return b;
}

inline size_t replay_bytes(int BH, int Dk, int Dv, int depth, bool pch)
{
    size_t off = 0;
    off = align256r(off + sizeof(int) * BH);
    off = align256r(off + sizeof(float) * BH * depth * Dk);
    off = align256r(off + sizeof(float) * BH * depth * (pch ? Dk : 1));
    off = align256r(off + sizeof(float) * BH * depth * Dv);
    return off;
}

// One token (TOKEN) or, without a token, only the fold of the buffer into the
// checkpoint (the current state materialised; the buffer emptied).
// Every load is issued up front: the checkpoint into registers (consumed by
// the two reads right after the barrier) and the buffered tokens straight into
// LDS.  Only a step that fills the buffer reads the checkpoint again, to fold
// into it.
template <typename TIn, int DK, int DV, bool PCH, bool TOKEN>
__global__ void __launch_bounds__((ReplayCfg<DK, DV>::NT))
replay_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
              const float* __restrict__ g, const float* __restrict__ beta,
              float* __restrict__ ckpt, ReplayBuf rb, TIn* __restrict__ o, float scale, int depth)
{
    using CF = ReplayCfg<DK, DV>;
    constexpr int GW = PCH ? DK : 1;
    constexpr int LM = REPLAY_MAX_DEPTH;
    __shared__ __align__(16) float sK[LM][DK], sD[LM][DV], sG[(LM * GW + 3) / 4 * 4];
    __shared__ float sGt[GW], skt[DK], sqt[DK], sal[LM], sga[LM];
    __shared__ float red[CF::NW][CF::VPR][9];
    const int bh = blockIdx.x;
    const int t = threadIdx.x;
    const int c4 = t % CF::VPR, r0 = t / CF::VPR;
    const int n = rb.n[bh];  // tokens in the buffer (< depth)
    float* Kb = rb.K + (size_t)bh * depth * DK;
    float* Gb = rb.G + (size_t)bh * depth * GW;
    float* Db = rb.D + (size_t)bh * depth * DV;
    float4* S = reinterpret_cast<float4*>(ckpt + (size_t)bh * DK * DV);

    // ---- every load up front: the checkpoint into registers, the buffered
    // tokens straight into LDS (16-byte direct-to-LDS loads, 1 KB per wave and
    // instruction, lane l landing at 16 l bytes; lanes past the end load nothing)
    float4 s[CF::NP];
    if (TOKEN) {
#pragma unroll
        for (int p = 0; p < CF::NP; ++p) s[p] = S[(r0 + p * CF::RPP) * CF::VPR + c4];
    }
    {
        const int w = t / 64, l = t % 64;
        auto to_lds = [&](const float* src, float* dst, int n4) {  // n4 16-byte words
            for (int u = w; u * 64 < n4; u += CF::NW) {
                const int i4 = u * 64 + l;
                if (i4 < n4) __builtin_amdgcn_global_load_lds(src + 4 * i4, dst + u * 256, 16, 0, 0);
            }
        };
        to_lds(Kb, &sK[0][0], n * (DK / 4));
        to_lds(Db, &sD[0][0], n * (DV / 4));
        if (PCH) to_lds(Gb, &sG[0], n * (GW / 4));
        else if (t < n) sG[t] = Gb[t];
    }
    for (int c = t; c < GW; c += CF::NT) {
        const float gp = n > 0 ? Gb[(n - 1) * GW + c] : 0.f;
        sGt[c] = TOKEN ? gp + g[(size_t)bh * GW + c] : gp;
    }
    if (TOKEN) {
        for (int c = t; c < DK; c += CF::NT) {
            skt[c] = to_f32(k[(size_t)bh * DK + c]);
            sqt[c] = to_f32(q[(size_t)bh * DK + c]);
        }
    }
    __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): the direct-to-LDS loads have landed
    __syncthreads();
    auto Gi = [&](int i, int c) { return sG[i * GW + (PCH ? c : 0)]; };

    float dtk[4] = {0.f, 0.f, 0.f, 0.f};  // the new token's delta (this thread's column)
    if (TOKEN) {
        // ---- checkpoint reads: S_c^T (e^G o k_t), S_c^T (e^G o q_t); and q_t . k_t
        float mk[4] = {0.f, 0.f, 0.f, 0.f}, mq[4] = {0.f, 0.f, 0.f, 0.f}, qk = 0.f;
#pragma unroll
        for (int p = 0; p < CF::NP; ++p) {
            const int row = r0 + p * CF::RPP;
            const float a = fast_exp(sGt[PCH ? row : 0]);
            const float kv = skt[row], qv = sqt[row];
            const float ka = kv * a, qa = qv * a;
            mk[0] += ka * s[p].x; mk[1] += ka * s[p].y; mk[2] += ka * s[p].z; mk[3] += ka * s[p].w;
            mq[0] += qa * s[p].x; mq[1] += qa * s[p].y; mq[2] += qa * s[p].z; mq[3] += qa * s[p].w;
            qk += qv * kv;
        }
#pragma unroll
        for (int off = CF::VPR; off < 64; off <<= 1) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                mk[e] += __shfl_xor(mk[e], off);
                mq[e] += __shfl_xor(mq[e], off);
            }
            qk += __shfl_xor(qk, off);
        }
        if (CF::NW > 1) {
            const int w = t / 64;
            if ((t % 64) < CF::VPR) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    red[w][c4][e] = mk[e];
                    red[w][c4][4 + e] = mq[e];
                }
                red[w][c4][8] = qk;
            }
        }
        // ---- buffered tokens: alpha_i, gamma_i (16 lanes per token, fixed butterfly)
        {
            const int sub = t % CF::SUB;
            for (int i0 = t / CF::SUB; i0 < LM; i0 += CF::NT / CF::SUB) {
                float al = 0.f, ga = 0.f;
                if (i0 < n) {
#pragma unroll
                    for (int cc = 0; cc < CF::CPS; ++cc) {
                        const int c = sub * CF::CPS + cc;
                        const float e = fast_exp(sGt[PCH ? c : 0] - Gi(i0, c));
                        const float kc = sK[i0][c] * e;
                        al += skt[c] * kc;
                        ga += sqt[c] * kc;
                    }
                }
#pragma unroll
                for (int off = 1; off < CF::SUB; off <<= 1) {
                    al += __shfl_xor(al, off);
                    ga += __shfl_xor(ga, off);
                }
                if (sub == 0) {
                    sal[i0] = al;
                    sga[i0] = ga;
                }
            }
        }
        __syncthreads();
        if (CF::NW > 1) {  // fixed order over waves: repeatable
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float a1 = red[0][c4][e], a2 = red[0][c4][4 + e];
#pragma unroll
                for (int ww = 1; ww < CF::NW; ++ww) {
                    a1 += red[ww][c4][e];
                    a2 += red[ww][c4][4 + e];
                }
                mk[e] = a1;
                mq[e] = a2;
            }
            float a3 = red[0][c4][8];
#pragma unroll
            for (int ww = 1; ww < CF::NW; ++ww) a3 += red[ww][c4][8];
            qk = a3;
        }
        // ---- the new delta and the output
        float ov[4] = {mq[0], mq[1], mq[2], mq[3]};
        for (int i = 0; i < n; ++i) {
            const float4 d4 = *reinterpret_cast<const float4*>(&sD[i][4 * c4]);
            const float al = sal[i], ga = sga[i];
            mk[0] += al * d4.x; mk[1] += al * d4.y; mk[2] += al * d4.z; mk[3] += al * d4.w;
            ov[0] += ga * d4.x; ov[1] += ga * d4.y; ov[2] += ga * d4.z; ov[3] += ga * d4.w;
        }
        const float bt = beta[bh];
        float* dt = dtk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            dt[e] = bt * (to_f32(v[(size_t)bh * DV + 4 * c4 + e]) - mk[e]);
            ov[e] = scale * (ov[e] + qk * dt[e]);
        }
        if (r0 == 0) {
            TIn* op = o + (size_t)bh * DV + 4 * c4;
#pragma unroll
            for (int e = 0; e < 4; ++e) op[e] = from_f32<TIn>(ov[e]);
            *reinterpret_cast<float4*>(&Db[n * DV + 4 * c4]) = float4{dt[0], dt[1], dt[2], dt[3]};
        }
        for (int c = t; c < DK; c += CF::NT) Kb[n * DK + c] = skt[c];
        for (int c = t; c < GW; c += CF::NT) Gb[n * GW + c] = sGt[c];
        if (n + 1 < depth) {
            if (t == 0) rb.n[bh] = n + 1;
            return;  // whole workgroup (n is uniform): no barrier follows
        }
        // ---- buffer full: fold it, with the token just added, into the checkpoint
    } else if (n == 0) {
        return;  // nothing buffered: the checkpoint is the state
    }
    // one checkpoint row at a time (few registers live): e^{G_t} S_c row, plus
    // each buffered token's e^{G_t - G_i} k_i d_i^T, plus the new token's k_t d_t^T
#pragma unroll 2
    for (int p = 0; p < CF::NP; ++p) {
        const int row = r0 + p * CF::RPP;
        const float gr = sGt[PCH ? row : 0];
        const float a = fast_exp(gr);
        const float4 c0 = S[row * CF::VPR + c4];
        float4 acc = float4{a * c0.x, a * c0.y, a * c0.z, a * c0.w};
        if (TOKEN) {
            const float kr = skt[row];
            acc.x += kr * dtk[0]; acc.y += kr * dtk[1]; acc.z += kr * dtk[2]; acc.w += kr * dtk[3];
        }
        for (int i = 0; i < n; ++i) {
            const float4 d4 = *reinterpret_cast<const float4*>(&sD[i][4 * c4]);
            const float w = sK[i][row] * fast_exp(gr - Gi(i, row));
            acc.x += w * d4.x; acc.y += w * d4.y; acc.z += w * d4.z; acc.w += w * d4.w;
        }
        S[row * CF::VPR + c4] = acc;
    }
    if (t == 0) rb.n[bh] = 0;
}

__global__ void replay_reset_kernel(int* __restrict__ n, int count)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < count) n[i] = 0;
}

template <typename TIn, int DK, int DV, bool TOKEN>
static gdn_status launch_replay(const gdn_shape* sh, const void* q, const void* k, const void* v,
                                const float* g, const float* beta, float* ckpt, void* buf,
                                int depth, void* o, float scale, hipStream_t st)
{
    using CF = ReplayCfg<DK, DV>;
    const int BH = sh->B * sh->H;
    const bool pch = sh->decay == GDN_DECAY_PER_CHANNEL;
    const ReplayBuf rb = replay_layout(buf, BH, DK, DV, depth, pch);
    return with_bool(pch, [&](auto pc) {
        GDN_LAUNCH(TOKEN ? "replay_step" : "replay_fold",
                   (replay_kernel<TIn, DK, DV, decltype(pc)::value, TOKEN>), dim3(BH),
                   dim3(CF::NT), st, (const TIn*)q, (const TIn*)k, (const TIn*)v, g, beta, ckpt,
                   rb, (TIn*)o, scale, depth);
        return GDN_OK;
    });
}

template <typename TIn, bool TOKEN>
static gdn_status dispatch_replay_t(const gdn_shape* sh, const void* q, const void* k,
                                    const void* v, const float* g, const float* beta, float* ckpt,
                                    void* buf, int depth, void* o, float scale, hipStream_t st)
{
#define GDN_REP(DK_, DV_)                                                                    \
    if (sh->Dk == DK_ && sh->Dv == DV_)                                                      \
        return launch_replay<TIn, DK_, DV_, TOKEN>(sh, q, k, v, g, beta, ckpt, buf, depth, o, \
                                                   scale, st);
    GDN_REP(16, 16) GDN_REP(32, 32) GDN_REP(64, 64) GDN_REP(128, 128)
#undef GDN_REP
    return GDN_ERR_UNSUPPORTED;
}

gdn_status replay_dispatch(const gdn_shape* sh, const void* q, const void* k, const void* v,
                           const float* g, const float* beta, float* ckpt, void* buf, int depth,
                           void* o, float scale, bool token, hipStream_t st)
{
    if (sh->dtype == GDN_BF16)
        return token ? dispatch_replay_t<bf16, true>(sh, q, k, v, g, beta, ckpt, buf, depth, o, scale, st)
                     : dispatch_replay_t<bf16, false>(sh, q, k, v, g, beta, ckpt, buf, depth, o, scale, st);
    return token ? dispatch_replay_t<float, true>(sh, q, k, v, g, beta, ckpt, buf, depth, o, scale, st)
                 : dispatch_replay_t<float, false>(sh, q, k, v, g, beta, ckpt, buf, depth, o, scale, st);
}

size_t replay_buffer_bytes(int BH, int Dk, int Dv, int depth, bool pch)
{
    return replay_bytes(BH, Dk, Dv, depth, pch);
}

gdn_status replay_reset(void* buf, int BH, hipStream_t st)
{
    GDN_LAUNCH("replay_reset", replay_reset_kernel, dim3((unsigned)((BH + 255) / 256)), dim3(256),
               st, (int*)buf, BH);
    return GDN_OK;
}

}  // namespace gdn
