// decode.hip -- single-token decode step of the gated delta rule, state in place.
//
// One token per (batch, head) (gated-deltanet card, "Method"):
//   S' = diag(a) S with a = exp(g);  m = S'^T k;  d = beta (v - m);
//   S_new = S' + k d^T;  o = scale S_new^T q = scale (S'^T q + (q.k) d).
// The state is the whole cost, so each state is read from HBM once and written
// once: a workgroup owns one (b, h), keeps its Dk x Dv fp32 slice in VGPRs
// between the read and the write, and reduces the two Dk-contractions
// (S'^T k and S'^T q) across lanes (cross-lane shuffles) and across waves (LDS).
//
// With L2N (use_qk_l2norm) q and k are first scaled to unit length,
// x / sqrt(|x|^2 + eps).  S'^T k, S'^T q and q.k are linear in them, so the
// squared lengths are reduced alongside and the three results rescaled.
//
// Thread map: a state row is Dv floats = Dv/4 float4 lanes (VPR).  Thread t
// owns float4 column c4 = t % VPR of rows r0 + p*RPP, r0 = t / VPR,
// RPP = NT / VPR, p = 0 .. Dk/RPP - 1.  Consecutive threads touch
// consecutive 16-byte words of a row, so every load and store is coalesced.
#include <type_traits>

#include "common.h"

namespace gdn {

template <int DK, int DV>
struct DecodeCfg {
    static constexpr int VPR = DV / 4;                       // float4 lanes per row
    static constexpr int NT = (DK * VPR < 256) ? DK * VPR : 256;  // threads
    static constexpr int RPP = NT / VPR;                     // rows per pass
    static constexpr int NP = DK / RPP;                      // passes
    static constexpr int NW = NT / 64;                       // waves
    static_assert(NT % 64 == 0, "decode block must be whole waves");
    static_assert(64 % VPR == 0 || VPR % 64 == 0, "row must tile a wave");
};

template <typename TIn, int DK, int DV, bool PER_CHANNEL, bool L2N>
__global__ void __launch_bounds__((DecodeCfg<DK, DV>::NT))
decode_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
              const float* __restrict__ g, const float* __restrict__ beta,
              float* __restrict__ state, TIn* __restrict__ o, int H, float scale)
{
    using C = DecodeCfg<DK, DV>;
    const int bh = blockIdx.x;  // = b*H + h; [B,1,H,*] inputs index the same way
    const int t = threadIdx.x;
    const int c4 = t % C::VPR;
    const int r0 = t / C::VPR;

    const TIn* qp = q + (size_t)bh * DK;
    const TIn* kp = k + (size_t)bh * DK;
    const TIn* vp = v + (size_t)bh * DV;
    float4* S = reinterpret_cast<float4*>(state + (size_t)bh * DK * DV);

    // the Dk-vectors (decay, k, q): one element per thread, shared through LDS,
    // exp taken once per row (instead of every thread loading and exponentiating
    // its rows' values)
    static_assert(DK <= C::NT, "one Dk element per thread");
    __shared__ float sa[DK], sk[DK], sq[DK];
    const int te = t < DK ? t : DK - 1;  // unconditional loads (the extra threads repeat one)
    const float ga = PER_CHANNEL ? g[(size_t)bh * DK + te] : g[bh];
    const TIn gk = kp[te], gq = qp[te];
    float4 s[C::NP];
#pragma unroll
    for (int p = 0; p < C::NP; ++p) s[p] = S[(r0 + p * C::RPP) * C::VPR + c4];
    if (t < DK) {
        sa[t] = fast_exp(ga);
        sk[t] = to_f32(gk);
        sq[t] = to_f32(gq);
    }
    __syncthreads();

    float kr[C::NP];
    float mk[4] = {0.f, 0.f, 0.f, 0.f}, mq[4] = {0.f, 0.f, 0.f, 0.f}, qk = 0.f, qq = 0.f, kk = 0.f;
#pragma unroll
    for (int p = 0; p < C::NP; ++p) {
        const int row = r0 + p * C::RPP;
        const float a = sa[row];
        const float kv = sk[row];
        const float qv = sq[row];
        kr[p] = kv;
        s[p].x *= a; s[p].y *= a; s[p].z *= a; s[p].w *= a;
        mk[0] += kv * s[p].x; mk[1] += kv * s[p].y; mk[2] += kv * s[p].z; mk[3] += kv * s[p].w;
        mq[0] += qv * s[p].x; mq[1] += qv * s[p].y; mq[2] += qv * s[p].z; mq[3] += qv * s[p].w;
        qk += qv * kv;
        if (L2N) {
            qq += qv * qv;
            kk += kv * kv;
        }
    }
    // reduce over the row groups inside a wave (lanes that share c4)
#pragma unroll
    for (int off = C::VPR; off < 64; off <<= 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            mk[e] += __shfl_xor(mk[e], off);
            mq[e] += __shfl_xor(mq[e], off);
        }
        qk += __shfl_xor(qk, off);
        if (L2N) {
            qq += __shfl_xor(qq, off);
            kk += __shfl_xor(kk, off);
        }
    }
    // reduce across waves through LDS, in a fixed order (deterministic)
    __shared__ float red[C::NW][C::VPR][11];
    if (C::NW > 1) {
        const int w = t / 64;
        if ((t % 64) < C::VPR) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                red[w][c4][e] = mk[e];
                red[w][c4][4 + e] = mq[e];
            }
            red[w][c4][8] = qk;
            red[w][c4][9] = qq;
            red[w][c4][10] = kk;
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float a1 = red[0][c4][e], a2 = red[0][c4][4 + e];
#pragma unroll
            for (int ww = 1; ww < C::NW; ++ww) {
                a1 += red[ww][c4][e];
                a2 += red[ww][c4][4 + e];
            }
            mk[e] = a1;
            mq[e] = a2;
        }
        float a3 = red[0][c4][8], a4 = red[0][c4][9], a5 = red[0][c4][10];
#pragma unroll
        for (int ww = 1; ww < C::NW; ++ww) {
            a3 += red[ww][c4][8];
            a4 += red[ww][c4][9];
            a5 += red[ww][c4][10];
        }
        qk = a3;
        qq = a4;
        kk = a5;
    }
    if (L2N) {
        const float rq = 1.f / sqrtf(qq + GDN_L2NORM_EPS), rk = 1.f / sqrtf(kk + GDN_L2NORM_EPS);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            mk[e] *= rk;
            mq[e] *= rq;
        }
        qk *= rq * rk;
#pragma unroll
        for (int p = 0; p < C::NP; ++p) kr[p] *= rk;
    }
    const float bt = beta[bh];
    float d[4], ov[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        d[e] = bt * (to_f32(vp[4 * c4 + e]) - mk[e]);
        ov[e] = scale * (mq[e] + qk * d[e]);
    }
    if (r0 == 0) {
        TIn* op = o + (size_t)bh * DV + 4 * c4;
#pragma unroll
        for (int e = 0; e < 4; ++e) op[e] = from_f32<TIn>(ov[e]);
    }
#pragma unroll
    for (int p = 0; p < C::NP; ++p) {
        float4 w = s[p];
        w.x += kr[p] * d[0]; w.y += kr[p] * d[1]; w.z += kr[p] * d[2]; w.w += kr[p] * d[3];
        S[(r0 + p * C::RPP) * C::VPR + c4] = w;
    }
}

template <typename TIn, int DK, int DV>
static gdn_status launch_decode(const gdn_shape* sh, const void* q, const void* k, const void* v,
                                const float* g, const float* beta, float* state, void* o,
                                float scale, hipStream_t st)
{
    using C = DecodeCfg<DK, DV>;
    dim3 grid(sh->B * sh->H), block(C::NT);
    auto launch = [&](auto pch, auto l2n) {
        GDN_LAUNCH("decode", (decode_kernel<TIn, DK, DV, decltype(pch)::value, decltype(l2n)::value>),
                   grid, block, st, (const TIn*)q, (const TIn*)k, (const TIn*)v, g, beta, state,
                   (TIn*)o, sh->H, scale);
        return GDN_OK;
    };
    using TT = std::true_type;
    using FF = std::false_type;
    if (sh->decay == GDN_DECAY_PER_CHANNEL)
        return sh->qk_l2norm ? launch(TT{}, TT{}) : launch(TT{}, FF{});
    return sh->qk_l2norm ? launch(FF{}, TT{}) : launch(FF{}, FF{});
}

template <typename TIn>
static gdn_status dispatch_decode_t(const gdn_shape* sh, const void* q, const void* k,
                                    const void* v, const float* g, const float* beta,
                                    float* state, void* o, float scale, hipStream_t st)
{
#define GDN_DEC(DK_, DV_)                                                                   \
    if (sh->Dk == DK_ && sh->Dv == DV_)                                                     \
        return launch_decode<TIn, DK_, DV_>(sh, q, k, v, g, beta, state, o, scale, st);
    GDN_DEC(16, 16) GDN_DEC(32, 32) GDN_DEC(64, 64) GDN_DEC(128, 128)
#undef GDN_DEC
    return GDN_ERR_UNSUPPORTED;
}

gdn_status decode_dispatch(const gdn_shape* sh, const void* q, const void* k, const void* v,
                           const float* g, const float* beta, float* state, void* o, float scale,
                           hipStream_t st)
{
    if (sh->dtype == GDN_BF16)
        return dispatch_decode_t<bf16>(sh, q, k, v, g, beta, state, o, scale, st);
    return dispatch_decode_t<float>(sh, q, k, v, g, beta, state, o, scale, st);
}

}  // namespace gdn
