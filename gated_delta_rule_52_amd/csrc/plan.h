// plan.h -- shape plan and workspace layout of the chunked path.
//
// The chunked form processes each (batch, head) sequence in chunks of C
// tokens; NC = ceil(T / C).  A chunk-head is one chunk of one (b, h); its
// index is ch = (b * H + h) * NC + n.  Workspace arrays are float32 unless noted
// below, indexed by chunk-head:
//   W   [ch][C][Dk]   W  = T diag(beta) (K o Gamma)        (WY form of the solve)
//   U   [ch][C][Dv]   U  = T diag(beta) V
//   Qg  [ch][C][Dk]   Qg = scale * (Q o Gamma)             (query read of the carried state)
//   Kh  [ch][C][Dk]   Kh = K o exp(G_{C-1} - G)            (key write into the next state)
//   Ps  [ch][C][C]    Ps = scale * P  (decayed query-key scores, lower incl. diagonal)
//   gam [ch][Dk]      gam = exp(G_{C-1})                   (whole-chunk decay)
//   rn  [ch][2][C]    with qk_l2norm: 1 / sqrt(|q_t|^2 + eps) (row 0) and the
//                     same for k_t (row 1); the backward scales q, k by them
//   dgc [GDN_DIAG_WORDS] uint32, with diag: the stage counters of the forward
// backward only:
//   Tm  [ch][C][C]    T = (I + A)^-1
//   Sst [ch][Dk][Dv]  state at the start of chunk n
//   dSt [ch][Dk][Dv]  gradient with respect to the state at the end of chunk n
//   dDt [ch][C][Dv]   gradient with respect to the chunk's deltas D
//   dQg [ch][C][Dk]   dL/dQg,  dWg [ch][C][Dk] dL/dW,  dKh [ch][C][Dk] dL/dKh
//   dPs [ch][C][C]    dL/dPs,  dT1 [ch][C][C]  dL/dT through U
//   dgm [ch][Dk]      dL/dgam, dbp [ch][C]     part of dL/dbeta (through U)
//   Dst [ch][C][Dv]   the chunk deltas D, saved by the state-saving forward scan
//                     at chunk 64 (bf16 with bf16 inputs, fp32 with fp32 inputs)
//   dbq [ch][2][C]    per channel-half partial dbeta, dgq [ch][2][C] partial
//                     per-head dg (bf16 inputs at chunk 64)
//   Wr  [ch][C][Dk] (bf16): with clip, the product T X_K before clipping, for
//                     the WY adjoint of the bf16 path
// With bf16 inputs at chunk 64, Sst, dSt, dDt and Dst are bf16 in 32-column
// slices, [ch][Dv / 32][rows][32] (slice32 in chunk_common.h).
// With bf16 inputs at chunk 64 the tables W, Qg, Kh, Ps are bf16, in the
// first half of their fp32-sized regions, in one orientation: W [C][Dk],
// Qg [C][Dk], Kh^T [Dk][C], Ps [C][C] (the backward scan reads their
// transposes with transposing LDS loads); the backward's hand-offs are bf16
// too: dQg, dKh, dPs;
// the dW region holds dX_K = T^T dW and the dT1 region the strictly lower
// dA = -(dX_V U^T + dX_K W^T).
// G is the chunk-local inclusive cumulative log-decay and Gamma = exp(G).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "gdn.h"

namespace gdn {

struct Plan {
    int B, T, H, Dk, Dv, C, NC, dtype, decay;
    bool l2n;  // qk_l2norm
    float scale;
    float clip, dinv;  // numerical-safety options: clip bound, 1 / (1 + wy_eps)
    bool diag;
    size_t n_ch;  // B * H * NC
    // byte offsets into the workspace
    size_t o_W, o_U, o_Qg, o_Kh, o_Ps, o_gam, o_rn, o_dgc, o_Tm, o_Sst, o_dSt, o_dDt;
    size_t o_dQg, o_dWg, o_dKh, o_dPs, o_dT1, o_dgm, o_dbp, o_Dst, o_dbq, o_dgq, o_Wr;
    size_t ws_fwd_bytes, ws_bwd_bytes;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline bool plan_supported(int Dk, int Dv, int C)
{
    if (Dk != Dv) return false;
    if (C == 64) return Dk == 64 || Dk == 128;
    if (C == 16) return Dk == 16;
    return false;
}

inline Plan make_plan(const gdn_shape& s, float scale)
{
    Plan p;
    p.B = s.B; p.T = s.T; p.H = s.H; p.Dk = s.Dk; p.Dv = s.Dv;
    p.C = s.chunk ? s.chunk : 64;
    p.NC = (s.T + p.C - 1) / p.C;
    p.dtype = s.dtype; p.decay = s.decay; p.scale = scale;
    p.l2n = s.qk_l2norm != 0;
    p.clip = s.clip;
    p.dinv = 1.0f / (1.0f + s.wy_eps);
    p.diag = s.diag != 0;
    p.n_ch = (size_t)s.B * s.H * p.NC;
    const size_t f = sizeof(float), n = p.n_ch, C = p.C, Dk = p.Dk, Dv = p.Dv;
    size_t off = 0;
    p.o_W = off;   off = align256(off + n * C * Dk * f);
    p.o_U = off;   off = align256(off + n * C * Dv * f);
    p.o_Qg = off;  off = align256(off + n * C * Dk * f);
    p.o_Kh = off;  off = align256(off + n * C * Dk * f);
    p.o_Ps = off;  off = align256(off + n * C * C * f);
    p.o_gam = off; off = align256(off + n * Dk * f);
    p.o_rn = off;  off = align256(off + (p.l2n ? n * 2 * C * f : 0));
    p.o_dgc = off; off = align256(off + (p.diag ? GDN_DIAG_WORDS * sizeof(unsigned int) : 0));
    p.ws_fwd_bytes = off;
    p.o_Tm = off;  off = align256(off + n * C * C * f);
    p.o_Sst = off; off = align256(off + n * Dk * Dv * f);
    p.o_dSt = off; off = align256(off + n * Dk * Dv * f);
    p.o_dDt = off; off = align256(off + n * C * Dv * f);
    p.o_dQg = off; off = align256(off + n * C * Dk * f);
    p.o_dWg = off; off = align256(off + n * C * Dk * f);
    p.o_dKh = off; off = align256(off + n * C * Dk * f);
    p.o_dPs = off; off = align256(off + n * C * C * f);
    p.o_dT1 = off; off = align256(off + n * C * C * f);
    p.o_dgm = off; off = align256(off + n * Dk * f);
    p.o_dbp = off; off = align256(off + n * C * f);
    p.o_Dst = off; off = align256(off + n * C * Dv * (s.dtype == GDN_F32 ? 4 : 2));
    p.o_dbq = off; off = align256(off + n * 2 * C * f);
    p.o_dgq = off; off = align256(off + n * 2 * C * f);
    const bool raw = s.clip > 0.f;
    p.o_Wr = off;  off = align256(off + (raw ? n * C * Dk * 2 : 0));
    p.ws_bwd_bytes = off;
    return p;
}

}  // namespace gdn
