// gdn_api.hip -- the C ABI declared in include/gdn.h: argument validation,
// workspace planning and dispatch to the gfx950 kernels.  Nothing here
// allocates device memory; every launch goes to the caller's stream.
#include <stdint.h>

#include <mutex>

#include "common.h"
#include "plan.h"

namespace gdn {
gdn_status decode_dispatch(const gdn_shape* sh, const void* q, const void* k, const void* v,
                           const float* g, const float* beta, float* state, void* o, float scale,
                           hipStream_t st);
gdn_status forward_dispatch(const Plan& p, const void* q, const void* k, const void* v,
                            const float* g, const float* beta, const float* h0, void* o, float* hT,
                            void* ws, hipStream_t st);
gdn_status backward_dispatch(const Plan& p, const void* q, const void* k, const void* v,
                             const float* g, const float* beta, const float* h0, const void* dO,
                             const float* dhT, void* dq, void* dk, void* dv, float* dg,
                             float* dbeta, float* dh0, void* ws, bool recompute, hipStream_t st);
gdn_status recompute_dispatch(const Plan& p, const void* q, const void* k, const void* v,
                              const float* g, const float* beta, const float* h0, void* o,
                              float* hT, bool out, void* ws, hipStream_t st);

gdn_status replay_dispatch(const gdn_shape* sh, const void* q, const void* k, const void* v,
                           const float* g, const float* beta, float* ckpt, void* buf, int depth,
                           void* o, float scale, bool token, hipStream_t st);
size_t replay_buffer_bytes(int BH, int Dk, int Dv, int depth, bool pch);
gdn_status replay_reset(void* buf, int BH, hipStream_t st);

__global__ void fill_zero_kernel(float4* __restrict__ p, size_t n4)
{
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < n4; i += stride) p[i] = float4{0.f, 0.f, 0.f, 0.f};
}
}  // namespace gdn

using namespace gdn;

// Workspace of gdn_forward_noalloc.  In host code `scratch` is only a handle for
// hipGetSymbolAddress: the device address of each device's copy is looked up
// once per device (with that device current) and kept in scratch_ptr; kernels
// and every other host use take that address, never the array's name.
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];  // device address of `scratch` on device i, or null

gdn_status scratch_on_current_device(void** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GDN_ERR_HIP;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GDN_ERR_HIP;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return GDN_OK;
}
}  // namespace

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static bool dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// Validate a shape and fill in defaults; returns GDN_OK or the error.
static gdn_status check_shape(const gdn_shape* sh, bool decode)
{
    if (!sh) return GDN_ERR_INVALID_ARG;
    if (sh->B <= 0 || sh->H <= 0 || sh->T < 0 || sh->Dk <= 0 || sh->Dv <= 0)
        return GDN_ERR_INVALID_ARG;
    if (sh->dtype != GDN_F32 && sh->dtype != GDN_BF16) return GDN_ERR_INVALID_ARG;
    if (sh->decay != GDN_DECAY_PER_HEAD && sh->decay != GDN_DECAY_PER_CHANNEL)
        return GDN_ERR_INVALID_ARG;
    if (!(sh->scale >= 0.f)) return GDN_ERR_INVALID_ARG;  // rejects NaN and negatives
    if (sh->qk_l2norm != 0 && sh->qk_l2norm != 1) return GDN_ERR_INVALID_ARG;
    if (!(sh->wy_eps >= 0.f && sh->wy_eps <= 1e30f)) return GDN_ERR_INVALID_ARG;  // also NaN
    if (!(sh->clip >= 0.f && sh->clip <= 3.0e38f)) return GDN_ERR_INVALID_ARG;
    if (sh->diag != 0 && sh->diag != 1) return GDN_ERR_INVALID_ARG;
    // the options act on the chunked form's stages; the decode step has none
    if (decode && (sh->wy_eps != 0.f || sh->clip != 0.f || sh->diag)) return GDN_ERR_UNSUPPORTED;
    if (decode && sh->T != 1) return GDN_ERR_INVALID_ARG;
    if (!dim_ok(sh->Dk) || !dim_ok(sh->Dv)) return GDN_ERR_UNSUPPORTED;
    if (!decode) {
        const int C = sh->chunk ? sh->chunk : 64;
        if (C != 16 && C != 64) return GDN_ERR_UNSUPPORTED;
        if (!plan_supported(sh->Dk, sh->Dv, C)) return GDN_ERR_UNSUPPORTED;
        // a chunk's token rows are addressed with 32-bit offsets from its first
        // row (H * max(Dk, Dv) elements per token row, C rows)
        const long long D = sh->Dk > sh->Dv ? sh->Dk : sh->Dv;
        if ((long long)sh->H * D * C > (1LL << 28)) return GDN_ERR_UNSUPPORTED;
        // token-heads of the padded chunks: every launch of a chunked call has at
        // most 32 work-items per token-head (the fp32 L2-normalisation adjoint;
        // the chunk kernels take at most 512 per chunk-head of 64), so a grid's
        // work-item count stays below 2^32 and chunk-head indices fit in int
        if ((long long)sh->B * sh->H * ((sh->T + C - 1) / C) * C >= (1LL << 27))
            return GDN_ERR_UNSUPPORTED;
    }
    return GDN_OK;
}

static float eff_scale(const gdn_shape* sh)
{
    return sh->scale > 0.f ? sh->scale : 1.0f / sqrtf((float)sh->Dk);
}

extern "C" {

const char* gdn_status_string(gdn_status s)
{
    switch (s) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_INVALID_ARG: return "GDN_ERR_INVALID_ARG: invalid shape, dtype or NULL pointer";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED: (chunk, Dk, Dv) not compiled in";
    case GDN_ERR_ALIGNMENT: return "GDN_ERR_ALIGNMENT: a pointer is not 16-byte aligned";
    case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE: workspace missing or too small";
    case GDN_ERR_HIP: return "GDN_ERR_HIP: a kernel launch failed";
    }
    return "unknown gdn_status";
}

gdn_status gdn_new_state(float* state, int B, int H, int Dk, int Dv, void* stream)
{
    if (!state || B <= 0 || H <= 0 || Dk <= 0 || Dv <= 0) return GDN_ERR_INVALID_ARG;
    if (!aligned16(state)) return GDN_ERR_ALIGNMENT;
    const size_t n = (size_t)B * H * Dk * Dv;
    if (n % 4) return GDN_ERR_INVALID_ARG;
    const size_t n4 = n / 4;
    size_t blocks = (n4 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    GDN_LAUNCH("fill_zero", fill_zero_kernel, dim3((unsigned)blocks), dim3(256), (hipStream_t)stream, (float4*)state, n4);
    GDN_HIP_CHECK_LAUNCH();
    return GDN_OK;
}

size_t gdn_workspace_bytes(const gdn_shape* sh, int for_backward)
{
    if (check_shape(sh, false) != GDN_OK) return 0;
    Plan p = make_plan(*sh, eff_scale(sh));
    return for_backward ? p.ws_bwd_bytes : p.ws_fwd_bytes;
}

gdn_status gdn_forward(const gdn_shape* sh, const void* q, const void* k, const void* v,
                       const float* g, const float* beta, const float* h0, void* o, float* hT,
                       void* ws, size_t ws_bytes, void* stream)
{
    gdn_status s = check_shape(sh, false);
    if (s != GDN_OK) return s;
    if (sh->T == 0) {  // no tokens: the state passes through unchanged
        if (hT && hT != h0) {
            if (!aligned16(hT) || (h0 && !aligned16(h0))) return GDN_ERR_ALIGNMENT;
            const size_t bytes = sizeof(float) * sh->B * sh->H * sh->Dk * sh->Dv;
            if (h0) {
                if (hipMemcpyAsync(hT, h0, bytes, hipMemcpyDeviceToDevice, (hipStream_t)stream) !=
                    hipSuccess)
                    return GDN_ERR_HIP;
            } else {
                return gdn_new_state(hT, sh->B, sh->H, sh->Dk, sh->Dv, stream);
            }
        }
        return GDN_OK;
    }
    if (!q || !k || !v || !g || !beta || !o) return GDN_ERR_INVALID_ARG;
    const void* ptrs[] = {q, k, v, g, beta, o, h0, hT, ws};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return GDN_ERR_ALIGNMENT;
    Plan p = make_plan(*sh, eff_scale(sh));
    if (p.ws_fwd_bytes && (!ws || ws_bytes < p.ws_fwd_bytes)) return GDN_ERR_WORKSPACE;
    return forward_dispatch(p, q, k, v, g, beta, h0, o, hT, ws, (hipStream_t)stream);
}

gdn_status gdn_forward_noalloc(const gdn_shape* sh, const void* q, const void* k, const void* v,
                               const float* g, const float* beta, const float* h0, void* o,
                               float* hT, void* stream)
{
    gdn_status s = check_shape(sh, false);
    if (s != GDN_OK) return s;
    if (sh->diag) return GDN_ERR_UNSUPPORTED;
    const size_t need = gdn_workspace_bytes(sh, 0);
    if (need > GDN_NOALLOC_SCRATCH_BYTES) return GDN_ERR_WORKSPACE;
    void* ws = nullptr;
    if (need) {
        s = scratch_on_current_device(&ws);
        if (s != GDN_OK) return s;
    }
    return gdn_forward(sh, q, k, v, g, beta, h0, o, hT, ws, need, stream);
}

static gdn_status backward_common(const gdn_shape* sh, const void* q, const void* k,
                                  const void* v, const float* g, const float* beta,
                                  const float* h0, const void* dO, const float* dhT, void* dq,
                                  void* dk, void* dv, float* dg, float* dbeta, float* dh0,
                                  void* ws, size_t ws_bytes, void* stream, bool recompute)
{
    gdn_status s = check_shape(sh, false);
    if (s != GDN_OK) return s;
    if (sh->T == 0) {  // no tokens: dh0 = dhT
        if (!dh0) return GDN_OK;
        if (!aligned16(dh0) || (dhT && !aligned16(dhT))) return GDN_ERR_ALIGNMENT;
        if (!dhT) return gdn_new_state(dh0, sh->B, sh->H, sh->Dk, sh->Dv, stream);
        const size_t bytes = sizeof(float) * sh->B * sh->H * sh->Dk * sh->Dv;
        if (hipMemcpyAsync(dh0, dhT, bytes, hipMemcpyDeviceToDevice, (hipStream_t)stream) !=
            hipSuccess)
            return GDN_ERR_HIP;
        return GDN_OK;
    }
    if (!q || !k || !v || !g || !beta || !dO || !dq || !dk || !dv || !dg || !dbeta)
        return GDN_ERR_INVALID_ARG;
    const void* ptrs[] = {q, k, v, g, beta, h0, dO, dhT, dq, dk, dv, dg, dbeta, dh0, ws};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return GDN_ERR_ALIGNMENT;
    Plan p = make_plan(*sh, eff_scale(sh));
    if (p.ws_bwd_bytes && (!ws || ws_bytes < p.ws_bwd_bytes)) return GDN_ERR_WORKSPACE;
    return backward_dispatch(p, q, k, v, g, beta, h0, dO, dhT, dq, dk, dv, dg, dbeta, dh0, ws,
                             recompute, (hipStream_t)stream);
}

gdn_status gdn_backward(const gdn_shape* sh, const void* q, const void* k, const void* v,
                        const float* g, const float* beta, const float* h0, const void* dO,
                        const float* dhT, void* dq, void* dk, void* dv, float* dg, float* dbeta,
                        float* dh0, void* ws, size_t ws_bytes, void* stream)
{
    return backward_common(sh, q, k, v, g, beta, h0, dO, dhT, dq, dk, dv, dg, dbeta, dh0, ws,
                           ws_bytes, stream, true);
}

gdn_status gdn_forward_train(const gdn_shape* sh, const void* q, const void* k, const void* v,
                             const float* g, const float* beta, const float* h0, void* o,
                             float* hT, void* ws, size_t ws_bytes, void* stream)
{
    gdn_status s = check_shape(sh, false);
    if (s != GDN_OK) return s;
    if (sh->T == 0) return gdn_forward(sh, q, k, v, g, beta, h0, o, hT, ws, ws_bytes, stream);
    if (!q || !k || !v || !g || !beta || !o) return GDN_ERR_INVALID_ARG;
    const void* ptrs[] = {q, k, v, g, beta, o, h0, hT, ws};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return GDN_ERR_ALIGNMENT;
    Plan p = make_plan(*sh, eff_scale(sh));
    if (!ws || ws_bytes < p.ws_bwd_bytes) return GDN_ERR_WORKSPACE;
    return recompute_dispatch(p, q, k, v, g, beta, h0, o, hT, true, ws, (hipStream_t)stream);
}

gdn_status gdn_backward_train(const gdn_shape* sh, const void* q, const void* k, const void* v,
                              const float* g, const float* beta, const void* dO, const float* dhT,
                              void* dq, void* dk, void* dv, float* dg, float* dbeta, float* dh0,
                              void* ws, size_t ws_bytes, void* stream)
{
    return backward_common(sh, q, k, v, g, beta, nullptr, dO, dhT, dq, dk, dv, dg, dbeta, dh0,
                           ws, ws_bytes, stream, false);
}

gdn_status gdn_diag_read(const gdn_shape* sh, const void* ws, unsigned int* counts, void* stream)
{
    gdn_status s = check_shape(sh, false);
    if (s != GDN_OK) return s;
    if (!sh->diag || !ws || !counts) return GDN_ERR_INVALID_ARG;
    Plan p = make_plan(*sh, eff_scale(sh));
    if (hipMemcpyAsync(counts, (const char*)ws + p.o_dgc, GDN_DIAG_WORDS * sizeof(unsigned int),
                       hipMemcpyDeviceToHost, (hipStream_t)stream) != hipSuccess)
        return GDN_ERR_HIP;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return GDN_ERR_HIP;
    return GDN_OK;
}

static bool depth_ok(int depth) { return depth >= 1 && depth <= 16; }

size_t gdn_replay_buffer_bytes(const gdn_shape* sh, int depth)
{
    if (check_shape(sh, true) != GDN_OK || !depth_ok(depth)) return 0;
    return replay_buffer_bytes(sh->B * sh->H, sh->Dk, sh->Dv, depth,
                               sh->decay == GDN_DECAY_PER_CHANNEL);
}

gdn_status gdn_replay_reset(const gdn_shape* sh, void* buf, int depth, void* stream)
{
    gdn_status s = check_shape(sh, true);
    if (s != GDN_OK) return s;
    if (!buf || !depth_ok(depth)) return GDN_ERR_INVALID_ARG;
    if (!aligned16(buf)) return GDN_ERR_ALIGNMENT;
    return replay_reset(buf, sh->B * sh->H, (hipStream_t)stream);
}

gdn_status gdn_replay_step(const gdn_shape* sh, const void* q, const void* k, const void* v,
                           const float* g, const float* beta, float* ckpt, void* buf, int depth,
                           void* o, void* stream)
{
    gdn_status s = check_shape(sh, true);
    if (s != GDN_OK) return s;
    if (!q || !k || !v || !g || !beta || !ckpt || !buf || !o || !depth_ok(depth))
        return GDN_ERR_INVALID_ARG;
    const void* ptrs[] = {q, k, v, g, beta, ckpt, buf, o};
    for (const void* p : ptrs)
        if (!aligned16(p)) return GDN_ERR_ALIGNMENT;
    return replay_dispatch(sh, q, k, v, g, beta, ckpt, buf, depth, o, eff_scale(sh), true,
                           (hipStream_t)stream);
}

gdn_status gdn_replay_fold(const gdn_shape* sh, float* ckpt, void* buf, int depth, void* stream)
{
    gdn_status s = check_shape(sh, true);
    if (s != GDN_OK) return s;
    if (!ckpt || !buf || !depth_ok(depth)) return GDN_ERR_INVALID_ARG;
    if (!aligned16(ckpt) || !aligned16(buf)) return GDN_ERR_ALIGNMENT;
    return replay_dispatch(sh, nullptr, nullptr, nullptr, nullptr, nullptr, ckpt, buf, depth,
                           nullptr, eff_scale(sh), false, (hipStream_t)stream);
}

gdn_status gdn_decode_step(const gdn_shape* sh, const void* q, const void* k, const void* v,
                           const float* g, const float* beta, float* state, void* o, void* stream)
{
    gdn_status s = check_shape(sh, true);
    if (s != GDN_OK) return s;
    if (!q || !k || !v || !g || !beta || !state || !o) return GDN_ERR_INVALID_ARG;
    const void* ptrs[] = {q, k, v, g, beta, state, o};
    for (const void* p : ptrs)
        if (!aligned16(p)) return GDN_ERR_ALIGNMENT;
    return decode_dispatch(sh, q, k, v, g, beta, state, o, eff_scale(sh), (hipStream_t)stream);
}

}  // extern "C"
