#include "common.h"
#include "plan.h"
namespace gdn {
gdn_status forward_dispatch(const Plan& p, const void* q, const void* k, const void* v,
                            const float* g, const float* beta, const float* h0, void* o, float* hT,
                            void* ws, hipStream_t st)
{
    return GDN_ERR_UNSUPPORTED;
}
gdn_status backward_dispatch(const Plan& p, const void* q, const void* k, const void* v,
                             const float* g, const float* beta, const float* h0, const void* dO,
                             const float* dhT, void* dq, void* dk, void* dv, float* dg,
                             float* dbeta, float* dh0, void* ws, hipStream_t st)
{
    return GDN_ERR_UNSUPPORTED;
}
}
