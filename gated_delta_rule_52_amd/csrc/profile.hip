// profile.hip -- the launch recorder declared in include/gdn_profile.h.  It
// exists only in the measurement build (GDN_PROFILE defined, libgdn_prof.so);
// the library proper keeps no recorder and exports none of these symbols.
#ifdef GDN_PROFILE
#include "common.h"
#include "gdn_profile.h"

namespace gdn {

static hipEvent_t* g_ev = nullptr;
static int g_pairs = 0, g_used = 0, g_last = 0;
static const char* g_names[GDN_PROFILE_MAX];

void prof_begin(const char* name, hipStream_t st)
{
    if (g_ev && g_used < g_pairs) {
        g_names[g_used] = name;
        hipEventRecord(g_ev[2 * g_used], st);
    }
}

void prof_end(hipStream_t st)
{
    if (g_ev && g_used < g_pairs) {
        hipEventRecord(g_ev[2 * g_used + 1], st);
        ++g_used;
    }
}

}  // namespace gdn

using namespace gdn;

extern "C" {

gdn_status gdn_profile_begin(void* const* events, int n_pairs)
{
    if (!events || n_pairs < 1 || n_pairs > GDN_PROFILE_MAX) return GDN_ERR_INVALID_ARG;
    g_ev = (hipEvent_t*)events;
    g_pairs = n_pairs;
    g_used = 0;
    return GDN_OK;
}

int gdn_profile_end(void)
{
    const int n = g_used;
    g_ev = nullptr;
    g_pairs = 0;
    g_used = 0;
    g_last = n;
    return n;
}

const char* gdn_profile_launch_name(int j)
{
    if (j < 0 || j >= g_last) return nullptr;
    return g_names[j];
}

}  // extern "C"

#endif  // GDN_PROFILE
