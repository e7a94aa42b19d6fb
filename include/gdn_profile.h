/*
 * gdn_profile.h -- launch-level timing of the gated delta-rule library, for
 * measurement tools (benchmarks, roofline reports).  Not needed to use the
 * layer, and not part of the library proper: only the measurement build,
 * libgdn_prof.so (the same sources compiled with GDN_PROFILE defined), exports
 * these entry points and consults the recorder around its launches; libgdn.so
 * keeps no recorder.
 *
 * gdn_profile_begin(events, n_pairs): from now on, the library records
 * events[2j] on the launch stream right before its j-th kernel launch and
 * events[2j+1] right after it, for j = 0 .. n_pairs-1, across every gdn_*
 * call; later launches are not recorded.  `events` holds 2*n_pairs hipEvent_t
 * handles created by the caller (timing enabled) and must stay valid until
 * gdn_profile_end().  n_pairs is at most GDN_PROFILE_MAX.
 * gdn_profile_end() stops recording and returns the number of launches
 * recorded; their elapsed times are read by the caller with
 * hipEventElapsedTime(events[2j], events[2j+1]) after synchronising.
 * gdn_profile_launch_name(j) is the kernel name of recorded launch j (a
 * static string), or NULL when j is out of range.
 * Errors: gdn_profile_begin returns GDN_ERR_INVALID_ARG for NULL events or
 * n_pairs outside [1, GDN_PROFILE_MAX].  In the measurement build the
 * recorder is process-global and not thread-safe: profile one host thread at
 * a time.
 */
#ifndef GDN_PROFILE_H
#define GDN_PROFILE_H

#include "gdn.h"

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_PROFILE_MAX 65536

gdn_status gdn_profile_begin(void *const *events, int n_pairs);
int gdn_profile_end(void);
const char *gdn_profile_launch_name(int j);

#ifdef __cplusplus
}
#endif
#endif /* GDN_PROFILE_H */
