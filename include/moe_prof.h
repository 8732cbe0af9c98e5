/*
 * moe_prof.h - measurement hooks of libmoe.so (not part of the layer's ABI in moe.h).
 *
 * While profiling is on, every kernel the library launches carries a start/stop hipEvent pair
 * attached to its dispatch on its own stream, so kernel times are read on the GPU's clock (a
 * benchmark uses them for per-kernel durations and roofline fractions).
 *
 * moe_profile_begin clears earlier records and turns profiling on (the first 4096 launches are
 * kept); moe_profile_end turns it off, waits for the recorded launches and returns the number of
 * distinct kernel names (or a negative moe_status); moe_profile_entry reads entry i: its name
 * (valid until the next moe_profile_begin), the summed kernel time in milliseconds and the number
 * of launches. Not thread-safe.
 */
#ifndef MOE_MI355X_PROF_H
#define MOE_MI355X_PROF_H

#include <stdint.h>

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

moe_status moe_profile_begin(void);
int moe_profile_end(void);
moe_status moe_profile_entry(int i, const char **name, double *total_ms, int32_t *launches);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_PROF_H */
