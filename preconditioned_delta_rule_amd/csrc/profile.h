// Optional per-launch timing (osdn_profile_begin / osdn_profile_end): while a
// profile is open on the calling thread, every kernel launch records a HIP
// event on its stream right after the launch.
#pragma once

#include <hip/hip_runtime.h>

namespace osdn {

// Record the end of the launch just enqueued on `s`; a no-op unless a
// profile is open on this thread.
void prof_mark(hipStream_t s, const char *kernel);

}  // namespace osdn
