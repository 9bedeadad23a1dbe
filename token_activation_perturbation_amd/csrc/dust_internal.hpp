// dust_internal.hpp -- declarations shared by the host and device translation
// units of libdust.so (no HIP types).
#pragma once

#include "dust.h"

namespace dust {
// Records `msg` as this thread's last error and returns `status`.
dust_status_t fail(dust_status_t status, const char* fmt, ...);
// Clears this thread's last error and returns DUST_OK.
dust_status_t ok();
}  // namespace dust
