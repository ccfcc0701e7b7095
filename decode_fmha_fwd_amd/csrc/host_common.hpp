// host_common.hpp -- host-side helpers shared by the library's translation
// units: the per-thread error string and argument checks.
#pragma once

#include <cstdarg>
#include <cstdint>

#include "../../include/fmha.h"

namespace fmha {

// Records a formatted detail message for fmha_last_error() and returns s.
fmha_status fail(fmha_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Maps a pending HIP launch error to FMHA_ERR_HIP.
fmha_status check_launch(const char* what);

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace fmha
