// Status and error-text helpers shared by the host sources of libqmv.
#pragma once

#include <stdint.h>

#include "qmv.h"

namespace qmv {

// Record a printf-style detail for qmv_last_error() and return `status`.
int32_t fail(int32_t status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Clear the thread's last error and return QMV_OK.
int32_t ok();

}  // namespace qmv
