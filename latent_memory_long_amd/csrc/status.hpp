// Error reporting shared by the C-ABI translation units: a status code plus a
// thread-local message that msa_last_error() returns.
#pragma once

#include <string>

#include "../../include/msa.h"

extern thread_local std::string g_last_error;

// Sets the thread's last-error message (printf format) and returns s.
msa_status fail(msa_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
