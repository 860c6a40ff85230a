// kvp_internal.h -- helpers shared by the library's translation units (not installed).
#pragma once

#include <cstdarg>
#include <cstdio>
#include <string>

#include "kvp.h"

namespace kvp {

// Thread-local last-error text behind kvp_last_error().
void set_error(const char *fmt, ...) __attribute__((format(printf, 1, 2)));
void clear_error();

inline kvp_status fail(kvp_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
inline kvp_status fail(kvp_status st, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    set_error("%s", buf);
    return st;
}

} // namespace kvp
