// Internal: per-thread error message behind kv_last_error().
#pragma once

#include <cstdarg>

namespace pkv {

// Records a printf-style message for kv_last_error() on the calling thread.
void set_error(const char *fmt, ...) __attribute__((format(printf, 1, 2)));

}  // namespace pkv

#define PKV_FAIL(code, ...)            \
    do {                               \
        ::pkv::set_error(__VA_ARGS__); \
        return (code);                 \
    } while (0)
