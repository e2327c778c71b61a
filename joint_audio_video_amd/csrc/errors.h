// Thread-local error text behind dit_last_error().
#pragma once

#include <cstdarg>
#include <cstdio>

#include "dit.h"

namespace dit {

char* error_buffer();   // 512 bytes, thread-local

inline void clear_error() { error_buffer()[0] = '\0'; }

inline dit_status fail(dit_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(error_buffer(), 512, fmt, ap);
  va_end(ap);
  return st;
}

}  // namespace dit
