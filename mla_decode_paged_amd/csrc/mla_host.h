// Host-side helpers shared by the libmla C entry points: the per-thread error
// message and argument checks common to several calls.
#pragma once

#include <cstdarg>
#include <cstdio>

#include "../../include/mla.h"

namespace mla {

inline char* error_buffer() {
  static thread_local char buf[512] = "";
  return buf;
}

// Record a message for mla_last_error() and return `code`.
inline int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(error_buffer(), 512, fmt, ap);
  va_end(ap);
  return code;
}

inline int clear_error() {
  error_buffer()[0] = '\0';
  return MLA_OK;
}

// Shapes every compute call accepts: b >= 1, 1 <= s_q <= 8, h in {16, 32, 64, 128}.
inline int check_shape(const char* fn, int b, int s_q, int h) {
  if (b < 1) return set_error(MLA_ERR_INVALID_ARG, "%s: b must be >= 1 (got %d)", fn, b);
  if (s_q < 1 || s_q > 8) return set_error(MLA_ERR_INVALID_ARG, "%s: s_q must be in [1, 8] (got %d)", fn, s_q);
  if (h != 16 && h != 32 && h != 64 && h != 128)
    return set_error(MLA_ERR_UNSUPPORTED, "%s: h must be 16, 32, 64 or 128 (got %d)", fn, h);
  return MLA_OK;
}

}  // namespace mla
