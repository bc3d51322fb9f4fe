// Internal helpers shared by the libddtree translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "ddtree.h"

namespace ddtree {

// Thread-local message behind ddtree_last_error().
void set_error(const char* fmt, ...);
void clear_error();

// Compute units of the current device (cached per device id); 0 on failure.
int device_cu_count();

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Report a failed launch (hipGetLastError) as DDTREE_EHIP.
inline int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: launch failed: %s", what, hipGetErrorString(e));
    return DDTREE_EHIP;
  }
  return DDTREE_OK;
}

}  // namespace ddtree

#define DDTREE_REQUIRE(cond, code, ...)   \
  do {                                    \
    if (!(cond)) {                        \
      ::ddtree::set_error(__VA_ARGS__);   \
      return (code);                      \
    }                                     \
  } while (0)
