// What the device-side stand-ins of launch_stubs.cpp saw last.
#pragma once
#include <stddef.h>

#include "tv_internal.h"

namespace stub {
struct Record {
  const char* name;
  int B, n_max, elem_bytes;
  size_t ws_bytes;
  const void* ws;
};
extern Record last;
extern int calls;
}  // namespace stub
